"""Python binding of the gfx950 FP8 block-scaled NT GEMM library (libdg.so).

The binding only marshals arguments: it checks dtypes, shapes and devices of
torch tensors, passes their device pointers and the current HIP stream to the
C ABI (include/dg.h), and raises on a non-zero status.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  PyTorch
supplies device memory and streams.

Layouts (all row-major, packed):
  a    [m, k] e4m3 codes (torch.float8_e4m3fn or uint8); masked: [g, max_m, k]
  sfa  slab-major fp32 [k/128, get_sfa_ld(m)]; masked: [g, k/128, get_sfa_ld(max_m)]
  b    [n, k] e4m3; grouped: [g, n, k]
  sfb  fp32 [ceil(n/128), k/128]; grouped: [g, ceil(n/128), k/128]
  d    bf16 [m, n]; masked: [g, max_m, n]
  hq   (SwiGLU) e4m3 [g, max_m, inter]; hs fp32 [g, inter/128, get_sfa_ld(max_m)]
  FP4  a [m, k/2], b [n, k/2] uint8, two e2m1 codes per byte (low nibble first),
       with the FP8 scale layouts
"""

import ctypes
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# DG_LIBRARY names another build of the same library (e.g. one whose host
# code is compiled with sanitizers); by default the in-tree libdg.so
LIB_PATH = os.environ.get("DG_LIBRARY") or os.path.join(_PKG_DIR, "libdg.so")

__all__ = [
    "DGError", "lib", "fp8_gemm_nt", "fp8_gemm_nt_noalloc", "m_grouped_fp8_gemm_nt_contiguous",
    "m_grouped_fp8_gemm_nt_masked", "m_grouped_fp8_gemm_nt_masked_swiglu", "m_grouped_fp8_gemm_nt_contiguous_swiglu",
    "quantize_a_1x128", "quantize_b_128x128",
    "k_grouped_fp8_gemm_nt", "bf16_gemm_nt", "fp4_gemm_nt", "quantize_a_1x128_fp4", "quantize_b_128x128_fp4", "get_m_alignment_for_contiguous_layout", "get_sfa_ld", "empty_sfa",
    "profile_next_launch",
    "reserve_workspace", "dense_workspace_size",
]


class DGError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status, message):
        super().__init__(f"dg status {status}: {message}")
        self.status = status


_lib = None
_vp, _ci = ctypes.c_void_p, ctypes.c_int
_SIGNATURES = {
    "dg_fp8_gemm_nt": [_vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _vp],
    "dg_fp8_gemm_nt_noalloc": [_vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _vp],
    "dg_m_grouped_fp8_gemm_nt_contiguous": [_vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _vp],
    "dg_m_grouped_fp8_gemm_nt_masked": [_vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _vp],
    "dg_m_grouped_fp8_gemm_nt_masked_swiglu": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _vp],
    "dg_m_grouped_fp8_gemm_nt_contiguous_swiglu": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _vp],
    "dg_k_grouped_fp8_gemm_nt": [_vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _vp],
    "dg_bf16_gemm_nt": [_vp, _vp, _vp, _ci, _ci, _ci, _vp],
    "dg_fp4_gemm_nt": [_vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _vp],
    "dg_quantize_a_1x128_fp4": [_vp, _vp, _vp, _ci, _ci, _vp],
    "dg_quantize_b_128x128_fp4": [_vp, _vp, _vp, _ci, _ci, _vp],
    "dg_get_m_alignment_for_contiguous_layout": [],
    "dg_get_sfa_ld": [_ci],
    "dg_quantize_a_1x128": [_vp, _vp, _vp, _ci, _ci, _vp],
    "dg_quantize_b_128x128": [_vp, _vp, _vp, _ci, _ci, _vp],
    "dg_status_string": [_ci],
    "dg_last_error_message": [],
    "dg_version": [],
    "dg_profile_next_launch": [_vp, _vp],
    "dg_reserve_workspace": [ctypes.c_size_t, _vp],
    "dg_dense_workspace_size": [_ci, _ci, _ci, _ci, ctypes.POINTER(ctypes.c_size_t)],
}
_RESTYPES = {"dg_status_string": ctypes.c_char_p, "dg_last_error_message": ctypes.c_char_p,
             "dg_version": ctypes.c_char_p}


def lib():
    """Load libdg.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run fp8_block_scaled_nt_amd/build.py")
        h = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            f = getattr(h, name)
            f.argtypes = args
            f.restype = _RESTYPES.get(name, ctypes.c_int)
        _lib = h
    return _lib


def _check(status):
    if status != 0:
        msg = lib().dg_last_error_message().decode()
        raise DGError(status, msg or lib().dg_status_string(status).decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


_FP8 = (torch.float8_e4m3fn, torch.uint8)


def _need(t, name, dtypes, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def profile_next_launch(start_event, stop_event):
    """Make the next GEMM launch on this thread record the two torch.cuda.Event
    objects (timing enabled, already recorded once so they exist) at the start
    and end of the kernel itself."""
    _check(lib().dg_profile_next_launch(start_event._as_parameter_, stop_event._as_parameter_))


def reserve_workspace(nbytes, stream=None):
    """Size the split-K workspace of a stream (default: the current one) on
    the current device for `nbytes` of partial tiles, so that later calls on
    that stream allocate nothing (and can be captured in a graph)."""
    st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream()
    _check(lib().dg_reserve_workspace(int(nbytes), st))


_DTYPES = {"fp8": 0, "bf16": 1, "fp4": 2}


def dense_workspace_size(m, n, k, dtype="fp8"):
    """Split-K workspace bytes a dense call (fp8_gemm_nt, bf16_gemm_nt or
    fp4_gemm_nt) of this shape makes on the current device; 0 if it does not
    split K.  Give it to reserve_workspace before capturing such calls."""
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be one of {sorted(_DTYPES)}")
    out = ctypes.c_size_t(0)
    _check(lib().dg_dense_workspace_size(_DTYPES[dtype], int(m), int(n), int(k), ctypes.byref(out)))
    return out.value


def get_m_alignment_for_contiguous_layout():
    return lib().dg_get_m_alignment_for_contiguous_layout()


def get_sfa_ld(m):
    return lib().dg_get_sfa_ld(int(m))


def empty_sfa(m, k, groups=None, device="cuda"):
    """Allocate a slab-major sfa buffer for m rows (optionally per group)."""
    shape = (k // 128, get_sfa_ld(m))
    if groups is not None:
        shape = (groups,) + shape
    return torch.empty(shape, dtype=torch.float32, device=device)


def fp8_gemm_nt(a_pair, b_pair, d):
    """D = A . B^T with block scales.  a_pair = (a [m,k], sfa), b_pair = (b [n,k], sfb),
    d: bf16 [m, n], written in place."""
    a, sfa = a_pair
    b, sfb = b_pair
    _need(a, "a", _FP8, 2)
    _need(b, "b", _FP8, 2)
    _need(d, "d", (torch.bfloat16,), 2)
    _need(sfa, "sfa", (torch.float32,), 2)
    _need(sfb, "sfb", (torch.float32,), 2)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError(f"shape mismatch a{tuple(a.shape)} b{tuple(b.shape)} d{tuple(d.shape)}")
    if tuple(sfa.shape) != (k // 128, get_sfa_ld(m)):
        raise ValueError(f"sfa must be [k/128, sfa_ld(m)] = {(k // 128, get_sfa_ld(m))}")
    if tuple(sfb.shape) != ((n + 127) // 128, k // 128):
        raise ValueError("sfb must be [ceil(n/128), k/128]")
    _check(lib().dg_fp8_gemm_nt(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), m, n, k, _stream()))
    return d


def fp8_gemm_nt_noalloc(a_pair, b_pair, d):
    """fp8_gemm_nt for callers that cannot allocate device memory: split-K
    scratch comes from the library's static per-GPU array (calls that
    overlap in time on one GPU race)."""
    a, sfa = a_pair
    b, sfb = b_pair
    _need(a, "a", _FP8, 2)
    _need(b, "b", _FP8, 2)
    _need(d, "d", (torch.bfloat16,), 2)
    _need(sfa, "sfa", (torch.float32,), 2)
    _need(sfb, "sfb", (torch.float32,), 2)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError(f"shape mismatch a{tuple(a.shape)} b{tuple(b.shape)} d{tuple(d.shape)}")
    if tuple(sfa.shape) != (k // 128, get_sfa_ld(m)) or tuple(sfb.shape) != ((n + 127) // 128, k // 128):
        raise ValueError("scale shape mismatch")
    _check(lib().dg_fp8_gemm_nt_noalloc(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), m, n, k, _stream()))
    return d


def m_grouped_fp8_gemm_nt_contiguous(a_pair, b_pair, d, m_indices):
    """Contiguous-layout grouped GEMM: row r of a uses expert m_indices[r]'s B."""
    a, sfa = a_pair
    b, sfb = b_pair
    _need(a, "a", _FP8, 2)
    _need(b, "b", _FP8, 3)
    _need(d, "d", (torch.bfloat16,), 2)
    _need(sfa, "sfa", (torch.float32,), 2)
    _need(sfb, "sfb", (torch.float32,), 3)
    _need(m_indices, "m_indices", (torch.int32,), 1)
    m, k = a.shape
    g, n, _ = b.shape
    if b.shape[2] != k or tuple(d.shape) != (m, n) or m_indices.numel() != m:
        raise ValueError("shape mismatch")
    if tuple(sfa.shape) != (k // 128, get_sfa_ld(m)) or tuple(sfb.shape) != (g, (n + 127) // 128, k // 128):
        raise ValueError("scale shape mismatch")
    _check(lib().dg_m_grouped_fp8_gemm_nt_contiguous(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), _ptr(m_indices), m, n, k, g, _stream()))
    return d


def m_grouped_fp8_gemm_nt_masked(a_pair, b_pair, d, masked_m, expected_m=0):
    """Masked-layout grouped GEMM: expert g computes its first masked_m[g] rows."""
    a, sfa = a_pair
    b, sfb = b_pair
    _need(a, "a", _FP8, 3)
    _need(b, "b", _FP8, 3)
    _need(d, "d", (torch.bfloat16,), 3)
    _need(sfa, "sfa", (torch.float32,), 3)
    _need(sfb, "sfb", (torch.float32,), 3)
    _need(masked_m, "masked_m", (torch.int32,), 1)
    g, max_m, k = a.shape
    n = b.shape[1]
    if b.shape[0] != g or b.shape[2] != k or tuple(d.shape) != (g, max_m, n) or masked_m.numel() != g:
        raise ValueError("shape mismatch")
    if tuple(sfa.shape) != (g, k // 128, get_sfa_ld(max_m)) or tuple(sfb.shape) != (g, (n + 127) // 128, k // 128):
        raise ValueError("scale shape mismatch")
    _check(lib().dg_m_grouped_fp8_gemm_nt_masked(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), _ptr(masked_m), g, max_m, n, k,
        int(expected_m), _stream()))
    return d


def m_grouped_fp8_gemm_nt_masked_swiglu(a_pair, b_pair, h_pair, masked_m, expected_m=0):
    """MoE FC1 + SwiGLU on the masked layout: B is [g, 2*inter, k] holding
    each expert's gate rows, then its up rows; h = silu(gate) * up of the
    valid rows is written as e4m3 codes hq [g, max_m, inter] with 1x128 fp32
    scales hs [g, inter/128, get_sfa_ld(max_m)], the A operand layout of the
    masked GEMM."""
    a, sfa = a_pair
    b, sfb = b_pair
    hq, hs = h_pair
    _need(a, "a", _FP8, 3)
    _need(b, "b", _FP8, 3)
    _need(hq, "hq", _FP8, 3)
    _need(sfa, "sfa", (torch.float32,), 3)
    _need(sfb, "sfb", (torch.float32,), 3)
    _need(hs, "hs", (torch.float32,), 3)
    _need(masked_m, "masked_m", (torch.int32,), 1)
    g, max_m, k = a.shape
    inter = b.shape[1] // 2
    if b.shape[0] != g or b.shape[2] != k or b.shape[1] != 2 * inter or masked_m.numel() != g:
        raise ValueError("shape mismatch")
    if tuple(hq.shape) != (g, max_m, inter) or tuple(hs.shape) != (g, inter // 128, get_sfa_ld(max_m)):
        raise ValueError("output shape mismatch")
    if tuple(sfa.shape) != (g, k // 128, get_sfa_ld(max_m)) or tuple(sfb.shape) != (g, (2 * inter + 127) // 128, k // 128):
        raise ValueError("scale shape mismatch")
    _check(lib().dg_m_grouped_fp8_gemm_nt_masked_swiglu(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(hq), _ptr(hs), _ptr(masked_m), g, max_m, inter, k,
        int(expected_m), _stream()))
    return hq, hs


def m_grouped_fp8_gemm_nt_contiguous_swiglu(a_pair, b_pair, h_pair, m_indices):
    """MoE FC1 + SwiGLU on the contiguous layout: B is [g, 2*inter, k] holding
    each expert's gate rows, then its up rows; h = silu(gate) * up of every
    row with a valid tag is written as e4m3 codes hq [m, inter] with 1x128
    fp32 scales hs [inter/128, get_sfa_ld(m)], the A operand layout of the
    contiguous GEMM."""
    a, sfa = a_pair
    b, sfb = b_pair
    hq, hs = h_pair
    _need(a, "a", _FP8, 2)
    _need(b, "b", _FP8, 3)
    _need(hq, "hq", _FP8, 2)
    _need(sfa, "sfa", (torch.float32,), 2)
    _need(sfb, "sfb", (torch.float32,), 3)
    _need(hs, "hs", (torch.float32,), 2)
    _need(m_indices, "m_indices", (torch.int32,), 1)
    m, k = a.shape
    g = b.shape[0]
    inter = b.shape[1] // 2
    if b.shape[2] != k or b.shape[1] != 2 * inter or m_indices.numel() != m:
        raise ValueError("shape mismatch")
    if tuple(hq.shape) != (m, inter) or tuple(hs.shape) != (inter // 128, get_sfa_ld(m)):
        raise ValueError("output shape mismatch")
    if tuple(sfa.shape) != (k // 128, get_sfa_ld(m)) or tuple(sfb.shape) != (g, (2 * inter + 127) // 128, k // 128):
        raise ValueError("scale shape mismatch")
    _check(lib().dg_m_grouped_fp8_gemm_nt_contiguous_swiglu(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(hq), _ptr(hs), _ptr(m_indices), m, inter, k, g, _stream()))
    return hq, hs


def k_grouped_fp8_gemm_nt(a_pair, b_pair, d, k_sizes):
    """K-grouped GEMM: group g uses the k_sizes[g] K columns after the groups
    before it; d: bf16 [g, m, n], written in place (zero for empty groups)."""
    a, sfa = a_pair
    b, sfb = b_pair
    _need(a, "a", _FP8, 2)
    _need(b, "b", _FP8, 2)
    _need(d, "d", (torch.bfloat16,), 3)
    _need(sfa, "sfa", (torch.float32,), 2)
    _need(sfb, "sfb", (torch.float32,), 2)
    _need(k_sizes, "k_sizes", (torch.int32,), 1)
    m, k = a.shape
    n = b.shape[0]
    g = k_sizes.numel()
    if b.shape[1] != k or tuple(d.shape) != (g, m, n):
        raise ValueError(f"shape mismatch a{tuple(a.shape)} b{tuple(b.shape)} d{tuple(d.shape)} groups={g}")
    if tuple(sfa.shape) != (k // 128, get_sfa_ld(m)) or tuple(sfb.shape) != ((n + 127) // 128, k // 128):
        raise ValueError("scale shape mismatch")
    _check(lib().dg_k_grouped_fp8_gemm_nt(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), _ptr(k_sizes), g, m, n, k,
                                           _stream()))
    return d


def bf16_gemm_nt(a, b, d):
    """BF16 NT GEMM: d (bf16 [m, n]) = a (bf16 [m, k]) . b (bf16 [n, k])^T, in place."""
    _need(a, "a", (torch.bfloat16,), 2)
    _need(b, "b", (torch.bfloat16,), 2)
    _need(d, "d", (torch.bfloat16,), 2)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError(f"shape mismatch a{tuple(a.shape)} b{tuple(b.shape)} d{tuple(d.shape)}")
    _check(lib().dg_bf16_gemm_nt(_ptr(a), _ptr(b), _ptr(d), m, n, k, _stream()))
    return d


def quantize_a_1x128(x, q=None, sfa=None):
    """fp32 [m, k] (or [g, m, k]) -> (e4m3 codes, slab-major sfa)."""
    _need(x, "x", (torch.float32,), x.dim())
    if x.dim() == 3:
        g, m, k = x.shape
        q = torch.empty((g, m, k), dtype=torch.float8_e4m3fn, device=x.device) if q is None else q
        sfa = empty_sfa(m, k, g, x.device) if sfa is None else sfa
        for i in range(g):
            quantize_a_1x128(x[i], q[i], sfa[i])
        return q, sfa
    m, k = x.shape
    q = torch.empty((m, k), dtype=torch.float8_e4m3fn, device=x.device) if q is None else q
    sfa = empty_sfa(m, k, None, x.device) if sfa is None else sfa
    _need(q, "q", _FP8, 2)
    _need(sfa, "sfa", (torch.float32,), 2)
    if tuple(q.shape) != (m, k) or tuple(sfa.shape) != (k // 128, get_sfa_ld(m)):
        raise ValueError("output shape mismatch")
    _check(lib().dg_quantize_a_1x128(_ptr(x), _ptr(q), _ptr(sfa), m, k, _stream()))
    return q, sfa


def quantize_b_128x128(x, q=None, sfb=None):
    """fp32 [n, k] (or [g, n, k]) -> (e4m3 codes, sfb [.., ceil(n/128), k/128])."""
    _need(x, "x", (torch.float32,), x.dim())
    if x.dim() == 3:
        g, n, k = x.shape
        q = torch.empty((g, n, k), dtype=torch.float8_e4m3fn, device=x.device) if q is None else q
        sfb = torch.empty((g, (n + 127) // 128, k // 128), dtype=torch.float32, device=x.device) if sfb is None else sfb
        for i in range(g):
            quantize_b_128x128(x[i], q[i], sfb[i])
        return q, sfb
    n, k = x.shape
    q = torch.empty((n, k), dtype=torch.float8_e4m3fn, device=x.device) if q is None else q
    sfb = torch.empty(((n + 127) // 128, k // 128), dtype=torch.float32, device=x.device) if sfb is None else sfb
    _need(q, "q", _FP8, 2)
    _need(sfb, "sfb", (torch.float32,), 2)
    if tuple(q.shape) != (n, k) or tuple(sfb.shape) != ((n + 127) // 128, k // 128):
        raise ValueError("output shape mismatch")
    _check(lib().dg_quantize_b_128x128(_ptr(x), _ptr(q), _ptr(sfb), n, k, _stream()))
    return q, sfb


def fp4_gemm_nt(a_pair, b_pair, d):
    """FP4 NT GEMM: a (uint8 [m, k/2], two e2m1 codes per byte) with sfa
    (slab-major [k/128, get_sfa_ld(m)]), b (uint8 [n, k/2]) with sfb
    ([ceil(n/128), k/128]); d is bf16 [m, n], written in place."""
    a, sfa = a_pair
    b, sfb = b_pair
    _need(a, "a", (torch.uint8,), 2)
    _need(b, "b", (torch.uint8,), 2)
    _need(d, "d", (torch.bfloat16,), 2)
    _need(sfa, "sfa", (torch.float32,), 2)
    _need(sfb, "sfb", (torch.float32,), 2)
    m, kh = a.shape
    n = b.shape[0]
    k = 2 * kh
    if b.shape[1] != kh or tuple(d.shape) != (m, n):
        raise ValueError(f"shape mismatch a{tuple(a.shape)} b{tuple(b.shape)} d{tuple(d.shape)}")
    if tuple(sfa.shape) != (k // 128, get_sfa_ld(m)) or tuple(sfb.shape) != ((n + 127) // 128, k // 128):
        raise ValueError("scale shape mismatch")
    _check(lib().dg_fp4_gemm_nt(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), m, n, k, _stream()))
    return d


def quantize_a_1x128_fp4(x, q=None, sfa=None):
    """fp32 [m, k] -> (packed e2m1 codes uint8 [m, k/2], slab-major sfa)."""
    _need(x, "x", (torch.float32,), 2)
    m, k = x.shape
    q = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device) if q is None else q
    sfa = empty_sfa(m, k, None, x.device) if sfa is None else sfa
    _need(q, "q", (torch.uint8,), 2)
    _need(sfa, "sfa", (torch.float32,), 2)
    if tuple(q.shape) != (m, k // 2) or tuple(sfa.shape) != (k // 128, get_sfa_ld(m)):
        raise ValueError("output shape mismatch")
    _check(lib().dg_quantize_a_1x128_fp4(_ptr(x), _ptr(q), _ptr(sfa), m, k, _stream()))
    return q, sfa


def quantize_b_128x128_fp4(x, q=None, sfb=None):
    """fp32 [n, k] -> (packed e2m1 codes uint8 [n, k/2], sfb [ceil(n/128), k/128])."""
    _need(x, "x", (torch.float32,), 2)
    n, k = x.shape
    q = torch.empty((n, k // 2), dtype=torch.uint8, device=x.device) if q is None else q
    sfb = torch.empty(((n + 127) // 128, k // 128), dtype=torch.float32, device=x.device) if sfb is None else sfb
    _need(q, "q", (torch.uint8,), 2)
    _need(sfb, "sfb", (torch.float32,), 2)
    if tuple(q.shape) != (n, k // 2) or tuple(sfb.shape) != ((n + 127) // 128, k // 128):
        raise ValueError("output shape mismatch")
    _check(lib().dg_quantize_b_128x128_fp4(_ptr(x), _ptr(q), _ptr(sfb), n, k, _stream()))
    return q, sfb
