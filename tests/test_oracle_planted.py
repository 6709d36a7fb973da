"""Planted mistakes in the oracle must be caught by its pins.

Each case copies the oracle, the CPU tests and the input generators into a
temporary directory, plants one plausible mistake in the copied oracle's
source (a dropped slab, a transposed operand, a wrong scale index, a wrong
sign, a rounding or saturation slip, ...), runs the CPU pin suite there and
expects at least one failure.  The repository's own oracle is never changed.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (oracle file, original text, planted text)
MUTATIONS = [
    # gemm: scale-row index of B, transposed/permuted operand, dropped slab,
    # sign, wrong A scale column, contiguous tag check, masked clamp,
    # grouped sfb index, per-expert B / sfb
    ("gemm.py", "np.arange(n) // SLAB", "np.arange(n) % SLAB"),
    ("gemm.py", "p = a_dec @ b_dec.T", "p = a_dec @ b_dec[::-1].T"),
    ("gemm.py", "for s in range(kb):\n        cols", "for s in range(kb - 1):\n        cols"),
    ("gemm.py", "r += p * scale", "r -= p * scale"),
    ("gemm.py", "scale = sa[:, s][:, None]", "scale = sa[:, 0][:, None]"),
    ("gemm.py", "valid = (idx >= 0) & (idx < g_cnt)", "valid = (idx >= 0)"),
    ("gemm.py", "return np.clip(np.asarray(masked_m, np.int64), 0, max_m)",
     "return np.clip(np.asarray(masked_m, np.int64), 0, max_m - 1)"),
    ("gemm.py", "sb[gg, cc // SLAB])\n    return out\n\n\ndef _masked",
     "sb[gg, cc % 2])\n    return out\n\n\ndef _masked"),
    ("gemm.py", "acc += p[:, s] * (np.float64(1) * sa_rows[c0:c1, s]",
     "acc += p[:, s] * (np.float64(1) * sa_rows[c0:c1, 0]"),
    ("gemm.py", "out[ok] = _entries(qa[gg, rr], sa[gg, rr], qb[gg, cc]",
     "out[ok] = _entries(qa[gg, rr], sa[gg, rr], qb[0, cc]"),
    ("gemm.py", "r[g, :c] = gemm_nt_ref(qa[g, :c], sfa[g, :c], qb[g], sfb[g])",
     "r[g, :c] = gemm_nt_ref(qa[g, :c], sfa[g, :c], qb[g], sfb[0])"),
    # K-grouped: group start off by one slab, scales of the wrong slabs,
    # unaligned sizes accepted
    ("gemm.py", "starts = ends - sizes", "starts = ends - sizes + SLAB * (sizes > 0)"),
    ("gemm.py", "np.asarray(sfa)[:, s0:s1], qb[:, cols]", "np.asarray(sfa)[:, 0:s1 - s0], qb[:, cols]"),
    ("gemm.py", "if np.any(sizes < 0) or np.any(sizes % SLAB):", "if np.any(sizes < 0):"),
    # SwiGLU: gate and up swapped, sigmoid of the wrong sign
    ("gemm.py", "return silu(r[..., :i]) * r[..., i:], valid", "return silu(r[..., i:]) * r[..., :i], valid"),
    ("gemm.py", "return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))"),
    ("gemm.py", "hq[e, :rows], hs[e, :rows] = quantize_a_1x128(h[e, :rows].astype(np.float32))",
     "hq[e, :rows], hs[e, :rows] = quantize_a_1x128(np.abs(h[e, :rows]).astype(np.float32))"),
    # contiguous SwiGLU: gate and up swapped, h of the wrong rows quantised
    ("gemm.py", "return silu(r[:, :i]) * r[:, i:], valid", "return silu(r[:, i:]) * r[:, :i], valid"),
    ("gemm.py", "hq[rows], hs[rows] = quantize_a_1x128(h[rows].astype(np.float32))",
     "hq[rows], hs[rows] = quantize_a_1x128(h[rows[::-1]].astype(np.float32))"),
    # BF16: wrong half of the fp32 word, transposed operand
    ("gemm.py", "b = np.asarray(bits, np.uint16).astype(np.uint32) << 16", "b = np.asarray(bits, np.uint16).astype(np.uint32) << 15"),
    ("gemm.py", "    return a @ b.T\n", "    return a @ b[::-1].T\n"),
    # FP4: decode exponent, tie rule, nibble order, range of the scale,
    # B scale block of a column
    ("e2m1.py", "(2 + f) * 2.0 ** (e - 2)", "(2 + f) * 2.0 ** (e - 1)"),
    ("e2m1.py", "q = np.rint(np.ldexp(a, -(e - 1)))", "q = np.floor(np.ldexp(a, -(e - 1)) + 0.5)"),
    ("e2m1.py", "out[..., 0::2] = p & 0xF\n    out[..., 1::2] = p >> 4", "out[..., 1::2] = p & 0xF\n    out[..., 0::2] = p >> 4"),
    ("quant.py", "s = (amax / np.float32(E2M1_MAX)).astype(np.float32)\n    scaled",
     "s = (amax / np.float32(E2M1_MAX + 1)).astype(np.float32)\n    scaled"),
    ("gemm.py", "(sa[:, s][:, None] * sb[block_of_col, s][None, :])\n    return r\n",
     "(sa[:, s][:, None] * sb[0, s][None])\n    return r\n"),
    # e4m3: tie rule, exponent bias, saturation code, subnormal boundary
    ("e4m3.py", "q = np.rint(steps)", "q = np.floor(steps + 0.5)"),
    ("e4m3.py", "mag = (8 + f) * 2.0 ** (e - 10)", "mag = (8 + f) * 2.0 ** (e - 9)"),
    ("e4m3.py", "code = np.minimum(code, 0x7E)", "code = np.minimum(code, 0x7D)"),
    ("e4m3.py", "e_unb = np.maximum(x - 1, _MIN_NORMAL_EXP)", "e_unb = np.maximum(x - 1, _MIN_NORMAL_EXP - 1)"),
    # quant: scale value, partial last block of B, reciprocal stored as the scale,
    # amax over the wrong extent
    ("quant.py", "amax = np.maximum(amax, AMAX_FLOOR)\n    s =",
     "amax = np.maximum(amax, AMAX_FLOOR) * np.float32(1.0001)\n    s ="),
    ("quant.py", "r0, r1 = bi * SLAB, min(n, (bi + 1) * SLAB)",
     "r0, r1 = bi * SLAB, min(n, (bi + 1) * SLAB + 0)\n        r0 = max(0, r1 - SLAB)"),
    ("quant.py", "s = (amax / _F448).astype(np.float32)  # correctly",
     "s = (_F448 / amax).astype(np.float32)  # correctly"),
    ("quant.py", "amax = np.max(np.abs(blk), axis=(0, 2))",
     "amax = np.max(np.abs(blk), axis=(2,)).max(axis=0) * np.float32(0.999)"),
]

PIN_TESTS = ["test_oracle_e4m3.py", "test_oracle_quant.py", "test_oracle_gemm.py", "test_oracle_fp4.py",
             "test_accounting.py"]


def _run_one(case, base):
    i, (fname, frm, to) = case
    d = os.path.join(base, f"m{i}")
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"))
    shutil.copytree(os.path.join(ROOT, "workloads"), os.path.join(d, "workloads"))
    os.makedirs(os.path.join(d, "tests"))
    for f in ["__init__.py", "conftest.py"] + PIN_TESTS:
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(d, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), d)
    path = os.path.join(d, "oracle", fname)
    with open(path) as fh:
        src = fh.read()
    if src.count(frm) < 1:
        return (fname, frm, "planted text not found in the oracle source")
    with open(path, "w") as fh:
        fh.write(src.replace(frm, to, 1))
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=d, capture_output=True, text=True, env=env, timeout=600)
    tail = (r.stdout.strip().splitlines() or [""])[-1]
    if r.returncode == 0 or "failed" not in tail:
        return (fname, frm, f"not caught: {tail}")
    return None


def test_planted_mistakes_are_caught(tmp_path):
    workers = min(8, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda c: _run_one(c, str(tmp_path)), enumerate(MUTATIONS)))
    missed = [r for r in results if r is not None]
    assert not missed, missed
