// Skinny-M (decode-shaped) FP8 block-scaled NT GEMM for gfx950: m <= 64.
//
// Same arithmetic as gemm_fp8_nt_kernel ("DeepSeek open-source week day 3",
// technical features: FP8 sums per 128-wide K slab, promoted into fp32 with
// the 1 x 128 activation scale and the 128 x 128 weight scale), organised for
// the shapes where D has too few 64-row tiles to occupy the GPU and the
// weight stream B is the whole cost (64 x 2112 x 7168: 15.1 MB of B against
// 0.46 MB of A).
//
// Work unit: one 128-wide K slab of one 64 x BN output tile.  The units are
// ordered tile-major (all slabs of tile 0, then tile 1, ...) and dealt to the
// workgroups in equal contiguous runs (stream-K style), at most NW * UPW per
// workgroup, so every workgroup moves the same bytes whatever the tile count.
// Wave w of a workgroup takes the UPW consecutive units UPW w .. UPW w + UPW-1
// of the run:
//
//  * it loads every unit's A slab (64 x 128 bytes) and B slab (BN x 128
//    bytes) into VGPRs up front, each 16-byte load instruction covering 8
//    whole 128-byte rows (a cache line per 8 lanes; rows that only partly
//    share an instruction cost about twice as long on gfx950), so a
//    workgroup keeps NW * UPW * (64 + BN) * 128 bytes in flight;
//  * per unit, it writes the rows into its own LDS area (row-major, 16-byte
//    chunks XOR-swizzled) and reads them back in the MFMA operand layout
//    (lane l: row l % 16 of a fragment, 32 K-bytes): the transpose costs no
//    barrier, only this wave's own LDS traffic;
//  * one v_mfma_f32_16x16x128_f8f6f4 per 16 x 16 fragment gives the slab's
//    fp32 sum p, and acc += p * (sa * sb) promotes it, one accumulator per
//    tile the wave's units touch;
//  * the waves' accumulators meet in LDS and are added per tile in unit
//    order (one "piece" per tile the run touches).
//
// A tile whose slabs all lie in one workgroup is stored as bf16 directly.  A
// tile cut by run boundaries has several contributing workgroups: each stores
// its fp32 partial into the tile's slot of the workspace and bumps the tile's
// arrival counter; the last to arrive adds the slots in contributor order
// (its own from LDS, so results are bit-for-bit reproducible), stores bf16 D
// and resets the counter for the next call.  (Taking the arrival ticket when
// a workgroup starts, and letting the last starter poll tagged partials,
// saves the atomic's round trip at the end but measured slower: the first
// poll mostly came too early, and each further poll is another round trip.)
//
// Memory ordering of that hand-off (the per-XCD L2s are not coherent with
// each other): partials go out as SC1 stores, which complete only once they
// are written beyond the XCD's L2 at the device coherence point; each
// storing thread waits vmcnt(0) for its own stores, the workgroup barrier
// then orders every thread's completed stores before the agent-scope
// atomic, performed at that same point.  The last contributor observes the
// count its atomic returns, crosses a barrier and only then issues SC1
// loads, which are served from the coherence point and not from its L1 or
// L2.  Every store of the other contributors completed before their atomics,
// and every atomic precedes the last one, so the loads see them.
#pragma once

#include "gemm_kernel.h"

namespace dg {

typedef unsigned v2u __attribute__((ext_vector_type(2)));

struct SkinnyParams {
  const uint8_t* a;
  const float* sfa;
  const uint8_t* b;
  const float* sfb;
  uint16_t* d;
  int m;            // rows of A and D (1..64)
  int n;
  int k;
  int kb_count;     // k / 128
  int sfa_ld;
  int tiles_n;      // ceil(n / BN)
  int per;          // units per workgroup: workgroup L takes per + (L < rem)
  int rem;
  int max_contrib;  // workspace slots per tile
  float* ws_partial;  // [tiles_n][max_contrib][64 * BN] fp32 partial tiles, fragment-native order
  int* ws_count;      // [tiles_n] arrival counters, zero between calls
};

// First unit of workgroup L, and the workgroup that owns unit u.
__device__ __forceinline__ int sk_start(int L, int per, int rem) { return L * per + min(L, rem); }
__device__ __forceinline__ int sk_owner(int u, int per, int rem) {
  const int big = rem * (per + 1);
  return u < big ? u / (per + 1) : rem + (u - big) / per;
}

constexpr int kSkinnyMaxPieces = 16;  // tiles one workgroup's run may touch (<= NW * UPW)
constexpr int kSkinnyMaxContrib = 16;  // workgroups that may contribute to one tile

// SA / SB: stage the A / B slab through LDS (loads of whole 128-byte rows,
// then the transpose into the MFMA layout) or load it straight into the MFMA
// layout (two 64-byte half rows per lane and row).
template <int BN, int NW, int UPW, bool SA, bool SB>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(SkinnyParams p) {
  constexpr int FM = 4;             // 64 rows: four 16-row A fragments
  constexpr int FN = BN / 16;
  constexpr int F = FM * FN;        // fragments of a tile
  constexpr int kLa = 8;            // 16-byte load instructions per A slab
  constexpr int kLb = BN / 8;       // ... per B slab
  constexpr int kStageA = SA ? 64 * 128 : 0;
  constexpr int kStage = kStageA + (SB ? BN * 128 : 0);  // one unit's staged rows in LDS
  static_assert(BN % 16 == 0 && 128 % BN == 0, "a tile's columns lie in one 128-row B scale block");
  static_assert(NW * UPW <= kSkinnyMaxPieces, "pieces per workgroup");
  static_assert(NW * kStage <= 160 * 1024 && NW * UPW * F * 1024 <= 160 * 1024, "LDS of one workgroup");
  static_assert(kLb == 2 * FN, "two 16-byte loads per B fragment row");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // [NW][kStage] per-wave staging during the main phase, then [NW][UPW][F][64]
  // v4f accumulators for the reduction
  v4f* red = reinterpret_cast<v4f*>(smem);
  __shared__ int s_piece[NW][UPW];    // piece of each accumulator slot (-1: none)
  __shared__ int s_last[kSkinnyMaxPieces];  // per piece: this workgroup adds the tile up

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int u0 = sk_start(L, p.per, p.rem);
  const int nu = sk_start(L + 1, p.per, p.rem) - u0;  // units of this workgroup (<= NW * UPW)
  const int KB = p.kb_count;
  const int fmv = min(FM, (p.m + 15) >> 4);            // A fragments that hold rows
  const int tf = u0 / KB;                              // first tile of the run
  const int np = nu > 0 ? (u0 + nu - 1) / KB - tf + 1 : 0;
  auto whole_piece = [&](int q) { return (tf + q) * KB >= u0 && (tf + q + 1) * KB <= u0 + nu; };

  // ---- this wave's units: loads first, all of them
  const uint32_t K = (uint32_t)p.k;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.a, 0, (int)((uint32_t)p.m * K), kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.b, 0, (int)((uint32_t)p.n * K), kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.sfa, 0, (int)((uint32_t)KB * (uint32_t)p.sfa_ld * 4u), kBufferRsrcWord3);
  // Staged operand: load instruction t of a slab covers rows 8t..8t+7; lane l
  // brings the 16-byte chunk that belongs in LDS slot l % 8 of row 8t + l / 8,
  // chunk (l % 8) ^ swz(row), so the LDS write is one linear 1 KiB store.
  // Direct operand: loads 2i and 2i+1 are fragment i's two 16-byte chunks of
  // lane l: row 16i + l % 16, K bytes [16 (l / 16), +16) and [64 + 16 (l / 16), +16).
  const int lrow = lane >> 3;
  auto load_off = [&](bool staged, int i, int row0) -> uint32_t {
    if (staged) {
      const int r = 8 * i + lrow;
      return (uint32_t)(row0 + r) * K + 16u * (uint32_t)((lane & 7) ^ swz(r));
    }
    return (uint32_t)(row0 + 16 * (i >> 1) + (lane & 15)) * K + 16u * (uint32_t)(lane >> 4) + 64u * (uint32_t)(i & 1);
  };
  v4i va[UPW][kLa];
  v4i vb[UPW][kLb];
  v4f sv[UPW][FM];
  float sbv[UPW];
  int tile_of[UPW];
  const int ubase = u0 + UPW * wave;
  // Every wave issues UPW units' loads (a wave with fewer units loads its
  // last unit again and ignores it); A load instructions that carry no row
  // below m are skipped, and rows past m or n read as zero (buffer range
  // check).
  const int na = SA ? min(kLa, (p.m + 7) >> 3) : 2 * fmv;
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int u = __builtin_amdgcn_readfirstlane(max(u0, min(ubase + j, u0 + nu - 1)));
    const int t = u / KB;
    const int kb = u - t * KB;
    const int n0 = t * BN;
    tile_of[j] = t;
    const int slab = kb * 128;
#pragma unroll
    for (int i = 0; i < kLa; ++i)
      if (i < na)  // instructions that carry rows of A
        va[j][i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)load_off(SA, i, 0), slab, 0));
#pragma unroll
    for (int i = 0; i < kLb; ++i)
      vb[j][i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)load_off(SB, i, n0), slab, 0));
    // row scales of the lane's four result rows per fragment: 16 i + 4 (l / 16) + e
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i >= fmv) continue;
      const int off = (kb * p.sfa_ld + 16 * i + 4 * (lane >> 4)) * 4;
      sv[j][i] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rsa, off, 0, 0));
    }
    sbv[j] = p.sfb[(size_t)(n0 >> 7) * KB + kb];  // the tile's one block scale (wave-uniform)
  }

  // ---- per unit: LDS transpose (staged operands), MFMA, promotion
  uint8_t* stage = smem + wave * kStage;
  const int fr = lane & 15;
  const uint32_t frag_lo = (uint32_t)(fr * 128 + 16 * ((lane >> 4) ^ swz(fr)));
  const uint32_t frag_hi = (uint32_t)(fr * 128 + 16 * ((4 + (lane >> 4)) ^ swz(fr)));
  v4f acc[UPW][F];
#pragma unroll
  for (int s = 0; s < UPW; ++s)
#pragma unroll
    for (int f = 0; f < F; ++f) acc[s][f] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    if (UPW * wave + j >= nu) continue;
    const int slot = tile_of[j] - tile_of[0];  // accumulator of this unit's tile
    if constexpr (SA) {
#pragma unroll
      for (int i = 0; i < kLa; ++i)
        if (i < na) *(v4i*)(stage + i * 1024 + lane * 16) = va[j][i];
    }
    if constexpr (SB) {
#pragma unroll
      for (int i = 0; i < kLb; ++i) *(v4i*)(stage + kStageA + i * 1024 + lane * 16) = vb[j][i];
    }
    if constexpr (SA || SB) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's rows are in LDS
    v8i bf[FN];
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) {
      v4i lo = vb[j][2 * jj], hi = vb[j][2 * jj + 1];
      if constexpr (SB) {
        lo = *(const v4i*)(stage + kStageA + jj * 2048 + frag_lo);
        hi = *(const v4i*)(stage + kStageA + jj * 2048 + frag_hi);
      }
      bf[jj] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    v8i af[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i >= fmv) continue;
      v4i lo = va[j][2 * i], hi = va[j][2 * i + 1];
      if constexpr (SA) {
        lo = *(const v4i*)(stage + i * 2048 + frag_lo);
        hi = *(const v4i*)(stage + i * 2048 + frag_hi);
      }
      af[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    if constexpr (SA || SB) __builtin_amdgcn_s_waitcnt(0xC07F);  // fragment reads done before the next unit's rows land
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i >= fmv) continue;
      const v4f sc = sv[j][i] * sbv[j];
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) {
        const v4f pr = mfma_fp8_16x16x128(af[i], bf[jj]);
#pragma unroll
        for (int s = 0; s < UPW; ++s)
          if (s == slot) {
            acc[s][i * FN + jj][0] = __builtin_fmaf(pr[0], sc[0], acc[s][i * FN + jj][0]);
            acc[s][i * FN + jj][1] = __builtin_fmaf(pr[1], sc[1], acc[s][i * FN + jj][1]);
            acc[s][i * FN + jj][2] = __builtin_fmaf(pr[2], sc[2], acc[s][i * FN + jj][2]);
            acc[s][i * FN + jj][3] = __builtin_fmaf(pr[3], sc[3], acc[s][i * FN + jj][3]);
          }
      }
    }
  }
  __syncthreads();  // every wave is done with its staging area

  // ---- accumulators into LDS: slot s of wave w holds piece s_piece[w][s]
  const int last_unit = min(UPW, nu - UPW * wave);  // units of this wave (may be <= 0)
  const int nslots = last_unit > 0 ? tile_of[last_unit - 1] - tile_of[0] + 1 : 0;
#pragma unroll
  for (int s = 0; s < UPW; ++s) {
    if (lane == 0) s_piece[wave][s] = s < nslots ? tile_of[0] + s - tf : -1;
    if (s >= nslots) continue;
#pragma unroll
    for (int f = 0; f < F; ++f)
      if (f / FN < fmv) red[((wave * UPW + s) * F + f) * 64 + lane] = acc[s][f];
  }
  __syncthreads();

  // ---- (piece, fragment) pairs r = wave, wave + NW, ...: the piece's sum in
  // unit order, read back from LDS where it is needed (the LDS copy stays
  // until the workgroup ends)
  auto piece_sum = [&](int q, int f) {
    v4f sum = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int t = 0; t < UPW; ++t)
        if (s_piece[w][t] == q) sum += red[((w * UPW + t) * F + f) * 64 + lane];
    return sum;
  };
  const int npairs = np * F;

  auto store_d = [&](const v4f& v, int tq, int f) {
    const int i = f / FN, jj = f - (f / FN) * FN;
    const int col = tq * BN + 16 * jj + (lane & 15);
    if (col >= p.n) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * i + 4 * (lane >> 4) + e;
      if (row < p.m) p.d[(size_t)row * p.n + col] = f32_to_bf16_rne(v[e]);
    }
  };
  constexpr int kTileFloats = 64 * BN;
  auto contributors = [&](int tq, int* c0, int* cnt) {
    *c0 = sk_owner(tq * KB, p.per, p.rem);
    *cnt = sk_owner((tq + 1) * KB - 1, p.per, p.rem) - *c0 + 1;
  };

  // ---- whole tiles are stored; cut tiles' partials go to their slots
  for (int r = wave; r < npairs; r += NW) {
    const int q = r / F, f = r - q * F;
    if (f / FN >= fmv) continue;
    const int tq = tf + q;
    const v4f own = piece_sum(q, f);
    if (whole_piece(q)) {
      store_d(own, tq, f);
      continue;
    }
    int c0, cnt;
    contributors(tq, &c0, &cnt);
    float* slot = p.ws_partial + ((size_t)tq * p.max_contrib + (L - c0)) * kTileFloats;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(slot, 0, kTileFloats * 4, kBufferRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b128(own, rs, (f * 64 + lane) * 16, 0, kCpolSc1);
  }
  const bool wg_cut = !whole_piece(0) || !whole_piece(np - 1);  // only the first and last piece can be cut
  if (!wg_cut) return;  // uniform over the workgroup

  wait_vmem_all();  // this thread's partial stores are complete at the coherence point
  __syncthreads();  // ... and every other thread's
  if (wave == 0 && lane < np) {
    int last = 0;
    if (!whole_piece(lane)) {
      int c0, cnt;
      contributors(tf + lane, &c0, &cnt);
      last = __hip_atomic_fetch_add(p.ws_count + tf + lane, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == cnt - 1;
    }
    s_last[lane] = last;
  }
  __syncthreads();

  // ---- the last contributor of a cut tile adds the slots up in contributor order
  for (int r = wave; r < npairs; r += NW) {
    const int q = r / F, f = r - q * F;
    if (f / FN >= fmv || !s_last[q]) continue;
    const int tq = tf + q;
    int c0, cnt;
    contributors(tq, &c0, &cnt);
    const int me = L - c0;
    const float* slots = p.ws_partial + (size_t)tq * p.max_contrib * kTileFloats;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)slots, 0, p.max_contrib * kTileFloats * 4, kBufferRsrcWord3);
    v4f sum = {0.f, 0.f, 0.f, 0.f};
    constexpr int kChunk = NW >= 16 ? 4 : 8;  // slots loaded at once (4 registers each)
    for (int c0c = 0; c0c < cnt; c0c += kChunk) {
      v4f part[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        const int cc = c0c + c;
        if (cc < cnt && cc != me)
          part[c] = __builtin_bit_cast(
              v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, cc * kTileFloats * 4 + (f * 64 + lane) * 16, 0, kCpolSc1));
      }
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        const int cc = c0c + c;
        if (cc >= cnt) break;
        sum += cc == me ? piece_sum(q, f) : part[c];
      }
    }
    store_d(sum, tq, f);
  }
  if (wave == 0 && lane < np && s_last[lane])  // ready for the next call
    __hip_atomic_store(p.ws_count + tf + lane, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dg
