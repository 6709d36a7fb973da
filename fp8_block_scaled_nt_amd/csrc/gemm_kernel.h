// FP8 (e4m3) block-scaled NT GEMM main loop for gfx950 (CDNA4).
//
// D = A . B^T, A [rows][k] with one fp32 scale per row and 128-wide K slab,
// B [n][k] with one fp32 scale per 128 x 128 block, D bf16.  The method is
// the one the DeepGEMM pages describe ("DeepSeek open-source week day 3",
// technical features: FP8 tensor-core sums per block, promoted into a
// higher-precision accumulator with the fine-grained scales; MoE contiguous
// and masked layouts; unified block scheduler with rasterisation).  The
// mechanism here is gfx950's own:
//
//  * one v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 fragment covers exactly
//    one 128-wide K slab, so its fp32 result p is the slab's partial sum;
//  * promotion: acc += p * (sa[row] * sb[col block]) in fp32 VGPRs after each
//    slab (the MFMA's own E8M0 scales stay neutral: the fp32 block scales
//    are not powers of two);
//  * operand tiles move HBM/L2 -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging), double buffered, one workgroup barrier per slab;
//  * the LDS tile is stored fragment-major: every 1 KiB holds exactly what
//    one ds_read_b128 of a whole wave needs, so LDS reads are contiguous per
//    wave (free of bank conflicts for any bank count) and each DMA
//    instruction writes one such 1 KiB block;
//  * the blockIdx -> tile map is XCD-aware: the 8 XCDs each take a
//    contiguous run of a grouped-raster tile order, so tiles that share A
//    rows or B columns sit in the same L2.
//
// MFMA operand layout (probed on gfx950): lane l of a 16x16x128 fp8 operand
// holds 32 K-bytes of row (l % 16); any K order works as long as A and B use
// the same one.  Here lane l holds K bytes [16*(l/16), +16) in its low four
// VGPRs and [64 + 16*(l/16), +16) in its high four.  The fp32 result lane l,
// element i is row 4*(l/16) + i, column l % 16 of the 16x16 fragment.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace dg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) const void* glb_ptr_t;

enum Variant { kDense = 0, kContiguous = 1, kMasked = 2 };

constexpr int kSlab = 128;        // K bytes per slab (one scale per slab)
constexpr int kNumXcd = 8;        // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kFragBytes = 1024;  // one wave-wide 16-byte-per-lane LDS block

struct GemmParams {
  const uint8_t* a;
  const float* sfa;
  const uint8_t* b;
  const float* sfb;
  uint16_t* d;
  const int32_t* m_indices;  // contiguous layout
  const int32_t* masked_m;   // masked layout
  int m;                     // rows of A (dense, contiguous) or max_m (masked)
  int n;
  int k;
  int kb_count;              // k / 128
  int nb_count;              // ceil(n / 128)
  int sfa_ld;                // leading dimension of slab-major sfa
  int num_groups;
  int tiles_m;               // per group for the masked layout
  int tiles_n;
  int num_tiles;
  int group_m;               // raster group height in tiles
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __bfloat16_as_ushort(__float2bfloat16(f));
}

__device__ __forceinline__ void lds_dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((glb_ptr_t)src, (lds_ptr_t)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ void lds_dma4(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((glb_ptr_t)src, (lds_ptr_t)lds_dst, 4, 0, 0);
}

// Wait for all of this wave's outstanding vector-memory loads (including the
// LDS DMA ones) to land.  gfx9 s_waitcnt encoding: vmcnt = 0, expcnt and
// lgkmcnt left at their maxima.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // fmt 0 = e4m3 for both operands; E8M0 scale 127 = 2^0 (neutral).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 127, 0, 127);
}

template <int BM, int BN>
struct Smem {
  static constexpr int kA = BM * kSlab;
  static constexpr int kB = BN * kSlab;
  static constexpr int kSa = BM * 4;
  static constexpr int kStage = kA + kB + kSa;
  static constexpr int kBytes = 2 * kStage;
};

// Map a linear tile id to (tile_m, tile_n) in grouped raster order: runs of
// group_m tile rows are walked column by column.
__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int grp = t / per_group;
  const int first_m = grp * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  const int r = t - grp * per_group;
  tm = first_m + r % gsz;
  tn = r / gsz;
}

// Deal consecutive logical tile ids to one XCD: workgroup b runs on XCD b % 8.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  if (nblocks % kNumXcd != 0) return bid;
  return (bid % kNumXcd) * (nblocks / kNumXcd) + bid / kNumXcd;
}

template <int BM, int BN, int WM, int WN, int VAR>
__global__ __launch_bounds__(WM * WN * 64) void gemm_fp8_nt_kernel(GemmParams p) {
  constexpr int kThreads = WM * WN * 64;
  constexpr int kWaves = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int kJa = BM / 8;  // DMA instructions per slab for A (1 KiB each)
  constexpr int kJb = BN / 8;
  using S = Smem<BM, BN>;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole fragments");
  static_assert(BM <= kThreads, "row-tag pass needs one thread per tile row");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_expert;
  __shared__ uint8_t s_row_ok[BM];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;

  // ---- tile -> (group, tile_m, tile_n)
  int g = 0, tm, tn;
  if (VAR == kMasked) {
    const int t = blockIdx.x;
    const int per_g = p.tiles_m * p.tiles_n;
    g = t / per_g;
    const int r = t - g * per_g;
    tm = r / p.tiles_n;
    tn = r - tm * p.tiles_n;
  } else {
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    raster(t, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  }
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  // ---- per-variant operand bases and the number of valid rows
  const uint8_t* A = p.a;
  const float* SFA = p.sfa;
  const uint8_t* B = p.b;
  const float* SFB = p.sfb;
  uint16_t* D = p.d;
  int row_limit = p.m;   // rows that exist in memory (load clamp)
  int valid_rows = p.m;  // rows with a result (masked: the expert's count)
  int expert = 0;
  if (VAR == kContiguous) {
    if (threadIdx.x == 0) s_expert = -1;
    __syncthreads();
    int tag = -1;
    if (threadIdx.x < BM) {
      tag = p.m_indices[m0 + threadIdx.x];
      if (tag >= 0 && tag < p.num_groups) atomicMax(&s_expert, tag);
    }
    __syncthreads();
    expert = s_expert;
    if (expert < 0) return;  // a block of padding rows only
    if (threadIdx.x < BM) s_row_ok[threadIdx.x] = (tag == expert);
    B += (size_t)expert * p.n * p.k;
    SFB += (size_t)expert * p.nb_count * p.kb_count;
  } else if (VAR == kMasked) {
    int cnt = p.masked_m[g];
    cnt = cnt < 0 ? 0 : (cnt > p.m ? p.m : cnt);
    if (m0 >= cnt) return;  // masked early exit: nothing valid in this tile
    valid_rows = cnt;
    A += (size_t)g * p.m * p.k;
    SFA += (size_t)g * p.kb_count * p.sfa_ld;
    B += (size_t)g * p.n * p.k;
    SFB += (size_t)g * p.nb_count * p.kb_count;
    D += (size_t)g * p.m * p.n;
  }
  const int KB = p.kb_count;
  const int K = p.k;

  // ---- slab loader: one wave-wide DMA instruction moves 1 KiB into LDS
  auto issue_slab = [&](int kb, int buf) {
    uint8_t* st = smem + buf * S::kStage;
#pragma unroll
    for (int j0 = 0; j0 < kJa + kJb; j0 += kWaves) {
      const int j = j0 + wave;
      if (j < kJa) {
        const int f = j >> 1, h = j & 1;
        if (VAR == kMasked && m0 + 16 * f >= valid_rows) continue;  // skip empty fragments
        int row = m0 + 16 * f + (lane & 15);
        row = row < row_limit ? row : row_limit - 1;
        const uint8_t* src = A + (size_t)row * K + kb * kSlab + 16 * (4 * h + (lane >> 4));
        lds_dma16(src, st + j * kFragBytes);
      } else if (j < kJa + kJb) {
        const int jb = j - kJa;
        const int f = jb >> 1, h = jb & 1;
        int row = n0 + 16 * f + (lane & 15);
        row = row < p.n ? row : p.n - 1;
        const uint8_t* src = B + (size_t)row * K + kb * kSlab + 16 * (4 * h + (lane >> 4));
        lds_dma16(src, st + S::kA + jb * kFragBytes);
      }
    }
    // row scales of this slab: BM floats, 64 per instruction
#pragma unroll
    for (int j0 = 0; j0 < (BM + 63) / 64; j0 += kWaves) {
      const int j = j0 + wave;
      if (j < (BM + 63) / 64 && j * 64 + lane < BM) {
        int row = m0 + j * 64 + lane;
        row = row < row_limit ? row : row_limit - 1;
        lds_dma4(SFA + (size_t)kb * p.sfa_ld + row, st + S::kA + S::kB + j * 256);
      }
    }
  };

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // B scale rows of this wave's fragments (clamped for columns past n)
  int sb_row[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int blk = (n0 + wn * TN + j * 16) >> 7;
    sb_row[j] = (blk < p.nb_count ? blk : p.nb_count - 1) * KB;
  }
  // fragments of this wave that hold at least one valid row
  const int frag_rows0 = m0 + wm * TM;
  int fm_valid = FM;
  if (VAR == kMasked) {
    const int left = valid_rows - frag_rows0;
    fm_valid = left <= 0 ? 0 : (left + 15) / 16;
  }

  issue_slab(0, 0);
  for (int kb = 0; kb < KB; ++kb) {
    wait_vmem_all();
    __syncthreads();  // slab kb is in LDS; every wave is done with slab kb-1
    if (kb + 1 < KB) issue_slab(kb + 1, (kb + 1) & 1);

    const uint8_t* st = smem + (kb & 1) * S::kStage;
    const uint8_t* sA = st;
    const uint8_t* sB = st + S::kA;
    const float* sSa = (const float*)(st + S::kA + S::kB);

    float sbv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) sbv[j] = SFB[sb_row[j] + kb];

    v8i bf[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int f = wn * FN + j;
      const v4i lo = *(const v4i*)(sB + (2 * f + 0) * kFragBytes + lane * 16);
      const v4i hi = *(const v4i*)(sB + (2 * f + 1) * kFragBytes + lane * 16);
      bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (VAR == kMasked && i >= fm_valid) continue;
      const int f = wm * FM + i;
      const v4i lo = *(const v4i*)(sA + (2 * f + 0) * kFragBytes + lane * 16);
      const v4i hi = *(const v4i*)(sA + (2 * f + 1) * kFragBytes + lane * 16);
      const v8i af = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const v4f sa = *(const v4f*)(sSa + wm * TM + i * 16 + 4 * (lane >> 4));
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const v4f pr = mfma_fp8_16x16x128(af, bf[j]);
        const v4f s = sa * sbv[j];
        acc[i][j][0] = __builtin_fmaf(pr[0], s[0], acc[i][j][0]);
        acc[i][j][1] = __builtin_fmaf(pr[1], s[1], acc[i][j][1]);
        acc[i][j][2] = __builtin_fmaf(pr[2], s[2], acc[i][j][2]);
        acc[i][j][3] = __builtin_fmaf(pr[3], s[3], acc[i][j][3]);
      }
    }
  }

  // ---- epilogue: bf16 round-to-nearest-even, valid rows and columns only
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (VAR == kMasked && i >= fm_valid) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rl = wm * TM + i * 16 + 4 * (lane >> 4) + e;
      const int row = m0 + rl;
      bool ok = row < valid_rows;
      if (VAR == kContiguous) ok = ok && s_row_ok[rl];
      if (!ok) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * TN + j * 16 + (lane & 15);
        if (col < p.n) D[(size_t)row * p.n + col] = f32_to_bf16_rne(acc[i][j][e]);
      }
    }
  }
}

}  // namespace dg
