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
//    staging), NST-stage buffered, one workgroup barrier per slab;
//  * each DMA instruction reads 8 whole 128-byte rows (8 lanes per cache
//    line): on gfx950 this moves ~3.7x more bytes per clock into a CU than
//    instructions that cover 16 half lines.  LDS keeps the tile row-major,
//    128 bytes per row, with the 16-byte chunk c of tile row r stored in
//    slot c ^ ((r >> 1) & 7): the 16 rows a fragment read touches then hit
//    16 distinct 16-byte bank groups, so ds_read_b128 is conflict-free;
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
constexpr int kDmaBytes = 1024;
// Word 3 of a raw buffer resource for gfx9 (32-bit data format; offsets past
// num_records read as zero) and the SC1 cache-policy bit of buffer accesses.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCpolSc1 = 16;   // LDS bytes one wave-wide 16-byte-per-lane DMA writes

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
  // split-K (dense): each tile's K slabs are shared by `splits` workgroups of
  // `split_slabs` slabs each; their fp32 partial tiles meet in a workspace and
  // the last workgroup to arrive adds them in split order and stores D.
  int splits;
  int split_slabs;
  float* ws_partial;         // [num_tiles][splits][BM * BN] fp32, fragment-native order
  int* ws_count;             // [num_tiles] arrival counters, zero between calls
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

// Wait until at most N of this wave's vector-memory loads (LDS DMA included)
// are outstanding; they retire in issue order.  gfx9 s_waitcnt encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vmem_all() { wait_vmem<0>(); }

// vmcnt wait with a wave-uniform run-time count (a scalar branch picks the
// immediate).  Counts above 47 wait for everything.
__device__ __forceinline__ void wait_vmem_dyn(int n) {
#define DG_VM_CASE(i) \
  case i:             \
    wait_vmem<i>();   \
    return;
  switch (n) {
    DG_VM_CASE(1) DG_VM_CASE(2) DG_VM_CASE(3) DG_VM_CASE(4) DG_VM_CASE(5) DG_VM_CASE(6) DG_VM_CASE(7)
    DG_VM_CASE(8) DG_VM_CASE(9) DG_VM_CASE(10) DG_VM_CASE(11) DG_VM_CASE(12) DG_VM_CASE(13) DG_VM_CASE(14)
    DG_VM_CASE(15) DG_VM_CASE(16) DG_VM_CASE(17) DG_VM_CASE(18) DG_VM_CASE(19) DG_VM_CASE(20) DG_VM_CASE(21)
    DG_VM_CASE(22) DG_VM_CASE(23) DG_VM_CASE(24) DG_VM_CASE(25) DG_VM_CASE(26) DG_VM_CASE(27) DG_VM_CASE(28)
    DG_VM_CASE(29) DG_VM_CASE(30) DG_VM_CASE(31) DG_VM_CASE(32) DG_VM_CASE(33) DG_VM_CASE(34) DG_VM_CASE(35)
    DG_VM_CASE(36) DG_VM_CASE(37) DG_VM_CASE(38) DG_VM_CASE(39) DG_VM_CASE(40) DG_VM_CASE(41) DG_VM_CASE(42)
    DG_VM_CASE(43) DG_VM_CASE(44) DG_VM_CASE(45) DG_VM_CASE(46) DG_VM_CASE(47)
    default:
      wait_vmem<0>();
      return;
  }
#undef DG_VM_CASE
}

// Workgroup barrier without a memory fence: the caller has already waited for
// the loads that must be visible.  (__syncthreads() would also wait for every
// outstanding LDS DMA, prefetches included.)  The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // fmt 0 = e4m3 for both operands; E8M0 scale 127 = 2^0 (neutral).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 127, 0, 127);
}

// LDS layout: NST stages, each holding one slab of the A tile, of the B
// tile, the A row scales and the B block scales of that slab; the epilogue
// reuses the space for the bf16 output tile.
template <int BM, int BN, int NST>
struct Smem {
  static constexpr int kA = BM * kSlab;
  static constexpr int kB = BN * kSlab;
  static constexpr int kSa = BM * 4;
  static constexpr int kSbCount = BN / 128 + 2;  // 128-row blocks a BN-wide tile can touch
  static constexpr int kSb = 256;                // one dword DMA instruction's footprint
  static constexpr int kStage = kA + kB + kSa + kSb;
  static constexpr int kOutPitch = BN * 2 + 16;  // bf16 output row pitch (bytes)
  static constexpr int kOut = BM * kOutPitch;
  static constexpr int kMain = NST * kStage;
  static constexpr int kBytes = kMain > kOut ? kMain : kOut;
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

// Number of slab DMA batches a wave has issued after the one of slab kb, at
// the top of iteration kb: the prologue issues slabs 0..NST-2 and iteration
// i issues slab i+NST-1 (nothing for slabs >= KB).
template <int NST>
__device__ __forceinline__ int loads_ahead(int kb, int KB) {
  int n = KB - 1 - kb;
  return n < NST - 2 ? n : NST - 2;
}

// LDS slot swizzle of tile row r (see the layout note at the top)
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <int BM, int BN, int WM, int WN, int NST, int VAR>
__global__ __launch_bounds__(WM * WN * 64) void gemm_fp8_nt_kernel(GemmParams p) {
  constexpr int kThreads = WM * WN * 64;
  constexpr int kWaves = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int kJa = BM / 8;  // DMA instructions per slab for A (1 KiB each)
  constexpr int kJb = BN / 8;
  using S = Smem<BM, BN, NST>;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole fragments");
  static_assert(BM <= kThreads, "row-tag pass needs one thread per tile row");
  static_assert(NST >= 2, "pipeline shape");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_flag;  // contiguous: block expert; split-K: last-arriver flag
  __shared__ uint8_t s_row_ok[BM];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;

  // ---- tile -> (group, tile_m, tile_n[, split])
  int g = 0, tm, tn, tile_id = 0, split = 0;
  if (VAR == kMasked) {
    // an expert's tiles are consecutive, and the XCD remap keeps consecutive
    // tiles on one XCD: the expert's A rows are fetched into one L2 only
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    const int per_g = p.tiles_m * p.tiles_n;
    g = t / per_g;
    const int r = t - g * per_g;
    tm = r / p.tiles_n;
    tn = r - tm * p.tiles_n;
  } else if (p.splits > 1) {
    tile_id = blockIdx.x / p.splits;
    split = blockIdx.x - tile_id * p.splits;
    tm = tile_id / p.tiles_n;
    tn = tile_id - tm * p.tiles_n;
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
  const int row_limit = p.m;  // rows that exist in memory (load clamp)
  int valid_rows = p.m;       // rows with a result (masked: the expert's count)
  if (VAR == kContiguous) {
    if (threadIdx.x == 0) s_flag = -1;
    __syncthreads();
    int tag = -1;
    if (threadIdx.x < BM) {
      tag = p.m_indices[m0 + threadIdx.x];
      if (tag >= 0 && tag < p.num_groups) atomicMax(&s_flag, tag);
    }
    __syncthreads();
    const int expert = s_flag;
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
  // K slabs of this workgroup: [kb0, kb0 + KB) (KB is local; p.kb_count is K/128)
  const int kb0 = split * p.split_slabs;
  const int KB = p.splits > 1 ? min(p.split_slabs, p.kb_count - kb0) : p.kb_count;
  const int K = p.k;
  // rows worth loading: the masked layout never reads rows past the count
  const int a_rows = VAR == kMasked ? valid_rows : row_limit;

  // ---- slab loader.  One wave-wide DMA instruction moves 1 KiB (one
  // fragment half) into LDS; each wave owns a fixed set of instructions whose
  // per-lane source offsets are computed once per tile.
  constexpr int kPerWaveA = kJa / kWaves;
  constexpr int kPerWaveB = kJb / kWaves;
  static_assert(kJa % kWaves == 0 && kJb % kWaves == 0, "DMA instructions must split evenly over waves");
  uint32_t a_off[kPerWaveA];
  uint32_t b_off[kPerWaveB];
  int a_live = 0;  // A DMA instructions this wave issues per slab (masked skips empty fragments)
  // instruction j covers tile rows 8j..8j+7; lane l fills LDS slot (l & 7) of
  // row 8j + (l >> 3) with the global chunk that belongs there
#pragma unroll
  for (int jj = 0; jj < kPerWaveA; ++jj) {
    const int j = jj * kWaves + wave;
    const int r = 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(r);
    int row = m0 + r;
    row = row < row_limit ? row : row_limit - 1;
    a_off[jj] = (uint32_t)row * (uint32_t)K + 16u * chunk;
    a_live += (m0 + 8 * j < a_rows) ? 1 : 0;
  }
#pragma unroll
  for (int jj = 0; jj < kPerWaveB; ++jj) {
    const int j = jj * kWaves + wave;
    const int r = 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(r);
    int row = n0 + r;
    row = row < p.n ? row : p.n - 1;
    b_off[jj] = (uint32_t)row * (uint32_t)K + 16u * chunk;
  }
  // Row scales: BM floats, one dword instruction per 64 rows.  Every wave
  // issues exactly one (waves past the needed count repeat a block with the
  // same data), so every wave issues the same number of loads per slab.
  constexpr int kSaInsts = (BM + 63) / 64;
  const int sa_blk = wave % kSaInsts;
  const bool sa_lane = sa_blk * 64 + lane < BM;
  uint32_t sa_off;
  {
    int row = m0 + sa_blk * 64 + lane;
    row = row < row_limit ? row : row_limit - 1;
    sa_off = (uint32_t)row;
  }
  // B block scales of the 128-row blocks this tile touches (every wave)
  const int nb0 = n0 >> 7;
  const bool sb_lane = lane < S::kSbCount;
  uint32_t sb_off;
  {
    int blk = nb0 + lane;
    blk = blk < p.nb_count ? blk : p.nb_count - 1;
    sb_off = (uint32_t)blk * (uint32_t)p.kb_count;  // sfb row stride: all K slabs
  }
  const int c_loads = a_live + kPerWaveB + 2;

  auto issue_slab = [&](int kl, int buf) {
    const int kb = kb0 + kl;  // global slab index
    uint8_t* st = smem + buf * S::kStage;
    const uint8_t* a_k = A + kb * kSlab;
    const uint8_t* b_k = B + kb * kSlab;
#pragma unroll
    for (int jj = 0; jj < kPerWaveA; ++jj) {
      const int j = jj * kWaves + wave;
      if (VAR == kMasked && m0 + 8 * j >= a_rows) continue;  // rows without results
      lds_dma16(a_k + a_off[jj], st + j * kDmaBytes);
    }
#pragma unroll
    for (int jj = 0; jj < kPerWaveB; ++jj) {
      const int j = jj * kWaves + wave;
      lds_dma16(b_k + b_off[jj], st + S::kA + j * kDmaBytes);
    }
    if (sa_lane) lds_dma4(SFA + (size_t)kb * p.sfa_ld + sa_off, st + S::kA + S::kB + sa_blk * 256);
    if (sb_lane) lds_dma4(SFB + sb_off + kb, st + S::kA + S::kB + S::kSa);
  };

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // index of each fragment's B scale block among the tile's blocks
  int sb_idx[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) sb_idx[j] = ((n0 + wn * TN + j * 16) >> 7) - nb0;
  constexpr bool kSbUniform = (128 % TN) == 0;  // a wave's columns lie in one block
  // fragments of this wave that hold at least one valid row
  int fm_valid = FM;
  if (VAR == kMasked) {
    const int left = valid_rows - (m0 + wm * TM);
    fm_valid = left <= 0 ? 0 : (left + 15) / 16;
  }

  // per-lane LDS byte offsets of the two 16-byte chunks of a fragment read
  // (row lane & 15 of the fragment, K chunks g and g + 4, g = lane >> 4)
  const int fr = lane & 15;
  const uint32_t frag_lo = (uint32_t)(fr * 128 + 16 * ((lane >> 4) ^ swz(fr)));
  const uint32_t frag_hi = (uint32_t)(fr * 128 + 16 * ((4 + (lane >> 4)) ^ swz(fr)));

  // ---- prologue: DMA of slabs 0..NST-2
#pragma unroll
  for (int s0 = 0; s0 <= NST - 2; ++s0)
    if (s0 < KB) issue_slab(s0, s0);

  for (int kb = 0; kb < KB; ++kb) {
    // slab kb's DMA must have landed (in every wave: then the barrier); the
    // loads issued after it may stay in flight.
    wait_vmem_dyn(c_loads * loads_ahead<NST>(kb, KB));
    block_barrier();  // also: every wave is done with the stage about to be refilled
    __builtin_amdgcn_sched_barrier(0);
    if (kb + NST - 1 < KB) issue_slab(kb + NST - 1, (kb + NST - 1) % NST);
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t* st = smem + (kb % NST) * S::kStage;
    const uint8_t* sA = st;
    const uint8_t* sB = st + S::kA;
    const float* sSa = (const float*)(st + S::kA + S::kB);
    const float* sSb = (const float*)(st + S::kA + S::kB + S::kSa);

    float sbv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) sbv[j] = sSb[kSbUniform ? sb_idx[0] : sb_idx[j]];

    v8i bf[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int f = wn * FN + j;
      const v4i lo = *(const v4i*)(sB + f * 2048 + frag_lo);
      const v4i hi = *(const v4i*)(sB + f * 2048 + frag_hi);
      bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }

    // Software pipeline over the wave's FM x FN fragments (row-major order t):
    // A rows are read from LDS kPf rows ahead, and fragment t's promotion
    // runs kLag fragments after its MFMA, so each MFMA has independent
    // promotion FMAs of earlier fragments to co-issue with.
    constexpr int kPf = FM < 2 ? FM : 2;
    constexpr int kAbuf = kPf + 1;
    constexpr int kSabuf = kPf + 2;
    constexpr int kLag = 2;
    constexpr int F = FM * FN;
    v8i abuf[kAbuf];
    v4f sabuf[kSabuf];
    v4f pr[kLag + 1];
    auto load_a = [&](int i) {
      const int f = wm * FM + i;
      const v4i lo = *(const v4i*)(sA + f * 2048 + frag_lo);
      const v4i hi = *(const v4i*)(sA + f * 2048 + frag_hi);
      abuf[i % kAbuf] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      sabuf[i % kSabuf] = *(const v4f*)(sSa + wm * TM + i * 16 + 4 * (lane >> 4));
    };
#pragma unroll
    for (int i = 0; i < kPf; ++i)
      if (VAR != kMasked || i < fm_valid) load_a(i);
#pragma unroll
    for (int t = 0; t < F + kLag; ++t) {
      if (t < F) {
        const int i = t / FN, j = t % FN;
        if (VAR != kMasked || i < fm_valid) {
          if (j == 0 && i + kPf < FM && (VAR != kMasked || i + kPf < fm_valid)) load_a(i + kPf);
          pr[t % (kLag + 1)] = mfma_fp8_16x16x128(abuf[i % kAbuf], bf[j]);
        }
      }
      if (t >= kLag) {
        const int u = t - kLag;
        const int i = u / FN, j = u % FN;
        if (VAR != kMasked || i < fm_valid) {
          const v4f sc = sabuf[i % kSabuf] * sbv[j];
          const v4f pv = pr[u % (kLag + 1)];
          acc[i][j][0] = __builtin_fmaf(pv[0], sc[0], acc[i][j][0]);
          acc[i][j][1] = __builtin_fmaf(pv[1], sc[1], acc[i][j][1]);
          acc[i][j][2] = __builtin_fmaf(pv[2], sc[2], acc[i][j][2]);
          acc[i][j][3] = __builtin_fmaf(pv[3], sc[3], acc[i][j][3]);
        }
      }
    }
  }

  wait_vmem_all();  // no LDS DMA may be in flight past this point

  // ---- split-K fix-up: publish this split's partial tile; the last split
  // to arrive adds all partials in split order (deterministic) and goes on to
  // store D.  Partials are laid out fragment-native (each lane owns 16
  // contiguous bytes per fragment) and move with SC1 buffer stores and loads,
  // which are coherent across the per-XCD L2s (the agent-scope path), so no
  // L2 write-back or invalidate is needed.  The reducer reads kChunk splits'
  // partials per batch; loads past the last split return zero.
  if (VAR == kDense && p.splits > 1) {
    constexpr int kTileFloats = BM * BN;
    constexpr int kChunk = (FM * FN * 4) >= 128 ? 1 : 128 / (FM * FN * 4);
    float* part = p.ws_partial + (size_t)tile_id * p.splits * kTileFloats;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(part, 0, p.splits * kTileFloats * 4, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(
            acc[i][j], rs, (split * kTileFloats + (((wave * FM + i) * FN + j) * 64 + lane) * 4) * 4, 0, kCpolSc1);
    wait_vmem_all();  // this thread's partial stores are complete (in memory)
    __syncthreads();  // ... and so are every other thread's
    if (threadIdx.x == 0) {
      const int arrived = __hip_atomic_fetch_add(p.ws_count + tile_id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_flag = (arrived == p.splits - 1) ? 1 : 0;
    }
    __syncthreads();
    if (s_flag == 0) return;  // not the last split: done
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < p.splits; sp0 += kChunk) {
      v4f part_v[kChunk][FM][FN];
#pragma unroll
      for (int c = 0; c < kChunk; ++c)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            part_v[c][i][j] = __builtin_amdgcn_raw_buffer_load_b128(
                rs, ((sp0 + c) * kTileFloats + (((wave * FM + i) * FN + j) * 64 + lane) * 4) * 4, 0, kCpolSc1);
#pragma unroll
      for (int c = 0; c < kChunk; ++c)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] += part_v[c][i][j];
    }
    if (threadIdx.x == 0)  // ready for the next call
      __hip_atomic_store(p.ws_count + tile_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue: bf16 (round to nearest even) through LDS, then 16-byte
  // coalesced row stores of valid rows and columns
  block_barrier();  // every wave is done reading the last stage
  uint8_t* so = smem;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (VAR == kMasked && i >= fm_valid) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int cl = wn * TN + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rl = wm * TM + i * 16 + 4 * (lane >> 4) + e;
        *(uint16_t*)(so + rl * S::kOutPitch + cl * 2) = f32_to_bf16_rne(acc[i][j][e]);
      }
    }
  }
  block_barrier();
  const int rows_here = min(BM, valid_rows - m0);  // rows of this tile with results
  const int cols_here = min(BN, p.n - n0);
  if ((p.n & 7) == 0) {
    constexpr int kChunks = BN / 8;  // 16-byte chunks per tile row
    for (int idx = threadIdx.x; idx < BM * kChunks; idx += kThreads) {
      const int rl = idx / kChunks, ch = idx % kChunks;
      if (rl >= rows_here || ch * 8 >= cols_here) continue;
      if (VAR == kContiguous && !s_row_ok[rl]) continue;
      const v4i v = *(const v4i*)(so + rl * S::kOutPitch + ch * 16);
      *(v4i*)(D + (size_t)(m0 + rl) * p.n + n0 + ch * 8) = v;
    }
  } else {
    for (int idx = threadIdx.x; idx < BM * BN; idx += kThreads) {
      const int rl = idx / BN, cl = idx % BN;
      if (rl >= rows_here || cl >= cols_here) continue;
      if (VAR == kContiguous && !s_row_ok[rl]) continue;
      D[(size_t)(m0 + rl) * p.n + n0 + cl] = *(const uint16_t*)(so + rl * S::kOutPitch + cl * 2);
    }
  }
}

}  // namespace dg
