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
//  * one v_mfma_f32_16x16x128_f8f6f4 per 16x16 fragment (the unscaled form
//    of the f8f6f4 MFMA) covers exactly one 128-wide K slab, so its fp32
//    result p is the slab's partial sum;
//  * promotion: acc += p * (sa[row] * sb[col block]) in fp32 VGPRs after each
//    slab (the block scales are arbitrary fp32 values, not the power-of-two
//    E8M0 scales the MFMA's scaled form could apply);
//  * operand tiles move HBM/L2 -> LDS with LDS DMA (buffer_load_dwordx4 ...
//    lds, no VGPR staging), NST-stage buffered, one workgroup barrier per
//    slab (the schedules below vary this);
//  * each DMA instruction reads 8 whole 128-byte rows (8 lanes per cache
//    line): on gfx950 this moves ~3.7x more bytes per clock into a CU than
//    instructions that cover 16 half lines.  LDS keeps the tile row-major,
//    128 bytes per row, with the 16-byte chunk c of tile row r stored in
//    slot c ^ ((r >> 1) & 7): the 16 rows a fragment read touches then hit
//    16 distinct 16-byte bank groups, so ds_read_b128 is conflict-free;
//  * the blockIdx -> tile map is XCD-aware: the 8 XCDs each take a
//    contiguous run of a grouped-raster tile order, so tiles that share A
//    rows or B columns sit in the same L2.  On the masked layout only
//    the tiles with valid rows are numbered, and the first workgroups take
//    them, dealt evenly over the XCDs.
//
// MFMA operand layout (probed on gfx950): lane l of a 16x16x128 fp8 operand
// holds 32 K-bytes of row (l % 16); any K order works as long as A and B use
// the same one.  Here lane l holds K bytes [16*(l/16), +16) in its low four
// VGPRs and [64 + 16*(l/16), +16) in its high four.  The fp32 result lane l,
// element i is row 4*(l/16) + i, column l % 16 of the 16x16 fragment.  The
// same kernel also runs bf16 operands (no scales) and e2m1 operands (FP4,
// block scales), and a SwiGLU + FP8 requantisation epilogue on the masked
// and contiguous layouts.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "quant_kernel.h"

namespace dg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) const void* glb_ptr_t;

enum Variant { kDense = 0, kContiguous = 1, kMasked = 2, kKGrouped = 3 };
// Operand type: e4m3 with block scales, bf16 without scales (a 128-byte slab
// row then holds 64 K values), or e2m1 (FP4, two per byte) with block scales
// (a 128-byte slab row then holds 256 K values: two scale slabs).
enum DType { kFp8 = 0, kBf16 = 1, kFp4 = 2 };
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
// Epilogue: store D as bf16, or (MoE FC1 on the masked or contiguous layout) pair each
// gate column with its up column, apply SwiGLU and quantise h with the 1 x 128
// activation rule, so the second GEMM reads h as FP8 without a round trip.
enum Epilogue { kEpiBf16 = 0, kEpiSwigluFp8 = 1 };

constexpr int kSlab = 128;        // K bytes per slab (fp8: one scale slab; fp4: two)
constexpr int kNumXcd = 8;        // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kDmaBytes = 1024;   // LDS bytes one wave-wide 16-byte-per-lane DMA writes
// Word 3 of a raw buffer resource for gfx9 (32-bit data format; offsets past
// num_records read as zero) and the SC1 cache-policy bit of buffer accesses.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCpolSc1 = 16;

struct GemmParams {
  const uint8_t* a;
  const float* sfa;
  const uint8_t* b;
  const float* sfb;
  uint16_t* d;
  const int32_t* m_indices;  // contiguous layout
  const int32_t* masked_m;   // masked layout
  const int32_t* k_sizes;    // K-grouped layout: K columns of each group
  uint8_t* hq;               // SwiGLU epilogue: h codes [groups][m][inter] (contiguous: [m][inter])
  float* hs;                 // SwiGLU epilogue: h scales [groups][inter/128][sfa_ld] (contiguous: one group)
  int inter;                 // SwiGLU epilogue: I (B holds 2I rows: gate, then up)
  int m;                     // rows of A (dense, contiguous) or max_m (masked)
  int n;
  int k;
  int kb_count;              // 128-byte K slabs per row (fp8: k / 128)
  int sk_count;              // 128-wide scale slabs per row (fp8: kb_count, fp4: 2 kb_count)
  int nb_count;              // ceil(n / 128)
  int sfa_ld;                // leading dimension of slab-major sfa
  int num_groups;
  int tiles_m;               // per group for the masked layout
  int tiles_n;
  int num_tiles;
  int group_m;               // raster group height in tiles
  int b_stream;              // 1: every B byte is read by one tile only (one row block
                             // of tiles): B's LDS DMA carries the non-temporal hint
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

// Direct global -> LDS copies (LDS DMA), buffer form: each lane's 16 (or 4)
// bytes at base + voffset + soffset land at M0 + lane * 16 (or 4).  The base
// and the byte size of the operand sit in a wave-uniform buffer descriptor,
// so a lane keeps only a 32-bit offset, the K slab goes into the scalar
// offset, and a read past the operand's size returns zeros instead of
// faulting.  They are issued from inline asm on purpose: the compiler cannot
// tell which LDS bytes an LDS DMA writes, and with one in flight it waits for
// every outstanding ds_read (lgkmcnt(0)) instead of the one it needs, which
// serialises the fragment prefetch.  The asm has no outputs (it writes only
// LDS), and its completion is tracked by this kernel's own vmcnt accounting
// (wait_vmem); compiler-placed vmcnt waits only become stricter when these
// extra loads are outstanding.  M0 is set inside the asm, with the one wait
// state the hardware needs before the DMA reads it; nothing else in these
// kernels keeps a value in M0.
//
// Back-to-back DMAs corrupt each other.  Measured on gfx950: a wave-wide
// 16-byte DMA sends its lanes to the texture unit in several passes, and
// when that unit is busy (several workgroups per CU loading) its last passes
// (lanes 24-31 and 56-63) can take the LDS destination of the DMA the wave
// issues next: a new M0, and also, with M0 kept, a different instruction
// offset (a variant that issued later DMAs of a wave with M0 kept and offsets
// of 1-3 KiB failed the same way).  Those lanes' bytes land at the next
// destination and the rows they should have filled keep stale data.  Wait
// states do not bound it (32 still failed under load).  What does: each DMA
// below starts with a load under EXEC = 0 (it touches neither memory nor
// registers), issued while M0 still holds the previous DMA's base and with
// offset 0, the previous DMA's own destination parameters; vector-memory
// instructions issue in order, so the M0 write and the next DMA come after
// it.  That load counts in vmcnt like any other (also measured), so every
// DMA is kVmPerDma vmcnt events.
typedef int v4i_rsrc __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Buffer descriptor of `bytes` bytes at `base` (wave-uniform values).
__device__ __forceinline__ v4i_rsrc make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  v4i_rsrc r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;  // 32-bit data format; offsets past num_records read as zero
  return r;
}

constexpr int kVmPerDma = 2;  // vmcnt events per lds_dma16 / lds_dma4: the EXEC = 0 load and the DMA

// The guard: s_and_saveexec saves EXEC and clears it (SCC is clobbered), the
// EXEC = 0 load names the offset register as its destination (with no lane
// active nothing is written), then M0 takes the new base and EXEC comes
// back; the EXEC restore is also the one wait state the DMA needs after the
// M0 write.
#define DG_M0_GUARD "s_and_saveexec_b64 %0, 0\n\tbuffer_load_dword %1, %1, %2, 0 offen\n\t"

__device__ __forceinline__ void lds_dma16(v4i_rsrc rs, uint32_t voff, uint32_t soff, void* lds_dst) {
  uint64_t exec_save;
  asm volatile(DG_M0_GUARD "s_mov_b32 m0, %4\n\ts_mov_b64 exec, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               : "=&s"(exec_save) : "v"(voff), "s"(rs), "s"(soff), "s"(lds_addr(lds_dst)) : "memory", "m0", "scc");
}

// The same with the non-temporal hint, for operand bytes read exactly once
// (B of a launch whose tiles all share one row block): they then do not
// push the rows every tile re-reads (A) out of the XCD's L2.
__device__ __forceinline__ void lds_dma16_stream(v4i_rsrc rs, uint32_t voff, uint32_t soff, void* lds_dst) {
  uint64_t exec_save;
  asm volatile(DG_M0_GUARD "s_mov_b32 m0, %4\n\ts_mov_b64 exec, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               : "=&s"(exec_save) : "v"(voff), "s"(rs), "s"(soff), "s"(lds_addr(lds_dst)) : "memory", "m0", "scc");
}

__device__ __forceinline__ void lds_dma4(v4i_rsrc rs, uint32_t voff, uint32_t soff, void* lds_dst) {
  uint64_t exec_save;
  asm volatile(DG_M0_GUARD "s_mov_b32 m0, %4\n\ts_mov_b64 exec, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               : "=&s"(exec_save) : "v"(voff), "s"(rs), "s"(soff), "s"(lds_addr(lds_dst)) : "memory", "m0", "scc");
}
#undef DG_M0_GUARD

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
// immediate).  Counts above 63, the counter's range, wait for everything.
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
    DG_VM_CASE(43) DG_VM_CASE(44) DG_VM_CASE(45) DG_VM_CASE(46) DG_VM_CASE(47) DG_VM_CASE(48) DG_VM_CASE(49)
    DG_VM_CASE(50) DG_VM_CASE(51) DG_VM_CASE(52) DG_VM_CASE(53) DG_VM_CASE(54) DG_VM_CASE(55) DG_VM_CASE(56)
    DG_VM_CASE(57) DG_VM_CASE(58) DG_VM_CASE(59) DG_VM_CASE(60) DG_VM_CASE(61) DG_VM_CASE(62) DG_VM_CASE(63)
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

// The f8f6f4 MFMA builtins below pass 0 for both block-scale operands: the
// compiler then emits the unscaled v_mfma_f32_16x16x128_f8f6f4 (8-byte
// encoding) instead of v_mfma_scale_* (16 bytes).  Its products carry no
// block scale; measured bitwise equal to the scaled form with E8M0 scales of
// 2^0 on every workload, and 1-5 % faster on the MFMA-bound loops.  The
// per-block scales are applied in the fp32 promotion instead.

// FP4: format 4 (e2m1) for both operands; a lane's 32 K values are 16 bytes,
// the low four dwords of the operand (the instruction reads only those).
__device__ __forceinline__ v4f mfma_fp4_16x16x128(const v4i& a, const v4i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, zero, 4, 4, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // fmt 0 = e4m3 for both operands; no block scale (see above)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// LDS layout: NST stages, each holding one slab of the A tile, of the B
// tile, the A row scales and the B block scales of that slab (SPS scale
// slabs per stage: 2 for FP4); with SB (single B buffer) the B tile has one
// buffer after the stages instead of one per stage.  The epilogue reuses the
// space for the bf16 output tile.
template <int BM, int BN, int NST, int SPS = 1, bool SB = false>
struct Smem {
  static constexpr int kA = BM * kSlab;
  static constexpr int kB = SB ? 0 : BN * kSlab;  // B bytes in each stage
  static constexpr int kSa = BM * 4 * SPS;
  static constexpr int kSbCount = BN / 128 + 2;  // 128-row blocks a BN-wide tile can touch
  static constexpr int kSb = 256 * SPS;          // one dword DMA instruction's footprint per scale slab
  static constexpr int kStage = kA + kB + kSa + kSb;
  static constexpr int kBShared = NST * kStage;  // SB: offset of the one B buffer
  static constexpr int kOutPitch = BN * 2 + 16;  // bf16 output row pitch (bytes)
  static constexpr int kOut = BM * kOutPitch;
  static constexpr int kMain = NST * kStage + (SB ? BN * kSlab : 0);
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

// Tile number v of workgroup b when only the first `total` workgroups have
// a tile: consecutive numbers go to one XCD (workgroup b runs on XCD b % 8)
// and every XCD gets total / 8 of them, the first total % 8 XCDs one more.
// A bijection of [0, total) for any total.
__device__ __forceinline__ int xcd_deal(int b, int total) {
  const int x = b % kNumXcd;
  const int q = total / kNumXcd, r = total % kNumXcd;
  return x * q + (x < r ? x : r) + b / kNumXcd;
}

// Masked layout: the count of expert e clamped to [0, max_m]; 0 past the
// last expert.
__device__ __forceinline__ int masked_count(const GemmParams& p, int e) {
  if (e >= p.num_groups) return 0;
  const int c = p.masked_m[e];
  return c < 0 ? 0 : (c > p.m ? p.m : c);
}

// Inclusive prefix sum over the 64 lanes of a wave, in DPP moves (no LDS):
// shifts by 1, 2, 4 and 8 lanes inside each row of 16, then row 0's total
// into row 1 and row 2's into row 3 (row_bcast:15), then lane 31's total
// into rows 2 and 3 (row_bcast:31).  Lanes without a source add 0.
__device__ __forceinline__ int wave_prefix_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Number of slab DMA batches a wave has issued after the one of slab kb, at
// the top of iteration kb: the prologue issues slabs 0..NST-2 and iteration
// i issues slab i+NST-1 (nothing for slabs >= KB).
template <int NST>
__device__ __forceinline__ int loads_ahead(int kb, int KB) {
  int n = KB - 1 - kb;
  return n < NST - 2 ? n : NST - 2;
}

// The same for steps of STEP slabs (kPair, kTriple): at the top of the step
// that consumes slabs kb .. kb+STEP-1, the batches issued after the last of
// them (the prologue issues slabs 0..NST-1-STEP, step kb issues
// kb+NST-STEP .. kb+NST-1).
template <int NST, int STEP>
__device__ __forceinline__ int loads_ahead_step(int kb, int KB) {
  const int hi = KB < kb + NST - STEP ? KB : kb + NST - STEP;
  const int lo = KB < kb + STEP ? KB : kb + STEP;
  return hi > lo ? hi - lo : 0;
}

// LDS slot swizzle of tile row r (see the layout note at the top)
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// SCHED selects the main-loop schedule: kInterleaved (every wave loads and
// computes each slab; one barrier per slab), kPingPong (8 waves in two
// groups that alternate load and compute steps, see below) or kSingleB (the
// interleaved loop with one B buffer: every wave reads its B fragments of a
// slab into registers first, and the next slab's B is loaded over them after
// a second barrier; the smaller LDS footprint fits two workgroups per CU,
// whose phases then overlap), or kPair / kTriple (the interleaved loop
// consuming two or three slabs per barrier step, for small tiles whose slab
// steps are latency chains rather than bandwidth: one wait, one barrier and
// one refill per step).
enum Schedule { kInterleaved = 0, kPingPong = 1, kSingleB = 2, kPair = 3, kTriple = 4 };

template <int BM, int BN, int WM, int WN, int NST, int VAR, int SCHED = kInterleaved, int DT = kFp8,
          int EPI = kEpiBf16>
__global__ __launch_bounds__(WM * WN * 64) void gemm_fp8_nt_kernel(GemmParams p) {
  constexpr int kThreads = WM * WN * 64;
  constexpr int kWaves = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int kJa = BM / 8;  // DMA instructions per slab for A (1 KiB each)
  constexpr int kJb = BN / 8;
  constexpr int kSps = DT == kFp4 ? 2 : 1;  // scale slabs per 128-byte slab
  constexpr bool kSB = SCHED == kSingleB;
  // slabs consumed per barrier step of the interleaved loop: kPair takes two,
  // halving the dependent wait / barrier / fragment-read / MFMA steps of a
  // workgroup that has few slabs and tiny tiles (decode shapes)
  constexpr int kStep = SCHED == kPair ? 2 : SCHED == kTriple ? 3 : 1;
  static_assert(kStep == 1 || (NST % kStep == 0 && NST >= 2 * kStep && EPI == kEpiBf16 && VAR == kDense),
                "multi-slab steps: dense, stages a multiple of (and at least twice) the step");
  using S = Smem<BM, BN, NST, kSps, kSB>;
  static_assert(!kSB || NST == 2, "one B buffer: the next slab's B lands while this one is computed");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole fragments");
  static_assert(BM <= kThreads, "row-tag pass needs one thread per tile row");
  static_assert(NST >= 2, "pipeline shape");
  // SwiGLU: a tile covers 128 h columns (one activation scale block), each
  // wave TN / 2 of them: its first TN / 2 tile columns are gate rows of B and
  // its last TN / 2 the matching up rows, so gate and up meet in one lane.
  static_assert(EPI == kEpiBf16 ||
                    ((VAR == kMasked || VAR == kContiguous) && DT == kFp8 && BN == 256 && TN % 32 == 0),
                "SwiGLU epilogue shape");
  static_assert(DT != kFp4 || (VAR == kDense && SCHED != kPingPong && EPI == kEpiBf16),
                "the FP4 path is the dense interleaved GEMM");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_flag;  // contiguous: block expert; split-K: last-arriver flag
  __shared__ uint8_t s_row_ok[BM];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;

  // ---- tile -> (group, tile_m, tile_n[, split])
  int g = 0, tm, tn, tile_id = 0, split = 0;
  int masked_rows = 0;  // masked: the expert's count, clamped to [0, max_m]
  if (VAR == kMasked) {
    // Only tiles with valid rows are visited.  The grid covers every
    // (expert, tile) of the max_m slab, so it does not depend on the counts
    // (a captured graph stays valid as they change); the valid tiles, tiles_n
    // per started BM-row block of each count, are numbered expert-major and
    // the first `total` workgroups take one each, dealt so that an expert's
    // consecutive tiles share one XCD's L2 and the 8 XCDs get equal shares.
    // The other workgroups exit having read the counts.  Every wave derives
    // the same values from the counts (lane e of a pass reads expert e).
    // Experts are read 64 at a time (lane e of a pass holds expert base + e);
    // with at most 64 experts one pass does both the count and the search.
    const auto tiles_of = [&](int c) { return (c + BM - 1) / BM * p.tiles_n; };
    int c = masked_count(p, lane);
    int x = tiles_of(c);
    int incl = wave_prefix_sum(x);
    int total = __builtin_amdgcn_readlane(incl, 63);
    for (int base = 64; base < p.num_groups; base += 64)
      total += __builtin_amdgcn_readlane(wave_prefix_sum(tiles_of(masked_count(p, base + lane))), 63);
    if ((int)blockIdx.x >= total) return;
    const int v = xcd_deal(blockIdx.x, total);
    int before = 0;  // valid tiles of the experts before g
    g = -1;
    for (int base = 0; base < p.num_groups; base += 64) {
      if (base > 0) {
        c = masked_count(p, base + lane);
        x = tiles_of(c);
        incl = wave_prefix_sum(x);
      }
      const unsigned long long hit = __ballot(before + incl > v);
      if (hit) {
        const int l = __ffsll(hit) - 1;
        g = base + l;
        before += __builtin_amdgcn_readlane(incl - x, l);
        masked_rows = __builtin_amdgcn_readlane(c, l);
        break;
      }
      before += __builtin_amdgcn_readlane(incl, 63);
    }
    if (g < 0 || g >= p.num_groups) return;  // not reached: v < total
    const int r = v - before;
    tm = r / p.tiles_n;
    tn = r - tm * p.tiles_n;
  } else if (VAR == kKGrouped) {
    // groups are consecutive runs of tiles, each run in grouped raster order
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    const int per_g = p.tiles_m * p.tiles_n;
    g = t / per_g;
    raster(t - g * per_g, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
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
    // The tile's expert is the largest valid tag of its 128-row alignment
    // block; a tile of fewer rows scans the whole block, so every tile of a
    // block agrees on it.
    constexpr int kBlk = BM < 128 ? 128 : BM;
    static_assert(kThreads >= kBlk, "one row tag per thread");
    const int blk0 = m0 & ~(kBlk - 1);
    if (threadIdx.x == 0) s_flag = -1;
    __syncthreads();
    int tag = -1;
    if (threadIdx.x < kBlk) {
      tag = p.m_indices[blk0 + threadIdx.x];
      if (tag >= 0 && tag < p.num_groups) atomicMax(&s_flag, tag);
    }
    __syncthreads();
    const int expert = s_flag;
    if (expert < 0) return;  // a block of padding rows only
    const int r = blk0 + (int)threadIdx.x - m0;  // this thread's row in the tile
    const bool mine = threadIdx.x < kBlk && r >= 0 && r < BM;
    if (mine) s_row_ok[r] = (tag == expert);
    if (!__syncthreads_or(mine && tag == expert)) return;  // no row of this tile has a result
    B += (size_t)expert * p.n * p.k;
    SFB += (size_t)expert * p.nb_count * p.sk_count;
  } else if (VAR == kMasked) {
    if (m0 >= masked_rows) return;  // not reached: the tile walk above visits valid tiles only
    valid_rows = masked_rows;
    A += (size_t)g * p.m * p.k;
    SFA += (size_t)g * p.sk_count * p.sfa_ld;
    B += (size_t)g * p.n * p.k;
    SFB += (size_t)g * p.nb_count * p.sk_count;
    D += (size_t)g * p.m * p.n;
  }
  // K slabs of this workgroup: [kb0, kb0 + KB) (KB is local; p.kb_count counts the row's 128-byte slabs)
  int kb0 = split * p.split_slabs;
  int KB = p.splits > 1 ? min(p.split_slabs, p.kb_count - kb0) : p.kb_count;
  if (VAR == kKGrouped) {
    // group g's slabs follow the groups before it; sizes are device values,
    // so they are clamped here (negative -> 0, whole slabs, inside K)
    int s0 = 0;
    for (int h = 0; h < g; ++h) s0 += max(p.k_sizes[h], 0) >> 7;
    s0 = min(s0, p.kb_count);
    kb0 = s0;
    KB = min(max(p.k_sizes[g], 0) >> 7, p.kb_count - s0);
    D += (size_t)g * p.m * p.n;
  }
  const int K = p.k;
  // rows worth loading: the masked layout never reads rows past the count
  const int a_rows = VAR == kMasked ? valid_rows : row_limit;

  // ---- slab loader.  One wave-wide DMA instruction moves 1 KiB (one
  // fragment half) into LDS; each wave owns a fixed set of instructions whose
  // per-lane source offsets are computed once per tile.
  // Instruction j of a slab belongs to wave j % kWaves; when the count does
  // not divide evenly (e.g. BN = 224) the first waves issue one more.
  constexpr int kPerWaveA = (kJa + kWaves - 1) / kWaves;
  constexpr int kPerWaveB = (kJb + kWaves - 1) / kWaves;
  uint32_t a_off[kPerWaveA];
  uint32_t b_off[kPerWaveB];
  int a_live = 0;  // A DMA instructions this wave issues per slab (masked skips empty fragments)
  int b_live = 0;  // B DMA instructions this wave issues per slab
  // instruction j covers tile rows 8j..8j+7; lane l fills LDS slot (l & 7) of
  // row 8j + (l >> 3) with the global chunk that belongs there
  #pragma unroll
  for (int jj = 0; jj < kPerWaveA; ++jj) {
    const int j = jj * kWaves + wave;
    const int r = 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(r);
    int row = m0 + r;
    row = row < row_limit ? row : row_limit - 1;
    // row * K is a multiple of 128 and the chunk offset is below 128: OR keeps
    // the offset one 32-bit value (an add lets the compiler form a 64-bit mad)
    a_off[jj] = ((uint32_t)row * (uint32_t)K) | (16u * chunk);
    a_live += (j < kJa && m0 + 8 * j < a_rows) ? 1 : 0;
  }
  #pragma unroll
  for (int jj = 0; jj < kPerWaveB; ++jj) {
    const int j = jj * kWaves + wave;
    const int r = 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(r);
    int row = n0 + r;
    if constexpr (EPI == kEpiSwigluFp8) {
      const int q = r % TN;
      row = (q < TN / 2 ? 0 : p.inter) + tn * (BN / 2) + (r / TN) * (TN / 2) + q % (TN / 2);
    }
    row = row < p.n ? row : p.n - 1;
    b_off[jj] = ((uint32_t)row * (uint32_t)K) | (16u * chunk);
    b_live += j < kJb ? 1 : 0;
  }
  // Row scales: BM floats, one dword instruction per 64 rows, issued by
  // waves 0 .. kSaInsts-1; the B block scales by the last wave.  Waves thus
  // issue different numbers of loads per slab (c_loads): each waits for its
  // own, and the barrier after those waits covers them all.
  constexpr int kSaInsts = (BM + 63) / 64;
  static_assert(kSaInsts <= kWaves, "one wave per 64 rows of row scales");
  const bool sa_wave = wave < kSaInsts;
  const bool sb_wave = wave == kWaves - 1;
  const int sa_blk = sa_wave ? wave : 0;
  const bool sa_lane = sa_blk * 64 + lane < BM;
  uint32_t sa_off;
  {
    int row = m0 + sa_blk * 64 + lane;
    row = row < row_limit ? row : row_limit - 1;
    sa_off = (uint32_t)row;
  }
  // B block scales of the 128-row blocks this tile touches
  // (SwiGLU: the gate block of the tile's h columns, then the up block)
  const int nb0 = n0 >> 7;
  const bool sb_lane = lane < (EPI == kEpiSwigluFp8 ? 2 : S::kSbCount);
  uint32_t sb_off;
  {
    int blk = EPI == kEpiSwigluFp8 ? (lane == 0 ? tn : (p.inter >> 7) + tn) : nb0 + lane;
    blk = blk < p.nb_count ? blk : p.nb_count - 1;
    sb_off = (uint32_t)blk * (uint32_t)p.sk_count;  // sfb row stride: all K scale slabs
  }
  // scale load slots per slab: row and block scales of each of its scale
  // slabs (bf16 operands carry no scales); a wave issues those it owns
  constexpr int kScaleDma = DT == kBf16 ? 0 : 2 * kSps;
  const int c_loads = a_live + b_live + (kScaleDma / 2) * ((sa_wave ? 1 : 0) + (sb_wave ? 1 : 0));

  // Buffer descriptors of this tile's operands (sizes in bytes; the host
  // keeps every operand below 4 GiB).
  const v4i_rsrc rs_a = make_rsrc(A, (uint32_t)row_limit * (uint32_t)K);
  const v4i_rsrc rs_b = make_rsrc(B, (uint32_t)p.n * (uint32_t)K);
  const v4i_rsrc rs_sa = make_rsrc(SFA, (uint32_t)p.sk_count * (uint32_t)p.sfa_ld * 4u);
  const v4i_rsrc rs_sb = make_rsrc(SFB, (uint32_t)p.nb_count * (uint32_t)p.sk_count * 4u);
  // DMA instruction d (0 .. kNumDma-1) of this wave for slab kl into stage
  // buf: the A rows, then the B rows, then the scale loads (row scales and
  // block scales of each scale slab of the slab).
  constexpr int kNumDma = kPerWaveA + kPerWaveB + kScaleDma;
  auto issue_one = [&](int kl, int buf, int d) {
    const int kb = kb0 + kl;  // global slab index
    uint8_t* st = smem + buf * S::kStage;
    if (d < kPerWaveA) {
      const int j = d * kWaves + wave;
      if (kJa % kWaves != 0 && j >= kJa) return;
      if (VAR == kMasked && m0 + 8 * j >= a_rows) return;  // rows without results
      lds_dma16(rs_a, a_off[d], (uint32_t)kb * kSlab, st + j * kDmaBytes);
    } else if (d < kPerWaveA + kPerWaveB) {
      const int jj = d - kPerWaveA;
      const int j = jj * kWaves + wave;
      if (kJb % kWaves != 0 && j >= kJb) return;
      uint8_t* dst = (kSB ? smem + S::kBShared : st + S::kA) + j * kDmaBytes;
      if (p.b_stream) lds_dma16_stream(rs_b, b_off[jj], (uint32_t)kb * kSlab, dst);
      else lds_dma16(rs_b, b_off[jj], (uint32_t)kb * kSlab, dst);
    } else {
      const int e = d - kPerWaveA - kPerWaveB;
      const int h = e >> 1;                 // scale slab of this slab
      const uint32_t ss = (uint32_t)(kb * kSps + h);
      if ((e & 1) == 0) {
        if (sa_wave && sa_lane)
          lds_dma4(rs_sa, sa_off * 4u, ss * (uint32_t)p.sfa_ld * 4u, st + S::kA + S::kB + h * BM * 4 + sa_blk * 256);
      } else {
        if (sb_wave && sb_lane) lds_dma4(rs_sb, sb_off * 4u, ss * 4u, st + S::kA + S::kB + S::kSa + h * 256);
      }
    }
  };
  auto issue_slab = [&](int kl, int buf) {
    #pragma unroll
    for (int d = 0; d < kNumDma; ++d) issue_one(kl, buf, d);
  };

  v4f acc[FM][FN];
  #pragma unroll
  for (int i = 0; i < FM; ++i)
    #pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // index of each fragment's B scale block among the tile's blocks
  int sb_idx[FN];
  #pragma unroll
  for (int j = 0; j < FN; ++j)
    sb_idx[j] = EPI == kEpiSwigluFp8 ? (j < FN / 2 ? 0 : 1) : ((n0 + wn * TN + j * 16) >> 7) - nb0;
  // a wave's columns lie in one block
  constexpr bool kSbUniform = EPI == kEpiBf16 && (128 % TN) == 0;
  // Otherwise they lie in two (TN = 112 of a 224-wide tile, or the gate and up
  // halves of a SwiGLU tile): fragments j < sb_split take the first block's
  // scale, the others the second's.  The fp8 main loop below is compiled once
  // per possible split (the choice is made once per tile), so the scale
  // products are formed once per row fragment and block.
  static_assert(TN <= 128, "a wave's columns span at most two B scale blocks");
  int sb_split = FN;
  #pragma unroll
  for (int j = FN - 1; j > 0; --j)
    if (sb_idx[j] != sb_idx[0]) sb_split = j;
  sb_split = __builtin_amdgcn_readfirstlane(sb_split);
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

  if constexpr (SCHED == kPingPong) {
    // ---- ping-pong schedule (256 x 256 tile, 8 waves, 2 stages).  Waves
    // 0-3 (group 0, tile rows 0-127) and waves 4-7 (group 1, rows 128-255)
    // sit two per SIMD, one of each group.  Each wave cuts its slab work
    // into kNch chunks of kFh A fragments and alternates a load step (LDS ->
    // registers: the slab's B fragments with chunk 0, then the chunk's A
    // fragments and row scales) and a compute step (the chunk's MFMAs and
    // promotions), with a workgroup barrier after every step.  Group 1 runs
    // one step behind group 0, so on every SIMD one wave feeds the matrix
    // core while the other moves data: LDS reads and LDS DMA overlap MFMA
    // work instead of alternating with it.  Steps of slab kb (2 * kNch):
    //
    //   step 2c     group 0: load (kb, c)        group 1: compute the chunk before (kb, c)
    //   step 2c+1   group 0: compute (kb, c)     group 1: load (kb, c)
    //
    // with the DMA of slab kb+1 issued in each group's first load step of
    // slab kb.  Slab kb is read only in its own 2 * kNch steps; slab kb+1
    // goes to the other stage, last read in the step before, and every wave
    // waits for its own DMA before the barrier that closes slab kb.  Every
    // step ends with lgkmcnt(0), so no LDS read is in flight when a stage is
    // refilled.
    static_assert(BM == 256 && BN == 256 && WM == 2 && WN == 4 && NST == 2, "ping-pong tile shape");
    static_assert(DT == kFp8, "ping-pong schedule is written for fp8 operands");
    static_assert(kSbUniform || EPI == kEpiSwigluFp8, "a wave's columns must share one B scale block");
    constexpr int kFh = 4;          // A fragments per chunk
    constexpr int kNch = FM / kFh;  // chunks per slab
    const int grp = wm;
    // The per-fragment validity test is a run-time branch for every variant
    // (dense: always true).  The uniform branches cost a scalar compare each,
    // and they keep the scheduler from hoisting the next steps' loads, which
    // otherwise raises register pressure past the 256-VGPR budget.
    asm volatile("" : "+s"(fm_valid));
    v8i bq[FN];
    v8i aq[kFh];
    v4f sq[kFh];
    float sbq = 0.f;   // B scale of the wave's columns (SwiGLU: of the gate half)
    float sbq2 = 0.f;  // SwiGLU: B scale of the up half
    // LDS reads address a per-step base register plus an immediate offset;
    // the opaque base keeps the compiler from precomputing a register per
    // fragment and stage (a stage is wider than the 16-bit offset field).
    auto lds_base = [&](const void* p0) {
      uint32_t b = lds_addr(p0);
      asm volatile("" : "+v"(b));
      return b;
    };
    auto rd16 = [&](uint32_t addr) { return *(const __attribute__((address_space(3))) v4i*)(uintptr_t)addr; };
    auto load_chunk = [&](int kb, int c) {
      const uint8_t* st = smem + (kb & 1) * S::kStage;
      if (c == 0) {
        const float* sSb = (const float*)(st + S::kA + S::kB + S::kSa);
        sbq = sSb[sb_idx[0]];
        if constexpr (EPI == kEpiSwigluFp8) sbq2 = sSb[1];
        const uint32_t bb_lo = lds_base(st + S::kA + wn * FN * 2048) + frag_lo;
        const uint32_t bb_hi = bb_lo - frag_lo + frag_hi;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v4i lo = rd16(bb_lo + j * 2048);
          const v4i hi = rd16(bb_hi + j * 2048);
          bq[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
      const uint32_t ab_lo = lds_base(st + (wm * FM + c * kFh) * 2048) + frag_lo;
      const uint32_t ab_hi = ab_lo - frag_lo + frag_hi;
      const uint32_t sab = lds_base(st + S::kA + S::kB + (wm * TM + c * kFh * 16) * 4) + 16 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < kFh; ++i) {
        if (c * kFh + i >= fm_valid) continue;
        const v4i lo = rd16(ab_lo + i * 2048);
        const v4i hi = rd16(ab_hi + i * 2048);
        aq[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const v4i sv = rd16(sab + i * 64);
        sq[i] = v4f{__int_as_float(sv[0]), __int_as_float(sv[1]), __int_as_float(sv[2]), __int_as_float(sv[3])};
      }
    };
    // MFMA of fragment t, promotion of fragment t - kLagPP (its result is
    // ready by then); the fixed order keeps promotions away from their MFMA.
    auto compute_chunk = [&](auto cc) {
      constexpr int c = decltype(cc)::value;
      constexpr int kLagPP = 4;  // measured: level with 2 on the masked GEMM, 3 % ahead with SwiGLU
      v4f pr[kLagPP + 1];
#pragma unroll
      for (int t = 0; t < kFh * FN + kLagPP; ++t) {
        if (t < kFh * FN) {
          const int i = t / FN, j = t % FN;
          if (c * kFh + i < fm_valid) pr[t % (kLagPP + 1)] = mfma_fp8_16x16x128(aq[i], bq[j]);
        }
        if (t >= kLagPP) {
          const int u = t - kLagPP;
          const int i = u / FN, j = u % FN;
          if (c * kFh + i < fm_valid) {
            const v4f sc = sq[i] * ((EPI == kEpiSwigluFp8 && j >= FN / 2) ? sbq2 : sbq);
            const v4f pv = pr[u % (kLagPP + 1)];
            acc[c * kFh + i][j][0] = __builtin_fmaf(pv[0], sc[0], acc[c * kFh + i][j][0]);
            acc[c * kFh + i][j][1] = __builtin_fmaf(pv[1], sc[1], acc[c * kFh + i][j][1]);
            acc[c * kFh + i][j][2] = __builtin_fmaf(pv[2], sc[2], acc[c * kFh + i][j][2]);
            acc[c * kFh + i][j][3] = __builtin_fmaf(pv[3], sc[3], acc[c * kFh + i][j][3]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto end_step = [&]() {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
      block_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // static loop over the chunks of a slab (c is a compile-time constant)
    auto for_chunks = [&](auto body) {
      [&]<int... C>(std::integer_sequence<int, C...>) {
        (body(std::integral_constant<int, C>{}), ...);
      }(std::make_integer_sequence<int, kNch>{});
    };

    if (KB > 0) issue_slab(0, 0);
    wait_vmem_all();
    block_barrier();
    // The two groups run separate copies of the loop (the same number of
    // barriers each): with one loop and per-step branches on the group, the
    // compiler cannot tell the paths apart and keeps extra live copies of
    // the fragment registers.
    if (grp == 0) {
      for (int kb = 0; kb < KB; ++kb) {
        for_chunks([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          load_chunk(kb, c);
          if (c == 0 && kb + 1 < KB) issue_slab(kb + 1, (kb + 1) & 1);
          end_step();
          compute_chunk(cc);
          if (c == kNch - 1) wait_vmem_all();  // this wave's share of slab kb+1 has landed
          end_step();
        });
      }
      end_step();  // group 1 finishes its last chunk
    } else {
      for (int kb = 0; kb < KB; ++kb) {
        for_chunks([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          if (c == 0) {
            if (kb > 0) compute_chunk(std::integral_constant<int, kNch - 1>{});
          } else {
            compute_chunk(std::integral_constant<int, (c > 0 ? c - 1 : 0)>{});
          }
          end_step();
          load_chunk(kb, c);
          if (c == 0 && kb + 1 < KB) issue_slab(kb + 1, (kb + 1) & 1);
          if (c == kNch - 1) wait_vmem_all();
          end_step();
        });
      }
      if (KB > 0) compute_chunk(std::integral_constant<int, kNch - 1>{});
      end_step();
    }
  } else {
    // ---- prologue: DMA of slabs 0..NST-1-kStep
    #pragma unroll
    for (int s0 = 0; s0 <= NST - 1 - kStep; ++s0)
      if (s0 < KB) issue_slab(s0, s0);

    // the main loop, compiled once per B scale split (kSplit: fragments of
    // this wave in the first block; FN when all are in one)
    auto main_loop = [&](auto split_c) {
    constexpr int kSplit = decltype(split_c)::value;
    for (int kb2 = 0; kb2 < KB; kb2 += kStep) {
      // the step's slabs (kb2, and kb2+1 for kPair) must have landed (in
      // every wave: then the barrier); the loads issued after them may stay
      // in flight.
      wait_vmem_dyn(kVmPerDma * c_loads *
                    (kStep == 1 ? loads_ahead<NST>(kb2, KB) : loads_ahead_step<NST, kStep>(kb2, KB)));
      block_barrier();  // also: every wave is done with the stages about to be refilled
      __builtin_amdgcn_sched_barrier(0);
      #pragma unroll
      for (int q = 0; q < kStep; ++q)
        if (!kSB && kb2 + NST - kStep + q < KB) issue_slab(kb2 + NST - kStep + q, (kb2 + NST - kStep + q) % NST);
      __builtin_amdgcn_sched_barrier(0);

    #pragma unroll
    for (int sub = 0; sub < kStep; ++sub) {
      const int kb = kb2 + sub;
      if (kStep > 1 && kb >= KB) break;
      const uint8_t* st = smem + (kb % NST) * S::kStage;
      const uint8_t* sA = st;
      const uint8_t* sB = kSB ? smem + S::kBShared : st + S::kA;
      const float* sSa = (const float*)(st + S::kA + S::kB);
      const float* sSb = (const float*)(st + S::kA + S::kB + S::kSa);

      float sbv[FN];
      #pragma unroll
      for (int j = 0; j < FN; ++j) sbv[j] = DT != kBf16 ? sSb[kSbUniform ? sb_idx[0] : sb_idx[j]] : 0.f;

      v8i bf[FN];
      #pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int f = wn * FN + j;
        const v4i lo = *(const v4i*)(sB + f * 2048 + frag_lo);
        const v4i hi = *(const v4i*)(sB + f * 2048 + frag_hi);
        bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      if constexpr (kSB) {
        // every wave holds its B fragments of slab kb: the B buffer is free
        // for slab kb + 1 (and the other A stage since the first barrier)
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's B reads are done
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (kb + 1 < KB) issue_slab(kb + 1, (kb + 1) % NST);
        __builtin_amdgcn_sched_barrier(0);
      }

      // Software pipeline over the wave's FM x FN fragments (row-major order t):
      // A rows are read from LDS kPf rows ahead, and fragment t's promotion
      // runs kLag fragments after its MFMA, so each MFMA has independent
      // promotion FMAs of earlier fragments to co-issue with.
      constexpr int kPf = FM < 2 ? FM : 2;
      constexpr int kAbuf = kPf + 1;
      constexpr int kLag = 4;  // measured: 4 >= 2 on every large shape; 6 and 8 cost registers
      // row scales stay live from their load (kPf rows ahead of the MFMAs) to
      // the promotion kLag fragments behind them: up to kPf + 1 + ceil(kLag / FN)
      // row fragments at once
      constexpr int kSabuf = kPf + 2 + (kLag - 1) / FN;
      constexpr int F = FM * FN;
      v8i abuf[kAbuf];
      v4f sabuf[kSabuf];
      v4f sabuf1[DT == kFp4 ? kSabuf : 1];  // FP4: row scales of the second scale slab
      v4f pr[kLag + 1];
      auto load_a = [&](int i) {
        const int f = wm * FM + i;
        const v4i lo = *(const v4i*)(sA + f * 2048 + frag_lo);
        const v4i hi = *(const v4i*)(sA + f * 2048 + frag_hi);
        abuf[i % kAbuf] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (DT != kBf16) sabuf[i % kSabuf] = *(const v4f*)(sSa + wm * TM + i * 16 + 4 * (lane >> 4));
        if constexpr (DT == kFp4) sabuf1[i % kSabuf] = *(const v4f*)(sSa + BM + wm * TM + i * 16 + 4 * (lane >> 4));
      };
      #pragma unroll
      for (int i = 0; i < kPf; ++i)
        if (VAR != kMasked || i < fm_valid) load_a(i);
      if constexpr (DT == kBf16) {
        // bf16: a slab row is 64 K values; the fragment read's low half
        // feeds one K=32 MFMA and its high half a second one, accumulating
        // in place (no scales, no promotion).  All low-half MFMAs of an A
        // fragment come before the high-half ones, so each MFMA's
        // predecessor on the same accumulator is FN-1 MFMAs back.
        auto lo8 = [](const v8i& x) { return __builtin_bit_cast(v8bf, v4i{x[0], x[1], x[2], x[3]}); };
        auto hi8 = [](const v8i& x) { return __builtin_bit_cast(v8bf, v4i{x[4], x[5], x[6], x[7]}); };
        #pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (VAR == kMasked && i >= fm_valid) continue;
          if (i + kPf < FM && (VAR != kMasked || i + kPf < fm_valid)) load_a(i + kPf);
          #pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo8(abuf[i % kAbuf]), lo8(bf[j]), acc[i][j], 0, 0, 0);
          #pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi8(abuf[i % kAbuf]), hi8(bf[j]), acc[i][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        continue;
      }
      if constexpr (DT == kFp4) {
        // FP4: the low 16 bytes of every fragment read lie in the slab's
        // first 64 bytes (its first scale slab, K 0..127 of the 256), the
        // high 16 bytes in the second; one FP4 MFMA per half, each promoted
        // with the scales of its own scale slab.  All MFMAs of an A fragment
        // are issued before its promotions.
        float sbv1[FN];
        #pragma unroll
        for (int j = 0; j < FN; ++j) sbv1[j] = sSb[64 + (kSbUniform ? sb_idx[0] : sb_idx[j])];
        auto lo4 = [](const v8i& x) { return v4i{x[0], x[1], x[2], x[3]}; };
        auto hi4 = [](const v8i& x) { return v4i{x[4], x[5], x[6], x[7]}; };
        #pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (i + kPf < FM) load_a(i + kPf);
          v4f p0[FN], p1[FN];
          #pragma unroll
          for (int j = 0; j < FN; ++j) p0[j] = mfma_fp4_16x16x128(lo4(abuf[i % kAbuf]), lo4(bf[j]));
          #pragma unroll
          for (int j = 0; j < FN; ++j) p1[j] = mfma_fp4_16x16x128(hi4(abuf[i % kAbuf]), hi4(bf[j]));
          const v4f sa0 = sabuf[i % kSabuf], sa1 = sabuf1[i % kSabuf];
          #pragma unroll
          for (int j = 0; j < FN; ++j) {
            const v4f sc0 = sa0 * sbv[j];
            const v4f sc1 = sa1 * sbv1[j];
            #pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[i][j][e] = __builtin_fmaf(p1[j][e], sc1[e], __builtin_fmaf(p0[j][e], sc0[e], acc[i][j][e]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        continue;
      }
      {
        const float sb_first = sbv[0], sb_second = sbv[FN - 1];
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
              const v4f sc = sabuf[i % kSabuf] * (j < kSplit ? sb_first : sb_second);
              const v4f pv = pr[u % (kLag + 1)];
              acc[i][j][0] = __builtin_fmaf(pv[0], sc[0], acc[i][j][0]);
              acc[i][j][1] = __builtin_fmaf(pv[1], sc[1], acc[i][j][1]);
              acc[i][j][2] = __builtin_fmaf(pv[2], sc[2], acc[i][j][2]);
              acc[i][j][3] = __builtin_fmaf(pv[3], sc[3], acc[i][j][3]);
            }
          }
          // keep this order: a promotion must not move up next to the MFMA
          // that produces its input (that stalls the wave on the result)
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    }
    };
    if constexpr (kSbUniform || DT != kFp8) {
      main_loop(std::integral_constant<int, FN>{});
    } else {
      [&]<int... J>(std::integer_sequence<int, J...>) {
        (void)((sb_split == J + 1 ? (main_loop(std::integral_constant<int, J + 1>{}), true) : false) || ...);
      }(std::make_integer_sequence<int, FN>{});
    }
  }

  wait_vmem_all();  // no LDS DMA may be in flight past this point

  if constexpr (EPI == kEpiSwigluFp8) {
    // ---- SwiGLU epilogue: h = silu(gate) * up in fp32 from the
    // accumulators, then h's 1 x 128 activation quantisation.  The tile holds
    // all 128 h columns of its block, so a row's amax is a max over the 16
    // lanes of a fragment row, the wave's fragments and the WN waves of a
    // tile row (through LDS).  One thread per tile row then forms the row's
    // scale and its reciprocal, and the waves quantise their h values with
    // them.  Codes are staged in LDS and leave as 16-byte row stores; scales
    // go to the slab-major layout the masked (contiguous) GEMM reads its A
    // scales from.  Rows past the expert's count (contiguous: rows that do
    // not carry the tile's expert tag) are not written.
    constexpr int FH = FN / 2;
    constexpr int kHalf = TN / 2;             // h columns per wave
    constexpr int kCodePitch = BN / 2 + 16;   // bytes per staged code row
    static_assert(WN * BM * 4 + 2 * BM * 4 + BM * kCodePitch <= S::kBytes, "SwiGLU staging fits the LDS");
    static_assert(BM <= kThreads, "one thread per tile row forms the scales");
    block_barrier();  // every wave is done reading the last stage
    float* s_amax = (float*)smem;                 // [WN][BM] per-wave row amax
    float* s_sc = s_amax + WN * BM;               // [BM] row scale
    float* s_rc = s_sc + BM;                      // [BM] its refined reciprocal
    uint8_t* s_code = (uint8_t*)(s_rc + BM);      // [BM][kCodePitch]
    // max over the 16 lanes of a DPP row (the lanes that hold one fragment
    // row): quad swaps, then mirrors inside 8 and 16 lanes
    auto row16_max = [](float v) {
      auto dpp = [](float x, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false));
      };
      v = fmaxf(v, dpp(v, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
      v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
      v = fmaxf(v, dpp(v, std::integral_constant<int, 0x141>{}));  // row_half_mirror
      v = fmaxf(v, dpp(v, std::integral_constant<int, 0x140>{}));  // row_mirror
      return v;
    };
    #pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i >= fm_valid) continue;
      #pragma unroll
      for (int e = 0; e < 4; ++e) {
        float mx = 0.f;
        #pragma unroll
        for (int jh = 0; jh < FH; ++jh) {
          // silu(g) = g / (1 + exp(-g)), the quotient through v_rcp_f32 (1 ulp);
          // exp(-g) = inf for g < -88 gives -0, the rounded value of silu there
          const float gt = acc[i][jh][e];
          const float h = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * acc[i][jh + FH][e];
          acc[i][jh][e] = h;
          mx = fmaxf(mx, fabsf(h));
        }
        mx = row16_max(mx);
        if ((lane & 15) == 0) s_amax[wn * BM + wm * TM + i * 16 + 4 * (lane >> 4) + e] = mx;
      }
    }
    block_barrier();
    if (threadIdx.x < BM) {
      const int rl = threadIdx.x;
      float amax = s_amax[rl];
      #pragma unroll
      for (int w = 1; w < WN; ++w) amax = fmaxf(amax, s_amax[w * BM + rl]);
      amax = fmaxf(amax, kAmaxFloor);
      const float sc = amax / kE4m3Max;  // correctly rounded (build flag)
      // reciprocal refined by one Newton step (for the quotients below)
      float y = __builtin_amdgcn_rcpf(sc);
      y = __builtin_fmaf(__builtin_fmaf(-sc, y, 1.f), y, y);
      s_sc[rl] = sc;
      s_rc[rl] = y;
      // (contiguous: g is 0, h rows are the rows of A; rows of another
      // expert's tag or padding get nothing)
      if (m0 + rl < valid_rows && (VAR != kContiguous || s_row_ok[rl]))
        p.hs[((size_t)g * (p.inter >> 7) + tn) * p.sfa_ld + m0 + rl] = sc;
    }
    block_barrier();
    #pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i >= fm_valid) continue;
      const int r0 = wm * TM + i * 16 + 4 * (lane >> 4);  // the lane's 4 rows: r0 .. r0 + 3
      const v4f sc4 = *(const v4f*)(s_sc + r0);
      const v4f y4 = *(const v4f*)(s_rc + r0);
      #pragma unroll
      for (int e = 0; e < 4; ++e) {
        // h / sc by Markstein's method: the quotient through the refined
        // reciprocal, corrected once by its exact residual (correctly rounded
        // whenever the refined reciprocal is; sc lies in [2^-23, 2^120], so
        // nothing over- or underflows)
        #pragma unroll
        for (int jh = 0; jh < FH; ++jh) {
          const float hv = acc[i][jh][e];
          const float q0 = hv * y4[e];
          const float q = __builtin_fmaf(__builtin_fmaf(-q0, sc4[e], hv), y4[e], q0);
          s_code[(r0 + e) * kCodePitch + wn * kHalf + jh * 16 + (lane & 15)] = e4m3_code(q);
        }
      }
    }
    block_barrier();
    const int rows_here = min(BM, valid_rows - m0);
    constexpr int kChunks = BN / 2 / 16;  // 16-byte chunks per h row of the tile
    uint8_t* HQ = p.hq + (size_t)g * p.m * p.inter + (size_t)tn * (BN / 2);
    for (int idx = threadIdx.x; idx < BM * kChunks; idx += kThreads) {
      const int rl = idx / kChunks, ch = idx % kChunks;
      if (rl >= rows_here) break;
      if (VAR == kContiguous && !s_row_ok[rl]) continue;
      *(v4i*)(HQ + (size_t)(m0 + rl) * p.inter + ch * 16) = *(const v4i*)(s_code + rl * kCodePitch + ch * 16);
    }
    return;
  }

  // ---- split-K fix-up: publish this split's partial tile; the last split
  // to arrive adds all partials in split order (deterministic) and goes on to
  // store D.  Partials are laid out fragment-native (each lane owns 16
  // contiguous bytes per fragment).  The reducer reads up to kChunk splits'
  // partials per batch, issuing loads for existing splits only.
  //
  // Why the hand-off is ordered across the per-XCD L2s without a release /
  // acquire pair: the partial stores and the reducer's loads carry SC1, the
  // agent-scope cache policy (the form of a relaxed agent-scope atomic store
  // and load on this target), so a store completes only once it is written
  // beyond the issuing XCD's L2 at the device coherence point, and a load is
  // served from that point, not from a possibly stale L1 or L2 line.  Each
  // thread waits vmcnt(0) for its own stores to complete; the barrier then
  // puts every thread's completed stores before thread 0's agent-scope
  // atomic, performed at the same point.  The reducer's atomic returns after
  // every other split's atomic, hence after all their stores completed; its
  // loads are issued only after that return is seen (a data dependency
  // through the barrier), so they find the stored values.  A release/acquire
  // atomic would add an L2 write-back and invalidate of every dirty line,
  // which measured twice as slow as these coherent accesses on decode shapes.
  if constexpr (VAR == kDense && SCHED != kPingPong) if (p.splits > 1) {
    constexpr int kTileFloats = BM * BN;
    constexpr int kChunkMax = (FM * FN * 4) >= 128 ? 1 : 128 / (FM * FN * 4);
    constexpr int kChunk = kChunkMax > 8 ? 8 : kChunkMax;
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
          for (int j = 0; j < FN; ++j) {
            // only the splits that exist: a load past the last one would
            // return zero but still cost its trip through the texture path
            part_v[c][i][j] = v4f{0.f, 0.f, 0.f, 0.f};
            if (sp0 + c < p.splits)
              part_v[c][i][j] = __builtin_amdgcn_raw_buffer_load_b128(
                  rs, ((sp0 + c) * kTileFloats + (((wave * FM + i) * FN + j) * 64 + lane) * 4) * 4, 0, kCpolSc1);
          }
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
