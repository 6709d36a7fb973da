// C ABI of the FP8 block-scaled NT GEMM library (declared in include/dg.h):
// argument validation, per-shape choice among the compile-time tile
// configurations, and the kernel launches.  The pages' DeepGEMM compiles a
// kernel per shape at run time ("DeepSeek open-source week day 3",
// technical features, JIT item); here every configuration is compiled ahead
// of time for gfx950 and the host picks one per call from (M, N, K, groups,
// CU count), which keeps the call free of compilation, allocation and
// synchronisation.
#include "../../include/dg.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "gemm_kernel.h"
#include "quant_kernel.h"

namespace {

thread_local std::string g_last_error;
// one-shot profiling events for the next GEMM launch on this thread
thread_local hipEvent_t g_prof_start = nullptr;
thread_local hipEvent_t g_prof_stop = nullptr;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return DG_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int sfa_ld(int m) { return (m + 3) / 4 * 4; }

bool log_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("DG_LOG");
    v = (e && *e && *e != '0') ? 1 : 0;
  }
  return v == 1;
}

// ---- per-device facts, queried once per device
struct DeviceInfo {
  int cus = 0;
  bool ok = false;
};
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

int current_device(int* dev, DeviceInfo** info) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(DG_ERR_NO_DEVICE, "no HIP device is visible");
  }
  if (hipGetDevice(dev) != hipSuccess || *dev < 0 || *dev >= kMaxDevices)
    return fail(DG_ERR_NO_DEVICE, "hipGetDevice failed");
  const int d = *dev;
  std::call_once(g_dev_once[d], [d]() {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, d) != hipSuccess) return;
    g_dev[d].cus = prop.multiProcessorCount;
    g_dev[d].ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  });
  if (!g_dev[d].ok) return fail(DG_ERR_NO_DEVICE, "device %d is not a gfx950 GPU", d);
  *info = &g_dev[d];
  return DG_OK;
}

// ---- tile configurations (compile-time instantiations; the host picks one)
struct Config {
  const char* name;
  int variant, bm, bn, wm, wn, nst, sched, dtype, epi;
  const void* fn;
  int smem;
  int threads() const { return wm * wn * 64; }
};

template <int BM, int BN, int WM, int WN, int NST, int VAR, int SCHED = dg::kInterleaved, int DT = dg::kFp8,
          int EPI = dg::kEpiBf16>
Config make_config(const char* name) {
  return Config{name, VAR, BM, BN, WM, WN, NST, SCHED, DT, EPI,
                reinterpret_cast<const void*>(&dg::gemm_fp8_nt_kernel<BM, BN, WM, WN, NST, VAR, SCHED, DT, EPI>),
                dg::Smem<BM, BN, NST, DT == dg::kFp4 ? 2 : 1, SCHED == dg::kSingleB>::kBytes};
}

const Config* configs(int* count) {
  static const Config table[] = {
      // dense
      make_config<256, 256, 2, 4, 2, dg::kDense>("dense_256x256_w8_s2"),
      make_config<256, 256, 2, 4, 2, dg::kDense, dg::kPingPong>("dense_256x256_w8_s2_pp"),
      make_config<128, 256, 1, 4, 2, dg::kDense, dg::kSingleB>("dense_128x256_w4_s2_sb"),
      make_config<256, 224, 4, 2, 2, dg::kDense>("dense_256x224_w8_s2"),
      make_config<128, 256, 1, 4, 3, dg::kDense>("dense_128x256_w4_s3_wide"),
      make_config<256, 128, 4, 2, 3, dg::kDense>("dense_256x128_w8_s3"),
      make_config<256, 128, 2, 2, 2, dg::kDense>("dense_256x128_w4_s2"),
      make_config<256, 128, 2, 2, 3, dg::kDense>("dense_256x128_w4_s3"),
      make_config<128, 256, 2, 2, 3, dg::kDense>("dense_128x256_w4_s3"),
      make_config<128, 256, 2, 4, 3, dg::kDense>("dense_128x256_w8_s3"),
      make_config<128, 128, 2, 2, 3, dg::kDense>("dense_128x128_w4_s3"),
      make_config<128, 128, 2, 2, 2, dg::kDense>("dense_128x128_w4_s2"),
      make_config<64, 64, 1, 4, 3, dg::kDense>("dense_64x64_w4_s3"),
      // skinny M: split-K over workgroups
      make_config<64, 64, 1, 4, 8, dg::kDense>("dense_64x64_w4_s8"),
      make_config<64, 32, 2, 2, 4, dg::kDense>("dense_64x32_w4_s4"),
      // contiguous (block rows <= the 128-row alignment)
      make_config<128, 256, 2, 4, 3, dg::kContiguous>("contig_128x256_w8_s3"),
      make_config<128, 128, 2, 2, 3, dg::kContiguous>("contig_128x128_w4_s3"),
      make_config<128, 128, 2, 2, 2, dg::kContiguous>("contig_128x128_w4_s2"),
      make_config<128, 256, 2, 4, 2, dg::kContiguous>("contig_128x256_w8_s2"),
      make_config<128, 256, 1, 4, 3, dg::kContiguous>("contig_128x256_w4_s3"),
      make_config<128, 256, 1, 4, 2, dg::kContiguous, dg::kSingleB>("contig_128x256_w4_s2_sb"),
      make_config<128, 256, 1, 4, 2, dg::kContiguous>("contig_128x256_w4_s2"),
      make_config<64, 64, 1, 4, 3, dg::kContiguous>("contig_64x64_w4_s3"),
      // masked
      make_config<256, 256, 2, 4, 2, dg::kMasked>("masked_256x256_w8_s2"),
      make_config<256, 256, 2, 4, 2, dg::kMasked, dg::kPingPong>("masked_256x256_w8_s2_pp"),
      make_config<256, 128, 4, 2, 2, dg::kMasked>("masked_256x128_w8_s2"),
      make_config<256, 128, 1, 4, 2, dg::kMasked>("masked_256x128_w4_s2"),
      make_config<256, 128, 1, 4, 3, dg::kMasked>("masked_256x128_w4_s3"),
      make_config<64, 64, 1, 4, 3, dg::kMasked>("masked_64x64_w4_s3"),
      make_config<128, 256, 2, 4, 3, dg::kMasked>("masked_128x256_w8_s3"),
      // K-grouped
      make_config<256, 256, 2, 4, 2, dg::kKGrouped>("kgrouped_256x256_w8_s2"),
      make_config<128, 128, 2, 2, 2, dg::kKGrouped>("kgrouped_128x128_w4_s2"),
      // BF16 dense (find_config matches the dtype too, so DG_FORCE_CONFIG
      // names pick among these only for the bf16 entry point)
      make_config<256, 256, 2, 4, 2, dg::kDense, dg::kInterleaved, dg::kBf16>("bf16_256x256_w8_s2"),
      make_config<128, 128, 2, 2, 2, dg::kDense, dg::kInterleaved, dg::kBf16>("bf16_128x128_w4_s2"),
      make_config<64, 32, 2, 2, 4, dg::kDense, dg::kInterleaved, dg::kBf16>("bf16_64x32_w4_s4"),
      make_config<64, 64, 1, 4, 3, dg::kDense, dg::kInterleaved, dg::kBf16>("bf16_64x64_w4_s3"),
      // FP4 (e2m1) dense (selected the same way by dtype)
      make_config<256, 256, 2, 4, 2, dg::kDense, dg::kInterleaved, dg::kFp4>("fp4_256x256_w8_s2"),
      make_config<128, 128, 2, 2, 2, dg::kDense, dg::kInterleaved, dg::kFp4>("fp4_128x128_w4_s2"),
      make_config<64, 32, 2, 2, 4, dg::kDense, dg::kInterleaved, dg::kFp4>("fp4_64x32_w4_s4"),
      make_config<64, 64, 1, 4, 3, dg::kDense, dg::kInterleaved, dg::kFp4>("fp4_64x64_w4_s3"),
      // MoE FC1 + SwiGLU + FP8 requantisation, masked layout (a 256-column
      // tile = 128 gate + 128 up columns = one 128-wide block of h)
      make_config<256, 256, 2, 4, 2, dg::kMasked, dg::kPingPong, dg::kFp8, dg::kEpiSwigluFp8>("swiglu_256x256_w8_s2_pp"),
      make_config<256, 256, 2, 4, 2, dg::kMasked, dg::kInterleaved, dg::kFp8, dg::kEpiSwigluFp8>("swiglu_256x256_w8_s2"),
      make_config<128, 256, 2, 4, 3, dg::kMasked, dg::kInterleaved, dg::kFp8, dg::kEpiSwigluFp8>("swiglu_128x256_w8_s3"),
      make_config<64, 256, 1, 4, 3, dg::kMasked, dg::kInterleaved, dg::kFp8, dg::kEpiSwigluFp8>("swiglu_64x256_w4_s3"),
  };
  *count = sizeof(table) / sizeof(table[0]);
  return table;
}

const Config* find_config(const char* name, int variant, int dtype = dg::kFp8, int epi = dg::kEpiBf16) {
  int cnt = 0;
  const Config* t = configs(&cnt);
  for (int i = 0; i < cnt; ++i)
    if (t[i].variant == variant && t[i].dtype == dtype && t[i].epi == epi && strcmp(t[i].name, name) == 0)
      return &t[i];
  return nullptr;
}

// DG_FORCE_CONFIG=<name> pins the configuration of the variant it names (for
// tuning sweeps); an unknown name is an error rather than silently ignored.
int forced_config(int variant, const Config** out, int dtype = dg::kFp8, int epi = dg::kEpiBf16) {
  *out = nullptr;
  const char* e = getenv("DG_FORCE_CONFIG");
  if (!e || !*e) return DG_OK;
  int cnt = 0;
  const Config* t = configs(&cnt);
  bool known = false;
  for (int i = 0; i < cnt; ++i) known = known || strcmp(t[i].name, e) == 0;
  if (!known) return fail(DG_ERR_INVALID_ARGUMENT, "DG_FORCE_CONFIG names no configuration: %s", e);
  *out = find_config(e, variant, dtype, epi);
  return DG_OK;
}

std::once_flag g_attr_once;
hipError_t g_attr_err = hipSuccess;
constexpr int kMaxConfigs = 64;
int g_per_cu[kMaxConfigs];  // resident workgroups per CU of each configuration (0: not known)

void set_kernel_attributes() {
  int cnt = 0;
  const Config* t = configs(&cnt);
  for (int i = 0; i < cnt; ++i) {
    hipError_t e = hipFuncSetAttribute(t[i].fn, hipFuncAttributeMaxDynamicSharedMemorySize, t[i].smem);
    if (e != hipSuccess) {
      g_attr_err = e;
      continue;
    }
    int blocks = 0;
    if (i < kMaxConfigs &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, t[i].fn, t[i].threads(), t[i].smem) == hipSuccess)
      g_per_cu[i] = blocks;
    else
      (void)hipGetLastError();
  }
}

int ensure_kernel_attributes() {
  std::call_once(g_attr_once, set_kernel_attributes);
  if (g_attr_err != hipSuccess)
    return fail(DG_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(g_attr_err));
  return DG_OK;
}

// Workgroups of configuration c that one CU holds at once (LDS, registers and
// waves permitting); 1 when the runtime could not say.
int per_cu(const Config* c) {
  int cnt = 0;
  const Config* t = configs(&cnt);
  const long i = c - t;
  return (i >= 0 && i < kMaxConfigs && g_per_cu[i] > 0) ? g_per_cu[i] : 1;
}

// ---- split-K workspace: library-owned device memory per device, grown on
// demand.  Layout: kCounterInts arrival counters (zeroed once, reset by the
// kernels), then the fp32 partial tiles.
constexpr size_t kCounterInts = 1 << 16;
struct Workspace {
  std::mutex mu;
  char* base = nullptr;
  size_t bytes = 0;
};
Workspace g_ws[kMaxDevices];

int ensure_workspace(int dev, size_t partial_bytes, float** partial, int** counters) {
  Workspace& w = g_ws[dev];
  std::lock_guard<std::mutex> lock(w.mu);
  const size_t need = kCounterInts * sizeof(int) + partial_bytes;
  if (w.bytes < need) {
    if (w.base) {
      hipError_t e = hipFree(w.base);  // synchronises the device
      w.base = nullptr;
      w.bytes = 0;
      if (e != hipSuccess) return fail(DG_ERR_HIP, "hipFree(workspace): %s", hipGetErrorString(e));
    }
    size_t alloc = need < ((size_t)16 << 20) ? ((size_t)16 << 20) : need;
    void* ptr = nullptr;
    hipError_t e = hipMalloc(&ptr, alloc);
    if (e != hipSuccess) return fail(DG_ERR_HIP, "hipMalloc(workspace %zu): %s", alloc, hipGetErrorString(e));
    e = hipMemset(ptr, 0, kCounterInts * sizeof(int));
    if (e != hipSuccess) return fail(DG_ERR_HIP, "hipMemset(workspace): %s", hipGetErrorString(e));
    w.base = (char*)ptr;
    w.bytes = alloc;
  }
  *counters = (int*)w.base;
  *partial = (float*)(w.base + kCounterInts * sizeof(int));
  return DG_OK;
}

int launch(const Config& c, dg::GemmParams& p, int grid, hipStream_t stream) {
  if (int s = ensure_kernel_attributes()) return s;
  if (log_enabled())
    fprintf(stderr, "[dg] %s m=%d n=%d k=%d groups=%d grid=%d threads=%d smem=%d per_cu=%d splits=%d\n", c.name,
            p.m, p.n, p.k, p.num_groups, grid, c.threads(), c.smem, per_cu(&c), p.splits);
  if (grid <= 0) return ok();
  void* args[] = {&p};
  hipError_t e;
  if (g_prof_start || g_prof_stop) {
    e = hipExtLaunchKernel(c.fn, dim3(grid), dim3(c.threads()), args, c.smem, stream, g_prof_start,
                           g_prof_stop, 0);
    g_prof_start = g_prof_stop = nullptr;
  } else {
    e = hipLaunchKernel(c.fn, dim3(grid), dim3(c.threads()), args, c.smem, stream);
  }
  if (e != hipSuccess) return fail(DG_ERR_HIP, "launch of %s failed: %s", c.name, hipGetErrorString(e));
  return ok();
}

void fill_common(dg::GemmParams& p, const Config& c, int m, int n, int k) {
  p.m = m;
  p.n = n;
  p.k = k;
  p.kb_count = k / 128;
  p.sk_count = p.kb_count;
  p.nb_count = (n + 127) / 128;
  p.sfa_ld = sfa_ld(m);
  p.tiles_m = (m + c.bm - 1) / c.bm;
  p.tiles_n = (n + c.bn - 1) / c.bn;
  // grouped raster height in tiles: 4 measured 1-2 % ahead of 8 and 16 on the
  // large dense and contiguous shapes (DG_GROUP_M overrides it for sweeps)
  p.group_m = 4;
  if (const char* e = getenv("DG_GROUP_M")) p.group_m = atoi(e) > 0 ? atoi(e) : 4;
}

// The launch grid is 32-bit: the output tiles (times a split count of up to
// 8) must fit it.
int set_num_tiles(dg::GemmParams& p, long long groups) {
  const long long t = groups * p.tiles_m * (long long)p.tiles_n;
  if (t > (1LL << 27)) return fail(DG_ERR_UNSUPPORTED_SHAPE, "too many output tiles (%lld)", t);
  p.num_tiles = (int)t;
  return DG_OK;
}

int check_k_n(int n, int k) {
  if (n < 1) return fail(DG_ERR_INVALID_ARGUMENT, "n must be >= 1 (got %d)", n);
  if (k < 128 || k % 128 != 0)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "k must be a positive multiple of 128 (got %d)", k);
  if ((long long)n * k > 0xFFFFFFFFLL)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "one B operand must stay below 4 GiB (n*k = %lld)", (long long)n * k);
  return DG_OK;
}

// The kernels address one operand matrix (one expert's, for the grouped
// layouts) with 32-bit byte offsets.
int check_rows(long long rows, int k) {
  if (rows * k > 0xFFFFFFFFLL)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "one A operand must stay below 4 GiB (rows*k = %lld)", rows * k);
  return DG_OK;
}

// The 256 x 256 tile (one workgroup per CU) while its tiles alone keep more
// than half the CUs busy, so that it needs no split-K; below that, 128 x 128
// tiles (two per CU, split over K when still too few) finish sooner.  The
// N- and M-shards of the large GEMM over 8 GPUs, 4096 x 896 x 16384 and
// 512 x 7168 x 16384, run in 83-90 us against 107 us for 256 x 256 tiles
// split 4 ways; 2048 x 7168 x 16384 (224 big tiles) keeps 256 x 256 tiles,
// 258 against 288 us.
bool big_tiles_enough(int m, int n, const DeviceInfo* info) {
  return 2 * (long long)((m + 255) / 256) * ((n + 255) / 256) > info->cus;
}

// Split count of a dense launch of num_tiles tiles over kb_count 128-byte K
// slabs (1: no split), and the slabs of each split.
//
// K is split over workgroups when the tiles alone cannot fill the GPU's
// workgroup slots: up to two resident workgroups per CU (one for the
// configurations that fit only one).  Decode-shaped calls are bound by HBM
// latency more than by bandwidth, and two workgroups per CU keep more loads
// in flight than one (64 x 2112 x 7168: 7 splits of 8 slabs of 64 x 32 tiles,
// 462 workgroups); mid-sized shapes with too few tiles gain the same way
// (4096 x 896 x 16384 in 128 x 128 tiles: 2 splits, 83 against 115 us).
// DG_SPLIT_K=<n> pins the count (for sweeps).
int dense_splits(const Config* c, int num_tiles, int kb_count, const DeviceInfo* info, int* split_slabs) {
  int splits = 1;
  const int slots = (per_cu(c) >= 2 ? 2 : 1) * info->cus;
  if (const char* e = getenv("DG_SPLIT_K")) splits = atoi(e);
  else if (c->sched != dg::kPingPong && num_tiles * 2 <= slots && kb_count >= 4) {
    splits = slots / num_tiles;
    // no more splits than it takes to shorten the longest one
    while (splits > 1 && (kb_count + splits - 2) / (splits - 1) == (kb_count + splits - 1) / splits) --splits;
    const int min_split_slabs = 2;
    if (splits > kb_count / min_split_slabs) splits = kb_count / min_split_slabs;
    if (splits > 8) splits = 8;  // partial-tile traffic grows with the count
  }
  *split_slabs = kb_count;
  if (splits <= 1) return 1;
  const int per = (kb_count + splits - 1) / splits;
  *split_slabs = per;
  return (kb_count + per - 1) / per;  // no empty splits
}

// The default configuration of a dense call (the rules and their
// measurements are next to big_tiles_enough and in the config table).
const Config* dense_default_config(int dtype, int m, int n, const DeviceInfo* info) {
  const bool mid = m <= 256 || n <= 256 || !big_tiles_enough(m, n, info);
  // Few 128 x 128 tiles: smaller tiles (four or more workgroups per CU), or
  // a third stage, keep more loads in flight per CU than split-K of the
  // 128 x 128 tile alone does.
  const long long t128 = (long long)((m + 127) / 128) * ((n + 127) / 128);
  const bool few = mid && m <= 256 && t128 <= 64;
  switch (dtype) {
    case dg::kBf16:
      if (m <= 64 || (few && n <= 1024)) return find_config("bf16_64x32_w4_s4", dg::kDense, dg::kBf16);
      if (few && n <= 4096) return find_config("bf16_64x64_w4_s3", dg::kDense, dg::kBf16);
      return find_config(mid ? "bf16_128x128_w4_s2" : "bf16_256x256_w8_s2", dg::kDense, dg::kBf16);
    case dg::kFp4:
      if (m <= 64 || (few && n <= 1024)) return find_config("fp4_64x32_w4_s4", dg::kDense, dg::kFp4);
      if (few || (mid && t128 <= 72 && n >= 1024)) return find_config("fp4_64x64_w4_s3", dg::kDense, dg::kFp4);
      return find_config(mid ? "fp4_128x128_w4_s2" : "fp4_256x256_w8_s2", dg::kDense, dg::kFp4);
    default: {
      if (m <= 64) return find_config(n <= 4096 ? "dense_64x32_w4_s4" : "dense_64x64_w4_s3", dg::kDense);
      if (!mid) return find_config("dense_256x256_w8_s2", dg::kDense);
      if (few) return find_config(n <= 1024 ? "dense_64x32_w4_s4" : "dense_64x64_w4_s3", dg::kDense);
      if (t128 <= 72 && n >= 1024) return find_config("dense_128x128_w4_s3", dg::kDense);
      return find_config("dense_128x128_w4_s2", dg::kDense);
    }
  }
}

// The configuration a dense call uses: DG_FORCE_CONFIG when it names one of
// this dtype's dense configurations, else the default.
int dense_config(int dtype, int m, int n, const DeviceInfo* info, const Config** out) {
  if (int s = forced_config(dg::kDense, out, dtype)) return s;
  if (!*out) *out = dense_default_config(dtype, m, n, info);
  if (!*out) return fail(DG_ERR_INTERNAL, "no dense configuration for dtype %d", dtype);
  return DG_OK;
}

// Dense launch with the split-K choice, shared by the fp8, bf16 and fp4 entry
// points; k_bytes is K in bytes (one per fp8 value, two per bf16 value, half
// per fp4 value) and scale_slabs the number of 128-wide scale slabs of K.
int launch_dense(const Config* c, dg::GemmParams& p, int dev, const DeviceInfo* info, int m, int n, int k_bytes,
                 int scale_slabs, dg_stream_t stream) {
  if (int s = ensure_kernel_attributes()) return s;
  p.num_groups = 1;
  fill_common(p, *c, m, n, k_bytes);
  p.sk_count = scale_slabs;
  if (int s = set_num_tiles(p, 1)) return s;
  p.splits = dense_splits(c, p.num_tiles, p.kb_count, info, &p.split_slabs);
  if (p.splits > 1) {
    if (c->sched == dg::kPingPong)
      return fail(DG_ERR_INVALID_ARGUMENT, "configuration %s does not support split-K", c->name);
    if ((size_t)p.num_tiles > kCounterInts)
      return fail(DG_ERR_UNSUPPORTED_SHAPE, "too many tiles for split-K (%d)", p.num_tiles);
    if ((long long)p.num_tiles * p.splits > 0x7FFFFFFFLL)
      return fail(DG_ERR_UNSUPPORTED_SHAPE, "split-K grid too large (%d x %d)", p.num_tiles, p.splits);
    const size_t part = (size_t)p.num_tiles * p.splits * c->bm * c->bn * sizeof(float);
    if (int s = ensure_workspace(dev, part, &p.ws_partial, &p.ws_count)) return s;
  }
  return launch(*c, p, p.num_tiles * p.splits, (hipStream_t)stream);
}

int quantize_a(const void* kernel, const float* x, uint8_t* q, float* sfa, int m, int k, dg_stream_t stream) {
  if (!x || !q || !sfa) return fail(DG_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (m < 0) return fail(DG_ERR_INVALID_ARGUMENT, "m must be >= 0 (got %d)", m);
  if (k < 128 || k % 128 != 0)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "k must be a positive multiple of 128 (got %d)", k);
  if (!aligned16(x) || !aligned16(q) || !aligned16(sfa))
    return fail(DG_ERR_MISALIGNED, "pointers must be 16-byte aligned");
  if (m == 0) return ok();
  int dev;
  DeviceInfo* info;
  if (int s = current_device(&dev, &info)) return s;
  const int ld = sfa_ld(m);
  const long long units = (long long)ld * ((k / 128 + 1) / 2);
  const long long grid = (units + 3) / 4;
  if (grid > 0x7fffffffLL) return fail(DG_ERR_UNSUPPORTED_SHAPE, "matrix too large");
  void* args[] = {&x, &q, &sfa, &m, &k, (void*)&ld};
  hipError_t e = hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(256), args, 0, (hipStream_t)stream);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "quant_a launch failed: %s", hipGetErrorString(e));
  return ok();
}

int quantize_b(const void* kernel, const float* x, uint8_t* q, float* sfb, int n, int k, dg_stream_t stream) {
  if (!x || !q || !sfb) return fail(DG_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (n < 0) return fail(DG_ERR_INVALID_ARGUMENT, "n must be >= 0 (got %d)", n);
  if (k < 128 || k % 128 != 0)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "k must be a positive multiple of 128 (got %d)", k);
  if (!aligned16(x) || !aligned16(q) || !aligned16(sfb))
    return fail(DG_ERR_MISALIGNED, "pointers must be 16-byte aligned");
  if (n == 0) return ok();
  int dev;
  DeviceInfo* info;
  if (int s = current_device(&dev, &info)) return s;
  const long long grid = (long long)((n + 127) / 128) * (k / 128);
  if (grid > 0x7fffffffLL) return fail(DG_ERR_UNSUPPORTED_SHAPE, "matrix too large");
  void* args[] = {&x, &q, &sfb, &n, &k};
  hipError_t e = hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(256), args, 0, (hipStream_t)stream);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "quant_b launch failed: %s", hipGetErrorString(e));
  return ok();
}


}  // namespace

extern "C" {

int dg_get_m_alignment_for_contiguous_layout(void) { return 128; }

int dg_get_sfa_ld(int m) { return m < 0 ? 0 : sfa_ld(m); }

static_assert((int)DG_DTYPE_FP8 == (int)dg::kFp8 && (int)DG_DTYPE_BF16 == (int)dg::kBf16 &&
                  (int)DG_DTYPE_FP4 == (int)dg::kFp4,
              "dtype codes of the ABI and the kernels agree");

const char* dg_version(void) { return "dg-gfx950 0.1"; }

int dg_reserve_workspace(size_t bytes) {
  int dev;
  DeviceInfo* info;
  if (int s = current_device(&dev, &info)) return s;
  float* part;
  int* cnt;
  if (int s = ensure_workspace(dev, bytes, &part, &cnt)) return s;
  return ok();
}

int dg_dense_workspace_size(int dtype, int m, int n, int k, size_t* bytes) {
  if (!bytes) return fail(DG_ERR_INVALID_ARGUMENT, "null pointer argument");
  *bytes = 0;
  int k_bytes = 0;
  switch (dtype) {
    case DG_DTYPE_FP8:
      if (k < 128 || k % 128 != 0)
        return fail(DG_ERR_UNSUPPORTED_SHAPE, "k must be a positive multiple of 128 (got %d)", k);
      k_bytes = k;
      break;
    case DG_DTYPE_BF16:
      if (k < 64 || k % 64 != 0 || k > (1 << 30))
        return fail(DG_ERR_UNSUPPORTED_SHAPE, "k must be a positive multiple of 64 (got %d)", k);
      k_bytes = 2 * k;
      break;
    case DG_DTYPE_FP4:
      if (k < 256 || k % 256 != 0)
        return fail(DG_ERR_UNSUPPORTED_SHAPE, "k must be a positive multiple of 256 (got %d)", k);
      k_bytes = k / 2;
      break;
    default:
      return fail(DG_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  }
  if (m < 0) return fail(DG_ERR_INVALID_ARGUMENT, "m must be >= 0 (got %d)", m);
  if (n < 1) return fail(DG_ERR_INVALID_ARGUMENT, "n must be >= 1 (got %d)", n);
  if (m == 0) return ok();
  int dev;
  DeviceInfo* info;
  if (int s = current_device(&dev, &info)) return s;
  if (int s = ensure_kernel_attributes()) return s;
  const Config* c;
  if (int s = dense_config(dtype, m, n, info, &c)) return s;
  const long long tiles = (long long)((m + c->bm - 1) / c->bm) * ((n + c->bn - 1) / c->bn);
  if (tiles > (1LL << 27)) return fail(DG_ERR_UNSUPPORTED_SHAPE, "too many output tiles (%lld)", tiles);
  int per = 0;
  const int splits = dense_splits(c, (int)tiles, k_bytes / 128, info, &per);
  if (splits > 1) *bytes = (size_t)tiles * splits * c->bm * c->bn * sizeof(float);
  return ok();
}

int dg_profile_next_launch(void* start_event, void* stop_event) {
  g_prof_start = (hipEvent_t)start_event;
  g_prof_stop = (hipEvent_t)stop_event;
  return ok();
}

const char* dg_status_string(int status) {
  switch (status) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DG_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case DG_ERR_MISALIGNED: return "misaligned pointer";
    case DG_ERR_NO_DEVICE: return "no usable gfx950 device";
    case DG_ERR_HIP: return "HIP runtime error";
    case DG_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

const char* dg_last_error_message(void) { return g_last_error.c_str(); }

int dg_fp8_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb, uint16_t* d,
                   int m, int n, int k, dg_stream_t stream) {
  if (!a || !sfa || !b || !sfb || !d) return fail(DG_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (m < 0) return fail(DG_ERR_INVALID_ARGUMENT, "m must be >= 0 (got %d)", m);
  if (int s = check_k_n(n, k)) return s;
  if (int s = check_rows(m, k)) return s;
  if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d))
    return fail(DG_ERR_MISALIGNED, "pointers must be 16-byte aligned");
  if (m == 0) return ok();
  int dev;
  DeviceInfo* info;
  if (int s = current_device(&dev, &info)) return s;
  const Config* c;
  if (int s = dense_config(dg::kFp8, m, n, info, &c)) return s;
  dg::GemmParams p{};
  p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.d = d;
  return launch_dense(c, p, dev, info, m, n, k, k / 128, stream);
}

int dg_bf16_gemm_nt(const uint16_t* a, const uint16_t* b, uint16_t* d, int m, int n, int k, dg_stream_t stream) {
  if (!a || !b || !d) return fail(DG_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (m < 0) return fail(DG_ERR_INVALID_ARGUMENT, "m must be >= 0 (got %d)", m);
  if (n < 1) return fail(DG_ERR_INVALID_ARGUMENT, "n must be >= 1 (got %d)", n);
  if (k < 64 || k % 64 != 0 || k > (1 << 30))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "k must be a positive multiple of 64 (got %d)", k);
  if (int s = check_k_n(n, 2 * k)) return s;
  if (int s = check_rows(m, 2 * k)) return s;
  if (!aligned16(a) || !aligned16(b) || !aligned16(d)) return fail(DG_ERR_MISALIGNED, "pointers must be 16-byte aligned");
  if (m == 0) return ok();
  int dev;
  DeviceInfo* info;
  if (int s = current_device(&dev, &info)) return s;
  const Config* c;
  if (int s = dense_config(dg::kBf16, m, n, info, &c)) return s;
  dg::GemmParams p{};
  p.a = reinterpret_cast<const uint8_t*>(a);
  p.b = reinterpret_cast<const uint8_t*>(b);
  p.d = d;
  return launch_dense(c, p, dev, info, m, n, 2 * k, 0, stream);
}

int dg_fp4_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb, uint16_t* d, int m,
                   int n, int k, dg_stream_t stream) {
  if (!a || !sfa || !b || !sfb || !d) return fail(DG_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (m < 0) return fail(DG_ERR_INVALID_ARGUMENT, "m must be >= 0 (got %d)", m);
  if (n < 1) return fail(DG_ERR_INVALID_ARGUMENT, "n must be >= 1 (got %d)", n);
  if (k < 256 || k % 256 != 0)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "k must be a positive multiple of 256 (got %d)", k);
  if (int s = check_k_n(n, k / 2)) return s;
  if (int s = check_rows(m, k / 2)) return s;
  if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d))
    return fail(DG_ERR_MISALIGNED, "pointers must be 16-byte aligned");
  if (m == 0) return ok();
  int dev;
  DeviceInfo* info;
  if (int s = current_device(&dev, &info)) return s;
  const Config* c;
  if (int s = dense_config(dg::kFp4, m, n, info, &c)) return s;
  dg::GemmParams p{};
  p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.d = d;
  return launch_dense(c, p, dev, info, m, n, k / 2, k / 128, stream);
}

int dg_m_grouped_fp8_gemm_nt_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                                        const float* sfb, uint16_t* d, const int32_t* m_indices, int m,
                                        int n, int k, int num_groups, dg_stream_t stream) {
  if (!a || !sfa || !b || !sfb || !d || !m_indices)
    return fail(DG_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (m < 0) return fail(DG_ERR_INVALID_ARGUMENT, "m must be >= 0 (got %d)", m);
  if (num_groups < 1) return fail(DG_ERR_INVALID_ARGUMENT, "num_groups must be >= 1 (got %d)", num_groups);
  if (int s = check_k_n(n, k)) return s;
  if (m % 128 != 0)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "m must be a multiple of the 128-row alignment (got %d)", m);
  if (int s = check_rows(m, k)) return s;
  if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d) ||
      (reinterpret_cast<uintptr_t>(m_indices) & 3u))
    return fail(DG_ERR_MISALIGNED, "pointers must be 16-byte aligned (m_indices 4-byte)");
  if (m == 0) return ok();
  int dev;
  DeviceInfo* info;
  if (int s = current_device(&dev, &info)) return s;
  const Config* c;
  if (int s = forced_config(dg::kContiguous, &c)) return s;
  if (!c) {
    // 128 x 256 tiles with one B buffer (two workgroups per CU) once there
    // are enough of them to fill the GPU; 128 x 128 tiles below that, and
    // 64 x 64 tiles (more workgroups per CU) while 128 x 128 tiles would be
    // at most 128: 4 x 128 rows, N 4096, K 7168 in 49.8 against 63.7 us,
    // N 2112 in 42.9 against 59.9 us; at 256 such tiles they lose (101
    // against 72 us).
    const long long tiles = (long long)(m / 128) * ((n + 255) / 256);
    const long long t128 = (long long)(m / 128) * ((n + 127) / 128);
    c = find_config(t128 <= 128        ? "contig_64x64_w4_s3"
                    : tiles >= info->cus ? "contig_128x256_w4_s2_sb"
                                         : "contig_128x128_w4_s2",
                    dg::kContiguous);
  }
  dg::GemmParams p{};
  p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.d = d; p.m_indices = m_indices;
  p.num_groups = num_groups;
  fill_common(p, *c, m, n, k);
  if (int s = set_num_tiles(p, 1)) return s;
  return launch(*c, p, p.num_tiles, (hipStream_t)stream);
}

// Masked-layout tiles (16 experts, max_m 256, N 4096, K 7168, counts uniform
// on 0..c, one process, same inputs; the 256-column tiles of the SwiGLU
// epilogue move the same way):
//  * while every expert fits one 128-row tile, 128 x 256 tiles with three
//    LDS stages stream B fastest: 77-85 us for c = 16-64 (6.1-5.6 TB/s) and
//    108 us for c = 128, against 90-113 us for the 256 x 256 interleaved
//    schedule and 118-124 us for the ping-pong one.  An expert past 128 rows
//    needs a second row of tiles that waits for a free CU (one workgroup per
//    CU): 166-202 us for c = 160-256.
//  * the 256 x 256 interleaved schedule leads up to c = 160 (123 against
//    128 us), the ping-pong one from c = 192 (131-139 against 140-164 us).
// So: max_m <= 128 (no expert can pass 128 rows) or a typical count
// (expected_m) up to 48 picks the 128-row tile when there are enough of its
// tiles to cover half the CUs; a typical count up to 80 the interleaved
// 256 x 256 schedule; larger or unknown (0) counts the ping-pong one.
enum class MaskedTile { kRows128, kInterleaved, kPingPong };
MaskedTile masked_tile(int num_groups, int max_m, int n, int expected_m, const DeviceInfo* info) {
  const bool enough = 2LL * num_groups * ((n + 255) / 256) >= info->cus;
  if (enough && (max_m <= 128 || (expected_m > 0 && expected_m <= 48))) return MaskedTile::kRows128;
  if (expected_m > 0 && expected_m <= 80) return MaskedTile::kInterleaved;
  return MaskedTile::kPingPong;
}

int dg_m_grouped_fp8_gemm_nt_masked(const uint8_t* a, const float* sfa, const uint8_t* b,
                                    const float* sfb, uint16_t* d, const int32_t* masked_m,
                                    int num_groups, int max_m, int n, int k, int expected_m,
                                    dg_stream_t stream) {
  if (!a || !sfa || !b || !sfb || !d || !masked_m)
    return fail(DG_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (num_groups < 0) return fail(DG_ERR_INVALID_ARGUMENT, "num_groups must be >= 0 (got %d)", num_groups);
  if (max_m < 0) return fail(DG_ERR_INVALID_ARGUMENT, "max_m must be >= 0 (got %d)", max_m);
  if (expected_m < 0) return fail(DG_ERR_INVALID_ARGUMENT, "expected_m must be >= 0 (got %d)", expected_m);
  if (int s = check_k_n(n, k)) return s;
  if (int s = check_rows(max_m, k)) return s;
  if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d) ||
      (reinterpret_cast<uintptr_t>(masked_m) & 3u))
    return fail(DG_ERR_MISALIGNED, "pointers must be 16-byte aligned (masked_m 4-byte)");
  if (num_groups == 0 || max_m == 0) return ok();
  int dev;
  DeviceInfo* info;
  if (int s = current_device(&dev, &info)) return s;
  const Config* c;
  if (int s = forced_config(dg::kMasked, &c)) return s;
  if (!c) {
    const MaskedTile t = masked_tile(num_groups, max_m, n, expected_m, info);
    c = find_config(t == MaskedTile::kRows128 ? "masked_128x256_w8_s3"
                    : max_m <= 64             ? "masked_64x64_w4_s3"
                    : t == MaskedTile::kInterleaved ? "masked_256x256_w8_s2"
                                                    : "masked_256x256_w8_s2_pp",
                    dg::kMasked);
  }
  dg::GemmParams p{};
  p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.d = d; p.masked_m = masked_m;
  p.num_groups = num_groups;
  fill_common(p, *c, max_m, n, k);
  if (int s = set_num_tiles(p, num_groups)) return s;
  return launch(*c, p, p.num_tiles, (hipStream_t)stream);
}

int dg_k_grouped_fp8_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb, uint16_t* d,
                             const int32_t* k_sizes, int num_groups, int m, int n, int k, dg_stream_t stream) {
  if (!a || !sfa || !b || !sfb || !d || !k_sizes) return fail(DG_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (m < 0) return fail(DG_ERR_INVALID_ARGUMENT, "m must be >= 0 (got %d)", m);
  if (num_groups < 0) return fail(DG_ERR_INVALID_ARGUMENT, "num_groups must be >= 0 (got %d)", num_groups);
  if (int s = check_k_n(n, k)) return s;
  if (int s = check_rows(m, k)) return s;
  if ((long long)num_groups * m * n > 0x7FFFFFFFFFFFLL)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "output too large");
  if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d) ||
      (reinterpret_cast<uintptr_t>(k_sizes) & 3u))
    return fail(DG_ERR_MISALIGNED, "pointers must be 16-byte aligned (k_sizes 4-byte)");
  if (m == 0 || num_groups == 0) return ok();
  int dev;
  DeviceInfo* info;
  if (int s = current_device(&dev, &info)) return s;
  const Config* c;
  if (int s = forced_config(dg::kKGrouped, &c)) return s;
  if (!c) c = find_config(m <= 256 || n <= 256 ? "kgrouped_128x128_w4_s2" : "kgrouped_256x256_w8_s2", dg::kKGrouped);
  dg::GemmParams p{};
  p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.d = d; p.k_sizes = k_sizes;
  p.num_groups = num_groups;
  fill_common(p, *c, m, n, k);
  if (int s = set_num_tiles(p, num_groups)) return s;
  p.splits = 1;
  p.split_slabs = p.kb_count;
  return launch(*c, p, p.num_tiles, (hipStream_t)stream);
}

int dg_m_grouped_fp8_gemm_nt_masked_swiglu(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                                           uint8_t* hq, float* hs, const int32_t* masked_m, int num_groups,
                                           int max_m, int inter, int k, int expected_m, dg_stream_t stream) {
  if (!a || !sfa || !b || !sfb || !hq || !hs || !masked_m)
    return fail(DG_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (num_groups < 0) return fail(DG_ERR_INVALID_ARGUMENT, "num_groups must be >= 0 (got %d)", num_groups);
  if (max_m < 0) return fail(DG_ERR_INVALID_ARGUMENT, "max_m must be >= 0 (got %d)", max_m);
  if (expected_m < 0) return fail(DG_ERR_INVALID_ARGUMENT, "expected_m must be >= 0 (got %d)", expected_m);
  if (inter < 128 || inter % 128 != 0 || inter > (1 << 29))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "inter must be a positive multiple of 128 (got %d)", inter);
  if (int s = check_k_n(2 * inter, k)) return s;
  if (int s = check_rows(max_m, k)) return s;
  if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(hq) || !aligned16(hs) ||
      (reinterpret_cast<uintptr_t>(masked_m) & 3u))
    return fail(DG_ERR_MISALIGNED, "pointers must be 16-byte aligned (masked_m 4-byte)");
  if (num_groups == 0 || max_m == 0) return ok();
  int dev;
  DeviceInfo* info;
  if (int s = current_device(&dev, &info)) return s;
  const Config* c;
  if (int s = forced_config(dg::kMasked, &c, dg::kFp8, dg::kEpiSwigluFp8)) return s;
  if (!c) {
    const MaskedTile t = masked_tile(num_groups, max_m, 2 * inter, expected_m, info);
    c = find_config(t == MaskedTile::kRows128 ? "swiglu_128x256_w8_s3"
                    : max_m <= 64             ? "swiglu_64x256_w4_s3"
                    : t == MaskedTile::kInterleaved ? "swiglu_256x256_w8_s2"
                                                    : "swiglu_256x256_w8_s2_pp",
                    dg::kMasked, dg::kFp8, dg::kEpiSwigluFp8);
  }
  dg::GemmParams p{};
  p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.masked_m = masked_m;
  p.hq = hq; p.hs = hs; p.inter = inter;
  p.num_groups = num_groups;
  fill_common(p, *c, max_m, 2 * inter, k);
  p.tiles_n = inter / 128;  // one tile per 128 h columns (128 gate + 128 up rows of B)
  if (int s = set_num_tiles(p, num_groups)) return s;
  return launch(*c, p, p.num_tiles, (hipStream_t)stream);
}

int dg_quantize_a_1x128(const float* x, uint8_t* q, float* sfa, int m, int k, dg_stream_t stream) {
  return quantize_a(reinterpret_cast<const void*>(&dg::quant_a_kernel), x, q, sfa, m, k, stream);
}

int dg_quantize_b_128x128(const float* x, uint8_t* q, float* sfb, int n, int k, dg_stream_t stream) {
  return quantize_b(reinterpret_cast<const void*>(&dg::quant_b_kernel), x, q, sfb, n, k, stream);
}

int dg_quantize_a_1x128_fp4(const float* x, uint8_t* q, float* sfa, int m, int k, dg_stream_t stream) {
  return quantize_a(reinterpret_cast<const void*>(&dg::quant_a_fp4_kernel), x, q, sfa, m, k, stream);
}

int dg_quantize_b_128x128_fp4(const float* x, uint8_t* q, float* sfb, int n, int k, dg_stream_t stream) {
  return quantize_b(reinterpret_cast<const void*>(&dg::quant_b_fp4_kernel), x, q, sfb, n, k, stream);
}

}  // extern "C"
