// Block quantisers for the FP8 block-scaled GEMM: fp32 -> e4m3 codes plus
// fp32 scales, 1x128 per row slab for activations (A) and 128x128 per block
// for weights (B); the same blocks with e2m1 codes (range 6) for FP4.  The pages call the scaling "fine-grained" and "block-wise,
// each small block scaled on its own" ("DeepSeek open-source week day 3",
// technical features; "DeepGEMM: making LLM matrix multiplication fly",
// core functions).  Per block: amax = max |x| (floored at 1e-4),
// s = amax / 448 (fp32, correctly rounded), code = e4m3(x / s) rounded to
// nearest even, saturated at +-448.
//
// Both kernels are HBM-bound streaming passes: every fp32 input byte is read
// once, coalesced as 16-byte loads; codes leave as 4-byte (A) or 4-byte (B)
// packed stores.  The e4m3 rounding is the hardware's v_cvt_pk_fp8_f32
// (OCP e4m3 on gfx950, nearest even); inputs are clamped to +-448 first so
// the conversion never sees an out-of-range value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

constexpr float kE4m3Max = 448.0f;
constexpr float kAmaxFloor = 1e-4f;

__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kE4m3Max), kE4m3Max);
  b = fminf(fmaxf(b, -kE4m3Max), kE4m3Max);
  c = fminf(fmaxf(c, -kE4m3Max), kE4m3Max);
  d = fminf(fmaxf(d, -kE4m3Max), kE4m3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);  // bytes 0,1
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);       // bytes 2,3
  return (uint32_t)w;
}

// One e4m3 code (the low byte of a packed conversion), saturated at +-448.
__device__ __forceinline__ uint8_t e4m3_code(float x) {
  x = fminf(fmaxf(x, -kE4m3Max), kE4m3Max);
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xFF);
}

// FP4 (e2m1) codes, the pages' other low-precision GEMM format: magnitudes
// 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7), sign in bit 3.  Rounding to
// nearest with ties to the even code is a count of the thresholds passed (a
// tie stays on the even side: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0,
// 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4); anything above 5 saturates at 6.
constexpr float kE2m1Max = 6.0f;

__device__ __forceinline__ uint32_t e2m1_code(float x) {
  const float a = fabsf(x);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.f);
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// Four e2m1 codes in two bytes, element 0 in the low nibble.
__device__ __forceinline__ uint32_t pack4_e2m1(float a, float b, float c, float d) {
  return e2m1_code(a) | (e2m1_code(b) << 4) | (e2m1_code(c) << 8) | (e2m1_code(d) << 12);
}

enum QuantFormat { kQE4m3 = 0, kQE2m1 = 1 };

// A quantiser: one wave covers two slabs of one row; lane l holds 4
// consecutive floats of slab (l / 32).  Rows in [m, ld) get a zero scale.
// e4m3 codes take a byte per element, e2m1 codes half a byte.
template <int FMT>
__device__ __forceinline__ void quant_a_body(const float* __restrict__ x, uint8_t* __restrict__ q,
                                             float* __restrict__ sfa, int m, int k, int ld) {
  const int lane = threadIdx.x & 63;
  const int kb_count = k / 128;
  const int pairs = (kb_count + 1) / 2;
  const long long unit = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, slab pair)
  const long long total = (long long)ld * pairs;
  if (unit >= total) return;
  const int row = (int)(unit / pairs);
  const int kb = (int)(unit % pairs) * 2 + (lane >> 5);
  const bool live = kb < kb_count;
  if (row >= m) {  // padding rows of the slab-major scale layout
    if (live && (lane & 31) == 0) sfa[(size_t)kb * ld + row] = 0.f;
    return;
  }
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  const size_t off = (size_t)row * k + (size_t)kb * 128 + (lane & 31) * 4;
  if (live) v = *(const float4*)(x + off);
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
  for (int s = 16; s >= 1; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
  amax = fmaxf(amax, kAmaxFloor);
  const float sc = amax / (FMT == kQE4m3 ? kE4m3Max : kE2m1Max);
  if (!live) return;
  if (FMT == kQE4m3)
    *(uint32_t*)(q + off) = pack4_e4m3(v.x / sc, v.y / sc, v.z / sc, v.w / sc);
  else
    *(uint16_t*)(q + off / 2) = (uint16_t)pack4_e2m1(v.x / sc, v.y / sc, v.z / sc, v.w / sc);
  if ((lane & 31) == 0) sfa[(size_t)kb * ld + row] = sc;
}

__global__ __launch_bounds__(256) void quant_a_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                      float* __restrict__ sfa, int m, int k, int ld) {
  quant_a_body<kQE4m3>(x, q, sfa, m, k, ld);
}

__global__ __launch_bounds__(256) void quant_a_fp4_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                          float* __restrict__ sfa, int m, int k, int ld) {
  quant_a_body<kQE2m1>(x, q, sfa, m, k, ld);
}

// B quantiser: one 256-thread workgroup per 128x128 block (the last row block
// may be partial).  Thread t covers column quad (t % 32) of rows t / 32 + 8 i.
template <int FMT>
__device__ __forceinline__ void quant_b_body(const float* __restrict__ x, uint8_t* __restrict__ q,
                                             float* __restrict__ sfb, int n, int k) {
  __shared__ float s_max[4];
  const int kb_count = k / 128;
  const int nb = blockIdx.x / kb_count;
  const int kb = blockIdx.x % kb_count;
  const int t = threadIdx.x;
  const int col = kb * 128 + (t & 31) * 4;
  const int r0 = nb * 128;
  float4 v[16];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = r0 + (t >> 5) + 8 * i;
    v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < n) v[i] = *(const float4*)(x + (size_t)row * k + col);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
  if ((t & 63) == 0) s_max[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  amax = fmaxf(amax, kAmaxFloor);
  const float sc = amax / (FMT == kQE4m3 ? kE4m3Max : kE2m1Max);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = r0 + (t >> 5) + 8 * i;
    if (row >= n) continue;
    const size_t off = (size_t)row * k + col;
    if (FMT == kQE4m3)
      *(uint32_t*)(q + off) = pack4_e4m3(v[i].x / sc, v[i].y / sc, v[i].z / sc, v[i].w / sc);
    else
      *(uint16_t*)(q + off / 2) = (uint16_t)pack4_e2m1(v[i].x / sc, v[i].y / sc, v[i].z / sc, v[i].w / sc);
  }
  if (t == 0) sfb[(size_t)nb * kb_count + kb] = sc;
}

__global__ __launch_bounds__(256) void quant_b_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                      float* __restrict__ sfb, int n, int k) {
  quant_b_body<kQE4m3>(x, q, sfb, n, k);
}

__global__ __launch_bounds__(256) void quant_b_fp4_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                          float* __restrict__ sfb, int n, int k) {
  quant_b_body<kQE2m1>(x, q, sfb, n, k);
}

}  // namespace dg
