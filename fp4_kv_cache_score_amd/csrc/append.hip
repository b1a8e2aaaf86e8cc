// Write side of the pool and the window: new compressed entries are encoded
// into the stored formats, and new tokens into the FP8 window ring.
//
// A Full layer generates the KV and index data that later layers reuse; the
// global entries are kept in FP4 (E2M1) and the window in FP8, restored at
// run time ("DeepSeek V4.1-Flash Cuts KV Cache by 437x", paragraphs on the
// three operating modes, FP4 quantisation and sliding window attention).  The
// pages give no encoding rule; the one used here:
//   * latent rows: per block of 32 consecutive elements an E8M0 scale
//     2^shared with shared = floor(log2(amax)) - 2 (clamped to [-127, 127],
//     0 for an all-zero block), elements divided by it and rounded to the
//     nearest E2M1 value with ties to the even code, saturating at 6, signs
//     kept (also for values that round to zero); element 2i in the low
//     nibble of byte i;
//   * index keys and window rows: E4M3 after clamping to +-448, nearest value
//     with ties to the even code (no NaN code is produced).
// Every rounding decision is taken on an exactly scaled float32 value.
//
// k_pool_append: one wave per new entry; lane l encodes latent elements
// 8l..8l+7 (four lanes share a 32-element block: the block's amax is a 4-lane
// max) and key elements 8l..8l+7, and stores its 4 + 8 bytes coalesced.
// k_window_append: one wave per new token row, ring row (pos0 + t) mod W.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kRowLanes = 64;

// floor(log2(a)) of a finite positive float, subnormals included.
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t u = __float_as_uint(a);
  const int e = (int)((u >> 23) & 0xFFu);
  if (e) return e - 127;
  return (31 - __builtin_clz(u & 0x7FFFFFu)) - 149;   // subnormal: mantissa * 2^-149
}

// E2M1 code (sign in bit 3) of y = x / 2^shared.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float m = fabsf(y);
  uint32_t c;
  if (m < 2.f) {
    c = (uint32_t)rintf(m * 2.f);                    // 0, 0.5, 1, 1.5, 2 -> codes 0..4
  } else if (m < 4.f) {
    c = 4u + (uint32_t)(rintf(m) - 2.f);             // 2, 3, 4 -> codes 4..6
  } else {
    const float q = fminf(2.f * rintf(m * 0.5f), 6.f);   // 4, 6 (8 saturates to 6)
    c = 6u + (uint32_t)((q - 4.f) * 0.5f);           // codes 6, 7
  }
  return c | (signbit(y) ? 8u : 0u);
}

// E4M3 byte of x: clamp to +-448, nearest value, ties to the even code.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const float c = fminf(fmaxf(x, -448.f), 448.f);
  const float m = fabsf(c);
  uint32_t code;
  if (m < 0.015625f) {                               // below 2^-6: multiples of 2^-9
    code = (uint32_t)rintf(m * 512.f);               // 8 -> the first normal, code 8
  } else {
    int e = floor_log2(m);                           // -6 .. 8
    float q = rintf(ldexpf(m, 3 - e));               // 8 .. 16
    if (q == 16.f) {
      q = 8.f;
      ++e;
    }
    code = ((uint32_t)(e + 7) << 3) | (uint32_t)(q - 8.f);
  }
  return code | (signbit(c) ? 0x80u : 0u);
}

__global__ __launch_bounds__(256)
void k_pool_append(uint8_t* __restrict__ latent, uint8_t* __restrict__ scale,
                   uint8_t* __restrict__ idx_key, int32_t M, const float* __restrict__ x_lat,
                   const float* __restrict__ x_key, const int32_t* __restrict__ slot, int32_t T,
                   int64_t rows, PoolMap map) {
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / kRowLanes) + (threadIdx.x / kRowLanes);
  if (r >= rows) return;
  const int lane = threadIdx.x & (kRowLanes - 1);
  const int64_t b = r / T;
  const int32_t e = slot[r];
  if (e < 0 || e >= M) return;                       // wave-uniform
  const size_t er = (size_t)pool_row(map, b, e, M);   // the entry's pool row

  {  // latent: 8 elements per lane, a block of 32 per 4 lanes
    const float4* src = reinterpret_cast<const float4*>(x_lat + (size_t)r * kD + 8 * lane);
    const float4 a = src[0], c = src[1];
    const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    int shared = 0;
    if (amax > 0.f) {
      shared = floor_log2(amax) - 2;
      shared = shared < -127 ? -127 : (shared > 127 ? 127 : shared);
    }
    uint32_t packed = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= e2m1_code(ldexpf(v[i], -shared)) << (4 * i);
    reinterpret_cast<uint32_t*>(latent + er * kLatRow)[lane] = packed;
    if ((lane & 3) == 0) scale[er * kScaleRow + (lane >> 2)] = (uint8_t)(shared + 127);
  }
  {  // index key: 8 elements per lane
    const float4* src = reinterpret_cast<const float4*>(x_key + (size_t)r * kKeyRow + 8 * lane);
    const float4 a = src[0], c = src[1];
    const uint32_t lo = e4m3_code(a.x) | (e4m3_code(a.y) << 8) | (e4m3_code(a.z) << 16) | (e4m3_code(a.w) << 24);
    const uint32_t hi = e4m3_code(c.x) | (e4m3_code(c.y) << 8) | (e4m3_code(c.z) << 16) | (e4m3_code(c.w) << 24);
    reinterpret_cast<uint2*>(idx_key + er * kKeyRow)[lane] = make_uint2(lo, hi);
  }
}

__global__ __launch_bounds__(256)
void k_window_append(uint8_t* __restrict__ swa, int32_t W, const float* __restrict__ x,
                     int64_t pos0, int32_t T, int32_t t0, int64_t rows) {
  // rows = B * (T - t0): the new tokens t0 .. T-1 of each sequence (the last W)
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / kRowLanes) + (threadIdx.x / kRowLanes);
  if (r >= rows) return;
  const int lane = threadIdx.x & (kRowLanes - 1);
  const int32_t n = T - t0;
  const int64_t b = r / n;
  const int32_t t = t0 + (int32_t)(r - b * n);
  const int64_t ring = (pos0 + t) % W;
  const float4* src = reinterpret_cast<const float4*>(x + ((size_t)b * T + t) * kD + 8 * lane);
  const float4 a = src[0], c = src[1];
  const uint32_t lo = e4m3_code(a.x) | (e4m3_code(a.y) << 8) | (e4m3_code(a.z) << 16) | (e4m3_code(a.w) << 24);
  const uint32_t hi = e4m3_code(c.x) | (e4m3_code(c.y) << 8) | (e4m3_code(c.z) << 16) | (e4m3_code(c.w) << 24);
  reinterpret_cast<uint2*>(swa + ((size_t)b * W + ring) * kD)[lane] = make_uint2(lo, hi);
}

}  // namespace

hipError_t launch_pool_append(uint8_t* latent, uint8_t* scale, uint8_t* idx_key, int32_t B,
                              int32_t M, const float* x_lat, const float* x_key, const int32_t* slot,
                              int32_t T, const PoolMap& map, hipStream_t s) {
  const int64_t rows = (int64_t)B * T;
  if (rows <= 0) return hipSuccess;
  const int64_t per = 256 / kRowLanes;
  k_pool_append<<<dim3((unsigned)((rows + per - 1) / per)), dim3(256), 0, s>>>(
      latent, scale, idx_key, M, x_lat, x_key, slot, T, rows, map);
  return hipGetLastError();
}

hipError_t launch_window_append(uint8_t* swa, int32_t B, int32_t W, const float* x, int64_t pos0,
                                int32_t T, hipStream_t s) {
  const int32_t t0 = T > W ? T - W : 0;
  const int64_t rows = (int64_t)B * (T - t0);
  if (rows <= 0) return hipSuccess;
  const int64_t per = 256 / kRowLanes;
  k_window_append<<<dim3((unsigned)((rows + per - 1) / per)), dim3(256), 0, s>>>(
      swa, W, x, pos0, T, t0, rows);
  return hipGetLastError();
}

}  // namespace csa2
