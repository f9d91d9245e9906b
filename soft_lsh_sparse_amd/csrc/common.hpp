// Device helpers shared by the SOCKET kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace socket_lsh {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bfloat16

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Element access for the two supported storage types.
struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
  __device__ __forceinline__ static float load(const float* p, int64_t i) {
    return p[i];
  }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) {
    p[i] = v;
  }
};

struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
  __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
  }
  __device__ __forceinline__ static void store(uint16_t* p, int64_t i,
                                               float v) {
    p[i] = f32_to_bf16_rne(v);
  }
};

// Unpack 16 bytes holding 8 bf16 (or 4 f32) values to float.
__device__ __forceinline__ void unpack8_bf16(const uint4& w, float* f) {
  f[0] = __uint_as_float(w.x << 16);
  f[1] = __uint_as_float(w.x & 0xffff0000u);
  f[2] = __uint_as_float(w.y << 16);
  f[3] = __uint_as_float(w.y & 0xffff0000u);
  f[4] = __uint_as_float(w.z << 16);
  f[5] = __uint_as_float(w.z & 0xffff0000u);
  f[6] = __uint_as_float(w.w << 16);
  f[7] = __uint_as_float(w.w & 0xffff0000u);
}

__device__ __forceinline__ void unpack4_f32(const uint4& w, float* f) {
  f[0] = __uint_as_float(w.x);
  f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z);
  f[3] = __uint_as_float(w.w);
}

// ------------------------------------------------------- wave reductions

template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = WIDTH / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = WIDTH / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// ---------------------------------------- double-double (error-free) sums

// Knuth's TwoSum: s + e == a + b exactly (round-to-nearest, no reassociation).
__device__ __forceinline__ void two_sum(double a, double b, double& s,
                                        double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// (ah, al) + (bh, bl) in double-double arithmetic, renormalised.
__device__ __forceinline__ void dd_add(double ah, double al, double bh,
                                       double bl, double& h, double& l) {
  double s, e;
  two_sum(ah, bh, s, e);
  e += al + bl;
  h = s + e;
  l = e - (h - s);
}

// Sum over the wave of one double-double (h, l) per lane. Returns the high
// part of the renormalised result; its sign is the sign of the sum.
__device__ __forceinline__ double wave_sum_dd(double h, double l) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) {
    double oh = __shfl_xor(h, m, kWave);
    double ol = __shfl_xor(l, m, kWave);
    dd_add(h, l, oh, ol, h, l);
  }
  return h;
}

// Order-preserving map of float bits to uint32 (ascending float order ->
// ascending unsigned order; -0.0 is mapped like +0.0).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace socket_lsh
