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

// DPP lane permutations: operand modifiers of a VALU move, no LDS round
// trip (unlike ds_bpermute-based shuffles).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Sum over each aligned group of 16 lanes, returned in every lane of the
// group: lane pairs (i, i^1), (i, i^2) within quads, then the two quads of
// each half-row (mirror) and the two half-rows (mirror). Each step adds the
// same two values in every lane of a pair, so all 16 results are identical.
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ double sum16_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return v;
}

// Inclusive prefix sum over the wave (lane i gets x_0 + ... + x_i): shifts
// by 1, 2, 4 and 8 within each row of 16 lanes, then the row totals are
// carried across rows with two broadcasts. Lanes a shift leaves without a
// source add 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan_dpp(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// The value of lane i ^ 16 (v_permlane16_swap: rows of 16 lanes trade in
// pairs).
__device__ __forceinline__ uint32_t xor16_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (threadIdx.x & 16) ? r[0] : r[1];
}

// The value of lane i ^ 32 (v_permlane32_swap: the two half-waves trade).
__device__ __forceinline__ uint32_t xor32_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}

// The value of lane i ^ O for O in {8, 16, 32}: permlane swaps for 16 and
// 32 (VALU), a shuffle otherwise.
template <int O>
__device__ __forceinline__ float xor_lanes(float v) {
  if constexpr (O == 16) return __uint_as_float(xor16_u32(__float_as_uint(v)));
  else if constexpr (O == 32) return __uint_as_float(xor32_u32(__float_as_uint(v)));
  else return __shfl_xor(v, O, kWave);
}

// Sum over each aligned group of W lanes (W in {8, 16, 32, 64}), in every
// lane of the group, by DPP and permlane swaps.
template <int W>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (W == 8) {
    v += dpp_f32<0xB1>(v);
    v += dpp_f32<0x4E>(v);
    v += dpp_f32<0x141>(v);
    return v;
  } else {
    v = sum16(v);
    if constexpr (W >= 32) v += xor_lanes<16>(v);
    if constexpr (W >= 64) v += xor_lanes<32>(v);
    return v;
  }
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
