// Soft bucket probabilities: projections, per-bit weights and bucket
// products of the table kernel.
//
// Soft assignment of SOCKET (page "Resumen Técnico: SOCKET - Estimador de
// Núcleo de Colisión Suave para Atención Escasa", section "Mecanismo Central:
// LSH Suave", item 2): the query's hyperplane projections pass through a
// temperature softmax over every bucket of a table. With the logit form
// logit(u) = (1/tau) * sum_j s_j(u) z_j (s_j = +1 when bit j of u is set,
// else -1) the softmax over the 2^P buckets factorises exactly into
//     p(u) = prod_j sigma(2 s_j(u) z_j / tau),
// since its normaliser sum_u exp(logit(u) - max) = prod_j (1 + exp(-2|z_j|/tau)).
#pragma once

#include "common.hpp"

namespace socket_lsh {

constexpr int kMaxBits = 8;

template <typename T>
__device__ __forceinline__ void load8(const typename T::storage* p, bool vec, int valid,
                                      float (&v)[8]);

template <>
__device__ __forceinline__ void load8<BF16>(const uint16_t* p, bool vec, int valid,
                                            float (&v)[8]) {
  if (vec) {
    unpack8_bf16(*reinterpret_cast<const uint4*>(p), v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < valid ? bf16_bits_to_f32(p[e]) : 0.f;
  }
}

template <>
__device__ __forceinline__ void load8<F32>(const float* p, bool vec, int valid,
                                           float (&v)[8]) {
  if (vec) {
    unpack4_f32(*reinterpret_cast<const uint4*>(p), v);
    unpack4_f32(*reinterpret_cast<const uint4*>(p + 4), v + 4);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < valid ? p[e] : 0.f;
  }
}

// Projections z[j][c] = q_j . R[:, c0 + c] for the G queries of a GQA group
// (rows q0 + j*d of Q) and the nc hyperplane columns starting at c0, written
// to out[j * nc + c] (float64). Block-cooperative: each lane accumulates 8
// consecutive columns over one sixteenth of the d coordinates (ascending,
// with fma, from 0); the sixteen parts of a column group sit in sixteen
// adjacent lanes and are combined by a butterfly of additions (the same
// pairing on every lane). bf16 and f32 products are exact in float64.
// blockDim.x must be a multiple of 64.
template <typename T>
__device__ void block_projections(const typename T::storage* Q, int64_t q0,
                                  const typename T::storage* R, int C, int c0,
                                  int nc, int d, int G, double* out) {
  constexpr int kParts = 16;
  constexpr int kMaxSlice = 8;  // d <= 128
  const int ncg = (nc + 7) / 8;
  const int items = G * ncg * kParts;
  const int dp = d / kParts;
  const bool aligned = (C % 8 == 0) && (c0 % 8 == 0);
  for (int base = 0; base < items; base += blockDim.x) {
    const int item = base + threadIdx.x;
    const bool active = item < items;  // whole groups of 16 lanes
    const int part = item % kParts;
    const int cgj = item / kParts;
    const int cg = cgj % ncg, j = cgj / ncg;
    const int valid = min(8, nc - cg * 8);
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    if (active) {
      const typename T::storage* qrow = Q + q0 + (int64_t)j * d;
      const typename T::storage* rcol = R + c0 + cg * 8;
      const bool vec = aligned && valid == 8;
      // all loads of this lane's slice first (dp <= kMaxSlice), then the fmas
      float qv[kMaxSlice];
      float rv[kMaxSlice][8];
#pragma unroll
      for (int k = 0; k < kMaxSlice; ++k) {
        if (k < dp) {
          const int i = part * dp + k;
          qv[k] = T::load(qrow, i);
          load8<T>(rcol + (int64_t)i * C, vec, valid, rv[k]);
        }
      }
#pragma unroll
      for (int k = 0; k < kMaxSlice; ++k) {
        if (k < dp) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fma((double)qv[k], (double)rv[k][e], acc[e]);
        }
      }
    }
#pragma unroll
    for (int m = 1; m < kParts; m <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] + __shfl_xor(acc[e], m, kWave);
    }
    if (active && part == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < valid) out[j * nc + cg * 8 + e] = acc[e];
    }
  }
}

// Logistic weight of bit value 1 (sigma(+2z/tau)) and of bit value 0
// (sigma(-2z/tau)), both formed from a = exp(-2|z|/tau) <= 1.
__device__ __forceinline__ void bit_weights(double z, double two_over_tau,
                                            double& w1, double& w0) {
  const double a = exp(-fabs(z) * two_over_tau);
  const double big = 1.0 / (1.0 + a), small = a / (1.0 + a);
  w1 = z > 0.0 ? big : (z < 0.0 ? small : 0.5);
  w0 = z > 0.0 ? small : (z < 0.0 ? big : 0.5);
}

// p(u) = prod_{j < P} (bit j of u ? w1[j] : w0[j]) in float64, in the fixed
// grouping ((bits 0-2) * (bits 3-5)) * (bits 6-7), each group multiplied in
// ascending bit order; w1[j] = w0[j] = 1 for j >= P.
__device__ __forceinline__ double bucket_prob(int u, const double (&w1)[kMaxBits],
                                              const double (&w0)[kMaxBits]) {
  double g[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    double p = 1.0;
#pragma unroll
    for (int j = 3 * k; j < 3 * k + 3 && j < kMaxBits; ++j)
      p *= ((u >> j) & 1) ? w1[j] : w0[j];
    g[k] = p;
  }
  return (g[0] * g[1]) * g[2];
}

}  // namespace socket_lsh
