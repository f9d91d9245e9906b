// Soft bucket probabilities, shared by the standalone table kernel and the
// score kernel that builds its table in LDS (both must produce bit-identical
// tables).
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

// z = sum_i q_i r_i in float64 (two interleaved partial sums, then added).
// bf16 and f32 products are exact in float64.
template <class QF, class RF>
__device__ __forceinline__ double proj_dot(QF q, RF r, int d) {
  double z0 = 0.0, z1 = 0.0;
  for (int i = 0; i < d; i += 2) {
    z0 = fma((double)q(i), (double)r(i), z0);
    z1 = fma((double)q(i + 1), (double)r(i + 1), z1);
  }
  return z0 + z1;
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

// p(u) = prod_{j < P} (bit j of u ? w1[j] : w0[j]), multiplied in ascending
// bit order in float64.
__device__ __forceinline__ double bucket_prob(int u, const double (&w1)[kMaxBits],
                                              const double (&w0)[kMaxBits], int P) {
  double p = 1.0;
#pragma unroll
  for (int j = 0; j < kMaxBits; ++j)
    if (j < P) p *= ((u >> j) & 1) ? w1[j] : w0[j];
  return p;
}

}  // namespace socket_lsh
