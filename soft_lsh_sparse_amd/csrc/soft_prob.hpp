// Soft bucket probabilities: projections, per-bit weights and bit-group
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
//
// Arithmetic:
//  * z = q . r in float64: each of d/16 lanes takes 16 consecutive
//    coordinates (fma from 0, ascending), and the d/16 partial sums of a
//    column are added by a fixed DPP pattern;
//  * a bit's weights from a = exp(-2|z|/tau): 1/(1+a) and a/(1+a);
//  * per table, the products of the bit groups (bits 0-2, 3-5, 6-7; each
//    multiplied in ascending bit order from 1.0), and
//    p(u) = (A[u & 7] * B[(u >> 3) & 7]) * C[u >> 6], rounded to float32.
#pragma once

#include <algorithm>

#include "common.hpp"

namespace socket_lsh {

template <bool BF>
__device__ __forceinline__ float load1(const void* base, int64_t elem) {
  if constexpr (BF) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[elem]);
  else return static_cast<const float*>(base)[elem];
}

// Sum over each aligned group of 8 (4) lanes (the same pairing in every lane).
__device__ __forceinline__ double sum8_f64(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  return v;
}
__device__ __forceinline__ double sum4_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  return v;
}

// 16 consecutive elements (bf16 when BF, else f32) at element `elem` of a
// 16-byte aligned array, as 16-byte words (2 for bf16, 4 for f32).
template <bool BF>
struct Raw16 {
  static constexpr int kWords = BF ? 2 : 4;
  uint4 w[kWords];
  __device__ __forceinline__ void load(const void* base, int64_t elem) {
    const uint4* p = BF ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem)
                        : reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = p[i];
  }
  // element e (0..15) as float; e must be a compile-time constant after unrolling
  __device__ __forceinline__ float at(int e) const {
    if constexpr (BF) {
      const uint4& q = w[e >> 3];
      const uint32_t x = (e & 7) < 2 ? q.x : (e & 7) < 4 ? q.y : (e & 7) < 6 ? q.z : q.w;
      return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
    } else {
      const uint4& q = w[e >> 2];
      const uint32_t x = (e & 3) == 0 ? q.x : (e & 3) == 1 ? q.y : (e & 3) == 2 ? q.z : q.w;
      return __uint_as_float(x);
    }
  }
};

// Projections z[j * nc + c] = q_j . R[:, c0 + c] (float64) of the `rows`
// query rows starting at element q0 of Q (d = 64 or 128 coordinates each,
// bf16 when BF, else f32) on nc of the C hyperplane columns of R [d][C].
// Block-cooperative: a lane accumulates 8 consecutive columns over 16
// consecutive coordinates, fma from 0 in ascending coordinate order, with
// all of its loads issued before the first fma; the d/16 parts of a column
// group sit in adjacent lanes and are added by a fixed DPP pattern.
// blockDim.x must be a multiple of 64; Q and R 16-byte aligned.
template <bool BF>
__device__ __forceinline__ void group_projections(const void* Q, int64_t q0, int rows, int d,
                                                  const void* R, int C, int c0, int nc,
                                                  double* out) {
  const int parts = d / 16;  // 4 or 8
  const int ncg = (nc + 7) / 8;
  const int items = rows * ncg * parts;
  const bool vec = C % 8 == 0 && c0 % 8 == 0;
  for (int base = 0; base < items; base += blockDim.x) {
    const int item = base + threadIdx.x;
    const bool active = item < items;  // whole groups of `parts` lanes
    const int part = item % parts;
    const int cg = (item / parts) % ncg;
    const int j = item / (parts * ncg);
    const int valid = min(8, nc - cg * 8);
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    if (active && vec) {
      Raw16<BF> qw;
      qw.load(Q, q0 + (int64_t)j * d + part * 16);
      // R: the 8 columns of each coordinate (16 bytes in bf16, 32 in f32)
      constexpr int kRound = BF ? 16 : 8;  // coordinates per round of loads
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += kRound) {
        uint4 rw[kRound][BF ? 1 : 2];
#pragma unroll
        for (int k = 0; k < kRound; ++k) {
          const int64_t el = (int64_t)(part * 16 + k0 + k) * C + c0 + cg * 8;
          if constexpr (BF) {
            rw[k][0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(R) + el);
          } else {
            const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(R) + el);
            rw[k][0] = p[0];
            rw[k][1] = p[1];
          }
        }
#pragma unroll
        for (int k = 0; k < kRound; ++k) {
          float rv[8];
          if constexpr (BF) {
            unpack8_bf16(rw[k][0], rv);
          } else {
            unpack4_f32(rw[k][0], rv);
            unpack4_f32(rw[k][1], rv + 4);
          }
          const double qk = (double)qw.at(k0 + k);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fma(qk, (double)rv[e], acc[e]);
        }
      }
    } else if (active) {
      for (int k = 0; k < 16; ++k) {
        const int i = part * 16 + k;
        const double qi = (double)load1<BF>(Q, q0 + (int64_t)j * d + i);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < valid)
            acc[e] = fma(qi, (double)load1<BF>(R, (int64_t)i * C + c0 + cg * 8 + e), acc[e]);
      }
    }
    if (parts == 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = sum8_f64(acc[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = sum4_f64(acc[e]);
    }
    if (active && part == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < valid) out[(int64_t)j * nc + cg * 8 + e] = acc[e];
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

// Entries of the bit-group products of one table: A (bits 0-2), B (bits
// 3-5), C (bits 6-7), each 2^(bits of the group below P).
struct GroupSizes {
  int a, b, c;
  __device__ __host__ explicit GroupSizes(int P)
      : a(1 << std::min(P, 3)), b(1 << std::min(std::max(P - 3, 0), 3)),
        c(1 << std::min(std::max(P - 6, 0), 2)) {}
  __device__ __host__ int total() const { return a + b + c; }
};

__device__ __forceinline__ double group_prob(const double* g, const GroupSizes& gs, int u) {
  return (g[u & (gs.a - 1)] * g[gs.a + ((u >> 3) & (gs.b - 1))]) * g[gs.a + gs.b + (u >> 6)];
}

// Strides (doubles) of the group products in LDS: table l of row j at
// j * row + l * table. The table stride is odd and the row stride is
// 16/G mod 16 (G: rows whose tables are read side by side, as the entries
// (u, l, j) with j fastest), so that 16 lanes reading entry k of
// consecutive (l, j) hit 16 different bank pairs.
struct GroupStrides {
  int table, row;
  __device__ __host__ GroupStrides(int L, int P, int G) {
    table = GroupSizes(P).total() | 1;
    const int want = G > 1 ? 16 / G : 0;
    row = L * table;
    if (G > 1) row += ((want - row) % 16 + 16) % 16;
  }
};

// LDS (doubles) of the set-up of nl tables of `rows` query rows:
// projections and the two weights, then the group products.
__device__ __host__ inline size_t table_zw_doubles(int rows, int nl, int P) {
  return (size_t)rows * 3 * (size_t)nl * P;
}
__device__ __host__ inline size_t table_gp_doubles(int rows, int nl, int P) {
  return (size_t)rows * (size_t)GroupStrides(nl, P, rows).row;
}

// Block-cooperative set-up of tables l0 .. l0+nl-1 of `rows` consecutive
// query rows (from element q0 of Q; bf16 when BF, else f32): projections
// and weights (in zw, table_zw_doubles), then the group products (in gp,
// table_gp_doubles): those of table l0 + ll of row j start at
// gp + j * GroupStrides(nl, P, rows).row + ll * GroupStrides(nl, P, rows).table.
// Contains __syncthreads(); zw is free again when it returns.
template <bool BF>
__device__ __forceinline__ void table_setup(const void* Q, int64_t q0, int rows, int d, const void* R, int L,
                            int l0, int nl, int P, double two_over_tau, double* zw,
                            double* gp) {
  const int C = L * P, nc = nl * P;
  const GroupSizes gs(P);
  const int gsz = gs.total();
  const GroupStrides st(nl, P, rows);
  double* z = zw;                         // [rows][nc]
  double* w1 = z + (size_t)rows * nc;     // [rows][nc]
  double* w0 = w1 + (size_t)rows * nc;    // [rows][nc]
  group_projections<BF>(Q, q0, rows, d, R, C, l0 * P, nc, z);
  __syncthreads();
  for (int i = threadIdx.x; i < rows * nc; i += blockDim.x)
    bit_weights(z[i], two_over_tau, w1[i], w0[i]);
  __syncthreads();
  for (int e = threadIdx.x; e < rows * nl * gsz; e += blockDim.x) {
    const int jl = e / gsz, k = e % gsz;  // jl = j * nl + ll
    int combo, j0, nb;
    if (k < gs.a) {
      combo = k; j0 = 0; nb = std::min(P, 3);
    } else if (k < gs.a + gs.b) {
      combo = k - gs.a; j0 = 3; nb = std::min(std::max(P - 3, 0), 3);
    } else {
      combo = k - gs.a - gs.b; j0 = 6; nb = std::max(P - 6, 0);
    }
    double p = 1.0;
    for (int jj = 0; jj < nb; ++jj) {
      const int c = jl * P + j0 + jj;  // column ll * P + bit of row j
      p *= ((combo >> jj) & 1) ? w1[c] : w0[c];
    }
    const int j = jl / nl, ll = jl % nl;
    gp[j * st.row + ll * st.table + k] = p;
  }
  __syncthreads();
}

}  // namespace socket_lsh
