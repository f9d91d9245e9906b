// Soft bucket probabilities of the decode queries.
//
// Step 2 of the soft-LSH mechanism of SOCKET (page "Resumen Técnico: SOCKET -
// Estimador de Núcleo de Colisión Suave para Atención Escasa", section
// "Mecanismo Central: LSH Suave", item 2; German page "SOCKET: SOft Collision
// Kernel EsTimator for Sparse Attention", Kernmechanismus, Weiche Zuweisung):
// the query's projections on the random hyperplanes go through a
// temperature-controlled softmax that spreads it over every bucket of every
// table.
//
// With the logit form logit(u) = (1/tau) * sum_j s_j(u) z_j (s_j = +1 when
// bit j of u is set, else -1) the softmax over the 2^P buckets equals the
// product over bits of logistic terms,
//     p(u) = prod_j sigma(2 s_j(u) z_j / tau),
// because the normaliser sum_u exp(logit(u) - max) factorises into
// prod_j (1 + exp(-2|z_j|/tau)). The kernel evaluates that product in
// float64 (P exponentials per table instead of 2^P) and stores float32. The
// projections z are float64 dot products of the bf16/f32 inputs (exact
// products), so the stored probabilities are float32 roundings of values
// accurate to a few float64 ulps.
//
// Output layout [B, Hkv, 2^P, L, G]: entry (b, g, u, l, j) belongs to query
// head g*G + j, so one 16-byte read gives a whole GQA group (G = 4) and, for
// a fixed bucket, the L tables sit in consecutive 16-byte slots.

#include "common.hpp"
#include "kernels.hpp"
#include "soft_prob.hpp"

#include <algorithm>

namespace socket_lsh {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void bucket_probs_kernel(
    const typename T::storage* __restrict__ Q,
    const typename T::storage* __restrict__ R, int Hq, int Hkv, int d, int L,
    int P, double two_over_tau, int tables_per_block,
    float* __restrict__ table, uint32_t* __restrict__ zero_ptr,
    int64_t zero_words) {
  extern __shared__ double zs[];  // [G][nl*P] projections, then weights
  const int G = Hq / Hkv;
  const int bg = blockIdx.x;  // b * Hkv + g
  const int b = bg / Hkv, g = bg % Hkv;
  const int l0 = blockIdx.y * tables_per_block;
  const int nl = min(tables_per_block, L - l0);
  const int C = L * P;
  const int ncols = nl * P;

  // Optional clearing of per-call counters (spread over all blocks).
  if (zero_ptr != nullptr) {
    const int64_t nblocks = (int64_t)gridDim.x * gridDim.y;
    const int64_t bid = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    for (int64_t i = bid * blockDim.x + threadIdx.x; i < zero_words;
         i += nblocks * blockDim.x)
      zero_ptr[i] = 0u;
  }

  block_projections<T>(Q, ((int64_t)b * Hq + g * G) * d, R, C, l0 * P, ncols, d, G, zs);
  __syncthreads();
  double* w1s = zs + G * ncols;  // bit weights, computed once per column
  double* w0s = w1s + G * ncols;
  for (int i = threadIdx.x; i < G * ncols; i += blockDim.x)
    bit_weights(zs[i], two_over_tau, w1s[i], w0s[i]);
  __syncthreads();

  // one thread per (bucket, table, head): consecutive threads write
  // consecutive (table, head) slots of one bucket row
  const int nbuckets = 1 << P;
  const int per_bucket = nl * G;
  const int total = nbuckets * per_bucket;
  float* out = table + (int64_t)bg * nbuckets * L * G;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int u = e / per_bucket;
    const int rem = e % per_bucket;
    const int ll = rem / G, j = rem % G;
    double w1[kMaxBits], w0[kMaxBits];
#pragma unroll
    for (int jj = 0; jj < kMaxBits; ++jj) {
      w1[jj] = 1.0;
      w0[jj] = 1.0;
      if (jj < P) {
        w1[jj] = w1s[j * ncols + ll * P + jj];
        w0[jj] = w0s[j * ncols + ll * P + jj];
      }
    }
    out[((int64_t)u * L + l0 + ll) * G + j] = (float)bucket_prob(u, w1, w0);
  }
}

}  // namespace

hipError_t launch_bucket_probs(const void* Q, const void* R, bool bf16, int B,
                               int Hq, int Hkv, int d, int L, int P,
                               float tau, float* table, uint32_t* zero_ptr,
                               int64_t zero_words, hipStream_t stream) {
  const int G = Hq / Hkv;
  const int bhkv = B * Hkv;
  // enough blocks to cover the chip; LDS per block: the float64 projections
  int tpb = (int)(((int64_t)L * bhkv + 511) / 512);
  tpb = std::max(1, std::min(tpb, L));
  const int nchunks = (L + tpb - 1) / tpb;
  const size_t shmem = (size_t)3 * G * tpb * P * sizeof(double);
  const double two_over_tau = 2.0 / (double)tau;
  dim3 grid(bhkv, nchunks);
  if (bf16)
    launch_kernel(bucket_probs_kernel<BF16>, grid, dim3(256), shmem,
                       stream, (const uint16_t*)Q, (const uint16_t*)R, Hq, Hkv,
                       d, L, P, two_over_tau, tpb, table, zero_ptr,
                       zero_words);
  else
    launch_kernel(bucket_probs_kernel<F32>, grid, dim3(256), shmem,
                       stream, (const float*)Q, (const float*)R, Hq, Hkv, d, L,
                       P, two_over_tau, tpb, table, zero_ptr, zero_words);
  return hipGetLastError();
}

}  // namespace socket_lsh
