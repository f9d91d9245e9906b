// Soft bucket probabilities of the decode queries.
//
// Step 2 of the soft-LSH mechanism of SOCKET (page "Resumen Técnico: SOCKET -
// Estimador de Núcleo de Colisión Suave para Atención Escasa", section
// "Mecanismo Central: LSH Suave", item 2; German page "SOCKET: SOft Collision
// Kernel EsTimator for Sparse Attention", Kernmechanismus, Weiche Zuweisung):
// the query's projections on the random hyperplanes go through a
// temperature-controlled softmax that spreads it over every bucket of every
// table. The softmax of the chosen logit form factorises into per-bit
// logistic terms; soft_prob.hpp holds the arithmetic, which the decode's
// score kernel shares (it builds its KV group's tables the same way).
//
// One block per (batch, KV head) and chunk of tables: it builds the tables
// of the chunk for the G query heads of the group (projections on the
// chunk's hyperplanes only). Output layout [B, Hkv, 2^P, L, G]: entry
// (b, g, u, l, j) belongs to query head g*G + j, so one 16-byte read gives a
// whole GQA group (G = 4) and, for a fixed bucket, the L tables sit in
// consecutive 16-byte slots. Consecutive threads write consecutive (l, j)
// entries of one bucket.

#include "common.hpp"
#include "kernels.hpp"
#include "soft_prob.hpp"

#include <algorithm>
#include <numeric>

namespace socket_lsh {
namespace {

constexpr int kProbThreads = 256;

struct ProbArgs {
  const void* Q;
  const void* R;
  int Hq, Hkv, d, L, P, tables_per_block;
  double two_over_tau;
  float* table;
};

template <bool BF>
__global__ __launch_bounds__(kProbThreads) void bucket_probs_kernel(ProbArgs a) {
  extern __shared__ __align__(16) double smem[];
  const int bg = blockIdx.x;  // b * Hkv + g
  const int G = a.Hq / a.Hkv;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int L = a.L, P = a.P;
  const int l0 = blockIdx.y * a.tables_per_block;
  const int nl = min(a.tables_per_block, L - l0);
  const GroupSizes gs(P);
  const GroupStrides st(nl, P, G);
  double* gp = smem + table_zw_doubles(G, nl, P);
  table_setup<BF>(a.Q, ((int64_t)b * a.Hq + (int64_t)g * G) * a.d, G, a.d, a.R, L, l0, nl, P,
                  a.two_over_tau, smem, gp);
  const int nbuckets = 1 << P;
  const int per_u = nl * G;  // entries (ll, j) of one bucket, j fastest
  float* out = a.table + (int64_t)bg * nbuckets * L * G + (int64_t)l0 * G;
  for (int e = threadIdx.x; e < nbuckets * per_u; e += blockDim.x) {
    const int u = e / per_u, r = e % per_u;
    const int ll = r / G, j = r % G;
    out[((int64_t)u * L + ll) * G + j] = (float)group_prob(gp + j * st.row + ll * st.table, gs, u);
  }
}

// Group table of the GQA group-shared variant: out[bg, u, l] = the sum over
// the G heads j (in order) of table[bg, u, l, j].
__global__ __launch_bounds__(256) void group_table_sum_kernel(const float* __restrict__ table,
                                                              int64_t entries, int G,
                                                              float* __restrict__ out) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < entries;
       e += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int j = 0; j < G; ++j) s += table[e * G + j];
    out[e] = s;
  }
}

}  // namespace

hipError_t launch_group_table_sum(const float* table, int bhkv, int L, int P, int G, float* out,
                                  hipStream_t stream) {
  const int64_t entries = (int64_t)bhkv * ((int64_t)1 << P) * L;
  const int grid = (int)std::min<int64_t>((entries + 255) / 256, 1024);
  launch_kernel(group_table_sum_kernel, dim3(grid), dim3(256), 0, stream, table, entries, G, out);
  return hipGetLastError();
}

hipError_t launch_bucket_probs(const void* Q, const void* R, bool bf16, int B,
                               int Hq, int Hkv, int d, int L, int P,
                               float tau, float* table, hipStream_t stream) {
  static bool lds_limit_set = false;
  if (!lds_limit_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&bucket_probs_kernel<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsBytesPerCU);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&bucket_probs_kernel<false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsBytesPerCU);
    lds_limit_set = true;
  }
  ProbArgs a{};
  a.Q = Q;
  a.R = R;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.L = L;
  a.P = P;
  a.two_over_tau = 2.0 / (double)tau;
  a.table = table;
  // about 512 blocks over the chip, at most 8 tables per block (bounds LDS);
  // a block's first column and column count are multiples of 8 where the
  // tables allow (whole 16-byte loads of the hyperplane rows: the
  // projections then take all their loads at once)
  const int bhkv = B * Hkv;
  int tpb = (int)(((int64_t)L * bhkv + 511) / 512);
  tpb = std::max(1, std::min(tpb, std::min(L, 8)));
  const int m = 8 / std::gcd(P, 8);  // tables per 8 columns
  if (m <= std::min(L, 8)) tpb = std::min((tpb + m - 1) / m * m, std::min(L, 8) / m * m);
  a.tables_per_block = tpb;
  const int G = Hq / Hkv;
  const size_t lds = (table_zw_doubles(G, tpb, P) + table_gp_doubles(G, tpb, P)) * sizeof(double);
  const dim3 grid(bhkv, (L + tpb - 1) / tpb);
  if (bf16)
    launch_kernel(bucket_probs_kernel<true>, grid, dim3(kProbThreads), lds, stream, a);
  else
    launch_kernel(bucket_probs_kernel<false>, grid, dim3(kProbThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace socket_lsh
