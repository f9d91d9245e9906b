// Exact softmax attention over the selected keys.
//
// Last part of step 4 of the soft-LSH mechanism of SOCKET (page "Resumen
// Técnico: SOCKET - Estimador de Núcleo de Colisión Suave para Atención
// Escasa", section "Mecanismo Central: LSH Suave", item 4; German page
// "SOCKET: SOft Collision Kernel EsTimator for Sparse Attention",
// Kernmechanismus, Auswahl): exact attention is computed over the selected
// subset only.
//
// Split-k flash decoding: each block takes one query row (b, h) and a chunk
// of its selected keys; each of its 4 waves gathers KPW key rows and the
// matching value rows with 16-byte loads (one row per LPR lanes, all loads
// of a wave issued before the first use), computes the scaled dot products,
// a wave-local softmax (max m, sum l) and the weighted value sum, and the
// block merges its 4 waves in LDS into one (m, l, acc[d]) partial. A second
// kernel merges the chunk partials of a row in chunk order (the online
// softmax merge) and writes the output in the input dtype. Everything runs
// in float32 in a fixed order, so results are reproducible run to run.
//
// Blocks are dealt to the 8 XCDs round-robin; the mapping below keeps all
// query heads of one KV head on one XCD and issues the G heads of a chunk
// back to back, so keys chosen by several heads of a group are likely to be
// served from that XCD's L2.

#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace socket_lsh {
namespace {

// Waves per block: 4, or 1 where 4-wave blocks would not give 512 blocks
// (a CU pulls gathered rows at a limited rate, so short rows are spread
// over more CUs).
constexpr int kAttnWaves = 4;
constexpr int kAttnLoads = 8;  // 16-byte loads per lane, tensor and batch

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& w, float* f);
template <>
__device__ __forceinline__ void unpack16<BF16>(const uint4& w, float* f) {
  unpack8_bf16(w, f);
}
template <>
__device__ __forceinline__ void unpack16<F32>(const uint4& w, float* f) {
  unpack4_f32(w, f);
}

// WAVES waves per block. DIRECT (one chunk per row): the block's merge is
// the row's, and the output is written in the input dtype (the merge
// kernel's arithmetic over a single chunk: at / lt).
template <typename T, int D, int KPW, int WAVES, bool DIRECT>
__global__ __launch_bounds__(WAVES * 64) void sparse_attn_kernel(
    const typename T::storage* __restrict__ Q,
    const typename T::storage* __restrict__ K,
    const typename T::storage* __restrict__ V, int Hq, int Hkv, int bhkv,
    int64_t stride, const int32_t* __restrict__ idx, int64_t kk, int chunks,
    float* __restrict__ partial, typename T::storage* __restrict__ final_out) {
  constexpr int kAttnThreads = WAVES * 64;
  constexpr int EPL = 16 / T::bytes;  // elements per 16-byte load
  constexpr int LPR = D / EPL;        // lanes per key row
  constexpr int KPI = 64 / LPR;       // key rows per wave-wide load
  constexpr int IT = kAttnLoads;      // loads per tensor per batch
  constexpr int KPB = IT * KPI;       // keys per batch
  constexpr int NB = KPW / KPB;       // batches per wave
  static_assert(NB * KPB == KPW && KPW % 64 == 0, "keys per wave");
  constexpr int NREG = KPW / 64;
  constexpr int CHUNK = KPW * WAVES;
  __shared__ float sm_m[WAVES], sm_l[WAVES];
  __shared__ float sm_acc[WAVES][D];

  const int G = Hq / Hkv;
  const int per_group = G * chunks;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int gi = xcd + 8 * (slot / per_group);
  if (gi >= bhkv) return;
  const int local = slot % per_group;
  const int chunk = local / G, j = local % G;
  const int b = gi / Hkv, g = gi % Hkv;
  const int h = g * G + j;
  const int64_t row = (int64_t)b * Hq + h;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / LPR, sub = lane % LPR;
  const float scale = 1.0f / sqrtf((float)D);

  // the wave's key indices, one position per lane and register; positions
  // past kk repeat the last selected key (loaded, then given weight 0) and
  // indices outside [0, stride) are clamped, so no load leaves the head
  const int64_t wbeg = (int64_t)chunk * CHUNK + wave * KPW;
  const int32_t* irow = idx + row * kk;
  int ireg[NREG];
#pragma unroll
  for (int r = 0; r < NREG; ++r) {
    const int64_t p = min<int64_t>(wbeg + r * 64 + lane, kk - 1);
    ireg[r] = (int)min<int64_t>(max(irow[p], 0), stride - 1);
  }

  float qf[EPL];
  {
    const uint4 w = *reinterpret_cast<const uint4*>(Q + row * D + sub * EPL);
    unpack16<T>(w, qf);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[e] *= scale;
  }

  const typename T::storage* Kh = K + (int64_t)gi * stride * D + sub * EPL;
  const typename T::storage* Vh = V + (int64_t)gi * stride * D + sub * EPL;

  // Batches of KPB keys, double-buffered: the loads of batch bt + 1 are in
  // flight while batch bt is consumed. The running softmax (m, l, acc) is
  // rescaled once per batch; m is the same in every lane of the wave.
  uint4 kr[2][IT], vr[2][IT];
  float m = -INFINITY, l = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  auto issue = [&](int bt) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int p = bt * KPB + it * KPI + grp;  // position within the wave
      const int key = __shfl(ireg[p >> 6], p & 63, kWave);
      kr[bt & 1][it] = *reinterpret_cast<const uint4*>(Kh + (int64_t)key * D);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int p = bt * KPB + it * KPI + grp;
      const int key = __shfl(ireg[p >> 6], p & 63, kWave);
      vr[bt & 1][it] = *reinterpret_cast<const uint4*>(Vh + (int64_t)key * D);
    }
  };

  issue(0);
#pragma unroll
  for (int bt = 0; bt < NB; ++bt) {
    if (bt + 1 < NB) issue(bt + 1);
    float s[IT];
    float mb = -INFINITY;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float f[EPL];
      unpack16<T>(kr[bt & 1][it], f);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(qf[e], f[e], dot);
      dot = lane_group_sum<LPR>(dot);
      const bool valid = wbeg + bt * KPB + it * KPI + grp < kk;
      s[it] = valid ? dot : -INFINITY;
      mb = fmaxf(mb, s[it]);
    }
    // the key groups of the wave hold different keys: combine across them
    // (lane i with lane i ^ o keeps the position within the row)
    if constexpr (LPR <= 8) mb = fmaxf(mb, xor_lanes<8>(mb));
    if constexpr (LPR <= 16) mb = fmaxf(mb, xor_lanes<16>(mb));
    if constexpr (LPR <= 32) mb = fmaxf(mb, xor_lanes<32>(mb));
    const float mn = fmaxf(m, mb);
    const float c = m == -INFINITY ? 0.f : __expf(m - mn);
    l *= c;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= c;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const float p = s[it] == -INFINITY ? 0.f : __expf(s[it] - mn);
      l += p;
      float f[EPL];
      unpack16<T>(vr[bt & 1][it], f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, f[e], acc[e]);
    }
    m = mn;
  }
  if constexpr (LPR <= 8) {
    l += xor_lanes<8>(l);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += xor_lanes<8>(acc[e]);
  }
  if constexpr (LPR <= 16) {
    l += xor_lanes<16>(l);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += xor_lanes<16>(acc[e]);
  }
  if constexpr (LPR <= 32) {
    l += xor_lanes<32>(l);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += xor_lanes<32>(acc[e]);
  }
  if (lane == 0) {
    sm_m[wave] = m;
    sm_l[wave] = l;
  }
  if (grp == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm_acc[wave][sub * EPL + e] = acc[e];
  }
  __syncthreads();

  float* out = partial + (row * chunks + chunk) * (D + 2);
  for (int t = threadIdx.x; t < D; t += kAttnThreads) {
    float mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) mt = fmaxf(mt, sm_m[w]);
    float lt = 0.f, at = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float c = sm_m[w] == -INFINITY ? 0.f : expf(sm_m[w] - mt);
      lt = fmaf(c, sm_l[w], lt);
      at = fmaf(c, sm_acc[w][t], at);
    }
    if constexpr (DIRECT) {
      T::store(final_out, row * D + t, at / lt);
      continue;
    }
    out[t] = at;
    if (t == 0) {
      out[D] = mt;
      out[D + 1] = lt;
    }
  }
}

constexpr int kMergeMaxChunks = 1024;

// Online-softmax merge of the chunk partials of one row, in chunk order.
// Up to kMergeRegChunks chunks (the sparse decode's 4-16): every thread
// requests the (m, l) pair and its coordinate of every chunk at once, one
// memory round trip, and merges them itself. More chunks (the dense
// baseline): the (m, l) pairs are staged in LDS first, then the
// accumulator loads, which are independent, are issued back to back. Both
// take the same steps in the same order, so their results are equal.
template <typename T, int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(
    const float* __restrict__ partial, int chunks,
    typename T::storage* __restrict__ out) {
  __shared__ float sw[kMergeMaxChunks];
  __shared__ float sl[kMergeMaxChunks];
  __shared__ float s_tot[2];
  const int64_t row = blockIdx.x;
  const float* p = partial + row * chunks * (D + 2);
  const int t = threadIdx.x;
  if (chunks <= kMergeRegChunks) {  // block-uniform
    float m[kMergeRegChunks], l[kMergeRegChunks], a[kMergeRegChunks];
#pragma unroll
    for (int c = 0; c < kMergeRegChunks; ++c) {
      const float* pc = p + (int64_t)min(c, chunks - 1) * (D + 2);
      m[c] = pc[D];
      l[c] = pc[D + 1];
      a[c] = pc[t];
    }
    float mt = -INFINITY;
#pragma unroll
    for (int c = 0; c < kMergeRegChunks; ++c)
      if (c < chunks) mt = fmaxf(mt, m[c]);
    float lt = 0.f, at = 0.f;
#pragma unroll
    for (int c = 0; c < kMergeRegChunks; ++c)
      if (c < chunks) {
        const float w = m[c] == -INFINITY ? 0.f : expf(m[c] - mt);
        lt = fmaf(w, l[c], lt);
        at = fmaf(w, a[c], at);
      }
    T::store(out, row * D + t, at / lt);
    return;
  }
  for (int c = t; c < chunks; c += D) {
    sw[c] = p[c * (D + 2) + D];
    sl[c] = p[c * (D + 2) + D + 1];
  }
  __syncthreads();
  if (t == 0) {
    float mt = -INFINITY;
    for (int c = 0; c < chunks; ++c) mt = fmaxf(mt, sw[c]);
    float lt = 0.f;
    for (int c = 0; c < chunks; ++c) {
      const float w = sw[c] == -INFINITY ? 0.f : expf(sw[c] - mt);
      sw[c] = w;
      lt = fmaf(w, sl[c], lt);
    }
    s_tot[0] = lt;
  }
  __syncthreads();
  float at = 0.f;
#pragma unroll 8
  for (int c = 0; c < chunks; ++c) at = fmaf(sw[c], p[c * (D + 2) + t], at);
  T::store(out, row * D + t, at / s_tot[0]);
}

template <typename T, int D, int KPW, int WAVES>
hipError_t launch_attn_t(const void* Q, const void* K, const void* V,
                         const AttnPlan& plan, int64_t stride,
                         const int32_t* idx, void* out, float* partial,
                         hipStream_t stream) {
  using S = typename T::storage;
  const int G = plan.Hq / plan.Hkv;
  const int bhkv = plan.B * plan.Hkv;
  const int per_group = G * plan.chunks;
  const int grid = ((bhkv + 7) / 8) * 8 * per_group;
  if (plan.chunks == 1) {  // the block's merge is the row's: output written directly
    launch_kernel((sparse_attn_kernel<T, D, KPW, WAVES, true>), dim3(grid), dim3(WAVES * 64),
                  0, stream, (const S*)Q, (const S*)K, (const S*)V, plan.Hq, plan.Hkv, bhkv,
                  stride, idx, plan.kk, 1, partial, (S*)out);
    return hipGetLastError();
  }
  launch_kernel((sparse_attn_kernel<T, D, KPW, WAVES, false>), dim3(grid), dim3(WAVES * 64), 0,
                stream, (const S*)Q, (const S*)K, (const S*)V, plan.Hq, plan.Hkv, bhkv, stride,
                idx, plan.kk, plan.chunks, partial, nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  launch_kernel((attn_merge_kernel<T, D>), dim3(plan.B * plan.Hq),
                     dim3(D), 0, stream, partial, plan.chunks, (S*)out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_attn_d(const void* Q, const void* K, const void* V,
                         const AttnPlan& plan, int64_t stride,
                         const int32_t* idx, void* out, float* partial,
                         hipStream_t stream) {
  if (plan.waves == 1)  // 64 keys per block (plan_attn)
    return launch_attn_t<T, D, 64, 1>(Q, K, V, plan, stride, idx, out, partial, stream);
  switch (plan.keys_per_wave) {
    case 256:
      return launch_attn_t<T, D, 256, kAttnWaves>(Q, K, V, plan, stride, idx, out, partial,
                                                  stream);
    case 128:
      return launch_attn_t<T, D, 128, kAttnWaves>(Q, K, V, plan, stride, idx, out, partial,
                                                  stream);
    default:
      return launch_attn_t<T, D, 64, kAttnWaves>(Q, K, V, plan, stride, idx, out, partial,
                                                 stream);
  }
}

}  // namespace

hipError_t launch_attn_merge(const float* partial, int rows, int chunks, int d, bool bf16,
                             void* out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (bf16) {
    if (d == 128)
      launch_kernel((attn_merge_kernel<BF16, 128>), dim3(rows), dim3(128), 0, stream, partial,
                    chunks, (BF16::storage*)out);
    else
      launch_kernel((attn_merge_kernel<BF16, 64>), dim3(rows), dim3(64), 0, stream, partial,
                    chunks, (BF16::storage*)out);
  } else {
    if (d == 128)
      launch_kernel((attn_merge_kernel<F32, 128>), dim3(rows), dim3(128), 0, stream, partial,
                    chunks, (F32::storage*)out);
    else
      launch_kernel((attn_merge_kernel<F32, 64>), dim3(rows), dim3(64), 0, stream, partial,
                    chunks, (F32::storage*)out);
  }
  return hipGetLastError();
}

AttnPlan plan_attn(int B, int Hq, int Hkv, int d, int64_t kk) {
  AttnPlan p{};
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.d = d;
  p.kk = kk;
  const int64_t rows = (int64_t)B * Hq;
  p.waves = kAttnWaves;
  // the most keys per wave that still give 512 blocks (two per CU)
  int kpw = 64;
  for (int cand : {256, 128}) {
    const int64_t chunks = (kk + cand * kAttnWaves - 1) / (cand * kAttnWaves);
    if (rows * chunks >= 512) {
      kpw = cand;
      break;
    }
  }
  int64_t chunks = (kk + kpw * kAttnWaves - 1) / (kpw * kAttnWaves);
  const int64_t wave_chunks = (kk + 63) / 64;
  if (rows * chunks < 512 && chunks > 1 && wave_chunks <= kMergeRegChunks) {
    // one-wave blocks of 64 keys: up to 4x the blocks, merged from registers
    p.waves = 1;
    chunks = wave_chunks;
  }
  p.keys_per_wave = kpw;
  p.chunk_keys = kpw * p.waves;
  p.chunks = (int)chunks;
  if (p.chunks < 1) p.chunks = 1;
  p.partial_bytes = (size_t)rows * p.chunks * (d + 2) * sizeof(float);
  return p;
}

hipError_t launch_sparse_attn(const void* Q, const void* K, const void* V,
                              bool bf16, const AttnPlan& plan, int64_t stride,
                              const int32_t* idx, void* out, float* partial,
                              hipStream_t stream) {
  if (plan.B == 0 || plan.Hq == 0) return hipSuccess;
  if (bf16) {
    if (plan.d == 128)
      return launch_attn_d<BF16, 128>(Q, K, V, plan, stride, idx, out, partial, stream);
    return launch_attn_d<BF16, 64>(Q, K, V, plan, stride, idx, out, partial, stream);
  }
  if (plan.d == 128)
    return launch_attn_d<F32, 128>(Q, K, V, plan, stride, idx, out, partial, stream);
  return launch_attn_d<F32, 64>(Q, K, V, plan, stride, idx, out, partial, stream);
}

}  // namespace socket_lsh
