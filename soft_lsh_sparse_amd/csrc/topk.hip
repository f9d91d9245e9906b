// Deterministic top-k of every score row.
//
// Step 4 of the soft-LSH mechanism of SOCKET (page "Resumen Técnico: SOCKET -
// Estimador de Núcleo de Colisión Suave para Atención Escasa", section
// "Mecanismo Central: LSH Suave", item 4, and "Contribuciones Clave", item 1;
// German page "SOCKET: SOft Collision Kernel EsTimator for Sparse Attention",
// Kernmechanismus, Auswahl): the k best keys by soft score are selected
// deterministically.
//
// Total order: key n ranks above key m when score[n] > score[m], or when
// they are equal and n < m. The kk = min(k, n) highest keys are returned in
// ascending index order. Scores are compared through an order-preserving
// map of their float32 bits to uint32 (u); the selection is a radix select
// on u with digits of 11, 11 and 10 bits:
//
//  1. hist   (rows x segments blocks): 2048-bin LDS histogram of u >> 21,
//            merged into a per-row global histogram with integer atomics
//            (order-independent, so the result is deterministic). The score
//            kernel can produce this histogram itself.
//  2. filter (rows x segments blocks): every block finds the bin b1 that
//            holds the kk-th key, then compacts the (u, index) pairs of its
//            segment with digit >= b1, in index order (wave ballots and a
//            block scan), into the segment's slice of the row's list.
//  3. refine (one block per row): two more radix passes over the candidates
//            of bin b1 give the exact threshold T and the number m of keys
//            equal to T that still have to be taken. A final in-order pass
//            keeps every key with u > T and the first m keys with u == T,
//            and writes their indices at positions given by a block scan,
//            so the output is ascending by index.

#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace socket_lsh {
namespace {

constexpr int kFilterThreads = 256;
constexpr int kRefineThreads = 1024;
constexpr int kFilterUnroll = 4;  // 16-byte loads per thread per iteration

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Exclusive scan of one uint32 per thread over the block; returns the
// thread's exclusive prefix and writes the block total to *total.
// `scratch` needs blockDim/64 + 1 words. Contains __syncthreads().
template <int NT>
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch,
                                         uint32_t* total) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int w = 0; w < NWV; ++w) {
      const uint32_t t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[NWV] = run;
  }
  __syncthreads();
  const uint32_t res = scratch[wave] + x - v;
  *total = scratch[NWV];
  __syncthreads();
  return res;
}

// Given a 2048-bin histogram (global or LDS), find the bin holding the
// need-th largest element (need >= 1, need <= sum of bins): the bin b with
// count(> b) < need <= count(>= b). Writes b and count(> b) to out[0..1].
template <int NT>
__device__ void find_threshold_bin(const uint32_t* bins, uint32_t need,
                                   uint32_t* scratch, uint32_t* out) {
  constexpr int PER = kHistBins / NT;
  if (threadIdx.x == 0) {
    out[0] = 0;
    out[1] = 0;
  }
  // thread t owns bins 2047 - (t*PER + i), i.e. bins in descending order
  uint32_t cnt[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    cnt[i] = bins[kHistBins - 1 - (threadIdx.x * PER + i)];
    sum += cnt[i];
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan<NT>(sum, scratch, &total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (run < need && run + cnt[i] >= need) {
      out[0] = kHistBins - 1 - (threadIdx.x * PER + i);
      out[1] = run;
    }
    run += cnt[i];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kFilterThreads) void topk_hist_kernel(
    const float* __restrict__ scores, int64_t n, int64_t seg_len,
    uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[kHistBins];
  const int row = blockIdx.y;
  for (int i = threadIdx.x; i < kHistBins; i += kFilterThreads) h[i] = 0;
  __syncthreads();
  const float* s = scores + (int64_t)row * n;
  const int64_t n0 = (int64_t)blockIdx.x * seg_len;
  const int64_t n1 = min(n, n0 + seg_len);
  for (int64_t i = n0 + threadIdx.x; i < n1; i += kFilterThreads)
    atomicAdd(&h[float_order_key(s[i]) >> 21], 1u);
  __syncthreads();
  uint32_t* hr = hist + (int64_t)row * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kFilterThreads)
    if (h[i]) atomicAdd(hr + i, h[i]);
}

// Wave-inclusive scan of one uint32 per lane.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

__global__ __launch_bounds__(kFilterThreads) void topk_filter_kernel(
    const float* __restrict__ scores, int64_t n, int64_t kk, int segs,
    int64_t seg_len, const uint32_t* __restrict__ hist,
    uint2* __restrict__ lists, uint32_t* __restrict__ seg_cnt, int vec4) {
  constexpr int NWV = kFilterThreads / 64;
  constexpr int E = kFilterUnroll;
  __shared__ uint32_t scratch[kFilterThreads / 64 + 1];
  __shared__ uint32_t thr[2];
  __shared__ uint32_t wtot[E * NWV];
  __shared__ uint32_t woff[E * NWV + 1];
  const int row = blockIdx.y, seg = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  find_threshold_bin<kFilterThreads>(hist + (int64_t)row * kHistBins,
                                     (uint32_t)kk, scratch, thr);
  const uint32_t b1 = thr[0];

  const float* s = scores + (int64_t)row * n;
  const int64_t n0 = (int64_t)seg * seg_len;
  const int64_t n1 = min(n, n0 + seg_len);
  uint2* out = lists + (int64_t)row * n + n0;
  uint32_t count = 0;
  // Each thread takes 4 consecutive scores per step (one 16-byte load);
  // element order within an iteration is (step, thread, lane-element), i.e.
  // ascending index, and the compaction preserves it.
  for (int64_t base = n0; base < n1; base += (int64_t)kFilterThreads * 4 * E) {
    uint32_t u[E][4];
    uint32_t fl[E];
    uint32_t excl[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t i0 = base + ((int64_t)e * kFilterThreads + threadIdx.x) * 4;
      float v[4];
      if (vec4 && i0 + 3 < n1) {
        const float4 x = *reinterpret_cast<const float4*>(s + i0);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = i0 + i < n1 ? s[i0 + i] : 0.f;
      }
      uint32_t f = 0, c = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u[e][i] = float_order_key(v[i]);
        if (i0 + i < n1 && (u[e][i] >> 21) >= b1) {
          f |= 1u << i;
          ++c;
        }
      }
      fl[e] = f;
      const uint32_t inc = wave_inclusive_scan(c);
      excl[e] = inc - c;
      if (lane == 63) wtot[e * NWV + wave] = inc;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t run = 0;
      for (int q = 0; q < E * NWV; ++q) {
        woff[q] = run;
        run += wtot[q];
      }
      woff[E * NWV] = run;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      uint32_t pos = count + woff[e * NWV + wave] + excl[e];
      const int64_t i0 = base + ((int64_t)e * kFilterThreads + threadIdx.x) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (fl[e] & (1u << i)) {
          out[pos] = make_uint2(u[e][i], (uint32_t)(i0 + i));
          ++pos;
        }
      }
    }
    count += woff[E * NWV];
    __syncthreads();
  }
  if (threadIdx.x == 0) seg_cnt[(int64_t)row * segs + seg] = count;
}

// Element p (0 <= p < total) of the concatenated segment lists of a row:
// from the LDS copy when the row's candidates fit there, else from HBM.
struct RowLists {
  const uint2* glob;      // row's list area (segment s at s * seg_len)
  const uint2* cache;     // LDS copy in list order, or nullptr
  const uint32_t* off;    // segment offsets in the concatenation (LDS)
  int segs;
  int64_t seg_len;
  __device__ __forceinline__ uint2 at(uint32_t p) const {
    if (cache) return cache[p];
    int lo = 0, hi = segs - 1;  // last segment with off[s] <= p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= p) lo = mid; else hi = mid - 1;
    }
    return glob[(int64_t)lo * seg_len + (p - off[lo])];
  }
};

constexpr int kRefineCache = 10240;  // (u, index) pairs kept in LDS (80 KB)

__global__ __launch_bounds__(kRefineThreads) void topk_refine_kernel(
    int64_t n, int64_t kk, int segs, int64_t seg_len,
    const uint32_t* __restrict__ hist, const uint2* __restrict__ lists,
    const uint32_t* __restrict__ seg_cnt, int32_t* __restrict__ idx) {
  __shared__ uint32_t scratch[kRefineThreads / 64 + 1];
  __shared__ uint32_t thr[2];
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t off[65];
  __shared__ uint2 cache[kRefineCache];
  const int row = blockIdx.x;

  find_threshold_bin<kRefineThreads>(hist + (int64_t)row * kHistBins,
                                     (uint32_t)kk, scratch, thr);
  const uint32_t b1 = thr[0];
  const uint32_t need1 = (uint32_t)kk - thr[1];

  if (threadIdx.x < 64) {  // segment offsets: one wave-wide scan (segs <= 64)
    const uint32_t c = threadIdx.x < segs ? seg_cnt[(int64_t)row * segs + threadIdx.x] : 0u;
    const uint32_t inc = wave_inclusive_scan(c);
    if (threadIdx.x < segs) off[threadIdx.x] = inc - c;
    if (threadIdx.x == 63) off[segs] = inc;
  }
  __syncthreads();
  const uint32_t total = off[segs];

  RowLists rl{lists + (int64_t)row * n, nullptr, off, segs, seg_len};
  if (total <= (uint32_t)kRefineCache) {
    for (uint32_t p = threadIdx.x; p < total; p += kRefineThreads) cache[p] = rl.at(p);
    __syncthreads();
    rl.cache = cache;
  }

  // pass 2: bits 20..10 of the candidates in bin b1
  for (int i = threadIdx.x; i < kHistBins; i += kRefineThreads) h[i] = 0;
  __syncthreads();
  for (uint32_t p = threadIdx.x; p < total; p += kRefineThreads) {
    const uint2 e = rl.at(p);
    if ((e.x >> 21) == b1) atomicAdd(&h[(e.x >> 10) & 2047u], 1u);
  }
  __syncthreads();
  find_threshold_bin<kRefineThreads>(h, need1, scratch, thr);
  const uint32_t b2 = thr[0];
  const uint32_t need2 = need1 - thr[1];
  const uint32_t pre2 = (b1 << 11) | b2;  // u >> 10 of the survivors

  // pass 3: bits 9..0
  for (int i = threadIdx.x; i < kHistBins; i += kRefineThreads) h[i] = 0;
  __syncthreads();
  for (uint32_t p = threadIdx.x; p < total; p += kRefineThreads) {
    const uint2 e = rl.at(p);
    if ((e.x >> 10) == pre2) atomicAdd(&h[e.x & 1023u], 1u);
  }
  __syncthreads();
  find_threshold_bin<kRefineThreads>(h, need2, scratch, thr);
  const uint32_t T = (pre2 << 10) | thr[0];
  const uint32_t ties = need2 - thr[1];  // keys equal to T still to take

  // final pass, in index order: each thread takes 4 consecutive list entries
  int32_t* o = idx + (int64_t)row * kk;
  uint32_t run_tie = 0, run_out = 0;
  for (uint32_t base = 0; base < total; base += 4 * kRefineThreads) {
    uint2 e[4];
    uint32_t n_tie = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t p = base + threadIdx.x * 4 + i;
      e[i] = p < total ? rl.at(p) : make_uint2(0u, 0u);
      if (p < total && e[i].x == T) ++n_tie;
    }
    uint32_t tie_tot;
    uint32_t tie_rank = run_tie + block_exclusive_scan<kRefineThreads>(n_tie, scratch, &tie_tot);
    bool sel[4];
    uint32_t n_sel = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t p = base + threadIdx.x * 4 + i;
      const bool valid = p < total;
      sel[i] = valid && e[i].x > T;
      if (valid && e[i].x == T) {
        sel[i] = tie_rank < ties;
        ++tie_rank;
      }
      n_sel += sel[i] ? 1u : 0u;
    }
    uint32_t sel_tot;
    uint32_t pos = run_out + block_exclusive_scan<kRefineThreads>(n_sel, scratch, &sel_tot);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (sel[i]) {
        if (pos < (uint32_t)kk) o[pos] = (int32_t)e[i].y;
        ++pos;
      }
    }
    run_tie += tie_tot;
    run_out += sel_tot;
  }
}

__global__ void zero_u32_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ void iota_rows_kernel(int32_t* idx, int rows, int64_t n) {
  const int64_t total = (int64_t)rows * n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x)
    idx[i] = (int32_t)(i % n);
}

}  // namespace

TopkPlan plan_topk(int rows, int64_t n, int64_t k) {
  TopkPlan p{};
  p.rows = rows;
  p.n = n;
  p.kk = k < n ? k : n;
  // segments of up to 8K scores (two filter iterations of 256 threads x 16);
  // more, shorter segments when there are too few rows to fill the chip
  int64_t segs = (n + 8191) / 8192;
  const int64_t want = (1024 + rows - 1) / rows;
  if (segs < want) segs = std::min<int64_t>(want, (n + 2047) / 2048);
  segs = std::max<int64_t>(1, std::min<int64_t>(segs, 64));
  int64_t seg_len = (n + segs - 1) / segs;
  seg_len = (seg_len + 255) / 256 * 256;
  p.seg_len = std::max<int64_t>(seg_len, 256);
  p.segs = (int)((n + p.seg_len - 1) / p.seg_len);
  if (p.segs < 1) p.segs = 1;
  size_t off = 0;
  p.hist_off = off;
  off = align256(off + (size_t)rows * kHistBins * 4);
  p.cnt_off = off;
  off = align256(off + (size_t)rows * p.segs * 4);
  p.list_off = off;
  off = align256(off + (size_t)rows * n * 8);
  p.total_bytes = off;
  return p;
}

hipError_t launch_zero_u32(uint32_t* p, int64_t words, hipStream_t stream) {
  if (words <= 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((words + 255) / 256, 1024);
  launch_kernel(zero_u32_kernel, dim3(grid), dim3(256), 0, stream, p,
                     words);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, const TopkPlan& plan, int32_t* idx,
                       void* ws, bool hist_ready, hipStream_t stream) {
  if (plan.rows == 0 || plan.n == 0) return hipSuccess;
  if (plan.kk == plan.n) {
    const int64_t total = (int64_t)plan.rows * plan.n;
    const int grid = (int)std::min<int64_t>((total + 255) / 256, 4096);
    launch_kernel(iota_rows_kernel, dim3(grid), dim3(256), 0, stream, idx,
                       plan.rows, plan.n);
    return hipGetLastError();
  }
  unsigned char* base = static_cast<unsigned char*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + plan.hist_off);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(base + plan.cnt_off);
  uint2* lists = reinterpret_cast<uint2*>(base + plan.list_off);
  hipError_t err;
  if (!hist_ready) {
    err = launch_zero_u32(hist, (int64_t)plan.rows * kHistBins, stream);
    if (err != hipSuccess) return err;
    launch_kernel(topk_hist_kernel, dim3(plan.segs, plan.rows),
                       dim3(kFilterThreads), 0, stream, scores, plan.n,
                       plan.seg_len, hist);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int vec4 = (plan.n % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0) ? 1 : 0;
  launch_kernel(topk_filter_kernel, dim3(plan.segs, plan.rows),
                     dim3(kFilterThreads), 0, stream, scores, plan.n, plan.kk,
                     plan.segs, plan.seg_len, hist, lists, cnt, vec4);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  launch_kernel(topk_refine_kernel, dim3(plan.rows), dim3(kRefineThreads),
                     0, stream, plan.n, plan.kk, plan.segs, plan.seg_len, hist,
                     lists, cnt, idx);
  return hipGetLastError();
}

}  // namespace socket_lsh
