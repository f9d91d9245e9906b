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
//            holds the kk-th key; each wave then compacts the (u, index)
//            pairs of its sub-segment with digit >= b1, in index order (four
//            ballots and lane prefix counts per step), into its own sub-list
//            of the row's list.
//  3. refine (one block per row): the sub-lists are copied back to back
//            into LDS; two more radix passes over the candidates of bin b1
//            give the exact threshold T and the number m of keys
//            equal to T that still have to be taken. A final in-order pass
//            keeps every key with u > T and the first m keys with u == T,
//            and writes their indices at positions given by a block scan,
//            so the output is ascending by index.

#include "common.hpp"
#include "kernels.hpp"
#include "radix.hpp"

#include <algorithm>

namespace socket_lsh {
namespace {

constexpr int kFilterThreads = 256;   // histogram kernel
constexpr int kSelectThreads = 256;   // filter kernel (4 waves, one sub-list each)
constexpr int kRefineThreads = 1024;  // refine kernel (one block per row)
constexpr int kMaxSubLists = 256;     // per row, filter path

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

// Element p (0 <= p < total) of the concatenated sub-lists of a row: from
// the LDS copy when the row's candidates fit there, else from memory.
struct RowLists {
  const uint2* glob;      // row's list area (sub-list s at s * sub_len)
  const uint2* cache;     // LDS copy of the first `cached` entries (order keys)
  uint32_t cached;
  const uint32_t* off;    // sub-list offsets in the concatenation (LDS)
  int subs;
  int64_t sub_len;
  bool score_bits;        // glob holds (score bits, index): map to order keys
  __device__ __forceinline__ uint2 from_memory(uint32_t p) const {
    int lo = 0, hi = subs - 1;  // last sub-list with off[s] <= p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= p) lo = mid; else hi = mid - 1;
    }
    uint2 e = glob[(int64_t)lo * sub_len + (p - off[lo])];
    if (score_bits) e.x = float_order_key(__uint_as_float(e.x));
    return e;
  }
  __device__ __forceinline__ uint2 operator()(uint32_t p) const {
    return p < cached ? cache[p] : from_memory(p);
  }
};

// Entry p of a row whose candidates are all in LDS.
struct CacheAt {
  const uint2* cache;
  __device__ __forceinline__ uint2 operator()(uint32_t p) const { return cache[p]; }
};

// Entry p of a full score row: (order key, p).
struct ScoreRowAt {
  const float* s;
  __device__ __forceinline__ uint2 operator()(uint32_t p) const {
    return make_uint2(float_order_key(s[p]), p);
  }
};

constexpr int kRefineCache = 16384;  // (u, index) pairs kept in LDS (128 KB)

struct RefineShared {
  uint32_t scratch[2 * (kRefineThreads / 64 + 1) + 4];
  uint32_t tmax[kRefineThreads / 64];
  uint32_t h[kHistBins];
  uint32_t off[kMaxSelectSubLists + 1];
  uint2 cache[kRefineCache];
};

// Offsets of the row's sub-lists in their concatenation, from their lengths
// (off[subs] = total). Each thread sums a run of consecutive sub-lists.
template <int NT>
__device__ uint32_t sublist_offsets(const uint32_t* cnt, int subs, uint32_t* off,
                                    uint32_t* scratch) {
  const int per = (subs + NT - 1) / NT;
  const int s0 = min(subs, (int)threadIdx.x * per), s1 = min(subs, s0 + per);
  uint32_t sum = 0;
  for (int s = s0; s < s1; ++s) sum += cnt[s];
  uint32_t total;
  uint32_t run = block_exclusive_scan<NT>(sum, scratch, &total);
  for (int s = s0; s < s1; ++s) {
    off[s] = run;
    run += cnt[s];
  }
  if (threadIdx.x == 0) off[subs] = total;
  __syncthreads();
  return total;
}

// The first min(total, kRefineCache) candidates into LDS: every thread
// fetches eight entries (located by binary search over the offsets) before
// storing any, so the loads overlap.
template <int NT>
__device__ void cache_candidates(RowLists& rl, uint2* cache, uint32_t total) {
  const uint32_t cached = min(total, (uint32_t)kRefineCache);
  constexpr int kBatch = 8;
  for (uint32_t base = 0; base < cached; base += kBatch * NT) {
    uint2 e[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const uint32_t p = base + i * NT + threadIdx.x;
      if (p < cached) e[i] = rl.from_memory(p);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const uint32_t p = base + i * NT + threadIdx.x;
      if (p < cached) cache[p] = e[i];
    }
  }
  __syncthreads();
  rl.cached = cached;
}

// Radix passes start_pass..2 (digits of 11, 11 and 10 bits) over the
// entries at(0 .. total) of one row with order key >= floor, which hold
// every key that can be among the kk best: `prefix` is the part of the
// order key fixed by the passes before start_pass and `need` the number of
// keys still to take under it. Then a final pass in entry (= index) order keeps every key
// above the threshold T and the first keys equal to T, and writes their
// indices at positions given by block scans: o[0 .. kk) ascending.
template <int NT, typename At>
__device__ void select_and_emit(const At& at, uint32_t total, uint32_t kk, int start_pass,
                                uint32_t prefix, uint32_t need, uint32_t floor,
                                RefineShared& sh, int32_t* o) {
  // the in-order loops below keep kB entries per lane in flight
  // (addresses clamped to the entries, results of the surplus ones unused)
  constexpr int kB = 8;
  uint32_t* res = sh.scratch + NT / 64 + 1;
  for (int pass = start_pass; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int pshift = pass == 1 ? 21 : 10;
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
    for (int i = threadIdx.x; i < kHistBins; i += NT) sh.h[i] = 0;
    __syncthreads();
    for (uint32_t p = threadIdx.x; p < total; p += NT) {
      const uint32_t u = at(p).x;
      if (u >= floor && (pass == 0 || (u >> pshift) == prefix))
        atomicAdd(&sh.h[(u >> shift) & dmask], 1u);
    }
    __syncthreads();
    find_threshold_bin<NT>(sh.h, need, sh.scratch, res);
    prefix = pass == 0 ? res[0] : (prefix << (pass == 2 ? 10 : 11)) | res[0];
    need -= res[1];
  }
  const uint32_t T = prefix;
  const uint32_t ties = need;  // keys equal to T still to take

  // final pass, in entry (= index) order: wave w takes a contiguous chunk
  // of entries, 64 per step. First every wave counts the keys above T and
  // equal to T in its chunk (ballots); then, from the counts of the waves
  // before it, it knows how many keys precede its chunk in the output and
  // how many of the ties are taken before it, and writes the indices it
  // keeps at consecutive positions (ballot, lane prefix).
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t chunk = (total + NW * 64 - 1) / (NW * 64) * 64;
  const uint32_t c0 = min(total, (uint32_t)wave * chunk), c1 = min(total, c0 + chunk);
  uint32_t n_gt = 0, n_eq = 0;  // wave-uniform
  for (uint32_t base = c0; base < c1; base += kB * 64) {  // wave-uniform
    uint32_t u[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) u[i] = at(min(base + i * 64 + lane, total - 1)).x;
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const bool valid = base + i * 64 + lane < c1;
      n_gt += (uint32_t)__popcll(__ballot(valid && u[i] > T));
      n_eq += (uint32_t)__popcll(__ballot(valid && u[i] == T));
    }
  }
  uint32_t* wc = sh.h;  // [NW][2]; the histogram is no longer read
  if (lane == 0) {
    wc[2 * wave] = n_gt;
    wc[2 * wave + 1] = n_eq;
  }
  __syncthreads();
  uint32_t before_gt = 0, before_eq = 0;
  for (int w = 0; w < wave; ++w) {
    before_gt += wc[2 * w];
    before_eq += wc[2 * w + 1];
  }
  uint32_t pos = before_gt + min(before_eq, ties);
  uint32_t eq_seen = before_eq;
  for (uint32_t base = c0; base < c1; base += kB * 64) {  // wave-uniform
    uint2 e[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) e[i] = at(min(base + i * 64 + lane, total - 1));
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const bool valid = base + i * 64 + lane < c1;
      const bool gt = valid && e[i].x > T, eq = valid && e[i].x == T;
      const uint64_t beq = __ballot(eq);
      const bool take = gt || (eq && eq_seen + lane_prefix(beq) < ties);
      const uint64_t bt = __ballot(take);
      const uint32_t slot = pos + lane_prefix(bt);
      if (take && slot < kk) o[slot] = (int32_t)e[i].y;
      pos += (uint32_t)__popcll(bt);
      eq_seen += (uint32_t)__popcll(beq);
    }
  }
}

// Refine of the score-row top-k. One block per row: passes 2 and 3 of the
// radix select over the row's candidates (all keys of first-digit bin b1 or
// above, in index order: the sub-lists back to back, copied into LDS as far
// as they fit) and the in-order emit of the kk selected indices.
__global__ __launch_bounds__(kRefineThreads) void topk_refine_kernel(
    int64_t n, int64_t kk, int subs, int64_t sub_len, const uint32_t* __restrict__ hist,
    const uint2* __restrict__ lists, const uint32_t* __restrict__ sub_cnt,
    int32_t* __restrict__ idx) {
  constexpr int NT = kRefineThreads;
  __shared__ RefineShared sh;
  const int row = blockIdx.x;
  uint32_t* res = sh.scratch + NT / 64 + 1;
  find_threshold_bin<NT>(hist + (int64_t)row * kHistBins, (uint32_t)kk, sh.scratch, res);
  const uint32_t b1 = res[0];
  const uint32_t need1 = (uint32_t)kk - res[1];
  const uint32_t total = sublist_offsets<NT>(sub_cnt + (int64_t)row * subs, subs, sh.off,
                                             sh.scratch);
  RowLists rl{lists + (int64_t)row * n, sh.cache, 0u, sh.off, subs, sub_len, false};
  cache_candidates<NT>(rl, sh.cache, total);
  if (total <= rl.cached)
    select_and_emit<NT>(CacheAt{sh.cache}, total, (uint32_t)kk, 1, b1, need1, 0u, sh,
                        idx + (int64_t)row * kk);
  else
    select_and_emit<NT>(rl, total, (uint32_t)kk, 1, b1, need1, 0u, sh, idx + (int64_t)row * kk);
}

// Selection of the decode path. One block per row. The score kernel's
// blocks each emitted (in index order) the keys whose score reached their
// own threshold; with T the largest of those thresholds, every key of the
// row with order key >= T is a candidate. When at least kk of them are, the
// kk best keys are among them: the candidates are copied into LDS as far as
// they fit and go through all three radix passes with floor T. Otherwise
// the block scores the whole row itself, with the score kernel's order of
// additions (hence the same float32 values), into the row's score buffer,
// and selects from that.
__global__ __launch_bounds__(kRefineThreads) void topk_select_kernel(SelectArgs a) {
  constexpr int NT = kRefineThreads;
  __shared__ RefineShared sh;
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t kk = (uint32_t)a.kk;
  int32_t* o = a.idx + (int64_t)row * a.kk;
  uint32_t* res = sh.scratch + NT / 64 + 1;
  // The first round of candidate copies (below) is requested before the
  // sub-list lengths are known: each wave loads the first kSpec * 64
  // entries of its kRound sub-lists (clamped to the row, unused beyond a
  // sub-list's length), in flight with the length and threshold loads.
  constexpr int kWaves = NT / 64, kRound = 8, kSpec = 1;
  const uint2* glob = a.lists + (int64_t)row * a.n;
  uint2 spec[kRound][kSpec];
#pragma unroll
  for (int k = 0; k < kRound; ++k) {
    const int sl = min(wave + k * kWaves, a.subs - 1);
#pragma unroll
    for (int t = 0; t < kSpec; ++t)
      spec[k][t] = glob[min((int64_t)sl * a.sub_len + t * 64 + lane, a.n - 1)];
  }
  // T (the largest block threshold of the row) and the sub-list lengths:
  // straight-line loads (segs <= subs / 16 <= NT, at most kMaxSelectSubLists
  // / NT lengths per thread, a run of consecutive sub-lists), all in flight
  // with the copies above
  constexpr int kPerMax = kMaxSelectSubLists / NT;
  const int per = (a.subs + NT - 1) / NT;
  const int s0 = min(a.subs, (int)threadIdx.x * per);
  const uint32_t* cnt = a.sub_cnt + (int64_t)row * a.subs;
  uint32_t cn[kPerMax];
#pragma unroll
  for (int q = 0; q < kPerMax; ++q) cn[q] = (q < per && s0 + q < a.subs) ? cnt[s0 + q] : 0u;
  uint32_t tmax = (int)threadIdx.x < a.segs ? a.thr[(int64_t)row * a.segs + threadIdx.x] : 0u;
  for (int i = threadIdx.x; i < kHistBins; i += NT) sh.h[i] = 0u;
  uint32_t total;
  {
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < kPerMax; ++q) sum += cn[q];
    uint32_t run = block_exclusive_scan<NT>(sum, sh.scratch, &total);
#pragma unroll
    for (int q = 0; q < kPerMax; ++q) {
      if (q < per && s0 + q < a.subs) sh.off[s0 + q] = run;
      run += cn[q];
    }
    if (threadIdx.x == 0) sh.off[a.subs] = total;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, m, 64));
  if (lane == 0) sh.tmax[wave] = tmax;
  __syncthreads();
  tmax = 0;
  for (int w = 0; w < NT / 64; ++w) tmax = max(tmax, sh.tmax[w]);

  // candidates into LDS (as far as they fit), counted into the first-digit
  // histogram when they reach T: each wave copies whole sub-lists, eight of
  // them per round, 64 entries of each per batch of loads
  RowLists rl{glob, sh.cache, 0u, sh.off, a.subs, a.sub_len, true};
  {
    const uint32_t cached = min(total, (uint32_t)kRefineCache);
    // the score kernel stores (score bits, index): cached as (order key, index)
    auto take = [&](const uint2& s, uint32_t p) {
      const uint2 e = make_uint2(float_order_key(__uint_as_float(s.x)), s.y);
      if (p < cached) sh.cache[p] = e;
      if (e.x >= tmax) atomicAdd(&sh.h[e.x >> 21], 1u);
    };
    for (int s0 = wave; s0 < a.subs; s0 += kWaves * kRound) {  // wave-uniform
      const bool first = s0 == wave;
      uint2 e[kRound][kSpec];
#pragma unroll
      for (int k = 0; k < kRound; ++k) {
        const int sl = s0 + k * kWaves;
#pragma unroll
        for (int t = 0; t < kSpec; ++t) {
          if (first) {
            e[k][t] = spec[k][t];
          } else if (sl < a.subs && (uint32_t)(t * 64 + lane) < sh.off[sl + 1] - sh.off[sl]) {
            e[k][t] = glob[(int64_t)sl * a.sub_len + t * 64 + lane];
          }
        }
      }
      // the next 64 entries of every sub-list that has them, all requested
      // before any is used
      uint2 x[kRound];
#pragma unroll
      for (int k = 0; k < kRound; ++k) {
        const int sl = s0 + k * kWaves;
        if (sl < a.subs && (uint32_t)(kSpec * 64 + lane) < sh.off[sl + 1] - sh.off[sl])
          x[k] = glob[(int64_t)sl * a.sub_len + kSpec * 64 + lane];
      }
#pragma unroll
      for (int k = 0; k < kRound; ++k) {
        const int sl = s0 + k * kWaves;
        if (sl >= a.subs) continue;
        const uint32_t o = sh.off[sl], c = sh.off[sl + 1] - o;
#pragma unroll
        for (int t = 0; t < kSpec; ++t)
          if ((uint32_t)(t * 64 + lane) < c) take(e[k][t], o + t * 64 + lane);
        if ((uint32_t)(kSpec * 64 + lane) < c) take(x[k], o + kSpec * 64 + lane);
        for (uint32_t i = (kSpec + 1) * 64 + lane; i < c; i += 64)
          take(glob[(int64_t)sl * a.sub_len + i], o + i);
      }
    }
    __syncthreads();
    rl.cached = cached;
  }
  find_threshold_bin<NT>(sh.h, kk, sh.scratch, res);
  const uint32_t b1 = res[0], above1 = res[1], n_above = res[2];
  if (n_above >= kk) {
    if (total <= rl.cached)
      select_and_emit<NT>(CacheAt{sh.cache}, total, kk, 1, b1, kk - above1, tmax, sh, o);
    else
      select_and_emit<NT>(rl, total, kk, 1, b1, kk - above1, tmax, sh, o);
    return;
  }

  const int G = a.Hq / a.Hkv;
  const int b = row / a.Hq, hq = row % a.Hq;
  const int bg = b * a.Hkv + hq / G, j = hq % G;
  const int L = a.L, nb = 1 << a.P;
  const float* tg = a.table + (int64_t)bg * nb * L * G + j;  // (u, l) at (u * L + l) * G
  float* tabs = reinterpret_cast<float*>(sh.cache);
  const bool lds_tab = (size_t)nb * L * sizeof(float) <= sizeof(sh.cache);
  if (lds_tab)
    for (int e = threadIdx.x; e < nb * L; e += NT) tabs[e] = tg[(int64_t)e * G];
  __syncthreads();
  float* srow = a.scores + (int64_t)row * a.n;
  const uint8_t* idh = a.ids + (int64_t)bg * a.stride * L;
  const float* vnh = a.vnorm + (int64_t)bg * a.stride;
  for (int64_t i = threadIdx.x; i < a.n; i += NT) {
    const int r = a.rotated ? (int)(i & 15) : 0;
    float acc = 0.f;
    for (int t = 0; t < L; ++t) {
      const int l = t + r < L ? t + r : t + r - L;
      const int u = idh[i * L + l] & (nb - 1);
      const float p = lds_tab ? tabs[u * L + l] : tg[(int64_t)(u * L + l) * G];
      acc = t == 0 ? p : acc + p;
    }
    srow[i] = vnh[i] * acc;
  }
  __syncthreads();
  select_and_emit<NT>(ScoreRowAt{srow}, (uint32_t)a.n, kk, 0, 0u, kk, 0u, sh, o);
}

// Filter. Block (seg, row) finds the bin b1 of the kk-th key from the
// row's first-digit histogram; each wave then streams its sub-segment of
// sub_len scores (64 lanes x 4 consecutive scores per step, eight steps of
// loads in flight) and appends the (u, index) pairs with digit >= b1 to its
// own sub-list in index order, the slots coming from four ballots and lane
// prefix counts (no block synchronisation after the threshold).
__global__ __launch_bounds__(kSelectThreads) void topk_filter_kernel(
    const float* __restrict__ scores, int64_t n, int64_t kk, int segs, int64_t sub_len,
    const uint32_t* __restrict__ hist, uint2* __restrict__ lists,
    uint32_t* __restrict__ sub_cnt, int vec4) {
  constexpr int kWaves = kSelectThreads / 64;
  __shared__ struct {
    uint32_t scratch[kSelectThreads / 64 + 1];
    uint32_t thr[3];
  } sh;
  const int row = blockIdx.y, seg = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int subs = segs * kWaves;

  find_threshold_bin<kSelectThreads>(hist + (int64_t)row * kHistBins, (uint32_t)kk,
                                     sh.scratch, sh.thr);
  const uint32_t b1 = sh.thr[0];

  const int sub = seg * kWaves + wave;
  const float* s = scores + (int64_t)row * n;
  const int64_t w0 = (int64_t)sub * sub_len;
  const int64_t w1 = min(n, w0 + sub_len);
  uint2* out = lists + (int64_t)row * n + w0;
  uint32_t count = 0;  // wave-uniform
  constexpr int kSteps = 8;  // 16-byte loads in flight per lane
  for (int64_t base = w0; base < w1; base += 256 * kSteps) {
    float v[kSteps][4];
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int64_t i0 = base + st * 256 + lane * 4;
      if (vec4 && i0 + 3 < w1) {
        const float4 x = *reinterpret_cast<const float4*>(s + i0);
        v[st][0] = x.x; v[st][1] = x.y; v[st][2] = x.z; v[st][3] = x.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[st][i] = i0 + i < w1 ? s[i0 + i] : 0.f;
      }
    }
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int64_t i0 = base + st * 256 + lane * 4;
      uint32_t u[4];
      uint64_t bal[4];
      uint32_t pos = count, tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u[i] = float_order_key(v[st][i]);
        bal[i] = __ballot(i0 + i < w1 && (u[i] >> 21) >= b1);
        pos += lane_prefix(bal[i]);  // entries of lower lanes, element i
        tot += (uint32_t)__popcll(bal[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if ((bal[i] >> lane) & 1ull) {
          out[pos] = make_uint2(u[i], (uint32_t)(i0 + i));
          ++pos;
        }
      }
      count += tot;
    }
  }
  if (lane == 0) sub_cnt[(int64_t)row * subs + sub] = count;
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
  // One sub-list per wave of sub_len scores (a multiple of 2048, one
  // iteration of a wave): about 4096 waves over the whole call, at most
  // kMaxSubLists sub-lists per row.
  constexpr int W = kSelectThreads / 64;
  int64_t sub_len = ((int64_t)rows * n + 4095) / 4096;
  sub_len = std::max<int64_t>(sub_len, (n + kMaxSubLists - 1) / kMaxSubLists);
  sub_len = std::max<int64_t>(2048, (sub_len + 2047) / 2048 * 2048);
  p.sub_len = sub_len;
  p.seg_len = sub_len * W;  // scores per block
  p.segs = (int)((n + p.seg_len - 1) / p.seg_len);
  if (p.segs < 1) p.segs = 1;
  p.subs = p.segs * W;
  size_t off = 0;
  p.hist_off = off;
  off += (size_t)rows * kHistBins * 4;
  p.zero_words = (int64_t)rows * kHistBins;
  off = align256(off);
  p.cnt_off = off;
  off = align256(off + (size_t)rows * p.subs * 4);
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

hipError_t launch_iota_rows(int32_t* idx, int rows, int64_t n, hipStream_t stream) {
  const int64_t total = (int64_t)rows * n;
  if (total == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 4096);
  launch_kernel(iota_rows_kernel, dim3(grid), dim3(256), 0, stream, idx, rows, n);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, const TopkPlan& plan, int32_t* idx,
                       void* ws, hipStream_t stream) {
  if (plan.rows == 0 || plan.n == 0) return hipSuccess;
  if (plan.kk == plan.n) return launch_iota_rows(idx, plan.rows, plan.n, stream);
  unsigned char* base = static_cast<unsigned char*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + plan.hist_off);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(base + plan.cnt_off);
  uint2* lists = reinterpret_cast<uint2*>(base + plan.list_off);
  hipError_t err = launch_zero_u32(hist, plan.zero_words, stream);
  if (err != hipSuccess) return err;
  launch_kernel(topk_hist_kernel, dim3(plan.segs, plan.rows), dim3(kFilterThreads), 0,
                stream, scores, plan.n, plan.seg_len, hist);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int vec4 = (plan.n % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0) ? 1 : 0;
  launch_kernel(topk_filter_kernel, dim3(plan.segs, plan.rows), dim3(kSelectThreads), 0,
                stream, scores, plan.n, plan.kk, plan.segs, plan.sub_len, hist, lists, cnt,
                vec4);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  launch_kernel(topk_refine_kernel, dim3(plan.rows), dim3(kRefineThreads), 0, stream, plan.n,
                plan.kk, plan.subs, plan.sub_len, hist, lists, cnt, idx);
  return hipGetLastError();
}

hipError_t launch_topk_select(const SelectArgs& a, int rows, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  launch_kernel(topk_select_kernel, dim3(rows), dim3(kRefineThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace socket_lsh
