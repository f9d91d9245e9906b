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
#include <type_traits>

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
// the LDS copy when the row's candidates fit there, else from memory. Each
// thread holds its own copy, whose cursor remembers the sub-list of the
// last position read from memory: the loops below read ascending positions
// per lane, so finding the next one's sub-list takes a step or two forward
// (a binary search only when a loop starts over).
struct RowLists {
  const uint2* glob;      // row's list area (sub-list s at sub_begin(s, ...))
  const uint2* cache;     // LDS copy of the first `cached` entries (order keys)
  uint32_t cached;
  const uint32_t* off;    // sub-list offsets in the concatenation (LDS)
  int subs;
  int64_t sub_len;
  bool score_bits;        // glob holds (score bits, index): map to order keys
  bool raw_cache;         // so does the LDS copy
  int skew0 = 0, skew1 = 0;
  mutable int cur = -1;   // sub-list of the last position read from memory
  // element index in glob of position p (moves the cursor)
  __device__ __forceinline__ int64_t locate(uint32_t p) const {
    if (cur < 0 || p < off[cur]) {
      int lo = 0, hi = subs - 1;  // last sub-list with off[s] <= p
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= p) lo = mid; else hi = mid - 1;
      }
      cur = lo;
    }
    while (cur + 1 < subs && off[cur + 1] <= p) ++cur;
    return sub_begin(cur, sub_len, skew0, skew1) + (p - off[cur]);
  }
  __device__ __forceinline__ uint2 from_memory(uint32_t p) const {
    uint2 e = glob[locate(p)];
    if (score_bits) e.x = float_order_key(__uint_as_float(e.x));
    return e;
  }
  __device__ __forceinline__ uint2 operator()(uint32_t p) const {
    if (p >= cached) return from_memory(p);
    uint2 e = cache[p];
    if (raw_cache) e.x = float_order_key(__uint_as_float(e.x));
    return e;
  }
  // positions below split() are in LDS; keys / entries requested per lane
  // at a time past it
  __device__ __forceinline__ uint32_t split() const { return cached; }
  static constexpr int kMemKeys = 8, kMemEntries = 8;
};

// Entry p of a row whose candidates are all in LDS.
struct CacheAt {
  const uint2* cache;
  __device__ __forceinline__ uint2 operator()(uint32_t p) const { return cache[p]; }
  __device__ __forceinline__ uint32_t split() const { return 0xffffffffu; }
  static constexpr int kMemKeys = 8, kMemEntries = 8;
};

// Entry p of a full score row: (order key, p).
struct ScoreRowAt {
  const float* s;
  __device__ __forceinline__ uint2 operator()(uint32_t p) const {
    return make_uint2(float_order_key(s[p]), p);
  }
  __device__ __forceinline__ uint32_t split() const { return 0u; }
  static constexpr int kMemKeys = 8, kMemEntries = 8;
};

constexpr int kRefineCache = 16384;  // (u, index) pairs kept in LDS (128 KB)

struct RefineShared {
  uint32_t scratch[2 * (kRefineThreads / 64 + 1) + 4];
  uint32_t tmax[kRefineThreads / 64];
  uint32_t wmax[kRefineThreads / 64];  // per-wave largest order keys of the candidates
  uint32_t cmax[kRefineThreads / 64];  // per-wave longest sub-lists
  uint32_t h[kHistBins];
  uint32_t off[kMaxSelectSubLists + 1];
  alignas(16) uint2 cache[kRefineCache];  // 16-byte direct-to-LDS copies
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
__device__ __forceinline__ void cache_candidates(RowLists& rl, uint2* cache, uint32_t total) {
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

// Entries each thread requests before it uses any, in the histogram passes
// below (entries read from memory then overlap instead of each waiting for
// the one before it).
constexpr int kPassBatch = 8;
// memory entries per lane and batch when a pass collects the keys in play
constexpr int kCollectMemKeys = 16;

// Wave w's share [c0, c1) of positions 0 .. total: contiguous runs of a
// multiple of 64 positions, in wave order (lane i reads positions c0 + i,
// c0 + 64 + i, ...: ascending per lane, consecutive across lanes).
struct WaveRun {
  uint32_t c0, c1;
  __device__ __forceinline__ WaveRun(uint32_t total, int nt) {
    const uint32_t nw = (uint32_t)nt / 64;
    const uint32_t chunk = (total + nw * 64 - 1) / (nw * 64) * 64;
    c0 = min(total, (threadIdx.x >> 6) * chunk);
    c1 = min(total, c0 + chunk);
  }
};

// Entries base + 64 i + lane (clamped to last), i < K, of any accessor.
template <int K, typename At>
__device__ __forceinline__ void read_run(const At& at, uint32_t base, uint32_t last,
                                         uint2 (&e)[K]) {
  const uint32_t lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < K; ++i) e[i] = at(min(base + i * 64 + lane, last));
}

// at[I ..] = element indices of positions base + 64 i + lane (clamped to
// last), written out one by one (constant indices: registers, although
// each step holds loops)
template <int I, int K>
__device__ __forceinline__ void locate_run(const RowLists& rl, uint32_t base, uint32_t last,
                                           int64_t (&at)[K]) {
  if constexpr (I < K) {
    at[I] = rl.locate(min(base + I * 64 + (threadIdx.x & 63), last));
    locate_run<I + 1, K>(rl, base, last, at);
  }
}

// The same for a row read partly from memory: when the whole run lies past
// the LDS copy (wave-uniform), every lane first finds the K addresses
// (cursor steps, LDS reads and branches) and only then issues the K loads,
// back to back, so that no branch separates them (at a branch the compiler
// would wait for every load in flight).
template <int K>
__device__ __forceinline__ void read_run(const RowLists& rl, uint32_t base, uint32_t last,
                                         uint2 (&e)[K]) {
  const uint32_t lane = threadIdx.x & 63;
  if (last < rl.cached) {  // wave-uniform: the whole run is in the LDS copy
#pragma unroll
    for (int i = 0; i < K; ++i) e[i] = rl.cache[min(base + i * 64 + lane, last)];
    if (rl.raw_cache) {
#pragma unroll
      for (int i = 0; i < K; ++i) e[i].x = float_order_key(__uint_as_float(e[i].x));
    }
    return;
  }
  if (base < rl.cached) {  // wave-uniform: the run starts in the LDS copy
#pragma unroll
    for (int i = 0; i < K; ++i) e[i] = rl(min(base + i * 64 + lane, last));
    return;
  }
  int64_t at[K];
  locate_run<0, K>(rl, base, last, at);
#pragma unroll
  for (int i = 0; i < K; ++i) e[i] = rl.glob[at[i]];
  if (rl.score_bits) {
#pragma unroll
    for (int i = 0; i < K; ++i) e[i].x = float_order_key(__uint_as_float(e[i].x));
  }
}

// Entry p of a row whose candidates were gathered into one contiguous run
// of (order key, index) pairs: from the LDS copy of its first `cached`
// entries, else from the run in memory.
struct SpillAt {
  const uint2* cache;
  uint32_t cached;
  const uint2* glob;
  __device__ __forceinline__ uint2 operator()(uint32_t p) const {
    return p < cached ? cache[p] : glob[p];
  }
  __device__ __forceinline__ uint32_t split() const { return cached; }
  // plain addresses: deep batches (one round of requests per pass at 22
  // memory entries per lane)
  static constexpr int kMemKeys = 24, kMemEntries = 16;
};

// Runs that lie wholly past the LDS copy load straight from the gathered
// run (consecutive addresses across the lanes, no branch between loads).
template <int K>
__device__ __forceinline__ void read_run(const SpillAt& at, uint32_t base, uint32_t last,
                                         uint2 (&e)[K]) {
  const uint32_t lane = threadIdx.x & 63;
  if (base >= at.cached) {  // wave-uniform
#pragma unroll
    for (int i = 0; i < K; ++i) e[i] = at.glob[min(base + i * 64 + lane, last)];
    return;
  }
  if (last < at.cached) {  // wave-uniform: the whole run is in LDS
#pragma unroll
    for (int i = 0; i < K; ++i) e[i] = at.cache[min(base + i * 64 + lane, last)];
    return;
  }
#pragma unroll
  for (int i = 0; i < K; ++i) e[i] = at(min(base + i * 64 + lane, last));
}

// Order keys only (the histogram passes and the emit's counts).
template <int K, typename At>
__device__ __forceinline__ void read_keys(const At& at, uint32_t base, uint32_t last,
                                          uint32_t (&u)[K]) {
  uint2 e[K];
  read_run(at, base, last, e);
#pragma unroll
  for (int i = 0; i < K; ++i) u[i] = e[i].x;
}

template <int K>
__device__ __forceinline__ void read_keys(const SpillAt& at, uint32_t base, uint32_t last,
                                          uint32_t (&u)[K]) {
  const uint32_t lane = threadIdx.x & 63;
  if (base >= at.cached) {  // wave-uniform: one dword of each entry
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(at.glob);
#pragma unroll
    for (int i = 0; i < K; ++i) u[i] = kw[2 * (size_t)min(base + i * 64 + lane, last)];
    return;
  }
  if (last < at.cached) {  // wave-uniform: the whole run is in LDS
#pragma unroll
    for (int i = 0; i < K; ++i) u[i] = at.cache[min(base + i * 64 + lane, last)].x;
    return;
  }
#pragma unroll
  for (int i = 0; i < K; ++i) u[i] = at(min(base + i * 64 + lane, last)).x;
}

// f(u, valid) for the order keys of positions [c0, c1), K per lane at a
// time (lane i: c0 + i, c0 + 64 + i, ...; valid is false for the padding
// of the last step).
template <int K, typename At, typename F>
__device__ __forceinline__ void for_keys(At at, uint32_t c0, uint32_t c1, F& f) {
  const uint32_t lane = threadIdx.x & 63;
  for (uint32_t base = c0; base < c1; base += K * 64) {  // wave-uniform
    uint32_t u[K];
    read_keys(at, base, c1 - 1, u);
#pragma unroll
    for (int i = 0; i < K; ++i) f(u[i], base + i * 64 + lane < c1);
  }
}

// f(u, valid) for the order key of every position in [0, total), in no
// particular order: each wave takes an equal contiguous share of the
// positions in LDS (below at.split()) and of those read from memory, so
// that every wave has memory requests in flight.
template <int NT, typename At, typename F>
__device__ __forceinline__ void for_all_keys(At at, uint32_t total, F&& f) {
  const uint32_t mid = min(at.split(), total);
  const WaveRun r0(mid, NT), r1(total - mid, NT);
  for_keys<kPassBatch>(at, r0.c0, r0.c1, f);
  for_keys<At::kMemKeys>(at, mid + r1.c0, mid + r1.c1, f);
}

// Row r's gather region: uint2 entries [start, start + cap) inside the
// bytes of float32 row r of an [rows][n] buffer, the start rounded up to 16
// bytes (so that each row's region lies within its own score row).
struct SpillRow {
  int64_t start;
  uint32_t cap;
};
__device__ __forceinline__ SpillRow spill_row(int64_t n, int row) {
  const int64_t w0 = (int64_t)row * n;  // float32 words
  const int64_t start = (w0 + 3) / 4 * 2, end = (w0 + n) / 2;
  return SpillRow{start, (uint32_t)(end > start ? end - start : 0)};
}

// Radix passes start_pass..2 (digits of 11, 11 and 10 bits) over the
// entries at(0 .. total) of one row with order key >= floor, which hold
// every key that can be among the kk best: `prefix` is the part of the
// order key fixed by the passes before start_pass and `need` the number of
// keys still to take under it. Then a final pass in entry (= index) order keeps every key
// above the threshold T and the first keys equal to T, and writes their
// indices at positions given by block scans: o[0 .. kk) ascending.
template <int NT, typename At>
__device__ __forceinline__ void emit_in_order(At at, uint32_t total, uint32_t kk, uint32_t T,
                                              uint32_t ties, RefineShared& sh, int32_t* o,
                                              bool counted = false);

template <int NT, typename At>
__device__ __forceinline__ void select_and_emit(At at, uint32_t total, uint32_t kk, int start_pass,
                                uint32_t prefix, uint32_t need, uint32_t floor,
                                RefineShared& sh, int32_t* o) {
  uint32_t* res = sh.scratch + NT / 64 + 1;
  for (int pass = start_pass; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int pshift = pass == 1 ? 21 : 10;
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
    for (int i = threadIdx.x; i < kHistBins; i += NT) sh.h[i] = 0;
    __syncthreads();
    for_all_keys<NT>(at, total, [&](uint32_t u, bool valid) {
      if (valid && u >= floor && (pass == 0 || (u >> pshift) == prefix))
        atomicAdd(&sh.h[(u >> shift) & dmask], 1u);
    });
    __syncthreads();
    find_threshold_bin<NT>(sh.h, need, sh.scratch, res);
    prefix = pass == 0 ? res[0] : (prefix << (pass == 2 ? 10 : 11)) | res[0];
    need -= res[1];
  }
  // keys above T = prefix, and the first `need` keys equal to it
  emit_in_order<NT>(at, total, kk, prefix, need, sh, o);
}

// The kk best entries among at(0 .. total) whose order keys lie in
// [lo, hi] (entries below lo are never among them; none is above hi),
// emitted in entry order; false (nothing written) when fewer than kk
// entries reach lo. Radix passes of up to 11 bits on x = u - lo, from the
// top bit of hi - lo down: the digits spread over the range the
// candidates actually span, so few keys share a histogram bin. A pass
// stops the search early when the bin holding the kk-th key is taken whole.
template <int NT, typename At>
__device__ __forceinline__ bool select_range_and_emit(At at, uint32_t total, uint32_t kk, uint32_t lo,
                                      uint32_t hi, RefineShared& sh, int32_t* o) {
  uint32_t* res = sh.scratch + NT / 64 + 1;
  int top = hi > lo ? 32 - __clz(hi - lo) : 0;  // bits of x still undecided
  const int nbits = top;
  uint32_t prefix = 0, need = kk;  // x >> top == prefix for the keys still in play
  bool whole = false, first = true;
  // Rows gathered into a run partly in memory: after the first pass the
  // keys still in play (those of the bin holding the kk-th key, counted
  // exactly by that pass) are collected into the sub-list offsets' LDS,
  // which such rows no longer read, so the later passes read no memory.
  // Each collected key is stored as its x below bit ct (the bits above are
  // cp, the same for all of them) tagged with its wave's chunk (bits 21..:
  // 2 * wave + 0 for the LDS part, + 1 for the memory part), and each wave
  // counts the keys of its chunks above the bin, so that the emit needs no
  // counting pass of its own.
  const uint32_t* ck = nullptr;  // block-uniform
  uint32_t nck = 0, cp = 0;
  int ct = 0;
  do {  // block-uniform; at least one pass, which counts the entries reaching lo
    const int db = min(11, top), shift = top - db;
    const uint32_t dmask = (1u << db) - 1u;
    for (int i = threadIdx.x; i < kHistBins; i += NT) sh.h[i] = 0;
    __syncthreads();
    auto count = [&](uint32_t u, bool valid) {
      if (!valid || u < lo) return;
      const uint32_t x = u - lo;
      if (top < nbits && (x >> top) != prefix) return;
      atomicAdd(&sh.h[(x >> shift) & dmask], 1u);
    };
    if (ck != nullptr) {
      for (uint32_t p = threadIdx.x; p < nck; p += NT)
        count(lo + ((cp << ct) | (ck[p] & ((1u << ct) - 1u))), true);
    } else {
      for_all_keys<NT>(at, total, count);
    }
    __syncthreads();
    find_threshold_bin<NT>(sh.h, need, sh.scratch, res);
    if (first && res[2] < kk) return false;
    first = false;
    const uint32_t bin = res[0], in_bin = sh.h[bin];
    prefix = (prefix << db) | bin;
    need -= res[1];
    top = shift;
    __syncthreads();  // every thread has read the bin before the next pass clears it
    if (in_bin == need) {
      whole = true;
      break;
    }
    if constexpr (std::is_same<At, SpillAt>::value) {
      if (ck == nullptr && top > 0 && total > at.split() && in_bin <= kMaxSelectSubLists + 1) {
        uint32_t* keys = sh.off;
        uint32_t* n_in = sh.scratch + 2 * (NT / 64 + 1);
        if (threadIdx.x == 0) *n_in = 0u;
        __syncthreads();
        const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const uint32_t low = (1u << top) - 1u;  // top <= 21 after the first pass
        uint32_t tag = 2u * wave, above = 0u;    // wave-uniform
        auto put = [&](uint32_t u, bool valid) {
          const uint32_t x = u - lo;
          const bool in = valid && u >= lo;
          const bool keep = in && (x >> top) == prefix;
          above += (uint32_t)__popcll(__ballot(in && (x >> top) > prefix));
          const uint64_t b = __ballot(keep);
          if (b != 0) {  // wave-uniform
            uint32_t base = 0u;
            if (lane == 0) base = atomicAdd(n_in, (uint32_t)__popcll(b));
            base = (uint32_t)__shfl((int)base, 0, 64);
            if (keep) keys[base + lane_prefix(b)] = (tag << 21) | (x & low);
          }
        };
        // each wave's chunk of the LDS part and of the memory part, as the
        // emit takes them (fewer memory loads per batch than the passes:
        // the slot bookkeeping needs registers too)
        const uint32_t mid = min(at.split(), total);
        const WaveRun r0(mid, NT), r1(total - mid, NT);
        for_keys<kPassBatch>(at, r0.c0, r0.c1, put);
        if (lane == 0) sh.tmax[wave] = above;
        tag += 1u;
        above = 0u;
        for_keys<kCollectMemKeys>(at, mid + r1.c0, mid + r1.c1, put);
        if (lane == 0) sh.cmax[wave] = above;
        __syncthreads();  // the keys and counts have landed
        ck = keys;
        nck = in_bin;
        cp = prefix;
        ct = top;
      }
    }
  } while (top > 0);
  // whole: every key from the bin's lowest up; else top == 0 and prefix is
  // the kk-th key's x
  const uint32_t T = lo + (prefix << top), ties = whole ? 0xffffffffu : need;
  if (ck != nullptr) {
    // the emit's counts: each wave's keys above the collected bin, plus the
    // collected keys above and equal to T by the chunk they came from
    uint32_t* wc = sh.h;
    for (int i = threadIdx.x; i < 4 * (NT / 64); i += NT) wc[i] = 0u;
    __syncthreads();
    for (uint32_t p = threadIdx.x; p < nck; p += NT) {
      const uint32_t e = ck[p], u = lo + ((cp << ct) | (e & ((1u << ct) - 1u)));
      const uint32_t w = (e >> 21) >> 1, part = (e >> 21) & 1u;
      if (u > T) atomicAdd(&wc[4 * w + 2 * part], 1u);
      else if (u == T) atomicAdd(&wc[4 * w + 2 * part + 1], 1u);
    }
    __syncthreads();
    if (threadIdx.x < NT / 64) {
      wc[4 * threadIdx.x] += sh.tmax[threadIdx.x];
      wc[4 * threadIdx.x + 2] += sh.cmax[threadIdx.x];
    }
    __syncthreads();
  }
  emit_in_order<NT>(at, total, kk, T, ties, sh, o, ck != nullptr);
  return true;
}

// Writes the kept entries of positions [c0, c1), in order, at output
// positions from pos on: every key above T, and keys equal to T while
// fewer than `ties` of them come before (eq_seen counts those before c0).
// One ballot and a lane prefix count per 64 entries.
template <int K, typename At>
__device__ __forceinline__ void emit_run(At at, uint32_t c0, uint32_t c1, uint32_t kk,
                                         uint32_t T, uint32_t ties, uint32_t pos,
                                         uint32_t eq_seen, int32_t* o) {
  const uint32_t lane = threadIdx.x & 63;
  for (uint32_t base = c0; base < c1; base += K * 64) {  // wave-uniform
    uint2 e[K];
    read_run(at, base, c1 - 1, e);
#pragma unroll
    for (int i = 0; i < K; ++i) {
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

// Writes, in entry (= index) order, every key above T and the first `ties`
// keys equal to T (all of them when ties is larger than their count):
// o[0 .. kk) ascending. The positions fall into two parts, those in LDS
// and those read from memory (either may be empty), and each wave takes a
// contiguous chunk of each part. First every wave counts the keys above T
// and equal to T in its chunks (ballots); then, from the counts of the
// chunks before each of its own (all of the LDS part's chunks come before
// the memory part's), it knows how many keys precede the chunk in the
// output and how many of the ties are taken before it, and writes the
// indices it keeps at consecutive positions. counted: the counts are
// already in sh.h ([wave][gt in LDS part, eq, gt in memory part, eq]) and
// visible to the block.
template <int NT, typename At>
__device__ __forceinline__ void emit_in_order(At at, uint32_t total, uint32_t kk, uint32_t T,
                                              uint32_t ties, RefineShared& sh, int32_t* o,
                                              bool counted) {
  constexpr int NW = NT / 64;
  const int wave = threadIdx.x >> 6;
  const uint32_t mid = min(at.split(), total);
  const WaveRun r0(mid, NT), r1(total - mid, NT);
  const uint32_t b0 = mid + r1.c0, b1 = mid + r1.c1;
  uint32_t* wc = sh.h;  // [NW][4]; the histogram is no longer read
  if (!counted) {  // block-uniform
    uint32_t n_gt0 = 0, n_eq0 = 0, n_gt1 = 0, n_eq1 = 0;  // wave-uniform
    auto count0 = [&](uint32_t u, bool valid) {
      n_gt0 += (uint32_t)__popcll(__ballot(valid && u > T));
      n_eq0 += (uint32_t)__popcll(__ballot(valid && u == T));
    };
    auto count1 = [&](uint32_t u, bool valid) {
      n_gt1 += (uint32_t)__popcll(__ballot(valid && u > T));
      n_eq1 += (uint32_t)__popcll(__ballot(valid && u == T));
    };
    for_keys<kPassBatch>(at, r0.c0, r0.c1, count0);
    for_keys<At::kMemKeys>(at, b0, b1, count1);
    if ((threadIdx.x & 63) == 0) {
      wc[4 * wave] = n_gt0;
      wc[4 * wave + 1] = n_eq0;
      wc[4 * wave + 2] = n_gt1;
      wc[4 * wave + 3] = n_eq1;
    }
    __syncthreads();
  }
  uint32_t gt0 = 0, eq0 = 0, gt0_all = 0, eq0_all = 0, gt1 = 0, eq1 = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) {
      gt0 += wc[4 * w];
      eq0 += wc[4 * w + 1];
      gt1 += wc[4 * w + 2];
      eq1 += wc[4 * w + 3];
    }
    gt0_all += wc[4 * w];
    eq0_all += wc[4 * w + 1];
  }
  emit_run<kPassBatch>(at, r0.c0, r0.c1, kk, T, ties, gt0 + min(eq0, ties), eq0, o);
  eq1 += eq0_all;
  emit_run<At::kMemEntries>(at, b0, b1, kk, T, ties, gt0_all + gt1 + min(eq1, ties), eq1, o);
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

// The select kernel's copy of short sub-lists: entries each thread
// requests at a time.
constexpr int kShortBatch = 8;

constexpr int kGatherThreads = 1024;
constexpr int kGatherPerWave = 4;  // sub-lists per wave
constexpr int kGatherSubs = kGatherThreads / 64 * kGatherPerWave;  // per block

// Gather (rows with many candidates). Block (g, row) takes sub-lists
// [64 g, 64 g + 64) of the row, four per wave: the lengths of the sub-lists
// before them give their place in the row's concatenation, and each wave
// copies its sub-lists there, in the row's gather region, as (order key,
// index) pairs. The first 128 entries of all four are requested before any
// is stored (eight loads per lane in flight); longer sub-lists continue in
// a second loop. The block's largest order key goes to bmax. A row whose
// candidates would not fit its region is left alone (the select kernel
// then reads the sub-lists themselves).
__global__ __launch_bounds__(kGatherThreads) void topk_gather_kernel(SelectArgs a) {
  constexpr int NT = kGatherThreads, NW = NT / 64, Q = kGatherPerWave;
  __shared__ uint32_t red[3 * NW];
  __shared__ uint32_t bc[kGatherSubs];
  if (a.subs > kMaxSelectSubLists) return;  // as in the select kernel
  const int row = blockIdx.y, g = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s0 = g * kGatherSubs;
  const uint32_t* cnt = a.sub_cnt + (int64_t)row * a.subs;
  // lengths before the block's sub-lists, and of the whole row
  if (threadIdx.x < kGatherSubs) bc[threadIdx.x] = 0u;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int s = threadIdx.x; s < a.subs; s += NT) {
    const uint32_t c = cnt[s];
    all += c;
    if (s < s0) before += c;
    else if (s < s0 + kGatherSubs) bc[s - s0] = c;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    before += (uint32_t)__shfl_xor((int)before, m, 64);
    all += (uint32_t)__shfl_xor((int)all, m, 64);
  }
  if (lane == 0) {
    red[wave] = before;
    red[NW + wave] = all;
  }
  __syncthreads();
  before = 0;
  all = 0;
  for (int w = 0; w < NW; ++w) {
    before += red[w];
    all += red[NW + w];
  }
  const SpillRow sr = spill_row(a.n, row);
  if (all > sr.cap) return;  // block-uniform
  // the wave's sub-lists: lengths, sources, destinations (wave-uniform)
  uint32_t off = before;
  for (int i = 0; i < Q * wave; ++i) off += bc[i];
  uint32_t len[Q];
  const uint2* src[Q];
  uint2* dst[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int sl = Q * wave + q;
    len[q] = bc[sl];  // 0 past the row's last sub-list
    // (an empty sub-list may start past the row's end, e.g. in the last,
    // partial segment: its slot stands in for it, read but not used)
    src[q] = a.lists + (int64_t)row * a.n +
             (len[q] > 0 ? sub_begin(s0 + sl, a.sub_len, a.skew0, a.skew1) : 0);
    dst[q] = a.spill + sr.start + off;
    off += len[q];
  }
  uint32_t umax = 0;
  {
    uint2 e[Q][2];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        e[q][i] = src[q][min((uint32_t)(i * 64 + lane), max(len[q], 1u) - 1)];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t j = i * 64 + lane;
        const uint32_t u = float_order_key(__uint_as_float(e[q][i].x));
        if (j < len[q]) {
          dst[q][j] = make_uint2(u, e[q][i].y);
          umax = max(umax, u);
        }
      }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    constexpr int kB = 4;
    for (uint32_t j0 = 128; j0 < len[q]; j0 += kB * 64) {  // wave-uniform
      uint2 e[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i) e[i] = src[q][min(j0 + i * 64 + lane, len[q] - 1)];
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        const uint32_t j = j0 + i * 64 + lane;
        const uint32_t u = float_order_key(__uint_as_float(e[i].x));
        if (j < len[q]) {
          dst[q][j] = make_uint2(u, e[i].y);
          umax = max(umax, u);
        }
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) umax = max(umax, (uint32_t)__shfl_xor((int)umax, m, 64));
  if (lane == 0) red[2 * NW + wave] = umax;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 0; w < NW; ++w) umax = max(umax, red[2 * NW + w]);
    a.bmax[(int64_t)row * gridDim.x + g] = umax;
  }
}

// Selection of the decode path. One block per row. The score kernel's
// blocks each emitted (in index order) the keys whose score reached their
// own threshold; with T the largest of those thresholds, every key of the
// row with order key >= T is a candidate. When at least kk of them are, the
// kk best keys are among them: the candidates are copied into LDS as far as
// they fit and go through the radix passes with floor T. Otherwise the
// block scores the whole row itself, with the score kernel's order of
// additions (hence the same float32 values), into the row's score buffer,
// and selects from that.
//
// Two dependent rounds of memory requests: the sub-list lengths and the
// block thresholds, then the candidates themselves, copied by
// direct-to-LDS loads (one dword per lane, so any entry offset will do)
// straight to their place in the concatenation. A row the gather kernel
// copied into one contiguous run (already order keys, its largest key
// known) is copied from there instead, 16 bytes per lane, and the entries
// past the LDS copy are read from that run. A row of short sub-lists that
// fits LDS is copied by plain loads, a few threads per sub-list.
__global__ __launch_bounds__(kRefineThreads) void topk_select_kernel(SelectArgs a) {
  constexpr int NT = kRefineThreads;
  __shared__ RefineShared sh;
  const int row = blockIdx.x;
  // the host never launches more sub-lists than the offsets hold; a row
  // that would have more is left alone rather than read out of bounds
  if (a.subs > kMaxSelectSubLists) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kWaves = NT / 64;
  const uint32_t kk = (uint32_t)a.kk;
  int32_t* o = a.idx + (int64_t)row * a.kk;
  const uint2* glob = a.lists + (int64_t)row * a.n;
  // T (the largest block threshold of the row) and the sub-list lengths:
  // straight-line loads (segs <= subs / 16 <= NT, at most
  // kMaxSelectSubLists / NT lengths per thread, a run of consecutive
  // sub-lists)
  constexpr int kPerMax = kMaxSelectSubLists / NT;
  const int per = (a.subs + NT - 1) / NT;
  const int s0 = min(a.subs, (int)threadIdx.x * per);
  const uint32_t* cnt = a.sub_cnt + (int64_t)row * a.subs;
  uint32_t cn[kPerMax];
#pragma unroll
  for (int q = 0; q < kPerMax; ++q) cn[q] = (q < per && s0 + q < a.subs) ? cnt[s0 + q] : 0u;
  uint32_t tmax = (int)threadIdx.x < a.segs ? a.thr[(int64_t)row * a.segs + threadIdx.x] : 0u;
  // gathered rows: the largest order key of each gather block
  const int gw = (a.subs + kGatherSubs - 1) / kGatherSubs;
  uint32_t gmax = a.spill && (int)threadIdx.x < gw ? a.bmax[(int64_t)row * gw + threadIdx.x] : 0u;
  uint32_t total, cmax = 0;  // cmax: the longest sub-list
  {
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < kPerMax; ++q) {
      sum += cn[q];
      cmax = max(cmax, cn[q]);
    }
    uint32_t run = block_exclusive_scan<NT>(sum, sh.scratch, &total);
#pragma unroll
    for (int q = 0; q < kPerMax; ++q) {
      if (q < per && s0 + q < a.subs) sh.off[s0 + q] = run;
      run += cn[q];
    }
    if (threadIdx.x == 0) sh.off[a.subs] = total;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, m, 64));
    gmax = max(gmax, (uint32_t)__shfl_xor((int)gmax, m, 64));
    cmax = max(cmax, (uint32_t)__shfl_xor((int)cmax, m, 64));
  }
  if (lane == 0) {
    sh.tmax[wave] = tmax;
    sh.wmax[wave] = gmax;
    sh.cmax[wave] = cmax;
  }
  __syncthreads();
  tmax = 0;
  gmax = 0;
  cmax = 0;
  for (int w = 0; w < kWaves; ++w) {
    tmax = max(tmax, sh.tmax[w]);
    gmax = max(gmax, sh.wmax[w]);
    cmax = max(cmax, sh.cmax[w]);
  }
  // (no key of a finite score has an order key below 1)
  const uint32_t floor = max(tmax, 1u);
  // the gather kernel copied the row's candidates when they fit its region
  const SpillRow sr = spill_row(a.n, row);
  const bool gathered = a.spill != nullptr && total <= sr.cap;  // block-uniform
  const uint32_t cached = min(total, (uint32_t)kRefineCache);
  unsigned char* cache_bytes = reinterpret_cast<unsigned char*>(sh.cache);
  const RowLists rl{glob,      sh.cache, cached, sh.off,  a.subs,
                    a.sub_len, true,     false,  a.skew0, a.skew1};
  const int tps = a.subs <= NT ? NT / a.subs : 1;  // threads per sub-list (short lists)
  uint32_t umax = 0;
  if (gathered) {
    // the first `cached` entries of the contiguous run into LDS, 16 bytes
    // (two entries) per lane and load; an odd last entry by one thread
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.spill + sr.start);
    const uint32_t pairs = cached / 2;
    for (uint32_t c0 = (uint32_t)wave * 64; c0 < pairs; c0 += NT) {  // wave-uniform
      if (c0 + lane < pairs)
        __builtin_amdgcn_global_load_lds(
            src + 4 * (size_t)(c0 + lane),
            (__attribute__((address_space(3))) void*)(cache_bytes + (size_t)c0 * 16), 16, 0, 0);
    }
    if ((cached & 1u) && threadIdx.x == 0) sh.cache[cached - 1] = a.spill[sr.start + cached - 1];
    __syncthreads();  // the copies have landed
    umax = gmax;
  } else if (total <= cached && cmax <= (uint32_t)tps * kShortBatch * 2) {
    // Short sub-lists (at most two requests per thread): tps threads per
    // sub-list copy it with plain loads, thread r of a sub-list taking
    // entries r, r + tps, ..., kShortBatch requested at a time, converted
    // to order keys on the way (no direct-to-LDS load per sub-list, no
    // conversion sweep).
    for (int t = threadIdx.x; t < a.subs * tps; t += NT) {
      const int sl = t / tps, r = t - sl * tps;
      const uint32_t o0 = sh.off[sl], n = sh.off[sl + 1] - o0;
      const uint2* src = glob + sub_begin(sl, a.sub_len, a.skew0, a.skew1);
      for (uint32_t j0 = r; j0 < n; j0 += tps * kShortBatch) {
        uint2 e[kShortBatch];
#pragma unroll
        for (int i = 0; i < kShortBatch; ++i) e[i] = src[min(j0 + i * tps, n - 1)];
#pragma unroll
        for (int i = 0; i < kShortBatch; ++i) {
          const uint32_t j = j0 + i * tps;
          const uint32_t u = float_order_key(__uint_as_float(e[i].x));
          if (j < n) {
            sh.cache[o0 + j] = make_uint2(u, e[i].y);
            umax = max(umax, u);
          }
        }
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) umax = max(umax, (uint32_t)__shfl_xor((int)umax, m, 64));
    if (lane == 0) sh.wmax[wave] = umax;
    __syncthreads();  // also completes the copy
    umax = 0;
    for (int w = 0; w < kWaves; ++w) umax = max(umax, sh.wmax[w]);
  } else {
    // The first `cached` entries of the concatenation into LDS: wave w
    // copies the run of sub-lists [w * spw, (w + 1) * spw), 32 entries (64
    // dwords) per load, lane i taking dword i. The run's offsets are read
    // once (one per lane) and handed to the issuing loop through lane reads.
    const int spw = (a.subs + kWaves - 1) / kWaves;
    const int sb = min(a.subs, wave * spw), se = min(a.subs, sb + spw);
    for (int k0 = sb; k0 < se; k0 += 63) {  // wave-uniform
      // lane i: the offset of sub-list k0 + i (i <= 63: its end too)
      const uint32_t offv = sh.off[min(k0 + lane, a.subs)];
      const int nk = min(63, se - k0);
      for (int k = 0; k < nk; ++k) {  // wave-uniform
        const uint32_t o0 = (uint32_t)__builtin_amdgcn_readlane((int)offv, k);
        if (o0 >= cached) break;  // offsets ascend
        const uint32_t o1 = min((uint32_t)__builtin_amdgcn_readlane((int)offv, k + 1), cached);
        const uint32_t dws = 2u * (o1 - o0);
        const uint32_t* src =
            reinterpret_cast<const uint32_t*>(glob + sub_begin(k0 + k, a.sub_len, a.skew0,
                                                                 a.skew1));
        for (uint32_t d0 = 0; d0 < dws; d0 += 64) {  // wave-uniform
          if (d0 + lane < dws)
            __builtin_amdgcn_global_load_lds(
                src + d0 + lane,
                (__attribute__((address_space(3))) void*)(cache_bytes +
                                                          ((size_t)o0 * 2 + d0) * 4),
                4, 0, 0);
        }
      }
    }
    __syncthreads();  // the copies have landed
    // score bits to order keys in place, and the largest order key of the
    // row (the entries beyond the LDS copy read from memory)
    for (uint32_t base = threadIdx.x; base < cached; base += kPassBatch * NT) {
      uint32_t uu[kPassBatch];
#pragma unroll
      for (int i = 0; i < kPassBatch; ++i)
        uu[i] = base + i * NT < cached ? sh.cache[base + i * NT].x : 0u;
#pragma unroll
      for (int i = 0; i < kPassBatch; ++i) {
        if (base + i * NT >= cached) break;
        const uint32_t u = float_order_key(__uint_as_float(uu[i]));
        sh.cache[base + i * NT].x = u;
        umax = max(umax, u);
      }
    }
    {
      // the entries past the LDS copy, wave-contiguous runs of positions
      const WaveRun mr(total - cached, NT);
      for (uint32_t base = cached + mr.c0; base < cached + mr.c1; base += kPassBatch * 64) {
        uint2 ee[kPassBatch];
        read_run(rl, base, cached + mr.c1 - 1, ee);
#pragma unroll
        for (int i = 0; i < kPassBatch; ++i) umax = max(umax, ee[i].x);
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) umax = max(umax, (uint32_t)__shfl_xor((int)umax, m, 64));
    if (lane == 0) sh.wmax[wave] = umax;
    __syncthreads();  // also completes the conversion
    umax = 0;
    for (int w = 0; w < kWaves; ++w) umax = max(umax, sh.wmax[w]);
  }
  if (umax >= floor) {
    bool done;
    if (total <= cached)
      done = select_range_and_emit<NT>(CacheAt{sh.cache}, total, kk, floor, umax, sh, o);
    else if (gathered)
      done = select_range_and_emit<NT>(SpillAt{sh.cache, cached, a.spill + sr.start}, total, kk,
                                       floor, umax, sh, o);
    else
      done = select_range_and_emit<NT>(rl, total, kk, floor, umax, sh, o);
    if (done) return;
  }

  const int G = a.Hq / a.Hkv;
  const int b = row / a.Hq, hq = row % a.Hq;
  const int bg = b * a.Hkv + hq / G, j = hq % G;
  const int64_t hg = bg / a.id_div;  // the KV head whose ids the row reads
  const int L = a.L, nb = 1 << a.P;
  const float* tg = a.table + (int64_t)bg * nb * L * G + j;  // (u, l) at (u * L + l) * G
  float* tabs = reinterpret_cast<float*>(sh.cache);
  const bool lds_tab = (size_t)nb * L * sizeof(float) <= sizeof(sh.cache);
  if (lds_tab)
    for (int e = threadIdx.x; e < nb * L; e += NT) tabs[e] = tg[(int64_t)e * G];
  __syncthreads();
  float* srow = a.scores + (int64_t)row * a.n;
  const uint8_t* idh = a.ids + hg * a.stride * L;
  const float* vnh = a.vnorm + hg * a.stride;
  // kKeys keys per thread at a time, their ids kTabs tables at a time: all
  // kKeys * kTabs id bytes are requested before any is looked up
  constexpr int kKeys = 4, kTabs = 8;
  for (int64_t i0 = threadIdx.x; i0 < a.n; i0 += (int64_t)NT * kKeys) {
    int64_t ik[kKeys];
    int rk[kKeys];
    float acc[kKeys], vk[kKeys];
#pragma unroll
    for (int k = 0; k < kKeys; ++k) {
      ik[k] = min(i0 + (int64_t)k * NT, a.n - 1);
      rk[k] = a.rotated ? (int)(ik[k] & 15) : 0;
      acc[k] = 0.f;
      vk[k] = vnh[ik[k]];
    }
    for (int t0 = 0; t0 < L; t0 += kTabs) {
      int lk[kKeys][kTabs], uk[kKeys][kTabs];
#pragma unroll
      for (int k = 0; k < kKeys; ++k)
#pragma unroll
        for (int q = 0; q < kTabs; ++q) {
          // the score kernel's order of additions
          const int t = min(t0 + q, L - 1), r = rk[k];
          lk[k][q] = a.region ? (t & ~15) | ((t + r) & 15) : (t + r < L ? t + r : t + r - L);
          uk[k][q] = idh[ik[k] * L + lk[k][q]];
        }
#pragma unroll
      for (int k = 0; k < kKeys; ++k)
#pragma unroll
        for (int q = 0; q < kTabs; ++q) {
          if (t0 + q >= L) break;
          const int u = uk[k][q] & (nb - 1), l = lk[k][q];
          const float p = lds_tab ? tabs[u * L + l] : tg[(int64_t)(u * L + l) * G];
          acc[k] = t0 + q == 0 ? p : acc[k] + p;
        }
    }
#pragma unroll
    for (int k = 0; k < kKeys; ++k)
      if (i0 + (int64_t)k * NT < a.n) srow[ik[k]] = vk[k] * acc[k];
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

int select_gather_blocks(int subs, int64_t kk) {
  // a row's candidates number about 2 to 4 kk: gather them when they would
  // overflow the select kernel's LDS copy
  return 3 * kk > kRefineCache ? (subs + kGatherSubs - 1) / kGatherSubs : 0;
}

hipError_t launch_topk_select(const SelectArgs& a, int rows, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  SelectArgs b = a;
  const int gw = b.spill && b.bmax ? select_gather_blocks(b.subs, b.kk) : 0;
  if (gw == 0) {
    b.spill = nullptr;
  } else {
    launch_kernel(topk_gather_kernel, dim3(gw, rows), dim3(kGatherThreads), 0, stream, b);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  launch_kernel(topk_select_kernel, dim3(rows), dim3(kRefineThreads), 0, stream, b);
  return hipGetLastError();
}

}  // namespace socket_lsh
