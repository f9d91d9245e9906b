// Soft collision scores.
//
// Step 3 of the soft-LSH mechanism of SOCKET (page "Resumen Técnico: SOCKET -
// Estimador de Núcleo de Colisión Suave para Atención Escasa", section
// "Mecanismo Central: LSH Suave", item 3; German page "SOCKET: SOft Collision
// Kernel EsTimator for Sparse Attention", Kernmechanismus, Bewertung): every
// key is scored by the probability mass the query puts on the key's own
// bucket, summed over the L tables and weighted by the key's value norm.
//
// One block owns one (batch, KV head) and a contiguous range of keys. It
// gets that head's probability table [2^P][L][G] (float32) into LDS, either
// copied from the table kernel's output or, in the decode path for bf16
// queries with P = 8, built in place with the table kernel's arithmetic
// (bit for bit the same table; no table kernel runs), then streams the
// bucket-id rows (L bytes per key, coalesced across lanes) and the value
// norms from HBM, two steps ahead in registers (the first steps are
// requested while the table is being set up). Each id byte is looked up
// once for the whole GQA group: the G probabilities of the group sit in one
// 16-byte LDS slot.
//
// Bank spread: with the [u][l][G] layout and L a multiple of 16, the LDS bank
// group of slot (u, l) depends only on l mod 16 (64 banks of 4 bytes,
// 16-byte slots). Lane i walks the tables in the rotated order l = (t + n)
// mod L for its key n (n mod 16 = i mod 16), so the 16 lanes the LDS serves
// together hit 16 different bank groups whatever buckets the keys fall in.
// The rotation is applied to the id bytes in registers once per key; the
// slot offset of step t is a per-lane base (two candidates, before and
// after the wrap) plus a compile-time immediate. The L probabilities are
// summed in float32 in that fixed order and multiplied by the value norm.
//
// Candidate emission (the decode path). Every wave owns a contiguous range
// of the block's keys. The block scores the first step of every wave (up to
// 2048 keys, spread over its range) and sets, per query row, a threshold
// that about m of those scores reach, with m = m0 + 6 sqrt(m0) + 8 for the
// m0 = kk * n_b / n keys of the row's top kk expected among its n_b sampled
// keys (exactly kk when the block sees the whole row): the sampled order
// keys are counted in 256 bins by their top 8 bits, then those of the bin
// holding the m-th largest in 256 bins by the next 8 bits, and the
// threshold is the lower edge of the sub-bin at which the count from the
// top reaches m. Thresholds are stored per block and row; every key of the
// block whose score's order key reaches the threshold is appended as
// (score bits, index) to its wave's sub-list, in index order (the test is
// one float compare against the smallest float with that key; slots from one
// ballot and lane prefix counts per row and step, no atomics), and the
// sub-list lengths are stored at the end. The selection that follows is
// exact whatever these thresholds are: it takes the largest
// threshold of the row, checks that at least kk candidates reach it (every
// key that does is a candidate) and otherwise scores the whole row.

#include "common.hpp"
#include "kernels.hpp"
#include "radix.hpp"
#include "soft_prob.hpp"

#include <algorithm>

namespace socket_lsh {
namespace {

// 16 waves per block, the most one CU holds at <= 128 VGPRs; the rotated
// path keeps two steps of ids and norms in flight per thread.
constexpr int kScoreThreads = 1024;
constexpr int kScoreWaves = kScoreThreads / 64;
constexpr int kPrefetch = 2;
// keys per wave are a multiple of one rotated-path iteration
constexpr int kWaveStep = 64 * kPrefetch;
// keeps every per-thread byte offset of a segment (key * L, L <= 1024) in 31 bits
constexpr int64_t kMaxSeg = 1 << 20;
// block thresholds: 256 bins per query row and pass (bits 24..31 of the
// order key, then bits 16..23)
constexpr int kThrBins = 256;

// v_cndmask_b32 with an explicit lane mask: b where the lane's mask bit is
// set, a elsewhere. Written out so the compiler keeps one select per word
// instead of rewriting the rotation below as a dynamically indexed array.
__device__ __forceinline__ uint32_t select_lanes(uint32_t a, uint32_t b, uint64_t mask) {
  uint32_t out;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(out) : "v"(a), "v"(b), "s"(mask));
  return out;
}

// Rotate the NB-byte array held in NW 32-bit words left by r bytes
// (0 <= r < 16): byte i of the result is byte (i + r) mod NB of the input.
// Two word-select stages (by one word in the lanes set in by1: bit 2 of r,
// by two words in those set in by2: bit 3 of r) and one byte funnel shift
// per word.
template <int NW>
__device__ __forceinline__ void rotate_bytes(uint32_t (&w)[NW], uint64_t by1, uint64_t by2,
                                             int rb) {
  uint32_t t[NW], v[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) t[i] = select_lanes(w[i], w[(i + 1) % NW], by1);
#pragma unroll
  for (int i = 0; i < NW; ++i) v[i] = select_lanes(t[i], t[(i + 2) % NW], by2);
#pragma unroll
  for (int i = 0; i < NW; ++i)
    w[i] = __builtin_amdgcn_alignbyte(v[(i + 1) % NW], v[i], rb);
}

// Ties the next ids to the running sums (empty asm, no instruction): every
// sum is complete before this point, and the words w[k0 .. k1) cannot be
// used, hence no lookup of theirs issued, before it. Keeps the compiler
// from issuing all lookups of a key at once and from deferring the sums,
// either of which holds one register per looked-up float.
template <int G, int LW>
__device__ __forceinline__ void fence_chunk(float (&acc)[G], uint32_t (&w)[LW], int k0,
                                            int k1) {
#pragma unroll
  for (int j = 0; j < G; ++j) asm volatile("" : "+v"(acc[j]), "+v"(w[k0]));
#pragma unroll
  for (int k = k0 + 1; k < k1; ++k) asm volatile("" : "+v"(w[k]) : "v"(w[k0]));
}

// Buffer resource over `bytes` bytes from base (raw, untyped accesses):
// loads and stores through it take a 32-bit lane offset and no 64-bit
// address arithmetic. base must be the same in every lane.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

template <int G>
__device__ __forceinline__ void lds_load_group(const float* p, float (&o)[G]) {
  if constexpr (G == 4) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
  } else if constexpr (G == 8) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    const float4 y = *reinterpret_cast<const float4*>(p + 4);
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    o[4] = y.x; o[5] = y.y; o[6] = y.z; o[7] = y.w;
  } else if constexpr (G == 2) {
    const float2 x = *reinterpret_cast<const float2*>(p);
    o[0] = x.x; o[1] = x.y;
  } else {
    o[0] = p[0];
  }
}

// Block -> (batch*KV head, key segment), placing all segments of one head
// on the same XCD (blocks are dealt to the 8 XCDs round-robin) so the head's
// probability table is fetched into that XCD's L2 once.
__device__ __forceinline__ bool score_block_coords(int bhkv, int segs, int& bg,
                                                   int& seg) {
  const int total = bhkv * segs;
  const int per_xcd = (total + 7) / 8;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int li = xcd * per_xcd + slot;
  if (slot >= per_xcd || li >= total) return false;
  bg = li / segs;
  seg = li % segs;
  return true;
}

// Region layout of the LDS table (G = 4 query heads, the rotated scorer;
// P = 8 with L = 16 or 32, P = 6 with L = 64): tables 16c .. 16c + 15 form
// region c at byte 2^P * 256 * c; in it, bucket u takes 256 bytes, 16 table
// slots of 16 bytes (the 4 heads' probabilities). Float index of entry
// (u, l, j):
__host__ __device__ __forceinline__ int region_index(int u, int l, int j, int P) {
  return (l >> 4) * (64 << P) + u * 64 + (l & 15) * 4 + j;
}

// The table of batch*KV head bg into LDS ([u][l][j], or the region layout
// when REGION). The blocks of one head run on one XCD and read the same
// table: each starts at its own round of 16 KB (start_round) so that they do
// not all ask the same L2 lines at once.
template <int G, bool REGION>
__device__ __forceinline__ void stage_table(float* tab, const float* table, int bg,
                                            int L, int P, int start_round, int id_div,
                                            int table_G) {
  const int tsize = (1 << P) * L * G;
  if (table_G != G) {
    // a pack of G of the table_G heads of each slot (socket_score on a
    // group table too large for one block): element by element
    const float* src = table + (int64_t)(bg / id_div) * ((int64_t)tsize / G * table_G) +
                       (bg % id_div) * G;
    for (int i = threadIdx.x; i < tsize; i += blockDim.x) {
      const int u = i / (L * G), l = (i / G) % L, j = i % G;
      tab[REGION ? region_index(u, l, j, P) : i] = src[(int64_t)(i / G) * table_G + j];
    }
  } else if (REGION) {
    // direct-to-LDS loads into the region layout: LDS slot f (16 bytes) of
    // region c, bucket u, table 16c + s holds table slot u * L + 16c + s
    const float4* src = reinterpret_cast<const float4*>(table + (int64_t)bg * tsize);
    const int n4 = tsize / 4;
    const int lane = threadIdx.x & 63;
    const int per_round = (int)blockDim.x;
    const int rounds = (n4 + per_round - 1) / per_round;
    const int first = start_round % rounds;
    for (int k = 0; k < rounds; ++k) {
      const int rr = k + first < rounds ? k + first : k + first - rounds;
      const int f0 = rr * per_round + (int)(threadIdx.x & ~63);  // wave-uniform
      const int f = f0 + lane;
      if (f0 < n4 && f < n4) {
        const int c = f >> (P + 4), u = (f >> 4) & ((1 << P) - 1), sl = f & 15;
        __builtin_amdgcn_global_load_lds(
            (const void*)(src + u * L + c * 16 + sl),
            (__attribute__((address_space(3))) void*)(tab + (size_t)f0 * 4), 16, 0, 0);
      }
    }
  } else if (tsize % 4 == 0) {  // every head's table then starts 16-byte aligned
    // direct-to-LDS loads: 64 lanes x 16 bytes per instruction into
    // consecutive LDS, no registers held, all in flight at once
    const float4* src = reinterpret_cast<const float4*>(table + (int64_t)bg * tsize);
    const int n4 = tsize / 4;
    const int lane = threadIdx.x & 63;
    const int per_round = (int)blockDim.x;
    const int rounds = (n4 + per_round - 1) / per_round;
    const int first = start_round % rounds;
    for (int k = 0; k < rounds; ++k) {
      const int rr = k + first < rounds ? k + first : k + first - rounds;
      const int w0 = rr * per_round + (int)(threadIdx.x & ~63);  // wave-uniform
      if (w0 < n4 && w0 + lane < n4)
        __builtin_amdgcn_global_load_lds(
            (const void*)(src + w0 + lane),
            (__attribute__((address_space(3))) void*)(tab + (size_t)w0 * 4), 16, 0, 0);
    }
  } else {
    for (int i = threadIdx.x; i < tsize; i += blockDim.x)
      tab[i] = table[(int64_t)bg * tsize + i];
  }
}


struct ScoreArgs {
  const float* table;  // [bhkv / id_div][2^P][L][table_G]
  const uint8_t* ids;
  const float* vnorm;
  int Hq, Hkv, bhkv, L, P, segs;  // Hkv, bhkv: virtual KV heads (score_pack)
  int id_div;          // virtual head bg reads the ids and norms of head bg / id_div
  int table_G;         // heads per table slot (G, or the whole group when packing a stage call)
  int64_t n_keys, stride, seg_len;
  int skew0, skew1;    // unequal wave shares (sub_begin)
  float* scores;       // [rows][n_keys] or null
  // candidate emission (decode path)
  int select;
  int64_t kk;
  uint32_t* thr;       // [rows][segs] block thresholds (order keys)
  uint2* lists;        // [rows][n_keys]; sub-list s at sub_begin(s, seg_len / 16, ...)
  uint32_t* sub_cnt;   // [rows][segs * 16]
  // table built in the kernel: bf16 query rows [B][Hq][d] and hyperplanes
  // [d][L*P]; the built table is also stored to table_out when given
  const uint16_t* Qb;
  const uint16_t* Rb;
  int d;
  double two_over_tau;
  float* table_out;
};

// LDS layout of a score block: the table, (when the block builds the
// table) the bit weights of the build, the per-row threshold histograms.
__host__ __device__ inline size_t score_table_region(int L, int P, int G) {
  return align256(((size_t)1 << P) * L * G * sizeof(float));
}
__host__ __device__ inline size_t build_weights_region(int L, int P, int G) {
  return align256((size_t)2 * P * L * G * sizeof(double));
}

// Scores of one key for the G heads of a group: written out (sk: the key's
// slot in the first head's score row, or null) and/or appended to the
// wave's sub-lists. Called by every lane of the wave (valid marks the lanes
// that hold a key); cnt is the wave's running count per head.
template <int G>
__device__ __forceinline__ void emit_scores(const ScoreArgs& a, const float (&acc)[G], float vn,
                                            bool valid, uint32_t key, float* sk,
                                            const __amdgpu_buffer_rsrc_t (&lst)[G],
                                            const float (&thrf)[G], uint32_t (&cnt)[G]) {
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float sc = vn * acc[j];
    if (sk != nullptr && valid) sk[(int64_t)j * a.n_keys] = sc;
    if (a.select) {
      const bool pass = valid && sc >= thrf[j];
      const uint64_t bal = __ballot(pass);
      if (pass) {
        const u32x2_t e = {__float_as_uint(sc), key};
        __builtin_amdgcn_raw_buffer_store_b64(e, lst[j], (cnt[j] + lane_prefix(bal)) * 8u, 0, 0);
      }
      cnt[j] += (uint32_t)__popcll(bal);
    }
  }
}

// The smallest float whose order key (float_order_key) is at least thr, so
// that for finite s, s >= threshold_float(thr) exactly when
// float_order_key(s) >= thr (-0 and +0 share one key); -inf for thr = 0.
__device__ __forceinline__ float threshold_float(uint32_t thr) {
  if (thr == 0u) return -INFINITY;
  return __uint_as_float(thr >= 0x80000000u ? (thr & 0x7fffffffu) : ~thr);
}

// Keys [n0 + wb, n0 + we) of this block's segment belong to this wave:
// its share (wlen keys, unequal across the waves) of the segment, cut at
// the row's end.
struct WaveRange {
  int64_t n0;
  int cnt, wlen, wb, we;
  int sub_len, skew0, skew1;
  __device__ WaveRange(const ScoreArgs& a, int seg)
      : sub_len((int)(a.seg_len / kScoreWaves)), skew0(a.skew0), skew1(a.skew1) {
    n0 = seg * a.seg_len;
    cnt = (int)(min(a.n_keys, n0 + a.seg_len) - n0);
    // (wave-uniform: in scalar registers, as the sub-list buffers need)
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    wb = (int)sub_begin(w, sub_len, skew0, skew1);
    wlen = (int)sub_size(w, sub_len, skew0, skew1);
    we = min(cnt, wb + wlen);
  }
  // keys in the first step (kWaveStep keys) of every wave of the block
  __device__ int first_step_keys() const {
    int n = 0;
    for (int w = 0; w < kScoreWaves; ++w) {
      const int b = (int)sub_begin(w, sub_len, skew0, skew1);
      const int e = min(cnt, b + (int)sub_size(w, sub_len, skew0, skew1));
      n += max(0, min(kWaveStep, e - b));
    }
    return n;
  }
};

// Rank m (1 = largest) of a block threshold among n_b sampled keys of a row
// of n keys of which kk are selected; 0: every key passes.
__device__ inline uint32_t threshold_rank(int64_t kk, int64_t n, int n_b) {
  if (n_b >= n) return (uint32_t)kk;
  const double m0 = (double)kk * n_b / (double)n;
  const double m = ceil(m0 + 6.0 * sqrt(m0) + 8.0);
  return m >= (double)n_b ? 0u : (uint32_t)m;
}

// Lane i ^ 8, i ^ 16, i ^ 32 of a double (DPP row rotation by 8, lane swaps).
__device__ __forceinline__ double xor8_f64(double v) { return dpp_f64<0x128>(v); }
__device__ __forceinline__ double xor16_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = xor16_u32((uint32_t)u), hi = xor16_u32((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, (hi << 32) | lo);
}
__device__ __forceinline__ double xor32_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = xor32_u32((uint32_t)u), hi = xor32_u32((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, (hi << 32) | lo);
}

// Builds the probability table of KV head bg in LDS (layout [u][l][j], as
// the table kernel writes it) from the G query rows of the group and the
// hyperplanes (bf16, P = 8, d = 64 or 128), with the table kernel's
// arithmetic, so both tables are equal bit for bit:
//  * z = q . r in float64: with P = 8 the 8 columns of table l are its 8
//    bits; the lane of (rows, table l, part) takes 16 consecutive
//    coordinates (fma from 0 ascending) for R_ROWS query rows at once, so
//    each hyperplane value is converted to float64 once per R_ROWS rows; the
//    d/16 parts sit 8 lanes apart (lane = part * 8 + table within a block of
//    8 tables: the 8 lanes of a part read 128 consecutive bytes of a
//    hyperplane row) and are added pairwise in the table kernel's order
//    ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7)) by a reduce-scatter
//    that leaves bit `part` (and part + 4 when d = 64) in each lane;
//  * the bit weights (bit_weights), then per (table, row) the bit-group
//    products (bits 0-2, 3-5, 6-7; each multiplied in ascending bit order
//    from 1.0) and p(u) = (A[u & 7] * B[(u >> 3) & 7]) * C[u >> 6] rounded
//    to float32.
// The hyperplanes and the query rows are staged in the table's LDS
// (direct-to-LDS loads); before() is called once they have landed (the
// barrier that waits for them waits for every load the wave has issued)
// and requests the caller's first ids and norms, which then arrive while
// the table is being built. The weights go to w as [bit][l][j]
// (2 * 8 * L * G doubles).
// The entries are written by 8 threads per (table, row) pair p = l * G + j:
// thread c takes buckets 32c .. 32c + 31, for which it needs the 8 products
// of group A, 4 of group B and 1 of group C. Contains __syncthreads().
template <int G, bool REGION, class Before>
__device__ __forceinline__ void build_table(float* tab, double* w, const ScoreArgs& a, int bg,
                                            Before before) {
  constexpr int P = 8;
  constexpr int R_ROWS = G >= 2 ? 2 : 1;  // query rows per lane
  const int L = a.L, d = a.d;
  const int C = L * P;
  const int parts = d / 16;  // 4 or 8
  const int pairs = L * G;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double* w1 = w;
  double* w0 = w + (size_t)P * pairs;
  const size_t r_bytes = (size_t)16 * d * L;
  unsigned char* stage = reinterpret_cast<unsigned char*>(tab);

  // hyperplanes, then the group's query rows, into LDS: 1 KB per wave and
  // instruction
  {
    const uint4* rsrc = reinterpret_cast<const uint4*>(a.Rb);
    const uint4* qsrc =
        reinterpret_cast<const uint4*>(a.Qb + ((int64_t)b * a.Hq + (int64_t)g * G) * d);
    const int nr = (int)(r_bytes / 16), nq = G * d / 8;
    for (int i0 = wave * 64; i0 < nr + nq; i0 += kScoreThreads) {  // wave-uniform
      const int i = i0 + lane;
      if (i < nr + nq)
        __builtin_amdgcn_global_load_lds(
            (const void*)(i < nr ? rsrc + i : qsrc + (i - nr)),
            (__attribute__((address_space(3))) void*)(stage + (size_t)i0 * 16), 16, 0, 0);
    }
  }
  __syncthreads();
  before();

  // units of (R_ROWS rows, 8 tables), 8 * parts lanes each
  const int lanes_per_unit = 8 * parts;
  const int per_wave = 64 / lanes_per_unit;  // 1 or 2
  const int row_groups = G / R_ROWS;
  const int units = row_groups * (L / 8);
  const int part = (lane / 8) % parts, li = lane % 8;
  const uint16_t* qs = reinterpret_cast<const uint16_t*>(stage + r_bytes);
  for (int u0 = wave * per_wave; u0 < units; u0 += kScoreWaves * per_wave) {  // wave-uniform
    const int unit = u0 + lane / lanes_per_unit;
    const bool active = unit < units;
    const int uc = min(unit, units - 1);
    const int jr = uc % row_groups, l = (uc / row_groups) * 8 + li;
    const unsigned char* rcol = stage + (size_t)l * 16;
    double acc[R_ROWS][8];
#pragma unroll
    for (int jj = 0; jj < R_ROWS; ++jj)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[jj][e] = 0.0;
    const unsigned char* rp = rcol + (size_t)part * 16 * C * 2;
    uint4 rnext = *reinterpret_cast<const uint4*>(rp);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      uint4 qh[R_ROWS];  // 8 coordinates of each row
#pragma unroll
      for (int jj = 0; jj < R_ROWS; ++jj)
        qh[jj] = *reinterpret_cast<const uint4*>(qs + (jr * R_ROWS + jj) * d + part * 16 + kh * 8);
#pragma unroll
      for (int k8 = 0; k8 < 8; ++k8) {
        const int k = kh * 8 + k8;
        // one hyperplane row ahead in flight, no more (registers)
        const uint4 rw = rnext;
        if (k + 1 < 16) rnext = *reinterpret_cast<const uint4*>(rp + (size_t)(k + 1) * C * 2);
        float rv[8];
        unpack8_bf16(rw, rv);
        double rd[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) rd[e] = (double)rv[e];
#pragma unroll
        for (int jj = 0; jj < R_ROWS; ++jj) {
          const uint32_t wq = k8 < 2 ? qh[jj].x : k8 < 4 ? qh[jj].y : k8 < 6 ? qh[jj].z : qh[jj].w;
          const double qk = (double)__uint_as_float((k8 & 1) ? (wq & 0xffff0000u) : (wq << 16));
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[jj][e] = fma(qk, rd[e], acc[jj][e]);
        }
        // every row's sums of this coordinate are complete here (keeps the
        // compiler from splitting the rows into passes that park rd)
#pragma unroll
        for (int jj = 0; jj < R_ROWS; ++jj)
          asm volatile("" : "+v"(acc[jj][0]), "+v"(acc[jj][1]), "+v"(acc[jj][2]), "+v"(acc[jj][3]),
                       "+v"(acc[jj][4]), "+v"(acc[jj][5]), "+v"(acc[jj][6]), "+v"(acc[jj][7]));
      }
    }
    // reduce-scatter over the parts (lane bits 3, 4, 5 = part bits 0, 1, 2)
    const bool b0 = (part & 1) != 0, b1 = (part & 2) != 0, b2 = (part & 4) != 0;
#pragma unroll
    for (int jj = 0; jj < R_ROWS; ++jj) {
      double s1[4], s2[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double keep = b0 ? acc[jj][2 * i + 1] : acc[jj][2 * i];
        const double send = b0 ? acc[jj][2 * i] : acc[jj][2 * i + 1];
        s1[i] = keep + xor8_f64(send);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const double keep = b1 ? s1[2 * m + 1] : s1[2 * m];
        const double send = b1 ? s1[2 * m] : s1[2 * m + 1];
        s2[m] = keep + xor16_f64(send);
      }
      const int j = jr * R_ROWS + jj;
      if (parts == 8) {
        const double z = (b2 ? s2[1] : s2[0]) + xor32_f64(b2 ? s2[0] : s2[1]);
        double x1, x0;
        bit_weights(z, a.two_over_tau, x1, x0);
        if (active) {
          w1[part * pairs + l * G + j] = x1;
          w0[part * pairs + l * G + j] = x0;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          double x1, x0;
          bit_weights(s2[m], a.two_over_tau, x1, x0);
          if (active) {
            w1[(part + 4 * m) * pairs + l * G + j] = x1;
            w0[(part + 4 * m) * pairs + l * G + j] = x0;
          }
        }
      }
    }
  }
  __syncthreads();

  // table entries
  constexpr int kPairsPerPass = kScoreThreads / 8;
  for (int p0 = 0; p0 < pairs; p0 += kPairsPerPass) {  // block-uniform
    const int np = min(kPairsPerPass, pairs - p0);
    const int t = threadIdx.x;
    if (t < np * 8) {
      const int p = p0 + t % np, c = t / np;
      double v1[8], v0[8];
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        v1[bit] = w1[bit * pairs + p];
        v0[bit] = w0[bit * pairs + p];
      }
      double A[8], Bq[4];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        double v = 1.0;
        v *= (x & 1) ? v1[0] : v0[0];
        v *= (x & 2) ? v1[1] : v0[1];
        v *= (x & 4) ? v1[2] : v0[2];
        A[x] = v;
      }
      const bool hb = (c & 1) != 0;  // bit 5 of these buckets
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        double v = 1.0;
        v *= (x & 1) ? v1[3] : v0[3];
        v *= (x & 2) ? v1[4] : v0[4];
        v *= hb ? v1[5] : v0[5];
        Bq[x] = v;
      }
      const int cc = c >> 1;  // bits 6-7 of these buckets
      double Cv = 1.0;
      Cv *= (cc & 1) ? v1[6] : v0[6];
      Cv *= (cc & 2) ? v1[7] : v0[7];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float e = (float)((A[i & 7] * Bq[i >> 3]) * Cv);
        if constexpr (REGION)  // p = l * 4 + j: region p / 64, slot p % 64
          tab[(p >> 6) * 16384 + (c * 32 + i) * 64 + (p & 63)] = e;
        else
          tab[(c * 32 + i) * pairs + p] = e;
      }
    }
  }
}

// The block's share (segment seg of segs) of its head's table, from LDS to
// table_out.
template <int G, bool REGION>
__device__ __forceinline__ void store_table_share(const float* tab, const ScoreArgs& a, int bg,
                                                  int seg) {
  const int tsize = (1 << a.P) * a.L * G;
  const int n4 = tsize / 4;
  const int per = (n4 + a.segs - 1) / a.segs;
  const int s1 = min(n4, (seg + 1) * per);
  float4* dst = reinterpret_cast<float4*>(a.table_out + (int64_t)bg * tsize);
  const float4* src = reinterpret_cast<const float4*>(tab);
  for (int i = seg * per + (int)threadIdx.x; i < s1; i += kScoreThreads) {
    // slot i = u * L + l of the [u][l][j] layout the select kernel reads
    dst[i] = REGION ? src[region_index(i / a.L, i % a.L, 0, a.P) / 4] : src[i];
  }
}

// Per query row j of the group: an order key that at least m of the sampled
// order keys uk[q][j] (valid[q]) reach, and few more. The first pass counts
// the keys by their top 8 bits (sign and 7 exponent bits: bins of two
// octaves) and finds, from the top, the bin b1 at which the count reaches
// m; the second counts bits 16..23 of the keys in b1 (bins of 1/128 of an
// octave) and finds b2 the same way. The threshold is the lowest key of
// (b1, b2), or 0 when fewer than m keys are valid. Wave j searches row j's
// bins (4 bins per lane, DPP prefix sums). hist: 2 * G * kThrBins
// counters, zero on entry. Contains __syncthreads().
template <int G>
__device__ __forceinline__ void block_thresholds(const uint32_t (&uk)[kPrefetch][G],
                                                 const bool (&valid)[kPrefetch], uint32_t m,
                                                 uint32_t* hist, uint32_t (&thr)[G]) {
  static_assert(kThrBins == 4 * 64, "four bins per lane");
  const int lane = threadIdx.x & 63;
  uint32_t* h1 = hist;                  // [G][256] by bits 24..31
  uint32_t* h2 = hist + G * kThrBins;   // [G][256] by bits 16..23 within b1
#pragma unroll
  for (int q = 0; q < kPrefetch; ++q)
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (valid[q]) atomicAdd(&h1[j * kThrBins + (uk[q][j] >> 24)], 1u);
  __syncthreads();
  // bin (from the top) at which the running count reaches need; lane 0
  // holds the 4 highest bins. Returns kThrBins when the bins hold fewer.
  // the bin (from the top) at which the running count of a row's bins hr
  // reaches need, and the count before it (kThrBins, 0 when the bins hold
  // fewer); lane 0 holds the 4 highest bins. One wave per row.
  auto find = [&](const uint32_t* hr, uint32_t need, uint32_t& before) {
    const uint4 c4 = *reinterpret_cast<const uint4*>(hr + kThrBins - 4 - 4 * lane);
    const uint32_t cs[4] = {c4.w, c4.z, c4.y, c4.x};  // descending bins
    const uint32_t sum = c4.x + c4.y + c4.z + c4.w;
    uint32_t run = wave_inclusive_scan_dpp(sum) - sum;
    uint32_t b = kThrBins, bef = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (run < need && run + cs[i] >= need) {
        b = (uint32_t)(kThrBins - 1 - 4 * lane - i);
        bef = run;
      }
      run += cs[i];
    }
    const uint64_t hit = __ballot(b != kThrBins);
    const int src = hit ? __ffsll((unsigned long long)hit) - 1 : 0;
    before = hit ? (uint32_t)__builtin_amdgcn_readlane((int)bef, src) : 0u;
    return hit ? (uint32_t)__builtin_amdgcn_readlane((int)b, src) : (uint32_t)kThrBins;
  };
  // wave j < G searches row j and leaves its result in the row's first
  // bins, which no other wave reads
  const int wave = threadIdx.x >> 6;
  if (wave < G) {
    uint32_t before;
    const uint32_t b = find(h1 + wave * kThrBins, m, before);
    if (lane == 0) {
      h1[wave * kThrBins] = b;
      h1[wave * kThrBins + 1] = m - before;
    }
  }
  __syncthreads();
  uint32_t b1[G], need2[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    b1[j] = h1[j * kThrBins];
    need2[j] = h1[j * kThrBins + 1];
  }
#pragma unroll
  for (int q = 0; q < kPrefetch; ++q)
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (valid[q] && b1[j] < kThrBins && (uk[q][j] >> 24) == b1[j])
        atomicAdd(&h2[j * kThrBins + ((uk[q][j] >> 16) & 255u)], 1u);
  __syncthreads();
  if (wave < G) {
    uint32_t before;
    const uint32_t b1w = h1[wave * kThrBins];
    // b2 is found whenever b1 is: bin b1 holds the m-th key
    const uint32_t b2 = find(h2 + wave * kThrBins, h1[wave * kThrBins + 1], before);
    if (lane == 0) h2[wave * kThrBins] = b1w < kThrBins ? (b1w << 24) | (b2 << 16) : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) thr[j] = h2[j * kThrBins];
}

// The common body of the score kernels. Scorer: prefetch() requests the
// first step of ids and norms; score(q, i, acc, vn) scores key i (relative
// to n0) of slot q of a step and requests the key kWaveStep further on.
template <int G, bool BUILD, bool REGION, class Scorer>
__device__ void score_block(const ScoreArgs& a, int bg, int seg, float* tab, Scorer& sc,
                            const WaveRange& wr) {
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int lane = threadIdx.x & 63;
  unsigned char* lds = reinterpret_cast<unsigned char*>(tab);
  const size_t treg = score_table_region(a.L, a.P, G);
  uint32_t* hist = reinterpret_cast<uint32_t*>(
      lds + treg + (BUILD ? build_weights_region(a.L, a.P, G) : 0));
  float* sseg = a.scores ? a.scores + ((int64_t)b * a.Hq + (int64_t)g * G) * a.n_keys + wr.n0
                         : nullptr;

  if (a.select)
    for (int i = threadIdx.x; i < 2 * G * kThrBins; i += kScoreThreads) hist[i] = 0u;
  if constexpr (BUILD) {
    build_table<G, REGION>(tab, reinterpret_cast<double*>(lds + treg), a, bg,
                           [&] { sc.prefetch(); });
  } else {
    sc.prefetch();
    stage_table<G, REGION>(tab, a.table, bg, a.L, a.P, seg, a.id_div, a.table_G);
  }
  __syncthreads();
  if constexpr (BUILD)
    if (a.table_out) store_table_share<G, REGION>(tab, a, bg, seg);

  // first step of every wave: scored, then (decode) the block thresholds
  float acc[kPrefetch][G], vn[kPrefetch];
  bool valid[kPrefetch];
#pragma unroll
  for (int q = 0; q < kPrefetch; ++q) {
    const int i = wr.wb + q * 64 + lane;
    valid[q] = i < wr.we;
    sc.score(q, i, valid[q], acc[q], vn[q]);
  }
  uint32_t thr[G], nsel[G];
  float thrf[G];
  __amdgpu_buffer_rsrc_t lst[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    thr[j] = 0u;
    nsel[j] = 0u;
    lst[j] = raw_rsrc(nullptr, 0u);
  }
  if (a.select) {
    const uint32_t m = threshold_rank(a.kk, a.n_keys, wr.first_step_keys());
    if (m != 0) {
      uint32_t uk[kPrefetch][G];
#pragma unroll
      for (int q = 0; q < kPrefetch; ++q)
#pragma unroll
        for (int j = 0; j < G; ++j) uk[q][j] = float_order_key(vn[q] * acc[q][j]);
      block_thresholds<G>(uk, valid, m, hist, thr);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int64_t row = (int64_t)b * a.Hq + (int64_t)g * G + j;
      if (threadIdx.x == 0) a.thr[row * a.segs + seg] = thr[j];
      // the wave's sub-list as a buffer in scalar registers (the stores then
      // take a 32-bit lane offset); at most wlen entries
      const uint64_t base = reinterpret_cast<uint64_t>(a.lists + row * a.n_keys + wr.n0 + wr.wb);
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
      lst[j] = raw_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                        (uint32_t)wr.wlen * 8u);
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) thrf[j] = threshold_float(thr[j]);
#pragma unroll
  for (int q = 0; q < kPrefetch; ++q) {
    const int i = wr.wb + q * 64 + lane;
    emit_scores<G>(a, acc[q], vn[q], valid[q], (uint32_t)(wr.n0 + i), sseg ? sseg + i : nullptr,
                   lst, thrf, nsel);
  }
  for (int base = wr.wb + kWaveStep; base < wr.we; base += kWaveStep) {  // wave-uniform
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q) {
      const int i = base + q * 64 + lane;
      const bool ok = i < wr.we;
      float a_q[G], v_q;
      sc.score(q, i, ok, a_q, v_q);
      emit_scores<G>(a, a_q, v_q, ok, (uint32_t)(wr.n0 + i), sseg ? sseg + i : nullptr, lst,
                     thrf, nsel);
    }
  }
  if (a.select && lane == 0) {
    const int subs = a.segs * kScoreWaves;
    const int sub = seg * kScoreWaves + (int)(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int64_t row = (int64_t)b * a.Hq + (int64_t)g * G + j;
      a.sub_cnt[row * subs + sub] = nsel[j];
    }
  }
}

// Fast path scorer: L a multiple of 16 (LW = L/4 words of ids per key),
// 16-byte id rows, rotated table order.
template <int G, int LW>
struct RotScorer {
  static constexpr int L = LW * 4;
  static constexpr int kChunk = 64 / G;  // lookups per dependency step (a multiple of 4)
  // the kernels planned with two resident 1024-thread blocks per CU, which
  // must stay within 64 VGPRs (see plan_score)
  static constexpr bool kTwoPerCU = (G == 1 && LW <= 8) || (G <= 4 && LW <= 4);
  __amdgpu_buffer_rsrc_t idseg, vseg;  // the segment's id rows and norms
  const float* tab;
  int P, we, wb;
  uint4 pf[kPrefetch][LW / 4];
  float pf_vn[kPrefetch];
  int r, rb, base_nowrap, base_wrap;

  __device__ RotScorer(const ScoreArgs& a, int bg, const WaveRange& wr, const float* tab_)
      : tab(tab_), P(a.P), we(wr.we), wb(wr.wb) {
    // block-uniform bases of this segment (buffers: per-thread offsets stay
    // 32-bit, seg_len * L < 2^31 bytes)
    const int64_t hg = bg / a.id_div;  // the KV head whose ids this block reads
    idseg = raw_rsrc(a.ids + (hg * a.stride + wr.n0) * L, (uint32_t)wr.cnt * L);
    vseg = raw_rsrc(a.vnorm + hg * a.stride + wr.n0, (uint32_t)wr.cnt * 4u);
    // n0 + wb is a multiple of 16, so every key of this lane has the same
    // rotation r = key index mod 16 and the same two bases
    const int lane = threadIdx.x & 63;
    r = lane & 15;
    rb = r & 3;
    base_nowrap = r * G;      // slot offset of step t: t*G + base
    base_wrap = (r - L) * G;  // ... once t + r >= L
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q) {
      pf_vn[q] = 0.f;
#pragma unroll
      for (int k = 0; k < LW / 4; ++k) pf[q][k] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  __device__ __forceinline__ void load(int q, int i) {
#pragma unroll
    for (int k = 0; k < LW / 4; ++k) {
      const u32x4v_t x = __builtin_amdgcn_raw_buffer_load_b128(idseg, (uint32_t)i * L + k * 16, 0, 0);
      pf[q][k] = make_uint4(x.x, x.y, x.z, x.w);
    }
    pf_vn[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vseg, (uint32_t)i * 4u, 0, 0));
  }

  __device__ __forceinline__ void prefetch() {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q) {
      const int i = wb + q * 64 + lane;
      if (i < we) load(q, i);
    }
  }

  __device__ __forceinline__ void score(int q, int i, bool valid, float (&acc)[G], float& vn) {
    uint32_t w[LW];
#pragma unroll
    for (int k = 0; k < LW / 4; ++k) {
      w[4 * k] = pf[q][k].x; w[4 * k + 1] = pf[q][k].y;
      w[4 * k + 2] = pf[q][k].z; w[4 * k + 3] = pf[q][k].w;
    }
    // rotated before the next ids are requested into the same registers
    // (the rotation's results are fresh registers: no copies of the buffer)
    rotate_bytes<LW>(w, __ballot(r & 4), __ballot(r & 8), rb);
    vn = pf_vn[q];
    if (i + kWaveStep < we) load(q, i + kWaveStep);
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = 0.f;
    if (!valid) return;
    if constexpr (kTwoPerCU) {
      // batches of 4 floats, each requested whole before it is added (the
      // registers of two resident blocks per CU; their 32 waves keep the
      // LDS busy)
      constexpr int kB = G >= 4 ? 1 : 4 / G;
#pragma unroll
      for (int t0 = 0; t0 < L; t0 += kB) {
        float pr[kB][G];
#pragma unroll
        for (int s = 0; s < kB; ++s) {
          const int t = t0 + s;
          // P bits of byte t: ids are < 2^P, so this never leaves the table
          const uint32_t u = __builtin_amdgcn_ubfe(w[t >> 2], (t & 3) * 8, P);
          const int off = (t + 15 < L) ? base_nowrap : (t + r < L ? base_nowrap : base_wrap);
          lds_load_group<G>(tab + (int)u * (L * G) + off + t * G, pr[s]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < kB; ++s)
#pragma unroll
          for (int j = 0; j < G; ++j) acc[j] = t0 + s == 0 ? pr[s][j] : acc[j] + pr[s][j];
        // the next kChunk lookups wait for these sums: at most 64 floats
        // of lookups in flight per lane, which bounds the registers
        const int t = t0 + kB - 1;
        if ((t + 1) % kChunk == 0 && t + 1 < L)
          fence_chunk<G, LW>(acc, w, (t + 1) / 4, std::min(LW, (t + 1 + kChunk) / 4));
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    // Lookups in batches of kBatch (16 floats): batch b + 1 is requested
    // before batch b is added (left to itself the compiler issues each read
    // right before its add, one read in flight per wave); the sums stay in
    // table order.
    constexpr int kBatch = 16 / G, NB = L / kBatch;
    float pr[2][kBatch * G];
    auto request = [&](int b) {
#pragma unroll
      for (int s = 0; s < kBatch; ++s) {
        const int t = b * kBatch + s;
        // P bits of byte t: ids are < 2^P, so this never leaves the table
        const uint32_t u = __builtin_amdgcn_ubfe(w[t >> 2], (t & 3) * 8, P);
        const int off = (t + 15 < L) ? base_nowrap : (t + r < L ? base_nowrap : base_wrap);
        lds_load_group<G>(tab + (int)u * (L * G) + off + t * G,
                          *reinterpret_cast<float(*)[G]>(&pr[b & 1][s * G]));
      }
    };
    request(0);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b + 1 < NB) request(b + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < kBatch; ++s)
#pragma unroll
        for (int j = 0; j < G; ++j)
          acc[j] = b + s == 0 ? pr[b & 1][s * G + j] : acc[j] + pr[b & 1][s * G + j];
      // the next kChunk lookups wait for these sums: at most 64 floats
      // of lookups in flight per lane, which bounds the registers
      const int t = b * kBatch + kBatch - 1;
      if ((t + 1) % kChunk == 0 && t + 1 < L)
        fence_chunk<G, LW>(acc, w, (t + 1) / 4, std::min(LW, (t + 1 + kChunk) / 4));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// Rotated scorer over the region layout (G = 4 query heads; P = 8 with
// L = 16 or 32, P = 6 with L = 64): lane key n walks the 16 tables of each
// region c in the order 16c + (t + r) mod 16, r = n mod 16 (the key's id
// row is rotated by r bytes within each 16-byte half), so the 16 lanes the
// LDS serves together hit 16 bank groups. One v_perm_b32 forms a lookup's
// LDS byte address 2^P * 256 * c + 256 u + 16 s: byte 1 the (rotated) id
// byte u, byte 0 the lane's slot s = (t + r) mod 16 times 16 from a
// per-lane constant; the region base is, for P = 8, byte 2 from another
// constant (65536 for region 1), for P = 6 the read's immediate offset
// (16384 c).
template <int LW, int P>
struct RegionScorer {
  static constexpr int G = 4;
  static constexpr int L = LW * 4;
  static constexpr int kChunk = 64 / G;  // lookups per dependency step
  static_assert((P == 8 && (LW == 4 || LW == 8)) || (P == 6 && LW == 16),
                "P = 8 with 16 or 32 tables, P = 6 with 64 tables");
  __amdgpu_buffer_rsrc_t idseg, vseg;
  const float* tab;
  int we, wb;
  uint4 pf[kPrefetch][LW / 4];
  float pf_vn[kPrefetch];
  int r, rb;
  uint32_t slot0[4];  // region 0: byte q of word k = slot of step 4k + q
  uint32_t slot1[8];  // region 1: bytes 0, 1 of word k = slots of steps 16 + 2k, + 1; bytes 2, 3 = 1

  __device__ RegionScorer(const ScoreArgs& a, int bg, const WaveRange& wr, const float* tab_)
      : tab(tab_), we(wr.we), wb(wr.wb) {
    const int64_t hg = bg / a.id_div;  // the KV head whose ids this block reads
    idseg = raw_rsrc(a.ids + (hg * a.stride + wr.n0) * L, (uint32_t)wr.cnt * L);
    vseg = raw_rsrc(a.vnorm + hg * a.stride + wr.n0, (uint32_t)wr.cnt * 4u);
    // n0 + wb is a multiple of 16: every key of this lane has r = lane mod 16
    const int lane = threadIdx.x & 63;
    r = lane & 15;
    rb = r & 3;
    auto slot = [&](int t) { return (uint32_t)(((t + r) & 15) << 4); };
#pragma unroll
    for (int k = 0; k < 4; ++k)
      slot0[k] = slot(4 * k) | slot(4 * k + 1) << 8 | slot(4 * k + 2) << 16 | slot(4 * k + 3) << 24;
#pragma unroll
    for (int k = 0; k < 8; ++k) slot1[k] = slot(2 * k) | slot(2 * k + 1) << 8 | 0x01010000u;
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q) {
      pf_vn[q] = 0.f;
#pragma unroll
      for (int k = 0; k < LW / 4; ++k) pf[q][k] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  __device__ __forceinline__ void load(int q, int i) {
#pragma unroll
    for (int k = 0; k < LW / 4; ++k) {
      const u32x4v_t x = __builtin_amdgcn_raw_buffer_load_b128(idseg, (uint32_t)i * L + k * 16, 0, 0);
      pf[q][k] = make_uint4(x.x, x.y, x.z, x.w);
    }
    pf_vn[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vseg, (uint32_t)i * 4u, 0, 0));
  }

  __device__ __forceinline__ void prefetch() {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q) {
      const int i = wb + q * 64 + lane;
      if (i < we) load(q, i);
    }
  }

  __device__ __forceinline__ void score(int q, int i, bool valid, float (&acc)[G], float& vn) {
    uint32_t w[LW];
    const uint64_t by1 = __ballot(r & 4), by2 = __ballot(r & 8);
#pragma unroll
    for (int k = 0; k < LW / 4; ++k) {  // each 16-byte half rotated by r
      uint32_t h[4] = {pf[q][k].x, pf[q][k].y, pf[q][k].z, pf[q][k].w};
      rotate_bytes<4>(h, by1, by2, rb);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[4 * k + e] = h[e];
    }
    vn = pf_vn[q];
    if (i + kWaveStep < we) load(q, i + kWaveStep);
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = 0.f;
    if (!valid) return;
    if constexpr (P < 8) {
      // P bits of every id byte: ids are < 2^P, so this never leaves the
      // region (as the other scorers, which take P bits)
#pragma unroll
      for (int k = 0; k < LW; ++k) w[k] &= 0x01010101u * ((1u << P) - 1u);
    }
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    // lookups in batches of kBatch, batch b + 1 requested before batch b is
    // added (as in RotScorer); the sums stay in table order
    constexpr int kBatch = 4, NB = L / kBatch;
    f32x4_t pr[2][kBatch];
    auto request = [&](int b) {
#pragma unroll
      for (int s = 0; s < kBatch; ++s) {
        const int t = b * kBatch + s;
        // byte selectors: 0-3 pick bytes of the slot word, 4-7 bytes of the
        // id word, 0x0c gives 0
        uint32_t addr;
        if (P < 8 || t < 16)
          addr = __builtin_amdgcn_perm(w[t >> 2], slot0[(t & 15) >> 2],
                                       0x0c0c0000u | ((4u + (t & 3)) << 8) | (uint32_t)(t & 3)) +
                 (P < 8 ? (uint32_t)(t >> 4) * (256u << P) : 0u);
        else
          addr = __builtin_amdgcn_perm(w[t >> 2], slot1[(t & 15) >> 1],
                                       0x0c020000u | ((4u + (t & 3)) << 8) | (uint32_t)(t & 1));
        // the table is the block's dynamic LDS, which starts at LDS address 0
        // (the kernel has no static LDS; the host checks it before launching
        // this scorer): addr is the slot's absolute LDS address
        pr[b & 1][s] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>(
            (uintptr_t)addr);
      }
    };
    request(0);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b + 1 < NB) request(b + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < kBatch; ++s) {
        const f32x4_t x = pr[b & 1][s];
        const float p4[G] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int j = 0; j < G; ++j) acc[j] = b + s == 0 ? p4[j] : acc[j] + p4[j];
      }
      const int t = b * kBatch + kBatch - 1;
      if ((t + 1) % kChunk == 0 && t + 1 < L)
        fence_chunk<G, LW>(acc, w, (t + 1) / 4, std::min(LW, (t + 1 + kChunk) / 4));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// General scorer: any L (byte loads of the ids, tables summed in order
// l = 0..L-1).
template <int G>
struct GenericScorer {
  const uint8_t* idseg;
  const float* vseg;
  const float* tab;
  int L, P;
  __device__ GenericScorer(const ScoreArgs& a, int bg, const WaveRange& wr, const float* tab_)
      : tab(tab_), L(a.L), P(a.P) {
    const int64_t hg = bg / a.id_div;
    idseg = a.ids + (hg * a.stride + wr.n0) * a.L;
    vseg = a.vnorm + hg * a.stride + wr.n0;
  }
  __device__ __forceinline__ void prefetch() {}
  __device__ __forceinline__ void score(int, int i, bool valid, float (&acc)[G], float& vn) {
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = 0.f;
    vn = 0.f;
    if (!valid) return;
    const uint8_t* id = idseg + (int64_t)i * L;
    for (int l = 0; l < L; ++l) {
      const int u = id[l] & ((1 << P) - 1);
      float pr[G];
#pragma unroll
      for (int j = 0; j < G; ++j) pr[j] = tab[(u * L + l) * G + j];
#pragma unroll
      for (int j = 0; j < G; ++j) acc[j] += pr[j];
    }
    vn = vseg[i];
  }
};

template <int G, int LW, bool BUILD, bool REGION>
__global__ __launch_bounds__(kScoreThreads) void score_kernel_rot(ScoreArgs a) {
  extern __shared__ __align__(16) float tab[];
  int bg, seg;
  if (!score_block_coords(a.bhkv, a.segs, bg, seg)) return;
  const WaveRange wr(a, seg);
  if constexpr (REGION) {
    // the region layouts: P = 8 with 16 or 32 tables, P = 6 with 64
    RegionScorer<LW, LW == 16 ? 6 : 8> sc(a, bg, wr, tab);
    score_block<G, BUILD, true>(a, bg, seg, tab, sc, wr);
  } else {
    RotScorer<G, LW> sc(a, bg, wr, tab);
    score_block<G, BUILD, false>(a, bg, seg, tab, sc, wr);
  }
}

template <int G>
__global__ __launch_bounds__(kScoreThreads) void score_kernel_generic(ScoreArgs a) {
  extern __shared__ __align__(16) float tab[];
  int bg, seg;
  if (!score_block_coords(a.bhkv, a.segs, bg, seg)) return;
  const WaveRange wr(a, seg);
  GenericScorer<G> sc(a, bg, wr, tab);
  score_block<G, false, false>(a, bg, seg, tab, sc, wr);
}

template <int G>
void set_lds_attributes() {
  static bool done = false;
  if (done) return;
  const int max_lds = (int)kLdsBytesPerCU;
  const void* fns[] = {
      reinterpret_cast<const void*>(&score_kernel_rot<G, 4, false, false>),
      reinterpret_cast<const void*>(&score_kernel_rot<G, 8, false, false>),
      reinterpret_cast<const void*>(&score_kernel_rot<G, 16, false, false>),
      reinterpret_cast<const void*>(&score_kernel_rot<G, 4, true, false>),
      reinterpret_cast<const void*>(&score_kernel_rot<G, 8, true, false>),
      reinterpret_cast<const void*>(&score_kernel_rot<G, 16, true, false>),
      reinterpret_cast<const void*>(&score_kernel_generic<G>)};
  for (const void* f : fns)
    (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
  if constexpr (G == 4) {
    const void* rf[] = {reinterpret_cast<const void*>(&score_kernel_rot<4, 4, false, true>),
                        reinterpret_cast<const void*>(&score_kernel_rot<4, 8, false, true>),
                        reinterpret_cast<const void*>(&score_kernel_rot<4, 16, false, true>),
                        reinterpret_cast<const void*>(&score_kernel_rot<4, 4, true, true>),
                        reinterpret_cast<const void*>(&score_kernel_rot<4, 8, true, true>)};
    for (const void* f : rf)
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
  }
  done = true;
}

template <int G, bool BUILD>
void launch_score_rot(const ScoreArgs& a, int grid, size_t lds, hipStream_t stream) {
  if constexpr (G == 4) {
    if (score_region(G, a.P, a.L)) {
      if (a.L == 32)
        launch_kernel((score_kernel_rot<4, 8, BUILD, true>), dim3(grid), dim3(kScoreThreads), lds,
                      stream, a);
      else if (a.L == 16)
        launch_kernel((score_kernel_rot<4, 4, BUILD, true>), dim3(grid), dim3(kScoreThreads), lds,
                      stream, a);
      else if constexpr (!BUILD)  // L = 64 (P = 6: the table is never built in the block)
        launch_kernel((score_kernel_rot<4, 16, false, true>), dim3(grid), dim3(kScoreThreads),
                      lds, stream, a);
      return;
    }
  }
  if (a.L == 32)
    launch_kernel((score_kernel_rot<G, 8, BUILD, false>), dim3(grid), dim3(kScoreThreads), lds,
                  stream, a);
  else if (a.L == 64)
    launch_kernel((score_kernel_rot<G, 16, BUILD, false>), dim3(grid), dim3(kScoreThreads), lds,
                  stream, a);
  else
    launch_kernel((score_kernel_rot<G, 4, BUILD, false>), dim3(grid), dim3(kScoreThreads), lds,
                  stream, a);
}

template <int G>
hipError_t launch_score_g(const ScoreArgs& a, hipStream_t stream) {
  const bool build = a.Qb != nullptr;
  const size_t lds = score_lds_bytes(a.L, a.P, G, build);
  const int total = a.bhkv * a.segs;
  const int grid = ((total + 7) / 8) * 8;
  set_lds_attributes<G>();
  if (build)
    launch_score_rot<G, true>(a, grid, lds, stream);
  else if (score_rotated(a.ids, a.stride, a.L))
    launch_score_rot<G, false>(a, grid, lds, stream);
  else
    launch_kernel((score_kernel_generic<G>), dim3(grid), dim3(kScoreThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_score_any(const ScoreArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_score_g<1>(a, stream);
    case 2: return launch_score_g<2>(a, stream);
    case 4: return launch_score_g<4>(a, stream);
    case 8: return launch_score_g<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

ScoreArgs base_args(const float* table, int table_G, const uint8_t* ids, const float* vnorm,
                    int B, int Hq, int Hkv, int id_div, int64_t n_keys, int64_t stride, int L,
                    int P) {
  const ScoreGeom geo = plan_score(B * Hkv, n_keys, L, P, Hq / Hkv);
  ScoreArgs a{};
  a.table = table;
  a.table_G = table_G;
  a.id_div = id_div;
  a.ids = ids;
  a.vnorm = vnorm;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.bhkv = B * Hkv;
  a.L = L;
  a.P = P;
  a.segs = geo.segs;
  a.seg_len = geo.seg_len;
  a.skew0 = geo.skew0;
  a.skew1 = geo.skew1;
  a.n_keys = n_keys;
  a.stride = stride;
  return a;
}

}  // namespace

size_t score_lds_bytes(int L, int P, int G, bool build) {
  return score_table_region(L, P, G) + (build ? build_weights_region(L, P, G) : 0) +
         (size_t)2 * G * kThrBins * sizeof(uint32_t);
}

bool score_builds_table(bool bf16, int d, const uint8_t* ids, int64_t stride, int L, int P,
                        int G) {
  // hyperplanes (16 * d * L bytes) and query rows (2 * G * d) staged in
  // the table's LDS
  return bf16 && P == 8 && (d == 64 || d == 128) && score_rotated(ids, stride, L) &&
         score_lds_bytes(L, P, G, true) <= kLdsBytesPerCU &&
         (size_t)16 * d * L + (size_t)2 * G * d <= score_table_region(L, P, G);
}

int score_pack(int L, int P, int G) {
  for (int gp = G; gp >= 1; gp >>= 1)
    if (G % gp == 0 && score_lds_bytes(L, P, gp, false) <= kLdsBytesPerCU) return gp;
  return 0;
}

namespace {
// The region scorer addresses its LDS table absolutely: it needs the
// kernels' dynamic LDS to start at address 0, i.e. no static LDS.
bool region_kernels_have_no_static_lds() {
  static const bool ok = [] {
    const void* fns[] = {reinterpret_cast<const void*>(&score_kernel_rot<4, 4, false, true>),
                         reinterpret_cast<const void*>(&score_kernel_rot<4, 8, false, true>),
                         reinterpret_cast<const void*>(&score_kernel_rot<4, 16, false, true>),
                         reinterpret_cast<const void*>(&score_kernel_rot<4, 4, true, true>),
                         reinterpret_cast<const void*>(&score_kernel_rot<4, 8, true, true>)};
    for (const void* f : fns) {
      hipFuncAttributes attr{};
      if (hipFuncGetAttributes(&attr, f) != hipSuccess || attr.sharedSizeBytes != 0) return false;
    }
    return true;
  }();
  return ok;
}
}  // namespace

bool score_region(int G, int P, int L) {
  return G == 4 && ((P == 8 && (L == 16 || L == 32)) || (P == 6 && L == 64)) &&
         region_kernels_have_no_static_lds();
}

bool score_rotated(const uint8_t* ids, int64_t stride, int L) {
  const bool aligned = (reinterpret_cast<uintptr_t>(ids) % 16 == 0) && ((stride * L) % 16 == 0);
  return aligned && (L == 16 || L == 32 || L == 64);
}

ScoreGeom plan_score(int bhkv, int64_t n_keys, int L, int P, int G) {
  ScoreGeom geo{};
  // the same geometry whether or not the block builds its table
  const bool could_build = P == 8 && (L == 16 || L == 32 || L == 64);
  const size_t lds = score_lds_bytes(L, P, G, could_build);
  // blocks resident per CU as limited by the 160 KB of LDS and by the
  // registers: two 1024-thread blocks need <= 64 VGPRs per lane, which
  // only the kernels for one query head per block with L <= 32 and the
  // table-copying kernels with L = 16 and G <= 4 use (the others take
  // 72-128); a second block that cannot be resident would run in a
  // second round
  const bool regs_fit_two = (G == 1 && L <= 32) || (L <= 16 && G <= 4 && P != 8);
  const int per_cu = regs_fit_two
                         ? (int)std::max<size_t>(1, std::min<size_t>(2, kLdsBytesPerCU / lds))
                         : 1;
  const int64_t target = (int64_t)256 * per_cu;
  constexpr int64_t kSegUnit = (int64_t)kScoreWaves * kWaveStep;
  int64_t segs = (target + bhkv - 1) / bhkv;
  segs = std::max<int64_t>(1, std::min<int64_t>(segs, (n_keys + kSegUnit - 1) / kSegUnit));
  int64_t seg_len = (n_keys + segs - 1) / segs;
  seg_len = (seg_len + kSegUnit - 1) / kSegUnit * kSegUnit;
  if (seg_len > kMaxSeg) seg_len = kMaxSeg;
  segs = (n_keys + seg_len - 1) / seg_len;
  geo.segs = (int)segs;
  geo.seg_len = seg_len;
  geo.subs = (int)(segs * kScoreWaves);
  geo.sub_len = seg_len / kScoreWaves;
  // unequal wave shares, in steps of kWaveStep keys out of S per wave. With
  // 64 tables (16 steps per wave at 1M keys) the last group of four waves
  // finished 27 us, about 7 steps' worth, after the first; shares {S+3,
  // S+1, S-1, S-3} leave ~5 us and take 8 us off the kernel. With 32
  // tables the groups end within ~3.6 us of each other and one step of
  // skew made the kernel slower (no skew there).
  const int S = (int)(geo.sub_len / kWaveStep);
  geo.skew0 = L >= 64 ? (S * 3 + 8) / 16 * kWaveStep : 0;
  geo.skew1 = L >= 64 ? S / 16 * kWaveStep : 0;
  return geo;
}

void set_build(ScoreArgs& a, const TableBuild* build, float* table_out) {
  if (!build) return;
  a.Qb = static_cast<const uint16_t*>(build->Q);
  a.Rb = static_cast<const uint16_t*>(build->R);
  a.d = build->d;
  a.two_over_tau = 2.0 / (double)build->tau;
  a.table_out = table_out;
}

hipError_t launch_score(const float* table, int table_G, const uint8_t* ids, const float* vnorm,
                        int B, int Hq, int Hkv, int id_div, int64_t n_keys, int64_t stride,
                        int L, int P, float* scores, const TableBuild* build,
                        hipStream_t stream) {
  if (n_keys == 0) return hipSuccess;
  ScoreArgs a = base_args(table, table_G, ids, vnorm, B, Hq, Hkv, id_div, n_keys, stride, L, P);
  a.scores = scores;
  set_build(a, build, nullptr);
  return launch_score_any(a, Hq / Hkv, stream);
}

hipError_t launch_score_select(const ScoreSelect& s, int B, int Hq, int Hkv, int64_t n_keys,
                               int64_t stride, int L, int P, float* scores,
                               const TableBuild* build, hipStream_t stream) {
  ScoreArgs a = base_args(s.table, Hq / Hkv, s.ids, s.vnorm, B, Hq, Hkv, s.id_div, n_keys, stride,
                          L, P);
  a.scores = scores;
  a.select = 1;
  a.kk = s.kk;
  a.thr = s.thr;
  a.lists = s.lists;
  a.sub_cnt = s.sub_cnt;
  set_build(a, build, const_cast<float*>(s.table));
  return launch_score_any(a, Hq / Hkv, stream);
}

}  // namespace socket_lsh
