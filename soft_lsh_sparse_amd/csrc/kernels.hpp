// Host-side launchers of the SOCKET kernels. Every launcher assumes its
// arguments were validated by the C-ABI layer and enqueues on `stream`.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace socket_lsh {

// Optional kernel timing for profiling: while set (by the profiled decode
// entry point), every launch takes the next two events of the list, which
// the dispatch itself records at the start and at the end of the kernel's
// execution (no extra stream packets, so the time between them is the
// kernel's own duration).
struct LaunchTrace {
  hipEvent_t* events;
  int n;
  int used;
};
extern thread_local LaunchTrace* g_trace;

// kernel<<<grid, block, lds, stream>>>(args...), timed under a trace.
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                          Args... args) {
  hipEvent_t start = nullptr, stop = nullptr;
  if (g_trace != nullptr && g_trace->used + 2 <= g_trace->n) {
    start = g_trace->events[g_trace->used++];
    stop = g_trace->events[g_trace->used++];
  }
  hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, start, stop, 0u, args...);
}

// Workspace sub-buffers start on 256-byte boundaries.
inline constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ------------------------------------------------------------- prefill hash
// Entries of the deferred sign fix-up list for n_total keys of C hyperplanes.
uint32_t hash_fix_capacity(int64_t n_total, int C);
// Workspace of the bf16 path: R^T, the fix-up counts and lists, the tile
// counter and the tile owners.
size_t hash_keys_bf16_workspace_bytes(int64_t n_heads, int64_t n_keys, int d, int C);
// ws: hash_keys_bf16_workspace_bytes(...) bytes, 256-byte aligned.
hipError_t launch_hash_keys_bf16(const uint16_t* K, const uint16_t* V,
                                 const uint16_t* R, int64_t n_heads,
                                 int64_t n_keys, int64_t stride, int d, int L,
                                 int P, uint8_t* ids, float* vnorm, void* ws,
                                 hipStream_t stream);
hipError_t launch_hash_keys_f32(const float* K, const float* V, const float* R,
                                int64_t n_heads, int64_t n_keys,
                                int64_t stride, int d, int L, int P,
                                uint8_t* ids, float* vnorm,
                                hipStream_t stream);

// ------------------------------------------------------ soft bucket table
hipError_t launch_bucket_probs(const void* Q, const void* R, bool bf16, int B,
                               int Hq, int Hkv, int d, int L, int P,
                               float tau, float* table, hipStream_t stream);

// ------------------------------------------------------------------ score
// Launch geometry of the score kernel: segs blocks per (batch, KV head) of
// seg_len keys each; every block's 16 waves own consecutive keys, sub_len
// of them on average (subs = segs * 16 sub-lists per row when emitting
// candidates). The shares can be unequal: each SIMD serves its oldest wave
// first, so with equal shares waves 0-3 finish first and waves 12-15 last,
// each group of four a few percent of the block's time after the one
// before. Waves 4g..4g+3 take sub_len + {skew0, skew1, -skew1, -skew0}[g]
// keys (multiples of 128; the plan sets a skew where it evens out the
// finish times: 64 tables).
struct ScoreGeom {
  int segs;
  int64_t seg_len;
  int subs;
  int64_t sub_len;
  int skew0, skew1;
};
// Sub-list s (= 16 * segment + wave) of a row: its keys start at
// sub_begin(s, ...) and number sub_size(s, ...) (fewer in a last, partial
// segment), and its candidates are stored from the same position.
__host__ __device__ inline int64_t sub_begin(int s, int64_t sub_len, int skew0, int skew1) {
  // wave w = 4g + i starts A(w) * skew0 + B(w) * skew1 past w * sub_len:
  // A = i, 4, 4, 4 - i and B = 0, i, 4 - i, 0 for g = 0..3 (4-bit fields)
  const int w = s & 15;
  const int a = (int)((0x1234444444443210ull >> (4 * w)) & 15u);
  const int b = (int)((0x0000123432100000ull >> (4 * w)) & 15u);
  return (int64_t)s * sub_len + a * skew0 + b * skew1;
}
__host__ __device__ inline int64_t sub_size(int s, int64_t sub_len, int skew0, int skew1) {
  const int g = (s & 15) >> 2;
  return sub_len + (g == 0 ? skew0 : g == 1 ? skew1 : g == 2 ? -skew1 : -skew0);
}
ScoreGeom plan_score(int bhkv, int64_t n_keys, int L, int P, int G);
// GQA packing. When the probability table of a whole group (2^P * L * G
// floats) does not fit a score block's LDS, each block scores Gp of the G
// query heads of its KV head: the score pipeline then runs over B * Hkv * np
// "virtual" KV heads of Gp query heads each (np = G / Gp; query head h
// belongs to virtual head h / Gp, which reads the ids and norms of KV head
// (virtual head) / np). Returns the largest such Gp (a power of two dividing
// G) whose table fits, or 0 when not even Gp = 1 does.
int score_pack(int L, int P, int G);
// true when the kernel sums each key's tables in a rotated order (r = key
// mod 16): l = (t + r) mod L, t = 0..L-1, or, when score_region(G, P, L),
// l = 16 c + (t' + r) mod 16 for t = 16 c + t' (each 16-table region
// rotated on its own); else l = t
bool score_rotated(const uint8_t* ids, int64_t stride, int L);
// The rotated path keeps the table in 16-table regions (G = 4; P = 8 with
// L = 16 or 32, P = 6 with L = 64).
bool score_region(int G, int P, int L);
// LDS bytes of one score block (build: the block builds its table).
size_t score_lds_bytes(int L, int P, int G, bool build);
constexpr size_t kLdsBytesPerCU = 160 * 1024;
// The score kernel builds each head's table itself (no table kernel) for
// bf16 queries and hyperplanes, P = 8, d in {64, 128}, the rotated path and
// a table plus build within the LDS of a CU; the table is equal bit for bit
// to launch_bucket_probs'.
bool score_builds_table(bool bf16, int d, const uint8_t* ids, int64_t stride, int L, int P,
                        int G);
struct TableBuild {
  const void* Q;  // [B, Hq, d] bf16
  const void* R;  // [d, L*P] bf16
  int d;
  float tau;
};
// Hkv: virtual KV heads (Hq / Hkv query heads each, see score_pack); the
// ids and norms of virtual head v are those of head v / id_div. table:
// [B*Hkv/id_div, 2^P, L, table_G] from launch_bucket_probs (virtual head v
// takes heads (v % id_div) * Hq/Hkv ... of its slots), or unused with build;
// scores [B*Hq, n_keys].
hipError_t launch_score(const float* table, int table_G, const uint8_t* ids, const float* vnorm,
                        int B, int Hq, int Hkv, int id_div, int64_t n_keys, int64_t stride,
                        int L, int P, float* scores, const TableBuild* build,
                        hipStream_t stream);
// Decode path: every block estimates a per-row threshold from its first
// keys (thr[row * segs + seg], an order key) and appends every key whose
// score's order key reaches it, as (float32 score bits, index), to sub-list (row, s)
// at lists[row * n_keys + sub_begin(s, ...)], in index order; sub_cnt[row *
// subs + s] receives the sub-list's length.
struct ScoreSelect {
  const float* table;  // [B*Hkv, 2^P, L, G] over virtual heads (written by the kernel with build)
  int id_div;          // virtual head v reads the ids and norms of head v / id_div
  const uint8_t* ids;
  const float* vnorm;
  int64_t kk;          // < n_keys
  uint32_t* thr;       // [B*Hq, segs]
  uint2* lists;        // [B*Hq, n_keys]
  uint32_t* sub_cnt;   // [B*Hq, subs]
};
// scores (optional): full score rows as well.
hipError_t launch_score_select(const ScoreSelect& s, int B, int Hq, int Hkv, int64_t n_keys,
                               int64_t stride, int L, int P, float* scores,
                               const TableBuild* build, hipStream_t stream);

// ------------------------------------------------------------------ top-k
struct TopkPlan {
  int rows;
  int64_t n, kk;
  int segs;          // blocks per row
  int64_t seg_len;   // scores per block
  int subs;          // sub-lists per row (one per wave)
  int64_t sub_len;   // scores per wave
  size_t hist_off, cnt_off, list_off, total_bytes;
  int64_t zero_words;  // words from hist_off that must be zero before a call
};
TopkPlan plan_topk(int rows, int64_t n, int64_t k);
hipError_t launch_zero_u32(uint32_t* p, int64_t words, hipStream_t stream);
hipError_t launch_topk(const float* scores, const TopkPlan& plan,
                       int32_t* idx, void* ws, hipStream_t stream);
hipError_t launch_iota_rows(int32_t* idx, int rows, int64_t n, hipStream_t stream);

// Selection from the score kernel's candidates (decode path), one block per
// row: with T the largest of the row's block thresholds, every key whose
// order key reaches T is a candidate; when at least kk do, the kk best
// candidates are the result, otherwise the row is scored in full into
// scores and selected from there.
constexpr int kMaxSelectSubLists = 4096;
struct SelectArgs {
  int64_t n, kk;              // kk < n
  int subs;                   // <= kMaxSelectSubLists
  int64_t sub_len;
  int skew0, skew1;           // sub-list s at sub_begin(s, sub_len, skew0, skew1)
  int segs;
  const uint32_t* thr;        // [rows][segs]
  const uint2* lists;
  const uint32_t* sub_cnt;
  int32_t* idx;               // [rows][kk]
  const float* table;         // full-row fallback: the score kernel's inputs
  const uint8_t* ids;
  const float* vnorm;
  int Hq, Hkv, L, P;          // Hkv: virtual KV heads (score_pack)
  int id_div;                 // virtual head v reads the ids of head v / id_div
  int64_t stride;
  int rotated;                // score_rotated(ids, stride, L)
  int region;                 // rotated and score_region(Hq / Hkv, P, L)
  float* scores;              // [rows][n] row buffers
  // Rows with many candidates (large kk): a gather kernel first copies each
  // row's candidates, as order keys in index order, into one contiguous run
  // inside the row's region of `spill` ([rows][n] float32 words, 16-byte
  // aligned; never the caller's score rows), with the largest order key of
  // each gather block in `bmax` [rows][select_gather_blocks(subs, kk)].
  // Null spill: no gather.
  uint2* spill;
  uint32_t* bmax;
};
// Gather blocks per row the selection launches for these sizes (0: none).
int select_gather_blocks(int subs, int64_t kk);
hipError_t launch_topk_select(const SelectArgs& a, int rows, hipStream_t stream);

// ------------------------------------------------------- sparse attention
// Chunk partials per row that one thread of the merge kernel combines from
// registers (more chunks are staged in LDS).
constexpr int kMergeRegChunks = 16;
// Largest selection one attention row supports: 1024 chunks of 256 keys.
constexpr int64_t kMaxSelected = 262144;
struct AttnPlan {
  int B, Hq, Hkv, d;
  int64_t kk;
  int waves;  // per block: 4, or 1 (64 keys per block) for short rows
  int keys_per_wave, chunk_keys, chunks;
  size_t partial_bytes;
};
AttnPlan plan_attn(int B, int Hq, int Hkv, int d, int64_t kk);
hipError_t launch_sparse_attn(const void* Q, const void* K, const void* V,
                              bool bf16, const AttnPlan& plan, int64_t stride,
                              const int32_t* idx, void* out, float* partial,
                              hipStream_t stream);

// Online-softmax merge of chunk partials [rows][chunks][d + 2] (acc[d], m,
// l) into out [rows, d] in the input dtype.
hipError_t launch_attn_merge(const float* partial, int rows, int chunks, int d, bool bf16,
                             void* out, hipStream_t stream);

// ------------------------------------------------- dense attention baseline
struct DensePlan {
  int B, Hq, Hkv, d;
  int64_t n;
  int chunks;            // of 1024 keys per (b, KV head)
  size_t partial_bytes;
};
// Largest context the dense baseline takes: 1024 chunks (the merge's limit).
constexpr int64_t kMaxDenseKeys = 1024 * 1024;
DensePlan plan_dense(int B, int Hq, int Hkv, int d, int64_t n);
// idx: nullptr for rows 0..n-1 of every KV head, else a shared index set per
// KV head [B*Hkv, n] (the GQA group-shared variant).
hipError_t launch_dense_attn(const void* Q, const void* K, const void* V, bool bf16,
                             const DensePlan& plan, int64_t stride, const int32_t* idx,
                             void* out, float* partial, hipStream_t stream);
// Group table [B*Hkv, 2^P, L] = the sum over the G heads of a table
// [B*Hkv, 2^P, L, G] (the GQA group-shared variant).
hipError_t launch_group_table_sum(const float* table, int bhkv, int L, int P, int G, float* out,
                                  hipStream_t stream);

}  // namespace socket_lsh
