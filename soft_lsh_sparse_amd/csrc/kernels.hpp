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
// Workspace of the bf16 path: R^T, the fix-up counter and list.
size_t hash_keys_bf16_workspace_bytes(int64_t n_total, int d, int C);
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
// zero_ptr/zero_words: optional device words cleared by the same launch.
hipError_t launch_bucket_probs(const void* Q, const void* R, bool bf16, int B,
                               int Hq, int Hkv, int d, int L, int P,
                               float tau, float* table, uint32_t* zero_ptr,
                               int64_t zero_words, hipStream_t stream);

// ------------------------------------------------------------------ score
// table: [B*Hkv, 2^P, L, G] from launch_bucket_probs.
// hist (optional): [B*Hq, 2048] first-digit histograms, accumulated with
// atomics; must be zero on entry.
hipError_t launch_score(const float* table, const uint8_t* ids, const float* vnorm,
                        int B, int Hq, int Hkv, int64_t n_keys, int64_t stride,
                        int L, int P, float* scores, uint32_t* hist,
                        hipStream_t stream);
// LDS bytes one score block needs: the probability table, plus the packed
// first-digit histogram when fused.
size_t score_lds_bytes(int L, int P, int G, bool with_hist);
constexpr size_t kLdsBytesPerCU = 160 * 1024;

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
constexpr int kHistBins = 2048;
hipError_t launch_zero_u32(uint32_t* p, int64_t words, hipStream_t stream);
// hist_ready: the histogram region of ws already holds the first-digit
// histogram (filled by the score kernel); otherwise it is built here.
hipError_t launch_topk(const float* scores, const TopkPlan& plan,
                       int32_t* idx, void* ws, bool hist_ready,
                       hipStream_t stream);

// ------------------------------------------------------- sparse attention
// Largest selection one attention row supports: 1024 chunks of 256 keys.
constexpr int64_t kMaxSelected = 262144;
struct AttnPlan {
  int B, Hq, Hkv, d;
  int64_t kk;
  int keys_per_wave, chunk_keys, chunks;
  size_t partial_bytes;
};
AttnPlan plan_attn(int B, int Hq, int Hkv, int d, int64_t kk);
hipError_t launch_sparse_attn(const void* Q, const void* K, const void* V,
                              bool bf16, const AttnPlan& plan, int64_t stride,
                              const int32_t* idx, void* out, float* partial,
                              hipStream_t stream);

}  // namespace socket_lsh
