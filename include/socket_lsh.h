/*
 * socket_lsh.h - C ABI of the SOCKET soft-collision sparse-attention decode
 * library for AMD Instinct MI355X (gfx950).
 *
 * The method (pages "Resumen Técnico: SOCKET - Estimador de Núcleo de
 * Colisión Suave para Atención Escasa", section "Mecanismo Central: LSH
 * Suave", items 1-4, and "SOCKET: SOft Collision Kernel EsTimator for Sparse
 * Attention", Technische Zusammenfassung, "Kernmechanismus: Soft LSH"):
 *   prefill : hash every key into L tables of P random-hyperplane sign bits
 *             and cache the Euclidean norm of every value row;
 *   decode  : turn the query's hyperplane projections into a temperature
 *             softmax over the 2^P buckets of each table, score each key by
 *             the probability mass on its own buckets summed over the tables
 *             and weighted by its value norm, keep the top-k keys
 *             deterministically and run exact softmax attention over them.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers, caller-allocated, contiguous,
 *     row-major in the layouts written next to each argument. The library
 *     allocates nothing, frees nothing and keeps no state between calls
 *     (socket_decode_noalloc aside: it works in a device array the library
 *     holds on each GPU, see there).
 *   - dtype selects the element type of Q, K, V, R and the attention output:
 *     SOCKET_DTYPE_F32 (float) or SOCKET_DTYPE_BF16 (bfloat16 bits, round to
 *     nearest even on output). Bucket ids are uint8, norms, probabilities
 *     and scores float32, selected indices int32.
 *   - stream is a hipStream_t (NULL = the default stream). Every call only
 *     enqueues work on it and returns; kernel faults surface at the caller's
 *     next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued. A
 *     non-OK status means nothing was enqueued (except SOCKET_ERR_HIP, which
 *     reports a failed launch). socket_last_error() then describes the
 *     problem (thread-local, valid until the next call on that thread).
 *   - Inputs must be finite. This is not checked on the device.
 *   - Supported sizes: d in {64, 128}; 1 <= P <= 8; 1 <= L and L*P <= 1024
 *     (L*P <= 512 for bf16 hashing); Hq a multiple of Hkv with
 *     G = Hq/Hkv in {1, 2, 4, 8}; k >= 1. The score kernel keeps the
 *     probability tables of Gp query heads of a KV head in the 160 KB LDS of
 *     a CU (2^P * L * Gp * 4 bytes plus 2 KB per head): Gp is the largest
 *     power of two dividing G that fits, and with Gp < G the ids of a KV head
 *     are streamed once per pack of Gp heads (every L*P <= 1024 fits at
 *     Gp = 1);
 *     head_stride_rows < 2^31 for decode (int32 key indices).
 *   - Unsupported but valid sizes return SOCKET_ERR_UNSUPPORTED.
 *
 * Readings of the pages used throughout (they state no formulas):
 *   - bit j of table l of key n is 1 iff the exact dot product K[n].R[:,l*P+j]
 *     is > 0; the bucket id is sum_j bit_j * 2^j;
 *   - the query assigns bucket u of table l the probability softmax_u of
 *     (1/tau) * sum_j s_j(u) * (q . R[:, l*P+j]), s_j(u) = +1 if bit j of u
 *     is set, else -1 (raw, unnormalised projections);
 *   - score[b,h,n] = vnorm[b,g,n] * sum_l prob[b,h,l,ids[b,g,n,l]], with
 *     g = floor(h / G) (grouped-query attention);
 *   - top-k keeps the min(k, N) largest scores, equal scores going to the
 *     lower index, and returns the indices in ascending order;
 *   - attention over the kept keys uses the scale 1/sqrt(d) and is
 *     renormalised over them only.
 */
#ifndef SOCKET_LSH_H
#define SOCKET_LSH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SOCKET_OK = 0,
  SOCKET_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size or parameter   */
  SOCKET_ERR_UNSUPPORTED = 2,      /* valid but not implemented (d, G, L*P) */
  SOCKET_ERR_WORKSPACE = 3,        /* workspace missing or too small        */
  SOCKET_ERR_HIP = 4               /* a HIP launch failed                   */
} socket_status;

typedef enum {
  SOCKET_DTYPE_F32 = 0,
  SOCKET_DTYPE_BF16 = 1
} socket_dtype;

/* Library version as (major << 16) | (minor << 8) | patch. */
int32_t socket_version(void);

/* Static description of a status code. Never NULL. */
const char* socket_status_string(socket_status status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* socket_last_error(void);

/*
 * Prefill: hash keys and cache value norms.
 * Defines: step 1 of the soft-LSH mechanism (prefill hashing into L tables
 * with random projections, value norms cached).
 *
 *   K, V   [n_heads, head_stride_rows, d]  dtype; rows [0, n_keys) are used
 *   R      [d, L*P] dtype; column l*P + j is hyperplane j of table l
 *   ids    [n_heads, head_stride_rows, L] uint8 (output, rows [0, n_keys))
 *   vnorm  [n_heads, head_stride_rows]   float32 (output, Euclidean norm)
 *
 * n_heads is B*Hkv. Appending keys at row offset o of every head works by
 * passing K, V, ids and vnorm advanced by o rows with the same stride. A
 * decode loop appends one key per head and step: bf16 calls of at most 32
 * keys in all run as one launch (one block per key), and their ids and
 * norms equal those a prefill of the same rows gives, bit for bit.
 * Bucket ids are exact: the sign of every projection is that of the exact
 * dot product (projections too close to zero for the fast float32 path are
 * re-evaluated in extended precision). n_keys == 0 is a no-op.
 *
 * Workspace: socket_hash_keys_workspace_bytes(dtype, n_heads, n_keys, d, L,
 * P) bytes of device memory, 256-byte aligned (0 bytes, NULL allowed, for
 * SOCKET_DTYPE_F32). It holds the transposed hyperplanes, the list of
 * projections settled in extended precision after the main pass and a
 * record of which wave hashed each 32-key tile; its contents on entry do not
 * matter. A smaller or misaligned workspace returns
 * SOCKET_ERR_WORKSPACE. K, V and R must be 16-byte aligned.
 */
size_t socket_hash_keys_workspace_bytes(socket_dtype dtype, int64_t n_heads,
                                        int64_t n_keys, int32_t d, int32_t L,
                                        int32_t P);
socket_status socket_hash_keys(const void* K, const void* V, const void* R,
                               socket_dtype dtype, int64_t n_heads,
                               int64_t n_keys, int64_t head_stride_rows,
                               int32_t d, int32_t L, int32_t P, uint8_t* ids,
                               float* vnorm, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Decode stage 1: soft bucket probabilities of the queries.
 * Defines: step 2 of the soft-LSH mechanism (soft assignment of the query
 * over all buckets of every table through a temperature softmax).
 *
 *   Q      [B, Hq, d] dtype
 *   R      [d, L*P] dtype
 *   table  [B, Hkv, 2^P, L, G] float32 (output); entry (b, g, u, l, j) is the
 *          probability that query head g*G + j gives to bucket u of table l
 *          (this order lets one 16-byte load serve a whole GQA group).
 * tau must be finite and > 0.
 */
socket_status socket_bucket_probs(const void* Q, const void* R,
                                  socket_dtype dtype, int32_t B, int32_t Hq,
                                  int32_t Hkv, int32_t d, int32_t L,
                                  int32_t P, float tau, float* table,
                                  void* stream);

/*
 * Hard-LSH comparison: the tau -> 0 limit of socket_bucket_probs, a one-hot
 * table with 1 at the query's own bucket of every table (the bucket of its
 * projection signs; a projection of exactly 0 splits its bit 1/2 : 1/2, as
 * every soft table does). socket_score on this table gives each key its
 * value norm times the number of tables in which it collides with the
 * query: the hard collision count the soft score replaces.
 * Defines: the tau -> 0 limit and the soft-versus-hard comparison of the
 * German page "SOCKET: SOft Collision Kernel EsTimator for Sparse
 * Attention", section "Theoretische Grundlage" (Stabilität, Korrelation).
 *
 *   Q, R, table: as for socket_bucket_probs.
 */
socket_status socket_hard_bucket_table(const void* Q, const void* R, socket_dtype dtype,
                                      int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t L,
                                      int32_t P, float* table, void* stream);

/*
 * Decode stage 2: soft collision scores.
 * Defines: step 3 of the soft-LSH mechanism (per key, the probability mass
 * on its own bucket summed over the L tables, weighted by its value norm).
 *
 *   table   [B, Hkv, 2^P, L, G] float32 (from socket_bucket_probs)
 *   ids     [B*Hkv, head_stride_rows, L] uint8
 *   vnorm   [B*Hkv, head_stride_rows] float32
 *   scores  [B, Hq, n_keys] float32 (output)
 * The L probabilities are summed in float32 in a fixed order, then
 * multiplied by the value norm. With r = key index mod 16, when L is 16, 32
 * or 64 and the id rows are 16-byte aligned (this spreads LDS banks): for
 * 4 query heads per block with P = 8 and 32 or 16 tables, or P = 6 and 64
 * tables, table 16c + (t + r) mod 16 at step 16c + t (t < 16: each run of
 * 16 tables rotated on its own); otherwise l = (t + r) mod L at step t. In
 * all other cases l = t.
 */
socket_status socket_score(const float* table, const uint8_t* ids,
                           const float* vnorm, int32_t B, int32_t Hq,
                           int32_t Hkv, int64_t n_keys,
                           int64_t head_stride_rows, int32_t L, int32_t P,
                           float* scores, void* stream);

/*
 * Decode stage 3: deterministic top-k of each row.
 * Defines: step 4 of the soft-LSH mechanism (deterministic selection of the
 * k best keys by soft score).
 *
 *   scores  [rows, n] float32 (non-negative, finite; -0.0 counts as +0.0)
 *   idx     [rows, min(k, n)] int32 (output), ascending within each row
 * Keeps the min(k, n) largest scores of each row; among equal scores the
 * lower index wins. The result is exact and identical on every run.
 * Workspace: socket_topk_workspace_bytes(rows, n, k) bytes of device memory.
 */
size_t socket_topk_workspace_bytes(int32_t rows, int64_t n, int64_t k);
socket_status socket_topk(const float* scores, int32_t rows, int64_t n,
                          int64_t k, int32_t* idx, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Decode stage 4: exact attention over the selected keys.
 * Defines: step 4 of the soft-LSH mechanism (exact attention over the
 * selected subset).
 *
 *   Q    [B, Hq, d] dtype
 *   K, V [B, Hkv, head_stride_rows, d] dtype
 *   idx  [B, Hq, kk] int32, every entry in [0, head_stride_rows); kk >= 1
 *   out  [B, Hq, d] dtype (output)
 * out[b,h] = sum_i softmax_i(q . k_i / sqrt(d)) v_i over the kk listed keys
 * (float32 accumulation; the result does not depend on the order of idx
 * beyond float32 rounding).
 * Workspace: socket_sparse_attn_workspace_bytes(B, Hq, d, kk) bytes.
 */
size_t socket_sparse_attn_workspace_bytes(int32_t B, int32_t Hq, int32_t d,
                                          int64_t kk);
socket_status socket_sparse_attn(const void* Q, const void* K, const void* V,
                                 socket_dtype dtype, int32_t B, int32_t Hq,
                                 int32_t Hkv, int32_t d,
                                 int64_t head_stride_rows, const int32_t* idx,
                                 int64_t kk, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Variant: GQA group-shared selection. One index set per KV head: the keys
 * are ranked by the sum of the soft scores of the G query heads of the group
 * (equivalently, by the group table sum_j p[u, l, j] in place of each head's
 * own), the kk best are kept (ties to the lower index), and every head of
 * the group attends over that same set, so one gather of K and V rows serves
 * the G heads. The pages leave GQA open (page "Resumen Técnico: SOCKET -
 * Estimador de Núcleo de Colisión Suave para Atención Escasa", section
 * "Mecanismo Central: LSH Suave"); socket_decode keeps per-head selection.
 *
 * Arguments as for socket_decode, except:
 *   idx_out     optional, [B, Hkv, min(k, n_keys)] int32, ascending
 *   scores_out  optional, [B, Hkv, n_keys] float32 group scores
 * Hq / Hkv <= 8 and min(k, n_keys) <= 2^20, else SOCKET_ERR_UNSUPPORTED.
 * Workspace: socket_decode_group_shared_workspace_bytes(...) bytes.
 */
size_t socket_decode_group_shared_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                                  int64_t n_keys, int32_t L, int32_t P,
                                                  int64_t k);
socket_status socket_decode_group_shared(const void* Q, const void* K, const void* V,
                                         const void* R, const uint8_t* ids, const float* vnorm,
                                         socket_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                         int32_t d, int64_t n_keys, int64_t head_stride_rows,
                                         int32_t L, int32_t P, float tau, int64_t k, void* out,
                                         int32_t* idx_out, float* scores_out, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * Baseline: dense attention decoding (every key), the comparison SOCKET's
 * speed-up is stated against.
 * Defines: the dense FlashAttention decoding of the pages' efficiency
 * results (page "Resumen Técnico: SOCKET - Estimador de Núcleo de Colisión
 * Suave para Atención Escasa", section "Resultados Experimentales").
 *
 *   Q    [B, Hq, d] dtype
 *   K, V [B, Hkv, head_stride_rows, d] dtype; rows 0..n-1 are attended
 *   out  [B, Hq, d] dtype (output)
 * out[b,h] = sum_{i<n} softmax_i(q . k_i / sqrt(d)) v_i with query head h
 * reading KV head h / (Hq / Hkv); float32 accumulation in a fixed order.
 * 1 <= n <= 2^20 and Hq / Hkv <= 8, else SOCKET_ERR_UNSUPPORTED.
 * Workspace: socket_dense_attn_workspace_bytes(B, Hq, d, n) bytes of device
 * memory (chunk partials); all pointers are device pointers the caller owns.
 */
size_t socket_dense_attn_workspace_bytes(int32_t B, int32_t Hq, int32_t d, int64_t n);
socket_status socket_dense_attn(const void* Q, const void* K, const void* V,
                                socket_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                int32_t d, int64_t n, int64_t head_stride_rows, void* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * One whole decode step: stages 1-4 back to back on one stream, no host
 * synchronisation.
 * Defines: steps 2-4 of the soft-LSH mechanism (the decode side).
 *
 *   Q           [B, Hq, d] dtype
 *   K, V        [B, Hkv, head_stride_rows, d] dtype (rows [0, n_keys) used)
 *   R           [d, L*P] dtype (the one used to hash the keys)
 *   ids, vnorm  from socket_hash_keys over the same rows
 *   out         [B, Hq, d] dtype (output)
 *   idx_out     [B, Hq, min(k, n_keys)] int32 (output) or NULL
 *   scores_out  [B, Hq, n_keys] float32 (output) or NULL
 * A NULL idx_out keeps the indices in the workspace. Score rows are written
 * only when scores_out is given (the selection itself keeps only the keys
 * that reach a sampled per-block threshold, verifies that they contain the
 * top k and otherwise scores the row in full); the indices are those of the
 * exact top k of the rows socket_score would produce, ties to the lower
 * index, in ascending order.
 * Workspace: socket_decode_workspace_bytes(...) bytes of device memory.
 * n_keys must be >= 1. With k < n_keys the selection reads at most 4096
 * candidate sub-lists per row (n_keys up to about 2^28 at one pack per CU,
 * fewer where two score blocks fit a CU); otherwise SOCKET_ERR_UNSUPPORTED.
 */
size_t socket_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv,
                                     int32_t d, int64_t n_keys, int32_t L,
                                     int32_t P, int64_t k);
socket_status socket_decode(const void* Q, const void* K, const void* V,
                            const void* R, const uint8_t* ids,
                            const float* vnorm, socket_dtype dtype, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t d,
                            int64_t n_keys, int64_t head_stride_rows,
                            int32_t L, int32_t P, float tau, int64_t k,
                            void* out, int32_t* idx_out, float* scores_out,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It is socket_decode with the workspace in a device array the
 * library owns instead of caller memory: SOCKET_DECODE_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, held by every GPU the library runs on until the process
 * ends. Arguments, validation and results are those of socket_decode (the
 * same kernels, bit for bit), without workspace and workspace_bytes.
 *   - A call whose socket_decode_workspace_bytes(...) exceeds the array
 *     returns SOCKET_ERR_UNSUPPORTED (e.g. B = 1 at 131072 keys fits,
 *     B = 4 at 131072 keys does not).
 *   - It calls no hipMalloc, hipFree or other allocating routine. The first
 *     call on each device resolves the array's address there
 *     (hipGetSymbolAddress, with that device current); make that first call
 *     outside graph capture.
 *   - All calls on one GPU share its array, which keeps the last call's
 *     contents (nothing in it needs clearing between calls). Calls that
 *     overlap on one GPU (several streams or threads at once) race on it:
 *     the caller must serialise them.
 */
#define SOCKET_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
socket_status socket_decode_noalloc(const void* Q, const void* K, const void* V,
                                    const void* R, const uint8_t* ids,
                                    const float* vnorm, socket_dtype dtype,
                                    int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                    int64_t n_keys, int64_t head_stride_rows,
                                    int32_t L, int32_t P, float tau, int64_t k,
                                    void* out, int32_t* idx_out,
                                    float* scores_out, void* stream);

/*
 * socket_decode with per-kernel timing: identical work and results. In
 * addition the i-th kernel it enqueues (i = 0, 1, ...) is dispatched with
 * events[2i] and events[2i+1] (hipEvent_t handles created by the caller) as
 * its start and stop events, which the dispatch records at the start and
 * end of that kernel's execution, for the first n_events / 2 kernels.
 * socket_decode_kernels names the kernels in this order. Unused events are
 * not touched. For profiling tools; events must not be NULL and n_events
 * must be >= 2 (else SOCKET_ERR_INVALID_ARGUMENT).
 */
socket_status socket_decode_profiled(
    const void* Q, const void* K, const void* V, const void* R,
    const uint8_t* ids, const float* vnorm, socket_dtype dtype, int32_t B,
    int32_t Hq, int32_t Hkv, int32_t d, int64_t n_keys,
    int64_t head_stride_rows, int32_t L, int32_t P, float tau, int64_t k,
    void* out, int32_t* idx_out, float* scores_out, void* workspace,
    size_t workspace_bytes, void* stream, void* const* events,
    int32_t n_events);

/*
 * The kernels socket_decode enqueues for these arguments, in launch order.
 * Host-only (no device work). With k < n_keys: the bucket table kernel
 * (only when the score kernel cannot build the tables itself, which it does
 * for bf16, P = 8, d in {64, 128}, L in {16, 32, 64}, 16-byte aligned id
 * rows and a table plus 16*P*L*G bytes of build state within the LDS), the
 * score kernel with candidate emission, the selection, the attention gather
 * and merge. With k >= n_keys: (table and score kernels only when
 * with_scores is nonzero) an index fill, the attention gather and merge.
 *   names  NULL, or cap bytes receiving the kernels' base names separated
 *          by commas, NUL-terminated
 * Returns the number of kernels; -1 for arguments socket_decode rejects
 * (socket_last_error() says why); -2 when the names do not fit in cap.
 */
int32_t socket_decode_kernels(const uint8_t* ids, socket_dtype dtype, int32_t B,
                              int32_t Hq, int32_t Hkv, int32_t d,
                              int64_t n_keys, int64_t head_stride_rows,
                              int32_t L, int32_t P, int64_t k,
                              int32_t with_scores, char* names, size_t cap);

#ifdef __cplusplus
}
#endif

#endif /* SOCKET_LSH_H */
