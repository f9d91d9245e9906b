// C ABI of the SOCKET decode library: host-side validation, workspace
// layout and kernel sequencing. Declarations and contracts are in
// include/socket_lsh.h.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "kernels.hpp"
#include "socket_lsh.h"

namespace {

using namespace socket_lsh;

thread_local std::string g_last_error;

socket_status fail(socket_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

socket_status ok() {
  g_last_error.clear();
  return SOCKET_OK;
}

socket_status from_hip(hipError_t err, const char* what) {
  if (err == hipSuccess) return ok();
  return fail(SOCKET_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

socket_status check_dtype(socket_dtype dt) {
  if (dt != SOCKET_DTYPE_F32 && dt != SOCKET_DTYPE_BF16)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dt);
  return SOCKET_OK;
}

socket_status check_d(int32_t d) {
  if (d <= 0) return fail(SOCKET_ERR_INVALID_ARGUMENT, "d must be > 0 (got %d)", d);
  if (d != 64 && d != 128)
    return fail(SOCKET_ERR_UNSUPPORTED, "d=%d is not supported (64 or 128)", d);
  return SOCKET_OK;
}

socket_status check_lp(int32_t L, int32_t P) {
  if (L < 1) return fail(SOCKET_ERR_INVALID_ARGUMENT, "L must be >= 1 (got %d)", L);
  if (P < 1 || P > 8)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "P must be in [1, 8] (got %d)", P);
  if ((int64_t)L * P > 1024)
    return fail(SOCKET_ERR_UNSUPPORTED, "L*P=%lld exceeds 1024 hyperplanes",
                (long long)L * P);
  return SOCKET_OK;
}

socket_status check_heads(int32_t B, int32_t Hq, int32_t Hkv) {
  if (B < 1 || Hq < 1 || Hkv < 1)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "B, Hq, Hkv must be >= 1 (got %d, %d, %d)",
                B, Hq, Hkv);
  if (Hq % Hkv != 0)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(SOCKET_ERR_UNSUPPORTED, "GQA group size %d is not supported (1, 2, 4, 8)", G);
  return SOCKET_OK;
}

// The score kernel holds the tables of Gp query heads of one KV head (the
// largest Gp dividing G that fits, see score_pack); fails only when not even
// one head's table fits.
socket_status check_table(int32_t L, int32_t P, int32_t G) {
  if (score_pack(L, P, G) == 0)
    return fail(SOCKET_ERR_UNSUPPORTED,
                "probability table of one query head (2^P*L*4 bytes) with the score "
                "kernel's other LDS (%zu bytes in all) exceeds the %zu bytes of LDS",
                score_lds_bytes(L, P, 1, false), kLdsBytesPerCU);
  return SOCKET_OK;
}

// Virtual KV heads of the score pipeline: Hkv * (G / Gp), see score_pack.
struct HeadPack {
  int gp;      // query heads per score block
  int np;      // packs per KV head (id divisor)
  int hkv_v;   // virtual KV heads
};
HeadPack head_pack(int32_t Hq, int32_t Hkv, int32_t L, int32_t P) {
  HeadPack hp{};
  const int G = Hq / Hkv;
  hp.gp = score_pack(L, P, G);
  if (hp.gp < 1) hp.gp = 1;
  hp.np = G / hp.gp;
  hp.hkv_v = Hkv * hp.np;
  return hp;
}

#define SOCKET_TRY(expr)                 \
  do {                                   \
    socket_status _st = (expr);          \
    if (_st != SOCKET_OK) return _st;    \
  } while (0)

struct DecodeLayout {
  size_t table_off, scores_off, idx_off, thr_off, cnt_off, list_off, bmax_off, attn_off, total;
  HeadPack pack;
  ScoreGeom score;
  AttnPlan attn;
};

// Workspace of one decode call: the probability tables, full score rows
// (written only for rows that need them; with large kk the rows' gathered
// candidates first), selected indices, block thresholds, candidate sub-list
// lengths and lists, the gather blocks' largest keys, attention partials.
DecodeLayout decode_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                           int64_t n_keys, int32_t L, int32_t P, int64_t k) {
  DecodeLayout lay{};
  const int rows = B * Hq;
  const int64_t kk = k < n_keys ? k : n_keys;
  const bool select = kk < n_keys;
  lay.pack = head_pack(Hq, Hkv, L, P);
  lay.score = plan_score(B * lay.pack.hkv_v, n_keys, L, P, lay.pack.gp);
  size_t off = 0;
  lay.table_off = off;
  off = align256(off + ((size_t)1 << P) * L * Hq * B * sizeof(float));
  lay.scores_off = off;
  off = align256(off + (select ? (size_t)rows * n_keys * sizeof(float) : 0));
  lay.idx_off = off;
  off = align256(off + (size_t)rows * kk * sizeof(int32_t));
  lay.thr_off = off;
  off = align256(off + (select ? (size_t)rows * lay.score.segs * sizeof(uint32_t) : 0));
  lay.cnt_off = off;
  off = align256(off + (select ? (size_t)rows * lay.score.subs * sizeof(uint32_t) : 0));
  lay.list_off = off;
  off = align256(off + (select ? (size_t)rows * n_keys * 8 : 0));
  lay.bmax_off = off;
  off = align256(off + (select ? (size_t)rows * select_gather_blocks(lay.score.subs, kk) * 4 : 0));
  lay.attn = plan_attn(B, Hq, Hkv, d, kk);
  lay.attn_off = off;
  off = align256(off + lay.attn.partial_bytes);
  lay.total = off;
  return lay;
}

}  // namespace

extern "C" {

int32_t socket_version(void) { return (0 << 16) | (1 << 8) | 0; }

const char* socket_status_string(socket_status status) {
  switch (status) {
    case SOCKET_OK: return "ok";
    case SOCKET_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SOCKET_ERR_UNSUPPORTED: return "unsupported configuration";
    case SOCKET_ERR_WORKSPACE: return "workspace missing or too small";
    case SOCKET_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* socket_last_error(void) { return g_last_error.c_str(); }

size_t socket_hash_keys_workspace_bytes(socket_dtype dtype, int64_t n_heads,
                                        int64_t n_keys, int32_t d, int32_t L,
                                        int32_t P) {
  if (dtype != SOCKET_DTYPE_BF16 || n_heads <= 0 || n_keys <= 0 || d <= 0 || L <= 0 ||
      P <= 0)
    return 0;
  return hash_keys_bf16_workspace_bytes(n_heads, n_keys, d, L * P);
}

socket_status socket_hash_keys(const void* K, const void* V, const void* R,
                               socket_dtype dtype, int64_t n_heads,
                               int64_t n_keys, int64_t head_stride_rows,
                               int32_t d, int32_t L, int32_t P, uint8_t* ids,
                               float* vnorm, void* workspace,
                               size_t workspace_bytes, void* stream) {
  SOCKET_TRY(check_dtype(dtype));
  SOCKET_TRY(check_d(d));
  SOCKET_TRY(check_lp(L, P));
  if (n_heads < 0 || n_keys < 0)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "n_heads and n_keys must be >= 0");
  if (head_stride_rows < n_keys)
    return fail(SOCKET_ERR_INVALID_ARGUMENT,
                "head_stride_rows (%lld) < n_keys (%lld)", (long long)head_stride_rows,
                (long long)n_keys);
  if (dtype == SOCKET_DTYPE_BF16 && (int64_t)L * P > 512)
    return fail(SOCKET_ERR_UNSUPPORTED,
                "bf16 hashing supports L*P <= 512 hyperplanes (got %lld)",
                (long long)L * P);
  if (n_heads == 0 || n_keys == 0) return ok();
  if (!K || !V || !R || !ids || !vnorm)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (!aligned16(K) || !aligned16(V) || !aligned16(R))
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "K, V and R must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (dtype == SOCKET_DTYPE_BF16) {
    if (n_heads * ((n_keys + 31) / 32) >= ((int64_t)1 << 31))
      return fail(SOCKET_ERR_UNSUPPORTED, "bf16 hashing supports < 2^31 tiles of 32 keys");
    const size_t need = hash_keys_bf16_workspace_bytes(n_heads, n_keys, d, L * P);
    if (!workspace || workspace_bytes < need ||
        (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
      return fail(SOCKET_ERR_WORKSPACE,
                  "hashing needs %zu workspace bytes at a 256-byte aligned address, got %zu",
                  need, workspace ? workspace_bytes : (size_t)0);
    err = launch_hash_keys_bf16((const uint16_t*)K, (const uint16_t*)V,
                                (const uint16_t*)R, n_heads, n_keys,
                                head_stride_rows, d, L, P, ids, vnorm, workspace, s);
  }
  else
    err = launch_hash_keys_f32((const float*)K, (const float*)V,
                               (const float*)R, n_heads, n_keys,
                               head_stride_rows, d, L, P, ids, vnorm, s);
  return from_hip(err, "socket_hash_keys launch");
}

socket_status socket_bucket_probs(const void* Q, const void* R,
                                  socket_dtype dtype, int32_t B, int32_t Hq,
                                  int32_t Hkv, int32_t d, int32_t L,
                                  int32_t P, float tau, float* table,
                                  void* stream) {
  SOCKET_TRY(check_dtype(dtype));
  SOCKET_TRY(check_heads(B, Hq, Hkv));
  SOCKET_TRY(check_d(d));
  SOCKET_TRY(check_lp(L, P));
  if (!(std::isfinite(tau) && tau > 0.f))
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "tau must be finite and > 0");
  if (!Q || !R || !table)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (!aligned16(R))
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "R must be 16-byte aligned");
  hipError_t err = launch_bucket_probs(Q, R, dtype == SOCKET_DTYPE_BF16, B, Hq,
                                       Hkv, d, L, P, tau, table,
                                       static_cast<hipStream_t>(stream));
  return from_hip(err, "socket_bucket_probs launch");
}

socket_status socket_hard_bucket_table(const void* Q, const void* R, socket_dtype dtype,
                                      int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t L,
                                      int32_t P, float* table, void* stream) {
  SOCKET_TRY(check_dtype(dtype));
  SOCKET_TRY(check_heads(B, Hq, Hkv));
  SOCKET_TRY(check_d(d));
  SOCKET_TRY(check_lp(L, P));
  if (!Q || !R || !table)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (!aligned16(R))
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "R must be 16-byte aligned");
  // tau = 0: 2 / tau = +inf makes every bit weight 1 or 0 (1/2 each for a
  // projection of exactly 0), the limit of the soft weights
  hipError_t err = launch_bucket_probs(Q, R, dtype == SOCKET_DTYPE_BF16, B, Hq, Hkv, d, L, P,
                                       0.0f, table, static_cast<hipStream_t>(stream));
  return from_hip(err, "socket_hard_bucket_table launch");
}

socket_status socket_score(const float* table, const uint8_t* ids,
                           const float* vnorm, int32_t B, int32_t Hq,
                           int32_t Hkv, int64_t n_keys,
                           int64_t head_stride_rows, int32_t L, int32_t P,
                           float* scores, void* stream) {
  SOCKET_TRY(check_heads(B, Hq, Hkv));
  SOCKET_TRY(check_lp(L, P));
  SOCKET_TRY(check_table(L, P, Hq / Hkv));
  if (n_keys < 0 || head_stride_rows < n_keys)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "need 0 <= n_keys <= head_stride_rows");
  if (n_keys == 0) return ok();
  if (!table || !ids || !vnorm || !scores)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (!aligned16(table))
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "table must be 16-byte aligned");
  const HeadPack hp = head_pack(Hq, Hkv, L, P);
  hipError_t err = launch_score(table, Hq / Hkv, ids, vnorm, B, Hq, hp.hkv_v, hp.np, n_keys,
                                head_stride_rows, L, P, scores, nullptr,
                                static_cast<hipStream_t>(stream));
  return from_hip(err, "socket_score launch");
}

size_t socket_topk_workspace_bytes(int32_t rows, int64_t n, int64_t k) {
  if (rows < 1 || n < 1 || k < 1) return 0;
  return plan_topk(rows, n, k).total_bytes;
}

socket_status socket_topk(const float* scores, int32_t rows, int64_t n,
                          int64_t k, int32_t* idx, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (rows < 0 || n < 0)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "rows and n must be >= 0");
  if (k < 1) return fail(SOCKET_ERR_INVALID_ARGUMENT, "k must be >= 1");
  if (n >= ((int64_t)1 << 31))
    return fail(SOCKET_ERR_UNSUPPORTED, "n must be < 2^31 (int32 indices)");
  if (rows == 0 || n == 0) return ok();
  if (!scores || !idx)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "null pointer argument");
  const TopkPlan plan = plan_topk(rows, n, k);
  if (plan.kk < n && (!workspace || workspace_bytes < plan.total_bytes))
    return fail(SOCKET_ERR_WORKSPACE, "top-k needs %zu workspace bytes, got %zu",
                plan.total_bytes, workspace ? workspace_bytes : (size_t)0);
  hipError_t err = launch_topk(scores, plan, idx, workspace,
                               static_cast<hipStream_t>(stream));
  return from_hip(err, "socket_topk launch");
}

size_t socket_sparse_attn_workspace_bytes(int32_t B, int32_t Hq, int32_t d,
                                          int64_t kk) {
  if (B < 1 || Hq < 1 || d < 1 || kk < 1) return 0;
  return plan_attn(B, Hq, Hq, d, kk).partial_bytes;
}

socket_status socket_sparse_attn(const void* Q, const void* K, const void* V,
                                 socket_dtype dtype, int32_t B, int32_t Hq,
                                 int32_t Hkv, int32_t d,
                                 int64_t head_stride_rows, const int32_t* idx,
                                 int64_t kk, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  SOCKET_TRY(check_dtype(dtype));
  SOCKET_TRY(check_heads(B, Hq, Hkv));
  SOCKET_TRY(check_d(d));
  if (kk < 1) return fail(SOCKET_ERR_INVALID_ARGUMENT, "kk must be >= 1");
  if (kk > kMaxSelected)
    return fail(SOCKET_ERR_UNSUPPORTED, "at most %lld selected keys per row",
                (long long)kMaxSelected);
  if (head_stride_rows < 1)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "head_stride_rows must be >= 1");
  if (head_stride_rows >= ((int64_t)1 << 31))
    return fail(SOCKET_ERR_UNSUPPORTED, "head_stride_rows must be < 2^31");
  if (!Q || !K || !V || !idx || !out)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V))
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "Q, K and V must be 16-byte aligned");
  const AttnPlan plan = plan_attn(B, Hq, Hkv, d, kk);
  if (!workspace || workspace_bytes < plan.partial_bytes)
    return fail(SOCKET_ERR_WORKSPACE, "attention needs %zu workspace bytes, got %zu",
                plan.partial_bytes, workspace ? workspace_bytes : (size_t)0);
  hipError_t err = launch_sparse_attn(Q, K, V, dtype == SOCKET_DTYPE_BF16, plan,
                                      head_stride_rows, idx, out,
                                      static_cast<float*>(workspace),
                                      static_cast<hipStream_t>(stream));
  return from_hip(err, "socket_sparse_attn launch");
}

size_t socket_dense_attn_workspace_bytes(int32_t B, int32_t Hq, int32_t d, int64_t n) {
  if (B < 1 || Hq < 1 || d < 1 || n < 1) return 0;
  return plan_dense(B, Hq, Hq, d, n).partial_bytes;
}

socket_status socket_dense_attn(const void* Q, const void* K, const void* V,
                                socket_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                int32_t d, int64_t n, int64_t head_stride_rows, void* out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  SOCKET_TRY(check_dtype(dtype));
  SOCKET_TRY(check_heads(B, Hq, Hkv));
  SOCKET_TRY(check_d(d));
  if (Hq / Hkv > 8)
    return fail(SOCKET_ERR_UNSUPPORTED, "dense attention takes at most 8 query heads per KV head");
  if (n < 1) return fail(SOCKET_ERR_INVALID_ARGUMENT, "n must be >= 1");
  if (n > kMaxDenseKeys)
    return fail(SOCKET_ERR_UNSUPPORTED, "dense attention takes at most %lld keys",
                (long long)kMaxDenseKeys);
  if (head_stride_rows < n)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "head_stride_rows (%lld) < n (%lld)",
                (long long)head_stride_rows, (long long)n);
  if (!Q || !K || !V || !out)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V))
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "Q, K and V must be 16-byte aligned");
  const DensePlan plan = plan_dense(B, Hq, Hkv, d, n);
  if (!workspace || workspace_bytes < plan.partial_bytes)
    return fail(SOCKET_ERR_WORKSPACE, "dense attention needs %zu workspace bytes, got %zu",
                plan.partial_bytes, workspace ? workspace_bytes : (size_t)0);
  hipError_t err = launch_dense_attn(Q, K, V, dtype == SOCKET_DTYPE_BF16, plan, head_stride_rows,
                                     nullptr, out, static_cast<float*>(workspace),
                                     static_cast<hipStream_t>(stream));
  return from_hip(err, "socket_dense_attn launch");
}

size_t socket_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv,
                                     int32_t d, int64_t n_keys, int32_t L,
                                     int32_t P, int64_t k) {
  if (B < 1 || Hq < 1 || Hkv < 1 || d < 1 || n_keys < 1 || L < 1 || P < 1 ||
      P > 8 || k < 1)
    return 0;
  return decode_layout(B, Hq, Hkv, d, n_keys, L, P, k).total;
}

}  // extern "C"

namespace {

// The candidate sub-lists the selection of one row reads must fit its
// offsets: checked on the geometry the score kernel is launched with.
socket_status check_sublists(const ScoreGeom& geo, int64_t n_keys, int64_t k) {
  if (k < n_keys && geo.subs > kMaxSelectSubLists)
    return fail(SOCKET_ERR_UNSUPPORTED, "n_keys=%lld needs %d candidate sub-lists per row "
                "(at most %d)", (long long)n_keys, geo.subs, kMaxSelectSubLists);
  return SOCKET_OK;
}

// Shapes and sizes both decode entry points accept (pointers, tau and the
// score geometry aside).
socket_status check_decode_common(socket_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                  int32_t d, int64_t n_keys, int64_t head_stride_rows, int32_t L,
                                  int32_t P, int64_t k) {
  SOCKET_TRY(check_dtype(dtype));
  SOCKET_TRY(check_heads(B, Hq, Hkv));
  SOCKET_TRY(check_d(d));
  SOCKET_TRY(check_lp(L, P));
  if (k < 1) return fail(SOCKET_ERR_INVALID_ARGUMENT, "k must be >= 1");
  if (n_keys < 1) return fail(SOCKET_ERR_INVALID_ARGUMENT, "n_keys must be >= 1");
  if ((k < n_keys ? k : n_keys) > kMaxSelected)
    return fail(SOCKET_ERR_UNSUPPORTED, "at most %lld selected keys per row",
                (long long)kMaxSelected);
  if (head_stride_rows < n_keys)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "head_stride_rows (%lld) < n_keys (%lld)",
                (long long)head_stride_rows, (long long)n_keys);
  if (head_stride_rows >= ((int64_t)1 << 31))
    return fail(SOCKET_ERR_UNSUPPORTED, "head_stride_rows must be < 2^31");
  return SOCKET_OK;
}

// Shapes and sizes socket_decode accepts (pointers and tau aside).
socket_status check_decode(socket_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                           int64_t n_keys, int64_t head_stride_rows, int32_t L, int32_t P,
                           int64_t k) {
  SOCKET_TRY(check_decode_common(dtype, B, Hq, Hkv, d, n_keys, head_stride_rows, L, P, k));
  SOCKET_TRY(check_table(L, P, Hq / Hkv));
  const HeadPack hp = head_pack(Hq, Hkv, L, P);
  return check_sublists(plan_score(B * hp.hkv_v, n_keys, L, P, hp.gp), n_keys, k);
}

socket_status decode_impl(const void* Q, const void* K, const void* V,
                          const void* R, const uint8_t* ids,
                          const float* vnorm, socket_dtype dtype, int32_t B,
                          int32_t Hq, int32_t Hkv, int32_t d, int64_t n_keys,
                          int64_t head_stride_rows, int32_t L, int32_t P,
                          float tau, int64_t k, void* out, int32_t* idx_out,
                          float* scores_out, void* workspace,
                          size_t workspace_bytes, void* stream,
                          void* const* events, int32_t n_events) {
  SOCKET_TRY(check_decode(dtype, B, Hq, Hkv, d, n_keys, head_stride_rows, L, P, k));
  if (!(std::isfinite(tau) && tau > 0.f))
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "tau must be finite and > 0");
  if (!Q || !K || !V || !R || !ids || !vnorm || !out)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(R))
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "Q, K, V and R must be 16-byte aligned");
  const DecodeLayout lay = decode_layout(B, Hq, Hkv, d, n_keys, L, P, k);
  if (!workspace || workspace_bytes < lay.total)
    return fail(SOCKET_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu",
                lay.total, workspace ? workspace_bytes : (size_t)0);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (events != nullptr && n_events < 2)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "n_events must be >= 2 with events");
  LaunchTrace trace{reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)),
                    events ? n_events : 0, 0};
  struct TraceScope {
    explicit TraceScope(LaunchTrace* t) { g_trace = t; }
    ~TraceScope() { g_trace = nullptr; }
  } scope(events ? &trace : nullptr);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* table = reinterpret_cast<float*>(ws + lay.table_off);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + lay.idx_off);
  float* partial = reinterpret_cast<float*>(ws + lay.attn_off);
  const bool bf16 = dtype == SOCKET_DTYPE_BF16;

  // Selection: the score kernel estimates per-block thresholds and emits
  // the keys that reach them; one block per row then selects the kk best
  // (from the candidates, or from the full row).
  const int rows = B * Hq;
  const int64_t kk = k < n_keys ? k : n_keys;
  // the score kernel builds the tables itself where it can (no table kernel);
  // the score pipeline runs over Hv virtual KV heads of Gp query heads each
  const HeadPack hp = lay.pack;
  const int Hv = hp.hkv_v;
  const bool build = score_builds_table(bf16, d, ids, head_stride_rows, L, P, hp.gp);
  const TableBuild tb{Q, R, d, tau};
  hipError_t err;
  if (kk < n_keys) {
    uint32_t* thr = reinterpret_cast<uint32_t*>(ws + lay.thr_off);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + lay.cnt_off);
    uint2* lists = reinterpret_cast<uint2*>(ws + lay.list_off);
    float* rowbuf = scores_out ? scores_out : reinterpret_cast<float*>(ws + lay.scores_off);
    if (!build) {
      err = launch_bucket_probs(Q, R, bf16, B, Hq, Hv, d, L, P, tau, table, s);
      if (err != hipSuccess) return from_hip(err, "socket_decode: bucket_probs");
    }
    ScoreSelect sel{};
    sel.table = table;
    sel.id_div = hp.np;
    sel.ids = ids;
    sel.vnorm = vnorm;
    sel.kk = kk;
    sel.thr = thr;
    sel.lists = lists;
    sel.sub_cnt = cnt;
    err = launch_score_select(sel, B, Hq, Hv, n_keys, head_stride_rows, L, P, scores_out,
                              build ? &tb : nullptr, s);
    if (err != hipSuccess) return from_hip(err, "socket_decode: score");
    SelectArgs sa{};
    sa.n = n_keys;
    sa.kk = kk;
    sa.subs = lay.score.subs;
    sa.sub_len = lay.score.sub_len;
    sa.skew0 = lay.score.skew0;
    sa.skew1 = lay.score.skew1;
    sa.segs = lay.score.segs;
    sa.thr = thr;
    sa.lists = lists;
    sa.sub_cnt = cnt;
    sa.idx = idx;
    sa.table = table;
    sa.ids = ids;
    sa.vnorm = vnorm;
    sa.Hq = Hq;
    sa.Hkv = Hv;
    sa.id_div = hp.np;
    sa.L = L;
    sa.P = P;
    sa.stride = head_stride_rows;
    sa.rotated = score_rotated(ids, head_stride_rows, L) ? 1 : 0;
    sa.region = sa.rotated && score_region(sa.Hq / sa.Hkv, P, L) ? 1 : 0;
    sa.scores = rowbuf;
    sa.spill = reinterpret_cast<uint2*>(ws + lay.scores_off);
    sa.bmax = reinterpret_cast<uint32_t*>(ws + lay.bmax_off);
    err = launch_topk_select(sa, rows, s);
    if (err != hipSuccess) return from_hip(err, "socket_decode: topk");
  } else {
    if (scores_out) {
      if (!build) {
        err = launch_bucket_probs(Q, R, bf16, B, Hq, Hv, d, L, P, tau, table, s);
        if (err != hipSuccess) return from_hip(err, "socket_decode: bucket_probs");
      }
      err = launch_score(table, hp.gp, ids, vnorm, B, Hq, Hv, hp.np, n_keys, head_stride_rows,
                         L, P, scores_out, build ? &tb : nullptr, s);
      if (err != hipSuccess) return from_hip(err, "socket_decode: score");
    }
    err = launch_iota_rows(idx, rows, n_keys, s);
    if (err != hipSuccess) return from_hip(err, "socket_decode: topk");
  }
  err = launch_sparse_attn(Q, K, V, bf16, lay.attn, head_stride_rows, idx, out,
                           partial, s);
  return from_hip(err, "socket_decode: sparse_attn");
}

// GQA group-shared variant: the per-KV-head decode layout (one score row
// per KV head, G = 1 over the group table) plus the heads' full table and
// the attention partials of the Hq query rows over the kk shared keys.
struct GroupLayout {
  DecodeLayout head;   // B rows of Hkv, "G = 1"
  size_t full_table_off, attn_off, total;
  DensePlan attn;
};

GroupLayout group_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t n_keys,
                         int32_t L, int32_t P, int64_t k) {
  GroupLayout g{};
  g.head = decode_layout(B, Hkv, Hkv, d, n_keys, L, P, k);
  size_t off = g.head.total;
  g.full_table_off = off;
  off = align256(off + ((size_t)1 << P) * L * Hq * B * sizeof(float));
  const int64_t kk = k < n_keys ? k : n_keys;
  g.attn = plan_dense(B, Hq, Hkv, d, kk);
  g.attn_off = off;
  off = align256(off + g.attn.partial_bytes);
  g.total = off;
  return g;
}

// Shapes the group-shared variant accepts: its score and selection run at
// one (summed) table per KV head, so both the LDS and the sub-list checks
// use that geometry.
socket_status check_group_decode(socket_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                 int32_t d, int64_t n_keys, int64_t head_stride_rows, int32_t L,
                                 int32_t P, int64_t k) {
  SOCKET_TRY(check_decode_common(dtype, B, Hq, Hkv, d, n_keys, head_stride_rows, L, P, k));
  SOCKET_TRY(check_table(L, P, 1));
  return check_sublists(plan_score(B * Hkv, n_keys, L, P, 1), n_keys, k);
}

socket_status decode_group_impl(const void* Q, const void* K, const void* V, const void* R,
                                const uint8_t* ids, const float* vnorm, socket_dtype dtype,
                                int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t n_keys,
                                int64_t head_stride_rows, int32_t L, int32_t P, float tau,
                                int64_t k, void* out, int32_t* idx_out, float* scores_out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  SOCKET_TRY(check_group_decode(dtype, B, Hq, Hkv, d, n_keys, head_stride_rows, L, P, k));
  if (!(std::isfinite(tau) && tau > 0.f))
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "tau must be finite and > 0");
  if (!Q || !K || !V || !R || !ids || !vnorm || !out)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(R))
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "Q, K, V and R must be 16-byte aligned");
  if (Hq / Hkv > 8)
    return fail(SOCKET_ERR_UNSUPPORTED, "at most 8 query heads per KV head");
  const int64_t kk = k < n_keys ? k : n_keys;
  if (kk > kMaxDenseKeys)
    return fail(SOCKET_ERR_UNSUPPORTED, "at most %lld selected keys", (long long)kMaxDenseKeys);
  const GroupLayout lay = group_layout(B, Hq, Hkv, d, n_keys, L, P, k);
  if (!workspace || workspace_bytes < lay.total)
    return fail(SOCKET_ERR_WORKSPACE, "group-shared decode needs %zu workspace bytes, got %zu",
                lay.total, workspace ? workspace_bytes : (size_t)0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* full = reinterpret_cast<float*>(ws + lay.full_table_off);
  float* gtable = reinterpret_cast<float*>(ws + lay.head.table_off);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + lay.head.idx_off);
  const bool bf16 = dtype == SOCKET_DTYPE_BF16;
  const int G = Hq / Hkv;
  const int rows = B * Hkv;
  hipError_t err = launch_bucket_probs(Q, R, bf16, B, Hq, Hkv, d, L, P, tau, full, s);
  if (err != hipSuccess) return from_hip(err, "group-shared decode: bucket_probs");
  err = launch_group_table_sum(full, B * Hkv, L, P, G, gtable, s);
  if (err != hipSuccess) return from_hip(err, "group-shared decode: group table");
  if (kk < n_keys) {
    // the per-head pipeline at G = 1 over the group tables
    uint32_t* thr = reinterpret_cast<uint32_t*>(ws + lay.head.thr_off);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + lay.head.cnt_off);
    uint2* lists = reinterpret_cast<uint2*>(ws + lay.head.list_off);
    float* rowbuf = scores_out ? scores_out : reinterpret_cast<float*>(ws + lay.head.scores_off);
    ScoreSelect sel{};
    sel.table = gtable;
    sel.id_div = 1;
    sel.ids = ids;
    sel.vnorm = vnorm;
    sel.kk = kk;
    sel.thr = thr;
    sel.lists = lists;
    sel.sub_cnt = cnt;
    err = launch_score_select(sel, B, Hkv, Hkv, n_keys, head_stride_rows, L, P, scores_out,
                              nullptr, s);
    if (err != hipSuccess) return from_hip(err, "group-shared decode: score");
    SelectArgs sa{};
    sa.n = n_keys;
    sa.kk = kk;
    sa.subs = lay.head.score.subs;
    sa.sub_len = lay.head.score.sub_len;
    sa.skew0 = lay.head.score.skew0;
    sa.skew1 = lay.head.score.skew1;
    sa.segs = lay.head.score.segs;
    sa.thr = thr;
    sa.lists = lists;
    sa.sub_cnt = cnt;
    sa.idx = idx;
    sa.table = gtable;
    sa.ids = ids;
    sa.vnorm = vnorm;
    sa.Hq = Hkv;
    sa.Hkv = Hkv;
    sa.id_div = 1;
    sa.L = L;
    sa.P = P;
    sa.stride = head_stride_rows;
    sa.rotated = score_rotated(ids, head_stride_rows, L) ? 1 : 0;
    sa.region = sa.rotated && score_region(sa.Hq / sa.Hkv, P, L) ? 1 : 0;
    sa.scores = rowbuf;
    sa.spill = reinterpret_cast<uint2*>(ws + lay.head.scores_off);
    sa.bmax = reinterpret_cast<uint32_t*>(ws + lay.head.bmax_off);
    err = launch_topk_select(sa, rows, s);
    if (err != hipSuccess) return from_hip(err, "group-shared decode: topk");
  } else {
    if (scores_out) {
      err = launch_score(gtable, 1, ids, vnorm, B, Hkv, Hkv, 1, n_keys, head_stride_rows, L, P,
                         scores_out, nullptr, s);
      if (err != hipSuccess) return from_hip(err, "group-shared decode: score");
    }
    err = launch_iota_rows(idx, rows, n_keys, s);
    if (err != hipSuccess) return from_hip(err, "group-shared decode: topk");
  }
  err = launch_dense_attn(Q, K, V, bf16, lay.attn, head_stride_rows, idx, out,
                          reinterpret_cast<float*>(ws + lay.attn_off), s);
  return from_hip(err, "group-shared decode: attention");
}

}  // namespace

extern "C" {

size_t socket_decode_group_shared_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                                  int64_t n_keys, int32_t L, int32_t P,
                                                  int64_t k) {
  if (B < 1 || Hq < 1 || Hkv < 1 || d < 1 || n_keys < 1 || L < 1 || P < 1 || P > 8 || k < 1)
    return 0;
  return group_layout(B, Hq, Hkv, d, n_keys, L, P, k).total;
}

socket_status socket_decode_group_shared(const void* Q, const void* K, const void* V,
                                         const void* R, const uint8_t* ids, const float* vnorm,
                                         socket_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                         int32_t d, int64_t n_keys, int64_t head_stride_rows,
                                         int32_t L, int32_t P, float tau, int64_t k, void* out,
                                         int32_t* idx_out, float* scores_out, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  return decode_group_impl(Q, K, V, R, ids, vnorm, dtype, B, Hq, Hkv, d, n_keys,
                           head_stride_rows, L, P, tau, k, out, idx_out, scores_out, workspace,
                           workspace_bytes, stream);
}

socket_status socket_decode(const void* Q, const void* K, const void* V,
                            const void* R, const uint8_t* ids,
                            const float* vnorm, socket_dtype dtype, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t d,
                            int64_t n_keys, int64_t head_stride_rows,
                            int32_t L, int32_t P, float tau, int64_t k,
                            void* out, int32_t* idx_out, float* scores_out,
                            void* workspace, size_t workspace_bytes,
                            void* stream) {
  return decode_impl(Q, K, V, R, ids, vnorm, dtype, B, Hq, Hkv, d, n_keys,
                     head_stride_rows, L, P, tau, k, out, idx_out, scores_out,
                     workspace, workspace_bytes, stream, nullptr, 0);
}

socket_status socket_decode_profiled(
    const void* Q, const void* K, const void* V, const void* R,
    const uint8_t* ids, const float* vnorm, socket_dtype dtype, int32_t B,
    int32_t Hq, int32_t Hkv, int32_t d, int64_t n_keys,
    int64_t head_stride_rows, int32_t L, int32_t P, float tau, int64_t k,
    void* out, int32_t* idx_out, float* scores_out, void* workspace,
    size_t workspace_bytes, void* stream, void* const* events,
    int32_t n_events) {
  if (events == nullptr)
    return fail(SOCKET_ERR_INVALID_ARGUMENT, "events must not be NULL");
  return decode_impl(Q, K, V, R, ids, vnorm, dtype, B, Hq, Hkv, d, n_keys,
                     head_stride_rows, L, P, tau, k, out, idx_out, scores_out,
                     workspace, workspace_bytes, stream, events, n_events);
}

}  // extern "C"

// ----------------------------------------------------- allocation-free decode
// The decode workspace in a device array of the library instead of caller
// memory. Every GPU the library runs on holds its own copy of the array (at
// its own address) until the process ends. In host code the array's name is
// only a stand-in: the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is used.
namespace {

static __device__ __align__(256) unsigned char scratch[SOCKET_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the array (resolved on the first call there).
socket_status current_scratch(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return from_hip(err, "socket_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SOCKET_ERR_UNSUPPORTED, "socket_decode_noalloc: device %d beyond the %d the "
                "library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr)
      return from_hip(err != hipSuccess ? err : hipErrorInvalidSymbol,
                      "socket_decode_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SOCKET_OK;
}

}  // namespace

extern "C" {

socket_status socket_decode_noalloc(const void* Q, const void* K, const void* V, const void* R,
                                    const uint8_t* ids, const float* vnorm, socket_dtype dtype,
                                    int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                    int64_t n_keys, int64_t head_stride_rows, int32_t L,
                                    int32_t P, float tau, int64_t k, void* out,
                                    int32_t* idx_out, float* scores_out, void* stream) {
  // shapes first (the workspace size below is only meaningful for them)
  SOCKET_TRY(check_decode(dtype, B, Hq, Hkv, d, n_keys, head_stride_rows, L, P, k));
  const size_t need = decode_layout(B, Hq, Hkv, d, n_keys, L, P, k).total;
  if (need > (size_t)SOCKET_DECODE_NOALLOC_SCRATCH_BYTES)
    return fail(SOCKET_ERR_UNSUPPORTED,
                "socket_decode_noalloc: this call needs %zu bytes of workspace, more than "
                "the library's %zu-byte device array (use socket_decode with a workspace)",
                need, (size_t)SOCKET_DECODE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  SOCKET_TRY(current_scratch(&ws));
  return decode_impl(Q, K, V, R, ids, vnorm, dtype, B, Hq, Hkv, d, n_keys, head_stride_rows, L,
                     P, tau, k, out, idx_out, scores_out, ws,
                     (size_t)SOCKET_DECODE_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0);
}

int32_t socket_decode_kernels(const uint8_t* ids, socket_dtype dtype, int32_t B,
                              int32_t Hq, int32_t Hkv, int32_t d,
                              int64_t n_keys, int64_t head_stride_rows,
                              int32_t L, int32_t P, int64_t k,
                              int32_t with_scores, char* names, size_t cap) {
  if (check_decode(dtype, B, Hq, Hkv, d, n_keys, head_stride_rows, L, P, k) != SOCKET_OK)
    return -1;
  const bool build = score_builds_table(dtype == SOCKET_DTYPE_BF16, d, ids, head_stride_rows,
                                        L, P, head_pack(Hq, Hkv, L, P).gp);
  // the launch sequence of decode_impl
  const char* seq[7];
  int n = 0;
  if (k < n_keys) {
    if (!build) seq[n++] = "bucket_probs_kernel";
    seq[n++] = "score_kernel";
    if (select_gather_blocks(decode_layout(B, Hq, Hkv, d, n_keys, L, P, k).score.subs, k) > 0)
      seq[n++] = "topk_gather_kernel";
    seq[n++] = "topk_select_kernel";
  } else {
    if (with_scores) {
      if (!build) seq[n++] = "bucket_probs_kernel";
      seq[n++] = "score_kernel";
    }
    seq[n++] = "iota_rows_kernel";
  }
  seq[n++] = "sparse_attn_kernel";
  if (decode_layout(B, Hq, Hkv, d, n_keys, L, P, k).attn.chunks > 1)
    seq[n++] = "attn_merge_kernel";
  if (names) {
    std::string joined;
    for (int i = 0; i < n; ++i) {
      if (i) joined += ',';
      joined += seq[i];
    }
    if (joined.size() + 1 > cap) return -2;
    std::memcpy(names, joined.c_str(), joined.size() + 1);
  }
  return n;
}

}  // extern "C"

namespace socket_lsh {
thread_local LaunchTrace* g_trace = nullptr;
}  // namespace socket_lsh
