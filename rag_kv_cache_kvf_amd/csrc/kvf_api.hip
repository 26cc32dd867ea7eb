// libkvfuse C ABI: argument validation and dispatch to the HIP launchers.
//
// Every entry point validates on the host before anything is enqueued, maps
// failures to kvf_status, records a thread-local message, and never lets a
// C++ exception cross the interface.
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <exception>

#include "kvf_common.h"

namespace {

thread_local char g_err[512] = "";

kvf_status fail(kvf_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kvf_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_err[0] = '\0';
    return KVF_OK;
  }
  return fail(KVF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// KVF_SYNC_CHECK=1 in the environment (read once): after a call has
// enqueued its kernels, synchronise its stream and report any launch or
// execution error of those kernels as that call's KVF_ERR_HIP.  A debugging
// aid: it serialises the host with the GPU, and is skipped on a stream that
// is being captured into a graph (synchronising one is illegal).
bool sync_check_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("KVF_SYNC_CHECK");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
  }();
  return on;
}

kvf_status finish(hipError_t e, hipStream_t st, const char* what) {
  if (e == hipSuccess && sync_check_enabled()) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(st, &cs);
    if (e == hipSuccess && cs == hipStreamCaptureStatusNone) {
      e = hipStreamSynchronize(st);
      if (e == hipSuccess) e = hipGetLastError();
    }
  }
  return from_hip(e, what);
}

#define KVF_CHECK(cond, st, ...)            \
  do {                                      \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

kvf_status check_layer(const kvf_layer_desc* L) {
  KVF_CHECK(L != nullptr, KVF_ERR_INVALID_ARG, "layer descriptor is NULL");
  KVF_CHECK(L->hidden > 0 && L->n_q_heads > 0 && L->n_kv_heads > 0 && L->head_dim > 0,
            KVF_ERR_INVALID_ARG, "layer sizes must be positive");
  KVF_CHECK(L->dtype == KVF_F32 || L->dtype == KVF_BF16, KVF_ERR_INVALID_ARG,
            "dtype %d is not a kvf_dtype", L->dtype);
  KVF_CHECK(L->n_q_heads % L->n_kv_heads == 0, KVF_ERR_UNSUPPORTED,
            "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", L->n_q_heads, L->n_kv_heads);
  KVF_CHECK(L->head_dim == 64 || L->head_dim == 128, KVF_ERR_UNSUPPORTED,
            "head_dim %d unsupported (64 or 128)", L->head_dim);
  KVF_CHECK(L->n_q_heads / L->n_kv_heads <= 64, KVF_ERR_UNSUPPORTED,
            "more than 64 query heads per kv head");
  KVF_CHECK(L->hidden % 64 == 0, KVF_ERR_UNSUPPORTED, "hidden %d must be a multiple of 64",
            L->hidden);
  KVF_CHECK((static_cast<int64_t>(L->n_q_heads) + 2 * L->n_kv_heads) * L->head_dim < (1 << 30),
            KVF_ERR_UNSUPPORTED, "layer too wide");
  return KVF_OK;
}

kvf_status check_batch(const kvf_batch* b, kvf::BatchArgs* out) {
  KVF_CHECK(b != nullptr, KVF_ERR_INVALID_ARG, "batch is NULL");
  KVF_CHECK(b->n_req >= 1 && b->n_req <= KVF_MAX_REQ, KVF_ERR_INVALID_ARG,
            "n_req %d outside [1, %d]", b->n_req, KVF_MAX_REQ);
  KVF_CHECK(b->cu_T != nullptr && b->n_ctx != nullptr, KVF_ERR_INVALID_ARG,
            "batch arrays are NULL");
  KVF_CHECK(b->cu_T[0] == 0, KVF_ERR_INVALID_ARG, "cu_T[0] must be 0");
  std::memset(out, 0, sizeof(*out));
  out->n_req = b->n_req;
  for (int r = 0; r < b->n_req; ++r) {
    const int T = b->cu_T[r + 1] - b->cu_T[r];
    KVF_CHECK(b->cu_T[r + 1] >= b->cu_T[r], KVF_ERR_INVALID_ARG, "cu_T decreases at %d", r);
    KVF_CHECK(b->n_ctx[r] >= 0 && b->n_ctx[r] <= T, KVF_ERR_INVALID_ARG,
              "n_ctx[%d] = %d outside [0, %d]", r, b->n_ctx[r], T);
    out->cu_T[r + 1] = b->cu_T[r + 1];
    out->n_ctx[r] = b->n_ctx[r];
    out->cu_N[r + 1] = out->cu_N[r] + b->n_ctx[r];
    out->cu_U[r + 1] = out->cu_U[r] + (T - b->n_ctx[r]);
  }
  return KVF_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// an int8-resident fused cache of at least `min_rows` rows
kvf_status check_q8(const kvf_q8_cache* c, int64_t min_rows) {
  KVF_CHECK(c != nullptr, KVF_ERR_INVALID_ARG, "kvf_q8_cache is NULL");
  KVF_CHECK(c->k_codes && c->v_codes && c->k_stats && c->v_stats, KVF_ERR_INVALID_ARG,
            "incomplete kvf_q8_cache");
  KVF_CHECK(c->rows >= min_rows, KVF_ERR_INVALID_ARG, "kvf_q8_cache holds %lld rows, need %lld",
            static_cast<long long>(c->rows), static_cast<long long>(min_rows));
  return KVF_OK;
}

}  // namespace

#define KVF_GUARD_BEGIN try {
#define KVF_GUARD_END                                                   \
  }                                                                     \
  catch (const std::exception& e) {                                     \
    return fail(KVF_ERR_INVALID_ARG, "internal error: %s", e.what());   \
  }                                                                     \
  catch (...) {                                                         \
    return fail(KVF_ERR_INVALID_ARG, "internal error");                 \
  }

extern "C" {

int32_t kvf_abi_version(void) { return KVF_ABI_VERSION; }

const char* kvf_status_string(kvf_status s) {
  switch (s) {
    case KVF_OK: return "KVF_OK";
    case KVF_ERR_INVALID_ARG: return "KVF_ERR_INVALID_ARG";
    case KVF_ERR_UNSUPPORTED: return "KVF_ERR_UNSUPPORTED";
    case KVF_ERR_WORKSPACE: return "KVF_ERR_WORKSPACE";
    case KVF_ERR_HIP: return "KVF_ERR_HIP";
  }
  return "KVF_UNKNOWN_STATUS";
}

const char* kvf_last_error(void) { return g_err; }

int32_t kvf_recompute_budget(int32_t n_ctx, int32_t ratio_pct) {
  if (n_ctx < 0 || ratio_pct < 0 || ratio_pct > 100) return -1;
  return static_cast<int32_t>((static_cast<int64_t>(n_ctx) * ratio_pct) / 100);
}

int32_t kvf_anchor_budget(int32_t len, int32_t ra_num, int32_t ra_den) {
  if (len < 0 || ra_den <= 0 || ra_num < 0 || ra_num > ra_den) return -1;
  const int64_t num = static_cast<int64_t>(len) * ra_num;
  return static_cast<int32_t>((num + ra_den - 1) / ra_den);
}

kvf_status kvf_rope_table(double base, int32_t head_dim, int32_t n_pos, float* cos_tab,
                          float* sin_tab, void* stream) {
  KVF_GUARD_BEGIN
  KVF_CHECK(base > 1.0, KVF_ERR_INVALID_ARG, "rope base must exceed 1");
  KVF_CHECK(head_dim > 0 && head_dim % 2 == 0 && head_dim <= 1024, KVF_ERR_INVALID_ARG,
            "head_dim %d must be even and at most 1024", head_dim);
  KVF_CHECK(n_pos >= 0, KVF_ERR_INVALID_ARG, "n_pos negative");
  if (n_pos == 0) return KVF_OK;
  KVF_CHECK(cos_tab && sin_tab, KVF_ERR_INVALID_ARG, "table pointers are NULL");
  return finish(kvf::launch_rope_table(base, head_dim, n_pos, cos_tab, sin_tab,
                                         as_stream(stream)),
                as_stream(stream), "kvf_rope_table");
  KVF_GUARD_END
}

namespace {

// kvf_rerotate's checks and launch; dev (optional) adds the deviation score
// of kvf_rerotate_deviation, whose own checks the caller has made.
kvf_status rerotate_impl(const kvf_layer_desc* layer, const kvf_chunk* chunks, int32_t n_chunks,
                         int32_t max_chunk_len, const void* pool_k, const void* pool_v,
                         const kvf_kivi* kivi, int64_t pool_rows, const float* rope_cos,
                         const float* rope_sin, int32_t rope_n_pos, void* fused_k, void* fused_v,
                         int64_t fused_rows, int32_t k_only, const kvf::RotDeviation* dev,
                         void* stream, const char* name) {
  KVF_CHECK(n_chunks >= 0 && max_chunk_len >= 0 && pool_rows >= 0 && fused_rows >= 0 &&
                rope_n_pos >= 0, KVF_ERR_INVALID_ARG, "negative size");
  KVF_CHECK(k_only == 0 || k_only == 1, KVF_ERR_INVALID_ARG, "k_only must be 0 or 1");
  if (n_chunks == 0 || max_chunk_len == 0) return KVF_OK;
  KVF_CHECK(chunks && rope_cos && rope_sin && fused_k && (k_only || fused_v), KVF_ERR_INVALID_ARG,
            "required pointer is NULL");
  if (k_only) {
    KVF_CHECK(kivi == nullptr, KVF_ERR_UNSUPPORTED,
              "keys-only re-positioning reads a dense cache (KIVI codes decode to new buffers)");
    KVF_CHECK(pool_k != nullptr, KVF_ERR_INVALID_ARG, "pool_k is NULL");
  } else if (kivi) {
    KVF_CHECK(layer->dtype == KVF_BF16, KVF_ERR_UNSUPPORTED, "KIVI caches decode to bf16 only");
    KVF_CHECK(kivi->bits == 8 || kivi->bits == 4, KVF_ERR_UNSUPPORTED,
              "KIVI codes are 8 or 4 bits, not %d", kivi->bits);
    KVF_CHECK(pool_k == nullptr && pool_v == nullptr, KVF_ERR_INVALID_ARG,
              "pass either dense pool pointers or kivi, not both");
    KVF_CHECK(kivi->k_codes && kivi->v_codes && kivi->k_min && kivi->k_scale && kivi->v_min &&
                  kivi->v_scale && kivi->n_pool_chunks > 0, KVF_ERR_INVALID_ARG,
              "incomplete kvf_kivi");
  } else {
    KVF_CHECK(pool_k && pool_v, KVF_ERR_INVALID_ARG, "pool pointers are NULL");
  }
  KVF_CHECK(max_chunk_len <= (1 << 24), KVF_ERR_UNSUPPORTED, "max_chunk_len too large");
  return finish(kvf::launch_rerotate(*layer, chunks, n_chunks, max_chunk_len, pool_k, pool_v,
                                       kivi, pool_rows, rope_cos, rope_sin, rope_n_pos, fused_k,
                                       fused_v, fused_rows, k_only, as_stream(stream), dev),
                as_stream(stream), name);
}

// kvf_rerotate_q8's checks and launch (dev as in rerotate_impl)
kvf_status rerotate_q8_impl(const kvf_layer_desc* layer, const kvf_chunk* chunks, int32_t n_chunks,
                            int32_t max_chunk_len, const void* pool_k, const void* pool_v,
                            const kvf_kivi* kivi, int64_t pool_rows, const float* rope_cos,
                            const float* rope_sin, int32_t rope_n_pos, const kvf_q8_cache* fused,
                            const kvf::RotDeviation* dev, void* stream, const char* name) {
  KVF_CHECK(layer->dtype == KVF_BF16, KVF_ERR_UNSUPPORTED, "int8-resident caches need a bf16 layer");
  KVF_CHECK(n_chunks >= 0 && max_chunk_len >= 0 && pool_rows >= 0 && rope_n_pos >= 0,
            KVF_ERR_INVALID_ARG, "negative size");
  kvf_status st = check_q8(fused, 0);
  if (st != KVF_OK) return st;
  if (n_chunks == 0 || max_chunk_len == 0) return KVF_OK;
  KVF_CHECK(chunks && rope_cos && rope_sin, KVF_ERR_INVALID_ARG, "required pointer is NULL");
  if (kivi) {
    KVF_CHECK(kivi->bits == 8, KVF_ERR_UNSUPPORTED,
              "int8-resident re-positioning reads 8-bit KIVI caches, not %d-bit", kivi->bits);
    KVF_CHECK(pool_k == nullptr && pool_v == nullptr, KVF_ERR_INVALID_ARG,
              "pass either dense pool pointers or kivi, not both");
    KVF_CHECK(kivi->k_codes && kivi->v_codes && kivi->k_min && kivi->k_scale && kivi->v_min &&
                  kivi->v_scale && kivi->n_pool_chunks > 0, KVF_ERR_INVALID_ARG,
              "incomplete kvf_kivi");
  } else {
    KVF_CHECK(pool_k && pool_v, KVF_ERR_INVALID_ARG, "pool pointers are NULL");
  }
  KVF_CHECK(max_chunk_len <= (1 << 24), KVF_ERR_UNSUPPORTED, "max_chunk_len too large");
  return finish(kvf::launch_rerotate_q8(*layer, chunks, n_chunks, max_chunk_len, pool_k, pool_v,
                                          kivi, pool_rows, rope_cos, rope_sin, rope_n_pos, *fused,
                                          as_stream(stream), dev),
                as_stream(stream), name);
}

// The deviation-score half of kvf_rerotate_deviation / kvf_rerotate_q8_deviation:
// checks its arguments and fills *dev; *skip when no context row is scored.
kvf_status deviation_args(const kvf_layer_desc* layer, const kvf_batch* batch, int ok_lanes,
                          const void* k_fresh, const uint8_t* eligible, int32_t accumulate,
                          float* scores, kvf::RotDeviation* dev, bool* skip) {
  kvf_status st = check_batch(batch, &dev->B);
  if (st != KVF_OK) return st;
  KVF_CHECK(accumulate == 0 || accumulate == 1, KVF_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  KVF_CHECK(ok_lanes > 0, KVF_ERR_UNSUPPORTED,
            "the fused deviation score reduces a row within one wave: Hkv %d, d %d is not supported",
            layer->n_kv_heads, layer->head_dim);
  *skip = dev->B.cu_N[dev->B.n_req] == 0;
  if (!*skip) KVF_CHECK(k_fresh && scores, KVF_ERR_INVALID_ARG, "k_fresh or scores is NULL");
  dev->k_fresh = k_fresh;
  dev->out = kvf::ScoreOut{scores, eligible, accumulate};
  return KVF_OK;
}

}  // namespace

kvf_status kvf_rerotate(const kvf_layer_desc* layer, const kvf_chunk* chunks, int32_t n_chunks,
                        int32_t max_chunk_len, const void* pool_k, const void* pool_v,
                        const kvf_kivi* kivi, int64_t pool_rows, const float* rope_cos,
                        const float* rope_sin, int32_t rope_n_pos, void* fused_k, void* fused_v,
                        int64_t fused_rows, int32_t k_only, void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  return rerotate_impl(layer, chunks, n_chunks, max_chunk_len, pool_k, pool_v, kivi, pool_rows,
                       rope_cos, rope_sin, rope_n_pos, fused_k, fused_v, fused_rows, k_only,
                       nullptr, stream, "kvf_rerotate");
  KVF_GUARD_END
}

kvf_status kvf_rerotate_deviation(const kvf_layer_desc* layer, const kvf_batch* batch,
                                  const kvf_chunk* chunks, int32_t n_chunks, int32_t max_chunk_len,
                                  const void* pool_k, const void* pool_v, const kvf_kivi* kivi,
                                  int64_t pool_rows, const float* rope_cos, const float* rope_sin,
                                  int32_t rope_n_pos, void* fused_k, void* fused_v,
                                  int64_t fused_rows, int32_t k_only, const void* k_fresh,
                                  const uint8_t* eligible, int32_t accumulate, float* scores,
                                  void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  kvf::RotDeviation dev;
  bool skip = false;
  st = deviation_args(layer, batch, kvf::rerotate_deviation_lanes(layer->n_kv_heads, layer->head_dim),
                      k_fresh, eligible, accumulate, scores, &dev, &skip);
  if (st != KVF_OK) return st;
  return rerotate_impl(layer, chunks, n_chunks, max_chunk_len, pool_k, pool_v, kivi, pool_rows,
                       rope_cos, rope_sin, rope_n_pos, fused_k, fused_v, fused_rows, k_only,
                       skip ? nullptr : &dev, stream, "kvf_rerotate_deviation");
  KVF_GUARD_END
}

kvf_status kvf_rerotate_q8(const kvf_layer_desc* layer, const kvf_chunk* chunks, int32_t n_chunks,
                           int32_t max_chunk_len, const void* pool_k, const void* pool_v,
                           const kvf_kivi* kivi, int64_t pool_rows, const float* rope_cos,
                           const float* rope_sin, int32_t rope_n_pos, const kvf_q8_cache* fused,
                           void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  return rerotate_q8_impl(layer, chunks, n_chunks, max_chunk_len, pool_k, pool_v, kivi, pool_rows,
                          rope_cos, rope_sin, rope_n_pos, fused, nullptr, stream, "kvf_rerotate_q8");
  KVF_GUARD_END
}

kvf_status kvf_rerotate_q8_deviation(const kvf_layer_desc* layer, const kvf_batch* batch,
                                     const kvf_chunk* chunks, int32_t n_chunks,
                                     int32_t max_chunk_len, const void* pool_k, const void* pool_v,
                                     const kvf_kivi* kivi, int64_t pool_rows, const float* rope_cos,
                                     const float* rope_sin, int32_t rope_n_pos,
                                     const kvf_q8_cache* fused, const void* k_fresh,
                                     const uint8_t* eligible, int32_t accumulate, float* scores,
                                     void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  kvf::RotDeviation dev;
  bool skip = false;
  st = deviation_args(layer, batch,
                      kvf::rerotate_q8_deviation_lanes(layer->n_kv_heads, layer->head_dim), k_fresh,
                      eligible, accumulate, scores, &dev, &skip);
  if (st != KVF_OK) return st;
  return rerotate_q8_impl(layer, chunks, n_chunks, max_chunk_len, pool_k, pool_v, kivi, pool_rows,
                          rope_cos, rope_sin, rope_n_pos, fused, skip ? nullptr : &dev, stream,
                          "kvf_rerotate_q8_deviation");
  KVF_GUARD_END
}

kvf_status kvf_kivi_encode(const kvf_layer_desc* layer, const void* pool_k, const void* pool_v,
                           const int32_t* pool_cu, int32_t n_pool_chunks, int64_t pool_rows,
                           int32_t max_chunk_len, const kvf_kivi* out, void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  KVF_CHECK(layer->dtype == KVF_BF16, KVF_ERR_UNSUPPORTED, "the KIVI encoder reads bf16 caches");
  KVF_CHECK(n_pool_chunks >= 0 && pool_rows >= 0 && max_chunk_len >= 0, KVF_ERR_INVALID_ARG,
            "negative size");
  if (n_pool_chunks == 0 || pool_rows == 0) return KVF_OK;
  KVF_CHECK(pool_k && pool_v && pool_cu && out, KVF_ERR_INVALID_ARG, "required pointer is NULL");
  KVF_CHECK(out->k_codes && out->v_codes && out->k_min && out->k_scale && out->v_min &&
                out->v_scale, KVF_ERR_INVALID_ARG, "incomplete output kvf_kivi");
  KVF_CHECK(out->bits == 8 || out->bits == 4, KVF_ERR_UNSUPPORTED,
            "KIVI codes are 8 or 4 bits, not %d", out->bits);
  KVF_CHECK(out->n_pool_chunks >= n_pool_chunks, KVF_ERR_INVALID_ARG,
            "output statistics hold %d chunks, need %d", out->n_pool_chunks, n_pool_chunks);
  return finish(kvf::launch_kivi_encode(*layer, pool_k, pool_v, pool_cu, n_pool_chunks,
                                          pool_rows, max_chunk_len, *out, as_stream(stream)),
                as_stream(stream), "kvf_kivi_encode");
  KVF_GUARD_END
}

size_t kvf_score_workspace_size(kvf_score_mode mode, const kvf_layer_desc* layer,
                                const kvf_batch* batch, int32_t n_last_q) {
  try {
    if ((static_cast<int>(mode) & ~KVF_SCORE_ACCUMULATE) != KVF_SCORE_ATTN_MASS) return 0;
    kvf::BatchArgs B;
    if (check_layer(layer) != KVF_OK || check_batch(batch, &B) != KVF_OK) return 0;
    return kvf::attn_mass_workspace(*layer, B, n_last_q);
  } catch (...) {
    return 0;
  }
}

kvf_status kvf_score(kvf_score_mode mode_flags, const kvf_layer_desc* layer,
                     const kvf_batch* batch, const void* fused_k, const void* k_fresh,
                     const void* q_u, int32_t n_last_q, const uint8_t* eligible, float* scores,
                     void* workspace, size_t ws_bytes, void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  kvf::BatchArgs B;
  st = check_batch(batch, &B);
  if (st != KVF_OK) return st;
  const int flags = static_cast<int>(mode_flags);
  KVF_CHECK((flags & ~(0xff | KVF_SCORE_ACCUMULATE)) == 0, KVF_ERR_INVALID_ARG,
            "unknown score flags 0x%x", flags);
  const int mode = flags & 0xff;
  KVF_CHECK(mode == KVF_SCORE_DEVIATION || mode == KVF_SCORE_ATTN_MASS ||
                mode == KVF_SCORE_KEY_NORM, KVF_ERR_INVALID_ARG, "unknown score mode %d", mode);
  if (B.cu_N[B.n_req] == 0) return KVF_OK;
  KVF_CHECK(fused_k && scores, KVF_ERR_INVALID_ARG, "required pointer is NULL");
  const kvf::ScoreOut out{scores, eligible, (flags & KVF_SCORE_ACCUMULATE) ? 1 : 0};
  if (mode == KVF_SCORE_DEVIATION) {
    KVF_CHECK(k_fresh != nullptr, KVF_ERR_INVALID_ARG, "k_fresh is NULL");
    return finish(kvf::launch_deviation(*layer, B, fused_k, k_fresh, out, as_stream(stream)),
                as_stream(stream), "kvf_score(deviation)");
  }
  if (mode == KVF_SCORE_KEY_NORM)
    return finish(kvf::launch_key_norm(*layer, B, fused_k, out, as_stream(stream)),
                as_stream(stream), "kvf_score(key_norm)");
  KVF_CHECK(q_u != nullptr, KVF_ERR_INVALID_ARG, "q_u is NULL");
  KVF_CHECK(kvf::attn_mass_key_tiles(B) <= 16384, KVF_ERR_UNSUPPORTED,
            "attention mass over %lld 128-key context tiles (at most 16384 per call)",
            static_cast<long long>(kvf::attn_mass_key_tiles(B)));
  const size_t need = kvf::attn_mass_workspace(*layer, B, n_last_q);
  KVF_CHECK(ws_bytes >= need, KVF_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  KVF_CHECK(need == 0 || workspace != nullptr, KVF_ERR_WORKSPACE, "workspace is NULL");
  return finish(kvf::launch_attn_mass(*layer, B, fused_k, q_u, n_last_q, out, workspace,
                                        ws_bytes, as_stream(stream)),
                as_stream(stream), "kvf_score(attn_mass)");
  KVF_GUARD_END
}

kvf_status kvf_rerotate_score_attn_mass(const kvf_layer_desc* layer, const kvf_batch* batch,
                                        const kvf_chunk* chunks, int32_t n_chunks,
                                        int32_t max_chunk_len, const void* pool_k, int64_t pool_rows,
                                        const float* rope_cos, const float* rope_sin,
                                        int32_t rope_n_pos, void* fused_k, int64_t fused_rows,
                                        const void* q_u, int32_t n_last_q,
                                        const uint8_t* eligible, int32_t accumulate, float* scores,
                                        void* workspace, size_t ws_bytes, void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  kvf::BatchArgs B;
  st = check_batch(batch, &B);
  if (st != KVF_OK) return st;
  KVF_CHECK(accumulate == 0 || accumulate == 1, KVF_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  KVF_CHECK(n_chunks >= 0 && max_chunk_len >= 0 && rope_n_pos >= 0 && fused_rows >= 0 &&
                pool_rows >= 0, KVF_ERR_INVALID_ARG, "negative size");
  KVF_CHECK(pool_rows <= INT32_MAX, KVF_ERR_UNSUPPORTED, "pool_rows too large");
  KVF_CHECK(fused_rows >= B.cu_T[B.n_req], KVF_ERR_INVALID_ARG,
            "the fused cache (%lld rows) must hold the batch (%d rows)",
            static_cast<long long>(fused_rows), B.cu_T[B.n_req]);
  KVF_CHECK(max_chunk_len <= (1 << 24), KVF_ERR_UNSUPPORTED, "max_chunk_len too large");
  KVF_CHECK(fused_k != nullptr, KVF_ERR_INVALID_ARG, "fused_k is NULL");
  const bool rotate = n_chunks > 0 && max_chunk_len > 0;
  KVF_CHECK(!rotate || (chunks && pool_k && rope_cos && rope_sin), KVF_ERR_INVALID_ARG,
            "required pointer is NULL");
  const kvf::MassRotate rot{chunks, n_chunks, max_chunk_len, pool_k, pool_rows,
                            rope_cos, rope_sin, rope_n_pos, fused_rows};
  if (B.cu_N[B.n_req] == 0) {          // nothing to score: the re-positioning alone
    if (!rotate) return KVF_OK;
    return finish(kvf::launch_rerotate(*layer, chunks, n_chunks, max_chunk_len, pool_k, nullptr,
                                         nullptr, pool_rows, rope_cos, rope_sin, rope_n_pos, fused_k,
                                         nullptr, fused_rows, 1, as_stream(stream)),
                  as_stream(stream), "kvf_rerotate_score_attn_mass");
  }
  KVF_CHECK(q_u && scores, KVF_ERR_INVALID_ARG, "q_u or scores is NULL");
  KVF_CHECK(kvf::attn_mass_key_tiles(B) <= 16384, KVF_ERR_UNSUPPORTED,
            "attention mass over %lld 128-key context tiles (at most 16384 per call)",
            static_cast<long long>(kvf::attn_mass_key_tiles(B)));
  const size_t need = kvf::attn_mass_workspace(*layer, B, n_last_q);
  KVF_CHECK(ws_bytes >= need, KVF_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  KVF_CHECK(need == 0 || workspace != nullptr, KVF_ERR_WORKSPACE, "workspace is NULL");
  const kvf::ScoreOut out{scores, eligible, accumulate};
  return finish(kvf::launch_attn_mass(*layer, B, fused_k, q_u, n_last_q, out, workspace, ws_bytes,
                                        as_stream(stream), rotate ? &rot : nullptr),
                as_stream(stream), "kvf_rerotate_score_attn_mass");
  KVF_GUARD_END
}

kvf_status kvf_score_q8(kvf_score_mode mode_flags, const kvf_layer_desc* layer,
                        const kvf_batch* batch, const kvf_q8_cache* fused, const void* k_fresh,
                        const uint8_t* eligible, float* scores, void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  KVF_CHECK(layer->dtype == KVF_BF16, KVF_ERR_UNSUPPORTED, "int8-resident caches need a bf16 layer");
  kvf::BatchArgs B;
  st = check_batch(batch, &B);
  if (st != KVF_OK) return st;
  const int flags = static_cast<int>(mode_flags);
  KVF_CHECK((flags & ~(0xff | KVF_SCORE_ACCUMULATE)) == 0, KVF_ERR_INVALID_ARG,
            "unknown score flags 0x%x", flags);
  const int mode = flags & 0xff;
  KVF_CHECK(mode == KVF_SCORE_DEVIATION || mode == KVF_SCORE_ATTN_MASS ||
                mode == KVF_SCORE_KEY_NORM, KVF_ERR_INVALID_ARG, "unknown score mode %d", mode);
  KVF_CHECK(mode != KVF_SCORE_ATTN_MASS, KVF_ERR_UNSUPPORTED,
            "attention-mass scoring reads a bf16 fused cache");
  st = check_q8(fused, B.cu_T[B.n_req]);
  if (st != KVF_OK) return st;
  if (B.cu_N[B.n_req] == 0) return KVF_OK;
  KVF_CHECK(scores != nullptr, KVF_ERR_INVALID_ARG, "scores is NULL");
  const kvf::ScoreOut out{scores, eligible, (flags & KVF_SCORE_ACCUMULATE) ? 1 : 0};
  if (mode == KVF_SCORE_DEVIATION) {
    KVF_CHECK(k_fresh != nullptr, KVF_ERR_INVALID_ARG, "k_fresh is NULL");
    return finish(kvf::launch_deviation_q8(*layer, B, *fused, k_fresh, out, as_stream(stream)),
                  as_stream(stream), "kvf_score_q8(deviation)");
  }
  return finish(kvf::launch_key_norm_q8(*layer, B, *fused, out, as_stream(stream)),
                as_stream(stream), "kvf_score_q8(key_norm)");
  KVF_GUARD_END
}

kvf_status kvf_score_attn_mass_noalloc(const kvf_layer_desc* layer, const kvf_batch* batch,
                                       const void* fused_k, const void* q_u, int32_t n_last_q,
                                       const uint8_t* eligible, float* scores, int32_t accumulate,
                                       void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  kvf::BatchArgs B;
  st = check_batch(batch, &B);
  if (st != KVF_OK) return st;
  KVF_CHECK(accumulate == 0 || accumulate == 1, KVF_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  if (B.cu_N[B.n_req] == 0) return KVF_OK;
  KVF_CHECK(fused_k && q_u && scores, KVF_ERR_INVALID_ARG, "required pointer is NULL");
  KVF_CHECK(kvf::attn_mass_key_tiles(B) <= 16384, KVF_ERR_UNSUPPORTED,
            "attention mass over %lld 128-key context tiles (at most 16384 per call)",
            static_cast<long long>(kvf::attn_mass_key_tiles(B)));
  const size_t need = kvf::attn_mass_workspace(*layer, B, n_last_q);
  KVF_CHECK(need <= KVF_NOALLOC_SCRATCH_BYTES, KVF_ERR_UNSUPPORTED,
            "this call needs %zu bytes of scratch; the allocation-free entry point holds %zu "
            "(use kvf_score with a caller workspace)", need,
            static_cast<size_t>(KVF_NOALLOC_SCRATCH_BYTES));
  const kvf::ScoreOut out{scores, eligible, accumulate};
  return finish(kvf::launch_attn_mass_noalloc(*layer, B, fused_k, q_u, n_last_q, out,
                                              as_stream(stream)),
                as_stream(stream), "kvf_score_attn_mass_noalloc");
  KVF_GUARD_END
}

size_t kvf_select_workspace_size(const kvf_batch* batch) {
  (void)batch;
  return 0;
}

kvf_status kvf_select_topk(const float* scores, const uint8_t* forced, const kvf_batch* batch,
                           const int32_t* k_per_req, int32_t* out_idx, int32_t* out_rows,
                           int32_t* out_pos, uint8_t* out_mask, void* workspace, size_t ws_bytes,
                           void* stream) {
  KVF_GUARD_BEGIN
  (void)workspace;
  (void)ws_bytes;
  kvf::BatchArgs B;
  kvf_status st = check_batch(batch, &B);
  if (st != KVF_OK) return st;
  KVF_CHECK(k_per_req != nullptr, KVF_ERR_INVALID_ARG, "k_per_req is NULL");
  int64_t total_k = 0, total_m = 0;
  for (int r = 0; r < B.n_req; ++r) {
    KVF_CHECK(k_per_req[r] >= 0 && k_per_req[r] <= B.n_ctx[r], KVF_ERR_INVALID_ARG,
              "k_per_req[%d] = %d outside [0, %d]", r, k_per_req[r], B.n_ctx[r]);
    total_k += k_per_req[r];
    total_m += k_per_req[r] + (B.cu_T[r + 1] - B.cu_T[r] - B.n_ctx[r]);
  }
  if (total_m == 0 && (out_mask == nullptr || B.cu_N[B.n_req] == 0)) return KVF_OK;
  KVF_CHECK(total_k == 0 || out_idx, KVF_ERR_INVALID_ARG, "out_idx is NULL");
  KVF_CHECK((out_rows == nullptr) == (out_pos == nullptr), KVF_ERR_INVALID_ARG,
            "out_rows and out_pos must both be given or both be NULL");
  return finish(kvf::launch_topk(scores, forced, B, k_per_req, out_idx, out_rows, out_pos,
                                   out_mask, as_stream(stream)),
                as_stream(stream), "kvf_select_topk");
  KVF_GUARD_END
}

kvf_status kvf_select_topk_segmented(const float* scores, const uint8_t* forced,
                                     const kvf_batch* batch, const kvf_segment* segs,
                                     int32_t n_segs, const int32_t* k_per_req, int32_t* out_idx,
                                     int32_t* out_rows, int32_t* out_pos, void* stream) {
  KVF_GUARD_BEGIN
  kvf::BatchArgs B;
  kvf_status st = check_batch(batch, &B);
  if (st != KVF_OK) return st;
  KVF_CHECK(k_per_req != nullptr, KVF_ERR_INVALID_ARG, "k_per_req is NULL");
  KVF_CHECK(n_segs >= 0 && n_segs <= (1 << 24), KVF_ERR_INVALID_ARG, "n_segs %d out of range",
            n_segs);
  int64_t total_k = 0, total_m = 0;
  for (int r = 0; r < B.n_req; ++r) {
    KVF_CHECK(k_per_req[r] >= 0 && k_per_req[r] <= B.n_ctx[r], KVF_ERR_INVALID_ARG,
              "k_per_req[%d] = %d outside [0, %d]", r, k_per_req[r], B.n_ctx[r]);
    total_k += k_per_req[r];
    total_m += k_per_req[r] + (B.cu_T[r + 1] - B.cu_T[r] - B.n_ctx[r]);
  }
  KVF_CHECK((out_rows == nullptr) == (out_pos == nullptr), KVF_ERR_INVALID_ARG,
            "out_rows and out_pos must both be given or both be NULL");
  if (out_rows == nullptr && (total_k == 0 || n_segs == 0)) return KVF_OK;
  if (total_m == 0) return KVF_OK;
  KVF_CHECK(total_k == 0 || out_idx, KVF_ERR_INVALID_ARG, "out_idx is NULL");
  KVF_CHECK(n_segs == 0 || segs, KVF_ERR_INVALID_ARG, "segs is NULL");
  return finish(kvf::launch_topk_segmented(scores, forced, B, segs, n_segs, k_per_req, out_idx,
                                             out_rows, out_pos, as_stream(stream)),
                as_stream(stream), "kvf_select_topk_segmented");
  KVF_GUARD_END
}

static kvf_status check_rules(const kvf_static_rules* rules) {
  KVF_CHECK(rules != nullptr, KVF_ERR_INVALID_ARG, "rules is NULL");
  KVF_CHECK(rules->sink >= 0 && rules->boundary >= 0 && rules->seam >= 0, KVF_ERR_INVALID_ARG,
            "static rules must be >= 0");
  return KVF_OK;
}

kvf_status kvf_select_static(const kvf_batch* batch, const kvf_chunk* chunks, int32_t n_chunks,
                             const kvf_static_rules* rules, uint8_t* mask, void* stream) {
  KVF_GUARD_BEGIN
  kvf::BatchArgs B;
  kvf_status st = check_batch(batch, &B);
  if (st != KVF_OK) return st;
  st = check_rules(rules);
  if (st != KVF_OK) return st;
  KVF_CHECK(n_chunks >= 0, KVF_ERR_INVALID_ARG, "n_chunks negative");
  if (B.cu_N[B.n_req] == 0) return KVF_OK;
  KVF_CHECK(mask != nullptr, KVF_ERR_INVALID_ARG, "mask is NULL");
  KVF_CHECK(n_chunks == 0 || chunks, KVF_ERR_INVALID_ARG, "chunks is NULL");
  return finish(kvf::launch_static_mask(B, chunks, n_chunks, *rules, mask, as_stream(stream)),
                as_stream(stream), "kvf_select_static");
  KVF_GUARD_END
}

kvf_status kvf_static_counts(const kvf_batch* batch, const kvf_chunk* chunks_host,
                             int32_t n_chunks, const kvf_static_rules* rules, int32_t* counts) {
  KVF_GUARD_BEGIN
  kvf::BatchArgs B;
  kvf_status st = check_batch(batch, &B);
  if (st != KVF_OK) return st;
  st = check_rules(rules);
  if (st != KVF_OK) return st;
  KVF_CHECK(n_chunks >= 0, KVF_ERR_INVALID_ARG, "n_chunks negative");
  KVF_CHECK(counts != nullptr, KVF_ERR_INVALID_ARG, "counts is NULL");
  KVF_CHECK(n_chunks == 0 || chunks_host, KVF_ERR_INVALID_ARG, "chunks_host is NULL");
  kvf::static_counts_host(B, chunks_host, n_chunks, *rules, counts);
  g_err[0] = '\0';
  return KVF_OK;
  KVF_GUARD_END
}

size_t kvf_recompute_workspace_size(const kvf_layer_desc* layer, int32_t M, uint32_t out_mask) {
  try {
    if (check_layer(layer) != KVF_OK || M <= 0 || (out_mask & ~7u) != 0) return 0;
    return kvf::recompute_workspace(*layer, M, out_mask);
  } catch (...) {
    return 0;
  }
}

kvf_status kvf_recompute_qkv(const kvf_layer_desc* layer, const void* x, int64_t x_rows,
                             const int32_t* row_src, const int32_t* row_pos, int32_t M,
                             const void* w_qkv, uint32_t out_mask, const float* rope_cos,
                             const float* rope_sin, int32_t rope_n_pos, void* q_out,
                             void* k_out, void* v_out, const int32_t* kv_out_row,
                             int64_t kv_out_rows, void* workspace, size_t ws_bytes,
                             void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  KVF_CHECK(M >= 0 && x_rows >= 0 && rope_n_pos >= 0, KVF_ERR_INVALID_ARG, "negative size");
  KVF_CHECK((out_mask & ~7u) == 0, KVF_ERR_INVALID_ARG, "unknown bits in out_mask");
  if (M == 0 || out_mask == 0) return KVF_OK;
  KVF_CHECK(x && w_qkv && row_pos, KVF_ERR_INVALID_ARG, "required pointer is NULL");
  KVF_CHECK(x_rows > 0, KVF_ERR_INVALID_ARG, "x has no rows");
  KVF_CHECK(kv_out_row == nullptr || kv_out_rows > 0, KVF_ERR_INVALID_ARG,
            "kv_out_row needs kv_out_rows > 0");
  KVF_CHECK(row_src != nullptr || M <= x_rows, KVF_ERR_INVALID_ARG,
            "identity row map needs M <= x_rows");
  KVF_CHECK(!(out_mask & KVF_OUT_Q) || q_out, KVF_ERR_INVALID_ARG, "q_out is NULL");
  KVF_CHECK(!(out_mask & KVF_OUT_K) || k_out, KVF_ERR_INVALID_ARG, "k_out is NULL");
  KVF_CHECK(!(out_mask & KVF_OUT_V) || v_out, KVF_ERR_INVALID_ARG, "v_out is NULL");
  KVF_CHECK(!(out_mask & (KVF_OUT_Q | KVF_OUT_K)) || (rope_cos && rope_sin && rope_n_pos > 0),
            KVF_ERR_INVALID_ARG, "rope tables needed for Q/K");
  KVF_CHECK(layer->dtype != KVF_BF16 ||
                ((layer->n_q_heads * layer->head_dim) % 128 == 0 &&
                 (layer->n_kv_heads * layer->head_dim) % 128 == 0),
            KVF_ERR_UNSUPPORTED, "bf16 projection needs Hq*d and Hkv*d multiples of 128");
  const size_t need = kvf::recompute_workspace(*layer, M, out_mask);
  KVF_CHECK(ws_bytes >= need && (need == 0 || workspace != nullptr), KVF_ERR_WORKSPACE,
            "workspace of %zu bytes given, %zu needed", ws_bytes, need);
  return finish(kvf::launch_recompute(*layer, x, x_rows, row_src, row_pos, M, w_qkv, out_mask,
                                        rope_cos, rope_sin, rope_n_pos, q_out, k_out, v_out,
                                        kv_out_row, kv_out_rows, workspace, ws_bytes,
                                        as_stream(stream)),
                as_stream(stream), "kvf_recompute_qkv");
  KVF_GUARD_END
}

kvf_status kvf_scatter_kv(const kvf_layer_desc* layer, const void* k_src,
                          const int32_t* k_src_row, int64_t k_src_rows, const void* v_src,
                          const int32_t* v_src_row, int64_t v_src_rows, const int32_t* dst_row,
                          int32_t M, void* fused_k, void* fused_v, int64_t fused_rows,
                          void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  KVF_CHECK(M >= 0 && k_src_rows >= 0 && v_src_rows >= 0 && fused_rows >= 0,
            KVF_ERR_INVALID_ARG, "negative size");
  if (M == 0 || (k_src == nullptr && v_src == nullptr)) return KVF_OK;
  KVF_CHECK(dst_row != nullptr, KVF_ERR_INVALID_ARG, "dst_row is NULL");
  KVF_CHECK(!k_src || fused_k, KVF_ERR_INVALID_ARG, "fused_k is NULL");
  KVF_CHECK(!v_src || fused_v, KVF_ERR_INVALID_ARG, "fused_v is NULL");
  KVF_CHECK(!k_src || k_src_row || M <= k_src_rows, KVF_ERR_INVALID_ARG,
            "identity k source map needs M <= k_src_rows");
  KVF_CHECK(!v_src || v_src_row || M <= v_src_rows, KVF_ERR_INVALID_ARG,
            "identity v source map needs M <= v_src_rows");
  return finish(kvf::launch_scatter(*layer, k_src, k_src_row, k_src_rows, v_src, v_src_row,
                                      v_src_rows, dst_row, M, fused_k, fused_v, fused_rows,
                                      as_stream(stream)),
                as_stream(stream), "kvf_scatter_kv");
  KVF_GUARD_END
}

kvf_status kvf_scatter_kv_q8(const kvf_layer_desc* layer, const void* k_src,
                             const int32_t* k_src_row, int64_t k_src_rows, const void* v_src,
                             const int32_t* v_src_row, int64_t v_src_rows, const int32_t* dst_row,
                             int32_t M, const kvf_q8_cache* fused, void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  KVF_CHECK(layer->dtype == KVF_BF16, KVF_ERR_UNSUPPORTED, "int8-resident caches need a bf16 layer");
  KVF_CHECK(M >= 0 && k_src_rows >= 0 && v_src_rows >= 0, KVF_ERR_INVALID_ARG, "negative size");
  st = check_q8(fused, 0);
  if (st != KVF_OK) return st;
  if (M == 0 || (k_src == nullptr && v_src == nullptr)) return KVF_OK;
  KVF_CHECK(dst_row != nullptr, KVF_ERR_INVALID_ARG, "dst_row is NULL");
  KVF_CHECK(!k_src || k_src_row || M <= k_src_rows, KVF_ERR_INVALID_ARG,
            "identity k source map needs M <= k_src_rows");
  KVF_CHECK(!v_src || v_src_row || M <= v_src_rows, KVF_ERR_INVALID_ARG,
            "identity v source map needs M <= v_src_rows");
  KVF_CHECK(M <= (1 << 28), KVF_ERR_UNSUPPORTED, "M too large");
  return finish(kvf::launch_scatter_q8(*layer, k_src, k_src_row, k_src_rows, v_src, v_src_row,
                                         v_src_rows, dst_row, M, *fused, as_stream(stream)),
                as_stream(stream), "kvf_scatter_kv_q8");
  KVF_GUARD_END
}

static kvf_status check_cu_q(const kvf::BatchArgs& B, const int32_t* cu_q) {
  KVF_CHECK(cu_q != nullptr, KVF_ERR_INVALID_ARG, "cu_q is NULL");
  KVF_CHECK(cu_q[0] == 0, KVF_ERR_INVALID_ARG, "cu_q[0] must be 0");
  for (int r = 0; r < B.n_req; ++r)
    KVF_CHECK(cu_q[r + 1] >= cu_q[r], KVF_ERR_INVALID_ARG, "cu_q decreases at %d", r);
  return KVF_OK;
}

size_t kvf_attention_workspace_size(const kvf_layer_desc* layer, const kvf_batch* batch,
                                    const int32_t* cu_q) {
  try {
    if (check_layer(layer) != KVF_OK) return 0;
    kvf::BatchArgs B;
    if (check_batch(batch, &B) != KVF_OK || check_cu_q(B, cu_q) != KVF_OK) return 0;
    return kvf::attention_workspace(*layer, B, cu_q);
  } catch (...) {
    return 0;
  }
}

kvf_status kvf_sparse_q_attention(const kvf_layer_desc* layer, const kvf_batch* batch,
                                  const void* q, const int32_t* q_pos, const int32_t* cu_q,
                                  const void* fused_k, const void* fused_v, float sm_scale,
                                  void* out, float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  kvf::BatchArgs B;
  st = check_batch(batch, &B);
  if (st != KVF_OK) return st;
  st = check_cu_q(B, cu_q);
  if (st != KVF_OK) return st;
  KVF_CHECK(sm_scale > 0.f && sm_scale < 1e30f, KVF_ERR_INVALID_ARG, "bad sm_scale");
  if (cu_q[B.n_req] == 0) return KVF_OK;
  KVF_CHECK(q && q_pos && fused_k && fused_v && out, KVF_ERR_INVALID_ARG,
            "required pointer is NULL");
  if (workspace != nullptr) {
    const size_t need = kvf::attention_workspace(*layer, B, cu_q);
    KVF_CHECK(workspace_bytes >= need, KVF_ERR_WORKSPACE,
              "attention workspace %zu bytes, needs %zu", workspace_bytes, need);
  }
  return finish(kvf::launch_attention(*layer, B, q, q_pos, cu_q, fused_k, fused_v, sm_scale,
                                        out, lse, workspace, workspace_bytes, as_stream(stream)),
                as_stream(stream), "kvf_sparse_q_attention");
  KVF_GUARD_END
}

kvf_status kvf_sparse_q_attention_q8(const kvf_layer_desc* layer, const kvf_batch* batch,
                                     const void* q, const int32_t* q_pos, const int32_t* cu_q,
                                     const kvf_q8_cache* fused, float sm_scale, void* out,
                                     float* lse, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  KVF_GUARD_BEGIN
  kvf_status st = check_layer(layer);
  if (st != KVF_OK) return st;
  KVF_CHECK(layer->dtype == KVF_BF16, KVF_ERR_UNSUPPORTED, "int8-resident caches need a bf16 layer");
  kvf::BatchArgs B;
  st = check_batch(batch, &B);
  if (st != KVF_OK) return st;
  st = check_cu_q(B, cu_q);
  if (st != KVF_OK) return st;
  KVF_CHECK(sm_scale > 0.f && sm_scale < 1e30f, KVF_ERR_INVALID_ARG, "bad sm_scale");
  st = check_q8(fused, B.cu_T[B.n_req]);
  if (st != KVF_OK) return st;
  if (cu_q[B.n_req] == 0) return KVF_OK;
  KVF_CHECK(q && q_pos && out, KVF_ERR_INVALID_ARG, "required pointer is NULL");
  if (workspace != nullptr) {
    const size_t need = kvf::attention_workspace(*layer, B, cu_q);
    KVF_CHECK(workspace_bytes >= need, KVF_ERR_WORKSPACE,
              "attention workspace %zu bytes, needs %zu", workspace_bytes, need);
  }
  return finish(kvf::launch_attention_q8(*layer, B, q, q_pos, cu_q, *fused, sm_scale, out, lse,
                                           workspace, workspace_bytes, as_stream(stream)),
                as_stream(stream), "kvf_sparse_q_attention_q8");
  KVF_GUARD_END
}

}  // extern "C"
