// C-ABI layer of libpkv: validate host-visible arguments, then enqueue.
// Every check runs before anything is launched, so a failing call leaves all
// device memory untouched (AstrAI commit 8e39d9d8 page, bullet on validating
// prefill inputs before KV allocation, and bullet on one forward with a
// shared argument check).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "internal.hpp"
#include "pkv.h"

namespace {

thread_local std::string g_err;

pkv_status fail(pkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

pkv_status ok() {
  g_err.clear();
  return PKV_OK;
}

pkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int32_t dtype) { return dtype == PKV_FP8_E4M3 ? 1 : dtype == PKV_BF16 ? 2 : 4; }

constexpr int32_t kMaxBatch = 65535;  // grid y/z limit of the decode and prefill launches

pkv_status check_pool(const pkv_kv_pool* pool, int32_t layer) {
  if (!pool) return fail(PKV_EINVAL, "pool is NULL");
  if (pool->dtype != PKV_F32 && pool->dtype != PKV_BF16 && pool->dtype != PKV_FP8_E4M3)
    return fail(PKV_EDTYPE, "pool dtype %d is not PKV_F32, PKV_BF16 or PKV_FP8_E4M3",
                pool->dtype);
  if (pool->dtype == PKV_FP8_E4M3 &&
      (!pool->kv_scales || ((uintptr_t)pool->kv_scales & 7u) != 0))
    return fail(PKV_EINVAL, "an FP8_E4M3 pool needs kv_scales (8-byte aligned device fp32)");
  if (!pool->k || !pool->v) return fail(PKV_EINVAL, "pool k or v is NULL");
  if (pool->n_layers <= 0 || pool->n_slots <= 0 || pool->n_kv_heads <= 0)
    return fail(PKV_ESHAPE, "pool needs n_layers, n_slots, n_kv_heads > 0 (got %lld, %lld, %d)",
                (long long)pool->n_layers, (long long)pool->n_slots, pool->n_kv_heads);
  if (!pkv::head_dim_supported(pool->head_dim))
    return fail(PKV_EUNSUPPORTED, "head_dim %d not in {64, 128}", pool->head_dim);
  if (pool->n_slots > 0x7fffffffLL) return fail(PKV_ESHAPE, "n_slots must fit int32");
  if (layer < 0 || layer >= pool->n_layers)
    return fail(PKV_EINVAL, "layer %d outside [0, %lld)", layer, (long long)pool->n_layers);
  if (!aligned16(pool->k) || !aligned16(pool->v))
    return fail(PKV_EALIGN, "pool k/v must be 16-byte aligned");
  return PKV_OK;
}

pkv_status check_meta(const pkv_batch_meta* m, bool need_qo) {
  if (!m) return fail(PKV_EINVAL, "meta is NULL");
  if (m->batch < 0 || m->batch > kMaxBatch)
    return fail(PKV_EINVAL, "batch %d outside [0, %d]", m->batch, kMaxBatch);
  if (m->batch == 0) return PKV_OK;
  if (!m->req_to_token || !m->req_pool_indices || !m->seq_lens)
    return fail(PKV_EINVAL, "req_to_token, req_pool_indices and seq_lens are required");
  if (m->req_to_token_stride <= 0 || m->req_to_token_stride > 0x7fffffffLL)
    return fail(PKV_EINVAL, "req_to_token_stride %lld outside [1, 2^31)",
                (long long)m->req_to_token_stride);
  if (m->n_req_rows <= 0) return fail(PKV_EINVAL, "n_req_rows must be > 0");
  if (need_qo && !m->qo_indptr) return fail(PKV_EINVAL, "qo_indptr is required for prefill");
  return PKV_OK;
}

pkv_status check_split(pkv_split_cfg s) {
  if (s.max_splits < 1 || s.max_splits > PKV_MAX_SPLITS)
    return fail(PKV_EINVAL, "max_splits %d outside [1, %d]", s.max_splits, PKV_MAX_SPLITS);
  if (s.fixed_splits < 0) return fail(PKV_EINVAL, "fixed_splits must be >= 0");
  if (s.split_tokens < PKV_SPLIT_ALIGN || s.split_tokens % PKV_SPLIT_ALIGN != 0)
    return fail(PKV_EINVAL, "split_tokens %d must be a positive multiple of %d", s.split_tokens,
                PKV_SPLIT_ALIGN);
  return PKV_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// o_part at 0, ml_part at the next 256-byte boundary.
size_t ws_bytes_for(int64_t batch, int64_t hq, int64_t d, int64_t max_splits, size_t* ml_off) {
  const size_t o = (size_t)(batch * hq * max_splits * d) * 4;
  const size_t ml = (size_t)(batch * hq * max_splits * 2) * 4;
  if (ml_off) *ml_off = round256(o);
  return round256(o) + round256(ml);
}

pkv_status check_heads(const pkv_kv_pool* pool, int32_t n_q_heads) {
  if (n_q_heads <= 0) return fail(PKV_ESHAPE, "n_q_heads must be > 0");
  if (n_q_heads % pool->n_kv_heads != 0)
    return fail(PKV_ESHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d", n_q_heads,
                pool->n_kv_heads);
  const int g = n_q_heads / pool->n_kv_heads;
  if (!pkv::group_supported(g))
    return fail(PKV_EUNSUPPORTED, "group size %d not in {1, 2, 4, 8, 16}", g);
  if (pool->n_kv_heads > 65535) return fail(PKV_EUNSUPPORTED, "n_kv_heads > 65535");
  return PKV_OK;
}

char* a_k_layer(const pkv_kv_pool* pool, int32_t layer) {
  const int64_t layer_bytes = pool->n_slots * pool->n_kv_heads * pool->head_dim *
                              (int64_t)elem_bytes(pool->dtype);
  return (char*)pool->k + (int64_t)layer * layer_bytes;
}

char* a_v_layer(const pkv_kv_pool* pool, int32_t layer) {
  const int64_t layer_bytes = pool->n_slots * pool->n_kv_heads * pool->head_dim *
                              (int64_t)elem_bytes(pool->dtype);
  return (char*)pool->v + (int64_t)layer * layer_bytes;
}

pkv_status decode_prepare(const pkv_kv_pool* pool, int32_t layer, const void* q, int32_t n_q_heads,
                          const pkv_batch_meta* meta, float scale, pkv_split_cfg split,
                          void* workspace, size_t ws_bytes, pkv::DecodeArgs* a) {
  pkv_status s;
  if ((s = check_pool(pool, layer)) != PKV_OK) return s;
  if ((s = check_heads(pool, n_q_heads)) != PKV_OK) return s;
  if ((s = check_meta(meta, false)) != PKV_OK) return s;
  if ((s = check_split(split)) != PKV_OK) return s;
  if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
    return fail(PKV_EINVAL, "scale must be finite");
  size_t ml_off = 0;
  const size_t need = ws_bytes_for(meta->batch, n_q_heads, pool->head_dim, split.max_splits, &ml_off);
  if (meta->batch > 0) {
    if (!q) return fail(PKV_EINVAL, "q is NULL");
    if (!aligned16(q)) return fail(PKV_EALIGN, "q must be 16-byte aligned");
    if (!workspace) return fail(PKV_EWORKSPACE, "workspace is NULL");
    if (((uintptr_t)workspace & 255u) != 0)
      return fail(PKV_EALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
      return fail(PKV_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  }
  a->n_slots = pool->n_slots;
  a->n_kv_heads = pool->n_kv_heads;
  a->head_dim = pool->head_dim;
  a->dtype = pool->dtype;
  a->n_q_heads = n_q_heads;
  a->q = q;
  a->req_to_token = meta->req_to_token;
  a->stride = meta->req_to_token_stride;
  a->n_rows = meta->n_req_rows;
  a->batch = meta->batch;
  a->req_pool_indices = meta->req_pool_indices;
  a->seq_lens = meta->seq_lens;
  a->scale = scale;
  a->split = split;
  a->o_part = (float*)workspace;
  a->ml_part = workspace ? (float*)((char*)workspace + ml_off) : nullptr;
  a->out = nullptr;
  a->merge_multi_only = false;
  a->k_new = nullptr;
  a->v_new = nullptr;
  a->k = (void*)a_k_layer(pool, layer);
  a->v = (void*)a_v_layer(pool, layer);
  a->kv_indptr_out = nullptr;
  a->loc_out = nullptr;
  a->splits_out = nullptr;
  a->prefix_len = nullptr;
  a->group_indptr = nullptr;
  a->group_members = nullptr;
  a->n_groups = 0;
  a->max_members = 0;
  a->n_members = 0;
  a->kv_scale = pool->dtype == PKV_FP8_E4M3 ? pool->kv_scales + 2 * (int64_t)layer : nullptr;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_str(pkv_status s) {
  switch (s) {
    case PKV_OK: return "PKV_OK";
    case PKV_EINVAL: return "PKV_EINVAL";
    case PKV_EDTYPE: return "PKV_EDTYPE";
    case PKV_ESHAPE: return "PKV_ESHAPE";
    case PKV_EALIGN: return "PKV_EALIGN";
    case PKV_EWORKSPACE: return "PKV_EWORKSPACE";
    case PKV_EUNSUPPORTED: return "PKV_EUNSUPPORTED";
    case PKV_EHIP: return "PKV_EHIP";
    default: return "PKV_UNKNOWN";
  }
}

const char* pkv_last_error(void) { return g_err.c_str(); }

pkv_status pkv_choose_split(int32_t max_len, int32_t batch, int64_t total_len, int32_t n_kv_heads,
                            int32_t n_cu, pkv_split_cfg* out) {
  if (!out) return fail(PKV_EINVAL, "out is NULL");
  if (max_len < 0 || batch < 1 || n_kv_heads < 1 || n_cu < 1)
    return fail(PKV_EINVAL, "need max_len >= 0, batch, n_kv_heads, n_cu >= 1 (got %d, %d, %d, %d)",
                max_len, batch, n_kv_heads, n_cu);
  const int64_t len = max_len > 0 ? max_len : 1;
  int64_t tokens;
  if (batch > 1 && total_len >= 0) {
    // about 1.8 workgroups per CU over all (request, KV head, split) items:
    // T = ceil(total * n_kv_heads / (1.8 * n_cu)), in integers
    const int64_t tot = total_len > 0 ? total_len : 1;
    tokens = (tot * n_kv_heads * 5 + 9 * (int64_t)n_cu - 1) / (9 * (int64_t)n_cu);
  } else {
    // the longest request's workgroups cover the device about once
    int64_t want = (int64_t)n_cu / ((int64_t)batch * n_kv_heads);
    if (want < 1) want = 1;
    tokens = (len + want - 1) / want;
  }
  tokens = (tokens + PKV_SPLIT_ALIGN - 1) / PKV_SPLIT_ALIGN * PKV_SPLIT_ALIGN;
  tokens = tokens < 64 ? 64 : (tokens > 1024 ? 1024 : tokens);
  int64_t splits = (len + tokens - 1) / tokens;
  splits = splits < 1 ? 1 : (splits > PKV_MAX_SPLITS ? PKV_MAX_SPLITS : splits);
  out->max_splits = (int32_t)splits;
  out->fixed_splits = 0;
  out->split_tokens = (int32_t)tokens;
  out->reserved = 0;
  return ok();
}

pkv_status pkv_kv_store(const pkv_kv_pool* pool, int32_t layer, const void* k_new,
                        const void* v_new, const int32_t* loc, int64_t n_tokens,
                        hipStream_t stream) {
  pkv_status s;
  if ((s = check_pool(pool, layer)) != PKV_OK) return s;
  if (n_tokens < 0) return fail(PKV_EINVAL, "n_tokens must be >= 0");
  if (n_tokens == 0) return ok();
  if (!k_new || !v_new || !loc) return fail(PKV_EINVAL, "k_new, v_new and loc are required");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_EALIGN, "k_new / v_new must be 16-byte aligned");
  if (n_tokens > (int64_t)1 << 40) return fail(PKV_EINVAL, "n_tokens too large");
  const int es = elem_bytes(pool->dtype);
  const int64_t row_bytes = (int64_t)pool->n_kv_heads * pool->head_dim * es;
  const int64_t layer_bytes = pool->n_slots * row_bytes;
  if (pool->dtype == PKV_FP8_E4M3)
    return hip_status(pkv::launch_kv_store_fp8((char*)pool->k + layer * layer_bytes,
                                               (char*)pool->v + layer * layer_bytes, pool->n_slots,
                                               row_bytes, k_new, v_new, loc, n_tokens,
                                               pool->kv_scales + 2 * (int64_t)layer, stream),
                      "kv_store launch");
  return hip_status(pkv::launch_kv_store((char*)pool->k + layer * layer_bytes,
                                         (char*)pool->v + layer * layer_bytes, pool->n_slots,
                                         row_bytes, k_new, v_new, loc, n_tokens, stream),
                    "kv_store launch");
}

pkv_status pkv_rope_kv_store(const pkv_kv_pool* pool, int32_t layer, const void* q, void* q_out,
                             int32_t n_q_heads, const void* k_new, const void* v_new,
                             const int32_t* positions, const float* freqs_cis, int32_t max_pos,
                             int32_t interleaved, const int32_t* loc, int64_t n_tokens,
                             hipStream_t stream) {
  pkv_status s;
  if ((s = check_pool(pool, layer)) != PKV_OK) return s;
  if (n_tokens < 0) return fail(PKV_EINVAL, "n_tokens must be >= 0");
  if (n_tokens > (int64_t)1 << 40) return fail(PKV_EINVAL, "n_tokens too large");
  if (interleaved != 0 && interleaved != 1) return fail(PKV_EINVAL, "interleaved must be 0 or 1");
  if (max_pos <= 0) return fail(PKV_EINVAL, "max_pos must be > 0");
  if ((q == nullptr) != (q_out == nullptr))
    return fail(PKV_EINVAL, "q and q_out must both be set or both be NULL");
  if (q && (s = check_heads(pool, n_q_heads)) != PKV_OK) return s;
  if (n_tokens == 0) return ok();
  if (!k_new || !v_new || !loc || !positions || !freqs_cis)
    return fail(PKV_EINVAL, "k_new, v_new, positions, freqs_cis and loc are required");
  if (!aligned16(k_new) || !aligned16(v_new) || (q && (!aligned16(q) || !aligned16(q_out))))
    return fail(PKV_EALIGN, "q / q_out / k_new / v_new must be 16-byte aligned");
  if (((uintptr_t)freqs_cis & 7) != 0) return fail(PKV_EALIGN, "freqs_cis must be 8-byte aligned");
  pkv::RopeArgs r{};
  r.kv_scale = pool->dtype == PKV_FP8_E4M3 ? pool->kv_scales + 2 * (int64_t)layer : nullptr;
  r.k_layer = a_k_layer(pool, layer);
  r.v_layer = a_v_layer(pool, layer);
  r.n_slots = pool->n_slots;
  r.n_kv_heads = pool->n_kv_heads;
  r.head_dim = pool->head_dim;
  r.dtype = pool->dtype;
  r.n_q_heads = q ? n_q_heads : 0;
  r.q = q;
  r.q_out = q_out;
  r.k_new = k_new;
  r.v_new = v_new;
  r.positions = positions;
  r.freqs_cis = freqs_cis;
  r.max_pos = max_pos;
  r.interleaved = interleaved;
  r.loc = loc;
  r.n_tokens = n_tokens;
  return hip_status(pkv::launch_rope_kv_store(r, stream), "rope_kv_store launch");
}

pkv_status pkv_build_metadata(const pkv_batch_meta* meta, int32_t mode, pkv_split_cfg split,
                              int32_t* kv_indptr_out, int32_t* loc_out, int64_t loc_capacity,
                              int32_t* splits_out, hipStream_t stream) {
  pkv_status s;
  if (mode != PKV_MODE_DECODE && mode != PKV_MODE_PREFILL)
    return fail(PKV_EINVAL, "mode %d is not DECODE or PREFILL", mode);
  if ((s = check_meta(meta, mode == PKV_MODE_PREFILL)) != PKV_OK) return s;
  if (mode == PKV_MODE_PREFILL && splits_out)
    return fail(PKV_EINVAL, "splits_out must be NULL in PREFILL mode");
  if (splits_out && (s = check_split(split)) != PKV_OK) return s;
  if (loc_out && loc_capacity < 0) return fail(PKV_EINVAL, "loc_capacity must be >= 0");
  if (loc_out && mode == PKV_MODE_DECODE && loc_capacity < meta->batch)
    return fail(PKV_EINVAL, "loc_capacity %lld < batch %d", (long long)loc_capacity, meta->batch);
  if (!kv_indptr_out && !loc_out && !splits_out) return ok();
  return hip_status(pkv::launch_metadata(*meta, mode, split, kv_indptr_out, loc_out, loc_capacity,
                                         splits_out, stream),
                    "metadata launch");
}

size_t pkv_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t head_dim,
                                  int32_t max_splits) {
  if (batch <= 0 || n_q_heads <= 0 || head_dim <= 0 || max_splits <= 0 ||
      max_splits > PKV_MAX_SPLITS)
    return 0;
  return ws_bytes_for(batch, n_q_heads, head_dim, max_splits, nullptr);
}

pkv_status pkv_decode_partials(const pkv_kv_pool* pool, int32_t layer, const void* q,
                               int32_t n_q_heads, const pkv_batch_meta* meta, float scale,
                               pkv_split_cfg split, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
  pkv::DecodeArgs a{};
  pkv_status s = decode_prepare(pool, layer, q, n_q_heads, meta, scale, split, workspace, ws_bytes, &a);
  if (s != PKV_OK) return s;
  return hip_status(pkv::launch_decode_partials(a, stream), "decode partial launch");
}

pkv_status pkv_decode_merge(const pkv_batch_meta* meta, int32_t n_q_heads, int32_t head_dim,
                            int32_t dtype, pkv_split_cfg split, const void* workspace,
                            size_t ws_bytes, void* out, hipStream_t stream) {
  pkv_status s;
  if (dtype != PKV_F32 && dtype != PKV_BF16)
    return fail(PKV_EDTYPE, "dtype %d is not PKV_F32 or PKV_BF16", dtype);
  if (!pkv::head_dim_supported(head_dim))
    return fail(PKV_EUNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  if (n_q_heads <= 0) return fail(PKV_ESHAPE, "n_q_heads must be > 0");
  if ((s = check_meta(meta, false)) != PKV_OK) return s;
  if ((s = check_split(split)) != PKV_OK) return s;
  if (meta->batch == 0) return ok();
  if (!out) return fail(PKV_EINVAL, "out is NULL");
  if (!aligned16(out)) return fail(PKV_EALIGN, "out must be 16-byte aligned");
  size_t ml_off = 0;
  const size_t need = ws_bytes_for(meta->batch, n_q_heads, head_dim, split.max_splits, &ml_off);
  if (!workspace) return fail(PKV_EWORKSPACE, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(PKV_EALIGN, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(PKV_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  if (n_q_heads > 65535) return fail(PKV_EUNSUPPORTED, "n_q_heads > 65535");
  pkv::DecodeArgs a = {};
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.n_q_heads = n_q_heads;
  a.stride = meta->req_to_token_stride;
  a.batch = meta->batch;
  a.seq_lens = meta->seq_lens;
  a.split = split;
  a.o_part = (float*)workspace;
  a.ml_part = (float*)((char*)workspace + ml_off);
  a.out = out;
  return hip_status(pkv::launch_decode_merge(a, stream), "decode merge launch");
}

pkv_status pkv_paged_decode_attn(const pkv_kv_pool* pool, int32_t layer, const void* q,
                                 int32_t n_q_heads, const pkv_batch_meta* meta, float scale,
                                 pkv_split_cfg split, void* workspace, size_t ws_bytes,
                                 void* out, hipStream_t stream) {
  pkv::DecodeArgs a{};
  pkv_status s = decode_prepare(pool, layer, q, n_q_heads, meta, scale, split, workspace, ws_bytes, &a);
  if (s != PKV_OK) return s;
  if (meta->batch == 0) return ok();
  if (!out) return fail(PKV_EINVAL, "out is NULL");
  if (!aligned16(out)) return fail(PKV_EALIGN, "out must be 16-byte aligned");
  a.out = out;
  a.merge_multi_only = true;
  hipError_t e = pkv::launch_decode_partials(a, stream);
  if (e != hipSuccess) return hip_status(e, "decode partial launch");
  return hip_status(pkv::launch_decode_merge(a, stream), "decode merge launch");
}

pkv_status pkv_paged_decode_attn_noalloc(const pkv_kv_pool* pool, int32_t layer, const void* q,
                                         int32_t n_q_heads, const pkv_batch_meta* meta,
                                         float scale, pkv_split_cfg split, void* out,
                                         hipStream_t stream) {
  // the arguments and the scratch size first: nothing touches the device on error
  pkv_status s;
  if ((s = check_pool(pool, layer)) != PKV_OK) return s;
  if ((s = check_heads(pool, n_q_heads)) != PKV_OK) return s;
  if ((s = check_meta(meta, false)) != PKV_OK) return s;
  if ((s = check_split(split)) != PKV_OK) return s;
  if (meta->batch == 0) return ok();
  const size_t need = ws_bytes_for(meta->batch, n_q_heads, pool->head_dim, split.max_splits, nullptr);
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES)
    return fail(PKV_EWORKSPACE,
                "the partials need %zu bytes, above the %zu-byte scratch of the no-allocation call "
                "(use pkv_paged_decode_attn with a workspace)",
                need, (size_t)PKV_NOALLOC_SCRATCH_BYTES);
  if (!out) return fail(PKV_EINVAL, "out is NULL");
  if (!aligned16(out)) return fail(PKV_EALIGN, "out must be 16-byte aligned");
  void* scratch = nullptr;
  hipError_t e = pkv::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "no-allocation scratch lookup");
  pkv::DecodeArgs a{};
  s = decode_prepare(pool, layer, q, n_q_heads, meta, scale, split, scratch,
                     (size_t)PKV_NOALLOC_SCRATCH_BYTES, &a);
  if (s != PKV_OK) return s;
  a.out = out;
  a.merge_multi_only = true;
  e = pkv::launch_decode_partials(a, stream);
  if (e != hipSuccess) return hip_status(e, "decode partial launch");
  return hip_status(pkv::launch_decode_merge(a, stream), "decode merge launch");
}

pkv_status pkv_cascade_decode_attn(const pkv_kv_pool* pool, int32_t layer, const void* q,
                                   int32_t n_q_heads, const pkv_batch_meta* meta,
                                   const pkv_prefix_groups* groups, float scale,
                                   pkv_split_cfg split, void* workspace, size_t ws_bytes,
                                   void* out, hipStream_t stream) {
  pkv::DecodeArgs a{};
  pkv_status s = decode_prepare(pool, layer, q, n_q_heads, meta, scale, split, workspace, ws_bytes, &a);
  if (s != PKV_OK) return s;
  if (!groups) return fail(PKV_EINVAL, "groups is NULL");
  if (pool->dtype != PKV_BF16 && pool->dtype != PKV_FP8_E4M3)
    return fail(PKV_EUNSUPPORTED, "cascade decode supports BF16 and FP8_E4M3 pools (MFMA prefix)");
  if (split.max_splits < 2) return fail(PKV_EINVAL, "cascade decode needs max_splits >= 2");
  if (groups->n_groups < 0 || groups->n_groups > kMaxBatch)
    return fail(PKV_EINVAL, "n_groups %d outside [0, %d]", groups->n_groups, kMaxBatch);
  const int g = n_q_heads / pool->n_kv_heads;
  if (groups->n_groups > 0) {
    if (!groups->prefix_len || !groups->group_indptr || !groups->members)
      return fail(PKV_EINVAL, "prefix_len, group_indptr and members are required");
    if (groups->max_members < 1 || groups->max_members > kMaxBatch)
      return fail(PKV_EINVAL, "max_members %d outside [1, %d]", groups->max_members, kMaxBatch);
    if (groups->n_members < 1) return fail(PKV_EINVAL, "n_members must be >= 1");
    const int64_t z = (int64_t)groups->n_groups *
                          pkv::cascade_tiles(n_q_heads, pool->n_kv_heads, groups->max_members) +
                      meta->batch;
    if (z > kMaxBatch)
      return fail(PKV_EINVAL, "n_groups x ceil(max_members / (16 / %d)) + batch = %lld > %d", g,
                  (long long)z, kMaxBatch);
  }
  if (meta->batch == 0) return ok();
  if (!out) return fail(PKV_EINVAL, "out is NULL");
  if (!aligned16(out)) return fail(PKV_EALIGN, "out must be 16-byte aligned");
  a.out = out;
  a.merge_multi_only = true;
  if (groups->n_groups > 0) {
    a.prefix_len = groups->prefix_len;
    a.group_indptr = groups->group_indptr;
    a.group_members = groups->members;
    a.n_groups = groups->n_groups;
    a.max_members = groups->max_members;
    a.n_members = groups->n_members;
  }
  hipError_t e = pkv::launch_cascade_partials(a, stream);
  if (e != hipSuccess) return hip_status(e, "cascade partial launch");
  return hip_status(pkv::launch_decode_merge(a, stream), "decode merge launch");
}

pkv_status pkv_decode_step(const pkv_kv_pool* pool, int32_t layer, const void* q,
                           const void* k_new, const void* v_new, int32_t n_q_heads,
                           const pkv_batch_meta* meta, float scale, pkv_split_cfg split,
                           int32_t* kv_indptr_out, int32_t* loc_out, int32_t* splits_out,
                           void* workspace, size_t ws_bytes, void* out, hipStream_t stream) {
  pkv::DecodeArgs a{};
  pkv_status s = decode_prepare(pool, layer, q, n_q_heads, meta, scale, split, workspace, ws_bytes, &a);
  if (s != PKV_OK) return s;
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(PKV_EINVAL, "k_new and v_new must both be set or both be NULL");
  if (meta->batch == 0) {
    if (kv_indptr_out) return hip_status(pkv::launch_zero(kv_indptr_out, 4, stream), "zero launch");
    return ok();
  }
  if (!out) return fail(PKV_EINVAL, "out is NULL");
  if (!aligned16(out)) return fail(PKV_EALIGN, "out must be 16-byte aligned");
  if (k_new && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(PKV_EALIGN, "k_new / v_new must be 16-byte aligned");
  a.out = out;
  a.k_new = k_new;
  a.v_new = v_new;
  a.kv_indptr_out = kv_indptr_out;
  a.loc_out = loc_out;
  a.splits_out = splits_out;
  a.merge_multi_only = true;
  hipError_t e = pkv::launch_decode_partials(a, stream);
  if (e != hipSuccess) return hip_status(e, "decode step launch");
  return hip_status(pkv::launch_decode_merge(a, stream), "decode merge launch");
}

pkv_status pkv_paged_prefill_attn(const pkv_kv_pool* pool, int32_t layer, const void* q,
                                  int32_t n_q_heads, const pkv_batch_meta* meta,
                                  int32_t total_q, int32_t max_q_len, float scale,
                                  int32_t causal, void* out, hipStream_t stream) {
  pkv_status s;
  if ((s = check_pool(pool, layer)) != PKV_OK) return s;
  if ((s = check_heads(pool, n_q_heads)) != PKV_OK) return s;
  if ((s = check_meta(meta, true)) != PKV_OK) return s;
  if (total_q < 0 || max_q_len < 0) return fail(PKV_EINVAL, "total_q and max_q_len must be >= 0");
  if (causal != 0 && causal != 1) return fail(PKV_EINVAL, "causal must be 0 or 1");
  if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
    return fail(PKV_EINVAL, "scale must be finite");
  if (meta->batch == 0 || total_q == 0 || max_q_len == 0) return ok();
  if (!q || !out) return fail(PKV_EINVAL, "q and out are required");
  if (!aligned16(q) || !aligned16(out)) return fail(PKV_EALIGN, "q / out must be 16-byte aligned");
  if (pool->dtype != PKV_BF16 && pool->dtype != PKV_FP8_E4M3)
    return fail(PKV_EUNSUPPORTED, "prefill supports BF16 and FP8_E4M3 pools (MFMA path)");
  pkv::PrefillArgs a{};
  const int64_t layer_elems = pool->n_slots * pool->n_kv_heads * pool->head_dim;
  const int es = elem_bytes(pool->dtype);
  a.k = (const char*)pool->k + (int64_t)layer * layer_elems * es;
  a.v = (const char*)pool->v + (int64_t)layer * layer_elems * es;
  a.n_slots = pool->n_slots;
  a.n_kv_heads = pool->n_kv_heads;
  a.head_dim = pool->head_dim;
  a.dtype = pool->dtype;
  a.n_q_heads = n_q_heads;
  a.q = q;
  a.req_to_token = meta->req_to_token;
  a.stride = meta->req_to_token_stride;
  a.n_rows = meta->n_req_rows;
  a.batch = meta->batch;
  a.req_pool_indices = meta->req_pool_indices;
  a.seq_lens = meta->seq_lens;
  a.qo_indptr = meta->qo_indptr;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.scale = scale;
  a.causal = causal;
  a.out = out;
  a.kv_scale = pool->dtype == PKV_FP8_E4M3 ? pool->kv_scales + 2 * (int64_t)layer : nullptr;
  return hip_status(pkv::launch_prefill(a, stream), "prefill launch");
}

pkv_status pkv_validate_meta(const pkv_batch_meta* meta, int32_t mode, int64_t n_slots,
                             int64_t total_q, hipStream_t stream) {
  pkv_status s;
  if (mode != PKV_MODE_DECODE && mode != PKV_MODE_PREFILL)
    return fail(PKV_EINVAL, "mode %d is not DECODE or PREFILL", mode);
  if ((s = check_meta(meta, mode == PKV_MODE_PREFILL)) != PKV_OK) return s;
  const int B = meta->batch;
  if (B == 0) return ok();
  const int64_t stride = meta->req_to_token_stride;
  const int64_t R = meta->n_req_rows;
  std::vector<int32_t> rows(B), lens(B), qo(B + 1, 0), ind(meta->kv_indptr ? B + 1 : 0);
  std::vector<int32_t> table((size_t)(R * stride));
  hipError_t e;
  e = hipMemcpyAsync(rows.data(), meta->req_pool_indices, B * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(lens.data(), meta->seq_lens, B * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(table.data(), meta->req_to_token, table.size() * 4, hipMemcpyDeviceToHost,
                       stream);
  if (e == hipSuccess && mode == PKV_MODE_PREFILL)
    e = hipMemcpyAsync(qo.data(), meta->qo_indptr, (B + 1) * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess && meta->kv_indptr)
    e = hipMemcpyAsync(ind.data(), meta->kv_indptr, (B + 1) * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "validate_meta copy");
  if (mode == PKV_MODE_PREFILL && qo[0] != 0) return fail(PKV_EINVAL, "qo_indptr[0] = %d != 0", qo[0]);
  int64_t acc = 0;
  for (int b = 0; b < B; ++b) {
    if (rows[b] < 0 || rows[b] >= R)
      return fail(PKV_EINVAL, "req_pool_indices[%d] = %d outside [0, %lld)", b, rows[b], (long long)R);
    if (lens[b] < 0 || lens[b] > stride)
      return fail(PKV_EINVAL, "seq_lens[%d] = %d outside [0, %lld]", b, lens[b], (long long)stride);
    for (int j = 0; j < lens[b]; ++j) {
      const int32_t slot = table[(size_t)rows[b] * stride + j];
      if (slot < 0 || slot >= n_slots)
        return fail(PKV_EINVAL, "req_to_token[%d, %d] = %d outside [0, %lld) (request %d)", rows[b],
                    j, slot, (long long)n_slots, b);
    }
    if (mode == PKV_MODE_PREFILL) {
      const int n = qo[b + 1] - qo[b];
      if (n < 0) return fail(PKV_EINVAL, "qo_indptr decreases at %d", b);
      if (n > lens[b]) return fail(PKV_EINVAL, "request %d has %d new tokens > seq_len %d", b, n, lens[b]);
    }
    acc += lens[b];
    if (meta->kv_indptr) {
      if (b == 0 && ind[0] != 0) return fail(PKV_EINVAL, "kv_indptr[0] = %d != 0", ind[0]);
      if ((int64_t)ind[b + 1] != acc)
        return fail(PKV_EINVAL, "kv_indptr[%d] = %d, prefix sum is %lld", b + 1, ind[b + 1], (long long)acc);
    }
  }
  if (mode == PKV_MODE_PREFILL && qo[B] > total_q)
    return fail(PKV_EINVAL, "qo_indptr[batch] = %d > total_q %lld", qo[B], (long long)total_q);
  return ok();
}

}  // extern "C"
