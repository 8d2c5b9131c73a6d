/*
 * pkv.h -- attention over a paged, slot-indexed KV cache on AMD MI355X (gfx950).
 *
 * A C ABI: plain device pointers, sizes and a HIP stream; no framework types.
 * Every entry point validates its host-visible arguments first and, on any
 * error, returns a status without enqueueing or writing anything. On success
 * the work is enqueued on `stream` and the call returns without synchronising;
 * the library never allocates device memory, never reads device data on the
 * host (except pkv_validate_meta, a debug aid) and keeps no pointer after it
 * returns, so the calls may be captured into a HIP graph. The one piece of
 * device state it holds is the fixed scratch array of
 * pkv_paged_decode_attn_noalloc, part of the code object, one per device.
 *
 * Citation key for the pages this library follows (AstrAI commit pages; a
 * "bullet" is one line of the commit message shown on that page):
 *   P1  commit 398e8a3e, page for tests/inference/test_cache.py
 *   P2  commit 8e39d9d8, page for astrai/inference/workspace.py
 *   P4  commit e58a728b, page for docs/developer/architecture.md
 *
 * Data model (P1, bullets on the 4D KVStorage layout and on single advanced
 * indexing buffer[layer_id, loc]; P1, bullet on int32 page-table, request-row
 * and cache-location indices):
 *   K and V pools: two contiguous tensors [n_layers, n_slots, n_kv_heads, head_dim].
 *   req_to_token:  int32 [n_req_rows, stride]; entry (r, j) is the slot holding
 *                  position j of the request stored in row r.
 *   seq_lens[b]:   keys visible to request b's last query, new tokens included.
 *   qo_indptr:     int32 [batch + 1]; request b's new tokens are the packed rows
 *                  qo_indptr[b] .. qo_indptr[b+1]-1 (P4, bullet on cumulative
 *                  query lengths).
 *   Query head h of a request reads KV head h / (n_q_heads / n_kv_heads).
 *
 * Supported: dtype F32 or BF16 (Q, K, V and output share it; accumulation is
 * always fp32; prefill takes BF16 or FP8_E4M3 pools), head_dim 64 or 128, group size
 * n_q_heads / n_kv_heads in {1, 2, 4, 8, 16}. FP8_E4M3 pools (one-byte codes
 * with per-layer K and V scales, see pkv_kv_pool) hold K/V for the decode
 * and prefill entry points and pkv_kv_store; there q, the new K/V rows and the
 * output are BF16 (P4, bullet on the fp8 MMA test kernel of the attention kernels; the
 * code format is the OCP 8-bit floating point E4M3 encoding).
 * The tuned paths are BF16 and FP8_E4M3. F32 decode is a precision path:
 * correct for every supported shape, but it reads one 16-token tile at a time
 * (no prefetch across tiles) and spills registers at group size 16.
 *
 * Memory safety: kernels clamp every device-supplied index to the buffer it
 * addresses (slots to [0, n_slots), request rows to [0, n_req_rows), positions
 * to [0, stride), packed rows to [0, total_q)), or, for the prefill kernel's
 * K/V and slot-id reads, read through buffer descriptors spanning exactly the
 * layer's pool and the request's table row (an access past the range reads
 * zeros), so malformed metadata gives undefined values but never an
 * out-of-bounds access. pkv_validate_meta reports such metadata.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 2

/* ---- status codes ---------------------------------------------------- */
typedef int32_t pkv_status;
#define PKV_OK 0
#define PKV_EINVAL 1       /* null pointer, negative size, index out of range, bad mode */
#define PKV_EDTYPE 2       /* dtype code not F32 / BF16 / FP8_E4M3 */
#define PKV_ESHAPE 3       /* inconsistent shapes, e.g. n_q_heads % n_kv_heads != 0 */
#define PKV_EALIGN 4       /* tensor pointer not 16-byte aligned, workspace not 256-byte aligned */
#define PKV_EWORKSPACE 5   /* workspace smaller than pkv_decode_workspace_bytes() */
#define PKV_EUNSUPPORTED 6 /* head_dim or group size outside the supported set */
#define PKV_EHIP 7         /* a kernel launch failed; see pkv_last_error() */

/* ---- dtypes and modes -------------------------------------------------- */
#define PKV_F32 0
#define PKV_BF16 1
#define PKV_FP8_E4M3 2 /* pools only: OCP E4M3 codes (bias 7, subnormals, NaN = S.1111.111, max 448) */

#define PKV_MODE_DECODE 0
#define PKV_MODE_PREFILL 1

/* Split boundaries are multiples of this many tokens. */
#define PKV_SPLIT_ALIGN 16
/* Largest accepted max_splits. */
#define PKV_MAX_SPLITS 4096

/* ---- descriptors ------------------------------------------------------- */

/* The KV pools. k and v are device pointers, 16-byte aligned, to contiguous
 * [n_layers, n_slots, n_kv_heads, head_dim] tensors of `dtype`. Owned by the caller.
 * kv_scales: FP8_E4M3 pools only (required there, 8-byte aligned, ignored
 * otherwise): device fp32 [n_layers, 2] = (k_scale, v_scale) of each layer,
 * read by the kernels at run time. A code c of layer l's K pool stands for
 * e4m3(c) * k_scale[l] (V likewise); stores write the code nearest to the fp32
 * quotient x / scale (ties to even, magnitudes beyond 448 saturated). */
typedef struct pkv_kv_pool {
  void* k;
  void* v;
  int64_t n_layers;
  int64_t n_slots;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  int32_t reserved;
  const float* kv_scales;
} pkv_kv_pool;

/* Per-batch metadata; all arrays are int32 device pointers owned by the caller.
 *   req_to_token      [n_req_rows, req_to_token_stride]
 *   req_pool_indices  [batch]  row of req_to_token used by request b
 *   seq_lens          [batch]  L_b (a decode row with L_b = 0 is padding)
 *   qo_indptr         [batch+1] packed new-token offsets; required for prefill,
 *                     ignored (may be NULL) for decode
 *   kv_indptr         [batch+1] optional (may be NULL); exclusive prefix sum
 *                     of seq_lens as written by pkv_build_metadata. The kernels
 *                     address K/V through req_to_token and do not read it;
 *                     pkv_validate_meta checks it when present. */
typedef struct pkv_batch_meta {
  const int32_t* req_to_token;
  int64_t req_to_token_stride;
  int32_t n_req_rows;
  int32_t batch;
  const int32_t* req_pool_indices;
  const int32_t* seq_lens;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
} pkv_batch_meta;

/* How decode splits each request's keys (P1, bullets on workspace-owned
 * decode_o_part / decode_ml_part split partials).
 *   max_splits    capacity of the workspace per (request, q head), 1..PKV_MAX_SPLITS
 *   fixed_splits  > 0: request this many splits; 0: automatic
 *   split_tokens  automatic mode requests ceil(L_b / split_tokens) splits;
 *                 a multiple of PKV_SPLIT_ALIGN, >= PKV_SPLIT_ALIGN
 * For a request of length L > 0 the requested count R is clamped to
 * [1, max_splits]; the chunk is C = round_up(ceil(L / R), PKV_SPLIT_ALIGN);
 * the split count is S = ceil(L / C) (never more than R, never an empty
 * split) and split s covers positions [s*C, min(L, (s+1)*C)). S = 0 when L = 0. */
typedef struct pkv_split_cfg {
  int32_t max_splits;
  int32_t fixed_splits;
  int32_t split_tokens;
  int32_t reserved;
} pkv_split_cfg;

/* The library's default split configuration for a decode batch, the one its
 * own measurements use (P2, bullet on keeping tuning constants in one place;
 * P1, bullet on the B=1 decode latency across 1K-32K contexts). A host-only
 * computation: no device access, safe to call without a GPU.
 *   max_len     longest seq_len of the batch (>= 0)
 *   batch       requests (>= 1)
 *   total_len   sum of the batch's seq_lens, or a negative value when unknown
 *   n_kv_heads  KV heads of the pool (>= 1)
 *   n_cu        compute units of the device (>= 1; 256 on MI355X)
 * Rule: one request, or a batch without total_len, takes tokens per split
 * T = ceil(max_len / max(1, n_cu / (batch * n_kv_heads))), so that the
 * (request, KV head, split) workgroups cover the device about once; a batch
 * with total_len takes T = ceil(5 * total_len * n_kv_heads / (9 * n_cu)),
 * about 1.8 workgroups per compute unit: all of them resident at once (two
 * per compute unit fit), with room for the rounding of each request's splits
 * (measured: item counts at or above two per compute unit run 7-13% slower
 * on the ragged 8-request batch). T is rounded up to a multiple of
 * PKV_SPLIT_ALIGN and clamped to [64, 1024]; the result is
 * { max_splits = clamp(ceil(max(1, max_len) / T), 1, PKV_MAX_SPLITS),
 *   fixed_splits = 0, split_tokens = T }. PKV_EINVAL (and *out untouched) for
 * an argument outside the ranges above or a NULL out. */
pkv_status pkv_choose_split(int32_t max_len, int32_t batch, int64_t total_len, int32_t n_kv_heads,
                            int32_t n_cu, pkv_split_cfg* out);

/* ---- library info ------------------------------------------------------ */
int pkv_abi_version(void);
const char* pkv_status_str(pkv_status s);
/* Message describing the last failure of a pkv_* call on the calling thread
 * ("" if none). The pointer stays valid until the next pkv_* call on the thread. */
const char* pkv_last_error(void);

/* ---- a2: store new K/V at cache locations -------------------------------
 * For every t < n_tokens with 0 <= loc[t] < n_slots:
 *   k[layer, loc[t], :, :] = k_new[t];  v[layer, loc[t], :, :] = v_new[t]
 * (P1, bullet on single advanced indexing buffer[layer_id, loc]). Negative
 * locations (padded rows) and locations >= n_slots are skipped. The copy is
 * bit-exact; locations must be unique within one call (duplicates race).
 * k_new, v_new: device [n_tokens, n_kv_heads, head_dim] of the pool dtype
 * (BF16 for an FP8_E4M3 pool, whose rows are quantised under the layer's
 * scales, the code of fl32(x / scale) rounded to nearest even and saturated
 * at +-448, NaN to a NaN code), 16-byte aligned. loc: device int32
 * [n_tokens]. n_tokens == 0 is a no-op. */
pkv_status pkv_kv_store(const pkv_kv_pool* pool, int32_t layer, const void* k_new,
                        const void* v_new, const int32_t* loc, int64_t n_tokens,
                        hipStream_t stream);

/* ---- rotary embedding of the new tokens fused with their store ----------
 * For every t < n_tokens, with p = positions[t] clamped to [0, max_pos):
 *   q_out[t, h] = rope(q[t, h], p)             for h < n_q_heads (if q != NULL)
 *   k[layer, loc[t]] = rope(k_new[t]);  v[layer, loc[t]] = v_new[t]
 * (P1, bullet on extending the rotary embedding to packed 3D inputs; P4, bullet
 * on the rotary table holding cos / sin values). rope rotates pair i of a row
 * by the table entry freqs_cis[p, i] = (cos, sin): a' = a cos - b sin,
 * b' = b cos + a sin, in fp32, rounded to the pool dtype (nearest-even for
 * BF16). Pair i is (2i, 2i+1) when interleaved = 1, else (i, i + head_dim/2).
 * Stores follow pkv_kv_store: loc outside [0, n_slots) is skipped, locations
 * must be unique within one call, v is copied bit-exactly.
 * q, q_out: device [n_tokens, n_q_heads, head_dim] of the pool dtype, 16-byte
 * aligned; q_out may equal q (in place); both NULL to rotate only k.
 * k_new, v_new: device [n_tokens, n_kv_heads, head_dim], 16-byte aligned, not
 * modified. positions, loc: device int32 [n_tokens]. freqs_cis: device float
 * [max_pos, head_dim/2, 2], 8-byte aligned. FP8_E4M3 pools: q, q_out,
 * k_new and v_new are BF16; k is rotated in fp32 with each product and sum
 * rounded once (a' = fl(fl(a cos) - fl(b sin)), b' = fl(fl(b cos) +
 * fl(a sin)), no fused multiply-add) and its codes are decided on that value
 * as pkv_kv_store decides them; v is quantised unrotated. */
pkv_status pkv_rope_kv_store(const pkv_kv_pool* pool, int32_t layer, const void* q, void* q_out,
                             int32_t n_q_heads, const void* k_new, const void* v_new,
                             const int32_t* positions, const float* freqs_cis, int32_t max_pos,
                             int32_t interleaved, const int32_t* loc, int64_t n_tokens,
                             hipStream_t stream);

/* ---- a1: index step ----------------------------------------------------
 * Writes, each only if its pointer is non-NULL (P1, bullet on updating
 * position_ids / seq_lens / kv_indptr in place each decode step):
 *   kv_indptr_out[0..batch]  exclusive prefix sum of seq_lens (int32; totals
 *                            of 2^31 or more wrap and are undefined)
 *   loc_out                  cache locations of the new tokens:
 *     DECODE:  loc_out[b] = req_to_token[r_b, L_b - 1], or -1 when L_b == 0
 *     PREFILL: loc_out[qo_indptr[b] + i] = req_to_token[r_b, L_b - n_b + i],
 *              i < n_b = qo_indptr[b+1] - qo_indptr[b]; rows >= loc_capacity
 *              are skipped
 *   splits_out[b]            decode split count S_b under `split` (DECODE only;
 *                            must be NULL in PREFILL mode)
 * loc_capacity: length of loc_out in elements (>= batch for DECODE). */
pkv_status pkv_build_metadata(const pkv_batch_meta* meta, int32_t mode, pkv_split_cfg split,
                              int32_t* kv_indptr_out, int32_t* loc_out, int64_t loc_capacity,
                              int32_t* splits_out, hipStream_t stream);

/* ---- decode workspace ----------------------------------------------------
 * The split partials live in a caller-owned workspace that is sized once and
 * passed down to the kernels on every call (P1, bullets on InferenceWorkspace
 * owning decode_o_part / decode_ml_part, on the C++ kernels taking
 * pre-allocated buffers, and on allocating once at executor start with no
 * allocation in the decode loop). This call returns the size.
 * Bytes of workspace one decode call over `batch` requests needs. Layout
 * (offsets from the workspace start, which must be 256-byte aligned):
 *   o_part  fp32 at 0:         [batch, n_q_heads, max_splits, head_dim]
 *           o_part[b,h,s,:] is split s's output, normalised by its own l
 *   ml_part fp32 at round_up(batch*n_q_heads*max_splits*head_dim*4, 256):
 *           [batch, n_q_heads, max_splits, 2] = (m, l) with
 *           l = sum_{j in split} exp(x_j - m), x_j = scale * q.k_j; m is a
 *           finite stabiliser the kernel picks (one of the x_j seen so far), so
 *           only m + ln(l), the split's log-sum-exp, is uniquely defined.
 * Entries for s >= S_b are not written; after pkv_paged_decode_attn or
 * pkv_decode_step, requests with a single split may not have partials either
 * (their output is written directly). Returns 0 if an argument is not positive
 * or max_splits > PKV_MAX_SPLITS. A workspace sized for batch B serves any
 * batch <= B with the same n_q_heads, head_dim and max_splits. */
size_t pkv_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t head_dim,
                                  int32_t max_splits);

/* ---- a3 + a4: split-KV paged decode attention ----------------------------
 * Flash-decoding over the paged cache (P1, bullets on workspace-owned
 * decode_o_part / decode_ml_part partials that the C++ decode kernels fill,
 * on reading K/V through the slot table instead of a gathered copy, and on the
 * B=1 decode latency across 1K-32K contexts).
 * One query token per request: for request b and q head h (KV head h/g),
 *   out[b, h, :] = softmax_j(scale * q[b,h,:] . K[j]) V[j],  j < L_b,
 * with K[j], V[j] read at slot req_to_token[r_b, j] of `layer`. Computed as
 * split partials in the workspace (a3) followed by a log-sum-exp merge (a4);
 * a request with a single split is finished by the first kernel, the merge
 * launch combines the others. Rows with L_b = 0 produce zeros.
 * q, out: device [batch, n_q_heads, head_dim] of the pool dtype (BF16 for an
 * FP8_E4M3 pool), 16-byte aligned; out is rounded to nearest-even. For BF16
 * the P.V products use P rounded to bf16 and the row sums use the same
 * rounded values. FP8_E4M3: K and V are the codes' values times the layer's
 * scales (codes widened exactly to bf16; the K scale joins the softmax
 * scale, the V scale multiplies the split outputs). The result is
 * bit-identical run to run and does not depend on where the slots sit in the
 * pool. Calls that share a workspace must not overlap in time. */
pkv_status pkv_paged_decode_attn(const pkv_kv_pool* pool, int32_t layer, const void* q,
                                 int32_t n_q_heads, const pkv_batch_meta* meta, float scale,
                                 pkv_split_cfg split, void* workspace, size_t ws_bytes,
                                 void* out, hipStream_t stream);

/* a1 + a2 + a3 in one launch, then the a4 merge: the index step (each output only if its
 * pointer is non-NULL: kv_indptr_out [batch+1], loc_out [batch], splits_out
 * [batch], as pkv_build_metadata in DECODE mode), the store of each request's
 * new token (k_new, v_new: device [batch, n_kv_heads, head_dim] of the pool
 * dtype, BF16 for FP8_E4M3 pools; 16-byte aligned, stored at slot req_to_token[r_b, L_b-1] as
 * pkv_kv_store would with those locations; both NULL to skip the store) and
 * the attention of pkv_paged_decode_attn, which reads the stored rows. The new
 * tokens' slots must not be read by another request of the same call. */
pkv_status pkv_decode_step(const pkv_kv_pool* pool, int32_t layer, const void* q,
                           const void* k_new, const void* v_new, int32_t n_q_heads,
                           const pkv_batch_meta* meta, float scale, pkv_split_cfg split,
                           int32_t* kv_indptr_out, int32_t* loc_out, int32_t* splits_out,
                           void* workspace, size_t ws_bytes, void* out, hipStream_t stream);

/* ---- decode without a caller workspace -----------------------------------
 * For callers that cannot allocate device memory at all (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * result of pkv_paged_decode_attn with the same arguments, computed by the
 * same kernels, with the split partials in a scratch array the library holds
 * in each device's memory (PKV_NOALLOC_SCRATCH_BYTES, kept until the process
 * ends) instead of a caller workspace. The call allocates nothing; its first
 * call on a device looks up that device's scratch address (with the device
 * current), later calls reuse it. Needs
 * pkv_decode_workspace_bytes(batch, n_q_heads, head_dim, split.max_splits)
 * <= PKV_NOALLOC_SCRATCH_BYTES, else PKV_EWORKSPACE before anything is
 * enqueued. Every call on a device shares that device's scratch, which keeps
 * the last call's partials (no call needs it cleared): calls that overlap in
 * time on one device (other streams, other threads) race and must not be
 * issued; the caller serialises them. */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
pkv_status pkv_paged_decode_attn_noalloc(const pkv_kv_pool* pool, int32_t layer, const void* q,
                                         int32_t n_q_heads, const pkv_batch_meta* meta,
                                         float scale, pkv_split_cfg split, void* out,
                                         hipStream_t stream);

/* ---- cascade (shared-prefix) decode --------------------------------------
 * Requests of a prefix group map their first P positions to the same slots
 * (P1, bullets on rebuilding request mappings for cached prefix pages and on
 * prefix-reuse regressions; P4, bullet on packing prompts with a shared
 * prefix start). The result is that of pkv_paged_decode_attn for the same
 * requests; the difference is that each group's prefix K/V is read once per
 * 16 / g members (g = n_q_heads / n_kv_heads): their query heads are the 16
 * columns of one MFMA tile. Prefix and private-suffix work run in one launch.
 *   prefix_len:   device int32 [batch], shared-prefix length P_b of request b
 *                 (0: none; clamped to [0, L_b]); every member of a group must
 *                 have the group's P, and its first P table entries must equal
 *                 those of the group's first member, whose entries are read.
 *                 A member whose P differs from the first member's gets no
 *                 prefix partials: its output is unspecified (memory-safe).
 *   group_indptr: device int32 [n_groups + 1], members: device int32 request
 *                 indices [n_members]; group i is members[group_indptr[i] ..
 *                 group_indptr[i+1]-1], a request in at most one group
 *                 (positions are clamped to [0, n_members)).
 *   max_members:  host bound on the size of every group, in [1, 65535] (extra
 *                 members are ignored); the launch has n_groups *
 *                 ceil(max_members / (16 / g)) prefix rows besides the batch,
 *                 at most 65535 in all (PKV_EINVAL otherwise). */
typedef struct pkv_prefix_groups {
  const int32_t* prefix_len;
  const int32_t* group_indptr;
  const int32_t* members;
  int32_t n_groups;
  int32_t max_members;
  int32_t n_members;
  int32_t reserved;
} pkv_prefix_groups;

/* Split plan: the prefix of a request forms splits under a cap of
 * max_splits / 2 (partial indices first), its private suffix of L_b - P_b keys
 * splits under the rest of the cap (after them); max_splits >= 2; BF16 or
 * FP8_E4M3 pools (F32: PKV_EUNSUPPORTED). The workspace is sized as for
 * pkv_paged_decode_attn. */
pkv_status pkv_cascade_decode_attn(const pkv_kv_pool* pool, int32_t layer, const void* q,
                                   int32_t n_q_heads, const pkv_batch_meta* meta,
                                   const pkv_prefix_groups* groups, float scale,
                                   pkv_split_cfg split, void* workspace, size_t ws_bytes,
                                   void* out, hipStream_t stream);

/* a3 alone: writes the split partials of pkv_paged_decode_attn into the workspace
 * (no merge). */
pkv_status pkv_decode_partials(const pkv_kv_pool* pool, int32_t layer, const void* q,
                               int32_t n_q_heads, const pkv_batch_meta* meta, float scale,
                               pkv_split_cfg split, void* workspace, size_t ws_bytes,
                               hipStream_t stream);

/* a4 alone: merges the partials a pkv_decode_partials call with the same meta,
 * n_q_heads, head_dim and split left in the workspace (or partials a caller
 * wrote there in the documented layout):
 *   out = sum_s w_s o_s / sum_s w_s,  w_s = l_s exp(m_s - max_s' m_s').
 * A request with one split gets that split's o unchanged (rounded to the output
 * dtype), as pkv_paged_decode_attn does. dtype is the output's: F32 or BF16
 * (BF16 after an FP8_E4M3 pool). */
pkv_status pkv_decode_merge(const pkv_batch_meta* meta, int32_t n_q_heads, int32_t head_dim,
                            int32_t dtype, pkv_split_cfg split, const void* workspace,
                            size_t ws_bytes, void* out, hipStream_t stream);

/* ---- a5: ragged packed paged prefill --------------------------------------
 * New token i < n_b of request b (packed row t = qo_indptr[b] + i) attends,
 * per q head h with KV head h/g, to positions j <= L_b - n_b + i when causal
 * (bottom-right aligned: the cached prefix plus the earlier new tokens), or to
 * all j < L_b when not (P4, bullets on packing prompts with a shared prefix
 * start into one forward; P1, bullet on cached prefix pages). The new tokens'
 * K/V must already be stored (pkv_kv_store). q, out: device
 * [total_q, n_q_heads, head_dim], 16-byte aligned. max_q_len >= every n_b sizes
 * the launch; rows i >= max_q_len of a request are never written. BF16 or FP8_E4M3 pools
 * (F32 returns PKV_EUNSUPPORTED; for FP8_E4M3, q and out are BF16 and the
 * codes are widened exactly to bf16, the K scale joining the softmax scale and
 * the V scale the output): QK^T and PV run on bf16 MFMA with fp32
 * accumulation, P is rounded to bf16 for PV and the row sums use those rounded
 * values; any finite scale, including 0 and negative values. Bit-identical run
 * to run and independent of where the slots sit in the pool. */
pkv_status pkv_paged_prefill_attn(const pkv_kv_pool* pool, int32_t layer, const void* q,
                                  int32_t n_q_heads, const pkv_batch_meta* meta,
                                  int32_t total_q, int32_t max_q_len, float scale,
                                  int32_t causal, void* out, hipStream_t stream);

/* ---- debug validator --------------------------------------------------------
 * Checks the batch's index arrays before they are trusted (P2, bullets on
 * validating prefill inputs before KV allocation and on one forward behind a
 * shared _check_fwd guard; the entry points check their host-visible
 * arguments the same way, this call extends the check to device contents).
 * Synchronous: copies the metadata to the host (on `stream`, then waits) and
 * checks req_pool_indices in [0, n_req_rows), 0 <= seq_lens <= stride, slots
 * of every live position in [0, n_slots), and for PREFILL qo_indptr
 * non-decreasing from 0 with n_b <= L_b and qo_indptr[batch] <= total_q; when
 * meta->kv_indptr is set, that it equals the prefix sum of seq_lens.
 * Returns PKV_EINVAL with a message naming the first bad entry. Not for the hot path. */
pkv_status pkv_validate_meta(const pkv_batch_meta* meta, int32_t mode, int64_t n_slots,
                             int64_t total_q, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
