// Host-side launchers shared between the C-ABI layer (api.cpp) and the kernel
// translation units. Arguments are already validated when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

struct DecodeArgs {
  int64_t n_slots;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  int32_t n_q_heads;
  const void* q;
  const int32_t* req_to_token;
  int64_t stride;
  int32_t n_rows;
  int32_t batch;
  const int32_t* req_pool_indices;
  const int32_t* seq_lens;
  float scale;
  pkv_split_cfg split;
  float* o_part;
  float* ml_part;
  void* out;  // non-null: the partial kernel finishes requests with S <= 1 itself
  bool merge_multi_only;  // merge kernel: leave requests with S <= 1 alone
  // optional fused steps (all may be null)
  const void* k_new;  // [batch, n_kv_heads, head_dim]: store at req_to_token[r_b, L_b-1]
  const void* v_new;
  void* k;  // pool layer bases, writable (for the fused store)
  void* v;
  int32_t* kv_indptr_out;
  int32_t* loc_out;
  int32_t* splits_out;
  // cascade (shared-prefix) decode; prefix_len null: no shared prefixes
  const int32_t* prefix_len;     // [batch] shared-prefix length of each request (0: none)
  const int32_t* group_indptr;   // [n_groups + 1] into group_members
  const int32_t* group_members;  // request indices of each prefix group
  int32_t n_groups;
  int32_t max_members;           // bound on the members of one group
  int32_t n_members;             // length of group_members
  // FP8 pools: this layer's (k_scale, v_scale); a code c stands for e4m3(c) * scale
  const float* kv_scale;
};

// Whether a partial-kernel launch also runs the index step (on one extra row
// of split workgroups, beside the others).
inline __host__ __device__ bool fuses_index_step(const DecodeArgs& a) {
  return a.kv_indptr_out || a.loc_out || a.splits_out;
}

// Cascade decode partials: the groups' prefix splits and every request's own
// (suffix) splits in one launch; the merge kernel follows.
hipError_t launch_cascade_partials(const DecodeArgs& a, hipStream_t stream);
// Prefix workgroups per group along the grid's z axis (16 / g members each).
int cascade_tiles(int n_q_heads, int n_kv_heads, int max_members);

hipError_t launch_decode_partials(const DecodeArgs& a, hipStream_t stream);
// Device address of the current device's no-allocation scratch
// (PKV_NOALLOC_SCRATCH_BYTES, 256-byte aligned), looked up on first use.
hipError_t noalloc_scratch(void** out);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);

hipError_t launch_kv_store(void* k_layer, void* v_layer, int64_t n_slots, int64_t row_bytes,
                           const void* k_new, const void* v_new, const int32_t* loc,
                           int64_t n_tokens, hipStream_t stream);
// FP8 pools: bf16 rows quantised to E4M3 codes (row_bytes = codes per row);
// kv_scale = this layer's (k_scale, v_scale)
hipError_t launch_kv_store_fp8(void* k_layer, void* v_layer, int64_t n_slots, int64_t row_bytes,
                               const void* k_new, const void* v_new, const int32_t* loc,
                               int64_t n_tokens, const float* kv_scale, hipStream_t stream);

hipError_t launch_metadata(const pkv_batch_meta& m, int32_t mode, pkv_split_cfg split,
                           int32_t* kv_indptr_out, int32_t* loc_out, int64_t loc_capacity,
                           int32_t* splits_out, hipStream_t stream);

struct PrefillArgs {
  const void* k;  // layer base
  const void* v;
  int64_t n_slots;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  int32_t n_q_heads;
  const void* q;
  const int32_t* req_to_token;
  int64_t stride;
  int32_t n_rows;
  int32_t batch;
  const int32_t* req_pool_indices;
  const int32_t* seq_lens;
  const int32_t* qo_indptr;
  int32_t total_q;
  int32_t max_q_len;
  float scale;
  int32_t causal;
  void* out;
  const float* kv_scale;  // E4M3 pools: this layer's (k_scale, v_scale)
  int32_t sorted;         // set by the launcher: 1-D grid, request by request, longest tile first
  int32_t row_shift;      // set by the launcher: log2 of the row stride in bytes, or -1
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

struct RopeArgs {
  void* k_layer;  // pools at the layer
  void* v_layer;
  int64_t n_slots;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  int32_t n_q_heads;  // 0 when q is not rotated
  const void* q;      // [T, Hq, D] or null
  void* q_out;        // may equal q
  const void* k_new;  // [T, Hkv, D]
  const void* v_new;
  const int32_t* positions;  // [T]
  const float* freqs_cis;    // [max_pos, D/2, 2]
  int32_t max_pos;
  int32_t interleaved;
  const int32_t* loc;  // [T]
  int64_t n_tokens;
  const float* kv_scale;  // E4M3 pools: this layer's (k_scale, v_scale)
};

hipError_t launch_rope_kv_store(const RopeArgs& r, hipStream_t stream);

// Supported group sizes / head dims (the dispatch tables in the kernels match these).
inline bool group_supported(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }
inline bool head_dim_supported(int d) { return d == 64 || d == 128; }

}  // namespace pkv
