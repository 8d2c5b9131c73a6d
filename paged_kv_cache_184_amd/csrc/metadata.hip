// Index step (a1): kv_indptr, new-token cache locations and the decode split plan.
//
// AstrAI commit 398e8a3e page: int32 page-table / request-row / location
// indices, and decode metadata (position_ids, seq_lens, kv_indptr) updated in
// place every step instead of re-allocated. AstrAI commit e58a728b page:
// packed prompts located by cumulative query lengths (qo_indptr).
//
// One workgroup of 1024 threads scans seq_lens (each thread owns a contiguous
// run of requests, runs are combined with an LDS scan), so the whole step is a
// single launch that needs no host synchronisation. Prefill locations use a
// second launch with one workgroup per request.
#include "common.hpp"
#include "internal.hpp"

namespace pkv {
namespace {

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void meta_scan_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ req_to_token, int64_t stride,
    int32_t n_rows, const int32_t* __restrict__ req_pool_indices, int32_t batch, int32_t mode,
    pkv_split_cfg split, int32_t* __restrict__ kv_indptr, int32_t* __restrict__ loc,
    int64_t loc_capacity, int32_t* __restrict__ splits) {
  __shared__ int64_t sums[kScanThreads];
  const int tid = threadIdx.x;
  const int per = (batch + kScanThreads - 1) / kScanThreads;
  const int begin = min(batch, tid * per);
  const int end = min(batch, begin + per);
  int64_t local = 0;
  for (int b = begin; b < end; ++b) local += seq_lens[b];
  sums[tid] = local;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread sums.
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int64_t x = tid >= off ? sums[tid - off] : 0;
    __syncthreads();
    sums[tid] += x;
    __syncthreads();
  }
  int64_t run = sums[tid] - local;  // exclusive prefix of this thread's run
  if (kv_indptr) {
    if (tid == 0) kv_indptr[0] = 0;
    for (int b = begin; b < end; ++b) {
      run += seq_lens[b];
      kv_indptr[b + 1] = (int32_t)run;
    }
  }
  if (mode == PKV_MODE_DECODE) {
    for (int b = begin; b < end; ++b) {
      int L = seq_lens[b];
      L = L < 0 ? 0 : (L > stride ? (int)stride : L);
      if (loc && b < loc_capacity) {
        if (L == 0) {
          loc[b] = -1;
        } else {
          const int r = clamp_index(req_pool_indices[b], n_rows);
          loc[b] = req_to_token[(int64_t)r * stride + (L - 1)];
        }
      }
      if (splits) {
        int chunk;
        splits[b] = split_count(L, split.max_splits, split.fixed_splits, split.split_tokens, &chunk);
      }
    }
  }
}

__global__ __launch_bounds__(256) void meta_prefill_loc_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qo_indptr,
    const int32_t* __restrict__ req_to_token, int64_t stride, int32_t n_rows,
    const int32_t* __restrict__ req_pool_indices, int32_t* __restrict__ loc, int64_t loc_capacity) {
  const int b = blockIdx.x;
  const int q0 = qo_indptr[b];
  const int n = qo_indptr[b + 1] - q0;
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > stride ? (int)stride : L);
  const int P = L - n;
  const int r = clamp_index(req_pool_indices[b], n_rows);
  const int32_t* row = req_to_token + (int64_t)r * stride;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t t = (int64_t)q0 + i;
    const int pos = P + i;
    if (t < 0 || t >= loc_capacity || pos < 0 || pos >= stride) continue;
    loc[t] = row[pos];
  }
}

}  // namespace

hipError_t launch_metadata(const pkv_batch_meta& m, int32_t mode, pkv_split_cfg split,
                           int32_t* kv_indptr_out, int32_t* loc_out, int64_t loc_capacity,
                           int32_t* splits_out, hipStream_t stream) {
  // batch == 0 still launches the scan so kv_indptr[0] is written by a kernel
  // (no memset node when the call is captured into a graph).
  const bool decode = mode == PKV_MODE_DECODE;
  meta_scan_kernel<<<1, kScanThreads, 0, stream>>>(
      m.seq_lens, m.req_to_token, m.req_to_token_stride, m.n_req_rows, m.req_pool_indices,
      m.batch, mode, split, kv_indptr_out, decode ? loc_out : nullptr, loc_capacity,
      decode ? splits_out : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!decode && loc_out && m.batch > 0) {
    meta_prefill_loc_kernel<<<m.batch, 256, 0, stream>>>(
        m.seq_lens, m.qo_indptr, m.req_to_token, m.req_to_token_stride, m.n_req_rows,
        m.req_pool_indices, loc_out, loc_capacity);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pkv
