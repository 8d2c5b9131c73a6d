// Split-KV paged decode attention for gfx950: partial kernel (a3) and
// log-sum-exp merge (a4).
//
// Source passages (AstrAI pages): decode writes split partials into
// workspace-owned o_part / "ml" buffers that a merge combines (commit 398e8a3e,
// bullets on decode_o_part / decode_ml_part and on pre-allocated partials);
// K/V are read through the req_to_token slot table instead of a gathered copy
// (same page, bullet on removing Storage.gather); int32 indices (same page).
//
// Partial kernel, one wave per (request b, KV head, split s):
//   * Lanes form 8 groups of 8; group t handles tokens t and t+8 of a 16-token
//     tile, lane c of the group holds 16-byte chunks c, c+8, ... of the
//     token's K and V rows (D*es bytes per (slot, KV head)), so every load is a
//     coalesced 16-byte gather and 8 lanes cover one row with full 128-byte
//     segments.
//   * All g = Hq/Hkv query heads of the KV head are processed by the same wave,
//     so each K/V byte is fetched from HBM once per request and reused g times
//     from registers.
//   * q.k: v_dot2_f32_bf16 on packed bf16 pairs (fp32 accumulate), then a
//     3-step DPP reduction inside the 8-lane group.
//   * Online softmax in base 2 with a wave-uniform stabiliser m per head that
//     is raised only when some score exceeds it by more than kTau (log2 units):
//     until then exp2(x - m) <= 2^kTau, so no rescale of the accumulators is
//     needed on most tiles. The final o / l does not depend on m.
//   * Loads for tile i+1 are issued before tile i is computed (two register
//     buffers, ping-pong).
//   * Tokens past the split end read the split's last valid token (clamped
//     position) and get p = 0, so padding slots are never read.
// The reduction order depends only on the logical token position, so results
// are bit-identical across runs and across slot relocations.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace pkv {

namespace {

constexpr float kTau = 8.0f;  // log2 headroom before the stabiliser is raised
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T, int D>
struct Geo {
  static constexpr int ES = elem_size<T>::value;
  static constexpr int ROW = D * ES;          // bytes of one (slot, KV head) row
  static constexpr int CH = ROW / (8 * 16);  // 16-byte chunks per lane per token
  static constexpr int EPC = 16 / ES;        // elements per chunk
  static constexpr int E = CH * EPC;         // elements per lane per token (D / 8)
  static_assert(CH >= 1 && CH <= 4, "row size");
};

template <typename T, int D>
struct TileBuf {
  u32x4 k[2][Geo<T, D>::CH];
  u32x4 v[2][Geo<T, D>::CH];
};

template <typename T, int D>
__device__ __forceinline__ void load_tile(TileBuf<T, D>& buf, const char* kbase, const char* vbase,
                                          int64_t row_stride, const int slot[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t off = (int64_t)slot[j] * row_stride;
#pragma unroll
    for (int k = 0; k < Geo<T, D>::CH; ++k) {
      buf.k[j][k] = *(const u32x4*)(kbase + off + 128 * k);
      buf.v[j][k] = *(const u32x4*)(vbase + off + 128 * k);
    }
  }
}

// Partial dot product of this lane's elements of q (head h) and k.
template <typename T, int D>
__device__ __forceinline__ float lane_dot(const u32x4 (&q)[Geo<T, D>::CH],
                                          const u32x4 (&k)[Geo<T, D>::CH]) {
  float acc = 0.f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < Geo<T, D>::CH; ++c) {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc = dot2_bf16(q[c][w], k[c][w], acc);
    }
  } else {
#pragma unroll
    for (int c = 0; c < Geo<T, D>::CH; ++c) {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc = fmaf(__uint_as_float(q[c][w]), __uint_as_float(k[c][w]), acc);
    }
  }
  return acc;
}

// Element e (0..E-1) of a lane's row chunk set, as fp32.
template <typename T, int D>
__device__ __forceinline__ float elem(const u32x4 (&r)[Geo<T, D>::CH], int e) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w = r[e / 8][(e % 8) / 2];
    return (e & 1) ? bf16hi_to_f32(w) : bf16lo_to_f32(w);
  } else {
    return __uint_as_float(r[e / 4][e % 4]);
  }
}

template <typename T, int D, int G>
struct State {
  float acc[G][Geo<T, D>::E];
  float l[G];
  float m[G];  // log2 units, wave-uniform
};

template <typename T, int D, int G>
__device__ __forceinline__ void compute_tile(State<T, D, G>& st, const TileBuf<T, D>& buf,
                                             const u32x4 (&q)[G][Geo<T, D>::CH], float scale2,
                                             bool valid0, bool valid1) {
  constexpr int E = Geo<T, D>::E;
  float sc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    // reduce unconditionally (all lanes active for the DPP moves), then mask
    const float x0 = sum8(lane_dot<T, D>(q[h], buf.k[0])) * scale2;
    const float x1 = sum8(lane_dot<T, D>(q[h], buf.k[1])) * scale2;
    sc[h][0] = valid0 ? x0 : -INFINITY;
    sc[h][1] = valid1 ? x1 : -INFINITY;
  }
  bool need = false;
#pragma unroll
  for (int h = 0; h < G; ++h) need |= fmaxf(sc[h][0], sc[h][1]) > st.m[h] + kTau;
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mnew = fmaxf(st.m[h], wave_max(fmaxf(sc[h][0], sc[h][1])));
      const float corr = __builtin_amdgcn_exp2f(st.m[h] - mnew);
      st.l[h] *= corr;
#pragma unroll
      for (int e = 0; e < E; ++e) st.acc[h][e] *= corr;
      st.m[h] = mnew;
    }
  }
  float v0[E], v1[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v0[e] = elem<T, D>(buf.v[0], e);
    v1[e] = elem<T, D>(buf.v[1], e);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float p0 = __builtin_amdgcn_exp2f(sc[h][0] - st.m[h]);
    const float p1 = __builtin_amdgcn_exp2f(sc[h][1] - st.m[h]);
    st.l[h] += p0 + p1;
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[h][e] = fmaf(p1, v1[e], fmaf(p0, v0[e], st.acc[h][e]));
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeArgs a) {
  using Gm = Geo<T, D>;
  constexpr int CH = Gm::CH;
  constexpr int E = Gm::E;
  const int lane = threadIdx.x;
  const int grp = lane >> 3;
  const int c = lane & 7;
  const int s = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;

  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.stride ? (int)a.stride : L);
  int chunk;
  const int S = split_count(L, a.split.max_splits, a.split.fixed_splits, a.split.split_tokens,
                            &chunk);
  if (s >= S) return;
  const int lo = s * chunk;
  const int hi = min(L, lo + chunk);

  const int r = clamp_index(a.req_pool_indices[b], a.n_rows);
  const int32_t* row = a.req_to_token + (int64_t)r * a.stride;
  const int n_slots = (int)(a.n_slots > 0x7fffffff ? 0x7fffffff : a.n_slots);
  const int64_t row_stride = (int64_t)a.n_kv_heads * Gm::ROW;
  const char* kbase = (const char*)a.k + (int64_t)kvh * Gm::ROW + 16 * c;
  const char* vbase = (const char*)a.v + (int64_t)kvh * Gm::ROW + 16 * c;

  // q chunks of the g heads, in the same lane layout as K.
  u32x4 q[G][CH];
  const char* qbase = (const char*)a.q + ((int64_t)b * a.n_q_heads + (int64_t)kvh * G) * Gm::ROW + 16 * c;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < CH; ++k) q[h][k] = *(const u32x4*)(qbase + (int64_t)h * Gm::ROW + 128 * k);

  const float scale2 = a.scale * kLog2e;
  State<T, D, G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.l[h] = 0.f;
    st.m[h] = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[h][e] = 0.f;
  }

  auto slots_of = [&](int base, int out[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pos = min(base + grp + 8 * j, hi - 1);
      out[j] = clamp_index(row[pos], n_slots);
    }
  };

  TileBuf<T, D> A, B;
  int slotA[2], slotB[2];
  slots_of(lo, slotA);
  load_tile<T, D>(A, kbase, vbase, row_stride, slotA);
  if (lo + 16 < hi) slots_of(lo + 16, slotB);

  for (int base = lo; base < hi; base += 32) {
    // tile at base is in A; tile at base+16 (if any) goes to B
    const bool hasB = base + 16 < hi;
    if (hasB) load_tile<T, D>(B, kbase, vbase, row_stride, slotB);
    if (base + 32 < hi) slots_of(base + 32, slotA);
    compute_tile<T, D, G>(st, A, q, scale2, base + grp < hi, base + grp + 8 < hi);
    if (!hasB) break;
    const bool hasA = base + 32 < hi;
    if (hasA) load_tile<T, D>(A, kbase, vbase, row_stride, slotA);
    if (base + 48 < hi) slots_of(base + 48, slotB);
    compute_tile<T, D, G>(st, B, q, scale2, base + 16 + grp < hi, base + 24 + grp < hi);
  }

  // Reduce over the 8 token groups: lanes with equal c hold the same elements.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.l[h] += dpp<kRowRor8>(st.l[h]);
    st.l[h] += __shfl_xor(st.l[h], 16);
    st.l[h] += __shfl_xor(st.l[h], 32);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float x = st.acc[h][e];
      x += dpp<kRowRor8>(x);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      st.acc[h][e] = x;
    }
  }

  const int qh0 = kvh * G;
  const int64_t part = ((int64_t)b * a.n_q_heads + qh0) * a.split.max_splits + s;
  if (lane < 8) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = 1.0f / st.l[h];
      float* o = a.o_part + (part + (int64_t)h * a.split.max_splits) * D;
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        // chunk (c + 8k) holds elements [(c + 8k) * EPC, +EPC); as fp32 that is
        // EPC floats at element offset (c + 8k) * EPC.
        float* dst = o + (c + 8 * k) * Gm::EPC;
#pragma unroll
        for (int e = 0; e < Gm::EPC; e += 4) {
          float4 w;
          w.x = st.acc[h][k * Gm::EPC + e + 0] * inv;
          w.y = st.acc[h][k * Gm::EPC + e + 1] * inv;
          w.z = st.acc[h][k * Gm::EPC + e + 2] * inv;
          w.w = st.acc[h][k * Gm::EPC + e + 3] * inv;
          *(float4*)(dst + e) = w;
        }
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float2 ml;
      ml.x = st.m[h] * kLn2;
      ml.y = st.l[h];
      *(float2*)(a.ml_part + 2 * (part + (int64_t)h * a.split.max_splits)) = ml;
    }
  }
}

// One wave per (request, q head): out = sum_s w_s o_s / sum_s w_s.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;  // elements per lane
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.stride ? (int)a.stride : L);
  int chunk;
  const int S = split_count(L, a.split.max_splits, a.split.fixed_splits, a.split.split_tokens,
                            &chunk);
  const int64_t part = ((int64_t)b * a.n_q_heads + h) * a.split.max_splits;
  const float* ml = a.ml_part + 2 * part;
  const float* o = a.o_part + part * D;

  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float den = 0.f;
  for (int s = 0; s < S; ++s) {
    const float w = ml[2 * s + 1] * __builtin_amdgcn_exp2f((ml[2 * s] - M) * kLog2e);
    den += w;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, o[(int64_t)s * D + lane * PER + e], acc[e]);
  }
  const float inv = S > 0 ? 1.0f / den : 0.f;
  const int64_t orow = ((int64_t)b * a.n_q_heads + h) * D + lane * PER;
  if constexpr (sizeof(T) == 2) {
    uint16_t* out = (uint16_t*)a.out + orow;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = (uint16_t)f32_to_bf16_rne(acc[e] * inv);
  } else {
    float* out = (float*)a.out + orow;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = acc[e] * inv;
  }
}

template <typename T, int D>
hipError_t partials_for_dim(const DecodeArgs& a, hipStream_t stream) {
  const int g = a.n_q_heads / a.n_kv_heads;
  dim3 grid(a.split.max_splits, a.n_kv_heads, a.batch);
  switch (g) {
    case 1: decode_partial_kernel<T, D, 1><<<grid, 64, 0, stream>>>(a); break;
    case 2: decode_partial_kernel<T, D, 2><<<grid, 64, 0, stream>>>(a); break;
    case 4: decode_partial_kernel<T, D, 4><<<grid, 64, 0, stream>>>(a); break;
    case 8: decode_partial_kernel<T, D, 8><<<grid, 64, 0, stream>>>(a); break;
    case 16: decode_partial_kernel<T, D, 16><<<grid, 64, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_partials(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (a.dtype == PKV_BF16)
    return a.head_dim == 128 ? partials_for_dim<bf16_t, 128>(a, stream)
                             : partials_for_dim<bf16_t, 64>(a, stream);
  return a.head_dim == 128 ? partials_for_dim<float, 128>(a, stream)
                           : partials_for_dim<float, 64>(a, stream);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  dim3 grid(a.n_q_heads, a.batch);
  if (a.dtype == PKV_BF16) {
    if (a.head_dim == 128) decode_merge_kernel<bf16_t, 128><<<grid, 64, 0, stream>>>(a);
    else decode_merge_kernel<bf16_t, 64><<<grid, 64, 0, stream>>>(a);
  } else {
    if (a.head_dim == 128) decode_merge_kernel<float, 128><<<grid, 64, 0, stream>>>(a);
    else decode_merge_kernel<float, 64><<<grid, 64, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace pkv
