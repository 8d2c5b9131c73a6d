// Split-KV paged decode attention for gfx950: partial kernel (a3) and
// log-sum-exp merge (a4). Instantiated per (dtype, head_dim) in the
// decode_*.hip translation units.
//
// Source passages (AstrAI pages): decode writes split partials into
// workspace-owned o_part / "ml" buffers that a merge combines (commit 398e8a3e,
// bullets on decode_o_part / decode_ml_part and on pre-allocated partials);
// K/V are read through the req_to_token slot table instead of a gathered copy
// (same page, bullet on removing Storage.gather); int32 indices (same page).
//
// Partial kernel: one workgroup of kWaves waves per (request b, KV head, split
// s); each wave takes a contiguous share (a multiple of 16 tokens) of the
// split's tokens.
//   * Lanes form 64/LPR groups of LPR lanes (LPR = 8, or 16 for g >= 8 where
//     the row allows); group t handles tokens t, t + 64/LPR, ... of a 16-token
//     tile, lane c of the group holds 16-byte chunks c, c+LPR, ... of the
//     token's K and V rows (D*es bytes per (slot, KV head)), so every load is a
//     coalesced 16-byte gather and the lanes of a group cover one row with full
//     128-byte segments. 16 lanes per row halve the per-lane q and accumulator
//     registers, which at g >= 8 keeps them out of the AGPR file.
//   * All g = Hq/Hkv query heads of the KV head are processed by the same wave,
//     so each K/V byte is fetched from HBM once per request and reused g times
//     from registers.
//   * q.k: v_dot2_f32_bf16 on packed bf16 pairs (fp32 accumulate), then a
//     3-step (LPR = 8) or 4-step (LPR = 16) DPP reduction inside the group.
//   * Online softmax in base 2 with a wave-uniform stabiliser m per head that
//     is raised only when some score exceeds it by more than kTau (log2 units):
//     until then exp2(x - m) <= 2^kTau, so no rescale of the accumulators is
//     needed on most tiles. The final o / l does not depend on m.
//   * Slot ids are staged per 128-token super-tile into LDS (the next
//     super-tile's ids are prefetched into registers), so the K/V gathers
//     depend on an LDS read only. A super-tile is straight-line code (one
//     instantiation per tile count) with three tile buffers: each tile's loads
//     are issued two tiles ahead of its use and no buffer is carried around a
//     loop, which keeps the hardware wait counts static.
//   * Tokens past the range end read its last valid token (clamped position)
//     and get p = 0, so padding slots are never read.
//   * The kWaves partial states are merged in LDS in a fixed order.
// The reduction order depends only on the logical token position, so results
// are bit-identical across runs and across slot relocations.
#pragma once

#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace pkv {
namespace decode_impl {

constexpr float kTau = 8.0f;  // log2 headroom before the stabiliser is raised
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Lanes per (slot, KV head) row: 8 in general; 16 for large groups (g >= 8)
// when the row has at least 16 chunks, which halves the per-lane q and
// accumulator registers (g heads x row elements per lane).
template <typename T, int D, int G>
constexpr int lanes_per_row() {
  return (G >= 8 && D * elem_size<T>::value >= 256) ? 16 : 8;
}

template <typename T, int D, int LPR>
struct Geo {
  static constexpr int ES = elem_size<T>::value;
  static constexpr int ROW = D * ES;            // bytes of one (slot, KV head) row
  static constexpr int CH = ROW / (LPR * 16);   // 16-byte chunks per lane per token
  static constexpr int EPC = 16 / ES;           // elements per chunk
  static constexpr int E = CH * EPC;            // elements per lane per token (D / LPR)
  static constexpr int GROUPS = 64 / LPR;       // token groups per wave
  static constexpr int TPG = 16 / GROUPS;       // tokens per group per 16-token tile
  static_assert(CH >= 1 && CH <= 4, "row size");
  static_assert(TPG % 2 == 0, "tokens of a group are paired for P.V");
};

template <typename T, int D, int LPR>
struct TileBuf {
  u32x4 k[Geo<T, D, LPR>::TPG][Geo<T, D, LPR>::CH];
  u32x4 v[Geo<T, D, LPR>::TPG][Geo<T, D, LPR>::CH];
};

template <typename T, int D, int LPR>
__device__ __forceinline__ void load_tile(TileBuf<T, D, LPR>& buf, const char* kbase,
                                          const char* vbase, int64_t row_stride,
                                          const int (&slot)[Geo<T, D, LPR>::TPG]) {
#pragma unroll
  for (int j = 0; j < Geo<T, D, LPR>::TPG; ++j) {
    const int64_t off = (int64_t)slot[j] * row_stride;
#pragma unroll
    for (int k = 0; k < Geo<T, D, LPR>::CH; ++k) {
      buf.k[j][k] = load_stream(kbase + off + 16 * LPR * k);
      buf.v[j][k] = load_stream(vbase + off + 16 * LPR * k);
    }
  }
}

// Partial dot product of this lane's elements of q (head h) and k.
template <int CH, typename T>
__device__ __forceinline__ float lane_dot(const u32x4 (&q)[CH], const u32x4 (&k)[CH]) {
  float acc = 0.f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc = dot2_bf16(q[c][w], k[c][w], acc);
    }
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc = fmaf(__uint_as_float(q[c][w]), __uint_as_float(k[c][w]), acc);
    }
  }
  return acc;
}

// Element e (0..E-1) of a lane's row chunk set, as fp32.
template <int CH, typename T>
__device__ __forceinline__ float elem(const u32x4 (&r)[CH], int e) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w = r[e / 8][(e % 8) / 2];
    return (e & 1) ? bf16hi_to_f32(w) : bf16lo_to_f32(w);
  } else {
    return __uint_as_float(r[e / 4][e % 4]);
  }
}

template <typename T, int D, int G, int LPR>
struct State {
  float acc[G][Geo<T, D, LPR>::E];
  float l[G];
  float m[G];  // log2 units, wave-uniform
};

// Sum over the LPR lanes of a row; every lane of the row gets the same bits.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  x = sum8(x);
  if constexpr (LPR == 16) x += dpp<kRowRor8>(x);
  return x;
}

template <typename T, int D, int G, int LPR>
__device__ __forceinline__ void compute_tile(State<T, D, G, LPR>& st, const TileBuf<T, D, LPR>& buf,
                                             const u32x4 (&q)[G][Geo<T, D, LPR>::CH],
                                             float scale2, const bool (&valid)[Geo<T, D, LPR>::TPG]) {
  using Gm = Geo<T, D, LPR>;
  constexpr int E = Gm::E;
  constexpr int CH = Gm::CH;
  constexpr int TPG = Gm::TPG;
  float sc[G][TPG];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
      // reduce unconditionally (all lanes active for the DPP moves), then mask
      const float x = row_sum<LPR>(lane_dot<CH, T>(q[h], buf.k[j])) * scale2;
      sc[h][j] = valid[j] ? x : -INFINITY;
    }
  }
  bool need = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = sc[h][0];
#pragma unroll
    for (int j = 1; j < TPG; ++j) mx = fmaxf(mx, sc[h][j]);
    need |= mx > st.m[h] + kTau;
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sc[h][0];
#pragma unroll
      for (int j = 1; j < TPG; ++j) mx = fmaxf(mx, sc[h][j]);
      const float mnew = fmaxf(st.m[h], wave_max(mx));
      const float corr = __builtin_amdgcn_exp2f(st.m[h] - mnew);
      st.l[h] *= corr;
#pragma unroll
      for (int e = 0; e < E; ++e) st.acc[h][e] *= corr;
      st.m[h] = mnew;
    }
  }
  if constexpr (sizeof(T) == 2) {
    // P.V on v_dot2_f32_bf16: P is rounded to bf16 (hardware round-to-nearest-
    // even) and the row sum takes the same rounded values; V needs no
    // conversion, only pairing of two tokens' values of each element.
#pragma unroll
    for (int jp = 0; jp < TPG; jp += 2) {
      uint32_t vp[E];
#pragma unroll
      for (int k = 0; k < CH; ++k)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          vp[k * 8 + 2 * w] =
              __builtin_amdgcn_perm(buf.v[jp + 1][k][w], buf.v[jp][k][w], 0x05040100u);
          vp[k * 8 + 2 * w + 1] =
              __builtin_amdgcn_perm(buf.v[jp + 1][k][w], buf.v[jp][k][w], 0x07060302u);
        }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p0 = __builtin_amdgcn_exp2f(sc[h][jp] - st.m[h]);
        const float p1 = __builtin_amdgcn_exp2f(sc[h][jp + 1] - st.m[h]);
        const bf16x2_t pb = {(__bf16)p0, (__bf16)p1};
        const uint32_t pp = __builtin_bit_cast(uint32_t, pb);
        st.l[h] += bf16lo_to_f32(pp) + bf16hi_to_f32(pp);
#pragma unroll
        for (int e = 0; e < E; ++e) st.acc[h][e] = dot2_bf16(pp, vp[e], st.acc[h][e]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
      float v[E];
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = elem<CH, T>(buf.v[j], e);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = __builtin_amdgcn_exp2f(sc[h][j] - st.m[h]);
        st.l[h] += p;
#pragma unroll
        for (int e = 0; e < E; ++e) st.acc[h][e] = fmaf(p, v[e], st.acc[h][e]);
      }
    }
  }
}

constexpr int kWaves = 4;  // waves per workgroup, each taking a contiguous share of the split
constexpr int kTiles = 8;   // 16-token tiles per super-tile (straight-line, fully unrolled)
constexpr int kSuper = 16 * kTiles;

// NT consecutive 16-token tiles starting at token cb (the last may end early at
// ce), as straight-line code: every load is unconditional and issued two tiles
// ahead of its use, so the wait counts are static and no tile buffer is carried
// around a loop. Positions past ce re-read the last valid token (cache hits)
// and are masked.
template <typename T, int D, int G, int LPR, int NT>
__device__ __forceinline__ void tile_run(State<T, D, G, LPR>& st, const int* slots, int cb, int ce,
                                         int grp, const char* kbase, const char* vbase,
                                         int64_t row_stride,
                                         const u32x4 (&q)[G][Geo<T, D, LPR>::CH], float scale2) {
  using Gm = Geo<T, D, LPR>;
  constexpr int TPG = Gm::TPG;
  constexpr int GR = Gm::GROUPS;
  TileBuf<T, D, LPR> buf[3];
  // token j of group grp in tile i is cb + 16 i + grp + GR j
  auto issue = [&](int i) {
    int sl[TPG];
#pragma unroll
    for (int j = 0; j < TPG; ++j) sl[j] = slots[min(16 * i + grp + GR * j, ce - cb - 1)];
    load_tile<T, D, LPR>(buf[i % 3], kbase, vbase, row_stride, sl);
  };
  issue(0);
  if (NT > 1) issue(1);
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    if (i + 2 < NT) issue(i + 2);
    const int t = cb + 16 * i + grp;
    bool valid[TPG];
#pragma unroll
    for (int j = 0; j < TPG; ++j) valid[j] = t + GR * j < ce;
    compute_tile<T, D, G, LPR>(st, buf[i % 3], q, scale2, valid);
  }
}

template <typename T, int D, int G, int LPR>
__device__ __forceinline__ void super_tile(State<T, D, G, LPR>& st, const int* slots, int cb,
                                           int ce, int grp, const char* kbase, const char* vbase,
                                           int64_t row_stride,
                                           const u32x4 (&q)[G][Geo<T, D, LPR>::CH],
                                           float scale2) {
  if constexpr (sizeof(T) == 4) {
    // fp32 inputs: one tile at a time (no cross-tile prefetch); a precision
    // path, not a bandwidth path
    for (int t0 = cb; t0 < ce; t0 += 16)
      tile_run<T, D, G, LPR, 1>(st, slots + (t0 - cb), t0, ce, grp, kbase, vbase, row_stride, q,
                                scale2);
    return;
  }
  switch (ceil_div(ce - cb, 16)) {
#define PKV_RUN(n)                                                                             \
  case n:                                                                                      \
    tile_run<T, D, G, LPR, n>(st, slots, cb, ce, grp, kbase, vbase, row_stride, q, scale2);    \
    break;
    PKV_RUN(1) PKV_RUN(2) PKV_RUN(3) PKV_RUN(4) PKV_RUN(5) PKV_RUN(6) PKV_RUN(7) PKV_RUN(8)
#undef PKV_RUN
    default: break;
  }
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  if constexpr (sizeof(T) == 2) {
    ((__bf16*)out)[idx] = (__bf16)x;
  } else {
    ((float*)out)[idx] = x;
  }
}

// Index step (a1) for the whole batch, run by one workgroup of NT threads: kv_indptr (exclusive prefix sum of seq_lens), new-token locations
// and split counts; each output only if its pointer is set.
template <int NT>
__device__ void index_step_block(const DecodeArgs& a, int* scan_lds) {
  const int tid = threadIdx.x;
  const int B = a.batch;
  const int per = (B + NT - 1) / NT;
  const int begin = min(B, tid * per);
  const int end = min(B, begin + per);
  int local = 0;
  for (int b = begin; b < end; ++b) local += a.seq_lens[b];
  scan_lds[tid] = local;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int x = tid >= off ? scan_lds[tid - off] : 0;
    __syncthreads();
    scan_lds[tid] += x;
    __syncthreads();
  }
  int run = scan_lds[tid] - local;
  if (a.kv_indptr_out && tid == 0) a.kv_indptr_out[0] = 0;
  for (int b = begin; b < end; ++b) {
    int L = a.seq_lens[b];
    run += L;
    if (a.kv_indptr_out) a.kv_indptr_out[b + 1] = run;
    L = L < 0 ? 0 : (L > a.stride ? (int)a.stride : L);
    if (a.loc_out)
      a.loc_out[b] = L == 0 ? -1
                            : a.req_to_token[(int64_t)clamp_index(a.req_pool_indices[b], a.n_rows) *
                                                 a.stride + (L - 1)];
    if (a.splits_out) {
      int chunk;
      a.splits_out[b] = split_count(L, a.split.max_splits, a.split.fixed_splits,
                                    a.split.split_tokens, &chunk);
    }
  }
  __syncthreads();
}

// Split plan of request b. Without a shared prefix its L keys form S splits
// (the split rule of pkv_split_cfg). With a shared prefix of P > 0 keys
// (cascade decode), the prefix forms Sp splits under a cap of max_splits / 2
// (computed once per prefix group by the prefix kernel, partial indices
// [0, Sp)) and the private suffix of L - P keys forms S splits under the rest
// of the cap (partial indices [Sp, Sp + S)).
struct Plan {
  int L, P;     // keys, shared-prefix keys
  int Sp;       // prefix splits
  int S, chunk; // suffix splits and their length
};

__host__ __device__ __forceinline__ int prefix_cap(int max_splits) { return max_splits / 2; }

// The split plan from a request's raw seq_lens and prefix_len words (the
// latter ignored without prefix lengths).
__device__ __forceinline__ Plan plan_from(const DecodeArgs& a, int L_raw, int P_raw) {
  Plan p;
  const int L = L_raw < 0 ? 0 : (L_raw > a.stride ? (int)a.stride : L_raw);
  p.L = L;
  int P = a.prefix_len ? P_raw : 0;
  P = P < 0 ? 0 : (P > L ? L : P);
  p.P = P;
  int cap = a.split.max_splits;
  p.Sp = 0;
  if (P > 0) {
    int chunk_p;
    p.Sp = split_count(P, prefix_cap(cap), a.split.fixed_splits, a.split.split_tokens, &chunk_p);
    cap -= prefix_cap(cap);
  }
  p.S = split_count(L - P, cap, a.split.fixed_splits, a.split.split_tokens, &p.chunk);
  return p;
}

__device__ __forceinline__ Plan plan_for(const DecodeArgs& a, int b) {
  return plan_from(a, a.seq_lens[b], a.prefix_len ? a.prefix_len[b] : 0);
}

// What a split workgroup needs to know about its request and token range.
struct SplitCtx {
  int L, S, chunk, lo, hi;
  int Sp;               // partial index of this request's first suffix split
  int64_t row_stride;   // bytes between consecutive slots of one pool layer
  const int32_t* row;   // req_to_token row of the request
  int n_slots;
};

// Request length, split plan and this (suffix) split's token range. Returns
// false when the workgroup has no split to compute (after zeroing a padded
// request's output rows when an output is given).
template <typename T, int D, int G, int NT>
__device__ __forceinline__ bool split_setup(const DecodeArgs& a, int b, int kvh, int s,
                                            SplitCtx& c) {
  constexpr int ROW = D * elem_size<T>::value;
  // The request's length, prefix length and row index are scalar loads, all
  // in flight before any is used: one memory round trip before the slot ids
  // instead of three. Without prefix lengths the second load re-reads
  // seq_lens[b].
  int L_raw = load_uniform(a.seq_lens + b);
  int P_raw = load_uniform((a.prefix_len ? a.prefix_len : a.seq_lens) + b);
  int r_raw = load_uniform(a.req_pool_indices + b);
  // an empty statement that takes the three words: every use comes after it,
  // so the compiler cannot put a use (and its wait) between two of the loads
  asm volatile("" : "+s"(L_raw), "+s"(P_raw), "+s"(r_raw));
  const Plan p = plan_from(a, L_raw, P_raw);
  c.L = p.L;
  c.S = p.S;
  c.Sp = p.Sp;
  c.chunk = p.chunk;
  if (s >= c.S) {
    // a padded request (L = 0) has no split: its rows are zero
    if (c.S == 0 && c.Sp == 0 && s == 0 && a.out)
      for (int i = threadIdx.x; i < G * D; i += NT)
        store_out<typename io_type<T>::type>(a.out, ((int64_t)b * a.n_q_heads + kvh * G) * D + i,
                                             0.f);
    return false;
  }
  c.lo = p.P + s * c.chunk;
  c.hi = min(c.L, c.lo + c.chunk);
  const int r = clamp_index(r_raw, a.n_rows);
  c.row = a.req_to_token + (int64_t)r * a.stride;
  c.n_slots = (int)(a.n_slots > 0x7fffffff ? 0x7fffffff : a.n_slots);
  c.row_stride = (int64_t)a.n_kv_heads * ROW;
  return true;
}

// Store of the new token (position L-1) of this KV head by the wave whose
// share [wlo, whi) holds it, completed before that wave reads it back. FP8
// pools take bf16 rows, quantised under the layer's K or V scale. The slot id
// and the new row are independent loads and are issued together; the caller
// may have loads of its own in flight, which the final wait also covers.
template <typename T, int D>
__device__ __forceinline__ void store_new_token(const DecodeArgs& a, const SplitCtx& c, int b,
                                                int kvh, int wlo, int whi, int lane) {
  constexpr int ES = elem_size<T>::value;
  constexpr int ROW = D * ES;
  if (!a.k_new || c.L - 1 < wlo || c.L - 1 >= whi) return;
  constexpr int CPR = ROW / 16;  // 16-byte chunks of one (slot, KV head) row of the pool
  const bool mine = lane < 2 * CPR;
  const bool is_k = lane < CPR;
  const int chk = lane % CPR;
  // a chunk of the pool row takes 16 bytes of the new row (bf16, f32) or 32
  // (bf16 values quantised to 16 E4M3 codes)
  constexpr int SRC = ES == 1 ? 32 : 16;
  const char* src = (const char*)(is_k ? a.k_new : a.v_new) +
                    ((int64_t)b * a.n_kv_heads + kvh) * (CPR * SRC) + SRC * chk;
  u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
  if (mine) {
    v0 = *(const u32x4*)src;
    if constexpr (ES == 1) v1 = *(const u32x4*)(src + 16);
  }
  const int raw = c.row[c.L - 1];
  if (raw >= 0 && raw < c.n_slots && mine) {
    char* dst = (char*)(is_k ? a.k : a.v) + (int64_t)raw * c.row_stride + (int64_t)kvh * ROW +
                16 * chk;
    if constexpr (ES == 1)
      *(u32x4*)dst = quant_bf16x16(v0, v1, a.kv_scale[is_k ? 0 : 1]);
    else
      *(u32x4*)dst = v0;
  }
  // the row is read back by this same wave: complete the stores first
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
}

// Merge the W waves' (m, l, acc) from LDS (fixed order) into the split's
// normalised output: written directly for a single-split request when an
// output is given, else as the split's partial (o, (m ln2, l)). Wave w's
// accumulator rows are red_acc[w * wstride + h * D + d].
template <typename T, int D, int G, int W>
__device__ __forceinline__ void finish_split(const DecodeArgs& a, const float* red_acc,
                                             int wstride, const float (*red_ml)[G][2], int b,
                                             int kvh, int s, const SplitCtx& c) {
  const int qh0 = kvh * G;
  const int64_t part0 = ((int64_t)b * a.n_q_heads + qh0) * a.split.max_splits + c.Sp;
  const bool direct = a.out != nullptr && c.Sp + c.S == 1;
  for (int i = threadIdx.x; i < G * D; i += 64 * W) {
    const int h = i / D;
    const int d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, red_ml[w][h][0]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = red_ml[w][h][0];
      const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      num = fmaf(f, red_acc[w * wstride + h * D + d], num);
      den = fmaf(f, red_ml[w][h][1], den);
    }
    const float o = num / den;
    if (direct) {
      store_out<typename io_type<T>::type>(a.out, ((int64_t)b * a.n_q_heads + qh0 + h) * D + d, o);
      continue;
    }
    const int64_t part = part0 + (int64_t)h * a.split.max_splits + s;
    a.o_part[part * D + d] = o;
    if (d == 0) {
      float2 ml;
      ml.x = M * kLn2;
      ml.y = den;
      *(float2*)(a.ml_part + 2 * part) = ml;
    }
  }
}

// Reduce-scatter of NV values per lane over the 64 / LPR token groups of a
// wave (lane = LPR grp + c): after it, v[k] of a lane holds the sum over the
// groups of element first + k of the lanes with its c, for k < NV / groups;
// returns first. Each halving step moves one half of the live values to the
// partner group and adds: lane halves (xor 32) and row pairs (xor 16) with the
// gfx950 row-swap instructions, and, with 8 lanes per row, row halves (xor 8)
// with a DPP rotation. Which half a lane keeps after a swap is read off the
// same instruction applied to the half indices, so no lane layout is assumed.
template <int LPR, int NV>
__device__ __forceinline__ int group_reduce_scatter(float (&v)[NV], int lane) {
  static_assert(NV % (64 / LPR) == 0, "values per lane");
  int first = 0;
  constexpr int H1 = NV / 2;
  {
    const auto t = __builtin_amdgcn_permlane32_swap(0u, 1u, false, false);  // 0: kept first half
    first += (int)t[0] * H1;
#pragma unroll
    for (int k = 0; k < H1; ++k) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]),
                                                      __float_as_uint(v[k + H1]), false, false);
      v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }
  constexpr int H2 = NV / 4;
  {
    const auto t = __builtin_amdgcn_permlane16_swap(0u, 1u, false, false);
    first += (int)t[0] * H2;
#pragma unroll
    for (int k = 0; k < H2; ++k) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[k]),
                                                      __float_as_uint(v[k + H2]), false, false);
      v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }
  if constexpr (LPR == 8) {
    // lanes 0-7 of each row keep the first half, lanes 8-15 the second; each
    // adds the value of the lane 8 away in its row (row_ror:8)
    constexpr int H3 = NV / 8;
    const bool hi = (lane & 8) != 0;
    first += hi ? H3 : 0;
#pragma unroll
    for (int k = 0; k < H3; ++k) {
      const float x = hi ? v[k + H3] : v[k];
      const float y = hi ? v[k] : v[k + H3];
      v[k] = x + dpp<kRowRor8>(y);
    }
  }
  return first;
}

// The work of one (KV head kvh, split s, request b) workgroup of kWaves waves.
// LDS comes from the caller: slot ids slot_lds[kWaves][kSuper], wave w's
// accumulator rows (G * D floats) at red_acc + w * wstride, and red_ml.
template <typename T, int D, int G>
__device__ __forceinline__ void decode_split(const DecodeArgs& a, int kvh, int s, int b,
                                             int (*slot_lds)[kSuper], float* red_acc,
                                             int wstride, float (*red_ml)[G][2]) {
  constexpr int LPR = lanes_per_row<T, D, G>();
  using Gm = Geo<T, D, LPR>;
  constexpr int CH = Gm::CH;
  constexpr int E = Gm::E;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int grp = lane / LPR;  // token group
  const int c = lane % LPR;    // this lane's first 16-byte chunk of a row

  SplitCtx sc;
  if (!split_setup<T, D, G, 64 * kWaves>(a, b, kvh, s, sc)) return;
  const int qh0 = kvh * G;
  // this wave's contiguous share of the split, a multiple of 16 tokens
  const int sub = ceil_div(ceil_div(sc.hi - sc.lo, kWaves), 16) * 16;
  const int wlo = min(sc.hi, sc.lo + wave * sub);
  const int whi = min(sc.hi, wlo + sub);
  const int32_t* row = sc.row;
  const int n_slots = sc.n_slots;
  const int64_t row_stride = sc.row_stride;

  const char* kbase = (const char*)a.k + (int64_t)kvh * Gm::ROW + 16 * c;
  const char* vbase = (const char*)a.v + (int64_t)kvh * Gm::ROW + 16 * c;
  // chunk k of this lane is row chunk c + LPR k

  // slot ids of the first super-tile: two per lane, issued before anything waits
  int ids[2];
  if (wlo < whi) {
#pragma unroll
    for (int j = 0; j < 2; ++j) ids[j] = row[min(wlo + lane + 64 * j, whi - 1)];
  }

  // q chunks of the g heads, in the same lane layout as K.
  u32x4 q[G][CH];
  const char* qbase = (const char*)a.q + ((int64_t)b * a.n_q_heads + qh0) * Gm::ROW + 16 * c;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < CH; ++k)
      q[h][k] = *(const u32x4*)(qbase + (int64_t)h * Gm::ROW + 16 * LPR * k);

  // with the ids and q in flight, so that its wait overlaps them
  store_new_token<T, D>(a, sc, b, kvh, wlo, whi, lane);

  const float scale2 = a.scale * kLog2e;
  State<T, D, G, LPR> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.l[h] = 0.f;
    st.m[h] = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[h][e] = 0.f;
  }

  int* slots = slot_lds[wave];
  for (int cb = wlo; cb < whi; cb += kSuper) {
    const int ce = min(whi, cb + kSuper);
#pragma unroll
    for (int j = 0; j < 2; ++j) slots[lane + 64 * j] = clamp_index(ids[j], n_slots);
    // other lanes of this wave read these ids: order the LDS writes first
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // prefetch the next super-tile's ids while this one runs
    const int nb = cb + kSuper;
    if (nb < whi) {
#pragma unroll
      for (int j = 0; j < 2; ++j) ids[j] = row[min(nb + lane + 64 * j, whi - 1)];
    }
    super_tile<T, D, G, LPR>(st, slots, cb, ce, grp, kbase, vbase, row_stride, q, scale2);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // before the next pass rewrites the ids
  }

  // Sum over the token groups (lanes c + LPR grp with equal c hold the same
  // elements). The accumulators, one flat array of G * E per lane, go through
  // a reduce-scatter: each halving step exchanges one half with the partner
  // group and adds, so each lane ends with the complete sums of a contiguous
  // run of NPL of them (within one head, chunk-aligned), stored to LDS as is.
  // The G row sums are summed over all groups in every lane.
  constexpr int NV = G * E;
  constexpr int NPL = NV / (64 / LPR);  // values each lane ends with
  constexpr int RUN = NPL < Gm::EPC ? NPL : Gm::EPC;  // contiguous elements per store
  static_assert(NPL % RUN == 0 && E % RUN == 0, "runs stay inside one chunk of one head");
  float v[NV];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) v[h * E + e] = st.acc[h][e];
  const int first = group_reduce_scatter<LPR, NV>(v, lane);  // index of this lane's v[0]
  auto over_groups = [&](float x) {
    if constexpr (LPR == 8) x += dpp<kRowRor8>(x);
    return add_xor32(add_xor16(x));
  };
#pragma unroll
  for (int h = 0; h < G; ++h) st.l[h] = over_groups(st.l[h]);
  // Hand the wave's (m, l, acc) to LDS; an empty wave leaves m = -inf, l = 0, acc = 0.
#pragma unroll
  for (int k = 0; k < NPL; k += RUN) {
    const int idx = first + k;
    const int h = idx / E, ee = idx % E;
    float* dst = red_acc + wave * wstride + h * D + (c + LPR * (ee / Gm::EPC)) * Gm::EPC +
                 ee % Gm::EPC;
    if constexpr (RUN % 4 == 0) {
#pragma unroll
      for (int r = 0; r < RUN; r += 4)
        *(float4*)(dst + r) = make_float4(v[k + r], v[k + r + 1], v[k + r + 2], v[k + r + 3]);
    } else {
#pragma unroll
      for (int r = 0; r < RUN; ++r) dst[r] = v[k + r];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      red_ml[wave][h][0] = st.m[h];
      red_ml[wave][h][1] = st.l[h];
    }
  }
  __syncthreads();

  finish_split<T, D, G, kWaves>(a, red_acc, wstride, red_ml, b, kvh, s, sc);
}

// One workgroup per (request b, KV head, split s), grid (Hkv, max_splits, B),
// plus one more row of splits (s = max_splits) when the index step is fused.
// Optional fused steps:
//   a.kv_indptr_out / loc_out / splits_out: workgroup (0, max_splits, 0) runs
//     the index step for the whole batch, beside the split workgroups (so no
//     split waits for it) and the rest of that row exits at once;
//   a.k_new / v_new: the wave whose share holds position L-1 first stores the
//     new token's K/V row of this KV head at slot req_to_token[r_b, L-1]
//     (skipped if that slot is out of range), then reads it like any other;
//   a.out: requests with one split are finished here (their normalised output
//     is the result) and padded requests get zero rows; requests with more
//     splits leave partials for the merge kernel.
template <typename T, int D, int G>
__global__ __launch_bounds__(64 * kWaves) void decode_partial_kernel(DecodeArgs a) {
  __shared__ int slot_lds[kWaves][kSuper];
  __shared__ float red_acc[kWaves][G][D];
  __shared__ float red_ml[kWaves][G][2];
  // KV head fastest: workgroups go to the XCDs round-robin by linear id, so
  // each XCD gets the same KV head(s) of every split of every request, and
  // requests with few splits do not pile their work onto a few XCDs.
  const int kvh = blockIdx.x;
  const int s = blockIdx.y;
  const int b = blockIdx.z;
  if (s == a.split.max_splits) {  // the index-step row
    if (kvh == 0 && b == 0) index_step_block<64 * kWaves>(a, &slot_lds[0][0]);
    return;
  }
  decode_split<T, D, G>(a, kvh, s, b, slot_lds, &red_acc[0][0][0], G * D, red_ml);
}

// One wave per (request, q head). Splits are taken 32 at a time: all 32
// partial rows and (m, l) pairs of a group are loaded before anything waits
// (one memory round trip for up to 32 splits), the group's weights
// w_s = l_s exp(m_s - M) are computed one split per lane and shared through
// LDS, and the running stabiliser M is raised between groups (acc and the
// weight sum rescaled), so the result is sum_s w_s o_s / sum_s w_s. The first
// group is loaded together with the request's length words, before the split
// count is known: the workspace holds max_splits rows per head, and rows past
// the count are replaced by zeros (their contents are stale) before use.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;  // elements per lane
  constexpr int U = 32;        // splits per group
  __shared__ float wts[U];
  const int lane = threadIdx.x;
  const int b = blockIdx.y;
  // q head of this workgroup: on the XCD that wrote its partials when the
  // KV-head count allows (a bijection of [0, Hq)); bounded before any index
  const int h = merge_head_of(blockIdx.x, a.n_q_heads, a.n_kv_heads);
  if (h < 0 || h >= a.n_q_heads) return;
  const int64_t part = ((int64_t)b * a.n_q_heads + h) * a.split.max_splits;
  const float2* ml = (const float2*)(a.ml_part + 2 * part);
  const float* o = a.o_part + part * D + lane * PER;
  float ov[U][PER];
  float2 mlv;
  // rows c0 .. c0 + U - 1 (clamped to the workspace) and this lane's (m, l)
  auto load_group = [&](int c0, int last) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < PER; ++e) ov[u][e] = o[(int64_t)min(c0 + u, last) * D + e];
    mlv = ml[min(c0 + lane, last)];
  };
  load_group(0, a.split.max_splits - 1);
  int L_raw = load_uniform(a.seq_lens + b);
  int P_raw = load_uniform((a.prefix_len ? a.prefix_len : a.seq_lens) + b);
  // the group's loads stay above this point; the plan's first use stays below
  asm volatile("" : "+s"(L_raw), "+s"(P_raw)::"memory");
  const Plan pl = plan_from(a, L_raw, P_raw);
  const int S = pl.Sp + pl.S;  // prefix splits first, then the suffix splits
  // After the partial kernel ran with an output, requests without prefix
  // splits and with 0 or 1 suffix split are already written.
  if (a.merge_multi_only && pl.Sp == 0 && pl.S <= 1) return;
  const int64_t orow = ((int64_t)b * a.n_q_heads + h) * D + lane * PER;
  if (S <= 1) {  // no split: zeros; one split: its normalised output is the result
#pragma unroll
    for (int e = 0; e < PER; ++e) store_out<T>(a.out, orow + e, S == 1 ? ov[0][e] : 0.f);
    return;
  }
  float M = -INFINITY, den = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int c0 = 0; c0 < S; c0 += U) {
    const int n = min(U, S - c0);
    if (c0 > 0) load_group(c0, S - 1);
    // drop what lies past the request's splits (zero weight, zero row)
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < PER; ++e) ov[u][e] = u < n ? ov[u][e] : 0.f;
    if (lane >= n) mlv = make_float2(-INFINITY, 0.f);
    const float Mn = fmaxf(M, wave_max(mlv.x));  // finite: the group is not empty
    const float r = __builtin_amdgcn_exp2f((M - Mn) * kLog2e);  // 0 on the first group
    M = Mn;
    den *= r;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= r;
    const float w = lane < n ? mlv.y * __builtin_amdgcn_exp2f((mlv.x - M) * kLog2e) : 0.f;
    den += w;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // earlier reads of wts first
    if (lane < U) wts[lane] = w;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wu = wts[u];  // 0 past the group's end
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(wu, ov[u][e], acc[e]);
    }
  }
  // sum of the weights over the wave (every lane gets the same bits)
  den = wave_sum(den);
  const float inv = 1.0f / den;
#pragma unroll
  for (int e = 0; e < PER; ++e) store_out<T>(a.out, orow + e, acc[e] * inv);
}

// Group sizes above MAXG are served by another kernel (the bf16 MFMA one) and
// are not instantiated here.
template <typename T, int D, int MAXG = 16>
hipError_t partials_for_dim(const DecodeArgs& a, hipStream_t stream) {
  const int g = a.n_q_heads / a.n_kv_heads;
  dim3 grid(a.n_kv_heads, a.split.max_splits + (fuses_index_step(a) ? 1 : 0), a.batch);
  switch (g) {
    case 1: decode_partial_kernel<T, D, 1><<<grid, 64 * kWaves, 0, stream>>>(a); break;
    case 2: decode_partial_kernel<T, D, 2><<<grid, 64 * kWaves, 0, stream>>>(a); break;
    case 4: decode_partial_kernel<T, D, 4><<<grid, 64 * kWaves, 0, stream>>>(a); break;
    case 8:
      if constexpr (MAXG >= 8) {
        decode_partial_kernel<T, D, 8><<<grid, 64 * kWaves, 0, stream>>>(a);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    case 16:
      if constexpr (MAXG >= 16) {
        decode_partial_kernel<T, D, 16><<<grid, 64 * kWaves, 0, stream>>>(a);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t merge_for_dim(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.n_q_heads, a.batch);
  decode_merge_kernel<T, D><<<grid, 64, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace decode_impl
}  // namespace pkv
