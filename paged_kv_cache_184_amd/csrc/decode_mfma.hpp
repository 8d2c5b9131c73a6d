// Split-KV paged decode on bf16 MFMA for large query groups (a3), the
// companion of the VALU kernel in decode_impl.hpp. Same grid, fused steps,
// partial layout and merge; only the per-wave inner loop differs.
//
// With g >= 8 query heads per KV head, the VALU kernel spends most of its
// instructions on per-head dot products and lane reductions. Here the g heads
// of a KV head are the 16 columns of an MFMA tile (unused columns hold zero
// queries), so per 32-key block a wave issues 2*D/32 MFMAs for S^T = K Q^T,
// D/16 for O^T += V^T P^T and one for the row sums, and its VALU work is 8
// softmax values per lane.
//   * K goes from global memory straight into the MFMA A operand (lane l loads
//     16 bytes of key l%16's row at byte 16*(l/16) + 64*ks); K and V of a
//     block are a ring of two register blocks.
//   * V rows are loaded into registers in the layout of a wave-wide 1 KiB
//     LDS transfer, written to a per-wave LDS tile (rows XOR-swizzled) when
//     their block is computed, and read back transposed with
//     ds_read_b64_tr_b16 as the A operand of O^T; P^T comes straight out of
//     the S^T accumulator layout as the B operand. (Direct-to-LDS loads would
//     save the registers, but with them in flight the compiler waits for all
//     outstanding loads before any register load is used.)
//   * Each block's loads are issued one block ahead of its use in straight-
//     line code per 128-key super-block, so every wait count is static.
//   * 8 KiB of LDS per wave (the wave-merge buffer reuses it) and at most 256
//     registers: two or more workgroups share a CU, so one hides the others'
//     start-up and drain.
//   * Online softmax in base 2 per head (lane column), with the same lazy
//     stabiliser as the VALU kernel; P is rounded to bf16 and the row sums are
//     those rounded values summed by one more MFMA (a ones operand times P^T).
#pragma once

#include "decode_impl.hpp"

namespace pkv {
namespace decode_mfma {

using decode_impl::finish_split;
using decode_impl::index_step_block;
using decode_impl::kLog2e;
using decode_impl::kTau;
using decode_impl::split_setup;
using decode_impl::SplitCtx;
using decode_impl::store_new_token;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kW = 4;      // waves per workgroup
constexpr int kBlk = 32;   // keys per block: two 16-key MFMA tiles
constexpr int kSB = 4;     // blocks per super-block (slot ids staged per super-block)
constexpr int kRing = 2;   // blocks in flight per wave (ring of K and V registers)
constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 1.0 in both halves


template <int D>
struct MGeo {
  static constexpr int ROW = D * 2;     // bytes of one (slot, KV head) row
  static constexpr int CPR = ROW / 16;  // 16-byte chunks per row
  static constexpr int KS = D / 32;     // MFMA k-steps over head_dim
  static constexpr int DT = D / 16;     // 16-row tiles of O^T over head_dim
  static constexpr int RPI = 64 / CPR;  // V rows per wave-wide 1 KiB transfer
  static constexpr int NI = kBlk / RPI; // V transfers per block
  static constexpr int VST = kBlk * ROW;  // bytes of one V tile
};

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Byte offset of logical 16-byte chunk c of row r in a swizzled V tile.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  return r * MGeo<D>::ROW + 16 * (c ^ (r & (MGeo<D>::CPR - 1)));
}

__device__ __forceinline__ u32x2 tr_read(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Per-lane loads of one 32-key block for a KV storage type. bf16: one
// 16-byte K load per k-step, V in the layout of its LDS tile. FP8 (E4M3
// codes): one 16-byte K load holds the 16 codes of two k-steps (key row
// bytes 16 quad + 64 kl .. +15), widened to bf16 before the MFMAs; V chunks
// are widened to bf16 before they are written to the (bf16) LDS tile.
template <int D, typename KV>
struct KVLd;
template <int D>
struct KVLd<D, bf16_t> {
  static constexpr int ROW = 2 * D;        // bytes of one (slot, KV head) row
  static constexpr int KL = D / 32;        // K loads per key tile
  static constexpr int NV = MGeo<D>::NI;   // V loads per block
};
template <int D>
struct KVLd<D, fp8_t> {
  static constexpr int ROW = D;
  static constexpr int KL = D / 64;
  static constexpr int CPR = D / 16;       // 16-byte chunks per code row
  static constexpr int RPI = 64 / CPR;     // rows per wave-wide 1 KiB load
  static constexpr int NV = kBlk / RPI;
};

template <int D, typename KV = bf16_t>
struct KBlock {
  u32x4 f[2][KVLd<D, KV>::KL];  // K: [key tile][load]
  u32x4 v[KVLd<D, KV>::NV];     // V: this lane's 16 bytes of each 1 KiB row group
};

// Per-wave state for NTC column tiles of 16 query rows each.
template <int D, int NTC>
struct WaveState {
  f32x4 o[NTC][MGeo<D>::DT];  // O^T: lane l holds d = 16 dt + 4 (l/16) + r of column l%16
  f32x4 lsum[NTC];            // row sums (every element of the lane's column)
  float m[NTC];               // stabiliser of column l%16, log2 units
};

template <int D, int NTC>
__device__ __forceinline__ void init_state(WaveState<D, NTC>& st) {
#pragma unroll
  for (int t = 0; t < NTC; ++t) {
#pragma unroll
    for (int dt = 0; dt < MGeo<D>::DT; ++dt) st.o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.lsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m[t] = -INFINITY;
  }
}

// Loads of block i of a super-block into registers: K fragments, and V in
// the layout its LDS tile is written in (lane l of row group t holds row
// RPI t + l / CPR, physical chunk l % CPR). Positions past ce re-read the
// last valid token. kStreamV: V rows (whole lines per load) take the streaming
// policy; launches that re-read the same rows keep the default.
template <int D, typename KV = bf16_t, bool kStreamV = true>
__device__ __forceinline__ void issue_block(KBlock<D, KV>& kb, const int* slots, int i, int cb,
                                            int ce, const char* kbase, const char* vbase,
                                            int64_t row_stride, int lane) {
  using Gm = MGeo<D>;
  using Ld = KVLd<D, KV>;
  const int col = lane & 15;
  const int quad = lane >> 4;
  const int last = ce - cb - 1;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int64_t off = (int64_t)slots[min(kBlk * i + 16 * kt + col, last)] * row_stride;
#pragma unroll
    for (int kl = 0; kl < Ld::KL; ++kl)
      kb.f[kt][kl] = *(const u32x4*)(kbase + off + 16 * quad + 64 * kl);
  }
  if constexpr (sizeof(KV) == 2) {
    const int prow = lane / Gm::CPR;
    const int pch = lane % Gm::CPR;
#pragma unroll
    for (int t = 0; t < Gm::NI; ++t) {
      const int r = Gm::RPI * t + prow;
      const int lch = pch ^ (r & (Gm::CPR - 1));
      const int64_t off = (int64_t)slots[min(kBlk * i + r, last)] * row_stride;
      kb.v[t] = kStreamV ? load_stream(vbase + off + 16 * lch) : *(const u32x4*)(vbase + off + 16 * lch);
    }
  } else {
    // lane l of load t: row RPI t + l / CPR, code chunk l % CPR
#pragma unroll
    for (int t = 0; t < Ld::NV; ++t) {
      const int r = Ld::RPI * t + lane / Ld::CPR;
      const int64_t off = (int64_t)slots[min(kBlk * i + r, last)] * row_stride;
      const char* p = vbase + off + 16 * (lane % Ld::CPR);
      kb.v[t] = kStreamV ? load_stream(p) : *(const u32x4*)p;
    }
  }
}

template <int D, int NTC, typename KV = bf16_t>
__device__ __forceinline__ void compute_block(WaveState<D, NTC>& st, const KBlock<D, KV>& kb,
                                              char* vstage,
                                              const u32x4 (&qf)[NTC][MGeo<D>::KS],
                                              float scale2, int key0, int whi, int lane) {
  using Gm = MGeo<D>;
  using Ld = KVLd<D, KV>;
  const int col = lane & 15;
  const int quad = lane >> 4;
  // V tile into LDS first (read back transposed below, after the S MFMAs;
  // this wave's earlier reads of the tile precede these writes in LDS order)
  if constexpr (sizeof(KV) == 2) {
#pragma unroll
    for (int t = 0; t < Gm::NI; ++t)
      *(u32x4*)(vstage + Gm::RPI * t * Gm::ROW + 16 * lane) = kb.v[t];
  } else {
#pragma unroll
    for (int t = 0; t < Ld::NV; ++t) {
      const int r = Ld::RPI * t + lane / Ld::CPR;
      const int c = lane % Ld::CPR;  // bf16 chunks 2c, 2c + 1 of row r
      u32x4 lo, hi;
      fp8x16_to_bf16x16(kb.v[t], lo, hi);
      *(u32x4*)(vstage + swz<D>(r, 2 * c)) = lo;
      *(u32x4*)(vstage + swz<D>(r, 2 * c + 1)) = hi;
    }
  }
  // K fragments as bf16, k-step ks (FP8: widened from half a 16-byte load)
  u32x4 kf[2][Gm::KS];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int kl = 0; kl < Ld::KL; ++kl) {
      if constexpr (sizeof(KV) == 2)
        kf[kt][kl] = kb.f[kt][kl];
      else
        fp8x16_to_bf16x16(kb.f[kt][kl], kf[kt][2 * kl], kf[kt][2 * kl + 1]);
    }
  u32x4 pf[NTC];
#pragma unroll
  for (int tc = 0; tc < NTC; ++tc) {
    // S^T: keys 16 kt + 4 quad + r, column col of tile tc
    f32x4 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < Gm::KS; ++ks) s[kt] = mfma16(kf[kt][ks], qf[tc][ks], s[kt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = key0 + 16 * kt + 4 * quad + r < whi ? s[kt][r] * scale2 : -INFINITY;
        s[kt][r] = x;
        mx = fmaxf(mx, x);
      }
    if (__builtin_amdgcn_ballot_w64(mx > st.m[tc] + kTau) != 0) {
      float x = fmaxf(mx, __shfl_xor(mx, 16));
      x = fmaxf(x, __shfl_xor(x, 32));
      const float mnew = fmaxf(st.m[tc], x);
      const float corr = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(st.m[tc] - mnew);
      st.lsum[tc] *= corr;
#pragma unroll
      for (int dt = 0; dt < Gm::DT; ++dt) st.o[tc][dt] *= corr;
      st.m[tc] = mnew;
    }
    // P^T in the B-operand layout: slots 0..3 = key tile 0, 4..7 = key tile 1
    const float mm = st.m[tc] == -INFINITY ? 0.f : st.m[tc];
    uint32_t w[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const bf16x2_t pb = {(__bf16)__builtin_amdgcn_exp2f(s[kt][r] - mm),
                             (__bf16)__builtin_amdgcn_exp2f(s[kt][r + 1] - mm)};
        w[2 * kt + r / 2] = __builtin_bit_cast(uint32_t, pb);
      }
    pf[tc] = u32x4{w[0], w[1], w[2], w[3]};
    st.lsum[tc] = mfma16(u32x4{kOnes, kOnes, kOnes, kOnes}, pf[tc], st.lsum[tc]);
  }
  // O^T += V^T P^T. ds_read_b64_tr_b16 hands lane i of each 16-lane group
  // element i%4 of the 8-byte segments of lanes i/4, i/4+4, i/4+8, i/4+12;
  // pointing those at keys 4 quad + (0..3) (+16) and columns 16 dt + 4 (col%4)
  // gives every lane its column's values in the key order of P^T. One V^T
  // fragment serves every column tile.
  const int s4 = col & 3;
  const int r0 = 4 * quad + (col >> 2);
#pragma unroll
  for (int dt = 0; dt < Gm::DT; ++dt) {
    const int chunk = 2 * dt + (s4 >> 1);
    const int half = 8 * (s4 & 1);
    const u32x2 lo = tr_read(vstage + swz<D>(r0, chunk) + half);
    const u32x2 hi = tr_read(vstage + swz<D>(r0 + 16, chunk) + half);
    const u32x4 va = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
    for (int tc = 0; tc < NTC; ++tc) st.o[tc][dt] = mfma16(va, pf[tc], st.o[tc][dt]);
  }
}

// NB consecutive 32-key blocks of one super-block, straight-line: block i's
// loads are issued kRing - 1 blocks before its compute, into ring entry
// i % kRing.
template <int D, int NTC, int NB, typename KV = bf16_t, bool kStreamV = true>
__device__ __forceinline__ void block_run(WaveState<D, NTC>& st, char* vstage, const int* slots,
                                          int cb, int ce, const u32x4 (&qf)[NTC][MGeo<D>::KS],
                                          const char* kbase, const char* vbase,
                                          int64_t row_stride, float scale2, int whi, int lane) {
  KBlock<D, KV> kb[kRing];
#pragma unroll
  for (int j = 0; j < kRing - 1; ++j)
    if (j < NB)
      issue_block<D, KV, kStreamV>(kb[j], slots, j, cb, ce, kbase, vbase, row_stride, lane);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (i + kRing - 1 < NB)
      issue_block<D, KV, kStreamV>(kb[(i + kRing - 1) % kRing], slots, i + kRing - 1, cb, ce,
                                   kbase, vbase, row_stride, lane);
    // keep the later blocks' loads ahead of this block's MFMAs
    __builtin_amdgcn_sched_barrier(0);
    compute_block<D, NTC, KV>(st, kb[i % kRing], vstage, qf, scale2, cb + kBlk * i, whi, lane);
  }
}

// A wave's contiguous key range [wlo, whi) of one request row, in 128-key
// super-blocks: the slot ids of each are staged in this wave's LDS row (the
// next super-block's prefetched into registers meanwhile).
template <int D, int NTC, typename KV = bf16_t, bool kStreamV = true>
__device__ __forceinline__ void wave_loop(WaveState<D, NTC>& st, int* slots, char* vtile,
                                          const int32_t* row, int n_slots, int wlo, int whi,
                                          const u32x4 (&qf)[NTC][MGeo<D>::KS], const char* kbase,
                                          const char* vbase, int64_t row_stride, float scale2,
                                          int lane) {
  constexpr int SBK = kSB * kBlk;  // keys per super-block
  int ids[SBK / 64];
  if (wlo < whi) {
#pragma unroll
    for (int j = 0; j < SBK / 64; ++j) ids[j] = row[min(wlo + lane + 64 * j, whi - 1)];
  }
  for (int cb = wlo; cb < whi; cb += SBK) {
    const int ce = min(whi, cb + SBK);
#pragma unroll
    for (int j = 0; j < SBK / 64; ++j) slots[lane + 64 * j] = clamp_index(ids[j], n_slots);
    // other lanes of this wave read these ids: order the LDS writes first
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const int nb = cb + SBK;
    if (nb < whi) {
#pragma unroll
      for (int j = 0; j < SBK / 64; ++j) ids[j] = row[min(nb + lane + 64 * j, whi - 1)];
    }
    switch (ceil_div(ce - cb, kBlk)) {
#define PKV_DM_RUN(n)                                                                          \
  case n:                                                                                      \
    if constexpr (n <= kSB)                                                                    \
      block_run<D, NTC, n, KV, kStreamV>(st, vtile, slots, cb, ce, qf, kbase, vbase, row_stride, \
                                         scale2, whi, lane);                                   \
    break;
      PKV_DM_RUN(1) PKV_DM_RUN(2) PKV_DM_RUN(3) PKV_DM_RUN(4)
      PKV_DM_RUN(5) PKV_DM_RUN(6) PKV_DM_RUN(7) PKV_DM_RUN(8)
#undef PKV_DM_RUN
      default: break;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // before the next pass rewrites the ids
  }
}

// The work of one (KV head kvh, split s, request b) workgroup of kW waves.
// LDS comes from the caller: the per-wave V tiles vs0 (which also take the
// waves' merge rows), slot ids slot_lds[kW][kSB * kBlk] and red_ml.
template <int D, int G, typename KV = bf16_t>
__device__ __forceinline__ void mfma_split(const DecodeArgs& a, int kvh, int s, int b,
                                           char (*vs0)[MGeo<D>::VST], int (*slot_lds)[kSB * kBlk],
                                           float (*red_ml)[G][2]) {
  using Gm = MGeo<D>;
  constexpr bool kFp8 = sizeof(KV) == 1;
  static_assert(G <= 16, "one MFMA column per query head");
  static_assert(G * D * 4 <= Gm::VST, "a wave's merge rows fit in its V tile");
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int quad = lane >> 4;

  SplitCtx sc;
  if (!split_setup<KV, D, G, 64 * kW>(a, b, kvh, s, sc)) return;
  // this wave's contiguous share of the split, a multiple of 32 tokens
  const int sub = ceil_div(ceil_div(sc.hi - sc.lo, kW), kBlk) * kBlk;
  const int wlo = min(sc.hi, sc.lo + wave * sub);
  const int whi = min(sc.hi, wlo + sub);
  store_new_token<KV, D>(a, sc, b, kvh, wlo, whi, lane);

  const char* kbase = (const char*)a.k + (int64_t)kvh * KVLd<D, KV>::ROW;
  const char* vbase = (const char*)a.v + (int64_t)kvh * KVLd<D, KV>::ROW;
  // Q^T fragments (B operand), column col = head, zero past the group. k-step
  // ks holds head_dim 32 ks + 8 quad .. +7 for bf16 K; for FP8 K it holds the
  // elements the K loads put there: 64 (ks/2) + 16 quad + 8 (ks%2) .. +7.
  const int qh0 = kvh * G;
  u32x4 qf[1][Gm::KS];
  const char* qp =
      (const char*)a.q + ((int64_t)b * a.n_q_heads + qh0 + min(col, G - 1)) * Gm::ROW;
#pragma unroll
  for (int ks = 0; ks < Gm::KS; ++ks) {
    const int byte = kFp8 ? 128 * (ks / 2) + 32 * quad + 16 * (ks % 2) : 64 * ks + 16 * quad;
    const u32x4 v = *(const u32x4*)(qp + byte);
    qf[0][ks] = col < G ? v : u32x4{0u, 0u, 0u, 0u};
  }
  // FP8: the K scale folds into the softmax scale, the V scale into O
  const float kscale = kFp8 ? a.kv_scale[0] : 1.f;
  const float vscale = kFp8 ? a.kv_scale[1] : 1.f;
  WaveState<D, 1> st;
  init_state(st);
  wave_loop<D, 1, KV>(st, slot_lds[wave], vs0[wave], sc.row, sc.n_slots, wlo, whi, qf, kbase,
                      vbase, sc.row_stride, a.scale * kLog2e * kscale, lane);

  // Hand the wave's (m, l, O) to LDS; an empty wave leaves m = -inf, l = 0, O = 0.
  // The O rows go into this wave's V tile (its transpose reads have returned:
  // their results fed the last MFMAs).
  if (col < G) {
    float* mine = (float*)vs0[wave];
#pragma unroll
    for (int dt = 0; dt < Gm::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        mine[col * D + 16 * dt + 4 * quad + r] = kFp8 ? st.o[0][dt][r] * vscale : st.o[0][dt][r];
    if (quad == 0) {
      red_ml[wave][col][0] = st.m[0];
      red_ml[wave][col][1] = st.lsum[0][0];
    }
  }
  __syncthreads();
  finish_split<KV, D, G, kW>(a, (const float*)&vs0[0][0], Gm::VST / 4, red_ml, b, kvh, s, sc);
}

template <int D, int G, typename KV>
__global__ __launch_bounds__(64 * kW, 2) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char vs0[kW][MGeo<D>::VST];
  __shared__ int slot_lds[kW][kSB * kBlk];
  __shared__ float red_ml[kW][G][2];
  const int kvh = blockIdx.x;  // KV head fastest: XCD-balanced (see decode_impl.hpp)
  const int s = blockIdx.y;
  const int b = blockIdx.z;
  if (s == a.split.max_splits) {  // the index-step row (see decode_partial_kernel)
    if (kvh == 0 && b == 0) index_step_block<64 * kW>(a, &slot_lds[0][0]);
    return;
  }
  mfma_split<D, G, KV>(a, kvh, s, b, vs0, slot_lds, red_ml);
}

// bf16 pools use this kernel for g >= 8 (the VALU kernel takes smaller
// groups); FP8 pools use it for every group size.
template <int D, typename KV = bf16_t>
hipError_t partials_for_dim(const DecodeArgs& a, hipStream_t stream) {
  const int g = a.n_q_heads / a.n_kv_heads;
  dim3 grid(a.n_kv_heads, a.split.max_splits + (fuses_index_step(a) ? 1 : 0), a.batch);
  if constexpr (sizeof(KV) == 1) {
    switch (g) {
      case 1: decode_mfma_kernel<D, 1, KV><<<grid, 64 * kW, 0, stream>>>(a); return hipGetLastError();
      case 2: decode_mfma_kernel<D, 2, KV><<<grid, 64 * kW, 0, stream>>>(a); return hipGetLastError();
      case 4: decode_mfma_kernel<D, 4, KV><<<grid, 64 * kW, 0, stream>>>(a); return hipGetLastError();
      default: break;
    }
  }
  switch (g) {
    case 8: decode_mfma_kernel<D, 8, KV><<<grid, 64 * kW, 0, stream>>>(a); break;
    case 16: decode_mfma_kernel<D, 16, KV><<<grid, 64 * kW, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace decode_mfma
}  // namespace pkv
