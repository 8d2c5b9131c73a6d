// Cascade (shared-prefix) decode: the K/V of a prefix shared by a group of
// requests is read once per group, in the same launch as every request's
// private suffix.
//
// AstrAI commit 398e8a3e page, bullets on rebuilding request mappings for
// cached prefix pages and on regressions for prefix reuse; commit e58a728b
// page, bullet on packing prompts with a shared prefix start: requests of a
// group map their first P positions to the same slots. Attention is a sum
// over keys, so the prefix keys can be taken once for all members: split s of
// the prefix (the split rule under a cap of max_splits / 2) gives every
// member's every query head a partial (o, m, l), written at partial index s;
// the member's suffix splits follow at indices Sp.. (the rest of the cap) and
// the merge combines all of them exactly as for a plain decode.
//
// One launch, grid (Hkv, max_splits, n_groups * n_tiles + B):
//   * z < n_groups * n_tiles: prefix workgroups, placed first so the shared
//     work starts first. Group z / n_tiles, column tile z % n_tiles: the 16
//     columns of one MFMA tile hold the (member, q head) pairs of 16 / g
//     members; the wave loop is the MFMA decode kernel's (K into the MFMA A
//     operand, V staged through a per-wave LDS tile and read back
//     transposed), so each K/V fragment serves all of the tile's members.
//   * z >= n_groups * n_tiles: the regular decode work of request
//     z - n_groups * n_tiles (bf16 pools: VALU kernel for g <= 4, MFMA kernel
//     for g >= 8; E4M3 pools: MFMA kernel), whose split plan places its suffix
//     splits after the prefix ones.
// Both kinds share one LDS layout (the MFMA V tiles also hold the wave-merge
// rows), so the launch keeps two workgroups per CU.
#include "decode_mfma.hpp"

namespace pkv {
namespace {

using namespace decode_mfma;
using decode_impl::plan_for;
using decode_impl::Plan;
using decode_impl::prefix_cap;

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kCols = 16;  // MFMA columns of one prefix workgroup

static_assert(decode_impl::kSuper == kSB * kBlk, "the two decode loops stage equal slot blocks");

// Prefix split s of group grp for members [tile * cpm, tile * cpm + cpm) of
// the group, cpm = 16 / g. Column c is (member tile * cpm + c / g, head c % g).
// The prefix's split plan and slots are those of the group's first member; a
// member whose own prefix length differs gets no prefix partials here.
template <int D, typename KV>
__device__ __forceinline__ void prefix_split(const DecodeArgs& a, int kvh, int s, int grp,
                                             int tile, char (*vs0)[MGeo<D>::VST],
                                             int (*slot_lds)[kSB * kBlk],
                                             float (*red_ml)[kCols][2]) {
  using Gm = MGeo<D>;
  constexpr bool kFp8 = sizeof(KV) == 1;
  constexpr int ROW = KVLd<D, KV>::ROW;  // bytes of a stored (slot, KV head) row
  static_assert(kCols * D * 4 <= Gm::VST, "a wave's merge rows fit in its V tile");
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int quad = lane >> 4;
  const int gq = a.n_q_heads / a.n_kv_heads;  // query heads per KV head, <= 16
  const int cpm = kCols / gq;                 // members per column tile

  const int m0 = clamp_index(a.group_indptr[grp], a.n_members);
  int M = a.group_indptr[grp + 1] - a.group_indptr[grp];
  M = M < 0 ? 0 : (M > a.max_members ? a.max_members : M);
  if (M > a.n_members - m0) M = a.n_members - m0;  // positions stay inside members[]
  const int j0 = tile * cpm;
  if (j0 >= M) return;
  const int nm = min(cpm, M - j0);  // members of this tile
  const int b0 = clamp_index(a.group_members[m0], a.batch);
  const Plan pl = plan_for(a, b0);
  if (s >= pl.Sp) return;
  int chunk_p;
  split_count(pl.P, prefix_cap(a.split.max_splits), a.split.fixed_splits, a.split.split_tokens,
              &chunk_p);
  const int lo = s * chunk_p;
  const int hi = min(pl.P, lo + chunk_p);
  const int sub = ceil_div(ceil_div(hi - lo, kW), kBlk) * kBlk;
  const int wlo = min(hi, lo + wave * sub);
  const int whi = min(hi, wlo + sub);
  const int32_t* row =
      a.req_to_token + (int64_t)clamp_index(a.req_pool_indices[b0], a.n_rows) * a.stride;
  const int n_slots = (int)(a.n_slots > 0x7fffffff ? 0x7fffffff : a.n_slots);
  const int64_t row_stride = (int64_t)a.n_kv_heads * ROW;

  // this lane's column: member bj, head hh; zero query unless it is a member
  // of this tile with the group's prefix length
  const int hh = col % gq;
  const int bj = clamp_index(a.group_members[m0 + j0 + min(col / gq, nm - 1)], a.batch);
  const bool valid = col < nm * gq && plan_for(a, bj).P == pl.P;
  u32x4 qf[1][Gm::KS];
  const char* qp =
      (const char*)a.q + ((int64_t)bj * a.n_q_heads + (int64_t)kvh * gq + hh) * Gm::ROW;
  // k-step order of the K loads (E4M3 loads carry two k-steps), as in the
  // MFMA decode kernel
#pragma unroll
  for (int ks = 0; ks < Gm::KS; ++ks) {
    const int byte = kFp8 ? 128 * (ks / 2) + 32 * quad + 16 * (ks % 2) : 64 * ks + 16 * quad;
    const u32x4 v = *(const u32x4*)(qp + byte);
    qf[0][ks] = valid ? v : u32x4{0u, 0u, 0u, 0u};
  }
  const char* kbase = (const char*)a.k + (int64_t)kvh * ROW;
  const char* vbase = (const char*)a.v + (int64_t)kvh * ROW;
  // E4M3 pools: the K scale joins the softmax scale, the V scale the outputs
  const float kscale = kFp8 ? a.kv_scale[0] : 1.f;
  const float vscale = kFp8 ? a.kv_scale[1] : 1.f;
  WaveState<D, 1> st;
  init_state(st);
  // the column tiles of a group re-read these rows: default cache policy
  wave_loop<D, 1, KV, false>(st, slot_lds[wave], vs0[wave], row, n_slots, wlo, whi, qf, kbase, vbase,
                      row_stride, a.scale * kLog2e * kscale, lane);

  // Hand the wave's (m, l, O) per column to LDS (O rows into the wave's own V
  // tile, whose transpose reads have returned); wave 0 also records each
  // column's request (-1: no output) in its slot block, which it no longer reads.
  float* mine = (float*)vs0[wave];
#pragma unroll
  for (int dt = 0; dt < Gm::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) mine[col * D + 16 * dt + 4 * quad + r] = st.o[0][dt][r] * vscale;
  if (quad == 0) {
    red_ml[wave][col][0] = st.m[0];
    red_ml[wave][col][1] = st.lsum[0][0];
    if (wave == 0) slot_lds[0][col] = valid ? bj : -1;
  }
  __syncthreads();
  // merge the waves (fixed order) into each column's partial at index s
  for (int i = threadIdx.x; i < nm * gq * D; i += 64 * kW) {
    const int c = i / D;
    const int d = i % D;
    const int bc = slot_lds[0][c];
    if (bc < 0) continue;
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kW; ++w) Mx = fmaxf(Mx, red_ml[w][c][0]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const float mw = red_ml[w][c][0];
      const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - Mx);
      num = fmaf(f, ((const float*)vs0[w])[c * D + d], num);
      den = fmaf(f, red_ml[w][c][1], den);
    }
    const int64_t part =
        ((int64_t)bc * a.n_q_heads + (int64_t)kvh * gq + c % gq) * a.split.max_splits + s;
    a.o_part[part * D + d] = num / den;
    if (d == 0) *(float2*)(a.ml_part + 2 * part) = make_float2(Mx * kLn2, den);
  }
}

template <int D, int G, typename KV>
__global__ __launch_bounds__(64 * kW, 2) void cascade_kernel(DecodeArgs a, int n_tiles) {
  __shared__ __attribute__((aligned(1024))) char vs0[kW][MGeo<D>::VST];
  __shared__ int slot_lds[kW][kSB * kBlk];
  __shared__ float red_ml[kW][kCols][2];
  const int kvh = blockIdx.x;  // KV head fastest: XCD-balanced, as in the decode kernels
  const int s = blockIdx.y;
  const int z = blockIdx.z;
  const int n_pz = a.n_groups * n_tiles;
  if (z < n_pz) {
    if (s < prefix_cap(a.split.max_splits))
      prefix_split<D, KV>(a, kvh, s, z / n_tiles, z % n_tiles, vs0, slot_lds, red_ml);
    return;
  }
  float(*ml)[G][2] = (float(*)[G][2]) & red_ml[0][0][0];
  if constexpr (G >= 8 || sizeof(KV) == 1) {
    mfma_split<D, G, KV>(a, kvh, s, z - n_pz, vs0, slot_lds, ml);
  } else {
    static_assert(G * D * 4 <= MGeo<D>::VST, "a wave's merge rows fit in its V tile");
    decode_impl::decode_split<bf16_t, D, G>(a, kvh, s, z - n_pz, slot_lds, (float*)&vs0[0][0],
                                            MGeo<D>::VST / 4, ml);
  }
}

template <int D, typename KV>
hipError_t cascade_for_dim(const DecodeArgs& a, int n_tiles, hipStream_t stream) {
  const int gq = a.n_q_heads / a.n_kv_heads;
  dim3 grid(a.n_kv_heads, a.split.max_splits, a.n_groups * n_tiles + a.batch);
  switch (gq) {
    case 1: cascade_kernel<D, 1, KV><<<grid, 64 * kW, 0, stream>>>(a, n_tiles); break;
    case 2: cascade_kernel<D, 2, KV><<<grid, 64 * kW, 0, stream>>>(a, n_tiles); break;
    case 4: cascade_kernel<D, 4, KV><<<grid, 64 * kW, 0, stream>>>(a, n_tiles); break;
    case 8: cascade_kernel<D, 8, KV><<<grid, 64 * kW, 0, stream>>>(a, n_tiles); break;
    case 16: cascade_kernel<D, 16, KV><<<grid, 64 * kW, 0, stream>>>(a, n_tiles); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int cascade_tiles(int n_q_heads, int n_kv_heads, int max_members) {
  const int cpm = kCols / (n_q_heads / n_kv_heads);
  return (max_members + cpm - 1) / cpm;
}

hipError_t launch_cascade_partials(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const int n_tiles = a.n_groups > 0 ? cascade_tiles(a.n_q_heads, a.n_kv_heads, a.max_members) : 0;
  if (a.dtype == PKV_FP8_E4M3)
    return a.head_dim == 128 ? cascade_for_dim<128, fp8_t>(a, n_tiles, stream)
                             : cascade_for_dim<64, fp8_t>(a, n_tiles, stream);
  return a.head_dim == 128 ? cascade_for_dim<128, bf16_t>(a, n_tiles, stream)
                           : cascade_for_dim<64, bf16_t>(a, n_tiles, stream);
}

}  // namespace pkv
