// Ragged packed paged prefill (a5) on gfx950 bf16 MFMA.
//
// AstrAI commit e58a728b page: prompts (possibly sharing a prefix start) are
// packed into one forward and located by cumulative query lengths; the CUDA
// backend's prefill reads a paged cache. AstrAI commit 398e8a3e page: cached
// prefix pages are reused, K/V are addressed through the int32 slot table.
// New token i of request b (packed row qo_indptr[b] + i) sees positions
// 0 .. L_b - n_b + i (bottom-right causal) or all L_b positions.
//
// Workgroup = 4 waves = one tile of 128 query rows of one (request, KV head):
// rows are (token, q head) pairs, row = token * g + head, so the g heads that
// share a KV head share every K/V tile (BQ = 128 / g tokens per tile).
//
// Per 64-key block:
//   * K and V rows are gathered through the slot table straight into LDS
//     (16-byte-per-lane buffer loads with the LDS bit, no registers; the
//     global form for pools past 32-bit offsets), row-major with the 16-byte
//     chunks of row r XOR-swizzled (K by r, V by 2r: each tile's reads then
//     meet no LDS bank conflict), into a two-stage ring: the next block
//     is in flight while one is computed, its transfers spread over the
//     current block's S^T MFMA groups. Each wave waits for its own transfers
//     with an explicit vmcnt; one barrier per block then publishes the stage
//     and frees the other one. Slot ids arrive the same way two blocks ahead,
//     so the queue is never drained inside the loop. The ring (66 KiB) and a
//     256-register cap let two workgroups share a CU, so one wave's softmax
//     overlaps the other's MFMAs on each SIMD.
//   * each wave computes S^T = K Q^T for its 32 rows with
//     v_mfma_f32_16x16x32_bf16 (K from LDS as the A operand, Q^T held in
//     registers as the B operand for the whole tile);
//   * softmax in base 2 with a per-row stabiliser that is raised only when a
//     score exceeds it by more than kTau (seen as a row sum above 2^kTau; the
//     scale folds into the exponent's FMA); P is rounded to bf16 and the row
//     sums are those rounded values summed by one more MFMA (a ones operand
//     times P^T);
//   * O^T += V^T P^T with the same MFMA: P^T comes straight out of the S^T
//     accumulator layout (lane l holds keys 4(l/16)+r of two 16-key tiles for
//     query column l%16); V^T comes from the row-major V tile through
//     ds_read_b64_tr_b16, which hands lane i of each 16-lane group element
//     i%4 of the 8-byte segments of lanes i/4, i/4+4, i/4+8, i/4+12: pointing
//     those lanes at keys base+4g+0..3 and columns 16dt+4(s%4) gives every
//     lane the 4 keys it needs at its own column.
// Only blocks that straddle the causal diagonal or the sequence end are
// masked. Up to 64 requests, the (request, tile) items run request by request
// (longest-tile order) and longest tile first within a request (a 1-D launch,
// KV head fastest); larger batches use a (tile, KV head, request) grid, each
// request's longest tiles first.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 128;   // query rows per workgroup
constexpr int kBK = 64;      // keys per block
constexpr int kThreads = 256;
constexpr int kStages = 2;
// log2 headroom of the fixed stabiliser (kTau = 64): a row sum above 2^kTau
// flags the tile
constexpr float kSumLimit = 0x1p64f;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct PGeo {
  static constexpr int ROW = D * 2;              // bytes of a (slot, KV head) row
  static constexpr int CPR = ROW / 16;           // 16-byte chunks per row (8 or 16)
  static constexpr int RPI = 64 / CPR;           // rows per wave-wide 1 KiB transfer
  static constexpr int NI = (kBK / 4) / RPI;     // transfers per wave per tile (K or V)
  static constexpr int TILE = kBK * ROW;         // bytes of one K (or V) tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int KSTEPS = D / 32;          // MFMA k-steps over head_dim
  static constexpr int DT = D / 16;              // 16-wide output tiles over head_dim
};

// Storage side of a K/V row for a pool type: bf16 rows (K and V both by
// direct-to-LDS transfers), or E4M3 code rows (K by direct-to-LDS transfers
// into a code tile; V through registers, widened to bf16 and written into the
// bf16 V tile, so the P.V path is the same for both).
template <int D, typename KV>
struct PStore {
  static constexpr int ROW = D * (int)sizeof(KV);  // bytes of a (slot, KV head) row
  static constexpr int CPR = ROW / 16;             // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;             // rows per wave-wide 1 KiB transfer
  static constexpr int NI = (kBK / 4) / RPI;       // transfers per wave per tile
  static constexpr int KTILE = kBK * ROW;          // bytes of the K tile
  static constexpr int STAGE = KTILE + PGeo<D>::TILE;  // K tile + bf16 V tile
  // code rows: rows sharing one 256-byte bank line, for the K-tile swizzle
  static constexpr int RPL = ROW >= 256 ? 1 : 256 / ROW;
};

// Byte offset of logical 16-byte chunk c of row r in a K code tile. Each
// group of 16 consecutive rows read at one chunk position hits 16 distinct
// 16-byte bank groups (rows sharing a 256-byte bank line differ in r % RPL,
// the XOR by r / RPL separates the rest).
template <int D>
__device__ __forceinline__ int swz8(int r, int c) {
  using S = PStore<D, fp8_t>;
  return r * S::ROW + 16 * (c ^ ((r / S::RPL) & (S::CPR - 1)));
}

// vmcnt(n) alone (expcnt, lgkmcnt left at their maxima), gfx9 encoding
#define PKV_VMCNT(n) ((((n) & 15)) | (7 << 4) | (15 << 8) | ((((n) >> 4) & 3) << 14))
// lgkmcnt(0) alone (vmcnt, expcnt left at their maxima)
#define PKV_LGKMCNT0 (15 | (7 << 4) | (0 << 8) | (3 << 14))

#define PKV_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define PKV_GLB(p) ((const __attribute__((address_space(1))) void*)(p))

// Buffer descriptor of `bytes` bytes at `base`: no stride, untyped 32-bit
// data format (the third descriptor word of the gfx9 family); an access past
// the range reads zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)0x00020000);
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Byte offset of logical 16-byte chunk c of row r in a swizzled K tile: the
// 16 rows that one K fragment read takes at one chunk position hit 16
// distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  return r * PGeo<D>::ROW + 16 * (c ^ (r & (PGeo<D>::CPR - 1)));
}

// The XOR that places row r's chunks in a V tile. A V^T transpose read takes,
// in each half of the wave, 8 rows at the chunk pair (2dt, 2dt+1); for those
// 16 (row, chunk) pieces to hit 16 distinct bank groups the 8 rows must land
// in 8 distinct chunk pairs (D = 128: XOR by 2r; D = 64, two 128-byte rows
// per 256-byte bank line: XOR by 2 ((r/2) % 4) within each line half).
template <int D>
__device__ __forceinline__ int vxor(int r) {
  return D == 128 ? (2 * r) & 15 : 2 * ((r >> 1) & 3);
}

// Byte offset of logical 16-byte chunk c of row r in a swizzled V tile.
template <int D>
__device__ __forceinline__ int swzv(int r, int c) {
  return r * PGeo<D>::ROW + 16 * (c ^ vxor<D>(r));
}

template <int D>
__device__ __forceinline__ u32x2 tr_read(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// bf16 1.0 in both halves: the A operand whose product with P^T gives the
// row sums of P (every output row of the tile is the same sum).
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;

// One 64-key block for this wave's 32 query rows, taken as two 32-key halves
// j (key tiles 2j, 2j+1). scale2 > 0 (the caller negates Q for a negative
// scale and zeroes it for a zero scale), so the largest scaled score is the
// scaled largest raw score, the scale folds into the exponent's FMA and a
// masked score (-inf) gives weight 0.
//
// The stabiliser m of a row is fixed for the whole pass and O is never
// rescaled here: m is set from the first 32 keys (init). No row maximum is
// taken after that: a later score more than kTau above m shows up as a row
// sum above 2^kTau, which the caller checks once per tile before it
// recomputes the tile with m = the exact row maxima (collected in mseen by a
// TRACK pass). Below that limit the weights, the row sums and O stay far from
// the fp32 / bf16 range limits.
// MASK: the block straddles the causal diagonal or the sequence end (a
// separate instantiation, so unmasked blocks carry no per-score selects).
//
// xfer(t), t < NT, queues transfer t of the next block; the transfers ride
// along with the S groups instead of leaving the barrier as one burst, which
// the CU's memory pipeline takes one at a time while the wave's MFMAs wait
// behind them in its instruction stream.
//
// Issue order. A dependent 16x16x32 MFMA waits about three times the issue
// interval of its predecessor, and an LDS read about as long as four MFMAs,
// so every MFMA group has four independent accumulators and its operands are
// read from LDS one group ahead (explicit scheduling fences keep the order):
//   S^T:  per (half, k-step) group, the K fragments of the half's two key
//         tiles, then the four (key tile, query tile) MFMAs;
//   O^T:  per pair of 16-wide head_dim tiles, four V^T transpose reads, then
//         the four MFMAs; the first group of a half is read before that
//         half's softmax, so the reads overlap the exponentials.
template <int D, int G, bool MASK, typename KV, bool TRACK, int NT, typename X>
__device__ __forceinline__ void attend_block(
    const char* __restrict__ lds_k, const char* __restrict__ lds_v,
    const u32x4 (&qf)[2][PGeo<D>::KSTEPS], f32x4 (&o)[PGeo<D>::DT][2], f32x4 (&lacc)[2],
    float (&m)[2], float (&mseen)[2], bool init, int k0,
    const int (&limit)[2], int wlim, float scale2, int lane, X&& xfer) {
  using Gm = PGeo<D>;
  constexpr int KS = Gm::KSTEPS;
  constexpr bool kFp8 = sizeof(KV) == 1;
  // S groups: bf16 K, one k-step per group; E4M3 K, one 16-byte read holds
  // the codes of k-steps 2kp and 2kp + 1, widened exactly to bf16 (the Q
  // fragments are loaded in the same order)
  constexpr int SG = kFp8 ? KS / 2 : KS;  // S groups per half
  constexpr int VG = Gm::DT / 2;          // O groups per half
  const int col = lane & 15;
  const int quad = lane >> 4;
  const int s4 = col & 3;
  const u32x4 ones = u32x4{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
  const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
  // MASK: a half whose first key is past the wave's last visible key (wlim,
  // wave-uniform) adds nothing and is skipped (if half 0 is, so is half 1);
  // the transfers and the operand reads stay unconditional
  bool live[2] = {true, true};
  if constexpr (MASK) {
    live[0] = k0 <= wlim;
    live[1] = k0 + 32 <= wlim;
  }

  // ---- S^T = K Q^T for both halves: sc[j][h][n] is key tile 2j+h x query tile n
  f32x4 sc[2][2][2];
  auto kread = [&](int g, u32x4 (&kb)[2]) {
    const int j = g / SG, ks = g % SG;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 16 * (2 * j + h) + col;
      kb[h] = kFp8 ? *(const u32x4*)(lds_k + swz8<D>(row, quad + 4 * ks))
                   : *(const u32x4*)(lds_k + swz<D>(row, 4 * ks + quad));
    }
  };
  auto smfma = [&](int g, const u32x4 (&kb)[2]) {
    const int j = g / SG, ks = g % SG;
    if constexpr (kFp8) {
      u32x4 lo[2], hi[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) fp8x16_to_bf16x16(kb[h], lo[h], hi[h]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          sc[j][h][n] = mfma16(lo[h], qf[n][2 * ks], ks == 0 ? zero : sc[j][h][n]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int n = 0; n < 2; ++n) sc[j][h][n] = mfma16(hi[h], qf[n][2 * ks + 1], sc[j][h][n]);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          sc[j][h][n] = mfma16(kb[h], qf[n][ks], ks == 0 ? zero : sc[j][h][n]);
    }
  };
  {
    u32x4 kb[2][2];
    kread(0, kb[0]);
#pragma unroll
    for (int g = 0; g < 2 * SG; ++g) {
      if (g + 1 < 2 * SG) kread(g + 1, kb[(g + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      // the next block's transfers, spread over the S groups
#pragma unroll
      for (int t = g * NT / (2 * SG); t < (g + 1) * NT / (2 * SG); ++t) xfer(t);
      if (live[g / SG]) smfma(g, kb[g & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- V^T fragments: group (j, gv) covers head_dim tiles 2gv, 2gv+1 of keys
  // 32j .. 32j+31. Column 16dt + 4(s%4) lives in logical chunk 2dt + (s%4)/2,
  // half (s%2) of the row-major V tile.
  auto vread = [&](int j, int gv, u32x4 (&vb)[2]) {
    const int r0 = 32 * j + 4 * quad + (col >> 2);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int dt = 2 * gv + e;
      const int chunk = 2 * dt + (s4 >> 1);
      const int half = 8 * (s4 & 1);
      const u32x2 lo = tr_read<D>(lds_v + swzv<D>(r0, chunk) + half);
      const u32x2 hi = tr_read<D>(lds_v + swzv<D>(r0 + 16, chunk) + half);
      vb[e] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  };
  u32x4 vb[2][2];
  vread(0, 0, vb[0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (!live[j]) break;
    f32x4 (&s)[2][2] = sc[j];
    // mask (blocks on the causal diagonal or the sequence end only), then the
    // stabiliser check on the raw maxima
    if constexpr (MASK) {
      // key k0 + 32 j + 4 quad + (16 h + r) is visible to row tile n when
      // 16 h + r <= rel[n]: one register per tile, immediates per element
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int rel = limit[n] - (k0 + 32 * j + 4 * quad);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[h][n][r] = 16 * h + r <= rel ? s[h][n][r] : -INFINITY;
      }
    }
    // this lane's raw row maxima of the half block, scaled (scale2 > 0: a
    // fully masked lane keeps -inf)
    auto row_max = [&](int n) {
      const float x = fmaxf(fmaxf(fmaxf(s[0][n][0], s[0][n][1]), fmaxf(s[0][n][2], s[0][n][3])),
                            fmaxf(fmaxf(s[1][n][0], s[1][n][1]), fmaxf(s[1][n][2], s[1][n][3])));
      return x * scale2;
    };
    if (init && j == 0) {
      // first 32 keys of the tile's first pass: the stabiliser is their row
      // maximum (key 0 is visible to every row, so it is finite); O and the
      // row sums are still zero, so nothing is rescaled
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const float mx = row_max(n);
        float x = fmaxf(mx, __shfl_xor(mx, 16));
        m[n] = fmaxf(x, __shfl_xor(x, 32));
      }
    }
    if constexpr (TRACK) {
#pragma unroll
      for (int n = 0; n < 2; ++n) mseen[n] = fmaxf(mseen[n], row_max(n));
    }
    // P^T (bf16) in the B-operand layout: slots 0..3 = key tile 2j, 4..7 = tile 2j+1
    u32x4 pf[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const float nm = m[n] == -INFINITY ? 0.f : -m[n];
      uint32_t w[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          // a masked key (-inf) gives exp2(-inf) = 0
          const bf16x2_t pb = {
              (__bf16)__builtin_amdgcn_exp2f(fmaf(s[h][n][r], scale2, nm)),
              (__bf16)__builtin_amdgcn_exp2f(fmaf(s[h][n][r + 1], scale2, nm))};
          w[2 * h + r / 2] = __builtin_bit_cast(uint32_t, pb);
        }
      }
      pf[n] = u32x4{w[0], w[1], w[2], w[3]};
    }
    // row sums of the rounded P: ones x P^T
    lacc[0] = mfma16(ones, pf[0], lacc[0]);
    lacc[1] = mfma16(ones, pf[1], lacc[1]);
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T P^T, the next group's V^T read ahead (across the halves too)
#pragma unroll
    for (int gv = 0; gv < VG; ++gv) {
      const int q = j * VG + gv;  // running group index
      if (q + 1 < 2 * VG) vread((q + 1) / VG, (q + 1) % VG, vb[(q + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        o[2 * gv + e][0] = mfma16(vb[q & 1][e], pf[0], o[2 * gv + e][0]);
        o[2 * gv + e][1] = mfma16(vb[q & 1][e], pf[1], o[2 * gv + e][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Largest batch whose tiles are ordered by cost (one request per lane of a wave).
constexpr int kSortedMaxBatch = 64;

// Work item k of the ordered launch (batch <= kSortedMaxBatch): items are the
// (request, query tile) pairs, request by request in decreasing cost of the
// request's longest tile (the 64-key blocks it reads; ties in request order),
// each request's tiles longest first; the KV head is fastest, so the heads of
// one item run side by side and, with the KV head count a multiple of 8, each
// XCD serves one head. Keeping a request's tiles together keeps the K/V that
// the tiles in flight share within an XCD's L2 (all requests' K/V of one head
// at once overflow it), and the shortest requests' short tiles end the launch.
// Every wave computes the same answer from the request words (one request per
// lane). Returns false when k is past the last item; otherwise words holds
// request b's raw qo_indptr[b], qo_indptr[b+1], seq_lens[b] and
// req_pool_indices[b] (taken from the lane that loaded them).
template <int BQ>
__device__ bool sorted_item(const PrefillArgs& a, int k, int& b, int& kvh, int& tile,
                            int (&words)[4]) {
  const int lane = threadIdx.x & 63;
  const int item = k / a.n_kv_heads;
  kvh = k - item * a.n_kv_heads;
  // this lane's request, clamped as the tile code clamps it
  int n = 0, P = 0, nt = 0, cmax = 0;
  int raw[4] = {0, 0, 0, 0};
  if (lane < a.batch) {
    raw[0] = a.qo_indptr[lane];
    raw[1] = a.qo_indptr[lane + 1];
    raw[2] = a.seq_lens[lane];
    raw[3] = a.req_pool_indices[lane];
    const int q0 = raw[0], q1 = raw[1];
    int L = raw[2];
    L = L < 0 ? 0 : (L > a.stride ? (int)a.stride : L);
    n = q1 - q0;
    n = n < 0 ? 0 : (n > L ? L : n);
    P = L - n;
    nt = min((n + BQ - 1) / BQ, (a.max_q_len + BQ - 1) / BQ);
    if (nt > 0) {
      const int last_end = a.causal ? P + min(nt * BQ, n) : L;
      cmax = (last_end + kBK - 1) / kBK;
    }
  }
  // the tiles of the requests ordered before this lane's request
  int before = 0;
  for (int i = 0; i < a.batch; ++i) {
    const int ci = __shfl(cmax, i);
    const int ni = __shfl(nt, i);
    before += ci > cmax || (ci == cmax && i < lane) ? ni : 0;
  }
  const bool mine = lane < a.batch && item >= before && item < before + nt;
  const uint64_t owner = __builtin_amdgcn_ballot_w64(mine);
  if (owner == 0) return false;
  b = __builtin_ctzll(owner);
  tile = __shfl(nt - 1 - (item - before), b);
#pragma unroll
  for (int w = 0; w < 4; ++w) words[w] = __shfl(raw[w], b);
  return true;
}

// BUF: the transfers into LDS are buffer loads against descriptors of the
// layer's K and V pools and the request's slot-table row (byte ranges below
// 2^32). With the global form, the compiler counts each LDS transfer in
// flight as an unordered LDS event and turns every wait for an LDS read of
// the block into a wait for all of them; the buffer form keeps those waits
// exact, so the fragment reads issued one group ahead stay in flight.
template <int D, int G, typename KV, bool BUF>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
  using Gm = PGeo<D>;
  using Sg = PStore<D, KV>;
  constexpr bool kFp8 = sizeof(KV) == 1;
  constexpr int BQ = kRows / G;  // tokens per tile
  // One LDS object per ring stage (tiles and slot ids), selected with
  // compile-time indices, so reads of one stage are not ordered behind the
  // transfers into another.
  __shared__ __attribute__((aligned(1024))) char st0[Sg::STAGE];  // K tile, then the bf16 V tile
  __shared__ __attribute__((aligned(1024))) char st1[Sg::STAGE];
  __shared__ __attribute__((aligned(16))) int id0[4][kBK];  // [wave][row]
  __shared__ __attribute__((aligned(16))) int id1[4][kBK];
  __shared__ int redo[4];  // per wave: a score rose past the stabiliser's headroom
  static_assert(kStages == 2, "two ring stages");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform: the LDS destinations of the transfers (M0) are then
  // computed in scalar registers, not read back from a vector lane per transfer
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int kvh, b, tile;
  int q0, q1, L, r_raw;  // the request's words
  if (a.sorted) {
    int w[4];
    if (!sorted_item<BQ>(a, blockIdx.x, b, kvh, tile, w)) return;
    b = __builtin_amdgcn_readfirstlane(b);
    kvh = __builtin_amdgcn_readfirstlane(kvh);
    tile = __builtin_amdgcn_readfirstlane(tile);
    q0 = __builtin_amdgcn_readfirstlane(w[0]);
    q1 = __builtin_amdgcn_readfirstlane(w[1]);
    L = __builtin_amdgcn_readfirstlane(w[2]);
    r_raw = __builtin_amdgcn_readfirstlane(w[3]);
  } else {
    kvh = blockIdx.y;
    b = blockIdx.z;
    tile = gridDim.x - 1 - blockIdx.x;  // longest work of the request first
    // scalar loads, all in flight before any is used
    q0 = load_uniform(a.qo_indptr + b);
    q1 = load_uniform(a.qo_indptr + b + 1);
    L = load_uniform(a.seq_lens + b);
    r_raw = load_uniform(a.req_pool_indices + b);
    asm volatile("" : "+s"(q0), "+s"(q1), "+s"(L), "+s"(r_raw));
  }
  const int t0 = tile * BQ;
  int n_new = q1 - q0;
  if (t0 >= n_new) return;
  L = L < 0 ? 0 : (L > a.stride ? (int)a.stride : L);
  if (n_new > L) n_new = L;
  if (t0 >= n_new) return;
  const int P = L - n_new;
  const int t_last = min(t0 + BQ, n_new) - 1;
  const int kv_end = a.causal ? P + t_last + 1 : L;  // keys the tile can see
  const int kv_full = a.causal ? P + t0 + 1 : L;     // keys every row of the tile sees
  const int nblk = (kv_end + kBK - 1) / kBK;

  const int r = clamp_index(r_raw, a.n_rows);
  const int32_t* row = a.req_to_token + (int64_t)r * a.stride;
  const int n_slots = (int)(a.n_slots > 0x7fffffff ? 0x7fffffff : a.n_slots);
  const int64_t row_stride = (int64_t)a.n_kv_heads * Sg::ROW;

  // This lane's transfer rows and logical chunk: transfer i of this wave
  // covers tile rows 16*wave + RPI*i .. +RPI-1; lane l lands at physical chunk
  // l % CPR of row 16*wave + RPI*i + l / CPR, so it fetches the logical chunk
  // that the swizzle puts there.
  const int prow = lane / Sg::CPR;
  const int pch = lane % Sg::CPR;
  const char* kbase = (const char*)a.k + (int64_t)kvh * Sg::ROW;
  const char* vbase = (const char*)a.v + (int64_t)kvh * Sg::ROW;
  // BUF: every transfer's offset from kbase / vbase is below the span (the
  // launcher takes this form only when the layer's pool is below 0xF0000000
  // bytes); the slot-table row's range ends at the tile's last visible key.
  // A transfer for a block past the end gets offset kNoBlock, past every
  // range: it reads zeros and touches no memory, and the wait counts stay
  // the same in every iteration without a branch around the transfers (a
  // branch there makes the compiler drain all of them before the next LDS
  // read).
  constexpr uint32_t kNoBlock = 0xFFFFFFF0u;
  const uint32_t span = BUF ? (uint32_t)((int64_t)n_slots * row_stride - (int64_t)kvh * Sg::ROW) : 0u;
  const auto krs = make_rsrc(kbase, span);
  const auto vrs = make_rsrc(vbase, span);
  const auto irs = make_rsrc(row, BUF ? 4u * (uint32_t)kv_end : 0u);
  // one 16-byte transfer per lane from base + off into LDS at dst + 16 lane
  auto dma16 = [&](const __amdgpu_buffer_rsrc_t& rs, const char* base, auto off, char* dst) {
    if constexpr (BUF)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, PKV_LDS(dst), 16, (uint32_t)off, 0, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(PKV_GLB(base + off), PKV_LDS(dst), 16, 0, 0);
  };

  // Slot ids of a block arrive by DMA too (one 4-byte transfer per lane into a
  // per-wave ring in LDS), so every vector-memory operation of the loop is
  // under the explicit wait counts below. Positions past the end are clamped
  // (global form) or not read (BUF).
  auto id_ring = [&](int ring) -> int* { return ring == 0 ? &id0[wave][0] : &id1[wave][0]; };
  auto stage_ptr = [&](int ring) -> char* { return ring == 0 ? st0 : st1; };
  auto load_ids = [&](int blk, int ring) {
    const int kb = min(blk, nblk - 1) * kBK;
    const int pos = min(kb + lane, kv_end - 1);
    if constexpr (BUF)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(irs, PKV_LDS(id_ring(ring)), 4,
                                               blk < nblk ? 4u * (uint32_t)pos : kNoBlock, 0, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(PKV_GLB(row + pos), PKV_LDS(id_ring(ring)), 4, 0, 0);
  };
  // the logical chunk the tile's swizzle puts at this lane's physical chunk
  auto chunk_of = [&](int rr) {
    if constexpr (kFp8)
      return pch ^ ((rr / Sg::RPL) & (Sg::CPR - 1));
    else
      return pch ^ (rr & (Sg::CPR - 1));
  };
  // BUF: 32-bit offsets from the descriptor bases (fewer live registers
  // while the transfers are spread over the S phase)
  using Off = std::conditional_t<BUF, uint32_t, int64_t>;
  // live: the block exists (BUF; the global form always reads a clamped block)
  auto offsets = [&](int ring, Off (&off)[Sg::NI], bool live) {
    const int* ids = id_ring(ring);
    if constexpr (BUF) {
      // no clamp: the descriptor's range check keeps any slot id in bounds
      // (an id past the pool reads zeros); a shift where the row stride is a
      // power of two (a 32-bit multiply is a quarter-rate instruction)
      uint32_t base[Sg::NI];
      if (a.row_shift >= 0) {
#pragma unroll
        for (int i = 0; i < Sg::NI; ++i)
          base[i] = (uint32_t)ids[16 * wave + Sg::RPI * i + prow] << a.row_shift;
      } else {
#pragma unroll
        for (int i = 0; i < Sg::NI; ++i)
          base[i] = (uint32_t)ids[16 * wave + Sg::RPI * i + prow] * (uint32_t)row_stride;
      }
#pragma unroll
      for (int i = 0; i < Sg::NI; ++i)
        off[i] = live ? base[i] + (uint32_t)(16 * chunk_of(16 * wave + Sg::RPI * i + prow))
                      : kNoBlock;
    } else {
#pragma unroll
      for (int i = 0; i < Sg::NI; ++i) {
        const int rr = 16 * wave + Sg::RPI * i + prow;
        // unsigned 32 x 32 -> 64-bit product (one multiply-add): the clamped
        // slot is non-negative and the row stride is below 2^24 (at most
        // 65535 KV heads of 256 bytes)
        off[i] = (Off)((uint64_t)(uint32_t)clamp_index(ids[rr], n_slots) * (uint32_t)row_stride +
                       (uint32_t)(16 * chunk_of(rr)));
      }
    }
  };
  // E4M3 pools: this lane's V chunks of the next block, in registers until
  // they are widened into the bf16 V tile
  u32x4 vreg[kFp8 ? Sg::NI : 1];
  // bf16 pools: per transfer, 16 x (K chunk XOR V chunk) of this lane's row
  // (the physical chunk pch holds logical chunk pch ^ (rr % CPR) in K and
  // pch ^ vxor(rr) in V)
  uint32_t vmove[Sg::NI];
#pragma unroll
  for (int i = 0; i < Sg::NI; ++i) {
    const int rr = 16 * wave + Sg::RPI * i + prow;
    vmove[i] = kFp8 ? 0u : 16u * (uint32_t)((rr & (Sg::CPR - 1)) ^ vxor<D>(rr));
  }
  // transfer t of a block: K rows (t even) or V rows (t odd) 16*wave + RPI*(t/2) ..
  constexpr int kNT = 2 * Sg::NI;
  auto issue_one = [&](int stage, const Off (&off)[Sg::NI], int t) {
    char* st = stage_ptr(stage);
    const int i = t >> 1;
    const int rbase = 16 * wave + Sg::RPI * i;
    if ((t & 1) == 0)
      dma16(krs, kbase, off[i], st + rbase * Sg::ROW);
    else if constexpr (!kFp8)
      // bf16 V rows land under the V swizzle: the offset's chunk bits (below
      // the 128-byte-aligned row base) move from this lane's K chunk to its V chunk
      dma16(vrs, vbase, off[i] ^ (Off)vmove[i], st + Sg::KTILE + rbase * Gm::ROW);
    else if constexpr (BUF)
      vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off[i], 0, 0));
    else
      vreg[i] = *(const u32x4*)(vbase + off[i]);
  };
  auto issue = [&](int stage, const Off (&off)[Sg::NI]) {
#pragma unroll
    for (int t = 0; t < kNT; ++t) issue_one(stage, off, t);
  };
  // E4M3 pools: widen this lane's V chunks (row rr, logical code chunk c ->
  // bf16 chunks 2c, 2c + 1) into the stage's bf16 V tile
  auto write_v = [&](int stage) {
    if constexpr (kFp8) {
      char* vt = stage_ptr(stage) + Sg::KTILE;
#pragma unroll
      for (int i = 0; i < Sg::NI; ++i) {
        const int rr = 16 * wave + Sg::RPI * i + prow;
        const int c = chunk_of(rr);
        u32x4 lo, hi;
        fp8x16_to_bf16x16(vreg[i], lo, hi);
        *(u32x4*)(vt + swzv<D>(rr, 2 * c)) = lo;
        *(u32x4*)(vt + swzv<D>(rr, 2 * c + 1)) = hi;
      }
    }
  };

  // Q^T fragments (B operand) for this wave's two 16-row tiles.
  const int col = lane & 15;
  const int quad = lane >> 4;
  u32x4 qf[2][Gm::KSTEPS];
  int limit[2];
  int tok[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int rr = wave * 32 + n * 16 + col;  // row within the tile
    const int t = t0 + rr / G;
    tok[n] = t;
    const int tc = min(t, n_new - 1);
    const int64_t qrow = ((int64_t)q0 + tc) * a.n_q_heads + (int64_t)kvh * G + rr % G;
    const char* qp = (const char*)a.q + qrow * Gm::ROW;
    // k-step ks: head_dim 32 ks + 8 quad .. +7 (bf16 K), or the order of the
    // E4M3 K reads, 64 (ks/2) + 16 quad + 8 (ks%2) .. +7
#pragma unroll
    for (int ks = 0; ks < Gm::KSTEPS; ++ks)
      qf[n][ks] = *(const u32x4*)(qp + (kFp8 ? 128 * (ks / 2) + 32 * quad + 16 * (ks % 2)
                                             : 64 * ks + 16 * quad));
    limit[n] = a.causal ? min(P + tc, L - 1) : L - 1;
  }
  // the wave's last visible key: that of its last row (wave-uniform)
  const int wlim =
      a.causal ? min(P + min(t0 + (wave * 32 + 31) / G, n_new - 1), L - 1) : L - 1;

  // a negative scale is applied as -scale on -Q (bf16 negation is exact), a
  // zero scale as scale 1 on Q = 0 (every score is exactly 0 either way)
  // E4M3 pools: the K scale joins the softmax scale, the V scale the output
  float scale2 = a.scale * kLog2e * (kFp8 ? a.kv_scale[0] : 1.f);
  const float vscale = kFp8 ? a.kv_scale[1] : 1.f;
  if (!(scale2 > 0.f)) {
    const uint32_t flip = scale2 < 0.f ? 0x80008000u : 0u;
    const uint32_t keep = scale2 < 0.f ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int ks = 0; ks < Gm::KSTEPS; ++ks) qf[n][ks] = (qf[n][ks] & keep) ^ flip;
    scale2 = scale2 < 0.f ? -scale2 : 1.f;
  }

  f32x4 o[Gm::DT][2];
  f32x4 lacc[2];
  float m[2] = {-INFINITY, -INFINITY};
  float mseen[2] = {-INFINITY, -INFINITY};
  // One pass over the tile's keys. With init_pass, each row's stabiliser is
  // fixed from its first 32 keys; with track, the exact row maxima are
  // gathered in mseen (that pass's O and row sums are not used).
  auto run_pass = [&](auto track, bool init_pass) {
#pragma unroll
    for (int dt = 0; dt < Gm::DT; ++dt) {
      o[dt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      o[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    lacc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    lacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Transfer order per wave, kept identical in every iteration so that the
    // explicit wait counts are exact: before block i is computed the queue
    // holds, oldest first, S(i+1) D(i) S(i+2), where D(k) = 2*NI tile transfers
    // of block k into stage k % 2 and S(k) = one slot-id transfer for block k
    // into id ring k % 2 (past the last block: clamped, or empty under BUF).
    // E4M3 pools: D(k) is NI K transfers plus NI V loads into registers, and
    // block i waits for everything in flight (all of it belongs to block i)
    // before its V is widened into the tile and S(i+2) is queued.
    Off off[Sg::NI];
    load_ids(0, 0);
    load_ids(1, 1);
    __builtin_amdgcn_s_waitcnt(PKV_VMCNT(0));
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    offsets(0, off, true);
    issue(0, off);

    // One block: wait for its transfers, queue the next ones, attend.
    auto block = [&](int i, int u, auto masked) {
      if constexpr (kFp8) {
        __builtin_amdgcn_s_waitcnt(PKV_VMCNT(0));  // S(i+1) and D(i) landed (this wave)
        write_v(u);  // stage u's V tile: block i-2, its last reader, is done
        load_ids(i + 2, u);
        __builtin_amdgcn_s_waitcnt(PKV_LGKMCNT0);  // the V writes, before the barrier
      } else {
        load_ids(i + 2, u);  // ring u held the ids of block i, already consumed
        __builtin_amdgcn_s_waitcnt(PKV_VMCNT(1));  // S(i+1) and D(i) landed (this wave)
      }
      __builtin_amdgcn_s_barrier();              // ... for every wave; block i-1 is done
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      // block i+1 goes into the stage block i-1 used
      offsets(u ^ 1, off, i + 1 < nblk);
      const char* st = stage_ptr(u);
      attend_block<D, G, decltype(masked)::value, KV, decltype(track)::value, kNT>(
          st, st + Sg::KTILE, qf, o, lacc, m, mseen, init_pass && i == 0, i * kBK, limit, wlim,
          scale2, lane, [&](int t) { issue_one(u ^ 1, off, t); });
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    };
    // Blocks that every row sees whole and that end inside the sequence need
    // no mask; they run in a loop of their own (an even count, so the ring
    // stages stay compile-time), the rest (the diagonal and the end) after it.
    const int nfull = min(nblk, min(kv_full, L) / kBK) & ~(kStages - 1);
    for (int i0 = 0; i0 < nfull; i0 += kStages) {
      block(i0, 0, std::false_type{});
      block(i0 + 1, 1, std::false_type{});
    }
    for (int i0 = nfull; i0 < nblk; i0 += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) {
        if (i0 + u >= nblk) break;
        block(i0 + u, u, std::true_type{});
      }
    }
    // drain the transfers past the end (before another pass or the exit)
    __builtin_amdgcn_s_waitcnt(PKV_VMCNT(0));
  };
  run_pass(std::false_type{}, true);
  // A score more than kTau above its row's stabiliser gives a weight above
  // 2^kTau, so that row's sum (of the same rounded weights) exceeds 2^kTau or
  // is not finite. Such a tile is done again: one pass gathers the exact row
  // maxima, the last one uses them as the stabiliser and cannot overflow.
  // Tested on the bits, so that NaN (an inf weight minus an inf) is caught
  // whatever the file's floating-point flags let the compiler assume.
  bool bad = false;
#pragma unroll
  for (int n = 0; n < 2; ++n)
    bad |= (__float_as_uint(lacc[n][0]) & 0x7fffffffu) > __float_as_uint(kSumLimit);
  // workgroup-wide decision; the barrier also frees the stages for the next pass
  if (lane == 0) redo[wave] = __builtin_amdgcn_ballot_w64(bad) != 0;
  __syncthreads();
  if (redo[0] | redo[1] | redo[2] | redo[3]) {
    run_pass(std::true_type{}, false);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      float x = fmaxf(mseen[n], __shfl_xor(mseen[n], 16));
      m[n] = fmaxf(x, __shfl_xor(x, 32));
    }
    __syncthreads();  // the stages are free for the last pass
    run_pass(std::false_type{}, false);
  }

#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int rr = wave * 32 + n * 16 + col;
    if (tok[n] >= n_new || tok[n] >= a.max_q_len) continue;  // rows past max_q_len stay unwritten
    const int64_t orow = ((int64_t)q0 + tok[n]) * a.n_q_heads + (int64_t)kvh * G + rr % G;
    const int64_t t_abs = (int64_t)q0 + tok[n];
    if (t_abs < 0 || t_abs >= a.total_q) continue;
    const float inv = vscale / lacc[n][0];  // the row sum over all keys, in every lane of the column
    uint16_t* out = (uint16_t*)a.out + orow * D;
#pragma unroll
    for (int dt = 0; dt < Gm::DT; ++dt) {
      const int d = 16 * dt + 4 * quad;
      const bf16x2_t w0 = {(__bf16)(o[dt][n][0] * inv), (__bf16)(o[dt][n][1] * inv)};
      const bf16x2_t w1 = {(__bf16)(o[dt][n][2] * inv), (__bf16)(o[dt][n][3] * inv)};
      u32x2 w;
      w[0] = __builtin_bit_cast(uint32_t, w0);
      w[1] = __builtin_bit_cast(uint32_t, w1);
      *(u32x2*)(out + d) = w;
    }
  }
}

template <int D, typename KV>
hipError_t prefill_for_dim(PrefillArgs a, hipStream_t stream) {
  const int g = a.n_q_heads / a.n_kv_heads;
  const int bq = kRows / g;
  const int64_t tiles_max = (a.max_q_len + bq - 1) / bq;
  dim3 grid((unsigned)tiles_max, a.n_kv_heads, a.batch);
  a.sorted = 0;
  if (a.batch <= kSortedMaxBatch) {
    // every (request, tile) item once: at most ceil(total_q / BQ) + batch items
    const int64_t items = std::min<int64_t>(tiles_max * a.batch,
                                            ((int64_t)a.total_q + bq - 1) / bq + a.batch);
    const int64_t blocks = items * a.n_kv_heads;
    if (blocks <= 0x7fffffff / kThreads) {
      a.sorted = 1;
      grid = dim3((unsigned)blocks, 1, 1);
    }
  }
  // buffer descriptors span 32-bit offsets: the layer's pool and the slot-table
  // row (int32 entries) must stay below the no-block offset 0xFFFFFFF0
  const int64_t pool_bytes = a.n_slots * (int64_t)a.n_kv_heads * D * (int64_t)sizeof(KV);
  const bool buf = pool_bytes <= 0xF0000000ll && a.stride <= 0x3C000000ll;
  // a (slot, KV head) row's byte stride as a shift when it is a power of two
  const int64_t rs = (int64_t)a.n_kv_heads * D * (int64_t)sizeof(KV);
  a.row_shift = (rs & (rs - 1)) == 0 ? __builtin_ctzll((unsigned long long)rs) : -1;
  auto launch = [&](auto gc) {
    constexpr int GG = decltype(gc)::value;
    if (buf)
      prefill_kernel<D, GG, KV, true><<<grid, kThreads, 0, stream>>>(a);
    else
      prefill_kernel<D, GG, KV, false><<<grid, kThreads, 0, stream>>>(a);
  };
  switch (g) {
    case 1: launch(std::integral_constant<int, 1>{}); break;
    case 2: launch(std::integral_constant<int, 2>{}); break;
    case 4: launch(std::integral_constant<int, 4>{}); break;
    case 8: launch(std::integral_constant<int, 8>{}); break;
    case 16: launch(std::integral_constant<int, 16>{}); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.max_q_len == 0) return hipSuccess;
  if (a.dtype == PKV_FP8_E4M3)
    return a.head_dim == 128 ? prefill_for_dim<128, fp8_t>(a, stream)
                             : prefill_for_dim<64, fp8_t>(a, stream);
  return a.head_dim == 128 ? prefill_for_dim<128, bf16_t>(a, stream)
                           : prefill_for_dim<64, bf16_t>(a, stream);
}

}  // namespace pkv
