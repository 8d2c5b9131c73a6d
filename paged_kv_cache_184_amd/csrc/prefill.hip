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
//   * the 256 threads gather the block's K rows (16-byte loads through the
//     slot table) into LDS row-major, and its V rows into LDS transposed
//     ([d][key], two keys packed per dword), both with padded row strides;
//   * each wave computes S^T = K Q^T for its 32 rows with
//     v_mfma_f32_16x16x32_bf16 (K from LDS as the A operand, Q^T held in
//     registers as the B operand for the whole tile);
//   * softmax in base 2 with a per-row stabiliser that is raised only when a
//     score exceeds it by more than kTau; P is rounded to bf16 and the row
//     sums accumulate those rounded values;
//   * O^T += V^T P^T with the same MFMA: P^T comes straight out of the S^T
//     accumulator layout (lane l holds keys 4(l/16)+r of two 16-key tiles for
//     query column l%16), V^T is read from the transposed LDS tile with the
//     same key order, so no register shuffles are needed.
// Only blocks that straddle the causal diagonal or the sequence end are
// masked. Tiles are issued longest-first (highest token offset first).
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRows = 128;   // query rows per workgroup
constexpr int kBK = 64;      // keys per block
constexpr int kThreads = 256;
constexpr float kTau = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct PGeo {
  static constexpr int ROW = D * 2;          // bytes of a (slot, KV head) row
  static constexpr int KS = ROW + 16;        // LDS row stride of the K tile
  static constexpr int VS = kBK * 2 + 8;     // LDS row stride of the V^T tile
  static constexpr int K_BYTES = kBK * KS;
  static constexpr int V_BYTES = D * VS;
  static constexpr int KSTEPS = D / 32;      // MFMA k-steps over head_dim
  static constexpr int DT = D / 16;          // 16-wide output tiles over head_dim
  static constexpr int CPR = ROW / 16;       // 16-byte chunks per row
};

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_round(float x) { return f32_to_bf16_rne(x); }

template <int D, int G, bool MASK>
__device__ __forceinline__ void attend_block(
    const char* __restrict__ lds_k, const char* __restrict__ lds_v, const u32x4 (&qf)[2][PGeo<D>::KSTEPS],
    f32x4 (&o)[PGeo<D>::DT][2], float (&m)[2], float (&l)[2], int k0, const int (&limit)[2],
    float scale2, int lane) {
  using Gm = PGeo<D>;
  const int col = lane & 15;
  const int quad = lane >> 4;
  // S^T for 4 key tiles x 2 query tiles
  f32x4 s[4][2];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    s[kt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    s[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < Gm::KSTEPS; ++ks) {
      const u32x4 a = *(const u32x4*)(lds_k + (16 * kt + col) * Gm::KS + 2 * (32 * ks + 8 * quad));
      s[kt][0] = mfma16(a, qf[0][ks], s[kt][0]);
      s[kt][1] = mfma16(a, qf[1][ks], s[kt][1]);
    }
  }
  // scale, mask, stabiliser check
  bool need = false;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = s[kt][n][r] * scale2;
        if (MASK) {
          const int key = k0 + 16 * kt + 4 * quad + r;
          x = key <= limit[n] ? x : -INFINITY;
        }
        s[kt][n][r] = x;
        need |= x > m[n] + kTau;
      }
    }
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kt][n][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[n], mx);
      // rows that have seen no visible key yet keep m = -inf (their p are 0)
      const float corr = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[n] - mnew);
      l[n] *= corr;
#pragma unroll
      for (int dt = 0; dt < Gm::DT; ++dt) o[dt][n] *= corr;
      m[n] = mnew;
    }
  }
  // P^T (bf16) in the B-operand layout: slots 0..3 = key tile 2j, 4..7 = tile 2j+1
  u32x4 pf[2][2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const float mm = m[n] == -INFINITY ? 0.f : m[n];
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const uint32_t lo = bf16_round(__builtin_amdgcn_exp2f(s[2 * j + h][n][r] - mm));
          const uint32_t hi = bf16_round(__builtin_amdgcn_exp2f(s[2 * j + h][n][r + 1] - mm));
          lsum += __uint_as_float(lo << 16) + __uint_as_float(hi << 16);
          w[2 * h + r / 2] = lo | (hi << 16);
        }
      }
      pf[n][j] = u32x4{w[0], w[1], w[2], w[3]};
    }
    l[n] += lsum;
  }
  // O^T += V^T P^T
#pragma unroll
  for (int dt = 0; dt < Gm::DT; ++dt) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const char* vrow = lds_v + (16 * dt + col) * Gm::VS + 2 * (32 * j + 4 * quad);
      const u32x2 lo = *(const u32x2*)(vrow);
      const u32x2 hi = *(const u32x2*)(vrow + 32);  // keys +16
      const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
      o[dt][0] = mfma16(a, pf[0][j], o[dt][0]);
      o[dt][1] = mfma16(a, pf[1][j], o[dt][1]);
    }
  }
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
  using Gm = PGeo<D>;
  constexpr int BQ = kRows / G;  // tokens per tile
  __shared__ __attribute__((aligned(16))) char lds[Gm::K_BYTES + Gm::V_BYTES];
  char* lds_k = lds;
  char* lds_v = lds + Gm::K_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int tile = gridDim.x - 1 - blockIdx.x;  // longest work first
  const int t0 = tile * BQ;

  const int q0 = a.qo_indptr[b];
  int n_new = a.qo_indptr[b + 1] - q0;
  if (t0 >= n_new) return;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.stride ? (int)a.stride : L);
  if (n_new > L) n_new = L;
  if (t0 >= n_new) return;
  const int P = L - n_new;
  const int t_last = min(t0 + BQ, n_new) - 1;
  const int kv_end = a.causal ? P + t_last + 1 : L;  // keys the tile can see
  const int kv_full = a.causal ? P + t0 + 1 : L;     // keys every row of the tile sees

  const int r = clamp_index(a.req_pool_indices[b], a.n_rows);
  const int32_t* row = a.req_to_token + (int64_t)r * a.stride;
  const int n_slots = (int)(a.n_slots > 0x7fffffff ? 0x7fffffff : a.n_slots);
  const int64_t row_stride = (int64_t)a.n_kv_heads * Gm::ROW;
  const char* kbase = (const char*)a.k + (int64_t)kvh * Gm::ROW;
  const char* vbase = (const char*)a.v + (int64_t)kvh * Gm::ROW;

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
    const char* qp = (const char*)a.q + qrow * Gm::ROW + 16 * quad;
#pragma unroll
    for (int ks = 0; ks < Gm::KSTEPS; ++ks) qf[n][ks] = *(const u32x4*)(qp + 64 * ks);
    limit[n] = a.causal ? min(P + tc, L - 1) : L - 1;
  }

  f32x4 o[Gm::DT][2];
#pragma unroll
  for (int dt = 0; dt < Gm::DT; ++dt) {
    o[dt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    o[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};
  const float scale2 = a.scale * kLog2e;

  for (int k0 = 0; k0 < kv_end; k0 += kBK) {
    __syncthreads();  // previous block's LDS reads are done
    // K: 64 keys x CPR chunks, row-major, coalesced 16-byte loads.
#pragma unroll
    for (int i = 0; i < (kBK * Gm::CPR) / kThreads; ++i) {
      const int c = tid + kThreads * i;
      const int j = c / Gm::CPR;
      const int cc = c % Gm::CPR;
      const int pos = min(k0 + j, kv_end - 1);
      const int slot = clamp_index(row[pos], n_slots);
      const u32x4 x = *(const u32x4*)(kbase + (int64_t)slot * row_stride + 16 * cc);
      *(u32x4*)(lds_k + j * Gm::KS + 16 * cc) = x;
    }
    // V: each thread takes two adjacent keys of one chunk and writes them
    // transposed, two keys per dword.
#pragma unroll
    for (int i = 0; i < (kBK / 2 * Gm::CPR) / kThreads; ++i) {
      const int c = tid + kThreads * i;
      const int j2 = c % (kBK / 2);
      const int cc = c / (kBK / 2);
      const int pa = min(k0 + 2 * j2, kv_end - 1);
      const int pb = min(k0 + 2 * j2 + 1, kv_end - 1);
      const int sa = clamp_index(row[pa], n_slots);
      const int sb = clamp_index(row[pb], n_slots);
      const u32x4 va = *(const u32x4*)(vbase + (int64_t)sa * row_stride + 16 * cc);
      const u32x4 vb = *(const u32x4*)(vbase + (int64_t)sb * row_stride + 16 * cc);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // dims 8cc + 2w (low halves) and 8cc + 2w + 1 (high halves)
        const uint32_t lo = (va[w] & 0xffffu) | (vb[w] << 16);
        const uint32_t hi = (va[w] >> 16) | (vb[w] & 0xffff0000u);
        *(uint32_t*)(lds_v + (8 * cc + 2 * w) * Gm::VS + 4 * j2) = lo;
        *(uint32_t*)(lds_v + (8 * cc + 2 * w + 1) * Gm::VS + 4 * j2) = hi;
      }
    }
    __syncthreads();
    if (k0 + kBK <= kv_full && k0 + kBK <= L)
      attend_block<D, G, false>(lds_k, lds_v, qf, o, m, lsum, k0, limit, scale2, lane);
    else
      attend_block<D, G, true>(lds_k, lds_v, qf, o, m, lsum, k0, limit, scale2, lane);
  }

  // Row sums: the four lanes of a query column hold disjoint keys.
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    lsum[n] += __shfl_xor(lsum[n], 16);
    lsum[n] += __shfl_xor(lsum[n], 32);
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int rr = wave * 32 + n * 16 + col;
    if (tok[n] >= n_new) continue;
    const int64_t orow = ((int64_t)q0 + tok[n]) * a.n_q_heads + (int64_t)kvh * G + rr % G;
    const int64_t t_abs = (int64_t)q0 + tok[n];
    if (t_abs < 0 || t_abs >= a.total_q) continue;
    const float inv = 1.0f / lsum[n];
    uint16_t* out = (uint16_t*)a.out + orow * D;
#pragma unroll
    for (int dt = 0; dt < Gm::DT; ++dt) {
      const int d = 16 * dt + 4 * quad;
      u32x2 w;
      w[0] = pack_bf16x2(o[dt][n][0] * inv, o[dt][n][1] * inv);
      w[1] = pack_bf16x2(o[dt][n][2] * inv, o[dt][n][3] * inv);
      *(u32x2*)(out + d) = w;
    }
  }
}

template <int D>
hipError_t prefill_for_dim(const PrefillArgs& a, hipStream_t stream) {
  const int g = a.n_q_heads / a.n_kv_heads;
  const int bq = kRows / g;
  dim3 grid((a.max_q_len + bq - 1) / bq, a.n_kv_heads, a.batch);
  switch (g) {
    case 1: prefill_kernel<D, 1><<<grid, kThreads, 0, stream>>>(a); break;
    case 2: prefill_kernel<D, 2><<<grid, kThreads, 0, stream>>>(a); break;
    case 4: prefill_kernel<D, 4><<<grid, kThreads, 0, stream>>>(a); break;
    case 8: prefill_kernel<D, 8><<<grid, kThreads, 0, stream>>>(a); break;
    case 16: prefill_kernel<D, 16><<<grid, kThreads, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.max_q_len == 0) return hipSuccess;
  return a.head_dim == 128 ? prefill_for_dim<128>(a, stream) : prefill_for_dim<64>(a, stream);
}

}  // namespace pkv
