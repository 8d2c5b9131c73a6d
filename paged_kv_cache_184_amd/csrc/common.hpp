// Device helpers shared by the pkv kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;
constexpr int kSplitAlign = 16;  // PKV_SPLIT_ALIGN

// Storage tags: bf16 is carried as raw 16-bit patterns.
struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct elem_size;
template <>
struct elem_size<float> {
  static constexpr int value = 4;
};
template <>
struct elem_size<bf16_t> {
  static constexpr int value = 2;
};

// One-byte E4M3 code of an FP8 KV pool (OCP 8-bit floating point, E4M3: bias
// 7, subnormals, no infinities, largest finite 448).
struct fp8_t {
  uint8_t bits;
};
template <>
struct elem_size<fp8_t> {
  static constexpr int value = 1;
};

// Element type of q and of the output for a KV storage type: the storage type
// itself, except bf16 for FP8 pools.
template <typename T>
struct io_type {
  using type = T;
};
template <>
struct io_type<fp8_t> {
  using type = bf16_t;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Two E4M3 codes (bytes 2 hi .. 2 hi + 1 of w) widened exactly to a packed
// bf16 pair (every E4M3 value, subnormals included, is a bf16 value).
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

// 16 codes -> 16 bf16 values: codes 0..7 in `a`, codes 8..15 in `b`.
__device__ __forceinline__ void fp8x16_to_bf16x16(u32x4 c, u32x4& a, u32x4& b) {
  a = u32x4{fp8x2_to_bf16x2<false>(c[0]), fp8x2_to_bf16x2<true>(c[0]),
            fp8x2_to_bf16x2<false>(c[1]), fp8x2_to_bf16x2<true>(c[1])};
  b = u32x4{fp8x2_to_bf16x2<false>(c[2]), fp8x2_to_bf16x2<true>(c[2]),
            fp8x2_to_bf16x2<false>(c[3]), fp8x2_to_bf16x2<true>(c[3])};
}

// E4M3 code of the fp32 quotient x / s (correctly rounded division), rounded
// to nearest even by the conversion; magnitudes beyond 448 saturate (the
// conversion alone would give NaN there); NaN stays a NaN code.
__device__ __forceinline__ float fp8_sat_quotient(float x, float s) {
  const float y = x / s;
  return fabsf(y) > 448.f ? copysignf(448.f, y) : y;
}
__device__ __forceinline__ uint32_t quant_fp8x4(float a, float b, float c, float d, float s) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_sat_quotient(a, s), fp8_sat_quotient(b, s), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_sat_quotient(c, s), fp8_sat_quotient(d, s), w, true);
  return (uint32_t)w;
}

// 16 bf16 values (two 16-byte chunks) -> 16 E4M3 codes under scale s.
__device__ __forceinline__ u32x4 quant_bf16x16(u32x4 a, u32x4 b, float s) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    r[i] = quant_fp8x4(bf16lo_to_f32(a[2 * i]), bf16hi_to_f32(a[2 * i]),
                       bf16lo_to_f32(a[2 * i + 1]), bf16hi_to_f32(a[2 * i + 1]), s);
    r[2 + i] = quant_fp8x4(bf16lo_to_f32(b[2 * i]), bf16hi_to_f32(b[2 * i]),
                           bf16lo_to_f32(b[2 * i + 1]), bf16hi_to_f32(b[2 * i + 1]), s);
  }
  return r;
}

// dot of two packed bf16 pairs accumulated into fp32 (v_dot2_f32_bf16).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP lane moves within rows of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
}
constexpr int kQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // row_half_mirror: lane i <-> 7-i within 8
constexpr int kRowMirror = 0x140;   // row_mirror: lane i <-> 15-i within 16
constexpr int kRowRor8 = 0x128;     // row_ror:8: lane i <- lane (i+8) mod 16

// x plus the value of lane l ^ 16 (add_xor16) or lane l ^ 32 (add_xor32), by
// the gfx950 row-swap instructions: a VALU exchange instead of an LDS permute.
// With both operands equal to x, v_permlane16_swap leaves (x of the even row,
// x of the odd row) of each row pair in its two results, and v_permlane32_swap
// (x of lanes 0-31, x of lanes 32-63); their sum is own + partner in either
// order, which is the same bits (fp addition is commutative).
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over each aligned group of 8 lanes; every lane of the group gets the
// same bits (each step adds a commutative pair).
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  x += dpp<kHalfMirror>(x);
  return x;
}

// Sum over the wave with the same bits in every lane and the same bits as the
// butterfly x += x[l ^ off] for off = 1, 2, ..., 32: after the first two steps
// a quad holds one value, so the half-row mirror pairs it with the quad at
// l ^ 4, and the row mirror then pairs each 8-lane half with the one at l ^ 8.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  x += dpp<kHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  return add_xor32(add_xor16(x));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kQuadSwap1>(x));
  x = fmaxf(x, dpp<kQuadSwap2>(x));
  x = fmaxf(x, dpp<kHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__host__ __device__ constexpr __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Merge placement: the q head that merge workgroup x (of n_q_heads) serves.
// Workgroups reach the 8 XCDs round-robin by linear id, and with n_kv_heads a
// multiple of 8 the partial kernel (KV head fastest in its grid) writes every
// split of KV head k from XCD k mod 8. Workgroup x takes a head of KV head
// (x mod 8) + 8 * (j / g), j = x / 8, so its partials are read on the XCD that
// wrote them; the map is a bijection of [0, n_q_heads) for every such
// n_kv_heads and g = n_q_heads / n_kv_heads >= 1. Any other head count
// (n_kv_heads = 0 included: the merge-only entry point does not know it) keeps
// the identity.
__host__ __device__ __forceinline__ int merge_head_of(int x, int n_q_heads, int n_kv_heads) {
  if (n_kv_heads > 0 && (n_kv_heads & 7) == 0 && n_q_heads >= n_kv_heads &&
      n_q_heads % n_kv_heads == 0) {
    const int g = n_q_heads / n_kv_heads;
    const int j = x >> 3;
    return ((x & 7) + 8 * (j / g)) * g + j % g;
  }
  return x;
}

// Split rule of pkv_split_cfg: returns S (0 when L <= 0) and the chunk length.
__host__ __device__ __forceinline__ int split_count(int L, int max_splits, int fixed_splits,
                                                    int split_tokens, int* chunk_out) {
  if (L <= 0) {
    *chunk_out = 0;
    return 0;
  }
  int req = fixed_splits > 0 ? fixed_splits : ceil_div(L, split_tokens);
  req = req < 1 ? 1 : (req > max_splits ? max_splits : req);
  int chunk = ceil_div(ceil_div(L, req), kSplitAlign) * kSplitAlign;
  *chunk_out = chunk;
  return ceil_div(L, chunk);
}

// K/V row bytes that a decode launch reads once, with the non-temporal cache
// policy, wherever one load instruction covers whole 128-byte lines: both
// rows in the VALU decode kernel, the V rows in the MFMA one. Measured:
// 5-11% shorter launches at 16K-32K contexts and on ragged batches, but 16%
// longer with 32 requests over one 4096-token prefix under plain attention,
// the case cascade decode serves. The MFMA kernel's K fragments read each line
// with two half-line instructions and keep the default policy (streaming them
// made large batches 6-8% slower).
__device__ __forceinline__ u32x4 load_stream(const char* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// A word that every lane of the workgroup reads at the same address and that
// no kernel writes while it runs (request lengths, row indices): loaded
// through the scalar data cache, so several such loads are in flight at once.
__device__ __forceinline__ int load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

__device__ __forceinline__ int clamp_index(int x, int n) {
  // maps any int to [0, n): negatives to 0, too-large to n - 1
  return x < 0 ? 0 : (x >= n ? n - 1 : x);
}

}  // namespace pkv
