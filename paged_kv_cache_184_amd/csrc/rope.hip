// Rotary position embedding of the new tokens fused with the store of their
// K/V rows (next to a2).
//
// AstrAI commit 398e8a3e page, bullet on extending the rotary embedding to
// packed 3D inputs: q [T, Hq, D] and k [T, Hkv, D] rows are rotated per token
// position. AstrAI commit e58a728b page, bullet on the rotary table being cos /
// sin values: the caller passes freqs_cis[max_pos, D/2, 2] = (cos, sin) of the
// angle of pair i at position p. Pair i is (2i, 2i+1) when interleaved, else
// (i, i + D/2); a' = a cos - b sin, b' = b cos + a sin, in fp32, rounded to the
// storage dtype. The rotated k row and the unrotated v row go to
// pool[layer, loc[t]] (skipped when loc[t] is outside [0, n_slots)); the rotated
// q row goes to q_out (which may be q itself).
//
// One thread per 16-byte chunk of a row; a token owns Hq + 2 Hkv rows (q, k, v).
// Interleaved: a chunk holds whole pairs. Half-split: a thread takes chunk c of
// the first half and chunk c of the second half together (the threads of the
// second half's chunks have no work on q / k rows). Every access is a 16-byte
// load or store; the table row of a position is a few hundred bytes and stays
// in cache across the token's heads.
#include "common.hpp"
#include "internal.hpp"

namespace pkv {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct RopeIO;

template <>
struct RopeIO<bf16_t> {
  static constexpr int EPC = 8;  // elements per 16-byte chunk
  static __device__ __forceinline__ void load(const char* p, float (&x)[EPC]) {
    const u32x4 w = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16lo_to_f32(w[i]);
      x[2 * i + 1] = bf16hi_to_f32(w[i]);
    }
  }
  static __device__ __forceinline__ void store(char* p, const float (&x)[EPC]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2_t h = {(__bf16)x[2 * i], (__bf16)x[2 * i + 1]};
      w[i] = __builtin_bit_cast(uint32_t, h);
    }
    *(u32x4*)p = w;
  }
};

template <>
struct RopeIO<float> {
  static constexpr int EPC = 4;
  static __device__ __forceinline__ void load(const char* p, float (&x)[EPC]) {
    const u32x4 w = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
  static __device__ __forceinline__ void store(char* p, const float (&x)[EPC]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(x[i]);
    *(u32x4*)p = w;
  }
};

__device__ __forceinline__ void rotate(float& a, float& b, float c, float s) {
  const float a2 = a * c - b * s;
  const float b2 = b * c + a * s;
  a = a2;
  b = b2;
}

// The same rotation with each product and each sum rounded once (no fused
// multiply-add), in a fixed order, so that a code decided on the result is
// reproducible: a' = fl(fl(a c) - fl(b s)), b' = fl(fl(b c) + fl(a s)).
__device__ __forceinline__ void rotate_rn(float& a, float& b, float c, float s) {
#pragma clang fp contract(off)
  const float ac = a * c;
  const float bs = b * s;
  const float bc = b * c;
  const float as = a * s;
  a = ac - bs;
  b = bc + as;
}

// Eight values -> eight E4M3 codes under scale s (two dwords).
__device__ __forceinline__ u32x2 quant8(const float (&x)[8], float s) {
  return u32x2{quant_fp8x4(x[0], x[1], x[2], x[3], s), quant_fp8x4(x[4], x[5], x[6], x[7], s)};
}

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kv_store_kernel(RopeArgs r) {
  using IO = RopeIO<T>;
  constexpr int EPC = IO::EPC;
  constexpr int ES = elem_size<T>::value;
  constexpr int ROW = D * ES;        // bytes of one head row
  constexpr int CPR = ROW / 16;      // chunks per row
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int rows_per_token = r.n_q_heads + 2 * r.n_kv_heads;
  const int64_t total = r.n_tokens * rows_per_token * CPR;
  if (idx >= total) return;
  const int c = (int)(idx % CPR);
  const int64_t row = idx / CPR;
  const int64_t t = row / rows_per_token;
  const int h = (int)(row - t * rows_per_token);
  int p = r.positions[t];
  p = p < 0 ? 0 : (p >= r.max_pos ? r.max_pos - 1 : p);
  const float2* tab = (const float2*)r.freqs_cis + (int64_t)p * (D / 2);

  // role of this row: q head, k head or v head
  const bool is_q = h < r.n_q_heads;
  const bool is_k = !is_q && h < r.n_q_heads + r.n_kv_heads;
  const int kvh = is_q ? 0 : (is_k ? h - r.n_q_heads : h - r.n_q_heads - r.n_kv_heads);
  int slot = -1;
  if (!is_q) {
    const int s = r.loc[t];
    slot = (s >= 0 && (int64_t)s < r.n_slots) ? s : -1;
  }
  const char* src;
  char* dst;
  if (is_q) {
    if (!r.q) return;
    const int64_t off = (t * r.n_q_heads + h) * (int64_t)ROW;
    src = (const char*)r.q + off;
    dst = (char*)r.q_out + off;
  } else {
    if (slot < 0) return;
    const int64_t off_new = (t * r.n_kv_heads + kvh) * (int64_t)ROW;
    const int64_t off_pool = ((int64_t)slot * r.n_kv_heads + kvh) * ROW;
    src = (const char*)(is_k ? r.k_new : r.v_new) + off_new;
    dst = (char*)(is_k ? r.k_layer : r.v_layer) + off_pool;
  }
  if (!is_q && !is_k) {  // v: unrotated copy
    *(u32x4*)(dst + 16 * c) = *(const u32x4*)(src + 16 * c);
    return;
  }
  if (r.interleaved) {
    float x[EPC];
    IO::load(src + 16 * c, x);
    const int i0 = c * (EPC / 2);  // first pair of this chunk
#pragma unroll
    for (int j = 0; j < EPC / 2; ++j) {
      const float2 cs = tab[i0 + j];
      rotate(x[2 * j], x[2 * j + 1], cs.x, cs.y);
    }
    IO::store(dst + 16 * c, x);
  } else {
    if (c >= CPR / 2) return;  // the partner thread of the first half does this chunk
    float a[EPC], b[EPC];
    IO::load(src + 16 * c, a);
    IO::load(src + ROW / 2 + 16 * c, b);
    const int i0 = c * EPC;  // pairs (i, i + D/2) for i = i0 .. i0 + EPC - 1
#pragma unroll
    for (int j = 0; j < EPC; ++j) {
      const float2 cs = tab[i0 + j];
      rotate(a[j], b[j], cs.x, cs.y);
    }
    IO::store(dst + 16 * c, a);
    IO::store(dst + ROW / 2 + 16 * c, b);
  }
}

// E4M3 pools: q, k_new, v_new and q_out are bf16; the pool rows hold codes.
// One thread per 16-byte chunk (8 elements) of a bf16 row, as in the kernel
// above; its k and v codes are 8 bytes at code offset 8 c (and D/2 + 8 c for
// the second half of a half-split pair). k is rotated with rotate_rn and
// quantised under the layer's K scale, v quantised unrotated under the V scale.
template <int D>
__global__ __launch_bounds__(256) void rope_kv_store_fp8_kernel(RopeArgs r) {
  using IO = RopeIO<bf16_t>;
  constexpr int ROW = 2 * D;   // bytes of one bf16 head row
  constexpr int CPR = ROW / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int rows_per_token = r.n_q_heads + 2 * r.n_kv_heads;
  const int64_t total = r.n_tokens * rows_per_token * CPR;
  if (idx >= total) return;
  const int c = (int)(idx % CPR);
  const int64_t row = idx / CPR;
  const int64_t t = row / rows_per_token;
  const int h = (int)(row - t * rows_per_token);
  int p = r.positions[t];
  p = p < 0 ? 0 : (p >= r.max_pos ? r.max_pos - 1 : p);
  const float2* tab = (const float2*)r.freqs_cis + (int64_t)p * (D / 2);
  const bool is_q = h < r.n_q_heads;
  const bool is_k = !is_q && h < r.n_q_heads + r.n_kv_heads;
  if (is_q) {  // as for bf16 pools
    if (!r.q) return;
    const int64_t off = (t * r.n_q_heads + h) * (int64_t)ROW;
    const char* src = (const char*)r.q + off;
    char* dst = (char*)r.q_out + off;
    if (r.interleaved) {
      float x[8];
      IO::load(src + 16 * c, x);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float2 cs = tab[c * 4 + j];
        rotate(x[2 * j], x[2 * j + 1], cs.x, cs.y);
      }
      IO::store(dst + 16 * c, x);
    } else if (c < CPR / 2) {
      float a[8], b[8];
      IO::load(src + 16 * c, a);
      IO::load(src + ROW / 2 + 16 * c, b);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float2 cs = tab[c * 8 + j];
        rotate(a[j], b[j], cs.x, cs.y);
      }
      IO::store(dst + 16 * c, a);
      IO::store(dst + ROW / 2 + 16 * c, b);
    }
    return;
  }
  const int kvh = is_k ? h - r.n_q_heads : h - r.n_q_heads - r.n_kv_heads;
  const int s = r.loc[t];
  if (s < 0 || (int64_t)s >= r.n_slots) return;
  const char* src =
      (const char*)(is_k ? r.k_new : r.v_new) + (t * r.n_kv_heads + kvh) * (int64_t)ROW;
  char* dst = (char*)(is_k ? r.k_layer : r.v_layer) + ((int64_t)s * r.n_kv_heads + kvh) * D;
  const float scale = r.kv_scale[is_k ? 0 : 1];
  if (!is_k) {  // v: quantised unrotated
    float x[8];
    IO::load(src + 16 * c, x);
    *(u32x2*)(dst + 8 * c) = quant8(x, scale);
    return;
  }
  if (r.interleaved) {
    float x[8];
    IO::load(src + 16 * c, x);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float2 cs = tab[c * 4 + j];
      rotate_rn(x[2 * j], x[2 * j + 1], cs.x, cs.y);
    }
    *(u32x2*)(dst + 8 * c) = quant8(x, scale);
  } else if (c < CPR / 2) {
    float a[8], b[8];
    IO::load(src + 16 * c, a);
    IO::load(src + ROW / 2 + 16 * c, b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float2 cs = tab[c * 8 + j];
      rotate_rn(a[j], b[j], cs.x, cs.y);
    }
    *(u32x2*)(dst + 8 * c) = quant8(a, scale);
    *(u32x2*)(dst + D / 2 + 8 * c) = quant8(b, scale);
  }
}

template <typename T, int D>
hipError_t launch_for(const RopeArgs& r, hipStream_t stream) {
  constexpr int CPR = D * elem_size<T>::value / 16;
  const int64_t total = r.n_tokens * (r.n_q_heads + 2 * r.n_kv_heads) * CPR;
  const int64_t blocks = (total + 255) / 256;
  rope_kv_store_kernel<T, D><<<dim3((unsigned)blocks), 256, 0, stream>>>(r);
  return hipGetLastError();
}

}  // namespace

template <int D>
hipError_t launch_fp8(const RopeArgs& r, hipStream_t stream) {
  constexpr int CPR = 2 * D / 16;
  const int64_t total = r.n_tokens * (r.n_q_heads + 2 * r.n_kv_heads) * CPR;
  const int64_t blocks = (total + 255) / 256;
  rope_kv_store_fp8_kernel<D><<<dim3((unsigned)blocks), 256, 0, stream>>>(r);
  return hipGetLastError();
}

hipError_t launch_rope_kv_store(const RopeArgs& r, hipStream_t stream) {
  if (r.n_tokens == 0) return hipSuccess;
  if (r.dtype == PKV_FP8_E4M3)
    return r.head_dim == 128 ? launch_fp8<128>(r, stream) : launch_fp8<64>(r, stream);
  if (r.dtype == PKV_BF16)
    return r.head_dim == 128 ? launch_for<bf16_t, 128>(r, stream) : launch_for<bf16_t, 64>(r, stream);
  return r.head_dim == 128 ? launch_for<float, 128>(r, stream) : launch_for<float, 64>(r, stream);
}

}  // namespace pkv
