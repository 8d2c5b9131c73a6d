// Split-KV paged decode: dtype / head_dim dispatch to the per-variant
// translation units (kernels in decode_impl.hpp).
#include "internal.hpp"

namespace pkv {

hipError_t launch_decode_partials_bf16_128(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_partials_bf16_64(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_partials_f32_128(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_partials_f32_64(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_partials_fp8_128(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_partials_fp8_64(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge_bf16_128(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge_bf16_64(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge_f32_128(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge_f32_64(const DecodeArgs& a, hipStream_t stream);

hipError_t launch_decode_partials(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (a.dtype == PKV_FP8_E4M3)
    return a.head_dim == 128 ? launch_decode_partials_fp8_128(a, stream)
                             : launch_decode_partials_fp8_64(a, stream);
  if (a.dtype == PKV_BF16)
    return a.head_dim == 128 ? launch_decode_partials_bf16_128(a, stream)
                             : launch_decode_partials_bf16_64(a, stream);
  return a.head_dim == 128 ? launch_decode_partials_f32_128(a, stream)
                           : launch_decode_partials_f32_64(a, stream);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (a.dtype == PKV_BF16 || a.dtype == PKV_FP8_E4M3)  // FP8 pools: bf16 output
    return a.head_dim == 128 ? launch_decode_merge_bf16_128(a, stream)
                             : launch_decode_merge_bf16_64(a, stream);
  return a.head_dim == 128 ? launch_decode_merge_f32_128(a, stream)
                           : launch_decode_merge_f32_64(a, stream);
}

}  // namespace pkv
