// Split-KV paged decode: dtype / head_dim dispatch to the per-variant
// translation units (kernels in decode_impl.hpp).
#include "internal.hpp"

namespace pkv {

hipError_t launch_decode_partials_bf16_128(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_partials_bf16_64(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_partials_f32_128(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_partials_f32_64(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge_bf16_128(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge_bf16_64(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge_f32_128(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge_f32_64(const DecodeArgs& a, hipStream_t stream);

hipError_t launch_decode_partials(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (a.dtype == PKV_BF16)
    return a.head_dim == 128 ? launch_decode_partials_bf16_128(a, stream)
                             : launch_decode_partials_bf16_64(a, stream);
  return a.head_dim == 128 ? launch_decode_partials_f32_128(a, stream)
                           : launch_decode_partials_f32_64(a, stream);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (a.dtype == PKV_BF16)
    return a.head_dim == 128 ? launch_decode_merge_bf16_128(a, stream)
                             : launch_decode_merge_bf16_64(a, stream);
  return a.head_dim == 128 ? launch_decode_merge_f32_128(a, stream)
                           : launch_decode_merge_f32_64(a, stream);
}

}  // namespace pkv
