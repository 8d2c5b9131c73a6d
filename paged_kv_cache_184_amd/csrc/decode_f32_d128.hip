// Decode kernel instantiations for fp32 K/V, head_dim 128
// (one translation unit per variant so the library builds in parallel).
#include "decode_impl.hpp"

namespace pkv {

hipError_t launch_decode_partials_f32_128(const DecodeArgs& a, hipStream_t stream) {
  return decode_impl::partials_for_dim<float, 128>(a, stream);
}

hipError_t launch_decode_merge_f32_128(const DecodeArgs& a, hipStream_t stream) {
  return decode_impl::merge_for_dim<float, 128>(a, stream);
}

}  // namespace pkv
