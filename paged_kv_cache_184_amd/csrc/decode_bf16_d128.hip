// Decode kernel instantiations for bf16 K/V, head_dim 128
// (one translation unit per variant so the library builds in parallel).
#include "decode_impl.hpp"
#include "decode_mfma.hpp"

namespace pkv {

hipError_t launch_decode_partials_bf16_128(const DecodeArgs& a, hipStream_t stream) {
  // g >= 8: MFMA kernel; smaller groups: VALU kernel
  if (a.n_q_heads / a.n_kv_heads >= 8) return decode_mfma::partials_for_dim<128>(a, stream);
  return decode_impl::partials_for_dim<bf16_t, 128, 4>(a, stream);
}

hipError_t launch_decode_merge_bf16_128(const DecodeArgs& a, hipStream_t stream) {
  return decode_impl::merge_for_dim<bf16_t, 128>(a, stream);
}

}  // namespace pkv
