// Decode kernel instantiations for bf16 K/V, head_dim 64
// (one translation unit per variant so the library builds in parallel).
#include "decode_impl.hpp"
#include "decode_mfma.hpp"

namespace pkv {

hipError_t launch_decode_partials_bf16_64(const DecodeArgs& a, hipStream_t stream) {
  // g >= 8: MFMA kernel; smaller groups: VALU kernel
  if (a.n_q_heads / a.n_kv_heads >= 8) return decode_mfma::partials_for_dim<64>(a, stream);
  return decode_impl::partials_for_dim<bf16_t, 64, 4>(a, stream);
}

hipError_t launch_decode_merge_bf16_64(const DecodeArgs& a, hipStream_t stream) {
  return decode_impl::merge_for_dim<bf16_t, 64>(a, stream);
}

}  // namespace pkv
