// Decode kernel instantiations for FP8 (E4M3) K/V with bf16 q and output,
// head_dim 128 (one translation unit per variant so the library builds in
// parallel). Every group size runs the MFMA kernel, with the codes widened to
// bf16 in registers; the merge is the bf16 one.
#include "decode_impl.hpp"
#include "decode_mfma.hpp"

namespace pkv {

hipError_t launch_decode_partials_fp8_128(const DecodeArgs& a, hipStream_t stream) {
  return decode_mfma::partials_for_dim<128, fp8_t>(a, stream);
}

}  // namespace pkv
