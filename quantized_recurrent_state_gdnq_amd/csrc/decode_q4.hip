// Decode step with the uniform 4-bit state (Low-Bit GDN ..., abstract: the
// "@4" budget): the kernel templates of decode_impl.h instantiated with
// 4-bit codes, in a unit of their own so that it compiles beside decode.hip.
#include "decode_impl.h"

namespace gdnq {

hipError_t launch_decode_q4(const DecodeLaunch& L, const DecodeArgs& a, hipStream_t stream) {
  return launch_qb<4>(L, a, stream);
}

}  // namespace gdnq
