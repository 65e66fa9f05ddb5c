// decode.hip -- dispatch of the decode kernels (decode_kernels.h) on the
// activation dtype; each dtype's kernels live in a source file of their own.
#include "bl_launch.h"

namespace bl {

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  switch (a.x_dtype) {
    case BL_F32: launch_decode_f32(a, stream); break;
    case BL_F16: launch_decode_f16(a, stream); break;
    default: launch_decode_bf16(a, stream); break;
  }
  return hipGetLastError();
}

// 16-bit activations only (decode_gated_fits)
hipError_t launch_decode_gated(const DecodeGateArgs &a, hipStream_t stream) {
  if (a.x_dtype == BL_F16) launch_decode_gated_f16(a, stream);
  else launch_decode_gated_bf16(a, stream);
  return hipGetLastError();
}

}  // namespace bl
