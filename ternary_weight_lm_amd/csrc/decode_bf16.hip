// decode_bf16.hip -- the decode kernels of decode_kernels.h for bf16 activations.
#include "decode_kernels.h"

namespace bl {

void launch_decode_bf16(const DecodeArgs &a, hipStream_t stream) { launch_decode_dt<BL_BF16>(a, stream); }
void launch_decode_gated_bf16(const DecodeGateArgs &a, hipStream_t stream) {
  launch_decode_gated_dt<BL_BF16>(a, stream);
}

}  // namespace bl
