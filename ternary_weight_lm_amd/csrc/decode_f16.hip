// decode_f16.hip -- the decode kernels of decode_kernels.h for fp16 activations.
#include "decode_kernels.h"

namespace bl {

void launch_decode_f16(const DecodeArgs &a, hipStream_t stream) { launch_decode_dt<BL_F16>(a, stream); }

}  // namespace bl
