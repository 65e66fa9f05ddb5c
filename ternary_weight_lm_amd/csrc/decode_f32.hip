// decode_f32.hip -- the decode kernels of decode_kernels.h for fp32 activations.
#include "decode_kernels.h"

namespace bl {

void launch_decode_f32(const DecodeArgs &a, hipStream_t stream) { launch_decode_dt<BL_F32>(a, stream); }

}  // namespace bl
