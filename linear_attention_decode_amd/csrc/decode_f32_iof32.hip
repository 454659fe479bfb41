// decode_f32_iof32.hip -- decode / verify kernels for a f32 checkpoint tile and
// float32 q / k / v.
#include "decode_impl.h"

namespace replay {
template hipError_t launch_decode_st<ST_F32, false>(int P, int N, const DecodeArgs &a, hipStream_t s);
}  // namespace replay
