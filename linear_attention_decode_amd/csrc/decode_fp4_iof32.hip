// decode_fp4_iof32.hip -- decode / verify kernels for an MX FP4 checkpoint copy and
// f32 q / k / v.
#include "decode_impl.h"

namespace replay {
template hipError_t launch_decode_st<ST_FP4, false>(int P, int N, const DecodeArgs &a, hipStream_t s);
}  // namespace replay
