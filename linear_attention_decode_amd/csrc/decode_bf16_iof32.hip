// decode_bf16_iof32.hip -- decode / verify kernels for a bf16 checkpoint tile and
// float32 q / k / v.
#include "decode_impl.h"

namespace replay {
template hipError_t launch_decode_st<ST_BF16, false>(int P, int N, const DecodeArgs &a, hipStream_t s);
}  // namespace replay
