// decode_fp8_iobf16.hip -- decode / verify kernels for a fp8 checkpoint tile and
// bf16 q / k / v.
#include "decode_impl.h"

namespace replay {
template hipError_t launch_decode_st<ST_FP8, true>(int P, int N, const DecodeArgs &a, hipStream_t s);
}  // namespace replay
