// decode_fp4_iobf16.hip -- decode / verify kernels for an MX FP4 checkpoint copy and
// bf16 q / k / v.
#include "decode_impl.h"

namespace replay {
template hipError_t launch_decode_st<ST_FP4, true>(int P, int N, const DecodeArgs &a, hipStream_t s);
}  // namespace replay
