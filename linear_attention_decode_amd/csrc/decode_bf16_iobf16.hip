// decode_bf16_iobf16.hip -- decode / verify kernels for a bf16 checkpoint tile and
// bf16 q / k / v.
#include "decode_impl.h"

namespace replay {
template hipError_t launch_decode_st<ST_BF16, true>(int P, int N, const DecodeArgs &a, hipStream_t s);
}  // namespace replay
