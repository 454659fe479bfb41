// decode.hip -- dispatch of the decode / verify kernels by checkpoint dtype and
// io dtype (kernels in decode_impl.h, instantiated in decode_<state>_<io>.hip).
#include "decode_impl.h"

namespace replay {

#define REPLAY_DECODE_EXTERN(ST, IOB) \
    extern template hipError_t launch_decode_st<ST, IOB>(int, int, const DecodeArgs &, hipStream_t);
REPLAY_DECODE_EXTERN(ST_F32, false)
REPLAY_DECODE_EXTERN(ST_F32, true)
REPLAY_DECODE_EXTERN(ST_BF16, false)
REPLAY_DECODE_EXTERN(ST_BF16, true)
REPLAY_DECODE_EXTERN(ST_FP8, false)
REPLAY_DECODE_EXTERN(ST_FP8, true)
REPLAY_DECODE_EXTERN(ST_FP4, false)
REPLAY_DECODE_EXTERN(ST_FP4, true)
#undef REPLAY_DECODE_EXTERN

hipError_t launch_decode(int P, int N, int st, const DecodeArgs &a, hipStream_t s) {
    const bool io = a.r.io_bf16 != 0;
    switch (st) {
        case ST_F32: return io ? launch_decode_st<ST_F32, true>(P, N, a, s) : launch_decode_st<ST_F32, false>(P, N, a, s);
        case ST_BF16: return io ? launch_decode_st<ST_BF16, true>(P, N, a, s) : launch_decode_st<ST_BF16, false>(P, N, a, s);
        case ST_FP8: return io ? launch_decode_st<ST_FP8, true>(P, N, a, s) : launch_decode_st<ST_FP8, false>(P, N, a, s);
        default: return io ? launch_decode_st<ST_FP4, true>(P, N, a, s) : launch_decode_st<ST_FP4, false>(P, N, a, s);
    }
}

}  // namespace replay
