// step_common.h -- tiling and row copies shared by the fused step kernels
// (step.hip, verify_step.hip).
#pragma once
#include "ring_mx.h"

namespace replay {

template <int P, int N>
struct StepShape {
    static constexpr int VEC = 4;
    static constexpr int CHUNKS = P * N / VEC;
    // streaming threads: at most 8 chunks a lane (4096 chunks: 8 wavefronts)
    static constexpr int NTS = CHUNKS >= 4096 ? 512 : (CHUNKS < 256 ? CHUNKS : 256);
    static constexpr int ITER = CHUNKS / NTS;
    static constexpr int LPR = N / VEC;
    static constexpr int RPI = NTS / LPR;
    static_assert(CHUNKS % NTS == 0 && NTS % 64 == 0, "bad tiling");
    static_assert(LPR <= 64 && 64 % LPR == 0, "row group must sit in a wavefront");
};

// Raw 32-bit words of one io row (N elements), copied by the 64 lanes.
template <int N, bool IOB>
struct RowWords {
    static constexpr int WORDS = N * (IOB ? 2 : 4) / 4;
    static constexpr int WPL = (WORDS + 63) / 64;
    uint32_t w[WPL];
    __device__ __forceinline__ void load(const void *row, int lane) {
#pragma unroll
        for (int i = 0; i < WPL; ++i) {
            const int k = lane + 64 * i;
            w[i] = static_cast<const uint32_t *>(row)[k < WORDS ? k : WORDS - 1];
        }
    }
    __device__ __forceinline__ void store(void *row, int lane) const {
#pragma unroll
        for (int i = 0; i < WPL; ++i) {
            const int k = lane + 64 * i;
            if (k < WORDS) static_cast<uint32_t *>(row)[k] = w[i];
        }
    }
};

}  // namespace replay
