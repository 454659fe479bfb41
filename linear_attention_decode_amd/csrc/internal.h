// internal.h -- private declarations shared by the HIP sources of libreplayssm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/replayssm.h"

namespace replay {

// Index of (sequence b, ring slot, head h) in the ring's dt and a, laid out
// [B][L][H] (slot-major: the values one step appends for a sequence, every
// head, are contiguous).  bh = b * H + h.
__host__ __device__ inline size_t dta_index(size_t b, size_t bh, int H, int L, int slot) {
    return (b * (size_t)L + (size_t)slot) * (size_t)H + (bh - b * (size_t)H);
}

// Storage kinds of a state tile.
enum StateKind : int { ST_F32 = 0, ST_BF16 = 1, ST_FP8 = 2, ST_FP4 = 3 };

// Largest ring and verify window the kernels are built for.
constexpr int kMaxRing = 32;
constexpr int kMaxWindow = 8;        // verify windows of the register kernel (decode_impl.h)
constexpr int kMaxWideWindow = 16;   // windows on the matrix cores (verify_wide.hip)
constexpr int kWideFrom = 6;         // replay_verify and the fused verify round take the matrix cores from here on
                                     // (where supported): both switch together, so a fused round equals the calls
                                     // bit for bit; at W = 5 the fused round is faster with register sums

// Arrival counters of the fused step, [B][G + 1] of them, one int32 per
// 128-byte line: a workgroup arrives at its group's counter, the last head
// of a group at the sequence's.  Counters that share a line, or one counter
// for all H heads, make the device-scope atomics queue behind each other.
constexpr int kSyncStride = 32;

// Everything a kernel needs to find one layer's ring.
struct RingView {
    const void *q;      // [B][G][L][N]
    const void *k;      // [B][G][L][N]
    const void *v;      // [B][H][L][P]
    const float *dt;    // [B][L][H] (slot-major, dta_index)
    const float *a;     // [B][L][H]
    const int32_t *pos;
    const int32_t *base;
    int32_t *err;       // [B+1]
    int32_t B, H, G, L;
    int32_t io_bf16;
};

struct DecodeArgs {
    RingView r;
    const void *S;          // state tile source: f32 master or the copy
    const void *scale;      // float [B][H] for an e4m3 copy, uint8 [B][H][P*N/32] for FP4, else unused
    float *y;               // [B][W][H][P]
    int32_t W;
};

struct FlushArgs {
    RingView r;
    const void *S_in;       // f32 master (separated) or the copy (shared) or a load source
    const void *scale_in;   // old scales when S_in is a copy: float per head (e4m3), E8M0 byte per block (FP4)
    float *S_out;           // f32 master to write, or nullptr
    void *copy_out;         // copy to write, or nullptr
    void *scale_out;        // scales to write: float per head (e4m3), E8M0 byte per block (FP4), or nullptr
    int32_t min_count;      // flush sequences with count >= max(min_count, 1)
    int32_t force_empty;    // 1: treat every sequence as due with an empty ring (checkpoint load)
    int32_t *base_out;      // base, set to pos by the last workgroup of a folded sequence
    int32_t *sync;          // arrival counters [B][G + 1][kSyncStride]
};

// One fused standard decode step (W = 1) or speculative-verify round
// (W drafts), float32 checkpoint.
struct StepArgs {
    void *ring_q, *ring_k, *ring_v;   // [B][G][L][N] x2, [B][H][L][P]
    float *ring_dt, *ring_a;          // [B][L][H] (slot-major, dta_index)
    int32_t *pos, *base, *err, *sync;  // sync: [B][G + 1][kSyncStride], element [..][0]
    float *S;                         // [B][H][P][N] master, read and (when folding) written
    const void *q, *k, *v;            // [B][W][G][N] x2, [B][W][H][P]
    const float *dt, *a;              // [B][W][H]
    float *y;                         // [B][W][H][P]
    int32_t B, H, G, L;
    int32_t flush_at;
    int32_t io_bf16;
    int32_t W;                        // drafts per round (the verify round; the step takes 1)
    const void *copy;                 // low-precision checkpoint copy the step reads (copy modes)
    const void *copy_scale;           // its scales: e4m3 float [B][H], FP4 E8M0 bytes [B][H][P*N/32]
    int32_t copy_st;                  // StateKind of the copy (ST_BF16, ST_FP8, ST_FP4)
    const int32_t *n_reject;          // verify round only: [B] rollback applied first, or null
};

// n layers of one shape stepped in one launch (step_layers_kernel); passed
// by value in the kernel arguments.
constexpr int kMaxStepLayers = 16;
struct StepLayersArgs {
    StepArgs l[kMaxStepLayers];
    int32_t n;
};

struct EagerArgs {
    const float *S_in;
    float *S_out;
    const void *q, *k, *v;  // [B][G][N], [B][G][N], [B][H][P]
    const float *dt, *a;    // [B][H]
    float *y;               // [B][H][P]
    int32_t B, H, G;
    int32_t io_bf16;
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_decode(int P, int N, int st, const DecodeArgs &a, hipStream_t s);
hipError_t launch_verify_wide(int P, int N, int st, const DecodeArgs &a, hipStream_t s);   // 1 <= W <= 16
bool verify_wide_supported(int st, const DecodeArgs &a);
hipError_t launch_flush(int P, int N, int st_in, int st_copy, bool write_master, const FlushArgs &a,
                        hipStream_t s);
// the fold of a shared checkpoint: the copy (type st) read, folded and rewritten in place
hipError_t launch_flush_shared(int P, int N, int st, const FlushArgs &a, hipStream_t s);

// Gated DeltaNet layers (gdn.hip): the output-only route (decode, W = 1, and
// verify, W <= kMaxWindow; DecodeArgs as launch_decode with a float32
// checkpoint), the fold of the ring into the float32 master, and the eager step.
// Where the entries of a fold come from: the ring (flush: entries 0..count-1
// of the sequence) or the call's one token (eager step).
struct GdnFoldArgs {
    RingView r;              // flush: the ring; eager: B, H, G, io_bf16 used
    const void *S_in;        // float32 checkpoint, or (shared) the low-precision copy
    const void *scale_in;    // shared: the copy's scales (e4m3 [B][H], FP4 one byte a block)
    float *S_out;            // float32 checkpoint written, or null (shared)
    void *copy_out;          // copy rewritten from the folded state, or null
    void *scale_out;         // its scales (e4m3, FP4), or null
    int32_t min_count;       // flush: fold sequences with count >= max(min_count, 1)
    int32_t *base_out;       // flush: base, set to pos by the last workgroup of a folded sequence
    int32_t *sync;           // flush: arrival counters [B][G + 1][kSyncStride]
    // eager: one token per (sequence, head)
    const void *q, *k, *v;   // [B][G][N], [B][G][N], [B][H][P]
    const float *beta, *alpha;   // [B][H]
    float *y;                // [B][H][P]
};
// st: the state read (ST_F32 for the master, else the copy's kind)
hipError_t launch_gdn_verify(int P, int N, int st, const DecodeArgs &a, hipStream_t s);
// st_in: ST_F32, or the copy's kind when the copy is the only checkpoint;
// st_copy: the copy written (-1: none); write_master: the float32 checkpoint is written
hipError_t launch_gdn_flush(int P, int N, int st_in, int st_copy, bool write_master, const GdnFoldArgs &a,
                            hipStream_t s);
hipError_t launch_gdn_eager(int P, int N, const GdnFoldArgs &a, hipStream_t s);
hipError_t launch_append(int P, int N, const RingView &r, void *ring_q, void *ring_k, void *ring_v,
                         float *ring_dt, float *ring_a, int32_t *pos, int32_t *sync, int32_t W, const void *q,
                         const void *k, const void *v, const float *dt, const float *a, hipStream_t s);
hipError_t launch_rollback(const RingView &r, int32_t *pos, const int32_t *n_reject, hipStream_t s);
hipError_t launch_fill_u32(void *dst, uint32_t value, size_t count, hipStream_t s);
hipError_t launch_eager(int P, int N, const EagerArgs &a, hipStream_t s);
hipError_t launch_step(int P, int N, const StepArgs &a, hipStream_t s);
hipError_t launch_step_layers(int P, int N, const StepLayersArgs &a, hipStream_t s);   // 1 <= a.n <= kMaxStepLayers
int step_workgroups_per_layer(int P, const StepArgs &a);   // compute workgroups of one layer's step
// Layers with more compute workgroups than this are stepped one launch
// each: there the single launch measured slower (8 layers, 128 x 128 heads:
// -4 % at 8192 workgroups a layer, +1.3 % at 16384, +5 % at 65536).
constexpr int kLayersOneLaunchMax = 8192;
hipError_t launch_verify_step(int P, int N, const StepArgs &a, hipStream_t s);
hipError_t launch_step_copy(int P, int N, const StepArgs &a, hipStream_t s);   // append + decode from the copy
bool verify_step_fused(int P, int N, const StepArgs &a);   // the fused round covers this case
hipError_t launch_verify_step_copy(int P, int N, const StepArgs &a, hipStream_t s);   // the round with an e4m3 / FP4 read
bool verify_step_copy_fused(int P, int N, const StepArgs &a);
hipError_t launch_eager_select(const float *snaps, int32_t W, const int32_t *n_accept, float *s,
                               int32_t B, size_t head_elems_per_seq, hipStream_t st);
hipError_t launch_probe(int mode, const void *src, void *dst, size_t bytes, hipStream_t s);

bool shape_supported(int P, int N);

}  // namespace replay
