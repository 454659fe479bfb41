// abi.hip -- the extern "C" boundary of libreplayssm: host-side validation,
// launch configuration and the handle.  Every compute step runs in the
// kernels of decode*.hip (output-only decode and register verify),
// verify_wide.hip (matrix-core verify), step.hip and step_copy.hip (the
// fused decode step, one layer or stacked layers), verify_step.hip (the
// fused speculative round), flush.hip and flush_shared.hip (the folds of a
// float32 master and of a shared low-precision checkpoint), gdn.hip (Gated
// DeltaNet layers), ring.hip (append, rollback, fills), eager.hip and
// probe.hip.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "count_bound.h"
#include "internal.h"

using namespace replay;

// Arrival counters owned by the library, for replay_step_static (callers
// that cannot allocate device memory).  Every GPU the library runs on holds
// its own copy of this array until the process ends.  Host code never uses
// the name as an address: replay_init resolves the current device's copy
// with hipGetSymbolAddress, once per device, and kernels get that pointer.
constexpr size_t kStaticCounterBytes = size_t(2) << 20;
static __device__ __align__(256) int32_t scratch[kStaticCounterBytes / sizeof(int32_t)];

struct replay_handle {
    replay_config cfg;
    replay_buffers bufs;
    CountBound bound;   // upper bounds on every sequence's count and pos
    bool graphed = false;   // a call that moves the pointers was recorded into a graph
    bool untracked = false; // the caller moves pos / base itself (replay_set_flush_skipping(0))
    int32_t *static_sync = nullptr;   // this device's copy of `scratch` (nullptr if it could not be resolved)
};

namespace {

constexpr int kNumBufferFields = 12;
constexpr int kSyncField = 11;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, resolved on first use on that device.
hipError_t static_counters(int32_t **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<int32_t *>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// bytes of arrival counters a configuration needs ([B][G + 1][kSyncStride] int32)
size_t counter_bytes(const replay_config &c) {
    return (size_t)c.batch * (size_t)(c.groups + 1) * kSyncStride * sizeof(int32_t);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

replay_status from_hip(hipError_t e) { return e == hipSuccess ? REPLAY_OK : REPLAY_ERR_HIP; }

int io_bytes(const replay_config &c) { return c.io_dtype == REPLAY_BF16 ? 2 : 4; }

int state_kind(int32_t dtype) {
    return dtype == REPLAY_BF16 ? ST_BF16 : (dtype == REPLAY_FP8_E4M3 ? ST_FP8 : (dtype == REPLAY_FP4_E2M1 ? ST_FP4 : ST_F32));
}

// Shape and dtype checks shared by every entry point that takes a config.
replay_status check_shape(const replay_config *c) {
    if (!c) return REPLAY_ERR_INVALID_ARG;
    if (c->batch < 1 || c->heads < 1 || c->groups < 1 || c->head_dim < 1 || c->state_dim < 1)
        return REPLAY_ERR_INVALID_ARG;
    if (c->heads % c->groups != 0) return REPLAY_ERR_INVALID_ARG;
    if ((int64_t)c->batch * c->heads > INT32_MAX) return REPLAY_ERR_UNSUPPORTED;
    if (!shape_supported(c->head_dim, c->state_dim)) return REPLAY_ERR_UNSUPPORTED;
    if (c->io_dtype != REPLAY_F32 && c->io_dtype != REPLAY_BF16) return REPLAY_ERR_UNSUPPORTED;
    if (c->rule != REPLAY_RULE_MAMBA2 && c->rule != REPLAY_RULE_GATED_DELTA) return REPLAY_ERR_INVALID_ARG;
    return REPLAY_OK;
}

replay_status check_config(const replay_config *c) {
    replay_status st = check_shape(c);
    if (st != REPLAY_OK) return st;
    if (c->ring_len < 1) return REPLAY_ERR_INVALID_ARG;
    if (c->ring_len > kMaxRing) return REPLAY_ERR_UNSUPPORTED;
    if (c->read_copy != REPLAY_NONE && c->read_copy != REPLAY_BF16 && c->read_copy != REPLAY_FP8_E4M3 &&
        c->read_copy != REPLAY_FP4_E2M1)
        return REPLAY_ERR_UNSUPPORTED;
    if (c->shared_lowp != 0 && c->shared_lowp != 1) return REPLAY_ERR_INVALID_ARG;
    if (c->shared_lowp && c->read_copy == REPLAY_NONE) return REPLAY_ERR_INVALID_ARG;
    return REPLAY_OK;
}

void buffer_bytes(const replay_config &c, size_t out[kNumBufferFields]) {
    const size_t B = c.batch, H = c.heads, G = c.groups, P = c.head_dim, N = c.state_dim,
                 L = c.ring_len, esz = io_bytes(c);
    const size_t state = B * H * P * N;
    out[0] = c.shared_lowp ? 0 : state * 4;                                            // s_master
    out[1] = c.read_copy == REPLAY_NONE ? 0
             : (c.read_copy == REPLAY_BF16 ? state * 2 : (c.read_copy == REPLAY_FP4_E2M1 ? state / 2 : state));  // s_copy
    out[2] = c.read_copy == REPLAY_FP8_E4M3 ? B * H * 4
             : (c.read_copy == REPLAY_FP4_E2M1 ? state / 32 : 0);                     // s_scale
    out[3] = B * G * L * N * esz;                                                       // ring_q
    out[4] = B * G * L * N * esz;                                                       // ring_k
    out[5] = B * H * L * P * esz;                                                       // ring_v
    out[6] = B * H * L * 4;                                                             // ring_dt
    out[7] = B * H * L * 4;                                                             // ring_a
    out[8] = B * 4;                                                                     // pos
    out[9] = B * 4;                                                                     // base
    out[10] = (B + 1) * 4;                                                              // err
    out[11] = B * (size_t)(c.groups + 1) * 4 * kSyncStride;                             // sync
}

const void *field(const replay_buffers &b, int i) {
    const void *f[kNumBufferFields] = {b.s_master, b.s_copy, b.s_scale, b.ring_q, b.ring_k, b.ring_v,
                                       b.ring_dt,  b.ring_a, b.pos,     b.base,   b.err,    b.sync};
    return f[i];
}

RingView ring_view(const replay_handle *h) {
    RingView r;
    r.q = h->bufs.ring_q;
    r.k = h->bufs.ring_k;
    r.v = h->bufs.ring_v;
    r.dt = h->bufs.ring_dt;
    r.a = h->bufs.ring_a;
    r.pos = h->bufs.pos;
    r.base = h->bufs.base;
    r.err = h->bufs.err;
    r.B = h->cfg.batch;
    r.H = h->cfg.heads;
    r.G = h->cfg.groups;
    r.L = h->cfg.ring_len;
    r.io_bf16 = h->cfg.io_dtype == REPLAY_BF16;
    return r;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

// A call recorded into a graph (stream capture) moves the pointers again on
// every replay without passing through the handle, so from then on the
// host-side count bounds no longer describe the device: the handle stops
// skipping flushes for good.  A failed query counts as a capture.
void note_capture(replay_handle *h, hipStream_t s) {
    if (h->graphed) return;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess || st != hipStreamCaptureStatusNone) h->graphed = true;
}

// Fold (or load) into the checkpoint and rewrite the copy, then move base.
replay_status run_flush(replay_handle *h, const float *load_src, int32_t min_count, hipStream_t s, int32_t *sync) {
    const replay_config &c = h->cfg;
    FlushArgs a;
    a.r = ring_view(h);
    a.min_count = min_count;
    a.force_empty = load_src != nullptr;
    a.base_out = h->bufs.base;
    a.sync = sync;
    a.S_out = c.shared_lowp ? nullptr : h->bufs.s_master;
    a.copy_out = c.read_copy == REPLAY_NONE ? nullptr : h->bufs.s_copy;
    a.scale_out = (c.read_copy == REPLAY_FP8_E4M3 || c.read_copy == REPLAY_FP4_E2M1) ? h->bufs.s_scale : nullptr;
    int st_in;
    if (load_src) {
        a.S_in = load_src;
        a.scale_in = nullptr;
        st_in = ST_F32;
    } else if (c.shared_lowp) {
        a.S_in = h->bufs.s_copy;
        a.scale_in = h->bufs.s_scale;
        st_in = state_kind(c.read_copy);
    } else {
        a.S_in = h->bufs.s_master;
        a.scale_in = nullptr;
        st_in = ST_F32;
    }
    const int st_copy = c.read_copy == REPLAY_NONE ? -1 : state_kind(c.read_copy);
    // no sequence can be due: the kernel would change nothing
    note_capture(h, s);
    if (!load_src && !h->graphed && !h->untracked && !h->bound.flush_may_fold(min_count)) return REPLAY_OK;
    hipError_t e;
    if (c.rule == REPLAY_RULE_GATED_DELTA && !load_src) {
        // the gated delta rule's fold (a checkpoint load, an empty ring, is the
        // same copy for both rules)
        GdnFoldArgs g{};
        g.r = a.r;
        g.S_in = a.S_in;
        g.scale_in = a.scale_in;
        g.S_out = a.S_out;
        g.copy_out = a.copy_out;
        g.scale_out = a.scale_out;
        g.min_count = min_count;
        g.base_out = h->bufs.base;
        g.sync = sync;
        e = launch_gdn_flush(c.head_dim, c.state_dim, st_in, st_copy, !c.shared_lowp, g, s);
    } else {
        e = launch_flush(c.head_dim, c.state_dim, st_in, st_copy, !c.shared_lowp, a, s);
    }
    if (e != hipSuccess) {
        h->bound.unknown();
        return REPLAY_ERR_HIP;
    }
    if (load_src)
        h->bound.load();
    else
        h->bound.flush(min_count);
    return REPLAY_OK;
}

replay_status run_verify(replay_handle *h, int32_t W, float *y, hipStream_t s) {
    const replay_config &c = h->cfg;
    if (!y || !aligned4(y)) return REPLAY_ERR_INVALID_ARG;
    if (W < 1 || W > kMaxWideWindow || W > c.ring_len) return REPLAY_ERR_INVALID_ARG;
    DecodeArgs a;
    a.r = ring_view(h);
    a.S = c.read_copy == REPLAY_NONE ? static_cast<const void *>(h->bufs.s_master) : h->bufs.s_copy;
    a.scale = h->bufs.s_scale;
    a.y = y;
    a.W = W;
    const int st = state_kind(c.read_copy);
    if (c.rule == REPLAY_RULE_GATED_DELTA) return from_hip(launch_gdn_verify(c.head_dim, c.state_dim, st, a, s));
    // bf16 io: the matrix-core kernel from kWideFrom on; float32 io: past the
    // register kernel's kMaxWindow
    const int wide_from = c.io_dtype == REPLAY_BF16 ? kWideFrom : kMaxWindow + 1;
    if (W >= wide_from && verify_wide_supported(st, a))
        return from_hip(launch_verify_wide(c.head_dim, c.state_dim, st, a, s));
    if (W > kMaxWindow) return REPLAY_ERR_UNSUPPORTED;
    return from_hip(launch_decode(c.head_dim, c.state_dim, st, a, s));
}

}  // namespace

namespace replay {
bool shape_supported(int P, int N) {
    return (P == 16 && N == 16) || (P == 64 && N == 64) || (P == 64 && N == 128) || (P == 128 && N == 128);
}
}  // namespace replay

extern "C" {

const char *replay_status_string(replay_status s) {
    switch (s) {
        case REPLAY_OK: return "ok";
        case REPLAY_ERR_INVALID_ARG: return "invalid argument";
        case REPLAY_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case REPLAY_ERR_HIP: return "HIP runtime error";
        case REPLAY_ERR_TOO_LARGE: return "batch too large for the library's static counters";
    }
    return "unknown status";
}

int32_t replay_abi_version(void) { return REPLAY_ABI_VERSION; }

replay_status replay_buffer_bytes(const replay_config *cfg, size_t bytes[12]) {
    replay_status st = check_config(cfg);
    if (st != REPLAY_OK) return st;
    if (!bytes) return REPLAY_ERR_INVALID_ARG;
    buffer_bytes(*cfg, bytes);
    return REPLAY_OK;
}

replay_status replay_init(const replay_config *cfg, const replay_buffers *bufs, void *stream,
                          replay_handle **out) {
    replay_status st = check_config(cfg);
    if (st != REPLAY_OK) return st;
    if (!bufs || !out) return REPLAY_ERR_INVALID_ARG;
    size_t need[kNumBufferFields];
    buffer_bytes(*cfg, need);
    for (int i = 0; i < kNumBufferFields; ++i) {
        const void *p = field(*bufs, i);
        if (need[i] == 0) continue;
        if (i == kSyncField && !p) continue;   // no counters: only replay_step_static steps this layer
        if (!p || !aligned16(p)) return REPLAY_ERR_INVALID_ARG;
    }
    replay_handle *h = new (std::nothrow) replay_handle;
    if (!h) return REPLAY_ERR_INVALID_ARG;
    h->cfg = *cfg;
    h->bufs = *bufs;
    h->bound.reset(cfg->ring_len);
    if (cfg->shared_lowp) h->bufs.s_master = nullptr;
    if (cfg->read_copy == REPLAY_NONE) h->bufs.s_copy = nullptr;
    if (cfg->read_copy != REPLAY_FP8_E4M3 && cfg->read_copy != REPLAY_FP4_E2M1) h->bufs.s_scale = nullptr;
    if (static_counters(&h->static_sync) != hipSuccess) h->static_sync = nullptr;

    hipStream_t s = as_stream(stream);
    hipError_t e = hipSuccess;
    if (h->bufs.s_master) e = launch_fill_u32(h->bufs.s_master, 0u, need[0] / 4, s);
    if (e == hipSuccess && h->bufs.s_copy) e = launch_fill_u32(h->bufs.s_copy, 0u, need[1] / 4, s);
    // e4m3 scales start at 1.0f; FP4 block scales at byte 0 (2^-127), the scale of an all-zero block
    if (e == hipSuccess && h->bufs.s_scale)
        e = launch_fill_u32(h->bufs.s_scale, cfg->read_copy == REPLAY_FP8_E4M3 ? 0x3f800000u : 0u, need[2] / 4, s);
    if (e == hipSuccess) e = launch_fill_u32(h->bufs.pos, 0u, need[8] / 4, s);
    if (e == hipSuccess) e = launch_fill_u32(h->bufs.base, 0u, need[9] / 4, s);
    if (e == hipSuccess) e = launch_fill_u32(h->bufs.err, 0u, need[10] / 4, s);
    if (e == hipSuccess && h->bufs.sync) e = launch_fill_u32(h->bufs.sync, 0u, need[kSyncField] / 4, s);
    if (e != hipSuccess) {
        delete h;
        return REPLAY_ERR_HIP;
    }
    *out = h;
    return REPLAY_OK;
}

replay_status replay_destroy(replay_handle *h, void *stream) {
    if (!h) return REPLAY_ERR_INVALID_ARG;
    hipError_t e = hipStreamSynchronize(as_stream(stream));
    delete h;
    return from_hip(e);
}

replay_status replay_load_checkpoint(replay_handle *h, const float *s_src, void *stream) {
    if (!h || !s_src || !aligned16(s_src) || !h->bufs.sync) return REPLAY_ERR_INVALID_ARG;
    return run_flush(h, s_src, 0, as_stream(stream), h->bufs.sync);
}

}  // extern "C"

namespace {

replay_status append_impl(replay_handle *h, int32_t W, const void *q, const void *k, const void *v,
                          const float *dt, const float *a, hipStream_t s, int32_t *sync) {
    if (!q || !k || !v || !dt || !a) return REPLAY_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned4(dt) || !aligned4(a))
        return REPLAY_ERR_INVALID_ARG;
    if (W < 1 || W > h->cfg.ring_len) return REPLAY_ERR_INVALID_ARG;
    note_capture(h, s);
    const RingView r = ring_view(h);
    const hipError_t e = launch_append(h->cfg.head_dim, h->cfg.state_dim, r, h->bufs.ring_q, h->bufs.ring_k,
                                       h->bufs.ring_v, h->bufs.ring_dt, h->bufs.ring_a, h->bufs.pos, sync,
                                       W, q, k, v, dt, a, s);
    if (e != hipSuccess) {
        h->bound.unknown();
        return REPLAY_ERR_HIP;
    }
    h->bound.append(W);
    return REPLAY_OK;
}

}  // namespace

extern "C" {

replay_status replay_append(replay_handle *h, int32_t W, const void *q, const void *k, const void *v,
                            const float *dt, const float *a, void *stream) {
    if (!h || !h->bufs.sync) return REPLAY_ERR_INVALID_ARG;
    return append_impl(h, W, q, k, v, dt, a, as_stream(stream), h->bufs.sync);
}

replay_status replay_decode(replay_handle *h, float *y, void *stream) {
    if (!h) return REPLAY_ERR_INVALID_ARG;
    return run_verify(h, 1, y, as_stream(stream));
}

replay_status replay_verify(replay_handle *h, int32_t W, float *y, void *stream) {
    if (!h) return REPLAY_ERR_INVALID_ARG;
    return run_verify(h, W, y, as_stream(stream));
}

replay_status replay_rollback(replay_handle *h, const int32_t *n_reject, void *stream) {
    if (!h || !n_reject || !aligned4(n_reject)) return REPLAY_ERR_INVALID_ARG;
    note_capture(h, as_stream(stream));
    h->bound.rollback();
    return from_hip(launch_rollback(ring_view(h), h->bufs.pos, n_reject, as_stream(stream)));
}

replay_status replay_flush(replay_handle *h, int32_t min_count, void *stream) {
    if (!h || !h->bufs.sync) return REPLAY_ERR_INVALID_ARG;
    return run_flush(h, nullptr, min_count, as_stream(stream), h->bufs.sync);
}

static StepArgs step_args(replay_handle *h, const void *q, const void *k, const void *v, const float *dt,
                          const float *a, float *y, int32_t flush_at, int32_t W, int32_t *sync) {
    const replay_config &c = h->cfg;
    StepArgs sa;
    sa.ring_q = h->bufs.ring_q;
    sa.ring_k = h->bufs.ring_k;
    sa.ring_v = h->bufs.ring_v;
    sa.ring_dt = h->bufs.ring_dt;
    sa.ring_a = h->bufs.ring_a;
    sa.pos = h->bufs.pos;
    sa.base = h->bufs.base;
    sa.err = h->bufs.err;
    sa.sync = sync;
    sa.S = h->bufs.s_master;
    sa.q = q;
    sa.k = k;
    sa.v = v;
    sa.dt = dt;
    sa.a = a;
    sa.y = y;
    sa.B = c.batch;
    sa.H = c.heads;
    sa.G = c.groups;
    sa.L = c.ring_len;
    sa.flush_at = flush_at;
    sa.io_bf16 = c.io_dtype == REPLAY_BF16;
    sa.W = W;
    sa.copy = h->bufs.s_copy;
    sa.copy_scale = h->bufs.s_scale;
    sa.copy_st = c.read_copy == REPLAY_NONE ? -1 : state_kind(c.read_copy);
    sa.n_reject = nullptr;
    return sa;
}

// One standard decode step with the arrival counters at `sync`.
static replay_status step_impl(replay_handle *h, const void *q, const void *k, const void *v, const float *dt,
                               const float *a, float *y, int32_t flush_at, hipStream_t s, int32_t *sync) {
    const replay_config &c = h->cfg;
    note_capture(h, s);
    if (c.rule == REPLAY_RULE_GATED_DELTA) {
        // the gated delta rule: append, the output-only route, the fold if due
        replay_status st = append_impl(h, 1, q, k, v, dt, a, s, sync);
        if (st == REPLAY_OK) st = run_verify(h, 1, y, s);
        if (st != REPLAY_OK) return st;
        return run_flush(h, nullptr, flush_at, s, sync);
    }
    const StepArgs sa = step_args(h, q, k, v, dt, a, y, flush_at, 1, sync);
    if (c.read_copy != REPLAY_NONE) {
        // copies: append + decode from an e4m3 or FP4 copy in one launch
        // (bf16 io), or the append and decode kernels in turn (a bf16 copy:
        // measured slower in one launch); then the flush kernel
        replay_status st;
        if (c.io_dtype == REPLAY_BF16 && c.read_copy != REPLAY_BF16) {
            st = from_hip(launch_step_copy(c.head_dim, c.state_dim, sa, s));
            if (st == REPLAY_OK)
                h->bound.append(1);
            else
                h->bound.unknown();
        } else {
            st = append_impl(h, 1, q, k, v, dt, a, s, sync);
            if (st == REPLAY_OK) st = run_verify(h, 1, y, s);
        }
        if (st != REPLAY_OK) return st;
        return run_flush(h, nullptr, flush_at, s, sync);
    }
    const hipError_t e = launch_step(c.head_dim, c.state_dim, sa, s);
    if (e != hipSuccess) {
        h->bound.unknown();
        return REPLAY_ERR_HIP;
    }
    h->bound.step(flush_at);
    return REPLAY_OK;
}

static bool step_args_ok(const void *q, const void *k, const void *v, const float *dt, const float *a,
                         const float *y) {
    if (!q || !k || !v || !dt || !a || !y) return false;
    return aligned16(q) && aligned16(k) && aligned16(v) && aligned4(dt) && aligned4(a) && aligned4(y);
}

replay_status replay_step(replay_handle *h, const void *q, const void *k, const void *v, const float *dt,
                          const float *a, float *y, int32_t flush_at, void *stream) {
    if (!h || !h->bufs.sync || !step_args_ok(q, k, v, dt, a, y)) return REPLAY_ERR_INVALID_ARG;
    return step_impl(h, q, k, v, dt, a, y, flush_at, as_stream(stream), h->bufs.sync);
}

replay_status replay_step_static(replay_handle *h, const void *q, const void *k, const void *v, const float *dt,
                                 const float *a, float *y, int32_t flush_at, void *stream) {
    if (!h || !step_args_ok(q, k, v, dt, a, y)) return REPLAY_ERR_INVALID_ARG;
    if (counter_bytes(h->cfg) > kStaticCounterBytes) return REPLAY_ERR_TOO_LARGE;
    if (!h->static_sync) return REPLAY_ERR_HIP;
    hipStream_t s = as_stream(stream);
    // the array keeps whatever the last call on this GPU left: clear the
    // counters this call uses (a fill kernel, no memset node in a graph)
    if (launch_fill_u32(h->static_sync, 0u, counter_bytes(h->cfg) / sizeof(int32_t), s) != hipSuccess)
        return REPLAY_ERR_HIP;
    return step_impl(h, q, k, v, dt, a, y, flush_at, s, h->static_sync);
}

replay_status replay_step_layers(replay_handle *const *layers, int32_t n, const void *const *q,
                                 const void *const *k, const void *const *v, const float *const *dt,
                                 const float *const *a, float *const *y, int32_t flush_at, void *stream) {
    if (!layers || !q || !k || !v || !dt || !a || !y || n < 1 || n > kMaxStepLayers) return REPLAY_ERR_INVALID_ARG;
    const replay_handle *h0 = layers[0];
    if (!h0) return REPLAY_ERR_INVALID_ARG;
    const replay_config &c0 = h0->cfg;
    for (int i = 0; i < n; ++i) {
        const replay_handle *h = layers[i];
        if (!h || !h->bufs.sync || !step_args_ok(q[i], k[i], v[i], dt[i], a[i], y[i])) return REPLAY_ERR_INVALID_ARG;
        const replay_config &c = h->cfg;
        if (c.batch != c0.batch || c.heads != c0.heads || c.groups != c0.groups || c.head_dim != c0.head_dim ||
            c.state_dim != c0.state_dim || c.ring_len != c0.ring_len || c.io_dtype != c0.io_dtype)
            return REPLAY_ERR_INVALID_ARG;
        if (c.read_copy != REPLAY_NONE || c.rule != REPLAY_RULE_MAMBA2) return REPLAY_ERR_UNSUPPORTED;
        for (int j = 0; j < i; ++j)
            if (layers[j] == h) return REPLAY_ERR_INVALID_ARG;   // one layer twice in one launch would race
    }
    hipStream_t s = as_stream(stream);
    StepLayersArgs la;
    la.n = n;
    for (int i = 0; i < n; ++i) {
        replay_handle *h = layers[i];
        note_capture(h, s);
        la.l[i] = step_args(h, q[i], k[i], v[i], dt[i], a[i], y[i], flush_at, 1, h->bufs.sync);
    }
    hipError_t e = hipSuccess;
    if (step_workgroups_per_layer(c0.head_dim, la.l[0]) <= kLayersOneLaunchMax) {
        e = launch_step_layers(c0.head_dim, c0.state_dim, la, s);
    } else {
        for (int i = 0; i < n && e == hipSuccess; ++i) e = launch_step(c0.head_dim, c0.state_dim, la.l[i], s);
    }
    for (int i = 0; i < n; ++i) {
        if (e != hipSuccess)
            layers[i]->bound.unknown();
        else
            layers[i]->bound.step(flush_at);
    }
    return from_hip(e);
}

// One speculative round, after the rollback n_reject when it is given: in
// the fused kernels the rollback is applied to the pointer they read; else
// the rollback kernel runs first and the round's calls follow.
static replay_status verify_round_impl(replay_handle *h, const int32_t *n_reject, int32_t W, const void *q,
                                       const void *k, const void *v, const float *dt, const float *a, float *y,
                                       int32_t flush_at, void *stream) {
    if (!h || !h->bufs.sync || !step_args_ok(q, k, v, dt, a, y)) return REPLAY_ERR_INVALID_ARG;
    if (n_reject && !aligned4(n_reject)) return REPLAY_ERR_INVALID_ARG;
    const replay_config &c = h->cfg;
    if (W < 1 || W > kMaxWideWindow || W > c.ring_len) return REPLAY_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    note_capture(h, s);
    StepArgs sa = step_args(h, q, k, v, dt, a, y, flush_at, W, h->bufs.sync);
    sa.n_reject = n_reject;
    const bool copy_fused = c.read_copy != REPLAY_NONE && !c.shared_lowp && c.rule == REPLAY_RULE_MAMBA2 &&
                            verify_step_copy_fused(c.head_dim, c.state_dim, sa);
    const bool fused = c.read_copy == REPLAY_NONE && c.rule == REPLAY_RULE_MAMBA2 &&
                       verify_step_fused(c.head_dim, c.state_dim, sa);
    if (copy_fused || fused) {
        // one launch: (rollback,) fold if due, append the drafts, score them;
        // with an e4m3 or FP4 read copy the fold also rewrites the copy
        const hipError_t e = copy_fused ? launch_verify_step_copy(c.head_dim, c.state_dim, sa, s)
                                        : launch_verify_step(c.head_dim, c.state_dim, sa, s);
        if (e != hipSuccess) {
            h->bound.unknown();
            return REPLAY_ERR_HIP;
        }
        if (n_reject) h->bound.rollback();
        h->bound.verify_round(flush_at, W);
        return REPLAY_OK;
    }
    {
        if (n_reject) {
            h->bound.rollback();
            const hipError_t e = launch_rollback(ring_view(h), h->bufs.pos, n_reject, s);
            if (e != hipSuccess) {
                h->bound.unknown();
                return REPLAY_ERR_HIP;
            }
        }
        // the flush, append and verify kernels in turn
        replay_status st = run_flush(h, nullptr, flush_at, s, h->bufs.sync);
        if (st != REPLAY_OK) return st;
        st = append_impl(h, W, q, k, v, dt, a, s, h->bufs.sync);
        if (st != REPLAY_OK) return st;
        return run_verify(h, W, y, s);
    }
}

replay_status replay_verify_step(replay_handle *h, int32_t W, const void *q, const void *k, const void *v,
                                 const float *dt, const float *a, float *y, int32_t flush_at, void *stream) {
    return verify_round_impl(h, nullptr, W, q, k, v, dt, a, y, flush_at, stream);
}

replay_status replay_rollback_verify_step(replay_handle *h, const int32_t *n_reject, int32_t W, const void *q,
                                          const void *k, const void *v, const float *dt, const float *a, float *y,
                                          int32_t flush_at, void *stream) {
    if (!n_reject) return REPLAY_ERR_INVALID_ARG;
    return verify_round_impl(h, n_reject, W, q, k, v, dt, a, y, flush_at, stream);
}

replay_status replay_set_flush_skipping(replay_handle *h, int32_t enable, void *stream) {
    if (!h || (enable != 0 && enable != 1)) return REPLAY_ERR_INVALID_ARG;
    if (!enable) {
        h->untracked = true;
        return REPLAY_OK;
    }
    // rebuild the bounds from the pointers on the device
    hipStream_t s = as_stream(stream);
    const int B = h->cfg.batch;
    int32_t *host = new (std::nothrow) int32_t[2 * (size_t)B];
    if (!host) return REPLAY_ERR_INVALID_ARG;
    hipError_t e = hipMemcpyAsync(host, h->bufs.pos, sizeof(int32_t) * B, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(host + B, h->bufs.base, sizeof(int32_t) * B, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        delete[] host;
        return REPLAY_ERR_HIP;
    }
    const bool ok = h->bound.from_pointers(host, host + B, B);
    delete[] host;
    if (!ok) return REPLAY_ERR_INVALID_ARG;   // pointers outside 0 <= base <= pos, count <= L: stay untracked
    h->untracked = false;
    h->graphed = false;
    return REPLAY_OK;
}

replay_status replay_get_error(replay_handle *h, int32_t *word, int32_t *per_seq, void *stream) {
    if (!h || !word) return REPLAY_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    const int B = h->cfg.batch;
    int32_t *host = new (std::nothrow) int32_t[B + 1];
    if (!host) return REPLAY_ERR_INVALID_ARG;
    hipError_t e = hipMemcpyAsync(host, h->bufs.err, sizeof(int32_t) * (B + 1), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = launch_fill_u32(h->bufs.err, 0u, (size_t)B + 1, s);
    if (e == hipSuccess) {
        *word = host[0];
        if (per_seq) std::memcpy(per_seq, host + 1, sizeof(int32_t) * B);
    }
    delete[] host;
    return from_hip(e);
}

replay_status replay_eager_step(const replay_config *cfg, const float *s_in, float *s_out, const void *q,
                                const void *k, const void *v, const float *dt, const float *a, float *y,
                                void *stream) {
    replay_status st = check_shape(cfg);
    if (st != REPLAY_OK) return st;
    const void *vec_ptrs[] = {s_in, s_out, q, k};
    for (const void *p : vec_ptrs)
        if (!p || !aligned16(p)) return REPLAY_ERR_INVALID_ARG;
    const void *scalar_ptrs[] = {v, dt, a, y};
    for (const void *p : scalar_ptrs)
        if (!p || !aligned4(p)) return REPLAY_ERR_INVALID_ARG;
    EagerArgs ea;
    ea.S_in = s_in;
    ea.S_out = s_out;
    ea.q = q;
    ea.k = k;
    ea.v = v;
    ea.dt = dt;
    ea.a = a;
    ea.y = y;
    ea.B = cfg->batch;
    ea.H = cfg->heads;
    ea.G = cfg->groups;
    ea.io_bf16 = cfg->io_dtype == REPLAY_BF16;
    if (cfg->rule == REPLAY_RULE_GATED_DELTA) {
        GdnFoldArgs g{};
        g.r.B = cfg->batch;
        g.r.H = cfg->heads;
        g.r.G = cfg->groups;
        g.r.L = 1;
        g.r.io_bf16 = ea.io_bf16;
        g.S_in = s_in;
        g.S_out = s_out;
        g.q = q;
        g.k = k;
        g.v = v;
        g.beta = dt;
        g.alpha = a;
        g.y = y;
        return from_hip(launch_gdn_eager(cfg->head_dim, cfg->state_dim, g, as_stream(stream)));
    }
    return from_hip(launch_eager(cfg->head_dim, cfg->state_dim, ea, as_stream(stream)));
}

replay_status replay_eager_select(const replay_config *cfg, const float *snaps, int32_t W,
                                  const int32_t *n_accept, float *s, void *stream) {
    replay_status st = check_shape(cfg);
    if (st != REPLAY_OK) return st;
    if (!snaps || !n_accept || !s || !aligned16(snaps) || !aligned16(s) || W < 1)
        return REPLAY_ERR_INVALID_ARG;
    const size_t per_seq = (size_t)cfg->heads * cfg->head_dim * cfg->state_dim;
    return from_hip(launch_eager_select(snaps, W, n_accept, s, cfg->batch, per_seq, as_stream(stream)));
}

replay_status replay_stream_probe(int32_t mode, const void *src, void *dst, size_t bytes, void *stream) {
    if ((mode != 0 && mode != 1) || !src || !dst || !aligned16(src) || !aligned16(dst) || bytes % 16 != 0)
        return REPLAY_ERR_INVALID_ARG;
    return from_hip(launch_probe(mode, src, dst, bytes, as_stream(stream)));
}

}  // extern "C"
