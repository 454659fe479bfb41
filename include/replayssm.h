/*
 * replayssm.h -- C ABI of the ReplaySSM decode path for Mamba-2-style SSM
 * layers on AMD Instinct MI355X (gfx950).
 *
 * Method (page "ReplaySSM: Cache SSM Inputs, Not State", arXiv 2610.13778
 * abstract page, Abstract; page "ReplaySSM: Cachear Inputs, No Estado",
 * sections "La solucion", "Los dos caminos", "Como funciona en la practica"):
 * the recurrent state of every (sequence, head) is held as a checkpoint S0
 * plus a ring of the most recent inputs (q, k, v, dt, a).  Outputs are
 * produced without materialising the state,
 *
 *     y_t = abar_t (S0 q_t) + sum_{j<=t} s_{j,t} v_j (k_j . q_t),
 *     abar_t = prod_{m=1..t} a_m,   s_{j,t} = dt_j prod_{m=j+1..t} a_m,
 *
 * with j counting the ring entries since the checkpoint (eq. "Ruta solo
 * salida"; abar and s are not defined on the pages -- this is the reading
 * that equals the eager recurrence S_t = a_t S_{t-1} + dt_t v_t k_t^T,
 * y_t = S_t q_t, eq. "Forma resumen").  A flush folds the ring into the
 * checkpoint once (eq. "Ruta estado y salida"); a speculative rollback only
 * moves the ring pointer back.
 *
 * Shapes: B sequences, H heads, G groups (heads h share the k, q of group
 * floor(h*G/H)), P = head_dim, N = state_dim, L = ring_len.
 * S is stored [P][N] per head, N fastest.
 *
 * Conventions for every call below
 *  - Every tensor pointer is HIP device memory owned by the caller; the
 *    library never allocates or frees device memory.  A handle borrows the
 *    buffers given to replay_init: they must outlive it.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call that
 *    enqueues work is asynchronous on that stream and performs no host
 *    synchronisation, except replay_get_error, replay_destroy and
 *    replay_set_flush_skipping(enable = 1), which synchronise the given stream.
 *  - Argument problems the host can see (NULL pointer, a misaligned pointer,
 *    a size outside the compiled specialisations, W out of range) return an
 *    error status and enqueue nothing.  State tiles, ring buffers and the
 *    q / k / v arguments of replay_append must be 16-byte aligned; scalar
 *    arrays (dt, a, y, n_reject, n_accept) 4-byte aligned.
 *  - Per-sequence problems only the device can see set that sequence's bits
 *    in the caller's error buffer and leave that sequence unchanged; read and
 *    clear them with replay_get_error.
 *  - A handle is not thread-safe; distinct handles are independent.  Calls on
 *    one handle must be issued in order on one stream (or ordered by the
 *    caller across streams).
 *  - Graphs: every call that enqueues work, except the synchronising ones
 *    above, may be recorded into a HIP graph by stream capture and
 *    replayed: it allocates nothing, records no memset and does not
 *    synchronise.  Replays read the pointer arguments given at capture, so
 *    new inputs go into those same buffers before each replay.
 *  - Specialisations: (P, N) in {(16,16), (64,64), (64,128), (128,128)},
 *    1 <= L <= 32, 1 <= G <= H with H % G == 0, verify windows 1 <= W <= 8
 *    (up to 16 with bf16 io and a float32, bf16 or e4m3 read; see replay_verify).
 */
#ifndef REPLAYSSM_H
#define REPLAYSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define REPLAY_ABI_VERSION 8

typedef enum {
    REPLAY_OK = 0,
    REPLAY_ERR_INVALID_ARG = 1,   /* NULL / misaligned pointer, bad size, W out of range */
    REPLAY_ERR_UNSUPPORTED = 2,   /* shape or dtype outside the compiled specialisations */
    REPLAY_ERR_HIP = 3,           /* a HIP runtime call failed (launch, copy, sync) */
    REPLAY_ERR_TOO_LARGE = 4      /* replay_step_static: the layer needs more arrival counters
                                     than the library's static array holds */
} replay_status;

/* Per-sequence error bits (device side, sticky until replay_get_error). */
#define REPLAY_SEQERR_RING_OVERFLOW  1  /* append(W) with count + W > L */
#define REPLAY_SEQERR_ROLLBACK_RANGE 2  /* rollback(r) with r < 0 or r > count */
#define REPLAY_SEQERR_TOO_FEW        4  /* decode / verify(W) with count < W; y of that sequence is NaN */
#define REPLAY_SEQERR_POS_OVERFLOW   8  /* append would take pos past 2^31 - 1 */

typedef enum {
    REPLAY_NONE = -1,
    REPLAY_F32 = 0,
    REPLAY_BF16 = 1,
    REPLAY_FP8_E4M3 = 2,          /* OCP E4M3 (e4m3fn), largest finite 448 */
    REPLAY_FP4_E2M1 = 3           /* OCP MX FP4: E2M1 codes (largest 6), 32 consecutive values of a
                                     head's row-major tile sharing one power-of-two scale (E8M0) */
} replay_dtype;

/* The recurrence of the layer (page "ReplaySSM: Cache SSM Inputs, Not State",
   Abstract: the replay serves Mamba-2 and Gated DeltaNet layers).
   MAMBA2:      S_t = a_t S_{t-1} + dt_t v_t k_t^T (page "ReplaySSM: Cachear
                Inputs, No Estado", eq. "Forma resumen").
   GATED_DELTA: S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
                the published gated delta rule (the pages print no equation for
                it); every dt argument and ring slot carries beta_t, every a
                argument and slot alpha_t.  Gated-delta layers take the same
                read copies, shared mode and verify windows (up to min(16, L))
                as Mamba-2 layers, and step stacked layers one call each
                (replay_step_layers: UNSUPPORTED).
   Both: y_t = S_t q_t. */
typedef enum {
    REPLAY_RULE_MAMBA2 = 0,
    REPLAY_RULE_GATED_DELTA = 1
} replay_rule;

typedef struct {
    int32_t batch;        /* B */
    int32_t heads;        /* H */
    int32_t groups;       /* G */
    int32_t head_dim;     /* P */
    int32_t state_dim;    /* N */
    int32_t ring_len;     /* L */
    int32_t io_dtype;     /* REPLAY_F32 or REPLAY_BF16: q, k, v inputs and their ring */
    int32_t read_copy;    /* REPLAY_NONE: outputs read the float32 master checkpoint;
                             REPLAY_BF16 / REPLAY_FP8_E4M3 / REPLAY_FP4_E2M1: outputs read
                             a low-precision copy, rewritten from the new checkpoint at every
                             flush (page "The SSM Layer Nobody Made Fast (Until Now):
                             ReplaySSM Explained", key technical takeaways: FP8/FP4 copies
                             serve the output reads) */
    int32_t shared_lowp;  /* 0: separated precisions (the float32 master takes every flush);
                             1: shared -- the low-precision copy is the only checkpoint and
                             each flush starts from it (needs a read_copy) */
    int32_t rule;         /* the layer's recurrence (replay_rule): REPLAY_RULE_MAMBA2 (0,
                             a zero-initialised config) or REPLAY_RULE_GATED_DELTA */
} replay_config;

/* Device buffers of one layer's decode state.  Sizes in elements; use
   replay_buffer_bytes for bytes.  Every pointer 16-byte aligned. */
typedef struct {
    float   *s_master;  /* [B][H][P][N] f32 checkpoint; NULL iff shared_lowp */
    void    *s_copy;    /* [B][H][P][N] bf16 or e4m3 copy, or [B][H][P*N/2] bytes of FP4 codes
                           (value 2i of a head's tile in the low nibble of byte i, value
                           2i+1 in the high nibble); NULL iff read_copy == NONE */
    void    *s_scale;   /* e4m3: float [B][H], the per-head scale (value = code * scale);
                           FP4: uint8 [B][H][P*N/32], the E8M0 scale of each block of 32
                           (value = code * 2^(byte - 127)); NULL for the other copies */
    void    *ring_q;    /* [B][G][L][N] io dtype */
    void    *ring_k;    /* [B][G][L][N] io dtype */
    void    *ring_v;    /* [B][H][L][P] io dtype */
    float   *ring_dt;   /* [B][L][H] (slot-major: one step's values of a sequence contiguous) */
    float   *ring_a;    /* [B][L][H] */
    int32_t *pos;       /* [B] tokens appended and not rolled back */
    int32_t *base;      /* [B] pos at the last flush; count = pos - base */
    int32_t *err;       /* [B + 1] error bits: err[0] = OR over sequences, err[1 + b] per sequence */
    int32_t *sync;      /* [B][G + 1][32] arrival counters of replay_step,
                           replay_append and the flush, one per 128-byte line (element [b][g][0] per
                           group, [b][G][0] per sequence; the rest is padding so that no
                           two counters share a line); zeroed by replay_init and zero
                           again whenever no call is in flight.  May be NULL: then
                           replay_append, replay_flush, replay_load_checkpoint,
                           replay_step and replay_verify_step return
                           REPLAY_ERR_INVALID_ARG for the handle, and replay_step_static
                           steps the layer */
} replay_buffers;

typedef struct replay_handle replay_handle;

/* Human-readable name of a status.  Never NULL. */
const char *replay_status_string(replay_status s);

/* REPLAY_ABI_VERSION of the built library. */
int32_t replay_abi_version(void);

/* Bytes needed by each replay_buffers field, in field order (12 entries);
   0 for a field the configuration does not use.  Host only. */
replay_status replay_buffer_bytes(const replay_config *cfg, size_t bytes[12]);

/* Validate `cfg` and `bufs`, create a handle, and enqueue the initial state:
   checkpoint 0 (page "ReplaySSM: Cachear Inputs, No Estado", eq. "Forma
   historia" starts from a zero state), copy 0 with scale 1, pos = base = 0,
   error bits 0.  Ring contents are left as they are (never read before
   being written).  On success *out owns a small host object. */
replay_status replay_init(const replay_config *cfg, const replay_buffers *bufs,
                          void *stream, replay_handle **out);

/* Synchronise `stream` and free the host handle (device buffers untouched). */
replay_status replay_destroy(replay_handle *h, void *stream);

/* Replace every sequence's checkpoint by `s_src` ([B][H][P][N] f32, e.g. the
   state a prefill produced), empty the ring (base = pos) and rewrite the
   low-precision copy from it (page "ReplaySSM: Cachear Inputs, No Estado",
   "Decodificacion estandar": the checkpoint is the state accumulated up to
   the last flush).  In shared mode only the copy is written. */
replay_status replay_load_checkpoint(replay_handle *h, const float *s_src, void *stream);

/* Append W tokens to every sequence's ring (same page, "Decodificacion
   estandar": recent (v, dt, k) go to the buffer; q and a are kept too).
   q, k: [B][W][G][N]; v: [B][W][H][P] (io dtype); dt, a: [B][W][H] f32.
   Token i of sequence b goes to slot (pos[b] + i) mod L; then pos[b] += W.
   Needs count + W <= L per sequence (else RING_OVERFLOW, sequence
   unchanged).  1 <= W <= L. */
replay_status replay_append(replay_handle *h, int32_t W, const void *q, const void *k,
                            const void *v, const float *dt, const float *a, void *stream);

/* Output of the newest token of every sequence by the output-only route
   (same page, section "Los dos caminos", eq. "Ruta solo salida"): reads the
   checkpoint (or its copy) once, writes no state.  y: [B][H][P] f32.
   Needs count >= 1 (else TOO_FEW and y of that sequence is NaN). */
replay_status replay_decode(replay_handle *h, float *y, void *stream);

/* Outputs of the W newest ring entries of every sequence against one read of
   the checkpoint (same page, "Paralelismo": all positions of a speculative
   window read the same checkpoint and buffer, entry j is visible to position
   t only when j <= t; abstract page: output-only verification).
   Position w (0-based) is ring entry t_w = count - W + 1 + w.
   y: [B][W][H][P] f32.  1 <= W <= min(16, L) for every configuration;
   windows from W = 6 on (bf16 io) or W = 9 on (float32 io) take the
   window's S Q^T and ring term on the matrix cores.  Needs count >= W per
   sequence (else TOO_FEW, NaN outputs for that sequence). */
replay_status replay_verify(replay_handle *h, int32_t W, float *y, void *stream);

/* Drop the n_reject[b] newest entries of every sequence by moving the pointer
   back: pos[b] -= n_reject[b] (same page, "Rollback"; page "The SSM Layer
   Nobody Made Fast (Until Now): ReplaySSM Explained", key technical
   takeaways: an O(1) pointer decrement).  n_reject: device int32 [B].
   Needs 0 <= n_reject[b] <= count (else ROLLBACK_RANGE, unchanged). */
replay_status replay_rollback(replay_handle *h, const int32_t *n_reject, void *stream);

/* Fold the ring into the checkpoint for every sequence with
   count >= max(min_count, 1) (same page, "Decodificacion estandar", step 4;
   eq. "Ruta estado y salida"): S0 <- abar_c S0 + sum_j s_{j,c} v_j k_j^T over
   the c = count entries, then base = pos, and the copy (and its per-head
   scale) is rewritten from the new checkpoint.  Other sequences: no-op.
   The handle keeps host-side bounds on every sequence's count from the calls
   that move the pointers; a flush that no sequence can be due for enqueues
   nothing (in the standard schedule, every flush but the one that folds).
   So pos and base must change only through this library's calls, or the
   caller turns the skipping off with replay_set_flush_skipping.  Once a
   call that moves the pointers has been recorded into a HIP graph, replays
   move them without the handle seeing it, and from then on every flush is
   enqueued. */
replay_status replay_flush(replay_handle *h, int32_t min_count, void *stream);

/* One standard decode step for every sequence: append one token, produce its
   output and, where the ring then holds count >= max(flush_at, 1) entries,
   fold it into the checkpoint (page "ReplaySSM: Cachear Inputs, No Estado",
   "Decodificacion estandar": buffer the inputs, output by the output-only
   route, flush when the buffer is full).  The output of a folding step is
   taken from the new checkpoint, y = S_new q (eq. "Ruta estado y salida",
   the route the flush needs), so the checkpoint is read once per step.
   Equivalent to replay_append(W=1); replay_decode; replay_flush(flush_at)
   up to the rounding of that route.  q, k: [B][G][N]; v: [B][H][P] (io
   dtype); dt, a: [B][H] f32; y: [B][H][P] f32.  With a float32 checkpoint
   read (read_copy == NONE) it is one kernel launch.  With an e4m3 or FP4
   copy and bf16 io the append and the output-only decode from the copy are
   one launch (its outputs equal replay_append(1); replay_decode bit for
   bit), followed by the flush kernel; otherwise (a bf16 copy, or float32
   io) the append, decode and flush kernels run in turn.  Errors as for
   replay_append: the sequence is unchanged, and its y is NaN (where the
   kernels run in turn, replay_decode's rules give y). */
replay_status replay_step(replay_handle *h, const void *q, const void *k, const void *v,
                          const float *dt, const float *a, float *y, int32_t flush_at, void *stream);

/* replay_step for n stacked layers of one shape in a single launch (page
   "ReplaySSM: Cachear Inputs, No Estado", "Resultados": decode is served
   under CUDA Graphs, where launch gaps between layers matter; here the
   layers' steps share one grid).  layers: host array of n distinct handles,
   1 <= n <= 16, whose configs agree in every shape field and io dtype, each
   with a float32 checkpoint read (read_copy NONE; else UNSUPPORTED) and its
   `sync` buffer; q, k, v, dt, a, y: host arrays of n device pointers, entry
   i laid out as replay_step's arguments for layer i.  Results equal
   replay_step on each layer in turn, bit for bit (the same kernel code; the
   layers are independent).  Errors as replay_step, per layer.  One launch
   covers all layers while a layer has at most 8192 compute workgroups
   (B * H, doubled for 128-row heads with bf16 io); larger layers are
   stepped by one launch each, which measured faster there. */
replay_status replay_step_layers(replay_handle *const *layers, int32_t n, const void *const *q,
                                 const void *const *k, const void *const *v, const float *const *dt,
                                 const float *const *a, float *const *y, int32_t flush_at, void *stream);

/* replay_step for callers that cannot allocate device memory (code under
   HIP graph capture, serving loops that forbid allocation): the same
   kernels, results equal replay_step's bit for bit, but the arrival counters
   live in a static array inside the library instead of the layer's `sync`
   buffer, which may then be NULL.  The array is 2 MiB per GPU (held by
   every GPU the library runs on until the process ends); a layer needs
   B * (G + 1) * 128 bytes of it, and a larger one returns
   REPLAY_ERR_TOO_LARGE and enqueues nothing (B * (G + 1) <= 16384, e.g.
   B = 1820 at G = 8).  Every call first clears the counters it uses with a
   fill kernel on `stream`; the array is shared by every handle on that GPU,
   so calls of replay_step_static that can overlap on one GPU (other streams,
   other threads) race and must be ordered by the caller.  Allocates
   nothing: no hipMalloc, hipFree or allocating library call. */
replay_status replay_step_static(replay_handle *h, const void *q, const void *k, const void *v,
                                 const float *dt, const float *a, float *y, int32_t flush_at, void *stream);

/* One speculative-verify round for every sequence: where the ring holds
   count >= max(flush_at, 1) entries, fold it into the checkpoint first; then
   append the W drafts and produce their W outputs against one read of the
   checkpoint (page "ReplaySSM: Cachear Inputs, No Estado", section
   "Paralelismo": every draft of the window reads the same checkpoint and
   buffer, entry j visible to draft t when j <= t; "Decodificacion
   estandar", step 4, for the fold; section "Rollback": the caller then
   drops rejected drafts with replay_rollback).  flush_at = L - W + 1 folds
   exactly when the drafts would not fit otherwise.
   Equivalent to replay_flush(flush_at); replay_append(W); replay_verify(W),
   bit for bit.  q, k: [B][W][G][N]; v: [B][W][H][P] (io dtype); dt, a:
   [B][W][H] f32; y: [B][W][H][P] f32, draft w at [b][w].  1 <= W <= min(16, L)
   (windows past 8 as for replay_verify, through the kernels in turn).
   With a float32 checkpoint read, bf16 io, L <= 16 and W <= 8 it is one kernel
   launch that reads each checkpoint once and writes it only where it folds.
   With an e4m3 or FP4 read copy (separated precisions), bf16 io, L <= 16,
   2 <= W <= 5 and (P, N) in {(16,16), (64,64), (64,128)} it is one launch
   too: a sequence that does not fold is scored from the copy, one that folds
   reads the master, writes the new master and copy (and scales) and is
   scored from the new codes (abstract page: output-only verification with a
   low-precision checkpoint serving the outputs).  Otherwise it runs the
   flush, append and verify kernels in turn.  A
   sequence whose drafts do not fit after the fold (count + W > L with
   count < flush_at) or whose pointer would pass 2^31 - 1 gets RING_OVERFLOW
   or POS_OVERFLOW, is left unchanged and its y is NaN (in the single-launch
   case; the calls in turn leave the verify outputs of such a sequence to
   replay_verify's rules). */
replay_status replay_verify_step(replay_handle *h, int32_t W, const void *q, const void *k,
                                 const void *v, const float *dt, const float *a, float *y,
                                 int32_t flush_at, void *stream);

/* The previous round's rollback followed by the next speculative round
   (page "ReplaySSM: Cachear Inputs, No Estado", section "Rollback": the
   rejected drafts are dropped by moving the pointer back; section
   "Paralelismo" for the round): equivalent to replay_rollback(n_reject) then
   replay_verify_step(W, ...), bit for bit, error bits included (an
   out-of-range n_reject[b] flags ROLLBACK_RANGE and leaves that sequence's
   pointer where it was, then the round runs).  n_reject: device int32 [B],
   caller-owned, read before any pointer moves.  Where replay_verify_step is
   one kernel launch, this is the same launch (its ring wavefronts apply the
   rollback to the pointer they read), which spares a serving loop the
   rollback kernel between rounds; elsewhere the rollback kernel runs first.
   The last round's rollback is a plain replay_rollback.  n_reject NULL or
   misaligned: REPLAY_ERR_INVALID_ARG, nothing enqueued. */
replay_status replay_rollback_verify_step(replay_handle *h, const int32_t *n_reject, int32_t W,
                                          const void *q, const void *k, const void *v, const float *dt,
                                          const float *a, float *y, int32_t flush_at, void *stream);

/* The host-side count bounds that let replay_flush skip launches (see
   replay_flush) hold only while pos and base change through this library.
   enable = 0: for engines that move pos or base themselves (a sampler that
   rewinds, a copy of another layer's pointers): from now on every flush is
   enqueued.  Enqueues nothing; may be called at any time.
   enable = 1: synchronise `stream`, read every sequence's pos and base back
   and rebuild the bounds from them, then skip flushes again where no
   sequence can be due (this also ends the "every flush" mode a graph
   capture starts: call it only when no recorded graph that moves these
   pointers will be replayed again).  If some sequence holds pos < 0,
   base < 0 or a count outside 0..L, returns REPLAY_ERR_INVALID_ARG and
   every flush stays enqueued.  Synchronising: not for stream capture. */
replay_status replay_set_flush_skipping(replay_handle *h, int32_t enable, void *stream);

/* Synchronise `stream`, copy the error bits to the host and clear them on the
   device.  *word = OR over sequences; per_seq (may be NULL): host int32 [B]. */
replay_status replay_get_error(replay_handle *h, int32_t *word, int32_t *per_seq, void *stream);

/* Eager baseline step (page "ReplaySSM: Cachear Inputs, No Estado", eq.
   "Forma resumen"; section "El problema": the whole state is read and
   written every token):  S_out = a S_in + dt v k^T,  y = S_out q.
   s_in, s_out: [B][H][P][N] f32 (equal pointers = in place, else they must
   not overlap); q, k: [B][G][N]; v: [B][H][P] (cfg->io_dtype); dt, a:
   [B][H] f32; y: [B][H][P] f32.  Uses only the shape fields of cfg. */
replay_status replay_eager_step(const replay_config *cfg, const float *s_in, float *s_out,
                                const void *q, const void *k, const void *v,
                                const float *dt, const float *a, float *y, void *stream);

/* Eager speculative restore (same page, "Rollback": without the buffer, a
   rejected draft means restoring a full stored state).  snaps: [W][B][H][P][N]
   f32, snapshot w = state after draft w+1; n_accept: device int32 [B] in
   0..W.  For every b with n_accept[b] >= 1: s[b] <- snaps[n_accept[b]-1][b];
   n_accept[b] == 0 leaves s[b].  Values outside 0..W are ignored. */
replay_status replay_eager_select(const replay_config *cfg, const float *snaps, int32_t W,
                                  const int32_t *n_accept, float *s, void *stream);

/* HBM stream probes, the bandwidth ceilings the other kernels are quoted
   against: every workgroup streams one 32 KiB tile with all its loads in
   flight, as the checkpoint stream of decode does.  mode 0: read `bytes`
   from src (dst: 4 * ceil(bytes / 32768) bytes, written only in the
   practically impossible case that a tile's xor equals a fixed constant);
   mode 1: copy `bytes` from src to dst (must not overlap).  bytes must be a
   multiple of 16. */
replay_status replay_stream_probe(int32_t mode, const void *src, void *dst, size_t bytes,
                                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_H */
