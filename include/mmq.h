/*
 * mmq.h -- C ABI of libmmq: q8-plane producers, q4_K / q6_K integer-dot
 * matmuls and q4_K / q5_K / q6_K one-token GEMVs for gfx950 (MI355X).
 *
 * The operations follow three pages of the "minfer" CUDA optimisation log:
 *   [r52] "55 · r52 — skip-write mode 2: skipping the f32 intermediate write-out"
 *   [r60] "64 · r60 — the coronation: flipping the verified gate set to default-on"
 *   [d37] "72 · D3-7 — attn_v-q6K MMVQ routing (2b) + rms wide-block / positions memo (2c)"
 *
 * Vocabulary.
 *   q8 plane   -- the block-32 quantisation of an f32 activation matrix
 *                 [n][d]: for every 32 consecutive values of a row, one f32
 *                 scale D = amax/127, 32 int8 codes q = clamp(rint(y/D),
 *                 -127, 127) and one int32 sum S = sum(q) [r52 2.2, 3.2].
 *                 Planes are owned by the context; rows are padded to a
 *                 multiple of MMQ_PLANE_ROWS and padded rows are all zero
 *                 [r52 3.2, the padded-tail zero-fill].
 *   plane key  -- the f32 buffer a plane was quantised from (or, for a
 *                 skip-write producer, the buffer it would have written);
 *                 consumers look planes up by (pointer, n, d) [r52 3.1, d37 A2].
 *   dead key   -- a skip-write producer's output buffer: it was never
 *                 written, so quantising it again, or feeding it to a
 *                 producer as an input, would read garbage; any request that
 *                 would do so is refused [r52 3.1-3.2].  Bytes stay dead
 *                 until the library writes them (a producer's y, a
 *                 consumer's out, an export) or the window ends.
 *   stale key  -- every write the library makes to caller memory drops the
 *                 cached planes whose key bytes it overwrites, so a later
 *                 lookup of those bytes misses and re-quantises.
 *
 * Conventions for every call.
 *   * Pointers named x, w, y, gate, up, a, out are DEVICE pointers on the
 *     context's device (f32, row-major, contiguous, 16-byte aligned).
 *     raw_host in mmq_register_weight is a HOST pointer.
 *   * stream is a hipStream_t (NULL = the legacy default stream).  All device
 *     work is enqueued on it in call order; calls never synchronise except
 *     mmq_register_weight.  One context serves one stream: plane slots are
 *     reused in enqueue order, so concurrent streams on one context race.
 *   * Return value: MMQ_OK or a negative MMQ_E_* status.  Every argument,
 *     shape, type and cache check runs before any launch, so a failing call
 *     enqueues nothing; mmq_last_error() describes the failure.  The
 *     library never aborts the process.
 *   * Not thread-safe per context; distinct contexts may be used from
 *     distinct threads.
 *   * HIP graph capture [r60 2.2]: producers and consumers may be captured
 *     while their stream is being captured.  Nothing is allocated during a
 *     capture: a call whose plane slot would have to grow fails with
 *     MMQ_E_ARG, so make the same calls once before capturing.  Cache
 *     bookkeeping happens when a call is captured, not when the graph is
 *     replayed; a replay rewrites the plane slots its calls used, so call
 *     mmq_cache_clear() after the capture and after each replay before eager
 *     calls look planes up again.  After any capture the context never frees
 *     plane memory before mmq_destroy (a grown slot keeps its old memory), so
 *     a graph stays valid for the context's lifetime; destroying the context
 *     invalidates its graphs.
 */
#ifndef MMQ_H
#define MMQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes --------------------------------------------------- */
#define MMQ_OK            0
#define MMQ_E_ARG        -1   /* null or misaligned pointer, bad flag       */
#define MMQ_E_SHAPE      -2   /* d % 256 != 0, n < 1, shape mismatch        */
#define MMQ_E_TYPE       -3   /* weight type does not fit the call          */
#define MMQ_E_OOM        -4   /* device allocation failed or cap exceeded   */
#define MMQ_E_DEAD_WRITE -5   /* request would quantise a dead key          */
#define MMQ_E_HIP        -6   /* HIP runtime or launch error                */
#define MMQ_E_DEVICE     -7   /* no usable gfx950 device / dry-run context  */

/* ---- weight types (values follow the GGUF type ids) ------------------ */
#define MMQ_Q4_K 12           /* 144-byte superblocks of 256 weights         */
#define MMQ_Q5_K 13           /* 176-byte superblocks of 256 weights (GEMV only) */
#define MMQ_Q6_K 14           /* 210-byte superblocks of 256 weights         */

/* ---- context flags --------------------------------------------------- */
#define MMQ_CTX_SYNC_CHECK 1u /* synchronise + check errors after each launch */
#define MMQ_CTX_DRYRUN     2u /* host bookkeeping only: validation, cache and
                                 statistics run, no device memory is touched
                                 and nothing is launched (host-logic tests)  */

/* ---- registration uses ------------------------------------------------ */
#define MMQ_USE_GEMM 1u       /* prefill matmul (any n)                      */
#define MMQ_USE_GEMV 2u       /* one-token GEMV (and the few-token band)      */
#define MMQ_USE_GEMM_PACKED 4u /* with MMQ_USE_GEMM, q4_K only: the matmul
                                 tiles keep the 4-bit codes (0.72 B per weight
                                 instead of 2.16) and the matmul expands them
                                 in registers; same results, bit for bit,
                                 while partial sums stay normal f32        */

#define MMQ_PLANE_ROWS 32       /* plane rows are padded to this multiple     */
#define MMQ_WRITE_AUTO (-1)     /* write_y: skip when allowed, degrade otherwise */
#define MMQ_FOREIGN_F32 1       /* mmq_register_foreign_consumer kinds */
#define MMQ_FOREIGN_QUANT 2

typedef struct mmq_ctx mmq_ctx;
typedef struct mmq_weight mmq_weight;

typedef struct mmq_stats_t {
    int64_t launches_quant_rms;
    int64_t launches_quant_swiglu;
    int64_t launches_quant_f32;     /* standalone quantise, incl. cache misses */
    int64_t launches_gemm_q4k;
    int64_t launches_gemm_q6k;
    int64_t launches_mmvq_q6k;
    int64_t cache_hits;
    int64_t cache_misses;
    int64_t cache_refusals;         /* MMQ_E_DEAD_WRITE returns               */
    int64_t cache_entries;          /* live table entries now                 */
    int64_t plane_bytes;            /* device bytes held by plane slots       */
    int64_t weight_bytes;           /* device bytes held by registered weights */
    int64_t launches_mmvq_q4k;
    int64_t degraded_writes;        /* skip-write requests that wrote y (mixed consumers) */
    int64_t unfused_fallbacks;      /* MMQ_WRITE_AUTO producers without plane memory      */
    int64_t small_n_gemv;           /* matmul calls served by the few-token GEMV path     */
    int64_t launches_mmvq_q5k;
    int64_t launches_gemv_f32;      /* q6_K GEMVs on an f32 activation (no plane) */
} mmq_stats_t;

/* ---- context (library infrastructure: no passage of the pages defines
 * these calls; they own the device, the plane slots and the error text) --- */

/* Create a context on HIP device `device` (must be gfx950; the device
 * becomes current on the calling thread).  flags: MMQ_CTX_*.  With
 * MMQ_CTX_DRYRUN no device is opened and `device` is ignored.
 * Errors: MMQ_E_ARG (out == NULL, unknown flag), MMQ_E_DEVICE. */
int mmq_create(int device, unsigned flags, mmq_ctx** out);

/* Free every plane slot and the context.  Registered weights stay valid
 * until mmq_weight_free.  NULL is ignored.  Synchronises the device. */
void mmq_destroy(mmq_ctx* ctx);

/* Description of the last failure on the calling thread ("" if none). */
const char* mmq_last_error(void);

/* Cap on the total bytes of plane slots (default: no cap).  A producer or
 * miss quantise that would grow past it returns MMQ_E_OOM. */
int mmq_set_scratch_cap(mmq_ctx* ctx, int64_t bytes);

/* Rows of a plane for n tokens: n rounded up to MMQ_PLANE_ROWS. */
int64_t mmq_plane_rows(int64_t n);

/* ---- registration [r60 3.1: weights are registered before the first
 * forward; the engine keeps registration-time planes of every q4_K/q6_K
 * weight] ---------------------------------------------------------------- */

/* Copy `rows` x `cols` weights of type `type` (raw superblocks, row-major
 * [rows][cols/256], 144, 176 or 210 bytes each) from host memory and repack
 * them into device tiles for the consumers named in `uses` (MMQ_USE_*; 0
 * means every consumer the type supports).  cols % 256 == 0.  raw_host may be
 * freed on return.  Synchronises the device.
 * The default uses: q4_K MMQ_USE_GEMM, q6_K MMQ_USE_GEMM | MMQ_USE_GEMV,
 * q5_K MMQ_USE_GEMV (q5_K has a decode arm only; MMQ_USE_GEMM with q5_K is
 * MMQ_E_TYPE).
 * MMQ_USE_GEMM_PACKED keeps a q4_K weight's matmul tiles as 4-bit codes
 * that the matmul expands in registers [r60 5, the "uint4 B-expand" step of
 * the campaign; r60 6 lesson 4 weighs an f16 weight cache against packed
 * weights, memory both ways].  The matmul returns the same bits as from the
 * default f16 tiles, in more time (the expanded operand carries a factor
 * 2^-14 that the stored d takes back, so a superblock's partial sum under
 * 2^-112 or over 2^112 may round differently).  It needs MMQ_USE_GEMM
 * (MMQ_E_ARG otherwise) and a q4_K weight (MMQ_E_TYPE otherwise).
 * Errors: MMQ_E_ARG, MMQ_E_SHAPE, MMQ_E_TYPE (unknown type), MMQ_E_OOM,
 * MMQ_E_HIP. */
int mmq_register_weight(mmq_ctx* ctx, int type, int64_t rows, int64_t cols,
                        const void* raw_host, unsigned uses, mmq_weight** out);

/* Release a weight's device tiles (NULL ignored; synchronises the device).
 * Library infrastructure; no passage defines it. */
void mmq_weight_free(mmq_weight* w);

/* Device bytes held by a registered weight (library infrastructure; the
 * pages count memory both ways [r60 4], this is the registered side). */
int64_t mmq_weight_bytes(const mmq_weight* w);

/* ---- producers [r52 2.2, 3.2; d37 Excerpt C] ----------------------------
 * Each quantises its f32 result in registers into a plane and records the
 * plane under key y.  write_y == 1 also stores y [n][d] (the entry is live);
 * write_y == 0 never touches y (the entry is dead: y is only the key).
 * The degradation ladder [r52 3.1; r60 3.3]: skip-write is honoured only
 * while the context is plane-only (mmq_plane_only); after
 * mmq_register_foreign_consumer, write_y == 0 writes y and the plane
 * (counted in degraded_writes).  write_y == MMQ_WRITE_AUTO skips the write
 * when allowed and, if no plane memory can be had (scratch cap or device
 * memory), falls back to writing y alone with no plane recorded (counted in
 * unfused_fallbacks; returns MMQ_OK) -- every tier is correct, a lower one
 * only costs time.
 * An input that overlaps a dead key (x or w for RMSNorm, gate or up for
 * SwiGLU) is refused with MMQ_E_DEAD_WRITE before any launch.
 * Preconditions: d % 256 == 0, n >= 1; x/gate/up/y 16-byte aligned.
 * Errors: MMQ_E_ARG, MMQ_E_SHAPE, MMQ_E_OOM, MMQ_E_DEAD_WRITE, MMQ_E_HIP. */

/* RMSNorm: y[t][i] = (x[t][i] * s_t) * w[i], s_t = 1/sqrt(mean_i x[t][i]^2 + eps). */
int mmq_quant_rms(mmq_ctx* ctx, const float* x, const float* w, float* y,
                  int64_t n, int64_t d, float eps, int write_y, void* stream);

/* SwiGLU: y = (g / (1 + exp(-g))) * u elementwise over [n][d]. */
int mmq_quant_swiglu(mmq_ctx* ctx, const float* gate, const float* up, float* y,
                     int64_t n, int64_t d, int write_y, void* stream);

/* Standalone quantise of an existing f32 buffer x [n][d]; records key x
 * (live).  Refuses with MMQ_E_DEAD_WRITE if x overlaps a dead key. */
int mmq_quant_f32(mmq_ctx* ctx, const float* x, int64_t n, int64_t d, void* stream);

/* ---- consumers [r60 3.2: int8 matmul over the plane, k32 chunks; q6_K
 * with a rescale per 16-element half; d37 Excerpts A, A2] ------------------
 * A consumer looks up the plane of `a` (key (a, n, cols)).  On a miss it
 * quantises a standalone (as mmq_quant_f32) and records it, unless `a`
 * overlaps a dead key, in which case it returns MMQ_E_DEAD_WRITE.
 * out[t][o] = sum_k D[t][k/32] q[t][k] * w[o][k] for t < n, o < rows,
 * row-major [n][rows] f32, caller-owned; w is the dequantised weight.
 * Writing out drops cached planes keyed in its bytes and revives dead bytes
 * there (the same holds for every consumer below).
 * The small-n band [r60 3.2: the matmul is tuned for n >= 16; d37 2]: on a
 * weight also registered with MMQ_USE_GEMV, the call runs on the dot4 GEMV
 * path (one launch per pass of up to 8 tokens, as many as the LDS holds at
 * this width) when one pass holds the n tokens, or when two passes do and
 * n <= 8 or rows * cols <= 16M (measured against the matmul on MI355X; n is
 * at most 16 either way); otherwise the matmul tiles, with K split across
 * workgroups when the output tiles alone do not fill the device (partials
 * held in the context's scratch, summed in a fixed order).
 * Errors: MMQ_E_ARG, MMQ_E_SHAPE, MMQ_E_TYPE, MMQ_E_DEAD_WRITE, MMQ_E_OOM,
 * MMQ_E_HIP. */
int mmq_gemm_q4k(mmq_ctx* ctx, const mmq_weight* w, const float* a, int64_t n,
                 float* out, void* stream);
int mmq_gemm_q6k(mmq_ctx* ctx, const mmq_weight* w, const float* a, int64_t n,
                 float* out, void* stream);

/* One-token q6_K GEMV (n == 1): out[o] = sum_k D[k/32] q[k] * w[o][k] for
 * o < rows, with (q, D) the plane of a.  a: f32 [cols] device pointer, the
 * plane key (a hit uses the recorded plane; a miss quantises a standalone
 * and records it, unless a overlaps a dead key); out: f32 [rows] device
 * pointer, caller-owned.  w must be a q6_K weight registered with
 * MMQ_USE_GEMV.  Errors: MMQ_E_ARG (null, misaligned or foreign pointer),
 * MMQ_E_TYPE (wrong type or not registered for the GEMV), MMQ_E_SHAPE,
 * MMQ_E_DEAD_WRITE, MMQ_E_OOM (no plane memory on a miss), MMQ_E_HIP. */
int mmvq_q6k(mmq_ctx* ctx, const mmq_weight* w, const float* a, float* out,
             void* stream);

/* ---- allocation-free one-token q6_K GEMV --------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  mmvq_q6k
 * without any allocation: a plane recorded under (a, 1, cols) serves as in
 * mmvq_q6k (a hit); on a miss, a (f32 [cols], written -- a dead key is refused
 * with MMQ_E_DEAD_WRITE) is quantised into a one-token plane held in a device
 * array of the library -- one copy per GPU, resolved when a context is
 * created on that GPU and kept until the process ends -- and nothing is
 * recorded in the cache.  cols <= MMQ_NOALLOC_MAX_COLS, else MMQ_E_SHAPE
 * before any launch.  The call never allocates or frees device memory.
 * Every call on one GPU shares that one array: calls in flight at the same
 * time on one GPU (on different streams, contexts or threads) race on it;
 * calls on one stream are ordered and never do.  The plane row is rewritten
 * whole by every miss, so nothing needs clearing between calls.
 * w, a, out and the other errors as for mmvq_q6k. */
#define MMQ_NOALLOC_MAX_COLS 32768
int mmvq_q6k_noalloc(mmq_ctx* ctx, const mmq_weight* w, const float* a, float* out,
                     void* stream);

/* One-token q4_K GEMV, the sibling decode arm of the same routing
 * [d37 Excerpt B: each K-quant type has its own one-token arm].  Per
 * 32-block: D * (d*sc_j * sum(q_w * q) - dmin*m_j * S).  w must be
 * registered with MMQ_USE_GEMV. */
int mmvq_q4k(mmq_ctx* ctx, const mmq_weight* w, const float* a, float* out,
             void* stream);

/* One-token q5_K GEMV, the third decode arm of the per-type routing
 * [d37 Excerpt B: the Q5_K decode arm].  A q5_K superblock is the q4_K one
 * plus a fifth bit per weight (codes 0..31); per 32-block the term is
 * D * (d*sc_j * sum(q_w * q) - dmin*m_j * S), as for q4_K.  w must be a
 * q5_K weight (registered with MMQ_USE_GEMV, the default for the type);
 * a, out and the errors as for mmvq_q6k. */
int mmvq_q5k(mmq_ctx* ctx, const mmq_weight* w, const float* a, float* out,
             void* stream);

/* One-token q6_K GEMV on the f32 activation itself, with no plane
 * [d37 2b and Excerpt A: below an od*id gate the q6_K decode arm runs a
 * kernel on the f32 activation; above it, the quantised GEMV].
 * out[o] = sum_k w[o][k] * x[k] for o < rows, w the dequantised weight, in
 * f32 arithmetic (the activation is not rounded to q8).  x: f32 [cols],
 * written (a dead key is refused with MMQ_E_DEAD_WRITE); it is neither
 * quantised nor recorded in the cache.  w must be q6_K registered with
 * MMQ_USE_GEMV; cols <= 16384 (MMQ_E_SHAPE otherwise).  Errors as for
 * mmvq_q6k. */
int mmq_gemv_q6k_f32(mmq_ctx* ctx, const mmq_weight* w, const float* x, float* out,
                     void* stream);

/* The routed one-token q6_K decode arm [d37 Excerpt A]: the f32-activation
 * GEMV when rows * cols < MMQ_DECODE_F32_GATE, cols <= 16384, x has no
 * recorded plane and is not a dead key; otherwise mmvq_q6k (which consults
 * the cache and quantises x on a miss).  The gate is the crossover measured
 * on MI355X between the f32 GEMV and a standalone quantise + quantised GEMV
 * (the pages' constants, 24M then 4M, were fitted on their GPU; the 4M also
 * counts on a second consumer sharing the quantise).  A caller whose
 * activation feeds further quantised consumers can call mmvq_q6k directly so
 * that the plane is recorded and shared.  Counted under launches_gemv_f32 or
 * launches_mmvq_q6k. */
#define MMQ_DECODE_F32_GATE 16000000LL
int mmq_decode_q6k(mmq_ctx* ctx, const mmq_weight* w, const float* x, float* out,
                   void* stream);

/* ---- consumer set [r60 3.2-3.3: the registration-time nb_bt_only flag] -- */

/* Declare a consumer outside this library that reads producer outputs as
 * f32 (MMQ_FOREIGN_F32: a 2-D f32 weight's matmul; MMQ_FOREIGN_QUANT: a
 * weight type with no plane path).  Clears the plane-only predicate for the
 * context's lifetime; prints one stderr line the first time.
 * Errors: MMQ_E_ARG. */
int mmq_register_foreign_consumer(mmq_ctx* ctx, int kind);

/* 1 while every consumer reads planes (skip-write allowed), else 0. */
int mmq_plane_only(const mmq_ctx* ctx);

/* ---- window boundary, hooks, statistics ---------------------------------- */

/* Drop every cache entry and dead key: the end of an execution window
 * [d37 Excerpt D, synchronize() clears the cache].  Plane slots are kept
 * for reuse. */
void mmq_cache_clear(mmq_ctx* ctx);

/* Drop the entries recorded under `key` and the dead range a skip-write
 * producer recorded for `key` (all of it that no later write revived), for a
 * buffer about to be reused with new contents inside a window (library
 * infrastructure: the pages only clear the whole cache [d37 D]).  Writes to
 * caller memory that the caller makes itself are invisible to the library:
 * call this before re-using a key buffer.  MMQ_OK even if absent. */
int mmq_cache_invalidate(mmq_ctx* ctx, const void* key);

/* Test hook (library infrastructure; no passage defines it).  Copy the
 * plane recorded under (key, n, d) into caller device buffers in the
 * canonical row-major layout: q int8 [r][d], dq f32 [r][d/32],
 * s int32 [r][d/32], with r = n, or mmq_plane_rows(n) if include_pad.
 * dq and s must be 4-byte aligned.
 * Errors: MMQ_E_ARG (no such plane, null or misaligned buffer), MMQ_E_HIP,
 * MMQ_E_DEVICE (dry run). */
int mmq_plane_export(mmq_ctx* ctx, const void* key, int64_t n, int64_t d,
                     int include_pad, int8_t* q, float* dq, int32_t* s,
                     void* stream);

/* Fill *st with counters since creation (library infrastructure: the
 * launch, hit and refusal counts the pages' checks count [r52 3.2]). */
int mmq_stats(mmq_ctx* ctx, mmq_stats_t* st);

#ifdef __cplusplus
}
#endif
#endif /* MMQ_H */
