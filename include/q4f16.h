/*
 * q4f16.h -- C ABI of the q4f16_1 weight-streaming decode library (MI355X, gfx950).
 *
 * The q4f16_1 format (Zero TVM documentation, section "Q4F16 quantization
 * format"): a weight matrix of logical shape [N][K] (N outputs, K inputs) is
 * stored as
 *   words  : uint32 [N][K/8]  -- eight 4-bit codes per word; element k of row n
 *                                is nibble (k % 8) of words[n][k/8], i.e.
 *                                (words[n][k/8] >> 4*(k%8)) & 0xF;
 *   scales : fp16   [N][K/32] -- one scale per group of 32 consecutive weights;
 * and W[n][k] = (code - 7) * scales[n][k/32].  K must be a multiple of 32, so a
 * group is exactly four consecutive words (16 bytes).  The everything-webgpu
 * AI.md format table gives the cost: 16 + 2 = 18 bytes per 32 weights.
 *
 * Conventions for every entry point:
 *  - fp16 values are passed as uint16_t bit patterns (IEEE binary16).
 *  - Every data pointer is DEVICE memory owned by the caller; the library never
 *    frees it and keeps no pointer after the call returns, except where a
 *    function says otherwise.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *    enqueued on it; results are valid once the caller synchronises that stream.
 *    No entry point synchronises the host with the device, allocates or frees
 *    device memory or creates a stream, except q4_step_status (which waits for
 *    the stream to read an error word) and the set-up of a token graph
 *    (q4_tokens_graph_create / _destroy).
 *  - Return value: a q4_status.  Argument errors are detected on the host before
 *    anything is enqueued (no partial execution).  Q4_ERR_DEVICE reports a HIP
 *    error at launch time; faults during execution surface at the caller's
 *    synchronisation.  q4_last_error_detail() gives a text naming the argument and
 *    value (thread-local, valid until the next call on the same thread).
 *  - Outputs are fp16, rounded to nearest even from an fp32 accumulation.  Any
 *    fp32 summation order is a correct result; every variant is deterministic
 *    (the same inputs give bitwise the same outputs, run to run).
 */
#ifndef Q4F16_H
#define Q4F16_H

#include <stddef.h>
#include <stdint.h>

#ifndef Q4_API
#define Q4_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef void* q4_stream_t;

typedef enum q4_status {
  Q4_OK = 0,
  Q4_ERR_NULL = 1,        /* a required pointer is NULL                         */
  Q4_ERR_SHAPE = 2,       /* N < 1, K < 32, K % 32 != 0, M outside [1, 8], ...  */
  Q4_ERR_ALIGN = 3,       /* a pointer is not aligned as documented             */
  Q4_ERR_WORKSPACE = 4,   /* ws NULL or smaller than the size the call needs    */
  Q4_ERR_DEVICE = 5,      /* a HIP call failed (no device, launch failure, ...) */
  Q4_ERR_UNSUPPORTED = 6, /* a size beyond what the kernels handle              */
  Q4_ERR_TIMEOUT = 7      /* a bounded wait inside a persistent kernel ran out  */
} q4_status;

/* Errors follow the everything-webgpu AI.md engine API ("Fail Fast": validate
 * early, throw descriptive errors; an error carries a code, a message and a
 * detail): every entry point returns a q4_status, and the text naming the
 * argument, value or wait is kept per thread. */

/* Name of a status code ("Q4_OK", ...).  Never NULL. */
Q4_API const char* q4_status_str(int status);

/* Detail of the last error on this thread ("" after a successful call), valid
 * until the next call on the same thread: the detail of the everything-webgpu
 * AI.md engine error. */
Q4_API const char* q4_last_error_detail(void);

/* The same text as q4_last_error_detail (everything-webgpu AI.md engine error
 * detail; the name this library used first). */
Q4_API const char* q4_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH (the MLC Model Artifact
 * Manifest page: a compiled library carries its contract's version, and a reader
 * rejects what it does not know). */
Q4_API int q4_version(void);

/* ------------------------------------------------------------------ codec -- */

/* q4_pack: codes uint8 [N][K] (device) -> words uint32 [N][K/8] (device).
 * Word j of row n = OR over i < 8 of (codes[n][8j+i] & 0xF) << 4i (Zero TVM
 * documentation, "Q4F16 quantization format": nibble i is (w >> 4i) & 0xF).
 * Codes above 15 are reduced to their low nibble.  Requires N >= 1, K >= 32,
 * K % 32 == 0; words 16-byte aligned; codes any alignment.  Bit-exact. */
Q4_API int q4_pack(const uint8_t* codes, uint32_t* words, int64_t N, int64_t K, q4_stream_t stream);

/* q4_unpack: the inverse of q4_pack, words [N][K/8] -> codes [N][K] (each 0..15):
 * code k of row n is (words[n][k/8] >> 4*(k%8)) & 0xF (Zero TVM documentation,
 * "Q4F16 quantization format").  Same shape and alignment rules. */
Q4_API int q4_unpack(const uint32_t* words, uint8_t* codes, int64_t N, int64_t K, q4_stream_t stream);

/* ------------------------------------------------------------------- GEMV -- */

/* q4_gemv: y[n] = fp16( sum_k (q[n][k] - 7) * scales[n][k/32] * x[k] ), n < N,
 * with fp32 accumulation (Zero TVM documentation, "Decode loop": the int4 matmul
 * of every projection and the LM head; "Q4F16 quantization format" for the
 * weights).  x: fp16 [K]; y: fp16 [N].  Chooses single-pass or split-K from the
 * shape and the device; the split-K variant needs a workspace of
 * q4_workspace_bytes(1, N, K) bytes (0 means none: ws may be NULL).
 * Alignment: words, x and ws 16 bytes; scales and y 2 bytes.  y must not
 * overlap any input. */
Q4_API int q4_gemv(const uint32_t* words, const uint16_t* scales, const uint16_t* x, uint16_t* y,
            int64_t N, int64_t K, void* ws, size_t ws_bytes, q4_stream_t stream);

/* q4_gemv_splitk: the same product (Zero TVM documentation, "Decode loop") with
 * an explicit number of K slices.
 * splits == 1 is the single-pass kernel (ws unused).  splits > 1 runs a first
 * pass writing fp32 partials part[s][n] over slice s of the K groups (groups are
 * divided as evenly as possible, each slice non-empty) into ws, then a second
 * pass y[n] = fp16(sum over s ascending of part[s][n]).  1 <= splits <= K/32
 * and splits <= 64; ws needs q4_splitk_workspace_bytes(1, N, splits) bytes. */
Q4_API int q4_gemv_splitk(const uint32_t* words, const uint16_t* scales, const uint16_t* x,
                   uint16_t* y, int64_t N, int64_t K, int64_t splits, void* ws,
                   size_t ws_bytes, q4_stream_t stream);

/* q4_gemv_batched: Y[m][n] = fp16( sum_k W[n][k] * X[m][k] ) for m < M <= 8,
 * the weights read once for all M rows (small-M decode: several tokens or
 * sequences share one pass over the weights, as the Splash page's draft cycles
 * of eight rows do).  X: fp16 [M][K] row-major; Y: fp16 [M][N] row-major.
 * Workspace: q4_workspace_bytes(M, N, K).  M == 1 is q4_gemv. */
Q4_API int q4_gemv_batched(const uint32_t* words, const uint16_t* scales, const uint16_t* X,
                    uint16_t* Y, int64_t M, int64_t N, int64_t K, void* ws,
                    size_t ws_bytes, q4_stream_t stream);

/* Workspace bytes q4_gemv (M == 1) or q4_gemv_batched (M > 1) needs for this
 * shape on the current device (0 = none), computed from the shapes as the MLC
 * Model Artifact Manifest page computes its sizes.  Returns 0 for an invalid
 * shape. */
Q4_API size_t q4_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Workspace bytes of q4_gemv_splitk (M == 1) with `splits` slices: 4 * splits *
 * M * N, from the shapes (MLC Model Artifact Manifest: sizes from shapes). */
Q4_API size_t q4_splitk_workspace_bytes(int64_t M, int64_t N, int64_t splits);

/* Size of the device array in which q4_gemv_batched_noalloc keeps its split-K
 * partials: 4 MiB, one copy per GPU the library runs on, held until the process
 * ends. */
#define Q4_NOALLOC_SCRATCH_BYTES (4 * 1024 * 1024)

/* q4_gemv_batched_noalloc: q4_gemv_batched (M == 1: q4_gemv) for callers that
 * cannot allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments without the workspace:
 * the split-K partials go to a library-owned static device array of
 * Q4_NOALLOC_SCRATCH_BYTES bytes, so the call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).  The caller still owns X, Y and the
 * weights.  Results are bitwise those of q4_gemv_batched with a workspace.
 * A shape whose split-K plan needs more than Q4_NOALLOC_SCRATCH_BYTES
 * (q4_workspace_bytes(M, N, K) > Q4_NOALLOC_SCRATCH_BYTES) is rejected with
 * Q4_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (on different streams,
 * or from several threads without ordering) race on it and may give wrong
 * results; calls ordered on one stream are safe.  The array needs no clearing:
 * every partial a call reads was written by that call. */
Q4_API int q4_gemv_batched_noalloc(const uint32_t* words, const uint16_t* scales,
                                   const uint16_t* X, uint16_t* Y, int64_t M, int64_t N,
                                   int64_t K, q4_stream_t stream);

/* ------------------------------------------------------------ decode step -- */

/* How a descriptor's GEMV input is formed from the memory at x. */
/* x is the input itself: fp16 [M][K]. */
#define Q4_X_PLAIN 0u
/* x is fp16 [M][2K], the output of a gate/up projection: gate = x[m][0 .. K),
 * up = x[m][K .. 2K); the GEMV input is h[m][k] = fp16(silu(gate[m][k]) *
 * up[m][k]) with silu(g) = g / (1 + exp(-g)), formed in fp32 and rounded to
 * nearest even -- the step between the gate/up and down projections of the
 * decode loop's feed-forward block (Zero TVM documentation, "Decode loop": gate,
 * up, SiLU, multiply and down are one fused FFN).  h is never written to memory
 * by the persistent kernel; it equals what q4_silu_mul writes (or differs from
 * the exactly rounded value by at most one fp16 unit in the last place). */
#define Q4_X_SILU_MUL 1u

/* One GEMV of a decode step: y = W h(x) (or Y = W h(X) for M rows), h per x_op.
 * y/Y: fp16 [M][N].  format (the variants are defined below): 0 for q4f16_1
 * (words [N][K/8], 16-byte aligned); Q4_FMT_Q3F16_1 (everything-webgpu AI.md,
 * "Which quantization to recompile with": words [N][3K/32], 4-byte aligned, a
 * group's three words one 96-bit value, weight = (q - 3) * s); or the MLX affine
 * format Q4_FMT_AF4_G64 (Splash docs/models.md, "MLX targets": words as q4f16_1,
 * bf16 scales and biases [N][K/64], weight = s * q + b; K % 64 == 0) or its fp16
 * variant Q4_FMT_AF4_G64_F16.  Every format but q4f16_1 is accepted at M = 1 only
 * (Q4_ERR_UNSUPPORTED otherwise); a list may mix them.  biases: the affine
 * formats' [N][K/64] biases (2-byte aligned), NULL for every other format. */
typedef struct q4_layer {
  const uint32_t* words;   /* [N][K/8] (q4f16_1, affine) or [N][3K/32] (q3f16_1) */
  const uint16_t* scales;  /* [N][K/32], or [N][K/64] (affine) */
  const uint16_t* x;       /* [M][K], or [M][2K] with Q4_X_SILU_MUL */
  uint16_t* y;             /* [M][N]    */
  int64_t N;
  int64_t K;
  uint32_t x_op;           /* Q4_X_PLAIN or Q4_X_SILU_MUL */
  uint32_t format;         /* 0 (q4f16_1), Q4_FMT_Q3F16_1, Q4_FMT_AF4_G64, Q4_FMT_AF4_G64_F16 */
  const uint16_t* biases;  /* affine formats: [N][K/64]; NULL otherwise */
} q4_layer;

/* Run every descriptor as its own kernel launch, in list order on the stream. */
#define Q4_STEP_LAUNCH_EACH 0x1u
/* Treat every descriptor as dependent on the one before it: descriptor k reads
 * its x only after descriptor k - 1 is complete (a chain of GEMVs, each feeding
 * the next, as the projections of a decode step do through the operations
 * between them).  Without this flag a descriptor waits only for earlier
 * descriptors whose y overlaps its x or y, or whose x overlaps its y. */
#define Q4_STEP_ORDERED 0x2u
/* (0x4 and 0x8 are not used.) */
/* Use the persistent kernel even for a list in which more than a quarter of the
 * descriptors wait for another (such lists otherwise run one kernel per
 * descriptor, which is faster for them), or for a one-descriptor list at M = 1. */
#define Q4_STEP_PERSISTENT 0x10u

/* The decode step over a layer list: the GEMVs of layers[0 .. n_layers) in list
 * order, as the Zero TVM decode loop walks the projections of every layer and then
 * the LM head ("Decode loop").  The results are those of calling q4_gemv (M == 1),
 * q4_gemv_batched (M > 1) or, for a format variant, q4_gemv_format on each
 * descriptor in turn, after forming its input per x_op (each within the GEMV
 * tolerance of the oracle; the kernels differ in rounding order); a descriptor's x
 * may lie in an earlier descriptor's y.
 *
 * How a list runs: a list whose rows are at most K = 8192 runs as ONE persistent
 * kernel (M == 1; for 2 <= M <= 8 when every K is a multiple of 128, every scales
 * pointer 8-byte aligned and every x_op Q4_X_PLAIN): the weights of later GEMVs
 * stream while earlier ones finish.  A descriptor waits only for earlier ones it
 * conflicts with (an earlier y overlapping its x or y, an earlier x overlapping
 * its y; with Q4_STEP_ORDERED also its predecessor).  When its only conflict is
 * one earlier descriptor whose y holds all of its x (M == 1), that y is also
 * handed over through the workspace as epoch-tagged values the reader polls;
 * other conflicts wait on per-descriptor completion counters in the workspace.
 * Every wait is bounded (about a second); one that runs out sets the workspace's
 * error word (q4_step_status).  Lists in which more than a quarter of the
 * descriptors wait for another (unless Q4_STEP_PERSISTENT), lists whose conflicts
 * one such wait cannot cover, and all other lists run one kernel per descriptor.
 *
 * Ownership (everything is the caller's): the plan is caller host memory of
 * q4_step_plan_bytes(n_layers) bytes, 8-byte aligned; the workspace is caller
 * device memory of q4_decode_step_workspace_bytes(...) bytes, 16-byte aligned,
 * holding the control block (error word, hand-over epoch, counters), the tagged
 * values, the list's device tables and split-K partials.  The library allocates
 * nothing, frees nothing, keeps no state between calls and creates no stream; the
 * only call that waits for the device is q4_step_status. */

/* Host bytes of the plan of a list of n_layers descriptors (0 if n_layers < 1). */
Q4_API size_t q4_step_plan_bytes(int64_t n_layers);

/* Workspace bytes a plan of this list needs on the current device (0 for an
 * invalid list), from the shapes (MLC Model Artifact Manifest: sizes from
 * shapes).  flags: Q4_STEP_* bits. */
Q4_API size_t q4_decode_step_workspace_bytes(const q4_layer* layers, int64_t n_layers, int64_t M,
                                             uint32_t flags);

/* q4_step_plan_init: set a list up once (the per-token path is q4_step_run), as
 * the Zero TVM decode loop prepares its per-token buffers before the loop
 * ("Decode loop").
 * Validates every descriptor (argument errors return before anything is
 * enqueued), works out the dependencies, the partition of the rows over the
 * workgroups and the launch, and writes them into `plan`; then enqueues on
 * `stream` the writes of the device tables into ws and the clearing of its
 * control block -- small kernels only: no allocation, no copy from host memory,
 * no wait, so the call can be captured in a HIP graph.  `layers` is read during
 * the call only.  The plan records ws: every run of it must pass the same ws, and
 * runs that share a workspace must be ordered on one stream.  A plan stays valid
 * while the descriptors' buffers do. */
Q4_API int q4_step_plan_init(const q4_layer* layers, int64_t n_layers, int64_t M, uint32_t flags,
                             void* plan, size_t plan_bytes, void* ws, size_t ws_bytes,
                             q4_stream_t stream);

/* q4_step_run: one decode step of a planned list (Zero TVM documentation,
 * "Decode loop": every projection of every layer, then the LM head), enqueued
 * on `stream`: the
 * persistent kernel's single launch (or one kernel per descriptor).  Host work is
 * a check of the plan and the launch: no planning, no allocation, no wait. */
Q4_API int q4_step_run(const void* plan, void* ws, size_t ws_bytes, q4_stream_t stream);

/* q4_step_status: wait for `stream`, then read the workspace's error word (the
 * everything-webgpu AI.md engine errors: fail fast with a code and a detail).
 * Q4_OK if no bounded wait inside a persistent kernel has run out since the last
 * check; otherwise Q4_ERR_TIMEOUT, with q4_last_error_detail() naming the wait
 * and the descriptor (the outputs of the step that ran out are not valid), and
 * the word is cleared.  The workspace's counters are left zero either way (every
 * workgroup of the kernel finishes: the waits are bounded), so later runs start
 * clean.  ws: a workspace set up by q4_step_plan_init, or by q4_tokens_plan_init
 * (the whole-token kernel keeps the same error word; the detail then names the
 * stage of the step). */
Q4_API int q4_step_status(void* ws, q4_stream_t stream);

/* q4_decode_step: plan and run a list in one call (Zero TVM documentation,
 * "Decode loop"), with no plan kept: each call
 * redoes q4_step_plan_init's work (the host planning and the writes of the
 * tables into ws) before the run, so it costs a few small kernels more than
 * q4_step_run.  ws: q4_decode_step_workspace_bytes(layers, n_layers, M, 0)
 * bytes.  q4_decode_step_flags takes Q4_STEP_* bits. */
Q4_API int q4_decode_step(const q4_layer* layers, int64_t n_layers, int64_t M, void* ws,
                          size_t ws_bytes, q4_stream_t stream);
Q4_API int q4_decode_step_flags(const q4_layer* layers, int64_t n_layers, int64_t M,
                                uint32_t flags, void* ws, size_t ws_bytes, q4_stream_t stream);

/* q4_silu_mul: out[m][i] = fp16(silu(gu[m][i]) * gu[m][H + i]) for m < M, i < H,
 * with silu(g) = g / (1 + exp(-g)) in fp32, rounded to nearest even (silu(+inf)
 * = +inf, silu(-inf) = -0, NaN propagates): the feed-forward glue between the
 * gate/up and down projections (Zero TVM documentation, "Decode loop").  gu: fp16
 * [M][2H] (gate | up per row); out: fp16 [M][H].  H % 8 == 0; both 16-byte
 * aligned; out must not overlap gu.  M >= 1, M * H < 2^31. */
Q4_API int q4_silu_mul(const uint16_t* gu, uint16_t* out, int64_t M, int64_t H,
                       q4_stream_t stream);

/* ---------------------------------------- the operations around the GEMVs -- */
/* The decode loop's steps between its projections (Zero TVM documentation,
 * "Decode loop"): the token's embedding row, RMSNorm, the residual add with
 * RMSNorm ("addNorm"), the argmax over the LM head's logits.  Rows are
 * independent; every fp16 pointer is 16-byte aligned and K % 8 == 0. */

/* q4_embed_rows: out[m][k] = fp16((q[t][k] - 7) * s[t][k/32]) with t = tokens[m]:
 * row t of a q4f16_1 embedding table (words [N][K/8], scales [N][K/32]).  tokens
 * is DEVICE memory (int32 [M]), read by the kernel, so a captured sequence can
 * take the token an earlier kernel wrote; a token outside [0, N) gives a row of
 * NaN (0x7E00).  Each output is the exact product rounded once. */
Q4_API int q4_embed_rows(const uint32_t* words, const uint16_t* scales, int64_t N, int64_t K,
                         const int32_t* tokens, int64_t M, uint16_t* out, q4_stream_t stream);

/* q4_rmsnorm (Zero TVM documentation, "Decode loop": the norm before each
 * block's projections):
 * out[m][k] = fp16(x[m][k] / sqrt(mean_k x[m][k]^2 + eps) * gamma[k]),
 * the sum of squares in fp32.  x, out: [M][K]; gamma: [K].  out must not overlap
 * x or gamma.  Results are within one fp16 unit in the last place of the
 * exactly computed value. */
Q4_API int q4_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M, int64_t K,
                      uint16_t* out, q4_stream_t stream);

/* q4_add_rmsnorm (Zero TVM documentation, "Decode loop": addNorm):
 * res_out = fp16(res_in + delta) (rounded once), then out =
 * RMSNorm(res_out) * gamma as q4_rmsnorm.  res_out may be res_in itself (in
 * place) but must not otherwise overlap an input; out must not overlap any other
 * argument. */
Q4_API int q4_add_rmsnorm(const uint16_t* delta, const uint16_t* res_in, const uint16_t* gamma,
                          float eps, int64_t M, int64_t K, uint16_t* res_out, uint16_t* out,
                          q4_stream_t stream);

/* q4_gemv_norm: the residual add, RMSNorm and the GEMV it feeds, in one kernel
 * (Zero TVM documentation, "Decode loop": addNorm followed by the next
 * projection).  h = fp16(res_in + delta) (rounded once; delta NULL: h = res_in),
 * written to res_out unless that is NULL.  flags:
 *   Q4_NORM_GLU: W is [2N][K] (gate rows, then up rows) and
 *     y[i] = fp16(silu(fp16(gate_i)) * fp16(up_i)) for i < N; else W is [N][K] and
 *     y[n] = fp16(...) for n < N.
 *   Q4_NORM_EXACT: the GEMV stages RMSNorm(h) * gamma formed as q4_rmsnorm forms
 *     it (the same sum of squares, order and rounding), so y is bitwise q4_add_rmsnorm
 *     followed by q4_gemv (and q4_silu_mul) wherever q4_gemv runs as one K slice
 *     (q4_workspace_bytes(1, rows, K) == 0); K <= 27296 (192 bytes of LDS per 32
 *     inputs; the decode step's default).
 *   otherwise (factored; the GEMV of Q4_MODEL_FACTORED_NORM): the GEMV stages
 *     fp16(h * gamma), forms sum(h^2) in fp32 alongside, and scales each fp32 output
 *     by 1 / sqrt(sum(h^2) / K + eps) before rounding it: no reduction precedes the
 *     staging.  It differs from the unfolded step by where the normalised input is
 *     rounded (there after the scaling, here before it): within the GEMV tolerance
 *     plus one fp16 rounding of each input term, not bitwise.  K <= 81920.
 * res_in, delta, gamma, res_out: fp16 [K], 16-byte aligned; res_out must not
 * overlap anything else; y must not overlap an input.  K % 32 == 0; a K beyond the
 * limit is Q4_ERR_UNSUPPORTED. */
#define Q4_NORM_GLU 0x1u
#define Q4_NORM_EXACT 0x2u
Q4_API int q4_gemv_norm(const uint32_t* words, const uint16_t* scales, const uint16_t* res_in,
                        const uint16_t* delta, const uint16_t* gamma, float eps,
                        uint16_t* res_out, uint16_t* y, int64_t N, int64_t K, uint32_t flags,
                        q4_stream_t stream);

/* q4_argmax (Zero TVM documentation, "Decode loop": greedy sampling of the next
 * token): out[m] = the index of the largest value of x[m][0 .. N) (fp16); ties
 * go to the lowest index; NaN entries are skipped (a row of NaN gives 0).  out:
 * int32 [M], device memory.  x 2-byte aligned. */
Q4_API int q4_argmax(const uint16_t* x, int64_t M, int64_t N, int32_t* out, q4_stream_t stream);

/* ------------------------------------------------------ format variants -- */
/* Formats beside q4f16_1 (everything-webgpu AI.md, "Which quantization to
 * recompile with": q3f16_1 at 14 bytes and q4f32_1 at 20 bytes per 32 weights;
 * Zero TVM documentation: MLX affine checkpoints, w = s * q + b in groups of 64;
 * Splash docs/models.md, "MLX targets": the affine scale and bias are the
 * group's bf16 .scales and .biases, the codes packed little-endian in 32-bit
 * words):
 *   Q4_FMT_Q3F16_1: words uint32 [N][3K/32] -- a group of 32 weights is three
 *     consecutive words read as one little-endian 96-bit value, code i in its
 *     bits [3i, 3i + 3); scales fp16 [N][K/32]; weight = (q - 3) * s; x, y fp16.
 *   Q4_FMT_Q4F32_1: words as q4f16_1 ([N][K/8]); scales fp32 [N][K/32];
 *     weight = (q - 7) * s; x, y fp32.
 *   Q4_FMT_AF4_G64: words as q4f16_1; scales and biases bf16 [N][K/64];
 *     weight = s * q + b; x, y fp16.  K % 64 == 0.  (The pages' format.)
 *   Q4_FMT_AF4_G64_F16: the same with fp16 scales and biases (an extra variant,
 *     not a format the pages describe).
 * The 3-bit packing and its zero point (2^(bits - 1) - 1, as q4f16_1's 7) are
 * our reading: the table gives only the bytes per group. */
#define Q4_FMT_Q3F16_1 1u
#define Q4_FMT_Q4F32_1 2u
#define Q4_FMT_AF4_G64 3u
#define Q4_FMT_AF4_G64_F16 4u
/* OR-ed into the format of a q3f16_1 call: load the words as 16-byte pieces
 * through an LDS stage, or as one 12-byte load per group.  Without either, the
 * first is taken when each team of lanes has at least eight trips of its rows
 * (large matrices), the second otherwise.  Results are bitwise the same. */
#define Q4_FMT_LOAD_STAGED 0x100u
#define Q4_FMT_LOAD_DIRECT 0x200u

/* q4_gemv_format: y = W x (M = 1) for a format variant (one of Q4_FMT_*, for
 * q3f16_1 optionally with one Q4_FMT_LOAD_* bit), fp32 accumulation, fp16
 * outputs rounded to nearest even (fp32 outputs for Q4_FMT_Q4F32_1).  biases: NULL
 * except for the two affine formats.  32 <= K <= 32768, K % 32 == 0 (% 64 for affine);
 * words and x 16-byte aligned (words 4-byte for q3f16_1), the rest aligned to
 * their element;
 * y must not overlap an input. */
Q4_API int q4_gemv_format(uint32_t format, const uint32_t* words, const void* scales,
                          const uint16_t* biases, const void* x, void* y, int64_t N, int64_t K,
                          q4_stream_t stream);

/* Bytes of words, scales and biases of an N x K matrix in a format (0 = q4f16_1):
 * the bytes per 32 weights of the everything-webgpu AI.md quantization table
 * (q4f16_1 18, q3f16_1 14, q4f32_1 20) and 36 per 64 for the affine formats;
 * 0 for an invalid format or shape. */
Q4_API size_t q4_format_weight_bytes(uint32_t format, int64_t N, int64_t K);

/* -------------------------------------------------------- decode tokens -- */
/* The decode loop end to end (Zero TVM documentation, "Decode loop"), weights
 * only: the token's embedding row; an RMSNorm; per block qkv, attention, o, the
 * residual add with RMSNorm, gate/up, SiLU-multiply, down, the residual add with
 * RMSNorm; the LM head; the argmax.  Attention runs at a single position: the
 * token attends only to itself, the softmax over its one score is 1, and the
 * attention output is the token's own value vector -- the last D values of the
 * qkv output (rotary embedding leaves values unchanged).  There is no KV cache.
 * The RMSNorm after each block's residual add uses the next block's attention
 * norm (the final norm after the last block). */

/* One q4f16_1 weight in device memory: words [N][K/8], scales [N][K/32]. */
typedef struct q4_weight {
  const uint32_t* words;
  const uint16_t* scales;
  int64_t N;
  int64_t K;
} q4_weight;

typedef struct q4_block {
  q4_weight qkv;                /* [3D][D]: q, k, v */
  q4_weight o;                  /* [D][D]  */
  q4_weight gate_up;            /* [2F][D]: gate rows, then up rows */
  q4_weight down;               /* [D][F]  */
  const uint16_t* attn_norm;    /* fp16 [D]: RMSNorm weight before qkv */
  const uint16_t* ffn_norm;     /* fp16 [D]: RMSNorm weight before gate/up */
} q4_block;

typedef struct q4_model {
  int64_t n_blocks;             /* >= 0 */
  int64_t D, F, V;              /* hidden size, FFN size, vocabulary (D, F % 32 == 0) */
  q4_weight embed;              /* [V][D] embedding table */
  const q4_block* blocks;       /* HOST array of n_blocks (read during the call) */
  const uint16_t* final_norm;   /* fp16 [D] */
  q4_weight lm_head;            /* [V][D] */
  float eps;                    /* RMSNorm epsilon, >= 0 */
  uint32_t options;             /* 0 or Q4_MODEL_FACTORED_NORM */
} q4_model;

/* Fold every residual add + RMSNorm into the GEMV it feeds: that GEMV stages
 * h * gamma (h = residual + the previous projection's output), forms sum(h^2)
 * alongside, and scales its outputs by 1 / sqrt(sum(h^2) / D + eps) -- the same
 * normalisation with the scalar applied after the product instead of before it,
 * so no reduction precedes the GEMV and the step has no separate norm kernels.
 * The rounding differs from the unfolded step (there the normalised vector is
 * rounded to fp16 before the product): results agree with it within fp16
 * rounding per stage, not bit for bit. */
#define Q4_MODEL_FACTORED_NORM 0x1u

/* Workspace bytes q4_decode_token and q4_decode_tokens need for this model
 * (activations, split-K partials, token bookkeeping); 0 if the model is invalid. */
Q4_API size_t q4_decode_token_workspace_bytes(const q4_model* model);

/* q4_decode_token: one decode step (Zero TVM documentation, "Decode loop":
 * decodeToken) for token_in[0] (DEVICE int32); writes the
 * argmax of the logits to token_out[0] (DEVICE int32) and, if logits is not NULL,
 * the logits (DEVICE fp16 [V]).  One kernel per operation, enqueued on `stream`.
 * ws: q4_decode_token_workspace_bytes(model), 16-byte aligned. */
Q4_API int q4_decode_token(const q4_model* model, const int32_t* token_in, int32_t* token_out,
                           uint16_t* logits, void* ws, size_t ws_bytes, q4_stream_t stream);

/* q4_decode_tokens: `steps` decode steps back to back with no host
 * synchronisation, each step's argmax the next step's token: tokens is DEVICE
 * int32 [steps + 1]; step i reads tokens[i] and writes tokens[i + 1] (the Zero
 * TVM decode loop's per-token dispatches, and the everything-webgpu page's
 * multi-step decode: several tokens per host submission).  Every step's kernels
 * are enqueued on `stream`; the results are those of `steps` calls of
 * q4_decode_token.  ws as for q4_decode_token; calls sharing it must be ordered
 * on one stream. */
Q4_API int q4_decode_tokens(const q4_model* model, int32_t* tokens, int64_t steps, void* ws,
                            size_t ws_bytes, q4_stream_t stream);

/* A decode step captured once as a HIP graph and replayed per token (the same
 * multi-step decode with one graph launch per token instead of ~200 kernel
 * launches).  The handle is the caller's: created and destroyed explicitly; the
 * library keeps no graph of its own. */
typedef struct q4_tokens_graph q4_tokens_graph;

/* q4_tokens_graph_create: set-up of the everything-webgpu page's multi-step
 * decode ("Multi-step decoding": several tokens per host submission).  Captures
 * one step (read tokens[counter], the
 * step, write tokens[counter + 1]) on `stream` -- a stream the caller created;
 * the null stream cannot be captured -- and instantiates it.  The graph holds
 * the model's pointers, `tokens` and `ws`: they must stay valid and unchanged
 * while the handle lives.  Allocates the handle (host) and, inside the HIP
 * runtime, the graph; nothing is enqueued. */
Q4_API int q4_tokens_graph_create(const q4_model* model, int32_t* tokens, void* ws,
                                  size_t ws_bytes, q4_stream_t stream, q4_tokens_graph** out);

/* q4_tokens_graph_run: `steps` decode steps (everything-webgpu AI.md,
 * "Multi-step decoding") as q4_decode_tokens computes them:
 * one kernel resets the step counter, then the graph is launched `steps` times
 * on `stream`.  No allocation, no wait. */
Q4_API int q4_tokens_graph_run(q4_tokens_graph* graph, int64_t steps, q4_stream_t stream);

/* q4_tokens_graph_destroy: free the handle and its graph (the everything-webgpu
 * page's multi-step decode, torn down by its owner).  The library does not
 * wait: the caller synchronises the streams the graph was launched on first.
 * NULL is accepted. */
Q4_API int q4_tokens_graph_destroy(q4_tokens_graph* graph);

/* --------------------------------------------------- whole-token kernel -- */
/* The decode loop of q4_decode_tokens with every stage of every step in ONE
 * persistent kernel launch (Zero TVM documentation, "Decode loop"; the
 * everything-webgpu page's host-side lever of submitting a whole token in one
 * command, "Multi-step decoding", taken to one kernel for several tokens): per
 * block qkv, o on the value part, gate/up with the SiLU-multiply, down, then the
 * LM head and the greedy argmax, the next step's embedding row from that
 * argmax.  Each workgroup keeps its own copy of the residual stream; the
 * projections hand their outputs to the next one as epoch-tagged pairs in the
 * workspace, and the weights of the next projection stream while the current
 * one waits for its input.  It always computes the factored-norm step
 * (Q4_MODEL_FACTORED_NORM; model->options is not consulted): results agree with
 * q4_decode_tokens on that model within fp32 rounding of the dot products (a
 * different summation order), not bit for bit; the token is the argmax of the
 * logits it computes (ties to the lowest index, NaN skipped).  Shapes: D <= 4096,
 * F <= 8192, V <= 2^24, n_blocks <= 4096.  A plan is made once per model and
 * workspace, then runs launch only. */

/* Bytes of the host plan buffer q4_tokens_plan_init fills (the everything-webgpu
 * page's multi-step decode, planned once). */
Q4_API size_t q4_tokens_plan_bytes(void);

/* Workspace bytes of the whole-token kernel for this model (Zero TVM
 * documentation, "Decode loop": every stage's activations; here the control
 * block, the stage table, the tagged pairs of every projection, q/k rows and
 * logits); 0 if the model is invalid or outside the shape limits. */
Q4_API size_t q4_tokens_workspace_bytes(const q4_model* model);

/* q4_tokens_plan_init: the set-up of the everything-webgpu page's multi-step
 * decode ("Multi-step decoding") for the whole-token kernel.  Plans the stages
 * into `plan` (host memory, q4_tokens_plan_bytes(), 8-byte aligned) and
 * enqueues on `stream` the writes of the stage table and the zeroing of the
 * control block and tagged pairs in `ws` (device memory,
 * q4_tokens_workspace_bytes(model), 256-byte aligned).  The plan holds the
 * model's pointers and ws: they must stay valid and unchanged while it is used.
 * No allocation, no wait. */
Q4_API int q4_tokens_plan_init(const q4_model* model, void* plan, size_t plan_bytes, void* ws,
                               size_t ws_bytes, q4_stream_t stream);

/* q4_tokens_run: `steps` decode steps (Zero TVM documentation, "Decode loop";
 * everything-webgpu AI.md, "Multi-step decoding"): tokens is DEVICE int32
 * [steps + 1]; step i reads tokens[i] (i = 0) or the previous step's argmax and
 * writes tokens[i + 1].  logits: DEVICE fp16 [V] receiving every step's logits
 * (the last one's remain), or NULL (they stay in the workspace).  One launch per
 * 4096 steps on `stream`; calls sharing a plan must be ordered on one stream.
 * No allocation, no wait; q4_step_status(ws, stream) reports a bounded wait
 * that ran out. */
Q4_API int q4_tokens_run(const void* plan, int32_t* tokens, int64_t steps, uint16_t* logits,
                         q4_stream_t stream);

/* q4_tokens_ws_offset: where the last step's activations stay in the workspace
 * (for inspection and tests of the Zero TVM decode loop's stages): byte offset
 * of Q4_TOKENS_QK (fp16 [2D]: the q and k rows of the last block's qkv),
 * Q4_TOKENS_LOGITS (fp16 [V], when run with logits NULL), or for block `block`
 * the tagged pairs of Q4_TOKENS_V (the value rows of qkv, D values),
 * Q4_TOKENS_O (D), Q4_TOKENS_H (the SiLU-multiply of gate/up, F) or
 * Q4_TOKENS_DOWN (D): 8 bytes per two values, {fp16 lo | fp16 hi << 16,
 * uint32 epoch}.  -1 for an invalid plan, `what` or block. */
#define Q4_TOKENS_QK 0u
#define Q4_TOKENS_V 1u
#define Q4_TOKENS_O 2u
#define Q4_TOKENS_H 3u
#define Q4_TOKENS_DOWN 4u
#define Q4_TOKENS_LOGITS 5u
Q4_API int64_t q4_tokens_ws_offset(const void* plan, uint32_t what, int64_t block);

/* ------------------------------------------------------ measurement aids -- */

/* Streaming-read ceiling probe (the everything-webgpu page measures the same
 * ceiling with a kernel that only streams a large buffer, swept over workgroup
 * counts): every byte of buf[0 .. bytes) is read once with 128-bit loads by
 * `blocks` workgroups of 256 threads (0 = one per compute unit times 8); a
 * value depending on all of them is written to sink[0].  bytes % 16 == 0,
 * buf 16-byte aligned. */
Q4_API int q4_probe_read(const void* buf, size_t bytes, uint32_t* sink, int64_t blocks,
                  q4_stream_t stream);

/* Plain device copy dst[0 .. bytes) = src[0 .. bytes) with 128-bit loads and
 * stores: the reference kernel that calibrates the traffic counters, beside the
 * everything-webgpu page's streaming-read probe ("Why not llama.cpp/Ollama-class").  bytes % 16 == 0,
 * both 16-byte aligned, no overlap. */
Q4_API int q4_probe_copy(const void* src, void* dst, size_t bytes, q4_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4F16_H */
