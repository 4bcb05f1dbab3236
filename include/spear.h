/*
 * spear.h -- C ABI of libspear: a W4A16 linear layer with a per-token gated
 * Error Compensator (EC), written for AMD Instinct MI355X (gfx950).
 *
 * Sources (page title, then section):
 *   "SPEAR: A System for Post-Quantization Error-Adaptive Recovery Enabling
 *   Efficient Low-Bit LLM Serving"
 *     - authors' abstract (fugumt.com record of arXiv 2606.11244): 4-bit
 *       per-channel weights, ECs modulated by per-token gates, the EC fused
 *       into the low-bit GEMM;
 *     - gist.science technical summary, section 2.1 A: the EC maps x to rank r
 *       with A, gates it per token, maps back with B; the effective weight is
 *       W + alpha B diag(gamma) A;
 *     - same summary, section 2.2 A: phase-aware dispatch -- at decode the EC
 *       is fused into the GEMM epilogue (one kernel), at prefill it runs
 *       semi-fused;
 *     - same summary, section 3.1: per-channel 4-bit quantizers (RTN, GPTQ,
 *       AWQ, OmniQuant) -- the layer takes their codes as given.
 *
 * Computation (all shapes row-major; tokens are rows):
 *   x     [M][K]  bf16 activations
 *   W     [N][K]  4-bit codes u (packed, see spear_pack_w4), per-output-channel
 *                 scale s[N] (fp32) and zero point z[N] (uint8; 8 when NULL)
 *   A     [r][K]  bf16 EC down-projection
 *   B     [N][r]  bf16 EC up-projection (alpha folded in)
 *   w_g   [K]     bf16 gate weights, b fp32 gate bias
 *
 *   z_m   = b + sum_k x[m][k] w_g[k]                  (gate logit, fp64 sum)
 *   g_m   = 1 / (1 + exp(-z_m))                       (fp32)
 *   act_m = hard ? (z_m > log(tau / (1 - tau))) : 1   (a tie skips)
 *   u_m[j] = sum_k A[j][k] x[m][k]                     (EC down-projection)
 *   y[m][n] = s_n sum_k x[m][k] (u[n][k] - z_n)
 *           + act_m g_m sum_j B[n][j] u_m[j]
 *
 * Optional vector gate (the summary's diag(gamma(Ax)), gamma a bottleneck MLP
 * on the rank-r projection): with gate_h > 0 the EC term becomes
 *           act_m g_m alpha sum_j B[n][j] gamma_j(u_m) u_m[j],
 *   gamma(u) = sigmoid(W2 relu(W1 u + c1) + c2),  W1 [h][r], c1 [h],
 *   W2 [r][h], c2 [r] (fp32).  With b = +inf (g = 1) and a soft gate this is
 *   the summary's W + alpha B diag(gamma(Ax)) A.
 *
 * Conventions shared by every entry point:
 *   - Data pointers are DEVICE pointers unless stated otherwise.  The caller
 *     allocates and owns all memory, including the workspace.  The library
 *     never allocates device memory.
 *   - State: the workspace carries state from call to call (launch counters
 *     and tagged partial results, see spear_workspace_init), so it is zeroed
 *     once and then left to the library.  The only other state is the
 *     process-wide wait limit (spear_set_wait_limit) and a per-device cache of
 *     the gfx950 check.
 *   - Every call enqueues work on `stream` (a hipStream_t; NULL is the null
 *     stream) and returns without synchronising.  Faults inside a kernel
 *     surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before any HIP call; a call that
 *     fails validation has enqueued nothing.  A call that makes several
 *     launches and returns SPEAR_E_HIP may have enqueued the launches before
 *     the one that failed; the outputs are then unspecified.
 *   - Entry points may be called from several threads at once.  A workspace
 *     must not be shared by calls that may run concurrently (for example on
 *     two streams).
 */
#ifndef SPEAR_H
#define SPEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEAR_ABI_VERSION 2

typedef uint16_t spear_bf16; /* raw bfloat16 bits */
typedef int32_t spear_status;

#define SPEAR_OK            0
#define SPEAR_E_NULL       -1 /* a required pointer is NULL                      */
#define SPEAR_E_SHAPE      -2 /* a size is out of range (see each entry point)   */
#define SPEAR_E_ALIGN      -3 /* a pointer is not aligned as required            */
#define SPEAR_E_ARG        -4 /* an enum is out of range or tau is NaN           */
#define SPEAR_E_WORKSPACE  -5 /* workspace smaller than spear_w4_linear_workspace_size */
#define SPEAR_E_HIP        -6 /* a HIP runtime call or kernel launch failed      */
#define SPEAR_E_DEVICE     -7 /* the current device is not gfx950                */

/* Code kinds accepted by spear_pack_w4. */
#define SPEAR_CODES_S4 0 /* int8 codes q in [-8, 7]; stored offset-binary u = q + 8, zero point 8 */
#define SPEAR_CODES_U4 1 /* uint8 codes u in [0, 15]; zero point per channel */

/* Output element types of spear_w4_linear. */
#define SPEAR_OUT_BF16 0 /* y rounded to bf16 (round to nearest even) */
#define SPEAR_OUT_F32  1 /* y in fp32 */

/* Kernel-path selection of spear_w4_linear_path. */
#define SPEAR_PATH_AUTO          0 /* decode path for M <= 16, prefill path otherwise   */
#define SPEAR_PATH_DECODE        1 /* M <= 16: one launch, EC fused into the epilogue   */
#define SPEAR_PATH_PREFILL       2 /* any M: EC pre-pass, then the MFMA GEMM whose
                                      epilogue applies the EC.  Tiles are 64 x 64
                                      up to 128 tokens, 256 x 128 above.  With few
                                      output tiles K is split and a second launch
                                      adds the slices.  With 64 x 64 tiles or a K
                                      split, and fewer than 2048 tokens, the
                                      pre-pass runs as the first blocks of the
                                      GEMM's launch                                  */
#define SPEAR_PATH_DECODE_2PASS  3 /* M <= 16: EC pre-pass, then the decode kernel      */
#define SPEAR_PATH_PREFILL_LARGE 4 /* any M: EC pre-pass, then the 256 x 128-tile MFMA
                                      GEMM over whole K (the prefill path's choice
                                      when there are enough tiles)                     */

/* Largest EC rank accepted; the rank must also be a multiple of 8. */
#define SPEAR_MAX_RANK 256
/* Largest hidden width of the optional vector gate's MLP. */
#define SPEAR_MAX_GATE_HIDDEN 64

/* Quantised weights (all device pointers). */
typedef struct spear_w4 {
    const uint8_t *packed; /* [N][K/2] from spear_pack_w4; 16-byte aligned          */
    const float *scales;   /* [N] per-channel scale s_n; 4-byte aligned              */
    const uint8_t *zeros;  /* [N] zero points in [0, 15], or NULL for zero point 8   */
    int64_t N;             /* output channels, >= 1                                   */
    int64_t K;             /* input channels, >= 32 and a multiple of 32              */
} spear_w4;

/* Error compensator and gate (device pointers; the *_out fields are optional). */
typedef struct spear_ec {
    const spear_bf16 *A;      /* [r][K]; 16-byte aligned                            */
    const spear_bf16 *B;      /* [N][r]; 16-byte aligned                            */
    const spear_bf16 *w_gate; /* [K]; 16-byte aligned                               */
    float b;                  /* gate bias (-inf gives g = 0)                       */
    float tau;                /* hard-gate threshold on g; must not be NaN          */
    int32_t hard;             /* 0: every token takes the EC; 1: only z_m > logit(tau) */
    int32_t r;                /* rank, a multiple of 8 in [8, SPEAR_MAX_RANK]       */
    float *g_out;             /* optional [M]: g_m                                  */
    int32_t *idx_out;         /* optional [M]: ascending indices of active tokens   */
    int32_t *n_active_out;    /* optional [1]: number of active tokens              */
    /* Optional vector gate (gate_h == 0: none; the other fields are then unused).
       Source: summary section 2.1 A.  All fp32, 4-byte aligned device pointers. */
    int32_t gate_h;           /* hidden width h, 0 or 1 .. SPEAR_MAX_GATE_HIDDEN     */
    float alpha;              /* scale of the vector-gated EC term                  */
    const float *gate_w1;     /* [h][r]                                             */
    const float *gate_c1;     /* [h]                                                */
    const float *gate_w2;     /* [r][h]                                             */
    const float *gate_c2;     /* [r]                                                */
} spear_ec;

/*
 * spear_pack_w4 -- pack 4-bit codes for spear_w4_linear.
 *   codes     [N][K] int8 (SPEAR_CODES_S4) or uint8 (SPEAR_CODES_U4); 16-byte aligned.
 *   packed    [N][K/2] output, 16-byte aligned: each row is a run of little-endian
 *             32-bit words, word w holding u[n][8w .. 8w+7]; nibble position p
 *             (bits 4p .. 4p+3) holds u[n][8w + perm[p]], perm = (0,2,4,6,1,3,5,7):
 *             byte 0 holds codes 0 and 2 (low, high nibble), byte 1 codes 4 and 6,
 *             byte 2 codes 1 and 3, byte 3 codes 5 and 7 (u = q + 8 for signed
 *             codes).  A shift and a mask then give bf16 pairs in natural order.
 *   bad_codes optional device int32 counter; the number of out-of-range codes is
 *             ADDED to it.  Out-of-range codes are packed as their low 4 bits.
 * Shapes: N >= 1, K >= 32, K % 32 == 0.  Source: the summary's section 3.1
 * (per-channel 4-bit codes from any quantizer); the layout is this library's.
 */
spear_status spear_pack_w4(const void *codes, int32_t code_kind, int64_t N, int64_t K,
                           uint8_t *packed, int32_t *bad_codes, void *stream);

/*
 * spear_gate -- the per-token gate and hard-gate token selection alone.
 *   x [M][K] bf16 (16-byte aligned), w_gate [K] bf16 (16-byte aligned).
 *   g        [M] fp32 output, g_m = sigmoid(z_m).
 *   idx      [M] int32 output; entries [0, n_active) are the active tokens in
 *            ascending order, the rest are left unspecified.
 *   n_active [1] int32 output.
 * Shapes: M >= 0 (M == 0 writes n_active = 0), K >= 32, K % 32 == 0.
 * Sources: abstract (per-token gates); summary section 2.1 A (input-dependent gate).
 */
spear_status spear_gate(const spear_bf16 *x, int64_t M, int64_t K, const spear_bf16 *w_gate,
                        float b, float tau, int32_t hard, float *g, int32_t *idx,
                        int32_t *n_active, void *stream);

/*
 * spear_w4_linear_workspace_size -- bytes of workspace spear_w4_linear needs
 * for these sizes (r = 0 when there is no EC).  Host-only, no HIP call.  The
 * size serves every smaller M with the same N, K and r; it is not monotone in
 * N or K (the GEMM's K split depends on the layer's shape), so a workspace
 * shared by layers of several shapes takes the largest of their sizes.
 */
size_t spear_w4_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r);

/*
 * spear_workspace_init -- zero a workspace before its first use (a workspace
 * allocated zero-filled needs no init).  Between calls the workspace holds
 * library state: a launch counter that every fused decode launch advances (its
 * producers tag the partial results they hand to the epilogues with it) and
 * the tagged partials themselves, so it is zeroed once, not per call, and
 * must not be modified by the caller afterwards.  Tags repeat after 2^32
 * fused launches on one workspace; re-initialise it before that.
 * ws: device pointer, 256-byte aligned; bytes >= 256.
 */
spear_status spear_workspace_init(void *ws, size_t bytes, void *stream);

/*
 * spear_w4_linear -- y = x W^T (dequantised) + gated EC; ec == NULL gives the
 * plain W4 linear.  Sources: abstract; summary sections 2.1 A and 2.2 A.
 *   x         [M][K] bf16, 16-byte aligned.  M >= 0 (M == 0 does nothing but
 *             write *n_active_out = 0 when that pointer is given).
 *   w         weights; w->N >= 1, w->K >= 32, w->K % 32 == 0.
 *   ec        EC and gate, or NULL.
 *   y         [M][N] output, fp32 or bf16 per out_dtype; 16-byte aligned.
 *   workspace device scratch of at least spear_w4_linear_workspace_size bytes,
 *             256-byte aligned, zeroed once (see spear_workspace_init).
 * Dispatch: M <= 16 takes the decode path (one launch; the gate, token
 * selection and EC down-projection run in the same kernel as the weight
 * stream, and the EC is applied in its epilogue); M > 16 takes the prefill
 * path (an EC pre-pass, then the MFMA GEMM with the EC in its epilogue).
 * The vector gate is formed where v is formed: in the fused decode kernel's
 * epilogue (ranks up to 32; larger ranks take the pre-pass form of the decode
 * path, two launches), or at the end of the EC pre-pass.
 * The result does not depend on the path beyond fp32 rounding order.
 * SPEAR_E_SHAPE also when a decode path's workspace layout would place the
 * regions its kernels use beyond 4 GiB (their offsets travel as 32-bit values;
 * only layers with billions of channel groups times K ranges come near).
 */
spear_status spear_w4_linear(const spear_bf16 *x, int64_t M, const spear_w4 *w,
                             const spear_ec *ec, void *y, int32_t out_dtype,
                             void *workspace, size_t ws_bytes, void *stream);

/* spear_w4_linear with an explicit SPEAR_PATH_* (the decode paths need M <= 16). */
spear_status spear_w4_linear_path(const spear_bf16 *x, int64_t M, const spear_w4 *w,
                                  const spear_ec *ec, void *y, int32_t out_dtype,
                                  void *workspace, size_t ws_bytes, int32_t path,
                                  void *stream);

/*
 * spear_w4_linear_semifused -- the prefill layer in the summary's semi-fused
 * form (section 2.2 A: at prefill the EC runs as a separate kernel beside the
 * low-bit GEMM, the two joined through the graph of the step).  On
 * `aux_stream`, forked from `stream` by ev_fork: the EC pre-pass (gate logit,
 * selection, v = g u, vector gate) and a ballot compaction of the active
 * tokens.  On `stream`, meanwhile: the plain W4 GEMM into y.  Then `stream`
 * waits for ev_join (recorded on aux_stream after the compaction) and one
 * more kernel adds B v into the rows of the active tokens only.  No kernel
 * waits on another stream's kernel; the fork and the join are event
 * dependencies, which HIP graph capture of `stream` records as graph edges.
 *   Arguments as for spear_w4_linear, except: y is fp32 only ([M][N]); ec may
 *   be NULL (then: the plain GEMM on `stream`, nothing on aux_stream);
 *   aux_stream is a stream other than `stream`; ev_fork and ev_join are
 *   hipEvent_t handles owned by the caller (created with timing disabled is
 *   enough), not used concurrently by other calls.  The workspace is that of
 *   spear_w4_linear (spear_w4_linear_workspace_size).
 */
spear_status spear_w4_linear_semifused(const spear_bf16 *x, int64_t M, const spear_w4 *w,
                                       const spear_ec *ec, float *y, void *workspace,
                                       size_t ws_bytes, void *stream, void *aux_stream,
                                       void *ev_fork, void *ev_join);

/* Size of the library's own scratch used by spear_w4_linear_noalloc, per GPU. */
#define SPEAR_NOALLOC_MAX_WORKSPACE ((size_t)48 << 20)

/*
 * spear_w4_linear_noalloc -- spear_w4_linear_path without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * kernels are those of spear_w4_linear_path; the workspace they need is a
 * file-scope device array of SPEAR_NOALLOC_MAX_WORKSPACE bytes inside the
 * library (one per GPU, zero when the library is loaded, held until the
 * process ends).  The call itself allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine.
 *   Arguments as for spear_w4_linear_path.  A layer whose workspace need
 *   (spear_w4_linear_workspace_size) exceeds SPEAR_NOALLOC_MAX_WORKSPACE is
 *   rejected with SPEAR_E_WORKSPACE before any HIP call.
 * Every call on one GPU uses that GPU's single scratch array, which carries
 * state from call to call (launch counters, tagged partials): calls that may
 * overlap on one GPU (two streams, two threads) race and must not be made.
 * Expired-wait counts of these calls stay inside the scratch (they are not
 * readable through spear_workspace_timeouts); the NaN outputs described below
 * still mark them.
 */
spear_status spear_w4_linear_noalloc(const spear_bf16 *x, int64_t M, const spear_w4 *w,
                                     const spear_ec *ec, void *y, int32_t out_dtype,
                                     int32_t path, void *stream);

/*
 * Some launches wait (bounded) for values that other workgroups of the same
 * launch produce: the fused decode kernel's epilogue (the EC partials), the
 * decode kernel's last K range (the other ranges' sums), the split pre-pass's
 * last slice and, where the pre-pass shares the GEMM's launch, the GEMM
 * epilogue.  If a wait exceeds the limit, every output whose sum it leaves
 * incomplete is written as NaN -- a decode workgroup's channels for all
 * tokens, a pre-pass token group's rows, a GEMM tile -- the affected g_out
 * entries are NaN, *n_active_out is -1, and a counter in the workspace is
 * incremented.  No expired wait ever yields a finite but wrong output.
 * spear_set_wait_limit sets the limit in polling rounds for launches enqueued
 * afterwards, from any thread (0 restores the default, about a second);
 * spear_workspace_timeouts synchronises `stream`, copies the counter to
 * *host_count and clears it.
 */
void spear_set_wait_limit(uint32_t rounds);
spear_status spear_workspace_timeouts(void *workspace, int32_t *host_count, void *stream);

/*
 * EC-aware prefill chunking under an inter-token-latency objective (host
 * only, no HIP call; all pointers are HOST pointers).  Source: the summary's
 * section 2.2 C -- the scheduler takes the largest prefill chunk whose
 * predicted inter-token latency meets the objective, from kernel-latency
 * tables computed ahead of time, and adapts to how many layers carry ECs --
 * and section 3.2 (stable latency objectives with dynamic chunking).
 *
 * The table holds, for each kind of linear call (a weight shape with or
 * without its EC), the measured time of one call at a grid of token counts,
 * and how many calls of that kind one forward step of the model makes (EC
 * density enters through these counts).  One step over m tokens is predicted
 * as overhead_us + sum_k count[k] L_k(m), with L_k the running maximum of the
 * kind's measurements (so the prediction never falls as m grows), linear
 * between grid points, its first value below the grid and its last segment's
 * slope above it.
 */
typedef struct spear_lut {
    int32_t npoints;        /* grid points, >= 1                                   */
    const int32_t *tokens;  /* [npoints] token counts, ascending, tokens[0] >= 1   */
    int32_t nkinds;         /* kinds of linear call, >= 1                          */
    const float *us;        /* [nkinds][npoints] microseconds per call, finite, >= 0 */
    const int32_t *count;   /* [nkinds] calls of each kind per step, >= 0          */
    float overhead_us;      /* fixed time per step outside these calls, >= 0      */
} spear_lut;

/* Predicted time of one step over `tokens` tokens (0 for no tokens). */
spear_status spear_slo_predict(const spear_lut *lut, int32_t tokens, float *us_out);

/*
 * spear_slo_pick_chunk -- the prefill chunk for the next step: the largest c,
 * either `pending` itself or a multiple of `align` below it, such that a step
 * over n_decode + c tokens (the running requests' decode tokens plus the
 * chunk) is predicted within slo_us.  0 when even the smallest chunk does not
 * fit.  *predicted_us (optional) receives the prediction for the chosen c.
 *   n_decode >= 0, pending >= 0 (prompt tokens waiting), align >= 1.
 */
spear_status spear_slo_pick_chunk(const spear_lut *lut, int32_t n_decode, int32_t pending,
                                  int32_t align, float slo_us, int32_t *chunk,
                                  float *predicted_us);

/*
 * spear_stream_read -- measurement helper, not part of the layer: reads every
 * byte of buf once (16-byte loads, four a thread in flight) and writes
 * nothing to *sink in practice (it is written only if the XOR of the data
 * equals a fixed constant, so that the loads cannot be optimised away).  Its
 * rate is the plain read floor that the decode kernel's bandwidth is compared
 * with, for buffers of the layer's size.
 *   buf  device pointer, 16-byte aligned; bytes >= 16 and a multiple of 16.
 *   sink device pointer to one uint32, 4-byte aligned.
 */
spear_status spear_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

const char *spear_status_string(spear_status s);
int32_t spear_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPEAR_H */
