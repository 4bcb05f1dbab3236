/*
 * spear_oracle.c -- plain CPU oracle for the W4A16 linear layer with a
 * per-token gated Error Compensator (EC).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  It exists so that the tests, the smoke check and
 * the CPU-baseline leg of the benchmark have an independent, obviously
 * correct result to compare the HIP path against.  It shares no code, header,
 * table or constant with the HIP library.
 *
 * Sources (page title, then section):
 *   [ABS]  "SPEAR: A System for Post-Quantization Error-Adaptive Recovery
 *          Enabling Efficient Low-Bit LLM Serving", authors' abstract
 *          (fugumt.com record of arXiv 2606.11244): W4 per-channel weights,
 *          lightweight ECs modulated by per-token gates.
 *   [P4-2.1A] same title, gist.science technical summary, section 2.1 A
 *          (input-adaptive error compensators): the EC projects x to a low
 *          rank with A, applies an input-dependent gate, projects back with
 *          B; effective weight W + alpha * B diag(gamma) A.
 *   [P4-3.1] same summary, section 3.1: the base quantizer is per-channel
 *          4-bit (RTN and others).
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *   - Orientation follows the summary's column-vector form: A is [r][K],
 *     B is [N][r], W is [N][K]; tokens are rows, y[m] = W_eff x[m].
 *   - The gate is a scalar per token, g_m = sigmoid(b + sum_k x[m][k] w_g[k]),
 *     alpha is folded into B (alpha = 1).
 *   - Hard gate: a token takes the EC iff its logit z_m > logit(tau); a tie
 *     skips.  Soft gate: every token takes it.
 *   - Vector gate (optional; the summary's diag(gamma(Ax)) with gamma a
 *     bottleneck MLP on the rank-r projection): gamma(u) =
 *     sigmoid(W2 relu(W1 u + c1) + c2), W1 [h][r], c1 [h], W2 [r][h], c2 [r]
 *     (fp32 parameters), applied rank by rank, on top of the scalar gate:
 *     e = act_m g_m alpha sum_j B[n][j] gamma_j(u) u_j.  h = 0 (no vector
 *     gate) is the scalar form above; b = +inf (g = 1) with a soft gate is the
 *     summary's form W + alpha B diag(gamma(Ax)) A.
 *   - Codes: signed codes q in [-8,7] are stored offset-binary u = q + 8 with
 *     zero point 8; unsigned codes u in [0,15] carry a per-channel zero point.
 *     Dequantised weight w = s_n * (u - z_n).
 *   - Packed layout (see nibble_index): rows of little-endian 32-bit words
 *     of 8 codes, nibble position p of a word holding code perm[p],
 *     perm = (0, 2, 4, 6, 1, 3, 5, 7).
 *
 * Precision: dequantised weights are formed in fp32 (s_n * (u - z_n)
 * evaluated in float); every sum (the main contraction, the gate logit, the
 * EC down- and up-projections) is carried in fp64; g is rounded to fp32.
 * Outputs are fp64.
 *
 * Pins (what ties this code to something other than itself) live in the
 * CPU test-suite: the hand-worked packing example, exhaustive pack/unpack
 * round trips, exact rational brute force on tiny shapes, the permutation
 * special case, the effective-weight identity (dense W + g B A against the
 * factored form), the rank-1 closed form, gate closed forms and the
 * reductions to plain W4 (A = 0, g = 0, tau = 1).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_CODES_S4 0
#define ORACLE_CODES_U4 1

/* bf16 bits -> float: a bf16 value is the upper half of an IEEE binary32. */
static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ---------------------------------------------------------------- packing */

/* Offset-binary nibble of one code; out-of-range codes are reduced to their
 * low 4 bits and counted.  [P4-3.1]: 4-bit per-channel codes. */
static uint8_t code_to_nibble(const void *codes, int kind, int64_t i, int64_t *bad)
{
    if (kind == ORACLE_CODES_S4) {
        int v = ((const int8_t *)codes)[i];
        if (v < -8 || v > 7)
            (*bad)++;
        return (uint8_t)((v + 8) & 0xF);
    }
    {
        int v = ((const uint8_t *)codes)[i];
        if (v > 15)
            (*bad)++;
        return (uint8_t)(v & 0xF);
    }
}

/* Packed layout (this library's; the pages give none): each row is a run of
 * 32-bit little-endian words, word w holding codes k = 8w .. 8w+7.  Nibble
 * position p of the word (bits 4p .. 4p+3) holds code 8w + perm[p] with
 * perm = (0, 2, 4, 6, 1, 3, 5, 7): byte 0 holds codes 0 and 2 (low, high
 * nibble), byte 1 codes 4 and 6, byte 2 codes 1 and 3, byte 3 codes 5 and 7.
 * The nibble position of code 8w + i is therefore i / 2 for even i and
 * 4 + i / 2 for odd i. */
static int64_t nibble_index(int64_t K, int64_t n, int64_t k)
{
    const int64_t w = k / 8, i = k % 8;
    const int64_t p = (i % 2 == 0) ? i / 2 : 4 + i / 2;
    return (n * (K / 2) + 4 * w) * 2 + p;          /* byte = index / 2, high nibble if odd */
}

int64_t oracle_pack_w4(const void *codes, int kind, int64_t N, int64_t K, uint8_t *packed)
{
    int64_t bad = 0;
    memset(packed, 0, (size_t)(N * (K / 2)));
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            const uint8_t u = code_to_nibble(codes, kind, n * K + k, &bad);
            const int64_t q = nibble_index(K, n, k);
            packed[q / 2] |= (uint8_t)((q % 2) ? (u << 4) : u);
        }
    }
    return bad;
}

/* Scalar unpack of one nibble. */
static int nibble_at(const uint8_t *packed, int64_t K, int64_t n, int64_t k)
{
    const int64_t q = nibble_index(K, n, k);
    const uint8_t byte = packed[q / 2];
    return (q % 2) ? (byte >> 4) : (byte & 0xF);
}

void oracle_unpack_w4(const uint8_t *packed, int64_t N, int64_t K, uint8_t *u)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            u[n * K + k] = (uint8_t)nibble_at(packed, K, n, k);
}

/* Dequantised weight in fp32: s_n * (u - z_n).  [P4-3.1] per-channel scale. */
static float dequant(const uint8_t *packed, const float *scales, const uint8_t *zeros,
                     int64_t K, int64_t n, int64_t k)
{
    int z = zeros ? (int)zeros[n] : 8;
    int q = nibble_at(packed, K, n, k) - z;
    return scales[n] * (float)q;
}

void oracle_dequant_w4(const uint8_t *packed, const float *scales, const uint8_t *zeros,
                       int64_t N, int64_t K, float *w)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            w[n * K + k] = dequant(packed, scales, zeros, K, n, k);
}

/* ------------------------------------------------------------------- gate */

/* Threshold in the logit domain: logit(tau) = log(tau / (1 - tau)).
 * tau >= 1 admits no token, tau <= 0 admits every token. */
double oracle_logit_threshold(float tau)
{
    double t = (double)tau;
    if (t >= 1.0)
        return INFINITY;
    if (t <= 0.0)
        return -INFINITY;
    return log(t / (1.0 - t));
}

/* Gate logit of one token, summed in fp64: z = b + sum_k x[k] w_g[k]. */
static double gate_logit(const uint16_t *xrow, const uint16_t *w_g, int64_t K, float b)
{
    double z = (double)b;
    for (int64_t k = 0; k < K; k++)
        z += (double)bf16_to_float(xrow[k]) * (double)bf16_to_float(w_g[k]);
    return z;
}

static float sigmoid_f(double z)
{
    return (float)(1.0 / (1.0 + exp(-z)));
}

static int token_active(double z, double t, int hard)
{
    return hard ? (z > t) : 1;
}

/* Per-token gate [ABS; P4-2.1A]: logits z (fp64), gate values g (fp32), and
 * the ascending list of tokens that take the EC. */
void oracle_gate(const uint16_t *x, int64_t M, int64_t K, const uint16_t *w_g, float b,
                 float tau, int hard, double *z, float *g, int32_t *idx, int32_t *n_active)
{
    double t = oracle_logit_threshold(tau);
    int32_t n = 0;
    for (int64_t m = 0; m < M; m++) {
        double zm = gate_logit(x + m * K, w_g, K, b);
        if (z)
            z[m] = zm;
        if (g)
            g[m] = sigmoid_f(zm);
        if (token_active(zm, t, hard)) {
            if (idx)
                idx[n] = (int32_t)m;
            n++;
        }
    }
    if (n_active)
        *n_active = n;
}

/* ---------------------------------------------------------- linear layer */

/* One output element.  Main term y0 = sum_k x[m][k] w[n][k]; EC term for an
 * active token: g_m * sum_j B[n][j] (sum_k A[j][k] x[m][k]).  The EC
 * down-projection u (length r) is passed in, computed once per token. */
static double linear_element(const uint16_t *xrow, int64_t K, int64_t n,
                             const uint8_t *packed, const float *scales, const uint8_t *zeros,
                             const double *u, const uint16_t *B, int64_t r, double g, int active)
{
    double y0 = 0.0;
    for (int64_t k = 0; k < K; k++)
        y0 += (double)bf16_to_float(xrow[k]) * (double)dequant(packed, scales, zeros, K, n, k);
    if (!active || u == NULL)
        return y0;
    double e = 0.0;
    for (int64_t j = 0; j < r; j++)
        e += (double)bf16_to_float(B[n * r + j]) * u[j];
    return y0 + g * e;
}

/* EC down-projection of one token: u[j] = sum_k A[j][k] x[k]. */
static void ec_down(const uint16_t *xrow, int64_t K, const uint16_t *A, int64_t r, double *u)
{
    for (int64_t j = 0; j < r; j++) {
        double s = 0.0;
        for (int64_t k = 0; k < K; k++)
            s += (double)bf16_to_float(A[j * K + k]) * (double)bf16_to_float(xrow[k]);
        u[j] = s;
    }
}

#define ORACLE_MAX_RANK 1024
#define ORACLE_MAX_HIDDEN 1024

/* Vector gate of one token [P4-2.1A]: gamma_j = sigmoid(c2[j] + sum_i
 * W2[j][i] relu(c1[i] + sum_l W1[i][l] u[l])), in fp64 from fp32 parameters.
 * The EC then uses gamma_j u_j in place of u_j. */
static void vector_gate(const double *u, int64_t r, int64_t h, const float *W1,
                        const float *c1, const float *W2, const float *c2, double *ug)
{
    double hid[ORACLE_MAX_HIDDEN];
    for (int64_t i = 0; i < h; i++) {
        double s = (double)c1[i];
        for (int64_t l = 0; l < r; l++)
            s += (double)W1[i * r + l] * u[l];
        hid[i] = s > 0.0 ? s : 0.0;
    }
    for (int64_t j = 0; j < r; j++) {
        double s = (double)c2[j];
        for (int64_t i = 0; i < h; i++)
            s += (double)W2[j * h + i] * hid[i];
        ug[j] = (1.0 / (1.0 + exp(-s))) * u[j];
    }
}

/* Optional vector-gate parameters (h = 0: none). */
typedef struct {
    int64_t h;
    const float *W1, *c1, *W2, *c2;
    double alpha;
} oracle_vgate;

/* Per-token EC set-up shared by the full and the sampled layer: gate value,
 * selection, and the rank vector the up-projection contracts with (u, or
 * gamma(u) u with the vector gate).  Returns the token's EC scale g alpha. */
static double token_ec(const uint16_t *xrow, int64_t K, const uint16_t *A, int64_t r,
                       const uint16_t *w_g, float b, double t, int hard,
                       const oracle_vgate *vg, int *active, double *u)
{
    double z = gate_logit(xrow, w_g, K, b);
    float g = sigmoid_f(z);
    *active = token_active(z, t, hard);
    if (!*active)
        return 0.0;
    ec_down(xrow, K, A, r, u);
    if (vg->h > 0) {
        double ug[ORACLE_MAX_RANK];
        vector_gate(u, r, vg->h, vg->W1, vg->c1, vg->W2, vg->c2, ug);
        for (int64_t j = 0; j < r; j++)
            u[j] = ug[j];
        return (double)g * vg->alpha;
    }
    return (double)g;
}

/*
 * Full layer: y[m][n] for all m < M, n < N (fp64 out).  has_ec = 0 gives the
 * plain W4 linear.  Tokens are independent, so rows are split over threads;
 * every sum keeps its natural k (or j) order.
 */
int oracle_w4_linear(const uint16_t *x, int64_t M, int64_t K, int64_t N,
                     const uint8_t *packed, const float *scales, const uint8_t *zeros,
                     int has_ec, const uint16_t *A, const uint16_t *B, int64_t r,
                     const uint16_t *w_g, float b, float tau, int hard,
                     int64_t gate_h, const float *W1, const float *c1, const float *W2,
                     const float *c2, float alpha, double *y)
{
    if (has_ec && (r < 1 || r > ORACLE_MAX_RANK))
        return -1;
    if (gate_h < 0 || gate_h > ORACLE_MAX_HIDDEN)
        return -3;
    const oracle_vgate vg = {gate_h, W1, c1, W2, c2, (double)alpha};
    double t = oracle_logit_threshold(tau);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++) {
        const uint16_t *xrow = x + m * K;
        double u[ORACLE_MAX_RANK];
        double g = 0.0;
        int active = 0;
        if (has_ec)
            g = token_ec(xrow, K, A, r, w_g, b, t, hard, &vg, &active, u);
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = linear_element(xrow, K, n, packed, scales, zeros,
                                          has_ec ? u : NULL, B, r, g, active);
    }
    return 0;
}

/*
 * Selected outputs only: y_s[i] = y[ms[i]][ns[i]].  Used where the full
 * product is too large for the CPU.  Same arithmetic as oracle_w4_linear.
 */
int oracle_w4_linear_sampled(const uint16_t *x, int64_t M, int64_t K, int64_t N,
                             const uint8_t *packed, const float *scales, const uint8_t *zeros,
                             int has_ec, const uint16_t *A, const uint16_t *B, int64_t r,
                             const uint16_t *w_g, float b, float tau, int hard,
                             int64_t gate_h, const float *W1, const float *c1, const float *W2,
                             const float *c2, float alpha,
                             int64_t S, const int64_t *ms, const int64_t *ns, double *y_s)
{
    if (has_ec && (r < 1 || r > ORACLE_MAX_RANK))
        return -1;
    if (gate_h < 0 || gate_h > ORACLE_MAX_HIDDEN)
        return -3;
    for (int64_t i = 0; i < S; i++)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return -2;
    const oracle_vgate vg = {gate_h, W1, c1, W2, c2, (double)alpha};
    double t = oracle_logit_threshold(tau);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < S; i++) {
        const uint16_t *xrow = x + ms[i] * K;
        double u[ORACLE_MAX_RANK];
        double g = 0.0;
        int active = 0;
        if (has_ec)
            g = token_ec(xrow, K, A, r, w_g, b, t, hard, &vg, &active, u);
        y_s[i] = linear_element(xrow, K, ns[i], packed, scales, zeros,
                                has_ec ? u : NULL, B, r, g, active);
    }
    return 0;
}
