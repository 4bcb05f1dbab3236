// decode.hip -- decode-sized W4A16 linear (M <= 16) with the gated error
// compensator fused into the same launch (gfx950).
//
// Source: "SPEAR: A System for Post-Quantization Error-Adaptive Recovery
// Enabling Efficient Low-Bit LLM Serving", gist.science summary section 2.2 A:
// at decode the layer is memory bound and the EC is folded into the low-bit
// GEMM's epilogue so that the compensated layer is a single kernel.  The EC
// itself follows section 2.1 A (down-projection A, per-token gate,
// up-projection B) with the scalar gate g = sigmoid(b + x.w_g).
//
// Work decomposition (one launch):
//  * a workgroup owns 16 output channels and a K range (all of K unless the
//    activations of the range would not fit in LDS).  Each of its stream waves
//    (4 with the fused EC; without it 8 over long K ranges on at most one
//    workgroup a CU, else 4) owns a run of 128-deep super-steps: it DMAs the
//    activations of exactly those steps into LDS (global_load_lds), issues
//    every 16-byte load of its packed-weight share (HBM -> registers), and
//    contracts each step as its load lands -- no workgroup barrier before the
//    contraction.  Several tokens: bf16 MFMA with the tokens (padded to 16) on
//    the MFMA's N side and a second MFMA against a constant-one operand for
//    the per-token activation sums that remove the unpack offset.  One token:
//    a wavefront-reduction GEMV (bf16 dot2 into fp32, four accumulators) and a
//    VALU activation sum.
//    The packed word order makes the unpacked pairs line up with the
//    activations' own pairs, so the activations are used as loaded.
//  * When K is split over workgroups, every range but the last stores its
//    sums as tagged words (below) and the channel group's last range -- its
//    highest block index -- adds them in range order (deterministic).
//  * EC (fused mode): the lowest block indices, which the dispatcher places
//    first, are `nprod` producer workgroups.  Each reads about 8 KB of A per
//    pair of tokens, at most 16 KB above 8 tokens (so a producer's share of
//    the memory system is no larger than a stream workgroup's), computes the
//    gate-logit partial (fp64) and A.x (MFMA; dot2 for one token) of every
//    token over its K slice, reduces its 4 waves in LDS and
//    stores the partials as 64-bit words {value, launch epoch}, one relaxed
//    device-coherent store each, then leaves.  The epilogue of each channel
//    group loads the words of its tokens (relaxed device-coherent loads, the 4
//    waves splitting the producers), re-loads until every tag carries this
//    launch's epoch (bounded), sums the producers in order, applies the gate
//    and the hard-gate selection, and adds g B (A x): B times A x as bf16
//    hi + lo (two MFMAs per 32 ranks; dot2 for one token), scaled by the gate
//    at the end so the fp64 sigmoid is off the MFMAs' path.  The first batch
//    of words is in flight while wave 0 reduces the stream waves.  Each word
//    is validated on its own, so no fence or counter orders the exchange;
//    every epilogue sums the same partials in the same order, and producers
//    never wait.
//  * The launch epoch comes from 64 counters in the workspace, 128 bytes
//    apart; block b adds to counter b % 64 so that no address is contended by
//    more than a few workgroups.  A launch adds exactly 2^32 to every counter
//    whatever its grid (see epoch_claim), and every block of the launch reads
//    the same upper half.  Graph replays and calls of other shapes on the same
//    workspace therefore never see a stale tag as current.
#include <atomic>

#include "spear_internal.hpp"

namespace spear {

namespace {

// Stream waves of a workgroup: DEC_WAVES with the fused EC (its producers and
// epilogue exchange are laid out for 4 waves); without it DEC_WAVES_PLAIN where
// plain_waves picks it.  The shared block is sized for the waves the kernel
// has: with the fused EC, a producer must fit on a CU beside a stream
// workgroup that holds nine token rows (2 x 79.3 KiB of LDS).
constexpr int DEC_WAVES_PLAIN = 8;
constexpr int64_t DEC_CUS = 256;                            // compute units of the chip
constexpr int DEC_DEVICES = 64;                             // devices a process may use, at most

template <int NW>
struct DecShared {
    float red[NW][64][5];
    alignas(16) float red16[NW][16];   // one token: each wave's channel sums
    float xs[NW];        // one token: the activation sum of each wave's chunks
    double zl[NW];       // one token, hard gate: each wave's gate-logit partial
    uint32_t u32[4];
};


__device__ __forceinline__ double dot8_f64(u32x4 x, u32x4 w, double acc)
{
    // bf16 x bf16 products are exact in fp32; the sum is carried in fp64
#pragma unroll
    for (int e = 0; e < 4; e++) {
        acc += (double)(__uint_as_float(x[e] << 16) * __uint_as_float(w[e] << 16));
        acc += (double)(__uint_as_float(x[e] & 0xFFFF0000u) * __uint_as_float(w[e] & 0xFFFF0000u));
    }
    return acc;
}

// ------------------------------------------------------------------ fused EC
constexpr int PCH = 256;                                  // producer K chunk per pass
constexpr int PS = PCH / 32;                              // 32-deep MFMA steps of a chunk
constexpr size_t EC_LDS_U = DEC_WAVES * 64 * 8 * sizeof(float);   // u partials of 4 waves
static_assert(EC_LDS_U >= DEC_WAVES * 16 * 32 * sizeof(float), "consumer u exchange");
constexpr size_t EC_LDS_Z = DEC_WAVES * 64 * sizeof(double);      // gate-logit partials
constexpr size_t EC_LDS = EC_LDS_U + EC_LDS_Z + 64;               // + tag and flags
// the vector gate's u [16][32] and hidden layer [16][SPEAR_MAX_GATE_HIDDEN], after EC_LDS
constexpr size_t EC_LDS_VG = (16 * 32 + 16 * SPEAR_MAX_GATE_HIDDEN) * sizeof(float);

// Vector gate of the fused decode (ranks up to 32, one rank block; summary
// section 2.1 A): wave 0, lane (lr, lg) holding ranks 8 lg .. 8 lg + 7 of token
// lr in (ua, ub), replaces them by gamma_j(u) u_j, gamma(u) = sigmoid(W2 relu(W1
// u + c1) + c2).  The token's u and hidden layer go through wave-local LDS
// (only wave 0 touches vl).
__device__ __forceinline__ void vgate_fused(const LinearArgs &a, float *vl, int lr, int lg,
                                            f32x4 &ua, f32x4 &ub)
{
    const int h = a.gate_h, r = a.r;
    float *vu = vl, *hid = vl + 16 * 32;
    *reinterpret_cast<f32x4 *>(vu + lr * 32 + 8 * lg) = ua;
    *reinterpret_cast<f32x4 *>(vu + lr * 32 + 8 * lg + 4) = ub;
    wait_lgkmcnt0();
    for (int i = lg; i < h; i += 4) {
        float sacc = a.gc1[i];
        const float *w1 = a.gw1 + (int64_t)i * r;
        for (int l = 0; l < r; l++)
            sacc = __builtin_fmaf(w1[l], vu[lr * 32 + l], sacc);
        hid[lr * SPEAR_MAX_GATE_HIDDEN + i] = sacc > 0.f ? sacc : 0.f;
    }
    wait_lgkmcnt0();
#pragma unroll
    for (int q = 0; q < 8; q++) {
        const int j = 8 * lg + q;
        float gam = 1.f;
        if (j < r) {
            float sacc = a.gc2[j];
            const float *w2 = a.gw2 + (int64_t)j * h;
            for (int i = 0; i < h; i++)
                sacc = __builtin_fmaf(w2[i], hid[lr * SPEAR_MAX_GATE_HIDDEN + i], sacc);
            gam = 1.f / (1.f + __expf(-sacc));
        }
        if (q < 4)
            ua[q] *= gam;
        else
            ub[q - 4] *= gam;
    }
}

// Producer workgroup p: wave w takes K slice [(4p + w) prod_k, +prod_k) and
// computes, for all 16 token slots, the gate-logit partial (fp64) and
// u[m][j] = sum_k A[j][k] x[m][k] (MFMA, fp32).  The waves are summed in order
// in LDS and wave 0 stores the rows of the M real tokens as tagged words.
__device__ void ec_produce(const LinearArgs &a, int64_t p, int wave, int lane, uint8_t *lds)
{
    const int tid = threadIdx.x, lr = lane & 15, lg = lane >> 4;
    const int64_t K = a.K, M = a.M;
    const int rpad = a.rpad, r = a.r;
    uint64_t claimed = opaque_zero64();
    if (tid == 0)
        claimed = epoch_claim(a, a.grid);                 // back long before it is used

    const int64_t k0 = (p * DEC_WAVES + wave) * a.prod_k;
    const int64_t k1 = (k0 + a.prod_k < K) ? k0 + a.prod_k : K;
    float *lu = reinterpret_cast<float *>(lds);
    double *lz = reinterpret_cast<double *>(lds + EC_LDS_U);
    uint32_t *ltag = reinterpret_cast<uint32_t *>(lds + EC_LDS_U + EC_LDS_Z);
    uint64_t *pu = reinterpret_cast<uint64_t *>(a.ws + a.D.pu);
    uint64_t *pz = reinterpret_cast<uint64_t *>(a.ws + a.D.pz);

    double zp = 0.0;
    for (int jp = 0; jp < rpad / 32; jp++) {
        f32x4 u0 = {0.f, 0.f, 0.f, 0.f}, u1 = {0.f, 0.f, 0.f, 0.f};
        const int j0 = 32 * jp + lr, j1 = j0 + 16;
        for (int64_t kc = k0; kc < k1; kc += PCH) {
            u32x4 xf[PS], a0[PS], a1[PS];
#pragma unroll
            for (int t = 0; t < PS; t++) {
                const int64_t k = kc + 32 * t + 8 * lg;
                const bool kv = kc + 32 * t < k1;
                xf[t] = (kv && lr < M) ? ld16(a.x + (int64_t)lr * K + k) : zero4();
                a0[t] = (kv && j0 < r) ? ld16(a.A + (int64_t)j0 * K + k) : zero4();
                a1[t] = (kv && j1 < r) ? ld16(a.A + (int64_t)j1 * K + k) : zero4();
            }
            if (jp == 0) {
                u32x4 wv[PS];
#pragma unroll
                for (int t = 0; t < PS; t++)
                    wv[t] = (kc + 32 * t < k1) ? ld16(a.wg + kc + 32 * t + 8 * lg) : zero4();
#pragma unroll
                for (int t = 0; t < PS; t++)
                    zp = dot8_f64(xf[t], wv[t], zp);
            }
#pragma unroll
            for (int t = 0; t < PS; t++) {
                u0 = mfma16(a0[t], xf[t], u0);
                u1 = mfma16(a1[t], xf[t], u1);
            }
        }
        // u0: ranks 32 jp + 4 lg + i, u1: ranks 32 jp + 16 + 4 lg + i; token lr
        float *mine = lu + (wave * 64 + lane) * 8;
        *reinterpret_cast<f32x4 *>(mine) = u0;
        *reinterpret_cast<f32x4 *>(mine + 4) = u1;
        if (jp == 0) {
            lz[wave * 64 + lane] = zp;
            if (tid == 0)
                *ltag = epoch_tag(claimed + opaque_zero64());   // not hoisted to the atomic
        }
        __syncthreads();
        if (wave == 0) {
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
            for (int w = 0; w < DEC_WAVES; w++) {
                s0 += *reinterpret_cast<const f32x4 *>(lu + (w * 64 + lane) * 8);
                s1 += *reinterpret_cast<const f32x4 *>(lu + (w * 64 + lane) * 8 + 4);
            }
            const uint32_t tag = *ltag;
            if (lr < M) {
                uint64_t *dst = pu + (p * 16 + lr) * rpad + 32 * jp + 4 * lg;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    store_tagged(dst + i, __float_as_uint(s0[i]), tag);
                    store_tagged(dst + 16 + i, __float_as_uint(s1[i]), tag);
                }
                if (jp == 0 && lg == 0) {
                    // z of token lr: waves in order, the four lane groups of each in order
                    double z = 0.0;
                    for (int w = 0; w < DEC_WAVES; w++)
                        z += ((lz[w * 64 + lr] + lz[w * 64 + lr + 16]) + lz[w * 64 + lr + 32]) +
                             lz[w * 64 + lr + 48];
                    const uint64_t zb = __builtin_bit_cast(uint64_t, z);
                    store_tagged(pz + (p * 16 + lr) * 2, (uint32_t)zb, tag);
                    store_tagged(pz + (p * 16 + lr) * 2 + 1, (uint32_t)(zb >> 32), tag);
                }
            }
        }
        __syncthreads();                                  // LDS reused by the next rank block
    }
}

// Producer workgroup p for one token (the GEMV decode): wave w takes K slice
// [(4p + w) prod_k, +prod_k); lane l takes rank 32 jp + l % 32 and the 32-deep
// half l / 32 of each 64-deep step, and contracts A's row with x by bf16 dot2
// (fp32) -- a plain matrix-vector product, no MFMA.  Lane 0 and 32 carry the
// gate-logit partial (fp64).  Halves, then waves, are summed in order.
__device__ void ec_produce_gv(const LinearArgs &a, int64_t p, int wave, int lane, uint8_t *lds)
{
    const int tid = threadIdx.x, j = lane & 31, h = lane >> 5;
    const int64_t K = a.K;
    const int rpad = a.rpad, r = a.r;
    uint64_t claimed = opaque_zero64();
    if (tid == 0)
        claimed = epoch_claim(a, a.grid);                 // back long before it is used

    const int64_t k0 = (p * DEC_WAVES + wave) * a.prod_k;
    const int64_t k1 = (k0 + a.prod_k < K) ? k0 + a.prod_k : K;   // k1 - k0: multiple of 32
    float *lu = reinterpret_cast<float *>(lds);                   // [wave][32]
    double *lz = reinterpret_cast<double *>(lds + EC_LDS_U);      // [wave]
    uint32_t *ltag = reinterpret_cast<uint32_t *>(lds + EC_LDS_U + EC_LDS_Z);
    uint64_t *pu = reinterpret_cast<uint64_t *>(a.ws + a.D.pu);
    uint64_t *pz = reinterpret_cast<uint64_t *>(a.ws + a.D.pz);

    double zp = 0.0;
    for (int jp = 0; jp < rpad / 32; jp++) {
        const int rank = 32 * jp + j;
        float u = 0.f;
        for (int64_t kc = k0; kc < k1; kc += 64) {
            const int64_t kk = kc + 32 * h;
            const bool kv = kk < k1;
            u32x4 xa[4], aa[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                xa[q] = kv ? ld16(a.x + kk + 8 * q) : zero4();
                aa[q] = (kv && rank < r) ? ld16(a.A + (int64_t)rank * K + kk + 8 * q) : zero4();
            }
            if (jp == 0 && j == 0) {
#pragma unroll
                for (int q = 0; q < 4; q++)
                    zp = dot8_f64(xa[q], kv ? ld16(a.wg + kk + 8 * q) : zero4(), zp);
            }
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    u = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(aa[q][e]), as_bf16x2(xa[q][e]), u,
                                                        false);
        }
        const float u_other = __shfl(u, (lane + 32) & 63);
        if (h == 0)
            lu[wave * 32 + j] = u + u_other;              // half 0, then half 1
        if (jp == 0) {
            const double z_other = __shfl(zp, 32);
            if (lane == 0)
                lz[wave] = zp + z_other;
            if (tid == 0)
                *ltag = epoch_tag(claimed + opaque_zero64());   // not hoisted to the atomic
        }
        __syncthreads();
        if (wave == 0 && h == 0) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < DEC_WAVES; w++)
                sum += lu[w * 32 + j];
            const uint32_t tag = *ltag;
            store_tagged(pu + p * 16 * rpad + 32 * jp + j, __float_as_uint(sum), tag);
            if (jp == 0 && j == 0) {
                double z = 0.0;
                for (int w = 0; w < DEC_WAVES; w++)
                    z += lz[w];
                const uint64_t zb = __builtin_bit_cast(uint64_t, z);
                store_tagged(pz + p * 16 * 2, (uint32_t)zb, tag);
                store_tagged(pz + p * 16 * 2 + 1, (uint32_t)(zb >> 32), tag);
            }
        }
        __syncthreads();                                  // LDS reused by the next rank block
    }
}

// Epilogue EC term (fused mode), called by all 4 waves of the workgroup that
// finishes channel group cg.  Wave w loads the words of producers
// [w np / 4, (w + 1) np / 4) in batches of 8 words a lane: per 32-rank block,
// lane l takes rank l % 32 of token rows l / 32 + 2 k, k < KM (consecutive
// lanes, consecutive words) of 8 / KM producers, and the gate-logit words of
// token l % 16 of producer l / 16 (+ 4); a batch is re-loaded until every tag is
// this launch's.  The wave subtotals meet in LDS and wave 0 finishes.  KM is
// ceil(M / 2) rounded up to a power of two.  `overlap` runs once in every wave,
// while the wave's first batch is in flight.  B u is formed first and the
// gate (act g) scales it at the end.  With GV (one token) B u is taken
// on the vector ALU in fp32: lane (c, g) forms the partial of channel c over
// ranks 8 g .. 8 g + 7, the four partials meet by shuffles in order, and each
// lane then picks its four output channels.  Returns, in wave 0, e[i] for
// channel 16 cg + 4 lg + i and token lr; *ok_out is false (and the term NaN)
// when a bounded wait expired.  Writes the gate outputs when cg == 0.
template <int KM, int GV, typename F>
__device__ f32x4 ec_consume(const LinearArgs &a, const u32x4 *bpre, int64_t cg, int wave, int lane,
                            uint8_t *lds, uint32_t tag, bool *ok_out, F overlap)
{
    constexpr int SPB = 8 / KM;                             // producers per batch
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t M = a.M, N = a.N, np = a.nprod;
    const int64_t n = cg * 16 + lr;
    const int rpad = a.rpad, r = a.r;
    const uint64_t *pu = reinterpret_cast<const uint64_t *>(a.ws + a.D.pu);
    const uint64_t *pz = reinterpret_cast<const uint64_t *>(a.ws + a.D.pz);
    float *lu = reinterpret_cast<float *>(lds);               // [wave][token][32]
    double *lz = reinterpret_cast<double *>(lds + EC_LDS_U);  // [wave][token]
    int32_t *lok = reinterpret_cast<int32_t *>(lds + EC_LDS_U + EC_LDS_Z);
    const int64_t p0 = np * wave / DEC_WAVES, p1 = np * (wave + 1) / DEC_WAVES;
    const int col = lane & 31, rh = lane >> 5;
    int64_t mrow[KM];
#pragma unroll
    for (int k = 0; k < KM; k++)
        mrow[k] = rh + 2 * k < M ? rh + 2 * k : M - 1;      // rows >= M re-read row M - 1
    const int64_t zm = lr < M ? lr : M - 1;

    f32x4 e = {0.f, 0.f, 0.f, 0.f};
    float g = 0.f;
    int act = 0;
    bool ok = true, overlapped = false;
    for (int t = 0; t < rpad / 32; t++) {
        float us[KM];
#pragma unroll
        for (int k = 0; k < KM; k++)
            us[k] = 0.f;
        double zs = 0.0;                                    // token lr, producers lg (mod 4)
        for (int64_t pc = p0; ok && pc < p1; pc += SPB) {
            uint64_t wu[SPB][KM], wz[(SPB + 3) / 4][2];
            for (uint32_t it = 0;; it++) {
                bool good = true;
#pragma unroll
                for (int c = 0; c < SPB; c++) {
                    const int64_t pp = (pc + c < p1) ? pc + c : p1 - 1;
#pragma unroll
                    for (int k = 0; k < KM; k++)
                        wu[c][k] = load_tagged(pu + (pp * 16 + mrow[k]) * rpad + 32 * t + col);
                }
                if (t == 0) {
#pragma unroll
                    for (int j = 0; j < (SPB + 3) / 4; j++) {
                        const int64_t q = pc + lg + 4 * j;
                        const int64_t pp = q < p1 ? q : p1 - 1;
                        wz[j][0] = load_tagged(pz + (pp * 16 + zm) * 2);
                        wz[j][1] = load_tagged(pz + (pp * 16 + zm) * 2 + 1);
                    }
                }
                if (t == 0 && pc == p0 && it == 0) {
                    overlap();                              // runs while the first words fly
                    overlapped = true;
                }
#pragma unroll
                for (int c = 0; c < SPB; c++)
#pragma unroll
                    for (int k = 0; k < KM; k++)
                        good &= (uint32_t)(wu[c][k] >> 32) == tag;
                if (t == 0) {
#pragma unroll
                    for (int j = 0; j < (SPB + 3) / 4; j++)
                        good &= (uint32_t)(wz[j][0] >> 32) == tag && (uint32_t)(wz[j][1] >> 32) == tag;
                }
                if (__all(good))
                    break;
                if (it >= a.wait_limit) {
                    ok = false;
                    if (lane == 0)
                        atomicAdd(reinterpret_cast<uint32_t *>(a.ws + a.D.hdr) + HDR_TIMEOUTS, 1u);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            if (!ok)
                break;
#pragma unroll
            for (int c = 0; c < SPB; c++)
                if (pc + c < p1)
#pragma unroll
                    for (int k = 0; k < KM; k++)
                        us[k] += __uint_as_float((uint32_t)wu[c][k]);
            if (t == 0) {
#pragma unroll
                for (int j = 0; j < (SPB + 3) / 4; j++)
                    if (lg + 4 * j < SPB && pc + lg + 4 * j < p1)
                        zs += __builtin_bit_cast(double, (uint64_t)(uint32_t)wz[j][0] |
                                                              ((uint64_t)(uint32_t)wz[j][1] << 32));
            }
        }
        if (!overlapped) {                                  // no producers in this wave, or a timeout
            overlap();
            overlapped = true;
        }
#pragma unroll
        for (int k = 0; k < KM; k++)
            if (rh + 2 * k < 16)
                lu[(wave * 16 + rh + 2 * k) * 32 + col] = us[k];
        if (t == 0) {
            // the four lane groups of token lr, in order
            const double z1 = __shfl(zs, lr + 16), z2 = __shfl(zs, lr + 32), z3 = __shfl(zs, lr + 48);
            if (lg == 0)
                lz[wave * 16 + lr] = ((zs + z1) + z2) + z3;
        }
        if (lane == 0)
            lok[wave] = ok;
        __syncthreads();
        const bool all_ok = lok[0] && lok[1] && lok[2] && lok[3];
        if (all_ok && wave == 0) {
            if (t == 0) {
                // Gate of token lr: producers summed in order.
                double z = (double)a.b;
                for (int w = 0; w < DEC_WAVES; w++)
                    z += lz[w * 16 + lr];
                g = (float)(1.0 / (1.0 + exp(-z)));
                act = (lr < M) && (a.hard ? (z > a.thr) : 1);
                if (cg == 0) {
                    const int a0 = (lane < 16) ? act : 0;
                    const uint64_t mask = __ballot(a0);
                    if (lane < 16 && lane < M && a.g_out)
                        a.g_out[lane] = g;
                    if (a0 && a.idx_out)
                        a.idx_out[__popcll(mask & ((1ull << lane) - 1ull))] = lane;
                    if (lane == 0 && a.nact_out)
                        *a.nact_out = __popcll(mask);
                }
            }
            if constexpr (GV) {
                // token 0's u[32 t + 8 lg + q], q = 0..7; lanes of other tokens drop
                // out.  B u first; the gate scales the sum at the end.
                f32x4 ua = {0.f, 0.f, 0.f, 0.f}, ub = ua;
#pragma unroll
                for (int w = 0; w < DEC_WAVES; w++) {
                    ua += *reinterpret_cast<const f32x4 *>(lu + w * 16 * 32 + 8 * lg);
                    ub += *reinterpret_cast<const f32x4 *>(lu + w * 16 * 32 + 8 * lg + 4);
                }
                if (a.gate_h > 0)
                    vgate_fused(a, reinterpret_cast<float *>(lds + EC_LDS), lr, lg, ua, ub);
                const int j = 32 * t + 8 * lg;
                u32x4 bf;
                if (t < 2)
                    bf = bpre[t == 0 ? 0 : 1];
                else
                    bf = (n < N && j < r) ? ld16(a.B + n * r + j) : zero4();
                float ep = 0.f;
#pragma unroll
                for (int q = 0; q < 8; q++) {
                    const float v = q < 4 ? ua[q] : ub[q - 4];
                    const uint32_t bw = bf[q / 2];
                    const float bq = __uint_as_float((q & 1) ? (bw & 0xFFFF0000u) : (bw << 16));
                    ep = __builtin_fmaf(bq, v, ep);
                }
                // channel lr: the four rank groups in order
                const float e1 = __shfl(ep, lr + 16), e2 = __shfl(ep, lr + 32),
                            e3 = __shfl(ep, lr + 48), e0 = __shfl(ep, lr);
                const float erow = ((e0 + e1) + e2) + e3;
#pragma unroll
                for (int i = 0; i < 4; i++)
                    e[i] += __shfl(erow, 4 * lg + i);
            } else {
                // u[lr][32 t + 8 lg + q]; rows >= M hold stale LDS and are zeroed.
                // B u first (hi + lo); the gate scales the sum at the end.
                f32x4 ua = {0.f, 0.f, 0.f, 0.f}, ub = ua;
#pragma unroll
                for (int w = 0; w < DEC_WAVES; w++) {
                    ua += *reinterpret_cast<const f32x4 *>(lu + (w * 16 + lr) * 32 + 8 * lg);
                    ub += *reinterpret_cast<const f32x4 *>(lu + (w * 16 + lr) * 32 + 8 * lg + 4);
                }
                if (a.gate_h > 0)
                    vgate_fused(a, reinterpret_cast<float *>(lds + EC_LDS), lr, lg, ua, ub);
                const int j = 32 * t + 8 * lg;
                u32x4 vh, vl;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const float v0 = lr < M ? (q < 2 ? ua[2 * q] : ub[2 * q - 4]) : 0.f;
                    const float v1 = lr < M ? (q < 2 ? ua[2 * q + 1] : ub[2 * q - 3]) : 0.f;
                    const uint16_t h0 = f2bf(v0), h1 = f2bf(v1);
                    vh[q] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                    vl[q] = (uint32_t)f2bf(v0 - bf16f(h0)) | ((uint32_t)f2bf(v1 - bf16f(h1)) << 16);
                }
                u32x4 bf;
                if (t < 2)
                    bf = bpre[t == 0 ? 0 : 1];
                else
                    bf = (n < N && j < r) ? ld16(a.B + n * r + j) : zero4();
                e = mfma16(bf, vh, e);
                e = mfma16(bf, vl, e);
            }
        }
        __syncthreads();                                  // LDS reused by the next rank block
        if (!all_ok) {
            ok = false;
            break;
        }
    }
    // the gate of the lane's token (token 0 with one token)
    const float ga = a.gate_h > 0 ? a.alpha : 1.f;    // the vector gate's scale
    const float gs = GV ? (__shfl(act, 0) ? __shfl(g, 0) * ga : 0.f) : (act ? g * ga : 0.f);
    *ok_out = ok;
    if (!ok) {
        // An expired wait: the EC term of every token of this channel group is
        // unknown, so its outputs become NaN; the first channel group also
        // marks the gate outputs (g NaN, n_active -1).
        const float qnan = __builtin_nanf("");
        if (cg == 0 && wave == 0) {
            if (lane < M && a.g_out)
                a.g_out[lane] = qnan;
            if (lane == 0 && a.nact_out)
                *a.nact_out = -1;
        }
        return f32x4{qnan, qnan, qnan, qnan};
    }
    return e * gs;
}

template <int EC_MODE, int OUT_F32, int SW, int GV, int NW>
__global__ __launch_bounds__(64 * NW) void decode_kernel(const LinearArgs a)
{
    static_assert(EC_MODE != 1 || NW == DEC_WAVES, "the fused EC's exchange is laid out for 4 waves");
    __shared__ DecShared<NW> sh;
    extern __shared__ __attribute__((aligned(16))) uint8_t s_x[];
    pin_dec_args(a);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // EC producers (fused mode) are the lowest block indices, which start first:
    // they store the partials of their K slices, then leave.
    int64_t bid = blockIdx.x;
    if (EC_MODE == 1) {
        if (bid < a.nprod) {
            if constexpr (GV)
                ec_produce_gv(a, bid, wave, lane, s_x);
            else
                ec_produce(a, bid, wave, lane, s_x);
            return;
        }
        bid -= a.nprod;
    }
    const bool stream = true;
    // Stream waves issue ahead of a co-resident producer's waves until their
    // contraction is done (a producer shares a CU with some stream workgroup,
    // which otherwise finishes last).
    if (EC_MODE == 1)
        __builtin_amdgcn_s_setprio(1);
    const int64_t ksplit = a.ksplit, spw = a.spw;
    const int64_t cg = bid / ksplit, ks = bid - cg * ksplit;
    const int64_t n0 = cg * 16;
    const int64_t K = a.K, N = a.N, M = a.M;
    const int64_t S = (K + 127) / 128;
    const int64_t s_begin = ks * spw;                        // first super-step of the range
    const int64_t s_count = (S - s_begin < spw) ? S - s_begin : spw;
    const int64_t rs_bytes = spw * 256 + 16;                 // LDS bytes per token row
    const int64_t cpr = s_count * 16;                        // 16-byte activation chunks per row
    const int64_t n = n0 + lr;
    const int64_t nc = n < N ? n : N - 1;                    // clamped: loads stay in bounds

    // 2. Epilogue operands, raw and without branches (used by wave 0 at the end):
    //    scales, zero points, and the B rows for ranks below 64.
    float sc_raw[4];
    uint32_t z_raw[4];
    u32x4 bpre[2] = {zero4(), zero4()};
    if (stream) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            int64_t nn = n0 + 4 * lg + i;
            nn = nn < N ? nn : N - 1;
            sc_raw[i] = a.scales[nn];
            z_raw[i] = load_zero_byte(a.zeros, a.scales, nn);
        }
        if (EC_MODE != 0) {
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int j = 32 * t + 8 * lg;
                bpre[t] = ld16(a.B + nc * a.r + (j < a.r ? j : a.r - 8));
            }
        }
    }

    // 3. Activations -> LDS directly (global_load_lds, 16 bytes a lane, 64
    //    consecutive chunks of one token row per wave instruction).  Each wave
    //    stages exactly the chunks of its own super-steps (the only ones it
    //    reads), so no workgroup barrier separates staging from contraction.
    //    Chunks past K and the wave's part of the extra row M (read by token
    //    slots >= M) are zeros.
    const int sl0 = wave * SW;                               // first local super-step
    const int64_t c0 = 16 * (int64_t)sl0;                    // the wave's chunks [c0, c1)
    const int64_t c1 = (c0 + 16 * SW < cpr) ? c0 + 16 * SW : cpr;
    if (stream) {
        for (int64_t m = 0; m < M; m++) {
            for (int64_t q0 = c0; q0 < c1; q0 += 64) {
                const int64_t q = q0 + lane;
                const int64_t k = s_begin * 128 + 8 * q;
                if (q < c1 && k < K)
                    __builtin_amdgcn_global_load_lds(
                        (const __attribute__((address_space(1))) void *)(a.x + m * K + k),
                        (__attribute__((address_space(3))) void *)(s_x + m * rs_bytes + 16 * q0),
                        16, 0, 0);
                else if (q < c1)
                    *reinterpret_cast<u32x4 *>(s_x + m * rs_bytes + 16 * q) = zero4();
            }
        }
        for (int64_t q = c0 + lane; q < c1; q += 64)
            *reinterpret_cast<u32x4 *>(s_x + M * rs_bytes + 16 * q) = zero4();
    }

    // 3b. One token under the hard gate, with all of K in this workgroup: the
    //     gate logit is formed here too, so that a token the gate skips takes
    //     no EC exchange at all.  The wave loads the w_g chunks of its own
    //     activation chunks before the weight stream, so the wait for the
    //     activations below also covers them.  Every workgroup sums the same
    //     products in the same order, so all agree on the selection.
    constexpr int WGQ = (SW + 3) / 4;                        // chunks a lane takes: c1 - c0 <= 16 SW
    const bool zloc = EC_MODE == 1 && GV && a.hard && ksplit == 1;
    u32x4 wgv[WGQ];
#pragma unroll
    for (int i = 0; i < WGQ; i++) {
        const int64_t q = c0 + lane + 64 * i;
        const int64_t k = s_begin * 128 + 8 * q;
        wgv[i] = (zloc && q < c1 && k < K) ? ld16(a.wg + k) : zero4();
    }

    // 4. The weight stream of this wave: SW loads, all in flight at once.  Out of
    //    range rows and depths read clamped in-bounds addresses; their products
    //    meet zero activations or are never stored.
    u32x4 wr[SW];
#pragma unroll
    for (int i = 0; i < SW; i++) {
        int64_t k = (s_begin + sl0 + i) * 128 + 32 * lg;
        k = k < K ? k : K - 32;
        wr[i] = ld16(a.packed + nc * (K / 2) + k / 2);
    }
    // Launch epoch (fused EC, or K split over workgroups), claimed behind the
    // weight loads so that its round trip overlaps the stream; it is first
    // needed in the epilogue.
    uint64_t claimed = opaque_zero64();
    if ((EC_MODE == 1 || a.ksplit > 1) && tid == 0)
        claimed = epoch_claim(a, a.grid);

    // Wait for everything but the weight stream (the SW youngest loads) and for
    // the LDS zero fills: the wave's activations are then in LDS.  The weight
    // loads stay in flight; each super-step waits for its own.  (In the wave
    // that claimed the epoch the claim is the youngest operation, so there the
    // first weight load is waited for too; it is needed next.)
    wait_vmcnt<SW>();
    wait_lgkmcnt0();

    // 5. One token: sum the wave's activations (the offset removal needs the
    //    token's activation sum), reduced across the wave in a fixed butterfly
    //    order.  More tokens take their sums from a ones-MFMA in the loop.
    if (GV) {
        float xsum = 0.f;
        double zp = 0.0;
#pragma unroll
        for (int i = 0; i < WGQ; i++) {
            const int64_t q = c0 + lane + 64 * i;
            if (q < c1) {
                const u32x4 xv = *reinterpret_cast<const u32x4 *>(s_x + 16 * q);
                xsum = sum8(xv, xsum);
                if (zloc)
                    zp = dot8_f64(xv, wgv[i], zp);
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            xsum += __shfl_xor(xsum, o);
        if (lane == 0)
            sh.xs[wave] = xsum;
        if (zloc) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1)
                zp += __shfl_xor(zp, o);
            if (lane == 0)
                sh.zl[wave] = zp;
        }
    }

    // 6. Contraction (stream waves), each super-step as soon as its weights land.
    if (GV) {
        // One token: a wavefront-reduction GEMV.  Lane (c, g) holds channel
        // n0 + c and 32 consecutive k of each super-step; the unpacked pairs
        // meet the activation pairs in bf16 dot2 (fp32), one accumulator per
        // 8-deep quarter.
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < SW; i++) {
            const int sl = sl0 + i;
            if (sl < s_count) {
                u32x4 xr[4];
#pragma unroll
                for (int d = 0; d < 4; d++)
                    xr[d] = *reinterpret_cast<const u32x4 *>(s_x + (16 * sl + 4 * lg + d) * 16);
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    const u32x4 uw = unpack8(wr[i][d]);
#pragma unroll
                    for (int q = 0; q < 4; q++)
                        acc[d] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(uw[q]),
                                                                 as_bf16x2(xr[d][q]), acc[d], false);
                }
            }
        }
        // the wave's four lane groups (k quarters of every step) of channel c
        float v = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (lane < 16)
            sh.red16[wave][lane] = v;
    } else {
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, rs0 = acc0, rs1 = acc0;
        const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
        const uint8_t *xrow = s_x + (lr < M ? lr : M) * rs_bytes;
#pragma unroll
        for (int i = 0; i < SW; i++) {
            const int sl = sl0 + i;
            if (sl < s_count) {
                u32x4 xr[4];
#pragma unroll
                for (int d = 0; d < 4; d++)
                    xr[d] = *reinterpret_cast<const u32x4 *>(xrow + (16 * sl + 4 * lg + d) * 16);
                acc0 = mfma16(unpack8(wr[i][0]), xr[0], acc0);
                rs0 = mfma16(ones, xr[0], rs0);
                acc1 = mfma16(unpack8(wr[i][1]), xr[1], acc1);
                rs1 = mfma16(ones, xr[1], rs1);
                acc0 = mfma16(unpack8(wr[i][2]), xr[2], acc0);
                rs0 = mfma16(ones, xr[2], rs0);
                acc1 = mfma16(unpack8(wr[i][3]), xr[3], acc1);
                rs1 = mfma16(ones, xr[3], rs1);
            }
        }
        const f32x4 acc = acc0 + acc1;
#pragma unroll
        for (int i = 0; i < 4; i++)
            sh.red[wave][lane][i] = acc[i];
        sh.red[wave][lane][4] = rs0[0] + rs1[0];
    }
    if (EC_MODE == 1)
        __builtin_amdgcn_s_setprio(0);
    if ((EC_MODE == 1 || ksplit > 1) && tid == 0)
        sh.u32[0] = epoch_tag(claimed + opaque_zero64());    // both halves live until here
    __syncthreads();

    // 7. Reduce the stream waves (fixed order).  Afterwards lane (t, g) of
    //    wave 0 holds channels n0 + 4 g + i of token t, and token t's sum of x.
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    float rst = 0.f;
    auto reduce_waves = [&]() {
        if (GV && wave == 0) {
            for (int w = 0; w < NW; w++) {
                tot += *reinterpret_cast<const f32x4 *>(&sh.red16[w][4 * lg]);
                rst += sh.xs[w];
            }
        } else if (wave == 0) {
            for (int w = 0; w < NW; w++) {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    tot[i] += sh.red[w][lane][i];
                rst += sh.red[w][lane][4];
            }
        }
    };

    // 9 (fused EC). The EC term, all 4 waves; the wave reduction above runs
    // while the first partial words are in flight when K is not split.
    f32x4 ec_e = {0.f, 0.f, 0.f, 0.f};
    auto consume = [&](auto overlap) {
        bool ok;
        const uint32_t tag = sh.u32[0];
        if (M <= 2)
            ec_e = ec_consume<1, (GV && 1 == 1)>(a, bpre, cg, wave, lane, s_x, tag, &ok, overlap);
        else if (M <= 4)
            ec_e = ec_consume<2, (GV && 2 == 1)>(a, bpre, cg, wave, lane, s_x, tag, &ok, overlap);
        else if (M <= 8)
            ec_e = ec_consume<4, (GV && 4 == 1)>(a, bpre, cg, wave, lane, s_x, tag, &ok, overlap);
        else
            ec_e = ec_consume<8, (GV && 8 == 1)>(a, bpre, cg, wave, lane, s_x, tag, &ok, overlap);
    };

    // A token the hard gate skips (logit formed in this workgroup): no EC
    // exchange; the first channel group reports the gate.
    bool skip_ec = false;
    if (zloc) {
        double z = (double)a.b;
        for (int w = 0; w < NW; w++)
            z += sh.zl[w];
        if (!(z > a.thr)) {
            skip_ec = true;
            if (cg == 0 && tid == 0) {
                if (a.g_out)
                    a.g_out[0] = (float)(1.0 / (1.0 + exp(-z)));
                if (a.nact_out)
                    *a.nact_out = 0;
            }
        }
    }
    bool epi = true;
    if (EC_MODE == 1 && ksplit == 1 && !skip_ec) {
        consume(reduce_waves);
    } else {
        reduce_waves();

        // 8. Reduce the K ranges.  Every range but the last stores wave 0's sums
        //    of its token lanes as tagged words {value, launch epoch} (relaxed
        //    device-coherent stores) and leaves; the channel group's last range
        //    -- its highest block index, dispatched after the others, which never
        //    wait -- re-loads them until every tag is this launch's (bounded; an
        //    expired wait is counted and makes the channels' outputs NaN), adds
        //    them in range order and then its own.  No fence: a release fence
        //    per workgroup would write back the whole L2 (measured: 20 against
        //    8.7 us for M = 16, K = 8192).
        if (ksplit > 1) {
            uint64_t *sp = reinterpret_cast<uint64_t *>(a.ws + a.D.splitp);
            const uint32_t tag = sh.u32[0];
            epi = ks == ksplit - 1;
            if (wave == 0 && lr < M) {
                if (!epi) {
                    uint64_t *d = sp + ((cg * ksplit + ks) * 64 + lane) * 5;
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        store_tagged(d + i, __float_as_uint(tot[i]), tag);
                    store_tagged(d + 4, __float_as_uint(rst), tag);
                } else {
                    constexpr int QB = 4;                     // ranges a batch
                    f32x4 st = {0.f, 0.f, 0.f, 0.f};
                    float sr = 0.f;
                    bool ok = true;
                    for (int64_t q0 = 0; ok && q0 < ksplit - 1; q0 += QB) {
                        uint64_t w[QB][5];
                        for (uint32_t it = 0;; it++) {
                            bool good = true;
#pragma unroll
                            for (int q = 0; q < QB; q++)
                                if (q0 + q < ksplit - 1) {    // uniform
                                    const uint64_t *src = sp + ((cg * ksplit + q0 + q) * 64 + lane) * 5;
#pragma unroll
                                    for (int i = 0; i < 5; i++)
                                        w[q][i] = load_tagged(src + i);
                                }
#pragma unroll
                            for (int q = 0; q < QB; q++)
                                if (q0 + q < ksplit - 1)
#pragma unroll
                                    for (int i = 0; i < 5; i++)
                                        good &= (uint32_t)(w[q][i] >> 32) == tag;
                            if (__all(good))
                                break;
                            if (it >= a.wait_limit) {
                                ok = false;
                                if (lane == 0)
                                    atomicAdd(reinterpret_cast<uint32_t *>(a.ws + a.D.hdr) + HDR_TIMEOUTS, 1u);
                                break;
                            }
                            __builtin_amdgcn_s_sleep(1);
                        }
                        if (!ok)
                            break;
#pragma unroll
                        for (int q = 0; q < QB; q++)
                            if (q0 + q < ksplit - 1) {
#pragma unroll
                                for (int i = 0; i < 4; i++)
                                    st[i] += __uint_as_float((uint32_t)w[q][i]);
                                sr += __uint_as_float((uint32_t)w[q][4]);
                            }
                    }
                    tot = st + tot;
                    rst = sr + rst;
                    if (!ok) {
                        // an expired wait: these channels' sums are incomplete
                        const float qnan = __builtin_nanf("");
                        tot = f32x4{qnan, qnan, qnan, qnan};
                        rst = qnan;
                    }
                }
            }
        }
        if (EC_MODE == 1 && epi && !skip_ec)
            consume([] {});
    }

    // 10. Wave 0 scales, removes the offset, adds the EC term and stores.
    if (epi && wave == 0) {
        float yv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t nn = n0 + 4 * lg + i;
            const float zc = UNPACK_OFF + zero_point(a.zeros, z_raw[i]);
            yv[i] = nn < N ? sc_raw[i] * __builtin_fmaf(-zc, rst, UNPACK_SCALE * tot[i]) : 0.f;
        }
        if (EC_MODE == 1) {
#pragma unroll
            for (int i = 0; i < 4; i++)
                yv[i] += ec_e[i];
        } else if (EC_MODE == 2) {
            // v precomputed by the pre-pass (bf16 hi + lo, zero for skipped tokens)
            const int32_t *active = reinterpret_cast<const int32_t *>(a.ws + a.D.active);
            const uint16_t *vhi = reinterpret_cast<const uint16_t *>(a.ws + a.D.vhi);
            const uint16_t *vlo = reinterpret_cast<const uint16_t *>(a.ws + a.D.vlo);
            const int act = (lr < M) ? active[lr] : 0;
            if (__ballot(act) != 0ull) {
                f32x4 e = {0.f, 0.f, 0.f, 0.f};
                const int rpad = a.rpad, r = a.r;
                for (int t = 0; t < rpad / 32; t++) {
                    const int j = 32 * t + 8 * lg;
                    u32x4 bf;
                    if (t < 2)
                        bf = bpre[t == 0 ? 0 : 1];
                    else
                        bf = (n < N && j < r) ? ld16(a.B + n * r + j) : zero4();
                    const u32x4 vh = ld16(vhi + lr * rpad + j);
                    const u32x4 vl = ld16(vlo + lr * rpad + j);
                    e = mfma16(bf, vh, e);
                    e = mfma16(bf, vl, e);
                }
#pragma unroll
                for (int i = 0; i < 4; i++)
                    yv[i] += e[i];
            }
        }
        if (lr < M) {
            const int64_t nb = n0 + 4 * lg;
            if (OUT_F32) {
                float *y = reinterpret_cast<float *>(a.y) + (int64_t)lr * N;
                if (nb + 3 < N && (N & 3) == 0) {
                    *reinterpret_cast<f32x4 *>(y + nb) = f32x4{yv[0], yv[1], yv[2], yv[3]};
                } else {
                    for (int i = 0; i < 4; i++)
                        if (nb + i < N)
                            y[nb + i] = yv[i];
                }
            } else {
                uint16_t *y = reinterpret_cast<uint16_t *>(a.y) + (int64_t)lr * N;
                if (nb + 3 < N && (N & 3) == 0) {
                    uint2 o;
                    o.x = (uint32_t)f2bf(yv[0]) | ((uint32_t)f2bf(yv[1]) << 16);
                    o.y = (uint32_t)f2bf(yv[2]) | ((uint32_t)f2bf(yv[3]) << 16);
                    *reinterpret_cast<uint2 *>(y + nb) = o;
                } else {
                    for (int i = 0; i < 4; i++)
                        if (nb + i < N)
                            y[nb + i] = f2bf(yv[i]);
                }
            }
        }
    }
}

// Dynamic LDS beyond 64 KiB must be enabled per kernel, once on each device.
template <int EC_MODE, int OUT_F32, int SW, int GV, int NW>
hipError_t launch_decode_k(const LinearArgs &a, hipStream_t s)
{
    static std::atomic<int> enabled[DEC_DEVICES];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= DEC_DEVICES)
        return hipErrorInvalidDevice;
    if (!enabled[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&decode_kernel<EC_MODE, OUT_F32, SW, GV, NW>),
            hipFuncAttributeMaxDynamicSharedMemorySize, DEC_LDS_MAX);
        if (e != hipSuccess)
            return e;
        enabled[dev].store(1, std::memory_order_release);
    }
    const int64_t npwg = EC_MODE == 1 ? a.nprod : 0;
    const dim3 grid((unsigned)(npwg + (int64_t)a.ncg * a.ksplit));
    const dim3 block(64 * NW);
    size_t lds = (size_t)(a.M + 1) * (size_t)(a.spw * 256 + 16);
    const size_t ec_lds = EC_LDS + (a.gate_h > 0 ? EC_LDS_VG : 0);
    if (EC_MODE == 1 && lds < ec_lds)
        lds = ec_lds;                                     // EC partials meet in the same LDS
    LinearArgs ka = a;
    ka.grid = grid.x;                                     // the kernels read it instead of gridDim
    hipLaunchKernelGGL((decode_kernel<EC_MODE, OUT_F32, SW, GV, NW>), grid, block, lds, s, ka);
    return hipGetLastError();
}

// SW = super-steps a stream wave takes: the workgroup's range split over its
// NW waves (at most DEC_WAVES * DEC_SW_MAX super-steps, so SW <= DEC_SW_MAX).
template <int EC_MODE, int OUT_F32, int GV, int NW>
hipError_t launch_decode_sw(const LinearArgs &a, hipStream_t s)
{
    switch ((a.spw + NW - 1) / NW) {
    case 1: return launch_decode_k<EC_MODE, OUT_F32, 1, GV, NW>(a, s);
    case 2: return launch_decode_k<EC_MODE, OUT_F32, 2, GV, NW>(a, s);
    case 3: return launch_decode_k<EC_MODE, OUT_F32, 3, GV, NW>(a, s);
    case 4: return launch_decode_k<EC_MODE, OUT_F32, 4, GV, NW>(a, s);
    case 5: return launch_decode_k<EC_MODE, OUT_F32, 5, GV, NW>(a, s);
    case 6: return launch_decode_k<EC_MODE, OUT_F32, 6, GV, NW>(a, s);
    case 7: return launch_decode_k<EC_MODE, OUT_F32, 7, GV, NW>(a, s);
    default: return launch_decode_k<EC_MODE, OUT_F32, 8, GV, NW>(a, s);
    }
}

// Stream waves of a workgroup without the fused EC.  Eight waves halve each
// wave's chain of super-steps, which pays only where a workgroup streams a long
// K range (at least 32 super-steps) and the grid is at most one workgroup a CU;
// otherwise four.  Measured on plain decode, 4 against 8 waves: 4096 x 4096
// at 1 / 4 / 8 tokens 5.75 / 6.84 / 7.81 against 5.64 / 6.08 / 6.31 us, and
// N = 2048, K = 8192 at 8 tokens 8.80 against 7.52 us; but K = 2048 at 16
// tokens 5.13 against 6.66 us and N = 14336, K = 4096 at 8 tokens 15.4
// against 18.2 us.
int plain_waves(const LinearArgs &a)
{
    return (a.spw >= 32 && a.ncg * a.ksplit <= DEC_CUS) ? DEC_WAVES_PLAIN : DEC_WAVES;
}

template <int EC_MODE, int OUT_F32, int GV>
hipError_t launch_decode_nw(const LinearArgs &a, hipStream_t s)
{
    if (EC_MODE != 1 && plain_waves(a) == DEC_WAVES_PLAIN)
        return launch_decode_sw<EC_MODE, OUT_F32, GV, (EC_MODE != 1 ? DEC_WAVES_PLAIN : DEC_WAVES)>(a, s);
    return launch_decode_sw<EC_MODE, OUT_F32, GV, DEC_WAVES>(a, s);
}

// One token takes the GEMV form (vector ALU); 2..16 tokens share every
// unpacked weight, a dense contraction, and take MFMA.  The pre-pass EC mode
// keeps the MFMA form for every M.
template <int EC_MODE, int OUT_F32>
hipError_t launch_decode_gv(const LinearArgs &a, hipStream_t s)
{
    if (EC_MODE != 2 && a.M == 1)
        return launch_decode_nw<EC_MODE, OUT_F32, (EC_MODE != 2 ? 1 : 0)>(a, s);
    return launch_decode_nw<EC_MODE, OUT_F32, 0>(a, s);
}

template <int EC_MODE>
hipError_t launch_decode_t(const LinearArgs &a, hipStream_t s)
{
    return a.out_f32 ? launch_decode_gv<EC_MODE, 1>(a, s) : launch_decode_gv<EC_MODE, 0>(a, s);
}

} // namespace

hipError_t launch_decode(const LinearArgs &a, int ec_mode, hipStream_t s)
{
    switch (ec_mode) {
    case 0:
        return launch_decode_t<0>(a, s);
    case 1:
        return launch_decode_t<1>(a, s);
    default:
        return launch_decode_t<2>(a, s);
    }
}

} // namespace spear
