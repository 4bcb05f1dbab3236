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
//    activations of the range would not fit in LDS).  Its 4 stream waves load
//    the activations of the range straight into LDS (global_load_lds), then
//    issue every 16-byte load of their packed-weight share (HBM -> registers),
//    wait once, and contract on bf16 MFMA (activations permuted to the unpack
//    order as they leave LDS) with the tokens (padded to 16) as the MFMA's N
//    side.  A second MFMA against a
//    constant-one operand gives the per-token activation sums that remove the
//    unpack offset in the epilogue.
//  * When K is split over workgroups, the last one of a channel group (atomic
//    counter) sums the partial tiles in slice order (deterministic).
//  * EC (fused mode): every workgroup has a fifth wave.  The first `nprod`
//    of these to start (atomic ticket: the election follows actual start
//    order) each compute the gate logit (fp64) and A.x (MFMA) of all tokens
//    over one K slice, publish them (release) and count themselves done.  The
//    epilogue wave of each channel group polls that count (plain coherent
//    loads, bounded), takes one acquire fence, reduces the slices in slice
//    order, applies the gate and the hard-gate selection, forms v = g (A x) as
//    bf16 hi + lo and adds B v with two MFMAs per 32 ranks.  Every epilogue
//    computes the same v in the same order.  Producers never wait, so every
//    wait ends.
//  * The last wave to finish returns the counters to zero.
#include "spear_internal.hpp"

namespace spear {

namespace {

constexpr int DEC_THREADS = 64 * DEC_WAVES;               // stream waves
constexpr int PS = PROD_K / 32;                           // 32-deep steps of a producer chunk

struct DecShared {
    float red[DEC_WAVES][64][5];
    uint32_t u32[4];
};

__device__ __forceinline__ uint32_t *hdr_of(const LinearArgs &a)
{
    return reinterpret_cast<uint32_t *>(a.ws + a.L.hdr);
}

__device__ __forceinline__ void release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

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

// Producer wave for K slice p: partial gate logits z[m] (fp64) and partial
// u[m][j] = sum_k A[j][k] x[m][k] (fp32) over the slice, for all 16 token slots.
__device__ void ec_produce_wave(const LinearArgs &a, uint32_t p, int lane)
{
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t K = a.K, M = a.M;
    const int64_t k0 = (int64_t)p * a.prod_k;
    const int64_t k1 = (k0 + a.prod_k < K) ? k0 + a.prod_k : K;
    float *produ = reinterpret_cast<float *>(a.ws + a.L.produ);
    double *prodz = reinterpret_cast<double *>(a.ws + a.L.prodz);
    const int rpad = a.rpad, r = a.r;

    double zp = 0.0;
    for (int jp = 0; jp < rpad / 32; jp++) {
        f32x4 u0 = {0.f, 0.f, 0.f, 0.f}, u1 = {0.f, 0.f, 0.f, 0.f};
        const int j0 = 32 * jp + lr, j1 = j0 + 16;
        for (int64_t kc = k0; kc < k1; kc += PROD_K) {
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
        float *dst = produ + ((int64_t)p * 16 + lr) * rpad + 32 * jp + 4 * lg;
        *reinterpret_cast<f32x4 *>(dst) = u0;
        *reinterpret_cast<f32x4 *>(dst + 16) = u1;
    }
    // z for token lr: the four lane groups in order
    const double z1 = __shfl(zp, lr + 16), z2 = __shfl(zp, lr + 32), z3 = __shfl(zp, lr + 48);
    if (lg == 0)
        prodz[(int64_t)p * 16 + lr] = ((zp + z1) + z2) + z3;
    release_agent();
    if (lane == 0)
        __hip_atomic_fetch_add(&hdr_of(a)[HDR_PROD_DONE], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

// Epilogue EC term (fused mode), wave 0 of the finishing workgroup: returns
// e[i] for channel n0 + 4 lg + i and token lr, and writes the gate outputs
// when this is channel group 0.
__device__ f32x4 ec_epilogue_fused(const LinearArgs &a, const u32x4 *bpre, int64_t cg, int lane,
                                   bool *ok_out)
{
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t M = a.M, N = a.N;
    const int64_t n = cg * 16 + lr;
    uint32_t *hdr = hdr_of(a);
    f32x4 e = {0.f, 0.f, 0.f, 0.f};

    uint32_t f = 0;
    if (lane == 0) {
        uint32_t it = 0;
        while ((f = __hip_atomic_load(&hdr[HDR_PROD_DONE], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT)) < (uint32_t)a.nprod) {
            if (++it > a.wait_limit) {
                atomicAdd(&hdr[HDR_TIMEOUTS], 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    f = __shfl(f, 0);
    *ok_out = f >= (uint32_t)a.nprod;
    if (!*ok_out)
        return e;
    acquire_agent();

    const double *prodz = reinterpret_cast<const double *>(a.ws + a.L.prodz);
    const float *produ = reinterpret_cast<const float *>(a.ws + a.L.produ);
    const int64_t np = a.nprod;
    const int rpad = a.rpad, r = a.r;

    // Gate of token lr: slices summed in order.
    double z = (double)a.b;
    for (int64_t p0 = 0; p0 < np; p0 += 16) {
        double zz[16];
#pragma unroll
        for (int i = 0; i < 16; i++)
            zz[i] = (p0 + i < np) ? prodz[(p0 + i) * 16 + lr] : 0.0;
#pragma unroll
        for (int i = 0; i < 16; i++)
            if (p0 + i < np)
                z += zz[i];
    }
    const float g = (float)(1.0 / (1.0 + exp(-z)));
    const int act = (lr < M) && (a.hard ? (z > a.thr) : 1);

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
    if (__ballot(act) == 0ull)
        return e;

    for (int t = 0; t < rpad / 32; t++) {
        const int j = 32 * t + 8 * lg;
        // u[lr][j .. j+7], slices in order
        f32x4 ua = {0.f, 0.f, 0.f, 0.f}, ub = {0.f, 0.f, 0.f, 0.f};
        for (int64_t p0 = 0; p0 < np; p0 += 8) {
            f32x4 va[8], vb[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float *src = produ + ((p0 + i) * 16 + lr) * rpad + j;
                const bool pv = p0 + i < np;
                va[i] = pv ? *reinterpret_cast<const f32x4 *>(src) : f32x4{0.f, 0.f, 0.f, 0.f};
                vb[i] = pv ? *reinterpret_cast<const f32x4 *>(src + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int i = 0; i < 8; i++) {
                if (p0 + i < np) {
                    ua += va[i];
                    ub += vb[i];
                }
            }
        }
        u32x4 vh, vl;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float v0 = act ? g * (q < 2 ? ua[2 * q] : ub[2 * q - 4]) : 0.f;
            const float v1 = act ? g * (q < 2 ? ua[2 * q + 1] : ub[2 * q - 3]) : 0.f;
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
    return e;
}

template <int EC_MODE, int OUT_F32, int SW>
__global__ __launch_bounds__(64 * DEC_WAVES) void decode_kernel(const LinearArgs a)
{
    __shared__ DecShared sh;
    extern __shared__ __attribute__((aligned(16))) uint8_t s_x[];
    pin_args(a);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    uint32_t *hdr = hdr_of(a);

    // EC producers (fused mode) are the lowest block indices, which start first:
    // each of their waves computes the partials of one K slice, then they leave.
    int64_t bid = blockIdx.x;
    if (EC_MODE == 1) {
        const int64_t npwg = (a.nprod + DEC_WAVES - 1) / DEC_WAVES;
        if (bid < npwg) {
            const int64_t p = bid * DEC_WAVES + wave;
            if (p < a.nprod)
                ec_produce_wave(a, (uint32_t)p, lane);
            __syncthreads();
            if (tid == 0) {
                const uint32_t old = __hip_atomic_fetch_add(&hdr[HDR_DONE], 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                if (old == gridDim.x - 1) {
                    atomic_store_relaxed(&hdr[HDR_PROD_DONE], 0u);
                    atomic_store_relaxed(&hdr[HDR_DONE], 0u);
                }
            }
            return;
        }
        bid -= npwg;
    }
    const bool stream = true;
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

    // 3. Activations of the K range -> LDS directly (global_load_lds, 16 bytes a
    //    lane, 64 consecutive chunks of one token row per wave instruction).
    //    Chunks past K and the extra row M (read by token slots >= M) are zeros.
    if (stream) {
        const int64_t npass = (cpr + DEC_THREADS - 1) / DEC_THREADS;
        for (int64_t m = 0; m < M; m++) {
            for (int64_t ps = 0; ps < npass; ps++) {
                const int64_t q0 = ps * DEC_THREADS + wave * 64;      // first chunk of this wave
                const int64_t q = q0 + lane;
                const int64_t k = s_begin * 128 + 8 * q;
                if (q0 < cpr && q < cpr && k < K)
                    __builtin_amdgcn_global_load_lds(
                        (const __attribute__((address_space(1))) void *)(a.x + m * K + k),
                        (__attribute__((address_space(3))) void *)(s_x + m * rs_bytes + 16 * q0),
                        16, 0, 0);
                else if (q < cpr)
                    *reinterpret_cast<u32x4 *>(s_x + m * rs_bytes + 16 * q) = zero4();
            }
        }
        for (int64_t q = tid; q < cpr; q += DEC_THREADS)
            *reinterpret_cast<u32x4 *>(s_x + M * rs_bytes + 16 * q) = zero4();
    }

    // 4. The weight stream of this wave: SW loads, all in flight at once.  Out of
    //    range rows and depths read clamped in-bounds addresses; their products
    //    meet zero activations or are never stored.
    u32x4 wr[SW];
    const int sl0 = wave * SW;                               // first local super-step
#pragma unroll
    for (int i = 0; i < SW; i++) {
        int64_t k = (s_begin + sl0 + i) * 128 + 32 * lg;
        k = k < K ? k : K - 32;
        wr[i] = ld16(a.packed + nc * (K / 2) + k / 2);
    }

    // Wait for everything but the weight stream (the SW youngest loads) and for
    // the LDS zero fills, then make the activations visible to the workgroup.
    // The weight loads stay in flight; each super-step waits for its own.
    wait_vmcnt<SW>();
    wait_lgkmcnt0();
    bare_barrier();

    // 5. Permute the activations in place to the unpack pair order, once.
    for (int64_t m = 0; m < M; m++) {
        for (int64_t q = tid; q < cpr; q += DEC_THREADS) {
            u32x4 *p = reinterpret_cast<u32x4 *>(s_x + m * rs_bytes + 16 * q);
            *p = perm8(*p);
        }
    }
    wait_lgkmcnt0();
    bare_barrier();

    // 6. Contraction (stream waves), each super-step as soon as its weights land.
    if (stream) {
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
    __syncthreads();

    // 7. Reduce the stream waves (fixed order).
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    float rst = 0.f;
    if (wave == 0) {
        for (int w = 0; w < DEC_WAVES; w++) {
#pragma unroll
            for (int i = 0; i < 4; i++)
                tot[i] += sh.red[w][lane][i];
            rst += sh.red[w][lane][4];
        }
    }

    // 8. Reduce the K ranges: the last workgroup of the channel group sums them in order.
    bool epi = true;
    if (ksplit > 1) {
        float *splitp = reinterpret_cast<float *>(a.ws + a.L.splitp);
        uint32_t *colcnt = reinterpret_cast<uint32_t *>(a.ws + a.L.colcnt);
        if (wave == 0) {
            if (lr < M) {
                float *pp = splitp + ((cg * ksplit + ks) * 64 + lane) * 5;
#pragma unroll
                for (int i = 0; i < 4; i++)
                    pp[i] = tot[i];
                pp[4] = rst;
            }
            release_agent();
            if (lane == 0)
                sh.u32[1] = __hip_atomic_fetch_add(&colcnt[cg], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        epi = sh.u32[1] == (uint32_t)(ksplit - 1);
        if (epi && wave == 0) {
            acquire_agent();
            if (lane == 0)
                atomic_store_relaxed(&colcnt[cg], 0u);
            tot = f32x4{0.f, 0.f, 0.f, 0.f};
            rst = 0.f;
            if (lr < M) {
                for (int64_t q = 0; q < ksplit; q++) {
                    const float *pp = splitp + ((cg * ksplit + q) * 64 + lane) * 5;
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        tot[i] += pp[i];
                    rst += pp[4];
                }
            }
        }
    }

    // 9. Epilogue (wave 0): scale, offset removal, EC, store.
    if (epi && wave == 0) {
        float yv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t nn = n0 + 4 * lg + i;
            const float zc = UNPACK_OFF + zero_point(a.zeros, z_raw[i]);
            yv[i] = nn < N ? sc_raw[i] * __builtin_fmaf(-zc, rst, UNPACK_SCALE * tot[i]) : 0.f;
        }
        if (EC_MODE == 1) {
            bool ok;
            const f32x4 e = ec_epilogue_fused(a, bpre, cg, lane, &ok);
#pragma unroll
            for (int i = 0; i < 4; i++)
                yv[i] += e[i];
        } else if (EC_MODE == 2) {
            // v precomputed by the pre-pass (bf16 hi + lo, zero for skipped tokens)
            const int32_t *active = reinterpret_cast<const int32_t *>(a.ws + a.L.active);
            const uint16_t *vhi = reinterpret_cast<const uint16_t *>(a.ws + a.L.vhi);
            const uint16_t *vlo = reinterpret_cast<const uint16_t *>(a.ws + a.L.vlo);
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

    // 10. Completion count (fused mode): the last workgroup restores the counters.
    //     Every counter access of this workgroup precedes this point (producers
    //     count themselves done before they leave; the epilogue polls above).
    if (EC_MODE == 1 && tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&hdr[HDR_DONE], 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (old == gridDim.x - 1) {
            atomic_store_relaxed(&hdr[HDR_PROD_DONE], 0u);
            atomic_store_relaxed(&hdr[HDR_DONE], 0u);
        }
    }
}

// Dynamic LDS beyond 64 KiB must be enabled per kernel once.
template <int EC_MODE, int OUT_F32, int SW>
hipError_t launch_decode_k(const LinearArgs &a, hipStream_t s)
{
    static const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_kernel<EC_MODE, OUT_F32, SW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, DEC_LDS_MAX);
    if (e != hipSuccess)
        return e;
    const int64_t npwg = EC_MODE == 1 ? (a.nprod + DEC_WAVES - 1) / DEC_WAVES : 0;
    const dim3 grid((unsigned)(npwg + a.ncg * a.ksplit));
    const dim3 block(64 * DEC_WAVES);
    const size_t lds = (size_t)(a.M + 1) * (size_t)(a.spw * 256 + 16);
    hipLaunchKernelGGL((decode_kernel<EC_MODE, OUT_F32, SW>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int EC_MODE, int OUT_F32>
hipError_t launch_decode_sw(const LinearArgs &a, hipStream_t s)
{
    switch ((a.spw + DEC_WAVES - 1) / DEC_WAVES) {
    case 1: return launch_decode_k<EC_MODE, OUT_F32, 1>(a, s);
    case 2: return launch_decode_k<EC_MODE, OUT_F32, 2>(a, s);
    case 3: return launch_decode_k<EC_MODE, OUT_F32, 3>(a, s);
    case 4: return launch_decode_k<EC_MODE, OUT_F32, 4>(a, s);
    case 5: return launch_decode_k<EC_MODE, OUT_F32, 5>(a, s);
    case 6: return launch_decode_k<EC_MODE, OUT_F32, 6>(a, s);
    case 7: return launch_decode_k<EC_MODE, OUT_F32, 7>(a, s);
    default: return launch_decode_k<EC_MODE, OUT_F32, 8>(a, s);
    }
}

template <int EC_MODE>
hipError_t launch_decode_t(const LinearArgs &a, hipStream_t s)
{
    return a.out_f32 ? launch_decode_sw<EC_MODE, 1>(a, s) : launch_decode_sw<EC_MODE, 0>(a, s);
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
