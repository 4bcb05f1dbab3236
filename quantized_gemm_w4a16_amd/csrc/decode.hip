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
//  * a workgroup (4 waves) owns 16 output channels and one of `ksplit` slices
//    of K; each wave takes two 128-deep super-steps of that slice.  Packed
//    weights go straight from HBM to registers with 16-byte loads (no LDS) and
//    are unpacked to bf16 in registers; the contraction runs on bf16 MFMA with
//    the tokens (padded to 16) as the MFMA's N side.  A second MFMA against a
//    constant-one operand yields the per-token activation sums that remove the
//    unpack offset in the epilogue.
//  * K slices are reduced deterministically: the last workgroup of a channel
//    group (atomic counter) sums the partial tiles in slice order.
//  * EC (fused mode): the first `nprod` workgroups to start (atomic ticket, so
//    the election follows actual start order, never dispatch assumptions) also
//    compute the gate logit (fp64) and A.x over one K slice each; the
//    last producer to finish reduces them, applies the gate and hard-gate
//    selection (wave ballot), forms v = g (A x) split into bf16 hi + lo, and
//    publishes a flag.  The epilogues wait for that flag (bounded) and add
//    B v with two MFMAs per 32 ranks.  Producers never wait, so every wait ends.
//  * The last workgroup to finish returns the counters to zero.
#include "spear_internal.hpp"

namespace spear {

namespace {

struct DecShared {
    float red[DEC_WAVES][64][5];
    double z[16][17];
    float g[16];
    int act[16];
    uint32_t u32[4];
};

__device__ __forceinline__ uint32_t *hdr_of(const LinearArgs &a)
{
    return reinterpret_cast<uint32_t *>(a.ws + a.L.hdr);
}

// The last producer: gate, selection, v = g (A x) as bf16 hi + lo, then the flag.
__device__ void ec_finalize(const LinearArgs &a, DecShared &sh, int tid)
{
    const int lane = tid & 63, wave = tid >> 6;
    const double *prodz = reinterpret_cast<const double *>(a.ws + a.L.prodz);
    const float *produ = reinterpret_cast<const float *>(a.ws + a.L.produ);
    uint16_t *vhi = reinterpret_cast<uint16_t *>(a.ws + a.L.vhi);
    uint16_t *vlo = reinterpret_cast<uint16_t *>(a.ws + a.L.vlo);
    int32_t *active = reinterpret_cast<int32_t *>(a.ws + a.L.active);
    const int rpad = a.rpad;

    if (wave == 0) {
        int act = 0;
        if (lane < 16) {
            double z = (double)a.b;
            for (int64_t p = 0; p < a.nprod; p++)
                z += prodz[p * 16 + lane];
            const float g = (float)(1.0 / (1.0 + exp(-z)));
            act = (lane < a.M) && (a.hard ? (z > a.thr) : 1);
            sh.g[lane] = g;
            sh.act[lane] = act;
            active[lane] = act;
            if (lane < a.M && a.g_out)
                a.g_out[lane] = g;
        }
        const uint64_t mask = __ballot(act);
        if (act && a.idx_out)
            a.idx_out[__popcll(mask & ((1ull << lane) - 1ull))] = lane;
        if (lane == 0 && a.nact_out)
            *a.nact_out = __popcll(mask);
    }
    __syncthreads();
    for (int e = tid; e < 16 * rpad; e += 256) {
        const int m = e / rpad, j = e - m * rpad;
        float u = 0.f;
        for (int64_t p = 0; p < a.nprod; p++)
            u += produ[(p * 16 + m) * rpad + j];
        const float v = sh.act[m] ? sh.g[m] * u : 0.f;
        const uint16_t hi = f2bf(v);
        vhi[e] = hi;
        vlo[e] = f2bf(v - bf16f(hi));
    }
    __threadfence();
    __syncthreads();
    if (tid == 0)
        atomic_store_release(&hdr_of(a)[HDR_FLAG], 1u);
}

// EC producer for K slice p: partial A.x (fp32, MFMA) and partial gate logit (fp64).
__device__ void ec_produce(const LinearArgs &a, DecShared &sh, uint32_t p, int tid)
{
    const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const int64_t K = a.K, M = a.M;
    const int64_t k0 = (int64_t)p * a.prod_k;
    const int64_t k1 = (k0 + a.prod_k < K) ? k0 + a.prod_k : K;
    float *produ = reinterpret_cast<float *>(a.ws + a.L.produ);
    double *prodz = reinterpret_cast<double *>(a.ws + a.L.prodz);
    const int rpad = a.rpad, r = a.r;

    for (int jf = wave; jf < rpad / 16; jf += DEC_WAVES) {
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
        const int j = 16 * jf + lr;
        for (int64_t k = k0 + 8 * lg; k < k1; k += 32) {
            const u32x4 af = (j < r) ? ld16(a.A + (int64_t)j * K + k) : zero4();
            const u32x4 xf = (lr < M) ? ld16(a.x + (int64_t)lr * K + k) : zero4();
            u = mfma16(af, xf, u);
        }
        // lane holds u[rank 16 jf + 4 lg + i][token lr]
        *reinterpret_cast<f32x4 *>(produ + ((int64_t)p * 16 + lr) * rpad + 16 * jf + 4 * lg) = u;
    }

    {
        const int m = tid & 15, q = tid >> 4;
        double zp = 0.0;
        for (int64_t k = k0 + 16 * q; m < M && k < k1; k += 256) {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const u32x4 xv = ld16(a.x + (int64_t)m * K + k + 8 * h);
                const u32x4 wv = ld16(a.wg + k + 8 * h);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    zp += (double)(__uint_as_float(xv[e] << 16) * __uint_as_float(wv[e] << 16));
                    zp += (double)(__uint_as_float(xv[e] & 0xFFFF0000u) *
                                   __uint_as_float(wv[e] & 0xFFFF0000u));
                }
            }
        }
        sh.z[m][q] = zp;
    }
    __syncthreads();
    if (tid < 16) {
        double t = 0.0;
        for (int q = 0; q < 16; q++)
            t += sh.z[tid][q];
        prodz[(int64_t)p * 16 + tid] = t;
    }
    __threadfence();
    __syncthreads();
    if (tid == 0)
        sh.u32[2] = atomic_add_acqrel(&hdr_of(a)[HDR_PROD_DONE], 1u);
    __syncthreads();
    if (sh.u32[2] == (uint32_t)(a.nprod - 1)) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        ec_finalize(a, sh, tid);
    }
}

template <int EC_MODE, int OUT_F32>
__global__ __launch_bounds__(256) void decode_kernel(const LinearArgs a)
{
    __shared__ DecShared sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t ksplit = a.ksplit;
    const int64_t cg = blockIdx.x / ksplit, ks = blockIdx.x - cg * ksplit;
    const int64_t n0 = cg * 16;
    const int64_t K = a.K, N = a.N, M = a.M;
    const int64_t S = (K + 127) / 128;
    uint32_t *hdr = hdr_of(a);

    if (EC_MODE == 1 && tid == 0)
        sh.u32[0] = atomicAdd(&hdr[HDR_TICKET], 1u);

    // Weight stream and activations for this wave's super-steps, all in flight.
    u32x4 wr[DEC_SW], xr[DEC_SW][4];
    const int64_t n = n0 + lr;
#pragma unroll
    for (int i = 0; i < DEC_SW; i++) {
        const int64_t s = ks * DEC_SPW + wave * DEC_SW + i;
        const int64_t k = s * 128 + 32 * lg;
        const bool kv = (s < S) && (k < K);
        wr[i] = (kv && n < N) ? ld16(a.packed + n * (K / 2) + k / 2) : zero4();
#pragma unroll
        for (int c = 0; c < 4; c++)
            xr[i][c] = (kv && lr < M) ? ld16(a.x + (int64_t)lr * K + k + 8 * c) : zero4();
    }

    if (EC_MODE == 1) {
        __syncthreads();
        const uint32_t ticket = sh.u32[0];
        if (ticket < (uint32_t)a.nprod)
            ec_produce(a, sh, ticket, tid);
    }

    // Contraction: rows = 16 channels, columns = 16 token slots.
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, rs = {0.f, 0.f, 0.f, 0.f};
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
    for (int i = 0; i < DEC_SW; i++) {
#pragma unroll
        for (int d = 0; d < 4; d++) {
            const u32x4 xb = perm8(xr[i][d]);
            acc = mfma16(unpack8(wr[i][d]), xb, acc);
            rs = mfma16(ones, xb, rs);
        }
    }

    // Reduce the 4 waves (fixed order).
#pragma unroll
    for (int i = 0; i < 4; i++)
        sh.red[wave][lane][i] = acc[i];
    sh.red[wave][lane][4] = rs[0];
    __syncthreads();
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

    // Reduce the K slices: the last workgroup of the channel group sums them in order.
    bool epi = true;
    if (ksplit > 1) {
        float *splitp = reinterpret_cast<float *>(a.ws + a.L.splitp);
        uint32_t *colcnt = reinterpret_cast<uint32_t *>(a.ws + a.L.colcnt);
        if (wave == 0 && lr < M) {
            float *pp = splitp + ((cg * ksplit + ks) * 64 + lane) * 5;
#pragma unroll
            for (int i = 0; i < 4; i++)
                pp[i] = tot[i];
            pp[4] = rst;
        }
        if (wave == 0)
            __threadfence();
        __syncthreads();
        if (tid == 0)
            sh.u32[1] = atomic_add_acqrel(&colcnt[cg], 1u);
        __syncthreads();
        epi = sh.u32[1] == (uint32_t)(ksplit - 1);
        if (epi && wave == 0) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
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

    if (epi && wave == 0) {
        float yv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t nn = n0 + 4 * lg + i;
            yv[i] = 0.f;
            if (nn < N) {
                const float zc = 128.f + (a.zeros ? (float)a.zeros[nn] : 8.f);
                yv[i] = a.scales[nn] * __builtin_fmaf(-zc, rst, tot[i]);
            }
        }
        if (EC_MODE != 0) {
            bool ok = true;
            if (EC_MODE == 1) {
                uint32_t f = 0;
                if (lane == 0) {
                    uint32_t it = 0;
                    while ((f = atomic_load_acquire(&hdr[HDR_FLAG])) == 0u) {
                        if (++it > a.wait_limit) {
                            atomicAdd(&hdr[HDR_TIMEOUTS], 1u);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                }
                f = __shfl(f, 0);
                ok = f != 0u;
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            if (ok) {
                const int32_t *active = reinterpret_cast<const int32_t *>(a.ws + a.L.active);
                const uint16_t *vhi = reinterpret_cast<const uint16_t *>(a.ws + a.L.vhi);
                const uint16_t *vlo = reinterpret_cast<const uint16_t *>(a.ws + a.L.vlo);
                const int act = (lr < M) ? active[lr] : 0;
                if (__ballot(act) != 0ull) {
                    f32x4 e = {0.f, 0.f, 0.f, 0.f};
                    const int rpad = a.rpad, r = a.r;
                    for (int t = 0; t < rpad / 32; t++) {
                        const int j = 32 * t + 8 * lg;
                        const u32x4 bf = (n < N && j < r) ? ld16(a.B + n * r + j) : zero4();
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

    if (EC_MODE == 1) {
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = atomic_add_acqrel(&hdr[HDR_DONE], 1u);
            if (old == gridDim.x - 1) {
                atomic_store_relaxed(&hdr[HDR_TICKET], 0u);
                atomic_store_relaxed(&hdr[HDR_PROD_DONE], 0u);
                atomic_store_relaxed(&hdr[HDR_FLAG], 0u);
                atomic_store_relaxed(&hdr[HDR_DONE], 0u);
            }
        }
    }
}

template <int EC_MODE>
hipError_t launch_decode_t(const LinearArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)(a.ncg * a.ksplit));
    if (a.out_f32)
        hipLaunchKernelGGL((decode_kernel<EC_MODE, 1>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((decode_kernel<EC_MODE, 0>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
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
