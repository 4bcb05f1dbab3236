// prefill.hip -- prefill-sized W4A16 linear: the EC pre-pass and the MFMA GEMM
// whose epilogue applies the gated error compensator (gfx950).
//
// Source: "SPEAR: A System for Post-Quantization Error-Adaptive Recovery
// Enabling Efficient Low-Bit LLM Serving", gist.science summary section 2.2 A:
// at prefill the layer is compute bound and the EC runs semi-fused -- here the
// gate and the EC down-projection run in a short pre-pass and the
// up-projection is folded into the GEMM epilogue.  The EC follows section
// 2.1 A with the scalar gate g = sigmoid(b + x.w_g).
#include "spear_internal.hpp"

namespace spear {

namespace {

// --------------------------------------------------------------------- pre-pass
// Per token: gate logit in fp64, g, hard-gate flag, u = A x (fp32 via MFMA,
// natural depth order on both operands), v = g u (0 for skipped tokens) stored
// as bf16 hi + lo.  Workgroup (group, slice): 16 tokens over one of pre_ks K
// slices; its PW waves split the slice (wave w takes part (w + block) % PW, so
// workgroups side by side read different parts of A).  A wave walks its part
// in chunks of PRE_T 32-deep steps and, per chunk, issues every load (x, up to
// PRE_RT 16-rank tiles of A, w_g) before it uses any, so one memory round trip
// covers the chunk.  With one slice the workgroup finishes the tokens itself.
// With several, every workgroup but the group's last slice stores its partials
// as tagged words {value, launch epoch} (relaxed device-coherent stores), and
// the last slice -- the group's highest block index, dispatched after the
// others, which never wait -- re-loads the other slices' words until every tag
// is this launch's (bounded; an expired wait is counted and makes the group's
// v, g and selection flags NaN / -1, so that its outputs come out NaN), adds
// the slices in order and finishes the tokens.  Each word is
// validated on its own, so no fence or counter is involved (a release fence
// per workgroup would write back the whole L2).
//
// The pre-pass runs either as its own launch (8 waves a workgroup; v goes to
// plain bf16 arrays that the GEMM launch reads) or as the first blocks of the
// K-split GEMM's launch (the GEMM's 4 or 8 waves a workgroup; v goes out as
// tagged words {hi | lo << 16, epoch} that the GEMM epilogues wait for).
constexpr int PRE_WAVES = 8;                   // waves of the stand-alone launch
constexpr int PRE_T = 8;                       // 32-deep steps per chunk
constexpr int PRE_RT = 4;                      // 16-rank tiles per pass over the slice
constexpr int PRE_TILES = SPEAR_MAX_RANK / 16;
constexpr int PRE_FE = 2;                      // finisher: u elements a thread adds up per batch
constexpr int PRE_FQ = 8;                      // finisher: slices per batch (loads in flight)
constexpr int CMB_U = 16;                      // split-K reduction: slice loads in flight

// The pre-pass's LDS (arrays of PW waves), wherever the launch keeps it.
template <int PW>
struct PreShared {
    f32x4 (*u)[PRE_RT][64];   // [PW / 2 or PW]: each wave's u tiles of the current pass ...
    f32x4 (*u_hi)[PRE_RT][64];  // ... and those of waves PW / 2 and up (may follow u)
    double (*z)[64];          // [PW]: each wave's logit partials
    u32x4 (*wg)[4 * PRE_T];   // [PW]: each wave's w_g of its chunk
    f32x4 (*uw)[64];          // [PRE_TILES]: the workgroup's u
    double *zw;               // [16]: the workgroup's logit sums
    float *g;                 // [16]
    int *act;                 // [16]
    uint32_t *tag, *bad;
    float *hid;               // [16][SPEAR_MAX_GATE_HIDDEN]: vector gate's hidden layer
};

// Vector gate of tokens m0 .. m0 + 15 (summary section 2.1 A: a bottleneck MLP
// on the rank-r projection): hid[m][i] = relu(c1[i] + sum_l W1[i][l] u_m[l])
// for every token slot, by all threads of the workgroup (nthreads); u_m[l] is
// read from the pre-pass layout (tile l / 16, lane 16 ((l % 16) / 4) + m,
// element l % 4).  The caller synchronises before reading hid.
__device__ void vgate_hidden(const LinearArgs &a, const f32x4 (*s_uw)[64], float *hid, int tid,
                             int nthreads)
{
    const int h = a.gate_h, r = a.r;
    for (int q = tid; q < 16 * h; q += nthreads) {
        const int m = q & 15, i = q >> 4;
        float s = a.gc1[i];
        const float *w1 = a.gw1 + (int64_t)i * r;
        for (int l = 0; l < r; l++)
            s = __builtin_fmaf(w1[l], s_uw[l >> 4][16 * ((l & 15) >> 2) + m][l & 3], s);
        hid[m * SPEAR_MAX_GATE_HIDDEN + i] = s > 0.f ? s : 0.f;
    }
}

// gamma_j of token slot m from its hidden layer: sigmoid(c2[j] + sum_i W2[j][i] hid[m][i]).
__device__ __forceinline__ float vgate_gamma(const LinearArgs &a, const float *hid, int m, int j)
{
    const int h = a.gate_h;
    float s = a.gc2[j];
    const float *w2 = a.gw2 + (int64_t)j * h;
    for (int i = 0; i < h; i++)
        s = __builtin_fmaf(w2[i], hid[m * SPEAR_MAX_GATE_HIDDEN + i], s);
    return 1.f / (1.f + __expf(-s));
}

// The last step of the pre-pass for tokens m0 .. m0 + 15, given their logit
// sums (without b) in s_zw and u in s_uw (tile t, lane l: ranks 16 t + 4 (l / 16)
// + i of token l % 16): gate, selection, v = g u as bf16 hi + lo.  Called by
// every thread of the workgroup; waves below nwaves write v (as tagged words
// when tagged).  bad (an expired wait upstream): the group's sums are
// incomplete, so g and v are NaN and each real token's selection flag is -1.
__device__ void prepass_finish(const LinearArgs &a, int64_t m0, const f32x4 (*s_uw)[64],
                               const double *s_zw, float *s_g, int *s_act, float *s_hid, int tid,
                               int lane, int wave, int nwaves, bool tagged, uint32_t tag, bool bad)
{
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t M = a.M, m = m0 + lr;
    const int rpad = a.rpad;
    uint16_t *vhi = reinterpret_cast<uint16_t *>(a.ws + a.P.vhi);
    uint16_t *vlo = reinterpret_cast<uint16_t *>(a.ws + a.P.vlo);
    uint64_t *vtag = reinterpret_cast<uint64_t *>(a.ws + a.P.vtag);
    int32_t *active = reinterpret_cast<int32_t *>(a.ws + a.P.active);
    if (tid < 16) {
        const double z = (double)a.b + s_zw[tid];
        const int64_t mm = m0 + tid;
        const float g = bad ? __builtin_nanf("") : (float)(1.0 / (1.0 + exp(-z)));
        const int act = bad ? (mm < M ? -1 : 0) : (mm < M) && (a.hard ? (z > a.thr) : 1);
        s_g[tid] = g;
        s_act[tid] = act;
        active[mm] = act;
        if (mm < M && a.g_out)
            a.g_out[mm] = g;
    }
    const bool vg = a.gate_h > 0;
    if (vg)
        vgate_hidden(a, s_uw, s_hid, tid, 64 * nwaves);
    __syncthreads();
    // rows m >= M (up to the 16-row padding) get v = 0
    const float g = s_act[lr] ? (vg ? s_g[lr] * a.alpha : s_g[lr]) : 0.f;
    for (int tile = wave; wave < nwaves && tile < rpad / 16; tile += nwaves) {
        const f32x4 u = s_uw[tile][lane];
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int j = 16 * tile + 4 * lg + i;
            const float gam = (vg && j < a.r) ? vgate_gamma(a, s_hid, lr, j) : 1.f;
            const float v = g * (gam * u[i]);
            hi[i] = f2bf(v);
            lo[i] = f2bf(v - bf16f(hi[i]));
        }
        const int64_t off = m * rpad + 16 * tile + 4 * lg;
        if (tagged) {
#pragma unroll
            for (int i = 0; i < 4; i++)
                store_tagged(vtag + off + i, (uint32_t)hi[i] | ((uint32_t)lo[i] << 16), tag);
        } else {
            uint2 h, l;
            h.x = (uint32_t)hi[0] | ((uint32_t)hi[1] << 16);
            h.y = (uint32_t)hi[2] | ((uint32_t)hi[3] << 16);
            l.x = (uint32_t)lo[0] | ((uint32_t)lo[1] << 16);
            l.y = (uint32_t)lo[2] | ((uint32_t)lo[3] << 16);
            *reinterpret_cast<uint2 *>(vhi + off) = h;
            *reinterpret_cast<uint2 *>(vlo + off) = l;
        }
    }
}

template <int PW>
__device__ __forceinline__ void prepass_tail(const LinearArgs &a, int64_t grp, int64_t ks,
                                             const PreShared<PW> &sh, uint64_t claimed, bool tagged);

// One pre-pass workgroup (block bid of the pre-pass grid, PW waves).  claimed
// is thread 0's epoch claim; the launch claims in every block when the slices
// exchange words or v goes out tagged.
template <int PW>
__device__ __forceinline__ void prepass_body(const LinearArgs &a, const int64_t bid,
                                             const PreShared<PW> &sh, const uint64_t claimed,
                                             const bool tagged)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t M = a.M, K = a.K, KS = a.pre_ks;
    const int64_t grp = bid / KS, ks = bid % KS;
    const int64_t m0 = grp * 16;
    const int64_t T = K / 32, s0 = ks * T / KS, s1 = (ks + 1) * T / KS;
    const int64_t part = (wave + bid) % PW;
    const int64_t t0 = s0 + part * (s1 - s0) / PW, t1 = s0 + (part + 1) * (s1 - s0) / PW;
    const int64_t m = m0 + lr;
    const bool mv = m < M;
    const int r = a.r, ntile = a.rpad / 16;

    for (int q0 = 0; q0 < ntile; q0 += PRE_RT) {
        f32x4 acc[PRE_RT];
#pragma unroll
        for (int q = 0; q < PRE_RT; q++)
            acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        double zp = 0.0;
        for (int64_t tc = t0; tc < t1; tc += PRE_T) {
            const int n = (int)(t1 - tc < PRE_T ? t1 - tc : PRE_T);   // wave-uniform
            u32x4 xf[PRE_T], av[PRE_T][PRE_RT];
#pragma unroll
            for (int i = 0; i < PRE_T; i++) {
                const int64_t k = 32 * (tc + i) + 8 * lg;
                xf[i] = (i < n && mv) ? ld16(a.x + m * K + k) : zero4();
#pragma unroll
                for (int q = 0; q < PRE_RT; q++) {
                    const int j = 16 * (q0 + q) + lr;
                    av[i][q] = (i < n && j < r) ? ld16(a.A + (int64_t)j * K + k) : zero4();
                }
            }
            // lane 4 i + p holds w_g[32 (tc + i) + 8 p .. + 7]
            const u32x4 wq = (q0 == 0 && lane < 4 * n) ? ld16(a.wg + 32 * tc + 8 * lane) : zero4();
            if (q0 == 0 && lane < 4 * PRE_T)
                sh.wg[wave][lane] = wq;
#pragma unroll
            for (int i = 0; i < PRE_T; i++) {
                if (i < n) {
#pragma unroll
                    for (int q = 0; q < PRE_RT; q++)
                        if (q0 + q < ntile)
                            acc[q] = mfma16(av[i][q], xf[i], acc[q]);
                    if (q0 == 0) {
                        const u32x4 w = sh.wg[wave][4 * i + lg];
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            zp += (double)(__uint_as_float(xf[i][e] << 16) *
                                           __uint_as_float(w[e] << 16));
                            zp += (double)(__uint_as_float(xf[i][e] & 0xFFFF0000u) *
                                           __uint_as_float(w[e] & 0xFFFF0000u));
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int q = 0; q < PRE_RT; q++)
            (wave < PW / 2 ? sh.u[wave] : sh.u_hi[wave - PW / 2])[q][lane] = acc[q];
        if (q0 == 0)
            sh.z[wave][lane] = zp;
        __syncthreads();
        // the workgroup's partials: waves in order (then lane groups for z)
        if (wave < PRE_RT && q0 + wave < ntile) {
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
            for (int w = 0; w < PW; w++)
                u += (w < PW / 2 ? sh.u[w] : sh.u_hi[w - PW / 2])[wave][lane];
            sh.uw[q0 + wave][lane] = u;
        }
        if (q0 == 0 && wave == PRE_RT % PW && lane < 16) {
            double z = 0.0;
            for (int w = 0; w < PW; w++)
                for (int q = 0; q < 4; q++)
                    z += sh.z[w][lane + 16 * q];
            sh.zw[lane] = z;
        }
        __syncthreads();
    }
    prepass_tail<PW>(a, grp, ks, sh, claimed, tagged);
}

// The rest of a pre-pass workgroup once sh.uw and sh.zw hold its partials:
// with K split, the exchange of the slices' tagged partials (the group's last
// slice adds them); then gate, selection and v.
template <int PW>
__device__ __forceinline__ void prepass_tail(const LinearArgs &a, const int64_t grp, const int64_t ks,
                                             const PreShared<PW> &sh, const uint64_t claimed,
                                             const bool tagged)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t KS = a.pre_ks, m0 = grp * 16;
    const int ntile = a.rpad / 16;
    uint32_t tag = 0;
    bool bad = false;
    if (KS > 1 || tagged) {
        if (tid == 0) {
            *sh.tag = epoch_tag(claimed + opaque_zero64());
            *sh.bad = 0;
        }
        __syncthreads();
        tag = *sh.tag;
    }
    if (KS > 1) {
        // Tagged slice partials: [slot][tile][lane][4] words of u and [slot][token][2]
        // words of the fp64 logit, slot = group * pre_ks + slice.
        uint64_t *pu = reinterpret_cast<uint64_t *>(a.ws + a.P.preu);
        uint64_t *pz = reinterpret_cast<uint64_t *>(a.ws + a.P.prez);
        const int nel = ntile * 256;                      // u elements of a slot
        const float *uw = reinterpret_cast<const float *>(sh.uw);
        if (ks < KS - 1) {
            uint64_t *du = pu + (grp * KS + ks) * nel;
            for (int e = tid; e < nel; e += 64 * PW)
                store_tagged(du + e, __float_as_uint(uw[e]), tag);
            if (tid < 16) {
                const uint64_t zb = __builtin_bit_cast(uint64_t, sh.zw[tid]);
                store_tagged(pz + ((grp * KS + ks) * 16 + tid) * 2, (uint32_t)zb, tag);
                store_tagged(pz + ((grp * KS + ks) * 16 + tid) * 2 + 1, (uint32_t)(zb >> 32), tag);
            }
            return;
        }
        // The group's last slice: add the other slices' words, in slice order,
        // then its own partials.
        float *uwm = reinterpret_cast<float *>(sh.uw);
        bool ok = true;
        for (int e0 = 0; ok && e0 < nel; e0 += 64 * PW * PRE_FE) {
            float sum[PRE_FE];
#pragma unroll
            for (int f = 0; f < PRE_FE; f++)
                sum[f] = 0.f;
            for (int64_t q0 = 0; ok && q0 < KS - 1; q0 += PRE_FQ) {
                uint64_t w[PRE_FE][PRE_FQ];
                for (uint32_t it = 0;; it++) {
                    bool good = true;
#pragma unroll
                    for (int f = 0; f < PRE_FE; f++) {
                        const int e = e0 + tid + 64 * PW * f;
                        const int ec = e < nel ? e : nel - 1;
#pragma unroll
                        for (int q = 0; q < PRE_FQ; q++) {
                            const int64_t qq = q0 + q < KS - 1 ? q0 + q : KS - 2;
                            w[f][q] = load_tagged(pu + (grp * KS + qq) * nel + ec);
                        }
                    }
#pragma unroll
                    for (int f = 0; f < PRE_FE; f++)
#pragma unroll
                        for (int q = 0; q < PRE_FQ; q++)
                            good &= (uint32_t)(w[f][q] >> 32) == tag;
                    if (__all(good))
                        break;
                    if (it >= a.wait_limit) {
                        ok = false;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
#pragma unroll
                for (int f = 0; f < PRE_FE; f++)
#pragma unroll
                    for (int q = 0; q < PRE_FQ; q++)
                        if (q0 + q < KS - 1)
                            sum[f] += __uint_as_float((uint32_t)w[f][q]);
            }
#pragma unroll
            for (int f = 0; f < PRE_FE; f++) {
                const int e = e0 + tid + 64 * PW * f;
                if (e < nel)
                    uwm[e] = sum[f] + uwm[e];
            }
        }
        if (tid < 16) {
            // token tid's logit words of every other slice, PRE_FQ slices at a time
            double z = 0.0;
            for (int64_t q0 = 0; ok && q0 < KS - 1; q0 += PRE_FQ) {
                uint64_t w[PRE_FQ][2];
                for (uint32_t it = 0;; it++) {
                    bool good = true;
#pragma unroll
                    for (int q = 0; q < PRE_FQ; q++) {
                        const int64_t qq = q0 + q < KS - 1 ? q0 + q : KS - 2;
                        const uint64_t *src = pz + ((grp * KS + qq) * 16 + tid) * 2;
                        w[q][0] = load_tagged(src);
                        w[q][1] = load_tagged(src + 1);
                    }
#pragma unroll
                    for (int q = 0; q < PRE_FQ; q++)
                        good &= (uint32_t)(w[q][0] >> 32) == tag && (uint32_t)(w[q][1] >> 32) == tag;
                    if (__all(good))
                        break;
                    if (it >= a.wait_limit) {
                        ok = false;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
#pragma unroll
                for (int q = 0; q < PRE_FQ; q++)
                    if (q0 + q < KS - 1)
                        z += __builtin_bit_cast(double, (uint64_t)(uint32_t)w[q][0] |
                                                            ((uint64_t)(uint32_t)w[q][1] << 32));
            }
            sh.zw[tid] = z + sh.zw[tid];
        }
        if (!ok)
            atomicOr(sh.bad, 1u);
        __syncthreads();
        bad = *sh.bad != 0;
        if (bad && tid == 0)          // an expired wait: counted; the group's v is NaN
            atomicAdd(reinterpret_cast<uint32_t *>(a.ws + a.P.hdr) + HDR_TIMEOUTS, 1u);
    }
    prepass_finish(a, m0, sh.uw, sh.zw, sh.g, sh.act, sh.hid, tid, lane, wave, PW, tagged, tag,
                   bad);
}

__global__ __launch_bounds__(64 * PRE_WAVES) void prepass_kernel(const LinearArgs a)
{
    __shared__ f32x4 s_u[PRE_WAVES][PRE_RT][64];
    __shared__ double s_z[PRE_WAVES][64];
    __shared__ u32x4 s_wg[PRE_WAVES][4 * PRE_T];
    __shared__ f32x4 s_uw[PRE_TILES][64];
    __shared__ double s_zw[16];
    __shared__ float s_g[16];
    __shared__ int s_act[16];
    __shared__ uint32_t s_tag, s_bad;
    __shared__ float s_hid[16 * SPEAR_MAX_GATE_HIDDEN];
    pin_pre_args(a);
    uint64_t claimed = opaque_zero64();
    if (a.pre_ks > 1 && threadIdx.x == 0)
        claimed = epoch_claim(a, a.grid);              // back long before it is used
    const PreShared<PRE_WAVES> sh = {s_u, s_u + PRE_WAVES / 2, s_z, s_wg, s_uw, s_zw, s_g, s_act,
                                     &s_tag, &s_bad, s_hid};
    prepass_body<PRE_WAVES>(a, blockIdx.x, sh, claimed, false);
}

// The same pre-pass for ranks up to 64 with its operands staged through LDS.
// Loaded straight into MFMA operand registers, every 16-byte load of x or A
// touches 16 rows (64 bytes of each), which caps what one CU takes in; here
// the workgroup DMAs whole contiguous rows of a K chunk (512 deep at rank 32,
// 256 at rank 64) -- 16 token rows of x, then rpad rows of A (zero rows past
// r) -- into a ring of three stage buffers (global_load_lds, 1 KB per
// instruction, 16-byte row chunks XOR-swizzled by row % 16 so the operand
// reads below fall in distinct banks), with one barrier per chunk as in the
// GEMM.  Wave w takes the 32-deep steps w, w + 8, ... of each chunk; its w_g
// words come by plain loads issued one chunk ahead, just before the next
// chunk's DMAs, so one vmcnt wait covers both.  (Six stages of 256-deep
// chunks at rank 32 measured slower: the CU's intake, not the depth in
// flight, is the limit.)  The sums, the exchange of K slices and the finish
// are those of prepass_body.
template <int RPAD>
__global__ __launch_bounds__(512) void prepass2_kernel(const LinearArgs a)
{
    constexpr int CK = RPAD == 32 ? 512 : 256;           // depth of a chunk
    constexpr int SPW = CK / 256;                        // steps of a chunk a wave takes
    constexpr int RB = CK * 2;                           // bytes of a staged row
    constexpr int SB = (16 + RPAD) * RB;                 // bytes of a stage
    constexpr int NI = SB / (8 * 1024);                  // DMAs a wave issues per stage
    constexpr int NT = RPAD / 16;                        // rank tiles
    constexpr int RING = 3;
    constexpr int WAIT = (RING - 2) * NI + (RING - 3) * SPW;   // loads younger than a chunk's
    static_assert(NI * 8 * 1024 == SB && NT <= PRE_TILES && WAIT < 64, "chunk geometry");
    static_assert(8 * NT * 64 * 16 <= SB && PRE_TILES * 64 * 16 <= SB, "sums inside the ring");
    __shared__ __attribute__((aligned(16))) uint8_t s_r0[SB];
    __shared__ __attribute__((aligned(16))) uint8_t s_r1[SB];
    __shared__ __attribute__((aligned(16))) uint8_t s_r2[SB];
    __shared__ double s_z[8][64];
    __shared__ double s_zw[16];
    __shared__ float s_g[16];
    __shared__ int s_act[16];
    __shared__ uint32_t s_tag, s_bad;
    __shared__ float s_hid[16 * SPEAR_MAX_GATE_HIDDEN];
    uint8_t *const ring[RING] = {s_r0, s_r1, s_r2};
    pin_pre_args(a);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t M = a.M, K = a.K, KS = a.pre_ks, r = a.r;
    uint64_t claimed = opaque_zero64();
    if (KS > 1 && tid == 0)
        claimed = epoch_claim(a, a.grid);
    const int64_t grp = blockIdx.x / KS, ks = blockIdx.x % KS;
    const int64_t m0 = grp * 16;
    const int64_t T = K / 32;
    const int64_t kb = 32 * (ks * T / KS), ke = 32 * ((ks + 1) * T / KS);   // this slice's depths
    const int64_t nch = (ke - kb + CK - 1) / CK;
    const uint8_t *zsrc = a.ws + a.P.zeros + 16 * (lane & 15);

    // DMA instruction i of this wave fills stage bytes (8 i + wave) KB + 16 lane:
    // row rho, swizzled position p, logical 16-byte chunk c of the row.
    const uint8_t *src[NI];
    int coff[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) {
        const int b = (8 * i + wave) * 1024 + 16 * lane;
        const int rho = b / RB, p = (b % RB) / 16;
        const int c = (p & ~15) | ((p & 15) ^ (rho & 15));
        coff[i] = 8 * c;
        if (rho < 16) {
            const int64_t m = m0 + rho < M ? m0 + rho : M - 1;
            src[i] = reinterpret_cast<const uint8_t *>(a.x + m * K + 8 * c);
        } else {
            const int64_t j = rho - 16;
            src[i] = j < r ? reinterpret_cast<const uint8_t *>(a.A + j * K + 8 * c) : nullptr;
        }
    }
    const int64_t clast = nch - 1;
    auto issue = [&](int64_t ci, uint8_t *buf) {
        const int64_t k0 = kb + (ci < clast ? ci : clast) * CK;
#pragma unroll
        for (int i = 0; i < NI; i++) {
            const bool v = src[i] != nullptr && k0 + coff[i] < ke;
            const void *g = v ? (const void *)(src[i] + 2 * k0) : (const void *)zsrc;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                             (__attribute__((address_space(3))) void *)(buf + (8 * i + wave) * 1024),
                                             16, 0, 0);
        }
    };
    auto issue_wg = [&](int64_t ci, u32x4 *w) {
#pragma unroll
        for (int q = 0; q < SPW; q++) {
            const int64_t k = kb + (ci < clast ? ci : clast) * CK + 32 * (wave + 8 * q) + 8 * lg;
            w[q] = k < ke ? ld16(a.wg + k) : zero4();
        }
    };
    // operand offsets inside a stage: row lr of x, rows 16 + 16 t + lr of A, all
    // at logical chunk 4 st + lg of step st (row % 16 == lr for every one of them)
    int cs[SPW];
#pragma unroll
    for (int q = 0; q < SPW; q++) {
        const int cc = 4 * (wave + 8 * q) + lg;
        cs[q] = ((cc & ~15) | ((cc & 15) ^ lr)) << 4;
    }

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    double zp = 0.0;
    u32x4 wgr[RING][SPW];
#pragma unroll
    for (int q = 0; q < RING - 2; q++) {
        issue(q, ring[q]);
        issue_wg(q, wgr[q]);
    }
    issue(RING - 2, ring[RING - 2]);
    for (int64_t c0 = 0; c0 < nch; c0 += RING) {
#pragma unroll
        for (int j = 0; j < RING; j++) {
            const int64_t ci = c0 + j;
            wait_vmcnt<WAIT>();                           // this wave's DMAs of chunk ci and its w_g
            bare_barrier();                               // every wave's part; chunk ci - 1 free
            issue_wg(ci + RING - 2, wgr[(j + RING - 2) % RING]);
            issue(ci + RING - 1, ring[(j + RING - 1) % RING]);
            if (ci < nch) {
                const uint8_t *buf = ring[j];
#pragma unroll
                for (int q = 0; q < SPW; q++) {
                    const u32x4 xf = *reinterpret_cast<const u32x4 *>(buf + lr * RB + cs[q]);
#pragma unroll
                    for (int t = 0; t < NT; t++) {
                        const u32x4 av = *reinterpret_cast<const u32x4 *>(buf + (16 + 16 * t + lr) * RB + cs[q]);
                        acc[t] = mfma16(av, xf, acc[t]);
                    }
                    const u32x4 w = wgr[j][q];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        zp += (double)(__uint_as_float(xf[e] << 16) * __uint_as_float(w[e] << 16));
                        zp += (double)(__uint_as_float(xf[e] & 0xFFFF0000u) *
                                       __uint_as_float(w[e] & 0xFFFF0000u));
                    }
                }
            }
        }
    }
    wait_vmcnt<0>();                                      // the clamped tail loads
    __syncthreads();                                      // the ring is free

    // the workgroup's partials: waves in order (then lane groups for z)
    f32x4 (*su)[NT][64] = reinterpret_cast<f32x4(*)[NT][64]>(s_r0);
    const PreShared<8> sh = {nullptr, nullptr, s_z, nullptr, reinterpret_cast<f32x4(*)[64]>(s_r1), s_zw, s_g,
                             s_act, &s_tag, &s_bad, s_hid};
#pragma unroll
    for (int t = 0; t < NT; t++)
        su[wave][t][lane] = acc[t];
    s_z[wave][lane] = zp;
    __syncthreads();
    if (wave < NT) {
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < 8; w++)
            u += su[w][wave][lane];
        sh.uw[wave][lane] = u;
    }
    if (wave == 4 && lane < 16) {
        double z = 0.0;
        for (int w = 0; w < 8; w++)
            for (int q = 0; q < 4; q++)
                z += s_z[w][lane + 16 * q];
        s_zw[lane] = z;
    }
    __syncthreads();
    prepass_tail<8>(a, grp, ks, sh, claimed, false);
}

// ------------------------------------------------------------------------ GEMM
// Output tile 16 FN WN channels x 16 FM WM tokens, 8 waves: 256 x 128 (4 wave
// columns along the channels x 2 along the tokens, each wave 64 x 64 as 4 x 4
// MFMA tiles), or 64 x 64 (2 x 2 waves, each 32 x 32 as 2 x 2 tiles, times 2
// along the depth of each stage).  K advances in stages of 128.  Both operands
// go HBM/L2 -> LDS by global_load_lds into a ring of stage buffers (3, or 6
// taken two at a time), so the only memory operations in flight are these
// DMAs: one stage is read while the next ones land.  Each wave waits for its
// own part of a stage (vmcnt) and one barrier per stage makes every part
// visible.  The stage buffers are separate LDS objects and nothing but the
// DMAs writes them, so the compiler can tell that reading one stage does not
// depend on the DMAs into the others and does not wait for them.
// Layouts are XOR-swizzled on the global side so the rows one MFMA operand
// reads fall in distinct banks: activation rows (256 bytes of bf16) swap their
// 16-byte chunks by row % 16, weight rows (64 bytes of nibbles) by
// (row / 2) % 4.  Weights are unpacked as they leave LDS (the packed word
// order makes the unpacked pairs line up with the activations' own pairs).
// Chunks past K are DMA'd from a zero block of the workspace.  The per-token
// activation sums of the offset removal come from one extra MFMA against a
// constant-one operand per token fragment: wave column c takes the 8-deep
// quarter c of every 32-deep step, so the extra work is spread evenly.
//
// Few tiles: K is split into a.g_ks slices, one workgroup each, so that about
// 256 workgroups run; a workgroup stores its scaled partial tile (with its
// share of the EC's rank chunks) and a second launch (splitk_reduce_kernel)
// adds the slices in order.  Up to 128 tokens the tile is 64 x 64 (eight
// waves: 2 along the tokens x 2 along the channels x 2 along the depth of each
// stage), which fills the chip on narrow layers with few or no K slices.
constexpr int G2_STAGES = 3;
constexpr int G2_WBA = 256 * 64;                          // bytes of a 256-channel weight stage

// LDS byte offsets: chunk c (0..15) of activation row r, chunk c (0..3) of weight row r.
__device__ __forceinline__ uint32_t g2_xoff(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }
__device__ __forceinline__ uint32_t g2_woff(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 3)) << 4); }

// Four 16-byte LDS reads.
__device__ __forceinline__ void lds_read4(const uint8_t *base, uint32_t a0, uint32_t a1, uint32_t a2,
                                          uint32_t a3, u32x4 &r0, u32x4 &r1, u32x4 &r2, u32x4 &r3)
{
    r0 = *reinterpret_cast<const u32x4 *>(base + a0);
    r1 = *reinterpret_cast<const u32x4 *>(base + a1);
    r2 = *reinterpret_cast<const u32x4 *>(base + a2);
    r3 = *reinterpret_cast<const u32x4 *>(base + a3);
}

template <int G2_WM, int G2_FM, int SPLIT, int EC, int OUT_F32, int G2_WK = 1, int G2_FN = 4, int G2_WN = 4,
          int G2_KF = 0>
__global__ __launch_bounds__(64 * G2_WN * G2_WM * G2_WK) void gemm2_kernel(const LinearArgs a)
{
    // G2_KF: K is a multiple of 128, so no DMA source ever needs clamping (its
    // per-lane selects are left out of the main loop).
    // G2_WK = 2 (64 x 64 tiles): two waves share each (token, channel) pair of
    // fragments, the first taking depth steps 0 and 1 of every 128-deep stage,
    // the second 2 and 3, so each SIMD holds two waves; the second adds its
    // sums into the first's after the main loop.
    static_assert((G2_WN == 4 && G2_FN == 4 && G2_WK == 1) ||
                      (G2_WN == 2 && G2_FN == 2 && G2_WM == 2 && G2_FM == 2 && G2_WK == 2),
                  "256-channel tiles, or 64 x 64 tiles with the depth split");
    constexpr int G2_BN = 16 * G2_FN * G2_WN;             // channels: 256 or 64
    constexpr int G2_WB = G2_BN * 64;                     // packed weight bytes of one stage
    constexpr int G2_NT = 64 * G2_WN * G2_WM * G2_WK;     // 256 or 512 threads
    constexpr int G2_BM = 16 * G2_FM * G2_WM;             // tokens
    constexpr int G2_XB = G2_BM * 256;                    // activation bytes of one stage
    constexpr int G2_XI = G2_XB / (G2_NT * 16);           // activation DMAs a lane, per stage
    // Weight DMAs a lane, per stage, of G2_WS bytes each: a 64-channel stage
    // (4 KB) is too small for one 16-byte DMA a lane, so every wave takes two
    // 4-byte DMAs of it.  Every wave then issues the same DMAs (no branch), which
    // keeps the compiler's tracking of the LDS DMAs exact: it waits for a stage's
    // own DMAs only, never for all of them.
    constexpr int G2_WS = G2_BN == 64 ? 4 : 16;
    constexpr int G2_WI = G2_WB / (G2_NT * G2_WS);
    static_assert(G2_XI * G2_NT * 16 == G2_XB && G2_WI * G2_NT * G2_WS == G2_WB, "stage split");
    // Ring depth: a 64-channel stage is 20 KB, so its ring holds six stages,
    // taken two at a time (four in flight, 120 KB of LDS); a 256-channel ring
    // holds three.
    constexpr int G2_ST = G2_BN == 64 ? 6 : G2_STAGES;
    constexpr int G2_WBS = G2_BN == 64 ? G2_WB : G2_WBA; // bytes of a weight stage buffer
    __shared__ __attribute__((aligned(16))) uint8_t s_x0[G2_XB];
    __shared__ __attribute__((aligned(16))) uint8_t s_x1[G2_XB];
    __shared__ __attribute__((aligned(16))) uint8_t s_x2[G2_XB];
    __shared__ __attribute__((aligned(16))) uint8_t s_x3[G2_ST > 3 ? G2_XB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_x4[G2_ST > 4 ? G2_XB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_x5[G2_ST > 5 ? G2_XB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_w0[G2_WBS];
    __shared__ __attribute__((aligned(16))) uint8_t s_w1[G2_WBS];
    __shared__ __attribute__((aligned(16))) uint8_t s_w2[G2_WBS];
    __shared__ __attribute__((aligned(16))) uint8_t s_w3[G2_ST > 3 ? G2_WBS : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_w4[G2_ST > 4 ? G2_WBS : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_w5[G2_ST > 5 ? G2_WBS : 16];
    __shared__ float s_rsp[4][G2_BM];         // activation sums of the four 32-deep steps
    static_assert(G2_ST == 3 || G2_ST == 6, "one LDS object per stage");
    uint8_t *const s_xb[6] = {s_x0, s_x1, s_x2, s_x3, s_x4, s_x5};
    uint8_t *const s_wb[6] = {s_w0, s_w1, s_w2, s_w3, s_w4, s_w5};

    __shared__ uint32_t s_tagg, s_tbad;
    pin_pre_args(a);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches

    // EC == 2: the launch's first a.npre blocks are the EC pre-pass (its LDS
    // carved out of the stage buffers); every block claims the launch epoch.
    uint64_t claimed = opaque_zero64();
    if constexpr (EC == 2) {
        if (tid == 0)
            claimed = epoch_claim(a, a.grid);
        if ((int64_t)blockIdx.x < a.npre) {
            // u: waves 0 .. PW/2 - 1 in s_x0, the others in s_x1; the workgroup's u in
            // s_x2; logit partials and w_g in c0 (s_w0, or s_x3 when the
            // weight buffers are small); the small arrays in c1 (s_w1 or s_x4).
            constexpr int PW = G2_NT / 64;
            constexpr int CB = G2_ST > 4 ? G2_XB : G2_WBS;
            static_assert((PW / 2) * PRE_RT * 64 * 16 <= G2_XB && PRE_TILES * 64 * 16 <= G2_XB &&
                          PW * 64 * 8 + PW * 4 * PRE_T * 16 <= CB &&
                          512 + 16 * SPEAR_MAX_GATE_HIDDEN * 4 <= CB,
                          "pre-pass LDS inside the stage buffers");
            uint8_t *const c0 = G2_ST > 4 ? s_x3 : s_w0;
            uint8_t *const c1 = G2_ST > 4 ? s_x4 : s_w1;
            const PreShared<PW> sh = {
                reinterpret_cast<f32x4(*)[PRE_RT][64]>(s_x0),
                reinterpret_cast<f32x4(*)[PRE_RT][64]>(s_x1),
                reinterpret_cast<double(*)[64]>(c0),
                reinterpret_cast<u32x4(*)[4 * PRE_T]>(c0 + PW * 64 * 8),
                reinterpret_cast<f32x4(*)[64]>(s_x2),
                reinterpret_cast<double *>(c1),
                reinterpret_cast<float *>(c1 + 128),
                reinterpret_cast<int *>(c1 + 192),
                reinterpret_cast<uint32_t *>(c1 + 256),
                reinterpret_cast<uint32_t *>(c1 + 260),
                reinterpret_cast<float *>(c1 + 512)};
            if ((int64_t)blockIdx.x < ((a.M + 15) / 16) * a.pre_ks)
                prepass_body<PW>(a, blockIdx.x, sh, claimed, true);
            return;
        }
    }
    const int lr = lane & 15, lg = lane >> 4;
    const int wn = wave % G2_WN, wm = (wave / G2_WN) % G2_WM, wk = wave / (G2_WN * G2_WM);
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t tiles_n = (N + G2_BN - 1) / G2_BN, tiles_m = (M + G2_BM - 1) / G2_BM;
    const int64_t ntiles = tiles_n * tiles_m;
    const int64_t KS = SPLIT ? a.g_ks : 1;
    const int64_t nunits = ntiles * KS;                   // unit = slice * ntiles + tile

    // Blocks are dealt round-robin to the 8 XCDs; give each XCD a contiguous run
    // of units (channels fastest, then tokens, then K slices) so its L2 shares
    // activation rows.
    const int64_t bid = (int64_t)blockIdx.x - (EC == 2 ? a.npre : 0);   // npre % 8 == 0
    const int64_t q8 = nunits / 8, r8 = nunits % 8;
    const int64_t xcd = bid % 8, loc = bid / 8;
    const int64_t unit = xcd * q8 + (xcd < r8 ? xcd : r8) + loc;
    const int64_t tile = unit % ntiles, ks = unit / ntiles;
    const int64_t n0 = (tile % tiles_n) * G2_BN, m0 = (tile / tiles_n) * G2_BM;
    const int64_t S = (K + 127) / 128;
    const int64_t sb = ks * S / KS, se = (ks + 1) * S / KS;   // this slice's stages
    const uint8_t *zsrc = a.ws + a.P.zeros + 16 * (lane & 15);

    // DMA of one stage.  Activations: instruction j of wave w fills rows
    // 4 (G2_XI w + j) .. +3, lane i the slot i of that 1 KB (chunk (i % 16) ^
    // (row % 16) of its row); rows past M repeat row M - 1 (never stored).
    // Weights: instruction j fills rows 16 (G2_WI w + j) .. +15, lane i the slot
    // i of that 1 KB (chunk (i % 4) ^ ((row / 2) % 4)); with 4-byte DMAs rows
    // 4 (G2_WI w + j) .. +3, lane i word i % 4 of slot i / 4.  Rows past N repeat
    // the last row.  Each lane's stage-0 source and the number of stages its chunk
    // stays inside K are computed once.  Activation chunks past K come from the
    // zero block; weight chunks past K re-read the lane's last chunk inside K
    // (finite values that meet zero activations).
    const uint8_t *xsrc[G2_XI], *wsrc[G2_WI];
    int64_t xlim[G2_XI], wlast[G2_WI];
#pragma unroll
    for (int j = 0; j < G2_XI; j++) {
        const int r = 4 * (G2_XI * wave + j) + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        const int64_t mm = m0 + r < M ? m0 + r : M - 1;
        xsrc[j] = reinterpret_cast<const uint8_t *>(a.x + mm * K + 8 * c);
        xlim[j] = (K - 8 * c + 127) / 128;                // stages st with 128 st + 8 c < K
    }
#pragma unroll
    for (int j = 0; j < G2_WI; j++) {
        const int slot = G2_WS == 16 ? lane : lane >> 2;  // 16-byte slot of the 1 KB or 256 B
        const int r = (G2_WS == 16 ? 16 : 4) * (G2_WI * wave + j) + (slot >> 2);
        const int c = (slot & 3) ^ ((r >> 1) & 3);
        const int64_t nn = n0 + r < N ? n0 + r : N - 1;
        wsrc[j] = a.packed + nn * (K / 2) + 16 * c + (G2_WS == 16 ? 0 : 4 * (lane & 3));
        wlast[j] = (K - 32 * c + 127) / 128 - 1;          // last stage with 128 st + 32 c < K
    }
    auto issue_x = [&](int64_t st, uint8_t *xbase, int j) {
        const void *src = (G2_KF || st < xlim[j]) ? (const void *)(xsrc[j] + 256 * st) : (const void *)zsrc;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)(xbase + 1024 * (G2_XI * wave + j)),
                                         16, 0, 0);
    };
    auto issue_w = [&](int64_t st, uint8_t *wbase, int j) {
        const int64_t sw = (G2_KF || st < wlast[j]) ? st : wlast[j];
        const auto *src = (const __attribute__((address_space(1))) void *)(wsrc[j] + 64 * sw);
        auto *dst = (__attribute__((address_space(3))) void *)(wbase + 64 * G2_WS * (G2_WI * wave + j));
        if constexpr (G2_BN == 64)
            __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
        else
            __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    };
    auto issue = [&](int64_t st, uint8_t *xbase, uint8_t *wbase) {
#pragma unroll
        for (int j = 0; j < G2_XI; j++)
            issue_x(st, xbase, j);
#pragma unroll
        for (int j = 0; j < G2_WI; j++)
            issue_w(st, wbase, j);
    };

    // EC operands of one 32-rank chunk t: v (hi, lo) of this wave's tokens and
    // B rows of its channels.  The slice's first chunk is loaded now, so its
    // round trip overlaps the main loop (48 registers, which both tile shapes
    // have to spare).
    auto ec_load = [&](int t, u32x4 *vh, u32x4 *vl, u32x4 *bf) {
        const uint16_t *vhi = reinterpret_cast<const uint16_t *>(a.ws + a.P.vhi);
        const uint16_t *vlo = reinterpret_cast<const uint16_t *>(a.ws + a.P.vlo);
        const int rpad = a.rpad, r = a.r;
        const int j = 32 * t + 8 * lg;
#pragma unroll
        for (int fm = 0; fm < G2_FM; fm++) {
            const int64_t mm = m0 + (wm * G2_FM + fm) * 16 + lr;
            vh[fm] = (mm < M) ? ld16(vhi + mm * rpad + j) : zero4();
            vl[fm] = (mm < M) ? ld16(vlo + mm * rpad + j) : zero4();
        }
#pragma unroll
        for (int fn = 0; fn < G2_FN; fn++) {
            const int64_t nn = n0 + (wn * G2_FN + fn) * 16 + lr;
            bf[fn] = (nn < N && j < r) ? ld16(a.B + nn * r + j) : zero4();
        }
    };
    constexpr bool ECPRE = EC == 1;
    u32x4 pvh[G2_FM], pvl[G2_FM], pbf[G2_FN];
    if (ECPRE && wk == 0 && ks < a.rpad / 32)
        ec_load((int)ks, pvh, pvl, pbf);
    // EC == 2, 64 x 64 tiles: the B rows of the slice's first two rank chunks
    // now (v comes from this launch's pre-pass blocks, at the end), in the
    // waves that apply the EC term (the first of each depth pair).
    constexpr bool PBF = G2_BN == 64;                     // registers to spare
    u32x4 pbf2[G2_FN];
    if (EC == 2 && PBF && wk == 0 && ks < a.rpad / 32) {
        const int j = 32 * (int)ks + 8 * lg, j2 = j + 32 * (int)KS;
#pragma unroll
        for (int fn = 0; fn < G2_FN; fn++) {
            const int64_t nn = n0 + (wn * G2_FN + fn) * 16 + lr;
            pbf[fn] = (nn < N && j < a.r) ? ld16(a.B + nn * a.r + j) : zero4();
            pbf2[fn] = (nn < N && j2 < a.r) ? ld16(a.B + nn * a.r + j2) : zero4();
        }
    }
    // The epilogue's scales and zero-point bytes, loaded now so that their round
    // trip overlaps the main loop.
    float sc_raw[G2_FN][4];
    uint32_t zb_raw[G2_FN][4];
#pragma unroll
    for (int fn = 0; fn < G2_FN; fn++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            int64_t nn = n0 + (wn * G2_FN + fn) * 16 + 4 * lg + i;
            nn = nn < N ? nn : N - 1;
            sc_raw[fn][i] = a.scales[nn];
            zb_raw[fn][i] = load_zero_byte(a.zeros, a.scales, nn);
        }

    f32x4 acc[G2_FN][G2_FM], acc1[G2_FN][G2_FM], rsq[G2_FM];
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
    for (int fn = 0; fn < G2_FN; fn++)
#pragma unroll
        for (int fm = 0; fm < G2_FM; fm++)
            acc[fn][fm] = acc1[fn][fm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int fm = 0; fm < G2_FM; fm++)
        rsq[fm] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS addresses this lane reads (stage-relative).
    // Fragment fm / fn adds a whole number of 16-row blocks, which leaves the
    // swizzles (they depend on the row modulo 16) unchanged: one base per depth
    // step plus immediate offsets.
    constexpr int G2_ND = 4 / G2_WK;                      // depth steps a wave takes per stage
    uint32_t xo[G2_ND];
#pragma unroll
    for (int dd = 0; dd < G2_ND; dd++)
        xo[dd] = g2_xoff(wm * G2_FM * 16 + lr, 4 * lg + G2_ND * wk + dd);
    const uint32_t wo = g2_woff(wn * G2_FN * 16 + lr, lg);

    // This wave's W words of one stage (wb).
    auto wread = [&](const uint8_t *wb, u32x4 *wv) {
        if constexpr (G2_WK == 1) {
            lds_read4(wb, wo, wo + 1024, wo + 2048, wo + 3072, wv[0], wv[1], wv[2], wv[3]);
        } else {
            // this wave's two words of each fragment (depth steps 2 wk, 2 wk + 1)
#pragma unroll
            for (int fn = 0; fn < G2_FN; fn++) {
                const uint2 w2 = *reinterpret_cast<const uint2 *>(wb + wo + 1024 * fn + 8 * wk);
                wv[fn] = u32x4{w2.x, w2.y, 0u, 0u};
            }
        }
    };
    // Depth step dd of one stage (xb, wv) into the accumulator set ac.
    auto step = [&](const uint8_t *xb, const u32x4 *wv, int dd, f32x4 (&ac)[G2_FN][G2_FM]) {
        const int d = G2_ND * wk + dd;
        u32x4 xf[G2_FM];
#pragma unroll
        for (int fm = 0; fm < G2_FM; fm++)
            xf[fm] = *reinterpret_cast<const u32x4 *>(xb + xo[dd] + 4096 * fm);
        if (d % G2_WN == wn) {                                // one wave column a step
#pragma unroll
            for (int fm = 0; fm < G2_FM; fm++)
                rsq[fm] = mfma16(ones, xf[fm], rsq[fm]);
        }
#pragma unroll
        for (int fn = 0; fn < G2_FN; fn++) {
            const u32x4 wa = unpack8(wv[fn][dd]);
            // Two waves a SIMD: the one issuing MFMAs goes first, so the other's
            // LDS reads and unpacking fill the gaps.
            if (G2_NT == 512)
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int fm = 0; fm < G2_FM; fm++)
                ac[fn][fm] = mfma16(wa, xf[fm], ac[fn][fm]);
            if (G2_NT == 512)
                __builtin_amdgcn_s_setprio(0);
        }
    };

    // Every stage slot issues its DMAs, past the end clamped to the last stage
    // (never used), so each wave always has the same number of further stages
    // in flight when it waits for the current ones.  The next stages' DMAs are
    // spread over this stage's depth steps (one or two before each step's
    // MFMAs) rather than issued all at once, so no wave stalls on a burst of
    // DMA issue while it has MFMAs ready.  Every slot issues all of them, also
    // past the slice's end, outside any branch: the compiler then tracks
    // exactly which stage each outstanding DMA fills.
    const int64_t slast = se - 1;
    if constexpr (G2_ST == 6) {
        // 64 x 64 tiles: the six slots are taken two at a time (256 deep a
        // barrier; two pairs in flight).  Each depth step accumulates into its
        // own set, so that back-to-back MFMAs do not wait on each other.
        static_assert(G2_ND == 2 && G2_XI == 2 && G2_WI == 2, "pair schedule");
        constexpr int G2_WAIT2 = (G2_XI + G2_WI) * 2;        // the next pair's DMAs
#pragma unroll
        for (int j = 0; j < 4; j++)
            issue(sb + j < slast ? sb + j : slast, s_xb[j], s_wb[j]);
        for (int64_t s0 = sb; s0 < se; s0 += 6) {
#pragma unroll
            for (int p = 0; p < 3; p++) {
                const int64_t s = s0 + 2 * p;
                wait_vmcnt<G2_WAIT2>();                       // this wave's part of stages s, s + 1
                bare_barrier();                               // every wave's part; pair p - 1 free
                const int64_t sn0 = (s + 4 < slast) ? s + 4 : slast, sn1 = (s + 5 < slast) ? s + 5 : slast;
                uint8_t *const nx0 = s_xb[(2 * p + 4) % 6], *const nw0 = s_wb[(2 * p + 4) % 6];
                uint8_t *const nx1 = s_xb[(2 * p + 5) % 6], *const nw1 = s_wb[(2 * p + 5) % 6];
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const bool live = s + h < se;
                    const uint8_t *xb = s_xb[2 * p + h], *wb = s_wb[2 * p + h];
                    u32x4 wv[G2_FN];
                    if (live)
                        wread(wb, wv);
#pragma unroll
                    for (int dd = 0; dd < 2; dd++) {
                        // the pair's eight DMAs, two before each of its four steps
                        const int q = 2 * h + dd;
                        if (q < 2) {
                            issue_x(sn0, nx0, q);
                            issue_w(sn0, nw0, q);
                        } else {
                            issue_x(sn1, nx1, q - 2);
                            issue_w(sn1, nw1, q - 2);
                        }
                        if (live) {
                            if (dd == 0)
                                step(xb, wv, 0, acc);
                            else
                                step(xb, wv, 1, acc1);
                        }
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < G2_ST - 1; j++)
            issue(sb + j < slast ? sb + j : slast, s_xb[j], s_wb[j]);
        constexpr int G2_WAIT = (G2_XI + G2_WI) * (G2_ST - 2);
        static_assert(G2_WAIT < 64, "vmcnt");
        for (int64_t s0 = sb; s0 < se; s0 += G2_ST) {
#pragma unroll
            for (int j = 0; j < G2_ST; j++) {
                const int64_t s = s0 + j;
                wait_vmcnt<G2_WAIT>();                        // this wave's part of stage s
                bare_barrier();                               // every wave's part; stage s - 1 free
                const int64_t sn = (s + G2_ST - 1 < slast) ? s + G2_ST - 1 : slast;
                uint8_t *const nxb = s_xb[(j + G2_ST - 1) % G2_ST];
                uint8_t *const nwb = s_wb[(j + G2_ST - 1) % G2_ST];
                const bool live = s < se;
                const uint8_t *xb = s_xb[j], *wb = s_wb[j];
                u32x4 wv[G2_FN];
                if (live)
                    wread(wb, wv);
#pragma unroll
                for (int dd = 0; dd < G2_ND; dd++) {
                    if (dd < G2_XI)
                        issue_x(sn, nxb, dd);
                    if (dd < G2_WI)
                        issue_w(sn, nwb, dd);
                    if (live)
                        step(xb, wv, dd, acc);
                }
#pragma unroll
                for (int jj = G2_ND; jj < G2_XI; jj++)
                    issue_x(sn, nxb, jj);
#pragma unroll
                for (int jj = G2_ND; jj < G2_WI; jj++)
                    issue_w(sn, nwb, jj);
            }
        }
    }
    wait_vmcnt<0>();                                          // the clamped tail DMAs
    if constexpr (G2_BN == 64) {
#pragma unroll
        for (int fn = 0; fn < G2_FN; fn++)
#pragma unroll
            for (int fm = 0; fm < G2_FM; fm++)
                acc[fn][fm] += acc1[fn][fm];
    }

    if constexpr (G2_WK == 2) {
        // the second wave of each (token, channel) pair adds its sums into the
        // first's (through the stage buffers, free once every wave is past the
        // main loop)
        __syncthreads();
        static_assert(G2_FN * G2_FM * 64 * 16 <= G2_XB && G2_ST > 3, "exchange");
        const int q = wm * G2_WN + wn;
        f32x4 *e = reinterpret_cast<f32x4 *>(q == 0 ? s_x0 : q == 1 ? s_x1 : q == 2 ? s_x2 : s_x3);
        if (wk == 1) {
#pragma unroll
            for (int fn = 0; fn < G2_FN; fn++)
#pragma unroll
                for (int fm = 0; fm < G2_FM; fm++)
                    e[(fn * G2_FM + fm) * 64 + lane] = acc[fn][fm];
        }
        // this wave formed the activation sums of step 2 wk + wn
        if (lg == 0) {
#pragma unroll
            for (int fm = 0; fm < G2_FM; fm++)
                s_rsp[2 * wk + wn][(wm * G2_FM + fm) * 16 + lr] = rsq[fm][0];
        }
        __syncthreads();
        // Only the first wave of each pair carries on, except through the
        // fused EC's v staging, whose barriers every wave takes part in.
        if (EC != 2 && wk == 1)
            return;
#pragma unroll
        for (int fn = 0; fn < G2_FN; fn++)
#pragma unroll
            for (int fm = 0; fm < G2_FM; fm++)
                acc[fn][fm] += e[(fn * G2_FM + fm) * 64 + lane];
    } else if (lg == 0) {
#pragma unroll
        for (int fm = 0; fm < G2_FM; fm++)
            s_rsp[wn][(wm * G2_FM + fm) * 16 + lr] = rsq[fm][0];
    }
    if (EC == 2 && tid == 0) {
        s_tagg = epoch_tag(claimed + opaque_zero64());
        s_tbad = 0;
    }
    if constexpr (G2_WK == 1 || EC == 2)
        __syncthreads();                                      // (the depth split synchronised s_rsp)

    // Epilogue: scale and offset removal, the EC term, store.
#pragma unroll
    for (int fn = 0; fn < G2_FN; fn++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float sn = sc_raw[fn][i];
            const float zc = UNPACK_OFF + zero_point(a.zeros, zb_raw[fn][i]);
#pragma unroll
            for (int fm = 0; fm < G2_FM; fm++) {
                const int row = (wm * G2_FM + fm) * 16 + lr;
                const float rsm = ((s_rsp[0][row] + s_rsp[1][row]) + s_rsp[2][row]) + s_rsp[3][row];
                acc[fn][fm][i] = sn * __builtin_fmaf(-zc, rsm, UNPACK_SCALE * acc[fn][fm][i]);
            }
        }
    }
    if (EC == 2 && ks < a.rpad / 32) {
        // v of the tile's tokens as tagged words from the launch's pre-pass
        // blocks: word {hi | lo << 16, epoch} per (token, rank).  The slice's rank
        // chunks are taken two at a time: each thread loads its share of both
        // chunks' words into LDS (stage buffer 0, free after the main loop) in
        // one poll, until every tag is this launch's, so a rank above 32 costs
        // no second round trip; when they are not all there at the first try,
        // a wave polls one word (one request) before it reloads, so that early
        // tiles do not flood the memory system the pre-pass needs.  Bounded; an
        // expired wait makes the whole tile NaN (its EC term is unknown) and is
        // counted.
        const uint64_t *vtag = reinterpret_cast<const uint64_t *>(a.ws + a.P.vtag);
        const uint32_t tag = s_tagg;
        const int rpad = a.rpad, r = a.r;
        const int64_t nch = rpad / 32;
        uint32_t *s_v = reinterpret_cast<uint32_t *>(s_x0);          // [2][G2_BM][32] payloads
        static_assert(2 * G2_BM * 32 * 4 <= G2_XB && (G2_BM * 32) % G2_NT == 0, "v staging");
        constexpr int VW = G2_BM * 32 / G2_NT;                        // words a thread loads a chunk
        // With the depth split only the first wave of each pair applies the
        // term (the second's sums are in it already); both load words and take
        // the barriers.
        const bool apply = G2_WK == 1 || wk == 0;                     // uniform
        for (int64_t t = ks; t < nch; t += 2 * KS) {
            const bool two = t + KS < nch;                            // uniform
            u32x4 bf[2][G2_FN];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int j = 32 * (int)(t + h * KS) + 8 * lg;
#pragma unroll
                for (int fn = 0; fn < G2_FN; fn++) {
                    const int64_t nn = n0 + (wn * G2_FN + fn) * 16 + lr;
                    bf[h][fn] = (PBF && t == ks) ? (h == 0 ? pbf[fn] : pbf2[fn])
                                : (apply && nn < N && j < r && (h == 0 || two)) ? ld16(a.B + nn * r + j)
                                                                                : zero4();
                }
            }
            bool ok = true;
            for (uint32_t it = 0;; it++) {
                bool good = true;
                uint64_t w[2][VW];
#pragma unroll
                for (int h = 0; h < 2; h++)
#pragma unroll
                    for (int q = 0; q < VW; q++) {
                        const int e = tid + G2_NT * q;                  // token e / 32, rank e % 32
                        const int64_t mm = m0 + e / 32 < M ? m0 + e / 32 : M - 1;
                        w[h][q] = (h == 0 || two) ? load_tagged(vtag + mm * rpad + 32 * (t + h * KS) + e % 32)
                                                  : (uint64_t)tag << 32;
                    }
#pragma unroll
                for (int h = 0; h < 2; h++)
#pragma unroll
                    for (int q = 0; q < VW; q++) {
                        good &= (uint32_t)(w[h][q] >> 32) == tag;
                        s_v[h * G2_BM * 32 + tid + G2_NT * q] = (uint32_t)w[h][q];
                    }
                if (__all(good))
                    break;
                if (it >= a.wait_limit) {
                    ok = false;
                    break;
                }
                if (it == 0) {
                    // not there yet: poll one word (one request a wave) until the
                    // tile's last token has it, rather than reload them all
                    const int64_t ml = m0 + G2_BM - 1 < M ? m0 + G2_BM - 1 : M - 1;
                    const uint64_t *probe = vtag + ml * rpad + 32 * (two ? t + KS : t) + 31;
                    for (uint32_t ip = 0; ip < a.wait_limit; ip++) {
                        if ((uint32_t)(load_tagged(probe) >> 32) == tag)
                            break;
                        __builtin_amdgcn_s_sleep(8);
                    }
                }
                __builtin_amdgcn_s_sleep(4);
            }
            if (!ok && lane == 0)
                atomicOr(&s_tbad, 1u << (t & 31));
            __syncthreads();
            if (s_tbad & (1u << (t & 31))) {
                if (tid == 0)
                    atomicAdd(reinterpret_cast<uint32_t *>(a.ws + a.P.hdr) + HDR_TIMEOUTS, 1u);
                const float qnan = __builtin_nanf("");
#pragma unroll
                for (int fn = 0; fn < G2_FN; fn++)
#pragma unroll
                    for (int fm = 0; fm < G2_FM; fm++)
                        acc[fn][fm] = f32x4{qnan, qnan, qnan, qnan};
                __syncthreads();                                      // s_v is rewritten next
                continue;
            }
#pragma unroll
            for (int h = 0; h < 2; h++) {
                if ((h == 1 && !two) || !apply)
                    break;
#pragma unroll
                for (int fm = 0; fm < G2_FM; fm++) {
                    const int row = (wm * G2_FM + fm) * 16 + lr;
                    const uint32_t *sv = s_v + h * G2_BM * 32 + row * 32 + 8 * lg;
                    const u32x4 p0 = *reinterpret_cast<const u32x4 *>(sv);
                    const u32x4 p1 = *reinterpret_cast<const u32x4 *>(sv + 4);
                    const uint32_t w8[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
                    const bool mv = m0 + row < M;
                    u32x4 vh, vl;
#pragma unroll
                    for (int p = 0; p < 4; p++) {
                        const uint32_t w0 = w8[2 * p], w1 = w8[2 * p + 1];
                        vh[p] = mv ? (w0 & 0xFFFFu) | (w1 << 16) : 0u;
                        vl[p] = mv ? (w0 >> 16) | (w1 & 0xFFFF0000u) : 0u;
                    }
#pragma unroll
                    for (int fn = 0; fn < G2_FN; fn++) {
                        acc[fn][fm] = mfma16(bf[h][fn], vh, acc[fn][fm]);
                        acc[fn][fm] = mfma16(bf[h][fn], vl, acc[fn][fm]);
                    }
                }
            }
            if (t + 2 * KS < nch)
                __syncthreads();                                      // s_v is rewritten next
        }
    }
    if (EC == 1 && ks < a.rpad / 32) {
        // Rank chunks of 32: slice ks takes chunks ks, ks + KS, ... (the
        // second launch adds the slices), so a K split also splits the EC.
        const int32_t *active = reinterpret_cast<const int32_t *>(a.ws + a.P.active);
        int any = 0;
#pragma unroll
        for (int fm = 0; fm < G2_FM; fm++) {
            const int64_t mm = m0 + (wm * G2_FM + fm) * 16 + lr;
            any |= (mm < M) ? active[mm] : 0;
        }
        if (__ballot(any) != 0ull) {
            for (int64_t t = ks; t < a.rpad / 32; t += KS) {
                u32x4 vh[G2_FM], vl[G2_FM], bf[G2_FN];
                if (ECPRE && t == ks) {
#pragma unroll
                    for (int fm = 0; fm < G2_FM; fm++) {
                        vh[fm] = pvh[fm];
                        vl[fm] = pvl[fm];
                    }
#pragma unroll
                    for (int fn = 0; fn < G2_FN; fn++)
                        bf[fn] = pbf[fn];
                } else {
                    ec_load((int)t, vh, vl, bf);
                }
#pragma unroll
                for (int fn = 0; fn < G2_FN; fn++)
#pragma unroll
                    for (int fm = 0; fm < G2_FM; fm++) {
                        acc[fn][fm] = mfma16(bf[fn], vh[fm], acc[fn][fm]);
                        acc[fn][fm] = mfma16(bf[fn], vl[fm], acc[fn][fm]);
                    }
            }
        }
    }
    if (G2_WK == 2 && wk == 1)
        return;                                               // the column's first wave stores
    if (SPLIT) {
        // the scaled partial tile of this slice: unit-major, row-major bm x 256
        float *part = reinterpret_cast<float *>(a.ws + a.P.gpart) + unit * (G2_BM * G2_BN);
#pragma unroll
        for (int fm = 0; fm < G2_FM; fm++) {
            const int row = (wm * G2_FM + fm) * 16 + lr;
            if (m0 + row >= M)
                continue;
#pragma unroll
            for (int fn = 0; fn < G2_FN; fn++)
                *reinterpret_cast<f32x4 *>(part + row * G2_BN + (wn * G2_FN + fn) * 16 + 4 * lg) =
                    acc[fn][fm];
        }
        return;
    }
#pragma unroll
    for (int fm = 0; fm < G2_FM; fm++) {
        const int64_t mm = m0 + (wm * G2_FM + fm) * 16 + lr;
        if (mm >= M)
            continue;
#pragma unroll
        for (int fn = 0; fn < G2_FN; fn++) {
            const int64_t nb = n0 + (wn * G2_FN + fn) * 16 + 4 * lg;
            const f32x4 v = acc[fn][fm];
            if (OUT_F32) {
                float *y = reinterpret_cast<float *>(a.y) + mm * N;
                if (nb + 3 < N && (N & 3) == 0) {
                    *reinterpret_cast<f32x4 *>(y + nb) = v;
                } else {
                    for (int i = 0; i < 4; i++)
                        if (nb + i < N)
                            y[nb + i] = v[i];
                }
            } else {
                uint16_t *y = reinterpret_cast<uint16_t *>(a.y) + mm * N;
                if (nb + 3 < N && (N & 3) == 0) {
                    uint2 o;
                    o.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
                    o.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
                    *reinterpret_cast<uint2 *>(y + nb) = o;
                } else {
                    for (int i = 0; i < 4; i++)
                        if (nb + i < N)
                            y[nb + i] = f2bf(v[i]);
                }
            }
        }
    }
}

// Second launch of a K-split GEMM: y = the sum of the slices' partial tiles in
// slice order; a thread takes 4 consecutive channels of one token.  Its few
// values come as plain arguments (one 64-byte line; read from the layer's
// argument block they would span five).
template <int OUT_F32>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(void *yv, const uint8_t *partv, int64_t M,
                                                            int64_t N, int32_t KS, int32_t bm, int32_t bn)
{
    const int64_t nq = (N + 3) / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * nq)
        return;
    const int64_t m = idx / nq, n = 4 * (idx % nq);
    const int64_t tiles_n = (N + bn - 1) / bn, ntiles = tiles_n * ((M + bm - 1) / bm);
    const int64_t tile = (m / bm) * tiles_n + n / bn;
    const int64_t off = (m % bm) * bn + n % bn;
    const f32x4 *part = reinterpret_cast<const f32x4 *>(partv);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (int64_t q0 = 0; q0 < KS; q0 += CMB_U) {
        f32x4 p[CMB_U];
#pragma unroll
        for (int i = 0; i < CMB_U; i++)
            if (q0 + i < KS)
                p[i] = part[(((q0 + i) * ntiles + tile) * bm * bn + off) / 4];
#pragma unroll
        for (int i = 0; i < CMB_U; i++)
            if (q0 + i < KS)
                v += p[i];
    }
    if (OUT_F32) {
        float *y = reinterpret_cast<float *>(yv) + m * N;
        if (n + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<f32x4 *>(y + n) = v;
        } else {
            for (int i = 0; i < 4; i++)
                if (n + i < N)
                    y[n + i] = v[i];
        }
    } else {
        uint16_t *y = reinterpret_cast<uint16_t *>(yv) + m * N;
        if (n + 3 < N && (N & 3) == 0) {
            uint2 o;
            o.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
            o.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
            *reinterpret_cast<uint2 *>(y + n) = o;
        } else {
            for (int i = 0; i < 4; i++)
                if (n + i < N)
                    y[n + i] = f2bf(v[i]);
        }
    }
}

template <int WM, int FM, int EC, int WK = 1, int FN = 4, int WN = 4, int KF = 0>
hipError_t launch_gemm2_t(const LinearArgs &a, hipStream_t s)
{
    const int64_t bm = 16 * FM * WM, bn = 16 * FN * WN;
    const int64_t ntiles = ((a.N + bn - 1) / bn) * ((a.M + bm - 1) / bm);
    const dim3 block(64 * WN * WM * WK);
    // EC == 2: the pre-pass blocks come first in the grid
    const int64_t pre = EC == 2 ? a.npre : 0;
    LinearArgs ka = a;
    ka.grid = (uint32_t)(pre + ntiles * (a.g_ks > 1 ? a.g_ks : 1));   // read instead of gridDim
    if (a.g_ks > 1) {
        hipLaunchKernelGGL((gemm2_kernel<WM, FM, 1, EC, 1, WK, FN, WN, KF>), dim3(ka.grid), block, 0, s, ka);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        const int64_t threads = a.M * ((a.N + 3) / 4);
        const uint8_t *part = a.ws + a.P.gpart;
        if (a.out_f32)
            hipLaunchKernelGGL(splitk_reduce_kernel<1>, dim3((unsigned)((threads + 255) / 256)),
                               dim3(256), 0, s, a.y, part, a.M, a.N, a.g_ks, a.g_bm, a.g_bn);
        else
            hipLaunchKernelGGL(splitk_reduce_kernel<0>, dim3((unsigned)((threads + 255) / 256)),
                               dim3(256), 0, s, a.y, part, a.M, a.N, a.g_ks, a.g_bm, a.g_bn);
        return hipGetLastError();
    }
    if (a.out_f32)
        hipLaunchKernelGGL((gemm2_kernel<WM, FM, 0, EC, 1, WK, FN, WN, KF>), dim3(ka.grid), block, 0, s, ka);
    else
        hipLaunchKernelGGL((gemm2_kernel<WM, FM, 0, EC, 0, WK, FN, WN, KF>), dim3(ka.grid), block, 0, s, ka);
    return hipGetLastError();
}

// ------------------------------------------------------------ EC apply kernel
// The separate EC kernel of the semi-fused prefill (summary section 2.2 A: at
// prefill the EC runs as its own kernel beside the GEMM, joined through the
// graph), after the join: y[m][n] += sum_j B[n][j] v[m][j] for the active
// tokens only, taken from the compacted list (ascending indices, then their
// count), so that tokens the hard gate skips cost no work and no traffic.
// v = g (alpha gamma) u is the pre-pass's, as bf16 hi + lo.  A workgroup takes
// 16 listed tokens x 256 channels (4 waves of 64): 16 x 16 MFMA tiles with
// the channels as rows, the tokens as columns, 32 ranks deep, then
// read-add-write of y (fp32).  A count of -1 (an expired wait in the
// pre-pass) walks every token instead and writes NaN where the selection
// flag is -1.
__global__ __launch_bounds__(256) void ec_apply_kernel(const LinearArgs a)
{
    const int64_t M = a.M, N = a.N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int32_t *list = reinterpret_cast<const int32_t *>(a.ws + a.P.idx);
    const int32_t *active = reinterpret_cast<const int32_t *>(a.ws + a.P.active);
    const int32_t nact = list[a.mpad];
    const bool bad = nact < 0;
    const int64_t cnt = bad ? M : nact;
    const int64_t t0 = (int64_t)blockIdx.x * 16;
    if (t0 >= cnt)
        return;
    const int64_t slot = t0 + lr;
    int64_t m = -1;                                   // the token of column lr
    if (slot < cnt)
        m = bad ? slot : list[slot];
    const int flag = m >= 0 ? active[m] : 0;
    const bool use = m >= 0 && flag != 0;
    const int64_t n0 = (int64_t)blockIdx.y * 256 + 64 * wave;
    const uint16_t *vhi = reinterpret_cast<const uint16_t *>(a.ws + a.P.vhi);
    const uint16_t *vlo = reinterpret_cast<const uint16_t *>(a.ws + a.P.vlo);
    const int rpad = a.rpad, r = a.r;
    f32x4 acc[4];
#pragma unroll
    for (int fn = 0; fn < 4; fn++)
        acc[fn] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < rpad / 32; t++) {
        const int j = 32 * t + 8 * lg;
        const u32x4 vh = use ? ld16(vhi + m * rpad + j) : zero4();
        const u32x4 vl = use ? ld16(vlo + m * rpad + j) : zero4();
#pragma unroll
        for (int fn = 0; fn < 4; fn++) {
            const int64_t n = n0 + 16 * fn + lr;
            const u32x4 bf = (n < N && j < r) ? ld16(a.B + n * r + j) : zero4();
            acc[fn] = mfma16(bf, vh, acc[fn]);
            acc[fn] = mfma16(bf, vl, acc[fn]);
        }
    }
    // lane (lr, lg) holds channels n0 + 16 fn + 4 lg + i of token m
    if (!use)
        return;
    float *yr = reinterpret_cast<float *>(a.y) + m * N;
    const float qnan = __builtin_nanf("");
#pragma unroll
    for (int fn = 0; fn < 4; fn++) {
        const int64_t nb = n0 + 16 * fn + 4 * lg;
        if (nb + 3 < N && (N & 3) == 0) {
            f32x4 v = *reinterpret_cast<const f32x4 *>(yr + nb);
            v = flag < 0 ? f32x4{qnan, qnan, qnan, qnan} : v + acc[fn];
            *reinterpret_cast<f32x4 *>(yr + nb) = v;
        } else {
            for (int i = 0; i < 4; i++)
                if (nb + i < N)
                    yr[nb + i] = flag < 0 ? qnan : yr[nb + i] + acc[fn][i];
        }
    }
}

} // namespace

hipError_t launch_ec_apply(const LinearArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)((a.M + 15) / 16), (unsigned)((a.N + 255) / 256));
    hipLaunchKernelGGL(ec_apply_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_prepass(const LinearArgs &a, hipStream_t s)
{
    const unsigned grid = (unsigned)((a.M + 15) / 16) * (unsigned)a.pre_ks;
    LinearArgs ka = a;
    ka.grid = grid;                                       // read instead of gridDim
    if (a.rpad == 32)
        hipLaunchKernelGGL(prepass2_kernel<32>, dim3(grid), dim3(512), 0, s, ka);
    else if (a.rpad == 64)
        hipLaunchKernelGGL(prepass2_kernel<64>, dim3(grid), dim3(512), 0, s, ka);
    else
        hipLaunchKernelGGL(prepass_kernel, dim3(grid), dim3(64 * PRE_WAVES), 0, s, ka);
    return hipGetLastError();
}

hipError_t launch_gemm(const LinearArgs &a, int ec_on, int force_large, hipStream_t s)
{
    (void)force_large;                                    // a.g_bm, a.g_bn, a.g_ks carry the choice
    if (a.g_bm == 64) {
        // Both tile shapes have a variant without the DMA-source clamps for K a
        // multiple of 128 (their per-lane selects cost about 8 % of the 64 x 64
        // loop).
        if (a.K % 128 == 0) {
            if (ec_on == 2)
                return launch_gemm2_t<2, 2, 2, 2, 2, 2, 1>(a, s);
            return ec_on ? launch_gemm2_t<2, 2, 1, 2, 2, 2, 1>(a, s) : launch_gemm2_t<2, 2, 0, 2, 2, 2, 1>(a, s);
        }
        if (ec_on == 2)
            return launch_gemm2_t<2, 2, 2, 2, 2, 2>(a, s);
        return ec_on ? launch_gemm2_t<2, 2, 1, 2, 2, 2>(a, s) : launch_gemm2_t<2, 2, 0, 2, 2, 2>(a, s);
    }
    if (a.K % 128 == 0) {
        if (ec_on == 2)
            return launch_gemm2_t<2, 4, 2, 1, 4, 4, 1>(a, s);
        return ec_on ? launch_gemm2_t<2, 4, 1, 1, 4, 4, 1>(a, s) : launch_gemm2_t<2, 4, 0, 1, 4, 4, 1>(a, s);
    }
    if (ec_on == 2)
        return launch_gemm2_t<2, 4, 2>(a, s);
    return ec_on ? launch_gemm2_t<2, 4, 1>(a, s) : launch_gemm2_t<2, 4, 0>(a, s);
}

} // namespace spear
