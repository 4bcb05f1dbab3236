// api.hip -- host side of libspear: argument validation, workspace layout and
// phase-aware dispatch (decode vs prefill) for gfx950.
//
// Source for the dispatch: "SPEAR: A System for Post-Quantization
// Error-Adaptive Recovery Enabling Efficient Low-Bit LLM Serving",
// gist.science summary section 2.2 A (decode: EC fused into the low-bit GEMM
// epilogue; prefill: EC semi-fused).
#include <atomic>
#include <math.h>
#include <mutex>
#include <string.h>

#include "spear_internal.hpp"

namespace spear {

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// EC producers of the fused decode: each workgroup's 4 waves take one K slice
// of *prod_k each, and there are enough workgroups that each reads about
// PROD_BYTES of A times ceil(M / 2).  A workgroup with more tokens streams
// longer (its activations take more LDS traffic), so its producers may read
// more each; fewer producers keep the partials every epilogue loads
// (producers x tokens x ranks) small.  Above 8 tokens the producers' own loads
// are the longest path, so each reads at most 2 PROD_BYTES of A, as long as
// the partials an epilogue loads stay within PROD_WORDS words.  A layer with
// more channel groups than CUs (two stream workgroups a CU) takes producers
// that read a quarter as much each, and above 8 tokens twice the words: there
// the producers' loads are the longer path at 4 to 16 tokens (N = 8192,
// K = 2048: 13.2 / 14.2 / 14.6 -> 10.9 / 11.9 / 13.2 us at 4 / 8 / 16 tokens),
// while the same change slows layers of up to one group a CU (C2: 1020 ->
// 921 GB/s).
constexpr int64_t EC_WIDE_GROUPS = 256;                     // channel groups: one a CU of the chip

static int64_t ec_producers(int64_t mr, int64_t K, int64_t rpad, int64_t ncg, int64_t *prod_k)
{
    const bool wide = ncg > EC_WIDE_GROUPS;
    const int64_t pbytes = wide ? PROD_BYTES / 4 : PROD_BYTES;
    const int64_t pwords = wide ? 2 * PROD_WORDS : PROD_WORDS;
    const int64_t per = mr > 8 ? 2 : cdiv(mr, 2);
    int64_t nprod = cdiv(K * rpad * 2, pbytes * per);
    if (mr > 8) {
        const int64_t cap = pwords / (mr * rpad);
        const int64_t base = cdiv(K * rpad * 2, pbytes * cdiv(mr, 2));
        const int64_t lim = cap > base ? cap : base;       // never fewer than before
        nprod = nprod > lim ? lim : nprod;
    }
    nprod = nprod < 1 ? 1 : (nprod > MAX_PROD ? MAX_PROD : nprod);
    const int64_t most = cdiv(K, DEC_WAVES * 32);           // slices at least 32 deep
    nprod = nprod > most ? most : nprod;
    *prod_k = cdiv(cdiv(K, DEC_WAVES * nprod), 32) * 32;
    return cdiv(K, DEC_WAVES * *prod_k);
}

// MFMA GEMM tiling: tokens and channels per tile, and the K slices a tile is
// split into so that about 256 workgroups run, each over at least 4 stages of
// 128 (one slice when the path takes whole tiles).  Up to 128 tokens the tile
// is 64 x 64, so that narrow layers fill the chip with few or no K slices.
static int64_t gemm_bm(int64_t M, int whole) { return (!whole && M <= 128) ? 64 : 128; }
static int64_t gemm_bn(int64_t bm) { return bm == 64 ? 64 : 256; }

static int64_t gemm_ks(int64_t M, int64_t N, int64_t K, int whole)
{
    if (whole)
        return 1;
    const int64_t bm = gemm_bm(M, 0);
    const int64_t tiles = cdiv(N, gemm_bn(bm)) * cdiv(M > 0 ? M : 1, bm);
    const int64_t most = cdiv(K, 128) / 4;
    int64_t ks = 256 / tiles;
    ks = ks < most ? ks : most;
    return ks > 1 ? ks : 1;
}

// Bytes of fp32 partial tiles a split GEMM writes for M tokens: one
// bm x bn tile per (slice, tile).  The region is sized for the most any token
// count up to M needs, so that a workspace sized for M serves every smaller M.
static size_t gemm_part_bytes(int64_t M, int64_t N, int64_t K)
{
    auto need = [&](int64_t m) -> size_t {
        const int64_t ks = gemm_ks(m, N, K, 0), bm = gemm_bm(m, 0), bn = gemm_bn(bm);
        return ks > 1 ? (size_t)(ks * cdiv(N, bn) * cdiv(m, bm) * bm * bn) * sizeof(float) : 0;
    };
    const int64_t m1 = M < 1 ? 1 : M;
    size_t best = need(m1 < 64 ? m1 : 64);            // up to 64 tokens: one 64-token tile row
    if (m1 > 64) {
        const size_t b2 = need(m1 < 128 ? m1 : 128);  // up to 128 tokens: two 64-token tile rows
        best = b2 > best ? b2 : best;
        for (int64_t tm = 2;; tm++) {                 // tm rows of 128-token tiles
            if (128 * (tm - 1) >= m1)
                break;
            const int64_t m = 128 * tm < m1 ? 128 * tm : m1;
            const size_t b = need(m);
            best = b > best ? b : best;
            if (128 * tm >= m1 || gemm_ks(m, N, K, 0) == 1)
                break;                                // no split for more rows either
        }
    }
    return best;
}

WsLayout ws_layout(int64_t M, int64_t N, int64_t K, int32_t r)
{
    WsLayout L;
    memset(&L, 0, sizeof L);
    L.ncg = cdiv(N, 16);
    // Decode: a workgroup stages the activations of its K range in LDS
    // (M rows of 128-deep super-steps, 256 bytes each plus 16 of padding); a
    // range holds at most DEC_WAVES * DEC_SW_MAX super-steps, split over the
    // workgroup's stream waves.
    const int64_t S = cdiv(K, 128);
    const int64_t mr = M < 1 ? 1 : (M > 16 ? 16 : M);
    int64_t smax = (DEC_LDS_MAX / (mr + 1) - 16) / 256;   // M + 1 rows (one of zeros)
    if (smax > DEC_WAVES * DEC_SW_MAX)
        smax = DEC_WAVES * DEC_SW_MAX;
    L.ksplit = cdiv(S, smax);
    L.spw = cdiv(S, L.ksplit);
    L.rpad = r > 0 ? cdiv(r, 32) * 32 : 0;
    L.mpad = cdiv(M > 0 ? M : 1, 16) * 16;
    L.nprod = r > 0 ? ec_producers(mr, K, L.rpad, L.ncg, &L.prod_k) : 0;
    // The partials region is sized for the most producers any token count
    // uses (one token), so that a workspace sized for some M also serves every
    // smaller M, and the decode path after the prefill path.
    int64_t pk1 = 0;
    const int64_t nprod_max = r > 0 ? ec_producers(1, K, L.rpad, L.ncg, &pk1) : 0;

    size_t off = 0;
    L.hdr = off;
    off = align256(off + HDR_WORDS * sizeof(uint32_t));
    L.epoch = off;
    off = align256(off + (size_t)EPOCH_CTRS * EPOCH_STRIDE);
    L.zeros = off;                                        // 256 bytes that stay zero: DMA source
    off = align256(off + 256);
    // Decode with K split over workgroups: tagged 64-bit words {value, launch
    // epoch} of each range's sums, [channel group][range][lane][5].
    L.splitp = off;
    if (L.ksplit > 1)                                     // any M: a larger M never needs less
        off = align256(off + (size_t)(L.ncg * L.ksplit * 64 * 5) * sizeof(uint64_t));
    // Producer partials, tagged 64-bit words {value, launch epoch}: u per
    // (producer, token slot, rank) and the fp64 gate logit as two words.
    L.pu = off;
    L.pz = off;
    if (r > 0) {
        off = align256(off + (size_t)(nprod_max * 16 * L.rpad) * sizeof(uint64_t));
        L.pz = off;
        off = align256(off + (size_t)(nprod_max * 16 * 2) * sizeof(uint64_t));
    }
    L.vhi = L.vlo = L.vtag = L.active = L.preu = L.prez = off;
    if (r > 0) {
        L.vhi = off;
        off = align256(off + (size_t)(L.mpad * L.rpad) * 2);
        L.vlo = off;
        off = align256(off + (size_t)(L.mpad * L.rpad) * 2);
        // v as tagged words, when the pre-pass shares the K-split GEMM's launch
        // (fewer than PRE_GROUPS token groups)
        L.vtag = off;
        const int64_t mt = L.mpad < PRE_GROUPS * 16 ? L.mpad : PRE_GROUPS * 16;
        off = align256(off + (size_t)(mt * L.rpad) * sizeof(uint64_t));
        L.active = off;
        off = align256(off + (size_t)L.mpad * 4);
        L.idx = off;                                      // token list, then its count
        off = align256(off + (size_t)(L.mpad + 1) * 4);
        // EC pre-pass with K split over workgroups: per-slot partials as tagged
        // 64-bit words (sized independently of M).
        L.preu = off;
        off = align256(off + (size_t)PRE_SLOTS * 16 * L.rpad * sizeof(uint64_t));
        L.prez = off;
        off = align256(off + (size_t)PRE_SLOTS * 16 * 2 * sizeof(uint64_t));
    }
    L.gpart = off;
    off = align256(off + gemm_part_bytes(M, N, K));
    L.total = off;
    return L;
}

// Wait limit of later launches (0: the default); set from any thread.
static std::atomic<uint32_t> g_wait_limit{0};
static const uint32_t DEFAULT_WAIT_LIMIT = 1u << 20;

// gfx950 check, cached per device.
static spear_status check_device()
{
    static std::mutex mu;
    static int known[64];   // 0 unknown, 1 ok, 2 not gfx950
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return SPEAR_E_HIP;
    if (dev < 0 || dev >= 64)
        return SPEAR_E_DEVICE;
    std::lock_guard<std::mutex> lk(mu);
    if (known[dev] == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess)
            return SPEAR_E_HIP;
        known[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    return known[dev] == 1 ? SPEAR_OK : SPEAR_E_DEVICE;
}

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

static double logit_threshold(float tau)
{
    const double t = (double)tau;
    if (t >= 1.0)
        return INFINITY;
    if (t <= 0.0)
        return -INFINITY;
    return log(t / (1.0 - t));
}

static spear_status hip_status(hipError_t e) { return e == hipSuccess ? SPEAR_OK : SPEAR_E_HIP; }

static const int64_t GRID_MAX = 0x7FFFFFFF;

} // namespace spear

using namespace spear;

extern "C" {

int32_t spear_abi_version(void) { return SPEAR_ABI_VERSION; }

const char *spear_status_string(spear_status s)
{
    switch (s) {
    case SPEAR_OK: return "ok";
    case SPEAR_E_NULL: return "a required pointer is NULL";
    case SPEAR_E_SHAPE: return "a size is out of range";
    case SPEAR_E_ALIGN: return "a pointer is not aligned as required";
    case SPEAR_E_ARG: return "an argument value is invalid";
    case SPEAR_E_WORKSPACE: return "workspace too small";
    case SPEAR_E_HIP: return "HIP runtime error";
    case SPEAR_E_DEVICE: return "current device is not gfx950";
    default: return "unknown status";
    }
}

void spear_set_wait_limit(uint32_t rounds) { g_wait_limit.store(rounds, std::memory_order_relaxed); }

spear_status spear_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream)
{
    if (!buf || !sink)
        return SPEAR_E_NULL;
    if (bytes < 16 || bytes % 16 != 0)
        return SPEAR_E_SHAPE;
    if (!aligned(buf, 16) || !aligned(sink, 4))
        return SPEAR_E_ALIGN;
    spear_status st = check_device();
    if (st != SPEAR_OK)
        return st;
    return hip_status(launch_stream_read(buf, bytes, sink, (hipStream_t)stream));
}

spear_status spear_pack_w4(const void *codes, int32_t code_kind, int64_t N, int64_t K,
                           uint8_t *packed, int32_t *bad_codes, void *stream)
{
    if (!codes || !packed)
        return SPEAR_E_NULL;
    if (N < 1 || K < 32 || K % 32 != 0 || N > ((int64_t)1 << 40) / K)
        return SPEAR_E_SHAPE;
    if (code_kind != SPEAR_CODES_S4 && code_kind != SPEAR_CODES_U4)
        return SPEAR_E_ARG;
    if (!aligned(codes, 16) || !aligned(packed, 16) || !aligned(bad_codes, 4))
        return SPEAR_E_ALIGN;
    if (cdiv(N * K / 16, 256) > GRID_MAX)
        return SPEAR_E_SHAPE;
    spear_status st = check_device();
    if (st != SPEAR_OK)
        return st;
    return hip_status(launch_pack(codes, code_kind, N, K, packed, bad_codes, (hipStream_t)stream));
}

spear_status spear_gate(const spear_bf16 *x, int64_t M, int64_t K, const spear_bf16 *w_gate,
                        float b, float tau, int32_t hard, float *g, int32_t *idx,
                        int32_t *n_active, void *stream)
{
    if (!w_gate || !n_active || (M > 0 && (!x || !g || !idx)))
        return SPEAR_E_NULL;
    if (M < 0 || K < 32 || K % 32 != 0 || cdiv(M, 4) > GRID_MAX)
        return SPEAR_E_SHAPE;
    if (isnan(tau) || isnan(b) || (hard != 0 && hard != 1))
        return SPEAR_E_ARG;
    if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(g, 4) || !aligned(idx, 4) ||
        !aligned(n_active, 4))
        return SPEAR_E_ALIGN;
    spear_status st = check_device();
    if (st != SPEAR_OK)
        return st;
    return hip_status(launch_gate(x, M, K, w_gate, b, logit_threshold(tau), hard, g, idx,
                                  n_active, (hipStream_t)stream));
}

size_t spear_w4_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r)
{
    if (M < 0 || N < 1 || K < 32 || r < 0)
        return 0;
    return ws_layout(M, N, K, r).total;
}

spear_status spear_workspace_init(void *ws, size_t bytes, void *stream)
{
    if (!ws)
        return SPEAR_E_NULL;
    if (bytes < 256)
        return SPEAR_E_WORKSPACE;
    if (!aligned(ws, 256))
        return SPEAR_E_ALIGN;
    spear_status st = check_device();
    if (st != SPEAR_OK)
        return st;
    return hip_status(launch_zero(ws, bytes, (hipStream_t)stream));
}

spear_status spear_workspace_timeouts(void *workspace, int32_t *host_count, void *stream)
{
    if (!workspace || !host_count)
        return SPEAR_E_NULL;
    if (!aligned(workspace, 256))
        return SPEAR_E_ALIGN;
    spear_status st = check_device();
    if (st != SPEAR_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    uint32_t *cnt = reinterpret_cast<uint32_t *>(workspace) + HDR_TIMEOUTS;
    uint32_t v = 0;
    if (hipMemcpyAsync(&v, cnt, sizeof v, hipMemcpyDeviceToHost, s) != hipSuccess)
        return SPEAR_E_HIP;
    if (launch_zero(cnt, sizeof v, s) != hipSuccess)
        return SPEAR_E_HIP;
    if (hipStreamSynchronize(s) != hipSuccess)
        return SPEAR_E_HIP;
    *host_count = (int32_t)v;
    return SPEAR_OK;
}

} // extern "C"

namespace spear {

// Host-only argument checks of a layer call (no HIP call); *path is resolved
// from SPEAR_PATH_AUTO.
static spear_status validate_linear(const spear_bf16 *x, int64_t M, const spear_w4 *w,
                                    const spear_ec *ec, const void *y, int32_t out_dtype,
                                    const void *workspace, size_t ws_bytes, int32_t *path_io)
{
    int32_t path = *path_io;
    if (!w || !workspace || !w->packed || !w->scales)
        return SPEAR_E_NULL;
    if (M > 0 && (!x || !y))
        return SPEAR_E_NULL;
    if (ec && (!ec->A || !ec->B || !ec->w_gate))
        return SPEAR_E_NULL;
    const int64_t N = w->N, K = w->K;
    if (M < 0 || N < 1 || K < 32 || K % 32 != 0)
        return SPEAR_E_SHAPE;
    if (ec && (ec->r < 8 || ec->r > SPEAR_MAX_RANK || ec->r % 8 != 0))
        return SPEAR_E_SHAPE;
    if (path < SPEAR_PATH_AUTO || path > SPEAR_PATH_PREFILL_LARGE)
        return SPEAR_E_ARG;
    if (out_dtype != SPEAR_OUT_BF16 && out_dtype != SPEAR_OUT_F32)
        return SPEAR_E_ARG;
    if (ec && (isnan(ec->tau) || isnan(ec->b) || (ec->hard != 0 && ec->hard != 1)))
        return SPEAR_E_ARG;
    if (ec && (ec->gate_h < 0 || ec->gate_h > SPEAR_MAX_GATE_HIDDEN))
        return SPEAR_E_SHAPE;
    if (ec && ec->gate_h > 0 &&
        (!ec->gate_w1 || !ec->gate_c1 || !ec->gate_w2 || !ec->gate_c2))
        return SPEAR_E_NULL;
    if (ec && ec->gate_h > 0 && isnan(ec->alpha))
        return SPEAR_E_ARG;
    if (path == SPEAR_PATH_AUTO)
        path = M <= 16 ? SPEAR_PATH_DECODE : SPEAR_PATH_PREFILL;
    if ((path == SPEAR_PATH_DECODE || path == SPEAR_PATH_DECODE_2PASS) && M > 16)
        return SPEAR_E_SHAPE;
    if (!aligned(x, 16) || !aligned(w->packed, 16) || !aligned(w->scales, 4) ||
        !aligned(y, 16) || !aligned(workspace, 256))
        return SPEAR_E_ALIGN;
    if (ec && (!aligned(ec->A, 16) || !aligned(ec->B, 16) || !aligned(ec->w_gate, 16) ||
               !aligned(ec->g_out, 4) || !aligned(ec->idx_out, 4) ||
               !aligned(ec->n_active_out, 4)))
        return SPEAR_E_ALIGN;
    if (ec && ec->gate_h > 0 &&
        (!aligned(ec->gate_w1, 4) || !aligned(ec->gate_c1, 4) || !aligned(ec->gate_w2, 4) ||
         !aligned(ec->gate_c2, 4)))
        return SPEAR_E_ALIGN;
    const int32_t r = ec ? ec->r : 0;
    const WsLayout L = ws_layout(M, N, K, r);
    if (ws_bytes < L.total)
        return SPEAR_E_WORKSPACE;
    if (L.ncg * L.ksplit > GRID_MAX || cdiv(N, 64) * cdiv(M, 64) > GRID_MAX)
        return SPEAR_E_SHAPE;
    // the decode kernels take their workspace offsets as 32-bit values
    if ((path == SPEAR_PATH_DECODE || path == SPEAR_PATH_DECODE_2PASS) && L.active > 0xFFFFFFFFull)
        return SPEAR_E_SHAPE;
    *path_io = path;
    return SPEAR_OK;
}

// The kernel arguments of a validated call.
static void fill_args(LinearArgs &a, const spear_bf16 *x, int64_t M, const spear_w4 *w,
                      const spear_ec *ec, void *y, int32_t out_dtype, void *workspace,
                      int32_t path, const WsLayout &L)
{
    const int64_t N = w->N, K = w->K;
    memset(&a, 0, sizeof a);
    a.x = x;
    a.packed = w->packed;
    a.scales = w->scales;
    a.zeros = w->zeros;
    a.y = y;
    a.ws = reinterpret_cast<uint8_t *>(workspace);
    a.M = M;
    a.N = N;
    a.K = K;
    a.ncg = (int32_t)L.ncg;
    a.ksplit = (int32_t)L.ksplit;
    a.spw = (int32_t)L.spw;
    a.nprod = (int32_t)L.nprod;
    a.prod_k = (int32_t)L.prod_k;
    a.mpad = L.mpad;
    {
        // EC pre-pass: few token groups split K so that up to about 256
        // workgroups run, each over at least 8 steps of 32 (one per wave).
        const int64_t tg = cdiv(M > 0 ? M : 1, 16), T = K / 32;
        int64_t ks = 1;
        if (tg < PRE_GROUPS) {
            ks = cdiv(256, tg);
            const int64_t most = T / 8 > 0 ? T / 8 : 1;
            ks = ks < most ? ks : most;
        }
        a.pre_ks = (int32_t)ks;
    }
    a.g_bm = (int32_t)gemm_bm(M, path == SPEAR_PATH_PREFILL_LARGE);
    a.g_bn = (int32_t)gemm_bn(a.g_bm);
    a.g_ks = (int32_t)gemm_ks(M, N, K, path == SPEAR_PATH_PREFILL_LARGE);
    a.L = L;
    a.P.hdr = L.hdr;
    a.P.zeros = L.zeros;
    a.P.vhi = L.vhi;
    a.P.vlo = L.vlo;
    a.P.vtag = L.vtag;
    a.P.active = L.active;
    a.P.preu = L.preu;
    a.P.prez = L.prez;
    a.P.gpart = L.gpart;
    a.P.idx = L.idx;
    // 32-bit copies for the decode kernels (checked on their paths; the
    // others read only hdr and epoch from here, at the start of the layout)
    a.D.hdr = (uint32_t)L.hdr;
    a.D.epoch = (uint32_t)L.epoch;
    a.D.splitp = (uint32_t)L.splitp;
    a.D.pu = (uint32_t)L.pu;
    a.D.pz = (uint32_t)L.pz;
    a.D.vhi = (uint32_t)L.vhi;
    a.D.vlo = (uint32_t)L.vlo;
    a.D.active = (uint32_t)L.active;
    a.out_f32 = out_dtype == SPEAR_OUT_F32;
    const uint32_t wl = g_wait_limit.load(std::memory_order_relaxed);
    a.wait_limit = wl ? wl : DEFAULT_WAIT_LIMIT;
    if (ec) {
        a.A = ec->A;
        a.B = ec->B;
        a.wg = ec->w_gate;
        a.b = ec->b;
        a.thr = logit_threshold(ec->tau);
        a.hard = ec->hard;
        a.r = ec->r;
        a.rpad = (int32_t)L.rpad;
        a.g_out = ec->g_out;
        a.idx_out = ec->idx_out;
        a.nact_out = ec->n_active_out;
        if (ec->gate_h > 0) {
            a.gate_h = ec->gate_h;
            a.alpha = ec->alpha;
            a.gw1 = ec->gate_w1;
            a.gc1 = ec->gate_c1;
            a.gw2 = ec->gate_w2;
            a.gc2 = ec->gate_c2;
        }
    }

}

// The launches of one path.
static spear_status launch_path(LinearArgs &a, const spear_ec *ec, int32_t path, hipStream_t s)
{
    const int64_t M = a.M, N = a.N, K = a.K;
    hipError_t e = hipSuccess;
    const int32_t *active = reinterpret_cast<const int32_t *>(a.ws + a.L.active);
    switch (path) {
    case SPEAR_PATH_DECODE:
        if (!(ec && ec->gate_h > 0 && a.rpad > 32)) {
            e = launch_decode(a, ec ? 1 : 0, s);
            break;
        }
        // a vector gate over more than one 32-rank block is formed by the
        // pre-pass: two launches
        [[fallthrough]];
    case SPEAR_PATH_DECODE_2PASS:
        if (ec) {
            e = launch_prepass(a, s);
            if (e == hipSuccess && (a.idx_out || a.nact_out))
                e = launch_compact(active, M, a.idx_out, a.nact_out, s);
        }
        if (e == hipSuccess)
            e = launch_decode(a, ec ? 2 : 0, s);
        break;
    default:
        if (ec && (a.g_ks > 1 || a.g_bm == 64) && cdiv(M, 16) < PRE_GROUPS) {
            // Few GEMM tiles (a K split, or 64 x 64 tiles): the pre-pass runs as
            // the first blocks of the GEMM's launch, on the CUs the GEMM's tiles
            // leave free, and the epilogues wait for its tagged v.  About that
            // many pre-pass workgroups (at least 32), each of its waves over at
            // least one step of 32.
            const int64_t tg = cdiv(M, 16), T = K / 32, pw = 8;   // the GEMM's 8 waves
            const int64_t gwg = cdiv(N, a.g_bn) * cdiv(M, a.g_bm) * a.g_ks;
            const int64_t room = gwg < 256 - 32 ? 256 - gwg : 32;
            int64_t ks = cdiv(room, tg);
            const int64_t most = T / pw > 0 ? T / pw : 1;
            ks = ks < most ? ks : most;
            a.pre_ks = (int32_t)ks;
            a.npre = (int32_t)(cdiv(tg * ks, 8) * 8);     // XCD-aligned start of the GEMM blocks
            e = launch_gemm(a, 2, 0, s);
            if (e == hipSuccess && (a.idx_out || a.nact_out))
                e = launch_compact(active, M, a.idx_out, a.nact_out, s);
            break;
        }
        if (ec) {
            e = launch_prepass(a, s);
            if (e == hipSuccess && (a.idx_out || a.nact_out))
                e = launch_compact(active, M, a.idx_out, a.nact_out, s);
        }
        if (e == hipSuccess)
            e = launch_gemm(a, ec ? 1 : 0, path == SPEAR_PATH_PREFILL_LARGE, s);
        break;
    }
    return hip_status(e);
}

// A validated layer call: dispatch and launch on `stream`.
static spear_status run_linear(const spear_bf16 *x, int64_t M, const spear_w4 *w,
                               const spear_ec *ec, void *y, int32_t out_dtype, void *workspace,
                               int32_t path, void *stream)
{
    const int64_t N = w->N, K = w->K;
    const WsLayout L = ws_layout(M, N, K, ec ? ec->r : 0);
    spear_status st = check_device();
    if (st != SPEAR_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;

    if (M == 0) {
        if (ec && ec->n_active_out)
            return hip_status(launch_zero(ec->n_active_out, sizeof(int32_t), s));
        return SPEAR_OK;
    }

    LinearArgs a;
    fill_args(a, x, M, w, ec, y, out_dtype, workspace, path, L);
    return launch_path(a, ec, path, s);
}


// Scratch of the allocation-free entry point: one copy per GPU, zero at load
// (static storage), held until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory; its device address is
// looked up once per device and kept in scratch_ptr.
static __device__ __align__(256) uint8_t scratch[SPEAR_NOALLOC_MAX_WORKSPACE];

static spear_status scratch_address(void **out)
{
    static std::mutex mu;
    static void *scratch_ptr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return SPEAR_E_HIP;
    if (dev < 0 || dev >= 64)
        return SPEAR_E_DEVICE;
    std::lock_guard<std::mutex> lk(mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return SPEAR_E_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return SPEAR_OK;
}

} // namespace spear

extern "C" {

spear_status spear_w4_linear_path(const spear_bf16 *x, int64_t M, const spear_w4 *w,
                                  const spear_ec *ec, void *y, int32_t out_dtype,
                                  void *workspace, size_t ws_bytes, int32_t path, void *stream)
{
    spear_status st = validate_linear(x, M, w, ec, y, out_dtype, workspace, ws_bytes, &path);
    if (st != SPEAR_OK)
        return st;
    return run_linear(x, M, w, ec, y, out_dtype, workspace, path, stream);
}

spear_status spear_w4_linear_noalloc(const spear_bf16 *x, int64_t M, const spear_w4 *w,
                                     const spear_ec *ec, void *y, int32_t out_dtype,
                                     int32_t path, void *stream)
{
    // validated against the scratch's size with an aligned stand-in address
    const void *standin = reinterpret_cast<const void *>((uintptr_t)256);
    spear_status st = validate_linear(x, M, w, ec, y, out_dtype, standin,
                                      SPEAR_NOALLOC_MAX_WORKSPACE, &path);
    if (st != SPEAR_OK)
        return st;
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != SPEAR_OK)
        return st;
    return run_linear(x, M, w, ec, y, out_dtype, ws, path, stream);
}

spear_status spear_w4_linear_semifused(const spear_bf16 *x, int64_t M, const spear_w4 *w,
                                       const spear_ec *ec, float *y, void *workspace,
                                       size_t ws_bytes, void *stream, void *aux_stream,
                                       void *ev_fork, void *ev_join)
{
    int32_t path = SPEAR_PATH_PREFILL;
    spear_status st = validate_linear(x, M, w, ec, y, SPEAR_OUT_F32, workspace, ws_bytes, &path);
    if (st != SPEAR_OK)
        return st;
    if (ec && (!ev_fork || !ev_join))
        return SPEAR_E_NULL;
    if (ec && aux_stream == stream)
        return SPEAR_E_ARG;
    if (!ec || M == 0)
        return run_linear(x, M, w, ec, y, SPEAR_OUT_F32, workspace, path, stream);
    st = check_device();
    if (st != SPEAR_OK)
        return st;
    const WsLayout L = ws_layout(M, w->N, w->K, ec->r);
    LinearArgs a;
    fill_args(a, x, M, w, ec, y, SPEAR_OUT_F32, workspace, path, L);
    hipStream_t s = (hipStream_t)stream, s2 = (hipStream_t)aux_stream;
    hipEvent_t e0 = (hipEvent_t)ev_fork, e1 = (hipEvent_t)ev_join;
    int32_t *active = reinterpret_cast<int32_t *>(a.ws + L.active);
    int32_t *list = reinterpret_cast<int32_t *>(a.ws + L.idx);
    // fork: the EC branch on the auxiliary stream
    hipError_t e = hipEventRecord(e0, s);
    if (e == hipSuccess)
        e = hipStreamWaitEvent(s2, e0, 0);
    if (e == hipSuccess)
        e = launch_prepass(a, s2);
    if (e == hipSuccess)
        e = launch_compact(active, M, list, list + L.mpad, s2, a.idx_out, a.nact_out);
    if (e == hipSuccess)
        e = hipEventRecord(e1, s2);
    // the plain W4 GEMM on the caller's stream, beside it
    if (e == hipSuccess)
        e = launch_gemm(a, 0, 0, s);
    // join, then the EC kernel over the active tokens
    if (e == hipSuccess)
        e = hipStreamWaitEvent(s, e1, 0);
    if (e == hipSuccess)
        e = launch_ec_apply(a, s);
    return hip_status(e);
}

spear_status spear_w4_linear(const spear_bf16 *x, int64_t M, const spear_w4 *w,
                             const spear_ec *ec, void *y, int32_t out_dtype, void *workspace,
                             size_t ws_bytes, void *stream)
{
    return spear_w4_linear_path(x, M, w, ec, y, out_dtype, workspace, ws_bytes,
                                SPEAR_PATH_AUTO, stream);
}

} // extern "C"
