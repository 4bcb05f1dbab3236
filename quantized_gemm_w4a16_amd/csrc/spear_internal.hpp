// spear_internal.hpp -- device helpers, workspace layout and launcher
// declarations shared by the translation units of libspear (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spear.h"

namespace spear {

// ---------------------------------------------------------------- vector types
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// One bf16 MFMA, 16x16 output, 32-deep.  Operand layout (wave64): lane l holds
// row (l % 16) of A and column (l % 16) of B, each for the 8 consecutive depth
// positions 8*(l / 16) .. +7; the result lane l holds rows 4*(l / 16) .. +3 of
// column (l % 16).  Any permutation of the depth positions applied to both
// operands alike leaves the result unchanged.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One packed word (8 codes; nibble position p holds code (0,2,4,6,1,3,5,7)[p])
// -> bf16 pairs holding 1 + u/16 exactly: the nibble becomes the top 4 of the 7
// mantissa bits of a value in [1, 2).  Pair p takes nibble positions (p, p + 4),
// i.e. codes (2p, 2p + 1): the pairs come out in natural order, as the
// activations' bf16 pairs lie.  The epilogue removes the offset and the zero point:
// 16 sum x (1 + u/16) - (16 + z) sum x = sum x (u - z).  Keeping the nibble in
// the high mantissa bits keeps that offset small (16 sum x).
__device__ __forceinline__ u32x4 unpack8(uint32_t w)
{
    // The mask and the exponent bits go through registers so that each output
    // is one shift and one v_and_or_b32 (two literals cannot share one VOP3).
    uint32_t m, c;
    asm("s_mov_b32 %0, 0x780078" : "=s"(m));
    asm("v_mov_b32 %0, 0x3f803f80" : "=v"(c));
    u32x4 r;
    r[0] = ((w << 3) & m) | c;
    r[1] = ((w >> 1) & m) | c;
    r[2] = ((w >> 5) & m) | c;
    r[3] = ((w >> 9) & m) | c;
    return r;
}

// Scale of the unpacked value and the offset it carries: unpacked = (OFF + u) / SCALE.
constexpr float UNPACK_SCALE = 16.0f;
constexpr float UNPACK_OFF = 16.0f;

__device__ __forceinline__ u32x4 ld16(const void *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ u32x4 zero4()
{
    u32x4 z = {0u, 0u, 0u, 0u};
    return z;
}

__device__ __forceinline__ float bf16f(uint16_t h)
{
    return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint16_t f2bf(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v)
{
    // element-wise bit casts of vector lanes miscompile with this toolchain;
    // copy through a scalar instead
    bf16x2 r;
    __builtin_memcpy(&r, &v, sizeof r);
    return r;
}

// sum of the 8 bf16 in d (fp32 accumulate, two per dot2).
__device__ __forceinline__ float sum8(u32x4 d, float acc)
{
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const uint32_t t = d[e];
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(t), one, acc, false);
    }
    return acc;
}

// Zero points are read without a branch (a load under a branch makes the
// compiler wait for every outstanding load where the branch ends): with no
// zero points the byte is read from the scales array, which is always valid
// and at least N bytes long, and replaced by 8 where it is used.
__device__ __forceinline__ uint32_t load_zero_byte(const uint8_t *zeros, const float *scales,
                                                   int64_t n)
{
    const uint8_t *p = zeros ? zeros : reinterpret_cast<const uint8_t *>(scales);
    return p[n];
}
__device__ __forceinline__ float zero_point(const uint8_t *zeros, uint32_t raw)
{
    return zeros ? (float)raw : 8.f;
}

// ------------------------------------------------------------ workspace layout
// Header: 64 uint32 counters, all zero between calls.
enum {
    HDR_TIMEOUTS = 4,  // bounded waits that expired (cleared by the host query)
    HDR_WORDS = 64
};

constexpr int DEC_WAVES = 4;        // decode workgroup: 4 waves split its K range
constexpr int DEC_SW_MAX = 8;       // 128-deep super-steps per decode wave, at most
constexpr int DEC_LDS_MAX = 81920;  // LDS bytes of staged activations (M + 1 rows), at most
// Launch epoch of the fused decode: 64-bit counters, one per 128-byte line so
// that the per-workgroup claims do not queue behind each other on one address.
constexpr int EPOCH_CTRS = 64;
constexpr int EPOCH_STRIDE = 128;

constexpr int PROD_BYTES = 8192;  // bytes of A an EC producer workgroup reads, about
constexpr int MAX_PROD = 32;      // at most this many EC producer workgroups
constexpr int PROD_WORDS = 4096;  // above 8 tokens: partial words an epilogue loads, at most
constexpr int PROD_CHUNK = 4;     // producer partials a consumer wave loads per batch
constexpr int PRE_SLOTS = 512;    // EC pre-pass: (token group, K slice) partial slots, at most
                                  // (fewer than PRE_GROUPS groups, about 256 workgroups)
constexpr int PRE_GROUPS = 128;   // EC pre-pass: token groups below which K is split

struct WsLayout {
    size_t hdr, epoch, zeros, splitp, pu, pz, vhi, vlo, vtag, active, preu, prez, gpart, total;
    size_t idx;         // semi-fused prefill: the active-token list [mpad], then its count
    int64_t ncg, ksplit, spw, nprod, prod_k, rpad, mpad;
};

WsLayout ws_layout(int64_t M, int64_t N, int64_t K, int32_t r);

// ------------------------------------------------------------- kernel params
// Offsets (bytes) of the workspace regions the decode kernels use.  A decode
// call's layout holds only small regions ahead of them (the host checks that
// they fit 32 bits).
struct DecOffsets {
    uint32_t hdr, epoch, splitp, pu, pz, vhi, vlo, active;
};

struct LinearArgs {
    // The leading block (212 bytes, four 64-byte lines) is what the decode
    // kernels load at entry.  Each further 64-byte line of arguments a kernel
    // loads adds about 0.35 us to its launch (measured in graph replay: 3.1 us
    // for one line, 3.9 us for four, 5.0 us for eight), so the fields they use
    // come first and no wider than they need to be.
    const uint16_t *x;
    const uint8_t *packed;
    const float *scales;
    const uint8_t *zeros;
    const uint16_t *A, *B, *wg;
    void *y;
    uint8_t *ws;
    float *g_out;
    int32_t *idx_out;
    int32_t *nact_out;
    int64_t M, N, K;
    double thr;      // logit(tau) for the hard gate
    float b;
    int32_t hard;
    int32_t r, rpad;
    int32_t ncg, ksplit, spw, nprod, prod_k;   // decode: channel groups, K ranges, EC producers
    uint32_t wait_limit;
    int32_t out_f32;
    int32_t gate_h;  // vector gate: hidden width (0: scalar gate only)
    float alpha;
    DecOffsets D;
    uint32_t grid;   // the launch's workgroups (gridDim's hidden argument sits in a line of its own)
    // The prefill kernels load the leading block and this one (bytes 0 to 359,
    // six lines): the vector gate MLP, the prefill tiling and the offsets of the
    // workspace regions they use (64-bit: a prefill workspace may pass 4 GiB).
    const float *gw1, *gc1, *gw2, *gc2;   // vector gate MLP (gate_h > 0)
    int32_t pre_ks;  // EC pre-pass: K slices per token group
    int32_t g_bm;    // MFMA GEMM: tokens per tile (64 or 128)
    int32_t g_bn;    // MFMA GEMM: channels per tile (64 with 64-token tiles, else 256)
    int32_t g_ks;    // MFMA GEMM: K slices per tile (partials reduced by a second launch)
    int32_t npre;    // K-split GEMM with the EC pre-pass in its launch: leading pre-pass blocks
    int64_t mpad;
    struct {
        size_t hdr, zeros, vhi, vlo, vtag, active, preu, prez, gpart, idx;
    } P;
    // Host side only.
    WsLayout L;
};
static_assert(offsetof(LinearArgs, gw1) == 216 && offsetof(LinearArgs, D) == 180 &&
                  offsetof(LinearArgs, grid) == 212 && offsetof(LinearArgs, L) == 360,
              "the decode kernels' leading block");

// Explicit counter waits (gfx9 s_waitcnt encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8) and a barrier without the fence of
// __syncthreads, for code that orders its memory operations itself.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void bare_barrier() { __builtin_amdgcn_s_barrier(); }

// Load the arguments a kernel uses at entry, in one batch.  The compiler
// otherwise fetches fields of a large argument struct lazily, in several
// batches that each cost a memory round trip before the first data load can
// be issued; and each 64-byte line of arguments loaded costs about 0.35 us a
// launch, so each kernel family loads only the leading lines it uses.
template <typename T>
__device__ __forceinline__ void pin_arg(const T &v)
{
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "scalar argument");
    if constexpr (sizeof(T) == 8)
        asm volatile("" ::"s"(__builtin_bit_cast(uint64_t, v)));
    else
        asm volatile("" ::"s"(__builtin_bit_cast(uint32_t, v)));
}


// The decode kernels' arguments: the leading block only (the vector gate's
// weights are loaded where that path needs them).
__device__ __forceinline__ void pin_dec_args(const LinearArgs &a)
{
    pin_arg(a.x); pin_arg(a.packed); pin_arg(a.scales); pin_arg(a.zeros); pin_arg(a.A);
    pin_arg(a.B); pin_arg(a.wg); pin_arg(a.y); pin_arg(a.ws); pin_arg(a.g_out);
    pin_arg(a.idx_out); pin_arg(a.nact_out); pin_arg(a.M); pin_arg(a.N); pin_arg(a.K);
    pin_arg(a.thr); pin_arg(a.b); pin_arg(a.hard); pin_arg(a.r); pin_arg(a.rpad);
    pin_arg(a.ncg); pin_arg(a.ksplit); pin_arg(a.spw); pin_arg(a.nprod); pin_arg(a.prod_k);
    pin_arg(a.wait_limit); pin_arg(a.out_f32); pin_arg(a.gate_h); pin_arg(a.alpha);
    pin_arg(a.D.hdr); pin_arg(a.D.epoch); pin_arg(a.D.splitp); pin_arg(a.D.pu);
    pin_arg(a.D.pz); pin_arg(a.D.vhi); pin_arg(a.D.vlo); pin_arg(a.D.active); pin_arg(a.grid);
}

// The prefill kernels' arguments: the leading block and the prefill block.
__device__ __forceinline__ void pin_pre_args(const LinearArgs &a)
{
    pin_dec_args(a);
    pin_arg(a.gw1); pin_arg(a.gc1); pin_arg(a.gw2); pin_arg(a.gc2);
    pin_arg(a.pre_ks); pin_arg(a.g_bm); pin_arg(a.g_bn); pin_arg(a.g_ks); pin_arg(a.npre);
    pin_arg(a.mpad);
    pin_arg(a.P.hdr); pin_arg(a.P.zeros); pin_arg(a.P.vhi); pin_arg(a.P.vlo); pin_arg(a.P.vtag);
    pin_arg(a.P.active); pin_arg(a.P.preu); pin_arg(a.P.prez); pin_arg(a.P.gpart); pin_arg(a.P.idx);
}

// ---------------------------------------------- tagged cross-workgroup exchange
// One atomic add per workgroup.  Block b claims on counter b % EPOCH_CTRS and
// a launch adds exactly 2^32 to every counter: the first block of each class
// adds 2^32 - (n - 1), the n - 1 others of the class 1 each, and block 0 adds
// 2^32 to the counters no block of a small grid uses.  Between launches all
// counters hold the same multiple of 2^32, so every block of a launch reads the
// same upper half whatever the order of the adds.  G is the launch's grid size.
__device__ __forceinline__ uint64_t epoch_claim(const LinearArgs &a, uint32_t G)
{
    uint8_t *base = a.ws + a.D.epoch;
    const uint32_t bid = blockIdx.x, c = bid % EPOCH_CTRS;
    uint64_t add = 1;
    if (bid < EPOCH_CTRS)
        add = (1ull << 32) - ((G - 1 - c) / EPOCH_CTRS + 1) + 1;
    if (bid == 0)
        for (uint32_t cc = G; cc < EPOCH_CTRS; cc++)
            __hip_atomic_fetch_add(reinterpret_cast<uint64_t *>(base + (size_t)cc * EPOCH_STRIDE),
                                   1ull << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __hip_atomic_fetch_add(reinterpret_cast<uint64_t *>(base + (size_t)c * EPOCH_STRIDE), add,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Tag of the launch (a zeroed workspace holds tag 0, which no launch uses).
__device__ __forceinline__ uint32_t epoch_tag(uint64_t claimed) { return (uint32_t)(claimed >> 32) + 1u; }

// A zero the compiler cannot see through.  The epoch claim returns into two
// registers long before its value is used; with a literal zero on the other
// path the tag arithmetic is folded (or hoisted) to right behind the atomic,
// and a dead low half lets its register be reused, and each of these makes the
// wave wait for the atomic and every older load there.  Adding this opaque
// zero at the use keeps the arithmetic, and both registers, where they belong.
__device__ __forceinline__ uint64_t opaque_zero64()
{
    uint32_t lo, hi;
    asm volatile("v_mov_b32 %0, 0" : "=v"(lo));
    asm volatile("v_mov_b32 %0, 0" : "=v"(hi));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void store_tagged(uint64_t *p, uint32_t bits, uint32_t tag)
{
    __hip_atomic_store(p, ((uint64_t)tag << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_tagged(const uint64_t *p)
{
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


hipError_t launch_pack(const void *codes, int32_t kind, int64_t N, int64_t K, uint8_t *packed,
                       int32_t *bad, hipStream_t s);
hipError_t launch_gate(const uint16_t *x, int64_t M, int64_t K, const uint16_t *wg, float b,
                       double thr, int32_t hard, float *g, int32_t *idx, int32_t *nact,
                       hipStream_t s);
hipError_t launch_compact(const int32_t *flags, int64_t M, int32_t *idx, int32_t *nact,
                          hipStream_t s, int32_t *idx2 = nullptr, int32_t *nact2 = nullptr);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_stream_read(const void *p, size_t bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_decode(const LinearArgs &a, int ec_mode, hipStream_t s);
hipError_t launch_prepass(const LinearArgs &a, hipStream_t s);
hipError_t launch_gemm(const LinearArgs &a, int ec_on, int force_large, hipStream_t s);
hipError_t launch_ec_apply(const LinearArgs &a, hipStream_t s);

} // namespace spear
