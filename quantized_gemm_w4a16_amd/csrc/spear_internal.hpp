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

// 8 packed nibbles (depth positions 0..7, position i in bits 4i..4i+3) ->
// bf16 pairs holding 128 + u exactly (bf16 has unit spacing on [128, 256)).
// Pair p carries positions (p, p + 4): (0,4) (1,5) (2,6) (3,7).  The zero
// point and the 128 offset are removed in the epilogue: sum x (128 + u) -
// (128 + z) sum x = sum x (u - z).
__device__ __forceinline__ u32x4 unpack8(uint32_t w)
{
    const uint32_t m = 0x000F000Fu, c = 0x43004300u;
    u32x4 r;
    r[0] = (w & m) | c;
    r[1] = ((w >> 4) & m) | c;
    r[2] = ((w >> 8) & m) | c;
    r[3] = ((w >> 12) & m) | c;
    return r;
}

// 8 bf16 in natural order (pairs (0,1) (2,3) (4,5) (6,7)) -> the pair order
// unpack8 produces: (0,4) (1,5) (2,6) (3,7).
__device__ __forceinline__ u32x4 perm8(u32x4 d)
{
    u32x4 o;
    o[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
    o[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
    o[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
    o[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
    return o;
}

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

// sum of the 8 bf16 in d (fp32 accumulate).
__device__ __forceinline__ float sum8(u32x4 d, float acc)
{
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d[0]), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d[1]), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d[2]), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d[3]), one, acc, false);
    return acc;
}

// Agent-scope atomics on workspace counters.
__device__ __forceinline__ uint32_t atomic_add_acqrel(uint32_t *p, uint32_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_load_acquire(uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_release(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_relaxed(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ workspace layout
// Header: 64 uint32 counters, all zero between calls.
enum {
    HDR_TICKET = 0,    // decode: workgroup start order (producer election)
    HDR_PROD_DONE = 1, // decode: producers finished
    HDR_DONE = 2,      // decode: workgroups finished (the last one resets)
    HDR_FLAG = 3,      // decode: EC vector published
    HDR_TIMEOUTS = 4,  // bounded waits that expired (cleared by the host query)
    HDR_WORDS = 64
};

constexpr int DEC_WAVES = 4;    // decode workgroup: 4 waves split the K range
constexpr int DEC_SW = 2;       // 128-deep super-steps per decode wave
constexpr int DEC_SPW = DEC_WAVES * DEC_SW;  // super-steps per decode workgroup
constexpr int PROD_K = 256;     // preferred K slice of one EC producer
constexpr int MAX_PROD = 64;    // at most this many producers (slices grow beyond)

struct WsLayout {
    size_t hdr, colcnt, splitp, produ, prodz, vhi, vlo, active, total;
    int64_t ncg, ksplit, nprod, prod_k, rpad, mpad;
};

WsLayout ws_layout(int64_t M, int64_t N, int64_t K, int32_t r);

// ------------------------------------------------------------- kernel params
struct LinearArgs {
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
    double thr;      // logit(tau) for the hard gate
    float b;
    int32_t hard;
    int32_t r, rpad;
    int64_t M, N, K;
    int64_t ncg, ksplit, nprod, prod_k, mpad;
    WsLayout L;
    uint32_t wait_limit;
    int32_t out_f32;
};

hipError_t launch_pack(const void *codes, int32_t kind, int64_t N, int64_t K, uint8_t *packed,
                       int32_t *bad, hipStream_t s);
hipError_t launch_gate(const uint16_t *x, int64_t M, int64_t K, const uint16_t *wg, float b,
                       double thr, int32_t hard, float *g, int32_t *idx, int32_t *nact,
                       hipStream_t s);
hipError_t launch_compact(const int32_t *flags, int64_t M, int32_t *idx, int32_t *nact,
                          hipStream_t s);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_decode(const LinearArgs &a, int ec_mode, hipStream_t s);
hipError_t launch_prepass(const LinearArgs &a, hipStream_t s);
hipError_t launch_gemm(const LinearArgs &a, int ec_on, hipStream_t s);

} // namespace spear
