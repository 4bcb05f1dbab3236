// pack_gate.hip -- load-time packing of 4-bit codes, the standalone per-token
// gate, token compaction and workspace zeroing (gfx950).
//
// Sources: "SPEAR: A System for Post-Quantization Error-Adaptive Recovery
// Enabling Efficient Low-Bit LLM Serving" -- gist.science summary section 3.1
// (per-channel 4-bit codes from any quantizer) and section 2.1 A plus the
// authors' abstract (an input-dependent gate per token).
#include "spear_internal.hpp"

namespace spear {

// ------------------------------------------------------------------- packing
// One thread: 16 codes (one 16-byte load) -> 8 packed bytes, two words of 8
// codes.  Signed codes are stored offset-binary: the low nibble of q + 8 is
// (q & 15) ^ 8.  Word layout: byte 0 holds codes 0 and 2 (low, high nibble),
// byte 1 codes 4 and 6, byte 2 codes 1 and 3, byte 3 codes 5 and 7.
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ codes,
                                                   int32_t kind, int64_t nchunks,
                                                   uint8_t *__restrict__ packed,
                                                   int32_t *__restrict__ bad)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nchunks)
        return;
    const u32x4 c = ld16(codes + 16 * i);
    uint32_t out[2];
    int nbad = 0;
    uint32_t u[4];
#pragma unroll
    for (int d = 0; d < 4; d++) {
        const uint32_t v = c[d];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t byte = (v >> (8 * j)) & 0xFFu;
            nbad += kind == SPEAR_CODES_S4 ? (((byte + 8u) & 0xFFu) > 15u) : (byte > 15u);
        }
        u[d] = v & 0x0F0F0F0Fu;
        if (kind == SPEAR_CODES_S4)
            u[d] ^= 0x08080808u;
    }
#pragma unroll
    for (int w = 0; w < 2; w++) {
        // a holds codes 0..3 of the word (one per byte), b codes 4..7; a | a >> 12
        // has codes 0 | 2 << 4 in byte 0 and codes 1 | 3 << 4 in byte 1.
        const uint32_t a = u[2 * w], b = u[2 * w + 1];
        const uint32_t ta = a | (a >> 12), tb = b | (b >> 12);
        out[w] = (ta & 0xFFu) | ((tb & 0xFFu) << 8) | (((ta >> 8) & 0xFFu) << 16) |
                 (((tb >> 8) & 0xFFu) << 24);
    }
    uint2 o;
    o.x = out[0];
    o.y = out[1];
    *reinterpret_cast<uint2 *>(packed + 8 * i) = o;
    if (nbad && bad)
        atomicAdd(bad, nbad);
}

hipError_t launch_pack(const void *codes, int32_t kind, int64_t N, int64_t K, uint8_t *packed,
                       int32_t *bad, hipStream_t s)
{
    const int64_t nchunks = N * K / 16;
    const int64_t blocks = (nchunks + 255) / 256;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const uint8_t *)codes, kind, nchunks, packed, bad);
    return hipGetLastError();
}

// ---------------------------------------------------------------------- gate
// One wave per token.  The logit is summed in fp64: each bf16 x bf16 product is
// exact in fp32, so only the fp64 additions round.  flags[m] = 1 if token m
// takes the EC.
__global__ __launch_bounds__(256) void gate_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                   int64_t K, const uint16_t *__restrict__ wg,
                                                   float b, double thr, int32_t hard,
                                                   float *__restrict__ g,
                                                   int32_t *__restrict__ flags)
{
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M)
        return;
    double acc = 0.0;
    for (int64_t k = 8 * lane; k < K; k += 512) {
        const u32x4 xv = ld16(x + m * K + k);
        const u32x4 wv = ld16(wg + k);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            acc += (double)(__uint_as_float(xv[e] << 16) * __uint_as_float(wv[e] << 16));
            acc += (double)(__uint_as_float(xv[e] & 0xFFFF0000u) *
                            __uint_as_float(wv[e] & 0xFFFF0000u));
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        acc += __shfl_xor(acc, off);
    if (lane == 0) {
        const double z = (double)b + acc;
        g[m] = (float)(1.0 / (1.0 + exp(-z)));
        flags[m] = hard ? (z > thr ? 1 : 0) : 1;
    }
}

// Stable compaction of flags[0..M) into ascending indices with wave ballots.
// One workgroup of 1024 threads walks the tokens in chunks of 1024.  flags may
// alias idx: a chunk's flags are all read before any of its indices is written,
// and every write lands below the next chunk.  idx may be NULL (count only).
// A negative flag marks a token whose gate is unknown (an expired wait
// upstream); the count is then -1.  A second destination (idx2, nact2) may
// receive the same list.
__global__ __launch_bounds__(1024) void compact_kernel(const int32_t *flags, int64_t M,
                                                       int32_t *idx, int32_t *nact, int32_t *idx2,
                                                       int32_t *nact2)
{
    __shared__ int wave_tot[16];
    __shared__ int any_bad;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0)
        any_bad = 0;
    __syncthreads();
    int64_t base = 0;
    for (int64_t c0 = 0; c0 < M; c0 += 1024) {
        const int64_t i = c0 + tid;
        const int32_t fv = (i < M) ? flags[i] : 0;
        const int f = fv != 0;
        const uint64_t mask = __ballot(f);
        if (fv < 0)
            any_bad = 1;
        if (lane == 0)
            wave_tot[wave] = __popcll(mask);
        __syncthreads();
        int64_t off = base;
        int total = 0;
        for (int w = 0; w < 16; w++) {
            total += wave_tot[w];
            if (w < wave)
                off += wave_tot[w];
        }
        if (f && idx)
            idx[off + __popcll(mask & ((1ull << lane) - 1ull))] = (int32_t)i;
        if (f && idx2)
            idx2[off + __popcll(mask & ((1ull << lane) - 1ull))] = (int32_t)i;
        base += total;
        __syncthreads();
    }
    if (tid == 0 && nact)
        *nact = any_bad ? -1 : (int32_t)base;
    if (tid == 0 && nact2)
        *nact2 = any_bad ? -1 : (int32_t)base;
}

hipError_t launch_gate(const uint16_t *x, int64_t M, int64_t K, const uint16_t *wg, float b,
                       double thr, int32_t hard, float *g, int32_t *idx, int32_t *nact,
                       hipStream_t s)
{
    if (M > 0) {
        hipLaunchKernelGGL(gate_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, x, M, K,
                           wg, b, thr, hard, g, idx);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return launch_compact(idx, M, idx, nact, s);
}

hipError_t launch_compact(const int32_t *flags, int64_t M, int32_t *idx, int32_t *nact,
                          hipStream_t s, int32_t *idx2, int32_t *nact2)
{
    hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(1024), 0, s, flags, M, idx, nact, idx2, nact2);
    return hipGetLastError();
}

// ------------------------------------------------------------------ zeroing
__global__ __launch_bounds__(256) void zero_kernel(uint8_t *p, size_t bytes)
{
    const size_t n16 = bytes / 16;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        *reinterpret_cast<u32x4 *>(p + 16 * i) = zero4();
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < bytes - 16 * n16)
        p[16 * n16 + t] = 0;
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s)
{
    size_t blocks = (bytes / 16 + 255) / 256;
    if (blocks < 1)
        blocks = 1;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint8_t *)p, bytes);
    return hipGetLastError();
}

// ------------------------------------------------------------ stream read
// Measurement helper: every 16-byte chunk of p is loaded once, four loads a
// thread in flight, and folded by XOR; the fold is stored only if it equals a
// constant, so the loads cannot be removed and (almost surely) nothing is
// written.  Its rate is the plain read floor of a buffer of that size.  The
// grid size comes as an argument: gridDim would load a further line of
// arguments, which costs a launch about 0.35 us.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p, size_t n16,
                                                          uint32_t *sink, uint32_t nblk)
{
    const size_t stride = (size_t)nblk * 256;
    uint32_t acc = 0;
    for (size_t base = (size_t)blockIdx.x * 256 + threadIdx.x; base < n16; base += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const size_t i = base + j * stride;
            v[j] = i < n16 ? p[i] : zero4();
        }
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    if (acc == 0x9E3779B9u)
        *sink = acc;
}

hipError_t launch_stream_read(const void *p, size_t bytes, uint32_t *sink, hipStream_t s)
{
    const size_t n16 = bytes / 16;
    size_t blocks = (n16 + 1023) / 1024;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const u32x4 *>(p), n16, sink, (uint32_t)blocks);
    return hipGetLastError();
}

} // namespace spear
