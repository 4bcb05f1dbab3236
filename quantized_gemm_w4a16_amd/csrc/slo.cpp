// slo.cpp -- host-side, EC-aware choice of the prefill chunk under an
// inter-token-latency (ITL) objective, from a table of measured kernel
// latencies.
//
// Source: "SPEAR: A System for Post-Quantization Error-Adaptive Recovery
// Enabling Efficient Low-Bit LLM Serving", gist.science summary section 2.2 C
// (the scheduler picks the largest prefill chunk whose predicted ITL meets the
// objective, using kernel-latency tables computed ahead of time, and adapts to
// how many layers carry ECs) and section 3.2 (stable ITL objectives with
// dynamic chunking); the authors' abstract names the SLO-aware, EC-aware
// scheduling.  No HIP call is made here.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spear.h"

namespace {

// Latency of one call of kind k at `tokens` tokens: linear between the grid
// points, the running maximum of the measured values (so the prediction never
// falls as the batch grows), and the last segment's slope beyond the grid.
double kind_us(const spear_lut *L, int32_t k, double tokens)
{
    const int32_t n = L->npoints;
    const float *v = L->us + (size_t)k * (size_t)n;
    double prev = v[0];
    if (tokens <= (double)L->tokens[0])
        return prev;                                            // below the grid: its first value
    for (int32_t i = 1; i < n; i++) {
        const double cur = v[i] > prev ? (double)v[i] : prev;      // monotone envelope
        const double t0 = L->tokens[i - 1], t1 = L->tokens[i];
        if (tokens <= t1 || i == n - 1) {
            const double slope = (cur - prev) / (t1 - t0);
            return prev + slope * (tokens - t0);
        }
        prev = cur;
    }
    return prev;
}

spear_status check_lut(const spear_lut *L)
{
    if (!L || !L->tokens || !L->us || !L->count)
        return SPEAR_E_NULL;
    if (L->npoints < 1 || L->nkinds < 1)
        return SPEAR_E_SHAPE;
    if (L->tokens[0] < 1 || isnan(L->overhead_us) || L->overhead_us < 0.f)
        return SPEAR_E_ARG;
    for (int32_t i = 1; i < L->npoints; i++)
        if (L->tokens[i] <= L->tokens[i - 1])
            return SPEAR_E_ARG;
    for (int32_t k = 0; k < L->nkinds; k++) {
        if (L->count[k] < 0)
            return SPEAR_E_ARG;
        for (int32_t i = 0; i < L->npoints; i++) {
            const float u = L->us[(size_t)k * L->npoints + i];
            if (!(u >= 0.f) || isinf(u))
                return SPEAR_E_ARG;
        }
    }
    return SPEAR_OK;
}

double predict(const spear_lut *L, int32_t tokens)
{
    if (tokens <= 0)
        return 0.0;
    double t = L->overhead_us;
    for (int32_t k = 0; k < L->nkinds; k++)
        if (L->count[k] > 0)
            t += (double)L->count[k] * kind_us(L, k, (double)tokens);
    return t;
}

} // namespace

extern "C" {

spear_status spear_slo_predict(const spear_lut *lut, int32_t tokens, float *us_out)
{
    const spear_status st = check_lut(lut);
    if (st != SPEAR_OK)
        return st;
    if (!us_out)
        return SPEAR_E_NULL;
    if (tokens < 0)
        return SPEAR_E_SHAPE;
    *us_out = (float)predict(lut, tokens);
    return SPEAR_OK;
}

spear_status spear_slo_pick_chunk(const spear_lut *lut, int32_t n_decode, int32_t pending,
                                  int32_t align, float slo_us, int32_t *chunk,
                                  float *predicted_us)
{
    const spear_status st = check_lut(lut);
    if (st != SPEAR_OK)
        return st;
    if (!chunk)
        return SPEAR_E_NULL;
    if (n_decode < 0 || pending < 0 || align < 1)
        return SPEAR_E_SHAPE;
    if (isnan(slo_us))
        return SPEAR_E_ARG;
    // Largest c in {pending} U {multiples of align below pending}, c <= pending,
    // with predict(n_decode + c) <= slo_us; the prediction is monotone in c, so
    // a binary search over the multiples finds it.  0 when none fits.
    int32_t best = 0;
    if (pending > 0 && predict(lut, n_decode + pending) <= (double)slo_us) {
        best = pending;
    } else {
        int32_t lo = 0, hi = (pending - 1) / align;   // multiples of align, all < pending
        if (pending == 0)
            hi = 0;
        while (lo < hi) {
            const int32_t mid = lo + (hi - lo + 1) / 2;
            if (predict(lut, n_decode + mid * align) <= (double)slo_us)
                lo = mid;
            else
                hi = mid - 1;
        }
        best = lo * align;
    }
    *chunk = best;
    if (predicted_us)
        *predicted_us = (float)predict(lut, n_decode + best);
    return SPEAR_OK;
}

} // extern "C"
