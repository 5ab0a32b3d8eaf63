/*
 * ORACLE -- test infrastructure, not part of the library.  Only the tests,
 * the smoke check and the benchmark's CPU-baseline leg may load this file's
 * shared object.  It shares no code with the HIP path.
 *
 * Router logits of the Mixture-of-Experts layer in one fixed ("canonical")
 * float32 summation order.
 *
 * "Hosting Qwen on Blackwell" (Perplexity), section "Pre-remplisseurs": each
 * token is routed to 8 of the 128 experts.  The pages do not give the router
 * function or its arithmetic; the score of expert e for token t is read here
 * as the linear projection
 *
 *     l[t,e] = sum_h x[t,h] * W[h,e]   (+ b[e] when a bias is given)
 *
 * evaluated in float32 as one fused multiply-add per term, h ascending,
 * starting from +0.0f, with the bias added once at the end.  A routing
 * decision (which experts win) is an integer result that depends on this
 * order near ties, so the order is part of the definition.
 *
 * Build: gcc -O2 -ffp-contract=off -mfma -fopenmp -shared -fPIC.  The only
 * fused operations are the explicit fmaf() calls.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <omp.h>

void oracle_router_logits(const float* x,      /* [T, H] row-major            */
                          const float* w,      /* [H, E] row-major            */
                          const float* bias,   /* [E] or NULL                 */
                          int64_t T, int64_t H, int64_t E,
                          float* logits)       /* [T, E] row-major, written   */
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        float* l = logits + t * E;
        for (int64_t e = 0; e < E; ++e) l[e] = 0.0f;
        for (int64_t h = 0; h < H; ++h) {
            const float xv = x[t * H + h];
            const float* wrow = w + h * E;
            for (int64_t e = 0; e < E; ++e) l[e] = fmaf(xv, wrow[e], l[e]);
        }
        if (bias != NULL) {
            for (int64_t e = 0; e < E; ++e) l[e] = l[e] + bias[e];
        }
    }
}

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}
