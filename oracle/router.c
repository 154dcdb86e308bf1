/*
 * Oracle router logits -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * Top-k gating (kwkr.cn explainer on Mixture-of-Kittens, section 4.1
 * "deterministic expert routing and load balancing": tokens are routed by
 * top-k gating over router logits). The pages fix no accumulation order; the
 * routing decision is an integer result, so it is taken here in the precision
 * and order the GPU kernel uses: for every (token t, expert e)
 *
 *   acc = +0.0f;  for h = 0 .. H-1 ascending: acc = fmaf(x[t][h], wr[e][h], acc);
 *   z[t][e] = acc + bias[e]            (one fp32 add; skipped when bias is NULL)
 *
 * Inputs are the bf16/fp32 values widened to float (exact).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

void oracle_router_logits(int64_t T, int32_t H, int32_t E, const float* x, const float* wr, const float* bias,
                          float* z) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const float* xt = x + t * (int64_t)H;
    for (int32_t e = 0; e < E; ++e) {
      const float* we = wr + (int64_t)e * H;
      float acc = 0.0f;
      for (int32_t h = 0; h < H; ++h) acc = fmaf(xt[h], we[h], acc);
      if (bias) acc = acc + bias[e];
      z[t * (int64_t)E + e] = acc;
    }
  }
}
