/*
 * Conv3D oracle — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, direct CPU convolution used to check the GPU library.
 * Only tests/, the smoke entry point and the benchmark's CPU-baseline leg
 * may load it. It shares no code, header or constant with the GPU library.
 *
 * What it computes (one output element at a time):
 *
 *   acc[m, co] = sum_{kd,kh,kw,ci} x[n, d, h, w, ci] * w[co, ci, kd, kh, kw]
 *
 * with d = do*sd + kd - pad_lo_d (likewise h, w) and taps whose input
 * coordinate falls outside the tensor contributing zero. This is PyTorch's
 * cross-correlation convention for F.conv3d, which the Qwen-Image PR page
 * ("T=1 degeneration") and the MiniMax H3 comment on the FlyDSL issue page
 * ("The call site is already a clean drop-in") both use; causal temporal
 * padding is pad_lo_d = 2, pad_hi_d = 0 (Qwen-Image PR page, "T=1
 * degeneration").
 *
 * Precision. The cuDNN page ("Operation Contract") fixes the accumulator to
 * FP32 and rounds to BF16 at named points, but leaves the order of the sum
 * open. The oracle therefore forms the sum in double precision — each
 * bf16*bf16 product is exact in double and the sum of at most a few tens of
 * thousands of them carries an error far below one fp32 ulp — and rounds it
 * once to fp32: the best fp32 accumulator any summation order can approach.
 * The post-operations follow the same contract line by line in fp32
 * (IEEE add, mul, div and sqrt are correctly rounded, so those steps have
 * one right answer); the sum of squares is formed in double and rounded
 * once to fp32, and exp is taken in double and rounded once to fp32.
 *
 * B(x) is fp32 -> bf16 conversion with round-to-nearest, ties to even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BIAS 1
#define ORC_RESIDUAL 2
#define ORC_NORM_SILU 4

/* ---- bf16 helpers (IEEE binary32 -> bfloat16, round to nearest even) ---- */

float oracle_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* B(x): keep the top 16 bits of the binary32 pattern, rounding the 16
 * dropped bits to nearest, ties to even. A carry out of the mantissa
 * correctly bumps the exponent (and the largest finite values round to
 * infinity). NaNs stay NaN (quiet bit forced). */
uint16_t oracle_bf16_round(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t hi = u >> 16;
  uint32_t lo = u & 0xffffu;
  if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

static float B(float f) { return oracle_bf16_to_f32(oracle_bf16_round(f)); }

/* Output extent along one dimension, PyTorch's formula. */
static int out_extent(int in, int k, int s, int plo, int phi) {
  int span = in + plo + phi - k;
  if (span < 0) return 0;
  return span / s + 1;
}

int oracle_output_dims(int D, int H, int W, int KD, int KH, int KW, const int* stride,
                       const int* pad_lo, const int* pad_hi, int* out3) {
  out3[0] = out_extent(D, KD, stride[0], pad_lo[0], pad_hi[0]);
  out3[1] = out_extent(H, KH, stride[1], pad_lo[1], pad_hi[1]);
  out3[2] = out_extent(W, KW, stride[2], pad_lo[2], pad_hi[2]);
  return (out3[0] > 0 && out3[1] > 0 && out3[2] > 0) ? 0 : -1;
}

/*
 * x:        bf16 bits, NDHWC [N][D][H][W][Ci]
 * w:        bf16 bits, OIDHW [Co][Ci][KD][KH][KW] (the checkpoint layout)
 * bias:     fp32 [Co] or NULL          (used when flags & ORC_BIAS)
 * residual: bf16 [M][Co] (NDHWC-flat) or NULL (flags & ORC_RESIDUAL)
 * gamma:    bf16 [Co] or NULL          (flags & ORC_NORM_SILU)
 * pix:      flat output-pixel indices m = ((n*Do+do)*Ho+ho)*Wo+wo to compute,
 *           or NULL for all M pixels in order; npix entries.
 * Outputs are [npix][Co]; every pointer but y may be NULL:
 *   y        bf16 result
 *   acc      fp32 accumulator (before any rounding to bf16)
 *   conv     B(acc); mainv = B(conv + bias); value = B(main + residual)
 *   affine   the contract's `affine` (norm path only)
 *   den      [npix] fp32 denominator (norm path only)
 * Returns 0, or -1 on a shape error.
 */
int oracle_conv3d(const uint16_t* x, const uint16_t* w, int N, int D, int H, int W, int Ci,
                  int Co, int KD, int KH, int KW, const int* stride, const int* pad_lo,
                  const int* pad_hi, const float* bias, const uint16_t* residual,
                  const uint16_t* gamma, int flags, const int64_t* pix, int64_t npix,
                  uint16_t* y, float* acc_out, uint16_t* conv_out, uint16_t* main_out,
                  uint16_t* value_out, uint16_t* affine_out, float* den_out) {
  int od[3];
  if (N <= 0 || Ci <= 0 || Co <= 0 || KD <= 0 || KH <= 0 || KW <= 0) return -1;
  if (stride[0] <= 0 || stride[1] <= 0 || stride[2] <= 0) return -1;
  if (oracle_output_dims(D, H, W, KD, KH, KW, stride, pad_lo, pad_hi, od) != 0) return -1;
  const int Do = od[0], Ho = od[1], Wo = od[2];
  const int64_t M = (int64_t)N * Do * Ho * Wo;
  if (pix == NULL) npix = M;
  const int ntap = KD * KH * KW;

  /* The oracle's own copy of the weight, [tap][ci][co] (bf16 values are
   * exact in fp32), so the innermost loop runs over independent accumulators
   * (one per co) without changing what any element sums. */
  float* wt = (float*)malloc(sizeof(float) * (size_t)ntap * Ci * Co);
  if (!wt) return -2;
  for (int co = 0; co < Co; ++co)
    for (int ci = 0; ci < Ci; ++ci)
      for (int t = 0; t < ntap; ++t)
        wt[((size_t)t * Ci + ci) * Co + co] =
            oracle_bf16_to_f32(w[((size_t)co * Ci + ci) * ntap + t]);

  const float sqrt_c = sqrtf((float)Co);
  int err = 0;

#pragma omp parallel
  {
    double* acc = (double*)malloc(sizeof(double) * Co);
    float* val = (float*)malloc(sizeof(float) * Co);
    if (!acc || !val) {
#pragma omp atomic write
      err = -2;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t i = 0; i < npix; ++i) {
      if (!acc || !val) continue;
      const int64_t m = pix ? pix[i] : i;
      int64_t r = m;
      const int wo = (int)(r % Wo); r /= Wo;
      const int ho = (int)(r % Ho); r /= Ho;
      const int dq = (int)(r % Do); r /= Do;
      const int n = (int)r;
      for (int co = 0; co < Co; ++co) acc[co] = 0.0;

      for (int kd = 0; kd < KD; ++kd) {
        const int d = dq * stride[0] + kd - pad_lo[0];
        if (d < 0 || d >= D) continue; /* zero padding contributes nothing */
        for (int kh = 0; kh < KH; ++kh) {
          const int h = ho * stride[1] + kh - pad_lo[1];
          if (h < 0 || h >= H) continue;
          for (int kw = 0; kw < KW; ++kw) {
            const int ww = wo * stride[2] + kw - pad_lo[2];
            if (ww < 0 || ww >= W) continue;
            const uint16_t* xp = x + ((((int64_t)n * D + d) * H + h) * W + ww) * Ci;
            const float* wp = wt + (size_t)((kd * KH + kh) * KW + kw) * Ci * Co;
            for (int ci = 0; ci < Ci; ++ci) {
              const double xv = (double)oracle_bf16_to_f32(xp[ci]);
              const float* wr = wp + (size_t)ci * Co;
              for (int co = 0; co < Co; ++co) acc[co] += xv * (double)wr[co];
            }
          }
        }
      }

      /* Post-operations, in the order and with the rounding points of the
       * cuDNN page's "Operation Contract". */
      for (int co = 0; co < Co; ++co) {
        const float a32 = (float)acc[co];
        const float conv = B(a32);
        const float mainv = (flags & ORC_BIAS) ? B(conv + bias[co]) : conv;
        float v = mainv;
        if (flags & ORC_RESIDUAL) v = B(mainv + oracle_bf16_to_f32(residual[m * Co + co]));
        val[co] = v;
        if (acc_out) acc_out[i * Co + co] = a32;
        if (conv_out) conv_out[i * Co + co] = oracle_bf16_round(conv);
        if (main_out) main_out[i * Co + co] = oracle_bf16_round(mainv);
        if (value_out) value_out[i * Co + co] = oracle_bf16_round(v);
      }
      if (flags & ORC_NORM_SILU) {
        double ss = 0.0;
        for (int co = 0; co < Co; ++co) ss += (double)val[co] * (double)val[co];
        const float den = fmaxf(sqrtf((float)ss), 1e-12f);
        if (den_out) den_out[i] = den;
        for (int co = 0; co < Co; ++co) {
          const float nrm = B(val[co] / den);
          const float scl = B(nrm * sqrt_c);
          const float aff = B(scl * oracle_bf16_to_f32(gamma[co]));
          const float e = (float)exp(-(double)aff);
          const float act = B(aff / (1.0f + e));
          if (affine_out) affine_out[i * Co + co] = oracle_bf16_round(aff);
          y[i * Co + co] = oracle_bf16_round(act);
        }
      } else {
        for (int co = 0; co < Co; ++co) y[i * Co + co] = oracle_bf16_round(val[co]);
      }
    }
    free(acc);
    free(val);
  }
  free(wt);
  return err;
}
