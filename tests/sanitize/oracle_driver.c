/* Runs the C oracle on small shapes (every post-operation flag, pixel
 * lists, strides, causal / valid / asymmetric padding, one-pixel extents)
 * under AddressSanitizer and UndefinedBehaviorSanitizer, with every output
 * array sized exactly, so an out-of-range read or write is reported.
 * Prints "oracle driver ok" and exits 0 when every call succeeds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_conv3d(const uint16_t* x, const uint16_t* w, int N, int D, int H, int W, int Ci,
                  int Co, int KD, int KH, int KW, const int* stride, const int* pad_lo,
                  const int* pad_hi, const float* bias, const uint16_t* residual,
                  const uint16_t* gamma, int flags, const int64_t* pix, int64_t npix,
                  uint16_t* y, float* acc_out, uint16_t* conv_out, uint16_t* main_out,
                  uint16_t* value_out, uint16_t* affine_out, float* den_out);
int oracle_output_dims(int D, int H, int W, int KD, int KH, int KW, const int* stride,
                       const int* pad_lo, const int* pad_hi, int* out3);

static uint32_t lcg = 12345u;
static uint16_t rnd_bf16(void) {
  lcg = lcg * 1664525u + 1013904223u;
  /* small finite values: exponent 120..130, any sign and mantissa */
  return (uint16_t)(((lcg >> 16) & 0x807fu) | ((120u + (lcg >> 28) % 11u) << 7));
}

static void* xalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

int main(void) {
  struct {
    int N, D, H, W, Ci, Co, K, s[3], lo[3], hi[3];
  } cases[] = {
      {1, 5, 7, 9, 8, 16, 3, {1, 1, 1}, {2, 1, 1}, {0, 1, 1}},
      {2, 3, 5, 6, 16, 8, 3, {1, 2, 2}, {2, 0, 0}, {0, 1, 1}},
      {1, 4, 4, 4, 8, 8, 3, {2, 2, 2}, {0, 0, 0}, {0, 0, 0}},
      {1, 1, 1, 1, 8, 16, 3, {1, 1, 1}, {2, 1, 1}, {0, 1, 1}},
      {1, 3, 6, 5, 24, 32, 1, {1, 1, 1}, {0, 0, 0}, {0, 0, 0}},
      {1, 2, 3, 7, 8, 24, 3, {1, 1, 1}, {2, 1, 0}, {0, 1, 2}},
  };
  int fail = 0;
  for (size_t c = 0; c < sizeof cases / sizeof cases[0]; ++c) {
    const int N = cases[c].N, D = cases[c].D, H = cases[c].H, W = cases[c].W;
    const int Ci = cases[c].Ci, Co = cases[c].Co, K = cases[c].K;
    int od[3];
    if (oracle_output_dims(D, H, W, K, K, K, cases[c].s, cases[c].lo, cases[c].hi, od) != 0) {
      ++fail;
      continue;
    }
    const int64_t M = (int64_t)N * od[0] * od[1] * od[2];
    const size_t nx = (size_t)N * D * H * W * Ci, nw = (size_t)Co * Ci * K * K * K;
    uint16_t* x = xalloc(nx * 2);
    uint16_t* w = xalloc(nw * 2);
    uint16_t* res = xalloc((size_t)M * Co * 2);
    uint16_t* gam = xalloc((size_t)Co * 2);
    float* bias = xalloc((size_t)Co * 4);
    for (size_t i = 0; i < nx; ++i) x[i] = rnd_bf16();
    for (size_t i = 0; i < nw; ++i) w[i] = rnd_bf16();
    for (int64_t i = 0; i < M * Co; ++i) res[i] = rnd_bf16();
    for (int i = 0; i < Co; ++i) {
      gam[i] = 0x3f80;
      bias[i] = 0.25f * (float)(i % 5) - 0.5f;
    }
    for (int flags = 0; flags < 8; ++flags) {
      for (int use_pix = 0; use_pix < 2; ++use_pix) {
        const int64_t npix = use_pix ? (M + 1) / 2 : M;
        int64_t* pix = NULL;
        if (use_pix) {
          pix = xalloc((size_t)npix * 8);
          for (int64_t i = 0; i < npix; ++i) pix[i] = (M - 1 - 2 * i) >= 0 ? M - 1 - 2 * i : 0;
        }
        uint16_t* y = xalloc((size_t)npix * Co * 2);
        float* acc = xalloc((size_t)npix * Co * 4);
        uint16_t* cv = xalloc((size_t)npix * Co * 2);
        uint16_t* mn = xalloc((size_t)npix * Co * 2);
        uint16_t* vl = xalloc((size_t)npix * Co * 2);
        uint16_t* af = xalloc((size_t)npix * Co * 2);
        float* den = xalloc((size_t)npix * 4);
        const int rc = oracle_conv3d(x, w, N, D, H, W, Ci, Co, K, K, K, cases[c].s, cases[c].lo,
                                     cases[c].hi, bias, res, gam, flags, pix, pix ? npix : 0, y,
                                     acc, cv, mn, vl, af, den);
        if (rc != 0) {
          fprintf(stderr, "case %zu flags %d: rc %d\n", c, flags, rc);
          ++fail;
        }
        free(y); free(acc); free(cv); free(mn); free(vl); free(af); free(den); free(pix);
      }
    }
    free(x); free(w); free(res); free(gam); free(bias);
  }
  if (fail) {
    fprintf(stderr, "%d oracle call(s) failed\n", fail);
    return 1;
  }
  printf("oracle driver ok\n");
  return 0;
}
