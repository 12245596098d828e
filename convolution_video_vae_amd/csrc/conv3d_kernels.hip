// HIP kernels for the bf16 3x3x3 NDHWC Conv3D on gfx950 (MI355X).
//
// The convolution is an implicit GEMM (FlyDSL issue "conv3d_implicit —
// accept and emit NDHWC ...", maintainer reply): D[co][m] = sum_k W[co][k] *
// X[k][m] with m an output pixel, k = (tap, input channel) and X gathered
// from the NDHWC input on the fly. Causal and spatial zero padding live only
// in the gather's range test (Qwen-Image PR page, "T=1 degeneration"):
// out-of-range taps load zeros through the buffer unit's range check, so no
// padded copy of the input exists anywhere.
//
// Main kernel layout (per work-group of WM x WN waves):
//  * weights: the [BN channels][32] slice of the packed weight for one K
//    step is staged in LDS (double-buffered, one barrier per step) and read
//    by every wave as the MFMA A operand;
//  * activations: each wave gathers its own 16*P pixels straight into VGPRs
//    in the MFMA B-operand layout (16 bytes = 8 channels per lane), one step
//    ahead of the MFMAs;
//  * v_mfma_f32_16x16x32_bf16 accumulates fp32 D[co][pixel] blocks. The
//    weight rows are permuted on their way into LDS so that each lane ends
//    up holding 4*J consecutive output channels of one pixel: the NDHWC
//    store is then a run of 16-byte writes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "conv3d_internal.h"

namespace conv3d {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

static constexpr unsigned kOobOffset = 0x80000000u;  // beyond any x (< 2 GiB)

__device__ __forceinline__ uint16_t f2bf(float f) {
  // fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, (unsigned)b << 16);
}
__device__ __forceinline__ float rbf(float f) { return bf2f(f2bf(f)); }

// Row swizzle of the LDS weight tile (rows of four 16-byte chunks): XOR the
// chunk index with bits of the row so that the 16 rows one MFMA operand read
// touches fall in distinct bank groups.
__device__ __forceinline__ int lds_idx(int row, int chunk) {
  return row * 4 + (chunk ^ (((row >> 1) ^ (row >> 3)) & 3));
}

__device__ __forceinline__ u32x4_t load_x(__amdgpu_buffer_rsrc_t rsrc, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, 0);
}

// --------------------------------------------------------------------------
// Implicit-GEMM main kernel.
// --------------------------------------------------------------------------
template <int WM, int WN, int P, int J, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void igemm_kernel(IgemmArgs a) {
  constexpr int NT = 64 * WM * WN;
  constexpr int BM = 16 * P * WM;
  constexpr int BN = 16 * J * WN;
  constexpr int CHUNKS = BN * 4;                 // 16-byte chunks per weight tile
  constexpr int CPT = (CHUNKS + NT - 1) / NT;    // chunks per thread
  __shared__ u32x4_t wlds[2][CHUNKS];
  __shared__ float red[(EPI == EPI_NORM) ? WM * WN * P * 16 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave % WM;
  const int wave_n = wave / WM;
  const int g = lane >> 4;   // k sub-block (8 channels) / output row group
  const int lr = lane & 15;  // pixel within a 16-pixel block

  // Work-groups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous run of tiles so neighbouring tiles (which share input rows
  // and weight slices) meet in the same L2.
  int bid = blockIdx.x;
  {
    const int G = gridDim.x;
    const int G8 = G & ~7;
    if (bid < G8) bid = (bid & 7) * (G8 >> 3) + (bid >> 3);
  }
  const int m_tile = bid % a.m_tiles;
  const int rest = bid / a.m_tiles;
  const int n_tile = rest % a.n_tiles;
  const int split = rest / a.n_tiles;
  const int m0 = m_tile * BM;
  const int co0 = n_tile * BN;

  // ---- per-lane pixel geometry --------------------------------------------
  const int rowbytes = a.Cin * 2;
  long long base[P];
  unsigned tapmask[P];  // bit t set: tap t of this lane's pixel is in range
  unsigned live = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int m = m0 + (wave_m * P + p) * 16 + lr;
    tapmask[p] = 0;
    base[p] = 0;
    if (m < a.M) {
      int r = m;
      const int wo = r % a.Wo; r /= a.Wo;
      const int ho = r % a.Ho; r /= a.Ho;
      const int dq = r % a.Do;
      const int n = r / a.Do;
      const int d0 = dq * a.sd - a.pd;
      const int h0 = ho * a.sh - a.ph;
      const int w0 = wo * a.sw - a.pw;
      unsigned vd = 0, vh = 0, vw = 0;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        vd |= (unsigned)(d0 + k >= 0 && d0 + k < a.D) << k;
        vh |= (unsigned)(h0 + k >= 0 && h0 + k < a.H) << k;
        vw |= (unsigned)(w0 + k >= 0 && w0 + k < a.W) << k;
      }
      unsigned tm = 0;
#pragma unroll
      for (int t = 0; t < 27; ++t)
        tm |= ((vd >> (t / 9)) & (vh >> ((t / 3) % 3)) & (vw >> (t % 3)) & 1u) << t;
      tapmask[p] = tm;
      base[p] = ((((long long)n * a.D + d0) * a.H + h0) * a.W + w0) * rowbytes + g * 16;
    }
    live |= tapmask[p];
  }
  // Taps that no pixel of this tile can see (e.g. the two leading causal
  // planes at T=1) are skipped for the whole work-group.
  __shared__ unsigned live_sh;
  if (tid == 0) live_sh = 0;
  __syncthreads();
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) live |= __shfl_xor(live, o);
  if (lane == 0) atomicOr(&live_sh, live);
  __syncthreads();
  live = live_sh;

  const __amdgpu_buffer_rsrc_t xr_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)a.x_bytes, 0x00020000);

  // ---- K range of this split ----------------------------------------------
  const int total_steps = 27 * a.CC;
  const int s_begin = split * a.steps_per_split;
  int s_end = s_begin + a.steps_per_split;
  if (s_end > total_steps) s_end = total_steps;

  auto next_live = [&](int s) -> int {
    while (s < s_end && !((live >> (s / a.CC)) & 1u)) ++s;
    return s;
  };

  f32x4_t acc[J][P];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int p = 0; p < P; ++p) acc[j][p] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Weight-tile chunk c -> (channel row, 16-byte chunk q) -> permuted LDS row
  // so MFMA block j of wave wn reads rows [wn*16J + 16j, +16) and each lane
  // ends with channels g*4J + 4j + i.
  auto wrow_of = [&](int c) -> int {
    const int col = c >> 2;                 // channel within the tile
    const int wn = col / (16 * J);
    const int cw = col % (16 * J);
    const int gg = cw / (4 * J);
    const int jj = (cw % (4 * J)) >> 2;
    const int ii = cw & 3;
    return wn * 16 * J + 16 * jj + 4 * gg + ii;
  };

  u32x4_t wreg[CPT];
  auto load_w = [&](int s) {
    const int t = s / a.CC;
    const int cc = s % a.CC;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        a.wp + ((long long)(t * a.CC + cc) * a.Cout + co0) * 32);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      wreg[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (c < CHUNKS && co0 + (c >> 2) < a.Cout) wreg[i] = src[c];
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (c < CHUNKS) wlds[buf][lds_idx(wrow_of(c), c & 3)] = wreg[i];
    }
  };
  auto load_x_step = [&](int s, u32x4_t (&dst)[P]) {
    const int t = s / a.CC;
    const int cc = s % a.CC;
    const int kd = t / 9, kh = (t / 3) % 3, kw = t % 3;
    const long long delta = ((long long)(kd * a.H + kh) * a.W + kw) * rowbytes + cc * 64;
    const bool chan_ok = cc * 32 + g * 8 < a.Cin;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const bool ok = chan_ok && ((tapmask[p] >> t) & 1u);
      const unsigned off = ok ? (unsigned)(base[p] + delta) : kOobOffset;
      dst[p] = load_x(xr_rsrc, off);
    }
  };

  int s = next_live(s_begin);
  if (s < s_end) {
    u32x4_t xcur[P];
    load_w(s);
    load_x_step(s, xcur);
    store_w(0);
    __syncthreads();
    int buf = 0;
    while (s < s_end) {
      const int sn = next_live(s + 1);
      u32x4_t xnext[P];
      if (sn < s_end) {
        load_w(sn);
        load_x_step(sn, xnext);
      }
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const u32x4_t wv = wlds[buf][lds_idx(wave_n * 16 * J + 16 * j + lr, g)];
        const bf16x8_t wa = __builtin_bit_cast(bf16x8_t, wv);
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const bf16x8_t xb = __builtin_bit_cast(bf16x8_t, xcur[p]);
          acc[j][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xb, acc[j][p], 0, 0, 0);
        }
      }
      if (sn < s_end) store_w(buf ^ 1);
      __syncthreads();
#pragma unroll
      for (int p = 0; p < P; ++p) xcur[p] = xnext[p];
      buf ^= 1;
      s = sn;
    }
  }

  // ---- epilogue --------------------------------------------------------------
  // Lane holds, for pixel block p, channels cbase .. cbase + 4J - 1 of pixel m.
  const int cbase = co0 + wave_n * 16 * J + g * 4 * J;
  if (EPI == EPI_PARTIAL) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int m = m0 + (wave_m * P + p) * 16 + lr;
      if (m >= a.M || cbase >= a.Cout) continue;
      f32x4_t* dst = reinterpret_cast<f32x4_t*>(
          a.partial + ((long long)split * a.M + m) * a.Cout + cbase);
#pragma unroll
      for (int j = 0; j < J; ++j) dst[j] = acc[j][p];
    }
    return;
  }

  // value = B(B(B(acc) + bias) + residual), each step only if enabled.
  float val[P][4 * J];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int m = m0 + (wave_m * P + p) * 16 + lr;
    const bool ok = (m < a.M) && (cbase < a.Cout);
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) val[p][4 * j + i] = rbf(acc[j][p][i]);
    if (!ok) continue;
    if (a.flags & F_BIAS) {
#pragma unroll
      for (int c = 0; c < 4 * J; ++c) val[p][c] = rbf(val[p][c] + a.bias[cbase + c]);
    }
    if (a.flags & F_RESIDUAL) {
      const uint16_t* rp = a.residual + (long long)m * a.Cout + cbase;
#pragma unroll
      for (int c = 0; c < 4 * J; c += 8) {
        const u32x4_t rv = *reinterpret_cast<const u32x4_t*>(rp + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t bits = (uint16_t)(rv[e >> 1] >> (16 * (e & 1)));
          val[p][c + e] = rbf(val[p][c + e] + bf2f(bits));
        }
      }
    }
    if (a.flags & F_RESIDUAL_OUT) {
      uint16_t* op = a.residual_out + (long long)m * a.Cout + cbase;
#pragma unroll
      for (int c = 0; c < 4 * J; c += 8) {
        u32x4_t ov;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          ov[q] = (unsigned)f2bf(val[p][c + 2 * q]) | ((unsigned)f2bf(val[p][c + 2 * q + 1]) << 16);
        *reinterpret_cast<u32x4_t*>(op + c) = ov;
      }
    }
  }

  if (EPI == EPI_NORM) {
    // Sum of squares over the pixel's full channel row: this lane's 4J
    // channels, then the four lanes of the same pixel, then the WN waves.
    float ss[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float t = 0.f;
#pragma unroll
      for (int c = 0; c < 4 * J; ++c) t += val[p][c] * val[p][c];
      t += __shfl_xor(t, 16);
      t += __shfl_xor(t, 32);
      ss[p] = t;
    }
    if (WN > 1) {
      if (g == 0) {
#pragma unroll
        for (int p = 0; p < P; ++p) red[((wave_n * WM + wave_m) * P + p) * 16 + lr] = ss[p];
      }
      __syncthreads();
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float t = 0.f;
        for (int wn = 0; wn < WN; ++wn) t += red[((wn * WM + wave_m) * P + p) * 16 + lr];
        ss[p] = t;
      }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float den = fmaxf(sqrtf(ss[p]), 1e-12f);
#pragma unroll
      for (int c = 0; c < 4 * J; ++c) {
        const int co = cbase + c;
        const float nrm = rbf(val[p][c] / den);
        const float scl = rbf(nrm * a.sqrt_c);
        const float gm = (co < a.Cout) ? bf2f(a.gamma[co]) : 0.f;
        const float aff = rbf(scl * gm);
        val[p][c] = rbf(aff / (1.0f + expf(-aff)));
      }
    }
  }

#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int m = m0 + (wave_m * P + p) * 16 + lr;
    if (m >= a.M || cbase >= a.Cout) continue;
    uint16_t* yp = a.y + (long long)m * a.Cout + cbase;
#pragma unroll
    for (int c = 0; c < 4 * J; c += 8) {
      u32x4_t ov;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        ov[q] = (unsigned)f2bf(val[p][c + 2 * q]) | ((unsigned)f2bf(val[p][c + 2 * q + 1]) << 16);
      *reinterpret_cast<u32x4_t*>(yp + c) = ov;
    }
  }
}

// --------------------------------------------------------------------------
// Split-K reduction: partial[s][m][c] summed over s = 0..S-1 in that fixed
// order, then the same epilogue as the main kernel.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void reduce_store_kernel(ReduceArgs a) {
  // One thread per (pixel, 8 channels).
  const long long groups = (long long)a.M * (a.Cout / 8);
  for (long long gi = (long long)blockIdx.x * blockDim.x + threadIdx.x; gi < groups;
       gi += (long long)gridDim.x * blockDim.x) {
    const long long m = gi / (a.Cout / 8);
    const int c0 = (int)(gi % (a.Cout / 8)) * 8;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const f32x4_t* src =
          reinterpret_cast<const f32x4_t*>(a.partial + ((long long)s * a.M + m) * a.Cout + c0);
      const f32x4_t lo = src[0], hi = src[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] += lo[e];
        v[4 + e] += hi[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = rbf(v[e]);
    if (a.flags & F_BIAS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = rbf(v[e] + a.bias[c0 + e]);
    }
    if (a.flags & F_RESIDUAL) {
      const u32x4_t rv = *reinterpret_cast<const u32x4_t*>(a.residual + m * a.Cout + c0);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = rbf(v[e] + bf2f((uint16_t)(rv[e >> 1] >> (16 * (e & 1)))));
    }
    u32x4_t ov;
#pragma unroll
    for (int q = 0; q < 4; ++q) ov[q] = (unsigned)f2bf(v[2 * q]) | ((unsigned)f2bf(v[2 * q + 1]) << 16);
    if (a.flags & F_RESIDUAL_OUT) *reinterpret_cast<u32x4_t*>(a.residual_out + m * a.Cout + c0) = ov;
    *reinterpret_cast<u32x4_t*>(a.y + m * a.Cout + c0) = ov;
  }
}

// Norm variant: one wave per pixel, each lane holding up to 4 groups of 8
// channels (Cout <= 2048).
__global__ __launch_bounds__(256) void reduce_norm_kernel(ReduceArgs a) {
  constexpr int MAXG = 4;
  const int lane = threadIdx.x & 63;
  const int ngroups = a.Cout / 8;
  const long long waves = (long long)gridDim.x * (blockDim.x / 64);
  for (long long m = (long long)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); m < a.M;
       m += waves) {
    float v[MAXG][8];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < MAXG; ++q) {
      const int gidx = lane + 64 * q;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[q][e] = 0.f;
      if (gidx >= ngroups) continue;
      const int c0 = gidx * 8;
      for (int s = 0; s < a.splits; ++s) {
        const f32x4_t* src =
            reinterpret_cast<const f32x4_t*>(a.partial + ((long long)s * a.M + m) * a.Cout + c0);
        const f32x4_t lo = src[0], hi = src[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[q][e] += lo[e];
          v[q][4 + e] += hi[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[q][e] = rbf(v[q][e]);
      if (a.flags & F_BIAS) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[q][e] = rbf(v[q][e] + a.bias[c0 + e]);
      }
      if (a.flags & F_RESIDUAL) {
        const u32x4_t rv = *reinterpret_cast<const u32x4_t*>(a.residual + m * a.Cout + c0);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[q][e] = rbf(v[q][e] + bf2f((uint16_t)(rv[e >> 1] >> (16 * (e & 1)))));
      }
      if (a.flags & F_RESIDUAL_OUT) {
        u32x4_t ov;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          ov[k] = (unsigned)f2bf(v[q][2 * k]) | ((unsigned)f2bf(v[q][2 * k + 1]) << 16);
        *reinterpret_cast<u32x4_t*>(a.residual_out + m * a.Cout + c0) = ov;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[q][e] * v[q][e];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float den = fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
    for (int q = 0; q < MAXG; ++q) {
      const int gidx = lane + 64 * q;
      if (gidx >= ngroups) continue;
      const int c0 = gidx * 8;
      u32x4_t ov;
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float nrm = rbf(v[q][e] / den);
        const float scl = rbf(nrm * a.sqrt_c);
        const float aff = rbf(scl * bf2f(a.gamma[c0 + e]));
        o[e] = rbf(aff / (1.0f + expf(-aff)));
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) ov[k] = (unsigned)f2bf(o[2 * k]) | ((unsigned)f2bf(o[2 * k + 1]) << 16);
      *reinterpret_cast<u32x4_t*>(a.y + m * a.Cout + c0) = ov;
    }
  }
}

// --------------------------------------------------------------------------
// Weight packing: OIDHW [Cout][Cin][27] -> [27][CC][Cout][32], zero beyond Cin.
// One thread per 16-byte output chunk (8 channels).
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint16_t* __restrict__ w,
                                                          uint16_t* __restrict__ wp, int cout,
                                                          int cin, int cc_n) {
  const long long total = 27LL * cc_n * cout * 4;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int q = (int)(i & 3);
    long long r = i >> 2;
    const int co = (int)(r % cout); r /= cout;
    const int cc = (int)(r % cc_n);
    const int t = (int)(r / cc_n);
    u32x4_t out;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      unsigned v2 = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ci = cc * 32 + q * 8 + 2 * k + h;
        const unsigned v = (ci < cin) ? w[((long long)co * cin + ci) * 27 + t] : 0u;
        v2 |= v << (16 * h);
      }
      out[k] = v2;
    }
    reinterpret_cast<u32x4_t*>(wp)[i] = out;
  }
}

// --------------------------------------------------------------------------
// Batched 2D transpose [n][A][B] -> [n][B][A] of 16-bit elements, through a
// 64x64 LDS tile. Reads run along B and writes along A, both coalesced.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src,
                                                        uint16_t* __restrict__ dst, int A, int B,
                                                        int tiles_a, int tiles_b) {
  __shared__ uint16_t tile[64][64 + 2];
  const int tb = blockIdx.x % tiles_b;
  const int ta = (blockIdx.x / tiles_b) % tiles_a;
  const long long n = blockIdx.x / ((long long)tiles_b * tiles_a);
  const int a0 = ta * 64, b0 = tb * 64;
  const uint16_t* s = src + n * (long long)A * B;
  uint16_t* d = dst + n * (long long)A * B;
  const int tx = threadIdx.x & 63;
  const int ty = threadIdx.x >> 6;  // 0..3
  for (int r = ty; r < 64; r += 4) {
    const int ai = a0 + r, bi = b0 + tx;
    if (ai < A && bi < B) tile[r][tx] = s[(long long)ai * B + bi];
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int bi = b0 + r, ai = a0 + tx;
    if (ai < A && bi < B) d[(long long)bi * A + ai] = tile[tx][r];
  }
}

// --------------------------------------------------------------------------
// Launchers.
// --------------------------------------------------------------------------
int launch_pack_weight(const uint16_t* w, uint16_t* wp, int cout, int cin, void* stream) {
  const int cc_n = (cin + 31) / 32;
  const long long total = 27LL * cc_n * cout * 4;
  long long blocks = (total + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, w, wp, cout, cin, cc_n);
  return (int)hipGetLastError();
}

int launch_transpose(const uint16_t* src, uint16_t* dst, int n, int A, int B, void* stream) {
  const int ta = (A + 63) / 64, tb = (B + 63) / 64;
  const long long blocks = (long long)n * ta * tb;
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     src, dst, A, B, ta, tb);
  return (int)hipGetLastError();
}

int launch_reduce(const ReduceArgs& args, void* stream) {
  if (args.flags & F_NORM) {
    long long blocks = ((long long)args.M + 3) / 4;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(reduce_norm_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, args);
  } else {
    const long long groups = (long long)args.M * (args.Cout / 8);
    long long blocks = (groups + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(reduce_store_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, args);
  }
  return (int)hipGetLastError();
}

namespace {
template <int WM, int WN, int P, int J, int EPI>
int launch_one(const IgemmArgs& args, int grid, void* stream) {
  hipLaunchKernelGGL((igemm_kernel<WM, WN, P, J, EPI>), dim3((unsigned)grid), dim3(64 * WM * WN),
                     0, (hipStream_t)stream, args);
  return (int)hipGetLastError();
}

struct Entry {
  int wm, wn, p, j, mode;
  int (*fn)(const IgemmArgs&, int, void*);
};

#define CONV3D_CFG(WM, WN, P, J, MODE) {WM, WN, P, J, MODE, &launch_one<WM, WN, P, J, MODE>}
const Entry kEntries[] = {
    CONV3D_CFG(4, 1, 4, 8, EPI_STORE),
    CONV3D_CFG(4, 1, 4, 6, EPI_STORE),
    CONV3D_CFG(4, 1, 4, 4, EPI_STORE),
    CONV3D_CFG(4, 1, 2, 8, EPI_PARTIAL),
    CONV3D_CFG(4, 1, 2, 6, EPI_PARTIAL),
    CONV3D_CFG(4, 1, 2, 4, EPI_PARTIAL),
    CONV3D_CFG(2, 2, 2, 10, EPI_NORM),
    CONV3D_CFG(2, 2, 2, 5, EPI_NORM),
    CONV3D_CFG(4, 1, 2, 8, EPI_NORM),
};
#undef CONV3D_CFG
}  // namespace

static const Entry* find_entry(const TileCfg& c, int mode) {
  for (const Entry& e : kEntries)
    if (e.wm == c.wm && e.wn == c.wn && e.p == c.p && e.j == c.j && e.mode == mode) return &e;
  return nullptr;
}

bool igemm_has_config(const TileCfg& cfg, int mode) { return find_entry(cfg, mode) != nullptr; }

int launch_igemm(const TileCfg& cfg, int mode, const IgemmArgs& args, int grid, void* stream) {
  const Entry* e = find_entry(cfg, mode);
  if (!e) return -1;
  return e->fn(args, grid, stream);
}

}  // namespace conv3d
