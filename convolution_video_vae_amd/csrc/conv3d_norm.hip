// Channels-last GroupNorm (+ SiLU) over NDHWC bf16 activations.
//
// The MiniMax H3 comment on the FlyDSL issue page "conv3d_implicit — accept
// and emit NDHWC so chained convs skip the layout round-trip" (its GroupNorm
// argument) describes the norm that sits between the encoder's convs: group
// statistics taken per frame once time is folded into the batch (a free view
// in NDHWC), fused with the SiLU that follows, and a group's C/G channels
// contiguous at every pixel. A "unit" below is one frame (n, d) when the
// statistics are time-isolated, else one sample n; its pixels are contiguous,
// P pixels of C channels each.
//
// Three launches, all streaming 16-byte vectors of 8 channels:
//   stats     one work-group per (unit, chunk of pixels): fp32 sums of
//             (x - s_g) and (x - s_g)^2 per thread and channel, where the
//             shift s_g is the group's first value in the unit (keeps the
//             variance free of cancellation when |mean| >> std); combined per
//             group in fp64, in a fixed order, into one partial per chunk.
//   finalize  one work-group per unit: the chunk partials in a fixed order
//             (fp64) -> mean and 1/sqrt(var + eps) per group (population
//             variance, as GroupNorm defines it).
//   apply     y = B((x - mean) * (rstd * gamma_c) + beta_c), then with SiLU
//             y = B(a * sigmoid(a)) of that rounded a; work-groups run from
//             the last chunk back, so the data the stats pass read most
//             recently (still in the memory-side cache) is read first.
// Thread t < ppi * V (V = C / 8 channel vectors per pixel, ppi = 256 / V
// pixels per pass) always holds channel vector t % V, so its 8 channels'
// shifts, means and scales stay in registers.
#include <hip/hip_runtime.h>

#include "conv3d_device.h"
#include "conv3d_internal.h"

namespace conv3d {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;        // 16-byte loads in flight per thread

struct Lanes {
  int cv, pl;
  bool active;
};

__device__ __forceinline__ Lanes lanes_of(const GroupNormArgs& a) {
  const int t = threadIdx.x;
  Lanes l;
  l.active = t < a.ppi * a.V;
  l.cv = l.active ? t % a.V : 0;
  l.pl = l.active ? t / a.V : 0;
  return l;
}

__device__ __forceinline__ void unpack8(const u32x4_t& v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, v[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, v[i] & 0xffff0000u);
  }
}

// a * sigmoid(a) with t = e^-|a| <= 1, so nothing overflows: sigmoid(a) is
// 1 / (1 + t) for a >= 0 and t / (1 + t) below.
__device__ __forceinline__ float silu(float v) {
  const float t = __builtin_amdgcn_exp2f(-fabsf(v) * 1.44269504088896341f);
  const float r = __builtin_amdgcn_rcpf(1.0f + t);
  return v * (v >= 0.0f ? r : t * r);
}

// One lane's share of a chunk: passes 0 .. n-1 at byte offsets 0, stride,
// 2 * stride, ... from `src` (32-bit offsets: a chunk is below 2^31 bytes).
// Blocks of kUnroll passes, the next block's 16-byte loads issued before the
// current block is consumed; body(v, i) sees pass i. init() runs once the
// first block's loads are in flight (its own loads then overlap them).
struct LaneStream {
  const char* src;
  unsigned stride;
  int n;
};

__device__ __forceinline__ u32x4_t load16(const char* p, unsigned off) {
  return *(const u32x4_t*)(p + off);
}

template <typename Init, typename Body>
__device__ __forceinline__ void stream_lane(const LaneStream& ls, Init init, Body body) {
  u32x4_t cur[kUnroll], nxt[kUnroll];
  int i = 0;
  if (kUnroll <= ls.n) {
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) cur[k] = load16(ls.src, (unsigned)k * ls.stride);
    init();
    for (;;) {
      const int in = i + kUnroll;
      const bool more = in + kUnroll <= ls.n;
      if (more) {
#pragma unroll
        for (int k = 0; k < kUnroll; ++k)
          nxt[k] = load16(ls.src, (unsigned)(in + k) * ls.stride);
      }
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) body(cur[k], i + k);
      i = in;
      if (!more) break;
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) cur[k] = nxt[k];
    }
  }
  // ragged tail: fewer than kUnroll passes left
#pragma unroll
  for (int k = 0; k < kUnroll; ++k)
    if (i + k < ls.n) cur[k] = load16(ls.src, (unsigned)(i + k) * ls.stride);
  if (i == 0) init();
#pragma unroll
  for (int k = 0; k < kUnroll; ++k)
    if (i + k < ls.n) body(cur[k], i + k);
}

// The lane's share of pixels [k * chunk_px, ...) of unit u: first pixel
// p0 + pl, then every ppi-th pixel.
__device__ __forceinline__ LaneStream lane_stream(const GroupNormArgs& a, const Lanes& l,
                                                  const uint16_t* t, int u, int k) {
  const long long p0 = (long long)k * a.chunk_px;
  const long long p1 = min(a.P, p0 + a.chunk_px);
  const long long first = p0 + l.pl;
  LaneStream ls;
  ls.src = (const char*)(t + ((size_t)u * a.P + first) * a.C) + (size_t)l.cv * 16;
  ls.stride = (unsigned)a.ppi * (unsigned)a.C * 2u;
  const int span = (int)(p1 - first);   // a chunk holds at most 2^20 pixels
  ls.n = span > 0 ? (span + a.ppi - 1) / a.ppi : 0;
  return ls;
}

__global__ __launch_bounds__(kThreads) void gn_stats_kernel(GroupNormArgs a) {
  __shared__ float s1[2048], s2[2048];   // [pixel lane][channel], ppi * C <= 2048
  const int u = blockIdx.x / a.chunks;
  const int k = blockIdx.x - u * a.chunks;
  const Lanes l = lanes_of(a);
  const uint16_t* base = a.x + (size_t)u * a.P * a.C;
  if (l.active) {
    float acc1[8], acc2[8], sh[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc1[j] = 0.0f;
      acc2[j] = 0.0f;
    }
    const auto load_shifts = [&]() {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = l.cv * 8 + j;
        sh[j] = bf2f(base[(c / a.cpg) * a.cpg]);
      }
    };
    stream_lane(lane_stream(a, l, a.x, u, k), load_shifts, [&](const u32x4_t& v, int) {
      float f[8];
      unpack8(v, f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = f[j] - sh[j];
        acc1[j] += d;
        acc2[j] = fmaf(d, d, acc2[j]);
      }
    });
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s1[l.pl * a.C + l.cv * 8 + j] = acc1[j];
      s2[l.pl * a.C + l.cv * 8 + j] = acc2[j];
    }
  }
  __syncthreads();
  // per channel over the pixel lanes (fp32, lane order), into row 0
  for (int c = threadIdx.x; c < a.C; c += kThreads) {
    float t1 = s1[c], t2 = s2[c];
    for (int pl = 1; pl < a.ppi; ++pl) {
      t1 += s1[pl * a.C + c];
      t2 += s2[pl * a.C + c];
    }
    s1[c] = t1;
    s2[c] = t2;
  }
  __syncthreads();
  // per group over its channels (fp64, channel order)
  for (int g = threadIdx.x; g < a.G; g += kThreads) {
    double S1 = 0.0, S2 = 0.0;
    for (int c = g * a.cpg; c < (g + 1) * a.cpg; ++c) {
      S1 += (double)s1[c];
      S2 += (double)s2[c];
    }
    double* out = a.partial + ((size_t)blockIdx.x * a.G + g) * 2;
    out[0] = S1;
    out[1] = S2;
  }
}

// One work-group per unit: lane k0 of group g sums chunks k0, k0 + L, ...
// (four loads in flight); the L lane sums are then added in lane order.
__global__ __launch_bounds__(kThreads) void gn_finalize_kernel(GroupNormArgs a) {
  __shared__ double r1[kThreads], r2[kThreads];
  const int u = blockIdx.x;
  const int L = kThreads / a.G;
  const int t = threadIdx.x;
  const int g = t % a.G, k0 = t / a.G;
  double S1 = 0.0, S2 = 0.0;
  if (k0 < L) {
    const double* part = a.partial + ((size_t)u * a.chunks * a.G + g) * 2;
    const size_t stride = (size_t)L * a.G * 2;
    int k = k0;
    for (; k + 3 * L < a.chunks; k += 4 * L) {
      const double* q = part + (size_t)k * a.G * 2;
      const double a0 = q[0], b0 = q[1];
      const double a1 = q[stride], b1 = q[stride + 1];
      const double a2 = q[2 * stride], b2 = q[2 * stride + 1];
      const double a3 = q[3 * stride], b3 = q[3 * stride + 1];
      S1 += a0; S1 += a1; S1 += a2; S1 += a3;
      S2 += b0; S2 += b1; S2 += b2; S2 += b3;
    }
    for (; k < a.chunks; k += L) {
      S1 += part[(size_t)k * a.G * 2];
      S2 += part[(size_t)k * a.G * 2 + 1];
    }
  }
  r1[t] = S1;
  r2[t] = S2;
  __syncthreads();
  if (t < a.G) {
    double T1 = 0.0, T2 = 0.0;
    for (int i = 0; i < L; ++i) {
      T1 += r1[i * a.G + t];
      T2 += r2[i * a.G + t];
    }
    const double n = (double)a.P * a.cpg;
    const double m = T1 / n;
    const double var = fmax(T2 / n - m * m, 0.0);
    const float shift = bf2f(a.x[(size_t)u * a.P * a.C + (size_t)t * a.cpg]);
    a.stats[((size_t)u * a.G + t) * 2] = (float)((double)shift + m);
    a.stats[((size_t)u * a.G + t) * 2 + 1] = (float)(1.0 / sqrt(var + (double)a.eps));
  }
}

// Finalize from a conv's per-tile partial sums. One work-group per unit.
// For each frame f of the unit, the tiles whose stored slots meet the frame
// are taken in chunks: the threads first copy the chunk's 64-float rows
// (tile t's frame slot f - f0(t), f0 the frame of its first slot, for every
// channel tile) into LDS with independent 16-byte loads; then thread
// (lane l, group g) adds, in fp64, the cpg / 4 subgroups of its group from
// the rows of chunk tiles l, l + L, ... The L lane sums of a group are
// finally added in lane order.
__global__ __launch_bounds__(kThreads) void gn_finalize_tiles_kernel(GroupNormArgs a, GnTileArgs t) {
  constexpr int kRows = 128;
  __shared__ double r1[kThreads], r2[kThreads];
  __shared__ f32x4_t rows[kRows][16];
  const int u = blockIdx.x;
  const int L = kThreads / a.G;
  const int tid = threadIdx.x;
  const int g = tid % a.G, l = tid / a.G;
  double S1 = 0.0, S2 = 0.0;
  const int c0 = g * a.cpg, nt = c0 / 128, sg0 = (c0 % 128) / 4, nsg = a.cpg / 4;
  const int nct = t.n_ctiles, per_chunk = kRows / nct;
  const long long FS = (long long)t.Ho * t.WP;   // slots per frame
  for (int k = 0; k < t.frames_per_unit; ++k) {
    const long long f = (long long)u * t.frames_per_unit + k;
    const long long fs0 = f * FS;                 // the frame's first slot
    const long long t_lo = fs0 / t.TS, t_hi = (fs0 + FS - 1) / t.TS;
    const int nt_f = (int)(t_hi - t_lo + 1);
    for (int ch = 0; ch < nt_f; ch += per_chunk) {
      const int cn = min(per_chunk, nt_f - ch);
      for (int idx = tid; idx < cn * nct * 16; idx += kThreads) {
        const int row = idx >> 4, i = row / nct, ct = row - i * nct;
        const long long m = t_lo + ch + i;
        // tile m starts in frame f - 1 when its first slot precedes fs0
        const int fslot = m * t.TS < fs0 ? 1 : 0;
        rows[row][idx & 15] = reinterpret_cast<const f32x4_t*>(
            t.part + ((m * nct + ct) * 2 + fslot) * 64)[idx & 15];
      }
      __syncthreads();
      if (l < L) {
        for (int i = l; i < cn; i += L) {
          const float* q = reinterpret_cast<const float*>(rows[i * nct + nt]) + sg0 * 2;
          for (int j = 0; j < nsg; ++j) {
            S1 += (double)q[2 * j];
            S2 += (double)q[2 * j + 1];
          }
        }
      }
      __syncthreads();
    }
  }
  r1[tid] = S1;
  r2[tid] = S2;
  __syncthreads();
  if (tid < a.G) {
    double T1 = 0.0, T2 = 0.0;
    for (int i = 0; i < L; ++i) {
      T1 += r1[i * a.G + tid];
      T2 += r2[i * a.G + tid];
    }
    const double n = (double)a.P * a.cpg;
    const double m = T1 / n;
    const double var = fmax(T2 / n - m * m, 0.0);
    a.stats[((size_t)u * a.G + tid) * 2] = (float)m;
    a.stats[((size_t)u * a.G + tid) * 2 + 1] = (float)(1.0 / sqrt(var + (double)a.eps));
  }
}

template <bool SILU>
__global__ __launch_bounds__(kThreads) void gn_apply_kernel(GroupNormArgs a) {
  const int item = gridDim.x - 1 - blockIdx.x;
  const int u = item / a.chunks;
  const int k = item - u * a.chunks;
  const Lanes l = lanes_of(a);
  if (!l.active) return;
  float mean[8], scale[8], beta[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = l.cv * 8 + j;
    const float* st = a.stats + ((size_t)u * a.G + c / a.cpg) * 2;
    mean[j] = st[0];
    scale[j] = st[1] * a.gamma[c];
    beta[j] = a.beta[c];
  }
  const LaneStream ls = lane_stream(a, l, a.x, u, k);
  char* dst = (char*)a.y + (ls.src - (const char*)a.x);
  stream_lane(ls, [] {}, [&](const u32x4_t& v, int i) {
    float f[8];
    unpack8(v, f);
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = fmaf(f[2 * e] - mean[2 * e], scale[2 * e], beta[2 * e]);
      const float hi = fmaf(f[2 * e + 1] - mean[2 * e + 1], scale[2 * e + 1], beta[2 * e + 1]);
      unsigned w = pack2(lo, hi);
      if (SILU)
        w = pack2(silu(__builtin_bit_cast(float, w << 16)),
                  silu(__builtin_bit_cast(float, w & 0xffff0000u)));
      o[e] = w;
    }
    *(u32x4_t*)(dst + (unsigned)i * ls.stride) = o;
  });
}

}  // namespace

int launch_group_norm_tiles(const GroupNormArgs& args, const GnTileArgs& t, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(gn_finalize_tiles_kernel, dim3(args.units), dim3(kThreads), 0, s, args, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  const unsigned items = (unsigned)args.units * (unsigned)args.chunks;
  if (args.silu)
    hipLaunchKernelGGL(gn_apply_kernel<true>, dim3(items), dim3(kThreads), 0, s, args);
  else
    hipLaunchKernelGGL(gn_apply_kernel<false>, dim3(items), dim3(kThreads), 0, s, args);
  e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}

int launch_group_norm(const GroupNormArgs& args, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const unsigned items = (unsigned)args.units * (unsigned)args.chunks;
  hipLaunchKernelGGL(gn_stats_kernel, dim3(items), dim3(kThreads), 0, s, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(gn_finalize_kernel, dim3(args.units), dim3(kThreads), 0, s, args);
  e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  if (args.silu)
    hipLaunchKernelGGL(gn_apply_kernel<true>, dim3(items), dim3(kThreads), 0, s, args);
  else
    hipLaunchKernelGGL(gn_apply_kernel<false>, dim3(items), dim3(kThreads), 0, s, args);
  e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}

}  // namespace conv3d
