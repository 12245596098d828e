// HIP kernels of the Conv3D library other than the implicit-GEMM main loop
// (conv3d_igemm.hip): the fixed-order split-K reduction with the epilogue,
// weight packing and the NCDHW <-> NDHWC boundary transpose.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "conv3d_device.h"
#include "conv3d_internal.h"

namespace conv3d {

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

// Fragment-order variant (partials of the halo kernel): one thread per 8
// consecutive channels of one pixel, at the position a lane's accumulator
// block holds them; summed over s = 0..S-1 in that fixed order.
__global__ __launch_bounds__(256) void reduce_frag_kernel(ReduceArgs a) {
  const int PB = a.pb, CB = a.cb, WM = a.wm, WN = 4 / WM;
  const int BM = 32 * PB * WM, BN = 32 * CB * WN;
  const long long tiles = (long long)a.m_tiles * a.n_tiles;
  const long long blocks_per_split = tiles * 4 * PB * CB;  // 16-float blocks of 64 lanes
  const long long tasks = blocks_per_split * 2 * 64;
  const f32x4_t* part = reinterpret_cast<const f32x4_t*>(a.partial);
  for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < tasks;
       t += (long long)gridDim.x * blockDim.x) {
    const int L = (int)(t & 63);
    long long r = t >> 6;
    const int qq = (int)(r & 1);
    r >>= 1;
    const long long blk = r;  // ((tile * 4 + w) * PB + p) * CB + cb
    const int cb = (int)(r % CB);
    r /= CB;
    const int p = (int)(r % PB);
    r /= PB;
    const int w = (int)(r & 3);
    const long long tile = r >> 2;
    const int mt = (int)(tile / a.n_tiles), nt = (int)(tile % a.n_tiles);
    const long long m = (long long)mt * BM + (w % WM) * PB * 32 + p * 32 + (L & 31);
    if (m >= a.M) continue;
    const int c0 = nt * BN + (w / WM) * 32 * CB + (L >> 5) * 16 * CB + 16 * cb + 8 * qq;
    // Partial tiles of this output tile, summed in slice order s = 0, 1, ...:
    // slot (s * m_tiles + mt) * n_tiles + nt of a uniform split, or slot
    // nt * per_n + split_base[mt] + s of a live-balanced one.
    const long long blk_in = blk - tile * (4LL * PB * CB);
    const long long bps = 4LL * PB * CB;
    long long slot0, sstep;
    int count;
    if (a.vsplit) {
      slot0 = (long long)nt * a.per_n + a.split_base[mt];
      sstep = 1;
      count = a.split_base[mt + 1] - a.split_base[mt];
    } else {
      slot0 = (long long)mt * a.n_tiles + nt;
      sstep = (long long)a.m_tiles * a.n_tiles;
      count = a.splits;
    }
    const f32x4_t* src0 = part + ((slot0 * bps + blk_in) * 4 + 2 * qq) * 64 + L;
    const long long step = sstep * bps * 4 * 64;   // f32x4 elements between slices
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    int s = 0;
    for (; s + 4 <= count; s += 4) {   // four slices' loads in flight, then the adds in order
      f32x4_t lo[4], hi[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        lo[u] = src0[(s + u) * step];
        hi[u] = src0[(s + u) * step + 64];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] += lo[u][e];
          v[4 + e] += hi[u][e];
        }
    }
    for (; s < count; ++s) {
      const f32x4_t lo = src0[s * step], hi = src0[s * step + 64];
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
    const float rden = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
    for (int q = 0; q < MAXG; ++q) {
      const int gidx = lane + 64 * q;
      if (gidx >= ngroups) continue;
      const int c0 = gidx * 8;
      u32x4_t ov;
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = norm_silu_value(v[q][e], rden, a.sqrt_c, bf2f(a.gamma[c0 + e]));
#pragma unroll
      for (int k = 0; k < 4; ++k) ov[k] = (unsigned)f2bf(o[2 * k]) | ((unsigned)f2bf(o[2 * k + 1]) << 16);
      *reinterpret_cast<u32x4_t*>(a.y + m * a.Cout + c0) = ov;
    }
  }
}

// --------------------------------------------------------------------------
// Padded outputs: the unpadded output y0 [N][Do][Ho][Wo][Cout] placed into
// y [N][Dy][Hy][Wy][Cout] at offset (pt, ph, pw), zeros everywhere else
// except the interiors of the history planes (the caller's), and the last
// cache_k frames also into the cache tail. One work-group per row (n, t, h)
// of y: an output row is one contiguous copy plus its two border runs.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void place_kernel(PlaceArgs a) {
  const long long rows = (long long)a.n * a.Dy * a.Hy;
  const int V = a.cout / 8;
  const u32x4_t z = {0u, 0u, 0u, 0u};
  if (blockIdx.x >= rows) {
    // the cache's older frames, from previous: row (n, f, h), f < cache_frames - cache_k
    const int old = a.cache_frames - a.cache_k;
    const long long r = blockIdx.x - rows;
    const int h = (int)(r % a.Ho);
    const int f = (int)((r / a.Ho) % old);
    const long long n = r / ((long long)a.Ho * old);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        a.previous + ((n * a.hist + (a.hist - old) + f) * a.Ho + h) * a.Wo * a.cout);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(
        a.cache + ((n * a.cache_frames + f) * a.Ho + h) * a.Wo * a.cout);
    for (int i = threadIdx.x; i < a.Wo * V; i += blockDim.x) dst[i] = src[i];
    return;
  }
  const long long row = blockIdx.x;
  const int hh = (int)(row % a.Hy);
  const long long nt = row / a.Hy;
  const int t = (int)(nt % a.Dy);
  const long long n = nt / a.Dy;
  u32x4_t* yr = reinterpret_cast<u32x4_t*>(a.y + row * a.Wy * a.cout);
  const int d = t - a.pt, h = hh - a.ph;
  const bool rowin = h >= 0 && h < a.Ho;
  if (d >= 0 && d < a.Do && rowin) {
    // The interior: copied from y0, or (y0 null) already written in place by
    // the conv, which the cache then copies from.
    u32x4_t* cr = nullptr;
    if (a.cache && d >= a.Do - a.cache_k)
      cr = reinterpret_cast<u32x4_t*>(
          a.cache + ((n * a.cache_frames + (a.cache_frames - a.Do) + d) * a.Ho + h) * a.Wo * a.cout);
    if (a.y0 || cr) {
      const u32x4_t* src =
          a.y0 ? reinterpret_cast<const u32x4_t*>(a.y0 + ((n * a.Do + d) * a.Ho + h) * a.Wo * a.cout)
               : yr + a.pw * V;
      const int inner = a.Wo * V;
      for (int i = threadIdx.x; i < inner; i += blockDim.x) {
        const u32x4_t v = src[i];
        if (a.y0) yr[a.pw * V + i] = v;
        if (cr) cr[i] = v;
      }
    }
  } else if (d < -a.hist || d >= a.Do || !rowin) {
    // a zero plane (before the history, or after the output) or a border row
    for (int i = threadIdx.x; i < a.Wy * V; i += blockDim.x) yr[i] = z;
    return;
  } else if (a.previous) {
    // a history row: copy the caller's previous frame into its interior
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        a.previous + ((n * a.hist + (d + a.hist)) * a.Ho + h) * a.Wo * a.cout);
    for (int i = threadIdx.x; i < a.Wo * V; i += blockDim.x) yr[a.pw * V + i] = src[i];
  }
  // left and right border columns of an output or history row
  const int lead = a.pw * V, tail = (a.Wy - a.pw - a.Wo) * V;
  for (int i = threadIdx.x; i < lead + tail; i += blockDim.x)
    yr[i < lead ? i : (a.pw + a.Wo) * V + (i - lead)] = z;
}

int launch_place(const PlaceArgs& a, void* stream) {
  long long rows = (long long)a.n * a.Dy * a.Hy;
  if (a.previous && a.cache) rows += (long long)a.n * (a.cache_frames - a.cache_k) * a.Ho;
  if (rows == 0) return 0;
  hipLaunchKernelGGL(place_kernel, dim3((unsigned)rows), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

// --------------------------------------------------------------------------
// Standalone post-operations: one wave per pixel, each lane up to 4 groups
// of 8 channels (C <= 2048), the same arithmetic as the fused epilogue with
// conv = x.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void norm_silu_kernel(NormSiluArgs a) {
  constexpr int MAXG = 4;
  const int lane = threadIdx.x & 63;
  const int ngroups = a.C / 8;
  const long long waves = (long long)gridDim.x * (blockDim.x / 64);
  const PlaceArgs& g = a.geo;
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
      const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(a.x + m * a.C + c0);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[q][e] = lane_bf(xv, e);
      if (a.flags & F_BIAS) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[q][e] = rbf(v[q][e] + a.bias[c0 + e]);
      }
      if (a.flags & F_RESIDUAL) {
        const u32x4_t rv = *reinterpret_cast<const u32x4_t*>(a.residual + m * a.C + c0);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[q][e] = rbf(v[q][e] + lane_bf(rv, e));
      }
      if (a.flags & F_RESIDUAL_OUT) {
        const u32x4_t ov = {pack2(v[q][0], v[q][1]), pack2(v[q][2], v[q][3]),
                            pack2(v[q][4], v[q][5]), pack2(v[q][6], v[q][7])};
        *reinterpret_cast<u32x4_t*>(a.residual_out + m * a.C + c0) = ov;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[q][e] * v[q][e];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float rden = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
    // where the pixel goes: y (padded when geo.Dy > 0) and maybe the cache
    long long yp = m, cp = -1;
    if (g.Dy > 0) {
      const int w = (int)(m % g.Wo);
      const long long r = m / g.Wo;
      const int h = (int)(r % g.Ho);
      const long long nd = r / g.Ho;
      const int d = (int)(nd % g.Do);
      const long long n = nd / g.Do;
      yp = ((n * g.Dy + d + g.pt) * g.Hy + h + g.ph) * g.Wy + w + g.pw;
      if (g.cache && d >= g.Do - g.cache_k)
        cp = ((n * g.cache_frames + (g.cache_frames - g.Do) + d) * g.Ho + h) * g.Wo + w;
    }
#pragma unroll
    for (int q = 0; q < MAXG; ++q) {
      const int gidx = lane + 64 * q;
      if (gidx >= ngroups) continue;
      const int c0 = gidx * 8;
      const u32x4_t gv = *reinterpret_cast<const u32x4_t*>(a.gamma + c0);
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = norm_silu_value(v[q][e], rden, a.sqrt_c, lane_bf(gv, e));
      const u32x4_t ov = {pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7])};
      *reinterpret_cast<u32x4_t*>(a.y + yp * a.C + c0) = ov;
      if (cp >= 0) *reinterpret_cast<u32x4_t*>(g.cache + cp * a.C + c0) = ov;
    }
  }
}

int launch_norm_silu(const NormSiluArgs& a, void* stream) {
  const long long blocks = std::min<long long>((a.M + 3) / 4, 8192);
  hipLaunchKernelGGL(norm_silu_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

// --------------------------------------------------------------------------
// Streaming first layer: padded [N][T+2][H+2][W+2][c_pad] from a strided
// channels-first chunk and P raw history frames (zeros in the border, the
// 2-P missing planes and channels >= C), then the cache: the last
// cache_frames frames of history ++ chunk, [N][cache_frames][H][W][C].
// One thread per padded pixel (16-byte stores of 8 channels), then one per
// cache pixel.
// --------------------------------------------------------------------------
__device__ __forceinline__ uint16_t stream_src(const StreamPackArgs& a, int nn, int s, int hq,
                                               int wq, int ch) {
  // frame s of history ++ chunk
  if (s < a.P)
    return a.history[((((long long)nn * a.P + s) * a.h + hq) * a.w + wq) * a.c + ch];
  return a.chunk[nn * a.sn + ch * a.sc + (long long)(s - a.P) * a.st + hq * a.sh + wq * a.sw];
}

__global__ __launch_bounds__(256) void stream_pack_kernel(StreamPackArgs a) {
  const long long np = (long long)a.n * (a.t + 2) * (a.h + 2) * (a.w + 2);
  const long long nc = (long long)a.n * a.cache_frames * a.h * a.w;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < np + nc;
       i += (long long)gridDim.x * blockDim.x) {
    if (i < np) {
      long long r = i;
      const int wp = (int)(r % (a.w + 2)); r /= a.w + 2;
      const int hp = (int)(r % (a.h + 2)); r /= a.h + 2;
      const int tp = (int)(r % (a.t + 2));
      const int nn = (int)(r / (a.t + 2));
      const bool inside = hp >= 1 && hp <= a.h && wp >= 1 && wp <= a.w && tp >= 2 - a.P;
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.padded + i * a.c_pad);
      for (int c8 = 0; c8 < a.c_pad; c8 += 8) {
        unsigned q[4] = {0u, 0u, 0u, 0u};
        if (inside) {
          for (int e = 0; e < 8 && c8 + e < a.c; ++e)
            q[e >> 1] |= (unsigned)stream_src(a, nn, tp - 2 + a.P, hp - 1, wp - 1, c8 + e)
                         << (16 * (e & 1));
        }
        dst[c8 / 8] = u32x4_t{q[0], q[1], q[2], q[3]};
      }
    } else {
      long long r = i - np;
      const int wq = (int)(r % a.w); r /= a.w;
      const int hq = (int)(r % a.h); r /= a.h;
      const int f = (int)(r % a.cache_frames);
      const int nn = (int)(r / a.cache_frames);
      const int s = a.P + a.t - a.cache_frames + f;
      uint16_t* dst = a.cache + (i - np) * a.c;
      for (int ch = 0; ch < a.c; ++ch) dst[ch] = stream_src(a, nn, s, hq, wq, ch);
    }
  }
}

int launch_stream_pack(const StreamPackArgs& a, void* stream) {
  const long long total = (long long)a.n * (a.t + 2) * (a.h + 2) * (a.w + 2) +
                          (long long)a.n * a.cache_frames * a.h * a.w;
  const long long blocks = std::min<long long>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(stream_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

// --------------------------------------------------------------------------
// Weight packing: OIDHW [Cout][Cin][27] -> [27][CC][Cout][32], zero beyond Cin.
// One thread per 16-byte output chunk (8 channels).
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint16_t* __restrict__ w,
                                                          uint16_t* __restrict__ wp, int cout,
                                                          int cin, int cc_n, int taps) {
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
        // a 9-tap (2D) weight fills the last temporal slice, t = 18 .. 26
        const int ts = t - (27 - taps);
        const unsigned v = (ci < cin && ts >= 0) ? w[((long long)co * cin + ci) * taps + ts] : 0u;
        v2 |= v << (16 * h);
      }
      out[k] = v2;
    }
    reinterpret_cast<u32x4_t*>(wp)[i] = out;
  }
}

// e4m3 weights: [cout][cin][27] bytes -> [27][cc_n][cout][64] bytes, zero
// beyond cin. One thread per 16-byte output chunk (16 channels).
__global__ __launch_bounds__(256) void pack_weight_fp8_kernel(const uint8_t* __restrict__ w,
                                                              uint8_t* __restrict__ wp, int cout,
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
      unsigned v4 = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int ci = cc * 64 + q * 16 + 4 * k + b;
        const unsigned v = (ci < cin) ? w[((long long)co * cin + ci) * 27 + t] : 0u;
        v4 |= v << (8 * b);
      }
      out[k] = v4;
    }
    reinterpret_cast<u32x4_t*>(wp)[i] = out;
  }
}

int launch_pack_weight_fp8(const uint8_t* w, uint8_t* wp, int cout, int cin, void* stream) {
  const int cc_n = (cin + 63) / 64;
  const long long total = 27LL * cc_n * cout * 4;
  const long long blocks = std::min<long long>((total + 255) / 256, 65535);
  hipLaunchKernelGGL(pack_weight_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, w, wp, cout, cin, cc_n);
  return (int)hipGetLastError();
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

// The same with 8-byte accesses, for A % 4 == 0 and B % 4 == 0 (every
// 4-element vector of a 64-aligned tile is then wholly inside or outside the
// array, and 8-byte aligned). Each thread loads four 4-element runs along B
// into the tile (rows padded to 68 elements, 8-byte aligned), then reads pairs
// of adjacent output rows as 32-bit words to assemble two 4-element runs along
// A at a time: a wave instruction moves 512 bytes instead of 128.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose4_kernel(const uint16_t* __restrict__ src,
                                                         uint16_t* __restrict__ dst, int A, int B,
                                                         int tiles_a, int tiles_b) {
  constexpr int RW = 68;   // tile row stride in elements
  __shared__ __align__(16) uint16_t tile[64 * RW];
  const int tb = blockIdx.x % tiles_b;
  const int ta = (blockIdx.x / tiles_b) % tiles_a;
  const long long n = blockIdx.x / ((long long)tiles_b * tiles_a);
  const int a0 = ta * 64, b0 = tb * 64;
  const uint16_t* s = src + n * (long long)A * B;
  uint16_t* d = dst + n * (long long)A * B;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int v = k * 256 + t;
    const int a = v >> 4, b4 = v & 15;
    if (a0 + a < A && b0 + b4 * 4 < B)
      *reinterpret_cast<uint2*>(&tile[a * RW + b4 * 4]) =
          *reinterpret_cast<const uint2*>(s + (long long)(a0 + a) * B + b0 + b4 * 4);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = k * 256 + t;
    const int a4 = q & 15, b2 = q >> 4;   // output rows 2*b2, 2*b2 + 1; A elements a4*4 .. +4
    unsigned w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = *reinterpret_cast<const unsigned*>(&tile[(a4 * 4 + i) * RW + 2 * b2]);
    const uint2 lo = {(w[0] & 0xffffu) | (w[1] << 16), (w[2] & 0xffffu) | (w[3] << 16)};
    const uint2 hi = {(w[0] >> 16) | (w[1] & 0xffff0000u), (w[2] >> 16) | (w[3] & 0xffff0000u)};
    const int bi = b0 + 2 * b2, ai = a0 + a4 * 4;
    if (ai < A) {
      if (bi < B) *reinterpret_cast<uint2*>(d + (long long)bi * A + ai) = lo;
      if (bi + 1 < B) *reinterpret_cast<uint2*>(d + (long long)(bi + 1) * A + ai) = hi;
    }
  }
}

// The same with 16-byte accesses and no LDS, for A % 8 == 0: each thread
// moves one 8 x 8 block of elements, eight 16-byte loads along B (two
// 8-byte loads per row when B % 8 == 4), a register transpose (one byte
// permute per output word) and eight 16-byte stores along A. A wave covers 8 x 8 blocks with the B block fastest across lanes,
// so every load and every store instruction moves eight whole 128-byte lines
// (8 rows x 8 lanes x 16 bytes). Blocks that reach past B, and every block
// when B % 4 != 0, move element by element.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose8_kernel(const uint16_t* __restrict__ src,
                                                         uint16_t* __restrict__ dst, int batch,
                                                         int A, int B, int groups_a, int groups_b) {
  const int lane = threadIdx.x & 63;
  const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long per_n = (long long)groups_a * groups_b;
  const long long n = wave / per_n;
  if (n >= batch) return;   // the last work-group's spare waves
  const int rest = (int)(wave - n * per_n);
  const int ga = rest / groups_b, gb = rest - ga * groups_b;
  const int a0 = (ga * 8 + (lane >> 3)) * 8;     // this thread's block: rows a0 .. a0 + 7
  const int b0 = (gb * 8 + (lane & 7)) * 8;      // columns b0 .. b0 + 7
  if (a0 >= A || b0 >= B) return;
  const uint16_t* s = src + n * (long long)A * B;
  uint16_t* d = dst + n * (long long)A * B;
  if (b0 + 8 <= B && (B & 3) == 0) {
    uint4 in[8];
    if ((B & 7) == 0) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        in[r] = *reinterpret_cast<const uint4*>(s + (long long)(a0 + r) * B + b0);
    } else {   // rows 8-byte aligned only: two 8-byte loads per row
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint2 lo = *reinterpret_cast<const uint2*>(s + (long long)(a0 + r) * B + b0);
        const uint2 hi = *reinterpret_cast<const uint2*>(s + (long long)(a0 + r) * B + b0 + 4);
        in[r] = uint4{lo.x, lo.y, hi.x, hi.y};
      }
    }
    const unsigned* w = reinterpret_cast<const unsigned*>(in);   // w[r * 4 + k]: halves 2k, 2k+1
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // output row b0 + c: element r is input row r's half c
      const unsigned sel = (c & 1) ? 0x07060302u : 0x05040100u;
      uint4 o;
      o.x = __builtin_amdgcn_perm(w[1 * 4 + c / 2], w[0 * 4 + c / 2], sel);
      o.y = __builtin_amdgcn_perm(w[3 * 4 + c / 2], w[2 * 4 + c / 2], sel);
      o.z = __builtin_amdgcn_perm(w[5 * 4 + c / 2], w[4 * 4 + c / 2], sel);
      o.w = __builtin_amdgcn_perm(w[7 * 4 + c / 2], w[6 * 4 + c / 2], sel);
      *reinterpret_cast<uint4*>(d + (long long)(b0 + c) * A + a0) = o;
    }
  } else {
    for (int c = 0; c < 8 && b0 + c < B; ++c)
      for (int r = 0; r < 8; ++r) d[(long long)(b0 + c) * A + a0 + r] = s[(long long)(a0 + r) * B + b0 + c];
  }
}

// --------------------------------------------------------------------------
// Zeroes the persistent tile queues before a launch (a kernel rather than a
// memset so the sequence can be captured in a graph).
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void queue_reset_kernel(unsigned* queue) {
  for (int i = threadIdx.x; i < (int)(kQueueBytes / 4); i += blockDim.x) queue[i] = 0u;
}

// --------------------------------------------------------------------------
// Launchers.
// --------------------------------------------------------------------------
int launch_pack_weight(const uint16_t* w, uint16_t* wp, int cout, int cin, int taps, void* stream) {
  const int cc_n = (cin + 31) / 32;
  const long long total = 27LL * cc_n * cout * 4;
  long long blocks = (total + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, w, wp, cout, cin, cc_n, taps);
  return (int)hipGetLastError();
}

int launch_transpose(const uint16_t* src, uint16_t* dst, int n, int A, int B, void* stream) {
  if (A % 8 == 0) {   // 16-byte path; ragged B handled inside
    const int ga = (A / 8 + 7) / 8, gb = ((B + 7) / 8 + 7) / 8;
    const long long waves = (long long)n * ga * gb;
    hipLaunchKernelGGL(transpose8_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       (hipStream_t)stream, src, dst, n, A, B, ga, gb);
    return (int)hipGetLastError();
  }
  const int ta = (A + 63) / 64, tb = (B + 63) / 64;
  const long long blocks = (long long)n * ta * tb;
  if (A % 4 == 0 && B % 4 == 0)
    hipLaunchKernelGGL(transpose4_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, src, dst, A, B, ta, tb);
  else
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, src, dst, A, B, ta, tb);
  return (int)hipGetLastError();
}

// --------------------------------------------------------------------------
// Scratch of the entry point that allocates nothing. In host code `scratch`
// names a host-side stand-in, not device memory: only the address
// hipGetSymbolAddress returns for the current device may reach a kernel.
// --------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int scratch_address(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int launch_queue_reset(unsigned* queue, void* stream) {
  hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, queue);
  return (int)hipGetLastError();
}

int launch_reduce(const ReduceArgs& args, void* stream) {
  if (args.frag) {
    const long long tasks = (long long)args.m_tiles * args.n_tiles * 4 * args.pb * args.cb * 128;
    long long blocks = (tasks + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(reduce_frag_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, args);
  } else if (args.flags & F_NORM) {
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

}  // namespace conv3d
