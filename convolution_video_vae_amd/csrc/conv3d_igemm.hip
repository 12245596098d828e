// Implicit-GEMM main kernels of the bf16 3x3x3 NDHWC Conv3D on gfx950.
//
// The convolution is a GEMM whose activation operand is gathered on the fly
// (FlyDSL issue "conv3d_implicit — accept and emit NDHWC ...", maintainer
// reply): D[co][m] = sum_k W[co][k] * X[k][m], m an output pixel and
// k = (tap, input channel). Causal and spatial zero padding live only in the
// gather (Qwen-Image PR page, "T=1 degeneration"): a tap outside the input
// gets an out-of-range offset and the buffer unit's range check returns zeros,
// so no padded copy of the input exists.
//
// One K step is 32 input channels of one tap. The accumulators are
// D[co][pixel] blocks of v_mfma_f32_32x32x16_bf16 (R = 32) or
// v_mfma_f32_16x16x32_bf16 (R = 16). Per work-group of WM x WN waves:
//  * weights: the [BN][32] slice of the packed weight for a K step is fetched
//    3 steps ahead into a register staging ring, copied into an LDS ring 2
//    steps ahead, and read into MFMA A-operand registers 1 step ahead, so no
//    global or LDS latency sits between consecutive steps' MFMAs; one barrier
//    per step. Weight rows are placed in a permuted order so that each lane's
//    accumulators are consecutive output channels of one pixel, which makes
//    the NDHWC stores 16-byte runs.
//  * activations: each wave gathers its own pixels straight into VGPRs in the
//    MFMA B-operand layout (16 bytes = 8 channels of one pixel per lane),
//    2 steps ahead.
//  * taps that no pixel of the tile can see (the two causal planes at T=1,
//    frame edges) are skipped; steps are walked as (tap, channel chunk) with a
//    find-first-set over the live-tap mask, and tap offsets come from the
//    kernel arguments, so the loop has no integer division.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "conv3d_device.h"
#include "conv3d_internal.h"

namespace conv3d {

namespace {

constexpr unsigned kOobOffset = 0x80000000u;  // beyond any operand (< 2 GiB)

// 16x16x32: lane l supplies operand row/col (l & 15) and channels
// 8*(l >> 4) .. +8 of the 32; it holds D rows 4*(l >> 4) + e, col (l & 15).
struct Mfma16 {
  static constexpr int R = 16;
  static constexpr int KS = 1;      // MFMAs per 32-channel K step
  static constexpr int NACC = 4;    // accumulator floats per lane per block
  static constexpr int KCH = 32;    // channels per K step (64 bytes a pixel)
  static constexpr int CCH = 8;     // channels per 16-byte chunk
  static constexpr int ESZ = 2;     // bytes per element
  static constexpr bool WIDE = false;  // one MFMA per chunk (not per K step)
  typedef f32x4_t acc_t;
  __device__ static int row(int lane) { return lane & 15; }
  __device__ static int grp(int lane) { return lane >> 4; }
  __device__ static int chunk(int lane, int /*h*/) { return lane >> 4; }
  __device__ static acc_t mma(bf16x8_t a, bf16x8_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // Wave-local channel that D row r of block cb stands for: a lane of group
  // g holds channels g*4*CB + 4*cb + e, one run of 4*CB.
  __device__ static int chan_of(int cb, int r, int CB) { return (r >> 2) * 4 * CB + 4 * cb + (r & 3); }
  __device__ static void row_of(int c, int CB, int& cb, int& r) {
    const int g = c / (4 * CB), rem = c % (4 * CB);
    cb = rem >> 2;
    r = 4 * g + (rem & 3);
  }
};

// 32x32x16: lane l supplies operand row/col (l & 31) and channels
// 16*h + 8*(l >> 5) .. +8 for K half h; it holds D rows
// 8*(e >> 2) + 4*(l >> 5) + (e & 3), col (l & 31).
struct Mfma32 {
  static constexpr int R = 32;
  static constexpr int KS = 2;
  static constexpr int NACC = 16;
  static constexpr int KCH = 32, CCH = 8, ESZ = 2;
  static constexpr bool WIDE = false;
  typedef f32x16_t acc_t;
  __device__ static int row(int lane) { return lane & 31; }
  __device__ static int grp(int lane) { return lane >> 5; }
  __device__ static int chunk(int lane, int h) { return 2 * h + (lane >> 5); }
  __device__ static acc_t mma(bf16x8_t a, bf16x8_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // A lane of group g holds channels g*16*CB + 16*cb + e.
  __device__ static int chan_of(int cb, int r, int CB) {
    return ((r >> 2) & 1) * 16 * CB + 16 * cb + 4 * (r >> 3) + (r & 3);
  }
  __device__ static void row_of(int c, int CB, int& cb, int& r) {
    const int g = c / (16 * CB), rem = c % (16 * CB);
    cb = rem >> 4;
    r = 8 * ((rem & 15) >> 2) + 4 * g + (rem & 3);
  }
};

// fp8 (e4m3) operands, v_mfma_f32_32x32x64_f8f6f4: a K step is 64 channels
// (64 bytes of a pixel, the same four 16-byte chunks as a bf16 step); lane l
// supplies row/col (l & 31) and the 32 bytes of chunks 2*(l >> 5) and
// 2*(l >> 5) + 1 of both operands, so the hardware's assignment of those
// bytes to K only has to agree between A and B, which it does. One MFMA per K
// step; D as for Mfma32.
typedef int i32x8_t __attribute__((ext_vector_type(8)));
struct Mfma32F8 : Mfma32 {
  static constexpr int KCH = 64, CCH = 16, ESZ = 1;
  static constexpr bool WIDE = true;
  __device__ static int chunk(int lane, int h) { return 2 * (lane >> 5) + h; }
  __device__ static acc_t mma2(const u32x4_t& a0, const u32x4_t& a1, const u32x4_t& b0,
                               const u32x4_t& b1, acc_t c) {
    const i32x8_t a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                       (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8_t b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                       (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    // formats 0/0: e4m3 x e4m3; zero scale operands select the unscaled form
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

// LDS weight tile: rows of four 16-byte chunks (32 channels). The chunk index
// is XORed with row bits so the 8 or 16 consecutive rows one operand read
// touches land in distinct bank groups.
__device__ __forceinline__ int lds_idx(int row, int chunk) {
  return row * 4 + (chunk ^ (((row >> 1) ^ (row >> 3)) & 3));
}

// Work-group -> (pixel tile, channel tile, K split). Work-groups are dealt
// round-robin to the 8 XCDs; give each XCD a contiguous run of tiles so tiles
// sharing input rows or a weight slice meet in the same L2.
struct TileCoord {
  int m0, co0, split;
  int m_end;   // slot kernel: end of the tile's slot range
  int nsplit;  // K slices of this tile
  int slot;    // halo-kernel partials: the work-group's partial tile
};
__device__ __forceinline__ int xcd_run(int bid) {
  const int G8 = gridDim.x & ~7;
  return bid < G8 ? (bid & 7) * (G8 >> 3) + (bid >> 3) : bid;
}
__device__ __forceinline__ TileCoord tile_coord(const IgemmArgs& a, int BM, int BN) {
  const int bid = xcd_run(blockIdx.x);
  const int m_tile = bid % a.m_tiles;
  const int rest = bid / a.m_tiles;
  TileCoord t;
  t.m0 = m_tile * BM;
  t.co0 = (rest % a.n_tiles) * BN;
  t.split = rest / a.n_tiles;
  t.nsplit = a.splits;
  t.slot = (t.split * a.m_tiles + m_tile) * a.n_tiles + rest % a.n_tiles;
  return t;
}
// The same for a live-balanced split (a.vsplit): the host's table entry of
// this work-group.
__device__ __forceinline__ TileCoord tile_coord_live(const IgemmArgs& a, int BM, int BN) {
  const unsigned long long e = a.vwg[blockIdx.x];
  TileCoord t;
  t.m0 = (int)(e & 0xFFFFu) * BM;
  t.co0 = (int)((e >> 16) & 0xFFFFu) * BN;
  t.split = (int)((e >> 32) & 0xFFu);
  t.nsplit = (int)((e >> 40) & 0xFFu);
  t.slot = (int)(e >> 48);
  return t;
}
// Next tile of a persistent work-group (called by one thread): hand-out
// position i comes from this XCD's queue (XCD x owns chunks x, x + 8, ... of
// kQueueChunk positions) until that reaches the shared tail of the last
// `tail` positions, which every XCD then draws from in turn. Tiles
// go out in reverse order (position i is tile T - 1 - i), longest first for
// a causal layer. Returns -1 when every tile is taken.
__device__ __forceinline__ int queue_take(unsigned* q, int T, int tail) {
  const int split = T - tail;
  const int x = blockIdx.x & 7;
  const int j = (int)atomicAdd(q + x * kQueueStride, 1u);
  int i = ((j / kQueueChunk) * 8 + x) * kQueueChunk + j % kQueueChunk;
  if (i >= split) i = split + (int)atomicAdd(q + 8 * kQueueStride, 1u);
  return i < T ? T - 1 - i : -1;
}

// Nominal K step (pair * CC + chunk) of the j-th live step, j < popc(live) * CC.
__device__ __forceinline__ int live_step(unsigned live, int j, int CC) {
  const int k = j / CC;
  unsigned m = live;
  for (int i = 0; i < k; ++i) m &= m - 1;
  return __builtin_ctz(m) * CC + (j - k * CC);
}

// Per-lane geometry of PB pixel blocks: byte offset of tap (0,0,0) and a
// 27-bit mask of the taps that fall inside the input. With reflect padding
// every spatial tap reads real input and bits 27-30 flag the pixels whose
// first row / last row / first column / last column tap is reflected.
template <int PB, int R, bool REF = false, int ESZ = 2>
__device__ __forceinline__ unsigned pixel_geometry(const IgemmArgs& a, int m_first,
                                                   long long (&base)[PB], unsigned (&tapmask)[PB]) {
  unsigned live = 0;
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const int m = m_first + p * R;
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
        vh |= (unsigned)(REF || (h0 + k >= 0 && h0 + k < a.H)) << k;
        vw |= (unsigned)(REF || (w0 + k >= 0 && w0 + k < a.W)) << k;
      }
      unsigned tm = 0;
#pragma unroll
      for (int t = 0; t < 27; ++t)
        tm |= ((vd >> (t / 9)) & (vh >> ((t / 3) % 3)) & (vw >> (t % 3)) & 1u) << t;
      if (REF)
        tm |= ((unsigned)(h0 < 0) << 27) | ((unsigned)(h0 + 2 >= a.H) << 28) |
              ((unsigned)(w0 < 0) << 29) | ((unsigned)(w0 + 2 >= a.W) << 30);
      tapmask[p] = tm;
      base[p] = ((((long long)n * a.D + d0) * a.H + h0) * a.W + w0) * (a.Cin * ESZ);
    }
    live |= tapmask[p];
  }
  return live & ((1u << 27) - 1u);
}

// floor(n / d) for 0 <= n < 2^22 and 0 < d < 2^22, from a float reciprocal
// and one correction each way.
__device__ __forceinline__ int small_div(int n, int d, float inv_d) {
  int q = (int)((float)n * inv_d);
  if ((q + 1) * d <= n) ++q;
  if (q * d > n) --q;
  return q;
}

// Index in y of output pixel m: m itself, or (a.ypad) its place in the
// padded output (pixel indices below 2^24, so the float splits are exact).
__device__ __forceinline__ int y_pixel(const IgemmArgs& a, int m) {
  if (!a.ypad) return m;
  const int r = small_div(m, a.Wo, a.inv_wo);
  const int t = small_div(r, a.Ho, a.inv_ho);
  const int n = small_div(t, a.Do, a.inv_do);
  return ((n * a.yDy + (t - n * a.Do) + a.ypt) * a.yHy + (r - t * a.Ho) + a.yph) * a.yWy +
         (m - r * a.Wo) + a.ypw;
}
// Elements of y: M x Cout, or the padded output's.
__device__ __forceinline__ unsigned y_elems(const IgemmArgs& a) {
  return a.ypad ? (unsigned)a.N * (unsigned)(a.yDy * a.yHy * a.yWy) * (unsigned)a.Cout
                : (unsigned)a.M * (unsigned)a.Cout;
}

// Reflect padding (the H3 encoder's spatial pad): index -1 reads 1 and index
// n reads n - 2 (pads of at most one, extents of at least two).
__device__ __forceinline__ int reflect_index(int i, int n) {
  return i < 0 ? -i : (i >= n ? 2 * n - 2 - i : i);
}

// (kd, kh) pairs of an output row whose input rows start at (d0, h0): bit
// kd * 3 + kh set when the pair reads real input. Time is always zero
// padded; with reflect padding every kh reads a real row, and bit 9 (h0 = -1:
// tap kh = 0 reads row 1, two rows down) and bit 10 (h0 + 2 = H: tap kh = 2
// reads row H - 2, two rows up) tell the gathers where to move.
template <bool REF>
__device__ __forceinline__ unsigned row_mask(const IgemmArgs& a, int d0, int h0) {
  unsigned m = 0;
#pragma unroll
  for (int kd = 0; kd < 3; ++kd)
#pragma unroll
    for (int kh = 0; kh < 3; ++kh) {
      const bool hv = REF || (h0 + kh >= 0 && h0 + kh < a.H);
      m |= (unsigned)(d0 + kd >= 0 && d0 + kd < a.D && hv) << (kd * 3 + kh);
    }
  if (REF) m |= ((unsigned)(h0 < 0) << 9) | ((unsigned)(h0 + 2 >= a.H) << 10);
  return m;
}

// Lane index of the calling lane, recomputed where it is called (volatile,
// so not hoisted into a register that lives through a main loop).
__device__ __forceinline__ int lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// OR of a 9-bit mask over the wave, through ballots (scalar results, no
// lane-index registers).
__device__ __forceinline__ unsigned wave_or9(unsigned v) {
  unsigned r = 0;
#pragma unroll
  for (int b = 0; b < 9; ++b) r |= (__builtin_amdgcn_ballot_w64(((v >> b) & 1u) != 0u) != 0 ? 1u : 0u) << b;
  return r;
}

__device__ __forceinline__ unsigned wave_or(unsigned v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= __shfl_xor(v, o);
  return v;
}

template <int I>
struct SlotC {
  static constexpr int value = I;
};

// Calls f(SlotC<0>{}) .. f(SlotC<N-1>{}): a loop whose index is a constant
// expression in the body.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(SlotC<I>{});
    static_for<N, I + 1>(f);
  }
}

// K steps are encoded e = (tap << 8) | channel chunk; kEnd marks none.
constexpr int kEnd = 0x7fffffff;

// Gather of K step e into MFMA B-operand fragments. Branch-free: an invalid
// tap or channel group ORs the top bit into the offset, which the buffer range
// check turns into zeros.
// A step of kEnd loads zeros (every offset out of range), so prefetches are
// issued unconditionally and the wait counts stay static.
template <class T, int PB, bool REF = false>
__device__ __forceinline__ void gather_x(const IgemmArgs& a, __amdgpu_buffer_rsrc_t rsrc, int e,
                                         int lane, const long long (&base)[PB],
                                         const unsigned (&tapmask)[PB], u32x4_t (&dst)[PB][T::KS]) {
  const bool valid = e != kEnd;
  const int t = valid ? e >> 8 : 0, cc = valid ? e & 255 : 0;
  const int kd = t / 9, kh = (t / 3) % 3, kw = t % 3;
  const long long delta =
      (((long long)kd * a.H + kh) * a.W + kw) * (long long)(a.Cin * T::ESZ) + cc * 64;
#pragma unroll
  for (int h = 0; h < T::KS; ++h) {
    const int ch = T::chunk(lane, h);
    const unsigned chan_ok = (unsigned)(valid && cc * T::KCH + ch * T::CCH < a.Cin);
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const unsigned ok = chan_ok & (tapmask[p] >> t);
      long long adj = 0;
      if (REF) {  // reflected taps: two rows / columns back inside
        const unsigned f = tapmask[p];
        const int rowb = a.W * a.Cin * T::ESZ, colb = a.Cin * T::ESZ;
        if (kh == 0 && ((f >> 27) & 1u)) adj += 2 * rowb;
        if (kh == 2 && ((f >> 28) & 1u)) adj -= 2 * rowb;
        if (kw == 0 && ((f >> 29) & 1u)) adj += 2 * colb;
        if (kw == 2 && ((f >> 30) & 1u)) adj -= 2 * colb;
      }
      const unsigned off =
          (unsigned)(base[p] + delta + adj + ch * 16) | (((ok & 1u) - 1u) & kOobOffset);
      dst[p][h] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, 0);
    }
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_rsrc(const IgemmArgs& a) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)a.x_bytes, 0x00020000);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t w_rsrc(const IgemmArgs& a) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)a.wp, (short)0, (int)(27u * a.CC * a.Cout * 64u),
                                           0x00020000);
}

// Output pixel of each of a lane's pixel blocks: m_first + p*R, or -1 past M.
template <int PB, int R>
__device__ __forceinline__ void block_pixels(int m_first, int M, int (&mp)[PB]) {
#pragma unroll
  for (int p = 0; p < PB; ++p) mp[p] = (m_first + p * R < M) ? m_first + p * R : -1;
}

// Epilogue. For pixel block p the lane holds channels cbase .. cbase+RUN-1 of
// output pixel mp[p] (none if negative): run position NACC*cb + e is
// acc[cb][p][e].
//   EPI_PARTIAL: fp32 partial sums of this K split.
//   EPI_STORE:   value = B(B(B(acc) + bias) + residual), each step if enabled.
//   EPI_NORM:    the whole contract; the work-group holds the pixel's full
//                channel row (BN == Cout), its WN waves meeting through `red`.
template <class T, int WM, int WN, int PB, int CB, int EPI>
__device__ __forceinline__ void epilogue(const IgemmArgs& a, typename T::acc_t (&acc)[CB][PB],
                                         const int (&mp)[PB], int cbase, int split, int wave_m, int wave_n,
                                         int lrow, int lgrp, float* red) {
  constexpr int R = T::R, NACC = T::NACC, RUN = NACC * CB;
  if (EPI == EPI_PARTIAL) {
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int m = mp[p];
      if (m < 0 || cbase >= a.Cout) continue;
      f32x4_t* dst =
          reinterpret_cast<f32x4_t*>(a.partial + ((long long)split * a.M + m) * a.Cout + cbase);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int q = 0; q < NACC / 4; ++q)
          dst[(NACC * cb) / 4 + q] = f32x4_t{acc[cb][p][4 * q], acc[cb][p][4 * q + 1],
                                             acc[cb][p][4 * q + 2], acc[cb][p][4 * q + 3]};
    }
    return;
  }
  if (EPI == EPI_STORE) {
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      // One pixel block at a time keeps the converted values' registers few.
      __builtin_amdgcn_sched_barrier(0);
      const int m = mp[p];
      if (m < 0 || cbase >= a.Cout) continue;
      const long long off = (long long)m * a.Cout + cbase;
      const long long yoff = (long long)y_pixel(a, m) * a.Cout + cbase;
#pragma unroll
      for (int c8 = 0; c8 < RUN; c8 += 8) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = rbf(acc[(c8 + e) / NACC][p][(c8 + e) % NACC]);
        if (a.flags & F_BIAS) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = rbf(v[e] + a.bias[cbase + c8 + e]);
        }
        if (a.flags & F_RESIDUAL) {
          const u32x4_t rv = *reinterpret_cast<const u32x4_t*>(a.residual + off + c8);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = rbf(v[e] + lane_bf(rv, e));
        }
        const u32x4_t ov = {pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
        if (a.flags & F_RESIDUAL_OUT) *reinterpret_cast<u32x4_t*>(a.residual_out + off + c8) = ov;
        *reinterpret_cast<u32x4_t*>(a.y + yoff + c8) = ov;
      }
    }
    return;
  }
  // EPI_NORM, one pixel block at a time: the block's values (bf16 by
  // construction, kept packed two per register) and its row sum of squares,
  // the sum over the WN waves sharing the pixel, then the post-operations.
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const int m = mp[p];
    const bool ok = m >= 0;
    const long long off = (long long)(ok ? m : 0) * a.Cout + cbase;
    const long long yoff = (long long)y_pixel(a, ok ? m : 0) * a.Cout + cbase;
    unsigned vpk[RUN / 2];
    float t = 0.f;
#pragma unroll
    for (int c8 = 0; c8 < RUN; c8 += 8) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = rbf(acc[(c8 + e) / NACC][p][(c8 + e) % NACC]);
      if (a.flags & F_BIAS) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = rbf(v[e] + a.bias[cbase + c8 + e]);
      }
      if ((a.flags & F_RESIDUAL) && ok) {
        const u32x4_t rv = *reinterpret_cast<const u32x4_t*>(a.residual + off + c8);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = rbf(v[e] + lane_bf(rv, e));
      }
      const u32x4_t ov = {pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
      if ((a.flags & F_RESIDUAL_OUT) && ok) *reinterpret_cast<u32x4_t*>(a.residual_out + off + c8) = ov;
#pragma unroll
      for (int q = 0; q < 4; ++q) vpk[c8 / 2 + q] = ov[q];
#pragma unroll
      for (int e = 0; e < 8; ++e) t += v[e] * v[e];
    }
#pragma unroll
    for (int o = R; o < 64; o <<= 1) t += __shfl_xor(t, o);  // lanes of the same pixel
    if (WN > 1) {  // ... and the WN waves (a slot per pixel block: no reuse)
      if (lgrp == 0) red[((wave_n * WM + wave_m) * PB + p) * R + lrow] = t;
      __syncthreads();
      t = 0.f;
      for (int wn = 0; wn < WN; ++wn) t += red[((wn * WM + wave_m) * PB + p) * R + lrow];
    }
    const float rden = 1.0f / fmaxf(sqrtf(t), 1e-12f);
#pragma unroll
    for (int c8 = 0; c8 < RUN; c8 += 8) {
      const u32x4_t gv = *reinterpret_cast<const u32x4_t*>(a.gamma + cbase + c8);
      const u32x4_t vv = {vpk[c8 / 2], vpk[c8 / 2 + 1], vpk[c8 / 2 + 2], vpk[c8 / 2 + 3]};
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = norm_silu_value(lane_bf(vv, e), rden, a.sqrt_c, lane_bf(gv, e));
      const u32x4_t ov = {pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7])};
      if (ok) *reinterpret_cast<u32x4_t*>(a.y + yoff + c8) = ov;
    }
  }
}

}  // namespace

// ----------------------------------------------------------------------------
// Main kernel. A pipeline step is KB consecutive live K steps (KB*32
// channels); NS is the depth of the rings (pixel fragments NS-1 steps
// ahead, weight fetches NS steps ahead, LDS stages 2 ahead, weight fragments
// 1 ahead).
// ----------------------------------------------------------------------------
template <class T, int WM, int WN, int PB, int CB, int KB, int NS, int EPI, bool REF = false>
__global__ __launch_bounds__(64 * WM * WN) void igemm_kernel(IgemmArgs a) {
  constexpr int R = T::R, KS = T::KS, NACC = T::NACC;
  constexpr int NT = 64 * WM * WN;
  constexpr int BM = R * PB * WM;
  constexpr int BN = R * CB * WN;
  constexpr int CHUNKS = BN * 4;               // 16-byte chunks per weight slice
  constexpr int CPT = (CHUNKS + NT - 1) / NT;  // chunks per thread
  constexpr int RUN = NACC * CB;
  typedef typename T::acc_t acc_t;
  static_assert(RUN % 8 == 0, "each lane must hold whole 16-byte runs of channels");
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  constexpr int NF = (NS % 2 == 0) ? 2 : NS;  // weight-fragment ring: current + next

  __shared__ u32x4_t wlds[NS][KB][CHUNKS];
  __shared__ float red[(EPI == EPI_NORM && WN > 1) ? WM * WN * PB * R : 1];
  __shared__ unsigned live_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave % WM;
  const int wave_n = wave / WM;
  const int lrow = T::row(lane);
  const int lgrp = T::grp(lane);
  const TileCoord tc = tile_coord(a, BM, BN);
  const int m_first = tc.m0 + wave_m * PB * R + lrow;

  long long base[PB];
  unsigned tapmask[PB];
  unsigned live = wave_or(pixel_geometry<PB, R, REF, T::ESZ>(a, m_first, base, tapmask));
  // Taps no pixel of the tile can see are skipped by the whole work-group.
  if (tid == 0) live_sh = 0;
  __syncthreads();
  if (lane == 0) atomicOr(&live_sh, live);
  __syncthreads();
  live = __builtin_amdgcn_readfirstlane(live_sh);
  const __amdgpu_buffer_rsrc_t xrsrc = x_rsrc(a);
  const __amdgpu_buffer_rsrc_t wrsrc = w_rsrc(a);

  // K steps of this split, in (tap, chunk) order, live taps only.
  const int s_begin = tc.split * a.steps_per_split;
  const int s_end = min(s_begin + a.steps_per_split, 27 * a.CC);
  auto valid_step = [&](int t, int cc) -> int {
    return (t < 27 && t * a.CC + cc < s_end) ? ((t << 8) | cc) : kEnd;
  };
  auto next_step = [&](int e) -> int {
    if (e == kEnd) return kEnd;
    int t = e >> 8, cc = (e & 255) + 1;
    if (cc == a.CC) {
      cc = 0;
      const unsigned rest = live & (~0u << (t + 1));
      t = rest ? __builtin_ctz(rest) : 27;
    }
    return valid_step(t, cc);
  };
  auto first_step = [&]() -> int {
    if (s_begin >= s_end) return kEnd;
    int t = s_begin / a.CC, cc = s_begin % a.CC;
    if (!((live >> t) & 1u)) {
      const unsigned rest = live & (~0u << t);
      t = rest ? __builtin_ctz(rest) : 27;
      cc = 0;
    }
    return valid_step(t, cc);
  };
  // A pipeline step: KB consecutive K steps starting after `prev`.
  auto next_group = [&](int prev, int (&g)[KB]) {
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      g[k] = next_step(prev);
      prev = g[k];
    }
  };

  acc_t acc[CB][PB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int p = 0; p < PB; ++p)
#pragma unroll
      for (int e = 0; e < NACC; ++e) acc[cb][p][e] = 0.f;

  // Weight slice chunk c (row c >> 2, 16-byte chunk c & 3) -> LDS row in
  // MFMA order: wave-column, block cb, D row r.
  auto lds_row_of = [&](int c) -> int {
    const int col = c >> 2;
    int cb, r;
    T::row_of(col % (R * CB), CB, cb, r);
    return ((col / (R * CB)) * CB + cb) * R + r;
  };
  unsigned woff[CPT];  // this thread's chunks, relative to a step's slice
  int wdst[CPT];       // and where they go in an LDS slice
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + i * NT;
    const bool ok = c < CHUNKS && tc.co0 + (c >> 2) < a.Cout;
    woff[i] = ok ? (unsigned)((tc.co0 * 4 + c) * 16) : kOobOffset;
    wdst[i] = (c < CHUNKS) ? lds_idx(lds_row_of(c), c & 3) : 0;
  }
  // Every fetch below is unconditional (a step of kEnd reads zeros, a
  // finished pipeline reads or writes LDS slots no later step uses), so the
  // compiler's wait counts are exact.
  auto load_w = [&](const int (&g)[KB], u32x4_t (&dst)[KB][CPT]) {
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int e = g[k];
      const unsigned soff =
          (e == kEnd) ? kOobOffset : (unsigned)((e >> 8) * a.CC + (e & 255)) * (unsigned)a.Cout * 64u;
#pragma unroll
      for (int i = 0; i < CPT; ++i)
        dst[k][i] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)(woff[i] + soff), 0, 0);
    }
  };
  auto store_w = [&](int stage, const u32x4_t (&src)[KB][CPT]) {
#pragma unroll
    for (int k = 0; k < KB; ++k)
#pragma unroll
      for (int i = 0; i < CPT; ++i)
        if (CHUNKS % NT == 0 || tid + i * NT < CHUNKS) wlds[stage][k][wdst[i]] = src[k][i];
  };
  auto read_frags = [&](int stage, u32x4_t (&dst)[KB][CB][KS]) {
#pragma unroll
    for (int k = 0; k < KB; ++k)
#pragma unroll
      for (int h = 0; h < KS; ++h)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          dst[k][cb][h] = wlds[stage][k][lds_idx((wave_n * CB + cb) * R + lrow, T::chunk(lane, h))];
  };
  auto gather = [&](const int (&g)[KB], u32x4_t (&dst)[KB][PB][KS]) {
#pragma unroll
    for (int k = 0; k < KB; ++k) gather_x<T, PB, REF>(a, xrsrc, g[k], lane, base, tapmask, dst[k]);
  };

  u32x4_t xr[NS][KB][PB][KS];   // pixel fragments
  u32x4_t wst[NS][KB][CPT];     // weight slices in flight to LDS
  u32x4_t wfr[NF][KB][CB][KS];  // weight fragments

  // Pipeline steps of iterations i .. i+NS: ev[j] (KB K steps each).
  int ev[NS + 1][KB];
  {
    int prev = first_step();
    ev[0][0] = prev;
#pragma unroll
    for (int k = 1; k < KB; ++k) ev[0][k] = prev = next_step(prev);
#pragma unroll
    for (int j = 1; j <= NS; ++j) {
      next_group(prev, ev[j]);
      prev = ev[j][KB - 1];
    }
  }
  // Prologue: pixels of steps 0..NS-2, weights of steps 0..NS-1, LDS stages
  // of steps 0 and 1, fragments of step 0.
#pragma unroll
  for (int j = 0; j < NS - 1; ++j) gather(ev[j], xr[j]);
#pragma unroll
  for (int j = 0; j < NS; ++j) load_w(ev[j], wst[j]);
  store_w(0, wst[0]);
  store_w(1, wst[1]);
  __syncthreads();
  read_frags(0, wfr[0]);

  // Iteration i (ring slot i % NS) computes step ev[0]. The body is
  // instantiated once per slot so every ring index is a constant.
  auto iteration = [&](auto slot_c) -> bool {
    constexpr int slot = decltype(slot_c)::value;
    constexpr int s1 = (slot + 1) % NS, s2 = (slot + 2) % NS, sx = (slot + NS - 1) % NS;
    constexpr int f0 = slot % NF, f1 = (slot + 1) % NF;
    if (ev[0][0] == kEnd) return false;
    // Next step's fragments first: their LDS latency overlaps this step's
    // MFMAs instead of the barrier.
    read_frags(s1, wfr[f1]);
    __builtin_amdgcn_sched_barrier(0);
    gather(ev[NS - 1], xr[sx]);
    load_w(ev[NS], wst[slot]);
    if constexpr (T::WIDE) {
#pragma unroll
      for (int k = 0; k < KB; ++k)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int p = 0; p < PB; ++p)
            acc[cb][p] = T::mma2(wfr[f0][k][cb][0], wfr[f0][k][cb][1], xr[slot][k][p][0],
                                 xr[slot][k][p][1], acc[cb][p]);
    } else {
#pragma unroll
      for (int k = 0; k < KB; ++k)
#pragma unroll
        for (int h = 0; h < KS; ++h)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int p = 0; p < PB; ++p)
              acc[cb][p] = T::mma(__builtin_bit_cast(bf16x8_t, wfr[f0][k][cb][h]),
                                  __builtin_bit_cast(bf16x8_t, xr[slot][k][p][h]), acc[cb][p]);
    }
    // Step i+2's slices into their stage, last read before the previous
    // barrier.
    store_w(s2, wst[s2]);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int k = 0; k < KB; ++k) ev[j][k] = ev[j + 1][k];
    next_group(ev[NS - 1][KB - 1], ev[NS]);
    return true;
  };
  for (;;) {
    if (!iteration(SlotC<0>{})) break;
    if (!iteration(SlotC<1>{})) break;
    if constexpr (NS > 2) {
      if (!iteration(SlotC<2 % NS>{})) break;
    }
    if constexpr (NS > 3) {
      if (!iteration(SlotC<3 % NS>{})) break;
    }
  }
  int mp[PB];
  block_pixels<PB, R>(m_first, a.M, mp);
  epilogue<T, WM, WN, PB, CB, EPI>(a, acc, mp, tc.co0 + wave_n * R * CB + lgrp * RUN, tc.split,
                                   wave_m, wave_n, lrow, lgrp, red);
}

// Plain store (no bias, residual or norm): each lane's RUN consecutive
// channels of its PB pixels, rounded to bf16, as 16-byte buffer stores; a
// pixel past M gets an out-of-range offset, so the store is dropped.
template <class T, int PB, int CB>
__device__ __forceinline__ void store_plain(const IgemmArgs& a, typename T::acc_t (&acc)[CB][PB],
                                            const int (&mp)[PB], int cbase) {
  constexpr int NACC = T::NACC, RUN = NACC * CB;
  const __amdgpu_buffer_rsrc_t yr =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.y, (short)0, (int)(y_elems(a) * 2u), 0x00020000);
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const int m = mp[p];
    const unsigned off = (m >= 0) ? (unsigned)(y_pixel(a, m) * a.Cout + cbase) * 2u : kOobOffset;
#pragma unroll
    for (int c8 = 0; c8 < RUN; c8 += 8) {
      u32x4_t ov;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        ov[q] = pack2(acc[(c8 + 2 * q) / NACC][p][(c8 + 2 * q) % NACC],
                      acc[(c8 + 2 * q + 1) / NACC][p][(c8 + 2 * q + 1) % NACC]);
      __builtin_amdgcn_raw_buffer_store_b128(ov, yr, (int)(off + c8 * 2), 0, 0);
    }
  }
}

// Split-K partials in fragment order (halo kernel): the partial block of
// (split, m tile, n tile, wave, p, cb) holds a lane's 16 accumulator floats
// as four 1 KB rows (float4 q of lanes 0..63), so every store instruction
// writes 1 KB of consecutive bytes; stores straight into the [M][Cout]
// layout would scatter 16-byte pieces over 64 rows per instruction.
// reduce_frag_kernel reads the blocks back in the same order.
template <int PB, int CB>
__device__ __forceinline__ void store_partial_frag(const IgemmArgs& a, f32x16_t (&acc)[CB][PB],
                                                   const TileCoord& tc, int BM, int BN, int wave,
                                                   int lane) {
  const long long tile = tc.slot;
  f32x4_t* base = reinterpret_cast<f32x4_t*>(a.partial) + (tile * 4 + wave) * (PB * CB * 4 * 64) + lane;
#pragma unroll
  for (int p = 0; p < PB; ++p)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        base[((p * CB + cb) * 4 + q) * 64] =
            f32x4_t{acc[cb][p][4 * q], acc[cb][p][4 * q + 1], acc[cb][p][4 * q + 2], acc[cb][p][4 * q + 3]};
}

// ----------------------------------------------------------------------------
// Tile kernel: both operands staged through LDS, as in a GEMM.
//
// A pipeline stage covers KB consecutive live K steps. The stage's pixel tile
// (BM pixels x KB*64 contiguous bytes of one tap each) is loaded with
// coalesced 16-byte loads, a wave instruction covering 64/(4*KB) whole pixel
// segments: far fewer cache lines per instruction than gathering straight
// into the MFMA operand layout, whose 32 lanes each touch a different pixel.
// The tile is stored in LDS with an XOR swizzle of its 16-byte chunks and read
// back in the MFMA B-operand layout; the weight slices likewise.
//
// Pipeline: three LDS stages. Iteration i computes stage i, stores stage i+2
// (fetched into registers during iteration i-1) and fetches stage i+3; one
// barrier. Within a stage the operand fragments of sub-step j+1 (one K half
// of one K step) are read while the MFMAs of sub-step j run, and the last
// sub-step reads the first fragments of stage i+1, whose LDS slot was filled
// before the previous barrier: no LDS latency sits in front of the MFMAs.
// ----------------------------------------------------------------------------
template <int XQ>
__device__ __forceinline__ int xs_idx(int pixel, int chunk) {
  // XQ 16-byte chunks per pixel row; the swizzle keeps 8- and 16-lane groups
  // reading one chunk of consecutive pixels in distinct bank groups.
  if constexpr (XQ == 8) return pixel * 8 + (chunk ^ (((pixel >> 1) ^ (pixel << 2)) & 7));
  else return pixel * 4 + (chunk ^ (((pixel >> 1) ^ (pixel >> 3)) & 3));
}

template <class T, int WM, int WN, int PB, int CB, int KB, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void igemm_tile_kernel(IgemmArgs a) {
  constexpr int R = T::R, KS = T::KS, NACC = T::NACC;
  constexpr int NT = 64 * WM * WN;
  constexpr int BM = R * PB * WM;
  constexpr int BN = R * CB * WN;
  constexpr int XQ = 4 * KB;                   // 16-byte chunks per pixel per stage
  constexpr int XCH = BM * XQ;                 // pixel-tile chunks per stage
  constexpr int XPT = XCH / NT;                // ... per thread
  constexpr int WCH = BN * 4;                  // weight chunks per K step
  constexpr int WPT = (WCH + NT - 1) / NT;     // ... per thread
  constexpr int RUN = NACC * CB;
  constexpr int NSTG = 3;                      // LDS stages
  constexpr int J = KB * KS;                   // MFMA sub-steps per stage
  typedef typename T::acc_t acc_t;
  static_assert(RUN % 8 == 0, "each lane must hold whole 16-byte runs of channels");
  static_assert(XQ == 4 || XQ == 8, "stage of 1 or 2 K steps");
  static_assert(XCH % NT == 0 && NT % XQ == 0, "pixel tile evenly split over threads");

  __shared__ u32x4_t xs[NSTG][XCH];
  __shared__ u32x4_t ws[NSTG][KB][WCH];
  __shared__ float red[(EPI == EPI_NORM && WN > 1) ? WM * WN * PB * R : 1];
  __shared__ unsigned live_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave % WM;
  const int wave_n = wave / WM;
  const int lrow = T::row(lane);
  const int lgrp = T::grp(lane);
  const TileCoord tc = tile_coord(a, BM, BN);

  // This thread loads chunk xj of the pixels tid/XQ + i*(NT/XQ) of the tile;
  // chunk xj belongs to K step xj/4 of the stage, bytes 16*(xj%4).. of it.
  const int xj = tid % XQ;
  const int xk = xj >> 2;
  constexpr int XSTRIDE = NT / XQ;
  long long base[XPT];
  unsigned tapmask[XPT];
  unsigned live = 0;
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    long long b1[1];
    unsigned t1[1];
    live |= pixel_geometry<1, 1>(a, tc.m0 + tid / XQ + i * XSTRIDE, b1, t1);
    base[i] = b1[0] + (xj & 3) * 16;
    tapmask[i] = t1[0];
  }
  live = wave_or(live);
  if (tid == 0) live_sh = 0;
  __syncthreads();
  if (lane == 0) atomicOr(&live_sh, live);
  __syncthreads();
  live = __builtin_amdgcn_readfirstlane(live_sh);
  const __amdgpu_buffer_rsrc_t xrsrc = x_rsrc(a);
  const __amdgpu_buffer_rsrc_t wrsrc = w_rsrc(a);

  const int s_begin = tc.split * a.steps_per_split;
  const int s_end = min(s_begin + a.steps_per_split, 27 * a.CC);
  auto valid_step = [&](int t, int cc) -> int {
    return (t < 27 && t * a.CC + cc < s_end) ? ((t << 8) | cc) : kEnd;
  };
  auto next_step = [&](int e) -> int {
    if (e == kEnd) return kEnd;
    int t = e >> 8, cc = (e & 255) + 1;
    if (cc == a.CC) {
      cc = 0;
      const unsigned rest = live & (~0u << (t + 1));
      t = rest ? __builtin_ctz(rest) : 27;
    }
    return valid_step(t, cc);
  };
  auto first_step = [&]() -> int {
    if (s_begin >= s_end) return kEnd;
    int t = s_begin / a.CC, cc = s_begin % a.CC;
    if (!((live >> t) & 1u)) {
      const unsigned rest = live & (~0u << t);
      t = rest ? __builtin_ctz(rest) : 27;
      cc = 0;
    }
    return valid_step(t, cc);
  };
  auto next_group = [&](int prev, int (&g)[KB]) {
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      g[k] = next_step(prev);
      prev = g[k];
    }
  };

  acc_t acc[CB][PB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int p = 0; p < PB; ++p)
#pragma unroll
      for (int e = 0; e < NACC; ++e) acc[cb][p][e] = 0.f;

  auto lds_row_of = [&](int c) -> int {
    const int col = c >> 2;
    int cb, r;
    T::row_of(col % (R * CB), CB, cb, r);
    return ((col / (R * CB)) * CB + cb) * R + r;
  };
  unsigned woff[WPT];
  int wdst[WPT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int c = tid + i * NT;
    const bool ok = c < WCH && tc.co0 + (c >> 2) < a.Cout;
    woff[i] = ok ? (unsigned)((tc.co0 * 4 + c) * 16) : kOobOffset;
    wdst[i] = (c < WCH) ? lds_idx(lds_row_of(c), c & 3) : 0;
  }

  // Staging registers for the stage in flight. Loads are unconditional: a
  // step of kEnd reads zeros, so the compiler's wait counts stay exact.
  u32x4_t xst[XPT];
  u32x4_t wst[KB][WPT];
  auto load_stage = [&](const int (&g)[KB]) {
    const int e = g[xk];
    const bool valid = e != kEnd;
    const int t = valid ? e >> 8 : 0, cc = valid ? e & 255 : 0;
    const long long delta =
        (((long long)(t / 9) * a.H + (t / 3) % 3) * a.W + t % 3) * (long long)(a.Cin * 2) + cc * 64;
    const unsigned chan_ok = (unsigned)(valid && cc * 32 + (xj & 3) * 8 < a.Cin);
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const unsigned ok = chan_ok & (tapmask[i] >> t);
      const unsigned off = (unsigned)(base[i] + delta) | (((ok & 1u) - 1u) & kOobOffset);
      xst[i] = __builtin_amdgcn_raw_buffer_load_b128(xrsrc, (int)off, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int ek = g[k];
      const unsigned soff =
          (ek == kEnd) ? kOobOffset : (unsigned)((ek >> 8) * a.CC + (ek & 255)) * (unsigned)a.Cout * 64u;
#pragma unroll
      for (int i = 0; i < WPT; ++i)
        wst[k][i] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)(woff[i] + soff), 0, 0);
    }
  };
  auto store_stage = [&](int stg) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) xs[stg][xs_idx<XQ>(tid / XQ + i * XSTRIDE, xj)] = xst[i];
#pragma unroll
    for (int k = 0; k < KB; ++k)
#pragma unroll
      for (int i = 0; i < WPT; ++i)
        if (WCH % NT == 0 || tid + i * NT < WCH) ws[stg][k][wdst[i]] = wst[k][i];
  };
  // Fragments of sub-step jj (K step jj / KS, half jj % KS) of LDS slot stg.
  auto read_frags = [&](int stg, int jj, u32x4_t (&xf)[PB], u32x4_t (&wf)[CB]) {
    const int k = jj / KS, h = jj % KS;
    const int q = 4 * k + T::chunk(lane, h);
#pragma unroll
    for (int p = 0; p < PB; ++p) xf[p] = xs[stg][xs_idx<XQ>((wave_m * PB + p) * R + lrow, q)];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      wf[cb] = ws[stg][k][lds_idx((wave_n * CB + cb) * R + lrow, T::chunk(lane, h))];
  };

  // Stages of iterations i .. i+3.
  int g0[KB], g1[KB], g2[KB], g3[KB];
  g0[0] = first_step();
#pragma unroll
  for (int k = 1; k < KB; ++k) g0[k] = next_step(g0[k - 1]);
  next_group(g0[KB - 1], g1);
  next_group(g1[KB - 1], g2);

  u32x4_t xf[2][PB], wf[2][CB];
  load_stage(g0);
  store_stage(0);
  load_stage(g1);
  store_stage(1);
  load_stage(g2);
  __syncthreads();
  read_frags(0, 0, xf[0], wf[0]);

  auto iteration = [&](auto slot_c) -> bool {
    constexpr int slot = decltype(slot_c)::value;
    constexpr int nxt = (slot + 1) % NSTG, far = (slot + 2) % NSTG;
    if (g0[0] == kEnd) return false;
    next_group(g2[KB - 1], g3);
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      // Fragments of the next sub-step (the first of stage i+1 at the end).
      if (jj + 1 < J) read_frags(slot, jj + 1, xf[(jj + 1) & 1], wf[(jj + 1) & 1]);
      else read_frags(nxt, 0, xf[(jj + 1) & 1], wf[(jj + 1) & 1]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int p = 0; p < PB; ++p)
          acc[cb][p] = T::mma(__builtin_bit_cast(bf16x8_t, wf[jj & 1][cb]),
                              __builtin_bit_cast(bf16x8_t, xf[jj & 1][p]), acc[cb][p]);
    }
    store_stage(far);
    load_stage(g3);
    __syncthreads();
    // J is even, so sub-step 0 of the next stage is in fragment slot 0.
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      g0[k] = g1[k];
      g1[k] = g2[k];
      g2[k] = g3[k];
    }
    return true;
  };
  static_assert(J % 2 == 0, "fragment double buffer");
  for (;;) {
    if (!iteration(SlotC<0>{})) break;
    if (!iteration(SlotC<1>{})) break;
    if (!iteration(SlotC<2>{})) break;
  }
  int mp[PB];
  block_pixels<PB, R>(tc.m0 + wave_m * PB * R + lrow, a.M, mp);
  epilogue<T, WM, WN, PB, CB, EPI>(a, acc, mp, tc.co0 + wave_n * R * CB + lgrp * RUN, tc.split,
                                   wave_m, wave_n, lrow, lgrp, red);
}

// ----------------------------------------------------------------------------
// Halo kernel: stride 1 along W and Cin % 32 == 0.
//
// For one (kd, kh) tap pair and one 32-channel chunk, the three kw taps of an
// output pixel read three neighbouring input pixels of the same input row.
// A pipeline stage therefore stages, per row segment that the tile's BM
// output pixels cover, that segment's input pixels plus the two-pixel halo
// once, and the kw taps read it at slot offsets 0, 1, 2: a third of the
// activation traffic of staging every tap separately. A slot is one pixel's
// 64 bytes; its four 16-byte chunks are XOR-swizzled by (slot / 4) % 4, which
// puts any sixteen consecutive slots of one chunk in the sixteen 16-byte bank
// groups of a 256-byte window (one ds_read_b128 cycle serves 16 lanes; a
// fragment read's lanes take consecutive slots, two skipped at a row break).
//
// Both operands reach LDS by buffer-to-LDS DMA (no staging registers); a
// padding tap is an out-of-range lane, which writes zeros. Each wave computes
// 128 pixels x 32*CB channels with v_mfma_f32_32x32x16_bf16 (16 accumulator
// blocks for CB = 4). Three activation buffers and two weight buffers: while
// stage i is computed, the weights of stage i+1 (half of them from the last
// sub-step of stage i-1 on) and the activations of stage i+2 are fetched.
// Every DMA instruction and fragment read goes out on its own between single
// MFMAs. One barrier per stage, before the last sub-step, whose MFMAs then
// cover the first fragment reads of stage i+1.
// ----------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, void* lds, unsigned voff,
                                      unsigned soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds, 16, (int)voff, (int)soff, 0, 0);
}

template <int CB, int WN, int XJ>
struct HaloShape {
  static constexpr int R = 32, PB = 4, NT = 256;
  static constexpr int WM = 4 / WN;
  static constexpr int BM = R * PB * WM;       // output pixels per tile
  static constexpr int BN = R * CB * WN;       // output channels per tile
  static constexpr int XU = XJ * 4 * 64;       // 16-byte units per activation buffer
  static constexpr int XSLOTS = XU / 4;        // 64-byte slots
  static constexpr int WU = BN * 4;            // 16-byte units per tap
  static constexpr int WJ = (WU / 64 + 3) / 4; // weight DMA instructions per wave per tap
  static constexpr int WUP = WJ * 256;         // tap stride: every lane of every wave has a slot
  // Row segments a tile may span: slot of the last pixel + 2 < XSLOTS.
  static constexpr int MAXSEG = (XSLOTS - BM - 2) / 2 + 1;
  static_assert(WN == 1 || WN == 2 || WN == 4, "4 waves");
  static_assert(XJ >= 3 && XJ <= 12, "activation DMA issued in three parts of 1..4");
};

__device__ __forceinline__ int xslot_chunk(int slot, int chunk) {
  return chunk ^ ((slot >> 2) & 3);
}

template <int CB, int WN, int XJ, int EPI, bool REF = false>
__global__ __launch_bounds__(256) void igemm_halo_kernel(IgemmArgs a) {
  using T = Mfma32;
  using S = HaloShape<CB, WN, XJ>;
  constexpr int R = S::R, PB = S::PB, WM = S::WM, NACC = T::NACC, RUN = NACC * CB;
  constexpr int XU = S::XU, WU = S::WU, WJ = S::WJ, WUP = S::WUP;
  constexpr int WTAP = WUP * 16;  // bytes
  typedef typename T::acc_t acc_t;
  static_assert(RUN % 8 == 0, "each lane must hold whole 16-byte runs of channels");

  // One array per buffer, so the compiler can tell the DMA into one buffer
  // from the fragment reads of another.
  __shared__ u32x4_t xbuf0[XU], xbuf1[XU], xbuf2[XU];
  __shared__ u32x4_t wbuf0[3 * WUP], wbuf1[3 * WUP];
  __shared__ float red[(EPI == EPI_NORM && WN > 1) ? WM * WN * PB * R : 1];

  const int tid = threadIdx.x;
  const int lane0 = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % WM;
  const int wave_n = wave / WM;
  const int lrow = lane0 & 31;
  const int lgrp = lane0 >> 5;

  // Tiles: one per work-group, or (a.queue set) a persistent work-group per
  // CU taking tiles from its XCD's queue. Work-groups are dealt to the 8
  // XCDs round-robin; XCD x owns chunks x, x+8, ... of kQueueChunk
  // consecutive tiles, handed out in reverse tile order so that the short
  // tiles of a causal layer's first frames come last (longest first).
  __shared__ int tile_sh;
  const int T_all = a.m_tiles * a.n_tiles * a.splits;
  auto fetch_tile = [&]() -> int {
    if (tid == 0) tile_sh = queue_take(a.queue, T_all, a.queue_tail);
    __syncthreads();
    return tile_sh;
  };
  const int rows_total = a.N * a.Do * a.Ho;
  const float inv_wo = a.inv_wo, inv_wo2 = a.inv_wp, inv_ho = a.inv_ho, inv_do = a.inv_do;
  int tile_lin = a.queue ? fetch_tile() : 0;
  while (tile_lin >= 0) {
  // Recomputing the per-lane set-up each tile is cheaper than the registers
  // (and spills) of keeping it across tiles: hide the lane id's invariance.
  int lane = lane0;
  asm volatile("" : "+v"(lane));
  TileCoord tc;
  if (a.queue) {
    tc.m0 = (tile_lin % a.m_tiles) * S::BM;
    const int rest = tile_lin / a.m_tiles;
    tc.co0 = (rest % a.n_tiles) * S::BN;
    tc.split = rest / a.n_tiles;
    tc.nsplit = a.splits;
    tc.slot = (tc.split * a.m_tiles + tile_lin % a.m_tiles) * a.n_tiles + rest % a.n_tiles;
  } else if (a.vsplit) {
    tc = tile_coord_live(a, S::BM, S::BN);
  } else {
    tc = tile_coord(a, S::BM, S::BN);
  }

  // Row segments of the tile: the first starts at output column wo0 of row
  // row0 and holds len0 pixels; each later one is a whole output row. Slot
  // of segment k's input column i: i for k = 0, else len0 + 2 + (k-1)(Wo+2) + i.
  const int row0 = tc.m0 / a.Wo;
  const int wo0 = tc.m0 - row0 * a.Wo;
  const int len0 = min(a.Wo - wo0, S::BM);
  const int nseg = (min(tc.m0 + S::BM, a.M) - 1) / a.Wo - row0 + 1;

  // Lane k describes row segment k: the input pixel index of (n, d0, h0, 0)
  // and the 9-bit set of (kd, kh) pairs that fall inside the input.
  int rbase = 0;
  unsigned rmask = 0;
  {
    const int r = row0 + lane;
    if (r < rows_total) {
      const int t2 = small_div(r, a.Ho, inv_ho);
      const int ho = r - t2 * a.Ho;
      const int n = small_div(t2, a.Do, inv_do);
      const int dq = t2 - n * a.Do;
      const int d0 = dq * a.sd - a.pd;
      const int h0 = ho * a.sh - a.ph;
      rmask = row_mask<REF>(a, d0, h0);
      rbase = ((n * a.D + d0) * a.H + h0) * a.W;
    }
  }
  // Live (kd, kh) pairs of the tile: the same in every wave, no LDS needed.
  const unsigned live = __builtin_amdgcn_readfirstlane(wave_or(lane < nseg ? rmask : 0u)) & 511u;

  // Activation DMA entries of this lane: LDS unit q of a buffer holds chunk
  // xslot_chunk(q / 4, q % 4) of slot q / 4. xbase is that chunk's byte offset
  // in x at kd = kh = 0 and channel chunk 0; xmask the (kd, kh) pairs for
  // which the pixel lies inside the input.
  int xbase[XJ];
  unsigned xmask[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int q = (j * 4 + wave) * 64 + lane;
    const int sl = q >> 2;
    const int c = xslot_chunk(sl, q & 3);
    // Branch-free, so the lane shuffles below issue back to back.
    const int rel = sl - len0 - 2;
    const int kq = small_div(max(rel, 0), a.Wo + 2, inv_wo2);
    const bool first = rel < 0;
    const int k = first ? 0 : 1 + kq;
    const int i = first ? sl : rel - kq * (a.Wo + 2);
    const int w_in = (first ? wo0 : 0) - a.pw + i;
    const int kk = min(k, 63);
    const unsigned m = __shfl(rmask, kk);
    const int rb = __shfl(rbase, kk);
    const bool wok = REF ? (w_in >= -1 && w_in <= a.W) : (w_in >= 0 && w_in < a.W);
    const int wc = REF ? reflect_index(w_in, a.W) : w_in;
    xmask[j] = wok ? m : 0u;
    xbase[j] = wok ? (rb + wc) * (a.Cin * 2) + c * 16 : 0;
  }

  // Weight DMA entries: LDS unit q of a tap holds row q / 4 of the permuted
  // channel order, 16-byte chunk (q % 4) XOR the row swizzle.
  unsigned woff[WJ];
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int q = (j * 4 + wave) * 64 + lane;
    const int row = q >> 2;
    const int c = (q & 3) ^ (((row >> 1) ^ (row >> 3)) & 3);
    const int col = (row / (R * CB)) * (R * CB) + T::chan_of((row / R) % CB, row % R, CB);
    woff[j] = (q < WU) ? (unsigned)((tc.co0 + col) * 64 + c * 16) : kOobOffset;
  }

  // Fragment addresses (bytes within a buffer). Pixel block p of this wave,
  // tap kw: slot s = slot_p + kw, chunk lgrp for K half 0; K half 1 is chunk
  // lgrp + 2, i.e. the address XOR 32.
  int ax[PB][3];
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const int rel = wave_m * (PB * R) + p * R + lrow;
    const int k = rel < len0 ? 0 : 1 + small_div(rel - len0, a.Wo, inv_wo);
    const int slot = rel + 2 * k;
#pragma unroll
    for (int kw = 0; kw < 3; ++kw) ax[p][kw] = (slot + kw) * 64 + xslot_chunk(slot + kw, lgrp) * 16;
  }
  int aw[CB][2];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int h = 0; h < 2; ++h) aw[cb][h] = lds_idx((wave_n * CB + cb) * R + lrow, 2 * h + lgrp) * 16;

  const __amdgpu_buffer_rsrc_t xrsrc = x_rsrc(a);
  const __amdgpu_buffer_rsrc_t wrsrc = w_rsrc(a);

  // Stages e = (pair << 8) | cc over the live (kd, kh) pairs. A uniform
  // split takes a fixed range of nominal steps; a live-balanced one the
  // tile's live steps [split * q, split * q + q), q = ceil(live / nsplit).
  int s_begin, s_end;
  if (a.vsplit) {
    const int L = __builtin_popcount(live) * a.CC;
    const int q = (L + tc.nsplit - 1) / tc.nsplit;
    const int j0 = min(tc.split * q, L), j1 = min(j0 + q, L);
    s_begin = j0 < L ? live_step(live, j0, a.CC) : 9 * a.CC;
    s_end = j1 < L ? live_step(live, j1, a.CC) : 9 * a.CC;
  } else {
    s_begin = tc.split * a.steps_per_split;
    s_end = min(s_begin + a.steps_per_split, 9 * a.CC);
  }
  auto valid_stage = [&](int pr, int cc) -> int {
    return (pr < 9 && pr * a.CC + cc < s_end) ? ((pr << 8) | cc) : kEnd;
  };
  auto next_stage = [&](int e) -> int {
    if (e == kEnd) return kEnd;
    int pr = e >> 8, cc = (e & 255) + 1;
    if (cc == a.CC) {
      cc = 0;
      const unsigned rest = live & (~0u << (pr + 1));
      pr = rest ? __builtin_ctz(rest) : 9;
    }
    return valid_stage(pr, cc);
  };
  auto first_stage = [&]() -> int {
    if (s_begin >= s_end) return kEnd;
    int pr = s_begin / a.CC, cc = s_begin % a.CC;
    if (!((live >> pr) & 1u)) {
      const unsigned rest = live & (~0u << pr);
      pr = rest ? __builtin_ctz(rest) : 9;
      cc = 0;
    }
    return valid_stage(pr, cc);
  };

  auto xbuf = [&](auto b_c) -> u32x4_t* {
    constexpr int b = decltype(b_c)::value;
    return b == 0 ? xbuf0 : (b == 1 ? xbuf1 : xbuf2);
  };
  auto wbuf = [&](auto b_c) -> u32x4_t* {
    constexpr int b = decltype(b_c)::value;
    return b == 0 ? wbuf0 : wbuf1;
  };
  // One DMA instruction of a stage's fetch. The weights of a stage are
  // NW = 3 * WJ instructions per wave (tap kw = k / WJ, piece j = k % WJ),
  // then come the XJ activation instructions. Branch-free: the per-stage
  // scalars come from stage_dma(), and a stage past the end loads nothing
  // but out-of-range zeros into a buffer nobody reads.
  constexpr int NW = 3 * WJ;
  struct StageDma {
    unsigned wsoff[3];   // weight byte offset of each kw tap
    unsigned wor;        // 0, or kOobOffset past the last stage
    unsigned pbit;       // bit of the (kd, kh) pair, 0 past the last stage
    int delta;           // activation byte offset of the pair and chunk
    unsigned rbit;       // reflect padding: row flag whose rows move by radj
    int radj;
  };
  auto stage_dma = [&](int e) -> StageDma {
    StageDma d;
    const bool ok = e != kEnd;
    const int pr = ok ? e >> 8 : 0, cc = ok ? e & 255 : 0;
    const int kd = pr / 3, kh = pr - kd * 3;
#pragma unroll
    for (int kw = 0; kw < 3; ++kw)
      d.wsoff[kw] = (unsigned)(((kd * 9 + kh * 3 + kw) * a.CC + cc) * a.Cout) * 64u;
    d.wor = ok ? 0u : kOobOffset;
    d.pbit = ok ? 1u << pr : 0u;
    d.delta = (kd * a.H + kh) * a.W * (a.Cin * 2) + cc * 64;
    d.rbit = REF ? (kh == 0 ? 1u << 9 : (kh == 2 ? 1u << 10 : 0u)) : 0u;
    d.radj = REF ? (kh == 0 ? 2 : -2) * a.W * (a.Cin * 2) : 0;
    return d;
  };
  auto issue_w_one = [&](const StageDma& d, auto b_c, auto k_c) {
    constexpr int k = decltype(k_c)::value;
    constexpr int kw = k / WJ, j = k % WJ;
    dma16(wrsrc, &wbuf(b_c)[kw * WUP + (j * 4 + wave) * 64], woff[j] | d.wor, d.wsoff[kw]);
  };
  auto issue_x_one = [&](const StageDma& d, auto b_c, auto j_c) {
    constexpr int j = decltype(j_c)::value;
    const int radj = (REF && (xmask[j] & d.rbit)) ? d.radj : 0;
    const unsigned off = (xmask[j] & d.pbit) ? (unsigned)(xbase[j] + d.delta + radj) : kOobOffset;
    dma16(xrsrc, &xbuf(b_c)[(j * 4 + wave) * 64], off, 0u);
  };

  acc_t acc[CB][PB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int p = 0; p < PB; ++p)
#pragma unroll
      for (int e = 0; e < NACC; ++e) acc[cb][p][e] = 0.f;

  u32x4_t xf[2][PB], wf[2][CB];
  // Fragments of sub-step u (tap kw = u / 2, K half h = u % 2) into register
  // set u % 2: pixel block p, channel block cb.
  auto read_x = [&](auto xb_c, int u, int p) {
    const char* xb = reinterpret_cast<const char*>(xbuf(xb_c));
    const int kw = u >> 1;
    xf[u & 1][p] = *reinterpret_cast<const u32x4_t*>(xb + ((u & 1) ? (ax[p][kw] ^ 32) : ax[p][kw]));
  };
  auto read_w = [&](auto wb_c, int u, int cb) {
    const char* wb = reinterpret_cast<const char*>(wbuf(wb_c));
    wf[u & 1][cb] = *reinterpret_cast<const u32x4_t*>(wb + aw[cb][u & 1] + (u >> 1) * WTAP);
  };

  int e0 = first_stage();
  int e1 = next_stage(e0);
  int e2 = next_stage(e1);
  {
    const StageDma d0 = stage_dma(e0), d1 = stage_dma(e1);
    static_for<NW>([&](auto k) { issue_w_one(d0, SlotC<0>{}, k); });
    static_for<XJ>([&](auto j) { issue_x_one(d0, SlotC<0>{}, j); });
    static_for<XJ>([&](auto j) { issue_x_one(d1, SlotC<1>{}, j); });
  }
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(XJ) : "memory");
  static_for<PB>([&](auto p) { read_x(SlotC<0>{}, 0, decltype(p)::value); });
  static_for<CB>([&](auto cb) { read_w(SlotC<0>{}, 0, decltype(cb)::value); });

  // Stage i (activation buffer i % 3, weight buffer i % 2): six sub-steps u
  // of CB * PB MFMAs (channel block cb = g / PB, pixel block p = g % PB). With
  // one wave per SIMD a wave issues one instruction per four cycles, so the
  // memory operations go out one or two between single MFMAs rather than in
  // bunches the matrix core would wait behind. Each sub-step first issues its
  // share of the DMA, then the next sub-step's fragments (pixel blocks, then
  // the weights, in the order its MFMAs use them; during sub-step 4 within
  // its first three quarters, so they have landed by the barrier):
  //   - sub-steps 0-4: weight DMA instructions [NW5, NW) of stage i+1, then
  //     the activations of stage i+2;
  //   - barrier between sub-steps 4 and 5: stage i+1 has landed everywhere
  //     (only stage i+2's activations, the last XJ DMA instructions, may be
  //     in flight), and no wave reads stage i's buffers any more;
  //   - sub-step 5: weight DMA instructions [0, NW5) of stage i+2 into stage
  //     i's weight buffer, which the barrier has just freed, and stage i+1's
  //     first fragments.
  constexpr int NM = CB * PB, NR = PB + CB, NW5 = NW / 2, ND = NW - NW5 + XJ;
  StageDma dnext = stage_dma(e1);
  StageDma dcar = stage_dma(e2);   // descriptor of stage e2
  const unsigned cstep = (unsigned)a.Cout * 64u;   // weight bytes per chunk
  static_for<NW5>([&](auto k) { issue_w_one(dnext, SlotC<1>{}, k); });
  auto iteration = [&](auto i_c) -> bool {
    constexpr int I = decltype(i_c)::value;
    constexpr int XB = I % 3, WB = I % 2;
    if (e0 == kEnd) return false;
    // (The weight DMA of stage i+1 reuses the descriptor formed for its
    // activations one stage earlier.)
    const StageDma dw = dnext, dx = dcar;
    static_for<6>([&](auto u_c) {
      constexpr int u = decltype(u_c)::value;
      constexpr int D0 = u < 5 ? u * ND / 5 : 0, D1 = u < 5 ? (u + 1) * ND / 5 : NW5;
      constexpr int NOPS = D1 - D0 + NR;
      constexpr int SPAN = u == 4 ? NM * 3 / 4 : NM;
      if constexpr (u == 5) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(XJ) : "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
      static_for<NM>([&](auto g_c) {
        constexpr int g = decltype(g_c)::value;
        static_for<NOPS>([&](auto o_c) {
          constexpr int o = decltype(o_c)::value;
          if constexpr (o * SPAN / NOPS == g) {
            if constexpr (o < D1 - D0) {
              constexpr int d = D0 + o;
              if constexpr (u == 5) issue_w_one(dx, SlotC<WB>{}, SlotC<d>{});
              else if constexpr (d < NW - NW5) issue_w_one(dw, SlotC<(I + 1) % 2>{}, SlotC<NW5 + d>{});
              else issue_x_one(dx, SlotC<(I + 2) % 3>{}, SlotC<d - (NW - NW5)>{});
            } else {
              constexpr int r = o - (D1 - D0), un = (u + 1) % 6;
              if constexpr (u < 5) {
                if constexpr (r < PB) read_x(SlotC<XB>{}, un, r);
                else read_w(SlotC<WB>{}, un, r - PB);
              } else {
                if constexpr (r < PB) read_x(SlotC<(I + 1) % 3>{}, un, r);
                else read_w(SlotC<(I + 1) % 2>{}, un, r - PB);
              }
            }
          }
        });
        __builtin_amdgcn_sched_barrier(0);
        constexpr int cb = g / PB, p = g % PB;
        acc[cb][p] = T::mma(__builtin_bit_cast(bf16x8_t, wf[u & 1][cb]),
                            __builtin_bit_cast(bf16x8_t, xf[u & 1][p]), acc[cb][p]);
        __builtin_amdgcn_sched_barrier(0);
      });
    });
    dnext = dx;
    e0 = e1;
    e1 = e2;
    // The next stage and its descriptor: the next chunk of the same (kd, kh)
    // pair moves both offsets by one chunk (the common case, a few scalar
    // adds); a new pair forms them afresh.
    const int cc2 = (e2 & 255) + 1;
    if (e2 != kEnd && cc2 < a.CC && (e2 >> 8) * a.CC + cc2 < s_end) {
      ++e2;
#pragma unroll
      for (int kw = 0; kw < 3; ++kw) dcar.wsoff[kw] += cstep;
      dcar.delta += 64;
    } else {
      e2 = next_stage(e2);
      dcar = stage_dma(e2);
    }
    return true;
  };
  for (;;) {
    if (!iteration(SlotC<0>{})) break;
    if (!iteration(SlotC<1>{})) break;
    if (!iteration(SlotC<2>{})) break;
    if (!iteration(SlotC<3>{})) break;
    if (!iteration(SlotC<4>{})) break;
    if (!iteration(SlotC<5>{})) break;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int mp[PB];
  block_pixels<PB, R>(tc.m0 + wave_m * PB * R + lrow, a.M, mp);
  if (EPI == EPI_STORE && a.flags == 0) {
    store_plain<T, PB, CB>(a, acc, mp, tc.co0 + wave_n * R * CB + lgrp * RUN);
  } else if (EPI == EPI_PARTIAL) {
    store_partial_frag<PB, CB>(a, acc, tc, S::BM, S::BN, wave, lane0);
  } else {
    epilogue<T, WM, WN, PB, CB, EPI>(a, acc, mp,
                                     tc.co0 + wave_n * R * CB + lgrp * RUN, tc.split, wave_m, wave_n,
                                     lrow, lgrp, red);
  }
  if (!a.queue) break;
  // The barrier in fetch_tile also keeps the next tile's DMA away from
  // buffers a slower wave may still read.
  tile_lin = fetch_tile();
  }
}

// ----------------------------------------------------------------------------
// Slot kernel: stride 1 along W and Cin % 32 == 0.
//
// Output pixels are addressed through slots: output row r = (n, do, ho) owns
// WP = Wo + 2 consecutive slots, slot c < Wo of the row being output column c
// and the last two unused. A tile computes BM consecutive slots and stores
// the first BM - 2 (tiles start BM - 2 apart). For one (kd, kh) tap pair and
// one 32-channel chunk, a stage stages BM slots of input: staged slot j holds
// the input pixel of row r(s0 + j) at column c(s0 + j) - pw. Output slot s at
// tap kw then reads staged slot s - s0 + kw for every stored s, across row
// ends too (an unused slot's result is dropped), so the three kw taps are
// plain slot offsets; the two extra computed slots, whose taps would reach
// past the staged range, are never stored. Column n of a wave's pixel
// fragment f holds slot n*PB + f (the fragments interleave), so the operand
// of tap kw for pixel block p is fragment p + kw: PB + 2 fragment reads per
// K half serve all three taps, against 3*PB when every tap is read on its
// own. The two unused slots of a row cost 2 / (Wo + 2) of the MFMA work.
//
// LDS layout of an activation buffer, PB = 2^SH: staged slot s (64 bytes,
// four 16-byte chunks) sits at position s ^ m, m = bit SH of s | bit SH + 3 of
// s << 1, its chunks XORed with (s >> (SH + 1)) & 3. A fragment read's lanes
// step PB slots, so lane-row bits 0, 3 pick m and bits 1-2 the chunk XOR: any
// 8 consecutive lanes hit 8 distinct 16-byte bank groups of a 128-byte window
// and any 16 consecutive lanes 16 distinct groups of a 256-byte window (one
// ds_read_b128 cycle serves 16 lanes). The permutation stays inside aligned
// groups of 16 slots, the span of one DMA instruction.
//
// Each wave computes R*PB slots x R*CB channels with v_mfma_f32_32x32x16_bf16.
// Operands reach LDS by buffer-to-LDS DMA (a padding pixel is an
// out-of-range lane: zeros). Three activation and two weight buffers; one
// barrier per stage, after sub-step 3 of the six (K half h = u / 3, tap
// kw = u % 3). Stage i's activation DMA goes out during its sub-steps 0-3,
// two stages ahead; its weight DMA during sub-steps 4-5, right after the
// barrier frees the buffer, also two stages ahead. LDS fragment reads run
// one to two sub-steps ahead of their MFMAs, every load and DMA spread
// between single MFMAs.
//
// e4m3 operands (F8): a stage is a 64-channel chunk, which is 64 bytes of a
// pixel as a bf16 stage's 32 channels are, so staging, LDS layout and
// fragment addresses are the bf16 ones. One v_mfma_f32_32x32x64_f8f6f4 per
// (tap, channel block, pixel block) takes the whole chunk: lane group g
// supplies the bytes of chunks g and g + 2 (the bf16 K halves' fragments) of
// both operands, so three sub-steps (s = kw) of CB*PB MFMAs, each as long as
// two bf16 ones. Memory operations of sub-step s of stage i:
//   s0: weight reads for taps 1 and 2, pixel fragments PB and PB+1 (the last
//       reads of stage i's buffers), the activation DMA of stage i+2;
//   s1: barrier (stage i+1 landed, stage i's buffers free), then stage
//       i+1's tap-0 weights and fragments 0 and 1 (fragment 1 once the MFMAs
//       reading its register have issued), half the weight DMA of stage i+2;
//   s2: stage i+1's fragments 2 .. PB-1, fragment f after the MFMAs of pixel
//       block f-2 (its register's last reader), the rest of the weight DMA.
// ----------------------------------------------------------------------------
// EPI_NORM epilogue of the slot kernel (the work-group holds its pixels'
// whole channel rows, BN == Cout). The arithmetic is the generic epilogue's,
// with these differences in how it is carried out:
//   - the tile's bias and gamma are staged once in LDS (sbuf: an activation
//     buffer no wave reads during the epilogue), so the lanes read them
//     without global-memory latency;
//   - the residual reads of pixel block p+1 are in flight while block p is
//     processed (for a pixel past the tile, pixel 0's row is read and its
//     values are never stored);
//   - values move as packed bf16 pairs: one conversion per two values, and
//     each pair's squares added to the row sum by one v_dot2_f32_bf16.
// HB / HR: bias / residual present (the caller dispatches on the flags).
template <class T, int WM, int WN, int PB, int CB, bool HB, bool HR>
__device__ __forceinline__ void epilogue_norm_slot(const IgemmArgs& a,
                                                   typename T::acc_t (&acc)[CB][PB],
                                                   const int (&mp)[PB], int co0, int cbase,
                                                   int wave_m, int wave_n, int lrow, int lgrp,
                                                   float* red, u32x4_t* sbuf) {
  constexpr int R = T::R, NACC = T::NACC, RUN = NACC * CB, NQ = RUN / 8;
  constexpr int BN = R * CB * WN, NT = 64 * WM * WN;
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  float* sb = reinterpret_cast<float*>(sbuf);            // [BN] bias
  uint16_t* sg = reinterpret_cast<uint16_t*>(sb + BN);   // [BN] gamma
  // Bias and gamma are read into registers before block 0's residual reads
  // are issued, so waiting for them leaves the residual reads in flight; the
  // barriers here wait for LDS operations only.
  constexpr int NS = (BN + NT - 1) / NT;
  float bv[NS];
  uint16_t gv[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i < BN) {
      if (HB) bv[k] = a.bias[co0 + i];
      gv[k] = a.gamma[co0 + i];
    }
  }
  const bool out_res = a.flags & F_RESIDUAL_OUT;
  u32x4_t rv[2][NQ];
  auto load_res = [&](int p, u32x4_t (&d)[NQ]) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        a.residual + (long long)(mp[p] >= 0 ? mp[p] : 0) * a.Cout + cbase);
#pragma unroll
    for (int q = 0; q < NQ; ++q) d[q] = src[q];
  };
  if (HR) load_res(0, rv[0]);
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i < BN) {
      if (HB) sb[i] = bv[k];
      sg[i] = gv[k];
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // staged bias and gamma visible
  const float* lb = sb + (cbase - co0);
  const u32x4_t* lg = reinterpret_cast<const u32x4_t*>(sg + (cbase - co0));
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    if (HR && p + 1 < PB) load_res(p + 1, rv[(p + 1) & 1]);
    const int m = mp[p];
    const bool ok = m >= 0;
    const long long off = (long long)(ok ? m : 0) * a.Cout + cbase;
    const long long yoff = (long long)y_pixel(a, ok ? m : 0) * a.Cout + cbase;
    unsigned vpk[RUN / 2];
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      f32x4_t b[2];
      if (HB) {
        b[0] = *reinterpret_cast<const f32x4_t*>(lb + 8 * q);
        b[1] = *reinterpret_cast<const f32x4_t*>(lb + 8 * q + 4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 8 * q + 2 * j;
        unsigned pk = pack2(acc[c / NACC][p][c % NACC], acc[(c + 1) / NACC][p][(c + 1) % NACC]);
        if (HB) pk = pack2(bf_lo(pk) + b[j >> 1][2 * (j & 1)], bf_hi(pk) + b[j >> 1][2 * (j & 1) + 1]);
        if (HR) {
          const unsigned r = rv[p & 1][q][j];
          pk = pack2(bf_lo(pk) + bf_lo(r), bf_hi(pk) + bf_hi(r));
        }
        vpk[c / 2] = pk;
        const bf16x2_t h = __builtin_bit_cast(bf16x2_t, pk);
        t = __builtin_amdgcn_fdot2_f32_bf16(h, h, t, false);
      }
      if (out_res && ok)
        *reinterpret_cast<u32x4_t*>(a.residual_out + off + 8 * q) =
            u32x4_t{vpk[4 * q], vpk[4 * q + 1], vpk[4 * q + 2], vpk[4 * q + 3]};
    }
#pragma unroll
    for (int o = R; o < 64; o <<= 1) t += __shfl_xor(t, o);  // lanes of the same pixel
    if (WN > 1) {  // ... and the WN waves (a slot per pixel block: no reuse)
      if (lgrp == 0) red[((wave_n * WM + wave_m) * PB + p) * R + lrow] = t;
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      t = 0.f;
      for (int wn = 0; wn < WN; ++wn) t += red[((wn * WM + wave_m) * PB + p) * R + lrow];
    }
    const float rden = 1.0f / fmaxf(sqrtf(t), 1e-12f);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const u32x4_t gv = lg[q];
      u32x4_t ov;
#pragma unroll
      for (int j = 0; j < 4; ++j) ov[j] = norm_silu_pair(vpk[4 * q + j], gv[j], rden, a.sqrt_c);
      if (ok) *reinterpret_cast<u32x4_t*>(a.y + yoff + 8 * q) = ov;
    }
  }
}

// ----------------------------------------------------------------------------
// Store of a 512-slot x 128-channel slot tile through LDS. The plain store's
// instructions each write 16-byte pieces of 32 pixels PB slots apart, which
// the store path absorbs about three times more slowly than whole lines. Here
// the tile goes out in PB/2 rounds: every lane writes the bf16 values of its
// pixel blocks 2*rho and 2*rho+1 into a [slot][128 channels] block of an idle
// activation buffer (16-byte unit u of row r at u ^ ((r >> 1) & 15), so
// consecutive lanes hit distinct banks); after a barrier the 256 threads read
// the block in row order and store it, 16 threads to a pixel's 256 bytes, so
// one instruction writes two pairs of adjacent pixels. Each wave issues
// PB * 4 stores, as the plain store does (dropped slots get out-of-range
// offsets), which the caller's wait counts rely on. Barriers wait for LDS
// operations only; the stores stay in flight.
//
// STATS (GroupNorm statistics of the stored values): as each lane packs its
// values for the LDS block it also adds them, and their squares, in fp32
// (v_dot2_f32_bf16 on the packed pairs) per 4-channel subgroup and per frame
// (the tile's stored slots span at most two frames; output rows from rnext
// on are the second); slots that are not stored add zeros. After the last
// round the lanes' sums go through LDS and threads 0-127 each add one
// (frame, subgroup, sum / sum of squares) over the 64 pixel lanes (wave_m,
// then lane row, ascending) and write the tile's 128 floats to gnp:
// [frame 0/1][subgroup 0-31 of the 128 channels][sum, sum of squares].
// A tile whose stored slots all precede row rnext (all but about one per
// frame) keeps one frame's sums only.
template <int PB, bool STATS = false>
__device__ __forceinline__ void store_staged(const IgemmArgs& a, const f32x16_t (&acc)[2][PB],
                                             u32x4_t* sbuf, int m0, int m_end, int WP,
                                             float inv_wp, int co0, int wave_m, int wave_n,
                                             int lrow, int lgrp, const int* mp = nullptr,
                                             float* gnp = nullptr, int rnext = 0) {
  constexpr int RBU = 16;                 // 16-byte units per slot row
  constexpr int UNITS = 32 * 2 * 2 * RBU; // per round: 64 lane rows x 2 pixel blocks
  constexpr int WM = 2;
  static_assert(PB % 2 == 0 && UNITS % 256 == 0, "rounds of two pixel blocks");
  const __amdgpu_buffer_rsrc_t yr =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.y, (short)0, (int)((unsigned)a.M * (unsigned)a.Cout * 2u),
                                        0x00020000);
  // (The thread index passes through an empty asm so that the addresses
  // formed from it are computed here, not hoisted to the kernel's start and
  // kept in registers through the main loop.)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  // (uniform: the output row of the tile's last stored slot)
  const int rpx = rnext * a.Wo;
  const bool two = STATS && small_div(min(m0 + PB * 64 - 2, m_end) - 1, WP, inv_wp) >= rnext;
  auto rounds = [&](auto two_c) {
    constexpr bool TWO = decltype(two_c)::value;
    // [frame][lane subgroup 0-7][sum, sum of squares]
    float st[TWO ? 2 : 1][8][2];
    if constexpr (STATS) {
#pragma unroll
      for (int f = 0; f < (TWO ? 2 : 1); ++f)
#pragma unroll
        for (int g = 0; g < 8; ++g) st[f][g][0] = st[f][g][1] = 0.f;
    }
    static_for<PB / 2>([&](auto rc) {
      constexpr int rho = decltype(rc)::value;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = (wave_m * 32 + lrow) * 2 + j;
        const int sw = (r >> 1) & 15;
        bool ok = false, f1 = false;
        if constexpr (STATS) {
          ok = mp[2 * rho + j] >= 0;
          f1 = TWO && mp[2 * rho + j] >= rpx;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          u32x4_t ov;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = 8 * k + 2 * q;   // lane channel 0 .. 31: acc[c / 16][p][c % 16]
            ov[q] = pack2(acc[c / 16][2 * rho + j][c % 16], acc[(c + 1) / 16][2 * rho + j][(c + 1) % 16]);
          }
          sbuf[r * RBU + ((wave_n * 8 + lgrp * 4 + k) ^ sw)] = ov;
          if constexpr (STATS) {
            const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int g = 2 * k + (q >> 1);
              if constexpr (TWO) {
                const bf16x2_t x0 = __builtin_bit_cast(bf16x2_t, (ok && !f1) ? ov[q] : 0u);
                const bf16x2_t x1 = __builtin_bit_cast(bf16x2_t, (ok && f1) ? ov[q] : 0u);
                st[0][g][0] = __builtin_amdgcn_fdot2_f32_bf16(x0, one, st[0][g][0], false);
                st[0][g][1] = __builtin_amdgcn_fdot2_f32_bf16(x0, x0, st[0][g][1], false);
                st[TWO ? 1 : 0][g][0] = __builtin_amdgcn_fdot2_f32_bf16(x1, one, st[TWO ? 1 : 0][g][0], false);
                st[TWO ? 1 : 0][g][1] = __builtin_amdgcn_fdot2_f32_bf16(x1, x1, st[TWO ? 1 : 0][g][1], false);
              } else {
                const bf16x2_t x = __builtin_bit_cast(bf16x2_t, ok ? ov[q] : 0u);
                st[0][g][0] = __builtin_amdgcn_fdot2_f32_bf16(x, one, st[0][g][0], false);
                st[0][g][1] = __builtin_amdgcn_fdot2_f32_bf16(x, x, st[0][g][1], false);
              }
            }
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int i = 0; i < UNITS / 256; ++i) {
        const int q = i * 256 + tid;
        const int r = q >> 4, pos = q & 15;
        const u32x4_t v = sbuf[r * RBU + (pos ^ ((r >> 1) & 15))];
        const int s = m0 + (r >> 1) * PB + 2 * rho + (r & 1);
        const int row = small_div(s, WP, inv_wp);
        const int col = s - row * WP;
        const bool ok = s < m_end && col < a.Wo;
        const unsigned off =
            ok ? (unsigned)((row * a.Wo + col) * a.Cout + co0 + pos * 8) * 2u : kOobOffset;
        __builtin_amdgcn_raw_buffer_store_b128(v, yr, (int)off, 0, 0);
      }
      // every wave has read this round's block before the next one overwrites it
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    });
    if constexpr (STATS) {
      // Lane sums at floats NV*tid ..; thread t < 128 adds output float t:
      // frame t / 64, subgroup sg = (t / 2) % 32 (wave column sg / 16, lane
      // group (sg / 8) % 2, lane subgroup sg % 8), sum or square sum t % 2.
      constexpr int NV = TWO ? 32 : 16;
      float* red = reinterpret_cast<float*>(sbuf);
#pragma unroll
      for (int i = 0; i < NV; ++i) red[tid * NV + i] = st[TWO ? (i >> 4) : 0][(i >> 1) & 7][i & 1];
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (tid < 128) {
        const int fr = tid >> 6, sg = (tid >> 1) & 31;
        const int i = (((sg & 7) << 1) | (tid & 1)) + 16 * fr;
        const int lane0 = (((sg >> 4) * WM) * 64 + ((sg >> 3) & 1) * 32) * NV + i;
        float sum = 0.f;
        if (TWO || fr == 0) {
          for (int wm = 0; wm < WM; ++wm)
            for (int lr = 0; lr < 32; ++lr) sum += red[lane0 + (wm * 64 + lr) * NV];
        }
        gnp[tid] = sum;
      }
    }
  };
  if (two) rounds(std::integral_constant<bool, true>{});
  else rounds(std::integral_constant<bool, false>{});
}

// The same for tiles whose waves each hold all BN = 32*CB channels of 32*PB
// consecutive slots (one wave across the channels, CB <= 4): round rho is
// wave rho's block, written by that wave alone as rows of 16 units (CB*4 of
// them used; unit u of row r at u ^ ((r / PB) & 15), so 16 consecutive lanes
// hit distinct banks) and stored by all 256 threads in row order, i.e.
// 32*PB consecutive slots of whole pixels. Each wave issues PB * CB * 2
// stores, as the plain store does.
template <int PB, int CB>
__device__ __forceinline__ void store_staged_rows(const IgemmArgs& a, const f32x16_t (&acc)[CB][PB],
                                                  u32x4_t* sbuf, int m0, int m_end, int WP,
                                                  float inv_wp, int co0, int wave, int lrow,
                                                  int lgrp) {
  constexpr int ROWS = 32 * PB, USED = CB * 4;   // 16-byte units used per row
  constexpr int UNITS = ROWS * USED;
  static_assert(USED <= 16 && UNITS % 256 == 0, "rows of at most 16 units");
  const __amdgpu_buffer_rsrc_t yr =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.y, (short)0, (int)((unsigned)a.M * (unsigned)a.Cout * 2u),
                                        0x00020000);
  int tid = threadIdx.x;   // (kept from being hoisted, as in store_staged)
  asm volatile("" : "+v"(tid));
  static_for<4>([&](auto rc) {
    constexpr int rho = decltype(rc)::value;
    if (wave == rho) {
#pragma unroll
      for (int p = 0; p < PB; ++p) {
        const int r = lrow * PB + p;
#pragma unroll
        for (int k = 0; k < 2 * CB; ++k) {
          u32x4_t ov;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = 8 * k + 2 * q;   // lane channel 0 .. 16*CB-1: acc[c / 16][p][c % 16]
            ov[q] = pack2(acc[c / 16][p][c % 16], acc[(c + 1) / 16][p][(c + 1) % 16]);
          }
          sbuf[r * 16 + ((lgrp * 2 * CB + k) ^ (lrow & 15))] = ov;
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int i = 0; i < UNITS / 256; ++i) {
      const int q = i * 256 + tid;
      const int r = q / USED, pos = q - r * USED;
      const u32x4_t v = sbuf[r * 16 + (pos ^ ((r / PB) & 15))];
      const int s = m0 + rho * ROWS + r;
      const int row = small_div(s, WP, inv_wp);
      const int col = s - row * WP;
      const unsigned off = (s < m_end && col < a.Wo)
                               ? (unsigned)((row * a.Wo + col) * a.Cout + co0 + pos * 8) * 2u
                               : kOobOffset;
      __builtin_amdgcn_raw_buffer_store_b128(v, yr, (int)off, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  });
}

// MFMA slot before which read o of e4m3 sub-step s goes out: evenly spread,
// but no earlier than the last MFMA reading the register it overwrites.
constexpr int f8_read_slot(int s, int o, int nrd, int nm, int cb) {
  const int g = o * nm / nrd;
  const int lo = s == 1 ? (o >= 2 * cb + 2 ? cb : 0) : (s == 2 ? (o / 2 + 1) * cb : 0);
  return g > lo ? g : lo;
}

template <int PB, int CB, int WN, int KW = 3>
struct SlotShape {
  static constexpr int R = 32;
  static constexpr int WM = 4 / WN;
  static constexpr int BM = R * PB * WM;            // slots computed per tile
  static constexpr int TS = BM - (KW - 1);          // slots stored per tile (tile stride)
  static constexpr int BN = R * CB * WN;            // output channels per tile
  static constexpr int XS = BM;                     // slots staged per stage
  static constexpr int XJ = (XS * 4 + 255) / 256;   // activation DMA instructions per wave
  static constexpr int XU = XJ * 256;               // 16-byte units per activation buffer
  static constexpr int NF = PB + KW - 1;            // pixel fragments per K half
  static constexpr int WU = BN * 4;                 // weight units per tap
  static constexpr int WJ = (WU / 64 + 3) / 4;      // weight DMA instructions per wave per tap
  static constexpr int WUP = WJ * 256;
  static constexpr int NW = KW * WJ;                // weight DMA instructions per wave per stage
  static_assert(PB == 3 || PB == 4 || PB == 8, "slot swizzle");
  static_assert(WN == 1 || WN == 2 || WN == 4, "4 waves");
  static_assert(XU % 64 == 0, "the slot permutation works on 16-slot groups");
};

// LDS 16-byte unit of (staged slot s, chunk c), and the inverse: the slot
// and chunk an LDS unit holds. PB = 3: slot s stays at position s, its chunks
// XORed by (s / 6) & 3 (slots 3 apart then alternate in parity and step the
// XOR every other lane).
template <int PB>
__device__ __forceinline__ int slot_unit(int s, int c) {
  if constexpr (PB == 3) {
    return (s << 2) | (c ^ ((s / 6) & 3));
  } else {
    constexpr int SH = PB == 4 ? 2 : 3;
    const int m = ((s >> SH) & 1) | (((s >> (SH + 3)) & 1) << 1);
    return ((s ^ m) << 2) | (c ^ ((s >> (SH + 1)) & 3));
  }
}
template <int PB>
__device__ __forceinline__ void unit_slot(int q, int& sl, int& c) {
  const int sp = q >> 2;
  if constexpr (PB == 3) {
    sl = sp;
    c = (q & 3) ^ ((sl / 6) & 3);
  } else {
    constexpr int SH = PB == 4 ? 2 : 3;
    // m depends on slot bits SH and SH + 3 only, which the XOR leaves alone
    sl = sp ^ (((sp >> SH) & 1) | (((sp >> (SH + 3)) & 1) << 1));
    c = (q & 3) ^ ((sl >> (SH + 1)) & 3);
  }
}

template <int PB, int CB, int WN, int EPI, bool REF = false, bool F8 = false, int KW = 3>
__global__ __launch_bounds__(256) void igemm_slot_kernel(IgemmArgs a) {
  using T = Mfma32;
  constexpr int ESZ = F8 ? 1 : 2;       // bytes per activation element
  using S = SlotShape<PB, CB, WN, KW>;
  static_assert(KW == 3 || (KW == 2 && !F8 && !REF), "two-tap pairs: bf16, zero padding");
  constexpr int R = S::R, WM = S::WM, NACC = T::NACC, RUN = NACC * CB;
  constexpr int XU = S::XU, XJ = S::XJ, NF = S::NF, WU = S::WU, WJ = S::WJ, WUP = S::WUP;
  constexpr int NW = S::NW;
  // Weight DMA instructions of a tile's second stage (two-tap pairs: an
  // odd-pixel chunk, whose pair tap 1 is not loaded).
  constexpr int NW1 = KW == 2 ? WJ : NW;
  constexpr int WTAP = WUP * 16;        // bytes
  constexpr int EPI_VM = PB * RUN / 8;  // stores of the plain epilogue per wave
  // tiles whose plain epilogue is a staged store (store_staged, store_staged_rows)
  constexpr bool STAGED = (PB == 8 && CB == 2 && WN == 2) || (PB == 4 && CB <= 4 && WN == 1);
  typedef typename T::acc_t acc_t;
  static_assert(RUN % 8 == 0, "each lane must hold whole 16-byte runs of channels");
  static_assert(EPI != EPI_NORM || WM * WN * PB * R * 4 <= 2048, "norm exchange area");
  static_assert(EPI != EPI_NORM || 6 * R * CB * WN <= XU * 16, "norm bias / gamma staging");
  static_assert(NW + XJ + EPI_VM <= 63, "vmcnt range");
  static_assert(!(F8 && REF), "e4m3 operands take zero padding only");
  static_assert(!(PB == 8 && CB == 2 && WN == 2) || XU >= 2048, "staged store block");
  static_assert(!(PB == 4 && CB <= 4 && WN == 1) || XU >= 32 * PB * 16, "staged store rows");
  static_assert(!(PB == 4 && CB <= 4 && WN == 1) || EPI_VM == PB * CB * 2, "store count");

  __shared__ u32x4_t xbuf0[XU], xbuf1[XU], xbuf2[XU];
  __shared__ u32x4_t wbuf0[KW * WUP], wbuf1[KW * WUP];
  // Fused norm: per-pixel sums of squares of the WN waves sharing a pixel.
  __shared__ float red[(EPI == EPI_NORM && WN > 1) ? WM * WN * PB * R : 1];
  // Stage table of the current tile (see start_tile).
  __shared__ u32x4_t stab[kSlotMaxStages];
  // GroupNorm statistics: the partials' address, the tile count and the
  // frame height, read back at each tile's end.
  __shared__ unsigned long long epi_sh[EPI == EPI_STATS ? 2 : 1];

  const int tid = threadIdx.x;
  const int lane0 = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % WM;
  const int wave_n = wave / WM;
  const int lrow = lane0 & 31;
  const int lgrp = lane0 >> 5;
  if (EPI == EPI_STATS && tid == 0) {   // (visible after the first barrier)
    epi_sh[0] = (unsigned long long)a.gnp;
    epi_sh[EPI == EPI_STATS ? 1 : 0] =
        (unsigned)a.n_tiles | ((unsigned long long)(unsigned)a.Ho << 32);
  }

  // Tiles: one per work-group, or (a.queue set) a persistent work-group per
  // CU taking tiles from its XCD's queue, as in the halo kernel. The ticket
  // of the next tile is taken when a tile starts, so its latency is hidden.
  __shared__ int tile_sh;
  const int T_all = a.m_tiles * a.n_tiles * a.splits;
  auto take_ticket = [&]() -> int { return queue_take(a.queue, T_all, a.queue_tail); };
  auto ticket_tile = [&](int t) -> int { return t; };
  const int rows_total = a.N * a.Do * a.Ho;
  const int WP = a.Wo + KW - 1;
  const float inv_wp = a.inv_wp, inv_ho = a.inv_ho, inv_do = a.inv_do;

  // Fragment addresses (bytes within a buffer): pixel fragment f of K half 0
  // is staged slot wave_m*R*PB + lrow*PB + f, chunk lgrp; K half 1 is chunk
  // lgrp + 2, i.e. the address XOR 32.
  int ax[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)  // (slots past the staged range feed unstored outputs only)
    ax[f] = slot_unit<PB>(min(wave_m * (PB * R) + lrow * PB + f, S::XS - 1), lgrp) * 16;
  int aw[CB][2];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int h = 0; h < 2; ++h) aw[cb][h] = lds_idx((wave_n * CB + cb) * R + lrow, 2 * h + lgrp) * 16;

  const __amdgpu_buffer_rsrc_t xrsrc = x_rsrc(a);
  // (two-tap pairs: a.CC counts the chunks of a pixel pair, twice the layer's)
  const __amdgpu_buffer_rsrc_t wrsrc =
      KW == 2 ? __builtin_amdgcn_make_buffer_rsrc((void*)a.wp, (short)0,
                                                  (int)(27u * (a.CC >> 1) * a.Cout * 64u), 0x00020000)
              : w_rsrc(a);

  // State of the current tile.
  TileCoord tc;
  unsigned live = 0;
  int krot = 0;   // kd of the first stage (frame order)
  int xbase[XJ];
  unsigned xmask[XJ];
  unsigned woff[WJ];
  int s_begin = 0, s_end = 0;
  int si = 0, nst = 0;   // index of the current stage in the tile, stages of the tile

  auto xbuf = [&](auto b_c) -> u32x4_t* {
    constexpr int b = decltype(b_c)::value;
    return b == 0 ? xbuf0 : (b == 1 ? xbuf1 : xbuf2);
  };
  auto wbuf = [&](auto b_c) -> u32x4_t* {
    constexpr int b = decltype(b_c)::value;
    return b == 0 ? wbuf0 : wbuf1;
  };
  struct StageDma {
    unsigned wsoff[KW];  // weight byte offset of each kw tap
    unsigned wtap[KW];   // 0, or kOobOffset for a tap without weights (two-tap pairs)
    unsigned wor;        // 0, or kOobOffset past the last stage
    unsigned pbit;       // bit of the (kd, kh) pair, 0 past the last stage
    int delta;           // activation byte offset of the pair and chunk
    unsigned rbit;       // reflect padding: row flag whose rows move by radj
    int radj;
  };
  // Stage j of a tile is the j-th live (pair, chunk) step of [s_begin,
  // s_end): pairs in stage order q (bit q of live), then chunks cc. Its
  // table entry (formed per lane at tile set-up): the weight byte offset of
  // (pair) tap 0; the activation byte offset; the pair's bit in the
  // original (kd, kh) order (bits 0-8), the reflect row flags (bits 9-10)
  // and, for two-tap pairs, the odd-pixel flag (bit 11); the reflect row
  // adjustment. Two-tap pairs: the input is viewed as pixel pairs of
  // 2 * Cin channels (chunks [0, CC / 2) the even pixel, the rest the odd
  // one); stage cc takes chunk cc / 2 of pixel cc % 2, so even and odd
  // pixels alternate. Pair tap kw' of a chunk of pixel e is the layer's tap
  // 2 * kw' + e; tap 3 does not exist and reads zeros.
  auto stage_entry = [&](int q, int cc) -> u32x4_t {
    const int kq = (q >= 3) + (q >= 6), kh = q - kq * 3;
    const int kd = kq + krot >= 3 ? kq + krot - 3 : kq + krot;
    const int pr = kd * 3 + kh;
    unsigned w0, odd = 0;
    int ch;
    if constexpr (KW == 2) {
      const int cco = a.CC >> 1, k = cc >> 1;
      odd = (unsigned)(cc & 1);
      w0 = (unsigned)(((pr * 3 + (int)odd) * cco + k) * a.Cout) * 64u;
      ch = (int)odd * cco + k;
    } else {
      w0 = (unsigned)((pr * 3 * a.CC + cc) * a.Cout) * 64u;
      ch = cc;
    }
    u32x4_t e;
    e[0] = w0;
    e[1] = (unsigned)((kd * a.H + kh) * a.W * (a.Cin * ESZ) + ch * 64);
    e[2] = (1u << pr) | (REF ? (kh == 0 ? 1u << 9 : (kh == 2 ? 1u << 10 : 0u)) : 0u) | (odd << 11);
    e[3] = REF ? (unsigned)((kh == 0 ? 2 : -2) * a.W * (a.Cin * ESZ)) : 0u;
    return e;
  };
  // The DMA descriptor of a (uniform) table entry; past the tile's last
  // stage (ok false) every load is out of range.
  const unsigned kws = (unsigned)((KW == 2 ? (a.CC >> 1) : a.CC) * a.Cout) * 64u;  // bytes per tap
  auto stage_decode = [&](unsigned w0, unsigned w1, unsigned w2, unsigned w3, bool ok) -> StageDma {
    StageDma d;
    if constexpr (KW == 2) {
      const unsigned odd = (w2 >> 11) & 1u;
      d.wsoff[0] = ok ? w0 : 0u;
      d.wsoff[1] = ok ? w0 + (2u - odd) * kws : 0u;
      d.wtap[0] = 0u;
      d.wtap[1] = odd ? kOobOffset : 0u;
    } else {
#pragma unroll
      for (int kw = 0; kw < KW; ++kw) {
        d.wsoff[kw] = ok ? w0 + (unsigned)kw * kws : 0u;
        d.wtap[kw] = 0u;
      }
    }
    d.wor = ok ? 0u : kOobOffset;
    d.pbit = ok ? (w2 & 511u) : 0u;
    d.delta = ok ? (int)w1 : 0;
    d.rbit = REF ? (w2 & (3u << 9)) : 0u;
    d.radj = REF ? (int)w3 : 0;
    return d;
  };
  // Table entry of stage si + 2 (uniform; decoded into scalar registers
  // where a stage starts).
  u32x4_t tnext;
  auto decode_uniform = [&](const u32x4_t& t, bool ok) -> StageDma {
    return stage_decode((unsigned)__builtin_amdgcn_readfirstlane((int)t[0]),
                        (unsigned)__builtin_amdgcn_readfirstlane((int)t[1]),
                        (unsigned)__builtin_amdgcn_readfirstlane((int)t[2]),
                        (unsigned)__builtin_amdgcn_readfirstlane((int)t[3]), ok);
  };
  // LDS destination of a DMA piece: the buffer's address plus a constant
  // plus this wave's 1 KB slice. The slice offset passes through an empty asm
  // at each use, so the compiler forms every destination with one scalar add
  // instead of keeping dozens of them in registers through the main loop.
  const unsigned wave_lds = (unsigned)wave * 1024u;
  auto lds_dst = [&](const void* buf, unsigned cst) -> void* {
    unsigned w = wave_lds;
    asm volatile("" : "+s"(w));
    return (void*)((const char*)buf + cst + w);
  };
  // Weight DMA instruction k of a stage (tap kw = k / WJ, piece k % WJ).
  auto issue_w_one = [&](const StageDma& d, auto b_c, auto k_c) {
    constexpr int k = decltype(k_c)::value;
    constexpr int kw = k / WJ, j = k % WJ;
    dma16(wrsrc, lds_dst(wbuf(b_c), (kw * WUP + j * 256) * 16), woff[j] | d.wor | d.wtap[kw],
          d.wsoff[kw]);
  };
  auto issue_x_one = [&](const StageDma& d, auto b_c, auto j_c) {
    constexpr int j = decltype(j_c)::value;
    const int radj = (REF && (xmask[j] & d.rbit)) ? d.radj : 0;
    const unsigned off = (xmask[j] & d.pbit) ? (unsigned)(xbase[j] + d.delta + radj) : kOobOffset;
    dma16(xrsrc, lds_dst(xbuf(b_c), j * 256 * 16), off, 0u);
  };

  // Set-up of tile t and the DMA of its first two stages.
  auto start_tile = [&](int t) {
    // Recomputing the per-lane set-up each tile is cheaper than the registers
    // of keeping it.
    const int lane = lane_id();
    if (a.queue) {
      tc.m0 = (t % a.m_tiles) * S::BM;
      const int rest = t / a.m_tiles;
      tc.co0 = (rest % a.n_tiles) * S::BN;
      tc.split = rest / a.n_tiles;
    } else {
      tc = tile_coord(a, S::BM, S::BN);
    }
    // Pixel tile mt: the mt-th run of TS slots, or (frame order) a run of
    // one frame, consecutive tiles taking the same rows of consecutive frames
    // (IgemmArgs::frames), and the tile walks its kd taps
    // starting from the input frame that is a multiple of 3: the tiles of
    // three consecutive frames then read each shared input frame at about
    // the same time.
    {
      const int mt = tc.m0 / S::BM;
      krot = 0;
      if (a.frames) {
        const int HT = a.N * a.head * a.frame_tiles;
        int f, b;
        if (mt < HT) {
          const int hf = mt / a.frame_tiles;
          b = mt - hf * a.frame_tiles;
          f = (hf / a.head) * a.Do + hf % a.head;
        } else {
          const int rest = a.Do - a.head, r = mt - HT;
          const int fr = r % (a.N * rest);
          b = r / (a.N * rest);
          f = (fr / rest) * a.Do + a.head + fr % rest;
        }
        tc.m0 = f * a.frame_slots + b * S::TS;
        tc.m_end = min(tc.m0 + S::TS, (f + 1) * a.frame_slots);
        const int d_in = (f % a.Do) * a.sd - a.pd;   // input frame of kd = 0
        krot = ((-d_in) % 3 + 3) % 3;
      } else {
        tc.m0 = mt * S::TS;
        tc.m_end = min(tc.m0 + S::TS, rows_total * WP);
      }
    }
    const int s0 = tc.m0;  // first slot of the tile
    const int row0 = small_div(s0, WP, inv_wp);
    const int s_last = tc.m_end - 1;
    const int nrows = small_div(s_last, WP, inv_wp) - row0 + 1;

    // Lane k describes output row row0 + k: the input pixel index of
    // (n, d0, h0, 0) and the 9-bit set of (kd, kh) pairs inside the input.
    int rbase = 0;
    unsigned rmask = 0;
    {
      const int r = row0 + lane;
      if (r < rows_total) {
        const int t2 = small_div(r, a.Ho, inv_ho);
        const int ho = r - t2 * a.Ho;
        const int n = small_div(t2, a.Do, inv_do);
        const int dq = t2 - n * a.Do;
        const int d0 = dq * a.sd - a.pd;
        const int h0 = ho * a.sh - a.ph;
        rmask = row_mask<REF>(a, d0, h0);
        rbase = ((n * a.D + d0) * a.H + h0) * a.W;
      }
    }
    // (kd, kh) pairs live for some row with an output in the tile.
    live = wave_or9(lane < nrows ? rmask : 0u);
    // Stage order: (kd, kh) pairs by (kd - krot) mod 3, then kh; bit q of
    // live becomes the q-th pair of that order.
    live = ((live >> (3 * krot)) | (live << (9 - 3 * krot))) & 0x1FFu;

    // Activation DMA entries: LDS unit q of a buffer holds chunk c of staged
    // slot sl (inverse of slot_unit). xbase is that chunk's byte offset in x
    // at kd = kh = 0 and channel chunk 0; xmask the pairs for which it lies
    // inside the input (0 for a padding column or a slot past the staged
    // range).
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int q = (j * 4 + wave) * 64 + lane;
      int sl, c;
      unit_slot<PB>(q, sl, c);
      const int s = s0 + sl;
      const int k = small_div(s, WP, inv_wp) - row0;
      const int w_in = s - (row0 + k) * WP - a.pw;
      const int kk = min(k, 63);
      const unsigned m = __shfl(rmask, kk);
      const int rb = __shfl(rbase, kk);
      const bool ok =
          sl < S::XS && (REF ? (w_in >= -1 && w_in <= a.W) : (w_in >= 0 && w_in < a.W));
      const int wc = REF ? reflect_index(w_in, a.W) : w_in;
      xmask[j] = ok ? m : 0u;
      xbase[j] = ok ? (rb + wc) * (a.Cin * ESZ) + c * 16 : 0;
    }
    // Weight DMA entries: LDS unit q of a tap holds row q / 4 of the permuted
    // channel order, 16-byte chunk (q % 4) XOR the row swizzle.
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      const int q = (j * 4 + wave) * 64 + lane;
      const int row = q >> 2;
      const int c = (q & 3) ^ (((row >> 1) ^ (row >> 3)) & 3);
      const int col = (row / (R * CB)) * (R * CB) + T::chan_of((row / R) % CB, row % R, CB);
      woff[j] = (q < WU) ? (unsigned)((tc.co0 + col) * 64 + c * 16) : kOobOffset;
    }
    s_begin = tc.split * a.steps_per_split;
    s_end = min(s_begin + a.steps_per_split, 9 * a.CC);
    // Stage table: a scalar walk over the live pairs hands out the steps;
    // lanes j = lane and 64 + lane of every wave form entries j and j + 64,
    // wave 0 stores them (read from the first barrier of the tile's main
    // loop on), and stages 0-2 come straight from lanes 0-2.
    // (Entries 64 and up only when the K range holds more than 64 steps.)
    const bool two = s_end - s_begin > 64;
    int sq[2] = {0, 0}, scc[2] = {0, 0};
    nst = 0;
    for (int q = 0; q < 9; ++q) {
      const int lo = max(s_begin, q * a.CC), hi = min(s_end, (q + 1) * a.CC);
      if (!((live >> q) & 1u) || lo >= hi) continue;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int j = p * 64 + lane - nst;
        if ((p == 0 || two) && j >= 0 && j < hi - lo) {
          sq[p] = q;
          scc[p] = lo - q * a.CC + j;
        }
      }
      nst += hi - lo;
    }
    si = 0;
    u32x4_t ent[2];
    ent[0] = stage_entry(sq[0], scc[0]);
    if (wave == 0 && lane < nst) stab[lane] = ent[0];
    if (two) {
      ent[1] = stage_entry(sq[1], scc[1]);
      if (wave == 0 && 64 + lane < nst) stab[64 + lane] = ent[1];
    }
    auto lane_entry = [&](int L) -> u32x4_t {
      u32x4_t t;
#pragma unroll
      for (int c = 0; c < 4; ++c) t[c] = (unsigned)__builtin_amdgcn_readlane((int)ent[0][c], L);
      return t;
    };
    const StageDma d0 = decode_uniform(lane_entry(0), 0 < nst), d1 = decode_uniform(lane_entry(1), 1 < nst);
    tnext = lane_entry(2);
    static_for<NW>([&](auto k) { issue_w_one(d0, SlotC<0>{}, k); });
    static_for<XJ>([&](auto j) { issue_x_one(d0, SlotC<0>{}, j); });
    static_for<NW1>([&](auto k) { issue_w_one(d1, SlotC<1>{}, k); });
    static_for<XJ>([&](auto j) { issue_x_one(d1, SlotC<1>{}, j); });
  };

  acc_t acc[CB][PB];
  // Epilogue of a finished tile (coordinates pt) from acc.
  auto finish_tile = [&](const TileCoord& pt) {
    // Lane-dependent values are formed here rather than hoisted into
    // registers that would have to live through the main loop.
    const int el = lane_id();
    const int elrow = el & 31, elgrp = el >> 5;
    // Output pixel of each pixel block: slot m0 + wave_m*R*PB + lrow*PB + p.
    int mp[PB];
    {
      const int sp0 = pt.m0 + wave_m * (PB * R) + elrow * PB;
      int r = small_div(sp0, WP, inv_wp);
      int c = sp0 - r * WP;
#pragma unroll
      for (int p = 0; p < PB; ++p) {
        mp[p] = (sp0 + p < pt.m_end && c < a.Wo) ? r * a.Wo + c : -1;
        if (++c == WP) {
          c = 0;
          ++r;
        }
      }
    }
    const int cbase = pt.co0 + wave_n * R * CB + elgrp * RUN;
    if constexpr (EPI == EPI_STATS) {
      // The plain store with GroupNorm statistics per (tile, channel tile):
      // the tile's first frame is that of its first slot's output row.
      static_assert(PB == 8 && CB == 2 && WN == 2 && KW == 3 && !F8, "512 x 128 bf16 tiles");
      // (The partials' address and the frame height come back from LDS:
      // kept in registers they would stay live through the main loop.)
      const unsigned long long gp = epi_sh[0], gq = epi_sh[1];
      float* gnp = reinterpret_cast<float*>(
          ((unsigned long long)__builtin_amdgcn_readfirstlane((int)(gp >> 32)) << 32) |
          (unsigned)__builtin_amdgcn_readfirstlane((int)gp));
      const int n_tiles = __builtin_amdgcn_readfirstlane((int)gq);
      const int ho = __builtin_amdgcn_readfirstlane((int)(gq >> 32));
      const int mt = pt.m0 / S::TS;
      const int f0 = small_div(small_div(pt.m0, WP, inv_wp), ho, inv_ho);
      store_staged<PB, true>(a, acc, xbuf2, pt.m0, pt.m_end, WP, inv_wp, pt.co0, wave_m, wave_n,
                             elrow, elgrp, mp, gnp + ((size_t)mt * n_tiles + pt.co0 / S::BN) * 128,
                             (f0 + 1) * ho);
    } else if (EPI == EPI_STORE && a.flags == 0 && !a.ypad) {
      // 512 x 128 tiles store through the activation buffer the next tile
      // first fills in its main loop (its set-up has filled the other two).
      if constexpr (PB == 8 && CB == 2 && WN == 2)
        store_staged<PB>(a, acc, xbuf2, pt.m0, pt.m_end, WP, inv_wp, pt.co0, wave_m, wave_n,
                         elrow, elgrp);
      else if constexpr (PB == 4 && CB <= 4 && WN == 1)
        store_staged_rows<PB, CB>(a, acc, xbuf2, pt.m0, pt.m_end, WP, inv_wp, pt.co0, wave_m,
                                  elrow, elgrp);
      else
        store_plain<T, PB, CB>(a, acc, mp, cbase);
    } else if constexpr (EPI == EPI_NORM) {
      auto run = [&](auto hb, auto hr) {
        epilogue_norm_slot<T, WM, WN, PB, CB, decltype(hb)::value, decltype(hr)::value>(
            a, acc, mp, pt.co0, cbase, wave_m, wave_n, elrow, elgrp, red, xbuf2);
      };
      using B1 = std::integral_constant<bool, true>;
      using B0 = std::integral_constant<bool, false>;
      if (a.flags & F_BIAS) {
        if (a.flags & F_RESIDUAL) run(B1{}, B1{});
        else run(B1{}, B0{});
      } else {
        if (a.flags & F_RESIDUAL) run(B0{}, B1{});
        else run(B0{}, B0{});
      }
    } else {
      epilogue<T, WM, WN, PB, CB, EPI>(a, acc, mp, cbase, pt.split, wave_m, wave_n, elrow, elgrp,
                                       red);
    }
  };

  // Pixel fragments by K half; weight fragments in a ring of three sub-steps
  // (sub-step t uses ring slot t % 3), for e4m3 both halves of each tap
  // (tap kw, half h in slot 2*kw + h).
  u32x4_t xf[2][NF], wf[F8 ? 6 : (KW == 2 ? 4 : 3)][CB];
  auto read_x = [&](auto b_c, int h, int f) {
    const char* xb = reinterpret_cast<const char*>(xbuf(b_c));
    xf[h][f] = *reinterpret_cast<const u32x4_t*>(xb + (h ? (ax[f] ^ 32) : ax[f]));
  };
  auto read_w = [&](auto b_c, int t, int cb) {
    const char* wb = reinterpret_cast<const char*>(wbuf(b_c));
    wf[t % 3][cb] = *reinterpret_cast<const u32x4_t*>(wb + aw[cb][t / 3] + (t % 3) * WTAP);
  };
  // Two-tap pairs: sub-step t is K half t / 2 of tap t % 2, ring slot t.
  auto read_w2 = [&](auto b_c, int t, int cb) {
    const char* wb = reinterpret_cast<const char*>(wbuf(b_c));
    wf[t][cb] = *reinterpret_cast<const u32x4_t*>(wb + aw[cb][t >> 1] + (t & 1) * WTAP);
  };
  auto read_w8 = [&](auto b_c, int kw, int h, int cb) {
    const char* wb = reinterpret_cast<const char*>(wbuf(b_c));
    wf[2 * kw + h][cb] = *reinterpret_cast<const u32x4_t*>(wb + aw[cb][h] + kw * WTAP);
  };

  // Main loop of one tile. Memory operations of sub-step u of a stage, in
  // issue order:
  //   urgent pixel reads: u0/u1 fragments PB / PB+1 of half 0 (needed one
  //     sub-step later); u4/u5 half-0 fragments of the next stage;
  //   CB weight reads for sub-step u + 2 (u4/u5: the next stage's 0 / 1);
  //   half-1 pixel reads: fragments [0, PB) over u0-u2, PB and PB+1 in u3;
  //   activation DMA of stage i+2 over u0-u3, weight DMA over u4-u5.
  auto iteration = [&](auto i_c) -> bool {
    constexpr int I = decltype(i_c)::value;
    constexpr int XB = I % 3, WB = I % 2;
    if (si >= nst) return false;
    const StageDma d2 = decode_uniform(tnext, si + 2 < nst);
    tnext = stab[min(si + 3, kSlotMaxStages - 1)];   // (for the next stage)
    if constexpr (KW == 2) {
      // Two-tap pairs: four sub-steps u (K half u / 2, tap u % 2), each CB*PB
      // MFMAs; tap kw of pixel block p reads fragment p + kw. Memory
      // operations of stage i, spread between single MFMAs:
      //   u0: fragment PB of half 0 (needed in u1), the weights of u2, the
      //       first half of the half-1 fragments, half of the activation DMA
      //       of stage i+2;
      //   u1: the weights of u3, the other half-1 fragments, the rest of the
      //       activation DMA;
      //   barrier (stage i+1 landed, stage i's buffers free), then
      //   u2: stage i+1's half-0 fragments [0, PB/2) and u0 weights, half the
      //       weight DMA of stage i+2 (into stage i's weight buffer);
      //   u3: stage i+1's half-0 fragments [PB/2, PB) and u1 weights, the
      //       rest of the weight DMA.
      // Each register a read overwrites was last read by an MFMA of an
      // earlier sub-step. Chunks of the odd pixel have no tap 3, so their
      // stages (every other one: the chunk order alternates pixels) skip
      // pair tap 1 (below).
      if constexpr (I % 2 == 0) static_for<4>([&](auto u_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr int h = u >> 1, kw = u & 1;
        constexpr int NM = CB * PB;
        constexpr int H1 = (NF + 1) / 2;
        constexpr int NX = u == 0 ? 1 + (H1) : (u == 1 ? NF - H1 : (u == 2 ? PB / 2 : PB - PB / 2));
        constexpr int ND = u < 2 ? (u == 0 ? XJ / 2 : XJ - XJ / 2) : (u == 2 ? NW / 2 : NW - NW / 2);
        constexpr int NOPS = NX + CB + ND;
        if constexpr (u == 2) {
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(XJ) : "memory");
          __builtin_amdgcn_sched_barrier(0);
        }
        static_for<NM>([&](auto g_c) {
          constexpr int g = decltype(g_c)::value;
          static_for<NOPS>([&](auto o_c) {
            constexpr int o = decltype(o_c)::value;
            if constexpr (o * NM / NOPS == g) {
              if constexpr (o < NX) {
                if constexpr (u == 0) {
                  if constexpr (o == 0) read_x(SlotC<XB>{}, 0, PB);
                  else read_x(SlotC<XB>{}, 1, o - 1);
                } else if constexpr (u == 1) {
                  read_x(SlotC<XB>{}, 1, H1 + o);
                } else if constexpr (u == 2) {
                  read_x(SlotC<(I + 1) % 3>{}, 0, o);
                } else {
                  read_x(SlotC<(I + 1) % 3>{}, 0, PB / 2 + o);
                }
              } else if constexpr (o < NX + CB) {
                constexpr int cb = o - NX;
                if constexpr (u < 2) read_w2(SlotC<WB>{}, u + 2, cb);
                else read_w2(SlotC<(I + 1) % 2>{}, u - 2, cb);
              } else {
                constexpr int k = o - NX - CB;
                if constexpr (u == 0) issue_x_one(d2, SlotC<(I + 2) % 3>{}, SlotC<k>{});
                else if constexpr (u == 1) issue_x_one(d2, SlotC<(I + 2) % 3>{}, SlotC<XJ / 2 + k>{});
                else if constexpr (u == 2) issue_w_one(d2, SlotC<WB>{}, SlotC<k>{});
                else issue_w_one(d2, SlotC<WB>{}, SlotC<NW / 2 + k>{});
              }
            }
          });
          __builtin_amdgcn_sched_barrier(0);
          constexpr int cb = g % CB, p = g / CB;
          acc[cb][p] = T::mma(__builtin_bit_cast(bf16x8_t, wf[u][cb]),
                              __builtin_bit_cast(bf16x8_t, xf[h][p + kw]), acc[cb][p]);
          __builtin_amdgcn_sched_barrier(0);
        });
      });
      else static_for<2>([&](auto v_c) {
        // Odd-pixel chunk (odd stages: a tile's stages start at chunk 0 of a
        // (kd, kh) pair, and each pair has an even number of them): pair
        // tap 0 (the layer's tap 1) alone, one sub-step per K half:
        //   v0: the half-1 fragments [0, PB) and tap-0 half-1 weights, all of
        //       the activation DMA of stage i+2;
        //   barrier, then
        //   v1: stage i+1's half-0 fragments [0, PB) and half-0 weights of
        //       both taps, the weight DMA of stage i+2 (pair tap 0 only).
        // (On entry, as for the four-sub-step form, half 0's fragments and
        // weights are in xf[0] and wf[0].)
        constexpr int v = decltype(v_c)::value;
        constexpr int NM = CB * PB;
        constexpr int NOPS = v == 0 ? PB + CB + XJ : PB + 2 * CB + WJ;
        if constexpr (v == 1) {
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(XJ) : "memory");
          __builtin_amdgcn_sched_barrier(0);
        }
        static_for<NM>([&](auto g_c) {
          constexpr int g = decltype(g_c)::value;
          static_for<NOPS>([&](auto o_c) {
            constexpr int o = decltype(o_c)::value;
            if constexpr (o * NM / NOPS == g) {
              if constexpr (v == 0) {
                if constexpr (o < PB) read_x(SlotC<XB>{}, 1, o);
                else if constexpr (o < PB + CB) read_w2(SlotC<WB>{}, 2, o - PB);
                else issue_x_one(d2, SlotC<(I + 2) % 3>{}, SlotC<o - PB - CB>{});
              } else {
                if constexpr (o < PB) read_x(SlotC<(I + 1) % 3>{}, 0, o);
                else if constexpr (o < PB + 2 * CB)
                  read_w2(SlotC<(I + 1) % 2>{}, (o - PB) / CB, (o - PB) % CB);
                else issue_w_one(d2, SlotC<WB>{}, SlotC<o - PB - 2 * CB>{});
              }
            }
          });
          __builtin_amdgcn_sched_barrier(0);
          constexpr int cb = g % CB, p = g / CB;
          acc[cb][p] = T::mma(__builtin_bit_cast(bf16x8_t, wf[2 * v][cb]),
                              __builtin_bit_cast(bf16x8_t, xf[v][p]), acc[cb][p]);
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    } else if constexpr (F8) {
      static_for<3>([&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        constexpr int NM = CB * PB;
        constexpr int NRD = s == 0 ? 4 * CB + 4 : (s == 1 ? 2 * CB + 4 : 2 * (PB - 2));
        constexpr int DW0 = s == 2 ? NW / 2 : 0;
        constexpr int ND = s == 0 ? XJ : (s == 1 ? NW / 2 : NW - NW / 2);
        if constexpr (s == 1) {
          // Stage i+1 has landed everywhere (only stage i+2's activations may
          // be in flight) and no wave reads stage i's buffers any more.
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(XJ) : "memory");
          __builtin_amdgcn_sched_barrier(0);
        }
        static_for<NM>([&](auto g_c) {
          constexpr int g = decltype(g_c)::value;
          static_for<NRD>([&](auto o_c) {
            constexpr int o = decltype(o_c)::value;
            if constexpr (f8_read_slot(s, o, NRD, NM, CB) == g) {
              if constexpr (s == 0) {
                if constexpr (o < 2 * CB)
                  read_w8(SlotC<WB>{}, 1, o / CB, o % CB);
                else if constexpr (o < 2 * CB + 4)
                  read_x(SlotC<XB>{}, (o - 2 * CB) % 2, PB + (o - 2 * CB) / 2);
                else
                  read_w8(SlotC<WB>{}, 2, (o - 2 * CB - 4) / CB, (o - 2 * CB - 4) % CB);
              } else if constexpr (s == 1) {
                if constexpr (o < 2 * CB)
                  read_w8(SlotC<(I + 1) % 2>{}, 0, o / CB, o % CB);
                else
                  read_x(SlotC<(I + 1) % 3>{}, (o - 2 * CB) % 2, (o - 2 * CB) / 2);
              } else {
                read_x(SlotC<(I + 1) % 3>{}, o % 2, 2 + o / 2);
              }
            }
          });
          static_for<ND>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            if constexpr (k * NM / ND == g) {
              if constexpr (s == 0) issue_x_one(d2, SlotC<(I + 2) % 3>{}, SlotC<k>{});
              else issue_w_one(d2, SlotC<WB>{}, SlotC<DW0 + k>{});
            }
          });
          __builtin_amdgcn_sched_barrier(0);
          constexpr int cb = g % CB, p = g / CB;
          acc[cb][p] = Mfma32F8::mma2(wf[2 * s][cb], wf[2 * s + 1][cb], xf[0][p + s],
                                      xf[1][p + s], acc[cb][p]);
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    } else {
      static_for<6>([&](auto u_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr int h = u / 3, kw = u % 3;
        constexpr int NURG = (u < 2) ? 1 : (u >= 4 ? (u - 3) * PB / 2 - (u - 4) * PB / 2 : 0);
        constexpr int URG0 = (u == 0) ? PB : (u == 1 ? PB + 1 : (u >= 4 ? (u - 4) * PB / 2 : 0));
        constexpr int H1LO = (u < 3) ? u * PB / 3 : (u == 3 ? PB : 0);
        constexpr int H1HI = (u < 3) ? (u + 1) * PB / 3 : (u == 3 ? PB + 2 : 0);
        constexpr int DXLO = (u < 4) ? u * XJ / 4 : 0, DXHI = (u < 4) ? (u + 1) * XJ / 4 : 0;
        constexpr int DWLO = (u >= 4) ? (u - 4) * NW / 2 : 0, DWHI = (u >= 4) ? (u - 3) * NW / 2 : 0;
        constexpr int NOPS = NURG + CB + (H1HI - H1LO) + (DXHI - DXLO) + (DWHI - DWLO);
        constexpr int NM = CB * PB;
        if constexpr (u == 4) {
          // Stage i+1 has landed everywhere (only stage i+2's activations may
          // be in flight) and no wave reads stage i's buffers any more.
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(XJ) : "memory");
          __builtin_amdgcn_sched_barrier(0);
        }
        static_for<NM>([&](auto g_c) {
          constexpr int g = decltype(g_c)::value;
          static_for<NOPS>([&](auto o_c) {
            constexpr int o = decltype(o_c)::value;
            if constexpr (o * NM / NOPS == g) {
              if constexpr (o < NURG) {
                if constexpr (u < 2) read_x(SlotC<XB>{}, 0, URG0 + o);
                else read_x(SlotC<(I + 1) % 3>{}, 0, URG0 + o);
              } else if constexpr (o < NURG + CB) {
                constexpr int cb = o - NURG;
                if constexpr (u < 4) read_w(SlotC<WB>{}, u + 2, cb);
                else read_w(SlotC<(I + 1) % 2>{}, u - 4, cb);
              } else if constexpr (o < NURG + CB + (H1HI - H1LO)) {
                read_x(SlotC<XB>{}, 1, H1LO + (o - NURG - CB));
              } else if constexpr (o < NURG + CB + (H1HI - H1LO) + (DXHI - DXLO)) {
                issue_x_one(d2, SlotC<(I + 2) % 3>{}, SlotC<DXLO + (o - NURG - CB - (H1HI - H1LO))>{});
              } else {
                issue_w_one(d2, SlotC<WB>{},
                            SlotC<DWLO + (o - NURG - CB - (H1HI - H1LO) - (DXHI - DXLO))>{});
              }
            }
          });
          __builtin_amdgcn_sched_barrier(0);
          constexpr int cb = g % CB, p = g / CB;
          acc[cb][p] = T::mma(__builtin_bit_cast(bf16x8_t, wf[u % 3][cb]),
                              __builtin_bit_cast(bf16x8_t, xf[h][p + kw]), acc[cb][p]);
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    }
    ++si;
    return true;
  };

  // Tile pipeline: the set-up and first DMA of tile t+1 go out before the
  // epilogue of tile t, so their latency hides behind its stores.
  int cur = 0;
  if (a.queue) {
    if (tid == 0) tile_sh = ticket_tile(take_ticket());
    __syncthreads();
    cur = __builtin_amdgcn_readfirstlane(tile_sh);
  }
  TileCoord prev;
  bool have_prev = false;
  for (;;) {
    int next_ticket = -1;
    if (cur >= 0) {
      if (a.queue && tid == 0) next_ticket = take_ticket();
      start_tile(cur);
    }
    if (have_prev) finish_tile(prev);
    if (cur < 0) break;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int p = 0; p < PB; ++p)
#pragma unroll
        for (int e = 0; e < NACC; ++e) acc[cb][p][e] = 0.f;
    // Stage 0 of this tile has landed everywhere; the previous tile's plain
    // stores (issued after this tile's DMA) may still be in flight.
    // (The barrier also publishes wave 0's stage table.)
    // The previous tile's stores follow this tile's first two stages' DMA.
    // A staged epilogue issues exactly EPI_VM stores per wave (out-of-range
    // ones included); any other may issue fewer, so the wait then covers its
    // stores too.
    if (have_prev && (EPI == EPI_STATS || (EPI == EPI_STORE && STAGED && a.flags == 0 && !a.ypad)))
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NW1 + XJ + EPI_VM) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NW1 + XJ) : "memory");
    if constexpr (F8) {
#pragma unroll
      for (int f = 0; f < PB; ++f) {
        read_x(SlotC<0>{}, 0, f);
        read_x(SlotC<0>{}, 1, f);
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        read_w8(SlotC<0>{}, 0, 0, cb);
        read_w8(SlotC<0>{}, 0, 1, cb);
      }
    } else {
#pragma unroll
      for (int f = 0; f < PB; ++f) read_x(SlotC<0>{}, 0, f);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        read_w(SlotC<0>{}, 0, cb);
        read_w(SlotC<0>{}, 1, cb);
      }
    }
    for (;;) {
      if (!iteration(SlotC<0>{})) break;
      if (!iteration(SlotC<1>{})) break;
      if (!iteration(SlotC<2>{})) break;
      if (!iteration(SlotC<3>{})) break;
      if (!iteration(SlotC<4>{})) break;
      if (!iteration(SlotC<5>{})) break;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // No wave reads this tile's buffers any more; the next tile's number is
    // visible to all.
    if (a.queue && tid == 0) tile_sh = ticket_tile(next_ticket);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    prev = tc;
    have_prev = true;
    cur = a.queue ? __builtin_amdgcn_readfirstlane(tile_sh) : -1;
  }
}

// ----------------------------------------------------------------------------
// Compiled configurations.
// ----------------------------------------------------------------------------
namespace {

template <class T, int WM, int WN, int PB, int CB, int KB, int NS, int EPI, bool REF>
int launch_one(const IgemmArgs& args, int grid, void* stream) {
  if constexpr (NS == -2)
    hipLaunchKernelGGL((igemm_slot_kernel<PB, CB, WN, EPI, REF, std::is_same<T, Mfma32F8>::value>),
                       dim3((unsigned)grid), dim3(256),
                       0, (hipStream_t)stream, args);
  else if constexpr (NS == -3)   // two-tap pairs: stride 2 along W on the pair view
    hipLaunchKernelGGL((igemm_slot_kernel<PB, CB, WN, EPI, false, false, 2>), dim3((unsigned)grid),
                       dim3(256), 0, (hipStream_t)stream, args);
  else if constexpr (NS < 0)
    hipLaunchKernelGGL((igemm_halo_kernel<CB, WN, KB, EPI, REF>), dim3((unsigned)grid), dim3(256),
                       0, (hipStream_t)stream, args);
  else if constexpr (NS == 0)
    hipLaunchKernelGGL((igemm_tile_kernel<T, WM, WN, PB, CB, KB, EPI>), dim3((unsigned)grid),
                       dim3(64 * WM * WN), 0, (hipStream_t)stream, args);
  else
    hipLaunchKernelGGL((igemm_kernel<T, WM, WN, PB, CB, KB, NS, EPI, REF>), dim3((unsigned)grid),
                       dim3(64 * WM * WN), 0, (hipStream_t)stream, args);
  return (int)hipGetLastError();
}

// The configurations are compiled in CONV3D_NPARTS translation units (the
// same source built with CONV3D_PART = 0 .. CONV3D_NPARTS - 1, so the build
// runs in parallel): every unit holds the whole table, and entry i's kernel
// is instantiated only in unit i % CONV3D_NPARTS. Unit 0 dispatches.
#ifndef CONV3D_PART
#define CONV3D_PART 0
#endif
#ifndef CONV3D_NPARTS
#define CONV3D_NPARTS 1
#endif
static_assert(CONV3D_NPARTS >= 1 && CONV3D_NPARTS <= 8 && CONV3D_PART < CONV3D_NPARTS,
              "between one and eight parts");

using LaunchFn = int (*)(const IgemmArgs&, int, void*);

template <int IDX, class T, int WM, int WN, int PB, int CB, int KB, int NS, int EPI, bool REF>
constexpr LaunchFn pick() {
  if constexpr (IDX % CONV3D_NPARTS == CONV3D_PART)
    return &launch_one<T, WM, WN, PB, CB, KB, NS, EPI, REF>;
  else
    return nullptr;
}

struct Entry {
  TileCfg cfg;
  int mode;
  bool reflect;   // spatial reflect padding compiled in
  bool fp8;       // e4m3 operands
  LaunchFn fn;    // null outside this entry's translation unit
};

constexpr int kCounterBase = __COUNTER__;
#define ENTRY(T, R, REFL, F8, WM, WN, PB, CB, KB, NS, MODE)                 \
  {{R, WM, WN, PB, CB, KB, NS}, MODE, REFL, F8,                              \
   pick<__COUNTER__ - kCounterBase - 1, T, WM, WN, PB, CB, KB, NS, MODE, REFL>()}
#define C32(...) ENTRY(Mfma32, 32, false, false, __VA_ARGS__)
#define C16(...) ENTRY(Mfma16, 16, false, false, __VA_ARGS__)
#define R32(...) ENTRY(Mfma32, 32, true, false, __VA_ARGS__)
#define R16(...) ENTRY(Mfma16, 16, true, false, __VA_ARGS__)
#define F32(...) ENTRY(Mfma32F8, 32, false, true, __VA_ARGS__)
const Entry kEntries[] = {
    // ns = -2: slot kernel (stride 1 along W, Cin % 32 == 0), 512-slot tiles.
    C32(2, 2, 8, 2, 0, -2, EPI_STORE),
    C32(4, 1, 4, 3, 0, -2, EPI_STORE),
    C32(2, 2, 3, 5, 0, -2, EPI_NORM),   // fused norm, Cout 320
    C32(4, 1, 3, 5, 0, -2, EPI_STORE),  // 384 slots x 160 channels
    C32(4, 1, 3, 5, 0, -2, EPI_NORM),   // fused norm, Cout 160
    // ns = -3: slot kernel on the pixel-pair view (stride 2 along W, two taps).
    C32(2, 2, 8, 2, 0, -3, EPI_STORE),
    C32(4, 1, 3, 4, 0, -3, EPI_STORE),
    C32(4, 1, 4, 4, 0, -3, EPI_STORE),
    // ns = -1: halo kernel (stride 1 along W, Cin % 32 == 0); kb = X DMA
    // instructions per wave and stage (the row-segment capacity).
    C32(4, 1, 4, 4, 9, -1, EPI_STORE),
    C32(4, 1, 4, 3, 9, -1, EPI_STORE),
    C32(4, 1, 4, 4, 9, -1, EPI_PARTIAL),
    C32(2, 2, 4, 4, 5, -1, EPI_PARTIAL),
    C32(2, 2, 4, 3, 5, -1, EPI_PARTIAL),
    // ns = 0: tile kernel (pixels staged through LDS too).
    C32(4, 1, 2, 4, 2, 0, EPI_STORE),
    C32(4, 1, 2, 4, 1, 0, EPI_STORE),
    C32(4, 1, 2, 3, 2, 0, EPI_STORE),
    C32(4, 1, 2, 4, 2, 0, EPI_PARTIAL),
    C16(2, 2, 2, 10, 2, 0, EPI_NORM),
    // Large-M layers: channel tile 128 / 96 / 64.
    C32(4, 1, 2, 4, 1, 3, EPI_STORE),
    C32(4, 1, 2, 4, 1, 4, EPI_STORE),
    C32(4, 1, 2, 4, 2, 4, EPI_STORE),
    C32(4, 1, 4, 4, 1, 2, EPI_STORE),
    C32(4, 1, 2, 3, 1, 3, EPI_STORE),
    C32(4, 1, 2, 3, 1, 4, EPI_STORE),
    C32(4, 1, 2, 2, 1, 3, EPI_STORE),
    // Split-K partials (small M, large K).
    C32(4, 1, 2, 4, 1, 3, EPI_PARTIAL),
    C32(4, 1, 1, 4, 1, 3, EPI_PARTIAL),
    C32(4, 1, 1, 4, 2, 3, EPI_PARTIAL),
    C32(4, 1, 2, 3, 1, 3, EPI_PARTIAL),
    C32(4, 1, 2, 2, 1, 3, EPI_PARTIAL),
    // Fused channel-row norm: the whole row of Cout channels in one group.
    C16(2, 2, 2, 10, 1, 3, EPI_NORM),  // Cout 320
    C16(4, 1, 2, 10, 1, 3, EPI_NORM),  // Cout 160
    // Any Cout % 16 == 0.
    C16(4, 1, 4, 2, 1, 3, EPI_STORE),
    C16(4, 1, 2, 2, 1, 3, EPI_PARTIAL),
    // Reflect spatial padding: slot, halo and the plain kernel's channel
    // tiles (the planner falls back to the last for anything else).
    R32(2, 2, 8, 2, 0, -2, EPI_STORE),
    R32(4, 1, 4, 3, 0, -2, EPI_STORE),
    R32(2, 2, 3, 5, 0, -2, EPI_NORM),
    R32(4, 1, 3, 5, 0, -2, EPI_STORE),
    R32(4, 1, 3, 5, 0, -2, EPI_NORM),
    R32(4, 1, 4, 4, 9, -1, EPI_STORE),
    R32(4, 1, 4, 3, 9, -1, EPI_STORE),
    R32(4, 1, 4, 4, 9, -1, EPI_PARTIAL),
    R32(2, 2, 4, 4, 5, -1, EPI_PARTIAL),
    R32(2, 2, 4, 3, 5, -1, EPI_PARTIAL),
    R32(4, 1, 2, 4, 1, 3, EPI_STORE),
    R32(4, 1, 2, 3, 1, 3, EPI_STORE),
    R32(4, 1, 2, 2, 1, 3, EPI_STORE),
    R32(4, 1, 2, 4, 1, 3, EPI_PARTIAL),
    R32(4, 1, 1, 4, 1, 3, EPI_PARTIAL),
    R32(4, 1, 2, 3, 1, 3, EPI_PARTIAL),
    R32(4, 1, 2, 2, 1, 3, EPI_PARTIAL),
    R16(2, 2, 2, 10, 1, 3, EPI_NORM),
    R16(4, 1, 2, 10, 1, 3, EPI_NORM),
    R16(4, 1, 4, 2, 1, 3, EPI_STORE),
    R16(4, 1, 2, 2, 1, 3, EPI_PARTIAL),
    // e4m3 operands: the slot kernel (Cin % 64 == 0) and the plain kernel's
    // 32-row channel tiles.
    F32(2, 2, 8, 2, 0, -2, EPI_STORE),
    F32(4, 1, 2, 4, 1, 3, EPI_STORE),
    F32(4, 1, 2, 3, 1, 3, EPI_STORE),
    F32(4, 1, 2, 2, 1, 3, EPI_STORE),
    F32(4, 1, 2, 4, 1, 3, EPI_PARTIAL),
    F32(4, 1, 1, 4, 1, 3, EPI_PARTIAL),
    F32(4, 1, 2, 3, 1, 3, EPI_PARTIAL),
    F32(4, 1, 2, 2, 1, 3, EPI_PARTIAL),
    // The 512 x 128 slot tile's plain store with GroupNorm statistics.
    C32(2, 2, 8, 2, 0, -2, EPI_STATS),
    R32(2, 2, 8, 2, 0, -2, EPI_STATS),
};
#undef C32
#undef C16
#undef R32
#undef R16
#undef F32
#undef ENTRY

constexpr int kNumEntries = (int)(sizeof kEntries / sizeof kEntries[0]);

int find_entry(const TileCfg& c, int mode, bool reflect, bool fp8) {
  for (int i = 0; i < kNumEntries; ++i) {
    const Entry& e = kEntries[i];
    if (e.cfg.r == c.r && e.cfg.wm == c.wm && e.cfg.wn == c.wn && e.cfg.pb == c.pb &&
        e.cfg.cb == c.cb && e.cfg.kb == c.kb && e.cfg.ns == c.ns && e.mode == mode &&
        e.reflect == reflect && e.fp8 == fp8)
      return i;
  }
  return -1;
}

}  // namespace

#define PART_FN_(P) igemm_launch_part_##P
#define PART_FN(P) PART_FN_(P)
// Launch of entry idx, which must belong to this translation unit.
int PART_FN(CONV3D_PART)(int idx, const IgemmArgs& args, int grid, void* stream) {
  return kEntries[idx].fn(args, grid, stream);
}

#if CONV3D_PART == 0
#if CONV3D_NPARTS > 1
int igemm_launch_part_1(int, const IgemmArgs&, int, void*);
#endif
#if CONV3D_NPARTS > 2
int igemm_launch_part_2(int, const IgemmArgs&, int, void*);
#endif
#if CONV3D_NPARTS > 3
int igemm_launch_part_3(int, const IgemmArgs&, int, void*);
#endif
#if CONV3D_NPARTS > 4
int igemm_launch_part_4(int, const IgemmArgs&, int, void*);
#endif
#if CONV3D_NPARTS > 5
int igemm_launch_part_5(int, const IgemmArgs&, int, void*);
#endif
#if CONV3D_NPARTS > 6
int igemm_launch_part_6(int, const IgemmArgs&, int, void*);
#endif
#if CONV3D_NPARTS > 7
int igemm_launch_part_7(int, const IgemmArgs&, int, void*);
#endif

bool igemm_has_config(const TileCfg& cfg, int mode, bool reflect, bool fp8) {
  return find_entry(cfg, mode, reflect, fp8) >= 0;
}

int launch_igemm(const TileCfg& cfg, int mode, bool reflect, bool fp8, const IgemmArgs& args,
                 int grid, void* stream) {
  const int i = find_entry(cfg, mode, reflect, fp8);
  if (i < 0) return -1;
  static int (*const parts[CONV3D_NPARTS])(int, const IgemmArgs&, int, void*) = {
      igemm_launch_part_0,
#if CONV3D_NPARTS > 1
      igemm_launch_part_1,
#endif
#if CONV3D_NPARTS > 2
      igemm_launch_part_2,
#endif
#if CONV3D_NPARTS > 3
      igemm_launch_part_3,
#endif
#if CONV3D_NPARTS > 4
      igemm_launch_part_4,
#endif
#if CONV3D_NPARTS > 5
      igemm_launch_part_5,
#endif
#if CONV3D_NPARTS > 6
      igemm_launch_part_6,
#endif
#if CONV3D_NPARTS > 7
      igemm_launch_part_7,
#endif
  };
  return parts[i % CONV3D_NPARTS](i, args, grid, stream);
}
#endif  // CONV3D_PART == 0

}  // namespace conv3d
