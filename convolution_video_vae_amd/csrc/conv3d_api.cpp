// C-ABI of the Conv3D library: argument checks, planning and dispatch.
//
// Every check here runs on the host before anything is enqueued, so a bad
// call never launches work or touches an output (cuDNN page,
// "Requirements": aligned operands, outputs that overlap no operand, no
// silent fallback for an unsupported case).
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>

#include "../../include/conv3d.h"
#include "conv3d_internal.h"

using namespace conv3d;

namespace {

constexpr long long kMaxTensorBytes = (1LL << 31) - 64;  // 32-bit buffer offsets

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
  bool empty() const { return hi <= lo; }
};

Range range_of(const void* p, long long bytes) {
  Range r;
  if (p && bytes > 0) {
    r.lo = (uintptr_t)p;
    r.hi = r.lo + (uintptr_t)bytes;
  }
  return r;
}

bool overlaps(const Range& a, const Range& b) {
  return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int out_extent(int in, int s, int lo, int hi) {
  const long long span = (long long)in + lo + hi - 3;
  if (span < 0) return 0;
  const long long o = span / s + 1;
  return o > 0x7fffffffLL ? 0x7fffffff : (int)o;
}

// Product of non-negative sizes, saturating at 2^62 (every size check
// rejects far smaller values), so no size computation overflows.
constexpr long long kSat = 1LL << 62;
long long prod(std::initializer_list<long long> v) {
  long long r = 1;
  for (long long a : v) {
    if (a <= 0) return a < 0 ? kSat : 0;
    r = (r > kSat / a) ? kSat : r * a;
  }
  return r;
}

// Everything derived from a descriptor.
struct Problem {
  int n, d, h, w, cin, cout;
  int sd, sh, sw, pd, ph, pw;
  int Do, Ho, Wo;
  long long M;
  long long x_bytes, y_bytes;
  int layout, out_layout;
  unsigned flags;
  bool reflect;    // spatial reflect padding
  bool fp8;        // e4m3 x and packed weight
  // Samples per pass: a call whose tensors exceed the 32-bit buffer range
  // runs as passes over nb consecutive samples each (N is the outermost
  // dimension of every tensor involved); nb == n for one pass.
  int nb;
};

struct Plan {
  TileCfg cfg;
  // live-balanced K split of halo-kernel partials (IgemmArgs::vsplit)
  bool vsplit = false;
  int per_n = 0;
  uint16_t split_base[kMaxVTiles + 1] = {};
  uint16_t wg[kMaxVWG] = {};
  int mode;        // EPI_STORE / EPI_NORM / EPI_PARTIAL
  int splits;      // >1 or reduce needed -> partial + reduce
  bool reduce;     // a reduce kernel finishes the epilogue
  int steps;       // 27 * CC
  int steps_per_split;
  int m_tiles, n_tiles;
  // slot kernels: frames tiled one by one, tiles of the same rows of
  // consecutive frames next to each other (IgemmArgs::frames)
  bool frame_order = false;
  int frame_slots = 0, frame_tiles = 0, head = 0;
  long long grid;
  // workspace carve (bytes, 256-aligned offsets)
  bool persistent; // one work-group per CU taking tiles from queues
  size_t off_x, off_y, off_res, off_rout, off_part, off_queue, total;
};

size_t packed_bytes(const Problem& pr) {
  return pr.fp8 ? conv3d_packed_weight_bytes_fp8(pr.cout, pr.cin)
                : conv3d_packed_weight_bytes(pr.cout, pr.cin);
}

// 64-byte K steps: 32 bf16 or 64 e4m3 channels.
int k_chunks(const Problem& pr) { return pr.fp8 ? (pr.cin + 63) / 64 : (pr.cin + 31) / 32; }

conv3d_status check_desc(const conv3d_desc* d, Problem* pr) {
  *pr = Problem{};   // (flags stay 0 until check_epi sets them)
  if (!d) return CONV3D_ERR_NULL;
  if (d->n <= 0 || d->d <= 0 || d->h <= 0 || d->w <= 0 || d->cin <= 0 || d->cout <= 0)
    return CONV3D_ERR_SHAPE;
  for (int i = 0; i < 3; ++i) {
    if (d->stride[i] <= 0 || d->pad_lo[i] < 0 || d->pad_hi[i] < 0) return CONV3D_ERR_SHAPE;
  }
  if (d->layout != CONV3D_NCDHW && d->layout != CONV3D_NDHWC) return CONV3D_ERR_SHAPE;
  if (d->out_layout != CONV3D_NCDHW && d->out_layout != CONV3D_NDHWC) return CONV3D_ERR_SHAPE;
  if (d->split_k < 0) return CONV3D_ERR_SHAPE;
  if (d->pad_mode != CONV3D_PAD_ZERO && d->pad_mode != CONV3D_PAD_REFLECT) return CONV3D_ERR_SHAPE;
  pr->reflect = d->pad_mode == CONV3D_PAD_REFLECT;
  if (d->dtype != CONV3D_BF16 && d->dtype != CONV3D_FP8_E4M3) return CONV3D_ERR_SHAPE;
  pr->fp8 = d->dtype == CONV3D_FP8_E4M3;
  if (pr->reflect) {
    if (d->h < 2 || d->w < 2) return CONV3D_ERR_SHAPE;
    for (int i = 1; i < 3; ++i)
      if (d->pad_lo[i] > 1 || d->pad_hi[i] > 1) return CONV3D_ERR_UNSUPPORTED;
  }
  pr->n = d->n; pr->d = d->d; pr->h = d->h; pr->w = d->w;
  pr->cin = d->cin; pr->cout = d->cout;
  pr->sd = d->stride[0]; pr->sh = d->stride[1]; pr->sw = d->stride[2];
  pr->pd = d->pad_lo[0]; pr->ph = d->pad_lo[1]; pr->pw = d->pad_lo[2];
  pr->Do = out_extent(d->d, d->stride[0], d->pad_lo[0], d->pad_hi[0]);
  pr->Ho = out_extent(d->h, d->stride[1], d->pad_lo[1], d->pad_hi[1]);
  pr->Wo = out_extent(d->w, d->stride[2], d->pad_lo[2], d->pad_hi[2]);
  if (pr->Do < 1 || pr->Ho < 1 || pr->Wo < 1) return CONV3D_ERR_SHAPE;
  pr->M = prod({d->n, pr->Do, pr->Ho, pr->Wo});
  pr->x_bytes = prod({d->n, d->d, d->h, d->w, d->cin, pr->fp8 ? 1 : 2});
  pr->y_bytes = prod({pr->M, d->cout, 2});
  pr->layout = d->layout;
  pr->out_layout = d->out_layout;
  if (d->cin % 8 != 0) return CONV3D_ERR_ALIGN;
  if (pr->fp8) {
    if (d->cin % 16 != 0) return CONV3D_ERR_ALIGN;
    if (d->cout % 32 != 0 || pr->reflect || d->layout != CONV3D_NDHWC ||
        d->out_layout != CONV3D_NDHWC)
      return CONV3D_ERR_UNSUPPORTED;
  }
  if (d->cin > 8160) return CONV3D_ERR_UNSUPPORTED;  // K steps are encoded in 8 bits per tap
  if (d->cout % 16 != 0) return CONV3D_ERR_UNSUPPORTED;
  // One sample's tensors must fit the 32-bit buffer range; larger batches
  // run in passes of nb samples.
  const long long xs = prod({d->d, d->h, d->w, d->cin, pr->fp8 ? 1 : 2});
  const long long ms = prod({pr->Do, pr->Ho, pr->Wo});
  const long long ys = prod({ms, d->cout, 2});
  if (xs > kMaxTensorBytes || ys > kMaxTensorBytes || ms > 0x7fffffffLL)
    return CONV3D_ERR_UNSUPPORTED;
  if ((long long)packed_bytes(*pr) > kMaxTensorBytes)
    return CONV3D_ERR_UNSUPPORTED;
  pr->nb = (int)std::min<long long>(
      {(long long)d->n, kMaxTensorBytes / xs, kMaxTensorBytes / ys, 0x7fffffffLL / ms});
  return CONV3D_OK;
}

conv3d_status check_epi(const conv3d_epilogue* e, Problem* pr) {
  pr->flags = e ? e->flags : 0u;
  const unsigned f = pr->flags;
  if (f & ~(unsigned)(F_BIAS | F_RESIDUAL | F_NORM | F_RESIDUAL_OUT)) return CONV3D_ERR_UNSUPPORTED;
  if ((f & F_RESIDUAL_OUT) && !(f & F_RESIDUAL)) return CONV3D_ERR_UNSUPPORTED;
  if ((f & F_BIAS) && !e->bias) return CONV3D_ERR_NULL;
  if ((f & F_RESIDUAL) && !e->residual) return CONV3D_ERR_NULL;
  if ((f & F_NORM) && !e->gamma) return CONV3D_ERR_NULL;
  if ((f & F_RESIDUAL_OUT) && !e->residual_out) return CONV3D_ERR_NULL;
  if ((f & F_BIAS) && !aligned16(e->bias)) return CONV3D_ERR_ALIGN;
  if ((f & F_RESIDUAL) && !aligned16(e->residual)) return CONV3D_ERR_ALIGN;
  if ((f & F_NORM) && !aligned16(e->gamma)) return CONV3D_ERR_ALIGN;
  if ((f & F_RESIDUAL_OUT) && !aligned16(e->residual_out)) return CONV3D_ERR_ALIGN;
  if ((f & F_NORM) && pr->cout > 2048) return CONV3D_ERR_UNSUPPORTED;
  return CONV3D_OK;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Kernel choice. Large-M layers run one work-group per (pixel tile, channel
// tile); small-M / large-K layers cut K into slices whose fp32 partials a
// second kernel sums in fixed order.
constexpr int kCUs = 256;

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Channel blocking: the widest tile that divides Cout (each lane's run of
// channels must stay inside Cout). `store` is the measured-fastest direct
// configuration, the plain one is used for split-K partials.
TileCfg channel_cfg(int cout) {
  if (cout % 128 == 0) return {32, 4, 1, 2, 4, 1, 3};
  if (cout % 96 == 0) return {32, 4, 1, 2, 3, 1, 3};
  if (cout % 32 == 0) return {32, 4, 1, 2, 2, 1, 3};
  return {16, 4, 1, 4, 2, 1, 3};
}

TileCfg store_channel_cfg(int cout) {
  if (cout % 128 == 0) return {32, 4, 1, 2, 4, 2, 0};   // three-stage LDS tile kernel
  if (cout % 96 == 0) return {32, 4, 1, 2, 3, 1, 4};
  return channel_cfg(cout);
}

// Halo kernel configurations {32, 4 / WN, WN, 4, CB, XJ, -1}: stride 1 along
// W and whole 32-channel chunks; kb = XJ, the X DMA instructions per wave and
// stage, sets how many output-row segments one tile may span.
int halo_maxseg(const TileCfg& c) { return (c.kb * 256 / 4 - c.bm() - 2) / 2 + 1; }

// Slot kernel {32, WM, WN, PB, CB, 0, -2}: stride 1 along W and whole
// K-step chunks (32 bf16 or 64 e4m3 channels). Output row r owns Wo + 2 slots and a tile is bm() of
// them; the bm() slots staged per stage must span at most 64 output rows
// (one lane each), and slot indices are split with a float-reciprocal
// division, exact below 2^24: the index converts to fp32 exactly, and for a
// divisor of at least 2 the product with the rounded reciprocal is within
// one of the quotient, which the kernel's correction steps absorb (a divisor
// of 1 is exact). A tile's stages (9 (kd, kh) pairs x chunks) must fit the
// kernel's per-tile stage table (kSlotMaxStages: Cin up to 448 bf16 or 896
// e4m3 channels, 224 on the pixel-pair view).
long long slot_rows(const Problem& pr) { return prod({pr.n, pr.Do, pr.Ho}); }

bool slot_ok(const Problem& pr, const TileCfg& c) {
  const long long wp = pr.Wo + 2;
  return pr.sw == 1 && pr.cin % (pr.fp8 ? 64 : 32) == 0 && c.bn() > 0 && pr.cout % c.bn() == 0 &&
         (c.bm() + 1) / wp + 2 <= 64 && slot_rows(pr) * wp + c.bm() + 2048 < (1LL << 24) &&
         9 * k_chunks(pr) <= kSlotMaxStages;
}

// Stride 2 along W on the pixel-pair view (slot kernel, ns = -3): the input
// [n][d][h][w][cin] read as [n][d][h][w / 2][2 * cin], a stride-1 conv with
// two taps along W (tap kw' of the pair view, chunk half e: the layer's tap
// 2 * kw' + e). It needs no leading W padding (output column wo then reads
// pairs wo and wo + 1), an even W and whole 32-channel chunks per pixel, so
// that each chunk of a pair lies in one of its two pixels.
Problem pair_view(const Problem& pr) {
  Problem v = pr;
  v.w = pr.w / 2;
  v.cin = 2 * pr.cin;
  v.sw = 1;
  v.pw = 0;
  return v;
}

bool pair_ok(const Problem& pr, const TileCfg& c) {
  if (pr.sw != 2 || pr.pw != 0 || pr.w % 2 != 0 || pr.cin % 32 != 0 || pr.reflect || pr.fp8)
    return false;
  const Problem v = pair_view(pr);
  const long long wp = v.Wo + 1;
  return c.bn() > 0 && v.cout % c.bn() == 0 && (c.bm() + 1) / wp + 2 <= 64 &&
         slot_rows(v) * wp + c.bm() + 2048 < (1LL << 24) && 9 * k_chunks(v) <= kSlotMaxStages;
}

bool halo_ok(const Problem& pr, const TileCfg& c) {
  if (c.ns >= 0) return true;
  if (c.ns == -2) return slot_ok(pr, c);
  if (c.ns == -3) return pair_ok(pr, c);
  // (Output rows are split with a float-reciprocal division, exact below 2^22.)
  return pr.sw == 1 && pr.cin % 32 == 0 && c.bn() > 0 && pr.cout % c.bn() == 0 &&
         ceil_div(c.bm() - 1, pr.Wo) + 1 <= halo_maxseg(c) &&
         prod({pr.n, pr.Do, pr.Ho}) < (1LL << 22);
}

const TileCfg kSlotStore[] = {{32, 2, 2, 8, 2, 0, -2}, {32, 4, 1, 4, 3, 0, -2},
                               {32, 4, 1, 3, 5, 0, -2}};
const TileCfg kHaloStore[] = {{32, 4, 1, 4, 4, 9, -1}, {32, 4, 1, 4, 3, 9, -1}};
// (512 x 128 tiles either way; one wave column across the 128 channels measured 4%
// faster on H3 L0's stride-(1,2,2) layer: 250 against 260-263 us alternating.)
const TileCfg kPairStore[] = {{32, 4, 1, 4, 4, 0, -3}, {32, 2, 2, 8, 2, 0, -3}};
const TileCfg kHaloPartial[] = {{32, 2, 2, 4, 4, 5, -1}, {32, 2, 2, 4, 3, 5, -1},
                                {32, 4, 1, 4, 4, 9, -1}};

template <int N>
bool pick_halo(const Problem& pr, const TileCfg (&cands)[N], int mode, TileCfg* out) {
  for (const TileCfg& c : cands)
    if (halo_ok(pr, c) && igemm_has_config(c, mode, pr.reflect, pr.fp8)) {
      *out = c;
      return true;
    }
  return false;
}

// Live K steps of halo-kernel pixel tile t (BM output pixels from t * BM):
// the (kd, kh) pairs for which some output row of the tile reads real input
// (the kernel's per-row masks, ORed over the tile's rows), times the
// 32-channel chunks.
int tile_live_steps(const Problem& pr, int BM, int t, int cc) {
  const long long m0 = (long long)t * BM, m1 = std::min<long long>(m0 + BM, pr.M) - 1;
  unsigned mask = 0;
  for (long long r = m0 / pr.Wo; r <= m1 / pr.Wo && mask != 511u; ++r) {
    const long long t2 = r / pr.Ho;
    const int ho = (int)(r - t2 * pr.Ho);
    const int dq = (int)(t2 % pr.Do);
    const int d0 = dq * pr.sd - pr.pd, h0 = ho * pr.sh - pr.ph;
    for (int kd = 0; kd < 3; ++kd)
      for (int kh = 0; kh < 3; ++kh) {
        const bool dv = d0 + kd >= 0 && d0 + kd < pr.d;
        const bool hv = pr.reflect || (h0 + kh >= 0 && h0 + kh < pr.h);
        if (dv && hv) mask |= 1u << (kd * 3 + kh);
      }
  }
  return __builtin_popcount(mask) * cc;
}

// Live-balanced K split of a halo-kernel partial plan: every pixel tile is
// cut into slices of at most q live K steps, q the smallest quota (of at
// least 4) whose slices fit one round of work-groups (kCUs over all channel
// tiles). Tiles
// that see fewer taps (a causal layer's first frames) get fewer slices, so
// all work-groups carry about the same live work. Launch order is slice-
// major (slice s of every tile, then s + 1), which keeps the same slice of
// tiles with the same live taps, i.e. the same weight rows, next to each
// other (they land on one XCD's L2). Returns false when the plan does not
// fit the tables.
bool plan_vsplit(const Problem& pr, int cc, Plan* pl) {
  const int T = pl->m_tiles, NT = pl->n_tiles;
  if (T > kMaxVTiles || NT <= 0) return false;
  const int cap = std::min(kCUs / NT, kMaxVWG);
  if (cap < T) return false;
  int L[kMaxVTiles];
  long long total = 0;
  for (int t = 0; t < T; ++t) {
    L[t] = tile_live_steps(pr, pl->cfg.bm(), t, cc);
    total += L[t];
  }
  // (at least 4 live steps per slice, as the uniform split keeps)
  int q = (int)std::max(4LL, ceil_div(total, cap));
  for (;; ++q) {
    long long n = 0;
    for (int t = 0; t < T; ++t) n += std::max(1LL, ceil_div(L[t], q));
    if (n <= cap) break;
  }
  int S[kMaxVTiles], smax = 0;
  pl->split_base[0] = 0;
  for (int t = 0; t < T; ++t) {
    S[t] = (int)std::max(1LL, ceil_div(L[t], q));
    if (S[t] > 255) return false;
    smax = std::max(smax, S[t]);
    pl->split_base[t + 1] = (uint16_t)(pl->split_base[t] + S[t]);
  }
  int i = 0;
  for (int sl = 0; sl < smax; ++sl)
    for (int t = 0; t < T; ++t)
      if (sl < S[t]) pl->wg[i++] = (uint16_t)((t << 8) | sl);
  pl->per_n = i;
  pl->vsplit = true;
  pl->splits = smax;
  pl->grid = (long long)i * NT;
  return true;
}

// K steps a kernel walks: 27 taps x 32-channel chunks, or for the halo
// kernel 9 (kd, kh) pairs x 32-channel chunks.
int steps_of(const TileCfg& c, int cc) {
  return c.ns == -3 ? 9 * 2 * cc : (c.ns < 0 ? 9 * cc : 27 * cc);   // pair view: 2 * cc chunks
}

void make_plan(const Problem& pr, int split_req, Plan* pl) {
  const int cc = k_chunks(pr);
  const bool norm = (pr.flags & F_NORM) != 0;
  TileCfg base = channel_cfg(pr.cout);
  const long long n_tiles = ceil_div(pr.cout, base.bn());

  TileCfg store_cfg = store_channel_cfg(pr.cout);
  if (!igemm_has_config(store_cfg, EPI_STORE, pr.reflect, pr.fp8)) store_cfg = base;
  if (!norm && !pick_halo(pr, kPairStore, EPI_STORE, &store_cfg) &&
      !pick_halo(pr, kSlotStore, EPI_STORE, &store_cfg))
    pick_halo(pr, kHaloStore, EPI_STORE, &store_cfg);
  TileCfg part_cfg = base;
  part_cfg.pb = 2;
  if (base.r == 32 && ceil_div(pr.M, part_cfg.bm()) * n_tiles < 64) {
    TileCfg c = base;
    c.pb = 1;
    if (igemm_has_config(c, EPI_PARTIAL, pr.reflect, pr.fp8)) part_cfg = c;
  }
  // (Fragment-order partials of the halo kernel have no norm reduction.)
  if (!norm) pick_halo(pr, kHaloPartial, EPI_PARTIAL, &part_cfg);

  // Fused-norm kernels hold the whole channel row of a pixel in one group.
  TileCfg norm_cfg = {0, 0, 0, 0, 0, 0, 0};
  if (norm) {
    const TileCfg cands[] = {{32, 2, 2, 3, 5, 0, -2}, {32, 4, 1, 3, 5, 0, -2},
                             {16, 2, 2, 2, 10, 2, 0}, {16, 2, 2, 2, 10, 1, 3},
                             {16, 4, 1, 2, 10, 1, 3}};
    for (const TileCfg& c : cands)
      if (norm_cfg.r == 0 && c.bn() == pr.cout && halo_ok(pr, c) &&
          igemm_has_config(c, EPI_NORM, pr.reflect, pr.fp8))
        norm_cfg = c;
  }

  // Too few tiles to fill the CUs: cut K. (The slot kernel's tiles run so
  // much faster than the plain kernel's split ones that a quarter of the CUs'
  // worth of them is enough: measured on the 160-channel Wan layers, 102
  // slot tiles take half the time of the split plan.)
  const long long store_tiles = ceil_div(pr.M, store_cfg.bm()) * ceil_div(pr.cout, store_cfg.bn());
  const long long min_tiles = store_cfg.ns <= -2 ? kCUs / 4 : kCUs / 2;
  const bool split = split_req > 1 || (split_req == 0 && store_tiles < min_tiles);

  // Development override of the tile (same kernels, another compiled
  // configuration): CONV3D_TILE="r,wm,wn,pb,cb,kb,ns".
  if (const char* env = getenv("CONV3D_TILE")) {
    TileCfg c;
    if (sscanf(env, "%d,%d,%d,%d,%d,%d,%d", &c.r, &c.wm, &c.wn, &c.pb, &c.cb, &c.kb, &c.ns) == 7 &&
        c.bn() > 0 && pr.cout % c.bn() == 0 && halo_ok(pr, c)) {
      const int mode = split ? EPI_PARTIAL : (norm ? EPI_NORM : EPI_STORE);
      // (A fused-norm tile must hold the whole channel row of a pixel, and the
      // fragment-order partials of the halo kernel have no norm reduction.)
      if (igemm_has_config(c, mode, pr.reflect, pr.fp8) && (mode != EPI_NORM || c.bn() == pr.cout) &&
          !(mode == EPI_PARTIAL && norm && c.ns == -1)) {
        if (mode == EPI_PARTIAL) part_cfg = c;
        else if (mode == EPI_NORM) norm_cfg = c;
        else store_cfg = c;
      }
    }
  }

  if (split || (norm && norm_cfg.r == 0)) {
    pl->cfg = part_cfg;
    pl->mode = EPI_PARTIAL;
    pl->reduce = true;
  } else if (norm) {
    pl->cfg = norm_cfg;
    pl->mode = EPI_NORM;
    pl->reduce = false;
  } else {
    pl->cfg = store_cfg;
    pl->mode = EPI_STORE;
    pl->reduce = false;
  }

  pl->steps = steps_of(pl->cfg, cc);
  int splits = 1;
  if (split_req > 1) {
    splits = split_req;
  } else if (split) {
    const long long tiles = ceil_div(pr.M, pl->cfg.bm()) * ceil_div(pr.cout, pl->cfg.bn());
    if (pl->cfg.ns < 0)   // one work-group per CU: fill one round
      splits = (int)std::max(1LL, std::min<long long>(kCUs / tiles, pl->steps / 4));
    else                  // about two groups per CU, at least 8 K steps each
      splits = (int)std::max(1LL, std::min<long long>(ceil_div(2 * kCUs, tiles), pl->steps / 8));
  }
  splits = std::max(1, std::min(splits, pl->steps));
  pl->steps_per_split = (pl->steps + splits - 1) / splits;
  pl->splits = (pl->steps + pl->steps_per_split - 1) / pl->steps_per_split;
  // (Slot kernel tiles compute bm() slots and store bm() - 2.)
  pl->m_tiles = pl->cfg.ns == -2   ? (int)ceil_div(slot_rows(pr) * (pr.Wo + 2), pl->cfg.bm() - 2)
                : pl->cfg.ns == -3 ? (int)ceil_div(slot_rows(pr) * (pr.Wo + 1), pl->cfg.bm() - 1)
                                   : (int)ceil_div(pr.M, pl->cfg.bm());
  // Frame order for the slot kernels (one K slice per tile): the L2 of an
  // XCD then serves the input frames that the tiles of consecutive output
  // frames share.
  pl->frame_order = false;
  if (pl->cfg.ns <= -2 && pl->steps_per_split == pl->steps) {
    const char* env = getenv("CONV3D_FRAME_ORDER");
    pl->frame_order = env ? atoi(env) != 0 : pl->cfg.ns == -3;
  }
  if (pl->frame_order) {
    const int ts = pl->cfg.bm() - (pl->cfg.ns == -3 ? 1 : 2);
    pl->frame_slots = pr.Ho * (pr.Wo + (pl->cfg.ns == -3 ? 1 : 2));
    pl->frame_tiles = (int)ceil_div(pl->frame_slots, ts);
    pl->m_tiles = (int)(prod({pr.n, pr.Do}) * pl->frame_tiles);
    // Leading frames whose kd = 0 tap lies before the input: handed out last
    // (the queues take tiles from the end), they shorten the final round.
    pl->head = std::min(pr.Do, (int)ceil_div(pr.pd, pr.sd));
  }
  pl->n_tiles = (int)ceil_div(pr.cout, pl->cfg.bn());
  pl->grid = (long long)pl->m_tiles * pl->n_tiles * pl->splits;
  // An automatic split of halo-kernel partials follows the live work.
  pl->vsplit = false;
  if (split && split_req == 0 && pl->mode == EPI_PARTIAL && pl->cfg.ns == -1 &&
      !getenv("CONV3D_UNIFORM_SPLIT"))
    plan_vsplit(pr, cc, pl);
  // Halo kernel with more tiles than CUs: persistent work-groups.
  pl->persistent = pl->cfg.ns < 0 && pl->grid > kCUs && !getenv("CONV3D_NO_PERSIST");
  if (pl->persistent) pl->grid = kCUs;

  // Workspace: NDHWC copies for NCDHW boundaries, split-K partials, tile
  // queues.
  size_t off = 0;
  pl->off_x = pl->off_y = pl->off_res = pl->off_rout = pl->off_part = pl->off_queue = 0;
  if (pr.layout == CONV3D_NCDHW) { pl->off_x = off; off = align256(off + pr.x_bytes); }
  if (pr.out_layout == CONV3D_NCDHW) {
    pl->off_y = off; off = align256(off + pr.y_bytes);
    if (pr.flags & F_RESIDUAL) { pl->off_res = off; off = align256(off + pr.y_bytes); }
    if (pr.flags & F_RESIDUAL_OUT) { pl->off_rout = off; off = align256(off + pr.y_bytes); }
  }
  if (pl->reduce) {
    // Halo-kernel partials are whole tiles in fragment order, one per
    // work-group.
    pl->off_part = off;
    if (pl->cfg.ns == -1) {
      off = align256(off + (size_t)pl->grid * pl->cfg.bm() * pl->cfg.bn() * 4);
    } else {
      off = align256(off + (size_t)pl->splits * (size_t)pr.M * (size_t)pr.cout * 4);
    }
  }
  if (pl->persistent) {
    pl->off_queue = off;
    off = align256(off + kQueueBytes);
  }
  pl->total = off;
}

// Padded-output placement (conv3d_fwd_padded).
struct PadPlan {
  bool on = false;
  long long y_bytes = 0;   // padded y
  PlaceArgs a{};
};

conv3d_status check_out_pad(const conv3d_out_pad* op, const Problem& pr, PadPlan* pp) {
  *pp = PadPlan();
  if (!op) return CONV3D_OK;
  for (int i = 0; i < 3; ++i)
    if (op->pad_lo[i] < 0 || op->pad_hi[i] < 0 || op->pad_lo[i] > 65536 || op->pad_hi[i] > 65536)
      return CONV3D_ERR_SHAPE;
  const int hist = op->history_frames;
  if (hist < 0 || hist > op->pad_lo[0]) return CONV3D_ERR_SHAPE;
  if (op->cache) {
    if (op->cache_frames < 1 || op->cache_frames > pr.Do + hist) return CONV3D_ERR_SHAPE;
    if (!aligned16(op->cache)) return CONV3D_ERR_ALIGN;
  }
  const bool padded = op->pad_lo[0] || op->pad_lo[1] || op->pad_lo[2] || op->pad_hi[0] ||
                      op->pad_hi[1] || op->pad_hi[2];
  if (!padded && !op->cache) return CONV3D_OK;
  if (pr.out_layout != CONV3D_NDHWC) return CONV3D_ERR_UNSUPPORTED;
  PlaceArgs& a = pp->a;
  a.n = pr.n; a.cout = pr.cout;
  a.Do = pr.Do; a.Ho = pr.Ho; a.Wo = pr.Wo;
  a.Dy = pr.Do + op->pad_lo[0] + op->pad_hi[0];
  a.Hy = pr.Ho + op->pad_lo[1] + op->pad_hi[1];
  a.Wy = pr.Wo + op->pad_lo[2] + op->pad_hi[2];
  a.pt = op->pad_lo[0]; a.ph = op->pad_lo[1]; a.pw = op->pad_lo[2];
  a.hist = hist;
  a.cache = (uint16_t*)op->cache;
  a.cache_frames = op->cache ? op->cache_frames : 0;
  a.cache_k = op->cache ? std::min(op->cache_frames, pr.Do) : 0;
  pp->y_bytes = prod({pr.n, a.Dy, a.Hy, a.Wy, pr.cout, 2});
  if (pp->y_bytes > kMaxTensorBytes || prod({pr.n, a.Dy, a.Hy}) > 0x7fffffffLL)
    return CONV3D_ERR_UNSUPPORTED;
  pp->on = true;
  return CONV3D_OK;
}

// Samples per pass for a call with output placement op (padded y, cache):
// pr.nb, lowered so that one pass's padded output stays in range too.
int batch_chunk(const Problem& pr, const conv3d_out_pad* op) {
  long long nb = pr.nb;
  if (op) {
    const long long dy = (long long)pr.Do + op->pad_lo[0] + op->pad_hi[0];
    const long long hy = (long long)pr.Ho + op->pad_lo[1] + op->pad_hi[1];
    const long long wy = (long long)pr.Wo + op->pad_lo[2] + op->pad_hi[2];
    const long long per = prod({dy, hy, wy, pr.cout, 2});
    if (per > 0) nb = std::min(nb, std::max(1LL, kMaxTensorBytes / per));
    if (dy * hy > 0) nb = std::min(nb, std::max(1LL, 0x7fffffffLL / (dy * hy)));
  }
  return (int)std::max(1LL, nb);
}

// The slot kernels write a padded output in place (IgemmArgs::ypad) when
// they finish the epilogue themselves; otherwise the output is staged in the
// workspace and placed by a second pass.
bool direct_pad(const Problem& pr, const Plan& pl, const PadPlan& pp) {
  return pp.on && pl.cfg.ns <= -2 && !pl.reduce && pr.M < (1LL << 24) &&
         pr.out_layout == CONV3D_NDHWC && !getenv("CONV3D_STAGED_PAD");
}

// GroupNorm planning: units, chunking and the workspace carve.
struct GnPlan {
  GroupNormArgs a;
  long long bytes;        // size of x (and y)
  size_t off_stats, total;
};

constexpr int kGnTargetGroups = 2048;   // work-groups per pass, about 8 per CU
constexpr long long kGnMaxChunk = 1 << 20;

conv3d_status plan_group_norm(const conv3d_group_norm_desc* d, GnPlan* pl) {
  if (!d) return CONV3D_ERR_NULL;
  if (d->n <= 0 || d->d <= 0 || d->h <= 0 || d->w <= 0 || d->c <= 0 || d->groups <= 0)
    return CONV3D_ERR_SHAPE;
  if (!(d->eps > 0.0f) || !isfinite(d->eps)) return CONV3D_ERR_SHAPE;
  if (d->c % d->groups) return CONV3D_ERR_SHAPE;
  if (d->c % 8) return CONV3D_ERR_ALIGN;
  if (d->c > 2048 || d->groups > 256) return CONV3D_ERR_UNSUPPORTED;
  const long long units = d->t_isolated ? prod({d->n, d->d}) : d->n;
  const long long P = prod({d->t_isolated ? 1LL : (long long)d->d, d->h, d->w});
  const long long bytes = prod({units, P, d->c, 2});
  if (bytes > (1LL << 40) || units > 0x7fffffffLL) return CONV3D_ERR_UNSUPPORTED;
  GroupNormArgs& a = pl->a;
  a = GroupNormArgs{};
  a.P = P;
  a.C = d->c;
  a.G = d->groups;
  a.cpg = d->c / d->groups;
  a.V = d->c / 8;
  a.ppi = 256 / a.V;
  const long long want = std::max(1LL, (kGnTargetGroups + units - 1) / units);
  // a chunk stays below 2^31 bytes (32-bit offsets inside the kernels)
  long long chunk = std::min((P + want - 1) / want, std::min(kGnMaxChunk, (1LL << 30) / d->c));
  chunk = (chunk + a.ppi - 1) / a.ppi * a.ppi;
  const long long chunks = (P + chunk - 1) / chunk;
  if (units * chunks > 0x7fffffffLL) return CONV3D_ERR_UNSUPPORTED;
  a.units = (int)units;
  a.chunks = (int)chunks;
  a.chunk_px = (int)chunk;
  a.eps = d->eps;
  a.silu = d->silu ? 1 : 0;
  pl->bytes = bytes;
  const size_t part = (size_t)units * chunks * a.G * 16;
  pl->off_stats = (part + 255) / 256 * 256;
  pl->total = pl->off_stats + ((size_t)units * a.G * 8 + 255) / 256 * 256;
  return CONV3D_OK;
}

// GroupNorm statistics from the conv's epilogue: the 512-slot x 128-channel
// slot plan with its plain staged store (no post-operations, NDHWC in and
// out, bf16, one pass, tiles in slot order) whose 510 stored slots span at
// most two frames.
bool gn_stats_ok(const Problem& pr, const Plan& pl) {
  const TileCfg& c = pl.cfg;
  return c.ns == -2 && c.wm == 2 && c.wn == 2 && c.pb == 8 && c.cb == 2 && pl.mode == EPI_STORE &&
         !pl.reduce && pl.splits == 1 && !pl.frame_order && pr.flags == 0 && !pr.fp8 &&
         pr.layout == CONV3D_NDHWC && pr.out_layout == CONV3D_NDHWC && pr.cout % 128 == 0 &&
         pr.nb >= pr.n && (long long)pr.Ho * (pr.Wo + 2) >= c.bm() - 2;
}

}  // namespace

extern "C" {

const char* conv3d_status_str(conv3d_status s) {
  switch (s) {
    case CONV3D_OK: return "ok";
    case CONV3D_ERR_NULL: return "required pointer is NULL";
    case CONV3D_ERR_SHAPE: return "invalid shape, stride, padding or layout";
    case CONV3D_ERR_ALIGN: return "pointer not 16-byte aligned or cin not a multiple of 8";
    case CONV3D_ERR_OVERLAP: return "an output overlaps an operand or another output";
    case CONV3D_ERR_WORKSPACE: return "workspace missing or too small";
    case CONV3D_ERR_UNSUPPORTED: return "unsupported configuration (no fallback)";
    case CONV3D_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

size_t conv3d_packed_weight_bytes(int cout, int cin) {
  if (cout <= 0 || cin <= 0) return 0;
  return (size_t)27 * ((cin + 31) / 32) * 32 * (size_t)cout * 2;
}

conv3d_status conv3d_pack_weight(const void* w_oidhw, void* w_packed, int cout, int cin,
                                 void* stream) {
  if (!w_oidhw || !w_packed) return CONV3D_ERR_NULL;
  if (cout <= 0 || cin <= 0) return CONV3D_ERR_SHAPE;
  if (!aligned16(w_oidhw) || !aligned16(w_packed)) return CONV3D_ERR_ALIGN;
  const long long in_bytes = 27LL * cout * cin * 2;
  if (overlaps(range_of(w_oidhw, in_bytes),
               range_of(w_packed, (long long)conv3d_packed_weight_bytes(cout, cin))))
    return CONV3D_ERR_OVERLAP;
  const int rc = launch_pack_weight((const uint16_t*)w_oidhw, (uint16_t*)w_packed, cout, cin, 27,
                                    stream);
  return rc ? CONV3D_ERR_HIP : CONV3D_OK;
}

size_t conv3d_packed_weight_bytes_fp8(int cout, int cin) {
  if (cout <= 0 || cin <= 0) return 0;
  return (size_t)27 * (size_t)((cin + 63) / 64 * 64) * (size_t)cout;
}

conv3d_status conv3d_pack_weight_fp8(const void* w_oidhw, void* w_packed, int cout, int cin,
                                     void* stream) {
  if (!w_oidhw || !w_packed) return CONV3D_ERR_NULL;
  if (cout <= 0 || cin <= 0) return CONV3D_ERR_SHAPE;
  if (!aligned16(w_packed)) return CONV3D_ERR_ALIGN;
  const long long in_bytes = 27LL * cout * cin;
  if (overlaps(range_of(w_oidhw, in_bytes),
               range_of(w_packed, (long long)conv3d_packed_weight_bytes_fp8(cout, cin))))
    return CONV3D_ERR_OVERLAP;
  return launch_pack_weight_fp8((const uint8_t*)w_oidhw, (uint8_t*)w_packed, cout, cin, stream)
             ? CONV3D_ERR_HIP
             : CONV3D_OK;
}

conv3d_status conv3d_pack_weight_2d(const void* w_oihw, void* w_packed, int cout, int cin,
                                    void* stream) {
  if (!w_oihw || !w_packed) return CONV3D_ERR_NULL;
  if (cout <= 0 || cin <= 0) return CONV3D_ERR_SHAPE;
  if (!aligned16(w_oihw) || !aligned16(w_packed)) return CONV3D_ERR_ALIGN;
  const long long in_bytes = 9LL * cout * cin * 2;
  if (overlaps(range_of(w_oihw, in_bytes),
               range_of(w_packed, (long long)conv3d_packed_weight_bytes(cout, cin))))
    return CONV3D_ERR_OVERLAP;
  const int rc = launch_pack_weight((const uint16_t*)w_oihw, (uint16_t*)w_packed, cout, cin, 9,
                                    stream);
  return rc ? CONV3D_ERR_HIP : CONV3D_OK;
}

conv3d_status conv3d_output_dims(const conv3d_desc* desc, int out_dhw[3]) {
  if (!out_dhw) return CONV3D_ERR_NULL;
  Problem pr;
  const conv3d_status st = check_desc(desc, &pr);
  if (st == CONV3D_ERR_NULL || st == CONV3D_ERR_SHAPE) return st;
  out_dhw[0] = pr.Do; out_dhw[1] = pr.Ho; out_dhw[2] = pr.Wo;
  return CONV3D_OK;
}

conv3d_status conv3d_workspace_bytes(const conv3d_desc* desc, const conv3d_epilogue* epi,
                                     size_t* bytes) {
  return conv3d_padded_workspace_bytes(desc, epi, nullptr, bytes);
}

conv3d_status conv3d_padded_workspace_bytes(const conv3d_desc* desc, const conv3d_epilogue* epi,
                                            const conv3d_out_pad* out_pad, size_t* bytes) {
  if (!bytes) return CONV3D_ERR_NULL;
  Problem full;
  conv3d_status st = check_desc(desc, &full);
  if (st != CONV3D_OK) return st;
  // The passes reuse one workspace: the largest of a full pass and the last,
  // shorter one (whose plan may differ).
  const int nb = batch_chunk(full, out_pad);
  const int sizes[2] = {std::min(nb, full.n), full.n % nb};
  size_t need = 0;
  for (int n : sizes) {
    if (n <= 0) continue;
    conv3d_desc ds = *desc;
    ds.n = n;
    Problem pr;
    st = check_desc(&ds, &pr);
    if (st != CONV3D_OK) return st;
    PadPlan pp;
    st = check_out_pad(out_pad, pr, &pp);
    if (st != CONV3D_OK) return st;
    pr.flags = epi ? epi->flags : 0u;
    Plan pl;
    make_plan(pr, desc->split_k, &pl);
    const bool staged = pp.on && !direct_pad(pr, pl, pp);
    need = std::max(need, staged ? pl.total + align256(pr.y_bytes) : pl.total);
  }
  *bytes = need;
  return CONV3D_OK;
}

conv3d_status conv3d_plan_describe(const conv3d_desc* desc, const conv3d_epilogue* epi,
                                   char* buf, size_t len) {
  Problem full;
  conv3d_status st = check_desc(desc, &full);
  if (st != CONV3D_OK) return st;
  conv3d_desc ds = *desc;   // (the plan of a full pass when the batch runs in passes)
  ds.n = full.nb;
  Problem pr;
  st = check_desc(&ds, &pr);
  if (st != CONV3D_OK) return st;
  const int passes = (full.n + full.nb - 1) / full.nb;
  pr.flags = epi ? epi->flags : 0u;
  Plan pl;
  make_plan(pr, desc->split_k, &pl);
  if (buf && len) {
    static const char* names[] = {"store", "norm", "partial"};
    snprintf(buf, len,
             "igemm mfma=%d wm=%d wn=%d pb=%d cb=%d kb=%d ns=%d bm=%d bn=%d mode=%s splits=%d "
             "steps=%d m_tiles=%d n_tiles=%d grid=%lld persistent=%d reduce=%d workspace=%zu%s%s",
             pl.cfg.r, pl.cfg.wm, pl.cfg.wn, pl.cfg.pb, pl.cfg.cb, pl.cfg.kb, pl.cfg.ns, pl.cfg.bm(),
             pl.cfg.bn(), names[pl.mode], pl.splits, pl.steps, pl.m_tiles, pl.n_tiles, pl.grid,
             (int)pl.persistent,
             (int)pl.reduce, pl.total, pl.vsplit ? " split=live" : "",
             pl.frame_order ? " order=frame" : "");
    if (passes > 1) {
      const size_t used = strlen(buf);
      if (used + 1 < len)
        snprintf(buf + used, len - used, " passes=%d samples_per_pass=%d", passes, full.nb);
    }
  }
  return CONV3D_OK;
}

conv3d_status conv3d_fwd(const conv3d_desc* desc, const void* x, const void* w_packed,
                         const conv3d_epilogue* epi, void* y, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return conv3d_fwd_padded(desc, x, w_packed, epi, nullptr, y, workspace, workspace_bytes, stream);
}

conv3d_status conv3d_fwd_noalloc(const conv3d_desc* desc, const void* x, const void* w_packed,
                                 const conv3d_epilogue* epi, void* y, void* stream) {
  size_t need = 0;
  const conv3d_status st = conv3d_workspace_bytes(desc, epi, &need);
  if (st != CONV3D_OK) return st;
  if (!x || !w_packed || !y) return CONV3D_ERR_NULL;
  if (need > kScratchBytes) return CONV3D_ERR_WORKSPACE;   // beyond the fixed scratch
  void* ws = nullptr;
  if (need > 0 && scratch_address(&ws) != 0) return CONV3D_ERR_HIP;
  return conv3d_fwd(desc, x, w_packed, epi, y, ws, need > 0 ? kScratchBytes : 0, stream);
}

static conv3d_status fwd_padded_pass(const conv3d_desc* desc, const void* x, const void* w_packed,
                                     const conv3d_epilogue* epi, const conv3d_out_pad* op, void* y,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     float* gn_partials);

conv3d_status conv3d_gn_partials_bytes(const conv3d_desc* desc, size_t* bytes) {
  if (!bytes) return CONV3D_ERR_NULL;
  *bytes = 0;
  Problem pr;
  const conv3d_status st = check_desc(desc, &pr);
  if (st != CONV3D_OK) return st;
  Plan pl;
  make_plan(pr, desc->split_k, &pl);
  if (!gn_stats_ok(pr, pl)) return CONV3D_ERR_UNSUPPORTED;
  *bytes = 512ull * pl.m_tiles * pl.n_tiles;
  return CONV3D_OK;
}

conv3d_status conv3d_fwd_gn_stats(const conv3d_desc* desc, const void* x, const void* w_packed,
                                  void* y, void* gn_partials, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!gn_partials) return CONV3D_ERR_NULL;
  return fwd_padded_pass(desc, x, w_packed, nullptr, nullptr, y, workspace, workspace_bytes, stream,
                         (float*)gn_partials);
}

// One pass: every tensor within the 32-bit buffer range (nb == n).
static conv3d_status fwd_padded_pass(const conv3d_desc* desc, const void* x, const void* w_packed,
                                     const conv3d_epilogue* epi, const conv3d_out_pad* op, void* y,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     float* gn_partials) {
  Problem pr;
  conv3d_status st = check_desc(desc, &pr);
  if (st != CONV3D_OK) return st;
  if (pr.nb < pr.n || batch_chunk(pr, op) < pr.n) return CONV3D_ERR_UNSUPPORTED;
  if (!x || !w_packed || !y) return CONV3D_ERR_NULL;
  st = check_epi(epi, &pr);
  if (st != CONV3D_OK) return st;
  if (!aligned16(x) || !aligned16(w_packed) || !aligned16(y)) return CONV3D_ERR_ALIGN;

  // Output placement: padded y and / or frame cache.
  PadPlan pp;
  st = check_out_pad(op, pr, &pp);
  if (st != CONV3D_OK) return st;
  Plan pl;
  make_plan(pr, desc->split_k, &pl);
  if (gn_partials && (pp.on || !gn_stats_ok(pr, pl))) return CONV3D_ERR_UNSUPPORTED;
  if (gn_partials && ((uintptr_t)gn_partials & 15)) return CONV3D_ERR_ALIGN;
  const bool direct = direct_pad(pr, pl, pp);
  const size_t off_stage = pl.total;                     // staged unpadded output
  const size_t ws_total = pp.on && !direct ? off_stage + align256(pr.y_bytes) : pl.total;
  if (ws_total > 0) {
    if (!workspace || workspace_bytes < ws_total) return CONV3D_ERR_WORKSPACE;
    if (!aligned16(workspace)) return CONV3D_ERR_ALIGN;
  }

  // Outputs (y, residual_out, workspace) must not overlap any operand or
  // each other.
  const unsigned f = pr.flags;
  const Range rx = range_of(x, pr.x_bytes);
  const Range rw = range_of(w_packed, (long long)packed_bytes(pr));
  const Range ry = range_of(y, pp.on ? pp.y_bytes : pr.y_bytes);
  const Range rcache = pp.a.cache ? range_of(pp.a.cache, prod({pr.n, pp.a.cache_frames, pr.Ho, pr.Wo, pr.cout, 2}))
                                  : Range();
  const Range rb = (f & F_BIAS) ? range_of(epi->bias, 4LL * pr.cout) : Range();
  const Range rr = (f & F_RESIDUAL) ? range_of(epi->residual, pr.y_bytes) : Range();
  const Range rg = (f & F_NORM) ? range_of(epi->gamma, 2LL * pr.cout) : Range();
  const Range ro = (f & F_RESIDUAL_OUT) ? range_of(epi->residual_out, pr.y_bytes) : Range();
  const Range rs = range_of(workspace, (long long)ws_total);
  const Range rgn = gn_partials ? range_of(gn_partials, 512LL * pl.m_tiles * pl.n_tiles) : Range();
  const Range outs[] = {ry, ro, rs, rcache, rgn};
  const Range ins[] = {rx, rw, rb, rr, rg};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlaps(o, i)) return CONV3D_ERR_OVERLAP;
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(outs[i], outs[j])) return CONV3D_ERR_OVERLAP;

  char* ws = (char*)workspace;
  const uint16_t* xin = (const uint16_t*)x;
  uint16_t* yout = pp.on && !direct ? (uint16_t*)(ws + off_stage) : (uint16_t*)y;
  const uint16_t* res = (f & F_RESIDUAL) ? (const uint16_t*)epi->residual : nullptr;
  uint16_t* rout = (f & F_RESIDUAL_OUT) ? (uint16_t*)epi->residual_out : nullptr;
  const int S = pr.d * pr.h * pr.w;
  const int So = pr.Do * pr.Ho * pr.Wo;

  if (pr.layout == CONV3D_NCDHW) {
    uint16_t* xt = (uint16_t*)(ws + pl.off_x);
    if (launch_transpose(xin, xt, pr.n, pr.cin, S, stream)) return CONV3D_ERR_HIP;
    xin = xt;
  }
  if (pr.out_layout == CONV3D_NCDHW) {
    yout = (uint16_t*)(ws + pl.off_y);
    if (res) {
      uint16_t* rt = (uint16_t*)(ws + pl.off_res);
      if (launch_transpose(res, rt, pr.n, pr.cout, So, stream)) return CONV3D_ERR_HIP;
      res = rt;
    }
    if (rout) rout = (uint16_t*)(ws + pl.off_rout);
  }

  IgemmArgs a;
  memset(&a, 0, sizeof a);
  a.x = xin;
  a.wp = (const uint16_t*)w_packed;
  a.y = yout;
  a.partial = pl.reduce ? (float*)(ws + pl.off_part) : nullptr;
  a.bias = (f & F_BIAS) ? epi->bias : nullptr;
  a.residual = res;
  a.gamma = (f & F_NORM) ? (const uint16_t*)epi->gamma : nullptr;
  a.residual_out = rout;
  a.N = pr.n; a.D = pr.d; a.H = pr.h; a.W = pr.w; a.Cin = pr.cin; a.Cout = pr.cout;
  a.Do = pr.Do; a.Ho = pr.Ho; a.Wo = pr.Wo;
  a.sd = pr.sd; a.sh = pr.sh; a.sw = pr.sw;
  a.pd = pr.pd; a.ph = pr.ph; a.pw = pr.pw;
  a.CC = k_chunks(pr);
  a.M = (int)pr.M;
  a.m_tiles = pl.m_tiles; a.n_tiles = pl.n_tiles; a.splits = pl.splits;
  a.steps_per_split = pl.steps_per_split;
  a.flags = pl.reduce ? 0u : f;
  a.x_bytes = (unsigned)pr.x_bytes;
  a.sqrt_c = sqrtf((float)pr.cout);
  a.inv_ho = 1.0f / (float)pr.Ho;
  a.inv_do = 1.0f / (float)pr.Do;
  a.inv_wp = 1.0f / (float)(pr.Wo + 2);
  a.inv_wo = 1.0f / (float)pr.Wo;
  if (direct) {   // the padded output written in place
    a.ypad = 1;
    a.yDy = pp.a.Dy; a.yHy = pp.a.Hy; a.yWy = pp.a.Wy;
    a.ypt = pp.a.pt; a.yph = pp.a.ph; a.ypw = pp.a.pw;
  }
  if (pl.cfg.ns == -3) {   // the pixel-pair view (stride 2 along W)
    const Problem v = pair_view(pr);
    a.W = v.w; a.Cin = v.cin; a.sw = v.sw; a.pw = v.pw;
    a.CC = 2 * k_chunks(pr);
    a.inv_wp = 1.0f / (float)(pr.Wo + 1);
  }
  if (pl.frame_order) {
    a.frames = pr.n * pr.Do;
    a.frame_slots = pl.frame_slots;
    a.frame_tiles = pl.frame_tiles;
    a.head = pl.head;
  }
  if (pl.vsplit) {
    a.vsplit = 1;
    a.per_n = pl.per_n;
    // Work-group b runs launch position xcd_run(b) (the device's XCD
    // mapping: XCD b % 8 takes a contiguous run of positions); position
    // nt * per_n + i computes slice wg[i] & 255 of pixel tile wg[i] >> 8 of
    // channel tile nt.
    const int grid = (int)pl.grid, G8 = grid & ~7;
    if (grid > kMaxVWG) return CONV3D_ERR_UNSUPPORTED;
    for (int b = 0; b < grid; ++b) {
      const int bid = b < G8 ? (b & 7) * (G8 >> 3) + (b >> 3) : b;
      const int nt = bid / pl.per_n, i = bid - nt * pl.per_n;
      const int mt = pl.wg[i] >> 8, sl = pl.wg[i] & 255;
      const int ns = pl.split_base[mt + 1] - pl.split_base[mt];
      const int slot = nt * pl.per_n + pl.split_base[mt] + sl;
      a.vwg[b] = (uint64_t)mt | ((uint64_t)nt << 16) | ((uint64_t)sl << 32) | ((uint64_t)ns << 40) |
                 ((uint64_t)slot << 48);
    }
  }
  if (pl.grid > 0x7fffffffLL) return CONV3D_ERR_UNSUPPORTED;
  if (pl.persistent) {
    const long long T = (long long)pl.m_tiles * pl.n_tiles * pl.splits;
    a.queue_tail = tail_tiles((int)T);
    // (development override of the shared tail's size, for A/B timing)
    if (const char* env = getenv("CONV3D_QUEUE_TAIL"))
      a.queue_tail = std::max(0, std::min((int)T, atoi(env)));
    a.queue = (unsigned*)(ws + pl.off_queue);
    if (launch_queue_reset(a.queue, stream)) return CONV3D_ERR_HIP;
  }
  a.gnp = gn_partials;
  const int rc = launch_igemm(pl.cfg, gn_partials ? (int)EPI_STATS : pl.mode, pr.reflect, pr.fp8, a,
                              (int)pl.grid, stream);
  if (rc) return rc < 0 ? CONV3D_ERR_UNSUPPORTED : CONV3D_ERR_HIP;

  if (pl.reduce) {
    ReduceArgs r;
    r.partial = a.partial;
    r.y = yout;
    r.bias = a.bias;
    r.residual = res;
    r.gamma = a.gamma;
    r.residual_out = rout;
    r.M = (int)pr.M;
    r.Cout = pr.cout;
    r.splits = pl.splits;
    r.flags = f;
    r.sqrt_c = a.sqrt_c;
    r.frag = pl.cfg.ns == -1;
    r.m_tiles = pl.m_tiles;
    r.n_tiles = pl.n_tiles;
    r.wm = pl.cfg.wm;
    r.pb = pl.cfg.pb;
    r.cb = pl.cfg.cb;
    r.vsplit = pl.vsplit ? 1 : 0;
    r.per_n = pl.per_n;
    memcpy(r.split_base, pl.split_base, sizeof r.split_base);
    if (launch_reduce(r, stream)) return CONV3D_ERR_HIP;
  }
  if (pp.on) {   // borders, history planes and cache (and the interior when staged)
    PlaceArgs pa = pp.a;
    pa.y0 = direct ? nullptr : yout;
    pa.y = (uint16_t*)y;
    if (launch_place(pa, stream)) return CONV3D_ERR_HIP;
  }

  if (pr.out_layout == CONV3D_NCDHW) {
    if (launch_transpose(yout, (uint16_t*)y, pr.n, So, pr.cout, stream)) return CONV3D_ERR_HIP;
    if (rout && launch_transpose(rout, (uint16_t*)epi->residual_out, pr.n, So, pr.cout, stream))
      return CONV3D_ERR_HIP;
  }
  return CONV3D_OK;
}

conv3d_status conv3d_fwd_padded(const conv3d_desc* desc, const void* x, const void* w_packed,
                                const conv3d_epilogue* epi, const conv3d_out_pad* op, void* y,
                                void* workspace, size_t workspace_bytes, void* stream) {
  Problem pr;
  conv3d_status st = check_desc(desc, &pr);
  if (st != CONV3D_OK) return st;
  const int nb = batch_chunk(pr, op);
  if (nb >= pr.n)
    return fwd_padded_pass(desc, x, w_packed, epi, op, y, workspace, workspace_bytes, stream,
                           nullptr);

  // A batch beyond the 32-bit buffer range: passes over nb consecutive
  // samples, in order on the stream, reusing the workspace. Each pass checks
  // its own slices; the whole tensors are checked for overlap here.
  if (!x || !w_packed || !y) return CONV3D_ERR_NULL;
  st = check_epi(epi, &pr);
  if (st != CONV3D_OK) return st;
  const unsigned f = pr.flags;
  const long long xs = prod({pr.d, pr.h, pr.w, pr.cin, pr.fp8 ? 1 : 2});
  const long long rs = prod({pr.Do, pr.Ho, pr.Wo, pr.cout, 2});
  long long ys = rs, cs = 0;
  if (op) {
    PadPlan pp;
    conv3d_desc d1 = *desc;
    d1.n = 1;
    Problem p1;
    st = check_desc(&d1, &p1);
    if (st != CONV3D_OK) return st;
    st = check_out_pad(op, p1, &pp);
    if (st != CONV3D_OK) return st;
    if (pp.on) ys = pp.y_bytes;
    if (op->cache) cs = prod({op->cache_frames, pr.Ho, pr.Wo, pr.cout, 2});
  }
  size_t ws_need = 0;
  st = conv3d_padded_workspace_bytes(desc, epi, op, &ws_need);
  if (st != CONV3D_OK) return st;
  const Range rx = range_of(x, prod({pr.n, xs}));
  const Range rw = range_of(w_packed, (long long)packed_bytes(pr));
  const Range ry = range_of(y, prod({pr.n, ys}));
  const Range rcache = (op && op->cache) ? range_of(op->cache, prod({pr.n, cs})) : Range();
  const Range rb = (f & F_BIAS) ? range_of(epi->bias, 4LL * pr.cout) : Range();
  const Range rr = (f & F_RESIDUAL) ? range_of(epi->residual, prod({pr.n, rs})) : Range();
  const Range rg = (f & F_NORM) ? range_of(epi->gamma, 2LL * pr.cout) : Range();
  const Range ro = (f & F_RESIDUAL_OUT) ? range_of(epi->residual_out, prod({pr.n, rs})) : Range();
  const Range rs_ = range_of(workspace, (long long)ws_need);
  const Range outs[] = {ry, ro, rs_, rcache};
  const Range ins[] = {rx, rw, rb, rr, rg};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlaps(o, i)) return CONV3D_ERR_OVERLAP;
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs[j])) return CONV3D_ERR_OVERLAP;
  for (int b0 = 0; b0 < pr.n; b0 += nb) {
    conv3d_desc ds = *desc;
    ds.n = std::min(nb, pr.n - b0);
    conv3d_epilogue es;
    if (epi) {
      es = *epi;
      if (f & F_RESIDUAL) es.residual = (const char*)epi->residual + b0 * rs;
      if (f & F_RESIDUAL_OUT) es.residual_out = (char*)epi->residual_out + b0 * rs;
    }
    conv3d_out_pad os;
    if (op) {
      os = *op;
      if (op->cache) os.cache = (char*)op->cache + b0 * cs;
    }
    st = fwd_padded_pass(&ds, (const char*)x + b0 * xs, w_packed, epi ? &es : nullptr,
                         op ? &os : nullptr, (char*)y + b0 * ys, workspace, workspace_bytes, stream,
                         nullptr);
    if (st != CONV3D_OK) return st;
  }
  return CONV3D_OK;
}

conv3d_status conv3d_norm_silu(const void* x, int n, int d, int h, int w, int c,
                               const conv3d_epilogue* epi, const conv3d_out_pad* op,
                               const void* previous, void* y, void* stream) {
  if (!x || !y || !epi) return CONV3D_ERR_NULL;
  if (n <= 0 || d <= 0 || h <= 0 || w <= 0 || c <= 0) return CONV3D_ERR_SHAPE;
  const unsigned f = epi->flags;
  if (!(f & F_NORM) || (f & ~(F_BIAS | F_RESIDUAL | F_NORM | F_RESIDUAL_OUT)))
    return CONV3D_ERR_UNSUPPORTED;
  if (!epi->gamma || ((f & F_BIAS) && !epi->bias) || ((f & F_RESIDUAL) && !epi->residual) ||
      ((f & F_RESIDUAL_OUT) && !epi->residual_out))
    return CONV3D_ERR_NULL;
  if (c % 8) return CONV3D_ERR_ALIGN;
  if (c > 2048) return CONV3D_ERR_UNSUPPORTED;
  const long long M = prod({n, d, h, w});
  const long long bytes = prod({M, c, 2});
  if (bytes > kMaxTensorBytes) return CONV3D_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y) || !aligned16(epi->gamma) ||
      ((f & F_RESIDUAL) && !aligned16(epi->residual)) ||
      ((f & F_RESIDUAL_OUT) && !aligned16(epi->residual_out)) ||
      ((f & F_BIAS) && ((uintptr_t)epi->bias & 3)))
    return CONV3D_ERR_ALIGN;
  // placement: the conv's padded-output rules with (Do, Ho, Wo) = (d, h, w)
  Problem pr;
  memset(&pr, 0, sizeof pr);
  pr.n = n; pr.Do = d; pr.Ho = h; pr.Wo = w; pr.cout = c;
  pr.out_layout = CONV3D_NDHWC;
  PadPlan pp;
  conv3d_status st = check_out_pad(op, pr, &pp);
  if (st != CONV3D_OK) return st;
  if (previous) {
    if (!op || op->history_frames < 1) return CONV3D_ERR_SHAPE;
    if (!aligned16(previous)) return CONV3D_ERR_ALIGN;
    if (op->cache && op->cache_frames - std::min(op->cache_frames, d) > op->history_frames)
      return CONV3D_ERR_SHAPE;   // older cache frames must come from previous
  }
  const long long y_bytes = pp.on ? pp.y_bytes : bytes;
  const Range rx = range_of(x, bytes), ry = range_of(y, y_bytes);
  const Range rr = (f & F_RESIDUAL) ? range_of(epi->residual, bytes) : Range();
  const Range ro = (f & F_RESIDUAL_OUT) ? range_of(epi->residual_out, bytes) : Range();
  const Range rg = range_of(epi->gamma, 2LL * c);
  const Range rb = (f & F_BIAS) ? range_of(epi->bias, 4LL * c) : Range();
  const Range rp = previous ? range_of(previous, prod({n, op->history_frames, h, w, c, 2}))
                            : Range();
  const Range rc = pp.a.cache ? range_of(pp.a.cache, prod({n, pp.a.cache_frames, h, w, c, 2}))
                              : Range();
  const Range outs[] = {ry, ro, rc};
  for (const Range& o : outs)
    for (const Range& i : {rx, rr, rg, rb, rp})
      if (overlaps(o, i)) return CONV3D_ERR_OVERLAP;
  if (overlaps(ry, ro) || overlaps(ry, rc) || overlaps(ro, rc)) return CONV3D_ERR_OVERLAP;

  NormSiluArgs a;
  memset(&a, 0, sizeof a);
  a.x = (const uint16_t*)x;
  a.bias = (f & F_BIAS) ? epi->bias : nullptr;
  a.residual = (f & F_RESIDUAL) ? (const uint16_t*)epi->residual : nullptr;
  a.gamma = (const uint16_t*)epi->gamma;
  a.residual_out = (f & F_RESIDUAL_OUT) ? (uint16_t*)epi->residual_out : nullptr;
  a.y = (uint16_t*)y;
  a.flags = f;
  a.M = (int)M;
  a.C = c;
  a.sqrt_c = sqrtf((float)c);
  if (pp.on) {
    a.geo = pp.a;
    a.geo.previous = (const uint16_t*)previous;
  }
  if (launch_norm_silu(a, stream)) return CONV3D_ERR_HIP;
  if (pp.on) {
    PlaceArgs pa = a.geo;
    pa.y0 = nullptr;
    pa.y = (uint16_t*)y;
    if (launch_place(pa, stream)) return CONV3D_ERR_HIP;
  }
  return CONV3D_OK;
}

conv3d_status conv3d_stream_pack_input(const void* chunk, const long long strides[5], int n,
                                       int c, int t, int h, int w, const void* history,
                                       int history_frames, void* padded, int c_pad, void* cache,
                                       int cache_frames, void* stream) {
  if (!chunk || !strides || !padded) return CONV3D_ERR_NULL;
  if (history_frames > 0 && !history) return CONV3D_ERR_NULL;
  if (n <= 0 || c <= 0 || t <= 0 || h <= 0 || w <= 0) return CONV3D_ERR_SHAPE;
  if (history_frames < 0 || history_frames > 2 || c_pad < c) return CONV3D_ERR_SHAPE;
  for (int i = 0; i < 5; ++i)
    if (strides[i] < 0) return CONV3D_ERR_SHAPE;
  if (cache && (cache_frames < 1 || cache_frames > t + history_frames)) return CONV3D_ERR_SHAPE;
  if (c_pad % 8) return CONV3D_ERR_ALIGN;
  if (!aligned16(padded) || ((uintptr_t)chunk & 1) || ((uintptr_t)history & 1) ||
      ((uintptr_t)cache & 1))
    return CONV3D_ERR_ALIGN;
  const long long padded_bytes = prod({n, t + 2LL, h + 2LL, w + 2LL, c_pad, 2});
  if (padded_bytes > kMaxTensorBytes) return CONV3D_ERR_UNSUPPORTED;
  const long long dims[5] = {n, c, t, h, w};
  long long last = 0;
  for (int i = 0; i < 5; ++i) last += (dims[i] - 1) * strides[i];
  const Range rchunk = range_of(chunk, (last + 1) * 2);
  const Range rhist = range_of(history, prod({n, history_frames, h, w, c, 2}));
  const Range rpad = range_of(padded, padded_bytes);
  const Range rcache = cache ? range_of(cache, prod({n, cache_frames, h, w, c, 2})) : Range();
  for (const Range& o : {rpad, rcache})
    for (const Range& i : {rchunk, rhist})
      if (overlaps(o, i)) return CONV3D_ERR_OVERLAP;
  if (overlaps(rpad, rcache)) return CONV3D_ERR_OVERLAP;
  StreamPackArgs a;
  a.chunk = (const uint16_t*)chunk;
  a.sn = strides[0]; a.sc = strides[1]; a.st = strides[2]; a.sh = strides[3]; a.sw = strides[4];
  a.history = (const uint16_t*)history;
  a.padded = (uint16_t*)padded;
  a.cache = (uint16_t*)cache;
  a.n = n; a.c = c; a.t = t; a.h = h; a.w = w;
  a.P = history_frames;
  a.c_pad = c_pad;
  a.cache_frames = cache ? cache_frames : 0;
  return launch_stream_pack(a, stream) ? CONV3D_ERR_HIP : CONV3D_OK;
}

conv3d_status conv3d_group_norm_workspace_bytes(const conv3d_group_norm_desc* desc,
                                                size_t* bytes) {
  if (!bytes) return CONV3D_ERR_NULL;
  GnPlan pl;
  const conv3d_status st = plan_group_norm(desc, &pl);
  if (st != CONV3D_OK) return st;
  *bytes = pl.total;
  return CONV3D_OK;
}

conv3d_status conv3d_group_norm(const conv3d_group_norm_desc* desc, const void* x,
                                const float* gamma, const float* beta, void* y,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!desc || !x || !gamma || !beta || !y) return CONV3D_ERR_NULL;
  GnPlan pl;
  const conv3d_status st = plan_group_norm(desc, &pl);
  if (st != CONV3D_OK) return st;
  if (!aligned16(x) || !aligned16(y) || !aligned16(gamma) || !aligned16(beta))
    return CONV3D_ERR_ALIGN;
  if (!workspace || workspace_bytes < pl.total) return CONV3D_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CONV3D_ERR_ALIGN;
  const Range rx = range_of(x, pl.bytes), ry = range_of(y, pl.bytes);
  const Range rg = range_of(gamma, (long long)desc->c * 4), rb = range_of(beta, (long long)desc->c * 4);
  const Range rw = range_of(workspace, (long long)pl.total);
  if (x != y && overlaps(rx, ry)) return CONV3D_ERR_OVERLAP;
  for (const Range& o : {ry, rw})
    for (const Range& i : {rg, rb})
      if (overlaps(o, i)) return CONV3D_ERR_OVERLAP;
  if (overlaps(rw, rx) || overlaps(rw, ry)) return CONV3D_ERR_OVERLAP;
  GroupNormArgs a = pl.a;
  a.x = (const uint16_t*)x;
  a.y = (uint16_t*)y;
  a.gamma = gamma;
  a.beta = beta;
  a.partial = (double*)workspace;
  a.stats = (float*)((char*)workspace + pl.off_stats);
  return launch_group_norm(a, stream) ? CONV3D_ERR_HIP : CONV3D_OK;
}

conv3d_status conv3d_group_norm_from_partials(const conv3d_group_norm_desc* desc,
                                             const conv3d_desc* conv, const void* gn_partials,
                                             const void* x, const float* gamma, const float* beta,
                                             void* y, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (!desc || !conv || !gn_partials || !x || !gamma || !beta || !y) return CONV3D_ERR_NULL;
  GnPlan gp;
  conv3d_status st = plan_group_norm(desc, &gp);
  if (st != CONV3D_OK) return st;
  Problem pr;
  st = check_desc(conv, &pr);
  if (st != CONV3D_OK) return st;
  Plan pl;
  make_plan(pr, conv->split_k, &pl);
  if (!gn_stats_ok(pr, pl)) return CONV3D_ERR_UNSUPPORTED;
  if (desc->n != pr.n || desc->d != pr.Do || desc->h != pr.Ho || desc->w != pr.Wo ||
      desc->c != pr.cout)
    return CONV3D_ERR_SHAPE;
  const int cpg = desc->c / desc->groups;
  if (cpg % 4 || 128 % cpg) return CONV3D_ERR_UNSUPPORTED;   // whole subgroups of one channel tile
  if (!aligned16(x) || !aligned16(y) || !aligned16(gamma) || !aligned16(beta) ||
      !aligned16(gn_partials))
    return CONV3D_ERR_ALIGN;
  if (!workspace || workspace_bytes < gp.total) return CONV3D_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CONV3D_ERR_ALIGN;
  const Range rx = range_of(x, gp.bytes), ry = range_of(y, gp.bytes);
  const Range rg = range_of(gamma, (long long)desc->c * 4), rb = range_of(beta, (long long)desc->c * 4);
  const Range rp = range_of(gn_partials, 512LL * pl.m_tiles * pl.n_tiles);
  const Range rw = range_of(workspace, (long long)gp.total);
  if (x != y && overlaps(rx, ry)) return CONV3D_ERR_OVERLAP;
  for (const Range& o : {ry, rw})
    for (const Range& i : {rg, rb, rp})
      if (overlaps(o, i)) return CONV3D_ERR_OVERLAP;
  if (overlaps(rw, rx) || overlaps(rw, ry)) return CONV3D_ERR_OVERLAP;
  GroupNormArgs a = gp.a;
  a.x = (const uint16_t*)x;
  a.y = (uint16_t*)y;
  a.gamma = gamma;
  a.beta = beta;
  a.partial = nullptr;
  a.stats = (float*)((char*)workspace + gp.off_stats);
  GnTileArgs t;
  t.part = (const float*)gn_partials;
  t.n_ctiles = pl.n_tiles;
  t.TS = pl.cfg.bm() - 2;
  t.WP = pr.Wo + 2;
  t.Ho = pr.Ho;
  t.frames_per_unit = desc->t_isolated ? 1 : pr.Do;
  return launch_group_norm_tiles(a, t, stream) ? CONV3D_ERR_HIP : CONV3D_OK;
}

conv3d_status conv3d_transpose(const void* src, int src_layout, void* dst, int n, int c, int d,
                               int h, int w, void* stream) {
  if (!src || !dst) return CONV3D_ERR_NULL;
  if (n <= 0 || c <= 0 || d <= 0 || h <= 0 || w <= 0) return CONV3D_ERR_SHAPE;
  if (src_layout != CONV3D_NCDHW && src_layout != CONV3D_NDHWC) return CONV3D_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return CONV3D_ERR_ALIGN;
  const long long s = prod({d, h, w});
  const long long bytes = prod({n, c, s, 2});
  if (s > 0x7fffffffLL || bytes > (1LL << 40)) return CONV3D_ERR_UNSUPPORTED;
  if (overlaps(range_of(src, bytes), range_of(dst, bytes))) return CONV3D_ERR_OVERLAP;
  const int rc = (src_layout == CONV3D_NCDHW)
                     ? launch_transpose((const uint16_t*)src, (uint16_t*)dst, n, c, (int)s, stream)
                     : launch_transpose((const uint16_t*)src, (uint16_t*)dst, n, (int)s, c, stream);
  return rc ? CONV3D_ERR_HIP : CONV3D_OK;
}

}  // extern "C"
