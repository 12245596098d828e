// Exercises every C entry point's host path (checks, planning, workspace
// carving, dispatch) under AddressSanitizer and UndefinedBehaviorSanitizer,
// linked with stub_launchers.cpp instead of the HIP kernels. Device
// pointers are fake, aligned and far apart; the stubs never dereference
// them. Prints "api driver ok" and exits 0 when every expectation holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>

#include "../../include/conv3d.h"

namespace conv3d {
extern int g_launches;
}

static int g_fail = 0;

#define EXPECT(expr, want)                                                              \
  do {                                                                                  \
    const int got_ = (int)(expr);                                                       \
    if (got_ != (int)(want)) {                                                          \
      fprintf(stderr, "%s:%d: %s = %d, want %d\n", __FILE__, __LINE__, #expr, got_,    \
              (int)(want));                                                             \
      ++g_fail;                                                                         \
    }                                                                                   \
  } while (0)

// Fake device buffer k: 16 GiB apart, 256-byte aligned.
static void* buf(int k) { return (void*)(uintptr_t)((uint64_t)(k + 1) << 34); }

static conv3d_desc make(int n, int d, int h, int w, int cin, int cout, int pd, int ph, int pw,
                        int qd, int qh, int qw, int sd = 1, int sh = 1, int sw = 1) {
  conv3d_desc c;
  memset(&c, 0, sizeof c);
  c.n = n; c.d = d; c.h = h; c.w = w; c.cin = cin; c.cout = cout;
  c.stride[0] = sd; c.stride[1] = sh; c.stride[2] = sw;
  c.pad_lo[0] = pd; c.pad_lo[1] = ph; c.pad_lo[2] = pw;
  c.pad_hi[0] = qd; c.pad_hi[1] = qh; c.pad_hi[2] = qw;
  c.layout = CONV3D_NDHWC;
  c.out_layout = CONV3D_NDHWC;
  return c;
}

// A valid call of conv3d_fwd / conv3d_fwd_padded for desc and epilogue flags.
static void run_ok(conv3d_desc d, unsigned flags, const conv3d_out_pad* op = nullptr) {
  conv3d_epilogue e;
  memset(&e, 0, sizeof e);
  e.flags = flags;
  e.bias = (const float*)buf(10);
  e.residual = buf(11);
  e.gamma = buf(12);
  e.residual_out = buf(13);
  size_t ws = 0;
  char plan[512];
  EXPECT(conv3d_plan_describe(&d, flags ? &e : nullptr, plan, sizeof plan), CONV3D_OK);
  if (op) {
    EXPECT(conv3d_padded_workspace_bytes(&d, flags ? &e : nullptr, op, &ws), CONV3D_OK);
    EXPECT(conv3d_fwd_padded(&d, buf(1), buf(2), flags ? &e : nullptr, op, buf(3), buf(4), ws,
                             nullptr), CONV3D_OK);
    if (ws) {
      EXPECT(conv3d_fwd_padded(&d, buf(1), buf(2), flags ? &e : nullptr, op, buf(3), buf(4),
                               ws - 1, nullptr), CONV3D_ERR_WORKSPACE);
    }
  } else {
    EXPECT(conv3d_workspace_bytes(&d, flags ? &e : nullptr, &ws), CONV3D_OK);
    const int before = conv3d::g_launches;
    EXPECT(conv3d_fwd(&d, buf(1), buf(2), flags ? &e : nullptr, buf(3), buf(4), ws, nullptr),
           CONV3D_OK);
    if (conv3d::g_launches == before) {
      fprintf(stderr, "no launch for a valid call (%s)\n", plan);
      ++g_fail;
    }
    if (ws) {
      const int n0 = conv3d::g_launches;
      EXPECT(conv3d_fwd(&d, buf(1), buf(2), flags ? &e : nullptr, buf(3), buf(4), ws - 1,
                        nullptr), CONV3D_ERR_WORKSPACE);
      EXPECT(conv3d::g_launches, n0);   // a failing call launches nothing
    }
  }
}

int main() {
  for (int s = 0; s <= 8; ++s)
    if (!conv3d_status_str((conv3d_status)s)) ++g_fail;

  // The layer shapes of the workloads, every epilogue, several K splits.
  const conv3d_desc layers[] = {
      make(1, 5, 16, 16, 64, 64, 2, 1, 1, 0, 1, 1),
      make(1, 5, 16, 16, 1024, 1024, 2, 1, 1, 0, 1, 1),
      make(1, 5, 16, 16, 512, 1024, 2, 1, 1, 0, 1, 1),
      make(1, 17, 256, 256, 128, 128, 2, 1, 1, 0, 1, 1),
      make(1, 17, 256, 256, 128, 128, 2, 0, 0, 0, 1, 1, 1, 2, 2),
      make(1, 6, 354, 642, 96, 96, 0, 0, 0, 0, 0, 0),
      make(1, 3, 46, 82, 384, 384, 0, 0, 0, 0, 0, 0),
      make(1, 1, 1024, 1024, 96, 96, 2, 1, 1, 0, 1, 1),
      make(1, 7, 66, 122, 160, 320, 0, 0, 0, 0, 0, 0),
      make(2, 3, 7, 9, 40, 48, 2, 1, 1, 0, 1, 1),
      make(1, 9, 12, 12, 64, 64, 2, 1, 1, 0, 1, 1, 2, 2, 2),
      make(1, 1, 1, 1, 8, 16, 2, 1, 1, 0, 1, 1),
  };
  const unsigned epis[] = {0u, CONV3D_EPI_BIAS, CONV3D_EPI_BIAS | CONV3D_EPI_RESIDUAL,
                           CONV3D_EPI_BIAS | CONV3D_EPI_RESIDUAL | CONV3D_EPI_L2NORM_SILU |
                               CONV3D_EPI_RESIDUAL_OUT};
  for (const conv3d_desc& base : layers) {
    for (unsigned f : epis) {
      if ((f & CONV3D_EPI_L2NORM_SILU) && base.cout > 2048) continue;
      for (int sk : {0, 1, 2, 5}) {
        conv3d_desc d = base;
        d.split_k = sk;
        run_ok(d, f);
      }
      conv3d_desc nc = base;
      nc.layout = CONV3D_NCDHW;
      nc.out_layout = CONV3D_NCDHW;
      run_ok(nc, f);
      if (base.h >= 2 && base.w >= 2 && base.pad_lo[1] <= 1 && base.pad_hi[1] <= 1 &&
          base.pad_lo[2] <= 1 && base.pad_hi[2] <= 1) {
        conv3d_desc r = base;
        r.pad_mode = CONV3D_PAD_REFLECT;
        run_ok(r, f);
      }
    }
    if (base.cin % 16 == 0 && base.cout % 32 == 0) {
      conv3d_desc q = base;
      q.dtype = CONV3D_FP8_E4M3;
      run_ok(q, 0u);
    }
  }

  // Padded outputs with history and cache.
  {
    conv3d_desc d = make(1, 7, 66, 122, 160, 320, 0, 0, 0, 0, 0, 0);
    conv3d_out_pad op;
    memset(&op, 0, sizeof op);
    op.pad_lo[0] = 2; op.pad_lo[1] = 1; op.pad_lo[2] = 1;
    op.pad_hi[1] = 1; op.pad_hi[2] = 1;
    op.history_frames = 2;
    op.cache_frames = 2;
    op.cache = buf(14);
    run_ok(d, CONV3D_EPI_BIAS | CONV3D_EPI_RESIDUAL | CONV3D_EPI_L2NORM_SILU, &op);
    op.history_frames = 3;   // more history than leading planes
    size_t ws = 0;
    EXPECT(conv3d_padded_workspace_bytes(&d, nullptr, &op, &ws), CONV3D_ERR_SHAPE);
  }

  // Rejected calls: nothing launches.
  {
    const int n0 = conv3d::g_launches;
    conv3d_desc d = make(1, 5, 16, 16, 64, 64, 2, 1, 1, 0, 1, 1);
    size_t ws = 0;
    EXPECT(conv3d_workspace_bytes(nullptr, nullptr, &ws), CONV3D_ERR_NULL);
    EXPECT(conv3d_fwd(&d, nullptr, buf(2), nullptr, buf(3), buf(4), 1 << 30, nullptr),
           CONV3D_ERR_NULL);
    conv3d_desc bad = d;
    bad.n = 0;
    EXPECT(conv3d_fwd(&bad, buf(1), buf(2), nullptr, buf(3), buf(4), 1 << 30, nullptr),
           CONV3D_ERR_SHAPE);
    bad = d;
    bad.d = 1; bad.pad_lo[0] = 0;
    EXPECT(conv3d_fwd(&bad, buf(1), buf(2), nullptr, buf(3), buf(4), 1 << 30, nullptr),
           CONV3D_ERR_SHAPE);
    bad = d;
    bad.cin = 12;
    EXPECT(conv3d_fwd(&bad, buf(1), buf(2), nullptr, buf(3), buf(4), 1 << 30, nullptr),
           CONV3D_ERR_ALIGN);
    EXPECT(conv3d_fwd(&d, (char*)buf(1) + 8, buf(2), nullptr, buf(3), buf(4), 1 << 30, nullptr),
           CONV3D_ERR_ALIGN);
    bad = d;
    bad.cout = 24;
    EXPECT(conv3d_fwd(&bad, buf(1), buf(2), nullptr, buf(3), buf(4), 1 << 30, nullptr),
           CONV3D_ERR_UNSUPPORTED);
    EXPECT(conv3d_fwd(&d, buf(1), buf(2), nullptr, (char*)buf(1) + 4096, buf(4), 1 << 30, nullptr),
           CONV3D_ERR_OVERLAP);
    EXPECT(conv3d_fwd(&d, buf(1), buf(2), nullptr, buf(3), (char*)buf(3) + 256, 1 << 30, nullptr),
           CONV3D_ERR_OVERLAP);
    // one sample above it is refused
    conv3d_desc one_big = make(1, 35, 512, 512, 128, 128, 2, 1, 1, 0, 1, 1);
    EXPECT(conv3d_fwd(&one_big, buf(1), buf(2), nullptr, buf(3), buf(4), 1 << 30, nullptr),
           CONV3D_ERR_UNSUPPORTED);
    conv3d_desc huge = make(0x7fffffff, 0x7fffffff, 0x7fffffff, 0x7fffffff, 0x7ffffff8,
                            0x7ffffff0, 2, 1, 1, 0, 1, 1);   // sizes that overflow 64 bits
    EXPECT(conv3d_workspace_bytes(&huge, nullptr, &ws) != CONV3D_OK, 1);
    conv3d_epilogue e;
    memset(&e, 0, sizeof e);
    e.flags = CONV3D_EPI_RESIDUAL_OUT;
    EXPECT(conv3d_fwd(&d, buf(1), buf(2), &e, buf(3), buf(4), 1 << 30, nullptr),
           CONV3D_ERR_UNSUPPORTED);
    e.flags = CONV3D_EPI_BIAS;
    EXPECT(conv3d_fwd(&d, buf(1), buf(2), &e, buf(3), buf(4), 1 << 30, nullptr), CONV3D_ERR_NULL);
    e.flags = 64;
    EXPECT(conv3d_fwd(&d, buf(1), buf(2), &e, buf(3), buf(4), 1 << 30, nullptr),
           CONV3D_ERR_UNSUPPORTED);
    EXPECT(conv3d::g_launches, n0);
  }

  // A batch above the 32-bit buffer range runs in passes of 7 samples, each
  // pass launching its own kernels; the whole tensors are checked first.
  {
    conv3d_desc big = make(16, 17, 256, 256, 128, 128, 2, 1, 1, 0, 1, 1);
    const int n0 = conv3d::g_launches;
    EXPECT(conv3d_fwd(&big, buf(1), buf(2), nullptr, buf(3), buf(4), 1 << 30, nullptr),
           CONV3D_OK);
    EXPECT(conv3d::g_launches - n0, 6);   // 3 passes x (queue reset + conv)
    char pd[512];
    EXPECT(conv3d_plan_describe(&big, nullptr, pd, sizeof pd), CONV3D_OK);
    EXPECT(strstr(pd, " passes=3 samples_per_pass=7") != nullptr, 1);
    conv3d_epilogue eb;
    memset(&eb, 0, sizeof eb);
    eb.flags = CONV3D_EPI_BIAS | CONV3D_EPI_RESIDUAL | CONV3D_EPI_RESIDUAL_OUT;
    eb.bias = (const float*)buf(5);
    eb.residual = buf(6);
    eb.residual_out = buf(7);
    EXPECT(conv3d_fwd(&big, buf(1), buf(2), &eb, buf(3), buf(4), 1 << 30, nullptr), CONV3D_OK);
    // residual_out 2 GiB into y: it misses the first pass's slice of y but
    // not y, so the call is refused before any pass launches
    const int n1 = conv3d::g_launches;
    eb.residual_out = (char*)buf(3) + (2LL << 30);
    EXPECT(conv3d_fwd(&big, buf(1), buf(2), &eb, buf(3), buf(4), 1 << 30, nullptr),
           CONV3D_ERR_OVERLAP);
    EXPECT(conv3d::g_launches, n1);
  }

  // The entry point without a workspace: the fixed scratch serves.
  {
    conv3d_desc d = make(1, 5, 16, 16, 1024, 1024, 2, 1, 1, 0, 1, 1);
    const int n0 = conv3d::g_launches;
    EXPECT(conv3d_fwd_noalloc(&d, buf(1), buf(2), nullptr, buf(3), nullptr), CONV3D_OK);
    if (conv3d::g_launches == n0) ++g_fail;
    conv3d_desc big = make(1, 17, 256, 256, 128, 128, 2, 1, 1, 0, 1, 1);
    big.layout = CONV3D_NCDHW;   // a 285 MB staging copy: more than the scratch
    const int n1 = conv3d::g_launches;
    EXPECT(conv3d_fwd_noalloc(&big, buf(1), buf(2), nullptr, buf(3), nullptr),
           CONV3D_ERR_WORKSPACE);
    EXPECT(conv3d_fwd_noalloc(&d, nullptr, buf(2), nullptr, buf(3), nullptr), CONV3D_ERR_NULL);
    EXPECT(conv3d::g_launches, n1);
  }

  // The other entry points.
  EXPECT(conv3d_pack_weight(buf(1), buf(2), 128, 128, nullptr), CONV3D_OK);
  EXPECT(conv3d_pack_weight(buf(1), buf(1), 128, 128, nullptr), CONV3D_ERR_OVERLAP);
  EXPECT(conv3d_pack_weight_fp8(buf(1), buf(2), 128, 128, nullptr), CONV3D_OK);
  EXPECT(conv3d_pack_weight_2d(buf(1), buf(2), 96, 96, nullptr), CONV3D_OK);
  EXPECT(conv3d_pack_weight(buf(1), buf(2), 0, 128, nullptr), CONV3D_ERR_SHAPE);
  EXPECT(conv3d_transpose(buf(1), CONV3D_NCDHW, buf(2), 1, 160, 7, 66, 122, nullptr), CONV3D_OK);
  EXPECT(conv3d_transpose(buf(1), CONV3D_NDHWC, buf(2), 1, 320, 5, 64, 120, nullptr), CONV3D_OK);
  EXPECT(conv3d_transpose(buf(1), 7, buf(2), 1, 320, 5, 64, 120, nullptr), CONV3D_ERR_SHAPE);
  {
    conv3d_group_norm_desc g = {1, 17, 256, 256, 128, 32, 1, 1, 1e-5f};
    size_t ws = 0;
    EXPECT(conv3d_group_norm_workspace_bytes(&g, &ws), CONV3D_OK);
    EXPECT(conv3d_group_norm(&g, buf(1), (const float*)buf(2), (const float*)buf(3), buf(4),
                             buf(5), ws, nullptr), CONV3D_OK);
    EXPECT(conv3d_group_norm(&g, buf(1), (const float*)buf(2), (const float*)buf(3), buf(1),
                             buf(5), ws, nullptr), CONV3D_OK);   // in place
    EXPECT(conv3d_group_norm(&g, buf(1), (const float*)buf(2), (const float*)buf(3), buf(4),
                             buf(5), ws - 1, nullptr), CONV3D_ERR_WORKSPACE);
    g.groups = 48;
    EXPECT(conv3d_group_norm_workspace_bytes(&g, &ws), CONV3D_ERR_SHAPE);
  }
  {
    conv3d_epilogue e;
    memset(&e, 0, sizeof e);
    e.flags = CONV3D_EPI_BIAS | CONV3D_EPI_RESIDUAL | CONV3D_EPI_L2NORM_SILU | CONV3D_EPI_RESIDUAL_OUT;
    e.bias = (const float*)buf(10);
    e.residual = buf(11);
    e.gamma = buf(12);
    e.residual_out = buf(13);
    conv3d_out_pad op;
    memset(&op, 0, sizeof op);
    op.pad_lo[0] = 2; op.pad_lo[1] = 1; op.pad_lo[2] = 1;
    op.pad_hi[1] = 1; op.pad_hi[2] = 1;
    op.history_frames = 2;
    op.cache_frames = 2;
    op.cache = buf(14);
    EXPECT(conv3d_norm_silu(buf(1), 1, 5, 16, 30, 640, &e, &op, buf(2), buf(3), nullptr), CONV3D_OK);
    EXPECT(conv3d_norm_silu(buf(1), 1, 5, 16, 30, 640, &e, nullptr, nullptr, buf(3), nullptr),
           CONV3D_OK);
    EXPECT(conv3d_norm_silu(buf(1), 1, 5, 16, 30, 640, &e, nullptr, nullptr, buf(1), nullptr),
           CONV3D_ERR_OVERLAP);
  }
  {
    const long long st[5] = {12LL * 17 * 64 * 120, 17LL * 64 * 120, 64 * 120, 120, 1};
    EXPECT(conv3d_stream_pack_input(buf(1), st, 1, 12, 5, 64, 120, buf(2), 2, buf(3), 32, buf(4),
                                    2, nullptr), CONV3D_OK);
    EXPECT(conv3d_stream_pack_input(buf(1), st, 1, 12, 5, 64, 120, buf(2), 3, buf(3), 32, buf(4),
                                    2, nullptr), CONV3D_ERR_SHAPE);
  }

  if (g_fail) {
    fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  printf("api driver ok (%d launches)\n", conv3d::g_launches);
  return 0;
}
