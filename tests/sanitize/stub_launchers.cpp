// Host-only stand-ins for the library's kernel launchers, so the C-ABI layer
// (argument checks, planning, workspace carving, dispatch) can be built and
// run under AddressSanitizer and UndefinedBehaviorSanitizer without a GPU.
// Every launcher checks what the real kernels rely on (non-null operands,
// positive sizes) and counts the launch; none touches the memory it is given.
#include <stdio.h>
#include <stdlib.h>

#include "../../convolution_video_vae_amd/csrc/conv3d_internal.h"

namespace conv3d {

int g_launches = 0;

static void require(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "stub launcher: %s\n", what);
    abort();
  }
}

int launch_pack_weight(const uint16_t* w, uint16_t* wp, int cout, int cin, int taps, void*) {
  require(w && wp && cout > 0 && cin > 0 && (taps == 27 || taps == 9), "pack_weight args");
  ++g_launches;
  return 0;
}
int launch_pack_weight_fp8(const uint8_t* w, uint8_t* wp, int cout, int cin, void*) {
  require(w && wp && cout > 0 && cin > 0, "pack_weight_fp8 args");
  ++g_launches;
  return 0;
}
int launch_transpose(const uint16_t* src, uint16_t* dst, int n, int a, int b, void*) {
  require(src && dst && n > 0 && a > 0 && b > 0 && src != dst, "transpose args");
  ++g_launches;
  return 0;
}
bool igemm_has_config(const TileCfg& cfg, int mode, bool, bool) {
  return cfg.r > 0 && mode >= EPI_STORE && mode <= EPI_STATS;
}
int launch_igemm(const TileCfg& cfg, int mode, bool, bool, const IgemmArgs& a, int grid, void*) {
  require(a.x && a.wp && a.y && grid > 0 && cfg.bm() > 0 && cfg.bn() > 0, "igemm args");
  require(mode != EPI_PARTIAL || a.partial, "partials need a workspace");
  require(mode != EPI_STATS || (a.gnp && cfg.bm() == 512 && cfg.bn() == 128 && cfg.ns == -2),
          "statistics need their buffer and the 512 x 128 slot tile");
  require(a.M > 0 && a.Cout > 0 && a.CC > 0 && a.steps_per_split > 0, "igemm sizes");
  ++g_launches;
  return 0;
}
int launch_reduce(const ReduceArgs& r, void*) {
  require(r.partial && r.y && r.M > 0 && r.Cout > 0 && r.splits > 0, "reduce args");
  ++g_launches;
  return 0;
}
int launch_queue_reset(unsigned* q, void*) {
  require(q != nullptr, "queue");
  ++g_launches;
  return 0;
}
int launch_group_norm(const GroupNormArgs& a, void*) {
  require(a.x && a.y && a.partial && a.stats && a.units > 0 && a.chunks > 0, "group norm args");
  ++g_launches;
  return 0;
}
int launch_group_norm_tiles(const GroupNormArgs& a, const GnTileArgs& t, void*) {
  require(a.x && a.y && a.stats && a.units > 0 && a.chunks > 0 && t.part && t.n_ctiles > 0 &&
              t.TS > 0 && t.WP > 0 && t.Ho > 0 && t.frames_per_unit > 0,
          "group norm from partials args");
  ++g_launches;
  return 0;
}
int launch_place(const PlaceArgs& a, void*) {
  require(a.y && a.n > 0 && a.cout > 0, "place args");
  ++g_launches;
  return 0;
}
int launch_norm_silu(const NormSiluArgs& a, void*) {
  require(a.x && a.y && a.gamma && a.M > 0 && a.C > 0, "norm_silu args");
  ++g_launches;
  return 0;
}
int scratch_address(void** ptr) {
  *ptr = (void*)(uintptr_t)(0x7ULL << 40);   // a fake device address, never dereferenced
  return 0;
}
int launch_stream_pack(const StreamPackArgs& a, void*) {
  require(a.chunk && a.padded && a.n > 0 && a.c > 0, "stream pack args");
  ++g_launches;
  return 0;
}

}  // namespace conv3d
