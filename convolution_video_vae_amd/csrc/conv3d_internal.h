// Internal interface between the C-ABI layer (argument checks, planning,
// workspace carving) and the HIP kernels. Not installed; the public surface
// is include/conv3d.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace conv3d {

// Epilogue modes of the implicit-GEMM kernel.
enum EpiMode : int {
  EPI_STORE = 0,    // bf16 out = value (bias / residual / residual_out per flags)
  EPI_NORM = 1,     // bf16 out = full contract with channel-row L2 norm + SiLU
  EPI_PARTIAL = 2,  // fp32 partial sums of one K slice (split-K)
  EPI_STATS = 3,    // EPI_STORE without post-operations, plus GroupNorm partial statistics
};

// Epilogue flag bits (same values as the public CONV3D_EPI_* flags).
enum : unsigned { F_BIAS = 1u, F_RESIDUAL = 2u, F_NORM = 4u, F_RESIDUAL_OUT = 8u };

// Live-balanced K split of the halo kernel: at most kMaxVTiles pixel tiles
// and kMaxVWG work-groups per channel tile.
constexpr int kMaxVTiles = 64;
constexpr int kMaxVWG = 256;
// Stages (live (kd, kh) pair x chunk steps) of one slot-kernel tile: its
// per-tile stage table holds at most this many.
constexpr int kSlotMaxStages = 128;

// Everything one implicit-GEMM launch needs; passed by value as the kernel
// argument. All tensors NDHWC.
struct IgemmArgs {
  const uint16_t* x;        // [N][D][H][W][Cin]
  const uint16_t* wp;       // packed [27][CC][Cout][32]
  uint16_t* y;              // [M][Cout]
  float* partial;           // [splits][M][Cout] (EPI_PARTIAL)
  // GroupNorm partial statistics (EPI_STATS): per pixel tile and channel tile,
  // [frame 0/1][4-channel subgroup][sum, sum of squares] of the stored values.
  float* gnp;
  const float* bias;        // [Cout]
  const uint16_t* residual; // [M][Cout]
  const uint16_t* gamma;    // [Cout]
  uint16_t* residual_out;   // [M][Cout]
  int N, D, H, W, Cin, Cout;
  int Do, Ho, Wo;
  int sd, sh, sw;           // stride
  int pd, ph, pw;           // leading zero pad
  int CC;                   // 32-channel K steps per tap = ceil(Cin / 32)
  int M;                    // output pixels
  int m_tiles, n_tiles, splits;
  int steps_per_split;      // K steps (of 32 channels) per split
  unsigned flags;
  unsigned x_bytes;         // size of x, for the buffer range check
  float sqrt_c;             // sqrtf((float)Cout)
  unsigned* queue;          // persistent tile queues (kQueueBytes, zeroed), or null
  int queue_tail;           // tiles of the shared tail queue (tail_tiles of the tile count)
  // fp32 reciprocals of Ho, Do and Wo + 2 (row splits with one correction
  // step each way; uniform, so they stay in scalar registers).
  float inv_ho, inv_do, inv_wp;
  // Live-balanced K split (halo kernel partials, vsplit != 0): a pixel
  // tile is cut into slices of about equal live work (taps that read real
  // input), so tiles of a causal layer's first frames, which see fewer
  // taps, get fewer slices. vwg[b] describes work-group b (blockIdx.x): its
  // pixel tile (bits 0-15), channel tile (16-31), slice (32-39), the
  // slices of its pixel tile (40-47) and the partial slot it writes
  // (48-63), all formed on the host so that the work-group's first scalar
  // load is its last.
  int vsplit, per_n;
  uint64_t vwg[kMaxVWG];
  // Padded output (ypad != 0; slot kernels without a reduce): y is
  // [N][yDy][yHy][yWy][Cout] and output pixel (n, d, h, w) is stored at
  // (n, d + ypt, h + yph, w + ypw); residual and residual_out stay unpadded.
  int ypad, yDy, yHy, yWy, ypt, yph, ypw;
  float inv_wo;             // fp32 reciprocal of Wo (the padded pixel split)
  // Slot kernels, frame order (frames != 0): the N * Do output frames of
  // frame_slots = Ho * (slots per row) slots each are tiled separately into
  // frame_tiles runs. Pixel tiles [0, N * head * frame_tiles) are the first
  // `head` frames of each sample (frames with taps before the input's
  // start, which cost less), frame by frame; the rest are the other frames
  // with run index major and frame minor, so consecutive tiles are the same
  // rows of consecutive frames.
  int frames, frame_slots, frame_tiles, head;
};

// Persistent tile queues: one counter per XCD, kQueueStride words apart;
// XCD x takes chunks of kQueueChunk consecutive tiles. The last tiles of
// the hand-out order (queue_tail, normally tail_tiles(T) of T) form a ninth, shared queue that
// the work-groups of every XCD draw from once their own share is done, so
// XCDs that run ahead take more of the tail.
constexpr int kQueueStride = 64;
constexpr int kQueueChunk = 8;
constexpr size_t kQueueBytes = 9 * kQueueStride * 4;
constexpr int tail_tiles(int T) { return T / 4 < 512 ? T / 4 : 512; }

struct ReduceArgs {
  const float* partial;     // [splits][M][Cout]
  uint16_t* y;
  const float* bias;
  const uint16_t* residual;
  const uint16_t* gamma;
  uint16_t* residual_out;
  int M, Cout, splits;
  unsigned flags;
  float sqrt_c;
  // Fragment-order partials of the halo kernel (frag != 0): tile grid and
  // shape (4 waves as wm x 4/wm, each pb x cb blocks of 32 x 32).
  int frag, m_tiles, n_tiles, wm, pb, cb;
  // Live-balanced split (as IgemmArgs): pixel tile t's slices are slots
  // split_base[t] .. split_base[t + 1] - 1 of each channel tile's per_n.
  int vsplit, per_n;
  uint16_t split_base[kMaxVTiles + 1];
};

// A main-kernel configuration: MFMA block size R (16: v_mfma_f32_16x16x32_bf16,
// 32: v_mfma_f32_32x32x16_bf16), WM x WN waves, each wave PB pixel blocks x
// CB channel blocks of R (BM = R*PB*WM pixels, BN = R*CB*WN channels); a
// pipeline step covers KB K steps of 32 channels and the pipeline rings are
// NS deep.
struct TileCfg {
  int r, wm, wn, pb, cb, kb, ns;
  int bm() const { return r * pb * wm; }
  int bn() const { return r * cb * wn; }
};

// Channels-last GroupNorm (conv3d_norm.hip). A unit is one frame (n, d) or
// one sample n; its P pixels of C channels are contiguous. Chunks of
// chunk_px pixels (a multiple of ppi) split each unit across work-groups.
struct GroupNormArgs {
  const uint16_t* x;        // [units][P][C]
  uint16_t* y;              // same shape; may be x itself
  const float* gamma;       // [C]
  const float* beta;        // [C]
  double* partial;          // [units][chunks][G][2]: shifted sum, sum of squares
  float* stats;             // [units][G][2]: mean, 1/sqrt(var + eps)
  long long P;              // pixels per unit
  int C, G, cpg;            // channels, groups, channels per group
  int V, ppi;               // C / 8 vectors per pixel; 256 / V pixels per pass
  int units, chunks, chunk_px;
  float eps;
  int silu;
};

// GroupNorm statistics from a conv's per-tile partial sums (IgemmArgs::gnp,
// 512 x 128 slot tiles of TS stored slots, output rows of WP slots, Ho rows
// per frame; a tile's slots span at most two frames).
struct GnTileArgs {
  const float* part;        // [m_tiles][n_ctiles][2][32][2]
  int n_ctiles;             // 128-channel tiles
  int TS, WP, Ho;
  int frames_per_unit;      // 1 (per frame) or the frames of a sample
};

// Launchers (conv3d_kernels.hip, conv3d_norm.hip). Each returns 0 on success or the HIP
// error code of the launch. `stream` is a hipStream_t.
// taps = 27: an OIDHW weight; taps = 9: a [cout][cin][3][3] weight placed in
// the last temporal slice (kd = 2), the other slices zero.
int launch_pack_weight(const uint16_t* w, uint16_t* wp, int cout, int cin, int taps, void* stream);
// e4m3 OIDHW [cout][cin][27] bytes -> [27][ceil(cin / 64)][cout][64] bytes, zero beyond cin.
int launch_pack_weight_fp8(const uint8_t* w, uint8_t* wp, int cout, int cin, void* stream);
int launch_transpose(const uint16_t* src, uint16_t* dst, int n, int a, int b, void* stream);
// Returns -1 if no kernel is compiled for (cfg, mode, reflect). reflect:
// spatial reflect padding instead of zeros (pads of at most one).
// fp8: e4m3 activations and packed weight (bf16 otherwise).
int launch_igemm(const TileCfg& cfg, int mode, bool reflect, bool fp8, const IgemmArgs& args,
                 int grid, void* stream);
bool igemm_has_config(const TileCfg& cfg, int mode, bool reflect = false, bool fp8 = false);
int launch_reduce(const ReduceArgs& args, void* stream);
// Scratch memory of conv3d_fwd_noalloc: a file-scope device array of
// kScratchBytes (conv3d_kernels.hip) that every GPU the library runs on
// holds until the process ends. scratch_address stores the current
// device's address of it in *ptr (looked up once per device with
// hipGetSymbolAddress) and returns 0, or a nonzero HIP error code.
constexpr size_t kScratchBytes = (size_t)96 << 20;
int scratch_address(void** ptr);
int launch_queue_reset(unsigned* queue, void* stream);
int launch_group_norm(const GroupNormArgs& args, void* stream);
// The same with the statistics formed from a conv's partial sums (no pass
// over x for them): a finalize work-group per unit, then the apply pass.
int launch_group_norm_tiles(const GroupNormArgs& args, const GnTileArgs& t, void* stream);
// Padded outputs: the unpadded output y0 [N][Do][Ho][Wo][Cout] placed into
// y [N][Dy][Hy][Wy][Cout] at (pt, ph, pw); zeros elsewhere except the
// interiors of the hist planes before pt; the last cache_k frames also into
// cache [N][cache_frames][Ho][Wo][Cout] at its last frames (cache may be null).
// y0 may be null: the interior is then already in y (written in place by
// the conv or the standalone norm) and the cache's current frames are copied
// from there. previous, when
// not null, holds hist frames [N][hist][Ho][Wo][Cout] that are copied into
// the history planes' interiors and, for the cache's older frames, into the
// cache.
struct PlaceArgs {
  const uint16_t* y0;
  uint16_t* y;
  uint16_t* cache;
  const uint16_t* previous;
  int n, cout, Do, Ho, Wo, Dy, Hy, Wy, pt, ph, pw, hist;
  int cache_frames, cache_k;
};
int launch_place(const PlaceArgs& args, void* stream);

// Standalone post-operations (bias -> residual -> L2 norm x sqrt(C) x gamma
// -> SiLU) on an existing bf16 tensor x [M][C], written to y as geo places
// it (geo.y0 unused; padded and cache only when geo.Dy > 0).
struct NormSiluArgs {
  const uint16_t* x;
  const float* bias;
  const uint16_t* residual;
  const uint16_t* gamma;
  uint16_t* residual_out;
  uint16_t* y;
  unsigned flags;
  int M, C;
  float sqrt_c;
  PlaceArgs geo;
};
int launch_norm_silu(const NormSiluArgs& args, void* stream);
// First layer of a streaming causal conv: a strided channels-first chunk and
// up to two raw history frames -> padded NDHWC input and the raw-frame cache.
struct StreamPackArgs {
  const uint16_t* chunk;
  long long sn, sc, st, sh, sw;   // chunk strides in elements
  const uint16_t* history;        // [N][P][H][W][C] or null
  uint16_t* padded;               // [N][T+2][H+2][W+2][c_pad]
  uint16_t* cache;                // [N][cache_frames][H][W][C]
  int n, c, t, h, w, P, c_pad, cache_frames;
};
int launch_stream_pack(const StreamPackArgs& args, void* stream);

}  // namespace conv3d
