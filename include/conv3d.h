/*
 * conv3d.h — bf16 3x3x3 Conv3D for causal video-VAE layers on AMD Instinct
 * MI355X (gfx950), channels-last (NDHWC), computed as an implicit GEMM:
 *
 *   M = N*Do*Ho*Wo output pixels, N = Cout, K = 27*Cin, fp32 accumulation.
 *
 * Sources of the operation (cited by page title and section):
 *  - "conv3d_implicit — accept and emit NDHWC so chained convs skip the layout
 *    round-trip" (FlyDSL issue): the layout / out_layout parameters ("Ask") and
 *    the split-K and non-split epilogues (maintainer reply).
 *  - "Add Qwen-Image VAE classic conv shapes to conv3d tests" (FlyDSL PR):
 *    causal padding, time (2 before, 0 after) and H/W (1, 1) ("T=1
 *    degeneration"); the zero pad (0,1,0,1) before a stride-2 conv ("Test
 *    shapes", table 2); packing a weight once instead of per call (commit
 *    "Stop the conv 1D/2D entry points from repacking weights every launch").
 *  - "Fused Conv3D + Bias + Residual + RMSNorm + SiLU" (cuDNN frontend):
 *    the post-operation contract and its rounding points ("Operation
 *    Contract"), operand rules ("Requirements") and weight packing once per
 *    weight ("Weight Packing").
 *  - The channels-last GroupNorm (+ SiLU) between the convs: the MiniMax H3
 *    comment on the FlyDSL issue page (its GroupNorm argument).
 *  - Streaming causal convs on temporal chunks: outputs written into padded
 *    buffers with history planes and a frame cache, and the first layer's
 *    chunk packing (cuDNN page: "Causal Conv3D with Cache", "Normalization
 *    and Padding Variant", "Spatial Padding Variant").
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers to bf16 data (raw 16-bit patterns),
 *    except `bias`, `gamma` and `beta` of the GroupNorm, which are fp32. All
 *    must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every entry point
 *    only enqueues work on `stream` and returns; nothing is synchronised.
 *  - The caller owns every buffer. The library allocates nothing, keeps no
 *    pointer after a call returns and holds no mutable global state, so calls
 *    from several host threads are safe and calls are graph-capturable.
 *  - Argument checks run before anything is enqueued: on an error the call
 *    returns a non-zero status and neither launches work nor writes any
 *    output. A failed launch returns CONV3D_ERR_HIP; faults inside a kernel
 *    surface asynchronously on `stream`.
 */
#ifndef CONV3D_MI355X_H
#define CONV3D_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CONV3D_OK = 0,
  CONV3D_ERR_NULL = 1,        /* a required pointer is NULL */
  CONV3D_ERR_SHAPE = 2,       /* non-positive size, bad stride/pad, empty output */
  CONV3D_ERR_ALIGN = 3,       /* pointer not 16-byte aligned, or Cin % 8 != 0 */
  CONV3D_ERR_OVERLAP = 4,     /* an output overlaps an input or another output */
  CONV3D_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  CONV3D_ERR_UNSUPPORTED = 6, /* a case the library does not implement (no fallback) */
  CONV3D_ERR_HIP = 7          /* the HIP runtime refused a launch */
} conv3d_status;

typedef enum { CONV3D_NCDHW = 0, CONV3D_NDHWC = 1 } conv3d_layout;

/* Epilogue flags (cuDNN page, "Operation Contract"). With B() = bf16
 * round-to-nearest-even and acc the fp32 accumulator:
 *   conv  = B(acc)
 *   main  = B(conv + bias)                      if CONV3D_EPI_BIAS, else conv
 *   value = B(main + residual)                  if CONV3D_EPI_RESIDUAL, else main
 *   out   = value                               without CONV3D_EPI_L2NORM_SILU
 * with CONV3D_EPI_L2NORM_SILU, over the full channel row of each pixel:
 *   den   = max(sqrt(sum_c value_c^2), 1e-12)  (a clamp, not an added eps)
 *   out   = B(a / (1 + exp(-a))),  a = B(B(B(value/den) * sqrt(Cout)) * gamma)
 * CONV3D_EPI_RESIDUAL_OUT additionally writes `value` (the pre-norm sum). */
enum {
  CONV3D_EPI_BIAS = 1,
  CONV3D_EPI_RESIDUAL = 2,
  CONV3D_EPI_L2NORM_SILU = 4,
  CONV3D_EPI_RESIDUAL_OUT = 8
};

/* One convolution. The kernel is fixed at 3x3x3, unit dilation, one group.
 * Input extents n, d, h, w; output extents follow PyTorch:
 *   Do = (d + pad_lo[0] + pad_hi[0] - 3) / stride[0] + 1   (likewise Ho, Wo).
 * Padding is zero padding folded into the input gather; nothing padded is
 * materialised. Causal time padding is pad_lo[0] = 2, pad_hi[0] = 0; a
 * pre-padded ("valid") input uses zeros everywhere; the stride-2 downsample
 * uses pad_lo = {2,0,0}, pad_hi = {0,1,1}. Index order is {d, h, w}.
 * layout is the input's layout; out_layout that of y, residual and
 * residual_out. NCDHW input or output costs a transpose through the
 * workspace, so chained layers should stay NDHWC.
 * split_k = 0 lets the library choose how many slices the K = 27*Cin sum is
 * cut into; a positive value forces that many (clamped to the number of
 * 32-channel K steps). Slices are summed in a fixed order, so results are
 * deterministic for a given split_k. */
typedef struct {
  int n, d, h, w;
  int cin, cout;
  int stride[3];
  int pad_lo[3];
  int pad_hi[3];
  int layout;      /* conv3d_layout of x */
  int out_layout;  /* conv3d_layout of y / residual / residual_out */
  int split_k;
  int pad_mode;    /* conv3d_pad_mode of the H and W padding (time is always zero padded) */
  int dtype;       /* conv3d_dtype of x and the packed weight (y, residual stay bf16) */
} conv3d_desc;

/* Operand type. FP8_E4M3 (Qwen PR: the FP8 suite of the implicit-GEMM conv,
 * e4m3fn activations and weights, fp32 bias, bf16 output): x holds e4m3fn
 * bytes, the weight is packed by conv3d_pack_weight_fp8, products and sums
 * are fp32 as for bf16 and the epilogue is unchanged. Requires cin % 16 == 0
 * (CONV3D_ERR_ALIGN), cout % 32 == 0, NDHWC, zero padding
 * (CONV3D_ERR_UNSUPPORTED). */
typedef enum { CONV3D_BF16 = 0, CONV3D_FP8_E4M3 = 1 } conv3d_dtype;

/* Spatial padding: zeros, or reflection as the H3 encoder pads before each
 * conv (FlyDSL issue, MiniMax H3 comment, the conv call site: spatial
 * reflect pad, temporal causal zero pad): index -1 reads 1, index h reads
 * h - 2. Reflect needs spatial pads of at most 1 (CONV3D_ERR_UNSUPPORTED
 * above) and h, w >= 2 (CONV3D_ERR_SHAPE below). */
typedef enum { CONV3D_PAD_ZERO = 0, CONV3D_PAD_REFLECT = 1 } conv3d_pad_mode;

/* Optional fused post-operations; pass NULL to conv3d_fwd for a plain conv
 * (out = B(acc)). Pointers a flag does not use are ignored.
 *   bias          fp32 [cout]                               (CONV3D_EPI_BIAS)
 *   residual      bf16, output shape, out_layout            (CONV3D_EPI_RESIDUAL)
 *   gamma         bf16 [cout]                               (CONV3D_EPI_L2NORM_SILU)
 *   residual_out  bf16, output shape, out_layout            (CONV3D_EPI_RESIDUAL_OUT,
 *                 requires CONV3D_EPI_RESIDUAL) */
typedef struct {
  unsigned flags;
  const float* bias;
  const void* residual;
  const void* gamma;
  void* residual_out;
} conv3d_epilogue;

/* Bytes of the packed weight for (cout, cin). */
size_t conv3d_packed_weight_bytes(int cout, int cin);

/* Pack an OIDHW checkpoint weight [cout][cin][3][3][3] (bf16) once, outside
 * the inference loop ("Weight Packing": pack once, reuse, repack after the
 * weights change). Packed layout, bf16:
 *   packed[t][c / 32][co][c % 32],  t = kd*9 + kh*3 + kw,  c < roundup(cin, 32)
 * with the channels c >= cin zero. Each 32-channel K step of one tap is then
 * one contiguous [cout][32] block. w_oidhw and w_packed must not overlap. */
conv3d_status conv3d_pack_weight(const void* w_oidhw, void* w_packed, int cout, int cin,
                                 void* stream);

/* Bytes of the packed e4m3 weight for (cout, cin). */
size_t conv3d_packed_weight_bytes_fp8(int cout, int cin);

/* Pack an e4m3fn OIDHW weight [cout][cin][3][3][3] (1 byte each):
 *   packed[t][c / 64][co][c % 64],  t = kd*9 + kh*3 + kw,  c < roundup(cin, 64)
 * with the channels c >= cin zero (one 64-channel K step of a tap is one
 * contiguous [cout][64] block). w and w_packed must not overlap. */
conv3d_status conv3d_pack_weight_fp8(const void* w_oidhw, void* w_packed, int cout, int cin,
                                     void* stream);

/* Pack a 2D weight [cout][cin][3][3] (bf16) as the last temporal slice
 * (kd = 2) of a 3x3x3 weight whose other slices are zero; same packed layout
 * and size as conv3d_pack_weight. A causal conv3d_fwd (pad_lo[0] = 2,
 * pad_hi[0] = 0) on single-frame inputs [n][1][h][w][c] with it is the 2D
 * conv of each image, because such a conv only ever sees its last temporal
 * tap (Qwen PR, "T=1 degeneration"); the zero slices are dead taps the
 * kernels skip. A 1x3x3 conv over d frames is the same call on the view
 * [n*d][1][h][w][c] of an NDHWC tensor (no copy). */
conv3d_status conv3d_pack_weight_2d(const void* w_oihw, void* w_packed, int cout, int cin,
                                    void* stream);

/* Output extents {Do, Ho, Wo} for desc; CONV3D_ERR_SHAPE if any is < 1. */
conv3d_status conv3d_output_dims(const conv3d_desc* desc, int out_dhw[3]);

/* Workspace bytes conv3d_fwd needs for (desc, epi); 0 for an NDHWC layer
 * that runs without split-K. epi may be NULL. */
conv3d_status conv3d_workspace_bytes(const conv3d_desc* desc, const conv3d_epilogue* epi,
                                     size_t* bytes);

/* y = conv3d(x, w) followed by the epilogue (see CONV3D_EPI_*).
 *   x          bf16, [n][d][h][w][cin] (NDHWC) or [n][cin][d][h][w] (NCDHW)
 *   w_packed   from conv3d_pack_weight for (cout, cin)
 *   y          bf16, output shape in out_layout
 *   workspace  device scratch of at least conv3d_workspace_bytes() bytes
 * y must not overlap x, w_packed, the workspace, residual or residual_out.
 * Channel requirements: cin % 8 == 0, cout % 16 == 0.
 * Size: one sample's input, output and (padded) output must each stay below
 * 2 GiB (CONV3D_ERR_UNSUPPORTED otherwise). A batch whose tensors exceed it
 * runs as passes over as many consecutive samples as fit, in order on the
 * stream, reusing the workspace (whose size conv3d_workspace_bytes already
 * covers); conv3d_plan_describe reports the passes. */
conv3d_status conv3d_fwd(const conv3d_desc* desc, const void* x, const void* w_packed,
                         const conv3d_epilogue* epi, void* y, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ------------------------------------------------------- padded outputs
 * Where conv3d_fwd_padded writes its output (cuDNN page, "Normalization and
 * Padding Variant" and "Spatial Padding Variant"): y is NDHWC
 *   [n][Do + pad_lo[0] + pad_hi[0]][Ho + pad_lo[1] + pad_hi[1]][Wo + pad_lo[2] + pad_hi[2]][cout]
 * with output pixel (d, h, w) at (d + pad_lo[0], h + pad_lo[1], w + pad_lo[2]).
 * Everything else in y is written with zeros, except the interiors of the
 * history_frames planes just before the output (pad_lo[0] - history_frames
 * .. pad_lo[0] - 1), which hold the caller's history (the previous chunk's
 * last activated frames) and are not touched. A following valid conv on y
 * then sees the history where a causal conv would see zero planes, and the
 * zero border as its spatial padding; pad_hi = {0, 1, 1} gives the zero
 * bottom row and right column a stride-2 conv expects.
 * With cache != NULL, the last min(cache_frames, Do) output frames of each
 * sample are also written to the last frames of cache, NDHWC
 * [n][cache_frames][Ho][Wo][cout]; older cache frames are the caller's. */
/* conv3d_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, semantics, kernels and results as conv3d_fwd, but no workspace
 * argument: the split-K partials, the tile queues and the NDHWC staging of
 * NCDHW operands live in a fixed device array of 96 MiB that the library
 * holds on every GPU it runs on until the process ends (looked up once per
 * device on the first call there, with that device current). Nothing is
 * allocated by the call.
 * Calls whose plan needs more than 96 MiB (conv3d_workspace_bytes) return
 * CONV3D_ERR_WORKSPACE before anything is enqueued. All calls on one GPU
 * share that GPU's array: calls that may overlap in time on one GPU (other
 * streams, other host threads) race and must be serialised by the caller;
 * calls on one stream are ordered and safe. Every value a call reads from
 * the array is written earlier in the same call (the tile queues are
 * cleared by a kernel, not by a memset). Other errors as conv3d_fwd;
 * CONV3D_ERR_HIP if the array's address cannot be obtained. */
conv3d_status conv3d_fwd_noalloc(const conv3d_desc* desc, const void* x, const void* w_packed,
                                 const conv3d_epilogue* epi, void* y, void* stream);

typedef struct {
  int pad_lo[3];       /* >= 0: time, h, w */
  int pad_hi[3];       /* >= 0 */
  int history_frames;  /* 0 .. pad_lo[0] */
  int cache_frames;    /* 1 .. Do + history_frames when cache != NULL */
  void* cache;         /* bf16, 16-byte aligned, or NULL */
} conv3d_out_pad;

/* Workspace bytes conv3d_fwd_padded needs (the conv's own workspace plus a
 * staged copy of the unpadded output when out_pad pads or caches). */
conv3d_status conv3d_padded_workspace_bytes(const conv3d_desc* desc, const conv3d_epilogue* epi,
                                            const conv3d_out_pad* out_pad, size_t* bytes);

/* conv3d_fwd with its output written as out_pad describes (out_layout must
 * be NDHWC; the epilogue is the same, residual and residual_out keep the
 * unpadded output shape). y, cache, residual_out and the workspace must not
 * overlap any operand or each other. out_pad == NULL is conv3d_fwd. */
conv3d_status conv3d_fwd_padded(const conv3d_desc* desc, const void* x, const void* w_packed,
                                const conv3d_epilogue* epi, const conv3d_out_pad* out_pad,
                                void* y, void* workspace, size_t workspace_bytes, void* stream);

/* First layer of a streaming causal encoder (cuDNN page, "Causal Conv3D
 * with Cache"): one temporal chunk, channels-first with arbitrary strides,
 * chunk[i_n * strides[0] + i_c * strides[1] + i_t * strides[2] + i_h * strides[3]
 *       + i_w * strides[4]] (elements, bf16, >= 0),
 * and history_frames (0..2) raw frames before it, NDHWC [n][history_frames][h][w][c]
 * -> padded NDHWC [n][t + 2][h + 2][w + 2][c_pad]: the chunk in planes 2..t+1
 * and the history in the planes before, at spatial offset (1, 1); zeros in
 * the border, the 2 - history_frames missing planes and channels c..c_pad-1.
 * A valid conv3d_fwd on padded is the chunk's causal conv.
 * With cache != NULL, cache NDHWC [n][cache_frames][h][w][c] receives the
 * last cache_frames raw frames of history ++ chunk (1 <= cache_frames <=
 * t + history_frames; 2 when the next chunk needs two).
 * c_pad % 8 == 0, c_pad >= c; padded 16-byte aligned; chunk, history and
 * cache 2-byte aligned; padded and cache must not overlap each other, chunk
 * or history. */
conv3d_status conv3d_stream_pack_input(const void* chunk, const long long strides[5], int n,
                                       int c, int t, int h, int w, const void* history,
                                       int history_frames, void* padded, int c_pad, void* cache,
                                       int cache_frames, void* stream);

/* Standalone post-operations on an existing bf16 tensor (cuDNN page,
 * "Standalone Normalization and Padding Variant": for output channel counts
 * above the fused tile, a raw conv is followed by this). x NDHWC
 * [n][d][h][w][c] is taken as `conv` of the contract (see CONV3D_EPI_*):
 *   main = B(x + bias) (CONV3D_EPI_BIAS), value = B(main + residual)
 *   (CONV3D_EPI_RESIDUAL), y = the L2 norm x sqrt(c) x gamma -> SiLU of value
 * (CONV3D_EPI_L2NORM_SILU must be set; gamma bf16 [c]). CONV3D_EPI_RESIDUAL_OUT
 * writes value to residual_out, with or without a residual. y is written as
 * out_pad places it (NULL: [n][d][h][w][c]); with previous != NULL (bf16
 * NDHWC [n][out_pad->history_frames][h][w][c], the previous chunk's last
 * activated frames) the history planes' interiors and the cache's older
 * frames are copied from it. c % 8 == 0, c <= 2048; every pointer 16-byte
 * aligned except bias (4); outputs must not overlap inputs or each other. */
conv3d_status conv3d_norm_silu(const void* x, int n, int d, int h, int w, int c,
                               const conv3d_epilogue* epi, const conv3d_out_pad* out_pad,
                               const void* previous, void* y, void* stream);

/* Layout change at a network boundary, bf16, exact:
 *   src_layout = CONV3D_NCDHW:  [n][c][d][h][w] -> [n][d][h][w][c]
 *   src_layout = CONV3D_NDHWC:  [n][d][h][w][c] -> [n][c][d][h][w]
 * src and dst must not overlap. */
conv3d_status conv3d_transpose(const void* src, int src_layout, void* dst, int n, int c, int d,
                               int h, int w, void* stream);

/* ------------------------------------------------------------- GroupNorm
 * Channels-last GroupNorm (+ SiLU), the norm between the convs of a causal
 * video-VAE encoder (FlyDSL issue page, MiniMax H3 comment, the GroupNorm
 * argument: statistics per frame once time is folded into the batch, which
 * NDHWC makes a free view; the SiLU after it fused in; a group's c/groups
 * channels contiguous at every pixel). On x [n][d][h][w][c] with groups of
 * c/groups consecutive channels, and a unit = one frame (n, d) when
 * t_isolated, else one sample n (all its frames):
 *   mean, var = population mean and variance over the unit's pixels and the
 *               group's channels
 *   a = B((x - mean) / sqrt(var + eps) * gamma[c] + beta[c])
 *   y = B(a * sigmoid(a)) with silu, else a
 * B() rounds fp32 to bf16, to nearest, ties to even. */
typedef struct {
  int n, d, h, w, c;  /* NDHWC extents */
  int groups;         /* 1..256, c % groups == 0 */
  int t_isolated;     /* 1: statistics per frame; 0: per sample */
  int silu;           /* 1: SiLU after the affine */
  float eps;          /* > 0, finite */
} conv3d_group_norm_desc;

/* Workspace bytes conv3d_group_norm needs for desc (always > 0: per-chunk
 * partial sums and the per-group statistics). */
conv3d_status conv3d_group_norm_workspace_bytes(const conv3d_group_norm_desc* desc,
                                                size_t* bytes);

/* y = GroupNorm(x) (+ SiLU) as above.
 *   x, y         bf16 NDHWC; y may be x itself (in place), any other overlap
 *                with x is CONV3D_ERR_OVERLAP
 *   gamma, beta  fp32 [c]
 *   workspace    device scratch of at least conv3d_group_norm_workspace_bytes()
 * Errors: c % 8 != 0 -> CONV3D_ERR_ALIGN; c % groups != 0, a size < 1, eps not
 * > 0 -> CONV3D_ERR_SHAPE; c > 2048, groups > 256 or a tensor over 2^40 bytes
 * -> CONV3D_ERR_UNSUPPORTED. The workspace, gamma and beta must not overlap
 * x or y. */
conv3d_status conv3d_group_norm(const conv3d_group_norm_desc* desc, const void* x,
                                const float* gamma, const float* beta, void* y,
                                void* workspace, size_t workspace_bytes, void* stream);

/* The conv and the GroupNorm after it, with the norm's statistics formed by
 * the conv (FlyDSL issue page, MiniMax H3 comment: conv and norm move
 * together; here the norm's read of x for its statistics is saved, the conv
 * sums what it stores). Available for convs that conv3d_fwd runs on the
 * 512-slot x 128-channel slot tile with a plain store: cout % 128 == 0, no
 * epilogue flags, NDHWC in and out, bf16, one batch pass, tiles in slot order
 * (conv3d_plan_describe shows "ns=-2 bm=512 bn=128" without "order=frame"),
 * and output frames of at least 510 slots (Ho * (Wo + 2) >= 510); anything
 * else is CONV3D_ERR_UNSUPPORTED.
 *
 * conv3d_gn_partials_bytes: bytes of the partial-statistics buffer for desc
 *   (512 per pixel tile and 128-channel tile).
 * conv3d_fwd_gn_stats: y = conv3d(x, w) exactly as conv3d_fwd with no
 *   epilogue computes it (bit for bit), plus gn_partials: per pixel tile and
 *   channel tile, fp32 sums and sums of squares of the stored bf16 values per
 *   frame of the tile (at most two) and 4-channel subgroup. gn_partials (16-byte
 *   aligned, conv3d_gn_partials_bytes) must not overlap any other tensor.
 * conv3d_group_norm_from_partials: y = GroupNorm(x) (+ SiLU) as
 *   conv3d_group_norm computes it, for x the y of a conv3d_fwd_gn_stats call
 *   on `conv` and gn_partials its partial statistics; the mean and variance
 *   come from the partials (summed in a fixed order in fp64), so they equal
 *   conv3d_group_norm's up to fp32 rounding of the partial sums. desc must
 *   describe the conv's output ([n][Do][Ho][Wo][cout]; else CONV3D_ERR_SHAPE),
 *   and each group must be whole 4-channel subgroups of one 128-channel tile
 *   (c / groups a multiple of 4 dividing 128; else CONV3D_ERR_UNSUPPORTED).
 *   workspace: conv3d_group_norm_workspace_bytes(desc). Other rules as
 *   conv3d_group_norm. The partials are only read. */
conv3d_status conv3d_gn_partials_bytes(const conv3d_desc* desc, size_t* bytes);
conv3d_status conv3d_fwd_gn_stats(const conv3d_desc* desc, const void* x, const void* w_packed,
                                  void* y, void* gn_partials, void* workspace,
                                  size_t workspace_bytes, void* stream);
conv3d_status conv3d_group_norm_from_partials(const conv3d_group_norm_desc* desc,
                                             const conv3d_desc* conv, const void* gn_partials,
                                             const void* x, const float* gamma, const float* beta,
                                             void* y, void* workspace, size_t workspace_bytes,
                                             void* stream);

/* Human-readable name of a status code (static string). */
const char* conv3d_status_str(conv3d_status status);

/* Describe the kernel choice conv3d_fwd would make for (desc, epi) into buf
 * (NUL-terminated, truncated to len). Returns the same status conv3d_fwd's
 * argument checks would for the shapes alone. */
conv3d_status conv3d_plan_describe(const conv3d_desc* desc, const conv3d_epilogue* epi,
                                   char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* CONV3D_MI355X_H */
