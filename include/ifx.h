/*
 * ifx.h -- C ABI of the MI355X (gfx950) fused int8 ResNet convolution library.
 *
 * The library computes the int8 convolution path described by two of the
 * source pages:
 *   - Inspur, MLPerf v2.0 ResNet50 convolution-merge article ("Inspur
 *     conv-merge article"): section 2.2 (the res3.x bottleneck and the fused
 *     Conv3+BN+Sum+ReLU), section 3.1 (NC/32HW32 activations, [O1,I1,O2,I2]
 *     weights), section 3.3 (implicit GEMM data[M,K] . weight[N,K]^T),
 *     section 3.4 (BN+Sum+ReLU applied to the accumulators in one epilogue).
 *   - DiDi Cloud IFX DAWNBench blog, inference-optimisation section:
 *     CONV+BN+RELU and CONV+BN+RELU+MAXPOOL each as one function.
 *
 * Conventions for every entry point:
 *   - Pointers named *_blk, x_nhwc, w_ohwi, bias, mult, shift, residual, y,
 *     logits and ws are DEVICE pointers (HIP global memory), 16-byte aligned.
 *     The caller owns all memory; the library never allocates or frees
 *     device memory (its only resources are a graph handle's host state and,
 *     for ifx_net_forward on a large batch, one stream and two events per
 *     device, created on first use and kept for the process).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it (kernels; for ifx_net_forward on a batch
 *     of 192 or more images also an event fork to the library's stream and
 *     the join back) and never synchronise; results are valid once the
 *     stream reaches that point.  Calls that overlap on the same output or
 *     workspace race.
 *   - Arguments are validated on the host before anything is launched.  On
 *     an error status nothing has been enqueued.  Validation touches no
 *     device, so every error path runs without a GPU.
 *   - All arithmetic is integer; results are deterministic and bit-exact.
 *
 * Layouts (Inspur conv-merge article, section 3.1):
 *   activation  NC/32HW32: [N, C1=ceil(C/32), H, W, 32] int8; channel c of
 *               pixel (b,y,x) sits at ((b*C1 + c/32)*H + y)*W + x)*32 + c%32;
 *               channels >= C hold 0.
 *   weights     [O1, KH, KW, I1, O2, I2=32] int8 with O2 = min(128, Oc
 *               rounded up to 32), O1 = ceil(Oc/O2), I1 = ceil(Ic/32); zero
 *               outside Oc x Ic.  For 1x1 this is the article's [O1,I1,O2,I2].
 *   stem weights (7x7, stride 2, pad 3, MAXPOOL, Ic <= 4): [Oc, 8, 8, 4]
 *               int8, element (o,ky,kx,c) = w[o,ky,kx,c] for ky,kx < 7,
 *               c < Ic, else 0.
 *   int32 out   IFX_OUT_I32 writes acc + bias as int32 NHWC [N, Ho, Wo, Oc].
 *
 * Fused epilogue of one convolution, per output element (the BN, Sum and
 * ReLU of the Inspur article section 3.4 in fixed point; the rounding and
 * scale readings are the library's, since the pages print no formula):
 *   y   = acc + bias[o]                                (int32)
 *   q   = round_half_away_from_zero(y * mult[o] / 2^(31 + shift[o]))
 *   q  += residual  (IFX_RESIDUAL; same packed shape as the output)
 *   q   = max(q, 0) (IFX_RELU)
 *   out = saturate_int8(q)
 *   IFX_MAXPOOL: 3x3 stride-2 pad-1 max-pool of `out`, out-of-range taps
 *   ignored (stem only).
 * Caller contract, not checked on the device: 0 <= mult[o] < 2^31,
 * 0 <= shift[o] <= 31, and acc + bias inside the int32 range
 * [-2^31, 2^31 - 1] (INT32_MIN included).
 */
#ifndef IFX_H
#define IFX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    IFX_OK = 0,
    IFX_E_NULL = 1,        /* a required pointer is NULL */
    IFX_E_SHAPE = 2,       /* non-positive or inconsistent dimensions */
    IFX_E_UNSUPPORTED = 3, /* kernel/stride/pad/flag combination not implemented */
    IFX_E_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
    IFX_E_WORKSPACE = 5,   /* workspace smaller than the *_workspace_bytes query */
    IFX_E_HIP = 6          /* a HIP launch failed; see ifx_last_hip_error() */
} ifx_status;

/* Per-convolution flags. */
enum {
    IFX_RELU = 1u,     /* ReLU before saturation */
    IFX_RESIDUAL = 2u, /* add the shortcut tensor before ReLU */
    IFX_MAXPOOL = 4u,  /* fused 3x3/s2/p1 max-pool after ReLU (7x7/s2/p3 stem only) */
    IFX_OUT_I32 = 8u,  /* write int32 acc + bias, NHWC, no requantisation */
    IFX_INPUT_NHWC = 16u, /* stem only: the input is the compact NHWC image [n, h, w, c_in]
                             int8 instead of the packed layout (the input pack is folded
                             into the stem's loads) */
    IFX_OUT_EVEN = 32u,   /* d3 of ifx_conv_chain_fused only: the block output is stored
                             only at even rows and columns, the pixels a stride-2 1x1
                             projection reads */
    IFX_OUT_PHASE = 64u,  /* the output is stored phase-split (layout below; even Ho, Wo) */
    IFX_IN_PHASE = 128u   /* 3x3 stride 2 pad 1 only: the input is phase-split (even H, W) */
};

/*
 * Phase-split layout of a packed tensor with even height and width:
 * [N, C1, 2, 2, H/2, W/2, 32], plane (py, px) holding the pixels (2i + py, 2j + px).
 * The same bytes as [N, C1, H, W, 32], permuted so that every tap of a stride-2 3x3
 * convolution reads runs of consecutive pixels (a plain layout gives it 32-byte
 * pieces 64 bytes apart).  The flags are accepted only where the general
 * implicit-GEMM kernel runs the convolution and would not split it over K
 * (ifx_conv_validate answers IFX_E_UNSUPPORTED for the stem, the small-K 1x1
 * and haloed 3x3 shapes, IFX_OUT_I32 and odd sizes); the shortcut and the output
 * keep the plain layout unless IFX_OUT_PHASE.  ifx_net_forward uses the layout
 * between conv1 and a stride-2 conv2 of a bottleneck.
 */

/*
 * One convolution.  Supported (kh, kw, stride, pad):
 *   (1,1,1,0) (1,1,2,0) (3,3,1,1) (3,3,2,1)  flags: any of RELU|RESIDUAL, or
 *                                            OUT_I32 alone; c_out a multiple of 4
 *   (7,7,2,3) with IFX_MAXPOOL (RELU, INPUT_NHWC optional), c_in <= 4
 * n, h, w, c_in, c_out > 0; the output size must be positive.
 */
typedef struct {
    int32_t n, h, w, c_in, c_out;
    int32_t kh, kw, stride, pad;
    uint32_t flags;
} ifx_conv_desc;

/* Host-only: validate a descriptor (shape and supported set); no device use. */
ifx_status ifx_conv_validate(const ifx_conv_desc *d);

/* Host-only: output height/width of d (after the pool when IFX_MAXPOOL). */
ifx_status ifx_conv_out_dims(const ifx_conv_desc *d, int32_t *ho, int32_t *wo);

/* Host-only: bytes of a packed activation, n * ceil(c/32) * h * w * 32. */
size_t ifx_act_bytes(int32_t n, int32_t h, int32_t w, int32_t c);

/* Host-only: bytes of the packed weights of d (0 if d is invalid). */
size_t ifx_wpack_bytes(const ifx_conv_desc *d);

/*
 * Activation pack NHWC -> NC/32HW32 (Inspur conv-merge article, section 3.1:
 * channels split into groups of 32 so one pixel's group is one 16-byte pair).
 * x_nhwc: [n,h,w,c] int8 (any alignment); x_blk: ifx_act_bytes() bytes.
 */
ifx_status ifx_pack_act(const int8_t *x_nhwc, int8_t *x_blk, int32_t n, int32_t h, int32_t w,
                        int32_t c, void *stream);

/* Inverse of ifx_pack_act (padding channels dropped); x_nhwc any alignment. */
ifx_status ifx_unpack_act(const int8_t *x_blk, int8_t *x_nhwc, int32_t n, int32_t h, int32_t w,
                          int32_t c, void *stream);

/*
 * Weight reblock OHWI [c_out, kh, kw, c_in] -> the packed layout of d
 * (Inspur conv-merge article, section 3.1).  w_ohwi any alignment; w_blk
 * ifx_wpack_bytes(d) bytes.
 */
ifx_status ifx_pack_weights(const ifx_conv_desc *d, const int8_t *w_ohwi, int8_t *w_blk, void *stream);

/*
 * One fused convolution (Inspur conv-merge article sections 3.3-3.4; DiDi
 * IFX blog inference section): implicit-GEMM int8 convolution with int32
 * accumulation followed by the fused epilogue above.
 *   x_blk      packed input [n, ceil(c_in/32), h, w, 32], or the compact
 *              [n, h, w, c_in] image for a stem with IFX_INPUT_NHWC
 *   w_blk      packed weights of d (ifx_pack_weights)
 *   bias, mult, shift   int32 [c_out]
 *   residual   packed [n, ceil(c_out/32), ho, wo, 32] when IFX_RESIDUAL, else NULL
 *   y          packed int8 output [n, ceil(c_out/32), ho', wo', 32] (pooled
 *              size with IFX_MAXPOOL), or int32 NHWC with IFX_OUT_I32
 * Input and output must not overlap.
 */
ifx_status ifx_conv_fused(const ifx_conv_desc *d, const int8_t *x_blk, const int8_t *w_blk,
                          const int32_t *bias, const int32_t *mult, const int32_t *shift,
                          const int8_t *residual, void *y, void *stream);

/*
 * ifx_conv_fused that also writes the output's even pixels (rows and columns
 * 0, 2, 4, ...) a second time, densely, to y_even [n, ceil(c_out/32),
 * ceil(ho/2), ceil(wo/2), 32].  A stride-2 pad-0 1x1 convolution reads exactly
 * those pixels (the projection shortcut of the Inspur article's section 2.2
 * stage-entry block), so the block that follows can run its projection with
 * unit stride on y_even and read contiguous runs instead of every other
 * 32-byte piece; y itself is written as by ifx_conv_fused.
 *   y_even     16-byte aligned, must not overlap the other tensors
 * Returns IFX_E_UNSUPPORTED, launching nothing, when the kernel that runs d
 * does not write the copy (ifx_conv_even_supported says which); IFX_OUT_I32,
 * IFX_OUT_PHASE and IFX_MAXPOOL descriptors are never supported.
 */
ifx_status ifx_conv_fused_even(const ifx_conv_desc *d, const int8_t *x_blk, const int8_t *w_blk,
                               const int32_t *bias, const int32_t *mult, const int32_t *shift,
                               const int8_t *residual, void *y, int8_t *y_even, void *stream);
/* Host-only: 1 when ifx_conv_fused_even(d, ...) would run, 0 when not or when d is invalid. */
int32_t ifx_conv_even_supported(const ifx_conv_desc *d);

/*
 * Conv3 of a bottleneck together with its projection shortcut, as one launch.
 * The Inspur conv-merge article (section 2.1) merges operators into one kernel
 * so that a tensor passed between them is neither written to nor read back from
 * global memory; here the passed tensor is the projection shortcut of the first
 * block of a stage (section 2.2 structure, with a 1x1 projection of the block
 * input in place of the input itself):
 *   sc = conv(x_blk; dp)                 requantised to int8, no ReLU
 *   y  = conv(t_blk; d3, RESIDUAL = sc)
 * The result is bit-identical to ifx_conv_fused(dp) followed by ifx_conv_fused(d3)
 * with that output as the residual; sc is never stored.
 *   d3      1x1, stride 1, pad 0, flags IFX_RESIDUAL, optionally IFX_RELU
 *   t_blk   packed input of d3, [n, ceil(d3.c_in/32), d3.h, d3.w, 32]
 *   dp      1x1, any stride, pad 0, flags 0
 *   x_blk   packed input of dp, [n, ceil(dp.c_in/32), dp.h, dp.w, 32]
 *   w3_blk, bias3, mult3, shift3 / wp_blk, biasp, multp, shiftp: packed weights
 *           and per-channel parameters of d3 / dp, as for ifx_conv_fused
 *   y_blk   packed int8 output [n, ceil(c_out/32), ho, wo, 32]; must not overlap
 *           the inputs
 * Both descriptors must have the same n and c_out and the same output height and
 * width (IFX_E_SHAPE otherwise); other kernel sizes, pads or flags give
 * IFX_E_UNSUPPORTED.  Nothing is launched on an error.
 */
ifx_status ifx_conv_proj_fused(const ifx_conv_desc *d3, const int8_t *t_blk, const int8_t *w3_blk,
                               const int32_t *bias3, const int32_t *mult3, const int32_t *shift3,
                               const ifx_conv_desc *dp, const int8_t *x_blk, const int8_t *wp_blk,
                               const int32_t *biasp, const int32_t *multp, const int32_t *shiftp,
                               int8_t *y_blk, void *stream);

/*
 * Conv3 of one bottleneck together with conv1 of the next, as one launch (the
 * consecutive-operator merge of the Inspur conv-merge article, section 2.1, across
 * the block boundary of the section 2.2 structure):
 *   y  = conv(t_blk; d3, RESIDUAL = residual_blk)    the block output, stored to y_blk
 *   t1 = conv(y; d1)                                 the next block's conv1, stored to t1_blk
 * y_blk is written (it is the next block's shortcut) but conv1 reads y on chip, so
 * the block output is read once less.  The result is bit-identical to
 * ifx_conv_fused(d3) followed by ifx_conv_fused(d1) on y_blk.
 *   d3   1x1, stride 1, pad 0, flags IFX_RESIDUAL | IFX_RELU, c_in <= 64,
 *        c_out = 256 (the block outputs of a ResNet-50 res2 stage); with
 *        IFX_OUT_EVEN added, y_blk receives only the even rows and columns of y,
 *        packed as [n, 8, ceil(h/2), ceil(w/2), 32] (what the next block's
 *        stride-2 projection reads: it then runs with stride 1 on that tensor),
 *        while conv1 still sees every pixel
 *   d1   1x1, stride 1, pad 0, flags IFX_RELU or 0, c_in = d3.c_out,
 *        c_out = 64 or 128, same n and the spatial size of d3's output
 *   t_blk, residual_blk: packed inputs of d3; y_blk, t1_blk: packed outputs;
 *   w3_blk, bias3, mult3, shift3 / w1_blk, bias1, mult1, shift1: as for
 *   ifx_conv_fused.  Buffers must not overlap.  Other shapes or flags give
 *   IFX_E_UNSUPPORTED (use two ifx_conv_fused calls); nothing is launched on an
 *   error.  ifx_net_forward chains every block whose shortcut is its input with
 *   the following block this way, with IFX_OUT_EVEN when the following block has a
 *   stride-2 projection (its only other reader of y).
 */
ifx_status ifx_conv_chain_fused(const ifx_conv_desc *d3, const int8_t *t_blk, const int8_t *w3_blk,
                                const int32_t *bias3, const int32_t *mult3, const int32_t *shift3,
                                const int8_t *residual_blk, int8_t *y_blk, const ifx_conv_desc *d1,
                                const int8_t *w1_blk, const int32_t *bias1, const int32_t *mult1,
                                const int32_t *shift1, int8_t *t1_blk, void *stream);

/*
 * Conv3 of a bottleneck whose shortcut is a 1x1 projection, together with that
 * projection and with conv1 of the next block, as one launch (the section 2.1
 * merge of ifx_conv_chain_fused, for the first block of a stage):
 *   sc = conv(x_blk; dp)                           the projection, no ReLU; not stored
 *   y  = conv(t_blk; d3, RESIDUAL = sc)            the block output, stored to y_blk
 *   t1 = conv(y; d1)                               the next block's conv1, stored to t1_blk
 * Bit-identical to ifx_conv_proj_fused(d3, dp) followed by ifx_conv_fused(d1) on
 * y_blk; conv1 reads y on chip.
 *   d3   1x1, stride 1, pad 0, flags IFX_RESIDUAL | IFX_RELU, c_in <= 64, c_out = 256
 *   dp   1x1, stride 1, pad 0, flags 0, c_in <= 64, c_out = d3.c_out, the same
 *        n, h and w as d3
 *   d1   1x1, stride 1, pad 0, flags IFX_RELU or 0, c_in = d3.c_out, c_out = 64,
 *        the same n, h and w
 *   Pointers as for ifx_conv_proj_fused and ifx_conv_chain_fused (device, packed,
 *   16-byte aligned, not overlapping).  Other shapes or flags give
 *   IFX_E_UNSUPPORTED; nothing is launched on an error.  ifx_net_forward runs the
 *   first block of a stage with the next block's conv1 this way where it applies
 *   (res2.1 -> res2.2 of ResNet-50).
 */
ifx_status ifx_conv_proj_chain_fused(const ifx_conv_desc *d3, const int8_t *t_blk, const int8_t *w3_blk,
                                     const int32_t *bias3, const int32_t *mult3, const int32_t *shift3,
                                     const ifx_conv_desc *dp, const int8_t *x_blk, const int8_t *wp_blk,
                                     const int32_t *biasp, const int32_t *multp, const int32_t *shiftp,
                                     int8_t *y_blk, const ifx_conv_desc *d1, const int8_t *w1_blk,
                                     const int32_t *bias1, const int32_t *mult1, const int32_t *shift1,
                                     int8_t *t1_blk, void *stream);

/*
 * Bottleneck block (Inspur conv-merge article, section 2.2):
 *   t1 = conv(x; d[0] 1x1, RELU)          c1
 *   t2 = conv(t1; d[1] 3x3 stride s, RELU) c2
 *   sc = x, or conv(x; d[3] 1x1 stride s, no ReLU) when has_proj
 *   y  = conv(t2; d[2] 1x1, RESIDUAL=sc, RELU)   c3
 * When c3 and the projection are 1x1 and the projection has no ReLU, both run
 * as ifx_conv_proj_fused and sc is not materialised.
 * Descriptors carry the batch in n.  Their flags must be: d[0], d[1] without
 * RESIDUAL/MAXPOOL/OUT_I32, d[2] with RESIDUAL, d[3] without RESIDUAL/MAXPOOL/
 * OUT_I32.  t1, t2 and sc live in the caller's workspace, and so do the int32
 * partial sums of a convolution that has few output tiles and a long
 * reduction (a small batch): it is split over K into parts whose sums a
 * second kernel adds (integer addition, so the result is the same in any
 * order) before applying the convolution's epilogue.
 */
typedef struct {
    ifx_conv_desc d[4]; /* c1, c2, c3, projection */
    int32_t has_proj;
    const int8_t *w_blk[4];
    const int32_t *bias[4];
    const int32_t *mult[4];
    const int32_t *shift[4];
} ifx_block_params;

/* Host-only: workspace bytes ifx_block_forward needs for p (0 if invalid). */
size_t ifx_block_workspace_bytes(const ifx_block_params *p);

ifx_status ifx_block_forward(const ifx_block_params *p, const int8_t *x_blk, int8_t *y_blk, void *ws,
                             size_t ws_bytes, void *stream);

/*
 * ifx_block_forward for callers that cannot allocate device memory (code
 * running under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same block, bit-identical results, with t1, t2, the
 * projection shortcut and the split-K partial sums in a scratch array the
 * library holds in device memory (IFX_BLOCK_SCRATCH_BYTES per device, for the
 * life of the process) instead of a caller workspace.  The call allocates
 * nothing.  A block whose ifx_block_workspace_bytes() exceeds
 * IFX_BLOCK_SCRATCH_BYTES returns IFX_E_WORKSPACE and launches nothing.
 * Every call on one device shares that device's scratch, which keeps the last
 * call's contents (nothing in it has to start cleared): calls that overlap in
 * time on one device, on any streams, race.  The first call on a device looks
 * up the scratch's device address (host-side, no device work).
 */
#define IFX_BLOCK_SCRATCH_BYTES (64u << 20)

ifx_status ifx_block_forward_noalloc(const ifx_block_params *p, const int8_t *x_blk, int8_t *y_blk,
                                     void *stream);

/*
 * ResNet-50-shaped network: stem (7x7/s2/p3 CONV+BN+RELU+MAXPOOL, DiDi IFX
 * blog) -> bottleneck blocks -> global average pool to int8 (round half away
 * from zero of the mean) -> FC with int32 logits = a . W^T + bias.
 * The n field of every descriptor inside p is ignored: the batch is the `n`
 * argument.  fc_w_blk is the FC weight [fc_out, fc_in] packed as a 1x1
 * convolution (ifx_pack_weights with kh = kw = 1, c_in = fc_in,
 * c_out = fc_out).  sub_batch > 0 runs the network over consecutive groups
 * of sub_batch images, one after another on `stream`; 0 runs the whole batch
 * at once, and a batch of 192 or more images then runs as two halves at the
 * same time: the first on `stream`, the second on a stream the library
 * creates (default priority, once per device, kept for the process), forked
 * from `stream` and joined back into it by events, so every result is still
 * ordered on `stream`.  Each half has its own part of the workspace.  Results
 * are identical for every sub_batch.  Calls from several host threads on one
 * device share that library stream (their second halves are serialised
 * there, still correct).  While `stream` is being captured into a graph both
 * halves run on `stream` itself, one after the other: the shared library
 * stream never joins a capture.
 *   x_blk   packed input [n, ceil(stem.c_in/32), stem.h, stem.w, 32], or the
 *           compact [n, stem.h, stem.w, stem.c_in] image when stem.flags has
 *           IFX_INPUT_NHWC
 *   logits  int32 [n, fc_out]
 */
typedef struct {
    ifx_conv_desc stem;
    const int8_t *stem_w;
    const int32_t *stem_bias, *stem_mult, *stem_shift;
    int32_t n_blocks;
    const ifx_block_params *blocks;
    const int8_t *fc_w_blk;
    const int32_t *fc_bias;
    int32_t fc_in, fc_out;
    int32_t sub_batch;
} ifx_net_params;

/* Host-only: workspace bytes ifx_net_forward needs for p at batch n (0 if invalid). */
size_t ifx_net_workspace_bytes(const ifx_net_params *p, int32_t n);

ifx_status ifx_net_forward(const ifx_net_params *p, const int8_t *x_blk, int32_t *logits, int32_t n,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * Fixed-shape network launches as one HIP graph (the batch-1 latency setting of
 * the DiDi IFX DAWNBench blog, whose ResNet26 inference is timed per image):
 * ifx_net_graph_create records the kernels ifx_net_forward(p, x_blk, logits,
 * n, ws, ws_bytes, .) enqueues, with exactly these buffers, into a graph;
 * ifx_graph_launch enqueues that whole sequence with one call (results as
 * ifx_net_forward; the buffers must stay valid and the parameter arrays p
 * points at unchanged while the graph exists); ifx_graph_destroy frees it.
 * Validation as ifx_net_forward; nothing runs during creation.  The recording
 * uses a stream (and, for two halves, a second stream and two events) of its
 * own, created for it and destroyed after it, so recording is independent of
 * other threads' calls.  The graph handle is host state owned by the library
 * until ifx_graph_destroy (NULL is accepted there).
 */
typedef struct ifx_graph_s *ifx_graph;

ifx_status ifx_net_graph_create(const ifx_net_params *p, const int8_t *x_blk, int32_t *logits, int32_t n, void *ws,
                                size_t ws_bytes, ifx_graph *out);
ifx_status ifx_graph_launch(ifx_graph g, void *stream);
ifx_status ifx_graph_destroy(ifx_graph g);

/*
 * Float -> fixed-point epilogue parameters of one conv + BN layer (BN folding
 * into the fused convolution: DiDi IFX DAWNBench blog, inference section, and
 * Inspur conv-merge article, section 3.4; the quantisation scales come from a
 * calibration outside this library, DiDi blog quantisation section).
 * Symmetric int8 quantisation, real = scale * code.  For output channel o:
 *   M[o] = gamma s_x s_w / (s_y sqrt(var + eps))
 *   B[o] = (b_conv - mean) / (s_x s_w) + beta sqrt(var + eps) / (gamma s_x s_w)
 * so that the layer's output code is M[o] * (acc + B[o]); the results are
 *   bias[o]  = round_half_away_from_zero(B[o])
 *   mult[o], shift[o] with M[o] ~= mult * 2^-(31 + shift), mult in [2^30, 2^31)
 *            (rounded half away from zero; shift capped at 31 with mult below
 *            2^30 for tiny scales)
 *   status[o] = 0 ok; 1 M >= 1 (not representable: mult = 2^31 - 1, shift 0);
 *               2 M <= 0 or not finite (bias = mult = shift = 0);
 *               3 bias outside int32 (clamped).
 * Computed on the device in IEEE double, one rounding per operation in the
 * order of the formulas, no fused multiply-add: results are reproducible.
 * A shortcut added by IFX_RESIDUAL must already be in the output's scale s_y.
 * All array pointers are DEVICE pointers of c_out elements (w_scale has 1
 * element when w_per_channel is 0; conv_bias may be NULL for no conv bias).
 */
typedef struct {
    int32_t c_out;
    float x_scale, y_scale, eps;
    int32_t w_per_channel;
    const float *w_scale, *conv_bias, *gamma, *beta, *mean, *var;
} ifx_bn_fold;

ifx_status ifx_fold_bn(const ifx_bn_fold *f, int32_t *bias, int32_t *mult, int32_t *shift, int32_t *status,
                       void *stream);

/*
 * Quantisation of the input image on the device (Alibaba inference article,
 * Hanguang 800 section: the engine runs on integer data, and the
 * quantisation before it, which had run on the host and taken most of the
 * latency, moves into the accelerated pre-processing).  The result is the
 * compact int8 NHWC image the stem reads with IFX_INPUT_NHWC, in the path's
 * symmetric codes (real = s_x * code).  Element i of the NHWC tensor
 * (channels innermost) belongs to channel ch = i % c:
 *   ifx_quantize_f32: code = sat8(round_half_away(x * mult[ch]))
 *   ifx_quantize_u8:  code = sat8(round_half_away(((float)u - mean[ch]) * mult[ch]))
 *                     (an ImageNet-style per-channel mean subtraction and
 *                     1 / (std * s_x) scaling fused into the quantisation)
 * One IEEE single-precision operation at a time (round to nearest even, no
 * fused multiply-add), round half away from zero, saturation to [-128, 127];
 * a NaN product gives code 0 and an infinite one saturates.
 *   x      DEVICE, `count` float32 or uint8 elements, 16-byte aligned
 *   q      DEVICE, `count` int8, 16-byte aligned, not overlapping x
 *   mean, mult  DEVICE float32 [c], 4-byte aligned
 *   count  0 <= count < 2^31 and a multiple of c (c >= 1)
 * Errors (nothing is launched): IFX_E_NULL, IFX_E_SHAPE, IFX_E_ALIGN.
 */
ifx_status ifx_quantize_f32(const float *x, int8_t *q, int64_t count, int32_t c, const float *mult, void *stream);
ifx_status ifx_quantize_u8(const uint8_t *x, int8_t *q, int64_t count, int32_t c, const float *mean,
                           const float *mult, void *stream);

/*
 * Dequantisation of int32 results, the FC's logits, after the engine (the
 * same article):  y = (float)q * scale  (the int32 -> float32 conversion
 * rounds to nearest even beyond 2^24; then one single-precision multiply).
 *   q, y   DEVICE, `count` elements each, 16-byte aligned, not overlapping
 *   count  0 <= count < 2^31
 * Errors (nothing is launched): IFX_E_NULL, IFX_E_SHAPE, IFX_E_ALIGN.
 */
ifx_status ifx_dequantize_i32(const int32_t *q, float *y, int64_t count, float scale, void *stream);

/*
 * Host-only: the kernel instance ifx_conv_fused(d, ...) launches, named as
 * profilers print it (e.g. "igemm_kernel<3, 3, 128, 128, 2, false, true,
 * false>"), written NUL-terminated into buf.  The name comes from the very
 * dispatch code of the launch, run with launching switched off, so it cannot
 * drift from what runs; it lets a measurement attribute per-kernel times.
 * ifx_conv_proj_kernel_name does the same for ifx_conv_proj_fused(d3, dp).
 * Validation as the launching calls; IFX_E_WORKSPACE when len is too small.
 */
ifx_status ifx_conv_kernel_name(const ifx_conv_desc *d, char *buf, size_t len);
ifx_status ifx_conv_proj_kernel_name(const ifx_conv_desc *d3, const ifx_conv_desc *dp, char *buf, size_t len);
/* The same for ifx_conv_chain_fused(d3, d1); IFX_E_UNSUPPORTED when the pair does not chain. */
ifx_status ifx_conv_chain_kernel_name(const ifx_conv_desc *d3, const ifx_conv_desc *d1, char *buf, size_t len);
/* The same for ifx_conv_proj_chain_fused(d3, dp, d1). */
ifx_status ifx_conv_proj_chain_kernel_name(const ifx_conv_desc *d3, const ifx_conv_desc *dp,
                                           const ifx_conv_desc *d1, char *buf, size_t len);

/* Host-only: a static, human-readable name of a status. */
const char *ifx_status_string(ifx_status s);

/* Host-only: the hipError_t behind the calling thread's last IFX_E_HIP (0 if none). */
int32_t ifx_last_hip_error(void);

/* Host-only: library version, major * 10000 + minor * 100 + patch. */
int32_t ifx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IFX_H */
