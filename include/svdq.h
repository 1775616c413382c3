/*
 * svdq.h - C ABI of the MI355X (gfx950) SVDQuant W4A4 NVFP4 linear layer.
 *
 * The layer (model card "nunchaku-z-image-turbo-svdq", section "What's stored
 * on disk", runtime reconstruction formula):
 *
 *   y = scaled_mma(quant(x * smooth), qweight, ascales, wscales) * wtscale * wcscales
 *       + (x @ proj_down) @ proj_up^T + bias
 *
 * NVFP4 = E2M1 values with one float8_e4m3fn scale per 16 consecutive K
 * elements (same card, header). On-disk tensors, all canonical row-major
 * (same section, tensor table):
 *   qweight   [N, K/2] int8   two E2M1 codes per byte, low nibble = even k
 *   wscales   [K/16, N] e4m3fn
 *   wcscales  [N] bf16        per output channel
 *   wtscale   [1] bf16        global alpha (read on the device)
 *   smooth    [K] bf16        smooth_factor
 *   proj_down [K, R] bf16     SVD residual, down
 *   proj_up   [N, R] bf16     SVD residual, up
 * Runtime tensors the card leaves unspecified, fixed by this library:
 *   x         [M, K] bf16     activations
 *   qact      [M, K/2] u8     activation codes, low nibble = even k
 *   ascales   [K/16, M] e4m3fn activation block scales (mirrors wscales)
 *   lora_act  [M, R] bf16     x @ proj_down (raw x, not smoothed)
 *   bias      [N] bf16        optional (NULL = no bias)
 *   y         [M, N] bf16     output, round to nearest even
 *
 * Activation quantisation rule (the pages only name "quant"): per row and
 * 16-block, v = x * smooth in fp32 (exact), s = max|v| / 6 rounded to e4m3
 * (nearest-even, saturating at 448), codes = E2M1 nearest-even of |v| / s
 * (saturating at 6) with the sign bit of v; a zero scale gives zero codes.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers on the current HIP device, except where a
 *    comment says otherwise; sizes are element counts. `stream` is a
 *    hipStream_t (NULL = the null stream). Work is enqueued on `stream` in
 *    order; no entry point synchronises the host or allocates device memory,
 *    and none keeps a pointer after it returns. The caller owns every buffer
 *    and keeps it alive until the stream has passed the enqueued work.
 *  - Every argument is checked on the host before any HIP call. On error
 *    nothing is enqueued and outputs are untouched; svdq_last_error() then
 *    returns a message for the calling thread. No C++ exception crosses
 *    the ABI. Entry points are thread-safe and reentrant.
 *  - M == 0 or N == 0 is a valid empty problem: nothing is enqueued.
 *  - K must be a positive multiple of 16 (the NVFP4 block). R must be 0 or a
 *    multiple of 16 (SVDQ_ERR_UNSUPPORTED otherwise). Every pointer must be
 *    16-byte aligned (SVDQ_ERR_ALIGN).
 *  - The quantisation step (also inside svdq_linear_w4a4) needs x, proj_down,
 *    lora_act and the packed activation buffer each below 2 GiB, and the
 *    GEMM on packed operands needs the packed activation and packed weight
 *    buffers each below 2 GiB (SVDQ_ERR_UNSUPPORTED otherwise).
 *  - NaN or Inf inputs are not checked; results are then unspecified.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_NULL = 1,         /* a required pointer is NULL                      */
  SVDQ_ERR_SHAPE = 2,        /* negative size, K not a positive multiple of 16  */
  SVDQ_ERR_UNSUPPORTED = 3,  /* valid for the format, outside these kernels      */
  SVDQ_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned                */
  SVDQ_ERR_WORKSPACE = 5,    /* workspace (or packed buffer) too small          */
  SVDQ_ERR_ALIAS = 6,        /* an output overlaps an input or another output   */
  SVDQ_ERR_HIP = 7,          /* a HIP launch reported an error                  */
  SVDQ_ERR_INVALID = 8       /* bad enum value or argument combination          */
} svdq_status;

/* Weight layouts accepted by the GEMM entry points. */
enum {
  SVDQ_WEIGHT_CANONICAL = 0, /* qweight [N, K/2] + wscales [K/16, N] as on disk            */
  SVDQ_WEIGHT_PACKED = 1     /* one buffer from svdq_repack_weight; wscales must be NULL    */
};

/* Layouts of quantised activations (codes + scales).                                     */
enum {
  SVDQ_ACT_CANONICAL = 0,    /* qact [M, K/2] + ascales [K/16, M]                            */
  SVDQ_ACT_PACKED = 1,       /* one buffer of svdq_packed_act_bytes(M, K) in the packed
                                weight layout with rows = tokens; ascales must be NULL.
                                Rows beyond M in the last 32-row panel are unspecified;
                                positions beyond K are zero.                               */
  SVDQ_ACT_MXFP4 = 2         /* the MXFP4 variant's operand instead of NVFP4 (see the
                                MXFP4 section below): qact = MX codes
                                (svdq_mx_codes_bytes(M, K)), ascales = MX scales
                                (svdq_mx_scales_bytes(M, K)); K % 128 == 0, dynamic
                                scales only (svdq_quantize_act).                          */
};

#define SVDQ_ABI_VERSION 1

int svdq_abi_version(void);
const char* svdq_status_string(int status);
/* Message describing the last error returned on the calling thread ("" if none). */
const char* svdq_last_error(void);
/* Debug mode: 1 when the environment variable SVDQ_DEBUG was 1, true, yes or on
 * (any case) when the library first read it (once per process), else 0. In debug
 * mode every entry point synchronises its stream after each kernel launch (not
 * while the stream is being captured into a graph) and returns SVDQ_ERR_HIP,
 * naming the launch, if the device reported an error. */
int svdq_debug_mode(void);

/* Tile shape of the W4A4 GEMM on packed operands (svdq_gemm_w4a4 with packed
 * activations, svdq_linear_w4a4 with a packed weight, and the gated and static
 * variants), for tests and tuning. Process-wide; it applies to launches made
 * after the call.
 *   tile 0: automatic (the default): the shape with the fewest estimated rounds
 *           of workgroups, weighted by each shape's measured time per round;
 *        1: 256 x 320, 2: 256 x 256, 3: 128 x 320, 4: 128 x 160 outputs per
 *           workgroup (the gated GEMM cannot take 4 and chooses automatically).
 * Every shape gives bit-identical results. The previous value goes to *previous
 * when previous is not NULL. SVDQ_ERR_INVALID (nothing changed) for a tile
 * outside 0..4. Host only: no device call. */
int svdq_set_gemm_tile(int tile, int* previous);

/*
 * Activation quantisation quant(x * smooth), and the down-projection of the
 * low-rank branch x @ proj_down (model card, section "What's stored on disk":
 * the activation operand of scaled_mma and the (x @ proj_down) factor).
 *
 *   x [M, K] bf16, smooth [K] bf16          inputs
 *   act_layout SVDQ_ACT_CANONICAL: qact [M, K/2] u8, ascales [K/16, M] u8;
 *              SVDQ_ACT_PACKED: qact = packed buffer (svdq_packed_act_bytes(M, K)
 *              bytes), ascales NULL. Outputs follow the rule in the file header.
 *              SVDQ_ACT_MXFP4: qact, ascales = the MXFP4 variant's code and scale
 *              buffers, as svdq_quantize_act_mxfp4 writes them (bit for bit), with
 *              the down-projection in the same pass; K % 128 == 0 and
 *              svdq_quantize_act_static rejects it (SVDQ_ERR_UNSUPPORTED).
 *   proj_down [K, R] bf16, lora_act [M, R] bf16: used when R > 0 (both
 *     required then); lora_act = bf16(x @ proj_down) with fp32 accumulation.
 *   workspace: device scratch of at least svdq_quantize_act_workspace_bytes(M, K, R)
 *     bytes (SVDQ_ERR_WORKSPACE if smaller). It holds fp32 partial sums of the
 *     down-projection when K is split across workgroups, which happens for
 *     R > 0 and small M; otherwise the size is 0 and workspace may be NULL.
 *     Its contents on entry do not matter and are unspecified afterwards.
 * qact and ascales are bit-exact functions of x and smooth.
 */
size_t svdq_quantize_act_workspace_bytes(int64_t M, int64_t K, int64_t R);
size_t svdq_packed_act_bytes(int64_t M, int64_t K);
int svdq_quantize_act(const void* x, const void* smooth, int64_t M, int64_t K,
                      const void* proj_down, int64_t R, int act_layout,
                      void* qact, void* ascales, void* lora_act,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Load-time weight repack into the library's MFMA-order layout, and its
 * inverse (model card, section "Why row-major": a one-shot pack at load time
 * forming a bit-exact pair with its unpack; section "Conversion source":
 * round trip verified bit-exact).
 *
 * Layout: n-panels of 32 channels, k-panels of 64 (four 16-blocks);
 * NP = ceil(N/32), KP = ceil(K/64). Code region: chunk (p, q) of 1024 bytes
 * at offset 1024*(p*NP+q); dword (h*32+c)*4+t holds the 4 canonical qweight
 * bytes of channel 32q+c at k = 64p+16t+8h .. +7. Scale region after it:
 * chunk (p, q) of 128 bytes at 1024*KP*NP + 128*(p*NP+q); byte c*4+t holds
 * wscales[4p+t, 32q+c]. Positions outside N or K are zero.
 *
 * svdq_repack_weight: qweight [N, K/2] u8 + wscales [K/16, N] u8 -> packed
 *   (packed_bytes >= svdq_repack_weight_bytes(N, K), else SVDQ_ERR_WORKSPACE).
 * svdq_unpack_weight: packed -> qweight_out, wscales_out (canonical), exact inverse.
 */
size_t svdq_repack_weight_bytes(int64_t N, int64_t K);
int svdq_repack_weight(const void* qweight, const void* wscales, int64_t N, int64_t K,
                       void* packed, size_t packed_bytes, void* stream);
int svdq_unpack_weight(const void* packed, size_t packed_bytes, int64_t N, int64_t K,
                       void* qweight_out, void* wscales_out, void* stream);

/*
 * The scaled GEMM with the low-rank up-projection and the epilogue, from
 * already quantised activations (model card, section "What's stored on disk",
 * runtime formula without the quant step):
 *
 *   y = bf16( scaled_mma(qact, weight, ascales, wscales) * wtscale * wcscales[n]
 *             + lora_act @ proj_up^T + bias[n] )
 *
 *   qact [M, K/2] u8 + ascales [K/16, M] u8 (act_layout SVDQ_ACT_CANONICAL), or
 *     a packed activation buffer with ascales NULL (SVDQ_ACT_PACKED), with either
 *     weight layout; lora_act [M, R] bf16 (R > 0)
 *   weight: qweight [N, K/2] (SVDQ_WEIGHT_CANONICAL, wscales [K/16, N] given)
 *           or a packed buffer (SVDQ_WEIGHT_PACKED, wscales NULL)
 *   wcscales [N] bf16, wtscale [1] bf16, proj_up [N, R] bf16 (R > 0), bias [N] bf16 or NULL
 *   y [M, N] bf16 output; must not overlap any input.
 * The main term is exact per 16-block (operands are dequantised exactly to
 * f16 and multiplied on the matrix cores with fp32 accumulation); the sum
 * over blocks and the epilogue round in fp32.
 */
int svdq_gemm_w4a4(const void* qact, const void* ascales, int act_layout, const void* lora_act,
                   const void* weight, const void* wscales, int weight_layout,
                   const void* wcscales, const void* wtscale, const void* proj_up,
                   const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                   void* y, void* stream);

/*
 * The whole layer: svdq_quantize_act into the workspace (packed activations),
 * then svdq_gemm_w4a4 on them with the weight in either layout.
 *   x [M, K] bf16, smooth [K] bf16, weight/wscales/weight_layout as above,
 *   wcscales, wtscale, proj_down [K, R], proj_up [N, R], bias (or NULL),
 *   y [M, N] bf16; workspace of at least svdq_linear_workspace_bytes(M, N, K, R)
 *   bytes (no initialisation needed).
 */
size_t svdq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t R);
int svdq_linear_w4a4(const void* x, const void* smooth,
                     const void* weight, const void* wscales, int weight_layout,
                     const void* wcscales, const void* wtscale,
                     const void* proj_down, const void* proj_up, const void* bias,
                     int64_t M, int64_t N, int64_t K, int64_t R,
                     void* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Static (calibrated) activation scales: the NVFP4 datatype-variant row's second
 * half. The blog page "Z-Image NVFP4 ..." says the Comfy-Org Z-Image Turbo NVFP4
 * checkpoint uses calibrated static activation scales; the pages give no rule.
 * Reading (NVFP4's two-level form): a per-tensor global activation scale g, fixed
 * offline from calibration activations, and per-16 e4m3 block scales still
 * computed per call relative to it:
 *   s = e4m3(max|v| / (6 g)) (nearest even, saturating at 448) -> ascales,
 *   codes = E2M1 nearest even of |v| / (dec(s) * g), sign of v kept,
 * with v = x * smooth in fp32. The GEMM's main term then carries g:
 *   y = bf16( scaled_mma(...) * g * wtscale * wcscales[n] + lora_act @ proj_up^T + bias[n] ).
 * g = 1 gives the dynamic rule exactly. Blocks above 6 * 448 * g saturate.
 *
 *   act_gscale: bf16 [1] on the device, a positive normal value in [2^-64, 2^64]
 *     (outside that the results are unspecified); bf16 precision keeps every
 *     rounding decision exact in fp32.
 * svdq_calibrate_act_gscale: act_gscale = bf16(max |x * smooth| / (6 * 448)) over
 *   a calibration batch x [M, K] (M >= 1), or 1 when that maximum is 0; workspace
 *   of svdq_calibrate_workspace_bytes(M, K) bytes; x below 2 GiB.
 * svdq_quantize_act_static, svdq_linear_w4a4_static: as svdq_quantize_act and
 *   svdq_linear_w4a4 with the block scales relative to *act_gscale (same
 *   layouts, workspace sizes and errors; act_gscale NULL is SVDQ_ERR_NULL).
 */
size_t svdq_calibrate_workspace_bytes(int64_t M, int64_t K);
int svdq_calibrate_act_gscale(const void* x, const void* smooth, int64_t M, int64_t K, void* act_gscale,
                              void* workspace, size_t workspace_bytes, void* stream);
int svdq_quantize_act_static(const void* x, const void* smooth, const void* act_gscale, int64_t M, int64_t K,
                             const void* proj_down, int64_t R, int act_layout, void* qact, void* ascales,
                             void* lora_act, void* workspace, size_t workspace_bytes, void* stream);
int svdq_linear_w4a4_static(const void* x, const void* smooth, const void* act_gscale,
                            const void* weight, const void* wscales, int weight_layout,
                            const void* wcscales, const void* wtscale,
                            const void* proj_down, const void* proj_up, const void* bias,
                            int64_t M, int64_t N, int64_t K, int64_t R,
                            void* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The whole layer without allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses that
 * forbid allocation. Same arguments and results as svdq_linear_w4a4 (bit for
 * bit: the same kernels run), minus the workspace: the library keeps it in a
 * static device array of svdq_noalloc_scratch_bytes() bytes (64 MiB), which
 * every GPU the library runs on holds until the process ends. A problem whose
 * svdq_linear_workspace_bytes(M, N, K, R) exceeds that returns
 * SVDQ_ERR_WORKSPACE before anything is enqueued. Calls that overlap on one
 * GPU (different streams or host threads) share the array and race; serialise
 * them. No hipMalloc, hipFree or other allocating call is made.
 */
size_t svdq_noalloc_scratch_bytes(void);
int svdq_linear_w4a4_noalloc(const void* x, const void* smooth,
                             const void* weight, const void* wscales, int weight_layout,
                             const void* wcscales, const void* wtscale,
                             const void* proj_down, const void* proj_up, const void* bias,
                             int64_t M, int64_t N, int64_t K, int64_t R, void* y, void* stream);

/*
 * FFN neighbour (gated): the DiT feed-forward layers w1 and w3 (blog page
 * "Z-Image NVFP4 ...", layer table and its key insight: FFN w1, w2, w3 are the
 * NVFP4 layers) run as ONE SVDQuant layer with 2F output channels that share x,
 * smooth, wtscale, proj_down and R: channels [0, F) are w1, [F, 2F) are w3.
 * Its output never leaves the chip: the epilogue combines it as
 *   h[:, c] = bf16( silu(y[:, c]) * y[:, F + c] ),  silu(z) = z / (1 + exp(-z)),
 * with y the fp32 layer result before rounding (the pages do not state the
 * combination; this gated form is the reading). h [M, F] bf16 is w2's input.
 *
 *   weight: PACKED layout of the 2F-channel layer (svdq_repack_weight with
 *     N = 2F); wcscales [2F], proj_up [2F, R], bias [2F] bf16 or NULL.
 *   F must be a multiple of 32 (SVDQ_ERR_UNSUPPORTED otherwise).
 *   svdq_gemm_w4a4_gated: packed activations (as svdq_gemm_w4a4 with
 *     SVDQ_ACT_PACKED) and lora_act [M, R].
 *   svdq_linear_w4a4_gated: the whole step from x, with a workspace of
 *     svdq_linear_gated_workspace_bytes(M, F, K, R) bytes.
 * Other conventions as for svdq_gemm_w4a4 / svdq_linear_w4a4.
 */
int svdq_gemm_w4a4_gated(const void* qact, const void* lora_act, const void* weight,
                         const void* wcscales, const void* wtscale, const void* proj_up,
                         const void* bias, int64_t M, int64_t F, int64_t K, int64_t R, void* h,
                         void* stream);
size_t svdq_linear_gated_workspace_bytes(int64_t M, int64_t F, int64_t K, int64_t R);
int svdq_linear_w4a4_gated(const void* x, const void* smooth, const void* weight,
                           const void* wcscales, const void* wtscale, const void* proj_down,
                           const void* proj_up, const void* bias, int64_t M, int64_t F, int64_t K,
                           int64_t R, void* h, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The gated step that also prepares w2's input (the rest of the FFN neighbour
 * fusion): as svdq_gemm_w4a4_gated, and the epilogue additionally quantises the
 * bf16 h it writes with w2's smooth factor, by the activation rule of the file
 * header, into next_qact: the packed activation layout of an [M, F] activation
 * (SVDQ_ACT_PACKED, svdq_packed_act_bytes(M, F) bytes), ready for
 * svdq_gemm_w4a4 with w2's packed weight. Each output tile of the gated GEMM
 * holds whole 16-blocks of h's rows, so this is local to the tile; w2's
 * down-projection h @ proj_down2 needs whole rows of h and is left to
 * svdq_lowrank_down. F must be a multiple of 64 (SVDQ_ERR_UNSUPPORTED).
 *   next_smooth [F] bf16 (w2's smooth_factor); next_qact must not overlap any input or h.
 * The codes and scales equal svdq_quantize_act(h, next_smooth) bit for bit.
 *
 * svdq_lowrank_down: lora_act [M, R] = bf16(x @ proj_down) alone (fp32
 * accumulation), x [M, K] bf16, proj_down [K, R] bf16, with a workspace of
 * svdq_quantize_act_workspace_bytes(M, K, R) bytes (fp32 K-split partial sums).
 */
int svdq_gemm_w4a4_gated_quant(const void* qact, const void* lora_act, const void* weight,
                               const void* wcscales, const void* wtscale, const void* proj_up,
                               const void* bias, int64_t M, int64_t F, int64_t K, int64_t R, void* h,
                               const void* next_smooth, void* next_qact, size_t next_qact_bytes, void* stream);
int svdq_lowrank_down(const void* x, const void* proj_down, int64_t M, int64_t K, int64_t R, void* lora_act,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Linears kept in bf16. A mixed-precision NVFP4 model leaves some linears
 * unquantised (blog page "Z-Image NVFP4 ...", variant table: the "Ultra"
 * variant keeps attention qkv/out and every linear of blocks 0-4 and 25-29 in
 * bf16, and its key insight names attention as the quantisation-sensitive
 * part). Such a layer is the original linear
 *
 *   y = bf16( x @ weight^T + bias[n] )
 *
 *   x [M, K] bf16, weight [N, K] bf16 (row-major, as stored in a bf16
 *   checkpoint), bias [N] bf16 or NULL, y [M, N] bf16 (round to nearest even);
 *   y must not overlap any input. Products are exact and accumulate in fp32
 *   on the matrix cores. K: a positive multiple of 16; M, N up to 2^24.
 *   Backend: the library's own kernel, or hipBLASLt (no workspace) for large
 *   products (M*N*K >= 1.6e10) whose grid of 256 x 320 output tiles is not a
 *   whole number of 256-workgroup rounds; a shape first seen while the stream
 *   is capturing takes the library's kernel. The environment variable
 *   SVDQ_BF16_GEMM=hip or =blaslt (read on every call) forces one of the two.
 *   Both meet the same bound: one bf16 rounding of an fp32 accumulation.
 */
int svdq_linear_bf16(const void* x, const void* weight, const void* bias, int64_t M, int64_t N,
                     int64_t K, void* y, void* stream);

/*
 * Load-time SVDQuant weight preparation: from a bf16 weight and its smooth
 * factor, the tensors a prepared layer stores (model card, section "What's
 * stored on disk": qweight, wscales, wcscales, wtscale, proj_down, proj_up;
 * the card cites SVDQuant but does not give the steps, which are read from
 * what the runtime formula needs):
 *   1. Ws = W / smooth[k];
 *   2. rank-R split by the randomized range finder: Y = Ws omega, `iters`
 *      rounds of Y = Ws orth(Ws^T orth(Y)), Q = orth(Y) (Cholesky QR, twice);
 *      proj_up = bf16(Q), proj_down = bf16(smooth[k] * (Ws^T Q)[k, :]);
 *   3. E = (W - proj_up proj_down^T) / smooth[k] in fp64 with the bf16
 *      factors (r summed in order), exact up to that order;
 *   4. wtscale = 1, wcscales[n] = bf16(max_k |E[n, k]| / (6 * 448));
 *   5. W' = bf16(E / wcscales[n]) (0 where wcscales is 0), quantised with the
 *      activation rule and smooth = 1 into qweight [N, K/2], wscales [K/16, N].
 *
 *   weight [N, K] bf16 row-major; smooth [K] bf16; omega [K, R] fp32, a
 *   Gaussian test matrix the caller draws (deterministic given omega);
 *   outputs as listed, canonical layout (repack with svdq_repack_weight).
 *   R: 0 (no low-rank part; omega, proj_down, proj_up may be NULL) or a
 *   multiple of 16, at most 128 and at most min(N, K) (SVDQ_ERR_UNSUPPORTED);
 *   iters 0..16 (SVDQ_ERR_INVALID). workspace: at least
 *   svdq_prepare_workspace_bytes(N, K, R) bytes, no initialisation needed.
 *   W, N*K*2 bytes, must stay below 2 GiB (SVDQ_ERR_UNSUPPORTED).
 * svdq_prepare_residual runs steps 3-5 for given factors (proj_down,
 *   proj_up are inputs there); given the factors, its outputs equal the float64
 *   definition above bit for bit.
 */
size_t svdq_prepare_workspace_bytes(int64_t N, int64_t K, int64_t R);
int svdq_prepare_weight(const void* weight, const void* smooth, const void* omega, int64_t N, int64_t K,
                        int64_t R, int iters, void* qweight, void* wscales, void* wcscales, void* wtscale,
                        void* proj_down, void* proj_up, void* workspace, size_t workspace_bytes, void* stream);
int svdq_prepare_residual(const void* weight, const void* smooth, const void* proj_down, const void* proj_up,
                          int64_t N, int64_t K, int64_t R, void* qweight, void* wscales, void* wcscales,
                          void* wtscale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * MXFP4 datatype variant (an out-of-tolerance speed point, not the pages'
 * arithmetic). The pages' NVFP4 uses e4m3 scales per 16 K (model card,
 * header); gfx950's block-scaled matrix instruction takes OCP MX instead: E2M1
 * with one power-of-two (E8M0) scale per 32 K. Here both operands are
 * re-rounded into that form. For a 32-block, X = floor(log2 max|v|) - 2 is
 * clamped to [-127, 127] and stored as X + 127; each code is the E2M1
 * nearest-even of v * 2^-X, saturating at 6. The weight is re-rounded from the
 * exact NVFP4 values, the activation from x * smooth. Epilogue, low-rank
 * branch and bias as in svdq_gemm_w4a4.
 *
 * MX operand buffers (rows = tokens or output channels, padded to 32):
 *   codes  svdq_mx_codes_bytes(rows, K): per 64-K step s and 32-row panel p, a
 *          1 KB chunk at 1024 * (s * P + p); byte 16 l + j (l = 32 h + c) holds
 *          row 32 p + c, k = 64 s + 32 h + 2 j (low nibble) and + 1 (high nibble).
 *   scales svdq_mx_scales_bytes(rows, K): [K/32, padded rows] bytes.
 *   Padding rows hold zero codes and scale byte 0.
 * K must be a multiple of 128 (SVDQ_ERR_UNSUPPORTED otherwise).
 * svdq_reround_weight_mxfp4: canonical qweight/wscales -> MX codes/scales (load time).
 * svdq_quantize_act_mxfp4: x [M, K], smooth [K] -> MX codes/scales. The same
 *   codes and scales with lora_act in one pass: svdq_quantize_act with
 *   act_layout SVDQ_ACT_MXFP4.
 * svdq_gemm_mxfp4: MX operands + lora_act [M, R] -> y [M, N] bf16.
 * svdq_linear_mxfp4: the whole variant layer from x (that one-pass quantisation,
 *   then the GEMM), with a workspace of svdq_linear_mxfp4_workspace_bytes(M, K, R)
 *   bytes.
 */
size_t svdq_mx_codes_bytes(int64_t rows, int64_t K);
size_t svdq_mx_scales_bytes(int64_t rows, int64_t K);
int svdq_reround_weight_mxfp4(const void* qweight, const void* wscales, int64_t N, int64_t K, void* mx_codes,
                              void* mx_scales, void* stream);
int svdq_quantize_act_mxfp4(const void* x, const void* smooth, int64_t M, int64_t K, void* mx_codes,
                            void* mx_scales, void* stream);
int svdq_gemm_mxfp4(const void* act_codes, const void* act_scales, const void* lora_act, const void* w_codes,
                    const void* w_scales, const void* wcscales, const void* wtscale, const void* proj_up,
                    const void* bias, int64_t M, int64_t N, int64_t K, int64_t R, void* y, void* stream);
size_t svdq_linear_mxfp4_workspace_bytes(int64_t M, int64_t K, int64_t R);
int svdq_linear_mxfp4(const void* x, const void* smooth, const void* w_codes, const void* w_scales,
                      const void* wcscales, const void* wtscale, const void* proj_down, const void* proj_up,
                      const void* bias, int64_t M, int64_t N, int64_t K, int64_t R, void* y, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Measurement helpers. Not part of the layer and not from the pages: they
 * calibrate the roofline figures reported beside AMD's published MI355X peaks.
 *
 * svdq_calib_mfma: `workgroups` workgroups of 8 waves (two per SIMD, the
 *   GEMM's occupancy), each wave holding the GEMM's 2 x 5 accumulator tiles
 *   and running `iters` iterations of 20 v_mfma_f32_32x32x16_f16 on operand
 *   fragments read once from `table` (svdq_calib_table_bytes() bytes of f16
 *   values the caller chooses: the power the chip draws, and so its clock,
 *   depends on how many operand bits toggle). Work per launch:
 *   iters * svdq_calib_flop_per_iteration(workgroups) flop.
 *   out: >= workgroups * 512 floats (sums that keep the results live);
 *   clocks: >= workgroups * 4 uint64, per workgroup the core-clock counter at
 *   its start and end, then the constant-rate counter at its start and end
 *   (rate in kHz from svdq_calib_wall_clock_khz).
 * svdq_calib_mfma_scaled: the same for the block-scaled instruction the MXFP4
 *   variant runs (v_mfma_scale_f32_32x32x64_f8f6f4), both operands in format
 *   `fmt` (4 = fp4 E2M1, using the first 16 bytes of each lane's operand; 0 =
 *   fp8 e4m3, using 32 bytes) and unit E8M0 scales, operands taken from the same
 *   table's bytes. Work per launch: iters * svdq_calib_scaled_flop_per_iteration(
 *   workgroups) flop. Another fmt returns SVDQ_ERR_UNSUPPORTED.
 * svdq_calib_lds: LDS bandwidth. `workgroups` workgroups of 8 waves each run
 *   `iters` iterations of 8 16-byte LDS accesses per lane on conflict-free slots
 *   of a 64 KB region: mode 0 reads only, 1 writes only, 2 three reads to one
 *   write. Bytes per launch: iters * svdq_calib_lds_bytes_per_iteration(
 *   workgroups). out: >= workgroups * 512 floats (keeps the reads live).
 * svdq_calib_copy: dst = src, `bytes` (a multiple of 16) by a streaming
 *   kernel; src and dst must not overlap. The device-copy rate is the
 *   practical HBM ceiling, and its byte counters calibrate the profiler's.
 * svdq_calib_wall_clock_khz: the constant counter's rate on the current
 *   device (a property query; nothing is enqueued).
 */
size_t svdq_calib_table_bytes(void);
int64_t svdq_calib_flop_per_iteration(int64_t workgroups);
int svdq_calib_mfma(const void* table, size_t table_bytes, int64_t iters, int64_t workgroups, void* out,
                    size_t out_bytes, void* clocks, size_t clocks_bytes, void* stream);
int64_t svdq_calib_scaled_flop_per_iteration(int64_t workgroups);
int svdq_calib_mfma_scaled(const void* table, size_t table_bytes, int64_t iters, int64_t workgroups, int fmt,
                           void* out, size_t out_bytes, void* clocks, size_t clocks_bytes, void* stream);
int64_t svdq_calib_lds_bytes_per_iteration(int64_t workgroups);
int svdq_calib_lds(int64_t iters, int64_t workgroups, int mode, void* out, size_t out_bytes, void* stream);
int svdq_calib_copy(const void* src, void* dst, size_t bytes, void* stream);
int svdq_calib_wall_clock_khz(int* khz);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
