/*
 * gbw.h -- 4-bit-weight GEMMs on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Every pointer argument named as a
 * device buffer is a device address owned by the caller (in practice the
 * data_ptr() of a torch tensor); descriptor structs are read during the call
 * only.  Every call is asynchronous on `stream` (a hipStream_t passed as
 * void*, NULL = the default stream); buffers must stay alive until the work
 * on that stream completes.  No call synchronizes the device, and no compute
 * entry point allocates device memory: where scratch is needed the caller
 * passes a workspace sized by gbw_workspace_size().
 *
 * Error behaviour: arguments are validated on the host before anything is
 * launched; a failed check returns a status code and launches nothing.  A
 * launch failure returns GBW_E_LAUNCH.  gbw_last_error() gives a message for
 * the last failure on the calling thread.  Nothing aborts or throws across
 * the ABI.  Shapes with a zero extent (M = 0, T = 0, rows = 0) are no-ops.
 *
 * Formats (MXCode: MX-Native Codebook Quantization, Table 1):
 *   GBW_FMT_E8M0_B32  E2M1 elements + one E8M0 scale per 32 along K (4.25 b/elt)
 *   GBW_FMT_E4M3_B16  E2M1 elements + one E4M3 scale per 16 along K + one
 *                     FP32 tensor scale (4.50 b/elt)
 *   GBW_FMT_E5M3_B16  E2M1 elements + one UE5M3 scale per 16 along K + one
 *                     FP32 tensor scale (4.50 b/elt).  UE5M3: unsigned, 5
 *                     exponent bits (bias 15), 3 mantissa bits; scales from
 *                     2^-17 to 114688 (code 0xFE), code 0xFF reserved.
 *   GBW_FMT_VQ4_E8M0  MXCode PreScale weights: 8-bit index per 4 consecutive K
 *                     elements into a 256-entry table of 4xE2M1 keys per
 *                     QBlock (qblock x qblock, 64 by default), plus the E8M0
 *                     per-32 prescale (abstract, Fig. 2, Fig. 3, Table 4
 *                     caption: d = 4, K = 256).
 *   GBW_FMT_VQ4_POST  MXCode PostScale: the same indices and tables, the
 *                     table of each QBlock quantized to MXFP4 with one E8M0
 *                     scale, which every 32-block of that QBlock's weights
 *                     carries (abstract; layout read from Table 2's BPE).
 *   GBW_FMT_VQ4_PLUS  MXCode PreScale+: the same indices and tables; the
 *                     per-32 E8M0 scales of a row are taken 8 at a time along
 *                     K and each 8-vector is stored as an 8-bit index into a
 *                     256-entry table of 8 E8M0 codes per matrix (abstract;
 *                     Table 4 caption: Ks = 256, ds = 8).
 *   GBW_FMT_VQ4_E4M3[_POST|_PLUS], GBW_FMT_VQ4_E5M3[_POST|_PLUS]: the same
 *                     three VQ layouts with E4M3 (UE5M3) block scales per 16
 *                     along K and FP32 tensor scales, as in E4M3-B16
 *                     (E5M3-B16) (Table 2's E4M3-B16-FP4 columns, Table 4):
 *                     PreScale scales [E][N][K/16], PostScale one per QBlock
 *                     table, PreScale+ indices [E][N][K/128] (8 scales of 16).
 * E2M1 nibbles are packed two per byte, element 2i in bits 3:0, element 2i+1
 * in bits 7:4, bit 3 of a nibble is the sign.  A VQ key holds element i of its
 * 4-vector in bits 4i+3:4i.  All matrices are row-major; weights are [N][K]
 * with K contiguous (the "K x N" weight of a linear layer stored per output
 * column), activations [M][K].
 */
#ifndef GBW_H
#define GBW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define GBW_OK 0
#define GBW_E_ARG 1         /* null pointer, negative extent, bad enum        */
#define GBW_E_SHAPE 2       /* K not a block multiple, tail misaligned, ...   */
#define GBW_E_ALIGN 3       /* device pointer not 16-byte aligned             */
#define GBW_E_UNSUPPORTED 4 /* format/dtype combination or device not gfx950  */
#define GBW_E_WORKSPACE 5   /* workspace missing or smaller than required     */
#define GBW_E_LAUNCH 6      /* a HIP launch failed                            */

/* ---- enums -------------------------------------------------------------- */
#define GBW_FMT_E8M0_B32 0
#define GBW_FMT_E4M3_B16 1
#define GBW_FMT_VQ4_E8M0 2
#define GBW_FMT_E5M3_B16 3
#define GBW_FMT_VQ4_POST 4
#define GBW_FMT_VQ4_PLUS 5
#define GBW_FMT_VQ4_E4M3 6
#define GBW_FMT_VQ4_E4M3_POST 7
#define GBW_FMT_VQ4_E4M3_PLUS 8
#define GBW_FMT_VQ4_E5M3 9
#define GBW_FMT_VQ4_E5M3_POST 10
#define GBW_FMT_VQ4_E5M3_PLUS 11

#define GBW_DTYPE_BF16 0
#define GBW_DTYPE_F32 1

/* flags */
#define GBW_TS_DYNAMIC 1     /* mx_quantize: compute the E4M3/E5M3 tensor scale from the data */
#define GBW_DETERMINISTIC 2  /* GEMMs: fixed summation order, bitwise repeatable          */
#define GBW_FP32_COMBINE 4   /* moe down: keep the per-pair outputs in fp32 (default bf16) */
#define GBW_ROTATE_H32 8     /* mx_quantize, E8M0-B32: rotate every 32-block (block Hadamard) */

/* moe_grouped_gemm stages */
#define GBW_MOE_GATEUP_SWIGLU 0
#define GBW_MOE_DOWN_COMBINE 1

/* gbw_workspace_size ops */
#define GBW_OP_QUANTIZE 0   /* d0 = rows, d1 = K                       */
#define GBW_OP_MX_GEMM 1    /* d0 = M, d1 = N, d2 = K + tail           */
#define GBW_OP_LUT_GEMM 2   /* d0 = M, d1 = N, d2 = K                  */
#define GBW_OP_MOE_ROUTE 3  /* d0 = T, d1 = E                          */
#define GBW_OP_MOE_GEMM 4   /* d0 = pairs, d1 = H, d2 = 1 for GBW_FP32_COMBINE */

/* ---- descriptors -------------------------------------------------------- */

/* A (possibly per-expert) quantized weight, each expert an [N][K] matrix. */
typedef struct gbw_weight {
  int32_t fmt;               /* GBW_FMT_*                                          */
  int32_t n_experts;         /* >= 1; expert e starts at e * (per-expert size)     */
  int64_t N, K;              /* per expert                                         */
  const uint8_t* codes;      /* E8M0/E4M3/E5M3: [E][N][K/2] nibbles; VQ*: [E][N][K/4] idx */
  const uint8_t* scales;     /* E8M0, VQ4_E8M0: [E][N][K/32] E8M0; E4M3/E5M3, VQ4_E4M3,
                                VQ4_E5M3: [E][N][K/16];
                                *_POST: [E][N/qb][K/qb], one per QBlock table;
                                VQ4_PLUS: [E][N][K/256], VQ4_E4M3_PLUS and
                                VQ4_E5M3_PLUS: [E][N][K/128] scale-vector indices  */
  const uint16_t* codebook;  /* VQ*: [E][N/qb][K/qb][256] keys, else NULL           */
  const float* tensor_scale; /* E4M3/E5M3 and their VQ forms: [E][ts_per_expert] fp32 */
  int32_t ts_per_expert;     /* E4M3/E5M3: rows split into this many equal segments,
                                segment s scaled by tensor_scale[e][s] (1 or 2;
                                moe_grouped_gemm: 2 for the gate/up stage -- gate
                                rows, up rows -- and 1 for the down stage)         */
  int32_t qblock;            /* VQ*: QBlock edge qb (64, 128 or 256; 0 means 64)    */
  const uint8_t* scale_codebook; /* *_PLUS: [E][256][8] scale codes, 4-byte
                                aligned: block scales 8i .. 8i+7 of row n of
                                expert e are entry scales[e][n][i]; else NULL  */
} gbw_weight;

/* A quantized activation: [rows][K], K contiguous. */
typedef struct gbw_act {
  int32_t fmt;               /* GBW_FMT_E8M0_B32, GBW_FMT_E4M3_B16 or GBW_FMT_E5M3_B16 */
  int64_t rows, K;
  const uint8_t* codes;      /* [rows][K/2]                                        */
  const uint8_t* scales;     /* [rows][K/32] (E8M0) or [rows][K/16] (E4M3, E5M3)   */
  const float* tensor_scale; /* E4M3/E5M3: device fp32[1]; else NULL               */
} gbw_act;

/* ---- utility ------------------------------------------------------------ */
const char* gbw_status_string(int status);
const char* gbw_last_error(void);
/* Bytes of workspace an op needs for the given extents (0 = none). */
size_t gbw_workspace_size(int32_t op, int64_t d0, int64_t d1, int64_t d2, int32_t fmt);

/* ---- online activation quantization ------------------------------------
 * mx_quantize: x [rows][K] (bf16 or fp32) -> codes [rows][(K+tail_copy)/2],
 * scales [rows][(K+tail_copy)/bs].
 *  E8M0-B32 (MXFP4): per block of 32, scale code = max(0, E(amax) - 2) with
 *    E the fp32 exponent field (OCP MX floor rule), element = RNE onto E2M1,
 *    ties to even, saturating at 6, sign kept.
 *  E4M3-B16: S_T = amax_tensor / 2688 (1 if the tensor is zero); per block
 *    of 16, scale = E4M3_RNE_sat(amax_blk / (6 S_T)), element =
 *    RNE(|x| / (scale * S_T)); each step one fp32 operation.  With
 *    GBW_TS_DYNAMIC, amax_tensor is computed from x and S_T written to
 *    tensor_scale[0] (workspace required); otherwise S_T is read from
 *    tensor_scale[0].
 *  E5M3-B16 (MXCode Table 1, E5M3-B16-FP4 row): the E4M3-B16 steps with
 *    UE5M3 block scales, S_T = amax_tensor / 688128 (= 6 * 114688) and
 *    scale = UE5M3_RNE_sat(amax_blk / (6 S_T)) saturating at 114688.
 *  GBW_ROTATE_H32 (E8M0-B32 only): each 32-element block is first multiplied
 *    by the normalized order-32 Sylvester-Hadamard matrix (H[i][j] =
 *    (-1)^popcount(i&j) / sqrt(32), symmetric and orthonormal) -- the online
 *    Hadamard of CodeQuant Table 2 ("had") applied within the MXFP4 blocks as
 *    PRQuant §2 ("Rotation and block-aware FP4 quantization") describes.
 *    Weights quantized with the same flag give X W^T = (X H)(W H)^T.  Computed
 *    in fp32 by the fast transform (stages of span 1, 2, 4, 8, 16, each
 *    (a, b) -> (a + b, a - b)), then one multiply by fp32(1/sqrt(32)).
 *  tail_copy > 0 (E8M0 only, multiple of 32, <= K) appends a copy of the
 *    quantized last tail_copy columns with their scales: PRQuant:
 *    Permutation Residual Quantization for Low-Overhead Inference, §4
 *    "Kernel design for efficient inference" (online copy).
 * Errors: GBW_E_SHAPE if K is not a multiple of the block size.
 */
int mx_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t K, int32_t fmt,
                int64_t tail_copy, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                int32_t flags, void* ws, size_t ws_bytes, void* stream);

/* mx_dequantize: decode expert `expert` of w to fp32 out [N][K] through the
 * same device decoders the GEMMs use (E8M0: e2m1*2^(s-127); E4M3 and E5M3:
 * e2m1*scale*tensor_scale[segment]; VQ*: QBlock table key nibble * 2^(s-127)
 * with s the stored, per-QBlock or table-decoded E8M0 scale).
 * Used to check decoded weights bit for bit and for offline preparation. */
int mx_dequantize(const gbw_weight* w, int32_t expert, float* out, void* stream);

/* mx_residual: PRQuant §4 Eq. (2) offline weight residual,
 * r[n][j] = w[n][K-tail+j] - deq(codes, scales)[n][K-tail+j] (fp32 RNE),
 * for w [N][K] fp32 and its E8M0-B32 quantization; r is [N][tail]. */
int mx_residual(const float* w, int64_t N, int64_t K, int64_t tail, const uint8_t* codes,
                const uint8_t* scales, float* r, void* stream);

/* ---- dense GEMMs ---------------------------------------------------------
 * mx_gemm: y[M][N] fp32 = deq(a) deq(w)^T, a [M][K] and w [N][K] both
 * E8M0-B32 (scaled MFMA, FP4 x FP4): the W4A4 linear layer Y = X W of
 * PRQuant: Permutation Residual Quantization for Low-Overhead Inference,
 * §4 Eq. (1) (with the permutation and scaling already folded into the
 * operands), on the E8M0-B32-FP4 format of MXCode: MX-Native Codebook
 * Quantization, Table 1; deq() decodes each element as e2m1 * 2^(scale-127).
 * K must be a multiple of 32.  y is overwritten.  When the grid needs the
 * reduction over K split across workgroups, the split partials go to the
 * workspace (gbw_workspace_size(GBW_OP_MX_GEMM, M, N, K [+ tail], 0) bytes)
 * and are summed in split order: with 17 or more rows and K segments that
 * are multiples of 128, inside the same kernel (the last workgroup of an
 * output tile to arrive adds the tile's partials; the arrival counters are
 * the workspace's first 64 KiB, which must be zero before the first call and
 * are left zero by every call, so calls that share a workspace must not
 * overlap in time), otherwise by a second kernel.  With a smaller or NULL
 * workspace a slower serial-K kernel is used.  Results are bitwise
 * repeatable.
 */
int mx_gemm(int64_t M, const gbw_act* a, const gbw_weight* w, float* y, int32_t flags,
            void* ws, size_t ws_bytes, void* stream);

/* residual_tail_gemm: the augmented MXFP4 GEMM of PRQuant §4 ("Offline
 * residual augmentation", W_aug^q = Q([W, R_W]), and "Kernel design"):
 *   y = deq(a) deq(w)^T + deq(a[:, K-tail:]) deq(r)^T
 * a [M][K] E8M0-B32 (the tail is re-read in place, no copy), w [N][K],
 * r [N][tail] the quantized residual.  tail % 32 == 0, tail <= K. */
int residual_tail_gemm(int64_t M, const gbw_act* a, const gbw_weight* w, const gbw_weight* r,
                       int64_t tail, float* y, int32_t flags, void* ws, size_t ws_bytes,
                       void* stream);

/* lut_gemm: codebook weights (CodeQuant: Unified Clustering and Quantization
 * for Enhanced Outlier Smoothing in Low-Precision Mixture-of-Experts,
 * Fig. 1 stage 3-4, Fig. 4):
 *   y[m][n] = sum_k bf16(x[m][k]) * fp16(centroids[n][k/group][idx[n][k]])
 * x [M][K] bf16 bits, idx [N][K/2] 4-bit indices, centroids [N][K/group][16]
 * fp16 bits, y [M][N] fp32 (overwritten).  group in {32, 64, 128},
 * K % 128 == 0.  Any finite bf16 x: each 128-element chunk of an x row is
 * scaled by a power of two into fp16's range for the fp16 matrix cores and
 * the chunk's partial sum is scaled back (both exact).
 * ws: gbw_workspace_size(GBW_OP_LUT_GEMM, M, N, K, 0) bytes (0 for M <= 16),
 * 16-byte aligned.  For M > 16 the reduction over K is split across
 * workgroups: each writes a partial tile into ws and the last of a tile's
 * workgroups to arrive (a counter per output tile at the start of ws) sums
 * them in a fixed order, so results are bitwise repeatable.  Those counters
 * must be zero before the first call with a workspace and every completed
 * call leaves them zero: zero the workspace once, then reuse it.  Calls that
 * share a workspace must not overlap in time.  With a smaller or NULL
 * workspace one workgroup covers all of K per tile (slower, no workspace). */
int lut_gemm(int64_t M, int64_t N, int64_t K, int32_t group, const uint16_t* x_bf16,
             const uint8_t* idx, const uint16_t* centroids_f16, float* y, int32_t flags,
             void* ws, size_t ws_bytes, void* stream);

/* ---- MoE ------------------------------------------------------------------
 * moe_route: the router of the mixture-of-experts FFNs whose experts the
 * pages quantize (CodeQuant Fig. 1-2: clustered weights in the MoE experts;
 * PRQuant §4 applies to the routed experts' down projections).  The pages do
 * not spell the router out; this is the top-k softmax routing their MoE
 * models use, read as: logits [T][E] fp32 -> top-k experts per token
 * (largest logit first, ties to the lower expert id; -0 ties +0, NaN ranks
 * after every number), weights exp(l_j - l_max) normalised over the k chosen
 * (a reading: the softmax is taken over the chosen k), and the pair list
 * sorted by (expert, token):
 *   topk_ids [T][k] i32, topk_w [T][k] f32, expert_offsets [E+1] i32,
 *   pair_token [T*k] i32, pair_pos [T][k] i32 (index of the pair in the list).
 * E <= 1024, 1 <= k <= min(E, 16).  ws: gbw_workspace_size(GBW_OP_MOE_ROUTE, T, E, 0, 0). */
int moe_route(const float* logits, int64_t T, int32_t E, int32_t topk, int32_t* topk_ids,
              float* topk_w, int32_t* expert_offsets, int32_t* pair_token, int32_t* pair_pos,
              void* ws, size_t ws_bytes, void* stream);

/* moe_route_noalloc: moe_route for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, outputs and results (bit for bit) as
 * moe_route, without the workspace: the per-chunk counts and bases go to a
 * fixed 1 MiB array the library holds on each GPU it runs on until the
 * process ends.  Limit: ceil(T / 64) * E <= 131072 (e.g. 65536 tokens with
 * 128 experts); larger problems fail with GBW_E_SHAPE before anything is
 * launched.  The call allocates nothing.  Every call on one GPU shares that
 * array, and each call writes all of it that it reads: calls that overlap
 * in time on one GPU (different streams, no ordering between them) race and
 * may return wrong pair lists; calls ordered on one stream are safe. */
int moe_route_noalloc(const float* logits, int64_t T, int32_t E, int32_t topk, int32_t* topk_ids,
                      float* topk_w, int32_t* expert_offsets, int32_t* pair_token, int32_t* pair_pos,
                      void* stream);

/* moe_grouped_gemm: one stage of the routed expert FFN (gated MLP of PRQuant
 * §4 Eq. (1), applied per expert as in CodeQuant Fig. 1-2):
 *  GBW_MOE_GATEUP_SWIGLU: for each pair p=(t,e): g,u = deq(a[t]) deq(w_e)^T
 *    with w_e the fused [2I][H] gate/up weight (gate rows first);
 *    h = bf16(silu(g) * u).  Writes h_bf16 [P][I] if non-NULL and, for
 *    E8M0-B32 activations, the quantized h into h_codes [P][I/2] / h_scales
 *    [P][I/32] (the requantization is fused).  For E4M3-B16 and E5M3-B16
 *    only h_bf16 is written; quantize it with mx_quantize(GBW_TS_DYNAMIC).
 *  GBW_MOE_DOWN_COMBINE: y[t] = sum_j topk_w[t][j] * deq(a[pair_pos[t][j]])
 *    deq(w_e)^T, a = quantized h in pair order, y [T][H] fp32 (overwritten).
 *    With a workspace, every pair's output goes once to row p of a [P][H]
 *    slot buffer (bf16, or fp32 with GBW_FP32_COMBINE) and a second kernel
 *    sums a token's rows pair_pos[t][0..topk-1] in slot order: bitwise
 *    repeatable.  With ws = NULL the
 *    outputs are added into y with fp32 atomics (no workspace, not
 *    repeatable; GBW_DETERMINISTIC then fails with GBW_E_WORKSPACE).
 * Weights: E8M0-B32, VQ4-E8M0 / VQ4_POST / VQ4_PLUS (decoded to MXFP4 in
 * LDS, scaled MFMA; N and K multiples of the QBlock edge; VQ4_POST and
 * VQ4_PLUS need K <= 8192, VQ4_PLUS also K % 256 == 0), the VQ4_E4M3* and
 * VQ4_E5M3* forms (expanded and decoded like E4M3-B16 / E5M3-B16; *_PLUS
 * needs K % 128 == 0),
 * E4M3-B16 (decoded exactly to fp16, fp16 MFMA) or E5M3-B16 (decoded exactly
 * to bf16 -- the products reach 6 * 114688, past fp16's range -- bf16 MFMA).
 * The activation format is E4M3-B16 for E4M3-B16 and VQ4_E4M3* weights,
 * E5M3-B16 for E5M3-B16 and VQ4_E5M3* weights, E8M0-B32 otherwise.
 * ws: gbw_workspace_size(GBW_OP_MOE_GEMM, P, H, fp32_combine, 0) bytes
 * (down stage only; the gate/up stage takes none). */
typedef struct gbw_moe_out {
  uint16_t* h_bf16;   /* GATEUP: [P][I] bf16 bits or NULL            */
  uint8_t* h_codes;   /* GATEUP, E8M0: [P][(I+h_tail)/2] or NULL      */
  uint8_t* h_scales;  /* GATEUP, E8M0: [P][(I+h_tail)/32] or NULL     */
  float* y;           /* DOWN: [T][H]                                 */
  int64_t h_tail;     /* GATEUP, E8M0: append a copy of the quantized
                         last h_tail columns of h with their scales
                         (PRQuant §4 online tail copy; multiple of 32,
                         <= I; 0 = none).  A down stage over I + h_tail
                         with weights [W_down | R] (R the quantized
                         residual of the last h_tail columns, PRQuant §4
                         Eq. (2)) is then PRQuant's augmented GEMM.      */
} gbw_moe_out;

int moe_grouped_gemm(int32_t stage, int64_t T, int32_t topk, const int32_t* expert_offsets,
                     const int32_t* pair_token, const int32_t* pair_pos, const float* topk_w,
                     const gbw_act* a, const gbw_weight* w, const gbw_moe_out* out,
                     int32_t flags, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GBW_H */
