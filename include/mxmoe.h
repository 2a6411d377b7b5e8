/*
 * mxmoe.h — C ABI of the MXFP4 mixture-of-experts layer for AMD MI355X (gfx950).
 *
 * The layer is the GPT-OSS expert block whose weights are stored in OCP
 * MXFP4: e2m1 values packed two per uint8 with one e8m0 power-of-two scale
 * per 32-value block (KerasFormers "mxfp4" page, intro and "Primitives").
 * gate_up_proj is laid out (E, 2I, H) and down_proj (E, H, I), each as
 * uint8 blocks (rows, K/32, 16) plus uint8 scales (rows, K/32), with
 * full-precision biases (same page, "As GPT-OSS's native format").  Rows 2i
 * and 2i+1 of gate_up are gate_i and up_i (interleaved).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned, row-major and densely packed in the shapes stated.  The
 *     library keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; no call synchronises the host.
 *   - All arguments are validated on the host before anything is launched.
 *     On any error the call returns a non-zero status, launches nothing and
 *     leaves every output untouched.  MXMOE_ERR_HIP means a HIP call failed
 *     after validation; the outputs are then undefined.
 *   - The library allocates no device memory: scratch space comes from the
 *     caller's workspace, sized by the matching *_workspace_bytes call
 *     (moe_mxfp4_forward_noalloc uses a fixed device array of the library
 *     instead).
 *   - Calls on distinct streams with distinct outputs and workspaces may run
 *     concurrently; two calls sharing a workspace must be ordered.
 *   - No C++ exception crosses this interface.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXMOE_OK = 0,
  MXMOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MXMOE_ERR_ALIGN = 2,       /* a pointer is not 16-byte aligned */
  MXMOE_ERR_SHAPE = 3,       /* a size is out of range, including a contracting dim % 32 != 0 */
  MXMOE_ERR_DTYPE = 4,       /* unknown dtype code, or a combination not offered */
  MXMOE_ERR_WORKSPACE = 5,   /* workspace smaller than the *_workspace_bytes figure */
  MXMOE_ERR_UNSUPPORTED = 6, /* a valid request outside what this library implements */
  MXMOE_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed */
  MXMOE_ERR_VALUE = 8        /* a non-size argument is out of range (e.g. an FP8 scale <= 0) */
} mxmoe_status_t;

typedef enum {
  MXMOE_F32 = 0,  /* IEEE binary32 */
  MXMOE_BF16 = 1  /* bfloat16 (raw 16-bit patterns) */
} mxmoe_dtype_t;

/* Limits of the layer entry points. */
#define MXMOE_MAX_EXPERTS 256
#define MXMOE_MAX_TOPK 8

/* Human-readable text of a status code (static storage, never NULL). */
const char* mxmoe_status_string(int32_t status);

/* Interface version, bumped on any ABI change (currently 4). */
int32_t mxmoe_version(void);

/*
 * mxfp4_unpack — dequantise MXFP4 to float ("Primitives": each nibble goes
 * through the FP4 codebook {0, 0.5, 1, 1.5, 2, 3, 4, 6} with bit 3 the sign,
 * times 2^(e8m0 - 127)).
 *
 *   blocks : (rows, k/32, 16) uint8.  Element 32*b + 2*j + n of a row is
 *            nibble n of byte j of block b, n = 0 being the low nibble.
 *   scales : (rows, k/32) uint8 e8m0.  Byte 255 decodes to NaN.
 *   out    : (rows, k) in out_dtype (MXMOE_BF16 or MXMOE_F32).
 *
 * The result is exact: every code times a power of two is representable,
 * except that results beyond the format's range become +-Inf and results
 * below it are kept as subnormals; nibble 8 gives -0.0.
 * Errors: k <= 0 or k % 32 != 0, rows < 0 -> MXMOE_ERR_SHAPE (the
 * "As a quantize_model scheme" section: a clear error when the contracting
 * dimension is not a multiple of 32).  rows == 0 is a no-op.
 */
mxmoe_status_t mxfp4_unpack(const uint8_t* blocks, const uint8_t* scales, int64_t rows, int64_t k,
                            void* out, int32_t out_dtype, void* stream);

/*
 * mxfp4_pack — quantise real values to MXFP4 ("Primitives": the e8m0 block
 * scale is floor(log2(amax)) - 2 and each value is rounded to the nearest
 * FP4 grid point).
 *
 *   w      : (rows, k) in w_dtype (MXMOE_BF16 or MXMOE_F32).
 *   blocks : (rows, k/32, 16) uint8 output; scales : (rows, k/32) output.
 *
 * Per 32-value block: e = floor(log2(amax)) - 2 from the exact binary
 * exponent, clamped to [-127, 127] (an all-zero block gets e = -127); the
 * scale byte is e + 127; w / 2^e is rounded to the nearest FP4 magnitude
 * with ties to the even code, saturating at 6, and keeps the sign bit of w
 * (-0.0 and negatives that round to zero give nibble 8).  NaN or Inf inputs
 * give unspecified bytes.  Errors as for mxfp4_unpack.
 */
mxmoe_status_t mxfp4_pack(const void* w, int32_t w_dtype, int64_t rows, int64_t k,
                          uint8_t* blocks, uint8_t* scales, void* stream);

/*
 * Storage orders of the expert weights.
 *
 * MXMOE_LAYOUT_ROWS is the checkpoint order: blocks (mats, rows, k/32, 16)
 * and scales (mats, rows, k/32), as mxfp4_pack writes them.
 *
 * MXMOE_LAYOUT_TILED holds the same bytes regrouped so that the expert
 * GEMMs read every weight tile as one contiguous piece.  For `mats`
 * matrices of (rows, k) values, with RG = ceil(rows / 64) row groups, 4*RG
 * row tiles of 16 rows and NC = ceil(k / 128) chunks of 4 blocks:
 *   tiled blocks: uint8 [mats][4*RG][NC][64][16].  Entry (m, t, c, s, j)
 *     with s = 4*r + (b ^ ((r >> 2) & 3)), r in 0..15, b in 0..3, is byte j
 *     of block 4c+b of row 16t+r of matrix m.
 *   tiled scales: uint8 [mats][RG][NC][64][4].  Entry (m, q, c, l, i) with
 *     l = 16*b + r is the scale of row 64q+16i+r, block 4c+b of matrix m.
 * Positions whose row >= rows or block >= k/32 hold 0 (the value +0 in
 * every block it pads).  Sizes come from mxfp4_tiled_bytes.
 */
typedef enum {
  MXMOE_LAYOUT_ROWS = 0,
  MXMOE_LAYOUT_TILED = 1
} mxmoe_layout_t;

/*
 * mxfp4_tiled_bytes — byte sizes of the MXMOE_LAYOUT_TILED copy of `mats`
 * MXFP4 matrices of (rows, k) values.  Host only; nothing is launched.
 * Errors: mats < 0, rows < 0, k <= 0 or k % 32 != 0 -> MXMOE_ERR_SHAPE;
 * NULL outputs -> MXMOE_ERR_NULL.
 */
mxmoe_status_t mxfp4_tiled_bytes(int64_t mats, int64_t rows, int64_t k, int64_t* blocks_bytes,
                                 int64_t* scales_bytes);

/*
 * mxfp4_tile — copy `mats` MXFP4 matrices of (rows, k) values from the
 * MXMOE_LAYOUT_ROWS order (blocks, scales) into the MXMOE_LAYOUT_TILED
 * order (tiled_blocks, tiled_scales, sized by mxfp4_tiled_bytes), padding
 * included.  A one-time step when weights are loaded; the values are not
 * changed.  The outputs must not overlap the inputs.  Errors as for
 * mxfp4_tiled_bytes, plus NULL / unaligned pointers.  mats or rows == 0 is
 * a no-op.
 */
mxmoe_status_t mxfp4_tile(const uint8_t* blocks, const uint8_t* scales, int64_t mats, int64_t rows, int64_t k,
                          uint8_t* tiled_blocks, uint8_t* tiled_scales, void* stream);

/*
 * mxfp4_linear — a weight-only MXFP4 dense layer, y = x W^T + b, with the
 * (N, K) weight stored as MXFP4 and dequantised in registers as the GEMM
 * consumes it (KerasFormers "mxfp4" page, "As a quantize_model scheme": a
 * Dense kernel kept packed and dequantised on the fly, its contracting
 * dimension a multiple of 32; the bias stays full precision).
 *
 *   x        : (T, K) in act_dtype (MXMOE_BF16 or MXMOE_F32).
 *   w_blocks, w_scales : the weight as one (rows N, k K) MXFP4 matrix in
 *              weight_layout order (MXMOE_LAYOUT_ROWS: (N, K/32, 16) and
 *              (N, K/32); MXMOE_LAYOUT_TILED: the outputs of mxfp4_tile
 *              with mats = 1).
 *   bias     : (N,) in act_dtype, or NULL for none.
 *   out      : (T, N) in act_dtype, accumulated in fp32 and rounded once.
 *   workspace: mxfp4_linear_workspace_bytes(T, N, act_dtype) bytes.
 * Errors: K or N not a positive multiple of 32, T < 0 -> MXMOE_ERR_SHAPE;
 * otherwise as moe_mxfp4_forward.  T == 0 is a no-op.
 */
size_t mxfp4_linear_workspace_bytes(int64_t T, int64_t N, int32_t act_dtype);
mxmoe_status_t mxfp4_linear(const void* x, int64_t T, int64_t K, const uint8_t* w_blocks, const uint8_t* w_scales,
                            int32_t weight_layout, const void* bias, int64_t N, int32_t act_dtype, void* out,
                            void* workspace, size_t ws_bytes, void* stream);

/*
 * Dense FP8 E4M3 layer with static per-tensor scales (W8A8): the attention
 * projections of the gpt-oss-120b-mxfp4-fp8attn-v2 page ("Model Details";
 * "Quantization Recipe", steps 1 and 2: weights and inputs in float8_e4m3fn,
 * symmetric, one static scale per tensor, stored as weight_scale and
 * input_scale next to the FP8 weight).
 *
 * fp8_tiled_bytes — bytes of the tiled FP8 order of an (N, K) weight.
 * fp8_tile — copy w, (N, K) float8_e4m3fn codes in row-major order (device),
 *   into that order (device): row tiles of 16 rows (N padded to a multiple
 *   of 64) x chunks of 128 K (K padded with zero codes), 2 KB per (row tile,
 *   chunk) in row-tile-major order; inside one, the 32 bytes of lane
 *   l = 16g + r are row r's bytes 16g .. 16g+15, then 64+16g .. 64+16g+15, of
 *   the chunk (the K order of an FP8 matrix-instruction operand).
 * fp8_linear — out = (x_q w^T) * (x_scale * w_scale) + bias, where
 *   x_q = sat448(rne(fp32(x) * (1 / x_scale))) as e4m3 (1/x_scale in fp32,
 *   the rule of the MoE FP8 mode) and w holds e4m3 codes of w / w_scale;
 *   fp32 accumulation, bias added in fp32, rounded once to bf16.
 *     x       : (T, K) bf16            out : (T, N) bf16
 *     w_tiled : fp8_tile output         bias: (N,) bf16 or NULL (zero)
 *     workspace: fp8_linear_workspace_bytes(T, K, N) bytes (holds x_q).
 * Errors: N or K not a positive multiple of 32 or above 2^20, or tensors
 * past the 32-bit buffer windows -> MXMOE_ERR_SHAPE; a scale not finite and
 * > 0 (or 1/x_scale, x_scale * w_scale not finite) -> MXMOE_ERR_VALUE; NULL,
 * misaligned, short workspace as for moe_mxfp4_forward.  T == 0 is a no-op.
 */
mxmoe_status_t fp8_tiled_bytes(int64_t N, int64_t K, int64_t* bytes);
mxmoe_status_t fp8_tile(const uint8_t* w, int64_t N, int64_t K, uint8_t* w_tiled, void* stream);
size_t fp8_linear_workspace_bytes(int64_t T, int64_t K, int64_t N);
mxmoe_status_t fp8_linear(const void* x, int64_t T, int64_t K, const uint8_t* w_tiled, float w_scale, float x_scale,
                          const void* bias, int64_t N, void* out, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * INT8 W8A8 mixture-of-experts layer: the gpt-oss-20b-BF16-w8a8-llmcompressor
 * page ("Quantization": weights int8, symmetric, one static scale per output
 * channel; activations int8, symmetric, one dynamic scale per token; the
 * router and every bias kept in bf16).  Same routing, SwiGLU and combine as
 * moe_mxfp4_forward; the experts' weights are int8 codes instead of MXFP4.
 *
 * int8_tiled_bytes / int8_tile — `mats` (rows, k) int8 weights, row-major
 *   codes (device), into the tiled 8-bit order of fp8_tile, matrix after
 *   matrix.  Errors: rows or k not a positive multiple of 32 (or above 2^20)
 *   -> MXMOE_ERR_SHAPE; NULL; misaligned.
 */
typedef struct {
  int32_t E, H, I, top_k;      /* as mxmoe_layer_t */
  const uint8_t* gate_up_w;    /* int8_tile of the (E, 2I, H) codes; rows gate (even) / up (odd) interleaved */
  const float* gate_up_scale;  /* (E, 2I) fp32: weight = code * scale of its row */
  const void* gate_up_bias;    /* (E, 2I) bf16 */
  const uint8_t* down_w;       /* int8_tile of the (E, H, I) codes */
  const float* down_scale;     /* (E, H) fp32 */
  const void* down_bias;       /* (E, H) bf16 */
  const void* router_w;        /* (E, H) bf16 */
  const void* router_b;        /* (E,) bf16 */
} mxmoe_int8_layer_t;

mxmoe_status_t int8_tiled_bytes(int64_t mats, int64_t rows, int64_t k, int64_t* bytes);
mxmoe_status_t int8_tile(const int8_t* w, int64_t mats, int64_t rows, int64_t k, uint8_t* w_tiled, void* stream);

/*
 * moe_int8_forward — x (T, H) bf16 -> out (T, H) bf16.  Routing as
 * moe_mxfp4_forward.  Each token's x and each routed (token, expert) row of
 * h is quantised with its own scale s = amax|row| / 127 (fp32, correctly
 * rounded division), code = clamp(rne(v / s), -127, 127) (all zero for an
 * all-zero row); G = (x_code . W_code) * s_x * s_w + b_gu with exact int32
 * sums, h = clamped SwiGLU of G rounded to bf16, Y = (h_code . W_code) *
 * s_h * s_w + b_d rounded to bf16, out_t = sum_j w_j Y_j (fp32, j order).
 * Inputs must be finite.  Optional topk_idx_out (T, top_k) int32 and
 * topk_w_out (T, top_k) fp32.  Workspace: moe_int8_workspace_bytes.
 * Errors as moe_mxfp4_forward; the 8-bit weights of one expert must fit a
 * 32-bit buffer window.
 */
size_t moe_int8_workspace_bytes(const mxmoe_int8_layer_t* layer, int64_t T);
mxmoe_status_t moe_int8_forward(const mxmoe_int8_layer_t* layer, const void* x, int64_t T, void* out,
                                int32_t* topk_idx_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                                void* stream);

/* One MoE layer's parameters, all device pointers (see the file header). */
typedef struct {
  int32_t E;            /* experts, 1..MXMOE_MAX_EXPERTS */
  int32_t H;            /* hidden size, multiple of 32 */
  int32_t I;            /* intermediate size, multiple of 32 */
  int32_t top_k;        /* experts per token, 1..min(E, MXMOE_MAX_TOPK) */
  int32_t param_dtype;  /* dtype of biases and router: MXMOE_BF16 or MXMOE_F32 */
  int32_t weight_layout; /* mxmoe_layout_t of the four MXFP4 tensors below */
  /* The shapes below are those of MXMOE_LAYOUT_ROWS; with
   * MXMOE_LAYOUT_TILED the same tensors are in the tiled order, with
   * (mats, rows, k) = (E, 2I, H) for gate_up and (E, H, I) for down. */
  const uint8_t* gate_up_blocks; /* (E, 2I, H/32, 16) */
  const uint8_t* gate_up_scales; /* (E, 2I, H/32) */
  const void* gate_up_bias;      /* (E, 2I) param_dtype; added before the SwiGLU */
  const uint8_t* down_blocks;    /* (E, H, I/32, 16) */
  const uint8_t* down_scales;    /* (E, H, I/32) */
  const void* down_bias;         /* (E, H) param_dtype; part of each expert's output */
  const void* router_w;          /* (E, H) param_dtype, never quantised */
  const void* router_b;          /* (E,)   param_dtype */
} mxmoe_layer_t;

/* Per-call options of the forward. */
typedef struct {
  int32_t act_dtype;  /* dtype of x and out: MXMOE_BF16 or MXMOE_F32 */
  int32_t fp8_act;    /* 1: W-MXFP4 A-FP8 mode (needs act_dtype MXMOE_BF16) */
  float x_scale;      /* FP8 mode: static per-tensor scale of x (> 0, finite) */
  float h_scale;      /* FP8 mode: static per-tensor scale of the SwiGLU output */
  int32_t* topk_idx_out; /* optional device (T, top_k) int32: chosen experts */
  float* topk_w_out;     /* optional device (T, top_k) fp32: their weights */
  /* optional: MXMOE_STAGE_EVENTS hipEvent_t handles created by the caller;
   * event i is recorded on `stream` just before stage i (router, grouping,
   * FP8 quantisation of x, gate_up + SwiGLU, down, combine) and the last one
   * after the combine, so stage i takes elapsed(event i, event i+1).  A
   * stage that does not run records its event at the same point as the
   * next.  NULL records nothing, and a NULL entry skips that one event:
   * each record takes a few microseconds of stream time, so a caller timing
   * one stage passes only the two handles around it.  A batch of at most 16
   * tokens runs router and grouping as one launch unless event 1 (between
   * them) is given.  A decode-shaped batch of at most 64 tokens on tiled
   * weights (bf16 or FP8 activations) forms the combine inside the down
   * launch: its combine stage is empty. */
  void* const* stage_events;
  int32_t expert_path;   /* mxmoe_path_t: which experts each token passes through */
} mxmoe_fwd_opts_t;

/* Experts evaluated by the forward. */
typedef enum {
  /* each token through its top_k experts only (grouped by expert) */
  MXMOE_PATH_ROUTED = 0,
  /* every token through every expert, then the same top_k combine: the
   * dense all-experts path of the KerasFormers "mxfp4" page ("As GPT-OSS's
   * native format"), which its long prefills take when cheaper.  The output
   * equals the routed path's up to the fp32 summation order inside the
   * GEMMs (E/top_k times the GEMM work, and a workspace for T*E rows of h
   * and Y). */
  MXMOE_PATH_DENSE = 1
} mxmoe_path_t;

/* Number of handles stage_events points to. */
#define MXMOE_STAGE_EVENTS 7

/*
 * Workspace size in bytes for moe_mxfp4_forward with these arguments
 * (0 if the arguments are invalid).
 */
size_t moe_mxfp4_workspace_bytes(const mxmoe_layer_t* layer, int64_t T, const mxmoe_fwd_opts_t* opts);

/*
 * moe_mxfp4_forward — the routed MoE layer (upstream GptOssExperts forward,
 * gpt-oss-15.5b-23E-nf4-GPU page, "Notes"; only the top-k experts of each
 * token are evaluated, KerasFormers "mxfp4" page, "As GPT-OSS's native
 * format").
 *
 *   x   : (T, H) act_dtype.   out : (T, H) act_dtype.   T >= 0 (0 = no-op).
 *
 * Per token t: logits = W_r x_t + b_r with fp32 accumulation from the
 * unquantised x; the top_k largest logits (ties to the lower expert id),
 * ordered by logit; w = softmax over those top_k logits in fp32.  For each
 * chosen expert e: G = W_gu[e] x + b_gu[e] (fp32 accumulation over decoded
 * MXFP4 weights), gate = min(G[2i], 7), up = clamp(G[2i+1], -7, 7),
 * h_i = (up + 1) * gate * sigmoid(1.702 * gate), rounded to act_dtype (or
 * quantised to FP8 with h_scale), Y = W_d[e] h + b_d[e]; then
 * out_t = sum_j w_j * Y_j summed in the order j = 0..top_k-1.
 *
 * FP8 mode (fp8_act = 1): x and h are quantised to float8_e4m3fn as
 * code = sat448(rne(fp32(v) * (1 / scale))), 1/scale computed once in fp32,
 * and both GEMMs run on scaled MXFP4 x FP8 matrix instructions with fp32
 * accumulation; the router still reads the unquantised x (and writes the
 * e4m3 codes of x as it reads it, so the quantisation stage is empty).
 *
 * With expert_path = MXMOE_PATH_DENSE the two GEMMs run over all T*E
 * (expert, token) pairs, row e*T + t, and the combine reads the top_k rows
 * the router chose; the router and the combine are the routed path's.
 *
 * The result is deterministic: identical inputs give identical bits.
 */
mxmoe_status_t moe_mxfp4_forward(const mxmoe_layer_t* layer, const void* x, int64_t T, void* out,
                                 const mxmoe_fwd_opts_t* opts, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * moe_mxfp4_forward_noalloc — moe_mxfp4_forward without a caller workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, results and errors as moe_mxfp4_forward; the scratch
 * space is a device array of MXMOE_NOALLOC_SCRATCH_BYTES inside the library
 * (one per GPU, held until the process ends; the call itself allocates
 * nothing).  A call whose moe_mxfp4_workspace_bytes figure exceeds it
 * returns MXMOE_ERR_WORKSPACE and launches nothing.  Nothing in that array
 * needs to start at any value: the forward writes every entry it reads.
 * All calls on one GPU share the array, so calls that may overlap on one
 * GPU (other streams, other threads) race and must be ordered by the
 * caller.  The first call on a device looks up that device's copy of the
 * array; the device must be current.
 */
#define MXMOE_NOALLOC_SCRATCH_BYTES (32u << 20)
mxmoe_status_t moe_mxfp4_forward_noalloc(const mxmoe_layer_t* layer, const void* x, int64_t T, void* out,
                                         const mxmoe_fwd_opts_t* opts, void* stream);

/*
 * moe_mxfp4_route — only the routing steps of the forward: router logits,
 * top-k, softmax over the k, and the grouping of the T*top_k (token, slot)
 * pairs by expert.
 *
 *   idx_out     : (T, top_k) int32       w_out      : (T, top_k) fp32
 *   counts_out  : (E,) int32 tokens per expert
 *   offsets_out : (E+1,) int32 exclusive prefix sum of counts
 *   sorted_out  : (T*top_k,) int32 flat slot ids t*top_k + j grouped by
 *                 expert, ascending slot id within an expert
 *   pos_out     : (T*top_k,) int32 row of each flat slot in sorted_out
 * Any of the five outputs may be NULL.  opts->act_dtype gives x's dtype;
 * the FP8 fields and expert_path are ignored (the grouping is the routed
 * one).  Workspace as for moe_mxfp4_forward.
 */
mxmoe_status_t moe_mxfp4_route(const mxmoe_layer_t* layer, const void* x, int64_t T,
                               const mxmoe_fwd_opts_t* opts, int32_t* idx_out, float* w_out,
                               int32_t* counts_out, int32_t* offsets_out, int32_t* sorted_out,
                               int32_t* pos_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_mxfp4_calibrate_fp8 — static per-tensor FP8 scales from a calibration
 * batch (min/max observer, symmetric: the FP8 script comment on the
 * gpt-oss-120b-mxfp4-fp8attn-v2 page; per-tensor activation scheme on the
 * amd/gpt-oss-20b-MoE-Quant-W-MXFP4-A-FP8-KV-FP8 page).
 *
 *   x_calib    : (T, H) bf16 calibration activations, T >= 1.
 *   scales_out : device float[2] = { amax(x)/448, amax(h)/448 } in fp32,
 *                h being the bf16-rounded SwiGLU output of every routed
 *                (token, expert) pair of the batch in the bf16 path.
 * Workspace: moe_mxfp4_workspace_bytes with act_dtype MXMOE_BF16, fp8_act 0.
 */
mxmoe_status_t moe_mxfp4_calibrate_fp8(const mxmoe_layer_t* layer, const void* x_calib, int64_t T,
                                       float* scales_out, void* workspace, size_t workspace_bytes,
                                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXMOE_H */
