// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxmoe {

// Arithmetic of the expert GEMMs: fp32 or bf16 activations on decoded
// weights, or FP8 activations on the scaled MXFP4 x FP8 instructions.
// ACT_W8A8: FP8 activations against FP8 (e4m3) weights in the tiled 8-bit
// order (dense linear only; phase 1 epilogue).  ACT_INT8: int8 activations
// against int8 weights in the same order, int32 accumulation, per-row
// weight scales and per-token activation scales applied in the epilogue.
enum Act : int { ACT_F32 = 0, ACT_BF16 = 1, ACT_FP8 = 2, ACT_W8A8 = 3, ACT_INT8 = 4 };

// Tile shape of the prefill grouped GEMM: weight rows per workgroup (4 row
// groups x 16*RT rows), tokens per workgroup tile, and LDS pipeline stages
// (128-K chunks in flight + 1).  Overridable at build time for tile sweeps.
#ifndef MXMOE_PREFILL_ROWS
#define MXMOE_PREFILL_ROWS 512
#endif
#ifndef MXMOE_PREFILL_TOKENS
#define MXMOE_PREFILL_TOKENS 128
#endif
#ifndef MXMOE_PREFILL_STAGES
#define MXMOE_PREFILL_STAGES 2
#endif
constexpr int kPrefillRows = MXMOE_PREFILL_ROWS;
constexpr int kPrefillTokens = MXMOE_PREFILL_TOKENS;

// Estimated cost of streaming one weight stripe, in units of one 16-token
// sub-tile's MFMA work (splits the tiled kernel's items over the XCDs).
#ifndef MXMOE_TILE_COST
#define MXMOE_TILE_COST 4
#endif
constexpr int kTileCost = MXMOE_TILE_COST;

// Rows per workgroup (64 per wave) of the tiled-order prefill kernel.
#ifndef MXMOE_PREFILL_TILED_ROWS
#define MXMOE_PREFILL_TILED_ROWS 256
#endif
constexpr int kTiledRows = MXMOE_PREFILL_TILED_ROWS;

// Workgroups of a tiled prefill launch over R weight rows with at most
// max_tiles token tiles: 8 G, G per XCD.
__host__ __device__ inline int64_t tiled_prefill_blocks(int R, int max_tiles) {
  return (int64_t(max_tiles) * ((R + kTiledRows - 1) / kTiledRows) + 7) / 8 * 8;
}

hipError_t launch_unpack(const uint8_t* blocks, const uint8_t* scales, int64_t nblocks, void* out, bool out_bf16,
                         hipStream_t stream);
hipError_t launch_pack(const void* w, bool in_bf16, int64_t nblocks, uint8_t* blocks, uint8_t* scales,
                       hipStream_t stream);
// Row order -> tiled order of `mats` (rows, 32*nb) matrices (layout in mxmoe.h).
hipError_t launch_tile(const uint8_t* blocks, const uint8_t* scales, int64_t mats, int rows, int nb,
                       uint8_t* tiled_blocks, uint8_t* tiled_scales, hipStream_t stream);

struct PermuteArgs {
  const int32_t* idx;   // (T*k)
  int n_slots, E;
  int32_t* counts;      // (E)
  int32_t* offsets;     // (E+1)
  int32_t* sorted;      // (T*k)
  int32_t* sorted_tok;  // (T*k): token id (slot / top_k) of each sorted row
  int top_k;
  int32_t* pos;         // (T*k)
  int4* active;         // (E + 1) slot records: active[0].x = number of active experts;
                        // active[1 + i] = {expert, first sorted row, rows, number of active
                        // experts} of the i-th active expert, ids ascending, and {0, 0, 0, 0} for the slots
                        // past them up to min(E, n_slots) (the decode grids' bound)
  int32_t* tile_off;    // (E+1): prefix of ceil(count / kPrefillTokens)
  int4* tiles;          // (tile_off[E]): {expert, first sorted row, tokens, 0} per prefill tile
  int32_t* counts_out;  // optional copies
  int32_t* offsets_out;
  // Optional: the work item of every workgroup of the two tiled prefill
  // launches that follow (gate_up, down), resolved here: blk_rec[g][b] =
  // {expert, first sorted row, tokens, row stripe} for workgroup b, tokens
  // 0 for a workgroup without an item; rec_stripes[g] row stripes and
  // rec_blocks[g] workgroups (tiled_prefill_blocks).
  int4* blk_rec[2];
  int rec_stripes[2];
  int rec_blocks[2];
  // optional: the 8 per-XCD list counters of each of those launches, set
  // here past the first item of each persistent workgroup
  // (GemmArgs::item_head)
  uint32_t* rec_head[2];
};
struct RouteArgs {
  const void* x;        // (T, H) act dtype
  const void* w_r;      // (E, H) same dtype
  const void* b_r;      // (E,)
  int act_bf16;         // 1 = bf16 x and router, 0 = fp32
  int T, H, E, top_k;
  int32_t* idx;         // (T, k) workspace
  float* wts;           // (T, k) workspace
  int32_t* idx_out;     // optional copies
  float* wts_out;
  // FP8 activation mode: (T, H) e4m3 codes of x, quantised with x_inv as
  // the router reads x (bf16 only); null: none
  uint8_t* xq;
  float x_inv;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);
// Router then grouping; one launch when one 16-wave router workgroup covers
// the batch (the grouping then runs in that workgroup after the top-k).
hipError_t launch_route_permute(const RouteArgs& a, const PermuteArgs& p, hipStream_t stream);

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream);

// Grouping of the dense all-experts path: rows e*T + t for every expert e
// and token t (sorted_tok, offsets, counts, active, tiles), and the row of
// each routed slot, pos[t*k + j] = idx[t*k + j] * T + t.
struct DenseGroupArgs {
  const int32_t* idx;   // (T*k) routed experts
  int T, E, top_k;
  int32_t* counts;      // (E)
  int32_t* offsets;     // (E+1)
  int32_t* sorted_tok;  // (T*E)
  int32_t* pos;         // (T*k)
  int4* active;         // (E+1) slot records (as PermuteArgs::active)
  int32_t* tile_off;    // (E+1)
  int4* tiles;          // (E * ceil(T / kPrefillTokens))
};
hipError_t launch_dense_group(const DenseGroupArgs& a, hipStream_t stream);

// FP8 static quantisation of a (rows, cols) bf16 tensor to e4m3 codes.
hipError_t launch_quant_fp8(const uint16_t* x, int64_t n, float inv_scale, uint8_t* q, hipStream_t stream);

// (mats, N, K) 8-bit codes (e4m3 or int8) -> the tiled 8-bit order.
hipError_t launch_byte_tile(const uint8_t* w, int64_t mats, int N, int K, uint8_t* out, hipStream_t stream);

// Symmetric int8 per row (dynamic scale amax / 127) of a (rows, K) bf16 tensor.
hipError_t launch_quant_rows_int8(const uint16_t* x, int64_t rows, int K, int8_t* q, float* scale,
                                  hipStream_t stream);

struct GemmArgs {
  int act;                    // Act: 0 f32, 1 bf16, 2 fp8
  int phase;                  // 0 = gate_up + SwiGLU -> h, 1 = down -> Y
  const uint8_t* wblk;        // (E, R, nb, 16), or the tiled order when `tiled`
  const uint8_t* wsc;         // (E, R, nb), or the tiled order
  int tiled;                  // 1: weights in the tiled order of mxfp4_tile
  const void* bias;           // (E, R)
  int bias_bf16;
  int R, nb, top_k, E;
  const void* bsrc;           // phase 0: x (T, K) act storage; phase 1: h (T*k, K) act storage
  int64_t b_rows;             // rows of bsrc (T or T*k)
  const int32_t* sorted;      // (T*k) flat slot ids in expert order
  const int32_t* sorted_tok;  // (T*k) their token ids
  const int32_t* offsets;     // (E+1)
  const int4* active;         // (E+1) slot records (as PermuteArgs::active)
  const int32_t* tile_off;    // (E+1)
  const int4* tiles;          // prefill tile table
  void* out;                  // phase 0: h (T*k, R/2) act storage; phase 1: Y (T*k, R), fp32 or bf16 (act != fp32)
  float acc_scale;            // fp8: the static scale of the B operand; else 1
  float out_inv_scale;        // phase 0 fp8: 1 / h_scale
  int max_active;             // grid bound: min(E, T*k)
  int max_tiles;              // grid bound of the prefill tile list
  int n_slots;                // T*k
  const float* row_scale;     // ACT_INT8: (E, R) weight scale per output row
  const float* tok_scale;     // ACT_INT8: activation scale per token (phase 0, by token id) or per row (phase 1)
  // Combine folded into the decode-shaped down GEMM (tiled weights, bf16 or
  // FP8 activations, at most kFusedCombineTokens tokens): the last of the
  // active experts' workgroups to finish a 64-row group of Y forms the
  // output rows of that group.  cmb_count: one arrival counter per row
  // group (n_cmb of them), cleared by the gate_up launch (which then needs
  // only cmb_count and n_cmb) and counted by the down launch.
  uint32_t* cmb_count;
  int n_cmb;
  void* cmb_out;              // down: (T, R) bf16 output; null = Y is left for combine_kernel
  const int32_t* pos;         // down: (T*k) sorted row of each routed slot
  const float* wts;           // down: (T, k) routing weights
  int T;                      // tokens of the batch (no expert sees more)
  // tiled prefill launch: each workgroup's item resolved by the grouping
  // (PermuteArgs::blk_rec); null: the workgroup resolves it itself
  const int4* blk_rec;
  // with blk_rec: 8 list counters (PermuteArgs::rec_head) for a persistent
  // launch of kPersistentBlocks workgroups that take the records as work
  // lists; null: one workgroup per record
  uint32_t* item_head;
};
// Workgroups of a persistent tiled prefill launch: two per CU of the
// 256-CU gfx950 parts.
constexpr int kPersistentBlocks = 512;
constexpr int kFusedCombineTokens = 64;
hipError_t launch_moe_gemm(const GemmArgs& a, bool prefill, hipStream_t stream);

// The routing tables of a dense layer seen as one expert with all T tokens
// (offsets, active list, prefill tiles) and, if zero_bias is set, N zero
// bias values of zero_bias_bytes each.
hipError_t launch_linear_setup(int T, int32_t* offsets, int4* active, int32_t* tile_off, int4* tiles,
                               void* zero_bias, int N, int zero_bias_bytes, hipStream_t stream);

struct CombineArgs {
  const void* Y;         // (T*k, H) in sorted order: bf16 (y_bf16) or fp32
  int y_bf16;
  const int32_t* pos;    // (T*k)
  const float* wts;      // (T, k)
  void* out;             // (T, H) act dtype
  int out_bf16;
  int T, H, top_k;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

// amax of bf16 tensors into two uint32 slots, then scales = amax / 448.
hipError_t launch_calib_init(uint32_t* slots, hipStream_t stream);
hipError_t launch_amax_bf16(const uint16_t* v, int64_t n, uint32_t* slot, hipStream_t stream);
hipError_t launch_calib_finish(const uint32_t* slots, float* scales_out, hipStream_t stream);

}  // namespace mxmoe
