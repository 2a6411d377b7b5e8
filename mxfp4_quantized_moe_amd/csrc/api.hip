// C ABI of the MXFP4 MoE layer: host-side validation, workspace layout and
// dispatch onto the gfx950 kernels.  Nothing here allocates device memory
// or synchronises the host; every check runs before the first launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/mxmoe.h"
#include "launch.h"

namespace {

using namespace mxmoe;

constexpr int64_t kMaxSlots = int64_t(1) << 26;  // T * top_k limit (grid sizes stay in range)
constexpr int64_t kMaxDim = int64_t(1) << 20;    // H, I, pack/unpack k
// One thread per element of the codec kernels' 1-D grids of 256-thread
// workgroups: the grid's work-item count must stay below 2^32.
constexpr int64_t kMaxGridItems = (int64_t(1) << 32) - 256;

// Bytes of the tiled copy of `mats` (rows, k) matrices (layout in mxmoe.h).
void tiled_sizes(int64_t mats, int64_t rows, int64_t k, int64_t* bb, int64_t* sb) {
  const int64_t rg = (rows + 63) / 64, nc = (k / 32 + 3) / 4;
  *bb = mats * 4 * rg * nc * 1024;
  *sb = mats * rg * nc * 256;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

struct Workspace {
  size_t idx, wts, counts, offsets, active, tile_off, tiles, rec0, rec1, heads, sorted, sorted_tok, pos, cmb, calib, xq,
      h, y,
      total;
};

// Rows of the two GEMMs: the T*k routed (token, expert) pairs, or all T*E
// of them on the dense path.
int64_t gemm_rows(const mxmoe_layer_t* L, int64_t T, bool dense) { return T * (dense ? L->E : L->top_k); }

// Byte offsets of the forward's scratch buffers inside the caller's workspace
// (`rows` = GEMM rows, T*k routed or T*E dense).
Workspace layout(int E, int H, int I, int k, int64_t T, int act_dtype, bool fp8, int64_t rows) {
  Workspace w{};
  const size_t slots = size_t(T) * size_t(k);
  const size_t grows = size_t(rows);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  w.idx = take(slots * 4);
  w.wts = take(slots * 4);
  w.counts = take(size_t(E) * 4);
  w.offsets = take(size_t(E + 1) * 4);
  w.active = take(size_t(E + 1) * 16);
  w.tile_off = take(size_t(E + 1) * 4);
  const size_t active_max = grows < size_t(E) ? grows : size_t(E);
  const int max_tiles = int((grows + kPrefillTokens - 1) / kPrefillTokens + active_max);
  w.tiles = take(size_t(max_tiles) * 16);
  // per-workgroup item records of the tiled prefill gate_up (2I rows) and
  // down (H rows) launches
  w.rec0 = take(size_t(tiled_prefill_blocks(2 * I, max_tiles)) * 16);
  w.rec1 = take(size_t(tiled_prefill_blocks(H, max_tiles)) * 16);
  w.heads = take(2 * 8 * 4);  // their per-XCD list counters (persistent launches)
  w.sorted = take(slots * 4);
  w.sorted_tok = take(grows * 4);
  w.pos = take(slots * 4);
  w.cmb = take(size_t((H + 63) / 64) * 4);  // arrival counters of the folded combine
  w.calib = take(16);
  w.xq = take(fp8 ? size_t(T) * size_t(H) : 0);
  const size_t hb = fp8 ? 1 : (act_dtype == MXMOE_BF16 ? 2 : 4);
  w.h = take(grows * size_t(I) * hb);
  w.y = take(grows * size_t(H) * (act_dtype == MXMOE_BF16 ? 2 : 4));  // Y: bf16 with bf16 activations
  w.total = o;
  return w;
}

mxmoe_status_t check_layer(const mxmoe_layer_t* L) {
  if (!L) return MXMOE_ERR_NULL;
  if (L->E < 1 || L->E > MXMOE_MAX_EXPERTS) return MXMOE_ERR_SHAPE;
  if (L->H <= 0 || L->I <= 0 || L->H > kMaxDim || L->I > kMaxDim) return MXMOE_ERR_SHAPE;
  if (L->H % 32 != 0 || L->I % 32 != 0) return MXMOE_ERR_SHAPE;
  if (L->top_k < 1 || L->top_k > MXMOE_MAX_TOPK || L->top_k > L->E) return MXMOE_ERR_SHAPE;
  if (L->param_dtype != MXMOE_F32 && L->param_dtype != MXMOE_BF16) return MXMOE_ERR_DTYPE;
  if (L->weight_layout != MXMOE_LAYOUT_ROWS && L->weight_layout != MXMOE_LAYOUT_TILED) return MXMOE_ERR_VALUE;
  const void* ptrs[] = {L->gate_up_blocks, L->gate_up_scales, L->gate_up_bias, L->down_blocks,
                        L->down_scales,    L->down_bias,      L->router_w,     L->router_b};
  for (const void* p : ptrs)
    if (!p) return MXMOE_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MXMOE_ERR_ALIGN;
  return MXMOE_OK;
}

// `forward`: the options of a forward call, whose FP8 fields and expert path
// are checked too (the routing-only call ignores them).
mxmoe_status_t check_opts(const mxmoe_layer_t* L, const mxmoe_fwd_opts_t* o, bool forward) {
  if (!o) return MXMOE_ERR_NULL;
  if (o->act_dtype != MXMOE_F32 && o->act_dtype != MXMOE_BF16) return MXMOE_ERR_DTYPE;
  if (o->act_dtype != L->param_dtype) return MXMOE_ERR_DTYPE;  // one dtype for x, router and biases
  if (forward) {
    if (o->fp8_act != 0 && o->fp8_act != 1) return MXMOE_ERR_VALUE;
    if (o->fp8_act) {
      if (o->act_dtype != MXMOE_BF16) return MXMOE_ERR_DTYPE;
      if (!(std::isfinite(o->x_scale) && o->x_scale > 0.f)) return MXMOE_ERR_VALUE;
      if (!(std::isfinite(o->h_scale) && o->h_scale > 0.f)) return MXMOE_ERR_VALUE;
      if (!std::isfinite(1.0f / o->x_scale) || !std::isfinite(1.0f / o->h_scale)) return MXMOE_ERR_VALUE;
    }
  }
  if (forward && o->expert_path != MXMOE_PATH_ROUTED && o->expert_path != MXMOE_PATH_DENSE) return MXMOE_ERR_VALUE;
  if (o->topk_idx_out && !aligned16(o->topk_idx_out)) return MXMOE_ERR_ALIGN;
  if (o->topk_w_out && !aligned16(o->topk_w_out)) return MXMOE_ERR_ALIGN;
  return MXMOE_OK;
}

// The kernels address each expert's weights, x, and each tile's rows of the
// intermediate h through 32-bit range-checked buffer windows below 2^31
// bytes (h as a whole may be larger: a dense layer's T*E rows).
constexpr int64_t kMaxWindow = (int64_t(1) << 31) - 1;

mxmoe_status_t check_tokens(const mxmoe_layer_t* L, int64_t T, bool dense = false) {
  if (T < 0) return MXMOE_ERR_SHAPE;
  if (T * int64_t(dense ? L->E : L->top_k) > kMaxSlots) return MXMOE_ERR_SHAPE;
  // x; and an expert's rows of h (at most T: a token meets an expert once)
  if (T * int64_t(L->H) * 4 > kMaxWindow || T * int64_t(L->I) * 4 > kMaxWindow) return MXMOE_ERR_SHAPE;
  if (int64_t(2) * L->I * L->H / 2 > kMaxWindow) return MXMOE_ERR_SHAPE;
  int64_t bb, sb;  // one expert's tiled gate_up (the larger of the two matrices)
  tiled_sizes(1, int64_t(2) * L->I, L->H, &bb, &sb);
  if (bb > kMaxWindow) return MXMOE_ERR_SHAPE;
  tiled_sizes(1, L->H, L->I, &bb, &sb);
  if (bb > kMaxWindow) return MXMOE_ERR_SHAPE;
  return MXMOE_OK;
}

mxmoe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MXMOE_OK : MXMOE_ERR_HIP; }

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(base) + off);
}

// Router + grouping into the workspace; optional copies for the caller.
hipError_t run_routing(const mxmoe_layer_t* L, const void* x, int64_t T, int act_dtype, const Workspace& w,
                       void* ws, int32_t* idx_out, float* w_out, int32_t* counts_out, int32_t* offsets_out,
                       int32_t* sorted_buf, int32_t* pos_buf, hipStream_t s, hipEvent_t mid = nullptr,
                       bool dense = false, uint8_t* xq = nullptr, float x_inv = 1.0f, bool item_records = false) {
  RouteArgs ra{};
  ra.x = x;
  ra.w_r = L->router_w;
  ra.b_r = L->router_b;
  ra.act_bf16 = act_dtype == MXMOE_BF16;
  ra.T = int(T);
  ra.H = L->H;
  ra.E = L->E;
  ra.top_k = L->top_k;
  ra.idx = at<int32_t>(ws, w.idx);
  ra.wts = at<float>(ws, w.wts);
  ra.idx_out = idx_out;
  ra.wts_out = w_out;
  ra.xq = xq;
  ra.x_inv = x_inv;
  if (dense) {
    hipError_t e = launch_route(ra, s);
    if (e != hipSuccess) return e;
    if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
    DenseGroupArgs da{};
    da.idx = ra.idx;
    da.T = int(T);
    da.E = L->E;
    da.top_k = L->top_k;
    da.counts = at<int32_t>(ws, w.counts);
    da.offsets = at<int32_t>(ws, w.offsets);
    da.sorted_tok = at<int32_t>(ws, w.sorted_tok);
    da.pos = at<int32_t>(ws, w.pos);
    da.active = at<int4>(ws, w.active);
    da.tile_off = at<int32_t>(ws, w.tile_off);
    da.tiles = at<int4>(ws, w.tiles);
    return launch_dense_group(da, s);
  }
  PermuteArgs pa{};
  pa.idx = ra.idx;
  pa.n_slots = int(T * L->top_k);
  pa.E = L->E;
  pa.counts = at<int32_t>(ws, w.counts);
  pa.offsets = at<int32_t>(ws, w.offsets);
  pa.sorted = sorted_buf ? sorted_buf : at<int32_t>(ws, w.sorted);
  pa.pos = pos_buf ? pos_buf : at<int32_t>(ws, w.pos);
  pa.sorted_tok = at<int32_t>(ws, w.sorted_tok);
  pa.top_k = L->top_k;
  pa.active = at<int4>(ws, w.active);
  pa.tile_off = at<int32_t>(ws, w.tile_off);
  pa.tiles = at<int4>(ws, w.tiles);
  pa.counts_out = counts_out;
  pa.offsets_out = offsets_out;
  if (item_records) {  // a tiled prefill forward follows: resolve its workgroups' items here
    const int64_t rows = T * L->top_k;
    const int max_tiles = int((rows + kPrefillTokens - 1) / kPrefillTokens + (rows < L->E ? rows : L->E));
    pa.blk_rec[0] = at<int4>(ws, w.rec0);
    pa.blk_rec[1] = at<int4>(ws, w.rec1);
    pa.rec_head[0] = at<uint32_t>(ws, w.heads);
    pa.rec_head[1] = at<uint32_t>(ws, w.heads) + 8;
    pa.rec_stripes[0] = (2 * L->I + kTiledRows - 1) / kTiledRows;
    pa.rec_stripes[1] = (L->H + kTiledRows - 1) / kTiledRows;
    pa.rec_blocks[0] = int(tiled_prefill_blocks(2 * L->I, max_tiles));
    pa.rec_blocks[1] = int(tiled_prefill_blocks(L->H, max_tiles));
  }
  if (mid) {  // the stage boundary is recorded: two launches
    hipError_t e = launch_route(ra, s);
    if (e != hipSuccess) return e;
    if ((e = hipEventRecord(mid, s)) != hipSuccess) return e;
    return launch_permute(pa, s);
  }
  return launch_route_permute(ra, pa, s);
}

GemmArgs gemm_args(const mxmoe_layer_t* L, const Workspace& w, void* ws, int64_t T, int act, int phase,
                   bool dense = false) {
  GemmArgs g{};
  g.act = act;
  g.phase = phase;
  g.bias_bf16 = L->param_dtype == MXMOE_BF16;
  g.top_k = L->top_k;
  g.E = L->E;
  g.sorted = at<int32_t>(ws, w.sorted);
  g.sorted_tok = at<int32_t>(ws, w.sorted_tok);
  g.offsets = at<int32_t>(ws, w.offsets);
  g.active = at<int4>(ws, w.active);
  g.tile_off = at<int32_t>(ws, w.tile_off);
  g.tiles = at<int4>(ws, w.tiles);
  const int64_t slots = gemm_rows(L, T, dense);
  g.n_slots = int(slots);
  g.max_active = int(slots < L->E ? slots : L->E);
  g.max_tiles = int((slots + kPrefillTokens - 1) / kPrefillTokens + g.max_active);
  g.acc_scale = 1.0f;
  g.out_inv_scale = 1.0f;
  g.T = int(T);
  g.tiled = L->weight_layout == MXMOE_LAYOUT_TILED;
  if (phase == 0) {
    g.wblk = L->gate_up_blocks;
    g.wsc = L->gate_up_scales;
    g.bias = L->gate_up_bias;
    g.R = 2 * L->I;
    g.nb = L->H / 32;
    g.b_rows = T;
    g.out = at<void>(ws, w.h);
  } else {
    g.wblk = L->down_blocks;
    g.wsc = L->down_scales;
    g.bias = L->down_bias;
    g.R = L->H;
    g.nb = L->I / 32;
    g.b_rows = slots;
    g.bsrc = at<void>(ws, w.h);
    g.out = at<void>(ws, w.y);
  }
  return g;
}

// Decode-shaped kernels while experts see few tokens on average; the
// LDS-staged MFMA tiles beyond that.
bool use_prefill(const mxmoe_layer_t* L, int64_t T, int act, bool dense = false) {
  if (act == ACT_F32) return false;
  const int64_t slots = gemm_rows(L, T, dense);
  const int64_t active = slots < L->E ? slots : L->E;
  return slots > 16 * active;
}

// The whole forward of moe_mxfp4_forward on a given scratch buffer.
mxmoe_status_t forward_impl(const mxmoe_layer_t* L, const void* x, int64_t T, void* out, const mxmoe_fwd_opts_t* o,
                            void* ws, size_t ws_bytes, void* stream) {
  mxmoe_status_t st = check_layer(L);
  if (st != MXMOE_OK) return st;
  if ((st = check_opts(L, o, true)) != MXMOE_OK) return st;
  const bool dense = o->expert_path == MXMOE_PATH_DENSE;
  if ((st = check_tokens(L, T, dense)) != MXMOE_OK) return st;
  if (T == 0) return MXMOE_OK;
  if (!x || !out || !ws) return MXMOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(out) || !aligned16(ws)) return MXMOE_ERR_ALIGN;
  const bool fp8 = o->fp8_act == 1;
  const Workspace w = layout(L->E, L->H, L->I, L->top_k, T, o->act_dtype, fp8, gemm_rows(L, T, dense));
  if (ws_bytes < w.total) return MXMOE_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  void* const* ev = o->stage_events;
  auto mark = [&](int i) { return ev && ev[i] ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) : hipSuccess; };
  if (mark(0) != hipSuccess) return MXMOE_ERR_HIP;
  const int act = fp8 ? ACT_FP8 : (o->act_dtype == MXMOE_BF16 ? ACT_BF16 : ACT_F32);
  const bool prefill = use_prefill(L, T, act, dense);
  const bool tiled = L->weight_layout == MXMOE_LAYOUT_TILED;
  // a routed prefill on tiled weights: the grouping resolves every GEMM
  // workgroup's item
  const bool records = prefill && tiled && !dense;
  const float inv_x = fp8 ? 1.0f / o->x_scale : 1.0f;
  const float inv_h = fp8 ? 1.0f / o->h_scale : 1.0f;
  // FP8 mode: the router quantises x to e4m3 as it reads it
  hipError_t e = run_routing(L, x, T, o->act_dtype, w, ws, o->topk_idx_out, o->topk_w_out, nullptr, nullptr, nullptr,
                             nullptr, s, ev ? static_cast<hipEvent_t>(ev[1]) : nullptr, dense,
                             fp8 ? at<uint8_t>(ws, w.xq) : nullptr, inv_x, records);
  if (e != hipSuccess) return MXMOE_ERR_HIP;
  if (mark(2) != hipSuccess) return MXMOE_ERR_HIP;
  if (mark(3) != hipSuccess) return MXMOE_ERR_HIP;
  // decode-shaped batches on the tiled decode kernels fold the combine
  // into the down GEMM (Y read back through a 32-bit buffer window)
  const bool fold = !prefill && tiled && act != ACT_F32 && T <= kFusedCombineTokens &&
                    gemm_rows(L, T, dense) * L->H * 2 <= kMaxWindow;
  GemmArgs g0 = gemm_args(L, w, ws, T, act, 0, dense);
  g0.bsrc = fp8 ? at<void>(ws, w.xq) : x;
  if (fp8) {
    g0.acc_scale = o->x_scale;
    g0.out_inv_scale = inv_h;
  }
  GemmArgs g1 = gemm_args(L, w, ws, T, act, 1, dense);
  if (fp8) g1.acc_scale = o->h_scale;
  if (records) {
    g0.blk_rec = at<int4>(ws, w.rec0);
    g1.blk_rec = at<int4>(ws, w.rec1);
    g0.item_head = at<uint32_t>(ws, w.heads);
    g1.item_head = at<uint32_t>(ws, w.heads) + 8;
  }
  if (fold) {
    g0.cmb_count = g1.cmb_count = at<uint32_t>(ws, w.cmb);
    g0.n_cmb = g1.n_cmb = (L->H + 63) / 64;
    g1.cmb_out = out;
    g1.pos = at<int32_t>(ws, w.pos);
    g1.wts = at<float>(ws, w.wts);
  }
  if ((e = launch_moe_gemm(g0, prefill, s)) != hipSuccess) return MXMOE_ERR_HIP;
  if (mark(4) != hipSuccess) return MXMOE_ERR_HIP;
  if ((e = launch_moe_gemm(g1, prefill, s)) != hipSuccess) return MXMOE_ERR_HIP;
  if (mark(5) != hipSuccess) return MXMOE_ERR_HIP;
  if (fold) return hip_status(mark(6));
  CombineArgs ca{};
  ca.Y = at<void>(ws, w.y);
  ca.y_bf16 = act != ACT_F32;
  ca.pos = at<int32_t>(ws, w.pos);
  ca.wts = at<float>(ws, w.wts);
  ca.out = out;
  ca.out_bf16 = o->act_dtype == MXMOE_BF16;
  ca.T = int(T);
  ca.H = L->H;
  ca.top_k = L->top_k;
  if ((e = launch_combine(ca, s)) != hipSuccess) return MXMOE_ERR_HIP;
  return hip_status(mark(6));
}

}  // namespace

extern "C" {

const char* mxmoe_status_string(int32_t s) {
  switch (s) {
    case MXMOE_OK: return "ok";
    case MXMOE_ERR_NULL: return "a required pointer is NULL";
    case MXMOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MXMOE_ERR_SHAPE: return "a size is out of range (the contracting dimension must be a multiple of 32)";
    case MXMOE_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case MXMOE_ERR_WORKSPACE: return "workspace too small";
    case MXMOE_ERR_UNSUPPORTED: return "request not supported by this library";
    case MXMOE_ERR_HIP: return "HIP runtime error";
    case MXMOE_ERR_VALUE: return "an argument value is out of range";
    default: return "unknown status";
  }
}

int32_t mxmoe_version(void) { return 4; }

mxmoe_status_t mxfp4_unpack(const uint8_t* blocks, const uint8_t* scales, int64_t rows, int64_t k, void* out,
                            int32_t out_dtype, void* stream) {
  if (rows < 0 || k <= 0 || k % 32 != 0 || k > kMaxDim) return MXMOE_ERR_SHAPE;
  if (out_dtype != MXMOE_F32 && out_dtype != MXMOE_BF16) return MXMOE_ERR_DTYPE;
  if (rows == 0) return MXMOE_OK;
  if (!blocks || !scales || !out) return MXMOE_ERR_NULL;
  if (!aligned16(blocks) || !aligned16(scales) || !aligned16(out)) return MXMOE_ERR_ALIGN;
  const int64_t nblocks = rows * (k / 32);
  if (nblocks / (k / 32) != rows || nblocks > kMaxGridItems) return MXMOE_ERR_SHAPE;
  return hip_status(launch_unpack(blocks, scales, nblocks, out, out_dtype == MXMOE_BF16,
                                  static_cast<hipStream_t>(stream)));
}

mxmoe_status_t mxfp4_pack(const void* w, int32_t w_dtype, int64_t rows, int64_t k, uint8_t* blocks,
                          uint8_t* scales, void* stream) {
  if (rows < 0 || k <= 0 || k % 32 != 0 || k > kMaxDim) return MXMOE_ERR_SHAPE;
  if (w_dtype != MXMOE_F32 && w_dtype != MXMOE_BF16) return MXMOE_ERR_DTYPE;
  if (rows == 0) return MXMOE_OK;
  if (!w || !blocks || !scales) return MXMOE_ERR_NULL;
  if (!aligned16(w) || !aligned16(blocks) || !aligned16(scales)) return MXMOE_ERR_ALIGN;
  const int64_t nblocks = rows * (k / 32);
  if (nblocks / (k / 32) != rows || nblocks > kMaxGridItems) return MXMOE_ERR_SHAPE;
  return hip_status(launch_pack(w, w_dtype == MXMOE_BF16, nblocks, blocks, scales, static_cast<hipStream_t>(stream)));
}

mxmoe_status_t mxfp4_tiled_bytes(int64_t mats, int64_t rows, int64_t k, int64_t* blocks_bytes,
                                 int64_t* scales_bytes) {
  if (mats < 0 || rows < 0 || k <= 0 || k % 32 != 0 || k > kMaxDim || rows > kMaxDim * 16) return MXMOE_ERR_SHAPE;
  if (!blocks_bytes || !scales_bytes) return MXMOE_ERR_NULL;
  int64_t bb, sb;
  tiled_sizes(1, rows, k, &bb, &sb);
  if (mats > 0 && bb > (int64_t(1) << 62) / mats) return MXMOE_ERR_SHAPE;
  *blocks_bytes = bb * mats;
  *scales_bytes = sb * mats;
  return MXMOE_OK;
}

mxmoe_status_t mxfp4_tile(const uint8_t* blocks, const uint8_t* scales, int64_t mats, int64_t rows, int64_t k,
                          uint8_t* tiled_blocks, uint8_t* tiled_scales, void* stream) {
  int64_t bb, sb;
  mxmoe_status_t st = mxfp4_tiled_bytes(mats, rows, k, &bb, &sb);
  if (st != MXMOE_OK) return st;
  if (mats == 0 || rows == 0) return MXMOE_OK;
  if (bb / 16 > kMaxGridItems) return MXMOE_ERR_SHAPE;
  if (!blocks || !scales || !tiled_blocks || !tiled_scales) return MXMOE_ERR_NULL;
  if (!aligned16(blocks) || !aligned16(scales) || !aligned16(tiled_blocks) || !aligned16(tiled_scales))
    return MXMOE_ERR_ALIGN;
  return hip_status(launch_tile(blocks, scales, mats, int(rows), int(k / 32), tiled_blocks, tiled_scales,
                                static_cast<hipStream_t>(stream)));
}

size_t moe_mxfp4_workspace_bytes(const mxmoe_layer_t* L, int64_t T, const mxmoe_fwd_opts_t* o) {
  if (check_layer(L) != MXMOE_OK || !o) return 0;
  if (o->expert_path != MXMOE_PATH_ROUTED && o->expert_path != MXMOE_PATH_DENSE) return 0;
  const bool dense = o->expert_path == MXMOE_PATH_DENSE;
  if (check_tokens(L, T, dense) != MXMOE_OK) return 0;
  if (o->act_dtype != MXMOE_F32 && o->act_dtype != MXMOE_BF16) return 0;
  return layout(L->E, L->H, L->I, L->top_k, T, o->act_dtype, o->fp8_act == 1, gemm_rows(L, T, dense)).total;
}

mxmoe_status_t moe_mxfp4_forward(const mxmoe_layer_t* L, const void* x, int64_t T, void* out,
                                 const mxmoe_fwd_opts_t* o, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(L, x, T, out, o, ws, ws_bytes, stream);
}

mxmoe_status_t moe_mxfp4_route(const mxmoe_layer_t* L, const void* x, int64_t T, const mxmoe_fwd_opts_t* o,
                               int32_t* idx_out, float* w_out, int32_t* counts_out, int32_t* offsets_out,
                               int32_t* sorted_out, int32_t* pos_out, void* ws, size_t ws_bytes, void* stream) {
  mxmoe_status_t st = check_layer(L);
  if (st != MXMOE_OK) return st;
  if ((st = check_opts(L, o, false)) != MXMOE_OK) return st;
  if ((st = check_tokens(L, T)) != MXMOE_OK) return st;
  if (T == 0) return MXMOE_OK;
  if (!x || !ws) return MXMOE_ERR_NULL;
  const void* outs[] = {x, ws, idx_out, w_out, counts_out, offsets_out, sorted_out, pos_out};
  for (const void* p : outs)
    if (p && !aligned16(p)) return MXMOE_ERR_ALIGN;
  const Workspace w = layout(L->E, L->H, L->I, L->top_k, T, o->act_dtype, o->fp8_act == 1, gemm_rows(L, T, false));
  if (ws_bytes < w.total) return MXMOE_ERR_WORKSPACE;
  return hip_status(run_routing(L, x, T, o->act_dtype, w, ws, idx_out, w_out, counts_out, offsets_out, sorted_out,
                                pos_out, static_cast<hipStream_t>(stream)));
}

mxmoe_status_t moe_mxfp4_calibrate_fp8(const mxmoe_layer_t* L, const void* x, int64_t T, float* scales_out, void* ws,
                                       size_t ws_bytes, void* stream) {
  mxmoe_status_t st = check_layer(L);
  if (st != MXMOE_OK) return st;
  if (L->param_dtype != MXMOE_BF16) return MXMOE_ERR_DTYPE;
  if ((st = check_tokens(L, T)) != MXMOE_OK) return st;
  if (T < 1) return MXMOE_ERR_SHAPE;
  if (!x || !scales_out || !ws) return MXMOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(scales_out) || !aligned16(ws)) return MXMOE_ERR_ALIGN;
  const Workspace w = layout(L->E, L->H, L->I, L->top_k, T, MXMOE_BF16, false, gemm_rows(L, T, false));
  if (ws_bytes < w.total) return MXMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool prefill = use_prefill(L, T, ACT_BF16);
  const bool records = prefill && L->weight_layout == MXMOE_LAYOUT_TILED;
  hipError_t e = run_routing(L, x, T, MXMOE_BF16, w, ws, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, s,
                             nullptr, false, nullptr, 1.0f, records);
  if (e != hipSuccess) return MXMOE_ERR_HIP;
  GemmArgs g0 = gemm_args(L, w, ws, T, ACT_BF16, 0);
  g0.bsrc = x;
  if (records) {
    g0.blk_rec = at<int4>(ws, w.rec0);
    g0.item_head = at<uint32_t>(ws, w.heads);
  }
  if (launch_moe_gemm(g0, prefill, s) != hipSuccess) return MXMOE_ERR_HIP;
  uint32_t* slots = at<uint32_t>(ws, w.calib);
  if (launch_calib_init(slots, s) != hipSuccess) return MXMOE_ERR_HIP;
  if (launch_amax_bf16(static_cast<const uint16_t*>(x), T * L->H, slots, s) != hipSuccess) return MXMOE_ERR_HIP;
  if (launch_amax_bf16(at<uint16_t>(ws, w.h), T * L->top_k * L->I, slots + 1, s) != hipSuccess) return MXMOE_ERR_HIP;
  return hip_status(launch_calib_finish(slots, scales_out, s));
}

}  // extern "C"

// ---------------------------------------------------------- dense layer

namespace {

struct LinearWorkspace {
  size_t offsets, active, tile_off, tiles, bias, total;
};

LinearWorkspace linear_layout(int64_t T, int64_t N, int act_dtype) {
  LinearWorkspace w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  w.offsets = take(2 * 4);
  w.active = take(2 * 16);
  w.tile_off = take(2 * 4);
  w.tiles = take(size_t((T + kPrefillTokens - 1) / kPrefillTokens) * 16 + 16);
  w.bias = take(size_t(N) * (act_dtype == MXMOE_BF16 ? 2 : 4));
  w.total = o;
  return w;
}

mxmoe_status_t check_linear(int64_t T, int64_t K, int64_t N, int32_t act_dtype, int32_t layout) {
  if (T < 0 || K <= 0 || N <= 0 || K % 32 != 0 || N % 32 != 0 || K > kMaxDim || N > kMaxDim) return MXMOE_ERR_SHAPE;
  if (T > kMaxSlots) return MXMOE_ERR_SHAPE;
  if (act_dtype != MXMOE_F32 && act_dtype != MXMOE_BF16) return MXMOE_ERR_DTYPE;
  if (layout != MXMOE_LAYOUT_ROWS && layout != MXMOE_LAYOUT_TILED) return MXMOE_ERR_VALUE;
  // 32-bit buffer windows over x, out and the weight (both orders)
  if (T * K * 4 > kMaxWindow || T * N * 4 > kMaxWindow) return MXMOE_ERR_SHAPE;
  int64_t bb, sb;
  tiled_sizes(1, N, K, &bb, &sb);
  if (bb > kMaxWindow || N * K / 2 > kMaxWindow) return MXMOE_ERR_SHAPE;
  return MXMOE_OK;
}

}  // namespace

extern "C" {

size_t mxfp4_linear_workspace_bytes(int64_t T, int64_t N, int32_t act_dtype) {
  if (T < 0 || N <= 0 || N > kMaxDim || T > kMaxSlots) return 0;
  if (act_dtype != MXMOE_F32 && act_dtype != MXMOE_BF16) return 0;
  return linear_layout(T, N, act_dtype).total;
}

mxmoe_status_t mxfp4_linear(const void* x, int64_t T, int64_t K, const uint8_t* w_blocks, const uint8_t* w_scales,
                            int32_t weight_layout, const void* bias, int64_t N, int32_t act_dtype, void* out,
                            void* ws, size_t ws_bytes, void* stream) {
  mxmoe_status_t st = check_linear(T, K, N, act_dtype, weight_layout);
  if (st != MXMOE_OK) return st;
  if (T == 0) return MXMOE_OK;
  if (!x || !w_blocks || !w_scales || !out || !ws) return MXMOE_ERR_NULL;
  const void* ptrs[] = {x, w_blocks, w_scales, out, ws, bias};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MXMOE_ERR_ALIGN;
  const LinearWorkspace w = linear_layout(T, N, act_dtype);
  if (ws_bytes < w.total) return MXMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ebytes = act_dtype == MXMOE_BF16 ? 2 : 4;
  if (launch_linear_setup(int(T), at<int32_t>(ws, w.offsets), at<int4>(ws, w.active), at<int32_t>(ws, w.tile_off),
                          at<int4>(ws, w.tiles), bias ? nullptr : at<void>(ws, w.bias), int(N), ebytes, s) != hipSuccess)
    return MXMOE_ERR_HIP;
  // the down-projection epilogue of the grouped GEMM (bias added, no
  // SwiGLU), over the token rows in order
  GemmArgs g{};
  g.act = act_dtype == MXMOE_BF16 ? ACT_BF16 : ACT_F32;
  g.phase = 1;
  g.wblk = w_blocks;
  g.wsc = w_scales;
  g.tiled = weight_layout == MXMOE_LAYOUT_TILED;
  g.bias = bias ? bias : at<void>(ws, w.bias);
  g.bias_bf16 = act_dtype == MXMOE_BF16;
  g.R = int(N);
  g.nb = int(K / 32);
  g.top_k = 1;
  g.E = 1;
  g.bsrc = x;
  g.b_rows = T;
  g.T = int(T);
  g.offsets = at<int32_t>(ws, w.offsets);
  g.active = at<int4>(ws, w.active);
  g.tile_off = at<int32_t>(ws, w.tile_off);
  g.tiles = at<int4>(ws, w.tiles);
  g.out = out;
  g.acc_scale = 1.0f;
  g.out_inv_scale = 1.0f;
  g.max_active = 1;
  g.max_tiles = int((T + kPrefillTokens - 1) / kPrefillTokens);
  g.n_slots = int(T);
  const bool prefill = g.act != ACT_F32 && T > 16;
  return hip_status(launch_moe_gemm(g, prefill, s));
}

}  // extern "C"

// ------------------------------------------------------- dense FP8 layer

namespace {

int64_t fp8_tiled_size(int64_t N, int64_t K) { return 4 * ((N + 63) / 64) * ((K + 127) / 128) * 2048; }

struct Fp8LinearWorkspace {
  size_t offsets, active, tile_off, tiles, bias, xq, total;
};

Fp8LinearWorkspace fp8_linear_layout(int64_t T, int64_t K, int64_t N) {
  Fp8LinearWorkspace w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  w.offsets = take(2 * 4);
  w.active = take(2 * 16);
  w.tile_off = take(2 * 4);
  w.tiles = take(size_t((T + kPrefillTokens - 1) / kPrefillTokens) * 16 + 16);
  w.bias = take(size_t(N) * 2);
  w.xq = take(size_t(T) * size_t(K));
  w.total = o;
  return w;
}

mxmoe_status_t check_fp8_dims(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % 32 != 0 || K % 32 != 0 || N > kMaxDim || K > kMaxDim) return MXMOE_ERR_SHAPE;
  if (fp8_tiled_size(N, K) > kMaxWindow) return MXMOE_ERR_SHAPE;
  return MXMOE_OK;
}

}  // namespace

extern "C" {

mxmoe_status_t fp8_tiled_bytes(int64_t N, int64_t K, int64_t* bytes) {
  mxmoe_status_t st = check_fp8_dims(N, K);
  if (st != MXMOE_OK) return st;
  if (!bytes) return MXMOE_ERR_NULL;
  *bytes = fp8_tiled_size(N, K);
  return MXMOE_OK;
}

mxmoe_status_t fp8_tile(const uint8_t* w, int64_t N, int64_t K, uint8_t* tiled, void* stream) {
  mxmoe_status_t st = check_fp8_dims(N, K);
  if (st != MXMOE_OK) return st;
  if (!w || !tiled) return MXMOE_ERR_NULL;
  if (!aligned16(w) || !aligned16(tiled)) return MXMOE_ERR_ALIGN;
  return hip_status(launch_byte_tile(w, 1, int(N), int(K), tiled, static_cast<hipStream_t>(stream)));
}

size_t fp8_linear_workspace_bytes(int64_t T, int64_t K, int64_t N) {
  if (T < 0 || T > kMaxSlots || check_fp8_dims(N, K) != MXMOE_OK) return 0;
  return fp8_linear_layout(T, K, N).total;
}

mxmoe_status_t fp8_linear(const void* x, int64_t T, int64_t K, const uint8_t* w_tiled, float w_scale, float x_scale,
                          const void* bias, int64_t N, void* out, void* ws, size_t ws_bytes, void* stream) {
  mxmoe_status_t st = check_fp8_dims(N, K);
  if (st != MXMOE_OK) return st;
  if (T < 0 || T > kMaxSlots) return MXMOE_ERR_SHAPE;
  // 32-bit buffer windows over x (bf16), its FP8 codes and out (bf16)
  if (T * K * 2 > kMaxWindow || T * N * 2 > kMaxWindow) return MXMOE_ERR_SHAPE;
  if (!(std::isfinite(w_scale) && w_scale > 0.f && std::isfinite(x_scale) && x_scale > 0.f)) return MXMOE_ERR_VALUE;
  if (!std::isfinite(1.0f / x_scale) || !std::isfinite(x_scale * w_scale)) return MXMOE_ERR_VALUE;
  if (T == 0) return MXMOE_OK;
  if (!x || !w_tiled || !out || !ws) return MXMOE_ERR_NULL;
  const void* ptrs[] = {x, w_tiled, out, ws, bias};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MXMOE_ERR_ALIGN;
  const Fp8LinearWorkspace w = fp8_linear_layout(T, K, N);
  if (ws_bytes < w.total) return MXMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_linear_setup(int(T), at<int32_t>(ws, w.offsets), at<int4>(ws, w.active), at<int32_t>(ws, w.tile_off),
                          at<int4>(ws, w.tiles), bias ? nullptr : at<void>(ws, w.bias), int(N), 2, s) != hipSuccess)
    return MXMOE_ERR_HIP;
  // x -> e4m3 codes with the static input scale (the MoE FP8 mode's rule)
  if (launch_quant_fp8(static_cast<const uint16_t*>(x), T * K, 1.0f / x_scale, at<uint8_t>(ws, w.xq), s) !=
      hipSuccess)
    return MXMOE_ERR_HIP;
  GemmArgs g{};
  g.act = ACT_W8A8;
  g.phase = 1;
  g.wblk = w_tiled;
  g.wsc = w_tiled;
  g.tiled = 1;
  g.bias = bias ? bias : at<void>(ws, w.bias);
  g.bias_bf16 = 1;
  g.R = int(N);
  g.nb = int(K / 32);
  g.top_k = 1;
  g.E = 1;
  g.bsrc = at<void>(ws, w.xq);
  g.b_rows = T;
  g.T = int(T);
  g.offsets = at<int32_t>(ws, w.offsets);
  g.active = at<int4>(ws, w.active);
  g.tile_off = at<int32_t>(ws, w.tile_off);
  g.tiles = at<int4>(ws, w.tiles);
  g.out = out;
  g.acc_scale = x_scale * w_scale;
  g.out_inv_scale = 1.0f;
  g.max_active = 1;
  g.max_tiles = int((T + kPrefillTokens - 1) / kPrefillTokens);
  g.n_slots = int(T);
  return hip_status(launch_moe_gemm(g, true, s));
}

}  // extern "C"

// ------------------------------------------------------ int8 W8A8 layer

namespace {

int64_t byte_tiled_size(int64_t rows, int64_t k) { return 4 * ((rows + 63) / 64) * ((k + 127) / 128) * 2048; }

mxmoe_status_t check_int8_layer(const mxmoe_int8_layer_t* L) {
  if (!L) return MXMOE_ERR_NULL;
  if (L->E < 1 || L->E > MXMOE_MAX_EXPERTS) return MXMOE_ERR_SHAPE;
  if (L->H <= 0 || L->I <= 0 || L->H > kMaxDim || L->I > kMaxDim || L->H % 32 != 0 || L->I % 32 != 0)
    return MXMOE_ERR_SHAPE;
  if (L->top_k < 1 || L->top_k > MXMOE_MAX_TOPK || L->top_k > L->E) return MXMOE_ERR_SHAPE;
  if (byte_tiled_size(2 * int64_t(L->I), L->H) > kMaxWindow || byte_tiled_size(L->H, L->I) > kMaxWindow)
    return MXMOE_ERR_SHAPE;
  const void* ptrs[] = {L->gate_up_w, L->gate_up_scale, L->gate_up_bias, L->down_w,
                        L->down_scale, L->down_bias,    L->router_w,     L->router_b};
  for (const void* p : ptrs)
    if (!p) return MXMOE_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MXMOE_ERR_ALIGN;
  return MXMOE_OK;
}

// The routing view of an int8 layer: dimensions, router and (for the GEMM
// argument setup) biases; the weight fields are replaced before each launch.
mxmoe_layer_t routing_view(const mxmoe_int8_layer_t* L) {
  mxmoe_layer_t r{};
  r.E = L->E;
  r.H = L->H;
  r.I = L->I;
  r.top_k = L->top_k;
  r.param_dtype = MXMOE_BF16;
  r.weight_layout = MXMOE_LAYOUT_TILED;
  r.gate_up_blocks = L->gate_up_w;
  r.gate_up_scales = L->gate_up_w;
  r.gate_up_bias = L->gate_up_bias;
  r.down_blocks = L->down_w;
  r.down_scales = L->down_w;
  r.down_bias = L->down_bias;
  r.router_w = L->router_w;
  r.router_b = L->router_b;
  return r;
}

struct Int8Workspace {
  Workspace base;  // routing tables, h (bf16), Y (bf16)
  size_t xq, sx, hq, sh, total;
};

Int8Workspace int8_layout(const mxmoe_int8_layer_t* L, int64_t T) {
  Int8Workspace w{};
  w.base = layout(L->E, L->H, L->I, L->top_k, T, MXMOE_BF16, false, T * L->top_k);
  size_t o = w.base.total;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t slots = size_t(T) * size_t(L->top_k);
  w.xq = take(size_t(T) * size_t(L->H));
  w.sx = take(size_t(T) * 4);
  w.hq = take(slots * size_t(L->I));
  w.sh = take(slots * 4);
  w.total = o;
  return w;
}

}  // namespace

extern "C" {

mxmoe_status_t int8_tiled_bytes(int64_t mats, int64_t rows, int64_t k, int64_t* bytes) {
  if (mats < 0 || rows <= 0 || k <= 0 || rows % 32 != 0 || k % 32 != 0 || rows > kMaxDim || k > kMaxDim)
    return MXMOE_ERR_SHAPE;
  if (!bytes) return MXMOE_ERR_NULL;
  const int64_t one = byte_tiled_size(rows, k);
  if (mats > 0 && one > (int64_t(1) << 62) / mats) return MXMOE_ERR_SHAPE;
  *bytes = one * mats;
  return MXMOE_OK;
}

mxmoe_status_t int8_tile(const int8_t* w, int64_t mats, int64_t rows, int64_t k, uint8_t* tiled, void* stream) {
  int64_t bytes;
  mxmoe_status_t st = int8_tiled_bytes(mats, rows, k, &bytes);
  if (st != MXMOE_OK) return st;
  if (mats == 0) return MXMOE_OK;
  if (bytes / 16 > kMaxGridItems) return MXMOE_ERR_SHAPE;
  if (!w || !tiled) return MXMOE_ERR_NULL;
  if (!aligned16(w) || !aligned16(tiled)) return MXMOE_ERR_ALIGN;
  return hip_status(launch_byte_tile(reinterpret_cast<const uint8_t*>(w), mats, int(rows), int(k), tiled,
                                     static_cast<hipStream_t>(stream)));
}

size_t moe_int8_workspace_bytes(const mxmoe_int8_layer_t* L, int64_t T) {
  if (check_int8_layer(L) != MXMOE_OK) return 0;
  const mxmoe_layer_t R = routing_view(L);
  if (check_tokens(&R, T) != MXMOE_OK) return 0;
  return int8_layout(L, T).total;
}

mxmoe_status_t moe_int8_forward(const mxmoe_int8_layer_t* L, const void* x, int64_t T, void* out,
                                int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  mxmoe_status_t st = check_int8_layer(L);
  if (st != MXMOE_OK) return st;
  const mxmoe_layer_t R = routing_view(L);
  if ((st = check_tokens(&R, T)) != MXMOE_OK) return st;
  if (T == 0) return MXMOE_OK;
  if (!x || !out || !ws) return MXMOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(out) || !aligned16(ws)) return MXMOE_ERR_ALIGN;
  if ((topk_idx_out && !aligned16(topk_idx_out)) || (topk_w_out && !aligned16(topk_w_out))) return MXMOE_ERR_ALIGN;
  const Int8Workspace w = int8_layout(L, T);
  if (ws_bytes < w.total) return MXMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Workspace& b = w.base;
  const bool prefill = use_prefill(&R, T, ACT_INT8);
  if (run_routing(&R, x, T, MXMOE_BF16, b, ws, topk_idx_out, topk_w_out, nullptr, nullptr, nullptr, nullptr, s,
                  nullptr, false, nullptr, 1.0f, prefill) != hipSuccess)
    return MXMOE_ERR_HIP;
  // per-token int8 x
  if (launch_quant_rows_int8(static_cast<const uint16_t*>(x), T, L->H, at<int8_t>(ws, w.xq), at<float>(ws, w.sx), s) !=
      hipSuccess)
    return MXMOE_ERR_HIP;
  // gate_up + SwiGLU -> h (bf16); decode-shaped batches take the decode
  // tile and fold the combine into the down GEMM, as the MXFP4 forward
  const bool fold = !prefill && T <= kFusedCombineTokens && T * L->top_k * int64_t(L->H) * 2 <= kMaxWindow;
  GemmArgs g0 = gemm_args(&R, b, ws, T, ACT_INT8, 0);
  g0.bsrc = at<void>(ws, w.xq);
  g0.row_scale = L->gate_up_scale;
  g0.tok_scale = at<float>(ws, w.sx);
  GemmArgs g1 = gemm_args(&R, b, ws, T, ACT_INT8, 1);
  g1.bsrc = at<void>(ws, w.hq);
  g1.row_scale = L->down_scale;
  g1.tok_scale = at<float>(ws, w.sh);
  if (prefill) {  // the grouping resolved every prefill workgroup's item
    g0.blk_rec = at<int4>(ws, b.rec0);
    g1.blk_rec = at<int4>(ws, b.rec1);
    g0.item_head = at<uint32_t>(ws, b.heads);
    g1.item_head = at<uint32_t>(ws, b.heads) + 8;
  }
  if (fold) {
    g0.cmb_count = g1.cmb_count = at<uint32_t>(ws, b.cmb);
    g0.n_cmb = g1.n_cmb = (L->H + 63) / 64;
    g1.cmb_out = out;
    g1.pos = at<int32_t>(ws, b.pos);
    g1.wts = at<float>(ws, b.wts);
  }
  if (launch_moe_gemm(g0, prefill, s) != hipSuccess) return MXMOE_ERR_HIP;
  // per-row int8 h
  const int64_t slots = T * L->top_k;
  if (launch_quant_rows_int8(at<uint16_t>(ws, b.h), slots, L->I, at<int8_t>(ws, w.hq), at<float>(ws, w.sh), s) !=
      hipSuccess)
    return MXMOE_ERR_HIP;
  // down -> Y (bf16), and the output when the combine is folded in
  if (launch_moe_gemm(g1, prefill, s) != hipSuccess) return MXMOE_ERR_HIP;
  if (fold) return MXMOE_OK;
  CombineArgs ca{};
  ca.Y = at<void>(ws, b.y);
  ca.y_bf16 = 1;
  ca.pos = at<int32_t>(ws, b.pos);
  ca.wts = at<float>(ws, b.wts);
  ca.out = out;
  ca.out_bf16 = 1;
  ca.T = int(T);
  ca.H = L->H;
  ca.top_k = L->top_k;
  return hip_status(launch_combine(ca, s));
}

}  // extern "C"

// ------------------------------------------- forward without allocation
//
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the forward's scratch space is one file-scope device array of
// MXMOE_NOALLOC_SCRATCH_BYTES, which every GPU the library runs on holds
// until the process ends.  In host code the array's name only stands in for
// it; its device address is looked up once per device with that device
// current, and only that address is handed to kernels.

namespace {

static __device__ __align__(256) uint8_t scratch[MXMOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// This device's copy of `scratch` (the current device's; looked up on its
// first use and kept).
mxmoe_status_t scratch_address(void** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MXMOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MXMOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return MXMOE_ERR_HIP;
    g_scratch_ptr[dev] = q;
  }
  *p = g_scratch_ptr[dev];
  return MXMOE_OK;
}

}  // namespace

extern "C" {

mxmoe_status_t moe_mxfp4_forward_noalloc(const mxmoe_layer_t* L, const void* x, int64_t T, void* out,
                                         const mxmoe_fwd_opts_t* o, void* stream) {
  mxmoe_status_t st = check_layer(L);
  if (st != MXMOE_OK) return st;
  if ((st = check_opts(L, o, true)) != MXMOE_OK) return st;
  const bool dense = o->expert_path == MXMOE_PATH_DENSE;
  if ((st = check_tokens(L, T, dense)) != MXMOE_OK) return st;
  if (T == 0) return MXMOE_OK;
  const size_t need = layout(L->E, L->H, L->I, L->top_k, T, o->act_dtype, o->fp8_act == 1, gemm_rows(L, T, dense)).total;
  if (need > MXMOE_NOALLOC_SCRATCH_BYTES) return MXMOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MXMOE_OK) return st;
  return forward_impl(L, x, T, out, o, ws, MXMOE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
