// Operand and epilogue helpers of the MXFP4 expert GEMMs (gfx950), shared
// by the prefill- and decode-shaped grouped-GEMM kernels.  The operand
// roles and K order they follow are described at the top of moe_gemm.hip.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace mxmoe {

// ------------------------------------------------------------ operands

struct AFrag {
  uint4 q;       // 16 bytes = 32 nibbles of one block of one weight row
  uint32_t sw;   // the aligned dword holding its e8m0 scale byte (0 past the tensor)
  uint32_t sh;   // bit position of that byte in sw
  // The scale byte is extracted at its use, not right after the load: an
  // extension next to the load would make every prefetch wait at once.
  __device__ __forceinline__ uint32_t scale() const { return (sw >> sh) & 0xFFu; }
};

// Weights of one expert as buffers.  Row order: blocks (R, nb, 16) and
// scales (R, nb).  Tiled order (declared in mxmoe.h): rt4 row tiles of 16
// rows x nc chunks, one 1 KB piece each, in the order the LDS tiles are
// read; scales in 256-byte groups per 64 rows and chunk, whose dword l
// holds the scales of lane l for the group's 4 row tiles.
struct WBuf {
  rsrc_t blk, sc;
  int R, nb;
  int rt4, nc;  // tiled order only
};

template <bool TILED>
__device__ __forceinline__ WBuf expert_weights(const GemmArgs& a, int e) {
  WBuf w;
  w.R = a.R;
  w.nb = a.nb;
  w.nc = (a.nb + 3) >> 2;
  w.rt4 = 4 * ((a.R + 63) >> 6);
  if constexpr (TILED) {
    const int64_t bb = int64_t(w.rt4) * w.nc * 1024, sb = int64_t(w.rt4 / 4) * w.nc * 256;
    w.blk = make_rsrc(a.wblk + int64_t(e) * bb, uint32_t(bb));
    w.sc = make_rsrc(a.wsc + int64_t(e) * sb, uint32_t(sb));
  } else {
    const int64_t rb = int64_t(a.R) * a.nb;
    w.blk = make_rsrc(a.wblk + int64_t(e) * rb * 16, uint32_t(rb * 16));
    w.sc = make_rsrc(a.wsc + int64_t(e) * rb, uint32_t(rb));
  }
  return w;
}

// 8-bit (e4m3 or int8) weights of expert e in the tiled 8-bit order
// (declared in mxmoe.h): rt4 row tiles of 16 rows x nc 128-wide chunks, 2 KB
// each, lane (g, r) holding row r's bytes 16g .. 16g+15 and 64+16g ..
// 64+16g+15 of the chunk (the K order of an 8-bit MFMA operand).  No block
// scales.
__device__ __forceinline__ WBuf byte_weights(const GemmArgs& a, int e) {
  WBuf w;
  w.R = a.R;
  w.nb = a.nb;
  w.nc = (a.nb + 3) >> 2;
  w.rt4 = 4 * ((a.R + 63) >> 6);
  const int64_t bb = int64_t(w.rt4) * w.nc * 2048;
  w.blk = make_rsrc(a.wblk + int64_t(e) * bb, uint32_t(bb));
  w.sc = w.blk;
  return w;
}

// Slot of block b of row r (both within a 16 x 4 piece) in a 1 KB tile:
// the block index is XOR-swizzled with the row so that the 16 lanes of a
// lane group read 16 distinct bank groups.
__device__ __forceinline__ int piece_slot(int r, int b) { return r * 4 + (b ^ ((r >> 2) & 3)); }

// Position of 16-byte piece p (K = 8p .. 8p+7 of the chunk) in the 256-byte
// LDS row of token tok, bf16 token tiles.  gfx950 serves ds_read_b128 16
// lanes at a time against 64 banks of 4 bytes; the 16 lanes of a group are
// the 4-lane blocks of one half-wave whose lane bits 2..4 have the same
// parity (measured with SQ_LDS_BANK_CONFLICT over lane patterns chosen to
// tell the candidate groupings apart), and a group is conflict-free when its
// 16 slots are distinct modulo 16.  In MFMA step st lane (g, r) reads piece
// 4g + st of token r; XOR-ing the piece with the token's low 4 bits rotated
// by 2 makes every group conflict-free for all four steps (checked for all
// of them against that grouping).
__device__ __forceinline__ int bf16_piece_pos(int tok, int p) { return p ^ (((tok << 2) | ((tok >> 2) & 3)) & 15); }

// Block `block` of weight row `row`; zero when either is out of range.
__device__ __forceinline__ AFrag load_a(const WBuf& w, int row, int block) {
  const bool ok = row < w.R && block < w.nb;
  const uint32_t o = uint32_t(row * w.nb + block);
  AFrag f;
  f.q = buf_load_b128(w.blk, ok ? o * 16u : kOOB);
  f.sw = buf_load_b32(w.sc, ok ? (o & ~3u) : kOOB);
  f.sh = (o & 3u) * 8u;
  return f;
}

// Tiled order: lane (g, r16) of row tile t, chunk c (block 4c+g of row
// 16t + r16); zero past the padded tensor.
__device__ __forceinline__ AFrag load_a_tiled(const WBuf& w, int t, int c, int r16, int g) {
  const bool ok = t < w.rt4 && c < w.nc;
  AFrag f;
  f.q = buf_load_b128(w.blk, ok ? uint32_t((t * w.nc + c) * 1024 + piece_slot(r16, g) * 16) : kOOB);
  f.sw = buf_load_b32(w.sc, ok ? uint32_t(((t >> 2) * w.nc + c) * 256 + (16 * g + r16) * 4) : kOOB);
  f.sh = uint32_t(t & 3) * 8u;
  return f;
}

__device__ __forceinline__ uint32_t dword(const uint4& q, int i) {
  return i == 0 ? q.x : (i == 1 ? q.y : (i == 2 ? q.z : q.w));
}

// The activation rows of a tile as a range-checked buffer: gate_up gathers
// x rows (any of the b_rows tokens) by token id; down reads its own n
// contiguous h rows from sorted row row_start on, so its window starts
// there (a dense layer's T*E rows of h can outgrow one 32-bit window).
__device__ __forceinline__ rsrc_t act_rows(const GemmArgs& a, int phase, int row_start, int n, uint32_t row_bytes) {
  if (phase == 0) return make_rsrc(a.bsrc, uint32_t(a.b_rows) * row_bytes);
  return make_rsrc(static_cast<const uint8_t*>(a.bsrc) + int64_t(row_start) * row_bytes, uint32_t(n) * row_bytes);
}

// Byte offset of token row j (of n >= 1) of a tile inside act_rows(...),
// or kOOB.  The token-id load is unconditional (clamped index) so it needs
// no branch.
__device__ __forceinline__ uint32_t act_row_offset(const GemmArgs& a, int phase, int row_start, int j, int n,
                                                   uint32_t row_bytes) {
  const int jc = min(j, n - 1);
  const int src_row = phase == 0 ? a.sorted_tok[row_start + jc] : jc;
  return j < n ? uint32_t(src_row) * row_bytes : kOOB;
}

// ------------------------------------------------------------ epilogue

// Store rows r0 .. r0+3 of one token (sorted row p), bias already added:
// gate_up applies the SwiGLU and writes h, down writes Y (bf16 when the
// activations are bf16, its only reader being the combine, which sums the
// k rows of a token in fp32; fp32 in the fp32 mode).
template <int ACT, int PHASE>
__device__ __forceinline__ void store_rows_biased(const GemmArgs& a, int r0, int64_t p, float v0, float v1, float v2,
                                                  float v3) {
  if constexpr (PHASE == 0) {
    // rows r0, r0+1 = (gate, up) of h column r0/2; rows r0+2, r0+3 the next
    const float h0 = clamped_swiglu(v0, v1);
    const float h1 = clamped_swiglu(v2, v3);
    const int64_t I = a.R / 2;
    const int64_t o = p * I + r0 / 2;
    if constexpr (ACT == ACT_BF16 || ACT == ACT_INT8) {  // int8: h stays bf16 until its per-row quantisation
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + o) = pack_bf16x2(h0, h1);
    } else if constexpr (ACT == ACT_F32) {
      *reinterpret_cast<float2*>(static_cast<float*>(a.out) + o) = make_float2(h0, h1);
    } else {
      const uint32_t q = pack_e4m3x4(h0 * a.out_inv_scale, h1 * a.out_inv_scale, 0.f, 0.f);
      *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(a.out) + o) = uint16_t(q & 0xFFFFu);
    }
  } else if constexpr (ACT == ACT_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + p * a.R + r0) = make_float4(v0, v1, v2, v3);
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + p * a.R + r0) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
  }
}

// Scale, add the bias of rows r0 .. r0+3 of expert e, and store.
template <int ACT, int PHASE>
__device__ __forceinline__ void store_rows(const GemmArgs& a, int e, int r0, int64_t p, float v0, float v1, float v2,
                                           float v3) {
  const int64_t bo = int64_t(e) * a.R + r0;
  store_rows_biased<ACT, PHASE>(a, r0, p, v0 * a.acc_scale + load_param(a.bias, bo + 0, a.bias_bf16),
                                v1 * a.acc_scale + load_param(a.bias, bo + 1, a.bias_bf16),
                                v2 * a.acc_scale + load_param(a.bias, bo + 2, a.bias_bf16),
                                v3 * a.acc_scale + load_param(a.bias, bo + 3, a.bias_bf16));
}

template <int N>
using IC = std::integral_constant<int, N>;

// Workgroup barrier that orders LDS traffic only: the global prefetches of
// later chunks stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace mxmoe
