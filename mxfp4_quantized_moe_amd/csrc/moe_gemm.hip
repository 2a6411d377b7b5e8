// MXFP4 grouped GEMMs of the MoE layer for gfx950, with the clamped-SwiGLU
// epilogue fused into gate_up and a routing-weighted combine.
//
// For each routed expert e (KerasFormers "mxfp4" page, "As GPT-OSS's native
// format": only the top-k experts of a token are evaluated, gate_up_proj is
// (E, 2I, H), down_proj is (E, H, I), biases full precision):
//   gate_up:  G = X_e W_gu[e]^T + b_gu[e],  h_i = swiglu(G[2i], G[2i+1])
//   down:     Y = h W_d[e]^T + b_d[e]
//   combine:  out_t = sum_j w[t, j] * Y(t, j)
//
// Operand roles.  Every MFMA takes A = weights (rows of W are the M
// dimension) and B = activations (tokens are the N dimension), so a lane's
// accumulator holds four consecutive weight rows of one token: with gate/up
// rows interleaved, (gate_i, up_i) sit in the same lane and the SwiGLU needs
// no data exchange.
//
// K order.  K is walked in chunks of 128 (four 32-value MXFP4 blocks).  In a
// chunk, lane group g (lanes 16g .. 16g+15) reads the whole 16-byte block
// 4c + g of its weight row with one 128-bit load plus its scale byte.  The
// activations are laid out to match:
//   bf16: step s (0..3) of the chunk consumes nibbles 8s..8s+7 of that block
//         (decoded by v_cvt_scalef32_pk_bf16_fp4 into the 16x16x32 bf16
//         MFMA) against x[128c + 32g + 8s .. +8];
//   f32:  step s (0..31) consumes value s of the block against x[128c+32g+s]
//         in the 16x16x4 f32 MFMA;
//   fp8:  the block goes straight into the scaled 16x16x128 MFMA (FP4 A
//         operand with its e8m0 scale byte), whose FP8 B operand holds
//         K = 128c + 16g .. +16 and 128c + 64 + 16g .. +16 in lane group g.
// This is a permutation of K applied to both operands, so each dot product
// is unchanged.  Blocks past K (when K/32 is not a multiple of 4) read as
// zero on both sides.
//
// All tile loads are range-checked buffer loads (see device_common.h): the
// tails read as zero without branches.
#include "decode_tile.h"
#include "gemm_common.h"
#include "xcd_split.h"

namespace mxmoe {

// Decode tile: row tiles of 16 weight rows per workgroup, and 128-K chunks
// whose weight loads each wave keeps in flight.  Overridable at build time
// for sweeps.
#ifndef MXMOE_DECODE_ROW_TILES
#define MXMOE_DECODE_ROW_TILES 1
#endif
#ifndef MXMOE_DECODE_CHUNKS
#define MXMOE_DECODE_CHUNKS 6
#endif
constexpr int kDecodeRowTiles = MXMOE_DECODE_ROW_TILES;
constexpr int kDecodeChunkBuf = MXMOE_DECODE_CHUNKS;


// =====================================================================
// Decode-shaped GEMM: few tokens per expert.  The bound is streaming the
// routed experts' packed weights, so each workgroup owns 16 weight rows of
// one active expert and its 4 waves split the K chunks (c = wave, wave+4,
// ...), issuing up to kDecodeChunkBuf 128-bit weight loads per lane before
// the first MFMA.  Partial sums are added across waves in a fixed order in
// LDS.  Activations (at most 64 tokens per pass) are read straight from
// global memory, where they stay cache-resident.
// =====================================================================

template <int ACT, int PHASE, bool TILED>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs a) {
  constexpr int RT = kDecodeRowTiles;
  __shared__ f32x4_t red[4][RT][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int slot = blockIdx.y;
  // one round trip: slots past the active experts hold empty records
  const int4 rec = a.active[1 + slot];
  hold_uniform(rec);
  if (rec.z == 0) return;
  const int e = rec.x, row_start = rec.y, n_e = rec.z;
  const int nb = a.nb, K = nb * 32;
  const int nchunks = (nb + 3) >> 2;
  const int rbase = blockIdx.x * (16 * RT);
  const WBuf wb = expert_weights<TILED>(a, e);
  constexpr int EB = ACT == ACT_F32 ? 4 : (ACT == ACT_BF16 ? 2 : 1);  // bytes per B element
  const uint32_t row_bytes = uint32_t(K) * EB;
  const rsrc_t bsrc = act_rows(a, PHASE, row_start, n_e, row_bytes);

  for (int tg = 0; tg < n_e; tg += 64) {
    // byte offset of this lane's token row for each of the 4 token sub-tiles
    uint32_t boff[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) boff[nt] = act_row_offset(a, PHASE, row_start, tg + nt * 16 + r16, n_e, row_bytes);
    const int nt_active = min(4, (n_e - tg + 15) >> 4);

    // specialised on the number of active token sub-tiles: no branches
    // between the loads and the MFMAs of a chunk group
    auto pass = [&](auto ntc) __attribute__((always_inline)) {
      constexpr int NA = decltype(ntc)::value;
      f32x4_t acc[RT][NA];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NA; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      for (int c0 = wave; c0 < nchunks; c0 += 4 * kDecodeChunkBuf) {
        AFrag af[kDecodeChunkBuf][RT];
#pragma unroll
        for (int u = 0; u < kDecodeChunkBuf; ++u)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            if constexpr (TILED)
              af[u][rt] = load_a_tiled(wb, (rbase >> 4) + rt, c0 + 4 * u, r16, g);
            else
              af[u][rt] = load_a(wb, rbase + 16 * rt + r16, 4 * (c0 + 4 * u) + g);
          }
        // chunks past the end are all zeros (range-checked loads)
#pragma unroll
        for (int u = 0; u < kDecodeChunkBuf; ++u) {
          const int c = c0 + 4 * u;
          if constexpr (ACT == ACT_BF16) {
            const uint32_t kofs = (4 * c + g < nb) ? uint32_t(128 * c + 32 * g) * 2 : kOOB;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              bf16x8_t b[NA];
#pragma unroll
              for (int nt = 0; nt < NA; ++nt)
                b[nt] = __builtin_bit_cast(bf16x8_t, buf_load_b128(bsrc, oob_add(boff[nt], kofs + 16 * s)));
#pragma unroll
              for (int rt = 0; rt < RT; ++rt) {
                const bf16x8_t av = fp4x8_to_bf16x8(dword(af[u][rt].q, s), e8m0_as_scale_operand(af[u][rt].scale()));
#pragma unroll
                for (int nt = 0; nt < NA; ++nt)
                  acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[nt], acc[rt][nt], 0, 0, 0);
              }
            }
          } else if constexpr (ACT == ACT_F32) {
#pragma unroll
            for (int s4 = 0; s4 < 8; ++s4) {
              const uint32_t kofs = (4 * c + g < nb) ? uint32_t(128 * c + 32 * g + 4 * s4) * 4 : kOOB;
              float4 b[NA];
#pragma unroll
              for (int nt = 0; nt < NA; ++nt) {
                const uint4 q = buf_load_b128(bsrc, oob_add(boff[nt], kofs));
                b[nt] = make_float4(__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z),
                                    __uint_as_float(q.w));
              }
#pragma unroll
              for (int rt = 0; rt < RT; ++rt) {
                const uint32_t w = dword(af[u][rt].q, s4 >> 1);
                const float sc = e8m0_as_scale_operand(af[u][rt].scale());
                f32x2_t lo, hi;
                if (s4 & 1) {
                  lo = fp4x2_to_f32x2<2>(w, sc);
                  hi = fp4x2_to_f32x2<3>(w, sc);
                } else {
                  lo = fp4x2_to_f32x2<0>(w, sc);
                  hi = fp4x2_to_f32x2<1>(w, sc);
                }
#pragma unroll
                for (int nt = 0; nt < NA; ++nt) {
                  acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(lo[0], b[nt].x, acc[rt][nt], 0, 0, 0);
                  acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(lo[1], b[nt].y, acc[rt][nt], 0, 0, 0);
                  acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(hi[0], b[nt].z, acc[rt][nt], 0, 0, 0);
                  acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(hi[1], b[nt].w, acc[rt][nt], 0, 0, 0);
                }
              }
            }
          } else {
            // FP8: B lane group g holds K = 128c + 16g .. +16 and 128c + 64 + 16g .. +16
            const uint32_t k0 = (4 * c + (g >> 1) < nb) ? uint32_t(128 * c + 16 * g) : kOOB;
            const uint32_t k1 = (4 * c + 2 + (g >> 1) < nb) ? uint32_t(128 * c + 64 + 16 * g) : kOOB;
            i32x8_t b[NA];
#pragma unroll
            for (int nt = 0; nt < NA; ++nt) {
              const uint4 p0 = buf_load_b128(bsrc, oob_add(boff[nt], k0));
              const uint4 p1 = buf_load_b128(bsrc, oob_add(boff[nt], k1));
              b[nt] = i32x8_t{int(p0.x), int(p0.y), int(p0.z), int(p0.w), int(p1.x), int(p1.y), int(p1.z), int(p1.w)};
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              const uint4 q = af[u][rt].q;
              const i32x8_t av = i32x8_t{int(q.x), int(q.y), int(q.z), int(q.w), 0, 0, 0, 0};
#pragma unroll
              for (int nt = 0; nt < NA; ++nt)
                acc[rt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b[nt], acc[rt][nt], 4, 0, 0,
                                                                               int(af[u][rt].scale()), 0, 127);
            }
          }
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NA; ++nt) red[wave][rt][nt][lane] = acc[rt][nt];
    };
    switch (nt_active) {
      case 1: pass(IC<1>{}); break;
      case 2: pass(IC<2>{}); break;
      case 3: pass(IC<3>{}); break;
      default: pass(IC<4>{}); break;
    }
    __syncthreads();

    // fixed-order sum of the 4 waves' partial sums; wave w finishes sub-tile w
    {
      const int nt = wave;
      const int j = tg + nt * 16 + r16;
      if (nt < nt_active && j < n_e) {
        const int64_t p = row_start + j;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if (rbase + 16 * rt < a.R) {  // R is a multiple of 16
            f32x4_t s = red[0][rt][nt][lane];
            s += red[1][rt][nt][lane];
            s += red[2][rt][nt][lane];
            s += red[3][rt][nt][lane];
            store_rows<ACT, PHASE>(a, e, rbase + 16 * rt + 4 * g, p, s[0], s[1], s[2], s[3]);
          }
        }
      }
    }
    __syncthreads();
  }
}

// Prefill-shaped GEMM: many tokens per expert, bound by the matrix cores.
//
// Workgroup tile = kPrefillRows weight rows x 128 tokens of one expert, K
// walked in 128-wide chunks, 8 waves of 16*RT rows x all 128 tokens each,
// two waves per SIMD so that one wave's MFMAs cover the other's LDS reads,
// decodes and barrier waits.  The tile is sized for the bytes a CU can
// pull from L2: with ~50 outstanding 64-byte misses per CU and ~360-cycle
// L2 latency a CU streams ~20 GB/s, so the tile must do ~250 flops per
// byte it fetches (a 256 x 64 tile does ~125 and stalls on memory).
//   * Both operands of a chunk travel global -> LDS by the buffer-to-LDS
//     DMA form of the loads (no registers held while in flight) into a ring
//     of S stages, so S-1 chunks are in flight while one is computed; one
//     barrier per chunk publishes a landed stage and frees the one computed
//     last.
//   * A (weights): 16 rows x 4 blocks (1 KB) per row tile, the block of each
//     16-byte piece XOR-swizzled with the row so that the 16 lanes of a lane
//     group read 16 different bank groups.  Scale bytes go to registers
//     (one aligned dword per row tile).
//   * B (activations): 64 gathered token rows of the chunk, pieces
//     XOR-swizzled by token (bf16_piece_pos for bf16).
// Each wave decodes its own weight rows into bf16 registers right before
// the MFMAs; a wave whose rows all lie past the matrix skips its MFMAs, so
// a partial last row stripe costs little.  The work list is (token tile, row stripe) with the stripe
// fastest, and workgroup ids are remapped so that consecutive items land on
// the same XCD and share its L2.  Expert, first row and token count of each
// tile come from the table the grouping kernel writes.
// =====================================================================

constexpr int kPrefillRT = kPrefillRows / 128;      // row tiles of 16 per row group
constexpr int kPrefillStages = MXMOE_PREFILL_STAGES;
constexpr int kPrefillThreads = 512;


template <int ACT, int PHASE, bool TILED>
__global__ __launch_bounds__(kPrefillThreads) void gemm_prefill_kernel(GemmArgs a) {
  static_assert(ACT == ACT_BF16 || ACT == ACT_FP8, "prefill path takes bf16 or fp8 activations");
  static_assert(kPrefillTokens == 128, "eight 16-token sub-tiles per tile");
  constexpr int RT = kPrefillRT, S = kPrefillStages;
  constexpr int EB = ACT == ACT_BF16 ? 2 : 1;
  constexpr int KB = 128 * EB;                  // bytes of one token row per chunk
  constexpr int PPR = KB / 16;                  // 16-byte pieces per token row (16 or 8)
  constexpr int TPL = 64 / PPR;                 // tokens per 1 KB B load (4 or 8)
  constexpr int NBL = 128 / TPL;                // B loads per chunk (32 or 16)
  constexpr int BLOADS = NBL / 8;               // B loads per wave per chunk (4 or 2)
  constexpr int A_BYTES = 8 * RT * 1024;        // A region of a stage
  constexpr int B_BYTES = 128 * KB;             // B region of a stage
  constexpr int SLOADS = TILED ? 1 : RT;        // scale dword loads per wave per chunk
  constexpr int LOADS = RT + SLOADS + BLOADS;   // VMEM instructions per wave per chunk
  static_assert(!TILED || RT == 1 || RT == 2 || RT == 4, "a wave's row tiles share one scale group");
  static_assert(S >= 2 && S <= 5, "2..5 stages");
  // One LDS object per stage and operand: distinct objects let the compiler
  // see that a DMA into one stage cannot alias reads of another, so it does
  // not drain the loads in flight before every LDS read.
  __shared__ __align__(16) uint8_t sA0[A_BYTES], sA1[A_BYTES], sA2[S > 2 ? A_BYTES : 16],
      sA3[S > 3 ? A_BYTES : 16], sA4[S > 4 ? A_BYTES : 16];
  __shared__ __align__(16) uint8_t sB0[B_BYTES], sB1[B_BYTES], sB2[S > 2 ? B_BYTES : 16],
      sB3[S > 3 ? B_BYTES : 16], sB4[S > 4 ? B_BYTES : 16];
  auto stage_a = [&](auto uc) -> uint8_t* {
    constexpr int u = decltype(uc)::value;
    if constexpr (u == 0) return sA0;
    else if constexpr (u == 1) return sA1;
    else if constexpr (u == 2) return sA2;
    else if constexpr (u == 3) return sA3;
    else return sA4;
  };
  auto stage_b = [&](auto uc) -> uint8_t* {
    constexpr int u = decltype(uc)::value;
    if constexpr (u == 0) return sB0;
    else if constexpr (u == 1) return sB1;
    else if constexpr (u == 2) return sB2;
    else if constexpr (u == 3) return sB3;
    else return sB4;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;

  // Work items (token tile, row stripe), stripe fastest.  The grid is sized
  // for the most tiles a routing can produce; the valid items are the first
  // nvalid.  Hardware places workgroup b on XCD b % 8, so XCD x takes the
  // x-th eighth of the valid items, in order: every XCD gets an even share
  // and the stripes of one token tile run on one XCD, sharing its L2.
  const int nstripes = (a.R + kPrefillRows - 1) / kPrefillRows;
  const int nvalid = a.tile_off[a.E] * nstripes;
  const int per_xcd = (nvalid + 7) >> 3;
  const int idx = blockIdx.x >> 3;
  const int item = (blockIdx.x & 7) * per_xcd + idx;
  if (idx >= per_xcd || item >= nvalid) return;
  const int tile = item / nstripes, stripe = item - tile * nstripes;
  const int4 ti = a.tiles[tile];  // {expert, first sorted row, tokens}
  const int e = ti.x, row_start = ti.y, ntok = ti.z;
  const int na = (ntok + 15) >> 4;  // active 16-token sub-tiles
  const int nb = a.nb, K = nb * 32;
  const int nchunks = (nb + 3) >> 2;
  const int grow = stripe * kPrefillRows + wave * (16 * RT);  // first row of this wave
  const int rt_active = max(0, min(RT, (a.R - grow) >> 4));
  const bool busy = rt_active > 0;  // wave-uniform
  const WBuf wb = expert_weights<TILED>(a, e);
  const uint32_t row_bytes = uint32_t(K) * EB;
  const rsrc_t bsrc = act_rows(a, PHASE, row_start, ntok, row_bytes);

  // bias of this lane's 4 output rows per row tile (bf16: the parameters
  // share the activations' dtype), fetched early as one 8-byte load each
  // (raw bits here; widened only in the epilogue so nothing waits on them)
  uint2 biasq[RT];
  {
    const rsrc_t br = make_rsrc(static_cast<const uint16_t*>(a.bias) + int64_t(e) * a.R, uint32_t(a.R) * 2u);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r0 = grow + 16 * rt + 4 * g;
      biasq[rt] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(br, r0 < a.R ? uint32_t(r0) * 2u : kOOB, 0, 0));
    }
  }

  // A DMA: each wave carries its own RT row tiles; lane i carries row
  // (i >> 2) of the tile, block slot i & 3.
  const int a_r = lane >> 2;
  const int a_blk = (lane & 3) ^ ((a_r >> 2) & 3);
  // B DMA: the 128 tokens are NBL loads of TPL tokens; wave w carries loads
  // BLOADS*w .. BLOADS*w + BLOADS-1; lane i carries token TPL*load + i/PPR,
  // piece slot i%PPR.
  uint32_t boff[BLOADS];
  int bpiece[BLOADS];
#pragma unroll
  for (int jj = 0; jj < BLOADS; ++jj) {
    const int tok = TPL * (BLOADS * wave + jj) + lane / PPR;
    const int slot = lane % PPR;
    const int p = ACT == ACT_BF16 ? bf16_piece_pos(tok, slot) : (slot ^ ((tok >> 1) & 7));
    bpiece[jj] = p;
    const uint32_t r = act_row_offset(a, PHASE, row_start, tok, ntok, row_bytes);
    boff[jj] = r == kOOB ? kOOB : r + uint32_t(16 * p);
  }
  const int t0 = grow >> 4;  // first row tile of this wave
  uint32_t sw[S][SLOADS];    // scale dwords per stage

  auto issue = [&](int c, auto stc, uint32_t* swd) __attribute__((always_inline)) {
    uint8_t* sta = stage_a(stc);
    uint8_t* stb = stage_b(stc);
    if constexpr (TILED) {
      // one contiguous 1 KB piece per row tile, already in LDS order, and
      // one scale dword per lane covering the wave's row tiles
      const bool cok = c < wb.nc;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const bool ok = cok && t0 + rt < wb.rt4;
        dma16(wb.blk, ok ? uint32_t(((t0 + rt) * wb.nc + c) * 1024 + lane * 16) : kOOB,
              sta + (wave * RT + rt) * 1024);
      }
      const bool sok = cok && t0 < wb.rt4;
      swd[0] = buf_load_b32(wb.sc, sok ? uint32_t(((t0 >> 2) * wb.nc + c) * 256 + lane * 4) : kOOB);
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int row = grow + 16 * rt + a_r;
        const int blk = 4 * c + a_blk;
        const bool ok = row < a.R && blk < nb;
        dma16(wb.blk, ok ? uint32_t(row * nb + blk) * 16u : kOOB, sta + (wave * RT + rt) * 1024);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int row = grow + 16 * rt + r16;
        const int blk = 4 * c + g;
        const bool ok = row < a.R && blk < nb;
        swd[rt] = buf_load_b32(wb.sc, ok ? (uint32_t(row * nb + blk) & ~3u) : kOOB);
      }
    }
#pragma unroll
    for (int jj = 0; jj < BLOADS; ++jj) {
      const bool kok = 128 * c + bpiece[jj] * (16 / EB) < K;
      dma16(bsrc, oob_add(boff[jj], kok ? uint32_t(c) * KB : kOOB), stb + (BLOADS * wave + jj) * 1024);
    }
  };

  // Barrier between chunks.  The empty asm statements keep the compiler
  // from moving LDS reads across it; the DMA of the chunk about to be read
  // was waited for just before (its own vmcnt), so no other wait is needed.
  auto barrier = [&]() __attribute__((always_inline)) {
    order_point();
    __builtin_amdgcn_s_barrier();
    order_point();
  };

  auto main_loop = [&](auto ntc) __attribute__((always_inline)) {
    constexpr int NA = decltype(ntc)::value;  // 1 .. 8 active sub-tiles
    f32x4_t acc[RT][NA];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NA; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](auto stc, const uint32_t* swd, int c) __attribute__((always_inline)) {
      if (busy) {
        const uint8_t* sa = stage_a(stc) + wave * RT * 1024;
        const uint8_t* sb = stage_b(stc);
        uint4 aq[RT];
        uint32_t ascb[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          aq[rt] = *reinterpret_cast<const uint4*>(sa + rt * 1024 + piece_slot(r16, g) * 16);
          if constexpr (TILED) {
            ascb[rt] = (swd[0] >> (((t0 + rt) & 3) * 8)) & 0xFFu;
          } else {
            const uint32_t o = uint32_t((grow + 16 * rt + r16) * nb + 4 * c + g);
            ascb[rt] = (swd[rt] >> ((o & 3u) * 8u)) & 0xFFu;
          }
        }
        if constexpr (ACT == ACT_BF16) {
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            bf16x8_t b[NA];
#pragma unroll
            for (int nt = 0; nt < NA; ++nt)
              b[nt] = *reinterpret_cast<const bf16x8_t*>(sb + ((nt * 16 + r16) * 16 + bf16_piece_pos(r16, 4 * g + st)) * 16);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              const bf16x8_t av = fp4x8_to_bf16x8(dword(aq[rt], st), e8m0_as_scale_operand(ascb[rt]));
#pragma unroll
              for (int nt = 0; nt < NA; ++nt)
                acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[nt], acc[rt][nt], 0, 0, 0);
            }
          }
        } else {
          i32x8_t b[NA];
          const int sw8 = (r16 >> 1) & 7;
#pragma unroll
          for (int nt = 0; nt < NA; ++nt) {
            const uint8_t* rowp = sb + (nt * 16 + r16) * 128;
            const uint4 p0 = *reinterpret_cast<const uint4*>(rowp + (g ^ sw8) * 16);
            const uint4 p1 = *reinterpret_cast<const uint4*>(rowp + ((4 + g) ^ sw8) * 16);
            b[nt] = i32x8_t{int(p0.x), int(p0.y), int(p0.z), int(p0.w), int(p1.x), int(p1.y), int(p1.z), int(p1.w)};
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const i32x8_t av = i32x8_t{int(aq[rt].x), int(aq[rt].y), int(aq[rt].z), int(aq[rt].w), 0, 0, 0, 0};
#pragma unroll
            for (int nt = 0; nt < NA; ++nt)
              acc[rt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b[nt], acc[rt][nt], 4, 0, 0,
                                                                             int(ascb[rt]), 0, 127);
          }
        }
      }
    };

    // prologue: chunks 0 .. S-2 in flight, issued in chunk order
    order_point();
    issue(0, IC<0>{}, sw[0]);
    order_point();
    if constexpr (S > 2) issue(1, IC<1>{}, sw[1]);
    order_point();
    if constexpr (S > 3) issue(2, IC<2>{}, sw[2]);
    order_point();
    if constexpr (S > 4) issue(3, IC<3>{}, sw[3]);
    order_point();

    // iteration c: wait for chunk c, barrier, refill the stage of chunk c-1
    // with chunk c+S-1, compute chunk c.  Every iteration issues the same
    // loads (chunks past the end read as zeros), so the wait count is fixed.
    auto iteration = [&](int c, auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;  // c % S
      wait_vmcnt<(S - 2) * LOADS>();
      barrier();
      issue(c + S - 1, IC<(u + S - 1) % S>{}, sw[(u + S - 1) % S]);
      order_point();
      compute(IC<u>{}, sw[u], c);
    };
    int c0 = 0;
    for (; c0 + S <= nchunks; c0 += S) {
      iteration(c0 + 0, IC<0>{});
      iteration(c0 + 1, IC<1>{});
      if constexpr (S > 2) iteration(c0 + 2, IC<2 % S>{});
      if constexpr (S > 3) iteration(c0 + 3, IC<3 % S>{});
      if constexpr (S > 4) iteration(c0 + 4, IC<4 % S>{});
    }
    if (c0 + 0 < nchunks) iteration(c0 + 0, IC<0>{});
    if (c0 + 1 < nchunks) iteration(c0 + 1, IC<1 % S>{});
    if constexpr (S > 3) if (c0 + 2 < nchunks) iteration(c0 + 2, IC<2 % S>{});
    if constexpr (S > 4) if (c0 + 3 < nchunks) iteration(c0 + 3, IC<3 % S>{});

    {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (rt < rt_active) {
#pragma unroll
          for (int nt = 0; nt < NA; ++nt) {
            const int j = nt * 16 + r16;
            if (j < ntok) {
              const f32x4_t v = acc[rt][nt];
              const uint2 q = biasq[rt];
              store_rows_biased<ACT, PHASE>(a, grow + 16 * rt + 4 * g, row_start + j,
                                            v[0] * a.acc_scale + __uint_as_float(q.x << 16),
                                            v[1] * a.acc_scale + __uint_as_float(q.x & 0xFFFF0000u),
                                            v[2] * a.acc_scale + __uint_as_float(q.y << 16),
                                            v[3] * a.acc_scale + __uint_as_float(q.y & 0xFFFF0000u));
            }
          }
        }
      }
    }
  };
  // the branches run the same loads and barriers; only the MFMA count differs
  switch (na) {
    case 1: main_loop(IC<1>{}); break;
    case 2: main_loop(IC<2>{}); break;
    case 3: main_loop(IC<3>{}); break;
    case 4: main_loop(IC<4>{}); break;
    case 5: main_loop(IC<5>{}); break;
    case 6: main_loop(IC<6>{}); break;
    case 7: main_loop(IC<7>{}); break;
    default: main_loop(IC<8>{}); break;
  }
}

// =====================================================================
// Prefill-shaped GEMM on the tiled weight order.
//
// Workgroup tile = kTiledRows weight rows x 128 tokens of one expert, K in
// 128-wide chunks, one wave per 64 rows (4 row tiles, one scale group) x
// all 128 tokens.  A wave's weight rows are its own, so they skip LDS: each
// chunk's four 1 KB pieces (already in MFMA lane order) and its scale dword
// load straight into registers.  Only the token tile, which all waves read,
// goes through LDS (buffer-to-LDS DMA) in an S-stage ring: S-1 chunks of
// weights and tokens stay in flight while one is computed, and one barrier
// per chunk publishes a landed stage and frees the one computed last.
// 256-row workgroups (4 waves, 64 KB of LDS) run two per CU: each one's
// per-chunk barrier and refill bubble is covered by the other's MFMAs,
// which outweighs the doubled token-tile reads from L2 (measured against
// one 512-row, three-stage workgroup per CU).
// =====================================================================

constexpr int kTiledWaves = kTiledRows / 64;
constexpr int kTiledThreads = 64 * kTiledWaves;

// LDS stages of the token tile for bf16 and FP8 activations (build-time
// knobs for sweeps; registers, not LDS, bound them at this tile size).
#ifndef MXMOE_PREFILL_TILED_STAGES
#define MXMOE_PREFILL_TILED_STAGES 2
#endif
#ifndef MXMOE_PREFILL_TILED_STAGES_FP8
#define MXMOE_PREFILL_TILED_STAGES_FP8 2
#endif

// Item records per workgroup from which a tiled prefill launch goes
// persistent.
#ifndef MXMOE_PERSIST_MIN
#define MXMOE_PERSIST_MIN 4
#endif
constexpr int kPersistMin = MXMOE_PERSIST_MIN;

// The kernel's GemmArgs argument (the first in its argument segment),
// loaded through a pointer that is opaque to the optimiser.
typedef const __attribute__((address_space(4))) GemmArgs* kernarg_args_t;
template <bool OPAQUE>
__device__ __forceinline__ GemmArgs item_args(const GemmArgs& args) {
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (OPAQUE) {
    kernarg_args_t p = (kernarg_args_t)__builtin_amdgcn_kernarg_segment_ptr();
    __asm__ __volatile__("" : "+s"(p));
    return *p;
  }
#endif
  return args;
}

// PERSIST: a persistent launch (below); a.item_head is set exactly then.
template <int ACT, int PHASE, bool PERSIST>
__global__ __launch_bounds__(kTiledThreads, 512 / kTiledThreads) void gemm_prefill_tiled_kernel(GemmArgs args) {
  static_assert(ACT == ACT_BF16 || ACT == ACT_FP8 || ACT == ACT_W8A8 || ACT == ACT_INT8,
                "prefill path takes bf16, fp8 or int8 activations");
  static_assert(ACT != ACT_W8A8 || PHASE == 1, "FP8 weights: dense layer epilogue only");
  static_assert(kPrefillTokens == 128, "eight 16-token sub-tiles per tile");
  static_assert(kTiledRows % 64 == 0, "waves of 4 row tiles: one scale group per wave");
  constexpr bool W8 = ACT == ACT_W8A8 || ACT == ACT_INT8;  // 8-bit weights (32 bytes per lane per chunk)
  constexpr bool I8 = ACT == ACT_INT8;  // int8 x int8 -> int32, scales in the epilogue
  constexpr int RT = 4, S = ACT == ACT_BF16 ? MXMOE_PREFILL_TILED_STAGES : MXMOE_PREFILL_TILED_STAGES_FP8;
  constexpr int EB = ACT == ACT_BF16 ? 2 : 1;
  constexpr int KB = 128 * EB;                  // bytes of one token row per chunk
  constexpr int PPR = KB / 16;                  // 16-byte pieces per token row (16 or 8)
  constexpr int TPL = 64 / PPR;                 // tokens per 1 KB B load (4 or 8)
  constexpr int NBL = 128 / TPL;                // B loads per chunk (32 or 16)
  constexpr int BLOADS = NBL / kTiledWaves;     // B loads per wave per chunk
  static_assert(NBL % kTiledWaves == 0, "B loads split evenly over the waves");
  constexpr int B_BYTES = 128 * KB;             // B stage
  constexpr int LOADS = RT + 1 + BLOADS;        // VMEM instructions per wave per chunk
  static_assert(S >= 2 && S <= 4, "2..4 stages");
  static_assert((S - 2) * LOADS < 64, "vmcnt range");
  __shared__ __align__(16) uint8_t sB0[B_BYTES], sB1[B_BYTES], sB2[S > 2 ? B_BYTES : 16], sB3[S > 3 ? B_BYTES : 16];
  auto stage_b = [&](auto uc) -> uint8_t* {
    constexpr int u = decltype(uc)::value;
    if constexpr (u == 0) return sB0;
    else if constexpr (u == 1) return sB1;
    else if constexpr (u == 2) return sB2;
    else return sB3;
  };
  // bf16 tiles of at most 64 tokens run a deeper ring in the same LDS: four
  // stages of 64 token rows (16 KB) in sB0 and sB1, so three chunks are in
  // flight while one is computed.  A short tile's few MFMAs cannot cover a
  // chunk's load latency with one chunk ahead.
  constexpr int SS = 4;                          // stages of a small tile
  constexpr int SBLOADS = BLOADS / 2;            // its B loads per wave per chunk
  static_assert(SS * (B_BYTES / 2) <= 2 * B_BYTES, "small stages fit in sB0 and sB1");
  static_assert((SS - 2) * (RT + 1 + SBLOADS) < 64, "vmcnt range");
  auto stage_small = [&](auto uc) -> uint8_t* {
    constexpr int u = decltype(uc)::value;
    return (u < 2 ? sB0 : sB1) + (u & 1) * (B_BYTES / 2);
  };

  // Work items (expert, row stripe, token tile), split over the XCDs as
  // xcd_split.h describes.  A persistent launch (a.item_head set, with the
  // grouping's item records) holds two workgroups per CU; each takes items
  // one after another from its XCD's record list through a device-scope
  // counter, so no slot waits for the dispatcher between items.  (Taking
  // items from the other XCDs' lists once its own is exhausted measured
  // slower: their experts' weights miss in this XCD's L2.)  Otherwise each
  // workgroup runs one item: its record, or one it resolves itself (one
  // record load instead of the scan and searches below).
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3, G = gridDim.x >> 3;
  __shared__ int4 s_rec;
  for (bool first_item = true;; first_item = false) {
    // The arguments and the lane's constants are produced anew for each
    // item (the arguments re-read from the kernel's argument segment through
    // a pointer the compiler cannot follow across items): the values derived
    // from them then live inside one item instead of being hoisted out of
    // the loop and held, and spilled, across all of it.
    const GemmArgs a = item_args<PERSIST>(args);
    uint32_t tid = threadIdx.x;
    if constexpr (PERSIST) hold(tid);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r16 = lane & 15;
    const int nstripes = (a.R + kTiledRows - 1) / kTiledRows;
    int e, row_start, ntok, stripe;
    if constexpr (PERSIST) {
      if (threadIdx.x == 0) {
        // this item's position in the XCD's list: idx for the first one (the
        // counter starts past the G of them), then the counter's next
        const uint32_t gr = uint32_t(tiled_prefill_blocks(a.R, a.max_tiles) >> 3);  // records per XCD
        const uint32_t q = first_item ? uint32_t(idx) : add_dev(a.item_head + xcd, 1u);
        s_rec = q < gr ? a.blk_rec[8 * q + xcd] : make_int4(0, 0, 0, 0);
      }
      // also the barrier between this workgroup's items: the new item's DMAs
      // reuse LDS the previous one read
      __syncthreads();
      const int4 r = s_rec;
      ntok = __builtin_amdgcn_readfirstlane(r.z);
      if (ntok == 0) return;  // the list is exhausted: uniform per workgroup
      e = __builtin_amdgcn_readfirstlane(r.x);
      row_start = __builtin_amdgcn_readfirstlane(r.y);
      stripe = __builtin_amdgcn_readfirstlane(r.w);
    } else if (a.blk_rec) {
      const int4 r = a.blk_rec[blockIdx.x];
      hold_uniform(r);
      if (r.z == 0) return;  // no item: uniform per workgroup
      e = r.x;
      row_start = r.y;
      ntok = r.z;
      stripe = r.w;
    } else {
      const int nvalid = a.tile_off[a.E] * nstripes;
      __shared__ int s_toff[257];  // E <= 256, checked on the host
      __shared__ int s_woff[257];  // prefix of the experts' per-stripe costs
      __shared__ int s_wtot[kTiledWaves];
      static_assert(kTiledThreads >= 256, "one thread per expert");
      int tile;
      if (a.E == 1) {
        // One weight matrix (a dense linear): stripe fastest instead, so each
        // XCD reads an eighth of the activations, which outweigh the 4- or
        // 8-bit weights, rather than all of them.  Its tiles are full but the
        // last, so equal item counts are equal work.
        const int per_xcd = (nvalid + 7) >> 3;
        const int item = xcd * per_xcd + idx;
        if (idx >= per_xcd || item >= nvalid) return;  // uniform per workgroup
        tile = item / nstripes;
        stripe = item - tile * nstripes;
      } else {
        // per-stripe costs of the experts: block-wide scan
        const int t = threadIdx.x;
        const int c = t < a.E ? expert_stripe_cost(a.offsets[t + 1] - a.offsets[t]) : 0;
        for (int i = t; i <= a.E; i += kTiledThreads) s_toff[i] = a.tile_off[i];
        int x = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(x, off);
          if (lane >= off) x += y;
        }
        if (lane == 63) s_wtot[wave] = x;
        __syncthreads();
        for (int w = 0; w < wave; ++w) x += s_wtot[w];
        if (t < a.E) s_woff[t + 1] = x;
        if (t == 0) s_woff[0] = 0;
        __syncthreads();
        int bx[9];
        xcd_bounds(s_woff, s_toff, a.E, nstripes, G, nvalid, lane, bx);
        int first = bx[0], last = bx[1];
#pragma unroll
        for (int xx = 1; xx < 8; ++xx)
          if (xcd == xx) {
            first = bx[xx];
            last = bx[xx + 1];
          }
        const int item = first + idx;
        if (item >= last) return;  // uniform per workgroup
        // Expert e owns items [tile_off[e], tile_off[e+1]) * nstripes
        int lo = 0, hi = a.E;  // s_toff[lo] * nstripes <= item < s_toff[hi] * nstripes
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_toff[mid] * nstripes <= item) lo = mid;
          else hi = mid;
        }
        const int nt_e = s_toff[lo + 1] - s_toff[lo];
        const int local = item - s_toff[lo] * nstripes;
        stripe = local / nt_e;
        tile = s_toff[lo] + (local - stripe * nt_e);
      }
      const int4 ti = a.tiles[tile];  // {expert, first sorted row, tokens}
      e = ti.x;
      row_start = ti.y;
      ntok = ti.z;
    }
    const int na = (ntok + 15) >> 4;  // active 16-token sub-tiles
    const int nb = a.nb, K = nb * 32;
    const WBuf wb = W8 ? byte_weights(a, e) : expert_weights<true>(a, e);
    const int nc = wb.nc;
    const int grow = stripe * kTiledRows + wave * (16 * RT);  // first row of this wave
    const int t0 = grow >> 4;                                   // its first row tile (a scale group start)
    const int rt_active = max(0, min(RT, (a.R - grow) >> 4));
    const bool busy = rt_active > 0;  // wave-uniform
    const bool wok = t0 < wb.rt4;
    const uint32_t row_bytes = uint32_t(K) * EB;
    const rsrc_t bsrc = act_rows(a, PHASE, row_start, ntok, row_bytes);
    const uint32_t aslot = uint32_t(piece_slot(r16, g)) * 16u;

    // The workgroup's kTiledRows bias values go to LDS by one DMA of wave 0,
    // issued before every chunk load: the first chunk's wait covers it and the
    // first barrier publishes it, so the epilogue finds it without a memory
    // round trip (lanes past the stripe read zeros).
    __shared__ __align__(16) uint8_t sBias[1024];
    static_assert(kTiledRows * 2 <= 1024, "one DMA covers the stripe's bias");
    if (wave == 0) {
      const rsrc_t br = make_rsrc(static_cast<const uint16_t*>(a.bias) + int64_t(e) * a.R, uint32_t(a.R) * 2u);
      const int r = stripe * kTiledRows + 8 * lane;
      dma16(br, (8 * lane < kTiledRows && r < a.R) ? uint32_t(r) * 2u : kOOB, sBias);
    }
    auto barrier = [&]() __attribute__((always_inline)) {
      order_point();
      __builtin_amdgcn_s_barrier();
      order_point();
    };

    auto main_loop = [&](auto ntc, auto smc) __attribute__((always_inline)) {
      constexpr int NA = decltype(ntc)::value;  // 1 .. 8 active sub-tiles
      constexpr bool SMALL = decltype(smc)::value != 0;
      constexpr int SX = SMALL ? SS : S;           // stages of the ring
      // B loads per wave per chunk: only the tile's 16 NA active token rows
      // (loads past ntok would read zeros), spread over the waves
      constexpr int BL = (16 * NA + TPL * kTiledWaves - 1) / (TPL * kTiledWaves);
      static_assert(BL <= (SMALL ? SBLOADS : BLOADS), "the active rows fit the stage");
      constexpr int LD = (W8 ? 2 * RT : RT + 1) + BL;  // VMEM instructions per wave per chunk
      static_assert(!SMALL || (ACT == ACT_BF16 && NA <= 4), "small ring: bf16 tiles of <= 64 tokens");
      auto stage = [&](auto uc) -> uint8_t* {
        if constexpr (SMALL) return stage_small(uc);
        else return stage_b(uc);
      };

      // B DMA: the tile's first 16 NA token rows are loads of TPL tokens;
      // wave w carries loads BL*w .. BL*w + BL-1; lane i carries token
      // TPL*load + i/PPR, piece slot i%PPR, XOR-swizzled by token
      // (bf16_piece_pos for bf16).  (clast: the last chunk whose part of this
      // piece lies inside K)
      uint32_t boff[BL];
      int clast[BL];
#pragma unroll
      for (int jj = 0; jj < BL; ++jj) {
        const int tok = TPL * (BL * wave + jj) + lane / PPR;
        const int slot = lane % PPR;
        const int p = ACT == ACT_BF16 ? bf16_piece_pos(tok, slot) : (slot ^ ((tok >> 1) & 7));
        clast[jj] = (K - 1 - p * (16 / EB)) >> 7;
        const uint32_t r = act_row_offset(a, PHASE, row_start, tok, ntok, row_bytes);
        boff[jj] = r == kOOB ? kOOB : r + uint32_t(16 * p);
      }
      uint4 aq[SX][RT];   // weight pieces per stage
      uint4 aq2[W8 ? SX : 1][RT];  // FP8 weights: the second 16 bytes of a lane's piece
      uint32_t sw[SX];    // scale dword per stage

      // weights and scales of chunk c into register stage u
      auto issue_w = [&](int c, auto stc) __attribute__((always_inline)) {
        constexpr int u = decltype(stc)::value;
        const bool cok = c < nc && wok;
        if constexpr (W8) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const uint32_t o = cok ? uint32_t(((t0 + rt) * nc + c) * 2048 + lane * 32) : kOOB;
            aq[u][rt] = buf_load_b128(wb.blk, o);
            aq2[u][rt] = buf_load_b128(wb.blk, oob_add(o, 16u));
          }
          sw[u] = 0;
        } else {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            aq[u][rt] = buf_load_b128(wb.blk, cok ? uint32_t(((t0 + rt) * nc + c) * 1024) + aslot : kOOB);
          sw[u] = buf_load_b32(wb.sc, cok ? uint32_t(((t0 >> 2) * nc + c) * 256 + lane * 4) : kOOB);
        }
      };
      // tokens of chunk c into LDS stage u
      auto issue_b = [&](int c, auto stc) __attribute__((always_inline)) {
        uint8_t* stb = stage(stc);
#pragma unroll
        for (int jj = 0; jj < BL; ++jj) {
          const bool kok = c <= clast[jj];
          dma16(bsrc, oob_add(boff[jj], kok ? uint32_t(c) * KB : kOOB), stb + (BL * wave + jj) * 1024);
        }
      };

      f32x4_t acc[RT][NA];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NA; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      // compute stage u; mid() (the next chunk's token DMA) runs once, halfway
      // through the MFMA steps, so the wave's loads do not all leave in one
      // burst after the barrier (measured 1-3% faster on the full tiles)
      auto compute = [&](auto stc, auto mid) __attribute__((always_inline)) {
        constexpr int u = decltype(stc)::value;
        if (!busy) mid();
        if (busy) {
          const uint8_t* sb = stage(stc);
          uint32_t ascb[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) ascb[rt] = (sw[u] >> (((t0 + rt) & 3) * 8)) & 0xFFu;
          if constexpr (ACT == ACT_BF16) {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              if (st == 2) mid();
              bf16x8_t b[NA];
#pragma unroll
              for (int nt = 0; nt < NA; ++nt)
                b[nt] = *reinterpret_cast<const bf16x8_t*>(
                    sb + ((nt * 16 + r16) * 16 + bf16_piece_pos(r16, 4 * g + st)) * 16);
#pragma unroll
              for (int rt = 0; rt < RT; ++rt) {
                const bf16x8_t av = fp4x8_to_bf16x8(dword(aq[u][rt], st), e8m0_as_scale_operand(ascb[rt]));
#pragma unroll
                for (int nt = 0; nt < NA; ++nt)
                  acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[nt], acc[rt][nt], 0, 0, 0);
              }
            }
          } else {
            // token fragments double-buffered by hand (sub-tile nt+1 is read
            // before sub-tile nt's MFMAs; the order points keep the compiler
            // from hoisting all of them, which would cost 8 registers each)
            const int sw8 = (r16 >> 1) & 7;
            auto load_b = [&](int nt) __attribute__((always_inline)) {
              const uint8_t* rowp = sb + (nt * 16 + r16) * 128;
              const uint4 p0 = *reinterpret_cast<const uint4*>(rowp + (g ^ sw8) * 16);
              const uint4 p1 = *reinterpret_cast<const uint4*>(rowp + ((4 + g) ^ sw8) * 16);
              return i32x8_t{int(p0.x), int(p0.y), int(p0.z), int(p0.w), int(p1.x), int(p1.y), int(p1.z), int(p1.w)};
            };
            i32x8_t av[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              const uint4 q = aq[u][rt];
              if constexpr (W8) {
                const uint4 q2 = aq2[u][rt];
                av[rt] = i32x8_t{int(q.x), int(q.y), int(q.z), int(q.w), int(q2.x), int(q2.y), int(q2.z), int(q2.w)};
              } else {
                av[rt] = i32x8_t{int(q.x), int(q.y), int(q.z), int(q.w), 0, 0, 0, 0};
              }
            }
            i32x8_t bcur = load_b(0);
#pragma unroll
            for (int nt = 0; nt < NA; ++nt) {
              if (nt == NA / 2) mid();
              i32x8_t bnext = bcur;
              if (nt + 1 < NA) bnext = load_b(nt + 1);
              order_point();
#pragma unroll
              for (int rt = 0; rt < RT; ++rt) {
                if constexpr (I8) {
                  // two K=64 halves (dwords 0-3, then 4-7 of both operands);
                  // the int32 sums live in the float accumulator registers
                  typedef int i32x4_t __attribute__((ext_vector_type(4)));
                  i32x4_t c = __builtin_bit_cast(i32x4_t, acc[rt][nt]);
                  c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_shufflevector(av[rt], av[rt], 0, 1, 2, 3),
                                                           __builtin_shufflevector(bcur, bcur, 0, 1, 2, 3), c, 0, 0, 0);
                  c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_shufflevector(av[rt], av[rt], 4, 5, 6, 7),
                                                           __builtin_shufflevector(bcur, bcur, 4, 5, 6, 7), c, 0, 0, 0);
                  acc[rt][nt] = __builtin_bit_cast(f32x4_t, c);
                } else {
                  acc[rt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                      av[rt], bcur, acc[rt][nt], W8 ? 0 : 4, 0, 0, W8 ? 127 : int(ascb[rt]), 0, 127);
                }
              }
              bcur = bnext;
            }
          }
        }
      };

      // prologue: chunks 0 .. SX-2 in flight, issued in chunk order
      auto issue = [&](int c, auto stc) __attribute__((always_inline)) {
        issue_w(c, stc);
        issue_b(c, stc);
      };
      order_point();
      issue(0, IC<0>{});
      order_point();
      if constexpr (SX > 2) { issue(1, IC<1>{}); order_point(); }
      if constexpr (SX > 3) { issue(2, IC<2>{}); order_point(); }

      // iteration c: wait for chunk c, barrier (its tokens have landed for
      // every wave, and chunk c-1's stage is free), refill that stage with
      // chunk c+S-1 (weights now, tokens from inside compute), compute chunk
      // c.  Every iteration issues the same loads (chunks past the end read
      // zeros), weights before tokens, so the wait count is fixed.
      auto iteration = [&](int c, auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;  // c % SX
        wait_vmcnt<(SX - 2) * LD>();
        barrier();
        issue_w(c + SX - 1, IC<(u + SX - 1) % SX>{});
        order_point();
        compute(IC<u>{}, [&]() __attribute__((always_inline)) {
          order_point();
          issue_b(c + SX - 1, IC<(u + SX - 1) % SX>{});
          order_point();
        });
      };
      int c0 = 0;
      for (; c0 + SX <= nc; c0 += SX) {
        iteration(c0 + 0, IC<0>{});
        iteration(c0 + 1, IC<1>{});
        if constexpr (SX > 2) iteration(c0 + 2, IC<2 % SX>{});
        if constexpr (SX > 3) iteration(c0 + 3, IC<3 % SX>{});
      }
      if (c0 + 0 < nc) iteration(c0 + 0, IC<0>{});
      if (c0 + 1 < nc) iteration(c0 + 1, IC<1 % SX>{});
      if constexpr (SX > 3) if (c0 + 2 < nc) iteration(c0 + 2, IC<2 % SX>{});
      wait_vmcnt<0>();
      // Never true (slot counts are non-negative).  It keeps every weight
      // prefetch live: the vmcnt waits count loads, so none may be dropped as
      // dead even when its chunk lies past the end.
      if (a.n_slots < 0) {
        uint32_t x = 0;
#pragma unroll
        for (int d = 0; d < SX; ++d) x ^= aq[d][0].x ^ aq[d][1].y ^ aq[d][2].z ^ aq[d][3].w ^ sw[d];
        if constexpr (W8) {
#pragma unroll
          for (int d = 0; d < SX; ++d) x ^= aq2[d][0].x ^ aq2[d][1].y ^ aq2[d][2].z ^ aq2[d][3].w;
        }
        static_cast<uint32_t*>(a.out)[0] = x;
      }

#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (rt < rt_active) {
          // bias of this lane's 4 output rows (raw bf16 bits)
          const uint2 q = *reinterpret_cast<const uint2*>(sBias + 2 * (wave * 16 * RT + 16 * rt + 4 * g));
          float4 rs = make_float4(1.f, 1.f, 1.f, 1.f);  // int8: weight scales of the 4 rows
          if constexpr (I8)
            rs = *reinterpret_cast<const float4*>(a.row_scale + int64_t(e) * a.R + grow + 16 * rt + 4 * g);
#pragma unroll
          for (int nt = 0; nt < NA; ++nt) {
            const int j = nt * 16 + r16;
            if (j < ntok) {
              f32x4_t v = acc[rt][nt];
              if constexpr (I8) {
                // exact int32 sums -> fp32, times the row's and the token's
                // scales (the whole vector is reinterpreted: a bit cast of one
                // element of a vector value reads element 0 with this compiler)
                typedef int i32x4_t __attribute__((ext_vector_type(4)));
                const i32x4_t iv = __builtin_bit_cast(i32x4_t, acc[rt][nt]);
                const int p = row_start + j;
                const float ts = a.tok_scale[PHASE == 0 ? a.sorted_tok[p] : p];
                v = f32x4_t{float(iv[0]) * rs.x * ts, float(iv[1]) * rs.y * ts, float(iv[2]) * rs.z * ts,
                            float(iv[3]) * rs.w * ts};
              }
              store_rows_biased<ACT, PHASE>(a, grow + 16 * rt + 4 * g, row_start + j,
                                            v[0] * a.acc_scale + __uint_as_float(q.x << 16),
                                            v[1] * a.acc_scale + __uint_as_float(q.x & 0xFFFF0000u),
                                            v[2] * a.acc_scale + __uint_as_float(q.y << 16),
                                            v[3] * a.acc_scale + __uint_as_float(q.y & 0xFFFF0000u));
            }
          }
        }
      }
    };
    constexpr int SM = ACT == ACT_BF16 ? 1 : 0;  // tiles of <= 64 tokens take the small ring
    switch (na) {
      case 1: main_loop(IC<1>{}, IC<SM>{}); break;
      case 2: main_loop(IC<2>{}, IC<SM>{}); break;
      case 3: main_loop(IC<3>{}, IC<SM>{}); break;
      case 4: main_loop(IC<4>{}, IC<SM>{}); break;
      case 5: main_loop(IC<5>{}, IC<0>{}); break;
      case 6: main_loop(IC<6>{}, IC<0>{}); break;
      case 7: main_loop(IC<7>{}, IC<0>{}); break;
      default: main_loop(IC<8>{}, IC<0>{}); break;
    }
    if constexpr (!PERSIST) return;  // one item per workgroup
  }  // items
}

// The folded combine of row group q (64 rows of H) once every active
// expert's Y rows of the group are in: out[t] = sum_j w[t, j] * Y[pos[t, j]]
// over j = 0 .. k-1 in that order, in fp32 (the arithmetic of
// combine_kernel), for all T tokens; 8 threads per token, 8 columns each.
__device__ void combine_group(const GemmArgs& a, int q) {
  const int H = a.R, k = a.top_k;
  const int c0 = 64 * q;
  const rsrc_t ys = make_rsrc(a.out, uint32_t(a.n_slots) * uint32_t(H) * 2u);
  for (int i = threadIdx.x; i < a.T * 8; i += blockDim.x) {
    const int t = i >> 3, c = c0 + 8 * (i & 7);
    if (c >= H) continue;
    int64_t row[MAX_TOPK_DEV];
    float w[MAX_TOPK_DEV];
#pragma unroll
    for (int j = 0; j < MAX_TOPK_DEV; ++j) {
      row[j] = j < k ? a.pos[int64_t(t) * k + j] : 0;
      w[j] = j < k ? a.wts[int64_t(t) * k + j] : 0.f;
    }
    uint4 y[MAX_TOPK_DEV];
#pragma unroll
    for (int j = 0; j < MAX_TOPK_DEV; ++j)
      y[j] = j < k ? buf_load_dev_b128(ys, uint32_t((row[j] * H + c) * 2)) : make_uint4(0, 0, 0, 0);
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < MAX_TOPK_DEV; ++j) {
      if (j < k) {
        const uint32_t yw[4] = {y[j].x, y[j].y, y[j].z, y[j].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          s[2 * m] += w[j] * __uint_as_float(yw[m] << 16);
          s[2 * m + 1] += w[j] * __uint_as_float(yw[m] & 0xFFFF0000u);
        }
      }
    }
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.cmb_out) + int64_t(t) * H + c) =
        make_uint4(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]), pack_bf16x2(s[4], s[5]), pack_bf16x2(s[6], s[7]));
  }
}

// Decode-shaped GEMM on the tiled weight order (bf16 and FP8 activations):
// one workgroup per (64-row group, active expert slot); the tile itself is
// decode_tile (decode_tile.h).  With the combine folded in (cmb_out set),
// the gate_up launch clears the arrival counters and each down workgroup
// signals its row group once its Y rows are stored; the last of the
// group's rec.w workgroups forms the output rows.
// Batches up to this many tokens run the decode tile with one 16-token
// sub-tile per pass (150 registers instead of 166 for bf16 tokens); an
// expert with more than 16 tokens then takes one pass over its weights per
// 16 (sweep knob; 64 measured 8% faster than 16 on the 20b T = 64 batch,
// whose experts see 8 tokens on average).
#ifndef MXMOE_DECODE_ONE_SUBTILE
#define MXMOE_DECODE_ONE_SUBTILE 64
#endif
constexpr int kDecodeOneSubtile = MXMOE_DECODE_ONE_SUBTILE;

template <int ACT, int PHASE, int MAXNA>
__global__ __launch_bounds__(256, 2) void gemm_decode_tiled_kernel(GemmArgs a) {
  const int slot = blockIdx.y;
  if (PHASE == 0 && a.cmb_count && slot == 0 && blockIdx.x == 0)
    for (int i = threadIdx.x; i < a.n_cmb; i += blockDim.x) a.cmb_count[i] = 0;
  // one round trip: slots past the active experts hold empty records
  const int4 rec = a.active[1 + slot];
  hold_uniform(rec);
  if (rec.z == 0) return;
  __shared__ __align__(16) uint8_t lds[kDecodeTileLds];
  decode_tile<ACT, PHASE, MAXNA>(a, rec.x, blockIdx.x, rec.y, rec.z, lds);
  if (PHASE == 1 && a.cmb_out) {
    __shared__ int last;
    wait_vmcnt<0>();  // this wave's Y stores have reached the point of coherence
    __syncthreads();
    if (threadIdx.x == 0) last = add_dev(a.cmb_count + blockIdx.x, 1u) == uint32_t(rec.w - 1);
    __syncthreads();
    if (last) combine_group(a, blockIdx.x);
  }
}

template <int ACT, int PHASE, bool TILED>
static void launch_layout(const GemmArgs& a, bool prefill, hipStream_t stream) {
  if constexpr (ACT == ACT_W8A8) {  // FP8 weights: the tiled LDS-staged kernel only
    const int64_t items = tiled_prefill_blocks(a.R, a.max_tiles);
    gemm_prefill_tiled_kernel<ACT, PHASE, false><<<dim3(unsigned(items)), dim3(kTiledThreads), 0, stream>>>(a);
  } else if (prefill) {
    if constexpr (ACT != ACT_F32) {
      if constexpr (TILED) {
        // the grid the grouping's item records (GemmArgs::blk_rec) assume,
        // or the persistent grid that takes them as work lists: when the
        // records allow at least kPersistMin items per workgroup (with
        // fewer, the launch's tail outweighs the dispatch gaps saved)
        const int64_t items = tiled_prefill_blocks(a.R, a.max_tiles);
        if (a.item_head && items >= int64_t(kPersistMin) * kPersistentBlocks) {
          gemm_prefill_tiled_kernel<ACT, PHASE, true>
              <<<dim3(unsigned(kPersistentBlocks)), dim3(kTiledThreads), 0, stream>>>(a);
        } else {
          GemmArgs b = a;
          b.item_head = nullptr;
          gemm_prefill_tiled_kernel<ACT, PHASE, false><<<dim3(unsigned(items)), dim3(kTiledThreads), 0, stream>>>(b);
        }
      } else {
        const int64_t items = (int64_t(a.max_tiles) * ((a.R + kPrefillRows - 1) / kPrefillRows) + 7) / 8 * 8;
        gemm_prefill_kernel<ACT, PHASE, TILED><<<dim3(unsigned(items)), dim3(kPrefillThreads), 0, stream>>>(a);
      }
    }
  } else if constexpr (TILED && ACT != ACT_F32) {
    const unsigned gx = unsigned((a.R + 63) / 64);  // row groups
    const dim3 grid(gx, unsigned(a.max_active));
    // tokens per expert <= tokens per batch: batches of at most
    // kDecodeOneSubtile tokens never need the 32-token pass
    if (a.T <= kDecodeOneSubtile)
      gemm_decode_tiled_kernel<ACT, PHASE, 1><<<grid, dim3(256), 0, stream>>>(a);
    else
      gemm_decode_tiled_kernel<ACT, PHASE, 2><<<grid, dim3(256), 0, stream>>>(a);
  } else {
    const unsigned gx = unsigned((a.R + 16 * kDecodeRowTiles - 1) / (16 * kDecodeRowTiles));
    gemm_decode_kernel<ACT, PHASE, TILED><<<dim3(gx, unsigned(a.max_active)), dim3(256), 0, stream>>>(a);
  }
}

template <int ACT, int PHASE>
static void launch_one(const GemmArgs& a, bool prefill, hipStream_t stream) {
  if (a.tiled)
    launch_layout<ACT, PHASE, true>(a, prefill, stream);
  else
    launch_layout<ACT, PHASE, false>(a, prefill, stream);
}

hipError_t launch_moe_gemm(const GemmArgs& a, bool prefill, hipStream_t stream) {
  if (a.max_active == 0) return hipSuccess;
  if (a.act == ACT_F32 && prefill) return hipErrorInvalidValue;
  switch (a.act * 2 + a.phase) {
    case ACT_F32 * 2 + 0: launch_one<ACT_F32, 0>(a, prefill, stream); break;
    case ACT_F32 * 2 + 1: launch_one<ACT_F32, 1>(a, prefill, stream); break;
    case ACT_BF16 * 2 + 0: launch_one<ACT_BF16, 0>(a, prefill, stream); break;
    case ACT_BF16 * 2 + 1: launch_one<ACT_BF16, 1>(a, prefill, stream); break;
    case ACT_FP8 * 2 + 0: launch_one<ACT_FP8, 0>(a, prefill, stream); break;
    case ACT_FP8 * 2 + 1: launch_one<ACT_FP8, 1>(a, prefill, stream); break;
    case ACT_W8A8 * 2 + 1:
      if (!a.tiled || !prefill) return hipErrorInvalidValue;  // only the tiled LDS-staged kernel
      launch_layout<ACT_W8A8, 1, true>(a, true, stream);
      break;
    case ACT_INT8 * 2 + 0:
    case ACT_INT8 * 2 + 1:
      if (!a.tiled) return hipErrorInvalidValue;  // the 8-bit tile order only
      if (a.phase == 0) launch_layout<ACT_INT8, 0, true>(a, prefill, stream);
      else launch_layout<ACT_INT8, 1, true>(a, prefill, stream);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------- combine
//
// out_t = sum_j w[t, j] * Y[pos[t*k + j]] in the order j = 0 .. k-1 (fp32),
// one workgroup per token; each thread takes 8 columns of bf16 Y (one
// 16-byte load per row) or 4 of fp32 Y.

template <bool Y_BF16>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int CPT = Y_BF16 ? 8 : 4;  // columns per thread
  const int t = blockIdx.x;
  const int k = a.top_k;
  int64_t rows[MAX_TOPK_DEV];
  float w[MAX_TOPK_DEV];
#pragma unroll
  for (int j = 0; j < MAX_TOPK_DEV; ++j) {
    rows[j] = 0;
    w[j] = 0.f;
    if (j < k) {
      rows[j] = int64_t(a.pos[int64_t(t) * k + j]) * a.H;
      w[j] = a.wts[int64_t(t) * k + j];
    }
  }
  for (int c = threadIdx.x * CPT; c < a.H; c += 256 * CPT) {
    float s[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) s[i] = 0.f;
#pragma unroll
    for (int j = 0; j < MAX_TOPK_DEV; ++j) {
      if (j < k) {
        if constexpr (Y_BF16) {
          const uint4 y = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.Y) + rows[j] + c);
          const uint32_t yw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s[2 * i] += w[j] * __uint_as_float(yw[i] << 16);
            s[2 * i + 1] += w[j] * __uint_as_float(yw[i] & 0xFFFF0000u);
          }
        } else {
          const float4 y = *reinterpret_cast<const float4*>(static_cast<const float*>(a.Y) + rows[j] + c);
          s[0] += w[j] * y.x;
          s[1] += w[j] * y.y;
          s[2] += w[j] * y.z;
          s[3] += w[j] * y.w;
        }
      }
    }
    const int64_t o = int64_t(t) * a.H + c;
    if (a.out_bf16) {
      if constexpr (CPT == 8)
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + o) =
            make_uint4(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]), pack_bf16x2(s[4], s[5]), pack_bf16x2(s[6], s[7]));
      else
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) = make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
    } else {
#pragma unroll
      for (int i = 0; i < CPT; i += 4)
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o + i) = make_float4(s[i], s[i + 1], s[i + 2], s[i + 3]);
    }
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (a.y_bf16)
    combine_kernel<true><<<dim3(unsigned(a.T)), dim3(256), 0, stream>>>(a);
  else
    combine_kernel<false><<<dim3(unsigned(a.T)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mxmoe
