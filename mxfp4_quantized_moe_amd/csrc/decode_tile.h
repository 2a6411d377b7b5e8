// Decode-shaped tile of the expert GEMMs on the tiled weight orders, for
// gfx950: one 64-row group of one routed expert against that expert's
// tokens.  MXFP4 weights with bf16 or FP8 activations, or int8 weights (the
// 8-bit tile order) with int8 activations.
//
// Bound by streaming the routed experts' packed weights.  The workgroup's 4
// waves split the K chunks (c = wave, wave + 4, ...) and every wave covers
// all 4 row tiles, so each activation fragment it loads feeds 4 MFMAs.  Per
// chunk a wave loads 4 contiguous 1 KB weight pieces, one scale dword (the
// 4 row tiles' scale bytes of its lane) and its token fragments, and keeps D
// chunks in flight in a register ring with explicit vmcnt waits.  A pass
// covers up to 32 tokens.  Partial sums meet in LDS in a fixed wave order,
// one token sub-tile at a time, right after the wave's last chunk (the ring's
// trailing loads, all past the end, still return meanwhile).
#pragma once

#include "gemm_common.h"

namespace mxmoe {

template <int ACT, int NA>
struct DecodeStage {
  // 16-byte B loads per token sub-tile: 4 for bf16 tokens (32 values), 2
  // for FP8 or int8 codes
  static constexpr int BL = ACT == ACT_BF16 ? 4 : 2;
  uint4 aq[4];                             // MXFP4: 32 nibbles per row tile; int8: K 16g .. 16g+15
  uint4 aq2[ACT == ACT_INT8 ? 4 : 1];      // int8: K 64+16g .. 64+16g+15
  uint32_t sw;                             // MXFP4: the 4 row tiles' scale bytes
  uint4 bq[NA][BL];
};

// LDS of one decode tile: the 4 waves' partial sums of one token sub-tile,
// then one 1 KB area per wave that its bias values land in.
constexpr int kDecodeRedLds = 4 * 4 * 64 * 16;
constexpr int kDecodeTileLds = kDecodeRedLds + 4 * 1024;

// Tile (expert e, row group q) for the n_e tokens in sorted rows row_start
// .. row_start + n_e - 1.  lds: kDecodeTileLds bytes.  MAXNA: token
// sub-tiles of 16 per pass (1 or 2); batches of at most 16 tokens (no
// expert sees more) take 1, which keeps the 32-token pass and its
// registers out of the kernel.
template <int ACT, int PHASE, int MAXNA>
__device__ __forceinline__ void decode_tile(const GemmArgs& a, int e, int q, int row_start, int n_e, uint8_t* lds) {
  static_assert(ACT == ACT_BF16 || ACT == ACT_FP8 || ACT == ACT_INT8, "bf16, fp8 or int8 activations");
  static_assert(MAXNA == 1 || MAXNA == 2, "one or two token sub-tiles per pass");
  constexpr bool I8 = ACT == ACT_INT8;  // int8 x int8 -> exact int32 sums, scales in the epilogue
  // [wave][row tile][lane] of one token sub-tile
  f32x4_t (*red)[4][64] = reinterpret_cast<f32x4_t (*)[4][64]>(lds);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint8_t* sbias = lds + kDecodeRedLds + wave * 1024;
  const int g = lane >> 4, r16 = lane & 15;
  const WBuf wb = I8 ? byte_weights(a, e) : expert_weights<true>(a, e);
  const int nb = a.nb, nc = wb.nc, K = nb * 32;
  constexpr int EB = ACT == ACT_BF16 ? 2 : 1;  // bytes per B element
  const uint32_t row_bytes = uint32_t(K) * EB;
  const rsrc_t bsrc = act_rows(a, PHASE, row_start, n_e, row_bytes);
  const int t0 = 4 * q;  // first row tile of the group
  const int nj = (nc - wave + 3) >> 2;  // chunks of this wave (0 when nc <= wave)
  const uint32_t aslot = uint32_t(piece_slot(r16, g)) * 16u;
  // The bias of the wave's row tile (rows 16 (t0 + wave) .. +16, raw bf16
  // bits) goes to LDS by one DMA before any other load, so every later wait
  // covers it and no register holds it through the K loop.  Lane h < 2
  // carries rows 8h .. 8h+7.
  {
    const rsrc_t br = make_rsrc(static_cast<const uint16_t*>(a.bias) + int64_t(e) * a.R, uint32_t(a.R) * 2u);
    const int r = 16 * (t0 + wave) + 8 * lane;
    dma16(br, (lane < 2 && r < a.R) ? uint32_t(r) * 2u : kOOB, sbias);
  }

  // up to 16 * MAXNA tokens per pass over the weights (registers bound
  // the tile)
  for (int tg = 0; tg < n_e; tg += 16 * MAXNA) {
    const int nt_active = min(MAXNA, (n_e - tg + 15) >> 4);

    auto pass = [&](auto ntc) __attribute__((always_inline)) {
      constexpr int NA = decltype(ntc)::value;
      constexpr int D = NA == 1 ? 3 : 2;  // chunks in flight per wave (3 measured faster than 2 and 4)
      static_assert(D == 2 || D == 3, "ring of 2 or 3 chunks");
      using St = DecodeStage<ACT, NA>;
      constexpr int LOADS = (I8 ? 8 : 5) + NA * St::BL;  // VMEM instructions per chunk
      // token rows of the pass: gate_up gathers x rows through the token
      // table (its loads go out first, see the prologue), down reads h in
      // sorted order
      int src[NA];
#pragma unroll
      for (int nt = 0; nt < NA; ++nt) {
        const int jc = min(tg + nt * 16 + r16, n_e - 1);
        src[nt] = PHASE == 0 ? a.sorted_tok[row_start + jc] : jc;
      }
      uint32_t boff[NA];
      St st[D];
      f32x4_t acc[4][NA];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int nt = 0; nt < NA; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      // chunk j of this wave is c = wave + 4j; past the wave's last chunk
      // every load reads zeros.  issue_a: its weights and scales; issue_b:
      // its token fragments.
      // The chunk's offsets are split into a per-lane part and a
      // wave-uniform part (chunk and row-tile strides, in scalar registers).
      auto issue_a = [&](int j, St& s) __attribute__((always_inline)) {
        const int c = wave + 4 * j;
        const bool ok = j < nj;
        if constexpr (I8) {
          // 2 KB per (row tile, chunk); lane l's 32 bytes at 32 l
          const uint32_t va = ok ? uint32_t(lane * 32) : kOOB;
          const uint32_t sa = ok ? uint32_t((t0 * nc + c) * 2048) : 0u;
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            s.aq[rt] = buf_load_b128(wb.blk, va, sa + uint32_t(rt * nc * 2048));
            s.aq2[rt] = buf_load_b128(wb.blk, va + 16u, sa + uint32_t(rt * nc * 2048));
          }
        } else {
          const uint32_t va = ok ? aslot : kOOB;
          const uint32_t sa = ok ? uint32_t((t0 * nc + c) * 1024) : 0u;
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) s.aq[rt] = buf_load_b128(wb.blk, va, sa + uint32_t(rt * nc * 1024));
          s.sw = buf_load_b32(wb.sc, ok ? uint32_t(lane * 4) : kOOB, ok ? uint32_t((q * nc + c) * 256) : 0u);
        }
      };
      auto issue_b = [&](int j, St& s) __attribute__((always_inline)) {
        const int c = wave + 4 * j;
        const bool ok = j < nj;
        const uint32_t sb = ok ? uint32_t(128 * c) * EB : 0u;
        if constexpr (ACT == ACT_BF16) {
          // lane group g holds K = 128c + 32g .. +32 (4 loads of 8 values)
          const bool okg = ok && 4 * c + g < nb;
#pragma unroll
          for (int nt = 0; nt < NA; ++nt) {
            const uint32_t vb = okg ? oob_add(boff[nt], 64u * g) : kOOB;
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) s.bq[nt][s4] = buf_load_b128(bsrc, vb + 16u * s4, sb);
          }
        } else {
          // FP8 / int8 B: lane group g holds K = 128c + 16g .. +16 and 128c + 64 + 16g .. +16
          const bool ok0 = ok && 4 * c + (g >> 1) < nb, ok1 = ok && 4 * c + 2 + (g >> 1) < nb;
#pragma unroll
          for (int nt = 0; nt < NA; ++nt) {
            s.bq[nt][0] = buf_load_b128(bsrc, ok0 ? oob_add(boff[nt], 16u * g * EB) : kOOB, sb);
            s.bq[nt][1] = buf_load_b128(bsrc, ok1 ? oob_add(boff[nt], (64u + 16u * g) * EB) : kOOB, sb);
          }
        }
      };
      auto issue = [&](int j, St& s) __attribute__((always_inline)) {
        issue_a(j, s);
        issue_b(j, s);
      };
      auto compute = [&](const St& s) __attribute__((always_inline)) {
        if constexpr (ACT == ACT_BF16) {
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
              const bf16x8_t av = fp4x8_to_bf16x8(dword(s.aq[rt], s4), e8m0_as_scale_operand((s.sw >> (8 * rt)) & 0xFFu));
#pragma unroll
              for (int nt = 0; nt < NA; ++nt)
                acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, s.bq[nt][s4]),
                                                                      acc[rt][nt], 0, 0, 0);
            }
          }
        } else if constexpr (I8) {
          // two K = 64 halves; the int32 sums live in the float accumulator registers
          typedef int i32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            const i32x4_t alo = __builtin_bit_cast(i32x4_t, s.aq[rt]), ahi = __builtin_bit_cast(i32x4_t, s.aq2[rt]);
#pragma unroll
            for (int nt = 0; nt < NA; ++nt) {
              i32x4_t c4 = __builtin_bit_cast(i32x4_t, acc[rt][nt]);
              c4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo, __builtin_bit_cast(i32x4_t, s.bq[nt][0]), c4, 0, 0, 0);
              c4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi, __builtin_bit_cast(i32x4_t, s.bq[nt][1]), c4, 0, 0, 0);
              acc[rt][nt] = __builtin_bit_cast(f32x4_t, c4);
            }
          }
        } else {
          i32x8_t bv[NA];
#pragma unroll
          for (int nt = 0; nt < NA; ++nt) {
            const uint4 p0 = s.bq[nt][0], p1 = s.bq[nt][1];
            bv[nt] = i32x8_t{int(p0.x), int(p0.y), int(p0.z), int(p0.w), int(p1.x), int(p1.y), int(p1.z), int(p1.w)};
          }
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            const uint4 q4 = s.aq[rt];
            const i32x8_t av = i32x8_t{int(q4.x), int(q4.y), int(q4.z), int(q4.w), 0, 0, 0, 0};
#pragma unroll
            for (int nt = 0; nt < NA; ++nt)
              acc[rt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv[nt], acc[rt][nt], 4, 0, 0,
                                                                             int((s.sw >> (8 * rt)) & 0xFFu), 0, 127);
          }
        }
      };

      // The fixed-order sum of the 4 waves' partials, one token sub-tile at
      // a time; wave w finishes row tile w.  Its bias comes from the wave's
      // LDS area (landed before the first chunk's wait returned).
      auto finish = [&]() __attribute__((always_inline)) {
        const int r0 = 16 * (t0 + wave) + 4 * g;
        const uint2 biasq = *reinterpret_cast<const uint2*>(sbias + 8 * g);
#pragma unroll
        for (int nt = 0; nt < NA; ++nt) {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) red[wave][rt][lane] = acc[rt][nt];
          __syncthreads();
          const int j = tg + nt * 16 + r16;
          if (j < n_e && r0 < a.R) {
            f32x4_t sum;
            if constexpr (I8) {
              // exact int32 sums of the 4 waves -> fp32, times the row's and
              // the token's scales (the prefill tile's int8 epilogue)
              typedef int i32x4_t __attribute__((ext_vector_type(4)));
              i32x4_t is = __builtin_bit_cast(i32x4_t, red[0][wave][lane]);
              is += __builtin_bit_cast(i32x4_t, red[1][wave][lane]);
              is += __builtin_bit_cast(i32x4_t, red[2][wave][lane]);
              is += __builtin_bit_cast(i32x4_t, red[3][wave][lane]);
              const float4 rs = *reinterpret_cast<const float4*>(a.row_scale + int64_t(e) * a.R + r0);
              const int p = row_start + j;
              const float ts = a.tok_scale[PHASE == 0 ? a.sorted_tok[p] : p];
              sum = f32x4_t{float(is[0]) * rs.x * ts, float(is[1]) * rs.y * ts, float(is[2]) * rs.z * ts,
                            float(is[3]) * rs.w * ts};
            } else {
              sum = red[0][wave][lane];
              sum += red[1][wave][lane];
              sum += red[2][wave][lane];
              sum += red[3][wave][lane];
            }
            const float v0 = sum[0] * a.acc_scale + __uint_as_float(biasq.x << 16);
            const float v1 = sum[1] * a.acc_scale + __uint_as_float(biasq.x & 0xFFFF0000u);
            const float v2 = sum[2] * a.acc_scale + __uint_as_float(biasq.y << 16);
            const float v3 = sum[3] * a.acc_scale + __uint_as_float(biasq.y & 0xFFFF0000u);
            if (PHASE == 1 && a.cmb_out) {
              // Y rows for the folded combine: read by another workgroup
              const rsrc_t ys = make_rsrc(a.out, uint32_t(a.n_slots) * uint32_t(a.R) * 2u);
              buf_store_dev_b64(ys, uint32_t((int64_t(row_start + j) * a.R + r0) * 2),
                                make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)));
            } else {
              store_rows_biased<ACT, PHASE>(a, r0, row_start + j, v0, v1, v2, v3);
            }
          }
          __syncthreads();
        }
      };

      // Prologue: the token ids (gate_up) are the oldest loads after the
      // bias DMA, then the weights of chunks 0 .. D-2, whose streaming need
      // not wait for the ids; the token fragments of those chunks follow
      // once the ids are in.  Queue: bias, ids, A0 .. A(D-2), B0 .. B(D-2).
      order_point();
      issue_a(0, st[0]);
      order_point();
      if constexpr (D > 2) { issue_a(1, st[1]); order_point(); }
      __builtin_amdgcn_sched_barrier(0);  // nothing that needs the ids moves above the weight loads
#pragma unroll
      for (int nt = 0; nt < NA; ++nt) hold(src[nt]);
#pragma unroll
      for (int nt = 0; nt < NA; ++nt) boff[nt] = tg + nt * 16 + r16 < n_e ? uint32_t(src[nt]) * row_bytes : kOOB;
      issue_b(0, st[0]);
      order_point();
      if constexpr (D > 2) { issue_b(1, st[1]); order_point(); }
      // iteration j: wait for chunk j (D-2 later chunks may stay in flight),
      // issue chunk j + D - 1 into the stage chunk j-1 used, compute chunk
      // j, and after the last chunk form the outputs.  Chunk 0 is complete
      // once only the token fragments of chunks 1 .. D-2 are outstanding;
      // from chunk 1 on the loads of every chunk were issued together.
      auto iteration = [&](int j, auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;  // j % D
        if constexpr (u == 0) {
          if (j == 0) wait_vmcnt<(D - 2) * NA * St::BL>();
          else wait_vmcnt<(D - 2) * LOADS>();
        } else {
          wait_vmcnt<(D - 2) * LOADS>();
        }
        issue(j + D - 1, st[(u + D - 1) % D]);
        order_point();
        compute(st[u]);
        if (j == nj - 1) finish();
      };
      int j0 = 0;
      for (; j0 + D <= nj; j0 += D) {
        iteration(j0, IC<0>{});
        iteration(j0 + 1, IC<1>{});
        if constexpr (D > 2) iteration(j0 + 2, IC<2>{});
      }
      if (j0 < nj) iteration(j0, IC<0>{});
      if constexpr (D > 2) if (j0 + 1 < nj) iteration(j0 + 1, IC<1>{});
      wait_vmcnt<0>();
      // Never true (slot counts are non-negative).  It keeps every prefetch
      // live: the vmcnt waits above count loads, so none may be dropped as
      // dead even when its chunk lies past the end.
      if (a.n_slots < 0) {
        uint32_t x = 0;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          x ^= st[d].aq[0].x ^ st[d].aq[1].y ^ st[d].aq[2].z ^ st[d].aq[3].w;
          if constexpr (I8) x ^= st[d].aq2[0].x ^ st[d].aq2[1].y ^ st[d].aq2[2].z ^ st[d].aq2[3].w;
          else x ^= st[d].sw;
#pragma unroll
          for (int nt = 0; nt < NA; ++nt)
#pragma unroll
            for (int b = 0; b < St::BL; ++b) x ^= st[d].bq[nt][b].x;
        }
        static_cast<uint32_t*>(a.out)[0] = x;
      }
      // a wave with no chunks (K of at most 3 chunks) still takes its part
      // in the sum (its partials are zero)
      if (nj == 0) finish();
    };
    if (MAXNA == 1 || nt_active == 1)
      pass(IC<1>{});
    else
      pass(IC<MAXNA>{});
  }
}

}  // namespace mxmoe
