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
#include "device_common.h"
#include "launch.h"

namespace mxmoe {

constexpr int kDecodeRowTiles = 1;  // 16 weight rows per decode workgroup
constexpr int kDecodeChunkBuf = 8;  // 128-K chunks kept in flight per wave

// ------------------------------------------------------------ operands

struct AFrag {
  uint4 q;       // 16 bytes = 32 nibbles of one block of one weight row
  uint32_t s;    // its e8m0 scale byte
};

__device__ __forceinline__ AFrag load_a(const uint8_t* wblk, const uint8_t* wsc, int row, int nb, int block) {
  AFrag f;
  if (block < nb) {
    const int64_t o = int64_t(row) * nb + block;
    f.q = *reinterpret_cast<const uint4*>(wblk + o * 16);
    f.s = wsc[o];
  } else {
    f.q = make_uint4(0, 0, 0, 0);
    f.s = 127;
  }
  return f;
}

__device__ __forceinline__ uint32_t dword(const uint4& q, int i) {
  return i == 0 ? q.x : (i == 1 ? q.y : (i == 2 ? q.z : q.w));
}

// ------------------------------------------------------------ epilogue

// Store one lane's 4 accumulator rows (r0 .. r0+3) of one token (sorted row p).
template <int ACT, int PHASE>
__device__ __forceinline__ void store_rows(const GemmArgs& a, int e, int r0, int64_t p, float v0, float v1, float v2,
                                           float v3) {
  const int64_t bo = int64_t(e) * a.R + r0;
  v0 = v0 * a.acc_scale + load_param(a.bias, bo + 0, a.bias_bf16);
  v1 = v1 * a.acc_scale + load_param(a.bias, bo + 1, a.bias_bf16);
  v2 = v2 * a.acc_scale + load_param(a.bias, bo + 2, a.bias_bf16);
  v3 = v3 * a.acc_scale + load_param(a.bias, bo + 3, a.bias_bf16);
  if constexpr (PHASE == 0) {
    // rows r0, r0+1 = (gate, up) of h column r0/2; rows r0+2, r0+3 the next
    const float h0 = clamped_swiglu(v0, v1);
    const float h1 = clamped_swiglu(v2, v3);
    const int64_t I = a.R / 2;
    const int64_t o = p * I + r0 / 2;
    if constexpr (ACT == ACT_BF16) {
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + o) = pack_bf16x2(h0, h1);
    } else if constexpr (ACT == ACT_F32) {
      *reinterpret_cast<float2*>(static_cast<float*>(a.out) + o) = make_float2(h0, h1);
    } else {
      const uint32_t q = pack_e4m3x4(h0 * a.out_inv_scale, h1 * a.out_inv_scale, 0.f, 0.f);
      *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(a.out) + o) = uint16_t(q & 0xFFFFu);
    }
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + p * a.R + r0) = make_float4(v0, v1, v2, v3);
  }
}

// =====================================================================
// Decode-shaped GEMM: few tokens per expert.  The bound is streaming the
// routed experts' packed weights, so each workgroup owns 16 weight rows of
// one active expert and its 4 waves split the K chunks (c = wave, wave+4,
// ...), issuing up to kDecodeChunkBuf 128-bit weight loads per lane before
// the first MFMA.  Partial sums are added across waves in a fixed order in
// LDS.  Activations (at most 64 tokens per pass) are read straight from
// global memory, where they stay cache-resident.
// =====================================================================

template <int ACT, int PHASE>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs a) {
  constexpr int RT = kDecodeRowTiles;
  __shared__ f32x4_t red[4][RT][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int slot = blockIdx.y;
  if (slot >= a.active[0]) return;
  const int e = a.active[1 + slot];
  const int row_start = a.offsets[e];
  const int n_e = a.offsets[e + 1] - row_start;
  const int nb = a.nb, K = nb * 32;
  const int nchunks = (nb + 3) >> 2;
  const int rbase = blockIdx.x * (16 * RT);
  const uint8_t* wblk = a.wblk + int64_t(e) * a.R * nb * 16;
  const uint8_t* wsc = a.wsc + int64_t(e) * a.R * nb;
  constexpr int EB = ACT == ACT_F32 ? 4 : (ACT == ACT_BF16 ? 2 : 1);  // bytes per B element
  const uint8_t* bsrc = static_cast<const uint8_t*>(a.bsrc);

  for (int tg = 0; tg < n_e; tg += 64) {
    // this lane's token row for each of the 4 token sub-tiles
    const uint8_t* brow[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int j = tg + nt * 16 + r16;
      brow[nt] = nullptr;
      if (j < n_e) {
        const int64_t p = row_start + j;
        const int64_t src_row = PHASE == 0 ? int64_t(a.sorted[p] / a.top_k) : p;
        brow[nt] = bsrc + src_row * K * EB;
      }
    }
    const int nt_active = min(4, (n_e - tg + 15) >> 4);

    f32x4_t acc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int c0 = wave; c0 < nchunks; c0 += 4 * kDecodeChunkBuf) {
      AFrag af[kDecodeChunkBuf][RT];
#pragma unroll
      for (int u = 0; u < kDecodeChunkBuf; ++u) {
        const int c = c0 + 4 * u;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          af[u][rt] = load_a(wblk, wsc, rbase + 16 * rt + r16, nb, c < nchunks ? 4 * c + g : nb);
      }
#pragma unroll
      for (int u = 0; u < kDecodeChunkBuf; ++u) {
        const int c = c0 + 4 * u;
        if (c >= nchunks) break;
        const bool kvalid = 4 * c + g < nb;
        if constexpr (ACT == ACT_BF16) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            bf16x8_t b[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              uint4 q = make_uint4(0, 0, 0, 0);
              if (brow[nt] && kvalid) q = *reinterpret_cast<const uint4*>(brow[nt] + (128 * c + 32 * g + 8 * s) * 2);
              b[nt] = __builtin_bit_cast(bf16x8_t, q);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              const bf16x8_t av = fp4x8_to_bf16x8(dword(af[u][rt].q, s), e8m0_as_scale_operand(af[u][rt].s));
#pragma unroll
              for (int nt = 0; nt < 4; ++nt)
                if (nt < nt_active) acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[nt], acc[rt][nt], 0, 0, 0);
            }
          }
        } else if constexpr (ACT == ACT_F32) {
#pragma unroll
          for (int s4 = 0; s4 < 8; ++s4) {
            float4 b[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              b[nt] = make_float4(0.f, 0.f, 0.f, 0.f);
              if (brow[nt] && kvalid) b[nt] = *reinterpret_cast<const float4*>(brow[nt] + (128 * c + 32 * g + 4 * s4) * 4);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              const uint32_t w = dword(af[u][rt].q, s4 >> 1);
              const float sc = e8m0_as_scale_operand(af[u][rt].s);
              f32x2_t lo, hi;
              if (s4 & 1) {
                lo = fp4x2_to_f32x2<2>(w, sc);
                hi = fp4x2_to_f32x2<3>(w, sc);
              } else {
                lo = fp4x2_to_f32x2<0>(w, sc);
                hi = fp4x2_to_f32x2<1>(w, sc);
              }
#pragma unroll
              for (int nt = 0; nt < 4; ++nt) {
                if (nt < nt_active) {
                  acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(lo[0], b[nt].x, acc[rt][nt], 0, 0, 0);
                  acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(lo[1], b[nt].y, acc[rt][nt], 0, 0, 0);
                  acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(hi[0], b[nt].z, acc[rt][nt], 0, 0, 0);
                  acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(hi[1], b[nt].w, acc[rt][nt], 0, 0, 0);
                }
              }
            }
          }
        } else {
          // FP8: B lane group g holds K = 128c + 16g .. +16 and 128c + 64 + 16g .. +16
          const bool v0 = 4 * c + (g >> 1) < nb;
          const bool v1 = 4 * c + 2 + (g >> 1) < nb;
          i32x8_t b[4];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            uint4 p0 = make_uint4(0, 0, 0, 0), p1 = make_uint4(0, 0, 0, 0);
            if (brow[nt]) {
              if (v0) p0 = *reinterpret_cast<const uint4*>(brow[nt] + 128 * c + 16 * g);
              if (v1) p1 = *reinterpret_cast<const uint4*>(brow[nt] + 128 * c + 64 + 16 * g);
            }
            b[nt] = i32x8_t{int(p0.x), int(p0.y), int(p0.z), int(p0.w), int(p1.x), int(p1.y), int(p1.z), int(p1.w)};
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const uint4 q = af[u][rt].q;
            const i32x8_t av = i32x8_t{int(q.x), int(q.y), int(q.z), int(q.w), 0, 0, 0, 0};
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
              if (nt < nt_active)
                acc[rt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b[nt], acc[rt][nt], 4, 0, 0,
                                                                               int(af[u][rt].s), 0, 127);
          }
        }
      }
    }

    // fixed-order reduction of the 4 waves' partial sums
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) red[wave][rt][nt][lane] = acc[rt][nt];
    __syncthreads();
    {
      const int nt = wave;  // wave w finishes token sub-tile w
      const int j = tg + nt * 16 + r16;
      if (nt < nt_active && j < n_e) {
        const int64_t p = row_start + j;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          f32x4_t s = red[0][rt][nt][lane];
          s += red[1][rt][nt][lane];
          s += red[2][rt][nt][lane];
          s += red[3][rt][nt][lane];
          store_rows<ACT, PHASE>(a, e, rbase + 16 * rt + 4 * g, p, s[0], s[1], s[2], s[3]);
        }
      }
    }
    __syncthreads();
  }
}

// =====================================================================
// Prefill-shaped GEMM: many tokens per expert, bound by the matrix cores.
// Workgroup tile = 256 weight rows (4 waves x 64 rows) x 64 tokens of one
// expert.  Activations of each 128-K chunk are staged in LDS (double
// buffered, rows padded by 16 bytes so the 16 lanes of a lane group hit
// distinct banks); each wave streams its own 64 weight rows straight into
// registers (one 128-bit load per row tile per chunk, prefetched a chunk
// ahead) and decodes them in registers.  The work list is (token tile,
// row stripe) with the stripe fastest; workgroup ids are remapped so that
// consecutive items land on the same XCD and share its L2.
// =====================================================================

__device__ __forceinline__ int find_expert(const int32_t* tile_off, int E, int tile) {
  // largest e with tile_off[e] <= tile (tile_off is non-decreasing)
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_off[mid] <= tile)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

template <int ACT, int PHASE>
__global__ __launch_bounds__(256) void gemm_prefill_kernel(GemmArgs a) {
  static_assert(ACT == ACT_BF16 || ACT == ACT_FP8, "prefill path takes bf16 or fp8 activations");
  constexpr int EB = ACT == ACT_BF16 ? 2 : 1;
  constexpr int KB = 128 * EB;  // bytes of one token row per chunk
  constexpr int LD = KB + 16;   // padded LDS row stride
  constexpr int PIECES = KB / 16;
  constexpr int PPT = PIECES / 4;  // 16-byte pieces per thread per chunk
  __shared__ __align__(16) uint8_t bs[2][64 * LD];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;

  // XCD-aware remap: hardware places workgroup b on XCD b % 8
  const int G = gridDim.x;  // multiple of 8
  const int item = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int nstripes = (a.R + kPrefillRows - 1) / kPrefillRows;
  const int tile = item / nstripes, stripe = item - tile * nstripes;
  if (tile >= a.tile_off[a.E]) return;
  const int e = find_expert(a.tile_off, a.E, tile);
  const int tok0 = (tile - a.tile_off[e]) * kPrefillTokens;
  const int row_start = a.offsets[e] + tok0;
  const int ntok = min(kPrefillTokens, a.offsets[e + 1] - a.offsets[e] - tok0);
  const int nt_active = (ntok + 15) >> 4;
  const int nb = a.nb, K = nb * 32;
  const int nchunks = (nb + 3) >> 2;
  const int wrow = stripe * kPrefillRows + wave * 64;
  const int rt_active = max(0, min(4, (a.R - wrow) >> 4));
  const uint8_t* wblk = a.wblk + int64_t(e) * a.R * nb * 16;
  const uint8_t* wsc = a.wsc + int64_t(e) * a.R * nb;

  // B staging: thread t copies row t/4, pieces (t%4) + 4i
  const int brow_j = threadIdx.x >> 2, bq = threadIdx.x & 3;
  const uint8_t* bsrc = nullptr;
  if (brow_j < ntok) {
    const int64_t p = row_start + brow_j;
    const int64_t src_row = PHASE == 0 ? int64_t(a.sorted[p] / a.top_k) : p;
    bsrc = static_cast<const uint8_t*>(a.bsrc) + src_row * int64_t(K) * EB;
  }
  uint4 breg[PPT];
  auto load_b = [&](int c) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int piece = bq + 4 * i;
      const int kel = 128 * c + piece * (16 / EB);  // first K index of the piece
      breg[i] = make_uint4(0, 0, 0, 0);
      if (bsrc && kel < K) breg[i] = *reinterpret_cast<const uint4*>(bsrc + int64_t(kel) * EB);
    }
  };
  auto store_b = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      *reinterpret_cast<uint4*>(&bs[buf][brow_j * LD + (bq + 4 * i) * 16]) = breg[i];
  };

  AFrag acur[4], anext[4];
  auto load_a4 = [&](AFrag* dst, int c) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
      if (rt < rt_active) dst[rt] = load_a(wblk, wsc, wrow + 16 * rt + r16, nb, 4 * c + g);
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_b(0);
  load_a4(acur, 0);
  store_b(0);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunks;
    if (more) {
      load_b(c + 1);
      load_a4(anext, c + 1);
    }
    const uint8_t* tileb = bs[buf];
    if constexpr (ACT == ACT_BF16) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t b[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          if (nt < nt_active)
            b[nt] = *reinterpret_cast<const bf16x8_t*>(tileb + (nt * 16 + r16) * LD + 64 * g + 16 * s);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          if (rt < rt_active) {
            const bf16x8_t av = fp4x8_to_bf16x8(dword(acur[rt].q, s), e8m0_as_scale_operand(acur[rt].s));
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
              if (nt < nt_active) acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[nt], acc[rt][nt], 0, 0, 0);
          }
        }
      }
    } else {
      i32x8_t b[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (nt < nt_active) {
          const uint8_t* r = tileb + (nt * 16 + r16) * LD;
          const uint4 p0 = *reinterpret_cast<const uint4*>(r + 16 * g);
          const uint4 p1 = *reinterpret_cast<const uint4*>(r + 64 + 16 * g);
          b[nt] = i32x8_t{int(p0.x), int(p0.y), int(p0.z), int(p0.w), int(p1.x), int(p1.y), int(p1.z), int(p1.w)};
        }
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (rt < rt_active) {
          const uint4 q = acur[rt].q;
          const i32x8_t av = i32x8_t{int(q.x), int(q.y), int(q.z), int(q.w), 0, 0, 0, 0};
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            if (nt < nt_active)
              acc[rt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b[nt], acc[rt][nt], 4, 0, 0,
                                                                             int(acur[rt].s), 0, 127);
        }
      }
    }
    if (more) {
      store_b(buf ^ 1);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acur[rt] = anext[rt];
    }
    __syncthreads();
  }

#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    if (rt < rt_active) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int j = nt * 16 + r16;
        if (nt < nt_active && j < ntok)
          store_rows<ACT, PHASE>(a, e, wrow + 16 * rt + 4 * g, row_start + j, acc[rt][nt][0], acc[rt][nt][1],
                                 acc[rt][nt][2], acc[rt][nt][3]);
      }
    }
  }
}

template <int ACT, int PHASE>
static void launch_one(const GemmArgs& a, bool prefill, hipStream_t stream) {
  if (prefill) {
    if constexpr (ACT != ACT_F32) {
      const int nstripes = (a.R + kPrefillRows - 1) / kPrefillRows;
      int64_t items = int64_t(a.max_tiles) * nstripes;
      items = (items + 7) / 8 * 8;
      gemm_prefill_kernel<ACT, PHASE><<<dim3(unsigned(items)), dim3(256), 0, stream>>>(a);
    }
  } else {
    const unsigned gx = unsigned(a.R / (16 * kDecodeRowTiles));
    gemm_decode_kernel<ACT, PHASE><<<dim3(gx, unsigned(a.max_active)), dim3(256), 0, stream>>>(a);
  }
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
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------- combine
//
// out_t = sum_j w[t, j] * Y[pos[t*k + j]] in the order j = 0 .. k-1 (fp32),
// one workgroup per token, four columns per thread.

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
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
  for (int c = threadIdx.x * 4; c < a.H; c += 256 * 4) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < MAX_TOPK_DEV; ++j) {
      if (j < k) {
        const float4 y = *reinterpret_cast<const float4*>(a.Y + rows[j] + c);
        s.x += w[j] * y.x;
        s.y += w[j] * y.y;
        s.z += w[j] * y.z;
        s.w += w[j] * y.w;
      }
    }
    const int64_t o = int64_t(t) * a.H + c;
    if (a.out_bf16)
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
    else
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o) = s;
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  combine_kernel<<<dim3(unsigned(a.T)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mxmoe
