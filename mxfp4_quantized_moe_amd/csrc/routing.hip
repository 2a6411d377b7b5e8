// Routing kernels of the MXFP4 MoE layer for gfx950: router GEMM with fused
// top-k + softmax, the token->expert grouping (histogram, scan, stable
// permutation by wavefront ballots), FP8 static quantisation of x and the
// calibration reductions.
//
// The router is the upstream GptOssExperts one (gpt-oss-15.5b-23E-nf4-GPU
// page, "Notes"): logits = W_r x + b_r from the unquantised activations (the
// router is excluded from quantisation on the gpt-oss-120b-mxfp4-fp8attn-v2
// and amd/gpt-oss-20b-MoE-Quant-W-MXFP4-A-FP8-KV-FP8 pages), the top-k
// logits, then a softmax over those k.
#include "device_common.h"
#include "launch.h"
#include "topk.h"
#include "xcd_split.h"

namespace mxmoe {

// Eight bf16 values (a 16-byte load) -> eight e4m3 codes (8 bytes) with the
// static per-tensor rule sat448(rne(fp32(v) * inv)), in the input's order.
__device__ __forceinline__ uint2 bf16x8_to_e4m3x8(uint4 v, float inv) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16) * inv;
    f[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u) * inv;
  }
  return make_uint2(pack_e4m3x4(f[0], f[1], f[2], f[3]), pack_e4m3x4(f[4], f[5], f[6], f[7]));
}

// ------------------------------------------------------------------ router
//
// One workgroup per 16 tokens.  The logits^T tile (E x 16) is an MFMA
// product with A = W_r rows (experts) and B = x rows (tokens); the KW waves
// of the workgroup split the contracting dimension into interleaved
// 128-wide chunks and their partial sums are added in a fixed order in LDS,
// so the logits are deterministic.  KW = 8 when there are many token groups
// (E <= 128); a decode-sized batch (few groups) uses up to 16 waves so that
// the chain of dependent weight loads per wave stays short.  In MFMA step s
// of chunk c, lane group g (lanes 16g .. 16g+15) holds K = 128c + 32s + 8g
// .. +8 (bf16): any permutation of K applied to both operands leaves the
// dot products unchanged.  All loads of a row-tile group are in flight before its first
// MFMA (a scheduling barrier): left to itself the scheduler hoists each MFMA
// up to its load and waits there, which serialises one L2 round trip per row
// tile and step.
//
// The loads themselves are coalesced: in load s of a row tile, lane l reads
// row l/4 at K granule (16 bytes) 4s + l%4, so each lane quad reads 64
// contiguous bytes of one row (one cache access instead of four).  A lane
// transpose through ds_bpermute (destination lane 16g + r takes source lane
// 4r + g) then gives every lane the MFMA fragment described above.
//
// Partial logits sit in LDS as [wave][row tile][g][token][i] (accumulator
// element i of lane (g, token) is expert 16*rt + 4g + i), so the 16 lanes of
// one lane group store 256 contiguous bytes.

constexpr int kRouteTokens = 16;
// K-splitting waves per 16-token group for large batches (sweep knob)
#ifndef MXMOE_ROUTE_KW_LARGE
#define MXMOE_ROUTE_KW_LARGE 8
#endif

// Top-k of token t's logits by the L lanes of its group, then the softmax
// over those k; the first k lanes of the group write the outputs.
template <int KM, int L>
__device__ __forceinline__ void topk_softmax(const RouteArgs& a, const float* lg, int t) {
  const int q = threadIdx.x % L;
  uint64_t l[KM];
  topk_keys<KM, L>(lg, a.E, q, l);
  float ex[KM];
  const float den = topk_softmax_terms<KM>(l, a.top_k, ex);
#pragma unroll
  for (int kk = 0; kk < KM; ++kk) {
    if (kk < a.top_k && q == kk) {
      const float w = ex[kk] / den;
      const int64_t o = int64_t(t) * a.top_k + kk;
      const int e = key_expert(l[kk]);
      a.idx[o] = e;
      a.wts[o] = w;
      if (a.idx_out) a.idx_out[o] = e;
      if (a.wts_out) a.wts_out[o] = w;
    }
  }
}

// The grouping of one workgroup of kPermThreads threads (defined below).
__device__ void permute_block(const PermuteArgs& a);

// The work items of the tiled prefill launches that follow (defined below).
__device__ void write_item_records(const PermuteArgs& a, const int* cnt, int e_lo, int e_hi, bool write_empty);

// The top-k, softmax and grouping of a batch of at most 16 tokens and 64
// experts, by the router's one workgroup (defined below).
__device__ void finish_small_batch(const RouteArgs& a, const PermuteArgs& pa, const float* part);

// RG row tiles of 16 experts have their loads issued together, NG groups
// cover E <= 16 * RG * NG.  FUSE: the workgroup (the only one, 16 waves)
// goes on to group the slots once its top-k are written.
template <bool BF16, int RG, int NG, int KW, bool FUSE>
__global__ __launch_bounds__(64 * KW) void route_kernel(RouteArgs a, PermuteArgs pa) {
  static_assert(!FUSE || KW == 16, "the grouping takes one workgroup of 16 waves");
  extern __shared__ float part[];  // [KW][16][E]
  __shared__ float sbias[256];     // b_r, read before the contraction
  constexpr int kLanesPerToken = 4 * KW;
  constexpr int EB = BF16 ? 2 : 4;          // bytes per element of x and W_r
  constexpr int XL = BF16 ? 4 : 8;          // 16-byte loads per lane per row and chunk
  constexpr int MRT = RG * NG;              // row tiles held in registers
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;  // MFMA fragment position
  const int lrow = lane >> 2, lq = lane & 3;  // coalesced load position
  const int perm = (4 * r16 + g) * 4;         // bpermute byte index
  const int E = a.E, H = a.H;
  const int t0 = blockIdx.x * kRouteTokens;
  const int tok = t0 + lrow;
  const int nrt = (E + 15) >> 4;
  const int nchunks = (H + 127) >> 7;
  const uint32_t row_bytes = uint32_t(H) * EB;
  // range-checked windows: lanes past T or E, and K past H, read zeros
  const rsrc_t xs = make_rsrc(a.x, uint32_t(a.T) * row_bytes);
  const rsrc_t wsrc = make_rsrc(a.w_r, uint32_t(E) * row_bytes);
  const uint32_t xrow = tok < a.T ? uint32_t(tok) * row_bytes : kOOB;

  for (int e = threadIdx.x; e < E; e += 64 * KW) sbias[e] = load_param(a.b_r, e, a.act_bf16);

  f32x4_t acc[MRT];
#pragma unroll
  for (int rt = 0; rt < MRT; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int c = wave; c < nchunks; c += KW) {
    // after the transpose, step s of lane group g covers K = 128c + (32s +
    // 8g) .. +8 (bf16) or 128c + (16s + 4g) .. +4 (fp32).  Each step's K
    // range is a multiple of 16 long and H of 32, so a step lies wholly
    // inside or outside H.
    uint32_t kofs[XL];
#pragma unroll
    for (int s = 0; s < XL; ++s) {
      const int k0 = 128 * c + (BF16 ? 32 : 16) * s;
      kofs[s] = k0 < H ? uint32_t(k0 + (BF16 ? 8 : 4) * lq) * EB : kOOB;
    }
    // every load of the chunk is issued before its first MFMA
    uint4 xq[XL];
#pragma unroll
    for (int s = 0; s < XL; ++s) xq[s] = buf_load_b128(xs, oob_add(xrow, kofs[s]));
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
      if (grp * RG < nrt) {  // uniform across the workgroup
        // the previous group's MFMAs stay ahead of this group's loads
        if (grp > 0) __builtin_amdgcn_sched_barrier(0);
        uint4 wq[RG][XL];
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          const int e = (grp * RG + r) * 16 + lrow;
          const uint32_t wrow = e < E ? uint32_t(e) * row_bytes : kOOB;
#pragma unroll
          for (int s = 0; s < XL; ++s) wq[r][s] = buf_load_b128(wsrc, oob_add(wrow, kofs[s]));
        }
        // neither loads nor MFMAs cross this point
        __builtin_amdgcn_sched_barrier(0);
        if (grp == 0) {
          // FP8 mode: the e4m3 codes of these x values (the first
          // quantisation of the path), stored before the lane transpose, 8
          // values per load; the weight loads are already in flight
          if constexpr (BF16) {
            if (a.xq && tok < a.T) {
#pragma unroll
              for (int s = 0; s < XL; ++s)
                if (kofs[s] != kOOB)
                  *reinterpret_cast<uint2*>(a.xq + int64_t(tok) * H + kofs[s] / 2) = bf16x8_to_e4m3x8(xq[s], a.x_inv);
            }
          }
#pragma unroll
          for (int s = 0; s < XL; ++s) xq[s] = lane_permute(xq[s], perm);
        }
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
          for (int s = 0; s < XL; ++s) wq[r][s] = lane_permute(wq[r][s], perm);
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          f32x4_t& ac = acc[grp * RG + r];
          if constexpr (BF16) {
#pragma unroll
            for (int s = 0; s < XL; ++s)
              ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wq[r][s]),
                                                           __builtin_bit_cast(bf16x8_t, xq[s]), ac, 0, 0, 0);
          } else {
#pragma unroll
            for (int s = 0; s < XL; ++s) {
              ac = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(wq[r][s].x), __uint_as_float(xq[s].x), ac, 0, 0, 0);
              ac = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(wq[r][s].y), __uint_as_float(xq[s].y), ac, 0, 0, 0);
              ac = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(wq[r][s].z), __uint_as_float(xq[s].z), ac, 0, 0, 0);
              ac = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(wq[r][s].w), __uint_as_float(xq[s].w), ac, 0, 0, 0);
            }
          }
        }
      }
    }
  }

  // partial logits of this wave (experts past E hold zeros: their W_r rows
  // read as zero)
  const int tile = kRouteTokens * 16 * nrt;
  float* mine = part + wave * tile + 64 * g + 4 * r16;
#pragma unroll
  for (int rt = 0; rt < MRT; ++rt)
    if (rt < nrt) *reinterpret_cast<f32x4_t*>(mine + 256 * rt) = acc[rt];
  __syncthreads();
  // fixed-order sum over the waves, plus the bias
  for (int j = threadIdx.x; j < tile; j += 64 * KW) {
    const int e = 16 * (j >> 8) + 4 * ((j >> 6) & 3) + (j & 3);
    if (e < E) {
      float s = part[j];
      for (int w = 1; w < KW; ++w) s += part[w * tile + j];
      part[j] = s + sbias[e];
    }
  }
  __syncthreads();

  if constexpr (FUSE) {
    finish_small_batch(a, pa, part);
  } else {
    // top-k + softmax: 4*KW lanes per token, all 16 tokens at once
    const int tl = threadIdx.x / kLanesPerToken;
    if (t0 + tl < a.T) {
      if (a.top_k <= 4) topk_softmax<4, kLanesPerToken>(a, part + 4 * tl, t0 + tl);
      else topk_softmax<MAX_TOPK_DEV, kLanesPerToken>(a, part + 4 * tl, t0 + tl);
    }
  }
}

template <bool BF16, int KW, bool FUSE = false>
static void launch_route_typed(const RouteArgs& a, unsigned grid, hipStream_t stream, const PermuteArgs& pa = {}) {
  const size_t lds = size_t(KW) * kRouteTokens * ((a.E + 15) & ~15) * sizeof(float);
  const dim3 g(grid), b(64 * KW);
  // register tiles sized to E (fp32 operands take twice the registers)
  if (a.E <= 32)
    route_kernel<BF16, 2, 1, KW, FUSE><<<g, b, lds, stream>>>(a, pa);
  else if constexpr (BF16 || KW <= 8) {  // fp32 past E = 32: at most 8 waves (registers)
    if (a.E <= 64)
      route_kernel<BF16, 4, 1, KW, FUSE><<<g, b, lds, stream>>>(a, pa);
    else if constexpr (KW <= 8) {  // E > 64 takes at most 8 waves (LDS bound)
      if (a.E <= 128)
        route_kernel<BF16, (BF16 ? 8 : 4), (BF16 ? 1 : 2), KW, FUSE><<<g, b, lds, stream>>>(a, pa);
      else if constexpr (KW == 4)  // E > 128 always takes 4 waves
        route_kernel<BF16, 4, 4, KW, FUSE><<<g, b, lds, stream>>>(a, pa);
    }
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const unsigned grid = unsigned((a.T + kRouteTokens - 1) / kRouteTokens);
  // few token groups: more waves split K (shorter chains of dependent
  // loads per wave); many groups: 8 waves each up to E = 128.
  // The LDS of the partial logits, KW x 16 x E floats (E rounded up to a
  // multiple of 16), stays <= 64 KB.
  // 16 waves take E <= 64 (bf16) or E <= 32 (fp32: twice the registers).
  const int e16 = a.act_bf16 ? 64 : 32;
  if (grid < 64 && a.E <= e16) {
    if (a.act_bf16) launch_route_typed<true, 16>(a, grid, stream);
    else launch_route_typed<false, 16>(a, grid, stream);
  } else if (grid < 64 && a.E <= 128) {
    if (a.act_bf16) launch_route_typed<true, 8>(a, grid, stream);
    else launch_route_typed<false, 8>(a, grid, stream);
  } else if (MXMOE_ROUTE_KW_LARGE == 16 && a.E <= e16) {
    if (a.act_bf16) launch_route_typed<true, 16>(a, grid, stream);
    else launch_route_typed<false, 16>(a, grid, stream);
  } else if (MXMOE_ROUTE_KW_LARGE >= 8 && a.E <= 128) {
    if (a.act_bf16) launch_route_typed<true, 8>(a, grid, stream);
    else launch_route_typed<false, 8>(a, grid, stream);
  } else {
    if (a.act_bf16) launch_route_typed<true, 4>(a, grid, stream);
    else launch_route_typed<false, 4>(a, grid, stream);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- permutation
//
// One workgroup of 16 waves.  (1) histogram of expert ids with LDS atomics
// (integer counts, order-free); (2) exclusive scan, active-expert list and
// prefill tile offsets by wave 0; (3) stable ranking in chunks of 1024 slots:
// inside a wave the lanes holding the same expert find each other with eight
// ballots over the id bits (rank = popcount of lower peers), across the 16
// waves of a chunk per-(wave, expert) counts are scanned in wave order, and
// a running base per expert carries over between chunks.  The result orders
// the slots by (expert, flat slot id), the same grouping a stable sort gives.

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

__device__ void permute_block(const PermuteArgs& a) {
  __shared__ int cnt[256];
  __shared__ int off[257];
  __shared__ int toff[257];
  __shared__ int run_base[256];
  __shared__ int chunk_total[256];
  __shared__ int wcnt[kPermWaves][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, N = a.n_slots;

  for (int e = tid; e < 256; e += kPermThreads) {
    cnt[e] = 0;
    run_base[e] = 0;
  }
  __syncthreads();
  for (int s = tid; s < N; s += kPermThreads) {
    int e = a.idx[s];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  if (wave == 0) {
    // each lane scans 4 consecutive experts
    int c[4], t[4], tsum = 0, csum = 0, act = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      c[j] = e < E ? cnt[e] : 0;
      t[j] = (c[j] + kPrefillTokens - 1) / kPrefillTokens;
      csum += c[j];
      tsum += t[j];
      act += c[j] > 0;
    }
    int ctot, ttot, atot;
    int cbase = wave_excl_scan(csum, lane, &ctot);
    int tbase = wave_excl_scan(tsum, lane, &ttot);
    int abase = wave_excl_scan(act, lane, &atot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      if (e < E) {
        off[e] = cbase;
        a.offsets[e] = cbase;
        a.counts[e] = c[j];
        a.tile_off[e] = tbase;
        toff[e] = tbase;
        if (a.counts_out) a.counts_out[e] = c[j];
        if (a.offsets_out) a.offsets_out[e] = cbase;
        if (c[j] > 0) a.active[1 + abase++] = make_int4(e, cbase, c[j], atot);
      }
      cbase += c[j];
      tbase += t[j];
    }
    if (lane == 0) {
      off[E] = ctot;
      a.offsets[E] = ctot;
      a.tile_off[E] = ttot;
      a.active[0] = make_int4(atot, 0, 0, 0);
      if (a.offsets_out) a.offsets_out[E] = ctot;
    }
    for (int i = atot + lane; i < min(E, N); i += 64) a.active[1 + i] = make_int4(0, 0, 0, 0);
  }
  __syncthreads();

  // prefill tile table: expert e owns tiles tile_off[e] .. tile_off[e+1)
  for (int e = tid; e < E; e += kPermThreads) {
    const int c = cnt[e];
    const int t0 = toff[e];
    for (int j = 0; j * kPrefillTokens < c; ++j) {
      const int2 tt = token_tile(c, j);
      a.tiles[t0 + j] = make_int4(e, off[e] + tt.x, tt.y, 0);
    }
  }
  write_item_records(a, cnt, 0, E, true);

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < N; base += kPermThreads) {
    for (int j = tid; j < kPermWaves * 256; j += kPermThreads) (&wcnt[0][0])[j] = 0;
    __syncthreads();
    const int s = base + tid;
    const bool valid = s < N;
    int key = 0;
    if (valid) {
      key = a.idx[s];
      key = key < 0 ? 0 : (key >= E ? E - 1 : key);
    }
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wcnt[wave][key] = __popcll(peers);
    __syncthreads();
    for (int e = tid; e < E; e += kPermThreads) {
      int r = 0;
      for (int w = 0; w < kPermWaves; ++w) {
        const int c = wcnt[w][e];
        wcnt[w][e] = r;
        r += c;
      }
      chunk_total[e] = r;
    }
    __syncthreads();
    if (valid) {
      const int p = off[key] + run_base[key] + wcnt[wave][key] + rank;
      a.sorted[p] = s;
      a.sorted_tok[p] = s / a.top_k;
      a.pos[s] = p;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kPermThreads) run_base[e] += chunk_total[e];
    __syncthreads();
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(PermuteArgs a) { permute_block(a); }

// The work item of every workgroup of the tiled prefill launches that
// follow (PermuteArgs::blk_rec), resolved once here instead of by each
// workgroup: the per-expert prefixes of token tiles, sorted rows and
// per-stripe costs (4 experts per lane) and the XCD ranges (xcd_split.h),
// by wave g for launch g, both at once; then one record per item of
// experts [e_lo, e_hi) at the workgroup that takes it, and (write_empty)
// an empty record for every workgroup past its XCD's range.  cnt: the
// experts' counts in LDS.  Every thread of the workgroup calls it.
__device__ void write_item_records(const PermuteArgs& a, const int* cnt, int e_lo, int e_hi, bool write_empty) {
  if (!a.blk_rec[0] && !a.blk_rec[1]) return;  // uniform
  __shared__ int s_tp[2][257], s_wp[2][257], s_cp[257], s_bx[2][9];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  static_assert(kPermWaves >= 2, "one wave per launch");
  const bool mine = wave < 2 && a.blk_rec[wave];  // uniform per wave
  int* tp = s_tp[wave & 1];
  int* wp = s_wp[wave & 1];
  int ttot = 0;
  if (mine) {
    // the sorted-row prefix is the same for both launches: the wave of
    // launch 0 writes it, or that of launch 1 when launch 0 has no records
    const bool own_cp = wave == 0 || !a.blk_rec[0];
    int tc[4], wc[4], cc[4], ts = 0, ws = 0, cs = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      const int n = e < E ? cnt[e] : 0;
      tc[j] = (n + kPrefillTokens - 1) / kPrefillTokens;
      wc[j] = e < E ? expert_stripe_cost(n) : 0;
      cc[j] = n;
      ts += tc[j];
      ws += wc[j];
      cs += cc[j];
    }
    int wtot, ctot;
    int tb = wave_excl_scan(ts, lane, &ttot), wb = wave_excl_scan(ws, lane, &wtot), cb = wave_excl_scan(cs, lane, &ctot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      if (e < E) {
        tp[e] = tb;
        wp[e] = wb;
        if (own_cp) s_cp[e] = cb;
      }
      tb += tc[j];
      wb += wc[j];
      cb += cc[j];
    }
    if (lane == 0) {
      tp[E] = ttot;
      wp[E] = wtot;
      if (own_cp) s_cp[E] = ctot;
    }
  }
  // the prefixes are read by every lane of the wave below (a barrier, not
  // program order: the compiler may move a lane's read of another lane's
  // entry ahead of that lane's write)
  __syncthreads();
  if (mine) {
    const int ns = a.rec_stripes[wave], nblk = a.rec_blocks[wave];
    int bx[9];
    xcd_bounds(wp, tp, E, ns, nblk >> 3, ttot * ns, lane, bx);
    if (lane == 0) {
#pragma unroll
      for (int xx = 0; xx < 9; ++xx) s_bx[wave][xx] = bx[xx];
    }
  }
  __syncthreads();
  for (int gi = 0; gi < 2; ++gi) {
    int4* rec = a.blk_rec[gi];
    if (!rec) continue;  // uniform
    const int ns = a.rec_stripes[gi], nblk = a.rec_blocks[gi];
    const int* tp = s_tp[gi];
    const int* bxp = s_bx[gi];
    const int i1 = tp[e_hi] * ns;
    for (int item = tp[e_lo] * ns + tid; item < i1; item += kPermThreads) {
      int lo = e_lo, hi = e_hi;  // tp[lo] * ns <= item < tp[hi] * ns
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tp[mid] * ns <= item) lo = mid;
        else hi = mid;
      }
      const int nt = tp[lo + 1] - tp[lo];
      const int local = item - tp[lo] * ns;
      const int st = local / nt, q = local - st * nt;
      int x = 0;
      while (x < 7 && item >= bxp[x + 1]) ++x;
      const int2 tt = token_tile(cnt[lo], q);
      rec[8 * (item - bxp[x]) + x] = make_int4(lo, s_cp[lo] + tt.x, tt.y, st);
    }
    // list counters of a persistent launch: past the first item of each of
    // its workgroups
    if (write_empty && a.rec_head[gi] && tid < 8) a.rec_head[gi][tid] = uint32_t(min(nblk, kPersistentBlocks) >> 3);
    if (write_empty)
      for (int b = tid; b < nblk; b += kPermThreads) {
        const int x = b & 7;
        if ((b >> 3) >= bxp[x + 1] - bxp[x]) rec[b] = make_int4(0, 0, 0, 0);
      }
  }
}

// A batch of at most 16 tokens (E <= 64, one router workgroup of 16
// waves, logits final in `part`).  Wave t takes token t with lane e on
// expert e and finds the k best keys with the merge network of topk_keys,
// in registers; the softmax follows topk_softmax_terms over them.  After
// one barrier, wave 0 makes the grouping permute_block makes, for at most
// 16 * 8 slots: per-expert counts of the slots' ids (LDS atomics), a wave
// scan for the offsets, the active-slot records and one prefill tile per
// active expert (an expert sees at most 16 tokens), then each slot's
// stable position from ballots over the ids.
template <int KM>
__device__ __forceinline__ void small_batch_topk(const RouteArgs& a, const float* part, int t, int lane, int* sids) {
  const float* pt = part + 4 * t;
  uint64_t l[KM];
  topk_keys<KM, 64>(pt, a.E, lane, l);
  float ex[KM];
  const float den = topk_softmax_terms<KM>(l, a.top_k, ex);
  float w = 0.f;
  int e = 0;
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j == lane) {
      w = ex[j] / den;
      e = key_expert(l[j]);
    }
  if (lane < a.top_k) {
    const int o = t * a.top_k + lane;
    a.idx[o] = e;
    a.wts[o] = w;
    if (a.idx_out) a.idx_out[o] = e;
    if (a.wts_out) a.wts_out[o] = w;
    sids[o] = e;
  }
}

__device__ void finish_small_batch(const RouteArgs& a, const PermuteArgs& pa, const float* part) {
  __shared__ int sids[kRouteTokens * MAX_TOPK_DEV];
  __shared__ int cnt[64];
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
  const int E = a.E, k = a.top_k, T = a.T, N = T * k;
  if (t == 0) cnt[lane] = 0;
  if (t < T) {  // uniform per wave
    if (k <= 4) small_batch_topk<4>(a, part, t, lane, sids);
    else small_batch_topk<MAX_TOPK_DEV>(a, part, t, lane, sids);
  }
  __syncthreads();
  if (t != 0) return;  // the rest is wave 0's, with no further barrier
  // per-expert counts (integer LDS atomics, order free; this wave's LDS
  // operations complete in program order)
  for (int s = lane; s < N; s += 64) atomicAdd(&cnt[sids[s]], 1);
  const int c = lane < E ? cnt[lane] : 0;
  int tot;
  const int off = wave_excl_scan(c, lane, &tot);
  const uint64_t act = __ballot(c > 0);
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int arank = __popcll(act & lt), atot = __popcll(act);
  if (lane < E) {
    pa.offsets[lane] = off;
    pa.counts[lane] = c;
    pa.tile_off[lane] = arank;
    if (pa.counts_out) pa.counts_out[lane] = c;
    if (pa.offsets_out) pa.offsets_out[lane] = off;
    if (c > 0) {
      pa.active[1 + arank] = make_int4(lane, off, c, atot);
      pa.tiles[arank] = make_int4(lane, off, c, 0);
    }
  }
  if (lane == 0) {
    pa.offsets[E] = tot;
    pa.tile_off[E] = atot;
    pa.active[0] = make_int4(atot, 0, 0, 0);
    if (pa.offsets_out) pa.offsets_out[E] = tot;
  }
  for (int i = atot + lane; i < min(E, N); i += 64) pa.active[1 + i] = make_int4(0, 0, 0, 0);
  // stable positions, 64 slots at a time in slot order: a slot's rank
  // among the lanes holding the same expert (six ballots over the id bits,
  // E <= 64) plus the slots of that expert placed before, from its offset
  if (lane < E) cnt[lane] = 0;  // slots of each expert placed so far
  for (int base = 0; base < N; base += 64) {
    const int s = base + lane;
    const bool valid = s < N;
    const int e = valid ? sids[s] : 0;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 6; ++b) {
      const uint64_t bm = __ballot((e >> b) & 1);
      m &= ((e >> b) & 1) ? bm : ~bm;
    }
    const int r = __popcll(m & lt);
    const int o = __shfl(off, e);
    const int before = cnt[e];
    if (valid) {
      const int p = o + before + r;
      pa.sorted[p] = s;
      pa.sorted_tok[p] = s / k;
      pa.pos[s] = p;
      // the highest of the expert's lanes moves its count on
      if ((m >> lane) == 1ull) cnt[e] = before + __popcll(m);
    }
  }
}

// Expert-parallel grouping for large batches: workgroup e handles expert e.
// Every workgroup builds the full histogram in LDS (integer counts, order
// free) and scans it, which gives all offsets without a second launch; it
// then writes the entries of its own expert: offsets, count, tile range and
// tiles, its slot in the active list, and the stable positions of its
// slots.  For those, each wave takes a contiguous range of slots, counts its
// matches with ballots, takes a prefix over the waves, and sweeps the range
// again writing positions in slot order.
// Batches up to this many slots keep their expert ids in LDS as bytes
// (E <= 256) after the histogram pass reads them, so the two ranking passes
// read LDS instead of global memory.
constexpr int kPermLdsSlots = 1 << 16;

__global__ __launch_bounds__(kPermThreads) void permute_by_expert_kernel(PermuteArgs a) {
  __shared__ int cnt[256];
  __shared__ int s_off, s_toff, s_act, s_atot;
  __shared__ int wsum[kPermWaves];
  __shared__ __align__(16) uint8_t sidx[kPermLdsSlots];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, N = a.n_slots, me = blockIdx.x;
  const bool cached = N <= kPermLdsSlots;

  for (int e = tid; e < 256; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  // histogram: a thread's loads for several slots leave together, so the
  // pass waits on one L2 round trip per batch rather than per slot
  if (cached) {
    // 4 ids per 16-byte load (range-checked: past N reads zeros, which are
    // not counted), kept in LDS as one dword of 4 bytes
    const rsrc_t ir = make_rsrc(a.idx, uint32_t(N) * 4u);
    constexpr int kQ = 4;
    for (int q0 = tid; 4 * q0 < N; q0 += kQ * kPermThreads) {
      uint4 v[kQ];
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        const int q = q0 + j * kPermThreads;
        v[j] = buf_load_b128(ir, 4 * q < N ? uint32_t(q) * 16u : kOOB);
      }
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        const int s = 4 * (q0 + j * kPermThreads);
        if (s < N) {
          const int ev[4] = {int(v[j].x), int(v[j].y), int(v[j].z), int(v[j].w)};
          uint32_t packed = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = ev[i] < 0 ? 0 : (ev[i] >= E ? E - 1 : ev[i]);
            if (s + i < N) atomicAdd(&cnt[e], 1);
            packed |= uint32_t(e) << (8 * i);
          }
          // s is a multiple of 4 below N <= kPermLdsSlots: inside sidx
          *reinterpret_cast<uint32_t*>(sidx + s) = packed;
        }
      }
    }
  } else {
    constexpr int kB = 8;
    for (int base = tid; base < N; base += kB * kPermThreads) {
      int ev[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int s = base + j * kPermThreads;
        ev[j] = s < N ? a.idx[s] : 0;
      }
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int s = base + j * kPermThreads;
        if (s < N) atomicAdd(&cnt[ev[j] < 0 ? 0 : (ev[j] >= E ? E - 1 : ev[j])], 1);
      }
    }
  }
  __syncthreads();

  if (wave == 0) {
    // each lane scans 4 consecutive experts
    int c[4], tsum = 0, csum = 0, act = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      c[j] = e < E ? cnt[e] : 0;
      csum += c[j];
      tsum += (c[j] + kPrefillTokens - 1) / kPrefillTokens;
      act += c[j] > 0;
    }
    int ctot, ttot, atot;
    int cbase = wave_excl_scan(csum, lane, &ctot);
    int tbase = wave_excl_scan(tsum, lane, &ttot);
    int abase = wave_excl_scan(act, lane, &atot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      if (e == me) {
        s_off = cbase;
        s_toff = tbase;
        s_act = abase;
      }
      cbase += c[j];
      tbase += (c[j] + kPrefillTokens - 1) / kPrefillTokens;
      abase += c[j] > 0;
    }
    if (lane == 0) s_atot = atot;
    if (me == 0 && lane == 0) {
      a.offsets[E] = ctot;
      a.tile_off[E] = ttot;
      a.active[0] = make_int4(atot, 0, 0, 0);
      if (a.offsets_out) a.offsets_out[E] = ctot;
    }
    if (me == 0)
      for (int i = atot + lane; i < min(E, N); i += 64) a.active[1 + i] = make_int4(0, 0, 0, 0);
  }
  __syncthreads();
  const int c_me = cnt[me], off_me = s_off, toff_me = s_toff;
  if (tid == 0) {
    a.offsets[me] = off_me;
    a.counts[me] = c_me;
    a.tile_off[me] = toff_me;
    if (a.counts_out) a.counts_out[me] = c_me;
    if (a.offsets_out) a.offsets_out[me] = off_me;
    if (c_me > 0) a.active[1 + s_act] = make_int4(me, off_me, c_me, s_atot);
  }
  for (int j = tid; j * kPrefillTokens < c_me; j += kPermThreads) {
    const int2 tt = token_tile(c_me, j);
    a.tiles[toff_me + j] = make_int4(me, off_me + tt.x, tt.y, 0);
  }

  write_item_records(a, cnt, me, me + 1, me == 0);

  // stable positions of this expert's slots: wave w takes a contiguous
  // range [s0, s1), counts its matches, takes the prefix over the waves and
  // sweeps the range again writing positions in slot order
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int end = off_me + c_me;  // positions stay inside the expert's range
  if (cached) {
    // 4 consecutive slots per lane and step: slot s + i of lane l comes
    // after every slot of the lanes below l and the i' < i of its own
    const int per_wave = ((N + kPermWaves - 1) / kPermWaves + 255) & ~255;
    const int s0 = wave * per_wave, s1 = min(N, s0 + per_wave);
    auto hits = [&](int s, bool (&h)[4]) __attribute__((always_inline)) {
      const uint32_t w4 = s < s1 ? *reinterpret_cast<const uint32_t*>(sidx + s) : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = s + i < s1 && ((w4 >> (8 * i)) & 0xFFu) == uint32_t(me);
    };
    int mine = 0;
    for (int b = s0; b < s1; b += 256) {
      bool h[4];
      hits(b + 4 * lane, h);
#pragma unroll
      for (int i = 0; i < 4; ++i) mine += __popcll(__ballot(h[i]));
    }
    if (lane == 0) wsum[wave] = mine;
    __syncthreads();
    int run = off_me;
    for (int w = 0; w < wave; ++w) run += wsum[w];
    for (int b = s0; b < s1; b += 256) {
      const int s = b + 4 * lane;
      bool h[4];
      hits(s, h);
      int before = 0, tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint64_t m = __ballot(h[i]);
        before += __popcll(m & lt_mask);
        tot += __popcll(m);
      }
      int p = run + before;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (h[i]) {
          if (p < end) {
            a.sorted[p] = s + i;
            a.sorted_tok[p] = (s + i) / a.top_k;
            a.pos[s + i] = p;
          }
          ++p;
        }
      }
      run += tot;
    }
  } else {
    auto key_at = [&](int s) -> int {
      const int e = a.idx[s];
      return e < 0 ? 0 : (e >= E ? E - 1 : e);
    };
    const int per_wave = ((N + kPermWaves - 1) / kPermWaves + 63) & ~63;
    const int s0 = wave * per_wave, s1 = min(N, s0 + per_wave);
    int mine = 0;
    for (int b = s0; b < s1; b += 64) {
      const int s = b + lane;
      const int key = s < s1 ? key_at(s) : -1;
      mine += __popcll(__ballot(key == me));
    }
    if (lane == 0) wsum[wave] = mine;
    __syncthreads();
    int run = off_me;
    for (int w = 0; w < wave; ++w) run += wsum[w];
    for (int b = s0; b < s1; b += 64) {
      const int s = b + lane;
      const int key = s < s1 ? key_at(s) : -1;
      const uint64_t m = __ballot(key == me);
      if (key == me) {
        const int p = run + __popcll(m & lt_mask);
        if (p < end) {
          a.sorted[p] = s;
          a.sorted_tok[p] = s / a.top_k;
          a.pos[s] = p;
        }
      }
      run += __popcll(m);
    }
  }
}

// Batches up to this many slots use the single-workgroup kernel (one
// launch-latency-bound pass); larger ones the expert-parallel kernel, which
// reads the expert ids three times per workgroup.
constexpr int kPermSmall = 2048;
constexpr int kPermLarge = 1 << 20;

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  if (a.n_slots == 0) return hipSuccess;
  if (a.n_slots > kPermSmall && a.n_slots <= kPermLarge)
    permute_by_expert_kernel<<<dim3(unsigned(a.E)), dim3(kPermThreads), 0, stream>>>(a);
  else
    permute_kernel<<<dim3(1), dim3(kPermThreads), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_route_permute(const RouteArgs& a, const PermuteArgs& p, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  static_assert(kPermThreads == 64 * 16, "the fused grouping runs on the router's 16 waves");
  const bool one_group = a.T <= kRouteTokens;  // one router workgroup
  if (one_group && a.E <= (a.act_bf16 ? 64 : 32) && p.n_slots <= kPermSmall) {
    if (a.act_bf16) launch_route_typed<true, 16, true>(a, 1, stream, p);
    else launch_route_typed<false, 16, true>(a, 1, stream, p);
    return hipGetLastError();
  }
  hipError_t e = launch_route(a, stream);
  if (e != hipSuccess) return e;
  return launch_permute(p, stream);
}

// --------------------------------------------------------------- FP8 quant
//
// code = sat448(rne_e4m3(fp32(x) * inv_scale)), inv_scale = 1 / s computed
// once in fp32 on the host (FP8 static per-tensor scheme).  8 values per
// thread: one 16-byte load, one 8-byte store.

__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint4* __restrict__ x, int64_t n8, float inv,
                                                        uint2* __restrict__ q) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  q[i] = bf16x8_to_e4m3x8(x[i], inv);
}

// ------------------------------------------------------------- dense layer
//
// A dense layer runs through the grouped GEMMs as one expert that every
// token routes to once: expert 0 owns sorted rows 0 .. T-1 (the token rows
// themselves), in ceil(T / kPrefillTokens) prefill tiles.

__global__ __launch_bounds__(256) void linear_setup_kernel(int T, int32_t* offsets, int4* active, int32_t* tile_off,
                                                           int4* tiles, void* zero_bias, int N, int zero_bias_bytes) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int ntiles = (T + kPrefillTokens - 1) / kPrefillTokens;
  if (i == 0) {
    offsets[0] = 0;
    offsets[1] = T;
    active[0] = make_int4(1, 0, 0, 0);
    active[1] = make_int4(0, 0, T, 1);
    tile_off[0] = 0;
    tile_off[1] = ntiles;
  }
  if (i < ntiles) {
    const int2 tt = token_tile(T, i);
    tiles[i] = make_int4(0, tt.x, tt.y, 0);
  }
  if (zero_bias && i < N) {
    if (zero_bias_bytes == 2)
      static_cast<uint16_t*>(zero_bias)[i] = 0;
    else
      static_cast<float*>(zero_bias)[i] = 0.f;
  }
}

hipError_t launch_linear_setup(int T, int32_t* offsets, int4* active, int32_t* tile_off, int4* tiles,
                               void* zero_bias, int N, int zero_bias_bytes, hipStream_t stream) {
  const int ntiles = (T + kPrefillTokens - 1) / kPrefillTokens;
  const int n = ntiles > N ? ntiles : N;
  linear_setup_kernel<<<dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream>>>(T, offsets, active, tile_off, tiles,
                                                                               zero_bias, N, zero_bias_bytes);
  return hipGetLastError();
}

// ---------------------------------------------------- dense all-experts
//
// Grouping of the dense path: row e*T + t is token t for expert e, every
// expert active with all T tokens; the combine finds slot (t, j) at row
// idx[t, j] * T + t.

__global__ __launch_bounds__(256) void dense_group_kernel(DenseGroupArgs a) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int T = a.T, E = a.E;
  const int64_t rows = int64_t(T) * E;
  const int ntiles = (T + kPrefillTokens - 1) / kPrefillTokens;
  if (i < rows) a.sorted_tok[i] = int(i % T);
  if (i < int64_t(T) * a.top_k) {
    int e = a.idx[i];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    a.pos[i] = e * T + int(i / a.top_k);
  }
  if (i <= E) {
    a.offsets[i] = int(i) * T;
    a.tile_off[i] = int(i) * ntiles;
    if (i < E) {
      a.counts[i] = T;
      a.active[1 + i] = make_int4(int(i), int(i) * T, T, E);
    } else {
      a.active[0] = make_int4(E, 0, 0, 0);
    }
  }
  if (i < int64_t(E) * ntiles) {
    const int e = int(i / ntiles), q = int(i % ntiles);
    const int2 tt = token_tile(T, q);
    a.tiles[i] = make_int4(e, e * T + tt.x, tt.y, 0);
  }
}

hipError_t launch_dense_group(const DenseGroupArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int64_t rows = int64_t(a.T) * a.E;
  const int64_t n = rows > a.E + 1 ? rows : a.E + 1;
  dense_group_kernel<<<dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const uint16_t* x, int64_t n, float inv_scale, uint8_t* q, hipStream_t stream) {
  const int64_t n8 = n / 8;  // n is a multiple of 32
  if (n8 == 0) return hipSuccess;
  quant_fp8_kernel<<<dim3(unsigned((n8 + 255) / 256)), dim3(256), 0, stream>>>(
      reinterpret_cast<const uint4*>(x), n8, inv_scale, reinterpret_cast<uint2*>(q));
  return hipGetLastError();
}

// ------------------------------------------------ int8 per-row quantisation
//
// Symmetric int8 with one dynamic scale per row (per token): s = amax / 127
// over the row's |values| (fp32, a correctly rounded division), code =
// clamp(rne(v / s), -127, 127), all codes 0 when the row is all zero (s = 0).
// One workgroup per row; each thread reads 8 bf16 values at a time.

__global__ __launch_bounds__(256) void quant_rows_int8_kernel(const uint4* __restrict__ x, int K8, int8_t* q,
                                                              float* scale) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint4* xr = x + row * K8;
  float m = 0.f;
  for (int i = threadIdx.x; i < K8; i += 256) {
    const uint4 v = xr[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w[j] << 16)));
      m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w[j] & 0xFFFF0000u)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const float s = amax / 127.0f;
  if (threadIdx.x == 0) scale[row] = s;
  uint2* qr = reinterpret_cast<uint2*>(q + row * int64_t(K8) * 8);
  for (int i = threadIdx.x; i < K8; i += 256) {
    const uint4 v = xr[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float f = __uint_as_float((j & 1) ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16));
      float c = amax > 0.f ? __builtin_rintf(f / s) : 0.f;
      c = __builtin_fminf(__builtin_fmaxf(c, -127.f), 127.f);
      packed[j >> 2] |= (uint32_t(int(c)) & 0xFFu) << (8 * (j & 3));
    }
    qr[i] = make_uint2(packed[0], packed[1]);
  }
}

// Rows of at most 64 * 8 * NL values: one wave per row (4 rows per
// workgroup) keeps the row in registers, NL 16-byte pieces per lane, so it
// is read once and the maximum needs no workgroup barrier.  Same arithmetic
// as above, so the same codes.
template <int NL>
__global__ __launch_bounds__(256) void quant_rows_int8_wave_kernel(const uint4* __restrict__ x, int64_t rows, int K8,
                                                                   int8_t* q, float* scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const uint4* xr = x + row * K8;
  uint4 v[NL];
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int i = lane + 64 * j;
    v[j] = i < K8 ? xr[i] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w[t] << 16)));
      m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w[t] & 0xFFFF0000u)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  const float amax = m;
  const float s = amax / 127.0f;
  if (lane == 0) scale[row] = s;
  uint2* qr = reinterpret_cast<uint2*>(q + row * int64_t(K8) * 8);
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int i = lane + 64 * j;
    if (i < K8) {
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float f = __uint_as_float((t & 1) ? (w[t >> 1] & 0xFFFF0000u) : (w[t >> 1] << 16));
        float c = amax > 0.f ? __builtin_rintf(f / s) : 0.f;
        c = __builtin_fminf(__builtin_fmaxf(c, -127.f), 127.f);
        packed[t >> 2] |= (uint32_t(int(c)) & 0xFFu) << (8 * (t & 3));
      }
      qr[i] = make_uint2(packed[0], packed[1]);
    }
  }
}

hipError_t launch_quant_rows_int8(const uint16_t* x, int64_t rows, int K, int8_t* q, float* scale,
                                  hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int K8 = K / 8;
  const int nl = (K8 + 63) / 64;  // 16-byte pieces per lane
  const dim3 g(unsigned((rows + 3) / 4)), b(256);
  switch (nl) {
    case 1: quant_rows_int8_wave_kernel<1><<<g, b, 0, stream>>>(xv, rows, K8, q, scale); break;
    case 2: quant_rows_int8_wave_kernel<2><<<g, b, 0, stream>>>(xv, rows, K8, q, scale); break;
    case 3: quant_rows_int8_wave_kernel<3><<<g, b, 0, stream>>>(xv, rows, K8, q, scale); break;
    case 4: quant_rows_int8_wave_kernel<4><<<g, b, 0, stream>>>(xv, rows, K8, q, scale); break;
    case 5: quant_rows_int8_wave_kernel<5><<<g, b, 0, stream>>>(xv, rows, K8, q, scale); break;
    case 6: quant_rows_int8_wave_kernel<6><<<g, b, 0, stream>>>(xv, rows, K8, q, scale); break;
    case 7: quant_rows_int8_wave_kernel<7><<<g, b, 0, stream>>>(xv, rows, K8, q, scale); break;
    case 8: quant_rows_int8_wave_kernel<8><<<g, b, 0, stream>>>(xv, rows, K8, q, scale); break;
    default: quant_rows_int8_kernel<<<dim3(unsigned(rows)), dim3(256), 0, stream>>>(xv, K8, q, scale); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- calibration
//
// amax over bf16 tensors: |v| as an unsigned bit pattern orders like the
// value, so an integer atomic max gives the exact, order-free maximum.

__global__ void calib_init_kernel(uint32_t* slots) {
  if (threadIdx.x < 2) slots[threadIdx.x] = 0u;
}

__global__ __launch_bounds__(256) void amax_bf16_kernel(const uint4* __restrict__ v, int64_t n8, uint32_t* slot) {
  uint32_t m = 0;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n8; i += int64_t(gridDim.x) * 256) {
    const uint4 q = v[i];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
      lo = lo > 0x7F80u ? 0u : lo;  // NaN does not count
      hi = hi > 0x7F80u ? 0u : hi;
      m = m > lo ? m : lo;
      m = m > hi ? m : hi;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(m, off);
    m = m > o ? m : o;
  }
  if ((threadIdx.x & 63) == 0) atomicMax(slot, m);
}

__global__ void calib_finish_kernel(const uint32_t* slots, float* out) {
  if (threadIdx.x < 2) out[threadIdx.x] = __uint_as_float(slots[threadIdx.x] << 16) / 448.0f;
}

hipError_t launch_calib_init(uint32_t* slots, hipStream_t stream) {
  calib_init_kernel<<<1, 64, 0, stream>>>(slots);
  return hipGetLastError();
}

hipError_t launch_amax_bf16(const uint16_t* v, int64_t n, uint32_t* slot, hipStream_t stream) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  int64_t grid = (n8 + 255) / 256;
  if (grid > 2048) grid = 2048;
  amax_bf16_kernel<<<dim3(unsigned(grid)), dim3(256), 0, stream>>>(reinterpret_cast<const uint4*>(v), n8, slot);
  return hipGetLastError();
}

hipError_t launch_calib_finish(const uint32_t* slots, float* scales_out, hipStream_t stream) {
  calib_finish_kernel<<<1, 64, 0, stream>>>(slots, scales_out);
  return hipGetLastError();
}

}  // namespace mxmoe
