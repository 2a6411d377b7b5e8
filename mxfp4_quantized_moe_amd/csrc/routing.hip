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
#include <climits>

#include "device_common.h"
#include "launch.h"

namespace mxmoe {

// ------------------------------------------------------------------ router
//
// One workgroup per 16 tokens.  The logits^T tile (E x 16) is an MFMA
// product with A = W_r rows (experts) and B = x rows (tokens); the KW waves
// of the workgroup split the contracting dimension into interleaved
// 128-wide chunks and their partial sums are added in a fixed order in LDS,
// so the logits are deterministic.  KW = 8 when there are many token groups
// (E <= 128); a decode-sized batch (few groups) uses up to 16 waves so that
// the chain of dependent weight loads per wave stays short.  In MFMA step s
// of a chunk, lane group g (lanes 16g .. 16g+15) holds K = 128c + 32s + 8g
// .. +8 (bf16), so the lane groups of a row read adjacent bytes: any
// permutation of K applied to both operands leaves the dot products
// unchanged.

constexpr int kRouteTokens = 16;
// K-splitting waves per 16-token group for large batches (sweep knob)
#ifndef MXMOE_ROUTE_KW_LARGE
#define MXMOE_ROUTE_KW_LARGE 8
#endif

// RG row tiles of 16 experts have their loads issued together, NG groups
// cover E <= 16 * RG * NG.
template <bool BF16, int RG, int NG, int KW>
__global__ __launch_bounds__(64 * KW) void route_kernel(RouteArgs a) {
  extern __shared__ float part[];  // [KW][16][E]
  constexpr int EB = BF16 ? 2 : 4;          // bytes per element of x and W_r
  constexpr int XL = BF16 ? 4 : 8;          // 16-byte loads per lane per row and chunk
  constexpr int MRT = RG * NG;              // row tiles held in registers
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int E = a.E, H = a.H;
  const int t0 = blockIdx.x * kRouteTokens;
  const int tok = t0 + r16;
  const int nrt = (E + 15) >> 4;
  const int nchunks = (H + 127) >> 7;
  const uint32_t row_bytes = uint32_t(H) * EB;
  // range-checked windows: lanes past T or E, and K past H, read zeros
  const rsrc_t xs = make_rsrc(a.x, uint32_t(a.T) * row_bytes);
  const rsrc_t wsrc = make_rsrc(a.w_r, uint32_t(E) * row_bytes);
  const uint32_t xrow = tok < a.T ? uint32_t(tok) * row_bytes : kOOB;

  f32x4_t acc[MRT];
#pragma unroll
  for (int rt = 0; rt < MRT; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int c = wave; c < nchunks; c += KW) {
    // load s of lane group g covers K = 128c + (32s + 8g) .. +8 (bf16) or
    // 128c + (16s + 4g) .. +4 (fp32): the four lane groups of a row read 64
    // contiguous bytes per instruction.  Each step's K range is a multiple
    // of 16 long and H of 32, so a step lies wholly inside or outside H.
    uint32_t kofs[XL];
#pragma unroll
    for (int s = 0; s < XL; ++s) {
      const int k0 = 128 * c + (BF16 ? 32 : 16) * s;
      kofs[s] = k0 < H ? uint32_t(k0 + (BF16 ? 8 : 4) * g) * EB : kOOB;
    }
    // every load of the chunk is issued before its first MFMA
    uint4 xq[XL];
#pragma unroll
    for (int s = 0; s < XL; ++s) xq[s] = buf_load_b128(xs, oob_add(xrow, kofs[s]));
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
      if (grp * RG < nrt) {  // uniform across the workgroup
        uint4 wq[RG][XL];
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          const int e = (grp * RG + r) * 16 + r16;
          const uint32_t wrow = e < E ? uint32_t(e) * row_bytes : kOOB;
#pragma unroll
          for (int s = 0; s < XL; ++s) wq[r][s] = buf_load_b128(wsrc, oob_add(wrow, kofs[s]));
        }
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

  // partial logits: accumulator element i of row tile rt is expert
  // rt*16 + 4g + i for token r16
  float* mine = part + (wave * kRouteTokens + r16) * E;
#pragma unroll
  for (int rt = 0; rt < MRT; ++rt) {
    if (rt < nrt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = rt * 16 + 4 * g + i;
        if (e < E) mine[e] = acc[rt][i];
      }
    }
  }
  __syncthreads();
  const int tile = kRouteTokens * E;
  for (int j = threadIdx.x; j < tile; j += 64 * KW) {
    const int e = j % E;
    float s = part[j];
    for (int w = 1; w < KW; ++w) s += part[w * tile + j];
    part[j] = s + load_param(a.b_r, e, a.act_bf16);
  }
  __syncthreads();

  // top-k + softmax: wave w handles tokens w, w + KW, ... of the tile
  for (int tl = wave; tl < kRouteTokens; tl += KW) {
    const int t = t0 + tl;
    if (t >= a.T) break;
    const float* lg = part + tl * E;
    float v[4];
    unsigned picked = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      float x = e < E ? lg[e] : -INFINITY;
      v[j] = (x != x) ? -INFINITY : x;  // a NaN logit ranks lowest
    }
    float sel_v[MAX_TOPK_DEV];
    int sel_i[MAX_TOPK_DEV];
#pragma unroll
    for (int kk = 0; kk < MAX_TOPK_DEV; ++kk) {
      sel_v[kk] = -INFINITY;
      sel_i[kk] = 0;
      if (kk < a.top_k) {
        float bv = -INFINITY;
        int bi = INT_MAX;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = lane + 64 * j;
          if (e < E && !((picked >> j) & 1u)) {
            if (v[j] > bv || (v[j] == bv && e < bi)) {
              bv = v[j];
              bi = e;
            }
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const float ov = __shfl_xor(bv, off);
          const int oi = __shfl_xor(bi, off);
          if (ov > bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
          }
        }
        sel_v[kk] = bv;
        sel_i[kk] = bi;
        if ((bi & 63) == lane) picked |= 1u << (bi >> 6);
      }
    }
    const float m = sel_v[0];
    float den = 0.f;
    float ex[MAX_TOPK_DEV];
#pragma unroll
    for (int kk = 0; kk < MAX_TOPK_DEV; ++kk) {
      ex[kk] = kk < a.top_k ? expf(sel_v[kk] - m) : 0.f;
      den += ex[kk];
    }
#pragma unroll
    for (int kk = 0; kk < MAX_TOPK_DEV; ++kk) {
      if (kk < a.top_k && lane == kk) {
        const float w = ex[kk] / den;
        const int64_t o = int64_t(t) * a.top_k + kk;
        a.idx[o] = sel_i[kk];
        a.wts[o] = w;
        if (a.idx_out) a.idx_out[o] = sel_i[kk];
        if (a.wts_out) a.wts_out[o] = w;
      }
    }
  }
}

template <bool BF16, int KW>
static void launch_route_typed(const RouteArgs& a, unsigned grid, hipStream_t stream) {
  const size_t lds = size_t(KW) * kRouteTokens * a.E * sizeof(float);
  const dim3 g(grid), b(64 * KW);
  // register tiles sized to E (fp32 operands take twice the registers)
  if (a.E <= 32)
    route_kernel<BF16, 2, 1, KW><<<g, b, lds, stream>>>(a);
  else if (a.E <= 64)
    route_kernel<BF16, 4, 1, KW><<<g, b, lds, stream>>>(a);
  else if (a.E <= 128)
    route_kernel<BF16, (BF16 ? 8 : 4), (BF16 ? 1 : 2), KW><<<g, b, lds, stream>>>(a);
  else if constexpr (KW == 4)  // E > 128 always takes 4 waves (LDS bound)
    route_kernel<BF16, 4, 4, KW><<<g, b, lds, stream>>>(a);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const unsigned grid = unsigned((a.T + kRouteTokens - 1) / kRouteTokens);
  // few token groups: more waves split K (shorter chains of dependent
  // loads per wave); many groups: 8 waves each up to E = 128.
  // The LDS of the partial logits, KW x 16 x E floats, stays <= 64 KB.
  if (grid < 64 && a.E <= 64) {
    if (a.act_bf16) launch_route_typed<true, 16>(a, grid, stream);
    else launch_route_typed<false, 16>(a, grid, stream);
  } else if (grid < 64 && a.E <= 128) {
    if (a.act_bf16) launch_route_typed<true, 8>(a, grid, stream);
    else launch_route_typed<false, 8>(a, grid, stream);
  } else if (MXMOE_ROUTE_KW_LARGE == 16 && a.E <= 64) {
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

__device__ __forceinline__ int wave_excl_scan(int v, int lane, int* total) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  *total = __shfl(x, 63);
  return x - v;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(PermuteArgs a) {
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
        if (c[j] > 0) a.active[1 + abase++] = e;
      }
      cbase += c[j];
      tbase += t[j];
    }
    if (lane == 0) {
      off[E] = ctot;
      a.offsets[E] = ctot;
      a.tile_off[E] = ttot;
      a.active[0] = atot;
      if (a.offsets_out) a.offsets_out[E] = ctot;
    }
  }
  __syncthreads();

  // prefill tile table: expert e owns tiles tile_off[e] .. tile_off[e+1)
  for (int e = tid; e < E; e += kPermThreads) {
    const int c = cnt[e];
    const int t0 = toff[e];
    for (int j = 0; j * kPrefillTokens < c; ++j)
      a.tiles[t0 + j] = make_int4(e, off[e] + j * kPrefillTokens, min(kPrefillTokens, c - j * kPrefillTokens), 0);
  }

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

// Expert-parallel grouping for large batches: workgroup e handles expert e.
// Every workgroup builds the full histogram in LDS (integer counts, order
// free) and scans it, which gives all offsets without a second launch; it
// then writes the entries of its own expert: offsets, count, tile range and
// tiles, its slot in the active list, and the stable positions of its
// slots.  For those, each wave takes a contiguous range of slots, counts its
// matches with ballots, takes a prefix over the waves, and sweeps the range
// again writing positions in slot order.
__global__ __launch_bounds__(kPermThreads) void permute_by_expert_kernel(PermuteArgs a) {
  __shared__ int cnt[256];
  __shared__ int s_off, s_toff, s_act;
  __shared__ int wsum[kPermWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, N = a.n_slots, me = blockIdx.x;

  for (int e = tid; e < 256; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  for (int s = tid; s < N; s += kPermThreads) {
    int e = a.idx[s];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    atomicAdd(&cnt[e], 1);
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
    if (me == 0 && lane == 0) {
      a.offsets[E] = ctot;
      a.tile_off[E] = ttot;
      a.active[0] = atot;
      if (a.offsets_out) a.offsets_out[E] = ctot;
    }
  }
  __syncthreads();
  const int c_me = cnt[me], off_me = s_off, toff_me = s_toff;
  if (tid == 0) {
    a.offsets[me] = off_me;
    a.counts[me] = c_me;
    a.tile_off[me] = toff_me;
    if (a.counts_out) a.counts_out[me] = c_me;
    if (a.offsets_out) a.offsets_out[me] = off_me;
    if (c_me > 0) a.active[1 + s_act] = me;
  }
  for (int j = tid; j * kPrefillTokens < c_me; j += kPermThreads)
    a.tiles[toff_me + j] = make_int4(me, off_me + j * kPrefillTokens, min(kPrefillTokens, c_me - j * kPrefillTokens), 0);

  // stable positions of this expert's slots
  const int per_wave = ((N + kPermWaves - 1) / kPermWaves + 63) & ~63;
  const int s0 = wave * per_wave, s1 = min(N, s0 + per_wave);
  int mine = 0;
  for (int b = s0; b < s1; b += 64) {
    const int s = b + lane;
    int key = -1;
    if (s < s1) {
      key = a.idx[s];
      key = key < 0 ? 0 : (key >= E ? E - 1 : key);
    }
    mine += __popcll(__ballot(key == me));
  }
  if (lane == 0) wsum[wave] = mine;
  __syncthreads();
  int run = off_me;
  for (int w = 0; w < wave; ++w) run += wsum[w];
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b = s0; b < s1; b += 64) {
    const int s = b + lane;
    int key = -1;
    if (s < s1) {
      key = a.idx[s];
      key = key < 0 ? 0 : (key >= E ? E - 1 : key);
    }
    const uint64_t m = __ballot(key == me);
    if (key == me) {
      const int p = run + __popcll(m & lt_mask);
      a.sorted[p] = s;
      a.sorted_tok[p] = s / a.top_k;
      a.pos[s] = p;
    }
    run += __popcll(m);
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

// --------------------------------------------------------------- FP8 quant
//
// code = sat448(rne_e4m3(fp32(x) * inv_scale)), inv_scale = 1 / s computed
// once in fp32 on the host (FP8 static per-tensor scheme).  8 values per
// thread: one 16-byte load, one 8-byte store.

__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint4* __restrict__ x, int64_t n8, float inv,
                                                        uint2* __restrict__ q) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 v = x[i];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16) * inv;
    f[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u) * inv;
  }
  q[i] = make_uint2(pack_e4m3x4(f[0], f[1], f[2], f[3]), pack_e4m3x4(f[4], f[5], f[6], f[7]));
}

// ------------------------------------------------------------- dense layer
//
// A dense layer runs through the grouped GEMMs as one expert that every
// token routes to once: expert 0 owns sorted rows 0 .. T-1 (the token rows
// themselves), in ceil(T / kPrefillTokens) prefill tiles.

__global__ __launch_bounds__(256) void linear_setup_kernel(int T, int32_t* offsets, int32_t* active, int32_t* tile_off,
                                                           int4* tiles, void* zero_bias, int N, int zero_bias_bytes) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int ntiles = (T + kPrefillTokens - 1) / kPrefillTokens;
  if (i == 0) {
    offsets[0] = 0;
    offsets[1] = T;
    active[0] = 1;
    active[1] = 0;
    tile_off[0] = 0;
    tile_off[1] = ntiles;
  }
  if (i < ntiles) tiles[i] = make_int4(0, i * kPrefillTokens, min(kPrefillTokens, T - i * kPrefillTokens), 0);
  if (zero_bias && i < N) {
    if (zero_bias_bytes == 2)
      static_cast<uint16_t*>(zero_bias)[i] = 0;
    else
      static_cast<float*>(zero_bias)[i] = 0.f;
  }
}

hipError_t launch_linear_setup(int T, int32_t* offsets, int32_t* active, int32_t* tile_off, int4* tiles,
                               void* zero_bias, int N, int zero_bias_bytes, hipStream_t stream) {
  const int ntiles = (T + kPrefillTokens - 1) / kPrefillTokens;
  const int n = ntiles > N ? ntiles : N;
  linear_setup_kernel<<<dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream>>>(T, offsets, active, tile_off, tiles,
                                                                               zero_bias, N, zero_bias_bytes);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const uint16_t* x, int64_t n, float inv_scale, uint8_t* q, hipStream_t stream) {
  const int64_t n8 = n / 8;  // n is a multiple of 32
  if (n8 == 0) return hipSuccess;
  quant_fp8_kernel<<<dim3(unsigned((n8 + 255) / 256)), dim3(256), 0, stream>>>(
      reinterpret_cast<const uint4*>(x), n8, inv_scale, reinterpret_cast<uint2*>(q));
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
