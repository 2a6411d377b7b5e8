// Top-k selection and lane helpers shared by the router kernels of the
// MXFP4 MoE layer (gfx950).
#pragma once

#include <climits>

#include "device_common.h"

namespace mxmoe {

// ------------------------------------------------------ top-k selection
//
// Order of the experts: larger logit first, the lower index first among
// equal logits (a NaN logit counts as -inf).  Both parts sit in one 64-bit
// key that compares as an unsigned integer: the high word is the logit
// mapped onto uint32 in the same order (-0 taken as +0, which ties with it
// anyway), the low word is ~expert.  Key 0 ranks below every expert.
//
// Each of the L lanes of a token keeps the KM best keys of its strided
// share of the logits as a sorted list; the lists are then merged pairwise,
// log2(L) times, until every lane holds the KM best of all E.  Merging two
// sorted lists A, B of disjoint experts: C[j] = max(A[j], B[KM-1-j]) is the
// KM best of the union as a bitonic sequence, which a bitonic merge network
// sorts.  Pairing: DPP row rotations by 1, 2, 4, 8 inside a 16-lane row
// (lane i then holds lanes i..i-15 of its row, each merge combining disjoint
// sets), then lane XOR 16 and 32 across rows.

__device__ __forceinline__ uint64_t expert_key(float x, int e) {
  x = (x != x) ? -INFINITY : (x == 0.f ? 0.f : x);
  const uint32_t u = __float_as_uint(x);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t(o) << 32) | uint32_t(~uint32_t(e));
}

__device__ __forceinline__ float key_logit(uint64_t k) {
  const uint32_t o = uint32_t(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ int key_expert(uint64_t k) { return int(~uint32_t(k)); }

template <int KM>
__device__ __forceinline__ void list_insert(uint64_t (&l)[KM], uint64_t x) {
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const uint64_t hi = l[j] > x ? l[j] : x;
    x = l[j] > x ? x : l[j];
    l[j] = hi;
  }
}

template <int KM>
__device__ __forceinline__ void list_merge(uint64_t (&l)[KM], const uint64_t (&p)[KM]) {
#pragma unroll
  for (int j = 0; j < KM; ++j) l[j] = l[j] > p[KM - 1 - j] ? l[j] : p[KM - 1 - j];
#pragma unroll
  for (int st = KM / 2; st >= 1; st >>= 1) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if ((j & st) == 0) {
        const uint64_t a0 = l[j], a1 = l[j + st];
        l[j] = a0 > a1 ? a0 : a1;
        l[j + st] = a0 > a1 ? a1 : a0;
      }
    }
  }
}

// the key of lane (i - R) mod 16 of this lane's 16-lane row
template <int R>
__device__ __forceinline__ uint64_t row_rotated(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(x)), 0x120 + R, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(x >> 32)), 0x120 + R, 0xF, 0xF, false);
  return (uint64_t(hi) << 32) | lo;
}

template <int R, int KM>
__device__ __forceinline__ void merge_rotated(uint64_t (&l)[KM]) {
  uint64_t p[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) p[j] = row_rotated<R>(l[j]);
  list_merge<KM>(l, p);
}

template <int KM>
__device__ __forceinline__ void merge_xor(uint64_t (&l)[KM], int mask) {
  uint64_t p[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const uint32_t lo = uint32_t(__shfl_xor(int(uint32_t(l[j])), mask));
    const uint32_t hi = uint32_t(__shfl_xor(int(uint32_t(l[j] >> 32)), mask));
    p[j] = (uint64_t(hi) << 32) | lo;
  }
  list_merge<KM>(l, p);
}

// Top-k of token t's logits (lg[256*(e/16) + 64*((e/4)%4) + e%4] for expert
// e) by the L lanes of its group, then the softmax over those k; the first
// k lanes of the group write the outputs.

// The KM best keys of one token's logits (lg[256*(e/16) + 64*((e/4)%4) +
// e%4] for expert e < E), found by the L lanes of its group: lane q starts
// from its strided share of the experts; after the merges every lane of the
// group holds the same sorted list.
template <int KM, int L>
__device__ __forceinline__ void topk_keys(const float* lg, int E, int q, uint64_t (&l)[KM]) {
  static_assert(L == 16 || L == 32 || L == 64, "a token's lanes are whole 16-lane rows");
#pragma unroll
  for (int j = 0; j < KM; ++j) l[j] = 0;
  for (int e = q; e < E; e += L) list_insert<KM>(l, expert_key(lg[256 * (e >> 4) + 64 * ((e >> 2) & 3) + (e & 3)], e));
  merge_rotated<1, KM>(l);
  merge_rotated<2, KM>(l);
  merge_rotated<4, KM>(l);
  merge_rotated<8, KM>(l);
  if constexpr (L >= 32) merge_xor<KM>(l, 16);
  if constexpr (L >= 64) merge_xor<KM>(l, 32);
}

// Softmax over the first k keys of a sorted list (k <= KM): ex[kk] =
// exp(logit_kk - logit_0) and their sum in kk order; weight kk is
// ex[kk] / den.
template <int KM>
__device__ __forceinline__ float topk_softmax_terms(const uint64_t (&l)[KM], int k, float (&ex)[KM]) {
  const float m = key_logit(l[0]);
  float den = 0.f;
#pragma unroll
  for (int kk = 0; kk < KM; ++kk) {
    ex[kk] = kk < k ? expf(key_logit(l[kk]) - m) : 0.f;
    den += ex[kk];
  }
  return den;
}

// Exclusive prefix sum of v over the 64 lanes of a wave; *total gets the sum.
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

// The 16 bytes of source lane (perm / 4), for every lane.
__device__ __forceinline__ uint4 lane_permute(uint4 v, int perm) {
  return make_uint4(uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(v.x))),
                    uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(v.y))),
                    uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(v.z))),
                    uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(v.w))));
}

}  // namespace mxmoe
