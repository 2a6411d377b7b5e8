// MXFP4 unpack (dequantise) and pack (quantise) kernels for gfx950.
//
// Format (KerasFormers "mxfp4" page, intro and "Primitives"): a row of K
// values is K/32 blocks of 16 bytes, element 32*b + 2*j + n being nibble n
// (low first) of byte j of block b, e2m1 with bit 3 the sign, times
// 2^(e8m0 - 127) from the block's scale byte.
#include "device_common.h"
#include "launch.h"

namespace mxmoe {

// ---------------------------------------------------------------- unpack
//
// HBM-bound: 17 bytes in, 64 (bf16) or 128 (fp32) bytes out per block.  The
// decode is the packed hardware conversion (exact for every byte and scale,
// including s = 0 -> 2^-127, s = 255 -> NaN and overflow -> Inf).  fp32
// output: each thread owns one 16-byte block (one 128-bit load, one scale
// byte, eight 128-bit stores).

__global__ __launch_bounds__(256) void unpack_f32_kernel(const u32x4_t* __restrict__ blocks,
                                                         const uint8_t* __restrict__ scales,
                                                         f32x4_t* __restrict__ out, int64_t nblocks) {
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= nblocks) return;
  const u32x4_t w = __builtin_nontemporal_load(blocks + i);
  const float sc = e8m0_as_scale_operand(scales[i]);
  f32x4_t* o = out + i * 8;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2_t a = fp4x2_to_f32x2<0>(w[d], sc);
    const f32x2_t b = fp4x2_to_f32x2<1>(w[d], sc);
    const f32x2_t c = fp4x2_to_f32x2<2>(w[d], sc);
    const f32x2_t e = fp4x2_to_f32x2<3>(w[d], sc);
    __builtin_nontemporal_store(f32x4_t{a[0], a[1], b[0], b[1]}, o + 2 * d);
    __builtin_nontemporal_store(f32x4_t{c[0], c[1], e[0], e[1]}, o + 2 * d + 1);
  }
}

// bf16 output with whole-wave stores: a wave owns 64 consecutive blocks
// (1 KB in, 4 KB out).  Store d of lane l writes output bytes
// [1 KB * d + 16 l, +16), which is quarter l % 4 of block 16 d + l / 4: the 8
// values of dword l % 4 of that block.  So each of the four dword loads of a
// lane is part of one contiguous 256-byte wave read, and each 16-byte store
// part of one contiguous 1 KB wave write.
__global__ __launch_bounds__(256) void unpack_bf16_kernel(const uint32_t* __restrict__ blocks,
                                                          const uint8_t* __restrict__ scales,
                                                          u32x4_t* __restrict__ out, int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int64_t b0 = ((int64_t(blockIdx.x) * 256 + threadIdx.x) >> 6) * 64;
  const int q = lane & 3;
  uint32_t w[4];
  float sc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int64_t blk = b0 + 16 * d + (lane >> 2);
    w[d] = 0;
    sc[d] = 0.f;
    if (blk < nblocks) {
      w[d] = __builtin_nontemporal_load(blocks + blk * 4 + q);
      sc[d] = e8m0_as_scale_operand(scales[blk]);
    }
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int64_t blk = b0 + 16 * d + (lane >> 2);
    if (blk < nblocks) {
      u32x4_t r;
      r[0] = fp4x2_to_bf16x2<0>(w[d], sc[d]);
      r[1] = fp4x2_to_bf16x2<1>(w[d], sc[d]);
      r[2] = fp4x2_to_bf16x2<2>(w[d], sc[d]);
      r[3] = fp4x2_to_bf16x2<3>(w[d], sc[d]);
      __builtin_nontemporal_store(r, out + blk * 4 + q);
    }
  }
}

hipError_t launch_unpack(const uint8_t* blocks, const uint8_t* scales, int64_t nblocks, void* out, bool out_bf16,
                         hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;
  int64_t grid = (nblocks + 255) / 256;
  if (out_bf16)
    unpack_bf16_kernel<<<dim3(unsigned(grid)), dim3(256), 0, stream>>>(reinterpret_cast<const uint32_t*>(blocks), scales,
                                                                      static_cast<u32x4_t*>(out), nblocks);
  else
    unpack_f32_kernel<<<dim3(unsigned(grid)), dim3(256), 0, stream>>>(reinterpret_cast<const u32x4_t*>(blocks), scales,
                                                                     static_cast<f32x4_t*>(out), nblocks);
  return hipGetLastError();
}

// ------------------------------------------------------------------ pack
//
// One thread per 32-value block ("Primitives": quantize).  The block
// exponent e = floor(log2(amax)) - 2 is read from the float's exponent
// field (subnormal amax via the leading-zero count), clamped to
// [-127, 127]; v = w * 2^-e is exact, and its magnitude maps to the FP4 code
// index by counting the rounding thresholds it passes.  The thresholds are
// the midpoints between neighbouring grid values; '>' at a midpoint whose
// lower neighbour has an even index and '>=' where the upper one does give
// round-half-to-even on the code.

__device__ __forceinline__ uint32_t fp4_index_of_magnitude(float a) {
  return uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
         uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
}

__device__ __forceinline__ int floor_log2_abs(float amax) {
  uint32_t u = __float_as_uint(amax) & 0x7FFFFFFFu;
  int ef = int(u >> 23);
  if (ef > 0) return ef - 127;
  // subnormal: value = m * 2^-149 with m = u (nonzero)
  return (31 - __clz(u)) - 149;
}

template <bool IN_BF16>
__global__ __launch_bounds__(256) void pack_kernel(const void* __restrict__ w, uint8_t* __restrict__ blocks,
                                                   uint8_t* __restrict__ scales, int64_t nblocks) {
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= nblocks) return;
  float v[32];
  if constexpr (IN_BF16) {
    const uint4* p = static_cast<const uint4*>(w) + i * 4;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint4 q = p[d];
      uint32_t qs[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[d * 8 + t * 2] = __uint_as_float(qs[t] << 16);
        v[d * 8 + t * 2 + 1] = __uint_as_float(qs[t] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = static_cast<const float4*>(w) + i * 8;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      float4 q = p[d];
      v[d * 4 + 0] = q.x;
      v[d * 4 + 1] = q.y;
      v[d * 4 + 2] = q.z;
      v[d * 4 + 3] = q.w;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int t = 0; t < 32; ++t) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[t]));
  int e = amax > 0.0f ? floor_log2_abs(amax) - 2 : -127;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  uint32_t words[4] = {0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    float a = __builtin_amdgcn_ldexpf(__builtin_fabsf(v[t]), -e);
    uint32_t nib = fp4_index_of_magnitude(a) | ((__float_as_uint(v[t]) >> 28) & 8u);
    words[t / 8] |= nib << (4 * (t % 8));
  }
  reinterpret_cast<uint4*>(blocks)[i] = make_uint4(words[0], words[1], words[2], words[3]);
  scales[i] = uint8_t(e + 127);
}

hipError_t launch_pack(const void* w, bool in_bf16, int64_t nblocks, uint8_t* blocks, uint8_t* scales,
                       hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;
  int64_t grid = (nblocks + 255) / 256;
  if (in_bf16)
    pack_kernel<true><<<dim3(unsigned(grid)), dim3(256), 0, stream>>>(w, blocks, scales, nblocks);
  else
    pack_kernel<false><<<dim3(unsigned(grid)), dim3(256), 0, stream>>>(w, blocks, scales, nblocks);
  return hipGetLastError();
}

// ------------------------------------------------------------------ tile
//
// Row order -> tiled order (declared in mxmoe.h).  A one-time layout step:
// one thread per 16-byte piece of the tiled blocks and one per dword of the
// tiled scales, so the writes stream contiguously and the reads gather.

__global__ __launch_bounds__(256) void tile_blocks_kernel(const uint4* __restrict__ blocks, uint4* __restrict__ out,
                                                          int rows, int nb, int rt4, int nc, int64_t total) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int s = int(i & 63);
  int64_t p = i >> 6;  // piece (m, t, c)
  const int c = int(p % nc);
  p /= nc;
  const int t = int(p % rt4);
  const int64_t m = p / rt4;
  const int r = s >> 2;
  const int b = (s & 3) ^ ((r >> 2) & 3);  // inverse of the slot swizzle
  const int row = 16 * t + r, blk = 4 * c + b;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < rows && blk < nb) v = blocks[(m * rows + row) * nb + blk];
  out[i] = v;
}

__global__ __launch_bounds__(256) void tile_scales_kernel(const uint8_t* __restrict__ scales,
                                                          uint32_t* __restrict__ out, int rows, int nb, int rg,
                                                          int nc, int64_t total) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int l = int(i & 63);
  int64_t p = i >> 6;  // group (m, q, c)
  const int c = int(p % nc);
  p /= nc;
  const int q = int(p % rg);
  const int64_t m = p / rg;
  const int b = l >> 4, r = l & 15;
  const int blk = 4 * c + b;
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 64 * q + 16 * j + r;
    if (row < rows && blk < nb) v |= uint32_t(scales[(m * rows + row) * nb + blk]) << (8 * j);
  }
  out[i] = v;
}

// 8-bit weights (mats, N, K) (e4m3 or int8 codes), row-major -> the tiled
// 8-bit order: for matrix m, row tile t (16 rows), chunk c (128 K) and lane
// l = 16g + r, 32 bytes: row 16t + r, K bytes 128c + 16g .. +16 then
// 128c + 64 + 16g .. +16 (zeros past N or K).  One thread per 16-byte half
// of a lane's piece.
__global__ __launch_bounds__(256) void byte_tile_kernel(const uint8_t* __restrict__ w, uint4* __restrict__ out, int N,
                                                       int K, int rt4, int nc, int64_t total) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int h = int(i & 1), l = int((i >> 1) & 63);
  const int64_t tc = i >> 7;  // (matrix, row tile, chunk)
  const int c = int(tc % nc);
  const int64_t mt = tc / nc;
  const int t = int(mt % rt4);
  const int64_t m = mt / rt4;
  const int row = 16 * t + (l & 15);
  const int k0 = 128 * c + 64 * h + 16 * (l >> 4);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < N && k0 < K) v = *reinterpret_cast<const uint4*>(w + (m * N + row) * int64_t(K) + k0);
  out[i] = v;
}

hipError_t launch_byte_tile(const uint8_t* w, int64_t mats, int N, int K, uint8_t* out, hipStream_t stream) {
  const int rt4 = 4 * ((N + 63) / 64), nc = (K + 127) / 128;
  const int64_t halves = mats * int64_t(rt4) * nc * 128;
  if (halves == 0) return hipSuccess;
  byte_tile_kernel<<<dim3(unsigned((halves + 255) / 256)), dim3(256), 0, stream>>>(w, reinterpret_cast<uint4*>(out), N,
                                                                                  K, rt4, nc, halves);
  return hipGetLastError();
}

hipError_t launch_tile(const uint8_t* blocks, const uint8_t* scales, int64_t mats, int rows, int nb,
                       uint8_t* tiled_blocks, uint8_t* tiled_scales, hipStream_t stream) {
  const int rg = (rows + 63) / 64, nc = (nb + 3) / 4;
  const int64_t pieces = mats * int64_t(4 * rg) * nc * 64;  // 16-byte pieces
  const int64_t words = mats * int64_t(rg) * nc * 64;       // scale dwords
  if (pieces == 0) return hipSuccess;
  tile_blocks_kernel<<<dim3(unsigned((pieces + 255) / 256)), dim3(256), 0, stream>>>(
      reinterpret_cast<const uint4*>(blocks), reinterpret_cast<uint4*>(tiled_blocks), rows, nb, 4 * rg, nc, pieces);
  tile_scales_kernel<<<dim3(unsigned((words + 255) / 256)), dim3(256), 0, stream>>>(
      scales, reinterpret_cast<uint32_t*>(tiled_scales), rows, nb, rg, nc, words);
  return hipGetLastError();
}

}  // namespace mxmoe
