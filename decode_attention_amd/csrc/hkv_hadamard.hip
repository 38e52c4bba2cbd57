// hkv_hadamard.hip -- blockwise orthonormal Walsh-Hadamard rotation of rows.
//
// The rotation of the cache formats as an operation of its own: y =
// FWHT_B(x * s) (rotate) or y = FWHT_B(x) * s (unrotate) for every block of
// B = 64, 128 or 256 consecutive values of a row, with an optional +-1
// pattern s given as sign words (bit i of word k set: element 32k + i
// negated).  Sources: vLLM API docs "vllm.v1.attention.ops.rocm_octave"
// (fwht_blocks; signs / sign_bits; rotate before quantization and unrotate
// after), and Strata pull request #928, "What's in it" (a block-128 Hadamard
// rotation of activations for weights stored in a rotated basis).
//
// Blocks are independent and contiguous, so the kernel walks a flat array of
// blocks, 16 lanes to a block and four blocks per wave (the layout of
// fwht_rows16), with the loads of the next two groups of four in flight
// while it transforms the current one.
// Each lane loads and stores 16 contiguous bytes per 64-wide group.
#include <cmath>

#include "hkv_internal.h"

namespace hkv {
namespace {

constexpr int kHadWaves = 4;
constexpr int kHadMaxGroups = 2048;

template <int Q, bool F16>
__device__ __forceinline__ void had_load(const void* x, int64_t blk, uint32_t (&r)[Q][F16 ? 2 : 4]) {
  const int l = lane_id() & 15;
  constexpr int B = 64 * Q;
  if (F16) {
    const uint2* p = (const uint2*)((const uint16_t*)x + blk * B + 4 * l);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const uint2 a = p[16 * q];
      r[q][0] = a.x, r[q][1] = a.y;
    }
  } else {
    const uint4* p = (const uint4*)((const float*)x + blk * B + 4 * l);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const uint4 a = p[16 * q];
      r[q][0] = a.x, r[q][1] = a.y, r[q][2] = a.z, r[q][3] = a.w;
    }
  }
}

// The four sign bits of elements 64q + 4l .. 64q + 4l + 3 of block position
// `pos` in the row, as fp32 sign masks.
template <int Q>
__device__ __forceinline__ void had_signs(const uint32_t* sign_bits, int pos, uint32_t (&m)[Q][4]) {
  const int l = lane_id() & 15;
  constexpr int B = 64 * Q;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int d = pos * B + 64 * q + 4 * l;
    const uint32_t w = sign_bits[d >> 5] >> (d & 31);
#pragma unroll
    for (int i = 0; i < 4; ++i) m[q][i] = ((w >> i) & 1u) << 31;
  }
}

// Rotates the four blocks whose raw words are in r (this lane-row's block
// `cur`) and stores them.
template <int Q, bool F16, bool SIGNS, bool INV>
__device__ __forceinline__ void had_block(const uint32_t (&r)[Q][F16 ? 2 : 4], int64_t cur,
                                          int64_t nblk, int bpr, float norm,
                                          const uint32_t* sign_bits, float* y) {
  const int l = lane_id() & 15;
  float v[Q][4];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (F16) {
      v[q][0] = h2f((uint16_t)r[q][0]);
      v[q][1] = h2f((uint16_t)(r[q][0] >> 16));
      v[q][2] = h2f((uint16_t)r[q][1]);
      v[q][3] = h2f((uint16_t)(r[q][1] >> 16));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[q][i] = __uint_as_float(r[q][i]);
    }
  }
  uint32_t sm[Q][4];
  if (SIGNS) {
    const int64_t c = min(cur, nblk - 1);
    const int pos = (c >> 31) == 0 ? (int)((uint32_t)c % (uint32_t)bpr) : (int)(c % bpr);
    had_signs<Q>(sign_bits, pos, sm);
  }
  if (SIGNS && !INV) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[q][i] = __uint_as_float(__float_as_uint(v[q][i]) ^ sm[q][i]);
  }
  fwht_rows16<Q>(v, norm);
  if (SIGNS && INV) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[q][i] = __uint_as_float(__float_as_uint(v[q][i]) ^ sm[q][i]);
  }
  if (cur < nblk) {
    float4* p = (float4*)(y + cur * (64 * Q) + 4 * l);
#pragma unroll
    for (int q = 0; q < Q; ++q) p[16 * q] = make_float4(v[q][0], v[q][1], v[q][2], v[q][3]);
  }
}

// nblk = rows * n / B blocks; block b is row b / bpr, position b % bpr.  Each
// wave keeps two groups of four blocks in flight: while it rotates one, the
// loads of the next two are outstanding.
template <int Q, bool F16, bool SIGNS, bool INV>
__global__ __launch_bounds__(kHadWaves * kWave) void hadamard_kernel(
    const void* x, float* y, int64_t nblk, int bpr, float norm, const uint32_t* sign_bits) {
  constexpr int R = F16 ? 2 : 4;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t stride = (int64_t)gridDim.x * kHadWaves * 4;
  int64_t base = ((int64_t)blockIdx.x * kHadWaves + wave) * 4;
  if (base >= nblk) return;
  int64_t blk = base + (lane >> 4);
  uint32_t ra[Q][R], rb[Q][R];
  had_load<Q, F16>(x, min(blk, nblk - 1), ra);
  if (base + stride < nblk) had_load<Q, F16>(x, min(blk + stride, nblk - 1), rb);
  for (;;) {
    // group at `base` is in ra, group at base + stride (if any) in rb
    uint32_t cur[Q][R];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < R; ++i) cur[q][i] = ra[q][i];
    if (base + 2 * stride < nblk) had_load<Q, F16>(x, min(blk + 2 * stride, nblk - 1), ra);
    had_block<Q, F16, SIGNS, INV>(cur, blk, nblk, bpr, norm, sign_bits, y);
    base += stride;
    blk += stride;
    if (base >= nblk) break;
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < R; ++i) cur[q][i] = rb[q][i];
    if (base + 2 * stride < nblk) had_load<Q, F16>(x, min(blk + 2 * stride, nblk - 1), rb);
    had_block<Q, F16, SIGNS, INV>(cur, blk, nblk, bpr, norm, sign_bits, y);
    base += stride;
    blk += stride;
    if (base >= nblk) break;
  }
}

template <int Q, bool F16>
hipError_t launch_q(const void* x, float* y, int64_t nblk, int bpr, float norm,
                    const uint32_t* sign_bits, bool inverse, hipStream_t s) {
  const int64_t groups = (nblk + 4 * kHadWaves - 1) / (4 * kHadWaves);
  const dim3 grid((unsigned)(groups < kHadMaxGroups ? groups : kHadMaxGroups));
  const dim3 block(kHadWaves * kWave);
  if (!sign_bits)
    hadamard_kernel<Q, F16, false, false><<<grid, block, 0, s>>>(x, y, nblk, bpr, norm, nullptr);
  else if (inverse)
    hadamard_kernel<Q, F16, true, true><<<grid, block, 0, s>>>(x, y, nblk, bpr, norm, sign_bits);
  else
    hadamard_kernel<Q, F16, true, false><<<grid, block, 0, s>>>(x, y, nblk, bpr, norm, sign_bits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hadamard(const void* x, bool in_f16, float* y, int64_t rows, int n, int block,
                           const uint32_t* sign_bits, bool inverse, hipStream_t s) {
  const int64_t nblk = rows * (n / block);
  if (nblk == 0) return hipSuccess;
  const int bpr = n / block;
  // fp32(1/sqrt(block)), computed as for the cache formats
  const float norm = (float)(1.0 / std::sqrt((double)block));
  switch (block) {
    case 64:
      return in_f16 ? launch_q<1, true>(x, y, nblk, bpr, norm, sign_bits, inverse, s)
                    : launch_q<1, false>(x, y, nblk, bpr, norm, sign_bits, inverse, s);
    case 128:
      return in_f16 ? launch_q<2, true>(x, y, nblk, bpr, norm, sign_bits, inverse, s)
                    : launch_q<2, false>(x, y, nblk, bpr, norm, sign_bits, inverse, s);
    case 256:
      return in_f16 ? launch_q<4, true>(x, y, nblk, bpr, norm, sign_bits, inverse, s)
                    : launch_q<4, false>(x, y, nblk, bpr, norm, sign_bits, inverse, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace hkv
