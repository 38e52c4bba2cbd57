// hkv_probe.hip -- measurement aid, not part of the library: a plain
// streaming-read kernel that gives the HBM read bandwidth this GPU actually
// delivers to a simple 16-byte-per-lane load loop, reported beside the
// 8 TB/s peak by the benchmark.
//
// Every thread walks the buffer with a grid stride, eight nontemporal 16-byte
// loads in flight per iteration (the fastest of the shapes tried: 1024-16384
// workgroups, 4/8/16 loads, cached or nontemporal), folds the words with xor
// (so the loads cannot be dropped) and writes one word per thread.
//
// It also holds a check of the library's reciprocal and x / 127 (recip_rn
// and div127_rn in hkv_device.h) against the IEEE quotients over every
// float, and of its square root for large arguments (sqrt_rn_large) against
// sqrtf, which the quantizers' bit-exactness rests on.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hkv_device.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* src, int64_t n16,
                                                               uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_nontemporal_load((const u32x4*)(src + i + u * stride));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// recip_rn(x) against 1.0f / x and div127_rn(x) against x / 127.0f, bit for
// bit, for the 2^31 float bit patterns base .. base + 2^31 - 1: out[0] and
// out[9] count the mismatches, out[1..8] and out[10..17] hold the first ones
// found.
__global__ __launch_bounds__(kThreads) void recip_check_kernel(uint32_t base, uint32_t* out) {
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < 0x80000000u; i += stride) {
    const uint32_t u = base + i;
    const float x = __uint_as_float(u);
    if (__float_as_uint(hkv::recip_rn(x)) != __float_as_uint(1.0f / x)) {
      const uint32_t k = atomicAdd(&out[0], 1u);
      if (k < 8) out[1 + k] = u;
    }
    if (__float_as_uint(hkv::div127_rn(x)) != __float_as_uint(x / 127.0f)) {
      const uint32_t k = atomicAdd(&out[9], 1u);
      if (k < 8) out[10 + k] = u;
    }
  }
}

// sqrt_rn_large(x) against sqrtf(x), bit for bit, for x = +0 and the 2^31
// bit patterns base .. base + 2^31 - 1 that are finite and at least 2^-96:
// out[0] counts the mismatches, out[1..8] hold the first ones found.
__global__ __launch_bounds__(kThreads) void sqrt_check_kernel(uint32_t base, uint32_t* out) {
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < 0x80000000u; i += stride) {
    const uint32_t u = base + i;
    if (!(u == 0u || (u >= 0x0F800000u && u <= 0x7F7FFFFFu))) continue;
    const float x = __uint_as_float(u);
    if (__float_as_uint(hkv::sqrt_rn_large(x)) != __float_as_uint(sqrtf(x))) {
      const uint32_t k = atomicAdd(&out[0], 1u);
      if (k < 8) out[1 + k] = u;
    }
  }
}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 16, 16-byte aligned) from src with `blocks`
// workgroups of 256 threads; sink holds blocks * 256 words.  Returns 0 on a
// successful launch.
int hkv_probe_stream_read(const void* src, int64_t bytes, int32_t blocks, uint32_t* sink,
                          void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 || blocks <= 0) return 1;
  stream_read_kernel<<<blocks, kThreads, 0, (hipStream_t)stream>>>((const uint4*)src, bytes / 16,
                                                                   sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Runs the reciprocal and the x / 127 checks over all 2^32 float bit
// patterns; out is 18 device words, zeroed by the caller (per check: the
// mismatch count, then the first mismatches).
int hkv_probe_recip_check(uint32_t* out, void* stream) {
  if (!out) return 1;
  for (uint32_t half = 0; half < 2; ++half)
    recip_check_kernel<<<4096, kThreads, 0, (hipStream_t)stream>>>(half << 31, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Runs the square-root check over the non-negative float bit patterns (the
// first half); out is 9 device words, zeroed by the caller.
int hkv_probe_sqrt_check(uint32_t* out, void* stream) {
  if (!out) return 1;
  sqrt_check_kernel<<<4096, kThreads, 0, (hipStream_t)stream>>>(0u, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
}
