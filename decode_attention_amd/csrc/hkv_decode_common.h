// hkv_decode_common.h -- arguments and wave helpers shared by the decode
// kernels (generic split-K kernel, the MFMA kernels and the split merge).
#pragma once

#include "hkv_internal.h"

namespace hkv {

constexpr int kWaves = 4;
constexpr int kTile = 64;
constexpr float kLog2e = 1.4426950408889634f;

struct DecArgs {
  const void* query;
  int q_f16;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int n_q;
  int rows;
  int rows_pad;     // rows rounded up to the kernel's row count (partial records per split)
  int num_queries;
  const uint8_t* cache;
  const int32_t* block_table;
  int max_pages;
  const int32_t* q_to_req;
  const int32_t* q_to_klen;
  float q_scale;  // sm_scale * log2(e): scores live in the exp2 domain
  int tokens_per_split;
  int num_splits;
  float* ws;
  int pstride;    // floats per partial record: 4 + D (m, l, pad, pad, o[D])
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// Partial record of one (query row, split): m, l, two pad words, o[D].
constexpr int kPartialHead = 4;

}  // namespace hkv
