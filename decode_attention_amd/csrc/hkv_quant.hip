// hkv_quant.hip -- quantize-append and dequantize kernels.
//
// One wave (a 64-thread workgroup) per (token, KV head).  The head vector
// lives "strided" in registers (register e of lane l = element 64e + l), is
// sign-flipped and Walsh-Hadamard rotated in registers, quantized with wave
// reductions, and the slot is assembled in LDS and written with 4-byte
// stores (consecutive lanes -> consecutive words).
//
// Sources: vLLM API docs "vllm.v1.attention.ops.rocm_octave"
// (reference_quantize, _quantize_lut, _pack, reference_dequantize) and Strata
// pull request #21 (Q4_0 block with one fp16 scale per 32 values; the max-abs
// tie-break of the merge note).
#include "hkv_internal.h"

namespace hkv {
namespace {

// Code = number of codebook midpoints strictly below y (a value on a
// midpoint takes the lower code: torch.bucketize with right=False), and the
// codebook value of that code.
template <int BITS>
__device__ __forceinline__ int bucket(float y, int* lv) {
  int code = 0;
  int val = (BITS == 3) ? kLut3[0] : kLut4[0];
  constexpr int N = 1 << BITS;
#pragma unroll
  for (int k = 0; k + 1 < N; ++k) {
    const float mid = (BITS == 3) ? (float)(kLut3[k] + kLut3[k + 1]) * 0.5f
                                  : (float)(kLut4[k] + kLut4[k + 1]) * 0.5f;
    const bool above = mid < y;
    code += above ? 1 : 0;
    val = above ? ((BITS == 3) ? kLut3[k + 1] : kLut4[k + 1]) : val;
  }
  *lv = val;
  return code;
}

// Sum of t[e0 .. e0+nreg) over all lanes in the canonical tree order:
// registers first (halving folds when nreg is a power of two, else left to
// right), then the 64 lanes as a pairwise tree.
template <int E>
__device__ __forceinline__ float block_tree_sum(float (&t)[E], int e0, int nreg) {
  float acc;
  if ((nreg & (nreg - 1)) == 0) {
    float u[E];
#pragma unroll
    for (int e = 0; e < E; ++e) u[e] = t[e];
#pragma unroll
    for (int half = E / 2; half >= 1; half >>= 1) {
      if (half * 2 <= nreg) {
#pragma unroll
        for (int e = 0; e < half; ++e) u[e0 + e] = u[e0 + e] + u[e0 + e + half];
      }
    }
    acc = u[e0];
  } else {
    acc = t[e0];
#pragma unroll
    for (int e = 1; e < E; ++e)
      if (e < nreg) acc = acc + t[e0 + e];
  }
  return wave_tree_sum(acc);
}

// Octave quantizer (_quantize_lut) over registers [e0, e0+nreg) of a strided
// vector: block RMS, nearest Lloyd-Max code, scale with x . x_hat = |x|^2.
template <int E, int BITS>
__device__ __forceinline__ uint16_t octave_block(const float (&x)[E], int e0, int nreg,
                                                 uint8_t* codes_lds) {
  const int lane = lane_id();
  float t[E];
#pragma unroll
  for (int e = 0; e < E; ++e) t[e] = x[e] * x[e];
  const float ss = block_tree_sum<E>(t, e0, nreg);
  float rms = sqrtf(ss / (float)(nreg * kWave));
  rms = rms < 1e-12f ? 1e-12f : rms;
  const float mult = (float)(BITS == 3 ? kLutMult3 : kLutMult4);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    t[e] = 0.0f;
    if (e >= e0 && e < e0 + nreg) {
      const float y = (x[e] / rms) * mult;
      int lv;
      const int c = bucket<BITS>(y, &lv);
      codes_lds[kWave * e + lane] = (uint8_t)c;
      t[e] = x[e] * (float)lv;
    }
  }
  const float dot = block_tree_sum<E>(t, e0, nreg);
  float sc = 0.0f;
  if (dot > 0.0f) sc = ss / (dot > 1e-30f ? dot : 1e-30f);
  return f2h(sc * (float)kLutOne);
}

// Q4_0 over one 32-value block = one half-register (lanes 0-31 or 32-63).
// Max-abs element with the tie-break (larger magnitude; equal magnitudes keep
// the larger signed value); d = m / -8; code = min(15, trunc(x/d + 8.5)).
__device__ __forceinline__ uint16_t q4_block(float x, uint8_t* code_lds) {
  float a = fabsf(x), m = x;
#pragma unroll
  for (int s = 16; s >= 1; s >>= 1) {
    const float a2 = shfl_xor(a, s), m2 = shfl_xor(m, s);
    if (a2 > a || (a2 == a && m2 > m)) {
      a = a2;
      m = m2;
    }
  }
  if (a == 0.0f) m = 0.0f;  // an all-zero block keeps the initial +0 of the scan
  const float d = m / -8.0f;
  const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  const float u = x * id + 8.5f;
  int c = (int)u;
  c = c > 15 ? 15 : c;
  *code_lds = (uint8_t)c;
  return f2h(d);
}

__device__ __forceinline__ uint32_t pack4_word(const uint8_t* c, int w) {
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    word |= (uint32_t)((c[8 * w + j] & 15) | ((c[8 * w + 4 + j] & 15) << 4)) << (8 * j);
  return word;
}

// Word at byte offset o of a 3-bit segment of n codes.
__device__ __forceinline__ uint32_t pack3_word(const uint8_t* c, int n, int o) {
  uint32_t word = 0;
  if (o < n / 4) {
    const int m = o / 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t b = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) b |= (uint32_t)(c[16 * m + 4 * i + j] & 3) << (2 * i);
      word |= b << (8 * j);
    }
  } else {
    const int m = (o - n / 4) / 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t b = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) b |= (uint32_t)((c[32 * m + 4 * i + j] >> 2) & 1) << i;
      word |= b << (8 * j);
    }
  }
  return word;
}

template <int E>
__device__ __forceinline__ void load_row(const void* src, bool f16, int64_t row, float (&x)[E]) {
  const int lane = lane_id();
  if (f16) {
    const uint16_t* p = (const uint16_t*)src + row * (E * kWave);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = h2f(p[kWave * e + lane]);
  } else {
    const float* p = (const float*)src + row * (E * kWave);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = p[kWave * e + lane];
  }
}

template <int E>
__global__ __launch_bounds__(64) void quantize_append_kernel(DevFmt f, const void* key,
                                                             const void* value, int in_f16,
                                                             int num_kv_heads,
                                                             const int64_t* slot_mapping,
                                                             uint8_t* cache) {
  const int64_t row = blockIdx.x;
  const int64_t t = row / num_kv_heads;
  const int h = (int)(row % num_kv_heads);
  const int64_t sm = slot_mapping[t];
  if (sm < 0) return;
  const int lane = lane_id();
  __shared__ uint8_t kc[E * kWave];
  __shared__ uint8_t vc[E * kWave];
  __shared__ uint16_t sc[2 * kMaxHead / 32 + 2];

  float k[E], v[E];
  load_row<E>(key, in_f16 != 0, row, k);
  load_row<E>(value, in_f16 != 0, row, v);
  if (f.use_signs) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      k[e] = apply_sign(f, k[e], kWave * e + lane);
      v[e] = apply_sign(f, v[e], kWave * e + lane);
    }
  }
  fwht_strided<E>(k, f.k_block, f.k_norm);
  fwht_strided<E>(v, f.v_block, f.v_norm);

  if (f.kind == HKV_KIND_Q4_0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int blk = 2 * e + (lane >> 5);
      const uint16_t dk = q4_block(k[e], &kc[kWave * e + lane]);
      const uint16_t dv = q4_block(v[e], &vc[kWave * e + lane]);
      if ((lane & 31) == 0) {
        sc[blk] = dk;
        sc[2 * E + blk] = dv;
      }
    }
  } else {
    if (f.compact) {
      const uint16_t s = octave_block<E, 3>(k, 0, E, kc);
      if (lane == 0) sc[0] = s;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint16_t s = (kWave * e < f.k_wide) ? octave_block<E, 4>(k, e, 1, kc)
                                                   : octave_block<E, 3>(k, e, 1, kc);
        if (lane == 0) sc[e] = s;
      }
    }
    const uint16_t s = (f.v_bits == 4) ? octave_block<E, 4>(v, 0, E, vc)
                                       : octave_block<E, 3>(v, 0, E, vc);
    if (lane == 0) sc[f.num_k_scales] = s;
  }
  __syncthreads();

  const int64_t page = sm / f.page_size;
  const int off = (int)(sm % f.page_size);
  uint32_t* dst = (uint32_t*)slot_ptr(f, cache, page, off, num_kv_heads, h);
  const int D = E * kWave;
  for (int w = lane; w < f.slot_bytes / 4; w += kWave) {
    const int o = 4 * w;
    uint32_t word;
    if (o < f.off_k_nope) {
      word = pack4_word(kc, w);
    } else if (o < f.off_v) {
      word = pack3_word(kc + f.k_wide, D - f.k_wide, o - f.off_k_nope);
    } else if (o < f.off_scales) {
      word = (f.kind == HKV_KIND_Q4_0 || f.v_bits == 4) ? pack4_word(vc, (o - f.off_v) / 4)
                                                        : pack3_word(vc, D, o - f.off_v);
    } else {
      const int i = (o - f.off_scales) / 2;
      const uint32_t lo = i < f.num_scales ? sc[i] : 0u;
      const uint32_t hi = i + 1 < f.num_scales ? sc[i + 1] : 0u;
      word = lo | (hi << 16);
    }
    dst[w] = word;
  }
}

template <int E>
__global__ __launch_bounds__(64) void dequantize_kernel(DevFmt f, const uint8_t* cache,
                                                        int num_kv_heads,
                                                        const int64_t* slot_ids, int rotated,
                                                        float* k_out, float* v_out) {
  const int64_t row = blockIdx.x;
  const int64_t t = row / num_kv_heads;
  const int h = (int)(row % num_kv_heads);
  const int lane = lane_id();
  const int64_t sid = slot_ids[t];
  float* ko = k_out + row * (E * kWave);
  float* vo = v_out + row * (E * kWave);
  if (sid < 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ko[kWave * e + lane] = 0.0f;
      vo[kWave * e + lane] = 0.0f;
    }
    return;
  }
  __shared__ __align__(16) uint8_t sb[kMaxSlot];
  const uint32_t* src =
      (const uint32_t*)slot_ptr(f, cache, sid / f.page_size, (int)(sid % f.page_size),
                                num_kv_heads, h);
  for (int w = lane; w < f.slot_bytes / 4; w += kWave) ((uint32_t*)sb)[w] = src[w];
  __syncthreads();
  float k[E], v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = k_value(f, sb, kWave * e + lane);
    v[e] = v_value(f, sb, kWave * e + lane);
  }
  if (!rotated) {
    fwht_strided<E>(k, f.k_block, f.k_norm);
    fwht_strided<E>(v, f.v_block, f.v_norm);
    if (f.use_signs) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        k[e] = apply_sign(f, k[e], kWave * e + lane);
        v[e] = apply_sign(f, v[e], kWave * e + lane);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ko[kWave * e + lane] = k[e];
    vo[kWave * e + lane] = v[e];
  }
}

}  // namespace

hipError_t launch_quantize_append(const DevFmt& f, const void* key, const void* value,
                                  bool in_f16, int64_t num_tokens, int num_kv_heads,
                                  const int64_t* slot_mapping, uint8_t* cache, hipStream_t s) {
  const int64_t rows = num_tokens * num_kv_heads;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)rows), block(kWave);
  switch (f.D / kWave) {
    case 1: quantize_append_kernel<1><<<grid, block, 0, s>>>(f, key, value, in_f16, num_kv_heads, slot_mapping, cache); break;
    case 2: quantize_append_kernel<2><<<grid, block, 0, s>>>(f, key, value, in_f16, num_kv_heads, slot_mapping, cache); break;
    case 3: quantize_append_kernel<3><<<grid, block, 0, s>>>(f, key, value, in_f16, num_kv_heads, slot_mapping, cache); break;
    case 4: quantize_append_kernel<4><<<grid, block, 0, s>>>(f, key, value, in_f16, num_kv_heads, slot_mapping, cache); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const DevFmt& f, const uint8_t* cache, int num_kv_heads,
                             const int64_t* slot_ids, int64_t num_tokens, bool rotated,
                             float* k_out, float* v_out, hipStream_t s) {
  const int64_t rows = num_tokens * num_kv_heads;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)rows), block(kWave);
  switch (f.D / kWave) {
    case 1: dequantize_kernel<1><<<grid, block, 0, s>>>(f, cache, num_kv_heads, slot_ids, rotated, k_out, v_out); break;
    case 2: dequantize_kernel<2><<<grid, block, 0, s>>>(f, cache, num_kv_heads, slot_ids, rotated, k_out, v_out); break;
    case 3: dequantize_kernel<3><<<grid, block, 0, s>>>(f, cache, num_kv_heads, slot_ids, rotated, k_out, v_out); break;
    case 4: dequantize_kernel<4><<<grid, block, 0, s>>>(f, cache, num_kv_heads, slot_ids, rotated, k_out, v_out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hkv
