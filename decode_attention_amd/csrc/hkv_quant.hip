// hkv_quant.hip -- quantize-append and dequantize kernels.
//
// Quantize-append: each wave takes (token, KV head) rows in turn and loads
// the next row while it works on the current one.  A row lives "strided" in
// registers (register e of lane l = element 64e + l); it is sign-flipped and
// Walsh-Hadamard rotated in registers, quantized with wave reductions, and
// its codes are packed into slot words in registers by OR-reductions over the
// lanes that share a word, then stored straight to the slot.
//
// Sources: vLLM API docs "vllm.v1.attention.ops.rocm_octave"
// (reference_quantize, _quantize_lut, _pack, reference_dequantize) and Strata
// pull request #21 (Q4_0 block with one fp16 scale per 32 values; the max-abs
// tie-break of the merge note).
#include <cmath>

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

// The Octave block quantizer (vLLM docs "vllm.v1.attention.ops.rocm_octave",
// _quantize_lut) rests on three properties, one helper each:
//  * the block is normalised by its RMS, sqrt(|x|^2 / n), floored at 1e-12 so
//    that an all-zero block divides by a positive number;
//  * each value takes the code of the nearest codebook entry to its
//    normalised value times the codebook's multiplier (bucket, above);
//  * the fp16 scale s makes the dequantized block x_hat = s * LUT[code] / 64
//    keep the block's norm along x: x . x_hat = |x|^2, i.e.
//    s = 64 * |x|^2 / (x . LUT[code]), and 0 when that dot product is not
//    positive (an all-zero block).
// Every sum is one of the block sums in their fixed order.
__device__ __forceinline__ float oct_block_rms(float ss, int n) {
  const float r = sqrtf(ss / (float)n);
  return r < 1e-12f ? 1e-12f : r;
}
__device__ __forceinline__ uint32_t oct_norm_preserving_scale(float ss, float dot) {
  const float q = dot > 0.0f ? ss / (dot > 1e-30f ? dot : 1e-30f) : 0.0f;
  return f2h(q * (float)kLutOne);
}

// The quantizer over registers [e0, e0+nreg) of a strided vector.  The codes
// land in codes[e0 .. e0+nreg); returns the fp16 bits of the scale (the same
// in every lane).
template <int E, int BITS>
__device__ __forceinline__ uint32_t octave_block(const float (&x)[E], int e0, int nreg,
                                                 uint32_t (&codes)[E]) {
  float t[E];
#pragma unroll
  for (int e = 0; e < E; ++e) t[e] = x[e] * x[e];
  const float ss = block_tree_sum<E>(t, e0, nreg);
  const float rms = oct_block_rms(ss, nreg * kWave);
  const float mult = (float)(BITS == 3 ? kLutMult3 : kLutMult4);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    t[e] = 0.0f;
    if (e >= e0 && e < e0 + nreg) {
      int lv;
      codes[e] = (uint32_t)bucket<BITS>((x[e] / rms) * mult, &lv);
      t[e] = x[e] * (float)lv;
    }
  }
  return oct_norm_preserving_scale(ss, block_tree_sum<E>(t, e0, nreg));
}

// Q4_0 over one 32-value block = one half-register (lanes 0-31 or 32-63).
// Max-abs element with the tie-break (larger magnitude; equal magnitudes keep
// the larger signed value) is the maximum of the key (|x| bits, x >= 0) --
// the fp32 bits rotated left by one with the sign bit inverted -- reduced
// over the half with unsigned max.  d = m / -8; code = min(15, trunc(x/d +
// 8.5)).  Returns the fp16 bits of d (the same in all lanes of the half).
__device__ __forceinline__ uint32_t q4_block(float x, uint32_t* code) {
  const uint32_t b = __float_as_uint(x);
  uint32_t key = (b << 1) | ((~b) >> 31);
  key = max(key, dpp<0xB1>(key));   // quad [1,0,3,2]
  key = max(key, dpp<0x4E>(key));   // quad [2,3,0,1]
  key = max(key, dpp<0x141>(key));  // half-row mirror: quad pairs
  key = max(key, dpp<0x140>(key));  // row mirror: half-row pairs
  {
    const auto r = __builtin_amdgcn_permlane16_swap(key, key, false, false);
    key = max(r[0], r[1]);
  }
  // an all-zero block keeps the initial +0 of the scan
  const float m = (key >> 1) == 0 ? 0.0f : __uint_as_float((key >> 1) | ((~key) << 31));
  const float d = m / -8.0f;
  const float id = (d != 0.0f) ? recip_rn(d) : 0.0f;
  const float u = x * id + 8.5f;
  int c = (int)u;
  c = c > 15 ? 15 : c;
  *code = (uint32_t)c;
  return f2h(d);
}

// OR of t over the lanes of each quad / 16-lane row / 32-lane half; every
// lane of the group ends with the result.
__device__ __forceinline__ uint32_t or_quad(uint32_t t) {
  t |= dpp<0xB1>(t);
  t |= dpp<0x4E>(t);
  return t;
}
__device__ __forceinline__ uint32_t or_row(uint32_t t) {
  t = or_quad(t);
  t |= dpp<0x141>(t);  // half-row mirror: quad pairs
  t |= dpp<0x140>(t);  // row mirror: half-row pairs
  return t;
}
__device__ __forceinline__ uint32_t or_half(uint32_t t) {
  t = or_row(t);
  const auto r = __builtin_amdgcn_permlane16_swap(t, t, false, false);
  return r[0] | r[1];
}

// [OCT] _pack of one register of codes (64 consecutive codes of a segment).
// 4-bit: word k holds codes 8k .. 8k+7, byte j = code 8k+j | code 8k+4+j << 4;
// lane 8k ends with word k.
__device__ __forceinline__ uint32_t pack4_lanes(uint32_t c) {
  const int lane = lane_id();
  uint32_t n = c | (xor_u32(c, 4) << 4);
  n = (lane & 4) ? 0u : n << (8 * (lane & 3));
  return or_quad(n);
}
// 3-bit, low two bits: word k holds codes 16k .. 16k+15, code 16k + 4i + j at
// bits 8j + 2i; lane 16k ends with word k.
__device__ __forceinline__ uint32_t pack3_lo_lanes(uint32_t c) {
  const int lane = lane_id();
  return or_row((c & 3u) << (2 * ((lane >> 2) & 3) + 8 * (lane & 3)));
}
// 3-bit, high bit: word h holds codes 32h .. 32h+31, code 32h + 4i + j at bit
// 8j + i; lane 32h ends with word h.
__device__ __forceinline__ uint32_t pack3_hi_lanes(uint32_t c) {
  const int lane = lane_id();
  return or_half(((c >> 2) & 1u) << (((lane >> 2) & 7) + 8 * (lane & 3)));
}

// Q4_0 row: FWHT over the head, 32-value blocks, codes K | V | scales.  The
// words are formed first and stored at the end (lane 8k holds word k of its
// register), so the row is one straight-line block.
template <int E>
__device__ __forceinline__ void q4_row(const DevFmt& f, float (&k)[E], float (&v)[E],
                                       uint32_t* dst) {
  const int lane = lane_id();
  fwht_strided<E>(k, f.k_block, f.k_norm);
  fwht_strided<E>(v, f.v_block, f.v_norm);
  uint32_t wk[E], wv[E];
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    uint32_t ck, cv;
    const uint32_t sk = q4_block(k[e], &ck);
    const uint32_t sv = q4_block(v[e], &cv);
    wk[e] = pack4_lanes(ck);
    wv[e] = pack4_lanes(cv);
    // Scale word e pairs the blocks of register e (lower half first); K
    // words then V words; lane q writes word q.
    const auto rk = __builtin_amdgcn_permlane32_swap(sk, sk, false, false);
    const auto rv = __builtin_amdgcn_permlane32_swap(sv, sv, false, false);
    word = (lane == e) ? (rk[0] | (rk[1] << 16)) : word;
    word = (lane == E + e) ? (rv[0] | (rv[1] << 16)) : word;
  }
  if ((lane & 7) == 0) {
    uint32_t* pk = dst + (lane >> 3);
    uint32_t* pv = dst + f.off_v / 4 + (lane >> 3);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      pk[8 * e] = wk[e];
      pv[8 * e] = wv[e];
    }
  }
  if (lane < 2 * E) dst[f.off_scales / 4 + lane] = word;
}

// Q8_0 over one 32-value block = one half-register: d = max|x| / 127,
// code = round(x * (1/d)), halves away from zero, as int8.  The magnitudes
// are reduced as fp32 bit patterns (non-negative floats order like their
// bits).  Returns the fp16 bits of d (the same in all lanes of the half).
__device__ __forceinline__ uint32_t q8_block(float x, uint32_t* code) {
  uint32_t a = __float_as_uint(x) & 0x7FFFFFFFu;
  a = max(a, dpp<0xB1>(a));
  a = max(a, dpp<0x4E>(a));
  a = max(a, dpp<0x141>(a));
  a = max(a, dpp<0x140>(a));
  {
    const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    a = max(r[0], r[1]);
  }
  const float d = div127_rn(__uint_as_float(a));
  const float id = (d != 0.0f) ? recip_rn(d) : 0.0f;
  const float t = x * id;
  *code = (uint32_t)(int)roundf(t) & 0xFFu;
  return f2h(d);
}

// Q8_0 row: FWHT over the head, 32-value blocks, int8 codes K | V, then the
// scales as for Q4_0.  Slot word k of register e is the codes of lanes
// 4k .. 4k+3; lane 4k ends with it.
template <int E>
__device__ __forceinline__ void q8_row(const DevFmt& f, float (&k)[E], float (&v)[E],
                                       uint32_t* dst) {
  const int lane = lane_id();
  fwht_strided<E>(k, f.k_block, f.k_norm);
  fwht_strided<E>(v, f.v_block, f.v_norm);
  uint32_t wk[E], wv[E];
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    uint32_t ck, cv;
    const uint32_t sk = q8_block(k[e], &ck);
    const uint32_t sv = q8_block(v[e], &cv);
    wk[e] = or_quad(ck << (8 * (lane & 3)));
    wv[e] = or_quad(cv << (8 * (lane & 3)));
    const auto rk = __builtin_amdgcn_permlane32_swap(sk, sk, false, false);
    const auto rv = __builtin_amdgcn_permlane32_swap(sv, sv, false, false);
    word = (lane == e) ? (rk[0] | (rk[1] << 16)) : word;
    word = (lane == E + e) ? (rv[0] | (rv[1] << 16)) : word;
  }
  if ((lane & 3) == 0) {
    uint32_t* pk = dst + (lane >> 2);
    uint32_t* pv = dst + f.off_v / 4 + (lane >> 2);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      pk[16 * e] = wk[e];
      pv[16 * e] = wv[e];
    }
  }
  if (lane < 2 * E) dst[f.off_scales / 4 + lane] = word;
}

// Octave row: sign flips, FWHT (64-blocks or the whole head), per-block
// Lloyd-Max codes; K codes (4-bit RoPE registers, then the 3-bit rest), V
// codes, then the fp16 scales (K scales, V scale, zero padding).  Word
// layout per register of a segment: 4-bit codes take 8 words (lane 8k holds
// word k); 3-bit codes 4 low-bit words (lane 16k holds word k) and, after
// all low words of the segment, 2 high-bit words (lane 32h holds word h).
template <int E>
__device__ __forceinline__ void octave_row(const DevFmt& f, float (&k)[E], float (&v)[E],
                                           uint32_t* dst) {
  const int lane = lane_id();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = apply_sign(f, k[e], kWave * e + lane);
    v[e] = apply_sign(f, v[e], kWave * e + lane);
  }
  fwht_strided<E>(k, f.k_block, f.k_norm);
  fwht_strided<E>(v, f.v_block, f.v_norm);
  uint32_t ck[E], cv[E], ks[E];
  const int kw = f.k_wide / kWave;  // registers of 4-bit K codes
  if (f.compact) {
    ks[0] = octave_block<E, 3>(k, 0, E, ck);
#pragma unroll
    for (int e = 1; e < E; ++e) ks[e] = 0;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e)
      ks[e] = (e < kw) ? octave_block<E, 4>(k, e, 1, ck) : octave_block<E, 3>(k, e, 1, ck);
  }
  const bool v4 = f.v_bits == 4;
  const uint32_t vs = v4 ? octave_block<E, 4>(v, 0, E, cv) : octave_block<E, 3>(v, 0, E, cv);
  // Scale i: K scales first, then the V scale, then zeros; word q holds
  // scales 2q and 2q+1.
  const int nks = f.num_k_scales;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i <= E; ++i) {
    const uint32_t sc = (i < nks) ? ks[i < E ? i : 0] : (i == nks ? vs : 0u);
    word |= (lane == (i >> 1)) ? (sc << (16 * (i & 1))) : 0u;
  }
  // 4-bit words (or 3-bit low words) and 3-bit high words per register.
  uint32_t k4[E], khi[E], v4w[E], vhi[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k4[e] = (e < kw) ? pack4_lanes(ck[e]) : pack3_lo_lanes(ck[e]);
    khi[e] = (e < kw) ? 0u : pack3_hi_lanes(ck[e]);
    v4w[e] = v4 ? pack4_lanes(cv[e]) : pack3_lo_lanes(cv[e]);
    vhi[e] = v4 ? 0u : pack3_hi_lanes(cv[e]);
  }
  const int wk3 = f.off_k_nope / 4, nk3 = kWave * (E - kw);
  const int wv0 = f.off_v / 4;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e < kw) {
      if ((lane & 7) == 0) dst[8 * e + (lane >> 3)] = k4[e];
    } else {
      if ((lane & 15) == 0) dst[wk3 + 4 * (e - kw) + (lane >> 4)] = k4[e];
      if ((lane & 31) == 0) dst[wk3 + nk3 / 16 + 2 * (e - kw) + (lane >> 5)] = khi[e];
    }
    if (v4) {
      if ((lane & 7) == 0) dst[wv0 + 8 * e + (lane >> 3)] = v4w[e];
    } else {
      if ((lane & 15) == 0) dst[wv0 + 4 * e + (lane >> 4)] = v4w[e];
      if ((lane & 31) == 0) dst[wv0 + kWave * E / 16 + 2 * e + (lane >> 5)] = vhi[e];
    }
  }
  if (lane < (f.slot_bytes - f.off_scales) / 4) dst[f.off_scales / 4 + lane] = word;
}

template <int E, bool F16>
__device__ __forceinline__ void fetch_row(const void* key, const void* value, int row,
                                          uint32_t (&rk)[E], uint32_t (&rv)[E]) {
  const int lane = lane_id();
  const int64_t base = (int64_t)row * (E * kWave) + lane;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (F16) {
      rk[e] = ((const uint16_t*)key)[base + kWave * e];
      rv[e] = ((const uint16_t*)value)[base + kWave * e];
    } else {
      rk[e] = ((const uint32_t*)key)[base + kWave * e];
      rv[e] = ((const uint32_t*)value)[base + kWave * e];
    }
  }
}

constexpr int kQuantWaves = 4;        // waves per workgroup
constexpr int kQuantMaxGroups = 2048; // 8 workgroups per CU on 256 CUs

// rows = num_tokens * num_kv_heads (below 2^31 less one grid stride);
// row = token * num_kv_heads + head.
template <int E, bool F16, int KIND>
__global__ __launch_bounds__(kQuantWaves * kWave) void quantize_append_kernel(
    DevFmt f, const void* key, const void* value, int rows, int num_kv_heads,
    const int64_t* slot_mapping, uint8_t* cache) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // The argument words in one fetch (the row count alone would otherwise go
  // first, ahead of the branch below, and the rest after it); the format's
  // words are read here once so that later reads of them hit the cache.
  int page_size = f.page_size;
  float k_norm = f.k_norm;
  asm("" : "+s"(rows), "+s"(num_kv_heads), "+s"(page_size), "+s"(k_norm));
  key = pin_global(key);
  value = pin_global(value);
  slot_mapping = pin_global(slot_mapping);
  cache = pin_global(cache);
  const int stride = (int)gridDim.x * kQuantWaves;
  int row = (int)blockIdx.x * kQuantWaves + wave;
  if (row >= rows) return;
  uint32_t rk[E], rv[E];
  fetch_row<E, F16>(key, value, row, rk, rv);
  int64_t sm = slot_mapping[row / num_kv_heads];
  for (;;) {
    float k[E], v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      k[e] = F16 ? h2f((uint16_t)rk[e]) : __uint_as_float(rk[e]);
      v[e] = F16 ? h2f((uint16_t)rv[e]) : __uint_as_float(rv[e]);
    }
    const int cur = row;
    const int64_t cur_sm = sm;
    row += stride;
    if (row < rows) {  // the next row's loads are in flight during this one
      fetch_row<E, F16>(key, value, row, rk, rv);
      sm = slot_mapping[row / num_kv_heads];
    }
    if (cur_sm >= 0) {
      int64_t page;
      int off;
      if ((cur_sm >> 32) == 0) {  // 32-bit division when the slot index fits
        const uint32_t s32 = (uint32_t)cur_sm;
        page = s32 / (uint32_t)f.page_size;
        off = (int)(s32 % (uint32_t)f.page_size);
      } else {
        page = cur_sm / f.page_size;
        off = (int)(cur_sm % f.page_size);
      }
      uint32_t* dst =
          (uint32_t*)slot_ptr(f, cache, page, off, num_kv_heads, cur % num_kv_heads);
      if (KIND == HKV_KIND_Q4_0) q4_row<E>(f, k, v, dst);
      else if (KIND == HKV_KIND_Q8_0) q8_row<E>(f, k, v, dst);
      else octave_row<E>(f, k, v, dst);
    }
    if (row >= rows) break;
  }
}

// ---------------------------------------------------------------------------
// Q4_0 and Q8_0 quantize-append of few rows (a decode step's new tokens): one
// wave per (row, K or V), so the append runs twice as many waves as rows,
// each with half of a row's work.  A few hundred waves leave most SIMDs
// empty, so the time of such an append is the latency of one wave's chain
// (argument fetch, row load, rotation, codes, stores), which this halves.
// The K and V halves write disjoint words of the slot: their code segments
// and their scale words (K scales first, then V, as in q4_row / q8_row).
constexpr int kHalfMaxRows = 1024;  // above this the one-row-per-wave kernel fills the chip

template <int E, bool F16, int KIND>
__global__ __launch_bounds__(kQuantWaves * kWave) void quantize_half_kernel(
    DevFmt f, const void* key, const void* value, int rows, int num_kv_heads,
    const int64_t* slot_mapping, uint8_t* cache) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  int page_size = f.page_size;
  float k_norm = f.k_norm;
  asm("" : "+s"(rows), "+s"(num_kv_heads), "+s"(page_size), "+s"(k_norm));
  key = pin_global(key);
  value = pin_global(value);
  slot_mapping = pin_global(slot_mapping);
  cache = pin_global(cache);
  const int item = (int)blockIdx.x * kQuantWaves + wave;  // 2 row + part
  if (item >= 2 * rows) return;
  const int row = item >> 1, part = item & 1;
  const void* src = part ? value : key;
  uint32_t raw[E];
  {
    const int64_t base = (int64_t)row * (E * kWave) + lane;
#pragma unroll
    for (int e = 0; e < E; ++e)
      raw[e] = F16 ? (uint32_t)((const uint16_t*)src)[base + kWave * e]
                   : ((const uint32_t*)src)[base + kWave * e];
  }
  const int64_t sm = slot_mapping[row / num_kv_heads];
  if (sm < 0) return;
  int64_t page;
  int off;
  if ((sm >> 32) == 0) {
    const uint32_t s32 = (uint32_t)sm;
    page = s32 / (uint32_t)page_size;
    off = (int)(s32 % (uint32_t)page_size);
  } else {
    page = sm / page_size;
    off = (int)(sm % page_size);
  }
  uint32_t* dst = (uint32_t*)slot_ptr(f, cache, page, off, num_kv_heads, row % num_kv_heads);
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = F16 ? h2f((uint16_t)raw[e]) : __uint_as_float(raw[e]);
  fwht_strided<E>(x, part ? f.v_block : f.k_block, part ? f.v_norm : k_norm);
  uint32_t w[E];
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    uint32_t c;
    uint32_t sc;
    if (KIND == HKV_KIND_Q8_0) {
      sc = q8_block(x[e], &c);
      w[e] = or_quad(c << (8 * (lane & 3)));
    } else {
      sc = q4_block(x[e], &c);
      w[e] = pack4_lanes(c);
    }
    // scale word e pairs the blocks of register e (lower half first)
    const auto r = __builtin_amdgcn_permlane32_swap(sc, sc, false, false);
    word = (lane == e) ? (r[0] | (r[1] << 16)) : word;
  }
  uint32_t* seg = dst + (part ? f.off_v / 4 : 0);
  if (KIND == HKV_KIND_Q8_0) {
    if ((lane & 3) == 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) seg[(lane >> 2) + 16 * e] = w[e];
    }
  } else if ((lane & 7) == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) seg[(lane >> 3) + 8 * e] = w[e];
  }
  if (lane < E) dst[f.off_scales / 4 + part * E + lane] = word;
}

// ---------------------------------------------------------------------------
// Q4_0 and Q8_0 quantize-append for many rows: 16 lanes per row, four rows
// per wave.
// A lane of a 16-lane row holds four consecutive elements 64q + 4e + i
// (i = 0..3) of its row for each 64-wide group q, so the element index bits
// 0-1 live in a register, bits 2-5 (e) in the lane (exchanges stay inside
// the 16-lane DPP row), bits 6-7 in q.  The butterfly stages still run in
// ascending stride (1, 2 in registers; 4..32 across lanes; 64, 128 in
// registers), each as the same (a + b, a - b) pair up to sign, so the bytes
// equal those of the kernel above.  A 32-value block is one q of one 8-lane
// half-row.

// Row cursor of the many-row kernels: a lane group's row r = t H + h (token
// t, KV head h of H), advanced by the grid stride with two adds and a carry
// instead of a division by H per step.
struct RowCursor {
  int row, tok, head;
  int dtok, dhead;  // the stride as dtok H + dhead
  __device__ __forceinline__ void init(int r, int stride, int H) {
    row = r;
    tok = r / H;
    head = r - tok * H;
    dtok = stride / H;
    dhead = stride - dtok * H;
  }
  __device__ __forceinline__ void advance(int stride, int H) {
    row += stride;
    tok += dtok;
    head += dhead;
    const bool carry = head >= H;
    head = carry ? head - H : head;
    tok += carry ? 1 : 0;
  }
};

// How the many-row kernels address a slot (uniform over the launch): with a
// power-of-two page size, H page_size below 2^24 and H page_size slot_bytes
// below 2^32, the page and offset of a slot id below 2^32 are a shift and a
// mask, and the slot's byte offset ((page H + h) page_size + offset)
// slot_bytes is page (H page_size slot_bytes) + (h page_size + offset)
// slot_bytes: one 32 x 32 -> 64-bit multiply-add, the second product on the
// 24-bit multipliers.
struct SlotAddr {
  bool fast;
  int shift;
  uint32_t page_bytes;
  __device__ __forceinline__ void init(const DevFmt& f, int H) {
    const uint32_t ps = (uint32_t)f.page_size;
    const uint64_t pb = (uint64_t)H * ps * (uint32_t)f.slot_bytes;
    fast = (ps & (ps - 1)) == 0 && (uint64_t)H * ps < (1u << 24) && pb <= 0xFFFFFFFFull;
    shift = __builtin_ctz(ps);
    page_bytes = (uint32_t)pb;
  }
  // Byte offset of slot id `slot` (>= 0) of KV head h.
  __device__ __forceinline__ uint64_t offset(const DevFmt& f, int64_t slot, int h, int H) const {
    if (fast && (slot >> 32) == 0) {
      const uint32_t s32 = (uint32_t)slot;
      uint32_t in_page = (uint32_t)__umul24(
          (uint32_t)__umul24((uint32_t)h, (uint32_t)f.page_size) + (s32 & ((uint32_t)f.page_size - 1u)),
          (uint32_t)f.slot_bytes);
      asm("" : "+v"(in_page));  // a 32-bit value: not re-associated into 64-bit products
      return (uint64_t)(s32 >> shift) * (uint64_t)page_bytes + (uint64_t)in_page;
    }
    const int64_t page = slot / f.page_size;
    const int off = (int)(slot % f.page_size);
    return (uint64_t)(((page * H + h) * (int64_t)f.page_size + off) * (int64_t)f.slot_bytes);
  }
};

// Lane order of the Q4_0 / Q8_0 many-row kernel.  Element bits 2-5 of a
// 64-wide group, e = (e2, e3, e4, e5), sit in lane e2 ^ 2 e3 ^ 7 e4 ^ 8 e5
// of the 16-lane row, so the partner of every cross-lane butterfly stage is
// one DPP move: lane xor 1 (quad_perm [1,0,3,2]), xor 2 (quad_perm
// [2,3,0,1]), xor 7 (row_half_mirror) and xor 8 (row_ror:8).  Flipping e5
// flips lane bit 3 only, so a 32-value block (fixed e5) is still a half-row;
// flipping e2 flips lane bit 0 only, so the two nibbles of a Q4_0 byte are
// still lanes l and l ^ 1.  Returns e (bits 0-3) of lane l.
__device__ __forceinline__ int qrow_elem(int l) {
  const int e4 = (l >> 2) & 1, e5 = (l >> 3) & 1;
  const int e3 = ((l >> 1) & 1) ^ e4, e2 = (l & 1) ^ e4;
  return e2 | (e3 << 1) | (e4 << 2) | (e5 << 3);
}

// One cross-lane butterfly stage as one fused DPP multiply-add per value:
// x + sgn * partner with sgn = -1 in the upper lanes of the stage.  The lower
// lane gets a + b; the upper lane gets b - a, the negated a - b.  The two
// lanes of a later pair differ only in a bit not yet transformed, so they
// carry the same sign, and the lower/upper results of that stage are again
// a + b and the negated a - b of the signed values; round-to-nearest is
// symmetric in the sign, so every magnitude is bitwise the one of the plain
// (a + b, a - b) stage.  The accumulated sign, (-1)^(e2 + e3 + e4 + e5), is
// removed by the final normalisation multiply.  (Only the sign of an exact
// zero can differ; neither quantizer reads it.)
//
// The compiler does not fold a DPP move into v_fmac_f32, so the stage is
// written out: v_fmac_f32_dpp x, x(partner), sgn reads the partner's x
// through the DPP lane pattern and adds sgn times it to the lane's own x.
// Each block opens with five wait states (s_nop 4: two are what a DPP read
// of a register needs after a VALU write of it, five what it needs after a
// VALU write of EXEC) and closes with two (a DPP read by the code after the
// block); inside a block no instruction reads a register an earlier one
// wrote.
#define HKV_FMAC_DPP(CTL, N) "v_fmac_f32_dpp %" #N ", %" #N ", %[s] " CTL " row_mask:0xf bank_mask:0xf\n\t"
#define HKV_FMAC_DPP4(CTL, A, B, C, D) \
  HKV_FMAC_DPP(CTL, A) HKV_FMAC_DPP(CTL, B) HKV_FMAC_DPP(CTL, C) HKV_FMAC_DPP(CTL, D)

template <int Q>
struct FwhtStageAsm;
template <>
struct FwhtStageAsm<1> {
  template <int CTRL>
  static __device__ __forceinline__ void run(float (&x)[1][4], float sgn);
};
template <>
struct FwhtStageAsm<2> {
  template <int CTRL>
  static __device__ __forceinline__ void run(float (&x)[2][4], float sgn);
};
template <>
struct FwhtStageAsm<4> {
  template <int CTRL>
  static __device__ __forceinline__ void run(float (&x)[4][4], float sgn);
};

#define HKV_STAGE_DEFS(CTRL, CTL)                                                                \
  template <>                                                                                   \
  __device__ __forceinline__ void FwhtStageAsm<1>::run<CTRL>(float (&x)[1][4], float sgn) {     \
    asm("s_nop 4\n\t" HKV_FMAC_DPP4(CTL, 0, 1, 2, 3) "s_nop 1"                                  \
        : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[0][2]), "+v"(x[0][3])                           \
        : [s] "v"(sgn));                                                                        \
  }                                                                                             \
  template <>                                                                                   \
  __device__ __forceinline__ void FwhtStageAsm<2>::run<CTRL>(float (&x)[2][4], float sgn) {     \
    asm("s_nop 4\n\t" HKV_FMAC_DPP4(CTL, 0, 1, 2, 3) HKV_FMAC_DPP4(CTL, 4, 5, 6, 7) "s_nop 1"   \
        : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[0][2]), "+v"(x[0][3]), "+v"(x[1][0]),            \
          "+v"(x[1][1]), "+v"(x[1][2]), "+v"(x[1][3])                                           \
        : [s] "v"(sgn));                                                                        \
  }                                                                                             \
  template <>                                                                                   \
  __device__ __forceinline__ void FwhtStageAsm<4>::run<CTRL>(float (&x)[4][4], float sgn) {     \
    asm("s_nop 4\n\t" HKV_FMAC_DPP4(CTL, 0, 1, 2, 3) HKV_FMAC_DPP4(CTL, 4, 5, 6, 7)              \
            HKV_FMAC_DPP4(CTL, 8, 9, 10, 11) HKV_FMAC_DPP4(CTL, 12, 13, 14, 15) "s_nop 1"         \
        : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[0][2]), "+v"(x[0][3]), "+v"(x[1][0]),            \
          "+v"(x[1][1]), "+v"(x[1][2]), "+v"(x[1][3]), "+v"(x[2][0]), "+v"(x[2][1]),            \
          "+v"(x[2][2]), "+v"(x[2][3]), "+v"(x[3][0]), "+v"(x[3][1]), "+v"(x[3][2]),            \
          "+v"(x[3][3])                                                                         \
        : [s] "v"(sgn));                                                                        \
  }

HKV_STAGE_DEFS(0xB1, "quad_perm:[1,0,3,2]")
HKV_STAGE_DEFS(0x4E, "quad_perm:[2,3,0,1]")
HKV_STAGE_DEFS(0x141, "row_half_mirror")
HKV_STAGE_DEFS(0x128, "row_ror:8")
#undef HKV_STAGE_DEFS
#undef HKV_FMAC_DPP4
#undef HKV_FMAC_DPP

template <int CTRL, int Q>
__device__ __forceinline__ void fwht_stage_fused(float (&x)[Q][4], float sgn) {
  FwhtStageAsm<Q>::template run<CTRL>(x, sgn);
}

// The same stage over four values, with the partner read through the DPP
// pattern from x itself (in place) or from a separate register t (for a
// partner two DPP patterns away: t holds the first, the fused instruction
// applies the second).
template <int CTRL>
__device__ __forceinline__ void fwht_fmac4(float (&x)[4], float sgn);
template <int CTRL>
__device__ __forceinline__ void fwht_fmac4_src(float (&x)[4], const float (&t)[4], float sgn);

#define HKV_FMAC4_DEF(CTRL, CTL)                                                                  \
  template <>                                                                                    \
  __device__ __forceinline__ void fwht_fmac4<CTRL>(float (&x)[4], float sgn) {                   \
    asm("s_nop 4\n\t"                                                                             \
        "v_fmac_f32_dpp %0, %0, %[s] " CTL " row_mask:0xf bank_mask:0xf\n\t"                      \
        "v_fmac_f32_dpp %1, %1, %[s] " CTL " row_mask:0xf bank_mask:0xf\n\t"                      \
        "v_fmac_f32_dpp %2, %2, %[s] " CTL " row_mask:0xf bank_mask:0xf\n\t"                      \
        "v_fmac_f32_dpp %3, %3, %[s] " CTL " row_mask:0xf bank_mask:0xf\n\t"                      \
        "s_nop 1"                                                                                \
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])                                         \
        : [s] "v"(sgn));                                                                         \
  }
#define HKV_FMAC4_SRC_DEF(CTRL, CTL)                                                              \
  template <>                                                                                    \
  __device__ __forceinline__ void fwht_fmac4_src<CTRL>(float (&x)[4], const float (&t)[4],       \
                                                       float sgn) {                              \
    asm("s_nop 4\n\t"                                                                             \
        "v_fmac_f32_dpp %0, %4, %[s] " CTL " row_mask:0xf bank_mask:0xf\n\t"                      \
        "v_fmac_f32_dpp %1, %5, %[s] " CTL " row_mask:0xf bank_mask:0xf\n\t"                      \
        "v_fmac_f32_dpp %2, %6, %[s] " CTL " row_mask:0xf bank_mask:0xf\n\t"                      \
        "v_fmac_f32_dpp %3, %7, %[s] " CTL " row_mask:0xf bank_mask:0xf\n\t"                      \
        "s_nop 1"                                                                                \
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])                                         \
        : "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]), [s] "v"(sgn));                             \
  }

HKV_FMAC4_DEF(0xB1, "quad_perm:[1,0,3,2]")
HKV_FMAC4_DEF(0x4E, "quad_perm:[2,3,0,1]")
HKV_FMAC4_DEF(0x128, "row_ror:8")
HKV_FMAC4_SRC_DEF(0x1B, "quad_perm:[3,2,1,0]")
#undef HKV_FMAC4_DEF
#undef HKV_FMAC4_SRC_DEF

// fwht_rows16 in the lane order of qrow_elem (from stride 2 when the
// caller has already done the stride-1 stage, kFrom2).  kFuseNorm (Q >= 2,
// fp16 inputs, a power-of-two norm): the last register stage takes the
// normalising multiply with it, (a + b) s = fma(a, s, b s) and
// (a - b) s = fma(a, s, -(b s)): b s is exact, and so is the product of a
// rounded sum by a power of two while it stays normal, which every nonzero
// value of an fp16 row does (each is a multiple of 2^-24 before the
// multiply), so the bits are those of the stage followed by the multiply.
template <int Q, bool kFrom2 = false, bool kFuseNorm = false>
__device__ __forceinline__ void fwht_rows16_q(float (&x)[Q][4], int e, float norm) {
  // h = 1, 2: registers
#pragma unroll
  for (int h = kFrom2 ? 2 : 1; h <= 2; h <<= 1)
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((i & h) == 0) {
          const float a = x[q][i], b = x[q][i + h];
          x[q][i] = a + b;
          x[q][i + h] = a - b;
        }
  // h = 4, 8, 16, 32: element bits 2, 3, 4, 5 across lanes
  fwht_stage_fused<0xB1>(x, (e & 1) ? -1.0f : 1.0f);
  fwht_stage_fused<0x4E>(x, (e & 2) ? -1.0f : 1.0f);
  fwht_stage_fused<0x141>(x, (e & 4) ? -1.0f : 1.0f);
  fwht_stage_fused<0x128>(x, (e & 8) ? -1.0f : 1.0f);
  // h = 64, 128: register groups (both values carry the lane's sign)
  constexpr bool kFuse = kFuseNorm && Q >= 2;
  constexpr int kLast = kFuse ? Q / 2 : Q;  // the stage fused with the multiply
#pragma unroll
  for (int hq = 1; hq < kLast; hq <<= 1)
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if ((q & hq) == 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = x[q][i], b = x[q + hq][i];
          x[q][i] = a + b;
          x[q + hq][i] = a - b;
        }
  const float sn = (__builtin_popcount(e) & 1) ? -norm : norm;
  if constexpr (kFuse) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if ((q & kLast) == 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = x[q][i], bs = x[q + kLast][i] * sn;
          x[q][i] = __builtin_fmaf(a, sn, bs);
          x[q + kLast][i] = __builtin_fmaf(a, sn, -bs);
        }
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[q][i] = x[q][i] * sn;
  }
}

// One 64-wide group: codes packed into the words of this lane pair and the
// fp16 scales of its two blocks, in the lane order of qrow_elem.  The group
// comes in negated, y = -x (the normalising multiply of fwht_rows16_q takes
// the negated factor, which costs nothing), so that the max-abs key
// (|x| bits, x >= +0) is the bits of y rotated left by one, and the scale
// d = m / -8 of the chosen element m is the key rotated right by one (the
// bits of -m) times 1/8; x (1/d) is y (-1/d).  Keys start at 1, the key of
// +0, so that a block of zeros of either sign takes m = +0 as the tie-break
// gives it.  On return `word` (lanes with e2 = 0) is slot word 8q + e/2 of
// the segment and `d` the scale of this lane's block (block 2q in lanes 0-7,
// 2q + 1 in lanes 8-15).
__device__ __forceinline__ void q4_group16(const float (&y)[4], uint32_t* word, float* d_out) {
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = __float_as_uint(y[i]);
    key[i] = __builtin_amdgcn_alignbit(b, b, 31);  // rotate left by one: see q4_block
  }
  uint32_t kmax = max(max(key[0], key[1]), key[2]);
  kmax = max(max(kmax, key[3]), 1u);
  kmax = max(kmax, dpp<0xB1>(kmax));   // quad [1,0,3,2]
  kmax = max(kmax, dpp<0x4E>(kmax));   // quad [2,3,0,1]
  kmax = max(kmax, dpp<0x141>(kmax));  // half-row mirror: the 8 lanes of the block
  const float d = __uint_as_float(__builtin_amdgcn_alignbit(kmax, kmax, 1)) * 0.125f;
  // 1/d: recip_rn's fast form when every lane of the wave has |d| in
  // [2^-100, 2^100] (|m| in [2^-97, 2^103]: keys 0x1E000000 .. 0xE6000001),
  // else recip_rn itself, 0 for d = 0.
  float id;
  if (__builtin_amdgcn_ballot_w64(kmax - 0x1E000000u > 0xE6000001u - 0x1E000000u) == 0) {
    const float r = __builtin_amdgcn_rcpf(d);
    id = __builtin_fmaf(__builtin_fmaf(-d, r, 1.0f), r, r);
  } else {
    id = (d != 0.0f) ? recip_rn(d) : 0.0f;
  }
  uint32_t c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float u = y[i] * -id + 8.5f;
    const int ci = (int)u;
    c[i] = (uint32_t)(ci > 15 ? 15 : ci);
  }
  // bytes of this lane's four codes; the odd lane's go to the high nibbles
  const uint32_t bytes = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
  *word = bytes | (dpp<0xB1>(bytes) << 4);
  *d_out = d;
}

// Q8_0 over one 64-wide group in the lane order of qrow_elem, negated as for
// Q4_0 (y = -x: the magnitudes are those of x, and round(x id) is
// round(y (-id)), rounding being symmetric): `word` is slot word 16q + e
// (this lane's four int8 codes), `d` the scale of this lane's block, as for
// Q4_0.
__device__ __forceinline__ void q8_group16(const float (&y)[4], uint32_t* word, float* d_out) {
  uint32_t a = max(max(__float_as_uint(y[0]) & 0x7FFFFFFFu, __float_as_uint(y[1]) & 0x7FFFFFFFu),
                   max(__float_as_uint(y[2]) & 0x7FFFFFFFu, __float_as_uint(y[3]) & 0x7FFFFFFFu));
  a = max(a, dpp<0xB1>(a));   // quad [1,0,3,2]
  a = max(a, dpp<0x4E>(a));   // quad [2,3,0,1]
  a = max(a, dpp<0x141>(a));  // half-row mirror: the 8 lanes of the block
  const float d = div127_rn(__uint_as_float(a));
  const float id = (d != 0.0f) ? recip_rn(d) : 0.0f;
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) w |= ((uint32_t)(int)roundf(y[i] * -id) & 0xFFu) << (8 * i);
  *word = w;
  *d_out = d;
}

// Elements 64q + e4 .. + 3 (q < Q) of the row's K and V, for this lane's
// element offset e4 in a 64-wide group.
template <int Q, bool F16>
__device__ __forceinline__ void fetch_rows16(const void* key, const void* value, int row, int e4,
                                             uint32_t (&rk)[Q][F16 ? 2 : 4],
                                             uint32_t (&rv)[Q][F16 ? 2 : 4]) {
  constexpr int D = 64 * Q;
  if (F16) {
    const uint2* pk = (const uint2*)((const uint16_t*)key + (int64_t)row * D + e4);
    const uint2* pv = (const uint2*)((const uint16_t*)value + (int64_t)row * D + e4);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const uint2 a = pk[16 * q], b = pv[16 * q];
      rk[q][0] = a.x, rk[q][1] = a.y;
      rv[q][0] = b.x, rv[q][1] = b.y;
    }
  } else {
    const uint4* pk = (const uint4*)((const float*)key + (int64_t)row * D + e4);
    const uint4* pv = (const uint4*)((const float*)value + (int64_t)row * D + e4);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const uint4 a = pk[16 * q], b = pv[16 * q];
      rk[q][0] = a.x, rk[q][1] = a.y, rk[q][2] = a.z, rk[q][3] = a.w;
      rv[q][0] = b.x, rv[q][1] = b.y, rv[q][2] = b.z, rv[q][3] = b.w;
    }
  }
}

template <int Q, bool F16>
__device__ __forceinline__ void widen16(const uint32_t (&r)[Q][F16 ? 2 : 4], float (&x)[Q][4]) {
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (F16) {
      x[q][0] = h2f((uint16_t)r[q][0]);
      x[q][1] = h2f((uint16_t)(r[q][0] >> 16));
      x[q][2] = h2f((uint16_t)r[q][1]);
      x[q][3] = h2f((uint16_t)(r[q][1] >> 16));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[q][i] = __uint_as_float(r[q][i]);
    }
  }
}

// widen16, and for f16 inputs the stride-1 butterfly stage with it: each
// sum or difference of two halves is one mixed-precision fma (x 1.0), whose
// single rounding of the exact fp32 sum is the plain stage's (the widening
// itself is exact).
template <int Q, bool F16>
__device__ __forceinline__ void widen16_stage1(const uint32_t (&r)[Q][F16 ? 2 : 4],
                                               float (&x)[Q][4]) {
  // (the 1.0 is opaque, so that the fma is not simplified to an add of two
  // widened values)
  float one = 1.0f;
  if (F16) asm volatile("v_mov_b32 %0, 1.0" : "=v"(one));
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (F16) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const float a = h2f((uint16_t)r[q][p]), b = h2f((uint16_t)(r[q][p] >> 16));
        x[q][2 * p] = __builtin_fmaf(a, one, b);
        x[q][2 * p + 1] = __builtin_fmaf(a, one, -b);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[q][i] = __uint_as_float(r[q][i]);
    }
  }
}

constexpr int kRows16MinRows = 4096;  // below this the one-row-per-wave kernel is faster

// rows as for quantize_append_kernel; key/value 8-byte (f16) or 16-byte (f32)
// aligned.
template <int Q, bool F16, int KIND, bool kFuseNorm>
__global__ __launch_bounds__(kQuantWaves * kWave) void quantize_rows16_kernel(
    DevFmt f, const void* key, const void* value, int rows, int num_kv_heads,
    const int64_t* slot_mapping, uint8_t* cache) {
  constexpr int R = F16 ? 2 : 4;
  const int lane = lane_id();
  const int l = lane & 15;
  const int e = qrow_elem(l);  // this lane's element bits 2-5
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int stride = (int)gridDim.x * kQuantWaves * 4;
  int base = ((int)blockIdx.x * kQuantWaves + wave) * 4;
  if (base >= rows) return;
  const int H = num_kv_heads;
  const int ntok = rows / H;
  SlotAddr sa;
  sa.init(f, H);
  RowCursor c;
  c.init(base + (lane >> 4), stride, H);
  // The next four rows load during this group, unconditionally (clamped to
  // the last row; a row past the end reads slot id -1).
  auto slot_of = [&](const RowCursor& rc) -> int64_t {
    const int64_t s = slot_mapping[min(rc.tok, ntok - 1)];
    return rc.tok < ntok ? s : -1;
  };
  uint32_t rk[Q][R], rv[Q][R];
  fetch_rows16<Q, F16>(key, value, min(c.row, rows - 1), 4 * e, rk, rv);
  int64_t sm = slot_of(c);
  for (;;) {
    float k[Q][4], v[Q][4];
    widen16_stage1<Q, F16>(rk, k);
    widen16_stage1<Q, F16>(rv, v);
    const int cur_head = c.head;
    const int64_t cur_sm = sm;
    base += stride;
    c.advance(stride, H);
    fetch_rows16<Q, F16>(key, value, min(c.row, rows - 1), 4 * e, rk, rv);
    sm = slot_of(c);
    // negated outputs (see q4_group16)
    fwht_rows16_q<Q, F16, kFuseNorm>(k, e, -f.k_norm);
    fwht_rows16_q<Q, F16, kFuseNorm>(v, e, -f.v_norm);
    uint32_t wk[Q], wv[Q];
    float dk[Q], dv[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      if (KIND == HKV_KIND_Q8_0) {
        q8_group16(k[q], &wk[q], &dk[q]);
        q8_group16(v[q], &wv[q], &dv[q]);
      } else {
        q4_group16(k[q], &wk[q], &dk[q]);
        q4_group16(v[q], &wv[q], &dv[q]);
      }
    }
    // scale words: lanes 0..Q-1 the K words, Q..2Q-1 the V words.  Lanes l
    // and l + 8 pick the scales of the same group (their blocks 2q and
    // 2q + 1), which one conversion and one row_ror:8 join into the word.
    const int ls = l & 7;
    float dsel = dk[0];
#pragma unroll
    for (int q = 1; q < Q; ++q) dsel = (ls == q) ? dk[q] : dsel;
#pragma unroll
    for (int q = 0; q < Q; ++q) dsel = (ls == Q + q) ? dv[q] : dsel;
    const uint32_t hsel = f2h(dsel);
    const uint32_t sw = hsel | (dpp<0x128>(hsel) << 16);
    if (cur_sm >= 0) {
      uint32_t* dst = (uint32_t*)(cache + sa.offset(f, cur_sm, cur_head, H));
      if (KIND == HKV_KIND_Q8_0) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          dst[16 * q + e] = wk[q];
          dst[f.off_v / 4 + 16 * q + e] = wv[q];
        }
      } else if ((e & 1) == 0) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          dst[8 * q + (e >> 1)] = wk[q];
          dst[f.off_v / 4 + 8 * q + (e >> 1)] = wv[q];
        }
      }
      if (l < 2 * Q) dst[f.off_scales / 4 + l] = sw;
    }
    if (base >= rows) break;
  }
}

// ---------------------------------------------------------------------------
// Octave quantize-append for many rows, in the 16-lanes-per-row layout of the
// kernel above (lane l of a 16-lane row holds elements 64q + 4l + i).
//
// Division.  The oracle's y = (x / rms) * mult needs the correctly rounded
// x / rms for every element.  With y_r = RN(1/rms), q0 = RN(x * y_r) and the
// exact remainder fma(-rms, q0, x), q = fma(remainder, y_r, q0) is that
// quotient (Markstein's theorem for round to nearest, which assumes no
// underflow); a quotient below 2^-100 is recomputed with the division.
//
// Codes.  The code is #{k : mid_k < y} with mid_k = (LUT[k] + LUT[k+1]) / 2,
// i.e. #{k : T_k < 2y} for the integers T_k = LUT[k] + LUT[k+1], which is
// #{k : T_k <= n} for the integer n = ceil(2y) - 1.  A table indexed by n
// (clamped to [-256, 255], which holds every T_k) gives LUT[code] in its low
// byte and the code in its high byte.  2y = RN(q * 2 mult) exactly, since
// doubling commutes with rounding.

struct OctTables {  // entry n + 256: LUT[code] (int8) | code << 8
  uint16_t t3[512];
  uint16_t t4[512];
};

__device__ void oct_tables_fill(OctTables& T) {
  for (int e = threadIdx.x; e < 1024; e += blockDim.x) {
    const int n = (e & 511) - 256;
    int c = 0, lv;
    if (e < 512) {
#pragma unroll
      for (int k = 0; k < 7; ++k) c += (kLut3[k] + kLut3[k + 1] <= n) ? 1 : 0;
      lv = kLut3[c];
      T.t3[e] = (uint16_t)((lv & 0xFF) | (c << 8));
    } else {
#pragma unroll
      for (int k = 0; k < 15; ++k) c += (kLut4[k] + kLut4[k + 1] <= n) ? 1 : 0;
      lv = kLut4[c];
      T.t4[e - 512] = (uint16_t)((lv & 0xFF) | (c << 8));
    }
  }
}

// The table entry of z = 2y (LUT[code] in its low byte, the code in byte 1)
// and LUT[code] as a float.
template <int BITS>
__device__ __forceinline__ uint32_t oct_code(const OctTables& T, float z, float* lv) {
  // n = ceil(z) - 1 = ~floor(-z), clamped to [-256, 255] as f = floor(-z) in
  // [-256, 255]; the entry is n + 256 = 255 - f.
  int f;
  asm("v_cvt_flr_i32_f32_e64 %0, -%1" : "=v"(f) : "v"(z));
  f = min(max(f, -256), 255);
  const uint16_t* t = BITS == 3 ? T.t3 : T.t4;
  const uint32_t e = *(const uint16_t*)((const char*)t + 510 + f * -2);
  *lv = (float)(int)(int8_t)(uint8_t)e;
  return e;
}

// fwht_rows16 for a transform block of 64 or 64Q values (the group stages
// run only below the block); from stride 2 when the caller has done the
// stride-1 stage (kFrom2).
template <int Q, bool kFrom2 = false>
__device__ __forceinline__ void fwht_rows16b(float (&x)[Q][4], int block, float norm) {
  const int l = lane_id() & 15;
#pragma unroll
  for (int h = kFrom2 ? 2 : 1; h <= 2; h <<= 1)
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((i & h) == 0) {
          const float a = x[q][i], b = x[q][i + h];
          x[q][i] = a + b;
          x[q][i + h] = a - b;
        }
  // h = 4 .. 32: lane strides 1, 2, 4, 8, one fused DPP multiply-add per
  // value (see fwht_stage_fused; lane xor 4 is the half-row mirror followed
  // by the quad reversal); the values end with the lane's sign
  // (-1)^popcount(l), removed with the normalisation.
#pragma unroll
  for (int q = 0; q < Q; ++q) fwht_fmac4<0xB1>(x[q], (l & 1) ? -1.0f : 1.0f);
#pragma unroll
  for (int q = 0; q < Q; ++q) fwht_fmac4<0x4E>(x[q], (l & 2) ? -1.0f : 1.0f);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = __uint_as_float(dpp<0x141>(__float_as_uint(x[q][i])));
    fwht_fmac4_src<0x1B>(x[q], t, (l & 4) ? -1.0f : 1.0f);
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) fwht_fmac4<0x128>(x[q], (l & 8) ? -1.0f : 1.0f);
#pragma unroll
  for (int hq = 1; hq < Q; hq <<= 1) {
    if (64 * hq < block) {
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if ((q & hq) == 0 && q + hq < Q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = x[q][i], b = x[q + hq][i];
            x[q][i] = a + b;
            x[q + hq][i] = a - b;
          }
    }
  }
  const float sn = (__builtin_popcount(l) & 1) ? -norm : norm;
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[q][i] = x[q][i] * sn;
}

// Sum of t over groups [q0, q0 + NQ) of one 16-lane row in the oracle's
// tree order: groups first (halving when NQ is a power of two, else left to
// right), then element strides 32, 16, 8, 4 (lanes 8, 4, 2, 1), then 2, 1
// (registers).  Every lane of the row ends with the sum.
template <int Q, int NQ>
__device__ __forceinline__ float tree16(const float (&t)[Q][4], int q0) {
  float u[4];
  if constexpr ((NQ & (NQ - 1)) == 0) {
    float w[NQ][4];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) w[q][i] = t[q0 + q][i];
#pragma unroll
    for (int h = NQ / 2; h >= 1; h >>= 1)
#pragma unroll
      for (int q = 0; q < h; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) w[q][i] = w[q][i] + w[q + h][i];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = w[0][i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u[i] = t[q0][i];
#pragma unroll
      for (int q = 1; q < NQ; ++q) u[i] = u[i] + t[q0 + q][i];
    }
  }
  // Element stride 32 (lanes 8) on all four registers; lanes l and l ^ 8
  // then hold the same sums (the add commutes bitwise), so the upper
  // half-row takes registers 1 and 3 in place of 0 and 2, and the strides
  // 16, 8, 4 (lanes 4, 2, 1) run on two registers instead of four.
  // Stride 2 pairs registers 0 and 2 (lanes 0-7) and 1 and 3 (lanes 8-15);
  // stride 1 adds the two half-rows.  The same pairs in the same order.
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = u[i] + shfl_xor(u[i], 8);
  const bool upper = (lane_id() & 8) != 0;
  float v01 = upper ? u[1] : u[0];
  float v23 = upper ? u[3] : u[2];
#pragma unroll
  for (int m = 4; m >= 1; m >>= 1) {
    v01 = v01 + shfl_xor(v01, m);
    v23 = v23 + shfl_xor(v23, m);
  }
  const float a = v01 + v23;
  return a + shfl_xor(a, 8);
}

// [OCT] _quantize_lut over groups [q0, q0 + NQ) of a row; codes (as table
// entries, the code in byte 1) into codes[q0 ..]; returns the fp16 bits of
// the scale (the same in the row).
// kHalfIn (fp16 rows): before the normalising multiply every nonzero value is
// a multiple of 2^-24 below 2^24 (a block of at most 256 fp16 values), so
// after it (by 1/sqrt(block) >= 1/16) every nonzero |x| lies in
// [2^-28, 2^20]: ss / n is zero or at least 2^-64, rms (clamped to
// >= 1e-12) lies in [2^-40, 2^20], a nonzero quotient x / rms is above
// 2^-48, and dot = sum of |x| |LUT[c]| (the codebooks are symmetric, so a
// code has the sign of its value; |LUT| >= 6) is zero or in [2^-26, 2^35],
// with ss / dot in [2^-44, 2^18].  So the square root needs no argument
// scaling (sqrt_rn_large), the reciprocal's fast form no range test,
// Markstein's quotient never takes its tiny-quotient fallback, and ss / dot
// is the same quotient (RN(1/dot), the product, its exact remainder, one
// correction) in place of the division.
template <int Q, int NQ, int BITS, bool kHalfIn>
__device__ __forceinline__ uint32_t oct_block16(const OctTables& T, const float (&x)[Q][4], int q0,
                                                uint32_t (&codes)[Q][4]) {
  float t[Q][4];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) t[q][i] = x[q][i] * x[q][i];
  const float ss = tree16<Q, NQ>(t, q0);
  float rms;
  if constexpr (kHalfIn) {
    // ss / n is zero or at least 2^-64 here: the square root needs no
    // argument scaling (oct_block_rms otherwise)
    const float r = sqrt_rn_large(ss / (float)(NQ * kWave));
    rms = r < 1e-12f ? 1e-12f : r;
  } else {
    rms = oct_block_rms(ss, NQ * kWave);
  }
  float ry;
  if constexpr (kHalfIn) {
    const float r = __builtin_amdgcn_rcpf(rms);
    ry = __builtin_fmaf(__builtin_fmaf(-rms, r, 1.0f), r, r);
  } else {
    ry = recip_rn(rms);
  }
  float qv[NQ][4];
  bool tiny = false;
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float xv = x[q0 + q][i];
      const float q0v = xv * ry;
      const float r = fmaf(-rms, q0v, xv);
      qv[q][i] = fmaf(r, ry, q0v);
      if constexpr (!kHalfIn) tiny |= xv != 0.0f && fabsf(qv[q][i]) < 0x1p-100f;
    }
  if (!kHalfIn && __builtin_amdgcn_ballot_w64(tiny) != 0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xv = x[q0 + q][i];
        if (xv != 0.0f && fabsf(qv[q][i]) < 0x1p-100f) qv[q][i] = xv / rms;
      }
  }
  const float m2 = (float)(2 * (BITS == 3 ? kLutMult3 : kLutMult4));
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lv;
      codes[q0 + q][i] = oct_code<BITS>(T, qv[q][i] * m2, &lv);
      t[q0 + q][i] = x[q0 + q][i] * lv;
    }
  const float dot = tree16<Q, NQ>(t, q0);
  if constexpr (kHalfIn) {
    // oct_norm_preserving_scale with the quotient as above (dot > 0 here
    // unless the row is zero, when ss = dot = 0 and the scale is 0)
    const float dd = dot > 1e-30f ? dot : 1e-30f;
    const float r = __builtin_amdgcn_rcpf(dd);
    const float y = __builtin_fmaf(__builtin_fmaf(-dd, r, 1.0f), r, r);
    const float g0 = ss * y;
    const float g = __builtin_fmaf(__builtin_fmaf(-dd, g0, ss), y, g0);
    return f2h((dot > 0.0f ? g : 0.0f) * (float)kLutOne);
  } else {
    return oct_norm_preserving_scale(ss, dot);
  }
}

// Slot words of one group's codes (segment-relative group qq, segment of n
// codes starting at word w0), stored by the lanes that hold them.  The codes
// come as table entries (code in byte 1), gathered into one byte each.
__device__ __forceinline__ uint32_t code_bytes16(const uint32_t (&c)[4]) {
  return __builtin_amdgcn_perm(c[1], c[0], 0x0C0C0501u) | __builtin_amdgcn_perm(c[3], c[2], 0x05010C0Cu);
}
__device__ __forceinline__ void store4_16(uint32_t* dst, int w0, int qq, const uint32_t (&c)[4]) {
  const int l = lane_id() & 15;
  const uint32_t bytes = code_bytes16(c);
  const uint32_t w = bytes | (dpp<0xB1>(bytes) << 4);  // odd lane: the high nibbles
  if ((l & 1) == 0) dst[w0 + 8 * qq + (l >> 1)] = w;
}
__device__ __forceinline__ void store3_16(uint32_t* dst, int w0, int n, int qq,
                                          const uint32_t (&c)[4]) {
  const int l = lane_id() & 15;
  const uint32_t bytes = code_bytes16(c);
  uint32_t lo = bytes & 0x03030303u;
  uint32_t hi = (bytes >> 2) & 0x01010101u;
  lo = or_quad(lo << (2 * (l & 3)));                    // low plane: 4 lanes a word
  hi <<= (l & 7);
  hi = or_quad(hi);
  hi |= dpp<0x141>(hi);                                 // high plane: 8 lanes a word
  if ((l & 3) == 0) dst[w0 + 4 * qq + (l >> 2)] = lo;
  if ((l & 7) == 0) dst[w0 + n / 16 + 2 * qq + (l >> 3)] = hi;
}

// rows as for quantize_append_kernel; key/value 8-byte (f16) or 16-byte (f32)
// aligned; D = 64Q.
template <int Q, bool F16>
__global__ __launch_bounds__(kQuantWaves * kWave) void quantize_oct_rows16_kernel(
    DevFmt f, const void* key, const void* value, int rows, int num_kv_heads,
    const int64_t* slot_mapping, uint8_t* cache) {
  __shared__ OctTables T;
  oct_tables_fill(T);
  __syncthreads();
  constexpr int R = F16 ? 2 : 4;
  const int lane = lane_id();
  const int l = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int stride = (int)gridDim.x * kQuantWaves * 4;
  int base = ((int)blockIdx.x * kQuantWaves + wave) * 4;
  if (base >= rows) return;
  // sign masks of this lane's elements (the same in every row)
  uint32_t smk[Q][4];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 64 * q + 4 * l + i;
      smk[q][i] = ((f.sign_bits[d >> 5] >> (d & 31)) & 1u) << 31;
    }
  // the same for fp16 inputs: the sign bits of the two halves of each word
  uint32_t smh[Q][2];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int p = 0; p < 2; ++p) smh[q][p] = (smk[q][2 * p] >> 16) | smk[q][2 * p + 1];
  const int kw = f.k_wide / kWave;  // groups of 4-bit K codes
  const int nks = f.num_k_scales;
  const int nsw = (f.slot_bytes - f.off_scales) / 4;
  const int H = num_kv_heads;
  const int ntok = rows / H;
  SlotAddr sa;
  sa.init(f, H);
  RowCursor c;
  c.init(base + (lane >> 4), stride, H);
  // The next four rows load during this group, unconditionally (clamped to
  // the last row; a row past the end reads slot id -1).
  auto slot_of = [&](const RowCursor& rc) -> int64_t {
    const int64_t s = slot_mapping[min(rc.tok, ntok - 1)];
    return rc.tok < ntok ? s : -1;
  };
  uint32_t rk[Q][R], rv[Q][R];
  fetch_rows16<Q, F16>(key, value, min(c.row, rows - 1), 4 * (lane & 15), rk, rv);
  int64_t sm = slot_of(c);
  for (;;) {
    float k[Q][4], v[Q][4];
    if (F16) {
      // signs flipped on the halves, then the stride-1 stage with the widening
      uint32_t sk[Q][R], sv[Q][R];
#pragma unroll
      for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int p = 0; p < R; ++p) {
          sk[q][p] = rk[q][p] ^ smh[q][p & 1];
          sv[q][p] = rv[q][p] ^ smh[q][p & 1];
        }
      widen16_stage1<Q, F16>(sk, k);
      widen16_stage1<Q, F16>(sv, v);
    } else {
      widen16<Q, F16>(rk, k);
      widen16<Q, F16>(rv, v);
#pragma unroll
      for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          k[q][i] = __uint_as_float(__float_as_uint(k[q][i]) ^ smk[q][i]);
          v[q][i] = __uint_as_float(__float_as_uint(v[q][i]) ^ smk[q][i]);
        }
    }
    const int cur_head = c.head;
    const int64_t cur_sm = sm;
    base += stride;
    c.advance(stride, H);
    fetch_rows16<Q, F16>(key, value, min(c.row, rows - 1), 4 * (lane & 15), rk, rv);
    sm = slot_of(c);
    fwht_rows16b<Q, F16>(k, f.k_block, f.k_norm);
    fwht_rows16b<Q, F16>(v, f.v_block, f.v_norm);
    uint32_t ck[Q][4], cv[Q][4], ks[Q];
    if (f.compact) {
      ks[0] = oct_block16<Q, Q, 3, F16>(T, k, 0, ck);
#pragma unroll
      for (int q = 1; q < Q; ++q) ks[q] = 0;
    } else {
#pragma unroll
      for (int q = 0; q < Q; ++q)
        ks[q] = (q < kw) ? oct_block16<Q, 1, 4, F16>(T, k, q, ck) : oct_block16<Q, 1, 3, F16>(T, k, q, ck);
    }
    const bool v4 = f.v_bits == 4;
    const uint32_t vs =
        v4 ? oct_block16<Q, Q, 4, F16>(T, v, 0, cv) : oct_block16<Q, Q, 3, F16>(T, v, 0, cv);
    // scale word w holds scales 2w and 2w + 1: K scales, the V scale, zeros
    uint32_t sw = 0;
#pragma unroll
    for (int i = 0; i <= Q; ++i) {
      const uint32_t sc = (i < nks) ? ks[i < Q ? i : 0] : (i == nks ? vs : 0u);
      sw |= (l == (i >> 1)) ? (sc << (16 * (i & 1))) : 0u;
    }
    if (cur_sm >= 0) {
      uint32_t* dst = (uint32_t*)(cache + sa.offset(f, cur_sm, cur_head, H));
      const int wk3 = f.off_k_nope / 4, nk3 = kWave * (Q - kw), wv0 = f.off_v / 4;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        if (q < kw) store4_16(dst, 0, q, ck[q]);
        else store3_16(dst, wk3, nk3, q - kw, ck[q]);
        if (v4) store4_16(dst, wv0, q, cv[q]);
        else store3_16(dst, wv0, kWave * Q, q, cv[q]);
      }
      if (l < nsw) dst[f.off_scales / 4 + l] = sw;
    }
    if (base >= rows) break;
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
  // row indices are int; row + grid stride (at most 4 rows per wave) must not overflow
  if (rows > INT32_MAX - 4 * kQuantMaxGroups * kQuantWaves) return hipErrorInvalidValue;
  const int64_t groups = (rows + kQuantWaves - 1) / kQuantWaves;
  const dim3 grid((unsigned)(groups < kQuantMaxGroups ? groups : kQuantMaxGroups));
  const dim3 block(kQuantWaves * kWave);
  const int r = (int)rows;
  const bool q4 = f.kind == HKV_KIND_Q4_0, q8 = f.kind == HKV_KIND_Q8_0;
  const uintptr_t align = in_f16 ? 8 : 16;
  if ((q4 || q8) && rows >= kRows16MinRows && ((uintptr_t)key % align) == 0 &&
      ((uintptr_t)value % align) == 0) {
    const int64_t g16 = (rows + 4 * kQuantWaves - 1) / (4 * kQuantWaves);
    const dim3 grid16((unsigned)(g16 < kQuantMaxGroups ? g16 : kQuantMaxGroups));
    // fp16 rows with power-of-two norms take the last stage fused with the
    // normalising multiply (see fwht_rows16_q)
    int ek, ev;
    const bool fuse = in_f16 && std::frexp(f.k_norm, &ek) == 0.5f && std::frexp(f.v_norm, &ev) == 0.5f;
#define HKV_Q16K(Q_, K_)                                                                     \
  (!in_f16 ? (quantize_rows16_kernel<Q_, false, K_, false><<<grid16, block, 0, s>>>(         \
                 f, key, value, r, num_kv_heads, slot_mapping, cache))                       \
   : fuse  ? (quantize_rows16_kernel<Q_, true, K_, true><<<grid16, block, 0, s>>>(           \
                 f, key, value, r, num_kv_heads, slot_mapping, cache))                       \
           : (quantize_rows16_kernel<Q_, true, K_, false><<<grid16, block, 0, s>>>(          \
                 f, key, value, r, num_kv_heads, slot_mapping, cache)))
#define HKV_Q16(Q_) (q8 ? HKV_Q16K(Q_, HKV_KIND_Q8_0) : HKV_Q16K(Q_, HKV_KIND_Q4_0))
    switch (f.D / kWave) {
      case 1: HKV_Q16(1); break;
      case 2: HKV_Q16(2); break;
      case 4: HKV_Q16(4); break;
      default: return hipErrorInvalidValue;
    }
#undef HKV_Q16
#undef HKV_Q16K
    return hipGetLastError();
  }
  if (!q4 && !q8 && rows >= kRows16MinRows && ((uintptr_t)key % align) == 0 &&
      ((uintptr_t)value % align) == 0) {
    const int64_t g16 = (rows + 4 * kQuantWaves - 1) / (4 * kQuantWaves);
    const dim3 grid16((unsigned)(g16 < kQuantMaxGroups ? g16 : kQuantMaxGroups));
#define HKV_O16(Q_)                                                                           \
  (in_f16 ? (quantize_oct_rows16_kernel<Q_, true><<<grid16, block, 0, s>>>(                   \
                f, key, value, r, num_kv_heads, slot_mapping, cache))                         \
          : (quantize_oct_rows16_kernel<Q_, false><<<grid16, block, 0, s>>>(                  \
                f, key, value, r, num_kv_heads, slot_mapping, cache)))
    switch (f.D / kWave) {
      case 1: HKV_O16(1); break;
      case 2: HKV_O16(2); break;
      case 3: HKV_O16(3); break;
      case 4: HKV_O16(4); break;
      default: return hipErrorInvalidValue;
    }
#undef HKV_O16
    return hipGetLastError();
  }
  if ((q4 || q8) && rows <= kHalfMaxRows) {
    const int64_t gh = (2 * rows + kQuantWaves - 1) / kQuantWaves;
    const dim3 gridh((unsigned)gh);
#define HKV_QHK(E_, K_)                                                                      \
  (in_f16 ? (quantize_half_kernel<E_, true, K_><<<gridh, block, 0, s>>>(                     \
                f, key, value, r, num_kv_heads, slot_mapping, cache))                        \
          : (quantize_half_kernel<E_, false, K_><<<gridh, block, 0, s>>>(                    \
                f, key, value, r, num_kv_heads, slot_mapping, cache)))
#define HKV_QH(E_) (q8 ? HKV_QHK(E_, HKV_KIND_Q8_0) : HKV_QHK(E_, HKV_KIND_Q4_0))
    switch (f.D / kWave) {
      case 1: HKV_QH(1); break;
      case 2: HKV_QH(2); break;
      case 3: HKV_QH(3); break;
      case 4: HKV_QH(4); break;
      default: return hipErrorInvalidValue;
    }
#undef HKV_QH
#undef HKV_QHK
    return hipGetLastError();
  }
#define HKV_QA1(E_, F16_, Q4_)                                                         \
  quantize_append_kernel<E_, F16_, Q4_><<<grid, block, 0, s>>>(f, key, value, r, num_kv_heads, \
                                                               slot_mapping, cache)
#define HKV_QA(E_)                                                        \
  do {                                                                    \
    if (q4) {                                                             \
      if (in_f16) HKV_QA1(E_, true, HKV_KIND_Q4_0);                       \
      else HKV_QA1(E_, false, HKV_KIND_Q4_0);                             \
    } else if (q8) {                                                      \
      if (in_f16) HKV_QA1(E_, true, HKV_KIND_Q8_0);                       \
      else HKV_QA1(E_, false, HKV_KIND_Q8_0);                             \
    } else {                                                              \
      if (in_f16) HKV_QA1(E_, true, HKV_KIND_OCTAVE);                     \
      else HKV_QA1(E_, false, HKV_KIND_OCTAVE);                           \
    }                                                                     \
  } while (0)
  switch (f.D / kWave) {
    case 1: HKV_QA(1); break;
    case 2: HKV_QA(2); break;
    case 3: HKV_QA(3); break;
    case 4: HKV_QA(4); break;
    default: return hipErrorInvalidValue;
  }
#undef HKV_QA
#undef HKV_QA1
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
