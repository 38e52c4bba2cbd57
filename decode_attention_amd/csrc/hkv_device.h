// hkv_device.h -- device-side building blocks shared by the libhkv kernels
// (gfx950, wave64): kernel-side format, wave shuffles, the Walsh-Hadamard
// butterfly on a register-resident vector, code extraction and the integer
// codebooks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hkv.h"

namespace hkv {

constexpr int kWave = 64;
constexpr int kMaxHead = HKV_MAX_HEAD;
constexpr int kMaxSlot = 2 * kMaxHead;  // generous bound of slot_bytes at D <= 256

// Kernel-side copy of the format, passed by value.
struct DevFmt {
  int kind;       // HKV_KIND_*
  int D;
  int rope;
  int v_bits;
  int compact;
  int page_size;
  int k_block;
  int v_block;
  int k_wide;     // leading K dims with 4-bit codes (all of K for Q4_0)
  int off_k_nope;
  int off_v;
  int off_scales;
  int num_k_scales;
  int num_scales;
  int slot_bytes;
  int use_signs;
  float k_norm;   // fp32(1/sqrt(k_block))
  float v_norm;   // fp32(1/sqrt(v_block))
  uint32_t sign_bits[kMaxHead / 32];
};

// A kernel-argument pointer held in scalar registers from this point on,
// still known to the compiler as a global-memory pointer.  (The empty asm
// makes the argument word an input at this point, so its fetch is issued
// with the other arguments pinned here rather than near its first use.)
template <class T>
__device__ __forceinline__ T* pin_global(T* p) {
  uint64_t v = (uint64_t)(uintptr_t)p;
  asm("" : "+s"(v));
  return (T*)(__attribute__((address_space(1))) T*)v;
}

// 1/x rounded to nearest, as the IEEE division gives it: v_rcp_f32 and one
// Newton step of two fused multiply-adds.  On gfx950 this equals the IEEE
// quotient for every float with 2^-100 <= |x| <= 2^100 (checked on the
// hardware over all such floats); outside that range the division is used.
__device__ __forceinline__ float recip_rn(float x) {
  const float ax = fabsf(x);
  if (ax >= 0x1p-100f && ax <= 0x1p100f) {
    const float r = __builtin_amdgcn_rcpf(x);
    return fmaf(fmaf(-x, r, 1.0f), r, r);
  }
  return 1.0f / x;
}

// x / 127 rounded to nearest, as the IEEE division gives it: the product
// with RN(1/127), its exact remainder and one correction (Markstein's
// quotient).  On gfx950 this equals the IEEE quotient for every float with
// 2^-100 <= |x| <= 2^100 (checked on the hardware over all such floats);
// outside that range the division is used.
__device__ __forceinline__ float div127_rn(float x) {
  const float ax = fabsf(x);
  if (ax >= 0x1p-100f && ax <= 0x1p100f) {
    constexpr float y = 1.0f / 127.0f;
    const float q0 = x * y;
    return fmaf(fmaf(-127.0f, q0, x), y, q0);
  }
  return x / 127.0f;
}

// sqrt(x) rounded to nearest, as sqrtf gives it, for x = +0 and every finite
// x >= 2^-96 (checked on the hardware over all such floats): v_sqrt_f32,
// which is within one ulp, then its neighbours s -+ 1 ulp are taken when the
// exact residual x - s' s says so.  Below 2^-96 those residuals are no longer
// exact; sqrtf scales the argument there, which is what this leaves out.
__device__ __forceinline__ float sqrt_rn_large(float x) {
  const float s = __builtin_amdgcn_sqrtf(x);
  const float sd = __uint_as_float(__float_as_uint(s) - 1u);
  const float su = __uint_as_float(__float_as_uint(s) + 1u);
  const float rd = __builtin_fmaf(-sd, s, x);
  const float ru = __builtin_fmaf(-su, s, x);
  const float r = rd <= 0.0f ? sd : s;
  return ru > 0.0f ? su : r;
}

// ---------------------------------------------------------------------------
// Wave shuffles.
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// DPP move of v.  Every pattern used here reads a lane inside the same row,
// so bound_ctrl (out-of-range lanes read 0) never applies; it lets the
// compiler fold the move into the consuming add / max / or.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Value of lane l ^ m.  Every caller passes a constant m (unrolled loops),
// so the switch folds to plain VALU data movement: DPP quad permutations for
// 1 and 2, a half-row mirror then a quad reversal for 4, a 16-lane rotate for
// 8, and the lane-swap instructions for 16 and 32 (swapping a value with
// itself leaves the partner's copy in one of the two results); anything else
// falls back to the LDS permute.
__device__ __forceinline__ uint32_t xor_u32(uint32_t u, int m) {
  switch (m) {
    case 1:
      return dpp<0xB1>(u);  // quad_perm [1,0,3,2]
    case 2:
      return dpp<0x4E>(u);  // quad_perm [2,3,0,1]
    case 4:
      return dpp<0x1B>(dpp<0x141>(u));  // row_half_mirror, then quad_perm [3,2,1,0]
    case 8:
      return dpp<0x128>(u);  // row_ror:8
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      return (lane_id() & 16) ? r[0] : r[1];
    }
    case 32: {
      const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      return (lane_id() & 32) ? r[0] : r[1];
    }
    default:
      return (uint32_t)__shfl_xor((int)u, m, kWave);
  }
}
__device__ __forceinline__ float shfl_xor(float v, int m) {
  return __uint_as_float(xor_u32(__float_as_uint(v), m));
}

// fp16 bits <-> fp32 (hardware conversions; round to nearest even).
__device__ __forceinline__ float h2f(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}
__device__ __forceinline__ uint16_t f2h(float f) {
  _Float16 v = (_Float16)f;
  uint16_t h;
  __builtin_memcpy(&h, &v, 2);
  return h;
}

// x * (+-1) from the sign pattern, as a flip of the fp32 sign bit.
__device__ __forceinline__ float apply_sign(const DevFmt& f, float x, int dim) {
  const uint32_t bit = (f.sign_bits[dim >> 5] >> (dim & 31)) & 1u;
  return __uint_as_float(__float_as_uint(x) ^ (bit << 31));
}

// ---------------------------------------------------------------------------
// Both lane-swap results of v with itself: of the pair (r[0], r[1]) one is the
// lane's own value and the other its partner's (lane ^ 16, or lane ^ 32) --
// r[0] the lower lane's value and r[1] the upper lane's in both lanes.  A
// sum r[0] + r[1] is then lower + upper in every lane, and
// fma(r[1], -1, r[0]) is lower - upper.
__device__ __forceinline__ float sum_xor16(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Orthonormal Walsh-Hadamard transform (vLLM rocm_octave docs, fwht_blocks)
// of a vector held "strided" across the wave: register e of lane l holds
// element 64*e + l.  Stages h = 1, 2, 4, ... < block in ascending order; the
// element with bit h clear becomes (mine + partner), the one with bit h set
// (partner - mine) -- the same pairs (a+b, a-b) as the sequential form, so
// the result is bitwise the same -- then one fp32 multiply by `norm`.
// Strides below 64 cross lanes, strides of 64 and up pair registers.
template <int E>
__device__ __forceinline__ void fwht_strided(float (&x)[E], int block, float norm) {
  const int lane = lane_id();
#pragma unroll
  for (int h = 1; h < kWave; h <<= 1) {
    if (h < block) {
      // lower (bit h clear): mine + partner; upper: partner - mine, as one
      // fma with an exact +-1 product.
      const float sgn = (lane & h) ? -1.0f : 1.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (h < 16) {
          x[e] = fmaf(x[e], sgn, shfl_xor(x[e], h));
        } else {
          const uint32_t u = __float_as_uint(x[e]);
          const auto r = (h == 16) ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                                   : __builtin_amdgcn_permlane32_swap(u, u, false, false);
          // r[0] = lower element, r[1] = upper element, in both lanes.
          x[e] = fmaf(__uint_as_float(r[1]), sgn, __uint_as_float(r[0]));
        }
      }
    }
  }
#pragma unroll
  for (int hr = 1; hr < E; hr <<= 1) {
    if (hr * kWave < block) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if ((e & hr) == 0 && e + hr < E) {
          const float a = x[e], b = x[e + hr];
          x[e] = a + b;
          x[e + hr] = a - b;
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = x[e] * norm;
}

// The same transform, for a block of 64Q values held 16 lanes to a block:
// lane l of a 16-lane row holds elements 64q + 4l + i (i = 0..3), so index
// bits 0-1 are in a register, bits 2-5 in the lane (exchanges stay inside the
// 16-lane DPP row), bits 6-7 in q.  The stages still run in ascending stride
// (1, 2 in registers; 4..32 across lanes; 64, 128 in registers), each as the
// same (a + b, a - b) pair, so the values are bitwise those of fwht_strided.
template <int Q>
__device__ __forceinline__ void fwht_rows16(float (&x)[Q][4], float norm) {
  const int l = lane_id() & 15;
  // h = 1, 2: registers
#pragma unroll
  for (int h = 1; h <= 2; h <<= 1)
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((i & h) == 0) {
          const float a = x[q][i], b = x[q][i + h];
          x[q][i] = a + b;
          x[q][i + h] = a - b;
        }
  // h = 4 .. 32: lane strides 1 .. 8 inside the 16-lane row
#pragma unroll
  for (int m = 1; m <= 8; m <<= 1) {
    const float sgn = (l & m) ? -1.0f : 1.0f;
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[q][i] = fmaf(x[q][i], sgn, shfl_xor(x[q][i], m));
  }
  // h = 64, 128: register groups
#pragma unroll
  for (int hq = 1; hq < Q; hq <<= 1)
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if ((q & hq) == 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = x[q][i], b = x[q + hq][i];
          x[q][i] = a + b;
          x[q + hq][i] = a - b;
        }
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[q][i] = x[q][i] * norm;
}


// Sum over the 64 lanes as a pairwise tree (strides 32, 16, ..., 1).  With
// xor partners every lane ends with the same bits as the sequential tree
// (a + b == b + a in IEEE arithmetic).
__device__ __forceinline__ float wave_tree_sum(float v) {
  v = sum_xor32(v);
  v = sum_xor16(v);
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v = v + shfl_xor(v, m);
  return v;
}
// Same over 32-lane halves (strides 16..1).
__device__ __forceinline__ float half_tree_sum(float v) {
  v = sum_xor16(v);
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v = v + shfl_xor(v, m);
  return v;
}

// ---------------------------------------------------------------------------
// Integer Lloyd-Max codebooks for N(0,1), int8 (a code c of a block with
// scale s stands for LUT[c] * s / 64).  Constants of the format.
constexpr int kLutOne = 64;
constexpr int kLut3[8] = {-127, -79, -45, -14, 14, 45, 79, 127};
constexpr int kLut4[16] = {-126, -95, -74, -58, -43, -30, -18, -6, 6, 18, 30, 43, 58, 74, 95, 126};
constexpr int kLutMult3 = 59;
constexpr int kLutMult4 = 46;
// The same tables packed as little-endian int8 words for v_perm_b32 lookups.
constexpr uint32_t kLut3W0 = 0xF2D3B181u, kLut3W1 = 0x7F4F2D0Eu;
constexpr uint32_t kLut4W0 = 0xC6B6A182u, kLut4W1 = 0xFAEEE2D5u;
constexpr uint32_t kLut4W2 = 0x2B1E1206u, kLut4W3 = 0x7E5F4A3Au;

// Codebook value of code c (0..7 or 0..15) as a signed int.
__device__ __forceinline__ int lut_value(int c, int bits) {
  uint32_t b;
  if (bits == 3) {
    b = __builtin_amdgcn_perm(kLut3W1, kLut3W0, (uint32_t)c);
  } else {
    const uint32_t lo = __builtin_amdgcn_perm(kLut4W1, kLut4W0, (uint32_t)(c & 7));
    const uint32_t hi = __builtin_amdgcn_perm(kLut4W3, kLut4W2, (uint32_t)(c & 7));
    b = (c & 8) ? hi : lo;
  }
  return (int)(int8_t)(b & 0xffu);
}

// ---------------------------------------------------------------------------
// Code extraction from packed segments (vLLM rocm_octave docs, module text
// and _pack).  `seg` points at the first byte of a packed segment of n codes.
// 4-bit: byte (i/8)*4 + (i%4), low nibble for i%8 < 4, high otherwise.
__device__ __forceinline__ int code4(const uint8_t* seg, int i) {
  const uint8_t b = seg[(i >> 3) * 4 + (i & 3)];
  return ((i >> 2) & 1) ? (b >> 4) : (b & 15);
}
// 3-bit: low 2 bits in a plane of n/4 bytes (a word per 16 codes, code
// 16m+4i+j at bits 2i of byte j of word m), high bit in the following plane
// of n/8 bytes (a word per 32 codes, code 32m+4i+j at bit i of byte j).
__device__ __forceinline__ int code3(const uint8_t* seg, int n, int i) {
  const uint8_t lo = seg[(i >> 4) * 4 + (i & 3)];
  const uint8_t hi = seg[n / 4 + (i >> 5) * 4 + (i & 3)];
  return ((lo >> (2 * ((i >> 2) & 3))) & 3) | (((hi >> ((i >> 2) & 7)) & 1) << 2);
}

__device__ __forceinline__ uint16_t rd16(const uint8_t* p) {
  return (uint16_t)(p[0] | ((uint16_t)p[1] << 8));
}

// Rotated-space value of K dim d of a slot: (code - 8) * fp16 scale for
// Q4_0, the int8 code * fp16 scale for Q8_0, LUT[code] * (fp16 scale / 64)
// for Octave.  Exact in fp32.
__device__ __forceinline__ float k_value(const DevFmt& f, const uint8_t* slot, int d) {
  if (f.kind == HKV_KIND_Q8_0)
    return (float)(int8_t)slot[d] * h2f(rd16(slot + f.off_scales + 2 * (d >> 5)));
  if (f.kind == HKV_KIND_Q4_0) {
    const int c = code4(slot, d);
    return (float)(c - 8) * h2f(rd16(slot + f.off_scales + 2 * (d >> 5)));
  }
  int c, bits, si;
  if (f.compact) {
    c = code3(slot, f.D, d);
    bits = 3;
    si = 0;
  } else if (d < f.k_wide) {
    c = code4(slot, d);
    bits = 4;
    si = d >> 6;
  } else {
    c = code3(slot + f.off_k_nope, f.D - f.k_wide, d - f.k_wide);
    bits = 3;
    si = d >> 6;
  }
  const float sc = h2f(rd16(slot + f.off_scales + 2 * si)) / (float)kLutOne;
  return (float)lut_value(c, bits) * sc;
}

__device__ __forceinline__ float v_value(const DevFmt& f, const uint8_t* slot, int d) {
  const uint8_t* seg = slot + f.off_v;
  if (f.kind == HKV_KIND_Q8_0)
    return (float)(int8_t)seg[d] * h2f(rd16(slot + f.off_scales + 2 * (f.D / 32 + (d >> 5))));
  if (f.kind == HKV_KIND_Q4_0) {
    const int c = code4(seg, d);
    return (float)(c - 8) * h2f(rd16(slot + f.off_scales + 2 * (f.D / 32 + (d >> 5))));
  }
  const int c = (f.v_bits == 4) ? code4(seg, d) : code3(seg, f.D, d);
  const float sc = h2f(rd16(slot + f.off_scales + 2 * f.num_k_scales)) / (float)kLutOne;
  return (float)lut_value(c, f.v_bits) * sc;
}

__device__ __forceinline__ const uint8_t* slot_ptr(const DevFmt& f, const uint8_t* cache,
                                                   int64_t page, int off, int num_kv_heads,
                                                   int h) {
  return cache + ((page * num_kv_heads + h) * (int64_t)f.page_size + off) * (int64_t)f.slot_bytes;
}

}  // namespace hkv
