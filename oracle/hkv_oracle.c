/*
 * hkv_oracle.c -- CPU oracle (test infrastructure only; see hkv_oracle.h).
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared -lm.
 * Every float operation below is one IEEE fp32 (or fp64) operation with
 * round-to-nearest-even; no fused multiply-add, no reassociation.
 */
#include "hkv_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Constants of the Octave format.                                           */
/* [OCT] OctaveFormat uses HADAMARD_BLOCK, ROPE_BITS and NOPE_BITS without   */
/* printing them; the module text fixes them: K is rotated in 64-dim blocks, */
/* RoPE blocks take 4-bit codes and NoPE blocks 3-bit codes.                 */
#define ORC_HADAMARD_BLOCK 64
#define ORC_ROPE_BITS 4
#define ORC_NOPE_BITS 3
/* READING: one LUT_ONE for every bit width ([OCT] reference_dequantize      */
/* divides all scales by the same constant); a power of two keeps the        */
/* division exact.                                                           */
#define ORC_LUT_ONE 64
/* Largest head size the oracle accepts. */
#define ORC_MAX_HEAD 4096

int32_t orc_lut_one(void) { return ORC_LUT_ONE; }

static int is_pow2(int32_t n) { return n > 0 && (n & (n - 1)) == 0; }

/* ------------------------------------------------------------------------ */
/* Format descriptor: [OCT] OctaveFormat (validation, from_cache_dtype,      */
/* kernel_code and the offset properties), and the Q4_0 slot READING.       */
int orc_format_init(orc_format* f, const char* cache_dtype, int32_t head_size,
                    int32_t rope_dim) {
  memset(f, 0, sizeof(*f));
  const int32_t d = head_size, r = rope_dim;
  if (strcmp(cache_dtype, "q4_0") == 0) {
    /* [Q4] "How" item 1-2: FWHT over the whole head (256 at D=256), Q4_0
     * blocks of 32 elements with one fp16 scale; no sign flips. */
    if (!is_pow2(d) || d < 32 || d > ORC_MAX_HEAD) return ORC_EINVAL;
    f->kind = ORC_KIND_Q4_0;
    f->head_size = d;
    f->rope_dim = 0;
    f->v_bits = 4;
    f->k_block = d;
    f->v_block = d;
    f->use_signs = 0;
    f->k_wide_dim = d;
    f->off_k_nope = d / 2; /* no NoPE part: equals off_v */
    f->off_v = d / 2;
    f->off_scales = d;
    f->num_k_scales = d / 32;
    f->num_scales = d / 16;
    f->slot_bytes = d + 2 * (d / 16);
    f->kernel_code = 0;
    return ORC_OK;
  }
  if (strcmp(cache_dtype, "q8_0") == 0) {
    /* READING of the int8 mode that [Q4] compares against (its footprint
     * note: the Q4_0 cache is half of Q8_0's; the merge note: int8 stays the
     * default) and that [M5] row 5 measures with FWHT: the same rotation as
     * Q4_0 (FWHT over the head, no signs) followed by the Q8_0 block type of
     * the GGML family, 32 int8 codes and one fp16 scale per block. */
    if (!is_pow2(d) || d < 32 || d > ORC_MAX_HEAD) return ORC_EINVAL;
    f->kind = ORC_KIND_Q8_0;
    f->head_size = d;
    f->rope_dim = 0;
    f->v_bits = 8;
    f->k_block = d;
    f->v_block = d;
    f->use_signs = 0;
    f->k_wide_dim = 0;
    f->off_k_nope = d; /* no NoPE part: equals off_v */
    f->off_v = d;
    f->off_scales = 2 * d;
    f->num_k_scales = d / 32;
    f->num_scales = d / 16;
    f->slot_bytes = 2 * d + 2 * (d / 16);
    f->kernel_code = 8;
    return ORC_OK;
  }
  int32_t v_bits, compact;
  if (strcmp(cache_dtype, "octave_k3v4") == 0) {
    v_bits = 4;
    compact = 0;
  } else if (strcmp(cache_dtype, "octave_k3v3") == 0) {
    v_bits = 3;
    compact = 0;
  } else if (strcmp(cache_dtype, "octave_k3v3_compact") == 0) {
    v_bits = 3;
    compact = 1;
  } else {
    return ORC_EINVAL;
  }
  /* [OCT] OctaveFormat.__post_init__ */
  if (v_bits != 3 && v_bits != 4) return ORC_EINVAL;
  if (compact && !is_pow2(d)) return ORC_EINVAL;
  if (d <= 0 || r < 0 || r % ORC_HADAMARD_BLOCK || d % ORC_HADAMARD_BLOCK)
    return ORC_EINVAL;
  if (d > ORC_MAX_HEAD) return ORC_EINVAL;
  /* READING: the NoPE part cannot have negative size. */
  if (r > d) return ORC_EINVAL;
  f->kind = ORC_KIND_OCTAVE;
  f->head_size = d;
  f->rope_dim = r;
  f->v_bits = v_bits;
  f->compact = compact;
  f->use_signs = 1;
  f->k_block = compact ? d : ORC_HADAMARD_BLOCK;           /* k_rotation_block */
  f->v_block = is_pow2(d) ? d : ORC_HADAMARD_BLOCK;         /* v_block */
  f->k_wide_dim = compact ? 0 : r;
  f->off_k_nope = f->k_wide_dim * ORC_ROPE_BITS / 8;
  f->off_v = f->off_k_nope + (d - f->k_wide_dim) * ORC_NOPE_BITS / 8;
  f->off_scales = f->off_v + d * v_bits / 8;
  f->num_k_scales = compact ? 1 : d / ORC_HADAMARD_BLOCK;
  f->num_scales = f->num_k_scales + 1;
  {
    const int32_t raw = f->off_scales + 2 * f->num_scales;
    const int32_t align = compact ? 4 : 8;
    f->slot_bytes = (raw + align - 1) / align * align;
  }
  f->kernel_code = v_bits + (compact ? 16 : 0);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* binary16 conversions (IEEE 754-2008), round to nearest, ties to even.     */
uint16_t orc_f32_to_f16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t exp = (u >> 23) & 0xffu;
  uint32_t man = u & 0x7fffffu;
  if (exp == 0xffu) { /* inf / nan */
    if (man) return (uint16_t)(sign | 0x7e00u | (man >> 13));
    return (uint16_t)(sign | 0x7c00u);
  }
  const int32_t e = (int32_t)exp - 127 + 15;
  if (e >= 31) return (uint16_t)(sign | 0x7c00u);
  if (e <= 0) { /* half subnormal (or zero) */
    if (e < -10) return (uint16_t)sign;
    man |= 0x800000u;
    const uint32_t shift = (uint32_t)(14 - e);
    uint32_t hm = man >> shift;
    const uint32_t rem = man & ((1u << shift) - 1u);
    const uint32_t halfway = 1u << (shift - 1u);
    if (rem > halfway || (rem == halfway && (hm & 1u))) hm++;
    return (uint16_t)(sign | hm);
  }
  uint32_t h = sign | ((uint32_t)e << 10) | (man >> 13);
  const uint32_t rem = man & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++; /* may carry to inf */
  return (uint16_t)h;
}

float orc_f16_to_f32(uint16_t h) {
  const uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
  const uint32_t exp = ((uint32_t)h >> 10) & 0x1fu;
  const uint32_t man = (uint32_t)h & 0x3ffu;
  uint32_t u;
  if (exp == 0) {
    if (man == 0) {
      u = sign;
    } else { /* subnormal: man * 2^-24, exact in fp32 */
      float v = (float)man * 5.9604644775390625e-08f;
      memcpy(&u, &v, 4);
      u |= sign;
    }
  } else if (exp == 31) {
    u = sign | 0x7f800000u | (man << 13);
  } else {
    u = sign | ((exp - 15u + 127u) << 23) | (man << 13);
  }
  float out;
  memcpy(&out, &u, 4);
  return out;
}

/* ------------------------------------------------------------------------ */
/* [OCT] fwht_blocks: stages h = 1, 2, 4, ... < block; at each stage the     */
/* pair (j, j+h) with bit h of j clear becomes (a+b, a-b); then one multiply */
/* by 1/sqrt(block).  The Python-double 1/sqrt(block) meets an fp32 tensor,  */
/* so it is rounded to fp32 first (torch semantics).                         */
void orc_fwht_f32(float* x, int32_t n, int32_t block) {
  const float norm = (float)(1.0 / sqrt((double)block));
  for (int32_t b0 = 0; b0 < n; b0 += block) {
    float* y = x + b0;
    for (int32_t h = 1; h < block; h *= 2) {
      for (int32_t i = 0; i < block; i += 2 * h) {
        for (int32_t j = i; j < i + h; ++j) {
          const float a = y[j];
          const float b = y[j + h];
          y[j] = a + b;
          y[j + h] = a - b;
        }
      }
    }
    for (int32_t j = 0; j < block; ++j) y[j] = y[j] * norm;
  }
}

void orc_fwht_f64(double* x, int32_t n, int32_t block) {
  const double norm = 1.0 / sqrt((double)block);
  for (int32_t b0 = 0; b0 < n; b0 += block) {
    double* y = x + b0;
    for (int32_t h = 1; h < block; h *= 2) {
      for (int32_t i = 0; i < block; i += 2 * h) {
        for (int32_t j = i; j < i + h; ++j) {
          const double a = y[j];
          const double b = y[j + h];
          y[j] = a + b;
          y[j + h] = a - b;
        }
      }
    }
    for (int32_t j = 0; j < block; ++j) y[j] = y[j] * norm;
  }
}

/* ------------------------------------------------------------------------ */
/* Sign pattern.  [OCT] signs / sign_bits give a fixed +-1 pattern per head  */
/* size, applied before the Hadamard transform, exported as int32 words with */
/* bit i set where the sign is -1.  The generator is not printed.            */
/* READING: SplitMix64 seeded with n; output word k supplies signs           */
/* 64k .. 64k+63, bit b set <=> sign -1.                                     */
uint64_t orc_splitmix64_next(uint64_t* state) {
  *state += 0x9E3779B97F4A7C15ull;
  uint64_t z = *state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

void orc_signs(int32_t n, float* s) {
  uint64_t state = (uint64_t)n;
  uint64_t word = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (i % 64 == 0) word = orc_splitmix64_next(&state);
    s[i] = ((word >> (i % 64)) & 1u) ? -1.0f : 1.0f;
  }
}

void orc_sign_bits(int32_t n, int32_t* words) {
  float* s = (float*)malloc(sizeof(float) * (size_t)n);
  orc_signs(n, s);
  for (int32_t w = 0; w < (n + 31) / 32; ++w) {
    uint32_t bits = 0;
    for (int32_t i = 0; i < 32 && 32 * w + i < n; ++i)
      if (s[32 * w + i] < 0.0f) bits |= 1u << i;
    memcpy(&words[w], &bits, 4);
  }
  free(s);
}

/* ------------------------------------------------------------------------ */
/* Lloyd-Max quantizer for N(0,1) (Lloyd 1957/1982; Max 1960): alternate     */
/* cell boundaries at level midpoints and levels at the cell centroids,      */
/* E[X | a < X < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)).                 */
static double std_pdf(double x) {
  if (isinf(x)) return 0.0;
  return exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
}
/* P(a < X < b), computed from the nearer tail to avoid cancellation. */
static double std_mass(double a, double b) {
  const double r2 = sqrt(2.0);
  if (a >= 0.0) return 0.5 * (erfc(a / r2) - erfc(b / r2));
  if (b <= 0.0) return 0.5 * (erfc(-b / r2) - erfc(-a / r2));
  return 1.0 - 0.5 * erfc(-a / r2) - 0.5 * erfc(b / r2);
}

void orc_lloyd_max(int32_t bits, double* L) {
  const int32_t N = 1 << bits;
  for (int32_t k = 0; k < N; ++k) L[k] = -3.0 + 6.0 * (k + 0.5) / N;
  double* nl = (double*)malloc(sizeof(double) * (size_t)N);
  for (int32_t it = 0; it < 200000; ++it) {
    double delta = 0.0;
    for (int32_t k = 0; k < N; ++k) {
      const double a = (k == 0) ? -INFINITY : 0.5 * (L[k - 1] + L[k]);
      const double b = (k == N - 1) ? INFINITY : 0.5 * (L[k] + L[k + 1]);
      nl[k] = (std_pdf(a) - std_pdf(b)) / std_mass(a, b);
      delta = fmax(delta, fabs(nl[k] - L[k]));
    }
    memcpy(L, nl, sizeof(double) * (size_t)N);
    if (delta < 1e-15) break;
  }
  free(nl);
}

/* READING of [OCT] "_lut" / LUT_MULT: integer codebook
 * lut[c] = round(level[c] * mult), mult the largest integer that keeps every
 * entry within int8. */
int32_t orc_codebook(int32_t bits, int32_t* lut) {
  const int32_t N = 1 << bits;
  double L[16];
  orc_lloyd_max(bits, L);
  int32_t mult = 1;
  while (lround(L[N - 1] * (double)(mult + 1)) <= 127) mult++;
  for (int32_t c = 0; c < N; ++c) lut[c] = (int32_t)lround(L[c] * (double)mult);
  return mult;
}

/* Codebooks are derived once, on first use (thread-safe). */
static pthread_once_t g_cb_once = PTHREAD_ONCE_INIT;
static int32_t g_lut[5][16];
static int32_t g_mult[5];
static void codebooks_build(void) {
  for (int32_t b = 3; b <= 4; ++b) g_mult[b] = orc_codebook(b, g_lut[b]);
}
static void codebooks_init(void) { pthread_once(&g_cb_once, codebooks_build); }

/* [OCT] _quantize_lut: torch.bucketize(y, midpoints) with right=False, i.e.
 * the number of midpoints strictly below y (a tie takes the lower code). */
int32_t orc_bucket(float y, int32_t bits) {
  codebooks_init();
  const int32_t N = 1 << bits;
  int32_t code = 0;
  for (int32_t k = 0; k + 1 < N; ++k) {
    const float mid = ((float)g_lut[bits][k] + (float)g_lut[bits][k + 1]) / 2.0f;
    if (mid < y) code++;
  }
  return code;
}

/* READING of the order of a block sum.  The pages sum the squares and the
 * products of a quantizer block over its last axis and leave the order of
 * the additions open.  Read here: the block is cut into pieces of
 * HADAMARD_BLOCK = 64 values, the unit the format rotates in ([OCT] module
 * text: every K block, and the V vector of a head size that is not a power
 * of two, are rotated in 64-value pieces).  The pieces are added position
 * by position first -- upper half of the pieces onto the lower half while
 * their count is even, then the remaining pieces from left to right -- and
 * the 64 partial sums are then folded the same way, upper half onto lower
 * half, down to one value.  A block shorter than 64 (a power of two) is
 * folded directly.  Every addition is one fp32 addition; t is overwritten. */
static float fold_halves(float* t, int32_t n) {
  while (n > 1 && n % 2 == 0) {
    const int32_t h = n / 2;
    for (int32_t i = 0; i < h; ++i) t[i] = t[i] + t[i + h];
    n = h;
  }
  float s = t[0];
  for (int32_t i = 1; i < n; ++i) s = s + t[i];
  return s;
}

static float block_sum_inplace(float* t, int32_t n) {
  const int32_t piece = ORC_HADAMARD_BLOCK;
  if (n <= piece || n % piece) return fold_halves(t, n);
  int32_t m = n / piece; /* pieces */
  while (m > 1 && m % 2 == 0) {
    const int32_t h = m / 2;
    for (int32_t i = 0; i < h * piece; ++i) t[i] = t[i] + t[i + h * piece];
    m = h;
  }
  for (int32_t b = 1; b < m; ++b)
    for (int32_t i = 0; i < piece; ++i) t[i] = t[i] + t[b * piece + i];
  return fold_halves(t, piece);
}

float orc_block_sum(const float* v, int32_t n) {
  float* t = (float*)malloc(sizeof(float) * (size_t)n);
  memcpy(t, v, sizeof(float) * (size_t)n);
  const float s = block_sum_inplace(t, n);
  free(t);
  return s;
}

/* [OCT] _quantize_lut over one block of n values: each value takes the
 * codebook entry nearest to it once the block is measured in units of its
 * RMS (the codebook is for N(0,1)), and the block's scale is chosen so that
 * the reconstruction x_hat keeps the dot product x . x_hat equal to |x|^2.
 * (A least-squares scale would shrink the reconstruction instead.)  The
 * steps and their fp32 roundings:
 *   ss    = block sum of x_i * x_i                     (order: orc_block_sum)
 *   rms   = sqrt(ss / n), at least 1e-12               (floor for zero blocks)
 *   c_i   = number of codebook midpoints below (x_i / rms) * LUT_MULT[bits]
 *   dot   = block sum of x_i * LUT[c_i]
 *   scale = LUT_ONE * (dot > 0 ? ss / max(dot, 1e-30) : 0)
 * so that x_i ~ LUT[c_i] * scale / LUT_ONE. */
static float block_rms(float ss, int32_t n) {
  const float r = sqrtf(ss / (float)n);
  return r < 1e-12f ? 1e-12f : r;
}

static float norm_preserving_scale(float ss, float dot) {
  const float q = dot > 0.0f ? ss / (dot > 1e-30f ? dot : 1e-30f) : 0.0f;
  return q * (float)ORC_LUT_ONE;
}

void orc_quantize_lut(const float* x, int32_t n, int32_t bits, uint8_t* codes,
                      float* scale) {
  codebooks_init();
  float* t = (float*)malloc(sizeof(float) * (size_t)n);
  for (int32_t i = 0; i < n; ++i) t[i] = x[i] * x[i];
  const float ss = block_sum_inplace(t, n);
  const float rms = block_rms(ss, n);
  const float mult = (float)g_mult[bits];
  for (int32_t i = 0; i < n; ++i) codes[i] = (uint8_t)orc_bucket((x[i] / rms) * mult, bits);
  for (int32_t i = 0; i < n; ++i) t[i] = x[i] * (float)g_lut[bits][codes[i]];
  const float dot = block_sum_inplace(t, n);
  *scale = norm_preserving_scale(ss, dot);
  free(t);
}

/* ------------------------------------------------------------------------ */
/* Q4_0 block of 32 values.  [Q4] fixes the block (32 codes of 4 bits and one
 * fp16 scale) and the maintainer's note fixes the max-abs tie-break
 * (a larger magnitude wins; equal magnitudes keep the larger signed value).
 * READING of the rest, the Q4_0 block type of the GGML family: the scale
 * d = m / -8 carries the sign of the chosen element m, so m maps to code 0;
 * code = min(15, trunc(x * (1/d) + 8.5)); the fp16 of d is stored. */
void orc_q4_0_block(const float* x, uint8_t* codes, uint16_t* d16) {
  float amax = 0.0f, mval = 0.0f;
  for (int32_t j = 0; j < 32; ++j) {
    const float v = x[j];
    const float a = fabsf(v);
    if (a > amax || (a == amax && v > mval)) {
      amax = a;
      mval = v;
    }
  }
  const float d = mval / -8.0f;
  const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  *d16 = orc_f32_to_f16(d);
  for (int32_t j = 0; j < 32; ++j) {
    const float t = x[j] * id;
    const float u = t + 8.5f;
    int32_t c = (int32_t)u; /* u >= 0: truncation is floor */
    if (c > 15) c = 15;
    codes[j] = (uint8_t)c;
  }
}

/* READING: the Q8_0 block type of the GGML family.  d = amax / 127 with
 * amax the largest magnitude, id = d != 0 ? 1/d : 0, code = round(x * id)
 * with halves away from zero (C roundf), so the largest-magnitude element
 * maps to +-127; the fp16 of d is stored. */
void orc_q8_0_block(const float* x, int8_t* codes, uint16_t* d16) {
  float amax = 0.0f;
  for (int32_t j = 0; j < 32; ++j) {
    const float a = fabsf(x[j]);
    if (a > amax) amax = a;
  }
  const float d = amax / 127.0f;
  const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  *d16 = orc_f32_to_f16(d);
  for (int32_t j = 0; j < 32; ++j) {
    const float t = x[j] * id;
    codes[j] = (int8_t)roundf(t);
  }
}

/* ------------------------------------------------------------------------ */
/* [OCT] _pack.  4-bit: every 8 codes form one little-endian word; byte j    */
/* holds code j in its low nibble and code j+4 in its high nibble.  3-bit: a */
/* plane of the low 2 bits (a word per 16 codes, byte j of word m holds      */
/* codes 16m+4i+j at bits 2i..2i+1) followed by a plane of the high bit (a   */
/* word per 32 codes, byte j of word m holds code 32m+4i+j at bit i).        */
void orc_pack(const uint8_t* c, int32_t n, int32_t bits, uint8_t* out) {
  if (bits == 4) {
    for (int32_t w = 0; w < n / 8; ++w)
      for (int32_t j = 0; j < 4; ++j)
        out[4 * w + j] = (uint8_t)((c[8 * w + j] & 15) | ((c[8 * w + 4 + j] & 15) << 4));
    return;
  }
  uint8_t* lo = out;
  uint8_t* hi = out + n / 4;
  for (int32_t m = 0; m < n / 16; ++m)
    for (int32_t j = 0; j < 4; ++j) {
      uint32_t b = 0;
      for (int32_t i = 0; i < 4; ++i) b |= (uint32_t)(c[16 * m + 4 * i + j] & 3) << (2 * i);
      lo[4 * m + j] = (uint8_t)b;
    }
  for (int32_t m = 0; m < n / 32; ++m)
    for (int32_t j = 0; j < 4; ++j) {
      uint32_t b = 0;
      for (int32_t i = 0; i < 8; ++i) b |= (uint32_t)((c[32 * m + 4 * i + j] >> 2) & 1) << i;
      hi[4 * m + j] = (uint8_t)b;
    }
}

void orc_unpack(const uint8_t* in, int32_t n, int32_t bits, uint8_t* c) {
  if (bits == 4) {
    for (int32_t w = 0; w < n / 8; ++w)
      for (int32_t j = 0; j < 4; ++j) {
        c[8 * w + j] = in[4 * w + j] & 15;
        c[8 * w + 4 + j] = in[4 * w + j] >> 4;
      }
    return;
  }
  const uint8_t* lo = in;
  const uint8_t* hi = in + n / 4;
  for (int32_t m = 0; m < n / 16; ++m)
    for (int32_t j = 0; j < 4; ++j)
      for (int32_t i = 0; i < 4; ++i)
        c[16 * m + 4 * i + j] = (lo[4 * m + j] >> (2 * i)) & 3;
  for (int32_t m = 0; m < n / 32; ++m)
    for (int32_t j = 0; j < 4; ++j)
      for (int32_t i = 0; i < 8; ++i)
        c[32 * m + 4 * i + j] |= (uint8_t)(((hi[4 * m + j] >> i) & 1) << 2);
}

/* ------------------------------------------------------------------------ */
static void put_f16(uint8_t* p, uint16_t h) {
  p[0] = (uint8_t)(h & 0xff);
  p[1] = (uint8_t)(h >> 8);
}
static uint16_t get_f16(const uint8_t* p) {
  return (uint16_t)(p[0] | ((uint16_t)p[1] << 8));
}

/* rotate(x, s, B) = fwht_blocks(x * s, B): signs first ([OCT] signs). */
static void rotate_f32(const orc_format* f, const float* s, float* x, int32_t block) {
  const int32_t d = f->head_size;
  if (f->use_signs)
    for (int32_t i = 0; i < d; ++i) x[i] = x[i] * s[i];
  orc_fwht_f32(x, d, block);
}
/* unrotate = inverse of rotate: the transform is its own inverse, then the
 * signs (READING of [OCT] unrotate, which is named but not printed). */
static void unrotate_f32(const orc_format* f, const float* s, float* x, int32_t block) {
  const int32_t d = f->head_size;
  orc_fwht_f32(x, d, block);
  if (f->use_signs)
    for (int32_t i = 0; i < d; ++i) x[i] = x[i] * s[i];
}

/* One (token, head): [OCT] reference_quantize; [Q4] for Q4_0. */
static void quantize_one(const orc_format* f, const float* sgn, const float* key,
                         const float* value, uint8_t* slot, float* kbuf,
                         float* vbuf, uint8_t* codes) {
  const int32_t d = f->head_size;
  memset(slot, 0, (size_t)f->slot_bytes); /* pad bytes stay zero */
  memcpy(kbuf, key, sizeof(float) * (size_t)d);
  memcpy(vbuf, value, sizeof(float) * (size_t)d);
  rotate_f32(f, sgn, kbuf, f->k_block);
  rotate_f32(f, sgn, vbuf, f->v_block);
  if (f->kind == ORC_KIND_Q8_0) {
    uint16_t h16;
    for (int32_t b = 0; b < d / 32; ++b) {
      orc_q8_0_block(kbuf + 32 * b, (int8_t*)(slot + 32 * b), &h16);
      put_f16(slot + f->off_scales + 2 * b, h16);
      orc_q8_0_block(vbuf + 32 * b, (int8_t*)(slot + f->off_v + 32 * b), &h16);
      put_f16(slot + f->off_scales + 2 * (d / 32 + b), h16);
    }
    return;
  }
  if (f->kind == ORC_KIND_Q4_0) {
    uint16_t h16;
    for (int32_t b = 0; b < d / 32; ++b) {
      orc_q4_0_block(kbuf + 32 * b, codes + 32 * b, &h16);
      put_f16(slot + f->off_scales + 2 * b, h16);
    }
    orc_pack(codes, d, 4, slot);
    for (int32_t b = 0; b < d / 32; ++b) {
      orc_q4_0_block(vbuf + 32 * b, codes + 32 * b, &h16);
      put_f16(slot + f->off_scales + 2 * (d / 32 + b), h16);
    }
    orc_pack(codes, d, 4, slot + f->off_v);
    return;
  }
  float ks[ORC_MAX_HEAD / ORC_HADAMARD_BLOCK];
  if (f->compact) {
    orc_quantize_lut(kbuf, d, ORC_NOPE_BITS, codes, &ks[0]);
    orc_pack(codes, d, ORC_NOPE_BITS, slot);
  } else {
    const int32_t nkb = d / ORC_HADAMARD_BLOCK;
    const int32_t nr = f->rope_dim / ORC_HADAMARD_BLOCK;
    for (int32_t b = 0; b < nkb; ++b)
      orc_quantize_lut(kbuf + ORC_HADAMARD_BLOCK * b, ORC_HADAMARD_BLOCK,
                       b < nr ? ORC_ROPE_BITS : ORC_NOPE_BITS,
                       codes + ORC_HADAMARD_BLOCK * b, &ks[b]);
    orc_pack(codes, f->rope_dim, ORC_ROPE_BITS, slot);
    orc_pack(codes + f->rope_dim, d - f->rope_dim, ORC_NOPE_BITS, slot + f->off_k_nope);
  }
  float vs;
  orc_quantize_lut(vbuf, d, f->v_bits, codes, &vs);
  orc_pack(codes, d, f->v_bits, slot + f->off_v);
  for (int32_t i = 0; i < f->num_k_scales; ++i)
    put_f16(slot + f->off_scales + 2 * i, orc_f32_to_f16(ks[i]));
  put_f16(slot + f->off_scales + 2 * f->num_k_scales, orc_f32_to_f16(vs));
}

void orc_quantize(const orc_format* f, const float* key, const float* value,
                  int64_t num_tokens, int32_t num_heads, uint8_t* slots) {
  const int32_t d = f->head_size;
  float* sgn = (float*)malloc(sizeof(float) * (size_t)d);
  float* kb = (float*)malloc(sizeof(float) * (size_t)d);
  float* vb = (float*)malloc(sizeof(float) * (size_t)d);
  uint8_t* codes = (uint8_t*)malloc((size_t)d);
  orc_signs(d, sgn);
  for (int64_t t = 0; t < num_tokens; ++t)
    for (int32_t h = 0; h < num_heads; ++h) {
      const int64_t i = t * num_heads + h;
      quantize_one(f, sgn, key + i * d, value + i * d, slots + i * f->slot_bytes, kb, vb, codes);
    }
  free(sgn);
  free(kb);
  free(vb);
  free(codes);
}

/* Rotated-space dequantization of one slot ([OCT] reference_dequantize with
 * rotated=True): code value times (fp16 scale / LUT_ONE) for Octave,
 * (code - 8) times the fp16 scale for Q4_0, and the int8 code times the fp16
 * scale for Q8_0.  All are exact in fp32. */
static void dequant_k_rot(const orc_format* f, const uint8_t* slot, float* k, uint8_t* codes) {
  const int32_t d = f->head_size;
  if (f->kind == ORC_KIND_Q8_0) {
    for (int32_t i = 0; i < d; ++i)
      k[i] = (float)(int8_t)slot[i] * orc_f16_to_f32(get_f16(slot + f->off_scales + 2 * (i / 32)));
    return;
  }
  if (f->kind == ORC_KIND_Q4_0) {
    orc_unpack(slot, d, 4, codes);
    for (int32_t i = 0; i < d; ++i)
      k[i] = (float)((int32_t)codes[i] - 8) * orc_f16_to_f32(get_f16(slot + f->off_scales + 2 * (i / 32)));
    return;
  }
  codebooks_init();
  const float one = (float)ORC_LUT_ONE;
  if (f->compact) {
    orc_unpack(slot, d, ORC_NOPE_BITS, codes);
    const float sc = orc_f16_to_f32(get_f16(slot + f->off_scales)) / one;
    for (int32_t i = 0; i < d; ++i) k[i] = (float)g_lut[ORC_NOPE_BITS][codes[i]] * sc;
    return;
  }
  const int32_t r = f->rope_dim;
  orc_unpack(slot, r, ORC_ROPE_BITS, codes);
  orc_unpack(slot + f->off_k_nope, d - r, ORC_NOPE_BITS, codes + r);
  for (int32_t i = 0; i < d; ++i) {
    const int32_t b = i / ORC_HADAMARD_BLOCK;
    const float sc = orc_f16_to_f32(get_f16(slot + f->off_scales + 2 * b)) / one;
    const int32_t lv = i < r ? g_lut[ORC_ROPE_BITS][codes[i]] : g_lut[ORC_NOPE_BITS][codes[i]];
    k[i] = (float)lv * sc;
  }
}

static void dequant_v_rot(const orc_format* f, const uint8_t* slot, float* v, uint8_t* codes) {
  const int32_t d = f->head_size;
  if (f->kind == ORC_KIND_Q8_0) {
    for (int32_t i = 0; i < d; ++i)
      v[i] = (float)(int8_t)slot[f->off_v + i] *
             orc_f16_to_f32(get_f16(slot + f->off_scales + 2 * (d / 32 + i / 32)));
    return;
  }
  if (f->kind == ORC_KIND_Q4_0) {
    orc_unpack(slot + f->off_v, d, 4, codes);
    for (int32_t i = 0; i < d; ++i)
      v[i] = (float)((int32_t)codes[i] - 8) *
             orc_f16_to_f32(get_f16(slot + f->off_scales + 2 * (d / 32 + i / 32)));
    return;
  }
  codebooks_init();
  orc_unpack(slot + f->off_v, d, f->v_bits, codes);
  const float sc = orc_f16_to_f32(get_f16(slot + f->off_scales + 2 * f->num_k_scales)) /
                   (float)ORC_LUT_ONE;
  for (int32_t i = 0; i < d; ++i) v[i] = (float)g_lut[f->v_bits][codes[i]] * sc;
}

void orc_dequantize(const orc_format* f, const uint8_t* slots, int64_t num_tokens,
                    int32_t num_heads, int32_t rotated, float* k_out, float* v_out) {
  const int32_t d = f->head_size;
  float* sgn = (float*)malloc(sizeof(float) * (size_t)d);
  uint8_t* codes = (uint8_t*)malloc((size_t)d);
  orc_signs(d, sgn);
  for (int64_t i = 0; i < num_tokens * num_heads; ++i) {
    const uint8_t* slot = slots + i * f->slot_bytes;
    float* k = k_out + i * d;
    float* v = v_out + i * d;
    dequant_k_rot(f, slot, k, codes);
    dequant_v_rot(f, slot, v, codes);
    if (!rotated) {
      unrotate_f32(f, sgn, k, f->k_block);
      unrotate_f32(f, sgn, v, f->v_block);
    }
  }
  free(sgn);
  free(codes);
}

/* Exact inverse rotation of the exact rotated values, in fp64. */
static void unrotate_f64(const orc_format* f, const float* sgn, const float* in,
                         double* out, int32_t block) {
  const int32_t d = f->head_size;
  for (int32_t i = 0; i < d; ++i) out[i] = (double)in[i];
  orc_fwht_f64(out, d, block);
  if (f->use_signs)
    for (int32_t i = 0; i < d; ++i) out[i] = out[i] * (double)sgn[i];
}

void orc_dequantize_f64(const orc_format* f, const uint8_t* slots, int64_t num_tokens,
                        int32_t num_heads, double* k_out, double* v_out) {
  const int32_t d = f->head_size;
  float* sgn = (float*)malloc(sizeof(float) * (size_t)d);
  float* tmp = (float*)malloc(sizeof(float) * (size_t)d);
  uint8_t* codes = (uint8_t*)malloc((size_t)d);
  orc_signs(d, sgn);
  for (int64_t i = 0; i < num_tokens * num_heads; ++i) {
    const uint8_t* slot = slots + i * f->slot_bytes;
    dequant_k_rot(f, slot, tmp, codes);
    unrotate_f64(f, sgn, tmp, k_out + i * d, f->k_block);
    dequant_v_rot(f, slot, tmp, codes);
    unrotate_f64(f, sgn, tmp, v_out + i * d, f->v_block);
  }
  free(sgn);
  free(tmp);
  free(codes);
}

/* ------------------------------------------------------------------------ */
/* [OCT] reference_attention, as its definition: query token i attends to the
 * first klen_i tokens of request q_to_req[i] (klen <= 0 gives a zero row);
 * query head h reads KV head h / (Hq / Hkv); out = softmax(scale * q.K^T) V
 * with K, V the dequantized cache in the unrotated space.  All in fp64. */
/* The attention of every query row, and, if lse is not NULL, the natural
 * log of its softmax denominator, m + log(l) over the row's scores
 * (sm_scale included); rows with no tokens get -inf. */
static void attention_rows(const orc_format* f, const float* query, int32_t num_q,
                           int32_t num_q_heads, const uint8_t* cache, int32_t num_kv_heads,
                           int32_t page_size, const int32_t* block_table,
                           int32_t max_pages_per_req, const int32_t* q_to_req,
                           const int32_t* q_to_klen, double sm_scale, double* out,
                           double* lse) {
  const int32_t d = f->head_size;
  const int32_t group = num_q_heads / num_kv_heads;
  float* sgn = (float*)malloc(sizeof(float) * (size_t)d);
  float* tmp = (float*)malloc(sizeof(float) * (size_t)d);
  double* vec = (double*)malloc(sizeof(double) * (size_t)d);
  double* acc = (double*)malloc(sizeof(double) * (size_t)d * (size_t)group);
  uint8_t* codes = (uint8_t*)malloc((size_t)d);
  orc_signs(d, sgn);
  memset(out, 0, sizeof(double) * (size_t)num_q * (size_t)num_q_heads * (size_t)d);
  if (lse)
    for (int64_t r = 0; r < (int64_t)num_q * num_q_heads; ++r) lse[r] = -INFINITY;
  for (int32_t i = 0; i < num_q; ++i) {
    const int32_t klen = q_to_klen[i];
    if (klen <= 0) continue;
    const int32_t req = q_to_req[i];
    double* s = (double*)malloc(sizeof(double) * (size_t)klen * (size_t)group);
    for (int32_t kvh = 0; kvh < num_kv_heads; ++kvh) {
      /* scores */
      for (int32_t t = 0; t < klen; ++t) {
        const int64_t page = block_table[(int64_t)req * max_pages_per_req + t / page_size];
        const uint8_t* slot =
            cache + ((page * num_kv_heads + kvh) * page_size + t % page_size) * f->slot_bytes;
        dequant_k_rot(f, slot, tmp, codes);
        unrotate_f64(f, sgn, tmp, vec, f->k_block);
        for (int32_t g = 0; g < group; ++g) {
          const float* q = query + ((int64_t)i * num_q_heads + kvh * group + g) * d;
          double dot = 0.0;
          for (int32_t j = 0; j < d; ++j) dot += (double)q[j] * vec[j];
          s[(int64_t)g * klen + t] = dot * sm_scale;
        }
      }
      /* softmax */
      for (int32_t g = 0; g < group; ++g) {
        double* sg = s + (int64_t)g * klen;
        double m = -INFINITY;
        for (int32_t t = 0; t < klen; ++t) m = fmax(m, sg[t]);
        double l = 0.0;
        for (int32_t t = 0; t < klen; ++t) {
          sg[t] = exp(sg[t] - m);
          l += sg[t];
        }
        for (int32_t t = 0; t < klen; ++t) sg[t] /= l;
        if (lse) lse[(int64_t)i * num_q_heads + kvh * group + g] = m + log(l);
      }
      /* weighted sum of V */
      memset(acc, 0, sizeof(double) * (size_t)d * (size_t)group);
      for (int32_t t = 0; t < klen; ++t) {
        const int64_t page = block_table[(int64_t)req * max_pages_per_req + t / page_size];
        const uint8_t* slot =
            cache + ((page * num_kv_heads + kvh) * page_size + t % page_size) * f->slot_bytes;
        dequant_v_rot(f, slot, tmp, codes);
        unrotate_f64(f, sgn, tmp, vec, f->v_block);
        for (int32_t g = 0; g < group; ++g) {
          const double p = s[(int64_t)g * klen + t];
          for (int32_t j = 0; j < d; ++j) acc[(int64_t)g * d + j] += p * vec[j];
        }
      }
      for (int32_t g = 0; g < group; ++g)
        memcpy(out + ((int64_t)i * num_q_heads + kvh * group + g) * d, acc + (int64_t)g * d,
               sizeof(double) * (size_t)d);
    }
    free(s);
  }
  free(sgn);
  free(tmp);
  free(vec);
  free(acc);
  free(codes);
}

void orc_attention(const orc_format* f, const float* query, int32_t num_q,
                   int32_t num_q_heads, const uint8_t* cache, int32_t num_kv_heads,
                   int32_t page_size, const int32_t* block_table,
                   int32_t max_pages_per_req, const int32_t* q_to_req,
                   const int32_t* q_to_klen, double sm_scale, double* out) {
  attention_rows(f, query, num_q, num_q_heads, cache, num_kv_heads, page_size, block_table,
                 max_pages_per_req, q_to_req, q_to_klen, sm_scale, out, NULL);
}

void orc_attention_lse(const orc_format* f, const float* query, int32_t num_q,
                       int32_t num_q_heads, const uint8_t* cache, int32_t num_kv_heads,
                       int32_t page_size, const int32_t* block_table,
                       int32_t max_pages_per_req, const int32_t* q_to_req,
                       const int32_t* q_to_klen, double sm_scale, double* out, double* lse) {
  attention_rows(f, query, num_q, num_q_heads, cache, num_kv_heads, page_size, block_table,
                 max_pages_per_req, q_to_req, q_to_klen, sm_scale, out, lse);
}
