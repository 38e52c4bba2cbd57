/*
 * hkv_oracle.h -- CPU oracle for the FWHT-rotated low-bit paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-threaded C
 * restatement of what the sources compute.  Only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or constant generator with the GPU library; the GPU library
 * never loads it.
 *
 * Sources (cited by page title and section):
 *   [Q4]  Strata pull request #21, "optional 4-bit (Q4_0) quantized KV cache
 *         mode with FWHT-256 rotation": sections "How" and "Verification",
 *         and the maintainer's merge note.
 *   [OCT] vLLM API docs, "vllm.v1.attention.ops.rocm_octave": module text,
 *         OctaveFormat, _pack, _quantize_lut, fwht_blocks,
 *         reference_attention, reference_dequantize, reference_quantize,
 *         sign_bits, signs, v_block.
 *
 * Readings taken where the sources are silent are marked READING below.
 *
 * Precision: quantize / pack / dequantize follow the sources' fp32
 * arithmetic step by step (float32 torch code in [OCT]); the attention is
 * its plain definition evaluated in fp64.
 *
 * Parity status: every function here is pinned by the CPU test-suite
 * (closed forms, textbook tables, library routines, brute force).  What is
 * NOT pinned is agreement with the bytes of the original projects, because
 * their constants (sign generator, codebook integers) are not published:
 * the sign generator and the integer codebooks are READINGS.
 */
#ifndef HKV_ORACLE_H
#define HKV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_KIND_Q4_0 = 0, ORC_KIND_OCTAVE = 1, ORC_KIND_Q8_0 = 2 };
enum { ORC_OK = 0, ORC_EINVAL = 1 };

/* Format descriptor; field meanings follow [OCT] OctaveFormat.  For Q4_0 the
 * slot is READING: [K nibbles D/2][V nibbles D/2][K fp16 scales D/32]
 * [V fp16 scales D/32].  For Q8_0 (READING, below) it is [K int8 D][V int8 D]
 * [K fp16 scales D/32][V fp16 scales D/32]. */
typedef struct {
  int32_t kind;
  int32_t head_size;
  int32_t rope_dim;
  int32_t v_bits;
  int32_t compact;
  int32_t k_block;      /* K (and query) rotation block                    */
  int32_t v_block;      /* V (and output) rotation block                   */
  int32_t use_signs;    /* Octave: 1, Q4_0: 0                              */
  int32_t k_wide_dim;   /* K dims with 4-bit codes (Octave RoPE part)      */
  int32_t off_k_nope;
  int32_t off_v;
  int32_t off_scales;
  int32_t num_k_scales;
  int32_t num_scales;
  int32_t slot_bytes;
  int32_t kernel_code;
} orc_format;

/* "q4_0", "q8_0", "octave_k3v4", "octave_k3v3", "octave_k3v3_compact". */
int orc_format_init(orc_format* f, const char* cache_dtype, int32_t head_size,
                    int32_t rope_dim);

/* IEEE binary16 <-> binary32, round to nearest even. */
uint16_t orc_f32_to_f16(float x);
float orc_f16_to_f32(uint16_t h);

/* Blockwise orthonormal Hadamard rotation: every run of `block` values is
 * transformed on its own ([OCT] fwht_blocks), in fp32 and in fp64.  n must
 * be a multiple of block. */
void orc_fwht_f32(float* x, int32_t n, int32_t block);
void orc_fwht_f64(double* x, int32_t n, int32_t block);

/* SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): one step. */
uint64_t orc_splitmix64_next(uint64_t* state);
/* Sign pattern of length n ([OCT] signs / sign_bits; generator READING). */
void orc_signs(int32_t n, float* s);
void orc_sign_bits(int32_t n, int32_t* words);

/* Lloyd-Max levels for N(0,1) with 2^bits levels, by Lloyd iteration. */
void orc_lloyd_max(int32_t bits, double* levels);
/* Integer codebook: lut[c] = round(level[c] * mult), mult the largest
 * integer keeping |lut| <= 127 (READING).  Returns mult. */
int32_t orc_codebook(int32_t bits, int32_t* lut);
int32_t orc_lut_one(void);
/* Code of a normalised value y: the number of codebook midpoints < y. */
int32_t orc_bucket(float y, int32_t bits);

/* Sum of n fp32 values in the order the quantizer block sums use (READING:
 * 64-value pieces added position by position, then folded in halves). */
float orc_block_sum(const float* v, int32_t n);

/* Block quantizers. */
void orc_quantize_lut(const float* x, int32_t n, int32_t bits, uint8_t* codes,
                      float* scale);
void orc_q4_0_block(const float* x, uint8_t* codes, uint16_t* d16);
/* Q8_0 block of 32 values: int8 codes in [-127, 127] and the fp16 scale. */
void orc_q8_0_block(const float* x, int8_t* codes, uint16_t* d16);

/* Bit packing of [OCT] _pack (4- and 3-bit) and its inverse. */
void orc_pack(const uint8_t* codes, int32_t n, int32_t bits, uint8_t* out);
void orc_unpack(const uint8_t* in, int32_t n, int32_t bits, uint8_t* codes);

/* (T, H, D) fp32 K and V -> (T, H, slot_bytes) slots. */
void orc_quantize(const orc_format* f, const float* key, const float* value,
                  int64_t num_tokens, int32_t num_heads, uint8_t* slots);

/* (T, H, slot) -> fp32 K, V (T, H, D); rotated != 0 keeps the rotated space. */
void orc_dequantize(const orc_format* f, const uint8_t* slots,
                    int64_t num_tokens, int32_t num_heads, int32_t rotated,
                    float* k_out, float* v_out);
/* Same, unrotated, with the inverse rotation evaluated in fp64. */
void orc_dequantize_f64(const orc_format* f, const uint8_t* slots,
                        int64_t num_tokens, int32_t num_heads, double* k_out,
                        double* v_out);

/* Per-query-token attention over a paged cache ([OCT] reference_attention),
 * evaluated in fp64.  query (Q, Hq, D) fp32; cache (pages, Hkv, page_size,
 * slot) bytes; block_table (R, max_pages) int32; out (Q, Hq, D) fp64. */
void orc_attention(const orc_format* f, const float* query, int32_t num_q,
                   int32_t num_q_heads, const uint8_t* cache,
                   int32_t num_kv_heads, int32_t page_size,
                   const int32_t* block_table, int32_t max_pages_per_req,
                   const int32_t* q_to_req, const int32_t* q_to_klen,
                   double sm_scale, double* out);

/* orc_attention plus lse (Q, Hq) fp64: the natural log of each row's softmax
 * denominator, m + log(sum exp(s - m)) over its scaled scores, -inf for a row
 * with no tokens.  Attention over disjoint token ranges merges exactly:
 * out = sum_k exp(lse_k - lse) out_k with lse = log sum_k exp(lse_k). */
void orc_attention_lse(const orc_format* f, const float* query, int32_t num_q,
                       int32_t num_q_heads, const uint8_t* cache,
                       int32_t num_kv_heads, int32_t page_size,
                       const int32_t* block_table, int32_t max_pages_per_req,
                       const int32_t* q_to_req, const int32_t* q_to_klen,
                       double sm_scale, double* out, double* lse);

#ifdef __cplusplus
}
#endif
#endif
