/*
 * hkv.h -- C ABI of libhkv: FWHT-rotated low-bit paged KV cache and decode
 * attention for AMD Instinct MI355X (gfx950).
 *
 * The operations are the ones defined by two public sources, cited by page
 * title and section:
 *   [Q4]  Strata pull request #21, "optional 4-bit (Q4_0) quantized KV cache
 *         mode with FWHT-256 rotation" ("How" items 1-2 and the
 *         maintainer's merge note).
 *   [OCT] vLLM API docs, "vllm.v1.attention.ops.rocm_octave" (module text,
 *         OctaveFormat, _pack, _quantize_lut, fwht_blocks, reference_quantize,
 *         reference_dequantize, reference_attention, signs, v_block).
 *
 * Conventions common to every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns and
 *     allocates every buffer, including the decode workspace; the library
 *     allocates no memory and keeps no state besides its code and the
 *     static scratch of hkv_decode_attention_noalloc.
 *   - Every call is asynchronous on `stream` (a hipStream_t, passed as void*;
 *     NULL is the legacy default stream); nothing synchronizes the host.
 *   - Arguments the host can check (format, sizes, null pointers, alignment,
 *     workspace size) are checked before anything is enqueued; on failure
 *     the call returns a non-zero hkv_status, enqueues nothing, and
 *     hkv_last_error() describes the problem.  A failed kernel launch returns
 *     HKV_ERR_HIP.
 *   - Index arrays that live on the device (slot_mapping, slot_ids,
 *     block_table, q_to_req, q_to_klen) are trusted: out-of-range values are
 *     undefined behaviour, as in the sources' reference code.
 *   - Tensors are dense, row-major (last index fastest).
 */
#ifndef HKV_H
#define HKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HKV_OK = 0,
  HKV_ERR_INVALID_ARG = 1,
  HKV_ERR_UNSUPPORTED = 2,
  HKV_ERR_WORKSPACE = 3,
  HKV_ERR_HIP = 4
} hkv_status;

/* Element types.  Entry points take them as int32_t (an hkv_dtype value), so
 * that an out-of-range value from a caller is an error the library reports,
 * not an invalid enum. */
typedef enum { HKV_F32 = 0, HKV_F16 = 1 } hkv_dtype;

typedef enum { HKV_KIND_Q4_0 = 0, HKV_KIND_OCTAVE = 1, HKV_KIND_Q8_0 = 2 } hkv_kind;

/* Largest head size the GPU kernels take. */
#define HKV_MAX_HEAD 256

/*
 * Cache format descriptor, filled by hkv_format_init; plain data owned by
 * the caller.  Field meanings follow [OCT] OctaveFormat (k_wide_dim,
 * off_k_nope, off_v, off_scales, num_k_scales, num_scales, slot_bytes,
 * kernel_code, k_rotation_block -> k_block, v_block).
 *
 * Slot = the bytes stored per (token, KV head):
 *   Octave: [k_rope codes][k_nope codes][v codes][fp16 scales][zero pad]
 *           ([OCT] module text; 4-bit and 3-bit packing as in _pack).
 *   Q4_0:   [K nibbles D/2][V nibbles D/2][K fp16 scales D/32][V fp16
 *           scales D/32]; nibbles in the 4-bit order of [OCT] _pack; one
 *           scale per 32 values ([Q4] "How" item 2).
 *   Q8_0:   [K int8 D][V int8 D][K fp16 scales D/32][V fp16 scales D/32]:
 *           the int8 mode [Q4] compares its footprint against, after the
 *           same rotation; codes round(x / d) with d = max|x| / 127 per 32
 *           values, halves away from zero.
 * sign_bits: the fixed +-1 pattern applied before the Hadamard transform
 *   ([OCT] signs / sign_bits), bit i of the words set where the sign is -1;
 *   all zero for Q4_0, which has no sign flips ([Q4] "How" item 1).
 */
typedef struct {
  int32_t kind;         /* hkv_kind                                        */
  int32_t head_size;    /* D                                               */
  int32_t rope_dim;     /* leading K dims that take 4-bit codes (Octave)   */
  int32_t v_bits;       /* 3 or 4 (8 for Q8_0)                             */
  int32_t compact;      /* Octave compact K (one full-head rotation)       */
  int32_t page_size;    /* tokens per cache page                           */
  int32_t k_block;      /* FWHT block of K and of the query                */
  int32_t v_block;      /* FWHT block of V and of the output               */
  int32_t k_wide_dim;
  int32_t off_k_nope;
  int32_t off_v;
  int32_t off_scales;
  int32_t num_k_scales;
  int32_t num_scales;
  int32_t slot_bytes;
  int32_t kernel_code;  /* [OCT] kernel_code: v_bits + 16*compact; 0 = Q4_0, 8 = Q8_0 */
  uint32_t sign_bits[HKV_MAX_HEAD / 32];
} hkv_format;

/*
 * hkv_format_init -- fill *f for a cache dtype.
 *   cache_dtype (host): "q4_0", "q8_0", "octave_k3v4", "octave_k3v3",
 *                       "octave_k3v3_compact" ([OCT] from_cache_dtype).
 *   head_size: Octave: multiple of 64, <= 256 (compact: a power of two);
 *              Q4_0 and Q8_0: 64, 128 or 256.
 *   rope_dim:  Octave: multiple of 64, <= head_size; ignored for Q4_0/Q8_0.
 *   page_size: tokens per page, 1..1024.
 * Errors mirror [OCT] OctaveFormat validation: HKV_ERR_INVALID_ARG.
 * Enqueues nothing.
 */
hkv_status hkv_format_init(hkv_format* f, const char* cache_dtype, int32_t head_size,
                           int32_t rope_dim, int32_t page_size);

/*
 * hkv_quantize_append -- rotate, quantize and pack K/V rows into their cache
 * slots ([OCT] reference_quantize; [Q4] "How" items 1-2).
 *   key, value:   (num_tokens, num_kv_heads, D), in_dtype f32 or f16.
 *   slot_mapping: (num_tokens,) int64: page * page_size + offset of each
 *                 token; negative entries are skipped.
 *   cache:        (num_pages, num_kv_heads, page_size, slot_bytes) uint8,
 *                 16-byte aligned; only the addressed slots are written.
 * The packed bytes are a pure function of the K/V values (deterministic).
 */
hkv_status hkv_quantize_append(const hkv_format* f /*host*/, const void* key,
                               const void* value, int32_t in_dtype,
                               int64_t num_tokens, int32_t num_kv_heads,
                               const int64_t* slot_mapping, uint8_t* cache,
                               void* stream);

/*
 * hkv_dequantize -- slots back to fp32 K and V ([OCT] reference_dequantize).
 *   slot_ids: (num_tokens,) int64, page * page_size + offset; a negative id
 *             gives zero rows.
 *   rotated:  non-zero keeps K and V in the rotated space the decode kernels
 *             use; zero applies the inverse rotation.
 *   k_out, v_out: (num_tokens, num_kv_heads, D) fp32.
 */
hkv_status hkv_dequantize(const hkv_format* f /*host*/, const uint8_t* cache,
                          int32_t num_kv_heads, const int64_t* slot_ids,
                          int64_t num_tokens, int32_t rotated, float* k_out,
                          float* v_out, void* stream);

/*
 * hkv_decode_workspace_bytes -- bytes of device workspace hkv_decode_attention
 * needs for these sizes (0 on invalid arguments).  max_klen is a host upper
 * bound of q_to_klen.
 * The workspace holds the split partial results; its contents need no
 * initialisation.  Calls that overlap in time must not share a workspace.
 */
size_t hkv_decode_workspace_bytes(const hkv_format* f /*host*/, int32_t num_queries,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t max_klen, int32_t queries_per_seq);

/* hkv_decode_attention flags. */
#define HKV_DECODE_DETERMINISTIC 1u

/*
 * hkv_decode_attention -- per-query-token attention over the paged quantized
 * cache ([OCT] reference_attention; query rotated like K and output rotated
 * back, [OCT] module text and [Q4] merge note).
 *   query:        (num_queries, num_q_heads, D), q_dtype f32 or f16.
 *   cache:        (num_pages, num_kv_heads, page_size, slot_bytes) uint8.
 *   block_table:  (num_seqs, max_pages_per_req) int32 page ids.
 *   q_to_req:     (num_queries,) int32 sequence of each query token.
 *   q_to_klen:    (num_queries,) int32: the query attends to the first
 *                 q_to_klen[i] tokens of its sequence; <= 0 gives a zero row.
 *   max_klen:     host upper bound of q_to_klen (sizes the split-K grid).
 *   queries_per_seq: the queries come in consecutive groups of this many
 *                 that share one sequence (1..16; a group's query rows --
 *                 num_q_heads / num_kv_heads per query -- read the cache
 *                 once per pass; more rows than a pass takes are split into
 *                 sub-groups of whole queries, each reading the cache).
 *                 num_queries must be a multiple.
 *   sm_scale:     softmax scale applied to q.k.
 *   flags:        0 or HKV_DECODE_DETERMINISTIC.  By default the waves of a
 *                 workgroup take the split's 32-token units from a shared
 *                 queue, which balances their load but lets the summation
 *                 order, and so the last bits of the result, vary between
 *                 calls.  HKV_DECODE_DETERMINISTIC gives each wave a fixed
 *                 set of units: bitwise the same result for the same inputs
 *                 on every call, at a cost of a few percent.
 *   out:          (num_queries, num_q_heads, D) fp32, unrotated space.
 *   workspace:    >= hkv_decode_workspace_bytes(...) bytes, 16-byte aligned.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
hkv_status hkv_decode_attention(const hkv_format* f /*host*/, const void* query,
                                int32_t q_dtype, int32_t num_queries,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                const uint8_t* cache, const int32_t* block_table,
                                int32_t max_pages_per_req, const int32_t* q_to_req,
                                const int32_t* q_to_klen, int32_t max_klen,
                                int32_t queries_per_seq, float sm_scale, uint32_t flags,
                                float* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Bytes of the static per-device scratch of hkv_decode_attention_noalloc. */
#define HKV_DECODE_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * hkv_decode_attention_noalloc -- hkv_decode_attention for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * kernels as hkv_decode_attention, without the workspace: the split partial
 * records go to a scratch array of HKV_DECODE_SCRATCH_BYTES (64 MiB) that the
 * library holds on each device it runs on, from the first call on that
 * device until the process ends.  The call itself allocates nothing.
 *   - The device is the current device; stream must belong to it.
 *   - Sizes whose hkv_decode_workspace_bytes exceeds
 *     HKV_DECODE_SCRATCH_BYTES return HKV_ERR_WORKSPACE and enqueue nothing
 *     (e.g. 64 sequences x 4 query tokens x 32 query heads over 4 KV heads at
 *     32K tokens needs 65 MiB: use hkv_decode_attention there).
 *   - All calls on one device share its scratch, and the scratch keeps the
 *     last call's contents (no call needs it zeroed).  Calls that may overlap
 *     in time on one device -- on different streams, or from different host
 *     threads without ordering -- race on it; order them on one stream.
 */
hkv_status hkv_decode_attention_noalloc(const hkv_format* f /*host*/, const void* query,
                                        int32_t q_dtype, int32_t num_queries,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        const uint8_t* cache, const int32_t* block_table,
                                        int32_t max_pages_per_req, const int32_t* q_to_req,
                                        const int32_t* q_to_klen, int32_t max_klen,
                                        int32_t queries_per_seq, float sm_scale,
                                        uint32_t flags, float* out, void* stream);

/*
 * hkv_hadamard -- blockwise orthonormal Walsh-Hadamard rotation of rows, the
 * rotation of the cache formats as an operation of its own ([OCT]
 * fwht_blocks, signs / sign_bits; the block-128 activation rotation of
 * Strata pull request #928, "What's in it").
 *   x:          (rows, n), in_dtype f32 or f16; 16-byte (f32) or 8-byte (f16)
 *               aligned.  n is a positive multiple of block.
 *   y:          (rows, n) fp32, 16-byte aligned.  y may be x itself (in place)
 *               when in_dtype is f32; any other overlap is an error.
 *   block:      64, 128 or 256.
 *   sign_bits:  NULL (no signs) or (n/32,) uint32 words, 4-byte aligned: bit
 *               i of word k set negates element 32k + i of every row.
 *   inverse:    0 rotates, y = FWHT_block(x * s); non-zero unrotates,
 *               y = FWHT_block(x) * s.
 * FWHT_block runs the butterfly stages h = 1, 2, ..., block/2 on pairs
 * (a + b, a - b) and multiplies once by fp32(1/sqrt(block)), the order the
 * cache rotation uses, so the values are bitwise those of the formats'
 * rotation.  The transform is its own inverse up to rounding.
 */
hkv_status hkv_hadamard(const void* x, int32_t in_dtype, float* y, int64_t rows, int32_t n,
                        int32_t block, const uint32_t* sign_bits, int32_t inverse,
                        void* stream);

/* Message for the last non-OK status returned on this thread (host). */
const char* hkv_last_error(void);

/* Library version string (host). */
const char* hkv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HKV_H */
