// hkv_api.hip -- the C ABI of libhkv: argument checks, format setup and
// kernel enqueue.  See include/hkv.h for the contract of every entry point.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "hkv_internal.h"

namespace {

thread_local char g_err[512] = "";

hkv_status fail(hkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

hkv_status hip_fail(hipError_t e, const char* what) {
  return fail(HKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

// Fixed sign pattern of length n: SplitMix64 (Steele, Lea & Flood, OOPSLA
// 2014) started from state n; output word k gives signs 64k .. 64k+63, a set
// bit meaning -1.
void make_sign_bits(int n, uint32_t* words) {
  uint64_t state = (uint64_t)n;
  for (int k = 0; k < (n + 63) / 64; ++k) {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    words[2 * k] = (uint32_t)(z & 0xffffffffu);
    if (2 * k + 1 < HKV_MAX_HEAD / 32) words[2 * k + 1] = (uint32_t)(z >> 32);
  }
}

// Re-derive every dependent field and compare, so a corrupted or hand-made
// descriptor is refused before anything is enqueued.
hkv_status check_format(const hkv_format* f) {
  if (!f) return fail(HKV_ERR_INVALID_ARG, "format is NULL");
  static const char* names[] = {"q4_0", "octave_k3v4", "octave_k3v3", "octave_k3v3_compact",
                                "q8_0"};
  const char* name = nullptr;
  if (f->kind == HKV_KIND_Q4_0) {
    name = names[0];
  } else if (f->kind == HKV_KIND_Q8_0) {
    name = names[4];
  } else if (f->kind == HKV_KIND_OCTAVE) {
    name = f->compact ? names[3] : (f->v_bits == 4 ? names[1] : names[2]);
  } else {
    return fail(HKV_ERR_INVALID_ARG, "format: unknown kind %d", f->kind);
  }
  hkv_format g;
  const hkv_status st = hkv_format_init(&g, name, f->head_size, f->rope_dim, f->page_size);
  if (st != HKV_OK) return st;
  if (std::memcmp(&g, f, sizeof(g)) != 0)
    return fail(HKV_ERR_INVALID_ARG, "format descriptor is inconsistent; use hkv_format_init");
  return HKV_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

namespace hkv {

DevFmt to_dev(const hkv_format& f) {
  DevFmt d;
  std::memset(&d, 0, sizeof(d));
  d.kind = f.kind;
  d.D = f.head_size;
  d.rope = f.rope_dim;
  d.v_bits = f.v_bits;
  d.compact = f.compact;
  d.page_size = f.page_size;
  d.k_block = f.k_block;
  d.v_block = f.v_block;
  d.k_wide = f.k_wide_dim;
  d.off_k_nope = f.off_k_nope;
  d.off_v = f.off_v;
  d.off_scales = f.off_scales;
  d.num_k_scales = f.num_k_scales;
  d.num_scales = f.num_scales;
  d.slot_bytes = f.slot_bytes;
  d.use_signs = f.kind == HKV_KIND_OCTAVE;
  // The transform's 1/sqrt(block) is applied as one fp32 multiply by the
  // fp32-rounded constant.
  d.k_norm = (float)(1.0 / std::sqrt((double)f.k_block));
  d.v_norm = (float)(1.0 / std::sqrt((double)f.v_block));
  std::memcpy(d.sign_bits, f.sign_bits, sizeof(d.sign_bits));
  return d;
}

}  // namespace hkv

extern "C" {

const char* hkv_last_error(void) { return g_err; }

const char* hkv_version(void) { return "hkv 0.1 (gfx950)"; }

hkv_status hkv_format_init(hkv_format* f, const char* cache_dtype, int32_t head_size,
                           int32_t rope_dim, int32_t page_size) {
  if (!f || !cache_dtype) return fail(HKV_ERR_INVALID_ARG, "format_init: NULL argument");
  if (page_size < 1 || page_size > 1024)
    return fail(HKV_ERR_INVALID_ARG, "page_size must be in [1, 1024], got %d", page_size);
  hkv_format g;
  std::memset(&g, 0, sizeof(g));
  const int d = head_size;
  g.head_size = d;
  g.page_size = page_size;
  if (std::strcmp(cache_dtype, "q4_0") == 0) {
    // Q4_0 + FWHT over the head (Strata PR #21): blocks of 32 with an fp16
    // scale, no sign flips.
    if (d != 64 && d != 128 && d != 256)
      return fail(HKV_ERR_INVALID_ARG, "q4_0 needs head_size 64, 128 or 256, got %d", d);
    g.kind = HKV_KIND_Q4_0;
    g.rope_dim = 0;
    g.v_bits = 4;
    g.k_block = d;
    g.v_block = d;
    g.k_wide_dim = d;
    g.off_k_nope = d / 2;
    g.off_v = d / 2;
    g.off_scales = d;
    g.num_k_scales = d / 32;
    g.num_scales = d / 16;
    g.slot_bytes = d + d / 8;
    g.kernel_code = 0;
    *f = g;
    return HKV_OK;
  }
  if (std::strcmp(cache_dtype, "q8_0") == 0) {
    // The int8 mode [Q4] compares against, after the same rotation (FWHT
    // over the head, no signs): 32 int8 codes and one fp16 scale per block.
    if (d != 64 && d != 128 && d != 256)
      return fail(HKV_ERR_INVALID_ARG, "q8_0 needs head_size 64, 128 or 256, got %d", d);
    g.kind = HKV_KIND_Q8_0;
    g.rope_dim = 0;
    g.v_bits = 8;
    g.k_block = d;
    g.v_block = d;
    g.k_wide_dim = 0;
    g.off_k_nope = d;
    g.off_v = d;
    g.off_scales = 2 * d;
    g.num_k_scales = d / 32;
    g.num_scales = d / 16;
    g.slot_bytes = 2 * d + d / 8;
    g.kernel_code = 8;
    *f = g;
    return HKV_OK;
  }
  int v_bits, compact;
  if (std::strcmp(cache_dtype, "octave_k3v4") == 0) {
    v_bits = 4, compact = 0;
  } else if (std::strcmp(cache_dtype, "octave_k3v3") == 0) {
    v_bits = 3, compact = 0;
  } else if (std::strcmp(cache_dtype, "octave_k3v3_compact") == 0) {
    v_bits = 3, compact = 1;
  } else {
    return fail(HKV_ERR_INVALID_ARG, "unknown cache dtype '%s'", cache_dtype);
  }
  // OctaveFormat validation (vLLM rocm_octave docs).
  constexpr int kBlock = 64;
  if (compact && !is_pow2(d))
    return fail(HKV_ERR_INVALID_ARG, "compact Octave K needs a power-of-two head_size, got %d", d);
  if (d <= 0 || rope_dim < 0 || rope_dim % kBlock || d % kBlock)
    return fail(HKV_ERR_INVALID_ARG,
                "Octave needs head_size and rope_dim in multiples of 64; got head_size=%d, rope_dim=%d",
                d, rope_dim);
  if (rope_dim > d)
    return fail(HKV_ERR_INVALID_ARG, "rope_dim %d exceeds head_size %d", rope_dim, d);
  if (d > HKV_MAX_HEAD)
    return fail(HKV_ERR_UNSUPPORTED, "head_size %d exceeds %d", d, HKV_MAX_HEAD);
  g.kind = HKV_KIND_OCTAVE;
  g.rope_dim = rope_dim;
  g.v_bits = v_bits;
  g.compact = compact;
  g.k_block = compact ? d : kBlock;
  g.v_block = is_pow2(d) ? d : kBlock;
  g.k_wide_dim = compact ? 0 : rope_dim;
  g.off_k_nope = g.k_wide_dim * 4 / 8;
  g.off_v = g.off_k_nope + (d - g.k_wide_dim) * 3 / 8;
  g.off_scales = g.off_v + d * v_bits / 8;
  g.num_k_scales = compact ? 1 : d / kBlock;
  g.num_scales = g.num_k_scales + 1;
  const int raw = g.off_scales + 2 * g.num_scales;
  const int al = compact ? 4 : 8;
  g.slot_bytes = (raw + al - 1) / al * al;
  g.kernel_code = v_bits + (compact ? 16 : 0);
  make_sign_bits(d, g.sign_bits);
  *f = g;
  return HKV_OK;
}

hkv_status hkv_quantize_append(const hkv_format* f, const void* key, const void* value,
                               int32_t in_dtype, int64_t num_tokens, int32_t num_kv_heads,
                               const int64_t* slot_mapping, uint8_t* cache, void* stream) {
  hkv_status st = check_format(f);
  if (st != HKV_OK) return st;
  if (num_tokens < 0 || num_kv_heads <= 0)
    return fail(HKV_ERR_INVALID_ARG, "quantize_append: num_tokens=%lld num_kv_heads=%d",
                (long long)num_tokens, num_kv_heads);
  if (in_dtype != HKV_F32 && in_dtype != HKV_F16)
    return fail(HKV_ERR_INVALID_ARG, "quantize_append: bad input dtype %d", (int)in_dtype);
  if (num_tokens == 0) return HKV_OK;
  if (!key || !value || !slot_mapping || !cache)
    return fail(HKV_ERR_INVALID_ARG, "quantize_append: NULL pointer");
  if (!aligned(cache, 16)) return fail(HKV_ERR_INVALID_ARG, "cache must be 16-byte aligned");
  if (num_tokens * num_kv_heads > 0x7fffffffLL)
    return fail(HKV_ERR_UNSUPPORTED, "quantize_append: too many rows");
  const hipError_t e = hkv::launch_quantize_append(hkv::to_dev(*f), key, value, in_dtype == HKV_F16,
                                                   num_tokens, num_kv_heads, slot_mapping, cache,
                                                   (hipStream_t)stream);
  return e == hipSuccess ? HKV_OK : hip_fail(e, "quantize_append launch");
}

hkv_status hkv_dequantize(const hkv_format* f, const uint8_t* cache, int32_t num_kv_heads,
                          const int64_t* slot_ids, int64_t num_tokens, int32_t rotated,
                          float* k_out, float* v_out, void* stream) {
  hkv_status st = check_format(f);
  if (st != HKV_OK) return st;
  if (num_tokens < 0 || num_kv_heads <= 0)
    return fail(HKV_ERR_INVALID_ARG, "dequantize: num_tokens=%lld num_kv_heads=%d",
                (long long)num_tokens, num_kv_heads);
  if (num_tokens == 0) return HKV_OK;
  if (!cache || !slot_ids || !k_out || !v_out)
    return fail(HKV_ERR_INVALID_ARG, "dequantize: NULL pointer");
  if (!aligned(cache, 16)) return fail(HKV_ERR_INVALID_ARG, "cache must be 16-byte aligned");
  if (num_tokens * num_kv_heads > 0x7fffffffLL)
    return fail(HKV_ERR_UNSUPPORTED, "dequantize: too many rows");
  const hipError_t e = hkv::launch_dequantize(hkv::to_dev(*f), cache, num_kv_heads, slot_ids,
                                              num_tokens, rotated != 0, k_out, v_out,
                                              (hipStream_t)stream);
  return e == hipSuccess ? HKV_OK : hip_fail(e, "dequantize launch");
}

hkv_status hkv_hadamard(const void* x, int32_t in_dtype, float* y, int64_t rows, int32_t n,
                        int32_t block, const uint32_t* sign_bits, int32_t inverse,
                        void* stream) {
  if (in_dtype != HKV_F32 && in_dtype != HKV_F16)
    return fail(HKV_ERR_INVALID_ARG, "hadamard: bad input dtype %d", (int)in_dtype);
  if (block != 64 && block != 128 && block != 256)
    return fail(HKV_ERR_INVALID_ARG, "hadamard: block must be 64, 128 or 256, got %d", block);
  if (rows < 0 || n <= 0 || n % block)
    return fail(HKV_ERR_INVALID_ARG, "hadamard: rows=%lld n=%d (n a positive multiple of %d)",
                (long long)rows, n, block);
  if (rows == 0) return HKV_OK;
  if (!x || !y) return fail(HKV_ERR_INVALID_ARG, "hadamard: NULL pointer");
  if (!aligned(x, in_dtype == HKV_F16 ? 8 : 16) || !aligned(y, 16))
    return fail(HKV_ERR_INVALID_ARG, "hadamard: x must be %d-byte and y 16-byte aligned",
                in_dtype == HKV_F16 ? 8 : 16);
  if (sign_bits && !aligned(sign_bits, 4))
    return fail(HKV_ERR_INVALID_ARG, "hadamard: sign_bits must be 4-byte aligned");
  const size_t esz = in_dtype == HKV_F16 ? 2 : 4;
  const uintptr_t xb = (uintptr_t)x, xe = xb + (size_t)rows * n * esz;
  const uintptr_t yb = (uintptr_t)y, ye = yb + (size_t)rows * n * 4;
  const bool same = xb == yb && in_dtype == HKV_F32;
  if (!same && xb < ye && yb < xe)
    return fail(HKV_ERR_INVALID_ARG, "hadamard: x and y overlap (only y == x with f32 input)");
  if (rows * (int64_t)(n / block) > ((int64_t)1 << 40))
    return fail(HKV_ERR_UNSUPPORTED, "hadamard: too many blocks");
  const hipError_t e = hkv::launch_hadamard(x, in_dtype == HKV_F16, y, rows, n, block, sign_bits,
                                            inverse != 0, (hipStream_t)stream);
  return e == hipSuccess ? HKV_OK : hip_fail(e, "hadamard launch");
}

size_t hkv_decode_workspace_bytes(const hkv_format* f, int32_t num_queries, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t max_klen,
                                  int32_t queries_per_seq) {
  if (check_format(f) != HKV_OK || num_queries < 0) return 0;
  hkv::DecodePlan p;
  if (!hkv::plan_decode(hkv::to_dev(*f), num_queries, num_q_heads, num_kv_heads, max_klen,
                        queries_per_seq, &p))
    return 0;
  return p.workspace_bytes;
}

}  // extern "C"

namespace {

// Checks shared by both decode entry points; on success *d and *p hold the
// device format and the launch plan.  *done is set when there is nothing to
// launch (no queries).
hkv_status decode_check(const char* who, const hkv_format* f, const void* query, int32_t q_dtype,
                        int32_t num_queries, int32_t num_q_heads, int32_t num_kv_heads,
                        const uint8_t* cache, const int32_t* block_table,
                        int32_t max_pages_per_req, const int32_t* q_to_req,
                        const int32_t* q_to_klen, int32_t max_klen, int32_t queries_per_seq,
                        float sm_scale, uint32_t flags, const float* out, hkv::DevFmt* d,
                        hkv::DecodePlan* p, bool* done) {
  *done = false;
  hkv_status st = check_format(f);
  if (st != HKV_OK) return st;
  if (num_queries < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(HKV_ERR_INVALID_ARG,
                "%s: need num_q_heads a positive multiple of num_kv_heads (%d, %d), "
                "num_queries >= 0 (%d)", who, num_q_heads, num_kv_heads, num_queries);
  if (queries_per_seq < 1 || queries_per_seq > 16 || num_queries % queries_per_seq)
    return fail(HKV_ERR_INVALID_ARG,
                "%s: queries_per_seq must be in [1, 16] and divide num_queries (%d, %d)", who,
                queries_per_seq, num_queries);
  if (q_dtype != HKV_F32 && q_dtype != HKV_F16)
    return fail(HKV_ERR_INVALID_ARG, "%s: bad query dtype %d", who, (int)q_dtype);
  if (max_klen < 0) return fail(HKV_ERR_INVALID_ARG, "%s: max_klen < 0", who);
  if (!std::isfinite(sm_scale)) return fail(HKV_ERR_INVALID_ARG, "%s: sm_scale not finite", who);
  if (flags & ~HKV_DECODE_DETERMINISTIC)
    return fail(HKV_ERR_INVALID_ARG, "%s: unknown flags 0x%x", who, flags);
  if (num_queries == 0) {
    *done = true;
    return HKV_OK;
  }
  if (!query || !cache || !block_table || !q_to_req || !q_to_klen || !out)
    return fail(HKV_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (max_pages_per_req <= 0) return fail(HKV_ERR_INVALID_ARG, "%s: max_pages_per_req <= 0", who);
  if (!aligned(cache, 16)) return fail(HKV_ERR_INVALID_ARG, "cache must be 16-byte aligned");
  *d = hkv::to_dev(*f);
  if (!hkv::plan_decode(*d, num_queries, num_q_heads, num_kv_heads, max_klen, queries_per_seq, p))
    return fail(HKV_ERR_UNSUPPORTED,
                "%s: unsupported shape (query rows per KV head = %d x %d must be <= 32)", who,
                num_q_heads / num_kv_heads, queries_per_seq);
  return HKV_OK;
}

}  // namespace

extern "C" {

hkv_status hkv_decode_attention(const hkv_format* f, const void* query, int32_t q_dtype,
                                int32_t num_queries, int32_t num_q_heads, int32_t num_kv_heads,
                                const uint8_t* cache, const int32_t* block_table,
                                int32_t max_pages_per_req, const int32_t* q_to_req,
                                const int32_t* q_to_klen, int32_t max_klen,
                                int32_t queries_per_seq, float sm_scale, uint32_t flags,
                                float* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  hkv::DevFmt d;
  hkv::DecodePlan p;
  bool done;
  const hkv_status st =
      decode_check("decode", f, query, q_dtype, num_queries, num_q_heads, num_kv_heads, cache,
                   block_table, max_pages_per_req, q_to_req, q_to_klen, max_klen,
                   queries_per_seq, sm_scale, flags, out, &d, &p, &done);
  if (st != HKV_OK || done) return st;
  if (workspace_bytes < p.workspace_bytes || (p.workspace_bytes && !workspace))
    return fail(HKV_ERR_WORKSPACE, "decode: workspace of %zu bytes needed, %zu given",
                p.workspace_bytes, workspace_bytes);
  if (workspace && !aligned(workspace, 16))
    return fail(HKV_ERR_INVALID_ARG, "decode: workspace must be 16-byte aligned");
  const hipError_t e = hkv::launch_decode(d, p, query, q_dtype == HKV_F16, num_q_heads,
                                          num_kv_heads, cache, block_table, max_pages_per_req,
                                          q_to_req, q_to_klen, sm_scale, out, workspace,
                                          (flags & HKV_DECODE_DETERMINISTIC) != 0,
                                          (hipStream_t)stream);
  return e == hipSuccess ? HKV_OK : hip_fail(e, "decode launch");
}

hkv_status hkv_decode_attention_noalloc(const hkv_format* f, const void* query, int32_t q_dtype,
                                        int32_t num_queries, int32_t num_q_heads,
                                        int32_t num_kv_heads, const uint8_t* cache,
                                        const int32_t* block_table, int32_t max_pages_per_req,
                                        const int32_t* q_to_req, const int32_t* q_to_klen,
                                        int32_t max_klen, int32_t queries_per_seq,
                                        float sm_scale, uint32_t flags, float* out,
                                        void* stream) {
  hkv::DevFmt d;
  hkv::DecodePlan p;
  bool done;
  const hkv_status st =
      decode_check("decode_noalloc", f, query, q_dtype, num_queries, num_q_heads, num_kv_heads,
                   cache, block_table, max_pages_per_req, q_to_req, q_to_klen, max_klen,
                   queries_per_seq, sm_scale, flags, out, &d, &p, &done);
  if (st != HKV_OK || done) return st;
  if (p.workspace_bytes > HKV_DECODE_SCRATCH_BYTES)
    return fail(HKV_ERR_WORKSPACE,
                "decode_noalloc: these sizes need %zu bytes of scratch, the library's static "
                "scratch holds %zu; call hkv_decode_attention with a workspace instead",
                p.workspace_bytes, (size_t)HKV_DECODE_SCRATCH_BYTES);
  void* scratch = nullptr;
  hipError_t e = hkv::decode_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "decode_noalloc: scratch address");
  e = hkv::launch_decode(d, p, query, q_dtype == HKV_F16, num_q_heads, num_kv_heads, cache,
                         block_table, max_pages_per_req, q_to_req, q_to_klen, sm_scale, out,
                         scratch, (flags & HKV_DECODE_DETERMINISTIC) != 0, (hipStream_t)stream);
  return e == hipSuccess ? HKV_OK : hip_fail(e, "decode_noalloc launch");
}

}  // extern "C"
