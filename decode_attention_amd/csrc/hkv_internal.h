// hkv_internal.h -- host-side declarations shared by the libhkv sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hkv.h"
#include "hkv_device.h"

namespace hkv {

DevFmt to_dev(const hkv_format& f);

// Kernel launchers; the arguments have been validated by the C ABI layer.
hipError_t launch_quantize_append(const DevFmt& f, const void* key, const void* value,
                                  bool in_f16, int64_t num_tokens, int num_kv_heads,
                                  const int64_t* slot_mapping, uint8_t* cache, hipStream_t s);

hipError_t launch_hadamard(const void* x, bool in_f16, float* y, int64_t rows, int n, int block,
                           const uint32_t* sign_bits, bool inverse, hipStream_t s);

hipError_t launch_dequantize(const DevFmt& f, const uint8_t* cache, int num_kv_heads,
                             const int64_t* slot_ids, int64_t num_tokens, bool rotated,
                             float* k_out, float* v_out, hipStream_t s);

struct DecodePlan {
  int group;            // query heads per KV head
  int n_q;              // queries per sequence group
  int rows;             // group * n_q rows sharing one KV head
  int rows_pad;         // rows of a partial record block (the kernel's row count)
  int num_groups;       // num_queries / n_q
  int nsub;             // query groups per request (queries_per_seq / n_q)
  int64_t num_wgs;      // workgroups of the decode kernel
  int tokens_per_split;
  int num_splits;
  size_t partial_floats;  // floats per (row, split) partial record
  size_t workspace_bytes;
  int kernel;           // which decode kernel runs
};

// Returns false (and leaves *p untouched) when the sizes are not supported.
bool plan_decode(const DevFmt& f, int num_queries, int num_q_heads, int num_kv_heads,
                 int max_klen, int queries_per_seq, DecodePlan* p);

hipError_t launch_decode(const DevFmt& f, const DecodePlan& p, const void* query, bool q_f16,
                         int num_q_heads, int num_kv_heads, const uint8_t* cache,
                         const int32_t* block_table, int max_pages_per_req,
                         const int32_t* q_to_req, const int32_t* q_to_klen, float sm_scale,
                         float* out, void* workspace, bool deterministic, hipStream_t s);

// Device address of the static decode scratch (HKV_DECODE_SCRATCH_BYTES) on
// the current device, looked up once per device.
hipError_t decode_scratch(void** ptr);

}  // namespace hkv
