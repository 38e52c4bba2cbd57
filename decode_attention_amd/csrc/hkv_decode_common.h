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
  int num_groups;   // query groups of n_q queries (num_queries / n_q)
  int nsub;         // groups per request when its queries are split into sub-groups, else 1
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
  int det;        // 1: each wave takes its units in a fixed order (no queue),
                  // so the summation order, and the result, never vary
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

// Lane l <- lane (l ^ 8) within each row of 16 (DPP row_ror:8).
__device__ __forceinline__ float ror8(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false));
}

// The 8-row matrix-core kernels hold the two parts of a score row in lanes n
// and n + 8 of each row of 16 and join them in both lanes, with the parts in
// opposite roles, so the two joins can differ in the last bit.  Lane n + 8
// then takes lane n's score: the lanes derive the leading fp16 part and the
// residual of one p, which must come from bitwise the same score.
__device__ __forceinline__ float pair_score(float own_join, int n) {
  const float from_n = ror8(own_join);
  return n < 8 ? own_join : from_n;
}

// Maximum over the lanes l, l ^ 16, l ^ 32, l ^ 48 with the lane-swap
// instructions (no LDS round trip): swapping a copy of v with itself leaves
// the partner's value in one of the two results.
__device__ __forceinline__ float max_xor16_32(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ uint4 lds_u4(const uint32_t* p) {
  return *(const uint4*)__builtin_assume_aligned(p, 16);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// The (split, KV head, query group) of this workgroup; false for the few ids
// past the last one.  Workgroup ids are dealt round-robin to the chip's 8
// XCDs (id mod 8), so the id order decides which XCD streams what:
//  * item w enumerates (request group, KV head) within a split, splits
//    slowest, so every XCD takes every split of an even share of the
//    requests (with the split index fastest, as in a (split, head, group)
//    grid, an XCD would take one split of every request: with ragged
//    lengths the XCD of split 0 does the most work and the late splits'
//    XCDs sit idle);
//  * id = 8 (nsub (w / 8) + s) + w % 8 gives the nsub sub-groups s of one
//    request's queries, which read the same K/V, one XCD and consecutive
//    dispatches there, so the second read of a tile can hit that XCD's L2.
__device__ __forceinline__ bool wg_item(const DecArgs& a, int& split, int& kvh, int& gi) {
  const uint32_t id = blockIdx.x;
  const uint32_t hi = id >> 3;
  const uint32_t nsub = (uint32_t)a.nsub;
  const uint32_t s = hi % nsub;
  const uint32_t w = 8u * (hi / nsub) + (id & 7u);
  const uint32_t per_split = (uint32_t)(a.num_groups / a.nsub) * (uint32_t)a.num_kv_heads;
  const uint32_t sp = w / per_split;
  if (sp >= (uint32_t)a.num_splits) return false;
  const uint32_t r = w - sp * per_split;
  const uint32_t rg = r / (uint32_t)a.num_kv_heads;
  split = (int)sp;
  kvh = (int)(r - rg * (uint32_t)a.num_kv_heads);
  gi = (int)(rg * nsub + s);
  return true;
}

// Every word of the decode arguments fetched at this point, in one round
// trip.  Left alone, the compiler loads each argument near its first use,
// which in a kernel prologue puts several dependent kernel-argument fetches
// ahead of the first cache load.  (The request map and the key lengths stay
// plain argument pointers, so that their uniform reads remain scalar loads,
// whose wait does not hold back the vector loads issued after them.)
// Three words of the format (x0, x1, y) join the same fetch: one statement,
// so that none of them is sunk to its first use, which can be late.
__device__ __forceinline__ void pin_args(DecArgs& a, int& x0, int& x1, float& y) {
  asm("" : "+s"(a.q_f16), "+s"(a.num_q_heads), "+s"(a.num_kv_heads), "+s"(a.group),
      "+s"(a.n_q), "+s"(a.rows), "+s"(a.rows_pad), "+s"(a.num_queries), "+s"(a.num_groups),
      "+s"(a.nsub), "+s"(a.max_pages), "+s"(a.tokens_per_split), "+s"(a.num_splits),
      "+s"(a.pstride), "+s"(a.det), "+s"(x0), "+s"(x1), "+s"(y));
  a.query = pin_global(a.query);
  a.cache = pin_global(a.cache);
  a.block_table = pin_global(a.block_table);
  a.ws = pin_global(a.ws);
}

// Raw bits of the values kWave e + lane (e < E) of query row r of the group
// at q0 for KV head kvh, as one batch of loads with no wait between them
// (rows past the group read row 0; query_value zeroes them).
template <int E>
__device__ __forceinline__ void query_row_raw(const DecArgs& a, int q0, int kvh, int r, int lane,
                                              uint32_t (&qw)[E]) {
  constexpr int D = E * kWave;
  const int rq = r < a.rows ? r : 0;
  const int64_t qrow = (int64_t)(q0 + rq / a.group) * a.num_q_heads + kvh * a.group + rq % a.group;
  if (a.q_f16) {
    const uint16_t* qp = (const uint16_t*)a.query + qrow * D + lane;
#pragma unroll
    for (int e = 0; e < E; ++e) qw[e] = qp[kWave * e];
  } else {
    const uint32_t* qp = (const uint32_t*)a.query + qrow * D + lane;
#pragma unroll
    for (int e = 0; e < E; ++e) qw[e] = qp[kWave * e];
  }
}

__device__ __forceinline__ float query_value(const DecArgs& a, uint32_t w, bool live) {
  const float v = a.q_f16 ? h2f((uint16_t)w) : __uint_as_float(w);
  return live ? v : 0.0f;
}

// Sign words of the dims kWave e + lane (e < E) of this lane (word
// 2 e + lane / 32, bit lane % 32), zero without a sign pattern.
template <int E>
__device__ __forceinline__ void lane_sign_words(const DevFmt& f, bool use_signs, int lane,
                                                uint32_t (&sw)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) sw[e] = use_signs ? f.sign_bits[2 * e + (lane >> 5)] : 0u;
}

__device__ __forceinline__ float flip_sign(float x, uint32_t w, int lane) {
  return __uint_as_float(__float_as_uint(x) ^ (((w >> (lane & 31)) & 1u) << 31));
}

// Key lengths of the group's queries, one per lane: lane l holds that of
// query q0 + min(l, n_q - 1) (n_q <= kWave), from one vector load.
__device__ __forceinline__ int group_klen_lane(const DecArgs& a, int q0, int lane) {
  return a.q_to_klen[q0 + min(lane, a.n_q - 1)];
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, kWave));
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, kWave));
  return __builtin_amdgcn_readfirstlane(v);
}

// Three int8 planes of a query code: qi = 2^16 hi + 2^8 mid + lo with hi in
// [-127, 127] and mid, lo in [-128, 127], for |qi| <= kQ3MaxI.  Against int8
// keys the three integer products give the score to about 23 bits of the
// row's largest query value, whatever that value's magnitude.
constexpr int kQ3MaxI = 127 * 65536 + 127 * 256 + 127;
__device__ __forceinline__ void q_split3(int qi, int& hi, int& mid, int& lo) {
  hi = (qi + 32896) >> 16;       // qi - 2^16 hi in [-32896, 32639]
  const int rem = qi - hi * 65536;
  mid = (rem + 128) >> 8;
  lo = rem - mid * 256;
}

// Workgroups of a decode launch (see wg_item).
inline int64_t decode_wgs(int num_groups, int nsub, int num_kv_heads, int num_splits) {
  const int64_t items = (int64_t)(num_groups / nsub) * num_kv_heads * num_splits;
  return 8 * (int64_t)nsub * ((items + 7) / 8);
}

// Partial record of one (query row, split): m, l, two pad words, o[D].
constexpr int kPartialHead = 4;

// The (m, l) pairs and o of C records, splits s0 + st c.
template <int E, int C>
struct MergeChunk {
  float2 ml[C];
  float o[C][E];
};

// Requests the records of one chunk; splits at or past `lim` (at most
// num_splits) load split 0's record instead, which is never counted for them.
template <int E, int C>
__device__ __forceinline__ void merge_load(MergeChunk<E, C>& k, const float* base, size_t sstride,
                                           int s0, int st, int lim, int lane) {
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int s = s0 + st * c;
    const float* ps = base + (s < lim ? s : 0) * sstride;
    k.ml[c] = *(const float2*)ps;
#pragma unroll
    for (int e = 0; e < E; ++e) k.o[c][e] = ps[kPartialHead + kWave * e + lane];
  }
}

// Folds a chunk into the running (M, L, acc) in the exp2 domain.  Records
// at or past `n_live` (or with m = -inf) are skipped by select, never
// multiplied, so whatever such a record holds cannot reach the sums.
template <int E, int C>
__device__ __forceinline__ void merge_fold(const MergeChunk<E, C>& k, int s0, int st, int n_live,
                                           float& M, float& L, float (&acc)[E]) {
  bool live[C];
  float Mc = M;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    live[c] = s0 + st * c < n_live && k.ml[c].x != -INFINITY;
    if (live[c]) Mc = fmaxf(Mc, k.ml[c].x);
  }
  // no live record yet: M = Mc = -inf and acc, L are still 0
  const float alpha = Mc == -INFINITY ? 1.0f : exp2f(M - Mc);
  L *= alpha;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] *= alpha;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const float w = live[c] ? exp2f(k.ml[c].x - Mc) : 0.0f;
    L = live[c] ? fmaf(k.ml[c].y, w, L) : L;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = live[c] ? fmaf(k.o[c][e], w, acc[e]) : acc[e];
  }
  M = Mc;
}

// Splits holding tokens of a row of key length klen: each of them holds at
// least one, so its whole record was written and is finite.
__device__ __forceinline__ int merge_live(const DecArgs& a, int klen) {
  return klen <= 0 ? 0 : min(a.num_splits, (klen + a.tokens_per_split - 1) / a.tokens_per_split);
}


}  // namespace hkv
