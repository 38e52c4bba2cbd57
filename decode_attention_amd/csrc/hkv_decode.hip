// hkv_decode.hip -- split-K paged decode attention over the rotated,
// quantized cache, and the split merge that rotates the output back.
//
// What is computed (vLLM API docs "vllm.v1.attention.ops.rocm_octave",
// reference_attention and module text; Strata pull request #21, "How" item 2
// and the merge note): for query token i and query head h,
//   out[i,h] = R_V^-1 sum_t softmax_t(scale * <R_K q[i,h], k'_t>) v'_t
// over the first q_to_klen[i] tokens of sequence q_to_req[i], where k'_t, v'_t
// are the cached codes dequantized in the rotated space and R_K, R_V the
// sign-flip + Walsh-Hadamard rotations of K and V.  Scores use the rotated
// query (the rotation is orthogonal, so <R q, R k> = <q, k>), values are
// dequantized in registers inside an online-softmax accumulation, and the
// output is rotated back once per query head.
//
// Generic kernel: grid (split, KV head, query group); 4 waves per workgroup.
// A query group is n_q consecutive query tokens of one sequence; its
// G * n_q query rows (G = query heads per KV head) share every K/V load.
// Each wave streams 64-token tiles: the tile's slots are copied into LDS
// with coalesced loads; scores are computed lane-per-token (the rotated,
// pre-scaled query rows sit in LDS and are read as broadcasts); the online
// softmax state is per row; P.V is computed lane-per-dimension.
#include "hkv_decode_common.h"

#include <algorithm>
#include <cstdint>
#include <mutex>

namespace hkv {
namespace {

__device__ __forceinline__ uint32_t lds_word(const uint32_t* p, int byte_off) {
  return p[byte_off >> 2];
}

// Code values (exact small integers) of K dims [d0, d0+32) of a slot held in
// LDS as words, and the fp32 factor that turns them into rotated-space values.
__device__ __forceinline__ void k_chunk(const DevFmt& f, const uint32_t* s, int d0,
                                        float (&cv)[32], float& sc) {
  const uint8_t* sb = (const uint8_t*)s;
  if (f.kind == HKV_KIND_Q8_0) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t word = lds_word(s, d0 + 4 * w);
#pragma unroll
      for (int j = 0; j < 4; ++j) cv[4 * w + j] = (float)(int8_t)(uint8_t)(word >> (8 * j));
    }
    sc = h2f(rd16(sb + f.off_scales + 2 * (d0 >> 5)));
    return;
  }
  if (f.kind == HKV_KIND_Q4_0) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t word = lds_word(s, d0 / 2 + 4 * w);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        cv[8 * w + j] = (float)((int)((word >> (8 * (j & 3) + 4 * (j >> 2))) & 15u) - 8);
    }
    sc = h2f(rd16(sb + f.off_scales + 2 * (d0 >> 5)));
    return;
  }
  const bool three = f.compact || d0 >= f.k_wide;
  const int si = f.compact ? 0 : (d0 >> 6);
  sc = h2f(rd16(sb + f.off_scales + 2 * si)) / (float)kLutOne;
  if (!three) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t word = lds_word(s, d0 / 2 + 4 * w);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        cv[8 * w + j] = (float)lut_value((int)((word >> (8 * (j & 3) + 4 * (j >> 2))) & 15u), 4);
    }
    return;
  }
  const int seg = f.compact ? 0 : f.off_k_nope;
  const int n = f.compact ? f.D : f.D - f.k_wide;
  const int i0 = f.compact ? d0 : d0 - f.k_wide;
  const uint32_t lo0 = lds_word(s, seg + i0 / 4), lo1 = lds_word(s, seg + i0 / 4 + 4);
  const uint32_t hi = lds_word(s, seg + n / 4 + i0 / 8);
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t lo = (j < 16) ? lo0 : lo1;
    const int c = (int)((lo >> (8 * (j & 3) + 2 * ((j >> 2) & 3))) & 3u) |
                  (int)(((hi >> (8 * (j & 3) + (j >> 2))) & 1u) << 2);
    cv[j] = (float)lut_value(c, 3);
  }
}

// Rotated-space value of V dim d of a slot held in LDS.
__device__ __forceinline__ float v_lds(const DevFmt& f, const uint32_t* s, int d) {
  return v_value(f, (const uint8_t*)s, d);
}

template <int E, int R>
__global__ __launch_bounds__(256) void decode_generic_kernel(DevFmt f, DecArgs a) {
  constexpr int D = E * kWave;
  extern __shared__ __align__(16) uint32_t smem[];
  const int slot_words = f.slot_bytes / 4;
  const int tstride = slot_words | 1;  // odd word stride: conflict-free lane-per-token reads
  float* qs = (float*)smem;                               // [R][D]
  float* pb = qs + R * D;                                 // [waves][R][kTile]
  float* ml = pb + kWaves * R * kTile;                    // [waves][R][2]
  uint32_t* tiles = (uint32_t*)(ml + kWaves * R * 2);     // [waves][kTile][tstride]

  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  int split, kvh, gi;
  if (!wg_item(a, split, kvh, gi)) return;
  const int q0 = gi * a.n_q;
  const int req = a.q_to_req[q0];
  int kmax = 0;
  for (int j = 0; j < a.n_q; ++j) kmax = max(kmax, a.q_to_klen[q0 + j]);
  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(t_begin + a.tokens_per_split, kmax);
  float* part = a.ws + (((size_t)gi * a.num_kv_heads + kvh) * a.num_splits + split) * R * a.pstride;

  if (t_begin >= t_end) {  // nothing to attend to in this split
    for (int r = threadIdx.x; r < a.rows; r += blockDim.x) {
      part[r * a.pstride + 0] = -INFINITY;
      part[r * a.pstride + 1] = 0.0f;
    }
    return;
  }

  // Query rows: rotate like K (signs, then the K-block transform), fold in
  // the softmax scale and log2(e); rows beyond a.rows are zero.
  for (int r = wave; r < R; r += kWaves) {
    float x[E];
    if (r < a.rows) {
      const int j = r / a.group, g = r % a.group;
      const int64_t qrow = (int64_t)(q0 + j) * a.num_q_heads + kvh * a.group + g;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int d = kWave * e + lane;
        x[e] = a.q_f16 ? h2f(((const uint16_t*)a.query)[qrow * D + d])
                       : ((const float*)a.query)[qrow * D + d];
        if (f.use_signs) x[e] = apply_sign(f, x[e], d);
      }
      fwht_strided<E>(x, f.k_block, f.k_norm);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) qs[r * D + kWave * e + lane] = x[e] * a.q_scale;
  }
  __syncthreads();

  int klen_row[R];
#pragma unroll
  for (int r = 0; r < R; ++r) klen_row[r] = (r < a.rows) ? a.q_to_klen[q0 + r / a.group] : 0;

  float m[R], l[R], o[R][E];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[r][e] = 0.0f;
  }

  uint32_t* tile = tiles + wave * kTile * tstride;
  float* pw = pb + wave * R * kTile;
  const int32_t* bt = a.block_table + (int64_t)req * a.max_pages;

  for (int t0 = t_begin + wave * kTile; t0 < t_end; t0 += kWaves * kTile) {
    const int nvalid = min(kTile, t_end - t0);
    // Stage the tile's slots in LDS: one slot per step, its words spread over
    // the lanes (a coalesced run of slot_bytes); the page lookup is uniform.
#pragma unroll 8
    for (int tt = 0; tt < nvalid; ++tt) {
      const int t = t0 + tt;
      const uint32_t* src = (const uint32_t*)slot_ptr(f, a.cache, bt[t / f.page_size],
                                                      t % f.page_size, a.num_kv_heads, kvh);
      for (int w = lane; w < slot_words; w += kWave) tile[tt * tstride + w] = src[w];
    }
    wave_sync_lds();

    // Scores, lane per token.
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = 0.0f;
    const uint32_t* my = tile + min(lane, nvalid - 1) * tstride;
    for (int d0 = 0; d0 < D; d0 += 32) {
      float cv[32], sc;
      k_chunk(f, my, d0, cv, sc);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float4* qv = (const float4*)(qs + r * D + d0);
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float4 q4 = qv[j];
          acc = fmaf(q4.x, cv[4 * j + 0], acc);
          acc = fmaf(q4.y, cv[4 * j + 1], acc);
          acc = fmaf(q4.z, cv[4 * j + 2], acc);
          acc = fmaf(q4.w, cv[4 * j + 3], acc);
        }
        s[r] = fmaf(acc, sc, s[r]);
      }
    }
    // Online softmax update (exp2 domain), per row.
    const int t = t0 + lane;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sr = (lane < nvalid && t < klen_row[r]) ? s[r] : -INFINITY;
      const float mt = wave_max(sr);
      const float mn = fmaxf(m[r], mt);
      const float alpha = (mn == -INFINITY) ? 1.0f : exp2f(m[r] - mn);
      const float p = (sr == -INFINITY) ? 0.0f : exp2f(sr - mn);
      l[r] = fmaf(l[r], alpha, p);
      m[r] = mn;
#pragma unroll
      for (int e = 0; e < E; ++e) o[r][e] *= alpha;
      pw[r * kTile + lane] = p;
    }
    wave_sync_lds();

    // P.V, lane per dimension (dims E*lane .. E*lane+E-1).
    for (int tt = 0; tt < nvalid; ++tt) {
      const uint32_t* sl = tile + tt * tstride;
      float vv[E];
#pragma unroll
      for (int e = 0; e < E; ++e) vv[e] = v_lds(f, sl, E * lane + e);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float p = pw[r * kTile + tt];
#pragma unroll
        for (int e = 0; e < E; ++e) o[r][e] = fmaf(p, vv[e], o[r][e]);
      }
    }
    wave_sync_lds();
  }

  // Merge the waves of the workgroup.  l holds per-lane partial sums.
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float lr = wave_tree_sum(l[r]);
    if (lane == 0) {
      ml[(wave * R + r) * 2 + 0] = m[r];
      ml[(wave * R + r) * 2 + 1] = lr;
    }
  }
  __syncthreads();
  float* ob = qs;  // reuse the query area: [R][D]
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml[(w * R + r) * 2]);
    const float fw = (m[r] == -INFINITY) ? 0.0f : exp2f(m[r] - M);
#pragma unroll
    for (int e = 0; e < E; ++e) o[r][e] *= fw;
  }
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float* dst = &ob[r * D + E * lane + e];
          *dst = (w == 0) ? o[r][e] : (*dst + o[r][e]);
        }
    }
    __syncthreads();
  }
  for (int r = wave; r < a.rows; r += kWaves) {
    float M = -INFINITY, L = 0.0f;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml[(w * R + r) * 2]);
    for (int w = 0; w < kWaves; ++w) {
      const float mw = ml[(w * R + r) * 2];
      if (mw != -INFINITY) L += ml[(w * R + r) * 2 + 1] * exp2f(mw - M);
    }
    float* pr = part + r * a.pstride;
    if (lane == 0) {
      pr[0] = M;
      pr[1] = L;
    }
    for (int d = lane; d < D; d += kWave) pr[4 + d] = ob[r * D + d];
  }
}

// Merge the split partials of one (query, head) row, normalise, rotate the
// output back (transform with the V block, then the signs) and store fp32.
// One workgroup per row; wave w takes splits w, w + kMergeWaves, ... in
// chunks of kMergeChunk, loading the (m, l) pair and o of every split of a
// chunk together (one memory round trip per chunk), and keeps a running
// (M, L, acc) in the exp2 domain; the waves then combine through LDS.  Only
// the splits that start below the row's own klen are counted: each of those
// holds at least one of the row's tokens, so its whole record was written and
// is finite.  The first chunk is requested before the klen is known (the
// records of any split of the launch are in bounds) and the others only for
// counted splits.
constexpr int kMergeWaves = 8;
constexpr int kMergeChunk = 4;

// Row (query i, head h) of merge workgroup `id`.  The split kernel puts all
// splits of one (request group, KV head) item on one XCD when the items per
// split are a multiple of 8 (see wg_item): XCD (rg Hkv + kvh) mod 8.  The
// merge ids are dealt the same way, id = 8 (rows_per_item (p / 8) + rr) +
// p mod 8 for row rr of item p, so a row is merged on the XCD whose L2 holds
// its partial records.  False for the ids past the last row.
__device__ __forceinline__ bool merge_row(const DecArgs& a, uint32_t id, int& i, int& h) {
  const uint32_t per_item = (uint32_t)(a.nsub * a.n_q * a.group);
  const uint32_t k = id >> 3;
  const uint32_t rr = k % per_item;
  const uint32_t p = 8u * (k / per_item) + (id & 7u);
  const uint32_t items = (uint32_t)(a.num_groups / a.nsub) * (uint32_t)a.num_kv_heads;
  if (p >= items) return false;
  const uint32_t rg = p / (uint32_t)a.num_kv_heads, kvh = p % (uint32_t)a.num_kv_heads;
  const uint32_t qg = (uint32_t)(a.n_q * a.group);
  const uint32_t sub = rr / qg, jg = rr % qg;
  const uint32_t gi = rg * (uint32_t)a.nsub + sub;
  i = (int)(gi * (uint32_t)a.n_q + jg / (uint32_t)a.group);
  h = (int)(kvh * (uint32_t)a.group + jg % (uint32_t)a.group);
  return true;
}

inline int64_t merge_wgs(int num_groups, int nsub, int num_kv_heads, int n_q, int group) {
  const int64_t items = (int64_t)(num_groups / nsub) * num_kv_heads;
  return 8 * (int64_t)nsub * n_q * group * ((items + 7) / 8);
}

// The first chunk of a row's records is requested together with the row's
// key length (one memory round trip), and folded once the length is known.
template <int E>
__global__ __launch_bounds__(kMergeWaves * kWave) void merge_kernel(DevFmt f, DecArgs a,
                                                                   float* out) {
  constexpr int D = E * kWave;
  __shared__ float red[kMergeWaves][D + 2];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  int v_block = f.v_block, use_signs = f.use_signs;
  float v_norm = f.v_norm;
  pin_args(a, v_block, use_signs, v_norm);
  out = pin_global(out);
  int i, h;
  if (!merge_row(a, blockIdx.x, i, h)) return;
  const int gi = i / a.n_q, j = i % a.n_q;
  const int kvh = h / a.group, g = h % a.group;
  const int r = j * a.group + g;
  const int Rp = a.rows_pad;
  const float* base = a.ws + (((size_t)gi * a.num_kv_heads + kvh) * a.num_splits) * Rp * a.pstride +
                      (size_t)r * a.pstride;
  const size_t sstride = (size_t)Rp * a.pstride;
  const int klen = a.q_to_klen[i];
  uint32_t sw[E];
  lane_sign_words<E>(f, use_signs, lane, sw);  // with the other loads
  float M = -INFINITY, L = 0.0f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  // wave w takes splits w, w + kMergeWaves, ... in chunks of kMergeChunk
  constexpr int kStep = kMergeWaves * kMergeChunk;
  MergeChunk<E, kMergeChunk> k;
  merge_load(k, base, sstride, wave, kMergeWaves, a.num_splits, lane);
  const int n_live = merge_live(a, klen);
  merge_fold(k, wave, kMergeWaves, n_live, M, L, acc);
  for (int s0 = wave + kStep; s0 < n_live; s0 += kStep) {
    merge_load(k, base, sstride, s0, kMergeWaves, n_live, lane);
    merge_fold(k, s0, kMergeWaves, n_live, M, L, acc);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[wave][kWave * e + lane] = acc[e];
  if (lane == 0) {
    red[wave][D] = M;
    red[wave][D + 1] = L;
  }
  __syncthreads();
  if (wave != 0) return;
  float Mt = -INFINITY;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) Mt = fmaxf(Mt, red[w][D]);
  float fw[kMergeWaves];
  L = 0.0f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    const float mw = red[w][D];
    fw[w] = mw == -INFINITY ? 0.0f : exp2f(mw - Mt);
    L = fmaf(red[w][D + 1], fw[w], L);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int d = kWave * e + lane;
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) t = fmaf(red[w][d], fw[w], t);
    acc[e] = t;
  }
  const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] *= inv;
  fwht_strided<E>(acc, v_block, v_norm);
  float* dst = out + ((int64_t)i * a.num_q_heads + h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e)
    dst[kWave * e + lane] = flip_sign(acc[e], sw[e], lane);
}

// The same merge with one wave per row (kMergeWaves rows per workgroup), for
// plans with at most kRowChunk splits: a row's records come in one memory
// round trip, together with its key length, and need no cross-wave combine,
// so many-row, few-split shapes (tens of thousands of short rows) do not pay
// a workgroup and a barrier per row.
constexpr int kRowChunk = 8;

template <int E>
__global__ __launch_bounds__(kMergeWaves * kWave) void merge_rows_kernel(DevFmt f, DecArgs a,
                                                                        float* out, int64_t rows) {
  constexpr int D = E * kWave;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  int v_block = f.v_block, use_signs = f.use_signs;
  float v_norm = f.v_norm;
  pin_args(a, v_block, use_signs, v_norm);
  out = pin_global(out);
  const int64_t rowid = (int64_t)blockIdx.x * kMergeWaves + wave;
  if (rowid >= rows) return;
  const int i = (int)(rowid / a.num_q_heads);
  const int h = (int)(rowid % a.num_q_heads);
  const int gi = i / a.n_q, j = i % a.n_q;
  const int kvh = h / a.group, g = h % a.group;
  const int r = j * a.group + g;
  const int Rp = a.rows_pad;
  const float* base = a.ws + (((size_t)gi * a.num_kv_heads + kvh) * a.num_splits) * Rp * a.pstride +
                      (size_t)r * a.pstride;
  const size_t sstride = (size_t)Rp * a.pstride;
  const int klen = a.q_to_klen[i];
  uint32_t sw[E];
  lane_sign_words<E>(f, use_signs, lane, sw);  // with the other loads
  float M = -INFINITY, L = 0.0f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  MergeChunk<E, kRowChunk> k;
  merge_load(k, base, sstride, 0, 1, a.num_splits, lane);
  const int n_live = merge_live(a, klen);
  merge_fold(k, 0, 1, n_live, M, L, acc);
  for (int s0 = kRowChunk; s0 < n_live; s0 += kRowChunk) {
    merge_load(k, base, sstride, s0, 1, n_live, lane);
    merge_fold(k, s0, 1, n_live, M, L, acc);
  }
  const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] *= inv;
  fwht_strided<E>(acc, v_block, v_norm);
  float* dst = out + ((int64_t)i * a.num_q_heads + h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e)
    dst[kWave * e + lane] = flip_sign(acc[e], sw[e], lane);
}

int round_rows(int rows) {
  int R = 1;
  while (R < rows) R <<= 1;
  return R;
}

size_t generic_lds_bytes(const DevFmt& f, int R) {
  const int tstride = (f.slot_bytes / 4) | 1;
  return sizeof(float) * ((size_t)R * f.D + (size_t)kWaves * R * kTile + (size_t)kWaves * R * 2) +
         sizeof(uint32_t) * (size_t)kWaves * kTile * tstride;
}

template <int E, int R>
hipError_t launch_generic_er(const DevFmt& f, const DecArgs& a, dim3 grid, hipStream_t s) {
  const size_t lds = generic_lds_bytes(f, R);
  // The dynamic-LDS limit of this kernel instance is raised once per process
  // (thread-safe); the largest size any format needs is set, since the
  // attribute is per kernel, not per launch.
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute((const void*)decode_generic_kernel<E, R>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr_err != hipSuccess) return attr_err;
  decode_generic_kernel<E, R><<<grid, dim3(kWaves * kWave), lds, s>>>(f, a);
  return hipGetLastError();
}

template <int E>
hipError_t launch_generic_e(const DevFmt& f, const DecArgs& a, int R, dim3 grid, hipStream_t s) {
  switch (R) {
    case 1: return launch_generic_er<E, 1>(f, a, grid, s);
    case 2: return launch_generic_er<E, 2>(f, a, grid, s);
    case 4: return launch_generic_er<E, 4>(f, a, grid, s);
    case 8: return launch_generic_er<E, 8>(f, a, grid, s);
    case 16: return launch_generic_er<E, 16>(f, a, grid, s);
    case 32: return launch_generic_er<E, 32>(f, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool q4_mfma_supported(const DevFmt& f, int rows);
hipError_t launch_decode_q4_mfma(const DevFmt& f, const DecArgs& a, dim3 grid, hipStream_t s);
bool q4w_mfma_supported(const DevFmt& f, int rows);
hipError_t launch_decode_q4w(const DevFmt& f, const DecArgs& a, dim3 grid, hipStream_t s);
bool q8_mfma_supported(const DevFmt& f, int rows);
hipError_t launch_decode_q8_mfma(const DevFmt& f, const DecArgs& a, dim3 grid, hipStream_t s);
int oct_mfma_rows(const DevFmt& f, int rows);
hipError_t launch_decode_oct(const DevFmt& f, const DecArgs& a, dim3 grid, hipStream_t s);

// Decode kernels: 0 the generic VALU kernel (every format), 1 the Q4_0 MFMA
// kernel (head size 256, 8 rows), 2 the Octave MFMA kernels (8, 16 or 32
// rows), 3 the Q8_0 MFMA kernel (head size 256, 8 rows), 4 the Q4_0 window
// kernel (head size 256, 9 to 32 rows in one pass).
constexpr int kKernelGeneric = 0, kKernelQ4 = 1, kKernelOctK3v4 = 2, kKernelQ8 = 3,
              kKernelQ4W = 4;

constexpr int64_t kTargetSplitsWgs = 512;
constexpr int kMaxRows = 32;          // query rows per KV head in one pass
constexpr int kMaxQueriesPerSeq = 16;

bool plan_decode(const DevFmt& f, int num_queries, int num_q_heads, int num_kv_heads,
                 int max_klen, int queries_per_seq, DecodePlan* p) {
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads) return false;
  if (queries_per_seq < 1 || queries_per_seq > kMaxQueriesPerSeq ||
      num_queries % queries_per_seq)
    return false;
  DecodePlan q;
  q.group = num_q_heads / num_kv_heads;
  q.n_q = queries_per_seq;
  q.rows = q.group * q.n_q;
  q.num_groups = num_queries / queries_per_seq;
  q.nsub = 1;
  auto mfma_kernel = [&](int rows) {
    return q4_mfma_supported(f, rows)    ? kKernelQ4
           : q4w_mfma_supported(f, rows) ? kKernelQ4W
           : q8_mfma_supported(f, rows)  ? kKernelQ8
           : oct_mfma_rows(f, rows) > 0 ? kKernelOctK3v4
                                        : kKernelGeneric;
  };
  q.kernel = mfma_kernel(q.rows);
  // More rows than one kernel pass takes (the matrix-core kernels: 8, 16 or
  // 32 query rows per KV head; the generic kernel: 32): the queries of a
  // sequence are split into the largest sub-groups that fit, preferring a
  // matrix-core kernel; each sub-group streams the sequence's K/V through its
  // own workgroups.
  if ((q.kernel == kKernelGeneric || q.rows > kMaxRows) && q.n_q > 1) {
    // (the generic kernel stages a tile of slots per wave in LDS, so large
    // slots bound its rows too)
    int best = 0;
    for (int nq = q.n_q - 1; nq >= 1 && !best; --nq)
      if (q.n_q % nq == 0 && mfma_kernel(q.group * nq) != kKernelGeneric) best = nq;
    for (int nq = q.n_q; nq >= 1 && !best; --nq)
      if (q.n_q % nq == 0 && q.group * nq <= kMaxRows &&
          generic_lds_bytes(f, round_rows(q.group * nq)) <= 160 * 1024)
        best = nq;
    if (best) {
      q.nsub = q.n_q / best;
      q.num_groups = num_queries / best;
      q.n_q = best;
      q.rows = q.group * best;
      q.kernel = mfma_kernel(q.rows);
    }
  }
  if (q.rows > kMaxRows) return false;
  q.rows_pad = q.kernel == kKernelQ4 || q.kernel == kKernelQ8 ? 8
               : q.kernel == kKernelQ4W                       ? 32
               : q.kernel == kKernelOctK3v4                   ? oct_mfma_rows(f, q.rows)
                                                              : round_rows(q.rows);
  // Split size: enough splits that (sequence group, KV head, split) fills the
  // chip with one resident round of workgroups (the MFMA kernel: one
  // 8-wave workgroup per CU; the generic kernel: two 4-wave ones), in whole
  // 64-token steps, capped where the per-split fixed cost (query set-up,
  // partial record) is well amortised.  An MFMA split takes at least 256
  // tokens, one 32-token unit per wave: shorter splits leave waves idle and
  // add workgroups and partial records for nothing (an 8K context: 64-token
  // splits 19.7 us per call, 256-token splits 16.7 us).
  {
    const int64_t units = (int64_t)q.num_groups * num_kv_heads;
    const bool mfma = q.kernel != kKernelGeneric;
    const int cap = mfma ? 4096 : 1024;
    const int64_t target = mfma ? kTargetSplitsWgs / 2 : kTargetSplitsWgs;
    int64_t tps = units > 0 ? ((int64_t)max(max_klen, 1) * units + target - 1) / target : cap;
    tps = (tps + 63) / 64 * 64;
    q.tokens_per_split = (int)std::min<int64_t>(cap, std::max<int64_t>(mfma ? 256 : 64, tps));
  }
  q.num_splits = max_klen > 0 ? (max_klen + q.tokens_per_split - 1) / q.tokens_per_split : 1;
  // Grid sizes in work-items are 32-bit (512-lane workgroups at most).
  const int64_t wgs = decode_wgs(q.num_groups, q.nsub, num_kv_heads, q.num_splits);
  const int64_t merge_rows = std::max<int64_t>(
      (int64_t)q.num_groups * q.n_q * num_q_heads,
      merge_wgs(q.num_groups, q.nsub, num_kv_heads, q.n_q, q.group));
  if (wgs * 512 > (int64_t)UINT32_MAX || merge_rows * kMergeWaves * kWave > (int64_t)UINT32_MAX)
    return false;
  q.num_wgs = wgs;
  q.partial_floats = kPartialHead + (size_t)f.D;
  const int R = q.rows_pad;
  q.workspace_bytes = sizeof(float) * q.partial_floats * R * (size_t)q.num_splits *
                      (size_t)q.num_groups * (size_t)num_kv_heads;
  if (q.kernel == kKernelGeneric && generic_lds_bytes(f, R) > 160 * 1024) return false;
  *p = q;
  return true;
}

hipError_t launch_decode(const DevFmt& f, const DecodePlan& p, const void* query, bool q_f16,
                         int num_q_heads, int num_kv_heads, const uint8_t* cache,
                         const int32_t* block_table, int max_pages_per_req,
                         const int32_t* q_to_req, const int32_t* q_to_klen, float sm_scale,
                         float* out, void* workspace, bool deterministic, hipStream_t s) {
  if (p.num_groups == 0) return hipSuccess;
  DecArgs a;
  a.query = query;
  a.q_f16 = q_f16 ? 1 : 0;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = p.group;
  a.n_q = p.n_q;
  a.rows = p.rows;
  a.rows_pad = p.rows_pad;
  a.num_queries = p.num_groups * p.n_q;
  a.num_groups = p.num_groups;
  a.nsub = p.nsub;
  a.cache = cache;
  a.block_table = block_table;
  a.max_pages = max_pages_per_req;
  a.q_to_req = q_to_req;
  a.q_to_klen = q_to_klen;
  a.q_scale = sm_scale * kLog2e;
  a.tokens_per_split = p.tokens_per_split;
  a.num_splits = p.num_splits;
  a.ws = (float*)workspace;
  a.pstride = (int)p.partial_floats;
  a.det = deterministic ? 1 : 0;
  const int R = round_rows(p.rows);
  const dim3 grid((unsigned)p.num_wgs);
  hipError_t e;
  if (p.kernel == kKernelQ4) {
    e = launch_decode_q4_mfma(f, a, grid, s);
  } else if (p.kernel == kKernelQ4W) {
    e = launch_decode_q4w(f, a, grid, s);
  } else if (p.kernel == kKernelQ8) {
    e = launch_decode_q8_mfma(f, a, grid, s);
  } else if (p.kernel == kKernelOctK3v4) {
    e = launch_decode_oct(f, a, grid, s);
  } else switch (f.D / kWave) {
    case 1: e = launch_generic_e<1>(f, a, R, grid, s); break;
    case 2: e = launch_generic_e<2>(f, a, R, grid, s); break;
    case 3: e = launch_generic_e<3>(f, a, R, grid, s); break;
    case 4: e = launch_generic_e<4>(f, a, R, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.num_groups * p.n_q * num_q_heads;
  const dim3 mblock(kMergeWaves * kWave);
  if (p.num_splits <= kRowChunk) {
    const dim3 mgrid((unsigned)((rows + kMergeWaves - 1) / kMergeWaves));
    switch (f.D / kWave) {
      case 1: merge_rows_kernel<1><<<mgrid, mblock, 0, s>>>(f, a, out, rows); break;
      case 2: merge_rows_kernel<2><<<mgrid, mblock, 0, s>>>(f, a, out, rows); break;
      case 3: merge_rows_kernel<3><<<mgrid, mblock, 0, s>>>(f, a, out, rows); break;
      case 4: merge_rows_kernel<4><<<mgrid, mblock, 0, s>>>(f, a, out, rows); break;
    }
  } else {
    const dim3 mgrid((unsigned)merge_wgs(p.num_groups, p.nsub, num_kv_heads, p.n_q, p.group));
    switch (f.D / kWave) {
      case 1: merge_kernel<1><<<mgrid, mblock, 0, s>>>(f, a, out); break;
      case 2: merge_kernel<2><<<mgrid, mblock, 0, s>>>(f, a, out); break;
      case 3: merge_kernel<3><<<mgrid, mblock, 0, s>>>(f, a, out); break;
      case 4: merge_kernel<4><<<mgrid, mblock, 0, s>>>(f, a, out); break;
    }
  }
  return hipGetLastError();
}

// Scratch of hkv_decode_attention_noalloc: the split partial records of one
// call, in place of a caller's workspace.  Every device the library runs on
// holds its own copy until the process ends.  In host code the name stands
// for a host-side handle, not a device address: host code uses only the
// address decode_scratch() obtains from the runtime.
__device__ __align__(256) uint8_t scratch[HKV_DECODE_SCRATCH_BYTES];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace hkv
