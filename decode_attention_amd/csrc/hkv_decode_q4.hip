// hkv_decode_q4.hip -- split-K paged decode attention over the Q4_0 cache on
// the matrix cores (gfx950), for head size 256 and up to 8 query rows per KV
// head (GQA group x query tokens).
//
// What is computed is the decode of Strata pull request #21 ("How" item 2:
// Q4_0 codes dequantized in registers during a flash-attention style score
// accumulation; the merge note: the query is rotated and the output rotated
// back) in the paged form of the vLLM docs "vllm.v1.attention.ops.
// rocm_octave" (reference_attention).
//
// One wave streams 16-token tiles of one sequence and one KV head.
//  * Scores, S^T = K Q^T on v_mfma_i32_16x16x32_i8: A = the 4-bit codes of
//    16 tokens x one 32-value Q4_0 block (exact small integers), B = the
//    rotated query as two int8 planes (q ~ s_h (256 hi + lo): 16 columns =
//    8 rows x {hi, lo}); the "- 8" of the codes rides in the accumulator
//    input; each block's int32 result is scaled by that token's fp16 block
//    scale in fp32.  The int8 planes keep ~15 significant bits of q.
//  * The score tile comes out with each lane holding 4 consecutive tokens of
//    one row -- exactly the A layout of v_mfma_f32_16x16x16_f16, so P.V needs
//    no transpose of P: A = p * v_scale (fp16), B = the V codes of the same
//    4 tokens for 16 dims, regrouped with v_perm_b32 from a transposed LDS
//    tile and turned into exact fp16 (c - 8) with the 0x6400 bias trick.
//  * K codes go straight to registers with 16-byte loads and a 4x4
//    lane-group transpose (v_permlane32_swap / v_permlane16_swap).
//  * Online softmax in the exp2 domain, rescaling only when a row maximum
//    grows; the four waves of a workgroup merge their partials in LDS and
//    write one partial record per row to the workspace; the shared merge
//    kernel combines the splits and rotates the output back.
#include "hkv_decode_common.h"

namespace hkv {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int2_t __attribute__((ext_vector_type(2)));

constexpr int kD = 256;        // head size handled here
constexpr int kNB = kD / 32;   // Q4_0 blocks per head vector
constexpr int kRows = 8;       // query rows per KV head
constexpr int kT = 16;         // tokens per tile
constexpr int kSlot = kD + kD / 8;  // Q4_0 slot bytes at head size 256
constexpr int kQMaxI = 32639;  // largest |q| code of the two-plane int8 split
constexpr float kQMax = 32639.0f;
constexpr int kVStride = kT + 4;  // padded token stride of the transposed V tile
constexpr float kLazy = 8.0f;     // log2 headroom before the running max is raised


// 4x4 transpose across the four 16-lane groups: register w of group g
// receives register g of group w.
__device__ __forceinline__ void lanegroup_transpose(uint32_t& r0, uint32_t& r1, uint32_t& r2,
                                                    uint32_t& r3) {
  auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = c[0];
  r1 = c[1];
  r2 = d[0];
  r3 = d[1];
}

__device__ __forceinline__ float ror8(float v) {  // lane l <- lane (l ^ 8) within 16
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false));
}

__device__ __forceinline__ float f16lo(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16hi(uint32_t w) { return h2f((uint16_t)(w >> 16)); }
// fp16 scale of block b from a 16-byte chunk of 8 fp16 values.
__device__ __forceinline__ float scale_of(const uint4& c, int b) {
  const uint32_t w = (b >> 1) == 0 ? c.x : (b >> 1) == 1 ? c.y : (b >> 1) == 2 ? c.z : c.w;
  return (b & 1) ? f16hi(w) : f16lo(w);
}

struct Tile {
  uint4 k0, k1, v0, v1, sc;
};

__device__ __forceinline__ void load_tile(Tile& x, const uint8_t* slot, int gq, bool scale_lane,
                                          int scale_kind) {
  x.k0 = *(const uint4*)(slot + 16 * gq);
  x.k1 = *(const uint4*)(slot + 16 * (4 + gq));
  x.v0 = *(const uint4*)(slot + kD / 2 + 16 * gq);
  x.v1 = *(const uint4*)(slot + kD / 2 + 16 * (4 + gq));
  if (scale_lane) x.sc = *(const uint4*)(slot + kD + 16 * scale_kind);
}

__global__ __launch_bounds__(256, 2) void decode_q4_mfma_kernel(DevFmt f, DecArgs a) {
  __shared__ __align__(16) int8_t qB[kNB][16][32];      // B operand bytes: [block][column][dim]
  __shared__ float qsc[kRows];                           // per-row score scale
  __shared__ __align__(16) uint32_t vt[kWaves][kNB][4][kVStride];  // V words, token-minor
  __shared__ __align__(16) uint4 scl[kWaves][2][kT];          // K / V scale chunks
  __shared__ float mlw[kWaves][kRows][2];
  __shared__ __align__(16) float ob[kRows][kD];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int split = blockIdx.x, kvh = blockIdx.y, gi = blockIdx.z;
  const int q0 = gi * a.n_q;
  const int req = a.q_to_req[q0];
  int kmax = 0;
  for (int j = 0; j < a.n_q; ++j) kmax = max(kmax, a.q_to_klen[q0 + j]);
  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(t_begin + a.tokens_per_split, kmax);
  float* part = a.ws + ((size_t)(gi * a.num_kv_heads + kvh) * a.num_splits + split) * kRows *
                           a.pstride;
  if (t_begin >= t_end) {
    for (int r = threadIdx.x; r < a.rows; r += blockDim.x) {
      part[r * a.pstride + 0] = -INFINITY;
      part[r * a.pstride + 1] = 0.0f;
    }
    return;
  }

  // ---- query rows -> rotated, scaled int8 planes (B operand) --------------
  for (int r = wave; r < kRows; r += kWaves) {
    float x[4];
    if (r < a.rows) {
      const int j = r / a.group, g = r % a.group;
      const int64_t qrow = (int64_t)(q0 + j) * a.num_q_heads + kvh * a.group + g;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = kWave * e + lane;
        x[e] = a.q_f16 ? h2f(((const uint16_t*)a.query)[qrow * kD + d])
                       : ((const float*)a.query)[qrow * kD + d];
        if (f.use_signs) x[e] = apply_sign(f, x[e], d);
      }
      fwht_strided<4>(x, f.k_block, f.k_norm);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = 0.0f;
    }
    float qmax = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) qmax = fmaxf(qmax, fabsf(x[e]));
    qmax = wave_max(qmax);
    // |q| <= 32639 keeps both planes in int8: hi = (q + 128) >> 8 in
    // [-127, 127], lo = q - 256 hi in [-128, 127].
    const float inv = qmax > 0.0f ? kQMax / qmax : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int qi = (int)rintf(x[e] * inv);
      qi = min(kQMaxI, max(-kQMaxI, qi));
      const int hi = (qi + 128) >> 8;
      const int lo = qi - hi * 256;
      const int d = kWave * e + lane;
      qB[d >> 5][r][d & 31] = (int8_t)hi;
      qB[d >> 5][8 + r][d & 31] = (int8_t)lo;
    }
    if (lane == 0) qsc[r] = (qmax / kQMax) * a.q_scale * 0.0625f;
  }
  __syncthreads();

  const int n = lane & 15;   // score column (row r = n & 7, plane = n >> 3)
  const int g = lane >> 4;   // lane group: tokens 4g..4g+3 of a tile in the score layout
  const int row = n & 7;
  const float qs = qsc[row];
  const int klen_row = row < a.rows ? a.q_to_klen[q0 + row / a.group] : 0;
  const bool live_row = row < a.rows;  // lanes n and n + 8 carry the same row
  const uint32_t vsel = (uint32_t)(n & 3) | (0x0Cu << 8) | ((uint32_t)(4 + (n & 3)) << 16) |
                        (0x0Cu << 24);
  // Nibble masks kept in VGPRs so that mask-and-bias fuses into v_and_or_b32.
  uint32_t m0f, mf0;
  asm volatile("v_mov_b32 %0, 0x0f0f0f0f" : "=v"(m0f));
  asm volatile("v_mov_b32 %0, 0xf0f0f0f0" : "=v"(mf0));
  int kmin = kmax;
  for (int j = 0; j < a.n_q; ++j) kmin = min(kmin, a.q_to_klen[q0 + j]);
  const int t_lim = min(t_end, kmin);  // tiles ending at or before this need no mask

  float4_t o[kNB][2];
#pragma unroll
  for (int b = 0; b < kNB; ++b) o[b][0] = o[b][1] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  // Tiles of this wave: t0 = t_begin + 16 * (wave + 4 k); a tile lies in one
  // page.  The page ids of 64 tiles at a time are fetched one per lane and
  // broadcast from there, so no tile waits on a page-table load.
  const int32_t* bt = a.block_table + (int64_t)req * a.max_pages;
  const int ps = f.page_size;                 // a power of two, multiple of kT
  const int ps_shift = 31 - __builtin_clz(ps);
  const int nt = (t_end - t_begin + kT - 1) / kT;              // tiles in the split
  const int my_tiles = nt > wave ? (nt - wave + kWaves - 1) / kWaves : 0;
  const int tl = lane & 15, gq = lane >> 4;
  const bool scale_lane = lane < 32;
  const int scale_kind = (lane >> 4) & 1;
  int pid = 0;
  auto load_pids = [&](int k0) {
    const int k = k0 + lane;
    if (k < my_tiles) pid = bt[(t_begin + kT * (wave + kWaves * k)) >> ps_shift];
  };
  // Tile k starts at token t0 of page `pid` (uniform): its slots are one
  // contiguous run of kT * slot_bytes; lane (tl, gq) reads token tl of it.
  auto tile_slot = [&](int k) -> const uint8_t* {
    const int t0 = t_begin + kT * (wave + kWaves * k);
    const int page = __builtin_amdgcn_readfirstlane(__shfl(pid, k & 63, kWave));
    const uint8_t* base = a.cache + ((((int64_t)page * a.num_kv_heads + kvh) << ps_shift) +
                                     (t0 & (ps - 1))) * (int64_t)kSlot;
    const int tlc = min(tl, t_end - 1 - t0);
    return base + tlc * kSlot;
  };
  load_pids(0);

  auto fetch = [&](Tile& x, int k) {
    if (k < my_tiles) {
      if (k > 0 && (k & 63) == 0) load_pids(k);
      load_tile(x, tile_slot(k), gq, scale_lane, scale_kind);
    }
  };
  auto process = [&](const Tile& cur, int k) {
    const int t0 = t_begin + kT * (wave + kWaves * k);
    // K words: word gq of block w (k0) and of block 4+w (k1).
    uint32_t kw[8] = {cur.k0.x, cur.k0.y, cur.k0.z, cur.k0.w, cur.k1.x, cur.k1.y, cur.k1.z, cur.k1.w};
    lanegroup_transpose(kw[0], kw[1], kw[2], kw[3]);
    lanegroup_transpose(kw[4], kw[5], kw[6], kw[7]);
    // V words and scales to LDS.
    uint32_t* vw = &vt[wave][0][0][tl];
    vw[((gq) * 4 + 0) * kVStride] = cur.v0.x;
    vw[((gq) * 4 + 1) * kVStride] = cur.v0.y;
    vw[((gq) * 4 + 2) * kVStride] = cur.v0.z;
    vw[((gq) * 4 + 3) * kVStride] = cur.v0.w;
    vw[((4 + gq) * 4 + 0) * kVStride] = cur.v1.x;
    vw[((4 + gq) * 4 + 1) * kVStride] = cur.v1.y;
    vw[((4 + gq) * 4 + 2) * kVStride] = cur.v1.z;
    vw[((4 + gq) * 4 + 3) * kVStride] = cur.v1.w;
    if (scale_lane) scl[wave][scale_kind][tl] = cur.sc;
    wave_sync_lds();
    uint4 ks[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ks[i] = scl[wave][0][4 * g + i];

    // Scores: per block an int32 tile (16 (code - 8) x int8 planes) scaled
    // by the token's block scale into fp32; the 1/16 is in the row scale.
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int4_t zero4 = {0, 0, 0, 0};
    int4_t C;
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      // Flipping bit 3 of a code turns it into the 4-bit two's complement of
      // (code - 8); placed in the high nibble of a byte it reads as the int8
      // 16 * (code - 8).  Low nibbles are dims 0..3, high nibbles dims 4..7.
      const uint32_t x = kw[b] ^ 0x88888888u;
      const int2_t A2 = {(int)((x << 4) & mf0), (int)(x & mf0)};
      C = __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, A2),
                                                 *(const long*)&qB[b][n][8 * g], zero4, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf((float)C[i], scale_of(ks[i], b), acc[i]);
    }
    float s[4];
    const bool full = t0 + kT <= t_lim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pt = ror8(acc[i]);
      const float hiv = n < 8 ? acc[i] : pt, lov = n < 8 ? pt : acc[i];
      s[i] = fmaf(hiv, 256.0f, lov) * qs;
    }
    if (!full) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 4 * g + i;
        s[i] = (tok < t_end && tok < klen_row) ? s[i] : -INFINITY;
      }
    }
    // Online softmax in the exp2 domain.  The running maximum is raised only
    // when a tile exceeds it by more than kLazy, so p <= 2^kLazy and the
    // rescale of the accumulators is rare.
    float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
      l_run *= alpha;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, (4 * g + i) & 7, kWave);
#pragma unroll
      for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[b][0][i] *= al[i];
          o[b][1][i] *= al[i];
        }
      m_run = m_new;
    }
    float p[4];
    const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;  // rows with nothing valid yet
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2f(s[i] - m_ref);  // exp2(-inf) = 0
      l_run += p[i];
      p[i] = live_row ? p[i] : 0.0f;
    }

    // P.V.  A rows 0-7 carry p rounded to fp16, rows 8-15 the residual
    // p - p_hi (scaled by 2^12 to stay in the normal fp16 range); B carries
    // (code - 8) * v_scale split exactly into an fp16 high part and the fp16
    // residual (a 4-bit integer times an 11-bit mantissa has <= 15 bits), so
    // P.V keeps ~22 bits of p and the exact dequantized values.
    half4_t A;
    {
      const half4_t h = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
      const half4_t r = {(_Float16)((p[0] - (float)h[0]) * 4096.0f),
                         (_Float16)((p[1] - (float)h[1]) * 4096.0f),
                         (_Float16)((p[2] - (float)h[2]) * 4096.0f),
                         (_Float16)((p[3] - (float)h[3]) * 4096.0f)};
      A = n < 8 ? h : r;
    }
    uint4 vs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vs[i] = scl[wave][1][4 * g + i];
    const half4_t c1032x4 = {(_Float16)-1032.0f, (_Float16)-1032.0f, (_Float16)-1032.0f, (_Float16)-1032.0f};
    const half4_t c16x4 = {(_Float16)0.0625f, (_Float16)0.0625f, (_Float16)0.0625f, (_Float16)0.0625f};
    const half4_t c72x4 = {(_Float16)-72.0f, (_Float16)-72.0f, (_Float16)-72.0f, (_Float16)-72.0f};
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const uint4 W = *(const uint4*)&vt[wave][b][n >> 2][4 * g];
      // Byte (n & 3) of the V word of tokens t0..t3 -> halves (t0, t1), (t2, t3).
      const uint32_t x01 = __builtin_amdgcn_perm(W.y, W.x, vsel);
      const uint32_t x23 = __builtin_amdgcn_perm(W.w, W.z, vsel);
      const uint2 lw = {(x01 & m0f) | 0x64006400u, (x23 & m0f) | 0x64006400u};
      const uint2 hw = {(x01 & mf0) | 0x64006400u, (x23 & mf0) | 0x64006400u};
      const half4_t lo = __builtin_bit_cast(half4_t, lw) + c1032x4;
      const half4_t hi = __builtin_elementwise_fma(__builtin_bit_cast(half4_t, hw), c16x4, c72x4);
      // v_scale of block b for tokens t0..t3.
      constexpr uint32_t kSel[2] = {0x05040100u, 0x07060302u};
      const uint32_t w0 = (b >> 1) == 0 ? vs[0].x : (b >> 1) == 1 ? vs[0].y : (b >> 1) == 2 ? vs[0].z : vs[0].w;
      const uint32_t w1 = (b >> 1) == 0 ? vs[1].x : (b >> 1) == 1 ? vs[1].y : (b >> 1) == 2 ? vs[1].z : vs[1].w;
      const uint32_t w2 = (b >> 1) == 0 ? vs[2].x : (b >> 1) == 1 ? vs[2].y : (b >> 1) == 2 ? vs[2].z : vs[2].w;
      const uint32_t w3 = (b >> 1) == 0 ? vs[3].x : (b >> 1) == 1 ? vs[3].y : (b >> 1) == 2 ? vs[3].z : vs[3].w;
      const half4_t dv = __builtin_bit_cast(half4_t, (uint2){__builtin_amdgcn_perm(w1, w0, kSel[b & 1]),
                                                             __builtin_amdgcn_perm(w3, w2, kSel[b & 1])});
      const half4_t loh = lo * dv, hih = hi * dv;
      const half4_t lol = __builtin_elementwise_fma(lo, dv, -loh);
      const half4_t hil = __builtin_elementwise_fma(hi, dv, -hih);
      o[b][0] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, loh, o[b][0], 0, 0, 0);
      o[b][0] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, lol, o[b][0], 0, 0, 0);
      o[b][1] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, hih, o[b][1], 0, 0, 0);
      o[b][1] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, hil, o[b][1], 0, 0, 0);
    }
    wave_sync_lds();
  };
  // Two tile buffers, unrolled by two: one tile is in flight while the other
  // is processed, and no registers are copied between iterations.
  Tile ta, tb;
  fetch(ta, 0);
  for (int k = 0; k < my_tiles; k += 2) {
    fetch(tb, k + 1);
    process(ta, k);
    if (k + 1 >= my_tiles) break;
    fetch(ta, k + 2);
    process(tb, k + 1);
  }

  // Rows 8-15 of the P.V tiles hold the residual part (x 2^12): fold them in.
#pragma unroll
  for (int b = 0; b < kNB; ++b)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[b][m][i] = fmaf(__shfl_xor(o[b][m][i], 32, kWave), 1.0f / 4096.0f, o[b][m][i]);

  // ---- merge the four waves ----------------------------------------------
  float lsum = l_run + __shfl_xor(l_run, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  if (g == 0 && n < kRows) {
    mlw[wave][n][0] = m_run;
    mlw[wave][n][1] = lsum;
  }
  __syncthreads();
  // This lane's output rows are 4*g + i (rows >= 8 hold nothing).
  float fw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (4 * g + i) & 7;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mlw[w][r][0]);
    const float mw = mlw[wave][r][0];
    fw[i] = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
  }
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w && g < 2) {
#pragma unroll
      for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int d = 32 * b + 8 * (n >> 2) + (n & 3) + 4 * m;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* dst = &ob[4 * g + i][d];
            const float v = o[b][m][i] * fw[i];
            *dst = (w == 0) ? v : (*dst + v);
          }
        }
    }
    __syncthreads();
  }
  for (int r = wave; r < a.rows; r += kWaves) {
    float M = -INFINITY, L = 0.0f;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mlw[w][r][0]);
    for (int w = 0; w < kWaves; ++w) {
      const float mw = mlw[w][r][0];
      if (mw != -INFINITY) L += mlw[w][r][1] * exp2f(mw - M);
    }
    float* pr = part + r * a.pstride;
    if (lane == 0) {
      pr[0] = M;
      pr[1] = L;
    }
    for (int d = lane; d < kD; d += kWave) pr[kPartialHead + d] = ob[r][d];
  }
}

}  // namespace

bool q4_mfma_supported(const DevFmt& f, int rows) {
  const bool pow2 = (f.page_size & (f.page_size - 1)) == 0;
  return f.kind == HKV_KIND_Q4_0 && f.D == kD && rows <= kRows && f.page_size % kT == 0 && pow2;
}

hipError_t launch_decode_q4_mfma(const DevFmt& f, const DecArgs& a, dim3 grid, hipStream_t s) {
  decode_q4_mfma_kernel<<<grid, dim3(kWaves * kWave), 0, s>>>(f, a);
  return hipGetLastError();
}

}  // namespace hkv
