// hkv_decode_q4w.hip -- split-K paged decode attention over the Q4_0 cache
// for 9 to 32 query rows per KV head in one pass (a query window: GQA group
// x query tokens), head size 256, on the 32x32 matrix-core shapes (gfx950).
//
// What is computed is the decode of Strata pull request #21 ("How" item 2:
// Q4_0 codes dequantized in registers during the score accumulation; the
// merge note: the query rotated, the output rotated back, and windowed
// paths over several query tokens) in the paged form of the vLLM docs
// "vllm.v1.attention.ops.rocm_octave" (reference_attention).  The 8-row
// kernel (hkv_decode_q4.hip) streams the cache once per 8 rows; this one
// reads it once for up to 32 rows, so every code is unpacked once for all
// of them.
//
// One wave streams units of 32 tokens (two 16-token tiles, each one page
// run) of one sequence and one KV head:
//  * Loads: lane (token l % 16, group l / 16) loads chunks g, g + 4, ...,
//    g + 16 of its token's 288-byte slot (18 chunks: 8 K blocks, 8 V blocks,
//    the 8 K and the 8 V fp16 scales), from the unit after the current one.
//    Tokens past the split's end load the last valid token instead, which
//    the softmax masks out.  Code words go to LDS as [word][token], scales as
//    [K | V][block][token].
//  * Scores, S^T = K Q^T on v_mfma_f32_32x32x16_f16, two products per
//    16-dim slice of a Q4_0 block: A = the codes as exact fp16 (c - 8), lane
//    l: token l % 32, one code word; B = the rotated query, each row scaled
//    into [2^14, 2^15), as an fp16 leading part and the unscaled fp16
//    residual, both into one fp32 accumulator per block, which is then
//    scaled by the tokens' fp16 block scales.  Lane l ends with the scores of
//    row l % 32 for tokens 8 j + 4 (l / 32) + i, j, i < 4.
//  * P.V on v_mfma_f32_32x32x16_f16 as O^T = V^T P^T (rows = dims, columns
//    = query rows), 8 tokens per product: a lane's k-slots are its own 4
//    tokens' fp16(p) (rounded to nearest) and their residuals x 2^6 -- the
//    scores it holds, so p never moves between lanes -- against the value
//    v = (c - 8) d_v split exactly into an fp16 leading part and residual:
//    [lead, lead x 2^-6] against [p, residual x 2^6] in one product per 8
//    tokens, [residual of 8 tokens] against [p of 8 tokens] in one more per
//    16 (the dropped residual x residual term is below 2^-22 of v p).  The
//    2^6 split keeps both scaled operands normal for all but the smallest
//    values and weights, where the term they carry is itself ~2^-11 of
//    the product and unbiased.
//  * V dims: tile (bp, half) of 32 dims (V blocks 2 bp, 2 bp + 1; the low or
//    high nibbles) has row a = 4 m + j holding dim 64 bp + 8 m + j + 4 half
//    (m < 8, j < 4): a lane gathers byte j of V word m of its 4 tokens once
//    and takes both tiles' values from it.
//  * Online softmax in the exp2 domain with the lazy rescale; the waves
//    merge in LDS and write one partial record per row; the shared merge
//    kernel combines the splits and rotates the output back.
#include "hkv_decode_common.h"

namespace hkv {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 256;             // head size handled here
constexpr int kNB = kD / 32;        // Q4_0 blocks per head vector
constexpr int kR = 32;              // query rows per KV head
constexpr int kT = 16;              // tokens per tile
constexpr int kTS = kT + 4;         // token stride (words) of the transposed tile
constexpr int kSlot = kD + kD / 8;  // 288: K codes, V codes, 8 K and 8 V fp16 scales
constexpr int kCodeWords = 64;      // K code words 0-31, V code words 32-63
constexpr int kLastChunk = kSlot / 16 - 1;  // 17
constexpr int kLoads = 5;           // chunks g, g + 4, ..., g + 16 per lane
constexpr int kQWaves = 8;          // waves per workgroup (two per SIMD)
constexpr int kMaxSplitTiles = 256;
constexpr float kLazy = 8.0f;       // log2 headroom before the running max is raised
constexpr int kOB = 65;             // row stride (floats) of the cross-wave sum
static_assert(kMaxSplitTiles <= kQWaves * kWave, "one page id per thread");

struct __align__(16) Q4wLds {
  float qsc[kR];             // per-row factor: q_scale / row scale
  float mlw[kQWaves][kR][2];
  int pid[kMaxSplitTiles];   // page of each tile of the split
  int next_unit;             // work queue: the next unit no wave has taken
  int pad_[3];
  union {
    struct {
      uint32_t tt[kQWaves][2][kCodeWords][kTS];  // [wave][tile][code word][token]
      _Float16 sc[kQWaves][2][2][kNB][kT];      // [wave][tile][K | V][block][token]
      // [lead | residual][block][row][k]; rows padded to 40 halves, so the
      // 16-byte reads of 16 rows at a time cover every bank once
      _Float16 qB[2][kNB][kR][40];
    } s;
    float ob[kQWaves][2][kR][kOB];  // [wave][l / 32][row][value], half of the dims at a time
  } u;
};

struct Tile {
  uint4 c[kLoads];
};

__global__ __launch_bounds__(kQWaves * kWave, 1) void decode_q4w32_kernel(DevFmt f, DecArgs a) {
  constexpr int W = kQWaves;
  constexpr int kE = kD / kWave;  // query values per lane
  constexpr int kQR = kR / W;     // query rows set up per wave
  __shared__ Q4wLds L;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int page_size = f.page_size, k_block = f.k_block;
  float k_norm = f.k_norm;
  pin_args(a, page_size, k_block, k_norm);
  int split, kvh, gi;
  if (!wg_item(a, split, kvh, gi)) return;
  const int q0 = gi * a.n_q;
  // ---- prologue: three memory round trips before the stream (query rows
  // and key lengths; page ids; the first tiles), every load unconditional.
  uint32_t qw[kQR][kE];
#pragma unroll
  for (int k = 0; k < kQR; ++k) query_row_raw<kE>(a, q0, kvh, wave + W * k, lane, qw[k]);
  const int kl = group_klen_lane(a, q0, lane);  // n_q <= kR
  const int req = a.q_to_req[q0];
  const int kmax = wave_max_int(kl);
  const int kmin = wave_min_int(kl);
  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(t_begin + a.tokens_per_split, kmax);
  float* part = a.ws + (((size_t)gi * a.num_kv_heads + kvh) * a.num_splits + split) * kR *
                           a.pstride;
  // (req < 0 never holds for a valid request map; testing it keeps the load
  // of req ahead of this branch, in the first round trip.)
  if (t_begin >= t_end || req < 0) {
    for (int r = threadIdx.x; r < a.rows; r += blockDim.x) {
      part[r * a.pstride + 0] = -INFINITY;
      part[r * a.pstride + 1] = 0.0f;
    }
    return;
  }

  const int32_t* bt = a.block_table + (int64_t)req * a.max_pages;
  const int ps = page_size;  // a power of two, multiple of kT
  const int ps_shift = 31 - __builtin_clz(ps);
  const int nt = (t_end - t_begin + kT - 1) / kT;  // tiles in the split
  const int nu = (nt + 1) >> 1;                     // units in the split
  const int tpid = min((int)threadIdx.x, nt - 1);
  const int pidv = bt[(t_begin + kT * tpid) >> ps_shift];
  __builtin_amdgcn_sched_barrier(0);
  const int tl = lane & 15, gq = lane >> 4;
  auto fetch_pid = [&](Tile& x, int kc, int page) {
    const int t0 = t_begin + kT * kc;
    const uint8_t* base = a.cache + ((((int64_t)page * a.num_kv_heads + kvh) << ps_shift) +
                                     (t0 & (ps - 1))) * (int64_t)kSlot;
    const uint8_t* slot = base + min(tl, t_end - 1 - t0) * kSlot;
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      x.c[i] = *(const uint4*)(slot + 16 * min(4 * i + gq, kLastChunk));
  };
  auto fetch = [&](Tile& x, int k) {
    const int kc = min(k, nt - 1);
    fetch_pid(x, kc, __builtin_amdgcn_readfirstlane(L.pid[kc]));
  };
  Tile ta, tb;
  const bool has_work = wave < nu;
  {
    const int k0 = min(2 * wave, nt - 1), k1 = min(2 * wave + 1, nt - 1);
    const int pg0 = bt[(t_begin + kT * k0) >> ps_shift];
    const int pg1 = bt[(t_begin + kT * k1) >> ps_shift];
    fetch_pid(ta, k0, pg0);
    fetch_pid(tb, k1, pg1);
  }
  __builtin_amdgcn_sched_barrier(0);
  L.pid[tpid] = pidv;
  if (threadIdx.x == 0) L.next_unit = W;
  // Query rows wave + W k, rotated, as the fp16 B operand: each row scaled
  // by 2^k so that its largest value lies in [2^14, 2^15); leading part and
  // exact residual.  Dim d of block b sits at k = 8 w + i with w = (d / 8)
  // % 4 and, for j = d % 8, i = j / 2 + 4 (j % 2) (the order in which the
  // code words unpack).
#pragma unroll
  for (int k = 0; k < kQR; ++k) {
    const int r = wave + W * k;
    float x[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) x[e] = query_value(a, qw[k][e], r < a.rows);
    fwht_strided<kE>(x, k_block, k_norm);
    float qmax = 0.0f;
#pragma unroll
    for (int e = 0; e < kE; ++e) qmax = fmaxf(qmax, fabsf(x[e]));
    qmax = wave_max(qmax);
    const float rs = qmax > 0.0f ? ldexpf(1.0f, 14 - ilogbf(qmax)) : 1.0f;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const float y = x[e] * rs;
      const _Float16 hi = (_Float16)y;
      const int d = kWave * e + lane;
      const int j = d & 7;
      const int kk = 8 * ((d >> 3) & 3) + (j >> 1) + 4 * (j & 1);
      L.u.s.qB[0][d >> 5][r][kk] = hi;
      L.u.s.qB[1][d >> 5][r][kk] = (_Float16)(y - (float)hi);  // exact difference
    }
    if (lane == 0) L.qsc[r] = a.q_scale / rs;
  }
  const int n = lane & 31;  // query row (scores, P.V columns); token / dim row of the A operands
  const int h = lane >> 5;
  const int klen_lane_row = __shfl(kl, (n < a.rows ? n : 0) / a.group, kWave);
  const int klen_row = n < a.rows ? klen_lane_row : 0;
  const int t_lim = min(t_end, kmin);  // units ending at or before this need no mask
  // V operand row n = 4 m + j: byte j of V word m (block m / 4, word m % 4)
  // of a block pair.
  const int vm = n >> 2;
  const uint32_t vsel = (uint32_t)(n & 3) | (0x0Cu << 8) | ((uint32_t)(4 + (n & 3)) << 16) |
                        (0x0Cu << 24);
  __syncthreads();
  // (kept positive so that a masked score, -inf, stays -inf through the fma)
  const float qs = fmaxf(L.qsc[n], 0x1p-126f);
  // Nibble masks kept in VGPRs so that mask-and-bias fuses into v_and_or_b32
  // (whose third operand, the fp16 exponent bias, then comes from an SGPR).
  uint32_t m000f, m00f0, m0f, mf0;
  asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(m000f));
  asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(m00f0));
  asm volatile("v_mov_b32 %0, 0x0f0f0f0f" : "=v"(m0f));
  asm volatile("v_mov_b32 %0, 0xf0f0f0f0" : "=v"(mf0));

  f32x16 o[kNB];  // tile 2 bp + half: V blocks 2 bp, 2 bp + 1, low or high nibbles
#pragma unroll
  for (int b = 0; b < kNB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  if (has_work) {
    uint32_t* const tw = &L.u.s.tt[wave][0][0][0];
    _Float16* const sw = &L.u.s.sc[wave][0][0][0][0];
    int u_cur = wave;
    for (;;) {
      // ---- stage the unit's two tiles (registers -> LDS) ----
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const Tile& x = hb ? tb : ta;
        uint32_t* w = tw + hb * (kCodeWords * kTS) + tl;
#pragma unroll
        for (int i = 0; i < kLoads - 1; ++i) {
          w[(16 * i + 4 * gq + 0) * kTS] = x.c[i].x;
          w[(16 * i + 4 * gq + 1) * kTS] = x.c[i].y;
          w[(16 * i + 4 * gq + 2) * kTS] = x.c[i].z;
          w[(16 * i + 4 * gq + 3) * kTS] = x.c[i].w;
        }
        if (gq < 2) {  // chunk 16: the K scales, chunk 17: the V scales
          _Float16* s = sw + ((hb * 2 + gq) * kNB) * kT + tl;
          const uint4 c = x.c[kLoads - 1];
          const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            s[(2 * q) * kT] = __builtin_bit_cast(_Float16, (uint16_t)(cw[q] & 0xffffu));
            s[(2 * q + 1) * kT] = __builtin_bit_cast(_Float16, (uint16_t)(cw[q] >> 16));
          }
        }
      }
      wave_sync_lds();
      int u_nxt = u_cur + W;  // deterministic mode: a fixed order
      if (!a.det) {
        if (lane == 0) u_nxt = atomicAdd(&L.next_unit, 1);
        u_nxt = __builtin_amdgcn_readfirstlane(u_nxt);
      }
      if (u_nxt < nu) {
        fetch(ta, 2 * u_nxt);
        fetch(tb, 2 * u_nxt + 1);
      }

      // ---- scores: 32 tokens x 32 rows ----
      float s[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = 0.0f;
      {
        const uint32_t* tk = tw + (n >> 4) * (kCodeWords * kTS) + (n & 15);
        const half2_t c1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
        const half2_t c16 = {(_Float16)0.0625f, (_Float16)0.0625f};
        const half2_t c72 = {(_Float16)-72.0f, (_Float16)-72.0f};
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
          f32x16 acc = {};
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) {
            // word 2 sl + h of block b: dims 8 (2 sl + h) .. + 7 as exact fp16
            const uint32_t x = tk[(4 * b + 2 * sl + h) * kTS], x8 = x >> 8;
            const half2_t h0 = __builtin_bit_cast(half2_t, (x & m000f) | 0x64006400u) + c1032;
            const half2_t h1 = __builtin_elementwise_fma(
                __builtin_bit_cast(half2_t, (x & m00f0) | 0x64006400u), c16, c72);
            const half2_t h2 = __builtin_bit_cast(half2_t, (x8 & m000f) | 0x64006400u) + c1032;
            const half2_t h3 = __builtin_elementwise_fma(
                __builtin_bit_cast(half2_t, (x8 & m00f0) | 0x64006400u), c16, c72);
            const half8_t A = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
            const half8_t bh = *(const half8_t*)&L.u.s.qB[0][b][n][16 * sl + 8 * h];
            const half8_t bl = *(const half8_t*)&L.u.s.qB[1][b][n][16 * sl + 8 * h];
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, bl, acc, 0, 0, 0);
          }
          // K scales of block b for tokens 8 j + 4 h + i
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const half4_t ks = *(const half4_t*)(sw + (((j >> 1) * 2 + 0) * kNB + b) * kT +
                                                 8 * (j & 1) + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) s[4 * j + i] = fmaf(acc[4 * j + i], (float)ks[i], s[4 * j + i]);
          }
        }
      }
      const int t0 = t_begin + 2 * kT * u_cur;
      if (!(t0 + 2 * kT <= t_lim)) {
        asm volatile("" ::: "memory");  // keep this a branch: only edge units mask
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = t0 + 8 * j + 4 * h + i;
            s[4 * j + i] = (t < t_end && t < klen_row) ? s[4 * j + i] : -INFINITY;
          }
      }
      float mt = s[0];
#pragma unroll
      for (int k = 1; k < 16; ++k) mt = fmaxf(mt, s[k]);
      {
        const uint32_t u = __float_as_uint(mt);
        const auto sw2 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        mt = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1])) * qs;
      }
      if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy) != 0) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < kNB; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[b][i] *= alpha;
        m_run = m_new;
      }
      const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;
      // P operands: step j, k-slots 0-3 fp16(p) of tokens 8 j + 4 h + i,
      // 4-7 the residuals x 2^6
      half8_t P[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[4 * j + i], qs, -m_ref));  // exp2(-inf) = 0
          l_run += p;
          const _Float16 ph = (_Float16)p;
          P[j][i] = ph;
          P[j][4 + i] = (_Float16)((p - (float)ph) * 64.0f);  // exact before the rounding
        }
      }
      // fp16(p) of steps (0, 1) and (2, 3): the partner of the value residuals
      const half8_t P2[2] = {
          {P[0][0], P[0][1], P[0][2], P[0][3], P[1][0], P[1][1], P[1][2], P[1][3]},
          {P[2][0], P[2][1], P[2][2], P[2][3], P[3][0], P[3][1], P[3][2], P[3][3]}};

      // ---- P.V: 8 accumulator tiles of 32 dims ----
      const half4_t c1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f, (_Float16)-1032.0f,
                             (_Float16)-1032.0f};
      const half4_t c16 = {(_Float16)0.0625f, (_Float16)0.0625f, (_Float16)0.0625f,
                           (_Float16)0.0625f};
      const half4_t c72 = {(_Float16)-72.0f, (_Float16)-72.0f, (_Float16)-72.0f, (_Float16)-72.0f};
      const half4_t c64 = {(_Float16)0.015625f, (_Float16)0.015625f, (_Float16)0.015625f,
                           (_Float16)0.015625f};
#pragma unroll
      for (int bp = 0; bp < kNB / 2; ++bp) {
        const int vb = 2 * bp + (vm >> 2);  // this lane's V block
        const uint32_t* vw = tw + (kCodeWords / 2 + 4 * vb + (vm & 3)) * kTS + 4 * h;
        const _Float16* vs = sw + (kNB + vb) * kT + 4 * h;  // V scales of block vb, tile 0
        half4_t lo_res[2], hi_res[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // byte n % 4 of V word vm of tokens 8 j + 4 h + i -> halves (t0, t1), (t2, t3)
          const uint4 Wd = lds_u4(vw + (j >> 1) * (kCodeWords * kTS) + 8 * (j & 1));
          const uint32_t x01 = __builtin_amdgcn_perm(Wd.y, Wd.x, vsel);
          const uint32_t x23 = __builtin_amdgcn_perm(Wd.w, Wd.z, vsel);
          const uint2 lw = {(x01 & m0f) | 0x64006400u, (x23 & m0f) | 0x64006400u};
          const uint2 hw = {(x01 & mf0) | 0x64006400u, (x23 & mf0) | 0x64006400u};
          const half4_t cl = __builtin_bit_cast(half4_t, lw) + c1032;  // c - 8, low nibbles
          const half4_t ch = __builtin_elementwise_fma(__builtin_bit_cast(half4_t, hw), c16, c72);
          const half4_t dv = *(const half4_t*)(vs + (j >> 1) * (2 * kNB * kT) + 8 * (j & 1));
          const half4_t lh = cl * dv, hh = ch * dv;
          const half4_t ll = __builtin_elementwise_fma(cl, dv, -lh);  // exact residuals
          const half4_t hl = __builtin_elementwise_fma(ch, dv, -hh);
          const half4_t ls = lh * c64, hs = hh * c64;
          const half8_t AL = {lh[0], lh[1], lh[2], lh[3], ls[0], ls[1], ls[2], ls[3]};
          const half8_t AH = {hh[0], hh[1], hh[2], hh[3], hs[0], hs[1], hs[2], hs[3]};
          o[2 * bp] = __builtin_amdgcn_mfma_f32_32x32x16_f16(AL, P[j], o[2 * bp], 0, 0, 0);
          o[2 * bp + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(AH, P[j], o[2 * bp + 1], 0, 0, 0);
          lo_res[j & 1] = ll;
          hi_res[j & 1] = hl;
          if (j & 1) {
            const half8_t RL = {lo_res[0][0], lo_res[0][1], lo_res[0][2], lo_res[0][3],
                                lo_res[1][0], lo_res[1][1], lo_res[1][2], lo_res[1][3]};
            const half8_t RH = {hi_res[0][0], hi_res[0][1], hi_res[0][2], hi_res[0][3],
                                hi_res[1][0], hi_res[1][1], hi_res[1][2], hi_res[1][3]};
            o[2 * bp] = __builtin_amdgcn_mfma_f32_32x32x16_f16(RL, P2[j >> 1], o[2 * bp], 0, 0, 0);
            o[2 * bp + 1] =
                __builtin_amdgcn_mfma_f32_32x32x16_f16(RH, P2[j >> 1], o[2 * bp + 1], 0, 0, 0);
          }
        }
      }
      if (u_nxt >= nu) break;
      u_cur = u_nxt;
    }
  }

  // ---- merge the waves ----------------------------------------------------
  // This lane: row n, register i of tile 2 bp + half holds dim
  // 64 bp + 16 (i / 4) + 8 h + 4 half + i % 4.
  float lsum;
  {
    const uint32_t lu = __float_as_uint(l_run);
    const auto ls = __builtin_amdgcn_permlane32_swap(lu, lu, false, false);
    lsum = __uint_as_float(ls[0]) + __uint_as_float(ls[1]);
  }
  if (h == 0) {
    L.mlw[wave][n][0] = m_run;
    L.mlw[wave][n][1] = lsum;
  }
  __syncthreads();
  float fw;
  {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, L.mlw[w][n][0]);
    fw = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - M);
  }
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2) {
    if (b2) __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) L.u.ob[wave][h][n][16 * t + i] = o[4 * b2 + t][i] * fw;
    __syncthreads();
    for (int idx = threadIdx.x; idx < a.rows * 128; idx += blockDim.x) {
      const int r = idx >> 7, dd = idx & 127;
      // dd = 64 bpl + 16 i4 + 8 hh + 4 half + ii -> tile 2 bpl + half, register 4 i4 + ii
      const int bpl = dd >> 6, i4 = (dd >> 4) & 3, hh = (dd >> 3) & 1, half = (dd >> 2) & 1,
                ii = dd & 3;
      const int k = 16 * (2 * bpl + half) + 4 * i4 + ii;
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) acc += L.u.ob[w][hh][r][k];
      part[r * a.pstride + kPartialHead + 128 * b2 + dd] = acc;
    }
  }
  if (threadIdx.x < a.rows) {
    const int r = threadIdx.x;
    float M = -INFINITY, L_ = 0.0f;
    for (int w = 0; w < W; ++w) M = fmaxf(M, L.mlw[w][r][0]);
    for (int w = 0; w < W; ++w) {
      const float mw = L.mlw[w][r][0];
      if (mw != -INFINITY) L_ += L.mlw[w][r][1] * exp2f(mw - M);
    }
    part[r * a.pstride + 0] = M;
    part[r * a.pstride + 1] = L_;
  }
}

}  // namespace

bool q4w_mfma_supported(const DevFmt& f, int rows) {
  const bool pow2 = (f.page_size & (f.page_size - 1)) == 0;
  return f.kind == HKV_KIND_Q4_0 && !f.use_signs && f.D == kD && f.slot_bytes == kSlot &&
         rows > 8 && rows <= kR && f.page_size % kT == 0 && pow2;
}

hipError_t launch_decode_q4w(const DevFmt& f, const DecArgs& a, dim3 grid, hipStream_t s) {
  // The page ids of a split's tiles are held in LDS.
  if ((a.tokens_per_split + kT - 1) / kT > kMaxSplitTiles || a.rows_pad != kR)
    return hipErrorInvalidValue;
  decode_q4w32_kernel<<<grid, dim3(kQWaves * kWave), 0, s>>>(f, a);
  return hipGetLastError();
}

}  // namespace hkv
