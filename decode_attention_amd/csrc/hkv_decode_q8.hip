// hkv_decode_q8.hip -- split-K paged decode attention over the Q8_0 cache on
// the matrix cores (gfx950), for head size 256 and up to 8 query rows per KV
// head (GQA group x query tokens).
//
// What is computed is the int8 mode Strata pull request #21 compares its
// Q4_0 cache against ("Why": int8 + FWHT as the default; the rotation of
// "How" item 1 applied the same way), decoded as in its "How" item 2 (codes
// dequantized in registers during the score accumulation, the query rotated
// and the output rotated back), in the paged form of the vLLM docs
// "vllm.v1.attention.ops.rocm_octave" (reference_attention).  A slot holds the
// 256 K codes, the 256 V codes, then 8 K and 8 V fp16 block scales (one per
// 32 values); a value is its code times its block's scale.
//
// One wave streams units of 32 tokens (two 16-token tiles) of one sequence
// and one KV head, one unit after another:
//  * Scores, S^T = K Q^T on v_mfma_i32_16x16x32_i8, one per 32-value block
//    and tile: A is the block's int8 codes as loaded (lane (n, g): token n,
//    codes 8 g .. 8 g + 7, one 8-byte load each), B the rotated query as
//    three int8 planes, q = 2^16 hi + 2^8 mid + lo per row (~23 bits of the
//    row's largest value, so the scores keep fp32 accuracy at any query
//    magnitude), in two products: B columns [hi | lo] (8 rows x 2), then
//    [mid | 0] accumulated onto the first result shifted left 8 bits, which
//    leaves 2^8 hi + mid and 2^8 lo in lanes n and n + 8; each block's int32
//    result is scaled by the token's fp16 block scale.
//  * A lane then holds 4 consecutive tokens of one row per tile: the 8
//    scores of a unit are the A operand of v_mfma_f32_16x16x32_f16 for P.V
//    (rows 0-7 fp16(p), rows 8-15 the residual x 2^12).  B is code x scale
//    split exactly into an fp16 leading part and residual (an 8-bit code
//    times an 11-bit mantissa has 19 bits), the code gathered from a
//    transposed LDS tile with v_perm_b32 and made an fp16 with the 0x6400
//    bias (sign bit flipped in the same XOR).
//  * The work is bound by the HBM stream (17 KB per unit against ~560 VALU
//    instructions), so a unit's loads are simply issued one unit ahead of
//    its use, with no interleaving of two units in the loop body.
//  * Online softmax in the exp2 domain, rescaling only when a row maximum
//    grows by more than kLazy; the eight waves merge in LDS and write one
//    partial record per row; the shared merge kernel combines the splits and
//    rotates the output back.
#include "hkv_decode_common.h"

namespace hkv {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 256;                 // head size handled here
constexpr int kNB = kD / 32;            // Q8_0 blocks per head vector
constexpr int kRows = 8;                // query rows per KV head
constexpr int kT = 16;                  // tokens per tile
constexpr int kSlot = 2 * kD + kD / 8;  // 544: K codes, V codes, 8 + 8 fp16 scales
constexpr int kQMaxI = kQ3MaxI;         // largest |q| code of the three-plane int8 split
constexpr float kQMax = (float)kQ3MaxI;
constexpr int kVS = kT + 4;             // padded token stride of the transposed V tile
constexpr float kLazy = 8.0f;           // log2 headroom before the running max is raised
constexpr int kQWaves = 8;              // waves per workgroup (two per SIMD)
constexpr int kMaxSplitTiles = 256;     // page ids of a split's tiles held in LDS
static_assert(kMaxSplitTiles <= kQWaves * kWave, "one page id per thread");

// Lane (tl, gq) of a tile: token tl's K codes 32 b + 8 gq .. + 7 of every
// block b (the score A operand of lane (tl, gq)), V chunks gq, 4 + gq,
// 8 + gq, 12 + gq (16 bytes each) and one 16-byte scale chunk (K scales for
// gq even, V for gq odd).
struct Tile8 {
  uint2 k[kNB];
  uint4 v[4];
  uint4 sc;
};

struct __align__(16) Q8Lds {
  // B operand bytes, [block][column][dim]: columns r (hi), 8 + r (lo),
  // 16 + r (mid) of row r, 24-31 zero.
  int8_t qB[kNB][32][32];
  float qsc[kRows];        // per-row score scale
  float mlw[kQWaves][kRows][2];
  int pid[kMaxSplitTiles];  // page of each tile of the split
  int next_unit;            // work queue: the next unit no wave has taken
  int pad_[3];
  union {
    struct {
      uint32_t vt[kQWaves][2][kNB][8][kVS];  // V words: [tile][block][word][token]
      // fp16 block scales: [K|V][block][token group g][tile][token 4g..4g+3],
      // so a lane's eight V scales of a block (both tiles) are 16 contiguous
      // bytes and its four K scales of a block and tile are 8
      uint16_t sh[kQWaves][2][kNB][4][2][4];
    } s;
    float ob[kQWaves][kRows][kD];  // wave merge, after the stream
  } u;
};

__global__ __launch_bounds__(kQWaves * kWave, 1) void decode_q8_mfma_kernel(DevFmt f, DecArgs a) {
  __shared__ Q8Lds L;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lane = threadIdx.x & 63;
  int page_size = f.page_size, k_block = f.k_block;
  float k_norm = f.k_norm;
  pin_args(a, page_size, k_block, k_norm);
  int split, kvh, gi;
  if (!wg_item(a, split, kvh, gi)) return;
  const int q0 = gi * a.n_q;
  // ---- prologue: three memory round trips before the stream -------------
  // (1) the query row of this wave (raw bits), the key lengths of the
  //     group's queries (one per lane) and the request; (2) the split's page
  //     ids, to LDS, and this wave's first two (scalar); (3) the first unit's
  //     tiles.  Every load of the prologue is unconditional (clamped
  //     indices), so no wait before the barrier covers a later round trip.
  uint32_t qw[4];
  query_row_raw<4>(a, q0, kvh, wave, lane, qw);
  uint32_t sw[4];
  lane_sign_words<4>(f, f.use_signs, lane, sw);
  const int kl = group_klen_lane(a, q0, lane);
  const int req = a.q_to_req[q0];
  const int kmax = wave_max_int(kl);
  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(t_begin + a.tokens_per_split, kmax);
  float* part = a.ws + (((size_t)gi * a.num_kv_heads + kvh) * a.num_splits + split) * kRows *
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
  const int ps = page_size;                   // a power of two, multiple of kT
  const int ps_shift = 31 - __builtin_clz(ps);
  const int nt = (t_end - t_begin + kT - 1) / kT;  // tiles in the split
  const int nu = (nt + 1) >> 1;                    // units in the split
  // One page id per thread (nt <= kMaxSplitTiles); threads past the last
  // tile load and later store the last one again.
  const int tpid = min((int)threadIdx.x, nt - 1);
  const int pidv = bt[(t_begin + kT * tpid) >> ps_shift];
  __builtin_amdgcn_sched_barrier(0);
  const int tl = lane & 15, gq = lane >> 4;
  // Tile k of the split (clamped to the last tile: the scores of a tile past
  // the end are masked, so reloading the last one keeps every load in
  // bounds), from its page id.
  auto fetch_pid = [&](Tile8& x, int kc, int page) {
    const int t0 = t_begin + kT * kc;
    const uint8_t* base = a.cache + ((((int64_t)page * a.num_kv_heads + kvh) << ps_shift) +
                                     (t0 & (ps - 1))) * (int64_t)kSlot;
    const uint8_t* slot = base + min(tl, t_end - 1 - t0) * kSlot;
#pragma unroll
    for (int b = 0; b < kNB; ++b) x.k[b] = *(const uint2*)(slot + 32 * b + 8 * gq);
#pragma unroll
    for (int i = 0; i < 4; ++i) x.v[i] = *(const uint4*)(slot + kD + 16 * (4 * i + gq));
    x.sc = *(const uint4*)(slot + 2 * kD + 16 * (gq & 1));
  };
  auto fetch = [&](Tile8& x, int k) {
    const int kc = min(k, nt - 1);
    fetch_pid(x, kc, __builtin_amdgcn_readfirstlane(L.pid[kc]));
  };
  // The first unit's tiles, with page ids read directly (a wave with no
  // unit loads the last tile and never uses it).
  Tile8 ta, tb;
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
  if (threadIdx.x == 0) L.next_unit = kQWaves;

  // Query row `wave` -> rotated, scaled int8 planes (B operand).
  {
    const int r = wave;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = flip_sign(query_value(a, qw[e], r < a.rows), sw[e], lane);
    fwht_strided<4>(x, k_block, k_norm);
    float qmax = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) qmax = fmaxf(qmax, fabsf(x[e]));
    qmax = wave_max(qmax);
    // |q| <= kQ3MaxI keeps the three planes in int8 (q_split3).
    const float inv = qmax > 0.0f ? kQMax / qmax : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int qi = (int)rintf(x[e] * inv);
      qi = min(kQMaxI, max(-kQMaxI, qi));
      int hi, mid, lo;
      q_split3(qi, hi, mid, lo);
      const int d = kWave * e + lane;
      L.qB[d >> 5][r][d & 31] = (int8_t)hi;
      L.qB[d >> 5][8 + r][d & 31] = (int8_t)lo;
      L.qB[d >> 5][16 + r][d & 31] = (int8_t)mid;
      L.qB[d >> 5][24 + r][d & 31] = 0;
    }
    if (lane == 0) L.qsc[r] = (qmax / kQMax) * a.q_scale;
  }
  const int n = lane & 15;   // score column (row r = n & 7, plane = n >> 3)
  const int g = lane >> 4;   // lane group: tokens 4g..4g+3 of a tile in the score layout
  const int row = n & 7;
  const int klen_lane_row = __shfl(kl, (row < a.rows ? row : 0) / a.group, kWave);
  const int klen_row = row < a.rows ? klen_lane_row : 0;
  const int kmin = wave_min_int(kl);
  __syncthreads();

  const float qs = L.qsc[row];
  // The query's B operand of every block, held in registers for the whole stream.
  // (the mid plane is read from LDS at each use: registers are full)
  long qreg[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) qreg[b] = *(const long*)&L.qB[b][n][8 * g];
  const long* const qmid = (const long*)&L.qB[0][16 + n][8 * g];
  const float w_own = n < 8 ? 256.0f * qs : qs * (1.0f / 256.0f);
  const float w_partner = n < 8 ? qs * (1.0f / 256.0f) : 256.0f * qs;
  const bool live_row = row < a.rows;  // lanes n and n + 8 carry the same row
  const float alpha_a = live_row ? (n < 8 ? 1.0f : 4096.0f) : 0.0f;
  const float beta_a = live_row ? (n < 8 ? 0.0f : -4096.0f) : 0.0f;
  // Byte (n & 3) of two tokens' V words into the low bytes of two halves.
  const uint32_t vsel = (uint32_t)(n & 3) | (0x0Cu << 8) | ((uint32_t)(4 + (n & 3)) << 16) |
                        (0x0Cu << 24);
  const int t_lim = min(t_end, kmin);  // units ending at or before this need no mask

  float4_t o[kNB][2];
#pragma unroll
  for (int b = 0; b < kNB; ++b) o[b][0] = o[b][1] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  if (has_work) {
    int u_cur = wave;
    for (;;) {
      // ---- V words and scales of the unit -> LDS ----
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const Tile8& x = hb ? tb : ta;
        uint32_t* vw = &L.u.s.vt[wave][hb][0][0][tl];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // chunk 4 i + gq: words 4 ((4 i + gq) & 1) .. + 3 of block (4 i + gq) >> 1
          const int c = 4 * i + gq;
          uint32_t* d = vw + ((c >> 1) * 8 + 4 * (c & 1)) * kVS;
          d[0 * kVS] = x.v[i].x;
          d[1 * kVS] = x.v[i].y;
          d[2 * kVS] = x.v[i].z;
          d[3 * kVS] = x.v[i].w;
        }
        if (gq < 2) {  // lanes 32-63 hold copies of the same scale chunks
          uint16_t* sw = &L.u.s.sh[wave][gq][0][tl >> 2][hb][tl & 3];
          constexpr int sb = 4 * 2 * 4;  // halves per block
          sw[0 * sb] = (uint16_t)x.sc.x;
          sw[1 * sb] = (uint16_t)(x.sc.x >> 16);
          sw[2 * sb] = (uint16_t)x.sc.y;
          sw[3 * sb] = (uint16_t)(x.sc.y >> 16);
          sw[4 * sb] = (uint16_t)x.sc.z;
          sw[5 * sb] = (uint16_t)(x.sc.z >> 16);
          sw[6 * sb] = (uint16_t)x.sc.w;
          sw[7 * sb] = (uint16_t)(x.sc.w >> 16);
        }
      }
      wave_sync_lds();
      uint2 ka[kNB], kb[kNB];
#pragma unroll
      for (int b = 0; b < kNB; ++b) ka[b] = ta.k[b], kb[b] = tb.k[b];
      int u_nxt = u_cur + kQWaves;  // deterministic mode: a fixed order
      if (!a.det) {
        if (lane == 0) u_nxt = atomicAdd(&L.next_unit, 1);
        u_nxt = __builtin_amdgcn_readfirstlane(u_nxt);
      }
      if (u_nxt < nu) {
        fetch(ta, 2 * u_nxt);
        fetch(tb, 2 * u_nxt + 1);
      }

      // ---- scores of both tiles ----
      float s[8];
      const int4_t zero4 = {0, 0, 0, 0};
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
          const uint2 kw = hb ? kb[b] : ka[b];
          const long ak = __builtin_bit_cast(long, kw);
          // (|2^8 hi + mid| sums stay below 2^28: 32 products of at most 2^14)
          int4_t C = __builtin_amdgcn_mfma_i32_16x16x32_i8(ak, qreg[b], zero4, 0, 0, 0);
          C = __builtin_amdgcn_mfma_i32_16x16x32_i8(ak, qmid[b * (32 * 32 / 8)], C << 8, 0, 0, 0);
          // K scales of block b for tokens 4g..4g+3 of this tile
          const uint2 ks = *(const uint2*)&L.u.s.sh[wave][0][b][g][hb][0];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t w = i < 2 ? ks.x : ks.y;
            const float sk = h2f((uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu)));
            acc[i] = fmaf((float)C[i], sk, acc[i]);
          }
          // (two blocks at a time: interleaving more holds more results live
          // than the registers allow)
          if (b & 1) __builtin_amdgcn_sched_barrier(0);
        }
        // lane n < 8 holds the hi plane and lane n + 8 the lo plane of a row
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[4 * hb + i] = pair_score(fmaf(acc[i], w_own, ror8(acc[i]) * w_partner), n);
      }

      // ---- softmax: mask, running max, p, the P.V A operand ----
      // (k = 8 g + j: j < 4 tile 0 token 4g+j, else tile 1 token 4g+j-4)
      const int t0a = t_begin + 2 * kT * u_cur;
      const int t0b = t0a + kT;
      if (!(t0b + kT <= t_lim)) {
        asm volatile("" ::: "memory");  // keep this a branch: only edge units mask
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ta_ = t0a + 4 * g + i, tb_ = t0b + 4 * g + i;
          s[i] = (ta_ < t_end && ta_ < klen_row) ? s[i] : -INFINITY;
          s[4 + i] = (tb_ < t_end && tb_ < klen_row) ? s[4 + i] : -INFINITY;
        }
      }
      float mt = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                       fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      mt = max_xor16_32(mt);
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
      const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;  // rows with nothing valid yet
      // Rows 0-7 of A carry fp16(p), rows 8-15 fp16((p - fp16(p)) * 2^12)
      // (zero for the padding rows past the group).
      half8_t A;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[i] - m_ref);  // exp2(-inf) = 0
        l_run += p;
        const _Float16 h = (_Float16)p;
        A[i] = (_Float16)fmaf((float)h, beta_a, p * alpha_a);
      }

      // ---- P.V: 16 tiles of 16 dims (dims 32 b + 16 m + n) ----
      const half8_t c1152 = {(_Float16)-1152.0f, (_Float16)-1152.0f, (_Float16)-1152.0f,
                             (_Float16)-1152.0f, (_Float16)-1152.0f, (_Float16)-1152.0f,
                             (_Float16)-1152.0f, (_Float16)-1152.0f};
      const uint32_t* vbase = &L.u.s.vt[wave][0][0][n >> 2][4 * g];
      constexpr int kVtTile = kNB * 8 * kVS;  // vt: dwords per tile
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        // V scales of block b for tokens 4g..4g+3 of both tiles, in the k
        // order of the A operand
        const half8_t dv = __builtin_bit_cast(
            half8_t, *(const uint4*)__builtin_assume_aligned(&L.u.s.sh[wave][1][b][g][0][0], 16));
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint4 W0 = lds_u4(vbase + (b * 8 + 4 * m) * kVS);
          const uint4 W1 = lds_u4(vbase + (b * 8 + 4 * m) * kVS + kVtTile);
          // code byte -> 0x64 (byte ^ 0x80): the fp16 1152 + code, exactly
          const uint4 x = {__builtin_amdgcn_perm(W0.y, W0.x, vsel) ^ 0x64806480u,
                           __builtin_amdgcn_perm(W0.w, W0.z, vsel) ^ 0x64806480u,
                           __builtin_amdgcn_perm(W1.y, W1.x, vsel) ^ 0x64806480u,
                           __builtin_amdgcn_perm(W1.w, W1.z, vsel) ^ 0x64806480u};
          const half8_t v = __builtin_bit_cast(half8_t, x) + c1152;
          const half8_t vh = v * dv;
          const half8_t vl = __builtin_elementwise_fma(v, dv, -vh);
          o[b][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, vh, o[b][m], 0, 0, 0);
          o[b][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, vl, o[b][m], 0, 0, 0);
        }
      }
      if (u_nxt >= nu) break;
      u_cur = u_nxt;
    }
  }

  // Rows 8-15 of the P.V tiles (lanes 32-63) hold the residual part (x 2^12):
  // fold them into rows 0-7 (lanes 0-31), which are the only ones used below.
#pragma unroll
  for (int b = 0; b < kNB; ++b)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u = __float_as_uint(o[b][m][i]);
        const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        o[b][m][i] = fmaf(__uint_as_float(sw[1]), 1.0f / 4096.0f, o[b][m][i]);
      }

  // ---- merge the waves ----------------------------------------------------
  float lsum = l_run + __shfl_xor(l_run, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  if (g == 0 && n < kRows) {
    L.mlw[wave][n][0] = m_run;
    L.mlw[wave][n][1] = lsum;
  }
  __syncthreads();  // every wave is past the stream: L.u may now hold ob
  // This lane's output rows are 4*g + i (lanes 0-31: rows 0-7).
  if (g < 2) {
    float fw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kQWaves; ++w) M = fmaxf(M, L.mlw[w][r][0]);
      const float mw = L.mlw[wave][r][0];
      fw[i] = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
    }
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int d = 32 * b + 16 * m + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) L.u.ob[wave][4 * g + i][d] = o[b][m][i] * fw[i];
      }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.rows * kD; idx += blockDim.x) {
    const int r = idx / kD, d = idx % kD;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kQWaves; ++w) acc += L.u.ob[w][r][d];
    part[r * a.pstride + kPartialHead + d] = acc;
  }
  if (threadIdx.x < a.rows) {
    const int r = threadIdx.x;
    float M = -INFINITY, L_ = 0.0f;
    for (int w = 0; w < kQWaves; ++w) M = fmaxf(M, L.mlw[w][r][0]);
    for (int w = 0; w < kQWaves; ++w) {
      const float mw = L.mlw[w][r][0];
      if (mw != -INFINITY) L_ += L.mlw[w][r][1] * exp2f(mw - M);
    }
    part[r * a.pstride + 0] = M;
    part[r * a.pstride + 1] = L_;
  }
}

}  // namespace

bool q8_mfma_supported(const DevFmt& f, int rows) {
  const bool pow2 = (f.page_size & (f.page_size - 1)) == 0;
  return f.kind == HKV_KIND_Q8_0 && f.D == kD && f.slot_bytes == kSlot && rows <= kRows &&
         f.page_size % kT == 0 && pow2;
}

hipError_t launch_decode_q8_mfma(const DevFmt& f, const DecArgs& a, dim3 grid, hipStream_t s) {
  // The page ids of a split's tiles are held in LDS.
  if ((a.tokens_per_split + kT - 1) / kT > kMaxSplitTiles) return hipErrorInvalidValue;
  decode_q8_mfma_kernel<<<grid, dim3(kQWaves * kWave), 0, s>>>(f, a);
  return hipGetLastError();
}

}  // namespace hkv
