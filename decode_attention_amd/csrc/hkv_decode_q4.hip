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
// One wave streams units of 32 tokens (two 16-token tiles, each one page run)
// of one sequence and one KV head.
//  * Scores, S^T = K Q^T on v_mfma_i32_16x16x32_i8 per tile: A = the 4-bit
//    codes of 16 tokens x one 32-value Q4_0 block as exact int8 16 (c - 8),
//    B = the rotated query as two int8 planes (q ~ s_h (256 hi + lo): 16
//    columns = 8 rows x {hi, lo}); each block's int32 result is scaled by the
//    token's fp16 block scale in fp32.  The int8 planes keep ~15 bits of q.
//  * Each lane ends up holding 4 consecutive tokens of one row per tile; the
//    8 scores of a unit are exactly the A operand of v_mfma_f32_16x16x32_f16
//    for P.V (k = 8 g + j), so P needs no transpose.  A rows 0-7 carry fp16(p),
//    rows 8-15 the residual x 2^12; B carries (c - 8) * v_scale split exactly
//    into an fp16 high part and the fp16 residual (a 4-bit integer times an
//    11-bit mantissa has <= 15 bits), regrouped from a transposed LDS tile
//    with v_perm_b32 and made exact fp16 with the 0x6400 bias trick.
//  * The loop body is {P.V of unit u; scores of unit u + 1} with no branch in
//    between, so the matrix cores and the VALU work of two units overlap;
//    loads past the wave's last tile are clamped to it (and masked), never
//    skipped by a branch.  V words, K words and scales pass through a
//    double-buffered per-wave LDS area.
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
typedef int int2_t __attribute__((ext_vector_type(2)));

constexpr int kD = 256;        // head size handled here
constexpr int kNB = kD / 32;   // Q4_0 blocks per head vector
constexpr int kRows = 8;       // query rows per KV head
constexpr int kT = 16;         // tokens per tile
constexpr int kSlot = kD + kD / 8;  // Q4_0 slot bytes at head size 256
constexpr int kQMaxI = 32639;  // largest |q| code of the two-plane int8 split
constexpr float kQMax = 32639.0f;
constexpr int kKStride = 4 * kNB + 4;  // dwords per token of the K tile ([word][block] + pad)
constexpr int kVStride = kT + 4;       // padded token stride of the transposed V tile
constexpr float kLazy = 8.0f;          // log2 headroom before the running max is raised
constexpr int kQWaves = 8;             // waves per workgroup (two per SIMD)
constexpr int kMaxSplitTiles = 256;    // page ids of a split's tiles held in LDS
static_assert(kMaxSplitTiles <= kQWaves * kWave, "one page id per thread");

__device__ __forceinline__ float f16lo(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16hi(uint32_t w) { return h2f((uint16_t)(w >> 16)); }


struct Tile {
  uint4 k0, k1, v0, v1, sc;
};

// Lane (tl, gq) of a tile reads token tl's K and V words of blocks gq and
// 4 + gq (16 bytes each) and one 16-byte scale chunk (K for gq even, V for gq
// odd; lanes 32-63 repeat the chunks of lanes 0-31, so no lane branches).
__device__ __forceinline__ void load_tile(Tile& x, const uint8_t* slot, int gq, int scale_kind) {
  x.k0 = *(const uint4*)(slot + 16 * gq);
  x.k1 = *(const uint4*)(slot + 16 * (4 + gq));
  x.v0 = *(const uint4*)(slot + kD / 2 + 16 * gq);
  x.v1 = *(const uint4*)(slot + kD / 2 + 16 * (4 + gq));
  x.sc = *(const uint4*)(slot + kD + 16 * scale_kind);
}

struct __align__(16) Q4Lds {
  int8_t qB[kNB][16][32];  // B operand bytes: [block][column][dim]
  float qsc[kRows];        // per-row score scale
  float mlw[kQWaves][kRows][2];
  int pid[kMaxSplitTiles];  // page of each tile of the split
  int next_unit;            // work queue: the next unit no wave has taken
  int pad_[3];
  union {
    struct {
      uint32_t kt[kQWaves][2][kT][kKStride];           // [tile of unit][token][word * 8 + block]
      uint32_t vt[kQWaves][2][2][kNB][4][kVStride];    // [buf][tile][block][word][token]
      // fp16 block scales, block-major: [buf][K|V][block][token group g][tile][token
      // 4g..4g+3], so one lane's eight V scales of a block (both tiles) are 16
      // contiguous bytes and its four K scales of a block and tile are 8
      uint16_t sh[kQWaves][2][2][kNB][4][2][4];
      uint16_t sh_dup[kQWaves][kNB][32];               // stores of lanes 32-63 (never read)
    } s;
    float ob[kQWaves][kRows][kD];  // wave merge, after the stream
  } u;
};

static_assert(sizeof(Q4Lds::u.s.sh[0][0][0][0]) == 4 * 2 * 4 * sizeof(uint16_t),
              "scale block stride");
static_assert(sizeof(Q4Lds::u.s.sh_dup[0][0]) == sizeof(Q4Lds::u.s.sh[0][0][0][0]),
              "dummy scale rows share the block stride");
static_assert(sizeof(Q4Lds::u.s.vt[0][0][0]) == kNB * 4 * kVStride * sizeof(uint32_t),
              "V tile stride");

__global__ __launch_bounds__(kQWaves * kWave, 1) void decode_q4_mfma_kernel(DevFmt f, DecArgs a) {
  __shared__ Q4Lds L;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lane = threadIdx.x & 63;
  int page_size = f.page_size, k_block = f.k_block;
  float k_norm = f.k_norm;
  pin_args(a, page_size, k_block, k_norm);
  int split, kvh, gi;
  if (!wg_item(a, split, kvh, gi)) return;
  const int q0 = gi * a.n_q;
  // ---- prologue: three memory round trips before the stream -------------
  // (1) the query row of this wave (raw bits), the request and the key
  //     lengths of the group's queries; (2) the split's page ids, to LDS, and
  //     this wave's first two (scalar); (3) the first unit's tiles.  Nothing
  //     waits on a later round trip before the barrier: every load of the
  //     prologue is unconditional (clamped indices), so the counter waits
  //     stay partial across the tile loads.  Rows past the group load row 0
  //     and are zeroed.
  const bool live_q = wave < a.rows;
  const int rq = live_q ? wave : 0;
  const int64_t qrow = (int64_t)(q0 + rq / a.group) * a.num_q_heads + kvh * a.group + rq % a.group;
  uint32_t qw[4];
  if (a.q_f16) {
    const uint16_t* qp = (const uint16_t*)a.query + qrow * kD + lane;
#pragma unroll
    for (int e = 0; e < 4; ++e) qw[e] = qp[kWave * e];
  } else {
    const uint32_t* qp = (const uint32_t*)a.query + qrow * kD + lane;
#pragma unroll
    for (int e = 0; e < 4; ++e) qw[e] = qp[kWave * e];
  }
  const int req = a.q_to_req[q0];
  int kl[kRows];  // key lengths of the group's queries (the last one repeated)
#pragma unroll
  for (int j = 0; j < kRows; ++j) kl[j] = a.q_to_klen[q0 + min(j, a.n_q - 1)];
  int kmax = kl[0], kmin = kl[0];
#pragma unroll
  for (int j = 1; j < kRows; ++j) {
    kmax = max(kmax, kl[j]);
    kmin = min(kmin, kl[j]);
  }
  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(t_begin + a.tokens_per_split, kmax);
  float* part = a.ws + (((size_t)gi * a.num_kv_heads + kvh) * a.num_splits + split) * kRows *
                           a.pstride;
  // (req < 0 never holds for a valid request map; testing it here keeps the
  // load of req ahead of this branch, in the same round trip as the key
  // lengths, instead of sunk below it.)
  if (t_begin >= t_end || req < 0) {
    for (int r = threadIdx.x; r < a.rows; r += blockDim.x) {
      part[r * a.pstride + 0] = -INFINITY;
      part[r * a.pstride + 1] = 0.0f;
    }
    return;
  }

  // The split is a queue of units of two consecutive 16-token tiles.  Wave w
  // starts with units w and w + 8 and then takes the next untaken unit, so
  // the two waves sharing a SIMD finish together however the issue slots
  // fall between them.
  const int32_t* bt = a.block_table + (int64_t)req * a.max_pages;
  const int ps = page_size;                   // a power of two, multiple of kT
  const int ps_shift = 31 - __builtin_clz(ps);
  const int nt = (t_end - t_begin + kT - 1) / kT;              // tiles in the split
  const int nu = (nt + 1) >> 1;                                // units in the split
  // One page id per thread (nt <= kMaxSplitTiles); threads past the last
  // tile load and later store the last one again.
  const int tpid = min((int)threadIdx.x, nt - 1);
  const int pidv = bt[(t_begin + kT * tpid) >> ps_shift];
  __builtin_amdgcn_sched_barrier(0);
  const int tl = lane & 15, gq = lane >> 4;
  const int scale_kind = (lane >> 4) & 1;
  // Tile k of the split (clamped to the last tile: the scores of a tile past
  // the end are masked, so reloading the last one keeps every load in
  // bounds), from its page id.
  auto fetch_pid = [&](Tile& x, int kc, int page) {
    const int t0 = t_begin + kT * kc;
    const uint8_t* base = a.cache + ((((int64_t)page * a.num_kv_heads + kvh) << ps_shift) +
                                     (t0 & (ps - 1))) * (int64_t)kSlot;
    const int tlc = min(tl, t_end - 1 - t0);
    load_tile(x, base + tlc * kSlot, gq, scale_kind);
  };
  auto fetch = [&](Tile& x, int k) {
    const int kc = min(k, nt - 1);
    fetch_pid(x, kc, __builtin_amdgcn_readfirstlane(L.pid[kc]));
  };
  // The first unit's tiles, with page ids read directly (a wave with no
  // unit loads the last tile and never uses it).
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
  if (threadIdx.x == 0) L.next_unit = 2 * kQWaves;

  // Query row `wave` -> rotated, scaled int8 planes (B operand).  Q4_0 has
  // no sign pattern.
  {
    const int r = wave;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = a.q_f16 ? h2f((uint16_t)qw[e]) : __uint_as_float(qw[e]);
      x[e] = live_q ? v : 0.0f;
    }
    fwht_strided<4>(x, k_block, k_norm);
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
      L.qB[d >> 5][r][d & 31] = (int8_t)hi;
      L.qB[d >> 5][8 + r][d & 31] = (int8_t)lo;
    }
    if (lane == 0) L.qsc[r] = (qmax / kQMax) * a.q_scale * 0.0625f;
  }
  const int n = lane & 15;   // score column (row r = n & 7, plane = n >> 3)
  const int g = lane >> 4;   // lane group: tokens 4g..4g+3 of a tile in the score layout
  const int row = n & 7;
  int klen_row = 0;
  if (row < a.rows) {
    const int jr = row / a.group;
#pragma unroll
    for (int j = 0; j < kRows; ++j) klen_row = j == jr ? kl[j] : klen_row;
  }
  __syncthreads();

  const float qs = L.qsc[row];
  // The query's B operand of every block, held in registers for the whole stream.
  long qreg[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) qreg[b] = *(const long*)&L.qB[b][n][8 * g];
  const float w_own = n < 8 ? 256.0f * qs : qs;
  const float w_partner = n < 8 ? qs : 256.0f * qs;
  const bool live_row = row < a.rows;  // lanes n and n + 8 carry the same row
  const float alpha_a = live_row ? (n < 8 ? 1.0f : 4096.0f) : 0.0f;
  const float beta_a = live_row ? (n < 8 ? 0.0f : -4096.0f) : 0.0f;
  const uint32_t vsel = (uint32_t)(n & 3) | (0x0Cu << 8) | ((uint32_t)(4 + (n & 3)) << 16) |
                        (0x0Cu << 24);
  // Nibble masks kept in VGPRs so that mask-and-bias fuses into v_and_or_b32.
  uint32_t m0f, mf0;
  asm volatile("v_mov_b32 %0, 0x0f0f0f0f" : "=v"(m0f));
  asm volatile("v_mov_b32 %0, 0xf0f0f0f0" : "=v"(mf0));
  const int t_lim = min(t_end, kmin);  // tiles ending at or before this need no mask

  float4_t o[kNB][2];
#pragma unroll
  for (int b = 0; b < kNB; ++b) o[b][0] = o[b][1] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  if (has_work) {

    // Scores of one tile (raw: before masking) from its registers, in two
    // halves (blocks 0-3, then 4-7); its V words and scales go to LDS buffer
    // `buf` for the P.V of the unit.
    struct SState {
      uint32_t kw[8];
      float acc[4];
    };
    auto stage_s0 = [&](const Tile& x, int half, int buf, SState& st) {
      uint32_t* kd = &L.u.s.kt[wave][half][tl][gq];
      kd[0] = x.k0.x;
      kd[8] = x.k0.y;
      kd[16] = x.k0.z;
      kd[24] = x.k0.w;
      kd[4] = x.k1.x;
      kd[12] = x.k1.y;
      kd[20] = x.k1.z;
      kd[28] = x.k1.w;
      uint32_t* vw = &L.u.s.vt[wave][buf][half][0][0][tl];
      vw[(gq * 4 + 0) * kVStride] = x.v0.x;
      vw[(gq * 4 + 1) * kVStride] = x.v0.y;
      vw[(gq * 4 + 2) * kVStride] = x.v0.z;
      vw[(gq * 4 + 3) * kVStride] = x.v0.w;
      vw[((4 + gq) * 4 + 0) * kVStride] = x.v1.x;
      vw[((4 + gq) * 4 + 1) * kVStride] = x.v1.y;
      vw[((4 + gq) * 4 + 2) * kVStride] = x.v1.z;
      vw[((4 + gq) * 4 + 3) * kVStride] = x.v1.w;
      {  // lanes 32-63 hold copies of lanes 0-31's chunks: they store to dummy rows
        uint16_t* sw = lane < 32 ? &L.u.s.sh[wave][buf][scale_kind][0][tl >> 2][half][tl & 3]
                                 : &L.u.s.sh_dup[wave][0][lane - 32];
        constexpr int sb = 4 * 2 * 4;  // halves per block, real and dummy rows alike
        sw[0 * sb] = (uint16_t)x.sc.x;
        sw[1 * sb] = (uint16_t)(x.sc.x >> 16);
        sw[2 * sb] = (uint16_t)x.sc.y;
        sw[3 * sb] = (uint16_t)(x.sc.y >> 16);
        sw[4 * sb] = (uint16_t)x.sc.z;
        sw[5 * sb] = (uint16_t)(x.sc.z >> 16);
        sw[6 * sb] = (uint16_t)x.sc.w;
        sw[7 * sb] = (uint16_t)(x.sc.w >> 16);
      }
      wave_sync_lds();
      // Word g of every block of token n: the A operand of 8 score MFMAs.
      const uint4 ka = lds_u4(&L.u.s.kt[wave][half][n][8 * g]);
      const uint4 kb = lds_u4(&L.u.s.kt[wave][half][n][8 * g + 4]);
      st.kw[0] = ka.x;
      st.kw[1] = ka.y;
      st.kw[2] = ka.z;
      st.kw[3] = ka.w;
      st.kw[4] = kb.x;
      st.kw[5] = kb.y;
      st.kw[6] = kb.z;
      st.kw[7] = kb.w;
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[i] = 0.0f;
    };
    auto stage_s_blocks = [&](int half, int buf, int bp0, SState& st) {
      const int4_t zero4 = {0, 0, 0, 0};
#pragma unroll
      for (int bp = bp0; bp < bp0 + 2; ++bp) {
        // K scales of blocks 2bp, 2bp + 1 for tokens 4g..4g+3 of this tile.
        const uint2 ks[2] = {*(const uint2*)&L.u.s.sh[wave][buf][0][2 * bp][g][half][0],
                             *(const uint2*)&L.u.s.sh[wave][buf][0][2 * bp + 1][g][half][0]};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int b = 2 * bp + h;
          // A code c in the high nibble of a byte with bit 7 flipped reads as
          // the int8 16 (c - 8).  Low nibbles are dims 0..3, high 4..7.
          const uint32_t w = st.kw[b];
          const int2_t A2 = {(int)(((w << 4) & mf0) ^ 0x80808080u), (int)((w & mf0) ^ 0x80808080u)};
          const int4_t C = __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, A2),
                                                                 qreg[b], zero4, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t w = i < 2 ? ks[h].x : ks[h].y;
            st.acc[i] = fmaf((float)C[i], (i & 1) ? f16hi(w) : f16lo(w), st.acc[i]);
          }
        }
      }
    };
    // Lane n < 8 holds the hi plane and lane n + 8 the lo plane of a row:
    // both form qs (256 hi + lo) from their own value and the partner's.
    auto stage_s_join = [&](const SState& st, float (&sc)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = fmaf(st.acc[i], w_own, ror8(st.acc[i]) * w_partner);
    };
    auto stage_s = [&](const Tile& x, int half, int buf, float (&sc)[4]) {
      SState st;
      stage_s0(x, half, buf, st);
      stage_s_blocks(half, buf, 0, st);
      stage_s_blocks(half, buf, 2, st);
      stage_s_join(st, sc);
    };

    // Softmax of unit u (tiles 2u, 2u + 1): mask, running max, p, and the
    // P.V A operand (k = 8 g + j: j < 4 tile 2u token 4g+j, else tile 2u+1).
    auto stage_m = [&](const float (&sa)[4], const float (&sb)[4], int u, half8_t& A) {
      float s[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = sa[i];
        s[4 + i] = sb[i];
      }
      const int t0a = t_begin + 2 * kT * u;
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
      // Online softmax in the exp2 domain.  The running maximum is raised
      // only when a unit exceeds it by more than kLazy, so p <= 2^kLazy and
      // the rescale of the accumulators is rare.
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
      // Rows 0-7 of A carry fp16(p), rows 8-15 fp16((p - fp16(p)) * 2^12):
      // a lane-dependent multiply-add gives either from the same operations
      // (and zero for the padding rows past the group).
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[i] - m_ref);  // exp2(-inf) = 0
        l_run += p;
        const _Float16 h = (_Float16)p;
        A[i] = (_Float16)fmaf((float)h, beta_a, p * alpha_a);
      }
    };

    // P.V of a unit from LDS buffer `buf`, block pairs [bp0, bp0 + nbp).
    auto stage_p = [&](const half8_t& A, int buf, int bp0, int nbp) {
      const half8_t c1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f, (_Float16)-1032.0f,
                             (_Float16)-1032.0f, (_Float16)-1032.0f, (_Float16)-1032.0f,
                             (_Float16)-1032.0f, (_Float16)-1032.0f};
      const half8_t c16 = {(_Float16)0.0625f, (_Float16)0.0625f, (_Float16)0.0625f,
                           (_Float16)0.0625f, (_Float16)0.0625f, (_Float16)0.0625f,
                           (_Float16)0.0625f, (_Float16)0.0625f};
      const half8_t c72 = {(_Float16)-72.0f, (_Float16)-72.0f, (_Float16)-72.0f,
                           (_Float16)-72.0f, (_Float16)-72.0f, (_Float16)-72.0f,
                           (_Float16)-72.0f, (_Float16)-72.0f};
      // Per-lane bases: tile 0 of the unit; tile 1 and the blocks are constant offsets.
      const uint32_t* vbase = &L.u.s.vt[wave][buf][0][0][n >> 2][4 * g];
      const uint16_t* sbase = &L.u.s.sh[wave][buf][1][0][g][0][0];
      constexpr int kShBlock = 4 * 2 * 4;          // sh: halves per block
      constexpr int kVtTile = kNB * 4 * kVStride;  // vt: dwords per tile
#pragma unroll
      for (int bp = bp0; bp < bp0 + nbp; ++bp) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int b = 2 * bp + h;
          const uint4 W0 = lds_u4(vbase + b * 4 * kVStride);
          const uint4 W1 = lds_u4(vbase + b * 4 * kVStride + kVtTile);
          // Byte (n & 3) of the V word of tokens t0..t3 -> halves (t0, t1), (t2, t3).
          const uint32_t x0 = __builtin_amdgcn_perm(W0.y, W0.x, vsel);
          const uint32_t x1 = __builtin_amdgcn_perm(W0.w, W0.z, vsel);
          const uint32_t x2 = __builtin_amdgcn_perm(W1.y, W1.x, vsel);
          const uint32_t x3 = __builtin_amdgcn_perm(W1.w, W1.z, vsel);
          const uint4 lw = {(x0 & m0f) | 0x64006400u, (x1 & m0f) | 0x64006400u,
                            (x2 & m0f) | 0x64006400u, (x3 & m0f) | 0x64006400u};
          const uint4 hw = {(x0 & mf0) | 0x64006400u, (x1 & mf0) | 0x64006400u,
                            (x2 & mf0) | 0x64006400u, (x3 & mf0) | 0x64006400u};
          const half8_t lo = __builtin_bit_cast(half8_t, lw) + c1032;
          const half8_t hi = __builtin_elementwise_fma(__builtin_bit_cast(half8_t, hw), c16, c72);
          // V scales of block b for tokens 4g..4g+3 of both tiles, in the k order
          // of the A operand.
          const half8_t dv = __builtin_bit_cast(
              half8_t, lds_u4((const uint32_t*)(sbase + (2 * bp + h) * kShBlock)));
          const half8_t loh = lo * dv, hih = hi * dv;
          const half8_t lol = __builtin_elementwise_fma(lo, dv, -loh);
          const half8_t hil = __builtin_elementwise_fma(hi, dv, -hih);
          o[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, loh, o[b][0], 0, 0, 0);
          o[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, lol, o[b][0], 0, 0, 0);
          o[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, hih, o[b][1], 0, 0, 0);
          o[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, hil, o[b][1], 0, 0, 0);
        }
      }
    };

    float sa[4], sb[4];
    int u_cur = wave, u_nxt = wave + kQWaves;
    stage_s(ta, 0, 0, sa);
    fetch(ta, 2 * u_nxt);
    stage_s(tb, 1, 0, sb);
    fetch(tb, 2 * u_nxt + 1);
    int buf = 0;
    half8_t A;
    while (u_nxt < nu) {
      int u_nn = 0;
      if (lane == 0) u_nn = atomicAdd(&L.next_unit, 1);
      u_nn = __builtin_amdgcn_readfirstlane(u_nn);
      stage_m(sa, sb, u_cur, A);
      // One basic block: P.V of unit u_cur and the scores of unit u_nxt in
      // eight groups; the matrix-core work issued at the end of a group runs
      // while the next group's VALU work issues, and the groups bound how
      // much the scheduler holds in registers at once.
      const int sbuf = buf ^ 1;
      SState st;
      stage_p(A, buf, 0, 1);
      __builtin_amdgcn_sched_barrier(0);
      stage_s0(ta, 0, sbuf, st);
      stage_s_blocks(0, sbuf, 0, st);
      __builtin_amdgcn_sched_barrier(0);
      stage_p(A, buf, 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      stage_s_blocks(0, sbuf, 2, st);
      stage_s_join(st, sa);
      fetch(ta, 2 * u_nn);
      __builtin_amdgcn_sched_barrier(0);
      stage_p(A, buf, 2, 1);
      __builtin_amdgcn_sched_barrier(0);
      stage_s0(tb, 1, sbuf, st);
      stage_s_blocks(1, sbuf, 0, st);
      __builtin_amdgcn_sched_barrier(0);
      stage_p(A, buf, 3, 1);
      __builtin_amdgcn_sched_barrier(0);
      stage_s_blocks(1, sbuf, 2, st);
      stage_s_join(st, sb);
      fetch(tb, 2 * u_nn + 1);
      // Keep these loads here: moved into the next iteration's head they
      // collide with the accumulators' registers and force copies of them.
      __builtin_amdgcn_sched_barrier(0);
      u_cur = u_nxt;
      u_nxt = u_nn;
      buf = sbuf;
    }
    stage_m(sa, sb, u_cur, A);
    stage_p(A, buf, 0, kNB / 2);
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
        const int d = 32 * b + 8 * (n >> 2) + (n & 3) + 4 * m;
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

bool q4_mfma_supported(const DevFmt& f, int rows) {
  const bool pow2 = (f.page_size & (f.page_size - 1)) == 0;
  return f.kind == HKV_KIND_Q4_0 && !f.use_signs && f.D == kD && rows <= kRows &&
         f.page_size % kT == 0 && pow2;
}

hipError_t launch_decode_q4_mfma(const DevFmt& f, const DecArgs& a, dim3 grid, hipStream_t s) {
  // The page ids of a split's tiles are held in LDS.
  if ((a.tokens_per_split + kT - 1) / kT > kMaxSplitTiles) return hipErrorInvalidValue;
  decode_q4_mfma_kernel<<<grid, dim3(kQWaves * kWave), 0, s>>>(f, a);
  return hipGetLastError();
}

}  // namespace hkv
