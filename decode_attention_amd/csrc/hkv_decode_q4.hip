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
//  * Loads.  A unit is nine 16-byte nontemporal loads per lane.  Load r reads
//    the 128-byte line r of each of the unit's eight 4-token quads (a quad is
//    4 x 288 = 1152 bytes, nine whole lines): every load instruction covers
//    whole cache lines, which the nontemporal hint needs (a line split
//    between two instructions is fetched twice).  Each 16-byte chunk is one
//    Q4_0 block of K or V codes of one token, or a token's eight K or eight V
//    scales.
//  * LDS planes.  Word w of every chunk goes to plane w, so each chunk is four
//    32-bit stores at one per-lane address plus fixed offsets.  Per plane and
//    buffer: K [token][block] (two 4-block halves swapped for tokens with bit
//    2 xor bit 3 set, so that the 16-byte K reads are free of bank
//    conflicts), V [block][token], K scale pairs [token] and V scale pairs
//    [token]; the V scales are then regrouped in place into [block][token
//    group][tile][4] halves, the order of the P.V operand.
//  * Scores, S^T = K Q^T on v_mfma_f32_16x16x32_f16 per tile and Q4_0 block:
//    A = the codes as exact fp16 (c - 8) of 16 tokens x 32 dims, B = the
//    rotated query as fp16 leading part and fp16 residual x 2^11 (16 columns
//    = 8 rows x 2 parts), after scaling each row by a power of two that puts
//    its largest value in [2^14, 2^15).  That keeps ~22 significant bits of
//    every query value whatever its magnitude.  Each block's result is scaled
//    by the token's fp16 block scale in fp32.
//  * The score MFMA's row i is token 4 (i % 4) + i / 4 of the tile (the LDS
//    regions store tokens in that order), so each lane ends up holding the
//    tokens g, g + 4, g + 8, g + 12 of one row per tile, and the 8 scores of a
//    unit are exactly the A operand of v_mfma_f32_16x16x32_f16 for P.V (k =
//    8 g + j), so P needs no transpose.  A rows 0-7 carry fp16(p),
//    rows 8-15 the residual x 2^12; B carries (c - 8) * v_scale split exactly
//    into an fp16 high part and the fp16 residual (a 4-bit integer times an
//    11-bit mantissa has <= 15 bits), regrouped with v_perm_b32 and made exact
//    fp16 with the 0x6400 bias trick.
//  * The loop body is {P.V of unit u; scores of unit u + 1} with no branch in
//    between, so the matrix cores and the VALU work of two units overlap.
//  * Online softmax in the exp2 domain, rescaling only when a row maximum
//    grows by more than kLazy; the eight waves merge in LDS and write one
//    partial record per row; the shared merge kernel combines the splits and
//    rotates the output back.
#include "hkv_decode_common.h"

namespace hkv {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 256;        // head size handled here
constexpr int kNB = kD / 32;   // Q4_0 blocks per head vector
constexpr int kRows = 8;       // query rows per KV head
constexpr int kT = 16;         // tokens per tile
constexpr int kSlot = kD + kD / 8;  // Q4_0 slot bytes at head size 256
constexpr int kQuadBytes = 4 * kSlot;  // 1152: nine 128-byte lines
constexpr int kLoads = 9;      // 16-byte loads per lane per unit
constexpr float kLazy = 8.0f;  // log2 headroom before the running max is raised
constexpr int kQWaves = 8;     // waves per workgroup (two per SIMD)
constexpr int kMaxSplitTiles = 256;  // page ids of a split's tiles held in LDS
static_assert(kMaxSplitTiles <= kQWaves * kWave, "one page id per thread");
static_assert(kLoads * 16 * kWave == 2 * kT * kSlot, "a unit is nine loads per lane");

// Words of one plane and buffer.  Tokens are stored in the order v(t) =
// 16 (t / 16) + pi(t % 16), pi(u) = 4 (u % 4) + u / 4, the order in which
// the score rows come out of the matrix cores (see below).
constexpr int kOffK = 0;       // [32 tokens v][8 blocks]
constexpr int kOffV = 256;     // [8 blocks][kVB words: 32 tokens v]
constexpr int kVB = 36;        // V block stride: stores and reads free of bank conflicts
constexpr int kOffSK = 540;    // [32 tokens v]: K scales of blocks (2w, 2w + 1) in plane w
constexpr int kOffSV = 580;    // [32 tokens v] V scale pairs, then [2][32] halves
constexpr int kBufW = 612;
constexpr int kPlaneW = 2 * kBufW + 8;   // 1232 = 16 mod 64: the four planes' banks differ
static_assert(kOffV + 7 * kVB + 32 <= kOffSK && kOffSV + 32 <= kBufW, "plane regions");

struct __align__(16) Q4Lds {
  float qsc[kRows];          // per-row factor of the leading part: q_scale / row scale
  float mlw[kQWaves][kRows][2];
  int pid[kMaxSplitTiles];   // page of each tile of the split
  int next_unit;             // work queue: the next unit no wave has taken
  int pad_[3];
  union {
    _Float16 qB[kNB][16][32];  // query B operand [block][column][k], prologue only
    uint32_t plane[kQWaves][4][kPlaneW];
    float ob[kQWaves][kRows][kD];  // wave merge, after the stream
  } u;
};

__device__ __forceinline__ float f16lo(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16hi(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

// Half-swap of the K words at position v (bit 2 xor bit 3).
__device__ __forceinline__ int kswz(int v) { return ((v >> 2) ^ (v >> 3)) & 1; }

// Storage position of token t (0..31) of a unit: the MFMA row order.
__device__ __forceinline__ int tok_pos(int t) {
  return (t & 16) | ((t & 3) << 2) | ((t >> 2) & 3);
}

// Word offset (in plane 0 of buffer 0) of the chunk that load r brings to
// this lane: lane = 8 G + l8 reads chunk 8 r + l8 of quad G (tokens 4G ..
// 4G + 3 of the unit; G < 4 is tile 0, G >= 4 tile 1).
__device__ __forceinline__ uint32_t chunk_word(int r, int lane) {
  const int cq = 8 * r + (lane & 7);
  const int tq = cq / 18, j = cq - 18 * tq;
  const int v = tok_pos(4 * (lane >> 3) + tq);
  if (j < 8) return kOffK + 8 * v + (j ^ (kswz(v) << 2));
  if (j < 16) return kOffV + kVB * (j - 8) + v;
  return (j == 16 ? kOffSK : kOffSV) + v;
}

// Position of the V scale stored at v in the [token group][tile][4] order of
// the P.V operand.
__device__ __forceinline__ int vs_pos(int v) { return ((v >> 2) & 3) * 8 + (v >> 4) * 4 + (v & 3); }

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
  //     this wave's first two (scalar); (3) the first unit's loads.  Every
  //     load of the prologue is unconditional (clamped indices), so no wait
  //     in between covers the later loads.  Rows past the group load row 0
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
  const bool empty = t_begin >= t_end || req < 0;  // (req < 0 never holds for a valid map)

  if (!empty) {
    // The split is a queue of units of two consecutive 16-token tiles.  Wave w
    // starts with units w and w + 8 and then takes the next untaken unit.
    const int32_t* bt = a.block_table + (int64_t)req * a.max_pages;
    const int ps = page_size;                   // a power of two, multiple of kT
    const int ps_shift = 31 - __builtin_clz(ps);
    const int nt = (t_end - t_begin + kT - 1) / kT;  // tiles in the split
    const int nu = (nt + 1) >> 1;                     // units in the split
    const int tpid = min((int)threadIdx.x, nt - 1);
    const int pidv = bt[(t_begin + kT * tpid) >> ps_shift];
    __builtin_amdgcn_sched_barrier(0);
    // This lane's part of a unit: tile lane / 32, quad (lane / 8) % 4, 16
    // bytes at 16 (lane % 8) of every line.
    const int lane_off = ((lane >> 3) & 3) * kQuadBytes + 16 * (lane & 7);
    const bool tile_b = lane >= 32;
    auto tile_base = [&](int k, int page) -> int64_t {
      const int t0 = t_begin + kT * k;
      return ((((int64_t)page * a.num_kv_heads + kvh) << ps_shift) + (t0 & (ps - 1))) *
             (int64_t)kSlot;
    };
    u32x4 ld[kLoads];
    auto load_unit_pages = [&](int u, int pa, int pb) {
      const int ka = min(2 * u, nt - 1), kb = min(2 * u + 1, nt - 1);
      const int64_t off = tile_b ? tile_base(kb, pb) : tile_base(ka, pa);
      const u32x4* src = (const u32x4*)(a.cache + off + lane_off);
#pragma unroll
      for (int r = 0; r < kLoads; ++r) ld[r] = __builtin_nontemporal_load(src + 8 * r);
    };
    auto load_unit = [&](int u) {
      const int ka = min(2 * u, nt - 1), kb = min(2 * u + 1, nt - 1);
      load_unit_pages(u, __builtin_amdgcn_readfirstlane(L.pid[ka]),
                      __builtin_amdgcn_readfirstlane(L.pid[kb]));
    };
    // The first unit's loads, with page ids read directly (a wave with no
    // unit loads the last tile and never uses it).
    const bool has_work = wave < nu;
    {
      const int u = min(wave, nu - 1);
      const int ka = min(2 * u, nt - 1), kb = min(2 * u + 1, nt - 1);
      load_unit_pages(u, bt[(t_begin + kT * ka) >> ps_shift], bt[(t_begin + kT * kb) >> ps_shift]);
    }
    __builtin_amdgcn_sched_barrier(0);
    L.pid[tpid] = pidv;
    if (threadIdx.x == 0) L.next_unit = 2 * kQWaves;

    // Query row `wave`, rotated, as the fp16 B operand: the row is scaled by
    // 2^k so that its largest value lies in [2^14, 2^15); the leading part
    // goes to column `wave`, the residual x 2^11 to column 8 + wave.  Dim d
    // of block b sits at k = 8 g + i with g = (d / 8) % 4 and, for j = d % 8,
    // i = j / 2 + 4 (j % 2) (the order in which the code words unpack).
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
      const float s = qmax > 0.0f ? ldexpf(1.0f, 14 - ilogbf(qmax)) : 1.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y = x[e] * s;
        const _Float16 hi = (_Float16)y;
        const _Float16 lo = (_Float16)((y - (float)hi) * 2048.0f);
        const int d = kWave * e + lane;
        const int j = d & 7;
        const int k = 8 * ((d >> 3) & 3) + (j >> 1) + 4 * (j & 1);
        L.u.qB[d >> 5][r][k] = hi;
        L.u.qB[d >> 5][8 + r][k] = lo;
      }
      if (lane == 0) L.qsc[r] = qmax > 0.0f ? a.q_scale / s : 0.0f;
    }
    // Store addresses of this lane's nine chunks, in bytes (plane 0, buffer 0).
    uint32_t* planes = &L.u.plane[wave][0][0];
    uint32_t wbase[kLoads];
#pragma unroll
    for (int r = 0; r < kLoads; ++r) wbase[r] = 4u * chunk_word(r, lane);
    // V-scale regrouping: lane reads plane lane / 16, tokens 2 (lane % 16) + {0, 1}.
    const int vs_plane = lane >> 4, vs_v = 2 * (lane & 15);
    const int vs_rd = vs_plane * kPlaneW + kOffSV + vs_v;                // words
    const int vs_wr = 2 * (vs_plane * kPlaneW + kOffSV) + vs_pos(vs_v);  // halves (even)
    // the unit tokens stored at positions vs_v and vs_v + 1 (tok_pos is an involution)
    const int vs_t0 = tok_pos(vs_v), vs_t1 = tok_pos(vs_v + 1);

    const int n = lane & 15;   // score column (row r = n & 7, part = n >> 3)
    const int g = lane >> 4;   // lane group: tokens 4g..4g+3 of a tile in the score layout
    const int row = n & 7;
    int klen_row = 0;
    if (row < a.rows) {
      const int jr = row / a.group;
#pragma unroll
      for (int j = 0; j < kRows; ++j) klen_row = j == jr ? kl[j] : klen_row;
    }
    __syncthreads();

    // The query's B operand of every block, held in registers for the whole
    // stream (the planes reuse its LDS once every wave has read it).
    half8_t qb[kNB];
#pragma unroll
    for (int b = 0; b < kNB; ++b) qb[b] = *(const half8_t*)&L.u.qB[b][n][8 * g];
    const float qs = L.qsc[row];
    __syncthreads();
    const float w_own = n < 8 ? qs : qs * (1.0f / 2048.0f);
    const float w_partner = n < 8 ? qs * (1.0f / 2048.0f) : qs;
    const bool live_row = row < a.rows;  // lanes n and n + 8 carry the same row
    const float alpha_a = live_row ? (n < 8 ? 1.0f : 4096.0f) : 0.0f;
    const float beta_a = live_row ? (n < 8 ? 0.0f : -4096.0f) : 0.0f;
    const uint32_t vsel = (uint32_t)(n & 3) | (0x0Cu << 8) | ((uint32_t)(4 + (n & 3)) << 16) |
                          (0x0Cu << 24);
    // Nibble masks kept in VGPRs so that mask-and-bias fuses into v_and_or_b32.
    uint32_t m0f, mf0, m000f, m00f0;
    asm volatile("v_mov_b32 %0, 0x0f0f0f0f" : "=v"(m0f));
    asm volatile("v_mov_b32 %0, 0xf0f0f0f0" : "=v"(mf0));
    asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(m000f));
    asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(m00f0));
    const int t_lim = min(t_end, kmin);  // units ending at or before this need no mask

    float4_t o[kNB][2];
#pragma unroll
    for (int b = 0; b < kNB; ++b) o[b][0] = o[b][1] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    if (has_work) {
      // Unit u's nine chunks from the load registers into buffer buf, then its
      // V scales regrouped into halves.  Scale words of tokens past the
      // split's end (a partial last tile, or a tile past the last one that
      // was loaded in its place) are zeroed, so that their codes, masked out
      // of the softmax, add nothing to P.V.
      auto store_unit = [&](int u, int buf) {
        uint8_t* pb = (uint8_t*)planes + 4 * kBufW * buf;
#pragma unroll
        for (int r = 0; r < kLoads; ++r) {
          uint32_t* p = (uint32_t*)(pb + wbase[r]);
          p[0] = ld[r].x;
          p[kPlaneW] = ld[r].y;
          p[2 * kPlaneW] = ld[r].z;
          p[3 * kPlaneW] = ld[r].w;
        }
        wave_sync_lds();
        const int nvalid = t_end - (t_begin + 2 * kT * u);
        uint2 sv = *(const uint2*)(planes + kBufW * buf + vs_rd);
        sv.x = vs_t0 < nvalid ? sv.x : 0u;
        sv.y = vs_t1 < nvalid ? sv.y : 0u;
        wave_sync_lds();
        uint32_t* hw = (uint32_t*)((_Float16*)(planes + kBufW * buf) + vs_wr);
        hw[0] = __builtin_amdgcn_perm(sv.y, sv.x, 0x05040100u);   // block 2p: low halves
        hw[16] = __builtin_amdgcn_perm(sv.y, sv.x, 0x07060302u);  // block 2p + 1: high halves
      };

      // Scores of tile h of the unit in buffer buf (raw: before masking),
      // blocks [b0, b0 + 4).
      struct SState {
        uint32_t kw[8];
        u32x4 ks[4];
        float acc[4];
      };
      auto stage_s0 = [&](int h, int buf, SState& st) {
        const int t = kT * h + n;
        const uint32_t* kp = planes + (size_t)g * kPlaneW + kBufW * buf + kOffK + 8 * t;
        const int sw = kswz(t) << 2;
        const uint4 ka = lds_u4(kp + sw);
        const uint4 kb = lds_u4(kp + (sw ^ 4));
        st.kw[0] = ka.x;
        st.kw[1] = ka.y;
        st.kw[2] = ka.z;
        st.kw[3] = ka.w;
        st.kw[4] = kb.x;
        st.kw[5] = kb.y;
        st.kw[6] = kb.z;
        st.kw[7] = kb.w;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint4 v = lds_u4(planes + (size_t)p * kPlaneW + kBufW * buf + kOffSK + kT * h + 4 * g);
          st.ks[p] = (u32x4){v.x, v.y, v.z, v.w};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) st.acc[i] = 0.0f;
      };
      auto stage_s_blocks = [&](int b0, SState& st) {
        const half2_t c1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
        const half2_t c16 = {(_Float16)0.0625f, (_Float16)0.0625f};
        const half2_t c72 = {(_Float16)-72.0f, (_Float16)-72.0f};
        const float4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int b = b0; b < b0 + 4; ++b) {
          // The codes of dims (0, 2) and (1, 3) of the lane's word, masked
          // into the low mantissa bits of fp16 1024, read 1024 + c; those of
          // dims (4, 6) and (5, 7), masked in place, read 1024 + 16 c.  Both
          // become the exact c - 8.
          const uint32_t w = st.kw[b], w8 = w >> 8;
          const half2_t h0 = __builtin_bit_cast(half2_t, (w & m000f) | 0x64006400u) + c1032;
          const half2_t h1 = __builtin_elementwise_fma(
              __builtin_bit_cast(half2_t, (w & m00f0) | 0x64006400u), c16, c72);
          const half2_t h2 = __builtin_bit_cast(half2_t, (w8 & m000f) | 0x64006400u) + c1032;
          const half2_t h3 = __builtin_elementwise_fma(
              __builtin_bit_cast(half2_t, (w8 & m00f0) | 0x64006400u), c16, c72);
          const half8_t A = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
          const float4_t C = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb[b], zero4, 0, 0, 0);
          const u32x4 ks = st.ks[b >> 1];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            st.acc[i] = fmaf(C[i], (b & 1) ? f16hi(ks[i]) : f16lo(ks[i]), st.acc[i]);
        }
      };
      // Lane n < 8 holds the leading part and lane n + 8 the residual of a
      // row: both form q_scale / s (lead + res / 2^11) from their own value
      // and the partner's, and lane n + 8 keeps lane n's result.
      auto stage_s_join = [&](const SState& st, float (&sc)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[i] = pair_score(fmaf(st.acc[i], w_own, ror8(st.acc[i]) * w_partner), n);
      };
      auto stage_s = [&](int h, int buf, float (&sc)[4]) {
        SState st;
        stage_s0(h, buf, st);
        stage_s_blocks(0, st);
        stage_s_blocks(4, st);
        stage_s_join(st, sc);
      };

      // Softmax of unit u (tiles 2u, 2u + 1): mask, running max, p, and the
      // P.V A operand (k = 8 g + j: j < 4 tile 2u token 4j+g, else tile 2u+1).
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
            const int ta_ = t0a + 4 * i + g, tb_ = t0b + 4 * i + g;
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

      // P.V of the unit in buffer buf, block pairs [bp0, bp0 + nbp).
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
        // V word n / 4 of a block, tokens 4g..4g+3 of tile 0 (+16: tile 1).
        const uint32_t* vbase = planes + (size_t)(n >> 2) * kPlaneW + kBufW * buf + kOffV + 4 * g;
#pragma unroll
        for (int bp = bp0; bp < bp0 + nbp; ++bp) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int b = 2 * bp + h;
            const uint4 W0 = lds_u4(vbase + kVB * b);
            const uint4 W1 = lds_u4(vbase + kVB * b + kT);
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
                half8_t, lds_u4(planes + (size_t)bp * kPlaneW + kBufW * buf + kOffSV + 16 * h +
                                4 * g));
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
      store_unit(u_cur, 0);
      load_unit(u_nxt);
      stage_s(0, 0, sa);
      stage_s(1, 0, sb);
      int buf = 0;
      half8_t A;
      while (u_nxt < nu) {
        int u_nn = u_nxt + kQWaves;  // deterministic mode: a fixed order
        if (!a.det) {
          if (lane == 0) u_nn = atomicAdd(&L.next_unit, 1);
          u_nn = __builtin_amdgcn_readfirstlane(u_nn);
        }
        stage_m(sa, sb, u_cur, A);
        const int sbuf = buf ^ 1;
        store_unit(u_nxt, sbuf);
        load_unit(u_nn);
        // One basic block: P.V of unit u_cur and the scores of unit u_nxt in
        // eight groups; the matrix-core work issued at the end of a group runs
        // while the next group's VALU work issues.
        SState st;
        stage_p(A, buf, 0, 1);
        __builtin_amdgcn_sched_barrier(0);
        stage_s0(0, sbuf, st);
        stage_s_blocks(0, st);
        __builtin_amdgcn_sched_barrier(0);
        stage_p(A, buf, 1, 1);
        __builtin_amdgcn_sched_barrier(0);
        stage_s_blocks(4, st);
        stage_s_join(st, sa);
        __builtin_amdgcn_sched_barrier(0);
        stage_p(A, buf, 2, 1);
        __builtin_amdgcn_sched_barrier(0);
        stage_s0(1, sbuf, st);
        stage_s_blocks(0, st);
        __builtin_amdgcn_sched_barrier(0);
        stage_p(A, buf, 3, 1);
        __builtin_amdgcn_sched_barrier(0);
        stage_s_blocks(4, st);
        stage_s_join(st, sb);
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

    // ---- merge the waves ------------------------------------------------
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
  } else {
    for (int r = threadIdx.x; r < a.rows; r += blockDim.x) {
      part[r * a.pstride + 0] = -INFINITY;
      part[r * a.pstride + 1] = 0.0f;
    }
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
