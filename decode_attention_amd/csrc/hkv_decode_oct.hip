// hkv_decode_oct.hip -- split-K paged decode attention over Octave caches on
// the matrix cores (gfx950), 8 or 16 query rows per KV head (and 32 in one
// pass for the compact layout), for four layouts:
//  * k3v4 at head size 128 with 64 RoPE dims: 4-bit K codes for the RoPE
//    block, 3-bit for the NoPE block (one scale each), 4-bit V (128-byte slots);
//  * k3v3 at head size 128 with 64 RoPE dims: the same K, 3-bit V (112-byte
//    slots);
//  * k3v4 at head size 192 with 64 RoPE dims: two 3-bit NoPE blocks, 4-bit V
//    (184-byte slots);
//  * k3v3 compact at head size 256: 3-bit K and V, one scale each (196-byte
//    slots).
//
// What is computed is reference_attention of the vLLM docs page
// "vllm.v1.attention.ops.rocm_octave" in the rotated space the module text
// describes: the query takes the K rotation (sign flips, 64-dim blocks),
// codes are dequantized as LUT[c] * scale / 64 (reference_dequantize), and
// the output is rotated back with the V transform and the signs.
//
// The stream and its driver follow the Q4_0 kernel (8-wave workgroups with a
// queue of 32-token units in LDS; P.V of one unit and the scores of the next
// in one branch-free block); the format-specific parts:
//  * A tile (16 slots) is loaded in 16-byte chunks of one token each and
//    stored in LDS transposed, [slot word][token], so a K operand is words of
//    one token and a V operand is one word of four tokens.
//  * Scores on v_mfma_i32_16x16x64_i8, one per 64-dim scale block: A = the
//    int8 codebook values of the codes (looked up with v_perm_b32; 16-entry
//    tables take two lookups and a per-byte select on the code's top bit),
//    B = the rotated query as three int8 planes (q = 2^16 hi + 2^8 mid + lo
//    per row, ~23 bits of the row's largest value, so the scores keep fp32
//    accuracy at any query magnitude).  8-row mode: B columns [hi | lo] and
//    [mid | 0]; the first product, shifted left 8 bits, accumulates the
//    second, leaving 2^8 hi + mid and 2^8 lo in lanes n and n + 8.  16-row
//    mode: one product per plane, 2^8 hi + mid joined the same way.  Each
//    block's int32 result is scaled by the token's fp16 block scale.
//  * P.V on v_mfma_f32_16x16x32_f16: B = the codebook value as an exact fp16
//    (4-bit: the biased byte LUT[c] + 128 under an 0x64 high byte reads
//    1152 + LUT[c], and one packed subtraction leaves LUT[c]; 3-bit: the low
//    and high bytes of fp16(LUT[c]) looked up from two tables), so no
//    residual is needed on this side.  The values enter unbiased: a bias
//    left in them would grow the accumulators by a factor of ~1152 / |LUT|
//    and cost ~8 bits of the output (relative to the row's largest value)
//    to the accumulators' rounding.  The token's V scale multiplies p
//    in the A operand, fp16(p s) plus its residual x 2^12, in one of two row
//    modes: with 8 query rows the residual takes A rows 8-15 (one MFMA per 32
//    tokens); with 16 rows it takes the other half of the K dimension: a
//    lane's 8 k-slots are its own 4 tokens' fp16(p s) and residuals, against
//    their values and values x 2^-12 in B (exact, and normal since |LUT| >= 6),
//    one MFMA per 16 tokens and no data moved between lanes.
#include "hkv_decode_common.h"

namespace hkv {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __fp16 half2_t __attribute__((ext_vector_type(2)));

// Slot layouts (slot words; vLLM docs, module text and OctaveFormat).
// kCompact: K is one 3-bit block under one scale (else a 4-bit RoPE block and
// kNope 3-bit NoPE blocks of 64 dims, a scale each); kV3: V is 3-bit (two bit
// planes), else 4-bit; the V scale is the half (kVSh) of slot word kWVS.
// kChunks 16-byte chunks are loaded per lane and tile (chunk 4 i + q by lane
// group q), of which the slot holds kNChunk (the last one only 8 bytes when
// kHalfLast).
struct FmtK3V4 {            // octave_k3v4, head size 128, rope 64
  static constexpr bool kCompact = false;
  static constexpr bool kV3 = false;
  static constexpr int kD = 128;
  static constexpr int kSlot = 128;
  static constexpr int kWNope = 8;    // NoPE low-bit plane (byte 32)
  static constexpr int kWNopeHi = 12; // NoPE high-bit plane (byte 48)
  static constexpr int kWV = 14;      // V codes (byte 56)
  static constexpr int kWScale = 30;  // K scales (RoPE | NoPE << 16); word 31: V scale
  static constexpr int kNope = 1;
  static constexpr int kWVS = 31, kVSh = 0;
  static constexpr int kChunks = 2;
  static constexpr int kNChunk = 8;
  static constexpr bool kHalfLast = false;
  static constexpr int kAcc = kD / 32 * 2;  // P.V accumulator tiles
};
struct FmtK3V4W {           // octave_k3v4, head size 192, rope 64
  static constexpr bool kCompact = false;
  static constexpr bool kV3 = false;
  static constexpr int kD = 192;
  static constexpr int kSlot = 184;
  static constexpr int kWNope = 8;    // NoPE low-bit plane, both blocks (byte 32)
  static constexpr int kWNopeHi = 16; // NoPE high-bit plane (byte 64)
  static constexpr int kWV = 20;      // V codes (byte 80)
  static constexpr int kWScale = 44;  // RoPE | NoPE 0 << 16; word 45: NoPE 1 | V << 16
  static constexpr int kNope = 2;
  static constexpr int kWVS = 45, kVSh = 16;
  static constexpr int kChunks = 3;
  static constexpr int kNChunk = 12;
  static constexpr bool kHalfLast = true;  // chunk 11: the two scale words only
  static constexpr int kAcc = kD / 32 * 2;
};
struct FmtK3V3 {            // octave_k3v3, head size 128, rope 64
  static constexpr bool kCompact = false;
  static constexpr bool kV3 = true;
  static constexpr int kD = 128;
  static constexpr int kSlot = 112;
  static constexpr int kWNope = 8;    // NoPE low-bit plane (byte 32)
  static constexpr int kWNopeHi = 12; // NoPE high-bit plane (byte 48)
  static constexpr int kWV = 14;      // V low-bit plane (byte 56)
  static constexpr int kWVHi = 22;    // V high-bit plane (byte 88)
  static constexpr int kWScale = 26;  // K scales (RoPE | NoPE << 16); word 27: V scale
  static constexpr int kNope = 1;
  static constexpr int kWVS = 27, kVSh = 0;
  static constexpr int kChunks = 2;
  static constexpr int kNChunk = 7;   // chunk 7 (lane group 3, second load) is past the slot
  static constexpr bool kHalfLast = false;
  static constexpr int kAcc = kD / 16;
};
struct FmtK3V3C {           // octave_k3v3_compact, head size 256
  static constexpr bool kCompact = true;
  static constexpr bool kV3 = true;
  static constexpr int kD = 256;
  static constexpr int kSlot = 196;
  static constexpr int kWKHi = 16;    // K high-bit plane (byte 64)
  static constexpr int kWV = 24;      // V low-bit plane (byte 96)
  static constexpr int kWVHi = 40;    // V high-bit plane (byte 160)
  static constexpr int kWScale = 48;  // K scale | V scale << 16
  static constexpr int kChunks = 3;   // 12 chunks of 16 bytes per slot: 3 per lane
  static constexpr int kNChunk = 12;  // (+ the scale word, loaded on its own)
  static constexpr bool kHalfLast = false;
  static constexpr int kWVS = 48, kVSh = 16;
  static constexpr int kAcc = kD / 16;
};
constexpr int kRowsMax = 16;       // query rows per KV head (16-row mode)
constexpr int kT = 16;             // tokens per tile
constexpr int kTS = kT + 4;        // token stride (words) of the transposed tile
constexpr int kQMaxI = kQ3MaxI;    // largest |q| code of the three-plane int8 split
constexpr float kQMax = (float)kQ3MaxI;
constexpr float kLazy = 8.0f;      // log2 headroom before the running max is raised
constexpr int kQWaves = 8;         // waves per workgroup (two per SIMD)
constexpr int kQWaves12 = 12;      // three per SIMD (8-row mode at head size 128)
constexpr int kMaxSplitTiles = 256;

// Codebook bytes for v_perm_b32 lookups: entries 4i..4i+3 in word i.
constexpr uint32_t lut_word(const int* lut, int i, int bias) {
  return (uint32_t)((lut[4 * i] + bias) & 255) | ((uint32_t)((lut[4 * i + 1] + bias) & 255) << 8) |
         ((uint32_t)((lut[4 * i + 2] + bias) & 255) << 16) |
         ((uint32_t)((lut[4 * i + 3] + bias) & 255) << 24);
}
constexpr uint32_t kK4[4] = {lut_word(kLut4, 0, 0), lut_word(kLut4, 1, 0), lut_word(kLut4, 2, 0),
                             lut_word(kLut4, 3, 0)};
constexpr uint32_t kK3[2] = {lut_word(kLut3, 0, 0), lut_word(kLut3, 1, 0)};
constexpr uint32_t kV4[4] = {lut_word(kLut4, 0, 128), lut_word(kLut4, 1, 128),
                             lut_word(kLut4, 2, 128), lut_word(kLut4, 3, 128)};

// The 3-bit codebook as fp16 bit patterns, low bytes and high bytes, entries
// 4 i .. 4 i + 3 in word i (one v_perm_b32 lookup each for four codes).
constexpr uint32_t half_bits_int(int v) {  // exact for |v| < 2048
  if (v == 0) return 0u;
  const uint32_t sgn = v < 0 ? 0x8000u : 0u;
  const int m = v < 0 ? -v : v;
  int e = 0;
  while ((m >> (e + 1)) != 0) ++e;
  return sgn | ((uint32_t)(e + 15) << 10) | (((uint32_t)m << (10 - e)) & 0x3ffu);
}
constexpr uint32_t half_byte_word(int i, int byte) {
  uint32_t w = 0;
  for (int k = 0; k < 4; ++k) w |= ((half_bits_int(kLut3[4 * i + k]) >> (8 * byte)) & 255u) << (8 * k);
  return w;
}
constexpr uint32_t kH3Lo[2] = {half_byte_word(0, 0), half_byte_word(1, 0)};
constexpr uint32_t kH3Hi[2] = {half_byte_word(0, 1), half_byte_word(1, 1)};

// fp16 values of the 3-bit codes in the four bytes of sel: the halves of
// codes 0, 1 in .x and of codes 2, 3 in .y.
__device__ __forceinline__ uint2 lut3_half(uint32_t sel, uint32_t hi0, uint32_t hi1) {
  const uint32_t lo = __builtin_amdgcn_perm(kH3Lo[1], kH3Lo[0], sel);
  const uint32_t hi = __builtin_amdgcn_perm(hi1, hi0, sel);
  return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
}
static_assert(half_bits_int(127) == 0x57F0u && half_bits_int(-14) == 0xCB00u, "fp16 bits");

// 0xFF in each byte whose bit 7 is set in y, else 0x00 (v_perm_b32
// sign-replicating selectors 8-11 read bit 7 of bytes 1, 3 of the low and
// high source words).
__device__ __forceinline__ uint32_t byte_sign_mask(uint32_t y) {
  return __builtin_amdgcn_perm(y << 8, y, 0x090B080Au);
}

// 16-entry byte lookup of four codes (one per byte, bits 0-2 in s7, the
// select mask m from bit 3): entries 0-7 in (t0, t1), 8-15 in (t2, t3).
__device__ __forceinline__ uint32_t lut16(uint32_t s7, uint32_t m, uint32_t t0, uint32_t t1,
                                          uint32_t t2, uint32_t t3) {
  const uint32_t lo = __builtin_amdgcn_perm(t1, t0, s7);
  const uint32_t hi = __builtin_amdgcn_perm(t3, t2, s7);
  return (hi & m) | (lo & ~m);
}

// int8 codebook values of the 8 codes in a 4-bit packed word (byte j holds
// codes j (low nibble) and 4 + j (high nibble)): {codes 0-3, codes 4-7}.
__device__ __forceinline__ void k4_word(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = lut16(w & 0x07070707u, byte_sign_mask(w << 4), kK4[0], kK4[1], kK4[2], kK4[3]);
  hi = lut16((w >> 4) & 0x07070707u, byte_sign_mask(w), kK4[0], kK4[1], kK4[2], kK4[3]);
}

// Chunk ci (16 bytes at 16 ci) of a slot: zeros past the slot's end, and
// only 8 bytes for a half last chunk.
template <class F>
__device__ __forceinline__ uint4 load_chunk(const uint8_t* slot, int ci) {
  if (F::kNChunk == 4 * F::kChunks && !F::kHalfLast) return *(const uint4*)(slot + 16 * ci);
  if (ci < F::kNChunk - (F::kHalfLast ? 1 : 0)) return *(const uint4*)(slot + 16 * ci);
  if (F::kHalfLast && ci == F::kNChunk - 1) {
    const uint2 h = *(const uint2*)(slot + 16 * ci);
    return make_uint4(h.x, h.y, 0u, 0u);
  }
  return make_uint4(0u, 0u, 0u, 0u);
}

// Chunks q, q + 4, q + 8 (16 bytes each) of token tl (the first kChunks),
// and for the compact layout the 4-byte scale word.
struct Tile {
  uint4 c[3];
  uint32_t sw;
};

template <class F, int RM, int NW>
struct __align__(16) OctLds {
  static constexpr int kD = F::kD;
  static constexpr int kSlotW = (F::kSlot + 3) / 4 > 16 * F::kChunks ? (F::kSlot + 3) / 4
                                                                      : 16 * F::kChunks;
  // B operand bytes, [64-dim block][column][dim].  8-row mode: columns r
  // (hi), 8 + r (lo), 16 + r (mid) of row r, 24-31 zero; 16-row mode: r (hi),
  // 16 + r (lo), 32 + r (mid).
  static constexpr int kQCols = RM == 8 ? 32 : 48;
  int8_t qB[kD / 64][kQCols][64];
  float qsc[RM];
  float mlw[NW][RM][2];
  int pid[kMaxSplitTiles];
  int next_unit;
  int pad_[3];
  union {
    uint32_t tt[NW][2][2][kSlotW][kTS];  // [buf][tile][slot word][token]
    float ob[NW][RM][kD];
  } u;
};

// NW waves per workgroup: 8 (two per SIMD), or 12 (three per SIMD) where the
// tiles of 12 waves fit the LDS (head size 128) and the kernel fits the 168
// VGPRs that three waves leave.
template <class F, int RM, int NW>
__global__ __launch_bounds__(NW * kWave, 1) void decode_oct_kernel(DevFmt f, DecArgs a) {
  constexpr int kD = F::kD;
  constexpr int kSlot = F::kSlot;
  constexpr int kE = kD / kWave;  // query values per lane
  constexpr int kAcc = F::kAcc;
  constexpr bool kK16 = RM == 16;       // residual of p in the K dimension
  constexpr int kQR = (RM + NW - 1) / NW;  // query rows per wave (rows wave + NW k < RM)
  __shared__ OctLds<F, RM, NW> L;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lane = threadIdx.x & 63;
  static_assert(kMaxSplitTiles <= NW * kWave, "one page id per thread");
  int page_size = f.page_size, k_block = f.k_block;
  float k_norm = f.k_norm;
  pin_args(a, page_size, k_block, k_norm);
  int split, kvh, gi;
  if (!wg_item(a, split, kvh, gi)) return;
  const int q0 = gi * a.n_q;
  // ---- prologue: three memory round trips before the stream -------------
  // (1) query rows wave + 8 k (raw bits), the key lengths of the group's
  //     queries (one per lane, n_q <= RM) and the request; (2) the split's
  //     page ids, to LDS, and this wave's first two (scalar); (3) the first
  //     unit's tiles.  Every load of the prologue is unconditional (clamped
  //     indices), so no wait before the barrier covers a later round trip.
  uint32_t qw[kQR][kE];
#pragma unroll
  for (int k = 0; k < kQR; ++k) query_row_raw<kE>(a, q0, kvh, wave + NW * k, lane, qw[k]);
  uint32_t sw[kE];
  lane_sign_words<kE>(f, f.use_signs, lane, sw);
  const int kl = group_klen_lane(a, q0, lane);
  const int req = a.q_to_req[q0];
  const int kmax = wave_max_int(kl);
  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(t_begin + a.tokens_per_split, kmax);
  float* part = a.ws + (((size_t)gi * a.num_kv_heads + kvh) * a.num_splits + split) * RM *
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
  const int nt = (t_end - t_begin + kT - 1) / kT;
  const int nu = (nt + 1) >> 1;
  // One page id per thread (nt <= kMaxSplitTiles); threads past the last
  // tile load and later store the last one again.
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
    for (int i = 0; i < F::kChunks; ++i) x.c[i] = load_chunk<F>(slot, 4 * i + gq);
    if constexpr (F::kCompact) x.sw = *(const uint32_t*)(slot + 4 * F::kWScale);
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
  if (threadIdx.x == 0) L.next_unit = 2 * NW;
#pragma unroll
  for (int k = 0; k < kQR; ++k) {
    const int r = wave + NW * k;
    if (RM % NW != 0 && r >= RM) break;  // (wave-uniform) waves past the rows
    float x[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) x[e] = flip_sign(query_value(a, qw[k][e], r < a.rows), sw[e], lane);
    fwht_strided<kE>(x, k_block, k_norm);
    float qmax = 0.0f;
#pragma unroll
    for (int e = 0; e < kE; ++e) qmax = fmaxf(qmax, fabsf(x[e]));
    qmax = wave_max(qmax);
    const float inv = qmax > 0.0f ? kQMax / qmax : 0.0f;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      int qi = (int)rintf(x[e] * inv);
      qi = min(kQMaxI, max(-kQMaxI, qi));
      int hi, mid, lo;
      q_split3(qi, hi, mid, lo);
      const int d = kWave * e + lane;
      L.qB[d >> 6][r][d & 63] = (int8_t)hi;
      L.qB[d >> 6][kK16 ? 16 + r : 8 + r][d & 63] = (int8_t)lo;
      L.qB[d >> 6][kK16 ? 32 + r : 16 + r][d & 63] = (int8_t)mid;
      if constexpr (!kK16) L.qB[d >> 6][24 + r][d & 63] = 0;
    }
    // 1/64: the codebook scale (LUT_ONE) of the K values.
    if (lane == 0) L.qsc[r] = (qmax / kQMax) * a.q_scale * (1.0f / 64.0f);
  }
  const int n = lane & 15;
  const int g = lane >> 4;
  // The score row of this lane: 8-row mode row n & 7 (lanes n, n + 8 hold its
  // hi and lo planes), 16-row mode row n.
  const int row = kK16 ? n : (n & 7);
  const int klen_lane_row = __shfl(kl, (row < a.rows ? row : 0) / a.group, kWave);
  const int klen_row = row < a.rows ? klen_lane_row : 0;
  const int kmin = wave_min_int(kl);
  __syncthreads();

  const float qs = L.qsc[row];
  // 8-row mode: lane n < 8 ends with 2^8 hi + mid of row n, lane n + 8 with
  // 2^8 lo (in units of the row's query step).
  const float w_own = n < 8 ? 256.0f * qs : qs * (1.0f / 256.0f);
  const float w_partner = n < 8 ? qs * (1.0f / 256.0f) : 256.0f * qs;
  // B operands of every block: 8-row mode [hi | lo] and [mid | 0] (columns =
  // rows x planes); 16-row mode the hi, lo and mid planes of 16 rows.
  int4_t qreg[kD / 64], qmid[kD / 64], qlo[kK16 ? kD / 64 : 1];
#pragma unroll
  for (int c = 0; c < kD / 64; ++c) {
    qreg[c] = *(const int4_t*)&L.qB[c][n][16 * g];
    qmid[c] = *(const int4_t*)&L.qB[c][(kK16 ? 32 : 16) + n][16 * g];
    if constexpr (kK16) qlo[c] = *(const int4_t*)&L.qB[c][16 + n][16 * g];
  }
  const bool live_row = row < a.rows;
  // Gathers byte (n & 3) of a word of tokens t0..t3 into bytes 0..3.
  const int jb = n & 3;
  const uint32_t gsel_lo = (uint32_t)jb | ((uint32_t)(jb + 4) << 8) | (0x0Cu << 16) | (0x0Cu << 24);
  const uint32_t gsel_hi = 0x0Cu | (0x0Cu << 8) | ((uint32_t)jb << 16) | ((uint32_t)(jb + 4) << 24);
  const int t_lim = min(t_end, kmin);
  // 3-bit segments: code 16 m + 4 i + j has its low bits at bits 2 i of byte
  // j of low-plane word m and its high bit at bit 4 (m & 1) + i of byte j of
  // high-plane word m >> 1 (vLLM docs, _pack).  For the K operand m = 4 c + g.
  const int hsh = 4 * (g & 1);
  // For the V operand of the compact layout lane n takes dim 16 m + n: i = n >> 2.
  const int vi = n >> 2;

  float4_t o[kAcc];
#pragma unroll
  for (int b = 0; b < kAcc; ++b) o[b] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  if (has_work) {
    // Scores of one tile (before masking) from its registers; the tile goes
    // to LDS buffer `buf` for the P.V of the unit.
    auto stage_s = [&](const Tile& x, int half, int buf, float (&sc)[4]) {
      uint32_t* tw = &L.u.tt[wave][buf][half][0][tl];
#pragma unroll
      for (int i = 0; i < F::kChunks; ++i) {
        tw[(16 * i + 4 * gq + 0) * kTS] = x.c[i].x;
        tw[(16 * i + 4 * gq + 1) * kTS] = x.c[i].y;
        tw[(16 * i + 4 * gq + 2) * kTS] = x.c[i].z;
        tw[(16 * i + 4 * gq + 3) * kTS] = x.c[i].w;
      }
      if constexpr (F::kCompact) tw[F::kWScale * kTS] = x.sw;  // lanes of one token store the same word
      wave_sync_lds();
      const uint32_t* tr = &L.u.tt[wave][buf][half][0][0];
      const int4_t zero4 = {0, 0, 0, 0};
      // Scales of tokens 4g..4g+3.
      const uint4 ks = lds_u4(&tr[F::kWScale * kTS + 4 * g]);
      const uint32_t ksw[4] = {ks.x, ks.y, ks.z, ks.w};
      if constexpr (!F::kCompact) {
        // K scale of block c (RoPE, NoPE 0, NoPE 1) for token 4 g + i
        uint32_t ksw2[4] = {0u, 0u, 0u, 0u};
        if constexpr (F::kNope > 1) {
          const uint4 k2 = lds_u4(&tr[(F::kWScale + 1) * kTS + 4 * g]);
          ksw2[0] = k2.x, ksw2[1] = k2.y, ksw2[2] = k2.z, ksw2[3] = k2.w;
        }
        auto kscale = [&](int c, int i) {
          const uint32_t w = c < 2 ? ksw[i] : ksw2[i];
          return h2f((uint16_t)((c & 1) ? (w >> 16) : (w & 0xffffu)));
        };
        // RoPE block: words 2g, 2g + 1 of token n (dims 16 g .. 16 g + 15).
        const uint32_t r0 = tr[(2 * g) * kTS + n], r1 = tr[(2 * g + 1) * kTS + n];
        int4_t A0;
        {
          uint32_t l0, h0, l1, h1;
          k4_word(r0, l0, h0);
          k4_word(r1, l1, h1);
          A0 = (int4_t){(int)l0, (int)h0, (int)l1, (int)h1};
        }
        // NoPE block b: low-bit plane word 4 b + g, high-bit plane word
        // 2 b + (g >> 1) (the planes span all NoPE dims).
        int4_t A[1 + F::kNope];
        A[0] = A0;
#pragma unroll
        for (int b = 0; b < F::kNope; ++b) {
          const uint32_t lw = tr[(F::kWNope + 4 * b + g) * kTS + n];
          const uint32_t hw = tr[(F::kWNopeHi + 2 * b + (g >> 1)) * kTS + n] >> hsh;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t s = ((lw >> (2 * i)) & 0x03030303u) | (((hw >> i) << 2) & 0x04040404u);
            A[1 + b][i] = (int)__builtin_amdgcn_perm(kK3[1], kK3[0], s);
          }
        }
        if constexpr (!kK16) {
          int4_t C[1 + F::kNope];
#pragma unroll
          for (int c = 0; c <= F::kNope; ++c)
            C[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[c], qreg[c], zero4, 0, 0, 0);
          // (|2^8 hi + mid| sums stay below 2^29: 64 products of at most 2^14)
#pragma unroll
          for (int c = 0; c <= F::kNope; ++c)
            C[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[c], qmid[c], C[c] << 8, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float acc = (float)C[0][i] * kscale(0, i);
#pragma unroll
            for (int c = 1; c <= F::kNope; ++c) acc = fmaf((float)C[c][i], kscale(c, i), acc);
            sc[i] = pair_score(fmaf(acc, w_own, ror8(acc) * w_partner), n);
          }
        } else {
          // 2^8 hi + mid joined in int32 (exact, below 2^29), then the lo
          // plane in fp32.
          int4_t H[1 + F::kNope], Lo[1 + F::kNope];
#pragma unroll
          for (int c = 0; c <= F::kNope; ++c) {
            H[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[c], qreg[c], zero4, 0, 0, 0);
            Lo[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[c], qlo[c], zero4, 0, 0, 0);
          }
#pragma unroll
          for (int c = 0; c <= F::kNope; ++c)
            H[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[c], qmid[c], H[c] << 8, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float acc = fmaf((float)H[0][i], 256.0f, (float)Lo[0][i]) * kscale(0, i);
#pragma unroll
            for (int c = 1; c <= F::kNope; ++c)
              acc = fmaf(fmaf((float)H[c][i], 256.0f, (float)Lo[c][i]), kscale(c, i), acc);
            sc[i] = acc * qs;
          }
        }
      } else {
        // Four 64-dim blocks under one scale: the int32 results add up (the
        // sums of one plane stay below 2^23, so 2^8 hi + mid below 2^31).
        int4_t C = zero4, Cm = zero4, Cl = zero4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t lw = tr[(4 * c + g) * kTS + n];
          const uint32_t hw = tr[(F::kWKHi + 2 * c + (g >> 1)) * kTS + n] >> hsh;
          int4_t Ac;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t s = ((lw >> (2 * i)) & 0x03030303u) | (((hw >> i) << 2) & 0x04040404u);
            Ac[i] = (int)__builtin_amdgcn_perm(kK3[1], kK3[0], s);
          }
          C = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ac, qreg[c], C, 0, 0, 0);
          Cm = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ac, qmid[c], Cm, 0, 0, 0);
          if constexpr (kK16) Cl = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ac, qlo[c], Cl, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hm = C[i] * 256 + Cm[i];  // 8-row mode lanes n >= 8: 2^8 lo (Cm = 0)
          if constexpr (!kK16) {
            const float acc = (float)hm * h2f((uint16_t)(ksw[i] & 0xffffu));
            sc[i] = pair_score(fmaf(acc, w_own, ror8(acc) * w_partner), n);
          } else {
            sc[i] = fmaf((float)hm, 256.0f, (float)Cl[i]) * h2f((uint16_t)(ksw[i] & 0xffffu)) * qs;
          }
        }
      }
    };

    // Softmax of unit u (tiles 2u, 2u + 1) and the P.V A operand: p times
    // the token's V scale (the 1/64 of the codebook is taken out of p and
    // put back into l at the end).
    struct AOps {
      half8_t a, b;  // 8-row mode: a only (both tiles); 16-row mode: per tile
    };
    auto stage_m = [&](const float (&sa)[4], const float (&sb)[4], int u, int buf, AOps& A) {
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
      float mt = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                       fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      mt = max_xor16_32(mt);
      if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy) != 0) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
        l_run *= alpha;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, kK16 ? 4 * g + i : (4 * g + i) & 7, kWave);
#pragma unroll
        for (int b = 0; b < kAcc; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[b][i] *= al[i];
        m_run = m_new;
      }
      const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;
      // V scale: low half of word 31 (k3v4), high half of the scale word (compact).
      constexpr int kWVs = F::kWVS;
      constexpr int kVsh = F::kVSh;
      const uint4 va = lds_u4(&L.u.tt[wave][buf][0][kWVs][4 * g]);
      const uint4 vb = lds_u4(&L.u.tt[wave][buf][1][kWVs][4 * g]);
      const uint32_t vw[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[i] - m_ref - 6.0f);  // p / 64
        l_run += p;
        pv[i] = p * h2f((uint16_t)((vw[i] >> kVsh) & 0xffffu));
      }
      // The leading fp16 parts come from one conversion instruction and the
      // residuals are taken against exactly those values, so that the matrix
      // cores see p s to 2^-21.
      _Float16 h[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half2_t hp = __builtin_amdgcn_cvt_pkrtz(pv[2 * j], pv[2 * j + 1]);
        h[2 * j] = (_Float16)hp[0];
        h[2 * j + 1] = (_Float16)hp[1];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const _Float16 r = (_Float16)(fmaf((float)h[i], -4096.0f, pv[i] * 4096.0f));  // exact before the rounding
        if constexpr (!kK16) {
          A.a[i] = live_row ? (n < 8 ? h[i] : r) : (_Float16)0.0f;
        } else {
          // k-slots 0-3: fp16(p s) of the tile's 4 tokens, 4-7: residual x 2^12.
          half8_t& At = i < 4 ? A.a : A.b;
          At[i & 3] = live_row ? h[i] : (_Float16)0.0f;
          At[4 + (i & 3)] = live_row ? r : (_Float16)0.0f;
        }
      }
    };

    // P.V of a unit from LDS buffer `buf`, accumulator tiles [w0, w0 + nw)
    // (k3v4: even and odd tiles are the low and high nibbles of V word group
    // b >> 1; compact: tile m holds dims 16 m .. 16 m + 15).
    // Two tiles' B operands in 16-row mode: values, then values x 2^-12.
    auto k16_ops = [&](const half8_t& v, half8_t& ba, half8_t& bb) {
      const _Float16 s12 = (_Float16)(1.0f / 4096.0f);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ba[i] = v[i];
        ba[4 + i] = v[i] * s12;
        bb[i] = v[4 + i];
        bb[4 + i] = v[4 + i] * s12;
      }
    };
    auto mma = [&](const AOps& A, const half8_t& v, float4_t& acc) {
      if constexpr (!kK16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.a, v, acc, 0, 0, 0);
      } else {
        half8_t ba, bb;
        k16_ops(v, ba, bb);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.a, ba, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.b, bb, acc, 0, 0, 0);
      }
    };
    auto stage_p = [&](const AOps& A, int buf, int w0, int nw) {
      const uint32_t* va = &L.u.tt[wave][buf][0][0][4 * g];
      const uint32_t* vb = &L.u.tt[wave][buf][1][0][4 * g];
      // Biased codebook bytes of 2 x four codes -> the exact fp16 values:
      // 1024 + byte = 1152 + LUT, less 1152.
      auto spread = [&](uint32_t x, uint32_t y) {
        const uint4 u = {__builtin_amdgcn_perm(0x64646464u, x, 0x04010400u),
                         __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u),
                         __builtin_amdgcn_perm(0x64646464u, y, 0x04010400u),
                         __builtin_amdgcn_perm(0x64646464u, y, 0x04030402u)};
        const half8_t c1152 = {(_Float16)-1152.0f, (_Float16)-1152.0f, (_Float16)-1152.0f,
                               (_Float16)-1152.0f, (_Float16)-1152.0f, (_Float16)-1152.0f,
                               (_Float16)-1152.0f, (_Float16)-1152.0f};
        return __builtin_bit_cast(half8_t, u) + c1152;
      };
      // Byte (n & 3) of a word of tokens 4g..4g+3.
      auto gather = [&](const uint4& W) {
        return __builtin_amdgcn_perm(W.y, W.x, gsel_lo) | __builtin_amdgcn_perm(W.w, W.z, gsel_hi);
      };
      if constexpr (!F::kV3) {
#pragma unroll
        for (int W = w0 / 2; W < (w0 + nw) / 2; ++W) {
          const int wrd = F::kWV + 4 * W + (n >> 2);
          const uint32_t ga = gather(lds_u4(va + wrd * kTS)), gb = gather(lds_u4(vb + wrd * kTS));
          // Biased codebook bytes of the low (dim 8w + j) and high (8w + 4 + j) nibbles.
          const uint32_t la = lut16(ga & 0x07070707u, byte_sign_mask(ga << 4), kV4[0], kV4[1], kV4[2], kV4[3]);
          const uint32_t ha = lut16((ga >> 4) & 0x07070707u, byte_sign_mask(ga), kV4[0], kV4[1], kV4[2], kV4[3]);
          const uint32_t lb = lut16(gb & 0x07070707u, byte_sign_mask(gb << 4), kV4[0], kV4[1], kV4[2], kV4[3]);
          const uint32_t hb = lut16((gb >> 4) & 0x07070707u, byte_sign_mask(gb), kV4[0], kV4[1], kV4[2], kV4[3]);
          const half8_t lo = spread(la, lb);
          const half8_t hi = spread(ha, hb);
          mma(A, lo, o[2 * W]);
          mma(A, hi, o[2 * W + 1]);
        }
      } else {
#pragma unroll
        for (int mp = w0 / 2; mp < (w0 + nw) / 2; ++mp) {
          // High-bit plane word mp serves dims 32 mp .. 32 mp + 31 (tiles 2mp, 2mp+1).
          const uint32_t gha = gather(lds_u4(va + (F::kWVHi + mp) * kTS));
          const uint32_t ghb = gather(lds_u4(vb + (F::kWVHi + mp) * kTS));
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int m = 2 * mp + h;
            const uint32_t gla = gather(lds_u4(va + (F::kWV + m) * kTS));
            const uint32_t glb = gather(lds_u4(vb + (F::kWV + m) * kTS));
            const int sh = 4 * h + vi;
            const uint32_t sa_ = ((gla >> (2 * vi)) & 0x03030303u) | (((gha >> sh) << 2) & 0x04040404u);
            const uint32_t sb_ = ((glb >> (2 * vi)) & 0x03030303u) | (((ghb >> sh) << 2) & 0x04040404u);
            const uint2 ha = lut3_half(sa_, kH3Hi[0], kH3Hi[1]);
            const uint2 hb = lut3_half(sb_, kH3Hi[0], kH3Hi[1]);
            const half8_t vv = __builtin_bit_cast(half8_t, make_uint4(ha.x, ha.y, hb.x, hb.y));
            mma(A, vv, o[m]);
          }
        }
      }
    };

    float sa[4], sb[4];
    int u_cur = wave, u_nxt = wave + NW;
    stage_s(ta, 0, 0, sa);
    fetch(ta, 2 * u_nxt);
    stage_s(tb, 1, 0, sb);
    fetch(tb, 2 * u_nxt + 1);
    int buf = 0;
    AOps A;
    while (u_nxt < nu) {
      int u_nn = u_nxt + NW;  // deterministic mode: a fixed order
      if (!a.det) {
        if (lane == 0) u_nn = atomicAdd(&L.next_unit, 1);
        u_nn = __builtin_amdgcn_readfirstlane(u_nn);
      }
      stage_m(sa, sb, u_cur, buf, A);
      // One basic block: P.V of unit u_cur and the scores of unit u_nxt.
      const int sbuf = buf ^ 1;
      stage_p(A, buf, 0, kAcc / 2);
      __builtin_amdgcn_sched_barrier(0);
      stage_s(ta, 0, sbuf, sa);
      fetch(ta, 2 * u_nn);
      __builtin_amdgcn_sched_barrier(0);
      stage_p(A, buf, kAcc / 2, kAcc / 2);
      __builtin_amdgcn_sched_barrier(0);
      stage_s(tb, 1, sbuf, sb);
      fetch(tb, 2 * u_nn + 1);
      // Keep these loads here (moved into the next iteration's head they
      // would collide with the accumulators' registers).
      __builtin_amdgcn_sched_barrier(0);
      u_cur = u_nxt;
      u_nxt = u_nn;
      buf = sbuf;
    }
    stage_m(sa, sb, u_cur, buf, A);
    stage_p(A, buf, 0, kAcc);
  }

  // 8-row mode: rows 8-15 of the P.V tiles (lanes 32-63) hold the residual
  // part (x 2^12): fold them into rows 0-7 (lanes 0-31).
  if constexpr (!kK16) {
#pragma unroll
    for (int b = 0; b < kAcc; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u = __float_as_uint(o[b][i]);
        const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        o[b][i] = fmaf(__uint_as_float(sw[1]), 1.0f / 4096.0f, o[b][i]);
      }
  }

  // ---- merge the waves ----------------------------------------------------
  float lsum = l_run + __shfl_xor(l_run, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  if (g == 0 && n < RM) {
    L.mlw[wave][n][0] = m_run;
    L.mlw[wave][n][1] = lsum * 64.0f;  // p was kept as p / 64
  }
  __syncthreads();
  if (kK16 || g < 2) {
    float fw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, L.mlw[w][r][0]);
      const float mw = L.mlw[wave][r][0];
      fw[i] = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
    }
#pragma unroll
    for (int b = 0; b < kAcc; ++b) {
      const int d = F::kV3 ? 16 * b + n : 32 * (b >> 1) + 8 * (n >> 2) + (n & 3) + 4 * (b & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) L.u.ob[wave][4 * g + i][d] = o[b][i] * fw[i];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.rows * kD; idx += blockDim.x) {
    const int r = idx / kD, d = idx % kD;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) acc += L.u.ob[w][r][d];
    part[r * a.pstride + kPartialHead + d] = acc;
  }
  if (threadIdx.x < a.rows) {
    const int r = threadIdx.x;
    float M = -INFINITY, L_ = 0.0f;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, L.mlw[w][r][0]);
    for (int w = 0; w < NW; ++w) {
      const float mw = L.mlw[w][r][0];
      if (mw != -INFINITY) L_ += L.mlw[w][r][1] * exp2f(mw - M);
    }
    part[r * a.pstride + 0] = M;
    part[r * a.pstride + 1] = L_;
  }
}


// ---- 32 query rows per KV head (k3v3 compact, head size 256), one pass ----
//
// The rows of a sequence group sharing a KV head (up to 32) take every tile
// once, so the codebook lookups of K and V are paid once for all of them.
// Both products run on the 32 x 32 matrix-core shapes:
//  * scores on v_mfma_f32_32x32x16_f16: A = the codebook values of 32
//    tokens x 16 dims as exact fp16 (a lane: token l % 32, 8 of the dims
//    16 (l / 32) .. + 15 of a 32-dim block, which are one low-plane word of
//    the token; two products per block), B = the rotated query, each row
//    scaled by a power of two so that its largest value lies in
//    [2^14, 2^15), as an fp16 leading part and the fp16 residual; both
//    planes go into one fp32 accumulator, which keeps about 23 bits of the
//    row's largest value whatever its magnitude.  (Three int8 planes would
//    need a third 16-register accumulator, which this kernel has no room
//    for.)  A lane ends with the scores of its row l % 32 for tokens
//    8 j + 4 (l / 32) + i, j, i < 4: the very k-slots that lane supplies as
//    the B operand of P.V, so p never moves between lanes.
//  * P.V on v_mfma_f32_32x32x16_f16 as O^T = V^T P^T (rows = dims, columns =
//    query rows), 8 tokens per step: a lane's k-slots are its 4 tokens'
//    fp16(p s) and their residuals x 2^12, against the tokens' values and
//    values x 2^-12: the values exact fp16 assembled from two byte tables
//    (the low and the high bytes) with two v_perm_b32 interleaves per four
//    codes, the copies one packed multiply by 2^-12 per two values (exact:
//    every |LUT| >= 14 stays a normal fp16).
//  * V dims: tile (b, i) of 32 dims has row a = 4 m' + j holding dim
//    16 (8 b + m') + 4 i + j; a lane gathers byte j of low-plane word 8 b + m'
//    of its 4 tokens once and takes the codes of all four i from it.
constexpr int kR32 = 32;
constexpr int kOB = 65;  // row stride (floats) of the cross-wave sum: 64 values + pad

template <int W>
struct __align__(16) Oct32Lds {
  static constexpr int kWords = 48;  // code words of a compact slot (the scale word is staged as floats)
  float qsc[kR32];
  float mlw[W][kR32][2];
  int pid[kMaxSplitTiles];
  int next_unit;
  int pad_[3];
  union {
    struct {
      uint32_t tt[W][2][kWords][kTS];  // [tile][slot word][token], one unit per wave
      float sc[W][2][2][kT];           // [tile][K | V][token] scales as fp32
      // [lead | residual][32-dim block][row][dim in block]; rows padded to 40
      // halves (20 words), so the 16-byte reads of 16 rows at a time cover
      // every bank once
      _Float16 qB[2][8][kR32][40];
    } s;
    float ob[W][2][kR32][kOB];         // [wave][l / 32][row][value] for one half of the dims
  } u;
};

template <int W>
__global__ __launch_bounds__(W * kWave, 1) void decode_oct32_kernel(DevFmt f, DecArgs a) {
  using F = FmtK3V3C;
  constexpr int kD = F::kD;
  constexpr int kSlot = F::kSlot;
  constexpr int kE = kD / kWave;
  constexpr int kQR = kR32 / W;  // query rows set up per wave
  __shared__ Oct32Lds<W> L;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  static_assert(kMaxSplitTiles <= W * kWave, "one page id per thread");
  int page_size = f.page_size, k_block = f.k_block;
  float k_norm = f.k_norm;
  pin_args(a, page_size, k_block, k_norm);
  int split, kvh, gi;
  if (!wg_item(a, split, kvh, gi)) return;
  const int q0 = gi * a.n_q;
  // ---- prologue: three memory round trips before the stream (as in
  // decode_oct_kernel): query rows and key lengths, page ids, first tiles.
  uint32_t qw[kQR][kE];
#pragma unroll
  for (int k = 0; k < kQR; ++k) query_row_raw<kE>(a, q0, kvh, wave + W * k, lane, qw[k]);
  uint32_t sw[kE];
  lane_sign_words<kE>(f, f.use_signs, lane, sw);
  const int kl = group_klen_lane(a, q0, lane);  // n_q <= kR32
  const int req = a.q_to_req[q0];
  const int kmax = wave_max_int(kl);
  const int kmin = wave_min_int(kl);
  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(t_begin + a.tokens_per_split, kmax);
  float* part = a.ws + (((size_t)gi * a.num_kv_heads + kvh) * a.num_splits + split) * kR32 *
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
  const int ps = page_size;
  const int ps_shift = 31 - __builtin_clz(ps);
  const int nt = (t_end - t_begin + kT - 1) / kT;
  const int nu = (nt + 1) >> 1;
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
    for (int i = 0; i < F::kChunks; ++i) x.c[i] = load_chunk<F>(slot, 4 * i + gq);
    x.sw = *(const uint32_t*)(slot + 4 * F::kWScale);
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
#pragma unroll
  for (int k = 0; k < kQR; ++k) {
    const int r = wave + W * k;
    float x[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) x[e] = flip_sign(query_value(a, qw[k][e], r < a.rows), sw[e], lane);
    fwht_strided<kE>(x, k_block, k_norm);
    float qmax = 0.0f;
#pragma unroll
    for (int e = 0; e < kE; ++e) qmax = fmaxf(qmax, fabsf(x[e]));
    qmax = wave_max(qmax);
    // x 2^k (exact) puts the row's largest value in [2^14, 2^15).
    const float rs = qmax > 0.0f ? ldexpf(1.0f, 14 - ilogbf(qmax)) : 1.0f;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const float y = x[e] * rs;
      const _Float16 hi = (_Float16)y;
      const int d = kWave * e + lane;
      L.u.s.qB[0][d >> 5][r][d & 31] = hi;
      L.u.s.qB[1][d >> 5][r][d & 31] = (_Float16)(y - (float)hi);  // exact difference
    }
    // 1/64: the codebook scale (LUT_ONE) of the K values.
    if (lane == 0) L.qsc[r] = a.q_scale * (1.0f / 64.0f) / rs;
  }
  const int n = lane & 31;  // this lane's query row (scores, P.V columns) and token (K operand)
  const int h = lane >> 5;
  const int klen_lane_row = __shfl(kl, (n < a.rows ? n : 0) / a.group, kWave);
  const int klen_row = n < a.rows ? klen_lane_row : 0;
  const int t_lim = min(t_end, kmin);
  // V operand rows: dim 16 (8 b + m') + 4 i + j for row n = 4 m' + j.
  const int vm = n >> 2, vj = n & 3;
  const uint32_t gsel_lo = (uint32_t)vj | ((uint32_t)(vj + 4) << 8) | (0x0Cu << 16) | (0x0Cu << 24);
  const uint32_t gsel_hi = 0x0Cu | (0x0Cu << 8) | ((uint32_t)vj << 16) | ((uint32_t)(vj + 4) << 24);
  const int vsh = 4 * (vm & 1);
  __syncthreads();
  // (kept positive so that a masked score, -inf, stays -inf through the fma)
  const float qs = fmaxf(L.qsc[n], 0x1p-126f);

  f32x16 o[8];
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  if (has_work) {
    uint32_t* const tw = &L.u.s.tt[wave][0][0][0];
    int u_cur = wave;
    for (;;) {
      // ---- stage the unit's two tiles (registers -> LDS, transposed) ----
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const Tile& x = hb ? tb : ta;
        uint32_t* w = tw + hb * (Oct32Lds<W>::kWords * kTS) + tl;
#pragma unroll
        for (int i = 0; i < F::kChunks; ++i) {
          w[(16 * i + 4 * gq + 0) * kTS] = x.c[i].x;
          w[(16 * i + 4 * gq + 1) * kTS] = x.c[i].y;
          w[(16 * i + 4 * gq + 2) * kTS] = x.c[i].z;
          w[(16 * i + 4 * gq + 3) * kTS] = x.c[i].w;
        }
        if (gq == 0) {
          L.u.s.sc[wave][hb][0][tl] = h2f((uint16_t)(x.sw & 0xffffu));
          L.u.s.sc[wave][hb][1][tl] = h2f((uint16_t)(x.sw >> 16));
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
      f32x16 acc = {};
      {
        const uint32_t* tk = tw + (n >> 4) * (Oct32Lds<W>::kWords * kTS) + (n & 15);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t lw = tk[(2 * c + h) * kTS];
          const uint32_t hw = tk[(F::kWKHi + c) * kTS] >> (4 * h);
          // dims 4 i + jb of the lane's 16 as fp16: product j takes i = 2 j, 2 j + 1
          uint32_t A[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t s = ((lw >> (2 * i)) & 0x03030303u) | (((hw >> i) << 2) & 0x04040404u);
            const uint32_t lb = __builtin_amdgcn_perm(kH3Lo[1], kH3Lo[0], s);
            const uint32_t hb = __builtin_amdgcn_perm(kH3Hi[1], kH3Hi[0], s);
            A[2 * i] = __builtin_amdgcn_perm(hb, lb, 0x05010400u);
            A[2 * i + 1] = __builtin_amdgcn_perm(hb, lb, 0x07030602u);
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint4 Aj = {A[4 * j], A[4 * j + 1], A[4 * j + 2], A[4 * j + 3]};
            const half8_t a8 = __builtin_bit_cast(half8_t, Aj);
            const half8_t bh = *(const half8_t*)&L.u.s.qB[0][c][n][16 * h + 8 * j];
            const half8_t bl = *(const half8_t*)&L.u.s.qB[1][c][n][16 * h + 8 * j];
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a8, bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a8, bl, acc, 0, 0, 0);
          }
        }
      }
      // score k = 4 j + i: token 8 j + 4 h + i of the unit (tile j >> 1),
      // held as s / qs until the exponent
      float s[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 ks = *(const float4*)&L.u.s.sc[wave][j >> 1][0][8 * (j & 1) + 4 * h];
        const float kk[4] = {ks.x, ks.y, ks.z, ks.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[4 * j + i] = acc[4 * j + i] * kk[i];
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
        const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * qs;
      }
      if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy) != 0) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[b][i] *= alpha;
        m_run = m_new;
      }
      const float m6 = ((m_run == -INFINITY) ? 0.0f : m_run) + 6.0f;
      // P operands: step j, k-slots 0-3 fp16(p s) of tokens 8 j + 4 h + i, 4-7 residuals x 2^12
      half8_t P[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 vs = *(const float4*)&L.u.s.sc[wave][j >> 1][1][8 * (j & 1) + 4 * h];
        const float vv[4] = {vs.x, vs.y, vs.z, vs.w};
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[4 * j + i], qs, -m6));  // p / 64
          l_run += p;
          pv[i] = p * vv[i];
        }
        // The leading fp16 parts come from one conversion instruction, so the
        // residuals are taken against exactly the values the product sees.
        const half2_t h01 = __builtin_amdgcn_cvt_pkrtz(pv[0], pv[1]);
        const half2_t h23 = __builtin_amdgcn_cvt_pkrtz(pv[2], pv[3]);
        const _Float16 hp[4] = {(_Float16)h01[0], (_Float16)h01[1], (_Float16)h23[0], (_Float16)h23[1]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          P[j][i] = hp[i];
          P[j][4 + i] = (_Float16)fmaf((float)hp[i], -4096.0f, pv[i] * 4096.0f);  // exact before the rounding
        }
      }

      // ---- P.V: 8 accumulator tiles of 32 dims ----
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t* vt = tw + (j >> 1) * (Oct32Lds<W>::kWords * kTS) + 8 * (j & 1) + 4 * h;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const uint4 wl = lds_u4(vt + (F::kWV + 8 * b + vm) * kTS);
          const uint4 wh = lds_u4(vt + (F::kWVHi + 4 * b + (vm >> 1)) * kTS);
          const uint32_t gl = __builtin_amdgcn_perm(wl.y, wl.x, gsel_lo) |
                              __builtin_amdgcn_perm(wl.w, wl.z, gsel_hi);
          const uint32_t gh = (__builtin_amdgcn_perm(wh.y, wh.x, gsel_lo) |
                               __builtin_amdgcn_perm(wh.w, wh.z, gsel_hi)) >> vsh;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t sel = ((gl >> (2 * i)) & 0x03030303u) | (((gh >> i) << 2) & 0x04040404u);
            const uint32_t xl = __builtin_amdgcn_perm(kH3Lo[1], kH3Lo[0], sel);
            const uint32_t xh = __builtin_amdgcn_perm(kH3Hi[1], kH3Hi[0], sel);
            const uint32_t a0 = __builtin_amdgcn_perm(xh, xl, 0x05010400u);
            const uint32_t a1 = __builtin_amdgcn_perm(xh, xl, 0x07030602u);
            // the copies x 2^-12: exact (every |LUT| >= 14 stays a normal fp16)
            const half2_t s12 = {(__fp16)(1.0f / 4096.0f), (__fp16)(1.0f / 4096.0f)};
            const uint4 A = {a0, a1, __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a0) * s12),
                             __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a1) * s12)};
            o[4 * b + i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(half8_t, A), P[j], o[4 * b + i], 0, 0, 0);
          }
        }
      }
      if (u_nxt >= nu) break;
      u_cur = u_nxt;
    }
  }

  // ---- merge the waves ----------------------------------------------------
  // This lane: row n, values of dims 16 (8 b + m') + 4 i + j for tile 4 b + i,
  // register 4 jj + ii, with 4 m' + j = 8 jj + 4 h + ii.
  float lsum;
  {
    const uint32_t lu = __float_as_uint(l_run);
    const auto ls = __builtin_amdgcn_permlane32_swap(lu, lu, false, false);
    lsum = __uint_as_float(ls[0]) + __uint_as_float(ls[1]);
  }
  if (h == 0) {
    L.mlw[wave][n][0] = m_run;
    L.mlw[wave][n][1] = lsum * 64.0f;  // p was kept as p / 64
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
  for (int b = 0; b < 2; ++b) {
    if (b) __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 16; ++k) L.u.ob[wave][h][n][16 * i + k] = o[4 * b + i][k] * fw;
    __syncthreads();
    for (int idx = threadIdx.x; idx < a.rows * 128; idx += blockDim.x) {
      const int r = idx >> 7, dd = idx & 127;
      // dd = 16 m' + 4 i + j -> lane half (m' & 1), register 4 (m' >> 1) + j of tile i
      const int mp = dd >> 4, i = (dd >> 2) & 3, j = dd & 3;
      const int hh = mp & 1, k = 4 * (mp >> 1) + j;
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) acc += L.u.ob[w][hh][r][16 * i + k];
      part[r * a.pstride + kPartialHead + 128 * b + dd] = acc;
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

// Rows the Octave MFMA kernels take for this format: 8 or 16 (the row
// mode), 32 (the compact layout's one-pass kernel), or 0 when the format
// or the row count is not one they handle.
int oct_mfma_rows(const DevFmt& f, int rows) {
  const bool pow2 = (f.page_size & (f.page_size - 1)) == 0;
  if (f.kind != HKV_KIND_OCTAVE || rows > (f.compact ? kR32 : kRowsMax) || f.page_size % kT != 0 ||
      !pow2)
    return 0;
  bool ok;
  if (!f.compact && f.v_bits == 4 && f.D == FmtK3V4W::kD)
    ok = f.k_wide == 64 && f.slot_bytes == FmtK3V4W::kSlot &&
         f.off_k_nope == 4 * FmtK3V4W::kWNope && f.off_v == 4 * FmtK3V4W::kWV &&
         f.off_scales == 4 * FmtK3V4W::kWScale && f.num_k_scales == 3 && f.k_block == 64;
  else if (!f.compact && f.v_bits == 4)
    ok = f.D == FmtK3V4::kD && f.k_wide == 64 &&
         f.slot_bytes == FmtK3V4::kSlot && f.off_k_nope == 4 * FmtK3V4::kWNope &&
         f.off_v == 4 * FmtK3V4::kWV && f.off_scales == 4 * FmtK3V4::kWScale &&
         f.num_k_scales == 2 && f.k_block == 64;
  else if (!f.compact)
    ok = f.D == FmtK3V3::kD && f.k_wide == 64 && f.v_bits == 3 &&
         f.slot_bytes == FmtK3V3::kSlot && f.off_k_nope == 4 * FmtK3V3::kWNope &&
         f.off_v == 4 * FmtK3V3::kWV && f.off_scales == 4 * FmtK3V3::kWScale &&
         f.num_k_scales == 2 && f.k_block == 64 && f.v_block == FmtK3V3::kD;
  else
    ok = f.D == FmtK3V3C::kD && f.v_bits == 3 && f.slot_bytes == FmtK3V3C::kSlot &&
         f.off_v == 4 * FmtK3V3C::kWV && f.off_scales == 4 * FmtK3V3C::kWScale &&
         f.num_k_scales == 1 && f.k_block == FmtK3V3C::kD;
  if (!ok) return 0;
  return rows <= 8 ? 8 : rows <= 16 ? 16 : 32;
}

hipError_t launch_decode_oct(const DevFmt& f, const DecArgs& a, dim3 grid, hipStream_t s) {
  if ((a.tokens_per_split + kT - 1) / kT > kMaxSplitTiles) return hipErrorInvalidValue;
  const dim3 block(kQWaves * kWave);
  const dim3 block12(kQWaves12 * kWave);
  if (a.rows_pad == 8) {
    if (f.compact) decode_oct_kernel<FmtK3V3C, 8, kQWaves><<<grid, block, 0, s>>>(f, a);
    else if (f.v_bits == 3) decode_oct_kernel<FmtK3V3, 8, kQWaves12><<<grid, block12, 0, s>>>(f, a);
    else if (f.D == FmtK3V4W::kD) decode_oct_kernel<FmtK3V4W, 8, kQWaves><<<grid, block, 0, s>>>(f, a);
    else decode_oct_kernel<FmtK3V4, 8, kQWaves12><<<grid, block12, 0, s>>>(f, a);
  } else if (a.rows_pad == 16) {
    if (f.compact) decode_oct_kernel<FmtK3V3C, 16, kQWaves><<<grid, block, 0, s>>>(f, a);
    else if (f.v_bits == 3) decode_oct_kernel<FmtK3V3, 16, kQWaves><<<grid, block, 0, s>>>(f, a);
    else if (f.D == FmtK3V4W::kD) decode_oct_kernel<FmtK3V4W, 16, kQWaves><<<grid, block, 0, s>>>(f, a);
    else decode_oct_kernel<FmtK3V4, 16, kQWaves><<<grid, block, 0, s>>>(f, a);
  } else if (a.rows_pad == kR32 && f.compact) {
    decode_oct32_kernel<kQWaves><<<grid, block, 0, s>>>(f, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hkv
