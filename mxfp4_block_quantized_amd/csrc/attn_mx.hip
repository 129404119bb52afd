// Fused MXFP4 attention forward for gfx950 (OCP, UOS, UOS+PNQ and UOS+EFQ
// modes).
//
// What it computes ("MXAttention: Data-Free Optimal Scaling and
// Pre-Normalization Quantization for MXFP4 Attention", abstract;
// "EFQ-Softmax", abstract): S = Q~ K~^T on block-scaled FP4 matrix cores,
// FlashAttention online softmax with the running max updated once per KV
// tile of 128 keys, the unnormalized exponentials p = exp(s - m) quantized
// in blocks of 32 keys (scale rule of the mode) into P~, O += P~ V~ on FP4
// matrix cores, and O / l at the end.  Under PNQ the denominator l sums the
// same P~ (computed on the matrix core against an all-ones operand);
// otherwise it sums the unquantized p.
//
// Mapping onto v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 x FP4, fp32 accum):
// an operand lane l holds row (l % 16) and the 32 K-elements of K-block
// (l / 16) plus that block's E8M0 scale (one byte of a register, picked by
// the instruction's op_sel); the accumulator lane l, register r holds row
// 4*(l/16) + r, column l % 16.
//  * S^T = K~ Q~^T: A = 16 keys x 128 d, B = 128 d x 16 queries, one MFMA
//    covers D = 128.  The 16 A-rows of key subtile t (0..7) of a 128-key tile
//    are the keys 32*(row/4) + 4*t + row%4, so accumulator lane l holds, over
//    t and r, exactly the 32 keys 32*(l/16) + 4*t + r: one whole P~ block of
//    query l % 16.  Block maxima and the fp4 packing are therefore in-lane;
//    only the row max needs two cross-lane swaps.
//  * O^T = V~^T P~^T: A = 16 channels x 128 keys, B = P~ (128 keys x 16
//    queries) straight from the registers above, with one E8M0 byte per
//    lane.  The accumulator keeps query l % 16 in every lane of a column,
//    matching the softmax state.
// Q is quantized in the kernel's prologue: each lane holds exactly one
// 32-element block of its query row (the B operand layout), so it applies
// the block rule of the mode to the raw bf16/fp32 elements it loads
// (mx_block.h, the same code as the standalone quantizer).
// The quantizer writes K~ and V~ as KV tile images already in these operand
// orders, so a tile moves to LDS with contiguous 16-byte-per-lane direct
// loads (global_load_lds) and every operand read is one ds_read per lane.
//
// P~ is formed in the scaled domain: for a block with scale exponent e,
// v = exp2((s - m) * log2(e)/sqrt(D) - e) is rounded by
// v_cvt_scalef32_pk_fp4_f32 (round to nearest even,
// saturating).  This keeps blocks whose probabilities lie below fp32's
// normal range exact in the same way the binary64 definition treats them.
// The UOS+EFQ mode skips the exp: the code of each score is an affine
// function of its log2 residual to the block's exponent, rounded and
// clamped by v_cvt_pk_u8_f32 (efq_block_exp, tile_stats, p_tile).
#include "internal.h"
#include "mx_block.h"

namespace mxk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQT = 2;              // 16-query tiles per wave
constexpr int kSub = kKvTile / 16;  // key subtiles per KV tile (8)
constexpr int kStages = 3;          // LDS ring of KV tile images
static_assert(kMxQTile == kWaves * kQT * 16, "query tile = waves x q-tiles x 16");
static_assert(kMxQTile % kKvTile == 0, "query tiles start on KV tile boundaries");

template <int SEL_A>
__device__ __forceinline__ v4f mfma_fp4(const uint4& a, const uint4& b, v4f c, uint32_t sa, int sb) {
  v8i av = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z),
            static_cast<int>(a.w), 0, 0, 0, 0};
  v8i bv = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z),
            static_cast<int>(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, SEL_A,
                                                          static_cast<int>(sa), 0, sb);
}
// A-scale taken from byte `sel` (a constant after unrolling) of `sa`.
__device__ __forceinline__ v4f mfma_fp4_sel(const uint4& a, const uint4& b, v4f c, uint32_t sa,
                                            int sel, int sb) {
  switch (sel) {
    case 0: return mfma_fp4<0>(a, b, c, sa, sb);
    case 1: return mfma_fp4<1>(a, b, c, sa, sb);
    case 2: return mfma_fp4<2>(a, b, c, sa, sb);
    default: return mfma_fp4<3>(a, b, c, sa, sb);
  }
}

// max / sum over the four lanes l, l^16, l^32, l^48 (same query column)
__device__ __forceinline__ float xlane_max4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xlane_sum4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Scale exponent e of a P~ block from x = log2 of its largest element,
// clamped to the E8M0 range (e >= -127; the byte is e + 127).  With
// E = floor(x) and mantissa 2^frac(x): OCP takes e = E - 2; UOS moves one
// binade up when the mantissa exceeds 1.8125, i.e. frac(x) > log2(1.8125),
// which is e = floor(x - log2(1.8125)) - 1.  A block with no unmasked key
// (x = -inf) gets -127.
template <int UOS>
__device__ __forceinline__ float p_block_exp(float x) {
  constexpr float kOfs = UOS ? 1.85798099512757209f : 2.0f;  // log2(1.8125) + 1, or 2
  return fmaxf(__builtin_floorf(x - kOfs), -127.0f);
}

// Exp-free P~ (UOS+EFQ mode; "EFQ-Softmax", abstract: exponent-only block
// scale from the local maximum, scores mapped to a residual domain,
// nonnegative E2M1 codes by one affine rule).  The page prints no constants;
// the reading implemented: on the log2 residual r = z - e of a block,
// code = clamp(round-half-even(2 r + beta), 0, 7) -- two codes per binade,
// as the E2M1 grid has above 1 -- with beta the least-squares fit of the
// rule's boundaries (c + 1/2 - beta)/2 to the E2M1 rounding boundaries
// log2((mag_c + mag_c+1)/2), c = 2..6:
//   beta = mean_c (c + 1/2 - 2 log2((mag_c + mag_c+1)/2)) = 1.8678023...
// and e the smallest exponent >= -127 with z_max - e < rho,
//   rho = (7.5 - beta)/2 - 2^-10,
// so that the block maximum stays below code 8 even after fp32 rounding.
constexpr float kEfqBeta = 1.8678023484890818f;
constexpr float kEfqRho = 2.8151222632554591f;

__device__ __forceinline__ float efq_block_exp(float x) {
  return fmaxf(__builtin_floorf(x - kEfqRho) + 1.0f, -127.0f);
}

// Per-wave softmax state and accumulators for kQT query tiles.
template <int D>
struct WaveState {
  v4f oacc[kQT][D / 16];
  v4f lacc[kQT];
  float m[kQT];     // running row max (raw score units), -inf before the first tile
  float mref[kQT];  // value subtracted from S on the matrix core
  float lsum[kQT];
};

// s_waitcnt on the vector-memory counter only (expcnt, lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
}

// A wave-uniform address kept in scalar registers, so that a direct load
// takes the scalar-base + 32-bit lane-offset form (one VGPR per lane for
// every load instead of a 64-bit address each).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Issue the direct loads of one KV tile image into an LDS stage: wave w
// moves the 1 KiB rows w, w + kWaves, ... of the image, lane l bytes
// [16 l, 16 l + 16) of each.  Buffer loads (a raw resource over the image,
// no range check), not the global form: with a global load-to-LDS in
// flight the compiler turns every LDS wait into a full lgkmcnt(0), so each
// operand read would also wait for the reads issued after it.
template <int D>
__device__ __forceinline__ void issue_tile(uint8_t* stage, const uint8_t* src, int wave, int lane) {
  constexpr int NL = img_bytes(D) / 1024;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(uniform_ptr(src)), 0, 0xFFFFFFFFu, 0x00020000);
  const uint32_t lo = static_cast<uint32_t>(lane) * 16u;
#pragma unroll
  for (int i = 0; i < (NL + kWaves - 1) / kWaves; ++i) {
    const int row = wave + i * kWaves;
    if (row < NL)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, stage + row * 1024, 16, lo, row * 1024, 0, 0);
  }
}

// Loads this wave issues per tile.
template <int D>
__device__ __forceinline__ int loads_per_tile(int wave) {
  constexpr int NL = img_bytes(D) / 1024;
  return NL / kWaves + (wave < NL % kWaves ? 1 : 0);
}

// S^T of one 16-query tile on the matrix core: d = S - mref, with -mref
// (the running max of the previous tiles, 0 before the first) as the
// accumulator input, so the subtraction happens before the single rounding
// of the result and elements near the maximum keep full relative precision.
__device__ __forceinline__ void s_tile(v4f (&s)[kSub], const uint4 (&kop)[kSub], const uint2& ksc,
                                       const uint4& qop, int qsc, float mref) {
  const v4f cneg = {-mref, -mref, -mref, -mref};
#pragma unroll
  for (int t = 0; t < kSub; ++t)
    s[t] = mfma_fp4_sel(kop[t], qop, cneg, t < 4 ? ksc.x : ksc.y, t & 3, qsc);
}

// Keys past `lim` (relative to this lane's 32-key block) are excluded.
__device__ __forceinline__ void mask_tile(v4f (&s)[kSub], int lim) {
  asm volatile("" : "+v"(lim));  // keeps the compares inside the caller's branch
#pragma unroll
  for (int t = 0; t < kSub; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) s[t][r] = (t * 4 + r > lim) ? -INFINITY : s[t][r];
}

// Largest of the 32 scores this lane holds (its P~ block of one query):
// a tree of v_max3 (depth 4) rather than one dependent chain.
__device__ __forceinline__ float block_max32(const v4f (&s)[kSub]) {
  // (the empty asm statements keep the compiler from re-associating the
  // tree into a chain)
  float a[kSub];
#pragma unroll
  for (int t = 0; t < kSub; ++t) a[t] = fmaxf(fmaxf(s[t][0], s[t][1]), s[t][2]);
  asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
               "+v"(a[7]));
  // 16 values: a[0..7] and s[t][3]
  float b0 = fmaxf(fmaxf(a[0], a[1]), a[2]);
  float b1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
  float b2 = fmaxf(fmaxf(a[6], a[7]), s[0][3]);
  float b3 = fmaxf(fmaxf(s[1][3], s[2][3]), s[3][3]);
  float b4 = fmaxf(fmaxf(s[4][3], s[5][3]), s[6][3]);
  asm volatile("" : "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3), "+v"(b4));
  float c0 = fmaxf(fmaxf(b0, b1), b2);
  float c1 = fmaxf(fmaxf(b3, b4), s[7][3]);
  asm volatile("" : "+v"(c0), "+v"(c1));
  return fmaxf(c0, c1);
}

// Online-softmax step of one query tile: row max, history factor alpha,
// this lane's P~ block scale (X, e) and the offset kofs of the scaled
// domain.  The history itself is rescaled by rescale_o.
struct TileStats {
  float alpha, kofs;
  int X;
};
// PNQ: 0 = denominator from the unquantized p (OCP, UOS); 1 = PNQ; 2 = PNQ
// with the exp-free EFQ codes.
template <int D, int UOS, int PNQ>
__device__ __forceinline__ TileStats tile_stats_nr(WaveState<D>& w, int u, const v4f (&s)[kSub], float sl2) {
  // row max: in-lane over this lane's 32-key block, then across the four
  // lanes holding this query
  const float bmax = block_max32(s);
  // delta = new max - mref.  Before the first tile the running max is -inf
  // (m - mref = -inf); afterwards m == mref, so delta = max(0, rowmax d).
  const float delta = fmaxf(w.m[u] - w.mref[u], xlane_max4(bmax));
  TileStats r;
  r.alpha = __builtin_amdgcn_exp2f((w.m[u] - w.mref[u] - delta) * sl2);  // 0 at first
  w.m[u] = w.mref[u] + delta;
  w.mref[u] = w.m[u];
  // scale of this lane's P~ block (the block holding the row maximum gets
  // x = 0 exactly); in the scaled domain
  // log2 v = (d - delta) * log2(e)/sqrt(D) - e = d*c - (delta*c + e)
  const float x = (bmax - delta) * sl2;
  const float e = PNQ == 2 ? efq_block_exp(x) : p_block_exp<UOS>(x);
  r.X = static_cast<int>(e) + 127;
  // EFQ: 2 r + beta = d * 2c + (beta - 2 (delta c + e)); else the exp2 offset
  r.kofs = PNQ == 2 ? kEfqBeta - 2.0f * fmaf(delta, sl2, e) : fmaf(delta, sl2, e);
  return r;
}

// History rescale by alpha: alpha == 1 exactly leaves the history
// unchanged, so the multiplies are skipped when that holds for the whole
// wave (a uniform branch).
template <int D, int PNQ>
__device__ __forceinline__ void rescale_o(WaveState<D>& w, int u, float alpha) {
  constexpr int NT = D / 16;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n) w.oacc[u][n] *= alpha;
    // the four lanes of a lacc column hold the same sum; only element 0 is
    // read at the end, so only it is kept rescaled (the others stay finite)
    if (PNQ) w.lacc[u][0] *= alpha;
  }
}

template <int D, int UOS, int PNQ>
__device__ __forceinline__ TileStats tile_stats(WaveState<D>& w, int u, const v4f (&s)[kSub], float sl2) {
  const TileStats r = tile_stats_nr<D, UOS, PNQ>(w, u, s, sl2);
  rescale_o<D, PNQ>(w, u, r.alpha);
  return r;
}

// P~ block of this lane: v = exp2(d*c - kofs) rounded to E2M1 (nearest
// even, saturating), packed in MFMA operand order; vsum = sum of v.
// EFQ (PNQ == 2): code = rne(d * 2c + kofs) by v_cvt_pk_u8_f32 (round half
// to even, saturating at 0; below 7.5 by the choice of e), even and odd
// elements into the bytes of two words, one shift-or per 8 codes.
template <int PNQ>
__device__ __forceinline__ uint4 p_tile(const v4f (&s)[kSub], float sl2, float kofs, float& vsum) {
  uint32_t pw[4];
  vsum = 0.0f;
  if (PNQ == 2) {
    const float c2 = 2.0f * sl2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = fmaf(s[2 * q + (i >> 2)][i & 3], c2, kofs);
      // all four bytes of each word are written, so the chains may start anywhere
      uint32_t a = __builtin_amdgcn_cvt_pk_u8_f32(t[0], 0, __float_as_uint(t[0]));
      a = __builtin_amdgcn_cvt_pk_u8_f32(t[2], 1, a);
      a = __builtin_amdgcn_cvt_pk_u8_f32(t[4], 2, a);
      a = __builtin_amdgcn_cvt_pk_u8_f32(t[6], 3, a);
      uint32_t b = __builtin_amdgcn_cvt_pk_u8_f32(t[1], 0, __float_as_uint(t[1]));
      b = __builtin_amdgcn_cvt_pk_u8_f32(t[3], 1, b);
      b = __builtin_amdgcn_cvt_pk_u8_f32(t[5], 2, b);
      b = __builtin_amdgcn_cvt_pk_u8_f32(t[7], 3, b);
      pw[q] = a | (b << 4);
    }
    return make_uint4(pw[0], pw[1], pw[2], pw[3]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // dword q holds key subtiles 2q and 2q+1
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = __builtin_amdgcn_exp2f(fmaf(s[2 * q + (i >> 2)][i & 3], sl2, -kofs));
      if (!PNQ) vsum += v[i];
    }
    // all four bytes are written, so the chain may start from any value
    uint32_t x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(__float_as_uint(v[0]), v[0], v[1], 1.0f, 0);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[2], v[3], 1.0f, 1);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[4], v[5], 1.0f, 2);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[6], v[7], 1.0f, 3);
    pw[q] = x;
  }
  return make_uint4(pw[0], pw[1], pw[2], pw[3]);
}

// Half h of dword q of p_tile's result: keys 8q + 4h .. 8q + 4h + 3 of this
// lane's block (subtile 2q + h), into bytes 2h and 2h+1 of x (the other
// half's bytes kept); vsum accumulates the unquantized v (non-PNQ modes).
// EFQ writes its code bytes into a (even keys) and b (odd keys) instead.
template <int PNQ, int h>
__device__ __forceinline__ void p_half(const v4f (&s)[kSub], int q, float sl2, float kofs, uint32_t& x,
                                       uint32_t& b, float& vsum) {
  const v4f& sv = s[2 * q + h];
  if (PNQ == 2) {
    const float c2 = 2.0f * sl2;
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = fmaf(sv[i], c2, kofs);
    // all four bytes of each word are written over the two halves
    x = __builtin_amdgcn_cvt_pk_u8_f32(t[0], 2 * h, h ? x : __float_as_uint(t[0]));
    x = __builtin_amdgcn_cvt_pk_u8_f32(t[2], 2 * h + 1, x);
    b = __builtin_amdgcn_cvt_pk_u8_f32(t[1], 2 * h, h ? b : __float_as_uint(t[1]));
    b = __builtin_amdgcn_cvt_pk_u8_f32(t[3], 2 * h + 1, b);
    if (h) x |= b << 4;
    return;
  }
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], sl2, -kofs));
    if (!PNQ) vsum += v[i];
  }
  // all four bytes are written over the two halves, so the first write may
  // start from any value
  x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h ? x : __float_as_uint(v[0]), v[0], v[1], 1.0f, 2 * h);
  x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[2], v[3], 1.0f, 2 * h + 1);
}

// Denominator and O^T += V~^T P~^T for one query tile.
template <int D, int PNQ>
__device__ __forceinline__ void pv_tile(WaveState<D>& w, int u, const uint4& pop, const TileStats& ts,
                                        float vsum, const uint4 (&vop)[D / 16], const uint32_t* vsc) {
  constexpr int NT = D / 16;
  if (PNQ) {
    const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);
    w.lacc[u] = mfma_fp4<0>(ones, pop, w.lacc[u], 127, ts.X);
  } else {
    w.lsum[u] = fmaf(w.lsum[u], ts.alpha, __builtin_amdgcn_ldexpf(vsum, ts.X - 127));
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) w.oacc[u][n] = mfma_fp4_sel(vop[n], pop, w.oacc[u][n], vsc[n >> 2], n & 3, ts.X);
}

template <int DUMP>
__device__ __forceinline__ void dump_tile(const MxAttnArgs& a, int64_t bh, int qrow, bool visit, int j0,
                                          int grp, const uint4& pop, int X) {
  if (DUMP && visit && qrow < a.Sq) {
    const int slot = a.row_slot[bh * a.Sq + qrow];
    if (slot >= 0) {
      *reinterpret_cast<uint4*>(a.p_codes + static_cast<int64_t>(slot) * (a.skv_ld / 2) + (j0 + grp * 32) / 2) = pop;
      a.p_scales[static_cast<int64_t>(slot) * (a.skv_ld / 32) + (j0 + grp * 32) / 32] = static_cast<uint8_t>(X);
    }
  }
}

// Q~ operand of one lane: query row `row` (global row index), d-block grp
// (< D/32), quantized from the raw row; the dump variants also store it.
template <int D, int UOS, int DUMP>
__device__ __forceinline__ void quant_q_block(const MxAttnArgs& a, int64_t row, int grp, uint4& qop,
                                              int& qsc) {
  const int64_t e0 = row * D + grp * 32;
  const void* src = a.q_bf16 ? static_cast<const void*>(static_cast<const uint16_t*>(a.q) + e0)
                             : static_cast<const void*>(static_cast<const float*>(a.q) + e0);
  uint32_t X;
  qop = quant_block32<UOS>(src, a.q_bf16 != 0, X);
  qsc = static_cast<int>(X);
  if (DUMP) {
    *reinterpret_cast<uint4*>(a.qc + row * (D / 2) + grp * 16) = qop;
    a.qs[row * (D / 32) + grp] = static_cast<uint8_t>(X);
  }
}

// Interleave n matrix-core instructions with the vector work around them
// (k vector or transcendental instructions after each), so that no wave
// issues matrix instructions back to back: a wave waiting for a busy
// matrix core holds up the other wave's vector instructions on its SIMD.
template <int N, int K>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x402, K, 0);  // VALU or TRANS
  }
}

// K~ and V~ operands of one KV tile, read from its LDS stage.
template <int D>
struct KOps {
  uint4 op[kSub];
  uint2 sc;
};
template <int D>
struct VOps {
  uint4 op[D / 16];
  uint32_t sc[(D / 16 + 3) / 4];
};
template <int D>
__device__ __forceinline__ void read_k(KOps<D>& k, const uint8_t* st, int lane) {
#pragma unroll
  for (int t = 0; t < kSub; ++t) k.op[t] = *reinterpret_cast<const uint4*>(st + kImgKc + t * 1024 + lane * 16);
  k.sc = *reinterpret_cast<const uint2*>(st + img_ks(D) + lane * 8);
}
template <int D>
__device__ __forceinline__ void read_v(VOps<D>& v, const uint8_t* st, int lane) {
  constexpr int NT = D / 16;
#pragma unroll
  for (int n = 0; n < NT; ++n) v.op[n] = *reinterpret_cast<const uint4*>(st + kImgVc + n * 1024 + lane * 16);
  if (NT == 8) {
    const uint2 v2 = *reinterpret_cast<const uint2*>(st + img_vs(D) + lane * 8);
    v.sc[0] = v2.x;
    v.sc[(NT + 3) / 4 - 1] = v2.y;
  } else {
    v.sc[0] = *reinterpret_cast<const uint32_t*>(st + img_vs(D) + lane * 4);
  }
}

// The two query tiles of a wave (A = 0, B = 1) run as a software pipeline
// with B half a KV tile behind A, so that every group of matrix
// instructions has independent vector work beside it.  For KV tile j:
//   step 1: P~V of B for tile j-1          | row max and scales of A, tile j
//   step 2: S^T of B for tile j            | P~ of A, tile j
//   step 3: P~V of A for tile j            | row max and scales of B, tile j
//   step 4: S^T of A for tile j+1          | P~ of B, tile j
// The history of A is rescaled between steps 1 and 2, that of B between
// steps 3 and 4 (a uniform branch, skipped when no row's max moved).  Each
// step's operands are read from LDS one step ahead and kept in registers
// while they are needed: V~ of tile j (read in step 2) serves steps 3 and
// the next step 1, K~ of tile j+1 (read in step 3) steps 4 and the next
// step 2.  At the last tile step 3 reads a stage with no pending loads and
// step 4's S^T is unused.
template <int D, int UOS, int PNQ>
struct Pipe {
  v4f sA[kSub], sB[kSub];  // S^T of A (tile j, from step 4 before) and of B
  TileStats tA, tB;
  uint4 pA, pB;            // P~ of A and B
  float vA, vB;            // sums of the unquantized p (non-PNQ modes)
  KOps<D> kk;              // K~ operands for steps 4 and 2
  VOps<D> vv;              // V~ operands for steps 3 and 1
};

// One fenced scheduling region: the compiler may order instructions within
// it but moves nothing across, so the interleave of matrix and vector work
// follows the source.  (This file is built with instruction selection in
// source order and without machine sinking, which would otherwise gather
// the side-effect-free matrix instructions ahead of the first fence or move
// them past the uniform rescale branches.)
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }
// Results passed through pin_out must exist at that point (an empty asm
// statement), so a fenced region's vector work stays inside it.
__device__ __forceinline__ void pin_out(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin_out(float& v) { asm volatile("" : "+v"(v)); }

// One P~V matrix instruction of query tile u: channel tile n < D/16, or
// (n == D/16, PNQ modes) the denominator against an all-ones operand.
template <int D, int PNQ>
__device__ __forceinline__ void pv_one(WaveState<D>& w, int u, int n, const uint4& pop, int X,
                                       const VOps<D>& vv) {
  constexpr int NT = D / 16;
  if (n < NT) {
    w.oacc[u][n] = mfma_fp4_sel(vv.op[n], pop, w.oacc[u][n], vv.sc[n >> 2], n & 3, X);
  } else if (PNQ) {
    const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);
    w.lacc[u] = mfma_fp4<0>(ones, pop, w.lacc[u], 127, X);
  }
}
// Non-PNQ denominator: l = alpha l + sum of the unquantized p of the tile.
template <int D, int PNQ>
__device__ __forceinline__ void l_plain(WaveState<D>& w, int u, const TileStats& ts, float vsum) {
  if (!PNQ) w.lsum[u] = fmaf(w.lsum[u], ts.alpha, __builtin_amdgcn_ldexpf(vsum, ts.X - 127));
}
// One S^T matrix instruction: key subtile t of query tile with operand qop.
__device__ __forceinline__ void s_one(v4f (&s)[kSub], int t, const uint4 (&kop)[kSub], const uint2& ksc,
                                      const uint4& qop, int qsc, const v4f& cneg) {
  s[t] = mfma_fp4_sel(kop[t], qop, cneg, t < 4 ? ksc.x : ksc.y, t & 3, qsc);
}

// Steps 1 / 3: P~V of the other tile (NPV matrix instructions) beside the
// row max and block scales of tile u (a dependent chain of vector work).
template <int D, int UOS, int PNQ, int MASK>
__device__ __forceinline__ TileStats stats_step(WaveState<D>& w, int u, v4f (&s)[kSub], int lim, int uo,
                                               const uint4& pop, const TileStats& to, float vo,
                                               const VOps<D>& vv, float sl2) {
  constexpr int NT = D / 16;
  if (MASK) mask_tile(s, lim);
  fence();
  pv_one<D, PNQ>(w, uo, 0, pop, to.X, vv);
  float a[kSub];
#pragma unroll
  for (int t = 0; t < 4; ++t) a[t] = fmaxf(fmaxf(s[t][0], s[t][1]), s[t][2]);
#pragma unroll
  for (int t = 0; t < 4; ++t) pin_out(a[t]);
  fence();
  pv_one<D, PNQ>(w, uo, 1, pop, to.X, vv);
#pragma unroll
  for (int t = 4; t < 8; ++t) a[t] = fmaxf(fmaxf(s[t][0], s[t][1]), s[t][2]);
#pragma unroll
  for (int t = 4; t < 8; ++t) pin_out(a[t]);
  fence();
  pv_one<D, PNQ>(w, uo, 2, pop, to.X, vv);
  float b0 = fmaxf(fmaxf(a[0], a[1]), a[2]);
  float b1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
  float b2 = fmaxf(fmaxf(a[6], a[7]), s[0][3]);
  pin_out(b0);
  pin_out(b1);
  pin_out(b2);
  fence();
  pv_one<D, PNQ>(w, uo, 3, pop, to.X, vv);
  const float b3 = fmaxf(fmaxf(s[1][3], s[2][3]), s[3][3]);
  const float b4 = fmaxf(fmaxf(s[4][3], s[5][3]), s[6][3]);
  const float c0 = fmaxf(fmaxf(b0, b1), b2);
  const float c1 = fmaxf(fmaxf(b3, b4), s[7][3]);
  float bmax = fmaxf(c0, c1);
  pin_out(bmax);
  fence();
  if (NT > 4) pv_one<D, PNQ>(w, uo, 4, pop, to.X, vv);
  // across the four lanes holding this query
  auto x1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
  float r1 = fmaxf(__uint_as_float(x1[0]), __uint_as_float(x1[1]));
  pin_out(r1);
  fence();
  if (NT > 5) pv_one<D, PNQ>(w, uo, 5, pop, to.X, vv);
  auto x2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(r1), __float_as_uint(r1), false, false);
  const float rowmax = fmaxf(__uint_as_float(x2[0]), __uint_as_float(x2[1]));
  // delta = new max - mref.  Before the first tile the running max is -inf
  // (m - mref = -inf); afterwards m == mref, so delta = max(0, rowmax d).
  float delta = fmaxf(w.m[u] - w.mref[u], rowmax);
  pin_out(delta);
  fence();
  if (NT > 6) pv_one<D, PNQ>(w, uo, 6, pop, to.X, vv);
  TileStats r;
  r.alpha = __builtin_amdgcn_exp2f((w.m[u] - w.mref[u] - delta) * sl2);  // 0 at first
  w.m[u] = w.mref[u] + delta;
  w.mref[u] = w.m[u];
  // scale of this lane's P~ block (the block holding the row maximum gets
  // x = 0 exactly); log2 v = d*c - (delta*c + e) in the scaled domain
  const float x = (bmax - delta) * sl2;
  float e = PNQ == 2 ? efq_block_exp(x) : p_block_exp<UOS>(x);
  pin_out(e);
  fence();
  if (NT > 7) pv_one<D, PNQ>(w, uo, 7, pop, to.X, vv);
  r.X = static_cast<int>(e) + 127;
  r.kofs = PNQ == 2 ? kEfqBeta - 2.0f * fmaf(delta, sl2, e) : fmaf(delta, sl2, e);
  l_plain<D, PNQ>(w, uo, to, vo);
  fence();
  pv_one<D, PNQ>(w, uo, NT, pop, to.X, vv);
  fence();
  return r;
}

// Steps 2 / 4: S^T of query tile us (eight matrix instructions) beside P~
// of tile u (per score one FMA, one exp2, half an FP4 conversion).
template <int D, int PNQ>
__device__ __forceinline__ uint4 ptile_step(v4f (&sn)[kSub], const KOps<D>& kk, const uint4& qop, int qsc,
                                           float mref, const v4f (&s)[kSub], float sl2, float kofs,
                                           float& vsum) {
  const v4f cneg = {-mref, -mref, -mref, -mref};
  uint32_t pw[4];
  vsum = 0.0f;
  fence();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t b = 0;
    s_one(sn, 2 * q, kk.op, kk.sc, qop, qsc, cneg);
    p_half<PNQ, 0>(s, q, sl2, kofs, pw[q], b, vsum);
    pin_out(pw[q]);
    if (PNQ == 2) pin_out(b);
    if (!PNQ) pin_out(vsum);
    fence();
    s_one(sn, 2 * q + 1, kk.op, kk.sc, qop, qsc, cneg);
    p_half<PNQ, 1>(s, q, sl2, kofs, pw[q], b, vsum);
    pin_out(pw[q]);
    if (!PNQ) pin_out(vsum);
    fence();
  }
  return make_uint4(pw[0], pw[1], pw[2], pw[3]);
}

template <int D, int UOS, int PNQ, int DUMP, int MASK>
__device__ __forceinline__ void kv_step(WaveState<D>& w, Pipe<D, UOS, PNQ>& p, const uint8_t* st_cur,
                                        const uint8_t* st_next, const uint4 (&qop)[kQT], const int (&qsc)[kQT],
                                        const int (&qrow)[kQT], const int (&klim)[kQT], bool visit, int j0,
                                        int lane, float sl2, const MxAttnArgs& a, int64_t bh) {
  const int grp = lane >> 4;

  // ---- step 1: P~V of B (tile j-1) | stats of A (tile j).  At tile 0, P~
  // of B is all zero codes (alpha 1, sum 0): the products add nothing.
  p.tA = stats_step<D, UOS, PNQ, MASK>(w, 0, p.sA, klim[0] - (j0 + grp * 32), 1, p.pB, p.tB, p.vB, p.vv,
                                       sl2);
  rescale_o<D, PNQ>(w, 0, p.tA.alpha);

  // ---- step 2: S^T of B (tile j) | P~ of A (tile j); V~ of tile j
  read_v<D>(p.vv, st_cur, lane);
  p.pA = ptile_step<D, PNQ>(p.sB, p.kk, qop[1], qsc[1], w.mref[1], p.sA, sl2, p.tA.kofs, p.vA);
  dump_tile<DUMP>(a, bh, qrow[0], visit, j0, grp, p.pA, p.tA.X);

  // ---- step 3: P~V of A (tile j) | stats of B (tile j); K~ of tile j+1
  read_k<D>(p.kk, st_next, lane);
  p.tB = stats_step<D, UOS, PNQ, MASK>(w, 1, p.sB, klim[1] - (j0 + grp * 32), 0, p.pA, p.tA, p.vA, p.vv,
                                       sl2);
  rescale_o<D, PNQ>(w, 1, p.tB.alpha);

  // ---- step 4: S^T of A (tile j+1) | P~ of B (tile j)
  p.pB = ptile_step<D, PNQ>(p.sA, p.kk, qop[0], qsc[0], w.mref[0], p.sB, sl2, p.tB.kofs, p.vB);
  dump_tile<DUMP>(a, bh, qrow[1], visit, j0, grp, p.pB, p.tB.X);
}

template <int D, int UOS, int PNQ, int CAUSAL, int DUMP>
__global__ __launch_bounds__(kThreads, 2) void attn_mx_kernel(MxAttnArgs a, float sl2) {
  constexpr int IMG = img_bytes(D);
  // One LDS object per stage, so that the compiler can tell which stage a
  // read touches and wait only for the direct loads into that stage.
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[IMG];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[IMG];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[IMG];
  static_assert(kStages == 3, "one LDS object per stage");
  // stage of ring position i (a constant after unrolling)
  auto lds_stage = [&](int i) -> uint8_t* {
    const int r = i % kStages;
    return r == 0 ? lds0 : r == 1 ? lds1 : lds2;
  };
  constexpr int DC = D / 32;  // 32-element blocks per Q~ row
  constexpr int NT = D / 16;  // output channel tiles

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nqb = (a.Sq + kMxQTile - 1) / kMxQTile;
  // Workgroup -> (head, query tile).  Workgroups are dispatched round-robin
  // over the 8 XCDs (each with its own L2), workgroup i to XCD i % 8.  Each
  // XCD is given a contiguous run of a list of (KV group, query head of the
  // group, query tile or causal pair), so a KV head's K~/V~ tile images are fetched from
  // HBM by one XCD (two at a run boundary) instead of all eight.  With
  // per-sequence lengths the KV groups gg = b * Hkv + g are listed in the
  // order of (gg % 8, gg / 8): each XCD then holds groups of every batch
  // entry, which keeps the XCDs equally loaded when the entries' lengths
  // differ (with equal lengths the plain order is kept).
  // Causal: one workgroup takes the query tiles p and nqb-1-p of a head
  // (nqb+1 KV tiles in all, the longer one first), so every workgroup of a
  // head does the same work and the fixed cost per workgroup is spread over
  // twice the tiles.
  const int nslot = CAUSAL ? (nqb + 1) / 2 : nqb;  // workgroups per query head
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int gi = (nwg >> 3) * xcd + min(xcd, nwg & 7) + (static_cast<int>(blockIdx.x) >> 3);
  const int G = a.Hq / a.Hkv;
  const int per_group = G * nslot;
  const int ngroups = a.B * a.Hkv;
  const int pos = gi / per_group;  // position of the KV group in that order
  const int rem = gi - pos * per_group;
  int gg = pos;
  if (a.lens_k) {
    int res = 0, first = 0;
    for (; res < 7; ++res) {
      const int cnt = (ngroups - res + 7) >> 3;  // groups with gg % 8 == res
      if (pos < first + cnt) break;
      first += cnt;
    }
    gg = res + 8 * (pos - first);
  }
  const int b = gg / a.Hkv;
  const int g = gg - b * a.Hkv;
  const int h = g * G + rem / nslot;
  const int slot = rem % nslot;
  const int njobs = (CAUSAL && 2 * slot + 1 != nqb) ? 2 : 1;
  const int col = lane & 15;   // query column within a 16-query tile
  const int grp = lane >> 4;   // K-block / lane group

  const int64_t bh = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t bg = static_cast<int64_t>(b) * a.Hkv + g;

  // This sequence's query rows and keys: the padded extents, or its own
  // lengths.  A sequence in which no row sees a key writes nothing.
  // (the lengths are read with vector loads; readfirstlane keeps them, and
  // every bound derived from them, in scalar registers and uniform branches)
  int sq = a.Sq, skv = a.Skv;
  if (a.lens_k) {
    skv = min(max(__builtin_amdgcn_readfirstlane(a.lens_k[b]), 0), a.Skv);
    sq = min(max(__builtin_amdgcn_readfirstlane(a.lens_q[b]), 0), a.Sq);
    if (skv == 0 || (CAUSAL && sq > skv)) sq = 0;
  }
  const int koff = CAUSAL ? skv - sq : 0;  // causal: row i sees keys j <= i + koff

  for (int job = 0; job < njobs; ++job) {
    // the query tile of this job (causal: the longer one first)
    const int qb = CAUSAL ? (job == 0 ? nqb - 1 - slot : slot) : slot;
    const int q0 = qb * kMxQTile;
    const int qw0 = q0 + wave * (kQT * 16);  // first query row of this wave
    if (q0 >= sq) continue;  // whole workgroup (uniform), before any barrier of the job
    // every wave is done with the previous job's stages before they refill
    if (job > 0) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }

    // Q~ operands (B of S^T): query column `col`, d-block `grp`, quantized
    // here; rows past the sequence (and d-blocks past D) are zero codes.
    uint4 qop[kQT];
    int qsc[kQT];
    int qrow[kQT];
#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      qrow[t] = qw0 + t * 16 + col;
      qop[t] = make_uint4(0, 0, 0, 0);
      qsc[t] = 127;
      if (grp < DC && qrow[t] < sq)
        quant_q_block<D, UOS, DUMP>(a, bh * a.Sq + qrow[t], grp, qop[t], qsc[t]);
    }

    WaveState<D> w;
#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      w.m[t] = -INFINITY;
      w.mref[t] = 0.0f;
      w.lsum[t] = 0.0f;
      w.lacc[t] = v4f{0, 0, 0, 0};
#pragma unroll
      for (int n = 0; n < NT; ++n) w.oacc[t][n] = v4f{0, 0, 0, 0};
    }

    const int nt = static_cast<int>(a.skv_ld / kKvTile);  // tiles per (b, KV head) image run
    const int ntk = (skv + kKvTile - 1) / kKvTile;          // tiles holding this sequence's keys
    // tiles this workgroup visits: all, or up to its last causal diagonal tile
    const int ntiles = CAUSAL ? min(ntk, (q0 + kMxQTile - 1 + koff) / kKvTile + 1) : ntk;
    // Tiles [0, nmain) are unmasked for every wave (whole tiles at or below
    // the first row's limit); the rest are computed masked.  A wave dumps P~
    // only up to its own last tile (the sequence end, or the causal limit of
    // its last row); a wave whose rows all lie past the sequence dumps none.
    const int nmain = CAUSAL ? min((q0 + koff + 1) / kKvTile, skv / kKvTile) : skv / kKvTile;
    const int last_w = qw0 >= sq ? -1 : (CAUSAL ? min((qw0 + kQT * 16 - 1 + koff) / kKvTile, ntk - 1) : ntk - 1);
    int klim[kQT];
#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      klim[t] = CAUSAL ? min(skv - 1, qrow[t] + koff) : skv - 1;
      if (qrow[t] >= sq) qrow[t] = a.Sq;  // past the sequence: never dumped or stored
    }

    // wave-uniform (the divisions above run on the vector unit): scalar
    // registers, so the tile loads take the scalar-base form
    const uint8_t* img = uniform_ptr(a.img + bg * nt * static_cast<int64_t>(IMG));
    const int nl = loads_per_tile<D>(wave);

    // Ring of kStages LDS stages: tile jt lives in stage jt % kStages.  Tiles 0
    // and 1 are requested up front, and S^T of A for tile 0 is formed once
    // tile 0 has landed.  At the top of iteration jt the wave waits for all
    // its loads (those of tile jt+1, requested an iteration earlier); the
    // barrier then makes every wave's loads visible and tells that every wave
    // has finished iteration jt-1, the last to read the stage of tile jt-1
    // (its V~, in step 2), which the loads of tile jt+2 then refill.
    issue_tile<D>(lds0, img, wave, lane);
    if (ntiles > 1) {
      issue_tile<D>(lds1, img + IMG, wave, lane);
      if (nl == 5) wait_vmcnt<5>(); else if (nl == 4) wait_vmcnt<4>(); else wait_vmcnt<3>();
    } else {
      wait_vmcnt<0>();
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    Pipe<D, UOS, PNQ> p;
    // P~ of B before tile 0: zero codes under scale 1 against zero V~ operands
    p.pB = make_uint4(0, 0, 0, 0);
    p.tB.alpha = 1.0f;
    p.tB.kofs = 0.0f;
    p.tB.X = 127;
    p.vA = 0.0f;
    p.vB = 0.0f;
#pragma unroll
    for (int n = 0; n < NT; ++n) p.vv.op[n] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int n = 0; n < (NT + 3) / 4; ++n) p.vv.sc[n] = 0x7F7F7F7Fu;
    read_k<D>(p.kk, lds0, lane);
    s_tile(p.sA, p.kk.op, p.kk.sc, qop[0], qsc[0], w.mref[0]);

    // tiles [0, nmain): no key masked; the ring position of each is a
    // compile-time constant (the loop is unrolled by the stage count)
    for (int jb = 0; jb < nmain; jb += kStages) {
#pragma unroll
      for (int k = 0; k < kStages; ++k) {
        const int jt = jb + k;
        if (jt < nmain) {
          wait_vmcnt<0>();
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          if (jt + 2 < ntiles)
            issue_tile<D>(lds_stage(k + 2), img + static_cast<int64_t>(jt + 2) * IMG, wave, lane);
          kv_step<D, UOS, PNQ, DUMP, 0>(w, p, lds_stage(k), lds_stage(k + 1), qop, qsc, qrow, klim,
                                        jt <= last_w, jt * kKvTile, lane, sl2, a, bh);
        }
      }
    }
    // tiles [nmain, ntiles): the sequence end or the causal diagonal (one or
    // two tiles), keys masked per row; stages picked at run time
    for (int jt = nmain; jt < ntiles; ++jt) {
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (jt + 2 < ntiles)
        issue_tile<D>(lds_stage(jt + 2), img + static_cast<int64_t>(jt + 2) * IMG, wave, lane);
      // every load of the ring has landed here except tile jt+2's, which
      // targets neither stage read below
      kv_step<D, UOS, PNQ, DUMP, 1>(w, p, lds_stage(jt), lds_stage(jt + 1), qop, qsc, qrow, klim,
                                    jt <= last_w, jt * kKvTile, lane, sl2, a, bh);
    }
    // P~V of B for the last tile (its V~ still in registers)
#pragma unroll
    for (int n = 0; n <= NT; ++n) pv_one<D, PNQ>(w, 1, n, p.pB, p.tB.X, p.vv);
    l_plain<D, PNQ>(w, 1, p.tB, p.vB);

    // The epilogue stores under a per-lane condition.  Pin the accumulators
    // here so that the matrix-core instructions producing them are not moved
    // into that divergent region: an MFMA issued with part of EXEC disabled
    // would drop the operands of the disabled lanes, which other lanes' results
    // depend on.
#pragma unroll
    for (int u = 0; u < kQT; ++u) {
#pragma unroll
      for (int n = 0; n < NT; ++n) asm volatile("" : "+v"(w.oacc[u][n]));
      asm volatile("" : "+v"(w.lacc[u]));
    }

    // ---- epilogue: O = O_acc / l ----
#pragma unroll
    for (int u = 0; u < kQT; ++u) {
      const float l = PNQ ? w.lacc[u][0] : xlane_sum4(w.lsum[u]);
      const float inv = 1.0f / l;
      if (qrow[u] < a.Sq) {
        float* orow = a.o + (bh * a.Sq + qrow[u]) * D;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          float4 v = make_float4(w.oacc[u][n][0] * inv, w.oacc[u][n][1] * inv, w.oacc[u][n][2] * inv,
                                 w.oacc[u][n][3] * inv);
          *reinterpret_cast<float4*>(orow + n * 16 + grp * 4) = v;
        }
      }
    }
  }  // job
}

template <int D, int UOS, int PNQ, int CAUSAL, int DUMP>
hipError_t launch_t(const MxAttnArgs& a, hipStream_t s) {
  const int nqb = (a.Sq + kMxQTile - 1) / kMxQTile;
  // causal: query tiles in pairs (see attn_mx_kernel)
  dim3 grid(static_cast<unsigned>(CAUSAL ? (nqb + 1) / 2 : nqb) * a.Hq * a.B);
  const float sl2 = static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(D)));
  hipLaunchKernelGGL((attn_mx_kernel<D, UOS, PNQ, CAUSAL, DUMP>), grid, dim3(kThreads), 0, s, a, sl2);
  return hipGetLastError();
}

template <int D, int UOS, int PNQ, int CAUSAL>
hipError_t pick_dump(const MxAttnArgs& a, hipStream_t s) {
  return a.row_slot ? launch_t<D, UOS, PNQ, CAUSAL, 1>(a, s) : launch_t<D, UOS, PNQ, CAUSAL, 0>(a, s);
}
template <int D, int UOS, int PNQ>
hipError_t pick_causal(const MxAttnArgs& a, hipStream_t s) {
  return a.causal ? pick_dump<D, UOS, PNQ, 1>(a, s) : pick_dump<D, UOS, PNQ, 0>(a, s);
}
template <int D>
hipError_t pick_mode(const MxAttnArgs& a, hipStream_t s) {
  switch (a.mode) {
    case 1: return pick_causal<D, 0, 0>(a, s);
    case 2: return pick_causal<D, 1, 0>(a, s);
    case 3: return pick_causal<D, 1, 1>(a, s);
    default: return pick_causal<D, 1, 2>(a, s);
  }
}

// ---- short-query attention over key splits ----------------------------
//
// One wave per (b, KV head g, split): its 16 query columns are the G x Sq
// queries of the GQA group (column c = h_local * Sq + i, G * Sq <= 16),
// so the group's K~/V~ are read once per split.  The wave runs the same
// tile step as above (S^T on the matrix core with -m as accumulator input,
// block scales, P~, O^T += V~^T P~^T) over the split's KV tiles, with its
// own running max from -inf, reading the tile images straight from global
// memory into the operand registers (nothing is shared between waves), the
// next tile's loads in flight during the current tile.  It leaves (m, l,
// unnormalized O) per query column; the merge kernel combines the splits
// in ascending order.  Columns with no visible key in the split leave
// m = -inf, l = 0, O = 0.
template <int D>
struct TileOps {
  uint4 kop[kSub];
  uint2 ksc;
  uint4 vop[D / 16];
  uint32_t vsc[(D / 16 + 3) / 4];
};

template <int D>
__device__ __forceinline__ void load_tile_ops(TileOps<D>& t, const uint8_t* st, int lane) {
  constexpr int NT = D / 16;
#pragma unroll
  for (int i = 0; i < kSub; ++i) t.kop[i] = *reinterpret_cast<const uint4*>(st + kImgKc + i * 1024 + lane * 16);
  t.ksc = *reinterpret_cast<const uint2*>(st + img_ks(D) + lane * 8);
#pragma unroll
  for (int n = 0; n < NT; ++n) t.vop[n] = *reinterpret_cast<const uint4*>(st + kImgVc + n * 1024 + lane * 16);
  if (NT == 8) {
    const uint2 v2 = *reinterpret_cast<const uint2*>(st + img_vs(D) + lane * 8);
    t.vsc[0] = v2.x;
    t.vsc[(NT + 3) / 4 - 1] = v2.y;
  } else {
    t.vsc[0] = *reinterpret_cast<const uint32_t*>(st + img_vs(D) + lane * 4);
  }
}

// Splits of entry b: its keys in spans of split_tiles tiles (0 for an entry
// with no key).
__device__ __forceinline__ int entry_splits(const MxDecodeArgs& d, int b) {
  const int span = d.split_tiles * kKvTile;
  const int skv = min(max(d.at.lens_k[b], 0), d.at.Skv);
  return (skv + span - 1) / span;
}

// Per-sequence lengths: the (entry, KV head, split) units that hold keys,
// numbered consecutively (entry, then KV head, then split).  Consecutive
// waves then take equal work whatever the lengths, and the round-robin of
// workgroups over the XCDs spreads it evenly (numbering every split of the
// padded extent instead puts split s of every group on the same XCD, and the
// splits that hold keys are the low ones).  The wave walks the entries 64 at
// a time (B <= kCompactMaxB), one entry per lane, and a wave-wide prefix sum
// of their unit counts locates unit u.  Returns false when u is past the
// last unit.  (A rolled loop: unrolled, its exits cost the tile loop
// registers.)
__device__ bool busy_unit(const MxDecodeArgs& d, int u, int& b, int& g, int& sp) {
  const int lane = threadIdx.x & 63;
  int base = 0;
#pragma unroll 1
  for (int c0 = 0; c0 < d.at.B; c0 += 64) {
    const int ns = c0 + lane < d.at.B ? entry_splits(d, c0 + lane) : 0;
    int incl = ns * d.at.Hkv;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const int tot = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
    if (u < base + tot) {
      const int l = __builtin_ctzll(__ballot(base + incl > u));
      const int n = __builtin_amdgcn_readfirstlane(__shfl(ns, l));
      const int local = u - (base + __builtin_amdgcn_readfirstlane(__shfl(incl, l)) - n * d.at.Hkv);
      b = c0 + l;
      g = local / n;
      sp = local - g * n;
      return true;
    }
    base += tot;
  }
  return false;
}

template <int D, int UOS, int PNQ, int DUMP, int COMPACT>
__global__ __launch_bounds__(kThreads, 2) void attn_decode_kernel(MxDecodeArgs d, float sl2) {
  const MxAttnArgs& a = d.at;
  constexpr int IMG = img_bytes(D);
  constexpr int NT = D / 16;
  constexpr int DC = D / 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  int b, g, sp;
  // (a compile-time choice: the scan left in the other form's code costs it
  // registers in the tile loop)
  if constexpr (COMPACT) {
    if (!busy_unit(d, static_cast<int>(unit), b, g, sp)) return;  // whole wave; no barriers here
  } else {
    const int64_t nunits = static_cast<int64_t>(a.B) * a.Hkv * d.nsplit;
    if (unit >= nunits) return;
    sp = static_cast<int>(unit % d.nsplit);
    b = static_cast<int>(unit / d.nsplit / a.Hkv);
    g = static_cast<int>(unit / d.nsplit % a.Hkv);
  }
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  sp = __builtin_amdgcn_readfirstlane(sp);
  const int64_t bg = static_cast<int64_t>(b) * a.Hkv + g;
  const int64_t slot = bg * d.nsplit + sp;  // partial-state slot
  const int G = a.Hq / a.Hkv;
  const int col = lane & 15, grp = lane >> 4;

  // query of this column; unused columns multiply zero codes and see every key
  const bool cvalid = col < G * a.Sq;
  const int hl = cvalid ? col / a.Sq : 0, qi = cvalid ? col % a.Sq : 0;
  const int64_t bh = static_cast<int64_t>(b) * a.Hq + g * G + hl;
  uint4 qop = make_uint4(0, 0, 0, 0);
  int qsc = 127;
  if (cvalid && grp < DC) {
    // every split of a group quantizes the same rows; split 0 dumps them
    if (DUMP && sp == 0)
      quant_q_block<D, UOS, 1>(a, bh * a.Sq + qi, grp, qop, qsc);
    else
      quant_q_block<D, UOS, 0>(a, bh * a.Sq + qi, grp, qop, qsc);
  }
  // this sequence's keys: the padded extent, or its own length
  const int skv = a.lens_k ? min(max(__builtin_amdgcn_readfirstlane(a.lens_k[b]), 0), a.Skv) : a.Skv;
  // causal: end-aligned; a row with no visible key (klim < 0) stays empty
  const int klim = (cvalid && a.causal) ? qi + (skv - a.Sq) : skv - 1;
  const int qrow = cvalid ? qi : a.Sq;  // rows >= Sq are never dumped

  const int nt = static_cast<int>(a.skv_ld / kKvTile);  // tiles per (b, KV head) image run
  const int ntk = (skv + kKvTile - 1) / kKvTile;          // tiles holding this sequence's keys
  const int t_begin = sp * d.split_tiles;
  const int t_end = min(t_begin + d.split_tiles, ntk);
  // tiles needing the per-key mask: past the key end, or past the first
  // causal limit (skv - Sq)
  const int first_masked = a.causal ? max(skv - a.Sq, 0) / kKvTile : skv / kKvTile;

  WaveState<D> w;
  w.m[0] = -INFINITY;
  w.mref[0] = 0.0f;
  w.lsum[0] = 0.0f;
  w.lacc[0] = v4f{0, 0, 0, 0};
#pragma unroll
  for (int n = 0; n < NT; ++n) w.oacc[0][n] = v4f{0, 0, 0, 0};

  const uint8_t* img = a.img + bg * nt * static_cast<int64_t>(IMG);
  TileOps<D> cur, nxt;
  if (t_begin < t_end) load_tile_ops<D>(cur, img + static_cast<int64_t>(t_begin) * IMG, lane);
  for (int t = t_begin; t < t_end; ++t) {
    if (t + 1 < t_end) load_tile_ops<D>(nxt, img + static_cast<int64_t>(t + 1) * IMG, lane);
    const int j0 = t * kKvTile;
    v4f s[kSub];
    s_tile(s, cur.kop, cur.ksc, qop, qsc, w.mref[0]);
    if (t >= first_masked) mask_tile(s, klim - (j0 + grp * 32));
    const TileStats ts = tile_stats<D, UOS, PNQ>(w, 0, s, sl2);
    float vsum;
    const uint4 pop = p_tile<PNQ>(s, sl2, ts.kofs, vsum);
    dump_tile<DUMP>(a, bh, qrow, j0 <= klim, j0, grp, pop, ts.X);
    pv_tile<D, PNQ>(w, 0, pop, ts, vsum, cur.vop, cur.vsc);
    if (t + 1 < t_end) cur = nxt;
  }

  // pin the accumulators ahead of the per-lane stores (see attn_mx_kernel)
#pragma unroll
  for (int n = 0; n < NT; ++n) asm volatile("" : "+v"(w.oacc[0][n]));
  asm volatile("" : "+v"(w.lacc[0]));
  const float l = PNQ ? w.lacc[0][0] : xlane_sum4(w.lsum[0]);
  const bool empty = klim < t_begin * kKvTile;  // no visible key in this split
  if (cvalid) {  // unused columns are never merged
    float* pr = d.part + (slot * 16 + col) * (D + 2);
    if (grp == 0) {
      pr[0] = empty ? -INFINITY : w.m[0];
      pr[1] = empty ? 0.0f : l;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const v4f v = empty ? v4f{0, 0, 0, 0} : w.oacc[0][n];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[2 + 16 * n + 4 * grp + r] = v[r];
    }
  }
}

// One wave per query row: O = sum_s 2^((m_s - M) c) O_s / sum_s 2^((m_s - M) c) l_s,
// M the largest m_s, splits in ascending order.  The partial outputs of the
// first kMergeChunk splits are loaded together with the splits' (m, l), so a
// row costs one memory round trip when nsplit <= kMergeChunk; the lanes take
// (m, l) in parallel (wave max and sum) and leave each split's weight in
// LDS; each lane then accumulates its channels over the splits in order.
constexpr int kMaxSplits = 1024;
constexpr int kMergeChunk = 32;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void attn_decode_merge_kernel(MxDecodeArgs d, float sl2) {
  __shared__ float wts[4][kMaxSplits];
  const MxAttnArgs& a = d.at;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wv;  // (b*Hq + h)*Sq + i
  if (row >= static_cast<int64_t>(a.B) * a.Hq * a.Sq) return;  // whole wave; no block barrier
  const int i = static_cast<int>(row % a.Sq);
  const int64_t bh = row / a.Sq;
  const int h = static_cast<int>(bh % a.Hq), b = static_cast<int>(bh / a.Hq);
  const int G = a.Hq / a.Hkv;
  const int64_t bg = static_cast<int64_t>(b) * a.Hkv + h / G;
  const int col = (h % G) * a.Sq + i;
  const float* base = d.part + (bg * d.nsplit * 16 + col) * (D + 2);
  const int64_t stride = 16 * static_cast<int64_t>(D + 2);
  // per-sequence lengths: only the splits that hold the entry's keys were written
  const int ns = a.lens_k ? __builtin_amdgcn_readfirstlane(entry_splits(d, b)) : d.nsplit;
  constexpr int PER = D / 64;
  const int n0 = min(ns, kMergeChunk);
  float o0[kMergeChunk][PER];
#pragma unroll
  for (int u = 0; u < kMergeChunk; ++u)
#pragma unroll
    for (int k = 0; k < PER; ++k) o0[u][k] = u < n0 ? base[u * stride + 2 + lane + 64 * k] : 0.0f;
  float ms = -INFINITY, ls = 0.0f;
  if (lane < ns) {
    ms = base[lane * stride];
    ls = base[lane * stride + 1];
  }
  float M = ms;
  for (int s = lane + 64; s < ns; s += 64) M = fmaxf(M, base[s * stride]);
  M = wave_max(M);
  if (M == -INFINITY) return;  // no split saw a key: the row is left unwritten
  float L = 0.0f;
  if (lane < ns) {
    const float wgt = __builtin_amdgcn_exp2f((ms - M) * sl2);  // 0 when the split is empty
    wts[wv][lane] = wgt;
    L = fmaf(wgt, ls, L);
  }
  for (int s = lane + 64; s < ns; s += 64) {
    const float wgt = __builtin_amdgcn_exp2f((base[s * stride] - M) * sl2);
    wts[wv][s] = wgt;
    L = fmaf(wgt, base[s * stride + 1], L);
  }
  L = wave_sum(L);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
#pragma unroll
  for (int u = 0; u < kMergeChunk; ++u) {
    if (u < n0) {
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] = fmaf(wts[wv][u], o0[u][k], acc[k]);
    }
  }
  int s = kMergeChunk;
  for (; s + 8 <= ns; s += 8) {
    float o[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int k = 0; k < PER; ++k) o[u][k] = base[(s + u) * stride + 2 + lane + 64 * k];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] = fmaf(wts[wv][s + u], o[u][k], acc[k]);
  }
  for (; s < ns; ++s)
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = fmaf(wts[wv][s], base[s * stride + 2 + lane + 64 * k], acc[k]);
  const float inv = 1.0f / L;
#pragma unroll
  for (int k = 0; k < PER; ++k) a.o[row * D + lane + 64 * k] = acc[k] * inv;
}

template <int D, int UOS, int PNQ, int DUMP, int COMPACT>
hipError_t launch_decode_t(const MxDecodeArgs& d, hipStream_t s) {
  const float sl2 = static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(D)));
  const int64_t nunits = static_cast<int64_t>(d.at.B) * d.at.Hkv * d.nsplit;
  hipLaunchKernelGGL((attn_decode_kernel<D, UOS, PNQ, DUMP, COMPACT>), dim3(static_cast<unsigned>((nunits + kWaves - 1) / kWaves)),
                     dim3(kThreads), 0, s, d, sl2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = static_cast<int64_t>(d.at.B) * d.at.Hq * d.at.Sq;
  hipLaunchKernelGGL((attn_decode_merge_kernel<D>), dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, s,
                     d, sl2);
  return hipGetLastError();
}

template <int D, int UOS, int PNQ>
hipError_t decode_pick_dump(const MxDecodeArgs& d, hipStream_t s) {
  if (d.compact)
    return d.at.row_slot ? launch_decode_t<D, UOS, PNQ, 1, 1>(d, s) : launch_decode_t<D, UOS, PNQ, 0, 1>(d, s);
  return d.at.row_slot ? launch_decode_t<D, UOS, PNQ, 1, 0>(d, s) : launch_decode_t<D, UOS, PNQ, 0, 0>(d, s);
}
template <int D>
hipError_t decode_pick_mode(const MxDecodeArgs& d, hipStream_t s) {
  switch (d.at.mode) {
    case 1: return decode_pick_dump<D, 0, 0>(d, s);
    case 2: return decode_pick_dump<D, 1, 0>(d, s);
    case 3: return decode_pick_dump<D, 1, 1>(d, s);
    default: return decode_pick_dump<D, 1, 2>(d, s);
  }
}

}  // namespace

hipError_t launch_attn_mx(const MxAttnArgs& a, hipStream_t stream) {
  return a.D == 64 ? pick_mode<64>(a, stream) : pick_mode<128>(a, stream);
}

hipError_t launch_attn_decode(const MxDecodeArgs& d, hipStream_t stream) {
  return d.at.D == 64 ? decode_pick_mode<64>(d, stream) : decode_pick_mode<128>(d, stream);
}

}  // namespace mxk
