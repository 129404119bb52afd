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
// Mapping onto v_mfma_scale_f32_32x32x64_f8f6f4 (FP4 x FP4, fp32 accum): an
// operand lane l holds row (l % 32) and the 32 K-elements of K-block (l / 32)
// plus that block's E8M0 scale (one byte of a register, picked by the
// instruction's op_sel); the accumulator lane l, register r holds row
// 8 (r/4) + 4 (l/32) + r%4, column l % 32.
//  * S^T = K~ Q~^T: A = 32 keys x 64 d, B = 64 d x 32 queries; D/64
//    instructions per 32-key subtile.  The 32 A-rows of subtile t (0..3) of a
//    128-key tile are keys chosen (in the quantizer's image order) so that
//    accumulator lane l holds, over the subtiles 2s and 2s+1, exactly the 32
//    keys 64 s + 32 (l/32) + 0..31 in register order: one whole P~ block of
//    query l % 32.  Block maxima and the FP4 packing stay in-lane; the row
//    max needs one swap between the two lane halves.
//  * O^T = V~^T P~^T: A = 32 channels x 64 keys, B = P~ (64 keys x 32
//    queries) straight from the registers above, with the lane's own block
//    scale.  The accumulator keeps query l % 32 in every register of a lane,
//    matching the softmax state.
//  * Under PNQ the denominator is one v_mfma_scale_f32_16x16x128_f8f6f4 per
//    64 keys with the same P~ register as B and a constant A that is 1.0
//    where (A-row / 4) and the K-block have the same parity and 0 elsewhere:
//    output lane l then receives the sum over the 64 keys of query l % 32.
// Q is quantized in the kernel's prologue: each lane holds whole 32-element
// blocks of its query row (the B operand layout), so it applies the block
// rule of the mode to the raw bf16/fp32 elements it loads (mx_block.h, the
// same code as the standalone quantizer).
// The quantizer writes K~ and V~ as KV tile images already in these operand
// orders, so a tile moves to LDS with contiguous 16-byte-per-lane direct
// loads and every operand read is one ds_read per lane.
//
// P~ is formed in the scaled domain: for a block with scale exponent e,
// v = exp2((s - m) * log2(e)/sqrt(D) - e) is rounded by
// v_cvt_scalef32_pk_fp4_f32 (round to nearest even, saturating).  This keeps
// blocks whose probabilities lie below fp32's normal range exact in the same
// way the binary64 definition treats them.  The UOS+EFQ mode skips the exp:
// the code of each score is an affine function of its log2 residual to the
// block's exponent, rounded and clamped by v_cvt_pk_u8_f32.
#include "internal.h"
#include "mx_block.h"

namespace mxk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 32;              // query rows per wave (one 32-column tile)
constexpr int kSub = kKvTile / 32;   // 32-key subtiles per KV tile (4)
constexpr int kStages = 4;           // LDS ring of KV tile images
static_assert(kMxQTile == kWaves * kQW, "query tile = waves x 32");
static_assert(kMxQTile % kKvTile == 0, "query tiles start on KV tile boundaries");
static_assert(kDecodeCols == kQW, "short-query waves use one 32-column tile");

template <int SA, int SB>
__device__ __forceinline__ v16f mfma32_t(const uint4& a, const uint4& b, const v16f& c, uint32_t sa, uint32_t sb) {
  const v8i av = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z),
                  static_cast<int>(a.w), 0, 0, 0, 0};
  const v8i bv = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z),
                  static_cast<int>(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, SA, static_cast<int>(sa), SB,
                                                         static_cast<int>(sb));
}
// A-scale from byte `sel` of `sa` (a constant after unrolling), B-scale from
// byte SB of `sb`.
template <int SB>
__device__ __forceinline__ v16f mfma32(const uint4& a, const uint4& b, const v16f& c, uint32_t sa, int sel,
                                       uint32_t sb) {
  switch (sel) {
    case 0: return mfma32_t<0, SB>(a, b, c, sa, sb);
    case 1: return mfma32_t<1, SB>(a, b, c, sa, sb);
    case 2: return mfma32_t<2, SB>(a, b, c, sa, sb);
    default: return mfma32_t<3, SB>(a, b, c, sa, sb);
  }
}
// PNQ denominator: the 16x16x128 product of the lane-parity ones operand
// `ones` with a P~ register (B-scale: the lane's block byte).
__device__ __forceinline__ v4f mfma_rowsum(uint32_t ones, const uint4& b, const v4f& c, uint32_t sb) {
  const v8i av = {static_cast<int>(ones), static_cast<int>(ones), static_cast<int>(ones),
                  static_cast<int>(ones), 0, 0, 0, 0};
  const v8i bv = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z),
                  static_cast<int>(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, 127, 0, static_cast<int>(sb));
}
// The ones operand of lane l: A-row l%16, K-block l/16; 1.0 (E2M1 code 2 in
// every nibble) where ((l%16)/4) % 2 == (l/16) % 2.  Output row 4(l/16)+r
// then sums the K-blocks of its own parity, i.e. the lanes l%16 + 16 p and
// l%16 + 16 p + 32 of the P~ operand (p = (l/16) % 2): both hold query l % 32.
__device__ __forceinline__ uint32_t rowsum_ones(int lane) {
  return (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 0x22222222u : 0u;
}

// max over the lanes l and l ^ 32 (same query)
__device__ __forceinline__ float xhalf_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
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

// Per-wave softmax state and accumulators of one 32-query tile.
template <int D>
struct WaveState {
  v16f oacc[D / 32];
  v4f lacc;       // PNQ denominator (element 0 is kept rescaled)
  v16f cneg;      // -mref in every element: the accumulator input of S^T
  float m;        // running row max (raw score units), -inf before the first tile
  float mref;     // value subtracted from S on the matrix core
  float lsum;     // non-PNQ denominator (this lane's blocks)
};

template <int D>
__device__ __forceinline__ void init_state(WaveState<D>& w) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) w.oacc[c][r] = 0.0f;
  w.lacc = v4f{0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < 16; ++r) w.cneg[r] = 0.0f;
  w.m = -INFINITY;
  w.mref = 0.0f;
  w.lsum = 0.0f;
}

// s_waitcnt on the vector-memory counter only (expcnt, lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at max).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// A wave-uniform address kept in scalar registers, so that a direct load
// takes the scalar-base + 32-bit lane-offset form (one VGPR per lane for
// every load instead of a 64-bit address each).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Direct loads of 1 KiB rows of a KV tile image into an LDS stage: rows
// r0, r0 + step, ... below the image's row count, lane l bytes
// [16 l, 16 l + 16) of each.  Buffer loads (a raw resource over the image,
// no range check), not the global form: with a global load-to-LDS in
// flight the compiler turns every LDS wait into a full lgkmcnt(0), so each
// operand read would also wait for the reads issued after it.
template <int D, int STEP>
__device__ __forceinline__ void issue_rows(uint8_t* stage, const uint8_t* src, int r0, int lane) {
  constexpr int NL = img_bytes(D) / 1024;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(uniform_ptr(src)), 0, 0xFFFFFFFFu, 0x00020000);
  const uint32_t lo = static_cast<uint32_t>(lane) * 16u;
#pragma unroll
  for (int i = 0; i < (NL + STEP - 1) / STEP; ++i) {
    const int row = r0 + i * STEP;
    if (row < NL) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, stage + row * 1024, 16, lo, row * 1024, 0, 0);
  }
}
// A workgroup's share: wave w moves rows w, w + kWaves, ...
template <int D>
__device__ __forceinline__ void issue_tile(uint8_t* stage, const uint8_t* src, int wave, int lane) {
  issue_rows<D, kWaves>(stage, src, wave, lane);
}
// Loads this wave issues per tile.
template <int D>
__device__ __forceinline__ int loads_per_tile(int wave) {
  constexpr int NL = img_bytes(D) / 1024;
  return NL / kWaves + (wave < NL % kWaves ? 1 : 0);
}

// ---- operand reads from an LDS stage ---------------------------------------
// E8M0 bytes of one lane: D/16 per image part (8 or 4), as 32-bit words.
template <int D>
struct Sc {
  uint32_t w[(D / 16 + 3) / 4];
};
template <int D>
__device__ __forceinline__ Sc<D> read_sc(const uint8_t* st, int off, int lane) {
  Sc<D> s;
  if (D == 128) {
    const uint2 v = *reinterpret_cast<const uint2*>(st + off + lane * 8);
    s.w[0] = v.x;
    s.w[(D / 16 + 3) / 4 - 1] = v.y;
  } else {
    s.w[0] = *reinterpret_cast<const uint32_t*>(st + off + lane * 4);
  }
  return s;
}
// K~ operand of (subtile t, d-half i); V~ operand of (channel tile c, key step s)
template <int D>
__device__ __forceinline__ uint4 k_op(const uint8_t* st, int t, int i, int lane) {
  return *reinterpret_cast<const uint4*>(st + kImgKc + (t * (D / 64) + i) * 1024 + lane * 16);
}
template <int D>
__device__ __forceinline__ uint4 v_op(const uint8_t* st, int c, int s, int lane) {
  return *reinterpret_cast<const uint4*>(st + img_vc(D) + (c * 2 + s) * 1024 + lane * 16);
}

// One S^T subtile t: d = S - mref, with -mref (the running max of the
// previous tiles, 0 before the first) as the accumulator input, so the
// subtraction happens inside the matrix core's accumulation and elements
// near the maximum keep their relative precision.
template <int D>
__device__ __forceinline__ v16f s_sub(int t, const uint4 (&kop)[D / 64], const Sc<D>& ksc,
                                      const uint4 (&qop)[D / 64], uint32_t qsc, const v16f& cneg);

// Contraction half I of S^T subtile t (accumulator input c).
template <int D, int I>
__device__ __forceinline__ v16f s_part(int t, const uint4& kop, const Sc<D>& ksc, const uint4 (&qop)[D / 64],
                                       uint32_t qsc, const v16f& c) {
  const int bi = t * (D / 64) + I;
  return mfma32<I>(kop, qop[I], c, ksc.w[bi >> 2], bi & 3, qsc);
}

template <int D>
__device__ __forceinline__ v16f s_sub(int t, const uint4 (&kop)[D / 64], const Sc<D>& ksc,
                                      const uint4 (&qop)[D / 64], uint32_t qsc, const v16f& cneg) {
  v16f r = s_part<D, 0>(t, kop[0], ksc, qop, qsc, cneg);
  if constexpr (D / 64 == 2) r = s_part<D, 1>(t, kop[1], ksc, qop, qsc, r);
  return r;
}

// Keys past `lim` (relative to the first key of this lane's blocks,
// 32 (l/32) into the tile) are excluded: register r of subtile t is key
// 64 (t/2) + 16 (t%2) + r past that.
__device__ __forceinline__ void mask_tile(v16f (&s)[kSub], int lim) {
  asm volatile("" : "+v"(lim));  // keeps the compares inside the caller's branch
#pragma unroll
  for (int t = 0; t < kSub; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[t][r] = (64 * (t >> 1) + 16 * (t & 1) + r > lim) ? -INFINITY : s[t][r];
}

// Online-softmax statistics of one tile: history factor alpha, the change
// delta of the reference max, and per P~ block s of this lane (keys
// 64 s + 32 (l/32) ..) its E8M0 byte X and the offset kofs of the scaled
// domain.
struct TileStats {
  float alpha, delta;
  float kofs[2];
  uint32_t X[2];
};

// First level of the block maxima: 10 v_max3 over 30 of a block's 32
// values (a = its first 16 keys, b = the next 16).
__device__ __forceinline__ void bmax_l1(const v16f& a, const v16f& b, float (&o)[10]) {
#pragma unroll
  for (int k = 0; k < 5; ++k) o[k] = fmaxf(fmaxf(a[3 * k], a[3 * k + 1]), a[3 * k + 2]);
  o[5] = fmaxf(fmaxf(a[15], b[0]), b[1]);
#pragma unroll
  for (int k = 0; k < 4; ++k) o[6 + k] = fmaxf(fmaxf(b[2 + 3 * k], b[3 + 3 * k]), b[4 + 3 * k]);
}
// Rest of the tree: the 10 values and b's last two to one (5 v_max3, one max).
__device__ __forceinline__ float bmax_l2(const float (&o)[10], const v16f& b) {
  const float p0 = fmaxf(fmaxf(o[0], o[1]), o[2]);
  const float p1 = fmaxf(fmaxf(o[3], o[4]), o[5]);
  const float p2 = fmaxf(fmaxf(o[6], o[7]), o[8]);
  const float p3 = fmaxf(fmaxf(o[9], b[14]), b[15]);
  return fmaxf(fmaxf(fmaxf(p0, p1), p2), p3);
}

// delta, alpha and the running max from the row max of this tile; then the
// scales of the lane's two blocks (block maxima b0, b1).
template <int UOS, int PNQ>
__device__ __forceinline__ float stats_delta(float& m, float& mref, float rowmax, float sl2, float& alpha) {
  // delta = new max - mref.  Before the first tile the running max is -inf
  // (m - mref = -inf); afterwards m == mref, so delta = max(0, rowmax d).
  const float delta = fmaxf(m - mref, rowmax);
  alpha = __builtin_amdgcn_exp2f((m - mref - delta) * sl2);  // 0 at the first tile
  m = mref + delta;
  mref = m;
  return delta;
}
template <int UOS, int PNQ>
__device__ __forceinline__ void block_scale(float bmax, float delta, float sl2, uint32_t& X, float& kofs) {
  // the block holding the row maximum gets x = 0 exactly; in the scaled
  // domain log2 v = (d - delta) * log2(e)/sqrt(D) - e = d*c - (delta*c + e)
  const float x = (bmax - delta) * sl2;
  const float e = PNQ == 2 ? efq_block_exp(x) : p_block_exp<UOS>(x);
  X = static_cast<uint32_t>(static_cast<int>(e) + 127);
  // EFQ: 2 r + beta = d * 2c + (beta - 2 (delta c + e)); else the exp2 offset
  kofs = PNQ == 2 ? kEfqBeta - 2.0f * fmaf(delta, sl2, e) : fmaf(delta, sl2, e);
}

// All statistics of a tile at once (the short-query kernel).
template <int UOS, int PNQ>
__device__ __forceinline__ TileStats tile_stats(float& m, float& mref, const v16f (&s)[kSub], float sl2) {
  float o0[10], o1[10];
  bmax_l1(s[0], s[1], o0);
  bmax_l1(s[2], s[3], o1);
  const float b0 = bmax_l2(o0, s[1]), b1 = bmax_l2(o1, s[3]);
  const float rowmax = xhalf_max(fmaxf(b0, b1));
  TileStats r;
  r.delta = stats_delta<UOS, PNQ>(m, mref, rowmax, sl2, r.alpha);
  block_scale<UOS, PNQ>(b0, r.delta, sl2, r.X[0], r.kofs[0]);
  block_scale<UOS, PNQ>(b1, r.delta, sl2, r.X[1], r.kofs[1]);
  return r;
}

// History rescale by alpha and the new accumulator input -mref.  Skipped
// for the whole wave (a uniform branch) when no row's reference moved and
// every alpha is exactly 1.
template <int D, int PNQ>
__device__ __forceinline__ void rescale(WaveState<D>& w, const TileStats& ts) {
  if (__builtin_amdgcn_ballot_w64(ts.alpha != 1.0f || ts.delta != 0.0f) != 0) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c) w.oacc[c] *= ts.alpha;
    // the four elements of lacc hold the same sum; only element 0 is read at
    // the end, so only it is kept rescaled (the others stay finite)
    if (PNQ) w.lacc[0] *= ts.alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) w.cneg[r] = -w.mref;
  }
}

// Four P~ values of this lane: registers r0..r0+3 of a subtile's S^T,
// v = exp2(d*c - kofs) rounded to E2M1 (nearest even, saturating) into
// bytes 2 HQ and 2 HQ + 1 of x (the other half's bytes kept); vsum
// accumulates the unquantized v (non-PNQ modes).  EFQ (PNQ == 2): code =
// rne(d * 2c + kofs) by v_cvt_pk_u8_f32 (round half to even, saturating at
// 0; below 7.5 by the choice of e), even and odd elements into the bytes of
// x and b, merged into nibbles (x |= b << 4) with the second half.
template <int PNQ, int HQ>
__device__ __forceinline__ void p_quad(const v16f& sv, int r0, float sl2, float kofs, uint32_t& x, uint32_t& b,
                                       float& vsum) {
  if (PNQ == 2) {
    const float c2 = 2.0f * sl2;
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = fmaf(sv[r0 + i], c2, kofs);
    // all four bytes of each word are written over the two halves
    x = __builtin_amdgcn_cvt_pk_u8_f32(t[0], 2 * HQ, HQ ? x : __float_as_uint(t[0]));
    x = __builtin_amdgcn_cvt_pk_u8_f32(t[2], 2 * HQ + 1, x);
    b = __builtin_amdgcn_cvt_pk_u8_f32(t[1], 2 * HQ, HQ ? b : __float_as_uint(t[1]));
    b = __builtin_amdgcn_cvt_pk_u8_f32(t[3], 2 * HQ + 1, b);
    if (HQ) x |= b << 4;
    return;
  }
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = __builtin_amdgcn_exp2f(fmaf(sv[r0 + i], sl2, -kofs));
    if (!PNQ) vsum += v[i];
  }
  // all four bytes are written over the two halves, so the first write may
  // start from any value
  x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(HQ ? x : __float_as_uint(v[0]), v[0], v[1], 1.0f, 2 * HQ);
  x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[2], v[3], 1.0f, 2 * HQ + 1);
}
// Eight values (registers 8 o .. 8 o + 7 of sv): one dword of P~ codes.
template <int PNQ>
__device__ __forceinline__ uint32_t p_oct(const v16f& sv, int o, float sl2, float kofs, float& vsum) {
  uint32_t x = 0, b = 0;
  p_quad<PNQ, 0>(sv, 8 * o, sl2, kofs, x, b, vsum);
  p_quad<PNQ, 1>(sv, 8 * o + 4, sl2, kofs, x, b, vsum);
  return x;
}

// Half HQ of both P~ dwords of one subtile (registers 4 HQ .. +3 and
// 8 + 4 HQ .. +3 of sv), the two conversion chains interleaved so that no
// conversion waits on the one just before it.
template <int PNQ, int HQ>
__device__ __forceinline__ void p_pair(const v16f& sv, float sl2, float kofs, uint32_t& x0, uint32_t& x1,
                                       uint32_t& b0, uint32_t& b1, float& vsum) {
  if (PNQ == 2) {
    const float c2 = 2.0f * sl2;
    float t[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t[i] = fmaf(sv[4 * HQ + i], c2, kofs);
      t[4 + i] = fmaf(sv[8 + 4 * HQ + i], c2, kofs);
    }
    // all four bytes of each word are written over the two halves
    x0 = __builtin_amdgcn_cvt_pk_u8_f32(t[0], 2 * HQ, HQ ? x0 : __float_as_uint(t[0]));
    x1 = __builtin_amdgcn_cvt_pk_u8_f32(t[4], 2 * HQ, HQ ? x1 : __float_as_uint(t[4]));
    b0 = __builtin_amdgcn_cvt_pk_u8_f32(t[1], 2 * HQ, HQ ? b0 : __float_as_uint(t[1]));
    b1 = __builtin_amdgcn_cvt_pk_u8_f32(t[5], 2 * HQ, HQ ? b1 : __float_as_uint(t[5]));
    x0 = __builtin_amdgcn_cvt_pk_u8_f32(t[2], 2 * HQ + 1, x0);
    x1 = __builtin_amdgcn_cvt_pk_u8_f32(t[6], 2 * HQ + 1, x1);
    b0 = __builtin_amdgcn_cvt_pk_u8_f32(t[3], 2 * HQ + 1, b0);
    b1 = __builtin_amdgcn_cvt_pk_u8_f32(t[7], 2 * HQ + 1, b1);
    if (HQ) {
      x0 |= b0 << 4;
      x1 |= b1 << 4;
    }
    return;
  }
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = __builtin_amdgcn_exp2f(fmaf(sv[4 * HQ + i], sl2, -kofs));
    v[4 + i] = __builtin_amdgcn_exp2f(fmaf(sv[8 + 4 * HQ + i], sl2, -kofs));
  }
  if (!PNQ) {
#pragma unroll
    for (int i = 0; i < 8; ++i) vsum += v[i];
  }
  // all four bytes are written over the two halves, so the first write may
  // start from any value
  x0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(HQ ? x0 : __float_as_uint(v[0]), v[0], v[1], 1.0f, 2 * HQ);
  x1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(HQ ? x1 : __float_as_uint(v[4]), v[4], v[5], 1.0f, 2 * HQ);
  x0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x0, v[2], v[3], 1.0f, 2 * HQ + 1);
  x1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x1, v[6], v[7], 1.0f, 2 * HQ + 1);
}

// Non-PNQ denominator: l = alpha l + sum of the unquantized p of the lane's
// two blocks of this tile (v sums in their scaled domains).
template <int D, int PNQ>
__device__ __forceinline__ void l_plain(WaveState<D>& w, const TileStats& ts, float v0, float v1) {
  if (!PNQ)
    w.lsum = fmaf(w.lsum, ts.alpha, __builtin_amdgcn_ldexpf(v0, static_cast<int>(ts.X[0]) - 127) +
                                        __builtin_amdgcn_ldexpf(v1, static_cast<int>(ts.X[1]) - 127));
}

// One O^T matrix instruction: channel tile c, key step s (P~ block pop of
// scale X); vsc holds the V~ E8M0 bytes of the tile.
template <int D>
__device__ __forceinline__ void pv_one(WaveState<D>& w, int c, int s, const uint4& vop, const Sc<D>& vsc,
                                       const uint4& pop, uint32_t X) {
  w.oacc[c] = mfma32<0>(vop, pop, w.oacc[c], vsc.w[(2 * c + s) >> 2], (2 * c + s) & 3, X);
}

// P~ dump (tests): this lane's block of key step s.
template <int DUMP>
__device__ __forceinline__ void dump_block(const MxAttnArgs& a, int64_t bh, int qrow, bool visit, int kb0,
                                           const uint4& pop, uint32_t X) {
  if (DUMP && visit && qrow < a.Sq) {
    const int slot = a.row_slot[bh * a.Sq + qrow];
    if (slot >= 0) {
      *reinterpret_cast<uint4*>(a.p_codes + static_cast<int64_t>(slot) * (a.skv_ld / 2) + kb0 / 2) = pop;
      a.p_scales[static_cast<int64_t>(slot) * (a.skv_ld / 32) + kb0 / 32] = static_cast<uint8_t>(X);
    }
  }
}

// The lane's Q~ operands (query row qrow, valid below sq): d-blocks
// 2 i + l/32 for d-half i; byte i of *qsc their E8M0 bytes.  Rows past the
// sequence are zero codes under scale 1.  The dump variants also store the
// codes and bytes.
template <int D, int UOS, int DUMP>
__device__ __forceinline__ void load_q(const MxAttnArgs& a, int64_t row0, int qrow, bool valid, int half,
                                       uint4 (&qop)[D / 64], uint32_t& qsc) {
  qsc = 0x7F7F7F7Fu;
  const int64_t row = row0 + qrow;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    qop[i] = make_uint4(0, 0, 0, 0);
    if (valid) {
      const int grp = 2 * i + half;
      const int64_t e0 = row * D + grp * 32;
      const void* src = a.q_bf16 ? static_cast<const void*>(static_cast<const uint16_t*>(a.q) + e0)
                                 : static_cast<const void*>(static_cast<const float*>(a.q) + e0);
      uint32_t X;
      qop[i] = quant_block32<UOS>(src, a.q_bf16 != 0, X);
      qsc = (qsc & ~(0xFFu << (8 * i))) | (X << (8 * i));
      if (DUMP) {
        *reinterpret_cast<uint4*>(a.qc + row * (D / 2) + grp * 16) = qop[i];
        a.qs[row * (D / 32) + grp] = static_cast<uint8_t>(X);
      }
    }
  }
}

// One fenced scheduling region: the compiler may order instructions within
// it but moves nothing across, so the interleave of matrix and vector work
// follows the source.  (This file is built with instruction selection in
// source order and without machine sinking, which would otherwise gather
// the side-effect-free matrix instructions ahead of the first fence or move
// them past the uniform rescale branches.)
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }
// The fences of the prefill kernel's tile steps.  The exp-free mode's
// vector slices are light enough that the compiler's own interleave runs it
// slightly faster (measured 1.3% on the DiT14 shape), so there they are off.
template <int PNQ>
__device__ __forceinline__ void step_fence() {
  if (PNQ != 2) fence();
}
// Results passed through pin_out must exist at that point (an empty asm
// statement), so a fenced region's vector work stays inside it.
__device__ __forceinline__ void pin_out(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin_out(float& v) { asm volatile("" : "+v"(v)); }

// Operands carried from one KV tile to the next: the second key step of
// the previous tile's O^T product (its V~ operands and scales, P~ and scale).
template <int D>
struct Carry {
  uint4 vop[D / 32];  // V~ of (channel tile c, key step 1)
  Sc<D> vsc;          // V~ E8M0 bytes of that tile
  uint4 pop;          // P~ of key step 1
  uint32_t X;         // its scale
};

// One KV tile j of the prefill kernel, as six fenced steps, each pairing a
// few matrix instructions with a slice of the vector work:
//   1: statistics of tile j            | O^T of tile j-1, key step 1 (first half), PNQ sum
//   2: P~ of subtile 0                 | O^T of tile j-1, key step 1 (second half)
//      (uniform branch: history rescale by alpha, new -mref)
//   3: P~ of subtile 1                 | S^T of tile j+1, subtile 0
//   4: P~ of subtile 2                 | S^T subtile 1; O^T of tile j, key step 0 (first half)
//   5: P~ of subtile 3                 | S^T subtile 2; O^T key step 0 (second half), PNQ sum
//   6: non-PNQ sum, dump; V~ operands of key step 1 | S^T subtile 3
// S^T of tile j+1 overwrites the registers of tile j subtile by subtile, after
// P~ has read them.  Operands are read from LDS one step ahead of their use.
template <int D, int UOS, int PNQ, int DUMP, int MASK>
__device__ __forceinline__ void kv_iter(WaveState<D>& w, v16f (&S)[kSub], Carry<D>& cy, const uint8_t* st_cur,
                                        const uint8_t* st_next, const uint4 (&qop)[D / 64], uint32_t qsc,
                                        uint32_t ones, int lim, int lane, float sl2, bool visit, int j0,
                                        const MxAttnArgs& a, int64_t bh, int qrow) {
  constexpr int NC = D / 32;
  constexpr int DH = D / 64;
  constexpr int NH = NC / 2;  // channel tiles per half of a key step
  const int half = lane >> 5;

  // ---- step 1: statistics of tile j | O^T (tile j-1, key step 1), first half
  if (MASK) mask_tile(S, lim);
  step_fence<PNQ>();
  TileStats ts;
  float o0[10], o1[10];
  pv_one<D>(w, 0, 1, cy.vop[0], cy.vsc, cy.pop, cy.X);
  bmax_l1(S[0], S[1], o0);
#pragma unroll
  for (int k = 0; k < 10; ++k) pin_out(o0[k]);
  step_fence<PNQ>();
  if (NH > 1) pv_one<D>(w, 1, 1, cy.vop[1], cy.vsc, cy.pop, cy.X);
  bmax_l1(S[2], S[3], o1);
#pragma unroll
  for (int k = 0; k < 10; ++k) pin_out(o1[k]);
  step_fence<PNQ>();
  if (PNQ) w.lacc = mfma_rowsum(ones, cy.pop, w.lacc, cy.X);
  float b0 = bmax_l2(o0, S[1]), b1 = bmax_l2(o1, S[3]);
  const float rowmax = xhalf_max(fmaxf(b0, b1));
  ts.delta = stats_delta<UOS, PNQ>(w.m, w.mref, rowmax, sl2, ts.alpha);
  block_scale<UOS, PNQ>(b0, ts.delta, sl2, ts.X[0], ts.kofs[0]);
  block_scale<UOS, PNQ>(b1, ts.delta, sl2, ts.X[1], ts.kofs[1]);
  pin_out(ts.kofs[0]);
  pin_out(ts.kofs[1]);
  pin_out(ts.X[0]);
  pin_out(ts.X[1]);
  pin_out(ts.alpha);
  step_fence<PNQ>();

  // ---- step 2: P~ of subtile 0 | O^T (tile j-1, key step 1), second half;
  // K~ operands of subtile 0 of tile j+1 read ahead
  uint4 kop[DH];
#pragma unroll
  for (int i = 0; i < DH; ++i) kop[i] = k_op<D>(st_next, 0, i, lane);
  const Sc<D> ksc = read_sc<D>(st_next, img_ks(D), lane);
  uint32_t pw[2][4], pb[2][4];
  float v0 = 0.0f, v1 = 0.0f;
  pv_one<D>(w, NH, 1, cy.vop[NH], cy.vsc, cy.pop, cy.X);
  p_pair<PNQ, 0>(S[0], sl2, ts.kofs[0], pw[0][0], pw[0][1], pb[0][0], pb[0][1], v0);
  pin_out(pw[0][0]);
  pin_out(pw[0][1]);
  if (PNQ == 2) {
    pin_out(pb[0][0]);
    pin_out(pb[0][1]);
  }
  if (!PNQ) pin_out(v0);
  step_fence<PNQ>();
  if (NH > 1) pv_one<D>(w, NH + 1, 1, cy.vop[NH + 1], cy.vsc, cy.pop, cy.X);
  p_pair<PNQ, 1>(S[0], sl2, ts.kofs[0], pw[0][0], pw[0][1], pb[0][0], pb[0][1], v0);
  pin_out(pw[0][0]);
  pin_out(pw[0][1]);
  if (!PNQ) pin_out(v0);
  step_fence<PNQ>();
  rescale<D, PNQ>(w, ts);

  // ---- step 3: P~ of subtile 1 | S^T (tile j+1) subtile 0; read K~ of
  // subtile 1 and V~ of tile j, key step 0 (first half)
  step_fence<PNQ>();
  uint4 kop1[DH];
#pragma unroll
  for (int i = 0; i < DH; ++i) kop1[i] = k_op<D>(st_next, 1, i, lane);
  const Sc<D> vsc = read_sc<D>(st_cur, img_vs(D), lane);
  uint4 vop0[NC];
#pragma unroll
  for (int c = 0; c < NH; ++c) vop0[c] = v_op<D>(st_cur, c, 0, lane);
  {
    v16f sn = s_part<D, 0>(0, kop[0], ksc, qop, qsc, w.cneg);
    p_pair<PNQ, 0>(S[1], sl2, ts.kofs[0], pw[0][2], pw[0][3], pb[0][2], pb[0][3], v0);
    pin_out(pw[0][2]);
    pin_out(pw[0][3]);
    if (PNQ == 2) {
      pin_out(pb[0][2]);
      pin_out(pb[0][3]);
    }
    if (!PNQ) pin_out(v0);
    step_fence<PNQ>();
    if constexpr (DH == 2) sn = s_part<D, 1>(0, kop[1], ksc, qop, qsc, sn);
    p_pair<PNQ, 1>(S[1], sl2, ts.kofs[0], pw[0][2], pw[0][3], pb[0][2], pb[0][3], v0);
    pin_out(pw[0][2]);
    pin_out(pw[0][3]);
    if (!PNQ) pin_out(v0);
    S[0] = sn;
    step_fence<PNQ>();
  }
  const uint4 p0 = make_uint4(pw[0][0], pw[0][1], pw[0][2], pw[0][3]);

  // ---- step 4: P~ of subtile 2 | S^T subtile 1; O^T (tile j, key step 0)
  // first half; read K~ of subtile 2 and the rest of V~ key step 0
  uint4 kop2[DH];
#pragma unroll
  for (int i = 0; i < DH; ++i) kop2[i] = k_op<D>(st_next, 2, i, lane);
#pragma unroll
  for (int c = NH; c < NC; ++c) vop0[c] = v_op<D>(st_cur, c, 0, lane);
  {
    v16f sn = s_part<D, 0>(1, kop1[0], ksc, qop, qsc, w.cneg);
    p_pair<PNQ, 0>(S[2], sl2, ts.kofs[1], pw[1][0], pw[1][1], pb[1][0], pb[1][1], v1);
    pin_out(pw[1][0]);
    pin_out(pw[1][1]);
    if (PNQ == 2) {
      pin_out(pb[1][0]);
      pin_out(pb[1][1]);
    }
    if (!PNQ) pin_out(v1);
    step_fence<PNQ>();
    if constexpr (DH == 2) sn = s_part<D, 1>(1, kop1[1], ksc, qop, qsc, sn);
    pv_one<D>(w, 0, 0, vop0[0], vsc, p0, ts.X[0]);
    p_pair<PNQ, 1>(S[2], sl2, ts.kofs[1], pw[1][0], pw[1][1], pb[1][0], pb[1][1], v1);
    pin_out(pw[1][0]);
    pin_out(pw[1][1]);
    if (!PNQ) pin_out(v1);
    S[1] = sn;
    step_fence<PNQ>();
  }
  if (NH > 1) pv_one<D>(w, 1, 0, vop0[1], vsc, p0, ts.X[0]);
  step_fence<PNQ>();

  // ---- step 5: P~ of subtile 3 | S^T subtile 2; O^T key step 0 second
  // half; PNQ sum of key step 0; read K~ of subtile 3
  uint4 kop3[DH];
#pragma unroll
  for (int i = 0; i < DH; ++i) kop3[i] = k_op<D>(st_next, 3, i, lane);
  {
    v16f sn = s_part<D, 0>(2, kop2[0], ksc, qop, qsc, w.cneg);
    p_pair<PNQ, 0>(S[3], sl2, ts.kofs[1], pw[1][2], pw[1][3], pb[1][2], pb[1][3], v1);
    pin_out(pw[1][2]);
    pin_out(pw[1][3]);
    if (PNQ == 2) {
      pin_out(pb[1][2]);
      pin_out(pb[1][3]);
    }
    if (!PNQ) pin_out(v1);
    step_fence<PNQ>();
    if constexpr (DH == 2) sn = s_part<D, 1>(2, kop2[1], ksc, qop, qsc, sn);
    pv_one<D>(w, NH, 0, vop0[NH], vsc, p0, ts.X[0]);
    p_pair<PNQ, 1>(S[3], sl2, ts.kofs[1], pw[1][2], pw[1][3], pb[1][2], pb[1][3], v1);
    pin_out(pw[1][2]);
    pin_out(pw[1][3]);
    if (!PNQ) pin_out(v1);
    S[2] = sn;
    step_fence<PNQ>();
  }
  if (NH > 1) pv_one<D>(w, NH + 1, 0, vop0[NH + 1], vsc, p0, ts.X[0]);
  if (PNQ) w.lacc = mfma_rowsum(ones, p0, w.lacc, ts.X[0]);
  const uint4 p1 = make_uint4(pw[1][0], pw[1][1], pw[1][2], pw[1][3]);
  step_fence<PNQ>();

  // ---- step 6: S^T subtile 3 | non-PNQ sum, dump; V~ operands of key step
  // 1 of tile j for the next tile's steps 1 and 2
  {
    S[3] = s_sub<D>(3, kop3, ksc, qop, qsc, w.cneg);
  }
  l_plain<D, PNQ>(w, ts, v0, v1);
#pragma unroll
  for (int c = 0; c < NC; ++c) cy.vop[c] = v_op<D>(st_cur, c, 1, lane);
  cy.vsc = vsc;
  cy.pop = p1;
  cy.X = ts.X[1];
  dump_block<DUMP>(a, bh, qrow, visit, j0 + 32 * half, p0, ts.X[0]);
  dump_block<DUMP>(a, bh, qrow, visit, j0 + 64 + 32 * half, p1, ts.X[1]);
  step_fence<PNQ>();
}

// Store a finished 32-column tile's O rows (lane l: its query row, channels
// 32 c + 8 g + 4 (l/32) + 0..3); nothing when orow is null.
template <int D>
__device__ __forceinline__ void store_o(float* orow, const v16f (&o)[D / 32], int half) {
  if (orow) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        *reinterpret_cast<float4*>(orow + 32 * c + 8 * gq + 4 * half) =
            make_float4(o[c][4 * gq], o[c][4 * gq + 1], o[c][4 * gq + 2], o[c][4 * gq + 3]);
  }
}

template <int D, int UOS, int PNQ, int CAUSAL, int DUMP>
__global__ __launch_bounds__(kThreads, 2) void attn_mx_kernel(MxAttnArgs a, float sl2) {
  constexpr int IMG = img_bytes(D);
  // One LDS object per stage, so that the compiler can tell which stage a
  // read touches and wait only for the direct loads into that stage.
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[IMG];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[IMG];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[IMG];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[IMG];
  static_assert(kStages == 4, "one LDS object per stage");
  // stage of ring position i (a constant after unrolling)
  auto lds_stage = [&](int i) -> uint8_t* {
    const int r = i % kStages;
    return r == 0 ? lds0 : r == 1 ? lds1 : r == 2 ? lds2 : lds3;
  };
  constexpr int NC = D / 32;  // output channel tiles

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nqb = (a.Sq + kMxQTile - 1) / kMxQTile;
  // Workgroup -> (head, query tile).  Workgroups are dispatched round-robin
  // over the 8 XCDs (each with its own L2), workgroup i to XCD i % 8.  Each
  // XCD is given a contiguous run of a list of (KV group, query head of the
  // group, query tile or causal pair), so a KV head's K~/V~ tile images are
  // fetched from HBM by one XCD (two at a run boundary) instead of all
  // eight.  With per-sequence lengths the KV groups gg = b * Hkv + g are
  // listed in the order of (gg % 8, gg / 8): each XCD then holds groups of
  // every batch entry, which keeps the XCDs equally loaded when the entries'
  // lengths differ (with equal lengths the plain order is kept).
  // Causal: one workgroup takes the query tiles p and nqb-1-p of a head
  // (nqb+1 KV tiles in all, the longer one first), so every workgroup of a
  // head does the same work and the fixed cost per workgroup is spread over
  // twice the tiles.
  // The list is cut into 8 runs, run x for XCD x; the first 7/8 of run x
  // go to its workgroups by index, and the rest through its work-queue
  // counter, which the XCD's later workgroups (the grid holds spares) pop
  // until the run is done and then turn to the other runs' counters, so
  // that no XCD idles while another still has items (the XCDs' speeds
  // differ by a few percent).  A workgroup that finds every run done exits.
  const int nslot = CAUSAL ? (nqb + 1) / 2 : nqb;  // workgroups per query head
  const int nitems = nslot * a.Hq * a.B;
  const int xcd = blockIdx.x & 7;
  const int per = nitems >> 3, extra = nitems & 7;
  const int cnt_x = per + (xcd < extra ? 1 : 0);
  const int j = static_cast<int>(blockIdx.x) >> 3;
  int gi;
  if (j < cnt_x - cnt_x / 8) {
    gi = per * xcd + min(xcd, extra) + j;
  } else {
    __shared__ int s_item;
    if (threadIdx.x == 0) {
      int item = -1;
      for (int v = 0; v < 8; ++v) {
        const int y = (xcd + v) & 7;
        const int cy = per + (y < extra ? 1 : 0);
        const uint32_t k = __hip_atomic_fetch_add(a.queue + y, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (k < static_cast<uint32_t>(cy / 8)) {
          item = per * y + min(y, extra) + (cy - cy / 8) + static_cast<int>(k);
          break;
        }
      }
      s_item = item;
    }
    __syncthreads();
    gi = s_item;
    if (gi < 0) return;  // whole workgroup: every item is taken
  }
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
  const int col = lane & 31;   // query column within the wave's 32
  const int half = lane >> 5;  // K-block / row group
  const uint32_t ones = rowsum_ones(lane);

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

  // The finished O rows of a job are held in registers until the next job
  // of the workgroup has requested its first KV tiles and Q rows: stores
  // count in the same in-order vector-memory counter as loads, so storing
  // first would make the next job's first waits wait for the stores too.
  v16f ofin[NC];
  float* orow = nullptr;  // this lane's pending row (null: none)
  for (int job = 0; job < njobs; ++job) {
    // the query tile of this job (causal: the longer one first)
    const int qb = CAUSAL ? (job == 0 ? nqb - 1 - slot : slot) : slot;
    const int q0 = qb * kMxQTile;
    const int qw0 = q0 + wave * kQW;  // first query row of this wave
    if (q0 >= sq) {  // whole workgroup (uniform), before any barrier of the job
      store_o<D>(orow, ofin, half);
      orow = nullptr;
      continue;
    }
    // every wave is done with the previous job's stages before they refill
    if (job > 0) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }

    int qrow = qw0 + col;
    const bool qvalid = qrow < sq;
    const int nt = static_cast<int>(a.skv_ld / kKvTile);  // tiles per (b, KV head) image run
    const int ntk = (skv + kKvTile - 1) / kKvTile;          // tiles holding this sequence's keys
    // tiles this workgroup visits: all, or up to its last causal diagonal tile
    const int ntiles = CAUSAL ? min(ntk, (q0 + kMxQTile - 1 + koff) / kKvTile + 1) : ntk;
    // Tiles [0, nmain) are unmasked for every wave (whole tiles at or below
    // the first row's limit); the rest are computed masked.  A wave dumps P~
    // only up to its own last tile (the sequence end, or the causal limit of
    // its last row); a wave whose rows all lie past the sequence dumps none.
    const int nmain = CAUSAL ? min((q0 + koff + 1) / kKvTile, skv / kKvTile) : skv / kKvTile;
    const int last_w = qw0 >= sq ? -1 : (CAUSAL ? min((qw0 + kQW - 1 + koff) / kKvTile, ntk - 1) : ntk - 1);
    const int klim = CAUSAL ? min(skv - 1, qrow + koff) : skv - 1;

    // wave-uniform (the divisions above run on the vector unit): scalar
    // registers, so the tile loads take the scalar-base form
    const uint8_t* img = uniform_ptr(a.img + bg * nt * static_cast<int64_t>(IMG));

    // Ring of kStages LDS stages: tile jt lives in stage jt % kStages.  Tiles
    // 0 and 1 are requested first, then this lane's Q rows; the previous
    // job's O rows are stored only once all of these have landed, so that
    // the stores drain while this job starts (the wait at the top of
    // iteration 0 is skipped: it would wait for them).  The barrier makes
    // every wave's loads visible.  At the top of iteration jt > 0 each wave
    // waits for its loads of tile jt+1 (requested an iteration earlier) and
    // the barrier tells that every wave has finished iteration jt-1.  The loads of tile jt+2 then refill the stage of tile
    // jt-2, whose last operands (V~ of key step 1, read in iteration jt-2)
    // were consumed in iteration jt-1.  Stage 3 stands for tile -1: the
    // second key step of its O^T product multiplies zero P~ codes, and only
    // its V~ scale bytes must be finite (set to 1.0 here).
    issue_tile<D>(lds0, img, wave, lane);
    if (ntiles > 1) issue_tile<D>(lds1, img + IMG, wave, lane);
    // Q~ operands (B of S^T): query column `col`, d-blocks 2 i + half;
    // rows past the sequence are zero codes.
    uint4 qop[D / 64];
    uint32_t qsc;
    load_q<D, UOS, DUMP>(a, bh * a.Sq, qrow, qvalid, half, qop, qsc);
    if (!qvalid) qrow = a.Sq;  // past the sequence: never dumped or stored
    wait_vmcnt<0>();  // tiles 0 and 1 (and Q) have landed
    asm volatile("" ::: "memory");
    store_o<D>(orow, ofin, half);
    orow = nullptr;
    for (int i = threadIdx.x; i < 64 * (D / 16) / 4; i += kThreads)
      reinterpret_cast<uint32_t*>(lds3 + img_vs(D))[i] = 0x7F7F7F7Fu;
    wait_lgkm0();  // the scale bytes above, written before any wave reads them
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    WaveState<D> w;
    init_state<D>(w);
    v16f S[kSub];
    {
      const Sc<D> ksc = read_sc<D>(lds0, img_ks(D), lane);
#pragma unroll
      for (int t = 0; t < kSub; ++t) {
        uint4 kop[D / 64];
#pragma unroll
        for (int i = 0; i < D / 64; ++i) kop[i] = k_op<D>(lds0, t, i, lane);
        S[t] = s_sub<D>(t, kop, ksc, qop, qsc, w.cneg);
      }
    }
    Carry<D> cy;
#pragma unroll
    for (int c = 0; c < NC; ++c) cy.vop[c] = v_op<D>(lds3, c, 1, lane);
    cy.vsc = read_sc<D>(lds3, img_vs(D), lane);
    cy.pop = make_uint4(0, 0, 0, 0);
    cy.X = 127;

    // tiles [0, nmain): no key masked; the ring position of each is a
    // compile-time constant (the loop is unrolled by the stage count)
    for (int jb = 0; jb < nmain; jb += kStages) {
#pragma unroll
      for (int k = 0; k < kStages; ++k) {
        const int jt = jb + k;
        if (jt < nmain) {
          if (jt > 0) wait_vmcnt<0>();  // tile 1 was waited for in the prologue
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          if (jt + 2 < ntiles)
            issue_tile<D>(lds_stage(k + 2), img + static_cast<int64_t>(jt + 2) * IMG, wave, lane);
          kv_iter<D, UOS, PNQ, DUMP, 0>(w, S, cy, lds_stage(k), lds_stage(k + 1), qop, qsc, ones,
                                        klim - (jt * kKvTile + 32 * half), lane, sl2, jt <= last_w,
                                        jt * kKvTile, a, bh, qrow);
        }
      }
    }
    // tiles [nmain, ntiles): the sequence end or the causal diagonal (one or
    // two tiles), keys masked per row; stages picked at run time
    for (int jt = nmain; jt < ntiles; ++jt) {
      if (jt > 0) wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (jt + 2 < ntiles)
        issue_tile<D>(lds_stage(jt + 2), img + static_cast<int64_t>(jt + 2) * IMG, wave, lane);
      // every load of the ring has landed here except tile jt+2's, which
      // targets neither stage read below
      kv_iter<D, UOS, PNQ, DUMP, 1>(w, S, cy, lds_stage(jt), lds_stage(jt + 1), qop, qsc, ones,
                                    klim - (jt * kKvTile + 32 * half), lane, sl2, jt <= last_w,
                                    jt * kKvTile, a, bh, qrow);
    }
    // O^T of the last tile, key step 1 (its operands carried in registers)
#pragma unroll
    for (int c = 0; c < NC; ++c) pv_one<D>(w, c, 1, cy.vop[c], cy.vsc, cy.pop, cy.X);
    if (PNQ) w.lacc = mfma_rowsum(ones, cy.pop, w.lacc, cy.X);

    // The stores run under a per-lane condition.  Pin the accumulators here
    // so that the matrix-core instructions producing them are not moved into
    // that divergent region: an MFMA issued with part of EXEC disabled would
    // drop the operands of the disabled lanes, which other lanes' results
    // depend on.
#pragma unroll
    for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(w.oacc[c]));
    asm volatile("" : "+v"(w.lacc));

    // O = O_acc / l; lane l holds channels 32 c + 8 g + 4 (l/32) + 0..3 of
    // its query row
    const float l = PNQ ? w.lacc[0] : xhalf_sum(w.lsum);
    const float inv = 1.0f / l;
#pragma unroll
    for (int c = 0; c < NC; ++c) ofin[c] = w.oacc[c] * inv;
    orow = qrow < a.Sq ? a.o + (bh * a.Sq + qrow) * D : nullptr;
  }  // job
  store_o<D>(orow, ofin, half);
}

// Clears the prefill kernel's work-queue counters (a kernel, not a memset,
// so that captured graphs replay it faithfully).
__global__ void clear_queue_kernel(uint32_t* q) {
  if (threadIdx.x < kQueueWords) q[threadIdx.x] = 0u;
}

template <int D, int UOS, int PNQ, int CAUSAL, int DUMP>
hipError_t launch_t(const MxAttnArgs& a, hipStream_t s) {
  const int nqb = (a.Sq + kMxQTile - 1) / kMxQTile;
  // causal: query tiles in pairs (see attn_mx_kernel)
  const int64_t nitems = static_cast<int64_t>(CAUSAL ? (nqb + 1) / 2 : nqb) * a.Hq * a.B;
  hipLaunchKernelGGL(clear_queue_kernel, dim3(1), dim3(64), 0, s, a.queue);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float sl2 = static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(D)));
  hipLaunchKernelGGL((attn_mx_kernel<D, UOS, PNQ, CAUSAL, DUMP>), dim3(static_cast<unsigned>(prefill_grid(nitems))),
                     dim3(kThreads), 0, s, a, sl2);
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
// One wave per (b, KV head g, split): its 32 query columns are the G x Sq
// queries of the GQA group (column c = h_local * Sq + i, G * Sq <= 32),
// so the group's K~/V~ are read once per split.  The wave runs the same
// tile step as above (S^T on the matrix core with -m as accumulator input,
// block scales, P~, O^T += V~^T P~^T) over the split's KV tiles, with its
// own running max from -inf.  Each wave streams its tiles through an LDS
// stage of its own (nothing is shared between waves): it reads a tile's
// operands into registers and then requests the next tile into the stage,
// whose loads are in flight during the rest of the tile's work.  It leaves
// (m, l, unnormalized O) per query column; the last wave of the group to
// finish merges the splits in ascending order.  Columns with no
// visible key in the split leave m = -inf, l = 0, O = 0.

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

// Merge of one (b, KV group) by the wave that finished it last.  Column c of
// the group is query (head g G + c / Sq, row c % Sq).  Each lane takes one
// column and CH channels of it, four columns per pass; the splits are folded
// in ascending order into the running (M, L, O), each rescaled to the larger
// max (O = sum_s 2^((m_s - M) c) O_s / sum_s 2^((m_s - M) c) l_s); a split
// that saw no key (m = -inf) adds nothing, and a column that no split saw
// stays unwritten.  The loads of kMergeChunk splits are issued together.
constexpr int kMergeChunk = 16;

// Partial states cross XCDs, whose L2 caches are not coherent with one
// another: they are stored and loaded with the device-scope coherence bit
// (the encoding the compiler gives agent-scope atomic stores and loads), so
// the stores write through to the coherent level and the loads read from
// it, and only the arrival counter needs ordering (a wait for the stores
// before the atomic increment).
constexpr int kCoherent = 16;  // cache-policy operand: sc1
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over split slot `slot` of the partial states (offsets
// within a group's splits stay far below 2^32 bytes).
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const MxDecodeArgs& d, int64_t slot) {
  float* p = d.part + slot * kDecodeCols * decode_slot(D);
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, 0xFFFFFFFFu, 0x00020000);
}

template <int D>
__device__ __forceinline__ void merge_group(const MxDecodeArgs& d, int b, int g, int64_t bg, float sl2,
                                            int lane) {
  const MxAttnArgs& a = d.at;
  constexpr int CH = D / 16;  // channels per lane: 16 lanes per column
  constexpr int SL = decode_slot(D);
  const int ncol = (a.Hq / a.Hkv) * a.Sq;
  const int ns = a.lens_k ? entry_splits(d, b) : d.nsplit;
  constexpr int sstride = kDecodeCols * SL;  // floats between splits
  const int ch = (lane & 15) * CH;
#pragma unroll 1
  for (int c0 = 0; c0 < ncol; c0 += 4) {
    const int c = c0 + (lane >> 4);
    const bool act = c < ncol;
    const __amdgpu_buffer_rsrc_t rs = part_rsrc<D>(d, bg * d.nsplit);  // split 0 of the group
    const int cb = (act ? c : 0) * SL * 4;
    float M = -INFINITY, L = 0.0f;
    float acc[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) acc[k] = 0.0f;
#pragma unroll 1
    for (int s0 = 0; s0 < ns; s0 += kMergeChunk) {
      float2 ml[kMergeChunk];
      float4 ov[kMergeChunk][CH / 4];
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u) {
        // past the last split: reload the last one, taken as empty
        const int off = cb + min(s0 + u, ns - 1) * sstride * 4;
        const float2 t = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kCoherent));
        ml[u] = make_float2(s0 + u < ns ? t.x : -INFINITY, t.y);
#pragma unroll
        for (int k = 0; k < CH / 4; ++k)
          ov[u][k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 4 * (4 + ch + 4 * k), 0, kCoherent));
      }
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u) {
        // branch-free, so that no load is sunk into a conditional block
        const float m = ml[u].x;
        const bool has = m != -INFINITY;
        const float Mn = has ? fmaxf(M, m) : M;
        const float wa = has ? __builtin_amdgcn_exp2f((M - Mn) * sl2) : 1.0f;  // 0 while M = -inf
        const float wb = has ? __builtin_amdgcn_exp2f((m - Mn) * sl2) : 0.0f;
        L = fmaf(L, wa, ml[u].y * wb);
#pragma unroll
        for (int k = 0; k < CH / 4; ++k) {
          acc[4 * k] = fmaf(acc[4 * k], wa, ov[u][k].x * wb);
          acc[4 * k + 1] = fmaf(acc[4 * k + 1], wa, ov[u][k].y * wb);
          acc[4 * k + 2] = fmaf(acc[4 * k + 2], wa, ov[u][k].z * wb);
          acc[4 * k + 3] = fmaf(acc[4 * k + 3], wa, ov[u][k].w * wb);
        }
        M = Mn;
      }
    }
    if (act && M != -INFINITY) {
      const int64_t row = (static_cast<int64_t>(b) * a.Hq + g * (a.Hq / a.Hkv) + c / a.Sq) * a.Sq + c % a.Sq;
      const float inv = 1.0f / L;
      float* out = a.o + row * D + ch;
#pragma unroll
      for (int k = 0; k < CH / 4; ++k)
        *reinterpret_cast<float4*>(out + 4 * k) =
            make_float4(acc[4 * k] * inv, acc[4 * k + 1] * inv, acc[4 * k + 2] * inv, acc[4 * k + 3] * inv);
    }
  }
}

template <int D, int UOS, int PNQ, int DUMP, int COMPACT>
__global__ __launch_bounds__(kThreads, 2) void attn_decode_kernel(MxDecodeArgs d, float sl2) {
  const MxAttnArgs& a = d.at;
  constexpr int IMG = img_bytes(D);
  constexpr int NC = D / 32;
  constexpr int DH = D / 64;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kWaves * IMG];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* st = lds + wave * IMG;  // this wave's stage
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
  const int col = lane & 31, half = lane >> 5;
  const uint32_t ones = rowsum_ones(lane);

  // query of this column; unused columns multiply zero codes and see every key
  const bool cvalid = col < G * a.Sq;
  const int hl = cvalid ? col / a.Sq : 0, qi = cvalid ? col % a.Sq : 0;
  const int64_t bh = static_cast<int64_t>(b) * a.Hq + g * G + hl;
  // this sequence's keys: the padded extent, or its own length
  const int skv = a.lens_k ? min(max(__builtin_amdgcn_readfirstlane(a.lens_k[b]), 0), a.Skv) : a.Skv;
  const int nt = static_cast<int>(a.skv_ld / kKvTile);  // tiles per (b, KV head) image run
  const int ntk = (skv + kKvTile - 1) / kKvTile;          // tiles holding this sequence's keys
  const int t_begin = sp * d.split_tiles;
  const int t_end = min(t_begin + d.split_tiles, ntk);
  // the first tile is requested before the Q rows, so that the two first
  // touches of memory overlap
  const uint8_t* img = uniform_ptr(a.img + bg * nt * static_cast<int64_t>(IMG));
  if (t_begin < t_end) issue_rows<D, 1>(st, img + static_cast<int64_t>(t_begin) * IMG, 0, lane);
  uint4 qop[DH];
  uint32_t qsc;
  // every split of a group quantizes the same rows; split 0 dumps them
  if (DUMP && sp == 0)
    load_q<D, UOS, 1>(a, bh * a.Sq, qi, cvalid, half, qop, qsc);
  else
    load_q<D, UOS, 0>(a, bh * a.Sq, qi, cvalid, half, qop, qsc);
  // causal: end-aligned; a row with no visible key (klim < 0) stays empty
  const int klim = (cvalid && a.causal) ? qi + (skv - a.Sq) : skv - 1;
  const int qrow = cvalid ? qi : a.Sq;  // rows >= Sq are never dumped
  // tiles needing the per-key mask: past the key end, or past the first
  // causal limit (skv - Sq)
  const int first_masked = a.causal ? max(skv - a.Sq, 0) / kKvTile : skv / kKvTile;

  WaveState<D> w;
  init_state<D>(w);

  for (int t = t_begin; t < t_end; ++t) {
    wait_vmcnt<0>();  // this wave's loads of tile t have landed in its stage
    asm volatile("" ::: "memory");
    const int j0 = t * kKvTile;
    v16f S[kSub];
    {
      const Sc<D> ksc = read_sc<D>(st, img_ks(D), lane);
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        uint4 kop[DH];
#pragma unroll
        for (int i = 0; i < DH; ++i) kop[i] = k_op<D>(st, u, i, lane);
        S[u] = s_sub<D>(u, kop, ksc, qop, qsc, w.cneg);
      }
    }
    uint4 vop[NC][2];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int s = 0; s < 2; ++s) vop[c][s] = v_op<D>(st, c, s, lane);
    const Sc<D> vsc = read_sc<D>(st, img_vs(D), lane);
    // every operand of tile t is in registers before the stage refills
    asm volatile("" ::: "memory");
    wait_lgkm0();
    asm volatile("" ::: "memory");
    if (t + 1 < t_end) issue_rows<D, 1>(st, img + static_cast<int64_t>(t + 1) * IMG, 0, lane);
    if (t >= first_masked) mask_tile(S, klim - (j0 + 32 * half));
    const TileStats ts = tile_stats<UOS, PNQ>(w.m, w.mref, S, sl2);
    rescale<D, PNQ>(w, ts);
    float v0 = 0.0f, v1 = 0.0f;
    const uint4 p0 = make_uint4(p_oct<PNQ>(S[0], 0, sl2, ts.kofs[0], v0), p_oct<PNQ>(S[0], 1, sl2, ts.kofs[0], v0),
                                p_oct<PNQ>(S[1], 0, sl2, ts.kofs[0], v0), p_oct<PNQ>(S[1], 1, sl2, ts.kofs[0], v0));
    const uint4 p1 = make_uint4(p_oct<PNQ>(S[2], 0, sl2, ts.kofs[1], v1), p_oct<PNQ>(S[2], 1, sl2, ts.kofs[1], v1),
                                p_oct<PNQ>(S[3], 0, sl2, ts.kofs[1], v1), p_oct<PNQ>(S[3], 1, sl2, ts.kofs[1], v1));
    const bool visit = j0 <= klim;
    dump_block<DUMP>(a, bh, qrow, visit, j0 + 32 * half, p0, ts.X[0]);
    dump_block<DUMP>(a, bh, qrow, visit, j0 + 64 + 32 * half, p1, ts.X[1]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      pv_one<D>(w, c, 0, vop[c][0], vsc, p0, ts.X[0]);
      pv_one<D>(w, c, 1, vop[c][1], vsc, p1, ts.X[1]);
    }
    if (PNQ) {
      w.lacc = mfma_rowsum(ones, p0, w.lacc, ts.X[0]);
      w.lacc = mfma_rowsum(ones, p1, w.lacc, ts.X[1]);
    }
    l_plain<D, PNQ>(w, ts, v0, v1);
  }

  // pin the accumulators ahead of the per-lane stores (see attn_mx_kernel)
#pragma unroll
  for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(w.oacc[c]));
  asm volatile("" : "+v"(w.lacc));
  const float l = PNQ ? w.lacc[0] : xhalf_sum(w.lsum);
  const bool empty = klim < t_begin * kKvTile;  // no visible key in this split
  if (cvalid) {  // unused columns are never merged
    // device-coherent stores (see part_rsrc): slot base in the resource,
    // byte offsets within the slot
    const __amdgpu_buffer_rsrc_t rs = part_rsrc<D>(d, slot);
    const int cb = col * decode_slot(D) * 4;
    if (half == 0) {
      const float2 ml = make_float2(empty ? -INFINITY : w.m, empty ? 0.0f : l);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ml), rs, cb, 0, kCoherent);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float4 ov = make_float4(w.oacc[c][4 * gq], w.oacc[c][4 * gq + 1], w.oacc[c][4 * gq + 2], w.oacc[c][4 * gq + 3]);
        if (empty) ov = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ov), rs,
                                               cb + 4 * (4 + 32 * c + 8 * gq + 4 * half), 0, kCoherent);
      }
  }

  // Arrival: once this wave's partial-state stores have completed (they
  // are written through to the device-coherent level), it is counted; the
  // wave that brings the group's count to its number of units (the splits
  // of the padded extent, or those holding the entry's keys) merges the
  // group, reading the partial states at that same level, and leaves the
  // counter at 0 for the next call.  (An agent-scope release fence would
  // also write back the whole L2 of the XCD, once per wave.)
  // (the empty asm statements keep the compiler from moving memory
  // operations across the wait and the increment)
  asm volatile("" ::: "memory");
  wait_vmcnt<0>();
  asm volatile("" ::: "memory");
  uint32_t before = 0;
  if (lane == 0) before = __hip_atomic_fetch_add(d.cnt + bg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  before = __builtin_amdgcn_readfirstlane(before);
  const int units = COMPACT ? entry_splits(d, b) : d.nsplit;
  if (static_cast<int>(before) != units - 1) return;
  asm volatile("" ::: "memory");
  merge_group<D>(d, b, g, bg, sl2, lane);
  asm volatile("" ::: "memory");
  if (lane == 0) __hip_atomic_store(d.cnt + bg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int UOS, int PNQ, int DUMP, int COMPACT>
hipError_t launch_decode_t(const MxDecodeArgs& d, hipStream_t s) {
  const float sl2 = static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(D)));
  const int64_t nunits = static_cast<int64_t>(d.at.B) * d.at.Hkv * d.nsplit;
  hipLaunchKernelGGL((attn_decode_kernel<D, UOS, PNQ, DUMP, COMPACT>), dim3(static_cast<unsigned>((nunits + kWaves - 1) / kWaves)),
                     dim3(kThreads), 0, s, d, sl2);
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
