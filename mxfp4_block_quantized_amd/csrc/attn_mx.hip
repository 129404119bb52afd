// Fused MXFP4 attention forward for gfx950 (OCP, UOS and UOS+PNQ modes).
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
// (l / 16) plus that block's E8M0 scale; the accumulator lane l, register
// r holds row 4*(l/16) + r, column l % 16.
//  * S^T = K~ Q~^T: A = 16 keys x 128 d, B = 128 d x 16 queries, one MFMA
//    covers D = 128.  The 16 A-rows of key subtile t (0..7) of a 128-key tile
//    are the keys 32*(row/4) + 4*t + row%4, so accumulator lane l holds, over
//    t and r, exactly the 32 keys 32*(l/16) + 4*t + r: one whole P~ block of
//    query l % 16.  Block maxima and the fp4 packing are therefore in-lane;
//    only the row max needs two cross-lane swaps.
//  * O^T = V~^T P~^T: A = 16 channels x 128 keys (V~ stored transposed,
//    blocks along keys), B = P~ (128 keys x 16 queries) straight from the
//    registers above, with one E8M0 byte per lane.  The accumulator keeps
//    query l % 16 in every lane of a column, matching the softmax state.
//
// P~ is formed in the scaled domain: for a block with scale exponent e,
// v = exp2((s - m) * log2(e)/sqrt(D) - e) is rounded by
// v_cvt_scalef32_pk_fp4_f32 (round to nearest even, saturating).  This keeps
// blocks whose probabilities lie below fp32's normal range exact in the same
// way the binary64 definition treats them.
#include "internal.h"

namespace mxk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQT = 2;                 // 16-query tiles per wave
constexpr int kSub = kKvTile / 16;     // key subtiles per KV tile (8)
static_assert(kQTile == kWaves * kQT * 16, "query tile = waves x q-tiles x 16");

__device__ __forceinline__ v4f mfma_fp4(const uint4& a, const uint4& b, v4f c, int sa, int sb) {
  v8i av = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z),
            static_cast<int>(a.w), 0, 0, 0, 0};
  v8i bv = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z),
            static_cast<int>(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
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

// E8M0 byte of a P~ block from x = log2 of its largest element (x <= 0).
// exp2 is taken 64 binades up so that maxima below fp32's normal range keep
// their exponent; X = max(0, Ef - 66 + up).
template <int UOS>
__device__ __forceinline__ int p_block_e8m0(float xmax) {
  uint32_t bits = __float_as_uint(__builtin_amdgcn_exp2f(xmax + 64.0f));
  int ef = static_cast<int>(bits >> 23);
  int up = UOS ? ((bits & 0x7FFFFFu) > 0x680000u ? 1 : 0) : 0;
  int X = ef - 66 + up;
  return X < 0 ? 0 : X;
}

// One pipeline stage of the LDS: a 128-key tile of K~ and V~^T, stored in
// MFMA operand order so that every operand read is one contiguous ds_read
// per lane.  Tiles arrive by direct global->LDS loads (global_load_lds):
// lane l of a load instruction lands in slot l of a 64-slot row, 16 bytes
// per slot for codes and one zero-extended byte per 4-byte slot for scales,
// so the key permutation is done by choosing each lane's source address.
struct Stage {
  uint4 kc[kSub * 64];         // K~ operands, [subtile][lane]
  uint4 vc[(128 / 16) * 64];   // V~^T operands, [channel tile][lane]
  uint32_t ks[kSub * 64];      // K~ scales (low byte), [subtile][lane]
  uint32_t vs[(128 / 16) * 64];
};

// Per-wave softmax state and accumulators for kQT query tiles.
template <int D>
struct WaveState {
  v4f oacc[kQT][D / 16];
  v4f lacc[kQT];
  float m[kQT];     // running row max (raw score units), -inf before the first tile
  float mref[kQT];  // value subtracted from S on the matrix core
  float lsum[kQT];
};

// Issue the loads of one KV tile (keys j0 .. j0+127) into a stage.  Wave w
// fills K~ subtiles 2w, 2w+1 and V~^T channel tiles (NT/4)*w ...; for
// D = 64 the lanes of the zero upper half of the contraction stay idle
// (their slots were zeroed once).
template <int D>
__device__ __forceinline__ void issue_tile(Stage& st, const uint8_t* kc_g, const uint8_t* ks_g,
                                           const uint8_t* vc_g, const uint8_t* vs_g,
                                           int64_t skv_ld, int j0, int wave, int lane) {
  constexpr int DC = D / 32;
  constexpr int NT = D / 16;
  const int rho = lane & 15, c = lane >> 4;
  if (c < DC) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = 2 * wave + i;
      const int64_t key = j0 + 32 * (rho >> 2) + 4 * t + (rho & 3);
      __builtin_amdgcn_global_load_lds(kc_g + key * (D / 2) + c * 16, &st.kc[t * 64], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(ks_g + key * DC + c, &st.ks[t * 64], 1, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < NT / 4; ++i) {
    const int n = (NT / 4) * wave + i;
    const int64_t d = 16 * n + rho;
    __builtin_amdgcn_global_load_lds(vc_g + d * (skv_ld / 2) + j0 / 2 + c * 16, &st.vc[n * 64], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vs_g + d * (skv_ld / 32) + j0 / 32 + c, &st.vs[n * 64], 1, 0, 0);
  }
}

// One KV tile for this wave's kQT query tiles.  MASK: keys beyond klim[u]
// (sequence end, causal diagonal) are excluded.
template <int D, int UOS, int PNQ, int DUMP, bool MASK>
__device__ __forceinline__ void compute_tile(WaveState<D>& w, const Stage& st, const uint4 (&qop)[kQT],
                                             const int (&qsc)[kQT], const int (&qrow)[kQT],
                                             const int (&klim)[kQT], int j0, int lane, float sl2,
                                             const MxAttnArgs& a, int64_t bh) {
  constexpr int NT = D / 16;
  const int grp = lane >> 4;
  const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);

#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    // d = S - mref on the matrix core: the accumulator input is -mref, the
    // reference running max of this row (0 before the first tile), so the
    // subtraction costs one rounding and no VALU work per element.
    const float nm = -w.mref[u];
    const v4f cneg = {nm, nm, nm, nm};
    v4f s[kSub];
#pragma unroll
    for (int t = 0; t < kSub; ++t)
      s[t] = mfma_fp4(st.kc[t * 64 + lane], qop[u], cneg, static_cast<int>(st.ks[t * 64 + lane]), qsc[u]);
    if (MASK) {
#pragma unroll
      for (int t = 0; t < kSub; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j0 + grp * 32 + t * 4 + r > klim[u]) s[t][r] = -INFINITY;
    }
    // row max: in-lane over this lane's 32-key block (a v_max3 chain), then
    // across the four lanes holding this query
    float bmax = s[0][0];
#pragma unroll
    for (int i = 1; i + 1 < 4 * kSub; i += 2)
      bmax = fmaxf(fmaxf(bmax, s[i >> 2][i & 3]), s[(i + 1) >> 2][(i + 1) & 3]);
    bmax = fmaxf(bmax, s[kSub - 1][3]);
    // delta = new max - mref.  Before the first tile the running max is -inf
    // (m - mref = -inf); afterwards m == mref, so delta = max(0, rowmax d).
    const float delta = fmaxf(w.m[u] - w.mref[u], xlane_max4(bmax));
    const float alpha = __builtin_amdgcn_exp2f((w.m[u] - w.mref[u] - delta) * sl2);
    w.m[u] = w.mref[u] + delta;
    w.mref[u] = w.m[u];

    // scale of this lane's P~ block, then the block in the scaled domain:
    // log2 v = (d - delta) * log2(e)/sqrt(D) - e = d*c - (delta*c + e)
    const int X = p_block_e8m0<UOS>((bmax - delta) * sl2);
    const float kofs = fmaf(delta, sl2, static_cast<float>(X - 127));
    uint32_t pw[4];
    float vsum = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // dword q holds key subtiles 2q and 2q+1
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = __builtin_amdgcn_exp2f(fmaf(s[2 * q + (i >> 2)][i & 3], sl2, -kofs));
        if (!PNQ) vsum += v[i];
      }
      uint32_t x = 0;
      x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[0], v[1], 1.0f, 0);
      x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[2], v[3], 1.0f, 1);
      x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[4], v[5], 1.0f, 2);
      x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[6], v[7], 1.0f, 3);
      pw[q] = x;
    }
    const uint4 pop = make_uint4(pw[0], pw[1], pw[2], pw[3]);

    if (DUMP && qrow[u] < a.Sq) {
      const int slot = a.row_slot[bh * a.Sq + qrow[u]];
      if (slot >= 0) {
        *reinterpret_cast<uint4*>(a.p_codes + static_cast<int64_t>(slot) * (a.skv_ld / 2) +
                                  (j0 + grp * 32) / 2) = pop;
        a.p_scales[static_cast<int64_t>(slot) * (a.skv_ld / 32) + (j0 + grp * 32) / 32] =
            static_cast<uint8_t>(X);
      }
    }

    // history rescale: alpha == 1 exactly leaves the history unchanged, so
    // the multiplies are skipped when that holds for the whole wave
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int n = 0; n < NT; ++n) w.oacc[u][n] *= alpha;
      if (PNQ) w.lacc[u] *= alpha;
    }
    if (PNQ) {
      w.lacc[u] = mfma_fp4(ones, pop, w.lacc[u], 127, X);
    } else {
      w.lsum[u] = fmaf(w.lsum[u], alpha, __builtin_amdgcn_ldexpf(vsum, X - 127));
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
      w.oacc[u][n] = mfma_fp4(st.vc[n * 64 + lane], pop, w.oacc[u][n], static_cast<int>(st.vs[n * 64 + lane]), X);
  }
}

template <int D, int UOS, int PNQ, int CAUSAL, int DUMP>
__global__ __launch_bounds__(kThreads, 2) void attn_mx_kernel(MxAttnArgs a, float sl2) {
  __shared__ Stage stage[2];
  constexpr int DC = D / 32;  // 16-byte chunks (32-element blocks) per row
  constexpr int NT = D / 16;  // output channel tiles

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int g = h / (a.Hq / a.Hkv);
  const int q0 = blockIdx.x * kQTile;
  const int col = lane & 15;   // query column within a 16-query tile
  const int grp = lane >> 4;   // K-block / lane group

  const int64_t bh = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t bg = static_cast<int64_t>(b) * a.Hkv + g;

  // Q~ operands (B of S^T): query column `col`, d-block `grp`.
  uint4 qop[kQT];
  int qsc[kQT];
  int qrow[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    qrow[t] = q0 + wave * (kQT * 16) + t * 16 + col;
    const int64_t row = bh * a.Sq + qrow[t];  // rows past Sq land in zeroed padding
    if (grp < DC) {
      qop[t] = *reinterpret_cast<const uint4*>(a.qc + row * (D / 2) + grp * 16);
      qsc[t] = a.qs[row * DC + grp];
    } else {
      qop[t] = make_uint4(0, 0, 0, 0);
      qsc[t] = 127;
    }
  }
  if (D == 64) {  // upper half of the contraction is zero for D = 64
    for (int i = tid; i < 2 * kSub * 32; i += kThreads) {
      const int sidx = i / (kSub * 32), t = (i / 32) % kSub, l = 32 + i % 32;
      stage[sidx].kc[t * 64 + l] = make_uint4(0, 0, 0, 0);
      stage[sidx].ks[t * 64 + l] = 127;
    }
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

  int ntiles = (a.Skv + kKvTile - 1) / kKvTile;
  if (CAUSAL) ntiles = min(ntiles, static_cast<int>(blockIdx.x) + 1);  // Sq == Skv, kQTile == kKvTile
  // only the last tile can hold keys past the end or past the causal diagonal
  const bool mask_last = CAUSAL || (a.Skv % kKvTile != 0);
  int klim[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) klim[t] = CAUSAL ? min(a.Skv - 1, qrow[t]) : a.Skv - 1;

  const uint8_t* kc_g = a.kc + bg * a.Skv * (D / 2);
  const uint8_t* ks_g = a.ks + bg * a.Skv * DC;
  const uint8_t* vc_g = a.vc + bg * D * (a.skv_ld / 2);
  const uint8_t* vs_g = a.vs + bg * D * (a.skv_ld / 32);

  // Tiles 0 .. nfull-1 need no masking; a masked last tile (sequence end
  // or causal diagonal) is handled after the loop.
  const int nfull = mask_last ? ntiles - 1 : ntiles;
  issue_tile<D>(stage[0], kc_g, ks_g, vc_g, vs_g, a.skv_ld, 0, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int jt = 0; jt < nfull; ++jt) {
    if (jt + 1 < ntiles)  // the other stage was released by the last barrier
      issue_tile<D>(stage[(jt + 1) & 1], kc_g, ks_g, vc_g, vs_g, a.skv_ld, (jt + 1) * kKvTile, wave, lane);
    compute_tile<D, UOS, PNQ, DUMP, false>(w, stage[jt & 1], qop, qsc, qrow, klim, jt * kKvTile, lane, sl2, a, bh);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's loads of the next tile have landed
    __syncthreads();
  }
  if (mask_last)
    compute_tile<D, UOS, PNQ, DUMP, true>(w, stage[nfull & 1], qop, qsc, qrow, klim, nfull * kKvTile, lane, sl2, a, bh);

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
}

template <int D, int UOS, int PNQ, int CAUSAL, int DUMP>
hipError_t launch_t(const MxAttnArgs& a, hipStream_t s) {
  dim3 grid((a.Sq + kQTile - 1) / kQTile, a.Hq, a.B);
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
    default: return pick_causal<D, 1, 1>(a, s);
  }
}

}  // namespace

hipError_t launch_attn_mx(const MxAttnArgs& a, hipStream_t stream) {
  return a.D == 64 ? pick_mode<64>(a, stream) : pick_mode<128>(a, stream);
}

}  // namespace mxk
