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

struct Smem {
  uint4 kc[kSub * 64];          // K~ operands, [subtile][lane]
  uint8_t ks[kSub * 64];        // K~ scales, [subtile][lane]
  uint4 vc[(128 / 16) * 64];    // V~^T operands, [channel tile][lane]
  uint8_t vs[(128 / 16) * 64];  // V~^T scales
};

template <int D, int UOS, int PNQ, int CAUSAL, int DUMP>
__global__ __launch_bounds__(kThreads, 2) void attn_mx_kernel(MxAttnArgs a, float sl2) {
  __shared__ Smem sm;
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
    for (int i = tid; i < kSub * 32; i += kThreads) {
      const int t = i / 32, l = 32 + i % 32;
      sm.kc[t * 64 + l] = make_uint4(0, 0, 0, 0);
      sm.ks[t * 64 + l] = 127;
    }
  }

  v4f oacc[kQT][NT];
  v4f lacc[kQT];
  float m[kQT], lsum[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    m[t] = -INFINITY;
    lsum[t] = 0.0f;
    lacc[t] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int n = 0; n < NT; ++n) oacc[t][n] = v4f{0, 0, 0, 0};
  }
  const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);

  int ntiles = (a.Skv + kKvTile - 1) / kKvTile;
  if (CAUSAL) ntiles = min(ntiles, blockIdx.x + 1);  // Sq == Skv, kQTile == kKvTile

  const uint8_t* kc_g = a.kc + bg * a.Skv * (D / 2);
  const uint8_t* ks_g = a.ks + bg * a.Skv * DC;
  const uint8_t* vc_g = a.vc + bg * D * (a.skv_ld / 2);
  const uint8_t* vs_g = a.vs + bg * D * (a.skv_ld / 32);

  for (int jt = 0; jt < ntiles; ++jt) {
    const int j0 = jt * kKvTile;
    // ---- stage K~ and V~^T of this tile into LDS, in operand order ----
    for (int i = tid; i < kKvTile * DC; i += kThreads) {
      const int key = i / DC, c = i % DC;
      const int t = (key & 31) >> 2;
      const int rho = ((key >> 5) << 2) | (key & 3);
      sm.kc[t * 64 + c * 16 + rho] =
          *reinterpret_cast<const uint4*>(kc_g + static_cast<int64_t>(j0 + key) * (D / 2) + c * 16);
      sm.ks[t * 64 + c * 16 + rho] = ks_g[static_cast<int64_t>(j0 + key) * DC + c];
    }
    for (int i = tid; i < D * 4; i += kThreads) {
      const int d = i >> 2, c = i & 3;
      sm.vc[(d >> 4) * 64 + c * 16 + (d & 15)] =
          *reinterpret_cast<const uint4*>(vc_g + static_cast<int64_t>(d) * (a.skv_ld / 2) + j0 / 2 + c * 16);
      sm.vs[(d >> 4) * 64 + c * 16 + (d & 15)] = vs_g[static_cast<int64_t>(d) * (a.skv_ld / 32) + j0 / 32 + c];
    }
    __syncthreads();

    // ---- S^T = K~ Q~^T ----
    v4f s[kQT][kSub];
#pragma unroll
    for (int t = 0; t < kSub; ++t) {
      const uint4 kop = sm.kc[t * 64 + lane];
      const int ksc = sm.ks[t * 64 + lane];
#pragma unroll
      for (int u = 0; u < kQT; ++u) s[u][t] = mfma_fp4(kop, qop[u], v4f{0, 0, 0, 0}, ksc, qsc[u]);
    }

    const bool need_mask = (j0 + kKvTile > a.Skv) || (CAUSAL && j0 + kKvTile > q0);
#pragma unroll
    for (int u = 0; u < kQT; ++u) {
      if (need_mask) {
        const int klim = CAUSAL ? min(a.Skv - 1, qrow[u]) : a.Skv - 1;
#pragma unroll
        for (int t = 0; t < kSub; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = j0 + grp * 32 + t * 4 + r;
            if (key > klim) s[u][t][r] = -INFINITY;
          }
      }
      // row max: in-lane over this lane's 32-key block, then across lanes
      float bmax = s[u][0][0];
#pragma unroll
      for (int t = 0; t < kSub; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) bmax = fmaxf(bmax, s[u][t][r]);
      const float mnew = fmaxf(m[u], xlane_max4(bmax));
      const float alpha = __builtin_amdgcn_exp2f((m[u] - mnew) * sl2);
      m[u] = mnew;

      // scale of this lane's P~ block, then the block in the scaled domain
      const int X = p_block_e8m0<UOS>((bmax - mnew) * sl2);
      const float ef = static_cast<float>(X - 127);
      uint32_t pw[4];
      float vsum = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {  // dword w holds key subtiles 2w and 2w+1
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[i] = __builtin_amdgcn_exp2f(fmaf(s[u][2 * w + (i >> 2)][i & 3] - mnew, sl2, -ef));
          if (!PNQ) vsum += v[i];
        }
        uint32_t x = 0;
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[0], v[1], 1.0f, 0);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[2], v[3], 1.0f, 1);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[4], v[5], 1.0f, 2);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[6], v[7], 1.0f, 3);
        pw[w] = x;
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

      // history rescale, numerator and denominator
#pragma unroll
      for (int n = 0; n < NT; ++n) oacc[u][n] *= alpha;
      if (PNQ) {
        lacc[u] *= alpha;
        lacc[u] = mfma_fp4(ones, pop, lacc[u], 127, X);
      } else {
        lsum[u] = fmaf(lsum[u], alpha, __builtin_amdgcn_ldexpf(vsum, X - 127));
      }
#pragma unroll
      for (int n = 0; n < NT; ++n)
        oacc[u][n] = mfma_fp4(sm.vc[n * 64 + lane], pop, oacc[u][n], sm.vs[n * 64 + lane], X);
    }
    __syncthreads();
  }

  // ---- epilogue: O = O_acc / l ----
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    const float l = PNQ ? lacc[u][0] : xlane_sum4(lsum[u]);
    const float inv = 1.0f / l;
    if (qrow[u] < a.Sq) {
      float* orow = a.o + (bh * a.Sq + qrow[u]) * D;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        float4 w = make_float4(oacc[u][n][0] * inv, oacc[u][n][1] * inv, oacc[u][n][2] * inv,
                               oacc[u][n][3] * inv);
        *reinterpret_cast<float4*>(orow + n * 16 + grp * 4) = w;
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
