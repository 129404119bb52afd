// 16-bit attention forward for gfx950: the unquantized ("FP16") mode that
// the MXFP4 modes are compared against.  Same FlashAttention loop as the FP4
// kernel (running max per 128-key tile, fp32 accumulation, O / l at the
// end, "EFQ-Softmax" abstract), with S^T = K Q^T on bf16 (or fp16) matrix
// cores and O^T = V^T P^T on fp16 matrix cores: P = exp(s - m) is rounded
// to fp16 for the numerator; the denominator sums the fp32 P.
//
// v_mfma_f32_16x16x32_{bf16,f16}: operand lane l holds row (l % 16) and
// K-elements 8*(l/16) .. 8*(l/16)+7; accumulator lane l, register r holds
// row 4*(l/16) + r, column l % 16.  Within each 32-key group G of a tile,
// key subtiles t = 2G and 2G+1 put key 32G + 8*(row/4) + 4*(t%2) + row%4 in
// A-row `row`, so accumulator lane l ends up with keys 32G + 8*(l/16) + 0..7
// of query l % 16 -- exactly its slice of the P^T operand of O^T = V^T P^T.
#include "internal.h"

namespace mxk {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQT = 2;
constexpr int kSub = kKvTile / 16;
static_assert(kQTile == kWaves * kQT * 16, "query tile = waves x q-tiles x 16");

template <int QK_F16>
__device__ __forceinline__ v4f mfma_qk(const uint4& a, const uint4& b, v4f c) {
  if (QK_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                                  __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  }
}
__device__ __forceinline__ v4f mfma_pv(const uint4& a, const uint4& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                                __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

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

__device__ __forceinline__ uint32_t pack_f16x2(float x, float y) {
  v2f f = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2h));
}

template <int D, int QK_F16, int CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_f16_kernel(F16AttnArgs a, float sl2) {
  constexpr int KK = D / 32;  // contraction steps of S^T
  constexpr int NT = D / 16;  // output channel tiles
  __shared__ uint4 skc[kSub * KK * 64];  // K operands [t][kk][lane]
  __shared__ uint4 svc[NT * 4 * 64];     // V^T operands [channel tile][G][lane]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int g = h / (a.Hq / a.Hkv);
  const int q0 = blockIdx.x * kQTile;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t bh = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t bg = static_cast<int64_t>(b) * a.Hkv + g;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + bh * a.Sq * D;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + bg * a.Skv * D;
  const uint16_t* vg = a.vt + bg * D * a.skv_ld;

  uint4 qop[kQT][KK];
  int qrow[kQT];
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    qrow[u] = q0 + wave * (kQT * 16) + u * 16 + col;
    const int64_t r = min(qrow[u], a.Sq - 1);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qop[u][kk] = *reinterpret_cast<const uint4*>(qg + r * D + kk * 32 + grp * 8);
  }

  v4f oacc[kQT][NT];
  float m[kQT], lsum[kQT];
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    m[u] = -INFINITY;
    lsum[u] = 0.0f;
#pragma unroll
    for (int n = 0; n < NT; ++n) oacc[u][n] = v4f{0, 0, 0, 0};
  }

  int ntiles = (a.Skv + kKvTile - 1) / kKvTile;
  if (CAUSAL) ntiles = min(ntiles, blockIdx.x + 1);

  for (int jt = 0; jt < ntiles; ++jt) {
    const int j0 = jt * kKvTile;
    for (int i = tid; i < kKvTile * (D / 8); i += kThreads) {
      const int key = i / (D / 8), ch = i % (D / 8);
      const int kk = ch >> 2, gq = ch & 3;
      const int G = key >> 5, rem = key & 31;
      const int t = 2 * G + ((rem >> 2) & 1);
      const int rho = ((rem >> 3) << 2) | (rem & 3);
      const int64_t kr = min(j0 + key, a.Skv - 1);
      skc[(t * KK + kk) * 64 + gq * 16 + rho] =
          *reinterpret_cast<const uint4*>(kg + kr * D + ch * 8);
    }
    for (int i = tid; i < D * 16; i += kThreads) {
      const int d = i >> 4, ch = i & 15;
      const int G = ch >> 2, gq = ch & 3;
      svc[((d >> 4) * 4 + G) * 64 + gq * 16 + (d & 15)] =
          *reinterpret_cast<const uint4*>(vg + static_cast<int64_t>(d) * a.skv_ld + j0 + ch * 8);
    }
    __syncthreads();

    v4f s[kQT][kSub];
#pragma unroll
    for (int t = 0; t < kSub; ++t) {
#pragma unroll
      for (int u = 0; u < kQT; ++u) s[u][t] = v4f{0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4 kop = skc[(t * KK + kk) * 64 + lane];
#pragma unroll
        for (int u = 0; u < kQT; ++u) s[u][t] = mfma_qk<QK_F16>(kop, qop[u][kk], s[u][t]);
      }
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
            const int key = j0 + (t >> 1) * 32 + grp * 8 + (t & 1) * 4 + r;
            if (key > klim) s[u][t][r] = -INFINITY;
          }
      }
      float bmax = s[u][0][0];
#pragma unroll
      for (int t = 0; t < kSub; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) bmax = fmaxf(bmax, s[u][t][r]);
      const float mnew = fmaxf(m[u], xlane_max4(bmax));
      const float alpha = __builtin_amdgcn_exp2f((m[u] - mnew) * sl2);
      m[u] = mnew;
      uint4 pop[kSub / 2];
      float psum = 0.0f;
#pragma unroll
      for (int G = 0; G < kSub / 2; ++G) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = __builtin_amdgcn_exp2f((s[u][2 * G + (i >> 2)][i & 3] - mnew) * sl2);
          psum += p[i];
        }
        pop[G] = make_uint4(pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]),
                            pack_f16x2(p[4], p[5]), pack_f16x2(p[6], p[7]));
      }
      lsum[u] = fmaf(lsum[u], alpha, psum);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        oacc[u][n] *= alpha;
#pragma unroll
        for (int G = 0; G < kSub / 2; ++G)
          oacc[u][n] = mfma_pv(svc[(n * 4 + G) * 64 + lane], pop[G], oacc[u][n]);
      }
    }
    __syncthreads();
  }

  // Pin the accumulators before the per-lane store condition so that no
  // matrix-core instruction is moved into that divergent region (an MFMA with
  // part of EXEC disabled drops operands other lanes' results depend on).
#pragma unroll
  for (int u = 0; u < kQT; ++u)
#pragma unroll
    for (int n = 0; n < NT; ++n) asm volatile("" : "+v"(oacc[u][n]));

#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    const float inv = 1.0f / xlane_sum4(lsum[u]);
    if (qrow[u] < a.Sq) {
      float* orow = a.o + (bh * a.Sq + qrow[u]) * D;
#pragma unroll
      for (int n = 0; n < NT; ++n)
        *reinterpret_cast<float4*>(orow + n * 16 + grp * 4) =
            make_float4(oacc[u][n][0] * inv, oacc[u][n][1] * inv, oacc[u][n][2] * inv,
                        oacc[u][n][3] * inv);
    }
  }
}

// V [batch][rows][cols] (bf16 bits or fp32) -> fp16 V^T [batch][cols][rows_ld],
// zero beyond `rows`.  64 x 64 tiles through LDS.
template <typename In>
__device__ __forceinline__ float ld_in(const In* p);
template <>
__device__ __forceinline__ float ld_in<uint16_t>(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}
template <>
__device__ __forceinline__ float ld_in<float>(const float* p) {
  return *p;
}

template <typename In>
__global__ __launch_bounds__(256) void v_to_f16t_kernel(const In* __restrict__ v, int64_t rows,
                                                        int64_t cols, int64_t rows_ld,
                                                        uint16_t* __restrict__ vt) {
  __shared__ float tile[64][65];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t c0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int64_t b = blockIdx.z;
  const In* vb = v + b * rows * cols;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? ld_in<In>(vb + r * cols + c) : 0.0f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows_ld)
      vt[(b * cols + c) * rows_ld + r] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(tile[tx][i]));
  }
}

__global__ __launch_bounds__(256) void f32_to_f16_kernel(const float* __restrict__ x, int64_t n,
                                                         int64_t n_write, uint16_t* __restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n_write)
    y[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(i < n ? x[i] : 0.0f));
}

template <int D, int QK_F16>
hipError_t launch_c(const F16AttnArgs& a, hipStream_t s) {
  dim3 grid((a.Sq + kQTile - 1) / kQTile, a.Hq, a.B);
  const float sl2 = static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(D)));
  if (a.causal)
    hipLaunchKernelGGL((attn_f16_kernel<D, QK_F16, 1>), grid, dim3(kThreads), 0, s, a, sl2);
  else
    hipLaunchKernelGGL((attn_f16_kernel<D, QK_F16, 0>), grid, dim3(kThreads), 0, s, a, sl2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f16(const F16AttnArgs& a, hipStream_t stream) {
  if (a.D == 64) return a.qk_f16 ? launch_c<64, 1>(a, stream) : launch_c<64, 0>(a, stream);
  return a.qk_f16 ? launch_c<128, 1>(a, stream) : launch_c<128, 0>(a, stream);
}

hipError_t launch_v_to_f16t(const void* v, int64_t batch, int64_t rows, int64_t cols,
                            int64_t rows_ld, Dtype dt, uint16_t* vt, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>((rows_ld + 63) / 64), static_cast<unsigned>((cols + 63) / 64),
            static_cast<unsigned>(batch));
  if (dt == Dtype::BF16)
    hipLaunchKernelGGL((v_to_f16t_kernel<uint16_t>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(v), rows, cols, rows_ld, vt);
  else
    hipLaunchKernelGGL((v_to_f16t_kernel<float>), grid, dim3(256), 0, stream,
                       static_cast<const float*>(v), rows, cols, rows_ld, vt);
  return hipGetLastError();
}

hipError_t launch_f32_to_f16(const float* x, int64_t n, int64_t n_write, uint16_t* y,
                             hipStream_t stream) {
  if (n_write <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((n_write + 255) / 256));
  hipLaunchKernelGGL(f32_to_f16_kernel, grid, dim3(256), 0, stream, x, n, n_write, y);
  return hipGetLastError();
}

}  // namespace mxk
