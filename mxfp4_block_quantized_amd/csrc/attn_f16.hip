// 16-bit attention forward for gfx950: the unquantized ("FP16") mode that
// the MXFP4 modes are compared against.  Same FlashAttention loop as the FP4
// kernel (running max per KV tile, fp32 accumulation, O / l at the end,
// "EFQ-Softmax" abstract), with S^T = K Q^T on bf16 (or fp16) matrix cores
// and O^T = V^T P^T on fp16 matrix cores: P = exp(s - m) is rounded to fp16,
// and the denominator sums that same fp16 P on the matrix core (an MFMA
// against an all-ones operand), so numerator and denominator carry the same
// rounding.  Without a P~
// quantization the tile size only changes rounding, so this mode uses
// 64-key tiles (kF16KvTile), which keeps a 2-stage ring of 32 KiB tiles at
// two workgroups per CU.
//
// v_mfma_f32_16x16x32_{bf16,f16}: operand lane l holds row (l % 16) and
// K-elements 8*(l/16) .. 8*(l/16)+7; accumulator lane l, register r holds
// row 4*(l/16) + r, column l % 16.  Within each 32-key group G of a tile,
// key subtiles t = 2G and 2G+1 put key 32G + 8*(row/4) + 4*(t%2) + row%4 in
// A-row `row`, so accumulator lane l ends up with keys 32G + 8*(l/16) + 0..7
// of query l % 16 -- exactly its slice of the P^T operand of O^T = V^T P^T.
// The prepare kernel writes K and V^T as 16-bit tile images already in
// these operand orders, so a tile moves to LDS with contiguous
// 16-byte-per-lane direct loads.
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
constexpr int kQT = 2;                  // 16-query tiles per wave
constexpr int kT = kF16KvTile;          // keys per tile
constexpr int kSub = kT / 16;           // key subtiles of S^T
constexpr int kGrp = kT / 32;           // 32-key groups (contraction steps of O^T)
static_assert(kQTile == kWaves * kQT * 16, "query tile = waves x q-tiles x 16");
static_assert(kQTile % kT == 0, "query tiles start on KV tile boundaries");

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

__device__ __forceinline__ uint32_t pack_f16x2(float x, float y) {
  v2f f = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2h));
}

// s_waitcnt on the vector-memory counter only.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
}

// Direct loads of one tile image into an LDS stage: wave w moves the 1 KiB
// rows w, w + kWaves, ... of the image, lane l bytes [16 l, 16 l + 16).
template <int D>
__device__ __forceinline__ void issue_tile(uint8_t* stage, const uint8_t* src, int wave, int lane) {
  constexpr int NL = f16_img_bytes(D) / 1024;
  static_assert(NL % kWaves == 0, "whole rows per wave");
  // uniform base + 32-bit lane offset: one address register for every load
  const uint32_t lofs = static_cast<uint32_t>(wave * 1024 + lane * 16);
#pragma unroll
  for (int i = 0; i < NL / kWaves; ++i)
    __builtin_amdgcn_global_load_lds(src + lofs + i * kWaves * 1024, stage + (wave + i * kWaves) * 1024, 16, 0, 0);
}

template <int D>
struct F16State {
  v4f oacc[kQT][D / 16];
  v4f lacc[kQT];    // row sums of P (every element of a column holds its query's sum)
  float m[kQT];     // running row max (raw score units)
};

// P of one query tile: row max, history factor alpha (returned), fp16 P
// operands and the running denominator.
template <int D>
__device__ __forceinline__ float softmax_tile(F16State<D>& w, int u, const v4f (&s)[kSub], float sl2,
                                              uint4 (&pop)[kGrp]) {
  float bmax = s[0][0];
#pragma unroll
  for (int i = 1; i + 1 < 4 * kSub; i += 2)
    bmax = fmaxf(fmaxf(bmax, s[i >> 2][i & 3]), s[(i + 1) >> 2][(i + 1) & 3]);
  bmax = fmaxf(bmax, s[kSub - 1][3]);
  const float mnew = fmaxf(w.m[u], xlane_max4(bmax));
  const float alpha = __builtin_amdgcn_exp2f((w.m[u] - mnew) * sl2);  // 0 on the first tile
  w.m[u] = mnew;
  const float ofs = mnew * sl2;
#pragma unroll
  for (int G = 0; G < kGrp; ++G) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(s[2 * G + (i >> 2)][i & 3], sl2, -ofs));
    pop[G] = make_uint4(pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]), pack_f16x2(p[4], p[5]),
                        pack_f16x2(p[6], p[7]));
  }
  return alpha;
}

// History rescale: skipped when alpha == 1 exactly for the whole wave.
template <int D>
__device__ __forceinline__ void rescale_tile(F16State<D>& w, int u, float alpha) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
    for (int n = 0; n < D / 16; ++n) w.oacc[u][n] *= alpha;
    w.lacc[u][0] *= alpha;  // only element 0 is read at the end
  }
}

// Interleave N matrix-core instructions with K vector instructions each.
template <int N, int K>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, K, 0);
  }
}

template <int D, int QK_F16>
__device__ __forceinline__ void s_tile(v4f (&s)[kSub], const uint4 (&kop)[kSub][D / 32], const uint4 (&qop)[D / 32]) {
#pragma unroll
  for (int t = 0; t < kSub; ++t) {
    s[t] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) s[t] = mfma_qk<QK_F16>(kop[t][kk], qop[kk], s[t]);
  }
}

// Keys past `lim` (relative to the tile) are excluded.
__device__ __forceinline__ void mask_tile(v4f (&s)[kSub], int lim, int grp) {
  asm volatile("" : "+v"(lim));  // keeps the compares inside the caller's branch
#pragma unroll
  for (int t = 0; t < kSub; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = (t >> 1) * 32 + grp * 8 + (t & 1) * 4 + r;
      s[t][r] = key > lim ? -INFINITY : s[t][r];
    }
}

template <int D>
__device__ __forceinline__ void pv_tile(F16State<D>& w, int u, const uint4 (&pop)[kGrp], const uint8_t* vst,
                                        int lane) {
  const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);  // fp16 1.0
#pragma unroll
  for (int G = 0; G < kGrp; ++G) w.lacc[u] = mfma_pv(ones, pop[G], w.lacc[u]);
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
#pragma unroll
    for (int G = 0; G < kGrp; ++G)
      w.oacc[u][n] = mfma_pv(*reinterpret_cast<const uint4*>(vst + (n * kGrp + G) * 1024 + lane * 16),
                             pop[G], w.oacc[u][n]);
}

// One KV tile (keys j0 .. j0+kT-1) for the wave's two query tiles.
template <int D, int QK_F16>
__device__ __forceinline__ void compute_tile(F16State<D>& w, const uint8_t* st, const uint4 (&qop)[kQT][D / 32],
                                             const int (&klim)[kQT], bool mask, int j0, int lane,
                                             float sl2) {
  constexpr int KK = D / 32;
  constexpr int NT = D / 16;
  const int grp = lane >> 4;
  uint4 kop[kSub][KK];
#pragma unroll
  for (int t = 0; t < kSub; ++t)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      kop[t][kk] = *reinterpret_cast<const uint4*>(st + (t * KK + kk) * 1024 + lane * 16);
  const uint8_t* vst = st + f16_img_vc(D);
  v4f s0[kSub], s1[kSub];
  uint4 pop0[kGrp], pop1[kGrp];
  s_tile<D, QK_F16>(s0, kop, qop[0]);
  if (mask) mask_tile(s0, klim[0] - j0, grp);
  // S^T of query tile 1 on the matrix core while P of tile 0 is formed
  s_tile<D, QK_F16>(s1, kop, qop[1]);
  float alpha0 = softmax_tile<D>(w, 0, s0, sl2, pop0);
  interleave_mfma_valu<kSub * KK, 6>();
  // keep P of tile 0 here, beside the S^T products of tile 1
#pragma unroll
  for (int G = 0; G < kGrp; ++G)
    asm volatile("" : "+v"(pop0[G].x), "+v"(pop0[G].y), "+v"(pop0[G].z), "+v"(pop0[G].w));
  asm volatile("" : "+v"(alpha0));
  rescale_tile<D>(w, 0, alpha0);
  if (mask) mask_tile(s1, klim[1] - j0, grp);
  // O^T of query tile 0 while P of tile 1 is formed
  pv_tile<D>(w, 0, pop0, vst, lane);
  const float alpha1 = softmax_tile<D>(w, 1, s1, sl2, pop1);
  interleave_mfma_valu<(NT + 1) * kGrp, 6>();
  rescale_tile<D>(w, 1, alpha1);
  pv_tile<D>(w, 1, pop1, vst, lane);
}

template <int D, int QK_F16, int CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_f16_kernel(F16AttnArgs a, float sl2) {
  constexpr int KK = D / 32;
  constexpr int NT = D / 16;
  constexpr int IMG = f16_img_bytes(D);
  // one LDS object per stage (the compiler then waits only for the loads of
  // the stage a read touches)
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[IMG];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[IMG];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nqb = (a.Sq + kQTile - 1) / kQTile;
  // workgroup -> (head, query tile): a contiguous run of heads per XCD
  // (workgroups are dispatched round-robin over the 8 XCDs); causal: the
  // longest query tiles of a head first
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int gi = (nwg >> 3) * xcd + min(xcd, nwg & 7) + (static_cast<int>(blockIdx.x) >> 3);
  const int hb = gi / nqb;
  const int qb = CAUSAL ? nqb - 1 - gi % nqb : gi % nqb;
  const int h = hb % a.Hq;
  const int b = hb / a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int q0 = qb * kQTile;
  const int qw0 = q0 + wave * (kQT * 16);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t bh = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t bg = static_cast<int64_t>(b) * a.Hkv + g;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + bh * a.Sq * D;

  uint4 qop[kQT][KK];
  int qrow[kQT];
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    qrow[u] = qw0 + u * 16 + col;
    const int64_t r = min(qrow[u], a.Sq - 1);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qop[u][kk] = *reinterpret_cast<const uint4*>(qg + r * D + kk * 32 + grp * 8);
  }

  F16State<D> w;
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    w.m[u] = -INFINITY;
    w.lacc[u] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int n = 0; n < NT; ++n) w.oacc[u][n] = v4f{0, 0, 0, 0};
  }

  const int nt = (a.Skv + kT - 1) / kT;
  const int ntiles = CAUSAL ? min(nt, (q0 + kQTile - 1) / kT + 1) : nt;
  // tiles [0, nmain) need no masking for any row of this workgroup; a row's
  // first tile always holds an unmasked key (key 0)
  const int nmain = CAUSAL ? min(q0 / kT, nt) : (a.Skv % kT != 0 ? nt - 1 : nt);
  int klim[kQT];
#pragma unroll
  for (int u = 0; u < kQT; ++u) klim[u] = CAUSAL ? min(a.Skv - 1, qrow[u]) : a.Skv - 1;
  const uint8_t* img = a.img + bg * nt * static_cast<int64_t>(IMG);

  // 2-stage ring, unrolled by 2: the loads of tile jt+1 run during the
  // compute of tile jt; the barrier at the top of an iteration makes every
  // wave's loads of tile jt visible and releases the stage of tile jt-1.
  issue_tile<D>(lds0, img, wave, lane);
  for (int jb = 0; jb < ntiles; jb += 2) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int jt = jb + k;
      if (jt < ntiles) {
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (jt + 1 < ntiles)
          issue_tile<D>(k == 0 ? lds1 : lds0, img + static_cast<int64_t>(jt + 1) * IMG, wave, lane);
        compute_tile<D, QK_F16>(w, k == 0 ? lds0 : lds1, qop, klim, jt >= nmain, jt * kT, lane, sl2);
      }
    }
  }

  // Pin the accumulators before the per-lane store condition so that no
  // matrix-core instruction is moved into that divergent region (an MFMA with
  // part of EXEC disabled drops operands other lanes' results depend on).
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
#pragma unroll
    for (int n = 0; n < NT; ++n) asm volatile("" : "+v"(w.oacc[u][n]));
    asm volatile("" : "+v"(w.lacc[u]));
  }

#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    const float inv = 1.0f / w.lacc[u][0];
    if (qrow[u] < a.Sq) {
      float* orow = a.o + (bh * a.Sq + qrow[u]) * D;
#pragma unroll
      for (int n = 0; n < NT; ++n)
        *reinterpret_cast<float4*>(orow + n * 16 + grp * 4) =
            make_float4(w.oacc[u][n][0] * inv, w.oacc[u][n][1] * inv, w.oacc[u][n][2] * inv,
                        w.oacc[u][n][3] * inv);
    }
  }
}

// ---- operand preparation: 16-bit tile images --------------------------------
//
// One workgroup per (batch, tile): the tile's V rows are converted to fp16
// and staged in LDS (padded rows), then every thread writes 16-byte chunks
// of the image: K chunks straight from the rows (bf16 kept, fp32 -> fp16),
// V^T chunks gathered down the LDS columns.  Rows past `rows` are zero.
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
__device__ __forceinline__ uint16_t to_f16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
__device__ __forceinline__ uint4 pack8_u16(const uint16_t (&hv)[8]) {
  return make_uint4(hv[0] | (uint32_t(hv[1]) << 16), hv[2] | (uint32_t(hv[3]) << 16),
                    hv[4] | (uint32_t(hv[5]) << 16), hv[6] | (uint32_t(hv[7]) << 16));
}

template <typename In, int D>
__global__ __launch_bounds__(256) void f16_image_kernel(const In* __restrict__ k, const In* __restrict__ v,
                                                        int rows, int ntiles, uint8_t* __restrict__ img) {
  constexpr int KK = D / 32;
  constexpr int NT = D / 16;
  constexpr int LD = D + 2;  // padded row (halves): column reads spread over banks
  __shared__ uint16_t vt[kT * LD];
  const int T = blockIdx.x % ntiles;
  const int64_t bgi = blockIdx.x / ntiles;
  const int j0 = T * kT;
  const In* kb = k + (bgi * rows) * D;
  const In* vb = v + (bgi * rows) * D;
  uint8_t* out = img + (bgi * ntiles + T) * static_cast<int64_t>(f16_img_bytes(D));
  for (int i = threadIdx.x; i < kT * D; i += 256) {
    const int r = i / D, c = i % D;
    vt[r * LD + c] = (j0 + r < rows) ? to_f16(ld_in<In>(vb + static_cast<int64_t>(j0 + r) * D + c)) : 0;
  }
  // K chunks: (subtile t, contraction step kk, lane l) -> key of A-row l % 16
  for (int i = threadIdx.x; i < kSub * KK * 64; i += 256) {
    const int l = i & 63, tk = i >> 6, t = tk / KK, kk = tk % KK;
    const int rho = l & 15, gq = l >> 4;
    const int key = (t >> 1) * 32 + (rho >> 2) * 8 + (t & 1) * 4 + (rho & 3);
    uint4 chunk = make_uint4(0u, 0u, 0u, 0u);
    if (j0 + key < rows) {
      const In* src = kb + static_cast<int64_t>(j0 + key) * D + kk * 32 + gq * 8;
      if (sizeof(In) == 2) {
        chunk = *reinterpret_cast<const uint4*>(src);
      } else {
        uint16_t hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = to_f16(ld_in<In>(src + e));
        chunk = pack8_u16(hv);
      }
    }
    *reinterpret_cast<uint4*>(out + tk * 1024 + l * 16) = chunk;
  }
  __syncthreads();
  // V^T chunks: (channel tile n, key group G, lane l) -> channel 16n + l % 16,
  // keys 32G + 8(l/16) .. +7
  for (int i = threadIdx.x; i < NT * kGrp * 64; i += 256) {
    const int l = i & 63, nG = i >> 6, n = nG / kGrp, G = nG % kGrp;
    const int d = 16 * n + (l & 15), key0 = 32 * G + 8 * (l >> 4);
    uint16_t hv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] = vt[(key0 + e) * LD + d];
    *reinterpret_cast<uint4*>(out + f16_img_vc(D) + nG * 1024 + l * 16) = pack8_u16(hv);
  }
}

__global__ __launch_bounds__(256) void f32_to_f16_kernel(const float* __restrict__ x, int64_t n,
                                                         int64_t n_write, uint16_t* __restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n_write) y[i] = to_f16(i < n ? x[i] : 0.0f);
}

template <int D, int QK_F16>
hipError_t launch_c(const F16AttnArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((a.Sq + kQTile - 1) / kQTile) * a.Hq * a.B);
  const float sl2 = static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(D)));
  if (a.causal)
    hipLaunchKernelGGL((attn_f16_kernel<D, QK_F16, 1>), grid, dim3(kThreads), 0, s, a, sl2);
  else
    hipLaunchKernelGGL((attn_f16_kernel<D, QK_F16, 0>), grid, dim3(kThreads), 0, s, a, sl2);
  return hipGetLastError();
}

template <typename In, int D>
hipError_t launch_img(const void* k, const void* v, int64_t batch, int rows, uint8_t* img,
                      hipStream_t s) {
  const int ntiles = (rows + kT - 1) / kT;
  hipLaunchKernelGGL((f16_image_kernel<In, D>), dim3(static_cast<unsigned>(batch * ntiles)), dim3(256), 0,
                     s, static_cast<const In*>(k), static_cast<const In*>(v), rows, ntiles, img);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f16(const F16AttnArgs& a, hipStream_t stream) {
  if (a.D == 64) return a.qk_f16 ? launch_c<64, 1>(a, stream) : launch_c<64, 0>(a, stream);
  return a.qk_f16 ? launch_c<128, 1>(a, stream) : launch_c<128, 0>(a, stream);
}

hipError_t launch_f16_images(const void* k, const void* v, int64_t batch, int rows, int D, Dtype dt,
                             uint8_t* img, hipStream_t stream) {
  if (batch <= 0 || rows <= 0) return hipSuccess;
  if (dt == Dtype::BF16)
    return D == 64 ? launch_img<uint16_t, 64>(k, v, batch, rows, img, stream)
                   : launch_img<uint16_t, 128>(k, v, batch, rows, img, stream);
  return D == 64 ? launch_img<float, 64>(k, v, batch, rows, img, stream)
                 : launch_img<float, 128>(k, v, batch, rows, img, stream);
}

hipError_t launch_f32_to_f16(const float* x, int64_t n, int64_t n_write, uint16_t* y,
                             hipStream_t stream) {
  if (n_write <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((n_write + 255) / 256));
  hipLaunchKernelGGL(f32_to_f16_kernel, grid, dim3(256), 0, stream, x, n, n_write, y);
  return hipGetLastError();
}

}  // namespace mxk
