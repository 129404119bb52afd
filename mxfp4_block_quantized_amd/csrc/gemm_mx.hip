// W4A4 product of two MXFP4 operands on gfx950 block-scaled FP4 matrix cores.
//
// What it computes ("MXCode", abstract: MX-native W4A4 operands; blocks of 32
// along the contraction with one E8M0 byte each, as in the OCP MX format):
//   y[m][n] = sum_k deq(a)[m][k] * deq(b)[n][k],   fp32 accumulation,
// with a [M][K] and b [N][K] stored as the quantizer writes row-major
// tensors: codes [rows][K/2] (low nibble first), E8M0 bytes [rows][K/32].
//
// Mapping onto v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 x FP4): an operand lane
// l holds row (l % 16) and the 32 K-elements of K-block (l / 16) of one
// 128-wide K-step -- 16 bytes, one contiguous quarter of that row's 64-byte
// segment -- plus that block's E8M0 byte.  The product is formed transposed,
// y^T tile = b-rows x a-rows^T, so that accumulator lane l, register r holds
// y[m = a-row (l % 16)][n = b-row 4 (l / 16) + r]: four consecutive outputs
// of one row, written with one 16-byte (fp32) or 8-byte (bf16) store.
//
// Workgroup = 8 waves (two per SIMD: one wave alone cannot issue the matrix
// instructions back to back) = a 256 (m) x 256 (n) output tile; wave (wm, wn)
// owns 128 (m) x 64 (n) of it as 8 x 4 accumulator tiles held in VGPRs.  Per
// K-step the workgroup needs
// 256 rows x 64 bytes of each operand's codes plus 256 x 4 E8M0 bytes of each;
// they move global -> LDS with direct loads (global_load_lds) in operand
// order: code subtile i (16 rows) occupies 1 KiB with lane l's 16 bytes at
// l * 16, so every operand read is one contiguous ds_read_b128 per lane.
// K-steps stream through a 4-stage LDS ring (one LDS object per stage, loop
// unrolled by 4, loads issued 3 steps ahead); each wave reads its step
// operands from LDS and issues 32 MFMAs, the other wave on its SIMD covering
// the read latency.
//
// Rows past M or N read the last valid row (their outputs are not stored).
// K must be a positive multiple of 128.
#include "internal.h"

namespace mxk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kGTile = 256;            // rows of a and of b per workgroup
constexpr int kGSubA = 8;              // 16-row a subtiles per wave (128 m)
constexpr int kGSubB = 4;              // 16-row b subtiles per wave (64 n)
constexpr int kGStages = 4;
// One K-step in LDS: [a codes 16 KiB][b codes 16 KiB][a E8M0 1 KiB][b E8M0 1 KiB]
constexpr int kStA = 0;
constexpr int kStB = kGTile * 64;
constexpr int kStSa = 2 * kGTile * 64;
constexpr int kStSb = kStSa + kGTile * 4;
constexpr int kStBytes = kStSb + kGTile * 4;
// direct loads per wave and K-step: 2 + 2 code subtiles, one E8M0 row group of 64
constexpr int kGLoads = 5;

__device__ __forceinline__ v4f mfma_fp4(const uint4& a, const uint4& b, v4f c, int sa, int sb) {
  v8i av = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z),
            static_cast<int>(a.w), 0, 0, 0, 0};
  v8i bv = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z),
            static_cast<int>(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

// s_waitcnt vmcnt(N) alone (gfx9 encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

struct GemmArgs {
  const uint8_t* ac;  // [M][K/2]
  const uint8_t* as;  // [M][K/32]
  const uint8_t* bc;  // [N][K/2]
  const uint8_t* bs;  // [N][K/32]
  void* y;            // [M][N] fp32 or bf16
  int64_t M, N, K;
  int out_bf16;
  int tiles_m, tiles_n;
};

// Per-lane source pointers of this wave's direct loads for K-step 0; step s
// adds s * 64 bytes (codes) or s * 4 bytes (E8M0).
struct LoadPtrs {
  const uint8_t* code[4];  // a subtiles wave, wave + 8; b subtiles wave, wave + 8
  const uint8_t* sc;       // E8M0 bytes of 64 rows (a for waves 0-3, b for 4-7)
};

__device__ __forceinline__ void issue_step(uint8_t* st, const LoadPtrs& p, int s, int wave) {
  const int64_t oc = static_cast<int64_t>(s) * 64;
  const int64_t os = static_cast<int64_t>(s) * 4;
  __builtin_amdgcn_global_load_lds(p.code[0] + oc, st + kStA + wave * 1024, 16, 0, 0);
  __builtin_amdgcn_global_load_lds(p.code[1] + oc, st + kStA + (wave + 8) * 1024, 16, 0, 0);
  __builtin_amdgcn_global_load_lds(p.code[2] + oc, st + kStB + wave * 1024, 16, 0, 0);
  __builtin_amdgcn_global_load_lds(p.code[3] + oc, st + kStB + (wave + 8) * 1024, 16, 0, 0);
  __builtin_amdgcn_global_load_lds(p.sc + os, st + kStSa + wave * 256, 4, 0, 0);
}

// The 32 MFMAs of one K-step on operands read from LDS stage `st`.
__device__ __forceinline__ void step_mfma(v4f (&acc)[kGSubB][kGSubA], const uint8_t* st, int wm,
                                          int wn, int lane) {
  const int row = lane & 15, grp = lane >> 4;
  uint4 a[kGSubA], b[kGSubB];
  int sa[kGSubA], sb[kGSubB];
#pragma unroll
  for (int i = 0; i < kGSubB; ++i) {
    const int sub = kGSubB * wn + i;
    b[i] = *reinterpret_cast<const uint4*>(st + kStB + sub * 1024 + lane * 16);
    sb[i] = st[kStSb + (16 * sub + row) * 4 + grp];
  }
#pragma unroll
  for (int j = 0; j < kGSubA; ++j) {
    const int sub = kGSubA * wm + j;
    a[j] = *reinterpret_cast<const uint4*>(st + kStA + sub * 1024 + lane * 16);
    sa[j] = st[kStSa + (16 * sub + row) * 4 + grp];
  }
#pragma unroll
  for (int j = 0; j < kGSubA; ++j) {
#pragma unroll
    for (int i = 0; i < kGSubB; ++i)
      acc[i][j] = mfma_fp4(b[i], a[j], acc[i][j], sb[i], sa[j]);
  }
}

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // finite inputs
}

__global__ __launch_bounds__(kGThreads, 1) void gemm_mx_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[kStBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[kStBytes];
  static_assert(kGStages == 4, "one LDS object per stage");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // 2 x 4 waves

  // Workgroup -> output tile.  Workgroups are dispatched round-robin over the
  // 8 XCDs (workgroup i to XCD i % 8); each XCD takes a contiguous run of the
  // tile list, which walks column groups of 8 n-tiles with m-tiles inside, so
  // the ~32 workgroups an XCD holds at once share 4 a-panels and 8 b-panels
  // in its L2.
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int gi = (nwg >> 3) * xcd + min(xcd, nwg & 7) + (static_cast<int>(blockIdx.x) >> 3);
  constexpr int kGroupN = 8;
  const int per_group = kGroupN * a.tiles_m;
  const int ng = gi / per_group;
  const int rem = gi - ng * per_group;
  const int gn = min(kGroupN, a.tiles_n - ng * kGroupN);  // n-tiles in this group
  const int tm = rem / gn;
  const int tn = ng * kGroupN + rem % gn;
  const int64_t m0 = static_cast<int64_t>(tm) * kGTile;
  const int64_t n0 = static_cast<int64_t>(tn) * kGTile;

  const int64_t ldc = a.K / 2, lds_ = a.K / 32;
  LoadPtrs p;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int sub = wave + 8 * i;
    const int64_t ra = min(m0 + 16 * sub + (lane & 15), a.M - 1);
    const int64_t rb = min(n0 + 16 * sub + (lane & 15), a.N - 1);
    p.code[i] = a.ac + ra * ldc + (lane >> 4) * 16;
    p.code[2 + i] = a.bc + rb * ldc + (lane >> 4) * 16;
  }
  if (wave < 4)
    p.sc = a.as + min(m0 + 64 * wave + lane, a.M - 1) * lds_;
  else
    p.sc = a.bs + min(n0 + 64 * (wave - 4) + lane, a.N - 1) * lds_;

  v4f acc[kGSubB][kGSubA];
#pragma unroll
  for (int i = 0; i < kGSubB; ++i) {
#pragma unroll
    for (int j = 0; j < kGSubA; ++j) acc[i][j] = v4f{0, 0, 0, 0};
  }

  const int nk = static_cast<int>(a.K / 128);
  // Ring: K-step s lives in stage s % 4, loaded three steps ahead.  Iteration
  // s waits for the wave's own loads of step s (those of s + 1 and s + 2 may
  // stay in flight); the barrier then makes every wave's loads of step s
  // visible and tells that every wave is done reading step s - 1, whose
  // stage the loads of step s + 3 refill.
  issue_step(lds0, p, 0, wave);
  if (nk > 1) issue_step(lds1, p, 1, wave);
  if (nk > 2) issue_step(lds2, p, 2, wave);
  for (int sb = 0; sb < nk; sb += kGStages) {
#pragma unroll
    for (int k = 0; k < kGStages; ++k) {
      const int s = sb + k;
      if (s < nk) {
        if (s + 2 < nk) wait_vmcnt<2 * kGLoads>();
        else if (s + 1 < nk) wait_vmcnt<kGLoads>();
        else wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        uint8_t* fill = k == 0 ? lds3 : k == 1 ? lds0 : k == 2 ? lds1 : lds2;  // stage of s + 3
        if (s + 3 < nk) issue_step(fill, p, s + 3, wave);
        const uint8_t* st = k == 0 ? lds0 : k == 1 ? lds1 : k == 2 ? lds2 : lds3;
        step_mfma(acc, st, wm, wn, lane);
      }
    }
  }

  // The epilogue stores under per-lane conditions: keep every MFMA ahead of
  // that divergent region (a matrix instruction issued with part of EXEC off
  // would drop the disabled lanes' operands, which other lanes' results use).
#pragma unroll
  for (int i = 0; i < kGSubB; ++i) {
#pragma unroll
    for (int j = 0; j < kGSubA; ++j) asm volatile("" : "+v"(acc[i][j]));
  }

  const int row = lane & 15, grp = lane >> 4;
  const bool vec = (a.N & 3) == 0;
#pragma unroll
  for (int j = 0; j < kGSubA; ++j) {
    const int64_t m = m0 + 16 * (kGSubA * wm + j) + row;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < kGSubB; ++i) {
      const int64_t n = n0 + 16 * (kGSubB * wn + i) + 4 * grp;
      if (n >= a.N) continue;
      const v4f v = acc[i][j];
      if (a.out_bf16) {
        uint16_t* y = static_cast<uint16_t*>(a.y) + m * a.N + n;
        if (vec) {
          const uint2 w = make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16),
                                     bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
          *reinterpret_cast<uint2*>(y) = w;
        } else {
          for (int r = 0; r < 4 && n + r < a.N; ++r) y[r] = static_cast<uint16_t>(bf16_rne(v[r]));
        }
      } else {
        float* y = static_cast<float*>(a.y) + m * a.N + n;
        if (vec) {
          *reinterpret_cast<float4*>(y) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          for (int r = 0; r < 4 && n + r < a.N; ++r) y[r] = v[r];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K, int out_bf16,
                          void* y, hipStream_t stream) {
  GemmArgs g{ac, as, bc, bs, y, M, N, K, out_bf16, 0, 0};
  g.tiles_m = static_cast<int>((M + kGTile - 1) / kGTile);
  g.tiles_n = static_cast<int>((N + kGTile - 1) / kGTile);
  const int64_t nwg = static_cast<int64_t>(g.tiles_m) * g.tiles_n;
  hipLaunchKernelGGL(gemm_mx_kernel, dim3(static_cast<unsigned>(nwg)), dim3(kGThreads), 0, stream,
                     g);
  return hipGetLastError();
}

}  // namespace mxk
