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
// 128-wide K-step -- 16 bytes -- plus that block's E8M0 byte, one byte of a
// register picked by the instruction's op_sel.  The product is formed
// transposed, y^T tile = b-rows x a-rows^T, so that accumulator lane l,
// register r holds y[m = a-row (l % 16)][n = b-row 4 (l / 16) + r]: four
// consecutive outputs of one row, one 16-byte (fp32) or 8-byte (bf16) store.
//
// Workgroup = 8 waves, two per SIMD (one wave alone cannot issue the matrix
// instructions back to back), = a 256 (m) x 256 (n) output tile; wave
// (wm, wn) owns 128 (m) x 64 (n) as 8 x 4 accumulator tiles in VGPRs.
//
// Codes move global -> LDS with direct loads (global_load_lds_dwordx4) in
// stages of 256 K: each row contributes one whole 128-byte line per stage
// (8 lanes per row), and a stage holds 256 rows of each operand, 64 KiB in
// all; two stages form the LDS ring.  Within a row the eight 16-byte chunks
// are stored XOR-swizzled (chunk c of row r in slot c ^ swz(r)) so that the
// matrix-operand reads -- 16 rows x one chunk per group of 16 lanes -- touch
// every bank once; the swizzle is applied through the global addresses the
// direct loads fetch, the LDS side of a direct load being fixed.
// E8M0 bytes reach the registers without LDS: a pre-pass lays each
// operand's bytes out as a "scale image", one 4-byte word per lane holding
// the bytes of four consecutive K-steps, read with one coalesced load per
// 16-row subtile every 512 K.
//
// Rows past M or N read the last valid row (their outputs are not stored).
// K must be a positive multiple of 128.
#include <atomic>
#include <mutex>

#include "internal.h"

namespace mxk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kGTile = 256;  // rows of a and of b per workgroup
constexpr int kGSubA = 8;    // 16-row a subtiles per wave (128 m)
constexpr int kGSubB = 4;    // 16-row b subtiles per wave (64 n)
// One stage: 256 K of the tile's 256 rows of a, then of b; 128 bytes a row.
constexpr int kStRow = 128;
constexpr int kStA = 0;
constexpr int kStB = kGTile * kStRow;
constexpr int kStBytes = 2 * kGTile * kStRow;  // 64 KiB

__host__ __device__ constexpr int64_t scale_groups(int64_t K) { return (K / 128 + 3) / 4; }

// slot of the chunks of row r: chunk c sits in slot c ^ swz(r).  Over 16
// consecutive rows (16 t .. 16 t + 15) the pairs (r % 2, slot) are all
// distinct, so the 16 lanes of a ds_read_b128 that read one chunk of 16 rows
// fall into distinct 16-byte bank groups; measured free of bank conflicts
// on gfx950 (and so is (r & 7), unlike mixes of both).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <int SEL>
__device__ __forceinline__ v4f mfma_fp4(const uint4& a, const uint4& b, v4f c, int sa, int sb) {
  v8i av = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z),
            static_cast<int>(a.w), 0, 0, 0, 0};
  v8i bv = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z),
            static_cast<int>(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, SEL, sa, SEL, sb);
}

// s_waitcnt vmcnt(N) alone (gfx9 encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct GemmArgs {
  const uint8_t* ac;   // [M][K/2]
  const uint8_t* bc;   // [N][K/2]
  const uint8_t* asi;  // scale image of a: [ceil(M/16)][groups][64] words
  const uint8_t* bsi;  // scale image of b
  void* y;             // [M][N] fp32 or bf16
  int64_t M, N, K;
  int out_bf16;
  int tiles_m, tiles_n;
};

// Scale image: the E8M0 byte of (row 16 t + l % 16, block 4 s + l / 16),
// K-step s = 4 g + j, goes to byte j of word [t][g][l].  Rows and blocks
// past the end read as 0.
__global__ void scale_image_kernel(const uint8_t* __restrict__ sc, int64_t rows, int64_t K,
                                   uint32_t* __restrict__ img) {
  const int64_t ng = scale_groups(K);
  const int64_t nb = K / 32;
  const int64_t total = (rows + 15) / 16 * ng * 64;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int l = static_cast<int>(i & 63);
    const int64_t g = (i >> 6) % ng;
    const int64_t t = (i >> 6) / ng;
    const int64_t r = 16 * t + (l & 15);
    uint32_t w = 0;
    if (r < rows) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t b = 4 * (4 * g + j) + (l >> 4);
        if (b < nb) w |= static_cast<uint32_t>(sc[r * nb + b]) << (8 * j);
      }
    }
    img[i] = w;
  }
}

// Direct-load sources of this wave: load q (0..3) of a (and of b) covers
// the tile rows 8 (wave + 8 q) .. + 7; lane L fetches row 8 (wave + 8 q) +
// L / 8, chunk (L % 8) ^ swz(row), so that the chunk lands in LDS slot L % 8
// of its row.  The chunk index is the same for all q.  Bases are uniform
// (the tile's first row); the per-lane byte offsets fit 32 bits (the row
// within the tile times K/2 < 2^31).
struct LoadPtrs {
  const uint8_t* abase;
  const uint8_t* bbase;
  uint32_t aoff[4], boff[4];
  uint32_t half_fix;  // 64 for lanes fetching the second 64 bytes of a row, else 0
};

// Direct loads of one stage (256 K; `off` = its byte offset along a row).
// In a last stage with one K-step (`half`) the second 64 bytes of a row do
// not exist: the lanes that would fetch them re-fetch the first half (data
// that the one K-step does not read from their slots).
// The stage's base addresses are wave-uniform: keeping them in scalar
// registers lets each load take the scalar-base + 32-bit lane-offset form.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ void issue_stage(uint8_t* st, const LoadPtrs& lp, int64_t off, bool half,
                                            int wave) {
  // Buffer loads over the stage's row bases (every offset is in range by
  // construction).  Not the global form: with a global load-to-LDS in
  // flight the compiler makes every LDS wait a full lgkmcnt(0), so each
  // operand read would also wait for the next stage's loads.
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(uniform_ptr(lp.abase + off)), 0, 0xFFFFFFFFu, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(uniform_ptr(lp.bbase + off)), 0, 0xFFFFFFFFu, 0x00020000);
  const uint32_t fix = half ? lp.half_fix : 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, st + kStA + (wave + 8 * q) * 1024, 16,
                                             lp.aoff[q] - fix, 0, 0, 0);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, st + kStB + (wave + 8 * q) * 1024, 16,
                                             lp.boff[q] - fix, 0, 0, 0);
}

// The 32 MFMAs of K-step h (0/1) of stage `st`, with E8M0 byte SEL of the
// scale words.  Operand reads: the four b subtiles and a-subtiles 0..3
// first; a-subtile j + 4 is read right after the MFMAs of a-subtile j have
// issued, into the registers they release, and is used three MFMA groups
// later, so its LDS latency stays hidden.  (Left to itself the scheduler
// reads each operand just before its first use and waits for it, exposing
// the LDS latency eight times per step.)
template <int SEL>
__device__ __forceinline__ void step_mfma(v4f (&acc)[kGSubB][kGSubA], const uint8_t* st, int h,
                                          const uint32_t (&sa)[kGSubA],
                                          const uint32_t (&sb)[kGSubB], int wm, int wn, int lane) {
  const int row = lane & 15;
  const int c = 4 * h + (lane >> 4);
  // swz(16 t + row) == swz(row)
  const int off = row * kStRow + ((c ^ swz(row)) << 4);
  const uint8_t* pa = st + kStA + kGSubA * wm * 16 * kStRow + off;
  const uint8_t* pb = st + kStB + kGSubB * wn * 16 * kStRow + off;
  uint4 a[kGSubA], b[kGSubB];
#pragma unroll
  for (int i = 0; i < kGSubB; ++i) b[i] = *reinterpret_cast<const uint4*>(pb + i * 16 * kStRow);
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const uint4*>(pa + j * 16 * kStRow);
#pragma unroll
  for (int j = 0; j < kGSubA; ++j) {
#pragma unroll
    for (int i = 0; i < kGSubB; ++i)
      acc[i][j] = mfma_fp4<SEL>(b[i], a[j], acc[i][j], static_cast<int>(sb[i]),
                                static_cast<int>(sa[j]));
    if (j + 4 < kGSubA) a[j + 4] = *reinterpret_cast<const uint4*>(pa + (j + 4) * 16 * kStRow);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, kGSubB, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4 * kGSubB, 0);
}

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // finite inputs
}

// Output tile of entry gi of the tile list: column groups of 8 n-tiles,
// m-tiles inside, so that workgroups working on neighbouring entries share
// a-panels and b-panels in their XCD's L2.
__device__ __forceinline__ void tile_origin(const GemmArgs& a, int gi, int64_t& m0, int64_t& n0) {
  constexpr int kGroupN = 8;
  const int per_group = kGroupN * a.tiles_m;
  const int ng = gi / per_group;
  const int rem = gi - ng * per_group;
  const int gn = min(kGroupN, a.tiles_n - ng * kGroupN);  // n-tiles in this group
  m0 = static_cast<int64_t>(rem / gn) * kGTile;
  n0 = static_cast<int64_t>(ng * kGroupN + rem % gn) * kGTile;
}

// Per-lane sources of a tile: direct loads (load q of a and of b covers tile
// rows 8 (wave + 8 q) .. + 7; lane L fetches row 8 (wave + 8 q) + L / 8,
// chunk (L % 8) ^ swz(row), which lands in LDS slot L % 8 of its row) and
// the scale-image words of the wave's subtiles.  Rows and row tiles past
// the end read the last valid one (their outputs are not stored).
struct TileSrc {
  LoadPtrs lp;
  const uint32_t* sia[kGSubA];  // uniform: scale-image row tiles of the wave
  const uint32_t* sib[kGSubB];
};

__device__ __forceinline__ void tile_sources(const GemmArgs& a, int64_t m0, int64_t n0, int wave,
                                             int wm, int wn, int lane, TileSrc& ts) {
  const int64_t ldc = a.K / 2;
  const int rl = lane >> 3;
  // swz(8 (wave + 8 q) + rl) = (4 wave + rl / 2) & 7 does not depend on q
  const int chunk = (lane & 7) ^ swz(8 * wave + rl);
  ts.lp.half_fix = chunk >= 4 ? 64u : 0u;
  ts.lp.abase = a.ac + m0 * ldc;
  ts.lp.bbase = a.bc + n0 * ldc;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 8 * (wave + 8 * q) + rl;
    ts.lp.aoff[q] = static_cast<uint32_t>((min(m0 + r, a.M - 1) - m0) * ldc) + chunk * 16;
    ts.lp.boff[q] = static_cast<uint32_t>((min(n0 + r, a.N - 1) - n0) * ldc) + chunk * 16;
  }
  const int64_t ngrp = scale_groups(a.K);
  const int64_t last_ta = (a.M + 15) / 16 - 1, last_tb = (a.N + 15) / 16 - 1;
#pragma unroll
  for (int j = 0; j < kGSubA; ++j) {
    const int64_t t = min(m0 / 16 + kGSubA * wm + j, last_ta);
    ts.sia[j] = reinterpret_cast<const uint32_t*>(a.asi) + t * ngrp * 64;
  }
#pragma unroll
  for (int i = 0; i < kGSubB; ++i) {
    const int64_t t = min(n0 / 16 + kGSubB * wn + i, last_tb);
    ts.sib[i] = reinterpret_cast<const uint32_t*>(a.bsi) + t * ngrp * 64;
  }
}

__device__ __forceinline__ void load_scale_group(const TileSrc& ts, int64_t g, int lane,
                                                 uint32_t (&na)[kGSubA], uint32_t (&nb)[kGSubB]) {
#pragma unroll
  for (int j = 0; j < kGSubA; ++j) na[j] = ts.sia[j][64 * g + lane];
#pragma unroll
  for (int i = 0; i < kGSubB; ++i) nb[i] = ts.sib[i][64 * g + lane];
}

__device__ __forceinline__ void store_tile(const GemmArgs& a, const v4f (&acc)[kGSubB][kGSubA],
                                           int64_t m0, int64_t n0, int wm, int wn, int lane) {
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

// bf16 epilogue through LDS: each wave owns an 8 KiB area of the free stage
// slot and, in two rounds of 64 rows, writes its 64-row x 64-column bf16
// block there (one 128-byte line per row; the eight 16-byte chunks of row r
// XOR-swizzled by r & 7 against bank conflicts), then reads it back as
// whole lines and stores each row with 8 lanes x 16 bytes.  Needs a full
// tile and N % 8 == 0; issues exactly 16 stores per wave.
__device__ __forceinline__ void store_tile_bf16_lds(const GemmArgs& a,
                                                    const v4f (&acc)[kGSubB][kGSubA], int64_t m0,
                                                    int64_t n0, int wm, int wn, int lane,
                                                    uint8_t* area) {
  const int row16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int lrow = 16 * jj + row16;
#pragma unroll
      for (int i = 0; i < kGSubB; ++i) {
        const v4f v = acc[i][4 * r + jj];
        const int chunk = 2 * i + (g >> 1);
        const int addr = lrow * 128 + ((chunk ^ (lrow & 7)) << 4) + (g & 1) * 8;
        *reinterpret_cast<uint2*>(area + addr) =
            make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
      }
    }
    // the area is this wave's alone: its own writes are in order before
    // its reads (LDS operations of one wave execute in order)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int lrow = 8 * q + (lane >> 3);
      const int p = lane & 7;
      const uint4 w = *reinterpret_cast<const uint4*>(area + lrow * 128 + (p << 4));
      const int chunk = p ^ (lrow & 7);
      const int64_t m = m0 + 128 * wm + 64 * r + lrow;
      const int64_t n = n0 + 64 * wn + 8 * chunk;
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.y) + m * a.N + n) = w;
    }
  }
}

// Persistent: one workgroup per CU walks a run of output tiles.  Workgroups
// are dispatched round-robin over the 8 XCDs (workgroup b to XCD b % 8);
// each XCD owns a contiguous run of the tile list and its workgroups take
// consecutive entries of it, so that the tiles in flight on an XCD are
// neighbours in the list.
__global__ __launch_bounds__(kGThreads, 1) void gemm_mx_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // 2 x 4 waves

  const int ntiles = a.tiles_m * a.tiles_n;
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int wg_x = (nwg >> 3) + (xcd < (nwg & 7) ? 1 : 0);             // workgroups on this XCD
  const int tiles_x = (ntiles >> 3) + (xcd < (ntiles & 7) ? 1 : 0);    // tiles of this XCD
  const int first_x = (ntiles >> 3) * xcd + min(xcd, ntiles & 7);
  int local = static_cast<int>(blockIdx.x) >> 3;
  if (local >= tiles_x) return;  // uniform over the workgroup

  const int nk = static_cast<int>(a.K / 128);  // K-steps
  const int nst = (nk + 1) / 2;                 // stages of two K-steps
  const int64_t ngrp = scale_groups(a.K);
  // The next tile's first stage (slot 0) is fetched right after the current
  // tile's last stage, before its stores, when that last stage sits in slot
  // 1 (an even number of stages).
  const bool chain = (nst & 1) == 0;

  int64_t m0, n0;
  tile_origin(a, first_x + local, m0, n0);
  TileSrc ts;
  tile_sources(a, m0, n0, wave, wm, wn, lane, ts);
  uint32_t sa[kGSubA], sb[kGSubB], na[kGSubA], nb[kGSubB];
  load_scale_group(ts, 0, lane, na, nb);
  issue_stage(lds0, ts.lp, 0, nk == 1, wave);
  bool stores_ahead = false;  // the previous tile's stores were issued after this tile's first loads
  bool staged_prev = false;   // ... and went through LDS (16 per wave)

  for (;;) {
    const int64_t cm0 = m0, cn0 = n0;  // this tile
    const int next = local + wg_x;
    const bool has_next = next < tiles_x;
    v4f acc[kGSubB][kGSubA];
#pragma unroll
    for (int i = 0; i < kGSubB; ++i) {
#pragma unroll
      for (int j = 0; j < kGSubA; ++j) acc[i][j] = v4f{0, 0, 0, 0};
    }

    // Stage t lives in LDS slot t % 2; its direct loads are issued at the top
    // of stage t - 1.  Each stage begins with a wait for the wave's loads of
    // this stage (and of the next scale group) and a barrier (every wave's
    // loads have landed, and every wave is done reading stage t - 1, whose
    // slot the loads of stage t + 1 then refill).  Scale group g (K-steps
    // 4 g .. 4 g + 3 = stages 2 g, 2 g + 1) is fetched at the top of stage
    // 2 g - 2.  Vector memory operations complete in issue order, so with
    // the previous tile's 32 stores issued after this tile's first loads,
    // vmcnt(32) waits for those loads alone.
    for (int tb = 0; tb < nst; tb += 2) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int t = tb + k;
        if (t < nst) {
          if (t == 0 && stores_ahead && staged_prev)
            wait_vmcnt<16>();
          else if (t == 0 && stores_ahead)
            wait_vmcnt<kGSubA * kGSubB>();
          else
            wait_vmcnt<0>();
          barrier();
          if (k == 0) {
#pragma unroll
            for (int j = 0; j < kGSubA; ++j) sa[j] = na[j];
#pragma unroll
            for (int i = 0; i < kGSubB; ++i) sb[i] = nb[i];
            if (t / 2 + 1 < ngrp) load_scale_group(ts, t / 2 + 1, lane, na, nb);
          }
          if (t + 1 < nst)
            issue_stage(k == 0 ? lds1 : lds0, ts.lp, static_cast<int64_t>(t + 1) * 128,
                        2 * (t + 1) + 1 >= nk, wave);
          const uint8_t* st = k == 0 ? lds0 : lds1;
          if (k == 0) {
            step_mfma<0>(acc, st, 0, sa, sb, wm, wn, lane);
            if (2 * t + 1 < nk) step_mfma<1>(acc, st, 1, sa, sb, wm, wn, lane);
          } else {
            step_mfma<2>(acc, st, 0, sa, sb, wm, wn, lane);
            if (2 * t + 1 < nk) step_mfma<3>(acc, st, 1, sa, sb, wm, wn, lane);
          }
        }
      }
    }

    // The epilogue stores under per-lane conditions: keep every MFMA ahead of
    // that divergent region (a matrix instruction issued with part of EXEC
    // off would drop the disabled lanes' operands, which other lanes' results
    // use).
#pragma unroll
    for (int i = 0; i < kGSubB; ++i) {
#pragma unroll
      for (int j = 0; j < kGSubA; ++j) asm volatile("" : "+v"(acc[i][j]));
    }
    if (chain && has_next) {
      // slot 0 (stage nst - 2) was released by the last stage's barrier
      tile_origin(a, first_x + next, m0, n0);
      tile_sources(a, m0, n0, wave, wm, wn, lane, ts);
      load_scale_group(ts, 0, lane, na, nb);
      issue_stage(lds0, ts.lp, 0, nk == 1, wave);
    }
    const bool full = cm0 + kGTile <= a.M && cn0 + kGTile <= a.N;
    const bool staged = full && a.out_bf16 && (a.N & 7) == 0;
    if (staged) {
      // slot 1 is free once every wave is done reading the last stage (the
      // next tile's first loads, if any, go to slot 0)
      barrier();
      store_tile_bf16_lds(a, acc, cm0, cn0, wm, wn, lane, lds1 + wave * 8192);
    } else {
      store_tile(a, acc, cm0, cn0, wm, wn, lane);
    }
    if (!has_next) break;
    // stores per wave of a full tile: 16 staged (bf16) or kGSubA * kGSubB direct
    stores_ahead = chain && full && (staged || (a.N & 3) == 0);
    staged_prev = staged;
    if (!chain) {
      wait_vmcnt<0>();
      barrier();  // every wave is done with both slots
      tile_origin(a, first_x + next, m0, n0);
      tile_sources(a, m0, n0, wave, wm, wn, lane, ts);
      load_scale_group(ts, 0, lane, na, nb);
      issue_stage(lds0, ts.lp, 0, nk == 1, wave);
    }
    local = next;
  }
}

// Compute units of the current device (cached per device).
hipError_t cu_count(int* out) {
  // filled on first use; host threads may race to fill an entry, all with
  // the same value
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  *out = n;
  return hipSuccess;
}

size_t scale_image_bytes(int64_t rows, int64_t K) {
  return static_cast<size_t>((rows + 15) / 16 * scale_groups(K) * 256);
}

hipError_t launch_scale_image(const uint8_t* sc, int64_t rows, int64_t K, uint8_t* img,
                              hipStream_t stream) {
  const int64_t total = (rows + 15) / 16 * scale_groups(K) * 64;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(scale_image_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     sc, rows, K, reinterpret_cast<uint32_t*>(img));
  return hipGetLastError();
}

// Scale images of the product without a caller workspace: a file-scope
// device array, one copy per GPU, kept until the process ends.  In host code
// the name `scratch` is not a device address; the device address is fetched
// per device (gemm_scratch) and only that is passed to kernels.
__device__ __align__(256) uint8_t scratch[kGemmScratchBytes];

}  // namespace

hipError_t gemm_scratch(uint8_t** out) {
  static std::atomic<uint8_t*> addr[64];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  uint8_t* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      // with `dev` current: this device's copy of the array
      void* sym = nullptr;
      e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (sym == nullptr) return hipErrorInvalidSymbol;
      p = static_cast<uint8_t*>(sym);
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return (scale_image_bytes(M, K) + 255) / 256 * 256 + scale_image_bytes(N, K);
}

hipError_t launch_gemm_mx(const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K, int out_bf16,
                          void* y, uint8_t* ws, hipStream_t stream) {
  uint8_t* asi = ws;
  uint8_t* bsi = ws + (scale_image_bytes(M, K) + 255) / 256 * 256;
  hipError_t e = launch_scale_image(as, M, K, asi, stream);
  if (e != hipSuccess) return e;
  e = launch_scale_image(bs, N, K, bsi, stream);
  if (e != hipSuccess) return e;
  GemmArgs g{ac, bc, asi, bsi, y, M, N, K, out_bf16, 0, 0};
  g.tiles_m = static_cast<int>((M + kGTile - 1) / kGTile);
  g.tiles_n = static_cast<int>((N + kGTile - 1) / kGTile);
  const int64_t ntiles = static_cast<int64_t>(g.tiles_m) * g.tiles_n;
  int cus = 0;
  e = cu_count(&cus);
  if (e != hipSuccess) return e;
  // one resident workgroup per CU (128 KiB of LDS and 512 threads each)
  const int64_t nwg = std::min<int64_t>(ntiles, cus);
  hipLaunchKernelGGL(gemm_mx_kernel, dim3(static_cast<unsigned>(nwg)), dim3(kGThreads), 0, stream,
                     g);
  return hipGetLastError();
}

}  // namespace mxk
