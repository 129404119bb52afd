// MXFP4 block quantizer and dequantizer kernels for gfx950 (block rule and
// rounding: mx_block.h).
#include "internal.h"
#include "mx_block.h"

namespace mxk {
namespace {

constexpr int kThreads = 256;

// Streamed data (read or written once) goes through nontemporal vector
// accesses, so that it does not displace reused lines in the caches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  // quad_perm [1,0,3,2] then [2,3,0,1]
  uint32_t t = static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true));
  v = max(v, t);
  t = static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, true));
  return max(v, t);
}

// Eight consecutive elements as fp32 bit patterns.
__device__ __forceinline__ void load8(const uint16_t* __restrict__ x, int64_t o,
                                      uint32_t f[8]) {
  const u32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + o * 8));
  const uint4 v = make_uint4(vv[0], vv[1], vv[2], vv[3]);
  f[0] = v.x << 16; f[1] = v.x & 0xFFFF0000u;
  f[2] = v.y << 16; f[3] = v.y & 0xFFFF0000u;
  f[4] = v.z << 16; f[5] = v.z & 0xFFFF0000u;
  f[6] = v.w << 16; f[7] = v.w & 0xFFFF0000u;
}
__device__ __forceinline__ void load8(const float* __restrict__ x, int64_t o,
                                      uint32_t f[8]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(x + o * 8);
  const u32x4 av = __builtin_nontemporal_load(p), bv = __builtin_nontemporal_load(p + 1);
  const uint4 a = make_uint4(av[0], av[1], av[2], av[3]), b = make_uint4(bv[0], bv[1], bv[2], bv[3]);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Blocks along the contiguous axis.  Each lane owns 8 consecutive elements
// (an "octet"); the 4 lanes of a DPP quad form one 32-element block.  Each
// wave instruction therefore reads a contiguous 1 KiB (bf16) and writes a
// contiguous 256 B of codes.
template <typename In, int UOS, int UNROLL>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(
    const In* __restrict__ x, int64_t n_oct, int64_t n_oct_write,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  uint32_t f[UNROLL][8];
  int64_t o[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    o[u] = (static_cast<int64_t>(blockIdx.x) * UNROLL + u) * kThreads + threadIdx.x;
    if (o[u] < n_oct) {
      load8(x, o[u], f[u]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[u][i] = 0u;
    }
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, f[u][i] & 0x7FFFFFFFu);
    uint32_t X = e8m0_of_amax<UOS>(quad_max_u32(m));
    uint32_t r = pack8(f[u], inv_scale_of(X));
    if (o[u] < n_oct_write) {
      __builtin_nontemporal_store(r, codes + o[u]);
      if ((threadIdx.x & 3) == 0) scales[o[u] >> 2] = static_cast<uint8_t>(X);
    }
  }
}

// Blocks along ROWS of [rows][cols] matrices, transposed output.  One
// workgroup stages a 64-row x 128-column tile in LDS (fp32, padded row to
// avoid bank conflicts on column reads), then each thread quantizes one
// 32-row block of one column and writes its 16 code bytes and scale byte.
constexpr int kColTileR = 64;
constexpr int kColTileC = 128;

template <typename In>
__device__ __forceinline__ float load1(const In* p);
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}
template <>
__device__ __forceinline__ float load1<float>(const float* p) {
  return *p;
}

template <typename In, int UOS>
__global__ __launch_bounds__(kThreads) void quant_cols_kernel(
    const In* __restrict__ x, int64_t rows, int64_t cols, int64_t rows_pad,
    uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t) {
  __shared__ float tile[kColTileR][kColTileC + 1];
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kColTileC;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kColTileR;
  const int64_t b = blockIdx.z;
  const In* xb = x + b * rows * cols;
  const int tc = threadIdx.x % kColTileC;
  const int tr = threadIdx.x / kColTileC;  // 0..1
#pragma unroll 4
  for (int i = 0; i < kColTileR / 2; ++i) {
    int r = tr + 2 * i;
    int64_t gr = r0 + r, gc = c0 + tc;
    tile[r][tc] = (gr < rows && gc < cols) ? load1<In>(xb + gr * cols + gc) : 0.0f;
  }
  __syncthreads();
  const int64_t gc = c0 + tc;
  const int kb = tr;  // which 32-row block of the tile
  const int64_t gr0 = r0 + kb * kBlock;
  if (gc >= cols || gr0 >= rows_pad) return;
  uint32_t f[kBlock];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kBlock; ++i) {
    f[i] = __float_as_uint(tile[kb * kBlock + i][tc]);
    m = max(m, f[i] & 0x7FFFFFFFu);
  }
  uint32_t X = e8m0_of_amax<UOS>(m);
  float inv = inv_scale_of(X);
  uint4 out;
  out.x = pack8(f + 0, inv);
  out.y = pack8(f + 8, inv);
  out.z = pack8(f + 16, inv);
  out.w = pack8(f + 24, inv);
  const int64_t col = b * cols + gc;
  *reinterpret_cast<uint4*>(codes_t + col * (rows_pad / 2) + gr0 / 2) = out;
  scales_t[col * (rows_pad / kBlock) + gr0 / kBlock] = static_cast<uint8_t>(X);
}

// KV tile images (layout in include/mxattn.h).  Rows at or past `rows` are
// quantized as zeros (codes 0, E8M0 byte 0).
//
// Key order inside a tile: accumulator lane l, register r of the S^T product
// of key subtile t (32 keys) holds row 8(r/4) + 4(l/32) + r%4 of that
// subtile; the subtile's rows are the keys
//   64 (t/2) + 32 (row/4 % 2) + 16 (t%2) + 4 (row/8) + row%4,
// so that register r of lane l, over the subtiles 2s and 2s+1, runs through
// the 32 keys 64 s + 32 (l/32) + 16 (t%2) + r: one whole P~ block of the
// lane's query, in key order.  Inverting it, key kk of a tile sits in
// subtile 2 (kk/64) + (kk%32)/16 at row 8 ((kk%16)/4) + 4 ((kk%64)/32) + kk%4.
__device__ __forceinline__ int kimg_subtile(int kk) { return 2 * (kk >> 6) + ((kk & 31) >> 4); }
__device__ __forceinline__ int kimg_row(int kk) { return 8 * ((kk & 15) >> 2) + 4 * ((kk & 63) >> 5) + (kk & 3); }

// K~: octet-per-lane as in quant_rows_kernel; block (row kr, d-block c)
// lands in subtile kimg_subtile, d-half c/2, lane kimg_row + 32 (c%2) of its
// tile, the A-operand order of the S^T product (lane l: row l%32, d-block
// 2 (d-half) + l/32).
template <typename In, int UOS, int D>
__global__ __launch_bounds__(kThreads) void quant_kimg_kernel(
    const In* __restrict__ x, int rows, int ntiles, int blocks_per_batch,
    uint8_t* __restrict__ img, const int32_t* __restrict__ lens, int per_len,
    uint32_t* __restrict__ cnt) {
  constexpr int OPR = D / 8;  // octets per row
  constexpr int DH = D / 64;  // d-halves (one 64-wide contraction each)
  constexpr int IMG = img_bytes(D);
  const int bgi = blockIdx.x / blocks_per_batch;
  // octet index within this (b, KV head): up to ntiles * 128 * D/8, past
  // 32 bits for the longest key extents
  const int64_t o = static_cast<int64_t>(blockIdx.x % blocks_per_batch) * kThreads + threadIdx.x;
  // the short-query kernel's arrival counter of this (b, KV head) starts at 0
  if (cnt && o == 0) cnt[bgi] = 0u;
  if (o >= static_cast<int64_t>(ntiles) * kKvTile * OPR) return;  // whole quads: OPR is a multiple of 4
  const int kr = static_cast<int>(o / OPR);
  const int w = static_cast<int>(o % OPR);
  // rows of this sequence: all, or its own length (rows past it are zeros)
  const int valid = lens ? min(max(lens[bgi / per_len], 0), rows) : rows;
  uint32_t f[8];
  if (kr < valid) {
    load8(x + (static_cast<int64_t>(bgi) * rows + kr) * D, w, f);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = 0u;
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, f[i] & 0x7FFFFFFFu);
  const uint32_t X = e8m0_of_amax<UOS>(quad_max_u32(m));
  const uint32_t r = pack8(f, inv_scale_of(X));
  const int c = w >> 2, part = w & 3;
  const int kk = kr % kKvTile;
  const int t = kimg_subtile(kk);
  const int l = kimg_row(kk) + 32 * (c & 1);
  const int op = t * DH + (c >> 1);  // operand index of (subtile, d-half)
  uint8_t* base = img + (static_cast<int64_t>(bgi) * ntiles + kr / kKvTile) * IMG;
  *reinterpret_cast<uint32_t*>(base + kImgKc + op * 1024 + l * 16 + part * 4) = r;
  if (part == 0) base[img_ks(D) + l * (D / 16) + op] = static_cast<uint8_t>(X);
  // zero the padding at the end of the image
  constexpr int kPadOff = img_vs(D) + 4 * D;
  const int pi = kk * OPR + w;
  if (pi < (IMG - kPadOff) / 4) *reinterpret_cast<uint32_t*>(base + kPadOff + pi * 4) = 0u;
}

// V~: blocks of 32 consecutive rows per channel.  A thread owns one 32-row
// block of 16 bytes' worth of channels (8 bf16 or 4 fp32): 32 row loads of
// 16 bytes, each wave instruction covering whole rows.  Block (channel d,
// row block kb; b = kb % 4 within its tile) lands in channel tile d / 32,
// key step b / 2, lane d % 32 + 32 (b % 2): the A-operand order of the O^T
// product (lane l: channel l%32, keys 64 (step) + 32 (l/32) .. +31).
template <typename In>
__device__ __forceinline__ uint32_t lane_bits(const uint4& r, int ch);
template <>
__device__ __forceinline__ uint32_t lane_bits<uint16_t>(const uint4& r, int ch) {
  const uint32_t wv = (ch >> 1) == 0 ? r.x : (ch >> 1) == 1 ? r.y : (ch >> 1) == 2 ? r.z : r.w;
  return (ch & 1) ? (wv & 0xFFFF0000u) : (wv << 16);
}
template <>
__device__ __forceinline__ uint32_t lane_bits<float>(const uint4& r, int ch) {
  return ch == 0 ? r.x : ch == 1 ? r.y : ch == 2 ? r.z : r.w;
}

template <typename In, int UOS, int D>
__global__ __launch_bounds__(kThreads) void quant_vimg_kernel(
    const In* __restrict__ x, int rows, int ntiles, int blocks_per_batch,
    uint8_t* __restrict__ img, const int32_t* __restrict__ lens, int per_len) {
  constexpr int CPT = 16 / static_cast<int>(sizeof(In));  // channels per thread
  constexpr int NCG = D / CPT;
  constexpr int IMG = img_bytes(D);
  const int bgi = blockIdx.x / blocks_per_batch;
  const int64_t i = static_cast<int64_t>(blockIdx.x % blocks_per_batch) * kThreads + threadIdx.x;
  if (i >= static_cast<int64_t>(ntiles) * (kKvTile / kBlock) * NCG) return;
  const int cg = static_cast<int>(i % NCG), kb = static_cast<int>(i / NCG);
  const int valid = lens ? min(max(lens[bgi / per_len], 0), rows) : rows;
  const In* src = x + (static_cast<int64_t>(bgi) * rows + kb * kBlock) * D + cg * CPT;
  uint4 r[kBlock];
#pragma unroll
  for (int k = 0; k < kBlock; ++k)
    if (kb * kBlock + k < valid) {
      const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(k) * D));
      r[k] = make_uint4(t[0], t[1], t[2], t[3]);
    } else {
      r[k] = make_uint4(0u, 0u, 0u, 0u);
    }
  uint8_t* base = img + (static_cast<int64_t>(bgi) * ntiles + kb / (kKvTile / kBlock)) * IMG;
  const int bt = kb % (kKvTile / kBlock);  // block within the tile
  const int step = bt >> 1;
#pragma unroll
  for (int ch = 0; ch < CPT; ++ch) {
    uint32_t f[kBlock];
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < kBlock; ++k) {
      f[k] = lane_bits<In>(r[k], ch);
      m = max(m, f[k] & 0x7FFFFFFFu);
    }
    const uint32_t X = e8m0_of_amax<UOS>(m);
    const float inv = inv_scale_of(X);
    uint4 out;
    out.x = pack8(f + 0, inv);
    out.y = pack8(f + 8, inv);
    out.z = pack8(f + 16, inv);
    out.w = pack8(f + 24, inv);
    const int d = cg * CPT + ch;
    const int l = (d & 31) + 32 * (bt & 1);
    const int op = (d >> 5) * 2 + step;  // operand index of (channel tile, key step)
    *reinterpret_cast<uint4*>(base + img_vc(D) + op * 1024 + l * 16) = out;
    base[img_vs(D) + l * (D / 16) + op] = static_cast<uint8_t>(X);
  }
}

// Dequantize: each lane expands UNROLL dwords of codes (8 elements each), a
// workgroup's lanes taking consecutive dwords in each of UNROLL rounds, so
// every wave instruction reads 256 contiguous bytes of codes and writes
// 1 KiB (bf16) or 2 KiB (fp32) of contiguous output; all loads of a lane
// are issued before its first store.
// Magnitudes times 2: {0,1,2,3,4,6,8,12} packed as nibbles.
__device__ __forceinline__ float dq(uint32_t code, int ex) {
  uint32_t m2 = (0xC8643210u >> (4u * (code & 7u))) & 0xFu;
  float v = __builtin_amdgcn_ldexpf(static_cast<float>(m2), ex);
  return (code & 8u) ? -v : v;
}

template <int OUT_BF16, int UNROLL>
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    int64_t n_oct, void* __restrict__ y) {
  uint32_t c[UNROLL], X[UNROLL];
  int64_t o[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    o[u] = (static_cast<int64_t>(blockIdx.x) * UNROLL + u) * kThreads + threadIdx.x;
    c[u] = 0;
    X[u] = 127;
    if (o[u] < n_oct) {
      c[u] = __builtin_nontemporal_load(codes + o[u]);
      X[u] = scales[o[u] >> 2];
    }
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    if (o[u] >= n_oct) continue;
    const int ex = static_cast<int>(X[u]) - 128;  // magnitude*2 * 2^(X-128)
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (X[u] == 255u) ? __builtin_nanf("") : dq((c[u] >> (4 * i)) & 0xFu, ex);
    if (OUT_BF16) {
      uint4 w;
      w.x = (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xFFFF0000u);
      w.y = (__float_as_uint(v[2]) >> 16) | (__float_as_uint(v[3]) & 0xFFFF0000u);
      w.z = (__float_as_uint(v[4]) >> 16) | (__float_as_uint(v[5]) & 0xFFFF0000u);
      w.w = (__float_as_uint(v[6]) >> 16) | (__float_as_uint(v[7]) & 0xFFFF0000u);
      const u32x4 wv = {w.x, w.y, w.z, w.w};
      __builtin_nontemporal_store(wv, reinterpret_cast<u32x4*>(y) + o[u]);
    } else {
      u32x4* p = reinterpret_cast<u32x4*>(y) + 2 * o[u];
      const u32x4 w0 = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
      const u32x4 w1 = {__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])};
      __builtin_nontemporal_store(w0, p);
      __builtin_nontemporal_store(w1, p + 1);
    }
  }
}

template <typename In, int UOS, int D>
hipError_t launch_kv_images_t(const void* k, const void* v, int64_t batch, int rows,
                              int ntiles, uint8_t* img, const int32_t* lens, int per_len,
                              uint32_t* cnt, hipStream_t stream) {
  // work items per (b, KV head) in 64 bits; the C ABI has checked that
  // batch * per-batch blocks fits the grid's 32-bit dimension
  const int64_t kper = (static_cast<int64_t>(ntiles) * kKvTile * (D / 8) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((quant_kimg_kernel<In, UOS, D>), dim3(static_cast<unsigned>(batch * kper)),
                     dim3(kThreads), 0, stream, static_cast<const In*>(k), rows, ntiles, static_cast<int>(kper), img,
                     lens, per_len, cnt);
  constexpr int CPT = 16 / static_cast<int>(sizeof(In));
  const int64_t vper = (static_cast<int64_t>(ntiles) * (kKvTile / kBlock) * (D / CPT) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((quant_vimg_kernel<In, UOS, D>), dim3(static_cast<unsigned>(batch * vper)),
                     dim3(kThreads), 0, stream, static_cast<const In*>(v), rows, ntiles, static_cast<int>(vper), img,
                     lens, per_len);
  return hipGetLastError();
}

template <typename In, int UOS>
hipError_t launch_kv_images_d(const void* k, const void* v, int64_t batch, int rows, int D,
                              int ntiles, uint8_t* img, const int32_t* lens, int per_len,
                              uint32_t* cnt, hipStream_t stream) {
  return D == 64 ? launch_kv_images_t<In, UOS, 64>(k, v, batch, rows, ntiles, img, lens, per_len, cnt, stream)
                 : launch_kv_images_t<In, UOS, 128>(k, v, batch, rows, ntiles, img, lens, per_len, cnt, stream);
}

}  // namespace

hipError_t launch_quant_kv_images(const void* k, const void* v, int64_t batch, int rows,
                                  int D, Dtype dt, int uos, uint8_t* img,
                                  const int32_t* lens, int per_len, uint32_t* cnt,
                                  hipStream_t stream) {
  if (batch <= 0 || rows <= 0) return hipSuccess;
  const int ntiles = (rows + kKvTile - 1) / kKvTile;
  if (dt == Dtype::BF16)
    return uos ? launch_kv_images_d<uint16_t, 1>(k, v, batch, rows, D, ntiles, img, lens, per_len, cnt, stream)
               : launch_kv_images_d<uint16_t, 0>(k, v, batch, rows, D, ntiles, img, lens, per_len, cnt, stream);
  return uos ? launch_kv_images_d<float, 1>(k, v, batch, rows, D, ntiles, img, lens, per_len, cnt, stream)
             : launch_kv_images_d<float, 0>(k, v, batch, rows, D, ntiles, img, lens, per_len, cnt, stream);
}

hipError_t launch_quant_rows(const void* x, int64_t n, int64_t n_write, Dtype dt,
                             int uos, uint8_t* codes, uint8_t* scales,
                             hipStream_t stream) {
  if (n_write <= 0) return hipSuccess;
  constexpr int U = 2;
  const int64_t n_oct = n / 8, n_oct_w = n_write / 8;
  const int64_t per_block = static_cast<int64_t>(kThreads) * U;
  dim3 grid(static_cast<unsigned>((n_oct_w + per_block - 1) / per_block));
  uint32_t* c32 = reinterpret_cast<uint32_t*>(codes);
  if (dt == Dtype::BF16) {
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    if (uos)
      hipLaunchKernelGGL((quant_rows_kernel<uint16_t, 1, U>), grid, dim3(kThreads), 0, stream, xp, n_oct, n_oct_w, c32, scales);
    else
      hipLaunchKernelGGL((quant_rows_kernel<uint16_t, 0, U>), grid, dim3(kThreads), 0, stream, xp, n_oct, n_oct_w, c32, scales);
  } else {
    const float* xp = static_cast<const float*>(x);
    if (uos)
      hipLaunchKernelGGL((quant_rows_kernel<float, 1, U>), grid, dim3(kThreads), 0, stream, xp, n_oct, n_oct_w, c32, scales);
    else
      hipLaunchKernelGGL((quant_rows_kernel<float, 0, U>), grid, dim3(kThreads), 0, stream, xp, n_oct, n_oct_w, c32, scales);
  }
  return hipGetLastError();
}

hipError_t launch_quant_cols(const void* x, int64_t batch, int64_t rows,
                             int64_t cols, int64_t rows_pad, Dtype dt, int uos,
                             uint8_t* codes_t, uint8_t* scales_t,
                             hipStream_t stream) {
  if (batch <= 0 || cols <= 0 || rows_pad <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((cols + kColTileC - 1) / kColTileC),
            static_cast<unsigned>((rows_pad + kColTileR - 1) / kColTileR),
            static_cast<unsigned>(batch));
  if (dt == Dtype::BF16) {
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    if (uos)
      hipLaunchKernelGGL((quant_cols_kernel<uint16_t, 1>), grid, dim3(kThreads), 0, stream, xp, rows, cols, rows_pad, codes_t, scales_t);
    else
      hipLaunchKernelGGL((quant_cols_kernel<uint16_t, 0>), grid, dim3(kThreads), 0, stream, xp, rows, cols, rows_pad, codes_t, scales_t);
  } else {
    const float* xp = static_cast<const float*>(x);
    if (uos)
      hipLaunchKernelGGL((quant_cols_kernel<float, 1>), grid, dim3(kThreads), 0, stream, xp, rows, cols, rows_pad, codes_t, scales_t);
    else
      hipLaunchKernelGGL((quant_cols_kernel<float, 0>), grid, dim3(kThreads), 0, stream, xp, rows, cols, rows_pad, codes_t, scales_t);
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n,
                          int out_bf16, void* y, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  constexpr int U = 4;
  const int64_t n_oct = n / 8;
  const int64_t per_block = static_cast<int64_t>(kThreads) * U;
  dim3 grid(static_cast<unsigned>((n_oct + per_block - 1) / per_block));
  const uint32_t* c32 = reinterpret_cast<const uint32_t*>(codes);
  if (out_bf16)
    hipLaunchKernelGGL((dequant_kernel<1, U>), grid, dim3(kThreads), 0, stream, c32, scales, n_oct, y);
  else
    hipLaunchKernelGGL((dequant_kernel<0, U>), grid, dim3(kThreads), 0, stream, c32, scales, n_oct, y);
  return hipGetLastError();
}

}  // namespace mxk
