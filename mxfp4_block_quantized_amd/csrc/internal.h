// Internal launch interface between the C ABI (capi.cpp) and the HIP
// kernels.  Host-side declarations only; every launcher enqueues on `stream`
// and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>
#include <algorithm>

namespace mxk {

// E8M0 / E2M1 element block size.
constexpr int kBlock = 32;

// Keys per KV tile of both attention kernels (the running-max schedule).
constexpr int kKvTile = 128;
// Query rows per workgroup of the 16-bit attention kernel.
constexpr int kQTile = 128;
// Query rows per workgroup of the MXFP4 attention kernel.
constexpr int kMxQTile = 128;
// Keys per KV tile of the 16-bit (FP16-mode) attention kernel.
constexpr int kF16KvTile = 64;

// KV tile image: the quantized K~ and V~ of one 128-key tile, stored in the
// operand order of v_mfma_scale_f32_32x32x64_f8f6f4 so that the attention
// kernels move it to LDS with contiguous 16-byte-per-lane loads (layout in
// include/mxattn.h):
//   K~ codes  [subtile 4][d-half D/64][lane 64][16 B]   at kImgKc
//   V~ codes  [channel tile D/32][key step 2][lane][16 B] at img_vc(D)
//   K~ scales [lane][subtile * D/64 + d-half]          at img_ks(D)
//   V~ scales [lane][channel tile * 2 + key step]      at img_vs(D)
// then zero padding to a whole number of KiB.
constexpr int kImgKc = 0;
__host__ __device__ constexpr int img_vc(int D) { return 64 * D; }
__host__ __device__ constexpr int img_ks(int D) { return 128 * D; }
__host__ __device__ constexpr int img_vs(int D) { return 132 * D; }
__host__ __device__ constexpr int img_bytes(int D) { return (136 * D + 1023) / 1024 * 1024; }

// 16-bit tile image of the FP16 mode (64 keys): K as [subtile 4][step D/32]
// [lane 64][8 x 16-bit], then V^T (fp16) as [channel tile D/16][key group 2]
// [lane 64][8 x fp16].
__host__ __device__ constexpr int f16_img_vc(int D) { return kF16KvTile * D * 2; }
__host__ __device__ constexpr int f16_img_bytes(int D) { return 2 * kF16KvTile * D * 2; }

enum class Dtype : int { F32 = 0, BF16 = 1 };

// Quantize n elements (n % 32 == 0) along the contiguous axis; elements in
// [n, n_write) are treated as zero (used to zero-fill padding rows).
hipError_t launch_quant_rows(const void* x, int64_t n, int64_t n_write, Dtype dt,
                             int uos, uint8_t* codes, uint8_t* scales,
                             hipStream_t stream);

// Quantize batch x [rows][cols] along rows, transposed output with row
// length rows_pad (multiple of 32, >= rows).
hipError_t launch_quant_cols(const void* x, int64_t batch, int64_t rows,
                             int64_t cols, int64_t rows_pad, Dtype dt, int uos,
                             uint8_t* codes_t, uint8_t* scales_t,
                             hipStream_t stream);

// Quantize K [batch][rows][D] (blocks along D) and V [batch][rows][D]
// (blocks along rows) into KV tile images [batch][ntiles][img_bytes(D)],
// ntiles = ceil(rows / kKvTile); rows past the end are quantized as zeros.
// lens (device, may be null): entry e of the batch holds lens[e / per_len]
// valid rows (clamped to [0, rows]); its rows past that are zeros too.
// cnt (device, may be null): batch words set to 0 (the short-query kernel's
// arrival counters, one per (b, KV head)).
hipError_t launch_quant_kv_images(const void* k, const void* v, int64_t batch, int rows,
                                  int D, Dtype dt, int uos, uint8_t* img,
                                  const int32_t* lens, int per_len, uint32_t* cnt,
                                  hipStream_t stream);

// Dequantize n elements to fp32 (out_bf16 == 0) or bf16.
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n,
                          int out_bf16, void* y, hipStream_t stream);

// Operands of the MXFP4 attention kernel (all device pointers).
struct MxAttnArgs {
  const void* q;       // [B][Hq][Sq][D] bf16 (q_bf16) or fp32, quantized in the kernel
  int q_bf16;
  // per-sequence lengths (device, may be null): batch entry b has lens_q[b]
  // query rows (<= Sq) and lens_k[b] keys (<= Skv); causal queries are
  // aligned to the end of the keys
  const int32_t* lens_q;
  const int32_t* lens_k;
  uint8_t* qc;         // dump only: the kernel's Q~ codes [B*Hq*Sq][D/2]
  uint8_t* qs;         // dump only: the kernel's Q~ E8M0 bytes [B*Hq*Sq][D/32]
  const uint8_t* img;  // KV tile images [B*Hkv][skv_ld/128][img_bytes(D)]
  float* o;            // [B][Hq][Sq][D]
  const int32_t* row_slot;  // dump only: [B*Hq*Sq]
  uint8_t* p_codes;         // dump only: [nslots][skv_ld/2]
  uint8_t* p_scales;        // dump only: [nslots][skv_ld/32]
  int B, Hq, Hkv, Sq, Skv, D;
  int64_t skv_ld;
  int causal;
  int mode;  // 1 OCP, 2 UOS, 3 UOS+PNQ, 4 UOS+EFQ
  // the prefill kernel's work-queue counters (kQueueWords words; the
  // launcher clears them before the kernel)
  uint32_t* queue;
};
hipError_t launch_attn_mx(const MxAttnArgs& a, hipStream_t stream);

// Work queue of the prefill kernels (both attention kernels): their items
// (query tiles, or causal pairs of them) are listed in 8 runs, one per XCD; a workgroup on XCD x takes
// item j of run x when j falls in the run's first 7/8, and otherwise pops
// the run's remaining items from counter x, then the other runs' (so the
// XCDs that run faster take over the ends of the slower ones).  The grid
// holds per-XCD spares for that.
constexpr int kQueueWords = 8;
__host__ __device__ constexpr int64_t prefill_items_per_xcd(int64_t nitems) { return (nitems + 7) / 8; }
__host__ __device__ constexpr int64_t prefill_grid(int64_t nitems) {
  return 8 * (prefill_items_per_xcd(nitems) + prefill_items_per_xcd(nitems) / 16 + 2);
}

// Short-query attention over key splits: one wave per (b, KV head, split)
// computes the partial softmax state of the (Hq/Hkv) x Sq queries of a GQA
// group (at most kDecodeCols) over its keys; the last wave of a group to
// finish (counted in cnt) merges the group's splits in order into o and sets
// its counter back to 0.  Causal queries are aligned to the end of the keys.
struct MxDecodeArgs {
  MxAttnArgs at;      // Q~, KV images, o, dump, shapes, mode (at.causal: end-aligned)
  float* part;        // [B*Hkv*nsplit][kDecodeCols][decode_slot(D)]: m, l, 2 unused, unnormalized O
  uint32_t* cnt;      // [B*Hkv] arrival counters, 0 on entry (left at 0)
  int split_tiles;    // KV tiles (128 keys) per split
  int nsplit;
  // per-sequence lengths only (at.lens_k set, B <= kCompactMaxB): waves take
  // the splits that hold keys, numbered consecutively, instead of every
  // (b, KV head, split) of the padded extent
  int compact;
};
// Query columns of one short-query wave (one 32 x 32 matrix-core tile).
constexpr int kDecodeCols = 32;
// Floats per query column of a split's partial state (O 16-byte aligned).
__host__ __device__ constexpr int decode_slot(int D) { return D + 4; }
// Largest batch for which the short-query kernel numbers its busy splits
// (each wave scans the B lengths).
constexpr int kCompactMaxB = 256;
hipError_t launch_attn_decode(const MxDecodeArgs& a, hipStream_t stream);

// W4A4 product y[M][N] = a[M][K] b[N][K]^T of MXFP4 operands (codes
// [rows][K/2], E8M0 [rows][K/32]); K % 128 == 0; fp32 (out_bf16 == 0) or
// bf16 output.  ws: gemm_workspace_bytes(M, N, K) bytes, 256-byte aligned
// (the operands' E8M0 bytes re-laid out for the kernel).
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_mx(const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K, int out_bf16,
                          void* y, uint8_t* ws, hipStream_t stream);
// The library's own GEMM scratch (gemm_mx.hip): kGemmScratchBytes per GPU;
// *out = this device's address of it (looked up once per device).
constexpr size_t kGemmScratchBytes = size_t(32) << 20;
hipError_t gemm_scratch(uint8_t** out);

// Operands of the 16-bit attention kernel.
struct F16AttnArgs {
  const void* q;       // [B][Hq][Sq][D], bf16 (qk_f16 == 0) or fp16
  const uint8_t* img;  // 16-bit tile images [B*Hkv][ceil(Skv/64)][f16_img_bytes(D)]
  float* o;
  int B, Hq, Hkv, Sq, Skv, D;
  int64_t skv_ld;
  int causal;
  int qk_f16;  // 1: q/k are fp16, 0: bf16
  uint32_t* queue;  // work-queue counters as for the MXFP4 prefill kernel
};
hipError_t launch_attn_f16(const F16AttnArgs& a, hipStream_t stream);

// FP16-mode operand preparation: K and V [batch][rows][D] (bf16 or fp32)
// into 16-bit tile images (K kept as bf16 for bf16 inputs, else fp16; V^T
// fp16), rows past the end zero; and fp32 -> fp16 conversion of n elements
// (zero-filling [n, n_write)).
hipError_t launch_f16_images(const void* k, const void* v, int64_t batch, int rows, int D,
                             Dtype dt, uint8_t* img, hipStream_t stream);
hipError_t launch_f32_to_f16(const float* x, int64_t n, int64_t n_write,
                             uint16_t* y, hipStream_t stream);

}  // namespace mxk
