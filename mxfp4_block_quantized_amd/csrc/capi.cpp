// C ABI of the MXFP4 quantizer, MXFP4 attention and the W4A4 product (see
// include/mxattn.h):
// argument validation (always before any HIP call), workspace layout and
// dispatch to the HIP launchers.
#include "mxattn.h"

#include <cstdint>
#include <limits>

#include "internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int to_status(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Byte layout of the workspace used by mxattn_fwd.  MX modes: the KV tile
// images first, then one arrival counter per (b, KV head) for the
// short-query kernel (zeroed with the images), the prefill kernel's work
// queue (cleared before each launch), then the Q~ codes and E8M0 bytes that
// only the dump variants write (total: images and counters; total_dump:
// with Q~).
struct Layout {
  size_t off[6];  // MX: qc qs images img-bytes | FP16: images, q16
  size_t cnt;     // MX: the arrival counters
  size_t queue;   // MX: the work-queue counters
  size_t total;
  size_t total_dump;
  int64_t skv_ld;
};

// A dispatch's work-item count per grid dimension is a 32-bit value on this
// runtime: shapes whose launches would exceed it are rejected up front.
constexpr int64_t kMaxItems = (int64_t(1) << 32) - 1;

// The attention launches (query-tile workgroups of 256 threads; operand
// preparation: MX K tile images one thread per 8 elements of the 128-key
// padded rows, the V images fewer; FP16 images one 256-thread workgroup per
// 64-key tile, fp32 Q one thread per element).
bool attn_grids_fit(int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype, int mode) {
  const int64_t qt = mode == MXATTN_FP16 ? mxk::kQTile : mxk::kMxQTile;
  if (static_cast<int64_t>(B) * Hq * ((Sq + qt - 1) / qt) * 256 > kMaxItems) return false;
  // the prefill grids add their per-XCD spares
  if (mxk::prefill_grid(static_cast<int64_t>(B) * Hq * ((Sq + qt - 1) / qt)) * 256 > kMaxItems)
    return false;
  if (mode == MXATTN_FP16) {
    const int64_t nt = (static_cast<int64_t>(Skv) + mxk::kF16KvTile - 1) / mxk::kF16KvTile;
    if (static_cast<int64_t>(B) * Hkv * nt * 256 > kMaxItems) return false;
    if (dtype == MX_F32 && static_cast<int64_t>(B) * Hq * Sq * D > kMaxItems) return false;
    return true;
  }
  const int64_t nt = (static_cast<int64_t>(Skv) + mxk::kKvTile - 1) / mxk::kKvTile;
  return static_cast<int64_t>(B) * Hkv * nt * mxk::kKvTile * (D / 8) <= kMaxItems;
}

int check_attn_shape(int dtype, int B, int Hq, int Hkv, int Sq, int Skv, int D,
                     int causal, int mode) {
  if (dtype != MX_F32 && dtype != MX_BF16) return MX_ERR_ARG;
  if (mode < MXATTN_FP16 || mode > MXATTN_UOS_EFQ) return MX_ERR_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || D < 1) return MX_ERR_ARG;
  if (causal != 0 && causal != 1) return MX_ERR_ARG;
  if (Hq % Hkv != 0) return MX_ERR_ARG;
  if (D != 64 && D != 128) return MX_ERR_UNSUPPORTED;
  if (causal && Sq != Skv) return MX_ERR_UNSUPPORTED;
  if (B > 65535 || Hq > 65535) return MX_ERR_UNSUPPORTED;
  // element counts must fit the kernels' 64-bit indexing comfortably and
  // the per-head row count must fit int32 tiles
  if (static_cast<int64_t>(B) * Hq * Sq * D > (int64_t(1) << 40)) return MX_ERR_UNSUPPORTED;
  // likewise K and V (this also keeps the workspace size far from overflow)
  if (static_cast<int64_t>(B) * Hkv * Skv * D > (int64_t(1) << 40)) return MX_ERR_UNSUPPORTED;
  if (!attn_grids_fit(B, Hq, Hkv, Sq, Skv, D, dtype, mode)) return MX_ERR_UNSUPPORTED;
  return MX_OK;
}

Layout make_layout(int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype, int mode) {
  Layout L{};
  const int64_t skv_ld = (static_cast<int64_t>(Skv) + mxk::kKvTile - 1) / mxk::kKvTile * mxk::kKvTile;
  L.skv_ld = skv_ld;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    size_t o = cur;
    cur = round_up(cur + bytes, 256);
    return o;
  };
  if (mode == MXATTN_FP16) {
    const size_t nt = (static_cast<size_t>(Skv) + mxk::kF16KvTile - 1) / mxk::kF16KvTile;
    L.off[0] = take(static_cast<size_t>(B) * Hkv * nt * mxk::f16_img_bytes(D));  // K / V^T images
    if (dtype == MX_F32) L.off[1] = take(static_cast<size_t>(B) * Hq * Sq * D * 2);  // Q fp16
    L.queue = take(mxk::kQueueWords * sizeof(uint32_t));
    L.total = L.total_dump = cur;
  } else {
    L.off[2] = take(static_cast<size_t>(B) * Hkv * (skv_ld / mxk::kKvTile) * mxk::img_bytes(D));
    L.cnt = take(static_cast<size_t>(B) * Hkv * sizeof(uint32_t));
    L.queue = take(mxk::kQueueWords * sizeof(uint32_t));
    L.total = cur;
    // the kernel's Q~ (dump variants only), one row per query row
    const size_t q_rows = static_cast<size_t>(B) * Hq * Sq;
    L.off[0] = take(q_rows * D / 2);
    L.off[1] = take(q_rows * D / 32);
    L.off[3] = static_cast<size_t>(mxk::img_bytes(D));
    L.off[4] = 0;
    L.off[5] = 0;
    L.total_dump = cur;
  }
  return L;
}

// Validation shared by every attention entry point.
int check_attn_call(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                    int Hkv, int Sq, int Skv, int D, int causal, int mode, const void* ws,
                    size_t ws_bytes, bool need_qk, bool need_v, Layout* L, bool dump = false) {
  int st = check_attn_shape(dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode);
  if (st != MX_OK) return st;
  if ((need_qk && (!q || !k)) || (need_v && !v)) return MX_ERR_ARG;
  if ((q && !aligned(q, 16)) || (k && !aligned(k, 16)) || (v && !aligned(v, 16)))
    return MX_ERR_ALIGN;
  *L = make_layout(B, Hq, Hkv, Sq, Skv, D, dtype, mode);
  if (!ws || ws_bytes < (dump ? L->total_dump : L->total)) return MX_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MX_ERR_ALIGN;
  return MX_OK;
}

// Operand preparation into the workspace (arguments already validated).
int run_prepare(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                int Hkv, int Sq, int Skv, int D, int mode, const Layout& L, void* ws,
                hipStream_t s, const int32_t* lens_k = nullptr) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  const mxk::Dtype dt = dtype == MX_BF16 ? mxk::Dtype::BF16 : mxk::Dtype::F32;
  const int64_t nq = static_cast<int64_t>(B) * Hq * Sq * D;
  hipError_t e;
  if (mode == MXATTN_FP16) {
    e = mxk::launch_f16_images(k, v, static_cast<int64_t>(B) * Hkv, Skv, D, dt, w + L.off[0], s);
    if (e != hipSuccess) return MX_ERR_HIP;
    if (dtype == MX_F32) {
      e = mxk::launch_f32_to_f16(static_cast<const float*>(q), nq, nq,
                                 reinterpret_cast<uint16_t*>(w + L.off[1]), s);
      if (e != hipSuccess) return MX_ERR_HIP;
    }
    return MX_OK;
  }
  // MX modes: Q is quantized inside the attention kernels
  const int uos = (mode == MXATTN_OCP) ? 0 : 1;
  e = mxk::launch_quant_kv_images(k, v, static_cast<int64_t>(B) * Hkv, Skv, D, dt, uos,
                                  w + L.off[2], lens_k, Hkv,
                                  reinterpret_cast<uint32_t*>(w + L.cnt), s);
  return to_status(e);
}

// The fused attention kernel on a prepared workspace.
int run_attention(const void* q, const void* k, int dtype, int B, int Hq, int Hkv, int Sq,
                  int Skv, int D, int causal, int mode, float* o, const Layout& L,
                  void* ws, const int32_t* row_slot, uint8_t* p_codes,
                  uint8_t* p_scales, hipStream_t s, const int32_t* lens_q = nullptr,
                  const int32_t* lens_k = nullptr) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  if (mode == MXATTN_FP16) {
    mxk::F16AttnArgs a{};
    if (dtype == MX_F32) {
      a.q = w + L.off[1];
      a.qk_f16 = 1;
    } else {
      a.q = q;
      a.qk_f16 = 0;
    }
    a.img = w + L.off[0];
    a.o = o;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Skv = Skv; a.D = D;
    a.skv_ld = L.skv_ld;
    a.causal = causal;
    a.queue = reinterpret_cast<uint32_t*>(w + L.queue);
    return to_status(mxk::launch_attn_f16(a, s));
  }
  mxk::MxAttnArgs a{};
  a.q = q;
  a.q_bf16 = dtype == MX_BF16;
  a.lens_q = lens_q;
  a.lens_k = lens_k;
  // written only by the dump variant
  a.qc = w + L.off[0];
  a.qs = w + L.off[1];
  a.img = w + L.off[2];
  a.o = o;
  a.row_slot = row_slot;
  a.p_codes = p_codes;
  a.p_scales = p_scales;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Skv = Skv; a.D = D;
  a.skv_ld = L.skv_ld;
  a.causal = causal;
  a.mode = mode;
  a.queue = reinterpret_cast<uint32_t*>(w + L.queue);
  return to_status(mxk::launch_attn_mx(a, s));
}

int attn_common(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                int Hkv, int Sq, int Skv, int D, int causal, int mode, float* o, void* ws,
                size_t ws_bytes, const int32_t* row_slot, uint8_t* p_codes,
                uint8_t* p_scales, bool dump, void* stream) {
  Layout L;
  if (dump && mode == MXATTN_FP16) return MX_ERR_ARG;
  int st = check_attn_call(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, ws, ws_bytes,
                           true, true, &L, dump);
  if (st != MX_OK) return st;
  if (!o) return MX_ERR_ARG;
  if (!aligned(o, 16)) return MX_ERR_ALIGN;
  if (dump && (!row_slot || !p_codes || !p_scales)) return MX_ERR_ARG;
  if (dump && (!aligned(p_codes, 16) || !aligned(row_slot, 4))) return MX_ERR_ALIGN;
  hipStream_t s = as_stream(stream);
  st = run_prepare(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, mode, L, ws, s);
  if (st != MX_OK) return st;
  return run_attention(q, k, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, o, L, ws,
                       dump ? row_slot : nullptr, dump ? p_codes : nullptr,
                       dump ? p_scales : nullptr, s);
}

// ---- short-query attention over key splits ----

// KV tiles per split: at least 4 (the per-split partial state is small next
// to the keys it covers), more when the (b, KV head) groups alone give
// about 1024 waves (one workgroup of 4 waves per CU: the one-tile-ahead
// stream of each wave still covers the memory latency, and a group's merge
// reads half the partial states of 2048 waves).
int decode_split_tiles(int B, int Hkv, int Skv) {
  const int64_t nt = (static_cast<int64_t>(Skv) + mxk::kKvTile - 1) / mxk::kKvTile;
  const int64_t groups = static_cast<int64_t>(B) * Hkv;
  int64_t st = (nt * groups + 1023) / 1024;
  if (st < 4) st = 4;
  if (st < (nt + 1023) / 1024) st = (nt + 1023) / 1024;  // at most 1024 splits per group
  if (st > nt) st = nt;
  return static_cast<int>(st);
}

int check_decode_shape(int dtype, int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                       int mode) {
  if (dtype != MX_F32 && dtype != MX_BF16) return MX_ERR_ARG;
  if (mode < MXATTN_FP16 || mode > MXATTN_UOS_EFQ) return MX_ERR_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || D < 1) return MX_ERR_ARG;
  if (causal != 0 && causal != 1) return MX_ERR_ARG;
  if (Hq % Hkv != 0) return MX_ERR_ARG;
  if (mode == MXATTN_FP16) return MX_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return MX_ERR_UNSUPPORTED;
  if ((Hq / Hkv) * static_cast<int64_t>(Sq) > mxk::kDecodeCols) return MX_ERR_UNSUPPORTED;
  if (causal && Sq > Skv) return MX_ERR_UNSUPPORTED;
  if (B > 65535 || Hq > 65535) return MX_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(B) * Hkv * Skv * D > (int64_t(1) << 40)) return MX_ERR_UNSUPPORTED;
  // launches: the K/V images as for mxattn_fwd; one 64-lane wave per (b, KV
  // head, split) and per query row of the merge
  if (!attn_grids_fit(B, Hq, Hkv, Sq, Skv, D, dtype, mode)) return MX_ERR_UNSUPPORTED;
  const int64_t nt = (static_cast<int64_t>(Skv) + mxk::kKvTile - 1) / mxk::kKvTile;
  const int64_t st = decode_split_tiles(B, Hkv, Skv);
  if (static_cast<int64_t>(B) * Hkv * ((nt + st - 1) / st) * 64 > kMaxItems) return MX_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(B) * Hq * Sq * 64 > kMaxItems) return MX_ERR_UNSUPPORTED;
  return MX_OK;
}

struct DecodeLayout {
  Layout L;        // KV images and Q~ as for mxattn_fwd_dump
  size_t part;     // partial states
  size_t total;
  int split_tiles, nsplit;
};

DecodeLayout make_decode_layout(int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype,
                                int mode) {
  DecodeLayout dl;
  dl.L = make_layout(B, Hq, Hkv, Sq, Skv, D, dtype, mode);
  dl.split_tiles = decode_split_tiles(B, Hkv, Skv);
  const int64_t nt = dl.L.skv_ld / mxk::kKvTile;
  dl.nsplit = static_cast<int>((nt + dl.split_tiles - 1) / dl.split_tiles);
  // the Q~ regions of a decode shape are a few hundred bytes per query row:
  // always reserved, the partial states follow them
  dl.part = round_up(dl.L.total_dump, 256);
  dl.total = dl.part + static_cast<size_t>(B) * Hkv * dl.nsplit * mxk::kDecodeCols * mxk::decode_slot(D) * sizeof(float);
  return dl;
}

int decode_common(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                  int Hkv, int Sq, int Skv, int D, int causal, int mode, float* o, void* ws,
                  size_t ws_bytes, const int32_t* row_slot, uint8_t* p_codes,
                  uint8_t* p_scales, bool prepare, bool dump, void* stream,
                  const int32_t* lens_k = nullptr) {
  int st = check_decode_shape(dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode);
  if (st != MX_OK) return st;
  if (!q || (prepare && (!k || !v))) return MX_ERR_ARG;
  if (!o) return MX_ERR_ARG;
  if ((q && !aligned(q, 16)) || (k && !aligned(k, 16)) || (v && !aligned(v, 16)) ||
      !aligned(o, 16))
    return MX_ERR_ALIGN;
  if (dump && (!row_slot || !p_codes || !p_scales)) return MX_ERR_ARG;
  if (dump && (!aligned(p_codes, 16) || !aligned(row_slot, 4))) return MX_ERR_ALIGN;
  const DecodeLayout dl = make_decode_layout(B, Hq, Hkv, Sq, Skv, D, dtype, mode);
  if (!ws || ws_bytes < dl.total) return MX_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MX_ERR_ALIGN;
  hipStream_t s = as_stream(stream);
  if (prepare) {
    st = run_prepare(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, mode, dl.L, ws, s, lens_k);
    if (st != MX_OK) return st;
  }
  uint8_t* w = static_cast<uint8_t*>(ws);
  mxk::MxDecodeArgs d{};
  d.at.q = q;
  d.at.q_bf16 = dtype == MX_BF16;
  d.at.lens_k = lens_k;
  d.at.qc = w + dl.L.off[0];
  d.at.qs = w + dl.L.off[1];
  d.at.img = w + dl.L.off[2];
  d.at.o = o;
  d.at.row_slot = dump ? row_slot : nullptr;
  d.at.p_codes = dump ? p_codes : nullptr;
  d.at.p_scales = dump ? p_scales : nullptr;
  d.at.B = B; d.at.Hq = Hq; d.at.Hkv = Hkv; d.at.Sq = Sq; d.at.Skv = Skv; d.at.D = D;
  d.at.skv_ld = dl.L.skv_ld;
  d.at.causal = causal;
  d.at.mode = mode;
  d.part = reinterpret_cast<float*>(w + dl.part);
  d.cnt = reinterpret_cast<uint32_t*>(w + dl.L.cnt);
  d.split_tiles = dl.split_tiles;
  d.nsplit = dl.nsplit;
  // the busy splits numbered on the device (unit numbers are int there)
  d.compact = lens_k && B <= mxk::kCompactMaxB &&
              static_cast<int64_t>(B) * Hkv * dl.nsplit < (int64_t(1) << 31);
  return to_status(mxk::launch_attn_decode(d, s));
}

}  // namespace

extern "C" {

const char* mx_strerror(int status) {
  switch (status) {
    case MX_OK: return "success";
    case MX_ERR_ARG: return "invalid argument (null pointer, bad enum or size)";
    case MX_ERR_UNSUPPORTED: return "unsupported configuration";
    case MX_ERR_WORKSPACE: return "workspace missing or too small";
    case MX_ERR_HIP: return "HIP launch or runtime error";
    case MX_ERR_ALIGN: return "device pointer not suitably aligned";
    default: return "unknown status";
  }
}

int mxq_quantize(const void* x, int64_t n, int dtype, int mode, uint8_t* codes,
                 uint8_t* scales, void* stream) {
  if (n < 0 || n % mxk::kBlock != 0) return MX_ERR_ARG;
  if (dtype != MX_F32 && dtype != MX_BF16) return MX_ERR_ARG;
  if (mode != MXQ_OCP && mode != MXQ_UOS) return MX_ERR_ARG;
  if (n == 0) return MX_OK;
  if (n / 16 + 256 > kMaxItems) return MX_ERR_UNSUPPORTED;  // one thread per 16 elements
  if (!x || !codes || !scales) return MX_ERR_ARG;
  if (!aligned(x, 16) || !aligned(codes, 16)) return MX_ERR_ALIGN;
  const mxk::Dtype dt = dtype == MX_BF16 ? mxk::Dtype::BF16 : mxk::Dtype::F32;
  return to_status(mxk::launch_quant_rows(x, n, n, dt, mode == MXQ_UOS, codes, scales,
                                          as_stream(stream)));
}

int mxq_quantize_t(const void* x, int64_t batch, int64_t rows, int64_t cols, int dtype,
                   int mode, int64_t rows_pad, uint8_t* codes_t, uint8_t* scales_t,
                   void* stream) {
  if (batch < 0 || rows < 0 || cols < 0) return MX_ERR_ARG;
  if (dtype != MX_F32 && dtype != MX_BF16) return MX_ERR_ARG;
  if (mode != MXQ_OCP && mode != MXQ_UOS) return MX_ERR_ARG;
  const int64_t min_pad = (rows + mxk::kBlock - 1) / mxk::kBlock * mxk::kBlock;
  if (rows_pad == 0) rows_pad = min_pad;
  if (rows_pad < min_pad || rows_pad % mxk::kBlock != 0) return MX_ERR_ARG;
  if (batch == 0 || cols == 0 || rows_pad == 0) return MX_OK;
  if (batch > 65535 || rows_pad / 64 + 1 > 65535) return MX_ERR_UNSUPPORTED;
  if ((cols + 127) / 128 * 256 > kMaxItems) return MX_ERR_UNSUPPORTED;  // 128-column tiles
  if (!x || !codes_t || !scales_t) return MX_ERR_ARG;
  if (!aligned(codes_t, 16)) return MX_ERR_ALIGN;
  if (!aligned(x, dtype == MX_F32 ? 4 : 2)) return MX_ERR_ALIGN;
  const mxk::Dtype dt = dtype == MX_BF16 ? mxk::Dtype::BF16 : mxk::Dtype::F32;
  return to_status(mxk::launch_quant_cols(x, batch, rows, cols, rows_pad, dt, mode == MXQ_UOS,
                                          codes_t, scales_t, as_stream(stream)));
}

int mxq_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, int out_dtype,
                   void* y, void* stream) {
  if (n < 0 || n % mxk::kBlock != 0) return MX_ERR_ARG;
  if (out_dtype != MX_F32 && out_dtype != MX_BF16) return MX_ERR_ARG;
  if (n == 0) return MX_OK;
  // at most one work item per 8 elements (the kernel takes 32 per thread)
  if (n / 8 + 256 > kMaxItems) return MX_ERR_UNSUPPORTED;
  if (!codes || !scales || !y) return MX_ERR_ARG;
  if (!aligned(codes, 16) || !aligned(y, 16)) return MX_ERR_ALIGN;
  return to_status(mxk::launch_dequant(codes, scales, n, out_dtype == MX_BF16, y,
                                       as_stream(stream)));
}

size_t mxattn_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype,
                              int mode) {
  if (check_attn_shape(dtype, B, Hq, Hkv, Sq, Skv, D, 0, mode) != MX_OK) return 0;
  return make_layout(B, Hq, Hkv, Sq, Skv, D, dtype, mode).total;
}

size_t mxattn_dump_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype,
                                   int mode) {
  if (mode == MXATTN_FP16) return 0;
  if (check_attn_shape(dtype, B, Hq, Hkv, Sq, Skv, D, 0, mode) != MX_OK) return 0;
  return make_layout(B, Hq, Hkv, Sq, Skv, D, dtype, mode).total_dump;
}

int mxattn_workspace_layout(int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype,
                            int mode, size_t* off, int64_t* skv_ld) {
  int st = check_attn_shape(dtype, B, Hq, Hkv, Sq, Skv, D, 0, mode);
  if (st != MX_OK) return st;
  if (mode == MXATTN_FP16 || !off || !skv_ld) return MX_ERR_ARG;
  const Layout L = make_layout(B, Hq, Hkv, Sq, Skv, D, dtype, mode);
  for (int i = 0; i < 6; ++i) off[i] = L.off[i];
  *skv_ld = L.skv_ld;
  return MX_OK;
}

int mxattn_kv_tile(int D, int mode) {
  if (mode < MXATTN_FP16 || mode > MXATTN_UOS_EFQ) return MX_ERR_ARG;
  if (D != 64 && D != 128) return MX_ERR_UNSUPPORTED;
  return mode == MXATTN_FP16 ? mxk::kF16KvTile : mxk::kKvTile;
}

int mxattn_fwd(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
               int Hkv, int Sq, int Skv, int D, int causal, int mode, float* o,
               void* workspace, size_t ws_bytes, void* stream) {
  return attn_common(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, o, workspace,
                     ws_bytes, nullptr, nullptr, nullptr, false, stream);
}

int mxattn_prepare(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                   int Hkv, int Sq, int Skv, int D, int mode, void* workspace,
                   size_t ws_bytes, void* stream) {
  Layout L;
  int st = check_attn_call(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, 0, mode, workspace,
                           ws_bytes, true, true, &L);
  if (st != MX_OK) return st;
  return run_prepare(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, mode, L, workspace,
                     as_stream(stream));
}

int mxattn_fwd_prepared(const void* q, const void* k, int dtype, int B, int Hq, int Hkv,
                        int Sq, int Skv, int D, int causal, int mode, float* o,
                        void* workspace, size_t ws_bytes, void* stream) {
  Layout L;
  int st = check_attn_call(q, k, nullptr, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode,
                           workspace, ws_bytes, false, false, &L);
  if (st != MX_OK) return st;
  // q is read directly (FP16 mode with bf16 input) or quantized in the kernel (MX modes)
  if (!q && (mode != MXATTN_FP16 || dtype == MX_BF16)) return MX_ERR_ARG;
  if (!o) return MX_ERR_ARG;
  if (!aligned(o, 16)) return MX_ERR_ALIGN;
  return run_attention(q, k, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, o, L, workspace,
                       nullptr, nullptr, nullptr, as_stream(stream));
}

int mxattn_fwd_dump(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                    int Hkv, int Sq, int Skv, int D, int causal, int mode, float* o,
                    void* workspace, size_t ws_bytes, const int32_t* row_slot,
                    uint8_t* p_codes, uint8_t* p_scales, void* stream) {
  return attn_common(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, o, workspace,
                     ws_bytes, row_slot, p_codes, p_scales, true, stream);
}

}  // extern "C"

namespace {
int check_gemm_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return MX_ERR_ARG;
  if (K % 128 != 0) return MX_ERR_UNSUPPORTED;
  if (M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31)) return MX_ERR_UNSUPPORTED;
  // the kernel's per-lane load offsets are 32-bit: a row within a 256-row
  // tile times the row pitch K/2, plus a 16-byte chunk of a 128-byte line
  if (255 * (K / 2) + 128 >= (int64_t(1) << 32)) return MX_ERR_UNSUPPORTED;
  // workgroup count (256 x 256 output tiles) must fit a 1-D grid
  if (((M + 255) / 256) * ((N + 255) / 256) >= (int64_t(1) << 31)) return MX_ERR_UNSUPPORTED;
  return MX_OK;
}
}  // namespace

size_t mxgemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_gemm_shape(M, N, K) != MX_OK) return 0;
  return mxk::gemm_workspace_bytes(M, N, K);
}

int mxgemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
           const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, int out_dtype, void* y,
           void* workspace, size_t ws_bytes, void* stream) {
  if (out_dtype != MX_F32 && out_dtype != MX_BF16) return MX_ERR_ARG;
  const int st = check_gemm_shape(M, N, K);
  if (st != MX_OK) return st;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !y) return MX_ERR_ARG;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(y, 16)) return MX_ERR_ALIGN;
  if (!workspace || ws_bytes < mxk::gemm_workspace_bytes(M, N, K)) return MX_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MX_ERR_ALIGN;
  return to_status(mxk::launch_gemm_mx(a_codes, a_scales, b_codes, b_scales, M, N, K,
                                       out_dtype == MX_BF16, y, static_cast<uint8_t*>(workspace),
                                       as_stream(stream)));
}

int mxgemm_noalloc(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                   const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, int out_dtype,
                   void* y, void* stream) {
  if (out_dtype != MX_F32 && out_dtype != MX_BF16) return MX_ERR_ARG;
  const int st = check_gemm_shape(M, N, K);
  if (st != MX_OK) return st;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !y) return MX_ERR_ARG;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(y, 16)) return MX_ERR_ALIGN;
  // the scale images must fit the library's scratch array
  if (mxk::gemm_workspace_bytes(M, N, K) > mxk::kGemmScratchBytes) return MX_ERR_UNSUPPORTED;
  uint8_t* ws = nullptr;
  if (mxk::gemm_scratch(&ws) != hipSuccess) return MX_ERR_HIP;
  return to_status(mxk::launch_gemm_mx(a_codes, a_scales, b_codes, b_scales, M, N, K,
                                       out_dtype == MX_BF16, y, ws, as_stream(stream)));
}

int mxattn_decode_split(int B, int Hkv, int Skv) {
  if (B < 1 || Hkv < 1 || Skv < 1) return MX_ERR_ARG;
  return decode_split_tiles(B, Hkv, Skv) * mxk::kKvTile;
}

size_t mxattn_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype,
                                     int mode) {
  if (check_decode_shape(dtype, B, Hq, Hkv, Sq, Skv, D, 0, mode) != MX_OK) return 0;
  return make_decode_layout(B, Hq, Hkv, Sq, Skv, D, dtype, mode).total;
}

int mxattn_decode(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv,
                  int Sq, int Skv, int D, int causal, int mode, float* o, void* workspace,
                  size_t ws_bytes, void* stream) {
  return decode_common(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, o, workspace,
                       ws_bytes, nullptr, nullptr, nullptr, true, false, stream);
}

int mxattn_decode_prepared(const void* q, int dtype, int B, int Hq, int Hkv, int Sq, int Skv,
                           int D, int causal, int mode, float* o, void* workspace,
                           size_t ws_bytes, void* stream) {
  return decode_common(q, nullptr, nullptr, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, o,
                       workspace, ws_bytes, nullptr, nullptr, nullptr, false, false, stream);
}

int mxattn_decode_dump(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                       int Hkv, int Sq, int Skv, int D, int causal, int mode, float* o,
                       void* workspace, size_t ws_bytes, const int32_t* row_slot,
                       uint8_t* p_codes, uint8_t* p_scales, void* stream) {
  return decode_common(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, o, workspace,
                       ws_bytes, row_slot, p_codes, p_scales, true, true, stream);
}

// ---- per-sequence lengths ----

namespace {
// Dump pointers of the varlen entry points: all null (no dump) or all set.
int check_optional_dump(const int32_t* row_slot, const uint8_t* p_codes, const uint8_t* p_scales,
                        bool* dump) {
  const int n = (row_slot != nullptr) + (p_codes != nullptr) + (p_scales != nullptr);
  if (n != 0 && n != 3) return MX_ERR_ARG;
  *dump = n == 3;
  return MX_OK;
}
}  // namespace

int mxattn_fwd_varlen(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                      int Hkv, int Sq, int Skv, int D, const int32_t* seqlens_q,
                      const int32_t* seqlens_k, int causal, int mode, float* o,
                      void* workspace, size_t ws_bytes, const int32_t* row_slot,
                      uint8_t* p_codes, uint8_t* p_scales, void* stream) {
  bool dump = false;
  int st = check_optional_dump(row_slot, p_codes, p_scales, &dump);
  if (st != MX_OK) return st;
  if (causal != 0 && causal != 1) return MX_ERR_ARG;
  Layout L;
  // shape checks as for mxattn_fwd, except that causal queries are aligned
  // to the end of each sequence's keys, so Sq and Skv may differ
  st = check_attn_call(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, 0, mode, workspace, ws_bytes,
                       true, true, &L, dump && mode != MXATTN_FP16);
  if (st != MX_OK) return st;
  if (mode == MXATTN_FP16) return MX_ERR_UNSUPPORTED;
  if (!o || !seqlens_q || !seqlens_k) return MX_ERR_ARG;
  if (!aligned(o, 16) || !aligned(seqlens_q, 4) || !aligned(seqlens_k, 4)) return MX_ERR_ALIGN;
  if (dump && (!aligned(p_codes, 16) || !aligned(row_slot, 4))) return MX_ERR_ALIGN;
  hipStream_t s = as_stream(stream);
  st = run_prepare(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, mode, L, workspace, s, seqlens_k);
  if (st != MX_OK) return st;
  return run_attention(q, k, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, o, L, workspace,
                       dump ? row_slot : nullptr, dump ? p_codes : nullptr,
                       dump ? p_scales : nullptr, s, seqlens_q, seqlens_k);
}

int mxattn_prepare_varlen(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                          int Hkv, int Sq, int Skv, int D, const int32_t* seqlens_k, int mode,
                          void* workspace, size_t ws_bytes, void* stream) {
  Layout L;
  int st = check_attn_call(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, 0, mode, workspace, ws_bytes,
                           true, true, &L);
  if (st != MX_OK) return st;
  if (mode == MXATTN_FP16) return MX_ERR_UNSUPPORTED;
  if (!seqlens_k) return MX_ERR_ARG;
  if (!aligned(seqlens_k, 4)) return MX_ERR_ALIGN;
  return run_prepare(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, mode, L, workspace,
                     as_stream(stream), seqlens_k);
}

int mxattn_decode_varlen_prepared(const void* q, int dtype, int B, int Hq, int Hkv, int Sq,
                                  int Skv, int D, const int32_t* seqlens_k, int causal, int mode,
                                  float* o, void* workspace, size_t ws_bytes, void* stream) {
  if (!seqlens_k) return MX_ERR_ARG;
  if (!aligned(seqlens_k, 4)) return MX_ERR_ALIGN;
  return decode_common(q, nullptr, nullptr, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, o,
                       workspace, ws_bytes, nullptr, nullptr, nullptr, false, false, stream,
                       seqlens_k);
}

int mxattn_decode_varlen(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                         int Hkv, int Sq, int Skv, int D, const int32_t* seqlens_k, int causal,
                         int mode, float* o, void* workspace, size_t ws_bytes,
                         const int32_t* row_slot, uint8_t* p_codes, uint8_t* p_scales,
                         void* stream) {
  bool dump = false;
  int st = check_optional_dump(row_slot, p_codes, p_scales, &dump);
  if (st != MX_OK) return st;
  if (!seqlens_k) return MX_ERR_ARG;
  if (!aligned(seqlens_k, 4)) return MX_ERR_ALIGN;
  return decode_common(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, o, workspace,
                       ws_bytes, row_slot, p_codes, p_scales, true, dump, stream, seqlens_k);
}
