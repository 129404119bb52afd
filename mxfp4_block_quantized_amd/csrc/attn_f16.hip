// 16-bit attention forward for gfx950: the unquantized ("FP16") mode that
// the MXFP4 modes are compared against.  Same FlashAttention loop as the FP4
// kernel (running max per KV tile, fp32 accumulation, O / l at the end,
// "EFQ-Softmax" abstract), with S^T = K Q^T on bf16 (or fp16) matrix cores
// and O^T = V^T P^T on fp16 matrix cores: P = exp(s - m) is rounded to fp16,
// and the denominator sums that same fp16 P on the matrix core, so numerator
// and denominator carry the same rounding.  Without a P~ quantization the
// tile size only changes rounding; this mode uses 64-key tiles
// (kF16KvTile).
//
// v_mfma_f32_32x32x16_{bf16,f16}: operand lane l holds row (l % 32) and
// K-elements 8 (l/32) .. +7; accumulator lane l, register r holds row
// 8 (r/4) + 4 (l/32) + r%4, column l % 32.  One wave owns 32 queries (the
// columns).  A-row R = 8 g + 4 h + k of key subtile t of S^T is the key
// 32 t + 16 (g/2) + 8 h + 4 (g%2) + k (the image stores K in that order), so
// accumulator registers 8u .. 8u+7 of lane l hold the keys 32 t + 16 u +
// 8 (l/32) + 0..7 of query l % 32: exactly the lane's slice of the P^T
// operand of the 16-key step 2t + u of O^T = V^T P^T.  The denominator is one
// v_mfma_f32_16x16x32_f16 per 16-key step with the same P register as B and
// a constant A that is 1.0 where (A-row / 4) and the K-group have the same
// parity: output lane l then receives its query's sum over those 16 keys.
// The prepare kernel writes K and V^T as 16-bit tile images already in
// these operand orders, so a tile moves to LDS with contiguous
// 16-byte-per-lane direct loads.
#include "internal.h"

namespace mxk {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 32;         // query rows per wave (one 32-column tile)
constexpr int kT = kF16KvTile;  // keys per tile (64)
constexpr int kSub = kT / 32;   // 32-key subtiles of S^T (2)
constexpr int kStep = kT / 16;  // 16-key contraction steps of O^T (4)
static_assert(kQTile == kWaves * kQW, "query tile = waves x 32");
static_assert(kQTile % kT == 0, "query tiles start on KV tile boundaries");

template <int QK_F16>
__device__ __forceinline__ v16f mfma_qk(const uint4& a, const uint4& b, const v16f& c) {
  if (QK_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c,
                                                  0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c,
                                                   0, 0, 0);
  }
}
__device__ __forceinline__ v16f mfma_pv(const uint4& a, const uint4& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0,
                                                0);
}
// Denominator: 16x16x32 product of the lane-parity ones operand with a P
// register (see the file comment).
__device__ __forceinline__ v4f mfma_rowsum(uint32_t ones, const uint4& b, const v4f& c) {
  const uint4 a = make_uint4(ones, ones, ones, ones);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0,
                                                0);
}
__device__ __forceinline__ uint32_t rowsum_ones(int lane) {
  return (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 0x3C003C00u : 0u;  // fp16 1.0 pairs
}

// max over the lanes l and l ^ 32 (same query)
__device__ __forceinline__ float xhalf_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
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

// s_waitcnt lgkmcnt(0) only (LDS reads).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Direct loads of NR 1 KiB rows starting at src into an LDS area: wave w
// moves rows w, w + kWaves, ..., lane l bytes [16 l, 16 l + 16) of each.
// Buffer loads (raw resource, no range check), not the global form: with a
// global load-to-LDS in flight the compiler makes every LDS wait a full
// lgkmcnt(0).
template <int NR>
__device__ __forceinline__ void issue_rows(uint8_t* dst, const uint8_t* src, int wave, int lane) {
  static_assert(NR % kWaves == 0, "whole rows per wave");
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(uniform_ptr(src)), 0, 0xFFFFFFFFu, 0x00020000);
  const uint32_t lo = static_cast<uint32_t>(lane) * 16u;
#pragma unroll
  for (int i = 0; i < NR / kWaves; ++i) {
    const int row = wave + i * kWaves;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + row * 1024, 16, lo, row * 1024, 0, 0);
  }
}

template <int D>
struct F16State {
  v16f oacc[D / 32];
  v4f lacc;  // denominator (the four elements hold the same sum; element 0 is kept rescaled)
  float m;   // running row max (raw score units), -inf before the first tile
};

// Keys past `lim` (relative to the first key of this lane's half, 8 (l/32)
// into the tile) are excluded: register r of subtile t is key
// 32 t + 16 (r/8) + (r%8) past that.
__device__ __forceinline__ void mask_tile(v16f (&s)[kSub], int lim) {
  asm volatile("" : "+v"(lim));  // keeps the compares inside the caller's branch
#pragma unroll
  for (int t = 0; t < kSub; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[t][r] = (32 * t + 16 * (r >> 3) + (r & 7) > lim) ? -INFINITY : s[t][r];
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }
__device__ __forceinline__ void pin_out(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin_out(uint32_t& v) { asm volatile("" : "+v"(v)); }

// Placement of the vector work of one KV tile among its NR fenced regions
// (one S^T matrix instruction each).  Regions 0..3 take the row maxima; the
// 16 fp16 pairs of P (pair p: step p/4, dword p%4) are spread over regions
// 4..NR-1; O^T instruction k (step k / NC, channel tile k % NC) goes to the
// first free region after its P step is complete, one per region, and what
// does not fit runs after the last region.
constexpr int kOPerRegion = 1;  // O^T instructions per region
__host__ __device__ constexpr int pair_region(int nr, int p) { return 4 + (p * (nr - 4)) / 16; }
__host__ __device__ constexpr int o_region(int nr, int nc, int k) {
  int r = -1;  // slot: kOPerRegion per region
  for (int i = 0; i <= k; ++i) {
    const int lo = kOPerRegion * (pair_region(nr, 4 * (i / nc) + 3) + 1);
    r = r + 1 > lo ? r + 1 : lo;
  }
  return r / kOPerRegion;
}

// One KV tile j as NR = 2 D/16 fenced regions, one S^T(j+1) matrix
// instruction each (subtile n / (D/16), d-step n % (D/16)); S^T of tile j (sc)
// was formed during tile j-1.  Regions 0..3 also take the row maxima of
// tile j, followed by a region of their own for the running max and the
// rescale (uniform branch); the later regions compute P of tile j and
// start O^T(j) as soon as a 16-key step of P is complete.  Each region
// issues the LDS reads of the next region's operands, so no matrix
// instruction waits for a read issued in its own region.
template <int D, int QK_F16>
__device__ __forceinline__ void f16_iter(F16State<D>& w, v16f (&sc)[kSub], v16f (&sn)[kSub], const uint8_t* kst,
                                         const uint8_t* vst, const uint4 (&qop)[D / 16], uint32_t ones, bool mask,
                                         int lim, int lane, float sl2) {
  constexpr int NS = D / 16;  // 16-wide contraction steps of S^T
  constexpr int NC = D / 32;  // output channel tiles
  constexpr int NR = 2 * NS;  // regions (S^T instructions)
  constexpr int NO = kStep * NC;  // O^T instructions
  auto kop = [&](int n) {
    return *reinterpret_cast<const uint4*>(kst + ((n / NS) * NS + n % NS) * 1024 + lane * 16);
  };
  auto vop = [&](int k) {
    return *reinterpret_cast<const uint4*>(vst + ((k % NC) * kStep + k / NC) * 1024 + lane * 16);
  };
  auto o_mfma = [&](int k, const uint4& v, const uint4 (&pop)[kStep]) {
    const int u = k / NC;
    w.oacc[k % NC] = mfma_pv(v, pop[u], w.oacc[k % NC]);
    if (k % NC == NC - 1) w.lacc = mfma_rowsum(ones, pop[u], w.lacc);
  };

  // (a uniform branch that rewrites sc in place: one body serves masked and
  // unmasked tiles, so the loop state needs no copies at a join)
  if (mask) mask_tile(sc, lim);
  const v16f zero = {};
  uint4 kb[2], vk[NO];
  uint32_t pw[16];
  uint4 pop[kStep];
  float bm[4];
  float ofs = 0.0f;
  kb[0] = kop(0);
  fence();
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    if (n + 1 < NR) kb[(n + 1) & 1] = kop(n + 1);
#pragma unroll
    for (int k = 0; k < NO; ++k)
      if (o_region(NR, NC, k) == n + 1) vk[k] = vop(k);
    sn[n / NS] = mfma_qk<QK_F16>(kb[n & 1], qop[n % NS], n % NS == 0 ? zero : sn[n / NS]);
    if (n < 4) {
      const v16f& sv = sc[n >> 1];
      const int r0 = 8 * (n & 1);
      bm[n] = fmaxf(fmaxf(fmaxf(sv[r0], sv[r0 + 1]), fmaxf(sv[r0 + 2], sv[r0 + 3])),
                    fmaxf(fmaxf(sv[r0 + 4], sv[r0 + 5]), fmaxf(sv[r0 + 6], sv[r0 + 7])));
      pin_out(bm[n]);
    }
    // The S^T subtiles this region reads are pinned here and the P words
    // after they are made, so the work can neither be hoisted into an
    // earlier region nor merged with another region's (pinning the whole
    // register tuple costs no copies, unlike pinning single elements).
#pragma unroll
    for (int t = 0; t < kSub; ++t) {
      bool used = false;
#pragma unroll
      for (int p = 0; p < 16; ++p) used = used || (pair_region(NR, p) == n && (p >> 3) == t);
      if (used) asm volatile("" : "+v"(sc[t]));
    }
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      if (pair_region(NR, p) == n) {
        const float x0 = sc[p >> 3][2 * (p & 7)];
        const float x1 = sc[p >> 3][2 * (p & 7) + 1];
        pw[p] = pack_f16x2(__builtin_amdgcn_exp2f(fmaf(x0, sl2, -ofs)), __builtin_amdgcn_exp2f(fmaf(x1, sl2, -ofs)));
        pin_out(pw[p]);
        if ((p & 3) == 3) pop[p >> 2] = make_uint4(pw[p - 3], pw[p - 2], pw[p - 1], pw[p]);
      }
    }
#pragma unroll
    for (int k = 0; k < NO; ++k)
      if (o_region(NR, NC, k) == n) o_mfma(k, vk[k], pop);
    fence();
    if (n == 3) {
      const float mnew = fmaxf(w.m, xhalf_max(fmaxf(fmaxf(bm[0], bm[1]), fmaxf(bm[2], bm[3]))));
      const float alpha = __builtin_amdgcn_exp2f((w.m - mnew) * sl2);  // 0 at the first tile
      w.m = mnew;
      ofs = mnew * sl2;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) w.oacc[c] *= alpha;
        w.lacc[0] *= alpha;
      }
      fence();
    }
  }
  // O^T instructions that found no region
#pragma unroll
  for (int k = 0; k < NO; ++k)
    if (o_region(NR, NC, k) >= NR) o_mfma(k, vop(k), pop);
  fence();
}

template <int D, int QK_F16, int CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_f16_kernel(F16AttnArgs a, float sl2) {
  constexpr int NS = D / 16;
  constexpr int NC = D / 32;
  constexpr int IMG = f16_img_bytes(D);
  constexpr int HALF = f16_img_vc(D);  // bytes of the K part (and of the V part)
  constexpr int NR = HALF / 1024;      // 1 KiB rows per part
  // Two K stages and two V stages, one LDS object each (the compiler then
  // waits only for the loads of the stage a read touches).  During tile j
  // the K stage of tile j+1 and the V stage of tile j are read; the loads of
  // K(j+2) and V(j+1) go to the other two.
  __shared__ __attribute__((aligned(1024))) uint8_t kst0[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t kst1[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t vst0[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t vst1[HALF];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nqb = (a.Sq + kQTile - 1) / kQTile;
  // workgroup -> (head, query tile): a contiguous run of heads per XCD
  // (workgroups are dispatched round-robin over the 8 XCDs), the last 1/8
  // of each run through its work-queue counter, which the other XCDs also
  // drain once their own runs are done (as in the MXFP4 kernel); causal:
  // the longest query tiles of a head first
  const int nitems = nqb * a.Hq * a.B;
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
  const int hb = gi / nqb;
  const int qb = CAUSAL ? nqb - 1 - gi % nqb : gi % nqb;
  const int h = hb % a.Hq;
  const int b = hb / a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int q0 = qb * kQTile;
  const int qw0 = q0 + wave * kQW;
  const int col = lane & 31;
  const int half = lane >> 5;
  const uint32_t ones = rowsum_ones(lane);
  const int64_t bh = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t bg = static_cast<int64_t>(b) * a.Hkv + g;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + bh * a.Sq * D;

  const int nt = (a.Skv + kT - 1) / kT;
  const int ntiles = CAUSAL ? min(nt, (q0 + kQTile - 1) / kT + 1) : nt;
  // tiles [0, nmain) need no masking for any row of this workgroup; a row's
  // first tile always holds an unmasked key (key 0)
  const int nmain = CAUSAL ? min(q0 / kT, nt) : (a.Skv % kT != 0 ? nt - 1 : nt);
  const uint8_t* img = uniform_ptr(a.img + bg * nt * static_cast<int64_t>(IMG));

  // K(0), V(0) and K(1) first; then the lane's Q operand: query `col`,
  // elements 16 s + 8 (l/32) .. +7 of d-step s
  issue_rows<NR>(kst0, img, wave, lane);
  issue_rows<NR>(vst0, img + HALF, wave, lane);
  if (ntiles > 1) issue_rows<NR>(kst1, img + IMG, wave, lane);
  const int qrow = qw0 + col;
  uint4 qop[NS];
  {
    const int64_t r = min(qrow, a.Sq - 1);
#pragma unroll
    for (int st = 0; st < NS; ++st)
      qop[st] = *reinterpret_cast<const uint4*>(qg + r * D + st * 16 + half * 8);
  }
  const int klim = CAUSAL ? min(a.Skv - 1, qrow) : a.Skv - 1;

  F16State<D> w;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) w.oacc[c][r] = 0.0f;
  w.lacc = v4f{0, 0, 0, 0};
  w.m = -INFINITY;

  wait_vmcnt<0>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // S^T of tile 0
  v16f sa[kSub], sb[kSub];
#pragma unroll
  for (int t = 0; t < kSub; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[t][r] = 0.0f;
#pragma unroll
    for (int st = 0; st < NS; ++st)
      sa[t] = mfma_qk<QK_F16>(*reinterpret_cast<const uint4*>(kst0 + (t * NS + st) * 1024 + lane * 16), qop[st],
                              sa[t]);
  }

  // Iteration jt: K(jt+1) and V(jt) were requested one iteration earlier (or
  // above); each wave waits for its loads, the barrier makes all of them
  // visible and tells that every wave is done with iteration jt-1, whose
  // stages K(jt) and V(jt-1) then receive K(jt+2) and V(jt+1).  The last
  // iteration's S^T of the tile past the end reads a stale stage and is
  // dropped.  The loop is
  // unrolled by two so that every stage index is a compile-time constant.
  for (int jb = 0; jb < ntiles; jb += 2) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int jt = jb + k;
      if (jt < ntiles) {
        // (jt == 0: the K(0) stage that S^T(0) was read from takes K(2);
        // each wave's reads of it must be complete before the barrier)
        if (jt > 0) wait_vmcnt<0>();
        else wait_lgkm0();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (jt + 2 < ntiles) issue_rows<NR>(k == 0 ? kst0 : kst1, img + static_cast<int64_t>(jt + 2) * IMG, wave, lane);
        if (jt + 1 < ntiles)
          issue_rows<NR>(k == 0 ? vst1 : vst0, img + static_cast<int64_t>(jt + 1) * IMG + HALF, wave, lane);
        const int lim = klim - (jt * kT + 8 * half);
        if (k == 0) f16_iter<D, QK_F16>(w, sa, sb, kst1, vst0, qop, ones, jt >= nmain, lim, lane, sl2);
        else f16_iter<D, QK_F16>(w, sb, sa, kst0, vst1, qop, ones, jt >= nmain, lim, lane, sl2);
      }
    }
  }

  // Pin the accumulators before the per-lane store condition so that no
  // matrix-core instruction is moved into that divergent region (an MFMA with
  // part of EXEC disabled drops operands other lanes' results depend on).
#pragma unroll
  for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(w.oacc[c]));
  asm volatile("" : "+v"(w.lacc));

  const float inv = 1.0f / w.lacc[0];
  if (qrow < a.Sq) {
    float* orow = a.o + (bh * a.Sq + qrow) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        *reinterpret_cast<float4*>(orow + 32 * c + 8 * gq + 4 * half) =
            make_float4(w.oacc[c][4 * gq] * inv, w.oacc[c][4 * gq + 1] * inv, w.oacc[c][4 * gq + 2] * inv,
                        w.oacc[c][4 * gq + 3] * inv);
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
  constexpr int NS = D / 16;
  constexpr int NC = D / 32;
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
  // K chunks (subtile t, d-step st, lane l): A-row R = l % 32 = 8 g + 4 h + k
  // of subtile t is the key 32 t + 16 (g/2) + 8 h + 4 (g%2) + k, elements
  // 16 st + 8 (l/32) .. +7
  for (int i = threadIdx.x; i < kSub * NS * 64; i += 256) {
    const int l = i & 63, ts = i >> 6, t = ts / NS, st = ts % NS;
    const int R = l & 31;
    const int key = 32 * t + 16 * (R >> 4) + 8 * ((R >> 2) & 1) + 4 * ((R >> 3) & 1) + (R & 3);
    uint4 chunk = make_uint4(0u, 0u, 0u, 0u);
    if (j0 + key < rows) {
      const In* src = kb + static_cast<int64_t>(j0 + key) * D + st * 16 + (l >> 5) * 8;
      if (sizeof(In) == 2) {
        chunk = *reinterpret_cast<const uint4*>(src);
      } else {
        uint16_t hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = to_f16(ld_in<In>(src + e));
        chunk = pack8_u16(hv);
      }
    }
    *reinterpret_cast<uint4*>(out + ts * 1024 + l * 16) = chunk;
  }
  __syncthreads();
  // V^T chunks (channel tile c, key step u, lane l): channel 32 c + l % 32,
  // keys 16 u + 8 (l/32) .. +7
  for (int i = threadIdx.x; i < NC * kStep * 64; i += 256) {
    const int l = i & 63, cu = i >> 6, c = cu / kStep, u = cu % kStep;
    const int d = 32 * c + (l & 31), key0 = 16 * u + 8 * (l >> 5);
    uint16_t hv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] = vt[(key0 + e) * LD + d];
    *reinterpret_cast<uint4*>(out + f16_img_vc(D) + cu * 1024 + l * 16) = pack8_u16(hv);
  }
}

__global__ __launch_bounds__(256) void f32_to_f16_kernel(const float* __restrict__ x, int64_t n,
                                                         int64_t n_write, uint16_t* __restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n_write) y[i] = to_f16(i < n ? x[i] : 0.0f);
}

// Clears the work-queue counters (a kernel, so that graphs replay it).
__global__ void clear_f16_queue_kernel(uint32_t* q) {
  if (threadIdx.x < kQueueWords) q[threadIdx.x] = 0u;
}

template <int D, int QK_F16>
hipError_t launch_c(const F16AttnArgs& a, hipStream_t s) {
  const int64_t nitems = static_cast<int64_t>((a.Sq + kQTile - 1) / kQTile) * a.Hq * a.B;
  dim3 grid(static_cast<unsigned>(prefill_grid(nitems)));
  hipLaunchKernelGGL(clear_f16_queue_kernel, dim3(1), dim3(64), 0, s, a.queue);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
