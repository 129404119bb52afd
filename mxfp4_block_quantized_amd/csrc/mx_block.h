// MXFP4 block quantization helpers shared by the standalone quantizer and
// the attention kernels (which quantize Q in their prologue).
//
// Format ("Quantization Error", section "Where the error comes from"; OCP
// Microscaling Formats v1.0): 32 elements share an E8M0 scale 2^(X-127);
// elements are E2M1 codes, rounded to nearest with ties to the even code and
// saturating at 6.  Scale rules ("MXAttention ...", abstract): OCP puts the
// block maximum into [4, 8) of the scaled domain, UOS into (3.625, 7.25]
// (boundary Qmax = 7.25, inclusive).
//
// Both rules reduce to the exponent field Ef and mantissa field of the
// block maximum |x|max:  X = max(0, Ef - 2 + up), with up = 1 only for UOS
// and a mantissa above 1.8125 (fp32 field > 0x680000), i.e. exactly when
// amax / 2^(Ef-129) > 7.25.  Zero and subnormal maxima give X = 0.
//
// Element rounding uses v_cvt_scalef32_pk_fp4_f32 (round to nearest even,
// saturating, sign kept) on v = x * 2^-e, which is exact in fp32 for every
// value that can round away from zero (fp32 denormals are kept).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mxk {

// Largest |x| of a block, as the fp32 bit pattern, to the E8M0 byte.
template <int UOS>
__device__ __forceinline__ uint32_t e8m0_of_amax(uint32_t abits) {
  int ef = static_cast<int>(abits >> 23);
  int up = UOS ? ((abits & 0x7FFFFFu) > 0x680000u ? 1 : 0) : 0;
  int x = ef - 2 + up;
  return x < 0 ? 0u : static_cast<uint32_t>(x);
}

// 2^-e for the E8M0 byte X (e = X - 127): always a normal fp32.
__device__ __forceinline__ float inv_scale_of(uint32_t X) {
  return __uint_as_float((254u - X) << 23);
}

// Pack 8 fp32 elements (bit patterns) under inverse scale `inv` into one
// dword of codes: element 2j -> low nibble of byte j.
__device__ __forceinline__ uint32_t pack8(const uint32_t f[8], float inv) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(f[0]) * inv,
                                               __uint_as_float(f[1]) * inv, 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(f[2]) * inv,
                                               __uint_as_float(f[3]) * inv, 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(f[4]) * inv,
                                               __uint_as_float(f[5]) * inv, 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(f[6]) * inv,
                                               __uint_as_float(f[7]) * inv, 1.0f, 3);
  return r;
}

// The raw bits of one 32-element block of a row: 4 (bf16) or 8 (fp32)
// 16-byte loads.  Split from the conversion so that a kernel can issue the
// loads early and convert later.
struct RawBlock32 {
  uint4 v[8];
};
__device__ __forceinline__ RawBlock32 load_block32(const void* src, bool in_bf16) {
  RawBlock32 r;
  const uint4* p = static_cast<const uint4*>(src);
  if (in_bf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = p[i];
#pragma unroll
    for (int i = 4; i < 8; ++i) r.v[i] = make_uint4(0, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = p[i];
  }
  return r;
}

// A loaded block to 16 bytes of codes (returned) and its E8M0 byte.
template <int UOS>
__device__ __forceinline__ uint4 quant_raw32(const RawBlock32& r, bool in_bf16, uint32_t& X) {
  uint32_t f[32];
  if (in_bf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = r.v[i];
      f[8 * i + 0] = v.x << 16; f[8 * i + 1] = v.x & 0xFFFF0000u;
      f[8 * i + 2] = v.y << 16; f[8 * i + 3] = v.y & 0xFFFF0000u;
      f[8 * i + 4] = v.z << 16; f[8 * i + 5] = v.z & 0xFFFF0000u;
      f[8 * i + 6] = v.w << 16; f[8 * i + 7] = v.w & 0xFFFF0000u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = r.v[i];
      f[4 * i + 0] = v.x; f[4 * i + 1] = v.y; f[4 * i + 2] = v.z; f[4 * i + 3] = v.w;
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, f[i] & 0x7FFFFFFFu);
  X = e8m0_of_amax<UOS>(m);
  const float inv = inv_scale_of(X);
  return make_uint4(pack8(f, inv), pack8(f + 8, inv), pack8(f + 16, inv), pack8(f + 24, inv));
}

// One 32-element block of a row (bf16 when in_bf16, else fp32) to 16 bytes
// of codes (returned) and its E8M0 byte.
template <int UOS>
__device__ __forceinline__ uint4 quant_block32(const void* src, bool in_bf16, uint32_t& X) {
  return quant_raw32<UOS>(load_block32(src, in_bf16), in_bf16, X);
}

}  // namespace mxk
