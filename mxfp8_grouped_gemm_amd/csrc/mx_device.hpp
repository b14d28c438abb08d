// mx_device.hpp -- device helpers for the gfx950 MXFP8 kernels: bf16 <-> fp32,
// the E8M0 scale rule and the OCP E4M3 / E5M2 encoders.
//
// MX groups (P1, "Blockwise MM Backward MXFP8 Kernel API Reference": MXFP8 with
// 32-element quantization groups): one E8M0 byte X+127 per group with
// X = floor(log2 amax) - emax (emax 8 for E4M3, 15 for E5M2), clamped to
// [-127,127]; element codes round v * 2^-X to nearest-even and saturate at the
// format's largest finite value.  The encoder below works on the fp32 bit
// pattern with integer arithmetic only, so it is exact for every input and
// independent of the FP environment (denormal flushing, rounding mode).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;

// The stage-major code layout of an operand with R rows contracted over K
// elements (K % 64 == 0), what the four-slot GEMM ring reads in whole cache
// lines: the rows in panels of kPanelRows (the last one may hold fewer), each
// panel [K/64][panel rows][64], so that the 64 elements of one ring stage of
// all the panel's rows form one contiguous run.  Byte (r, k):
constexpr int kPanelRows = 256;
__host__ __device__ __forceinline__ int64_t stage_major_off(int64_t r, int64_t k, int64_t R, int64_t K) {
  const int64_t p0 = r & ~int64_t(kPanelRows - 1);              // the panel's first row
  const int64_t rp = R - p0 < kPanelRows ? R - p0 : kPanelRows;  // its rows
  return p0 * K + ((k >> 6) * rp + (r - p0)) * 64 + (k & 63);
}

// Stores with the nontemporal hint (streaming: written lines are not kept in
// the caches as if they would be read again soon), for results written once
// and read, if at all, only after far more data than L2 and the infinity cache
// hold has passed through them.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, static_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_nt(void* p, uint2 v) {
  __builtin_nontemporal_store(u32x2_t{v.x, v.y}, static_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void store_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// |x| as the integer bit pattern (for max-reductions on non-negative floats:
// ordering of non-negative IEEE patterns is the ordering of their values).
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7fffffffu; }
__device__ __forceinline__ uint32_t abs_bits_bf16(uint16_t b) { return (uint32_t(b) & 0x7fffu) << 16; }

// E8M0 scale exponent X for a group whose largest magnitude has fp32 bits
// `amax_bits`: floor(log2 amax) is the biased exponent field minus 127 for
// normal numbers; zeros and subnormals (field 0) fall below -127 - emax and
// clamp to -127, which is the all-zero rule as well.
template <int FMT>
__device__ __forceinline__ int scale_exp(uint32_t amax_bits) {
  constexpr int emax = FMT == kE4M3 ? 8 : 15;
  int X = int(amax_bits >> 23) - 127 - emax;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// Round-to-nearest-even right shift of a positive significand.
__device__ __forceinline__ uint32_t rne_shr(uint32_t x, int s) {
  if (s <= 0) return x;
  if (s >= 32) return 0;
  const uint32_t r = x >> s;
  const uint32_t rem = x & ((1u << s) - 1u);
  const uint32_t half = 1u << (s - 1);
  return r + ((rem > half) || (rem == half && (r & 1u)) ? 1u : 0u);
}

// Code of v * 2^-X in format FMT (v given as fp32 bits; finite).
template <int FMT>
__device__ __forceinline__ uint32_t encode(uint32_t vbits, int X) {
  constexpr int mbits = FMT == kE4M3 ? 3 : 2;
  constexpr int bias = FMT == kE4M3 ? 7 : 15;
  constexpr int emin = 1 - bias;                       // exponent of the smallest normal
  constexpr int emax = FMT == kE4M3 ? 8 : 15;          // exponent of the largest binade
  constexpr uint32_t qmax = FMT == kE4M3 ? 14u : 7u;   // largest significand in that binade
  constexpr uint32_t maxcode = FMT == kE4M3 ? 0x7Eu : 0x7Bu;
  const uint32_t sign = (vbits >> 24) & 0x80u;
  const uint32_t ef = (vbits >> 23) & 0xffu;
  uint32_t sig = vbits & 0x7fffffu;
  int e;                                               // v = sig * 2^(e-23), sig in [2^23, 2^24)
  if (ef == 0) {
    if (sig == 0) return sign;
    const int lz = __clz(sig) - 8;                     // normalise an fp32 subnormal
    sig <<= lz;
    e = -126 - lz;
  } else {
    sig |= 0x800000u;
    e = int(ef) - 127;
  }
  int ey = e - X;                                      // exponent of y = v * 2^-X
  if (ey > emax) return sign | maxcode;
  if (ey >= emin) {
    uint32_t q = rne_shr(sig, 23 - mbits);             // in [2^mbits, 2^(mbits+1)]
    if (q == (2u << mbits)) { q = 1u << mbits; ++ey; }
    if (ey > emax || (ey == emax && q > qmax)) return sign | maxcode;
    return sign | (uint32_t(ey + bias) << mbits) | (q - (1u << mbits));
  }
  // subnormal target: multiples of 2^(emin - mbits)
  const int s = 23 - mbits + emin - ey;                // > 23 - mbits
  return sign | rne_shr(sig, s);
}

// 2^-X in fp32 for a scale exponent that scale_exp can return (X <= 127 - emax,
// so the result is a normal number).
__device__ __forceinline__ float inv_scale(int X) { return __uint_as_float(uint32_t(127 - X) << 23); }

// Four codes packed little-endian into a word, through the hardware converter:
// y = v * 2^-X is exact (a power-of-two scale of a value inside its group
// stays normal or underflows far below the format's smallest subnormal), the
// clamp to +-max finite is the encoder's saturation, and v_cvt_pk_fp8_f32 /
// v_cvt_pk_bf8_f32 round to nearest-even into the OCP formats.  Equal to
// encode<FMT> for every finite fp32 input and every scale the group rule can
// produce (checked exhaustively over all bf16 patterns and all such scales).
// encode4s: the same with a scale per value (four groups, e.g. four columns).
template <int FMT>
__device__ __forceinline__ uint32_t encode4s(float v0, float v1, float v2, float v3, float i0, float i1, float i2,
                                             float i3) {
  constexpr float M = FMT == kE4M3 ? 448.f : 57344.f;
  const float y0 = fminf(fmaxf(v0 * i0, -M), M), y1 = fminf(fmaxf(v1 * i1, -M), M);
  const float y2 = fminf(fmaxf(v2 * i2, -M), M), y3 = fminf(fmaxf(v3 * i3, -M), M);
  int w;
  if (FMT == kE4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(y2, y3, w, true);
  }
  return uint32_t(w);
}
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float v0, float v1, float v2, float v3, float inv) {
  return encode4s<FMT>(v0, v1, v2, v3, inv, inv, inv, inv);
}

// Codes of bf16 values, two packed per word (value 2k in the low half), with
// scale 2^X: v_cvt_scalef32_pk_fp8_bf16 / _bf8_bf16 divide by the E8M0 scale
// whose byte is the exponent field of their fp32 scale operand (byte 0
// included: the float 0.0 stands for 2^-127) and round to nearest-even, but
// return NaN / Inf past the format's largest finite value instead of
// saturating.  So the magnitudes are clamped first to max * 2^X, in the bf16
// domain: |bf16| orders like its 15-bit pattern, so one packed 16-bit minimum
// clamps both halves.  Checked exhaustively on the GPU: every bf16 pair
// pattern x every scale the group rule can produce gives the codes of
// encode4 (clamp-and-convert in fp32).
// bf16 bits of max * 2^X (max = 1.75 * 2^emax in both formats)
template <int FMT>
__device__ __forceinline__ uint32_t bf16_limit(int X) {
  return (uint32_t(X + 127 + (FMT == kE4M3 ? 8 : 15)) << 7) | 0x60u;
}
// |w| clamped halfwise to the limits in lim2 (low and high half)
__device__ __forceinline__ uint32_t clamp_bf16x2(uint32_t w, uint32_t lim2) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 m = __builtin_elementwise_min(__builtin_bit_cast(u16x2, w & 0x7fff7fffu), __builtin_bit_cast(u16x2, lim2));
  return (w & 0x80008000u) | __builtin_bit_cast(uint32_t, m);
}
// halfwise max of |w| and m (packed 16-bit magnitudes)
__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t m, uint32_t w) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, m),
                                                                __builtin_bit_cast(u16x2, w & 0x7fff7fffu)));
}
// the scale operand of the converters for 2^X
__device__ __forceinline__ float cvt_scale(int X) { return __uint_as_float(uint32_t(X + 127) << 23); }
// four codes from two clamped pairs (values 0, 1 in p01; 2, 3 in p23)
template <int FMT>
__device__ __forceinline__ uint32_t encode_bf16x4(uint32_t p01, uint32_t p23, float s) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
  s16x2 r = {0, 0};
  if (FMT == kE4M3) {
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(b16x2, p01), s, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(b16x2, p23), s, true);
  } else {
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(b16x2, p01), s, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(b16x2, p23), s, true);
  }
  return __builtin_bit_cast(uint32_t, r);
}
// low / high halves of two words, packed (a's in the low half)
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// bf16 round-to-nearest-even through the hardware converter (finite inputs;
// equal to f32_to_bf16 there).
__device__ __forceinline__ uint16_t bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float bf16_round(float f) { return bf16_to_f32(bf16_rne(f)); }

// Two fp32 values rounded to bf16 (nearest even) and packed, a in the low half:
// one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_pack(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Runtime-format dispatch.
__device__ __forceinline__ int scale_exp_rt(int fmt, uint32_t amax_bits) {
  return fmt == kE4M3 ? scale_exp<kE4M3>(amax_bits) : scale_exp<kE5M2>(amax_bits);
}
__device__ __forceinline__ uint32_t encode_rt(int fmt, uint32_t vbits, int X) {
  return fmt == kE4M3 ? encode<kE4M3>(vbits, X) : encode<kE5M2>(vbits, X);
}

// ---- wavefront (64-lane) reductions ------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_xor(uint32_t v, int width) {
  for (int o = 1; o < width; o <<= 1) v = max(v, uint32_t(__shfl_xor(int(v), o, 64)));
  return v;
}
__device__ __forceinline__ float wave_sum_xor(float v, int width) {
  for (int o = 1; o < width; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace mx
