// Device-side helpers shared by the LatentMoE HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// SwiGLU: silu(g) * u = g / (1 + e^-g) * u, with the hardware exponential
// (__expf: v_exp_f32 on g * log2 e) and reciprocal (v_rcp_f32).  Their error,
// about 1e-6 relative at |g| <= 20, is far below the bf16 rounding that
// follows; e^-g overflowing to inf gives -0, as the exact form does.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// 16x16x32 bf16 MFMA: D(16x16 f32) = A(16x32) * B(32x16) + C.
// Operand layout (lane l): A row l%16, K elements 8*(l/16) .. +8; B column
// l%16, the same K elements.  Result: lane l holds column l%16 of rows
// 4*(l/16) .. +4.
__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// 16-byte global load (p 16-byte aligned).
__device__ __forceinline__ uint4 ldg16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// The same with the nontemporal hint, for data that one pass reads once
// (expert outputs in the combine, weights streamed at decode, logits): the
// lines are not kept in the caches for reuse.
__device__ __forceinline__ uint4 ldnt16(const void* p) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v r = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return uint4{r[0], r[1], r[2], r[3]};
}

// Workgroup id -> logical tile id such that consecutive logical ids share an
// XCD (the hardware deals workgroups to the 8 XCDs round robin), which keeps
// tiles that reuse the same operand rows in one L2.
__device__ __forceinline__ uint32_t xcd_swizzle(uint32_t b, uint32_t nb) {
  const uint32_t full = (nb / 8u) * 8u;
  if (b >= full) return b;
  return (b % 8u) * (nb / 8u) + b / 8u;
}

// Persistent grids over the same order: workgroup b (on XCD b mod 8, slot
// b/8 of the G = grid/8 there; grid a multiple of 8) walks its XCD's run of
// the order (the run xcd_swizzle gives that XCD, then its one remainder tile)
// in passes of G tiles, slot j taking tile j of even passes and G-1-j of odd
// ones, so a workgroup alternates between the ends of a pass.  (A fixed
// stride hands each slot tiles at one offset in every period of the order:
// with an expert's two row tiles adjacent in it, half the workgroups got
// only the larger ones.)  Returns false once the pass is past the run.
__device__ __forceinline__ bool mirrored_tile(uint32_t b, uint32_t grid, uint32_t nb, uint32_t pass, uint32_t& lt) {
  const uint32_t xcd = b % 8u, slot = b / 8u, G = grid / 8u, per = nb / 8u;
  const uint32_t mine = per + (xcd < nb % 8u ? 1u : 0u);
  const uint32_t pos = pass * G + ((pass & 1u) ? G - 1u - slot : slot);
  if (pos >= mine) return false;
  lt = pos < per ? xcd * per + pos : 8u * per + xcd;
  return true;
}

// e8m0 scale code -> the fp32 multiplier 2^(code-127) (code 0: 2^-127, a
// denormal; 255: NaN), the operand the scaled conversion takes.
__device__ __forceinline__ float e8m0_multiplier(uint32_t c) {
  return __uint_as_float(c == 0 ? 0x00400000u : (c == 255 ? 0x7fc00000u : c << 23));
}

// 8 e2m1 codes (one dword, K ascending from the low nibble) x scale -> bf16x8.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t codes, float scale) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  const bf16x4_t lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const bf16x4_t hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A tile's rows split between its two rows of waves in whole 32-row
// subtiles, the first row of waves taking the larger half (a 101-row tile:
// 64 + 37 rows, not 96 + 5), so that a partial tile's time follows its row
// count: wave row wm's first row (r0) and subtile count (fa, at most fm).
struct WaveRows {
  int r0, fa;
};
__device__ __forceinline__ WaveRows wave_rows(int wm, int nrows, int fm) {
  const int ns = (nrows + 31) / 32, s0 = (ns + 1) / 2;
  if (wm == 0) return WaveRows{0, min(fm, s0)};
  return WaveRows{32 * s0, max(0, min(fm, ns - s0))};
}

// ---- MXFP8 (OCP Microscaling Formats v1.0: e4m3fn elements, one e8m0 scale
// per 32 consecutive elements); used by the block-scaled expert path

// Four e4m3fn codes (byte i = code of v[i]): the nearest code, ties to the
// even one, saturating to +-448 (1.75 * 2^8, the largest finite e4m3fn
// value).  gfx950's converter rounds to nearest even in the OCP e4m3fn format
// but turns magnitudes that round past 448 into NaN, so inputs are clamped to
// +-448 first.  For every finite input of magnitude below 2^9 (all that the
// block quantiser below produces) this equals the code written out from the
// format's definition (checked over every bf16 bit pattern on the device).
__device__ __forceinline__ uint32_t e4m3x4(float v0, float v1, float v2, float v3) {
  constexpr float kMax = 448.0f;
  v0 = fminf(fmaxf(v0, -kMax), kMax);
  v1 = fminf(fmaxf(v1, -kMax), kMax);
  v2 = fminf(fmaxf(v2, -kMax), kMax);
  v3 = fminf(fmaxf(v3, -kMax), kMax);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);  // bytes 0, 1
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);       // bytes 2, 3
  return uint32_t(w);
}

// MXFP8 quantisation of one 32-element block (OCP MX: one shared e8m0 scale
// per 32 elements): scale exponent = floor(log2 amax) - 8 (clamped to e8m0's
// range; an all-zero block gets code 0), elements = e4m3(v / 2^exp).  A block
// holding a NaN or an infinity (e4m3fn has no infinity) becomes a NaN block:
// scale code 255 (e8m0's NaN) and every element code 0x7F (e4m3fn's NaN), so
// NaN reaches the product.  raw holds the block's 32 bf16 values; codes
// receives 32 e4m3 bytes.
__device__ __forceinline__ uint8_t quant_block32(const uint4 (&raw)[4], uint4 (&codes)[2]) {
  const bf16_t* h = reinterpret_cast<const bf16_t*>(raw);
  // the largest magnitude as a bf16 bit pattern: magnitudes order like their
  // patterns, infinity is 0x7F80 and every NaN lies above it
  uint32_t amag = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) amag = max(amag, uint32_t(h[i]) & 0x7fffu);
  if (amag >= 0x7f80u) {
    codes[0] = codes[1] = uint4{0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu};
    return uint8_t(255);
  }
  const float amax = __uint_as_float(amag << 16);
  int sexp = -127;
  if (amax > 0.0f) {
    const uint32_t au = __float_as_uint(amax);
    const int ebits = int((au >> 23) & 0xffu);
    // floor(log2 amax); bf16 subnormals (ebits == 0) are below 2^-126
    const int fl = ebits ? ebits - 127 : -127;
    sexp = max(-127, min(127, fl - 8));
  }
  const float inv = __uint_as_float(uint32_t(127 - sexp) << 23);  // 2^-sexp, exact (|sexp| <= 126 here)
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 8; ++w)
    out[w] = e4m3x4(bf16_to_f32(h[w * 4]) * inv, bf16_to_f32(h[w * 4 + 1]) * inv, bf16_to_f32(h[w * 4 + 2]) * inv,
                    bf16_to_f32(h[w * 4 + 3]) * inv);
  codes[0] = uint4{out[0], out[1], out[2], out[3]};
  codes[1] = uint4{out[4], out[5], out[6], out[7]};
  return uint8_t(sexp + 127);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Direct-to-LDS load: lane l's 16 bytes from gptr land at LDS byte
// lds_base + 16 l.  Inline asm, so the compiler sees no LDS write that
// it would order before every later LDS read (it cannot tell ring entries
// apart); the kernels order them with vmcnt waits and barriers.  lds_base goes
// to m0, so it must be wave-uniform.
template <bool NT = false>
__device__ __forceinline__ void g2lds16(const void* gptr, uint32_t lds_base) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds_base), "v"(gptr) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gptr) : "memory", "m0");
}

// The same from a wave-uniform base address plus a 32-bit lane offset (the
// base in scalar registers, so a kernel keeps one 32-bit register per lane
// and load instead of a 64-bit address).
template <bool NT = false>
__device__ __forceinline__ void g2lds16_so(const void* base, uint32_t off, uint32_t lds_base) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds_base), "v"(off), "s"(base)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(off), "s"(base)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N), leaving the other counters alone
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace lmoe
