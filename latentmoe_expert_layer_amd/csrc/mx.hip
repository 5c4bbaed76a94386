// MXFP4 expert path ("w4a8", TokenSpeed Day-0 post, "TensorRT-LLM Stable
// LatentMoE": MXFP4 weights; activations block-quantised to MXFP8 so the
// expert GEMMs run on FP8-activation MFMA; FC1's output is requantised to
// MXFP8 before FC2).  Encodings per OCP Microscaling Formats v1.0:
//   e2m1 weights, two per byte (even K index in the low nibble);
//   e4m3fn activations (OCP, not the fnuz variant);
//   one e8m0 scale (2^(code-127)) per 32 consecutive K elements.
#include <type_traits>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

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

// MXFP8 quantisation of bf16 rows [rows, K] -> e4m3 codes [rows, K] and e8m0
// scales [rows, K/32], one thread per 32-element block.
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const bf16_t* __restrict__ src, int64_t nblocks,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* p = reinterpret_cast<const uint4*>(src + b * 32);
  uint4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = p[i];
  uint4 q[2];
  scales[b] = quant_block32(raw, q);
  uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
  dst[0] = q[0];
  dst[1] = q[1];
}

typedef int i32x8v __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// D(32x32) += (A fp8 x B fp4) with e8m0 scales.  Operand layout (lane l,
// g = l/32, for one 64-wide K step): A row l%32 holds K [16g, 16g+16) in
// bytes 0-15 and K [32+16g, 32+16g+16) in bytes 16-31; B column l%32 holds K
// [32g, 32g+32) as 16 packed bytes; scale_a / scale_b are the e8m0 scales of
// the 32-element block g of that row / column.  Output layout as the bf16
// 32x32 MFMA.
__device__ __forceinline__ f32x16 mfma_mx(const i32x8v& a, const i32x8v& b, int sa, int sb, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0 /*A: fp8 e4m3*/, 4 /*B: fp4 e2m1*/, 0, sa, 0, sb);
}

constexpr int kMxBK = 128;               // K elements per LDS stage
constexpr int kMxARow = kMxBK + 16;      // A LDS row stride (bytes; fp8)
constexpr int kMxBRow = kMxBK / 2 + 16;  // B LDS row stride (bytes; packed fp4)

struct MxArgs {
  int N, K;
  const uint8_t* A;       // fp8 codes [rows, K]
  const uint8_t* As;      // scales [rows, K/32]
  const int32_t* a_rows;  // gather (FC1): row = a_rows[p] / a_row_div
  int a_row_div;
  const uint8_t* B;       // fp4 [E, N, K/2]
  const uint8_t* Bs;      // scales [E, N, K/32]
  const uint8_t* B3;      // gated: up projection
  const uint8_t* B3s;
  uint16_t* C;
  int64_t ldc;
  uint8_t* Cq;            // non-NULL: the output is written MXFP8-quantised (codes [rows, N], ldc)
  uint8_t* Cqs;           //   with e8m0 scales [rows, N/32] (row stride ldc/32), and C is not written
  const Tile* tiles;
  const int32_t* ntiles;
};

template <bool GATED, int BM = 256>
constexpr int mx_lds_bytes() {
  constexpr int stage = BM * kMxARow + 256 * kMxBRow + 512 * 4;  // one scale word per thread
  constexpr int epi = BM * ((GATED ? 128 : 256) + 8) * 2;
  return 2 * stage > epi ? 2 * stage : epi;
}

// Grouped block-scaled GEMM.  Macro tile = (expert segment of <= 256 rows,
// 256 B rows: plain -> 256 output columns; gated -> 128 gate + 128 up rows ->
// 128 output columns).  8 waves, 2 per SIMD, as 2 x 4 with 128 x 64 wave
// tiles (4 x 2 scaled 32x32x64 MFMAs per 64-wide K step); K in stages of 128
// through a double-buffered LDS holding A codes, B codes and both operands'
// e8m0 scales.  Per stage: MFMAs on the first 64 K | LDS writes of the next
// stage (loaded one stage earlier) | global loads of the stage after | MFMAs
// on the second 64 K | barrier.  A wave multiplies only its 32-row subtiles
// that hold rows of the tile; 64-row A chunks past the tile's rows are not
// loaded.
//
// DEEP (K >= 512): tiles of at most kTiledBM = 192 rows (the routing's cut),
// 96 x 64 wave tiles, and a second register set for the weight codes and the
// scale words, so those are loaded two stages ahead of their LDS write (the
// activation codes, from a cached matrix, one stage ahead): the accumulators
// this frees (96 instead of 128 registers per lane) pay for it, and twice as
// much of the weight stream is in flight per CU.  The same MFMAs in the same
// K order: bit-identical results.
// One macro tile: lt = m-tile * tiles_n + n-tile (in the XCD-aware order).
template <bool GATED, bool DEEP>
__device__ __forceinline__ void mx_tile(const MxArgs& g, uint32_t lt, uint8_t* lds) {
  constexpr int NTH = 512, BM = DEEP ? kTiledBM : 256, BR = 256, NOUT = GATED ? 128 : 256;
  constexpr int WAVES_N = 4, WM = BM / 2, WN = 64, FM = WM / 32, FN = 2;
  constexpr int A_CH = BM / 64;  // A rows i*64 + tid/8 per thread and stage
  static_assert(BM % 64 == 0 && BM + BR <= NTH, "tile shape");
  constexpr int A_STAGE = BM * kMxARow, B_STAGE = BR * kMxBRow;
  constexpr int STAGE = A_STAGE + B_STAGE + NTH * 4;  // scale words: one slot per thread

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int tiles_n = (g.N + NOUT - 1) / NOUT;
  const int tn = int(lt % uint32_t(tiles_n)), tm = int(lt / uint32_t(tiles_n));
  const Tile tl = g.tiles[tm];
  const int row0 = tl.row_start, nrows = tl.nrows, expert = tl.expert;
  const int n0 = tn * NOUT;
  const int K = g.K, KB = K / 32, nk = K / kMxBK;

  // Loads per stage: A rows i*64 + tid/8, 16-byte chunk tid%8 (i < 4); B rows
  // i*128 + tid/4, chunk tid%4 (i < 2; gated: i = 0 gate, i = 1 up); one
  // 4-byte scale word: A row tid (tid < 256) or B row tid - 256.
  auto a_src = [&](int r) __attribute__((always_inline)) -> int64_t {
    int64_t src = int64_t(row0) + min(r, nrows - 1);
    if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
    return src;
  };
  auto b_row = [&](int r, bool up) __attribute__((always_inline)) -> int64_t { return int64_t(expert) * g.N + min(n0 + r, g.N - 1); };
  const uint8_t* pa[A_CH];
  const uint8_t* pb[2];
  const uint8_t* ps;
#pragma unroll
  for (int i = 0; i < A_CH; ++i) pa[i] = g.A + a_src(i * 64 + tid / 8) * K + (tid % 8) * 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const bool up = GATED && i == 1;
    const int r = (GATED ? 0 : i * 128) + tid / 4;
    pb[i] = (up ? g.B3 : g.B) + b_row(r, up) * (K / 2) + (tid % 4) * 16;
  }
  // scale words: A row tid (tid < BM) or B row tid - BM (tid < BM + BR);
  // threads past that (DEEP) re-read B row 0's word into a slot nobody reads
  const bool has_scale = tid < BM + BR;
  if (tid < BM) {
    ps = g.As + a_src(tid) * KB;
  } else {
    const int r = has_scale ? tid - BM : 0;
    const bool up = GATED && r >= BR / 2;
    ps = (up ? g.B3s : g.Bs) + b_row(up ? r - BR / 2 : r, up) * KB;
  }

  u32x4v ra[A_CH], rb[2];  // native vectors, so the stage stays in registers
  uint32_t rs;
  u32x4v rb2[DEEP ? 2 : 1];  // DEEP: the second set of weight codes and scale word
  uint32_t rs2;
  // DEEP loads every A chunk (rows past the tile repeat its last row): with
  // no branch around them the two-ahead pipeline keeps its registers
  auto gload_a = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      if (DEEP || i * 64 < nrows) ra[i] = *reinterpret_cast<const u32x4v*>(pa[i]);
      pa[i] += kMxBK;
    }
  };
  auto gload_b = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rb[i] = *reinterpret_cast<const u32x4v*>(pb[i]);
      pb[i] += kMxBK / 2;
    }
    rs = *reinterpret_cast<const uint32_t*>(ps);
    ps += kMxBK / 32;
  };
  auto gload_b2 = [&]() __attribute__((always_inline)) {  // (separate code: a lambda taking
#pragma unroll                                              //  either set by reference would
    for (int i = 0; i < 2; ++i) {                           //  move the sets to memory)
      rb2[i] = *reinterpret_cast<const u32x4v*>(pb[i]);
      pb[i] += kMxBK / 2;
    }
    rs2 = *reinterpret_cast<const uint32_t*>(ps);
    ps += kMxBK / 32;
  };
  auto gload = [&]() __attribute__((always_inline)) {
    gload_a();
    gload_b();
  };
  auto lstore_a = [&](int buf) __attribute__((always_inline)) {
    uint8_t* sA = lds + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      if (DEEP || i * 64 < nrows) *reinterpret_cast<u32x4v*>(sA + (i * 64 + tid / 8) * kMxARow + (tid % 8) * 16) = ra[i];
  };
  auto lstore_b = [&](int buf) __attribute__((always_inline)) {
    uint8_t* sB = lds + buf * STAGE + A_STAGE;
    uint8_t* sS = sB + B_STAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4v*>(sB + (i * 128 + tid / 4) * kMxBRow + (tid % 4) * 16) = rb[i];
    if (DEEP || has_scale) *reinterpret_cast<uint32_t*>(sS + tid * 4) = rs;
  };
  auto lstore_b2 = [&](int buf) __attribute__((always_inline)) {
    uint8_t* sB = lds + buf * STAGE + A_STAGE;
    uint8_t* sS = sB + B_STAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4v*>(sB + (i * 128 + tid / 4) * kMxBRow + (tid % 4) * 16) = rb2[i];
    if (DEEP || has_scale) *reinterpret_cast<uint32_t*>(sS + tid * 4) = rs2;
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    lstore_a(buf);
    lstore_b(buf);
  };

  // B-tile row of this wave's n-subtile j (gated: j = 0 gate, j = 1 up)
  auto brow = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (GATED) return j == 0 ? wn * 32 : BR / 2 + wn * 32;
    else return wn * WN + j * 32;
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int gsel = lane >> 5, rl = lane & 31;
  auto mainloop = [&](auto fa_c) __attribute__((always_inline)) {
    constexpr int FA = decltype(fa_c)::value;
    // B fragments first, then A fragments two at a time (each fragment is 8
    // VGPRs; all four at once would push the 8-wave register budget)
    auto compute = [&](int buf, int ks) __attribute__((always_inline)) {
      if constexpr (FA > 0) {
        const uint8_t* sA = lds + buf * STAGE;
        const uint8_t* sB = sA + A_STAGE;
        const uint8_t* sS = sB + B_STAGE;
        i32x8v bf[FN];
        int sb[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = brow(j) + rl;
          const uint4 bw = *reinterpret_cast<const uint4*>(sB + r * kMxBRow + ks * 32 + 16 * gsel);
          bf[j] = i32x8v{int(bw.x), int(bw.y), int(bw.z), int(bw.w), 0, 0, 0, 0};
          sb[j] = sS[(BM + r) * 4 + ks * 2 + gsel];
        }
#pragma unroll
        for (int i0 = 0; i0 < FA; i0 += 2) {
          i32x8v af[2];
          int sa[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            if (i0 + u < FA) {
              const int r = wm * WM + (i0 + u) * 32 + rl;
              const uint4 lo = *reinterpret_cast<const uint4*>(sA + r * kMxARow + ks * 64 + 16 * gsel);
              const uint4 hi = *reinterpret_cast<const uint4*>(sA + r * kMxARow + ks * 64 + 32 + 16 * gsel);
              af[u] = i32x8v{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
              sa[u] = sS[r * 4 + ks * 2 + gsel];
            }
          }
#pragma unroll
          for (int u = 0; u < 2; ++u)
            if (i0 + u < FA)
#pragma unroll
              for (int j = 0; j < FN; ++j) acc[i0 + u][j] = mfma_mx(af[u], bf[j], sa[u], sb[j], acc[i0 + u][j]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    if constexpr (DEEP) {
      // step k: MFMAs on stage k (buffer k&1) around the LDS writes of stage
      // k+1 (weights from set 1 for even k, set 2 for odd k) and the loads of
      // A(k+2) and of the weights of stage k+3 into the set just written out;
      // each call site has a fixed set of writes and loads, so no load sits
      // behind a branch.  Needs nk even, >= 4.
      auto step = [&](int buf, bool second, bool st, bool la, bool lb) __attribute__((always_inline)) {
        compute(buf, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (st) {
          lstore_a(buf ^ 1);
          if (second) lstore_b2(buf ^ 1);
          else lstore_b(buf ^ 1);
        }
        if (la) gload_a();
        if (lb) {
          if (second) gload_b2();
          else gload_b();
        }
        __builtin_amdgcn_sched_barrier(0);
        compute(buf, 1);
        __syncthreads();
      };
      gload();
      lstore(0);
      gload();     // stage 1: A -> ra, weights -> set 1
      gload_b2();  // weights of stage 2 -> set 2
      __syncthreads();
      for (int kt = 0; kt < nk - 4; kt += 2) {
        step(0, false, true, true, true);
        step(1, true, true, true, true);
      }
      step(0, false, true, true, true);    // k = nk-4: loads A(nk-2), weights(nk-1)
      step(1, true, true, true, false);    // k = nk-3: loads A(nk-1)
      step(0, false, true, false, false);  // k = nk-2: writes stage nk-1
      step(1, true, false, false, false);
    } else {
      gload();
      lstore(0);
      if (nk > 1) gload();
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        compute(buf, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < nk) lstore(buf ^ 1);
        if (kt + 2 < nk) gload();
        __builtin_amdgcn_sched_barrier(0);
        compute(buf, 1);
        __syncthreads();
      }
    }
  };
  const int fa = wm * WM < nrows ? min(FM, (nrows - wm * WM + 31) / 32) : 0;
  switch (fa) {
    case 0: mainloop(std::integral_constant<int, 0>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 3: mainloop(std::integral_constant<int, 3>{}); break;
    default: mainloop(std::integral_constant<int, FM>{}); break;
  }

  // Epilogue (gated: SwiGLU of subtile 0 with its up subtile 1), bf16 staging
  // in LDS, then 16-byte row-contiguous stores.
  constexpr int CLD = NOUT + 8;
  static_assert(BM * CLD * 2 <= mx_lds_bytes<GATED, BM>(), "epilogue staging fits");
  bf16_t* Cs = reinterpret_cast<bf16_t*>(lds);
  constexpr int JO = GATED ? 1 : FN, WO = GATED ? WN / 2 : WN;
#pragma unroll
  for (int i = 0; i < FM; ++i)
    if (i < fa)
#pragma unroll
      for (int j = 0; j < JO; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int col = wn * WO + j * 32 + rl;
          float x = acc[i][j][v];
          if constexpr (GATED) x = silu_mul(x, acc[i][1][v]);
          Cs[row * CLD + col] = f32_to_bf16(x);
        }
  __syncthreads();
  if (g.Cq) {
    // quantised output (the next GEMM's MXFP8 operand): one thread per
    // (row, 32-column block) of the bf16 tile staged above
    constexpr int BPR = NOUT / 32;
    for (int c = tid; c < BM * BPR; c += NTH) {
      const int row = c / BPR, b = c % BPR, col = n0 + b * 32;
      if (row < nrows && col < g.N) {
        uint4 raw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = *reinterpret_cast<const uint4*>(&Cs[row * CLD + b * 32 + i * 8]);
        uint4 q[2];
        const int64_t r = int64_t(row0) + row;
        g.Cqs[r * (g.ldc / 32) + col / 32] = quant_block32(raw, q);
        uint4* dst = reinterpret_cast<uint4*>(g.Cq + r * g.ldc + col);
        dst[0] = q[0];
        dst[1] = q[1];
      }
    }
    return;
  }
  constexpr int OCPR = NOUT / 8;
  for (int c = tid; c < BM * OCPR; c += NTH) {
    const int row = c / OCPR, cc = c % OCPR;
    if (row < nrows && n0 + cc * 8 < g.N) {
      *reinterpret_cast<uint4*>(g.C + (int64_t(row0) + row) * g.ldc + n0 + cc * 8) =
          *reinterpret_cast<const uint4*>(&Cs[row * CLD + cc * 8]);
    }
  }
}

// The grid covers an upper bound on the tile count: blocks past the
// device-side count exit, and the XCD-aware order spans the real tiles only,
// so they spread over every XCD.  PERSIST: one workgroup per CU takes tiles
// b, b + grid, ... (block b stays on its XCD, so the order keeps its
// meaning); a tile's output stores drain while the next tile's loads and
// MFMAs run.
template <bool GATED, bool DEEP, bool PERSIST>
__global__ __launch_bounds__(512, 1) void mx_grouped_kernel(MxArgs g) {
  extern __shared__ uint4 lds_u4[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(lds_u4);
  constexpr int NOUT = GATED ? 128 : 256;
  const uint32_t nreal = uint32_t(*g.ntiles) * uint32_t((g.N + NOUT - 1) / NOUT);
  if constexpr (PERSIST) {
    for (uint32_t b = blockIdx.x; b < nreal; b += gridDim.x) {
      mx_tile<GATED, DEEP>(g, xcd_swizzle(b, nreal), lds);
      __syncthreads();  // the next tile's first stage reuses the LDS the epilogue read
    }
  } else {
    if (blockIdx.x >= nreal) return;
    mx_tile<GATED, DEEP>(g, xcd_swizzle(blockIdx.x, nreal), lds);
  }
}

template <bool GATED, bool DEEP, bool PERSIST>
hipError_t run_mx(const MxArgs& a, int64_t max_tiles, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  constexpr int NOUT = GATED ? 128 : 256;
  constexpr size_t lds = size_t(mx_lds_bytes<GATED, DEEP ? kTiledBM : 256>());
  auto kern = mx_grouped_kernel<GATED, DEEP, PERSIST>;
  if (hipError_t e = allow_dynamic_lds((const void*)kern, int(lds)); e != hipSuccess) return e;
  int64_t nblk = max_tiles * ((a.N + NOUT - 1) / NOUT);
  if (nblk <= 0) return hipSuccess;
  if (PERSIST) {
    int dev = 0, ncu = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
    if (hipError_t e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev); e != hipSuccess)
      return e;
    nblk = std::min<int64_t>(nblk, ncu);  // one workgroup per CU (its LDS and registers allow no more)
  }
  return launch_kernel((const void*)kern, dim3{uint32_t(nblk)}, dim3{512}, lds, s, a, t0, t1);
}

}  // namespace

hipError_t launch_quant_mxfp8(const uint16_t* src, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
  const int64_t nb = rows * (K / 32);
  if (nb <= 0) return hipSuccess;
  quant_mxfp8_kernel<<<dim3{uint32_t((nb + 255) / 256)}, dim3{256}, 0, s>>>(src, nb, codes, scales);
  return hipGetLastError();
}

hipError_t launch_grouped_mx(const GroupedMx& g, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  MxArgs a{};
  a.N = g.N;
  a.K = g.K;
  a.A = g.A;
  a.As = g.As;
  a.a_rows = g.a_rows;
  a.a_row_div = g.a_row_div;
  a.B = g.B;
  a.Bs = g.Bs;
  a.B3 = g.B3;
  a.B3s = g.B3s;
  a.C = g.C;
  a.ldc = g.ldc;
  a.Cq = g.Cq;
  a.Cqs = g.Cqs;
  a.tiles = g.tiles;
  a.ntiles = g.ntiles;
  // routing cuts tiles at kTiledBM rows, within both kernels' reach; the deep
  // pipeline needs an even number (>= 4) of 128-wide K stages
  static_assert(kTiledBM <= 256 && kTiledBM % 64 == 0, "tile table granularity");
  // FC2 (plain, bf16 output) writes 2 bytes per output against a short K:
  // in the deep form its stores get the persistent grid, to drain behind the
  // next tile (the 256-row form has no registers to spare for it)
  if (g.K % 256 == 0 && g.K >= 512)
    return g.gated ? run_mx<true, true, false>(a, g.max_tiles, s, t0, t1)
                   : run_mx<false, true, true>(a, g.max_tiles, s, t0, t1);
  return g.gated ? run_mx<true, false, false>(a, g.max_tiles, s, t0, t1)
                 : run_mx<false, false, false>(a, g.max_tiles, s, t0, t1);
}

}  // namespace lmoe
