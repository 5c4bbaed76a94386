// MXFP4 expert path ("w4a8", TokenSpeed Day-0 post, "TensorRT-LLM Stable
// LatentMoE": MXFP4 weights; activations block-quantised to MXFP8 so the
// expert GEMMs run on FP8-activation MFMA; FC1's output is requantised to
// MXFP8 before FC2).  Encodings per OCP Microscaling Formats v1.0:
//   e2m1 weights, two per byte (even K index in the low nibble);
//   e4m3fn activations (OCP, not the fnuz variant);
//   one e8m0 scale (2^(code-127)) per 32 consecutive K elements.
#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

// Nearest e4m3fn code to v (finite), ties to the even code, saturating to
// +-448 (1.75 * 2^8, the largest finite e4m3fn value).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal codes m * 2^-9, m = 0..8
    const uint32_t m = uint32_t(rintf(a * 512.0f));  // exact scaling, rint = nearest even
    return sign | m;                                  // m == 8 is the smallest normal (code 8)
  }
  const uint32_t au = __float_as_uint(a);
  int e = int((au >> 23) & 0xffu) - 127;              // -6 .. 8
  uint32_t q = (au >> 20) & 7u;                       // top 3 mantissa bits
  const uint32_t rest = au & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (q & 1u))) ++q;
  if (q == 8u) {
    q = 0u;
    ++e;
  }
  return sign | (uint32_t(e + 7) << 3) | q;           // a < 448 keeps the code <= 0x7E
}

// MXFP8 quantisation of bf16 rows [rows, K] -> e4m3 codes [rows, K] and e8m0
// scales [rows, K/32]: scale exponent = floor(log2 amax) - 8 (clamped to
// e8m0's range; an all-zero block gets code 0), elements = e4m3(v / 2^exp).
// One thread per 32-element block.
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const bf16_t* __restrict__ src, int64_t nblocks,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* p = reinterpret_cast<const uint4*>(src + b * 32);
  uint4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = p[i];
  const bf16_t* h = reinterpret_cast<const bf16_t*>(raw);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(bf16_to_f32(h[i])));
  int sexp = -127;
  if (amax > 0.0f) {
    const uint32_t au = __float_as_uint(amax);
    const int ebits = int((au >> 23) & 0xffu);
    // floor(log2 amax); bf16 subnormals (ebits == 0) are below 2^-126
    const int fl = ebits ? ebits - 127 : -127;
    sexp = max(-127, min(127, fl - 8));
  }
  scales[b] = uint8_t(sexp + 127);
  const float inv = __uint_as_float(uint32_t(127 - sexp) << 23);  // 2^-sexp, exact (|sexp| <= 126 here)
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) word |= e4m3_rne(bf16_to_f32(h[w * 4 + i]) * inv) << (8 * i);
    out[w] = word;
  }
  uint4* q = reinterpret_cast<uint4*>(codes + b * 32);
  q[0] = uint4{out[0], out[1], out[2], out[3]};
  q[1] = uint4{out[4], out[5], out[6], out[7]};
}

typedef int i32x8v __attribute__((ext_vector_type(8)));

// D(32x32) += (A fp8 x B fp4) with e8m0 scales.  Operand layout (lane l,
// g = l/32, for one 64-wide K step): A row l%32 holds K [16g, 16g+16) in
// bytes 0-15 and K [32+16g, 32+16g+16) in bytes 16-31; B column l%32 holds K
// [32g, 32g+32) as 16 packed bytes; scale_a / scale_b are the e8m0 scales of
// the 32-element block g of that row / column.  Output layout as the bf16
// 32x32 MFMA.
__device__ __forceinline__ f32x16 mfma_mx(const i32x8v& a, const i32x8v& b, int sa, int sb, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0 /*A: fp8 e4m3*/, 4 /*B: fp4 e2m1*/, 0, sa, 0, sb);
}

constexpr int kMxBK = 128;            // K elements per LDS stage
constexpr int kMxARow = kMxBK + 16;   // A LDS row stride (bytes)
constexpr int kMxBRow = kMxBK / 2 + 16;  // B LDS row stride (bytes)

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
  bool gated;
  uint16_t* C;
  int64_t ldc;
  const Tile* tiles;
  const int32_t* ntiles;
};

// Grouped block-scaled GEMM.  Tile = (expert segment of <= 256 rows, 128 B
// rows: plain -> 128 output columns, gated -> 64 gate + 64 up -> 64 output
// columns).  4 waves stacked along M (64 rows each; a wave with no rows
// skips its MFMAs); K in stages of 128 through a double-buffered LDS.
template <bool GATED>
__global__ __launch_bounds__(256, 1) void mx_grouped_kernel(MxArgs g) {
  constexpr int BM = 256, BR = 128, NOUT = GATED ? 64 : 128;
  constexpr int A_STAGE = BM * kMxARow, B_STAGE = BR * kMxBRow;
  constexpr int AS_STAGE = BM * (kMxBK / 32), BS_STAGE = BR * (kMxBK / 32);
  constexpr int STAGE = A_STAGE + B_STAGE + AS_STAGE + BS_STAGE;
  extern __shared__ uint4 lds_u4[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(lds_u4);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int tiles_n = (g.N + NOUT - 1) / NOUT;
  const uint32_t lt = xcd_swizzle(blockIdx.x, gridDim.x);
  const int tn = int(lt % uint32_t(tiles_n)), tm = int(lt / uint32_t(tiles_n));
  if (tm >= *g.ntiles) return;
  const Tile tl = g.tiles[tm];
  const int row0 = tl.row_start, nrows = tl.nrows, expert = tl.expert;
  const int n0 = tn * NOUT;
  const bool active = wid * 64 < nrows;
  const int K = g.K, KB = K / 32;

  // global -> register assignments (per stage): A 256 rows x 128 B = 8 x 16 B
  // per thread; B 128 rows x 64 B = 2 x 16 B per thread; scales 4 B per row.
  const uint8_t* ap[8];
  const uint8_t* asp;
  const uint8_t* bp[2];
  const uint8_t* bsp = nullptr;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
    int64_t src = int64_t(row0) + min(r, nrows - 1);
    if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
    ap[i] = g.A + src * K + kc * 16;
  }
  {
    int64_t src = int64_t(row0) + min(tid, nrows - 1);
    if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
    asp = g.As + src * KB;
  }
  auto brow_ptr = [&](int r, const uint8_t* base, const uint8_t* base3, int64_t stride) -> const uint8_t* {
    const bool up = GATED && r >= BR / 2;
    const int rn = min(n0 + (up ? r - BR / 2 : r), g.N - 1);
    return (up ? base3 : base) + (int64_t(expert) * g.N + rn) * stride;
  };
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i, r = c >> 2, kc = c & 3;
    bp[i] = brow_ptr(r, g.B, g.B3, K / 2) + kc * 16;
  }
  if (tid < BR) bsp = brow_ptr(tid, g.Bs, g.B3s, KB);

  uint4 ra[8], rb[2];
  uint32_t rsa = 0, rsb = 0;
  auto gload = [&](int kt) {
    const int ko = kt * kMxBK;
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = *reinterpret_cast<const uint4*>(ap[i] + ko);
#pragma unroll
    for (int i = 0; i < 2; ++i) rb[i] = *reinterpret_cast<const uint4*>(bp[i] + ko / 2);
    rsa = *reinterpret_cast<const uint32_t*>(asp + ko / 32);
    if (tid < BR) rsb = *reinterpret_cast<const uint32_t*>(bsp + ko / 32);
  };
  auto lstore = [&](int buf) {
    uint8_t* st = lds + buf * STAGE;
    uint8_t* sA = st;
    uint8_t* sB = st + A_STAGE;
    uint8_t* sAs = sB + B_STAGE;
    uint8_t* sBs = sAs + AS_STAGE;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<uint4*>(sA + (c >> 3) * kMxARow + (c & 7) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<uint4*>(sB + (c >> 2) * kMxBRow + (c & 3) * 16) = rb[i];
    }
    *reinterpret_cast<uint32_t*>(sAs + tid * 4) = rsa;
    if (tid < BR) *reinterpret_cast<uint32_t*>(sBs + tid * 4) = rsb;
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = K / kMxBK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int gsel = lane >> 5, rl = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    if (active) {
      const uint8_t* st = lds + buf * STAGE;
      const uint8_t* sA = st;
      const uint8_t* sB = st + A_STAGE;
      const uint8_t* sAs = sB + B_STAGE;
      const uint8_t* sBs = sAs + AS_STAGE;
#pragma unroll
      for (int ks = 0; ks < kMxBK / 64; ++ks) {
        i32x8v af[2];
        int sa[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = wid * 64 + i * 32 + rl;
          const uint4 lo = *reinterpret_cast<const uint4*>(sA + r * kMxARow + ks * 64 + 16 * gsel);
          const uint4 hi = *reinterpret_cast<const uint4*>(sA + r * kMxARow + ks * 64 + 32 + 16 * gsel);
          af[i] = i32x8v{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
          sa[i] = sAs[r * 4 + ks * 2 + gsel];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = j * 32 + rl;
          const uint4 bw = *reinterpret_cast<const uint4*>(sB + r * kMxBRow + ks * 32 + 16 * gsel);
          const i32x8v bf = i32x8v{int(bw.x), int(bw.y), int(bw.z), int(bw.w), 0, 0, 0, 0};
          const int sb = sBs[r * 4 + ks * 2 + gsel];
#pragma unroll
          for (int i = 0; i < 2; ++i) acc[i][j] = mfma_mx(af[i], bf, sa[i], sb, acc[i][j]);
        }
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue (SwiGLU for gated: subtiles 0-1 gate, 2-3 up), bf16 staging in
  // LDS, then 16-byte row-contiguous stores.
  constexpr int CLD = NOUT + 8;
  bf16_t* Cs = reinterpret_cast<bf16_t*>(lds);
  static_assert(BM * CLD * 2 <= 2 * STAGE, "epilogue staging fits");
  if (active) {
    constexpr int JO = GATED ? 2 : 4;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < JO; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wid * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int col = j * 32 + rl;
          float x = acc[i][j][v];
          if constexpr (GATED) x = silu_mul(x, acc[i][j + 2][v]);
          Cs[row * CLD + col] = f32_to_bf16(x);
        }
  }
  __syncthreads();
  constexpr int OCPR = NOUT / 8;
  for (int c = tid; c < BM * OCPR; c += 256) {
    const int row = c / OCPR, cc = c % OCPR;
    if (row < nrows && n0 + cc * 8 < g.N) {
      *reinterpret_cast<uint4*>(g.C + (int64_t(row0) + row) * g.ldc + n0 + cc * 8) =
          *reinterpret_cast<const uint4*>(&Cs[row * CLD + cc * 8]);
    }
  }
}

template <bool GATED>
hipError_t run_mx(const MxArgs& a, int64_t max_tiles, hipStream_t s) {
  constexpr int NOUT = GATED ? 64 : 128;
  constexpr int STAGE = 256 * kMxARow + 128 * kMxBRow + 256 * (kMxBK / 32) + 128 * (kMxBK / 32);
  const size_t lds = size_t(2) * STAGE;
  auto kern = mx_grouped_kernel<GATED>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t nblk = max_tiles * ((a.N + NOUT - 1) / NOUT);
  if (nblk <= 0) return hipSuccess;
  kern<<<dim3{uint32_t(nblk)}, dim3{256}, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_mxfp8(const uint16_t* src, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
  const int64_t nb = rows * (K / 32);
  if (nb <= 0) return hipSuccess;
  quant_mxfp8_kernel<<<dim3{uint32_t((nb + 255) / 256)}, dim3{256}, 0, s>>>(src, nb, codes, scales);
  return hipGetLastError();
}

hipError_t launch_grouped_mx(const GroupedMx& g, hipStream_t s) {
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
  a.gated = g.gated;
  a.C = g.C;
  a.ldc = g.ldc;
  a.tiles = g.tiles;
  a.ntiles = g.ntiles;
  return g.gated ? run_mx<true>(a, g.max_tiles, s) : run_mx<false>(a, g.max_tiles, s);
}

}  // namespace lmoe
