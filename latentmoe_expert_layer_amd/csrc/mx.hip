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

// Epilogue of a tile of BM rows whose accumulators are acc (this wave's fa
// 32x32 fragments of rows from tile row r0, x 64 columns): gated, SwiGLU of
// subtile 0 with its up subtile 1; the bf16 tile is staged in the LDS (free
// on entry), then written as MXFP8 codes and scales (Cq set) or as bf16, in
// 16-byte row-contiguous stores.
template <bool GATED, int BM, int FM, int LDSB>
__device__ __forceinline__ void mx_epilogue(const MxArgs& g, const f32x16 (&acc)[FM][2], int fa, int r0, uint8_t* lds,
                                            int row0, int nrows, int n0) {
  constexpr int NTH = 512, NOUT = GATED ? 128 : 256, WAVES_N = 4, WN = 64, FN = 2;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, rl = lane & 31;
  const int wn = wid % WAVES_N;
  constexpr int CLD = NOUT + 8;
  static_assert(BM * CLD * 2 <= LDSB, "epilogue staging fits");
  bf16_t* Cs = reinterpret_cast<bf16_t*>(lds);
  constexpr int JO = GATED ? 1 : FN, WO = GATED ? WN / 2 : WN;
#pragma unroll
  for (int i = 0; i < FM; ++i)
    if (i < fa)
#pragma unroll
      for (int j = 0; j < JO; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = r0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
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

  mx_epilogue<GATED, BM, FM, mx_lds_bytes<GATED, BM>()>(g, acc, fa, wm * WM, lds, row0, nrows, n0);
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


// ------------------------------------------------ direct-to-LDS ring form ---
// The deep form's tiles (at most 192 rows; 8 waves as 2 x 4 with 96 x 64 wave
// tiles) with the operands moved into LDS by direct-to-LDS loads of whole
// 128-byte lines, as the bf16 ring kernels do, instead of through registers.
// A stage is 128 K: 192 rows x 128 B of activation codes.  A stage's weight
// codes are 64 B per row, half a line, so the weights travel in pairs of
// stages (256 rows x 128 B).  The e8m0 scales (4 bytes per row and stage)
// travel in groups of four stages: 16 bytes per row, one load per 64 rows.
// Loaded one stage at a time they would be 4-byte gathers, each asking for 64
// separate lines: more line requests than all the codes together, and the
// largest cost of the loads.  LDS slots: three for activation stages, two for
// weight pairs, two for scale groups (152 KB).  The prologue loads S0 W0 A0
// A1 W1 A2 (S: a scale group, W: a weight pair, A: a stage's activation
// codes).  After the barrier of stage s, the stage reloads its activation
// slot with A(s+3); an odd stage, the last user of its pair, also reloads the
// pair's slot with the pair (s+3)/2; a stage 4g also loads scale group g+1
// into the slot group g-1 left.  Codes land three stages before their use,
// scales four.  One barrier per stage, before its second 64-K step: each wave
// first waits for its LDS reads (lgkmcnt) and for its loads of stage s+1.
// vmcnt counts in issue order, so the wait names how many of the wave's
// newest loads may still be in flight: in the loop, after stage s mod 4 =
// 0, 1, 2, 3, these are 7 (a pair and A(s+2)), 4 (a scale group and A(s+2)),
// 7 and 3 (A(s+2)); in the last four stages 7, 3, 0 and none.  After the
// barrier stage s+1 is visible and the slots stage s freed are refilled while
// the second step's MFMAs run from registers.  Code rows are 128 B with the
// 16-byte chunks XOR-swizzled by (row / 2) mod 8.  The MFMAs and their K
// order are the deep form's: the results are bit-identical.  Needs K a
// multiple of 512.
constexpr int kMxrA = kTiledBM * kMxBK;         // one stage's activation codes: 24 KB
constexpr int kMxrB = 256 * 128;                // a weight pair: 32 KB
constexpr int kMxrS = 512 * 16;                 // a scale group: 192 + 256 rows (+64 spare) x 16 B
constexpr int kMxrBOff = 3 * kMxrA;             // weight pair slots
constexpr int kMxrSOff = kMxrBOff + 2 * kMxrB;  // scale group slots
constexpr int kMxrLds = kMxrSOff + 2 * kMxrS;   // 152 KiB

// One tile.  Operand addresses are 32-bit offsets from wave-uniform bases:
// the activation codes and scales from A and As (which the host checks to be
// below 2^31 bytes), the weights from the tile's expert matrices.
template <bool GATED>
__device__ __forceinline__ void mx_ring_tile(const MxArgs& g, uint32_t lt, uint8_t* lds, uint32_t lds0) {
  constexpr int NW = 8, BM = kTiledBM, BR = 256, NOUT = GATED ? 128 : 256, WAVES_N = 4;
  constexpr int WM = BM / 2, WN = 64, FM = WM / 32, FN = 2, ROWB = 128;
  constexpr int LA = BM / 8 / NW;   // activation code loads (1 KB each) per wave and stage
  constexpr int LB = BR / 8 / NW;   // weight code loads per wave and stage pair
  constexpr int LS = 1;             // scale loads per wave and group
  static_assert(BM % (8 * NW) == 0 && BM + BR <= NW * 64 && LB == 4, "tile rows");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int tiles_n = (g.N + NOUT - 1) / NOUT;
  const int tn = int(lt % uint32_t(tiles_n)), tm = int(lt / uint32_t(tiles_n));
  const Tile tl = g.tiles[tm];
  const int row0 = __builtin_amdgcn_readfirstlane(tl.row_start);
  const int nrows = __builtin_amdgcn_readfirstlane(tl.nrows);
  const int expert = __builtin_amdgcn_readfirstlane(tl.expert);
  const int n0 = tn * NOUT;
  const int K = g.K, KB = K / 32, nk = K / kMxBK;
  const WaveRows wr = wave_rows(wm, nrows, FM);  // this wave row's first tile row and subtiles

  // tile row r's activation row (rows past the tile repeat its last one)
  auto a_src = [&](int r) __attribute__((always_inline)) -> uint32_t {
    int src = row0 + min(r, nrows - 1);
    if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
    return uint32_t(src);
  };
  // LDS weight row r (gated: 128 gate rows, then 128 up rows): its row in the
  // expert's matrix
  auto w_row = [&](int r) __attribute__((always_inline)) -> uint32_t {
    return uint32_t(min(n0 + (GATED && r >= BR / 2 ? r - BR / 2 : r), g.N - 1));
  };
  const int64_t wexp = int64_t(expert) * g.N;
  const uint8_t* wg = g.B + wexp * (K / 2);  // the expert's gate (plain: only) codes
  const uint8_t* wu = GATED ? g.B3 + wexp * (K / 2) : wg;
  // Code loads: lane l of wave w takes row 8 (w + 8 q) + l/8 of its operand,
  // into chunk l%8 of the LDS row, from global chunk (l%8) ^ ((row/2) mod 8);
  // weight loads q < 2 take rows 0..127 (gated: gate rows), q >= 2 rows
  // 128..255 (gated: up rows).  Scale loads: lane l of wave w takes the 16
  // bytes of scale row 64 w + l of [192 activation rows, 256 weight rows,
  // weight rows 0..63 again (a spare copy that nobody reads)], so each wave's
  // scale base is uniform.
  const uint32_t gc = uint32_t(((lane & 7) ^ ((((wid & 1) << 2) + (lane >> 4)) & 7)) * 16);
  uint32_t oa[LA], ob[LB], os;
#pragma unroll
  for (int q = 0; q < LA; ++q) oa[q] = a_src(8 * (wid + NW * q) + (lane >> 3)) * uint32_t(K) + gc;
#pragma unroll
  for (int q = 0; q < LB; ++q) ob[q] = w_row(8 * (wid + NW * q) + (lane >> 3)) * uint32_t(K / 2) + gc;
  const uint8_t* sbase;
  {
    const int idx = wid * 64 + lane;
    if (wid < BM / 64) {
      sbase = g.As;
      os = a_src(idx) * uint32_t(KB);
    } else {
      const int r = wid < (BM + BR) / 64 ? idx - BM : idx - BM - BR;
      sbase = (GATED && wid >= (BM + BR / 2) / 64 && wid < (BM + BR) / 64 ? g.B3s : g.Bs) + wexp * KB;
      os = w_row(r) * uint32_t(KB);
    }
  }
  auto rfl = [](uint32_t v) __attribute__((always_inline)) -> uint32_t {
    return uint32_t(__builtin_amdgcn_readfirstlane(int(v)));
  };
  auto issue_a = [&](int slot, int q) __attribute__((always_inline)) {
    g2lds16_so(g.A, oa[q], rfl(lds0 + slot * kMxrA + (wid + NW * q) * 1024));
  };
  auto next_a = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LA; ++q) oa[q] += kMxBK;
  };
  auto issue_b = [&](int slot, int q) __attribute__((always_inline)) {
    g2lds16_so(q < LB / 2 ? wg : wu, ob[q], rfl(lds0 + kMxrBOff + slot * kMxrB + (wid + NW * q) * 1024));
  };
  auto next_b = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LB; ++q) ob[q] += kMxBK;  // two stages of packed codes
  };
  auto issue_s = [&](int slot) __attribute__((always_inline)) {
    g2lds16_so(sbase, os, rfl(lds0 + kMxrSOff + slot * kMxrS + wid * 1024));
    os += 4 * kMxBK / 32;
  };
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

  const int fr = lane & 31, fsw = (fr >> 1) & 7, fh = lane >> 5;  // fragment row, its swizzle, K half
  auto mainloop = [&](auto fa_c) __attribute__((always_inline)) {
    constexpr int FA = decltype(fa_c)::value, FAR = FA > 0 ? FA : 1;
    // one set of activation fragments, each reloaded after its last MFMA;
    // two sets of weight fragments (the 64-K step t's set is t)
    i32x8v af[FAR];
    int sa[FAR];
    uint4 bq[2][FN];
    int sb[2][FN];
    // Fragments of the 64-K step t of stage s, R = s mod 4: its activation
    // codes in slot as, its pair in slot bs, its scales in group slot ss.
    auto rd_a = [&](int as, int ss, int R, int t, int i) __attribute__((always_inline)) {
      const uint8_t* E = lds + as * kMxrA;
      const int r = wr.r0 + i * 32 + fr;
      const uint4 lo = *reinterpret_cast<const uint4*>(E + r * ROWB + (((4 * t + fh) ^ fsw) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(E + r * ROWB + (((4 * t + 2 + fh) ^ fsw) << 4));
      af[i] = i32x8v{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      sa[i] = lds[kMxrSOff + ss * kMxrS + r * 16 + 4 * R + 2 * t + fh];
    };
    auto rd_b = [&](int bs, int ss, int R, int t, int j) __attribute__((always_inline)) {
      const int r = brow(j) + fr;
      bq[t][j] = *reinterpret_cast<const uint4*>(lds + kMxrBOff + bs * kMxrB + r * ROWB +
                                                 (((4 * (R & 1) + 2 * t + fh) ^ fsw) << 4));
      sb[t][j] = lds[kMxrSOff + ss * kMxrS + (BM + r) * 16 + 4 * R + 2 * t + fh];
    };
    // the 64-K step t's MFMAs (activation fragment major).  With rd set, the
    // fragments of step tn of the stage (as, bs, ss, R) are read under them:
    // the weight set after the first MFMA, each activation fragment after its
    // last MFMA.  The nside side items (loads) are spread over the MFMAs in
    // order: MFMA m is followed by items c m .. c m + c - 1, c = ceil(nside /
    // NM) (all at once if NM = 0).  The order matters: the waits count on
    // each wave's loads leaving in the order issued.
    auto mm = [&](int t, bool rd, int as, int bs, int ss, int R, int tn, int nside, auto side)
                  __attribute__((always_inline)) {
      constexpr int NM = FA * FN;
      const int c = NM > 0 ? (nside + NM - 1) / NM : 0;
#pragma unroll
      for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint4 b = bq[t][j];
          acc[i][j] = mfma_mx(af[i], i32x8v{int(b.x), int(b.y), int(b.z), int(b.w), 0, 0, 0, 0}, sa[i], sb[t][j],
                              acc[i][j]);
          const int m = i * FN + j;
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (k >= m * c && k < m * c + c && k < nside) side(k);
          if (rd && m == 0)
#pragma unroll
            for (int j2 = 0; j2 < FN; ++j2) rd_b(bs, ss, R, tn, j2);
          if (rd && j == FN - 1) rd_a(as, ss, R, tn, i);
          __builtin_amdgcn_sched_barrier(0);
        }
      if constexpr (NM == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < nside) side(k);
        if (rd)
#pragma unroll
          for (int j2 = 0; j2 < FN; ++j2) rd_b(bs, ss, R, tn, j2);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(LS + LB + LA <= 8, "side items");
    int as0 = 0;  // A(s)'s slot: s mod 3
    int ss0 = 0;  // stage s's scale group slot
    // stage s, R = s mod 4.  W: loads allowed in flight at the barrier (-1:
    // the last stage, no barrier); IA / IB / IS: load A(s+3) / the pair
    // (s+3)/2 (odd R) / scale group s/4 + 1 (R = 0)
    auto step = [&](auto r_c, auto w_c, auto ia_c, auto ib_c, auto is_c) __attribute__((always_inline)) {
      constexpr int R = decltype(r_c)::value, W = decltype(w_c)::value;
      constexpr bool IA = decltype(ia_c)::value, IB = decltype(ib_c)::value, IS = decltype(is_c)::value;
      static_assert(!IB || (R & 1), "pairs are reloaded by odd stages");
      static_assert(!IS || R == 0, "scale groups are loaded by stages 4g");
      constexpr int BS = R >> 1, BSN = ((R + 1) & 3) >> 1;  // pair slots of stages s and s+1
      mm(0, true, as0, BS, ss0, R, 1, 0, [&](int) {});
      if constexpr (W >= 0) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of stage s are done
        wait_vmcnt<W>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");       // no LDS read moves above the barrier
      }
      __builtin_amdgcn_sched_barrier(0);
      const int as1 = as0 == 2 ? 0 : as0 + 1, ss1 = R == 3 ? ss0 ^ 1 : ss0;
      constexpr int NS = IS ? LS : 0, NB = IB ? LB : 0, NA = IA ? LA : 0;
      mm(1, W >= 0, as1, BSN, ss1, (R + 1) & 3, 0, NS + NB + NA, [&](int k) __attribute__((always_inline)) {
        if (k < NS) issue_s(ss0 ^ 1);         // scale group s/4 + 1
        else if (k < NS + NB) issue_b(BS, k - NS);  // the pair (s+3)/2 into the slot of pair s/2
        else issue_a(as0, k - NS - NB);       // A(s+3) into A(s)'s slot
      });
      if constexpr (NB > 0) next_b();
      if constexpr (NA > 0) next_a();
      as0 = as1;
      ss0 = ss1;
    };
    using T = std::true_type;
    using F = std::false_type;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using W7 = std::integral_constant<int, LB + LA>;
    using W4 = std::integral_constant<int, LS + LA>;
    using W3 = std::integral_constant<int, LA>;
    using W0 = std::integral_constant<int, 0>;
    using Wm = std::integral_constant<int, -1>;
    issue_s(0);  // S0
#pragma unroll
    for (int q = 0; q < LB; ++q) issue_b(0, q);  // W0
    next_b();
#pragma unroll
    for (int e = 0; e < 2; ++e) {  // A0, A1
#pragma unroll
      for (int q = 0; q < LA; ++q) issue_a(e, q);
      next_a();
    }
#pragma unroll
    for (int q = 0; q < LB; ++q) issue_b(1, q);  // W1
    next_b();
#pragma unroll
    for (int q = 0; q < LA; ++q) issue_a(2, q);  // A2
    next_a();
    wait_vmcnt<2 * LA + LB>();  // S0, W0 and A0 have landed; A1, W1, A2 may be in flight
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < FN; ++j) rd_b(0, 0, 0, 0, j);
#pragma unroll
    for (int i = 0; i < FA; ++i) rd_a(0, 0, 0, 0, i);
    for (int s = 0; s + 4 < nk; s += 4) {
      step(I0{}, W7{}, T{}, F{}, T{});
      step(I1{}, W4{}, T{}, T{}, F{});
      step(I2{}, W7{}, T{}, F{}, F{});
      step(I3{}, W3{}, T{}, T{}, F{});
    }
    step(I0{}, W7{}, T{}, F{}, F{});  // s = nk-4: A(nk-1)
    step(I1{}, W3{}, F{}, F{}, F{});
    step(I2{}, W0{}, F{}, F{}, F{});
    step(I3{}, Wm{}, F{}, F{}, F{});
  };
  const int fa = wr.fa;
  switch (fa) {
    case 0: mainloop(std::integral_constant<int, 0>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    default: mainloop(std::integral_constant<int, FM>{}); break;
  }
  __syncthreads();
  mx_epilogue<GATED, BM, FM, kMxrLds>(g, acc, fa, wr.r0, lds, row0, nrows, n0);
}

// A persistent grid (one workgroup per CU) in mirrored_tile's order, so a
// tile's output stores drain while the next tile's first stages load.
template <bool GATED>
__global__ __launch_bounds__(512, 1) void mx_ring_kernel(MxArgs g) {
#if defined(__HIP_DEVICE_COMPILE__)
  extern __shared__ uint4 lds_u4[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(lds_u4);
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)lds));
  constexpr int NOUT = GATED ? 128 : 256;
  const uint32_t nreal = uint32_t(*g.ntiles) * uint32_t((g.N + NOUT - 1) / NOUT);
  uint32_t lt;
  for (uint32_t pass = 0; mirrored_tile(blockIdx.x, gridDim.x, nreal, pass, lt); ++pass) {
    mx_ring_tile<GATED>(g, lt, lds, lds0);
    __syncthreads();  // the epilogue's LDS reads are done before the next tile's loads land
  }
#endif
}

template <bool GATED>
hipError_t run_mx_ring(const MxArgs& a, int64_t max_tiles, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  constexpr int NOUT = GATED ? 128 : 256;
  auto kern = mx_ring_kernel<GATED>;
  if (hipError_t e = allow_dynamic_lds((const void*)kern, kMxrLds); e != hipSuccess) return e;
  int64_t nblk = max_tiles * ((a.N + NOUT - 1) / NOUT);
  if (nblk <= 0) return hipSuccess;
  nblk = std::min<int64_t>((nblk + 7) / 8 * 8, (device_cus() + 7) / 8 * 8);  // the persistent grid
  return launch_kernel((const void*)kern, dim3{uint32_t(nblk)}, dim3{512}, size_t(kMxrLds), s, a, t0, t1);
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
  // routing cuts tiles at kTiledBM rows, within every form's reach
  static_assert(kTiledBM <= 256 && kTiledBM % 64 == 0, "tile table granularity");
  // FC2 (plain, bf16 output) writes 2 bytes per output against a short K:
  // in the deep form its stores get the persistent grid, to drain behind the
  // next tile (the 256-row form has no registers to spare for it)
  // the ring form needs K % 512 == 0 and 32-bit offsets into A, As and an
  // expert's weights; the deep form an even number (>= 4) of 128-wide stages
  constexpr int64_t kOff = int64_t(1) << 31;
  if (g.K % 512 == 0 && g.a_rows_n > 0 && g.a_rows_n * g.K < kOff && int64_t(g.N) * g.K / 2 < kOff)
    return g.gated ? run_mx_ring<true>(a, g.max_tiles, s, t0, t1) : run_mx_ring<false>(a, g.max_tiles, s, t0, t1);
  if (g.K % 256 == 0 && g.K >= 512)
    return g.gated ? run_mx<true, true, false>(a, g.max_tiles, s, t0, t1)
                   : run_mx<false, true, true>(a, g.max_tiles, s, t0, t1);
  return g.gated ? run_mx<true, false, false>(a, g.max_tiles, s, t0, t1)
                 : run_mx<false, false, false>(a, g.max_tiles, s, t0, t1);
}

}  // namespace lmoe
