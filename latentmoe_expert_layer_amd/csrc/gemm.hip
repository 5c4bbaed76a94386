// bf16 MFMA GEMMs of the LatentMoE layer (gfx950).
//
// All operands are "[rows, K]" with K contiguous (activations [M,K], weights
// [N,K] in the [out, in] layout), so C = A * B^T reads both operands along K.
//
//  * ring64_dense_kernel / ring64_grouped_kernel: the dense projections at
//    prefill (bf16 outputs) and the prefill-shaped grouped expert GEMMs (bf16
//    row-major weights), K a multiple of 64, streamed through LDS in 64-wide
//    stages by direct-to-LDS loads of whole 128-byte lines, a ring of half
//    stages.
//  * ring_dense_kernel: the same with 32-wide stages in a five-slot ring, for
//    K a multiple of 32 only.
//  * tiled_gemm_kernel: LDS double-buffered macro tiles for the dense
//    projections (latent down-proj fused with the shared experts' gate/up,
//    and the latent up-proj K-concatenated with the shared experts' down
//    proj) and for prefill-shaped grouped expert GEMMs (vLLM Kimi K3 post,
//    section 1: experts run in the latent; TokenSpeed Day-0 post,
//    "TensorRT-LLM Stable LatentMoE": FC1 with its gate as one gated GEMM,
//    then FC2).  Grouped tiles come from the device-side tile table, so no
//    per-expert row count ever reaches the host.
// (The decode-shaped weight-streaming grouped GEMM is in skinny.hip.)
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "router_core.h"

namespace lmoe {

// compute units of the current device (cached per device)
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

namespace {

constexpr int kBK = 64;          // K per LDS stage
constexpr int kLdsK = kBK + 8;   // padded LDS row (bf16): 144 B
static_assert(kBK == 64, "a tile-packed block holds 64 K columns: one stage");

// [E, N, K] row-major -> tile-packed (kernels.h), one 16-byte chunk (8
// elements along K) per thread, threads in packed order so the writes are
// contiguous; each read is 16 bytes of a row.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                          int64_t nchunks, int N, int K) {
  const int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x;  // packed chunk index
  if (q >= nchunks) return;
  const int kq = int(q % 8);                                   // chunk within the block's 64 columns
  const int64_t rest = q / 8;
  const int rin = int(rest % kPackRows);                       // row within the 128-row block
  const int64_t blk = rest / kPackRows;                        // (e, n/128, k/64) block
  const int kb = int(blk % (K / 64));
  const int64_t en = blk / (K / 64);                           // e * N/128 + n/128
  const int64_t row = en * kPackRows + rin;                    // e * N + n
  dst[q] = src[(row * K + int64_t(kb) * 64) / 8 + kq];
}

struct TiledArgs {
  int M, N;
  int nseg;
  GemmSeg seg[5];
  // grouped
  const int32_t* a_rows;
  int a_row_div;
  int64_t b_estride;
  const Tile* tiles;
  const int32_t* ntiles;
  uint16_t* C;
  float* Cf;  // F32OUT: fp32 output
  int64_t ldc;
};

// 32x32x16 bf16 MFMA: D(32x32 f32) = A(32x16) * B(16x32) + C.  Lane l feeds A
// row l%32 and B column l%32 with K elements 8*(l/32) .. +8; it receives
// column l%32 of rows 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Macro tile: 256 rows x 256 B rows (plain: 256 output columns; gated: 128
// gate + 128 up rows -> 128 output columns), K staged 64 at a time through a
// double-buffered LDS (2 x 72 KB).  8 waves = 2 per SIMD, so one wave's LDS
// reads and memory instructions overlap the other's MFMAs; WAVES_M x
// (8/WAVES_M) layout (2 x 4: wave tile 128 x 64; 4 x 2: 64 x 128, which lets a
// grouped tile with few rows idle whole waves).  Each wave keeps 8 32x32
// accumulators.  Main loop per 64-wide K stage, with one register set:
//   MFMAs on the first half of stage k | LDS writes of stage k+1 (loaded one
//   stage earlier) | global loads of stage k+2 | MFMAs on the second half |
//   barrier
// so every global load has a whole stage to arrive.  The K of all segments
// is one sequence of stages; rows of a partial tile and B rows past N are
// clamped (loaded but never stored).  F32OUT (plain GEMMs): fp32 results are
// stored straight from the accumulators (32 consecutive columns per half-wave
// and row), any N.
template <int NW, int WAVES_M, bool GATED, bool GROUPED, bool SWZ, bool F32OUT = false>
__global__ __launch_bounds__(NW * 64, 1) void tiled_gemm_kernel(TiledArgs g) {
  static_assert(!F32OUT || (!GATED && !GROUPED), "fp32 output is for plain dense GEMMs");
  constexpr int NTH = NW * 64;
  constexpr int BM = 256, BR = 256;                 // A rows, B rows per tile
  constexpr int NOUT = GATED ? 128 : 256;           // output columns per tile
  constexpr int WAVES_N = NW / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BR / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;         // 32x32 subtiles per wave
  constexpr int CPR = kBK / 8;                      // 16-byte chunks per row
  constexpr int A_CH = BM * CPR / NTH, B_CH = BR * CPR / NTH;
  static_assert(!GATED || FN % 2 == 0, "gated waves need matching gate and up subtiles");

  extern __shared__ uint4 lds_u4[];
  bf16_t* As = reinterpret_cast<bf16_t*>(lds_u4);  // [2][BM][kLdsK]
  bf16_t* Bs = As + 2 * BM * kLdsK;                 // [2][BR][kLdsK]

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int tiles_n = (g.N + NOUT - 1) / NOUT;
  // Grouped launches size the grid for an upper bound on the tile count; the
  // blocks past the device-side count exit at once, and the XCD-aware order
  // is taken over the real blocks only (over the whole padded grid it would
  // put every real tile on the first few XCDs and leave the others idle).
  uint32_t nreal = gridDim.x;
  if constexpr (GROUPED) {
    nreal = uint32_t(*g.ntiles) * uint32_t(tiles_n);
    if (blockIdx.x >= nreal) return;
  }
  const uint32_t lt = SWZ ? xcd_swizzle(blockIdx.x, nreal) : blockIdx.x;
  const int tn = int(lt % uint32_t(tiles_n));
  const int tm = int(lt / uint32_t(tiles_n));
  int expert = 0, row0, nrows;
  if constexpr (GROUPED) {
    const Tile tl = g.tiles[tm];
    expert = tl.expert;
    row0 = tl.row_start;
    nrows = tl.nrows;
  } else {
    row0 = tm * BM;
    nrows = min(BM, g.M - row0);
  }
  const int n0 = tn * NOUT;
  const bool active = wm * WM < nrows;  // this wave has rows to compute

  // B-tile row of this wave's n-subtile j (gated: first half gate, second up)
  auto brow = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (GATED) {
      return j < FN / 2 ? wn * (WN / 2) + j * 32 : BR / 2 + wn * (WN / 2) + (j - FN / 2) * 32;
    } else {
      return wn * WN + j * 32;
    }
  };

  // Load cursor.  Thread tid loads, for every stage, the 16-byte chunk kc8 of
  // A rows i*64 + tid/8 and B rows i*64 + tid/8 (i < A_CH, B_CH).  Gated
  // tiles take B rows 0..127 from the gate matrix and 128..255 from the up
  // matrix, so chunks i < B_CH/2 read B and the others B3.  The source
  // pointers are set once per segment and advance by kBK per stage; stages
  // are loaded strictly in order.
  constexpr int RPC = NTH / CPR;                    // rows per load chunk
  static_assert(!GATED || B_CH % 2 == 0, "gated B chunks split evenly between gate and up");
  int arow[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int r = i * RPC + tid / CPR;
    int src = row0 + min(r, nrows - 1);
    if constexpr (GROUPED) {
      if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
    }
    arow[i] = src;
  }
  const int kc8 = (tid % CPR) * 8;  // this thread's column chunk (same for all its rows)

  int nk = 0;
  for (int s = 0; s < g.nseg; ++s) nk += g.seg[s].K / kBK;

  const bf16_t* pa[A_CH];
  const bf16_t* pb[B_CH];
  int lseg = -1, lleft = 0;  // segment of the next stage to load, stages left in it
  auto set_seg = [&](int s) __attribute__((always_inline)) {
    const GemmSeg& sg = g.seg[s];
    lleft = sg.K / kBK;
    const int64_t be = int64_t(expert) * g.b_estride;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) pa[i] = sg.A + int64_t(arow[i]) * sg.lda + kc8;
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const bool up = GATED && i >= B_CH / 2;
      const int r = (up ? i - B_CH / 2 : i) * RPC + tid / CPR;
      pb[i] = (up ? sg.B3 : sg.B) + be + int64_t(min(n0 + r, g.N - 1)) * sg.ldb + kc8;
    }
  };

  uint4 ra[A_CH], rb[B_CH];
  auto gload = [&]() __attribute__((always_inline)) {
    while (lleft == 0) set_seg(++lseg);
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      if (i * RPC < nrows) ra[i] = ldg16(pa[i]);
      pa[i] += kBK;
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      rb[i] = ldg16(pb[i]);
      pb[i] += kBK;
    }
    --lleft;
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    bf16_t* An = As + buf * BM * kLdsK;
    bf16_t* Bn = Bs + buf * BR * kLdsK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NTH;
      if (i * RPC < nrows) *reinterpret_cast<uint4*>(&An[(c / CPR) * kLdsK + (c % CPR) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NTH;
      *reinterpret_cast<uint4*>(&Bn[(c / CPR) * kLdsK + (c % CPR) * 8]) = rb[i];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // FA = this wave's 32-row subtiles that hold rows < nrows; the others are
  // neither read from LDS nor multiplied (a tile's padding rows cost nothing
  // beyond their clamped A loads, which whole 64-row chunks also skip)
  auto mainloop = [&](auto fa_c) __attribute__((always_inline)) {
    constexpr int FA = decltype(fa_c)::value;
    auto compute = [&](int buf, int ks0, int ks1) __attribute__((always_inline)) {
      const bf16_t* Ab = As + buf * BM * kLdsK;
      const bf16_t* Bb = Bs + buf * BR * kLdsK;
#pragma unroll
      for (int ks = ks0; ks < ks1; ++ks) {
        const int kof = ks * 16 + (lane >> 5) * 8;
        bf16x8 af[FA > 0 ? FA : 1];
#pragma unroll
        for (int i = 0; i < FA; ++i)
          af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&Ab[(wm * WM + i * 32 + (lane & 31)) * kLdsK + kof]));
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (FA > 0) {
            const bf16x8 bf = as_bf16x8(*reinterpret_cast<const uint4*>(&Bb[(brow(j) + (lane & 31)) * kLdsK + kof]));
#pragma unroll
            for (int i = 0; i < FA; ++i) acc[i][j] = mfma_32x32x16(af[i], bf, acc[i][j]);
          }
        }
      }
    };
    gload();
    lstore(0);
    if (nk > 1) gload();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      compute(buf, 0, kBK / 32);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < nk) lstore(buf ^ 1);
      if (kt + 2 < nk) gload();
      __builtin_amdgcn_sched_barrier(0);
      compute(buf, kBK / 32, kBK / 16);
      __syncthreads();
    }
  };
  const int fa = active ? min(FM, (nrows - wm * WM + 31) / 32) : 0;
  static_assert(FM <= 8, "main loop specialisations cover up to 8 row subtiles per wave");
  switch (fa) {
    case 0: mainloop(std::integral_constant<int, 0>{}); break;
    case 1: mainloop(std::integral_constant<int, (FM >= 1 ? 1 : 0)>{}); break;
    case 2: mainloop(std::integral_constant<int, (FM >= 2 ? 2 : 0)>{}); break;
    case 3: mainloop(std::integral_constant<int, (FM >= 3 ? 3 : 0)>{}); break;
    case 4: mainloop(std::integral_constant<int, (FM >= 4 ? 4 : 0)>{}); break;
    case 5: mainloop(std::integral_constant<int, (FM >= 5 ? 5 : 0)>{}); break;
    case 6: mainloop(std::integral_constant<int, (FM >= 6 ? 6 : 0)>{}); break;
    case 7: mainloop(std::integral_constant<int, (FM >= 7 ? 7 : 0)>{}); break;
    default: mainloop(std::integral_constant<int, FM>{}); break;
  }

  if constexpr (F32OUT) {
    if (active) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        if (i < fa)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int row = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
              const int col = n0 + wn * WN + j * 32 + (lane & 31);
              if (row < nrows && col < g.N) g.Cf[(int64_t(row0) + row) * g.ldc + col] = acc[i][j][v];
            }
    }
    return;
  }
  // Epilogue: stage the bf16 tile in LDS, then 16-byte row-contiguous stores.
  constexpr int CLD = NOUT + 8;
  static_assert(BM * CLD <= 2 * (BM + BR) * kLdsK, "epilogue staging fits in the LDS buffers");
  bf16_t* Cs = As;
  if (active) {
    constexpr int JO = GATED ? FN / 2 : FN;       // output subtiles per wave
    constexpr int WO = GATED ? WN / 2 : WN;       // output columns per wave
#pragma unroll
    for (int i = 0; i < FM; ++i)
      if (i < fa)
#pragma unroll
      for (int j = 0; j < JO; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int col = wn * WO + j * 32 + (lane & 31);
          float x = acc[i][j][v];
          if constexpr (GATED) x = silu_mul(x, acc[i][j + FN / 2][v]);
          Cs[row * CLD + col] = f32_to_bf16(x);
        }
  }
  __syncthreads();
  constexpr int OCPR = NOUT / 8;
  for (int c = tid; c < BM * OCPR; c += NTH) {
    const int row = c / OCPR, cc = c % OCPR;
    if (row < nrows && n0 + cc * 8 < g.N) {
      *reinterpret_cast<uint4*>(g.C + (int64_t(row0) + row) * g.ldc + n0 + cc * 8) =
          *reinterpret_cast<const uint4*>(&Cs[row * CLD + cc * 8]);
    }
  }
}

template <int NW, int WAVES_M, bool GATED, bool GROUPED, bool SWZ, bool F32OUT = false>
hipError_t run_tiled(const TiledArgs& a, int64_t mtiles, hipStream_t s, hipEvent_t t0 = nullptr,
                     hipEvent_t t1 = nullptr) {
  constexpr int NOUT = GATED ? 128 : 256;
  const size_t lds = size_t(2) * (256 + 256) * kLdsK * sizeof(bf16_t);
  auto kern = tiled_gemm_kernel<NW, WAVES_M, GATED, GROUPED, SWZ, F32OUT>;
  if (hipError_t e = allow_dynamic_lds((const void*)kern, int(lds)); e != hipSuccess) return e;
  const int64_t nblk = mtiles * ((a.N + NOUT - 1) / NOUT);
  if (nblk <= 0) return hipSuccess;
  return launch_kernel((const void*)kern, dim3{uint32_t(nblk)}, dim3{uint32_t(NW * 64)}, lds, s, a, t0, t1);
}

// ---------------------------------------------- grouped, B two stages ahead ---
// Grouped expert GEMMs on tiles of at most kTiledBM = 192 rows (the routing's
// cut): 192 rows x 256 B rows (gated: 128 gate + 128 up), 8 waves as 2 x 4
// with 96 x 64 wave tiles, K staged 64 at a time through two LDS buffers as
// in tiled_gemm_kernel.  The smaller accumulator set (96 instead of 128
// registers per lane) pays for a second register set for B, so B is loaded
// two stages ahead of its LDS write (A, from a cached activation matrix, one
// stage ahead): at prefill ~146 rows per expert leave the kernel waiting on
// the weight stream, and the deeper B pipeline keeps twice as much of it in
// flight.  The results are bit-identical to tiled_gemm_kernel's (the same
// MFMAs in the same K order).  Needs K a multiple of 128 and >= 256.  It
// serves the two forms below; row-major bf16 weights go to
// ring64_grouped_kernel, whose direct-to-LDS stream is faster.
// PACKED: the weights are in the tile-packed layout (kernels.h): a stage's
// 128-row block of B is 16 KB of contiguous memory.
// W4: MXFP4 weights with bf16 activations (w4a16 at prefill size; TokenSpeed
// Day-0 post, "Gluon kernels on AMD GPUs > Stable LatentMoE": weights upcast
// in the K loop, activations in bf16): per stage each thread loads the 16 code
// bytes (32 e2m1 values, one MX block) of one B row's K half and its e8m0
// scale, two stages ahead, and writes them to LDS as 32 bf16 values (gfx950's
// scaled conversion: exact, an e2m1 value times a power of two); the MFMA loop
// is the bf16 one.
template <bool GATED, bool PACKED = false, bool W4 = false>
__global__ __launch_bounds__(512, 1) void grouped_tiled_kernel(GroupedGemm g) {
  constexpr int NTH = 512, BM = kTiledBM, BR = 256, NOUT = GATED ? 128 : 256;
  constexpr int WAVES_N = 4, WM = BM / 2, WN = BR / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32, CPR = kBK / 8, RPC = NTH / CPR;
  constexpr int A_CH = BM / RPC, B_CH = BR / RPC;
  static_assert(BM % RPC == 0 && WM % 32 == 0, "tile shape");
  static_assert(!GATED || B_CH % 2 == 0, "gated B chunks split evenly between gate and up");
  extern __shared__ uint4 lds_u4[];
  bf16_t* As = reinterpret_cast<bf16_t*>(lds_u4);  // [2][BM][kLdsK]
  bf16_t* Bs = As + 2 * BM * kLdsK;                 // [2][BR][kLdsK]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int tiles_n = (g.N + NOUT - 1) / NOUT;
  // grid sized for the host's upper bound; XCD-aware order over the real count
  const uint32_t nreal = uint32_t(*g.ntiles) * uint32_t(tiles_n);
  if (blockIdx.x >= nreal) return;
  const uint32_t lt = xcd_swizzle(blockIdx.x, nreal);
  const int tn = int(lt % uint32_t(tiles_n)), tm = int(lt / uint32_t(tiles_n));
  const Tile tl = g.tiles[tm];
  const int expert = tl.expert, row0 = tl.row_start, nrows = min(tl.nrows, BM);
  const int n0 = tn * NOUT;
  const bool active = wm * WM < nrows;
  auto brow = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (GATED) return j < FN / 2 ? wn * (WN / 2) + j * 32 : BR / 2 + wn * (WN / 2) + (j - FN / 2) * 32;
    else return wn * WN + j * 32;
  };
  // thread tid loads the 16-byte chunk kc8 of A rows i*64 + tid/8 and of B
  // rows i*64 + tid/8 (gated: chunks i < B_CH/2 from the gate matrix)
  const int kc8 = (tid % CPR) * 8;
  const bf16_t* pa[A_CH];
  const bf16_t* pb[B_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    int src = row0 + min(i * RPC + tid / CPR, nrows - 1);
    if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
    pa[i] = g.A + int64_t(src) * g.lda + kc8;
  }
  const int64_t be = int64_t(expert) * g.b_estride;
  if constexpr (!W4) {
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const bool up = GATED && i >= B_CH / 2;
      const int r = (up ? i - B_CH / 2 : i) * RPC + tid / CPR;
      const int n = min(n0 + r, g.N - 1);
      if constexpr (PACKED) {
        pb[i] = (up ? g.B3 : g.B) + be + int64_t(n / kPackRows) * g.K * kPackRows + (n % kPackRows) * kBK + kc8;
      } else {
        pb[i] = (up ? g.B3 : g.B) + be + int64_t(n) * g.ldb + kc8;
      }
    }
  }
  // W4: thread tid covers B tile row tid/2 (gated: rows >= 128 from B3), K
  // half tid%2 of each stage: code bytes qb (16 per stage half), scale qs
  const uint8_t* qb = nullptr;
  const uint8_t* qs = nullptr;
  if constexpr (W4) {
    const int r = tid >> 1, h = tid & 1;
    const bool up = GATED && r >= BR / 2;
    const int n = min(n0 + (up ? r - BR / 2 : r), g.N - 1);
    const int64_t row = int64_t(expert) * g.N + n;
    qb = reinterpret_cast<const uint8_t*>(up ? g.B3 : g.B) + row * (g.K / 2) + h * 16;
    qs = (up ? g.B3s : g.Bs) + row * (g.K / 32) + h;
  }
  // B advances one stage: kBK columns of a row, or one packed block
  constexpr int BSTEP = PACKED ? kPackRows * kBK : kBK;
  const int nk = g.K / kBK;
  uint4 ra[A_CH], rbx[W4 ? 1 : B_CH], rby[W4 ? 1 : B_CH];  // A one stage ahead; B stages alternate X / Y
  uint32_t sbx = 0, sby = 0;                                  // W4: the e8m0 scale codes of X / Y
  auto load_a = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      if (i * RPC < nrows) ra[i] = ldg16(pa[i]);
      pa[i] += kBK;
    }
  };
  // (separate code for the two B sets: a lambda taking either set by
  // reference would move them to memory)
  auto load_bx = [&]() __attribute__((always_inline)) {
    if constexpr (W4) {
      rbx[0] = *reinterpret_cast<const uint4*>(qb);
      sbx = *qs;
      qb += kBK / 2;
      qs += kBK / 32;
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        rbx[i] = ldg16(pb[i]);
        pb[i] += BSTEP;
      }
    }
  };
  auto load_by = [&]() __attribute__((always_inline)) {
    if constexpr (W4) {
      rby[0] = *reinterpret_cast<const uint4*>(qb);
      sby = *qs;
      qb += kBK / 2;
      qs += kBK / 32;
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        rby[i] = ldg16(pb[i]);
        pb[i] += BSTEP;
      }
    }
  };
  // W4: 32 e2m1 codes and their scale -> 32 bf16 at B row tid/2, K half tid%2
  auto store_w4 = [&](bf16_t* Bn, const uint4& q, uint32_t sc) __attribute__((always_inline)) {
    const float f = e8m0_multiplier(sc);
    bf16_t* dst = &Bn[(tid >> 1) * kLdsK + (tid & 1) * 32];
    *reinterpret_cast<bf16x8*>(dst + 0) = fp4x8_to_bf16(q.x, f);
    *reinterpret_cast<bf16x8*>(dst + 8) = fp4x8_to_bf16(q.y, f);
    *reinterpret_cast<bf16x8*>(dst + 16) = fp4x8_to_bf16(q.z, f);
    *reinterpret_cast<bf16x8*>(dst + 24) = fp4x8_to_bf16(q.w, f);
  };
  auto store_a = [&](int buf) __attribute__((always_inline)) {
    bf16_t* An = As + buf * BM * kLdsK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NTH;
      if (i * RPC < nrows) *reinterpret_cast<uint4*>(&An[(c / CPR) * kLdsK + (c % CPR) * 8]) = ra[i];
    }
  };
  auto store_bx = [&](int buf) __attribute__((always_inline)) {
    bf16_t* Bn = Bs + buf * BR * kLdsK;
    if constexpr (W4) {
      store_w4(Bn, rbx[0], sbx);
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * NTH;
        *reinterpret_cast<uint4*>(&Bn[(c / CPR) * kLdsK + (c % CPR) * 8]) = rbx[i];
      }
    }
  };
  auto store_by = [&](int buf) __attribute__((always_inline)) {
    bf16_t* Bn = Bs + buf * BR * kLdsK;
    if constexpr (W4) {
      store_w4(Bn, rby[0], sby);
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * NTH;
        *reinterpret_cast<uint4*>(&Bn[(c / CPR) * kLdsK + (c % CPR) * 8]) = rby[i];
      }
    }
  };
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  auto mainloop = [&](auto fa_c) __attribute__((always_inline)) {
    constexpr int FA = decltype(fa_c)::value;
    auto compute = [&](int buf, int ks0, int ks1) __attribute__((always_inline)) {
      const bf16_t* Ab = As + buf * BM * kLdsK;
      const bf16_t* Bb = Bs + buf * BR * kLdsK;
#pragma unroll
      for (int ks = ks0; ks < ks1; ++ks) {
        const int kof = ks * 16 + (lane >> 5) * 8;
        bf16x8 af[FA > 0 ? FA : 1];
#pragma unroll
        for (int i = 0; i < FA; ++i)
          af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&Ab[(wm * WM + i * 32 + (lane & 31)) * kLdsK + kof]));
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (FA > 0) {
            const bf16x8 bf = as_bf16x8(*reinterpret_cast<const uint4*>(&Bb[(brow(j) + (lane & 31)) * kLdsK + kof]));
#pragma unroll
            for (int i = 0; i < FA; ++i) acc[i][j] = mfma_32x32x16(af[i], bf, acc[i][j]);
          }
        }
      }
    };
    // step k: MFMAs on stage k (buffer k&1) around the LDS writes of stage
    // k+1 (A from ra, B from set X for even k, Y for odd k) and the loads of
    // A(k+2) and B(k+3) into the set just written out; which writes and loads
    // a step has is fixed per call site, so no load sits behind a branch
    auto step = [&](int buf, bool y, bool st, bool la, bool lb) __attribute__((always_inline)) {
      compute(buf, 0, kBK / 32);
      __builtin_amdgcn_sched_barrier(0);
      if (st) {
        store_a(buf ^ 1);
        if (y) store_by(buf ^ 1);
        else store_bx(buf ^ 1);
      }
      if (la) load_a();
      if (lb) {
        if (y) load_by();
        else load_bx();
      }
      __builtin_amdgcn_sched_barrier(0);
      compute(buf, kBK / 32, kBK / 16);
      __syncthreads();
    };
    load_a();
    load_bx();  // stage 0
    store_a(0);
    store_bx(0);
    load_a();
    load_bx();  // stage 1
    load_by();  // B of stage 2
    __syncthreads();
    for (int kt = 0; kt < nk - 4; kt += 2) {
      step(0, false, true, true, true);
      step(1, true, true, true, true);
    }
    step(0, false, true, true, true);    // k = nk-4: loads A(nk-2), B(nk-1)
    step(1, true, true, true, false);    // k = nk-3: loads A(nk-1)
    step(0, false, true, false, false);  // k = nk-2: writes stage nk-1
    step(1, true, false, false, false);  // k = nk-1
  };
  const int fa = active ? min(FM, (nrows - wm * WM + 31) / 32) : 0;
  static_assert(FM == 3, "main loop specialisations cover up to 3 row subtiles per wave");
  switch (fa) {
    case 0: mainloop(std::integral_constant<int, 0>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 3: mainloop(std::integral_constant<int, 3>{}); break;
    default: mainloop(std::integral_constant<int, FM>{}); break;  // (unreached; in this form the
  }                                                                // register allocator does not spill)

  // Epilogue: stage the bf16 tile in LDS, then 16-byte row-contiguous stores.
  constexpr int CLD = NOUT + 8;
  static_assert(BM * CLD <= 2 * (BM + BR) * kLdsK, "epilogue staging fits in the LDS buffers");
  bf16_t* Cs = As;
  if (active) {
    constexpr int JO = GATED ? FN / 2 : FN, WO = GATED ? WN / 2 : WN;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      if (i < fa)
#pragma unroll
        for (int j = 0; j < JO; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            const int col = wn * WO + j * 32 + (lane & 31);
            float x = acc[i][j][v];
            if constexpr (GATED) x = silu_mul(x, acc[i][j + FN / 2][v]);
            Cs[row * CLD + col] = f32_to_bf16(x);
          }
  }
  __syncthreads();
  constexpr int OCPR = NOUT / 8;
  for (int c = tid; c < BM * OCPR; c += NTH) {
    const int row = c / OCPR, cc = c % OCPR;
    if (row < nrows && n0 + cc * 8 < g.N) {
      *reinterpret_cast<uint4*>(g.C + (int64_t(row0) + row) * g.ldc + n0 + cc * 8) =
          *reinterpret_cast<const uint4*>(&Cs[row * CLD + cc * 8]);
    }
  }
}

template <bool GATED, bool PACKED, bool W4 = false>
hipError_t run_grouped(const GroupedGemm& g, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  constexpr int NOUT = GATED ? 128 : 256;
  const size_t lds = size_t(2) * (kTiledBM + 256) * kLdsK * sizeof(bf16_t);
  auto kern = grouped_tiled_kernel<GATED, PACKED, W4>;
  if (hipError_t e = allow_dynamic_lds((const void*)kern, int(lds)); e != hipSuccess) return e;
  const int64_t nblk = g.max_tiles * ((g.N + NOUT - 1) / NOUT);
  if (nblk <= 0) return hipSuccess;
  return launch_kernel((const void*)kern, dim3{uint32_t(nblk)}, dim3{512u}, lds, s, g, t0, t1);
}

// ------------------------------------------------------- small-M dense split-K ---
// Dense GEMMs with few rows (decode-sized batches): one 16-row x 32-column
// output tile per workgroup; the 4 waves split the (segment-concatenated) K
// into contiguous quarters, so each wave has a single round of loads in
// flight, and the partial sums are added in LDS in wave order
// (deterministic).  Up to two independent sub-GEMMs (e.g. the latent
// down-projection and the shared experts' gated gate/up projection, which
// read the same x) share one launch.  With an fp32 output (Cf), N may be
// ragged: B rows past N are clamped (loaded, never stored).
struct SplitKPart {
  int N;
  int nseg;
  GemmSeg seg[5];
  int gated;
  uint16_t* C;
  float* Cf;
  int64_t ldc;
};
struct SplitKArgs {
  int M;
  int nparts;
  int nblk0;
  SplitKPart part[2];
};

constexpr int kSkNS = 2;     // 16-column subtiles per wave
constexpr int kSkBatch = 4;  // 32-wide K steps whose loads are issued together

// One wave's share [st0, st1) of the K steps (32 wide, numbered across the
// concatenated segments).  Segment parameters are read once per segment; the
// steps of a batch are loaded together (a short last batch re-loads its last
// step, whose copies are not used).
template <bool GATED>
__device__ __forceinline__ void splitk_accumulate(const SplitKPart& P, int64_t arow, int ncol, int kof, int st0,
                                                  int st1, f32x4 (&acc)[kSkNS], f32x4 (&acc3)[kSkNS]) {
  int brow[kSkNS];
#pragma unroll
  for (int j = 0; j < kSkNS; ++j) brow[j] = min(ncol + 16 * j, P.N - 1);
  int base = 0;
  for (int s = 0; s < P.nseg; ++s) {
    const GemmSeg sg = P.seg[s];
    const int ns = sg.K / 32;
    const int lo = max(st0, base), hi = min(st1, base + ns);
    const bf16_t* ap = sg.A + arow * sg.lda + kof;
    const bf16_t* bp = sg.B + kof;
    const bf16_t* b3p = GATED ? sg.B3 + kof : nullptr;
    for (int c0 = lo; c0 < hi; c0 += kSkBatch) {
      const int cnt = min(kSkBatch, hi - c0);
      uint4 a[kSkBatch], b[kSkNS][kSkBatch], b3[kSkNS][GATED ? kSkBatch : 1];
#pragma unroll
      for (int u = 0; u < kSkBatch; ++u) {
        const int k = (c0 + min(u, cnt - 1) - base) * 32;
        a[u] = ldg16(ap + k);
#pragma unroll
        for (int j = 0; j < kSkNS; ++j) {
          b[j][u] = ldg16(bp + int64_t(brow[j]) * sg.ldb + k);
          if constexpr (GATED) b3[j][u] = ldg16(b3p + int64_t(brow[j]) * sg.ldb + k);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kSkBatch; ++u) {
        if (u < cnt) {
#pragma unroll
          for (int j = 0; j < kSkNS; ++j) {
            acc[j] = mfma_16x16x32(as_bf16x8(a[u]), as_bf16x8(b[j][u]), acc[j]);
            if constexpr (GATED) acc3[j] = mfma_16x16x32(as_bf16x8(a[u]), as_bf16x8(b3[j][u]), acc3[j]);
          }
        }
      }
    }
    base += ns;
  }
}

// Split-K workgroup `blk` of the launch (256 threads; every thread reaches
// the one barrier).
__device__ __forceinline__ void splitk_block(const SplitKArgs& g, int blk) {
  __shared__ f32x4 red[3][2][kSkNS][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int pi = (g.nparts > 1 && blk >= g.nblk0) ? 1 : 0;
  const int bb = blk - (pi ? g.nblk0 : 0);
  const SplitKPart& P = g.part[pi];
  const int tiles_n = (P.N + 16 * kSkNS - 1) / (16 * kSkNS);
  const int tm = bb / tiles_n, tn = bb % tiles_n;
  const int row0 = tm * 16, nrows = min(16, g.M - row0);
  const int64_t arow = row0 + min(lane & 15, nrows - 1);
  const int kof = (lane >> 4) * 8;
  const int ncol = tn * 16 * kSkNS + (lane & 15);
  const bool gated = P.gated != 0;

  int total = 0;
  for (int s = 0; s < P.nseg; ++s) total += P.seg[s].K / 32;
  const int per = (total + 3) / 4;
  const int st0 = wid * per, st1 = min(total, st0 + per);

  f32x4 acc[kSkNS], acc3[kSkNS];
#pragma unroll
  for (int j = 0; j < kSkNS; ++j) {
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc3[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (gated) splitk_accumulate<true>(P, arow, ncol, kof, st0, st1, acc, acc3);
  else splitk_accumulate<false>(P, arow, ncol, kof, st0, st1, acc, acc3);

  if (wid > 0) {
#pragma unroll
    for (int j = 0; j < kSkNS; ++j) {
      red[wid - 1][0][j][lane] = acc[j];
      red[wid - 1][1][j][lane] = acc3[j];
    }
  }
  __syncthreads();
  if (wid == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int j = 0; j < kSkNS; ++j) {
        acc[j] += red[w][0][j][lane];
        acc3[j] += red[w][1][j][lane];
      }
#pragma unroll
    for (int j = 0; j < kSkNS; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = (lane >> 4) * 4 + r;
        if (P.Cf) {
          if (row < nrows && ncol + 16 * j < P.N) P.Cf[(int64_t(row0) + row) * P.ldc + ncol + 16 * j] = acc[j][r];
        } else if (row < nrows) {
          float v = acc[j][r];
          if (gated) v = silu_mul(v, acc3[j][r]);
          P.C[(int64_t(row0) + row) * P.ldc + ncol + 16 * j] = f32_to_bf16(v);
        }
      }
  }
}

__global__ __launch_bounds__(256) void splitk_dense_kernel(SplitKArgs g) { splitk_block(g, int(blockIdx.x)); }

// Router top-k of T tokens (4 per workgroup, one per wave) in the same launch
// as the split-K GEMMs, which do not read its output: workgroups [0, nrb)
// route, the rest are the split-K grid.
template <int VPL>
__global__ __launch_bounds__(256) void splitk_router_kernel(SplitKArgs g, FrontRoute r, int nrb) {
  if (int(blockIdx.x) < nrb) {
    __shared__ uint64_t cbuf[4][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t t = int64_t(blockIdx.x) * 4 + wv;
    if (t < r.T) route_token<VPL>(r.logits, t, r.E, r.k, lane, cbuf[wv], r.ids, r.w);
    return;
  }
  splitk_block(g, int(blockIdx.x) - nrb);
}

// ---------------------------------------------------- dense, five-slot ring ---
// Dense projections on 256 x 256 output tiles (gated: 128 gate + 128 up B
// rows), 8 waves as 2 x 4 with 128 x 64 wave tiles, as tiled_gemm_kernel, but
// K goes through LDS in 32-wide stages that global_load_lds_dwordx4 writes
// straight into a ring of five slots (no register staging; three stages in
// flight behind the one being computed).  One barrier per stage: each wave
// first waits for its own loads of stage s+1, so after the barrier stage s+1
// is visible to all and the slot of stage s-1 is free for stage s+4.  Inside
// a stage the second 16-K half's fragments are read while the first half's
// MFMAs run, and the next stage's first-half fragments while the second
// half's run.  A slot row is 64 B (32 bf16); its four 16-byte chunks sit
// XOR-swizzled by (row / 4) % 4, so the 16 lanes of each ds_read_b128 phase
// (16 consecutive rows, one chunk) hit 16 distinct 4-bank groups.  The MFMAs
// and their K order are tiled_gemm_kernel's: the results are bit-identical.
constexpr int kRingBK = 32;                 // K per stage
constexpr int kRingRow = kRingBK * 2;       // bytes per slot row
constexpr int kRingSlots = 5;
constexpr int kRingStage = (256 + 256) * kRingRow;
constexpr int kRingLds = kRingSlots * kRingStage;  // 160 KiB: all of a CU's LDS

template <bool GATED>
__global__ __launch_bounds__(512, 1) void ring_dense_kernel(DenseGemm g) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = 256, BR = 256, NOUT = GATED ? 128 : 256, WAVES_N = 4, WM = BM / 2, WN = 64;
  constexpr int FM = WM / 32, FN = 2, NS = kRingSlots, BK = kRingBK, ROWB = kRingRow;
  constexpr int A_BYTES = BM * ROWB, STAGE = kRingStage;
  constexpr int L = 4;  // 1 KB load instructions per wave and stage: 2 of A, 2 of B
  extern __shared__ uint4 lds_u4[];
  char* lds = reinterpret_cast<char*>(lds_u4);
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)lds));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int tiles_n = (g.N + NOUT - 1) / NOUT;
  const uint32_t lt = xcd_swizzle(blockIdx.x, gridDim.x);
  const int tn = int(lt % uint32_t(tiles_n)), tm = int(lt / uint32_t(tiles_n));
  const int row0 = tm * BM, nrows = min(BM, g.M - row0), n0 = tn * NOUT;
  // wave w loads A and B rows 16w .. 16w+15 and 16(w+8) .. +15 of each stage;
  // lane l: row l/4 of those 16, slot chunk l%4, global chunk (l%4)^((l/16)%4)
  const int lrow = lane >> 2, lchunk = (lane & 3) ^ ((lane >> 4) & 3);
  int a_row[2], b_row[2];
  bool b_up[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wid + 8 * i) * 16 + lrow;
    a_row[i] = row0 + min(r, nrows - 1);
    if constexpr (GATED) {
      b_up[i] = r >= BR / 2;
      b_row[i] = min(n0 + (b_up[i] ? r - BR / 2 : r), g.N - 1);
    } else {
      b_up[i] = false;
      b_row[i] = min(n0 + r, g.N - 1);
    }
  }
  const bf16_t* pa[2];
  const bf16_t* pb[2];
  auto set_seg = [&](const GemmSeg& sg) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      pa[i] = reinterpret_cast<const bf16_t*>(sg.A) + int64_t(a_row[i]) * sg.lda + lchunk * 8;
      pb[i] = reinterpret_cast<const bf16_t*>(b_up[i] ? sg.B3 : sg.B) + int64_t(b_row[i]) * sg.ldb + lchunk * 8;
    }
  };
  set_seg(g.seg[0]);
  int nk = 0;
#pragma unroll
  for (int q = 0; q < 5; ++q)
    if (q < g.nseg) nk += g.seg[q].K / BK;
  int ls = 0, lk = g.seg[0].K / BK;  // loader: segment, stages left in it
  const int fr = lane & 31, sw = (fr >> 2) & 3;
  const int off0 = fr * ROWB + (((lane >> 5) + 0) ^ sw) * 16;  // K 0..15 of a stage
  const int off1 = fr * ROWB + (((lane >> 5) + 2) ^ sw) * 16;  // K 16..31
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

  auto mainloop = [&](auto fa_c) __attribute__((always_inline)) {
    constexpr int FA = decltype(fa_c)::value;
    bf16x8 a0[FA > 0 ? FA : 1], b0[FN], a1[FA > 0 ? FA : 1], b1[FN];
    auto issue = [&](int stage) __attribute__((always_inline)) {
      const uint32_t sb = uint32_t(__builtin_amdgcn_readfirstlane(int(lds0 + (stage % NS) * STAGE)));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        g2lds16(pa[i], sb + (wid + 8 * i) * 1024);
        g2lds16(pb[i], sb + A_BYTES + (wid + 8 * i) * 1024);
        pa[i] += BK;
        pb[i] += BK;
      }
      if (--lk == 0 && ls + 1 < g.nseg) {
        ++ls;
        switch (ls) {  // (static indices: the arguments stay in the kernarg segment)
          case 1: set_seg(g.seg[1]); lk = g.seg[1].K / BK; break;
          case 2: set_seg(g.seg[2]); lk = g.seg[2].K / BK; break;
          case 3: set_seg(g.seg[3]); lk = g.seg[3].K / BK; break;
          default: set_seg(g.seg[4]); lk = g.seg[4].K / BK; break;
        }
      }
    };
    auto rd = [&](int stage, int off, bf16x8* af, bf16x8* bf) __attribute__((always_inline)) {
      const char* sb = lds + (stage % NS) * STAGE;
#pragma unroll
      for (int i = 0; i < FA; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(sb + (wm * WM + i * 32) * ROWB + off));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[j] = as_bf16x8(*reinterpret_cast<const uint4*>(sb + A_BYTES + brow(j) * ROWB + off));
    };
    auto mm = [&](bf16x8* af, bf16x8* bf) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FA; ++i) acc[i][j] = mfma_32x32x16(af[i], bf[j], acc[i][j]);
    };
    // stage s: W = stages allowed in flight behind stage s+1 at the top wait
    // (-1: there is no stage s+1); ISSUE: load stage s+NS-1
    auto step = [&](int s, auto w_c, auto issue_c) __attribute__((always_inline)) {
      constexpr int W = decltype(w_c)::value;
      constexpr bool ISSUE = decltype(issue_c)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (W >= 0) {
        wait_vmcnt<W * L>();
        __builtin_amdgcn_s_barrier();
      }
      if constexpr (ISSUE) issue(s + NS - 1);
      if constexpr (FA > 0) {
        rd(s, off1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        mm(a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (W >= 0) rd(s + 1, off0, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mm(a1, b1);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int p = 0; p < NS - 1; ++p) issue(p);
    wait_vmcnt<(NS - 2) * L>();
    __builtin_amdgcn_s_barrier();
    if constexpr (FA > 0) rd(0, off0, a0, b0);
    int s = 0;
    for (; s <= nk - NS; ++s) step(s, std::integral_constant<int, NS - 3>{}, std::true_type{});
    static_assert(NS == 5, "the tail below drains a five-slot ring");
    step(s, std::integral_constant<int, 2>{}, std::false_type{});
    step(s + 1, std::integral_constant<int, 1>{}, std::false_type{});
    step(s + 2, std::integral_constant<int, 0>{}, std::false_type{});
    step(s + 3, std::integral_constant<int, -1>{}, std::false_type{});
  };
  const int fa = max(0, min(FM, (nrows - wm * WM + 31) / 32));
  switch (fa) {
    case 0: mainloop(std::integral_constant<int, 0>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 3: mainloop(std::integral_constant<int, 3>{}); break;
    default: mainloop(std::integral_constant<int, 4>{}); break;
  }
  __syncthreads();
  // epilogue: stage the bf16 tile in LDS, then 16-byte row-contiguous stores
  constexpr int CLD = NOUT + 8;
  static_assert(BM * CLD * 2 <= kRingLds, "epilogue staging fits in the ring");
  bf16_t* Cs = reinterpret_cast<bf16_t*>(lds);
  constexpr int JO = GATED ? 1 : FN, WO = GATED ? 32 : WN;
#pragma unroll
  for (int i = 0; i < FM; ++i)
    if (i < fa)
#pragma unroll
      for (int j = 0; j < JO; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int col = wn * WO + j * 32 + (lane & 31);
          float x = acc[i][j][v];
          if constexpr (GATED) x = silu_mul(x, acc[i][1][v]);
          Cs[row * CLD + col] = f32_to_bf16(x);
        }
  __syncthreads();
  constexpr int OCPR = NOUT / 8;
  for (int c = tid; c < BM * OCPR; c += 512) {
    const int row = c / OCPR, cc = c % OCPR;
    if (row < nrows && n0 + cc * 8 < g.N)
      *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(g.C) + (int64_t(row0) + row) * g.ldc + n0 + cc * 8) =
          *reinterpret_cast<const uint4*>(&Cs[row * CLD + cc * 8]);
  }
#endif
}

// ------------------------------------------ 64-wide stages, half-stage ring ---
// The dense projections and the prefill-shaped grouped expert GEMMs on 8
// waves as 2 x 4 (wave tiles BM/2 x 64 of 32x32x16 bf16 MFMAs; B tiles of 256
// rows, gated: 128 gate + 128 up), with K going through LDS in 64-wide stages:
// a row of a stage is 128 bytes, so each direct-to-LDS instruction (8 rows x
// 128 B) asks L2 for whole 128-byte lines.  With 32-wide stages every request
// is half a line, and the same loads reach only ~13 TB/s into LDS across the
// chip against ~21 TB/s for whole lines.  A 64-wide stage takes up to 64 KB,
// so the 160 KB of LDS is a ring of five 32 KB entries, each holding one
// operand's half of a stage: B (the weights, issued two stages ahead: for the
// grouped GEMMs they stream from HBM, and the dense projections gain 1-2% too)
// sits in entry 2s mod 5, A (one stage ahead) in entry 2s+1 mod 5.  One
// barrier per stage,
// before its last 16-K step: each wave first waits for its LDS reads
// (lgkmcnt) and for its loads of stage s+1, so after the barrier stage s+1 is
// visible and both entries of stage s are free.  Under that last step's
// MFMAs go, in this order, the loads of A(s+2) into stage s's B entry, the
// reads of stage s+1's first fragments, and the loads of B(s+3) into stage
// s's A entry: 1.5 stages are in flight behind the one computed.  The waits
// count on that order (vmcnt is in order: A(s+1) has arrived once at most
// B(s+2)'s loads remain).  Rows are 128 B with the eight
// 16-byte chunks XOR-swizzled by (row / 2) mod 8, so the 16 lanes of each
// ds_read_b128 phase (16 consecutive rows, one chunk) hit 16 distinct 4-bank
// groups.  The MFMAs and their K order are tiled_gemm_kernel's: the results
// are bit-identical.  Needs K a multiple of 64 in every segment and at least
// 3 stages in all.
constexpr int kR64BK = 64;                // K per stage
constexpr int kR64Row = kR64BK * 2;       // bytes per LDS row
constexpr int kR64Ent = 256 * kR64Row;    // one operand's half of a stage: 32 KB
constexpr int kR64Lds = 5 * kR64Ent;      // 160 KiB: all of a CU's LDS

// Lane l of wave w loads row l/8 of the 8-row groups w, w+8, ... of a half
// stage, into chunk l%8 of its LDS row, from global chunk (l%8) ^ ((row/2)%8);
// row/2 mod 8 = 4 (group mod 2) + (l/8)/2, and a group's parity is its wave's.
__device__ __forceinline__ int ring64_gchunk(int wid, int lane) {
  return (lane & 7) ^ ((((wid & 1) << 2) + ((lane >> 3) >> 1)) & 7);
}

// Epilogue of a 64-wide-ring tile (BM rows x 256 B rows on 8 waves as 2 x 4,
// this wave's fa 32-row subtiles from tile row r0 in acc, as wave_rows
// splits the tile); the LDS is free on entry.  Gated: SwiGLU of each
// gate subtile with its up subtile.  Rows row0 .. row0+nrows-1 of C, columns
// n0 .. (below N), are written; NT: with nontemporal stores.
template <bool GATED, int BM, bool NT>
__device__ __forceinline__ void ring64_store(char* lds, const f32x16 (&acc)[BM / 64][2], int fa, int r0, int wn,
                                             int lane, int tid, uint16_t* C, int64_t ldc, int64_t row0, int nrows,
                                             int n0, int N, uint8_t* Cq = nullptr, uint8_t* Cqs = nullptr) {
  constexpr int NTH = 512, NOUT = GATED ? 128 : 256, WN = 64, FM = BM / 64, FN = 2;
  // epilogue: stage the bf16 tile in LDS, then 16-byte row-contiguous stores
  constexpr int CLD = NOUT + 8;
  static_assert(BM * CLD * 2 <= kR64Lds, "epilogue staging fits in the ring");
  bf16_t* Cs = reinterpret_cast<bf16_t*>(lds);
  constexpr int JO = GATED ? 1 : FN, WO = GATED ? 32 : WN;
#pragma unroll
  for (int i = 0; i < FM; ++i)
    if (i < fa)
#pragma unroll
      for (int j = 0; j < JO; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = r0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int col = wn * WO + j * 32 + (lane & 31);
          float x = acc[i][j][v];
          if constexpr (GATED) x = silu_mul(x, acc[i][1][v]);
          Cs[row * CLD + col] = f32_to_bf16(x);
        }
  __syncthreads();
  constexpr int OCPR = NOUT / 8;
  for (int c = tid; c < BM * OCPR; c += NTH) {
    const int row = c / OCPR, cc = c % OCPR;
    if (row < nrows && n0 + cc * 8 < N)
    {
      const uint4 val = *reinterpret_cast<const uint4*>(&Cs[row * CLD + cc * 8]);
      uint4* dst = reinterpret_cast<uint4*>(C + (row0 + row) * ldc + n0 + cc * 8);
      if constexpr (NT) {
        __builtin_nontemporal_store(val.x, &dst->x);
        __builtin_nontemporal_store(val.y, &dst->y);
        __builtin_nontemporal_store(val.z, &dst->z);
        __builtin_nontemporal_store(val.w, &dst->w);
      } else {
        *dst = val;
      }
    }
  }
  if (!GATED && Cq) {
    // the MXFP8 copy: one thread per (row, 32-column block) of the staged tile
    constexpr int BPR = NOUT / 32;
    for (int c = tid; c < BM * BPR; c += NTH) {
      const int row = c / BPR, b = c % BPR, col = n0 + b * 32;
      if (row < nrows && col < N) {
        uint4 raw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = *reinterpret_cast<const uint4*>(&Cs[row * CLD + b * 32 + i * 8]);
        uint4 q[2];
        const int64_t r = row0 + row;
        Cqs[r * (ldc / 32) + col / 32] = quant_block32(raw, q);
        uint4* dst = reinterpret_cast<uint4*>(Cq + r * ldc + col);
        dst[0] = q[0];
        dst[1] = q[1];
      }
    }
  }
}

// Main loop and epilogue of a 64-wide-ring tile.  pa / pb: this lane's
// global addresses of its A / B rows at stage 0 (LA = BM/64 and 4 rows);
// next_a / next_b advance them by one stage (and may switch segments).  The
// tile's rows row0 .. row0+nrows-1 of C, columns n0 .. of N, are written;
// NT: with nontemporal stores.  B_ONCE: B is read by this tile alone (an
// expert's only row tile), so its loads carry the nontemporal hint, which
// leaves L2 to the A rows that every column tile re-reads.
template <bool GATED, int BM, bool NT, bool B_ONCE, class NextA, class NextB>
__device__ __forceinline__ void ring64_tile(char* lds, uint32_t lds0, int wid, int lane, int tid, int nk, int nrows,
                                            const bf16_t* (&pa)[BM / 64], const bf16_t* (&pb)[4], NextA next_a,
                                            NextB next_b, uint16_t* C, int64_t ldc, int64_t row0, int n0, int N,
                                            uint8_t* Cq = nullptr, uint8_t* Cqs = nullptr) {
  constexpr int NW = 8, WAVES_N = 4;
  constexpr int BR = 256, WM = BM / 2, WN = 64;
  constexpr int FM = WM / 32, FN = WN / 32, ROWB = kR64Row, ENT = kR64Ent;
  constexpr int LA = BM / 8 / NW, LB = BR / 8 / NW;  // 1 KB loads per wave and A / B half stage
  static_assert(BM % (8 * NW) == 0 && BM * ROWB <= ENT && FM >= 1 && FM <= 4, "tile rows");
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const WaveRows wr = wave_rows(wm, nrows, FM);  // this wave row's first tile row and subtiles
  const int fr = lane & 31, fsw = (fr >> 1) & 7, fh = lane >> 5;  // fragment row, its swizzle, K half
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
  auto ent = [&](int e) __attribute__((always_inline)) -> uint32_t {
    return uint32_t(__builtin_amdgcn_readfirstlane(int(lds0 + e * ENT)));
  };
  // (the LDS address goes to m0, so it must be wave-uniform: readfirstlane)
  auto issue_a = [&](uint32_t eb, int q) __attribute__((always_inline)) {
    g2lds16(pa[q], uint32_t(__builtin_amdgcn_readfirstlane(int(eb + (wid + NW * q) * 1024))));
  };
  auto issue_b = [&](uint32_t eb, int q) __attribute__((always_inline)) {
    g2lds16<B_ONCE>(pb[q], uint32_t(__builtin_amdgcn_readfirstlane(int(eb + (wid + NW * q) * 1024))));
  };

  auto mainloop = [&](auto fa_c) __attribute__((always_inline)) {
    constexpr int FA = decltype(fa_c)::value;
    bf16x8 af[2][FA > 0 ? FA : 1], bfr[2][FN];
    // fragment q (q < FA: A, then the FN of B) of the 16-K step t of the
    // stage whose B is in entry eb and A in ea
    auto rd = [&](int eb, int ea, int t, int q, int buf) __attribute__((always_inline)) {
      const int off = fr * ROWB + (((2 * t + fh) ^ fsw) << 4);
      if (q < FA) af[buf][q] = as_bf16x8(*reinterpret_cast<const uint4*>(lds + ea * ENT + (wr.r0 + q * 32) * ROWB + off));
      else bfr[buf][q - FA] = as_bf16x8(*reinterpret_cast<const uint4*>(lds + eb * ENT + brow(q - FA) * ROWB + off));
    };
    // a 16-K step's MFMAs on fragment set buf, with the side items 0 .. nside-1
    // spread over them in order: MFMA m is followed by items c m .. c m + c - 1,
    // c = ceil(nside / NM), NM being the MFMA count (all items at once if 0).
    // The order matters: the vmcnt waits count on each wave's loads of
    // A(s+2) leaving before those of B(s+3).
    auto mm = [&](int buf, int nside, auto side) __attribute__((always_inline)) {
      constexpr int NM = FA * FN;
      const int c = NM > 0 ? (nside + NM - 1) / NM : 0;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FA; ++i) {
          acc[i][j] = mfma_32x32x16(af[buf][i], bfr[buf][j], acc[i][j]);
          const int m = j * FA + i;
#pragma unroll
          for (int k = 0; k < 16; ++k)
            if (k >= m * c && k < m * c + c && k < nside) side(k);
          __builtin_amdgcn_sched_barrier(0);
        }
      if constexpr (NM == 0) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (k < nside) side(k);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // stage s: B in e0 = 2s mod 5, A in e0+1; stage s+1 in e0+2, e0+3.  W: B
    // half stages issued after A(s+1) (the wait before the barrier; -1: there
    // is no stage s+1); IA / IB: issue A(s+2) into e0 / B(s+3) into e0+1
    int e0 = 0;
    auto step = [&](auto w_c, auto ia_c, auto ib_c) __attribute__((always_inline)) {
      constexpr int W = decltype(w_c)::value;
      constexpr bool IA = decltype(ia_c)::value, IB = decltype(ib_c)::value;
      const int e1 = e0 + 1 >= 5 ? e0 - 4 : e0 + 1;
      const int e2 = e0 + 2 >= 5 ? e0 - 3 : e0 + 2;
      const int e3 = e0 + 3 >= 5 ? e0 - 2 : e0 + 3;
#pragma unroll
      for (int t = 0; t < 3; ++t)
        mm(t & 1, FA + FN, [&](int q) __attribute__((always_inline)) { rd(e0, e1, t + 1, q, (t + 1) & 1); });
      if constexpr (W >= 0) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of stage s are done
        wait_vmcnt<W * LB>();
        __builtin_amdgcn_s_barrier();
      }
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t b0 = ent(e0), b1 = ent(e1);
      constexpr int NA = IA ? LA : 0, NRD = W >= 0 ? FA + FN : 0, NB = IB ? LB : 0;
      mm(1, NA + NRD + NB, [&](int k) __attribute__((always_inline)) {
        if (k < NA) issue_a(b0, k);
        else if (k < NA + NRD) rd(e2, e3, 0, k - NA, 0);  // stage s+1's first fragments
        else issue_b(b1, k - NA - NRD);
      });
      if constexpr (IA) next_a();
      if constexpr (IB) next_b();
      e0 = e2;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using Im = std::integral_constant<int, -1>;
    // B(0), A(0), B(1), A(1), B(2) into entries 0..4
    {
      const uint32_t base = ent(0);
#pragma unroll
      for (int h = 0; h < 5; ++h) {
        if (h % 2 == 0) {
#pragma unroll
          for (int q = 0; q < LB; ++q) issue_b(base + h * ENT, q);
          next_b();
        } else {
#pragma unroll
          for (int q = 0; q < LA; ++q) issue_a(base + h * ENT, q);
          next_a();
        }
      }
    }
    wait_vmcnt<2 * LB + LA>();  // stage 0; B(1), A(1), B(2) may be in flight
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < FA + FN; ++q) rd(0, 1, 0, q, 0);
    int s = 0;
    for (; s + 3 < nk; ++s) step(I1{}, std::true_type{}, std::true_type{});
    step(I1{}, std::true_type{}, std::false_type{});   // s = nk-3: A(nk-1)
    step(I0{}, std::false_type{}, std::false_type{});  // s = nk-2
    step(Im{}, std::false_type{}, std::false_type{});  // s = nk-1
  };
  const int fa = wr.fa;
  switch (fa) {
    case 0: mainloop(std::integral_constant<int, 0>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 3: mainloop(std::integral_constant<int, FM >= 3 ? 3 : FM>{}); break;
    default: mainloop(std::integral_constant<int, FM>{}); break;
  }
  __syncthreads();
  ring64_store<GATED, BM, NT>(lds, acc, fa, wr.r0, wn, lane, tid, C, ldc, row0, nrows, n0, N, Cq, Cqs);
}

// Dense projections: 256 x 256 tiles over up to five K segments (the A and B
// loaders walk the segments separately, B a stage ahead of A).  When the
// tiles leave a last round of workgroups at most half full, the last nsplit
// tiles run as two 128-row halves each, so that last round fills the GPU:
// blocks below nt - nsplit take whole tiles in the XCD-aware order, the
// 2 nsplit blocks after them the halves (a half tile loads 3/4 of a whole
// one's operands for 1/2 of its MFMAs).
template <bool GATED, bool NT>
__global__ __launch_bounds__(512, 1) void ring64_dense_kernel(DenseGemm g, int nsplit) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BR = 256, NOUT = GATED ? 128 : 256, NW = 8, LB = 4, BK = kR64BK;
  extern __shared__ uint4 lds_u4[];
  char* lds = reinterpret_cast<char*>(lds_u4);
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)lds));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_n = (g.N + NOUT - 1) / NOUT;
  const uint32_t nwhole = gridDim.x - 2 * uint32_t(nsplit);  // blocks taking whole tiles
  uint32_t t;
  int half = -1;  // -1: a whole tile; else which 128-row half
  if (blockIdx.x < nwhole) {
    t = xcd_swizzle(blockIdx.x, nwhole);
  } else {
    const uint32_t h = xcd_swizzle(blockIdx.x - nwhole, 2 * uint32_t(nsplit));
    t = nwhole + h / 2;
    half = int(h % 2);
  }
  // within an XCD's run of tile indices, groups of 4 row tiles x all column
  // tiles, row tile fastest: the 32 tiles an XCD runs at once are 4 x 8, so
  // their A and B slices are shared through its L2 (the 16k up-projection
  // 617 -> 583 us against plain row-major; the down-projection unchanged)
  constexpr int GM = 4;
  const int tiles_m = (g.M + 255) / 256;
  const int first = int(t) / (GM * tiles_n) * GM, gs = min(tiles_m - first, GM), w = int(t) % (GM * tiles_n);
  const int tm = first + w % gs, tn = w / gs;
  const int row0 = tm * 256 + (half > 0 ? 128 : 0);
  const int nrows = min(half >= 0 ? 128 : 256, g.M - row0), n0 = tn * NOUT;
  if (nrows <= 0) return;  // (the empty second half of a short last row tile)
  const int lr = lane >> 3, gchunk = ring64_gchunk(wid, lane);
  int b_row[LB];
  bool b_up[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (wid + NW * i) * 8 + lr;
    b_up[i] = GATED && r >= BR / 2;
    b_row[i] = min(n0 + (b_up[i] ? r - BR / 2 : r), g.N - 1);
  }
  int nk = 0;
#pragma unroll
  for (int q = 0; q < 5; ++q)
    if (q < g.nseg) nk += g.seg[q].K / BK;
  auto tile = [&](auto bm_c) __attribute__((always_inline)) {
    constexpr int BM = decltype(bm_c)::value, LA = BM / 64;
    int a_row[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) a_row[i] = row0 + min((wid + NW * i) * 8 + lr, nrows - 1);
    const bf16_t* pa[LA];
    const bf16_t* pb[LB];
    auto set_a = [&](const GemmSeg& sg) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < LA; ++i) pa[i] = reinterpret_cast<const bf16_t*>(sg.A) + int64_t(a_row[i]) * sg.lda + gchunk * 8;
    };
    auto set_b = [&](const GemmSeg& sg) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < LB; ++i)
        pb[i] = reinterpret_cast<const bf16_t*>(b_up[i] ? sg.B3 : sg.B) + int64_t(b_row[i]) * sg.ldb + gchunk * 8;
    };
    set_a(g.seg[0]);
    set_b(g.seg[0]);
    int lsa = 0, lka = g.seg[0].K / BK, lsb = 0, lkb = g.seg[0].K / BK;
    auto next_a = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < LA; ++i) pa[i] += BK;
      if (--lka == 0 && lsa + 1 < g.nseg) {
        ++lsa;
        switch (lsa) {  // (static indices: the arguments stay in the kernarg segment)
          case 1: set_a(g.seg[1]); lka = g.seg[1].K / BK; break;
          case 2: set_a(g.seg[2]); lka = g.seg[2].K / BK; break;
          case 3: set_a(g.seg[3]); lka = g.seg[3].K / BK; break;
          default: set_a(g.seg[4]); lka = g.seg[4].K / BK; break;
        }
      }
    };
    auto next_b = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < LB; ++i) pb[i] += BK;
      if (--lkb == 0 && lsb + 1 < g.nseg) {
        ++lsb;
        switch (lsb) {
          case 1: set_b(g.seg[1]); lkb = g.seg[1].K / BK; break;
          case 2: set_b(g.seg[2]); lkb = g.seg[2].K / BK; break;
          case 3: set_b(g.seg[3]); lkb = g.seg[3].K / BK; break;
          default: set_b(g.seg[4]); lkb = g.seg[4].K / BK; break;
        }
      }
    };
    ring64_tile<GATED, BM, NT, false>(lds, lds0, wid, lane, tid, nk, nrows, pa, pb, next_a, next_b, g.C, g.ldc, row0,
                                         n0, g.N, g.Cq, g.Cqs);
  };
  if (half >= 0) tile(std::integral_constant<int, 128>{});
  else tile(std::integral_constant<int, 256>{});
#endif
}

// Grouped expert GEMMs on the routing's tiles of at most kTiledBM = 192 rows
// (tile table, gathered activation rows, the tile's expert's B).  FC1 (gated)
// writes H with nontemporal stores: at prefill its 134 MB of output otherwise
// pushes the weight stream and the gathered rows out of L2 (FC1 780 -> 745 us
// in the layer, alternated builds).  For FC2's Y the same hint was a wash (FC2
// slower by about what the combine that reads Y gained).
template <bool GATED>
__global__ __launch_bounds__(512, 1) void ring64_grouped_kernel(GroupedGemm g) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = kTiledBM, BR = 256, NOUT = GATED ? 128 : 256, NW = 8, LA = BM / 64, LB = 4, BK = kR64BK;
  extern __shared__ uint4 lds_u4[];
  char* lds = reinterpret_cast<char*>(lds_u4);
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)lds));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_n = (g.N + NOUT - 1) / NOUT;
  // grid sized for the host's upper bound; XCD-aware order over the real count
  const uint32_t nreal = uint32_t(*g.ntiles) * uint32_t(tiles_n);
  // a persistent grid (one workgroup per CU, in mirrored_tile's order), so a
  // tile's output stores drain while the next tile's first stages load
  uint32_t lt;
  for (uint32_t pass = 0; mirrored_tile(blockIdx.x, gridDim.x, nreal, pass, lt); ++pass) {
  const int tn = int(lt % uint32_t(tiles_n)), tm = int(lt / uint32_t(tiles_n));
  const Tile tl = g.tiles[tm];
  const int row0 = tl.row_start, nrows = min(tl.nrows, BM), n0 = tn * NOUT;
  const int lr = lane >> 3, gchunk = ring64_gchunk(wid, lane);
  const bf16_t* pa[LA];
  const bf16_t* pb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    int src = row0 + min((wid + NW * i) * 8 + lr, nrows - 1);
    if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
    pa[i] = reinterpret_cast<const bf16_t*>(g.A) + int64_t(src) * g.lda + gchunk * 8;
  }
  const int64_t be = int64_t(tl.expert) * g.b_estride;
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (wid + NW * i) * 8 + lr;
    const bool up = GATED && r >= BR / 2;
    const int n = min(n0 + (up ? r - BR / 2 : r), g.N - 1);
    pb[i] = reinterpret_cast<const bf16_t*>(up ? g.B3 : g.B) + be + int64_t(n) * g.ldb + gchunk * 8;
  }
  auto next_a = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LA; ++i) pa[i] += BK;
  };
  auto next_b = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LB; ++i) pb[i] += BK;
  };
  // (The hint is an instruction bit: one copy of the tile's code for each
  // form.)
  if (tl.solo)
    ring64_tile<GATED, BM, GATED, true>(lds, lds0, wid, lane, tid, g.K / BK, nrows, pa, pb, next_a, next_b, g.C, g.ldc,
                                        row0, n0, g.N);
  else
    ring64_tile<GATED, BM, GATED, false>(lds, lds0, wid, lane, tid, g.K / BK, nrows, pa, pb, next_a, next_b, g.C,
                                         g.ldc, row0, n0, g.N);
  __syncthreads();  // the epilogue's LDS reads are done before the next tile's loads land
  }
#endif
}

// ---------------------------------------- w4a16: MXFP4 weights, 64-wide ring ---
// Grouped expert GEMMs with MXFP4 weights and bf16 activations at prefill
// size (TokenSpeed Day-0 post, "Gluon kernels on AMD GPUs > Stable
// LatentMoE": MXFP4 weights upcast inside the K loop, bf16 activations): the
// tiles of ring64_grouped_kernel (<= 192 rows x 256 B rows, gated: 128 gate +
// 128 up; 8 waves as 2 x 4 with 96 x 64 wave tiles of 32x32x16 bf16 MFMAs),
// with every operand moved into LDS by direct-to-LDS loads of whole 128-byte
// lines and the weights upcast from LDS to bf16 fragments in registers by
// gfx950's scaled conversion (exact: an e2m1 value times a power of two).
// A 64-K stage holds 192 rows x 128 B of activations.  A weight row's codes
// for one stage are 32 B, a quarter line, so they travel in groups of four
// stages (256 rows x 128 B), and its e8m0 scales (2 B per stage) in groups
// of eight stages (16 B per row: one load per 64 rows; waves 4-7 load a copy
// that nobody reads, so every wave issues the same loads).  LDS: two code
// group slots (32 KB), two scale group slots (8 KB), two activation slots
// (24 KB): 128 KB.
// K order: in the 16-K step t of a stage, lane half h of both operands'
// fragments holds the stage's K 32 h + 8 t .. +7, so a lane's codes for the
// whole stage are one 16-byte LDS read, under one MX scale, per B column.
// Each product is summed once, in another order than the bf16 ring's.
// Schedule (group g = s / 4 in code slot g % 2, scale group h = s / 8 in
// scale slot h % 2, A(s) in slot s % 2): the prologue loads S0 G0 A0 A1 S1
// G1.  After the barrier of stage s (before its last step, whose fragments
// are already in registers) it loads, in this order: A(s + 2); code group
// s/4 + 2 on the last stage of a group; scale group s/8 + 2 on the last stage
// of a scale group.  Past the end a scale group is clamped to the last one (a
// harmless reload into a slot that is not read again), so the counts stay
// fixed.  vmcnt counts in issue order: before the barrier of stage s the
// wave waits for A(s + 1) and lets the groups issued after it fly.  Needs K
// a multiple of 512.
constexpr int kW4A = kTiledBM * 128;             // one stage's activations: 24 KB
constexpr int kW4B = 256 * 128;                  // a code group: 32 KB
constexpr int kW4S = 8 * 1024;                   // a scale group (and its spare copy)
// code slots first, so that a fragment read's slot and row offsets fit the
// LDS instructions' 16-bit immediate offset
constexpr int kW4BOff = 0;
constexpr int kW4SOff = kW4BOff + 2 * kW4B;
constexpr int kW4AOff = kW4SOff + 2 * kW4S;
constexpr int kW4Lds = kW4AOff + 2 * kW4A;       // 128 KiB

template <bool GATED>
__global__ __launch_bounds__(512, 1) void w4ring_grouped_kernel(GroupedGemm g) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = kTiledBM, BR = 256, NOUT = GATED ? 128 : 256, NW = 8, WAVES_N = 4;
  constexpr int WM = BM / 2, WN = 64, FM = WM / 32, FN = 2, ROWB = 128;
  constexpr int LA = BM / 64, LB = 4, LS = 1;
  static_assert(kW4Lds <= kR64Lds && BM * (NOUT + 8) * 2 <= kW4Lds, "LDS");
  extern __shared__ uint4 lds_u4[];
  char* lds = reinterpret_cast<char*>(lds_u4);
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)lds));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int tiles_n = (g.N + NOUT - 1) / NOUT;
  // grid sized for the host's upper bound; XCD-aware order over the real count
  const uint32_t nreal = uint32_t(*g.ntiles) * uint32_t(tiles_n);
  // a persistent grid in mirrored_tile's order (as ring64_grouped_kernel)
  uint32_t lt;
  for (uint32_t pass = 0; mirrored_tile(blockIdx.x, gridDim.x, nreal, pass, lt); ++pass) {
  const int tn = int(lt % uint32_t(tiles_n)), tm = int(lt / uint32_t(tiles_n));
  const Tile tl = g.tiles[tm];
  const int row0 = tl.row_start, nrows = min(tl.nrows, BM), n0 = tn * NOUT;
  const int K = g.K, nk = K / 64;
  const WaveRows wr = wave_rows(wm, nrows, FM);  // this wave row's first tile row and subtiles
  const int lr = lane >> 3, gchunk = ring64_gchunk(wid, lane);
  // Operand addresses: wave-uniform bases (advanced stage by stage) plus
  // fixed 32-bit lane offsets.  Lane l of wave w loads row 8 (w + 8 q) + l/8
  // of its operand into chunk l%8 of the LDS row, from global chunk
  // (l%8) ^ ((row/2) mod 8); weight loads q < 2 take rows 0..127 (gated: the
  // gate rows), q >= 2 rows 128..255 (gated: the up rows).  Scale loads: lane
  // l of wave w takes the 16 bytes of weight row 64 (w mod 4) + l.
  uint32_t oa[LA], ob[LB], os;
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    int src = row0 + min((wid + NW * i) * 8 + lr, nrows - 1);
    if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
    oa[i] = uint32_t(src) * uint32_t(g.lda * 2) + uint32_t(gchunk * 16);
  }
  // weight row r of the tile (gated: 128 gate rows, then 128 up rows): its
  // row in the expert's [N, K] matrix
  auto w_row = [&](int r) __attribute__((always_inline)) -> uint32_t {
    return uint32_t(min(n0 + (GATED && r >= BR / 2 ? r - BR / 2 : r), g.N - 1));
  };
#pragma unroll
  for (int i = 0; i < LB; ++i) ob[i] = w_row((wid + NW * i) * 8 + lr) * uint32_t(K / 2) + uint32_t(gchunk * 16);
  os = w_row(64 * (wid & 3) + lane) * uint32_t(K / 32);
  const int64_t wexp = int64_t(tl.expert) * g.N;
  const char* abase = reinterpret_cast<const char*>(g.A);
  const uint8_t* gbase = reinterpret_cast<const uint8_t*>(g.B) + wexp * (K / 2);
  const uint8_t* ubase = GATED ? reinterpret_cast<const uint8_t*>(g.B3) + wexp * (K / 2) : gbase;
  const uint8_t* sbase = (GATED && (wid & 3) >= 2 ? g.B3s : g.Bs) + wexp * (K / 32);
  const int nsg = nk / 8;
  auto rfl = [](uint32_t v) __attribute__((always_inline)) -> uint32_t {
    return uint32_t(__builtin_amdgcn_readfirstlane(int(v)));
  };
  auto issue_a = [&](int slot, int q) __attribute__((always_inline)) {
    g2lds16_so(abase, oa[q], rfl(lds0 + kW4AOff + slot * kW4A + (wid + NW * q) * 1024));
  };
  auto next_a = [&]() __attribute__((always_inline)) { abase += 128; };
  // the weight codes with the nontemporal hint: FC2's always (816-824 ->
  // 805-807 us at the 16k-token w4a16 shape, traced alternately), FC1's for
  // an expert's only tile (read once)
  const bool b_once = !GATED || tl.solo != 0;
  auto issue_g = [&](int slot, int q) __attribute__((always_inline)) {
    const uint32_t lb = rfl(lds0 + kW4BOff + slot * kW4B + (wid + NW * q) * 1024);
    if (b_once) g2lds16_so<true>(q < LB / 2 ? gbase : ubase, ob[q], lb);
    else g2lds16_so(q < LB / 2 ? gbase : ubase, ob[q], lb);
  };
  auto next_g = [&]() __attribute__((always_inline)) {  // four stages of packed codes
    gbase += 128;
    ubase += 128;
  };
  int sg_next = 0;  // the next scale group to load
  auto issue_s = [&](int slot) __attribute__((always_inline)) {
    g2lds16_so(sbase + min(sg_next, nsg - 1) * 16, os, rfl(lds0 + kW4SOff + slot * kW4S + wid * 1024));
    ++sg_next;
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
    bf16x8 af[2][FAR];  // activation fragments, by step parity
    uint4 bq[FN];       // a stage's weight codes (the next stage's are read
    uint32_t bs[FN];    // after the last step's conversion) and scale codes
    auto rd_a = [&](int aslot, int t, int i, int buf) __attribute__((always_inline)) {
      const int r = wr.r0 + i * 32 + fr;
      af[buf][i] = as_bf16x8(*reinterpret_cast<const uint4*>(lds + kW4AOff + aslot * kW4A + r * ROWB +
                                                             (((4 * fh + t) ^ fsw) << 4)));
    };
    // stage s's codes and scales, R = s mod 8, in code slot cs / scale slot ss
    auto rd_b = [&](int cs, int ss, int R, int j) __attribute__((always_inline)) {
      const int r = brow(j) + fr;
      bq[j] = *reinterpret_cast<const uint4*>(lds + kW4BOff + cs * kW4B + r * ROWB +
                                                   (((2 * (R & 3) + fh) ^ fsw) << 4));
      bs[j] = uint32_t(*reinterpret_cast<const uint8_t*>(lds + kW4SOff + ss * kW4S + r * 16 + 2 * R + fh));
    };
    // the 16-K step t's MFMAs on the stage's codes and activation set t & 1,
    // with the side items 0 .. nside-1 spread over them in order (MFMA m is
    // followed by items c m .. c m + c - 1, c = ceil(nside / NM); all at once
    // if NM = 0).  The order matters: the vmcnt waits count on each wave's
    // loads leaving in the order issued.
    auto mm = [&](int t, int nside, auto side) __attribute__((always_inline)) {
      constexpr int NM = FA * FN;
      const int c = NM > 0 ? (nside + NM - 1) / NM : 0;
      bf16x8 bf[FN];
      if constexpr (FA > 0)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint4 q = bq[j];
          const uint32_t w = t == 0 ? q.x : t == 1 ? q.y : t == 2 ? q.z : q.w;
          bf[j] = fp4x8_to_bf16(w, e8m0_multiplier(bs[j]));
        }
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FA; ++i) {
          acc[i][j] = mfma_32x32x16(af[t & 1][i], bf[j], acc[i][j]);
          const int m = j * FA + i;
#pragma unroll
          for (int k = 0; k < 16; ++k)
            if (k >= m * c && k < m * c + c && k < nside) side(k);
          __builtin_amdgcn_sched_barrier(0);
        }
      if constexpr (NM == 0) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (k < nside) side(k);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    int ss0 = 0;  // stage s's scale slot
    // stage s, R = s mod 8 (its A slot is R mod 2), LAST: in the last eight
    // stages.  W: loads allowed in flight at the barrier (-1: the last stage,
    // no barrier): those issued after A(s + 1), at stage s - 1
    auto stage = [&](auto r_c, auto last_c) __attribute__((always_inline)) {
      constexpr int R = decltype(r_c)::value;
      constexpr bool LAST = decltype(last_c)::value;
      constexpr bool IA = !LAST || R < 6, IG = !LAST && (R == 3 || R == 7), IS = !LAST && R == 7;
      constexpr int W = (LAST && R == 7) ? -1 : R == 0 ? LB + LS : (R == 4 && !LAST) ? LB : 0;
      constexpr int AS = R & 1, ASN = AS ^ 1;                                // A slots of s and s+1
      constexpr int CS = R >= 4 ? 1 : 0, CSN = ((R + 1) & 7) >= 4 ? 1 : 0;  // code slots of s and s+1
#pragma unroll
      for (int t = 0; t < 3; ++t)
        mm(t, FA, [&](int i) __attribute__((always_inline)) { rd_a(AS, t + 1, i, (t + 1) & 1); });
      if constexpr (W >= 0) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of stage s are done
        wait_vmcnt<W>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");       // no LDS read moves above the barrier
      }
      __builtin_amdgcn_sched_barrier(0);
      const int ss1 = R == 7 ? ss0 ^ 1 : ss0;
      constexpr int NA = IA ? LA : 0, NG = IG ? LB : 0, NS = IS ? LS : 0;
      constexpr int NRB = (W >= 0 && FA > 0) ? FN : 0, NRA = W >= 0 ? FA : 0;
      mm(3, NA + NG + NS + NRB + NRA, [&](int k) __attribute__((always_inline)) {
        if (k < NA) issue_a(AS, k);                        // A(s+2) into A(s)'s slot
        else if (k < NA + NG) issue_g(CS, k - NA);         // code group s/4 + 2 into group s/4's slot
        else if (k < NA + NG + NS) issue_s(ss0);           // scale group s/8 + 2 into s/8's slot
        else if (k < NA + NG + NS + NRB) rd_b(CSN, ss1, (R + 1) & 7, k - NA - NG - NS);
        else rd_a(ASN, 0, k - NA - NG - NS - NRB, 0);      // stage s+1's first fragments
      });
      if constexpr (NA > 0) next_a();
      if constexpr (NG > 0) next_g();
      ss0 = ss1;
    };
    using T = std::true_type;
    using F = std::false_type;
    // prologue: S0 G0 A0 A1 S1 G1
    issue_s(0);
#pragma unroll
    for (int q = 0; q < LB; ++q) issue_g(0, q);
    next_g();
#pragma unroll
    for (int e = 0; e < 2; ++e) {
#pragma unroll
      for (int q = 0; q < LA; ++q) issue_a(e, q);
      next_a();
    }
    issue_s(1);
#pragma unroll
    for (int q = 0; q < LB; ++q) issue_g(1, q);
    next_g();
    wait_vmcnt<LA + LS + LB>();  // S0, G0 and A0 have landed
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (FA > 0)
#pragma unroll
      for (int j = 0; j < FN; ++j) rd_b(0, 0, 0, j);
#pragma unroll
    for (int i = 0; i < FA; ++i) rd_a(0, 0, i, 0);
    using std::integral_constant;
    for (int s = 0; s + 8 < nk; s += 8) {
      stage(integral_constant<int, 0>{}, F{});
      stage(integral_constant<int, 1>{}, F{});
      stage(integral_constant<int, 2>{}, F{});
      stage(integral_constant<int, 3>{}, F{});
      stage(integral_constant<int, 4>{}, F{});
      stage(integral_constant<int, 5>{}, F{});
      stage(integral_constant<int, 6>{}, F{});
      stage(integral_constant<int, 7>{}, F{});
    }
    stage(integral_constant<int, 0>{}, T{});
    stage(integral_constant<int, 1>{}, T{});
    stage(integral_constant<int, 2>{}, T{});
    stage(integral_constant<int, 3>{}, T{});
    stage(integral_constant<int, 4>{}, T{});
    stage(integral_constant<int, 5>{}, T{});
    stage(integral_constant<int, 6>{}, T{});
    stage(integral_constant<int, 7>{}, T{});
  };
  const int fa = wr.fa;
  switch (fa) {
    case 0: mainloop(std::integral_constant<int, 0>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    default: mainloop(std::integral_constant<int, FM>{}); break;
  }
  __syncthreads();
  ring64_store<GATED, BM, GATED>(lds, acc, fa, wr.r0, wn, lane, tid, g.C, g.ldc, row0, nrows, n0, g.N);
  __syncthreads();  // the epilogue's LDS reads are done before the next tile's loads land
  }
#endif
}

// ring64_dense_kernel takes bf16 outputs and segments whose K are multiples
// of 64, at least 3 stages in all.
bool ring64_fits(const DenseGemm& d) {
  if (d.Cf || d.nseg < 1 || d.nseg > 5 || d.M <= 0 || d.N <= 0) return false;
  int nk = 0;
  for (int i = 0; i < d.nseg; ++i) {
    if (d.seg[i].K <= 0 || d.seg[i].K % kR64BK) return false;
    nk += d.seg[i].K / kR64BK;
  }
  return nk >= 3;
}

bool dense_gemm_quant_fits_impl(const DenseGemm& d) {
  return ring64_fits(d) && !d.gated && d.N % 32 == 0 && d.ldc % 32 == 0;
}

template <bool GATED>
hipError_t run_ring64(const DenseGemm& d, hipStream_t s) {
  constexpr int NOUT = GATED ? 128 : 256;
  auto kern = d.stream_c ? ring64_dense_kernel<GATED, true> : ring64_dense_kernel<GATED, false>;
  if (hipError_t e = allow_dynamic_lds((const void*)kern, kR64Lds); e != hipSuccess) return e;
  const int64_t nt = int64_t((d.M + 255) / 256) * ((d.N + NOUT - 1) / NOUT);
  if (nt <= 0) return hipSuccess;
  // one workgroup per CU at a time: split the tiles of a last round that
  // would be at most half full into 128-row halves
  const int64_t cus = device_cus(), rest = nt % cus;
  const int64_t nsplit = rest <= cus / 2 ? rest : 0;
  const int64_t nblk = nt + nsplit;
  if (nblk > int64_t(0x7fffffff)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3{uint32_t(nblk)}, dim3{512u}, kR64Lds, s, d, int(nsplit));
  return hipGetLastError();
}

template <bool GATED>
hipError_t run_ring64_grouped(const GroupedGemm& g, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  constexpr int NOUT = GATED ? 128 : 256;
  auto kern = ring64_grouped_kernel<GATED>;
  if (hipError_t e = allow_dynamic_lds((const void*)kern, kR64Lds); e != hipSuccess) return e;
  int64_t nblk = g.max_tiles * ((g.N + NOUT - 1) / NOUT);
  if (nblk <= 0) return hipSuccess;
  if (nblk > int64_t(0x7fffffff)) return hipErrorInvalidValue;
  // one workgroup per CU, or fewer when the tiles are fewer; a multiple of 8
  // either way (mirrored_tile: blockIdx mod 8 is the XCD the hardware deals
  // a workgroup to, and every XCD holds grid/8 of them)
  nblk = std::min<int64_t>((nblk + 7) / 8 * 8, (device_cus() + 7) / 8 * 8);
  return launch_kernel((const void*)kern, dim3{uint32_t(nblk)}, dim3{512u}, kR64Lds, s, g, t0, t1);
}

template <bool GATED>
hipError_t run_w4ring_grouped(const GroupedGemm& g, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  constexpr int NOUT = GATED ? 128 : 256;
  auto kern = w4ring_grouped_kernel<GATED>;
  if (hipError_t e = allow_dynamic_lds((const void*)kern, kW4Lds); e != hipSuccess) return e;
  int64_t nblk = g.max_tiles * ((g.N + NOUT - 1) / NOUT);
  if (nblk <= 0) return hipSuccess;
  if (nblk > int64_t(0x7fffffff)) return hipErrorInvalidValue;
  nblk = std::min<int64_t>((nblk + 7) / 8 * 8, (device_cus() + 7) / 8 * 8);  // the persistent grid
  return launch_kernel((const void*)kern, dim3{uint32_t(nblk)}, dim3{512u}, kW4Lds, s, g, t0, t1);
}

// The ring kernel takes bf16 outputs and segments whose K are multiples of
// 32, at least 4 stages in all.
bool ring_fits(const DenseGemm& d) {
  if (d.Cf || d.nseg < 1 || d.nseg > 5 || d.M <= 0 || d.N <= 0) return false;
  int nk = 0;
  for (int i = 0; i < d.nseg; ++i) {
    if (d.seg[i].K <= 0 || d.seg[i].K % kRingBK) return false;
    nk += d.seg[i].K / kRingBK;
  }
  return nk >= kRingSlots - 1;
}

template <bool GATED>
hipError_t run_ring(const DenseGemm& d, hipStream_t s) {
  constexpr int NOUT = GATED ? 128 : 256;
  auto kern = ring_dense_kernel<GATED>;
  if (hipError_t e = allow_dynamic_lds((const void*)kern, kRingLds); e != hipSuccess) return e;
  const int64_t nblk = int64_t((d.M + 255) / 256) * ((d.N + NOUT - 1) / NOUT);
  if (nblk <= 0) return hipSuccess;
  if (nblk > int64_t(0x7fffffff)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3{uint32_t(nblk)}, dim3{512u}, kRingLds, s, d);
  return hipGetLastError();
}

}  // namespace

bool dense_gemm_quant_fits(const DenseGemm& d) { return dense_gemm_quant_fits_impl(d); }

hipError_t launch_dense_gemm(const DenseGemm& d, hipStream_t s) {
  if ((d.Cq || d.Cqs) && !dense_gemm_quant_fits_impl(d)) return hipErrorInvalidValue;
  if (ring64_fits(d)) return d.gated ? run_ring64<true>(d, s) : run_ring64<false>(d, s);
  if (ring_fits(d)) return d.gated ? run_ring<true>(d, s) : run_ring<false>(d, s);
  TiledArgs a{};
  a.M = d.M;
  a.N = d.N;
  a.nseg = d.nseg;
  for (int i = 0; i < d.nseg; ++i) a.seg[i] = d.seg[i];
  a.a_rows = nullptr;
  a.a_row_div = 1;
  a.b_estride = 0;
  a.C = d.C;
  a.Cf = d.Cf;
  a.ldc = d.ldc;
  const int64_t mt = (d.M + 255) / 256;
  if (d.Cf) {
    if (d.gated) return hipErrorInvalidValue;
    return run_tiled<8, 2, false, false, false, true>(a, mt, s);
  }
  if (d.gated) return run_tiled<8, 2, true, false, false>(a, mt, s);
  return run_tiled<8, 2, false, false, false>(a, mt, s);
}

hipError_t launch_pack_weights(const uint16_t* src, uint16_t* dst, int E, int N, int K, hipStream_t s) {
  if (E <= 0 || N % kPackRows || K % 64) return hipErrorInvalidValue;
  const int64_t nchunks = int64_t(E) * N * (K / 8);
  const int64_t nblk = (nchunks + 255) / 256;
  if (nblk > int64_t(0x7fffffff)) return hipErrorInvalidValue;
  pack_weights_kernel<<<dim3{uint32_t(nblk)}, dim3{256}, 0, s>>>(reinterpret_cast<const uint4*>(src),
                                                                  reinterpret_cast<uint4*>(dst), nchunks, N, K);
  return hipGetLastError();
}

hipError_t launch_grouped_tiled(const GroupedGemm& g, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  // routing cuts tiles at kTiledBM rows; both kernels take tiles of up to 192 rows
  static_assert(kTiledBM <= 192, "tile table granularity");
  if (g.w4) {
    // (the bf16 fallback below has no MXFP4 form)
    if (g.packed || g.K % 128 || g.K < 256 || !g.Bs || (g.gated && !g.B3s)) return hipErrorInvalidValue;
    // K a multiple of 512 and 32-bit offsets into A and an expert's codes:
    // the direct-to-LDS ring form
    constexpr int64_t kOff = int64_t(1) << 31;
    if (g.K % 512 == 0 && g.a_rows_n > 0 && g.a_rows_n * g.lda * 2 < kOff && int64_t(g.N) * g.K / 2 < kOff)
      return g.gated ? run_w4ring_grouped<true>(g, s, t0, t1) : run_w4ring_grouped<false>(g, s, t0, t1);
    return g.gated ? run_grouped<true, false, true>(g, s, t0, t1) : run_grouped<false, false, true>(g, s, t0, t1);
  }
  if (g.packed) {
    // the tile-packed layout has only the register-staged form
    if (g.K % 128 || g.K < 256) return hipErrorInvalidValue;
    return g.gated ? run_grouped<true, true>(g, s, t0, t1) : run_grouped<false, true>(g, s, t0, t1);
  }
  if (g.K % kR64BK == 0 && g.K >= 3 * kR64BK)
    return g.gated ? run_ring64_grouped<true>(g, s, t0, t1) : run_ring64_grouped<false>(g, s, t0, t1);
  TiledArgs a{};
  a.M = 0;
  a.N = g.N;
  a.nseg = 1;
  a.seg[0] = GemmSeg{g.A, g.lda, g.B, g.B3, g.ldb, g.K};
  a.a_rows = g.a_rows;
  a.a_row_div = g.a_row_div;
  a.b_estride = g.b_estride;
  a.tiles = g.tiles;
  a.ntiles = g.ntiles;
  a.C = g.C;
  a.ldc = g.ldc;
  if (g.gated) return run_tiled<8, 2, true, true, true>(a, g.max_tiles, s, t0, t1);
  return run_tiled<8, 2, false, true, true>(a, g.max_tiles, s, t0, t1);
}

static int64_t splitk_args(const DenseGemm* parts, int nparts, SplitKArgs& a) {
  a.M = parts[0].M;
  a.nparts = nparts;
  int64_t nblk = 0;
  for (int i = 0; i < nparts; ++i) {
    const DenseGemm& d = parts[i];
    SplitKPart& P = a.part[i];
    P.N = d.N;
    P.nseg = d.nseg;
    for (int j = 0; j < d.nseg; ++j) P.seg[j] = d.seg[j];
    P.gated = d.gated ? 1 : 0;
    P.C = d.C;
    P.Cf = d.Cf;
    P.ldc = d.ldc;
    if (d.Cf && d.gated) return -1;
    const int64_t nb = int64_t((d.M + 15) / 16) * ((d.N + 16 * kSkNS - 1) / (16 * kSkNS));
    if (i == 0) a.nblk0 = int(nb);
    nblk += nb;
  }
  return nblk;
}

hipError_t launch_small_dense(const DenseGemm* parts, int nparts, hipStream_t s) {
  SplitKArgs a{};
  const int64_t nblk = splitk_args(parts, nparts, a);
  if (nblk < 0) return hipErrorInvalidValue;
  if (nblk == 0) return hipSuccess;
  splitk_dense_kernel<<<dim3{uint32_t(nblk)}, dim3{256}, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_small_dense_with_router(const DenseGemm* parts, int nparts, const FrontRoute& r, hipStream_t s) {
  SplitKArgs a{};
  const int64_t nblk = splitk_args(parts, nparts, a);
  if (nblk < 0 || r.E > 1024) return hipErrorInvalidValue;
  const int nrb = int((r.T + 3) / 4);
  const dim3 grid{uint32_t(nblk + nrb)}, block{256};
  if (grid.x == 0) return hipSuccess;
  if (r.E <= 128) splitk_router_kernel<2><<<grid, block, 0, s>>>(a, r, nrb);
  else if (r.E <= 256) splitk_router_kernel<4><<<grid, block, 0, s>>>(a, r, nrb);
  else if (r.E <= 512) splitk_router_kernel<8><<<grid, block, 0, s>>>(a, r, nrb);
  else splitk_router_kernel<16><<<grid, block, 0, s>>>(a, r, nrb);
  return hipGetLastError();
}

}  // namespace lmoe
