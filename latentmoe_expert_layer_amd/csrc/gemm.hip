// bf16 MFMA GEMMs of the LatentMoE layer (gfx950).
//
// All operands are "[rows, K]" with K contiguous (activations [M,K], weights
// [N,K] in the [out, in] layout), so C = A * B^T reads both operands along K.
//
//  * tiled_gemm_kernel: LDS double-buffered macro tiles for the dense
//    projections (latent down-proj fused with the shared experts' gate/up,
//    and the latent up-proj K-concatenated with the shared experts' down
//    proj) and for prefill-shaped grouped expert GEMMs (vLLM Kimi K3 post,
//    section 1: experts run in the latent; TokenSpeed Day-0 post,
//    "TensorRT-LLM Stable LatentMoE": FC1 with its gate as one gated GEMM,
//    then FC2).  Grouped tiles come from the device-side tile table, so no
//    per-expert row count ever reaches the host.
//  * skinny_grouped_kernel: decode-shaped grouped GEMMs where every expert
//    sees a handful of rows and the cost is streaming its weights once; each
//    wave keeps a whole K chunk of loads in flight and skips LDS.
#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

constexpr int kBK = 64;          // K per LDS stage
constexpr int kLdsK = kBK + 8;   // padded LDS row (bf16): 144 B, conflict-free 16 B reads

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
  int64_t ldc;
};

__device__ __forceinline__ uint4 ldg16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATED, bool GROUPED>
__global__ __launch_bounds__(64 * WAVES_M* WAVES_N) void tiled_gemm_kernel(TiledArgs g) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int BNT = GATED ? 2 * BN : BN;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int CPR = kBK / 8;                 // 16-byte chunks per row per stage
  constexpr int A_CH = BM * CPR / NT;
  constexpr int B_CH = BNT * CPR / NT;
  static_assert(BM * CPR % NT == 0 && BNT * CPR % NT == 0, "tile/threads mismatch");
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");

  extern __shared__ uint4 lds_u4[];
  bf16_t* As = reinterpret_cast<bf16_t*>(lds_u4);  // [2][BM][kLdsK]
  bf16_t* Bs = As + 2 * BM * kLdsK;                 // [2][BNT][kLdsK]

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int tiles_n = g.N / BN;
  const uint32_t lt = xcd_swizzle(blockIdx.x, gridDim.x);
  const int tn = int(lt % uint32_t(tiles_n));
  const int tm = int(lt / uint32_t(tiles_n));
  int expert = 0, row0, nrows;
  if constexpr (GROUPED) {
    if (tm >= *g.ntiles) return;
    const Tile tl = g.tiles[tm];
    expert = tl.expert;
    row0 = tl.row_start;
    nrows = tl.nrows;
  } else {
    row0 = tm * BM;
    nrows = min(BM, g.M - row0);
  }
  const int n0 = tn * BN;

  f32x4 acc[FM][FN];
  f32x4 acc3[GATED ? FM : 1][GATED ? FN : 1];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (GATED) acc3[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  for (int s = 0; s < g.nseg; ++s) {
    const GemmSeg sg = g.seg[s];
    const bf16_t* ap[A_CH];
    const bf16_t* bp[B_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT, r = c / CPR, kc = c % CPR;
      const int rr = min(r, nrows - 1);
      int64_t src = int64_t(row0) + rr;
      if constexpr (GROUPED) {
        if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
      }
      ap[i] = sg.A + src * sg.lda + kc * 8;
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NT, r = c / CPR, kc = c % CPR;
      const bf16_t* base = (GATED && r >= BN) ? sg.B3 : sg.B;
      const int rn = (GATED && r >= BN) ? r - BN : r;
      bp[i] = base + int64_t(expert) * g.b_estride + int64_t(n0 + rn) * sg.ldb + kc * 8;
    }
    const int nk = sg.K / kBK;
    uint4 ra[A_CH], rb[B_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[i] = ldg16(ap[i]);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[i] = ldg16(bp[i]);
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(&As[(c / CPR) * kLdsK + (c % CPR) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(&Bs[(c / CPR) * kLdsK + (c % CPR) * 8]) = rb[i];
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) {
        const int koff = (kt + 1) * kBK;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) ra[i] = ldg16(ap[i] + koff);
#pragma unroll
        for (int i = 0; i < B_CH; ++i) rb[i] = ldg16(bp[i] + koff);
      }
      const bf16_t* Ab = As + buf * BM * kLdsK;
      const bf16_t* Bb = Bs + buf * BNT * kLdsK;
#pragma unroll
      for (int ks = 0; ks < kBK / 32; ++ks) {
        const int kof = ks * 32 + (lane >> 4) * 8;
        bf16x8 af[FM], bf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&Ab[(wm * WM + i * 16 + (lane & 15)) * kLdsK + kof]));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bf[j] = as_bf16x8(*reinterpret_cast<const uint4*>(&Bb[(wn * WN + j * 16 + (lane & 15)) * kLdsK + kof]));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma_16x16x32(af[i], bf[j], acc[i][j]);
        if constexpr (GATED) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
            bf[j] = as_bf16x8(
                *reinterpret_cast<const uint4*>(&Bb[(BN + wn * WN + j * 16 + (lane & 15)) * kLdsK + kof]));
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc3[i][j] = mfma_16x16x32(af[i], bf[j], acc3[i][j]);
        }
      }
      if (kt + 1 < nk) {
        bf16_t* An = As + (buf ^ 1) * BM * kLdsK;
        bf16_t* Bn = Bs + (buf ^ 1) * BNT * kLdsK;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
          const int c = tid + i * NT;
          *reinterpret_cast<uint4*>(&An[(c / CPR) * kLdsK + (c % CPR) * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
          const int c = tid + i * NT;
          *reinterpret_cast<uint4*>(&Bn[(c / CPR) * kLdsK + (c % CPR) * 8]) = rb[i];
        }
      }
      __syncthreads();
    }
  }

  // Epilogue: stage the bf16 tile in LDS, then 16-byte row-contiguous stores.
  constexpr int CLD = BN + 8;
  bf16_t* Cs = As;  // BM * CLD <= 2 * (BM + BNT) * kLdsK
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * WM + i * 16 + (lane >> 4) * 4 + r;
        const int col = wn * WN + j * 16 + (lane & 15);
        float v = acc[i][j][r];
        if constexpr (GATED) v = silu_mul(v, acc3[i][j][r]);
        Cs[row * CLD + col] = f32_to_bf16(v);
      }
  __syncthreads();
  constexpr int OCPR = BN / 8;
  for (int c = tid; c < BM * OCPR; c += NT) {
    const int row = c / OCPR, cc = c % OCPR;
    if (row < nrows) {
      *reinterpret_cast<uint4*>(g.C + (int64_t(row0) + row) * g.ldc + n0 + cc * 8) =
          *reinterpret_cast<const uint4*>(&Cs[row * CLD + cc * 8]);
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATED, bool GROUPED>
hipError_t run_tiled(const TiledArgs& a, int64_t mtiles, hipStream_t s) {
  constexpr int BNT = GATED ? 2 * BN : BN;
  const size_t lds = size_t(2) * (BM + BNT) * kLdsK * sizeof(bf16_t);
  static_assert(size_t(BM) * (BN + 8) <= size_t(2) * (BM + BNT) * kLdsK, "epilogue staging fits");
  auto kern = tiled_gemm_kernel<BM, BN, WAVES_M, WAVES_N, GATED, GROUPED>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t nblk = mtiles * (a.N / BN);
  if (nblk <= 0) return hipSuccess;
  kern<<<dim3(uint32_t(nblk)), dim3(64 * WAVES_M * WAVES_N), lds, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------- skinny grouped ---
// Block = (m-tile of <= 16 rows, 64 output columns); wave w owns columns
// n0 + 16w .. +16 and runs 16x16x32 MFMAs over K, KCH steps of 32 per chunk
// with all of a chunk's loads issued together.
template <bool GATED, int KCH>
__global__ __launch_bounds__(256) void skinny_grouped_kernel(GroupedGemm g) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int tiles_n = g.N / 64;
  const uint32_t lt = xcd_swizzle(blockIdx.x, gridDim.x);
  const int tm = int(lt / uint32_t(tiles_n)), tn = int(lt % uint32_t(tiles_n));
  if (tm >= *g.ntiles) return;
  const Tile tl = g.tiles[tm];
  const int arow = min(lane & 15, tl.nrows - 1);
  int64_t src = int64_t(tl.row_start) + arow;
  if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
  const int kof = (lane >> 4) * 8;
  const bf16_t* ap = g.A + src * g.lda + kof;
  const int n = tn * 64 + wid * 16 + (lane & 15);
  const int64_t boff = int64_t(tl.expert) * g.b_estride + int64_t(n) * g.ldb + kof;
  const bf16_t* bp = g.B + boff;
  const bf16_t* b3p = GATED ? g.B3 + boff : nullptr;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc3 = {0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < g.K; kc += 32 * KCH) {
    uint4 a[KCH], b[KCH], b3[GATED ? KCH : 1];
#pragma unroll
    for (int s = 0; s < KCH; ++s) {
      a[s] = ldg16(ap + kc + s * 32);
      b[s] = ldg16(bp + kc + s * 32);
      if constexpr (GATED) b3[s] = ldg16(b3p + kc + s * 32);
    }
#pragma unroll
    for (int s = 0; s < KCH; ++s) {
      acc = mfma_16x16x32(as_bf16x8(a[s]), as_bf16x8(b[s]), acc);
      if constexpr (GATED) acc3 = mfma_16x16x32(as_bf16x8(a[s]), as_bf16x8(b3[s]), acc3);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = (lane >> 4) * 4 + r;
    if (row < tl.nrows) {
      float v = acc[r];
      if constexpr (GATED) v = silu_mul(v, acc3[r]);
      g.C[(int64_t(tl.row_start) + row) * g.ldc + n] = f32_to_bf16(v);
    }
  }
}

}  // namespace

hipError_t launch_dense_gemm(const DenseGemm& d, hipStream_t s) {
  TiledArgs a{};
  a.M = d.M;
  a.N = d.N;
  a.nseg = d.nseg;
  for (int i = 0; i < d.nseg; ++i) a.seg[i] = d.seg[i];
  a.a_rows = nullptr;
  a.a_row_div = 1;
  a.b_estride = 0;
  a.C = d.C;
  a.ldc = d.ldc;
  constexpr int BM = 128;
  const int64_t mt = (d.M + BM - 1) / BM;
  if (d.gated) return run_tiled<BM, 64, 2, 2, true, false>(a, mt, s);
  if (d.N % 128 == 0) return run_tiled<BM, 128, 2, 2, false, false>(a, mt, s);
  return run_tiled<BM, 64, 2, 2, false, false>(a, mt, s);
}

hipError_t launch_grouped_tiled(const GroupedGemm& g, hipStream_t s) {
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
  static_assert(kTiledBM == 128, "tile table granularity");
  if (g.gated) return run_tiled<128, 64, 2, 2, true, true>(a, g.max_tiles, s);
  if (g.N % 128 == 0) return run_tiled<128, 128, 2, 2, false, true>(a, g.max_tiles, s);
  return run_tiled<128, 64, 2, 2, false, true>(a, g.max_tiles, s);
}

hipError_t launch_grouped_skinny(const GroupedGemm& g, hipStream_t s) {
  const int64_t nblk = g.max_tiles * (g.N / 64);
  if (nblk <= 0) return hipSuccess;
  const dim3 grid{uint32_t(nblk)}, block{256};
  if (g.K % 256 == 0) {
    if (g.gated) skinny_grouped_kernel<true, 8><<<grid, block, 0, s>>>(g);
    else skinny_grouped_kernel<false, 8><<<grid, block, 0, s>>>(g);
  } else {
    if (g.gated) skinny_grouped_kernel<true, 2><<<grid, block, 0, s>>>(g);
    else skinny_grouped_kernel<false, 2><<<grid, block, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace lmoe
