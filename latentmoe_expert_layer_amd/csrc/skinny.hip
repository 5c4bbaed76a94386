// Decode-shaped grouped expert GEMMs (gfx950): every expert sees a handful of
// rows (256 tokens x top-16 over 896 experts is ~4.6 rows each), so the cost
// is streaming each touched expert's weights from HBM once (vLLM Kimi K3
// post, section 1: the experts run in the latent space; TokenSpeed Day-0
// post, "TensorRT-LLM Stable LatentMoE": FC1 with its gate as one gated GEMM,
// then FC2).  Each wave keeps a whole K chunk of loads in flight and the
// operands go straight from registers into the MFMAs, with no LDS.
#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

// ---------------------------------------------------------- skinny grouped ---
// Block = (m-tile of <= 16 rows, 64*NS output columns); wave w owns NS
// 16-column subtiles and runs 16x16x32 MFMAs over K in chunks of KCH steps of
// 32, each chunk's loads issued together (the scheduling barrier keeps the
// compiler from interleaving them with the MFMAs, which would leave only a few
// loads in flight per wave).  Blocks take tiles in plain launch order: the
// hardware deals consecutive blocks to different XCDs, so at any moment all
// XCDs stream neighbouring weight rows, which measured ~20% faster here than
// grouping an expert's blocks on one XCD.
template <bool GATED, int KCH, int NS>
__global__ __launch_bounds__(256) void skinny_grouped_kernel(GroupedGemm g) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int WCOLS = 16 * NS, BCOLS = 4 * WCOLS;
  const int tiles_n = g.N / BCOLS;
  const uint32_t lt = blockIdx.x;
  const int tm = int(lt / uint32_t(tiles_n)), tn = int(lt % uint32_t(tiles_n));
  if (tm >= *g.ntiles) return;
  const Tile tl = g.tiles[tm];
  const int arow = min(lane & 15, tl.nrows - 1);
  int64_t src = int64_t(tl.row_start) + arow;
  if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
  const int kof = (lane >> 4) * 8;
  const bf16_t* ap = g.A + src * g.lda + kof;
  const int nb = tn * BCOLS + wid * WCOLS + (lane & 15);
  const bf16_t* bp[NS];
  const bf16_t* b3p[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int64_t boff = int64_t(tl.expert) * g.b_estride + int64_t(nb + 16 * j) * g.ldb + kof;
    bp[j] = g.B + boff;
    b3p[j] = GATED ? g.B3 + boff : nullptr;
  }
  f32x4 acc[NS], acc3[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc3[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int kc = 0; kc < g.K; kc += 32 * KCH) {
    uint4 a[KCH], b[NS][KCH], b3[NS][GATED ? KCH : 1];
#pragma unroll
    for (int s = 0; s < KCH; ++s) a[s] = ldg16(ap + kc + s * 32);
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int s = 0; s < KCH; ++s) {
        b[j][s] = ldg16(bp[j] + kc + s * 32);
        if constexpr (GATED) b3[j][s] = ldg16(b3p[j] + kc + s * 32);
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KCH; ++s)
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        acc[j] = mfma_16x16x32(as_bf16x8(a[s]), as_bf16x8(b[j][s]), acc[j]);
        if constexpr (GATED) acc3[j] = mfma_16x16x32(as_bf16x8(a[s]), as_bf16x8(b3[j][s]), acc3[j]);
      }
  }
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (lane >> 4) * 4 + r;
      if (row < tl.nrows) {
        float v = acc[j][r];
        if constexpr (GATED) v = silu_mul(v, acc3[j][r]);
        g.C[(int64_t(tl.row_start) + row) * g.ldc + nb + 16 * j] = f32_to_bf16(v);
      }
    }
}

}  // namespace

hipError_t launch_grouped_skinny(const GroupedGemm& g, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const int64_t nblk = g.max_tiles * (g.N / 64);
  if (nblk <= 0) return hipSuccess;
  const dim3 grid{uint32_t(nblk)}, block{256};
  const void* kern;
  if (g.gated) {
    kern = g.K % 128 == 0 ? (const void*)skinny_grouped_kernel<true, 4, 1> : (const void*)skinny_grouped_kernel<true, 2, 1>;
  } else {
    kern = g.K % 256 == 0   ? (const void*)skinny_grouped_kernel<false, 8, 1>
           : g.K % 128 == 0 ? (const void*)skinny_grouped_kernel<false, 4, 1>
                            : (const void*)skinny_grouped_kernel<false, 2, 1>;
  }
  return launch_kernel(kern, grid, block, 0, s, g, t0, t1);
}

}  // namespace lmoe
