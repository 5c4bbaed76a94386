// Host-side launchers of the LatentMoE HIP kernels (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per (device, kernel); thread-safe.  Host code (defined in api.hip).
hipError_t allow_dynamic_lds(const void* kernel, int bytes);

// kernel<<<grid, block, lds, s>>>(arg); with t0 / t1 set, the launch goes
// through hipExtLaunchKernel, which records them at the kernel's own start
// and end (the expert GEMMs' stage timing).
template <class Arg>
hipError_t launch_kernel(const void* kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, const Arg& arg,
                         hipEvent_t t0, hipEvent_t t1) {
  void* args[] = {const_cast<Arg*>(&arg)};
  if (t0 || t1) return hipExtLaunchKernel(kernel, grid, block, args, lds, s, t0, t1, 0);
  return hipLaunchKernel(kernel, grid, block, args, lds, s);
}

// One grouped-GEMM m-tile: rows [row_start, row_start + nrows) of one expert's
// segment in the permuted (expert-major) row order.
struct Tile {
  int32_t expert;
  int32_t row_start;
  int32_t nrows;
  int32_t solo;  // 1: the expert's only tile, so the launch reads its weights once
};

// Row-tile granularities of the tile tables that routing builds.
constexpr int kSkinnyBM = 16;   // weight-streaming (decode-shaped) kernel
constexpr int kTiledBM = 192;   // LDS-tiled (prefill-shaped) kernels: a tile holds <= 192 rows

inline int64_t max_tiles(int64_t rows, int64_t E, int bm) {
  return rows / bm + (rows < E ? rows : E) + 1;
}

// ---- router / permute -------------------------------------------------------
hipError_t launch_router(const float* logits, int64_t T, int E, int k, int32_t* ids, float* w,
                         hipStream_t s);
hipError_t launch_copy_ids(const int32_t* ids_in, const float* w_in, int64_t n, int32_t* ids,
                           float* w, hipStream_t s);
// Stable counting sort of R rows by expert plus the two tile tables.
// scratch: permute_scratch_ints(R, E) int32 of device memory (may be NULL when
// that is 0); large batches keep their per-chunk expert counts there.
hipError_t launch_permute(const int32_t* ids, int64_t R, int E, int32_t* offsets, int32_t* sorted_row,
                          int32_t* row_pos, Tile* tiles_skinny, int32_t* n_skinny, Tile* tiles_tiled,
                          int32_t* n_tiled, int32_t* scratch, hipStream_t s);
int64_t permute_scratch_ints(int64_t R, int E);
int permute_waves(int E);  // 0 if E is too large

// ---- GEMMs --------------------------------------------------------------------
// C[M,N] (bf16) = sum over segments of A_s[M,K_s] * B_s[N,K_s]^T, fp32 accumulate.
// gated: C = silu(A B^T) * (A B3^T) with B = gate rows, B3 = up rows.
struct GemmSeg {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  const uint16_t* B3;
  int64_t ldb;
  int K;
};

// Cf != NULL (plain GEMMs only): C is written as fp32 to Cf (C is ignored), and
// N may be any positive number; otherwise N is a multiple of 8 (tiled) or 32
// (few-row).
struct DenseGemm {
  int M, N;
  int nseg;
  GemmSeg seg[1 + 4];
  bool gated;
  uint16_t* C;
  float* Cf;
  int64_t ldc;
  // optional (dense_gemm_quant_fits): C's MXFP8 copy as well, codes [M, N]
  // (row stride ldc) and e8m0 scales [M, N/32] (row stride ldc/32), each
  // 32-column block quantised from the bf16 values written to C
  uint8_t* Cq = nullptr;
  uint8_t* Cqs = nullptr;
  // C written with the nontemporal hint (the 64-wide ring form).  The layer
  // sets it on its dense projections: they are MFMA-bound, and output lines
  // left dirty in the caches would be written back during the bandwidth-bound
  // grouped FC1 that follows (its prefill time 728 -> 699 us; the dense
  // launches +5 us in all, traced alternately)
  bool stream_c = false;
};
hipError_t launch_dense_gemm(const DenseGemm& g, hipStream_t s);
// compute units of the current device (cached per device; 256 if unknown)
int device_cus();
// Whether launch_dense_gemm writes the MXFP8 copy for this GEMM (a plain
// GEMM on the 64-wide ring with N and ldc multiples of 32); otherwise the
// caller quantises C itself.
bool dense_gemm_quant_fits(const DenseGemm& g);
// Few-row variant (M <= kSmallM): 16-row tiles, K split across the 4 waves of
// a workgroup; up to two sub-GEMMs with the same M in one launch.
constexpr int kSmallM = 512;
hipError_t launch_small_dense(const DenseGemm* parts, int nparts, hipStream_t s);
// The same GEMMs with the router's top-k of T tokens (as launch_router, E <=
// 1024) in the same launch: the router's workgroups run beside the GEMM's.
struct FrontRoute {
  const float* logits;
  int64_t T;
  int E, k;
  int32_t* ids;
  float* w;
};
hipError_t launch_small_dense_with_router(const DenseGemm* parts, int nparts, const FrontRoute& r, hipStream_t s);

// Grouped over experts: for each tile (expert e, rows p in the tile):
//   C[p, :] = A[row(p)] * B_e^T  (gated: silu(A B_e^T) * (A B3_e^T)),
//   row(p) = a_rows ? a_rows[p] / a_row_div : p,   B_e = B + e * b_estride.
// Tile-packed bf16 expert weights (latent_moe_pack_weights): element (e, n, k)
// of an [E, N, K] matrix sits at
//   (((e * N/kPackRows + n/kPackRows) * K/64 + k/64) * kPackRows + n%kPackRows) * 64 + k%64,
// so the 64 K columns of 128 consecutive rows that a tile's stage reads are
// one 16 KB block.  N a multiple of kPackRows, K of 64.
constexpr int kPackRows = 128;
hipError_t launch_pack_weights(const uint16_t* src, uint16_t* dst, int E, int N, int K, hipStream_t s);

struct GroupedGemm {
  int N, K;
  const uint16_t* A;
  int64_t lda;
  const int32_t* a_rows;
  int a_row_div;
  const uint16_t* B;
  const uint16_t* B3;
  int64_t ldb;
  int64_t b_estride;
  bool gated;
  uint16_t* C;
  int64_t ldc;
  const Tile* tiles;
  const int32_t* ntiles;
  int64_t max_tiles;
  // output-stationary launches (no tile table): the routed expert of every
  // (token, slot) row r = t*k + j, and the row count
  const int32_t* os_ids;
  int64_t os_R;
  bool packed;  // B and B3 in the tile-packed layout (b_estride = N*K, ldb unused)
  // w4a16 (launch_grouped_tiled only): B and B3 point to e2m1 codes [E, N, K/2]
  // (even K in the low nibble) with e8m0 scales Bs / B3s [E, N, K/32], upcast
  // to bf16 on their way into LDS; ldb and b_estride are unused
  bool w4;
  const uint8_t* Bs;
  const uint8_t* B3s;
  // rows of A (0: unknown); the w4a16 ring form addresses A by 32-bit
  // offsets and is used only when A's rows end below 2^31 bytes
  int64_t a_rows_n = 0;
};
hipError_t launch_grouped_skinny(const GroupedGemm& g, hipStream_t s, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// Output-stationary decode (TokenSpeed Day-0 post, "Gluon kernels on AMD GPUs >
// Stable LatentMoE": organised around outputs, no route sorting, padding or
// gather buffers): workgroup (expert e, 64 output columns) finds the rows r
// with os_ids[r] == e by scanning os_ids and computes C[r, cols] =
// A[r / a_row_div] * B_e^T (gated: SwiGLU) for them, 16 rows at a time, in
// (token, slot) order.  K a multiple of 128; os_R <= kOsMaxRows.
constexpr int kOsMaxRows = 8192;
hipError_t launch_grouped_skinny_os(const GroupedGemm& g, int E, hipStream_t s, hipEvent_t t0 = nullptr,
                                    hipEvent_t t1 = nullptr);
hipError_t launch_grouped_tiled(const GroupedGemm& g, hipStream_t s, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

// Grouped, decode-shaped, MXFP4 weights with bf16 activations (w4a16): as
// GroupedGemm with the skinny tile table, but B / B3 are e2m1 codes [E, N, K/2]
// (even K in the low nibble) with e8m0 scales Bs / B3s [E, N, K/32], upcast to
// bf16 in registers.  K is a multiple of 128.
struct GroupedW4 {
  int N, K;
  const uint16_t* A;
  int64_t lda;
  const int32_t* a_rows;
  int a_row_div;
  const uint8_t* B;
  const uint8_t* Bs;
  const uint8_t* B3;
  const uint8_t* B3s;
  bool gated;
  uint16_t* C;
  int64_t ldc;
  const Tile* tiles;
  const int32_t* ntiles;
  int64_t max_tiles;
};
hipError_t launch_grouped_w4a16(const GroupedW4& g, hipStream_t s, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// The whole w4a16 expert MLP (FC1, SwiGLU, FC2) in one launch, for latent =
// intermediate = 256 (kW4MlpWidth): Y [rows, 256] from A rows gathered as in
// GroupedGemm and the three MXFP4 matrices; H stays in LDS.
constexpr int kW4MlpWidth = 256;
struct W4Mlp {
  const uint16_t* A;
  int64_t lda;
  const int32_t* a_rows;
  int a_row_div;
  const uint8_t* W1;
  const uint8_t* S1;
  const uint8_t* W3;
  const uint8_t* S3;
  const uint8_t* W2;
  const uint8_t* S2;
  uint16_t* Y;
  int64_t ldy;
  const Tile* tiles;
  const int32_t* ntiles;
  int64_t max_tiles;
  const int32_t* os_ids;  // output-stationary launches, as in GroupedGemm
  int64_t os_R;
};
hipError_t launch_w4a16_mlp(const W4Mlp& g, hipStream_t s, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// The same MLP output-stationary: one workgroup per expert, rows found by
// scanning os_ids, Y in (token, slot) order.
hipError_t launch_w4a16_mlp_os(const W4Mlp& g, int E, hipStream_t s, hipEvent_t t0 = nullptr,
                               hipEvent_t t1 = nullptr);

// ---- MXFP4 (w4a8) expert path ------------------------------------------------
// bf16 [rows, K] -> MXFP8 e4m3 codes [rows, K] + e8m0 scales [rows, K/32].
hipError_t launch_quant_mxfp8(const uint16_t* src, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);
// Grouped block-scaled GEMM: MXFP8 activations (rows gathered as in
// GroupedGemm) x MXFP4 weights [E, N, K/2] with scales [E, N, K/32]; bf16
// output (gated: SwiGLU of gate and up), or with Cq set the output rounded to
// bf16 and then MXFP8-quantised as launch_quant_mxfp8 would.  Tiles from the
// 256-row table.
struct GroupedMx {
  int N, K;
  const uint8_t* A;
  const uint8_t* As;
  const int32_t* a_rows;
  int a_row_div;
  const uint8_t* B;
  const uint8_t* Bs;
  const uint8_t* B3;
  const uint8_t* B3s;
  bool gated;
  uint16_t* C;
  int64_t ldc;
  uint8_t* Cq = nullptr;   // non-NULL: output written as MXFP8 codes [rows, N] (row stride ldc)
  uint8_t* Cqs = nullptr;  //   and e8m0 scales [rows, N/32]; C is then not written
  const Tile* tiles;
  const int32_t* ntiles;
  int64_t max_tiles;
  int64_t a_rows_n = 0;  // rows of A (and As); 0: unknown
};
hipError_t launch_grouped_mx(const GroupedMx& g, hipStream_t s, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

// ---- combine ----------------------------------------------------------------
// out[t] = bf16(RMSNorm(sum_j w[t,j] Y[row_pos[t*k+j]]))   (norm skipped if gain == NULL;
// row_pos == NULL: Y rows in (token, slot) order)
hipError_t launch_combine(const uint16_t* Y, const int32_t* row_pos, const float* w, int64_t T, int k,
                          int l, const uint16_t* gain, float eps, uint16_t* out, hipStream_t s);

}  // namespace lmoe
