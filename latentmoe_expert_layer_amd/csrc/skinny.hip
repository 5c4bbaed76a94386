// Decode-shaped grouped expert GEMMs (gfx950): every expert sees a handful of
// rows (256 tokens x top-16 over 896 experts is ~4.6 rows each), so the cost
// is streaming each touched expert's weights from HBM once (vLLM Kimi K3
// post, section 1: the experts run in the latent space; TokenSpeed Day-0
// post, "TensorRT-LLM Stable LatentMoE": FC1 with its gate as one gated GEMM,
// then FC2).  Each wave keeps a whole K chunk of loads in flight and the
// operands go straight from registers into the MFMAs, with no LDS.
#include "common.h"
#include "kernels.h"
#include "permute_core.h"

namespace lmoe {

namespace {

// ------------------------------------------------- output-stationary rows ---
// The rows of one expert, found without a permutation: thread t of the
// 256-thread workgroup looks at ids [t*per, t*per + per) (per a multiple of 4,
// at most 32), keeps a bit mask of the ones equal to the expert, and a block
// scan of the counts gives each thread the rank of its first match, so the
// rows come out in ascending r (the order the permutation would give).  Ids
// past R are -1 and never match.
struct OsRows {
  uint32_t mask;  // matches among this thread's ids
  int32_t pre;    // matches in the threads before this one
  int32_t n;      // matches in the batch
  int32_t base;   // first id index of this thread
};

// The ids this thread looks at, loaded (positions past R read as -1).  Split
// from the ranking below so that a kernel can issue these loads, then its
// weight loads (which do not depend on the rows), and rank while both are
// in flight.
struct OsIds {
  int4 v[8];
  int per, base;
};

__device__ __forceinline__ OsIds os_load(const int32_t* __restrict__ ids, int64_t R) {
  OsIds d;
  d.per = int(((R + 1023) / 1024) * 4);  // ids per thread: 4 * ceil(R / 1024) <= 32
  d.base = int(threadIdx.x) * d.per;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    d.v[q] = int4{-1, -1, -1, -1};
    const int64_t r = int64_t(d.base) + 4 * q;
    if (4 * q < d.per) {
      if (r + 3 < R) {
        d.v[q] = *reinterpret_cast<const int4*>(ids + r);
      } else {
        if (r < R) d.v[q].x = ids[r];
        if (r + 1 < R) d.v[q].y = ids[r + 1];
        if (r + 2 < R) d.v[q].z = ids[r + 2];
      }
    }
  }
  return d;
}

__device__ __forceinline__ OsRows os_rank(const OsIds& d, int e, int32_t* red) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  OsRows o{};
  o.base = d.base;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    o.mask |= uint32_t(d.v[q].x == e) << (4 * q) | uint32_t(d.v[q].y == e) << (4 * q + 1) |
              uint32_t(d.v[q].z == e) << (4 * q + 2) | uint32_t(d.v[q].w == e) << (4 * q + 3);
  const int cnt = __popc(o.mask);
  const int incl = wave_incl_scan(cnt);
  if (lane == 63) red[wid] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int v = red[w];
    before += w < wid ? v : 0;
    total += v;
  }
  o.pre = before + incl - cnt;
  o.n = total;
  return o;
}

// Rows of ranks [c0, c0 + 16) of the scan into lst[0..15].
__device__ __forceinline__ void os_chunk(const OsRows& o, int c0, int32_t* lst) {
  const int cnt = __popc(o.mask);
  if (cnt && o.pre < c0 + 16 && o.pre + cnt > c0) {
    uint32_t m = o.mask;
    int rank = o.pre;
    while (m) {
      const int b = __builtin_ctz(m);
      if (rank >= c0 && rank < c0 + 16) lst[rank - c0] = o.base + b;
      ++rank;
      m &= m - 1;
    }
  }
}

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

// ------------------------------------------------------- skinny, LDS-staged ---
// The same tiles and outputs as skinny_grouped_kernel (bit-identical: the same
// MFMAs over the same K order), with the weight rows read 1 KB per load
// instruction: 4 rows x 256 B of a 128-wide K chunk, 16 lanes per row.  On the
// decode FC1 weights that pattern streams at ~6.2 TB/s against ~5.5 TB/s for
// loading the MFMA fragments directly (16 rows x 64 B per instruction).  Each
// wave turns a chunk into 16x16x32 B fragments through its own padded LDS
// block (16 rows x 272 B: the fragment reads of 16 lanes hit 16 distinct
// 16-byte bank groups).  Per batch of NCH chunks, the a_rows load, then every
// weight load and then every A load of the wave are issued before the first
// MFMA.
__device__ __forceinline__ void wave_lds_sync() {
  // the block is private to the wave, whose LDS accesses complete in order;
  // this only keeps the compiler from moving them across each other
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// One chunk of one weight matrix: 4 loaded uint4 per lane (lane l holds row
// 4i + l/16, 16-byte column l%16 of load i) -> LDS -> fragments of k-steps
// 0..3 -> 4 MFMAs with the matching A fragments.
__device__ __forceinline__ f32x4 lds_chunk_mfma(uint4* L, int lane, uint4 v0, uint4 v1, uint4 v2, uint4 v3,
                                                uint4 a0, uint4 a1, uint4 a2, uint4 a3, f32x4 acc) {
  wave_lds_sync();
  const int w = (lane >> 4) * 17 + (lane & 15);
  L[w] = v0;
  L[w + 4 * 17] = v1;
  L[w + 8 * 17] = v2;
  L[w + 12 * 17] = v3;
  wave_lds_sync();
  const int r = (lane & 15) * 17 + (lane >> 4);  // row n = lane%16, 16-byte column 4s + lane/16
  const uint4 f0 = L[r], f1 = L[r + 4], f2 = L[r + 8], f3 = L[r + 12];
  acc = mfma_16x16x32(as_bf16x8(a0), as_bf16x8(f0), acc);
  acc = mfma_16x16x32(as_bf16x8(a1), as_bf16x8(f1), acc);
  acc = mfma_16x16x32(as_bf16x8(a2), as_bf16x8(f2), acc);
  acc = mfma_16x16x32(as_bf16x8(a3), as_bf16x8(f3), acc);
  return acc;
}

// OS: the output-stationary form (no tile table): the grid is experts x
// column blocks, each workgroup scans the routed ids for its expert's rows
// and runs them 16 at a time; rows are written at their (token, slot) index.
// PACKED: the weights are in the tile-packed layout (kernels.h); a lane's 16
// bytes (row n, K k..k+7) are the same elements, at another address.
template <bool GATED, int NCH, bool OS = false, bool PACKED = false>
__global__ __launch_bounds__(256) void skinny_lds_kernel(GroupedGemm g) {
  __shared__ uint4 lds[4][16 * 17];
  __shared__ int32_t os_lst[OS ? 16 : 1];
  __shared__ int32_t os_red[OS ? 4 : 1];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles_n = g.N / 64;
  const int tm = int(blockIdx.x / uint32_t(tiles_n)), tn = int(blockIdx.x % uint32_t(tiles_n));
  int expert;
  Tile tl{};
  OsRows o{};
  OsIds oid;
  if constexpr (OS) {
    expert = tm;
    oid = os_load(g.os_ids, g.os_R);  // ranked below, once the first weight loads are out
  } else {
    const int ntiles = *g.ntiles;
    tl = g.tiles[tm];  // tm < max_tiles: inside the table even past the real count
    if (tm >= ntiles) return;
    expert = tl.expert;
  }
  for (int c0 = 0;; c0 += 16) {
    int nrows = 0;
    int64_t pos = 0;
    int32_t sr = 0;
    if constexpr (!OS) {
      nrows = tl.nrows;
      pos = int64_t(tl.row_start) + min(lane & 15, tl.nrows - 1);
      if (g.a_rows) sr = g.a_rows[pos];
    }
    // lane (row 4j + lane/16 of the wave's 16, 16-byte column lane%16 of a
    // 128-wide K chunk); uint4 offsets: rs per 4 rows, ks(k) for chunk k
    int64_t wb, lofs, rs;
    if constexpr (PACKED) {
      const int nb0 = tn * 64 + wid * 16;  // 16 rows inside one 128-row block
      wb = int64_t(expert) * g.b_estride + int64_t(nb0 / kPackRows) * g.K * kPackRows + (nb0 % kPackRows) * 64;
      lofs = int64_t((lane & 15) >> 3) * (kPackRows * 8) + (lane >> 4) * 8 + (lane & 7);
      rs = 4 * 8;
    } else {
      wb = int64_t(expert) * g.b_estride + int64_t(tn * 64 + wid * 16) * g.ldb;
      lofs = (lane >> 4) * (g.ldb / 8) + (lane & 15);
      rs = 4 * (g.ldb / 8);
    }
    auto ks = [&](int k) __attribute__((always_inline)) -> int64_t {
      return PACKED ? int64_t(k / 64) * (kPackRows * 8) : int64_t(k / 8);
    };
    const uint4* gp = reinterpret_cast<const uint4*>(g.B + wb) + lofs;
    const uint4* up = GATED ? reinterpret_cast<const uint4*>(g.B3 + wb) + lofs : nullptr;
    uint4* L = lds[wid];
    const bf16_t* ap = nullptr;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc3 = {0.f, 0.f, 0.f, 0.f};
    for (int kc = 0; kc < g.K; kc += 128 * NCH) {
      uint4 gv[NCH][4], uv[NCH][GATED ? 4 : 1], a[NCH][4];
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // the weights are read once per step: nontemporal (FC1 42.1 -> 37.8
          // us, FC2 22.1 -> 20.4 us at decode, traced alternately)
          gv[c][j] = ldnt16(gp + j * rs + ks(kc + 128 * c));
          if constexpr (GATED) uv[c][j] = ldnt16(up + j * rs + ks(kc + 128 * c));
        }
      __builtin_amdgcn_sched_barrier(0);
      if (kc == 0) {
        if constexpr (OS) {
          // the weights are in flight: rank this expert's rows (first chunk
          // only), then this chunk's list
          if (c0 == 0) {
            o = os_rank(oid, expert, os_red);
            if (o.n == 0) return;  // the whole workgroup: an expert no row picked
          }
          os_chunk(o, c0, os_lst);
          __syncthreads();
          nrows = min(16, o.n - c0);
          sr = os_lst[min(lane & 15, nrows - 1)];
          ap = g.A + int64_t(sr / g.a_row_div) * g.lda + (lane >> 4) * 8;
        } else {
          ap = g.A + (g.a_rows ? int64_t(sr / g.a_row_div) : pos) * g.lda + (lane >> 4) * 8;
        }
      }
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int s = 0; s < 4; ++s) a[c][s] = ldg16(ap + kc + 128 * c + 32 * s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        acc = lds_chunk_mfma(L, lane, gv[c][0], gv[c][1], gv[c][2], gv[c][3], a[c][0], a[c][1], a[c][2], a[c][3],
                             acc);
        if constexpr (GATED)
          acc3 = lds_chunk_mfma(L, lane, uv[c][0], uv[c][1], uv[c][2], uv[c][3], a[c][0], a[c][1], a[c][2],
                                a[c][3], acc3);
      }
    }
    const int nb = tn * 64 + wid * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (lane >> 4) * 4 + r;
      if (row < nrows) {
        float v = acc[r];
        if constexpr (GATED) v = silu_mul(v, acc3[r]);
        const int64_t orow = OS ? int64_t(os_lst[row]) : int64_t(tl.row_start) + row;
        g.C[orow * g.ldc + nb] = f32_to_bf16(v);
      }
    }
    if constexpr (!OS) break;
    if (c0 + 16 >= o.n) break;
    __syncthreads();  // every wave is done with this chunk's row list
  }
}

// ------------------------------------------------------ skinny w4a16 (MXFP4) ---
// TokenSpeed Day-0 post, "TensorRT-LLM Stable LatentMoE": w4a16 keeps the
// activations in bf16 and is the small-batch mode of the MXFP4 experts.  The
// layout of skinny_grouped_kernel (16-row tile; NS 16-column subtiles per
// wave, so a workgroup covers 64*NS columns), with the weights read as e2m1
// codes and upcast in registers by gfx950's scaled conversion (exact: an e2m1
// value times a power of two).  K is taken in chunks of 128: lane (n, gq) loads the 16 code bytes
// of row n at K offset 32*gq of the chunk and their one e8m0 scale, and k-step
// s of the chunk multiplies codes 8s .. 8s+7 of them, so lane gq of step s
// covers K = chunk + 32*gq + 8s .. +8; the A fragments take the same K order.

template <bool GATED, int NCH, int NS>
__global__ __launch_bounds__(256) void skinny_w4a16_kernel(GroupedW4 g) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int BCOLS = 64 * NS;  // output columns per workgroup (NS 16-column subtiles per wave)
  const int tiles_n = g.N / BCOLS;
  const uint32_t lt = blockIdx.x;
  const int tm = int(lt / uint32_t(tiles_n)), tn = int(lt % uint32_t(tiles_n));
  if (tm >= *g.ntiles) return;
  const Tile tl = g.tiles[tm];
  const int arow = min(lane & 15, tl.nrows - 1);
  int64_t src = int64_t(tl.row_start) + arow;
  if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
  const int gq = lane >> 4;
  const bf16_t* ap = g.A + src * g.lda + 32 * gq;
  const int nb = tn * BCOLS + wid * 16 * NS + (lane & 15);  // column of subtile 0
  const uint8_t* bp[NS];
  const uint8_t* sp[NS];
  const uint8_t* b3p[NS];
  const uint8_t* s3p[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int64_t wrow = int64_t(tl.expert) * g.N + nb + 16 * j;  // weight row of this lane
    bp[j] = g.B + wrow * (g.K / 2) + 16 * gq;
    sp[j] = g.Bs + wrow * (g.K / 32);
    b3p[j] = GATED ? g.B3 + wrow * (g.K / 2) + 16 * gq : nullptr;
    s3p[j] = GATED ? g.B3s + wrow * (g.K / 32) : nullptr;
  }
  f32x4 acc[NS], acc3[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc3[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int kc = 0; kc < g.K; kc += 128 * NCH) {
    uint4 a[NCH][4], b[NS][NCH], b3[NS][GATED ? NCH : 1];
    uint32_t sc[NS][NCH], sc3[NS][GATED ? NCH : 1];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int k0 = kc + 128 * c;
#pragma unroll
      for (int st = 0; st < 4; ++st) a[c][st] = ldg16(ap + k0 + 8 * st);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        b[j][c] = *reinterpret_cast<const uint4*>(bp[j] + k0 / 2);
        sc[j][c] = *reinterpret_cast<const uint32_t*>(sp[j] + k0 / 32);  // the chunk's 4 scales; byte gq is this lane's
        if constexpr (GATED) {
          b3[j][c] = *reinterpret_cast<const uint4*>(b3p[j] + k0 / 2);
          sc3[j][c] = *reinterpret_cast<const uint32_t*>(s3p[j] + k0 / 32);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const float f = e8m0_multiplier((sc[j][c] >> (8 * gq)) & 0xffu);
        const uint32_t w[4] = {b[j][c].x, b[j][c].y, b[j][c].z, b[j][c].w};
#pragma unroll
        for (int st = 0; st < 4; ++st)
          acc[j] = mfma_16x16x32(as_bf16x8(a[c][st]), fp4x8_to_bf16(w[st], f), acc[j]);
        if constexpr (GATED) {
          const float f3 = e8m0_multiplier((sc3[j][c] >> (8 * gq)) & 0xffu);
          const uint32_t w3[4] = {b3[j][c].x, b3[j][c].y, b3[j][c].z, b3[j][c].w};
#pragma unroll
          for (int st = 0; st < 4; ++st)
            acc3[j] = mfma_16x16x32(as_bf16x8(a[c][st]), fp4x8_to_bf16(w3[st], f3), acc3[j]);
        }
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

// Fused w4a16 expert MLP for the decode shape (latent = intermediate = 256):
// one workgroup per 16-row tile runs FC1, SwiGLU and FC2 with the tile's z
// rows and its H rows in LDS, so the expert's three weight matrices stream as
// one sequence and H never leaves the workgroup (TokenSpeed Day-0 post,
// "TensorRT-LLM Stable LatentMoE": the runner's FC1 then FC2 over the routed
// tokens).  Wave w owns H columns [64w, 64w+64) and Y columns [64w, 64w+64).
// Its weight loads form six chunks of 4 code loads (16 B) and 4 scale words,
// two in flight (at 124 registers four workgroups fit per CU, which holds a
// whole decode batch's tiles at once):
//   chunks 0..3 (FC1): H columns 32*(c>>1) .. +32 of the wave, K chunk c&1;
//     slot i = subtile i>>1, matrix i&1 (gate, up);
//   chunks 4, 5 (FC2): K chunk c-4; slot i = Y subtile i (16 columns).
// The K order within a 128-wide chunk is skinny_w4a16_kernel's, so H and Y
// are bit-identical to that two-launch path.
// OS: the output-stationary form, one workgroup per expert, its rows found by
// scanning the routed ids (16 at a time), Y written at (token, slot) rows.
template <bool OS = false>
__global__ __launch_bounds__(256) void skinny_w4a16_mlp_kernel(W4Mlp g) {
  constexpr int L = 256, IM = 256, ZS = L + 8, HS = IM + 8;  // padded LDS rows (bf16)
  static_assert(L == kW4MlpWidth && IM == kW4MlpWidth, "the chunk layout below is for 256 x 256");
  __shared__ __attribute__((aligned(16))) bf16_t Zs[16 * ZS];
  __shared__ __attribute__((aligned(16))) bf16_t Hs[16 * HS];
  __shared__ int32_t os_lst[OS ? 16 : 1];
  __shared__ int32_t os_red[OS ? 4 : 1];
  const int lane = threadIdx.x & 63, gq = lane >> 4, n16 = lane & 15;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, so row bases stay scalar
  int expert;
  Tile tl{};
  OsRows o{};
  OsIds oid;
  if constexpr (OS) {
    expert = int(blockIdx.x);
    oid = os_load(g.os_ids, g.os_R);  // ranked below, once the first weight loads are out
  } else {
    if (int(blockIdx.x) >= *g.ntiles) return;
    tl = g.tiles[blockIdx.x];
    expert = tl.expert;
  }
  const int64_t e1 = int64_t(expert) * IM, e2 = int64_t(expert) * L;
  // code rows are K/2 = 128 bytes and scale rows K/32 = 8 bytes for both
  // GEMMs; each load is a wave-uniform row base plus a 32-bit lane offset
  const uint32_t coff = uint32_t(n16) * 128u + 16u * uint32_t(gq), soff = uint32_t(n16) * 8u;
  auto load = [&](uint4 (&w)[4], uint32_t (&sc)[4], int c) __attribute__((always_inline)) {
    const bool f1 = c < 4;
    const int kc = f1 ? (c & 1) : (c - 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row0 = f1 ? e1 + wid * (IM / 4) + 32 * (c >> 1) + 16 * (i >> 1) : e2 + wid * (L / 4) + 16 * i;
      const uint8_t* cb = (f1 ? ((i & 1) ? g.W3 : g.W1) : g.W2) + row0 * 128;
      const uint8_t* sb = (f1 ? ((i & 1) ? g.S3 : g.S1) : g.S2) + row0 * 8;
      w[i] = *reinterpret_cast<const uint4*>(cb + (coff + 64u * uint32_t(kc)));
      sc[i] = *reinterpret_cast<const uint32_t*>(sb + (soff + 4u * uint32_t(kc)));  // byte gq is this lane's
    }
  };
  for (int c0 = 0;; c0 += 16) {
  int nrows = OS ? 0 : tl.nrows;
  // FC1: acc[2j] gate and acc[2j+1] up of H subtile j; FC2: acc[j] of Y subtile j
  f32x4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const uint4 (&w)[4], const uint32_t (&sc)[4], int c) __attribute__((always_inline)) {
    const bool f1 = c < 4;
    const int kc = f1 ? (c & 1) : (c - 4);
    if (!f1 && kc == 0) __syncthreads();  // every wave's H columns are in LDS
    const bf16_t* As = f1 ? Zs : Hs;
    const int AS = f1 ? ZS : HS;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&As[n16 * AS + 128 * kc + 32 * gq + 8 * st]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
        acc[i] = mfma_16x16x32(a, fp4x8_to_bf16(ww[st], e8m0_multiplier((sc[i] >> (8 * gq)) & 0xffu)), acc[i]);
      }
    }
    if (kc == 1) {
      if (f1) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Hs[(4 * gq + r) * HS + wid * (IM / 4) + 32 * (c >> 1) + 16 * j + n16] =
                f32_to_bf16(silu_mul(acc[2 * j][r], acc[2 * j + 1][r]));
      } else {
        // Y through LDS (the z rows' buffer, free since FC1 ended), so that a
        // wave writes each of its rows' 128 bytes as one 16-byte-per-lane
        // store: full lines, not 32-byte pieces
        bf16_t* Ys = Zs + wid * (L / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) Ys[(4 * gq + r) * ZS + 16 * j + n16] = f32_to_bf16(acc[j][r]);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();  // (the wave reads back only its own columns)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int row = 8 * q + (lane >> 3);
          if (row < nrows) {
            const int64_t orow = OS ? int64_t(os_lst[row]) : int64_t(tl.row_start) + row;
            *reinterpret_cast<uint4*>(g.Y + orow * g.ldy + wid * (L / 4) + 8 * (lane & 7)) =
                *reinterpret_cast<const uint4*>(&Ys[row * ZS + 8 * (lane & 7)]);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  uint4 w0[4], w1[4];
  uint32_t s0[4], s1[4];
  load(w0, s0, 0);
  load(w1, s1, 1);
  if constexpr (OS) {
    // the first weight chunks are in flight: rank this expert's rows (first
    // chunk only), then this chunk's list
    if (c0 == 0) {
      o = os_rank(oid, expert, os_red);
      if (o.n == 0) return;
    }
    os_chunk(o, c0, os_lst);
    __syncthreads();
    nrows = min(16, o.n - c0);
  }
  // the tile's z rows (gathered) into LDS while the first two chunks load
  for (int i = threadIdx.x; i < 16 * (L / 8); i += 256) {
    const int r = i / (L / 8), cq = i % (L / 8);
    int64_t src;
    if constexpr (OS) {
      src = os_lst[min(r, nrows - 1)] / g.a_row_div;
    } else {
      src = int64_t(tl.row_start) + min(r, tl.nrows - 1);
      if (g.a_rows) src = g.a_rows[src] / g.a_row_div;
    }
    *reinterpret_cast<uint4*>(&Zs[r * ZS + cq * 8]) = ldg16(g.A + src * g.lda + cq * 8);
  }
  __syncthreads();
  compute(w0, s0, 0);
  load(w0, s0, 2);
  compute(w1, s1, 1);
  load(w1, s1, 3);
  compute(w0, s0, 2);
  load(w0, s0, 4);
  compute(w1, s1, 3);
  load(w1, s1, 5);
  compute(w0, s0, 4);
  compute(w1, s1, 5);
  if constexpr (!OS) break;
  if (c0 + 16 >= o.n) break;
  __syncthreads();  // every wave is done with this chunk's rows (Zs, Hs, the list)
  }
}

}  // namespace

hipError_t launch_grouped_w4a16(const GroupedW4& g, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  // 16-column subtiles per wave: two for the gated FC1 (two weight matrices
  // per subtile), four for FC2 (measured best at the decode shape), fewer
  // when N does not divide
  const int want = g.gated ? 2 : 4;
  const int ns = want == 4 && g.N % 256 == 0 ? 4 : (g.N % 128 == 0 ? 2 : 1);
  const int64_t nblk = g.max_tiles * (g.N / (64 * ns));
  if (nblk <= 0) return hipSuccess;
  const dim3 grid{uint32_t(nblk)}, block{256};
  const bool two = g.K % 256 == 0;
  const void* kern;
#define LMOE_W4_PICK(NS_)                                                                                 \
  kern = g.gated ? (two ? (const void*)skinny_w4a16_kernel<true, 2, NS_> : (const void*)skinny_w4a16_kernel<true, 1, NS_>) \
                 : (two ? (const void*)skinny_w4a16_kernel<false, 2, NS_> : (const void*)skinny_w4a16_kernel<false, 1, NS_>)
  if (ns == 4) {
    LMOE_W4_PICK(4);
  } else if (ns == 2) {
    LMOE_W4_PICK(2);
  } else {
    LMOE_W4_PICK(1);
  }
#undef LMOE_W4_PICK
  return launch_kernel(kern, grid, block, 0, s, g, t0, t1);
}

hipError_t launch_w4a16_mlp(const W4Mlp& g, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (g.max_tiles <= 0) return hipSuccess;
  // Y rows go out as 16-byte stores
  if (g.ldy % 8 || reinterpret_cast<uintptr_t>(g.Y) % 16) return hipErrorInvalidValue;
  return launch_kernel((const void*)skinny_w4a16_mlp_kernel<false>, dim3{uint32_t(g.max_tiles)}, dim3{256}, 0, s, g,
                       t0, t1);
}

hipError_t launch_w4a16_mlp_os(const W4Mlp& g, int E, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (g.os_R <= 0 || E <= 0) return hipSuccess;
  if (g.os_R > kOsMaxRows || !g.os_ids) return hipErrorInvalidValue;
  if (g.ldy % 8 || reinterpret_cast<uintptr_t>(g.Y) % 16) return hipErrorInvalidValue;
  return launch_kernel((const void*)skinny_w4a16_mlp_kernel<true>, dim3{uint32_t(E)}, dim3{256}, 0, s, g, t0, t1);
}

hipError_t launch_grouped_skinny_os(const GroupedGemm& g, int E, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (g.os_R <= 0 || E <= 0) return hipSuccess;
  if (g.os_R > kOsMaxRows || !g.os_ids || g.K % 128 != 0 || g.N % 64 != 0) return hipErrorInvalidValue;
  const dim3 grid{uint32_t(int64_t(E) * (g.N / 64))}, block{256};
  const void* kern;
  if (g.packed) {
    kern = g.gated ? (g.K % 256 == 0 ? (const void*)skinny_lds_kernel<true, 2, true, true>
                                     : (const void*)skinny_lds_kernel<true, 1, true, true>)
                   : (g.K % 256 == 0 ? (const void*)skinny_lds_kernel<false, 2, true, true>
                                     : (const void*)skinny_lds_kernel<false, 1, true, true>);
  } else {
    kern = g.gated ? (g.K % 256 == 0 ? (const void*)skinny_lds_kernel<true, 2, true>
                                     : (const void*)skinny_lds_kernel<true, 1, true>)
                   : (g.K % 256 == 0 ? (const void*)skinny_lds_kernel<false, 2, true>
                                     : (const void*)skinny_lds_kernel<false, 1, true>);
  }
  return launch_kernel(kern, grid, block, 0, s, g, t0, t1);
}

hipError_t launch_grouped_skinny(const GroupedGemm& g, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const int64_t nblk = g.max_tiles * (g.N / 64);
  if (nblk <= 0) return hipSuccess;
  const dim3 grid{uint32_t(nblk)}, block{256};
  const void* kern;
  if (g.packed) {
    if (g.K % 128) return hipErrorInvalidValue;  // the tile-packed layout runs on the LDS-staged kernel
    kern = g.gated ? (g.K % 256 == 0 ? (const void*)skinny_lds_kernel<true, 2, false, true>
                                     : (const void*)skinny_lds_kernel<true, 1, false, true>)
                   : (g.K % 256 == 0 ? (const void*)skinny_lds_kernel<false, 2, false, true>
                                     : (const void*)skinny_lds_kernel<false, 1, false, true>);
  } else if (g.gated) {
    kern = g.K % 256 == 0   ? (const void*)skinny_lds_kernel<true, 2>
           : g.K % 128 == 0 ? (const void*)skinny_lds_kernel<true, 1>
                            : (const void*)skinny_grouped_kernel<true, 2, 1>;
  } else {
    kern = g.K % 256 == 0   ? (const void*)skinny_lds_kernel<false, 2>
           : g.K % 128 == 0 ? (const void*)skinny_lds_kernel<false, 1>
                            : (const void*)skinny_grouped_kernel<false, 2, 1>;
  }
  return launch_kernel(kern, grid, block, 0, s, g, t0, t1);
}

}  // namespace lmoe
