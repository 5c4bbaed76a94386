// Router (top-k + softmax) and the stable per-expert permutation.
//
// Router: each token picks k of E routed experts (TokenSpeed AgentX post,
// "Model architecture": 16 of 896), ranked by (logit descending, expert index
// ascending); the combine weights are the softmax over the k selected logits.
// Permutation: the route sorting / gather metadata that a grouped-GEMM MoE
// builds (TokenSpeed Day-0 post, "Gluon kernels on AMD GPUs > Stable
// LatentMoE"), here a stable counting sort of rows r = t*k + j by expert.
#include "common.h"
#include "kernels.h"
#include "permute_core.h"
#include "router_core.h"

namespace lmoe {

// ----------------------------------------------------------------- router ---
// One wave per token; lane l holds logits e = l + 64*j (coalesced rows).
template <int VPL>
__global__ __launch_bounds__(256) void router_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                     int k, int32_t* __restrict__ ids,
                                                     float* __restrict__ w) {
  __shared__ uint64_t cbuf[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = int64_t(blockIdx.x) * 4 + wv;
  if (t >= T) return;
  route_token<VPL>(logits, t, E, k, lane, cbuf[wv], ids, w);
}

hipError_t launch_router(const float* logits, int64_t T, int E, int k, int32_t* ids, float* w,
                         hipStream_t s) {
  const dim3 grid{uint32_t((T + 3) / 4)}, block{256};
  if (E <= 128) router_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 256) router_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 512) router_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else router_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

__global__ void copy_ids_kernel(const int32_t* __restrict__ ids_in, const float* __restrict__ w_in,
                                int64_t n, int32_t* __restrict__ ids, float* __restrict__ w) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) {
    if (ids) ids[i] = ids_in[i];
    if (w) w[i] = w_in[i];
  }
}

hipError_t launch_copy_ids(const int32_t* ids_in, const float* w_in, int64_t n, int32_t* ids, float* w,
                           hipStream_t s) {
  copy_ids_kernel<<<dim3(uint32_t((n + 255) / 256)), dim3(256), 0, s>>>(ids_in, w_in, n, ids, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------- permute ---
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

constexpr int kPermLdsBudget = 150 * 1024;

int permute_waves(int E) {
  for (int w = 16; w >= 8; w >>= 1)
    if (permute_lds_bytes(E, w) <= kPermLdsBudget) return w;
  return 0;
}

// Small batches: one 1024-thread workgroup (permute_block).
template <int NW, bool MASKS = false>
__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_row, int32_t* __restrict__ row_pos, Tile* __restrict__ tiles_a,
    int32_t* __restrict__ n_a, Tile* __restrict__ tiles_b, int32_t* __restrict__ n_b) {
  extern __shared__ uint64_t lds64[];
  permute_block<NW, kPermThreads, MASKS>(ids, R, E, offsets, sorted_row, row_pos, tiles_a, n_a, tiles_b, n_b,
                                         reinterpret_cast<int32_t*>(lds64));
}

// -------------------------------------------------- permute, large batches ---
// Above kPermOneWgMaxRows rows one workgroup is too slow (its waves walk
// R/16 rows each), so the same three phases run over G = ceil(R / kPermChunk)
// workgroups that each own kPermChunk consecutive rows, with the per-chunk
// counts in a global scratch array counts[G][E]:
//   count:   counts[g][e] = rows of expert e in chunk g;
//   scan:    one workgroup turns every counts[.][e] into its exclusive prefix
//            over chunks and scans the per-expert totals and tile counts
//            (offsets, both tile tables);
//   scatter: chunk g re-reads its ids, splits them over its waves as the
//            one-workgroup kernel does, and starts expert e's rows at
//            offsets[e] + counts[g][e].
// Chunks are consecutive and each keeps its rows in order, so the result is
// the same stable permutation.
constexpr int kPermChunk = 4096;
// the scan leaves an expert's tile-table entries to the whole workgroup when
// it has more 16-row tiles than this (up to kPermHeavyMax such experts)
constexpr int kPermSerialTiles = 64;
constexpr int kPermHeavyMax = 1024;
constexpr int64_t kPermOneWgMaxRows = 8192;
constexpr int kPermMaxExperts = 4096;  // the scan's threads own at most 4 experts each

int64_t permute_scratch_ints(int64_t R, int E) {
  if (R <= kPermOneWgMaxRows) return 0;
  return ((R + kPermChunk - 1) / kPermChunk) * int64_t(E);
}

__global__ __launch_bounds__(kPermThreads) void permute_count_kernel(const int32_t* __restrict__ ids, int64_t R,
                                                                     int E, int32_t* __restrict__ counts) {
  extern __shared__ int32_t lds[];  // [E]
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPermThreads) lds[e] = 0;
  __syncthreads();
  constexpr int PER = kPermChunk / kPermThreads;
  const int64_t r0 = int64_t(blockIdx.x) * kPermChunk + tid;
  int32_t v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) v[u] = ids[min(r0 + int64_t(u) * kPermThreads, R - 1)];
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (r0 + int64_t(u) * kPermThreads < R) atomicAdd(&lds[clamp_id(v[u], E)], 1);
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) counts[int64_t(blockIdx.x) * E + e] = lds[e];
}

__global__ __launch_bounds__(kPermThreads) void permute_scan_kernel(
    int32_t* __restrict__ counts, int G, int64_t R, int E, int32_t* __restrict__ offsets,
    Tile* __restrict__ tiles_a, int32_t* __restrict__ n_a, Tile* __restrict__ tiles_b, int32_t* __restrict__ n_b) {
  __shared__ int32_t ws[3 * kPermWaves];
  // experts with more than kPermSerialTiles 16-row tiles, whose tile-table
  // entries the whole workgroup writes: (expert, row offset, rows, first
  // entry of each table)
  __shared__ int32_t s_nheavy;
  __shared__ int32_t s_heavy[kPermHeavyMax][5];
  constexpr int kMaxPer = kPermMaxExperts / kPermThreads;
  constexpr int kG = 16;  // chunk counts loaded together
  const int tid = threadIdx.x;
  if (tid == 0) s_nheavy = 0;  // ordered before its use by the scan's barrier
  const int per = (E + kPermThreads - 1) / kPermThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int32_t tot[kMaxPer];
  int32_t run[3] = {0, 0, 0};
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q) {
    const int e = e0 + q;
    tot[q] = 0;
    if (e < e1) {
      int32_t c = 0;
      for (int g0 = 0; g0 < G; g0 += kG) {
        int32_t v[kG];
#pragma unroll
        for (int u = 0; u < kG; ++u) v[u] = counts[int64_t(min(g0 + u, G - 1)) * E + e];
#pragma unroll
        for (int u = 0; u < kG; ++u)
          if (g0 + u < G) {
            counts[int64_t(g0 + u) * E + e] = c;
            c += v[u];
          }
      }
      tot[q] = c;
      run[0] += c;
      run[1] += (c + kSkinnyBM - 1) / kSkinnyBM;
      run[2] += (c + kTiledBM - 1) / kTiledBM;
    }
  }
  const Scan3 sc = block_exclusive_scan3<kPermWaves>(run, ws);
  int32_t o = sc.x[0], ta = sc.x[1], tb = sc.x[2];
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q) {
    const int e = e0 + q;
    if (e < e1) {
      const int32_t cnt = tot[q];
      offsets[e] = o;
      const int32_t na = (cnt + kSkinnyBM - 1) / kSkinnyBM, nb = (cnt + kTiledBM - 1) / kTiledBM;
      // a long run of entries (a skewed load) is left to the whole workgroup
      // below, while the list has room
      const int h = na > kPermSerialTiles ? atomicAdd(&s_nheavy, 1) : kPermHeavyMax;
      if (h < kPermHeavyMax) {
        s_heavy[h][0] = e;
        s_heavy[h][1] = o;
        s_heavy[h][2] = cnt;
        s_heavy[h][3] = ta;
        s_heavy[h][4] = tb;
        ta += na;
        tb += nb;
      } else {
        for (int32_t r = 0; r < cnt; r += kSkinnyBM, ++ta)
          tiles_a[ta] = Tile{e, o + r, min(kSkinnyBM, cnt - r), cnt <= kSkinnyBM};
        for (int32_t r = 0; r < cnt; r += kTiledBM, ++tb)
          tiles_b[tb] = Tile{e, o + r, min(kTiledBM, cnt - r), cnt <= kTiledBM};
      }
      o += cnt;
    }
  }
  if (tid == 0) {
    offsets[E] = int32_t(R);
    *n_a = sc.total[1];
    *n_b = sc.total[2];
  }
  lds_barrier();  // the heavy list; the stores above need not land first
  const int nh = min(s_nheavy, kPermHeavyMax);
  for (int h = 0; h < nh; ++h) {
    const int e = s_heavy[h][0];
    const int32_t oe = s_heavy[h][1], cnt = s_heavy[h][2], ta0 = s_heavy[h][3], tb0 = s_heavy[h][4];
    for (int32_t j = tid; j * kSkinnyBM < cnt; j += kPermThreads)
      tiles_a[ta0 + j] = Tile{e, oe + j * kSkinnyBM, min(kSkinnyBM, cnt - j * kSkinnyBM), cnt <= kSkinnyBM};
    for (int32_t j = tid; j * kTiledBM < cnt; j += kPermThreads)
      tiles_b[tb0 + j] = Tile{e, oe + j * kTiledBM, min(kTiledBM, cnt - j * kTiledBM), cnt <= kTiledBM};
  }
}

template <int NW, bool MASKS = false>
__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_row, int32_t* __restrict__ row_pos) {
  constexpr int S = NW + 1;
  extern __shared__ uint64_t lds64[];  // MASKS: [NW][E] lane masks, then [E][S]
  uint64_t* masks = lds64;
  int32_t* hist = reinterpret_cast<int32_t*>(lds64 + (MASKS ? int64_t(NW) * E : 0));
  const int tid = threadIdx.x, wid = tid >> 6;
  if constexpr (MASKS)
    for (int i = tid; i < NW * E; i += kPermThreads) masks[i] = 0ull;
  for (int i = tid; i < E * S; i += kPermThreads) hist[i] = 0;
  __syncthreads();
  constexpr int64_t kWaveRows = kPermChunk / NW;
  static_assert(kWaveRows % 64 == 0, "whole 64-row steps per wave");
  const int64_t c0 = int64_t(blockIdx.x) * kPermChunk, c1 = min(R, c0 + kPermChunk);
  const int64_t r0 = min(c1, c0 + wid * kWaveRows), r1 = min(c1, r0 + kWaveRows);
  int32_t first[kPermBatch];
  if (wid < NW) wave_histogram<NW>(ids, R, E, r0, r1, first, hist);
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) {
    int32_t c[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) c[w] = hist[e * S + w];
    int32_t start = offsets[e] + counts[int64_t(blockIdx.x) * E + e];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      hist[e * S + w] = start;
      start += c[w];
    }
  }
  __syncthreads();
  if (wid < NW) stable_scatter<NW, MASKS>(ids, R, E, r0, r1, first, hist, sorted_row, row_pos, masks);
}

template <int NW>
static hipError_t launch_permute_nw(const int32_t* ids, int64_t R, int E, int32_t* offsets,
                                    int32_t* sorted_row, int32_t* row_pos, Tile* tiles_a, int32_t* n_a,
                                    Tile* tiles_b, int32_t* n_b, int32_t* scratch, hipStream_t s) {
  if (hipError_t e = allow_dynamic_lds((const void*)permute_kernel<NW>, kPermLdsBudget); e != hipSuccess) return e;
  if (hipError_t e = allow_dynamic_lds((const void*)permute_scatter_kernel<NW>, kPermLdsBudget); e != hipSuccess)
    return e;
  if (R <= kPermOneWgMaxRows) {
    // the mask form of the scatter (8 row-splitting waves) where its masks fit
    const int64_t mlds = permute_masks_bytes(E, 8) + permute_lds_bytes(E, 8);
    if (mlds <= kPermLdsBudget) {
      if (hipError_t e = allow_dynamic_lds((const void*)permute_kernel<8, true>, kPermLdsBudget); e != hipSuccess)
        return e;
      permute_kernel<8, true><<<dim3(1), dim3(kPermThreads), size_t(mlds), s>>>(ids, R, E, offsets, sorted_row,
                                                                                  row_pos, tiles_a, n_a, tiles_b, n_b);
      return hipGetLastError();
    }
    permute_kernel<NW><<<dim3(1), dim3(kPermThreads), size_t(permute_lds_bytes(E, NW)), s>>>(
        ids, R, E, offsets, sorted_row, row_pos, tiles_a, n_a, tiles_b, n_b);
    return hipGetLastError();
  }
  if (!scratch) return hipErrorInvalidValue;
  const int64_t G = (R + kPermChunk - 1) / kPermChunk;
  permute_count_kernel<<<dim3(uint32_t(G)), dim3(kPermThreads), size_t(E) * 4, s>>>(ids, R, E, scratch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  permute_scan_kernel<<<dim3(1), dim3(kPermThreads), 0, s>>>(scratch, int(G), R, E, offsets, tiles_a, n_a, tiles_b,
                                                             n_b);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t mlds = permute_masks_bytes(E, 8) + permute_lds_bytes(E, 8);
  if (mlds <= kPermLdsBudget) {  // the mask form of the scatter where its masks fit
    if ((e = allow_dynamic_lds((const void*)permute_scatter_kernel<8, true>, kPermLdsBudget)) != hipSuccess) return e;
    permute_scatter_kernel<8, true><<<dim3(uint32_t(G)), dim3(kPermThreads), size_t(mlds), s>>>(
        ids, R, E, scratch, offsets, sorted_row, row_pos);
    return hipGetLastError();
  }
  permute_scatter_kernel<NW><<<dim3(uint32_t(G)), dim3(kPermThreads), size_t(permute_lds_bytes(E, NW)), s>>>(
      ids, R, E, scratch, offsets, sorted_row, row_pos);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int64_t R, int E, int32_t* offsets, int32_t* sorted_row,
                          int32_t* row_pos, Tile* tiles_a, int32_t* n_a, Tile* tiles_b, int32_t* n_b,
                          int32_t* scratch, hipStream_t s) {
  switch (permute_waves(E)) {
    case 16:
      return launch_permute_nw<16>(ids, R, E, offsets, sorted_row, row_pos, tiles_a, n_a, tiles_b, n_b, scratch, s);
    case 8:
      return launch_permute_nw<8>(ids, R, E, offsets, sorted_row, row_pos, tiles_a, n_a, tiles_b, n_b, scratch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lmoe
