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

// Expert ids outside [0, E) (invalid input) are clamped so that every write
// stays inside the caller's buffers; valid ids are unchanged.
__device__ __forceinline__ int32_t clamp_id(int32_t id, int E) { return min(max(id, 0), E - 1); }
constexpr int kPermLdsBudget = 150 * 1024;

// LDS of the permute kernel: the [E][NW+1] histogram plus the scan scratch.
static int64_t permute_lds_bytes(int E, int nw) { return (int64_t(E) * (nw + 1) + 64) * 4; }

int permute_waves(int E) {
  for (int w = 16; w >= 8; w >>= 1)
    if (permute_lds_bytes(E, w) <= kPermLdsBudget) return w;
  return 0;
}

// Inclusive wave scan (sum) with DPP: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then row 0's total into row 1 and row 2's into row 3, then the
// total of rows 0-1 into rows 2 and 3.  Lanes without a source read 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int32_t dpp_add(int32_t v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
  v = dpp_add<0x111>(v);        // row_shr:1
  v = dpp_add<0x112>(v);        // row_shr:2
  v = dpp_add<0x114>(v);        // row_shr:4
  v = dpp_add<0x118>(v);        // row_shr:8
  v = dpp_add<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// Exclusive scan of three per-thread values over the 1024-thread block, in
// thread order; also returns the three totals.  One barrier: every wave
// scans the 16 wave totals itself.
struct Scan3 { int32_t x[3], total[3]; };
__device__ __forceinline__ Scan3 block_exclusive_scan3(const int32_t (&v)[3], int32_t* ws) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int32_t incl[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    incl[c] = wave_incl_scan(v[c]);
    if (lane == 63) ws[c * kPermWaves + wid] = incl[c];
  }
  __syncthreads();
  Scan3 r;
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int32_t wt = lane < kPermWaves ? ws[c * kPermWaves + lane] : 0;
    const int32_t wi = wave_incl_scan(wt);
    const int32_t before = wid == 0 ? 0 : __builtin_amdgcn_readlane(wi, wid - 1);
    r.x[c] = before + incl[c] - v[c];
    r.total[c] = __builtin_amdgcn_readlane(wi, kPermWaves - 1);
  }
  return r;
}

// Stable scatter of rows [r0, r1) by one wave: walks its rows 64 at a time;
// lanes with equal expert find each other with ballots over the id bits,
// take consecutive slots in lane order from the wave's running start
// hist[id * (NW+1) + wave], and the group's lowest lane advances it.  The
// first kBatch * 64 ids come in registers.
constexpr int kPermBatch = 8;
template <int NW>
__device__ __forceinline__ void stable_scatter(const int32_t* __restrict__ ids, int64_t R, int E, int64_t r0,
                                               int64_t r1, const int32_t (&first)[kPermBatch], int32_t* hist,
                                               int32_t* __restrict__ sorted_row, int32_t* __restrict__ row_pos) {
  constexpr int S = NW + 1;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t rb = r0; rb < r1; rb += 64 * kPermBatch) {
    int32_t idv[kPermBatch];
    if (rb == r0) {
#pragma unroll
      for (int u = 0; u < kPermBatch; ++u) idv[u] = first[u];
    } else {
#pragma unroll
      for (int u = 0; u < kPermBatch; ++u) idv[u] = ids[min(rb + 64 * u + lane, R - 1)];
    }
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      const int64_t base_r = rb + 64 * u;
      if (base_r >= r1) break;
      const int64_t r = base_r + lane;
      const bool valid = r < r1;
      const int32_t id = valid ? clamp_id(idv[u], E) : 0;
      uint64_t peers = ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (id >> b) & 1;
        const uint64_t m = ballot(bit);
        peers &= bit ? m : ~m;
      }
      int32_t base = 0;
      if (valid) base = hist[id * S + wid];
      const int rank = __popcll(peers & below);
      if (valid && rank == 0) hist[id * S + wid] = base + __popcll(peers);
      if (valid) {
        const int32_t p = base + rank;
        sorted_row[p] = int32_t(r);
        row_pos[r] = p;
      }
    }
  }
}

// Per-wave histogram of rows [r0, r1) into hist[id * (NW+1) + wave] (LDS
// atomics); keeps the first kBatch * 64 ids in registers for the scatter.
template <int NW>
__device__ __forceinline__ void wave_histogram(const int32_t* __restrict__ ids, int64_t R, int E, int64_t r0,
                                               int64_t r1, int32_t (&first)[kPermBatch], int32_t* hist) {
  constexpr int S = NW + 1;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int64_t rb = r0; rb < r1; rb += 64 * kPermBatch) {
    int32_t idv[kPermBatch];
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) idv[u] = ids[min(rb + 64 * u + lane, R - 1)];
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      if (rb == r0) first[u] = idv[u];
      if (rb + 64 * u + lane < r1) atomicAdd(&hist[clamp_id(idv[u], E) * S + wid], 1);
    }
  }
}

// One 1024-thread workgroup; NW waves split the rows into contiguous chunks.
//  (1) histogram: hist[e][w] = rows of expert e in wave w's chunk (LDS
//      atomics; the per-expert stride NW+1 is odd, so lanes with different
//      experts hit different banks);
//  (2) each thread owns a run of consecutive experts: its row count and its
//      16-row and 256-row tile counts are scanned over the block in one pass,
//      giving offsets[e], every (expert, wave) start slot, and the tile
//      tables' start entries;
//  (3) each wave walks its chunk 64 rows at a time: lanes with equal expert
//      find each other with ballots over the id bits, take consecutive slots
//      in lane order, and the group's lowest lane advances the running start.
// Rows keep their order within an expert (stable), so the result is unique.
// A wave's first batch of ids (64 * kBatch rows) stays in registers between
// (1) and (3).
template <int NW>
__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_row, int32_t* __restrict__ row_pos, Tile* __restrict__ tiles_a,
    int32_t* __restrict__ n_a, Tile* __restrict__ tiles_b, int32_t* __restrict__ n_b) {
  constexpr int S = NW + 1;
  extern __shared__ int32_t lds[];
  int32_t* hist = lds;                        // [E][S]
  int32_t* ws = hist + int64_t(E) * S;        // [3 * kPermWaves]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

  for (int i = tid; i < E * S; i += kPermThreads) hist[i] = 0;
  __syncthreads();

  const int64_t chunk = ((R + NW - 1) / NW + 63) / 64 * 64;
  const int64_t r0 = int64_t(wid) * chunk, r1 = min(R, r0 + chunk);
  int32_t first[kPermBatch];
  if (wid < NW) wave_histogram<NW>(ids, R, E, r0, r1, first, hist);
  __syncthreads();

  // (2) experts [e0, e1) belong to this thread
  const int per = (E + kPermThreads - 1) / kPermThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int32_t run[3] = {0, 0, 0};
  for (int e = e0; e < e1; ++e) {
    int32_t c = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) c += hist[e * S + w];
    run[0] += c;
    run[1] += (c + kSkinnyBM - 1) / kSkinnyBM;
    run[2] += (c + kTiledBM - 1) / kTiledBM;
  }
  const Scan3 sc = block_exclusive_scan3(run, ws);
  int32_t o = sc.x[0], ta = sc.x[1], tb = sc.x[2];
  for (int e = e0; e < e1; ++e) {
    int32_t c[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) c[w] = hist[e * S + w];
    offsets[e] = o;
    int32_t start = o;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      hist[e * S + w] = start;
      start += c[w];
    }
    const int32_t cnt = start - o;
    for (int32_t r = 0; r < cnt; r += kSkinnyBM, ++ta) tiles_a[ta] = Tile{e, o + r, min(kSkinnyBM, cnt - r), 0};
    for (int32_t r = 0; r < cnt; r += kTiledBM, ++tb) tiles_b[tb] = Tile{e, o + r, min(kTiledBM, cnt - r), 0};
    o = start;
  }
  if (tid == 0) {
    offsets[E] = int32_t(R);
    *n_a = sc.total[1];
    *n_b = sc.total[2];
  }
  __syncthreads();

  // (3) stable scatter
  if (wid < NW) stable_scatter<NW>(ids, R, E, r0, r1, first, hist, sorted_row, row_pos);
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
  constexpr int kMaxPer = kPermMaxExperts / kPermThreads;
  constexpr int kG = 16;  // chunk counts loaded together
  const int tid = threadIdx.x;
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
  const Scan3 sc = block_exclusive_scan3(run, ws);
  int32_t o = sc.x[0], ta = sc.x[1], tb = sc.x[2];
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q) {
    const int e = e0 + q;
    if (e < e1) {
      const int32_t cnt = tot[q];
      offsets[e] = o;
      for (int32_t r = 0; r < cnt; r += kSkinnyBM, ++ta) tiles_a[ta] = Tile{e, o + r, min(kSkinnyBM, cnt - r), 0};
      for (int32_t r = 0; r < cnt; r += kTiledBM, ++tb) tiles_b[tb] = Tile{e, o + r, min(kTiledBM, cnt - r), 0};
      o += cnt;
    }
  }
  if (tid == 0) {
    offsets[E] = int32_t(R);
    *n_a = sc.total[1];
    *n_b = sc.total[2];
  }
}

template <int NW>
__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_row, int32_t* __restrict__ row_pos) {
  constexpr int S = NW + 1;
  extern __shared__ int32_t lds[];  // [E][S]
  int32_t* hist = lds;
  const int tid = threadIdx.x, wid = tid >> 6;
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
  if (wid < NW) stable_scatter<NW>(ids, R, E, r0, r1, first, hist, sorted_row, row_pos);
}

template <int NW>
static hipError_t launch_permute_nw(const int32_t* ids, int64_t R, int E, int32_t* offsets,
                                    int32_t* sorted_row, int32_t* row_pos, Tile* tiles_a, int32_t* n_a,
                                    Tile* tiles_b, int32_t* n_b, int32_t* scratch, hipStream_t s) {
  if (hipError_t e = allow_dynamic_lds((const void*)permute_kernel<NW>, kPermLdsBudget); e != hipSuccess) return e;
  if (hipError_t e = allow_dynamic_lds((const void*)permute_scatter_kernel<NW>, kPermLdsBudget); e != hipSuccess)
    return e;
  if (R <= kPermOneWgMaxRows) {
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
