// Device code of the stable per-expert permutation (a counting sort of rows
// r = t*k + j by expert, the route sorting / gather metadata of a grouped-GEMM
// MoE: TokenSpeed Day-0 post, "Gluon kernels on AMD GPUs > Stable LatentMoE"),
// shared by the permutation kernels and the launch that permutes right after
// the router's top-k.
#pragma once

#include "common.h"
#include "kernels.h"

namespace lmoe {

// Expert ids outside [0, E) (invalid input) are clamped so that every write
// stays inside the caller's buffers; valid ids are unchanged.
__device__ __forceinline__ int32_t clamp_id(int32_t id, int E) { return min(max(id, 0), E - 1); }

// Workgroup barrier that orders LDS only: the waves' global stores may still
// be in flight (unlike __syncthreads, which waits for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// LDS of the one-workgroup permutation: the [E][NW+1] histogram plus the
// scan scratch.
inline int64_t permute_lds_bytes(int E, int nw) { return (int64_t(E) * (nw + 1) + 64) * 4; }
// ... plus, for the mask form of the scatter, one 64-bit lane mask per
// (wave, expert) in front of it.
inline int64_t permute_masks_bytes(int E, int nw) { return int64_t(nw) * E * 8; }

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

// Exclusive scan of three per-thread values over a block of NWAVES waves, in
// thread order; also returns the three totals.  One barrier: every wave
// scans the wave totals itself.  ws: 3 * NWAVES ints of LDS.
struct Scan3 { int32_t x[3], total[3]; };
template <int NWAVES>
__device__ __forceinline__ Scan3 block_exclusive_scan3(const int32_t (&v)[3], int32_t* ws) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int32_t incl[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    incl[c] = wave_incl_scan(v[c]);
    if (lane == 63) ws[c * NWAVES + wid] = incl[c];
  }
  __syncthreads();
  Scan3 r;
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int32_t wt = lane < NWAVES ? ws[c * NWAVES + lane] : 0;
    const int32_t wi = wave_incl_scan(wt);
    const int32_t before = wid == 0 ? 0 : __builtin_amdgcn_readlane(wi, wid - 1);
    r.x[c] = before + incl[c] - v[c];
    r.total[c] = __builtin_amdgcn_readlane(wi, NWAVES - 1);
  }
  return r;
}

// Stable scatter of rows [r0, r1) by one wave: walks its rows 64 at a time;
// lanes with equal expert find each other with ballots over the id bits,
// take consecutive slots in lane order from the wave's running start
// hist[id * (NW+1) + wave], and the group's lowest lane advances it.  The
// first kBatch * 64 ids come in registers.
// MASKS: the lanes with equal expert find each other through the wave's own
// LDS mask of that expert instead: every lane ORs in its lane bit (OR does
// not depend on the order), one read gives the group's lanes, and the group's
// lowest lane clears the mask again.  The same ranks, in far fewer
// instructions than one ballot per id bit.
constexpr int kPermBatch = 8;
template <int NW, bool MASKS = false>
__device__ __forceinline__ void stable_scatter(const int32_t* __restrict__ ids, int64_t R, int E, int64_t r0,
                                               int64_t r1, const int32_t (&first)[kPermBatch], int32_t* hist,
                                               int32_t* __restrict__ sorted_row, int32_t* __restrict__ row_pos,
                                               uint64_t* masks = nullptr) {
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
      uint64_t peers;
      if constexpr (MASKS) {
        uint64_t* mk = masks + int64_t(wid) * E + id;  // this wave's mask of the lane's expert
        if (valid) atomicOr(reinterpret_cast<unsigned long long*>(mk), 1ull << lane);
        // the wave's LDS accesses complete in order; this only keeps the
        // compiler from moving the read above the ORs
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        peers = valid ? *mk : 0ull;
      } else {
        peers = ballot(valid);
        for (int b = 0; b < nbits; ++b) {
          const bool bit = (id >> b) & 1;
          const uint64_t m = ballot(bit);
          peers &= bit ? m : ~m;
        }
      }
      int32_t base = 0;
      if (valid) base = hist[id * S + wid];
      const int rank = __popcll(peers & below);
      if (valid && rank == 0) {
        hist[id * S + wid] = base + __popcll(peers);
        if constexpr (MASKS) masks[int64_t(wid) * E + id] = 0ull;  // after every lane's read above
      }
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

// One workgroup of NTHREADS threads; its first NW waves split the rows into
// contiguous chunks.
//  (1) histogram: hist[e][w] = rows of expert e in wave w's chunk (LDS
//      atomics; the per-expert stride NW+1 is odd, so lanes with different
//      experts hit different banks);
//  (2) each thread owns a run of consecutive experts: its row count and its
//      16-row and kTiledBM-row tile counts are scanned over the block in one pass,
//      giving offsets[e], every (expert, wave) start slot, and the tile
//      tables' start entries;
//  (3) each wave walks its chunk 64 rows at a time: lanes with equal expert
//      find each other with ballots over the id bits, take consecutive slots
//      in lane order, and the group's lowest lane advances the running start.
// Rows keep their order within an expert (stable), so the result is unique.
// A wave's first batch of ids (64 * kBatch rows) stays in registers between
// (1) and (3).
// lds: permute_lds_bytes(E, NW) bytes (MASKS: permute_masks_bytes(E, NW) more,
// 8-byte aligned).
template <int NW, int NTHREADS, bool MASKS = false>
__device__ __forceinline__ void permute_block(const int32_t* __restrict__ ids, int64_t R, int E,
                                              int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_row,
                                              int32_t* __restrict__ row_pos, Tile* __restrict__ tiles_a,
                                              int32_t* __restrict__ n_a, Tile* __restrict__ tiles_b,
                                              int32_t* __restrict__ n_b, int32_t* lds) {
  static_assert(NW <= NTHREADS / 64, "the row-splitting waves belong to the block");
  constexpr int S = NW + 1;
  uint64_t* masks = reinterpret_cast<uint64_t*>(lds);                      // MASKS: [NW][E]
  int32_t* hist = lds + (MASKS ? int64_t(NW) * E * 2 : 0);                 // [E][S]
  int32_t* ws = hist + int64_t(E) * S;                                      // [3 * NTHREADS / 64]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

  if constexpr (MASKS)
    for (int i = tid; i < NW * E; i += NTHREADS) masks[i] = 0ull;
  for (int i = tid; i < E * S; i += NTHREADS) hist[i] = 0;
  __syncthreads();

  const int64_t chunk = ((R + NW - 1) / NW + 63) / 64 * 64;
  const int64_t r0 = int64_t(wid) * chunk, r1 = min(R, r0 + chunk);
  int32_t first[kPermBatch];
  if (wid < NW) wave_histogram<NW>(ids, R, E, r0, r1, first, hist);
  __syncthreads();

  // (2) experts [e0, e1) belong to this thread
  const int per = (E + NTHREADS - 1) / NTHREADS;
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
  const Scan3 sc = block_exclusive_scan3<NTHREADS / 64>(run, ws);
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
    for (int32_t r = 0; r < cnt; r += kSkinnyBM, ++ta)
      tiles_a[ta] = Tile{e, o + r, min(kSkinnyBM, cnt - r), cnt <= kSkinnyBM};
    for (int32_t r = 0; r < cnt; r += kTiledBM, ++tb)
      tiles_b[tb] = Tile{e, o + r, min(kTiledBM, cnt - r), cnt <= kTiledBM};
    o = start;
  }
  if (tid == 0) {
    offsets[E] = int32_t(R);
    *n_a = sc.total[1];
    *n_b = sc.total[2];
  }
  __syncthreads();

  // (3) stable scatter
  if (wid < NW) stable_scatter<NW, MASKS>(ids, R, E, r0, r1, first, hist, sorted_row, row_pos, masks);
}

}  // namespace lmoe
