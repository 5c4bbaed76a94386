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

namespace lmoe {

// ----------------------------------------------------------------- router ---
// A logit and its expert index packed into one 64-bit key whose unsigned
// order is the ranking order: high word = the float mapped to an order-
// preserving unsigned (+0 and -0 both map to the same key, every NaN maps to
// 0, below -inf), low word = ~index so that the lower index wins ties.  An
// empty slot is key 0, below every real entry (whose low word is > 0).
__device__ __forceinline__ uint64_t rank_key(float v, uint32_t e) {
  uint32_t u = __float_as_uint(v);
  uint32_t key;
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    key = 0u;                                  // NaN
  } else {
    if (u == 0x80000000u) u = 0u;              // -0 -> +0
    key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return (uint64_t(key) << 32) | uint64_t(0xffffffffu - e);
}

__device__ __forceinline__ float key_value(uint64_t k) {
  uint32_t key = uint32_t(k >> 32);
  uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;  // key 0 -> NaN
  return __uint_as_float(u);
}

// DPP move of a 32-bit value; lanes without a source (or outside row_mask)
// read 0, the identity of an unsigned max.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROW_MASK, 0xf, false));
}

// Wave-wide max of an unsigned 32-bit value with DPP row operations:
// butterflies inside each quad, shifts inside each 16-lane row, then the row
// broadcasts; the maximum ends in lane 63 and is returned wave-uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_move<0xb1>(v));        // quad_perm [1,0,3,2]
  v = max(v, dpp_move<0x4e>(v));        // quad_perm [2,3,0,1]
  v = max(v, dpp_move<0x114>(v));       // row_shr:4
  v = max(v, dpp_move<0x118>(v));       // row_shr:8
  v = max(v, dpp_move<0x142, 0xa>(v));  // row_bcast:15 into rows 1 and 3
  v = max(v, dpp_move<0x143, 0xc>(v));  // row_bcast:31 into rows 2 and 3
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), lane));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), lane));
  return (uint64_t(hi) << 32) | lo;
}

// In-register bitonic sort of N keys, descending (N a power of two; all
// indices are compile-time constants, so the keys stay in registers).
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&a)[N]) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int p = i ^ j;
        if (p > i) {
          const bool desc = (i & k) == 0;
          const uint64_t x = a[i], y = a[p];
          const bool swap = desc ? (x < y) : (x > y);
          a[i] = swap ? y : x;
          a[p] = swap ? x : y;
        }
      }
}

// Position of the current lane among the lanes set in a ballot mask.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u)));
}

// Serial selection: each lane sorts its VPL keys once; then each of the k
// rounds takes the wave-wide maximum of the lanes' current heads (a 32-bit max
// of the value word and, only when several lanes tie on it, a second max of the
// index word) and the winning lane pops its head.  Returns the i-th selected
// key in lane i.
template <int VPL>
__device__ __forceinline__ uint64_t select_serial(uint64_t (&cand)[VPL], int k, int lane) {
  sort_desc<VPL>(cand);
  uint64_t mine = 0;
  for (int i = 0; i < k; ++i) {
    const uint64_t head = cand[0];
    const uint32_t hi = uint32_t(head >> 32);
    const uint32_t mh = wave_max_u32(hi);
    uint64_t tied = ballot(hi == mh);
    if (__popcll(tied) > 1) {
      const uint32_t lo = (hi == mh) ? uint32_t(head) : 0u;
      const uint32_t ml = wave_max_u32(lo);
      tied = ballot(hi == mh && uint32_t(head) == ml);
    }
    const int winner = __ffsll(static_cast<unsigned long long>(tied)) - 1;
    const uint64_t top = readlane_u64(head, winner);
    if (lane == i) mine = top;
    if (lane == winner) {
#pragma unroll
      for (int j = 0; j + 1 < VPL; ++j) cand[j] = cand[j + 1];
      cand[VPL - 1] = 0;
    }
  }
  return mine;
}

// One wave per token; lane l holds logits e = l + 64*j (coalesced rows).
//
// Threshold selection.  Let tau be the k-th largest of the 64 lane maxima of
// the value words.  At least k entries (those lane maxima) have a value word
// >= tau, so every one of the top k does, and the candidate set
// C = {entries with value word >= tau} contains the answer.  tau comes from a
// most-significant-bit-first search whose count is one ballot per bit.  For
// i.i.d. logits C holds about k + 2 entries; they are compacted into LDS and
// each candidate's rank is the number of candidate keys above its own (keys
// are unique, so ranks are).  When C exceeds 64 entries (many equal values,
// NaN floods) the serial selection runs instead; both give the same result.
template <int VPL>
__global__ __launch_bounds__(256) void router_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                     int k, int32_t* __restrict__ ids,
                                                     float* __restrict__ w) {
  __shared__ uint64_t cbuf[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = int64_t(blockIdx.x) * 4 + wv;
  if (t >= T) return;
  const float* row = logits + t * int64_t(E);
  // all VPL loads are issued unconditionally (clamped index) so that they are
  // in flight together; slots past E are then emptied
  float v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) v[j] = row[min(lane + 64 * j, E - 1)];
  uint64_t cand[VPL];
  uint32_t lane_max = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + 64 * j;
    cand[j] = (e < E) ? rank_key(v[j], uint32_t(e)) : 0ull;
    lane_max = max(lane_max, uint32_t(cand[j] >> 32));
  }
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = tau | (1u << b);
    if (__popcll(ballot(lane_max >= c)) >= k) tau = c;
  }
  int total = 0;  // wave-uniform candidate count
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const bool is_c = cand[j] != 0 && uint32_t(cand[j] >> 32) >= tau;
    const uint64_t m = ballot(is_c);
    if (m != 0) {
      const int pos = total + lanes_below(m);
      if (is_c && pos < 64) cbuf[wv][pos] = cand[j];
      total += __popcll(m);
    }
  }

  uint64_t mine;  // lane i < k ends with the i-th selected key
  if (total <= 64) {
    // cbuf[wv] is private to this wave, whose LDS accesses complete in order;
    // the fences only keep the compiler from moving them across each other
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const uint64_t my = lane < total ? cbuf[wv][lane] : 0ull;
    int rank = 0;
    for (int i = 0; i < total; ++i) rank += readlane_u64(my, i) > my ? 1 : 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (lane < total && rank < k) cbuf[wv][rank] = my;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    mine = lane < k ? cbuf[wv][lane] : 0ull;
  } else {
    mine = select_serial<VPL>(cand, k, lane);
  }

  const float lv = key_value(mine);
  const float vmax = __shfl(lv, 0, kWave);
  float ex = (lane < k) ? expf(lv - vmax) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, kWave);
  if (lane < k) {
    ids[t * k + lane] = int32_t(0xffffffffu - uint32_t(mine));
    w[t * k + lane] = ex / sum;
  }
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

// Expert ids outside [0, E) (invalid input) are clamped so that every write
// stays inside the caller's buffers; valid ids are unchanged.
__device__ __forceinline__ int32_t clamp_id(int32_t id, int E) { return min(max(id, 0), E - 1); }
constexpr int kPermLdsBudget = 150 * 1024;

int permute_waves(int E) {
  // per-wave histograms [waves][E] plus two (E+1) scan arrays in LDS
  const int64_t fixed = 2 * int64_t(E + 1) * 4 + 64 * 4;
  for (int w = 16; w >= 1; w >>= 1)
    if (int64_t(w) * E * 4 + fixed <= kPermLdsBudget) return w;
  return 0;
}

// Exclusive scans of a[0..n) and b[0..n) in LDS by a 1024-thread block
// (n <= 16 * 1024), both at once; returns the two totals.  Each thread scans a
// contiguous run, then the run sums are scanned across lanes and waves.  b may
// be null (a scanned alone).
struct ScanTotals { int32_t a, b; };
__device__ ScanTotals block_exclusive_scan2(int32_t* a, int32_t* b, int n, int32_t* wave_sums) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int kW = kPermThreads / 64;
  const int per = (n + kPermThreads - 1) / kPermThreads;
  const int i0 = tid * per, i1 = min(n, i0 + per);
  int32_t ra = 0, rb = 0;
  for (int i = i0; i < i1; ++i) {
    ra += a[i];
    if (b) rb += b[i];
  }
  int32_t ia = ra, ib = rb;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t oa = __shfl_up(ia, off, kWave), ob = __shfl_up(ib, off, kWave);
    if (lane >= off) {
      ia += oa;
      ib += ob;
    }
  }
  if (lane == 63) {
    wave_sums[wid] = ia;
    wave_sums[kW + 1 + wid] = ib;
  }
  __syncthreads();
  if (wid == 0) {
    const int32_t va = lane < kW ? wave_sums[lane] : 0, vb = lane < kW ? wave_sums[kW + 1 + lane] : 0;
    int32_t xa = va, xb = vb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t oa = __shfl_up(xa, off, kWave), ob = __shfl_up(xb, off, kWave);
      if (lane >= off) {
        xa += oa;
        xb += ob;
      }
    }
    if (lane < kW) {
      wave_sums[lane] = xa - va;  // exclusive
      wave_sums[kW + 1 + lane] = xb - vb;
    }
    if (lane == kW - 1) {
      wave_sums[kW] = xa;
      wave_sums[2 * kW + 1] = xb;
    }
  }
  __syncthreads();
  int32_t base_a = wave_sums[wid] + ia - ra, base_b = wave_sums[kW + 1 + wid] + ib - rb;
  for (int i = i0; i < i1; ++i) {
    const int32_t ca = a[i];
    a[i] = base_a;
    base_a += ca;
    if (b) {
      const int32_t cb = b[i];
      b[i] = base_b;
      base_b += cb;
    }
  }
  const ScanTotals tot{wave_sums[kW], wave_sums[2 * kW + 1]};
  __syncthreads();
  return tot;
}

// Tile tables of granularity bm_a and bm_b from the offsets: every expert's
// segment split into runs of at most bm rows.  ta/tb are LDS scratch of E
// entries each.
__device__ void emit_tiles(const int32_t* off, int E, int32_t* ta, int32_t* tb, int32_t* wave_sums,
                           int bm_a, Tile* __restrict__ tiles_a, int32_t* __restrict__ n_a,
                           int bm_b, Tile* __restrict__ tiles_b, int32_t* __restrict__ n_b) {
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    const int32_t cnt = off[e + 1] - off[e];
    ta[e] = (cnt + bm_a - 1) / bm_a;
    tb[e] = (cnt + bm_b - 1) / bm_b;
  }
  __syncthreads();
  const ScanTotals tot = block_exclusive_scan2(ta, tb, E, wave_sums);
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    const int32_t o = off[e], cnt = off[e + 1] - o;
    int32_t t = ta[e];
    for (int32_t r = 0; r < cnt; r += bm_a, ++t) tiles_a[t] = Tile{e, o + r, min(bm_a, cnt - r), 0};
    t = tb[e];
    for (int32_t r = 0; r < cnt; r += bm_b, ++t) tiles_b[t] = Tile{e, o + r, min(bm_b, cnt - r), 0};
  }
  if (threadIdx.x == 0) {
    *n_a = tot.a;
    *n_b = tot.b;
  }
}

// One 1024-thread workgroup.  Wave w owns the contiguous row chunk
// [w*C, (w+1)*C).  (1) per-wave LDS histograms; (2) per expert, prefix over
// waves; (3) exclusive scan over experts -> offsets; (4) each wave walks its
// chunk 64 rows at a time: lanes with equal expert find each other with
// ballots over the id bits, take consecutive slots in lane order, and the
// group's lowest lane advances the running base.  Rows keep their order
// within an expert (stable), so the result is unique.  A wave's first batch
// of ids (64 * kBatch rows) stays in registers between (1) and (4).
__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int nwaves, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_row, int32_t* __restrict__ row_pos, Tile* __restrict__ tiles_a,
    int32_t* __restrict__ n_a, Tile* __restrict__ tiles_b, int32_t* __restrict__ n_b) {
  extern __shared__ int32_t lds[];
  int32_t* hist = lds;                          // [nwaves][E]
  int32_t* off = hist + int64_t(nwaves) * E;    // [E+1]
  int32_t* tmp = off + (E + 1);                 // [E+1]
  int32_t* wave_sums = tmp + (E + 1);           // [2 * (waves + 1)]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

  for (int i = tid; i < nwaves * E; i += kPermThreads) hist[i] = 0;
  __syncthreads();

  const int64_t chunk = ((R + nwaves - 1) / nwaves + 63) / 64 * 64;
  const int64_t r0 = int64_t(wid) * chunk, r1 = min(R, r0 + chunk);
  // ids are read kBatch rows per lane at a time with clamped (in-bounds)
  // indices, so a batch's loads are in flight together
  constexpr int kBatch = 8;
  int32_t first[kBatch];
  if (wid < nwaves) {
    for (int64_t rb = r0; rb < r1; rb += 64 * kBatch) {
      int32_t idv[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) idv[u] = ids[min(rb + 64 * u + lane, R - 1)];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (rb == r0) first[u] = idv[u];
        if (rb + 64 * u + lane < r1) atomicAdd(&hist[wid * E + clamp_id(idv[u], E)], 1);
      }
    }
  }
  __syncthreads();

  for (int e = tid; e < E; e += kPermThreads) {
    int32_t run = 0;
    for (int w = 0; w < nwaves; ++w) {
      const int32_t c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
    off[e] = run;
  }
  __syncthreads();
  block_exclusive_scan2(off, nullptr, E, wave_sums);
  for (int e = tid; e < E; e += kPermThreads) {
    const int32_t o = off[e];
    offsets[e] = o;
    for (int w = 0; w < nwaves; ++w) hist[w * E + e] += o;
  }
  if (tid == 0) {
    off[E] = int32_t(R);
    offsets[E] = int32_t(R);
  }
  __syncthreads();

  if (wid < nwaves) {
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t rb = r0; rb < r1; rb += 64 * kBatch) {
      int32_t idv[kBatch];
      if (rb == r0) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) idv[u] = first[u];
      } else {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) idv[u] = ids[min(rb + 64 * u + lane, R - 1)];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
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
        if (valid) base = hist[wid * E + id];
        const int rank = __popcll(peers & below);
        if (valid && rank == 0) hist[wid * E + id] = base + __popcll(peers);
        if (valid) {
          const int32_t p = base + rank;
          sorted_row[p] = int32_t(r);
          row_pos[r] = p;
        }
      }
    }
  }
  __syncthreads();
  emit_tiles(off, E, tmp, hist, wave_sums, kSkinnyBM, tiles_a, n_a, kTiledBM, tiles_b, n_b);
}

hipError_t launch_permute(const int32_t* ids, int64_t R, int E, int32_t* offsets, int32_t* sorted_row,
                          int32_t* row_pos, Tile* tiles_a, int32_t* n_a, Tile* tiles_b, int32_t* n_b,
                          hipStream_t s) {
  const int nw = permute_waves(E);
  if (nw == 0) return hipErrorInvalidValue;
  const size_t lds = (size_t(nw) * E + 2 * size_t(E + 1) + 64) * 4;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)permute_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kPermLdsBudget + 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  permute_kernel<<<dim3(1), dim3(kPermThreads), lds, s>>>(ids, R, E, nw, offsets, sorted_row, row_pos,
                                                          tiles_a, n_a, tiles_b, n_b);
  return hipGetLastError();
}

}  // namespace lmoe
