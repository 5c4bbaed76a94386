// Device code of the router's top-k selection and softmax, shared by the
// router kernel and the launch that runs the top-k beside the split-K
// down-projection.
//
// Each token picks k of E routed experts (TokenSpeed AgentX post, "Model
// architecture": 16 of 896), ranked by (logit descending, expert index
// ascending); the combine weights are the softmax over the k selected logits.
#pragma once

#include "common.h"

namespace lmoe {

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

// Selection of one token's top k by a wave.
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
// route_row: selection, softmax and output of one token whose logits the wave
// holds (lane l: v[j] = logit l + 64j, any value for l + 64j >= E).  cb: 64
// keys of LDS private to the wave.
template <int VPL>
__device__ __forceinline__ void route_row(const float (&v)[VPL], int E, int k, int lane, uint64_t* cb,
                                          int32_t* __restrict__ ids_row, float* __restrict__ w_row) {
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
      if (is_c && pos < 64) cb[pos] = cand[j];
      total += __popcll(m);
    }
  }

  uint64_t mine;  // lane i < k ends with the i-th selected key
  if (total <= 64) {
    // cb is private to this wave, whose LDS accesses complete in order; the
    // fences only keep the compiler from moving them across each other
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const uint64_t my = lane < total ? cb[lane] : 0ull;
    int rank = 0;
    for (int i = 0; i < total; ++i) rank += readlane_u64(my, i) > my ? 1 : 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (lane < total && rank < k) cb[rank] = my;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    mine = lane < k ? cb[lane] : 0ull;
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
    ids_row[lane] = int32_t(0xffffffffu - uint32_t(mine));
    w_row[lane] = ex / sum;
  }
}

// One token's routing by one wave: lane l loads logits l + 64j of row t
// (coalesced), then route_row.  cb: 64 keys of LDS private to the wave.
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int64_t t, int E, int k, int lane,
                                            uint64_t* cb, int32_t* __restrict__ ids, float* __restrict__ w) {
  const float* row = logits + t * int64_t(E);
  // all VPL loads are issued unconditionally (clamped index) so that they are
  // in flight together; slots past E are emptied by route_row.  The logits
  // are read once: nontemporal loads (prefill router 16.6 -> 15.9 us)
  float v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) v[j] = __builtin_nontemporal_load(&row[min(lane + 64 * j, E - 1)]);
  route_row<VPL>(v, E, k, lane, cb, ids + t * k, w + t * k);
}

}  // namespace lmoe
