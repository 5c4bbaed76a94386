// Gather-weight-accumulate combine of the routed expert outputs, fused with
// the routed-latent RMSNorm.
//
// The combine merges a token's expert contributions while still in the
// latent (vLLM Kimi K3 post, section 1, LatentMoE dataflow: the all-to-all
// combine aggregates the low-dimensional tensors); the RMSNorm of the reduced
// routed latent precedes the up-projection (vLLM post, section 6 "Latent MoE
// Tail"; TokenSpeed Day-0 post, "Iris and communication", which also keeps a
// whole routed row in one workgroup so the norm's sum stays local — here one
// wave owns one row).
//
//   c[t]   = sum_{j<k} w[t,j] * Y[row_pos[t*k+j]]     fp32, j ascending
//            (row_pos == NULL: Y is in (token, slot) order, row t*k+j)
//   out[t] = bf16(c * (1/sqrt(mean(c^2) + eps)) * gain)  or bf16(c) without gain
#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

template <int VEC>
struct VecT;
template <>
struct VecT<8> { typedef uint4 type; };
template <>
struct VecT<4> { typedef uint2 type; };
template <>
struct VecT<2> { typedef uint32_t type; };
template <>
struct VecT<1> { typedef uint16_t type; };

template <int VEC>
__device__ __forceinline__ void unpack(const typename VecT<VEC>::type& v, float* f) {
  const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
  for (int i = 0; i < VEC; ++i) f[i] = bf16_to_f32(h[i]);
}

// A VEC-element piece of an expert-output row, which the combine reads once:
// 16-byte pieces with the nontemporal hint (prefill combine 114.6 -> 101.8
// us, MXFP4 prefill 246 -> 213 us, traced alternately), narrower ones plain.
template <int VEC>
__device__ __forceinline__ typename VecT<VEC>::type ld_once(const bf16_t* p) {
  if constexpr (VEC == 8) return ldnt16(p);
  else return *reinterpret_cast<const typename VecT<VEC>::type*>(p);
}

constexpr int kRowsInFlight = 16;

// One wave per token row; lane owns VEC contiguous elements of every
// 64*VEC-wide chunk.  Lane j < k first fetches the j-th slot's row position
// and weight; each chunk then keeps 16 rows' loads in flight.  The fp32 row
// is parked in LDS between the two passes (weighted sum + sum of squares,
// then scale and store).
template <int VEC>
__global__ __launch_bounds__(256) void combine_kernel(const bf16_t* __restrict__ Y, const int32_t* __restrict__ row_pos,
                                                      const float* __restrict__ w, int64_t T, int k, int l,
                                                      const bf16_t* __restrict__ gain, float eps,
                                                      bf16_t* __restrict__ out) {
  typedef typename VecT<VEC>::type V;
  extern __shared__ float crow[];  // [4][l]
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t t = int64_t(blockIdx.x) * 4 + wid;
  if (t >= T) return;
  float* c = crow + wid * l;
  int32_t my_p = 0;
  float my_w = 0.0f;
  if (lane < k) {
    my_p = row_pos ? row_pos[t * k + lane] : int32_t(t * k + lane);
    my_w = w[t * k + lane];
  }
  float ss = 0.0f;
  for (int base = 0; base < l; base += 64 * VEC) {
    const int col = base + lane * VEC;
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += kRowsInFlight) {
      V v[kRowsInFlight];
      // loads past the last slot re-read slot k-1 (no branch, so all of
      // them are in flight together); their values are not used
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        const int64_t p = __builtin_amdgcn_readlane(my_p, min(j0 + u, k - 1));
        v[u] = ld_once<VEC>(Y + p * l + col);
      }
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        if (j0 + u < k) {
          const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j0 + u));
          float f[VEC];
          unpack<VEC>(v[u], f);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[i] += wj * f[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      c[col + i] = acc[i];
      ss += acc[i] * acc[i];
    }
  }
  float scale = 1.0f;
  if (gain) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    scale = 1.0f / sqrtf(ss / float(l) + eps);
  }
  for (int base = 0; base < l; base += 64 * VEC) {
    const int col = base + lane * VEC;
    uint16_t o[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      float v = c[col + i];
      if (gain) v = v * scale * bf16_to_f32(gain[col + i]);
      o[i] = f32_to_bf16(v);
    }
    *reinterpret_cast<V*>(out + t * l + col) = *reinterpret_cast<const V*>(o);
  }
}

// Register-resident form for widths l == WPT * NC * 64 * VEC: a token's row is
// split over WPT waves of the 256-thread block (WPT divides 4); each wave
// holds its NC chunks of 64*VEC columns in registers from the weighted sum
// to the store, keeping 16 loads in flight (16/NC rows at a time).  The
// sum of squares adds the waves' partial sums in part order through LDS.
// More and shorter waves than one-wave-per-token, and no LDS round trip of
// the row.  Every element sums its slots in ascending order.
template <int VEC, int WPT, int NC>
__global__ __launch_bounds__(256) void combine_reg_kernel(const bf16_t* __restrict__ Y,
                                                          const int32_t* __restrict__ row_pos,
                                                          const float* __restrict__ w, int64_t T, int k, int l,
                                                          const bf16_t* __restrict__ gain, float eps,
                                                          bf16_t* __restrict__ out) {
  static_assert(4 % WPT == 0, "a token's waves share one block");
  typedef typename VecT<VEC>::type V;
  constexpr int TPB = 4 / WPT;                              // tokens per block
  constexpr int RPR = NC >= kRowsInFlight ? 1 : kRowsInFlight / NC;  // rows per round
  __shared__ float part_ss[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t t = int64_t(blockIdx.x) * TPB + wid / WPT;
  const bool live = t < T;
  const int col0 = (wid % WPT) * NC * 64 * VEC + lane * VEC;
  int32_t my_p = 0;
  float my_w = 0.0f;
  if (live && lane < k) {
    my_p = row_pos ? row_pos[t * k + lane] : int32_t(t * k + lane);
    my_w = w[t * k + lane];
  }
  float acc[NC][VEC];
#pragma unroll
  for (int q = 0; q < NC; ++q)
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[q][i] = 0.0f;
  if (live) {
    for (int j0 = 0; j0 < k; j0 += RPR) {
      V v[RPR][NC];
      // loads past the last slot re-read slot k-1 (no branch, so all of
      // them are in flight together); their values are not used
#pragma unroll
      for (int u = 0; u < RPR; ++u) {
        const int64_t p = __builtin_amdgcn_readlane(my_p, min(j0 + u, k - 1));
#pragma unroll
        for (int q = 0; q < NC; ++q) v[u][q] = ld_once<VEC>(Y + p * l + col0 + q * 64 * VEC);
      }
#pragma unroll
      for (int u = 0; u < RPR; ++u) {
        if (j0 + u < k) {
          const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j0 + u));
#pragma unroll
          for (int q = 0; q < NC; ++q) {
            float f[VEC];
            unpack<VEC>(v[u][q], f);
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[q][i] += wj * f[i];
          }
        }
      }
    }
  }
  float scale = 1.0f;
  if (gain) {
    float ss = 0.0f;
#pragma unroll
    for (int q = 0; q < NC; ++q)
#pragma unroll
      for (int i = 0; i < VEC; ++i) ss += acc[q][i] * acc[q][i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    if constexpr (WPT > 1) {
      // every wave of the block reaches the barrier, live or not
      if (lane == 0) part_ss[wid] = ss;
      __syncthreads();
      ss = 0.0f;
#pragma unroll
      for (int q = 0; q < WPT; ++q) ss += part_ss[(wid / WPT) * WPT + q];
    }
    scale = 1.0f / sqrtf(ss / float(l) + eps);
  }
  if (!live) return;
#pragma unroll
  for (int q = 0; q < NC; ++q) {
    const int col = col0 + q * 64 * VEC;
    float g[VEC];
    if (gain) unpack<VEC>(*reinterpret_cast<const V*>(gain + col), g);
    uint16_t o[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = f32_to_bf16(gain ? acc[q][i] * scale * g[i] : acc[q][i]);
    *reinterpret_cast<V*>(out + t * l + col) = *reinterpret_cast<const V*>(o);
  }
}

// k == 1 without a norm (one expert-parallel rank's share): out[r] =
// bf16(w[r] * Y[row_pos[r]]), the weighted un-permutation of the received
// rows.  One wave per row; lane owns VEC contiguous elements of each
// 64*VEC-wide chunk, and up to 8 chunks' loads are in flight together.
template <int VEC>
__global__ __launch_bounds__(256) void unpermute_kernel(const bf16_t* __restrict__ Y, const int32_t* __restrict__ row_pos,
                                                        const float* __restrict__ w, int64_t R, int l,
                                                        bf16_t* __restrict__ out) {
  typedef typename VecT<VEC>::type V;
  constexpr int kChunks = 8;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t r = int64_t(blockIdx.x) * 4 + wid;
  if (r >= R) return;
  const int64_t p = row_pos ? int64_t(row_pos[r]) : r;
  const float wr = w[r];
  const int nch = l / (64 * VEC);
  for (int c0 = 0; c0 < nch; c0 += kChunks) {
    V v[kChunks];
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int col = min(c0 + u, nch - 1) * 64 * VEC + lane * VEC;  // past the last chunk: re-read it, unused
      // (plain loads: the nontemporal hint made this kernel slower, 22 -> 27 us
      // at the expert-parallel share)
      v[u] = *reinterpret_cast<const V*>(Y + p * l + col);
    }
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      if (c0 + u < nch) {
        float f[VEC];
        unpack<VEC>(v[u], f);
        uint16_t o[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = f32_to_bf16(wr * f[i]);
        *reinterpret_cast<V*>(out + r * l + (c0 + u) * 64 * VEC + lane * VEC) = *reinterpret_cast<const V*>(o);
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const uint16_t* Y, const int32_t* row_pos, const float* w, int64_t T, int k, int l,
                          const uint16_t* gain, float eps, uint16_t* out, hipStream_t s) {
  const dim3 grid{uint32_t((T + 3) / 4)}, block{256};
  if (k == 1 && !gain) {
    if (l % 512 == 0) unpermute_kernel<8><<<grid, block, 0, s>>>(Y, row_pos, w, T, l, out);
    else if (l % 256 == 0) unpermute_kernel<4><<<grid, block, 0, s>>>(Y, row_pos, w, T, l, out);
    else if (l % 128 == 0) unpermute_kernel<2><<<grid, block, 0, s>>>(Y, row_pos, w, T, l, out);
    else unpermute_kernel<1><<<grid, block, 0, s>>>(Y, row_pos, w, T, l, out);
    return hipGetLastError();
  }
  // register-resident widths: a token's row over WPT waves, NC chunks each
#define LMOE_COMBINE_REG(VEC, WPT, NC)                                                                   \
  if (l == WPT * NC * 64 * VEC) {                                                                        \
    combine_reg_kernel<VEC, WPT, NC><<<dim3{uint32_t((T + 4 / WPT - 1) / (4 / WPT))}, block, 0, s>>>(   \
        Y, row_pos, w, T, k, l, gain, eps, out);                                                         \
    return hipGetLastError();                                                                            \
  }
  LMOE_COMBINE_REG(8, 4, 2)  // 4096
  LMOE_COMBINE_REG(8, 4, 1)  // 2048
  LMOE_COMBINE_REG(8, 2, 1)  // 1024
  LMOE_COMBINE_REG(8, 1, 1)  // 512
  LMOE_COMBINE_REG(1, 4, 1)  // 256
  LMOE_COMBINE_REG(2, 1, 1)  // 128
  LMOE_COMBINE_REG(1, 1, 1)  // 64
#undef LMOE_COMBINE_REG
  // other widths: one wave per token, the fp32 row parked in LDS
  const size_t lds = size_t(4) * l * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  if (l % 512 == 0) combine_kernel<8><<<grid, block, lds, s>>>(Y, row_pos, w, T, k, l, gain, eps, out);
  else if (l % 256 == 0) combine_kernel<4><<<grid, block, lds, s>>>(Y, row_pos, w, T, k, l, gain, eps, out);
  else if (l % 128 == 0) combine_kernel<2><<<grid, block, lds, s>>>(Y, row_pos, w, T, k, l, gain, eps, out);
  else combine_kernel<1><<<grid, block, lds, s>>>(Y, row_pos, w, T, k, l, gain, eps, out);
  return hipGetLastError();
}

}  // namespace lmoe
