// TwELL kernels: the stand-alone pack, the overflow-flag list and the
// fused sparse up/down projection.
//
// TwELL (tile-wise ELLPACK) keeps, for every (token row, 128-column tile)
// of the gate activations, a fixed-capacity list of (value, neuron) plus a
// count ("Sparser, Faster, Lighter Transformer Language Models", gist.science
// explainer, 2. Methodology A). The fused up/down projection walks each
// token's list, takes the dot product of the token with the neuron's up
// weights and adds the scalar times the neuron's down weights to the
// token's output, so the dense hidden tensor never exists in memory (same
// page, 2. Methodology B).
#include "sffn_internal.hpp"

namespace sffn {
namespace {

// One wave per (32-row group, tile): reads z, packs 32 rows and writes the
// group's overflow word.
__global__ __launch_bounds__(256) void pack_kernel(const float* __restrict__ z, int64_t T, int F,
                                                   int C, float* __restrict__ val,
                                                   uint16_t* __restrict__ idx,
                                                   int32_t* __restrict__ cnt,
                                                   uint32_t* __restrict__ ovf, int ovf_words) {
  const int lane = threadIdx.x & 63;
  const int n_t = F / kTile;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)ovf_words * n_t) return;
  const int b = (int)(item % n_t);
  const int w = (int)(item / n_t);
  uint32_t bits = 0;
  for (int q = 0; q < 32; ++q) {
    const int64_t t = (int64_t)w * 32 + q;
    if (t >= T) break;
    const f32x2_t v = *(const f32x2_t*)(z + t * F + (int64_t)b * kTile + 2 * lane);
    const int64_t slot = t * n_t + b;
    const int n = twell_pack_row(v[0], v[1], lane, b * kTile, C, val + slot * C, idx + slot * C,
                                 cnt + slot);
    bits |= (n > C ? 1u : 0u) << q;
  }
  if (lane == 0) ovf[(int64_t)b * ovf_words + w] = bits;
}

// One workgroup: OR the overflow words over tiles, write the per-row flags
// and the ascending list of flagged rows (block-wide exclusive scan of the
// per-word counts, words taken 1024 at a time in order).
__global__ __launch_bounds__(1024) void flags_kernel(const uint32_t* __restrict__ ovf, int n_t,
                                                     int ovf_words, int64_t T,
                                                     uint8_t* __restrict__ row_flag,
                                                     int32_t* __restrict__ flagged,
                                                     int32_t* __restrict__ n_flagged) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < ovf_words; base += 1024) {
    const int w = base + tid;
    uint32_t m = 0;
    if (w < ovf_words) {
      for (int b = 0; b < n_t; ++b) m |= ovf[(int64_t)b * ovf_words + w];
      const int64_t r0 = (int64_t)w * 32;
      if (r0 + 32 <= T) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t v = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) v |= ((m >> (4 * i + k)) & 1u) << (8 * k);
          *(uint32_t*)(row_flag + r0 + 4 * i) = v;
        }
      } else {
        for (int i = 0; r0 + i < T; ++i) row_flag[r0 + i] = (uint8_t)((m >> i) & 1u);
      }
    }
    // inclusive scan inside the wave
    const int c = __popc(m);
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int wbase = 0;
    int total = 0;
    for (int k = 0; k < 16; ++k) {
      if (k < wave) wbase += wsum[k];
      total += wsum[k];
    }
    int off = carry + wbase + inc - c;
    while (m) {
      const int i = __ffs(m) - 1;
      m &= m - 1;
      flagged[off++] = w * 32 + i;
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) *n_flagged = carry;
}

template <typename E> struct SE;
template <> struct SE<uint16_t> {
  static constexpr int EPC = 8;
  __device__ static void unpack(const u32x4_t& v, float* o) {
#pragma unroll
    for (int k = 0; k < 4; ++k) { o[2 * k] = bf16lo(v[k]); o[2 * k + 1] = bf16hi(v[k]); }
  }
};
template <> struct SE<float> {
  static constexpr int EPC = 4;
  __device__ static void unpack(const u32x4_t& v, float* o) {
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = __uint_as_float(v[k]);
  }
};

// One wave per token. The lane owns elements c*CH + lane*EPC + e of the
// d-vector (c < NCH chunks, e < EPC), so each 16-byte load of a weight row
// is coalesced across the wave. The token's TwELL slots are scanned 64 at
// a time; the active ones are visited in ascending neuron order, two per
// step so that four weight rows are in flight at once.
template <typename E, int NCH, bool GATED>
__global__ __launch_bounds__(256) void sparse_updown_kernel(
    const E* __restrict__ x, const E* __restrict__ wu, const E* __restrict__ wd,
    const float* __restrict__ val, const uint16_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, const uint8_t* __restrict__ row_flag, int64_t T, int d,
    int n_t, int C, float* __restrict__ y) {
  constexpr int EPC = SE<E>::EPC;
  constexpr int CH = 64 * EPC;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (row_flag[t]) return;  // the dense path writes flagged rows

  float xr[NCH][EPC];
  float yr[NCH][EPC];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const u32x4_t v = *(const u32x4_t*)(x + t * d + c * CH + lane * EPC);
    SE<E>::unpack(v, xr[c]);
#pragma unroll
    for (int e = 0; e < EPC; ++e) yr[c][e] = 0.0f;
  }

  const int total = n_t * C;
  const int64_t tb = t * n_t;
  for (int base = 0; base < total; base += 64) {
    const int q = base + lane;
    bool act = false;
    float a = 0.0f;
    int j = 0;
    if (q < total) {
      const int b = q / C;
      const int s = q - b * C;
      if (s < cnt[tb + b]) {
        a = val[tb * C + q];
        j = idx[tb * C + q];
        act = true;
      }
    }
    uint64_t mask = __ballot(act);
    while (mask) {
      const int s0 = __ffsll((unsigned long long)mask) - 1;
      mask &= mask - 1;
      const bool two = mask != 0;
      const int s1 = two ? __ffsll((unsigned long long)mask) - 1 : s0;
      if (two) mask &= mask - 1;
      const int j0 = __builtin_amdgcn_readlane(j, s0);
      const int j1 = __builtin_amdgcn_readlane(j, s1);
      const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), s0));
      const float a1 = two ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), s1)) : 0.0f;

      u32x4_t d0[NCH], d1[NCH];
      const E* wd0 = wd + (int64_t)j0 * d + lane * EPC;
      const E* wd1 = wd + (int64_t)j1 * d + lane * EPC;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        d0[c] = *(const u32x4_t*)(wd0 + c * CH);
        d1[c] = *(const u32x4_t*)(wd1 + c * CH);
      }
      float h0 = a0, h1 = a1;
      if constexpr (GATED) {
        u32x4_t u0[NCH], u1[NCH];
        const E* wu0 = wu + (int64_t)j0 * d + lane * EPC;
        const E* wu1 = wu + (int64_t)j1 * d + lane * EPC;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          u0[c] = *(const u32x4_t*)(wu0 + c * CH);
          u1[c] = *(const u32x4_t*)(wu1 + c * CH);
        }
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          float w0[EPC], w1[EPC];
          SE<E>::unpack(u0[c], w0);
          SE<E>::unpack(u1[c], w1);
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            p0 = fmaf(xr[c][e], w0[e], p0);
            p1 = fmaf(xr[c][e], w1[e], p1);
          }
        }
        h0 = a0 * wave_sum(p0);
        h1 = a1 * wave_sum(p1);
      }
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        float w0[EPC], w1[EPC];
        SE<E>::unpack(d0[c], w0);
        SE<E>::unpack(d1[c], w1);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          yr[c][e] = fmaf(h0, w0[e], yr[c][e]);
          yr[c][e] = fmaf(h1, w1[e], yr[c][e]);
        }
      }
    }
  }

  float* yo = y + t * d + lane * EPC;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
#pragma unroll
    for (int e = 0; e < EPC; e += 4)
      *(f32x4_t*)(yo + c * CH + e) = f32x4_t{yr[c][e], yr[c][e + 1], yr[c][e + 2], yr[c][e + 3]};
  }
}

template <typename E, bool G>
hipError_t launch_sparse_t(int nch, const void* x, const void* wu, const void* wd,
                           const float* val, const uint16_t* idx, const int32_t* cnt,
                           const uint8_t* row_flag, int64_t T, int d, int n_t, int C, float* y,
                           hipStream_t s) {
  const dim3 grid((unsigned)((T + 3) / 4));
  const E* xe = (const E*)x;
  const E* ue = (const E*)wu;
  const E* de = (const E*)wd;
  switch (nch) {
#define SFFN_SP_CASE(N)                                                                          \
  case N:                                                                                        \
    hipLaunchKernelGGL((sparse_updown_kernel<E, N, G>), grid, dim3(256), 0, s, xe, ue, de, val, \
                       idx, cnt, row_flag, T, d, n_t, C, y);                                     \
    break;
    SFFN_SP_CASE(1)
    SFFN_SP_CASE(2)
    SFFN_SP_CASE(4)
    SFFN_SP_CASE(8)
#undef SFFN_SP_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const float* z, int64_t T, int F, int C, float* val, uint16_t* idx,
                       int32_t* cnt, uint32_t* ovf, int ovf_words, hipStream_t s) {
  const int64_t items = (int64_t)ovf_words * (F / kTile);
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, z, T, F, C,
                     val, idx, cnt, ovf, ovf_words);
  return hipGetLastError();
}

hipError_t launch_flags(const uint32_t* ovf, int n_t, int ovf_words, int64_t T, uint8_t* row_flag,
                        int32_t* flagged, int32_t* n_flagged, hipStream_t s) {
  hipLaunchKernelGGL(flags_kernel, dim3(1), dim3(1024), 0, s, ovf, n_t, ovf_words, T, row_flag,
                     flagged, n_flagged);
  return hipGetLastError();
}

hipError_t launch_sparse_updown(Dtype dt, bool gated, const void* x, const void* wu,
                                const void* wd, const float* val, const uint16_t* idx,
                                const int32_t* cnt, const uint8_t* row_flag, int64_t T, int d,
                                int n_t, int C, float* y, hipStream_t s) {
  const int ch = dt == kBF16 ? 512 : 256;
  const int nch = d / ch;
  if (dt == kBF16)
    return gated ? launch_sparse_t<uint16_t, true>(nch, x, wu, wd, val, idx, cnt, row_flag, T, d,
                                                   n_t, C, y, s)
                 : launch_sparse_t<uint16_t, false>(nch, x, wu, wd, val, idx, cnt, row_flag, T,
                                                    d, n_t, C, y, s);
  return gated ? launch_sparse_t<float, true>(nch, x, wu, wd, val, idx, cnt, row_flag, T, d, n_t,
                                              C, y, s)
               : launch_sparse_t<float, false>(nch, x, wu, wd, val, idx, cnt, row_flag, T, d, n_t,
                                               C, y, s);
}

}  // namespace sffn
