// TwELL kernels: the stand-alone pack of a given pre-activation tensor and
// the overflow-flag list.
//
// TwELL (tile-wise ELLPACK) keeps, for every (token row, 128-column tile)
// of the gate activations, a fixed-capacity list of (value, neuron) plus a
// count ("Sparser, Faster, Lighter Transformer Language Models", gist.science
// explainer, 2. Methodology A).
#include <algorithm>

#include "sffn_internal.hpp"

namespace sffn {
namespace {

// One wave per (32-row group, tile): reads z, packs 32 rows and writes the
// group's overflow word.
__global__ __launch_bounds__(256) void pack_kernel(const float* __restrict__ z, int64_t T, int F,
                                                   int C, int sb, void* __restrict__ val,
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
    const int n = twell_pack_row(v[0], v[1], lane, b * kTile, C,
                                 (char*)val + slot * C * (sb ? 2 : 4), idx + slot * C,
                                 cnt + slot, sb);
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

}  // namespace

hipError_t launch_pack(const float* z, int64_t T, int F, int C, int sb, void* val, uint16_t* idx,
                       int32_t* cnt, uint32_t* ovf, int ovf_words, hipStream_t s) {
  const int64_t items = (int64_t)ovf_words * (F / kTile);
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, z, T, F, C,
                     sb, val, idx, cnt, ovf, ovf_words);
  return hipGetLastError();
}

namespace {
// Over the rows whose TwELL did not overflow (row_flag 0): the sum of
// their tile counts into out[0] and their number into out[1] (64-bit).
// One thread per row, per-block sums, one atomic add per block and value.
__global__ __launch_bounds__(256) void count_sum_kernel(const int32_t* __restrict__ cnt,
                                                        const uint8_t* __restrict__ row_flag,
                                                        int64_t T, int n_t,
                                                        unsigned long long* __restrict__ out) {
  __shared__ unsigned long long part[2][4];
  unsigned long long s = 0, r = 0;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < T;
       t += (int64_t)gridDim.x * blockDim.x) {
    if (row_flag[t]) continue;
    const int32_t* c = cnt + t * n_t;
    for (int b = 0; b < n_t; ++b) s += (unsigned long long)(uint32_t)c[b];
    r += 1;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    s += __shfl_xor(s, o, 64);
    r += __shfl_xor(r, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    part[0][threadIdx.x >> 6] = s;
    part[1][threadIdx.x >> 6] = r;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    const int k = threadIdx.x;
    atomicAdd(out + k, part[k][0] + part[k][1] + part[k][2] + part[k][3]);
  }
}
}  // namespace

hipError_t launch_count_sum(const int32_t* cnt, const uint8_t* row_flag, int64_t T, int n_t,
                            unsigned long long* out, hipStream_t s) {
  hipLaunchKernelGGL(count_sum_kernel, dim3(256), dim3(256), 0, s, cnt, row_flag, T, n_t, out);
  return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(256) void zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  if (p == nullptr || bytes % 4 != 0 || (uintptr_t)p % 4 != 0) return hipErrorInvalidValue;
  const int64_t n = (int64_t)(bytes / 4);
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)p, n);
  return hipGetLastError();
}

hipError_t launch_flags(const uint32_t* ovf, int n_t, int ovf_words, int64_t T, uint8_t* row_flag,
                        int32_t* flagged, int32_t* n_flagged, hipStream_t s) {
  hipLaunchKernelGGL(flags_kernel, dim3(1), dim3(1024), 0, s, ovf, n_t, ovf_words, T, row_flag,
                     flagged, n_flagged);
  return hipGetLastError();
}

}  // namespace sffn
