// Device-rate probes for the ceilings that bound the bf16 MFMA GEMMs on
// gfx950 (built as libsffn_probe.so, apart from the layer library):
//   * LDS: 16-byte fragment reads (ds_read_b128) alone, 16-byte
//     direct-to-LDS copies (global_load_lds_dwordx4, L2-resident source)
//     alone, and both kinds issued together;
//   * L2 -> registers: 16-byte loads in two lane layouts that fetch the
//     same bytes: four lanes per 64-byte row piece (the layout of a
//     direct-to-LDS copy), and the 32 x 32 MFMA operand layout (lane l:
//     row l % 32, 16-byte piece l / 32).
// Every probe reads inside its own buffers; rates are bytes per second per
// compute unit, timed with HIP events around one launch after two warm-up
// launches.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "sffn_probe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRowB = 4096;    // bytes per source row
constexpr int kRows = 8192;    // source rows (32 MiB)

// MODE 0: reads, 1: copies, 2: both. Each wave owns 8 KB of LDS, walked in
// 1 KB steps with lane-contiguous 16-byte pieces (no bank conflicts).
template <int MODE>
__global__ __launch_bounds__(256) void lds_probe(const char* __restrict__ src, u32x4* out, int reps) {
  // reads walk the first 32 KB, copies land in the second (8 KB per wave in
  // each half)
  __shared__ __align__(16) u32x4 smem[64 * 1024 / 16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rb = (((blockIdx.x / 8) % 4) * 4 + wave) * 16;   // rows < 256: L2-resident
  const char* s = src + (int64_t)(rb + (lane >> 2)) * kRowB + (lane & 3) * 16;
  for (int i = threadIdx.x; i < 2048; i += 256) smem[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0, 0, 0, 0};
  // the wave's 8 KB: 8 pieces of 64 lanes x 16 bytes
  int base = wave * 512 + lane;
  for (int r = 0; r < reps; ++r) {
    // an offset the compiler cannot see through, so that every repetition
    // reads LDS again (all 8 reads issued before their results are used)
    asm volatile("" : "+v"(base));
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (MODE != 0)
        __builtin_amdgcn_global_load_lds((const void*)(s + ((r * 8 + c) & 63) * 64),
                                         (void*)(smem + 2048 + wave * 512 + c * 64), 16, 0, 0);
      if (MODE != 1) acc ^= smem[base + c * 64];
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // no copy in flight when the wave ends
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// P 0: four lanes per 64-byte row piece; P 1: 32 x 32 MFMA operand layout.
// A wave reads 32 rows x 4 KB per repetition, 4 loads per 128-byte window.
template <int P>
__global__ __launch_bounds__(256) void load_probe(const char* __restrict__ src, u32x4* out, int reps) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rb = (((blockIdx.x / 8) % 4) * 4 + wave) * 32;   // rows < 512: L2-resident
  u32x4 acc = {0, 0, 0, 0};
  for (int r = 0; r < reps; ++r) {
#pragma unroll 4
    for (int kw = 0; kw < kRowB / 128; ++kw) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        int row, off;
        if (P == 0) {
          row = rb + (c >> 1) * 16 + (lane >> 2);
          off = kw * 128 + (c & 1) * 64 + (lane & 3) * 16;
        } else {
          row = rb + (lane & 31);
          off = kw * 128 + (lane >> 5) * 64 + c * 16;
        }
        acc ^= *(const u32x4*)(src + (int64_t)row * kRowB + off);
      }
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

template <typename F>
hipError_t timed(F launch, float* ms) {
  hipEvent_t e0, e1;
  hipError_t st = hipEventCreate(&e0);
  if (st != hipSuccess) return st;
  st = hipEventCreate(&e1);
  if (st != hipSuccess) { (void)hipEventDestroy(e0); return st; }
  for (int it = 0; it < 3 && st == hipSuccess; ++it) {
    st = hipEventRecord(e0, 0);
    if (st == hipSuccess) launch();
    if (st == hipSuccess) st = hipGetLastError();
    if (st == hipSuccess) st = hipEventRecord(e1, 0);
    if (st == hipSuccess) st = hipEventSynchronize(e1);
    if (st == hipSuccess) st = hipEventElapsedTime(ms, e0, e1);
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return st;
}

}  // namespace

// declared and documented in include/sffn_probe.h
extern "C" int sffn_probe_rates(int num_cu, double* out, int n_out) {
  if (num_cu <= 0 || out == nullptr || n_out < 5) return (int)hipErrorInvalidValue;
  char* src = nullptr;
  u32x4* sink = nullptr;
  const int lds_blocks = 2 * num_cu;
  const int load_blocks = 8 * num_cu;
  hipError_t st = hipMalloc(&src, (size_t)kRows * kRowB);
  if (st == hipSuccess) st = hipMalloc(&sink, (size_t)load_blocks * 256 * sizeof(u32x4));
  if (st == hipSuccess) st = hipMemset(src, 1, (size_t)kRows * kRowB);
  float ms = 0.0f;
  const int lreps = 2000;
  const double lds_bytes = (double)lds_blocks * 4 * lreps * 8 * 1024;   // per kind
  if (st == hipSuccess) {
    st = timed([&] { hipLaunchKernelGGL(lds_probe<0>, dim3(lds_blocks), dim3(256), 0, 0, src, sink, lreps); }, &ms);
    out[0] = lds_bytes / (ms * 1e-3) / num_cu;
  }
  if (st == hipSuccess) {
    st = timed([&] { hipLaunchKernelGGL(lds_probe<1>, dim3(lds_blocks), dim3(256), 0, 0, src, sink, lreps); }, &ms);
    out[1] = lds_bytes / (ms * 1e-3) / num_cu;
  }
  if (st == hipSuccess) {
    st = timed([&] { hipLaunchKernelGGL(lds_probe<2>, dim3(lds_blocks), dim3(256), 0, 0, src, sink, lreps); }, &ms);
    out[2] = 2.0 * lds_bytes / (ms * 1e-3) / num_cu;
  }
  const int treps = 8;
  const double load_bytes = (double)load_blocks * 4 * treps * 32 * kRowB;
  if (st == hipSuccess) {
    st = timed([&] { hipLaunchKernelGGL(load_probe<0>, dim3(load_blocks), dim3(256), 0, 0, src, sink, treps); }, &ms);
    out[3] = load_bytes / (ms * 1e-3) / num_cu;
  }
  if (st == hipSuccess) {
    st = timed([&] { hipLaunchKernelGGL(load_probe<1>, dim3(load_blocks), dim3(256), 0, 0, src, sink, treps); }, &ms);
    out[4] = load_bytes / (ms * 1e-3) / num_cu;
  }
  if (src) (void)hipFree(src);
  if (sink) (void)hipFree(sink);
  return (int)st;
}
