// Row compaction (TwELL -> ELL + dense-backup routing) and the sparse
// up/down projection over the compacted rows.
//
// The Hybrid format of "Sparser, Faster, Lighter Transformer Language
// Models" routes each token row either to a compact ELL matrix (few
// non-zeros) or to a dense backup (many non-zeros) (gist.science explainer,
// 2. Methodology A, Hybrid Format for Training; wispaper blog, 2. The Hybrid
// Training Algorithm). The same conversion with an ELL capacity of n_t * C
// serves inference: then only rows whose TwELL overflowed go to the backup.
//
// Up/down projection (same explainer, 2. Methodology B: fused up/down
// projection): for every active (neuron j, value a) of a row, u = x . W_u[j],
// h = a * u, y += h * W_d[j]. MI355X has 8 XCDs with a private 4 MB L2
// each and a workgroup with id b runs on XCD b % 8. The model dimension is
// cut into NS slices (8 at d = 2048) and slice s is processed only by
// workgroups with b % NS == s, so each XCD's L2 holds one slice of W_up and
// W_down (5632 x 256 bf16 = 2.9 MB each at the 1.5B shape) instead of
// streaming whole 8 KB neuron rows from HBM/MALL. Phase 1 writes per-slice
// partial dot products (one float per active pair and slice); phase 2 sums
// them in slice order (deterministic), scales by the activation and adds
// the neuron's down weights into the row's y slice. No dense hidden tensor
// is formed.
#include "sffn_internal.hpp"

namespace sffn {
namespace {

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One wave per token row: count its positives, decide the route, and if
// the row stays sparse, concatenate its TwELL tile lists (ascending neuron)
// into ELL slots 0..nnz-1. Lane b takes tile b (64 tiles per pass): an
// exclusive prefix of the stored counts gives each tile's first ELL slot,
// and the lane copies its tile's entries, so only live slots are read.
__global__ __launch_bounds__(256) void rows_kernel(EllArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int32_t* cnt = a.cnt + t * a.n_t;
  int nnz = 0;
  bool over = false;
  int c0 = 0;  // the count of tile `lane` (first pass of 64 tiles)
  for (int b = lane; b < a.n_t; b += 64) {
    const int c = cnt[b];
    if (b < 64) c0 = c;
    nnz += c;
    over |= c > a.C;
  }
  nnz = wave_sum_int(nnz);
  const bool flag = __ballot(over) != 0;
  const bool backup = flag || nnz > a.K;
  if (lane == 0) {
    if (a.row_flag) a.row_flag[t] = flag ? 1 : 0;
    a.bk[t] = backup ? 1 : 0;
    a.ell_cnt[t] = backup ? 0 : nnz;
  }
  if (backup || nnz == 0) return;
  // not flagged: every tile count is <= C, so all entries are stored
  const int64_t dst = t * (int64_t)a.K;
  int base = 0;
  for (int b0 = 0; b0 < a.n_t; b0 += 64) {
    const int b = b0 + lane;
    const int c = b < a.n_t ? (b0 == 0 ? c0 : cnt[b]) : 0;
    int inc = c;  // inclusive prefix over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    const int64_t src = (t * a.n_t + b) * (int64_t)a.C;
    const int64_t pos = dst + base + inc - c;
    for (int s = 0; s < c; ++s) {
      a.ell_idx[pos + s] = a.idx[src + s];
      a.ell_a[pos + s] = a.val[src + s];
    }
    base += __shfl(inc, 63, 64);
  }
}

// One workgroup: list the backup rows in ascending order (the first cap of
// them), their true count and, when requested, every row's backup slot
// (-1 for ELL rows).
__global__ __launch_bounds__(1024) void backup_list_kernel(const uint8_t* __restrict__ bk,
                                                           int64_t T, int32_t* __restrict__ brow,
                                                           int64_t cap,
                                                           int32_t* __restrict__ n_backup,
                                                           int32_t* __restrict__ slot) {
  constexpr int RPT = 16;
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int carry = 0;
  for (int64_t base = 0; base < T; base += 1024 * RPT) {
    const int64_t r0 = base + (int64_t)tid * RPT;
    uint32_t bits = 0;
    if (r0 + RPT <= T) {
      const u32x4_t v = *(const u32x4_t*)(bk + r0);
#pragma unroll
      for (int i = 0; i < RPT; ++i) bits |= ((v[i >> 2] >> (8 * (i & 3))) & 0xFFu) ? (1u << i) : 0u;
    } else {
      for (int i = 0; r0 + i < T; ++i) bits |= bk[r0 + i] ? (1u << i) : 0u;
    }
    const int c = __popc(bits);
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int wbase = 0, total = 0;
    for (int k = 0; k < 16; ++k) {
      if (k < wave) wbase += wsum[k];
      total += wsum[k];
    }
    int off = carry + wbase + inc - c;
    for (int i = 0; i < RPT && r0 + i < T; ++i) {
      if (bits & (1u << i)) {
        if (off < cap) brow[off] = (int32_t)(r0 + i);
        if (slot) slot[r0 + i] = off;
        ++off;
      } else if (slot) {
        slot[r0 + i] = -1;
      }
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) *n_backup = carry;
}

constexpr int GRP = 32;  // active pairs in flight per wave

// One butterfly exchange at lane distance W over the first 2*HALF values:
// the lane keeps one half (the upper one if bit W of its lane id is set),
// sends the other half to its partner and adds what it receives. Template
// recursion keeps every register index a compile-time constant.
template <int W, int HALF>
__device__ __forceinline__ void butterfly(float* v, int lane) {
  const bool up = (lane & W) != 0;
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const float send = up ? v[i] : v[i + HALF];
    const float keep = up ? v[i + HALF] : v[i];
    v[i] = keep + __shfl_xor(send, W, 64);
  }
  if constexpr (HALF > 1) butterfly<W / 2, HALF / 2>(v, lane);
}

// Wave totals of 32 per-lane values at once: five butterfly exchanges
// (distances 32, 16, 8, 4, 2) and a last one between lane pairs. On return
// lane l holds the total of value (l >> 1) & 31. The order of additions is
// fixed.
__device__ __forceinline__ float wave_sum32(float* v, int lane) {
  butterfly<32, 16>(v, lane);
  return v[0] + __shfl_xor(v[0], 1, 64);
}

// Phase 1: upart[s][t][k] = x_t[slice s] . W_u[j_k][slice s].
template <typename E, int NS, int SW>
__global__ __launch_bounds__(256) void up_partial_kernel(SliceArgs a) {
  using G = SliceGeom<E, SW>;
  constexpr int EPL = G::EPL, RPW = G::RPW;
  using R = typename G::R;
  const int lane = threadIdx.x & 63;
  const int hf = RPW == 2 ? lane >> 5 : 0;
  const int l = lane & (G::LPR - 1);
  const int i = lane & 31;
  const int s = blockIdx.x % NS;
  const int64_t t = ((int64_t)(blockIdx.x / NS) * 4 + (threadIdx.x >> 6)) * RPW + hf;
  if (t - hf >= a.T) return;
  const bool ok = t < a.T;
  const int64_t tr = ok ? t : a.T - 1;
  const int d = NS * SW;
  const int64_t col = (int64_t)s * SW + l * EPL;
  // weight rows are addressed as a uniform base plus a 32-bit byte offset
  // (F * d * sizeof(E) < 4 GiB), so a load needs one offset register
  const char* wu = (const char*)a.wu;
  const uint32_t colb = (uint32_t)(col * sizeof(E));
  const uint32_t rowb = (uint32_t)(d * sizeof(E));
  const int64_t rb = tr * a.K;
  // count, x slice and the first group's ids, all at once
  const int n = ok ? a.ell_cnt[tr] : 0;
  const R xv = *(const R*)((const E*)a.x + tr * d + col);
  int jraw = a.ell_idx[rb + min(i, a.K - 1)];
  int nmax = __builtin_amdgcn_readlane(n, 0);
  if constexpr (RPW == 2) nmax = max(nmax, __builtin_amdgcn_readlane(n, 32));
  if (nmax == 0) return;
  float xr[EPL];
  G::V::cvt(xv, xr);
  float* up = a.upart + ((int64_t)s * a.T + tr) * a.Kp;
  for (int k0 = 0; k0 < nmax; k0 += GRP) {
    if (k0 > 0) jraw = a.ell_idx[rb + min(k0 + i, a.K - 1)];
    const bool live = k0 + i < n;
    const int jl = live ? jraw : 0;
    // all 32 slots are loaded (slots past the count read neuron 0; their
    // totals are never stored)
    R w[GRP];
#pragma unroll
    for (int q = 0; q < GRP; ++q)
      w[q] = *(const R*)(wu + ((uint32_t)slot_id<RPW>(jl, q, hf) * rowb + colb));
    // keep every load of the group in flight before the first use
    __builtin_amdgcn_sched_barrier(0);
    float p[GRP];
#pragma unroll
    for (int q = 0; q < GRP; ++q) {
      if constexpr (sizeof(E) == 2) {
        // bf16 pairs straight into v_dot2c_f32_bf16 (the products of two
        // bf16 values are exact in fp32), fp32 accumulation
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL / 2; ++e) {
          const uint32_t xe = xv[e], we = w[q][e];
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xe),
                                                __builtin_bit_cast(bf16x2_t, we), acc, false);
        }
        p[q] = acc;
      } else {
        float f[EPL];
        G::V::cvt(w[q], f);
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(xr[e], f[e], acc);
        p[q] = acc;
      }
    }
    if constexpr (RPW == 2) {
      // totals over the 32 lanes of each row: lane i ends with slot k0 + i
      butterfly<16, 16>(p, lane);
      if (live) up[k0 + i] = p[0];
    } else {
      const float u = wave_sum32(p, lane);
      const int q = lane >> 1;
      if ((lane & 1) == 0 && k0 + q < n) up[k0 + q] = u;
    }
  }
}

// Between the phases (gated): u_k = sum of the slice partials in slice
// order and h_k = a_k * u_k, written over slice 0's partial (the lane that
// reads a slot's partials is the one that writes it); u_k is saved for
// training. One wave per row.
template <int NS>
__global__ __launch_bounds__(256) void hsum_kernel(SliceArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int n = a.ell_cnt[t];
  for (int k = lane; k < n; k += 64) {
    float u = 0.0f;
#pragma unroll
    for (int r = 0; r < NS; ++r) u += a.upart[((int64_t)r * a.T + t) * a.Kp + k];
    const int64_t q = t * a.K + k;
    if (a.ell_u) a.ell_u[q] = u;
    a.upart[t * a.Kp + k] = a.ell_a[q] * u;
  }
}

// Phase 2: y_t[slice s] = sum_k h_k * W_d[j_k][slice s], h_k from the sum
// above (non-gated: h_k = a_k). Rows routed to the dense backup are skipped.
template <typename E, int NS, int SW, bool GATED>
__global__ __launch_bounds__(256) void down_kernel(SliceArgs a) {
  using G = SliceGeom<E, SW>;
  constexpr int EPL = G::EPL, RPW = G::RPW;
  using R = typename G::R;
  const int lane = threadIdx.x & 63;
  const int hf = RPW == 2 ? lane >> 5 : 0;
  const int l = lane & (G::LPR - 1);
  const int i = lane & 31;
  const int s = blockIdx.x % NS;
  const int64_t t = ((int64_t)(blockIdx.x / NS) * 4 + (threadIdx.x >> 6)) * RPW + hf;
  if (t - hf >= a.T) return;
  const bool ok = t < a.T;
  const int64_t tr = ok ? t : a.T - 1;
  const int d = NS * SW;
  const int64_t col = (int64_t)s * SW + l * EPL;
  const char* wd = (const char*)a.wd;
  const uint32_t colb = (uint32_t)(col * sizeof(E));
  const uint32_t rowb = (uint32_t)(d * sizeof(E));
  const int64_t rb = tr * a.K;
  const bool store = ok && a.bk[tr] == 0;
  const int n = ok ? a.ell_cnt[tr] : 0;
  int nmax = __builtin_amdgcn_readlane(n, 0);
  if constexpr (RPW == 2) nmax = max(nmax, __builtin_amdgcn_readlane(n, 32));
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  for (int k0 = 0; k0 < nmax; k0 += GRP) {
    const int k = min(k0 + i, a.K - 1);
    const bool live = k0 + i < n;
    int jl = a.ell_idx[rb + k];
    float hl = GATED ? a.upart[tr * a.Kp + k] : a.ell_a[rb + k];
    jl = live ? jl : 0;
    hl = live ? hl : 0.0f;
    // blocks of 8 slots that some row of the wave has (wave-uniform); the
    // other slots of a block read neuron 0 with h = 0
    const int nb = (min(GRP, nmax - k0) + 7) >> 3;
    R w[GRP];
#pragma unroll
    for (int b = 0; b < GRP / 8; ++b)
      if (b < nb)
#pragma unroll
        for (int q = 8 * b; q < 8 * b + 8; ++q)
          w[q] = *(const R*)(wd + ((uint32_t)slot_id<RPW>(jl, q, hf) * rowb + colb));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < GRP / 8; ++b)
      if (b < nb)
#pragma unroll
        for (int q = 8 * b; q < 8 * b + 8; ++q) {
          const float h = slot_val<RPW>(hl, q, hf);
          float f[EPL];
          G::V::cvt(w[q], f);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] = fmaf(h, f[e], acc[e]);
        }
  }
  if (store) {
    float* yo = a.y + t * d + col;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) *(f32x4_t*)(yo + e) = f32x4_t{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
  }
}

template <typename E, int NS, int SW>
hipError_t launch_slices(const SliceArgs& a, bool gated, int phase, hipStream_t st) {
  constexpr int RPW = SliceGeom<E, SW>::RPW;
  const dim3 grid((unsigned)(NS * ((a.T + 4 * RPW - 1) / (4 * RPW))));
  if (phase == 0) {
    hipLaunchKernelGGL((up_partial_kernel<E, NS, SW>), grid, dim3(256), 0, st, a);
  } else if (phase == 2) {
    hipLaunchKernelGGL((hsum_kernel<NS>), dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, st, a);
  } else if (gated) {
    hipLaunchKernelGGL((down_kernel<E, NS, SW, true>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((down_kernel<E, NS, SW, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void gather_relu_rows_kernel(const float* __restrict__ z, int F,
                                                               const int32_t* __restrict__ rows,
                                                               const int32_t* __restrict__ n,
                                                               int cap, float* __restrict__ out) {
  const int R = device_rows(n, cap);
  const int f4 = F / 4;
  const int64_t total = (int64_t)R * f4;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(e / f4);
    const int c = (int)(e - (int64_t)m * f4) * 4;
    f32x4_t v = *(const f32x4_t*)(z + (int64_t)rows[m] * F + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = v[q] > 0.0f ? v[q] : 0.0f;
    *(f32x4_t*)(out + (int64_t)m * F + c) = v;
  }
}

}  // namespace

hipError_t launch_gather_relu_rows(const float* z, int F, const int32_t* rows, const int32_t* n,
                                   int cap, float* out, hipStream_t s) {
  hipLaunchKernelGGL(gather_relu_rows_kernel, dim3(512), dim3(256), 0, s, z, F, rows, n, cap, out);
  return hipGetLastError();
}

void slice_shape(Dtype, int d, int* ns, int* epl) {
  int n = d / 256;
  if (n > 8) n = 8;
  if (n < 1) n = 1;
  *ns = n;
  *epl = d / (64 * n);
}

hipError_t launch_rows(const EllArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(rows_kernel, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_backup_list(const uint8_t* bk, int64_t T, int32_t* brow, int64_t cap,
                              int32_t* n_backup, int32_t* slot, hipStream_t s) {
  hipLaunchKernelGGL(backup_list_kernel, dim3(1), dim3(1024), 0, s, bk, T, brow, cap, n_backup,
                     slot);
  return hipGetLastError();
}

hipError_t launch_updown(Dtype dt, bool gated, int phase, const SliceArgs& a, hipStream_t s) {
  int ns, epl;
  slice_shape(dt, a.d, &ns, &epl);
  const int sw = a.d / ns;
#define SFFN_SL(E, NS_, SW_) \
  if (ns == NS_ && sw == SW_) return launch_slices<E, NS_, SW_>(a, gated, phase, s);
  if (dt == kBF16) {
    SFFN_SL(uint16_t, 2, 256)
    SFFN_SL(uint16_t, 4, 256)
    SFFN_SL(uint16_t, 8, 256)
    SFFN_SL(uint16_t, 8, 512)
  } else {
    SFFN_SL(float, 1, 256)
    SFFN_SL(float, 2, 256)
    SFFN_SL(float, 4, 256)
    SFFN_SL(float, 8, 256)
  }
#undef SFFN_SL
  return hipErrorInvalidValue;
}

}  // namespace sffn
