// Sparse backward of the feedforward layer over the Hybrid format: the
// gradients are taken over the stored active entries, with the Hybrid
// regrouped by neuron for the weight gradients and no dense hidden tensor
// rebuilt (gist.science explainer of "Sparser, Faster, Lighter Transformer
// Language Models", 2. Methodology B, training kernels).
//
// For an active slot (neuron j, activation a, up value u) of ELL row t and
// upstream gradient dy_t: dh = dy_t . W_d[j]; dU = dh * a; dZ = dh * u + l1
// (gated; non-gated dZ = dh + l1), the ReLU mask being the slot itself.
// dx_t = sum dZ W_g[j] + dU W_u[j]; dW_g[j] = sum_t dZ x_t,
// dW_u[j] = sum_t dU x_t, dW_d[j] = sum_t (a u) dy_t.
//
// The partial dot products dy_t . W_d[j] reuse the sliced phase-1 kernel
// (sparse.hip); a row pass sums them into dZ, dU per slot. dx is
// accumulated per (row, d slice) like the forward's down projection. dW
// needs the slots grouped by neuron: a counting sort over blocks of slot
// units (per-block counts, per-neuron prefixes, in-order placement) gives
// every neuron its slots in ascending row order, so the float sums of dW
// are accumulated in a fixed order (no float atomics). Rows on the dense
// backup path are handled by GEMMs (api.hip) before the dW sums, which
// then add to the backup rows' stored products.
#include "sffn_internal.hpp"

namespace sffn {
namespace {

// dZ and dU per ELL slot from the slice partials of dh = dy . W_d[j]
// (summed in slice order): dU = dh * a, dZ = dh * u + l1 (non-gated
// dZ = dh + l1). One wave per row.
template <int NS, bool GATED>
__global__ __launch_bounds__(256) void dzu_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int n = a.ell_cnt[t];
  for (int k = lane; k < n; k += 64) {
    float dh = 0.0f;
#pragma unroll
    for (int r = 0; r < NS; ++r) dh += a.dpart[((int64_t)r * a.T + t) * a.Kp + k];
    const int64_t q = t * a.K + k;
    float gz, gu = 0.0f, hv;
    if constexpr (GATED) {
      const float av = sload(a.ell_a, q, a.store_bf16), uv = sload(a.ell_u, q, a.store_bf16);
      gu = dh * av;
      gz = dh * uv + a.l1;
      hv = av * uv;
    } else {
      gz = dh + a.l1;
      hv = sload(a.ell_a, q, a.store_bf16);
    }
    a.drec[q] = f32x4_t{__int_as_float((int)a.ell_idx[q]), gz, gu, hv};
  }
}

// dx of the ELL rows: dx_t = sum over the row's slots of dZ W_g[j] + dU W_u[j]
// (backup rows are left to the dense path). A lane loads 16 bytes of a
// weight row, a row's SW-column slice takes LPR lanes, so a wave sums RPW
// rows. Workgroup b runs on XCD b mod 8 and the blocks are ordered slice
// phase first, so an XCD gathers from one slice of W_g and W_u at a time
// (F * SW * 4 bytes, within its L2). The wave stages its rows' slot records
// {neuron, dZ, dU} in LDS, 64 per row at a time, and reads them back as
// broadcasts; records past a row's count are zero (neuron 0, no weight).
template <typename E, int SW, bool GATED, int GRP>
__device__ __forceinline__ void dx_sparse_rows(const BwdArgs& a, int64_t blk) {
  constexpr int EPL = 16 / (int)sizeof(E);
  constexpr int LPR = SW / EPL;
  constexpr int RPW = 64 / LPR;
  constexpr int CH = 64;
  static_assert(RPW >= 1 && RPW <= 8 && CH % GRP == 0, "slice geometry");
  using V = Vec<E, EPL>;
  using R = typename V::raw;
  __shared__ f32x4_t rec[4][RPW][CH];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPR;
  const int l = lane % LPR;
  const int nsl = a.d / SW;
  const int64_t nbk = (a.T + 4 * RPW - 1) / (4 * RPW);
  int slice;
  int64_t grp;
  if (nsl % 8 == 0) {
    const int64_t q = blk / 8;
    slice = (int)(q / nbk) * 8 + (int)(blk % 8);
    grp = q % nbk;
  } else {
    slice = (int)(blk % nsl);
    grp = blk / nsl;
  }
  const int64_t tw = (grp * 4 + wave) * RPW;
  if (tw >= a.T) return;
  const int64_t t = tw + r;
  const bool store = t < a.T && a.slot[t] < 0;
  const int n = store ? a.ell_cnt[t] : 0;
  int nmax = 0;
#pragma unroll
  for (int q = 0; q < RPW; ++q) nmax = max(nmax, __builtin_amdgcn_readlane(n, q * LPR));
  const int col = slice * SW + l * EPL;
  const char* wg = (const char*)a.wg;
  const char* wu = (const char*)a.wu;
  const uint32_t colb = (uint32_t)col * sizeof(E);
  const uint32_t rowb = (uint32_t)a.d * sizeof(E);
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  for (int k0 = 0; k0 < nmax; k0 += CH) {
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int nq = __builtin_amdgcn_readlane(n, q * LPR);
      f32x4_t v = {};
      if (k0 + lane < nq) v = a.drec[(tw + q) * a.K + k0 + lane];
      rec[wave][q][lane] = v;
    }
    // a wave's LDS accesses complete in issue order: no barrier is needed
    // between its own writes and reads
    const int m = min(CH, nmax - k0);
    for (int g0 = 0; g0 < m; g0 += GRP) {
      f32x4_t md[GRP];
      R w[GRP], w2[GATED ? GRP : 1];
#pragma unroll
      for (int k = 0; k < GRP; ++k) md[k] = rec[wave][r][g0 + k];
#pragma unroll
      for (int k = 0; k < GRP; ++k) {
        const uint32_t off = (uint32_t)__float_as_int(md[k][0]) * rowb + colb;
        w[k] = *(const R*)(wg + off);
        if constexpr (GATED) w2[k] = *(const R*)(wu + off);
      }
#pragma unroll
      for (int k = 0; k < GRP; ++k) {
        float f[EPL];
        V::cvt(w[k], f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(md[k][1], f[e], acc[e]);
        if constexpr (GATED) {
          V::cvt(w2[k], f);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] = fmaf(md[k][2], f[e], acc[e]);
        }
      }
    }
  }
  if (store) {
    float* o = a.dx + t * a.d + col;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) *(f32x4_t*)(o + e) = f32x4_t{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
  }
}

template <typename E, int SW, bool GATED, int GRP>
__global__ __launch_bounds__(256) void dx_sparse_kernel(BwdArgs a) {
  dx_sparse_rows<E, SW, GATED, GRP>(a, blockIdx.x);
}

// The same with the split-K reduce of the backup rows' dx product into their
// rows of dx (rows the ELL sums skip) in the first nred workgroups; nred is
// a multiple of 8, so that workgroup b of the sums still runs on XCD b mod 8.
template <typename E, int SW, bool GATED, int GRP>
__global__ __launch_bounds__(256) void dx_sparse_reduce_kernel(BwdArgs a, GemmArgs g, int nred) {
  if ((int)blockIdx.x < nred) {
    splitk_reduce_rows(g, a.dx, a.d, blockIdx.x, nred);
    return;
  }
  dx_sparse_rows<E, SW, GATED, GRP>(a, (int64_t)blockIdx.x - nred);
}

constexpr int kDwGrp = 4;   // slots in flight per wave in the dW sums

// ---------------------------------------------------------------- transpose

// The ELL slots grouped by neuron, ascending rows within a neuron, as a
// counting sort without global atomics. The slots are taken in units of 64
// (row t, slots 64c .. 64c + 63, ceil(K / 64) units per row, units in row
// order) and the units in blocks of kUnitsPerBlock. A neuron occurs at most
// once in a row, so its place is fixed by (block, order inside the block):
// per block a count of every neuron, per neuron the prefix of its block
// counts, then per block the units in order. A neuron's count inside a
// block is below 256: the counts are bytes, four to a 32-bit word, in LDS.
constexpr int kUnitsPerBlock = 32;

// The first kUnitsPerBlock units of block b: lane i < nu returns the
// number of slots of unit i (of its row's slots from 64 c on, at most 64
// used), with t0 / c0 the row and chunk of the block's first unit. The
// counts are loaded by all lanes at once, not one dependent load per unit.
__device__ __forceinline__ int unit_counts(const BwdArgs& a, int cpr, int u0, int nu, int lane,
                                           int& t0, int& c0) {
  t0 = u0 / cpr;
  c0 = u0 - t0 * cpr;
  int n = 0;
  if (lane < nu) {
    const int u = u0 + lane;
    const int t = u / cpr;
    n = a.ell_cnt[t] - (u - t * cpr) * 64;
  }
  return n;
}

// Per block of units: every neuron's count, as bytes [nblk][F4 words].
__global__ __launch_bounds__(256) void block_count_kernel(BwdArgs a, int cpr, int nunits, int F4,
                                                          uint32_t* __restrict__ hist) {
  extern __shared__ uint32_t c4[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < F4; i += 256) c4[i] = 0;
  const int u0 = blockIdx.x * kUnitsPerBlock;
  const int nu = min(kUnitsPerBlock, nunits - u0);
  int t0, c0;
  const int ucnt = unit_counts(a, cpr, u0, nu, lane, t0, c0);
  // wave w takes units w, w + 4, ...: ids first, then the counts
  constexpr int PER = kUnitsPerBlock / 4;
  int jv[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int i = p * 4 + wave;
    const int n = __builtin_amdgcn_readlane(ucnt, i);
    const int c = c0 + i;
    const int64_t t = t0 + c / cpr;
    const int k = (c % cpr) * 64 + lane;
    jv[p] = (i < nu && lane < n) ? (int)a.ell_idx[t * a.K + k] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < PER; ++p)
    if (jv[p] >= 0) atomicAdd(&c4[jv[p] >> 2], 1u << ((jv[p] & 3) * 8));
  __syncthreads();
  for (int i = tid; i < F4; i += 256) hist[(int64_t)blockIdx.x * F4 + i] = c4[i];
}

// Per neuron: the exclusive prefix of its block counts (off [nblk][4 F4])
// and its total (ncnt). A workgroup takes 64 neurons (16 count words);
// thread (s, w) sums word w over the s-th of 16 runs of blocks, the runs'
// sums are combined in LDS, then each thread writes its run's prefixes.
// The run is read in batches of 16 loads.
__global__ __launch_bounds__(256) void block_scan_kernel(const uint32_t* __restrict__ hist,
                                                         int nblk, int F4,
                                                         int32_t* __restrict__ off,
                                                         int32_t* __restrict__ ncnt) {
  __shared__ i32x4_t part[16][16];
  const int w = threadIdx.x & 15;
  const int s = threadIdx.x >> 4;
  const int W = blockIdx.x * 16 + w;
  const int L = (nblk + 15) / 16;
  const int b0 = min(nblk, s * L), b1 = min(nblk, b0 + L);
  auto bytes = [](uint32_t v) {
    return i32x4_t{(int)(v & 0xFF), (int)((v >> 8) & 0xFF), (int)((v >> 16) & 0xFF), (int)(v >> 24)};
  };
  i32x4_t sum = {0, 0, 0, 0};
  if (W < F4) {
    for (int bb = b0; bb < b1; bb += 16) {
      uint32_t v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = bb + q < b1 ? hist[(int64_t)(bb + q) * F4 + W] : 0u;
#pragma unroll
      for (int q = 0; q < 16; ++q) sum += bytes(v[q]);
    }
  }
  part[s][w] = sum;
  __syncthreads();
  i32x4_t base = {0, 0, 0, 0}, total = {0, 0, 0, 0};
  for (int q = 0; q < 16; ++q) {
    if (q < s) base += part[q][w];
    total += part[q][w];
  }
  if (W >= F4) return;
  for (int bb = b0; bb < b1; bb += 16) {
    uint32_t v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = bb + q < b1 ? hist[(int64_t)(bb + q) * F4 + W] : 0u;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (bb + q < b1) *(i32x4_t*)(off + ((int64_t)(bb + q) * F4 + W) * 4) = base;
      base += bytes(v[q]);
    }
  }
  if (s == 0) *(i32x4_t*)(ncnt + (int64_t)W * 4) = total;
}

// Exclusive scan of the F counts into F + 1 offsets; one workgroup.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ ncnt, int F,
                                                    int32_t* __restrict__ noff) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < F; base += 1024) {
    const int j = base + tid;
    const int c = j < F ? ncnt[j] : 0;
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
    if (j < F) noff[j] = carry + wbase + inc - c;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) noff[F] = carry;
}

// Per block of units, one wave: the units in order, each slot taking the
// next place of its neuron (noff + block prefix + the block's earlier
// units holding the neuron), stored as the record the dW sums read: {row,
// dZ, dU, h}. The neuron ids are loaded first, then the places are taken
// in unit order (a wave's LDS operations complete in issue order), then
// the records are moved, the loads of all 32 units issued together.
__global__ __launch_bounds__(64) void block_place_kernel(BwdArgs a, int cpr, int nunits, int F4,
                                                         const int32_t* __restrict__ off) {
  extern __shared__ uint32_t c4[];
  const int lane = threadIdx.x;
  for (int i = lane; i < F4; i += 64) c4[i] = 0;
  const int u0 = blockIdx.x * kUnitsPerBlock;
  const int nu = min(kUnitsPerBlock, nunits - u0);
  int t0, c0;
  const int ucnt = unit_counts(a, cpr, u0, nu, lane, t0, c0);
  int jv[kUnitsPerBlock];
  int64_t q[kUnitsPerBlock];
#pragma unroll
  for (int i = 0; i < kUnitsPerBlock; ++i) {
    const int n = __builtin_amdgcn_readlane(ucnt, i);
    const int c = c0 + i;
    const int64_t t = t0 + c / cpr;
    q[i] = t * a.K + (c % cpr) * 64 + lane;
    jv[i] = (i < nu && lane < n) ? (int)a.ell_idx[q[i]] : -1;
  }
  int loc[kUnitsPerBlock];
#pragma unroll
  for (int i = 0; i < kUnitsPerBlock; ++i) {
    loc[i] = 0;
    if (jv[i] >= 0) {
      const int sh = (jv[i] & 3) * 8;
      loc[i] = (int)((atomicAdd(&c4[jv[i] >> 2], 1u << sh) >> sh) & 0xFF);
    }
  }
  const int32_t* offb = off + (int64_t)blockIdx.x * F4 * 4;
  constexpr int G = 32;
#pragma unroll
  for (int g0 = 0; g0 < kUnitsPerBlock; g0 += G) {
    int pos[G];
    f32x4_t r[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int j = max(jv[g0 + i], 0);
      pos[i] = a.noff[j] + offb[j] + loc[g0 + i];
      r[i] = jv[g0 + i] >= 0 ? a.drec[q[g0 + i]] : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (jv[g0 + i] < 0) continue;
      const int t = t0 + (c0 + g0 + i) / cpr;
      a.meta[pos[i]] = f32x4_t{__int_as_float(t), r[i][1], r[i][2], r[i][3]};
    }
  }
}

// dW rows of every neuron: the sums over the neuron's ELL slots in
// ascending row order of (dZ*x, dU*x) (SIDE 0: dW_g, dW_u) or h*dy (SIDE 1:
// dW_d), added to dW's rows when accumulating (the backup rows' products
// are stored there); otherwise neurons without slots get zero rows. A lane
// loads 16 bytes of a row, a neuron's SW-column slice takes LPR lanes, so a
// wave sums RPW neurons. The rows a slice gathers are random over all T
// rows, so an XCD keeps to one slice at a time: workgroup b runs on XCD b
// mod 8 and the blocks are ordered slice phase first, so that the columns
// in use on an XCD (T * SW * 2 bytes of x or of dy: one operand per launch)
// stay within its L2. The wave stages the slot records of its neurons in
// LDS, 64 per neuron at a time, and reads them back as broadcasts; records
// past a neuron's count are zero (row 0, no weight).
template <typename E, int SW, bool GATED, int GRP, int SIDE>
__global__ __launch_bounds__(256) void dw_sparse_kernel(BwdArgs a) {
  constexpr int EPL = 16 / (int)sizeof(E);
  constexpr int LPR = SW / EPL;
  constexpr int RPW = 64 / LPR;
  constexpr int CH = 64;
  constexpr bool TWO = SIDE == 0 && GATED;   // dW_g and dW_u from the same x rows
  static_assert(RPW >= 1 && RPW <= 8 && CH % GRP == 0, "slice geometry");
  using V = Vec<E, EPL>;
  using R = typename V::raw;
  __shared__ f32x4_t rec[4][RPW][CH];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPR;
  const int l = lane % LPR;
  const int nsl = a.d / SW;
  const int nbk = (a.F + 4 * RPW - 1) / (4 * RPW);
  int slice, grp;
  if (nsl % 8 == 0) {
    const int q = blockIdx.x / 8;
    slice = (q / nbk) * 8 + blockIdx.x % 8;
    grp = q % nbk;
  } else {
    slice = blockIdx.x % nsl;
    grp = blockIdx.x / nsl;
  }
  const int jw = (grp * 4 + wave) * RPW;
  if (jw >= a.F) return;
  const int j = jw + r;
  const bool ok = j < a.F;
  const int b0 = ok ? a.noff[j] : 0;
  const int n = ok ? a.noff[j + 1] - b0 : 0;
  int nmax = 0;
#pragma unroll
  for (int q = 0; q < RPW; ++q) nmax = max(nmax, __builtin_amdgcn_readlane(n, q * LPR));
  const int col = slice * SW + l * EPL;
  const int64_t ro = (int64_t)j * a.d + col;
  const E* src = (const E*)(SIDE == 0 ? a.x : a.dy) + col;
  float* out0 = SIDE == 0 ? a.dwg : a.dwd;
  float* out1 = a.dwu;
  float g0[EPL], g1[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) g0[e] = g1[e] = 0.0f;
  if (a.accumulate && ok) {
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const f32x4_t v0 = *(const f32x4_t*)(out0 + ro + e);
      f32x4_t v1 = {};
      if (TWO) v1 = *(const f32x4_t*)(out1 + ro + e);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        g0[e + c] = v0[c];
        g1[e + c] = v1[c];
      }
    }
  }
  for (int i0 = 0; i0 < nmax; i0 += CH) {
    // stage the records of slots i0 .. i0+63 of the wave's neurons
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int bq = __builtin_amdgcn_readlane(b0, q * LPR);
      const int nq = __builtin_amdgcn_readlane(n, q * LPR);
      f32x4_t v = {};
      if (i0 + lane < nq) v = a.meta[bq + i0 + lane];
      rec[wave][q][lane] = v;
    }
    // a wave's LDS accesses complete in issue order: no barrier is needed
    // between its own writes and reads
    const int m = min(CH, nmax - i0);
    for (int gg = 0; gg < m; gg += GRP) {
      f32x4_t md[GRP];
      R xv[GRP];
#pragma unroll
      for (int k = 0; k < GRP; ++k) md[k] = rec[wave][r][gg + k];
#pragma unroll
      for (int k = 0; k < GRP; ++k) xv[k] = *(const R*)(src + (int64_t)__float_as_int(md[k][0]) * a.d);
#pragma unroll
      for (int k = 0; k < GRP; ++k) {
        float fx[EPL];
        V::cvt(xv[k], fx);
        const float w0 = SIDE == 0 ? md[k][1] : md[k][3];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          g0[e] = fmaf(w0, fx[e], g0[e]);
          if (TWO) g1[e] = fmaf(md[k][2], fx[e], g1[e]);
        }
      }
    }
  }
  if (ok) {
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      *(f32x4_t*)(out0 + ro + e) = f32x4_t{g0[e], g0[e + 1], g0[e + 2], g0[e + 3]};
      if (TWO) *(f32x4_t*)(out1 + ro + e) = f32x4_t{g1[e], g1[e + 1], g1[e + 2], g1[e + 3]};
    }
  }
}

// ---------------------------------------------------------------- backup rows

// Rows r < R of x (and dy) gathered through brow into the k-stacked
// operands of the dW GEMMs: bf16 [2Rp, d] (rows r and Rp + r both hold
// row brow[r], others zero; the hi and lo parts of the gradient rows meet
// the same data) or fp32 [Rp, d].
template <typename E>
__global__ __launch_bounds__(256) void gather_stack_kernel(const E* __restrict__ src, int d,
                                                           const int32_t* __restrict__ brow,
                                                           const int32_t* __restrict__ n, int cap,
                                                           E* __restrict__ dst) {
  constexpr int REP = sizeof(E) == 2 ? 2 : 1;
  const int R = device_rows(n, cap);
  const int Rp = (R + 63) / 64 * 64;
  constexpr int EPV = 16 / sizeof(E);
  const int dv = d / EPV;
  const int64_t total = (int64_t)REP * Rp * dv;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int row = (int)(e / dv);
    const int c = (int)(e - (int64_t)row * dv) * EPV;
    const int r = row % Rp;
    u32x4_t v = {0, 0, 0, 0};
    if (r < R) v = *(const u32x4_t*)(src + (int64_t)brow[r] * d + c);
    *(u32x4_t*)(dst + (int64_t)row * d + c) = v;
  }
}

// bf16: the same rows transposed, column-major [d, ldt]: column c holds
// x[brow[r]][c] at k = r and k = Rp + r for r < R, zeros up to 2 Rp, so that
// both operands of the dW GEMMs are k-contiguous. A workgroup moves 64 rows
// x 64 columns through LDS: 16-byte loads along the rows, 16-byte stores
// along the columns.
__global__ __launch_bounds__(256) void gather_stack_t_kernel(GatherT a) {
  gather_stack_t_tiles(a, blockIdx.x, gridDim.x, blockIdx.y);
}

// From dH of the backup rows: dZ, dU (and H = a u for dW_d) in the layouts
// of the GEMMs that consume them. Row-major rows of stride ld_rm, hi | lo
// (bf16, 2F wide) or fp32 (F wide), for dx; neuron-major rows of stride ldt holding hi in
// columns [0, Rp) and lo in [Rp, 2Rp), zero past R (bf16), or [0, Rp)
// (fp32), for dW. A workgroup takes 64 rows x 64 neurons at a time; a
// thread takes two neighbouring neurons of a row on the row-major side and
// two neighbouring rows of a neuron on the neuron-major side (through LDS),
// so every access is coalesced and at least 4 bytes wide.
template <typename E, bool GATED>
__global__ __launch_bounds__(256) void backup_grad_kernel(BwdArgs a) {
  constexpr bool BF = sizeof(E) == 2;
  // per element: hi | lo << 16 (bf16) or the fp32 bits; [neuron][row]
  __shared__ uint32_t tz[64][66], tu[64][66], th[64][66];
  const int R = device_rows(a.n_backup, a.cap);
  const int Rp = (R + 63) / 64 * 64;
  const int F = a.F;
  const int tid = threadIdx.x;
  const int c2 = (tid & 31) * 2;   // neuron pair (load side) or row pair (store side)
  const int g = tid >> 5;
  const int ntj = F / 64;
  const int ntiles = (Rp / 64) * ntj;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int r0 = (tile / ntj) * 64;
    const int j0 = (tile - (tile / ntj) * ntj) * 64;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int rl = p * 8 + g;
      const int r = r0 + rl;
      const int j = j0 + c2;
      float dz[2] = {0.0f, 0.0f}, du[2] = {0.0f, 0.0f}, h[2] = {0.0f, 0.0f};
      if (r < R) {
        const int64_t q = (int64_t)r * F + j;
        const f32x2_t dh = *(const f32x2_t*)(a.dH + q);
        const f32x2_t av = sload2(a.bk_a, q, a.store_bf16);
        f32x2_t uv = {0.0f, 0.0f};
        if (GATED) uv = sload2(a.bk_u, q, a.store_bf16);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const bool on = av[e] > 0.0f;
          if constexpr (GATED) {
            du[e] = dh[e] * av[e];
            dz[e] = on ? dh[e] * uv[e] + a.l1 : 0.0f;
            h[e] = av[e] * uv[e];
          } else {
            dz[e] = on ? dh[e] + a.l1 : 0.0f;
            h[e] = av[e];
          }
        }
      }
      if constexpr (BF) {
        uint32_t zh[2], zl[2], uh[2], ul[2], hh[2], hl[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          zh[e] = f32_to_bf16(dz[e]);
          uh[e] = f32_to_bf16(du[e]);
          hh[e] = f32_to_bf16(h[e]);
          zl[e] = f32_to_bf16(dz[e] - __uint_as_float(zh[e] << 16));
          ul[e] = f32_to_bf16(du[e] - __uint_as_float(uh[e] << 16));
          hl[e] = f32_to_bf16(h[e] - __uint_as_float(hh[e] << 16));
          tz[c2 + e][rl] = zh[e] | (zl[e] << 16);
          tu[c2 + e][rl] = uh[e] | (ul[e] << 16);
          th[c2 + e][rl] = hh[e] | (hl[e] << 16);
        }
        if (r < R) {
          uint32_t* gzr = (uint32_t*)((uint16_t*)a.gz_rm + r * a.ld_rm + j);
          gzr[0] = zh[0] | (zh[1] << 16);
          gzr[F / 2] = zl[0] | (zl[1] << 16);
          if (GATED) {
            uint32_t* gur = (uint32_t*)((uint16_t*)a.gu_rm + r * a.ld_rm + j);
            gur[0] = uh[0] | (uh[1] << 16);
            gur[F / 2] = ul[0] | (ul[1] << 16);
          }
        }
      } else {
        if (r < R) {
          *(f32x2_t*)((float*)a.gz_rm + r * a.ld_rm + j) = f32x2_t{dz[0], dz[1]};
          if (GATED) *(f32x2_t*)((float*)a.gu_rm + r * a.ld_rm + j) = f32x2_t{du[0], du[1]};
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          tz[c2 + e][rl] = __float_as_uint(dz[e]);
          tu[c2 + e][rl] = __float_as_uint(du[e]);
          th[c2 + e][rl] = __float_as_uint(h[e]);
        }
      }
    }
    __syncthreads();
#pragma unroll 2
    for (int p = 0; p < 8; ++p) {
      const int jl = p * 8 + g;
      const int64_t tr = (int64_t)(j0 + jl) * a.ldt + r0 + c2;
      const uint32_t z0 = tz[jl][c2], z1 = tz[jl][c2 + 1];
      const uint32_t u0 = tu[jl][c2], u1 = tu[jl][c2 + 1];
      const uint32_t h0 = th[jl][c2], h1 = th[jl][c2 + 1];
      if constexpr (BF) {
        uint32_t* gzt = (uint32_t*)((uint16_t*)a.gz_t + tr);
        gzt[0] = (z0 & 0xFFFFu) | (z1 << 16);
        gzt[Rp / 2] = (z0 >> 16) | (z1 & 0xFFFF0000u);
        if (GATED) {
          uint32_t* gut = (uint32_t*)((uint16_t*)a.gu_t + tr);
          gut[0] = (u0 & 0xFFFFu) | (u1 << 16);
          gut[Rp / 2] = (u0 >> 16) | (u1 & 0xFFFF0000u);
        }
        uint32_t* ght = (uint32_t*)((uint16_t*)a.gh_t + tr);
        ght[0] = (h0 & 0xFFFFu) | (h1 << 16);
        ght[Rp / 2] = (h0 >> 16) | (h1 & 0xFFFF0000u);
      } else {
        *(f32x2_t*)((float*)a.gz_t + tr) = f32x2_t{__uint_as_float(z0), __uint_as_float(z1)};
        if (GATED)
          *(f32x2_t*)((float*)a.gu_t + tr) = f32x2_t{__uint_as_float(u0), __uint_as_float(u1)};
        *(f32x2_t*)((float*)a.gh_t + tr) = f32x2_t{__uint_as_float(h0), __uint_as_float(h1)};
      }
    }
    __syncthreads();
  }
}

template <typename E, int NS, int SW>
hipError_t launch_bwd_t(const BwdArgs& a, bool gated, int which, hipStream_t st) {
  if (which == 0 || which == 2) {
    const dim3 rows((unsigned)((a.T + 3) / 4));
    if (gated) hipLaunchKernelGGL((dzu_kernel<NS, true>), rows, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((dzu_kernel<NS, false>), rows, dim3(256), 0, st, a);
  }
  if (which == 0 || which == 3) {
    // 128-column slices (bf16: four rows per wave)
    constexpr int XSW = 128;
    constexpr int XRPW = 64 / (XSW * (int)sizeof(E) / 16);
    const dim3 grid((unsigned)((a.d / XSW) * ((a.T + 4 * XRPW - 1) / (4 * XRPW))));
    if (gated) hipLaunchKernelGGL((dx_sparse_kernel<E, XSW, true, 4>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((dx_sparse_kernel<E, XSW, false, 4>), grid, dim3(256), 0, st, a);
  }
  if (which == 1) {
    // 256-column slices (bf16: two neurons per wave): one gathered operand
    // per launch keeps an XCD's slice of it (T x 512 bytes) near its L2
    constexpr int DSW = 256;
    constexpr int DRPW = 64 / (DSW * (int)sizeof(E) / 16);
    const dim3 grid((unsigned)((a.d / DSW) * ((a.F + 4 * DRPW - 1) / (4 * DRPW))));
    // x side (dW_g, dW_u), then dy side (dW_d): one gathered operand per launch
    if (gated) {
      hipLaunchKernelGGL((dw_sparse_kernel<E, DSW, true, kDwGrp, 0>), grid, dim3(256), 0, st, a);
      hipLaunchKernelGGL((dw_sparse_kernel<E, DSW, true, kDwGrp, 1>), grid, dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL((dw_sparse_kernel<E, DSW, false, kDwGrp, 0>), grid, dim3(256), 0, st, a);
      hipLaunchKernelGGL((dw_sparse_kernel<E, DSW, false, kDwGrp, 1>), grid, dim3(256), 0, st, a);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_sparse(Dtype dt, bool gated, int which, const BwdArgs& a, hipStream_t s) {
  int ns, epl;
  slice_shape(dt, a.d, &ns, &epl);
  const int sw = a.d / ns;
#define SFFN_BW(E, NS_, SW_) \
  if (ns == NS_ && sw == SW_) return launch_bwd_t<E, NS_, SW_>(a, gated, which, s);
  if (dt == kBF16) {
    SFFN_BW(uint16_t, 2, 256)
    SFFN_BW(uint16_t, 4, 256)
    SFFN_BW(uint16_t, 8, 256)
    SFFN_BW(uint16_t, 8, 512)
  } else {
    SFFN_BW(float, 1, 256)
    SFFN_BW(float, 2, 256)
    SFFN_BW(float, 4, 256)
    SFFN_BW(float, 8, 256)
  }
#undef SFFN_BW
  return hipErrorInvalidValue;
}

int64_t transpose_blocks(int64_t T, int K) {
  const int64_t nunits = T * ((K + 63) / 64);
  return (nunits + kUnitsPerBlock - 1) / kUnitsPerBlock;
}

hipError_t launch_transpose(const BwdArgs& a, hipStream_t s) {
  const int cpr = (a.K + 63) / 64;
  const int nunits = (int)(a.T * cpr);
  const int64_t nblk = transpose_blocks(a.T, a.K);
  const int F4 = (a.F + 3) / 4;
  if (nblk == 0 || F4 * 4 > 65536) return hipErrorInvalidValue;
  const size_t lds = (size_t)F4 * 4;
  hipLaunchKernelGGL(block_count_kernel, dim3((unsigned)nblk), dim3(256), lds, s, a, cpr, nunits,
                     F4, a.thist);
  hipLaunchKernelGGL(block_scan_kernel, dim3((unsigned)((F4 + 15) / 16)), dim3(256), 0, s,
                     a.thist, (int)nblk, F4, a.toff, a.ncnt);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, a.ncnt, a.F, a.noff);
  hipLaunchKernelGGL(block_place_kernel, dim3((unsigned)nblk), dim3(64), lds, s, a, cpr, nunits,
                     F4, a.toff);
  return hipGetLastError();
}

GatherT gather_args(const BwdArgs& a) {
  return GatherT{(const uint16_t*)a.x, (const uint16_t*)a.dy, a.d, a.brow, a.n_backup, a.cap,
                 (uint16_t*)a.xb, (uint16_t*)a.dyb, a.ldt};
}

hipError_t launch_dx_with_reduce(Dtype dt, bool gated, const BwdArgs& a, const GemmArgs& g,
                                 hipStream_t s) {
  if (dt != kBF16) return hipErrorInvalidValue;
  constexpr int XSW = 128;
  constexpr int XRPW = 64 / (XSW * 2 / 16);
  if (a.d % XSW != 0) return hipErrorInvalidValue;
  const int nred = 256;
  const dim3 grid((unsigned)(nred + (a.d / XSW) * ((a.T + 4 * XRPW - 1) / (4 * XRPW))));
  if (gated)
    hipLaunchKernelGGL((dx_sparse_reduce_kernel<uint16_t, XSW, true, 4>), grid, dim3(256), 0, s, a, g, nred);
  else
    hipLaunchKernelGGL((dx_sparse_reduce_kernel<uint16_t, XSW, false, 4>), grid, dim3(256), 0, s, a, g, nred);
  return hipGetLastError();
}

hipError_t launch_backup_prep(Dtype dt, bool gated, const BwdArgs& a, hipStream_t s) {
  const dim3 g(1024), b(256);
  if (dt == kBF16) {
    hipLaunchKernelGGL(gather_stack_t_kernel, dim3(kGatherBlocks, 2), b, 0, s, gather_args(a));
  } else {
    hipLaunchKernelGGL(gather_stack_kernel<float>, g, b, 0, s, (const float*)a.x, a.d, a.brow,
                       a.n_backup, a.cap, (float*)a.xb);
    hipLaunchKernelGGL(gather_stack_kernel<float>, g, b, 0, s, (const float*)a.dy, a.d, a.brow,
                       a.n_backup, a.cap, (float*)a.dyb);
  }
  return hipGetLastError();
}

hipError_t launch_backup_grad(Dtype dt, bool gated, const BwdArgs& a, hipStream_t s) {
  const dim3 g(1024), b(256);
  if (dt == kBF16) {
    if (gated) hipLaunchKernelGGL((backup_grad_kernel<uint16_t, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((backup_grad_kernel<uint16_t, false>), g, b, 0, s, a);
  } else {
    if (gated) hipLaunchKernelGGL((backup_grad_kernel<float, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((backup_grad_kernel<float, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace sffn
