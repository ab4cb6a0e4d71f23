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
// cut into 256-column slices (up: 512 at d = 4096, where 8 slices cover
// it) and each grid is ordered so that an XCD works
// on one slice at a time, so its L2 holds one slice of W_up or W_down
// (5632 x 256 bf16 = 2.9 MB at the 1.5B shape) instead of streaming whole
// 4 KB neuron rows from HBM/MALL. Phase 1 writes per-slice partial dot
// products (one float per active pair and slice); a small kernel sums them
// in slice order (deterministic) and scales by the activation; phase 2 adds
// the neurons' down weights into the rows' y slices. No dense hidden tensor
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
// into ELL slots 0..nnz-1. Lane b takes tile b (64 tiles per pass) and an
// exclusive prefix of the counts gives each tile's first ELL slot (kept in
// LDS); then the wave copies the row's slots 64 at a time, lane o taking
// ELL slot o from the tile whose range holds it (binary search of the tile
// starts), so loads and stores are contiguous runs.
constexpr int kMaxTiles = 512;   // F <= 65408 with 128-column tiles

__global__ __launch_bounds__(256) void rows_kernel(EllArgs a) {
  __shared__ int tstart[4][kMaxTiles + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
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
  int* ts = tstart[wave];
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
    if (b < a.n_t) ts[b] = base + inc - c;
    base += __shfl(inc, 63, 64);
  }
  // a wave's LDS accesses complete in issue order: no barrier is needed
  // between its own writes and reads
  const int64_t dst = t * (int64_t)a.K;
  const int64_t src0 = t * a.n_t * (int64_t)a.C;
  for (int o0 = 0; o0 < nnz; o0 += 64) {
    const int o = o0 + lane;
    if (o < nnz) {
      // the last tile whose start is <= o (empty tiles share a start with
      // the next tile and are skipped by taking the last)
      int lo = 0, hi = a.n_t - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ts[mid] <= o) lo = mid;
        else hi = mid - 1;
      }
      const int64_t src = src0 + (int64_t)lo * a.C + (o - ts[lo]);
      a.ell_idx[dst + o] = a.idx[src];
      // the stored value as is (fp32 or bf16 bits)
      if (a.store_bf16) ((uint16_t*)a.ell_a)[dst + o] = ((const uint16_t*)a.val)[src];
      else ((float*)a.ell_a)[dst + o] = ((const float*)a.val)[src];
    }
  }
}

// One workgroup of NTH threads: list the backup rows in ascending order
// (the first cap of them), their true count and, when requested, every
// row's backup slot (-1 for ELL rows).
template <int NTH>
__device__ __forceinline__ void list_rows(const ListArgs& L, int64_t T) {
  const uint8_t* __restrict__ bk = L.bk;
  int32_t* __restrict__ brow = L.brow;
  const int64_t cap = L.cap;
  int32_t* __restrict__ n_backup = L.n;
  int32_t* __restrict__ slot = L.slot;
  constexpr int RPT = 16;
  constexpr int NW = NTH / 64;
  __shared__ int wsum[NW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int carry = 0;
  for (int64_t base = 0; base < T; base += NTH * RPT) {
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
    for (int k = 0; k < NW; ++k) {
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
  if (tid == 0) {
    *n_backup = carry;
    if (L.status && carry > cap) *L.status = 1;
  }
  if (L.reset)
    for (int i = tid; i < L.n_reset; i += NTH) L.reset[i * kCtrStride] = 0;
}

__global__ __launch_bounds__(1024) void backup_list_kernel(ListArgs l0, ListArgs l1, int64_t T) {
  // workgroup b builds list b (two lists in one launch in training)
  list_rows<1024>(blockIdx.x ? l1 : l0, T);
}

// Sum over the 8 lanes of each lane octet, result in all 8 (quad swaps,
// then the half-row mirror pairs lane i with 7 - i); a fixed order.
__device__ __forceinline__ float octet_sum(float v) {
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, true);  // row_half_mirror
  return v;
}

// Phase 1: upart[s][t][k] = x_t[slice s] . W_u[j_k][slice s]. One row per
// wave; the wave's 8 lane octets take 8 slots at once, an octet's lanes
// split the SW-column slice (16-byte loads, 8 lanes cover 128 contiguous
// bytes) and an octet sum gives the slot's partial. The row's neuron ids
// are staged in LDS, 64 at a time, and read back as broadcasts; ids past
// the count are 0 (the partial is not stored). Workgroup b runs on XCD
// b mod 8, so with 8 slices an XCD gathers from one slice of W_u.
template <typename E, int NS, int SW>
__device__ __forceinline__ void up_partial(const SliceArgs& a, int64_t blk) {
  constexpr int EPL = 16 / (int)sizeof(E);
  constexpr int NLD = SW / 8 / EPL;      // 16-byte loads per lane per slot
  constexpr int CH = 64;
  constexpr int U = 1;                   // steps of 8 slots in flight
  using R = u32x4_t;
  __shared__ int rec[4][CH];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 3;
  const int l = lane & 7;
  const int s = (int)(blk % NS);
  const int64_t t = (blk / NS) * 4 + wave;
  if (t >= a.T) return;
  const int n = a.ell_cnt[t];
  if (n == 0) return;
  // this lane's columns of load i: s * SW + i * 8 * EPL + l * EPL
  const int col0 = s * SW + l * EPL;
  const char* wu = (const char*)a.wu;
  const uint32_t colb = (uint32_t)col0 * sizeof(E);
  const uint32_t rowb = (uint32_t)a.d * sizeof(E);
  R xv[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) xv[i] = *(const R*)((const E*)a.x + t * a.d + col0 + i * 8 * EPL);
  float* up = a.upart + ((int64_t)s * a.T + t) * a.Kp;
  for (int c0 = 0; c0 < n; c0 += CH) {
    rec[wave][lane] = c0 + lane < n ? (int)a.ell_idx[t * a.K + c0 + lane] : 0;
    // a wave's LDS accesses complete in issue order: no barrier is needed
    // between its own writes and reads
    const int m = min(CH, n - c0);
    for (int k0 = 0; k0 < m; k0 += 8 * U) {
      R w[U][NLD];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t off = (uint32_t)rec[wave][k0 + 8 * u + g] * rowb + colb;
#pragma unroll
        for (int i = 0; i < NLD; ++i) w[u][i] = *(const R*)(wu + off + i * 8 * 16);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          if constexpr (sizeof(E) == 2) {
            // bf16 pairs straight into v_dot2c_f32_bf16 (the products of two
            // bf16 values are exact in fp32), fp32 accumulation
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t xe = xv[i][e], we = w[u][i][e];
              acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xe),
                                                    __builtin_bit_cast(bf16x2_t, we), acc, false);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc = fmaf(__uint_as_float(xv[i][e]), __uint_as_float(w[u][i][e]), acc);
          }
        }
        acc = octet_sum(acc);
        const int k = c0 + k0 + 8 * u + g;
        if (l == 0 && k0 + 8 * u + g < m) up[k] = acc;
      }
    }
  }
}

template <typename E, int NS, int SW>
__global__ __launch_bounds__(256) void up_partial_kernel(SliceArgs a) {
  up_partial<E, NS, SW>(a, blockIdx.x);
}

// The same with the dense path's row lists (one or two) built beside it:
// workgroups 0 .. 7 are the list builders (those past the lists return at
// once; eight keep workgroup b of the up projection on XCD b mod 8).
template <typename E, int NS, int SW>
__global__ __launch_bounds__(256) void up_partial_list_kernel(SliceArgs a, ListArgs l0,
                                                               ListArgs l1, int nl, int64_t T) {
  if (blockIdx.x < 8) {
    if ((int)blockIdx.x < nl) list_rows<256>(blockIdx.x ? l1 : l0, T);
    return;
  }
  up_partial<E, NS, SW>(a, (int64_t)blockIdx.x - 8);
}

// The backward's dh (phase 0 on dy and W_d) with the backup rows' x and dy
// gathered beside it: workgroups [0, 2 kGatherBlocks) gather (a multiple of
// 8, so that workgroup b of the products still runs on XCD b mod 8).
template <typename E, int NS, int SW>
__global__ __launch_bounds__(256) void up_partial_gather_kernel(SliceArgs a, GatherT gt) {
  if (blockIdx.x < 2 * kGatherBlocks) {
    gather_stack_t_tiles(gt, blockIdx.x % kGatherBlocks, kGatherBlocks, blockIdx.x / kGatherBlocks);
    return;
  }
  up_partial<E, NS, SW>(a, (int64_t)blockIdx.x - 2 * kGatherBlocks);
}

// Between the phases (gated): the slice sums (hsum_rows, in the header,
// shared with the dense path's combine launch)
template <int NS>
__global__ __launch_bounds__(256) void hsum_kernel(SliceArgs a) {
  hsum_rows<NS>(a, blockIdx.x);
}

// Phase 2: y_t = sum_k h_k * W_d[j_k], h_k from the sum above (non-gated:
// h_k = a_k); rows routed to the dense path are skipped. A lane loads 16
// bytes of a W_d row, a row's SW-column slice takes LPR lanes, so a wave
// sums RPW rows. Workgroup b runs on XCD b mod 8 and the blocks are ordered
// slice phase first, so an XCD gathers from one slice of W_d at a time. The
// wave stages its rows' slot records {neuron, h} in LDS, 64 per row at a
// time, and reads them back as broadcasts; records past a row's count are
// zero (neuron 0, no weight).
template <typename E, int SW, bool GATED, int G>
__device__ __forceinline__ void down_rows(const SliceArgs& a, int64_t blk) {
  constexpr int EPL = 16 / (int)sizeof(E);
  constexpr int LPR = SW / EPL;
  constexpr int RPW = 64 / LPR;
  constexpr int CH = 64;
  static_assert(RPW >= 1 && RPW <= 8 && CH % G == 0, "slice geometry");
  using V = Vec<E, EPL>;
  using R = typename V::raw;
  __shared__ f32x2_t rec[4][RPW][CH];
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
  const bool store = t < a.T && a.bk[t] == 0;
  const int n = store ? a.ell_cnt[t] : 0;
  int nmax = 0;
#pragma unroll
  for (int q = 0; q < RPW; ++q) nmax = max(nmax, __builtin_amdgcn_readlane(n, q * LPR));
  const int col = slice * SW + l * EPL;
  const char* wd = (const char*)a.wd;
  const uint32_t colb = (uint32_t)col * sizeof(E);
  const uint32_t rowb = (uint32_t)a.d * sizeof(E);
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  for (int k0 = 0; k0 < nmax; k0 += CH) {
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int nq = __builtin_amdgcn_readlane(n, q * LPR);
      f32x2_t v = {};
      if (k0 + lane < nq) {
        const int64_t tq = tw + q;
        v[0] = __int_as_float((int)a.ell_idx[tq * a.K + k0 + lane]);
        v[1] = GATED ? a.upart[tq * a.Kp + k0 + lane]
                     : sload(a.ell_a, tq * a.K + k0 + lane, a.store_bf16);
      }
      rec[wave][q][lane] = v;
    }
    // a wave's LDS accesses complete in issue order: no barrier is needed
    // between its own writes and reads
    const int m = min(CH, nmax - k0);
    for (int g0 = 0; g0 < m; g0 += G) {
      f32x2_t md[G];
      R w[G];
#pragma unroll
      for (int k = 0; k < G; ++k) md[k] = rec[wave][r][g0 + k];
#pragma unroll
      for (int k = 0; k < G; ++k)
        w[k] = *(const R*)(wd + ((uint32_t)__float_as_int(md[k][0]) * rowb + colb));
#pragma unroll
      for (int k = 0; k < G; ++k) {
        float f[EPL];
        V::cvt(w[k], f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(md[k][1], f[e], acc[e]);
      }
    }
  }
  if (store) {
    float* yo = a.y + t * a.d + col;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) *(f32x4_t*)(yo + e) = f32x4_t{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
  }
}

template <typename E, int SW, bool GATED, int G>
__global__ __launch_bounds__(256) void down_kernel(SliceArgs a) {
  down_rows<E, SW, GATED, G>(a, blockIdx.x);
}

// The same with the split-K reduce of the dense path's down product into
// its rows of y (rows the down projection skips) in the first nred
// workgroups; nred is a multiple of 8, so that workgroup b of the down
// projection still runs on XCD b mod 8.
template <typename E, int SW, bool GATED, int G>
__global__ __launch_bounds__(256) void down_reduce_kernel(SliceArgs a, GemmArgs g, int nred) {
  if ((int)blockIdx.x < nred) {
    splitk_reduce_rows(g, a.y, a.d, blockIdx.x, nred);
    return;
  }
  down_rows<E, SW, GATED, G>(a, (int64_t)blockIdx.x - nred);
}

// The up and down projections in one kernel, without the d slices: one
// wave per row; a lane holds D / 64 contiguous bf16 of x and accumulates
// the same columns of y in registers. Per active pair (G at a time): the
// W_u row's full dot product with x (wave sum), h = a * u (u stays in
// registers; with 16-bit storage it is rounded as it would be stored),
// then h * W_d row into y. The rows' {neuron, a} records are staged in LDS
// as in the sliced kernels. No per-slice partials, one launch; the weight
// rows come from the whole W_u, W_d on every XCD.
template <int D, bool GATED, int G>
__global__ __launch_bounds__(256) void fused_updown_kernel(SliceArgs a) {
  constexpr int EPL = D / 64;     // bf16 per lane
  constexpr int NL = EPL / 8;     // 16-byte loads per lane and row
  static_assert(NL >= 1, "d >= 512");
  __shared__ f32x2_t rec[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= a.T || a.bk[t]) return;
  const int n = a.ell_cnt[t];
  const uint32_t colb = (uint32_t)lane * EPL * 2;
  const uint32_t rowb = (uint32_t)D * 2;
  const char* wu = (const char*)a.wu;
  const char* wd = (const char*)a.wd;
  u32x4_t xv[NL];
  if (GATED) {
#pragma unroll
    for (int i = 0; i < NL; ++i)
      xv[i] = *(const u32x4_t*)((const char*)a.x + (uint64_t)t * rowb + colb + i * 16);
  }
  float y[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) y[e] = 0.0f;
  for (int c0 = 0; c0 < n; c0 += 64) {
    f32x2_t v = {0.0f, 0.0f};
    if (c0 + lane < n) {
      const int64_t q = t * a.K + c0 + lane;
      v[0] = __int_as_float((int)a.ell_idx[q]);
      v[1] = sload(a.ell_a, q, a.store_bf16);
    }
    rec[wave][lane] = v;
    // a wave's LDS accesses complete in issue order: no barrier is needed
    // between its own writes and reads
    const int m = min(64, n - c0);
    for (int k0 = 0; k0 < m; k0 += G) {
      f32x2_t md[G];
#pragma unroll
      for (int g = 0; g < G; ++g) md[g] = k0 + g < m ? rec[wave][k0 + g] : f32x2_t{0.0f, 0.0f};
      float h[G];
      if (GATED) {
        u32x4_t w[G][NL];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int i = 0; i < NL; ++i)
            w[g][i] = *(const u32x4_t*)(wu + (uint32_t)__float_as_int(md[g][0]) * rowb + colb +
                                        i * 16);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = 0.0f;
#pragma unroll
          for (int i = 0; i < NL; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // the dwords as values first: a bit_cast of a vector element
              // reads the vector's first element
              const uint32_t xe = xv[i][e], we = w[g][i][e];
              acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xe),
                                                    __builtin_bit_cast(bf16x2_t, we), acc, false);
            }
          // octet sums (DPP), then the 8 octets' sums in a fixed order
          const int oc = __float_as_int(octet_sum(acc));
          float u = 0.0f;
#pragma unroll
          for (int o = 0; o < 8; ++o) u += __int_as_float(__builtin_amdgcn_readlane(oc, 8 * o));
          h[g] = md[g][1] * sround(u, a.store_bf16);
        }
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) h[g] = md[g][1];
      }
      u32x4_t w2[G][NL];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < NL; ++i)
          w2[g][i] = *(const u32x4_t*)(wd + (uint32_t)__float_as_int(md[g][0]) * rowb + colb +
                                       i * 16);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[i * 8 + 2 * e] = fmaf(h[g], bf16lo(w2[g][i][e]), y[i * 8 + 2 * e]);
            y[i * 8 + 2 * e + 1] = fmaf(h[g], bf16hi(w2[g][i][e]), y[i * 8 + 2 * e + 1]);
          }
    }
  }
  float* yo = a.y + t * D + lane * EPL;
#pragma unroll
  for (int e = 0; e < EPL; e += 4) *(f32x4_t*)(yo + e) = f32x4_t{y[e], y[e + 1], y[e + 2], y[e + 3]};
}

template <typename E, int NS, int SW>
hipError_t launch_slices(const SliceArgs& a, bool gated, int phase, hipStream_t st) {
  if (phase == 0) {
    hipLaunchKernelGGL((up_partial_kernel<E, NS, SW>), dim3((unsigned)(NS * ((a.T + 3) / 4))),
                       dim3(256), 0, st, a);
  } else if (phase == 2) {
    hipLaunchKernelGGL((hsum_kernel<NS>), dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, st, a);
  } else {
    // 256-column slices (bf16: two rows per wave)
    constexpr int DSW = 256;
    constexpr int DRPW = 64 / (DSW * (int)sizeof(E) / 16);
    const dim3 dgrid((unsigned)((a.d / DSW) * ((a.T + 4 * DRPW - 1) / (4 * DRPW))));
    if (gated) hipLaunchKernelGGL((down_kernel<E, DSW, true, 4>), dgrid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((down_kernel<E, DSW, false, 4>), dgrid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void gather_relu_rows_kernel(const float* __restrict__ z, int F,
                                                               int sb,
                                                               const int32_t* __restrict__ rows,
                                                               const int32_t* __restrict__ n,
                                                               int cap, void* __restrict__ out) {
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
    sstore4(out, (int64_t)m * F + c, v, sb);
  }
}

}  // namespace

hipError_t launch_gather_relu_rows(const float* z, int F, int sb, const int32_t* rows,
                                   const int32_t* n, int cap, void* out, hipStream_t s) {
  hipLaunchKernelGGL(gather_relu_rows_kernel, dim3(512), dim3(256), 0, s, z, F, sb, rows, n, cap,
                     out);
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

template <typename E, int NS, int SW>
hipError_t launch_up_lists_t(const SliceArgs& a, const ListArgs& l0, const ListArgs* l1,
                             int64_t T, hipStream_t st) {
  const ListArgs none = {};
  hipLaunchKernelGGL((up_partial_list_kernel<E, NS, SW>),
                     dim3((unsigned)(8 + NS * ((a.T + 3) / 4))), dim3(256), 0, st, a, l0,
                     l1 ? *l1 : none, l1 ? 2 : 1, T);
  return hipGetLastError();
}

template <typename E, int NS, int SW>
hipError_t launch_up_gather_t(const SliceArgs& a, const GatherT& gt, hipStream_t st) {
  hipLaunchKernelGGL((up_partial_gather_kernel<E, NS, SW>),
                     dim3((unsigned)(2 * kGatherBlocks + NS * ((a.T + 3) / 4))), dim3(256), 0, st,
                     a, gt);
  return hipGetLastError();
}

hipError_t launch_up_with_gather(Dtype dt, const SliceArgs& a, const GatherT& gt, hipStream_t s) {
  int ns, epl;
  slice_shape(dt, a.d, &ns, &epl);
  const int sw = a.d / ns;
  if (dt != kBF16) return hipErrorInvalidValue;
  if (ns == 2 && sw == 256) return launch_up_gather_t<uint16_t, 2, 256>(a, gt, s);
  if (ns == 4 && sw == 256) return launch_up_gather_t<uint16_t, 4, 256>(a, gt, s);
  if (ns == 8 && sw == 256) return launch_up_gather_t<uint16_t, 8, 256>(a, gt, s);
  if (ns == 8 && sw == 512) return launch_up_gather_t<uint16_t, 8, 512>(a, gt, s);
  return hipErrorInvalidValue;
}

hipError_t launch_up_with_lists(Dtype dt, const SliceArgs& a, const ListArgs& l0,
                                const ListArgs* l1, int64_t T, hipStream_t s) {
  int ns, epl;
  slice_shape(dt, a.d, &ns, &epl);
  const int sw = a.d / ns;
  if (dt != kBF16) return hipErrorInvalidValue;
  if (ns == 2 && sw == 256) return launch_up_lists_t<uint16_t, 2, 256>(a, l0, l1, T, s);
  if (ns == 4 && sw == 256) return launch_up_lists_t<uint16_t, 4, 256>(a, l0, l1, T, s);
  if (ns == 8 && sw == 256) return launch_up_lists_t<uint16_t, 8, 256>(a, l0, l1, T, s);
  if (ns == 8 && sw == 512) return launch_up_lists_t<uint16_t, 8, 512>(a, l0, l1, T, s);
  return hipErrorInvalidValue;
}

hipError_t launch_down_with_reduce(Dtype dt, bool gated, const SliceArgs& a, const GemmArgs& g,
                                   hipStream_t s) {
  if (dt != kBF16) return hipErrorInvalidValue;
  constexpr int DSW = 256;
  constexpr int DRPW = 64 / (DSW * 2 / 16);
  if (a.d % DSW != 0) return hipErrorInvalidValue;
  const int nred = 256;
  const dim3 grid((unsigned)(nred + (a.d / DSW) * ((a.T + 4 * DRPW - 1) / (4 * DRPW))));
  if (gated)
    hipLaunchKernelGGL((down_reduce_kernel<uint16_t, DSW, true, 4>), grid, dim3(256), 0, s, a, g, nred);
  else
    hipLaunchKernelGGL((down_reduce_kernel<uint16_t, DSW, false, 4>), grid, dim3(256), 0, s, a, g, nred);
  return hipGetLastError();
}

hipError_t launch_backup_list(const ListArgs& l0, const ListArgs* l1, int64_t T, hipStream_t s) {
  const ListArgs none = {};
  hipLaunchKernelGGL(backup_list_kernel, dim3(l1 ? 2 : 1), dim3(1024), 0, s, l0, l1 ? *l1 : none,
                     T);
  return hipGetLastError();
}

hipError_t launch_fused_updown(bool gated, const SliceArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.T + 3) / 4)), block(256);
#define SFFN_FU(D_)                                                                      \
  if (a.d == D_) {                                                                       \
    if (gated) hipLaunchKernelGGL((fused_updown_kernel<D_, true, 4>), grid, block, 0, s, a); \
    else hipLaunchKernelGGL((fused_updown_kernel<D_, false, 4>), grid, block, 0, s, a);     \
    return hipGetLastError();                                                            \
  }
  SFFN_FU(512)
  SFFN_FU(1024)
  SFFN_FU(2048)
  SFFN_FU(4096)
#undef SFFN_FU
  return hipErrorInvalidValue;
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
