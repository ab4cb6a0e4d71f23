// Internal declarations shared by the library's translation units:
// vector types, wave-level helpers, the TwELL row packer and the launcher
// entry points that the C ABI (api.hip) calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace sffn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kTile = 128;  // TwELL tile width W
constexpr int kSplitCap = 16;  // most K splits of a split-K GEMM
constexpr int kCtrStride = 32; // int32 words between two device counters (one per 128-byte line)

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------- stored activations

// Stored activation values (TwELL values, ELL a and u, backup rows' a and
// u) are float32, or bf16 bits when the layer stores 16-bit activations
// (sb != 0): then a value is rounded once, to nearest even, where it is
// stored, and the layer computes with the stored value.
__device__ __forceinline__ float sround(float v, int sb) {
  return sb ? __uint_as_float(f32_to_bf16(v) << 16) : v;
}
__device__ __forceinline__ float sload(const void* p, int64_t i, int sb) {
  return sb ? bf16lo(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}
__device__ __forceinline__ void sstore(void* p, int64_t i, float v, int sb) {
  if (sb) ((uint16_t*)p)[i] = (uint16_t)f32_to_bf16(v);
  else ((float*)p)[i] = v;
}
// four consecutive values (16-byte aligned fp32 / 8-byte aligned bf16)
__device__ __forceinline__ void sstore4(void* p, int64_t i, f32x4_t v, int sb) {
  if (sb) {
    *(u32x2_t*)((uint16_t*)p + i) = u32x2_t{f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16),
                                            f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16)};
  } else {
    *(f32x4_t*)((float*)p + i) = v;
  }
}
// two consecutive values (8-byte aligned fp32 / 4-byte aligned bf16)
__device__ __forceinline__ f32x2_t sload2(const void* p, int64_t i, int sb) {
  if (sb) {
    const uint32_t v = *(const uint32_t*)((const uint16_t*)p + i);
    return f32x2_t{bf16lo(v), bf16hi(v)};
  }
  return *(const f32x2_t*)((const float*)p + i);
}

// ---------------------------------------------------------------- wave ops

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// ---------------------------------------------------------------- gathers

// Raw 8- or 16-byte loads of bf16 or fp32 elements and their conversion.
template <typename E, int EPL> struct Vec;
template <> struct Vec<uint16_t, 4> {
  typedef u32x2_t raw;
  __device__ static void cvt(const raw& v, float* o) {
    o[0] = bf16lo(v[0]); o[1] = bf16hi(v[0]); o[2] = bf16lo(v[1]); o[3] = bf16hi(v[1]);
  }
};
template <> struct Vec<uint16_t, 8> {
  typedef u32x4_t raw;
  __device__ static void cvt(const raw& v, float* o) {
#pragma unroll
    for (int k = 0; k < 4; ++k) { o[2 * k] = bf16lo(v[k]); o[2 * k + 1] = bf16hi(v[k]); }
  }
};
template <> struct Vec<float, 4> {
  typedef u32x4_t raw;
  __device__ static void cvt(const raw& v, float* o) {
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = __uint_as_float(v[k]);
  }
};

// ---------------------------------------------------------------- TwELL row

// Pack one (row, tile) of 128 pre-activations held as two per lane
// (columns 2*lane and 2*lane+1 of the tile) into TwELL: the positive
// entries in ascending column order go to slots 0..C-1 (slots past the
// count are left as they are; values stored as sstore with sb) and the
// uncapped count is returned to every lane. Wave-uniform control flow; one
// wave per call.
__device__ __forceinline__ int twell_pack_row(float z0, float z1, int lane, int col0, int C,
                                              void* __restrict__ val, uint16_t* __restrict__ idx,
                                              int32_t* __restrict__ cnt_out, int sb) {
  const bool p0 = z0 > 0.0f;
  const bool p1 = z1 > 0.0f;
  const uint64_t b0 = __ballot(p0);
  const uint64_t b1 = __ballot(p1);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int r0 = __popcll(b0 & below) + __popcll(b1 & below);
  const int r1 = r0 + (p0 ? 1 : 0);
  const int n = __popcll(b0) + __popcll(b1);
  if (p0 && r0 < C) { sstore(val, r0, z0, sb); idx[r0] = (uint16_t)(col0 + 2 * lane); }
  if (p1 && r1 < C) { sstore(val, r1, z1, sb); idx[r1] = (uint16_t)(col0 + 2 * lane + 1); }
  if (lane == 0) *cnt_out = n;
  return n;
}

// ---------------------------------------------------------------- launchers

enum Dtype { kF32 = 0, kBF16 = 1 };

// Epilogues of the MFMA GEMM.
enum Epi {
  kEpiTwell = 0,   // ReLU + TwELL pack + overflow bits (gate GEMM)
  kEpiStoreF32,    // C (or split-K partial) stored as float32, optional row scatter
  kEpiHiddenBF16,  // H = act(C) rounded to bf16 (dense baseline hidden)
  kEpiHiddenSplit, // H = act(C) stored as bf16 hi and lo parts (flagged rows)
  kEpiHiddenSplitK,// as kEpiHiddenSplit (fp32 H for fp32 layers), or split-K
                   // partials of every B operand when the device-sized
                   // problem splits K (then a combine kernel finishes it)
  kEpiTrainFwd,    // dense bf16 training forward (z | u GEMM): Z_s = bf16(z),
                   // U_s = bf16(u) to save_z / save_u, H = bf16(ReLU(Z_s) U_s)
                   // to out
};

struct GemmArgs {
  // A: [M, K] row-major (k contiguous); logical row m reads physical row
  // a_rows[m] when a_rows is set. M comes from *m_dev when set.
  const void* A;
  int64_t lda;
  const int32_t* a_rows;
  int M;
  const int32_t* m_dev;
  int m_cap;                 // > 0: a device M is capped at m_cap
  // B: [N, K] (k contiguous) or, when b_trans, [K, N] (n contiguous).
  // With two B operands (gate and up) both share A. With kcat > 0 (small
  // GEMM, n-contiguous B) the two operands follow each other along K
  // instead: k < kcat reads B0, k >= kcat reads B1 at k - kcat. The k index
  // into B is then taken modulo kwrap when kwrap > 0.
  const void* B0;
  const void* B1;
  int64_t ldb;
  int N;
  int K;
  int kwrap;
  int kcat;
  // dual A (small GEMM, n-contiguous B): A's lo part sits alo columns after
  // its hi part (for k >= kcat the hi part itself starts alo later) and
  // C = A_hi B + A_lo B over the K columns of B
  int64_t alo;
  // K from the device (when k_dev is set): K = k_mult * round_up(min(*k_dev,
  // k_cap), 64); operands must hold zeros in their padding
  const int32_t* k_dev;
  int k_cap;
  int k_mult;
  // output
  void* out;
  int64_t ldo;
  const int32_t* out_rows;   // scatter of stored rows (kEpiStoreF32)
  int accumulate;            // kEpiStoreF32 / split-K reduce: out += result
  int act;                   // 1: ReLU on the single-B result; dual B is always ReLU(z)*u
  int lo_off;                // column offset of the lo part (kEpiHiddenSplit)
  void* out_a;               // kEpiHiddenSplitK: ReLU(z) rows, stored values [M, ldo_au]
  void* out_u;               // kEpiHiddenSplitK: u rows, stored values [M, ldo_au] (nullable)
  int store_bf16;            // stored activation values are bf16 (TwELL values, out_a/out_u)
  int64_t ldo_au;
  // split-K (kEpiStoreF32 with a device M): the number of splits S is
  // chosen on the device so that tiles * S stays near split_target; when
  // S > 1 the partials go to part[S][Mpad][N] and a reduce kernel adds them.
  int split_target;
  int split_max;
  float* part;
  // TwELL (kEpiTwell)
  void* tw_val;
  uint16_t* tw_idx;
  int32_t* tw_cnt;
  uint32_t* ovf;             // [n_t][ovf_words] overflow bits, bit r of word w = row 32w+r
  float* zovf;               // bf16 gate: fp32 pre-activations of the tile rows whose
                             // count exceeds C, one 128-float record per such tile row:
                             // tile column b owns records [b * ovf_cap, (b + 1) * ovf_cap)
                             // [n_t * ovf_cap, 128], taken in order from its counter
                             // ovf_ctr[b * kCtrStride]; the record of row t, tile b is
                             // ovf_map[t * n_t + b] (-1: past the capacity, not stored;
                             // written only for the overflowing tile rows)
  int32_t* ovf_map;
  int32_t* ovf_ctr;
  int ovf_cap;
  int C;
  int n_t;
  int ovf_words;
  // dense bf16 training forward (kEpiTrainFwd)
  void* save_z;              // bf16 [M, ld_save]
  void* save_u;              // bf16 [M, ld_save] (gated; nullptr otherwise)
  int64_t ld_save;
  int nsplit;                // > 0: columns [0, nsplit) from B0, the rest from B1
                             // (gemm_small.hip, k-contiguous B)
  int grid;                  // persistent grid size (small-tile kernel)
  int num_cu;                // compute units (large-tile kernel's grid)
};

// Runs the large-tile bf16 kernel (gemm_big.hip) when it supports the
// problem (host-sized M, no row gather/scatter, no split-K), else the
// small-tile kernel.
hipError_t launch_gemm(Dtype dt, int nb, bool b_trans, Epi epi, const GemmArgs& g,
                       hipStream_t s);
bool gemm_big_supported(Dtype dt, int nb, bool bt, Epi epi, const GemmArgs& g);
// bf16 GEMM of the dense path's few, device-counted rows (gemm_small.hip):
// kEpiStoreF32 (split-K partials for launch_splitk_reduce when split, else
// stored with out_rows / accumulate) or kEpiHiddenSplitK (always partials,
// finished by launch_flag_hidden).
bool gemm_small_supported(const GemmArgs& g, bool bt, Epi epi);
int gemm_small_grid(int num_cu);
hipError_t launch_gemm_small(bool bt, Epi epi, const GemmArgs& g, hipStream_t s);
int gemm_big_grid(const GemmArgs& g, int nb);
hipError_t launch_gemm_big(int nb, bool bt, Epi epi, const GemmArgs& g, hipStream_t s);
int gemm_grid(Dtype dt, int nb, int num_cu);

// split-K reduce: y[rows[m]][n] = sum_s part[s][m][n] for m < *m_dev.
hipError_t launch_splitk_reduce(const GemmArgs& g, float* y, int64_t ldy, hipStream_t s);
// split-K combine of the hidden GEMM (kEpiHiddenSplitK): sums the partials
// and writes H; a no-op when the GEMM did not split.
hipError_t launch_hidden_combine(Dtype dt, int nb, const GemmArgs& g, hipStream_t s);
// Hidden rows of the dense path from the gate GEMM's own outputs (bf16):
// for row m (physical row a_rows[m]) a = ReLU(z) from its TwELL tiles
// (tw_*, C, n_t; tiles with a count above C from zovf), u from the split-K
// partials of x W_u (gated, as gemm_small's kEpiHiddenSplitK leaves them),
// H = a u (or a) stored as bf16 hi | lo into out; a and u rows into
// out_a / out_u when set.
hipError_t launch_flag_hidden(int nb, const GemmArgs& g, hipStream_t s);
struct SliceArgs;
// bf16 gated layers: launch_flag_hidden (two B operands) and the sparse
// path's slice sums (launch_updown phase 2) in one launch
hipError_t launch_flag_hidden_hsum(Dtype dt, const GemmArgs& g, const SliceArgs& a,
                                   hipStream_t s);

hipError_t launch_pack(const float* z, int64_t T, int F, int C, int sb, void* val, uint16_t* idx,
                       int32_t* cnt, uint32_t* ovf, int ovf_words, hipStream_t s);
// The dense bf16 training backward's elementwise step: from dH [T, F]
// fp32 and the saved Z_s, U_s [T, F] bf16 (U_s nullptr when non-gated),
// M = 1[Z_s > 0], dZ = bf16(dH U_s M + l1 M) (non-gated dH M + l1 M) and
// dU = bf16(dH ReLU(Z_s)): rows into dzu [T, 2F] (dZ | dU) and transposed
// into dzt, dut [F, T]. T and F multiples of 64.
hipError_t launch_dense_grad(const float* dh, const uint16_t* zs, const uint16_t* us, float l1,
                             int64_t T, int64_t F, uint16_t* dzu, uint16_t* dzt, uint16_t* dut,
                             hipStream_t s);
// bf16 transpose: out[c * ldo + r] = in[r * ldi + c] for r < R, c < C
// (R, C multiples of 64; ldi, ldo multiples of 8)
hipError_t launch_transpose_bf16(const uint16_t* in, int64_t ldi, uint16_t* out, int64_t ldo,
                                 int64_t R, int64_t C, hipStream_t s);
// zero `bytes` (a multiple of 4) at p (4-byte aligned) with a kernel on s:
// a stream that a caller captures into a HIP graph then records a kernel
// node, not a memset node
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
// over the rows t < T with row_flag[t] == 0: out[0] += the sum of their
// n_t tile counts, out[1] += their number (the caller zeroes out first)
hipError_t launch_count_sum(const int32_t* cnt, const uint8_t* row_flag, int64_t T, int n_t,
                            unsigned long long* out, hipStream_t s);
hipError_t launch_flags(const uint32_t* ovf, int n_t, int ovf_words, int64_t T, uint8_t* row_flag,
                        int32_t* flagged, int32_t* n_flagged, hipStream_t s);
// TwELL -> ELL rows + dense-backup routing (one wave per token row).
struct EllArgs {
  const void* val;        // TwELL [T, n_t, C] stored values
  const uint16_t* idx;
  const int32_t* cnt;     // [T, n_t]
  int64_t T;
  int n_t;
  int C;
  int K;                  // ELL capacity
  void* ell_a;            // [T, K] out, stored values
  int store_bf16;
  uint16_t* ell_idx;      // [T, K] out
  int32_t* ell_cnt;       // [T] out (0 for backup rows)
  uint8_t* row_flag;      // [T] out, TwELL overflow (nullable)
  uint8_t* bk;            // [T] out, 1 = dense backup row
};
hipError_t launch_rows(const EllArgs& a, hipStream_t s);
// Ascending list of the rows with bk[t] != 0 (the first cap of them), their
// true count and (nullable) every row's backup slot (-1 for ELL rows).
// One workgroup per list (two lists, l1 non-null, in one launch); bk must
// be 16-byte aligned. When the count exceeds cap and status is set,
// *status gets bit 0; when reset is set, reset[i * kCtrStride] is zeroed
// for i < n_reset at the end (the gate epilogue's overflow-record
// counters, consumed by then).
struct ListArgs {
  const uint8_t* bk;
  int32_t* brow;
  int64_t cap;
  int32_t* n;
  int32_t* slot;
  int32_t* status;
  int32_t* reset;
  int n_reset;
};
hipError_t launch_backup_list(const ListArgs& l0, const ListArgs* l1, int64_t T, hipStream_t s);

// The number of rows of a GEMM whose M lives on the device.
__device__ __forceinline__ int device_rows(const int32_t* m_dev, int m_cap) {
  const int m = *m_dev;
  return (m_cap > 0 && m > m_cap) ? m_cap : m;
}

// Number of K splits of a split-K GEMM over 128 x 128 tiles (mt x ntl of
// them), as the GEMMs of gemm.hip and gemm_small.hip choose it. The host
// keeps split_max <= the number of K stages, so every split owns at least
// one stage.
__device__ __forceinline__ int splitk_count(const GemmArgs& g, int mt, int ntl) {
  if (g.part == nullptr) return 1;
  int s = g.split_target / (mt * ntl);
  if (s > g.split_max) s = g.split_max;
  if (s > kSplitCap) s = kSplitCap;
  return s < 1 ? 1 : s;
}

// y[out_rows[m], :] (+)= sum of the S split-K partials of row m, in split
// order (deterministic); workgroup blk of nblk, grid-stride over 4 columns
// per thread. Nothing to do with a single split (the GEMM stored y).
__device__ __forceinline__ void splitk_reduce_rows(const GemmArgs& g, float* y, int64_t ldy,
                                                   int64_t blk, int64_t nblk) {
  const int M = device_rows(g.m_dev, g.m_cap);
  if (M <= 0) return;
  const int mt = (M + 127) / 128;
  const int ntl = g.N / 128;
  const int S = splitk_count(g, mt, ntl);
  if (S <= 1) return;
  const int Mpad = mt * 128;
  const int n4 = g.N / 4;
  const int64_t total = (int64_t)M * n4;
  const int64_t pstride = (int64_t)Mpad * g.N;
  for (int64_t e = blk * blockDim.x + threadIdx.x; e < total; e += nblk * blockDim.x) {
    const int m = (int)(e / n4);
    const int c = (int)(e - (int64_t)m * n4) * 4;
    const float* p = g.part + (int64_t)m * g.N + c;
    float* dst = y + (int64_t)(g.out_rows ? g.out_rows[m] : m) * ldy + c;
    f32x4_t v[kSplitCap];
#pragma unroll
    for (int k = 0; k < kSplitCap; ++k)
      if (k < S) v[k] = *(const f32x4_t*)(p + k * pstride);
    f32x4_t acc = v[0];
#pragma unroll
    for (int k = 1; k < kSplitCap; ++k)
      if (k < S) acc += v[k];
    if (g.accumulate) acc += *(const f32x4_t*)dst;
    *(f32x4_t*)dst = acc;
  }
}

// rows[m] for m < min(*n, cap): out[m, :] = ReLU(z[rows[m], :]) (stored
// values, F wide)
hipError_t launch_gather_relu_rows(const float* z, int F, int sb, const int32_t* rows, const int32_t* n,
                                   int cap, void* out, hipStream_t s);

// Sparse up/down over ELL rows, d cut into NS slices (one per XCD group).
struct SliceArgs {
  const void* x;          // [T, d]
  const void* wu;         // [F, d] (gated)
  const void* wd;         // [F, d]
  const uint16_t* ell_idx;
  const void* ell_a;      // stored values
  const int32_t* ell_cnt;
  const uint8_t* bk;      // rows written by the dense path are skipped
  int64_t T;
  int d;
  int K;                  // ELL row stride
  int Kp;                 // partial-dot row stride (K rounded up to 8)
  float* upart;           // [NS, T, Kp] per-slice partial dot products
  void* ell_u;            // [T, K] u per slot, stored values (nullable)
  int store_bf16;
  float* y;               // [T, d]
};
void slice_shape(Dtype dt, int d, int* ns, int* epl);

// Between the sparse up and down phases (gated): u_k = sum of the slice
// partials in slice order and h_k = a_k * u_k, written over slice 0's
// partial (the lane that reads a slot's partials is the one that writes
// it); u_k is saved for training. With 16-bit storage a_k is the stored
// value and u_k is rounded as it would be stored, so that h is what the
// backward recomputes. One wave per row, four rows per workgroup blk.
template <int NS>
__device__ __forceinline__ void hsum_rows(const SliceArgs& a, int64_t blk) {
  const int lane = threadIdx.x & 63;
  const int64_t t = blk * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int n = a.ell_cnt[t];
  for (int k = lane; k < n; k += 64) {
    float u = 0.0f;
#pragma unroll
    for (int r = 0; r < NS; ++r) u += a.upart[((int64_t)r * a.T + t) * a.Kp + k];
    const int64_t q = t * a.K + k;
    u = sround(u, a.store_bf16);
    if (a.ell_u) sstore(a.ell_u, q, u, a.store_bf16);
    a.upart[t * a.Kp + k] = sload(a.ell_a, q, a.store_bf16) * u;
  }
}
// phase 0: per-slice partial dot products (gated layers only);
// phase 2: their sums u and h = a * u (gated; h over slice 0's partials);
// phase 1: down projection into y.
hipError_t launch_updown(Dtype dt, bool gated, int phase, const SliceArgs& a, hipStream_t s);
// bf16 gated layers: phase 0 with the row lists of launch_backup_list built
// beside it in the same launch (l1 nullable)
hipError_t launch_up_with_lists(Dtype dt, const SliceArgs& a, const ListArgs& l0,
                                const ListArgs* l1, int64_t T, hipStream_t s);
// The backup rows of x and dy (bf16), transposed for the backward's dW
// GEMMs: column c of dst0 (dst1) holds src0[brow[r]][c] (src1) at k = r and
// k = Rp + r for r < R = min(*n, cap), Rp = R rounded up to 64, zeros up
// to 2 Rp (both operands of those GEMMs k-contiguous, the bf16 hi and lo
// parts of the other operand meeting the same rows).
struct GatherT {
  const uint16_t* src0;
  const uint16_t* src1;
  int d;
  const int32_t* brow;
  const int32_t* n;
  int cap;
  uint16_t* dst0;
  uint16_t* dst1;
  int64_t ldt;
};
constexpr int kGatherBlocks = 512;   // workgroups per operand

// Workgroup bx of nbx of operand by: 64 rows x 64 columns at a time through
// LDS, 16-byte loads along the rows, 16-byte stores along the columns.
__device__ __forceinline__ void gather_stack_t_tiles(const GatherT& a, int bx, int nbx, int by) {
  const int d = a.d;
  const int64_t ldt = a.ldt;
  const int32_t* __restrict__ brow = a.brow;
  __shared__ __align__(16) uint16_t tile[64][72];   // [column][row]
  // by: x (0) or dy (1)
  const uint16_t* src = by ? a.src1 : a.src0;
  uint16_t* dst = by ? a.dst1 : a.dst0;
  const int R = device_rows(a.n, a.cap);
  const int Rp = (R + 63) / 64 * 64;
  const int tid = threadIdx.x;
  const int nct = d / 64;
  const int ntiles = (Rp / 64) * nct;
  for (int t = bx; t < ntiles; t += nbx) {
    const int r0 = (t / nct) * 64;
    const int c0 = (t - (t / nct) * nct) * 64;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int e = p * 256 + tid;     // 64 rows x 8 chunks of 8 columns
      const int rl = e >> 3;
      const int ch = e & 7;
      u32x4_t v = {0, 0, 0, 0};
      if (r0 + rl < R) v = *(const u32x4_t*)(src + (int64_t)brow[r0 + rl] * d + c0 + ch * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        tile[ch * 8 + 2 * q][rl] = (uint16_t)(v[q] & 0xFFFFu);
        tile[ch * 8 + 2 * q + 1][rl] = (uint16_t)(v[q] >> 16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int e = p * 256 + tid;     // 64 columns x 8 chunks of 8 rows
      const int cl = e >> 3;
      const int ch = e & 7;
      const u32x4_t v = *(const u32x4_t*)&tile[cl][ch * 8];
      uint16_t* o = dst + (int64_t)(c0 + cl) * ldt + r0 + ch * 8;
      *(u32x4_t*)o = v;
      *(u32x4_t*)(o + Rp) = v;
    }
    __syncthreads();
  }
}

// bf16 layers: phase 0 (the backward's dh, with x := dy and W_u := W_d)
// with the backup rows' gather of gather_stack_t_tiles in the same launch
hipError_t launch_up_with_gather(Dtype dt, const SliceArgs& a, const GatherT& gt, hipStream_t s);

// bf16 layers: phase 1 with the split-K reduce of the dense path's down
// product (launch_splitk_reduce(g, a.y, a.d)) in the same launch
hipError_t launch_down_with_reduce(Dtype dt, bool gated, const SliceArgs& a, const GemmArgs& g,
                                   hipStream_t s);
// bf16 layers, d in {512, 1024, 2048, 4096}: the up and down projections of
// the ELL rows in one kernel without d slices (rows with bk set skipped)
hipError_t launch_fused_updown(bool gated, const SliceArgs& a, hipStream_t s);

// Sparse backward over a Hybrid (backward.hip).
struct BwdArgs {
  const void* x;          // [T, d]
  const void* dy;         // [T, d]
  const void* wg;         // [F, d]
  const void* wu;         // [F, d] (gated)
  const void* ell_a;      // [T, K] stored values
  const void* ell_u;      // [T, K] (gated)
  int store_bf16;
  const uint16_t* ell_idx;
  const int32_t* ell_cnt;
  const int32_t* slot;    // [T] backup slot or -1
  int64_t T;
  int d;
  int F;
  int K;
  int Kp;
  float l1;
  const float* dpart;     // [NS, T, Kp] partial dy . W_d[j]
  f32x4_t* drec;          // [T, K] {neuron, dZ, dU, h} per ELL slot
  float* dx;              // [T, d]
  float* dwg;             // [F, d]
  float* dwu;             // [F, d] (gated)
  float* dwd;             // [F, d]
  int accumulate;         // dW of the ELL slots adds to what dW holds
  int32_t* ncnt;          // [4 F4] per-neuron slot counts (F4 = ceil(F / 4))
  int32_t* noff;          // [F + 1]
  uint32_t* thist;        // [nblk, F4] per block of slot units: neuron counts, bytes
  int32_t* toff;          // [nblk, 4 F4] per block: each neuron's slots in earlier blocks
  f32x4_t* meta;          // [T*K] {row, dZ, dU, h} grouped by neuron, ascending rows
  // backup rows
  const int32_t* brow;
  const int32_t* n_backup;
  int cap;                // rows of the backup buffers
  const void* bk_a;       // [cap, F] stored values
  const void* bk_u;       // [cap, F]
  const float* dH;        // [cap, F]
  void* xb;               // stacked gathered x rows
  void* dyb;              // stacked gathered dy rows
  void* gz_rm;            // dZ rows for dx (bf16 hi|lo or fp32), row stride ld_rm
  void* gu_rm;            // dU rows, the same layout
  int64_t ld_rm;
  void* gz_t;             // neuron-major dZ for dW ([F, ldt])
  void* gu_t;
  void* gh_t;
  int64_t ldt;
};
// which = 0: dZ/dU per slot and dx of the ELL rows (2: dZ/dU only, 3: dx
// only); 1: dW of every neuron
hipError_t launch_bwd_sparse(Dtype dt, bool gated, int which, const BwdArgs& a, hipStream_t s);
hipError_t launch_transpose(const BwdArgs& a, hipStream_t s);
// blocks of slot units of the transpose's counting sort (sizes thist, toff)
int64_t transpose_blocks(int64_t T, int K);
hipError_t launch_backup_prep(Dtype dt, bool gated, const BwdArgs& a, hipStream_t s);
hipError_t launch_backup_grad(Dtype dt, bool gated, const BwdArgs& a, hipStream_t s);
// the gather of launch_backup_prep (bf16) as launch_up_with_gather takes it
GatherT gather_args(const BwdArgs& a);
// bf16: which = 3 of launch_bwd_sparse with the split-K reduce of the backup
// rows' dx product (launch_splitk_reduce(g, a.dx, a.d)) in the same launch
hipError_t launch_dx_with_reduce(Dtype dt, bool gated, const BwdArgs& a, const GemmArgs& g,
                                 hipStream_t s);

}  // namespace sffn
