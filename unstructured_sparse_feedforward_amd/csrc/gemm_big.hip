// Large-tile bf16 MFMA GEMM for gfx950: the gate GEMM with the fused ReLU +
// TwELL epilogue, the gate pre-activations, and the dense layer's GEMMs.
//
// C[M, N] = A[M, K] * B^T with A row-major (k contiguous) and B either
// [N, K] (k contiguous) or [K, N] (n contiguous, transposed in registers on
// its way into LDS). One workgroup of 4 waves (2 x 2) computes a 256 x 256
// tile (two B operands: 256 x 128 each); a wave owns 128 x 128 (or 128 x 64
// per B operand), i.e. 4 x 4 v_mfma_f32_32x32x16_bf16 blocks whose
// accumulators live in AGPRs. Per 16-wide k substep a wave reads 8 16-byte
// fragments from LDS for 16 MFMAs, and those reads are spread over the
// previous substep's MFMAs.
//
// k-contiguous operands stream through a ring of LDS slots filled by
// direct-to-LDS copies that are spread over the MFMAs as well: 32 k per
// slot (gemm_ring_kernel). The ring runs on across a workgroup's tiles, so
// a tile starts with its first fragments in registers. An n-contiguous B
// goes through registers instead, with two 64-wide stages
// (gemm_bt_kernel).
//
// Every epilogue works on the accumulator registers. For the gate GEMM a
// wave's 128 columns are exactly one 128-column TwELL tile (the TwELL of
// "Sparser, Faster, Lighter Transformer Language Models", gist.science
// explainer, 2. Methodology A, written in the gate GEMM's epilogue as in
// 2. Methodology B): its accumulators go through a 16 KB LDS staging tile
// per wave, 32 rows at a time, and each lane packs half a row from there
// (twell_block_lds), so that the epilogue is mostly straight-line vector
// work with little latency exposed while the matrix cores wait.
#include "sffn_internal.hpp"

namespace sffn {
namespace {

constexpr int NT = 256;
constexpr int BM = 256;
constexpr int NXCD = 8;
constexpr int GROUP_M = 4;

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8); a field at its maximum does not wait.
constexpr int wait_imm(int vm, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}
constexpr int kWaitLgkm0 = wait_imm(63, 0);
constexpr int kWaitAll = wait_imm(0, 0);

// Workgroup barrier that is also a compiler memory barrier, without the
// wait for every outstanding load that a release fence would add: the
// waits each barrier needs (LDS reads done, the right direct-to-LDS copies
// landed) are issued explicitly before it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from base + voff + soff into LDS at lds (+ 16 x lane):
// a buffer load into LDS over a raw resource on the operand (byte offsets
// from it; the whole 32-bit range is in bounds, and every offset the
// kernels form stays inside the operand, since rows are clamped to the last
// valid one). Word 3 is the gfx9 raw-buffer format (32-bit data). The
// resource is the same for every copy of an operand, so it is formed once.
__device__ __forceinline__ void copy16_lds(const void* base, uint32_t voff, uint32_t soff,
                                           char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000),
      (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Read one accumulator element out of its AGPR at the point of use, so the
// epilogue streams through the 256 accumulators instead of copying them
// all to VGPRs at once.
__device__ __forceinline__ float agpr(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

template <int NB>
struct Cfg {
  static constexpr int BN = NB == 2 ? 128 : 256;  // per B operand
  static constexpr int WN = BN / 2;               // wave columns per B operand
  static constexpr int JB = WN / 32;              // MFMA blocks per wave row
};

// Tiles in groups of GROUP_M row tiles (all column tiles of a group before
// the next), and each XCD (workgroups b with b % 8 equal) takes one
// contiguous eighth of that order, so the 32 CUs of an XCD share A row
// panels and B column panels in their L2.
struct TileSched {
  int mt, ntl, t_begin, t_end, local, G8;
  __device__ TileSched(int M, int N, int BN) {
    mt = (M + BM - 1) / BM;
    ntl = (N + BN - 1) / BN;
    const int ntiles = mt * ntl;
    const int xcd = blockIdx.x % NXCD;
    G8 = gridDim.x / NXCD;
    local = blockIdx.x / NXCD;
    const int per = (ntiles + NXCD - 1) / NXCD;
    t_begin = xcd * per;
    t_end = min(ntiles, t_begin + per);
  }
  __device__ void coords(int L, int BN, int& m0, int& n0) const {
    const int grp = L / (GROUP_M * ntl);
    const int first_m = grp * GROUP_M;
    const int gsz = min(mt - first_m, GROUP_M);
    const int rr = L - grp * GROUP_M * ntl;
    m0 = (first_m + rr % gsz) * BM;
    n0 = (rr / gsz) * BN;
  }
};

// 8 fragment reads spread over the first 8 of a substep's 16 MFMAs: a burst
// of LDS reads ahead of the MFMAs would hold the wave's issue slot while
// the matrix core idles.
__device__ __forceinline__ void interleave_reads() {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
}

// A substep's 16 MFMAs carry its 8 fragment reads (one before each of the
// first 8) and half a stage of copies, one before MFMAs 2, 6, 10 and 14, so
// that the L2-to-LDS path (about a quarter of the MFMA rate in bytes per
// clock) drains the copies as they come instead of stalling the wave's
// in-order issue, and with it the matrix core, behind a burst. The copies
// cannot move past reads in program order (the compiler cannot tell that
// they write other LDS slots than the reads read), so the caller emits
// them as r0 r1 r2 c0 r3 r4 r5 r6 c1 r7 c2 c3.
__device__ __forceinline__ void interleave_spread() {
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
  __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

template <int NB>
__device__ __forceinline__ void mfma_substep(f32x16_t (&acc)[NB][4][Cfg<NB>::JB],
                                             const u32x4_t (&af)[4],
                                             const u32x4_t (&bf)[NB][Cfg<NB>::JB]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < Cfg<NB>::JB; ++j)
        acc[nb][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, af[i]), __builtin_bit_cast(bf16x8_t, bf[nb][j]),
            acc[nb][i][j], 0, 0, 0);
}

// ---------------------------------------------------------------- epilogues

// ReLU + TwELL of a wave's 128 x 128 accumulator block (one TwELL tile of
// 128 rows), 32 rows at a time. Lane l takes row l % 32 and its half l / 32
// of the 128 columns:
//  - the positives' masks come from wave ballots of the accumulator
//    registers: one ballot of register q of column block j holds two rows'
//    32 columns, and two lane writes move them to the lanes that own those
//    row halves;
//  - the block's 64 accumulator registers also go to the wave's 16 KB
//    staging tile (row-major), from where each lane reads the values of its
//    row's first C positives, four at a time;
//  - a popcount and one exchange between the lane halves give the row's
//    count and the second half's first slot.
// The staging tile holds row r's float c at r * 128 + 4 * (((c / 4) ^ r) %
// 32) + c % 4 (16-byte chunks XOR-swizzled by row, so that 16-byte reads of
// one chunk index across 16 rows hit 16 distinct bank groups).
__device__ __forceinline__ int stage_off(int r, int c) {
  return r * 128 + ((((c >> 2) ^ r) & 31) << 2) + (c & 3);
}

// v_writelane_b32: lane `lane` of the result is `val`, the others are `old`
extern "C" __device__ uint32_t sffn_writelane(uint32_t val, uint32_t lane, uint32_t old)
    __asm("llvm.amdgcn.writelane.i32");

// x of this lane plus x of the lane 32 away (v_permlane32_swap trades the
// upper half of one copy with the lower half of the other; the sum of the
// two results is the pair's sum whichever way the halves go)
__device__ __forceinline__ int pair_sum(int x) {
  const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (int)p[0] + (int)p[1];
}

template <bool SB>
__device__ __forceinline__ void twell_block_lds(const GemmArgs& g, f32x16_t (&blk)[4], int rbase,
                                                int tb, int lane, float* stage) {
  const int M = g.M;
  if (rbase >= M) return;
  const int h = lane >> 5;
  const int c32 = lane & 31;
  // the previous block's reads of the staging tile are done
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  // register q of block j: row r = 8 (q / 4) + q % 4 + 4 h, column
  // 32 j + c32. Its staging offset splits into a lane part, one of four by
  // q % 4 (the chunk index's low bits are c32 / 4 ^ 4 h ^ q % 4), and a
  // constant (the row, and the chunk's high bits j ^ q / 4), so that only
  // four addresses are live.
  int lb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) lb[k] = 512 * h + ((((c32 >> 2) ^ (4 * h) ^ k)) << 2) + (c32 & 3);
  // w0, w1: this lane's row mask over columns 64 (lane / 32) + 0..31 and
  // + 32..63. The ballot of register q of block j has row ra's columns
  // 32 j + 0..31 in its low word and row ra + 4's in its high word; both go
  // to word j % 2 of the lanes (row) + 32 (j / 2).
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int ra = 8 * (q >> 2) + (q & 3);
    float v[4];
    uint64_t m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = agpr(blk[j][q]);
      stage[lb[q & 3] + ((q >> 2) * 8 + (q & 3)) * 128 + (((j ^ (q >> 2)) & 3) << 5)] = v[j];
    }
    // four ballots before their lane writes, so that no write waits on
    // the compare just before it
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = __builtin_amdgcn_ballot_w64(v[j] > 0.0f);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t ln = ra + 32 * (j >> 1);
      if (j & 1) {
        w1 = sffn_writelane((uint32_t)m[j], ln, w1);
        w1 = sffn_writelane((uint32_t)(m[j] >> 32), ln + 4, w1);
      } else {
        w0 = sffn_writelane((uint32_t)m[j], ln, w0);
        w0 = sffn_writelane((uint32_t)(m[j] >> 32), ln + 4, w0);
      }
    }
    // a few register indices at a time (bounded register pressure)
    if ((q & 1) == 1) __builtin_amdgcn_sched_barrier(0);
  }
  const int rr = lane & 31;        // this lane's row of the block
  const int hh = lane >> 5;        // and its half of the 128 columns
  const bool row_ok = rbase + rr < M;
  const uint64_t mask = row_ok ? ((uint64_t)w1 << 32) | w0 : 0;
  const int n_own = __popcll(mask);
  const int total = pair_sum(n_own);
  const int n_other = total - n_own;
  const int C = g.C;
  const int64_t row = (int64_t)rbase + rr;
  // the staging tile is complete before any lane reads another's values
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  if (hh == 0 && row_ok) g.tw_cnt[row * g.n_t + tb] = total;
  // a tile row past C keeps all its pre-activations in a record of its
  // own (the tile column's counter hands out the column's next record; its
  // number goes to the row's entry of the tile map)
  if (g.zovf != nullptr) {
    const bool ovf = row_ok && total > C;
    int rec = 0;
    if (ovf && hh == 0) rec = atomicAdd(g.ovf_ctr + tb * kCtrStride, 1);
    rec = pair_sum(rec);   // one of the two lanes holds it
    if (ovf) {
      const int id = rec < g.ovf_cap ? tb * g.ovf_cap + rec : -1;
      if (id >= 0) {
        float* zr = g.zovf + (int64_t)id * kTile + 64 * hh;
#pragma unroll
        for (int k16 = 0; k16 < 16; ++k16) {
          const int c = 16 * hh + k16;
          *(f32x4_t*)(zr + 4 * k16) = *(const f32x4_t*)(stage + rr * 128 + (((c ^ rr) & 31) << 2));
        }
      }
      if (hh == 0) g.ovf_map[row * g.n_t + tb] = id;
    }
  }
  // this half's positives in ascending column order, ranks from the first
  // half's count for the second half; four values read from the staging
  // tile per round, then stored
  int rank = hh ? n_other : 0;
  int todo = min(n_own, C - rank);
  const int64_t e0 = (row * g.n_t + tb) * C;
  uint64_t m = mask;
  while (todo > 0) {
    int col[4];
    float val[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = m != 0 ? (int)__builtin_ctzll(m) : 0;
      m &= m - 1;
      col[u] = 64 * hh + k;
      val[u] = stage[stage_off(rr, col[u])];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < todo) {
        if constexpr (SB) ((uint16_t*)g.tw_val)[e0 + rank + u] = (uint16_t)f32_to_bf16(val[u]);
        else ((float*)g.tw_val)[e0 + rank + u] = val[u];
        g.tw_idx[e0 + rank + u] = (uint16_t)(tb * kTile + col[u]);
      }
    }
    rank += 4;
    todo -= 4;
  }
}

template <int I, int NI, bool SB>
struct TwellBlocksLds {
  static __device__ __forceinline__ void run(const GemmArgs& g, f32x16_t (&acc)[NI][4],
                                             int rbase0, int tb, int lane, float* stage) {
    twell_block_lds<SB>(g, acc[I], rbase0 + I * 32, tb, lane, stage);
    TwellBlocksLds<I + 1, NI, SB>::run(g, acc, rbase0, tb, lane, stage);
  }
};
template <int NI, bool SB>
struct TwellBlocksLds<NI, NI, SB> {
  static __device__ __forceinline__ void run(const GemmArgs&, f32x16_t (&)[NI][4], int, int, int,
                                             float*) {}
};

template <int NI>
__device__ __forceinline__ void twell_epilogue_lds(const GemmArgs& g, f32x16_t (&acc)[NI][4],
                                                   int rbase0, int tb, int lane, float* stage) {
  if (tb * kTile >= g.N) return;
  if (g.store_bf16) TwellBlocksLds<0, NI, true>::run(g, acc, rbase0, tb, lane, stage);
  else TwellBlocksLds<0, NI, false>::run(g, acc, rbase0, tb, lane, stage);
}

template <int NB, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& g, f32x16_t (&acc)[NB][4][Cfg<NB>::JB],
                                         int m0, int n0, int wr, int wc, int lane,
                                         float* stage = nullptr) {
  constexpr int JB = Cfg<NB>::JB;
  const int M = g.M;
  const int h = lane >> 5;     // which of the register's two rows
  const int c32 = lane & 31;   // column inside the 32-column block
  if constexpr (EPI == kEpiTwell) {
    // a wave's 128 columns are one TwELL tile
    static_assert(NB == 1, "TwELL epilogue: one B operand");
    twell_epilogue_lds<4>(g, acc[0], m0 + wr * 128, (n0 >> 7) + wc, lane, stage);
    return;
  }
  if constexpr (EPI == kEpiTrainFwd) {
    // register q of block (i, j) holds rows 8 (q / 4) + 4 h + q % 4 of the
    // block's 32, column j * 32 + lane % 32
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        const int col = n0 + wc * Cfg<NB>::WN + j * 32 + c32;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int row0 = m0 + wr * 128 + i * 32 + g4 * 8 + h * 4;
          if (row0 >= M || col >= g.N) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = g4 * 4 + r;
            const int64_t row = row0 + r;
            const int64_t e = row * g.ld_save + col;
            {
              const uint32_t zs = f32_to_bf16(agpr(acc[0][i][j][q]));
              const float zf = __uint_as_float(zs << 16);
              const float a = zf > 0.0f ? zf : 0.0f;
              uint32_t hb;
              if constexpr (NB == 2) {
                const uint32_t us = f32_to_bf16(agpr(acc[1][i][j][q]));
                ((uint16_t*)g.save_u)[e] = (uint16_t)us;
                hb = f32_to_bf16(a * __uint_as_float(us << 16));
              } else {
                hb = f32_to_bf16(a);
              }
              ((uint16_t*)g.save_z)[e] = (uint16_t)zs;
              ((uint16_t*)g.out)[row * g.ldo + col] = (uint16_t)hb;
            }
          }
        }
      }
    return;
  }
  // the whole block tile inside the output: stores without bounds tests
  const bool full = m0 + BM <= M && n0 + 2 * Cfg<NB>::WN <= g.N;
  if (EPI == kEpiStoreF32 && NB == 1 && g.accumulate) {
    // out += acc: a block row's 16 x JB old values are loaded together,
    // then added and stored
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float prev[16][JB];
#pragma unroll
      for (int q = 0; q < 16; ++q)
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          const int row = m0 + wr * 128 + i * 32 + (q >> 2) * 8 + h * 4 + (q & 3);
          const int col = n0 + wc * Cfg<NB>::WN + j * 32 + c32;
          prev[q][j] = (row < M && col < g.N) ? ((const float*)g.out)[(int64_t)row * g.ldo + col] : 0.0f;
        }
      // every sum before the first store: a store issued between two of
      // the loads' uses would make each use wait for all memory operations
#pragma unroll
      for (int q = 0; q < 16; ++q)
#pragma unroll
        for (int j = 0; j < JB; ++j) prev[q][j] += agpr(acc[0][i][j][q]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 16; ++q)
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          const int row = m0 + wr * 128 + i * 32 + (q >> 2) * 8 + h * 4 + (q & 3);
          const int col = n0 + wc * Cfg<NB>::WN + j * 32 + c32;
          if (row < M && col < g.N) ((float*)g.out)[(int64_t)row * g.ldo + col] = prev[q][j];
        }
    }
  } else {
    // a block row's 16 x JB values are read out of the accumulators into
    // registers of their own first, then stored: with one register reused
    // for every value each store would wait for the previous one to leave
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[16][JB];
#pragma unroll
      for (int q = 0; q < 16; ++q)
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          if constexpr (NB == 2) {
            const float z = agpr(acc[0][i][j][q]);
            v[q][j] = (z > 0.0f ? z : 0.0f) * agpr(acc[1][i][j][q]);
          } else {
            const float t = agpr(acc[0][i][j][q]);
            v[q][j] = g.act ? (t > 0.0f ? t : 0.0f) : t;
          }
        }
      auto put = [&](int q, int j, int row, int col) {
        if constexpr (EPI == kEpiStoreF32) {
          ((float*)g.out)[(int64_t)row * g.ldo + col] = v[q][j];
        } else {  // kEpiHiddenBF16
          ((uint16_t*)g.out)[(int64_t)row * g.ldo + col] = (uint16_t)f32_to_bf16(v[q][j]);
        }
      };
      if (full) {
#pragma unroll
        for (int q = 0; q < 16; ++q)
#pragma unroll
          for (int j = 0; j < JB; ++j)
            put(q, j, m0 + wr * 128 + i * 32 + (q >> 2) * 8 + h * 4 + (q & 3),
                n0 + wc * Cfg<NB>::WN + j * 32 + c32);
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = m0 + wr * 128 + i * 32 + (q >> 2) * 8 + h * 4 + (q & 3);
          if (row >= M) continue;
#pragma unroll
          for (int j = 0; j < JB; ++j) {
            const int col = n0 + wc * Cfg<NB>::WN + j * 32 + c32;
            if (col < g.N) put(q, j, row, col);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- ring kernel

constexpr int RBK = 32;    // k per ring stage (64 bytes per LDS row)
constexpr int RROWB = 64;

// 64-byte LDS rows of 4 16-byte chunks, 4 rows per 256-byte bank line: the
// chunk is XORed with (row >> 2) & 3, so the 16 rows that one pass of a
// 16-byte fragment read touches (same logical chunk) fill 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int rswz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int rlds_off(int row, int chunk) {
  return row * RROWB + ((chunk ^ rswz(row)) << 4);
}

template <int NB, int EPI, int NSLOT>
__global__ __launch_bounds__(NT, 1) void gemm_ring_kernel(GemmArgs g) {
  using C_ = Cfg<NB>;
  constexpr int BN = C_::BN;
  constexpr int JB = C_::JB;
  constexpr int SLOT = (BM + NB * BN) * RROWB;
  constexpr int BPW = BN / 64;           // 16-row copies of B per wave and operand
  constexpr int LPS = 4 + NB * BPW;      // direct-to-LDS copies per wave and stage
  static_assert(LPS == 8, "stage = 8 copies per wave");
  static_assert((NSLOT - 1) * LPS <= 63, "vmcnt range");
  // the TwELL epilogue's staging tiles (16 KB per wave) follow the ring
  constexpr int STAGE = EPI == kEpiTwell ? 4 * 32 * 128 * 4 : 0;
  __shared__ __align__(16) char smem[NSLOT * SLOT + STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
  const int wr = wave >> 1;
  const int wc = wave & 1;
  float* const stage = STAGE ? (float*)(smem + NSLOT * SLOT) + wave * 4096 : nullptr;
  const int M = g.M;
  // K may live on the device (as in the n-contiguous kernel below)
  const int Kd = g.k_dev ? g.k_mult * ((device_rows(g.k_dev, g.k_cap) + 63) / 64 * 64) : g.K;
  const int nkt = Kd / RBK;
  if (nkt == 0 && g.accumulate) return;
  const TileSched ts(M, g.N, BN);

  const char* Ab = (const char*)g.A;
  const char* Bb[2] = {(const char*)g.B0, (const char*)g.B1};
  const int64_t lda_b = g.lda * 2;
  const int64_t ldb_b = g.ldb * 2;

  // Direct-to-LDS copy: one instruction moves 16 rows x 64 bytes, lane L
  // landing at row L/4, physical chunk L%4, so it fetches logical chunk
  // (L%4) ^ rswz(row); copies start at multiples of 16 rows, where
  // rswz(row) = (L >> 4) & 3. Rows past M (N) are clamped to the last
  // valid one; their results are never stored.
  const int lr = lane >> 2;
  const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);

  // Per-lane copy sources of tile L, as 32-bit byte offsets from the
  // operand bases: A rows m0 + 64 wave + 16 i + lane/4, B rows (columns of
  // C) n0 + BN/4 wave + 16 i + lane/4. A stage's copies are buffer loads
  // into LDS with these fixed offsets and the stage's k as the scalar
  // offset, so no vector instruction rewrites an address register between
  // two copies (a copy reads its address registers after issue: rewriting
  // them at once, as global loads with 64-bit addresses needed, held up the
  // wave, and with it the matrix cores, on every copy).
  struct Src {
    uint32_t a[4];
    uint32_t b[NB][BPW];
  };
  auto tile_src = [&](int L, Src& t) {
    int m0, n0;
    ts.coords(L, BN, m0, n0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = min(m0 + wave * 64 + i * 16 + lr, M - 1);
      t.a[i] = (uint32_t)((int64_t)m * lda_b + lchunk * 16);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int n = min(n0 + wave * (BN / 4) + i * 16 + lr, g.N - 1);
        t.b[nb][i] = (uint32_t)((int64_t)n * ldb_b + lchunk * 16);
      }
  };
  // a stage's copies go out in two halves of LPS / 2: its A rows, then its
  // B rows
  static_assert(NB * BPW == 4 && 4 + NB * JB == 8, "halves of 4 copies, 8 reads");

  f32x16_t acc[NB][4][JB];
  auto zero_acc = [&]() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[nb][i][j][q] = 0.0f;
  };

  u32x4_t af[2][4];
  u32x4_t bfr[2][NB][JB];
  // fragment i of substep s of the stage in slot `slot`: A blocks 0..3,
  // then the B blocks
  auto read_one = [&](int slot, int s, int buf, int i) {
    const char* sa = smem + slot * SLOT;
    const int ch = 2 * s + (lane >> 5);
    if (i < 4) {
      af[buf][i] = *(const u32x4_t*)(sa + rlds_off(wr * 128 + i * 32 + (lane & 31), ch));
    } else {
      const int nb = (i - 4) / JB, j = (i - 4) % JB;
      bfr[buf][nb][j] = *(const u32x4_t*)(sa + (BM + nb * BN) * RROWB +
                                          rlds_off(wc * C_::WN + j * 32 + (lane & 31), ch));
    }
  };
  // copy i (0..3) of stage kt's A half (its 4 16-row pieces of A) or B half
  // into slot `slot`
  auto copy_one = [&](bool is_b, const Src& t, int kt, int slot, int i) {
    char* base = smem + slot * SLOT;
    const uint32_t kb = (uint32_t)kt * RBK * 2;
    if (!is_b) {
      copy16_lds(Ab, t.a[i], kb, base + (wave * 64 + i * 16) * RROWB);
    } else {
      const int nb = i / BPW, ii = i % BPW;
      copy16_lds(Bb[nb], t.b[nb][ii], kb, base + (BM + nb * BN + wave * (BN / 4) + ii * 16) * RROWB);
    }
  };
  auto read_frags = [&](int slot, int s, int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) read_one(slot, s, buf, i);
  };
  auto issue_half = [&](bool is_b, const Src& t, int kt, int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i) copy_one(is_b, t, kt, slot, i);
  };
  // the fragment reads of substep s from slot rslot and the A (B) half of
  // stage kt's copies into slot cslot, in the order interleave_spread places
  auto frags_copies = [&](int rslot, int s, int buf, bool is_b, const Src& t, int kt, int cslot) {
    read_one(rslot, s, buf, 0);
    read_one(rslot, s, buf, 1);
    read_one(rslot, s, buf, 2);
    copy_one(is_b, t, kt, cslot, 0);
    read_one(rslot, s, buf, 3);
    read_one(rslot, s, buf, 4);
    read_one(rslot, s, buf, 5);
    read_one(rslot, s, buf, 6);
    copy_one(is_b, t, kt, cslot, 1);
    read_one(rslot, s, buf, 7);
    copy_one(is_b, t, kt, cslot, 2);
    copy_one(is_b, t, kt, cslot, 3);
  };

  // One ring stage: substep 0 of stage kt (fragments already in registers)
  // while the B half of stage `pend` (its A half went out one iteration
  // earlier) is copied into slot `pslot`; then, after the barrier, substep 1
  // while the fragments of the stage in slot `next` are read and the A half
  // of stage `issue` is copied into the slot stage kt leaves. With SW set,
  // `cur` is switched to tile Lsw between the two (the B half before it is
  // the old tile's, the A half after it the new tile's).
  //
  // Pipeline. Stage kt lives in slot (slot0 + kt) % NSLOT; NSLOT stages are
  // in flight ahead of the one multiplied. After the barrier of iteration kt
  // (which every wave reaches only once done reading stage kt) the stage
  // NSLOT further on starts into the slot stage kt leaves; its second half
  // follows in the next iteration's first substep, so each substep carries
  // half a stage of copies. Every iteration issues the same number of
  // copies, so "stage kt+1 has landed" is always "at most NSLOT - 2 stages
  // in flight". A substep first waits for its own fragments (read one
  // substep earlier, at most 8 reads in flight, which lgkmcnt can count),
  // then reads the next ones while it multiplies; the second substep of a
  // stage runs after the barrier and reads the first fragments of the
  // next stage.
  Src cur;
  auto ring_step = [&](int slot, int next, int pend, int pslot, int issue, auto sw, int Lsw) {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // fragments of substep 0
    __builtin_amdgcn_sched_barrier(0);
    frags_copies(slot, 1, 1, true, cur, pend, pslot);
    mfma_substep<NB>(acc, af[0], bfr[0]);
    interleave_spread();
    __builtin_amdgcn_sched_barrier(0);
    // stage kt+1 has landed in this wave's copies, and the fragments of
    // substep 1 are in registers; the barrier makes every wave's copies
    // visible and frees stage kt's slot
    __builtin_amdgcn_s_waitcnt(wait_imm((NSLOT - 2) * LPS, 0));
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(sw)::value) tile_src(Lsw, cur);
    frags_copies(next, 0, 0, false, cur, issue, slot);
    mfma_substep<NB>(acc, af[1], bfr[1]);
    interleave_spread();
    __builtin_amdgcn_sched_barrier(0);
  };
  // The ring's first NSLOT stages, the last of them without its B half
  // (the first iteration issues it); then stage 0 has landed once at most
  // NSLOT - 2 stages and a half are in flight.
  auto fill_ring = [&](int last) {
#pragma unroll
    for (int p = 0; p < NSLOT - 1; ++p) {
      issue_half(false, cur, min(p, last), p);
      issue_half(true, cur, min(p, last), p);
    }
    issue_half(false, cur, min(NSLOT - 1, last), NSLOT - 1);
    __builtin_amdgcn_s_waitcnt(wait_imm((NSLOT - 2) * LPS + LPS / 2, 15));
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(0, 0, 0);
  };

  int L = ts.t_begin + ts.local;
  if (L >= ts.t_end) return;

  if (nkt >= NSLOT) {
    // The ring runs on across this workgroup's tiles: the last NSLOT
    // iterations of a tile copy the first stages of the next one, so the
    // next tile's first fragments are in registers before the epilogue
    // and its copies land while the epilogue runs. After the last tile the
    // copies repeat its last stage into slots never read again.
    tile_src(L, cur);
    bool has_next = L + ts.G8 < ts.t_end;
    fill_ring(nkt - 1);
    int slot = 0, pend = NSLOT - 1, pslot = NSLOT - 1;
    auto step = [&](int issue, auto sw, int Lsw) {
      const int next = slot + 1 == NSLOT ? 0 : slot + 1;
      ring_step(slot, next, pend, pslot, issue, sw, Lsw);
      pend = issue;
      pslot = slot;
      slot = next;
    };
    for (;;) {
      zero_acc();
      const int tail = nkt - NSLOT;
      for (int kt = 0; kt < tail; ++kt) step(kt + NSLOT, Flag<false>{}, 0);
      // the tail copies the next tile's first stages (`cur` switches to the
      // next tile inside its first step)
      int kt = tail;
      if (has_next) {
        step(0, Flag<true>{}, L + ts.G8);
        ++kt;
      }
      for (; kt < nkt; ++kt) step(has_next ? kt - tail : nkt - 1, Flag<false>{}, 0);
      int m0, n0;
      ts.coords(L, BN, m0, n0);
      epilogue<NB, EPI>(g, acc, m0, n0, wr, wc, lane, stage);
      if (!has_next) break;
      L += ts.G8;
      has_next = L + ts.G8 < ts.t_end;
    }
    // no direct-to-LDS copy may still be in flight when the wave ends
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    return;
  }

  // K shorter than the ring: each tile fills and drains the ring itself.
  for (; L < ts.t_end; L += ts.G8) {
    int m0, n0;
    ts.coords(L, BN, m0, n0);
    tile_src(L, cur);
    zero_acc();
    if (nkt > 0) {
      __builtin_amdgcn_s_waitcnt(kWaitAll);
      wg_barrier();   // the previous tile's readers are done with LDS
      __builtin_amdgcn_sched_barrier(0);
      fill_ring(nkt - 1);
      int slot = 0, pend = min(NSLOT - 1, nkt - 1), pslot = NSLOT - 1;
      for (int kt = 0; kt < nkt; ++kt) {
        const int next = slot + 1 == NSLOT ? 0 : slot + 1;
        // past the last stage the copies repeat it (stale reads, never used)
        const int issue = min(kt + NSLOT, nkt - 1);
        ring_step(slot, next, pend, pslot, issue, Flag<false>{}, 0);
        pend = issue;
        pslot = slot;
        slot = next;
      }
    }
    epilogue<NB, EPI>(g, acc, m0, n0, wr, wc, lane, stage);
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);
}

// ---------------------------------------------------------------- n-contiguous B

constexpr int BK = 64;        // bf16 elements of K per stage (128 bytes per row)
constexpr int ROWB = 128;

// 128-byte LDS rows of 8 16-byte chunks, two rows per 256-byte bank line:
// the chunk is XORed with (row >> 1) & 7.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ swz(row)) << 4);
}

// B [K, N] n-contiguous (one operand, BN = 256), fp32 output. A arrives by
// direct-to-LDS copies; thread (bg, bkg) loads 8 k rows x 8 n of B into
// registers and transposes them into LDS (holding the registers across a
// stage to hide their latency costs more registers than the kernel has).
template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm_bt_kernel(GemmArgs g) {
  constexpr int NB = 1;
  constexpr int BN = 256;
  constexpr int STAGE = (BM + BN) * ROWB;
  __shared__ __align__(16) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1;
  const int wc = wave & 1;
  const int M = g.M;
  // K may live on the device (rows of a backup list, in blocks of 64,
  // times k_mult for stacked hi/lo parts); a K of 0 leaves an accumulated
  // output as it is and stores zeros otherwise
  const int Kd = g.k_dev ? g.k_mult * ((device_rows(g.k_dev, g.k_cap) + 63) / 64 * 64) : g.K;
  const int nkt = Kd / BK;
  if (nkt == 0 && g.accumulate) return;
  const TileSched ts(M, g.N, BN);

  const char* Ab = (const char*)g.A;
  const char* Bb = (const char*)g.B0;
  const int64_t lda_b = g.lda * 2;
  const int64_t ldb_b = g.ldb * 2;

  for (int L = ts.t_begin + ts.local; L < ts.t_end; L += ts.G8) {
    int m0, n0;
    ts.coords(L, BN, m0, n0);

    // one direct-to-LDS instruction moves 8 rows x 128 bytes, lane L
    // landing at row L/8, physical chunk L%8 (logical (L%8) ^ swz(row))
    const int lr = lane >> 3;
    const int lchunk0 = (lane & 7) ^ swz(lr);
    const int lchunk1 = (lane & 7) ^ swz(8 + lr);
    const char* a_src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = min(m0 + wave * 64 + i * 8 + lr, M - 1);
      a_src[i] = Ab + (int64_t)m * lda_b + ((i & 1) ? lchunk1 : lchunk0) * 16;
    }
    const int bg = tid & 31;
    const int bkg = tid >> 5;
    const bool bt_ok = n0 + 8 * bg < g.N;
    u32x4_t rb[8];

    auto load_b = [&](int kt) {
      const char* p = Bb + ((int64_t)kt * BK + bkg * 8) * ldb_b + (int64_t)(bt_ok ? n0 + 8 * bg : 0) * 2;
#pragma unroll
      for (int q = 0; q < 8; ++q) rb[q] = *(const u32x4_t*)(p + q * ldb_b);
    };
    auto copy_a = [&](int kt, int st) {
      char* base = smem + st * STAGE;
      const int64_t ka = (int64_t)kt * BK * 2;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(a_src[i] + ka),
                                         (void*)(base + (wave * 64 + i * 8) * ROWB), 16, 0, 0);
    };
    // 8 k rows x 8 n columns (bf16) -> 8 n rows x 8 k
    auto store_b = [&](int st) {
      char* bbase = smem + st * STAGE + BM * ROWB;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4_t o;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t r0 = rb[2 * p][c >> 1];
          const uint32_t r1 = rb[2 * p + 1][c >> 1];
          o[p] = (c & 1) ? ((r0 >> 16) | (r1 & 0xFFFF0000u)) : ((r0 & 0xFFFFu) | (r1 << 16));
        }
        *(u32x4_t*)(bbase + lds_off(8 * bg + c, bkg)) = o;
      }
    };

    f32x16_t acc[NB][4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[0][i][j][q] = 0.0f;

    u32x4_t af[2][4];
    u32x4_t bfr[2][1][4];
    auto read_frags = [&](int st, int s, int buf) {
      const char* sa = smem + st * STAGE;
      const int ch = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[buf][i] = *(const u32x4_t*)(sa + lds_off(wr * 128 + i * 32 + (lane & 31), ch));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[buf][0][j] = *(const u32x4_t*)(sa + BM * ROWB + lds_off(wc * 128 + j * 32 + (lane & 31), ch));
    };

    if (nkt > 0) {
      __builtin_amdgcn_s_waitcnt(kWaitAll);
      wg_barrier();   // the previous tile's readers are done with LDS
      __builtin_amdgcn_sched_barrier(0);
      load_b(0);
      copy_a(0, 0);
      store_b(0);
      if (nkt > 1) {
        load_b(1);
        copy_a(1, 1);
        store_b(1);
      }
      __builtin_amdgcn_s_waitcnt(kWaitAll);
      wg_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_frags(0, 0, 0);

      for (int kt = 0; kt < nkt; ++kt) {
        const int st = kt & 1;
        // B of stage kt+2 into registers now (its LDS buffer is still being
        // read); into LDS after the barrier, so the loads have three
        // substeps to arrive
        const bool pre = kt + 2 < nkt;
        if (pre) load_b(kt + 2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // fragments of substep s
          __builtin_amdgcn_sched_barrier(0);
          read_frags(st, s + 1, (s + 1) & 1);
          mfma_substep<NB>(acc, af[s & 1], bfr[s & 1]);
          interleave_reads();
          __builtin_amdgcn_sched_barrier(0);
        }
        // stage kt+1 is in LDS
        __builtin_amdgcn_s_waitcnt(kWaitAll);
        wg_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (pre) {
          copy_a(kt + 2, st);
          store_b(st);
        }
        __builtin_amdgcn_sched_barrier(0);
        read_frags(st ^ 1, 0, 0);
        mfma_substep<NB>(acc, af[1], bfr[1]);
        interleave_reads();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    epilogue<NB, EPI>(g, acc, m0, n0, wr, wc, lane);
  }
}

// 3, 4 and 5 slots time the same on the gate GEMM (the clock, not the
// load latency, sets the pace once the copies are spread over the MFMAs).
constexpr int kSlots = 4;

template <int NB, int EPI>
hipError_t launch_ring(const GemmArgs& g, hipStream_t s) {
  hipLaunchKernelGGL((gemm_ring_kernel<NB, EPI, kSlots>), dim3(g.grid), dim3(NT), 0, s, g);
  return hipGetLastError();
}

// the gate GEMM + TwELL on the ring: three 32 KB slots and 64 KB of
// staging tiles fill the 160 KB of LDS
hipError_t launch_ring_twell(const GemmArgs& g, hipStream_t s) {
  hipLaunchKernelGGL((gemm_ring_kernel<1, kEpiTwell, 3>), dim3(g.grid), dim3(NT), 0, s, g);
  return hipGetLastError();
}

}  // namespace

bool gemm_big_supported(Dtype dt, int nb, bool bt, Epi epi, const GemmArgs& g) {
  if (dt != kBF16 || g.m_dev || g.a_rows || g.out_rows || g.part || g.kwrap) return false;
  // the ring kernel addresses its operands by 32-bit byte offsets
  const int64_t kmax = g.k_dev ? (int64_t)g.k_mult * ((g.k_cap + 63) / 64 * 64) : g.K;
  const int64_t lim = (int64_t)UINT32_MAX;
  if ((int64_t)std::max(g.M, 1) * g.lda * 2 + kmax * 2 > lim ||
      (int64_t)std::max(g.N, 1) * g.ldb * 2 + kmax * 2 > lim)
    return false;
  if (g.accumulate && epi != kEpiStoreF32) return false;
  // a device-sized K: one B operand, float32 output
  if (g.k_dev) return nb == 1 && epi == kEpiStoreF32 && g.k_mult >= 1;
  if (g.K % (bt ? BK : RBK) != 0) return false;
  if (bt) return nb == 1 && epi == kEpiStoreF32;
  if (epi == kEpiTwell) return nb == 1 && g.ovf == nullptr;
  if (epi == kEpiStoreF32) return nb == 1;
  if (epi == kEpiHiddenBF16) return true;
  if (epi == kEpiTrainFwd) return true;
  return false;
}

// Persistent grid, one workgroup per CU (the LDS ring allows one): measured
// faster than one tile per workgroup on the 8192 x 5632 x 2048 gate GEMM.
int gemm_big_grid(const GemmArgs& g, int nb) {
  (void)nb;
  return (g.num_cu / NXCD) * NXCD;
}

hipError_t launch_gemm_big(int nb, bool bt, Epi epi, const GemmArgs& g, hipStream_t s) {
  if (bt) {
    hipLaunchKernelGGL((gemm_bt_kernel<kEpiStoreF32>), dim3(g.grid), dim3(NT), 0, s, g);
    return hipGetLastError();
  }
  if (epi == kEpiTwell) return launch_ring_twell(g, s);
  // float32 output, K on the host or on the device (the backup rows' dW
  // products)
  if (epi == kEpiStoreF32) return launch_ring<1, kEpiStoreF32>(g, s);
  if (epi == kEpiHiddenBF16) return nb == 2 ? launch_ring<2, kEpiHiddenBF16>(g, s)
                                            : launch_ring<1, kEpiHiddenBF16>(g, s);
  if (epi == kEpiTrainFwd) return nb == 2 ? launch_ring<2, kEpiTrainFwd>(g, s)
                                          : launch_ring<1, kEpiTrainFwd>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace sffn
