// bf16 MFMA GEMM for the few rows of the dense path (flagged rows at
// inference, backup rows in training), whose row count lives on the device.
//
// C[M, N] = A[M, K] * B^T. A is row-major (k contiguous); logical row m
// reads row a_rows[m] when a list is given. B is [N, K] (k contiguous,
// copied straight into LDS) or [K, N] (n contiguous, loaded into registers
// and written into LDS transposed). With nsplit > 0 the N columns are two
// operands side by side: columns [0, nsplit) from B0, the rest from B1 (the
// gate and up projections of the same rows); with kcat > 0 they follow
// each other along K (dZ W_g + dU W_u as one product). The k index into B
// wraps at kwrap (the bf16 hi and lo parts of an fp32 operand meet the
// same B), or, with alo > 0, A holds the lo part alo columns after the hi
// part and every B stage is read once for both (twice the MFMAs).
//
// 128 x 128 tiles, 4 waves of 64 x 64 (2 x 2 v_mfma_f32_32x32x16_bf16),
// two workgroups per CU. K streams through a ring of NSLOT LDS slots of
// 32 k each, NSLOT - 1 stages in flight: with only a few hundred rows the
// work is a stream of operand tiles, and the rate at which a CU's copies
// arrive from L2 (about the same with one or two workgroups per CU, or
// with a deeper ring), not the MFMAs, sets the pace. The registers of an
// n-contiguous B stage are held for NSLOT - 1 stages (one register set per
// slot, selected at compile time by unrolling the k loop NSLOT times)
// before they are written into LDS. K may come from the device (backup
// rows). K is split over workgroups (the device chooses the split so that
// there are about split_target tiles); partials go to part[S][Mpad][N] for
// the reduce or combine kernels of gemm.hip, which use the same tiling.
#include "sffn_internal.hpp"

namespace sffn {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int NT = 256;
constexpr int NXCD = 8;
constexpr int BK = 32;       // k per slot (64 bytes per LDS row)
constexpr int ROWB = 64;
constexpr int kGroupRows = 8;   // row tiles per group of the tile order

// Ring geometry: a slot holds an A tile and a B tile (16 KB), or with a
// dual A (hi and lo parts) two A tiles and a B tile (24 KB); four slots,
// or three with a dual A, so that two workgroups fit a CU's LDS. LPS is
// the memory operations per wave and stage: A copies (two, or four with a
// dual A), then two B copies or, for an n-contiguous B, eight B loads.
template <bool DUAL, bool BT> struct Ring {
  static constexpr int SLOT = ((DUAL ? 2 : 1) * BM + BN) * ROWB;
  static constexpr int NSLOT = DUAL ? 3 : 4;
  static constexpr int LPS = (DUAL ? 4 : 2) + (BT ? 8 : 2);
  static_assert((NSLOT - 1) * LPS <= 63, "vmcnt range");
};

constexpr int wait_imm(int vm, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}
constexpr int kWaitLgkm0 = wait_imm(63, 0);
constexpr int kWaitAll = wait_imm(0, 0);

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 64-byte rows of 4 chunks, 4 rows per 256-byte bank line: chunk ^= (row >> 2) & 3
__device__ __forceinline__ int rlds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// number of K splits, as the reduce and combine kernels compute it
__device__ __forceinline__ int small_splits(const GemmArgs& g, int mt, int ntl) {
  if (g.part == nullptr) return 1;
  int s = g.split_target / (mt * ntl);
  if (s > g.split_max) s = g.split_max;
  if (s > kSplitCap) s = kSplitCap;
  return s < 1 ? 1 : s;
}

template <bool BT, int EPI, bool DUAL>
__global__ __launch_bounds__(NT, 2) void gemm_small_kernel(GemmArgs g) {
  constexpr int SLOT = Ring<DUAL, BT>::SLOT;
  constexpr int NSLOT = Ring<DUAL, BT>::NSLOT;
  constexpr int LPS = Ring<DUAL, BT>::LPS;
  __shared__ __align__(16) char smem[NSLOT * SLOT];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1;
  const int wc = wave & 1;

  const int M = g.m_dev ? device_rows(g.m_dev, g.m_cap) : g.M;
  if (M <= 0) return;
  const int mt = (M + BM - 1) / BM;
  const int ntl = g.N / BN;
  // K may live on the device (backup rows, in blocks of 64, times k_mult
  // for stacked hi and lo parts); a K of 0 leaves an accumulated output as
  // it is and stores zeros otherwise
  const int nkt_all =
      (g.k_dev ? g.k_mult * ((device_rows(g.k_dev, g.k_cap) + 63) / 64 * 64) : g.K) / BK;
  if (nkt_all == 0 && g.accumulate) return;
  // partials whenever K is split; the hidden GEMM always leaves them to
  // the combine kernel (ReLU(z) * u needs both operands' tiles)
  const int S = small_splits(g, mt, ntl);
  const bool to_part = EPI == kEpiHiddenSplitK || S > 1;
  const int Mpad = mt * BM;
  const int ntiles = mt * ntl * S;
  const int xcd = blockIdx.x % NXCD;
  const int G8 = gridDim.x / NXCD;
  const int per = (ntiles + NXCD - 1) / NXCD;
  const int t_end = min(ntiles, (xcd + 1) * per);

  const int64_t lda_b = g.lda * 2;
  const int64_t ldb_b = g.ldb * 2;
  // direct-to-LDS copy lane layout: 16 rows x 64 bytes per instruction
  const int lr = lane >> 2;
  const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);
  // n-contiguous B: lane l of wave w loads k rows 8 w .. 8 w + 7 of
  // columns 2 l and 2 l + 1 (4 bytes each: a wave reads 256 contiguous
  // bytes of a k row per load) and writes them as 16 bytes of each
  // column's LDS row (16 lanes of a store touch 8 distinct 16-byte bank
  // groups: at most two-way conflicts)

  for (int L = xcd * per + blockIdx.x / NXCD; L < t_end; L += G8) {
    // the splits of a tile are consecutive, then up to 8 row tiles of one
    // column block (they share B in L2), then the group's next column
    // block (the group's A rows stay in L2 while the columns stream past)
    const int ks = L % S;
    const int rem = L / S;
    const int grp = rem / (kGroupRows * ntl);
    const int gm0 = grp * kGroupRows;
    const int gcount = min(kGroupRows, mt - gm0);
    const int r2 = rem - grp * kGroupRows * ntl;
    const int tn = r2 / gcount;
    const int tm = gm0 + (r2 - tn * gcount);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int kt0 = (int)((int64_t)ks * nkt_all / S);
    const int nkt = (int)((int64_t)(ks + 1) * nkt_all / S) - kt0;
    const char* Bb = (const char*)g.B0;
    int nb0 = n0;
    if (g.nsplit > 0 && n0 >= g.nsplit) {
      Bb = (const char*)g.B1;
      nb0 = n0 - g.nsplit;
    }

    const char* a_src[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = min(m0 + wave * 32 + i * 16 + lr, M - 1);
      const int64_t pr = g.a_rows ? g.a_rows[m] : m;
      a_src[i] = (const char*)g.A + pr * lda_b + lchunk * 16;
    }
    const char* b_src[2];
    if constexpr (!BT) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        b_src[i] = Bb + (int64_t)(nb0 + wave * 32 + i * 16 + lr) * ldb_b + lchunk * 16;
    }
    uint32_t rbs[NSLOT][8];   // n-contiguous B stages in flight

    auto kb_of = [&](int kt) {
      int64_t kb = (int64_t)(kt0 + kt) * BK;
      if (g.kcat > 0 && kb >= g.kcat) kb -= g.kcat;
      if (g.kwrap > 0) kb %= g.kwrap;
      return kb;
    };
    // stage kt (relative to the split) into slot `slot` (B registers into set `set`)
    auto issue = [&](int kt, int slot, uint32_t (&rb)[8]) {
      char* base = smem + slot * SLOT;
      // A column of the stage: with a dual A the hi part of the second
      // operand (k >= kcat) starts alo after the first's
      int64_t kac = (int64_t)(kt0 + kt) * BK;
      if (DUAL && g.kcat > 0 && kac >= g.kcat) kac += g.alo;
      const int64_t ka = kac * 2;
      const int64_t kb = kb_of(kt);
      if constexpr (BT) {
        const char* bs =
            g.kcat > 0 && (int64_t)(kt0 + kt) * BK >= g.kcat ? (const char*)g.B1 : Bb;
        const char* p = bs + (kb + 8 * wave) * ldb_b + (int64_t)(nb0 + 2 * lane) * 2;
        // issued as opaque loads: the compiler's own wait insertion loses
        // count of these across the unrolled loop's back edge and drains
        // every load in flight; the explicit waits below cover them
#pragma unroll
        for (int r = 0; r < 8; ++r)
          asm volatile("global_load_dword %0, %1, off" : "=v"(rb[r]) : "v"(p + r * ldb_b));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(a_src[i] + ka),
                                         (void*)(base + (wave * 32 + i * 16) * ROWB), 16, 0, 0);
      if constexpr (DUAL) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          __builtin_amdgcn_global_load_lds((const void*)(a_src[i] + ka + g.alo * 2),
                                           (void*)(base + (BM + BN + wave * 32 + i * 16) * ROWB),
                                           16, 0, 0);
      }
      if constexpr (!BT) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          __builtin_amdgcn_global_load_lds((const void*)(b_src[i] + kb * 2),
                                           (void*)(base + (BM + wave * 32 + i * 16) * ROWB), 16,
                                           0, 0);
      }
    };
    // 8 k rows x columns (2 l, 2 l + 1) -> chunk w of LDS rows 2 l, 2 l + 1
    auto store_b = [&](int slot, const uint32_t (&rb)[8]) {
      if constexpr (BT) {
        char* bbase = smem + slot * SLOT + BM * ROWB;
        u32x4_t lo, hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          lo[q] = (rb[2 * q] & 0xFFFFu) | (rb[2 * q + 1] << 16);
          hi[q] = (rb[2 * q] >> 16) | (rb[2 * q + 1] & 0xFFFF0000u);
        }
        *(u32x4_t*)(bbase + rlds_off(2 * lane, wave)) = lo;
        *(u32x4_t*)(bbase + rlds_off(2 * lane + 1, wave)) = hi;
      }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    u32x4_t af[2][2], bf[2][2], al[2][DUAL ? 2 : 1];
    auto read_frags = [&](int slot, int s, int buf) {
      const char* sa = smem + slot * SLOT;
      const int ch = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[buf][i] = *(const u32x4_t*)(sa + rlds_off(wr * 64 + i * 32 + (lane & 31), ch));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[buf][j] = *(const u32x4_t*)(sa + BM * ROWB + rlds_off(wc * 64 + j * 32 + (lane & 31), ch));
      if constexpr (DUAL) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          al[buf][i] = *(const u32x4_t*)(sa + (BM + BN) * ROWB +
                                         rlds_off(wr * 64 + i * 32 + (lane & 31), ch));
      }
    };
    auto mfmas = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, af[buf][i]), __builtin_bit_cast(bf16x8_t, bf[buf][j]),
              acc[i][j], 0, 0, 0);
      if constexpr (DUAL) {
        // the lo part meets the same B fragments
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, al[buf][i]), __builtin_bit_cast(bf16x8_t, bf[buf][j]),
                acc[i][j], 0, 0, 0);
      }
    };
    auto spread = [&]() {
#pragma unroll
      for (int k = 0; k < (DUAL ? 6 : 4); ++k) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
      if constexpr (DUAL) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    };

    // Pipeline: stage kt lives in slot kt % NSLOT; every slot is filled up
    // front (stages past the last one repeat it into slots that are never
    // read), after the barrier of iteration kt stage kt + NSLOT is issued
    // into the slot stage kt leaves, and "stage kt+1 has landed" is "at
    // most NSLOT - 2 stages of copies in flight". n-contiguous B: stage
    // kt + 1's registers are written into its slot just before the barrier
    // of iteration kt.
    if (nkt > 0) {
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    wg_barrier();   // the previous tile's readers are done with LDS
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < NSLOT; ++p) issue(min(p, nkt - 1), p, rbs[p]);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(wait_imm((NSLOT - 1) * LPS, 15));   // stage 0 landed
    __builtin_amdgcn_sched_barrier(0);
    store_b(0, rbs[0]);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(0, 0, 0);

    // one stage: kt's second half-step and kt+1's first, with stage kt+1
    // landed, written (n-contiguous B) and made visible in between
    auto stage = [&](int kt, int u) __attribute__((always_inline)) {
      const int nu = (u + 1) % NSLOT;   // slot (and register set) of stage kt + 1
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_sched_barrier(0);
      read_frags(u, 1, 1);
      mfmas(0);
      spread();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(wait_imm((NSLOT - 2) * LPS, 0));  // stage kt+1 landed
      __builtin_amdgcn_sched_barrier(0);
      store_b(nu, rbs[nu]);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      wg_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_frags(nu, 0, 0);
      issue(min(kt + NSLOT, nkt - 1), u, rbs[u]);
      mfmas(1);
      spread();
      __builtin_amdgcn_sched_barrier(0);
    };
    // whole groups of NSLOT stages (the slot and register set of a stage
    // are compile-time constants after unrolling), then the last few
    // stages outside the loop: no exit from inside the unrolled group
    int kb0 = 0;
    for (; kb0 + NSLOT <= nkt; kb0 += NSLOT) {
#pragma unroll
      for (int u = 0; u < NSLOT; ++u) stage(kb0 + u, u);
    }
#pragma unroll
    for (int u = 0; u < NSLOT - 1; ++u) {
      if (kb0 + u >= nkt) break;
      stage(kb0 + u, u);
    }
    if constexpr (BT) {
      // the repeats past the last stage were loaded into registers too:
      // they land before any of those registers is given to another value
      __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
#pragma unroll
      for (int u = 0; u < NSLOT; ++u)
#pragma unroll
        for (int r = 0; r < 8; ++r) asm volatile("" ::"v"(rbs[u][r]));
    }
    }

    // ---- epilogue
    const int h = lane >> 5;
    const int c32 = lane & 31;
    if (to_part) {
      float* pbase = g.part + ((int64_t)ks * Mpad + m0 + wr * 64 + h * 4) * g.N + n0 + wc * 64 + c32;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (m0 + wr * 64 + i * 32 >= M) continue;   // a block of padding rows
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = m0 + wr * 64 + i * 32 + (q >> 2) * 8 + h * 4 + (q & 3);
          if (m >= M) continue;
          float* dst = pbase + (int64_t)(i * 32 + (q >> 2) * 8 + (q & 3)) * g.N;
#pragma unroll
          for (int j = 0; j < 2; ++j) dst[j * 32] = acc[i][j][q];
        }
      }
    } else if (g.accumulate) {
      // out += C: the tile row block's old values are loaded together first
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float prev[16][2];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = m0 + wr * 64 + i * 32 + (q >> 2) * 8 + h * 4 + (q & 3);
          const int64_t orow = m < M ? (g.out_rows ? g.out_rows[m] : m) : 0;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            prev[q][j] = m < M ? ((const float*)g.out)[orow * g.ldo + n0 + wc * 64 + j * 32 + c32] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = m0 + wr * 64 + i * 32 + (q >> 2) * 8 + h * 4 + (q & 3);
          if (m < M) {
            const int64_t orow = g.out_rows ? g.out_rows[m] : m;
            float* dst = (float*)g.out + orow * g.ldo + n0 + wc * 64 + c32;
#pragma unroll
            for (int j = 0; j < 2; ++j) dst[j * 32] = prev[q][j] + acc[i][j][q];
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = m0 + wr * 64 + i * 32 + (q >> 2) * 8 + h * 4 + (q & 3);
          if (m < M) {
            const int64_t orow = g.out_rows ? g.out_rows[m] : m;
            float* dst = (float*)g.out + orow * g.ldo + n0 + wc * 64 + c32;
#pragma unroll
            for (int j = 0; j < 2; ++j) dst[j * 32] = acc[i][j][q];
          }
        }
    }
  }
}

}  // namespace

bool gemm_small_supported(const GemmArgs& g, bool bt, Epi epi) {
  if (epi != kEpiStoreF32 && epi != kEpiHiddenSplitK) return false;
  if (g.N % BN != 0) return false;
  // a device-sized K: one plain product per tile (no split, no second operand)
  if (g.k_dev)
    return bt && epi == kEpiStoreF32 && g.part == nullptr && g.k_mult >= 1 && g.kcat == 0 &&
           g.alo == 0 && g.kwrap == 0 && g.nsplit == 0;
  if (g.K % BK != 0 || g.K < BK) return false;
  if (g.kwrap > 0 && g.kwrap % BK != 0) return false;
  if (g.kcat > 0 && (!bt || g.nsplit > 0 || g.kcat % BK != 0 || g.B1 == nullptr)) return false;
  if (g.alo > 0 && (!bt || epi != kEpiStoreF32 || g.kwrap > 0 || g.nsplit > 0)) return false;
  if (g.nsplit > 0 && (g.nsplit % BN != 0 || bt)) return false;
  if (epi == kEpiHiddenSplitK && (g.part == nullptr || g.act != 1)) return false;
  return true;
}

// two workgroups per CU (64 or 72 KB of LDS each)
int gemm_small_grid(int num_cu) { return (2 * num_cu / NXCD) * NXCD; }

hipError_t launch_gemm_small(bool bt, Epi epi, const GemmArgs& g, hipStream_t s) {
  if (!gemm_small_supported(g, bt, epi) || g.grid < NXCD || g.grid % NXCD != 0)
    return hipErrorInvalidValue;
  const dim3 grid(g.grid), block(NT);
  if (epi == kEpiHiddenSplitK) {
    hipLaunchKernelGGL((gemm_small_kernel<false, kEpiHiddenSplitK, false>), grid, block, 0, s, g);
  } else if (bt && g.alo > 0) {
    hipLaunchKernelGGL((gemm_small_kernel<true, kEpiStoreF32, true>), grid, block, 0, s, g);
  } else if (bt) {
    hipLaunchKernelGGL((gemm_small_kernel<true, kEpiStoreF32, false>), grid, block, 0, s, g);
  } else {
    hipLaunchKernelGGL((gemm_small_kernel<false, kEpiStoreF32, false>), grid, block, 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace sffn
