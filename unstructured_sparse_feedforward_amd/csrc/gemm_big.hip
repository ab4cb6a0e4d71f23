// Large-tile bf16 MFMA GEMM for gfx950: the gate GEMM with the fused ReLU +
// TwELL epilogue, the gate pre-activations, and the dense layer's GEMMs.
//
// C[M, N] = A[M, K] * B^T with A row-major (k contiguous) and B either
// [N, K] (k contiguous) or [K, N] (n contiguous, transposed in registers on
// its way into LDS). One workgroup of 4 waves (2 x 2) computes a 256 x 256
// tile (two B operands: 256 x 128 each); a wave owns 128 x 128 (or 128 x 64
// per B operand), i.e. 4 x 4 v_mfma_f32_32x32x16_bf16 blocks whose
// accumulators live in AGPRs. Per 16-wide k substep a wave reads 8 16-byte
// fragments from LDS for 16 MFMAs, half the LDS traffic per MFMA of a 64 x 64
// wave tile. Fragment reads for the next substep are issued before the
// current substep's MFMAs. K is staged 64 at a time through two LDS buffers
// (A + B = 64 KB per stage) with 16-byte chunks XOR-swizzled by row.
//
// Every epilogue works on the accumulator registers directly. In the
// 32 x 32 MFMA layout register q of a block holds, for lanes 0-31 and
// 32-63, 32 consecutive columns of two different rows; a wave's 128
// columns are exactly one 128-column TwELL tile, so the four blocks of a
// register index give two complete tile rows: four ballots, scalar
// popcounts and a lane prefix count place every positive entry in its
// ascending slot (the TwELL of "Sparser, Faster, Lighter Transformer
// Language Models", gist.science explainer, 2. Methodology A, written in
// the gate GEMM's epilogue as in 2. Methodology B).
#include "sffn_internal.hpp"

namespace sffn {
namespace {

constexpr int NT = 256;
constexpr int BM = 256;
constexpr int BK = 64;        // bf16 elements of K per stage (128 bytes per row)
constexpr int ROWB = 128;
constexpr int NXCD = 8;
constexpr int GROUP_M = 4;

// 128-byte LDS rows of 8 16-byte chunks. gfx950's LDS serves 16 lanes of a
// 16-byte read per cycle across 64 banks (256 bytes): two 128-byte rows per
// bank line, so the chunk is XORed with (row >> 1) & 7 and 16 consecutive
// rows at the same logical chunk hit 16 distinct bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ swz(row)) << 4);
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
  static constexpr int STAGE = (BM + NB * BN) * ROWB;
};

template <int NB, bool BT, int EPI>
__global__ __launch_bounds__(NT, 1) void gemm_big_kernel(GemmArgs g) {
  using C_ = Cfg<NB>;
  constexpr int BN = C_::BN;
  constexpr int JB = C_::JB;
  constexpr int STAGE = C_::STAGE;
  __shared__ __align__(16) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1;
  const int wc = wave & 1;

  const int M = g.M;
  const int mt = (M + BM - 1) / BM;
  const int ntl = (g.N + BN - 1) / BN;
  const int nkt = g.K / BK;
  const int ntiles = mt * ntl;

  const int G = gridDim.x;
  const int xcd = blockIdx.x % NXCD;
  const int G8 = G / NXCD;
  const int local = blockIdx.x / NXCD;
  const int per = (ntiles + NXCD - 1) / NXCD;
  const int t_begin = xcd * per;
  const int t_end = min(ntiles, t_begin + per);

  const char* Ab = (const char*)g.A;
  const char* Bb[2] = {(const char*)g.B0, (const char*)g.B1};
  const int64_t lda_b = g.lda * 2;
  const int64_t ldb_b = g.ldb * 2;

  for (int L = t_begin + local; L < t_end; L += G8) {
    const int grp = L / (GROUP_M * ntl);
    const int first_m = grp * GROUP_M;
    const int gsz = min(mt - first_m, GROUP_M);
    const int rr = L - grp * GROUP_M * ntl;
    const int tm = first_m + rr % gsz;
    const int tn = rr / gsz;
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    // ---- global -> LDS. Rows of A and of a k-contiguous B are copied by
    //      direct-to-LDS loads: one instruction moves 8 rows x 128 bytes,
    //      lane L landing at LDS row L/8, physical chunk L%8, so it fetches
    //      logical chunk (L%8) ^ swz(row). Wave w copies rows
    //      [64w, 64w + 64) of A (and of B). Rows past M (N) are clamped to
    //      the last valid one; their results are never stored.
    const int lr = lane >> 3;
    // logical chunk of the lane for LDS row 8*i + lr (rows of a wave's
    // group start at multiples of 64, so only i's parity and lr matter)
    const int lchunk0 = (lane & 7) ^ swz(lr);
    const int lchunk1 = (lane & 7) ^ swz(8 + lr);
    const char* a_src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = min(m0 + wave * 64 + i * 8 + lr, M - 1);
      a_src[i] = Ab + (int64_t)m * lda_b + ((i & 1) ? lchunk1 : lchunk0) * 16;
    }
    constexpr int BPW = BN / 32;   // B rows per wave / 8 (per operand)
    const char* b_src[NB][BPW > 0 ? BPW : 1];
    if constexpr (!BT) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
          const int n = min(n0 + wave * (BN / 4) + i * 8 + lr, g.N - 1);
          b_src[nb][i] = Bb[nb] + (int64_t)n * ldb_b + ((i & 1) ? lchunk1 : lchunk0) * 16;
        }
    }
    // n-contiguous B (single operand, BN = 256): thread (bg, bkg) loads
    // 8 k rows x 8 n through registers and transposes them
    const int bg = tid & 31;
    const int bkg = tid >> 5;
    const bool bt_ok = n0 + 8 * bg < g.N;
    u32x4_t rb[BT ? 8 : 1];

    auto issue_stage = [&](int kt, int st) {
      char* base = smem + st * STAGE;
      const int64_t ka = (int64_t)kt * BK * 2;
      const int64_t kb = (int64_t)kt * BK;
      // register loads of an n-contiguous B go first so that waiting for
      // them does not also wait for the direct-to-LDS copies after them
      if constexpr (BT) {
        const char* p = Bb[0] + (kb + bkg * 8) * ldb_b + (int64_t)(bt_ok ? n0 + 8 * bg : 0) * 2;
#pragma unroll
        for (int q = 0; q < 8; ++q) rb[q] = *(const u32x4_t*)(p + q * ldb_b);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(a_src[i] + ka),
                                         (void*)(base + (wave * 64 + i * 8) * ROWB), 16, 0, 0);
      if constexpr (!BT) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < BPW; ++i)
            __builtin_amdgcn_global_load_lds(
                (const void*)(b_src[nb][i] + kb * 2),
                (void*)(base + (BM + nb * BN + wave * (BN / 4) + i * 8) * ROWB), 16, 0, 0);
      }
    };

    // n-contiguous B: 8 k rows x 8 n columns (bf16) -> 8 n rows x 8 k
    auto store_bt = [&](int st) {
      if constexpr (BT) {
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
      }
    };

    f32x16_t acc[NB][4][JB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[nb][i][j][q] = 0.0f;

    u32x4_t af[2][4];
    u32x4_t bfr[2][NB][JB];
    auto read_frags = [&](int st, int s, int buf) {
      const char* sa = smem + st * STAGE;
      const int ch = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wr * 128 + i * 32 + (lane & 31);
        af[buf][i] = *(const u32x4_t*)(sa + lds_off(row, ch));
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          const int row = wc * C_::WN + j * 32 + (lane & 31);
          bfr[buf][nb][j] = *(const u32x4_t*)(sa + (BM + nb * BN) * ROWB + lds_off(row, ch));
        }
    };
    auto mfmas = [&](int buf) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < JB; ++j)
            acc[nb][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, af[buf][i]), __builtin_bit_cast(bf16x8_t, bfr[buf][nb][j]),
                acc[nb][i][j], 0, 0, 0);
    };

    // Pipeline: stage k+1's copies land while stage k is multiplied. An
    // iteration starts with the last substep of the previous stage (its
    // fragments were read and drained before the barrier), so the next
    // fragment reads always overlap 16 MFMAs and no fragment register is
    // carried across the loop's back edge with a load still in flight.
    // sched_barrier(0) fences keep the compiler from sinking fragment reads
    // next to their use (one wave per SIMD has nothing else to run).
    __syncthreads();  // the previous tile's readers are done with LDS
    issue_stage(0, 0);
    store_bt(0);
    if (nkt > 1) {
      issue_stage(1, 1);
      store_bt(1);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
      const int st = kt & 1;
      read_frags(st, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (kt > 0) mfmas(1);  // substep 3 of stage kt-1
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        read_frags(st, s + 1, (s + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(s & 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // this wave's reads of stage kt are complete; stage kt+1 has landed
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      __syncthreads();
      if (kt + 2 < nkt) {
        issue_stage(kt + 2, st);
        store_bt(st);
      }
    }
    mfmas(1);  // substep 3 of the last stage

    // ---- epilogues straight from the accumulators
    const int h = lane >> 5;     // which of the register's two rows
    const int c32 = lane & 31;   // column inside the 32-column block
    if constexpr (EPI == kEpiTwell) {
      // wave columns [n0 + wc*128, +128) are TwELL tile tb
      const int tb = (n0 >> 7) + wc;
      if (tb * kTile < g.N) {
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rbase = m0 + wr * 128 + i * 32;
          int cnt_lane = 0;  // lane r < 32 collects the count of row rbase + r
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r0 = (q >> 2) * 8 + (q & 3);   // block row of the lane half h = 0
            const int row = rbase + r0 + h * 4;
            const bool rok = row < M;
            float av[4];
            uint64_t bal[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              av[j] = agpr(acc[0][i][j][q]);
              bal[j] = __ballot(rok && av[j] > 0.0f);
            }
            // positives of the two rows before block j, and in total
            int pre0[4], pre1[4];
            int n0c = 0, n1c = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              pre0[j] = n0c;
              pre1[j] = n1c;
              n0c += __popc((uint32_t)bal[j]);
              n1c += __popc((uint32_t)(bal[j] >> 32));
            }
            cnt_lane = lane == r0 ? n0c : (lane == r0 + 4 ? n1c : cnt_lane);
            if (rok) {
              const int64_t slot = ((int64_t)row * g.n_t + tb) * g.C;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                if (av[j] > 0.0f) {
                  const int rank = (h ? pre1[j] - __popc((uint32_t)bal[j]) : pre0[j]) +
                                   __popcll(bal[j] & below);
                  if (rank < g.C) {
                    g.tw_val[slot + rank] = av[j];
                    g.tw_idx[slot + rank] = (uint16_t)(tb * kTile + j * 32 + c32);
                  }
                }
              }
            }
            // one register index at a time: keeps the accumulator reads of
            // later groups from being hoisted
            __builtin_amdgcn_sched_barrier(0);
          }
          if (lane < 32 && rbase + lane < M) g.tw_cnt[(int64_t)(rbase + lane) * g.n_t + tb] = cnt_lane;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = m0 + wr * 128 + i * 32 + (q >> 2) * 8 + h * 4 + (q & 3);
          __builtin_amdgcn_sched_barrier(0);
          if (row >= M) continue;
#pragma unroll
          for (int j = 0; j < JB; ++j) {
            const int col = n0 + wc * C_::WN + j * 32 + c32;
            if (col >= g.N) continue;
            float v;
            if constexpr (NB == 2) {
              const float z = agpr(acc[0][i][j][q]);
              v = (z > 0.0f ? z : 0.0f) * agpr(acc[1][i][j][q]);
            } else {
              v = agpr(acc[0][i][j][q]);
              if (g.act) v = v > 0.0f ? v : 0.0f;
            }
            if constexpr (EPI == kEpiStoreF32) {
              ((float*)g.out)[(int64_t)row * g.ldo + col] = v;
            } else {  // kEpiHiddenBF16
              ((uint16_t*)g.out)[(int64_t)row * g.ldo + col] = (uint16_t)f32_to_bf16(v);
            }
          }
        }
    }
  }
}

template <int NB, bool BT, int EPI>
hipError_t launch_big_t(const GemmArgs& g, hipStream_t s) {
  hipLaunchKernelGGL((gemm_big_kernel<NB, BT, EPI>), dim3(g.grid), dim3(NT), 0, s, g);
  return hipGetLastError();
}

}  // namespace

bool gemm_big_supported(Dtype dt, int nb, bool bt, Epi epi, const GemmArgs& g) {
  if (dt != kBF16 || g.m_dev || g.a_rows || g.out_rows || g.part || g.kwrap || g.k_dev ||
      g.accumulate)
    return false;
  if (g.K % BK != 0) return false;
  if (bt && nb != 1) return false;
  if (epi == kEpiTwell) return nb == 1 && !bt && g.ovf == nullptr;
  if (epi == kEpiStoreF32) return nb == 1;
  if (epi == kEpiHiddenBF16) return !bt;
  return false;
}

// Persistent grid, one workgroup per CU (the 128 KB of LDS allows one):
// measured faster than one tile per workgroup on the 8192 x 5632 x 2048
// gate GEMM (171 vs 196 us for the main loop alone).
int gemm_big_grid(const GemmArgs& g, int nb) {
  (void)nb;
  return (g.num_cu / NXCD) * NXCD;
}

hipError_t launch_gemm_big(int nb, bool bt, Epi epi, const GemmArgs& g, hipStream_t s) {
  if (epi == kEpiTwell) return launch_big_t<1, false, kEpiTwell>(g, s);
  if (epi == kEpiStoreF32) return bt ? launch_big_t<1, true, kEpiStoreF32>(g, s)
                                     : launch_big_t<1, false, kEpiStoreF32>(g, s);
  if (epi == kEpiHiddenBF16) return nb == 2 ? launch_big_t<2, false, kEpiHiddenBF16>(g, s)
                                            : launch_big_t<1, false, kEpiHiddenBF16>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace sffn
