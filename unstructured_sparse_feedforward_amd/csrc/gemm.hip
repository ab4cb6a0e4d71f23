// MFMA GEMM for gfx950 with the epilogues the feedforward layer needs.
//
// C[M, N] = A[M, K] * B^T, A row-major with k contiguous, B either [N, K]
// (k contiguous: W_gate and W_up stored neuron-major) or [K, N] (n
// contiguous: W_down stored neuron-major, used by the down projection).
// bf16 operands use v_mfma_f32_32x32x16_bf16; fp32 operands use the full
// precision v_mfma_f32_32x32x2_f32, so an fp32 layer never rounds to a
// narrower type.
//
// Block tile 128 x 128, 256 threads as 2 x 2 waves of 64 x 64 (2 x 2 MFMA
// 32 x 32 tiles each). Each stage holds 128 bytes of K per row (64 bf16 or
// 32 fp32) for A and every B operand; stages are double-buffered in LDS
// with the next stage prefetched into registers while the current one is
// multiplied. LDS rows are 8 chunks of 16 bytes with the chunk index XORed
// by (row >> 1) & 7, so the 16-byte fragment reads of 16 consecutive rows
// hit distinct banks. A [K, N] operand is transposed in registers on its way
// into LDS, so every fragment read is the same 16-byte k-contiguous load.
//
// The grid is persistent: each workgroup walks a strided list of tiles.
// Consecutive workgroup ids are placed on different XCDs by the hardware,
// so tiles are first split into one contiguous range per XCD and, inside
// it, ordered in groups of 8 M-tiles so that the workgroups running at the
// same time on one XCD share A rows and B columns in its L2.
#include "sffn_internal.hpp"

namespace sffn {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int NT = 256;
constexpr int ROWB = 128;                 // bytes of K per LDS row per stage
constexpr int TILEB = BM * ROWB;          // 16 KB per operand per stage
constexpr int LDC = BN + 4;               // fp32 epilogue tile pitch
constexpr int NXCD = 8;
constexpr int GROUP_M = 8;

template <typename E> struct ET;
template <> struct ET<uint16_t> { static constexpr int EPC = 8; static constexpr int BK = 64; };
template <> struct ET<float> { static constexpr int EPC = 4; static constexpr int BK = 32; };

template <int NB>
constexpr int smem_bytes() {
  constexpr int main_b = 2 * (1 + NB) * TILEB;
  constexpr int epi_b = BM * LDC * 4;
  return main_b > epi_b ? main_b : epi_b;
}

// 128-byte LDS rows of 8 16-byte chunks. gfx950's LDS serves 16 lanes of a
// 16-byte read per cycle across 64 banks (256 bytes): two 128-byte rows per
// bank line, so the chunk is XORed with (row >> 1) & 7 and 16 consecutive
// rows at the same logical chunk hit 16 distinct bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ u32x4_t ld16(const char* p) { return *(const u32x4_t*)p; }
__device__ __forceinline__ u32x2_t ld8(const char* p) { return *(const u32x2_t*)p; }

// Number of K splits for a (possibly device-sized) problem.
// The host keeps split_max <= the number of K stages, so every split owns
// at least one stage.
__device__ __forceinline__ int num_splits(const GemmArgs& g, int mt, int ntl) {
  static_assert(BM == 128 && BN == 128, "splitk_count's tiles");
  return splitk_count(g, mt, ntl);
}

template <typename E>
__device__ __forceinline__ void mfma_step(const u32x4_t& a, const u32x4_t& b, f32x16_t& c);

template <>
__device__ __forceinline__ void mfma_step<uint16_t>(const u32x4_t& a, const u32x4_t& b, f32x16_t& c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                              __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_step<float>(const u32x4_t& a, const u32x4_t& b, f32x16_t& c) {
  // lane half h holds k = 4*(2s+h) .. +3; the four MFMAs each take one of
  // them, A and B agreeing on which k every lane half contributes.
#pragma unroll
  for (int e = 0; e < 4; ++e)
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0, 0, 0);
}

template <typename E, int NB, bool BT, int EPI>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs g) {
  constexpr int BK = ET<E>::BK;
  constexpr int STAGE = (1 + NB) * TILEB;
  __shared__ __align__(16) char smem[smem_bytes<NB>()];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1;
  const int wc = wave & 1;

  const int M = g.m_dev ? device_rows(g.m_dev, g.m_cap) : g.M;
  if (M <= 0) return;
  const int mt = (M + BM - 1) / BM;
  const int ntl = g.N / BN;
  const int Kd = g.k_dev ? g.k_mult * ((device_rows(g.k_dev, g.k_cap) + 63) / 64 * 64) : g.K;
  const int nkt = Kd / BK;
  const int S = (EPI == kEpiStoreF32 || EPI == kEpiHiddenSplitK) ? num_splits(g, mt, ntl) : 1;
  const int ntiles = mt * ntl * S;
  const int Mpad = mt * BM;

  // XCD-contiguous tile ranges
  const int G = gridDim.x;
  const int xcd = blockIdx.x % NXCD;
  const int G8 = G / NXCD;
  const int local = blockIdx.x / NXCD;
  const int per = (ntiles + NXCD - 1) / NXCD;
  const int t_begin = xcd * per;
  const int t_end = min(ntiles, t_begin + per);

  const char* Ab = (const char*)g.A;
  const char* Bb[2] = {(const char*)g.B0, (const char*)g.B1};
  const int64_t lda_b = g.lda * (int64_t)sizeof(E);
  const int64_t ldb_b = g.ldb * (int64_t)sizeof(E);

  for (int L = t_begin + local; L < t_end; L += G8) {
    // decode (split, m-tile, n-tile) with grouped M ordering
    const int ks = L / (mt * ntl);
    const int r = L - ks * mt * ntl;
    const int grp = r / (GROUP_M * ntl);
    const int first_m = grp * GROUP_M;
    const int gsz = min(mt - first_m, GROUP_M);
    const int rr = r - grp * GROUP_M * ntl;
    const int tm = first_m + rr % gsz;
    const int tn = rr / gsz;
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int kt0 = (int)((int64_t)ks * nkt / S);
    const int kt1 = (int)((int64_t)(ks + 1) * nkt / S);

    // ---- per-thread global addresses
    const int lrow = tid >> 3;   // + 32*i
    const int lch = tid & 7;
    const char* a_src[4];
    bool a_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + lrow + 32 * i;
      a_ok[i] = m < M;
      int64_t pr = a_ok[i] ? (g.a_rows ? g.a_rows[m] : m) : 0;
      a_src[i] = Ab + pr * lda_b + lch * 16;
    }
    // B, k-contiguous: rows n0 + lrow + 32 i; B, n-contiguous: see below
    const int bg = tid & 31;     // n group of 4
    const int bkg = tid >> 5;    // k group
    constexpr int RK = ET<E>::EPC;  // k rows per thread when transposing

    u32x4_t ra[4];
    u32x4_t rb[NB][4];
    u32x2_t rbt[NB][8];

    auto load_stage = [&](int kt) {
      const int64_t ka = (int64_t)kt * BK * sizeof(E);
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = a_ok[i] ? ld16(a_src[i] + ka) : u32x4_t{0, 0, 0, 0};
      int64_t kb = (int64_t)kt * BK;
      if (g.kwrap > 0) kb %= g.kwrap;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (!BT) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = n0 + lrow + 32 * i;
            rb[nb][i] = ld16(Bb[nb] + n * ldb_b + kb * sizeof(E) + lch * 16);
          }
        } else {
          // rows k = kb + bkg*RK + q, columns n0 + 4*bg .. +3
          const char* p = Bb[nb] + (kb + bkg * RK) * ldb_b + (int64_t)(n0 + 4 * bg) * sizeof(E);
          if constexpr (sizeof(E) == 2) {
#pragma unroll
            for (int q = 0; q < 8; ++q) rbt[nb][q] = ld8(p + q * ldb_b);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) rb[nb][q] = ld16(p + q * ldb_b);
          }
        }
      }
    };

    auto store_stage = [&](int st) {
      char* base = smem + st * STAGE;
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4_t*)(base + lds_off(lrow + 32 * i, lch)) = ra[i];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        char* bbase = base + (1 + nb) * TILEB;
        if constexpr (!BT) {
#pragma unroll
          for (int i = 0; i < 4; ++i) *(u32x4_t*)(bbase + lds_off(lrow + 32 * i, lch)) = rb[nb][i];
        } else if constexpr (sizeof(E) == 2) {
          // 8 k rows x 4 bf16 columns -> 4 n rows x 8 k
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            u32x4_t o;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const uint32_t r0 = rbt[nb][2 * p][c >> 1];
              const uint32_t r1 = rbt[nb][2 * p + 1][c >> 1];
              o[p] = (c & 1) ? ((r0 >> 16) | (r1 & 0xFFFF0000u)) : ((r0 & 0xFFFFu) | (r1 << 16));
            }
            *(u32x4_t*)(bbase + lds_off(4 * bg + c, bkg)) = o;
          }
        } else {
          // 4 k rows x 4 fp32 columns -> 4 n rows x 4 k
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            u32x4_t o = {rb[nb][0][c], rb[nb][1][c], rb[nb][2][c], rb[nb][3][c]};
            *(u32x4_t*)(bbase + lds_off(4 * bg + c, bkg)) = o;
          }
        }
      }
    };

    f32x16_t acc[NB][2][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[nb][i][j][q] = 0.0f;

    __syncthreads();  // LDS free (previous tile's epilogue done)
    if (kt0 < kt1) {
      load_stage(kt0);
      store_stage(0);
    }
    __syncthreads();

    for (int kt = kt0; kt < kt1; ++kt) {
      const int st = (kt - kt0) & 1;
      const bool more = kt + 1 < kt1;
      if (more) load_stage(kt + 1);
      const char* sa = smem + st * STAGE;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ch = 2 * s + (lane >> 5);
        u32x4_t af[2];
        u32x4_t bfr[NB][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = wr * 64 + i * 32 + (lane & 31);
          af[i] = *(const u32x4_t*)(sa + lds_off(row, ch));
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int row = wc * 64 + j * 32 + (lane & 31);
            bfr[nb][j] = *(const u32x4_t*)(sa + (1 + nb) * TILEB + lds_off(row, ch));
          }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) mfma_step<E>(af[i], bfr[nb][j], acc[nb][i][j]);
      }
      if (more) store_stage(st ^ 1);
      __syncthreads();
    }

    // ---- split-K partials of the hidden GEMM: raw accumulators of every
    //      B operand straight from registers, 32 consecutive floats per
    //      half-wave row
    if constexpr (EPI == kEpiHiddenSplitK) {
      if (S > 1) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int q = 0; q < 16; ++q) {
                const int m = m0 + wr * 64 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
                const int n = n0 + wc * 64 + j * 32 + (lane & 31);
                if (m < M) g.part[((int64_t)(nb * S + ks) * Mpad + m) * g.N + n] = acc[nb][i][j][q];
              }
        continue;
      }
    }

    // ---- saved ReLU(z) and u rows (training backup rows), straight from
    //      the accumulators
    if constexpr (EPI == kEpiHiddenSplitK) {
      if (g.out_a) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int m = m0 + wr * 64 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
              const int n = n0 + wc * 64 + j * 32 + (lane & 31);
              if (m < M) {
                const float zv = acc[0][i][j][q];
                sstore(g.out_a, (int64_t)m * g.ldo_au + n, zv > 0.0f ? zv : 0.0f, g.store_bf16);
                if (NB == 2 && g.out_u)
                  sstore(g.out_u, (int64_t)m * g.ldo_au + n, acc[NB - 1][i][j][q], g.store_bf16);
              }
            }
      }
    }

    // ---- epilogue: accumulators -> fp32 tile in LDS
    float* sC = (float*)smem;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = wr * 64 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
          const int col = wc * 64 + j * 32 + (lane & 31);
          float v;
          if constexpr (NB == 2) {
            const float zv = acc[0][i][j][q];
            v = (zv > 0.0f ? zv : 0.0f) * acc[1][i][j][q];
          } else {
            v = acc[0][i][j][q];
            if (EPI != kEpiTwell && g.act) v = v > 0.0f ? v : 0.0f;
          }
          sC[row * LDC + col] = v;
        }
    __syncthreads();

    uint32_t bits = 0;
    for (int q = 0; q < 32; ++q) {
      const int row = wave * 32 + q;
      const int m = m0 + row;
      if (m >= M) break;
      const f32x2_t v = *(const f32x2_t*)(sC + row * LDC + 2 * lane);
      const int col = n0 + 2 * lane;
      if constexpr (EPI == kEpiTwell) {
        const int64_t slot = ((int64_t)m * g.n_t + tn);
        const int n = twell_pack_row(v[0], v[1], lane, n0, g.C,
                                     (char*)g.tw_val + slot * g.C * (g.store_bf16 ? 2 : 4),
                                     g.tw_idx + slot * g.C, g.tw_cnt + slot, g.store_bf16);
        bits |= (n > g.C ? 1u : 0u) << q;
      } else if constexpr (EPI == kEpiStoreF32) {
        float* dst;
        if (S > 1) {
          dst = g.part + ((int64_t)ks * Mpad + m) * g.N;
        } else {
          const int64_t orow = g.out_rows ? g.out_rows[m] : m;
          dst = (float*)g.out + orow * g.ldo;
        }
        if (g.accumulate && S == 1) {
          *(f32x2_t*)(dst + col) += v;
        } else {
          *(f32x2_t*)(dst + col) = v;
        }
      } else if constexpr (EPI == kEpiHiddenBF16) {
        uint16_t* dst = (uint16_t*)g.out + (int64_t)m * g.ldo;
        *(uint32_t*)(dst + col) = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      } else if (EPI == kEpiHiddenSplitK && sizeof(E) == 4) {
        // fp32 layer: H kept in fp32
        *(f32x2_t*)((float*)g.out + (int64_t)m * g.ldo + col) = v;
      } else {  // bf16 hidden as hi + lo
        uint16_t* dst = (uint16_t*)g.out + (int64_t)m * g.ldo;
        const uint32_t h0 = f32_to_bf16(v[0]);
        const uint32_t h1 = f32_to_bf16(v[1]);
        const uint32_t l0 = f32_to_bf16(v[0] - __uint_as_float(h0 << 16));
        const uint32_t l1 = f32_to_bf16(v[1] - __uint_as_float(h1 << 16));
        *(uint32_t*)(dst + col) = h0 | (h1 << 16);
        *(uint32_t*)(dst + g.lo_off + col) = l0 | (l1 << 16);
      }
    }
    if constexpr (EPI == kEpiTwell) {
      const int word = (m0 + wave * 32) >> 5;
      if (g.ovf && lane == 0 && m0 + wave * 32 < M) g.ovf[(int64_t)tn * g.ovf_words + word] = bits;
    }
  }
}

// Sum the split-K partials of the hidden GEMM (gemm_kernel: z splits then
// u splits, [Mpad, F] each) and apply its epilogue: H = ReLU(z) * u (two B
// operands) or ReLU(z), stored as bf16 hi and lo parts (bf16 layers) or
// float32. A no-op when the GEMM did not split (it has written H itself).
template <typename E, int NB>
__global__ __launch_bounds__(256) void hidden_combine_kernel(GemmArgs g) {
  const int M = device_rows(g.m_dev, g.m_cap);
  if (M <= 0) return;
  const int mt = (M + BM - 1) / BM;
  const int ntl = g.N / BN;
  const int S = num_splits(g, mt, ntl);
  if (S <= 1) return;
  const int Mpad = mt * BM;
  const int Fh = g.N;   // hidden width
  const int n4 = Fh / 4;
  const int64_t total = (int64_t)M * n4;
  const int64_t pstride = (int64_t)Mpad * g.N;  // one split's partials
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(e / n4);
    const int c = (int)(e - (int64_t)m * n4) * 4;
    const float* pz = g.part + (int64_t)m * g.N + c;
    const float* pu = pz + (int64_t)S * pstride;
    // every split's partials are loaded before the first add (in split
    // order, so the sums are deterministic)
    f32x4_t vz[kSplitCap], vu[kSplitCap];
#pragma unroll
    for (int k = 0; k < kSplitCap; ++k) {
      if (k < S) {
        vz[k] = *(const f32x4_t*)(pz + k * pstride);
        if (NB == 2) vu[k] = *(const f32x4_t*)(pu + k * pstride);
      }
    }
    f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f}, u = z;
#pragma unroll
    for (int k = 0; k < kSplitCap; ++k) {
      if (k < S) {
        z += vz[k];
        if (NB == 2) u += vu[k];
      }
    }
    f32x4_t h, a;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = z[q] > 0.0f ? z[q] : 0.0f;
      h[q] = NB == 2 ? a[q] * u[q] : a[q];
    }
    if (g.out_a) {
      sstore4(g.out_a, (int64_t)m * g.ldo_au + c, a, g.store_bf16);
      if (NB == 2 && g.out_u) sstore4(g.out_u, (int64_t)m * g.ldo_au + c, u, g.store_bf16);
    }
    if constexpr (sizeof(E) == 4) {
      *(f32x4_t*)((float*)g.out + (int64_t)m * g.ldo + c) = h;
    } else {
      uint16_t* dst = (uint16_t*)g.out + (int64_t)m * g.ldo;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hi[q] = f32_to_bf16(h[q]);
        lo[q] = f32_to_bf16(h[q] - __uint_as_float(hi[q] << 16));
      }
      *(u32x2_t*)(dst + c) = u32x2_t{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
      *(u32x2_t*)(dst + g.lo_off + c) = u32x2_t{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
    }
  }
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g, float* y, int64_t ldy) {
  splitk_reduce_rows(g, y, ldy, blockIdx.x, gridDim.x);
}

template <typename E, int NB, bool BT, int EPI>
hipError_t launch_t(const GemmArgs& g, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<E, NB, BT, EPI>), dim3(g.grid), dim3(NT), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int gemm_grid(Dtype, int nb, int num_cu) {
  // workgroups resident per CU given the LDS footprint (160 KB per CU)
  const int lds = nb == 2 ? smem_bytes<2>() : smem_bytes<1>();
  int per_cu = (160 * 1024) / lds;
  if (per_cu < 1) per_cu = 1;
  int g = num_cu * per_cu;
  return (g / NXCD) * NXCD;
}

hipError_t launch_gemm(Dtype dt, int nb, bool bt, Epi epi, const GemmArgs& g, hipStream_t s) {
  if (g.num_cu > 0 && gemm_big_supported(dt, nb, bt, epi, g)) {
    GemmArgs b = g;
    b.grid = gemm_big_grid(g, nb);
    return launch_gemm_big(nb, bt, epi, b, s);
  }
#define SFFN_GEMM_CASE(E, NB_, BT_, EPI_) \
  if (nb == NB_ && bt == BT_ && epi == EPI_) return launch_t<E, NB_, BT_, EPI_>(g, s);
  if (dt == kBF16) {
    SFFN_GEMM_CASE(uint16_t, 1, false, kEpiTwell)
    SFFN_GEMM_CASE(uint16_t, 1, false, kEpiStoreF32)
    SFFN_GEMM_CASE(uint16_t, 1, false, kEpiHiddenBF16)
    SFFN_GEMM_CASE(uint16_t, 1, false, kEpiHiddenSplit)
    SFFN_GEMM_CASE(uint16_t, 2, false, kEpiHiddenBF16)
    SFFN_GEMM_CASE(uint16_t, 2, false, kEpiHiddenSplit)
    SFFN_GEMM_CASE(uint16_t, 1, true, kEpiStoreF32)
    SFFN_GEMM_CASE(uint16_t, 1, false, kEpiHiddenSplitK)
    SFFN_GEMM_CASE(uint16_t, 2, false, kEpiHiddenSplitK)
  } else {
    SFFN_GEMM_CASE(float, 1, false, kEpiTwell)
    SFFN_GEMM_CASE(float, 1, false, kEpiStoreF32)
    SFFN_GEMM_CASE(float, 2, false, kEpiStoreF32)
    SFFN_GEMM_CASE(float, 1, true, kEpiStoreF32)
    SFFN_GEMM_CASE(float, 1, false, kEpiHiddenSplitK)
    SFFN_GEMM_CASE(float, 2, false, kEpiHiddenSplitK)
  }
#undef SFFN_GEMM_CASE
  return hipErrorInvalidValue;
}

namespace {

// One thread per 4 columns of a dense-path row. a = ReLU(z) is the tile's
// saved pre-activations when its count exceeds C, else the tile's TwELL
// entries that fall on the 4 columns (at most C ascending ids, read by all
// the tile's threads); u is the sum of the split-K partials in split order.
template <int NB>
__device__ __forceinline__ void flag_hidden_rows(const GemmArgs& g, int64_t blk, int64_t nblk) {
  const int M = device_rows(g.m_dev, g.m_cap);
  if (M <= 0) return;
  const int F = g.N;
  const int mt = (M + BM - 1) / BM;
  const int S = NB == 2 ? num_splits(g, mt, F / BN) : 0;
  const int64_t pstride = (int64_t)mt * BM * F;
  const int f4 = F / 4;
  const int64_t total = (int64_t)M * f4;
  for (int64_t e = blk * blockDim.x + threadIdx.x; e < total; e += nblk * blockDim.x) {
    const int m = (int)(e / f4);
    const int c = (int)(e - (int64_t)m * f4) * 4;
    // the partials depend on the dense-path row only: in flight first
    f32x4_t pv[kSplitCap];
    if (NB == 2) {
      const float* pu = g.part + (int64_t)m * F + c;
#pragma unroll
      for (int k = 0; k < kSplitCap; ++k)
        if (k < S) pv[k] = *(const f32x4_t*)(pu + k * pstride);
    }
    const int64_t t = g.a_rows[m];
    const int b = c / kTile;
    const int cnt = g.tw_cnt[t * g.n_t + b];
    const int sb = g.store_bf16;
    f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
    if (cnt > g.C) {
      // the tile row's saved pre-activations; a record past the capacity
      // was not stored (the call then reports the overflow) and reads as 0
      const int rec = g.ovf_map[t * g.n_t + b];
      if (rec >= 0) {
        a = *(const f32x4_t*)(g.zovf + (int64_t)rec * kTile + (c - b * kTile));
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = sround(a[q] > 0.0f ? a[q] : 0.0f, sb);
      }
    } else {
      const int64_t e0 = (t * g.n_t + b) * g.C;
      for (int k = 0; k < cnt; ++k) {
        const int d = (int)g.tw_idx[e0 + k] - c;
        if (d >= 0 && d < 4) a[d] = sload(g.tw_val, e0 + k, sb);
      }
    }
    // with 16-bit storage a and u are the stored (rounded) values, and
    // H = a u is exact in fp32 (two 8-bit significands)
    f32x4_t u = {0.0f, 0.0f, 0.0f, 0.0f};
    if (NB == 2) {
#pragma unroll
      for (int k = 0; k < kSplitCap; ++k)
        if (k < S) u += pv[k];
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] = sround(u[q], sb);
    }
    f32x4_t h;
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = NB == 2 ? a[q] * u[q] : a[q];
    if (g.out_a) {
      sstore4(g.out_a, (int64_t)m * g.ldo_au + c, a, sb);
      if (NB == 2 && g.out_u) sstore4(g.out_u, (int64_t)m * g.ldo_au + c, u, sb);
    }
    uint16_t* dst = (uint16_t*)g.out + (int64_t)m * g.ldo;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hi[q] = f32_to_bf16(h[q]);
      lo[q] = f32_to_bf16(h[q] - __uint_as_float(hi[q] << 16));
    }
    *(u32x2_t*)(dst + c) = u32x2_t{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
    *(u32x2_t*)(dst + g.lo_off + c) = u32x2_t{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
  }
}

template <int NB>
__global__ __launch_bounds__(256) void flag_hidden_kernel(GemmArgs g) {
  flag_hidden_rows<NB>(g, blockIdx.x, gridDim.x);
}

// The same beside the sparse path's slice sums, in one launch: workgroups
// [0, nflag) combine the dense path's rows, the rest sum the slices. Both
// are short chains of dependent loads, so they overlap each other's
// latency.
template <int NS>
__global__ __launch_bounds__(256) void flag_hidden_hsum_kernel(GemmArgs g, SliceArgs a,
                                                               int nflag) {
  if ((int)blockIdx.x < nflag) flag_hidden_rows<2>(g, blockIdx.x, nflag);
  else hsum_rows<NS>(a, (int64_t)blockIdx.x - nflag);
}

}  // namespace

namespace {
// 64 x 64 tiles through LDS: a thread loads 16 bytes (8 columns) of two
// rows and, after the barrier, stores 16 bytes (8 rows) of two output rows
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in,
                                                             int64_t ldi,
                                                             uint16_t* __restrict__ out,
                                                             int64_t ldo, int64_t R, int64_t C) {
  __shared__ uint16_t tile[64][72];
  const int tid = threadIdx.x;
  const int64_t tc = C / 64;
  const int64_t ntiles = (R / 64) * tc;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t r0 = (t / tc) * 64, c0 = (t % tc) * 64;
    const int cc = (tid & 7) * 8;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int rr = (tid >> 3) + 32 * p;
      const u32x4_t v = *(const u32x4_t*)(in + (r0 + rr) * ldi + c0 + cc);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        tile[rr][cc + 2 * k] = (uint16_t)(v[k] & 0xFFFFu);
        tile[rr][cc + 2 * k + 1] = (uint16_t)(v[k] >> 16);
      }
    }
    __syncthreads();
    const int rr = (tid & 7) * 8;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c = (tid >> 3) + 32 * p;
      u32x4_t v;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[k] = (uint32_t)tile[rr + 2 * k][c] | ((uint32_t)tile[rr + 2 * k + 1][c] << 16);
      *(u32x4_t*)(out + (c0 + c) * ldo + r0 + rr) = v;
    }
    __syncthreads();
  }
}
}  // namespace

namespace {
// 64 x 64 tiles: a thread takes 8 neighbouring neurons of two rows (16-byte
// loads of dH, Z_s, U_s; 16-byte stores of dZ, dU), and after the barrier
// 8 neighbouring rows of two neurons from LDS for the transposed stores
__global__ __launch_bounds__(256) void dense_grad_kernel(const float* __restrict__ dh,
                                                         const uint16_t* __restrict__ zs,
                                                         const uint16_t* __restrict__ us,
                                                         float l1, int64_t T, int64_t F,
                                                         uint16_t* __restrict__ dzu,
                                                         uint16_t* __restrict__ dzt,
                                                         uint16_t* __restrict__ dut) {
  __shared__ uint16_t tz[64][72], tu[64][72];
  const int tid = threadIdx.x;
  const int64_t tc = F / 64;
  const int64_t ntiles = (T / 64) * tc;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t r0 = (t / tc) * 64, c0 = (t % tc) * 64;
    const int cc = (tid & 7) * 8;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int rr = (tid >> 3) + 32 * p;
      const int64_t e = (r0 + rr) * F + c0 + cc;
      const f32x4_t h0 = *(const f32x4_t*)(dh + e);
      const f32x4_t h1 = *(const f32x4_t*)(dh + e + 4);
      const u32x4_t z = *(const u32x4_t*)(zs + e);
      u32x4_t u = {0u, 0u, 0u, 0u};
      if (us) u = *(const u32x4_t*)(us + e);
      uint32_t oz[4], ou[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t bz[2], bu[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int c = 2 * k + q;
          const float hv = c < 4 ? h0[c] : h1[c - 4];
          const float zv = q ? bf16hi(z[k]) : bf16lo(z[k]);
          const bool on = zv > 0.0f;
          float dz, du = 0.0f;
          if (us) {
            const float uv = q ? bf16hi(u[k]) : bf16lo(u[k]);
            dz = on ? hv * uv + l1 : 0.0f;
            du = on ? hv * zv : 0.0f;
          } else {
            dz = on ? hv + l1 : 0.0f;
          }
          bz[q] = f32_to_bf16(dz);
          bu[q] = f32_to_bf16(du);
          tz[rr][cc + c] = (uint16_t)bz[q];
          tu[rr][cc + c] = (uint16_t)bu[q];
        }
        oz[k] = bz[0] | (bz[1] << 16);
        ou[k] = bu[0] | (bu[1] << 16);
      }
      uint16_t* d = dzu + (r0 + rr) * 2 * F + c0 + cc;
      *(u32x4_t*)d = u32x4_t{oz[0], oz[1], oz[2], oz[3]};
      if (us) *(u32x4_t*)(d + F) = u32x4_t{ou[0], ou[1], ou[2], ou[3]};
    }
    __syncthreads();
    const int rr = (tid & 7) * 8;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c = (tid >> 3) + 32 * p;
      u32x4_t vz, vu;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        vz[k] = (uint32_t)tz[rr + 2 * k][c] | ((uint32_t)tz[rr + 2 * k + 1][c] << 16);
        vu[k] = (uint32_t)tu[rr + 2 * k][c] | ((uint32_t)tu[rr + 2 * k + 1][c] << 16);
      }
      *(u32x4_t*)(dzt + (c0 + c) * T + r0 + rr) = vz;
      if (us) *(u32x4_t*)(dut + (c0 + c) * T + r0 + rr) = vu;
    }
    __syncthreads();
  }
}
}  // namespace

hipError_t launch_dense_grad(const float* dh, const uint16_t* zs, const uint16_t* us, float l1,
                             int64_t T, int64_t F, uint16_t* dzu, uint16_t* dzt, uint16_t* dut,
                             hipStream_t s) {
  const int64_t ntiles = (T / 64) * (F / 64);
  const unsigned grid = (unsigned)(ntiles < 4096 ? ntiles : 4096);
  hipLaunchKernelGGL(dense_grad_kernel, dim3(grid), dim3(256), 0, s, dh, zs, us, l1, T, F, dzu,
                     dzt, dut);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t ldi, uint16_t* out, int64_t ldo,
                                 int64_t R, int64_t C, hipStream_t s) {
  const int64_t ntiles = (R / 64) * (C / 64);
  const unsigned grid = (unsigned)(ntiles < 4096 ? ntiles : 4096);
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(grid), dim3(256), 0, s, in, ldi, out, ldo, R, C);
  return hipGetLastError();
}

hipError_t launch_flag_hidden(int nb, const GemmArgs& g, hipStream_t s) {
  // several units per CU in flight: each is a short chain of dependent loads
  const dim3 grid((unsigned)(8 * g.num_cu)), block(256);
  if (nb == 2) hipLaunchKernelGGL(flag_hidden_kernel<2>, grid, block, 0, s, g);
  else hipLaunchKernelGGL(flag_hidden_kernel<1>, grid, block, 0, s, g);
  return hipGetLastError();
}

hipError_t launch_flag_hidden_hsum(Dtype dt, const GemmArgs& g, const SliceArgs& a,
                                   hipStream_t s) {
  int ns, epl;
  slice_shape(dt, a.d, &ns, &epl);
  const int nflag = 8 * g.num_cu;
  const dim3 grid((unsigned)(nflag + (a.T + 3) / 4)), block(256);
  if (ns == 2) hipLaunchKernelGGL(flag_hidden_hsum_kernel<2>, grid, block, 0, s, g, a, nflag);
  else if (ns == 4) hipLaunchKernelGGL(flag_hidden_hsum_kernel<4>, grid, block, 0, s, g, a, nflag);
  else if (ns == 8) hipLaunchKernelGGL(flag_hidden_hsum_kernel<8>, grid, block, 0, s, g, a, nflag);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_hidden_combine(Dtype dt, int nb, const GemmArgs& g, hipStream_t s) {
  const dim3 grid(g.grid), block(256);
  if (dt == kBF16) {
    if (nb == 2) hipLaunchKernelGGL((hidden_combine_kernel<uint16_t, 2>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((hidden_combine_kernel<uint16_t, 1>), grid, block, 0, s, g);
  } else {
    if (nb == 2) hipLaunchKernelGGL((hidden_combine_kernel<float, 2>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((hidden_combine_kernel<float, 1>), grid, block, 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const GemmArgs& g, float* y, int64_t ldy, hipStream_t s) {
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(g.grid), dim3(256), 0, s, g, y, ldy);
  return hipGetLastError();
}

}  // namespace sffn
