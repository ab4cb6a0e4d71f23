// C ABI of the sparse feedforward library: argument validation, workspace
// layout and the order of kernel launches for each call. See include/sffn.h
// for the contract of every entry point.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "sffn.h"
#include "sffn_internal.hpp"

struct sffn_prof_rec {
  int k;
  hipEvent_t a, b;
};

struct sffn_handle {
  sffn_desc desc;
  int device;
  int num_cu;
  int n_t;
  std::string err;
  // per-kernel event timing
  bool prof = false;
  std::vector<hipEvent_t> pool;
  std::vector<sffn_prof_rec> recs;
  double tot_ms[SFFN_K_COUNT] = {};
  int32_t launches[SFFN_K_COUNT] = {};
  // the backward's second stream (created on first use): the neuron-major
  // grouping runs beside the backup rows' dW products, which leave CUs free
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  // device state: word 0 the capacity-overflow status (read and cleared by
  // sffn_check); from byte kCtrOffset the gate epilogue's overflow-record
  // counters, one per TwELL tile column, kCtrStride words apart (zeroed by
  // the list kernel that follows the gate GEMM; dirty when a call stopped
  // in between, then zeroed before the next gate GEMM)
  int32_t* dstate = nullptr;
  bool ctr_dirty = false;
  // this device's copy of the static scratch (sffn_forward_noalloc)
  void* scratch = nullptr;
  std::string scratch_err;
};

// Workspace of sffn_forward_noalloc, for callers that cannot allocate:
// a file-scope device array, one copy per GPU, held until the process
// ends. Host code never passes the array's name to a kernel or a copy:
// its device address comes from hipGetSymbolAddress, looked up once per
// device (with that device current) when the first handle is created
// there, and kept below.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr size_t kCtrOffset = 256;
constexpr size_t kStateBytes = kCtrOffset + (size_t)512 * sffn::kCtrStride * 4;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's scratch address (device `dev` must be current)
hipError_t scratch_address(int dev, void** out) {
  *out = nullptr;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

namespace {

using namespace sffn;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

sffn_status fail(sffn_handle* h, sffn_status st, const std::string& msg) {
  if (h) h->err = msg;
  return st;
}

sffn_status hip_fail(sffn_handle* h, hipError_t e, const char* where) {
  return fail(h, SFFN_E_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

sffn_status validate_desc(const sffn_desc* d) {
  if (!d) return SFFN_E_ARG;
  if (d->dtype != SFFN_F32 && d->dtype != SFFN_BF16) return SFFN_E_ARG;
  if (d->gated != 0 && d->gated != 1) return SFFN_E_ARG;
  if (d->d <= 0 || d->d_ff <= 0 || d->tile <= 0 || d->twell_cap <= 0 || d->ell_cap < 0 ||
      d->dense_rows < 0)
    return SFFN_E_ARG;
  if (d->store_dtype != SFFN_F32 && d->store_dtype != SFFN_BF16) return SFFN_E_ARG;
  if (!(d->dense_above >= 0.0f)) return SFFN_E_ARG;
  if (d->updown != 0 && d->updown != 1) return SFFN_E_ARG;
  // the one-kernel up/down serves bf16 layers
  if (d->updown == 1 && d->dtype != SFFN_BF16) return SFFN_E_UNSUPPORTED;
  // 16-bit stored activations serve bf16 layers
  if (d->store_dtype == SFFN_BF16 && d->dtype != SFFN_BF16) return SFFN_E_UNSUPPORTED;
  if (d->tile != kTile) return SFFN_E_UNSUPPORTED;
  if (d->d_ff % kTile != 0 || d->d_ff > 65408) return SFFN_E_UNSUPPORTED;
  if (d->twell_cap > kTile) return SFFN_E_UNSUPPORTED;
  const int ch = d->dtype == SFFN_BF16 ? 512 : 256;
  if (d->d % ch != 0 || d->d / ch > 8) return SFFN_E_UNSUPPORTED;
  const int nch = d->d / ch;
  if (nch != 1 && nch != 2 && nch != 4 && nch != 8) return SFFN_E_UNSUPPORTED;
  return SFFN_OK;
}

Dtype dt_of(const sffn_handle* h) { return h->desc.dtype == SFFN_BF16 ? kBF16 : kF32; }
size_t esize(const sffn_handle* h) { return h->desc.dtype == SFFN_BF16 ? 2 : 4; }
// stored activation values: bf16 bits or float32
int sb_of(const sffn_handle* h) { return h->desc.store_dtype == SFFN_BF16 ? 1 : 0; }
size_t ssize(const sffn_handle* h) { return h->desc.store_dtype == SFFN_BF16 ? 2 : 4; }
int ovf_words(int64_t T) { return (int)((T + 31) / 32); }
constexpr int kSplitMax = kSplitCap;

// R: the dense path's row capacity of a call over T rows
int64_t dense_cap(const sffn_handle* h, int64_t T) {
  return h->desc.dense_rows > 0 ? std::min<int64_t>(h->desc.dense_rows, T) : T;
}

// K: the ELL capacity of the sparse path (training: the Hybrid's K;
// inference: ell_cap when set and below n_t * C, else n_t * C)
int ell_k(const sffn_handle* h, bool train) {
  const int full = h->n_t * h->desc.twell_cap;
  if (train) return h->desc.ell_cap;
  return (h->desc.ell_cap > 0 && h->desc.ell_cap < full) ? h->desc.ell_cap : full;
}

// Workspace layout. Every region starts at a 256-byte boundary.
struct Layout {
  size_t ovf = 0, tw_val = 0, tw_idx = 0, tw_cnt = 0, tw_flag = 0, tw_list = 0, tw_nf = 0;
  size_t ell_a = 0, ell_idx = 0, ell_cnt = 0, bk = 0, upart = 0, dlist = 0, ndense = 0;
  size_t hid = 0, zovf = 0, ovf_map = 0, part = 0, total = 0;
  // dense layer: W_d transposed to [d, F] (bf16)
  size_t wdt = 0;
  // backward
  size_t drec = 0, ncnt = 0, noff = 0, thist = 0, toff = 0, meta = 0, dH = 0, gz_rm = 0;
  size_t gz_t = 0, gu_t = 0, gh_t = 0, xb = 0, dyb = 0;
  // dense training step (transposed weights and inputs, bf16: the
  // k-contiguous operands of its long-K GEMMs)
  size_t dh_f = 0, dh_rm = 0, dz_t = 0, du_t = 0, h_t = 0, wgu_t = 0, x_t = 0, dy_t = 0;
  int64_t ldt = 0;
};

Layout layout(const sffn_handle* h, int64_t T, int op) {
  Layout L;
  const int64_t F = h->desc.d_ff, d = h->desc.d, C = h->desc.twell_cap, nt = h->n_t;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  if (op == SFFN_OP_PACK) {
    L.ovf = take((size_t)nt * ovf_words(T) * 4);
  }
  if (op == SFFN_OP_HYBRID) {
    L.bk = take((size_t)T);
  }
  if (op == SFFN_OP_FORWARD_SPARSE || op == SFFN_OP_FORWARD_TRAIN) {
    // ELL rows of capacity K (inference: lossless for every row whose TwELL
    // did not overflow when K = n_t * C); the dense path holds R rows
    const bool train = op == SFFN_OP_FORWARD_TRAIN;
    const int64_t K = ell_k(h, train);
    const int64_t Kp = (K + 7) / 8 * 8;
    const int64_t R = dense_cap(h, T);
    int ns, epl;
    slice_shape(dt_of(h), (int)d, &ns, &epl);
    L.ell_a = take((size_t)T * K * ssize(h));
    L.ell_idx = take((size_t)T * K * 2);
    L.ell_cnt = take((size_t)T * 4);
    L.bk = take((size_t)T);
    L.upart = take((size_t)ns * T * Kp * 4);
    L.tw_val = take((size_t)T * nt * C * ssize(h));
    L.tw_idx = take((size_t)T * nt * C * 2);
    L.tw_cnt = take((size_t)T * nt * 4);
    L.tw_flag = take((size_t)T);
    L.tw_list = take((size_t)T * 4);
    L.tw_nf = take(4);
    // inference: the dense path's rows (training keeps them in the Hybrid)
    if (!train) {
      L.dlist = take((size_t)R * 4);
      L.ndense = take(4);
    }
    // hidden rows of the dense path: bf16 hi|lo [R, 2F] or fp32 [R, F]
    L.hid = take((size_t)R * F * 4);
    // bf16: the gate pre-activations of overflowing tile rows, one
    // 128-float record each, R per tile column (a dense-path row
    // overflows a column at most once), and every (row, tile)'s record
    if (h->desc.dtype == SFFN_BF16) {
      L.zovf = take((size_t)R * nt * kTile * 4);
      L.ovf_map = take((size_t)T * nt * 4);
    }
    // split-K partials of the flagged rows' GEMMs (used one after the
    // other): a split problem has at most split_target / n_tiles row tiles
    // of 128 rows; the hidden GEMM keeps one partial set per B operand
    const int tiles_d = std::max(1, h->num_cu / (int)(d / 128));
    const int tiles_h = std::max(1, h->num_cu / (int)(F / 128));
    // bf16: the small-row GEMM keeps split partials of at most
    // 2 * num_cu tiles, and always the up partials of every dense row
    const size_t part_small =
        h->desc.dtype == SFFN_BF16
            ? std::max((size_t)2 * h->num_cu * 128 * 128, (size_t)((R + 127) / 128 * 128) * F)
            : 0;
    const size_t part_d = (size_t)tiles_d * 128 * d;
    const size_t part_h = (size_t)2 * tiles_h * 128 * F;
    L.part = take(std::max({part_d, part_h, part_small}) * 4);
  }
  if (op == SFFN_OP_FORWARD_DENSE) {
    L.hid = take((size_t)T * F * esize(h));
    if (h->desc.dtype == SFFN_BF16) L.wdt = take((size_t)F * d * 2);
  }
  if (op == SFFN_OP_TRAIN_DENSE) {
    // W_d transposed [d, F]
    L.wdt = take((size_t)F * d * 2);
  }
  if (op == SFFN_OP_BACKWARD_DENSE) {
    // dH [T, F] fp32; dZ | dU rows [T, 2F], and dZ, dU and H transposed
    // [F, T], bf16; W_g | W_u transposed [d, 2F] (non-gated: [d, F]); x
    // and dy transposed [d, T]
    L.dh_f = take((size_t)T * F * 4);
    L.dh_rm = take((size_t)T * F * 2 * 2);
    L.dz_t = take((size_t)T * F * 2);
    L.du_t = take((size_t)T * F * 2);
    L.h_t = take((size_t)T * F * 2);
    L.wgu_t = take((size_t)d * F * 2 * (h->desc.gated ? 2 : 1));
    L.x_t = take((size_t)d * T * 2);
    L.dy_t = take((size_t)d * T * 2);
  }
  if (op == SFFN_OP_BACKWARD) {
    // sized for up to R backup rows
    const int64_t K = h->desc.ell_cap, Kp = (K + 7) / 8 * 8;
    const int64_t R = dense_cap(h, T);
    int ns, epl;
    slice_shape(dt_of(h), (int)d, &ns, &epl);
    const bool split = h->desc.dtype == SFFN_BF16;
    const int64_t Rp = (R + 63) / 64 * 64;
    L.ldt = split ? 2 * Rp : Rp;
    L.upart = take((size_t)ns * T * Kp * 4);
    L.drec = take((size_t)T * K * 16);
    const int64_t F4 = (F + 3) / 4, nblk = transpose_blocks(T, (int)K);
    L.ncnt = take((size_t)F4 * 16);
    L.noff = take((size_t)(F + 1) * 4);
    L.thist = take((size_t)nblk * F4 * 4);
    L.toff = take((size_t)nblk * F4 * 16);
    L.meta = take((size_t)T * K * 16);
    L.dH = take((size_t)R * F * 4);
    // dZ and dU rows: bf16 [R, 4F] (dZ hi | lo, dU hi | lo), fp32 two [R, F]
    L.gz_rm = take((size_t)R * F * 8);
    L.gz_t = take((size_t)F * L.ldt * esize(h));
    L.gu_t = take((size_t)F * L.ldt * esize(h));
    L.gh_t = take((size_t)F * L.ldt * esize(h));
    L.xb = take((size_t)L.ldt * d * esize(h));
    L.dyb = take((size_t)L.ldt * d * esize(h));
    const int tiles_d = std::max(1, h->num_cu / (int)(d / 128));
    const int tiles_h = std::max(1, h->num_cu / (int)(F / 128));
    L.part = take(std::max({(size_t)tiles_d * 128 * d, (size_t)tiles_h * 128 * F,
                            (size_t)2 * h->num_cu * 128 * 128}) * 4);
  }
  L.total = o;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) { return (P*)((char*)ws + off); }

hipEvent_t take_event(sffn_handle* h) {
  if (!h->pool.empty()) {
    hipEvent_t e = h->pool.back();
    h->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one kernel launch with events when profiling is on.
struct ProfScope {
  sffn_handle* h;
  int k;
  hipStream_t s;
  hipEvent_t a = nullptr;
  ProfScope(sffn_handle* h_, int k_, hipStream_t s_) : h(h_), k(k_), s(s_) {
    if (h->prof && (a = take_event(h)) != nullptr) (void)hipEventRecord(a, s);
  }
  ~ProfScope() {
    if (!a) return;
    hipEvent_t b = take_event(h);
    if (!b) {
      h->pool.push_back(a);
      return;
    }
    (void)hipEventRecord(b, s);
    h->recs.push_back({k, a, b});
  }
};

}  // namespace

extern "C" {

const char* sffn_status_string(sffn_status s) {
  switch (s) {
    case SFFN_OK: return "SFFN_OK";
    case SFFN_E_ARG: return "SFFN_E_ARG";
    case SFFN_E_UNSUPPORTED: return "SFFN_E_UNSUPPORTED";
    case SFFN_E_HIP: return "SFFN_E_HIP";
    case SFFN_E_CAPACITY: return "SFFN_E_CAPACITY";
    default: return "unknown status";
  }
}

sffn_status sffn_create(const sffn_desc* desc, sffn_handle** out) {
  if (!out) return SFFN_E_ARG;
  *out = nullptr;
  const sffn_status st = validate_desc(desc);
  if (st != SFFN_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SFFN_E_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SFFN_E_HIP;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return SFFN_E_UNSUPPORTED;
  int32_t* dstate = nullptr;
  if (hipMalloc((void**)&dstate, kStateBytes) != hipSuccess) return SFFN_E_HIP;
  if (hipMemset(dstate, 0, kStateBytes) != hipSuccess) {
    (void)hipFree(dstate);
    return SFFN_E_HIP;
  }
  sffn_handle* h = new sffn_handle();
  h->desc = *desc;
  h->device = dev;
  h->num_cu = prop.multiProcessorCount;
  h->n_t = desc->d_ff / kTile;
  h->dstate = dstate;
  const hipError_t se = scratch_address(dev, &h->scratch);
  if (se != hipSuccess) h->scratch_err = hipGetErrorString(se);
  *out = h;
  return SFFN_OK;
}

void sffn_destroy(sffn_handle* h) {
  if (!h) return;
  for (auto& r : h->recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (auto e : h->pool) (void)hipEventDestroy(e);
  if (h->fork) (void)hipEventDestroy(h->fork);
  if (h->join) (void)hipEventDestroy(h->join);
  if (h->side) (void)hipStreamDestroy(h->side);
  if (h->dstate) (void)hipFree(h->dstate);
  delete h;
}

const char* sffn_last_error(const sffn_handle* h) { return h ? h->err.c_str() : ""; }

sffn_status sffn_workspace_bytes(const sffn_handle* h, int64_t T, int32_t op, size_t* bytes) {
  if (!h || !bytes || T < 0) return SFFN_E_ARG;
  if (op < SFFN_OP_PACK || op > SFFN_OP_BACKWARD_DENSE) return SFFN_E_ARG;
  *bytes = layout(h, T, op).total;
  return SFFN_OK;
}

static bool twell_ok(const sffn_twell* tw) {
  return tw && aligned16(tw->val) && aligned16(tw->idx) && aligned16(tw->cnt) &&
         aligned16(tw->row_flag) && aligned16(tw->flagged) && aligned16(tw->n_flagged);
}

sffn_status sffn_pack_twell(sffn_handle* h, const float* z, int64_t T, const sffn_twell* tw,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!h) return SFFN_E_ARG;
  if (T < 0 || T > (int64_t)1 << 30) return fail(h, SFFN_E_ARG, "T out of range");
  if (T == 0) return SFFN_OK;
  if (!aligned16(z)) return fail(h, SFFN_E_ARG, "z must be a non-null 16-byte aligned pointer");
  if (!twell_ok(tw)) return fail(h, SFFN_E_ARG, "TwELL buffers must be non-null and 16-byte aligned");
  const Layout L = layout(h, T, SFFN_OP_PACK);
  if (!ws || ws_bytes < L.total || ((uintptr_t)ws % kAlign) != 0)
    return fail(h, SFFN_E_ARG, "workspace missing, too small or not 256-byte aligned");
  const int ow = ovf_words(T);
  uint32_t* ovf = at<uint32_t>(ws, L.ovf);
  hipError_t e;
  {
    ProfScope ps(h, SFFN_K_PACK, stream);
    e = launch_pack(z, T, h->desc.d_ff, h->desc.twell_cap, sb_of(h), tw->val, tw->idx, tw->cnt, ovf, ow,
                    stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "pack");
  {
    ProfScope ps(h, SFFN_K_FLAGS, stream);
    e = launch_flags(ovf, h->n_t, ow, T, tw->row_flag, tw->flagged, tw->n_flagged, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "flags");
  return SFFN_OK;
}

sffn_status sffn_gate_preact(sffn_handle* h, const void* x, const void* w_gate, int64_t T,
                             float* z, hipStream_t stream) {
  if (!h) return SFFN_E_ARG;
  if (T < 0 || T > (int64_t)1 << 30) return fail(h, SFFN_E_ARG, "T out of range");
  if (T == 0) return SFFN_OK;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(z))
    return fail(h, SFFN_E_ARG, "x, w_gate and z must be non-null 16-byte aligned pointers");
  GemmArgs g = {};
  g.A = x;
  g.lda = h->desc.d;
  g.M = (int)T;
  g.B0 = w_gate;
  g.ldb = h->desc.d;
  g.N = h->desc.d_ff;
  g.K = h->desc.d;
  g.out = z;
  g.ldo = h->desc.d_ff;
  g.num_cu = h->num_cu;
  g.grid = gemm_grid(dt_of(h), 1, h->num_cu);
  hipError_t e;
  {
    ProfScope ps(h, SFFN_K_GATE_PREACT, stream);
    e = launch_gemm(dt_of(h), 1, false, kEpiStoreF32, g, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "gate GEMM");
  return SFFN_OK;
}

// split-K target of the small-row GEMMs: two workgroups per CU
static int small_split_target(const sffn_handle* h) { return 2 * h->num_cu; }

static sffn_status forward_dense(sffn_handle* h, const void* x, const void* wg, const void* wu,
                                 const void* wd, int64_t T, float* y, void* ws,
                                 const Layout& L, hipStream_t stream) {
  const sffn_desc& D = h->desc;
  const Dtype dt = dt_of(h);
  void* hid = at<char>(ws, L.hid);
  // H = ReLU(x W_g) * (x W_u)  (or ReLU(x W_1)), bf16-rounded for bf16 layers
  GemmArgs g = {};
  g.A = x;
  g.lda = D.d;
  g.M = (int)T;
  g.B0 = wg;
  g.B1 = wu;
  g.ldb = D.d;
  g.N = D.d_ff;
  g.K = D.d;
  g.out = hid;
  g.ldo = D.d_ff;
  g.act = 1;
  const int nb = D.gated ? 2 : 1;
  g.num_cu = h->num_cu;
  g.grid = gemm_grid(dt, nb, h->num_cu);
  hipError_t e;
  {
    ProfScope ps(h, SFFN_K_DENSE_GATEUP, stream);
    e = launch_gemm(dt, nb, false, dt == kBF16 ? kEpiHiddenBF16 : kEpiStoreF32, g, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "dense gate/up GEMM");
  // y = H W_d. bf16: W_d [F, d] is first transposed into the workspace, so
  // that both operands of the down GEMM are k-contiguous (the long-K ring)
  GemmArgs g2 = {};
  g2.A = hid;
  g2.lda = D.d_ff;
  g2.M = (int)T;
  g2.B0 = wd;
  g2.ldb = D.d;
  g2.N = D.d;
  g2.K = D.d_ff;
  g2.out = y;
  g2.ldo = D.d;
  g2.num_cu = h->num_cu;
  g2.grid = gemm_grid(dt, 1, h->num_cu);
  {
    ProfScope ps(h, SFFN_K_DENSE_DOWN, stream);
    if (dt == kBF16) {
      uint16_t* wdt = at<uint16_t>(ws, L.wdt);
      e = launch_transpose_bf16((const uint16_t*)wd, D.d, wdt, D.d_ff, D.d_ff, D.d, stream);
      g2.B0 = wdt;
      g2.ldb = D.d_ff;
      if (e == hipSuccess) e = launch_gemm(dt, 1, false, kEpiStoreF32, g2, stream);
    } else {
      e = launch_gemm(dt, 1, true, kEpiStoreF32, g2, stream);
    }
  }
  if (e != hipSuccess) return hip_fail(h, e, "dense down GEMM");
  return SFFN_OK;
}

static bool hybrid_ok(const sffn_handle* h, const sffn_hybrid* hy, bool need_u) {
  if (!hy || hy->max_backup < 0) return false;
  if (!aligned16(hy->ell_a) || !aligned16(hy->ell_idx) || !aligned16(hy->ell_cnt) ||
      !aligned16(hy->slot) || !aligned16(hy->n_backup))
    return false;
  if (hy->max_backup > 0 && (!aligned16(hy->brow) || !aligned16(hy->bk_a))) return false;
  if (need_u && h->desc.gated) {
    if (!aligned16(hy->ell_u)) return false;
    if (hy->max_backup > 0 && !aligned16(hy->bk_u)) return false;
  }
  return true;
}

// The sparse forward shared by inference (hy == NULL: ELL capacity n_t*C,
// only TwELL-overflow rows take the dense path) and training (hy != NULL:
// capacity K = ell_cap, the Hybrid of the step is saved).
static sffn_status sparse_forward(sffn_handle* h, const void* x, const void* w_gate,
                                  const void* w_up, const void* w_down, int64_t T, float* y,
                                  const sffn_twell* tw, const sffn_hybrid* hy, void* ws,
                                  const Layout& L, hipStream_t stream) {
  const sffn_desc& D = h->desc;
  const Dtype dt = dt_of(h);
  const bool train = hy != nullptr;
  sffn_twell t;
  if (tw) {
    t = *tw;
  } else {
    t.val = at<char>(ws, L.tw_val);
    t.idx = at<uint16_t>(ws, L.tw_idx);
    t.cnt = at<int32_t>(ws, L.tw_cnt);
    t.row_flag = at<uint8_t>(ws, L.tw_flag);
    t.flagged = at<int32_t>(ws, L.tw_list);
    t.n_flagged = at<int32_t>(ws, L.tw_nf);
  }
  const int K = ell_k(h, train);
  const int Kp = (K + 7) / 8 * 8;
  const int64_t R = dense_cap(h, T);
  // rows the dense path computes: training min(max_backup, R), inference R
  const int mcap = (int)(train ? std::min<int64_t>(hy->max_backup, R) : R);
  int32_t* status = h->dstate;
  int32_t* ovf_ctr = h->dstate + kCtrOffset / 4;
  hipError_t e = hipSuccess;
  if (dt == kBF16 && h->ctr_dirty) {
    // a call stopped between its gate GEMM and its list kernel
    e = launch_zero(ovf_ctr, (size_t)h->n_t * kCtrStride * 4, stream);
    if (e != hipSuccess) return hip_fail(h, e, "overflow-record counter");
    h->ctr_dirty = false;
  }

  // 1. gate GEMM, ReLU + TwELL pack in the epilogue
  GemmArgs g = {};
  g.A = x;
  g.lda = D.d;
  g.M = (int)T;
  g.B0 = w_gate;
  g.ldb = D.d;
  g.N = D.d_ff;
  g.K = D.d;
  g.tw_val = t.val;
  g.tw_idx = t.idx;
  g.tw_cnt = t.cnt;
  g.C = D.twell_cap;
  g.n_t = h->n_t;
  g.store_bf16 = sb_of(h);
  if (dt == kBF16) {
    g.zovf = at<float>(ws, L.zovf);
    g.ovf_map = at<int32_t>(ws, L.ovf_map);
    g.ovf_ctr = ovf_ctr;
    g.ovf_cap = (int)R;
    h->ctr_dirty = true;
  }
  g.num_cu = h->num_cu;
  g.grid = gemm_grid(dt, 1, h->num_cu);
  {
    ProfScope ps(h, SFFN_K_GATE_TWELL, stream);
    e = launch_gemm(dt, 1, false, kEpiTwell, g, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "gate GEMM + TwELL");

  // 2. per-row route and ELL compaction
  EllArgs ea = {};
  ea.val = t.val;
  ea.idx = t.idx;
  ea.cnt = t.cnt;
  ea.T = T;
  ea.n_t = h->n_t;
  ea.C = D.twell_cap;
  ea.K = K;
  ea.ell_a = train ? hy->ell_a : at<char>(ws, L.ell_a);
  ea.store_bf16 = sb_of(h);
  ea.ell_idx = train ? hy->ell_idx : at<uint16_t>(ws, L.ell_idx);
  ea.ell_cnt = train ? hy->ell_cnt : at<int32_t>(ws, L.ell_cnt);
  ea.row_flag = t.row_flag;
  ea.bk = at<uint8_t>(ws, L.bk);
  {
    ProfScope ps(h, SFFN_K_ROWS, stream);
    e = launch_rows(ea, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "row compaction");

  // 3. the dense path's rows: their ascending list (the first mcap of them;
  //    more raise the capacity status), and the TwELL's own list of
  //    overflowing rows
  int32_t* brow = train ? hy->brow : at<int32_t>(ws, L.dlist);
  int32_t* n_bk = train ? hy->n_backup : at<int32_t>(ws, L.ndense);
  // the sparse up/down over the ELL rows, d sliced across the XCDs (step 5)
  SliceArgs sa = {};
  sa.x = x;
  sa.wu = w_up;
  sa.wd = w_down;
  sa.ell_idx = ea.ell_idx;
  sa.ell_a = ea.ell_a;
  sa.ell_cnt = ea.ell_cnt;
  sa.bk = ea.bk;
  sa.T = T;
  sa.d = D.d;
  sa.K = K;
  sa.Kp = Kp;
  sa.upart = at<float>(ws, L.upart);
  sa.ell_u = (train && D.gated) ? hy->ell_u : nullptr;
  sa.store_bf16 = sb_of(h);
  sa.y = y;
  // bf16 gated layers with the sliced up/down: the lists are built by eight
  // extra workgroups of the up projection's launch, and the dense path's
  // hidden rows are combined in the launch of the slice sums, so that
  // these short latency-bound steps overlap the sparse ones
  const bool joint = dt == kBF16 && D.gated && (train || D.updown != 1);
  {
    const ListArgs lb = {ea.bk, brow, mcap, n_bk, train ? hy->slot : nullptr, status,
                         dt == kBF16 ? ovf_ctr : nullptr, h->n_t};
    const ListArgs lf = {t.row_flag, t.flagged, T, t.n_flagged, nullptr, nullptr, nullptr, 0};
    if (joint) {
      ProfScope ps(h, SFFN_K_SPARSE_UP, stream);
      e = launch_up_with_lists(dt, sa, lb, &lf, T, stream);
    } else {
      ProfScope ps(h, SFFN_K_FLAGS, stream);
      e = launch_backup_list(lb, &lf, T, stream);
    }
  }
  if (e != hipSuccess) return hip_fail(h, e, joint ? "sparse up + backup list" : "backup list");
  h->ctr_dirty = false;

  // 4. dense path: hidden rows H = ReLU(z) * (x W_u) (split-K over the
  //    few rows, then a combine that stores H as bf16 hi + lo, or fp32, and
  //    in training the ReLU(z) and u rows), then y = H W_d scattered into
  //    the rows (split-K + reduce). The dense path touches only its rows of
  //    y (and its own workspace), the sparse phases only the others. It
  //    runs in line on the caller's stream: on a second stream its few
  //    workgroups were starved beside the sparse grids and ended last,
  //    which measured slower than running it in line.
  void* hid = at<char>(ws, L.hid);
  float* part = at<float>(ws, L.part);
  GemmArgs down_late = {};   // bf16: the dense path's down product, run last
  GemmArgs hid_late = {};    // joint: the hidden rows' combine, beside the slice sums
  if (mcap > 0 && dt == kBF16) {
    // ReLU(z) of the rows comes from the gate GEMM itself (their TwELL
    // tiles, and the saved pre-activations of the tiles that overflowed);
    // gated layers add u = x W_u (split-K partials) and the combine forms
    // H = ReLU(z) u as bf16 hi | lo (and ReLU(z), u rows in training)
    const int nb = D.gated ? 2 : 1;
    GemmArgs f = {};
    f.A = x;
    f.lda = D.d;
    f.a_rows = brow;
    f.m_dev = n_bk;
    f.m_cap = mcap;
    f.B0 = w_up;
    f.ldb = D.d;
    f.N = D.d_ff;
    f.K = D.d;
    f.out = hid;
    f.act = 1;
    f.ldo = 2 * (int64_t)D.d_ff;
    f.lo_off = D.d_ff;
    if (train) {
      f.out_a = hy->bk_a;
      f.out_u = D.gated ? hy->bk_u : nullptr;
      f.ldo_au = D.d_ff;
    }
    f.tw_val = t.val;
    f.tw_idx = t.idx;
    f.tw_cnt = t.cnt;
    f.C = D.twell_cap;
    f.n_t = h->n_t;
    f.store_bf16 = sb_of(h);
    f.zovf = at<float>(ws, L.zovf);
    f.ovf_map = at<int32_t>(ws, L.ovf_map);
    f.ovf_cap = (int)R;
    f.part = part;
    // about one tile per CU: with only a few rows a deeper split costs
    // more in partials than it gains in parallel loads
    f.split_target = h->num_cu;
    f.split_max = std::min(kSplitMax, D.d / 32);
    f.num_cu = h->num_cu;
    f.grid = gemm_small_grid(h->num_cu);
    {
      ProfScope ps(h, SFFN_K_FLAG_GATEUP, stream);
      if (D.gated) e = launch_gemm_small(false, kEpiHiddenSplitK, f, stream);
      if (e == hipSuccess && !joint) e = launch_flag_hidden(nb, f, stream);
    }
    if (e != hipSuccess) return hip_fail(h, e, "dense-path hidden rows");
    if (joint) hid_late = f;
    // H_hi W_d + H_lo W_d: a dual A over the F rows of W_d
    GemmArgs f2 = {};
    f2.A = hid;
    f2.lda = 2 * (int64_t)D.d_ff;
    f2.alo = D.d_ff;
    f2.m_dev = n_bk;
    f2.m_cap = mcap;
    f2.B0 = w_down;
    f2.ldb = D.d;
    f2.N = D.d;
    f2.K = D.d_ff;
    f2.out = y;
    f2.ldo = D.d;
    f2.out_rows = brow;
    f2.part = part;
    f2.split_target = small_split_target(h);
    f2.split_max = std::min(kSplitMax, f2.K / 32);
    f2.num_cu = h->num_cu;
    f2.grid = gemm_small_grid(h->num_cu);
    // launched after the sparse down projection (joint: before it, its
    // reduce inside that launch)
    down_late = f2;
  } else if (mcap > 0) {
    GemmArgs f = {};
    f.A = x;
    f.lda = D.d;
    f.a_rows = brow;
    f.m_dev = n_bk;
    f.m_cap = mcap;
    f.B0 = w_gate;
    f.B1 = w_up;
    f.ldb = D.d;
    f.N = D.d_ff;
    f.K = D.d;
    f.out = hid;
    f.act = 1;
    f.ldo = dt == kBF16 ? 2 * (int64_t)D.d_ff : (int64_t)D.d_ff;
    f.lo_off = D.d_ff;
    if (train) {
      f.out_a = hy->bk_a;
      f.out_u = D.gated ? hy->bk_u : nullptr;
      f.ldo_au = D.d_ff;
    }
    f.part = part;
    f.split_target = h->num_cu;
    f.split_max = std::min(kSplitMax, D.d / (dt == kBF16 ? 64 : 32));
    const int nb = D.gated ? 2 : 1;
    f.num_cu = h->num_cu;
    f.grid = gemm_grid(dt, nb, h->num_cu);
    {
      ProfScope ps(h, SFFN_K_FLAG_GATEUP, stream);
      e = launch_gemm(dt, nb, false, kEpiHiddenSplitK, f, stream);
      if (e == hipSuccess) e = launch_hidden_combine(dt, nb, f, stream);
    }
    if (e != hipSuccess) return hip_fail(h, e, "dense-path hidden rows");
    GemmArgs f2 = {};
    f2.A = hid;
    f2.m_dev = n_bk;
    f2.m_cap = mcap;
    f2.B0 = w_down;
    f2.ldb = D.d;
    f2.N = D.d;
    if (dt == kBF16) {
      // [H_hi | H_lo] x [W_d ; W_d]: K = 2F with the B index wrapped at F
      f2.lda = 2 * (int64_t)D.d_ff;
      f2.K = 2 * D.d_ff;
      f2.kwrap = D.d_ff;
    } else {
      f2.lda = D.d_ff;
      f2.K = D.d_ff;
    }
    f2.out = y;
    f2.ldo = D.d;
    f2.out_rows = brow;
    f2.part = part;
    f2.split_target = h->num_cu;
    const int nkt = f2.K / (dt == kBF16 ? 64 : 32);
    f2.split_max = std::min(kSplitMax, nkt);
    f2.num_cu = h->num_cu;
    f2.grid = gemm_grid(dt, 1, h->num_cu);
    {
      ProfScope ps(h, SFFN_K_FLAG_DOWN, stream);
      e = launch_gemm(dt, 1, true, kEpiStoreF32, f2, stream);
    }
    if (e != hipSuccess) return hip_fail(h, e, "dense-path down GEMM");
    {
      ProfScope ps(h, SFFN_K_SPLITK_REDUCE, stream);
      e = launch_splitk_reduce(f2, y, D.d, stream);
    }
    if (e != hipSuccess) return hip_fail(h, e, "split-K reduce");
  }

  // 5. sparse up/down over the ELL rows (the up projection already ran when
  //    joint)
  if (!train && D.updown == 1) {
    ProfScope ps(h, SFFN_K_FUSED_UPDOWN, stream);
    e = launch_fused_updown(D.gated != 0, sa, stream);
  } else {
    if (D.gated && !joint) {
      ProfScope ps(h, SFFN_K_SPARSE_UP, stream);
      e = launch_updown(dt, true, 0, sa, stream);
    }
    if (D.gated && e == hipSuccess) {
      ProfScope ps(h, SFFN_K_SPARSE_HSUM, stream);
      e = hid_late.out != nullptr ? launch_flag_hidden_hsum(dt, hid_late, sa, stream)
                                  : launch_updown(dt, true, 2, sa, stream);
    }
    if (e == hipSuccess && joint && down_late.out != nullptr) {
      // the dense path's down product first, its split-K reduce in the
      // launch of the sparse down projection (they write other rows of y)
      {
        ProfScope ps(h, SFFN_K_FLAG_DOWN, stream);
        e = launch_gemm_small(true, kEpiStoreF32, down_late, stream);
      }
      if (e != hipSuccess) return hip_fail(h, e, "dense-path down GEMM");
      ProfScope ps(h, SFFN_K_SPARSE_DOWN, stream);
      e = launch_down_with_reduce(dt, D.gated != 0, sa, down_late, stream);
      down_late = {};
    } else if (e == hipSuccess) {
      ProfScope ps(h, SFFN_K_SPARSE_DOWN, stream);
      e = launch_updown(dt, D.gated != 0, 1, sa, stream);
    }
  }
  if (e != hipSuccess) return hip_fail(h, e, "sparse up/down");
  if (down_late.out != nullptr) {
    {
      ProfScope ps(h, SFFN_K_FLAG_DOWN, stream);
      e = launch_gemm_small(true, kEpiStoreF32, down_late, stream);
    }
    if (e != hipSuccess) return hip_fail(h, e, "dense-path down GEMM");
    {
      ProfScope ps(h, SFFN_K_SPLITK_REDUCE, stream);
      e = launch_splitk_reduce(down_late, y, D.d, stream);
    }
    if (e != hipSuccess) return hip_fail(h, e, "split-K reduce");
  }
  return SFFN_OK;
}

static sffn_status forward_args(sffn_handle* h, const void* x, const void* w_gate,
                                const void* w_up, const void* w_down, int64_t T, const float* y,
                                const sffn_twell* tw) {
  const sffn_desc& D = h->desc;
  if (T < 0 || T > (int64_t)1 << 30) return fail(h, SFFN_E_ARG, "T out of range");
  if (T == 0) return SFFN_OK;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_down) || !aligned16(y))
    return fail(h, SFFN_E_ARG, "x, w_gate, w_down and y must be non-null 16-byte aligned pointers");
  if (D.gated ? !aligned16(w_up) : w_up != nullptr)
    return fail(h, SFFN_E_ARG, "w_up must be a 16-byte aligned pointer iff the layer is gated");
  if (tw && !twell_ok(tw))
    return fail(h, SFFN_E_ARG, "TwELL buffers must be non-null and 16-byte aligned");
  return SFFN_OK;
}

static bool ws_ok(void* ws, size_t ws_bytes, const Layout& L) {
  if (L.total == 0) return true;
  return ws && ws_bytes >= L.total && ((uintptr_t)ws % kAlign) == 0;
}

sffn_status sffn_forward(sffn_handle* h, const void* x, const void* w_gate, const void* w_up,
                         const void* w_down, int64_t T, float* y, const sffn_twell* tw,
                         int32_t mode, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!h) return SFFN_E_ARG;
  if (mode != SFFN_SPARSE && mode != SFFN_DENSE) return fail(h, SFFN_E_ARG, "unknown mode");
  sffn_status st = forward_args(h, x, w_gate, w_up, w_down, T, y, tw);
  if (st != SFFN_OK || T == 0) return st;
  if (mode == SFFN_DENSE && tw) return fail(h, SFFN_E_ARG, "dense mode takes no TwELL");
  const Layout L = layout(h, T, mode == SFFN_SPARSE ? SFFN_OP_FORWARD_SPARSE : SFFN_OP_FORWARD_DENSE);
  if (!ws_ok(ws, ws_bytes, L))
    return fail(h, SFFN_E_ARG, "workspace missing, too small or not 256-byte aligned");
  if (mode == SFFN_DENSE) return forward_dense(h, x, w_gate, w_up, w_down, T, y, ws, L, stream);
  return sparse_forward(h, x, w_gate, w_up, w_down, T, y, tw, nullptr, ws, L, stream);
}

sffn_status sffn_forward_noalloc(sffn_handle* h, const void* x, const void* w_gate,
                                 const void* w_up, const void* w_down, int64_t T, float* y,
                                 const sffn_twell* tw, int32_t mode, hipStream_t stream) {
  if (!h) return SFFN_E_ARG;
  if (mode != SFFN_SPARSE && mode != SFFN_DENSE) return fail(h, SFFN_E_ARG, "unknown mode");
  sffn_status st = forward_args(h, x, w_gate, w_up, w_down, T, y, tw);
  if (st != SFFN_OK || T == 0) return st;
  if (mode == SFFN_DENSE && tw) return fail(h, SFFN_E_ARG, "dense mode takes no TwELL");
  if (h->scratch == nullptr)
    return fail(h, SFFN_E_HIP, "static scratch unavailable: " + h->scratch_err);
  const Layout L = layout(h, T, mode == SFFN_SPARSE ? SFFN_OP_FORWARD_SPARSE : SFFN_OP_FORWARD_DENSE);
  if (L.total > kScratchBytes)
    return fail(h, SFFN_E_ARG,
                "the call needs " + std::to_string(L.total) + " bytes of workspace; the static "
                "scratch holds " + std::to_string(kScratchBytes) + " (use sffn_forward)");
  // no timing events here: creating one may allocate
  const bool prof = h->prof;
  h->prof = false;
  st = mode == SFFN_DENSE
           ? forward_dense(h, x, w_gate, w_up, w_down, T, y, h->scratch, L, stream)
           : sparse_forward(h, x, w_gate, w_up, w_down, T, y, tw, nullptr, h->scratch, L, stream);
  h->prof = prof;
  return st;
}

sffn_status sffn_forward_train(sffn_handle* h, const void* x, const void* w_gate,
                               const void* w_up, const void* w_down, int64_t T, float* y,
                               const sffn_twell* tw, const sffn_hybrid* hy, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  if (!h) return SFFN_E_ARG;
  if (h->desc.ell_cap < 1) return fail(h, SFFN_E_ARG, "training needs desc.ell_cap >= 1");
  sffn_status st = forward_args(h, x, w_gate, w_up, w_down, T, y, tw);
  if (st != SFFN_OK || T == 0) return st;
  if (!hybrid_ok(h, hy, true))
    return fail(h, SFFN_E_ARG, "Hybrid buffers must be non-null and 16-byte aligned");
  const Layout L = layout(h, T, SFFN_OP_FORWARD_TRAIN);
  if (!ws_ok(ws, ws_bytes, L))
    return fail(h, SFFN_E_ARG, "workspace missing, too small or not 256-byte aligned");
  return sparse_forward(h, x, w_gate, w_up, w_down, T, y, tw, hy, ws, L, stream);
}

// the dense training step's saved activations: Z_s, U_s (gated) and H,
// [T, F] bf16 each
static size_t train_dense_act_elems(const sffn_handle* h, int64_t T) {
  return (size_t)T * h->desc.d_ff * (h->desc.gated ? 3 : 2);
}

static sffn_status train_dense_args(sffn_handle* h, int64_t T) {
  if (h->desc.dtype != SFFN_BF16)
    return fail(h, SFFN_E_UNSUPPORTED, "the dense training step is the bf16 layer's");
  if (T < 0 || T > (int64_t)1 << 30) return fail(h, SFFN_E_ARG, "T out of range");
  if (T % 64 != 0)
    return fail(h, SFFN_E_UNSUPPORTED, "the dense training step needs T % 64 == 0");
  return SFFN_OK;
}

sffn_status sffn_train_dense_act_bytes(const sffn_handle* h, int64_t T, size_t* bytes) {
  if (!h || !bytes || T < 0) return SFFN_E_ARG;
  *bytes = train_dense_act_elems(h, T) * 2;
  return SFFN_OK;
}

sffn_status sffn_forward_train_dense(sffn_handle* h, const void* x, const void* w_gate,
                                     const void* w_up, const void* w_down, int64_t T, float* y,
                                     void* act, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!h) return SFFN_E_ARG;
  sffn_status st = train_dense_args(h, T);
  if (st != SFFN_OK) return st;
  st = forward_args(h, x, w_gate, w_up, w_down, T, y, nullptr);
  if (st != SFFN_OK || T == 0) return st;
  if (!aligned16(act)) return fail(h, SFFN_E_ARG, "act must be a non-null 16-byte aligned pointer");
  const Layout L = layout(h, T, SFFN_OP_TRAIN_DENSE);
  if (!ws_ok(ws, ws_bytes, L))
    return fail(h, SFFN_E_ARG, "workspace missing, too small or not 256-byte aligned");
  const sffn_desc& D = h->desc;
  const int64_t TF = T * (int64_t)D.d_ff;
  uint16_t* a16 = (uint16_t*)act;
  uint16_t* hid = a16 + (D.gated ? 2 : 1) * TF;
  GemmArgs g = {};
  g.A = x;
  g.lda = D.d;
  g.M = (int)T;
  g.B0 = w_gate;
  g.B1 = w_up;
  g.ldb = D.d;
  g.N = D.d_ff;
  g.K = D.d;
  g.out = hid;
  g.ldo = D.d_ff;
  g.save_z = a16;
  g.save_u = D.gated ? a16 + TF : nullptr;
  g.ld_save = D.d_ff;
  g.num_cu = h->num_cu;
  const int nb = D.gated ? 2 : 1;
  g.grid = gemm_grid(kBF16, nb, h->num_cu);
  hipError_t e;
  {
    ProfScope ps(h, SFFN_K_TRAIN_DENSE_GATEUP, stream);
    e = launch_gemm(kBF16, nb, false, kEpiTrainFwd, g, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "dense training gate/up GEMM");
  GemmArgs g2 = {};
  g2.A = hid;
  g2.lda = D.d_ff;
  g2.M = (int)T;
  g2.N = D.d;
  g2.K = D.d_ff;
  g2.out = y;
  g2.ldo = D.d;
  g2.num_cu = h->num_cu;
  g2.grid = gemm_grid(kBF16, 1, h->num_cu);
  {
    // W_d transposed first: both operands of the down GEMM k-contiguous
    ProfScope ps(h, SFFN_K_TRAIN_DENSE_DOWN, stream);
    uint16_t* wdt = at<uint16_t>(ws, L.wdt);
    e = launch_transpose_bf16((const uint16_t*)w_down, D.d, wdt, D.d_ff, D.d_ff, D.d, stream);
    g2.B0 = wdt;
    g2.ldb = D.d_ff;
    if (e == hipSuccess) e = launch_gemm(kBF16, 1, false, kEpiStoreF32, g2, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "dense training down GEMM");
  return SFFN_OK;
}

sffn_status sffn_backward_dense(sffn_handle* h, const void* x, const void* w_gate,
                                const void* w_up, const void* w_down, const void* act,
                                const void* dy, int64_t T, float* dx, float* dw_gate,
                                float* dw_up, float* dw_down, float l1_coeff, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  if (!h) return SFFN_E_ARG;
  sffn_status st = train_dense_args(h, T);
  if (st != SFFN_OK) return st;
  const sffn_desc& D = h->desc;
  if (!aligned16(dw_gate) || !aligned16(dw_down) || (D.gated ? !aligned16(dw_up) : dw_up != nullptr))
    return fail(h, SFFN_E_ARG, "dW pointers must be 16-byte aligned (dw_up iff the layer is gated)");
  if (T == 0) {
    hipError_t e = launch_zero(dw_gate, (size_t)D.d_ff * D.d * 4, stream);
    if (e == hipSuccess && dw_up) e = launch_zero(dw_up, (size_t)D.d_ff * D.d * 4, stream);
    if (e == hipSuccess) e = launch_zero(dw_down, (size_t)D.d_ff * D.d * 4, stream);
    return e == hipSuccess ? SFFN_OK : hip_fail(h, e, "zero dW");
  }
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_down) || !aligned16(dy) ||
      !aligned16(dx) || !aligned16(act))
    return fail(h, SFFN_E_ARG, "x, weights, act, dy and dx must be non-null 16-byte aligned pointers");
  if (D.gated ? !aligned16(w_up) : w_up != nullptr)
    return fail(h, SFFN_E_ARG, "w_up must be a 16-byte aligned pointer iff the layer is gated");
  const Layout L = layout(h, T, SFFN_OP_BACKWARD_DENSE);
  if (!ws_ok(ws, ws_bytes, L))
    return fail(h, SFFN_E_ARG, "workspace missing, too small or not 256-byte aligned");
  const int64_t TF = T * (int64_t)D.d_ff;
  const uint16_t* a16 = (const uint16_t*)act;
  uint16_t* dzu = at<uint16_t>(ws, L.dh_rm);
  uint16_t* dzt = at<uint16_t>(ws, L.dz_t);
  uint16_t* dut = at<uint16_t>(ws, L.du_t);
  uint16_t* ht = at<uint16_t>(ws, L.h_t);
  hipError_t e;
  // dH = dy W_d^T (fp32), then dZ, dU from it and the saved Z_s, U_s
  // (rows and transposed)
  float* dhf = at<float>(ws, L.dh_f);
  GemmArgs g = {};
  g.A = dy;
  g.lda = D.d;
  g.M = (int)T;
  g.B0 = w_down;
  g.ldb = D.d;
  g.N = D.d_ff;
  g.K = D.d;
  g.out = dhf;
  g.ldo = D.d_ff;
  g.num_cu = h->num_cu;
  g.grid = gemm_grid(kBF16, 1, h->num_cu);
  {
    ProfScope ps(h, SFFN_K_BWD_DENSE_DH, stream);
    e = launch_gemm(kBF16, 1, false, kEpiStoreF32, g, stream);
    if (e == hipSuccess)
      e = launch_dense_grad(dhf, a16, D.gated ? a16 + TF : nullptr, l1_coeff, T, D.d_ff, dzu, dzt,
                            dut, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "dense backward dH, dZ, dU");
  // dx = [dZ | dU] [W_g | W_u]^T as one GEMM over K = 2F (non-gated: dZ
  // W_1^T over K = F), with the weights transposed first so that both
  // operands are k-contiguous
  {
    ProfScope ps(h, SFFN_K_BWD_DENSE_DX, stream);
    uint16_t* wt = at<uint16_t>(ws, L.wgu_t);
    const int64_t ldw = (D.gated ? 2 : 1) * (int64_t)D.d_ff;
    e = launch_transpose_bf16((const uint16_t*)w_gate, D.d, wt, ldw, D.d_ff, D.d, stream);
    if (e == hipSuccess && D.gated)
      e = launch_transpose_bf16((const uint16_t*)w_up, D.d, wt + D.d_ff, ldw, D.d_ff, D.d, stream);
    GemmArgs f = {};
    f.A = dzu;
    f.lda = 2 * (int64_t)D.d_ff;
    f.M = (int)T;
    f.B0 = wt;
    f.ldb = ldw;
    f.N = D.d;
    f.K = (int)ldw;
    f.out = dx;
    f.ldo = D.d;
    f.num_cu = h->num_cu;
    f.grid = gemm_grid(kBF16, 1, h->num_cu);
    if (e == hipSuccess) e = launch_gemm(kBF16, 1, false, kEpiStoreF32, f, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "dense backward dx GEMM");
  // H, x and dy transposed ([F, T], [d, T]: the k-contiguous operands of
  // the dW GEMMs)
  uint16_t* xt = at<uint16_t>(ws, L.x_t);
  uint16_t* dyt = at<uint16_t>(ws, L.dy_t);
  {
    ProfScope ps(h, SFFN_K_BWD_DENSE_DW, stream);
    e = launch_transpose_bf16(a16 + (D.gated ? 2 : 1) * TF, D.d_ff, ht, T, T, D.d_ff, stream);
    if (e == hipSuccess) e = launch_transpose_bf16((const uint16_t*)x, D.d, xt, T, T, D.d, stream);
    if (e == hipSuccess) e = launch_transpose_bf16((const uint16_t*)dy, D.d, dyt, T, T, D.d, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "dense backward transpose");
  // dW_g = dZ^T x, dW_u = dU^T x, dW_d = H^T dy
  for (int pass = 0; pass < 3; ++pass) {
    if (pass == 1 && !D.gated) continue;
    GemmArgs w = {};
    w.A = pass == 0 ? (const void*)dzt : pass == 1 ? (const void*)dut : (const void*)ht;
    w.lda = T;
    w.M = D.d_ff;
    w.B0 = pass == 2 ? dyt : xt;
    w.ldb = T;
    w.N = D.d;
    w.K = (int)T;
    w.out = pass == 0 ? dw_gate : pass == 1 ? dw_up : dw_down;
    w.ldo = D.d;
    w.num_cu = h->num_cu;
    w.grid = gemm_grid(kBF16, 1, h->num_cu);
    ProfScope ps(h, SFFN_K_BWD_DENSE_DW, stream);
    e = launch_gemm(kBF16, 1, false, kEpiStoreF32, w, stream);
    if (e != hipSuccess) return hip_fail(h, e, "dense backward dW GEMM");
  }
  return SFFN_OK;
}

sffn_status sffn_hybrid_compact(sffn_handle* h, const sffn_twell* tw, const float* z, int64_t T,
                                const sffn_hybrid* hy, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (!h) return SFFN_E_ARG;
  if (h->desc.ell_cap < 1) return fail(h, SFFN_E_ARG, "the Hybrid needs desc.ell_cap >= 1");
  if (T < 0 || T > (int64_t)1 << 30) return fail(h, SFFN_E_ARG, "T out of range");
  if (T == 0) return SFFN_OK;
  if (!twell_ok(tw)) return fail(h, SFFN_E_ARG, "TwELL buffers must be non-null and 16-byte aligned");
  if (!hybrid_ok(h, hy, false))
    return fail(h, SFFN_E_ARG, "Hybrid buffers must be non-null and 16-byte aligned");
  if (z && !aligned16(z)) return fail(h, SFFN_E_ARG, "z must be 16-byte aligned");
  const Layout L = layout(h, T, SFFN_OP_HYBRID);
  if (!ws_ok(ws, ws_bytes, L))
    return fail(h, SFFN_E_ARG, "workspace missing, too small or not 256-byte aligned");
  EllArgs ea = {};
  ea.val = tw->val;
  ea.idx = tw->idx;
  ea.cnt = tw->cnt;
  ea.T = T;
  ea.n_t = h->n_t;
  ea.C = h->desc.twell_cap;
  ea.K = h->desc.ell_cap;
  ea.ell_a = hy->ell_a;
  ea.ell_idx = hy->ell_idx;
  ea.ell_cnt = hy->ell_cnt;
  ea.row_flag = nullptr;
  ea.store_bf16 = sb_of(h);
  ea.bk = at<uint8_t>(ws, L.bk);
  hipError_t e;
  {
    ProfScope ps(h, SFFN_K_ROWS, stream);
    e = launch_rows(ea, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "row compaction");
  {
    ProfScope ps(h, SFFN_K_FLAGS, stream);
    const ListArgs lb = {ea.bk, hy->brow, hy->max_backup, hy->n_backup, hy->slot, nullptr,
                         nullptr, 0};
    e = launch_backup_list(lb, nullptr, T, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "backup list");
  if (z && hy->max_backup > 0) {
    e = launch_gather_relu_rows(z, h->desc.d_ff, sb_of(h), hy->brow, hy->n_backup,
                                (int)std::min<int64_t>(hy->max_backup, T), hy->bk_a, stream);
    if (e != hipSuccess) return hip_fail(h, e, "backup rows");
  }
  return SFFN_OK;
}

sffn_status sffn_backward(sffn_handle* h, const void* x, const void* w_gate, const void* w_up,
                          const void* w_down, const sffn_hybrid* hy, const void* dy, int64_t T,
                          float* dx, float* dw_gate, float* dw_up, float* dw_down, float l1_coeff,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!h) return SFFN_E_ARG;
  const sffn_desc& D = h->desc;
  if (D.ell_cap < 1) return fail(h, SFFN_E_ARG, "the backward needs desc.ell_cap >= 1");
  if (T < 0 || T > (int64_t)1 << 30 || T * (int64_t)D.ell_cap >= ((int64_t)1 << 31))
    return fail(h, SFFN_E_ARG, "T out of range");
  if (!aligned16(dw_gate) || !aligned16(dw_down) || (D.gated ? !aligned16(dw_up) : dw_up != nullptr))
    return fail(h, SFFN_E_ARG, "dW pointers must be 16-byte aligned (dw_up iff the layer is gated)");
  if (T == 0) {
    // no rows: the weight gradients are zero
    hipError_t e = launch_zero(dw_gate, (size_t)D.d_ff * D.d * 4, stream);
    if (e == hipSuccess && dw_up) e = launch_zero(dw_up, (size_t)D.d_ff * D.d * 4, stream);
    if (e == hipSuccess) e = launch_zero(dw_down, (size_t)D.d_ff * D.d * 4, stream);
    return e == hipSuccess ? SFFN_OK : hip_fail(h, e, "zero dW");
  }
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_down) || !aligned16(dy) || !aligned16(dx))
    return fail(h, SFFN_E_ARG, "x, weights, dy and dx must be non-null 16-byte aligned pointers");
  if (D.gated ? !aligned16(w_up) : w_up != nullptr)
    return fail(h, SFFN_E_ARG, "w_up must be a 16-byte aligned pointer iff the layer is gated");
  if (!hybrid_ok(h, hy, true))
    return fail(h, SFFN_E_ARG, "Hybrid buffers must be non-null and 16-byte aligned");
  const Layout L = layout(h, T, SFFN_OP_BACKWARD);
  if (!ws_ok(ws, ws_bytes, L))
    return fail(h, SFFN_E_ARG, "workspace missing, too small or not 256-byte aligned");
  const Dtype dt = dt_of(h);
  const bool gated = D.gated != 0;
  const int K = D.ell_cap;
  const int Kp = (K + 7) / 8 * 8;
  const int cap = (int)std::min<int64_t>(hy->max_backup, dense_cap(h, T));
  hipError_t e;

  BwdArgs ba = {};
  ba.x = x;
  ba.dy = dy;
  ba.wg = w_gate;
  ba.wu = w_up;
  ba.ell_a = hy->ell_a;
  ba.ell_u = hy->ell_u;
  ba.store_bf16 = sb_of(h);
  ba.ell_idx = hy->ell_idx;
  ba.ell_cnt = hy->ell_cnt;
  ba.slot = hy->slot;
  ba.T = T;
  ba.d = D.d;
  ba.F = D.d_ff;
  ba.K = K;
  ba.Kp = Kp;
  ba.l1 = l1_coeff;
  ba.dpart = at<float>(ws, L.upart);
  ba.drec = at<f32x4_t>(ws, L.drec);
  ba.dx = dx;
  ba.dwg = dw_gate;
  ba.dwu = dw_up;
  ba.dwd = dw_down;
  ba.ncnt = at<int32_t>(ws, L.ncnt);
  ba.noff = at<int32_t>(ws, L.noff);
  ba.thist = at<uint32_t>(ws, L.thist);
  ba.toff = at<int32_t>(ws, L.toff);
  ba.meta = at<f32x4_t>(ws, L.meta);
  ba.brow = hy->brow;
  ba.n_backup = hy->n_backup;
  ba.cap = cap;
  ba.bk_a = hy->bk_a;
  ba.bk_u = hy->bk_u;
  ba.dH = at<float>(ws, L.dH);
  ba.xb = at<char>(ws, L.xb);
  ba.dyb = at<char>(ws, L.dyb);
  ba.gz_rm = at<char>(ws, L.gz_rm);
  if (dt == kBF16) {
    ba.gu_rm = at<char>(ws, L.gz_rm) + (size_t)2 * D.d_ff * 2;
    ba.ld_rm = (int64_t)4 * D.d_ff;
  } else {
    ba.gu_rm = at<char>(ws, L.gz_rm) + (size_t)dense_cap(h, T) * D.d_ff * 4;
    ba.ld_rm = D.d_ff;
  }
  ba.gz_t = at<char>(ws, L.gz_t);
  ba.gu_t = at<char>(ws, L.gu_t);
  ba.gh_t = at<char>(ws, L.gh_t);
  ba.ldt = L.ldt;

  // bf16 with backup rows: their x and dy rows are gathered (transposed)
  // by extra workgroups of the dh launch, and the split-K reduce of their dx
  // product runs in the launch of the ELL rows' dx sums
  const bool joint = dt == kBF16 && cap > 0;

  // 1. dh = dy . W_d[j] per ELL slot, as per-slice partial dot products
  SliceArgs sa = {};
  sa.x = dy;
  sa.wu = w_down;
  sa.ell_idx = hy->ell_idx;
  sa.ell_cnt = hy->ell_cnt;
  sa.T = T;
  sa.d = D.d;
  sa.K = K;
  sa.Kp = Kp;
  sa.upart = at<float>(ws, L.upart);
  {
    ProfScope ps(h, SFFN_K_BWD_SDDMM, stream);
    e = joint ? launch_up_with_gather(dt, sa, gather_args(ba), stream)
              : launch_updown(dt, true, 0, sa, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "backward dh");


  // 2. dZ, dU per slot and dx of the ELL rows
  {
    ProfScope ps(h, SFFN_K_BWD_DX, stream);
    // with backup rows the dx sums of the ELL rows run later, on the
    // second stream beside the dW products
    e = launch_bwd_sparse(dt, gated, cap > 0 ? 2 : 0, ba, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "backward dx");
  // 3. backup rows, densely: dH = dy W_d^T, then dZ/dU, dx rows and their
  // dW products (zeros when no row took the backup path)
  // once work is forked to the second stream, every return below first
  // makes the caller's stream wait for it (event join; a host wait of the
  // second stream if even the join event could not be recorded)
  bool forked = false;
  hipError_t join_rec = hipSuccess;
  auto join_side = [&]() -> hipError_t {
    if (!forked) return hipSuccess;
    forked = false;
    if (join_rec == hipSuccess) return hipStreamWaitEvent(stream, h->join, 0);
    return hipStreamSynchronize(h->side);
  };
  bool transposed = false;
  GemmArgs dx_late = {};   // joint: the backup rows' dx reduce, on the second stream
  if (cap > 0) {
    ProfScope ps(h, SFFN_K_BWD_DENSE, stream);
    const bool split = dt == kBF16;
    float* part = at<float>(ws, L.part);
    if (!joint) e = launch_backup_prep(dt, gated, ba, stream);
    if (e != hipSuccess) return hip_fail(h, e, "backup rows gather");
    GemmArgs g = {};
    g.A = dy;
    g.lda = D.d;
    g.a_rows = hy->brow;
    g.m_dev = hy->n_backup;
    g.m_cap = cap;
    g.B0 = w_down;
    g.ldb = D.d;
    g.N = D.d_ff;
    g.K = D.d;
    g.out = const_cast<float*>(ba.dH);
    g.ldo = D.d_ff;
    g.part = part;
    g.num_cu = h->num_cu;
    if (split) {
      g.split_target = small_split_target(h);
      g.split_max = std::min(kSplitMax, D.d / 32);
      g.grid = gemm_small_grid(h->num_cu);
      e = launch_gemm_small(false, kEpiStoreF32, g, stream);
    } else {
      g.split_target = h->num_cu;
      g.split_max = std::min(kSplitMax, D.d / 32);
      g.grid = gemm_grid(dt, 1, h->num_cu);
      e = launch_gemm(dt, 1, false, kEpiStoreF32, g, stream);
    }
    if (e == hipSuccess) e = launch_splitk_reduce(g, (float*)ba.dH, D.d_ff, stream);
    if (e == hipSuccess) e = launch_backup_grad(dt, gated, ba, stream);
    if (e != hipSuccess) return hip_fail(h, e, "backup dH");
    // dx rows = dZ W_g (+ dU W_u), scattered into the backup rows: bf16 as
    // one product (dZ hi and lo against W_g, then dU hi and lo against W_u),
    // fp32 as two
    for (int pass = 0; pass < (gated && !split ? 2 : 1); ++pass) {
      GemmArgs f = {};
      f.A = pass == 0 ? ba.gz_rm : ba.gu_rm;
      f.lda = ba.ld_rm;
      f.m_dev = hy->n_backup;
      f.m_cap = cap;
      f.B0 = pass == 0 ? w_gate : w_up;
      f.ldb = D.d;
      f.N = D.d;
      if (split) {
        // dual A (hi | lo parts F apart) over the F rows of W_g, then of W_u
        f.K = (gated ? 2 : 1) * D.d_ff;
        f.alo = D.d_ff;
        if (gated) {
          f.B1 = w_up;
          f.kcat = D.d_ff;
        }
      } else {
        f.K = D.d_ff;
      }
      f.out = dx;
      f.ldo = D.d;
      f.out_rows = hy->brow;
      f.accumulate = pass;
      f.part = part;
      f.num_cu = h->num_cu;
      if (split) {
        f.split_target = small_split_target(h);
        f.split_max = std::min(kSplitMax, f.K / 32);
        f.grid = gemm_small_grid(h->num_cu);
        e = launch_gemm_small(true, kEpiStoreF32, f, stream);
      } else {
        f.split_target = h->num_cu;
        f.split_max = std::min(kSplitMax, f.K / 32);
        f.grid = gemm_grid(dt, 1, h->num_cu);
        e = launch_gemm(dt, 1, true, kEpiStoreF32, f, stream);
      }
      if (e == hipSuccess && !joint) e = launch_splitk_reduce(f, dx, D.d, stream);
      if (e != hipSuccess) return hip_fail(h, e, "backup dx");
      if (joint) dx_late = f;
    }
    // the neuron-major grouping (needs only the slot records) on the second
    // stream, beside the dW products
    if (!h->side) {
      e = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&h->fork, hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&h->join, hipEventDisableTiming);
      if (e != hipSuccess) return hip_fail(h, e, "second stream");
    }
    e = hipEventRecord(h->fork, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->fork, 0);
    if (e != hipSuccess) return hip_fail(h, e, "backward fork");
    forked = true;
    {
      ProfScope ps(h, SFFN_K_BWD_DX, h->side);
      e = dx_late.out != nullptr ? launch_dx_with_reduce(dt, gated, ba, dx_late, h->side)
                                 : launch_bwd_sparse(dt, gated, 3, ba, h->side);
    }
    if (e == hipSuccess) {
      ProfScope ps(h, SFFN_K_BWD_TRANSPOSE, h->side);
      e = launch_transpose(ba, h->side);
    }
    join_rec = hipEventRecord(h->join, h->side);
    if (e == hipSuccess) e = join_rec;
    if (e != hipSuccess) {
      (void)join_side();
      return hip_fail(h, e, "backward transpose");
    }
    transposed = true;
    // dW = (dZ, dU, H)^T (x, x, dy) over the backup rows
    for (int pass = 0; pass < 3; ++pass) {
      if (pass == 1 && !gated) continue;
      GemmArgs w = {};
      w.A = pass == 0 ? ba.gz_t : (pass == 1 ? ba.gu_t : ba.gh_t);
      w.lda = L.ldt;
      w.M = D.d_ff;
      // bf16: x and dy rows transposed ([d, ldt], k-contiguous like A);
      // fp32: row-major [Rp, d]
      w.B0 = pass == 2 ? ba.dyb : ba.xb;
      w.ldb = split ? L.ldt : D.d;
      w.N = D.d;
      w.k_dev = hy->n_backup;
      w.k_cap = cap;
      w.k_mult = split ? 2 : 1;
      w.out = pass == 0 ? dw_gate : (pass == 1 ? dw_up : dw_down);
      w.ldo = D.d;
      w.accumulate = 0;
      w.num_cu = h->num_cu;
      w.grid = gemm_grid(dt, 1, h->num_cu);
      e = launch_gemm(dt, 1, !split, kEpiStoreF32, w, stream);
      if (e != hipSuccess) {
        (void)join_side();
        return hip_fail(h, e, "backup dW");
      }
    }
  }
  // 4. slots grouped by neuron in ascending row order (with backup rows it
  //    ran on the second stream beside their dW products: join it here)
  if (transposed) {
    e = join_side();
  } else {
    ProfScope ps(h, SFFN_K_BWD_TRANSPOSE, stream);
    e = launch_transpose(ba, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "backward transpose");
  // 5. dW rows of every neuron from the ELL slots, added to the backup
  // rows' products when there are backup buffers
  {
    ProfScope ps(h, SFFN_K_BWD_DW, stream);
    ba.accumulate = cap > 0;
    e = launch_bwd_sparse(dt, gated, 1, ba, stream);
  }
  if (e != hipSuccess) return hip_fail(h, e, "backward dW");

  return SFFN_OK;
}

// Mean active neurons per token (over the rows that stay sparse) above
// which the dense layer is faster than the sparse one, from a cost model
// of the two paths on MI355X (per token; d model width, F neurons; f the
// fraction of rows whose TwELL overflowed):
//   dense   t_d = (3 gated, 2 non-gated) * 2 d F flop at 1.2 PFLOP/s
//   sparse  2 d F flop (gate GEMM) at 1.1 PFLOP/s + 6 ns (routing, lists,
//           slice sums, launches)
//           + (1 - f) * per active neuron (2 gated, 1 non-gated) * 2 d bytes
//             of weight rows gathered at 27.5 TB/s
//           + f * 2 t_d (overflowing rows on the dense path, whose hidden
//             rows enter the down GEMM as two bf16 parts)
// The GEMM rates are the ones measured here for the gate GEMM and the dense
// layer at d = 2048, F = 5632; the gather rate and the 6 ns are the slope
// and the intercept (less the gate GEMM) of the sparse layer's time against
// its mean active count over the 18 layers of the chained stack (T = 16384,
// 15 to 119 active per token), averaged over two boxes whose measured
// crossovers were about 90 and 105 active per token (the gather rate varies
// more from box to box than the GEMM rates). With f = 0 the model puts the
// crossover at 103 active per token for the gated layer at F = 5632 and at
// 130 for the non-gated one at F = 8192; at the stack's f of about 0.02 the
// gated crossover is 98.
static float model_crossover(const sffn_desc& D, double f) {
  const double dF = (double)D.d * D.d_ff;
  const double t_dense = (D.gated ? 3.0 : 2.0) * 2.0 * dF / 1.2e15;
  const double t_fixed = 2.0 * dF / 1.1e15 + 6e-9 + f * 2.0 * t_dense;
  const double t_pair = (1.0 - f) * (D.gated ? 2.0 : 1.0) * 2.0 * D.d / 27.5e12;
  const double n = t_pair > 0.0 ? (t_dense - t_fixed) / t_pair : 0.0;
  return (float)(n > 0.0 ? n : 0.0);
}

sffn_status sffn_choose_mode(sffn_handle* h, const sffn_twell* tw, int64_t T, int32_t* mode,
                             float* mean_active, float* crossover, hipStream_t stream) {
  if (!h || !mode) return SFFN_E_ARG;
  if (T < 0 || T > (int64_t)1 << 30) return fail(h, SFFN_E_ARG, "T out of range");
  if (T > 0 && !twell_ok(tw))
    return fail(h, SFFN_E_ARG, "TwELL buffers must be non-null and 16-byte aligned");
  double mean = 0.0, f = 0.0;
  if (T > 0) {
    unsigned long long* sum = (unsigned long long*)(h->dstate + 2);
    hipError_t e = launch_zero(sum, 2 * sizeof(*sum), stream);
    if (e == hipSuccess) e = launch_count_sum(tw->cnt, tw->row_flag, T, h->n_t, sum, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    unsigned long long v[2] = {0, 0};
    if (e == hipSuccess) e = hipMemcpy(v, sum, sizeof(v), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(h, e, "active count");
    mean = v[1] > 0 ? (double)v[0] / (double)v[1] : 0.0;
    f = 1.0 - (double)v[1] / (double)T;
  }
  const float cross =
      h->desc.dense_above > 0.0f ? h->desc.dense_above : model_crossover(h->desc, f);
  *mode = mean > cross ? SFFN_DENSE : SFFN_SPARSE;
  if (mean_active) *mean_active = (float)mean;
  if (crossover) *crossover = cross;
  return SFFN_OK;
}

sffn_status sffn_hybrid_check(sffn_handle* h, const sffn_hybrid* hy, hipStream_t stream) {
  if (!h || !hy || !aligned16(hy->n_backup)) return SFFN_E_ARG;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(h, e, "stream");
  int32_t n = 0;
  e = hipMemcpy(&n, hy->n_backup, sizeof(n), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(h, e, "n_backup");
  int64_t cap = hy->max_backup;
  if (h->desc.dense_rows > 0) cap = std::min<int64_t>(cap, h->desc.dense_rows);
  if (n > cap)
    return fail(h, SFFN_E_CAPACITY, "backup rows " + std::to_string(n) + " exceed the capacity " +
                                        std::to_string(cap) + " (max_backup, dense_rows)");
  return SFFN_OK;
}

static void drop_records(sffn_handle* h) {
  for (auto& r : h->recs) {
    h->pool.push_back(r.a);
    h->pool.push_back(r.b);
  }
  h->recs.clear();
}

sffn_status sffn_profile_enable(sffn_handle* h, int32_t enable) {
  if (!h) return SFFN_E_ARG;
  h->prof = enable != 0;
  if (!h->prof) drop_records(h);
  for (int k = 0; k < SFFN_K_COUNT; ++k) {
    h->tot_ms[k] = 0;
    h->launches[k] = 0;
  }
  return SFFN_OK;
}

sffn_status sffn_profile_read(sffn_handle* h, double* total_ms, int32_t* launches, int32_t n) {
  if (!h || n < 0 || (n > 0 && (!total_ms || !launches))) return SFFN_E_ARG;
  sffn_status st = SFFN_OK;
  for (auto& r : h->recs) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) {
      st = hip_fail(h, e, "profile events");
      continue;
    }
    h->tot_ms[r.k] += ms;
    h->launches[r.k] += 1;
  }
  drop_records(h);
  for (int k = 0; k < n; ++k) {
    total_ms[k] = k < SFFN_K_COUNT ? h->tot_ms[k] : 0.0;
    launches[k] = k < SFFN_K_COUNT ? h->launches[k] : 0;
  }
  for (int k = 0; k < SFFN_K_COUNT; ++k) {
    h->tot_ms[k] = 0;
    h->launches[k] = 0;
  }
  return st;
}

const char* sffn_kernel_name(int32_t k) {
  static const char* names[SFFN_K_COUNT] = {
      "gate_gemm_twell", "flags",        "sparse_up",  "flagged_gateup", "flagged_down",
      "splitk_reduce",   "dense_gateup", "dense_down", "pack_twell",     "gate_preact",
      "rows",            "sparse_down",  "bwd_sddmm",  "bwd_dx",         "bwd_transpose",
      "bwd_dw",          "bwd_dense",    "sparse_hsum",  "train_dense_gateup", "train_dense_down",
      "bwd_dense_dh",    "bwd_dense_dx", "bwd_dense_dw", "fused_updown"};
  return (k >= 0 && k < SFFN_K_COUNT) ? names[k] : "";
}

sffn_status sffn_check(sffn_handle* h, hipStream_t stream) {
  if (!h) return SFFN_E_ARG;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(h, e, "stream");
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(h, e, "async");
  int32_t st = 0;
  e = hipMemcpy(&st, h->dstate, sizeof(st), hipMemcpyDeviceToHost);
  if (e == hipSuccess && st != 0) e = hipMemset(h->dstate, 0, sizeof(st));
  if (e != hipSuccess) return hip_fail(h, e, "status");
  if (st != 0)
    return fail(h, SFFN_E_CAPACITY,
                "more rows took the dense path than its capacity (desc.dense_rows, or "
                "max_backup in training); those rows were not computed");
  return SFFN_OK;
}

}  // extern "C"
