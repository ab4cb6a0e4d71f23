/*
 * sffn.h - activation-sparse ReLU feedforward layer for AMD Instinct MI355X
 * (gfx950), C ABI.
 *
 * The layer is the feedforward block of "Sparser, Faster, Lighter
 * Transformer Language Models" (Cetin et al.):
 *
 *   gated      y = (ReLU(x W_g) * (x W_u)) W_d
 *   non-gated  y = ReLU(x W_1) W_2
 *
 * (gist.science explainer, "2. Methodology" B, inference kernels; appendix
 * Table 2 for the gated/non-gated shapes). The sparse forward packs the gate
 * activations into TwELL inside the gate GEMM's epilogue and then runs the
 * up and down projections only over each token's active neurons, without a
 * dense hidden tensor in memory (same section). TwELL is tile-wise ELLPACK:
 * each row's columns are cut into 1-D tiles of W columns and every
 * (row, tile) keeps a fixed-capacity list of (value, column) plus a count
 * ("2. Methodology" A; wispaper blog, "1. TwELL: Tile-wise ELLPACK").
 *
 * Conventions shared by every call:
 *   - Every call returns an sffn_status and never aborts or throws.
 *   - Device memory the library needs per call is the caller's workspace;
 *     its size (sffn_workspace_bytes) follows the sparse work: the ELL
 *     capacity K and the dense path's row capacity R (desc.dense_rows),
 *     never T x F. Data-dependent overflow of R (more rows on the dense
 *     path than it holds) is not an argument error: the dense path's rows
 *     are then not valid, and sffn_check() reports SFFN_E_CAPACITY.
 *   - Argument errors (null or misaligned pointers, bad sizes) are found on
 *     the host before anything is enqueued and return SFFN_E_ARG.
 *   - All device work is ordered on the caller's stream; no call
 *     synchronises the stream except sffn_check() and sffn_hybrid_check().
 *     sffn_backward forks part of its work to a second stream of the handle
 *     (created on first use, default priority) and joins it back through
 *     events before it returns; work enqueued on the caller's stream after
 *     the call sees all of its results.
 *   - Pointers are device pointers unless stated; every array is
 *     caller-owned and must be 16-byte aligned. The library never frees
 *     caller memory.
 *   - A handle is not thread-safe; use one handle per concurrently used
 *     stream.
 *   - T = 0 is a no-op that returns SFFN_OK.
 *   - Layouts (row-major, contiguous):
 *       x, dy        [T, d]            dtype of the descriptor
 *       w_gate, w_up [F, d]            neuron-major (row j = column j of
 *                                      the math d x F matrix, i.e. the
 *                                      nn.Linear weight layout)
 *       w_down       [F, d]            row j = neuron j's output weights
 *                                      (the math F x d matrix as is)
 *       y, dx        [T, d]            float32
 *       z            [T, F]            float32 gate pre-activations
 *   - "active" means strictly z > 0; slots inside a tile ascend by column.
 */
#ifndef SFFN_H
#define SFFN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sffn_status;
#define SFFN_OK             0
#define SFFN_E_ARG         -1  /* null/misaligned pointer, bad size or enum */
#define SFFN_E_UNSUPPORTED -2  /* shape outside the supported set, wrong GPU */
#define SFFN_E_HIP         -3  /* HIP runtime or launch error; see sffn_last_error */
#define SFFN_E_CAPACITY    -4  /* a caller buffer was too small (data dependent) */

/* element type of x, the weights and dy */
#define SFFN_F32  0
#define SFFN_BF16 1

/* forward modes */
#define SFFN_SPARSE 0   /* gate GEMM + TwELL, sparse up/down, dense path for flagged rows */
#define SFFN_DENSE  1   /* plain dense layer: the same library's baseline */

/* operations, for sffn_workspace_bytes */
#define SFFN_OP_PACK           0
#define SFFN_OP_FORWARD_SPARSE 1
#define SFFN_OP_FORWARD_DENSE  2
#define SFFN_OP_HYBRID         3
#define SFFN_OP_FORWARD_TRAIN  4
#define SFFN_OP_BACKWARD       5
#define SFFN_OP_TRAIN_DENSE    6   /* sffn_forward_train_dense */
#define SFFN_OP_BACKWARD_DENSE 7   /* sffn_backward_dense */

typedef struct sffn_handle sffn_handle;

/*
 * Layer descriptor.
 *   d          model width; d % 64 == 0, bf16: d % 512 == 0 and d <= 4096,
 *              f32: d % 256 == 0 and d <= 2048 (SFFN_E_UNSUPPORTED otherwise)
 *   d_ff       F, the number of neurons; F % 128 == 0, F <= 65408 so a
 *              neuron id fits uint16
 *   gated      1 gated, 0 non-gated (w_up unused and must be NULL)
 *   tile       TwELL tile width W; 128 is the one supported width
 *   twell_cap  C, TwELL slots per (row, tile); 1 <= C <= 128
 *   ell_cap    K, the ELL capacity of the sparse path: a row with more
 *              than K active neurons, or with a TwELL tile holding more
 *              than C, takes the dense path (the Hybrid routing rule,
 *              "2. Methodology" A on the gist.science explainer). Training
 *              needs K >= 1. At inference K = 0 means n_t * C (only rows
 *              with an overflowing tile go dense); a K above n_t * C acts
 *              as n_t * C.
 *   dtype      SFFN_BF16 (bf16 inputs, fp32 accumulation) or SFFN_F32
 *              (fp32 inputs and fp32 arithmetic throughout)
 *   store_dtype  SFFN_F32 (0): the stored activations (TwELL values, ELL
 *              a and u, backup rows' a and u) are float32, the accumulator
 *              values. SFFN_BF16 (bf16 layers only): they are bf16, rounded
 *              once (to nearest, ties to even) where they are stored, which
 *              halves the format's value bytes; the layer then computes
 *              with the stored values, H = bf16(a) * bf16(u) (the dense
 *              path's rows too), and the backward reads them, so the
 *              roundings pass gradients unchanged.
 *   dense_above  mean active neurons per token (over the rows that stay
 *              sparse) above which sffn_choose_mode picks the dense layer;
 *              0 = the library's cost model of the two paths on MI355X
 *   updown     how the inference forward runs the up/down projection of
 *              the ELL rows: 0 (default) three launches with the model
 *              width cut into slices that each XCD's L2 holds (per-slice
 *              partial dot products, their sums h = a * u, the down
 *              projection); 1 (bf16 layers) one fused kernel without
 *              slices, u and y kept in registers (the single fused kernel
 *              of "2. Methodology" B on the gist.science explainer). The
 *              training forward always runs the sliced form.
 *   dense_rows R, the most rows one call computes on the dense path
 *              (rows routed away from the ELL at inference, backup rows in
 *              training); the workspace holds R dense rows. 0 means T
 *              (every row may go dense; the workspace then grows as T x F).
 *              More routed rows than R: see sffn_check.
 */
typedef struct sffn_desc {
  int32_t d;
  int32_t d_ff;
  int32_t gated;
  int32_t tile;
  int32_t twell_cap;
  int32_t ell_cap;
  int32_t dtype;
  int32_t dense_rows;
  int32_t store_dtype;
  float   dense_above;
  int32_t updown;
} sffn_desc;

/*
 * TwELL buffers (device, caller-owned). n_t = F / W.
 *   val       [T, n_t, C] float32   slot values, the gate pre-activation
 *                                   z[t, j] (> 0) as accumulated in fp32
 *                                   (bf16 bits, uint16, when
 *                                   desc.store_dtype is SFFN_BF16)
 *   idx       [T, n_t, C] uint16    slot neuron ids j (global)
 *                                   Slots s >= min(cnt, C) of a (row, tile)
 *                                   are not written and hold unspecified
 *                                   values.
 *   cnt       [T, n_t]    int32     true number of positives in the tile
 *                                   (not capped at C)
 *   row_flag  [T]         uint8     1 iff some tile of the row has cnt > C
 *   flagged   [T]         int32     the flagged rows in ascending order;
 *                                   the first *n_flagged entries are valid
 *   n_flagged [1]         int32     number of flagged rows
 * Rows whose tiles all fit (row_flag 0) are stored losslessly; a flagged
 * row keeps its first C slots per tile and the layer computes it densely.
 */
typedef struct sffn_twell {
  void*     val;
  uint16_t* idx;
  int32_t*  cnt;
  uint8_t*  row_flag;
  int32_t*  flagged;
  int32_t*  n_flagged;
} sffn_twell;

/*
 * Hybrid buffers (device, caller-owned): the training-side format of
 * "2. Methodology" A ("Hybrid Format for Training") on the gist.science
 * explainer and "2. The Hybrid Training Algorithm" on the wispaper blog.
 * A row goes to the dense backup iff its total count of positives exceeds
 * K (desc.ell_cap) or one of its TwELL tiles overflowed C; every other row
 * keeps its positives as ELL slots 0..ell_cnt-1 in ascending neuron order.
 *   ell_a      [T, K]   float32  a = z > 0 of each ELL slot
 *   ell_u      [T, K]   float32  u = x . W_u[j] of each ELL slot (gated
 *                                layers; written by sffn_forward_train)
 *              (ell_a, ell_u, bk_a and bk_u hold bf16 bits, uint16,
 *              when desc.store_dtype is SFFN_BF16)
 *   ell_idx    [T, K]   uint16   neuron ids
 *   ell_cnt    [T]      int32    slots used (0 for backup rows)
 *                                (slots >= ell_cnt are unspecified)
 *   slot       [T]      int32    backup slot of the row, -1 for ELL rows
 *   brow       [max_backup] int32  backup rows in ascending order
 *   n_backup   [1]      int32    true number of backup rows (may exceed
 *                                the capacity R' = min(max_backup,
 *                                desc.dense_rows): then the rows from
 *                                slot R' on were not computed and the
 *                                result is invalid; see sffn_hybrid_check)
 *   bk_a       [max_backup, F] float32  ReLU(z) rows of the backup rows
 *   bk_u       [max_backup, F] float32  u rows of the backup rows (gated)
 *   max_backup capacity of brow, bk_a and bk_u in rows
 */
typedef struct sffn_hybrid {
  void*     ell_a;
  void*     ell_u;
  uint16_t* ell_idx;
  int32_t*  ell_cnt;
  int32_t*  slot;
  int32_t*  brow;
  int32_t*  n_backup;
  void*     bk_a;
  void*     bk_u;
  int64_t   max_backup;
} sffn_hybrid;

/* Create a handle for the current HIP device. Validates the descriptor
 * (SFFN_E_ARG / SFFN_E_UNSUPPORTED) before touching the device; returns
 * SFFN_E_UNSUPPORTED when the current device is not gfx950 and SFFN_E_HIP
 * when no device can be queried. Allocates host memory and one block of
 * device memory of about 64 KiB (the handle's status word and counters,
 * zeroed here; freed by sffn_destroy). Per-kernel timing events and the
 * backward's second stream and its two events are created on demand, on
 * the device current at that call. Calls on the handle must be made with
 * the same device current. */
sffn_status sffn_create(const sffn_desc* desc, sffn_handle** out);

/* Destroy a handle (NULL is allowed). */
void sffn_destroy(sffn_handle* h);

/* Text of the last error recorded on the handle ("" if none). The string
 * lives until the next call on the handle. */
const char* sffn_last_error(const sffn_handle* h);

/* Static name of a status code. */
const char* sffn_status_string(sffn_status s);

/* Bytes of device workspace that operation op needs for T tokens. The
 * workspace is caller-allocated, at least 256-byte aligned, and its
 * contents need not be initialised. */
sffn_status sffn_workspace_bytes(const sffn_handle* h, int64_t T, int32_t op,
                                 size_t* bytes);

/* ReLU + TwELL pack of a given pre-activation tensor z [T, F] float32
 * (the format of "2. Methodology" A on the gist.science explainer, here as
 * a stand-alone kernel that reads z). Fills every field of *tw. The result
 * is a pure function of z (bit-exact, deterministic). */
sffn_status sffn_pack_twell(sffn_handle* h, const float* z, int64_t T,
                            const sffn_twell* tw, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Gate pre-activations z = x W_g, [T, F] float32, computed by the same
 * MFMA main loop as the fused gate GEMM of sffn_forward (so packing this z
 * with sffn_pack_twell reproduces the forward's TwELL bit for bit). */
sffn_status sffn_gate_preact(sffn_handle* h, const void* x, const void* w_gate,
                             int64_t T, float* z, hipStream_t stream);

/*
 * Forward pass y [T, d] float32.
 *   mode SFFN_SPARSE: gate GEMM with ReLU + TwELL pack in its epilogue
 *     ("2. Methodology" B: gate projection), then the fused up/down
 *     projection over each unflagged row's active neurons (same section:
 *     fused up/down projection); flagged rows (a tile overflowed C) are
 *     computed by a dense path restricted to those rows, the dense backup
 *     of the Hybrid format used as a safety valve at inference. If tw is
 *     non-NULL the TwELL is written there, else into the workspace.
 *   mode SFFN_DENSE: the plain dense layer with the same kernels' GEMMs;
 *     for bf16 the hidden activations are rounded once to bf16 between the
 *     two GEMMs, as in a standard bf16 feedforward, and W_d is transposed
 *     into the workspace first (both operands of the down GEMM then read
 *     k-contiguous). tw must be NULL.
 * w_up must be NULL iff the layer is non-gated. The workspace must hold
 * sffn_workspace_bytes(op = SFFN_OP_FORWARD_SPARSE or _DENSE).
 * SPARSE: rows whose TwELL overflowed, or with more than K = desc.ell_cap
 * active neurons, take the dense path; when more than desc.dense_rows rows
 * do, the outputs of the dense path's rows are not valid (rows past the
 * capacity are not computed, and the saved pre-activations of overflowing
 * tiles may not all fit), the rows on the ELL path are unaffected, and the
 * next sffn_check returns SFFN_E_CAPACITY.
 */
sffn_status sffn_forward(sffn_handle* h, const void* x, const void* w_gate,
                         const void* w_up, const void* w_down, int64_t T,
                         float* y, const sffn_twell* tw, int32_t mode,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * sffn_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). Same arguments, kernels and
 * results as sffn_forward; the workspace is instead a static device array
 * of the library (128 MiB on each GPU the library runs on, held until the
 * process ends). A call whose sffn_workspace_bytes exceeds 128 MiB
 * returns SFFN_E_ARG before anything is enqueued (at d = 2048, F = 5632,
 * C = 8, K = 64, dense_rows = 512 that is above T = 15815). The
 * call allocates nothing: no hipMalloc, hipFree or event creation
 * (per-kernel timing is skipped for it). The scratch array is shared by
 * every call on a GPU, from every handle: calls that overlap on one GPU
 * (on different streams) race, so the caller orders them. Its contents
 * need no initialisation.
 */
sffn_status sffn_forward_noalloc(sffn_handle* h, const void* x, const void* w_gate,
                                 const void* w_up, const void* w_down, int64_t T, float* y,
                                 const sffn_twell* tw, int32_t mode, hipStream_t stream);

/* TwELL -> Hybrid ("Hybrid Conversion", "2. Methodology" B on the
 * gist.science explainer): routes every row, fills ell_a, ell_idx, ell_cnt,
 * slot, brow and n_backup of *hy from *tw. When z [T, F] float32 is given,
 * the backup rows' bk_a rows are set to ReLU(z) (ell_u and bk_u are not
 * touched). The result is a pure function of the TwELL (and z). */
sffn_status sffn_hybrid_compact(sffn_handle* h, const sffn_twell* tw, const float* z,
                                int64_t T, const sffn_hybrid* hy, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* Training forward: y [T, d] float32 as sffn_forward(SFFN_SPARSE), and the
 * Hybrid of the step saved for sffn_backward: the TwELL of the gate GEMM
 * (into tw, or the workspace when tw is NULL) is converted with ELL
 * capacity K = desc.ell_cap (>= 1); ELL rows' up/down projections run over
 * their slots and save u per slot; backup rows run densely and save their
 * ReLU(z) and u rows in fp32 (backup rows on the matrix cores, sparse rows
 * on the vector units: "2. Methodology" B, training kernels). */
sffn_status sffn_forward_train(sffn_handle* h, const void* x, const void* w_gate,
                               const void* w_up, const void* w_down, int64_t T, float* y,
                               const sffn_twell* tw, const sffn_hybrid* hy, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/*
 * Sparse backward over the Hybrid saved by sffn_forward_train ("2.
 * Methodology" B, training kernels: backpropagation, on the gist.science
 * explainer). With M = 1[z > 0]: dH = dy W_d^T (only where M = 1),
 * dU = dH * a, dZ = dH * u * M + l1_coeff * M (non-gated: dZ = dH * M +
 * l1_coeff * M); dx = dZ W_g^T + dU W_u^T; dW_g = x^T dZ, dW_u = x^T dU,
 * dW_d = (a * u)^T dy (non-gated: a^T dy). ELL rows run over their slots
 * (the slots are regrouped by neuron, in ascending row order, for dW);
 * backup rows run as dense GEMMs. Outputs are overwritten: dx [T, d],
 * dw_gate, dw_up (NULL iff non-gated), dw_down [F, d] neuron-major, all
 * float32; rows of never-active neurons are zero. dy has the descriptor's
 * dtype. The workspace holds min(T, desc.dense_rows) backup rows; rows
 * from slot min(max_backup, desc.dense_rows) on are not processed (the
 * training forward has then already flagged the overflow: see
 * sffn_hybrid_check and sffn_check). T = 0 stores zero weight gradients
 * (no workspace needed). With backup
 * rows the ELL rows' dx sums and the neuron-major regrouping run on the
 * handle's second stream, beside the backup rows' dW products, joined
 * before the dW sums.
 */
sffn_status sffn_backward(sffn_handle* h, const void* x, const void* w_gate, const void* w_up,
                          const void* w_down, const sffn_hybrid* hy, const void* dy, int64_t T,
                          float* dx, float* dw_gate, float* dw_up, float* dw_down, float l1_coeff,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Per-layer choice between the sparse and the dense forward, made from
 * the layer's own TwELL (the pages attribute the speed-up to each layer's
 * activation sparsity, which differs from layer to layer: listing page,
 * Figure 6 and Figures 10-11; at 108 active per token the gain is small,
 * Table 5). Reads the counts and row flags of *tw (T rows, as a sparse
 * forward of the layer wrote them), synchronises the stream and sets *mode
 * to SFFN_DENSE when the mean active neurons per token over the rows whose
 * TwELL did not overflow exceeds the crossover (desc.dense_above, or when
 * that is 0 the library's cost model of the two paths on MI355X, which
 * also counts the overflowing rows' dense-path work), else SFFN_SPARSE.
 * mean_active and crossover (nullable) receive the two numbers. T = 0
 * gives SFFN_SPARSE. */
sffn_status sffn_choose_mode(sffn_handle* h, const sffn_twell* tw, int64_t T, int32_t* mode,
                             float* mean_active, float* crossover, hipStream_t stream);

/*
 * The same library's dense training step of the layer, the comparator of
 * the sparse step (sffn_forward_train + sffn_backward): a standard bf16
 * layer that keeps its hidden activations dense (listing page, Table 1:
 * training step of the dense models; gist.science explainer, "2.
 * Methodology" B for the layer and its backpropagation). bf16 layers only,
 * T a multiple of 64 (SFFN_E_UNSUPPORTED otherwise).
 * Forward: Z_s = bf16(x W_g), U_s = bf16(x W_u) (gated), H =
 * bf16(ReLU(Z_s) U_s) (non-gated: ReLU(Z_s)), y = H W_d (float32 [T, d]).
 * act (caller-owned, sffn_train_dense_act_bytes) receives Z_s [T, F], U_s
 * [T, F] (gated) and H [T, F], all bf16: the saved activations the
 * backward reads. The workspace is sffn_workspace_bytes(
 * SFFN_OP_TRAIN_DENSE) (W_d transposed, F x d bf16: both operands of the
 * down GEMM k-contiguous).
 */
sffn_status sffn_train_dense_act_bytes(const sffn_handle* h, int64_t T, size_t* bytes);
sffn_status sffn_forward_train_dense(sffn_handle* h, const void* x, const void* w_gate,
                                     const void* w_up, const void* w_down, int64_t T, float* y,
                                     void* act, void* ws, size_t ws_bytes, hipStream_t stream);
/* Backward of sffn_forward_train_dense from its act: with M = 1[Z_s > 0],
 * dH = dy W_d^T; dZ = bf16(dH U_s M + l1_coeff M) (non-gated: dH M +
 * l1_coeff M); dU = bf16(dH ReLU(Z_s)); dx = dZ W_g^T + dU W_u^T;
 * dW_g = x^T dZ, dW_u = x^T dU, dW_d = H^T dy. Outputs float32 and
 * overwritten, dW neuron-major [F, d] as in sffn_backward. The workspace is
 * sffn_workspace_bytes(SFFN_OP_BACKWARD_DENSE) (dH [T, F] fp32, dZ | dU
 * [T, 2F] and dZ, dU, H transposed, and W_g | W_u, x and dy transposed,
 * bf16). T = 0 stores zero weight gradients. */
sffn_status sffn_backward_dense(sffn_handle* h, const void* x, const void* w_gate,
                                const void* w_up, const void* w_down, const void* act,
                                const void* dy, int64_t T, float* dx, float* dw_gate,
                                float* dw_up, float* dw_down, float l1_coeff, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* Synchronise the stream and return SFFN_E_CAPACITY when *hy->n_backup
 * exceeds hy->max_backup or desc.dense_rows (when that is set), else
 * SFFN_OK (or SFFN_E_HIP). */
sffn_status sffn_hybrid_check(sffn_handle* h, const sffn_hybrid* hy, hipStream_t stream);

/* Synchronise the stream and report the first asynchronous error since
 * the last check (SFFN_E_HIP); else SFFN_E_CAPACITY when a call since the
 * last check routed more rows to the dense path than it could hold
 * (desc.dense_rows, or max_backup in training), so that some rows were not
 * computed; else SFFN_OK. The capacity report is cleared by the check. */
sffn_status sffn_check(sffn_handle* h, hipStream_t stream);

/*
 * Per-kernel timing. While enabled, every kernel launch of the library is
 * bracketed by two HIP events recorded on the call's stream, so that each
 * interval holds one kernel id's launches alone. sffn_profile_read waits
 * for the recorded events, writes for each kernel id k < n the summed
 * milliseconds and the
 * number of launches since the last read (or since enabling), and resets
 * the sums. Disabling drops pending records. Kernel ids:
 */
#define SFFN_K_GATE_TWELL    0  /* gate GEMM with the ReLU + TwELL epilogue */
#define SFFN_K_FLAGS         1  /* overflow flags and flagged-row list */
#define SFFN_K_SPARSE_UP     2  /* sparse up projection: per-slice partial dots */
#define SFFN_K_FLAG_GATEUP   3  /* hidden rows of the dense path: bf16 up GEMM + combine
                                    from the gate's own outputs, fp32 gate/up GEMM + combine */
#define SFFN_K_FLAG_DOWN     4  /* down GEMM of the flagged rows (split-K) */
#define SFFN_K_SPLITK_REDUCE 5  /* split-K reduction into the flagged rows */
#define SFFN_K_DENSE_GATEUP  6  /* dense mode: gate/up GEMM */
#define SFFN_K_DENSE_DOWN    7  /* dense mode: down GEMM */
#define SFFN_K_PACK          8  /* stand-alone TwELL pack */
#define SFFN_K_GATE_PREACT   9  /* gate GEMM writing z */
#define SFFN_K_ROWS         10  /* per-row route + ELL compaction of the TwELL */
#define SFFN_K_SPARSE_DOWN  11  /* sparse down projection into y */
#define SFFN_K_BWD_SDDMM    12  /* backward: dy . W_d[j] per ELL slot (partial dots) */
#define SFFN_K_BWD_DX       13  /* backward: dZ, dU per slot and dx of ELL rows */
#define SFFN_K_BWD_TRANSPOSE 14 /* backward: ELL slots grouped by neuron */
#define SFFN_K_BWD_DW       15  /* backward: dW rows from the ELL slots */
#define SFFN_K_BWD_DENSE    16  /* backward: the backup rows' dense GEMMs */
#define SFFN_K_SPARSE_HSUM  17  /* sparse up projection: slice partials summed, h = a * u */
#define SFFN_K_TRAIN_DENSE_GATEUP 18  /* dense training step: gate/up GEMM saving Z, U, H^T */
#define SFFN_K_TRAIN_DENSE_DOWN   19  /* dense training step: down GEMM */
#define SFFN_K_BWD_DENSE_DH       20  /* dense backward: dH GEMM forming dZ, dU */
#define SFFN_K_BWD_DENSE_DX       21  /* dense backward: dx GEMMs */
#define SFFN_K_BWD_DENSE_DW       22  /* dense backward: dW GEMMs */
#define SFFN_K_FUSED_UPDOWN       23  /* inference up/down in one kernel (desc.updown = 1) */
#define SFFN_K_COUNT        24
sffn_status sffn_profile_enable(sffn_handle* h, int32_t enable);
sffn_status sffn_profile_read(sffn_handle* h, double* total_ms, int32_t* launches, int32_t n);
/* Static name of a kernel id ("" if out of range). */
const char* sffn_kernel_name(int32_t k);

#ifdef __cplusplus
}
#endif

#endif /* SFFN_H */
