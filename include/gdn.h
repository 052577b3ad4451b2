/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule library (libgdn.so).
 *
 * The operation (mlx-lm PR "Add gated_delta_update VJP -- trainable
 * GatedDeltaNet on Apple Silicon", section "What this PR adds": a drop-in
 * gated_delta_update_vjp(q, k, v, a, b, A_log, dt_bias, state, mask) with a
 * VJP for every primal argument; torch-to-nnef GDN page, "Op contract": the
 * tensor layouts, GQA head mapping and q/k normalisation):
 *
 *   value head h reads query/key head j = h / G, G = Hv / Hk;
 *   qn = q / sqrt(|q|^2 + 1e-6) / sqrt(Dk),  kn = k / sqrt(|k|^2 + 1e-6);
 *   x = a + dt_bias[h],  l = -exp(A_log[h]) * softplus(min(x, 20)),
 *   g = exp(l),  beta = sigmoid(b);
 *   valid step:  S <- g S;  delta = beta (v - S^T kn);  S <- S + kn delta^T;
 *   every step:  o = S^T qn   (a masked step leaves S unchanged).
 *
 * S is the per-(batch, value head) state, Dk x Dv, fp32.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers to dense row-major tensors with
 *    the layouts given below.  The caller owns all memory: the library never
 *    allocates or frees device memory and keeps no state between calls
 *    (apart from the optional timing events of gdn_set_kernel_events, kept
 *    per host thread, and the static workspace array of gdn_fwd_noalloc).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream): they validate, enqueue kernels and return.  No host sync.
 *  - All arguments are validated before anything is enqueued; on a non-zero
 *    return nothing was enqueued (except GDN_ERR_HIP, where a launch failed).
 *  - q, k, v, a, b, o, dO, dq, dk, dv, da, db use `dtype`; A_log, dt_bias,
 *    the states, the checkpoints, dstate, dA_log and ddt_bias are fp32.
 *  - NaN / Inf inputs propagate; nothing traps.
 *  - Results are deterministic: repeated calls with the same inputs produce
 *    identical bits (no atomics; every sum runs in a fixed order).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Steps per state checkpoint (PR, "Why chunked instead of single-shot?":
 * CHUNK_SIZE = 64). */
#define GDN_CHUNK 64

enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* bad dims, NULL required pointer, bad alias   */
  GDN_ERR_UNSUPPORTED = 2, /* Dk / Dv / dtype / algo not built             */
  GDN_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required      */
  GDN_ERR_HIP = 4          /* a HIP launch failed                          */
};

enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 };

/* Kernel family.
 *   SCAN   the per-step recurrence in fp32 (every dtype and supported size).
 *   CHUNK  the chunked matrix form over 64-step chunks: bf16 matrix-core
 *          products with fp32 accumulation and an fp32 state carried between
 *          chunks.  Built for dtype bf16, Dk in {64, 128, 192, 256} and Dv a
 *          multiple of 32 up to 256, and only while its per-chunk tensors
 *          stay below 4 GiB each: B * Hv * ceil(T/64) * 8192 bytes (the 64 x 64
 *          bf16 chunk matrices) and B * Hk * ceil(T/64) * Dk * 128 bytes (the
 *          transposed k / q rows).  Other shapes return GDN_ERR_UNSUPPORTED
 *          (AUTO runs SCAN for them).
 *          Its results agree with SCAN to bf16 rounding (about 1e-2 relative,
 *          normwise), not bitwise.
 *   AUTO   CHUNK where it is built and T > 1, else SCAN; the CHUNK forward
 *          runs T-parallel (as CHUNK_TPAR) where that pays.
 * Both produce the same checkpoint layout, so a checkpoint from one can be
 * used by the other (with save unset; see gdn_ckpt_elems). */
/*   CHUNK_TPAR  the CHUNK family with a T-parallel forward (mlx-lm PR,
 *          "Associative prefix-scan scaffold": each step, and so each chunk,
 *          is an affine map of the state, and maps compose associatively).
 *          The chunks are grouped into segments; each segment's composed map
 *          [A | B] (A: Dk x Dk, B: Dk x Dv) is computed in parallel over the
 *          segments, a short fp32 chain over the segment maps gives every
 *          segment's start state, and the segments then run their outputs in
 *          parallel.  This pays when B * Hv * Dv / 32 is small against the
 *          GPU's 256 compute units and T is long (a long single sequence with
 *          few heads); the library picks the segment count from the sizes and
 *          falls back to CHUNK's single pass when one segment is best.  Same
 *          sizes, checkpoints and saved record as CHUNK; gdn_bwd runs CHUNK.
 *          Results agree with CHUNK to bf16 rounding, not bitwise. */
enum gdn_algo { GDN_ALGO_AUTO = 0, GDN_ALGO_SCAN = 1, GDN_ALGO_CHUNK = 2, GDN_ALGO_CHUNK_TPAR = 3 };

typedef struct gdn_dims {
  int64_t B, T, Hk, Hv, Dk, Dv; /* T >= 0; Hv % Hk == 0                     */
  int32_t dtype;                /* enum gdn_dtype                           */
  int32_t algo;                 /* enum gdn_algo                            */
  int32_t save;                 /* CHUNK family only: nonzero = the checkpoint
                                   buffer becomes the library's own record of
                                   what gdn_bwd needs -- the chunk-start
                                   states in bf16 and the chunk matrices --
                                   written by gdn_fwd so that gdn_bwd neither
                                   recomputes nor converts anything (see
                                   gdn_ckpt_elems).  Ignored by SCAN.        */
} gdn_dims;

/* Supported sizes: Dk in {16, 32, 64, 128, 192, 256}; Dv a multiple of 8
 * with Dv <= 256 and (Dv <= 24 or Dv % 32 == 0). */

/* Number of fp32 elements of the checkpoint buffer:
 * (ceil(T/64) - 1) * B * Hv * Dk * Dv  (0 when T <= 64), the fp32 states at
 * steps 64, 128, ... in the layout given at gdn_fwd.
 * When d->save is set and the call runs the CHUNK family, instead a buffer
 * whose contents are private to the library: the state at the start of every
 * chunk (initial state included) rounded to bf16, which is the precision the
 * chunk products consume it in, and the per-chunk matrices the backward needs
 * (the in-chunk inverse, the decayed query/key Gram matrix, the chunk's q rows
 * transposed, the per-step chunk scalars) and every step's X = v - u (the
 * value minus the state's prediction of it, bf16), which spares the backward
 * its recomputation:
 * about ceil(T/64) * (B * Hv * (Dk * Dv / 2 + 32 * Dv + 4864) + B * Hk * Dk * 32)
 * elements.  It holds no fp32 states; such a checkpoint is read only by a
 * gdn_bwd with the same dims (including save). */
int gdn_ckpt_elems(const gdn_dims* d, size_t* out);
/* The same in bytes (gdn_ckpt_elems * 4). */
int gdn_ckpt_bytes(const gdn_dims* d, size_t* out);

/* Device workspace bytes needed by gdn_fwd / gdn_bwd for these dims (less
 * with d->save set, which moves the chunk matrices and the bf16 states into
 * the checkpoint buffer). */
int gdn_fwd_workspace_bytes(const gdn_dims* d, size_t* out);
int gdn_bwd_workspace_bytes(const gdn_dims* d, size_t* out);
/* Either of the two: for_bwd = 0 the forward's, nonzero the backward's. */
int gdn_workspace_bytes(const gdn_dims* d, int for_bwd, size_t* out);

/*
 * Forward scan.
 *   q, k     [B,T,Hk,Dk] dtype        v  [B,T,Hv,Dv] dtype
 *   a, b     [B,T,Hv]    dtype        A_log, dt_bias [Hv] fp32
 *   state0   [B,Hv,Dk,Dv] fp32, NULL = zeros
 *   mask     [B,T] uint8, nonzero = valid step; NULL = all valid
 *   o        [B,T,Hv,Dv] dtype (out)
 *   state_out[B,Hv,Dk,Dv] fp32 (out); may alias state0 exactly (in-place
 *            update; such a call runs the single-pass forward, never the
 *            T-parallel one); no other overlap between outputs and inputs is
 *            allowed
 *   ckpt     [ceil(T/64)-1, B,Hv,Dk,Dv] fp32 (out): ckpt[c-1] = state before
 *            step 64c; when d->save applies, the library's own record
 *            instead (gdn_ckpt_elems elements).  NULL = not written
 *            (inference; GDN_ERR_INVALID_ARG when save applies).  Required
 *            by gdn_bwd.
 *   ws       device workspace of at least gdn_fwd_workspace_bytes()
 */
int gdn_fwd(const gdn_dims* d, const void* q, const void* k, const void* v,
            const void* a, const void* b, const float* A_log,
            const float* dt_bias, const float* state0, const uint8_t* mask,
            void* o, float* state_out, float* ckpt, void* ws, size_t ws_bytes,
            void* stream);

/*
 * gdn_fwd for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments, results and errors as gdn_fwd without ws / ws_bytes:
 * the workspace is a static device array inside the library, one copy per GPU,
 * of GDN_NOALLOC_SCRATCH_BYTES, held until the process ends.  A call whose
 * workspace (gdn_fwd_workspace_bytes, or the single pass's when state_out ==
 * state0) exceeds it returns GDN_ERR_WORKSPACE before anything is enqueued.
 * The call uses the copy of the current device (hipGetDevice), so `stream`
 * must belong to that device; the first call on a device looks the copy up
 * (GDN_ERR_HIP if that fails).  Nothing is allocated or freed.  Every call on
 * one GPU shares that GPU's copy: calls that overlap in time on one GPU (on
 * different streams, or from different host threads without ordering) race
 * on it; calls ordered on one stream do not.  Each call writes every
 * workspace location it reads, so no state carries over between calls.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)
int gdn_fwd_noalloc(const gdn_dims* d, const void* q, const void* k, const void* v,
                    const void* a, const void* b, const float* A_log,
                    const float* dt_bias, const float* state0, const uint8_t* mask,
                    void* o, float* state_out, float* ckpt, void* stream);

/*
 * VJP of gdn_fwd (reverse sweep; PR "Design notes": chunk-wise recompute from
 * the checkpoints, deterministic reductions without atomics).
 *   q ... mask    the inputs given to gdn_fwd (same values)
 *   ckpt          the checkpoints gdn_fwd wrote for those inputs (may be NULL
 *                 only when T <= 64 and save is unset)
 *   dO            [B,T,Hv,Dv] dtype, cotangent of o
 *   dS_final      [B,Hv,Dk,Dv] fp32, cotangent of state_out; NULL = zeros
 *   dq, dk        [B,T,Hk,Dk] dtype (out)     dv [B,T,Hv,Dv] dtype (out)
 *   da, db        [B,T,Hv] dtype (out)        dA_log, ddt_bias [Hv] fp32 (out)
 *   dstate        [B,Hv,Dk,Dv] fp32 (out), cotangent of state0
 * Gradients are overwritten, not accumulated.  The mask gets no gradient;
 * masked steps get dv = da = db = 0.
 */
int gdn_bwd(const gdn_dims* d, const void* q, const void* k, const void* v,
            const void* a, const void* b, const float* A_log,
            const float* dt_bias, const float* state0, const uint8_t* mask,
            const float* ckpt, const void* dO, const float* dS_final, void* dq,
            void* dk, void* dv, void* da, void* db, float* dA_log,
            float* ddt_bias, float* dstate, void* ws, size_t ws_bytes,
            void* stream);

/*
 * One decode step (T = 1) preceded by the depthwise causal conv1d + SiLU
 * update of the token's mixed projection (torch-to-nnef GDN page, the
 * causal-conv-update drop-in: hidden_states [b, C, S], conv_state [b, C, k],
 * weight [C, k] -> out, final_state; mlx-lm PR, "Extension 2 -- Inference
 * kernel fusion": the T = 1 steps fused into one kernel), in one kernel.
 *   d         dims with T == 1 (else GDN_ERR_INVALID_ARG); algo and save are
 *             ignored; Dk, Dv as for the decode kernel (Dk in {16, 32, 64,
 *             128, 192, 256}, Dv a multiple of 32 up to 256), else
 *             GDN_ERR_UNSUPPORTED
 *   x         [B, C] dtype, C = 2 Hk Dk + Hv Dv: the token's projection before
 *             the conv, channels q (Hk heads of Dk), then k, then v (Hv heads
 *             of Dv), each head-major
 *   conv_w    [C, conv_k] dtype: taps, oldest sample first
 *   conv_state[B, C, conv_k] dtype: the conv_k carried samples, oldest first
 *   conv_state_out [B, C, conv_k] dtype (out): the carried samples shifted by
 *             one with x appended; may alias conv_state exactly (in place)
 *   conv_k    taps, 1 .. 8 (else GDN_ERR_INVALID_ARG)
 *   a, b, A_log, dt_bias, state0, mask, o, state_out: as gdn_fwd with T = 1
 *             (state_out may alias state0 exactly)
 * Per channel, out_c = SiLU(sum_i conv_w[c][i] w_i) over the window w of the
 * conv_k newest samples (the newest conv_k - 1 carried ones, then x); q, k, v
 * are those outputs, kept in fp32, and the step is gdn_fwd's.  A masked batch
 * row (mask[b] == 0) keeps both its carried samples and its state (its o is
 * still read from the state).  No workspace.
 */
int gdn_decode_conv(const gdn_dims* d, const void* x, const void* conv_w, const void* conv_state,
                    void* conv_state_out, int32_t conv_k, const void* a, const void* b,
                    const float* A_log, const float* dt_bias, const float* state0,
                    const uint8_t* mask, void* o, float* state_out, void* stream);

/*
 * Per-key-channel gate (mlx-lm VJP PR, "Models covered" and "Scope and
 * follow-ups": Kimi-Linear runs the same rule with a gate that holds one
 * value per key channel, g.ndim == 4).  The gate of step t and value head h
 * is a vector g in R^Dk that scales the rows of the state:
 *   S' = diag(g) S;  u = S'^T kn;  delta = beta (v - u);  S = S' + kn delta^T;
 *   o = S^T qn,
 * with kn, qn, beta = sigmoid(b) and masking as in gdn_fwd.  The pages give
 * no formula that produces g, so the caller passes its logarithm directly
 * (as the torch-to-nnef op contract passes a log-decay):
 *   lg        [B,T,Hv,Dk] fp32, lg = log g (finite; -inf is not allowed)
 * Kernel families: SCAN (fp32 per-step scan, every size gdn_fwd's scan
 * takes) and CHUNK (the chunked bf16 matrix-core form, with the decays
 * e^{G_t - G_s} of the in-chunk cumulative log-gates taken per channel inside
 * the chunk products: bf16 I/O, Dk 64, 128 or 192, Dv a multiple of 32 up to
 * 128, the per-(head, chunk) buffers below 4 GiB).  AUTO takes CHUNK where it
 * is built and T > 1, else SCAN; CHUNK_TPAR gives GDN_ERR_UNSUPPORTED.  The
 * chunk form is exact (up to rounding) while every in-chunk factor
 * e^{|G_t - G_s|} stays within fp32 range, which holds for any lg <= 0 (a
 * decay); for growing gates (lg > 0) use SCAN.  Sizes and dtypes as
 * gdn_fwd.  Without save, ckpt has gdn_fwd's layout without save (the fp32
 * states at the chunk boundaries) in both families, so a forward of either
 * family pairs with a backward of either.  With d->save set and the call on
 * CHUNK, ckpt is instead the library's own record, written by gdn_fwd_vg:
 * the state at every chunk start (the initial state included) rounded to
 * bf16, the precision the gradient products take it in, and what the
 * backward would otherwise recompute (the per-channel decayed k rows and their
 * transposes, the chunk inverse and Gram matrices, the chunk scalars, and X =
 * v - u of every step in bf16).  It holds no fp32 states; such a record is
 * read only by a gdn_bwd_vg with the same dims
 * (including save), and ckpt may then not be NULL in either call
 * (GDN_ERR_INVALID_ARG).  SCAN ignores save.  The sizes of ckpt and of the
 * workspaces come from the _vg queries (they depend on the family and save).
 */
/* Number of fp32 elements of gdn_fwd_vg's checkpoint buffer: as
 * gdn_ckpt_elems without save, or with d->save set on CHUNK the record's size,
 * about ceil(T/64) * B * Hv * (Dk * Dv / 2 + 128 Dk + 6k + 512) + B * T * Hv *
 * Dv / 2.  gdn_vg_ckpt_bytes: the same in bytes. */
int gdn_vg_ckpt_elems(const gdn_dims* d, size_t* out);
int gdn_vg_ckpt_bytes(const gdn_dims* d, size_t* out);
int gdn_fwd_vg_workspace_bytes(const gdn_dims* d, size_t* out);
int gdn_bwd_vg_workspace_bytes(const gdn_dims* d, size_t* out);

/* Forward with the per-key-channel gate.  Arguments as gdn_fwd, with lg in
 * place of a, A_log, dt_bias. */
int gdn_fwd_vg(const gdn_dims* d, const void* q, const void* k, const void* v, const float* lg,
               const void* b, const float* state0, const uint8_t* mask, void* o,
               float* state_out, float* ckpt, void* ws, size_t ws_bytes, void* stream);

/* VJP of gdn_fwd_vg.  Arguments as gdn_bwd, with lg in place of a, A_log,
 * dt_bias, and
 *   dlg       [B,T,Hv,Dk] fp32 (out), the cotangent of lg
 * in place of da, dA_log, ddt_bias.  Masked steps get dv = dlg = db = 0.
 * Deterministic: every sum runs in a fixed order. */
int gdn_bwd_vg(const gdn_dims* d, const void* q, const void* k, const void* v, const float* lg,
               const void* b, const float* state0, const uint8_t* mask, const float* ckpt,
               const void* dO, const float* dS_final, void* dq, void* dk, void* dv, float* dlg,
               void* db, float* dstate, void* ws, size_t ws_bytes, void* stream);

/*
 * Optional per-kernel timing, for benchmarks and profilers.  While `events`
 * is non-NULL, each kernel that the following gdn_fwd / gdn_bwd calls launch
 * (in launch order, i = 0, 1, ...) records events[2i] on the call's stream
 * just before it and events[2i+1] just after it, for as long as 2i+1 < n;
 * later kernels are not timed.  Each call of this function restarts the count
 * at i = 0.  events are hipEvent_t handles created (and destroyed) by the
 * caller.  NULL turns timing off.  The setting belongs to the calling host
 * thread: it applies to the gdn_fwd / gdn_bwd calls that thread makes, and
 * other threads are not affected.  Returns GDN_ERR_INVALID_ARG if events is
 * non-NULL and n < 2.
 */
int gdn_set_kernel_events(void* const* events, int n);

/* Static description of a status code. */
const char* gdn_status_string(int status);

/* Library version string. */
const char* gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
