// Host-side interfaces between the C ABI (gdn_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct bf16;

struct Dims {
  int B, T, Hk, Hv, Dk, Dv;
  __host__ __device__ int G() const { return Hv / Hk; }
  __host__ __device__ int nchunk() const { return (T + 63) / 64; }
};

// Per-step scalars produced by the prep kernel (fp32, in the workspace).
struct StepScalars {
  float* rq;   // [B,T,Hk]  (|q|^2 + eps)^-1/2 / sqrt(Dk)
  float* rk;   // [B,T,Hk]  (|k|^2 + eps)^-1/2
  float* kq;   // [B,T,Hk]  kn . qn
  float* ell;  // [B,T,Hv]  log gate (0 on masked steps)
  float* beta; // [B,T,Hv]  write strength (0 on masked steps)
};

struct PrepArgs {
  Dims d;
  const void *q, *k, *a, *b;
  const float *A_log, *dt_bias;
  const uint8_t* mask;
  StepScalars s;
};

struct ScanFwdArgs {
  Dims d;
  const void *q, *k, *v;
  const float* state0;  // may be null
  StepScalars s;
  void* o;
  float* state_out;
  float* ckpt;  // may be null
  // Per-key-channel gate: log-gates [B,T,Hv,Dk] fp32 (null = the scalar gate
  // s.ell) and the mask they need (a masked step has gate 1).
  const float* lg;
  const uint8_t* mask;
};

// Sweep of the backward: recompute each chunk from its checkpoint, then walk
// it in reverse carrying dL/dS.  Writes the per-step column quantities and the
// per-chunk boundary gradients used by the chunk-gradient kernel.
struct ScanBwdArgs {
  Dims d;
  const void *q, *k, *v, *dO;
  const float *state0, *ckpt, *dS_final;  // state0/dS_final may be null
  StepScalars s;
  float* U;       // [B,T,Hv,Dv]  u  = S'^T kn (read of the decayed state)
  float* E;       // [B,T,Hv,Dv]  Din^T kn (dL/d delta minus its own-step term)
  void* dv;       // [B,T,Hv,Dv]  dtype
  float* dHend;   // [NC,B,Hv,Dk,Dv] dL/d(state at the end of chunk c)
  float* dstate;  // [B,Hv,Dk,Dv]
};

// Reverse sweep with a per-key-channel gate (log-gates lg [B,T,Hv,Dk]).
struct ScanBwdVgArgs {
  Dims d;
  const void *q, *k, *v, *dO;
  const float* lg;
  const uint8_t* mask;
  const float *state0, *ckpt, *dS_final;  // state0 / dS_final may be null
  StepScalars s;                          // rq, rk, beta (ell unused)
  float* sub;     // sub-checkpoints, vg_sub_floats(d)
  float* part;    // [B,T,Hv,nslice,3,Dk] row partials of dqn, dkn, dlg per column slice
  float* pdb;     // [B,T,Hv,nslice] partials of dL/dbeta
  void* dv;       // [B,T,Hv,Dv] dtype
  float* dstate;  // [B,Hv,Dk,Dv]
};
struct VgReduceArgs {
  Dims d;
  int nslice;
  const void *q, *k;
  StepScalars s;
  const float *part, *pdb;
  void *dq, *dk, *db;  // dtype
  float* dlg;          // [B,T,Hv,Dk]
};
// Lane rows of the per-channel-gate sweep (rows l + 64 m, m < vg_rows).
inline int vg_rows(int Dk) { return Dk <= 64 ? 1 : Dk / 64; }
// Sub-checkpoint floats: every 4 steps, the states of all (b, h) (rows padded
// to 64 vg_rows).
inline size_t vg_sub_floats(const Dims& d) {
  return static_cast<size_t>(d.B) * d.Hv * d.Dv * vg_rows(d.Dk) * 64 * (64 / 4);
}

struct ChunkGradArgs {
  Dims d;
  const void *q, *k, *v, *dO, *a;
  const float *A_log, *dt_bias;
  const uint8_t* mask;
  const float *state0, *ckpt;
  StepScalars s;
  const float *U, *E, *dHend;
  void *dq, *dk, *da, *db;
  double* part_dA;   // [B,NC,Hv] per-chunk sums of dl * l
  double* part_ddt;  // [B,NC,Hv] per-chunk sums of da
};

// Chunk-form intermediates (bf16, in the workspace).  L = 64 rows per chunk,
// rows past the end of the sequence are zero.
struct ChunkBufs {
  bf16* Tx;   // [B*Hv, NC, L, L] (I + N)^-1, N[t,s] = [s<t] e^{g_t-g_s} rk_t rk_s beta_s (k_t.k_s)
  bf16* Mq;   // [B*Hv, NC, L, L] [s<=t] e^{g_t-g_s} rq_t rk_s beta_s (q_t.k_s)
  // backward only
  bf16* PqT;  // [B*Hv, NC, L, L] transpose of [s<=t] e^{g_t-g_s} rq_t rk_s (q_t.k_s)
  bf16* QT;   // [B*Hk, NC, Dk, L] raw q of the chunk, transposed
  // per-step chunk scalars, fp32 [B*Hv, NC, SC_ROWS, L]
  float* sc;
  // [NC, B*Hv, Dk, Dv] the state at the start of chunk c, bf16 (the operand
  // precision of the chunk products); written by chunk_fwd when non-null
  bf16* Hb;
  // [B, T, Hv, Dv] X_t = v_t - u_t of every step, bf16 (the precision of the
  // chunk products): written by chunk_fwd and read by chunk_bwd_grad in place
  // of recomputing it, when non-null
  bf16* X;
  // Per-key-channel gate (vg_chunk_prep), per value head, with G_t the
  // in-chunk cumulative log-gate vector (G_t = lg_0 + ... + lg_t, masked
  // steps 0) and rows past the end of the sequence zero:
  bf16* Kb;   // [B*Hv, NC, L, Dk] kn_t * e^{G_t}
  bf16* Kh;   // [B*Hv, NC, L, Dk] kn_t * e^{G_L - G_t}
  bf16* Qb;   // [B*Hv, NC, L, Dk] qn_t * e^{G_t} / sqrt(Dk)  (forward)
  bf16* KbT;  // [B*Hv, NC, Dk, L] Kb transposed              (backward)
  bf16* QbT;  // [B*Hv, NC, Dk, L] Qb transposed              (backward)
  float* vsc; // [B*Hv, NC, VSC_ROWS, L] beta_t (row 0), e^{G_L} (rows 1.., Dk values)
};
// Rows of ChunkBufs::vsc.
enum : int { VSC_BETA = 0, VSC_EGL = 1, VSC_ROWS = 8 };
// Rows of ChunkBufs::sc (per chunk, per step t; g = gamma):
enum : int {
  SC_CR = 0,     // e^{g_t} rk_t
  SC_CO = 1,     // e^{g_t} rq_t
  SC_W = 2,      // beta_t e^{g_L - g_t} rk_t
  SC_EGL = 3,    // [0] = e^{g_L}   (rows 0..3: what the forward state pass reads)
  SC_KL = 4,     // e^{g_L - g_t} rk_t
  SC_BETA = 5,   // beta_t
  SC_GAM = 6,    // g_t
  SC_EG = 7,     // e^{g_t}
  SC_EL = 8,     // e^{g_L - g_t}
  SC_RK = 9,     // rk_t  (k norm factor)
  SC_RQ = 10,    // rq_t  (q norm factor, with 1/sqrt(Dk))
  SC_ELL = 11,   // l_t   (log gate; 0 on masked steps)
  SC_ROWS = 12
};

// Block index -> (b, h, slice).  Blocks of one (batch, key head) group go to
// one XCD when the group count is a multiple of the XCD count (8); workgroups
// are dealt to the XCDs round-robin in launch order.
// The scalar-gate chunk form's bf16 hand-off from the state passes to the
// gradient pass (the chunk-start states and dH', each a Dk x Dv block per
// (chunk, value head)) is stored tile by tile: the 32-column slices one after
// another, each in groups of 16 rows, each group as its two 16 x 16 tiles
// (columns 0-15, then 16-31) with rows of 16 elements.  A store of 16 rows x
// 16 columns and a load of 16 rows x 32 columns then each cover contiguous
// memory (512 B, 1 KB).  Element offset of (i, v) within the block:
__device__ __forceinline__ uint32_t hand_off(int dk, int i, int v) {
  return static_cast<uint32_t>((v >> 5) * dk * 32 + (i >> 4) * 512 + ((v >> 4) & 1) * 256 + (i & 15) * 16 + (v & 15));
}

__device__ inline void block_coords(const Dims& d, int nslice, int& b, int& h, int& slice) {
  const int n = blockIdx.x, G = d.G(), groups = d.B * d.Hk, per = G * nslice;
  int g, r;
  if (groups % 8 == 0) {
    const int xcd = n % 8, m = n / 8;
    g = xcd + 8 * (m / per);
    r = m % per;
  } else {
    g = n / per;
    r = n % per;
  }
  b = g / d.Hk;
  h = (g % d.Hk) * G + r / nslice;
  slice = r % nslice;
}

// The chunk form computes its per-step scalars (norm factors, gates) in
// chunk_prep itself; it does not use StepScalars.
struct ChunkPrepArgs {
  Dims d;
  const void *q, *k, *a, *b;
  const float *A_log, *dt_bias;
  const uint8_t* mask;
  ChunkBufs cb;
  int bwd;  // 0: the forward's buffers (Tx, Mq, sc); 1: the backward's (Tx, sc,
            // P^T, Q^T); 2: both
};

// Chunk matrices of the per-key-channel gate: Tx, Mq / P^T (as
// ChunkBufs, with the decay e^{G_t - G_s} taken per channel inside the
// products) and the pre-scaled rows Kb, Kh, Qb / KbT, QbT and vsc.
struct VgChunkPrepArgs {
  Dims d;
  const void *q, *k, *b;
  const float* lg;
  const uint8_t* mask;
  ChunkBufs cb;
  int bwd;  // 0: Tx, Mq, Kb, Kh, Qb, vsc; 1: Tx, P^T, Kb, Kh, KbT, QbT, vsc; 2: all of them
};
// Gradient pass of the per-key-channel gate's chunk form, in three kernels:
// vg_chunk_x (one workgroup per (chunk, batch, value head)) recomputes X from
// the fp32 checkpoint and writes it (or, with xsv, reads the forward's saved
// copy) and writes dP, dA and db; vg_chunk_grad (one
// workgroup per (chunk, batch, value head, 32 channels)) writes dlg and the
// value head's parts of dL/d(s qn) and dL/dkn; vg_norm_bwd sums the parts of
// a key head's value heads and turns them into dq, dk (the L2-norm backward).
struct VgChunkGradArgs {
  Dims d;
  const void *q, *k, *v, *b, *dO;
  const float* lg;
  const uint8_t* mask;
  const float *state0, *ckpt;  // state0 may be null
  StepScalars s;               // rk, rq
  ChunkBufs cb;                // Tx, Kb, vsc
  const bf16* dHend;           // [NC, B*Hv, Dk, Dv] dL/d(state at the end of chunk c)
  const void* dv;              // [B,T,Hv,Dv] dv (= Ehat) from the reverse state pass
  bf16* X;                     // [B,T,Hv,Dv] X_t = v_t - u_t of every step
  bf16* dPA;                   // [B*Hv, NC, 2, L, L] dP, dA
  bf16* qk;                    // [B,T,Hv,2,Dk] each value head's parts of the rows of d(s qn), d(kn), bf16
  void *dq, *dk, *db;          // outputs (input dtype)
  float* dlg;                  // [B,T,Hv,Dk]
  int xsv = 0;                 // X is the forward's saved copy (vg_chunk_x does not recompute it)
};
// Channels per vg_chunk_grad workgroup.
constexpr int kVgGradChannels = 32;
// The chunk form of the per-key-channel gate: bf16 I/O, Dk up to 192 (the
// state passes hold a second k tile in LDS), Dv a multiple of 32 up to 128
// (the gradient pass holds Dv-wide row operands in registers).
inline bool vg_chunk_supported(int Dk, int Dv, bool bf16) {
  return bf16 && (Dk == 64 || Dk == 128 || Dk == 192) && Dv % 32 == 0 && Dv <= 128;
}

struct ChunkFwdArgs {
  Dims d;
  const void *q, *k, *v;
  const float* state0;
  ChunkBufs cb;
  void* o;
  float* state_out;
  float* ckpt;
  // Segments of the T-parallel forward (seg = chunks per segment, 0: one
  // segment, the whole sequence; blockIdx.y = segment).  Output mode (map = 0):
  // segment s > 0 starts from hseg[s - 1] ([nseg - 1, B*Hv, Dk, Dv] fp32).
  // Map mode (map = 1): each segment's chain runs on the augmented state
  // [I | 0] with values [0 | V] (Dk + Dv columns: the identity columns read
  // v from vzero, 64 zero bytes) and its final state, the segment's affine
  // map [A | B], goes to maps ([nseg, B*Hv, Dk, Dk + Dv] fp32); nothing else
  // is written.
  int seg, map;
  const float* hseg;
  float* maps;
  const bf16* vzero;
  int vg;  // 1: per-key-channel gate (operands Kb, Kh, Qb and vsc of cb)
  int stream;  // 1: the bf16 chunk-start states are stored non-temporal (scalar gate)
};
// Start states of the segments: H_{s+1} = A_s H_s + B_s over the segment maps.
struct SegChainArgs {
  Dims d;
  int nseg;
  const float* state0;  // may be null
  const float* maps;    // [nseg, B*Hv, Dk, Dk + Dv]
  float* hseg;          // [nseg - 1, B*Hv, Dk, Dv]
  int reverse;          // 1: from the last segment back (the backward's chain):
                        // hseg[s - 1] = A_s hseg[s] + B_s, hseg[nseg - 1] = state0
};

// Chunk-form backward.  The reverse state pass writes dv, eps (dL/d delta) and
// the per-chunk gradients w.r.t. the state at each chunk's end; the gradient
// pass turns them into dq, dk, da, db and the per-chunk parameter sums.
struct ChunkBwdArgs {
  Dims d;
  const void *q, *k, *v, *dO, *a;
  const float *A_log, *dt_bias;
  const uint8_t* mask;
  const float *state0, *ckpt, *dS_final;  // state0 / dS_final may be null
  ChunkBufs cb;
  bf16* dHend;    // [NC, B*Hv, Dk, Dv]  dL/d(state at the end of chunk c)
  void *dq, *dk, *dv, *da, *db;
  float* dstate;     // [B,Hv,Dk,Dv]
  double* part_dA;   // [B,NC,Hv] per-chunk sums of dl * l
  double* part_ddt;  // [B,NC,Hv] per-chunk sums of da
  // T-parallel reverse state pass (as ChunkFwdArgs, in reverse): segment s
  // runs its chunks last to first; output mode starts it from hseg[s] (dL/d
  // the state at its end, [nseg - 1, B*Hv, Dk, Dv]; the last segment from
  // dS_final); map mode runs the augmented [I | 0] with dO = [0 | dO] and
  // stores the segment's map [A | B] (dL/d its start state) to maps.
  int seg, map;
  const float* hseg;
  float* maps;
  const bf16* vzero;
  int vg;  // 1: per-key-channel gate (operands Kh, KbT, QbT and vsc of cb)
  int stream;  // 1: dH' is stored non-temporal (scalar gate)
};

// bf16 copies of the states at the chunk starts from the fp32 checkpoints:
// Hb[0] = state0 (zeros when null), Hb[c] = ckpt[c - 1].
struct StateBf16Args {
  int nslot;            // chunks
  size_t slot;          // elements per slot (B*Hv*Dk*Dv, a multiple of 8)
  int dk, dv;           // the block of one head is Dk x Dv (written in the hand-off layout)
  const float *state0, *ckpt;
  bf16* Hb;
};

struct ParamReduceArgs {
  int B, NC, Hv;
  const double *part_dA, *part_ddt;
  float *dA_log, *ddt_bias;
};

// Single-step forward (T = 1), fused prep and update.
struct DecodeArgs {
  Dims d;
  const void *q, *k, *v, *a, *b;
  const float *A_log, *dt_bias;
  const float* state0;  // may be null; may alias state_out exactly
  const uint8_t* mask;
  void* o;
  float* state_out;
};
// Single-step forward with the preceding depthwise causal conv1d + SiLU
// update of the token's mixed projection (channels q, k, v).
constexpr int kMaxConvTaps = 8;
struct DecodeConvArgs {
  Dims d;
  const void* x;           // [B, C] input dtype, C = 2 Hk Dk + Hv Dv
  const void* conv_w;      // [C, K] input dtype
  const void* conv_state;  // [B, C, K] input dtype
  void* conv_state_out;    // [B, C, K]; may alias conv_state exactly
  int K;                   // taps, 1 .. kMaxConvTaps
  const void *a, *b;       // [B, Hv] input dtype
  const float *A_log, *dt_bias;
  const float* state0;     // may be null; may alias state_out exactly
  const uint8_t* mask;     // [B] or null
  void* o;                 // [B, Hv, Dv] input dtype
  float* state_out;
};
inline bool decode_supported(int Dk, int Dv) {
  return (Dk == 16 || Dk == 32 || Dk == 64 || Dk == 128 || Dk == 192 || Dk == 256) && Dv % 32 == 0 && Dv <= 256;
}

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t st);
hipError_t launch_decode_conv(const DecodeConvArgs& a, bool bf16, hipStream_t st);
// LDS of the decode-with-conv kernel: the conv outputs of one key-head group.
inline size_t conv_lds_bytes(const Dims& d) { return (2 * static_cast<size_t>(d.Dk) + static_cast<size_t>(d.G()) * d.Dv) * 4; }
constexpr size_t kMaxConvLds = 64 * 1024;
hipError_t launch_prep(const PrepArgs& a, bool bf16, hipStream_t st);
hipError_t launch_scan_fwd(const ScanFwdArgs& a, bool bf16, hipStream_t st);
hipError_t launch_scan_bwd(const ScanBwdArgs& a, bool bf16, hipStream_t st);
hipError_t launch_chunk_grad(const ChunkGradArgs& a, bool bf16, hipStream_t st);
hipError_t launch_scan_bwd_vg(const ScanBwdVgArgs& a, bool bf16, hipStream_t st);
hipError_t launch_vg_reduce(const VgReduceArgs& a, bool bf16, hipStream_t st);
hipError_t launch_param_reduce(const ParamReduceArgs& a, hipStream_t st);
hipError_t launch_chunk_prep(const ChunkPrepArgs& a, hipStream_t st);
hipError_t launch_vg_chunk_prep(const VgChunkPrepArgs& a, hipStream_t st);
hipError_t launch_vg_chunk_x(const VgChunkGradArgs& a, hipStream_t st);
hipError_t launch_vg_chunk_grad(const VgChunkGradArgs& a, hipStream_t st);
hipError_t launch_vg_norm_bwd(const VgChunkGradArgs& a, hipStream_t st);
hipError_t launch_chunk_fwd(const ChunkFwdArgs& a, hipStream_t st);
hipError_t launch_seg_chain(const SegChainArgs& a, hipStream_t st);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st);
hipError_t launch_chunk_bwd_state(const ChunkBwdArgs& a, hipStream_t st);
hipError_t launch_chunk_bwd_grad(const ChunkBwdArgs& a, hipStream_t st);
hipError_t launch_state_bf16(const StateBf16Args& a, hipStream_t st);

// Segments of the T-parallel chunk forward.  The segment maps cost
// (Dk + Dv) / Dv times a chunk pass on top of the output pass, so segments pay
// only when the single pass (B Hv Dv / 32 workgroups, one per compute unit)
// leaves at least three quarters of the 256 compute units idle.  Then: enough
// segments that the output pass has about one workgroup per compute unit (the
// segment passes are then bound by the chip's throughput, and the chain over
// the segments, which is bound by latency, stays short), at least 8 chunks
// each.  Returns the chunks per segment (0: one segment).
inline int tpar_seg_len(const Dims& d) {
  const int nc = d.nchunk();
  const long wgs = static_cast<long>(d.B) * d.Hv * (d.Dv / 32);
  if (wgs * 4 > 256) return 0;
  long p = (256 + wgs - 1) / wgs;
  if (p > nc / 8) p = nc / 8;
  if (p < 2) return 0;
  const int seg = static_cast<int>((nc + p - 1) / p);
  return (nc + seg - 1) / seg >= 2 ? seg : 0;
}
inline int tpar_nseg(const Dims& d, int seg) { return seg ? (d.nchunk() + seg - 1) / seg : 1; }

// The chunk form runs bf16 I/O with Dk a multiple of 32 and Dv a multiple of 32.
inline bool chunk_supported(int Dk, int Dv, bool bf16) {
  return bf16 && (Dk == 64 || Dk == 128 || Dk == 192 || Dk == 256) && Dv % 32 == 0 && Dv <= 256;
}

// Column-slice geometry of the scan kernels: NW waves x 8 columns each.
inline int scan_waves(int Dv) { return Dv % 32 == 0 ? 4 : 1; }
inline int scan_nslice(int Dv) { return Dv / (8 * scan_waves(Dv)); }
inline int vg_nslice(int Dv) { return scan_nslice(Dv); }
inline bool scan_supported(int Dk, int Dv) {
  bool dk = Dk == 16 || Dk == 32 || Dk == 64 || Dk == 128 || Dk == 192 || Dk == 256;
  bool dv = Dv >= 8 && Dv <= 256 && Dv % 8 == 0 && (Dv <= 24 || Dv % 32 == 0);
  return dk && dv;
}

}  // namespace gdn
