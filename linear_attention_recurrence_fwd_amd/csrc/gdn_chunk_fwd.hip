// Chunked (matrix) form of the gated delta rule forward on gfx950 bf16 MFMA.
//
// The recurrence (mlx-lm VJP PR, "What this PR adds"; torch-to-nnef GDN page,
// "Op contract") over a chunk of L = 64 steps, written with the state H at the
// chunk start, gamma_t = l_0 + ... + l_t and X_t = v_t - u_t (u_t = S'_t^T kn_t,
// so delta_t = beta_t X_t):
//   X   = Tx (V - diag(e^gamma rk) K H),      Tx = (I + N)^-1,
//         N[t,s] = [s<t] e^{g_t-g_s} rk_t rk_s beta_s (k_t . k_s)
//   O   = diag(e^gamma rq) Q H + Mq X,        Mq[t,s] = [s<=t] e^{g_t-g_s} rq_t rk_s beta_s (q_t . k_s)
//   H'  = e^{gamma_L} H + K^T diag(w) X,      w_t = beta_t e^{g_L-g_t} rk_t
// (K, Q raw rows; rk, rq the normalisation factors).  The per-step algorithm
// and this form agree up to the order of floating-point operations (the
// torch-to-nnef page notes the same of HF's chunked variant).  Decays enter
// only as e^{g_t - g_s} with s <= t, never as e^{-g}.
//
// Kernels:
//   chunk_prep  one workgroup per (chunk, batch, value head): the chunk's k and
//               q rows staged in LDS by coalesced loads, K K^T and Q K^T on
//               MFMA, the gates and gamma by a wave scan, N, Tx by blocked
//               forward substitution (fp32), Mq and the per-step chunk scalars.
//               With `bwd` set it writes the transposes the backward needs
//               instead of Mq, and the first value head of each key head
//               writes Q^T.  All outputs go to the workspace (bf16 / fp32),
//               16 bytes per store.
//   chunk_fwd   one workgroup per (batch, value head, 32-column slice of Dv),
//               walking the chunks in order with H in MFMA accumulators (fp32),
//               the next chunk's operands prefetched into registers while the
//               current chunk computes (the in-chunk barriers wait for LDS
//               only, so the prefetch stays in flight across them).  Blocks
//               that share a key head run on one XCD, so their K / Q reads
//               hit that XCD's L2.  Writes o, the checkpoints and the
//               final state, and for the backward's saved record the bf16
//               chunk-start states and X of every step.
#include <type_traits>

#include "gdn_dev.h"
#include "gdn_internal.h"
#include "gdn_tri.h"

namespace gdn {
namespace {

constexpr int L = kChunk;
constexpr int NT = 256;

// ------------------------------------------------------------------ prep

template <int DK>
struct ChunkPrep {
  // The k / q rows are staged in passes of CW channels (18 KB), which share
  // the LDS with the matrices of the last phase (35 KB): four workgroups fit
  // on a compute unit at every Dk.  The Gram products accumulate over the
  // passes in the order of a single pass.
  static constexpr int CW = 64;      // channels per pass
  static constexpr int NPASS = DK / CW;
  static constexpr int RS = CW + 8;  // bf16 row stride of the staged k / q rows (conflict-free operand reads)
  static constexpr int SP = tri::SP;  // fp32 row stride of N and the staging matrix
  static constexpr int NLD = L * CW / 8 / NT;  // 16-byte pieces of one of k, q per thread and pass
  static_assert(DK % CW == 0 && L * CW / 8 % NT == 0, "whole pieces per thread");
  struct Rows {
    bf16 k[L * RS];
    bf16 q[L * RS];
  };
  struct Mats {
    float nf[L * SP];  // N; its diagonal 16x16 blocks are replaced by their inverses
    float st[L * SP];  // staging of the matrices written out
  };
  union Big {
    Rows r;
    Mats m;
  };
  struct Smem {
    alignas(16) Big u;
    float gam[L], rk[L], rq[L], beta[L], ell[L];
  };

  __device__ static void store_mat(const Smem& sm, bf16* dst, int tid) { tri::store_mat(sm.u.m.st, dst, tid, NT); }

  // Rows [t][i] of the staged pass -> dst [i][t] (bf16, L steps per row; dst
  // at the pass's first channel).
  __device__ static void store_transposed(const bf16* rows, bf16* dst, int tid) {
    for (int u = tid; u < CW * L / 8; u += NT) {
      const int i = u % CW, t8 = 8 * (u / CW);
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        wv[e] = static_cast<uint32_t>(rows[(t8 + 2 * e) * RS + i].x) |
                (static_cast<uint32_t>(rows[(t8 + 2 * e + 1) * RS + i].x) << 16);
      *reinterpret_cast<uint4*>(dst + static_cast<size_t>(i) * L + t8) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
  }

  // Tx = (I + N)^-1 in 16x16 blocks (fp32), gdn_tri.h.
  __device__ static void invert_diagonal_block(Smem& sm, int w, int l) { tri::invert_diagonal_block(sm.u.m.nf, w, l); }
  __device__ static void lower_blocks(Smem& sm, int j) { tri::lower_blocks(sm.u.m.nf, sm.u.m.st, j); }

  // One workgroup per (chunk, batch, value head).  The G workgroups of a key
  // head recompute its K K^T and Q K^T (cheap on the matrix cores; the k / q
  // rows come from L2) and, for the backward, the first of them writes Q^T.
  __device__ static void run(const ChunkPrepArgs& p, Smem& sm) {
    const Dims& d = p.d;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int G = d.G(), NC = d.nchunk();
    const int b = bh / d.Hv, h = bh % d.Hv, j = h / G;
    const bool first = h % G == 0;
    const int t0 = c * L, Lc = min(L, d.T - t0), tl = Lc - 1;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    const size_t qk0 = (static_cast<size_t>(b) * d.T + t0) * d.Hk + j;
    const uint32_t qk_row = d.Hk * DK;
    const bf16* kc = static_cast<const bf16*>(p.k) + qk0 * DK;
    const bf16* qc = static_cast<const bf16*>(p.q) + qk0 * DK;
    const size_t mat = (static_cast<size_t>(bh) * NC + c) * L * L;

    // ---- the gate inputs of step t = l (wave 0)
    float ell = 0.f, beta = 0.f;
    if (w == 0) {
      // l = -e^{A_log} softplus(min(a + dt_bias, 20)), beta = sigmoid(b);
      // a masked step (or a row past the end) gets l = 0, beta = 0
      const int t = min(l, tl);
      const size_t o = (static_cast<size_t>(b) * d.T + t0 + t) * d.Hv + h;
      const float av = to_f32(static_cast<const bf16*>(p.a)[o]), bv = to_f32(static_cast<const bf16*>(p.b)[o]);
      const rsrc_t rm = make_rsrc(p.mask ? static_cast<const void*>(p.mask) : p.a,
                                  p.mask ? static_cast<size_t>(d.B) * d.T : 0);
      const uint32_t mrow = static_cast<uint32_t>(b * d.T + t0 + t);
      const bool valid = l < Lc && (p.mask == nullptr || __builtin_amdgcn_raw_buffer_load_b8(rm, mrow, 0, 0) != 0);
      const float x = av + p.dt_bias[h], alog = p.A_log[h];
      if (valid) {
        ell = -expf(alog) * softplus_f(fminf(x, kClamp));
        beta = sigmoid_f(bv);
      }
    }
    if (w == 0) {  // gamma by a wave-wide inclusive scan
      float g = ell;
#pragma unroll
      for (int off = 1; off < L; off <<= 1) {
        const float y = __shfl_up(g, off);
        if (l >= off) g += y;
      }
      sm.gam[l] = g;
      sm.ell[l] = ell;
      sm.beta[l] = beta;
    }
    const bool fwd_out = p.bwd != 1, bwd_out = p.bwd != 0;

    // ---- K K^T and Q K^T (raw rows), wave w = row tile w; Q Q^T on the
    // diagonal tile gives |q_t|^2; per pass of CW channels: the k / q rows of
    // the chunk (clamped into the sequence), coalesced 16-byte loads, and the
    // raw rows transposed for the backward (written once per key head)
    f32x4 akk[4], aqk[4], aqq = f4zero();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) akk[ct] = aqk[ct] = f4zero();
#pragma unroll
    for (int pc = 0; pc < NPASS; ++pc) {
      const int c0 = pc * CW;
      u32x4 kv[NLD], qv[NLD];
#pragma unroll
      for (int e = 0; e < NLD; ++e) {
        const int u = tid + e * NT, t = u / (CW / 8), i8 = 8 * (u % (CW / 8));
        const uint32_t o = static_cast<uint32_t>(min(t, tl)) * qk_row + c0 + i8;
        kv[e] = *reinterpret_cast<const u32x4*>(kc + o);
        qv[e] = *reinterpret_cast<const u32x4*>(qc + o);
      }
      if (pc > 0) __syncthreads();  // the previous pass is done with the staged rows
#pragma unroll
      for (int e = 0; e < NLD; ++e) {
        const int u = tid + e * NT, t = u / (CW / 8), i8 = 8 * (u % (CW / 8));
        *reinterpret_cast<u32x4*>(&sm.u.r.k[t * RS + i8]) = kv[e];
        *reinterpret_cast<u32x4*>(&sm.u.r.q[t * RS + i8]) = qv[e];
      }
      __syncthreads();
#pragma unroll
      for (int kt = 0; kt < CW / 32; ++kt) {
        const int oa = (16 * w + lr) * RS + 32 * kt + 8 * lg;
        const bf16x8 ak = load_bf16x8(&sm.u.r.k[oa]), aq = load_bf16x8(&sm.u.r.q[oa]);
        aqq = mfma16(aq, aq, aqq);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const bf16x8 bk = load_bf16x8(&sm.u.r.k[(16 * ct + lr) * RS + 32 * kt + 8 * lg]);
          akk[ct] = mfma16(ak, bk, akk[ct]);
          aqk[ct] = mfma16(aq, bk, aqk[ct]);
        }
      }
      if (first && bwd_out) {
        const size_t base = (static_cast<size_t>(b * d.Hk + j) * NC + c) * DK * L + static_cast<size_t>(c0) * L;
        store_transposed(sm.u.r.q, p.cb.QT + base, tid);
      }
    }
    // norm factors from the Gram diagonals: (|x|^2 + eps)^-1/2, q also / sqrt(Dk)
    // (the lane holding element (t, t) of tile (w, w) writes them)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (lr == 4 * lg + r) {
        const int t = 16 * w + 4 * lg + r;
        float kk = 0.f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          if (ct == w) kk = akk[ct][r];
        const bool in = t < Lc;
        sm.rk[t] = in ? 1.f / sqrtf(kk + kNormEps) : 0.f;
        sm.rq[t] = in ? (1.f / sqrtf(static_cast<float>(DK))) / sqrtf(aqq[r] + kNormEps) : 0.f;
      }
    __syncthreads();  // the staged rows are dead from here on; rk, rq visible

    // ---- per-step chunk scalars
    if (tid < L) {
      const int t = tid;
      const float gl = sm.gam[Lc - 1];
      const float eg = expf(sm.gam[t]), el = expf(gl - sm.gam[t]);
      float* sc = p.cb.sc + (static_cast<size_t>(bh) * NC + c) * SC_ROWS * L;
      sc[SC_CR * L + t] = eg * sm.rk[t];
      sc[SC_CO * L + t] = eg * sm.rq[t];
      sc[SC_W * L + t] = sm.beta[t] * el * sm.rk[t];
      sc[SC_KL * L + t] = el * sm.rk[t];
      sc[SC_BETA * L + t] = sm.beta[t];
      sc[SC_EGL * L + t] = t == 0 ? expf(gl) : 0.f;
      sc[SC_GAM * L + t] = sm.gam[t];
      sc[SC_EG * L + t] = eg;
      sc[SC_EL * L + t] = el;
      sc[SC_RK * L + t] = sm.rk[t];
      sc[SC_RQ * L + t] = sm.rq[t];
      sc[SC_ELL * L + t] = sm.ell[t];
    }

    // ---- N (fp32), and the decayed Grams: Mq (forward) or P^T (backward; the
    // gradient pass forms A and P itself from the raw Grams).
    // The per-step values are read first and the terms selected, not branched
    // on (a branch would wait for each element's reads in turn).
    float gt[4], rkt[4], rqt[4], gs[4], rks[4], bs[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * w + 4 * lg + r;
      gt[r] = sm.gam[t];
      rkt[r] = sm.rk[t];
      rqt[r] = sm.rq[t];
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int s = 16 * ct + lr;
      gs[ct] = sm.gam[s];
      rks[ct] = sm.rk[s];
      bs[ct] = sm.beta[s];
    }
    float mq[4][4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * w + 4 * lg + r, s = 16 * ct + lr;
        const bool le = s <= t, lt = s < t;
        // hardware exp: its error (about |x| 2^-24 relative) is far below the
        // bf16 rounding of every matrix this decay enters; for s > t (term
        // unused) the argument is 0, so no overflow is computed
        const float dec = __expf(le ? gt[r] - gs[ct] : 0.f);
        const float at = lt ? dec * rkt[r] * rks[ct] * akk[ct][r] : 0.f;
        const float nv = at * bs[ct];
        const float pq = le ? dec * rqt[r] * rks[ct] * aqk[ct][r] : 0.f;
        sm.u.m.nf[t * SP + s] = nv;
        if (bwd_out) {
          sm.u.m.st[s * SP + t] = pq;  // P^T
        } else {
          sm.u.m.st[t * SP + s] = pq * bs[ct];  // Mq
        }
        mq[ct][r] = pq;
      }
    __syncthreads();
    invert_diagonal_block(sm, w, l);
    if (bwd_out) {
      store_mat(sm, p.cb.PqT + mat, tid);
      if (fwd_out) {
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s = 16 * ct + lr;
            sm.u.m.st[(16 * w + 4 * lg + r) * SP + s] = mq[ct][r] * sm.beta[s];  // Mq
          }
        __syncthreads();
        store_mat(sm, p.cb.Mq + mat, tid);
      }
    } else {
      store_mat(sm, p.cb.Mq + mat, tid);
    }

    // ---- the blocks of Tx below the diagonal (the diagonal ones are in nf)
    __syncthreads();  // the staging matrix is free (P^T / Mq stored); the D_i are visible
    if (w < 3)
      lower_blocks(sm, w);
    else  // diagonal blocks into the staging matrix, zeros above them
      tri::diagonal_blocks(sm.u.m.nf, sm.u.m.st, l);
    __syncthreads();
    store_mat(sm, p.cb.Tx + mat, tid);
  }
};

template <int DK>
__global__ void __launch_bounds__(NT) chunk_prep_kernel(ChunkPrepArgs p) {
  __shared__ typename ChunkPrep<DK>::Smem sm;
  ChunkPrep<DK>::run(p, sm);
}

// ------------------------------------------------------------ state pass

// ST: the bf16 chunk-start states are stored non-temporal (ChunkFwdArgs::stream).
template <int DK, bool VG = false, bool ST = false>
struct ChunkFwd {
  // Twelve waves in three groups of four (w = wave index within the group):
  //   A (waves 0-3):  K H, R and X = Tx R for row tile w.  A also streams the
  //                   chunk's k rows, Tx, v slice and chunk scalars into a
  //                   ring of LDS slots with direct-to-LDS buffer loads, PD
  //                   chunks ahead, so these operands never pass through
  //                   registers;
  //   B (waves 4-7):  the state update H <- e^{gL} H + K^T diag(w) X for its
  //                   row tiles of H (K^T read transposed from the ring), and
  //                   the checkpoints (fp32, and / or the bf16 copies the
  //                   backward's gradient pass reads);
  //   C (waves 8-11): Q H and the output O = diag(e^g rq) Q H + Mq X for row
  //                   tile w (q and Mq prefetched two chunks ahead in
  //                   registers).
  // B and C work at the same time once X is in LDS.
  // With the per-key-channel gate (VG) the operands come pre-scaled from
  // vg_chunk_prep: A reads Kb rows (no row scale), B reads Kh^T from a second
  // k tile of the ring and decays H row-wise by e^{G_L}, C reads Qb rows, and
  // the weights of X are beta.
  static constexpr int NTS = 768;
  static constexpr int NV = 32;                   // Dv columns per workgroup
  static constexpr int RTW = DK / 64;             // H row tiles per group-B wave
  static constexpr int HS = DK + 8;               // bf16 row stride of H^T
  static constexpr int XS = L + 8;                // bf16 row stride of R^T / X^T
  static constexpr int NPK = DK / 8;              // 16-byte pieces of a k row
  static constexpr int NSL = VG ? (DK <= 128 ? 3 : 2) : (DK <= 192 ? 3 : 2);  // ring slots
  static constexpr int PD = NSL - 1;              // chunks loaded ahead
  static constexpr int KDMA = DK / 32;            // k loads per group-A wave per chunk
  static constexpr int NDMA = KDMA * (VG ? 2 : 1) + 2 + 1 + 1;  // ring loads per group-A wave per chunk
  static constexpr int SCR = VG ? VSC_ROWS : SC_ROWS;  // chunk scalar rows per chunk
  // A ring slot.  Lane i of a direct-to-LDS load writes its 16 (or 4) bytes at
  // the load's base + 16 i (4 i), so the layouts are set through the global
  // addresses: 16-byte piece p of row t sits at t * (pieces per row) +
  // (p ^ swizzle(t)), which keeps the operand reads free of bank conflicts.
  struct SlotBase {
    bf16 k[L * DK];   // k rows [t][i] (VG: Kb), swizzle t & 7
    bf16 tx[L * L];   // Tx rows, swizzle t & 7
    bf16 v[L * NV];   // v rows of this slice's columns, swizzle t & 3
    float sc[4 * L];  // chunk scalar rows 0 .. 3 (SC_CR, SC_CO, SC_W, SC_EGL; VG: beta, e^{G_L})
  };
  struct SlotVg : SlotBase {
    bf16 kh[L * DK];  // Kh rows [t][i], swizzle t & 7
  };
  using Slot = std::conditional_t<VG, SlotVg, SlotBase>;
  static_assert(SC_CR < 4 && SC_CO < 4 && SC_W < 4 && SC_EGL < 4, "rows held in a ring slot");
  static_assert(!VG || DK <= 3 * L, "e^{G_L} of every channel in rows 1 .. 3 of the slot");
  // the k tile group B reads transposed
  __device__ static __forceinline__ const bf16* b_tile(const Slot& s) {
    if constexpr (VG)
      return s.kh;
    else
      return s.k;
  }
  struct Smem {
    alignas(16) Slot ring[NSL];
    alignas(16) bf16 hb[NV * HS];   // H^T (bf16), the B operand of K H and Q H
    alignas(16) bf16 rb[NV * XS];   // R^T
    alignas(16) bf16 xb[NV * XS];   // X^T
    alignas(16) bf16 xw[NV * XS];   // (diag(w) X)^T
  };
  // Group C's operands of one chunk, held in registers.  Every load is
  // unconditional, from an address clamped into the sequence, so no load sits
  // in a branch (a load in a branch makes the compiler wait for all
  // outstanding loads, prefetch included).  Rows past the end of the sequence
  // hold copies of its last row and need no zeroing: their chunk scalars (rk,
  // rq, w) are zero, Tx and Mq are lower triangular and their outputs are not
  // stored, so they never reach a stored value (inputs are finite).
  struct StageC {
    bf16x8 qa[DK / 32];               // q rows t = 16 w + lr
    bf16x8 mqa[2];                    // Mq rows t = 16 w + lr
  };
  // Per-workgroup values (uniform) and per-lane coordinates (w = wave index
  // within the group, uniform).  Addresses are a uniform descriptor plus a
  // 32-bit lane offset.
  struct Lane {
    int b, h, j, bh, bj, col0, w, l, lr, lg, ta, tc0, last, NC;
    int cs, ce, seg, mode;       // chunk range of the segment; 0 output, 1 map identity, 2 map values
    int scol;                    // first state column of the slice (Dk + Dv columns in map mode)
    uint32_t vstep, vbase;       // v elements per step and offset (0, 0: the zero rows)
    uint32_t qk_row, v_row;   // element strides of one step in q/k and v/o
    rsrc_t rq, rmq;              // buffer descriptors of group C's operands
    i32x4 dk, dkh, dv, dtx, dsc; // raw descriptors of the ring's operands
  };

  // element offsets of 16-byte piece p of row t in the ring tiles
  __device__ static __forceinline__ int kpos(int t, int p) { return 8 * (t * NPK + (p ^ (t & 7))); }
  __device__ static __forceinline__ int xpos(int t, int p) { return 8 * (t * 8 + (p ^ (t & 7))); }
  __device__ static __forceinline__ int vpos(int t, int p) { return 8 * (t * 4 + (p ^ (t & 3))); }

  // Group A: the NDMA ring loads of this wave for chunk c into slot sl.  Load
  // n of a tile covers its 16-byte positions 64 n .. 64 n + 63.
  __device__ static void issue_ring(const ChunkFwdArgs& p, Smem& sm, const Lane& q, int c, int sl) {
    const Dims& d = p.d;
    const int t0 = c * L, tl = q.last - t0, l = q.l;
    Slot& s = sm.ring[sl];
#pragma unroll
    for (int jj = 0; jj < KDMA; ++jj) {
      const int n = KDMA * q.w + jj, pos = 64 * n + l, t = pos / NPK, pc = (pos % NPK) ^ (t & 7);
      if constexpr (VG) {  // Kb and Kh rows of this (head, chunk); rows past the end are zero
        const uint32_t o = 2 * ((static_cast<uint32_t>(q.bh * q.NC + c) * L + t) * DK + 8 * pc);
        dma16(q.dk, &s.k[512 * n], o);
        dma16(q.dkh, &s.kh[512 * n], o);
      } else {
        dma16(q.dk, &s.k[512 * n], 2 * ((static_cast<uint32_t>(q.b * d.T + t0 + min(t, tl)) * d.Hk + q.j) * DK + 8 * pc));
      }
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int n = 2 * q.w + jj, pos = 64 * n + l, t = pos / 8, pc = (pos % 8) ^ (t & 7);
      dma16(q.dtx, &s.tx[512 * n], 2 * (static_cast<uint32_t>(q.bh * q.NC + c) * L * L + t * L + 8 * pc));
    }
    {  // the v slice: read by this workgroup only, once (non-temporal)
      const int pos = 64 * q.w + l, t = pos / 4, pc = (pos % 4) ^ (t & 3);
      dma16_nt(q.dv, &s.v[512 * q.w],
            2 * (static_cast<uint32_t>(q.b * d.T + t0 + min(t, tl)) * q.vstep + q.vbase + 8 * pc));
    }
    dma4(q.dsc, &s.sc[L * q.w], 4 * (static_cast<uint32_t>(q.bh * q.NC + c) * SCR * L + L * q.w + l));
  }

  __device__ static void load_c(const ChunkFwdArgs& p, const Lane& q, int c, StageC& s) {
    const Dims& d = p.d;
    const int t0 = c * L, tl = q.last - t0;
    const int cr_ = 16 * q.w + coal_row(q.l), cp_ = coal_piece(q.l);  // quad-coalesced (see to_mfma_layout)
    const uint32_t ko = VG ? 2 * ((static_cast<uint32_t>(q.bh * q.NC + c) * L + cr_) * DK + 8 * cp_)
                           : 2 * ((static_cast<uint32_t>(q.b * d.T + t0 + min(cr_, tl)) * d.Hk + q.j) * DK + 8 * cp_);
#pragma unroll
    for (int kt = 0; kt < DK / 32; ++kt) s.qa[kt] = buf_bf16x8(q.rq, ko + 64 * kt);
    const uint32_t mo = 2 * (static_cast<uint32_t>(q.bh * q.NC + c) * L * L + cr_ * L + 8 * cp_);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s.mqa[kt] = buf_bf16x8(q.rmq, mo + 64 * kt);
  }

  __device__ static void put_h(Smem& sm, const Lane& q, const f32x4 (&H)[RTW][2]) {
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        *reinterpret_cast<uint2*>(&sm.hb[(16 * ct + q.lr) * HS + 16 * (q.w * RTW + it) + 4 * q.lg]) =
            pack4_bf16(H[it][ct][0], H[it][ct][1], H[it][ct][2], H[it][ct][3]);
  }

  // Group A, one chunk: K H -> R -> X from slot c, with the ring loads of
  // chunk c + PD issued after barrier 1 (so that they do not hold up the
  // chain to barrier 1, nor the other groups' global accesses at the start of
  // the chunk).  Before barrier 3 each wave waits for its loads of chunk
  // c + 1 (the loads of PD - 1 later chunks may stay in flight); barrier 3
  // then makes slot c + 1 complete for every wave.  The slot refilled here
  // was last read (by B and C) before barrier 3 of the previous chunk.
  __device__ static void step_a(const ChunkFwdArgs& p, Smem& sm, const Lane& q, int c) {
    const Slot& s = sm.ring[c % NSL];
    const int lr = q.lr, lg = q.lg, ta = q.ta;
    bf16x8 ka[DK / 32], txa[2];
#pragma unroll
    for (int kt = 0; kt < DK / 32; ++kt) ka[kt] = load_bf16x8(&s.k[kpos(ta, 4 * kt + lg)]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) txa[kt] = load_bf16x8(&s.tx[xpos(ta, 4 * kt + lg)]);
    const float4 cr = VG ? make_float4(1.f, 1.f, 1.f, 1.f) : *reinterpret_cast<const float4*>(&s.sc[SC_CR * L + q.tc0]);
    const float4 wv = *reinterpret_cast<const float4*>(&s.sc[(VG ? VSC_BETA : SC_W) * L + q.tc0]);
    const float wvv[4] = {wv.x, wv.y, wv.z, wv.w};
    const float crv[4] = {cr.x, cr.y, cr.z, cr.w};
    f32x4 kh[2];
    kh[0] = kh[1] = f4zero();
#pragma unroll
    for (int kt = 0; kt < DK / 32; ++kt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        kh[ct] = mfma16(ka[kt], load_bf16x8(&sm.hb[(16 * ct + lr) * HS + 32 * kt + 8 * lg]), kh[ct]);
    // R = V - diag(e^g rk) K H; v read transposed: rows q.tc0 .. + 3 of column 16 ct + lr
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int tv = q.tc0 + (lr >> 2);
      const uint2 v4 = lds_read_tr16(&s.v[vpos(tv, 2 * ct + ((lr >> 1) & 1)) + 4 * (lr & 1)]);
      const float vr[4] = {__uint_as_float(v4.x << 16), __uint_as_float(v4.x & 0xffff0000u),
                           __uint_as_float(v4.y << 16), __uint_as_float(v4.y & 0xffff0000u)};
      float rv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) rv[r] = vr[r] - crv[r] * kh[ct][r];
      *reinterpret_cast<uint2*>(&sm.rb[(16 * ct + lr) * XS + q.tc0]) = pack4_bf16(rv[0], rv[1], rv[2], rv[3]);
    }
    lds_barrier();  // 1: R complete
    issue_ring(p, sm, q, min(c + PD, q.ce - 1), (c + PD) % NSL);
    f32x4 x[2];
    x[0] = x[1] = f4zero();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        x[ct] = mfma16(txa[kt], load_bf16x8(&sm.rb[(16 * ct + lr) * XS + 32 * kt + 8 * lg]), x[ct]);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      *reinterpret_cast<uint2*>(&sm.xb[(16 * ct + lr) * XS + q.tc0]) = pack4_bf16(x[ct][0], x[ct][1], x[ct][2], x[ct][3]);
      *reinterpret_cast<uint2*>(&sm.xw[(16 * ct + lr) * XS + q.tc0]) =
          pack4_bf16(wvv[0] * x[ct][0], wvv[1] * x[ct][1], wvv[2] * x[ct][2], wvv[3] * x[ct][3]);
    }
    lds_barrier();  // 2: X complete
    wait_vm<(PD - 1) * NDMA>();
    lds_barrier();  // 3: H of the next chunk complete; slot c + 1 complete
  }

  // Group B, one chunk: H update.  The K^T operand comes from the ring's k
  // tile through transposing LDS reads: for row tile it and steps
  // 32 kt + 8 lg .. + 7, lane (lr, lg) gets column i = 16 (w RTW + it) + lr.
  // The stores of the previous chunk's results -- its X and the state at
  // this chunk's start (checkpoint and / or bf16 copy) -- are issued in
  // phase 1, where B waits for group A anyway: issued right after the update
  // they stall behind the memory pipeline and hold up barrier 3.
  __device__ static void step_b(const ChunkFwdArgs& p, Smem& sm, const Lane& q, int c, f32x4 (&H)[RTW][2]) {
    const int lr = q.lr, lg = q.lg;
    const Slot& s = sm.ring[c % NSL];
    store_x(p, sm, q, c - 1, c > q.cs);  // group A rewrites X^T after barrier 1
    store_states(p, q, H, c - 1, c > q.cs);
    lds_barrier();  // 1
    lds_barrier();  // 2: X complete
    const float egl = s.sc[SC_EGL * L];
    const bf16* kb = b_tile(s);
    bf16x8 kta[RTW][2];
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int t = 32 * kt + 8 * lg + (lr >> 2), pc = 2 * (q.w * RTW + it) + ((lr >> 1) & 1);
        const uint2 lo = lds_read_tr16(&kb[kpos(t, pc) + 4 * (lr & 1)]);
        const uint2 hi = lds_read_tr16(&kb[kpos(t + 4, pc) + 4 * (lr & 1)]);
        kta[it][kt] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // VG: e^{G_L} of row i = 16 (w RTW + it) + 4 lg + r
        const float e = VG ? s.sc[VSC_EGL * L + 16 * (q.w * RTW + it) + 4 * lg + r] : egl;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) H[it][ct][r] *= e;
      }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      bf16x8 bx[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) bx[ct] = load_bf16x8(&sm.xw[(16 * ct + lr) * XS + 32 * kt + 8 * lg]);
#pragma unroll
      for (int it = 0; it < RTW; ++it)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) H[it][ct] = mfma16(kta[it][kt], bx[ct], H[it][ct]);
    }
    put_h(sm, q, H);
    lds_barrier();  // 3: H of the next chunk complete
  }
  // The state at the end of chunk c (= the start of chunk c + 1): the fp32
  // checkpoint and / or its bf16 copy.  The stores are unconditional within
  // each kind; without a slot (the sequence's last chunk, or `on` false) the
  // descriptor is empty and they are dropped.
  __device__ static void store_states(const ChunkFwdArgs& p, const Lane& q, const f32x4 (&H)[RTW][2], int c, bool on) {
    const Dims& d = p.d;
    const int lr = q.lr, lg = q.lg;
    const bool slot = on && c + 1 < q.NC;
    if (p.ckpt != nullptr) {
      const size_t hsz = static_cast<size_t>(DK) * d.Dv;
      const rsrc_t rck = make_rsrc(slot ? static_cast<const void*>(p.ckpt + (static_cast<size_t>(c) * d.B * d.Hv + q.bh) * hsz)
                                        : static_cast<const void*>(p.state_out),
                                   slot ? hsz * 4 : 0);
      const uint32_t co = 4 * (static_cast<uint32_t>(16 * q.w * RTW + 4 * lg) * d.Dv + q.col0 + lr);
#pragma unroll
      for (int it = 0; it < RTW; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t o = co + 4 * static_cast<uint32_t>(16 * it + r) * d.Dv;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(H[it][0][r]), rck, o, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(H[it][1][r]), rck, o + 64, 0, 0);
        }
    }
    if (p.cb.Hb != nullptr) store_hb(p, q, H, slot ? c + 1 : -1);
  }

  // X of chunk c for the backward (bf16 [B, T, Hv, Dv]; dropped when cb.X is
  // null or `on` is false), from X^T in LDS while group B waits for A: a
  // transposing read gives lane 16 g + s four consecutive columns (group g)
  // of step 16 w + s, and groups_to_quads puts one step's four groups in each
  // quad of lanes, stored with 8-byte non-temporal stores.  Steps past the end
  // of the sequence fall outside the descriptor.  Group B issues no global
  // loads in its loop, so these stores hold up no wait for a load.
  __device__ static void store_x(const ChunkFwdArgs& p, const Smem& sm, const Lane& q, int c, bool on) {
    const Dims& d = p.d;
    on = on && p.cb.X != nullptr;
    const int t0 = max(c, 0) * L, Lc = min(L, d.T - t0);
    const size_t base = ((static_cast<size_t>(q.b) * d.T + t0) * d.Hv + q.h) * d.Dv + q.col0;
    const rsrc_t r = make_rsrc(on ? static_cast<const void*>(p.cb.X + base) : p.v,
                               on ? (static_cast<size_t>(Lc - 1) * q.v_row + NV) * 2 : 0);
    const uint32_t to = 2 * static_cast<uint32_t>(16 * q.w + (q.l >> 2)) * q.v_row;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int v0 = 4 * (4 * n + q.lg);
      const uint2 x4 = lds_read_tr16(&sm.xb[(v0 + (q.lr >> 2)) * XS + 16 * q.w + 4 * (q.lr & 3)]);
      buf_store_u2_nt(r, to + 2 * 4 * (4 * n + (q.l & 3)), groups_to_quads(x4));
    }
  }

  // bf16 copy of H as the state at the start of chunk `slot` (dropped when
  // slot < 0), in the hand-off layout of gdn_internal.h (row-major [i][v] with
  // the per-key-channel gate).  A quad transpose gives each lane four
  // consecutive columns of one row, quads_to_rows one row per quad of lanes:
  // each store covers a 16 x 16 tile, 512 contiguous bytes.  Non-temporal under ST (the
  // backward's hand-off does not fit the memory-side cache): nothing in
  // the forward reads them again, and as plain writes they would stay dirty in
  // the caches until the reverse state pass, whose chain then pays for their
  // write-back.
  __device__ static void store_hb(const ChunkFwdArgs& p, const Lane& q, const f32x4 (&H)[RTW][2], int slot) {
    const Dims& d = p.d;
    const size_t hsz = static_cast<size_t>(DK) * d.Dv;
    const rsrc_t r = make_rsrc(p.cb.Hb + (static_cast<size_t>(max(slot, 0)) * d.B * d.Hv + q.bh) * hsz,
                               slot >= 0 ? hsz * 2 : 0);
    // row 16 (w RTW + it) + 4 lg + lr / 4, columns col0 + 16 ct + 4 (lr % 4) ..;
    // the per-key-channel gate keeps row-major [i][v] blocks
    const int r16 = 4 * q.lg + (q.lr >> 2), c4 = 4 * (q.lr & 3);
    const uint32_t o = VG ? 2 * (static_cast<uint32_t>(16 * q.w * RTW + r16) * d.Dv + q.col0 + c4)
                          : 2 * hand_off(DK, 16 * q.w * RTW + r16, q.col0 + c4);
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const f32x4 tr = quad_transpose(H[it][ct]);
        const uint2 v = quads_to_rows(pack4_bf16(tr[0], tr[1], tr[2], tr[3]));
        const uint32_t ot = o + 2 * (VG ? 16 * it * d.Dv + 16 * ct : 512 * it + 256 * ct);
        if constexpr (ST)
          buf_store_u2_nt(r, ot, v);
        else
          buf_store_u2(r, ot, v);
      }
  }

  // Group C, one chunk: (Q H)^T, then O^T = (Q H)^T diag(e^gamma rq) + X^T Mq^T,
  // which gives each lane one step and four consecutive columns to store.
  __device__ static void step_c(const ChunkFwdArgs& p, Smem& sm, const Lane& q, int c, StageC& cur) {
#pragma unroll
    for (int kt = 0; kt < DK / 32; ++kt) cur.qa[kt] = to_mfma_layout(cur.qa[kt]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) cur.mqa[kt] = to_mfma_layout(cur.mqa[kt]);
    const Dims& d = p.d;
    const int t0 = c * L, Lc = min(L, d.T - t0);
    const int lr = q.lr, lg = q.lg;
    const float co = VG ? 1.f : sm.ring[c % NSL].sc[SC_CO * L + q.ta];
    f32x4 o[2];  // rows v = 16 ct + 4 lg + r, column t = 16 w + lr
    o[0] = o[1] = f4zero();
#pragma unroll
    for (int kt = 0; kt < DK / 32; ++kt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        o[ct] = mfma16(load_bf16x8(&sm.hb[(16 * ct + lr) * HS + 32 * kt + 8 * lg]), cur.qa[kt], o[ct]);
    lds_barrier();  // 1
    lds_barrier();  // 2: X complete
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[ct][r] *= co;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        o[ct] = mfma16(load_bf16x8(&sm.xb[(16 * ct + lr) * XS + 32 * kt + 8 * lg]), cur.mqa[kt], o[ct]);
    {  // rows past the end of the sequence fall outside the descriptor: dropped
      const rsrc_t ro = make_rsrc(static_cast<bf16*>(p.o) + ((static_cast<size_t>(q.b) * d.T + t0) * d.Hv + q.h) * d.Dv,
                                  (static_cast<size_t>(Lc - 1) * q.v_row + d.Dv) * 2);
      // lane 16 lg + lr holds step 16 w + lr, columns 16 ct + 4 lg .. + 3;
      // groups_to_quads gives each quad of lanes one step's four groups
      const uint32_t oo = 2 * (static_cast<uint32_t>(16 * q.w + (q.l >> 2)) * q.v_row + q.col0 + 4 * (q.l & 3));
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        buf_store_u2(ro, oo + 32 * ct, groups_to_quads(pack4_bf16(o[ct][0], o[ct][1], o[ct][2], o[ct][3])));
    }
    lds_barrier();  // 3
  }

  __device__ static void run_a(const ChunkFwdArgs& p, Smem& sm, const Lane& q) {
#pragma unroll
    for (int c = 0; c < PD; ++c) issue_ring(p, sm, q, min(q.cs + c, q.ce - 1), (q.cs + c) % NSL);
    wait_vm<(PD - 1) * NDMA>();
    lds_barrier();  // 0: initial H; slot of chunk cs complete
    for (int c = q.cs; c < q.ce; ++c) step_a(p, sm, q, c);
    wait_vm<0>();  // no direct-to-LDS load may land after the workgroup ends
  }

  __device__ static void run_b(const ChunkFwdArgs& p, Smem& sm, const Lane& q) {
    const Dims& d = p.d;
    const size_t sbase = static_cast<size_t>(q.bh) * DK * d.Dv;
    // H: rows i = 16 (w RTW + it) + 4 lg + r, columns col0 + 16 ct + lr.
    // Unconditional buffer loads; an absent initial state reads through an
    // empty descriptor, i.e. as zeros (a load under a branch would wait alone).
    // The start state: state0 (first segment), the segment's start state, the
    // identity columns (map mode) or zeros (map mode, value columns).
    const float* h0 = q.mode != 0 ? nullptr
                      : q.seg == 0 ? p.state0
                                   : p.hseg + static_cast<size_t>(q.seg - 1) * d.B * d.Hv * DK * d.Dv;
    const rsrc_t rs0 = make_rsrc(h0 ? static_cast<const void*>(h0 + sbase) : static_cast<const void*>(p.k),
                                 h0 ? static_cast<size_t>(DK) * d.Dv * 4 : 0);
    f32x4 H[RTW][2];
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * (q.w * RTW + it) + 4 * q.lg + r;
          H[it][ct][r] = buf_f1(rs0, 4 * static_cast<uint32_t>(i * d.Dv + q.col0 + 16 * ct + q.lr));
          if (q.mode == 1) H[it][ct][r] = i == q.scol + 16 * ct + q.lr ? 1.f : 0.f;
        }
    put_h(sm, q, H);
    // the bf16 start state of chunk cs: here for the first segment only; a
    // later segment's start slot is the previous segment's end state (written
    // by its last chunk, as the fp32 checkpoint of that boundary is)
    if (p.cb.Hb != nullptr && q.seg == 0) store_hb(p, q, H, 0);
    lds_barrier();  // 0
    for (int c = q.cs; c < q.ce; ++c) step_b(p, sm, q, c, H);
    store_states(p, q, H, q.ce - 1, true);  // the last chunk's end: the next segment's start
    store_x(p, sm, q, q.ce - 1, true);  // the last chunk's X (X^T is no longer rewritten)
    if (q.mode == 0 && q.ce < q.NC) return;  // not the last segment: no final state
    const int ostride = q.mode == 0 ? d.Dv : DK + d.Dv;
    float* out = q.mode == 0 ? p.state_out + sbase
                             : p.maps + (static_cast<size_t>(q.seg) * d.B * d.Hv + q.bh) * DK * ostride;
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * (q.w * RTW + it) + 4 * q.lg + r;
          out[static_cast<size_t>(i) * ostride + q.scol + 16 * ct + q.lr] = H[it][ct][r];
        }
  }

  __device__ static void run_c(const ChunkFwdArgs& p, Smem& sm, const Lane& q) {
    lds_barrier();  // 0: initial H
    if (q.mode != 0) {  // map mode: no outputs; keep the chunk's barriers
      for (int c = q.cs; c < q.ce; ++c) {
        lds_barrier();
        lds_barrier();
        lds_barrier();
      }
      return;
    }
    // Prefetch two chunks ahead through three register stages.  The loads are
    // unconditional, from a chunk index clamped to the segment's last chunk: a
    // load under a branch makes the compiler wait for every outstanding load
    // where the branch joins, which would void the prefetch.
    const int cl = q.ce - 1;
    StageC s0, s1, s2;
    load_c(p, q, q.cs, s0);
    load_c(p, q, min(q.cs + 1, cl), s1);
    for (int c = q.cs; c < q.ce; c += 3) {
      load_c(p, q, min(c + 2, cl), s2);
      step_c(p, sm, q, c, s0);
      if (c + 1 >= q.ce) break;
      load_c(p, q, min(c + 3, cl), s0);
      step_c(p, sm, q, c + 1, s1);
      if (c + 2 >= q.ce) break;
      load_c(p, q, min(c + 4, cl), s1);
      step_c(p, sm, q, c + 2, s2);
    }
  }

  __device__ static void run(const ChunkFwdArgs& p, Smem& sm) {
    const Dims& d = p.d;
    Lane q;
    const int nslice = (p.map ? DK + d.Dv : d.Dv) / NV;
    int slice;
    block_coords(d, nslice, q.b, q.h, slice);
    q.NC = d.nchunk();
    q.seg = blockIdx.y;
    q.cs = p.seg ? q.seg * p.seg : 0;
    q.ce = p.seg ? min(q.cs + p.seg, q.NC) : q.NC;
    q.mode = !p.map ? 0 : slice < DK / NV ? 1 : 2;
    q.j = q.h / d.G();
    q.bh = q.b * d.Hv + q.h;
    q.bj = q.b * d.Hk + q.j;
    q.scol = slice * NV;
    q.col0 = q.mode == 0 ? q.scol : q.mode == 1 ? 0 : q.scol - DK;  // v / o columns
    const int tid = threadIdx.x, l = tid & 63;
    q.w = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
    q.l = l;
    q.lr = l & 15;
    q.lg = l >> 4;
    q.ta = 16 * q.w + q.lr;
    q.tc0 = 16 * q.w + 4 * q.lg;
    q.last = d.T - 1;
    q.qk_row = d.Hk * DK;
    q.v_row = d.Hv * d.Dv;
    {
      const size_t bt = static_cast<size_t>(d.B) * d.T, nmat = static_cast<size_t>(d.B) * d.Hv * q.NC;
      if constexpr (VG) {
        q.dk = raw_desc(p.cb.Kb, nmat * L * DK * 2);
        q.dkh = raw_desc(p.cb.Kh, nmat * L * DK * 2);
        q.rq = make_rsrc(p.cb.Qb, nmat * L * DK * 2);
      } else {
        q.dk = q.dkh = raw_desc(p.k, bt * d.Hk * DK * 2);
        q.rq = make_rsrc(p.q, bt * d.Hk * DK * 2);
      }
      q.dv = q.mode == 1 ? raw_desc(p.vzero, 64) : raw_desc(p.v, bt * d.Hv * d.Dv * 2);
      q.vstep = q.mode == 1 ? 0u : static_cast<uint32_t>(d.Hv * d.Dv);
      q.vbase = q.mode == 1 ? 0u : static_cast<uint32_t>(q.h * d.Dv + q.col0);
      q.dtx = raw_desc(p.cb.Tx, nmat * L * L * 2);
      q.rmq = make_rsrc(p.cb.Mq, nmat * L * L * 2);
      q.dsc = VG ? raw_desc(p.cb.vsc, nmat * VSC_ROWS * L * 4) : raw_desc(p.cb.sc, nmat * SC_ROWS * L * 4);
    }
    if (q.ce <= q.cs) return;
    if (tid < 256)
      run_a(p, sm, q);
    else if (tid < 512)
      run_b(p, sm, q);
    else
      run_c(p, sm, q);
  }
};

template <int DK, bool VG, bool ST = false>
__global__ void __launch_bounds__(768) chunk_fwd_kernel(ChunkFwdArgs p) {
  __shared__ typename ChunkFwd<DK, VG, ST>::Smem sm;
  ChunkFwd<DK, VG, ST>::run(p, sm);
}

// ------------------------------------------------ T-parallel segment chain
//
// The chunked forward is an affine map per chunk, H -> A_c H + B_c (the
// associative form of the mlx-lm PR's "Associative prefix-scan scaffold"
// extension, with A_c = e^{gL} I - K^T diag(w) Tx diag(e^g rk) K and
// B_c = K^T diag(w) Tx V), and the composition of maps is associative.  The
// T-parallel forward composes the chunks of each segment in parallel (the
// chunk kernel's map mode) and chains only the segments here:
// H_{s+1} = A_s H_s + B_s, in fp32 on the matrix cores (16x16x4 f32).  One
// workgroup per (b, h, 16 columns of Dv) (the chain is bound by latency: more,
// smaller workgroups); wave w owns the output row tiles w, w + 4, ...; A is
// staged through LDS in blocks of 32 columns, the next block loaded while the
// current one is multiplied.
template <int DK>
struct SegChain {
  static constexpr int NTC = 256;
  static constexpr int NCOL = 16;           // columns of H per workgroup
  static constexpr int HSTR = 36;           // row stride of H (and of the A block)
  static constexpr int RT = DK / 16 / 4;    // row tiles per wave
  static constexpr int APT = DK * 32 / NTC; // A block floats per thread
  struct Smem {
    float h[DK * HSTR];
    float a[DK * HSTR];
  };

  __device__ static void load_a(const float* M, int W, int m0, float (&r)[APT]) {
#pragma unroll
    for (int n = 0; n < APT; ++n) {
      const int e = threadIdx.x + n * NTC, i = e / 32, m = e % 32;
      r[n] = M[static_cast<size_t>(i) * W + m0 + m];
    }
  }

  __device__ static void run(const SegChainArgs& p, Smem& sm) {
    const Dims& d = p.d;
    const int bh = blockIdx.x, c0 = blockIdx.y * NCOL;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    const size_t BH = static_cast<size_t>(d.B) * d.Hv;
    const int W = DK + d.Dv;
    for (int e = tid; e < DK * NCOL; e += NTC) {
      const int i = e / NCOL, c = e % NCOL;
      sm.h[i * HSTR + c] = p.state0 ? p.state0[(static_cast<size_t>(bh) * DK + i) * d.Dv + c0 + c] : 0.f;
    }
    // forward: maps 0 .. nseg - 2 give starts 0 .. nseg - 2 (of segments 1 ..);
    // reverse: maps nseg - 1 .. 1 give hseg nseg - 2 .. 0
    const int first = p.reverse ? p.nseg - 1 : 0, step = p.reverse ? -1 : 1;
    float ar[APT];
    load_a(p.maps + (static_cast<size_t>(first) * BH + bh) * DK * W, W, 0, ar);
    for (int s = 0; s + 1 < p.nseg; ++s) {
      const int ms = first + step * s, os = p.reverse ? ms - 1 : ms;
      const float* M = p.maps + (static_cast<size_t>(ms) * BH + bh) * DK * W;
      f32x4 acc[RT];
#pragma unroll
      for (int it = 0; it < RT; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[it][r] = M[static_cast<size_t>(16 * (w + 4 * it) + 4 * lg + r) * W + DK + c0 + lr];
      for (int m0 = 0; m0 < DK; m0 += 32) {
        __syncthreads();  // the previous block of A is consumed; H complete
#pragma unroll
        for (int n = 0; n < APT; ++n) {
          const int e = tid + n * NTC;
          sm.a[(e / 32) * HSTR + e % 32] = ar[n];
        }
        __syncthreads();
        // the next block: this step's next columns, or the next step's first
        if (m0 + 32 < DK)
          load_a(M, W, m0 + 32, ar);
        else if (s + 2 < p.nseg)
          load_a(M + step * static_cast<ptrdiff_t>(BH * DK * W), W, 0, ar);
#pragma unroll
        for (int it = 0; it < RT; ++it)
#pragma unroll
          for (int kk = 0; kk < 32; kk += 16)
            acc[it] = mm16f(acc[it], &sm.a[16 * (w + 4 * it) * HSTR + kk], HSTR, &sm.h[(m0 + kk) * HSTR], HSTR);
      }
      __syncthreads();  // every read of H done
      float* out = p.hseg + (static_cast<size_t>(os) * BH + bh) * DK * d.Dv;
#pragma unroll
      for (int it = 0; it < RT; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * (w + 4 * it) + 4 * lg + r;
          sm.h[i * HSTR + lr] = acc[it][r];
          out[static_cast<size_t>(i) * d.Dv + c0 + lr] = acc[it][r];
        }
    }
  }
};

template <int DK>
__global__ void __launch_bounds__(256) seg_chain_kernel(SegChainArgs p) {
  __shared__ typename SegChain<DK>::Smem sm;
  SegChain<DK>::run(p, sm);
}

__global__ void __launch_bounds__(256) fill_zero_kernel(float* p, size_t n) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += 256ull * gridDim.x) p[i] = 0.f;
}

}  // namespace

hipError_t launch_chunk_prep(const ChunkPrepArgs& a, hipStream_t st) {
  if (a.d.T == 0) return hipSuccess;
  dim3 grid(a.d.nchunk(), a.d.B * a.d.Hv);
  switch (a.d.Dk) {
    case 64: chunk_prep_kernel<64><<<grid, NT, 0, st>>>(a); break;
    case 128: chunk_prep_kernel<128><<<grid, NT, 0, st>>>(a); break;
    case 192: chunk_prep_kernel<192><<<grid, NT, 0, st>>>(a); break;
    case 256: chunk_prep_kernel<256><<<grid, NT, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_seg_chain(const SegChainArgs& a, hipStream_t st) {
  if (a.nseg < 2) return hipSuccess;
  const dim3 grid(a.d.B * a.d.Hv, a.d.Dv / SegChain<64>::NCOL);
  switch (a.d.Dk) {
    case 64: seg_chain_kernel<64><<<grid, 256, 0, st>>>(a); break;
    case 128: seg_chain_kernel<128><<<grid, 256, 0, st>>>(a); break;
    case 192: seg_chain_kernel<192><<<grid, 256, 0, st>>>(a); break;
    case 256: seg_chain_kernel<256><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t nb = (n + 255) / 256;
  fill_zero_kernel<<<static_cast<unsigned>(nb < 1024 ? nb : 1024), 256, 0, st>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkFwdArgs& a, hipStream_t st) {
  const int NV = ChunkFwd<64>::NV;
  const int nseg = a.seg ? (a.d.nchunk() + a.seg - 1) / a.seg : 1;
  const dim3 nblk(a.d.B * a.d.Hv * ((a.map ? a.d.Dk + a.d.Dv : a.d.Dv) / NV), nseg);
  if (a.vg) {
    if (a.seg || a.map) return hipErrorInvalidValue;
    switch (a.d.Dk) {
      case 64: chunk_fwd_kernel<64, true><<<nblk, ChunkFwd<64, true>::NTS, 0, st>>>(a); break;
      case 128: chunk_fwd_kernel<128, true><<<nblk, ChunkFwd<128, true>::NTS, 0, st>>>(a); break;
      case 192: chunk_fwd_kernel<192, true><<<nblk, ChunkFwd<192, true>::NTS, 0, st>>>(a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
#define GDN_FWD_CASE(D)                                                      \
  case D:                                                                    \
    if (a.stream)                                                            \
      chunk_fwd_kernel<D, false, true><<<nblk, ChunkFwd<D>::NTS, 0, st>>>(a);  \
    else                                                                     \
      chunk_fwd_kernel<D, false, false><<<nblk, ChunkFwd<D>::NTS, 0, st>>>(a); \
    break;
  switch (a.d.Dk) {
    GDN_FWD_CASE(64)
    GDN_FWD_CASE(128)
    GDN_FWD_CASE(192)
    GDN_FWD_CASE(256)
    default: return hipErrorInvalidValue;
  }
#undef GDN_FWD_CASE
  return hipGetLastError();
}

}  // namespace gdn
