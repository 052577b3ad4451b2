// Chunked (matrix) form of the gated delta rule backward on gfx950 bf16 MFMA.
//
// Per chunk of L = 64 steps (local t, H = state at the chunk start, dH' =
// dL/d(state at the chunk end), gamma_t = l_0 + ... + l_t, X_t = v_t - u_t,
// delta_t = beta_t X_t, eps_t = dL/d delta_t), the per-step backward of the
// recurrence (mlx-lm VJP PR, "What this PR adds": the reverse pass carrying
// dL/dS) unrolls to
//   eps  = rhs - A^T Ehat,   Ehat = Tx^T diag(beta) rhs  (= dv),
//   rhs  = diag(e^{gL-g} rk) K dH' + P^T dO,
//   dH   = e^{gL} dH' + Q^T diag(e^g rq) dO - K^T diag(e^g rk) Ehat,
// with A[r,t] = [t<r] e^{g_r-g_t} kn_r.kn_t, P[r,t] = [t<=r] e^{g_r-g_t}
// qn_r.kn_t and Tx = (I + A diag(beta))^-1 (Tx^T inverts the transposed
// system).  Derivation: dL/dS before step t's output term is
// e^{gL-g_t} dH' + sum_{r>t} e^{g_r-g_t} (qn_r dO_r^T - beta_r kn_r eps_r^T),
// and eps_t is its product with kn_t plus (qn_t . kn_t) dO_t.
//
// The per-chunk gradients (same expansion as the scan path's chunk assembly),
// written with dv = diag(beta) eps: eps enters every term with a beta factor
// (delta_t = beta_t X_t and X_t does not depend on beta_t), so the gradient
// pass reads the dv output and no eps buffer is kept:
//   dQn = diag(e^g) dO H^T + Wq Kn
//   dKn = diag(e^{gL-g} beta) X dH'^T - diag(e^g) dv H^T + Wk1 Qn + Wk2 Kn
//   Wq[t,s]  = [s<=t] e^{g_t-g_s} beta_s (dO_t . X_s)
//   Wk1[t,r] = [r>=t] e^{g_r-g_t} beta_t (dO_r . X_t)
//   Wk2[t,s] = -([s<t] e^{g_t-g_s} beta_s (X_s . dv_t) + [s>t] e^{g_s-g_t} beta_t (X_t . dv_s))
//   dl_t = e^{gL} <dH', H> + sum_{s<t} a_s + sum_{r>=t} b_r
//          + sum_{r>=t} sum_{s<t} e^{g_r-g_s} beta_s [(qn_r.kn_s)(dO_r.X_s) - (kn_r.kn_s)(dv_r.X_s)]
//   a_s = e^{gL-g_s} beta_s kn_s^T dH' X_s,  b_r = e^{g_r} (qn_r^T H dO_r - kn_r^T H dv_r)
//   db_t = (dv_t . X_t) (1 - beta_t)   (dL/dbeta_t = eps_t . X_t, dbeta/db = beta (1 - beta))
// with X the forward's saved copy, or recomputed from the checkpointed H as in
// the forward when there is no saved record.  Every decay is
// e^{-|g_t - g_s|}; nothing is divided by a decay.
//
// Kernels:
//   chunk_bwd_state  one workgroup per (batch, value head, 32-column slice of
//                    Dv), walking the chunks from last to first with dH in MFMA
//                    accumulators (fp32) and the next chunk's operands
//                    prefetched.  Writes dv, dH' of every chunk (bf16,
//                    transposed) and dstate.
//   chunk_bwd_grad   one workgroup per (chunk, batch, key head), looping over
//                    the group's value heads and 32-column slabs of Dv, with H
//                    read from the bf16 copies of the chunk-start states and
//                    X from the forward's saved copy (else recomputed).
//                    Writes dq, dk (after the L2-normalisation backward), da,
//                    db and the per-chunk parameter sums.  Fixed summation
//                    order throughout; no atomics.
//   state_bf16       the bf16 copies of the chunk-start states from fp32
//                    checkpoints (when the forward did not write them).
#include <algorithm>
#include <type_traits>

#include "gdn_dev.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int L = kChunk;

// ------------------------------------------------------- reverse state pass

// ST: dH' is stored non-temporal (ChunkBwdArgs::stream).
template <int DK, bool VG = false, bool ST = false>
struct ChunkBwdState {
  // Eight waves in two groups of four (w = wave index within the group):
  //   A (waves 0-3): for row tile w of the chunk, the dependent chain
  //                  rhs = diag(e^{gL-g} rk) K dH' + P^T dO, Ehat = Tx^T diag(beta) rhs
  //                  (= dv).  A also streams the chunk's k rows, P^T, Tx^T,
  //                  dO slice and chunk scalars into a
  //                  2-slot LDS ring with direct-to-LDS loads, one chunk ahead.
  //   B (waves 4-7): dH for its RTW row tiles, in MFMA accumulators: stores dH'
  //                  of the chunk, adds e^{gL} dH' + Q^T diag(e^g rq) dO while A
  //                  works (it does not depend on Ehat), then - K^T diag(e^g rk)
  //                  Ehat with K^T read transposed from the ring.
  // Three barriers per chunk: Y (rhs ready), Z (Ehat ready), X (dH of the
  // previous chunk ready, next ring slot complete).
  // With the per-key-channel gate (VG) the operands come pre-scaled from
  // vg_chunk_prep: the ring's k tile holds Kh (rhs = Kh dH' + P^T dO), B
  // takes Qb^T and Kb^T from registers (dH = diag(e^{G_L}) dH' + Qb^T dO -
  // Kb^T Ehat) and decays dH row-wise.
  static constexpr int NTS = 512;
  static constexpr int NV = 32;        // Dv columns per workgroup
  static constexpr int RTW = DK / 64;  // dH row tiles per group-B wave
  static constexpr int HS = DK + 8;    // bf16 row stride of dH^T
  static constexpr int XS = L + 8;     // bf16 row stride of the [v][t] tiles
  static constexpr int NPK = DK / 8;   // 16-byte pieces of a k row
  static constexpr int KDMA = DK / 32;
  static constexpr int NDMA = KDMA + 4 + 1 + 2;  // ring loads per group-A wave per chunk
  static constexpr int SCR = VG ? VSC_ROWS : SC_ROWS;  // chunk scalar rows per chunk
  static_assert(!VG || DK <= 4 * L, "e^{G_L} of every channel in rows 1 .. 4 of the slot");
  // A ring slot (layouts as in the forward state pass: 16-byte piece p of row
  // t at t * (pieces per row) + (p ^ swizzle(t))).
  struct Slot {
    bf16 k[L * DK];    // k rows, swizzle t & 7
    bf16 pt[L * L];    // P^T rows, swizzle t & 7
    bf16 tx[L * L];    // Tx rows, swizzle t & 7 (Tx^T operands by transposing reads)
    bf16 dO[L * NV];   // dO rows of this slice's columns, swizzle t & 3
    float sc[8 * L];   // chunk scalar rows 0 .. 7
  };
  static_assert(SC_CR < 8 && SC_CO < 8 && SC_EGL < 8 && SC_KL < 8 && SC_BETA < 8, "rows held in a ring slot");
  struct Smem {
    alignas(16) Slot ring[2];
    alignas(16) bf16 hb[NV * HS];   // dH'^T, the B operand of K dH'
    alignas(16) bf16 rb[NV * XS];   // (diag(beta) rhs)^T
    alignas(16) bf16 eb[NV * XS];   // Ehat^T
    alignas(16) bf16 es[NV * XS];   // -(diag(e^g rk) Ehat)^T
  };
  // Group B's Q^T operand of one chunk, in registers (quad-coalesced loads,
  // permuted at use), loaded a chunk ahead from clamped addresses.
  struct StageB {
    bf16x8 qta[RTW][2];            // Q^T (VG: Qb^T) rows i = 16 (w RTW + it) + lr
    bf16x8 kta[VG ? RTW : 1][2];   // VG: Kb^T rows i
  };
  struct Lane {
    int b, h, j, bh, bj, col0, w, l, lr, lg, ta, tc0, last, NC;
    int cs, ce, seg, mode;       // chunk range of the segment; 0 output, 1 map identity, 2 map values
    int scol;                    // first state column of the slice (Dk + Dv columns in map mode)
    uint32_t ostep, obase;       // dO elements per step and offset (0, 0: the zero rows)
    uint32_t v_row;
    rsrc_t rqt, rkt;
    i32x4 dk, dpt, dtx, ddo, dsc;  // raw descriptors of the ring's operands
  };

  __device__ static __forceinline__ int kpos(int t, int p) { return 8 * (t * NPK + (p ^ (t & 7))); }
  __device__ static __forceinline__ int xpos(int t, int p) { return 8 * (t * 8 + (p ^ (t & 7))); }
  __device__ static __forceinline__ int vpos(int t, int p) { return 8 * (t * 4 + (p ^ (t & 3))); }

  // Group A: the NDMA ring loads of this wave for chunk c into slot sl.
  __device__ static void issue_ring(const ChunkBwdArgs& p, Smem& sm, const Lane& q, int c, int sl) {
    const Dims& d = p.d;
    const int t0 = c * L, tl = q.last - t0, l = q.l;
    Slot& s = sm.ring[sl];
#pragma unroll
    for (int jj = 0; jj < KDMA; ++jj) {
      const int n = KDMA * q.w + jj, pos = 64 * n + l, t = pos / NPK, pc = (pos % NPK) ^ (t & 7);
      const uint32_t o = VG ? 2 * ((static_cast<uint32_t>(q.bh * q.NC + c) * L + t) * DK + 8 * pc)
                            : 2 * ((static_cast<uint32_t>(q.b * d.T + t0 + min(t, tl)) * d.Hk + q.j) * DK + 8 * pc);
      dma16(q.dk, &s.k[512 * n], o);
    }
    const uint32_t mat = static_cast<uint32_t>(q.bh * q.NC + c) * L * L;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int n = 2 * q.w + jj, pos = 64 * n + l, t = pos / 8, pc = (pos % 8) ^ (t & 7);
      const uint32_t o = 2 * (mat + t * L + 8 * pc);
      dma16(q.dpt, &s.pt[512 * n], o);
      dma16(q.dtx, &s.tx[512 * n], o);
    }
    {
      const int pos = 64 * q.w + l, t = pos / 4, pc = (pos % 4) ^ (t & 3);
      dma16(q.ddo, &s.dO[512 * q.w],
            2 * (static_cast<uint32_t>(q.b * d.T + t0 + min(t, tl)) * q.ostep + q.obase + 8 * pc));
    }
    const uint32_t so = static_cast<uint32_t>(q.bh * q.NC + c) * SCR * L;
#pragma unroll
    for (int e = 0; e < 2; ++e) dma4(q.dsc, &s.sc[L * (2 * q.w + e)], 4 * (so + L * (2 * q.w + e) + l));
  }

  __device__ static void load_b(const ChunkBwdArgs& p, const Lane& q, int c, StageB& st) {
    (void)p;
    const uint32_t o = 2 * (static_cast<uint32_t>((VG ? q.bh : q.bj) * q.NC + c) * DK * L +
                            (16 * q.w * RTW + coal_row(q.l)) * L + 8 * coal_piece(q.l));
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        st.qta[it][kt] = buf_bf16x8(q.rqt, o + 2 * (it * 16 * L) + 64 * kt);
        if constexpr (VG) st.kta[it][kt] = buf_bf16x8(q.rkt, o + 2 * (it * 16 * L) + 64 * kt);
      }
  }

  // The B operand of a product with dO^T over the chunk's steps: steps
  // 32 kt + 8 lg .. + 7 of column 16 ct + lr, read transposed from the ring.
  __device__ static __forceinline__ uint4 dO_operand(const Slot& s, const Lane& q, int kt, int ct) {
    const int t = 32 * kt + 8 * q.lg + (q.lr >> 2), pc = 2 * ct + ((q.lr >> 1) & 1), sub = 4 * (q.lr & 1);
    const uint2 lo = lds_read_tr16(&s.dO[vpos(t, pc) + sub]);
    const uint2 hi = lds_read_tr16(&s.dO[vpos(t + 4, pc) + sub]);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }

  __device__ static void put_h(Smem& sm, const Lane& q, const f32x4 (&H)[RTW][2]) {
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        *reinterpret_cast<uint2*>(&sm.hb[(16 * ct + q.lr) * HS + 16 * (q.w * RTW + it) + 4 * q.lg]) =
            pack4_bf16(H[it][ct][0], H[it][ct][1], H[it][ct][2], H[it][ct][3]);
  }

  // dv / eps rows of this wave: a transpose inside each quad of lanes gives
  // every lane 4 consecutive columns of one step, and a lane move puts one
  // step's 4 column groups in each quad (coalesced stores); steps past the end
  // of the sequence fall outside the descriptor and are dropped.
  __device__ static void store_rows(const ChunkBwdArgs& p, const Lane& q, void* dst, int t0, int Lc,
                                    const f32x4 (&x)[2], float sign) {
    const Dims& d = p.d;
    const rsrc_t r = make_rsrc(static_cast<bf16*>(dst) + ((static_cast<size_t>(q.b) * d.T + t0) * d.Hv + q.h) * d.Dv,
                               q.mode == 0 ? (static_cast<size_t>(Lc - 1) * q.v_row + d.Dv) * 2 : 0);
    const uint32_t o = 2 * (static_cast<uint32_t>(q.tc0 + (q.lr >> 2)) * q.v_row + q.col0 + 4 * (q.lr & 3));
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const f32x4 tr = quad_transpose(x[ct]);
      buf_store_u2(r, o + 32 * ct, quads_to_rows(pack4_bf16(sign * tr[0], sign * tr[1], sign * tr[2], sign * tr[3])));
    }
  }

  // Group A, one chunk (chunks run last to first).  The slot refilled here
  // (chunk c - 1) was last read before barrier X of the previous chunk; before
  // barrier X of this chunk each wave waits for its ring loads (its 4 later
  // stores may stay pending), so the slot is complete for every wave after X.
  __device__ static void step_a(const ChunkBwdArgs& p, Smem& sm, const Lane& q, int c) {
    issue_ring(p, sm, q, max(c - 1, q.cs), (c - 1) & 1);
    const Dims& d = p.d;
    const int t0 = c * L, Lc = min(L, d.T - t0);
    const Slot& s = sm.ring[c & 1];
    const int lr = q.lr, lg = q.lg, ta = q.ta;
    bf16x8 ka[DK / 32], pqa[2], txa[2];
#pragma unroll
    for (int kt = 0; kt < DK / 32; ++kt) ka[kt] = load_bf16x8(&s.k[kpos(ta, 4 * kt + lg)]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      pqa[kt] = load_bf16x8(&s.pt[xpos(ta, 4 * kt + lg)]);
      // row ta of Tx^T: column ta of rows 32 kt + 8 lg .. + 7 of Tx, by two
      // transposing reads of four rows each
      const int sr = 32 * kt + 8 * lg + (lr >> 2), pc = 2 * q.w + ((lr >> 1) & 1);
      const uint2 lo = lds_read_tr16(&s.tx[xpos(sr, pc) + 4 * (lr & 1)]);
      const uint2 hi = lds_read_tr16(&s.tx[xpos(sr + 4, pc) + 4 * (lr & 1)]);
      txa[kt] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
    const float4 one4 = make_float4(1.f, 1.f, 1.f, 1.f);
    const float4 kl4 = VG ? one4 : *reinterpret_cast<const float4*>(&s.sc[SC_KL * L + q.tc0]);
    const float4 bt4 = *reinterpret_cast<const float4*>(&s.sc[(VG ? VSC_BETA : SC_BETA) * L + q.tc0]);
    const float4 cr4 = VG ? one4 : *reinterpret_cast<const float4*>(&s.sc[SC_CR * L + q.tc0]);
    const float klv[4] = {kl4.x, kl4.y, kl4.z, kl4.w};
    const float btv[4] = {bt4.x, bt4.y, bt4.z, bt4.w};
    const float crv[4] = {cr4.x, cr4.y, cr4.z, cr4.w};
    // rhs = diag(e^{gL-g} rk) K dH' + P^T dO for row tile w
    f32x4 kdh[2], rhs[2];
    kdh[0] = kdh[1] = rhs[0] = rhs[1] = f4zero();
#pragma unroll
    for (int kt = 0; kt < DK / 32; ++kt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        kdh[ct] = mfma16(ka[kt], load_bf16x8(&sm.hb[(16 * ct + lr) * HS + 32 * kt + 8 * lg]), kdh[ct]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) rhs[ct] = mfma16(pqa[kt], as_bf16x8(dO_operand(s, q, kt, ct)), rhs[ct]);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int r = 0; r < 4; ++r) rhs[ct][r] += klv[r] * kdh[ct][r];
      *reinterpret_cast<uint2*>(&sm.rb[(16 * ct + lr) * XS + q.tc0]) =
          pack4_bf16(btv[0] * rhs[ct][0], btv[1] * rhs[ct][1], btv[2] * rhs[ct][2], btv[3] * rhs[ct][3]);
    }
    lds_barrier();  // Y: diag(beta) rhs complete
    // Ehat = Tx^T diag(beta) rhs  (= dv)
    f32x4 eh[2];
    eh[0] = eh[1] = f4zero();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        eh[ct] = mfma16(txa[kt], load_bf16x8(&sm.rb[(16 * ct + lr) * XS + 32 * kt + 8 * lg]), eh[ct]);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      *reinterpret_cast<uint2*>(&sm.eb[(16 * ct + lr) * XS + q.tc0]) =
          pack4_bf16(eh[ct][0], eh[ct][1], eh[ct][2], eh[ct][3]);
      *reinterpret_cast<uint2*>(&sm.es[(16 * ct + lr) * XS + q.tc0]) =
          pack4_bf16(-crv[0] * eh[ct][0], -crv[1] * eh[ct][1], -crv[2] * eh[ct][2], -crv[3] * eh[ct][3]);
    }
    lds_barrier();  // Z: Ehat complete
    store_rows(p, q, p.dv, t0, Lc, eh, 1.f);
    // eps = rhs - A^T Ehat is not formed: the gradient kernels take every eps
    // term times beta, i.e. read dv = diag(beta) eps
    wait_vm<2>();  // the ring loads (the 2 later stores may stay pending)
    lds_barrier();  // X: dH of the next chunk complete; slot c - 1 complete
  }

  // Group B, one chunk, with Q^T of chunk cn loaded into nxt (a chunk ahead).
  __device__ static void step_b(const ChunkBwdArgs& p, Smem& sm, const Lane& q, int c, StageB& cur,
                                f32x4 (&dH)[RTW][2], StageB& nxt, int cn) {
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        cur.qta[it][kt] = to_mfma_layout(cur.qta[it][kt]);
        if constexpr (VG) cur.kta[it][kt] = to_mfma_layout(cur.kta[it][kt]);
      }
    const Dims& d = p.d;
    const int lr = q.lr, lg = q.lg;
    const Slot& s = sm.ring[c & 1];
    // dH' of this chunk for the gradient pass, bf16 (the hand-off layout, or
    // row-major [i][v] with the per-key-channel gate); a transpose inside each
    // quad of lanes gives every lane 4 consecutive columns of one row, and
    // quads_to_rows one row per quad (coalesced stores).  Packed now, stored after barrier Z:
    // stores issued here would wait behind group A's ring loads and hold up
    // the products below.
    uint2 dhp[RTW][2];
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const f32x4 tr = quad_transpose(dH[it][ct]);
        dhp[it][ct] = pack4_bf16(tr[0], tr[1], tr[2], tr[3]);
      }
    // dH <- e^{gL} dH' + Q^T diag(e^g rq) dO (the operand scaled by e^g rq per step)
    const float egl = s.sc[SC_EGL * L];
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // VG: e^{G_L} of row i = 16 (w RTW + it) + 4 lg + r
        const float e = VG ? s.sc[VSC_EGL * L + 16 * (q.w * RTW + it) + 4 * lg + r] : egl;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) dH[it][ct][r] *= e;
      }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float cov[8];
      if constexpr (!VG) {
        const float4 c0 = *reinterpret_cast<const float4*>(&s.sc[SC_CO * L + 32 * kt + 8 * lg]);
        const float4 c1 = *reinterpret_cast<const float4*>(&s.sc[SC_CO * L + 32 * kt + 8 * lg + 4]);
        cov[0] = c0.x, cov[1] = c0.y, cov[2] = c0.z, cov[3] = c0.w;
        cov[4] = c1.x, cov[5] = c1.y, cov[6] = c1.z, cov[7] = c1.w;
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const uint4 u = dO_operand(s, q, kt, ct);
        bf16x8 bq;
        if constexpr (VG) {
          bq = as_bf16x8(u);  // Qb^T already carries e^{G_t} / sqrt(Dk)
        } else {
          const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
          uint32_t o4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o4[i] = pack2_bf16(cov[2 * i] * __uint_as_float(w4[i] << 16), cov[2 * i + 1] * __uint_as_float(w4[i] & 0xffff0000u));
          bq = as_bf16x8(make_uint4(o4[0], o4[1], o4[2], o4[3]));
        }
#pragma unroll
        for (int it = 0; it < RTW; ++it) dH[it][ct] = mfma16(cur.qta[it][kt], bq, dH[it][ct]);
      }
    }
    lds_barrier();  // Y
    load_b(p, q, cn, nxt);  // the next chunk's Q^T, issued while waiting for Ehat
    lds_barrier();  // Z: Ehat complete
    {  // map mode: an empty descriptor, nothing stored.  Non-temporal under
       // ST (the hand-off does not fit the memory-side cache):
       // only the gradient pass reads dH', after this kernel, and dirty lines
       // held in the caches then cost this chain more than that pass gains
      const rsrc_t rdh = make_rsrc(p.dHend + (static_cast<size_t>(c) * d.B * d.Hv + q.bh) * DK * d.Dv,
                                   q.mode == 0 ? static_cast<size_t>(DK) * d.Dv * 2 : 0);
      // the scalar gate's hand-off layout (hand_off); row-major [i][v] blocks
      // for the per-key-channel gate
      const int r16 = 4 * lg + (lr >> 2), c4 = 4 * (lr & 3);
      const uint32_t o = VG ? 2 * (static_cast<uint32_t>(16 * q.w * RTW + r16) * d.Dv + q.col0 + c4)
                            : 2 * hand_off(DK, 16 * q.w * RTW + r16, q.col0 + c4);
#pragma unroll
      for (int it = 0; it < RTW; ++it)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const uint32_t ot = o + 2 * (VG ? static_cast<uint32_t>(16 * it) * d.Dv + 16 * ct : 512 * it + 256 * ct);
          if constexpr (ST)
            buf_store_u2_nt(rdh, ot, quads_to_rows(dhp[it][ct]));
          else
            buf_store_u2(rdh, ot, quads_to_rows(dhp[it][ct]));
        }
    }
    // dH -= K^T diag(e^g rk) Ehat, K^T read transposed from the ring's k tile
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      bf16x8 be[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) be[ct] = load_bf16x8(&sm.es[(16 * ct + lr) * XS + 32 * kt + 8 * lg]);
#pragma unroll
      for (int it = 0; it < RTW; ++it) {
        bf16x8 kta;
        if constexpr (VG) {
          kta = cur.kta[it][kt];  // Kb^T (es holds -Ehat^T)
        } else {
          const int t = 32 * kt + 8 * lg + (lr >> 2), pc = 2 * (q.w * RTW + it) + ((lr >> 1) & 1);
          const uint2 lo = lds_read_tr16(&s.k[kpos(t, pc) + 4 * (lr & 1)]);
          const uint2 hi = lds_read_tr16(&s.k[kpos(t + 4, pc) + 4 * (lr & 1)]);
          kta = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) dH[it][ct] = mfma16(kta, be[ct], dH[it][ct]);
      }
    }
    put_h(sm, q, dH);
    lds_barrier();  // X
  }

  __device__ static void run_a(const ChunkBwdArgs& p, Smem& sm, const Lane& q) {
    issue_ring(p, sm, q, q.ce - 1, (q.ce - 1) & 1);
    wait_vm<0>();
    lds_barrier();  // X: initial dH; first slot complete
    for (int c = q.ce - 1; c >= q.cs; --c) step_a(p, sm, q, c);
    wait_vm<0>();  // no direct-to-LDS load may land after the workgroup ends
  }

  __device__ static void run_b(const ChunkBwdArgs& p, Smem& sm, const Lane& q) {
    const Dims& d = p.d;
    const size_t sbase = static_cast<size_t>(q.bh) * DK * d.Dv;
    // dH: rows i = 16 (w RTW + it) + 4 lg + r, columns col0 + 16 ct + lr.
    // Unconditional buffer loads; an absent dS_final reads through an empty
    // descriptor, i.e. as zeros (a load under a branch would wait alone).
    // The start: dS_final (last segment), dL/d the state at the segment's end
    // (other segments), the identity columns (map mode) or zeros (map mode,
    // value columns).
    const int nseg = gridDim.y;
    const float* h0 = q.mode != 0 ? nullptr
                      : q.seg == nseg - 1 ? p.dS_final
                                          : p.hseg + static_cast<size_t>(q.seg) * d.B * d.Hv * DK * d.Dv;
    const rsrc_t rsf = make_rsrc(h0 ? static_cast<const void*>(h0 + sbase) : static_cast<const void*>(p.k),
                                 h0 ? static_cast<size_t>(DK) * d.Dv * 4 : 0);
    f32x4 dH[RTW][2];
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * (q.w * RTW + it) + 4 * q.lg + r;
          dH[it][ct][r] = buf_f1(rsf, 4 * static_cast<uint32_t>(i * d.Dv + q.col0 + 16 * ct + q.lr));
          if (q.mode == 1) dH[it][ct][r] = i == q.scol + 16 * ct + q.lr ? 1.f : 0.f;
        }
    put_h(sm, q, dH);
    StageB s0, s1;
    load_b(p, q, q.ce - 1, s0);
    lds_barrier();  // X
    // The prefetches are unconditional, from a chunk index clamped to the
    // segment's first chunk: a load under a branch makes the compiler wait for
    // every outstanding load where the branch joins, which would void the
    // prefetch.
    for (int c = q.ce - 1; c >= q.cs; c -= 2) {
      step_b(p, sm, q, c, s0, dH, s1, max(c - 1, q.cs));
      if (c < q.cs + 1) break;
      step_b(p, sm, q, c - 1, s1, dH, s0, max(c - 2, q.cs));
    }
    if (q.mode == 0 && q.cs > 0) return;  // not the first segment: no dstate
    const int ostride = q.mode == 0 ? d.Dv : DK + d.Dv;
    float* out = q.mode == 0 ? p.dstate + sbase
                             : p.maps + (static_cast<size_t>(q.seg) * d.B * d.Hv + q.bh) * DK * ostride;
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * (q.w * RTW + it) + 4 * q.lg + r;
          out[static_cast<size_t>(i) * ostride + q.scol + 16 * ct + q.lr] = dH[it][ct][r];
        }
  }

  __device__ static void run(const ChunkBwdArgs& p, Smem& sm) {
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
    q.col0 = q.mode == 0 ? q.scol : q.mode == 1 ? 0 : q.scol - DK;  // dO / dv / eps columns
    q.ostep = q.mode == 1 ? 0u : static_cast<uint32_t>(d.Hv * d.Dv);
    q.obase = q.mode == 1 ? 0u : static_cast<uint32_t>(q.h * d.Dv + q.col0);
    const int tid = threadIdx.x, l = tid & 63;
    q.w = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
    q.l = l;
    q.lr = l & 15;
    q.lg = l >> 4;
    q.ta = 16 * q.w + q.lr;
    q.tc0 = 16 * q.w + 4 * q.lg;
    q.last = d.T - 1;
    q.v_row = d.Hv * d.Dv;
    {
      const size_t bt = static_cast<size_t>(d.B) * d.T, nmat = static_cast<size_t>(d.B) * d.Hv * q.NC;
      q.dk = VG ? raw_desc(p.cb.Kh, nmat * L * DK * 2) : raw_desc(p.k, bt * d.Hk * DK * 2);
      q.ddo = q.mode == 1 ? raw_desc(p.vzero, 64) : raw_desc(p.dO, bt * d.Hv * d.Dv * 2);
      q.dpt = raw_desc(p.cb.PqT, nmat * L * L * 2);
      q.dtx = raw_desc(p.cb.Tx, nmat * L * L * 2);
      if constexpr (VG) {
        q.dsc = raw_desc(p.cb.vsc, nmat * VSC_ROWS * L * 4);
        q.rqt = make_rsrc(p.cb.QbT, nmat * DK * L * 2);
        q.rkt = make_rsrc(p.cb.KbT, nmat * DK * L * 2);
      } else {
        q.dsc = raw_desc(p.cb.sc, nmat * SC_ROWS * L * 4);
        q.rqt = q.rkt = make_rsrc(p.cb.QT, static_cast<size_t>(d.B) * d.Hk * q.NC * DK * L * 2);
      }
    }
    if (q.ce <= q.cs) return;
    if (tid < 256)
      run_a(p, sm, q);
    else
      run_b(p, sm, q);
  }
};

template <int DK, bool VG, bool ST = false>
__global__ void __launch_bounds__(512) chunk_bwd_state_kernel(ChunkBwdArgs p) {
  __shared__ typename ChunkBwdState<DK, VG, ST>::Smem sm;
  ChunkBwdState<DK, VG, ST>::run(p, sm);
}

// ------------------------------------------------------------ gradient pass

constexpr int NTG = 512;  // threads of a gradient-pass workgroup (8 waves)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
// Sum over the 8 lanes of a half DPP row (lanes 8k .. 8k+7); every lane of
// the group ends with the same bits.
__device__ __forceinline__ float oct_sum(float v) {
  v = quad_sum(v);
  return v + dpp<kRowHalfMirror>(v);
}

// XSV: X comes from the forward's saved copy (ChunkBufs::X) instead of being
// recomputed as Tx (V - diag(e^g rk) K H); both variants use X in bf16, so
// they give the same bits when the saved X is the recomputed one.
template <int DK, bool XSV>
struct ChunkBwdGrad {
  static constexpr int NS = 32;          // Dv columns per slab
  static constexpr int IT = DK / 16;     // 16-row tiles of Dk
  static constexpr int IH = IT / 2;      // tiles of Dk per wave
  static constexpr int KS = DK / 32;     // MFMA steps over Dk
  static constexpr int VS = NS + 8;      // bf16 row stride of the recomputed X tiles
  static constexpr int TS = L + 8;       // bf16 row stride of [v][t] tiles and Wq rows
  static constexpr int WS = 2 * L + 8;   // bf16 row stride of [Wk1 | Wk2] rows
  static constexpr int FS = DK + 4;      // fp32 row stride of the final accumulators
  // The slabs (value head, 32 columns) stream through a ring of NSLOT LDS
  // slots, filled by direct-to-LDS loads issued PD = NSLOT - 1 slabs ahead of
  // their use: one barrier per slab, and the loads of the next PD slabs stay
  // in flight across the per-head sections.  Three slots (two slabs ahead)
  // where they fit in LDS.
  static constexpr int NSLOT = (XSV && DK <= 192) ? 3 : 2;
  static constexpr int PD = NSLOT - 1;
  static constexpr int HJ = DK / 16;       // 1 KB loads of one H or dH' slab (DK rows x 64 bytes)
  static constexpr int NJ = 2 * HJ + 12;   // loads of one slab: H, dH' and three 64 x 32 tiles
  static constexpr int JW = (NJ + 7) / 8;  // loads per wave (waves >= NJ % 8 issue one fewer)
  static constexpr int JR = NJ % 8 == 0 ? 8 : NJ % 8;  // waves that issue JW loads
  // One ring slot.  Rows of 64 bytes (4 pieces of 16 bytes); piece p of row i
  // sits at 4 i + (p ^ sw(i)), which keeps the 16-byte operand reads of 8
  // consecutive rows and the transposing reads of 4 rows x 2 pieces free of
  // bank conflicts.
  struct Slot {
    bf16 hv[DK * NS];    // H   [i][v]
    bf16 dhv[DK * NS];   // dH' [i][v]
    bf16 vt[3][L * NS];  // X (or v), dO, dv of the slab   [t][v]
  };
  struct XRec {          // X recomputed from v (no saved copy)
    bf16 rt[NS * TS];    // R   [v][t]
    bf16 xr[L * VS];     // X   [t][v]
    bf16 xs[L * VS];     // diag(e^{gL-g} beta) X   [t][v]
  };
  struct Ring {
    Slot s[NSLOT];
    std::conditional_t<XSV, int, XRec> xrec;
  };
  struct Wts {
    bf16 wq[L * TS];    // sum over the group of Wq diag(rk)   [t][s]
    bf16 wk[L * WS];    // sum over the group of [Wk1 diag(rq) | Wk2 diag(rk)]   [t][r]
  };
  static constexpr int KQS = DK + 8;  // bf16 row stride of the k / q row tiles
  struct KQ {
    bf16 k[L * KQS];  // the chunk's k rows   [t][i]
    bf16 q[L * KQS];  // the chunk's q rows   [t][i]
  };
  // dQn and dKn go through LDS for the L2-norm backward together where both
  // fit in the space of the ring (else one after the other)
  static constexpr int NFIN = 2 * L * FS * 4 <= (sizeof(Ring) > sizeof(KQ) ? sizeof(Ring) : sizeof(KQ)) ? 2 : 1;
  struct Fin {
    float acc[NFIN][L * FS];
  };
  // The start stages the chunk's k rows in the weight tiles' space and its q
  // rows in ring slot 2 where both fit (else each wave loads its rows itself).
  static constexpr bool KQL = NSLOT == 3 && L * KQS * 2 <= sizeof(Wts) && L * KQS * 2 <= sizeof(Slot);
  union Big {
    Ring r;
    KQ kq;
    Fin f;
  };
  static constexpr int HB = 4;  // value heads per batch of the deferred gate-gradient section (one wave each)
  struct Smem {
    alignas(16) Big u;
    alignas(16) Wts wt;  // bf16 group sums of the L x L weights, for the final products
    alignas(16) float rk[L];
    alignas(16) float rq[L];
    // per value head of a batch (slot = head % HB): the partial sums of its
    // gate-gradient terms -- b_r and a_s per half of the columns, the db
    // factor, the row sums (per half of the columns) and column sums (per row
    // tile) of E, <dH', H> per wave -- combined in the batch's deferred section
    float bv[HB][2][L], pa[HB][2][L], pdb[HB][2][L];
    float rowp[HB][2][L], colp[HB][4][L];
    float red[HB][NTG / 64];
    // per value head of a batch, loaded when the batch starts: the per-step
    // gamma, e^g, e^{gL-g}, beta and l, the scalars e^{gamma_L}, A_log and
    // dt_bias, a (fp32) and the mask (1 = valid step)
    alignas(16) float bsc[HB][5][L];  // rows: gamma, e^g, e^{gL-g}, beta, l (0 past the end)
    float hegl[HB], hal[HB], hdt[HB];
    float ha[HB][L], hm[HB][L];
  };
  struct Ctx {
    int b, j, c, NC, G, t0, Lc, tl;
    uint32_t v_row;
  };

  __device__ static __forceinline__ int sw(int i) { return (i & 2) | ((i >> 2) & 1); }
  // element offset of piece p of row i in a ring tile
  __device__ static __forceinline__ int rpos(int i, int p) { return 8 * (4 * i + (p ^ sw(i))); }

  // This wave's direct-to-LDS loads of slab n (value head j G + n / nsl,
  // columns 32 (n % nsl) ..) into ring slot n % NSLOT.  Load jb of the slab
  // (wave jb % 8) covers 64 pieces: H (jb < HJ) or dH' (jb < 2 HJ) rows
  // 16 jb' .. + 15, or rows 16 b' .. + 15 of tile (jb - 2 HJ) / 4.  H is the
  // bf16 copy of the state at the chunk's start, in the hand-off layout of dH'
  // (hand_off: each of these loads reads 1 KB of contiguous memory); tile
  // rows past the end of the sequence are clamped to the last.  The H and dH'
  // tiles are read by this workgroup only, once, as whole lines: their loads
  // are non-temporal.  The X / dO / dv tiles are 64-byte pieces of rows whose
  // other half the slab of the next columns reads, so those stay cached.
  __device__ static void issue_slab(const ChunkBwdArgs& p, Smem& sm, const Ctx& x, int n) {
    const Dims& d = p.d;
    const int nsl = d.Dv / NS;
    const int h = x.j * x.G + n / nsl, v0 = NS * (n % nsl);
    Slot& s = sm.u.r.s[n % NSLOT];
    const int bh = x.b * d.Hv + h;
    const size_t hsz = static_cast<size_t>(DK) * d.Dv;
    const size_t so = (static_cast<size_t>(x.c) * d.B * d.Hv + bh) * hsz;
    const size_t vbase = ((static_cast<size_t>(x.b) * d.T + x.t0) * d.Hv + h) * d.Dv;
    const size_t vbytes = (static_cast<size_t>(d.B) * d.T * d.Hv * d.Dv - vbase) * 2;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < JW; ++k) {
      const int jb = w + 8 * k;
      if (jb < 2 * HJ) {
        const bool isd = jb >= HJ;
        const int blk = isd ? jb - HJ : jb;
        const int ps = 64 * blk + l, i = ps >> 2;
        const uint32_t o = 2 * hand_off(DK, i, v0 + 8 * ((ps & 3) ^ sw(i)));
        if (isd)
          dma16_nt(raw_desc(p.dHend + so, hsz * 2), &s.dhv[512 * blk], o);
        else
          dma16_nt(raw_desc(p.cb.Hb + so, hsz * 2), &s.hv[512 * blk], o);
      } else if (jb < NJ) {
        const int u = jb - 2 * HJ, ten = u >> 2, blk = u & 3;
        const int t = 16 * blk + (l >> 2);
        const uint32_t o = 2 * (static_cast<uint32_t>(min(t, x.tl)) * x.v_row + v0 + 8 * ((l & 3) ^ sw(t)));
        const bf16* src = ten == 0 ? (XSV ? p.cb.X : static_cast<const bf16*>(p.v))
                          : ten == 1 ? static_cast<const bf16*>(p.dO) : static_cast<const bf16*>(p.dv);
        dma16(raw_desc(src + vbase, vbytes), &s.vt[ten][512 * blk], o);
      }
    }
  }
  // Waits for this wave's loads of every slab but the newest `later` ones.
  __device__ static void wait_slabs(bool later) {
    if (PD > 1 && later) {
      if (__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6) < JR)
        wait_vm<JW>();
      else
        wait_vm<JW - 1>();
    } else {
      wait_vm<0>();
    }
  }

  // The per-step and per-head scalars of value heads hb0 .. hb0 + HB - 1 of
  // the group (clamped to the group) into the batch arrays.
  __device__ static void load_batch(const ChunkBwdArgs& p, const Ctx& x, Smem& sm, int hb0) {
    const Dims& d = p.d;
    const int tid = threadIdx.x, t = tid & 63, k = tid >> 6;
#pragma unroll
    for (int rr0 = 0; rr0 < HB * 5; rr0 += NTG / 64) {
      const int rr = rr0 + k;
      if (rr < HB * 5) {
        const int hk = rr / 5, row = rr % 5;
        const int h = x.j * x.G + min(hb0 + hk, x.G - 1);
        const float* scc = p.cb.sc + (static_cast<size_t>(x.b * d.Hv + h) * x.NC + x.c) * SC_ROWS * L;
        const int sr = row == 0 ? SC_GAM : row == 1 ? SC_EG : row == 2 ? SC_EL : row == 3 ? SC_BETA : SC_ELL;
        const float v = scc[sr * L + t];
        sm.bsc[hk][row][t] = row == 4 && t >= x.Lc ? 0.f : v;
      }
    }
    if (tid < HB * 64) {
      const int hk = k, h = x.j * x.G + min(hb0 + hk, x.G - 1);
      const int tc = min(t, x.tl);
      const float av = __uint_as_float(static_cast<uint32_t>(
          static_cast<const unsigned short*>(p.a)[(static_cast<size_t>(x.b) * d.T + x.t0 + tc) * d.Hv + h]) << 16);
      const rsrc_t rm = make_rsrc(p.mask ? static_cast<const void*>(p.mask) : p.a,
                                  p.mask ? static_cast<size_t>(d.B) * d.T : 0);
      const uint32_t mv = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b8(rm, x.b * d.T + x.t0 + tc, 0, 0));
      sm.ha[hk][t] = av;
      sm.hm[hk][t] = p.mask == nullptr || mv != 0 ? 1.f : 0.f;
      if (t == 0) {
        const float* scc = p.cb.sc + (static_cast<size_t>(x.b * d.Hv + h) * x.NC + x.c) * SC_ROWS * L;
        sm.hegl[hk] = scc[SC_EGL * L];
        sm.hal[hk] = p.A_log[h];
        sm.hdt[hk] = p.dt_bias[h];
      }
    }
  }
  // Tx row ta of value head h (only where X is recomputed).
  __device__ static void load_tx(const ChunkBwdArgs& p, const Ctx& x, int h, bf16x8 (&txb)[2]) {
    if constexpr (XSV) {
      txb[0] = txb[1] = bf16x8{};
    } else {
      const int tid = threadIdx.x;
      const int ta = 16 * ((tid >> 6) & 3) + (tid & 15), lg = (tid & 63) >> 4;
      const size_t bh = static_cast<size_t>(x.b) * p.d.Hv + h;
      const bf16* txr = p.cb.Tx + (bh * x.NC + x.c) * L * L + ta * L + 8 * lg;
      txb[0] = load_bf16x8(txr);
      txb[1] = load_bf16x8(txr + 32);
    }
  }

  // Lane coordinates.  Recomputed from an opaque copy of the thread index at
  // the top of each loop so that the compiler rebuilds the addresses derived
  // from them there instead of keeping them all live across the loops.
  struct Lanes {
    int tid, l, w, tt, hw, lr, lg, ta, tc0;
    __device__ Lanes() {
      tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      l = tid & 63;
      w = tid >> 6;
      tt = w & 3;
      hw = w >> 2;
      lr = l & 15;
      lg = l >> 4;
      ta = 16 * tt + lr;
      tc0 = 16 * tt + 4 * lg;
    }
  };

  struct HeadAcc {
    f32x4 dox[2], xe[2];
    float pb[4], pa, pdb, phdh;
  };
  // Contractions over the slab's columns: dQn, dKn (state terms) and the
  // Grams dO X^T, X dv^T, and the waves of row tile 0 (one per half of Dk)
  // <dH', H> from the same operand reads.  xr8 / xs8: rows ta of X and of
  // diag(e^{gL-g} beta) X; xt: the X tile [t][v] (a ring tile, or with XR
  // the recomputed one).
  template <bool XR>
  __device__ static void contract(const Smem& sm, int slot, const Slot& s, const bf16* xt, int ta, int lr, int lg,
                                  int hw, int tt, const bf16x8& xr8, const bf16x8& xs8, f32x4 (&accQ)[IH],
                                  f32x4 (&accK)[IH], HeadAcc& ac) {
    const bf16* dt = s.vt[1];
    const bf16* et = s.vt[2];
    const float sq = sm.bsc[slot][1][ta];
    const bf16x8 do8 = load_bf16x8(&dt[rpos(ta, lg)]);
    const bf16x8 dos8 = scale8(do8, sq), dvs8 = scale8(load_bf16x8(&et[rpos(ta, lg)]), -sq);
#pragma unroll
    for (int k = 0; k < IH; ++k) {
      const int it = hw * IH + k;
      const bf16x8 bhv = load_bf16x8(&s.hv[rpos(16 * it + lr, lg)]);
      const bf16x8 bdh = load_bf16x8(&s.dhv[rpos(16 * it + lr, lg)]);
      accQ[k] = mfma16(dos8, bhv, accQ[k]);
      accK[k] = mfma16(dvs8, bhv, accK[k]);
      accK[k] = mfma16(xs8, bdh, accK[k]);
      if (__builtin_amdgcn_readfirstlane(tt) == 0) {
        const uint4 hu = __builtin_bit_cast(uint4, bhv), du = __builtin_bit_cast(uint4, bdh);
        ac.phdh = dot2_bf16(hu.x, du.x, ac.phdh);
        ac.phdh = dot2_bf16(hu.y, du.y, ac.phdh);
        ac.phdh = dot2_bf16(hu.z, du.z, ac.phdh);
        ac.phdh = dot2_bf16(hu.w, du.w, ac.phdh);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int sr = 16 * (2 * hw + u) + lr;
      const int xo = XR ? sr * VS + 8 * lg : rpos(sr, lg);
      ac.dox[u] = mfma16(do8, load_bf16x8(&xt[xo]), ac.dox[u]);
      ac.xe[u] = mfma16(xr8, load_bf16x8(&et[rpos(sr, lg)]), ac.xe[u]);
    }
  }
  // Slab n (of ns in all): wait for its loads, meet the other waves, issue
  // the loads of slab n + PD into the slot that slab n - 1 used, and
  // accumulate.
  __device__ static void slab(const ChunkBwdArgs& p, Smem& sm, const Ctx& x, int n, int ns, int slot,
                              const bf16x8 (&ka)[KS], const bf16x8 (&qa)[KS], const bf16x8 (&txb)[2],
                              f32x4 (&accQ)[IH], f32x4 (&accK)[IH], HeadAcc& ac) {
    wait_slabs(n + 1 < ns);
    lds_barrier();  // slab n complete in its slot; every wave is done with slab n - 1
    if (n + PD < ns) issue_slab(p, sm, x, n + PD);
    const Lanes q;
    const int lr = q.lr, lg = q.lg, ta = q.ta, tc0 = q.tc0, hw = q.hw;
    const Slot& s = sm.u.r.s[n % NSLOT];
    const bf16* vt = s.vt[0];
    const bf16* dt = s.vt[1];
    const bf16* et = s.vt[2];
    // ---- K H, Q H (rows tc0 + r, cols 16 hw + lr) and (K dH')^T (rows 16 hw + 4 lg + r, col ta).
    // The H and dH' operands (rows 32 kt + 8 lg .. + 7 of column 16 hw + lr)
    // are read transposed from the [i][v] tiles.
    f32x4 kh = f4zero(), qh = f4zero(), kdt = f4zero();
#pragma unroll
    for (int kt = 0; kt < KS; ++kt) {
      const int r0 = 32 * kt + 8 * lg + (lr >> 2), pc = 2 * hw + ((lr >> 1) & 1), e = 4 * (lr & 1);
      const uint2 h0 = lds_read_tr16(&s.hv[rpos(r0, pc) + e]), h1 = lds_read_tr16(&s.hv[rpos(r0 + 4, pc) + e]);
      const uint2 d0 = lds_read_tr16(&s.dhv[rpos(r0, pc) + e]), d1 = lds_read_tr16(&s.dhv[rpos(r0 + 4, pc) + e]);
      const bf16x8 bh8 = as_bf16x8(make_uint4(h0.x, h0.y, h1.x, h1.y));
      kh = mfma16(ka[kt], bh8, kh);
      qh = mfma16(qa[kt], bh8, qh);
      kdt = mfma16(as_bf16x8(make_uint4(d0.x, d0.y, d1.x, d1.y)), ka[kt], kdt);
    }
    // element (t, 16 hw + lr) and the 4 columns 16 hw + 4 lg .. of row ta in the ring tiles
    const int pe = 2 * hw + (lr >> 3), ee = lr & 7;
    const int pv = 2 * hw + (lg >> 1), ev = 4 * (lg & 1);
    if constexpr (XSV) {
      // ---- b_r partial sums; X (tile 0) is loaded
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tc0 + r, o = rpos(t, pe) + ee;
        const float eg = sm.bsc[slot][1][t], cr = eg * sm.rk[t];
        const float dov = to_f32(dt[o]), dvv = to_f32(et[o]);
        ac.pb[r] = fmaf(eg * sm.rq[t] * qh[r], dov, ac.pb[r]);
        ac.pb[r] = fmaf(-cr * kh[r], dvv, ac.pb[r]);
      }
      // X[ta][16 hw + 4 lg + r], in the layout of (K dH')^T
      const uint2 x4 = *reinterpret_cast<const uint2*>(&vt[rpos(ta, pv) + ev]);
      const uint2 e4 = *reinterpret_cast<const uint2*>(&et[rpos(ta, pv) + ev]);
      const float x4f[4] = {__uint_as_float(x4.x << 16), __uint_as_float(x4.x & 0xffff0000u),
                            __uint_as_float(x4.y << 16), __uint_as_float(x4.y & 0xffff0000u)};
      const float e4f[4] = {__uint_as_float(e4.x << 16), __uint_as_float(e4.x & 0xffff0000u),
                            __uint_as_float(e4.y << 16), __uint_as_float(e4.y & 0xffff0000u)};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ac.pdb = fmaf(e4f[r], x4f[r], ac.pdb);
        ac.pa = fmaf(kdt[r], x4f[r], ac.pa);
      }
      const bf16x8 xr8 = load_bf16x8(&vt[rpos(ta, lg)]);
      contract<false>(sm, slot, s, vt, ta, lr, lg, hw, q.tt, xr8, scale8(xr8, sm.bsc[slot][2][ta] * sm.bsc[slot][3][ta]),
                      accQ, accK, ac);
    } else {
      XRec& xr = sm.u.r.xrec;
      // ---- R = V - diag(e^g rk) K H -> R^T; b_r partial sums
      {
        float rv[4];
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = tc0 + r, o = rpos(t, pe) + ee;
          const float eg = sm.bsc[slot][1][t], cr = eg * sm.rk[t];
          const float vv = to_f32(vt[o]), dov = to_f32(dt[o]), dvv = to_f32(et[o]);
          rv[r] = vv - cr * kh[r];
          ac.pb[r] = fmaf(eg * sm.rq[t] * qh[r], dov, ac.pb[r]);
          ac.pb[r] = fmaf(-cr * kh[r], dvv, ac.pb[r]);
        }
        *reinterpret_cast<uint2*>(&xr.rt[(16 * hw + lr) * TS + tc0]) = pack4_bf16(rv[0], rv[1], rv[2], rv[3]);
      }
      lds_barrier();
      // ---- X^T = R^T Tx^T: the lane holds X[ta][16 hw + 4 lg + r]
      {
        f32x4 xt = f4zero();
  #pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          xt = mfma16(load_bf16x8(&xr.rt[(16 * hw + lr) * TS + 32 * kt + 8 * lg]), txb[kt], xt);
        const int vc = 16 * hw + 4 * lg;
        const float sx = sm.bsc[slot][2][ta] * sm.bsc[slot][3][ta];
        // X in bf16, as the forward saves it: the gate terms and the scaled copy
        // use the rounded values
        const uint2 x4 = pack4_bf16(xt[0], xt[1], xt[2], xt[3]);
        const float x4f[4] = {__uint_as_float(x4.x << 16), __uint_as_float(x4.x & 0xffff0000u),
                              __uint_as_float(x4.y << 16), __uint_as_float(x4.y & 0xffff0000u)};
        *reinterpret_cast<uint2*>(&xr.xr[ta * VS + vc]) = x4;
        *reinterpret_cast<uint2*>(&xr.xs[ta * VS + vc]) = pack4_bf16(sx * x4f[0], sx * x4f[1], sx * x4f[2], sx * x4f[3]);
        const uint2 e4 = *reinterpret_cast<const uint2*>(&et[rpos(ta, pv) + ev]);
        const float e4f[4] = {__uint_as_float(e4.x << 16), __uint_as_float(e4.x & 0xffff0000u),
                              __uint_as_float(e4.y << 16), __uint_as_float(e4.y & 0xffff0000u)};
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          ac.pdb = fmaf(e4f[r], x4f[r], ac.pdb);
          ac.pa = fmaf(kdt[r], x4f[r], ac.pa);
        }
      }
      lds_barrier();
      contract<true>(sm, slot, s, xr.xr, ta, lr, lg, hw, q.tt, load_bf16x8(&xr.xr[ta * VS + 8 * lg]),
                     load_bf16x8(&xr.xs[ta * VS + 8 * lg]), accQ, accK, ac);
    }
  }

  __device__ static void run(const ChunkBwdArgs& p, Smem& sm) {
    const Dims& d = p.d;
    Ctx x;
    x.c = blockIdx.x;
    const int bj = blockIdx.y;
    x.b = bj / d.Hk;
    x.j = bj % d.Hk;
    const int G = d.G();
    x.NC = d.nchunk();
    x.G = G;
    x.t0 = x.c * L;
    x.Lc = min(L, d.T - x.t0);
    x.tl = x.Lc - 1;
    x.v_row = d.Hv * d.Dv;
    const int Lc = x.Lc, c = x.c, NC = x.NC;
    const size_t qk0 = (static_cast<size_t>(x.b) * d.T + x.t0) * d.Hk + x.j;  // [B,T,Hk] index of step t0
    const uint32_t qk_row = d.Hk * DK;
    const bf16* kc = static_cast<const bf16*>(p.k) + qk0 * DK;
    const bf16* qc = static_cast<const bf16*>(p.q) + qk0 * DK;
    const int tid0 = threadIdx.x;
    // The chunk's k and q rows (KQL: coalesced, for LDS), the norm factors
    // (the same for every value head of the group; 0 past the end) and the
    // first batch of value heads' scalars: all issued before any is waited
    // for, so that their latencies overlap.
    constexpr int NPT = KQL ? L * DK / 8 / NTG : 1;
    static_assert(!KQL || L * DK / 8 % NTG == 0, "whole pieces per thread");
    uint4 kv[NPT], qv[NPT];
    if constexpr (KQL) {
#pragma unroll
      for (int u = 0; u < NPT; ++u) {
        const int pc = tid0 + u * NTG, row = pc / (DK / 8), c8 = 8 * (pc % (DK / 8));
        const uint32_t o = static_cast<uint32_t>(min(row, x.tl)) * qk_row + c8;
        kv[u] = *reinterpret_cast<const uint4*>(kc + o);
        qv[u] = *reinterpret_cast<const uint4*>(qc + o);
      }
    }
    float rk0, rq0;
    {
      const float* scc = p.cb.sc + (static_cast<size_t>(x.b * d.Hv + x.j * G) * NC + c) * SC_ROWS * L;
      rk0 = scc[SC_RK * L + (tid0 & 63)];
      rq0 = scc[SC_RQ * L + (tid0 & 63)];
    }
    load_batch(p, x, sm, 0);
    f32x4 accQ[IH], accK[IH];
#pragma unroll
    for (int k = 0; k < IH; ++k) accQ[k] = accK[k] = f4zero();
    // k and q rows of this wave's row tile, for every head and slab of the
    // workgroup (loading them inside the slab loop would make each wait for
    // them also wait for the next slab's prefetch, issued before them)
    bf16x8 ka[KS], qa[KS];
    // The raw Grams of the chunk in the accumulator layout of the L x L terms:
    // lane register r of [u] holds element (a, b), a = tc0 + r, b = 16 (2 hw +
    // u) + lr, of kk = K K^T and qk = Q K^T (the products chunk_prep forms
    // for A and P, in the same order).  With them every L x L term of a head
    // is formed in registers: A[b][a] = e^{-|g_a - g_b|} rk_a rk_b kk, P[a][b]
    // = e^{g_a - g_b} rq_a rk_b qk (b <= a).
    f32x4 kk[2], qk[2];
    const int ns = G * (d.Dv / NS);  // slabs of the workgroup
    if constexpr (KQL) {
      // The chunk's k and q rows, each loaded once with coalesced 16-byte
      // loads into LDS that nothing uses before the first slab (k rows in the
      // space of the weight tiles, q rows in ring slot 2); every wave reads
      // its operands (k and q rows of its row tile, k rows of its two Gram
      // column tiles) from there in the matrix-core layout.
      bf16* ks = reinterpret_cast<bf16*>(&sm.wt);
      bf16* qs = reinterpret_cast<bf16*>(&sm.u.r.s[2]);
#pragma unroll
      for (int u = 0; u < NPT; ++u) {
        const int pc = tid0 + u * NTG, row = pc / (DK / 8), c8 = 8 * (pc % (DK / 8));
        *reinterpret_cast<uint4*>(&ks[row * KQS + c8]) = kv[u];
        *reinterpret_cast<uint4*>(&qs[row * KQS + c8]) = qv[u];
      }
#pragma unroll
      for (int n = 0; n < PD; ++n)
        if (n < ns) issue_slab(p, sm, x, n);
      __syncthreads();
      const Lanes q;
#pragma unroll
      for (int kt = 0; kt < KS; ++kt) {
        ka[kt] = load_bf16x8(&ks[q.ta * KQS + 32 * kt + 8 * q.lg]);
        qa[kt] = load_bf16x8(&qs[q.ta * KQS + 32 * kt + 8 * q.lg]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        kk[u] = qk[u] = f4zero();
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) {
          const bf16x8 bk = load_bf16x8(&ks[(16 * (2 * q.hw + u) + q.lr) * KQS + 32 * kt + 8 * q.lg]);
          kk[u] = mfma16(ka[kt], bk, kk[u]);
          qk[u] = mfma16(qa[kt], bk, qk[u]);
        }
      }
    } else {
      // the k rows of the column tiles 2 hw, 2 hw + 1 of this wave's L x L
      // terms (the B operands of its Gram tiles)
      bf16x8 kb[2][KS];
      {  // quad-coalesced (lane m reads piece m % 4 of row m / 4: four lanes cover
         // 64 contiguous bytes); moved to the operand layout below, once the
         // first slabs' loads are issued
        const int l = tid0 & 63, tr0 = 16 * ((tid0 >> 6) & 3) + coal_row(l);
        const uint32_t o = static_cast<uint32_t>(min(tr0, x.tl)) * qk_row + 8 * coal_piece(l);
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) {
          ka[kt] = load_bf16x8(kc + o + 32 * kt);
          qa[kt] = load_bf16x8(qc + o + 32 * kt);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int tb = 16 * (2 * (tid0 >> 8) + u) + coal_row(l);
          const uint32_t ob = static_cast<uint32_t>(min(tb, x.tl)) * qk_row + 8 * coal_piece(l);
#pragma unroll
          for (int kt = 0; kt < KS; ++kt) kb[u][kt] = load_bf16x8(kc + ob + 32 * kt);
        }
      }
#pragma unroll
      for (int n = 0; n < PD; ++n)
        if (n < ns) issue_slab(p, sm, x, n);
#pragma unroll
      for (int kt = 0; kt < KS; ++kt) {
        ka[kt] = to_mfma_layout(ka[kt]);
        qa[kt] = to_mfma_layout(qa[kt]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        kk[u] = qk[u] = f4zero();
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) {
          const bf16x8 bk = to_mfma_layout(kb[u][kt]);
          kk[u] = mfma16(ka[kt], bk, kk[u]);
          qk[u] = mfma16(qa[kt], bk, qk[u]);
        }
      }
    }
    // the group sums of the L x L weights, same layout: Wq diag(rk), V1 (=
    // (Wk1 diag(rq))^T) and U (Wk2 diag(rk) = (U + U^T) diag(rk))
    f32x4 wq[2], v1[2], uu[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) wq[u] = v1[u] = uu[u] = f4zero();
    if (tid0 < L) {
      sm.rk[tid0] = rk0;
      sm.rq[tid0] = rq0;
    }
    const int nsl = d.Dv / NS;
    int n = 0;
    for (int hh = 0; hh < G; ++hh) {
      const int h = x.j * G + hh, slot = hh % HB;
      if (slot == 0 && hh > 0) {
        // a later batch of value heads (groups of more than HB): its scalars,
        // after the previous batch's deferred section (these loads wait for
        // the ring's, once per batch)
        __syncthreads();
        load_batch(p, x, sm, hh);
      }
      bf16x8 txb[2];
      load_tx(p, x, h, txb);
      // (the head's scalars are read from the batch arrays; the first slab's
      // barrier orders them after the batch loads)
      HeadAcc ac;
      ac.dox[0] = ac.dox[1] = ac.xe[0] = ac.xe[1] = f4zero();
      ac.pb[0] = ac.pb[1] = ac.pb[2] = ac.pb[3] = ac.pa = ac.pdb = ac.phdh = 0.f;
      for (int si = 0; si < nsl; ++si, ++n) slab(p, sm, x, n, ns, slot, ka, qa, txb, accQ, accK, ac);

      // ---- per-row sums of head h; its L x L weights (added to the group
      // sums) and rectangle terms of dl, in the lane's accumulator layout
      // (a = tc0 + r, b = 16 (2 hw + u) + lr, d = e^{-|g_a - g_b|}; dox =
      // dO_a . X_b, xe = X_a . dv_b):
      //   Wq diag(rk): [b <= a] d beta_b dox rk_b
      //   V1:          [b <= a] d beta_b dox rq_a     (Wk1 diag(rq) = V1^T)
      //   U:          -[a < b]  d beta_a xe           (Wk2 diag(rk) = (U + U^T) diag(rk))
      // The rectangle terms m[r][s] = [s < r] beta_s (P[r][s] dox[r][s] -
      // A[r][s] xe[s][r]) enter dl only through colsum(m) - rowsum(m), which
      // equals colsum(E) - rowsum(E) for E[a][b] = [b < a] beta_b P[a][b] dox +
      // [a < b] beta_a A[b][a] xe (the second part is minus the xe term of
      // m[b][a]).
      {
        const Lanes q;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = row_sum16(ac.pb[r]);
          if (q.lr == 0) sm.bv[slot][q.hw][q.tc0 + r] = v;
        }
        float pa = ac.pa, pdb = ac.pdb;
        pa += __shfl_xor(pa, 16);
        pa += __shfl_xor(pa, 32);
        pdb += __shfl_xor(pdb, 16);
        pdb += __shfl_xor(pdb, 32);
        if (q.lg == 0) {
          sm.pa[slot][q.hw][q.ta] = pa;
          sm.pdb[slot][q.hw][q.ta] = pdb;
        }
        const float phdh = wave_sum(ac.phdh);
        if (q.l == 0) sm.red[slot][q.w] = phdh;

        const int tc0 = q.tc0;
        const float* gam = sm.bsc[slot][0];
        const float* bet = sm.bsc[slot][3];
        const float4 g4 = *reinterpret_cast<const float4*>(&gam[tc0]);
        const float4 b4 = *reinterpret_cast<const float4*>(&bet[tc0]);
        const float4 q4 = *reinterpret_cast<const float4*>(&sm.rq[tc0]);
        const float4 k4 = *reinterpret_cast<const float4*>(&sm.rk[tc0]);
        const float ga[4] = {g4.x, g4.y, g4.z, g4.w}, ba[4] = {b4.x, b4.y, b4.z, b4.w};
        const float rqa[4] = {q4.x, q4.y, q4.z, q4.w}, rka[4] = {k4.x, k4.y, k4.z, k4.w};
        float rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int b = 16 * (2 * q.hw + u) + q.lr;
          const float gb = gam[b], bb = bet[b], rkb = sm.rk[b];
          float colp = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int a = tc0 + r;
            const bool ok = a < Lc && b < Lc;
            const bool lo = ok && b <= a, st = ok && b < a, up = ok && a < b;
            const float dec = __expf(-fabsf(ga[r] - gb));  // hardware exp (bf16-level weights)
            const float bd = dec * bb * ac.dox[u][r];    // d beta_b dox
            const float ux = dec * ba[r] * ac.xe[u][r];  // d beta_a xe
            wq[u][r] += lo ? bd * rkb : 0.f;
            v1[u][r] += lo ? bd * rqa[r] : 0.f;
            uu[u][r] -= up ? ux : 0.f;
            const float e = st ? bd * rqa[r] * rkb * qk[u][r] : up ? ux * rka[r] * rkb * kk[u][r] : 0.f;
            rowp[r] += e;
            colp += e;
          }
          // column b: the lane's four rows, then the wave's four row groups
          colp += __shfl_xor(colp, 16);
          colp += __shfl_xor(colp, 32);
          if (q.lg == 0) sm.colp[slot][q.tt][b] = colp;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = row_sum16(rowp[r]);
          if (q.lr == 0) sm.rowp[slot][q.hw][tc0 + r] = v;
        }
      }
      // ---- deferred section, one wave per value head of the batch:
      // dl_t = e^{gL} <dH', H> + sum_{u<t} (a_u + cs_u - rs_u) + sum_{r>=t} b_r; da, db
      // (cs, rs: the column and row sums of E)
      if (slot == HB - 1 || hh == G - 1) {
        __syncthreads();
        const Lanes q;
        const int hb0 = hh - slot, nh = slot + 1;
        if (q.w < nh) {
          const int k = q.w, hd = x.j * G + hb0 + k, t = q.l;
          const bool in = t < Lc;
          const float av = sm.ha[k][t];
          const bool valid = sm.hm[k][t] != 0.f;
          const float beta = sm.bsc[k][3][t];
          const float as = in ? sm.bsc[k][2][t] * beta * sm.rk[t] * (sm.pa[k][0][t] + sm.pa[k][1][t]) : 0.f;
          const float csum = (sm.colp[k][0][t] + sm.colp[k][1][t]) + (sm.colp[k][2][t] + sm.colp[k][3][t]);
          const float hu = as + (csum - (sm.rowp[k][0][t] + sm.rowp[k][1][t]));
          const float hbr = in ? sm.bv[k][0][t] + sm.bv[k][1][t] : 0.f;
          float hdh = 0.f;
#pragma unroll
          for (int i = 0; i < NTG / 64; ++i) hdh += sm.red[k][i];
          // sum over u < t: the prefix sum of the terms shifted by one step;
          // sum over r >= t: the prefix sum of the terms in reverse order,
          // taken back from lane 63 - t
          const float hus = __shfl_up(hu, 1);
          const float pre = wave_prefix_sum(t > 0 ? hus : 0.f);
          const float suf = __shfl(wave_prefix_sum(__shfl(hbr, L - 1 - t)), L - 1 - t);
          const float ell = sm.bsc[k][4][t];
          const float dl = expf(ell) == 0.f ? 0.f : sm.hegl[k] * hdh + pre + suf;
          float da = 0.f, db = 0.f, dll = 0.f;
          if (in && valid) {
            const float xa = av + sm.hdt[k];
            da = xa <= kClamp ? dl * (-expf(sm.hal[k])) * sigmoid_f(fminf(xa, kClamp)) : 0.f;
            db = (sm.pdb[k][0][t] + sm.pdb[k][1][t]) * (1.f - beta);
            dll = dl != 0.f ? dl * ell : 0.f;
          }
          // steps past the end of the sequence fall outside the descriptors
          const size_t r0 = (static_cast<size_t>(x.b) * d.T + x.t0) * d.Hv + hd;
          const size_t nb = (static_cast<size_t>(Lc - 1) * d.Hv + 1) * 2;
          const uint32_t ro = 2 * static_cast<uint32_t>(t * d.Hv);
          __builtin_amdgcn_raw_buffer_store_b16(bf16_of(da).x, make_rsrc(static_cast<bf16*>(p.da) + r0, nb), ro, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b16(bf16_of(db).x, make_rsrc(static_cast<bf16*>(p.db) + r0, nb), ro, 0, 0);
          const double sa = wave_sum_f64_dpp(static_cast<double>(dll));
          const double sd = wave_sum_f64_dpp(static_cast<double>(da));
          if (t == 0) {
            const size_t pi = (static_cast<size_t>(x.b) * NC + c) * d.Hv + hd;
            p.part_dA[pi] = sa;
            p.part_ddt[pi] = sd;
          }
        }
        // drained, so that the per-slab waits count only the ring's loads
        if (hh + 1 < G) wait_vm<0>();
      }
    }
    wait_vm<0>();  // no direct-to-LDS load may land in the union's later uses

    // ---- the q / k rows of the normalisation backward, loaded now (the slabs'
    // loads are done) so that their latency overlaps the final products; the
    // barriers below wait for LDS only
    constexpr int QW = DK / 8;                // columns per thread in the normalisation backward
    uint4 qrow[QW / 8], krow[QW / 8];
    {
      const Lanes q;
      const uint32_t ro = static_cast<uint32_t>(min(q.tid >> 3, x.tl)) * qk_row + (q.tid & 7) * QW;
#pragma unroll
      for (int u = 0; u < QW / 8; ++u) {
        qrow[u] = *reinterpret_cast<const uint4*>(qc + ro + 8 * u);
        krow[u] = *reinterpret_cast<const uint4*>(kc + ro + 8 * u);
      }
    }

    // ---- final products with the group sums: dQn += Wq Kn, dKn += Wk1 Qn + Wk2 Kn.
    // Their Kn / Qn operands are the chunk's k and q rows the waves have held
    // since the start (each wave its 16-step row tile), put in LDS as [t][i]
    // tiles and read transposed; the group sums go from the registers to bf16
    // [t][s] tiles (Wk1 diag(rq) = V1^T, Wk2 diag(rk) = (U + U^T) diag(rk)
    // with U strictly upper triangular: the lane of (a, b), a < b, writes
    // both (a, b) and (b, a), the lane of (a, a) writes the zero diagonal).
    lds_barrier();
    {
      const Lanes q;
      // waves 0-3 (hw = 0) put their k rows, waves 4-7 their q rows
      bf16* kqt = q.hw == 0 ? sm.u.kq.k : sm.u.kq.q;
#pragma unroll
      for (int kt = 0; kt < KS; ++kt)
        *reinterpret_cast<uint4*>(&kqt[q.ta * KQS + 32 * kt + 8 * q.lg]) =
            __builtin_bit_cast(uint4, q.hw == 0 ? ka[kt] : qa[kt]);
      const float4 k4 = *reinterpret_cast<const float4*>(&sm.rk[q.tc0]);
      const float rka[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int b = 16 * (2 * q.hw + u) + q.lr;
        const float rkb = sm.rk[b];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int a = q.tc0 + r;
          sm.wt.wq[a * TS + b] = bf16_of(wq[u][r]);
          sm.wt.wk[b * WS + a] = bf16_of(v1[u][r]);
          if (a <= b) {
            sm.wt.wk[a * WS + L + b] = bf16_of(uu[u][r] * rkb);
            sm.wt.wk[b * WS + L + a] = bf16_of(uu[u][r] * rka[r]);
          }
        }
      }
    }
    lds_barrier();
    {
      const Lanes q;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 aq = load_bf16x8(&sm.wt.wq[q.ta * TS + 32 * kt + 8 * q.lg]);
        const bf16x8 a1 = load_bf16x8(&sm.wt.wk[q.ta * WS + 32 * kt + 8 * q.lg]);
        const bf16x8 a2 = load_bf16x8(&sm.wt.wk[q.ta * WS + L + 32 * kt + 8 * q.lg]);
#pragma unroll
        for (int k = 0; k < IH; ++k) {
          // steps 32 kt + 8 lg .. + 7 of channel 16 (hw IH + k) + lr
          const int o0 = (32 * kt + 8 * q.lg + (q.lr >> 2)) * KQS + 16 * (q.hw * IH + k) + 4 * (q.lr & 3);
          const uint2 k0 = lds_read_tr16(&sm.u.kq.k[o0]), k1 = lds_read_tr16(&sm.u.kq.k[o0 + 4 * KQS]);
          const uint2 q0 = lds_read_tr16(&sm.u.kq.q[o0]), q1 = lds_read_tr16(&sm.u.kq.q[o0 + 4 * KQS]);
          const bf16x8 vk = as_bf16x8(make_uint4(k0.x, k0.y, k1.x, k1.y));
          const bf16x8 vq = as_bf16x8(make_uint4(q0.x, q0.y, q1.x, q1.y));
          accQ[k] = mfma16(aq, vk, accQ[k]);
          accK[k] = mfma16(a1, vq, accK[k]);
          accK[k] = mfma16(a2, vk, accK[k]);
        }
      }
    }

    // ---- L2-normalisation backward: dq = rq (dQn - Dk qn (qn . dQn)), dk = rk (dKn - kn (kn . dKn)).
    // dQn and dKn go to LDS (together, or one after the other), then each
    // thread takes 1/8 of a row: dot product with the row, and the output.
#pragma unroll
    for (int p0 = 0; p0 < 2; p0 += NFIN) {
      const Lanes q;
      lds_barrier();
#pragma unroll
      for (int f = 0; f < NFIN; ++f)
#pragma unroll
        for (int k = 0; k < IH; ++k)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sm.u.f.acc[f][(q.tc0 + r) * FS + 16 * (q.hw * IH + k) + q.lr] = p0 + f == 0 ? accQ[k][r] : accK[k][r];
      lds_barrier();
      const int t = q.tid >> 3, qd = q.tid & 7;
#pragma unroll
      for (int f = 0; f < NFIN; ++f) {
        const int pass = p0 + f;
        const uint4* xr = pass == 0 ? qrow : krow;
        const float* ac = &sm.u.f.acc[f][t * FS + qd * QW];
        float dot = 0.f;
#pragma unroll
        for (int u = 0; u < QW; u += 8) {
          float xv[8];
          Vec16<bf16>::unpack(xr[u / 8], xv);
#pragma unroll
          for (int e = 0; e < 8; ++e) dot = fmaf(xv[e], ac[u + e], dot);
        }
        dot = oct_sum(dot);
        if (t < Lc) {
          const float r1 = pass == 0 ? sm.rq[t] : sm.rk[t];
          const float coef = (pass == 0 ? static_cast<float>(DK) : 1.f) * r1 * r1 * dot;
          bf16* dst = static_cast<bf16*>(pass == 0 ? p.dq : p.dk) + (qk0 + static_cast<size_t>(t) * d.Hk) * DK + qd * QW;
#pragma unroll
          for (int u = 0; u < QW; u += 8) {
            float xv[8], y[8];
            Vec16<bf16>::unpack(xr[u / 8], xv);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = r1 * (ac[u + e] - coef * xv[e]);
            *reinterpret_cast<uint4*>(dst + u) = make_uint4(pack2_bf16(y[0], y[1]), pack2_bf16(y[2], y[3]),
                                                            pack2_bf16(y[4], y[5]), pack2_bf16(y[6], y[7]));
          }
        }
      }    }
  }
};

template <int DK, bool XSV>
__global__ void __launch_bounds__(NTG) chunk_bwd_grad_kernel(ChunkBwdArgs p) {
  __shared__ typename ChunkBwdGrad<DK, XSV>::Smem sm;
  ChunkBwdGrad<DK, XSV>::run(p, sm);
}

// bf16 copies of the chunk-start states: 8 elements per thread, grid-stride.
__global__ void __launch_bounds__(256) state_bf16_kernel(StateBf16Args a) {
  const size_t per = a.slot / 8, n = per * a.nslot;
  for (size_t u = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; u < n; u += static_cast<size_t>(gridDim.x) * 256) {
    const size_t sl = u / per, e = 8 * (u % per);
    const float* src = sl == 0 ? a.state0 : a.ckpt + (sl - 1) * a.slot;
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (src != nullptr) {
      x0 = *reinterpret_cast<const float4*>(src + e);
      x1 = *reinterpret_cast<const float4*>(src + e + 4);
    }
    // into the hand-off layout of the (chunk, head) block (8 columns of a row
    // stay contiguous there)
    const size_t blk = static_cast<size_t>(a.dk) * a.dv, bh = e / blk;
    const int i = static_cast<int>((e % blk) / a.dv), v = static_cast<int>(e % a.dv);
    *reinterpret_cast<uint4*>(a.Hb + sl * a.slot + bh * blk + hand_off(a.dk, i, v)) =
        make_uint4(pack2_bf16(x0.x, x0.y), pack2_bf16(x0.z, x0.w), pack2_bf16(x1.x, x1.y), pack2_bf16(x1.z, x1.w));
  }
}

}  // namespace

hipError_t launch_state_bf16(const StateBf16Args& a, hipStream_t st) {
  const size_t n = a.slot / 8 * a.nslot;
  if (n == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 8192));
  state_bf16_kernel<<<blocks, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd_state(const ChunkBwdArgs& a, hipStream_t st) {
  const int NV = ChunkBwdState<64>::NV;
  const int nseg = a.seg ? (a.d.nchunk() + a.seg - 1) / a.seg : 1;
  const dim3 nblk(a.d.B * a.d.Hv * ((a.map ? a.d.Dk + a.d.Dv : a.d.Dv) / NV), nseg);
  if (a.vg) {
    if (a.seg || a.map) return hipErrorInvalidValue;
    switch (a.d.Dk) {
      case 64: chunk_bwd_state_kernel<64, true><<<nblk, ChunkBwdState<64, true>::NTS, 0, st>>>(a); break;
      case 128: chunk_bwd_state_kernel<128, true><<<nblk, ChunkBwdState<128, true>::NTS, 0, st>>>(a); break;
      case 192: chunk_bwd_state_kernel<192, true><<<nblk, ChunkBwdState<192, true>::NTS, 0, st>>>(a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
#define GDN_BWD_CASE(D)                                                                \
  case D:                                                                              \
    if (a.stream)                                                                      \
      chunk_bwd_state_kernel<D, false, true><<<nblk, ChunkBwdState<D>::NTS, 0, st>>>(a);  \
    else                                                                               \
      chunk_bwd_state_kernel<D, false, false><<<nblk, ChunkBwdState<D>::NTS, 0, st>>>(a); \
    break;
  switch (a.d.Dk) {
    GDN_BWD_CASE(64)
    GDN_BWD_CASE(128)
    GDN_BWD_CASE(192)
    GDN_BWD_CASE(256)
    default: return hipErrorInvalidValue;
  }
#undef GDN_BWD_CASE
  return hipGetLastError();
}

hipError_t launch_chunk_bwd_grad(const ChunkBwdArgs& a, hipStream_t st) {
  if (a.d.T == 0) return hipSuccess;
  dim3 grid(a.d.nchunk(), a.d.B * a.d.Hk);
  const bool xs = a.cb.X != nullptr;
  switch (a.d.Dk) {
    case 64: xs ? chunk_bwd_grad_kernel<64, true><<<grid, NTG, 0, st>>>(a) : chunk_bwd_grad_kernel<64, false><<<grid, NTG, 0, st>>>(a); break;
    case 128: xs ? chunk_bwd_grad_kernel<128, true><<<grid, NTG, 0, st>>>(a) : chunk_bwd_grad_kernel<128, false><<<grid, NTG, 0, st>>>(a); break;
    case 192: xs ? chunk_bwd_grad_kernel<192, true><<<grid, NTG, 0, st>>>(a) : chunk_bwd_grad_kernel<192, false><<<grid, NTG, 0, st>>>(a); break;
    case 256: xs ? chunk_bwd_grad_kernel<256, true><<<grid, NTG, 0, st>>>(a) : chunk_bwd_grad_kernel<256, false><<<grid, NTG, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
