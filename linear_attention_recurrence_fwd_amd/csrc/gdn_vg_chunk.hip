// Chunked (matrix) form of the gated delta rule with a per-key-channel gate
// on gfx950 bf16 MFMA.
//
// The gate is a vector g_t = e^{lg_t} over the key channels that scales the
// rows of the state before each step's read and write (the per-channel
// ("vectorised") gating of the mlx-lm VJP PR's model list, the Kimi-Linear
// case).  Over a chunk of L = 64 steps, with H the state at the chunk start
// and G_t = lg_0 + ... + lg_t the in-chunk cumulative log-gate (a vector over
// the channels; masked steps add 0), the recurrence unrolls to the scalar
// gate's chunk form with the decays moved into the operands:
//   Kb_t = kn_t e^{G_t},  Kh_t = kn_t e^{G_L - G_t},  Qb_t = qn_t e^{G_t} / sqrt(Dk)
//   A[t,s] = [s<t]  sum_i kn_ti kn_si e^{G_ti - G_si},  N = A diag(beta),  Tx = (I + N)^-1
//   P[t,s] = [s<=t] sum_i qn_ti kn_si e^{G_ti - G_si} / sqrt(Dk),  Mq = P diag(beta)
//   X  = Tx (V - Kb H),  O = Qb H + Mq X,  H' = diag(e^{G_L}) H + Kh^T diag(beta) X.
// Every factor is e^{G_t - G_s} with s <= t (at most 1 for a decay).  The
// products A and P cannot be split into a product of a row and a column
// factor in one piece (e^{-G_s} alone overflows for strong decays), so they
// are taken in 16-step sub-blocks: for t in sub-block I > J (s in J) with
// r = 16 I - 1 the last step before I,
//   e^{G_t - G_s} = e^{G_t - G_r} e^{G_r - G_s}    (both factors <= 1),
// a bf16 MFMA product of rows scaled by each factor.  Inside a diagonal
// sub-block the same split at the step before the block holds for every
// channel that decays by at most e^60 there (both factors stay in the normal
// range of fp32 and bf16), also on MFMA; the other channels of the block are
// taken in fp32 on the vector units, with the split at the end of the earlier
// 4-step group for pairs in different groups and the exact exponential within
// a group.
//
// Kernels:
//   vg_chunk_prep  one workgroup per (chunk, batch, value head), the channels
//                  in passes of 64: Gamma by per-wave running sums, the
//                  norms (factored out of the Gram sums), A and P, Tx by the
//                  blocked inverse of gdn_tri.h, and the pre-scaled rows and
//                  matrices the state passes and the gradient pass read (the
//                  forward's, the backward's, or both for the saved record).
//   vg_chunk_x     one workgroup per (chunk, batch, value head): X (the
//                  forward's saved copy, or recomputed from the fp32
//                  checkpoint), then
//     dP = lower(dO X^T) diag(beta),  dA = -strictlower(Ehat X^T) diag(beta),
//     db_t = (Ehat_t . X_t) (1 - beta_t),
//                  with Ehat = dv of the reverse state pass (dL/d beta_t =
//                  eps_t . X_t with eps = dL/d delta, and Ehat = diag(beta)
//                  eps, so eps itself is not needed).
//   vg_chunk_grad  one workgroup per (chunk, batch, value head, 32 channels):
//     dQb = dO H^T,  dKb = -Ehat H^T,  dKh = diag(beta) X dH'^T
//                  (dH' = dL/d the state at the chunk end), then, per channel
//                  i, the three roles of the rows (s the 1/sqrt(Dk) scale):
//     dq_t  = e^{G_t} dQb_t + sum_{u<=t} dP[t,u] kn_u e^{G_t-G_u}            (w.r.t. s qn)
//     dkR_t = e^{G_t} dKb_t + sum_{u<t}  dA[t,u] kn_u e^{G_t-G_u}            (k as a reader)
//     dkW_u = e^{G_L-G_u} dKh_u + sum_{t>=u} (dP[t,u] s qn_t + dA[t,u] kn_t) e^{G_t-G_u}  (writer)
//     dG_t  = s qn_t dq_t + kn_t (dkR_t - dkW_t) + [t = L-1] (e^{G_L} <dH', H> + sum_u Kh_u dKh_u)
//     dlg_t = sum_{t' >= t} dG_t' (0 on masked steps),   dkn = dkR + dkW;
//                  every e^{G} factor enters as e^{G_t - G_u} with u <= t (so
//                  lg enters through G_t - G_u only).  The expansions take the
//                  sub-blocks of the prep: MFMA with the split at the
//                  previous block's end off the diagonal, on the diagonal MFMA
//                  where the block's decays allow, else fp32 with decays built
//                  step by step.  Writes dlg and the value head's parts of the
//                  rows of dq, dkn.
//   vg_norm_bwd    one wave per (batch, step, key head): the parts of the key
//                  head's value heads summed, and the L2-normalisation
//                  backward of q and k.
#include "gdn_dev.h"
#include "gdn_internal.h"
#include "gdn_tri.h"

namespace gdn {
namespace {

constexpr int L = kChunk;
constexpr int NT = 256;
// Largest in-block decay exponent the MFMA form of a diagonal block takes.
constexpr float kDiagSpan = 60.f;

// Tiles (tt, uu), uu <= tt, of a 16 x 16 diagonal sub-block in 4 x 4 steps:
// index tt (tt + 1) / 2 + uu.
__device__ __forceinline__ int tile_t(int ti) { return static_cast<int>((0x3333222110ull >> (4 * ti)) & 15); }
__device__ __forceinline__ int tile_u(int ti) { return static_cast<int>((0x3210210100ull >> (4 * ti)) & 15); }

__device__ __forceinline__ void unpack8(uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(w[e] << 16);
    f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}
// Sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ float lanes_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]), pack2_bf16(f[4], f[5]), pack2_bf16(f[6], f[7]));
}

template <int DK>
struct VgPrep {
  // The channels go through in passes of CW: the staged k / q / Gamma rows of
  // one pass (36 KB) share the LDS with the matrices of the last phase (52
  // KB), which leaves room for two workgroups per compute unit.  The Gram
  // sums take raw rows times the decays; the norms factor out of every sum
  // (A[t,s] = rk_t rk_s sum_i k_ti k_si e^{...}) and are applied at the end.
  static constexpr int CW = 64;          // channels per pass
  static constexpr int NPASS = DK / CW;
  static constexpr int RS = CW + 8;      // bf16 row stride of the staged k / q rows
  static constexpr int GS = CW + 4;      // fp32 row stride of Gamma
  static constexpr int SP = tri::SP;
  static constexpr int NTASK = 40;       // (sub-block, 4x4 tile) tasks of the far channels
  static constexpr int NLD = L * CW / 8 / NT;  // 16-byte pieces of one of k, q per thread and pass
  static constexpr int NLG = L * CW / 4 / NT;  // 16-byte pieces of lg per thread and pass
  static_assert(DK % CW == 0 && L * CW / 8 % NT == 0 && L * CW / 4 % NT == 0, "whole pieces per thread");
  struct Rows {
    bf16 k[L * RS];
    bf16 q[L * RS];
    float gam[L * GS];
  };
  struct Mats {
    float nf[L * SP];   // N (its diagonal 16x16 blocks replaced by their inverses)
    float st[L * SP];   // Mq, or A^T, then Tx
    float st2[L * SP];  // P^T
  };
  union Big {
    Rows r;
    Mats m;
  };
  struct Smem {
    alignas(16) Big u;
    alignas(16) float dp[NTASK * 32];  // far-channel sums of the diagonal sub-blocks: 16 of A, 16 of P per task
    alignas(16) float dg[4][2][16][17];  // diagonal sub-blocks over the channels in range (A, P)
    float rk[L], rq[L], beta[L], valid[L];
    unsigned char far[4][CW];            // channel c0 + i decays by more than e^kDiagSpan inside sub-block I
    unsigned long long fmask[4];         // the same as bits
    float gtot[4][CW];                   // per wave: the sum of lg over its 16 steps
  };

  __device__ static void run(const VgChunkPrepArgs& p, Smem& sm) {
    const Dims& d = p.d;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int G = d.G(), NC = d.nchunk();
    const int b = bh / d.Hv, h = bh % d.Hv, j = h / G;
    const int t0 = c * L, Lc = min(L, d.T - t0), tl = Lc - 1;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    // mode 0: the forward's outputs; 1: the backward's; 2: both (saved record)
    const bool fwd = p.bwd != 1, bwd = p.bwd != 0;
    const size_t qk0 = (static_cast<size_t>(b) * d.T + t0) * d.Hk + j;
    const uint32_t qk_row = d.Hk * DK;
    const bf16* kc = static_cast<const bf16*>(p.k) + qk0 * DK;
    const bf16* qc = static_cast<const bf16*>(p.q) + qk0 * DK;
    const uint32_t lg_row = d.Hv * DK;
    const float* lgc = p.lg + ((static_cast<size_t>(b) * d.T + t0) * d.Hv + h) * DK;
    const size_t cidx = static_cast<size_t>(bh) * NC + c;
    const size_t rowbase = cidx * L * DK;

    // ---- the first pass's rows, then the norm factors (four lanes per row,
    // from the whole rows) and beta and the step's validity (wave 0)
    {
      const int t = tid >> 2, part = tid & 3;
      const uint32_t o = static_cast<uint32_t>(min(t, tl)) * qk_row + (DK / 4) * part;
      constexpr int NQ = DK / 4 / 8;  // 16-byte pieces of a quarter row
      float kk = 0.f, qq = 0.f;
#pragma unroll
      for (int e = 0; e < NQ; ++e) {
        float kf[8], qf[8];
        unpack8(*reinterpret_cast<const uint4*>(kc + o + 8 * e), kf);
        unpack8(*reinterpret_cast<const uint4*>(qc + o + 8 * e), qf);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          kk = fmaf(kf[x], kf[x], kk);
          qq = fmaf(qf[x], qf[x], qq);
        }
      }
      kk = quad_sum(kk);
      qq = quad_sum(qq);
      if (part == 0) {
        const bool in = t < Lc;
        sm.rk[t] = in ? 1.f / sqrtf(kk + kNormEps) : 0.f;
        sm.rq[t] = in ? (1.f / sqrtf(static_cast<float>(DK))) / sqrtf(qq + kNormEps) : 0.f;
      }
    }
    if (w == 0) {
      const int t = min(l, tl);
      const size_t o = (static_cast<size_t>(b) * d.T + t0 + t) * d.Hv + h;
      const float bv = to_f32(static_cast<const bf16*>(p.b)[o]);
      const rsrc_t rm = make_rsrc(p.mask ? static_cast<const void*>(p.mask) : p.b,
                                  p.mask ? static_cast<size_t>(d.B) * d.T : 0);
      const uint32_t mrow = static_cast<uint32_t>(b * d.T + t0 + t);
      const bool valid = l < Lc && (p.mask == nullptr || __builtin_amdgcn_raw_buffer_load_b8(rm, mrow, 0, 0) != 0);
      sm.beta[l] = valid ? sigmoid_f(bv) : 0.f;
      sm.valid[l] = valid ? 1.f : 0.f;
    }

    // sums over the passes: A and P off the diagonal sub-blocks (waves 1..3:
    // row block I = w against the column blocks J < I, reference r = 16 I - 1),
    // the diagonal sub-block w over the channels in range, and the far
    // channels' fp32 tasks (threads < NTASK), all of raw rows
    f32x4 accA[3], accP[3], da = f4zero(), dpq = f4zero();
#pragma unroll
    for (int J = 0; J < 3; ++J) accA[J] = accP[J] = f4zero();
    float pa[16], pp[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) pa[x] = pp[x] = 0.f;

#pragma unroll
    for (int pc = 0; pc < NPASS; ++pc) {
      const int c0 = pc * CW;
      // the pass's k / q / lg rows (clamped into the sequence), all loads
      // issued before any is used
      // (vector-typed registers: arrays of the HIP vector structs would be
      // copied through private memory)
      u32x4 kv[NLD], qv[NLD], gv[NLG];
#pragma unroll
      for (int e = 0; e < NLD; ++e) {
        const int u = tid + e * NT, t = u / (CW / 8), i8 = 8 * (u % (CW / 8));
        const uint32_t o = static_cast<uint32_t>(min(t, tl)) * qk_row + c0 + i8;
        kv[e] = *reinterpret_cast<const u32x4*>(kc + o);
        qv[e] = *reinterpret_cast<const u32x4*>(qc + o);
      }
#pragma unroll
      for (int e = 0; e < NLG; ++e) {
        const int u = tid + e * NT, t = u / (CW / 4), i4 = 4 * (u % (CW / 4));
        gv[e] = *reinterpret_cast<const u32x4*>(lgc + static_cast<uint32_t>(min(t, tl)) * lg_row + c0 + i4);
      }
      if (pc > 0) __syncthreads();  // the previous pass is done with the staged rows
#pragma unroll
      for (int e = 0; e < NLD; ++e) {
        const int u = tid + e * NT, t = u / (CW / 8), i8 = 8 * (u % (CW / 8));
        *reinterpret_cast<u32x4*>(&sm.u.r.k[t * RS + i8]) = kv[e];
        *reinterpret_cast<u32x4*>(&sm.u.r.q[t * RS + i8]) = qv[e];
      }
#pragma unroll
      for (int e = 0; e < NLG; ++e) {
        const int u = tid + e * NT, t = u / (CW / 4), i4 = 4 * (u % (CW / 4));
        *reinterpret_cast<u32x4*>(&sm.u.r.gam[t * GS + i4]) = gv[e];
      }
      __syncthreads();

      // ---- Gamma: wave w sums steps 16 w .. 16 w + 15 of channel l of the
      // pass in turn (a masked step or a row past the end adds 0), then adds
      // the earlier waves' totals in order; the far flags of sub-block w
      {
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) x[t] = sm.valid[16 * w + t] * sm.u.r.gam[(16 * w + t) * GS + l];
#pragma unroll
        for (int t = 1; t < 16; ++t) x[t] += x[t - 1];
        sm.gtot[w][l] = x[15];
        __syncthreads();
        float before = 0.f;  // G at the step before the block (0 before the chunk)
        for (int J = 0; J < w; ++J) before += sm.gtot[J][l];
#pragma unroll
        for (int t = 0; t < 16; ++t) sm.u.r.gam[(16 * w + t) * GS + l] = x[t] + before;
        const int f = before - (x[15] + before) > kDiagSpan ? 1 : 0;
        sm.far[w][l] = static_cast<unsigned char>(f);
        const unsigned long long m = __ballot(f);
        if (l == 0) sm.fmask[w] = m;
      }
      __syncthreads();

      // ---- A and P off the diagonal sub-blocks
      if (w >= 1) {
        const int I = w, r = 16 * I - 1, ta = 16 * I + lr;
#pragma unroll
        for (int kt = 0; kt < CW / 32; ++kt) {
          const int i0 = 32 * kt + 8 * lg;
          float kf[8], qf[8];
          unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.k[ta * RS + i0]), kf);
          unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.q[ta * RS + i0]), qf);
          float gr[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            gr[x] = sm.u.r.gam[r * GS + i0 + x];
            const float ex = __expf(sm.u.r.gam[ta * GS + i0 + x] - gr[x]);
            kf[x] *= ex;
            qf[x] *= ex;
          }
          const bf16x8 ak = as_bf16x8(pack8(kf)), aq = as_bf16x8(pack8(qf));
#pragma unroll
          for (int J = 0; J < 3; ++J) {
            if (J >= I) continue;
            const int su = 16 * J + lr;
            float uf[8];
            unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.k[su * RS + i0]), uf);
#pragma unroll
            for (int x = 0; x < 8; ++x) uf[x] *= __expf(gr[x] - sm.u.r.gam[su * GS + i0 + x]);
            const bf16x8 bk = as_bf16x8(pack8(uf));
            accA[J] = mfma16(ak, bk, accA[J]);
            accP[J] = mfma16(aq, bk, accP[J]);
          }
        }
      }

      // ---- the diagonal sub-blocks: wave w takes sub-block w on MFMA with the
      // split at c = 16 w - 1 (G_{-1} = 0) over the channels that decay by at
      // most e^kDiagSpan inside it (both factors then stay in the normal range)
      {
        const int b0 = 16 * w, ta = b0 + lr;
#pragma unroll
        for (int kt = 0; kt < CW / 32; ++kt) {
          const int i0 = 32 * kt + 8 * lg;
          float kf[8], qf[8];
          unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.k[ta * RS + i0]), kf);
          unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.q[ta * RS + i0]), qf);
          float ka[8], kb[8], qa[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const float gcx = w == 0 ? 0.f : sm.u.r.gam[(b0 - 1) * GS + i0 + x];
            const float gx = sm.u.r.gam[ta * GS + i0 + x];
            const bool near = sm.far[w][i0 + x] == 0;
            const float dn = near ? __expf(gx - gcx) : 0.f, up = near ? __expf(gcx - gx) : 0.f;
            ka[x] = kf[x] * dn;
            qa[x] = qf[x] * dn;
            kb[x] = kf[x] * up;
          }
          const bf16x8 akb = as_bf16x8(pack8(ka)), aqb = as_bf16x8(pack8(qa)), bkb = as_bf16x8(pack8(kb));
          // the B operand is row s = ta of the same sub-block: each lane holds both
          da = mfma16(akb, bkb, da);
          dpq = mfma16(aqb, bkb, dpq);
        }
      }

      // ---- ... and in fp32 for the far channels: task (block I, 4x4 tile)
      if (tid < NTASK) {
        const int I = tid / 10, ti = tid % 10;
        const int tt = tile_t(ti), uu = tile_u(ti);
        const int tb = 16 * I + 4 * tt, ub = 16 * I + 4 * uu;
        const bool split = tt > uu;  // different 4-step groups: split at the end of ub's group
        unsigned long long m = sm.fmask[I];
        while (m) {
          const int i = __builtin_ctzll(m);
          m &= m - 1;
          float gt[4], gu[4], kt_[4], qt_[4], ku[4];
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            gt[a] = sm.u.r.gam[(tb + a) * GS + i];
            gu[a] = sm.u.r.gam[(ub + a) * GS + i];
            kt_[a] = to_f32(sm.u.r.k[(tb + a) * RS + i]);
            qt_[a] = to_f32(sm.u.r.q[(tb + a) * RS + i]);
            ku[a] = to_f32(sm.u.r.k[(ub + a) * RS + i]);
          }
          if (split) {
            float e1k[4], e1q[4], e2[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const float e1 = __expf(gt[a] - gu[3]);
              e1k[a] = kt_[a] * e1;
              e1q[a] = qt_[a] * e1;
              e2[a] = ku[a] * __expf(gu[3] - gu[a]);
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
              for (int bb = 0; bb < 4; ++bb) {
                pa[4 * a + bb] = fmaf(e1k[a], e2[bb], pa[4 * a + bb]);
                pp[4 * a + bb] = fmaf(e1q[a], e2[bb], pp[4 * a + bb]);
              }
          } else {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
              for (int bb = 0; bb <= a; ++bb) {
                const float e = ku[bb] * __expf(gt[a] - gu[bb]);
                pa[4 * a + bb] = fmaf(kt_[a], e, pa[4 * a + bb]);
                pp[4 * a + bb] = fmaf(qt_[a], e, pp[4 * a + bb]);
              }
          }
        }
      }

      // ---- the pre-scaled rows of the pass's channels: Kb, Kh ([t][i]);
      // forward Qb ([t][i]); backward Kb^T, Qb^T ([i][t]); e^{G_L}
      for (int u = tid; u < L * CW / 8; u += NT) {
        const int t = u / (CW / 8), i0 = 8 * (u % (CW / 8));
        float kf[8], qf[8], kh[8];
        unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.k[t * RS + i0]), kf);
        unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.q[t * RS + i0]), qf);
        const float rkt = sm.rk[t], rqt = sm.rq[t];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float g = sm.u.r.gam[t * GS + i0 + x], gl = sm.u.r.gam[(L - 1) * GS + i0 + x];
          const float e = __expf(g);
          kh[x] = kf[x] * rkt * __expf(gl - g);
          kf[x] *= rkt * e;
          qf[x] *= rqt * e;
        }
        const size_t o = rowbase + static_cast<size_t>(t) * DK + c0 + i0;
        *reinterpret_cast<uint4*>(p.cb.Kh + o) = pack8(kh);
        *reinterpret_cast<uint4*>(p.cb.Kb + o) = pack8(kf);
        if (fwd) *reinterpret_cast<uint4*>(p.cb.Qb + o) = pack8(qf);
      }
      if (bwd) {
        for (int u = tid; u < CW * L / 8; u += NT) {
          const int i = u % CW, t8 = 8 * (u / CW);
          float kf[8], qf[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int t = t8 + x;
            const float e = __expf(sm.u.r.gam[t * GS + i]);
            kf[x] = to_f32(sm.u.r.k[t * RS + i]) * sm.rk[t] * e;
            qf[x] = to_f32(sm.u.r.q[t * RS + i]) * sm.rq[t] * e;
          }
          const size_t o = rowbase + static_cast<size_t>(c0 + i) * L + t8;
          *reinterpret_cast<uint4*>(p.cb.KbT + o) = pack8(kf);
          *reinterpret_cast<uint4*>(p.cb.QbT + o) = pack8(qf);
        }
      }
      if (tid < CW) p.cb.vsc[cidx * VSC_ROWS * L + VSC_EGL * L + c0 + tid] = __expf(sm.u.r.gam[(L - 1) * GS + tid]);
    }

    // ---- the chunk scalars beyond the passes: beta, and zeros past e^{G_L}
    {
      float* vsc = p.cb.vsc + cidx * VSC_ROWS * L;
      if (tid < L) vsc[VSC_BETA * L + tid] = sm.beta[tid];
      for (int i = DK + tid; i < (VSC_ROWS - 1) * L; i += NT) vsc[VSC_EGL * L + i] = 0.f;
    }
    // the norm factors of the sums; the diagonal sub-blocks' MFMA part and the
    // far channels' raw sums (scaled by the norms where they are added)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * w + 4 * lg + r, s = 16 * w + lr;
      sm.dg[w][0][4 * lg + r][lr] = da[r] * sm.rk[t] * sm.rk[s];
      sm.dg[w][1][4 * lg + r][lr] = dpq[r] * sm.rq[t] * sm.rk[s];
    }
    if (w >= 1) {
#pragma unroll
      for (int J = 0; J < 3; ++J)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * w + 4 * lg + r, s = 16 * J + lr;
          accA[J][r] *= sm.rk[t] * sm.rk[s];
          accP[J][r] *= sm.rq[t] * sm.rk[s];
        }
    }
    if (tid < NTASK) {
      float* dst = &sm.dp[tid * 32];
#pragma unroll
      for (int x = 0; x < 16; x += 4) {
        *reinterpret_cast<float4*>(&dst[x]) = make_float4(pa[x], pa[x + 1], pa[x + 2], pa[x + 3]);
        *reinterpret_cast<float4*>(&dst[16 + x]) = make_float4(pp[x], pp[x + 1], pp[x + 2], pp[x + 3]);
      }
    }
    __syncthreads();  // the staged rows and Gamma are dead from here on
    // ---- N = A diag(beta) and Mq = P diag(beta) (forward only), or A^T, P^T
    // (backward, and both; Mq then comes from P^T); every element written
    // once: the lower off-diagonal sub-blocks by the MFMA waves, the rest here
    float* nf = sm.u.m.nf;
    float* st = sm.u.m.st;
    float* st2 = sm.u.m.st2;
    if (w >= 1) {
      const int I = w;
#pragma unroll
      for (int J = 0; J < 3; ++J) {
        if (J >= I) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * I + 4 * lg + r, s = 16 * J + lr;
          const float bs = sm.beta[s];
          nf[t * SP + s] = accA[J][r] * bs;
          if (bwd) {
            st[s * SP + t] = accA[J][r];
            st2[s * SP + t] = accP[J][r];
          } else {
            st[t * SP + s] = accP[J][r] * bs;
          }
        }
      }
    }
    // the diagonal sub-blocks: the MFMA part plus the far channels' sums
    for (int e = tid; e < 4 * 256; e += NT) {
      const int bi = e >> 8, t = 16 * bi + ((e >> 4) & 15), s = 16 * bi + (e & 15);
      const int tt = (t >> 2) & 3, uu = (s >> 2) & 3;
      float av = sm.dg[bi][0][t & 15][s & 15], pv = sm.dg[bi][1][t & 15][s & 15];
      if (uu <= tt) {  // the far sums (zero where no channel was far)
        const int x = 4 * (t & 3) + (s & 3), rest = bi * 10 + tt * (tt + 1) / 2 + uu;
        av += sm.dp[rest * 32 + x] * sm.rk[t] * sm.rk[s];
        pv += sm.dp[rest * 32 + 16 + x] * sm.rq[t] * sm.rk[s];
      }
      av = s < t ? av : 0.f;
      pv = s <= t ? pv : 0.f;
      const float bs = sm.beta[s];
      nf[t * SP + s] = av * bs;
      if (bwd) {
        st2[s * SP + t] = pv;
      } else {
        st[t * SP + s] = pv * bs;
      }
    }
    // zeros above the diagonal sub-blocks: pairs (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
    for (int e = tid; e < 6 * 256; e += NT) {
      const int pr = e >> 8, bi = (0x211000 >> (4 * pr)) & 15, bj = (0x332321 >> (4 * pr)) & 15;
      const int t = 16 * bi + ((e >> 4) & 15), s = 16 * bj + (e & 15);
      nf[t * SP + s] = 0.f;
      if (bwd) {
        st2[s * SP + t] = 0.f;
      } else {
        st[t * SP + s] = 0.f;
      }
    }
    __syncthreads();

    // ---- Tx = (I + N)^-1, and the stores
    tri::invert_diagonal_block(nf, w, l);
    const size_t mat = cidx * L * L;
    if (bwd) {
      tri::store_mat(st2, p.cb.PqT + mat, tid, NT);
      if (fwd) {  // Mq[t][s] = P^T[s][t] beta_s: row t, columns s8 .. s8 + 7 per thread
        for (int u = tid; u < L * L / 8; u += NT) {
          const int t = u >> 3, s8 = 8 * (u & 7);
          float mv[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) mv[x] = st2[(s8 + x) * SP + t] * sm.beta[s8 + x];
          *reinterpret_cast<uint4*>(p.cb.Mq + mat + t * L + s8) = pack8(mv);
        }
      }
    } else {
      tri::store_mat(st, p.cb.Mq + mat, tid, NT);
    }
    __syncthreads();  // st is free; the D_i are visible
    if (w < 3)
      tri::lower_blocks(nf, st, w);
    else
      tri::diagonal_blocks(nf, st, l);
    __syncthreads();
    tri::store_mat(st, p.cb.Tx + mat, tid, NT);
  }
};

template <int DK>
__global__ void __launch_bounds__(NT) vg_chunk_prep_kernel(VgChunkPrepArgs p) {
  __shared__ typename VgPrep<DK>::Smem sm;
  VgPrep<DK>::run(p, sm);
}


// ------------------------------------------------------------ gradient pass

// vg_chunk_x: X = Tx (V - Kb H) from the fp32 checkpoint H (XSV: X read
// from the forward's saved copy instead), then dP = lower(dO X^T) diag(beta),
// dA = -strictlower(Ehat X^T) diag(beta) and db_t = (Ehat_t . X_t) (1 -
// beta_t).  Writes dP, dA, db (bf16) and, when it computes X, X ([B,T,Hv,Dv]
// bf16, the layout the forward saves it in).  Wave w takes steps 16 w .. 16 w
// + 15.
template <int DK, int DV, bool XSV>
struct VgX {
  static constexpr int NV = DV / 32;
  static constexpr int NVT = DV / 16;
  static constexpr int HS = DV + 8;  // bf16 row stride of H [i][v]
  static constexpr int TS = L + 8;   // bf16 row stride of the L-wide tiles
  static constexpr int XS = DV + 8;  // bf16 row stride of X
  static constexpr int HN = DK * HS > L * XS ? DK * HS : L * XS;
  static constexpr int RTN = (DV > L ? DV : L) * TS;
  struct SmemFull {
    alignas(16) bf16 hs[HN];    // H [i][v] (bf16); X [t][v] takes its place
    alignas(16) bf16 rT[RTN];   // R^T [v][s]; dP [t][s] later
    alignas(16) bf16 txs[L * TS];  // Tx [t][s]; dA [t][s] later
    float beta[L];
  };
  struct SmemSaved {
    alignas(16) bf16 xs[L * XS];  // X [t][v]
    alignas(16) bf16 dP[L * TS];
    alignas(16) bf16 dA[L * TS];
    float beta[L];
  };
  using Smem = std::conditional_t<XSV, SmemSaved, SmemFull>;

  // X = Tx (V - Kb H) of the chunk into xs (rows [t][v]), from the fp32
  // checkpoint; every wave has passed the last barrier when it returns.
  __device__ static void compute_x(const VgChunkGradArgs& p, SmemFull& sm, const float* H, size_t cidx,
                                   size_t vrow0, int tl, int tid, int w, int lr, int lg) {
    const Dims& d = p.d;
    bf16* xs = sm.hs;
    // ---- H (bf16, rows [i][v]) and Tx
    for (int u = tid; u < DK * DV / 4; u += NT) {
      const int i = u / (DV / 4), v4 = 4 * (u % (DV / 4));
      const float4 x = H ? *reinterpret_cast<const float4*>(H + static_cast<size_t>(i) * DV + v4)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<uint2*>(&sm.hs[i * HS + v4]) = pack4_bf16(x.x, x.y, x.z, x.w);
    }
    {
      const bf16* txg = p.cb.Tx + cidx * L * L;
      for (int u = tid; u < L * L / 8; u += NT) {
        const int t = u >> 3, s8 = 8 * (u & 7);
        *reinterpret_cast<uint4*>(&sm.txs[t * TS + s8]) = *reinterpret_cast<const uint4*>(txg + t * L + s8);
      }
    }
    __syncthreads();

    // ---- R^T = V^T - H^T Kb^T (Kb rows from the prep: zero past the end); the
    // rows of H^T by transposing reads of H: rows i0 .. i0 + 7 of column
    // 16 vt + lr
    {
      const int tb = 16 * w + lr;
      const bf16* kbr = p.cb.Kb + (cidx * L + tb) * DK;
      f32x4 acc[NVT];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) acc[vt] = f4zero();
#pragma unroll
      for (int kt = 0; kt < DK / 32; ++kt) {
        const int i0 = 32 * kt + 8 * lg;
        const bf16x8 kb = as_bf16x8(*reinterpret_cast<const uint4*>(kbr + i0));
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
          const uint2 lo = lds_read_tr16(&sm.hs[(i0 + (lr >> 2)) * HS + 16 * vt + 4 * (lr & 3)]);
          const uint2 hi = lds_read_tr16(&sm.hs[(i0 + 4 + (lr >> 2)) * HS + 16 * vt + 4 * (lr & 3)]);
          acc[vt] = mfma16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), kb, acc[vt]);
        }
      }
      const bf16* vg = static_cast<const bf16*>(p.v) + (vrow0 + static_cast<size_t>(min(tb, tl)) * d.Hv) * DV;
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const uint2 v4 = *reinterpret_cast<const uint2*>(vg + 16 * vt + 4 * lg);
        const float vv[4] = {__uint_as_float(v4.x << 16), __uint_as_float(v4.x & 0xffff0000u),
                             __uint_as_float(v4.y << 16), __uint_as_float(v4.y & 0xffff0000u)};
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.rT[(16 * vt + 4 * lg + r) * TS + tb] = bf16_of(vv[r] - acc[vt][r]);
      }
    }
    __syncthreads();

    // ---- X = Tx R, into H^T's place
    {
      f32x4 xa[NVT];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) xa[vt] = f4zero();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 a = load_bf16x8(&sm.txs[(16 * w + lr) * TS + 32 * kk + 8 * lg]);
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
          xa[vt] = mfma16(a, load_bf16x8(&sm.rT[(16 * vt + lr) * TS + 32 * kk + 8 * lg]), xa[vt]);
      }
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r) xs[(16 * w + 4 * lg + r) * XS + 16 * vt + lr] = bf16_of(xa[vt][r]);
    }
    __syncthreads();
  }

  __device__ static void run(const VgChunkGradArgs& p, Smem& sm) {
    const Dims& d = p.d;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int NC = d.nchunk();
    const int b = bh / d.Hv, h = bh % d.Hv;
    const int t0 = c * L, Lc = min(L, d.T - t0), tl = Lc - 1;
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t vrow0 = (static_cast<size_t>(b) * d.T + t0) * d.Hv + h;
    const size_t cidx = static_cast<size_t>(bh) * NC + c;
    bf16 *xs, *dPs, *dAs;
    if (tid < L) sm.beta[tid] = p.cb.vsc[cidx * VSC_ROWS * L + VSC_BETA * L + tid];
    if constexpr (XSV) {
      xs = sm.xs;
      dPs = sm.dP;
      dAs = sm.dA;
      // the saved X rows (clamped into the sequence: rows past the end meet
      // beta = 0 or a zero norm factor wherever they are used)
      for (int u = tid; u < L * DV / 8; u += NT) {
        const int t = u / (DV / 8), v8 = 8 * (u % (DV / 8));
        *reinterpret_cast<uint4*>(&xs[t * XS + v8]) =
            *reinterpret_cast<const uint4*>(p.X + (vrow0 + static_cast<size_t>(min(t, tl)) * d.Hv) * DV + v8);
      }
      __syncthreads();
    } else {
      xs = sm.hs;
      dPs = sm.rT;
      dAs = sm.txs;
      const float* H = c == 0 ? (p.state0 ? p.state0 + static_cast<size_t>(bh) * DK * DV : nullptr)
                              : p.ckpt + (static_cast<size_t>(c - 1) * d.B * d.Hv + bh) * DK * DV;
      compute_x(p, sm, H, cidx, vrow0, tl, tid, w, lr, lg);
    }

    // ---- dO X^T, Ehat X^T -> dP, dA; db; X out
    {
      const int ta = 16 * w + lr;
      const size_t ro = (vrow0 + static_cast<size_t>(min(ta, tl)) * d.Hv) * DV;
      const bf16* dOg = static_cast<const bf16*>(p.dO) + ro;
      const bf16* Eg = static_cast<const bf16*>(p.dv) + ro;
      f32x4 g1[4], g2[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) g1[st] = g2[st] = f4zero();
#pragma unroll
      for (int kv = 0; kv < NV; ++kv) {
        const bf16x8 dof = as_bf16x8(*reinterpret_cast<const uint4*>(dOg + 32 * kv + 8 * lg));
        const bf16x8 ef = as_bf16x8(*reinterpret_cast<const uint4*>(Eg + 32 * kv + 8 * lg));
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16x8 bx = load_bf16x8(&xs[(16 * st + lr) * XS + 32 * kv + 8 * lg]);
          g1[st] = mfma16(dof, bx, g1[st]);
          g2[st] = mfma16(ef, bx, g2[st]);
        }
      }
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * w + 4 * lg + r, s = 16 * st + lr;
          const float bs = sm.beta[s];
          dPs[t * TS + s] = bf16_of(s <= t ? g1[st][r] * bs : 0.f);
          dAs[t * TS + s] = bf16_of(s < t ? -g2[st][r] * bs : 0.f);
        }
    }
    {  // db_t = (dv_t . X_t) (1 - beta_t), four lanes per step (0 on masked steps: dv 0)
      const int t = tid >> 2, part = tid & 3;
      const bf16* eg = static_cast<const bf16*>(p.dv) + (vrow0 + static_cast<size_t>(min(t, tl)) * d.Hv) * DV;
      float sdot = 0.f;
#pragma unroll
      for (int e = 0; e < DV / 32; ++e) {
        const int v0 = (DV / 4) * part + 8 * e;
        float ef[8], xf[8];
        unpack8(*reinterpret_cast<const uint4*>(eg + v0), ef);
        unpack8(*reinterpret_cast<const uint4*>(&xs[t * XS + v0]), xf);
#pragma unroll
        for (int x = 0; x < 8; ++x) sdot = fmaf(ef[x], xf[x], sdot);
      }
      sdot = quad_sum(sdot);
      const float bt = sm.beta[t];
      if (part == 0 && t < Lc) static_cast<bf16*>(p.db)[vrow0 + static_cast<size_t>(t) * d.Hv] = bf16_of(sdot * (1.f - bt));
    }
    if constexpr (!XSV) {  // rows of the sequence only
      for (int u = tid; u < L * DV / 8; u += NT) {
        const int t = u / (DV / 8), v8 = 8 * (u % (DV / 8));
        if (t < Lc)
          *reinterpret_cast<uint4*>(p.X + (vrow0 + static_cast<size_t>(t) * d.Hv) * DV + v8) =
              *reinterpret_cast<const uint4*>(&xs[t * XS + v8]);
      }
    }
    __syncthreads();
    {
      bf16* pg = p.dPA + cidx * 2 * L * L;
      for (int u = tid; u < 2 * L * L / 8; u += NT) {
        const int m = u / (L * L / 8), r = u % (L * L / 8), t = r >> 3, s8 = 8 * (r & 7);
        const bf16* src = m ? dAs : dPs;
        *reinterpret_cast<uint4*>(pg + m * L * L + t * L + s8) = *reinterpret_cast<const uint4*>(&src[t * TS + s8]);
      }
    }
  }
};

// vg_chunk_grad: the per-channel expansions for CH channels of one (chunk,
// head).  Every global read of the workgroup is issued at its start (the
// chunk's dP and dA, the CH channels of lg, k, q, H and dH', this wave's dO,
// Ehat and diag(beta) X rows), so it waits on memory once; the rest runs from
// LDS and registers.  Wave w takes the 16-step block w, in the matrix-core
// output layout: lane (lr, lg) holds steps 16 w + 4 lg + r (r < 4) of channel
// lr of the current 16-channel tile, as a row (dq, dkR: sums over the earlier
// steps) and as a column (dkW: sums over the later steps).  The direct terms
// and the parts off the diagonal blocks are MFMA products (the blocks before
// w split at r = 16 w - 1, those after it at e = 16 w + 15), the diagonal
// block too where its decays allow, else fp32 with the decays built step by
// step.  The in-chunk suffix sums of dG run over r, the lanes of a block and
// the blocks.  Gamma, k and q are held channel-major (the expansions read 8 or
// 16 consecutive steps of one channel); the transposed operands of dP and dA
// come from transposing LDS reads.
template <int DK, int DV, bool HBF>
struct VgG {
  static constexpr int CH = kVgGradChannels;
  static constexpr int NTL = CH / 16;  // 16-channel tiles per workgroup
  static constexpr int NV = DV / 32;
  static constexpr int GT = L + 4;     // fp32 row stride of the channel-major Gamma
  static constexpr int KT = L + 8;     // bf16 row stride of the channel-major k, q
  static constexpr int TS = L + 8;     // bf16 row stride of dP, dA
  static constexpr int HS = DV + 4;    // fp32 row stride of H
  static constexpr int DS = DV + 8;    // bf16 row stride of dH'
  static constexpr int NPM = 2 * L * L / 8 / NT;      // 16-byte pieces of dP, dA per thread
  static constexpr int NLG = L * CH / 4 / NT;         // of lg
  static constexpr int NKQ = 2 * L * CH / 8 / NT;     // of k and q
  static constexpr int NH = CH * DV / 4 / NT;         // of H (fp32)
  static constexpr int NDHP = CH * DV / 8;             // pieces of dH'
  static constexpr int NDH = (NDHP + NT - 1) / NT;    // of dH' per thread (the last may be idle)
  static_assert(2 * L * L / 8 % NT == 0 && L * CH / 4 % NT == 0 && 2 * L * CH / 8 % NT == 0 &&
                CH * DV / 4 % NT == 0, "whole pieces per thread");
  struct Smem {
    alignas(16) float gT[CH * GT];
    alignas(16) bf16 kT[CH * KT];
    alignas(16) bf16 qT[CH * KT];
    alignas(16) bf16 dP[L * TS];
    alignas(16) bf16 dA[L * TS];
    alignas(16) float hs[CH * HS];
    alignas(16) bf16 dhs[CH * DS];
    alignas(16) float rk[L];
    alignas(16) float rq[L];
    float valid[L], beta[L];
    float btot[4][16], rdot[4][16], rdh[16];
  };

  // 8 consecutive steps s0 .. s0 + 7 of a channel-major row: fp32 and bf16
  __device__ static __forceinline__ void ld8f(const float* p, float (&f)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x, f[1] = a.y, f[2] = a.z, f[3] = a.w, f[4] = b.x, f[5] = b.y, f[6] = b.z, f[7] = b.w;
  }
  __device__ static __forceinline__ void ld8b(const bf16* p, float (&f)[8]) {
    unpack8(*reinterpret_cast<const uint4*>(p), f);
  }
  // Rows t0 .. t0 + 7 of column c0 + lr of a row-major [t][s] tile (stride
  // TS) as an MFMA operand (its transpose's row c0 + lr), by two transposing
  // reads; t0 is this lane group's (t0 = base + 8 lg).
  __device__ static __forceinline__ bf16x8 col8(const bf16* m, int t0, int c0, int lr) {
    const uint2 lo = lds_read_tr16(&m[(t0 + (lr >> 2)) * TS + c0 + 4 * (lr & 3)]);
    const uint2 hi = lds_read_tr16(&m[(t0 + 4 + (lr >> 2)) * TS + c0 + 4 * (lr & 3)]);
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
  }

  // Workgroup n -> (chunk c, head bh, channel group cg).  The DK / CH groups
  // of one (chunk, head) read the same dO, Ehat, X, dP and dA: they go to one
  // XCD (workgroups are dealt to the 8 XCDs round-robin in launch order) one
  // after another, so those reads hit that XCD's L2.  (chunk, head) pairs are
  // dealt to the XCDs in turn; the grid is padded to a multiple of 8 of them.
  __device__ static bool coords(const Dims& d, int& c, int& bh, int& cg) {
    const int NG = DK / CH, NC = d.nchunk();
    const int n = blockIdx.x, xcd = n & 7, m = n >> 3;
    cg = m % NG;
    const int pr = (m / NG) * 8 + xcd;
    if (pr >= NC * d.B * d.Hv) return false;
    c = pr % NC;
    bh = pr / NC;
    return true;
  }

  __device__ static void run(const VgChunkGradArgs& p, Smem& sm) {
    const Dims& d = p.d;
    int c, bh, cg;
    if (!coords(d, c, bh, cg)) return;
    const int G = d.G(), NC = d.nchunk();
    const int b = bh / d.Hv, h = bh % d.Hv, j = h / G;
    const int t0 = c * L, Lc = min(L, d.T - t0), tl = Lc - 1;
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ch0 = cg * CH;
    const size_t vrow0 = (static_cast<size_t>(b) * d.T + t0) * d.Hv + h;
    const size_t krow0 = (static_cast<size_t>(b) * d.T + t0) * d.Hk + j;
    const size_t cidx = static_cast<size_t>(bh) * NC + c;
    // H: the fp32 checkpoint (or state0), or (HBF) the saved bf16 state at the chunk start
    const float* H = c == 0 ? (p.state0 ? p.state0 + static_cast<size_t>(bh) * DK * DV : nullptr)
                            : p.ckpt + (static_cast<size_t>(c - 1) * d.B * d.Hv + bh) * DK * DV;
    const bf16* Hb = HBF ? p.cb.Hb + (static_cast<size_t>(c) * d.B * d.Hv + bh) * DK * DV : nullptr;
    const bf16* dHp = p.dHend + (static_cast<size_t>(c) * d.B * d.Hv + bh) * DK * DV;

    // ---- every global read, issued before any is used
    uint4 pmv[NPM], kqv[NKQ], dhv[NDH];
    float4 lgv[NLG], hv[NH];
    bf16x8 dOf[NV], Ef[NV], bXf[NV];
    {
      const bf16* pg = p.dPA + cidx * 2 * L * L;
#pragma unroll
      for (int e = 0; e < NPM; ++e) pmv[e] = *reinterpret_cast<const uint4*>(pg + 8 * (tid + e * NT));
#pragma unroll
      for (int e = 0; e < NLG; ++e) {
        const int u = tid + e * NT, t = u / (CH / 4), i4 = 4 * (u % (CH / 4));
        lgv[e] = *reinterpret_cast<const float4*>(p.lg + (vrow0 + static_cast<size_t>(min(t, tl)) * d.Hv) * DK + ch0 + i4);
      }
#pragma unroll
      for (int e = 0; e < NKQ; ++e) {
        const int u = tid + e * NT, m = u / (L * CH / 8), r = u % (L * CH / 8), t = r / (CH / 8), i8 = 8 * (r % (CH / 8));
        const bf16* src = static_cast<const bf16*>(m ? p.q : p.k) + (krow0 + static_cast<size_t>(min(t, tl)) * d.Hk) * DK;
        kqv[e] = *reinterpret_cast<const uint4*>(src + ch0 + i8);
      }
#pragma unroll
      for (int e = 0; e < NH; ++e) {
        const int u = tid + e * NT, ch = u / (DV / 4), v4 = 4 * (u % (DV / 4));
        if constexpr (HBF) {
          const uint2 h4 = *reinterpret_cast<const uint2*>(Hb + static_cast<size_t>(ch0 + ch) * DV + v4);
          hv[e] = make_float4(__uint_as_float(h4.x << 16), __uint_as_float(h4.x & 0xffff0000u),
                              __uint_as_float(h4.y << 16), __uint_as_float(h4.y & 0xffff0000u));
        } else {
          hv[e] = H ? *reinterpret_cast<const float4*>(H + static_cast<size_t>(ch0 + ch) * DV + v4)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int e = 0; e < NDH; ++e) {  // clamped: a thread past the last piece reloads it
        const int u = min(tid + e * NT, NDHP - 1), ch = u / (DV / 8), v8 = 8 * (u % (DV / 8));
        dhv[e] = *reinterpret_cast<const uint4*>(dHp + static_cast<size_t>(ch0 + ch) * DV + v8);
      }
      const int ta = 16 * w + lr;
      const size_t ro = (vrow0 + static_cast<size_t>(min(ta, tl)) * d.Hv) * DV;
      const bf16* dOg = static_cast<const bf16*>(p.dO) + ro;
      const bf16* Eg = static_cast<const bf16*>(p.dv) + ro;
      const bf16* Xg = p.X + ro;  // [B,T,Hv,Dv], the row of dO's
#pragma unroll
      for (int kv = 0; kv < NV; ++kv) {
        dOf[kv] = as_bf16x8(*reinterpret_cast<const uint4*>(dOg + 32 * kv + 8 * lg));
        Ef[kv] = as_bf16x8(*reinterpret_cast<const uint4*>(Eg + 32 * kv + 8 * lg));
        bXf[kv] = as_bf16x8(*reinterpret_cast<const uint4*>(Xg + 32 * kv + 8 * lg));
      }
      if (tid < L) {
        const int t = tid;
        const bool in = t < Lc;
        const size_t kr = krow0 + static_cast<size_t>(min(t, tl)) * d.Hk;
        sm.rk[t] = in ? p.s.rk[kr] : 0.f;
        sm.rq[t] = in ? p.s.rq[kr] : 0.f;
        const bool valid = in && (p.mask == nullptr || p.mask[static_cast<size_t>(b) * d.T + t0 + t] != 0);
        sm.valid[t] = valid ? 1.f : 0.f;
        sm.beta[t] = p.cb.vsc[cidx * VSC_ROWS * L + VSC_BETA * L + t];
      }
    }
    // ---- into LDS (k, q and lg channel-major)
#pragma unroll
    for (int e = 0; e < NPM; ++e) {
      const int u = tid + e * NT, m = u / (L * L / 8), r = u % (L * L / 8), t = r >> 3, s8 = 8 * (r & 7);
      *reinterpret_cast<uint4*>(&(m ? sm.dA : sm.dP)[t * TS + s8]) = pmv[e];
    }
#pragma unroll
    for (int e = 0; e < NLG; ++e) {
      const int u = tid + e * NT, t = u / (CH / 4), i4 = 4 * (u % (CH / 4));
      sm.gT[(i4 + 0) * GT + t] = lgv[e].x;
      sm.gT[(i4 + 1) * GT + t] = lgv[e].y;
      sm.gT[(i4 + 2) * GT + t] = lgv[e].z;
      sm.gT[(i4 + 3) * GT + t] = lgv[e].w;
    }
#pragma unroll
    for (int e = 0; e < NKQ; ++e) {
      const int u = tid + e * NT, m = u / (L * CH / 8), r = u % (L * CH / 8), t = r / (CH / 8), i8 = 8 * (r % (CH / 8));
      bf16* dst = m ? sm.qT : sm.kT;
      const uint32_t wv[4] = {kqv[e].x, kqv[e].y, kqv[e].z, kqv[e].w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        dst[(i8 + 2 * x) * KT + t] = __builtin_bit_cast(bf16, static_cast<uint16_t>(wv[x] & 0xffffu));
        dst[(i8 + 2 * x + 1) * KT + t] = __builtin_bit_cast(bf16, static_cast<uint16_t>(wv[x] >> 16));
      }
    }
#pragma unroll
    for (int e = 0; e < NH; ++e) {
      const int u = tid + e * NT, ch = u / (DV / 4), v4 = 4 * (u % (DV / 4));
      *reinterpret_cast<float4*>(&sm.hs[ch * HS + v4]) = hv[e];
    }
#pragma unroll
    for (int e = 0; e < NDH; ++e) {
      const int u = min(tid + e * NT, NDHP - 1), ch = u / (DV / 8), v8 = 8 * (u % (DV / 8));
      *reinterpret_cast<uint4*>(&sm.dhs[ch * DS + v8]) = dhv[e];  // a duplicate writes the same bytes
    }
    __syncthreads();
    // ---- Gamma (a running sum per channel: 16 lanes of 4 steps each, a
    // prefix over the lanes); diag(beta) X
    for (int u = tid; u < CH * 16; u += NT) {
      const int ch = u >> 4, seg = u & 15;
      float* g = &sm.gT[ch * GT + 4 * seg];
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = sm.valid[4 * seg + r] * g[r];
      x[1] += x[0];
      x[2] += x[1];
      x[3] += x[2];
      float run = x[3];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const float y = __shfl_up(run, off, 16);
        if (seg >= off) run += y;
      }
      const float before = run - x[3];
#pragma unroll
      for (int r = 0; r < 4; ++r) g[r] = x[r] + before;
    }
    {
      const float bt = sm.beta[16 * w + lr];
#pragma unroll
      for (int kv = 0; kv < NV; ++kv) bXf[kv] = scale8(bXf[kv], bt);
    }
    __syncthreads();

    const int b0 = 16 * w;        // this wave's block
    const int tr0 = b0 + 4 * lg;  // this lane's first step
    float dqv[NTL][4], dknv[NTL][4];

#pragma unroll
    for (int tile = 0; tile < NTL; ++tile) {
      const int cl = 16 * tile + lr;  // channel within the workgroup
      const float* gch = &sm.gT[cl * GT];
      const bf16* kch = &sm.kT[cl * KT];
      const bf16* qch = &sm.qT[cl * KT];
      float gt[4], knt[4], qst[4];
      {
        const float4 g4 = *reinterpret_cast<const float4*>(&gch[tr0]);
        gt[0] = g4.x, gt[1] = g4.y, gt[2] = g4.z, gt[3] = g4.w;
        const uint2 k4 = *reinterpret_cast<const uint2*>(&kch[tr0]);
        const uint2 q4 = *reinterpret_cast<const uint2*>(&qch[tr0]);
        const float4 rk4 = *reinterpret_cast<const float4*>(&sm.rk[tr0]);
        const float4 rq4 = *reinterpret_cast<const float4*>(&sm.rq[tr0]);
        knt[0] = __uint_as_float(k4.x << 16) * rk4.x;
        knt[1] = __uint_as_float(k4.x & 0xffff0000u) * rk4.y;
        knt[2] = __uint_as_float(k4.y << 16) * rk4.z;
        knt[3] = __uint_as_float(k4.y & 0xffff0000u) * rk4.w;
        qst[0] = __uint_as_float(q4.x << 16) * rq4.x;
        qst[1] = __uint_as_float(q4.x & 0xffff0000u) * rq4.y;
        qst[2] = __uint_as_float(q4.y << 16) * rq4.z;
        qst[3] = __uint_as_float(q4.y & 0xffff0000u) * rq4.w;
      }
      const float gL = gch[L - 1];

      // direct terms: dQb = dO H^T, dKb = -Ehat H^T, dKh = diag(beta) X dH'^T
      float dq[4], dkr[4], dkw[4];
      {
        f32x4 aq = f4zero(), ak = f4zero(), ah = f4zero();
        float rh = 0.f;
#pragma unroll
        for (int kv = 0; kv < NV; ++kv) {
          const int v0 = 32 * kv + 8 * lg;
          float hf[8];
          ld8f(&sm.hs[cl * HS + v0], hf);
          const uint4 dhu = *reinterpret_cast<const uint4*>(&sm.dhs[cl * DS + v0]);
          const bf16x8 hb = as_bf16x8(pack8(hf));
          aq = mfma16(dOf[kv], hb, aq);
          ak = mfma16(Ef[kv], hb, ak);
          ah = mfma16(bXf[kv], as_bf16x8(dhu), ah);
          if (w == 0) {
            float df[8];
            unpack8(dhu, df);
#pragma unroll
            for (int x = 0; x < 8; ++x) rh = fmaf(df[x], hf[x], rh);
          }
        }
        float rd = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float eg = __expf(gt[r]), el = __expf(gL - gt[r]);
          dq[r] = eg * aq[r];
          dkr[r] = -eg * ak[r];
          dkw[r] = el * ah[r];
          rd = fmaf(knt[r], dkw[r], rd);  // Kh dKh = kn e^{G_L - G} dKh
        }
        rd += __shfl_xor(rd, 16);
        rd += __shfl_xor(rd, 32);
        if (lg == 0) sm.rdot[w][lr] = rd;
        if (w == 0) {
          rh += __shfl_xor(rh, 16);
          rh += __shfl_xor(rh, 32);
          if (lg == 0) sm.rdh[lr] = rh;
        }
      }

      // rows of block w against the blocks before it (split at r0 = 16 w - 1)
      if (w >= 1) {
        const int r0 = b0 - 1;
        const float Gr = gch[r0];
        f32x4 oq = f4zero(), orr = f4zero();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (32 * kk >= b0) continue;  // uniform
          const int s0 = 32 * kk + 8 * lg;
          float kf[8], gf[8], rkf[8];
          ld8b(&kch[s0], kf);
          ld8f(&gch[s0], gf);
          ld8f(&sm.rk[s0], rkf);
          float y[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) y[x] = s0 + x < b0 ? kf[x] * rkf[x] * __expf(Gr - gf[x]) : 0.f;
          const bf16x8 yb = as_bf16x8(pack8(y));
          oq = mfma16(load_bf16x8(&sm.dP[(b0 + lr) * TS + s0]), yb, oq);
          orr = mfma16(load_bf16x8(&sm.dA[(b0 + lr) * TS + s0]), yb, orr);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sc = __expf(gt[r] - Gr);
          dq[r] = fmaf(sc, oq[r], dq[r]);
          dkr[r] = fmaf(sc, orr[r], dkr[r]);
        }
      }
      // columns of block w against the blocks after it (split at e0 = 16 w + 15)
      if (w <= 2) {
        const int e0 = b0 + 15;
        const float Ge = gch[e0];
        f32x4 ow = f4zero();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (b0 + 16 + 32 * kk >= L) continue;  // uniform
          const int tbase = b0 + 16 + 32 * kk;
          const int tb = tbase + 8 * lg;
          const int tc = tb < L ? tb : L - 8;  // lanes past the end read in range, zeroed below
          float kf[8], qf[8], gf[8], rkf[8], rqf[8];
          ld8b(&kch[tc], kf);
          ld8b(&qch[tc], qf);
          ld8f(&gch[tc], gf);
          ld8f(&sm.rk[tc], rkf);
          ld8f(&sm.rq[tc], rqf);
          float yq[8], yk[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const float ee = tb < L ? __expf(gf[x] - Ge) : 0.f;
            yq[x] = qf[x] * rqf[x] * ee;
            yk[x] = kf[x] * rkf[x] * ee;
          }
          // dP^T, dA^T rows b0 + lr over this group's steps tc .. tc + 7
          const bf16x8 ap = col8(sm.dP, tc, b0, lr), aa = col8(sm.dA, tc, b0, lr);
          const bool use = tb < L;
          ow = mfma16(use ? ap : zero8(), as_bf16x8(pack8(yq)), ow);
          ow = mfma16(use ? aa : zero8(), as_bf16x8(pack8(yk)), ow);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) dkw[r] = fmaf(__expf(Ge - gt[r]), ow[r], dkw[r]);
      }
      // the diagonal block.  Where every channel of the tile decays by less
      // than e^60 inside the block, on MFMA with the split at c = 16 w - 1,
      // the step before the block (G_{-1} = 0): e^{G_t - G_s} =
      // e^{G_t - G_c} e^{G_c - G_s}, the second factor at most e^60, both in
      // the normal range of fp32 and bf16.  Else in fp32: rows tr0 + r (over
      // s <= t) and columns tr0 + r (over t >= s), decays built step by step.
      const float Gc = b0 == 0 ? 0.f : gch[b0 - 1];
      if (__all(Gc - gch[b0 + 15] <= kDiagSpan)) {
        const int s0 = b0 + 8 * lg;
        const bool in = lg < 2;  // k-steps 16 .. 31 of the MFMA are padding
        const int sc = in ? s0 : b0;
        float kf[8], qf[8], gf[8], rkf[8], rqf[8];
        ld8b(&kch[sc], kf);
        ld8b(&qch[sc], qf);
        ld8f(&gch[sc], gf);
        ld8f(&sm.rk[sc], rkf);
        ld8f(&sm.rq[sc], rqf);
        float y[8], yq[8], yk[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float kn = kf[x] * rkf[x];
          const float up = in ? __expf(Gc - gf[x]) : 0.f, dn = in ? __expf(gf[x] - Gc) : 0.f;
          y[x] = kn * up;
          yk[x] = kn * dn;
          yq[x] = qf[x] * rqf[x] * dn;
        }
        const bf16x8 yb = as_bf16x8(pack8(y));
        const bf16x8 ap = in ? load_bf16x8(&sm.dP[(b0 + lr) * TS + sc]) : zero8();
        const bf16x8 aa = in ? load_bf16x8(&sm.dA[(b0 + lr) * TS + sc]) : zero8();
        const bf16x8 apt = in ? col8(sm.dP, sc, b0, lr) : zero8();  // dP^T rows b0 + lr
        const bf16x8 aat = in ? col8(sm.dA, sc, b0, lr) : zero8();
        const f32x4 oq = mfma16(ap, yb, f4zero());
        const f32x4 orr = mfma16(aa, yb, f4zero());
        f32x4 ow = mfma16(apt, as_bf16x8(pack8(yq)), f4zero());
        ow = mfma16(aat, as_bf16x8(pack8(yk)), ow);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float dn = __expf(gt[r] - Gc), up = __expf(Gc - gt[r]);
          dq[r] = fmaf(dn, oq[r], dq[r]);
          dkr[r] = fmaf(dn, orr[r], dkr[r]);
          dkw[r] = fmaf(up, ow[r], dkw[r]);
        }
      } else {
        float gb[16], kb[16], qb[16], gg[16];
        ld8f(&gch[b0], *reinterpret_cast<float(*)[8]>(&gb[0]));
        ld8f(&gch[b0 + 8], *reinterpret_cast<float(*)[8]>(&gb[8]));
        ld8b(&kch[b0], *reinterpret_cast<float(*)[8]>(&kb[0]));
        ld8b(&kch[b0 + 8], *reinterpret_cast<float(*)[8]>(&kb[8]));
        ld8b(&qch[b0], *reinterpret_cast<float(*)[8]>(&qb[0]));
        ld8b(&qch[b0 + 8], *reinterpret_cast<float(*)[8]>(&qb[8]));
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          kb[x] *= sm.rk[b0 + x];
          qb[x] *= sm.rq[b0 + x];
        }
        gg[0] = 1.f;
#pragma unroll
        for (int x = 1; x < 16; ++x) gg[x] = __expf(gb[x] - gb[x - 1]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tloc = 4 * lg + r;  // per lane
          float pr[16], ar[16];
          ld8b(&sm.dP[(b0 + tloc) * TS + b0], *reinterpret_cast<float(*)[8]>(&pr[0]));
          ld8b(&sm.dP[(b0 + tloc) * TS + b0 + 8], *reinterpret_cast<float(*)[8]>(&pr[8]));
          ld8b(&sm.dA[(b0 + tloc) * TS + b0], *reinterpret_cast<float(*)[8]>(&ar[0]));
          ld8b(&sm.dA[(b0 + tloc) * TS + b0 + 8], *reinterpret_cast<float(*)[8]>(&ar[8]));
          float e = 0.f, sq = 0.f, sr = 0.f;
#pragma unroll
          for (int s = 15; s >= 0; --s) {
            const float gn = s < 15 ? gg[s + 1] : 0.f;  // (s is a constant here: no read past gg)
            e = s < tloc ? e * gn : (s == tloc ? 1.f : 0.f);  // e^{G_t - G_s}, 0 above
            const float ke = kb[s] * e;
            sq = fmaf(pr[s], ke, sq);
            sr = fmaf(ar[s], ke, sr);
          }
          dq[r] += sq;
          dkr[r] += sr;
          float pc[16], ac[16];  // column b0 + tloc of dP, dA
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            pc[t] = to_f32(sm.dP[(b0 + t) * TS + b0 + tloc]);
            ac[t] = to_f32(sm.dA[(b0 + t) * TS + b0 + tloc]);
          }
          e = 0.f;
          float sw = 0.f;
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            e = t > tloc ? e * gg[t] : (t == tloc ? 1.f : 0.f);  // e^{G_t - G_s}, 0 before
            sw = fmaf(fmaf(pc[t], qb[t], ac[t] * kb[t]), e, sw);
          }
          dkw[r] += sw;
        }
      }

      // dG, the suffix sums inside the block, and the block total
      float suf[4];
      {
        float dg[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dg[r] = fmaf(qst[r], dq[r], knt[r] * (dkr[r] - dkw[r]));
          dqv[tile][r] = dq[r];
          dknv[tile][r] = dkr[r] + dkw[r];
        }
        suf[3] = dg[3];
        suf[2] = dg[2] + suf[3];
        suf[1] = dg[1] + suf[2];
        suf[0] = dg[0] + suf[1];
        // lanes lg + 1 .. 3 of the same channel hold the later steps of the block
        const float tot = suf[0];
        const float n1 = __shfl_down(tot, 16), n2 = __shfl_down(tot, 32), n3 = __shfl_down(tot, 48);
        const float later = (lg < 3 ? n1 : 0.f) + (lg < 2 ? n2 : 0.f) + (lg < 1 ? n3 : 0.f);
#pragma unroll
        for (int r = 0; r < 4; ++r) suf[r] += later;
        if (lg == 0) sm.btot[w][lr] = tot + later;
      }
      __syncthreads();
      {  // dlg: rows tr0 .. + 3, channel ch0 + cl (0 on masked steps)
        float add = __expf(gL) * sm.rdh[lr] + sm.rdot[0][lr] + sm.rdot[1][lr] + sm.rdot[2][lr] + sm.rdot[3][lr];
#pragma unroll
        for (int ww = 0; ww < 4; ++ww)
          if (ww > w) add += sm.btot[ww][lr];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = tr0 + r;
          if (t < Lc)
            p.dlg[(vrow0 + static_cast<size_t>(t) * d.Hv) * DK + ch0 + cl] = sm.valid[t] != 0.f ? suf[r] + add : 0.f;
        }
      }
      __syncthreads();  // btot, rdot, rdh are rewritten by the next tile
    }

    // ---- this value head's parts of the row gradients of s qn and kn: rows
    // tr0 .. + 3, channels ch0 + 16 tile + lr
#pragma unroll
    for (int tile = 0; tile < NTL; ++tile)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tr0 + r;
        if (t < Lc) {
          bf16* dst = p.qk + (vrow0 + static_cast<size_t>(t) * d.Hv) * 2 * DK + ch0 + 16 * tile + lr;
          dst[0] = bf16_of(dqv[tile][r]);
          dst[DK] = bf16_of(dknv[tile][r]);
        }
      }
  }
};

// vg_norm_bwd: the L2-normalisation backward of q and k (torch-to-nnef GDN
// page, "Op contract": q, k normalised with eps 1e-6 inside the root).  g, the
// gradient w.r.t. the normalised row as the chunk form uses it (s qn for q, kn
// for k), is the sum of the parts of the key head's G value heads (in head
// order); with r the norm factor (for q also 1 / sqrt(Dk), so that s qn = r q),
// dx = r (g - x^ (x^ . g)), x^ = x (|x|^2 + eps)^-1/2.  One wave per (b, t, key
// head), DK / 64 channels per lane.
template <int DK>
__global__ void __launch_bounds__(64) vg_norm_bwd_kernel(VgChunkGradArgs p) {
  constexpr int RM = DK / 64;
  const Dims& d = p.d;
  const size_t row = blockIdx.x;  // (b t) Hk + j
  const int lane = threadIdx.x;
  const float rq = p.s.rq[row], rk = p.s.rk[row];
  const float qs = rq * sqrtf(static_cast<float>(DK));  // q^ = q qs
  const bf16* qg = static_cast<const bf16*>(p.q) + row * DK;
  const bf16* kg = static_cast<const bf16*>(p.k) + row * DK;
  const int G = d.G();
  const bf16* gq = p.qk + row * G * 2 * DK;  // rows (b t) Hv + j G + hh
  float qh[RM], kn[RM], dq[RM], dk[RM], pq = 0.f, pk = 0.f;
#pragma unroll
  for (int m = 0; m < RM; ++m) dq[m] = dk[m] = 0.f;
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int m = 0; m < RM; ++m) {
      dq[m] += to_f32(gq[hh * 2 * DK + lane + 64 * m]);
      dk[m] += to_f32(gq[hh * 2 * DK + DK + lane + 64 * m]);
    }
#pragma unroll
  for (int m = 0; m < RM; ++m) {
    const int i = lane + 64 * m;
    qh[m] = to_f32(qg[i]) * qs;
    kn[m] = to_f32(kg[i]) * rk;
    pq = fmaf(qh[m], dq[m], pq);
    pk = fmaf(kn[m], dk[m], pk);
  }
  pq = lanes_sum(pq);
  pk = lanes_sum(pk);
#pragma unroll
  for (int m = 0; m < RM; ++m) {
    const int i = lane + 64 * m;
    static_cast<bf16*>(p.dq)[row * DK + i] = bf16_of(rq * (dq[m] - qh[m] * pq));
    static_cast<bf16*>(p.dk)[row * DK + i] = bf16_of(rk * (dk[m] - kn[m] * pk));
  }
}

template <int DK, int DV, bool XSV>
__global__ void __launch_bounds__(NT) vg_chunk_x_kernel(VgChunkGradArgs p) {
  __shared__ typename VgX<DK, DV, XSV>::Smem sm;
  VgX<DK, DV, XSV>::run(p, sm);
}

template <int DK, int DV, bool HBF>
__global__ void __launch_bounds__(NT) vg_chunk_grad_kernel(VgChunkGradArgs p) {
  __shared__ typename VgG<DK, DV, HBF>::Smem sm;
  VgG<DK, DV, HBF>::run(p, sm);
}

template <int DK, bool X>
hipError_t launch_grad_dk(const VgChunkGradArgs& a, hipStream_t st) {
  const long pairs = static_cast<long>(a.d.nchunk()) * a.d.B * a.d.Hv;
  const dim3 grid = X ? dim3(a.d.nchunk(), a.d.B * a.d.Hv)
                      : dim3(static_cast<unsigned>((pairs + 7) / 8 * 8 * (DK / kVgGradChannels)));
  switch (a.d.Dv) {
#define GDN_VG_DV(DV)                                          \
  case DV:                                                     \
    if (X && a.xsv)                                            \
      vg_chunk_x_kernel<DK, DV, true><<<grid, NT, 0, st>>>(a); \
    else if (X)                                                \
      vg_chunk_x_kernel<DK, DV, false><<<grid, NT, 0, st>>>(a); \
    else if (a.cb.Hb != nullptr)                               \
      vg_chunk_grad_kernel<DK, DV, true><<<grid, NT, 0, st>>>(a); \
    else                                                       \
      vg_chunk_grad_kernel<DK, DV, false><<<grid, NT, 0, st>>>(a); \
    break;
    GDN_VG_DV(32)
    GDN_VG_DV(64)
    GDN_VG_DV(96)
    GDN_VG_DV(128)
#undef GDN_VG_DV
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vg_chunk_prep(const VgChunkPrepArgs& a, hipStream_t st) {
  if (a.d.T == 0) return hipSuccess;
  const dim3 grid(a.d.nchunk(), a.d.B * a.d.Hv);
  switch (a.d.Dk) {
    case 64: vg_chunk_prep_kernel<64><<<grid, NT, 0, st>>>(a); break;
    case 128: vg_chunk_prep_kernel<128><<<grid, NT, 0, st>>>(a); break;
    case 192: vg_chunk_prep_kernel<192><<<grid, NT, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn

namespace gdn {

hipError_t launch_vg_chunk_x(const VgChunkGradArgs& a, hipStream_t st) {
  if (a.d.T == 0) return hipSuccess;
  switch (a.d.Dk) {
    case 64: return launch_grad_dk<64, true>(a, st);
    case 128: return launch_grad_dk<128, true>(a, st);
    case 192: return launch_grad_dk<192, true>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_vg_chunk_grad(const VgChunkGradArgs& a, hipStream_t st) {
  if (a.d.T == 0) return hipSuccess;
  switch (a.d.Dk) {
    case 64: return launch_grad_dk<64, false>(a, st);
    case 128: return launch_grad_dk<128, false>(a, st);
    case 192: return launch_grad_dk<192, false>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_vg_norm_bwd(const VgChunkGradArgs& a, hipStream_t st) {
  const unsigned n = static_cast<unsigned>(static_cast<size_t>(a.d.B) * a.d.T * a.d.Hk);
  if (n == 0) return hipSuccess;
  switch (a.d.Dk) {
    case 64: vg_norm_bwd_kernel<64><<<n, 64, 0, st>>>(a); break;
    case 128: vg_norm_bwd_kernel<128><<<n, 64, 0, st>>>(a); break;
    case 192: vg_norm_bwd_kernel<192><<<n, 64, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
