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
// a bf16 MFMA product of rows scaled by each factor; inside a diagonal
// sub-block every pair is taken in fp32 on the vector units, with the same
// split at the end of the earlier 4-step group for pairs in different groups
// and the exact exponential within a group.
//
// Kernels:
//   vg_chunk_prep  one workgroup per (chunk, batch, value head): Gamma by a
//                  per-channel scan, the norms, A and P (MFMA off the
//                  diagonal sub-blocks, fp32 on them), Tx by the blocked
//                  inverse of gdn_tri.h, and the pre-scaled rows the state
//                  passes read.
//   vg_chunk_grad  one workgroup per (chunk, batch, value head): the chunk's
//                  gradients from dH' (= dL/d the state at the chunk end),
//                  Ehat (= dv) and eps (= dL/d delta) of the reverse state
//                  pass, with X recomputed from the fp32 checkpoint:
//     dQb = dO H^T,  dKb = -Ehat H^T,  dKh = diag(beta) X dH'^T,
//     dP = lower(dO X^T) diag(beta),  dA = -strictlower(Ehat X^T) diag(beta),
//     dbeta_t = eps_t . X_t,
//   then, per channel i, the three roles of the rows (s the 1/sqrt(Dk) scale):
//     dq_t  = e^{G_t} dQb_t + sum_{u<=t} dP[t,u] kn_u e^{G_t-G_u}            (w.r.t. s qn)
//     dkR_t = e^{G_t} dKb_t + sum_{u<t}  dA[t,u] kn_u e^{G_t-G_u}            (k as a reader)
//     dkW_u = e^{G_L-G_u} dKh_u + sum_{t>=u} (dP[t,u] s qn_t + dA[t,u] kn_t) e^{G_t-G_u}  (writer)
//     dG_t  = s qn_t dq_t + kn_t (dkR_t - dkW_t) + [t = L-1] (e^{G_L} <dH', H> + sum_u Kh_u dKh_u)
//     dlg_t = sum_{t' >= t} dG_t' (0 on masked steps),   dkn = dkR + dkW;
//   every e^{G} factor enters as e^{G_t - G_u} with u <= t (so lg enters
//   through G_t - G_u only).  The expansions take the sub-blocks of the
//   forward: MFMA with the split at the previous block's end off the
//   diagonal, fp32 with decays built step by step inside it.
#include "gdn_dev.h"
#include "gdn_internal.h"
#include "gdn_tri.h"

namespace gdn {
namespace {

constexpr int L = kChunk;
constexpr int NT = 256;

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
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]), pack2_bf16(f[4], f[5]), pack2_bf16(f[6], f[7]));
}

template <int DK>
struct VgPrep {
  static constexpr int RS = DK + 8;      // bf16 row stride of the staged k / q rows
  static constexpr int GS = DK + 4;      // fp32 row stride of Gamma
  static constexpr int SP = tri::SP;
  static constexpr int NSL = DK / 32;    // channel slices of the diagonal sub-blocks
  static constexpr int NTASK = 40 * NSL; // (sub-block, 4x4 tile, slice)
  static constexpr int NLD = L * DK / 8 / NT;  // 16-byte pieces of one of k, q per thread
  static constexpr int NLG = L * DK / 4 / NT;  // 16-byte pieces of lg per thread
  static_assert(NTASK <= NT, "one diagonal task per thread");
  static_assert(L * DK / 8 % NT == 0 && L * DK / 4 % NT == 0, "whole pieces per thread");
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
    alignas(16) float dp[NTASK * 32];  // diagonal sub-block partial sums: 16 of A, 16 of P per task
    float rk[L], rq[L], beta[L], valid[L];
  };

  __device__ static void run(const VgChunkPrepArgs& p, Smem& sm) {
    const Dims& d = p.d;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int G = d.G(), NC = d.nchunk();
    const int b = bh / d.Hv, h = bh % d.Hv, j = h / G;
    const int t0 = c * L, Lc = min(L, d.T - t0), tl = Lc - 1;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    const bool bwd = p.bwd != 0;
    const size_t qk0 = (static_cast<size_t>(b) * d.T + t0) * d.Hk + j;
    const uint32_t qk_row = d.Hk * DK;
    const bf16* kc = static_cast<const bf16*>(p.k) + qk0 * DK;
    const bf16* qc = static_cast<const bf16*>(p.q) + qk0 * DK;
    const uint32_t lg_row = d.Hv * DK;
    const float* lgc = p.lg + ((static_cast<size_t>(b) * d.T + t0) * d.Hv + h) * DK;
    const size_t cidx = static_cast<size_t>(bh) * NC + c;

    // ---- k / q / lg rows of the chunk (clamped into the sequence), all
    // loads issued before any is used; beta and the step's validity (wave 0)
    uint4 kv[NLD], qv[NLD];
    float4 gv[NLG];
#pragma unroll
    for (int e = 0; e < NLD; ++e) {
      const int u = tid + e * NT, t = u / (DK / 8), i8 = 8 * (u % (DK / 8));
      const uint32_t o = static_cast<uint32_t>(min(t, tl)) * qk_row + i8;
      kv[e] = *reinterpret_cast<const uint4*>(kc + o);
      qv[e] = *reinterpret_cast<const uint4*>(qc + o);
    }
#pragma unroll
    for (int e = 0; e < NLG; ++e) {
      const int u = tid + e * NT, t = u / (DK / 4), i4 = 4 * (u % (DK / 4));
      gv[e] = *reinterpret_cast<const float4*>(lgc + static_cast<uint32_t>(min(t, tl)) * lg_row + i4);
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
#pragma unroll
    for (int e = 0; e < NLD; ++e) {
      const int u = tid + e * NT, t = u / (DK / 8), i8 = 8 * (u % (DK / 8));
      *reinterpret_cast<uint4*>(&sm.u.r.k[t * RS + i8]) = kv[e];
      *reinterpret_cast<uint4*>(&sm.u.r.q[t * RS + i8]) = qv[e];
    }
#pragma unroll
    for (int e = 0; e < NLG; ++e) {
      const int u = tid + e * NT, t = u / (DK / 4), i4 = 4 * (u % (DK / 4));
      *reinterpret_cast<float4*>(&sm.u.r.gam[t * GS + i4]) = gv[e];
    }
    __syncthreads();

    // ---- norm factors (four lanes per row) and Gamma (one thread per
    // channel, a running sum over the steps; a masked step or a row past the
    // end adds 0)
    {
      const int t = tid >> 2, part = tid & 3;
      float kk = 0.f, qq = 0.f;
#pragma unroll
      for (int e = 0; e < DK / 32; ++e) {
        float kf[8], qf[8];
        unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.k[t * RS + (DK / 4) * part + 8 * e]), kf);
        unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.q[t * RS + (DK / 4) * part + 8 * e]), qf);
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
    if (tid < DK) {
      float g = 0.f;
#pragma unroll 8
      for (int t = 0; t < L; ++t) {
        g += sm.valid[t] * sm.u.r.gam[t * GS + tid];
        sm.u.r.gam[t * GS + tid] = g;
      }
    }
    __syncthreads();

    // ---- A and P off the diagonal sub-blocks: wave I (1..3) takes row block
    // I against the column blocks J < I, reference r = 16 I - 1
    f32x4 accA[3], accP[3];
#pragma unroll
    for (int J = 0; J < 3; ++J) accA[J] = accP[J] = f4zero();
    if (w >= 1) {
      const int I = w, r = 16 * I - 1, ta = 16 * I + lr;
      const float rkt = sm.rk[ta], rqt = sm.rq[ta];
#pragma unroll
      for (int kt = 0; kt < DK / 32; ++kt) {
        const int i0 = 32 * kt + 8 * lg;
        float kf[8], qf[8], ex[8];
        unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.k[ta * RS + i0]), kf);
        unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.q[ta * RS + i0]), qf);
        float gr[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          gr[x] = sm.u.r.gam[r * GS + i0 + x];
          ex[x] = __expf(sm.u.r.gam[ta * GS + i0 + x] - gr[x]);
          kf[x] *= rkt * ex[x];
          qf[x] *= rqt * ex[x];
        }
        const bf16x8 ak = as_bf16x8(pack8(kf)), aq = as_bf16x8(pack8(qf));
#pragma unroll
        for (int J = 0; J < 3; ++J) {
          if (J >= I) continue;
          const int su = 16 * J + lr;
          const float rku = sm.rk[su];
          float uf[8];
          unpack8(*reinterpret_cast<const uint4*>(&sm.u.r.k[su * RS + i0]), uf);
#pragma unroll
          for (int x = 0; x < 8; ++x) uf[x] *= rku * __expf(gr[x] - sm.u.r.gam[su * GS + i0 + x]);
          const bf16x8 bk = as_bf16x8(pack8(uf));
          accA[J] = mfma16(ak, bk, accA[J]);
          accP[J] = mfma16(aq, bk, accP[J]);
        }
      }
    }

    // ---- the diagonal sub-blocks in fp32: task (block I, 4x4 tile, 32
    // channels); raw-row products, scaled by the norms when summed
    if (tid < NTASK) {
      const int sl = tid % NSL, rest = tid / NSL, I = rest / 10, ti = rest % 10;
      const int tt = tile_t(ti), uu = tile_u(ti);
      const int tb = 16 * I + 4 * tt, ub = 16 * I + 4 * uu;
      float pa[16], pp[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) pa[x] = pp[x] = 0.f;
      const bool split = tt > uu;  // different 4-step groups: split at the end of ub's group
      for (int i = 32 * sl; i < 32 * sl + 32; ++i) {
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
      float* dst = &sm.dp[(rest * NSL + sl) * 32];
#pragma unroll
      for (int x = 0; x < 16; x += 4) {
        *reinterpret_cast<float4*>(&dst[x]) = make_float4(pa[x], pa[x + 1], pa[x + 2], pa[x + 3]);
        *reinterpret_cast<float4*>(&dst[16 + x]) = make_float4(pp[x], pp[x + 1], pp[x + 2], pp[x + 3]);
      }
    }

    // ---- the pre-scaled rows: forward Kb, Kh, Qb ([t][i]); backward Kh and
    // Kb^T, Qb^T ([i][t]); and the chunk scalars (beta, e^{G_L})
    {
      const size_t rowbase = cidx * L * DK;
      for (int u = tid; u < L * DK / 8; u += NT) {
        const int t = u / (DK / 8), i0 = 8 * (u % (DK / 8));
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
        const size_t o = rowbase + static_cast<size_t>(t) * DK + i0;
        *reinterpret_cast<uint4*>(p.cb.Kh + o) = pack8(kh);
        if (!bwd) {
          *reinterpret_cast<uint4*>(p.cb.Kb + o) = pack8(kf);
          *reinterpret_cast<uint4*>(p.cb.Qb + o) = pack8(qf);
        }
      }
      if (bwd) {
        for (int u = tid; u < DK * L / 8; u += NT) {
          const int i = u % DK, t8 = 8 * (u / DK);
          float kf[8], qf[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int t = t8 + x;
            const float e = __expf(sm.u.r.gam[t * GS + i]);
            kf[x] = to_f32(sm.u.r.k[t * RS + i]) * sm.rk[t] * e;
            qf[x] = to_f32(sm.u.r.q[t * RS + i]) * sm.rq[t] * e;
          }
          const size_t o = rowbase + static_cast<size_t>(i) * L + t8;
          *reinterpret_cast<uint4*>(p.cb.KbT + o) = pack8(kf);
          *reinterpret_cast<uint4*>(p.cb.QbT + o) = pack8(qf);
        }
      }
      float* vsc = p.cb.vsc + cidx * VSC_ROWS * L;
      if (tid < L) vsc[VSC_BETA * L + tid] = sm.beta[tid];
      for (int i = tid; i < (VSC_ROWS - 1) * L; i += NT)
        vsc[VSC_EGL * L + i] = i < DK ? __expf(sm.u.r.gam[(L - 1) * GS + i]) : 0.f;
    }
    __syncthreads();  // the staged rows and Gamma are dead from here on

    // ---- N = A diag(beta) and Mq = P diag(beta) (forward), or A^T, P^T
    // (backward); every element written once: the lower off-diagonal
    // sub-blocks by the MFMA waves, the rest here
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
    for (int e = tid; e < L * L; e += NT) {
      const int t = e >> 6, s = e & 63, bi = t >> 4, bj = s >> 4;
      if (bi > bj) continue;
      float av = 0.f, pv = 0.f;
      const int tt = (t >> 2) & 3, uu = (s >> 2) & 3;
      if (bi == bj && uu <= tt) {
        const int rest = bi * 10 + tt * (tt + 1) / 2 + uu, x = 4 * (t & 3) + (s & 3);
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
          av += sm.dp[(rest * NSL + sl) * 32 + x];
          pv += sm.dp[(rest * NSL + sl) * 32 + 16 + x];
        }
        av = s < t ? av * sm.rk[t] * sm.rk[s] : 0.f;
        pv = s <= t ? pv * sm.rq[t] * sm.rk[s] : 0.f;
      }
      const float bs = sm.beta[s];
      nf[t * SP + s] = av * bs;
      if (bwd) {
        st[s * SP + t] = av;
        st2[s * SP + t] = pv;
      } else {
        st[t * SP + s] = pv * bs;
      }
    }
    __syncthreads();

    // ---- Tx = (I + N)^-1, and the stores
    tri::invert_diagonal_block(nf, w, l);
    const size_t mat = cidx * L * L;
    if (bwd) {
      tri::store_mat(st, p.cb.AtT + mat, tid, NT);
      tri::store_mat(st2, p.cb.PqT + mat, tid, NT);
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

template <int DK, int DV>
struct VgGrad {
  static constexpr int NV = DV / 32;    // 32-column k-steps over Dv
  static constexpr int NVT = DV / 16;   // 16-column tiles of Dv
  static constexpr int NCT = DK / 16;   // 16-channel tiles
  static constexpr int GS = DK + 4;     // fp32 row stride of Gamma
  static constexpr int RS = DK + 8;     // bf16 row stride of k / q rows and H^T
  static constexpr int TS = L + 8;      // bf16 row stride of the L-wide tiles
  static constexpr int XS = DV + 8;     // bf16 row stride of X
  static constexpr int AS = 17;         // fp32 row stride of the per-tile sums
  static constexpr int NLD = L * DK / 8 / NT;
  static constexpr int NLG = L * DK / 4 / NT;
  static constexpr int HVI = DV * RS > L * XS ? DV * RS : L * XS;
  struct PhaseA {
    bf16 hvi[HVI];     // H^T [v][i] (bf16); X later takes its place
    bf16 rT[DV * TS];  // R^T [v][s]
    bf16 txs[L * TS];  // Tx [t][s]
  };
  struct PhaseC {
    bf16 xs[L * XS];       // X [t][v]
    bf16 qrow[L * RS];     // raw q rows
    bf16 dP[L * TS];       // dP [t][s]
    bf16 dA[L * TS];       // dA [t][s]
    float acc[3 * L * AS]; // per tile: dq, dkR (then dkn), dkW (then dlg), [t][16 channels]
  };
  union U {
    PhaseA a;
    PhaseC c;
  };
  struct Smem {
    alignas(16) float gam[L * GS];
    alignas(16) bf16 krow[L * RS];
    alignas(16) U u;
    float rk[L], rq[L], beta[L], valid[L];
    float rdot[4][16], rdh[16];
  };

  __device__ static void run(const VgChunkGradArgs& p, Smem& sm) {
    const Dims& d = p.d;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int G = d.G(), NC = d.nchunk();
    const int b = bh / d.Hv, h = bh % d.Hv, j = h / G;
    const int t0 = c * L, Lc = min(L, d.T - t0), tl = Lc - 1;
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t qk0 = (static_cast<size_t>(b) * d.T + t0) * d.Hk + j;
    const uint32_t qk_row = d.Hk * DK;
    const bf16* kc = static_cast<const bf16*>(p.k) + qk0 * DK;
    const bf16* qc = static_cast<const bf16*>(p.q) + qk0 * DK;
    const float* lgc = p.lg + ((static_cast<size_t>(b) * d.T + t0) * d.Hv + h) * DK;
    const uint32_t lg_row = d.Hv * DK;
    const size_t vrow0 = (static_cast<size_t>(b) * d.T + t0) * d.Hv + h;  // row of step t0 in [B,T,Hv]
    const size_t cidx = static_cast<size_t>(bh) * NC + c;
    const float* H = c == 0 ? (p.state0 ? p.state0 + static_cast<size_t>(bh) * DK * DV : nullptr)
                            : p.ckpt + (static_cast<size_t>(c - 1) * d.B * d.Hv + bh) * DK * DV;
    const bf16* dHp = p.dHend + (static_cast<size_t>(c) * d.B * d.Hv + bh) * DK * DV;
    bf16* hvi = sm.u.a.hvi;
    bf16* rT = sm.u.a.rT;
    bf16* txs = sm.u.a.txs;

    // ---- A0: k and lg rows, beta, H^T (bf16), Tx
    {
      uint4 kv[NLD];
      float4 gv[NLG];
#pragma unroll
      for (int e = 0; e < NLD; ++e) {
        const int u = tid + e * NT, t = u / (DK / 8), i8 = 8 * (u % (DK / 8));
        kv[e] = *reinterpret_cast<const uint4*>(kc + static_cast<uint32_t>(min(t, tl)) * qk_row + i8);
      }
#pragma unroll
      for (int e = 0; e < NLG; ++e) {
        const int u = tid + e * NT, t = u / (DK / 4), i4 = 4 * (u % (DK / 4));
        gv[e] = *reinterpret_cast<const float4*>(lgc + static_cast<uint32_t>(min(t, tl)) * lg_row + i4);
      }
      if (w == 0) {
        const int t = min(l, tl);
        const float bv = to_f32(static_cast<const bf16*>(p.b)[vrow0 + static_cast<size_t>(t) * d.Hv]);
        const rsrc_t rm = make_rsrc(p.mask ? static_cast<const void*>(p.mask) : p.b,
                                    p.mask ? static_cast<size_t>(d.B) * d.T : 0);
        const bool valid = l < Lc && (p.mask == nullptr ||
                                      __builtin_amdgcn_raw_buffer_load_b8(rm, static_cast<uint32_t>(b * d.T + t0 + t), 0, 0) != 0);
        sm.beta[l] = valid ? sigmoid_f(bv) : 0.f;
        sm.valid[l] = valid ? 1.f : 0.f;
      }
#pragma unroll
      for (int e = 0; e < NLD; ++e) {
        const int u = tid + e * NT, t = u / (DK / 8), i8 = 8 * (u % (DK / 8));
        *reinterpret_cast<uint4*>(&sm.krow[t * RS + i8]) = kv[e];
      }
#pragma unroll
      for (int e = 0; e < NLG; ++e) {
        const int u = tid + e * NT, t = u / (DK / 4), i4 = 4 * (u % (DK / 4));
        *reinterpret_cast<float4*>(&sm.gam[t * GS + i4]) = gv[e];
      }
      for (int u = tid; u < DK * DV / 4; u += NT) {
        const int i = u / (DV / 4), v4 = 4 * (u % (DV / 4));
        const float4 x = H ? *reinterpret_cast<const float4*>(H + static_cast<size_t>(i) * DV + v4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
        hvi[(v4 + 0) * RS + i] = bf16_of(x.x);
        hvi[(v4 + 1) * RS + i] = bf16_of(x.y);
        hvi[(v4 + 2) * RS + i] = bf16_of(x.z);
        hvi[(v4 + 3) * RS + i] = bf16_of(x.w);
      }
      const bf16* txg = p.cb.Tx + cidx * L * L;
      for (int u = tid; u < L * L / 8; u += NT) {
        const int t = u >> 3, s8 = 8 * (u & 7);
        *reinterpret_cast<uint4*>(&txs[t * TS + s8]) = *reinterpret_cast<const uint4*>(txg + t * L + s8);
      }
    }
    __syncthreads();

    // ---- A1: k norms; Gamma
    {
      const int t = tid >> 2, part = tid & 3;
      float kk = 0.f;
#pragma unroll
      for (int e = 0; e < DK / 32; ++e) {
        float kf[8];
        unpack8(*reinterpret_cast<const uint4*>(&sm.krow[t * RS + (DK / 4) * part + 8 * e]), kf);
#pragma unroll
        for (int x = 0; x < 8; ++x) kk = fmaf(kf[x], kf[x], kk);
      }
      kk = quad_sum(kk);
      if (part == 0) sm.rk[t] = t < Lc ? 1.f / sqrtf(kk + kNormEps) : 0.f;
    }
    if (tid < DK) {
      float g = 0.f;
#pragma unroll 8
      for (int t = 0; t < L; ++t) {
        g += sm.valid[t] * sm.gam[t * GS + tid];
        sm.gam[t * GS + tid] = g;
      }
    }
    __syncthreads();

    // ---- A2: R^T = V^T - H^T Kb^T (wave w: steps 16 w .. + 15)
    {
      const int tb = 16 * w + lr;
      const float rkt = sm.rk[tb];
      f32x4 acc[NVT];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) acc[vt] = f4zero();
#pragma unroll
      for (int kt = 0; kt < DK / 32; ++kt) {
        const int i0 = 32 * kt + 8 * lg;
        float kf[8];
        unpack8(*reinterpret_cast<const uint4*>(&sm.krow[tb * RS + i0]), kf);
#pragma unroll
        for (int x = 0; x < 8; ++x) kf[x] *= rkt * __expf(sm.gam[tb * GS + i0 + x]);
        const bf16x8 kb = as_bf16x8(pack8(kf));
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
          acc[vt] = mfma16(load_bf16x8(&hvi[(16 * vt + lr) * RS + i0]), kb, acc[vt]);
      }
      const bf16* vg = static_cast<const bf16*>(p.v) + (vrow0 + static_cast<size_t>(min(tb, tl)) * d.Hv) * DV;
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const uint2 v4 = *reinterpret_cast<const uint2*>(vg + 16 * vt + 4 * lg);
        const float vv[4] = {__uint_as_float(v4.x << 16), __uint_as_float(v4.x & 0xffff0000u),
                             __uint_as_float(v4.y << 16), __uint_as_float(v4.y & 0xffff0000u)};
#pragma unroll
        for (int r = 0; r < 4; ++r) rT[(16 * vt + 4 * lg + r) * TS + tb] = bf16_of(vv[r] - acc[vt][r]);
      }
    }
    __syncthreads();

    // ---- A3: X = Tx R (wave w: steps 16 w .. + 15), into X's place (H^T is dead)
    bf16* xs = sm.u.c.xs;
    {
      f32x4 xa[NVT];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) xa[vt] = f4zero();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 a = load_bf16x8(&txs[(16 * w + lr) * TS + 32 * kk + 8 * lg]);
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
          xa[vt] = mfma16(a, load_bf16x8(&rT[(16 * vt + lr) * TS + 32 * kk + 8 * lg]), xa[vt]);
      }
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r) xs[(16 * w + 4 * lg + r) * XS + 16 * vt + lr] = bf16_of(xa[vt][r]);
    }
    __syncthreads();

    // ---- B: q rows; dO, Ehat, X and diag(beta) X rows of this wave as
    // MFMA operands; dO X^T, Ehat X^T -> dP, dA; dbeta
    bf16* qrow = sm.u.c.qrow;
    bf16* dPm = sm.u.c.dP;
    bf16* dAm = sm.u.c.dA;
    float* acc = sm.u.c.acc;
#pragma unroll
    for (int e = 0; e < NLD; ++e) {
      const int u = tid + e * NT, t = u / (DK / 8), i8 = 8 * (u % (DK / 8));
      *reinterpret_cast<uint4*>(&qrow[t * RS + i8]) =
          *reinterpret_cast<const uint4*>(qc + static_cast<uint32_t>(min(t, tl)) * qk_row + i8);
    }
    bf16x8 dOf[NV], Ef[NV], bXf[NV];
    {
      const int ta = 16 * w + lr;
      const size_t ro = (vrow0 + static_cast<size_t>(min(ta, tl)) * d.Hv) * DV;
      const bf16* dOg = static_cast<const bf16*>(p.dO) + ro;
      const bf16* Eg = static_cast<const bf16*>(p.dv) + ro;
      const float bt = sm.beta[ta];
#pragma unroll
      for (int kv = 0; kv < NV; ++kv) {
        dOf[kv] = as_bf16x8(*reinterpret_cast<const uint4*>(dOg + 32 * kv + 8 * lg));
        Ef[kv] = as_bf16x8(*reinterpret_cast<const uint4*>(Eg + 32 * kv + 8 * lg));
        bXf[kv] = scale8(load_bf16x8(&xs[ta * XS + 32 * kv + 8 * lg]), bt);
      }
      f32x4 g1[4], g2[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) g1[st] = g2[st] = f4zero();
#pragma unroll
      for (int kv = 0; kv < NV; ++kv)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16x8 bx = load_bf16x8(&xs[(16 * st + lr) * XS + 32 * kv + 8 * lg]);
          g1[st] = mfma16(dOf[kv], bx, g1[st]);
          g2[st] = mfma16(Ef[kv], bx, g2[st]);
        }
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * w + 4 * lg + r, s = 16 * st + lr;
          const float bs = sm.beta[s];
          dPm[t * TS + s] = bf16_of(s <= t ? g1[st][r] * bs : 0.f);
          dAm[t * TS + s] = bf16_of(s < t ? -g2[st][r] * bs : 0.f);
        }
    }
    {  // dbeta_t = eps_t . X_t (four lanes per step)
      const int t = tid >> 2, part = tid & 3;
      const bf16* eg = p.E + (vrow0 + static_cast<size_t>(min(t, tl)) * d.Hv) * DV;
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
      if (part == 0 && t < Lc) p.pdb[vrow0 + static_cast<size_t>(t) * d.Hv] = sdot;
    }
    __syncthreads();
    {  // q norms (with 1/sqrt(Dk))
      const int t = tid >> 2, part = tid & 3;
      float qq = 0.f;
#pragma unroll
      for (int e = 0; e < DK / 32; ++e) {
        float qf[8];
        unpack8(*reinterpret_cast<const uint4*>(&qrow[t * RS + (DK / 4) * part + 8 * e]), qf);
#pragma unroll
        for (int x = 0; x < 8; ++x) qq = fmaf(qf[x], qf[x], qq);
      }
      qq = quad_sum(qq);
      if (part == 0) sm.rq[t] = t < Lc ? (1.f / sqrtf(static_cast<float>(DK))) / sqrtf(qq + kNormEps) : 0.f;
    }
    __syncthreads();

    float* acc0 = acc;
    float* acc1 = acc + L * AS;
    float* acc2 = acc + 2 * L * AS;
    for (int ct = 0; ct < NCT; ++ct) {
      const int i0c = 16 * ct;
      // ---- C1: dQb, dKb, dKh for this wave's steps and channels i0c .. + 15;
      // their direct terms; the row sums of Kh dKh; <dH', H> (wave 0)
      {
        const int ic = i0c + lr;
        f32x4 aq = f4zero(), ak = f4zero(), ah = f4zero();
        float rh = 0.f;
#pragma unroll
        for (int kv = 0; kv < NV; ++kv) {
          const int v0 = 32 * kv + 8 * lg;
          float hf[8];
          if (H) {
            const float4 h0 = *reinterpret_cast<const float4*>(H + static_cast<size_t>(ic) * DV + v0);
            const float4 h1 = *reinterpret_cast<const float4*>(H + static_cast<size_t>(ic) * DV + v0 + 4);
            hf[0] = h0.x, hf[1] = h0.y, hf[2] = h0.z, hf[3] = h0.w;
            hf[4] = h1.x, hf[5] = h1.y, hf[6] = h1.z, hf[7] = h1.w;
          } else {
#pragma unroll
            for (int x = 0; x < 8; ++x) hf[x] = 0.f;
          }
          const uint4 dhu = *reinterpret_cast<const uint4*>(dHp + static_cast<size_t>(ic) * DV + v0);
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
        const float gL = sm.gam[(L - 1) * GS + ic];
        float rd = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * w + 4 * lg + r;
          const float g = sm.gam[t * GS + ic], eg = __expf(g), el = __expf(gL - g);
          acc0[t * AS + lr] = eg * aq[r];
          acc1[t * AS + lr] = -eg * ak[r];
          acc2[t * AS + lr] = el * ah[r];
          rd = fmaf(to_f32(sm.krow[t * RS + ic]) * sm.rk[t] * el, ah[r], rd);
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
      __syncthreads();

      // ---- C2: the diagonal sub-blocks in fp32 (every wave: lanes = 16
      // channels x 4 blocks; wave w takes the steps w, w + 4, ... of its block,
      // as rows and as columns) ...
      float dqd[4], dkrd[4], dkwd[4];
      {
        const int il = l & 15, I = l >> 4, b0 = 16 * I, icd = i0c + il;
        float Gv[16], kn[16], qs[16], gg[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          Gv[x] = sm.gam[(b0 + x) * GS + icd];
          kn[x] = to_f32(sm.krow[(b0 + x) * RS + icd]) * sm.rk[b0 + x];
          qs[x] = to_f32(qrow[(b0 + x) * RS + icd]) * sm.rq[b0 + x];
        }
        gg[0] = 1.f;
#pragma unroll
        for (int x = 1; x < 16; ++x) gg[x] = __expf(Gv[x] - Gv[x - 1]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int tt = w + 4 * m;  // uniform
          const bf16* prow = &dPm[(b0 + tt) * TS + b0];
          const bf16* arow = &dAm[(b0 + tt) * TS + b0];
          float e = 1.f, sq = 0.f, sr = 0.f;
#pragma unroll
          for (int s = 15; s >= 0; --s) {
            if (s > tt) continue;
            if (s < tt) e *= gg[s + 1];  // e = e^{G_tt - G_s}
            const float ke = kn[s] * e;
            sq = fmaf(to_f32(prow[s]), ke, sq);
            sr = fmaf(to_f32(arow[s]), ke, sr);
          }
          dqd[m] = sq;
          dkrd[m] = sr;
          e = 1.f;
          float sw = 0.f;
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            if (t < tt) continue;
            if (t > tt) e *= gg[t];  // e = e^{G_t - G_tt}
            sw = fmaf(fmaf(to_f32(dPm[(b0 + t) * TS + b0 + tt]), qs[t], to_f32(dAm[(b0 + t) * TS + b0 + tt]) * kn[t]), e, sw);
          }
          dkwd[m] = sw;
        }
      }
      // ... and off the diagonal on MFMA (wave I = 1 .. 3: rows of block I
      // against the blocks before it, split at r = 16 I - 1; rows of block
      // J = I - 1 against the blocks after it, split at e = 16 J + 15)
      if (w >= 1) {
        const int I = w, J = I - 1, ic = i0c + lr;
        const int r0 = 16 * I - 1, e0 = 16 * J + 15;
        const float Gr = sm.gam[r0 * GS + ic], Ge = sm.gam[e0 * GS + ic];
        f32x4 oq = f4zero(), orr = f4zero(), ow = f4zero();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (32 * kk >= 16 * I) continue;  // uniform
          float y[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int s = 32 * kk + 8 * lg + x;
            y[x] = s < 16 * I ? to_f32(sm.krow[s * RS + ic]) * sm.rk[s] * __expf(Gr - sm.gam[s * GS + ic]) : 0.f;
          }
          const bf16x8 yb = as_bf16x8(pack8(y));
          oq = mfma16(load_bf16x8(&dPm[(16 * I + lr) * TS + 32 * kk + 8 * lg]), yb, oq);
          orr = mfma16(load_bf16x8(&dAm[(16 * I + lr) * TS + 32 * kk + 8 * lg]), yb, orr);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (16 * I + 32 * kk >= L) continue;  // uniform
          float yq[8], yk[8], ap[8], aa[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int t = 16 * I + 32 * kk + 8 * lg + x;
            const bool in = t < L;
            const int tc = in ? t : L - 1;
            const float ee = in ? __expf(sm.gam[tc * GS + ic] - Ge) : 0.f;
            yq[x] = to_f32(qrow[tc * RS + ic]) * sm.rq[tc] * ee;
            yk[x] = to_f32(sm.krow[tc * RS + ic]) * sm.rk[tc] * ee;
            ap[x] = to_f32(dPm[tc * TS + 16 * J + lr]);
            aa[x] = to_f32(dAm[tc * TS + 16 * J + lr]);
          }
          ow = mfma16(as_bf16x8(pack8(ap)), as_bf16x8(pack8(yq)), ow);
          ow = mfma16(as_bf16x8(pack8(aa)), as_bf16x8(pack8(yk)), ow);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * I + 4 * lg + r, s = 16 * J + 4 * lg + r;
          const float sc = __expf(sm.gam[t * GS + ic] - Gr), sc2 = __expf(Ge - sm.gam[s * GS + ic]);
          acc0[t * AS + lr] += sc * oq[r];
          acc1[t * AS + lr] += sc * orr[r];
          acc2[s * AS + lr] += sc2 * ow[r];
        }
      }
      __syncthreads();
      {
        const int il = l & 15, b0 = 16 * (l >> 4);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int t = b0 + w + 4 * m;
          acc0[t * AS + il] += dqd[m];
          acc1[t * AS + il] += dkrd[m];
          acc2[t * AS + il] += dkwd[m];
        }
      }
      __syncthreads();

      // ---- C3: dG, dkn and the reverse cumulative sum (16 lanes per
      // channel, 4 steps each)
      {
        const int il = tid >> 4, seg = tid & 15, ic = i0c + il;
        const float rowdot = __expf(sm.gam[(L - 1) * GS + ic]) * sm.rdh[il] + sm.rdot[0][il] + sm.rdot[1][il] +
                             sm.rdot[2][il] + sm.rdot[3][il];
        float dg[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int t = 4 * seg + x;
          const float dq = acc0[t * AS + il], dkr = acc1[t * AS + il], dkw = acc2[t * AS + il];
          const float qv = to_f32(qrow[t * RS + ic]) * sm.rq[t], kv = to_f32(sm.krow[t * RS + ic]) * sm.rk[t];
          dg[x] = fmaf(qv, dq, kv * (dkr - dkw)) + (t == L - 1 ? rowdot : 0.f);
          acc1[t * AS + il] = dkr + dkw;
        }
        float suf[4];
        suf[3] = dg[3];
        suf[2] = dg[2] + suf[3];
        suf[1] = dg[1] + suf[2];
        suf[0] = dg[0] + suf[1];
        float run = suf[0];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          const float y = __shfl_down(run, off, 16);
          if (seg + off < 16) run += y;
        }
        const float later = run - suf[0];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int t = 4 * seg + x;
          acc2[t * AS + il] = sm.valid[t] != 0.f ? suf[x] + later : 0.f;
        }
      }
      __syncthreads();
      // ---- C4: the partials of this tile's channels
      for (int e = tid; e < L * 16; e += NT) {
        const int t = e >> 4, il = e & 15;
        if (t < Lc) {
          float* dst = p.part + (vrow0 + static_cast<size_t>(t) * d.Hv) * 3 * DK + i0c + il;
          dst[0] = acc0[t * AS + il];
          dst[DK] = acc1[t * AS + il];
          dst[2 * DK] = acc2[t * AS + il];
        }
      }
      __syncthreads();
    }
  }
};

template <int DK, int DV>
__global__ void __launch_bounds__(NT) vg_chunk_grad_kernel(VgChunkGradArgs p) {
  __shared__ typename VgGrad<DK, DV>::Smem sm;
  VgGrad<DK, DV>::run(p, sm);
}

template <int DK>
hipError_t launch_grad_dk(const VgChunkGradArgs& a, hipStream_t st) {
  const dim3 grid(a.d.nchunk(), a.d.B * a.d.Hv);
  switch (a.d.Dv) {
    case 32: vg_chunk_grad_kernel<DK, 32><<<grid, NT, 0, st>>>(a); break;
    case 64: vg_chunk_grad_kernel<DK, 64><<<grid, NT, 0, st>>>(a); break;
    case 96: vg_chunk_grad_kernel<DK, 96><<<grid, NT, 0, st>>>(a); break;
    case 128: vg_chunk_grad_kernel<DK, 128><<<grid, NT, 0, st>>>(a); break;
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

hipError_t launch_vg_chunk_grad(const VgChunkGradArgs& a, hipStream_t st) {
  if (a.d.T == 0) return hipSuccess;
  switch (a.d.Dk) {
    case 64: return launch_grad_dk<64>(a, st);
    case 128: return launch_grad_dk<128>(a, st);
    case 192: return launch_grad_dk<192>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
