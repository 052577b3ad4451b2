// Chunk-level gradient assembly of the gated delta rule backward on gfx950.
//
// Inside a chunk of L <= 64 steps (local t = 0..L-1, H = state before step 0,
// dH = dL/d(state after step L-1), gamma_t = l_0 + ... + l_t, gamma_L =
// gamma_{L-1}), with delta = beta X, X = V - U, and eps = dL/d delta, the
// states and the gradients w.r.t. the decayed states unroll to
//   S'_t  = e^{gamma_t} H + sum_{s<t} e^{gamma_t-gamma_s} kn_s delta_s^T
//   dS'_t = e^{gamma_L-gamma_t} dH
//           + sum_{r>=t} e^{gamma_r-gamma_t} (qn_r dO_r^T - beta_r kn_r eps_r^T)
// and D_t = dS'_t + beta_t kn_t eps_t^T.  The per-step gradients
//   dqn_t = S_t dO_t,   dkn_t = D_t delta_t + S'_t du_t   (du = -beta eps)
// become chunk products (masks and decays applied elementwise to L x L
// matrices, never as e^{-gamma}):
//   dQn = diag(e^g) dO H^T + Wq Kn,          Wq[t,s]  = [s<=t] e^{g_t-g_s} beta_s (dO_t . X_s)
//   dKn = diag(e^{gL-g} beta) X dH^T - diag(e^g beta) eps H^T + Wk1 Qn + Wk2 Kn
//         Wk1[t,r] = [r>=t] e^{g_r-g_t} beta_t (dO_r . X_t)
//         Wk2[t,s] = -beta_t beta_s ([s<t] e^{g_t-g_s} (X_s . eps_t) + [s>t] e^{g_s-g_t} (X_t . eps_s))
// The weights of the G value heads of a key head are summed before the final
// products, since Kn and Qn are shared by the group.
//
// Gate gradient: dl_t = <dS'_t, S'_t> (S'_t = g_t S_{t-1}), expanded the same way:
//   dl_t = e^{gL} <dH, H> + sum_{s<t} a_s + sum_{r>=t} b_r
//          + sum_{r>=t} sum_{s<t} e^{g_r-g_s} beta_s [(qn_r.kn_s)(dO_r.X_s)
//                                                    - beta_r (kn_r.kn_s)(eps_r.X_s)]
//   a_s = e^{gL-g_s} kn_s^T dH delta_s,   b_r = e^{g_r} (qn_r^T H dO_r - beta_r kn_r^T H eps_r).
// Every term carries the decay across step t, so a strongly decayed step is not
// the difference of large numbers; a step whose gate underflows gets exactly 0.
// Then da = dl (-e^{A_log}) sigmoid(x_c) [x <= 20], db = (eps . X) beta (1-beta),
// and the per-head parameter sums get sum_t dl_t l_t and sum_t da_t per chunk.
//
// Finally the L2-normalisation backward: dq = rq (dQn - q^ (q^ . dQn)) with
// q^ = qn sqrt(Dk), dk = rk (dKn - kn (kn . dKn)).
// All sums run in a fixed order; no atomics.
#include "gdn_dev.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int L = kChunk;   // rows per chunk (padded)
constexpr int NT = 512;     // 32 x 16 threads: RPT rows x (4 columns or Dk / 16 channels) each
constexpr int RPT = L / (NT / 16);  // rows per thread
constexpr int SLAB = 32;    // Dv columns per pass
constexpr int GB = 64;      // Dk columns per pass of the Gram matrices
constexpr int LP = L + 1;   // padded row stride of L x L arrays

template <int DK>
struct ChunkGrad {
  static constexpr int TI = DK / 16;        // Dk columns per thread
  static constexpr int HS = DK + 4;         // padded row stride of H^T slabs
  static constexpr int GW = DK < GB ? DK : GB;
  // Region R (floats), reused by the three phases:
  //   Gram phase:  Kn / Qn column blocks [L][GW+1]
  static constexpr int G_KS = 0;
  static constexpr int G_QS = L * (GW + 1);
  static constexpr int G_END = 2 * L * (GW + 1);
  //   slab phase:  H^T, dH^T [SLAB][HS]; X^T, eps^T, dO^T [SLAB][L]
  static constexpr int A_HT = 0;
  static constexpr int A_DHT = A_HT + SLAB * HS;
  static constexpr int A_XT = A_DHT + SLAB * HS;
  static constexpr int A_ET = A_XT + SLAB * L;
  static constexpr int A_DOT = A_ET + SLAB * L;
  static constexpr int A_END = A_DOT + SLAB * L;
  //   final phase: Kn (then Qn) rows [L][DK]; two transposed weights [L][L]
  static constexpr int C_KS = 0;
  static constexpr int C_W1 = C_KS + L * DK;
  static constexpr int C_W2 = C_W1 + L * L;
  static constexpr int C_END = C_W2 + L * L;
  static constexpr int R_END = (A_END > C_END ? (A_END > G_END ? A_END : G_END)
                                              : (C_END > G_END ? C_END : G_END));
  // Region B, live across phases.
  static constexpr int B_DOX = R_END;          // [L][LP]  dO_t . X_s
  static constexpr int B_XE = B_DOX + L * LP;  // X_t . eps_s
  static constexpr int B_M = B_XE + L * LP;    // rectangle terms of dl
  static constexpr int B_EG = B_M + L * LP;    // e^{gamma}
  static constexpr int B_EGL = B_EG + L;       // e^{gamma_L - gamma}
  static constexpr int B_BET = B_EGL + L;
  static constexpr int B_ELL = B_BET + L;
  static constexpr int B_DB = B_ELL + L;       // eps . X per row
  static constexpr int B_AV = B_DB + L;        // a_s
  static constexpr int B_BV = B_AV + L;        // b_r
  static constexpr int B_DLL = B_BV + L;       // dl_t l_t (valid steps)
  static constexpr int B_DAV = B_DLL + L;      // da_t (valid steps)
  static constexpr int B_RED = B_DAV + L;      // [NT] block-reduction scratch
  static constexpr int B_HDH = B_RED + NT;     // <dH, H>
  static constexpr int B_GAM = B_HDH + 2;      // gamma, fp64 (2 floats each)
  static constexpr int TOTAL = B_GAM + 2 * L;

  template <typename T>
  __device__ static void run(const ChunkGradArgs& p, float* sm) {
    const Dims& d = p.d;
    const int c = blockIdx.x, bj = blockIdx.y;
    const int b = bj / d.Hk, j = bj % d.Hk, G = d.G();
    const int t0 = c * L, Lc = min(L, d.T - t0);
    // lane coordinates; the head loop rebuilds them from an opaque copy of the
    // thread index, so that the addresses derived from them are not all kept
    // live across it
    int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    int rt = tid >> 3, rq8 = tid & 7;  // row / eighth for slab loads
    const size_t slab_sz = static_cast<size_t>(d.B) * d.Hv * DK * d.Dv;
    double* gam = reinterpret_cast<double*>(sm + B_GAM);
    const T* qg = static_cast<const T*>(p.q);
    const T* kg = static_cast<const T*>(p.k);
    auto qk_row = [&](int t) { return (static_cast<size_t>(b) * d.T + t0 + t) * d.Hk + j; };

    // The thread's own TI columns of kn / qn in row RPT tr + a (0 past the end),
    // read where they are used (after each head and in the normalisation
    // backward) rather than held in registers across the kernel, where the
    // accumulators of the key-head group already fill the register file.  The
    // row index passes through an empty asm statement so that the compiler
    // cannot prove two reloads equal and keep the values live in between.
    auto own = [&](const T* src, const float* scale, int a, float (&out)[TI]) {
      const int t = tr * RPT + a;
      const bool in = t < Lc;
      int ri = in ? static_cast<int>(qk_row(t)) : 0;
      asm volatile("" : "+v"(ri));
      const size_t row = static_cast<size_t>(ri);
      const float sc = in ? scale[row] : 0.f;
#pragma unroll
      for (int i = 0; i < TI; ++i) out[i] = to_f32(src[row * DK + tc * TI + i]) * sc;
    };
    // ---- the Gram matrices of the chunk
    float gqk[RPT][4], gkk[RPT][4];  // qn_r . kn_s, kn_r . kn_s for r = RPT tr + a, s = 4 tc + s
#pragma unroll
    for (int a = 0; a < RPT; ++a)
#pragma unroll
      for (int s = 0; s < 4; ++s) gqk[a][s] = gkk[a][s] = 0.f;
    for (int i0 = 0; i0 < DK; i0 += GW) {
      for (int e = tid; e < L * GW; e += NT) {
        const int t = e / GW, i = e % GW;
        float kv = 0.f, qv = 0.f;
        if (t < Lc) {
          const size_t row = qk_row(t);
          kv = to_f32(kg[row * DK + i0 + i]) * p.s.rk[row];
          qv = to_f32(qg[row * DK + i0 + i]) * p.s.rq[row];
        }
        sm[G_KS + t * (GW + 1) + i] = kv;
        sm[G_QS + t * (GW + 1) + i] = qv;
      }
      __syncthreads();
#pragma unroll 4
      for (int i = 0; i < GW; ++i) {
        float qr[RPT], kr[RPT], ks[4];
#pragma unroll
        for (int a = 0; a < RPT; ++a) {
          qr[a] = sm[G_QS + (tr * RPT + a) * (GW + 1) + i];
          kr[a] = sm[G_KS + (tr * RPT + a) * (GW + 1) + i];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) ks[a] = sm[G_KS + (tc * 4 + a) * (GW + 1) + i];
#pragma unroll
        for (int a = 0; a < RPT; ++a)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            gqk[a][s] = fmaf(qr[a], ks[s], gqk[a][s]);
            gkk[a][s] = fmaf(kr[a], ks[s], gkk[a][s]);
          }
      }
      __syncthreads();
    }

    float accQ[RPT][TI], accK[RPT][TI];
    float wq[RPT][4], wk1[RPT][4], wk2[RPT][4];
#pragma unroll
    for (int a = 0; a < RPT; ++a) {
#pragma unroll
      for (int i = 0; i < TI; ++i) accQ[a][i] = accK[a][i] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) wq[a][s] = wk1[a][s] = wk2[a][s] = 0.f;
    }

    for (int hh = 0; hh < G; ++hh) {
      tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      tr = tid >> 4;
      tc = tid & 15;
      rt = tid >> 3;
      rq8 = tid & 7;
      const int h = j * G + hh, bh = b * d.Hv + h;
      // ---- per-step scalars of head h, gamma in fp64
      if (tid < L) {
        const bool in = tid < Lc;
        const size_t r = (static_cast<size_t>(b) * d.T + t0 + tid) * d.Hv + h;
        sm[B_ELL + tid] = in ? p.s.ell[r] : 0.f;
        sm[B_BET + tid] = in ? p.s.beta[r] : 0.f;
      }
      __syncthreads();
      if (tid == 0) {
        double gsum = 0.0;
        for (int t = 0; t < L; ++t) {
          gsum += static_cast<double>(sm[B_ELL + t]);
          gam[t] = gsum;
        }
      }
      __syncthreads();
      if (tid < L) {
        sm[B_EG + tid] = expf(static_cast<float>(gam[tid]));
        sm[B_EGL + tid] = expf(static_cast<float>(gam[Lc - 1] - gam[tid]));
      }
      float accQh[RPT][TI], accKA[RPT][TI], accKE[RPT][TI];
      float acc_xe[RPT][4], acc_dox[RPT][4];
#pragma unroll
      for (int a = 0; a < RPT; ++a) {
#pragma unroll
        for (int i = 0; i < TI; ++i) accQh[a][i] = accKA[a][i] = accKE[a][i] = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) acc_xe[a][s] = acc_dox[a][s] = 0.f;
      }
      float part_db = 0.f, part_hdh = 0.f;
      const float* H = c == 0 ? p.state0 : p.ckpt + static_cast<size_t>(c - 1) * slab_sz;
      if (H) H += static_cast<size_t>(bh) * DK * d.Dv;
      const float* dH = p.dHend + static_cast<size_t>(c) * slab_sz + static_cast<size_t>(bh) * DK * d.Dv;
      const float kq = rt < Lc ? p.s.kq[qk_row(rt)] : 0.f;
      __syncthreads();

      for (int s0 = 0; s0 < d.Dv; s0 += SLAB) {
        tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        tr = tid >> 4;
        tc = tid & 15;
        rt = tid >> 3;
        rq8 = tid & 7;
        const int ns = min(SLAB, d.Dv - s0);
        // H^T and dH^T slabs, and <dH, H> over them
        for (int e = tid; e < DK * SLAB; e += NT) {
          const int i = e / SLAB, jj = e % SLAB;
          float hv = 0.f, dhv = 0.f;
          if (jj < ns) {
            const size_t o = static_cast<size_t>(i) * d.Dv + s0 + jj;
            hv = H ? H[o] : 0.f;
            dhv = dH[o];
          }
          part_hdh = fmaf(hv, dhv, part_hdh);
          sm[A_HT + jj * HS + i] = hv;
          sm[A_DHT + jj * HS + i] = dhv;
        }
        // X = v - U, eps = ein + (kn . qn) dO, dO slabs (transposed)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = rq8 * 4 + e;
          float x = 0.f, ev = 0.f, dov = 0.f;
          if (rt < Lc && jj < ns) {
            const size_t o = ((static_cast<size_t>(b) * d.T + t0 + rt) * d.Hv + h) * d.Dv + s0 + jj;
            x = to_f32(static_cast<const T*>(p.v)[o]) - p.U[o];
            dov = to_f32(static_cast<const T*>(p.dO)[o]);
            ev = fmaf(kq, dov, p.E[o]);
            part_db = fmaf(ev, x, part_db);
          }
          sm[A_XT + jj * L + rt] = x;
          sm[A_ET + jj * L + rt] = ev;
          sm[A_DOT + jj * L + rt] = dov;
        }
        __syncthreads();
        float rs_q[RPT], rs_x[RPT], rs_e[RPT];
#pragma unroll
        for (int a = 0; a < RPT; ++a) {
          const int t = tr * RPT + a;
          const float bet = sm[B_BET + t];
          rs_q[a] = sm[B_EG + t];
          rs_x[a] = sm[B_EGL + t] * bet;
          rs_e[a] = -sm[B_EG + t] * bet;
        }
#pragma unroll 2
        for (int jj = 0; jj < SLAB; ++jj) {
          float hv[TI], dhv[TI];
#pragma unroll
          for (int i = 0; i < TI; ++i) {
            hv[i] = sm[A_HT + jj * HS + tc * TI + i];
            dhv[i] = sm[A_DHT + jj * HS + tc * TI + i];
          }
          float dor[RPT], xr[RPT], er[RPT], xc[4], ec[4];
#pragma unroll
          for (int a = 0; a < RPT; ++a) {
            dor[a] = sm[A_DOT + jj * L + tr * RPT + a];
            xr[a] = sm[A_XT + jj * L + tr * RPT + a];
            er[a] = sm[A_ET + jj * L + tr * RPT + a];
          }
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            xc[a] = sm[A_XT + jj * L + tc * 4 + a];
            ec[a] = sm[A_ET + jj * L + tc * 4 + a];
          }
#pragma unroll
          for (int a = 0; a < RPT; ++a) {
            const float qs = dor[a] * rs_q[a];
            const float xs = xr[a] * rs_x[a];
            const float es = er[a] * rs_e[a];
#pragma unroll
            for (int i = 0; i < TI; ++i) {
              accQh[a][i] = fmaf(qs, hv[i], accQh[a][i]);
              accKA[a][i] = fmaf(xs, dhv[i], accKA[a][i]);
              accKE[a][i] = fmaf(es, hv[i], accKE[a][i]);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              acc_dox[a][s] = fmaf(dor[a], xc[s], acc_dox[a][s]);  // dO_t . X_s
              acc_xe[a][s] = fmaf(xr[a], ec[s], acc_xe[a][s]);     // X_t . eps_s
            }
          }
        }
        __syncthreads();
      }

      // ---- a_s, b_r from the diagonal terms; merge them into the group sums
#pragma unroll
      for (int a = 0; a < RPT; ++a) {
        float pa = 0.f, pb = 0.f;
        float kown[TI], qown[TI];
        own(kg, p.s.rk, a, kown);
        own(qg, p.s.rq, a, qown);
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          pa = fmaf(kown[i], accKA[a][i], pa);
          pb = fmaf(qown[i], accQh[a][i], fmaf(kown[i], accKE[a][i], pb));
          accQ[a][i] += accQh[a][i];
          accK[a][i] += accKA[a][i] + accKE[a][i];
        }
        pa = row_sum16(pa);
        pb = row_sum16(pb);
        if (tc == 0) {
          sm[B_AV + tr * RPT + a] = pa;
          sm[B_BV + tr * RPT + a] = pb;
        }
      }
#pragma unroll
      for (int a = 0; a < RPT; ++a)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          sm[B_DOX + (tr * RPT + a) * LP + tc * 4 + s] = acc_dox[a][s];
          sm[B_XE + (tr * RPT + a) * LP + tc * 4 + s] = acc_xe[a][s];
        }
      part_db += __shfl_xor(part_db, 1);
      part_db += __shfl_xor(part_db, 2);
      part_db += __shfl_xor(part_db, 4);
      if (rq8 == 0) sm[B_DB + rt] = part_db;
      sm[B_RED + tid] = part_hdh;
      __syncthreads();

      // ---- L x L weights of head h and the rectangle terms of dl
#pragma unroll
      for (int a = 0; a < RPT; ++a) {
        const int t = tr * RPT + a;
        const float bt = sm[B_BET + t];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int s = tc * 4 + s4;
          const float bs = sm[B_BET + s];
          float m = 0.f;
          if (s <= t) {
            const float e = expf(static_cast<float>(gam[t] - gam[s]));
            wq[a][s4] = fmaf(e * bs, acc_dox[a][s4], wq[a][s4]);
            if (s < t) {
              const float xe_st = sm[B_XE + s * LP + t];  // X_s . eps_t
              wk2[a][s4] = fmaf(-bt * bs * e, xe_st, wk2[a][s4]);
              // (r, s) = (t, s): e^{g_t-g_s} beta_s [(qn_t.kn_s)(dO_t.X_s) - beta_t (kn_t.kn_s)(eps_t.X_s)]
              m = e * bs * (gqk[a][s4] * acc_dox[a][s4] - bt * gkk[a][s4] * xe_st);
            }
          }
          if (s >= t) {
            const float e = expf(static_cast<float>(gam[s] - gam[t]));
            wk1[a][s4] = fmaf(e * bt, sm[B_DOX + s * LP + t], wk1[a][s4]);
            if (s > t) wk2[a][s4] = fmaf(-bt * bs * e, acc_xe[a][s4], wk2[a][s4]);
          }
          sm[B_M + t * LP + s] = m;
        }
      }
      if (tid == 0) {
        float hdh = 0.f;
        for (int i = 0; i < NT; ++i) hdh += sm[B_RED + i];
        sm[B_HDH] = hdh;
      }
      __syncthreads();

      // ---- gate gradients of head h, one thread per step
      if (tid < Lc) {
        const int t = tid;
        double acc = static_cast<double>(expf(static_cast<float>(gam[Lc - 1]))) * sm[B_HDH];
        for (int s = 0; s < t; ++s) acc += sm[B_AV + s];
        for (int r = t; r < Lc; ++r) acc += sm[B_BV + r];
        for (int r = t; r < Lc; ++r) {
          float row = 0.f;
          for (int s = 0; s < t; ++s) row += sm[B_M + r * LP + s];
          acc += row;
        }
        const float ell = sm[B_ELL + t];
        const float dl = expf(ell) == 0.f ? 0.f : static_cast<float>(acc);
        const size_t r = (static_cast<size_t>(b) * d.T + t0 + t) * d.Hv + h;
        const bool valid = p.mask == nullptr || p.mask[static_cast<size_t>(b) * d.T + t0 + t] != 0;
        float da = 0.f, db = 0.f, dll = 0.f;
        if (valid) {
          const float x = to_f32(static_cast<const T*>(p.a)[r]) + p.dt_bias[h];
          const float xc = fminf(x, kClamp);
          da = x <= kClamp ? dl * (-expf(p.A_log[h])) * sigmoid_f(xc) : 0.f;
          const float beta = sm[B_BET + t];
          db = sm[B_DB + t] * beta * (1.f - beta);
          dll = dl != 0.f ? dl * ell : 0.f;
        }
        static_cast<T*>(p.da)[r] = from_f32<T>(da);
        static_cast<T*>(p.db)[r] = from_f32<T>(db);
        sm[B_DLL + t] = dll;
        sm[B_DAV + t] = da;
      }
      __syncthreads();
      if (tid == 0) {
        double sa = 0.0, sd = 0.0;
        for (int t = 0; t < Lc; ++t) {
          sa += sm[B_DLL + t];
          sd += sm[B_DAV + t];
        }
        const size_t pi = (static_cast<size_t>(b) * d.nchunk() + c) * d.Hv + h;
        p.part_dA[pi] = sa;
        p.part_ddt[pi] = sd;
      }
      __syncthreads();
    }

    // ---- final products with the shared kn / qn rows
    tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    tr = tid >> 4;
    tc = tid & 15;
    auto load_rows = [&](const T* src, const float* scale) {
      for (int e = tid; e < L * DK; e += NT) {
        const int t = e / DK, i = e % DK;
        float v = 0.f;
        if (t < Lc) {
          const size_t row = qk_row(t);
          v = to_f32(src[row * DK + i]) * scale[row];
        }
        sm[C_KS + e] = v;
      }
    };
    // pass 1: kn rows; dQn += Wq Kn, dKn += Wk2 Kn
    load_rows(kg, p.s.rk);
#pragma unroll
    for (int a = 0; a < RPT; ++a)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sm[C_W1 + (tc * 4 + s) * L + tr * RPT + a] = wq[a][s];   // stored [s][t]
        sm[C_W2 + (tc * 4 + s) * L + tr * RPT + a] = wk2[a][s];
      }
    __syncthreads();
#pragma unroll 2
    for (int s = 0; s < L; ++s) {
      float kv[TI];
#pragma unroll
      for (int i = 0; i < TI; ++i) kv[i] = sm[C_KS + s * DK + tc * TI + i];
#pragma unroll
      for (int a = 0; a < RPT; ++a) {
        const float w1 = sm[C_W1 + s * L + tr * RPT + a], w2 = sm[C_W2 + s * L + tr * RPT + a];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          accQ[a][i] = fmaf(w1, kv[i], accQ[a][i]);
          accK[a][i] = fmaf(w2, kv[i], accK[a][i]);
        }
      }
    }
    __syncthreads();
    // pass 2: qn rows; dKn += Wk1 Qn
    load_rows(qg, p.s.rq);
#pragma unroll
    for (int a = 0; a < RPT; ++a)
#pragma unroll
      for (int s = 0; s < 4; ++s) sm[C_W1 + (tc * 4 + s) * L + tr * RPT + a] = wk1[a][s];
    __syncthreads();
#pragma unroll 2
    for (int s = 0; s < L; ++s) {
      float qv[TI];
#pragma unroll
      for (int i = 0; i < TI; ++i) qv[i] = sm[C_KS + s * DK + tc * TI + i];
#pragma unroll
      for (int a = 0; a < RPT; ++a) {
        const float w1 = sm[C_W1 + s * L + tr * RPT + a];
#pragma unroll
        for (int i = 0; i < TI; ++i) accK[a][i] = fmaf(w1, qv[i], accK[a][i]);
      }
    }
    // ---- normalisation backward and output
    const float dkf = static_cast<float>(DK);
#pragma unroll
    for (int a = 0; a < RPT; ++a) {
      const int t = tr * RPT + a;
      float dq_dot = 0.f, dk_dot = 0.f;
      float kown[TI], qown[TI];
      own(kg, p.s.rk, a, kown);
      own(qg, p.s.rq, a, qown);
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        dq_dot = fmaf(qown[i], accQ[a][i], dq_dot);
        dk_dot = fmaf(kown[i], accK[a][i], dk_dot);
      }
      dq_dot = row_sum16(dq_dot);
      dk_dot = row_sum16(dk_dot);
      if (t < Lc) {
        const size_t row = qk_row(t);
        const float rq = p.s.rq[row], rk = p.s.rk[row];
        T* dq = static_cast<T*>(p.dq) + row * DK;
        T* dk = static_cast<T*>(p.dk) + row * DK;
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          dq[tc * TI + i] = from_f32<T>(rq * (accQ[a][i] - dkf * qown[i] * dq_dot));
          dk[tc * TI + i] = from_f32<T>(rk * (accK[a][i] - kown[i] * dk_dot));
        }
      }
    }
  }
};

template <int DK, typename T>
__global__ void __launch_bounds__(NT) chunk_grad_kernel(ChunkGradArgs p) {
  __shared__ float sm[ChunkGrad<DK>::TOTAL];
  ChunkGrad<DK>::template run<T>(p, sm);
}

template <typename T>
hipError_t launch_t(const ChunkGradArgs& a, hipStream_t st) {
  dim3 grid(a.d.nchunk(), a.d.B * a.d.Hk);
  switch (a.d.Dk) {
    case 16: chunk_grad_kernel<16, T><<<grid, NT, 0, st>>>(a); break;
    case 32: chunk_grad_kernel<32, T><<<grid, NT, 0, st>>>(a); break;
    case 64: chunk_grad_kernel<64, T><<<grid, NT, 0, st>>>(a); break;
    case 128: chunk_grad_kernel<128, T><<<grid, NT, 0, st>>>(a); break;
    case 192: chunk_grad_kernel<192, T><<<grid, NT, 0, st>>>(a); break;
    case 256: chunk_grad_kernel<256, T><<<grid, NT, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// dA_log[h] = sum over (b, chunk) of the per-chunk sums, ddt_bias likewise,
// in fp64: one wave per head; lane l adds the entries l, l + 64, ... in that
// order, then the 64 lane sums meet in a fixed butterfly, so the result does
// not depend on timing.
__global__ void __launch_bounds__(64) param_reduce_kernel(ParamReduceArgs p) {
  const int h = blockIdx.x, l = threadIdx.x;
  const int n = p.B * p.NC;
  double sa = 0.0, sd = 0.0;
  for (int e = l; e < n; e += 64) {
    const size_t i = static_cast<size_t>(e) * p.Hv + h;  // e = b * NC + c
    sa += p.part_dA[i];
    sd += p.part_ddt[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sa += __shfl_xor(sa, off);
    sd += __shfl_xor(sd, off);
  }
  if (l == 0) {
    p.dA_log[h] = static_cast<float>(sa);
    p.ddt_bias[h] = static_cast<float>(sd);
  }
}

}  // namespace

hipError_t launch_chunk_grad(const ChunkGradArgs& a, bool bf16, hipStream_t st) {
  if (a.d.T == 0 || a.d.B * a.d.Hk == 0) return hipSuccess;
  return bf16 ? launch_t<gdn::bf16>(a, st) : launch_t<float>(a, st);
}

hipError_t launch_param_reduce(const ParamReduceArgs& a, hipStream_t st) {
  param_reduce_kernel<<<a.Hv, 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace gdn
