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
//   chunk_prep  one workgroup per (chunk, batch, value head): K K^T and Q K^T on
//               MFMA, N, Tx by forward substitution (fp32), Mq and the per-step
//               chunk scalars; the first head of each key-head group also
//               writes K^T.  With `bwd` set it also writes the transposes the
//               backward needs.  All outputs go to the workspace (bf16 / fp32).
//   chunk_fwd   one workgroup per (batch, value head, 32-column slice of Dv),
//               walking the chunks in order with H in MFMA accumulators (fp32),
//               the next chunk's operands prefetched into registers while the
//               current chunk computes (the in-chunk barriers wait for LDS
//               only, so the prefetch stays in flight across them).  Blocks
//               that share a key head run on one XCD, so their K / Q / K^T
//               reads hit that XCD's L2.  Writes o, the checkpoints and the
//               final state.
#include "gdn_dev.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int L = kChunk;
constexpr int LP = L + 1;
constexpr int NT = 256;

// ------------------------------------------------------------------ prep

template <int DK>
struct ChunkPrep {
  static constexpr int KS = DK + 8;  // bf16 row stride of the staged K / Q tile
  static constexpr int MAT_BYTES = 2 * L * LP * 4;
  static constexpr int TILE_BYTES = L * KS * 2;
  static constexpr int BUF_BYTES = MAT_BYTES > TILE_BYTES ? MAT_BYTES : TILE_BYTES;
  struct Smem {
    alignas(16) char buf[BUF_BYTES];  // N / Tx and a transpose stage, or a K / Q tile
    float gam[L], rk[L], rq[L], beta[L];
  };

  __device__ static void run(const ChunkPrepArgs& p, Smem& sm) {
    const Dims& d = p.d;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int G = d.G(), NC = d.nchunk();
    const int b = bh / d.Hv, h = bh % d.Hv, j = h / G, hh = h % G, bj = b * d.Hk + j;
    const int t0 = c * L, Lc = min(L, d.T - t0);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    const bf16* kg = static_cast<const bf16*>(p.k);
    const bf16* qg = static_cast<const bf16*>(p.q);
    float* nm = reinterpret_cast<float*>(sm.buf);   // [L][LP]
    float* st = nm + L * LP;                         // [L][LP] transpose stage
    const size_t mat = (static_cast<size_t>(bh) * NC + c) * L * L;
    auto qk_row = [&](int t) { return (static_cast<size_t>(b) * d.T + t0 + t) * d.Hk + j; };

    // ---- per-step scalars; gamma by a wave-wide inclusive scan
    if (w == 0) {
      float ell = 0.f, beta = 0.f, rk = 0.f, rq = 0.f;
      if (l < Lc) {
        const size_t bt = static_cast<size_t>(b) * d.T + t0 + l;
        ell = p.s.ell[bt * d.Hv + h];
        beta = p.s.beta[bt * d.Hv + h];
        rk = p.s.rk[bt * d.Hk + j];
        rq = p.s.rq[bt * d.Hk + j];
      }
      float g = ell;
#pragma unroll
      for (int off = 1; off < L; off <<= 1) {
        const float y = __shfl_up(g, off);
        if (l >= off) g += y;
      }
      sm.gam[l] = g;
      sm.rk[l] = rk;
      sm.rq[l] = rq;
      sm.beta[l] = beta;
    }
    __syncthreads();
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
    }

    // ---- K K^T and Q K^T (raw rows): wave w computes row tile w
    f32x4 akk[4], aqk[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) akk[ct] = aqk[ct] = f4zero();
    {
      const int ta = 16 * w + lr;
#pragma unroll
      for (int kt = 0; kt < DK / 32; ++kt) {
        const int e0 = 32 * kt + 8 * lg;
        const bf16x8 ak = ta < Lc ? load_bf16x8(kg + qk_row(ta) * DK + e0) : zero8();
        const bf16x8 aq = ta < Lc ? load_bf16x8(qg + qk_row(ta) * DK + e0) : zero8();
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int tb = 16 * ct + lr;
          const bf16x8 bk = tb < Lc ? load_bf16x8(kg + qk_row(tb) * DK + e0) : zero8();
          akk[ct] = mfma16(ak, bk, akk[ct]);
          aqk[ct] = mfma16(aq, bk, aqk[ct]);
        }
      }
    }
    // ---- N, Mq (and the backward's A~, P) from the accumulators
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * w + 4 * lg + r, s = 16 * ct + lr;
        float nv = 0.f, mq = 0.f, at = 0.f, pq = 0.f;
        if (s <= t) {
          const float dec = expf(sm.gam[t] - sm.gam[s]);
          const float krs = dec * sm.rk[t] * sm.rk[s];
          if (s < t) {
            at = krs * akk[ct][r];
            nv = at * sm.beta[s];
          }
          pq = dec * sm.rq[t] * sm.rk[s] * aqk[ct][r];
          mq = pq * sm.beta[s];
        }
        nm[t * LP + s] = nv;
        p.cb.Mq[mat + t * L + s] = bf16_of(mq);
        if (p.bwd) {
          st[s * LP + t] = at;   // staged transposed
          akk[ct][r] = pq;       // keep P for the second stage
        }
      }
    __syncthreads();
    if (p.bwd) {
      for (int e = tid; e < L * L; e += NT) p.cb.AtT[mat + e] = bf16_of(st[(e / L) * LP + e % L]);
      __syncthreads();
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[(16 * ct + lr) * LP + 16 * w + 4 * lg + r] = akk[ct][r];
      __syncthreads();
      for (int e = tid; e < L * L; e += NT) p.cb.PqT[mat + e] = bf16_of(st[(e / L) * LP + e % L]);
    }

    // ---- Tx = (I + N)^-1 by forward substitution: column `col`, four threads
    // per column, thread q4 holding the entries at rows 4m + q4.
    float x[L / 4];
    {
      const int col = tid >> 2, q4 = tid & 3;
#pragma unroll
      for (int m = 0; m < L / 4; ++m) x[m] = 0.f;
#pragma unroll
      for (int t = 0; t < L; ++t) {
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int m = 0; m < L / 4; m += 2) {
          p0 = fmaf(nm[t * LP + 4 * m + q4], x[m], p0);
          p1 = fmaf(nm[t * LP + 4 * m + 4 + q4], x[m + 1], p1);
        }
        const float xt = (t == col ? 1.f : 0.f) - quad_sum(p0 + p1);
        if ((t & 3) == q4) x[t >> 2] = xt;
      }
      __syncthreads();  // every thread is done reading N
#pragma unroll
      for (int m = 0; m < L / 4; ++m) nm[(4 * m + q4) * LP + col] = x[m];
    }
    __syncthreads();
    for (int e = tid; e < L * L; e += NT) {
      const int t = e / L, s = e % L;
      p.cb.Tx[mat + e] = bf16_of(nm[t * LP + s]);
      if (p.bwd) p.cb.TxT[mat + e] = bf16_of(nm[s * LP + t]);
    }

    // ---- raw k (and q) of the chunk transposed, once per key-head group
    if (hh == 0) {
      bf16* tile = reinterpret_cast<bf16*>(sm.buf);
      const size_t base = (static_cast<size_t>(bj) * NC + c) * DK * L;
      for (int pass = 0; pass < (p.bwd ? 2 : 1); ++pass) {
        const bf16* src = pass == 0 ? kg : qg;
        bf16* dst = pass == 0 ? p.cb.KT : p.cb.QT;
        __syncthreads();
        for (int u = tid; u < L * DK / 8; u += NT) {
          const int t = u / (DK / 8), e0 = (u % (DK / 8)) * 8;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (t < Lc) v = *reinterpret_cast<const uint4*>(src + qk_row(t) * DK + e0);
          *reinterpret_cast<uint4*>(&tile[t * KS + e0]) = v;
        }
        __syncthreads();
        for (int e = tid; e < DK * L; e += NT) dst[base + e] = tile[(e % L) * KS + e / L];
      }
    }
  }
};

template <int DK>
__global__ void __launch_bounds__(NT) chunk_prep_kernel(ChunkPrepArgs p) {
  __shared__ typename ChunkPrep<DK>::Smem sm;
  ChunkPrep<DK>::run(p, sm);
}

// ------------------------------------------------------------ state pass

template <int DK>
struct ChunkFwd {
  static constexpr int NV = 32;             // Dv columns per workgroup
  static constexpr int RTW = DK / 64;       // H row tiles per wave
  static constexpr int HS = DK + 8;         // bf16 row stride of H^T
  static constexpr int XS = L + 8;          // bf16 row stride of R^T / X^T
  struct Smem {
    alignas(16) bf16 hb[NV * HS];   // H^T (bf16), the B operand of K H and Q H
    alignas(16) bf16 rb[NV * XS];   // R^T
    alignas(16) bf16 xb[NV * XS];   // X^T
    alignas(16) bf16 xw[NV * XS];   // (diag(w) X)^T
  };
  // The operands of one chunk, held in registers (prefetched one chunk ahead).
  // Every load is unconditional, from an address clamped into the sequence, so
  // no load sits in a branch (a load in a branch makes the compiler wait for
  // all outstanding loads, prefetch included).  Rows past the end of the
  // sequence hold copies of its last row and need no zeroing: their chunk
  // scalars (rk, w) are zero, Tx and Mq are lower triangular and their outputs
  // are not stored, so they never reach a stored value (inputs are finite).
  struct Stage {
    bf16x8 ka[DK / 32], qa[DK / 32];  // k, q rows t = 16 w + lr
    bf16x8 txa[2], mqa[2];            // Tx, Mq rows t = 16 w + lr
    bf16x8 kta[RTW][2];               // K^T rows i = 16 (w RTW + it) + lr
    unsigned short vv[2][4];          // v bits at rows t = 16 w + 4 lg + r, cols 16 ct + lr
    float4 cr, co, wv;                // chunk scalars at rows 16 w + 4 lg + r
    float egl;
  };
  // Per-workgroup values (uniform) and per-lane 32-bit offsets.  Addresses are
  // formed as a uniform 64-bit base plus a 32-bit lane offset.
  struct Lane {
    int b, h, j, bh, bj, col0, w, lr, lg, ta, tc0, last, NC;
    uint32_t qk_row, v_row, o_row;   // element strides of one step in q/k, v, o
  };

  __device__ static void load_stage(const ChunkFwdArgs& p, const Lane& q, int c, Stage& s) {
    const Dims& d = p.d;
    const int t0 = c * L, tl = q.last - t0;
    const bf16* kc = static_cast<const bf16*>(p.k) + ((static_cast<size_t>(q.b) * d.T + t0) * d.Hk + q.j) * DK;
    const bf16* qc = static_cast<const bf16*>(p.q) + ((static_cast<size_t>(q.b) * d.T + t0) * d.Hk + q.j) * DK;
    const uint32_t ko = static_cast<uint32_t>(min(q.ta, tl)) * q.qk_row + 8 * q.lg;
#pragma unroll
    for (int kt = 0; kt < DK / 32; ++kt) {
      s.ka[kt] = load_bf16x8(kc + ko + 32 * kt);
      s.qa[kt] = load_bf16x8(qc + ko + 32 * kt);
    }
    const size_t mat = (static_cast<size_t>(q.bh) * q.NC + c) * L * L;
    const bf16* txc = p.cb.Tx + mat;
    const bf16* mqc = p.cb.Mq + mat;
    const uint32_t mo = q.ta * L + 8 * q.lg;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s.txa[kt] = load_bf16x8(txc + mo + 32 * kt);
      s.mqa[kt] = load_bf16x8(mqc + mo + 32 * kt);
    }
    const bf16* ktc = p.cb.KT + (static_cast<size_t>(q.bj) * q.NC + c) * DK * L;
    const uint32_t kto = (16 * q.w * RTW + q.lr) * L + 8 * q.lg;
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s.kta[it][kt] = load_bf16x8(ktc + kto + (it * 16 * L + 32 * kt));
    const unsigned short* vc = static_cast<const unsigned short*>(p.v) +
                               ((static_cast<size_t>(q.b) * d.T + t0) * d.Hv + q.h) * d.Dv + q.col0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t vo = static_cast<uint32_t>(min(q.tc0 + r, tl)) * q.v_row + q.lr;
      s.vv[0][r] = vc[vo];
      s.vv[1][r] = (vc + vo)[16];
    }
    const float* scc = p.cb.sc + (static_cast<size_t>(q.bh) * q.NC + c) * SC_ROWS * L;
    const float* scl = scc + q.tc0;
    s.cr = *reinterpret_cast<const float4*>(scl + SC_CR * L);
    s.co = *reinterpret_cast<const float4*>(scl + SC_CO * L);
    s.wv = *reinterpret_cast<const float4*>(scl + SC_W * L);
    s.egl = scc[SC_EGL * L];
  }

  __device__ static void put_h(Smem& sm, const Lane& q, const f32x4 (&H)[RTW][2]) {
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        *reinterpret_cast<uint2*>(&sm.hb[(16 * ct + q.lr) * HS + 16 * (q.w * RTW + it) + 4 * q.lg]) =
            pack4_bf16(H[it][ct][0], H[it][ct][1], H[it][ct][2], H[it][ct][3]);
  }

  // One chunk: o for its rows, H advanced to the next chunk's start.
  __device__ static void step(const ChunkFwdArgs& p, Smem& sm, const Lane& q, int c,
                              const Stage& cur, f32x4 (&H)[RTW][2]) {
    const Dims& d = p.d;
    const int t0 = c * L, Lc = min(L, d.T - t0);
    const int lr = q.lr, lg = q.lg;
    const float crv[4] = {cur.cr.x, cur.cr.y, cur.cr.z, cur.cr.w};
    const float cov[4] = {cur.co.x, cur.co.y, cur.co.z, cur.co.w};
    const float wvv[4] = {cur.wv.x, cur.wv.y, cur.wv.z, cur.wv.w};

    // step 1: K H and Q H for row tile w
    f32x4 kh[2], qh[2];
    kh[0] = kh[1] = qh[0] = qh[1] = f4zero();
#pragma unroll
    for (int kt = 0; kt < DK / 32; ++kt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const bf16x8 bh8 = load_bf16x8(&sm.hb[(16 * ct + lr) * HS + 32 * kt + 8 * lg]);
        kh[ct] = mfma16(cur.ka[kt], bh8, kh[ct]);
        qh[ct] = mfma16(cur.qa[kt], bh8, qh[ct]);
      }
    // step 2: R = V - diag(e^gamma rk) K H  -> rb (transposed, bf16)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float rv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rv[r] = __uint_as_float(static_cast<uint32_t>(cur.vv[ct][r]) << 16) - crv[r] * kh[ct][r];
      }
      *reinterpret_cast<uint2*>(&sm.rb[(16 * ct + lr) * XS + q.tc0]) = pack4_bf16(rv[0], rv[1], rv[2], rv[3]);
    }
    lds_barrier();
    // step 3: X = Tx R for row tile w; X and diag(w) X to LDS
    f32x4 x[2];
    x[0] = x[1] = f4zero();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        x[ct] = mfma16(cur.txa[kt], load_bf16x8(&sm.rb[(16 * ct + lr) * XS + 32 * kt + 8 * lg]), x[ct]);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      *reinterpret_cast<uint2*>(&sm.xb[(16 * ct + lr) * XS + q.tc0]) =
          pack4_bf16(x[ct][0], x[ct][1], x[ct][2], x[ct][3]);
      *reinterpret_cast<uint2*>(&sm.xw[(16 * ct + lr) * XS + q.tc0]) =
          pack4_bf16(wvv[0] * x[ct][0], wvv[1] * x[ct][1], wvv[2] * x[ct][2], wvv[3] * x[ct][3]);
    }
    lds_barrier();
    // step 4: O = diag(e^gamma rq) Q H + Mq X for row tile w
    {
      f32x4 o[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[ct][r] = cov[r] * qh[ct][r];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          o[ct] = mfma16(cur.mqa[kt], load_bf16x8(&sm.xb[(16 * ct + lr) * XS + 32 * kt + 8 * lg]), o[ct]);
      bf16* oc = static_cast<bf16*>(p.o) + ((static_cast<size_t>(q.b) * d.T + t0) * d.Hv + q.h) * d.Dv + q.col0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = q.tc0 + r;
        if (t < Lc) {
          const uint32_t oo = static_cast<uint32_t>(t) * q.o_row + lr;
          oc[oo] = bf16_of(o[0][r]);
          (oc + oo)[16] = bf16_of(o[1][r]);
        }
      }
    }
    // step 5: H = e^{gamma_L} H + K^T diag(w) X for the wave's row tiles
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) H[it][ct][r] *= cur.egl;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      bf16x8 bx[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) bx[ct] = load_bf16x8(&sm.xw[(16 * ct + lr) * XS + 32 * kt + 8 * lg]);
#pragma unroll
      for (int it = 0; it < RTW; ++it)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) H[it][ct] = mfma16(cur.kta[it][kt], bx[ct], H[it][ct]);
    }
    // step 6: H^T for the next chunk; checkpoint of the state at chunk c+1's start
    put_h(sm, q, H);
    if (p.ckpt && c + 1 < q.NC) {
      float* ck = p.ckpt + (static_cast<size_t>(c) * d.B * d.Hv + q.bh) * DK * d.Dv + q.col0 +
                  (static_cast<uint32_t>(16 * q.w * RTW + 4 * lg) * d.Dv + lr);
#pragma unroll
      for (int it = 0; it < RTW; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* cp = ck + static_cast<uint32_t>(16 * it + r) * d.Dv;
          cp[0] = H[it][0][r];
          cp[16] = H[it][1][r];
        }
    }
    lds_barrier();
  }

  __device__ static void run(const ChunkFwdArgs& p, Smem& sm) {
    const Dims& d = p.d;
    Lane q;
    const int nslice = d.Dv / NV;
    int slice;
    block_coords(d, nslice, q.b, q.h, slice);
    q.NC = d.nchunk();
    q.j = q.h / d.G();
    q.bh = q.b * d.Hv + q.h;
    q.bj = q.b * d.Hk + q.j;
    q.col0 = slice * NV;
    const int tid = threadIdx.x, l = tid & 63;
    q.w = tid >> 6;
    q.lr = l & 15;
    q.lg = l >> 4;
    q.ta = 16 * q.w + q.lr;
    q.tc0 = 16 * q.w + 4 * q.lg;
    q.last = d.T - 1;
    q.qk_row = d.Hk * DK;
    q.v_row = q.o_row = d.Hv * d.Dv;
    const size_t sbase = static_cast<size_t>(q.bh) * DK * d.Dv;

    // H: rows i = 16 (w RTW + it) + 4 lg + r, columns col0 + 16 ct + lr
    f32x4 H[RTW][2];
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * (q.w * RTW + it) + 4 * q.lg + r;
          H[it][ct][r] = p.state0 ? p.state0[sbase + static_cast<size_t>(i) * d.Dv + q.col0 + 16 * ct + q.lr] : 0.f;
        }
    put_h(sm, q, H);
    lds_barrier();

    Stage s0, s1;
    if (q.NC > 0) load_stage(p, q, 0, s0);
    for (int c = 0; c < q.NC; c += 2) {
      if (c + 1 < q.NC) load_stage(p, q, c + 1, s1);
      step(p, sm, q, c, s0, H);
      if (c + 1 >= q.NC) break;
      if (c + 2 < q.NC) load_stage(p, q, c + 2, s0);
      step(p, sm, q, c + 1, s1, H);
    }
#pragma unroll
    for (int it = 0; it < RTW; ++it)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * (q.w * RTW + it) + 4 * q.lg + r;
          p.state_out[sbase + static_cast<size_t>(i) * d.Dv + q.col0 + 16 * ct + q.lr] = H[it][ct][r];
        }
  }
};

template <int DK>
__global__ void __launch_bounds__(NT) chunk_fwd_kernel(ChunkFwdArgs p) {
  __shared__ typename ChunkFwd<DK>::Smem sm;
  ChunkFwd<DK>::run(p, sm);
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

hipError_t launch_chunk_fwd(const ChunkFwdArgs& a, hipStream_t st) {
  const int nblk = a.d.B * a.d.Hv * (a.d.Dv / ChunkFwd<64>::NV);
  switch (a.d.Dk) {
    case 64: chunk_fwd_kernel<64><<<nblk, NT, 0, st>>>(a); break;
    case 128: chunk_fwd_kernel<128><<<nblk, NT, 0, st>>>(a); break;
    case 192: chunk_fwd_kernel<192><<<nblk, NT, 0, st>>>(a); break;
    case 256: chunk_fwd_kernel<256><<<nblk, NT, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
