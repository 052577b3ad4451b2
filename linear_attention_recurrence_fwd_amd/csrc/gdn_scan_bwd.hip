// Backward sweep of the gated delta rule on gfx950 (mlx-lm VJP PR, "What this
// PR adds" / "Design notes": reverse sweep over each 64-step chunk, recomputed
// from the chunk's checkpoint).
//
// For a valid step t (S' = g S_{t-1}, u = S'^T kn, delta = beta (v - u),
// S_t = S' + kn delta^T, o = S_t^T qn) and D = dL/dS_t accumulated from later
// steps only, the reverse step is
//   ein  = D^T kn                      (read before this step's output term)
//   eps  = ein + (kn . qn) dO          (= dL/d delta)
//   D    = g (D + qn dO^T - beta kn eps^T)   (= dL/dS_{t-1}, later steps only)
// A masked step is l = 0, beta = 0: D += qn dO^T only.
//
// Every quantity above is per column of S, so the sweep runs on column slices
// exactly like the forward scan (Dk reductions = DPP row sums).  Per chunk it
// writes, for the slice's columns:
//   phase 1 (forward recompute from the checkpoint):
//     U  = S'^T kn                           (fp32, per step)
//   phase 2 (reverse):
//     E = ein, dv = beta eps                 (per step)
//   dHend[c] = dL/d(state at the end of chunk c)
// The Dk-vector gradients (dq, dk) and the gate gradients need sums over all
// Dv columns; the chunk-gradient kernel forms them from these outputs.
#include "gdn_dev.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int TS = 16;                 // steps per staged tile
constexpr int TPC = kChunk / TS;       // tiles per full chunk

template <int RI, int NW, typename T>
struct ScanBwd {
  static constexpr int DK = 16 * RI;
  static constexpr int JS = 8 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int EPU = 16 / sizeof(T);
  static constexpr int QK_UNITS = TS * DK / EPU;
  static constexpr int QK_PER_T = (QK_UNITS + NT - 1) / NT;
  static constexpr int C_UNITS = TS * JS / EPU;
  static constexpr int C_PER_T = (C_UNITS + NT - 1) / NT;

  struct Smem {
    float k[TS][DK];
    float q[TS][DK];
    float c[TS][JS];  // v (phase 1) or dO (phase 2)
    float ell[TS], beta[TS], kq[TS];
    float outA[TS][JS], outB[TS][JS];
    float st[DK][JS + 1];
  };

  struct Stage {
    uint4 k[QK_PER_T], q[QK_PER_T], c[C_PER_T];
    float rk[QK_PER_T], rq[QK_PER_T];
    float ell, beta, kq;
  };

  // Job n of the sweep: chunks from last to first; per chunk its tiles in
  // forward order (phase 1), then in reverse order (phase 2).
  __device__ static void job(int n, int nc, int ntl_last, int& c, int& phase, int& tile) {
    int per, m;
    if (n < 2 * ntl_last) {
      c = nc - 1;
      per = ntl_last;
      m = n;
    } else {
      m = n - 2 * ntl_last;
      c = nc - 2 - m / (2 * TPC);
      per = TPC;
      m = m % (2 * TPC);
    }
    if (m < per) {
      phase = 1;
      tile = m;
    } else {
      phase = 2;
      tile = 2 * per - 1 - m;
    }
  }

  __device__ static void load_tile(const ScanBwdArgs& p, int b, int h, int j, int col0, int t0,
                                   int t_end, const void* cin, Stage& s) {
    const Dims& d = p.d;
    const int tid = threadIdx.x;
    const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int n = 0; n < QK_PER_T; ++n) {
      const int u = tid + n * NT;
      const int tt = u / (DK / EPU), e0 = (u % (DK / EPU)) * EPU;
      const int t = t0 + tt;
      s.k[n] = zero;
      s.q[n] = zero;
      s.rk[n] = 0.f;
      s.rq[n] = 0.f;
      if (u < QK_UNITS && t < t_end) {
        const size_t row = (static_cast<size_t>(b) * d.T + t) * d.Hk + j;
        s.k[n] = *reinterpret_cast<const uint4*>(static_cast<const T*>(p.k) + row * DK + e0);
        s.q[n] = *reinterpret_cast<const uint4*>(static_cast<const T*>(p.q) + row * DK + e0);
        s.rk[n] = p.s.rk[row];
        s.rq[n] = p.s.rq[row];
      }
    }
#pragma unroll
    for (int n = 0; n < C_PER_T; ++n) {
      const int u = tid + n * NT;
      const int tt = u / (JS / EPU), e0 = (u % (JS / EPU)) * EPU;
      const int t = t0 + tt;
      s.c[n] = zero;
      if (u < C_UNITS && t < t_end) {
        const size_t row = (static_cast<size_t>(b) * d.T + t) * d.Hv + h;
        s.c[n] = *reinterpret_cast<const uint4*>(static_cast<const T*>(cin) + row * d.Dv + col0 + e0);
      }
    }
    s.ell = 0.f;
    s.beta = 0.f;
    s.kq = 0.f;
    if (tid < TS && t0 + tid < t_end) {
      const size_t bt = static_cast<size_t>(b) * d.T + t0 + tid;
      s.ell = p.s.ell[bt * d.Hv + h];
      s.beta = p.s.beta[bt * d.Hv + h];
      s.kq = p.s.kq[bt * d.Hk + j];
    }
  }

  __device__ static void store_tile(Smem& sm, const Stage& s) {
    const int tid = threadIdx.x;
    float f[EPU];
#pragma unroll
    for (int n = 0; n < QK_PER_T; ++n) {
      const int u = tid + n * NT;
      if (u < QK_UNITS) {
        const int tt = u / (DK / EPU), e0 = (u % (DK / EPU)) * EPU;
        Vec16<T>::unpack(s.k[n], f);
#pragma unroll
        for (int e = 0; e < EPU; ++e) sm.k[tt][e0 + e] = f[e] * s.rk[n];
        Vec16<T>::unpack(s.q[n], f);
#pragma unroll
        for (int e = 0; e < EPU; ++e) sm.q[tt][e0 + e] = f[e] * s.rq[n];
      }
    }
#pragma unroll
    for (int n = 0; n < C_PER_T; ++n) {
      const int u = tid + n * NT;
      if (u < C_UNITS) {
        const int tt = u / (JS / EPU), e0 = (u % (JS / EPU)) * EPU;
        Vec16<T>::unpack(s.c[n], f);
#pragma unroll
        for (int e = 0; e < EPU; ++e) sm.c[tt][e0 + e] = f[e];
      }
    }
    if (tid < TS) {
      sm.ell[tid] = s.ell;
      sm.beta[tid] = s.beta;
      sm.kq[tid] = s.kq;
    }
  }

  __device__ static void state_from_global(Smem& sm, const float* src, int col0, int Dv,
                                           float (&S)[RI][2], int li, int lc) {
    for (int e = threadIdx.x; e < DK * JS; e += NT) {
      const int i = e / JS, c = e % JS;
      sm.st[i][c] = src ? src[static_cast<size_t>(i) * Dv + col0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RI; ++r) {
      S[r][0] = sm.st[li * RI + r][lc];
      S[r][1] = sm.st[li * RI + r][lc + 1];
    }
    __syncthreads();
  }

  __device__ static void state_to_global(Smem& sm, float* dst, int col0, int Dv,
                                         const float (&S)[RI][2], int li, int lc) {
#pragma unroll
    for (int r = 0; r < RI; ++r) {
      sm.st[li * RI + r][lc] = S[r][0];
      sm.st[li * RI + r][lc + 1] = S[r][1];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < DK * JS; e += NT) {
      const int i = e / JS, c = e % JS;
      dst[static_cast<size_t>(i) * Dv + col0 + c] = sm.st[i][c];
    }
    __syncthreads();
  }

  __device__ static void run(const ScanBwdArgs& p, Smem& sm) {
    const Dims& d = p.d;
    const int bh = blockIdx.x, slice = blockIdx.y;
    const int b = bh / d.Hv, h = bh % d.Hv, j = h / d.G();
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int li = lane & 15, jr = lane >> 4;
    const int lc = w * 8 + jr * 2;
    const int col0 = slice * JS;
    const size_t sbase = static_cast<size_t>(bh) * DK * d.Dv;
    const size_t slab = static_cast<size_t>(d.B) * d.Hv * DK * d.Dv;
    const int nc = d.nchunk();

    float D[RI][2], S[RI][2];
    state_from_global(sm, p.dS_final ? p.dS_final + sbase : nullptr, col0, d.Dv, D, li, lc);

    const int ntl_last = nc > 0 ? (d.T - (nc - 1) * kChunk + TS - 1) / TS : 0;
    const int njob = nc > 0 ? 2 * ntl_last + 2 * TPC * (nc - 1) : 0;
    T* dv = static_cast<T*>(p.dv);

    Stage stg;
    auto issue = [&](int n) {
      int c, ph, tile;
      job(n, nc, ntl_last, c, ph, tile);
      const int t0 = c * kChunk + tile * TS;
      const int t_end = min(d.T, (c + 1) * kChunk);
      load_tile(p, b, h, j, col0, t0, t_end, ph == 1 ? p.v : p.dO, stg);
    };
    if (njob > 0) issue(0);

    for (int n = 0; n < njob; ++n) {
      int c, ph, tile;
      job(n, nc, ntl_last, c, ph, tile);
      const int cstart = c * kChunk;
      const int t_end = min(d.T, cstart + kChunk);
      const int t0 = cstart + tile * TS;
      const int nsteps = min(TS, t_end - t0);
      if (ph == 1 && tile == 0) {
        // chunk start: state at the chunk start, and dL/d(state at chunk end)
        const float* H = c == 0 ? (p.state0 ? p.state0 + sbase : nullptr)
                                : p.ckpt + static_cast<size_t>(c - 1) * slab + sbase;
        state_from_global(sm, H, col0, d.Dv, S, li, lc);
        state_to_global(sm, p.dHend + static_cast<size_t>(c) * slab + sbase, col0, d.Dv, D, li, lc);
      }
      store_tile(sm, stg);
      __syncthreads();
      if (n + 1 < njob) issue(n + 1);

      if (ph == 1) {
        for (int tt = 0; tt < nsteps; ++tt) {
          float pu0 = 0.f, pu1 = 0.f;
          float kr[RI];
#pragma unroll
          for (int r = 0; r < RI; ++r) {
            kr[r] = sm.k[tt][li * RI + r];
            pu0 = fmaf(S[r][0], kr[r], pu0);
            pu1 = fmaf(S[r][1], kr[r], pu1);
          }
          pu0 = row_sum16(pu0);
          pu1 = row_sum16(pu1);
          const float g = expf(sm.ell[tt]), beta = sm.beta[tt];
          const float u0 = g * pu0, u1 = g * pu1;
          float d0 = beta * (sm.c[tt][lc] - u0);
          float d1 = beta * (sm.c[tt][lc + 1] - u1);
          if (beta == 0.f) d0 = d1 = 0.f;
#pragma unroll
          for (int r = 0; r < RI; ++r) {
            S[r][0] = fmaf(kr[r], d0, g * S[r][0]);
            S[r][1] = fmaf(kr[r], d1, g * S[r][1]);
          }
          if (li == 0) {
            sm.outA[tt][lc] = u0;
            sm.outA[tt][lc + 1] = u1;
          }
        }
      } else {
        for (int tt = nsteps - 1; tt >= 0; --tt) {
          const float do0 = sm.c[tt][lc], do1 = sm.c[tt][lc + 1];
          float kr[RI], qr[RI];
          float i0 = 0.f, i1 = 0.f;
#pragma unroll
          for (int r = 0; r < RI; ++r) {
            kr[r] = sm.k[tt][li * RI + r];
            qr[r] = sm.q[tt][li * RI + r];
            i0 = fmaf(D[r][0], kr[r], i0);
            i1 = fmaf(D[r][1], kr[r], i1);
          }
          i0 = row_sum16(i0);
          i1 = row_sum16(i1);
          const float g = expf(sm.ell[tt]), beta = sm.beta[tt], kq = sm.kq[tt];
          const float e0 = fmaf(kq, do0, i0), e1 = fmaf(kq, do1, i1);
          const float m0 = -g * beta * e0, m1 = -g * beta * e1;
          const float n0 = g * do0, n1 = g * do1;
#pragma unroll
          for (int r = 0; r < RI; ++r) {
            D[r][0] = fmaf(kr[r], m0, fmaf(qr[r], n0, g * D[r][0]));
            D[r][1] = fmaf(kr[r], m1, fmaf(qr[r], n1, g * D[r][1]));
          }
          if (li == 0) {
            sm.outA[tt][lc] = i0;
            sm.outA[tt][lc + 1] = i1;
            sm.outB[tt][lc] = beta * e0;
            sm.outB[tt][lc + 1] = beta * e1;
          }
        }
      }
      __syncthreads();
      // flush the tile's per-step column outputs
      for (int e = tid; e < nsteps * JS; e += NT) {
        const int tt = e / JS, cc = e % JS;
        const size_t idx = ((static_cast<size_t>(b) * d.T + t0 + tt) * d.Hv + h) * d.Dv + col0 + cc;
        if (ph == 1) {
          p.U[idx] = sm.outA[tt][cc];
        } else {
          p.E[idx] = sm.outA[tt][cc];
          dv[idx] = from_f32<T>(sm.outB[tt][cc]);
        }
      }
      __syncthreads();
    }
    state_to_global(sm, p.dstate + sbase, col0, d.Dv, D, li, lc);
  }
};

template <int RI, int NW, typename T>
__global__ void __launch_bounds__(64 * NW) scan_bwd_kernel(ScanBwdArgs p) {
  using K = ScanBwd<RI, NW, T>;
  __shared__ typename K::Smem sm;
  K::run(p, sm);
}

template <int RI, typename T>
hipError_t launch_nw(const ScanBwdArgs& a, hipStream_t st) {
  dim3 grid(a.d.B * a.d.Hv, scan_nslice(a.d.Dv));
  if (scan_waves(a.d.Dv) == 4)
    scan_bwd_kernel<RI, 4, T><<<grid, 256, 0, st>>>(a);
  else
    scan_bwd_kernel<RI, 1, T><<<grid, 64, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const ScanBwdArgs& a, hipStream_t st) {
  switch (a.d.Dk) {
    case 16: return launch_nw<1, T>(a, st);
    case 32: return launch_nw<2, T>(a, st);
    case 64: return launch_nw<4, T>(a, st);
    case 128: return launch_nw<8, T>(a, st);
    case 192: return launch_nw<12, T>(a, st);
    case 256: return launch_nw<16, T>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan_bwd(const ScanBwdArgs& a, bool bf16, hipStream_t st) {
  if (a.d.B * a.d.Hv == 0) return hipSuccess;
  return bf16 ? launch_t<gdn::bf16>(a, st) : launch_t<float>(a, st);
}

}  // namespace gdn
