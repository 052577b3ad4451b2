// Forward scan of the gated delta rule on gfx950 (sequential in T).
//
// Step (mlx-lm VJP PR, "What this PR adds"; torch-to-nnef GDN "Op contract"):
//   S' = g S;  u = S'^T kn;  delta = beta (v - u);  S = S' + kn delta^T;
//   o = S^T qn.
// Both Dk reductions read the state before the update:
//   p = S^T qn, u = g (S^T kn), o = g p + (kn . qn) delta,
// so one pass over S produces both and the update follows.
//
// Mapping: one workgroup per (b, h, column slice).  Each wave owns 8 columns;
// lane l holds rows i = (l & 15) * RI + r (r < RI, Dk = 16 RI) of columns
// 2 (l >> 4) + {0, 1}.  A Dk reduction is a sum over the 16 lanes of a DPP
// row, done with four DPP adds (no LDS, no barrier in the step).  Columns are
// independent in the recurrence, so slices never communicate.
//
// Per tile of TS steps, q/k rows of the key head, the v slice and the step
// scalars are staged in LDS; the next tile's global loads are issued before
// the current tile is computed (register prefetch), so their latency hides
// behind the scan.  States go to/from global memory through an LDS transpose
// so every global access is row-contiguous.
//
// Per-key-channel gate (mlx-lm VJP PR, "Models covered": Kimi-Linear's gate
// has one value per key channel): the rows of S are scaled by g_i = e^{lg_i}
// instead of one scalar; the lane multiplies its rows' kn, qn by g_i before
// the two reads and its rows of S by g_i in the update.
#include "gdn_dev.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int TS = 16;  // steps per staged tile (divides the checkpoint period)

template <int RI, int NW, typename T, bool VG>
struct ScanFwd {
  static constexpr int DK = 16 * RI;
  static constexpr int JS = 8 * NW;   // columns per workgroup
  static constexpr int NT = 64 * NW;  // threads
  static constexpr int EPU = 16 / sizeof(T);          // elements per 16-byte unit
  static constexpr int QK_UNITS = TS * DK / EPU;      // per array per tile
  static constexpr int QK_PER_T = (QK_UNITS + NT - 1) / NT;
  static constexpr int V_UNITS = TS * JS / EPU;
  static constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
  static constexpr int LG_UNITS = VG ? TS * DK / 4 : 0;   // fp32 log-gates, 4 per unit
  static constexpr int LG_PER_T = VG ? (LG_UNITS + NT - 1) / NT : 1;

  struct Smem {
    float k[2][TS][DK];
    float q[2][TS][DK];
    float v[2][TS][JS];
    float gs[2][TS], beta[2][TS], kq[2][TS];  // gs: the scalar gate e^l
    float g[VG ? 2 : 1][TS][VG ? DK : 1];  // per-channel gates e^lg (1 on masked steps)
    float o[TS][JS];
    float st[DK][JS + 1];
  };

  // Registers holding one tile in flight.
  struct Stage {
    uint4 k[QK_PER_T], q[QK_PER_T], v[V_PER_T];
    float rk[QK_PER_T], rq[QK_PER_T];
    float ell, beta, kq;
    float4 lg[LG_PER_T];
  };

  __device__ static void load_tile(const ScanFwdArgs& p, int b, int h, int j, int col0,
                                   int t0, Stage& s) {
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
      if (u < QK_UNITS && t < d.T) {
        const size_t row = (static_cast<size_t>(b) * d.T + t) * d.Hk + j;
        s.k[n] = *reinterpret_cast<const uint4*>(static_cast<const T*>(p.k) + row * DK + e0);
        s.q[n] = *reinterpret_cast<const uint4*>(static_cast<const T*>(p.q) + row * DK + e0);
        s.rk[n] = p.s.rk[row];
        s.rq[n] = p.s.rq[row];
      }
    }
#pragma unroll
    for (int n = 0; n < V_PER_T; ++n) {
      const int u = tid + n * NT;
      const int tt = u / (JS / EPU), e0 = (u % (JS / EPU)) * EPU;
      const int t = t0 + tt;
      s.v[n] = zero;
      if (u < V_UNITS && t < d.T) {
        const size_t row = (static_cast<size_t>(b) * d.T + t) * d.Hv + h;
        s.v[n] = *reinterpret_cast<const uint4*>(static_cast<const T*>(p.v) + row * d.Dv + col0 + e0);
      }
    }
    if constexpr (VG) {
#pragma unroll
      for (int n = 0; n < LG_PER_T; ++n) {
        const int u = tid + n * NT;
        const int tt = u / (DK / 4), e0 = (u % (DK / 4)) * 4;
        const int t = t0 + tt;
        s.lg[n] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (u < LG_UNITS && t < d.T) {
          const size_t r = static_cast<size_t>(b) * d.T + t;
          if (p.mask == nullptr || p.mask[r] != 0)
            s.lg[n] = *reinterpret_cast<const float4*>(p.lg + (r * d.Hv + h) * DK + e0);
        }
      }
    }
    s.ell = 0.f;
    s.beta = 0.f;
    s.kq = 0.f;
    if (tid < TS && t0 + tid < d.T) {
      const size_t r = static_cast<size_t>(b) * d.T + t0 + tid;
      if constexpr (!VG) s.ell = p.s.ell[r * d.Hv + h];
      s.beta = p.s.beta[r * d.Hv + h];
      s.kq = p.s.kq[r * d.Hk + j];
    }
  }

  __device__ static void store_tile(Smem& sm, int buf, const Stage& s) {
    const int tid = threadIdx.x;
    float f[EPU];
#pragma unroll
    for (int n = 0; n < QK_PER_T; ++n) {
      const int u = tid + n * NT;
      if (u < QK_UNITS) {
        const int tt = u / (DK / EPU), e0 = (u % (DK / EPU)) * EPU;
        Vec16<T>::unpack(s.k[n], f);
#pragma unroll
        for (int e = 0; e < EPU; ++e) sm.k[buf][tt][e0 + e] = f[e] * s.rk[n];
        Vec16<T>::unpack(s.q[n], f);
#pragma unroll
        for (int e = 0; e < EPU; ++e) sm.q[buf][tt][e0 + e] = f[e] * s.rq[n];
      }
    }
#pragma unroll
    for (int n = 0; n < V_PER_T; ++n) {
      const int u = tid + n * NT;
      if (u < V_UNITS) {
        const int tt = u / (JS / EPU), e0 = (u % (JS / EPU)) * EPU;
        Vec16<T>::unpack(s.v[n], f);
#pragma unroll
        for (int e = 0; e < EPU; ++e) sm.v[buf][tt][e0 + e] = f[e];
      }
    }
    if (tid < TS) {
      sm.gs[buf][tid] = expf(s.ell);
      sm.beta[buf][tid] = s.beta;
      sm.kq[buf][tid] = s.kq;
    }
    if constexpr (VG) {
#pragma unroll
      for (int n = 0; n < LG_PER_T; ++n) {
        const int u = tid + n * NT;
        if (u < LG_UNITS) {
          const int tt = u / (DK / 4), e0 = (u % (DK / 4)) * 4;
          sm.g[buf][tt][e0 + 0] = expf(s.lg[n].x);
          sm.g[buf][tt][e0 + 1] = expf(s.lg[n].y);
          sm.g[buf][tt][e0 + 2] = expf(s.lg[n].z);
          sm.g[buf][tt][e0 + 3] = expf(s.lg[n].w);
        }
      }
    }
  }

  // One step's operands from the staged tile.
  struct Ops {
    float kr[RI], qr[RI], gr[RI];  // gr: per-channel gates (unused for the scalar gate)
    float v0, v1, g, beta, kq;
  };
  __device__ static void load_ops(const Smem& sm, int buf, int tt, int li, int lc, Ops& o) {
#pragma unroll
    for (int r = 0; r < RI; ++r) {
      o.kr[r] = sm.k[buf][tt][li * RI + r];
      o.qr[r] = sm.q[buf][tt][li * RI + r];
      if constexpr (VG) o.gr[r] = sm.g[buf][tt][li * RI + r];
    }
    o.v0 = sm.v[buf][tt][lc];
    o.v1 = sm.v[buf][tt][lc + 1];
    o.g = sm.gs[buf][tt];
    o.beta = sm.beta[buf][tt];
    o.kq = sm.kq[buf][tt];
  }

  // Global [Dk, Dv] state (slice columns) <-> registers, via sm.st.
  __device__ static void state_from_global(Smem& sm, const float* src, int col0,
                                           int Dv, float (&S)[RI][2], int li, int lc) {
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

  __device__ static void run(const ScanFwdArgs& p, Smem& sm) {
    const Dims& d = p.d;
    const int bh = blockIdx.x, slice = blockIdx.y;
    const int b = bh / d.Hv, h = bh % d.Hv, j = h / d.G();
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int li = lane & 15, jr = lane >> 4;
    const int lc = w * 8 + jr * 2;  // first local column of this lane
    const int col0 = slice * JS;
    const size_t sbase = static_cast<size_t>(bh) * DK * d.Dv;
    const size_t slab = static_cast<size_t>(d.B) * d.Hv * DK * d.Dv;

    float S[RI][2];
    state_from_global(sm, p.state0 ? p.state0 + sbase : nullptr, col0, d.Dv, S, li, lc);

    const int ntile = (d.T + TS - 1) / TS;
    Stage stg;
    if (ntile > 0) {
      load_tile(p, b, h, j, col0, 0, stg);
      store_tile(sm, 0, stg);
    }
    __syncthreads();

    T* o = static_cast<T*>(p.o);
    for (int it = 0; it < ntile; ++it) {
      const int buf = it & 1, t0 = it * TS;
      if (it + 1 < ntile) load_tile(p, b, h, j, col0, t0 + TS, stg);
      const int nsteps = min(TS, d.T - t0);
      // A step's LDS operands are read one step ahead (their latency hides
      // behind the previous step); the read past the tile's last step is of a
      // row of the same buffer and is not used.
      Ops nx;
      load_ops(sm, buf, 0, li, lc, nx);
      for (int tt = 0; tt < nsteps; ++tt) {
        const Ops cu = nx;
        load_ops(sm, buf, min(tt + 1, TS - 1), li, lc, nx);
        const float(&kr)[RI] = cu.kr;
        const float(&qr)[RI] = cu.qr;
        const float(&gr)[RI] = cu.gr;
        // Per-channel gate: both reads see the decayed rows, u = S^T (g o kn),
        // p = S^T (g o qn), and o = p + (kn . qn) delta.
        float pu0 = 0.f, pu1 = 0.f, pp0 = 0.f, pp1 = 0.f;
#pragma unroll
        for (int r = 0; r < RI; ++r) {
          const float kg = VG ? kr[r] * gr[r] : kr[r];
          const float qg = VG ? qr[r] * gr[r] : qr[r];
          pu0 = fmaf(S[r][0], kg, pu0);
          pu1 = fmaf(S[r][1], kg, pu1);
          pp0 = fmaf(S[r][0], qg, pp0);
          pp1 = fmaf(S[r][1], qg, pp1);
        }
        pu0 = row_sum16(pu0);
        pu1 = row_sum16(pu1);
        pp0 = row_sum16(pp0);
        pp1 = row_sum16(pp1);
        const float g = VG ? 1.f : cu.g;
        const float beta = cu.beta, kq = cu.kq;
        float d0 = beta * (cu.v0 - g * pu0);
        float d1 = beta * (cu.v1 - g * pu1);
        if (beta == 0.f) d0 = d1 = 0.f;  // masked step: v is not read
#pragma unroll
        for (int r = 0; r < RI; ++r) {
          const float gg = VG ? gr[r] : g;
          S[r][0] = fmaf(kr[r], d0, gg * S[r][0]);
          S[r][1] = fmaf(kr[r], d1, gg * S[r][1]);
        }
        if (li == 0) {
          sm.o[tt][lc] = fmaf(kq, d0, g * pp0);
          sm.o[tt][lc + 1] = fmaf(kq, d1, g * pp1);
        }
      }
      __syncthreads();  // o tile complete; tile `buf` no longer read
      for (int e = tid; e < nsteps * JS; e += NT) {
        const int tt = e / JS, c = e % JS;
        const size_t row = (static_cast<size_t>(b) * d.T + t0 + tt) * d.Hv + h;
        o[row * d.Dv + col0 + c] = from_f32<T>(sm.o[tt][c]);
      }
      if (it + 1 < ntile) store_tile(sm, buf ^ 1, stg);
      const int done = t0 + nsteps;
      if (p.ckpt && done % kChunk == 0 && done < d.T)
        state_to_global(sm, p.ckpt + static_cast<size_t>(done / kChunk - 1) * slab + sbase,
                        col0, d.Dv, S, li, lc);
      __syncthreads();
    }
    state_to_global(sm, p.state_out + sbase, col0, d.Dv, S, li, lc);
  }
};

template <int RI, int NW, typename T, bool VG>
__global__ void __launch_bounds__(64 * NW) scan_fwd_kernel(ScanFwdArgs p) {
  using K = ScanFwd<RI, NW, T, VG>;
  __shared__ typename K::Smem sm;
  K::run(p, sm);
}

template <int RI, typename T>
hipError_t launch_nw(const ScanFwdArgs& a, hipStream_t st) {
  const int nw = scan_waves(a.d.Dv);
  dim3 grid(a.d.B * a.d.Hv, scan_nslice(a.d.Dv));
  if (a.lg) {
    if (nw == 4)
      scan_fwd_kernel<RI, 4, T, true><<<grid, 256, 0, st>>>(a);
    else
      scan_fwd_kernel<RI, 1, T, true><<<grid, 64, 0, st>>>(a);
  } else {
    if (nw == 4)
      scan_fwd_kernel<RI, 4, T, false><<<grid, 256, 0, st>>>(a);
    else
      scan_fwd_kernel<RI, 1, T, false><<<grid, 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const ScanFwdArgs& a, hipStream_t st) {
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

hipError_t launch_scan_fwd(const ScanFwdArgs& a, bool bf16, hipStream_t st) {
  if (a.d.B * a.d.Hv == 0) return hipSuccess;
  return bf16 ? launch_t<gdn::bf16>(a, st) : launch_t<float>(a, st);
}

}  // namespace gdn
