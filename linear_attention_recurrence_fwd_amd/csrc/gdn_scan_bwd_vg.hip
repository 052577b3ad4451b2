// Reverse sweep of the gated delta rule with a per-key-channel gate (mlx-lm
// VJP PR, "Models covered": Kimi-Linear's gate holds one value per key
// channel; "Design notes": reverse sweep over each 64-step chunk, recomputed
// from the chunk's checkpoint).
//
// Step t (valid): S' = diag(g) S_{t-1}, u = S'^T kn, X = v - u, delta = beta X,
// S_t = S' + kn delta^T, o = S_t^T qn.  With D = dL/dS_t (later steps and this
// step's own output term qn dO^T) the reverse step is
//   eps  = D^T kn               (= dL/d delta)      dv = beta eps
//   dbeta = eps . X             du = -beta eps
//   dS'  = D + kn du^T          dqn = S_t dO        dkn = D delta + S' du
//   dlg_i = g_i sum_c dS'[i,c] S_{t-1}[i,c]         D <- diag(g) dS'
// A masked step is g = 1, beta = 0 and gets dlg = 0.
//
// The gate gradient is a sum along each row of the state, and so are dqn and
// dkn: the lane layout makes those sums lane-local.  One workgroup per (b, h,
// slice of 8 NW columns); wave w owns 8 columns and lane l the rows l + 64 m
// (m < RM = Dk/64, rows past Dk held as zeros) of them.  The per-step column
// sums (u, eps) are wave reductions, eight columns at a time (wave_sum8).
//
// The reverse walk needs S_{t-1} at every step.  Per chunk:
//   phase 1, forward from the chunk's checkpoint: stores the state every NB
//     steps (a sub-checkpoint, in the workspace) and X per step (in LDS);
//   phase 2, blocks of NB steps from last to first: reloads the block's
//     sub-checkpoint, recomputes its NB states into registers (no reductions:
//     delta comes from X), then walks them in reverse.
// Per block, the row partials of dqn, dkn, dlg of each wave go through LDS,
// are summed over the workgroup's waves and written per column slice; a
// second kernel sums the slices (and the value heads of a key head) in a fixed
// order and applies the normalisation backward.
#include <type_traits>

#include "gdn_dev.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int TS = 16;             // steps per staged tile
constexpr int NB = 4;              // steps per recompute block
constexpr int NSUB = kChunk / NB;  // sub-checkpoints per chunk

// Sum over the 64 lanes of a wave, the same bits in every lane: row sums by
// butterflies, rows 0+1 and 2+3 by a row broadcast, then row 3 gets rows 0-1,
// and lane 63's value is read by all.
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  v += dpp_or0<kRowBcast15, 0xa>(v);
  v += dpp_or0<kRowBcast31, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Eight sums over the 64 lanes of a wave, out[c] = sum of v[c], the same bits
// in every lane (scalars).  A reduce-scatter: v_permlane32_swap exchanges the
// upper lanes of v[c] with the lower lanes of v[c + 4], so that after the add
// lanes 0-31 hold the pair sums of columns 0-3 and lanes 32-63 those of 4-7;
// v_permlane16_swap does the same between odd and even rows of 16 lanes,
// leaving in u[k] column k (row 0), k + 2 (row 1), k + 4 (row 2), k + 6
// (row 3); then two row sums, and each column read from its row.  28
// instructions against 56 for eight separate wave sums.
__device__ __forceinline__ void wave_sum8(const float (&v)[8], float (&out)[8]) {
  float s[4], u[2];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[c]), __float_as_uint(v[c + 4]), false, false);
    s[c] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[k]), __float_as_uint(s[k + 2]), false, false);
    u[k] = row_sum16(__uint_as_float(r[0]) + __uint_as_float(r[1]));
  }
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int row = 0; row < 4; ++row)
      out[k + 2 * row] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u[k]), 16 * row));
}

// Eight wave-uniform values to 8 consecutive LDS floats (16-byte aligned),
// written by lane 0.
__device__ __forceinline__ void put8(float* dst, const float (&x)[8], float s, int lane) {
  if (lane == 0) {
    reinterpret_cast<float4*>(dst)[0] = make_float4(s * x[0], s * x[1], s * x[2], s * x[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(s * x[4], s * x[5], s * x[6], s * x[7]);
  }
}

template <int DK, int NW, typename T>
struct ScanBwdVg {
  static constexpr int RM = DK <= 64 ? 1 : DK / 64;  // rows per lane
  static constexpr int DKP = 64 * RM;                // rows of the lane layout (padded)
  static constexpr int JS = 8 * NW;                  // columns per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int NRB = RM <= 3 ? 2 : 1;        // buffers of the partials
  static constexpr int EPU = 16 / sizeof(T);         // elements per 16-byte unit
  static constexpr int KU = TS * DK / EPU;           // units of k (or q) per tile
  static constexpr int KPT = (KU + NT - 1) / NT;
  static constexpr int LU = TS * DK / 4;             // float4 units of lg per tile
  static constexpr int LPT = (LU + NT - 1) / NT;
  static constexpr int CU = TS * JS / EPU;           // units of v or dO per tile
  static constexpr int CPT = (CU + NT - 1) / NT;

  struct alignas(16) Smem {
    float k[TS][DKP];  // kn; 0 on padded rows
    float q[TS][DKP];  // qn (with 1/sqrt(Dk))
    float g[TS][DKP];  // e^lg; 1 on masked steps and padded rows
    float v[TS][JS];
    float dO[TS][JS];
    float beta[TS], valid[TS];
    alignas(16) float X[kChunk][JS];      // v - u, per step of the chunk
    alignas(16) float red[NRB][NB][3][NW][DKP];  // per-wave row partials: dqn, dkn, dlg
    float rdb[NRB][NB][NW];               // per-wave dbeta
    alignas(16) float dv[TS][JS];
  };

  // One tile's inputs in flight (16-byte loads, all issued before any use).
  struct Stage {
    uint4 k[KPT], q[KPT], c[CPT];
    float rk[KPT], rq[KPT];
    float4 lg[LPT];
    float lv[LPT];  // 1: a valid step inside the tile
    float beta, valid;
  };

  // Loads steps [t0, t0 + n) of the tile: kn, lg always; v (phase 1) or qn
  // and dO (phase 2).  Addresses are clamped into the tensors and values past
  // the tile zeroed by selects, so no load sits behind a branch.
  template <bool PH2>
  __device__ static void load_tile(const ScanBwdVgArgs& p, int b, int h, int j, int col0, int t0,
                                   int n, Stage& s) {
    const Dims& d = p.d;
    const int tid = threadIdx.x;
    const T* kg = static_cast<const T*>(p.k);
    const T* qg = static_cast<const T*>(p.q);
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int u0 = tid + m * NT, u = min(u0, KU - 1);
      const int tt = u / (DK / EPU), e0 = (u % (DK / EPU)) * EPU;
      const size_t row = (static_cast<size_t>(b) * d.T + min(t0 + tt, d.T - 1)) * d.Hk + j;
      const bool ok = u0 < KU && tt < n;
      s.k[m] = *reinterpret_cast<const uint4*>(kg + row * DK + e0);
      s.rk[m] = ok ? p.s.rk[row] : 0.f;
      if constexpr (PH2) {
        s.q[m] = *reinterpret_cast<const uint4*>(qg + row * DK + e0);
        s.rq[m] = ok ? p.s.rq[row] : 0.f;
      }
    }
#pragma unroll
    for (int m = 0; m < LPT; ++m) {
      const int u0 = tid + m * NT, u = min(u0, LU - 1);
      const int tt = u / (DK / 4), e0 = (u % (DK / 4)) * 4;
      const size_t r = static_cast<size_t>(b) * d.T + min(t0 + tt, d.T - 1);
      s.lg[m] = *reinterpret_cast<const float4*>(p.lg + (r * d.Hv + h) * DK + e0);
      const bool mv = p.mask == nullptr || p.mask[r] != 0;
      s.lv[m] = (u0 < LU && tt < n && mv) ? 1.f : 0.f;
    }
    const T* cg = static_cast<const T*>(PH2 ? p.dO : p.v);
    const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int u0 = tid + m * NT, u = min(u0, CU - 1);
      const int tt = u / (JS / EPU), e0 = (u % (JS / EPU)) * EPU;
      const size_t r = (static_cast<size_t>(b) * d.T + min(t0 + tt, d.T - 1)) * d.Hv + h;
      const uint4 x = *reinterpret_cast<const uint4*>(cg + r * d.Dv + col0 + e0);
      s.c[m] = (u0 < CU && tt < n) ? x : zero;
    }
    {
      const int tt = min(tid, TS - 1);
      const size_t r = static_cast<size_t>(b) * d.T + min(t0 + tt, d.T - 1);
      const float bv = p.s.beta[r * d.Hv + h];
      const bool mv = p.mask == nullptr || p.mask[r] != 0;
      s.beta = tt < n ? bv : 0.f;
      s.valid = (tt < n && mv) ? 1.f : 0.f;
    }
  }

  template <bool PH2>
  __device__ static void store_tile(Smem& sm, const Stage& s) {
    const int tid = threadIdx.x;
    float f[EPU];
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int u = tid + m * NT;
      if (u < KU) {
        const int tt = u / (DK / EPU), e0 = (u % (DK / EPU)) * EPU;
        Vec16<T>::unpack(s.k[m], f);
#pragma unroll
        for (int e = 0; e < EPU; ++e) sm.k[tt][e0 + e] = f[e] * s.rk[m];
        if constexpr (PH2) {
          Vec16<T>::unpack(s.q[m], f);
#pragma unroll
          for (int e = 0; e < EPU; ++e) sm.q[tt][e0 + e] = f[e] * s.rq[m];
        }
      }
    }
#pragma unroll
    for (int m = 0; m < LPT; ++m) {
      const int u = tid + m * NT;
      if (u < LU) {
        const int tt = u / (DK / 4), e0 = (u % (DK / 4)) * 4;
        const bool on = s.lv[m] != 0.f;
        sm.g[tt][e0 + 0] = on ? expf(s.lg[m].x) : 1.f;
        sm.g[tt][e0 + 1] = on ? expf(s.lg[m].y) : 1.f;
        sm.g[tt][e0 + 2] = on ? expf(s.lg[m].z) : 1.f;
        sm.g[tt][e0 + 3] = on ? expf(s.lg[m].w) : 1.f;
      }
    }
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int u = tid + m * NT;
      if (u < CU) {
        const int tt = u / (JS / EPU), e0 = (u % (JS / EPU)) * EPU;
        Vec16<T>::unpack(s.c[m], f);
#pragma unroll
        for (int e = 0; e < EPU; ++e) {
          if constexpr (PH2)
            sm.dO[tt][e0 + e] = f[e];
          else
            sm.v[tt][e0 + e] = f[e];
        }
      }
    }
    if (tid < TS) {
      sm.beta[tid] = s.beta;
      sm.valid[tid] = s.valid;
    }
  }

  // [Dk, Dv] fp32 state (this lane's rows and the wave's 8 columns) <-> registers.
  __device__ static void load_state(const float* src, int Dk, int Dv, int col, int lane,
                                    float (&S)[RM][8]) {
#pragma unroll
    for (int m = 0; m < RM; ++m) {
      const int i = lane + 64 * m;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), c = a;
      if (src && i < Dk) {
        const float* r = src + static_cast<size_t>(i) * Dv + col;
        a = *reinterpret_cast<const float4*>(r);
        c = *reinterpret_cast<const float4*>(r + 4);
      }
      S[m][0] = a.x; S[m][1] = a.y; S[m][2] = a.z; S[m][3] = a.w;
      S[m][4] = c.x; S[m][5] = c.y; S[m][6] = c.z; S[m][7] = c.w;
    }
  }
  __device__ static void store_state(float* dst, int Dk, int Dv, int col, int lane,
                                     const float (&S)[RM][8]) {
#pragma unroll
    for (int m = 0; m < RM; ++m) {
      const int i = lane + 64 * m;
      if (i < Dk) {
        float* r = dst + static_cast<size_t>(i) * Dv + col;
        *reinterpret_cast<float4*>(r) = make_float4(S[m][0], S[m][1], S[m][2], S[m][3]);
        *reinterpret_cast<float4*>(r + 4) = make_float4(S[m][4], S[m][5], S[m][6], S[m][7]);
      }
    }
  }
  // Sub-checkpoints: each thread's 8 RM values contiguous.
  __device__ static void put_sub(float* slot, const float (&S)[RM][8]) {
    float4* o = reinterpret_cast<float4*>(slot) + threadIdx.x * (2 * RM);
#pragma unroll
    for (int m = 0; m < RM; ++m) {
      o[2 * m] = make_float4(S[m][0], S[m][1], S[m][2], S[m][3]);
      o[2 * m + 1] = make_float4(S[m][4], S[m][5], S[m][6], S[m][7]);
    }
  }
  __device__ static void get_sub(const float* slot, float (&S)[RM][8]) {
    const float4* o = reinterpret_cast<const float4*>(slot) + threadIdx.x * (2 * RM);
#pragma unroll
    for (int m = 0; m < RM; ++m) {
      const float4 a = o[2 * m], c = o[2 * m + 1];
      S[m][0] = a.x; S[m][1] = a.y; S[m][2] = a.z; S[m][3] = a.w;
      S[m][4] = c.x; S[m][5] = c.y; S[m][6] = c.z; S[m][7] = c.w;
    }
  }

  __device__ static void run(const ScanBwdVgArgs& p, Smem& sm) {
    const Dims& d = p.d;
    const int bh = blockIdx.x, slice = blockIdx.y, nslice = gridDim.y;
    const int b = bh / d.Hv, h = bh % d.Hv, j = h / d.G();
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col0 = slice * JS;    // the workgroup's first column
    const int lcol = w * 8;         // the wave's first local column
    const size_t sbase = static_cast<size_t>(bh) * d.Dk * d.Dv;
    const size_t slab = static_cast<size_t>(d.B) * d.Hv * d.Dk * d.Dv;
    const size_t subsz = static_cast<size_t>(NT) * RM * 8;  // floats per sub-checkpoint
    float* sub = p.sub + (static_cast<size_t>(bh) * nslice + slice) * NSUB * subsz;
    T* dvg = static_cast<T*>(p.dv);

    if constexpr (DK < DKP) {  // padded rows: never staged, kn = qn = 0, g = 1
      for (int e = tid; e < TS * (DKP - DK); e += NT) {
        const int tt = e / (DKP - DK), i = DK + e % (DKP - DK);
        sm.k[tt][i] = 0.f;
        sm.q[tt][i] = 0.f;
        sm.g[tt][i] = 1.f;
      }
    }
    float D[RM][8];
    load_state(p.dS_final ? p.dS_final + sbase : nullptr, d.Dk, d.Dv, col0 + lcol, lane, D);
    int rb = 0;  // partials buffer
    Stage stg;

    for (int c = d.nchunk() - 1; c >= 0; --c) {
      const int c0 = c * kChunk, Lc = min(kChunk, d.T - c0);
      float S[RM][8];
      const float* src = c == 0 ? p.state0 : p.ckpt + static_cast<size_t>(c - 1) * slab;
      load_state(src ? src + sbase : nullptr, d.Dk, d.Dv, col0 + lcol, lane, S);

      // ---- phase 1: forward over the chunk
      for (int t0 = c0; t0 < c0 + Lc; t0 += TS) {
        const int n = min(TS, c0 + Lc - t0);
        load_tile<false>(p, b, h, j, col0, t0, n, stg);
        __syncthreads();
        store_tile<false>(sm, stg);
        __syncthreads();
        for (int tt = 0; tt < n; ++tt) {
          const int tl = t0 + tt - c0;
          if (tl % NB == 0) put_sub(sub + (tl / NB) * subsz, S);
          float km[RM], pu[8];
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) pu[cc] = 0.f;
#pragma unroll
          for (int m = 0; m < RM; ++m) {
            const float gm = sm.g[tt][lane + 64 * m];
            km[m] = sm.k[tt][lane + 64 * m];
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
              S[m][cc] *= gm;
              pu[cc] = fmaf(S[m][cc], km[m], pu[cc]);
            }
          }
          const float beta = sm.beta[tt];
          float X[8], su[8];
          wave_sum8(pu, su);
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            X[cc] = sm.v[tt][lcol + cc] - su[cc];
            const float dl = beta * X[cc];
#pragma unroll
            for (int m = 0; m < RM; ++m) S[m][cc] = fmaf(km[m], dl, S[m][cc]);
          }
          put8(&sm.X[tl][lcol], X, 1.f, lane);
        }
      }
      wave_lds_sync();  // X: each wave reads back only its own columns
      float Pf[RM][8];  // the next block's sub-checkpoint, loaded a block ahead
      get_sub(sub + ((Lc - 1) / NB) * subsz, Pf);

      // ---- phase 2: blocks of NB steps, last to first
      const int ntile = (Lc + TS - 1) / TS;
      for (int it = ntile - 1; it >= 0; --it) {
        const int t0 = c0 + it * TS, n = min(TS, c0 + Lc - t0);
        load_tile<true>(p, b, h, j, col0, t0, n, stg);
        __syncthreads();
        store_tile<true>(sm, stg);
        __syncthreads();
        const int nblk = (n + NB - 1) / NB;
        for (int bl = nblk - 1; bl >= 0; --bl) {
          const int tb = bl * NB, nb = min(NB, n - tb);  // tile-local first step, steps
          const int tl0 = t0 + tb - c0;                   // chunk-local first step
          auto walk = [&](auto full) {
          constexpr bool FULL = decltype(full)::value;
          float St[NB][RM][8];
#pragma unroll
          for (int m = 0; m < RM; ++m)
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) S[m][cc] = Pf[m][cc];
          if (tl0 >= NB) get_sub(sub + (tl0 / NB - 1) * subsz, Pf);
#pragma unroll
          for (int jj = 0; jj < NB; ++jj) {
            if (FULL || jj < nb) {
              const int tt = tb + jj;
              const float beta = sm.beta[tt];
#pragma unroll
              for (int m = 0; m < RM; ++m) {
                const float gm = sm.g[tt][lane + 64 * m], km = sm.k[tt][lane + 64 * m];
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                  St[jj][m][cc] = S[m][cc];
                  S[m][cc] = fmaf(km, beta * sm.X[tl0 + jj][lcol + cc], gm * S[m][cc]);
                }
              }
            }
          }
#pragma unroll
          for (int jj = NB - 1; jj >= 0; --jj) {
            if (FULL || jj < nb) {
              const int tt = tb + jj;
              const float beta = sm.beta[tt], valid = sm.valid[tt];
              float X[8], dOc[8], del[8];
#pragma unroll
              for (int cc = 0; cc < 8; ++cc) {
                X[cc] = sm.X[tl0 + jj][lcol + cc];
                dOc[cc] = sm.dO[tt][lcol + cc];
                del[cc] = beta * X[cc];
              }
              float km[RM], gm[RM], dq[RM], pe[8];
#pragma unroll
              for (int cc = 0; cc < 8; ++cc) pe[cc] = 0.f;
#pragma unroll
              for (int m = 0; m < RM; ++m) {
                km[m] = sm.k[tt][lane + 64 * m];
                gm[m] = sm.g[tt][lane + 64 * m];
                const float qm = sm.q[tt][lane + 64 * m];
                dq[m] = 0.f;
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                  const float st = fmaf(km[m], del[cc], gm[m] * St[jj][m][cc]);  // S_t
                  D[m][cc] = fmaf(qm, dOc[cc], D[m][cc]);
                  dq[m] = fmaf(st, dOc[cc], dq[m]);
                  pe[cc] = fmaf(D[m][cc], km[m], pe[cc]);
                }
              }
              float eps[8], du[8], db = 0.f;
              wave_sum8(pe, eps);
#pragma unroll
              for (int cc = 0; cc < 8; ++cc) {
                db = fmaf(eps[cc], X[cc], db);
                du[cc] = -beta * eps[cc];
              }
#pragma unroll
              for (int m = 0; m < RM; ++m) {
                float dk = 0.f, dl = 0.f;
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                  const float sp = gm[m] * St[jj][m][cc];  // S'
                  const float dsp = fmaf(km[m], du[cc], D[m][cc]);
                  dk = fmaf(D[m][cc], del[cc], fmaf(sp, du[cc], dk));
                  dl = fmaf(dsp, St[jj][m][cc], dl);
                  D[m][cc] = gm[m] * dsp;
                }
                const int i = lane + 64 * m;
                sm.red[rb][jj][0][w][i] = dq[m];
                sm.red[rb][jj][1][w][i] = dk;
                sm.red[rb][jj][2][w][i] = valid != 0.f ? gm[m] * dl : 0.f;
              }
              if (lane == 0) sm.rdb[rb][jj][w] = db;
              put8(&sm.dv[tt][lcol], eps, beta, lane);
            }
          }
          };
          if (nb == NB)
            walk(std::true_type{});
          else
            walk(std::false_type{});
          __syncthreads();
          // sums over the waves (in order) -> per-slice partials of the block's
          // steps, 4 rows per thread and item
          const int t_abs = t0 + tb;
          constexpr int Q4 = 3 * DK / 4;
          const size_t o0 = ((static_cast<size_t>(b) * d.T + t_abs) * d.Hv + h) * nslice + slice;
          const size_t ostep = static_cast<size_t>(d.Hv) * nslice * 3 * DK;
          for (int e = tid; e < nb * Q4; e += NT) {
            const int jj = e / Q4, r4 = e - jj * Q4, qq = r4 / (DK / 4), i = (r4 - qq * (DK / 4)) * 4;
            float4 a = *reinterpret_cast<const float4*>(&sm.red[rb][jj][qq][0][i]);
#pragma unroll
            for (int ww = 1; ww < NW; ++ww) {
              const float4 x = *reinterpret_cast<const float4*>(&sm.red[rb][jj][qq][ww][i]);
              a.x += x.x;
              a.y += x.y;
              a.z += x.z;
              a.w += x.w;
            }
            *reinterpret_cast<float4*>(p.part + o0 * 3 * DK + jj * ostep + qq * DK + i) = a;
          }
          if (tid < nb) {
            float s = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) s += sm.rdb[rb][tid][ww];
            p.pdb[((static_cast<size_t>(b) * d.T + t_abs + tid) * d.Hv + h) * nslice + slice] = s;
          }
          if constexpr (NRB == 1)
            __syncthreads();  // partials read before the next block writes them
          else
            rb ^= 1;
        }
        // dv of the tile (every block's writes precede its barrier)
        for (int e = tid; e < n * JS; e += NT) {
          const int tt = e / JS, cc = e % JS;
          const size_t r = (static_cast<size_t>(b) * d.T + t0 + tt) * d.Hv + h;
          dvg[r * d.Dv + col0 + cc] = from_f32<T>(sm.dv[tt][cc]);
        }
      }
    }
    store_state(p.dstate + sbase, d.Dk, d.Dv, col0 + lcol, lane, D);
  }
};

template <int DK, int NW, typename T>
__global__ void __launch_bounds__(64 * NW) scan_bwd_vg_kernel(ScanBwdVgArgs p) {
  using K = ScanBwdVg<DK, NW, T>;
  __shared__ typename K::Smem sm;
  K::run(p, sm);
}

// Sums of the per-slice partials: dqn, dkn over the slices and the G value
// heads of the key head (head, then slice, ascending), the L2-normalisation
// backward (dq = rq (dqn - q^ (q^ . dqn)), q^ = q rq sqrt(Dk); dk = rk (dkn -
// kn (kn . dkn))), dlg over the slices, db = beta (1 - beta) sum dbeta.  One
// wave per (b, t, key head); lane l holds rows l + 64 m.
template <int RM, typename T>
__global__ void __launch_bounds__(64) vg_reduce_kernel(VgReduceArgs p) {
  const Dims& d = p.d;
  const int G = d.G(), ns = p.nslice;
  const int bt = blockIdx.x / d.Hk, j = blockIdx.x % d.Hk;
  const int lane = threadIdx.x;
  const size_t qrow = static_cast<size_t>(bt) * d.Hk + j;
  float dqn[RM], dkn[RM];
#pragma unroll
  for (int m = 0; m < RM; ++m) dqn[m] = dkn[m] = 0.f;
  for (int hh = 0; hh < G; ++hh) {
    const int h = j * G + hh;
    const size_t hb = (static_cast<size_t>(bt) * d.Hv + h) * ns;
    float dl[RM];
#pragma unroll
    for (int m = 0; m < RM; ++m) dl[m] = 0.f;
    float dbs = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float* pp = p.part + (hb + s) * 3 * d.Dk;
#pragma unroll
      for (int m = 0; m < RM; ++m) {
        const int i = lane + 64 * m;
        if (i < d.Dk) {
          dqn[m] += pp[i];
          dkn[m] += pp[d.Dk + i];
          dl[m] += pp[2 * d.Dk + i];
        }
      }
      dbs += p.pdb[hb + s];
    }
#pragma unroll
    for (int m = 0; m < RM; ++m) {
      const int i = lane + 64 * m;
      if (i < d.Dk) p.dlg[(static_cast<size_t>(bt) * d.Hv + h) * d.Dk + i] = dl[m];
    }
    if (lane == 0) {
      const float beta = p.s.beta[static_cast<size_t>(bt) * d.Hv + h];
      static_cast<T*>(p.db)[static_cast<size_t>(bt) * d.Hv + h] = from_f32<T>(dbs * beta * (1.f - beta));
    }
  }
  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const float rq = p.s.rq[qrow], rk = p.s.rk[qrow];
  const float qs = rq * sqrtf(static_cast<float>(d.Dk));  // q^ = q qs
  float qh[RM], kn[RM], pq = 0.f, pk = 0.f;
#pragma unroll
  for (int m = 0; m < RM; ++m) {
    const int i = lane + 64 * m;
    qh[m] = i < d.Dk ? to_f32(qg[qrow * d.Dk + i]) * qs : 0.f;
    kn[m] = i < d.Dk ? to_f32(kg[qrow * d.Dk + i]) * rk : 0.f;
    pq = fmaf(qh[m], dqn[m], pq);
    pk = fmaf(kn[m], dkn[m], pk);
  }
  pq = wave_sum(pq);
  pk = wave_sum(pk);
#pragma unroll
  for (int m = 0; m < RM; ++m) {
    const int i = lane + 64 * m;
    if (i < d.Dk) {
      static_cast<T*>(p.dq)[qrow * d.Dk + i] = from_f32<T>(rq * (dqn[m] - qh[m] * pq));
      static_cast<T*>(p.dk)[qrow * d.Dk + i] = from_f32<T>(rk * (dkn[m] - kn[m] * pk));
    }
  }
}

template <int DK, typename T>
hipError_t launch_dk(const ScanBwdVgArgs& a, hipStream_t st) {
  dim3 grid(a.d.B * a.d.Hv, vg_nslice(a.d.Dv));
  if (scan_waves(a.d.Dv) == 4)
    scan_bwd_vg_kernel<DK, 4, T><<<grid, 256, 0, st>>>(a);
  else
    scan_bwd_vg_kernel<DK, 1, T><<<grid, 64, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const ScanBwdVgArgs& a, hipStream_t st) {
  switch (a.d.Dk) {
    case 16: return launch_dk<16, T>(a, st);
    case 32: return launch_dk<32, T>(a, st);
    case 64: return launch_dk<64, T>(a, st);
    case 128: return launch_dk<128, T>(a, st);
    case 192: return launch_dk<192, T>(a, st);
    case 256: return launch_dk<256, T>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_reduce_t(const VgReduceArgs& a, hipStream_t st) {
  const int n = a.d.B * a.d.T * a.d.Hk;
  switch (vg_rows(a.d.Dk)) {
    case 1: vg_reduce_kernel<1, T><<<n, 64, 0, st>>>(a); break;
    case 2: vg_reduce_kernel<2, T><<<n, 64, 0, st>>>(a); break;
    case 3: vg_reduce_kernel<3, T><<<n, 64, 0, st>>>(a); break;
    case 4: vg_reduce_kernel<4, T><<<n, 64, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_bwd_vg(const ScanBwdVgArgs& a, bool bf16, hipStream_t st) {
  if (a.d.B * a.d.Hv == 0) return hipSuccess;
  return bf16 ? launch_t<gdn::bf16>(a, st) : launch_t<float>(a, st);
}

hipError_t launch_vg_reduce(const VgReduceArgs& a, bool bf16, hipStream_t st) {
  if (a.d.B * a.d.T * a.d.Hk == 0) return hipSuccess;
  return bf16 ? launch_reduce_t<gdn::bf16>(a, st) : launch_reduce_t<float>(a, st);
}

}  // namespace gdn
