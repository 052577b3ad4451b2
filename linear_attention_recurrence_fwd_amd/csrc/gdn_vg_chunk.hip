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
//                  passes and the gradient pass read.
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
