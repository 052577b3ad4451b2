// Per-step scalars of the gated delta rule: q/k normalisation factors and the
// gates (torch-to-nnef GDN page, "Op contract": q/k L2-normalised with eps
// 1e-6, q scaled by 1/sqrt(width); mlx-lm VJP PR: g = exp(-exp(A_log) *
// softplus(a + dt_bias)) with the softplus argument clamped, beta = sigmoid(b)).
// A masked step is stored as l = 0 (g = 1) and beta = 0, which leaves the state
// unchanged and still reads o from it.  With a per-key-channel gate (a null)
// only the norms and beta are produced.
#include "gdn_dev.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <typename T>
__global__ void __launch_bounds__(256) prep_kernel(PrepArgs p) {
  const Dims d = p.d;
  const int bt = blockIdx.x;  // b * T + t
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const T* q = static_cast<const T*>(p.q);
  const T* k = static_cast<const T*>(p.k);
  const float scale = 1.0f / sqrtf(static_cast<float>(d.Dk));
  for (int j = w; j < d.Hk; j += 4) {
    const size_t base = (static_cast<size_t>(bt) * d.Hk + j) * d.Dk;
    float sq = 0.f, sk = 0.f, sqk = 0.f;
    for (int i = lane; i < d.Dk; i += 64) {
      float qi = to_f32(q[base + i]), ki = to_f32(k[base + i]);
      sq += qi * qi;
      sk += ki * ki;
      sqk += qi * ki;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      sq += __shfl_xor(sq, m);
      sk += __shfl_xor(sk, m);
      sqk += __shfl_xor(sqk, m);
    }
    if (lane == 0) {
      const float rq = scale / sqrtf(sq + kNormEps);
      const float rk = 1.0f / sqrtf(sk + kNormEps);
      const size_t o = static_cast<size_t>(bt) * d.Hk + j;
      p.s.rq[o] = rq;
      p.s.rk[o] = rk;
      p.s.kq[o] = sqk * rq * rk;
    }
  }
  const T* a = static_cast<const T*>(p.a);
  const T* b = static_cast<const T*>(p.b);
  const bool valid = p.mask == nullptr || p.mask[bt] != 0;
  for (int h = threadIdx.x; h < d.Hv; h += blockDim.x) {
    const size_t o = static_cast<size_t>(bt) * d.Hv + h;
    float ell = 0.f, beta = 0.f;
    if (valid) {
      if (a) {
        const float x = to_f32(a[o]) + p.dt_bias[h];
        const float xc = fminf(x, kClamp);
        ell = -expf(p.A_log[h]) * softplus_f(xc);
      }
      beta = sigmoid_f(to_f32(b[o]));
    }
    if (p.s.ell) p.s.ell[o] = ell;
    p.s.beta[o] = beta;
  }
}

}  // namespace

hipError_t launch_prep(const PrepArgs& a, bool bf16, hipStream_t st) {
  const int nblk = a.d.B * a.d.T;
  if (nblk == 0) return hipSuccess;
  if (bf16)
    prep_kernel<gdn::bf16><<<nblk, 256, 0, st>>>(a);
  else
    prep_kernel<float><<<nblk, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace gdn
