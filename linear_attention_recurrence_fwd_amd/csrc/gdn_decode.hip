// Single-step forward of the gated delta rule (decode: one token per
// sequence and call), fused: the q/k normalisation and the gates (torch-to-
// nnef GDN page, "Op contract"; mlx-lm VJP PR, "What this PR adds") and the
// state update in one kernel that reads and writes the state once.
//
//   S' = g S;  u = S'^T kn;  delta = beta (v - u);  S = S' + kn delta^T;  o = S^T qn
//
// with a masked step leaving S unchanged (g = 1, beta = 0) and still reading o
// from it.  The state is the whole traffic of a call (Dk x Dv fp32 per head,
// read and written), so the kernel is a stream over it:
//   one workgroup per (batch, value head), one wave per 32-column slice of
//   Dv; lane l = 8 rg + cq holds rows rg Dk/8 .. + Dk/8 - 1 of columns
//   32 w + 4 cq .. + 3 in registers (16-byte loads and stores, 128
//   contiguous bytes per row per 8 lanes).  The two column sums over Dk
//   (u and o) add the lane's rows, then the 8 row groups across lanes
//   (lane xor 8, 16, 32).
#include "gdn_dev.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <typename T, int DK>
__global__ void __launch_bounds__(512) decode_kernel(DecodeArgs p) {
  constexpr int RL = DK / 8;  // state rows per lane
  const Dims& d = p.d;
  const int bh = blockIdx.x, b = bh / d.Hv, h = bh % d.Hv, j = h / d.G();
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, rg = l >> 3, cq = l & 7;
  const int col = 32 * w + 4 * cq;
  const T* qr = static_cast<const T*>(p.q) + (static_cast<size_t>(b) * d.Hk + j) * DK;
  const T* kr = static_cast<const T*>(p.k) + (static_cast<size_t>(b) * d.Hk + j) * DK;

  // |q|^2, |k|^2 over the wave
  float sq = 0.f, sk = 0.f;
  for (int i = l; i < DK; i += 64) {
    const float qi = to_f32(qr[i]), ki = to_f32(kr[i]);
    sq += qi * qi;
    sk += ki * ki;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    sq += __shfl_xor(sq, m);
    sk += __shfl_xor(sk, m);
  }
  const float rq = (1.0f / sqrtf(static_cast<float>(DK))) / sqrtf(sq + kNormEps);
  const float rk = 1.0f / sqrtf(sk + kNormEps);

  // gates: l = -e^{A_log} softplus(min(a + dt_bias, 20)), beta = sigmoid(b);
  // a masked step gets l = 0, beta = 0
  const size_t ab = static_cast<size_t>(b) * d.Hv + h;
  float ell = 0.f, beta = 0.f;
  if (p.mask == nullptr || p.mask[b] != 0) {
    const float x = to_f32(static_cast<const T*>(p.a)[ab]) + p.dt_bias[h];
    ell = -expf(p.A_log[h]) * softplus_f(fminf(x, kClamp));
    beta = sigmoid_f(to_f32(static_cast<const T*>(p.b)[ab]));
  }
  const float g = expf(ell);

  float kn[RL], qn[RL];
#pragma unroll
  for (int r = 0; r < RL; ++r) {
    kn[r] = to_f32(kr[rg * RL + r]) * rk;
    qn[r] = to_f32(qr[rg * RL + r]) * rq;
  }
  // the state slice of this lane, by unconditional buffer loads; an absent
  // initial state reads through an empty descriptor, i.e. as zeros (loads
  // under a branch would wait one by one)
  const size_t sb = static_cast<size_t>(bh) * DK * d.Dv + static_cast<size_t>(rg * RL) * d.Dv + col;
  const size_t hs = static_cast<size_t>(bh) * DK * d.Dv;
  const rsrc_t rs0 = make_rsrc(p.state0 ? static_cast<const void*>(p.state0 + hs) : static_cast<const void*>(p.state_out),
                               p.state0 ? static_cast<size_t>(DK) * d.Dv * 4 : 0);
  float4 s[RL];
#pragma unroll
  for (int r = 0; r < RL; ++r) s[r] = buf_f4(rs0, 4 * static_cast<uint32_t>((rg * RL + r) * d.Dv + col));
  // S' = g S, u = S'^T kn
  float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int r = 0; r < RL; ++r) {
    s[r].x *= g; s[r].y *= g; s[r].z *= g; s[r].w *= g;
    u.x = fmaf(kn[r], s[r].x, u.x);
    u.y = fmaf(kn[r], s[r].y, u.y);
    u.z = fmaf(kn[r], s[r].z, u.z);
    u.w = fmaf(kn[r], s[r].w, u.w);
  }
#pragma unroll
  for (int m = 8; m <= 32; m <<= 1) {
    u.x += __shfl_xor(u.x, m);
    u.y += __shfl_xor(u.y, m);
    u.z += __shfl_xor(u.z, m);
    u.w += __shfl_xor(u.w, m);
  }
  // delta = beta (v - u);  S = S' + kn delta^T;  o = S^T qn
  const T* vr = static_cast<const T*>(p.v) + ab * d.Dv + col;
  const float dx = beta * (to_f32(vr[0]) - u.x), dy = beta * (to_f32(vr[1]) - u.y);
  const float dz = beta * (to_f32(vr[2]) - u.z), dw = beta * (to_f32(vr[3]) - u.w);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int r = 0; r < RL; ++r) {
    s[r].x = fmaf(kn[r], dx, s[r].x);
    s[r].y = fmaf(kn[r], dy, s[r].y);
    s[r].z = fmaf(kn[r], dz, s[r].z);
    s[r].w = fmaf(kn[r], dw, s[r].w);
    o.x = fmaf(qn[r], s[r].x, o.x);
    o.y = fmaf(qn[r], s[r].y, o.y);
    o.z = fmaf(qn[r], s[r].z, o.z);
    o.w = fmaf(qn[r], s[r].w, o.w);
  }
#pragma unroll
  for (int r = 0; r < RL; ++r) *reinterpret_cast<float4*>(p.state_out + sb + static_cast<size_t>(r) * d.Dv) = s[r];
#pragma unroll
  for (int m = 8; m <= 32; m <<= 1) {
    o.x += __shfl_xor(o.x, m);
    o.y += __shfl_xor(o.y, m);
    o.z += __shfl_xor(o.z, m);
    o.w += __shfl_xor(o.w, m);
  }
  if (rg == 0) {
    T* orow = static_cast<T*>(p.o) + ab * d.Dv + col;
    orow[0] = from_f32<T>(o.x);
    orow[1] = from_f32<T>(o.y);
    orow[2] = from_f32<T>(o.z);
    orow[3] = from_f32<T>(o.w);
  }
}

// ------------------------------------------------ decode with conv update
//
// The token's mixed projection x (channels q, k, v of all heads) first goes
// through the depthwise causal conv1d + SiLU update with a K-sample carry
// state (torch-to-nnef GDN page, the causal-conv-update drop-in): channel c's
// output is SiLU of the tap-weighted sum of its K newest samples -- the K - 1
// newest carried ones, then x -- and the carried samples shift by one with x
// appended.  A masked batch row keeps its carried samples, as it keeps its
// recurrent state.  The conv outputs feed the recurrence step in fp32.
//
// One workgroup per (batch, key head): it owns every channel of the key-head
// group (q and k of the key head, v of its G value heads), so each carried
// sample is read and then rewritten by one thread, and the conv state may be
// updated in place.  All of the group's conv outputs go to LDS first; the
// value heads then follow one another with the state slice mapping of the
// decode kernel above.

// Conv update of channel ch of batch row b; returns SiLU of the window sum.
template <typename T>
__device__ __forceinline__ float conv_channel(const DecodeConvArgs& p, int b, int ch, int C, bool valid) {
  const int K = p.K;
  const size_t row = static_cast<size_t>(b) * C + ch;
  const T* st = static_cast<const T*>(p.conv_state) + row * K;
  const T* wt = static_cast<const T*>(p.conv_w) + static_cast<size_t>(ch) * K;
  T* so = static_cast<T*>(p.conv_state_out) + row * K;
  const T xn = static_cast<const T*>(p.x)[row];
  T old[kMaxConvTaps + 1];
#pragma unroll
  for (int i = 0; i < kMaxConvTaps; ++i)
    if (i < K) old[i] = st[i];
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxConvTaps; ++i)
    if (i < K) z = fmaf(to_f32(wt[i]), to_f32(i + 1 < K ? old[i + 1] : xn), z);  // taps oldest first
#pragma unroll
  for (int i = 0; i < kMaxConvTaps; ++i)
    if (i < K) so[i] = valid ? (i + 1 < K ? old[i + 1] : xn) : old[i];
  return z * sigmoid_f(z);
}

template <typename T, int DK>
__global__ void __launch_bounds__(512) decode_conv_kernel(DecodeConvArgs p) {
  constexpr int RL = DK / 8;  // state rows per lane
  // conv outputs of the group: q [DK], k [DK], then v of its G value heads [G Dv]
  extern __shared__ float cv[];
  float* qc = cv;
  float* kc = cv + DK;
  float* vc = cv + 2 * DK;
  const Dims& d = p.d;
  const int bj = blockIdx.x, b = bj / d.Hk, j = bj % d.Hk, G = d.G();
  const int nt = blockDim.x, tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, rg = l >> 3, cq = l & 7;
  const int col = 32 * w + 4 * cq;
  const int C = 2 * d.Hk * DK + d.Hv * d.Dv;
  const bool valid = p.mask == nullptr || p.mask[b] != 0;

  // every channel of the group: q, k of key head j, v of heads j G .. j G + G - 1
  for (int c = tid; c < 2 * DK + G * d.Dv; c += nt) {
    const int ch = c < DK ? j * DK + c
                 : c < 2 * DK ? d.Hk * DK + j * DK + (c - DK)
                              : 2 * d.Hk * DK + j * G * d.Dv + (c - 2 * DK);
    cv[c] = conv_channel<T>(p, b, ch, C, valid);
  }
  __syncthreads();
  float sq = 0.f, sk = 0.f;
  for (int i = l; i < DK; i += 64) {
    sq += qc[i] * qc[i];
    sk += kc[i] * kc[i];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    sq += __shfl_xor(sq, m);
    sk += __shfl_xor(sk, m);
  }
  const float rq = (1.0f / sqrtf(static_cast<float>(DK))) / sqrtf(sq + kNormEps);
  const float rk = 1.0f / sqrtf(sk + kNormEps);
  float kn[RL], qn[RL];
#pragma unroll
  for (int r = 0; r < RL; ++r) {
    kn[r] = kc[rg * RL + r] * rk;
    qn[r] = qc[rg * RL + r] * rq;
  }

  for (int hh = 0; hh < G; ++hh) {
    const int h = j * G + hh, bh = b * d.Hv + h;
    // the state slice of this lane (unconditional buffer loads; an absent
    // initial state reads zeros)
    const size_t hs = static_cast<size_t>(bh) * DK * d.Dv;
    const rsrc_t rs0 = make_rsrc(p.state0 ? static_cast<const void*>(p.state0 + hs) : static_cast<const void*>(p.state_out),
                                 p.state0 ? static_cast<size_t>(DK) * d.Dv * 4 : 0);
    float4 s[RL];
#pragma unroll
    for (int r = 0; r < RL; ++r) s[r] = buf_f4(rs0, 4 * static_cast<uint32_t>((rg * RL + r) * d.Dv + col));
    const float* vh = vc + hh * d.Dv;

    // gates: l = -e^{A_log} softplus(min(a + dt_bias, 20)), beta = sigmoid(b);
    // a masked step gets l = 0, beta = 0
    const size_t ab = static_cast<size_t>(b) * d.Hv + h;
    float ell = 0.f, beta = 0.f;
    if (valid) {
      const float x = to_f32(static_cast<const T*>(p.a)[ab]) + p.dt_bias[h];
      ell = -expf(p.A_log[h]) * softplus_f(fminf(x, kClamp));
      beta = sigmoid_f(to_f32(static_cast<const T*>(p.b)[ab]));
    }
    const float g = expf(ell);
    // S' = g S, u = S'^T kn
    float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      s[r].x *= g; s[r].y *= g; s[r].z *= g; s[r].w *= g;
      u.x = fmaf(kn[r], s[r].x, u.x);
      u.y = fmaf(kn[r], s[r].y, u.y);
      u.z = fmaf(kn[r], s[r].z, u.z);
      u.w = fmaf(kn[r], s[r].w, u.w);
    }
#pragma unroll
    for (int m = 8; m <= 32; m <<= 1) {
      u.x += __shfl_xor(u.x, m);
      u.y += __shfl_xor(u.y, m);
      u.z += __shfl_xor(u.z, m);
      u.w += __shfl_xor(u.w, m);
    }
    // delta = beta (v - u);  S = S' + kn delta^T;  o = S^T qn
    const float dx = beta * (vh[col] - u.x), dy = beta * (vh[col + 1] - u.y);
    const float dz = beta * (vh[col + 2] - u.z), dw = beta * (vh[col + 3] - u.w);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      s[r].x = fmaf(kn[r], dx, s[r].x);
      s[r].y = fmaf(kn[r], dy, s[r].y);
      s[r].z = fmaf(kn[r], dz, s[r].z);
      s[r].w = fmaf(kn[r], dw, s[r].w);
      o.x = fmaf(qn[r], s[r].x, o.x);
      o.y = fmaf(qn[r], s[r].y, o.y);
      o.z = fmaf(qn[r], s[r].z, o.z);
      o.w = fmaf(qn[r], s[r].w, o.w);
    }
    float* so = p.state_out + hs + static_cast<size_t>(rg * RL) * d.Dv + col;
#pragma unroll
    for (int r = 0; r < RL; ++r) *reinterpret_cast<float4*>(so + static_cast<size_t>(r) * d.Dv) = s[r];
#pragma unroll
    for (int m = 8; m <= 32; m <<= 1) {
      o.x += __shfl_xor(o.x, m);
      o.y += __shfl_xor(o.y, m);
      o.z += __shfl_xor(o.z, m);
      o.w += __shfl_xor(o.w, m);
    }
    if (rg == 0) {
      T* orow = static_cast<T*>(p.o) + ab * d.Dv + col;
      orow[0] = from_f32<T>(o.x);
      orow[1] = from_f32<T>(o.y);
      orow[2] = from_f32<T>(o.z);
      orow[3] = from_f32<T>(o.w);
    }
  }
}

template <typename T>
hipError_t launch_conv_t(const DecodeConvArgs& a, hipStream_t st) {
  const int nblk = a.d.B * a.d.Hk, nt = 64 * (a.d.Dv / 32);
  const size_t lds = conv_lds_bytes(a.d);
  switch (a.d.Dk) {
    case 16: decode_conv_kernel<T, 16><<<nblk, nt, lds, st>>>(a); break;
    case 32: decode_conv_kernel<T, 32><<<nblk, nt, lds, st>>>(a); break;
    case 64: decode_conv_kernel<T, 64><<<nblk, nt, lds, st>>>(a); break;
    case 128: decode_conv_kernel<T, 128><<<nblk, nt, lds, st>>>(a); break;
    case 192: decode_conv_kernel<T, 192><<<nblk, nt, lds, st>>>(a); break;
    case 256: decode_conv_kernel<T, 256><<<nblk, nt, lds, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const DecodeArgs& a, hipStream_t st) {
  const int nblk = a.d.B * a.d.Hv, nt = 64 * (a.d.Dv / 32);
  switch (a.d.Dk) {
    case 16: decode_kernel<T, 16><<<nblk, nt, 0, st>>>(a); break;
    case 32: decode_kernel<T, 32><<<nblk, nt, 0, st>>>(a); break;
    case 64: decode_kernel<T, 64><<<nblk, nt, 0, st>>>(a); break;
    case 128: decode_kernel<T, 128><<<nblk, nt, 0, st>>>(a); break;
    case 192: decode_kernel<T, 192><<<nblk, nt, 0, st>>>(a); break;
    case 256: decode_kernel<T, 256><<<nblk, nt, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t st) {
  if (a.d.B * a.d.Hv == 0) return hipSuccess;
  return bf16 ? launch_t<gdn::bf16>(a, st) : launch_t<float>(a, st);
}

hipError_t launch_decode_conv(const DecodeConvArgs& a, bool bf16, hipStream_t st) {
  if (a.d.B * a.d.Hk == 0) return hipSuccess;
  return bf16 ? launch_conv_t<gdn::bf16>(a, st) : launch_conv_t<float>(a, st);
}

}  // namespace gdn
