// The chunk form's triangular inverse Tx = (I + N)^-1 (N strictly lower
// triangular, 64 x 64, fp32 in LDS with row stride SP), shared by the scalar
// and the per-channel gate chunk preparation.  Tx is unit lower triangular:
// its diagonal 16 x 16 blocks are D_i = (I + N_ii)^-1 and, for i > j,
// Tx_ij = -D_i (sum over j <= k < i of N_ik Tx_kj) (the block rows of
// (I + N) Tx = I).
#pragma once

#include "gdn_dev.h"

namespace gdn {
namespace tri {

constexpr int L = kChunk;
constexpr int SP = L + 4;  // fp32 row stride of N and the staging matrix (16-byte aligned rows)

// Wave w inverts D_w by forward substitution -- lane 4c + q holds rows
// 4m + q of column c -- and writes it over N_ww.
__device__ __forceinline__ void invert_diagonal_block(float* nf, int w, int l) {
  const int c = l >> 2, q = l & 3;
  float* nb = &nf[16 * w * SP + 16 * w];
  float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    // rows s >= t of x are still zero, and N[t][s] = 0 for s >= t
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < (t + 3) / 4; ++m) acc = fmaf(nb[t * SP + 4 * m + q], x[m], acc);
    const float xt = (t == c ? 1.f : 0.f) - quad_sum(acc);
    if ((t & 3) == q) x[t >> 2] = xt;
  }
  wave_lds_sync();  // every lane's reads of N_ww are done
#pragma unroll
  for (int m = 0; m < 4; ++m) nb[(4 * m + q) * SP + c] = x[m];
}

// Block column j < 3 of Tx below the diagonal, top to bottom, on fp32 MFMA,
// into the staging matrix st.  The partial sums pass through the (zero,
// unused) block (0, j + 1) of nf to become an operand.
__device__ __forceinline__ void lower_blocks(float* nf, float* st, int j) {
  const int l = threadIdx.x & 63, lr = l & 15, lg = l >> 4;
  float* part = &nf[16 * (j + 1)];
  for (int i = j + 1; i < 4; ++i) {
    f32x4 acc = f4zero();
    acc = mm16f(acc, &nf[16 * i * SP + 16 * j], SP, &nf[16 * j * SP + 16 * j], SP);
    for (int k = j + 1; k < i; ++k) acc = mm16f(acc, &nf[16 * i * SP + 16 * k], SP, &st[16 * k * SP + 16 * j], SP);
#pragma unroll
    for (int r = 0; r < 4; ++r) part[(4 * lg + r) * SP + lr] = acc[r];
    wave_lds_sync();
    const f32x4 tij = mm16f(f4zero(), &nf[16 * i * SP + 16 * i], SP, part, SP);
#pragma unroll
    for (int r = 0; r < 4; ++r) st[(16 * i + 4 * lg + r) * SP + 16 * j + lr] = -tij[r];
    wave_lds_sync();  // Tx_ij is an operand of the next block; part is rewritten
  }
}

// The diagonal blocks of Tx (in nf after invert_diagonal_block) and zeros
// above them, into st (one wave).
__device__ __forceinline__ void diagonal_blocks(const float* nf, float* st, int l) {
#pragma unroll
  for (int blk = 0; blk < 16; ++blk) {
    const int bi = blk >> 2, bj = blk & 3;
    if (bi > bj) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * bi + 4 * e + (l >> 4), col = 16 * bj + (l & 15);
      st[row * SP + col] = bi == bj ? nf[row * SP + col] : 0.f;
    }
  }
}

// st (fp32 [L][SP]) -> dst (bf16 [L][L]), 8 elements per store.
__device__ __forceinline__ void store_mat(const float* st, bf16* dst, int tid, int nt) {
  for (int u = tid; u < L * L / 8; u += nt) {
    const int r = u >> 3, c8 = 8 * (u & 7);
    const float4 a = *reinterpret_cast<const float4*>(&st[r * SP + c8]);
    const float4 b = *reinterpret_cast<const float4*>(&st[r * SP + c8 + 4]);
    *reinterpret_cast<uint4*>(dst + r * L + c8) =
        make_uint4(pack2_bf16(a.x, a.y), pack2_bf16(a.z, a.w), pack2_bf16(b.x, b.y), pack2_bf16(b.z, b.w));
  }
}

}  // namespace tri
}  // namespace gdn
