// Device helpers shared by the gfx950 kernels of libgdn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;        // steps per checkpoint
constexpr float kNormEps = 1e-6f; // inside the square root of the L2 norm
constexpr float kClamp = 20.0f;   // upper bound of the softplus argument

// bf16 storage type (raw bits).
struct bf16 {
  uint16_t x;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) {
  return __uint_as_float(static_cast<uint32_t>(v.x) << 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// Round to nearest, ties to even (the gfx950 conversion instruction); NaN
// stays NaN.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) {
  return bf16{__builtin_bit_cast(uint16_t, static_cast<__bf16>(v))};
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
// Two floats -> two bf16 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// Four floats -> four consecutive bf16 (8 bytes).
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2(pack2_bf16(a, b), pack2_bf16(c, d));
}

// Unpack 16 bytes of storage into fp32 values.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(uint4 u, float* out) {
    out[0] = __uint_as_float(u.x);
    out[1] = __uint_as_float(u.y);
    out[2] = __uint_as_float(u.z);
    out[3] = __uint_as_float(u.w);
  }
};
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(uint4 u, float* out) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// DPP lane exchange within a row of 16 lanes.
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over the 16 lanes of a DPP row.  Every lane of the row ends with the
// same bits: each stage adds a value to its partner's value (a + b == b + a).
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowHalfMirror>(v);
  v += dpp<kRowMirror>(v);
  return v;
}

// DPP move with a row mask: lanes of disabled rows, and lanes whose source is
// outside their row, receive 0.
template <int CTRL, int ROW_MASK = 0xf> __device__ __forceinline__ float dpp_or0(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142;  // lane 15 of each row to the next row
constexpr int kRowBcast31 = 0x143;  // lane 31 to rows 2 and 3

// Inclusive prefix sum over the 64 lanes of a wave, in lane order: shifted
// adds within each row of 16 lanes, then each row's total carried into the
// rows after it (row 0 -> 1 and 2 -> 3, then rows 0-1 -> 2 and 3).
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp_or0<kRowShr1>(v);
  v += dpp_or0<kRowShr2>(v);
  v += dpp_or0<kRowShr4>(v);
  v += dpp_or0<kRowShr8>(v);
  v += dpp_or0<kRowBcast15, 0xa>(v);
  v += dpp_or0<kRowBcast31, 0xc>(v);
  return v;
}

// Sum over the 64 lanes of a wave in fp64, the same bits in every lane: the
// sum of each row of 16 lanes (butterfly), then the four row sums in order.
template <int CTRL> __device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(b), CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(b >> 32), CTRL, 0xf, 0xf, true);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
__device__ __forceinline__ double lane_f64(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
  v += dpp_f64<kQuadXor1>(v);
  v += dpp_f64<kQuadXor2>(v);
  v += dpp_f64<kRowHalfMirror>(v);
  v += dpp_f64<kRowMirror>(v);
  return (lane_f64(v, 0) + lane_f64(v, 16)) + (lane_f64(v, 32) + lane_f64(v, 48));
}

__device__ __forceinline__ float softplus_f(float x) {
  return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}
__device__ __forceinline__ float sigmoid_f(float x) {
  if (x >= 0.f) return 1.f / (1.f + expf(-x));
  float e = expf(x);
  return e / (1.f + e);
}

}  // namespace gdn

// ---- bf16 matrix cores (gfx950 v_mfma_f32_16x16x32_bf16)
// One wave computes a 16x16 fp32 tile D = A (16x32) * B (32x16) + C.
// Lane l supplies A[l%16][8*(l/16) + 0..7] and B[8*(l/16) + 0..7][l%16], and
// holds D[4*(l/16) + 0..3][l%16].
namespace gdn {
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 f4zero() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// fp32 matrix cores (v_mfma_f32_16x16x4f32): D = A (16x4) * B (4x16) + C with
// lane l supplying A[l%16][l/16] and B[l/16][l%16] and holding D as above.
__device__ __forceinline__ f32x4 mfma16f(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// acc + A B for 16x16 fp32 tiles in LDS (row strides as, bs), 4 MFMAs.
__device__ __forceinline__ f32x4 mm16f(f32x4 acc, const float* A, int as, const float* B, int bs) {
  const int l = threadIdx.x & 63, lr = l & 15, lg = l >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) acc = mfma16f(A[lr * as + 4 * kb + lg], B[(4 * kb + lg) * bs + lr], acc);
  return acc;
}

// 16 bytes of bf16 storage <-> operand register.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ bf16x8 load_bf16x8(const void* p) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16 bf16_of(float v) { return from_f32<bf16>(v); }
__device__ __forceinline__ bf16x8 zero8() { return as_bf16x8(make_uint4(0, 0, 0, 0)); }
// a.lo b.lo + a.hi b.hi + c for two packed bf16 pairs (one dot2 instruction;
// the bf16 products are exact in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}
// Every bf16 of x multiplied by s (fp32 product, rounded to nearest even).
__device__ __forceinline__ bf16x8 scale8(const bf16x8& x, float s) {
  const uint4 u = __builtin_bit_cast(uint4, x);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack2_bf16(__uint_as_float(w[i] << 16) * s, __uint_as_float(w[i] & 0xffff0000u) * s);
  return as_bf16x8(make_uint4(o[0], o[1], o[2], o[3]));
}
// 4x4 transpose inside each DPP quad: lane e of the quad returns element e
// of every lane's x, i.e. out[r] on lane e = (x[e] on lane r).  Two
// butterfly exchanges (lane xor 1, lane xor 2), moves and selects only.
__device__ __forceinline__ f32x4 quad_transpose(const f32x4& x) {
  const int e = threadIdx.x & 3;
  f32x4 y, z;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float o = dpp<kQuadXor1>(x[r ^ 1]);
    y[r] = ((e ^ r) & 1) ? o : x[r];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float o = dpp<kQuadXor2>(y[r ^ 2]);
    z[r] = ((e ^ r) & 2) ? o : y[r];
  }
  return z;
}
// Lane moves that make 8-byte stores coalesce: the memory pipeline handles a
// quad of lanes at a time, so four consecutive lanes should write one row's
// 32 contiguous bytes rather than four rows.  Both are ds_bpermute pairs (no
// LDS memory is used).
__device__ __forceinline__ uint2 bpermute_u2(int src_lane, uint2 v) {
  return make_uint2(static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * src_lane, static_cast<int>(v.x))),
                    static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * src_lane, static_cast<int>(v.y))));
}
// Within each group of 16 lanes, lane 4 a + b takes the value of lane 4 b + a.
// After quad_transpose of an accumulator tile, lane 4 a + b of group g holds
// row 4 g + b, columns 4 a .. 4 a + 3; after this move it holds row
// 4 g + a, columns 4 b .. 4 b + 3.
__device__ __forceinline__ uint2 quads_to_rows(uint2 v) {
  const int l = threadIdx.x & 63;
  return bpermute_u2((l & 48) + 4 * (l & 3) + ((l >> 2) & 3), v);
}
// Lane l takes the value of lane 16 (l % 4) + l / 4.  When lane 16 g + s holds
// row s, 4-column group g (a transposing LDS read, or an accumulator tile's
// column s), lane 4 s + g afterwards holds row s, 4-column group g.
__device__ __forceinline__ uint2 groups_to_quads(uint2 v) {
  const int l = threadIdx.x & 63;
  return bpermute_u2(16 * (l & 3) + (l >> 2), v);
}

// Sum over the 4 lanes of a DPP quad; every lane of the quad gets the same bits.
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  return v;
}

// MFMA operands are loaded quad-coalesced -- lane m reads 16-byte piece m % 4
// of tile row m / 4, so four lanes cover 64 contiguous bytes -- and then moved
// to the operand layout (lane l: row l % 16, piece l / 16) by this lane
// permutation: lane l takes the register of lane 4 (l % 16) + l / 16.
__device__ __forceinline__ int coal_row(int l) { return l >> 2; }
__device__ __forceinline__ int coal_piece(int l) { return l & 3; }
__device__ __forceinline__ bf16x8 to_mfma_layout(const bf16x8& v) {
  const int l = threadIdx.x & 63;
  const int src = 4 * (4 * (l & 15) + (l >> 4));
  const uint4 u = __builtin_bit_cast(uint4, v);
  uint4 o;
  o.x = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src, static_cast<int>(u.x)));
  o.y = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src, static_cast<int>(u.y)));
  o.z = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src, static_cast<int>(u.z)));
  o.w = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src, static_cast<int>(u.w)));
  return __builtin_bit_cast(bf16x8, o);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element i % 4 of the 8-byte pieces addressed by lanes
// i / 4 + 4 e of its group, as element e (e = 0..3).  Used on a row-major tile
// with lane s of a group addressing row r0 + s / 4, columns c0 + 4 (s % 4)
// .. + 3, lane s gets rows r0 .. r0 + 3 of column c0 + s: four rows of one
// column, the layout of an MFMA accumulator or of a transposed operand.
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Buffer loads: a wave-uniform resource descriptor (base, byte size) in
// scalar registers plus a 32-bit byte offset per lane.  Reads at or past the
// size return zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
// Every descriptor here is built from wave-uniform values; reading them
// through readfirstlane states that to the compiler, which otherwise may not
// prove it and wraps each buffer access in a loop over distinct descriptors.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, size_t bytes) {
  const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : static_cast<uint32_t>(bytes);
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* pu = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(pu, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(n)), 0x00020000);
}
__device__ __forceinline__ bf16x8 buf_bf16x8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 buf_u2(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ float4 buf_f4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_f1(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Buffer stores: a store at or past the descriptor's size is dropped.  Used
// where a store would otherwise sit under a branch: after a branch that
// issued stores on one path only, the compiler's wait for an earlier load
// must also wait for those stores, which voids the prefetch.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
__device__ __forceinline__ void buf_store_u4(rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store_u2(rsrc_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, off, 0, 0);
}
// The same store marked non-temporal (streamed: data another kernel reads
// much later, which should not displace what the running kernels reuse).
__device__ __forceinline__ void buf_store_u2_nt(rsrc_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, off, 0, 2);
}

// Direct-to-LDS buffer loads (lane i of a load writes its 16 or 4 bytes at
// the wave's LDS base + 16 i or 4 i), issued through inline assembly: the
// compiler does not see them, so it does not make every later LDS read wait
// for them.  The caller waits explicitly (wait_vm) before the barrier that
// publishes the data.  M0 holds the wave's LDS base; the s_nop is the wait
// state required between an M0 write and a load to LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const void lds_cvoid;
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cvoid*)p)));
}
__device__ __forceinline__ void dma16(const i32x4& r, const void* lds, uint32_t off) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds_addr(lds)) : "memory");
}
// The same load marked non-temporal: data read once, which should not
// displace what other workgroups reuse from the caches.
__device__ __forceinline__ void dma16_nt(const i32x4& r, const void* lds, uint32_t off) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(off), "s"(r), "{m0}"(lds_addr(lds)) : "memory");
}
__device__ __forceinline__ void dma4(const i32x4& r, const void* lds, uint32_t off) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds_addr(lds)) : "memory");
}
// Raw buffer descriptor words (as make_rsrc) for the inline loads.
__device__ __forceinline__ i32x4 raw_desc(const void* p, size_t bytes) {
  const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : static_cast<uint32_t>(bytes);
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return i32x4{static_cast<int>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a))),
               static_cast<int>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xffffu)),
               static_cast<int>(__builtin_amdgcn_readfirstlane(n)), 0x00020000};
}
// Wait until at most N of this wave's vector memory operations (loads, stores
// and direct-to-LDS loads, counted in issue order) are pending.
template <int N> __device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// (lgkmcnt) and meets the other waves, without waiting for outstanding global
// loads, so loads issued ahead of time (prefetches) stay in flight across it.
// The memory clobbers keep the compiler from moving LDS accesses across it.
// Global memory written before it is NOT made visible to the other waves.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Orders LDS accesses within one wave: waits for this wave's LDS operations,
// which the LDS executes in issue order, so that lanes read what other lanes
// of the same wave wrote before it.  No cross-wave effect.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
}  // namespace gdn
