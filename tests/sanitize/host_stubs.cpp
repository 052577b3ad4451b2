// Stand-ins for the kernel launchers of libgdn.so, for the host-only
// sanitizer build of the C ABI (gdn_api.hip): no GPU is touched.  Each stub
// reads the first and the last byte of every workspace or checkpoint region
// the host code hands to that kernel, with the extent the kernel addresses
// (from the dims), and counts the launch.  The driver allocates the
// workspace and the checkpoint buffer with malloc at exactly the sizes the
// library asks for, so a region that reaches past its buffer is an
// out-of-bounds read for AddressSanitizer.  Input and output tensors
// (q, k, v, o, ...) are placeholders that are never read.
#include <stddef.h>
#include <stdio.h>

#include "../../linear_attention_recurrence_fwd_amd/csrc/gdn_internal.h"

namespace {
long g_launches = 0;
volatile unsigned char g_sink;

void touch(const void* p, size_t bytes) {
  if (!p || !bytes) return;
  const volatile unsigned char* c = static_cast<const volatile unsigned char*>(p);
  g_sink = c[0];
  g_sink = c[bytes - 1];
}
size_t bt(const gdn::Dims& d) { return static_cast<size_t>(d.B) * d.T; }
size_t nmat(const gdn::Dims& d) { return static_cast<size_t>(d.B) * d.Hv * d.nchunk(); }
size_t slots(const gdn::Dims& d) { return nmat(d) * d.Dk * d.Dv; }
size_t kts(const gdn::Dims& d) { return static_cast<size_t>(d.B) * d.Hk * d.nchunk() * d.Dk * 64; }
void touch_scalars(const gdn::Dims& d, const gdn::StepScalars& s) {
  touch(s.rq, bt(d) * d.Hk * 4);
  touch(s.rk, bt(d) * d.Hk * 4);
  touch(s.kq, bt(d) * d.Hk * 4);
  touch(s.ell, bt(d) * d.Hv * 4);
  touch(s.beta, bt(d) * d.Hv * 4);
}
void touch_ckpt(const gdn::Dims& d, const float* ckpt) {
  const size_t nc = d.nchunk();
  if (nc > 1) touch(ckpt, (nc - 1) * static_cast<size_t>(d.B) * d.Hv * d.Dk * d.Dv * 4);
}
void touch_chunk(const gdn::Dims& d, const gdn::ChunkBufs& cb) {
  touch(cb.Tx, nmat(d) * 64 * 64 * 2);
  touch(cb.Mq, nmat(d) * 64 * 64 * 2);
  touch(cb.PqT, nmat(d) * 64 * 64 * 2);
  touch(cb.QT, kts(d) * 2);
  touch(cb.sc, nmat(d) * gdn::SC_ROWS * 64 * 4);
  touch(cb.Hb, slots(d) * 2);
  touch(cb.X, bt(d) * d.Hv * d.Dv * 2);
  for (const gdn::bf16* r : {cb.Kb, cb.Kh, cb.Qb, cb.KbT, cb.QbT}) touch(r, nmat(d) * 64 * d.Dk * 2);
  touch(cb.vsc, nmat(d) * gdn::VSC_ROWS * 64 * 4);
}
size_t map_floats(const gdn::Dims& d, int seg) {
  return static_cast<size_t>(gdn::tpar_nseg(d, seg)) * d.B * d.Hv * d.Dk * (d.Dk + d.Dv);
}
size_t hseg_floats(const gdn::Dims& d, int seg) {
  return static_cast<size_t>(gdn::tpar_nseg(d, seg) - 1) * d.B * d.Hv * d.Dk * d.Dv;
}
}  // namespace

extern "C" long gdn_stub_launches() { return g_launches; }

namespace gdn {
hipError_t launch_prep(const PrepArgs& a, bool, hipStream_t) {
  touch_scalars(a.d, a.s);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_scan_fwd(const ScanFwdArgs& a, bool, hipStream_t) {
  touch_scalars(a.d, a.s);
  touch_ckpt(a.d, a.ckpt);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_scan_bwd(const ScanBwdArgs& a, bool, hipStream_t) {
  touch_scalars(a.d, a.s);
  touch_ckpt(a.d, a.ckpt);
  touch(a.U, bt(a.d) * a.d.Hv * a.d.Dv * 4);
  touch(a.E, bt(a.d) * a.d.Hv * a.d.Dv * 4);
  touch(a.dHend, slots(a.d) * 4);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_chunk_grad(const ChunkGradArgs& a, bool, hipStream_t) {
  touch_scalars(a.d, a.s);
  touch(a.U, bt(a.d) * a.d.Hv * a.d.Dv * 4);
  touch(a.E, bt(a.d) * a.d.Hv * a.d.Dv * 4);
  touch(a.dHend, slots(a.d) * 4);
  touch(a.part_dA, nmat(a.d) * 8);
  touch(a.part_ddt, nmat(a.d) * 8);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_scan_bwd_vg(const ScanBwdVgArgs& a, bool, hipStream_t) {
  touch(a.s.rq, bt(a.d) * a.d.Hk * 4);
  touch(a.s.beta, bt(a.d) * a.d.Hv * 4);
  touch(a.sub, vg_sub_floats(a.d) * 4);
  touch(a.part, bt(a.d) * a.d.Hv * vg_nslice(a.d.Dv) * 3 * a.d.Dk * 4);
  touch(a.pdb, bt(a.d) * a.d.Hv * vg_nslice(a.d.Dv) * 4);
  touch_ckpt(a.d, a.ckpt);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_vg_reduce(const VgReduceArgs& a, bool, hipStream_t) {
  touch(a.part, bt(a.d) * a.d.Hv * a.nslice * 3 * a.d.Dk * 4);
  touch(a.pdb, bt(a.d) * a.d.Hv * a.nslice * 4);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_param_reduce(const ParamReduceArgs& a, hipStream_t) {
  touch(a.part_dA, static_cast<size_t>(a.B) * a.NC * a.Hv * 8);
  touch(a.part_ddt, static_cast<size_t>(a.B) * a.NC * a.Hv * 8);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_chunk_prep(const ChunkPrepArgs& a, hipStream_t) {
  touch_chunk(a.d, a.cb);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_vg_chunk_prep(const VgChunkPrepArgs& a, hipStream_t) {
  touch_chunk(a.d, a.cb);
  ++g_launches;
  return hipSuccess;
}
void touch_vg_grad(const VgChunkGradArgs& a) {
  touch_chunk(a.d, a.cb);
  touch(a.dHend, slots(a.d) * 2);
  if (a.cb.Hb == nullptr) touch_ckpt(a.d, a.ckpt);  // else the bf16 states of the saved record (touch_chunk)
  touch(a.X, bt(a.d) * a.d.Hv * a.d.Dv * 2);
  touch(a.dPA, nmat(a.d) * 2 * 64 * 64 * 2);
  touch(a.qk, bt(a.d) * a.d.Hv * 2 * a.d.Dk * 2);
  ++g_launches;
}
hipError_t launch_vg_chunk_x(const VgChunkGradArgs& a, hipStream_t) {
  touch_vg_grad(a);
  return hipSuccess;
}
hipError_t launch_vg_chunk_grad(const VgChunkGradArgs& a, hipStream_t) {
  touch_vg_grad(a);
  return hipSuccess;
}
hipError_t launch_vg_norm_bwd(const VgChunkGradArgs& a, hipStream_t) {
  touch(a.qk, bt(a.d) * a.d.Hv * 2 * a.d.Dk * 2);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_chunk_fwd(const ChunkFwdArgs& a, hipStream_t) {
  touch_chunk(a.d, a.cb);
  touch_ckpt(a.d, a.ckpt);
  if (a.seg) {
    if (a.map) touch(a.maps, map_floats(a.d, a.seg) * 4);
    else touch(a.hseg, hseg_floats(a.d, a.seg) * 4);
    touch(a.vzero, 64 * 4);
  }
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_seg_chain(const SegChainArgs& a, hipStream_t) {
  const int seg = (a.d.nchunk() + a.nseg - 1) / a.nseg;
  touch(a.maps, static_cast<size_t>(a.nseg) * a.d.B * a.d.Hv * a.d.Dk * (a.d.Dk + a.d.Dv) * 4);
  touch(a.hseg, hseg_floats(a.d, seg) * 4);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t) {
  touch(p, n * 4);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_chunk_bwd_state(const ChunkBwdArgs& a, hipStream_t) {
  touch_chunk(a.d, a.cb);
  touch(a.dHend, slots(a.d) * 2);
  if (a.seg) {
    if (a.map) touch(a.maps, map_floats(a.d, a.seg) * 4);
    else touch(a.hseg, hseg_floats(a.d, a.seg) * 4);
    touch(a.vzero, 64 * 4);
  }
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_chunk_bwd_grad(const ChunkBwdArgs& a, hipStream_t) {
  touch_chunk(a.d, a.cb);
  touch(a.dHend, slots(a.d) * 2);
  touch(a.part_dA, nmat(a.d) * 8);
  touch(a.part_ddt, nmat(a.d) * 8);
  if (!a.cb.X) touch_ckpt(a.d, a.ckpt);  // fp32 checkpoints (the saved record has X)
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_state_bf16(const StateBf16Args& a, hipStream_t) {
  touch(a.Hb, static_cast<size_t>(a.nslot) * a.slot * 2);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs&, bool, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode_conv(const DecodeConvArgs&, bool, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace gdn
