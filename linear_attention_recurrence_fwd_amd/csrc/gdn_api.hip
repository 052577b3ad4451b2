// C ABI of libgdn.so (declared in include/gdn.h): argument validation,
// workspace layout, kernel selection and launch.  No allocation, no host sync.
#include "../../include/gdn.h"
#include "gdn_internal.h"

#include <limits.h>

#include <mutex>

namespace {

using gdn::Dims;

constexpr size_t kAlign = 256;

size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t rq, rk, kq, ell, beta;                 // prep scalars
  size_t U, E, dHend, pdA, pdt;                 // backward only
  size_t Tx, Mq, PqT, QT, SC;              // chunk form
  size_t HB;                                    // chunk backward: bf16 chunk-start states
  size_t maps, hseg, vzero;                     // T-parallel chunk forward
  size_t total;
};

// Elements of the bf16 chunk-start states (one slot per chunk).
size_t state_slots_elems(const Dims& d) {
  return static_cast<size_t>(d.nchunk()) * d.B * d.Hv * static_cast<size_t>(d.Dk) * d.Dv;
}

// The checkpoint buffer under gdn_dims.save (chunk family): the bf16
// chunk-start states and the chunk matrices (offsets in fp32 elements,
// 256-byte aligned).
struct Saved {
  size_t HB, Tx, PqT, QT, SC, X, total;
};

Saved saved_layout(const Dims& d) {
  Saved S{};
  size_t off = 0;
  auto take = [&](size_t nfloat) {
    size_t o = off;
    off += align_up(nfloat * sizeof(float)) / sizeof(float);
    return o;
  };
  const size_t nc = d.nchunk();
  const size_t mats = static_cast<size_t>(d.B) * d.Hv * nc * 64 * 64;  // bf16 each
  const size_t kts = static_cast<size_t>(d.B) * d.Hk * nc * d.Dk * 64;
  S.HB = take((state_slots_elems(d) + 1) / 2);
  S.Tx = take((mats + 1) / 2);
  S.PqT = take((mats + 1) / 2);
  S.QT = take((kts + 1) / 2);
  S.SC = take(static_cast<size_t>(d.B) * d.Hv * nc * gdn::SC_ROWS * 64);
  S.X = take((static_cast<size_t>(d.B) * d.T * d.Hv * d.Dv + 1) / 2);
  S.total = off;
  return S;
}

size_t ckpt_state_elems(const Dims& d) {
  const size_t nc = d.nchunk();
  return nc > 1 ? (nc - 1) * d.B * d.Hv * static_cast<size_t>(d.Dk) * d.Dv : 0;
}

// Workspace layout.  `saved`: the chunk matrices live in the checkpoint tail.
// `tseg`: chunks per segment of the T-parallel forward (0: none).
Layout layout(const Dims& d, bool bwd, bool chunk, bool saved, int tseg = 0) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t nfloat) {
    size_t o = off;
    off += align_up(nfloat * sizeof(float));
    return o;
  };
  const size_t bt = static_cast<size_t>(d.B) * d.T;
  if (!chunk) {  // the chunk form computes its per-step scalars in chunk_prep
    L.rq = take(bt * d.Hk);
    L.rk = take(bt * d.Hk);
    L.kq = take(bt * d.Hk);
    L.ell = take(bt * d.Hv);
    L.beta = take(bt * d.Hv);
  }
  if (bwd) {
    const size_t nc = d.nchunk();
    const size_t col = bt * d.Hv * d.Dv;
    const size_t dh = nc * d.B * d.Hv * static_cast<size_t>(d.Dk) * d.Dv;
    if (chunk) {  // dH' in bf16 (the gradient pass reads dv = diag(beta) eps, not eps)
      L.dHend = take((dh + 1) / 2);
      if (!saved) L.HB = take((state_slots_elems(d) + 1) / 2);
    } else {
      L.U = take(col);
      L.E = take(col);
      L.dHend = take(dh);
    }
    L.pdA = take(2 * static_cast<size_t>(d.B) * nc * d.Hv);  // fp64
    L.pdt = take(2 * static_cast<size_t>(d.B) * nc * d.Hv);
  }
  if (chunk) {
    const size_t nc = d.nchunk();
    const size_t mats = static_cast<size_t>(d.B) * d.Hv * nc * 64 * 64;  // bf16 each
    const size_t kts = static_cast<size_t>(d.B) * d.Hk * nc * d.Dk * 64;
    if (!bwd) L.Mq = take((mats + 1) / 2);
    if (!saved) {
      L.Tx = take((mats + 1) / 2);
      L.SC = take(static_cast<size_t>(d.B) * d.Hv * nc * gdn::SC_ROWS * 64);
      if (bwd) {
        L.PqT = take((mats + 1) / 2);
        L.QT = take((kts + 1) / 2);
      }
    }
  }
  if (chunk && tseg) {  // the segment maps (forward or reverse) and start states
    const size_t ns = gdn::tpar_nseg(d, tseg), BH = static_cast<size_t>(d.B) * d.Hv;
    L.maps = take(ns * BH * d.Dk * (static_cast<size_t>(d.Dk) + d.Dv));
    L.hseg = take((ns - 1) * BH * d.Dk * d.Dv);
    L.vzero = take(64);
  }
  L.total = off;
  return L;
}

// The chunk kernels address their per-(head, chunk) matrices, the transposed
// q rows and the per-step chunk scalars through buffer descriptors whose size
// and 32-bit byte offsets cover the whole tensor, so each must stay below
// 4 GiB: the 64 x 64 bf16 matrices (B Hv ceil(T/64) of them) and the
// transposed rows (B Hk ceil(T/64) Dk x 64, bf16).  q, k, v, o, the saved X
// and every per-chunk state slot are within that bound once their element
// counts fit in int32 (2 bytes per element).
bool chunk_fits(const gdn_dims* p) {
  const double lim = 4294967296.0;
  const double nc = static_cast<double>((p->T + 63) / 64);
  const double mats = static_cast<double>(p->B) * p->Hv * nc * 64.0 * 64.0 * 2.0;
  const double kts = static_cast<double>(p->B) * p->Hk * nc * p->Dk * 64.0 * 2.0;
  return mats < lim && kts < lim;
}
bool chunk_ok(const gdn_dims* p) {
  return gdn::chunk_supported(static_cast<int>(p->Dk), static_cast<int>(p->Dv), p->dtype == GDN_BF16) &&
         chunk_fits(p);
}

// Checks everything that does not depend on pointers.
int check_dims(const gdn_dims* p, Dims* out) {
  if (!p) return GDN_ERR_INVALID_ARG;
  if (p->B < 1 || p->T < 0 || p->Hk < 1 || p->Hv < 1 || p->Dk < 1 || p->Dv < 1)
    return GDN_ERR_INVALID_ARG;
  if (p->Hv % p->Hk != 0) return GDN_ERR_INVALID_ARG;
  if (p->dtype != GDN_F32 && p->dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  if (p->algo != GDN_ALGO_AUTO && p->algo != GDN_ALGO_SCAN && p->algo != GDN_ALGO_CHUNK &&
      p->algo != GDN_ALGO_CHUNK_TPAR)
    return GDN_ERR_INVALID_ARG;
  if ((p->algo == GDN_ALGO_CHUNK || p->algo == GDN_ALGO_CHUNK_TPAR) && !chunk_ok(p))
    return GDN_ERR_UNSUPPORTED;
  if (!gdn::scan_supported(static_cast<int>(p->Dk), static_cast<int>(p->Dv)))
    return GDN_ERR_UNSUPPORTED;
  // every tensor's element count (and the checkpoint slab count) fits in int32
  const double big = static_cast<double>(INT_MAX);
  const double bt = static_cast<double>(p->B) * p->T;
  const double nc = static_cast<double>((p->T + 63) / 64);
  if (bt * p->Hv * p->Dv > big || bt * p->Hk * p->Dk > big ||
      nc * p->B * p->Hv * p->Dk * p->Dv > big || static_cast<double>(p->B) * p->Hv > 65535.0 * 1024)
    return GDN_ERR_UNSUPPORTED;
  *out = Dims{static_cast<int>(p->B), static_cast<int>(p->T), static_cast<int>(p->Hk),
              static_cast<int>(p->Hv), static_cast<int>(p->Dk), static_cast<int>(p->Dv)};
  return GDN_OK;
}

// Per-kernel timing events (gdn_set_kernel_events), per host thread: a
// thread's setting applies to the calls that thread makes.
struct Timing {
  void* const* ev = nullptr;
  int n = 0;
  int next = 0;
};
thread_local Timing g_timing;

// Launches one kernel through `fn`, bracketed by the timing events if set.
template <typename F>
bool launch(hipStream_t st, F&& fn) {
  const bool timed = g_timing.ev && g_timing.next + 1 < g_timing.n;
  if (timed &&
      hipEventRecord(static_cast<hipEvent_t>(g_timing.ev[g_timing.next]), st) != hipSuccess)
    return false;
  if (fn() != hipSuccess) return false;
  if (timed) {
    if (hipEventRecord(static_cast<hipEvent_t>(g_timing.ev[g_timing.next + 1]), st) != hipSuccess)
      return false;
    g_timing.next += 2;
  }
  return true;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

// Kernel family of a call: the chunk form where asked for, and under AUTO for
// bf16 with a supported head size and more than one step (single steps, the
// decode case, stay on the scan).
bool use_chunk(const gdn_dims* p) {
  if (p->algo == GDN_ALGO_CHUNK || p->algo == GDN_ALGO_CHUNK_TPAR) return true;
  if (p->algo == GDN_ALGO_SCAN) return false;
  return p->T > 1 && chunk_ok(p);
}
bool use_chunk_fwd(const gdn_dims* p) { return use_chunk(p); }
// Chunks per segment of the T-parallel forward (0: the single-pass forward).
// AUTO takes it where the chunk form runs and the segments pay.
int tpar_seg(const gdn_dims* p, const Dims& d) {
  const bool on = p->algo == GDN_ALGO_CHUNK_TPAR || (p->algo == GDN_ALGO_AUTO && use_chunk(p));
  return on && d.T > 0 ? gdn::tpar_seg_len(d) : 0;
}
bool use_chunk_bwd(const gdn_dims* p) { return use_chunk(p); }
// The chunk matrices go through the checkpoint tail.
bool use_saved(const gdn_dims* p) { return p->save != 0 && use_chunk(p); }
// Whether the state passes store the bf16 chunk-start states and dH'
// non-temporal: when the backward's hand-off (those two, and the dO, dv and X
// rows it reads with them) exceeds the 256 MB memory-side cache, it cannot
// stay there anyway, and dirty lines of it held in the caches slow the
// reverse state pass's chain.
bool stream_handoff(const Dims& d) {
  const double states = static_cast<double>(d.nchunk()) * d.B * d.Hv * d.Dk * d.Dv * 2;
  const double rows = 3.0 * d.B * d.T * d.Hv * d.Dv * 2;
  return 2 * states + rows > 256.0 * 1024 * 1024;
}

gdn::ChunkBufs chunk_bufs(void* ws, const Layout& L, bool bwd) {
  gdn::ChunkBufs cb{};
  cb.Tx = at<gdn::bf16>(ws, L.Tx);
  cb.sc = at<float>(ws, L.SC);
  if (!bwd) cb.Mq = at<gdn::bf16>(ws, L.Mq);
  if (bwd) {
    cb.PqT = at<gdn::bf16>(ws, L.PqT);
    cb.QT = at<gdn::bf16>(ws, L.QT);
  }
  return cb;
}

// The saved states and matrices in the checkpoint buffer (every pointer but Mq).
void saved_bufs(const Dims& d, const float* ckpt, gdn::ChunkBufs& cb) {
  const Saved S = saved_layout(d);
  float* tail = const_cast<float*>(ckpt);
  cb.Hb = reinterpret_cast<gdn::bf16*>(tail + S.HB);
  cb.Tx = reinterpret_cast<gdn::bf16*>(tail + S.Tx);
  cb.PqT = reinterpret_cast<gdn::bf16*>(tail + S.PqT);
  cb.QT = reinterpret_cast<gdn::bf16*>(tail + S.QT);
  cb.sc = tail + S.SC;
  cb.X = reinterpret_cast<gdn::bf16*>(tail + S.X);
}

gdn::StepScalars scalars(void* ws, const Layout& L) {
  return gdn::StepScalars{at<float>(ws, L.rq), at<float>(ws, L.rk), at<float>(ws, L.kq),
                          at<float>(ws, L.ell), at<float>(ws, L.beta)};
}

// ---- per-key-channel gate

struct VgLayout {
  size_t rq, rk, kq, beta, sub, part, pdb;
  size_t Kb, Kh, Qb, KbT, QbT, Tx, Mq, PqT, vsc;  // chunk form
  size_t dHend, X, dPA;                           // chunk form, backward
  size_t total;
};

// The chunk form of the per-key-channel gate addresses its per-(head, chunk)
// rows and matrices through 32-bit buffer offsets: each must stay below 4 GiB.
bool vg_chunk_fits(const gdn_dims* p) {
  const double lim = 4294967296.0;
  const double nc = static_cast<double>((p->T + 63) / 64);
  const double bhc = static_cast<double>(p->B) * p->Hv * nc;
  return bhc * 64.0 * p->Dk * 2.0 < lim && bhc * 64.0 * 64.0 * 2.0 < lim &&
         bhc * gdn::VSC_ROWS * 64.0 * 4.0 < lim;
}
bool vg_chunk_ok(const gdn_dims* p) {
  return gdn::vg_chunk_supported(static_cast<int>(p->Dk), static_cast<int>(p->Dv), p->dtype == GDN_BF16) &&
         vg_chunk_fits(p);
}
// Kernel family of a per-channel-gate call: the chunk form where asked for,
// and under AUTO where it is built and there is more than one step.
// (An empty sequence takes the scan path, which passes the state through.)
bool use_vg_chunk(const gdn_dims* p) {
  if (p->T == 0) return false;
  if (p->algo == GDN_ALGO_CHUNK) return true;
  if (p->algo == GDN_ALGO_SCAN) return false;
  return p->T > 1 && vg_chunk_ok(p);
}

// Under gdn_dims.save (chunk form) the checkpoint buffer holds the state at
// every chunk start (the initial state included) in bf16, the precision the
// gradient pass's products take it in, then the chunk rows and matrices the
// backward reads and X of every step, all written by the forward (offsets in
// fp32 elements, 256-byte aligned).  It holds no fp32 states.
struct VgSaved {
  size_t HB, Kb, Kh, KbT, QbT, Tx, PqT, vsc, X, total;
};

VgSaved vg_saved_layout(const Dims& d) {
  VgSaved S{};
  size_t off = 0;
  auto take = [&](size_t nfloat) {
    size_t o = off;
    off += align_up(nfloat * sizeof(float)) / sizeof(float);
    return o;
  };
  const size_t bhc = static_cast<size_t>(d.B) * d.Hv * d.nchunk();
  const size_t rows = (bhc * 64 * d.Dk + 1) / 2, mats = (bhc * 64 * 64 + 1) / 2;  // bf16, in floats
  S.HB = take((state_slots_elems(d) + 1) / 2);
  S.Kb = take(rows);
  S.Kh = take(rows);
  S.KbT = take(rows);
  S.QbT = take(rows);
  S.Tx = take(mats);
  S.PqT = take(mats);
  S.vsc = take(bhc * gdn::VSC_ROWS * 64);
  S.X = take((static_cast<size_t>(d.B) * d.T * d.Hv * d.Dv + 1) / 2);
  S.total = off;
  return S;
}
bool use_vg_saved(const gdn_dims* p) { return p->save != 0 && use_vg_chunk(p); }

// `saved`: the chunk rows, matrices and X live in the checkpoint buffer.
VgLayout vg_layout(const Dims& d, bool bwd, bool chunk, bool saved) {
  VgLayout L{};
  size_t off = 0;
  auto take = [&](size_t nfloat) {
    size_t o = off;
    off += align_up(nfloat * sizeof(float));
    return o;
  };
  const size_t bt = static_cast<size_t>(d.B) * d.T;
  if (chunk) {
    const size_t nc = d.nchunk(), bhc = static_cast<size_t>(d.B) * d.Hv * nc;
    const size_t rows = (bhc * 64 * d.Dk + 1) / 2, mats = (bhc * 64 * 64 + 1) / 2;  // bf16, in floats
    if (!saved) {
      L.Kb = take(rows);
      L.Kh = take(rows);
      L.Tx = take(mats);
      L.vsc = take(bhc * gdn::VSC_ROWS * 64);
    }
    if (!bwd) {
      L.Qb = take(rows);
      L.Mq = take(mats);
      L.total = off;
      return L;
    }
    if (!saved) {
      L.KbT = take(rows);
      L.QbT = take(rows);
      L.PqT = take(mats);
      L.X = take((bt * d.Hv * d.Dv + 1) / 2);
    }
    L.dPA = take(2 * mats);
  }
  L.rq = take(bt * d.Hk);
  L.rk = take(bt * d.Hk);
  L.kq = take(bt * d.Hk);
  L.beta = take(bt * d.Hv);
  if (bwd && chunk) {  // dH', and the value heads' parts of the row gradients
    const size_t nc = d.nchunk();
    L.dHend = take((nc * d.B * d.Hv * static_cast<size_t>(d.Dk) * d.Dv + 1) / 2);
    L.part = take((bt * d.Hv * 2 * d.Dk + 1) / 2);  // bf16
  } else if (bwd) {
    const size_t ns = gdn::vg_nslice(d.Dv);
    L.sub = take(gdn::vg_sub_floats(d));
    L.part = take(bt * d.Hv * ns * 3 * d.Dk);
    L.pdb = take(bt * d.Hv * ns);
  }
  L.total = off;
  return L;
}

gdn::StepScalars vg_scalars(void* ws, const VgLayout& L) {
  return gdn::StepScalars{at<float>(ws, L.rq), at<float>(ws, L.rk), at<float>(ws, L.kq), nullptr,
                          at<float>(ws, L.beta)};
}

// The chunk buffers in the workspace, or (saved) in the checkpoint buffer;
// under save the forward's Qb and Mq stay in its workspace, and cb.Hb and
// cb.X are set, so that the forward's state pass stores the bf16 chunk-start
// states and X there.
gdn::ChunkBufs vg_chunk_bufs(void* ws, const VgLayout& L, bool bwd, const Dims& d, const float* ckpt,
                             bool saved) {
  gdn::ChunkBufs cb{};
  if (saved) {
    const VgSaved S = vg_saved_layout(d);
    float* rec = const_cast<float*>(ckpt);
    cb.Hb = reinterpret_cast<gdn::bf16*>(rec + S.HB);
    cb.Kb = reinterpret_cast<gdn::bf16*>(rec + S.Kb);
    cb.Kh = reinterpret_cast<gdn::bf16*>(rec + S.Kh);
    cb.KbT = reinterpret_cast<gdn::bf16*>(rec + S.KbT);
    cb.QbT = reinterpret_cast<gdn::bf16*>(rec + S.QbT);
    cb.Tx = reinterpret_cast<gdn::bf16*>(rec + S.Tx);
    cb.PqT = reinterpret_cast<gdn::bf16*>(rec + S.PqT);
    cb.vsc = rec + S.vsc;
    cb.X = reinterpret_cast<gdn::bf16*>(rec + S.X);
  } else {
    cb.Kb = at<gdn::bf16>(ws, L.Kb);
    cb.Kh = at<gdn::bf16>(ws, L.Kh);
    cb.Tx = at<gdn::bf16>(ws, L.Tx);
    cb.vsc = at<float>(ws, L.vsc);
    if (bwd) {
      cb.KbT = at<gdn::bf16>(ws, L.KbT);
      cb.QbT = at<gdn::bf16>(ws, L.QbT);
      cb.PqT = at<gdn::bf16>(ws, L.PqT);
    }
  }
  if (!bwd) {
    cb.Qb = at<gdn::bf16>(ws, L.Qb);
    cb.Mq = at<gdn::bf16>(ws, L.Mq);
  }
  return cb;
}

int check_vg(const gdn_dims* p, Dims* out) {
  if (p && p->algo == GDN_ALGO_CHUNK_TPAR) return GDN_ERR_UNSUPPORTED;
  if (p && p->algo == GDN_ALGO_CHUNK && !vg_chunk_ok(p)) return GDN_ERR_UNSUPPORTED;
  gdn_dims q;
  if (p) {  // the scalar checks, without the scalar chunk form's own limits
    q = *p;
    if (q.algo == GDN_ALGO_CHUNK) q.algo = GDN_ALGO_SCAN;
  }
  int rc = check_dims(p ? &q : nullptr, out);
  if (rc) return rc;
  if (static_cast<double>(p->B) * p->T * p->Hv * p->Dk > static_cast<double>(INT_MAX))
    return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_ckpt_elems(const gdn_dims* d, size_t* out) {
  Dims dd;
  int rc = check_dims(d, &dd);
  if (rc) return rc;
  if (!out) return GDN_ERR_INVALID_ARG;
  *out = use_saved(d) ? saved_layout(dd).total : ckpt_state_elems(dd);
  return GDN_OK;
}

int gdn_ckpt_bytes(const gdn_dims* d, size_t* out) {
  size_t n = 0;
  const int rc = gdn_ckpt_elems(d, &n);
  if (rc) return rc;
  *out = n * sizeof(float);
  return GDN_OK;
}

int gdn_workspace_bytes(const gdn_dims* d, int for_bwd, size_t* out) {
  return for_bwd ? gdn_bwd_workspace_bytes(d, out) : gdn_fwd_workspace_bytes(d, out);
}

int gdn_fwd_workspace_bytes(const gdn_dims* d, size_t* out) {
  Dims dd;
  int rc = check_dims(d, &dd);
  if (rc) return rc;
  if (!out) return GDN_ERR_INVALID_ARG;
  *out = layout(dd, false, use_chunk_fwd(d), use_saved(d), tpar_seg(d, dd)).total;
  return GDN_OK;
}

int gdn_bwd_workspace_bytes(const gdn_dims* d, size_t* out) {
  Dims dd;
  int rc = check_dims(d, &dd);
  if (rc) return rc;
  if (!out) return GDN_ERR_INVALID_ARG;
  *out = layout(dd, true, use_chunk_bwd(d), use_saved(d), use_chunk_bwd(d) ? tpar_seg(d, dd) : 0).total;
  return GDN_OK;
}

}  // extern "C"

namespace {

// The forward's route and workspace layout for these dims and pointers.  An
// in-place update (state_out == state0) runs the single pass: in the
// T-parallel output pass the first segment's workgroups read state0 while the
// last segment's write state_out, with nothing ordering the two.
struct FwdRoute {
  bool chunk;
  int tseg;
  Layout L;
};
FwdRoute fwd_route(const gdn_dims* d, const Dims& dd, const float* state0, const float* state_out) {
  FwdRoute r{};
  r.chunk = use_chunk_fwd(d);
  const bool in_place = state0 != nullptr && state0 == state_out;
  r.tseg = r.chunk && !in_place ? tpar_seg(d, dd) : 0;
  r.L = layout(dd, false, r.chunk, use_saved(d), r.tseg);
  return r;
}

// Pointer checks of gdn_fwd (after check_dims).
int check_fwd_ptrs(const gdn_dims* d, const Dims& dd, const void* q, const void* k, const void* v,
                   const void* a, const void* b, const float* A_log, const float* dt_bias, const void* o,
                   const float* state_out, const float* ckpt) {
  const bool has_t = dd.T > 0;
  if (!A_log || !dt_bias || !state_out) return GDN_ERR_INVALID_ARG;
  if (has_t && (!q || !k || !v || !a || !b || !o)) return GDN_ERR_INVALID_ARG;
  if (use_saved(d) && !ckpt) return GDN_ERR_INVALID_ARG;  // the matrices are saved there
  return GDN_OK;
}

// gdn_fwd after validation: enqueues the route's kernels with the workspace ws.
int fwd_launch(const gdn_dims* d, const Dims& dd, const FwdRoute& R, const void* q, const void* k,
               const void* v, const void* a, const void* b, const float* A_log, const float* dt_bias,
               const float* state0, const uint8_t* mask, void* o, float* state_out, float* ckpt,
               void* ws, void* stream) {
  const bool chunk = R.chunk;
  const int tseg = R.tseg;
  const Layout& L = R.L;
  const bool bf = d->dtype == GDN_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const gdn::StepScalars s = scalars(ws, L);

  if (chunk) {
    gdn::ChunkBufs cb = chunk_bufs(ws, L, false);
    // under save chunk_prep also writes the backward's matrices, into the
    // checkpoint tail
    const bool save = use_saved(d);
    if (save) saved_bufs(dd, ckpt, cb);
    gdn::ChunkPrepArgs ca{dd, q, k, a, b, A_log, dt_bias, mask, cb, save ? 2 : 0};
    if (!launch(st, [&] { return gdn::launch_chunk_prep(ca, st); })) return GDN_ERR_HIP;
    // under save the states go to the checkpoint buffer as bf16 only
    gdn::ChunkFwdArgs fa{dd, q, k, v, state0, cb, o, state_out, save ? nullptr : ckpt};
    fa.stream = stream_handoff(dd);
    if (tseg) {  // T-parallel: segment maps, their chain, then every segment's outputs
      const int nseg = gdn::tpar_nseg(dd, tseg);
      float* maps = at<float>(ws, L.maps);
      float* hseg = at<float>(ws, L.hseg);
      float* vz = at<float>(ws, L.vzero);
      if (!launch(st, [&] { return gdn::launch_fill_zero(vz, 64, st); })) return GDN_ERR_HIP;
      gdn::ChunkBufs mcb = cb;
      mcb.Hb = nullptr;
      mcb.X = nullptr;
      gdn::ChunkFwdArgs ma{dd, q, k, v, nullptr, mcb, nullptr, nullptr, nullptr,
                           tseg, 1, nullptr, maps, reinterpret_cast<const gdn::bf16*>(vz)};
      if (!launch(st, [&] { return gdn::launch_chunk_fwd(ma, st); })) return GDN_ERR_HIP;
      gdn::SegChainArgs sa{dd, nseg, state0, maps, hseg, 0};
      if (!launch(st, [&] { return gdn::launch_seg_chain(sa, st); })) return GDN_ERR_HIP;
      fa.seg = tseg;
      fa.hseg = hseg;
    }
    if (!launch(st, [&] { return gdn::launch_chunk_fwd(fa, st); })) return GDN_ERR_HIP;
    return GDN_OK;
  }
  if (dd.T == 1 && gdn::decode_supported(dd.Dk, dd.Dv)) {  // one token: the fused single-step kernel
    gdn::DecodeArgs da{dd, q, k, v, a, b, A_log, dt_bias, state0, mask, o, state_out};
    if (!launch(st, [&] { return gdn::launch_decode(da, bf, st); })) return GDN_ERR_HIP;
    return GDN_OK;
  }
  gdn::PrepArgs pa{dd, q, k, a, b, A_log, dt_bias, mask, s};
  if (!launch(st, [&] { return gdn::launch_prep(pa, bf, st); })) return GDN_ERR_HIP;
  gdn::ScanFwdArgs fa{dd, q, k, v, state0, s, o, state_out, ckpt};
  if (!launch(st, [&] { return gdn::launch_scan_fwd(fa, bf, st); })) return GDN_ERR_HIP;
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_fwd(const gdn_dims* d, const void* q, const void* k, const void* v, const void* a,
            const void* b, const float* A_log, const float* dt_bias, const float* state0,
            const uint8_t* mask, void* o, float* state_out, float* ckpt, void* ws,
            size_t ws_bytes, void* stream) {
  Dims dd;
  int rc = check_dims(d, &dd);
  if (rc) return rc;
  rc = check_fwd_ptrs(d, dd, q, k, v, a, b, A_log, dt_bias, o, state_out, ckpt);
  if (rc) return rc;
  const FwdRoute R = fwd_route(d, dd, state0, state_out);
  if (R.L.total > ws_bytes || (R.L.total > 0 && !ws)) return GDN_ERR_WORKSPACE;
  return fwd_launch(d, dd, R, q, k, v, a, b, A_log, dt_bias, state0, mask, o, state_out, ckpt, ws, stream);
}

}  // extern "C"

// ---- the forward without a workspace argument (gdn_fwd_noalloc)
//
// Its workspace is this file-scope device array, one copy per GPU (held until
// the process ends).  In host code `scratch` names a host-side stand-in, not
// device memory: kernels get the device address that hipGetSymbolAddress
// returns for the current device, taken once per device on the first call.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// This device's copy of `scratch` (the current device's), or null if HIP
// cannot name it.
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int gdn_fwd_noalloc(const gdn_dims* d, const void* q, const void* k, const void* v, const void* a,
                    const void* b, const float* A_log, const float* dt_bias, const float* state0,
                    const uint8_t* mask, void* o, float* state_out, float* ckpt, void* stream) {
  Dims dd;
  int rc = check_dims(d, &dd);
  if (rc) return rc;
  rc = check_fwd_ptrs(d, dd, q, k, v, a, b, A_log, dt_bias, o, state_out, ckpt);
  if (rc) return rc;
  const FwdRoute R = fwd_route(d, dd, state0, state_out);
  if (R.L.total > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (R.L.total > 0) {
    ws = scratch_of_current_device();
    if (!ws) return GDN_ERR_HIP;
  }
  return fwd_launch(d, dd, R, q, k, v, a, b, A_log, dt_bias, state0, mask, o, state_out, ckpt, ws, stream);
}

int gdn_bwd(const gdn_dims* d, const void* q, const void* k, const void* v, const void* a,
            const void* b, const float* A_log, const float* dt_bias, const float* state0,
            const uint8_t* mask, const float* ckpt, const void* dO, const float* dS_final,
            void* dq, void* dk, void* dv, void* da, void* db, float* dA_log, float* ddt_bias,
            float* dstate, void* ws, size_t ws_bytes, void* stream) {
  Dims dd;
  int rc = check_dims(d, &dd);
  if (rc) return rc;
  const bool has_t = dd.T > 0;
  if (!A_log || !dt_bias || !dA_log || !ddt_bias || !dstate) return GDN_ERR_INVALID_ARG;
  if (has_t && (!q || !k || !v || !a || !b || !dO || !dq || !dk || !dv || !da || !db))
    return GDN_ERR_INVALID_ARG;
  if ((dd.nchunk() > 1 || use_saved(d)) && !ckpt) return GDN_ERR_INVALID_ARG;
  const bool chunk = use_chunk_bwd(d);
  const int tseg = chunk ? tpar_seg(d, dd) : 0;
  const Layout L = layout(dd, true, chunk, use_saved(d), tseg);
  if (L.total > ws_bytes || (L.total > 0 && !ws)) return GDN_ERR_WORKSPACE;
  const bool bf = d->dtype == GDN_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const gdn::StepScalars s = scalars(ws, L);

  gdn::ParamReduceArgs ra{dd.B, dd.nchunk(), dd.Hv, at<double>(ws, L.pdA), at<double>(ws, L.pdt),
                          dA_log, ddt_bias};
  if (chunk) {
    gdn::ChunkBufs cb = chunk_bufs(ws, L, true);
    if (use_saved(d)) {  // the forward saved the chunk matrices
      saved_bufs(dd, ckpt, cb);
    } else {
      gdn::ChunkPrepArgs ca{dd, q, k, a, b, A_log, dt_bias, mask, cb, 1};
      if (!launch(st, [&] { return gdn::launch_chunk_prep(ca, st); })) return GDN_ERR_HIP;
      cb.Hb = at<gdn::bf16>(ws, L.HB);
      gdn::StateBf16Args sa{dd.nchunk(), static_cast<size_t>(dd.B) * dd.Hv * dd.Dk * dd.Dv, dd.Dk, dd.Dv, state0, ckpt, cb.Hb};
      if (!launch(st, [&] { return gdn::launch_state_bf16(sa, st); })) return GDN_ERR_HIP;
    }
    gdn::ChunkBwdArgs ba{dd, q, k, v, dO, a, A_log, dt_bias, mask, state0, ckpt, dS_final, cb,
                         at<gdn::bf16>(ws, L.dHend),
                         dq, dk, dv, da, db, dstate, at<double>(ws, L.pdA), at<double>(ws, L.pdt)};
    ba.stream = stream_handoff(dd);
    if (tseg) {  // T-parallel reverse pass: segment maps, their chain (last to first), then the segments
      const int nseg = gdn::tpar_nseg(dd, tseg);
      float* maps = at<float>(ws, L.maps);
      float* hseg = at<float>(ws, L.hseg);
      float* vz = at<float>(ws, L.vzero);
      if (!launch(st, [&] { return gdn::launch_fill_zero(vz, 64, st); })) return GDN_ERR_HIP;
      gdn::ChunkBwdArgs ma = ba;
      ma.map = 1;
      ma.seg = tseg;
      ma.maps = maps;
      ma.vzero = reinterpret_cast<const gdn::bf16*>(vz);
      if (!launch(st, [&] { return gdn::launch_chunk_bwd_state(ma, st); })) return GDN_ERR_HIP;
      gdn::SegChainArgs sa{dd, nseg, dS_final, maps, hseg, 1};
      if (!launch(st, [&] { return gdn::launch_seg_chain(sa, st); })) return GDN_ERR_HIP;
      ba.seg = tseg;
      ba.hseg = hseg;
    }
    if (!launch(st, [&] { return gdn::launch_chunk_bwd_state(ba, st); })) return GDN_ERR_HIP;
    if (!launch(st, [&] { return gdn::launch_chunk_bwd_grad(ba, st); })) return GDN_ERR_HIP;
    if (!launch(st, [&] { return gdn::launch_param_reduce(ra, st); })) return GDN_ERR_HIP;
    return GDN_OK;
  }
  gdn::PrepArgs pa{dd, q, k, a, b, A_log, dt_bias, mask, s};
  if (!launch(st, [&] { return gdn::launch_prep(pa, bf, st); })) return GDN_ERR_HIP;
  gdn::ScanBwdArgs ba{dd, q, k, v, dO, state0, ckpt, dS_final, s,
                      at<float>(ws, L.U), at<float>(ws, L.E), dv, at<float>(ws, L.dHend), dstate};
  if (!launch(st, [&] { return gdn::launch_scan_bwd(ba, bf, st); })) return GDN_ERR_HIP;
  gdn::ChunkGradArgs ca{dd, q, k, v, dO, a, A_log, dt_bias, mask, state0, ckpt, s,
                        at<float>(ws, L.U), at<float>(ws, L.E), at<float>(ws, L.dHend),
                        dq, dk, da, db, at<double>(ws, L.pdA), at<double>(ws, L.pdt)};
  if (!launch(st, [&] { return gdn::launch_chunk_grad(ca, bf, st); })) return GDN_ERR_HIP;
  if (!launch(st, [&] { return gdn::launch_param_reduce(ra, st); })) return GDN_ERR_HIP;
  return GDN_OK;
}

int gdn_decode_conv(const gdn_dims* d, const void* x, const void* conv_w, const void* conv_state,
                    void* conv_state_out, int32_t conv_k, const void* a, const void* b,
                    const float* A_log, const float* dt_bias, const float* state0,
                    const uint8_t* mask, void* o, float* state_out, void* stream) {
  Dims dd;
  int rc = check_dims(d, &dd);
  if (rc) return rc;
  if (dd.T != 1) return GDN_ERR_INVALID_ARG;
  if (conv_k < 1 || conv_k > gdn::kMaxConvTaps) return GDN_ERR_INVALID_ARG;
  if (!x || !conv_w || !conv_state || !conv_state_out || !a || !b || !A_log || !dt_bias || !o || !state_out)
    return GDN_ERR_INVALID_ARG;
  if (!gdn::decode_supported(dd.Dk, dd.Dv) || gdn::conv_lds_bytes(dd) > gdn::kMaxConvLds)
    return GDN_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  gdn::DecodeConvArgs ca{dd, x, conv_w, conv_state, conv_state_out, conv_k, a, b, A_log, dt_bias,
                         state0, mask, o, state_out};
  if (!launch(st, [&] { return gdn::launch_decode_conv(ca, d->dtype == GDN_BF16, st); })) return GDN_ERR_HIP;
  return GDN_OK;
}

int gdn_vg_ckpt_elems(const gdn_dims* d, size_t* out) {
  Dims dd;
  int rc = check_vg(d, &dd);
  if (rc) return rc;
  if (!out) return GDN_ERR_INVALID_ARG;
  *out = use_vg_saved(d) ? vg_saved_layout(dd).total : ckpt_state_elems(dd);
  return GDN_OK;
}

int gdn_vg_ckpt_bytes(const gdn_dims* d, size_t* out) {
  size_t n = 0;
  const int rc = gdn_vg_ckpt_elems(d, &n);
  if (rc) return rc;
  *out = n * sizeof(float);
  return GDN_OK;
}

int gdn_fwd_vg_workspace_bytes(const gdn_dims* d, size_t* out) {
  Dims dd;
  int rc = check_vg(d, &dd);
  if (rc) return rc;
  if (!out) return GDN_ERR_INVALID_ARG;
  *out = vg_layout(dd, false, use_vg_chunk(d), use_vg_saved(d)).total;
  return GDN_OK;
}

int gdn_bwd_vg_workspace_bytes(const gdn_dims* d, size_t* out) {
  Dims dd;
  int rc = check_vg(d, &dd);
  if (rc) return rc;
  if (!out) return GDN_ERR_INVALID_ARG;
  *out = vg_layout(dd, true, use_vg_chunk(d), use_vg_saved(d)).total;
  return GDN_OK;
}

int gdn_fwd_vg(const gdn_dims* d, const void* q, const void* k, const void* v, const float* lg,
               const void* b, const float* state0, const uint8_t* mask, void* o,
               float* state_out, float* ckpt, void* ws, size_t ws_bytes, void* stream) {
  Dims dd;
  int rc = check_vg(d, &dd);
  if (rc) return rc;
  if (!state_out) return GDN_ERR_INVALID_ARG;
  if (dd.T > 0 && (!q || !k || !v || !lg || !b || !o)) return GDN_ERR_INVALID_ARG;
  const bool chunk = use_vg_chunk(d), saved = use_vg_saved(d);
  if (saved && !ckpt) return GDN_ERR_INVALID_ARG;  // the record is written there
  const VgLayout L = vg_layout(dd, false, chunk, saved);
  if (L.total > ws_bytes || (L.total > 0 && !ws)) return GDN_ERR_WORKSPACE;
  const bool bf = d->dtype == GDN_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (chunk) {
    // under save the prep also writes the backward's rows and matrices, and
    // the state pass X, into the record; the fp32 states sit at its start
    const gdn::ChunkBufs cb = vg_chunk_bufs(ws, L, false, dd, ckpt, saved);
    gdn::VgChunkPrepArgs pa{dd, q, k, b, lg, mask, cb, saved ? 2 : 0};
    if (!launch(st, [&] { return gdn::launch_vg_chunk_prep(pa, st); })) return GDN_ERR_HIP;
    // under save the states go to the record as bf16 only
    gdn::ChunkFwdArgs fa{dd, q, k, v, state0, cb, o, state_out, saved ? nullptr : ckpt};
    fa.vg = 1;
    if (!launch(st, [&] { return gdn::launch_chunk_fwd(fa, st); })) return GDN_ERR_HIP;
    return GDN_OK;
  }
  const gdn::StepScalars s = vg_scalars(ws, L);
  gdn::PrepArgs pa{dd, q, k, nullptr, b, nullptr, nullptr, mask, s};
  if (!launch(st, [&] { return gdn::launch_prep(pa, bf, st); })) return GDN_ERR_HIP;
  gdn::ScanFwdArgs fa{dd, q, k, v, state0, s, o, state_out, ckpt, lg, mask};
  if (!launch(st, [&] { return gdn::launch_scan_fwd(fa, bf, st); })) return GDN_ERR_HIP;
  return GDN_OK;
}

int gdn_bwd_vg(const gdn_dims* d, const void* q, const void* k, const void* v, const float* lg,
               const void* b, const float* state0, const uint8_t* mask, const float* ckpt,
               const void* dO, const float* dS_final, void* dq, void* dk, void* dv, float* dlg,
               void* db, float* dstate, void* ws, size_t ws_bytes, void* stream) {
  Dims dd;
  int rc = check_vg(d, &dd);
  if (rc) return rc;
  if (!dstate) return GDN_ERR_INVALID_ARG;
  if (dd.T > 0 && (!q || !k || !v || !lg || !b || !dO || !dq || !dk || !dv || !dlg || !db))
    return GDN_ERR_INVALID_ARG;
  const bool chunk = use_vg_chunk(d), saved = use_vg_saved(d);
  if ((dd.nchunk() > 1 || saved) && !ckpt) return GDN_ERR_INVALID_ARG;
  const VgLayout L = vg_layout(dd, true, chunk, saved);
  if (L.total > ws_bytes || (L.total > 0 && !ws)) return GDN_ERR_WORKSPACE;
  const bool bf = d->dtype == GDN_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const gdn::StepScalars s = vg_scalars(ws, L);
  gdn::PrepArgs pa{dd, q, k, nullptr, b, nullptr, nullptr, mask, s};
  if (!launch(st, [&] { return gdn::launch_prep(pa, bf, st); })) return GDN_ERR_HIP;
  if (chunk) {
    const gdn::ChunkBufs cb = vg_chunk_bufs(ws, L, true, dd, ckpt, saved);
    if (!saved) {  // else the forward saved the rows and matrices
      gdn::VgChunkPrepArgs ca{dd, q, k, b, lg, mask, cb, 1};
      if (!launch(st, [&] { return gdn::launch_vg_chunk_prep(ca, st); })) return GDN_ERR_HIP;
    }
    gdn::bf16* dHend = at<gdn::bf16>(ws, L.dHend);
    gdn::ChunkBwdArgs ba{dd, q, k, v, dO, nullptr, nullptr, nullptr, mask, state0, ckpt, dS_final, cb,
                         dHend, dq, dk, dv, nullptr, db, dstate, nullptr, nullptr};
    ba.vg = 1;
    if (!launch(st, [&] { return gdn::launch_chunk_bwd_state(ba, st); })) return GDN_ERR_HIP;
    gdn::VgChunkGradArgs ga{dd, q, k, v, b, dO, lg, mask, state0, ckpt, s, cb, dHend, dv,
                            saved ? cb.X : at<gdn::bf16>(ws, L.X), at<gdn::bf16>(ws, L.dPA),
                            at<gdn::bf16>(ws, L.part), dq, dk, db, dlg, saved ? 1 : 0};
    if (!launch(st, [&] { return gdn::launch_vg_chunk_x(ga, st); })) return GDN_ERR_HIP;
    if (!launch(st, [&] { return gdn::launch_vg_chunk_grad(ga, st); })) return GDN_ERR_HIP;
    if (!launch(st, [&] { return gdn::launch_vg_norm_bwd(ga, st); })) return GDN_ERR_HIP;
    return GDN_OK;
  }
  gdn::ScanBwdVgArgs ba{dd, q, k, v, dO, lg, mask, state0, ckpt, dS_final, s,
                        at<float>(ws, L.sub), at<float>(ws, L.part), at<float>(ws, L.pdb), dv, dstate};
  if (!launch(st, [&] { return gdn::launch_scan_bwd_vg(ba, bf, st); })) return GDN_ERR_HIP;
  gdn::VgReduceArgs ra{dd, gdn::vg_nslice(dd.Dv), q, k, s, at<float>(ws, L.part), at<float>(ws, L.pdb),
                       dq, dk, db, dlg};
  if (!launch(st, [&] { return gdn::launch_vg_reduce(ra, bf, st); })) return GDN_ERR_HIP;
  return GDN_OK;
}

int gdn_set_kernel_events(void* const* events, int n) {
  if (events && n < 2) return GDN_ERR_INVALID_ARG;
  g_timing.ev = events;
  g_timing.n = events ? n : 0;
  g_timing.next = 0;
  return GDN_OK;
}

const char* gdn_status_string(int s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported shape, dtype or algorithm";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* gdn_version(void) { return "gdn-mi355x 0.1 (gfx950)"; }

}  // extern "C"
