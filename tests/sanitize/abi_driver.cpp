// Host-side driver of the C ABI for the sanitizer build (AddressSanitizer +
// UndefinedBehaviorSanitizer on the host code, kernel launchers replaced by
// the stubs of host_stubs.cpp).  Over a grid of shapes, dtypes, kernel
// families and the saved record it checks:
//  - the size queries (checkpoint elements, fwd / bwd workspace bytes);
//  - gdn_fwd / gdn_bwd / gdn_fwd_vg / gdn_bwd_vg / gdn_decode_conv with the
//    workspace and checkpoint buffers malloc'ed at exactly the queried sizes
//    return GDN_OK and hand every kernel regions inside those buffers (the
//    stubs read both ends of each);
//  - one byte less of workspace gives GDN_ERR_WORKSPACE, a NULL required
//    pointer GDN_ERR_INVALID_ARG;
//  - gdn_fwd_noalloc refuses a workspace larger than its static array;
//  - invalid dims are refused.
// Exits 0 when every expectation holds; prints the first failure otherwise.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gdn.h"

extern "C" long gdn_stub_launches();

static int g_fail = 0;
#define EXPECT(cond, ...)                                  \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                        \
      fprintf(stderr, "\n");                               \
      g_fail = 1;                                          \
      return;                                              \
    }                                                      \
  } while (0)

// Placeholder device pointers for the tensors the stubs never read.
static void* fake(int i) { return reinterpret_cast<void*>(static_cast<uintptr_t>(0x100000u * (i + 1))); }

static void run_case(int64_t B, int64_t T, int64_t Hk, int64_t Hv, int64_t Dk, int64_t Dv, int dt, int algo, int save) {
  gdn_dims d = {B, T, Hk, Hv, Dk, Dv, dt, algo, save};
  size_t nck = 0, fws = 0, bws = 0;
  const int rc = gdn_ckpt_elems(&d, &nck);
  if (rc == GDN_ERR_UNSUPPORTED || rc == GDN_ERR_INVALID_ARG) {
    EXPECT(gdn_fwd_workspace_bytes(&d, &fws) == rc, "fwd query disagrees");
    EXPECT(gdn_bwd_workspace_bytes(&d, &bws) == rc, "bwd query disagrees");
    return;
  }
  EXPECT(rc == GDN_OK, "ckpt query rc %d", rc);
  EXPECT(gdn_fwd_workspace_bytes(&d, &fws) == GDN_OK, "fwd query");
  EXPECT(gdn_bwd_workspace_bytes(&d, &bws) == GDN_OK, "bwd query");
  unsigned char* wf = static_cast<unsigned char*>(malloc(fws ? fws : 1));
  unsigned char* wb = static_cast<unsigned char*>(malloc(bws ? bws : 1));
  float* ck = nck ? static_cast<float*>(malloc(nck * sizeof(float))) : nullptr;
  const void* q = fake(0); const void* k = fake(1); const void* v = fake(2);
  const void* a = fake(3); const void* b = fake(4);
  const float* Al = static_cast<const float*>(fake(5)); const float* dtb = static_cast<const float*>(fake(6));
  const float* s0 = static_cast<const float*>(fake(7));
  void* o = fake(8); float* so = static_cast<float*>(fake(9));
  const long before = gdn_stub_launches();
  int r = gdn_fwd(&d, q, k, v, a, b, Al, dtb, s0, nullptr, o, so, ck, fws ? wf : nullptr, fws, nullptr);
  EXPECT(r == GDN_OK, "gdn_fwd rc %d (B%ld T%ld Hk%ld Hv%ld Dk%ld Dv%ld dt%d algo%d save%d)", r, (long)B, (long)T,
         (long)Hk, (long)Hv, (long)Dk, (long)Dv, dt, algo, save);
  // in place (the single pass where the T-parallel route would run)
  r = gdn_fwd(&d, q, k, v, a, b, Al, dtb, so, nullptr, o, so, ck, fws ? wf : nullptr, fws, nullptr);
  EXPECT(r == GDN_OK, "gdn_fwd in place rc %d", r);
  if (fws) {
    r = gdn_fwd(&d, q, k, v, a, b, Al, dtb, s0, nullptr, o, so, ck, wf, fws - 1, nullptr);
    EXPECT(r == GDN_ERR_WORKSPACE, "short fwd workspace rc %d", r);
  }
  r = gdn_fwd(&d, q, k, v, a, b, nullptr, dtb, s0, nullptr, o, so, ck, wf, fws, nullptr);
  EXPECT(r == GDN_ERR_INVALID_ARG, "null A_log rc %d", r);
  if (fws > GDN_NOALLOC_SCRATCH_BYTES) {
    r = gdn_fwd_noalloc(&d, q, k, v, a, b, Al, dtb, s0, nullptr, o, so, ck, nullptr);
    EXPECT(r == GDN_ERR_WORKSPACE, "noalloc over its array rc %d", r);
  }
  void* g[5] = {fake(10), fake(11), fake(12), fake(13), fake(14)};
  float* dA = static_cast<float*>(fake(15)); float* ddt = static_cast<float*>(fake(16));
  float* dst = static_cast<float*>(fake(17));
  const void* dO = fake(18); const float* dSf = static_cast<const float*>(fake(19));
  r = gdn_bwd(&d, q, k, v, a, b, Al, dtb, s0, nullptr, ck, dO, dSf, g[0], g[1], g[2], g[3], g[4], dA, ddt, dst,
              bws ? wb : nullptr, bws, nullptr);
  EXPECT(r == GDN_OK, "gdn_bwd rc %d", r);
  r = gdn_bwd(&d, q, k, v, a, b, Al, dtb, s0, nullptr, ck, dO, dSf, g[0], g[1], g[2], g[3], g[4], dA, ddt, dst,
              wb, bws ? bws - 1 : 0, nullptr);
  EXPECT(bws == 0 || r == GDN_ERR_WORKSPACE, "short bwd workspace rc %d", r);
  EXPECT(T == 0 || gdn_stub_launches() > before, "nothing launched");
  // the per-key-channel gate (scan or chunk form, as the dims select)
  if (algo == GDN_ALGO_SCAN || algo == GDN_ALGO_AUTO || algo == GDN_ALGO_CHUNK) {
    size_t vf = 0, vb = 0;
    if (gdn_fwd_vg_workspace_bytes(&d, &vf) == GDN_OK && gdn_bwd_vg_workspace_bytes(&d, &vb) == GDN_OK) {
      gdn_dims ds = d;  // save as the case gives it: the chunk form's record, or the fp32 states
      size_t nvk = 0;
      gdn_vg_ckpt_elems(&ds, &nvk);
      float* vck = nvk ? static_cast<float*>(malloc(nvk * sizeof(float))) : nullptr;
      unsigned char* vwf = static_cast<unsigned char*>(malloc(vf ? vf : 1));
      unsigned char* vwb = static_cast<unsigned char*>(malloc(vb ? vb : 1));
      const float* lg = static_cast<const float*>(fake(20));
      r = gdn_fwd_vg(&ds, q, k, v, lg, b, s0, nullptr, o, so, vck, vf ? vwf : nullptr, vf, nullptr);
      if (r == GDN_OK)
        r = gdn_bwd_vg(&ds, q, k, v, lg, b, s0, nullptr, vck, dO, dSf, g[0], g[1], g[2], static_cast<float*>(g[3]),
                       g[4], dst, vb ? vwb : nullptr, vb, nullptr);
      free(vck);
      free(vwf);
      free(vwb);
      EXPECT(r == GDN_OK, "vg rc %d", r);
    }
  }
  if (T == 1) {
    const int K = 4;
    r = gdn_decode_conv(&d, fake(21), fake(22), fake(23), fake(23), K, a, b, Al, dtb, s0, nullptr, o, so, nullptr);
    EXPECT(r == GDN_OK || r == GDN_ERR_UNSUPPORTED, "decode_conv rc %d", r);
  }
  free(wf);
  free(wb);
  free(ck);
}

int main() {
  const int64_t shapes[][6] = {
      {1, 8, 2, 4, 16, 8},      {4, 65, 4, 8, 64, 32},   {4, 1024, 4, 8, 64, 32}, {1, 2048, 16, 64, 192, 128},
      {2, 200, 2, 4, 128, 64},  {1, 130, 2, 2, 256, 32}, {2, 150, 2, 8, 64, 96},  {1, 32768, 2, 4, 128, 128},
      {1, 4096, 1, 1, 64, 32},  {2, 3000, 2, 4, 64, 32}, {2, 0, 1, 2, 16, 8},     {3, 1, 1, 3, 32, 16},
      {64, 1, 16, 32, 128, 128}, {3, 70, 1, 3, 32, 16},  {2, 77, 2, 4, 192, 24},  {1, 64, 1, 1, 256, 256},
  };
  const int nshape = sizeof(shapes) / sizeof(shapes[0]);
  for (int s = 0; s < nshape; ++s)
    for (int dt = 0; dt < 2; ++dt)
      for (int algo = 0; algo < 4; ++algo)
        for (int save = 0; save < 2; ++save) {
          run_case(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], shapes[s][4], shapes[s][5], dt, algo, save);
          if (g_fail) return 1;
        }
  // invalid dims are refused by every query
  const int64_t bad[][6] = {{1, 8, 3, 4, 16, 8}, {0, 8, 2, 4, 16, 8}, {1, -1, 2, 4, 16, 8}, {1, 8, 2, 4, 48, 8},
                            {64, 65536, 4, 8, 64, 32}};
  for (int i = 0; i < 5; ++i) {
    gdn_dims d = {bad[i][0], bad[i][1], bad[i][2], bad[i][3], bad[i][4], bad[i][5], GDN_BF16, GDN_ALGO_CHUNK, 0};
    size_t x;
    if (gdn_fwd_workspace_bytes(&d, &x) == GDN_OK) {
      fprintf(stderr, "FAIL: invalid dims %d accepted\n", i);
      return 1;
    }
  }
  printf("ok: %ld stub launches\n", gdn_stub_launches());
  return 0;
}
