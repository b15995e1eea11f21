// Host-side driver for the AddressSanitizer / UndefinedBehaviorSanitizer run
// of the CPU tests (tests/test_sanitizers.py): it links the C ABI's host code
// (argument validation, workspace layout, the state-blob format) and the fp64
// oracle, both built with the sanitizers, and drives every host path that
// needs no GPU: rejected calls of every entry point on canary buffers, blob
// validation on good and corrupted blobs, and small oracle runs.  The kernel
// launchers are stubs that abort: no rejected call may reach them.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../../gated_deltanet_layer_gdn_amd/csrc/gdn_internal.h"
#include "../../include/gdn.h"

extern "C" {
int oracle_conv_silu(int B, int64_t T, int C_ch, int W, int dtype, const void *x, const void *w,
                     const void *hist, double *out);
int oracle_conv_history_next(int B, int64_t T, int C_ch, int W, int dtype, const void *x,
                             const void *hist, void *hist_out);
int oracle_l2norm(int64_t n, int d, const double *in, double eps, double scale, double *out);
int oracle_recurrence(int B, int64_t T, int H_k, int H_v, int d_k, int d_v, const double *q,
                      const double *k, const double *v, const double *g, const double *beta,
                      const double *z, double *S, double *y, double *o);
int oracle_layer(int B, int64_t T, int H_k, int H_v, int d_k, int d_v, int W, int dtype,
                 double eps, double q_scale, const void *x, const void *z, const float *g,
                 const float *beta, const void *w, const void *hist, double *S, double *y,
                 const int32_t *tasks, int n_tasks, int nthreads);
int oracle_gated_rmsnorm(int64_t groups, int d, const double *o, const double *z, const double *w,
                         double eps, double *y);
}

// ---- launcher stubs: reaching one of them is a failure of the validation
namespace gdn {
[[noreturn]] static void reached(const char *f) {
  std::fprintf(stderr, "launcher %s reached by a call that should have been rejected\n", f);
  std::abort();
}
hipError_t noalloc_scratch(hipStream_t, void **) { reached("noalloc_scratch"); }
hipError_t launch_conv_plain(const Geom &, int64_t, const void *, const void *, void *, float *,
                             hipStream_t) { reached("conv_plain"); }
hipError_t launch_conv_prefill(const Geom &, const PrefillWs &, const void *, const void *,
                               const void *, char *, hipStream_t, const KernelEvents *) {
  reached("conv_prefill");
}
hipError_t launch_conv_roll(const Geom &, int64_t, const void *, void *, hipStream_t) {
  reached("conv_roll");
}
hipError_t launch_conv_step(const Geom &, int, const void *, const void *, void *, float *,
                            const int32_t *, const int32_t *, int, hipStream_t,
                            const KernelEvents *) {
  reached("conv_step");
}
hipError_t launch_decode(const Geom &, int, const float *, const void *, const float *,
                         const float *, float *, void *, int, const int32_t *, const int32_t *,
                         hipStream_t, const KernelEvents *) { reached("decode"); }
hipError_t launch_gated_rmsnorm(const Geom &, int64_t, const float *, const void *, const float *,
                                float, void *, hipStream_t) { reached("gated_rmsnorm"); }
size_t attn_ws_bytes(const AttnGeom &, int64_t, int64_t) { return 256; }
hipError_t launch_attn_prefill(const AttnGeom &, int64_t, int64_t, const void *, const void *,
                               const void *, void *, void *, int64_t, void *, void *,
                               hipStream_t) { reached("attn"); }
hipError_t launch_in_proj(const Geom &, int64_t, int, const void *, const void *, const float *,
                          const float *, void *, void *, float *, float *, hipStream_t) {
  reached("in_proj");
}
hipError_t launch_prefill_prep(const Geom &, const PrefillWs &, const float *, const float *,
                               char *, const void *, const void *, void *, hipStream_t,
                               const KernelEvents *) {
  reached("prep");
}
hipError_t launch_prefill_state(const Geom &, const PrefillWs &, const void *, float *, void *,
                                const char *, const void *, const void *, void *, hipStream_t,
                                const KernelEvents *) {
  reached("state");
}
}  // namespace gdn

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

// Host stand-ins for device buffers, filled with canary bytes.
struct Canary {
  std::vector<unsigned char> raw, snap;
  explicit Canary(size_t n) : raw(n + 256), snap() {
    for (size_t i = 0; i < raw.size(); ++i) raw[i] = static_cast<unsigned char>(i * 131 + 7);
    snap = raw;
  }
  void *p(size_t shift = 0) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(raw.data());
    return reinterpret_cast<void *>(((a + 255) & ~uintptr_t(255)) + shift);
  }
  bool unchanged() const { return raw == snap; }
};

static uint64_t fnv(const void *p, size_t n, uint64_t h = 0xcbf29ce484222325ull) {
  const unsigned char *c = static_cast<const unsigned char *>(p);
  for (size_t i = 0; i < n; ++i) h = (h ^ c[i]) * 0x100000001b3ull;
  return h;
}

static void boundary(const gdn_dims &d0) {
  gdn_dims d = d0;
  const int T = 20, C = 32;
  const size_t C_ch = 2 * d.H_k * d.d_k + d.H_v * d.d_v;
  const size_t ws = gdn_prefill_workspace_bytes(&d, T, C);
  EXPECT(ws > 0);
  Canary x(d.B * T * C_ch * 2), z(d.B * T * d.H_v * d.d_v * 2), g(d.B * T * d.H_v * 4),
      be(d.B * T * d.H_v * 4), w(C_ch * 4 * 2), hist(d.B * 3 * C_ch * 2),
      S(d.B * d.H_v * d.d_v * d.d_k * 4), y(d.B * T * d.H_v * d.d_v * 4), wsb(ws);
  auto pre = [&](int Tc, int Cc, void *yp, size_t wsn) {
    return gdn_prefill_chunked(&d, Tc, Cc, x.p(), z.p(), static_cast<const float *>(g.p()),
                               static_cast<const float *>(be.p()), w.p(), hist.p(),
                               static_cast<float *>(S.p()), yp, wsb.p(), wsn, nullptr);
  };
  EXPECT(pre(0, C, y.p(), ws) == GDN_ERR_INVALID_ARG);
  EXPECT(pre((1 << 24) + 1, C, y.p(), ws) == GDN_ERR_INVALID_ARG);
  EXPECT(pre(T, 48, y.p(), ws) == GDN_ERR_UNSUPPORTED);
  EXPECT(pre(T, C, x.p(), ws) == GDN_ERR_ALIAS);
  EXPECT(pre(T, C, y.p(2), ws) == GDN_ERR_ALIGNMENT);
  EXPECT(pre(T, C, y.p(), ws - 1) == GDN_ERR_WORKSPACE);
  EXPECT(gdn_prefill_chunked(nullptr, T, C, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr, nullptr, 0, nullptr) == GDN_ERR_INVALID_ARG);
  gdn_dims bad = d;
  bad.d_k = bad.d_v = 64;
  EXPECT(gdn_rec_state_bytes(&bad) == 0);
  bad = d;
  bad.l2_eps = NAN;
  EXPECT(gdn_conv_state_bytes(&bad) == 0);
  // decode, multi-token decode, varlen, the norm, the no-alloc step
  EXPECT(gdn_decode_step(&d, x.p(), z.p(), static_cast<const float *>(g.p()),
                         static_cast<const float *>(be.p()), w.p(), hist.p(),
                         static_cast<float *>(S.p()), z.p(), wsb.p(), ws, nullptr) == GDN_ERR_ALIAS);
  int32_t slots[64] = {0};
  EXPECT(gdn_decode_multi(&d, 5, x.p(), z.p(), static_cast<const float *>(g.p()),
                          static_cast<const float *>(be.p()), w.p(), hist.p(),
                          static_cast<float *>(S.p()), d.B, slots, nullptr, y.p(), wsb.p(), ws,
                          nullptr) == GDN_ERR_INVALID_ARG);
  EXPECT(gdn_decode_step_noalloc(&d, nullptr, z.p(), static_cast<const float *>(g.p()),
                                 static_cast<const float *>(be.p()), w.p(), hist.p(),
                                 static_cast<float *>(S.p()), y.p(), nullptr) == GDN_ERR_INVALID_ARG);
  int64_t cu[3] = {0, 7, 5};
  int32_t sl[2] = {0, 1};
  EXPECT(gdn_prefill_varlen_workspace_bytes(&d, cu, 64) == 0);
  cu[2] = 12;
  sl[1] = 0;
  gdn_dims dv = d;
  dv.B = 2;
  EXPECT(gdn_prefill_varlen(&dv, cu, 64, x.p(), z.p(), static_cast<const float *>(g.p()),
                            static_cast<const float *>(be.p()), w.p(), hist.p(),
                            static_cast<float *>(S.p()), 2, sl, y.p(), wsb.p(), ws,
                            nullptr) == GDN_ERR_INVALID_ARG);
  EXPECT(gdn_gated_rmsnorm(&d, 3, static_cast<const float *>(y.p()), z.p(), nullptr, -1.f, z.p(),
                           nullptr) == GDN_ERR_INVALID_ARG);
  EXPECT(gdn_in_proj(&d, T, 100, x.p(), w.p(), static_cast<const float *>(g.p()),
                     static_cast<const float *>(be.p()), y.p(), z.p(), static_cast<float *>(S.p()),
                     static_cast<float *>(hist.p()), nullptr) == GDN_ERR_UNSUPPORTED);  // hidden % 64
  EXPECT(x.unchanged() && z.unchanged() && g.unchanged() && be.unchanged() && w.unchanged() &&
         hist.unchanged() && S.unchanged() && y.unchanged() && wsb.unchanged());
  for (int c = -13; c <= 0; ++c) EXPECT(gdn_status_str(c) != nullptr);
}

static void blobs(const gdn_dims &d) {
  const size_t cb = gdn_conv_state_bytes(&d), rb = gdn_rec_state_bytes(&d);
  const size_t n = gdn_state_blob_bytes(&d);
  EXPECT(n == 128 + cb + rb);
  std::vector<unsigned char> blob(n, 0);
  for (size_t i = 128; i < n; ++i) blob[i] = static_cast<unsigned char>(i * 17);
  unsigned char *h = blob.data();
  std::memcpy(h, "GDNSTATE", 8);
  const uint32_t ver = 1, hb = 128;
  std::memcpy(h + 8, &ver, 4);
  std::memcpy(h + 12, &hb, 4);
  const int32_t f[8] = {d.B, d.H_k, d.H_v, d.d_k, d.d_v, d.W, d.in_dtype, GDN_F32};
  std::memcpy(h + 16, f, sizeof f);
  const uint64_t cb64 = cb, rb64 = rb, ps = fnv(h + 128, cb + rb);
  std::memcpy(h + 48, &cb64, 8);
  std::memcpy(h + 56, &rb64, 8);
  std::memcpy(h + 64, &ps, 8);
  const uint64_t hs = fnv(h, 72);
  std::memcpy(h + 72, &hs, 8);
  EXPECT(gdn_state_check(&d, blob.data(), n) == GDN_OK);
  EXPECT(gdn_state_check(&d, blob.data(), n - 1) == GDN_ERR_BLOB_SIZE);
  EXPECT(gdn_state_check(&d, blob.data(), 100) == GDN_ERR_BLOB_SIZE);
  for (size_t pos : {size_t(0), size_t(9), size_t(20), size_t(70), size_t(200), n - 1}) {
    std::vector<unsigned char> bad = blob;
    bad[pos] ^= 0x20;
    EXPECT(gdn_state_check(&d, bad.data(), n) != GDN_OK);
  }
  gdn_dims other = d;
  other.H_v *= 2;
  EXPECT(gdn_state_check(&other, blob.data(), n) != GDN_OK);
}

static void oracle_runs() {
  const int B = 2, T = 21, H_k = 2, H_v = 4, d = 16, W = 4;
  const int C_ch = 2 * H_k * d + H_v * d;
  std::mt19937 rng(3);
  std::normal_distribution<float> nd(0.f, 1.f);
  std::vector<float> x(B * T * C_ch), z(B * T * H_v * d), g(B * T * H_v), be(B * T * H_v),
      w(C_ch * W), hist(B * (W - 1) * C_ch), hn(B * (W - 1) * C_ch);
  for (auto &v : x) v = nd(rng);
  for (auto &v : z) v = nd(rng);
  for (auto &v : g) v = -std::log1p(std::exp(nd(rng)));
  for (auto &v : be) v = 1.f / (1.f + std::exp(-nd(rng)));
  for (auto &v : w) v = 0.5f * nd(rng);
  for (auto &v : hist) v = nd(rng);
  std::vector<double> S(B * H_v * d * d, 0.0), y(B * T * H_v * d), u(B * T * C_ch);
  EXPECT(oracle_layer(B, T, H_k, H_v, d, d, W, 0, 1e-6, 1.0, x.data(), z.data(), g.data(),
                      be.data(), w.data(), hist.data(), S.data(), y.data(), nullptr, 0, 4) == 0);
  for (double v : y) EXPECT(std::isfinite(v));
  std::vector<double> y2(y.size()), S2(S.size(), 0.0);
  EXPECT(oracle_layer(B, T, H_k, H_v, d, d, W, 0, 1e-6, 1.0, x.data(), nullptr, g.data(),
                      be.data(), w.data(), hist.data(), S2.data(), y2.data(), nullptr, 0, 1) == 0);
  EXPECT(S2 == S);  // the gate does not touch the state
  EXPECT(oracle_conv_silu(B, T, C_ch, W, 0, x.data(), w.data(), hist.data(), u.data()) == 0);
  EXPECT(oracle_conv_history_next(B, T, C_ch, W, 0, x.data(), hist.data(), hn.data()) == 0);
  EXPECT(std::memcmp(hn.data(), x.data() + (T - 3) * C_ch, 3 * C_ch * sizeof(float)) == 0);
  std::vector<double> nrm(u.size());
  EXPECT(oracle_l2norm(B * T * C_ch / d, d, u.data(), 1e-6, 1.0, nrm.data()) == 0);
  std::vector<double> q(B * T * H_k * d), k(q.size()), v(B * T * H_v * d), gd(g.begin(), g.end()),
      bd(be.begin(), be.end()), zd(z.begin(), z.end()), S3(S.size(), 0.0), y3(y.size()), o3(y.size());
  for (int bt = 0; bt < B * T; ++bt)
    for (int c = 0; c < H_k * d; ++c) {
      q[bt * H_k * d + c] = nrm[bt * C_ch + c];
      k[bt * H_k * d + c] = nrm[bt * C_ch + H_k * d + c];
    }
  for (int bt = 0; bt < B * T; ++bt)
    for (int c = 0; c < H_v * d; ++c) v[bt * H_v * d + c] = u[bt * C_ch + 2 * H_k * d + c];
  EXPECT(oracle_recurrence(B, T, H_k, H_v, d, d, q.data(), k.data(), v.data(), gd.data(),
                           bd.data(), zd.data(), S3.data(), y3.data(), o3.data()) == 0);
  std::vector<double> yn(y.size());
  EXPECT(oracle_gated_rmsnorm(B * T * H_v, d, o3.data(), zd.data(), nullptr, 1e-6, yn.data()) == 0);
  EXPECT(oracle_layer(-1, T, H_k, H_v, d, d, W, 0, 1e-6, 1.0, x.data(), z.data(), g.data(),
                      be.data(), w.data(), hist.data(), S.data(), y.data(), nullptr, 0, 1) == -1);
}

int main() {
  gdn_dims d{GDN_ABI_VERSION, 2, 2, 6, 16, 16, 4, GDN_BF16, GDN_F32, 1e-6f, 1.0f};
  boundary(d);
  blobs(d);
  gdn_dims d128{GDN_ABI_VERSION, 1, 16, 48, 128, 128, 4, GDN_BF16, GDN_F32, 1e-6f, 1.0f};
  blobs(d128);
  oracle_runs();
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("sanitized host paths: all checks passed\n");
  return 0;
}
