// gdn_api.cpp -- the C ABI of libgdn.so: argument validation, workspace
// layout, the state blob, and the launch sequence of each entry point.
//
// Every check runs before anything is enqueued, so an error leaves every
// caller byte unchanged ("Implement the Qwen3.8 Flash Next Rust and Metal
// text core", implementation comment: fail before unsafe or partial
// execution, without mutating session state).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

thread_local std::string g_last_hip_error;

constexpr int64_t kMaxTokens = int64_t(1) << 28;  // keeps every per-call index in range
constexpr int kMaxBatch = 65535;                  // grid z / y limits

int set_hip_error(hipError_t e, const char *where) {
  g_last_hip_error = std::string(where) + ": " + hipGetErrorString(e);
  return GDN_ERR_HIP;
}

size_t esize(int dt) { return dt == GDN_F32 ? 4 : 2; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Validate dims and fill the kernel geometry.
int check_dims(const gdn_dims *d, Geom *g) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->abi != GDN_ABI_VERSION) return GDN_ERR_UNSUPPORTED;
  if (d->B < 1 || d->B > kMaxBatch || d->H_k < 1 || d->H_v < 1 || d->d_k < 1 || d->d_v < 1 ||
      d->W < 1)
    return GDN_ERR_INVALID_ARG;
  if (d->H_v % d->H_k) return GDN_ERR_UNSUPPORTED;
  if (d->d_k != d->d_v || (d->d_k != 16 && d->d_k != 128)) return GDN_ERR_UNSUPPORTED;
  if (d->W != 4) return GDN_ERR_UNSUPPORTED;
  if ((d->in_dtype != GDN_F32 && d->in_dtype != GDN_BF16) ||
      (d->out_dtype != GDN_F32 && d->out_dtype != GDN_BF16))
    return GDN_ERR_UNSUPPORTED;
  if (!(d->l2_eps >= 0.f) || !(d->l2_eps < 1e30f)) return GDN_ERR_INVALID_ARG;
  if (!(d->q_scale > -1e30f && d->q_scale < 1e30f)) return GDN_ERR_INVALID_ARG;
  const int64_t heads = static_cast<int64_t>(2) * d->H_k + d->H_v;
  if (heads * d->d_k > (int64_t(1) << 24)) return GDN_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(d->B) * d->H_v * (d->d_v / 16) > (int64_t(1) << 30))
    return GDN_ERR_UNSUPPORTED;
  g->B = d->B;
  g->H_k = d->H_k;
  g->H_v = d->H_v;
  g->D = d->d_k;
  g->W = d->W;
  g->G = d->H_v / d->H_k;
  g->C_ch = static_cast<int>(heads * d->d_k);
  g->in_dt = d->in_dtype;
  g->out_dt = d->out_dtype;
  g->eps = d->l2_eps;
  g->q_scale = d->q_scale;
  return GDN_OK;
}

struct Buf {
  const void *p;
  size_t n;
  size_t align;  // required alignment in bytes
};

bool overlaps(const Buf &a, const Buf &b) {
  if (!a.n || !b.n) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Null and alignment checks, then: no written buffer may overlap any other
// buffer (read-only inputs may overlap each other).
int check_buffers(const Buf *in, int n_in, const Buf *out, int n_out) {
  for (int i = 0; i < n_in + n_out; ++i) {
    const Buf &b = i < n_in ? in[i] : out[i - n_in];
    if (!b.p) return GDN_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(b.p) % b.align) return GDN_ERR_ALIGNMENT;
  }
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(out[i], in[j])) return GDN_ERR_ALIAS;
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(out[i], out[j])) return GDN_ERR_ALIAS;
  }
  return GDN_OK;
}

bool injected_launch_failure() {
  const char *e = std::getenv("GDN_TEST_FAIL_LAUNCH");
  if (e && *e && *e != '0') {
    g_last_hip_error = "injected launch failure (GDN_TEST_FAIL_LAUNCH)";
    return true;
  }
  return false;
}

uint64_t fnv1a64(const void *p, size_t n, uint64_t h = 0xcbf29ce484222325ull) {
  const unsigned char *c = static_cast<const unsigned char *>(p);
  for (size_t i = 0; i < n; ++i) {
    h ^= c[i];
    h *= 0x100000001b3ull;
  }
  return h;
}

constexpr size_t kBlobHeader = 128;
constexpr uint32_t kBlobVersion = 1;
const char kMagic[8] = {'G', 'D', 'N', 'S', 'T', 'A', 'T', 'E'};

struct BlobHeader {
  char magic[8];
  uint32_t version, header_bytes;
  int32_t B, H_k, H_v, d_k, d_v, W;
  int32_t conv_dtype, rec_dtype;
  uint64_t conv_bytes, rec_bytes;
  uint64_t payload_sum, header_sum;
  unsigned char pad[48];
};
static_assert(sizeof(BlobHeader) == kBlobHeader, "blob header is 128 bytes");

size_t conv_state_bytes(const Geom &g) {
  return static_cast<size_t>(g.B) * (g.W - 1) * g.C_ch * esize(g.in_dt);
}
size_t rec_state_bytes(const Geom &g) {
  return static_cast<size_t>(g.B) * g.H_v * g.D * g.D * 4;
}

// Optional HIP events around each launch of one call, for the timed entry
// points.  Records on the caller's stream; elapsed() waits for the last one.
struct LaunchTimer {
  float *out;
  int n = 0;
  hipEvent_t ev[8] = {};
  explicit LaunchTimer(float *o) : out(o) {}
  ~LaunchTimer() {
    for (int i = 0; i < n; ++i) (void)hipEventDestroy(ev[i]);
  }
  hipError_t mark(hipStream_t s) {
    if (!out) return hipSuccess;
    hipError_t e = hipEventCreate(&ev[n]);
    if (e != hipSuccess) return e;
    return hipEventRecord(ev[n++], s);
  }
  hipError_t elapsed() {
    if (!out) return hipSuccess;
    hipError_t e = hipEventSynchronize(ev[n - 1]);
    for (int i = 0; e == hipSuccess && i + 1 < n; ++i) e = hipEventElapsedTime(&out[i], ev[i], ev[i + 1]);
    return e;
  }
};

}  // namespace

bool prefill_ws_layout(const Geom &g, int64_t T, int C, PrefillWs *w) {
  if (T < 1 || T > kMaxTokens) return false;
  if (C != 16 && C != 32 && C != 64 && C != 128) return false;
  w->T = T;
  w->C = C;
  w->Cp = C < 32 ? 32 : C;
  w->Dp = g.D < 32 ? 32 : g.D;
  w->T_pad = static_cast<int64_t>(round_up(static_cast<size_t>(T), w->Cp));
  w->NC = static_cast<int>((T + C - 1) / C);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  const size_t tp = static_cast<size_t>(w->T_pad);
  const size_t tok = static_cast<size_t>(g.B) * g.H_k * tp * w->Dp * 2;
  // The split-role pass keeps the low halves of q, k and P as e4m3 bytes with
  // a power-of-two scale 2^(e - 15), where 2^e bounds the values: normalised k
  // is at most 1 in magnitude, q and P at most |q_scale|.  Validation keeps
  // |q_scale| below 1e30 < 2^100, so e <= 100; below 2^-100 the low halves of
  // q and P lose precision but cannot overflow.
  const bool split = prefill_split_roles(g, *w);
  const float qmax = std::fabs(g.q_scale);
  const int qe = qmax > 0.f ? std::max(-100, std::min(100, static_cast<int>(std::ceil(std::log2(qmax))))) : 0;
  w->q_lo_scale = split ? std::ldexp(1.0f, qe - 15) : 0.f;
  w->k_lo_scale = split ? std::ldexp(1.0f, -15) : 0.f;
  w->q_hi = take(tok);
  w->q_lo = take(split ? tok / 2 : tok);
  w->k_hi = take(tok);
  w->k_lo = take(split ? tok / 2 : tok);
  // The split-role state pass builds the dim-major k in LDS and computes v
  // from x: those regions are empty for it.
  const size_t kt = split ? 0 : static_cast<size_t>(g.B) * g.H_k * tp * g.D * 2;
  w->kT_hi = take(kt);
  w->kT_lo = take(kt);
  w->vT = take(split ? 0 : static_cast<size_t>(g.B) * g.H_v * tp * g.D * 4);
  const size_t mat = static_cast<size_t>(g.B) * g.H_v * w->NC * C * w->Cp * 2;
  w->Tm = take(mat);
  w->P_hi = take(mat);
  w->P_lo = take(split ? mat / 2 : mat);  // e4m3 low halves for the split-role pass
  w->gates = take(static_cast<size_t>(g.B) * g.H_v * w->NC * 4 * C * 4);
  w->total = off;
  return true;
}

size_t decode_ws_bytes(const Geom &g) {
  return round_up(static_cast<size_t>(g.B) * g.C_ch * 4, 256);
}

}  // namespace gdn

using namespace gdn;

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char *gdn_status_str(int s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported geometry, dtype or ABI version";
    case GDN_ERR_ALIGNMENT: return "device pointer misaligned";
    case GDN_ERR_ALIAS: return "output or workspace overlaps another buffer";
    case GDN_ERR_WORKSPACE: return "workspace too small";
    case GDN_ERR_BLOB_MAGIC: return "state blob: bad magic";
    case GDN_ERR_BLOB_VERSION: return "state blob: unsupported format version";
    case GDN_ERR_BLOB_SHAPE: return "state blob: dims or dtype mismatch";
    case GDN_ERR_BLOB_SIZE: return "state blob: size mismatch";
    case GDN_ERR_BLOB_CHECKSUM: return "state blob: checksum mismatch";
    case GDN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *gdn_last_hip_error(void) { return g_last_hip_error.c_str(); }

size_t gdn_rec_state_bytes(const gdn_dims *dims) {
  Geom g;
  return check_dims(dims, &g) == GDN_OK ? rec_state_bytes(g) : 0;
}

size_t gdn_conv_state_bytes(const gdn_dims *dims) {
  Geom g;
  return check_dims(dims, &g) == GDN_OK ? conv_state_bytes(g) : 0;
}

size_t gdn_state_blob_bytes(const gdn_dims *dims) {
  Geom g;
  return check_dims(dims, &g) == GDN_OK ? kBlobHeader + conv_state_bytes(g) + rec_state_bytes(g)
                                        : 0;
}

size_t gdn_prefill_workspace_bytes(const gdn_dims *dims, int64_t T, int32_t chunk) {
  Geom g;
  PrefillWs L;
  if (check_dims(dims, &g) != GDN_OK || !prefill_ws_layout(g, T, chunk, &L)) return 0;
  return L.total;
}

size_t gdn_decode_workspace_bytes(const gdn_dims *dims) {
  Geom g;
  return check_dims(dims, &g) == GDN_OK ? decode_ws_bytes(g) : 0;
}

int gdn_conv1d(const gdn_dims *dims, int64_t T, const void *x, const void *conv_w,
               void *conv_state, float *qkv_out, void *stream) {
  Geom g;
  int rc = check_dims(dims, &g);
  if (rc) return rc;
  if (T < 1 || T > kMaxTokens) return GDN_ERR_INVALID_ARG;
  const size_t es = esize(g.in_dt);
  const Buf in[] = {{x, static_cast<size_t>(g.B) * T * g.C_ch * es, es},
                    {conv_w, static_cast<size_t>(g.C_ch) * g.W * es, es}};
  const Buf out[] = {{conv_state, conv_state_bytes(g), es},
                     {qkv_out, static_cast<size_t>(g.B) * T * g.C_ch * 4, 4}};
  if ((rc = check_buffers(in, 2, out, 2))) return rc;
  if (injected_launch_failure()) return GDN_ERR_HIP;
  hipError_t e = launch_conv_plain(g, T, x, conv_w, conv_state, qkv_out,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : set_hip_error(e, "gdn_conv1d");
}

static int prefill_impl(const gdn_dims *dims, int64_t T, int32_t chunk, const void *x,
                        const void *z, const float *gl, const float *beta,
                        const void *conv_w, void *conv_state, float *rec_state, void *y,
                        void *ws, size_t ws_bytes, void *stream, float *kernel_ms) {
  Geom g;
  int rc = check_dims(dims, &g);
  if (rc) return rc;
  if (T < 1 || T > kMaxTokens) return GDN_ERR_INVALID_ARG;
  PrefillWs L;
  if (!prefill_ws_layout(g, T, chunk, &L)) return GDN_ERR_UNSUPPORTED;
  const size_t es = esize(g.in_dt), eo = esize(g.out_dt);
  const size_t bt = static_cast<size_t>(g.B) * T;
  // x and the conv history are read in 16-byte pieces by the state pass.
  const Buf in[] = {{x, bt * g.C_ch * es, 16},
                    {z, bt * g.H_v * g.D * es, 16},
                    {gl, bt * g.H_v * 4, 4},
                    {beta, bt * g.H_v * 4, 4},
                    {conv_w, static_cast<size_t>(g.C_ch) * g.W * es, es}};
  const Buf out[] = {{conv_state, conv_state_bytes(g), 16},
                     {rec_state, rec_state_bytes(g), 16},
                     {y, bt * g.H_v * g.D * eo, eo},
                     {ws, L.total, 16}};
  if ((rc = check_buffers(in, 5, out, 4))) return rc;
  if (ws_bytes < L.total) return GDN_ERR_WORKSPACE;
  if (injected_launch_failure()) return GDN_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *w = static_cast<char *>(ws);
  LaunchTimer tm(kernel_ms);
  hipError_t e = tm.mark(s);
  if (e == hipSuccess) e = launch_conv_prefill(g, L, x, conv_w, conv_state, w, s);
  if (e == hipSuccess) e = tm.mark(s);
  if (e == hipSuccess) e = launch_prefill_prep(g, L, gl, beta, w, x, conv_state, s);
  if (e == hipSuccess) e = tm.mark(s);
  if (e == hipSuccess) e = launch_prefill_state(g, L, z, rec_state, y, w, x, conv_w, conv_state, s);
  if (e == hipSuccess) e = tm.mark(s);
  if (e == hipSuccess) e = tm.elapsed();
  return e == hipSuccess ? GDN_OK : set_hip_error(e, "gdn_prefill_chunked");
}

int gdn_prefill_chunked(const gdn_dims *dims, int64_t T, int32_t chunk, const void *x,
                        const void *z, const float *gl, const float *beta,
                        const void *conv_w, void *conv_state, float *rec_state, void *y,
                        void *ws, size_t ws_bytes, void *stream) {
  return prefill_impl(dims, T, chunk, x, z, gl, beta, conv_w, conv_state, rec_state, y, ws,
                      ws_bytes, stream, nullptr);
}

int gdn_prefill_chunked_timed(const gdn_dims *dims, int64_t T, int32_t chunk, const void *x,
                              const void *z, const float *gl, const float *beta,
                              const void *conv_w, void *conv_state, float *rec_state, void *y,
                              void *ws, size_t ws_bytes, void *stream, float *kernel_ms) {
  if (!kernel_ms) return GDN_ERR_INVALID_ARG;
  return prefill_impl(dims, T, chunk, x, z, gl, beta, conv_w, conv_state, rec_state, y, ws,
                      ws_bytes, stream, kernel_ms);
}

static int decode_impl(const gdn_dims *dims, const void *x, const void *z, const float *gl,
                    const float *beta, const void *conv_w, void *conv_state,
                    float *rec_state, void *y, void *ws, size_t ws_bytes, void *stream,
                    float *kernel_ms) {
  Geom g;
  int rc = check_dims(dims, &g);
  if (rc) return rc;
  const size_t es = esize(g.in_dt), eo = esize(g.out_dt);
  const size_t B = static_cast<size_t>(g.B);
  const size_t need = decode_ws_bytes(g);
  const Buf in[] = {{x, B * g.C_ch * es, es},
                    {z, B * g.H_v * g.D * es, es},
                    {gl, B * g.H_v * 4, 4},
                    {beta, B * g.H_v * 4, 4},
                    {conv_w, static_cast<size_t>(g.C_ch) * g.W * es, es}};
  const Buf out[] = {{conv_state, conv_state_bytes(g), es},
                     {rec_state, rec_state_bytes(g), 16},
                     {y, B * g.H_v * g.D * eo, eo},
                     {ws, need, 16}};
  if ((rc = check_buffers(in, 5, out, 4))) return rc;
  if (ws_bytes < need) return GDN_ERR_WORKSPACE;
  if (injected_launch_failure()) return GDN_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *qkv = static_cast<float *>(ws);
  LaunchTimer tm(kernel_ms);
  hipError_t e = tm.mark(s);
  if (e == hipSuccess) e = launch_conv_plain(g, 1, x, conv_w, conv_state, qkv, s);
  if (e == hipSuccess) e = tm.mark(s);
  if (e == hipSuccess) e = launch_decode(g, qkv, z, gl, beta, rec_state, y, s);
  if (e == hipSuccess) e = tm.mark(s);
  if (e == hipSuccess) e = tm.elapsed();
  return e == hipSuccess ? GDN_OK : set_hip_error(e, "gdn_decode_step");
}

int gdn_decode_step(const gdn_dims *dims, const void *x, const void *z, const float *gl,
                    const float *beta, const void *conv_w, void *conv_state,
                    float *rec_state, void *y, void *ws, size_t ws_bytes, void *stream) {
  return decode_impl(dims, x, z, gl, beta, conv_w, conv_state, rec_state, y, ws, ws_bytes,
                     stream, nullptr);
}

int gdn_decode_step_timed(const gdn_dims *dims, const void *x, const void *z, const float *gl,
                          const float *beta, const void *conv_w, void *conv_state,
                          float *rec_state, void *y, void *ws, size_t ws_bytes, void *stream,
                          float *kernel_ms) {
  if (!kernel_ms) return GDN_ERR_INVALID_ARG;
  return decode_impl(dims, x, z, gl, beta, conv_w, conv_state, rec_state, y, ws, ws_bytes,
                     stream, kernel_ms);
}

int gdn_state_check(const gdn_dims *dims, const void *blob, size_t blob_bytes) {
  Geom g;
  int rc = check_dims(dims, &g);
  if (rc) return rc;
  if (!blob) return GDN_ERR_INVALID_ARG;
  if (blob_bytes < kBlobHeader) return GDN_ERR_BLOB_SIZE;
  BlobHeader h;
  std::memcpy(&h, blob, sizeof h);
  if (std::memcmp(h.magic, kMagic, 8)) return GDN_ERR_BLOB_MAGIC;
  if (h.version != kBlobVersion || h.header_bytes != kBlobHeader) return GDN_ERR_BLOB_VERSION;
  if (fnv1a64(&h, offsetof(BlobHeader, header_sum)) != h.header_sum) return GDN_ERR_BLOB_CHECKSUM;
  if (h.B != g.B || h.H_k != g.H_k || h.H_v != g.H_v || h.d_k != g.D || h.d_v != g.D ||
      h.W != g.W || h.conv_dtype != g.in_dt || h.rec_dtype != GDN_F32)
    return GDN_ERR_BLOB_SHAPE;
  const size_t cb = conv_state_bytes(g), rb = rec_state_bytes(g);
  if (h.conv_bytes != cb || h.rec_bytes != rb || blob_bytes != kBlobHeader + cb + rb)
    return GDN_ERR_BLOB_SIZE;
  const char *payload = static_cast<const char *>(blob) + kBlobHeader;
  if (fnv1a64(payload, cb + rb) != h.payload_sum) return GDN_ERR_BLOB_CHECKSUM;
  return GDN_OK;
}

int gdn_state_save(const gdn_dims *dims, const void *conv_state, const float *rec_state,
                   void *blob, size_t blob_bytes, void *stream) {
  Geom g;
  int rc = check_dims(dims, &g);
  if (rc) return rc;
  const size_t cb = conv_state_bytes(g), rb = rec_state_bytes(g);
  const Buf in[] = {{conv_state, cb, esize(g.in_dt)}, {rec_state, rb, 16}};
  if ((rc = check_buffers(in, 2, nullptr, 0))) return rc;
  if (!blob) return GDN_ERR_INVALID_ARG;
  if (blob_bytes != kBlobHeader + cb + rb) return GDN_ERR_BLOB_SIZE;
  if (injected_launch_failure()) return GDN_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *payload = static_cast<char *>(blob) + kBlobHeader;
  hipError_t e = hipMemcpyAsync(payload, conv_state, cb, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(payload + cb, rec_state, rb, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return set_hip_error(e, "gdn_state_save");
  BlobHeader h;
  std::memset(&h, 0, sizeof h);
  std::memcpy(h.magic, kMagic, 8);
  h.version = kBlobVersion;
  h.header_bytes = kBlobHeader;
  h.B = g.B;
  h.H_k = g.H_k;
  h.H_v = g.H_v;
  h.d_k = g.D;
  h.d_v = g.D;
  h.W = g.W;
  h.conv_dtype = g.in_dt;
  h.rec_dtype = GDN_F32;
  h.conv_bytes = cb;
  h.rec_bytes = rb;
  h.payload_sum = fnv1a64(payload, cb + rb);
  h.header_sum = fnv1a64(&h, offsetof(BlobHeader, header_sum));
  std::memcpy(blob, &h, sizeof h);
  return GDN_OK;
}

int gdn_state_restore(const gdn_dims *dims, const void *blob, size_t blob_bytes,
                      void *conv_state, float *rec_state, void *stream) {
  int rc = gdn_state_check(dims, blob, blob_bytes);
  if (rc) return rc;
  Geom g;
  check_dims(dims, &g);
  const size_t cb = conv_state_bytes(g), rb = rec_state_bytes(g);
  const Buf out[] = {{conv_state, cb, esize(g.in_dt)}, {rec_state, rb, 16}};
  if ((rc = check_buffers(nullptr, 0, out, 2))) return rc;
  if (injected_launch_failure()) return GDN_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char *payload = static_cast<const char *>(blob) + kBlobHeader;
  hipError_t e = hipMemcpyAsync(conv_state, payload, cb, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(rec_state, payload + cb, rb, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? GDN_OK : set_hip_error(e, "gdn_state_restore");
}

}  // extern "C"
