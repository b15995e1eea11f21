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
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

thread_local std::string g_last_hip_error;

// Largest T per call.  The split-role state pass addresses the four 32-wide
// d_k slices of q and k as one buffer base plus a 32-bit scalar offset of up
// to 3 * T_pad * 64 bytes; 2^24 tokens keep that below 2^32 (the first T to
// wrap would be about 22.4M).  Every other per-call index is 64-bit.
constexpr int64_t kMaxTokens = int64_t(1) << 24;
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
      (d->out_dtype != GDN_F32 && d->out_dtype != GDN_BF16 && d->out_dtype != GDN_F16))
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
  size_t align;  // required alignment in bytes; 0: an optional buffer left out
};

// z may be null (ungated output); then its entry is left out of the checks.
Buf optional_buf(const void *p, size_t n, size_t align) {
  return p ? Buf{p, n, align} : Buf{nullptr, 0, 0};
}

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
    if (!b.align) continue;
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
// Start and stop events of each kernel of a timed call, recorded at the
// kernels' own boundaries (see launch_kernel); durations in milliseconds.
struct CallTimer {
  static constexpr int kMax = 3;
  float *out;
  hipEvent_t ev[2 * kMax] = {};
  KernelEvents k[kMax] = {};
  bool ran[kMax] = {};
  hipError_t err = hipSuccess;
  explicit CallTimer(float *o, int n) : out(o) {
    for (int i = 0; o && err == hipSuccess && i < 2 * n; ++i) err = hipEventCreate(&ev[i]);
    for (int i = 0; i < kMax; ++i) k[i] = KernelEvents{ev[2 * i], ev[2 * i + 1]};
  }
  ~CallTimer() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
  }
  // Events for kernel i of the call (null when the call is not timed).
  const KernelEvents *at(int i) {
    if (!out) return nullptr;
    ran[i] = true;
    return &k[i];
  }
  // Waits for the call's last kernel; kernels that did not run report 0.
  hipError_t elapsed(int n) {
    if (!out) return hipSuccess;
    hipError_t e = hipSuccess;
    for (int i = 0; e == hipSuccess && i < n; ++i) {
      out[i] = 0.f;
      if (!ran[i]) continue;
      e = hipEventSynchronize(k[i].stop);
      if (e == hipSuccess) e = hipEventElapsedTime(&out[i], k[i].start, k[i].stop);
    }
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

// Decode workspace: the fp32 [B][T][C_ch] output of the conv step (q
// scaled and normalised, k normalised, v), read by the state stream.
size_t decode_ws_bytes(const Geom &g, int T) {
  return round_up(static_cast<size_t>(g.B) * T * g.C_ch * 4, 256);
}

int check_attn(const gdn_attn_dims *d, AttnGeom *a) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->abi != GDN_ABI_VERSION) return GDN_ERR_UNSUPPORTED;
  if (d->B < 1 || d->B > kMaxBatch || d->H_q < 1 || d->H_kv < 1 || d->H_q > 4096)
    return GDN_ERR_INVALID_ARG;
  if (d->H_q % d->H_kv) return GDN_ERR_UNSUPPORTED;
  if (d->d_h != 128 && d->d_h != 256) return GDN_ERR_UNSUPPORTED;
  if (d->rot_dim < 0 || d->rot_dim > d->d_h || d->rot_dim % 16) return GDN_ERR_INVALID_ARG;
  if (d->in_dtype != GDN_BF16 || (d->out_dtype != GDN_F32 && d->out_dtype != GDN_BF16))
    return GDN_ERR_UNSUPPORTED;
  if (!(d->rope_base > 1.f && d->rope_base < 1e30f)) return GDN_ERR_INVALID_ARG;
  if (!(d->scale > -1e30f && d->scale < 1e30f)) return GDN_ERR_INVALID_ARG;
  a->B = d->B;
  a->H_q = d->H_q;
  a->H_kv = d->H_kv;
  a->D = d->d_h;
  a->rot = d->rot_dim;
  a->base = d->rope_base;
  a->scale = d->scale;
  a->in_dt = d->in_dtype;
  a->out_dt = d->out_dtype;
  return GDN_OK;
}

// The launches of an attention call keep their work-item counts (grid x
// block) below 2^31: the RoPE pass B T (H_q + H_kv) d_h / 2, the attention
// pass about 4 B H_q T.
bool attn_fits(const AttnGeom &a, int64_t T, int64_t pos0) {
  constexpr int64_t lim = int64_t(1) << 31;
  (void)pos0;
  return int64_t(a.B) * T * (a.H_q + a.H_kv) * (a.D / 2) < lim &&
         int64_t(a.B) * a.H_q * T * 4 + int64_t(a.B) * a.H_kv * 512 < lim;
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
    case GDN_ERR_TOO_LARGE: return "request exceeds the fixed scratch of the no-allocation entry point";
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
  return check_dims(dims, &g) == GDN_OK ? decode_ws_bytes(g, 1) : 0;
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

// The three launches of one prefill call (conv, prep with the q/k history
// roll, state pass with the v history roll and the gate).
static hipError_t enqueue_prefill(const Geom &g, const PrefillWs &L, const void *x, const void *z,
                                  const float *gl, const float *beta, const void *conv_w,
                                  void *conv_state, float *rec_state, void *y, char *w,
                                  hipStream_t s, CallTimer *tm) {
  hipError_t e = tm ? tm->err : hipSuccess;
  if (e == hipSuccess && !prep_fuses_conv(g, L))
    e = launch_conv_prefill(g, L, x, conv_w, conv_state, w, s, tm ? tm->at(0) : nullptr);
  if (e == hipSuccess)
    e = launch_prefill_prep(g, L, gl, beta, w, x, conv_w, conv_state, s, tm ? tm->at(1) : nullptr);
  if (e == hipSuccess)
    e = launch_prefill_state(g, L, z, rec_state, y, w, x, conv_w, conv_state, s,
                             tm ? tm->at(2) : nullptr);
  return e;
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
                    optional_buf(z, bt * g.H_v * g.D * es, 16),
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
  CallTimer tm(kernel_ms, 3);
  hipError_t e = enqueue_prefill(g, L, x, z, gl, beta, conv_w, conv_state, rec_state, y,
                                 static_cast<char *>(ws), s, &tm);
  if (e == hipSuccess) e = tm.elapsed(3);
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

// One decode call of T tokens per sequence on slot-indexed states (the plain
// decode step is T = 1 with the states as a pool of B slots, sequence b in
// slot b).  validate_only: run every check except those of `ws` (which may be
// null then) and return without any HIP call.
struct DecodeArgs {
  int T;
  const void *x, *z;
  const float *gl, *beta;
  const void *conv_w;
  void *conv_pool;
  float *rec_pool;
  int n_slots;
  const int32_t *in_slots, *out_slots;  // device arrays or null
  void *y, *ws;
  size_t ws_bytes;
  void *stream;
  float *kernel_ms;  // timed variant: [0] conv step, [1] state stream
};

static int decode_run(const gdn_dims *dims, const DecodeArgs &a, const char *where,
                      bool validate_only = false) {
  Geom g;
  int rc = check_dims(dims, &g);
  if (rc) return rc;
  if (a.T < 1 || a.T > kMaxMultiTokens || a.n_slots < 1) return GDN_ERR_INVALID_ARG;
  const size_t es = esize(g.in_dt), eo = esize(g.out_dt);
  const size_t bt = static_cast<size_t>(g.B) * a.T;
  const size_t ns = static_cast<size_t>(a.n_slots);
  const size_t need = decode_ws_bytes(g, a.T);
  Buf in[7] = {{a.x, bt * g.C_ch * es, es},
               optional_buf(a.z, bt * g.H_v * g.D * es, es),
               {a.gl, bt * g.H_v * 4, 4},
               {a.beta, bt * g.H_v * 4, 4},
               {a.conv_w, static_cast<size_t>(g.C_ch) * g.W * es, es}};
  int n_in = 5;
  if (a.in_slots) in[n_in++] = {a.in_slots, static_cast<size_t>(g.B) * 4, 4};
  if (a.out_slots) in[n_in++] = {a.out_slots, bt * 4, 4};
  const Buf out[] = {{a.conv_pool, ns * (g.W - 1) * g.C_ch * es, es},
                     {a.rec_pool, ns * g.H_v * g.D * g.D * 4, 16},
                     {a.y, bt * g.H_v * g.D * eo, eo},
                     {a.ws, need, 16}};
  if ((rc = check_buffers(in, n_in, out, validate_only ? 3 : 4))) return rc;
  if (validate_only) return GDN_OK;
  if (a.ws_bytes < need) return GDN_ERR_WORKSPACE;
  if (injected_launch_failure()) return GDN_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  float *qkv = static_cast<float *>(a.ws);
  // The timed variant: events at each kernel's own start and end (the two
  // kernels take a few microseconds at small B, about as long as the launch
  // latency that events recorded between launches would add).
  CallTimer tm(a.kernel_ms, 2);
  hipError_t e = tm.err;
  if (e == hipSuccess)
    e = launch_conv_step(g, a.T, a.x, a.conv_w, a.conv_pool, qkv, a.in_slots, a.out_slots,
                         a.n_slots, s, tm.at(0));
  if (e == hipSuccess)
    e = launch_decode(g, a.T, qkv, a.z, a.gl, a.beta, a.rec_pool, a.y, a.n_slots, a.in_slots,
                      a.out_slots, s, tm.at(1));
  if (e == hipSuccess) e = tm.elapsed(2);
  return e == hipSuccess ? GDN_OK : set_hip_error(e, where);
}

static int decode_impl(const gdn_dims *dims, const void *x, const void *z, const float *gl,
                       const float *beta, const void *conv_w, void *conv_state,
                       float *rec_state, void *y, void *ws, size_t ws_bytes, void *stream,
                       float *kernel_ms, bool validate_only = false) {
  const DecodeArgs a{1, x, z, gl, beta, conv_w, conv_state, rec_state, dims ? dims->B : 0,
                     nullptr, nullptr, y, ws, ws_bytes, stream, kernel_ms};
  return decode_run(dims, a, "gdn_decode_step", validate_only);
}

int gdn_decode_step(const gdn_dims *dims, const void *x, const void *z, const float *gl,
                    const float *beta, const void *conv_w, void *conv_state,
                    float *rec_state, void *y, void *ws, size_t ws_bytes, void *stream) {
  return decode_impl(dims, x, z, gl, beta, conv_w, conv_state, rec_state, y, ws, ws_bytes,
                     stream, nullptr);
}

int gdn_decode_step_noalloc(const gdn_dims *dims, const void *x, const void *z, const float *gl,
                            const float *beta, const void *conv_w, void *conv_state,
                            float *rec_state, void *y, void *stream) {
  Geom g;
  int rc = check_dims(dims, &g);
  if (rc) return rc;
  const size_t need = decode_ws_bytes(g, 1);
  if (need > kNoAllocScratchBytes) return GDN_ERR_TOO_LARGE;
  // Every other check (pointers, alignment, aliasing) runs in decode_impl
  // before the first launch; the scratch itself is checked against the
  // buffers there as the workspace.  Validate first, so an invalid call
  // makes no HIP call at all.
  rc = decode_impl(dims, x, z, gl, beta, conv_w, conv_state, rec_state, y, nullptr, need,
                   stream, nullptr, /*validate_only=*/true);
  if (rc) return rc;
  if (injected_launch_failure()) return GDN_ERR_HIP;
  void *ws = nullptr;
  const hipError_t e = noalloc_scratch(static_cast<hipStream_t>(stream), &ws);
  if (e != hipSuccess) return set_hip_error(e, "gdn_decode_step_noalloc");
  return decode_impl(dims, x, z, gl, beta, conv_w, conv_state, rec_state, y, ws, need, stream,
                     nullptr);
}

int gdn_decode_step_timed(const gdn_dims *dims, const void *x, const void *z, const float *gl,
                          const float *beta, const void *conv_w, void *conv_state,
                          float *rec_state, void *y, void *ws, size_t ws_bytes, void *stream,
                          float *kernel_ms) {
  if (!kernel_ms) return GDN_ERR_INVALID_ARG;
  return decode_impl(dims, x, z, gl, beta, conv_w, conv_state, rec_state, y, ws, ws_bytes,
                     stream, kernel_ms);
}

int gdn_decode_multi(const gdn_dims *dims, int32_t T, const void *x, const void *z,
                     const float *gl, const float *beta, const void *conv_w, void *conv_pool,
                     float *rec_pool, int32_t n_slots, const int32_t *in_slots,
                     const int32_t *out_slots, void *y, void *ws, size_t ws_bytes,
                     void *stream) {
  if (!in_slots) return GDN_ERR_INVALID_ARG;
  const DecodeArgs a{T, x, z, gl, beta, conv_w, conv_pool, rec_pool, n_slots, in_slots,
                     out_slots, y, ws, ws_bytes, stream, nullptr};
  return decode_run(dims, a, "gdn_decode_multi");
}

// Packed variable-length prefill: host-side sequence table, validated in
// full before anything is enqueued; then each non-empty sequence runs the
// chunked prefill on its own rows and its own slot, in stream order, all
// sharing one workspace.
// Packed variable-length prefill runs its sequences on up to kVarlenLanes
// streams at once: the caller's stream and up to two auxiliary ones of the
// library, forked from and joined back to the caller's stream by events.  A
// short sequence's three passes leave most compute units idle; side by side,
// the sequences' state passes share the GPU.  Each lane has its own workspace
// part, so the workspace is lanes x the largest single-sequence workspace.
// Three lanes, not four: a process gets four hardware queues by default,
// and next to the caller's stream there is usually another stream of the
// framework (a graph-capture stream, for one), so a third auxiliary stream
// shared a queue with another lane and waited behind it (8 mixed sequences
// in a process that had captured graphs: 573-575 us with three lanes against
// 618-621 with four; about equal in a fresh process).
constexpr int kVarlenLanes = 3;
constexpr int64_t kVarlenSeqTokens = 1536;
constexpr int kMaxDevices = 64;

struct VarlenStreams {
  hipStream_t aux[kVarlenLanes - 1] = {};
  hipEvent_t fork = nullptr, join[kVarlenLanes - 1] = {};
};
std::mutex g_varlen_mu;
VarlenStreams g_varlen[kMaxDevices];

// The auxiliary streams and events of the current device, created on first
// use (non-blocking, default priority) and kept until the process ends.
// Called with g_varlen_mu held.
static hipError_t varlen_streams(VarlenStreams **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  VarlenStreams &v = g_varlen[dev];
  if (!v.fork) {
    VarlenStreams n;
    for (int k = 0; e == hipSuccess && k < kVarlenLanes - 1; ++k) {
      e = hipStreamCreateWithFlags(&n.aux[k], hipStreamNonBlocking);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join[k], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    v = n;
  }
  *out = &v;
  return hipSuccess;
}

// Lanes of a sequence table: one per non-empty sequence, at most kVarlenLanes.
static int varlen_lanes(const Geom &g, const int64_t *cu) {
  int n = 0;
  for (int i = 0; i < g.B; ++i) n += cu[i + 1] > cu[i];
  return std::max(1, std::min(n, kVarlenLanes));
}

static int varlen_check(const Geom &g, const int64_t *cu, int32_t chunk, size_t *ws_need,
                        int64_t *T_total) {
  if (!cu) return GDN_ERR_INVALID_ARG;
  if (cu[0] != 0) return GDN_ERR_INVALID_ARG;
  size_t need = 0;
  for (int n = 0; n < g.B; ++n) {
    const int64_t len = cu[n + 1] - cu[n];
    if (len < 0 || len > kMaxTokens) return GDN_ERR_INVALID_ARG;
    if (len == 0) continue;
    Geom g1 = g;
    g1.B = 1;
    PrefillWs L;
    if (!prefill_ws_layout(g1, len, chunk, &L)) return GDN_ERR_UNSUPPORTED;
    need = std::max(need, L.total);
  }
  if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return GDN_ERR_UNSUPPORTED;
  if (cu[g.B] > (int64_t(1) << 40)) return GDN_ERR_INVALID_ARG;
  need = (need + 255) / 256 * 256;  // each lane's part 256-byte aligned
  *ws_need = std::max<size_t>(need, 256) * varlen_lanes(g, cu);
  *T_total = cu[g.B];
  return GDN_OK;
}

size_t gdn_prefill_varlen_workspace_bytes(const gdn_dims *dims, const int64_t *cu_seqlens,
                                          int32_t chunk) {
  Geom g;
  size_t need = 0;
  int64_t T_total = 0;
  if (check_dims(dims, &g) != GDN_OK || varlen_check(g, cu_seqlens, chunk, &need, &T_total))
    return 0;
  return need;
}

int gdn_prefill_varlen(const gdn_dims *dims, const int64_t *cu_seqlens, int32_t chunk,
                       const void *x, const void *z, const float *gl, const float *beta,
                       const void *conv_w, void *conv_pool, float *rec_pool, int32_t n_slots,
                       const int32_t *slots, void *y, void *ws, size_t ws_bytes, void *stream) {
  Geom g;
  int rc = check_dims(dims, &g);
  if (rc) return rc;
  size_t need = 0;
  int64_t T_total = 0;
  if ((rc = varlen_check(g, cu_seqlens, chunk, &need, &T_total))) return rc;
  if (!slots || n_slots < 1) return GDN_ERR_INVALID_ARG;
  for (int n = 0; n < g.B; ++n) {
    if (slots[n] < 0 || slots[n] >= n_slots) return GDN_ERR_INVALID_ARG;
    for (int m = 0; m < n; ++m)
      if (slots[m] == slots[n]) return GDN_ERR_INVALID_ARG;  // two sequences, one state
  }
  const size_t es = esize(g.in_dt), eo = esize(g.out_dt);
  const size_t tt = static_cast<size_t>(T_total), ns = static_cast<size_t>(n_slots);
  const size_t conv_slot = static_cast<size_t>(g.W - 1) * g.C_ch * es;
  const size_t rec_slot = static_cast<size_t>(g.H_v) * g.D * g.D * 4;
  const Buf in[] = {{x, tt * g.C_ch * es, 16},
                    optional_buf(z, tt * g.H_v * g.D * es, 16),
                    {gl, tt * g.H_v * 4, 4},
                    {beta, tt * g.H_v * 4, 4},
                    {conv_w, static_cast<size_t>(g.C_ch) * g.W * es, es}};
  const Buf out[] = {{conv_pool, ns * conv_slot, 16},
                     {rec_pool, ns * rec_slot, 16},
                     {y, tt * g.H_v * g.D * eo, eo},
                     {ws, need, 16}};
  // Inputs and outputs may be empty (all sequences of length 0): then only
  // the state pools and the workspace are checked.
  if (T_total == 0) {
    if ((rc = check_buffers(nullptr, 0, out, 2))) return rc;
  } else if ((rc = check_buffers(in, 5, out, 4))) {
    return rc;
  }
  if (T_total > 0 && ws_bytes < need) return GDN_ERR_WORKSPACE;
  if (injected_launch_failure()) return GDN_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  CallTimer *tm = nullptr;  // not timed
  Geom g1 = g;
  g1.B = 1;
  const int lanes = varlen_lanes(g, cu_seqlens);
  const size_t lane_ws = need / lanes;
  std::unique_lock<std::mutex> lock(g_varlen_mu, std::defer_lock);
  VarlenStreams *vs = nullptr;
  hipStream_t ls[kVarlenLanes] = {s};
  hipError_t e = hipSuccess;
  if (lanes > 1) {
    lock.lock();
    e = varlen_streams(&vs);
    if (e == hipSuccess) e = hipEventRecord(vs->fork, s);
    for (int k = 1; e == hipSuccess && k < lanes; ++k) {
      ls[k] = vs->aux[k - 1];
      e = hipStreamWaitEvent(ls[k], vs->fork, 0);
    }
  }
  // Longest sequences first, each to the lane with the least work so far: a
  // sequence costs its tokens plus kVarlenSeqTokens, the fixed latency of its
  // three launches (about 50 us, the state pass's time for 24 chunks of 64)
  // expressed in tokens.  Measured on 8 mixed sequences: 553-560 us against
  // 567-576 with tokens alone.
  std::vector<int> order;
  for (int n = 0; n < g.B; ++n)
    if (cu_seqlens[n + 1] > cu_seqlens[n]) order.push_back(n);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return cu_seqlens[a + 1] - cu_seqlens[a] > cu_seqlens[b + 1] - cu_seqlens[b];
  });
  int64_t load[kVarlenLanes] = {};
  for (size_t i = 0; e == hipSuccess && i < order.size(); ++i) {
    const int n = order[i];
    const int64_t t0 = cu_seqlens[n], len = cu_seqlens[n + 1] - t0;
    const int k = static_cast<int>(std::min_element(load, load + lanes) - load);
    load[k] += len + kVarlenSeqTokens;
    PrefillWs L;
    prefill_ws_layout(g1, len, chunk, &L);
    const size_t tok = static_cast<size_t>(t0);
    e = enqueue_prefill(
        g1, L, static_cast<const char *>(x) + tok * g.C_ch * es,
        static_cast<const char *>(z) + tok * g.H_v * g.D * es, gl + tok * g.H_v,
        beta + tok * g.H_v, conv_w, static_cast<char *>(conv_pool) + slots[n] * conv_slot,
        rec_pool + static_cast<size_t>(slots[n]) * (rec_slot / 4),
        static_cast<char *>(y) + tok * g.H_v * g.D * eo, static_cast<char *>(ws) + k * lane_ws,
        ls[k], tm);
  }
  // The caller's stream continues once every lane is done.
  for (int k = 1; e == hipSuccess && k < lanes; ++k) {
    e = hipEventRecord(vs->join[k - 1], ls[k]);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, vs->join[k - 1], 0);
  }
  if (e != hipSuccess) return set_hip_error(e, "gdn_prefill_varlen");
  return GDN_OK;
}

int gdn_gated_rmsnorm(const gdn_dims *dims, int64_t rows, const float *o, const void *z,
                      const float *norm_w, float norm_eps, void *y, void *stream) {
  Geom g;
  int rc = check_dims(dims, &g);
  if (rc) return rc;
  if (rows < 0 || rows > (int64_t(1) << 40) / (static_cast<int64_t>(g.H_v) * g.D))
    return GDN_ERR_INVALID_ARG;
  if (!(norm_eps >= 0.f) || !(norm_eps < 1e30f)) return GDN_ERR_INVALID_ARG;
  const size_t n = static_cast<size_t>(rows) * g.H_v * g.D;
  const Buf in[] = {{o, n * 4, 16}, optional_buf(z, n * esize(g.in_dt), 16),
                    optional_buf(norm_w, static_cast<size_t>(g.D) * 4, 16)};
  const Buf out[] = {{y, n * esize(g.out_dt), 16}};
  if (rows == 0) return GDN_OK;
  if ((rc = check_buffers(in, 3, out, 1))) return rc;
  if (injected_launch_failure()) return GDN_ERR_HIP;
  const hipError_t e = launch_gated_rmsnorm(g, rows, o, z, norm_w, norm_eps, y,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : set_hip_error(e, "gdn_gated_rmsnorm");
}

int gdn_in_proj(const gdn_dims *dims, int64_t T, int32_t hidden, const void *h,
                const void *w_in, const float *A_log, const float *dt_bias, void *x, void *z,
                float *gl, float *beta, void *stream) {
  Geom g;
  int rc = check_dims(dims, &g);
  if (rc) return rc;
  if (g.in_dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;  // bf16 activations and weights
  if (T < 1 || T > kMaxTokens) return GDN_ERR_INVALID_ARG;
  if (hidden < 64 || hidden % 64 || hidden > (1 << 20)) return GDN_ERR_UNSUPPORTED;
  const size_t M = static_cast<size_t>(g.B) * T;
  const size_t N = static_cast<size_t>(g.C_ch) + g.H_v * g.D + 2 * g.H_v;
  const Buf in[] = {{h, M * hidden * 2, 16},
                    {w_in, N * hidden * 2, 16},
                    {A_log, static_cast<size_t>(g.H_v) * 4, 4},
                    {dt_bias, static_cast<size_t>(g.H_v) * 4, 4}};
  const Buf out[] = {{x, M * g.C_ch * 2, 2},
                     {z, M * g.H_v * g.D * 2, 2},
                     {gl, M * g.H_v * 4, 4},
                     {beta, M * g.H_v * 4, 4}};
  if ((rc = check_buffers(in, 4, out, 4))) return rc;
  if (injected_launch_failure()) return GDN_ERR_HIP;
  const hipError_t e = launch_in_proj(g, static_cast<int64_t>(M), hidden, h, w_in, A_log, dt_bias,
                                      x, z, gl, beta, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : set_hip_error(e, "gdn_in_proj");
}

size_t gdn_attn_workspace_bytes(const gdn_attn_dims *dims, int64_t T, int64_t pos0) {
  AttnGeom a;
  if (check_attn(dims, &a) || T < 1 || pos0 < 0 || pos0 + T > kMaxTokens || !attn_fits(a, T, pos0))
    return 0;
  return attn_ws_bytes(a, T, pos0);
}

int gdn_attn_prefill(const gdn_attn_dims *dims, int64_t T, int64_t pos0, const void *q,
                     const void *k, const void *v, void *k_cache, void *v_cache, int64_t T_max,
                     void *o, void *ws, size_t ws_bytes, void *stream) {
  AttnGeom a;
  int rc = check_attn(dims, &a);
  if (rc) return rc;
  if (T < 1 || pos0 < 0 || T_max < 1 || T_max > kMaxTokens || pos0 + T > T_max ||
      !attn_fits(a, T, pos0))
    return GDN_ERR_INVALID_ARG;
  const size_t bt = static_cast<size_t>(a.B) * T, D = static_cast<size_t>(a.D);
  const size_t need = attn_ws_bytes(a, T, pos0);
  const size_t cache = static_cast<size_t>(a.B) * T_max * a.H_kv * D * 2;
  const Buf in[] = {{q, bt * a.H_q * D * 2, 16}, {k, bt * a.H_kv * D * 2, 16},
                    {v, bt * a.H_kv * D * 2, 16}};
  const Buf out[] = {{k_cache, cache, 16}, {v_cache, cache, 16},
                     {o, bt * a.H_q * D * esize(a.out_dt), esize(a.out_dt)}, {ws, need, 16}};
  if ((rc = check_buffers(in, 3, out, 4))) return rc;
  if (ws_bytes < need) return GDN_ERR_WORKSPACE;
  if (injected_launch_failure()) return GDN_ERR_HIP;
  const hipError_t e = launch_attn_prefill(a, T, pos0, q, k, v, k_cache, v_cache, T_max, o, ws,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : set_hip_error(e, "gdn_attn_prefill");
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
