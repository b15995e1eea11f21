// decode.hip -- one token of the gated delta rule per sequence, fused with the
// sigmoid output gate.  Separately tuned single-step decode behind the same
// semantic interface as prefill ("Add a performance-parity Qwen3.8-27B Q4 and
// Q8 text backend on Metal", section Scope).
//
// Per state row i of value head h (S is d_v x d_k, fp32, o = S q):
//   p = S_i . k,  r = S_i . q                     (old state)
//   u = beta (v_i - a p)
//   S_i <- a S_i + u k                            == a S (I - beta k k^T) + beta v k^T
//   o_i = a r + u (k . q)                         == (updated S_i) . q
//   y_i = o_i * sigmoid(z_i)
// The state is streamed from HBM once and written back once, so the kernel is
// HBM-bound: 2 * d_v * d_k * 4 bytes per head and step dominate the traffic.
//
// Layout: LPR lanes share one row, each holding NPL consecutive-by-4 floats
// (d_k = 128: 8 lanes x 16 floats, every load instruction covers 128
// contiguous bytes per row); the two dot products are reduced across those
// lanes with xor shuffles.  A block of 4 waves takes 256 / LPR consecutive
// state rows (32 at d = 128), loading all of them before computing: with
// nontemporal stores, these small blocks (12,288 at B = 64) stream faster
// than one block per (sequence, head) walking four such groups (67.7-68.4
// vs 75.4-75.6 us at B = 64, measured side by side).
#include <mutex>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// The state is read exactly once and written exactly once per step:
// nontemporal loads and stores keep that stream from displacing cached data
// (measured at B = 64: the loads about 12% faster, the stores another 7%).
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float4 *p) {
  const f4v r = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(p));
  return make_float4(r[0], r[1], r[2], r[3]);
}
__device__ __forceinline__ void store_stream(float4 *p, float4 v) {
  const f4v r = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(r, reinterpret_cast<f4v *>(p));
}

template <int D>
struct DecodeShape {
  static constexpr int NPL = (D >= 128) ? 16 : 4;  // floats per lane per row
  static constexpr int LPR = D / NPL;              // lanes per row
  static constexpr int RPW = kWave / LPR;          // rows per wave per pass
  static constexpr int RPB = 4 * RPW;              // rows per block per pass
};

template <int D, int DTZ, int DTY, int PASSES>
__global__ __launch_bounds__(256) void decode_kernel(Geom g, const float *__restrict__ qkv,
                                                     const void *__restrict__ z,
                                                     const float *__restrict__ gl,
                                                     const float *__restrict__ beta,
                                                     float *__restrict__ S, void *__restrict__ y,
                                                     int64_t total_rows) {
  using Sh = DecodeShape<D>;
  constexpr int NPL = Sh::NPL, LPR = Sh::LPR, NV = NPL / 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane % LPR;  // column slot of this lane
  const int64_t base_row = static_cast<int64_t>(blockIdx.x) * (PASSES * Sh::RPB);

  float4 s[PASSES][NV];
  int64_t rows[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    rows[p] = base_row + p * Sh::RPB + wave * Sh::RPW + lane / LPR;
    if (rows[p] < total_rows) {
      const float4 *src = reinterpret_cast<const float4 *>(S + rows[p] * D);
#pragma unroll
      for (int m = 0; m < NV; ++m) s[p][m] = load_stream(src + j + LPR * m);
    }
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int64_t R = rows[p];
    const bool live = R < total_rows;
    // (b, h, i) of this row; rows of dead lanes alias row 0 for the loads.
    const int64_t Rc = live ? R : 0;
    const int i = static_cast<int>(Rc % D);
    const int64_t bh = Rc / D;
    const int h = static_cast<int>(bh % g.H_v);
    const int b = static_cast<int>(bh / g.H_v);
    const int kh = h / g.G;
    const float *qrow = qkv + static_cast<size_t>(b) * g.C_ch + kh * D;
    const float *krow = qrow + g.H_k * D;
    float4 kv[NV], qv[NV];
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      kv[m] = reinterpret_cast<const float4 *>(krow)[j + LPR * m];
      qv[m] = reinterpret_cast<const float4 *>(qrow)[j + LPR * m];
    }
    float pk = 0.f, pq = 0.f, kq = 0.f;
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const float4 sv = live ? s[p][m] : make_float4(0.f, 0.f, 0.f, 0.f);
      pk = __builtin_fmaf(sv.x, kv[m].x, pk);
      pk = __builtin_fmaf(sv.y, kv[m].y, pk);
      pk = __builtin_fmaf(sv.z, kv[m].z, pk);
      pk = __builtin_fmaf(sv.w, kv[m].w, pk);
      pq = __builtin_fmaf(sv.x, qv[m].x, pq);
      pq = __builtin_fmaf(sv.y, qv[m].y, pq);
      pq = __builtin_fmaf(sv.z, qv[m].z, pq);
      pq = __builtin_fmaf(sv.w, qv[m].w, pq);
      kq = __builtin_fmaf(kv[m].x, qv[m].x, kq);
      kq = __builtin_fmaf(kv[m].y, qv[m].y, kq);
      kq = __builtin_fmaf(kv[m].z, qv[m].z, kq);
      kq = __builtin_fmaf(kv[m].w, qv[m].w, kq);
    }
#pragma unroll
    for (int msk = LPR / 2; msk >= 1; msk >>= 1) {
      pk += __shfl_xor(pk, msk, kWave);
      pq += __shfl_xor(pq, msk, kWave);
      kq += __shfl_xor(kq, msk, kWave);
    }
    const size_t gh = static_cast<size_t>(b) * g.H_v + h;
    const float a = __expf(gl[gh]);
    const float bt = beta[gh];
    const float vi = qkv[static_cast<size_t>(b) * g.C_ch + 2 * g.H_k * D + h * D + i];
    const float u = bt * (vi - a * pk);
    const float o = a * pq + u * kq;
    if (live) {
      float4 *dst = reinterpret_cast<float4 *>(S + R * D);
#pragma unroll
      for (int m = 0; m < NV; ++m) {
        float4 n;
        n.x = __builtin_fmaf(u, kv[m].x, a * s[p][m].x);
        n.y = __builtin_fmaf(u, kv[m].y, a * s[p][m].y);
        n.z = __builtin_fmaf(u, kv[m].z, a * s[p][m].z);
        n.w = __builtin_fmaf(u, kv[m].w, a * s[p][m].w);
        store_stream(dst + j + LPR * m, n);
      }
      if (j == 0) {
        const size_t yi = gh * D + i;
        store_elem<DTY>(y, yi, o * sigmoidf_(load_elem<DTZ>(z, yi)));
      }
    }
  }
}

template <int D, int DTZ, int DTY>
static void launch_decode_t(const Geom &g, dim3 grid, const float *qkv, const void *z,
                            const float *gl, const float *beta, float *S, void *y, int64_t rows,
                            hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<D, DTZ, DTY, 1>), grid, dim3(256), 0, s, g, qkv, z, gl,
                     beta, S, y, rows);
}

hipError_t launch_decode(const Geom &g, const float *qkv, const void *z, const float *gl,
                         const float *beta, float *S, void *y, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(g.B) * g.H_v * g.D;
  const int rpb = (g.D == 128) ? DecodeShape<128>::RPB : DecodeShape<16>::RPB;
  dim3 grid(static_cast<unsigned>((rows + rpb - 1) / rpb));
  const int key = (g.in_dt << 1) | g.out_dt;
#define GDN_DEC(Dv)                                                               \
  switch (key) {                                                                  \
    case 0: launch_decode_t<Dv, 0, 0>(g, grid, qkv, z, gl, beta, S, y, rows, s); break; \
    case 1: launch_decode_t<Dv, 0, 1>(g, grid, qkv, z, gl, beta, S, y, rows, s); break; \
    case 2: launch_decode_t<Dv, 1, 0>(g, grid, qkv, z, gl, beta, S, y, rows, s); break; \
    default: launch_decode_t<Dv, 1, 1>(g, grid, qkv, z, gl, beta, S, y, rows, s); break; \
  }
  if (g.D == 128) {
    GDN_DEC(128)
  } else {
    GDN_DEC(16)
  }
#undef GDN_DEC
  return hipGetLastError();
}

// ---------------------------------------------------------------- fixed scratch
// The decode workspace of gdn_decode_step_noalloc lives in this array: one
// copy per GPU, loaded with the code object, kept until the process ends.
// Host code never passes the array's name to a kernel (on the host it only
// stands for the symbol); it passes the device address that
// hipGetSymbolAddress returns for the GPU the call runs on, fetched once per
// GPU with that GPU current.
namespace {
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxGpus = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxGpus] = {};
}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void **out) {
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxGpus) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace gdn
