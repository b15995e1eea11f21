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
// contiguous bytes per row; at B <= 4, 32 lanes x 4 floats, for four times
// the blocks); the two dot products are reduced across those lanes with xor
// shuffles.  A block of 4 waves takes 256 / LPR consecutive state rows (32
// at d = 128 and B > 4), loading all of them before computing: with
// nontemporal stores, these small blocks (12,288 at B = 64) stream faster
// than one block per (sequence, head) walking four such groups (67.7-68.4
// vs 75.4-75.6 us at B = 64, measured side by side).
//
// Several tokens per sequence (gdn_decode_multi): the rows stay in registers
// across the TT tokens, so the state is read once for all of them; the rows
// after token t are stored to the slot chosen for t, if any.  The conv step
// (conv.hip) runs as its own launch before this one: it owns the conv
// history roll, which the blocks here could not do without knowing that
// every other block of the key head has read the history (a device-wide
// counter for that cost about 4 us per step at B = 1 on MI355X, more than
// the second launch).
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

template <int D, int NPL_>
struct DecodeShape {
  static constexpr int NPL = NPL_;         // floats per lane per row
  static constexpr int LPR = D / NPL;      // lanes per row
  static constexpr int RPW = kWave / LPR;  // rows per wave
  static constexpr int RPB = 4 * RPW;      // rows per block
};

// Slots (gdn_decode_multi): sequence b reads its state from slot
// in_slots[b] (b itself when in_slots is null) and stores the state after
// token t to slot out_slots[b * TT + t] (when out_slots is null: the in slot
// after the last token, nothing before).  An in slot outside [0, n_slots)
// makes b a padding row: zero y, nothing read or stored; an out slot outside
// that range is not stored.  A block only stores rows it has already read,
// so a sequence may name its in slot as an out slot.
struct SlotArgs {
  const int32_t *in_slots, *out_slots;
  int n_slots;
};

__device__ __forceinline__ int in_slot(const SlotArgs &sa, int b) {
  const int s = sa.in_slots ? sa.in_slots[b] : b;
  return (s >= 0 && s < sa.n_slots) ? s : -1;
}

template <int TT>
__device__ __forceinline__ int out_slot(const SlotArgs &sa, int b, int t, int sin) {
  const int o = sa.out_slots ? sa.out_slots[static_cast<size_t>(b) * TT + t]
                             : (t == TT - 1 ? sin : -1);
  return (o >= 0 && o < sa.n_slots) ? o : -1;
}

// qkv: [B][TT][C_ch] fp32 from the conv step (q scaled and normalised, k
// normalised, v).  z, y: [B][TT][H_v][D]; gl, beta: [B][TT][H_v].
template <int D, int NPL, int DTZ, int DTY, int TT>
__global__ __launch_bounds__(256) void decode_kernel(Geom g, const float *__restrict__ qkv,
                                                     const void *__restrict__ z,
                                                     const float *__restrict__ gl,
                                                     const float *__restrict__ beta,
                                                     float *__restrict__ S, void *__restrict__ y,
                                                     SlotArgs sa, int64_t total_rows) {
  using Sh = DecodeShape<D, NPL>;
  constexpr int LPR = Sh::LPR, NV = NPL / 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane % LPR;  // column slot of this lane
  const int64_t R = static_cast<int64_t>(blockIdx.x) * Sh::RPB + wave * Sh::RPW + lane / LPR;
  if (R >= total_rows) return;  // whole row groups only: shuffles stay within live lanes
  // (b, h, i) of this row.
  const int i = static_cast<int>(R % D);
  const int64_t bh = R / D;
  const int h = static_cast<int>(bh % g.H_v);
  const int b = static_cast<int>(bh / g.H_v);
  const int kh = h / g.G;
  const size_t bt0 = static_cast<size_t>(b) * TT;
  const int sin = in_slot(sa, b);
  if (sin < 0) {  // padding row
    if (j == 0)
      for (int t = 0; t < TT; ++t)
        store_elem<out_type(DTY)>(y, ((bt0 + t) * g.H_v + h) * D + i, 0.f);
    return;
  }
  const size_t row_off = (static_cast<size_t>(h) * D + i) * D;
  const size_t pool_stride = static_cast<size_t>(g.H_v) * D * D;
  float4 s[NV];
  {
    const float4 *src = reinterpret_cast<const float4 *>(S + sin * pool_stride + row_off);
#pragma unroll
    for (int m = 0; m < NV; ++m) s[m] = load_stream(src + j + LPR * m);
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float *qrow = qkv + (bt0 + t) * g.C_ch + kh * D;
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
      pk = __builtin_fmaf(s[m].x, kv[m].x, pk);
      pk = __builtin_fmaf(s[m].y, kv[m].y, pk);
      pk = __builtin_fmaf(s[m].z, kv[m].z, pk);
      pk = __builtin_fmaf(s[m].w, kv[m].w, pk);
      pq = __builtin_fmaf(s[m].x, qv[m].x, pq);
      pq = __builtin_fmaf(s[m].y, qv[m].y, pq);
      pq = __builtin_fmaf(s[m].z, qv[m].z, pq);
      pq = __builtin_fmaf(s[m].w, qv[m].w, pq);
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
    const size_t gh = (bt0 + t) * g.H_v + h;
    const float a = __expf(gl[gh]);
    const float bt = beta[gh];
    const float vi = qkv[(bt0 + t) * g.C_ch + 2 * g.H_k * D + h * D + i];
    const float u = bt * (vi - a * pk);
    const float o = a * pq + u * kq;
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      s[m].x = __builtin_fmaf(u, kv[m].x, a * s[m].x);
      s[m].y = __builtin_fmaf(u, kv[m].y, a * s[m].y);
      s[m].z = __builtin_fmaf(u, kv[m].z, a * s[m].z);
      s[m].w = __builtin_fmaf(u, kv[m].w, a * s[m].w);
    }
    const int so = out_slot<TT>(sa, b, t, sin);
    if (so >= 0) {
      float4 *dst = reinterpret_cast<float4 *>(S + so * pool_stride + row_off);
#pragma unroll
      for (int m = 0; m < NV; ++m) store_stream(dst + j + LPR * m, s[m]);
    }
    if (j == 0) {
      const size_t yi = gh * D + i;
      if constexpr (out_gated(DTY))
        store_elem<out_type(DTY)>(y, yi, o * sigmoidf_(load_elem<DTZ>(z, yi)));
      else
        store_elem<out_type(DTY)>(y, yi, o);
    }
  }
}

template <int D, int NPL, int TT>
static void launch_decode_t(const Geom &g, const float *qkv, const void *z, const float *gl,
                            const float *beta, float *S, void *y, const SlotArgs &sa,
                            hipStream_t s, const KernelEvents *ev) {
  const int64_t rows = static_cast<int64_t>(g.B) * g.H_v * D;
  const dim3 grid(static_cast<unsigned>((rows + DecodeShape<D, NPL>::RPB - 1) /
                                        DecodeShape<D, NPL>::RPB));
#define GDN_DEC(ZT, OC) \
  launch_kernel(decode_kernel<D, NPL, ZT, OC, TT>, grid, dim3(256), s, ev, g, qkv, z, gl, beta, S, y, sa, rows)
  GDN_OUT_DISPATCH(g.in_dt, out_code(g.out_dt, z), GDN_DEC);
#undef GDN_DEC
}

template <int TT>
static void launch_decode_tt(const Geom &g, const float *qkv, const void *z, const float *gl,
                             const float *beta, float *S, void *y, const SlotArgs &sa,
                             hipStream_t s, const KernelEvents *ev) {
  // d = 128: 8 lanes x 16 floats per row, 32 rows per block; at B <= 4, 32
  // lanes x 4 floats, 8 rows per block (768 blocks at B = 1 instead of 192:
  // 5.36-5.38 against 5.62-5.64 us per graph-replayed step, measured side by
  // side; 16 lanes x 8 floats 5.40-5.45).
  if (g.D == 128 && g.B <= 4)
    launch_decode_t<128, 4, TT>(g, qkv, z, gl, beta, S, y, sa, s, ev);
  else if (g.D == 128)
    launch_decode_t<128, 16, TT>(g, qkv, z, gl, beta, S, y, sa, s, ev);
  else
    launch_decode_t<16, 4, TT>(g, qkv, z, gl, beta, S, y, sa, s, ev);
}

hipError_t launch_decode(const Geom &g, int T, const float *qkv, const void *z, const float *gl,
                         const float *beta, float *S, void *y, int n_slots,
                         const int32_t *in_slots, const int32_t *out_slots, hipStream_t s,
                         const KernelEvents *ev) {
  const SlotArgs sa{in_slots, out_slots, n_slots};
  switch (T) {
    case 1: launch_decode_tt<1>(g, qkv, z, gl, beta, S, y, sa, s, ev); break;
    case 2: launch_decode_tt<2>(g, qkv, z, gl, beta, S, y, sa, s, ev); break;
    case 3: launch_decode_tt<3>(g, qkv, z, gl, beta, S, y, sa, s, ev); break;
    case 4: launch_decode_tt<4>(g, qkv, z, gl, beta, S, y, sa, s, ev); break;
    default: return hipErrorInvalidValue;
  }
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
