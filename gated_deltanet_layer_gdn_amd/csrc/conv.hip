// conv.hip -- causal width-4 depthwise Conv1D + SiLU + per-head L2 norm.
//
// Layer steps 1-2 ("Implement the Qwen3.8 Flash Next Rust and Metal text
// core", section Implementation: convolution width 4, L2-normalised q/k with
// the epsilon placement fixed; its implementation comment: a BF16 width-4
// convolution history).  Reading taken: xi_t = sum_j w[c][j] x[t-3+j], tap 3
// on the current token, rows before t = 0 from the history (oldest first),
// u = SiLU(xi), q/k heads divided by sqrt(sum u^2 + eps), q times q_scale.
//
// One thread owns one channel and walks the tokens of its tile with the
// three previous inputs in registers, so each input is read once from HBM
// (coalesced across the 128 channels of a block).  The head sum of squares
// for q/k is a wave reduction (plus one LDS exchange when a head spans two
// waves).  HBM-bound: bytes per token = C_ch * (in + out) element sizes.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kConvThreads = 128;  // channels per block
constexpr int kConvTT = 32;        // tokens per block

enum { kOutPlain = 0, kOutPrefill = 1 };

struct ConvArgs {
  const void *x;
  const void *w;
  void *hist;   // conv history [B][3][C_ch]; written only when fuse_roll
  float *out;   // plain output [B][T][C_ch]
  char *ws;     // prefill workspace
  PrefillWs L;
  int64_t T;       // real tokens
  int64_t T_iter;  // tokens the grid walks (T, or T_pad for the prefill layout)
  int fuse_roll;   // single tile holds every token: roll the history in place
};

// Sum over the D consecutive threads of one head.
template <int D>
__device__ __forceinline__ float head_sum(float v, float *red) {
  if constexpr (D <= 64) {
#pragma unroll
    for (int m = D / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
  } else {
    static_assert(D == 128, "heads of 16 or 128 channels");
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    const float s = red[0] + red[1];
    __syncthreads();
    return s;
  }
}

template <int DT, int D, int MODE>
__global__ __launch_bounds__(kConvThreads) void conv_kernel(Geom g, ConvArgs a) {
  __shared__ float red[2];
  const int ch = blockIdx.y * kConvThreads + threadIdx.x;
  const int b = blockIdx.z;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kConvTT;
  const bool active = ch < g.C_ch;
  const int nq = g.H_k * D;
  const int nqk = 2 * nq;
  const bool is_q = ch < nq;
  const bool is_k = !is_q && ch < nqk;
  // For D = 128 a block is exactly one head, so this is uniform per block.
  const bool qk_block = (D == 128) ? (blockIdx.y * kConvThreads < nqk) : true;

  float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f;
  if (active) {
    w0 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 0);
    w1 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 1);
    w2 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 2);
    w3 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 3);
  }
  auto xin = [&](int64_t tau) -> float {
    if (tau >= 0)
      return tau < a.T ? load_elem<DT>(a.x, (static_cast<size_t>(b) * a.T + tau) * g.C_ch + ch)
                       : 0.f;
    return load_elem<DT>(a.hist, (static_cast<size_t>(b) * 3 + 3 + tau) * g.C_ch + ch);
  };
  float x0 = 0.f, x1 = 0.f, x2 = 0.f;
  if (active) {
    x0 = xin(t0 - 3);
    x1 = xin(t0 - 2);
    x2 = xin(t0 - 1);
  }
  const int64_t t_end = (t0 + kConvTT < a.T_iter) ? t0 + kConvTT : a.T_iter;
  for (int64_t t = t0; t < t_end; ++t) {
    const float x3 = active ? xin(t) : 0.f;
    const float u = siluf_(conv4(w0, w1, w2, w3, x0, x1, x2, x3));
    float val = u;
    if (qk_block) {
      const float ss = head_sum<D>(u * u, red);
      if (is_q || is_k) {
        const float inv = 1.0f / __builtin_sqrtf(ss + g.eps);
        val = u * inv * (is_q ? g.q_scale : 1.0f);
      }
    }
    const bool valid = t < a.T;
    if (active) {
      if constexpr (MODE == kOutPlain) {
        if (valid) a.out[(static_cast<size_t>(b) * a.T + t) * g.C_ch + ch] = val;
      } else {
        const PrefillWs &L = a.L;
        const float vv = valid ? val : 0.f;
        if (is_q || is_k) {
          const int kh = (is_q ? ch : ch - nq) / D;
          const int j = ch % D;
          const size_t row = (static_cast<size_t>(b) * g.H_k + kh) * L.T_pad + t;
          const int pos = (j & ~31) + kslot(j & 31);
          uint16_t hi, lo;
          split_bf16(vv, hi, lo);
          uint16_t *phi = reinterpret_cast<uint16_t *>(a.ws + (is_q ? L.q_hi : L.k_hi));
          uint16_t *plo = reinterpret_cast<uint16_t *>(a.ws + (is_q ? L.q_lo : L.k_lo));
          phi[row * L.Dp + pos] = hi;
          plo[row * L.Dp + pos] = lo;
          if constexpr (D < 32) {  // zero the unused half of the 32-wide K step
            phi[row * L.Dp + kslot(j + 16)] = 0;
            plo[row * L.Dp + kslot(j + 16)] = 0;
          }
          if (is_k) {
            const size_t blk = (static_cast<size_t>(b) * g.H_k + kh) * (L.T_pad / 32) + t / 32;
            const size_t idx = (blk * D + j) * 32 + kslot(static_cast<int>(t & 31));
            reinterpret_cast<uint16_t *>(a.ws + L.kT_hi)[idx] = hi;
            reinterpret_cast<uint16_t *>(a.ws + L.kT_lo)[idx] = lo;
          }
        } else {
          const int h = (ch - nqk) / D;
          const int j = ch % D;
          const size_t blk = (static_cast<size_t>(b) * g.H_v + h) * (L.T_pad / 16) + t / 16;
          reinterpret_cast<float *>(a.ws + L.vT)[(blk * D + j) * 16 + (t & 15)] = vv;
        }
      }
    }
    x0 = x1;
    x1 = x2;
    x2 = x3;
  }
  if (a.fuse_roll && active) {
    // The block walked every token, so (x0, x1, x2) are the last three rows of
    // concat(history, x); this thread alone reads and writes its channel.
    store_elem<DT>(a.hist, (static_cast<size_t>(b) * 3 + 0) * g.C_ch + ch, x0);
    store_elem<DT>(a.hist, (static_cast<size_t>(b) * 3 + 1) * g.C_ch + ch, x1);
    store_elem<DT>(a.hist, (static_cast<size_t>(b) * 3 + 2) * g.C_ch + ch, x2);
  }
}

// History after T tokens: the last three rows of concat(history, x), copied
// bit for bit.  Runs after every reader of the old history has finished.
template <typename E>
__global__ __launch_bounds__(256) void roll_kernel(int C_ch, int64_t T, const E *x, E *hist) {
  const int ch = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (ch >= C_ch) return;
  E v[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int64_t src = T + r;  // index into concat(history[0..2], x[0..T-1])
    v[r] = src < 3 ? hist[(static_cast<size_t>(b) * 3 + src) * C_ch + ch]
                   : x[(static_cast<size_t>(b) * T + (src - 3)) * C_ch + ch];
  }
#pragma unroll
  for (int r = 0; r < 3; ++r) hist[(static_cast<size_t>(b) * 3 + r) * C_ch + ch] = v[r];
}

template <int MODE>
static hipError_t launch_conv(const Geom &g, const ConvArgs &a, hipStream_t s) {
  const int64_t tiles = (a.T_iter + kConvTT - 1) / kConvTT;
  dim3 grid(static_cast<unsigned>(tiles), (g.C_ch + kConvThreads - 1) / kConvThreads, g.B);
  dim3 block(kConvThreads);
  if (g.D == 128) {
    if (g.in_dt == 0)
      hipLaunchKernelGGL((conv_kernel<0, 128, MODE>), grid, block, 0, s, g, a);
    else
      hipLaunchKernelGGL((conv_kernel<1, 128, MODE>), grid, block, 0, s, g, a);
  } else {
    if (g.in_dt == 0)
      hipLaunchKernelGGL((conv_kernel<0, 16, MODE>), grid, block, 0, s, g, a);
    else
      hipLaunchKernelGGL((conv_kernel<1, 16, MODE>), grid, block, 0, s, g, a);
  }
  return hipGetLastError();
}

hipError_t launch_conv_roll(const Geom &g, int64_t T, const void *x, void *hist,
                            hipStream_t s) {
  dim3 grid((g.C_ch + 255) / 256, g.B);
  if (g.in_dt == 0)
    hipLaunchKernelGGL(roll_kernel<uint32_t>, grid, dim3(256), 0, s, g.C_ch, T,
                       static_cast<const uint32_t *>(x), static_cast<uint32_t *>(hist));
  else
    hipLaunchKernelGGL(roll_kernel<uint16_t>, grid, dim3(256), 0, s, g.C_ch, T,
                       static_cast<const uint16_t *>(x), static_cast<uint16_t *>(hist));
  return hipGetLastError();
}

hipError_t launch_conv_plain(const Geom &g, int64_t T, const void *x, const void *w,
                             void *hist, float *out, hipStream_t s) {
  ConvArgs a{};
  a.x = x;
  a.w = w;
  a.hist = hist;
  a.out = out;
  a.T = T;
  a.T_iter = T;
  a.fuse_roll = T <= kConvTT;
  hipError_t e = launch_conv<kOutPlain>(g, a, s);
  if (e != hipSuccess || a.fuse_roll) return e;
  return launch_conv_roll(g, T, x, hist, s);
}

hipError_t launch_conv_prefill(const Geom &g, const PrefillWs &L, const void *x,
                               const void *w, const void *hist, char *ws, hipStream_t s) {
  ConvArgs a{};
  a.x = x;
  a.w = w;
  a.hist = const_cast<void *>(hist);
  a.ws = ws;
  a.L = L;
  a.T = L.T;
  a.T_iter = L.T_pad;
  a.fuse_roll = 0;
  return launch_conv<kOutPrefill>(g, a, s);
}

}  // namespace gdn
