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

// Sums of squares over the D consecutive threads of one head, for all kConvTT
// tokens of the tile at once (one LDS exchange when a head spans two waves).
template <int D, int TT>
__device__ __forceinline__ void head_sums(float (&ss)[TT], float (*red)[kConvTT]) {
  if constexpr (D <= 64) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int m = D / 2; m >= 1; m >>= 1) ss[t] += __shfl_xor(ss[t], m, kWave);
  } else {
    static_assert(D == 128, "heads of 16 or 128 channels");
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float v = wave_sum(ss[t]);
      if ((threadIdx.x & 63) == 0) red[w][t] = v;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TT; ++t) ss[t] = red[0][t] + red[1][t];
  }
}

// One thread per channel and kConvTT tokens: the tile's inputs (plus the three
// previous rows) are loaded up front, so every x element is read once and all
// loads are in flight together; the per-channel outputs stay in registers,
// which makes the dim-major workspace rows contiguous per thread.
template <int DT, int D, int MODE, int TT>
__global__ __launch_bounds__(kConvThreads) void conv_kernel(Geom g, ConvArgs a) {
  __shared__ float red[2][kConvTT];
  const int ch = blockIdx.y * kConvThreads + threadIdx.x;
  const int b = blockIdx.z;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TT;
  const bool active = ch < g.C_ch;
  const int nq = g.H_k * D;
  const int nqk = 2 * nq;
  const bool is_q = ch < nq;
  const bool is_k = !is_q && ch < nqk;
  // For D = 128 a block is exactly one head, so this is uniform per block.
  const bool qk_block = (D == 128) ? (blockIdx.y * kConvThreads < nqk) : true;

  float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f;
  float xv[TT + 3];
  if (active) {
    w0 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 0);
    w1 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 1);
    w2 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 2);
    w3 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 3);
  }
#pragma unroll
  for (int i = 0; i < TT + 3; ++i) {
    const int64_t tau = t0 - 3 + i;
    float v = 0.f;
    if (active && tau < a.T) {
      v = tau >= 0 ? load_elem<DT>(a.x, (static_cast<size_t>(b) * a.T + tau) * g.C_ch + ch)
                   : load_elem<DT>(a.hist, (static_cast<size_t>(b) * 3 + 3 + tau) * g.C_ch + ch);
    }
    xv[i] = v;
  }
  float val[TT], ss[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    val[t] = siluf_(conv4(w0, w1, w2, w3, xv[t], xv[t + 1], xv[t + 2], xv[t + 3]));
    ss[t] = val[t] * val[t];
  }
  if (qk_block) {
    head_sums<D, TT>(ss, red);
    if (is_q || is_k) {
      const float sc = is_q ? g.q_scale : 1.0f;
#pragma unroll
      for (int t = 0; t < TT; ++t) val[t] = val[t] * (1.0f / __builtin_sqrtf(ss[t] + g.eps)) * sc;
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t)
    if (t0 + t >= a.T) val[t] = 0.f;  // padding tokens of the prefill layout
  if (!active) return;

  if constexpr (MODE == kOutPlain) {
    const int64_t n = (a.T - t0 < TT) ? a.T - t0 : TT;
#pragma unroll
    for (int t = 0; t < TT; ++t)
      if (t < n) a.out[(static_cast<size_t>(b) * a.T + t0 + t) * g.C_ch + ch] = val[t];
    if (a.fuse_roll) {
      // The block holds every token, so rows T..T+2 of xv are the last three
      // rows of concat(history, x); this thread alone reads and writes them.
      const int T = static_cast<int>(a.T);
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < TT + 3; ++i)
          if (i == T + r) v = xv[i];
        store_elem<DT>(a.hist, (static_cast<size_t>(b) * 3 + r) * g.C_ch + ch, v);
      }
    }
  } else if constexpr (TT == kConvTT) {
    const PrefillWs &L = a.L;
    const int j = ch % D;
    if (is_q || is_k) {
      const int kh = (is_q ? ch : ch - nq) / D;
      // slice-major: [b][kh][j / 32][t][32]
      const size_t row0 = ((static_cast<size_t>(b) * g.H_k + kh) * (L.Dp / 32) + (j >> 5)) * L.T_pad + t0;
      const int pos = kslot(j & 31);
      uint16_t *phi = reinterpret_cast<uint16_t *>(a.ws + (is_q ? L.q_hi : L.k_hi));
      uint16_t *plo = reinterpret_cast<uint16_t *>(a.ws + (is_q ? L.q_lo : L.k_lo));
      uint16_t hi[TT], lo[TT];
#pragma unroll
      for (int t = 0; t < TT; t += 2) {
        uint32_t h2, l2;
        split2(val[t], val[t + 1], h2, l2);
        hi[t] = static_cast<uint16_t>(h2);
        hi[t + 1] = static_cast<uint16_t>(h2 >> 16);
        lo[t] = static_cast<uint16_t>(l2);
        lo[t + 1] = static_cast<uint16_t>(l2 >> 16);
      }
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        phi[(row0 + t) * 32 + pos] = hi[t];
        plo[(row0 + t) * 32 + pos] = lo[t];
        if constexpr (D < 32) {  // zero the unused half of the 32-wide K step
          phi[(row0 + t) * 32 + kslot(j + 16)] = 0;
          plo[(row0 + t) * 32 + kslot(j + 16)] = 0;
        }
      }
      if (is_k) {
        // Dim-major row of this channel: 32 tokens in permuted K order.
        u16x8 rh[4], rl[4];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int sl = kslot(t);
          rh[sl >> 3][sl & 7] = hi[t];
          rl[sl >> 3][sl & 7] = lo[t];
        }
        const size_t blk = (static_cast<size_t>(b) * g.H_k + kh) * (L.T_pad / 32) + t0 / 32;
        u16x8 *dh = reinterpret_cast<u16x8 *>(reinterpret_cast<uint16_t *>(a.ws + L.kT_hi) + (blk * D + j) * 32);
        u16x8 *dl = reinterpret_cast<u16x8 *>(reinterpret_cast<uint16_t *>(a.ws + L.kT_lo) + (blk * D + j) * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          dh[q] = rh[q];
          dl[q] = rl[q];
        }
      }
    } else {
      const int h = (ch - nqk) / D;
#pragma unroll
      for (int half = 0; half < TT / 16; ++half) {
        const size_t blk = (static_cast<size_t>(b) * g.H_v + h) * (L.T_pad / 16) + t0 / 16 + half;
        float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.ws + L.vT) + (blk * D + j) * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dst[q] = make_float4(val[16 * half + 4 * q], val[16 * half + 4 * q + 1],
                               val[16 * half + 4 * q + 2], val[16 * half + 4 * q + 3]);
      }
    }
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

template <int MODE, int TT>
static hipError_t launch_conv(const Geom &g, const ConvArgs &a, hipStream_t s) {
  const int64_t tiles = (a.T_iter + TT - 1) / TT;
  dim3 grid(static_cast<unsigned>(tiles), (g.C_ch + kConvThreads - 1) / kConvThreads, g.B);
  dim3 block(kConvThreads);
  if (g.D == 128) {
    if (g.in_dt == 0)
      hipLaunchKernelGGL((conv_kernel<0, 128, MODE, TT>), grid, block, 0, s, g, a);
    else
      hipLaunchKernelGGL((conv_kernel<1, 128, MODE, TT>), grid, block, 0, s, g, a);
  } else {
    if (g.in_dt == 0)
      hipLaunchKernelGGL((conv_kernel<0, 16, MODE, TT>), grid, block, 0, s, g, a);
    else
      hipLaunchKernelGGL((conv_kernel<1, 16, MODE, TT>), grid, block, 0, s, g, a);
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
  // One token per sequence (decode): a one-token tile does no wasted work.
  hipError_t e = (T == 1) ? launch_conv<kOutPlain, 1>(g, a, s) : launch_conv<kOutPlain, kConvTT>(g, a, s);
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
  return launch_conv<kOutPrefill, kConvTT>(g, a, s);
}

}  // namespace gdn
