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
constexpr int kConvQKTT = 16;      // tokens per block of the q/k prefill conv

// kOutPrefillQK: the prefill layout for the q and k channels only, without
// the dim-major k copy (so without the LDS staging buffer, which would cap
// the blocks per CU).
enum { kOutPlain = 0, kOutPrefill = 1, kOutPrefillQK = 2 };

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
  int write_kT;    // prefill layout: also write the dim-major copy of k
  int write_v;     // prefill layout: also compute and write v (else q, k only)
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

// Per-token factor sc / sqrt(sum of squares + eps) of one 128-channel head
// held by the block's two waves, for 32 tokens.  On entry ss[t] is this
// lane's square for token t, on exit the factor for token t.  The 32 sums over
// 64 lanes are a transpose-reduce: every exchange hands half of the remaining
// tokens to a partner lane and keeps the other half, so the lane-swap
// instructions of gfx950 (distance 32, then 16) and DPP (the rest) need
// 16 + 8 + 4 + 2 + 1 + 1 exchanges, after which lane l holds token l / 2.  The
// two waves' partial sums meet in LDS, one reciprocal square root per lane
// follows, and a wave-local LDS broadcast hands every lane all 32 factors.
__device__ __forceinline__ void head_scale_128x32(float (&ss)[32], float eps, float sc,
                                                  float (*red)[kConvTT],
                                                  float (*bc)[kConvTT]) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss[i]),
                                                    __float_as_uint(ss[i + 16]), false, false);
    ss[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(ss[i]),
                                                    __float_as_uint(ss[i + 8]), false, false);
    ss[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  tr_step<8, 0x140, 8>(ss, lane);
  tr_step<4, 0x141, 4>(ss, lane);
  tr_step<2, 0x4E, 2>(ss, lane);
  const float s = ss[0] + dpp_f<0xB1>(ss[0]);
  const int t = lane >> 1;
  if ((lane & 1) == 0) red[w][t] = s;
  __syncthreads();
  const float f = __builtin_amdgcn_rsqf(red[0][t] + red[1][t] + eps) * sc;
  if ((lane & 1) == 0) bc[w][t] = f;
  // Only this wave reads bc[w], after its own writes (LDS keeps a wave's
  // accesses in order).
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < kConvTT; ++i) ss[i] = bc[w][i];
}

// One thread per channel and kConvTT tokens: the tile's inputs (plus the three
// previous rows) are loaded up front, so every x element is read once and all
// loads are in flight together; the per-channel outputs stay in registers,
// which makes the dim-major workspace rows contiguous per thread.
template <int DT, int D, int MODE, int TT>
__global__ __launch_bounds__(kConvThreads, (MODE == kOutPrefillQK && D == 128 ? 8 : 1)) void conv_kernel(Geom g, ConvArgs a) {
  __shared__ float red[2][kConvTT];
  __shared__ float bc[2][kConvTT];
  // One grid dimension over (tile, channel block), channel block fastest: the
  // blocks in flight together read whole token rows of x.
  const int nchb = (MODE == kOutPrefillQK ? 2 * g.H_k * D : g.C_ch + kConvThreads - 1) / kConvThreads;
  const int cb = static_cast<int>(blockIdx.x % nchb);
  const int ch = cb * kConvThreads + threadIdx.x;
  const int b = blockIdx.z;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x / nchb) * TT;
  const bool active = ch < g.C_ch;
  // Lanes past the last channel load a valid channel and drop their results,
  // so every load below is unconditional per lane.
  const int chc = active ? ch : g.C_ch - 1;
  const int nq = g.H_k * D;
  const int nqk = 2 * nq;
  // For D = 128 a block is exactly one head: the kind is uniform per block.
  const int head0 = (D == 128) ? cb * kConvThreads : ch;
  const bool is_q = head0 < nq;
  const bool is_k = !is_q && head0 < nqk;
  const bool qk_block = (D == 128) ? (is_q || is_k) : true;
  constexpr int ES = DT == 0 ? 4 : 2;
  const size_t rowb = static_cast<size_t>(g.C_ch) * ES;
  const uint32_t lane_off = static_cast<uint32_t>(chc) * ES;

  auto ld = [&](const void *row_base) -> float {
    if constexpr (DT == 0)
      return *reinterpret_cast<const float *>(static_cast<const char *>(row_base) + lane_off);
    else
      return bf16_bits_to_f32(
          *reinterpret_cast<const uint16_t *>(static_cast<const char *>(row_base) + lane_off));
  };
  const char *wrow = static_cast<const char *>(a.w);
  const float w0 = load_elem<DT>(wrow, static_cast<size_t>(chc) * 4 + 0);
  const float w1 = load_elem<DT>(wrow, static_cast<size_t>(chc) * 4 + 1);
  const float w2 = load_elem<DT>(wrow, static_cast<size_t>(chc) * 4 + 2);
  const float w3 = load_elem<DT>(wrow, static_cast<size_t>(chc) * 4 + 3);
  float xv[TT + 3];
  const char *xb = static_cast<const char *>(a.x) + static_cast<size_t>(b) * a.T * rowb;
  if (t0 >= 3 && t0 + TT <= a.T) {
    // Interior tile: rows t0 - 3 .. t0 + TT - 1 all come from x.
    const char *r0 = xb + static_cast<size_t>(t0 - 3) * rowb;
#pragma unroll
    for (int i = 0; i < TT + 3; ++i) xv[i] = ld(r0 + i * rowb);
  } else {
    const char *hb = static_cast<const char *>(a.hist) + static_cast<size_t>(b) * 3 * rowb;
#pragma unroll
    for (int i = 0; i < TT + 3; ++i) {
      const int64_t tau = t0 - 3 + i;  // uniform per block
      float v = 0.f;
      if (tau < 0)
        v = ld(hb + static_cast<size_t>(3 + tau) * rowb);
      else if (tau < a.T)
        v = ld(xb + static_cast<size_t>(tau) * rowb);
      xv[i] = v;
    }
  }
  float val[TT], ss[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    val[t] = siluf_(conv4(w0, w1, w2, w3, xv[t], xv[t + 1], xv[t + 2], xv[t + 3]));
    ss[t] = val[t] * val[t];
  }
  if (qk_block) {
    if constexpr (D == 128 && TT == kConvTT) {
      head_scale_128x32(ss, g.eps, is_q ? g.q_scale : 1.0f, red, bc);
#pragma unroll
      for (int t = 0; t < TT; ++t) val[t] *= ss[t];
    } else {
      head_sums<D, TT>(ss, red);
      if (is_q || is_k) {
        const float sc = is_q ? g.q_scale : 1.0f;
#pragma unroll
        for (int t = 0; t < TT; ++t) val[t] *= __builtin_amdgcn_rsqf(ss[t] + g.eps) * sc;
      }
    }
  }
  if (t0 + TT > a.T) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
      if (t0 + t >= a.T) val[t] = 0.f;  // padding tokens of the prefill layout
  }
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
    // 16 KB: one head's dim-major block (v: 2 x 16 tokens fp32; k: hi and lo).
    __shared__ uint4 stage[(D == kConvThreads && MODE == kOutPrefill) ? 1024 : 1];
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
      if (MODE == kOutPrefill && is_k && a.write_kT) {
        // Dim-major row of this channel: 32 tokens in permuted K order.
        u16x8 rh[4], rl[4];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int sl = kslot(t);
          rh[sl >> 3][sl & 7] = hi[t];
          rl[sl >> 3][sl & 7] = lo[t];
        }
        const size_t blk = (static_cast<size_t>(b) * g.H_k + kh) * (L.T_pad / 32) + t0 / 32;
        if constexpr (D == kConvThreads) {
          // The head's rows form one 8 KB block per half (hi, lo): gather it
          // in LDS and write it with lane-contiguous 16-byte stores.
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            stage[j * 4 + q] = __builtin_bit_cast(uint4, rh[q]);
            stage[512 + j * 4 + q] = __builtin_bit_cast(uint4, rl[q]);
          }
          __syncthreads();
          uint4 *dh = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.ws + L.kT_hi) + blk * D * 32);
          uint4 *dl = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.ws + L.kT_lo) + blk * D * 32);
#pragma unroll
          for (int u = 0; u < 4; ++u) st_stream(dh + threadIdx.x + kConvThreads * u, stage[threadIdx.x + kConvThreads * u]);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            st_stream(dl + threadIdx.x + kConvThreads * u, stage[512 + threadIdx.x + kConvThreads * u]);
        } else {
          u16x8 *dh = reinterpret_cast<u16x8 *>(reinterpret_cast<uint16_t *>(a.ws + L.kT_hi) + (blk * D + j) * 32);
          u16x8 *dl = reinterpret_cast<u16x8 *>(reinterpret_cast<uint16_t *>(a.ws + L.kT_lo) + (blk * D + j) * 32);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            dh[q] = rh[q];
            dl[q] = rl[q];
          }
        }
      }
    } else if constexpr (MODE == kOutPrefill) {
      const int h = (ch - nqk) / D;
      if constexpr (D == kConvThreads) {
        // Both 16-token blocks of the head are one contiguous 16 KB run:
        // gather it in LDS and write it with lane-contiguous 16-byte stores.
#pragma unroll
        for (int half = 0; half < TT / 16; ++half)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            stage[(half * D + j) * 4 + q] = __builtin_bit_cast(
                uint4, make_float4(val[16 * half + 4 * q], val[16 * half + 4 * q + 1],
                                   val[16 * half + 4 * q + 2], val[16 * half + 4 * q + 3]));
        __syncthreads();
        const size_t blk = (static_cast<size_t>(b) * g.H_v + h) * (L.T_pad / 16) + t0 / 16;
        uint4 *dst = reinterpret_cast<uint4 *>(reinterpret_cast<float *>(a.ws + L.vT) + blk * D * 16);
#pragma unroll
        for (int u = 0; u < 8; ++u) st_stream(dst + threadIdx.x + kConvThreads * u, stage[threadIdx.x + kConvThreads * u]);
      } else {
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
}

// Prefill conv of the q and k channels at d = 128, one head per block, for
// NTL consecutive 16-token tiles: with NTL > 1 the next tile's inputs are
// loaded while the current tile is computed and stored.  One 16-token tile
// per block (NTL = 1, twice conv_kernel's block count) measured faster than
// 32-token tiles and than several tiles per block: the blocks on a CU drift
// apart, so one block's loads overlap another's arithmetic and stores.  Same
// conv and output layout as conv_kernel's prefill layout; the head sums add
// in another order.
template <int DT, int NTL>
__global__ __launch_bounds__(kConvThreads) void conv_qk_kernel(Geom g, ConvArgs a) {
  constexpr int TT = kConvQKTT, D = 128;
  static_assert(kConvThreads == 128 && TT == 16, "store pieces sized for 128 threads x 16 tokens");
  __shared__ float red[2][TT];
  __shared__ float bc[2][TT];
  const PrefillWs &L = a.L;
  // One grid dimension over (tile group, head), head fastest: the blocks in
  // flight together read whole token rows of x (each block 256 bytes of a row).
  const int nheads = 2 * g.H_k;
  const int hd = static_cast<int>(blockIdx.x % nheads);
  const int ch = hd * kConvThreads + threadIdx.x;  // a q or k channel
  const int b = blockIdx.z;
  const int nq = g.H_k * D;
  const bool is_q = hd < g.H_k;  // uniform
  const int kh = (is_q ? ch : ch - nq) / D;
  const int j = ch % D;
  const float sc = is_q ? g.q_scale : 1.0f;
  constexpr int ES = DT == 0 ? 4 : 2;
  const size_t rowb = static_cast<size_t>(g.C_ch) * ES;
  const uint32_t lane_off = static_cast<uint32_t>(ch) * ES;
  auto ld = [&](const char *row_base) -> float {
    if constexpr (DT == 0)
      return *reinterpret_cast<const float *>(row_base + lane_off);
    else
      return bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(row_base + lane_off));
  };
  const float w0 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 0);
  const float w1 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 1);
  const float w2 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 2);
  const float w3 = load_elem<DT>(a.w, static_cast<size_t>(ch) * 4 + 3);
  const char *xb = static_cast<const char *>(a.x) + static_cast<size_t>(b) * a.T * rowb;
  const char *hb = static_cast<const char *>(a.hist) + static_cast<size_t>(b) * 3 * rowb;
  auto load_tile = [&](int64_t t0, float (&xv)[TT + 3]) {
    if (t0 >= 3 && t0 + TT <= a.T) {
      const char *r0 = xb + static_cast<size_t>(t0 - 3) * rowb;
#pragma unroll
      for (int i = 0; i < TT + 3; ++i) xv[i] = ld(r0 + i * rowb);
    } else {
#pragma unroll
      for (int i = 0; i < TT + 3; ++i) {
        const int64_t tau = t0 - 3 + i;  // uniform per block
        float v = 0.f;
        if (tau < 0)
          v = ld(hb + static_cast<size_t>(3 + tau) * rowb);
        else if (tau < a.T)
          v = ld(xb + static_cast<size_t>(tau) * rowb);
        xv[i] = v;
      }
    }
  };
  uint16_t *phi = reinterpret_cast<uint16_t *>(a.ws + (is_q ? L.q_hi : L.k_hi));
  uint8_t *plo = reinterpret_cast<uint8_t *>(a.ws + (is_q ? L.q_lo : L.k_lo));  // e4m3 low halves
  const float lo_scale = is_q ? L.q_lo_scale : L.k_lo_scale;
  // Slice 0 of this head: [b][kh][slice][T_pad][32] token-major layout.
  const size_t slice0 = (static_cast<size_t>(b) * g.H_k + kh) * (L.Dp / 32) * L.T_pad;
  const int pos = kslot(j & 31);
  __shared__ __attribute__((aligned(16))) uint16_t stage_hi[4][TT][32];
  __shared__ __attribute__((aligned(16))) uint8_t stage_lo[4][TT][32];
  const int64_t first = static_cast<int64_t>(blockIdx.x / nheads) * NTL * TT;
  const int64_t last_t0 = a.T_iter - TT;  // last tile of the sequence
  float xa[TT + 3];
  load_tile(first, xa);
#pragma unroll
  for (int it = 0; it < NTL; ++it) {
    const int64_t t0 = first + it * TT;
    if (t0 > last_t0) break;  // uniform: the grid's last block may hold fewer tiles
    float xn[TT + 3];
    if (it + 1 < NTL) load_tile(t0 + TT <= last_t0 ? t0 + TT : t0, xn);
    float val[TT], ss[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      val[t] = siluf_(conv4(w0, w1, w2, w3, xa[t], xa[t + 1], xa[t + 2], xa[t + 3]));
      ss[t] = val[t] * val[t];
    }
    head_scale_128x16(ss, g.eps, sc, red, bc, threadIdx.x >> 6);
#pragma unroll
    for (int t = 0; t < TT; ++t) val[t] *= ss[t];
    if (t0 + TT > a.T) {
#pragma unroll
      for (int t = 0; t < TT; ++t)
        if (t0 + t >= a.T) val[t] = 0.f;  // padding tokens of the prefill layout
    }
    // The head's token-major output for the tile is four 1 KB runs of hi
    // (bf16) and four 512-byte runs of lo (e4m3), one per 32-channel slice:
    // gather them in LDS, then write 16-byte pieces (three store
    // instructions per thread instead of 32).
#pragma unroll
    for (int t = 0; t < TT; t += 2) {
      uint32_t h2;
      uint16_t l2;
      split2_lo8(val[t], val[t + 1], lo_scale, h2, l2);
      stage_hi[j >> 5][t][pos] = static_cast<uint16_t>(h2);
      stage_hi[j >> 5][t + 1][pos] = static_cast<uint16_t>(h2 >> 16);
      stage_lo[j >> 5][t][pos] = static_cast<uint8_t>(l2);
      stage_lo[j >> 5][t + 1][pos] = static_cast<uint8_t>(l2 >> 8);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int piece = threadIdx.x + kConvThreads * u;  // 16-byte piece of the 4 KB of hi
      const int sl = piece >> 6, tok = (piece >> 2) & 15, part = piece & 3;
      uint16_t *dst = phi + ((slice0 + sl * L.T_pad + t0 + tok) * 32 + 8 * part);
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(&stage_hi[sl][tok][8 * part]),
                                  reinterpret_cast<u32x4 *>(dst));
    }
    {
      const int piece = threadIdx.x;  // 16-byte piece of the 2 KB of lo
      const int sl = piece >> 5, tok = (piece >> 1) & 15, part = piece & 1;
      uint8_t *dst = plo + ((slice0 + sl * L.T_pad + t0 + tok) * 32 + 16 * part);
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(&stage_lo[sl][tok][16 * part]),
                                  reinterpret_cast<u32x4 *>(dst));
    }
    if (it + 1 < NTL) {
      // red, bc and the stages are reused by the next tile.
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TT + 3; ++i) xa[i] = xn[i];
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

// Decode step of TT tokens per sequence: one thread owns one channel for BB
// sequences, so a block does BB rows of work and the per-head sums of all BB
// rows and TT tokens share one LDS exchange.  The history is read from the
// sequence's in slot and the history after token t (the last three raw
// inputs up to t) is stored to its out slot for t, by the thread that read
// the channel, after it has read it; a sequence whose in slot lies outside
// [0, n_slots) is skipped (slot rules as in decode.hip).
// out: [B][TT][C_ch] fp32, read by the state-stream kernel.
template <int DT, int D, int BB, int TT>
__global__ __launch_bounds__(kConvThreads) void conv_step_kernel(Geom g, const void *x,
                                                                 const void *w, void *hist,
                                                                 float *out, const int32_t *in_slots,
                                                                 const int32_t *out_slots,
                                                                 int n_slots) {
  static_assert(BB * TT <= kConvTT, "one LDS exchange for all rows and tokens");
  __shared__ float red[2][kConvTT];
  const int ch = blockIdx.x * kConvThreads + threadIdx.x;
  const int b0 = blockIdx.y * BB;
  const bool active = ch < g.C_ch;
  const int chc = active ? ch : g.C_ch - 1;
  const int nq = g.H_k * D;
  const int head0 = (D == 128) ? static_cast<int>(blockIdx.x) * kConvThreads : ch;
  const bool is_q = head0 < nq;
  const bool is_k = !is_q && head0 < 2 * nq;
  const bool qk_block = (D == 128) ? (is_q || is_k) : true;
  const size_t C = g.C_ch;
  const float w0 = load_elem<DT>(w, static_cast<size_t>(chc) * 4 + 0);
  const float w1 = load_elem<DT>(w, static_cast<size_t>(chc) * 4 + 1);
  const float w2 = load_elem<DT>(w, static_cast<size_t>(chc) * 4 + 2);
  const float w3 = load_elem<DT>(w, static_cast<size_t>(chc) * 4 + 3);
  float xv[BB][3 + TT], val[BB * TT], ss[BB * TT];
  int sin[BB];
#pragma unroll
  for (int r = 0; r < BB; ++r) {
    const int b = b0 + r < g.B ? b0 + r : g.B - 1;  // rows past B re-read the last one
    const int sl = in_slots ? in_slots[b] : b;
    sin[r] = (b0 + r < g.B && sl >= 0 && sl < n_slots) ? sl : -1;
    const int src = sin[r] >= 0 ? sin[r] : 0;  // padding rows read slot 0, use nothing
#pragma unroll
    for (int k = 0; k < 3; ++k) xv[r][k] = load_elem<DT>(hist, (static_cast<size_t>(src) * 3 + k) * C + chc);
#pragma unroll
    for (int t = 0; t < TT; ++t)
      xv[r][3 + t] = load_elem<DT>(x, (static_cast<size_t>(b) * TT + t) * C + chc);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      val[r * TT + t] = siluf_(conv4(w0, w1, w2, w3, xv[r][t], xv[r][t + 1], xv[r][t + 2], xv[r][t + 3]));
      ss[r * TT + t] = val[r * TT + t] * val[r * TT + t];
    }
  }
  if (qk_block) {
    head_sums<D, BB * TT>(ss, red);
    if (is_q || is_k) {
      const float sc = is_q ? g.q_scale : 1.0f;
#pragma unroll
      for (int k = 0; k < BB * TT; ++k) val[k] *= __builtin_amdgcn_rsqf(ss[k] + g.eps) * sc;
    }
  }
  if (!active) return;
#pragma unroll
  for (int r = 0; r < BB; ++r) {
    const int b = b0 + r;
    if (sin[r] < 0) continue;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      out[(static_cast<size_t>(b) * TT + t) * C + ch] = val[r * TT + t];
      const int o = out_slots ? out_slots[static_cast<size_t>(b) * TT + t]
                              : (t == TT - 1 ? sin[r] : -1);
      if (o >= 0 && o < n_slots) {
#pragma unroll
        for (int k = 0; k < 3; ++k)
          store_elem<DT>(hist, (static_cast<size_t>(o) * 3 + k) * C + ch, xv[r][t + 1 + k]);
      }
    }
  }
}

template <int D, int BB, int TT>
static hipError_t launch_conv_step_t(const Geom &g, const void *x, const void *w, void *hist,
                                     float *out, const int32_t *in_slots,
                                     const int32_t *out_slots, int n_slots, hipStream_t s,
                                     const KernelEvents *ev) {
  dim3 grid((g.C_ch + kConvThreads - 1) / kConvThreads, (g.B + BB - 1) / BB);
  if (g.in_dt == 0)
    launch_kernel(conv_step_kernel<0, D, BB, TT>, grid, dim3(kConvThreads), s, ev, g, x, w, hist, out,
                  in_slots, out_slots, n_slots);
  else
    launch_kernel(conv_step_kernel<1, D, BB, TT>, grid, dim3(kConvThreads), s, ev, g, x, w, hist, out,
                  in_slots, out_slots, n_slots);
  return hipGetLastError();
}

template <int TT>
static hipError_t launch_conv_step_tt(const Geom &g, const void *x, const void *w, void *hist,
                                      float *out, const int32_t *in_slots,
                                      const int32_t *out_slots, int n_slots, hipStream_t s,
                                      const KernelEvents *ev) {
  // d = 128: two sequences per block (B = 64: 2,560 blocks) measured faster
  // than eight (640 blocks: too few waves in flight for the short loads).
  if (g.D == 128)
    return g.B >= 8 ? launch_conv_step_t<128, 2, TT>(g, x, w, hist, out, in_slots, out_slots, n_slots, s, ev)
                    : launch_conv_step_t<128, 1, TT>(g, x, w, hist, out, in_slots, out_slots, n_slots, s, ev);
  return g.B >= 8 && TT == 1
             ? launch_conv_step_t<16, 8, TT>(g, x, w, hist, out, in_slots, out_slots, n_slots, s, ev)
             : launch_conv_step_t<16, 1, TT>(g, x, w, hist, out, in_slots, out_slots, n_slots, s, ev);
}

hipError_t launch_conv_step(const Geom &g, int T, const void *x, const void *w, void *hist,
                            float *out, const int32_t *in_slots, const int32_t *out_slots,
                            int n_slots, hipStream_t s, const KernelEvents *ev) {
  switch (T) {
    case 1: return launch_conv_step_tt<1>(g, x, w, hist, out, in_slots, out_slots, n_slots, s, ev);
    case 2: return launch_conv_step_tt<2>(g, x, w, hist, out, in_slots, out_slots, n_slots, s, ev);
    case 3: return launch_conv_step_tt<3>(g, x, w, hist, out, in_slots, out_slots, n_slots, s, ev);
    case 4: return launch_conv_step_tt<4>(g, x, w, hist, out, in_slots, out_slots, n_slots, s, ev);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE, int TT>
static hipError_t launch_conv(const Geom &g, const ConvArgs &a, hipStream_t s,
                              const KernelEvents *ev = nullptr) {
  const int64_t tiles = (a.T_iter + TT - 1) / TT;
  // Without v the grid covers the q and k channels only (whole heads at d = 128).
  const int chans = (MODE == kOutPrefillQK) ? 2 * g.H_k * g.D : g.C_ch;
  dim3 grid(static_cast<unsigned>(tiles * ((chans + kConvThreads - 1) / kConvThreads)), 1, g.B);
  dim3 block(kConvThreads);
  if (g.D == 128) {
    if (g.in_dt == 0)
      launch_kernel(conv_kernel<0, 128, MODE, TT>, grid, block, s, ev, g, a);
    else
      launch_kernel(conv_kernel<1, 128, MODE, TT>, grid, block, s, ev, g, a);
  } else {
    if (g.in_dt == 0)
      launch_kernel(conv_kernel<0, 16, MODE, TT>, grid, block, s, ev, g, a);
    else
      launch_kernel(conv_kernel<1, 16, MODE, TT>, grid, block, s, ev, g, a);
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
  a.write_v = 1;
  a.x = x;
  a.w = w;
  a.hist = hist;
  a.out = out;
  a.T = T;
  a.T_iter = T;
  a.fuse_roll = T <= kConvTT;
  if (T == 1) return launch_conv_step(g, 1, x, w, hist, out, nullptr, nullptr, g.B, s);
  hipError_t e = launch_conv<kOutPlain, kConvTT>(g, a, s);
  if (e != hipSuccess || a.fuse_roll) return e;
  return launch_conv_roll(g, T, x, hist, s);
}

hipError_t launch_conv_prefill(const Geom &g, const PrefillWs &L, const void *x,
                               const void *w, const void *hist, char *ws, hipStream_t s,
                               const KernelEvents *ev) {
  ConvArgs a{};
  a.x = x;
  a.w = w;
  a.hist = const_cast<void *>(hist);
  a.ws = ws;
  a.L = L;
  a.T = L.T;
  a.T_iter = L.T_pad;
  a.fuse_roll = 0;
  a.write_kT = !prefill_split_roles(g, L);
  a.write_v = !prefill_split_roles(g, L);
  if (a.write_v) return launch_conv<kOutPrefill, kConvTT>(g, a, s, ev);
  // q and k only (the split-role state pass computes v): d = 128.
  constexpr int NTL = 1;
  const int64_t tiles = a.T_iter / kConvQKTT;  // T_pad is a multiple of the 64-token chunk
  dim3 grid(static_cast<unsigned>(2 * g.H_k * ((tiles + NTL - 1) / NTL)), 1, g.B);
  if (g.in_dt == 0)
    launch_kernel(conv_qk_kernel<0, NTL>, grid, dim3(kConvThreads), s, ev, g, a);
  else
    launch_kernel(conv_qk_kernel<1, NTL>, grid, dim3(kConvThreads), s, ev, g, a);
  return hipGetLastError();
}

}  // namespace gdn
