// prefill.hip -- chunked gated delta rule (WY / UT-transform form) on bf16
// MFMA for gfx950, fused with the sigmoid output gate.
//
// For one value head, a chunk of C tokens with entry state S0 (d_v x d_k),
// G_t = sum_{r<=t} g_r, gamma_t = exp(G_t), D_ts = exp(G_t - G_s):
//   A   = strict_lower(diag(beta) (D * K K^T))          chunk-local
//   Tm  = (I + A)^{-1}                                  chunk-local
//   P   = tril(D) * (Q K^T)                             chunk-local
//   R   = diag(beta) (V - diag(gamma) K S0^T)           needs S0
//   U   = Tm R                                          the delta-rule updates
//   O   = diag(gamma) Q S0^T + P U,   y = O * sigmoid(Z)
//   S   = gamma_last S0 + U^T diag(D_last,.) K
// This is the sequential recurrence of the gated delta rule (Yang, Kautz,
// Hatamizadeh, "Gated Delta Networks", ICLR 2025) regrouped per chunk, exact
// up to rounding; the pages ask for a separately tuned GDN prefill behind the
// same interface as decode ("Add a performance-parity Qwen3.8-27B Q4 and Q8
// text backend on Metal", section Scope) and for prefill/decode equivalence
// across chunk sizes ("Implement the Qwen3.8 Flash Next Rust and Metal text
// core", section Verification).
//
// Kernels:
//   prep  (B x H_k x chunks, parallel): K K^T and Q K^T once per key head on
//         MFMA (hi/lo split operands, fp32 accumulate), then for each of the
//         key head's value heads the fp32 blocked triangular inverse Tm and P,
//         stored as MFMA A operands.
//   state (B x H_v x d_v/16, serial over chunks): 16 rows of S per block, the
//         4 waves split d_k in quarters; S^T stays in MFMA accumulator
//         registers for the whole sequence.  Per chunk: K S^T and Q S^T
//         partials (reduced through LDS), U = Tm R, O = gamma QS + P U with
//         the gate fused into the store, and the rank-C state update.
// Precision: every product that carries the value path uses split bf16
// operands (hi + lo, 16 significant bits) with fp32 accumulation; only Tm
// (unit diagonal, small off-diagonal) is rounded to plain bf16.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// ---------------------------------------------------------------- shared helpers

// Prefix sums of the log decay over one chunk, computed by one wave.  Lane t
// gets G[t] in g0 and (C = 128) G[64 + t] in g1.  Tokens past the end of the
// sequence count as g = 0 (a padding token with beta = 0 changes nothing).
template <int C>
__device__ __forceinline__ void chunk_prefix(const float *__restrict__ gl, size_t base,
                                             int H_v, int n_valid, float &g0, float &g1) {
  const int lane = threadIdx.x & 63;
  float a = (lane < C && lane < n_valid) ? gl[base + static_cast<size_t>(lane) * H_v] : 0.f;
  g0 = wave_incl_scan(a);
  g1 = 0.f;
  if constexpr (C > 64) {
    float b = (64 + lane < n_valid) ? gl[base + static_cast<size_t>(64 + lane) * H_v] : 0.f;
    g1 = wave_incl_scan(b) + __shfl(g0, 63, kWave);
  }
}

template <int C>
__device__ __forceinline__ float prefix_at(float g0, float g1, int t) {
  if constexpr (C > 64) {
    const float lo = __shfl(g0, t & 63, kWave);
    const float hi = __shfl(g1, t & 63, kWave);
    return t < 64 ? lo : hi;
  } else {
    return __shfl(g0, t, kWave);
  }
}

__device__ __forceinline__ u16x8 load8(const uint16_t *p) {
  return *reinterpret_cast<const u16x8 *>(p);
}

__device__ __forceinline__ int tri_index(int mt, int nt) { return mt * (mt + 1) / 2 + nt; }

// ---------------------------------------------------------------- prep kernel

template <int D, int C>
struct PrepShape {
  static constexpr int NT = C / 16;               // 16-token tiles per chunk
  static constexpr int NTRI = NT * (NT + 1) / 2;  // lower tiles incl. diagonal
  static constexpr int Dp = D < 32 ? 32 : D;
  static constexpr int Cp = C < 32 ? 32 : C;
  static constexpr int KS_D = Dp / 32;  // K steps over the head dimension
};

template <int D, int C>
__global__ __launch_bounds__(256) void prep_kernel(Geom g, PrefillWs L,
                                                   const float *__restrict__ gl,
                                                   const float *__restrict__ beta,
                                                   char *__restrict__ ws) {
  using Sh = PrepShape<D, C>;
  constexpr int NT = Sh::NT, NTRI = Sh::NTRI, Dp = Sh::Dp, Cp = Sh::Cp;
  __shared__ float KK[NTRI][256];  // Gram tiles, row-major 16 x 16
  __shared__ float QK[NTRI][256];
  __shared__ float TI[NTRI][256];  // (I + A)^{-1}
  __shared__ float XS[NT > 1 ? NT - 1 : 1][256];
  __shared__ float Gs[C], Bs[C];

  const int chunk = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, gq = lane >> 4;
  const int64_t tau0 = static_cast<int64_t>(chunk) * C;
  const int n_valid = static_cast<int>((L.T - tau0) < C ? (L.T - tau0) : C);

  // 1. K K^T and Q K^T, lower tiles only, split operands.
  {
    const size_t row0 = (static_cast<size_t>(b) * g.H_k + kh) * L.T_pad + tau0;
    const uint16_t *khi = reinterpret_cast<const uint16_t *>(ws + L.k_hi);
    const uint16_t *klo = reinterpret_cast<const uint16_t *>(ws + L.k_lo);
    const uint16_t *qhi = reinterpret_cast<const uint16_t *>(ws + L.q_hi);
    const uint16_t *qlo = reinterpret_cast<const uint16_t *>(ws + L.q_lo);
    for (int job = wave; job < 2 * NTRI; job += 4) {
      const bool is_q = job >= NTRI;
      const int tri = is_q ? job - NTRI : job;
      int mt = 0;
      while (tri_index(mt + 1, 0) <= tri) ++mt;
      const int nt = tri - tri_index(mt, 0);
      const uint16_t *ah = is_q ? qhi : khi;
      const uint16_t *al = is_q ? qlo : klo;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < Sh::KS_D; ++ks) {
        const size_t ao = (row0 + 16 * mt + c) * Dp + 32 * ks + 8 * gq;
        const size_t bo = (row0 + 16 * nt + c) * Dp + 32 * ks + 8 * gq;
        acc = mfma_split3(load8(ah + ao), load8(al + ao), load8(khi + bo), load8(klo + bo), acc);
      }
      float *dst = is_q ? QK[tri] : KK[tri];
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(4 * gq + r) * 16 + c] = acc[r];
    }
  }

  for (int jv = 0; jv < g.G; ++jv) {
    const int h = kh * g.G + jv;
    __syncthreads();  // Gram tiles written; previous head's readers done
    if (wave == 0) {
      float g0, g1;
      const size_t base = (static_cast<size_t>(b) * L.T + tau0) * g.H_v + h;
      chunk_prefix<C>(gl, base, g.H_v, n_valid, g0, g1);
      if (lane < C) {
        Gs[lane] = g0;
        Bs[lane] = lane < n_valid ? beta[base + static_cast<size_t>(lane) * g.H_v] : 0.f;
      }
      if constexpr (C > 64) {
        Gs[64 + lane] = g1;
        Bs[64 + lane] =
            (64 + lane < n_valid) ? beta[base + static_cast<size_t>(64 + lane) * g.H_v] : 0.f;
      }
    }
    __syncthreads();

    // A[t][s] = beta_t exp(G_t - G_s) KK[t][s] for s < t.
    auto Aval = [&](int t, int s) -> float {
      return Bs[t] * __expf(Gs[t] - Gs[s]) * KK[tri_index(t >> 4, s >> 4)][(t & 15) * 16 + (s & 15)];
    };

    // 2a. Diagonal 16 x 16 blocks by forward substitution, one column per thread.
    if (threadIdx.x < NT * 16) {
      const int blk = threadIdx.x >> 4, col = threadIdx.x & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = (r == col) ? 1.f : 0.f;
        if (r > col) {
          float acc = 0.f;
#pragma unroll
          for (int k = 0; k < 16; ++k)
            if (k >= col && k < r) acc = __builtin_fmaf(Aval(16 * blk + r, 16 * blk + k), x[k], acc);
          v = -acc;
        }
        x[r] = v;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) TI[tri_index(blk, blk)][r * 16 + col] = x[r];
    }
    // 2b. Off-diagonal blocks, one block diagonal at a time:
    //     Tm_ij = -Tm_ii sum_{k=j}^{i-1} A_ik Tm_kj.
    for (int d = 1; d < NT; ++d) {
      __syncthreads();
      const int r = threadIdx.x >> 4, cc = threadIdx.x & 15;
      for (int i = d; i < NT; ++i) {
        const int j = i - d;
        float acc = 0.f;
        for (int k = j; k < i; ++k)
          for (int m = 0; m < 16; ++m)
            acc = __builtin_fmaf(Aval(16 * i + r, 16 * k + m), TI[tri_index(k, j)][m * 16 + cc], acc);
        XS[i - d][r * 16 + cc] = acc;
      }
      __syncthreads();
      for (int i = d; i < NT; ++i) {
        const int j = i - d;
        float acc = 0.f;
        for (int m = 0; m < 16; ++m)
          acc = __builtin_fmaf(TI[tri_index(i, i)][r * 16 + m], XS[i - d][m * 16 + cc], acc);
        TI[tri_index(i, j)][r * 16 + cc] = -acc;
      }
    }
    __syncthreads();

    // 3. Store Tm (bf16) and P (hi/lo) as A operands: row t, column s at its
    //    permuted K slot; zero above the diagonal and in the padding columns.
    const size_t mat = ((static_cast<size_t>(b) * g.H_v + h) * L.NC + chunk) * C * Cp;
    uint16_t *Tm = reinterpret_cast<uint16_t *>(ws + L.Tm) + mat;
    uint16_t *Ph = reinterpret_cast<uint16_t *>(ws + L.P_hi) + mat;
    uint16_t *Pl = reinterpret_cast<uint16_t *>(ws + L.P_lo) + mat;
    for (int e = threadIdx.x; e < C * Cp; e += 256) {
      const int t = e / Cp, s = e % Cp;
      float tv = 0.f, pv = 0.f;
      if (s < C && s <= t) {
        const int tr = tri_index(t >> 4, s >> 4), off = (t & 15) * 16 + (s & 15);
        tv = TI[tr][off];
        pv = __expf(Gs[t] - Gs[s]) * QK[tr][off];
      }
      const size_t o = static_cast<size_t>(t) * Cp + (s & ~31) + kslot(s & 31);
      Tm[o] = f32_to_bf16_bits(tv);
      uint16_t hi, lo;
      split_bf16(pv, hi, lo);
      Ph[o] = hi;
      Pl[o] = lo;
    }
  }
}

// ---------------------------------------------------------------- state kernel

template <int D>
struct StateShape {
  static constexpr int NWV = D >= 128 ? 4 : 1;   // waves; each owns a slice of d_k
  static constexpr int NDT = D >= 32 ? 2 : 1;    // 16-wide d_k tiles per wave
  static constexpr int Dp = D < 32 ? 32 : D;
};

// Bijection on [0, n) that gives each of the 8 XCDs a contiguous logical
// range (hardware hands consecutive block ids to consecutive XCDs), so the
// blocks that share a key head also share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  if (n % 8) return bid;
  const int per = n / 8;
  return (bid % 8) * per + bid / 8;
}

template <int D, int C, int DTZ, int DTY>
__global__ __launch_bounds__(StateShape<D>::NWV * 64) void state_kernel(
    Geom g, PrefillWs L, const void *__restrict__ z, const float *__restrict__ gl,
    const float *__restrict__ beta, float *__restrict__ S, void *__restrict__ y,
    const char *__restrict__ ws) {
  using SS = StateShape<D>;
  constexpr int NWV = SS::NWV, NDT = SS::NDT, Dp = SS::Dp;
  constexpr int NT = C / 16, Cp = C < 32 ? 32 : C, KSC = Cp / 32;
  __shared__ float part[NWV][2][NT][4][64];  // K S^T / Q S^T partial sums
  __shared__ float Ush[NT][4][64];           // U tiles in D-register order

  const int RB = D / 16;
  const int nblk = g.B * g.H_v * RB;
  const int lid = xcd_remap(blockIdx.x, nblk);
  const int rb = lid % RB;
  const int h = (lid / RB) % g.H_v;
  const int b = lid / (RB * g.H_v);
  const int kh = h / g.G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, gq = lane >> 4;

  // S^T tiles of this wave: rows d_k = 32*wave + 16*dt + 4*gq + r, column = state row 16*rb + c.
  float *Sh = S + ((static_cast<size_t>(b) * g.H_v + h) * D + 16 * rb + c) * D;
  f32x4 st[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const float4 v = *reinterpret_cast<const float4 *>(Sh + 32 * wave + 16 * dt + 4 * gq);
    st[dt] = f32x4{v.x, v.y, v.z, v.w};
  }

  const uint16_t *khi = reinterpret_cast<const uint16_t *>(ws + L.k_hi);
  const uint16_t *klo = reinterpret_cast<const uint16_t *>(ws + L.k_lo);
  const uint16_t *qhi = reinterpret_cast<const uint16_t *>(ws + L.q_hi);
  const uint16_t *qlo = reinterpret_cast<const uint16_t *>(ws + L.q_lo);
  const uint16_t *kThi = reinterpret_cast<const uint16_t *>(ws + L.kT_hi);
  const uint16_t *kTlo = reinterpret_cast<const uint16_t *>(ws + L.kT_lo);
  const float *vT = reinterpret_cast<const float *>(ws + L.vT);
  const size_t kbase = (static_cast<size_t>(b) * g.H_k + kh) * L.T_pad;
  const size_t kTbase = (static_cast<size_t>(b) * g.H_k + kh) * (L.T_pad / 32);
  const size_t vbase = (static_cast<size_t>(b) * g.H_v + h) * (L.T_pad / 16);

  for (int chunk = 0; chunk < L.NC; ++chunk) {
    const int64_t tau0 = static_cast<int64_t>(chunk) * C;
    const int n_valid = static_cast<int>((L.T - tau0) < C ? (L.T - tau0) : C);
    const size_t gbase = (static_cast<size_t>(b) * L.T + tau0) * g.H_v + h;

    // Gates for this chunk (every wave computes the same values).
    float g0, g1;
    chunk_prefix<C>(gl, gbase, g.H_v, n_valid, g0, g1);
    const float Glast = prefix_at<C>(g0, g1, C - 1);

    // 1. Partial K S^T and Q S^T over this wave's d_k slice.
    {
      u16x8 bh, bl;
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      pack_split(st[0], NDT > 1 ? st[NDT - 1] : zero, bh, bl);
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        const size_t ao = (kbase + tau0 + 16 * m + c) * Dp + 32 * wave + 8 * gq;
        f32x4 ak = mfma_split3(load8(khi + ao), load8(klo + ao), bh, bl, zero);
        f32x4 aq = mfma_split3(load8(qhi + ao), load8(qlo + ao), bh, bl, zero);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          part[wave][0][m][r][lane] = ak[r];
          part[wave][1][m][r][lane] = aq[r];
        }
      }
    }
    __syncthreads();

    // 2. R tiles (needed up to this wave's last output tile), then U = Tm R.
    int max_m = -1;
    for (int m = wave; m < NT; m += NWV) max_m = m;
    const size_t mat = ((static_cast<size_t>(b) * g.H_v + h) * L.NC + chunk) * C * Cp;
    const uint16_t *Tm = reinterpret_cast<const uint16_t *>(ws + L.Tm) + mat;
    const uint16_t *Ph = reinterpret_cast<const uint16_t *>(ws + L.P_hi) + mat;
    const uint16_t *Pl = reinterpret_cast<const uint16_t *>(ws + L.P_lo) + mat;
    f32x4 Rt[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      Rt[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (m <= max_m) {
        const float4 vv = *reinterpret_cast<const float4 *>(
            vT + ((vbase + (tau0 + 16 * m) / 16) * D + 16 * rb + c) * 16 + 4 * gq);
        const float va[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * m + 4 * gq + r;
          float ks = 0.f;
#pragma unroll
          for (int w = 0; w < NWV; ++w) ks += part[w][0][m][r][lane];
          const float Gt = prefix_at<C>(g0, g1, t);
          const float bt = (t < n_valid) ? beta[gbase + static_cast<size_t>(t) * g.H_v] : 0.f;
          Rt[m][r] = bt * (va[r] - __expf(Gt) * ks);
        }
      }
    }
    for (int m = wave; m < NT; m += NWV) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks <= m / 2; ++ks) {
        u16x8 bh, bl;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        pack_split(Rt[2 * ks], (2 * ks + 1 < NT) ? Rt[2 * ks + 1] : zero, bh, bl);
        acc = mfma_split2(load8(Tm + static_cast<size_t>(16 * m + c) * Cp + 32 * ks + 8 * gq), bh, bl,
                          acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) Ush[m][r][lane] = acc[r];
    }
    __syncthreads();

    // 3. O = gamma * QS + P U, gated store.
    for (int m = wave; m < NT; m += NWV) {
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * m + 4 * gq + r;
        float qs = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) qs += part[w][1][m][r][lane];
        acc[r] = __expf(prefix_at<C>(g0, g1, t)) * qs;
      }
      for (int ks = 0; ks <= m / 2; ++ks) {
        f32x4 u0, u1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) u0[r] = Ush[2 * ks][r][lane];
        if (2 * ks + 1 < NT) {
#pragma unroll
          for (int r = 0; r < 4; ++r) u1[r] = Ush[2 * ks + 1][r][lane];
        }
        u16x8 bh, bl;
        pack_split(u0, u1, bh, bl);
        const size_t ao = static_cast<size_t>(16 * m + c) * Cp + 32 * ks + 8 * gq;
        acc = mfma_split3(load8(Ph + ao), load8(Pl + ao), bh, bl, acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * m + 4 * gq + r;
        if (t < n_valid) {
          const size_t yi = ((static_cast<size_t>(b) * L.T + tau0 + t) * g.H_v + h) * D + 16 * rb + c;
          store_elem<DTY>(y, yi, acc[r] * sigmoidf_(load_elem<DTZ>(z, yi)));
        }
      }
    }

    // 4. S^T <- gamma_last S^T + K^T (D_last * U) for this wave's d_k slice.
    {
      const float gl_last = __expf(Glast);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[dt][r] *= gl_last;
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        f32x4 u0 = {0.f, 0.f, 0.f, 0.f}, u1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int m = 2 * ks + half;
          if (m < NT) {
            f32x4 &u = half ? u1 : u0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 16 * m + 4 * gq + r;
              u[r] = __expf(Glast - prefix_at<C>(g0, g1, t)) * Ush[m][r][lane];
            }
          }
        }
        // A 16-token chunk fills one half of a 32-token key block.
        if (C == 16 && (tau0 & 16)) {
          u1 = u0;
          u0 = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        u16x8 bh, bl;
        pack_split(u0, u1, bh, bl);
        const size_t blk = kTbase + (tau0 + 32 * ks) / 32;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const size_t ao = (blk * D + 32 * wave + 16 * dt + c) * 32 + 8 * gq;
          st[dt] = mfma_split3(load8(kThi + ao), load8(kTlo + ao), bh, bl, st[dt]);
        }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    *reinterpret_cast<float4 *>(Sh + 32 * wave + 16 * dt + 4 * gq) =
        make_float4(st[dt][0], st[dt][1], st[dt][2], st[dt][3]);
}

// ---------------------------------------------------------------- launchers

template <int D, int C>
static void launch_prep_t(const Geom &g, const PrefillWs &L, const float *gl, const float *beta,
                          char *ws, hipStream_t s) {
  dim3 grid(L.NC, g.H_k, g.B);
  hipLaunchKernelGGL((prep_kernel<D, C>), grid, dim3(256), 0, s, g, L, gl, beta, ws);
}

hipError_t launch_prefill_prep(const Geom &g, const PrefillWs &L, const float *gl,
                               const float *beta, char *ws, hipStream_t s) {
#define GDN_PREP(Dv)                                              \
  switch (L.C) {                                                  \
    case 16: launch_prep_t<Dv, 16>(g, L, gl, beta, ws, s); break; \
    case 32: launch_prep_t<Dv, 32>(g, L, gl, beta, ws, s); break; \
    case 64: launch_prep_t<Dv, 64>(g, L, gl, beta, ws, s); break; \
    default: launch_prep_t<Dv, 128>(g, L, gl, beta, ws, s); break; \
  }
  if (g.D == 128) {
    GDN_PREP(128)
  } else {
    GDN_PREP(16)
  }
#undef GDN_PREP
  return hipGetLastError();
}

template <int D, int C>
static void launch_state_t(const Geom &g, const PrefillWs &L, const void *z, const float *gl,
                           const float *beta, float *S, void *y, const char *ws, hipStream_t s) {
  dim3 grid(g.B * g.H_v * (D / 16));
  dim3 block(StateShape<D>::NWV * 64);
  const int key = (g.in_dt << 1) | g.out_dt;
  switch (key) {
    case 0: hipLaunchKernelGGL((state_kernel<D, C, 0, 0>), grid, block, 0, s, g, L, z, gl, beta, S, y, ws); break;
    case 1: hipLaunchKernelGGL((state_kernel<D, C, 0, 1>), grid, block, 0, s, g, L, z, gl, beta, S, y, ws); break;
    case 2: hipLaunchKernelGGL((state_kernel<D, C, 1, 0>), grid, block, 0, s, g, L, z, gl, beta, S, y, ws); break;
    default: hipLaunchKernelGGL((state_kernel<D, C, 1, 1>), grid, block, 0, s, g, L, z, gl, beta, S, y, ws); break;
  }
}

hipError_t launch_prefill_state(const Geom &g, const PrefillWs &L, const void *z,
                                const float *gl, const float *beta, float *S, void *y,
                                const char *ws, hipStream_t s) {
#define GDN_STATE(Dv)                                                         \
  switch (L.C) {                                                              \
    case 16: launch_state_t<Dv, 16>(g, L, z, gl, beta, S, y, ws, s); break;   \
    case 32: launch_state_t<Dv, 32>(g, L, z, gl, beta, S, y, ws, s); break;   \
    case 64: launch_state_t<Dv, 64>(g, L, z, gl, beta, S, y, ws, s); break;   \
    default: launch_state_t<Dv, 128>(g, L, z, gl, beta, S, y, ws, s); break;  \
  }
  if (g.D == 128) {
    GDN_STATE(128)
  } else {
    GDN_STATE(16)
  }
#undef GDN_STATE
  return hipGetLastError();
}

}  // namespace gdn
