// prep.hip -- chunk-local pass of the chunked gated delta rule (WY / UT
// form) for gfx950.  For each chunk of C tokens and key head (the blocks run
// in parallel over chunks):
//   K K^T and Q K^T, lower 16 x 16 tiles only, on the bf16 MFMA with split
//   (hi + lo) operands and fp32 accumulation, once per key head;
// then for each value head that reads the key head, with G_t the prefix sum
// of the log decay g over the chunk and D_ts = exp(G_t - G_s):
//   the gate table (exp(G_t), exp(G_last - G_t), beta_t) of the state pass,
//   A  = strict_lower(diag(beta) (D * K K^T)),
//   Tm = (I + A)^{-1}, by 16 x 16 blocks in fp32 (forward substitution on
//        the diagonal blocks, the off-diagonal blocks on the fp32 MFMA),
//   P  = tril(D) * (Q K^T),
// stored as MFMA A operands (Tm plain bf16, P split) for the state pass.
// The blocks of the first chunk also roll the conv history of the q and k
// channels (or of all channels, when the state pass does not roll v).
// The chunked form is the sequential recurrence of the gated delta rule
// (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025) regrouped per
// chunk, exact up to rounding.
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

// Conv history after the whole sequence: the last three rows of
// concat(history, x), copied bit for bit, for the channels [c0, c1).  Each
// thread reads its channel's three values before writing them.
template <typename E>
__device__ __forceinline__ void roll_history(int C_ch, int64_t T, int b, int c0, int c1,
                                             const E *__restrict__ x, E *__restrict__ hist) {
  for (int ch = c0 + static_cast<int>(threadIdx.x); ch < c1; ch += blockDim.x) {
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
}

template <int D, int C>
__global__ __launch_bounds__(256, (C <= 64 ? 4 : 1)) void prep_kernel(Geom g, PrefillWs L,
                                                   const float *__restrict__ gl,
                                                   const float *__restrict__ beta,
                                                   char *__restrict__ ws,
                                                   const void *__restrict__ x,
                                                   void *__restrict__ hist) {
  using Sh = PrepShape<D, C>;
  constexpr int NT = Sh::NT, NTRI = Sh::NTRI, Dp = Sh::Dp, Cp = Sh::Cp;
  __shared__ float KK[NTRI][256];  // Gram tiles, row-major 16 x 16
  __shared__ float QK[NTRI][256];
  __shared__ float TI[NTRI][256];  // A, then (I + A)^{-1} in place
  __shared__ float Gs[C], Bs[C];

  const int chunk = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, gq = lane >> 4;
  const int64_t tau0 = static_cast<int64_t>(chunk) * C;
  const int n_valid = static_cast<int>((L.T - tau0) < C ? (L.T - tau0) : C);

  // 0. The conv history roll rides on the first chunk's blocks (one slice of
  //    the channels per key head): the conv pass, its only reader, has
  //    finished before this kernel starts.
  if (chunk == 0) {
    // With the split-role state pass, that pass rolls the v channels itself.
    const int nroll = prefill_split_roles(g, L) ? 2 * g.H_k * g.D : g.C_ch;
    const int per = (nroll + g.H_k - 1) / g.H_k;
    const int c0 = kh * per, c1 = c0 + per < nroll ? c0 + per : nroll;
    if (g.in_dt == 0)
      roll_history(g.C_ch, L.T, b, c0, c1, static_cast<const uint32_t *>(x), static_cast<uint32_t *>(hist));
    else
      roll_history(g.C_ch, L.T, b, c0, c1, static_cast<const uint16_t *>(x), static_cast<uint16_t *>(hist));
  }

  // 1. K K^T and Q K^T, lower tiles only, split operands.  The tiles go to
  //    the waves in contiguous runs of the column-major order (column nt,
  //    then row mt), so a wave loads each K column tile it needs (the B
  //    operand of both products) once, and each K and Q row tile once.
  {
    constexpr int KS = Sh::KS_D;
    const size_t head0 = (static_cast<size_t>(b) * g.H_k + kh) * (Dp / 32);  // first 32-slice
    const uint16_t *khi = reinterpret_cast<const uint16_t *>(ws + L.k_hi);
    const uint16_t *klo = reinterpret_cast<const uint16_t *>(ws + L.k_lo);
    const uint16_t *qhi = reinterpret_cast<const uint16_t *>(ws + L.q_hi);
    const uint16_t *qlo = reinterpret_cast<const uint16_t *>(ws + L.q_lo);
    // With the split-role state pass (d = 128, C = 64) the low halves are
    // e4m3 bytes (same element index) with a power-of-two scale.
    constexpr bool kLo8 = D == 128 && C == 64;
    auto load_tile = [&](const uint16_t *hi, const uint16_t *lo, float lo_scale, int t,
                         u16x8 (&h)[KS], u16x8 (&l)[KS]) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const size_t o = (((head0 + ks) * L.T_pad + tau0) + 16 * t + c) * 32 + 8 * gq;
        h[ks] = load8(hi + o);
        if constexpr (kLo8)
          l[ks] = lo8_to_bf16x8(*reinterpret_cast<const uint2 *>(reinterpret_cast<const uint8_t *>(lo) + o), lo_scale);
        else
          l[ks] = load8(lo + o);
      }
    };
    // Owner of the tile at column-major position cm.
    auto owner = [](int cm) { return cm * 4 / NTRI; };
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int cm0 = nt * NT - nt * (nt - 1) / 2;  // column-major position of (nt, nt)
      if (owner(cm0) > wave || owner(cm0 + NT - 1 - nt) < wave) continue;
      u16x8 bh[KS], bl[KS];
      load_tile(khi, klo, L.k_lo_scale, nt, bh, bl);
#pragma unroll
      for (int mt = nt; mt < NT; ++mt) {
        if (owner(cm0 + mt - nt) != wave) continue;
        u16x8 akh[KS], akl[KS], aqh[KS], aql[KS];
        if (mt == nt) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            akh[ks] = bh[ks];
            akl[ks] = bl[ks];
          }
        } else {
          load_tile(khi, klo, L.k_lo_scale, mt, akh, akl);
        }
        load_tile(qhi, qlo, L.q_lo_scale, mt, aqh, aql);
        f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          kk = mfma_split3(akh[ks], akl[ks], bh[ks], bl[ks], kk);
          qk = mfma_split3(aqh[ks], aql[ks], bh[ks], bl[ks], qk);
        }
        const int tri = tri_index(mt, nt);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          KK[tri][(4 * gq + r) * 16 + c] = kk[r];
          QK[tri][(4 * gq + r) * 16 + c] = qk[r];
        }
      }
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

    // Gate factors of this chunk for the state pass.
    {
      if constexpr (D == 128 && C == 64) {
        // Interleaved per token for the split-role state pass: one 16-byte
        // load gives a token's gamma, decay to the chunk end, beta and the
        // chunk's gamma_last.
        float4 *gt = reinterpret_cast<float4 *>(ws + L.gates) +
                     ((static_cast<size_t>(b) * g.H_v + h) * L.NC + chunk) * C;
        const float glast = __expf(Gs[C - 1]);
        for (int t = threadIdx.x; t < C; t += blockDim.x)
          gt[t] = make_float4(__expf(Gs[t]), __expf(Gs[C - 1] - Gs[t]), Bs[t], glast);
      } else {
        float *gt = reinterpret_cast<float *>(ws + L.gates) +
                    ((static_cast<size_t>(b) * g.H_v + h) * L.NC + chunk) * 3 * C;
        for (int t = threadIdx.x; t < C; t += blockDim.x) {
          gt[t] = __expf(Gs[t]);
          gt[C + t] = __expf(Gs[C - 1] - Gs[t]);
          gt[2 * C + t] = Bs[t];
        }
      }
    }

    // 2. Tm = (I + A)^{-1}, A[t][s] = beta_t exp(G_t - G_s) KK[t][s] (s < t),
    //    blocked by 16 x 16 tiles and computed in place in TI:
    //    (a) A, one exponential per entry;
    //    (b) diagonal blocks X_ii = (I + A_ii)^{-1} by forward substitution;
    //    (c) Y_ik = X_ii A_ik for k < i;
    //    (d) block row by block row, X_ij = -sum_{k=j}^{i-1} Y_ik X_kj
    //        (from sum_{k=j}^{i} L_ik X_kj = 0 for the block lower triangular
    //        L = I + A).
    // (The opaque copies keep per-lane constants inside this loop: hoisted
    // out of it they would live across all value heads and spill.)
    int r16 = threadIdx.x >> 4, c16 = threadIdx.x & 15;
    asm volatile("" : "+v"(r16), "+v"(c16));
#pragma unroll
    for (int tri = 0; tri < NTRI; ++tri) {
      int mt = 0;
      while (tri_index(mt + 1, 0) <= tri) ++mt;
      const int nt = tri - tri_index(mt, 0);
      const int t = 16 * mt + r16, sc = 16 * nt + c16;
      TI[tri][threadIdx.x] = sc < t ? Bs[t] * __expf(Gs[t] - Gs[sc]) * KK[tri][threadIdx.x] : 0.f;
    }
    __syncthreads();
    if (threadIdx.x < NT * 16) {
      // Column col of diagonal block blk; the block's lanes share one wave and
      // run in lockstep, so every read below precedes the writes that follow.
      const int blk = r16, col = c16;
      const float *Ad = TI[tri_index(blk, blk)];
      // x[r] = [r == col] - sum_{k<r} A[r][k] x[k]; entries above col are
      // zero, so the sum needs no per-lane bounds.
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < r; ++k) acc = __builtin_fmaf(Ad[r * 16 + k], x[k], acc);
        x[r] = (r == col ? 1.f : 0.f) - acc;
      }
      float *Xd = TI[tri_index(blk, blk)];
#pragma unroll
      for (int r = 0; r < 16; ++r) Xd[r * 16 + col] = x[r];
    }
    __syncthreads();
    if constexpr (NT > 1) {
      // 16 x 16 x 16 fp32 products on the fp32 MFMA, one wave per output
      // block.  v_mfma_f32_16x16x4_f32: lane (c, g) supplies A[c][k] and
      // B[k][c] of one 4-wide K step and holds D[4g + r][c].  The K index of
      // step s for lane group g is 4g + s, so a lane's A values of all four
      // steps are one contiguous row piece.
      const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
      const int c = lane & 15, g4 = lane >> 4;
      auto prod = [&](const float *A, const float *Bm, f32x4 acc) {
        const float4 av = *reinterpret_cast<const float4 *>(A + c * 16 + 4 * g4);
        const float a4[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int st = 0; st < 4; ++st)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[st], Bm[(4 * g4 + st) * 16 + c], acc, 0, 0, 0);
        return acc;
      };
      // (c) Y_ik = X_ii A_ik, in place: only the wave that forms Y_ik reads A_ik.
#pragma unroll
      for (int i = 1, q = 0; i < NT; ++i)
#pragma unroll
        for (int k = 0; k < i; ++k, ++q)
          if (q % 4 == wave) {
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const f32x4 y = prod(TI[tri_index(i, i)], TI[tri_index(i, k)], zero);
            float *dst = TI[tri_index(i, k)];
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(4 * g4 + r) * 16 + c] = y[r];
          }
      // (d) block row i: X_ij = -sum_{k=j}^{i-1} Y_ik X_kj for j < i, block j
      //     on wave j % 4; all of the row's reads precede its writes.
#pragma unroll
      for (int i = 1; i < NT; ++i) {
        __syncthreads();
        f32x4 xr[(NT + 2) / 4];
#pragma unroll
        for (int j = 0; j < i; ++j)
          if (j % 4 == wave) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = j; k < i; ++k) acc = prod(TI[tri_index(i, k)], TI[tri_index(k, j)], acc);
            xr[j / 4] = acc;
          }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < i; ++j)
          if (j % 4 == wave) {
            float *dst = TI[tri_index(i, j)];
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(4 * g4 + r) * 16 + c] = -xr[j / 4][r];
          }
      }
    }
    __syncthreads();

    // 3. Store Tm (bf16) and P (hi/lo) as A operands: row t, column s at its
    //    permuted K slot; zero above the diagonal and in the padding columns.
    //    One item is the 16-byte piece of slots 8q..8q+7 of a 32-column step,
    //    which holds columns 4q..4q+3 and 16+4q..16+4q+3 of that step.
    const size_t mat = ((static_cast<size_t>(b) * g.H_v + h) * L.NC + chunk) * C * Cp;
    uint16_t *Tm = reinterpret_cast<uint16_t *>(ws + L.Tm) + mat;
    uint16_t *Ph = reinterpret_cast<uint16_t *>(ws + L.P_hi) + mat;
    uint16_t *Pl = reinterpret_cast<uint16_t *>(ws + L.P_lo) + mat;
    // For the split-role state pass (d = 128, C = 64) the low half of P is
    // e4m3 bytes (|P| <= |q_scale|, so q's scale), at the same element index.
    constexpr bool kLo8 = D == 128 && C == 64;
    uint8_t *Pl8 = reinterpret_cast<uint8_t *>(ws + L.P_lo) + mat;
    // The split-role pass reads K step 1 only for rows 32..63 (a row's
    // product stops at its own 32-column step), so there the pieces of K
    // step 1 for rows 0..31, all zero, are not stored: 384 items, K step 0 of
    // every row first.
    constexpr int ITEMS = kLo8 ? 384 : C * (Cp / 32) * 4;
    for (int it = threadIdx.x; it < ITEMS; it += 256) {
      int t, kk, q;
      if constexpr (kLo8) {
        kk = it >> 8;
        t = 32 * kk + ((it & 255) >> 2);
        q = it & 3;
      } else {
        t = it / (Cp / 8);
        const int rem = it % (Cp / 8);
        kk = rem >> 2;
        q = rem & 3;
      }
      u16x8 tv8;
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int sc = 32 * kk + (i < 4 ? 4 * q + i : 16 + 4 * q + (i - 4));
        float tv = 0.f;
        pv[i] = 0.f;
        if (sc < C && sc <= t) {
          const int tr = tri_index(t >> 4, sc >> 4), off = (t & 15) * 16 + (sc & 15);
          tv = TI[tr][off];
          pv[i] = __expf(Gs[t] - Gs[sc]) * QK[tr][off];
        }
        tv8[i] = f32_to_bf16_bits(tv);
      }
      const size_t o = static_cast<size_t>(t) * Cp + 32 * kk + 8 * q;
      *reinterpret_cast<u16x8 *>(Tm + o) = tv8;
      if constexpr (kLo8) {
        uint32_t h[4];
        uint16_t l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split2_lo8(pv[2 * i], pv[2 * i + 1], L.q_lo_scale, h[i], l[i]);
        const u32x4 hv = {h[0], h[1], h[2], h[3]};
        *reinterpret_cast<u16x8 *>(Ph + o) = __builtin_bit_cast(u16x8, hv);
        *reinterpret_cast<uint2 *>(Pl8 + o) =
            make_uint2(l[0] | (static_cast<uint32_t>(l[1]) << 16), l[2] | (static_cast<uint32_t>(l[3]) << 16));
      } else {
        u16x8 ph8, pl8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint16_t hi, lo;
          split_bf16(pv[i], hi, lo);
          ph8[i] = hi;
          pl8[i] = lo;
        }
        *reinterpret_cast<u16x8 *>(Ph + o) = ph8;
        *reinterpret_cast<u16x8 *>(Pl + o) = pl8;
      }
    }
  }
}

// ---------------------------------------------------------------- launcher

template <int D, int C>
static void launch_prep_t(const Geom &g, const PrefillWs &L, const float *gl, const float *beta,
                          char *ws, const void *x, void *hist, hipStream_t s) {
  dim3 grid(L.NC, g.H_k, g.B);
  hipLaunchKernelGGL((prep_kernel<D, C>), grid, dim3(256), 0, s, g, L, gl, beta, ws, x, hist);
}

hipError_t launch_prefill_prep(const Geom &g, const PrefillWs &L, const float *gl,
                               const float *beta, char *ws, const void *x, void *hist,
                               hipStream_t s) {
#define GDN_PREP(Dv)                                                       \
  switch (L.C) {                                                           \
    case 16: launch_prep_t<Dv, 16>(g, L, gl, beta, ws, x, hist, s); break;  \
    case 32: launch_prep_t<Dv, 32>(g, L, gl, beta, ws, x, hist, s); break;  \
    case 64: launch_prep_t<Dv, 64>(g, L, gl, beta, ws, x, hist, s); break;  \
    default: launch_prep_t<Dv, 128>(g, L, gl, beta, ws, x, hist, s); break; \
  }
  if (g.D == 128) {
    GDN_PREP(128)
  } else {
    GDN_PREP(16)
  }
#undef GDN_PREP
  return hipGetLastError();
}

}  // namespace gdn
