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
// channels (or of all channels, when the state pass does not roll v).  On
// the largest grids (prep_fuses_conv) each block first computes its chunk of
// q-hat and k-hat from x itself, in place of the conv pass.
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

// Value heads processed in parallel by the per-wave form of the kernel (one
// head per wave, waves 0 .. kHeadSlots - 1; each head's inverse in a slot of
// its own in LDS).
constexpr int kHeadSlots = 3;

// One value head h of one chunk (C <= 64), computed by one wave: the gate
// table, A, Tm = (I + A)^{-1} in place in TI (the head's NTRI tiles), and the
// stores of Tm and P.  The operations and their order are those of the
// four-wave form in prep_kernel, entry by entry, so the results are the same
// to the bit; G_t and beta_t stay in registers (lane t) and are read with
// shuffles instead of from LDS.  All of it runs in one wave, whose LDS
// accesses complete in program order, so the steps need no block barrier
// (the compiler barriers below keep it from moving LDS accesses across
// steps).
template <int D, int C>
__device__ __forceinline__ void prep_head_wave(const Geom &g, const PrefillWs &L,
                                               const float *__restrict__ gl,
                                               const float *__restrict__ beta, char *__restrict__ ws,
                                               const float (*KK)[256], const float (*QK)[256],
                                               float (*TI)[256], int b, int h, int chunk,
                                               int64_t tau0, int n_valid) {
  using Sh = PrepShape<D, C>;
  constexpr int NT = Sh::NT, NTRI = Sh::NTRI, Cp = Sh::Cp;
  static_assert(C <= 64, "one token per lane");
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g4 = lane >> 4;

  // Lane t: G_t, the prefix sum of the log decay, and beta_t (0 past the end).
  float g0, g1;
  const size_t base = (static_cast<size_t>(b) * L.T + tau0) * g.H_v + h;
  chunk_prefix<C>(gl, base, g.H_v, n_valid, g0, g1);
  const float b0 = (lane < C && lane < n_valid) ? beta[base + static_cast<size_t>(lane) * g.H_v] : 0.f;
  const float g_last = __shfl(g0, C - 1, kWave);

  // Gate factors of this chunk for the state pass.
  if constexpr (D == 128 && C == 64) {
    float4 *gt = reinterpret_cast<float4 *>(ws + L.gates) +
                 ((static_cast<size_t>(b) * g.H_v + h) * L.NC + chunk) * C;
    const f32x4 gv = {__expf(g0), __expf(g_last - g0), b0, __expf(g_last)};
    __builtin_nontemporal_store(gv, reinterpret_cast<f32x4 *>(gt + lane));
  } else {
    float *gt = reinterpret_cast<float *>(ws + L.gates) +
                ((static_cast<size_t>(b) * g.H_v + h) * L.NC + chunk) * 3 * C;
    if (lane < C) {
      gt[lane] = __expf(g0);
      gt[C + lane] = __expf(g_last - g0);
      gt[2 * C + lane] = b0;
    }
  }

  // (a) A[t][s] = beta_t exp(G_t - G_s) KK[t][s] for s < t, tile by tile.
#pragma unroll
  for (int tri = 0; tri < NTRI; ++tri) {
    int mt = 0;
    while (tri_index(mt + 1, 0) <= tri) ++mt;
    const int nt = tri - tri_index(mt, 0);
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int e = lane + 64 * e4;
      const int t = 16 * mt + (e >> 4), sc = 16 * nt + (e & 15);
      const float bt = __shfl(b0, t, kWave), gtv = __shfl(g0, t, kWave), gsv = __shfl(g0, sc, kWave);
      TI[tri][e] = sc < t ? bt * __expf(gtv - gsv) * KK[tri][e] : 0.f;
    }
  }
  asm volatile("" ::: "memory");
  // (b) diagonal blocks X_ii = (I + A_ii)^{-1} by forward substitution, one
  //     lane per column (block lane / 16, column lane % 16).
  if (lane < NT * 16) {
    const int blk = lane >> 4, col = lane & 15;
    const float *Ad = TI[tri_index(blk, blk)];
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
  asm volatile("" ::: "memory");
  if constexpr (NT > 1) {
    auto prod = [&](const float *A, const float *Bm, f32x4 acc) {
      const float4 av = *reinterpret_cast<const float4 *>(A + c * 16 + 4 * g4);
      const float a4[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[st], Bm[(4 * g4 + st) * 16 + c], acc, 0, 0, 0);
      return acc;
    };
    // (c) Y_ik = X_ii A_ik in place of A_ik.
#pragma unroll
    for (int i = 1; i < NT; ++i)
#pragma unroll
      for (int k = 0; k < i; ++k) {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 y = prod(TI[tri_index(i, i)], TI[tri_index(i, k)], zero);
        float *dst = TI[tri_index(i, k)];
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(4 * g4 + r) * 16 + c] = y[r];
        asm volatile("" ::: "memory");
      }
    // (d) block row i: X_ij = -sum_{k=j}^{i-1} Y_ik X_kj for j < i; the whole
    //     row is read before any of it is written.
#pragma unroll
    for (int i = 1; i < NT; ++i) {
      f32x4 xr[NT - 1];
#pragma unroll
      for (int j = 0; j < i; ++j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = j; k < i; ++k) acc = prod(TI[tri_index(i, k)], TI[tri_index(k, j)], acc);
        xr[j] = acc;
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < i; ++j) {
        float *dst = TI[tri_index(i, j)];
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(4 * g4 + r) * 16 + c] = -xr[j][r];
      }
      asm volatile("" ::: "memory");
    }
  }

  // (e) Tm (bf16) and P (hi/lo) as A operands, as in the four-wave form.
  const size_t mat = ((static_cast<size_t>(b) * g.H_v + h) * L.NC + chunk) * C * Cp;
  uint16_t *Tm = reinterpret_cast<uint16_t *>(ws + L.Tm) + mat;
  uint16_t *Ph = reinterpret_cast<uint16_t *>(ws + L.P_hi) + mat;
  uint16_t *Pl = reinterpret_cast<uint16_t *>(ws + L.P_lo) + mat;
  constexpr bool kLo8 = D == 128 && C == 64;
  uint8_t *Pl8 = reinterpret_cast<uint8_t *>(ws + L.P_lo) + mat;
  constexpr int ITEMS = kLo8 ? 384 : C * (Cp / 32) * 4;
  static_assert(ITEMS % 64 == 0, "every lane takes the same number of items");
  for (int it = lane; it < ITEMS; it += 64) {
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
    const float gtv = __shfl(g0, t & 63, kWave);
    u16x8 tv8;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int sc = 32 * kk + (i < 4 ? 4 * q + i : 16 + 4 * q + (i - 4));
      const float gsv = __shfl(g0, sc & 63, kWave);
      float tv = 0.f;
      pv[i] = 0.f;
      if (sc < C && sc <= t) {
        const int tr = tri_index(t >> 4, sc >> 4), off = (t & 15) * 16 + (sc & 15);
        tv = TI[tr][off];
        pv[i] = __expf(gtv - gsv) * QK[tr][off];
      }
      tv8[i] = f32_to_bf16_bits(tv);
    }
    const size_t o = static_cast<size_t>(t) * Cp + 32 * kk + 8 * q;
    __builtin_nontemporal_store(tv8, reinterpret_cast<u16x8 *>(Tm + o));
    if constexpr (kLo8) {
      uint32_t hh[4];
      uint16_t ll[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split2_lo8(pv[2 * i], pv[2 * i + 1], L.q_lo_scale, hh[i], ll[i]);
      const u32x4 hv = {hh[0], hh[1], hh[2], hh[3]};
      __builtin_nontemporal_store(__builtin_bit_cast(u16x8, hv), reinterpret_cast<u16x8 *>(Ph + o));
      const u32x2 lv = {ll[0] | (static_cast<uint32_t>(ll[1]) << 16), ll[2] | (static_cast<uint32_t>(ll[3]) << 16)};
      __builtin_nontemporal_store(lv, reinterpret_cast<u32x2 *>(Pl8 + o));
    } else {
      u16x8 ph8, pl8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint16_t hi, lo;
        split_bf16(pv[i], hi, lo);
        ph8[i] = hi;
        pl8[i] = lo;
      }
      __builtin_nontemporal_store(ph8, reinterpret_cast<u16x8 *>(Ph + o));
      __builtin_nontemporal_store(pl8, reinterpret_cast<u16x8 *>(Pl + o));
    }
  }
}

// The conv, SiLU and L2 norm of one key head's q and k channels for one
// chunk, computed the way the q/k conv pass computes them (the same loads,
// products, reduction tree and rounding, so the same bits).  The results go
// to the workspace's token-major q/k rows (bf16 high halves, e4m3 low halves)
// for the state pass, and straight to the block's operands of the Gram
// products: K's rows into the LDS staging rows (krows: hi, then lo widened
// to bf16, 16-byte pieces XOR-swizzled by token), wave w's Q operands of
// token tile w into registers, so nothing is read back from memory.
// Threads 0..127 take the q head's channels, 128..255 the k head's; the
// chunk's rows of x (and the three before it) are loaded at once, then
// reduced and stored one 16-token tile at a time.  sa, sb: scratch of
// kPrepConvScratchA and kPrepConvScratchB bytes (16-byte aligned), free
// again on return.
constexpr int kPrepConvTT = 16;
constexpr size_t kPrepConvScratchA = 512 + 8 * kPrepConvTT * 32 * 2;  // sums, hi stage
constexpr size_t kPrepConvScratchB = 8 * kPrepConvTT * 32;            // lo stage
template <int DT, int C>
__device__ __forceinline__ void prep_conv_qk(const Geom &g, const PrefillWs &L,
                                             const void *__restrict__ x,
                                             const void *__restrict__ w,
                                             const void *__restrict__ hist, char *__restrict__ ws,
                                             int b, int kh, int64_t tau0, unsigned char *sa,
                                             unsigned char *sb, uint16_t (*krows)[128],
                                             u16x8 (&qh_op)[4], u16x8 (&ql_op)[4]) {
  constexpr int D = 128, TT = kPrepConvTT;
  static_assert(C == 4 * TT, "wave w keeps the Q operands of tile w");
  const int hp = threadIdx.x >> 7;  // 0: q head kh, 1: k head kh (uniform per wave)
  const int j = threadIdx.x & 127;
  const int nq = g.H_k * D;
  const int ch = hp * nq + kh * D + j;
  const float sc = hp == 0 ? g.q_scale : 1.0f;
  const float lo_scale = hp == 0 ? L.q_lo_scale : L.k_lo_scale;
  float (*red)[16] = reinterpret_cast<float (*)[16]>(sa);  // [head][wave in head][token]
  float (*bc)[16] = reinterpret_cast<float (*)[16]>(sa + 256);
  uint16_t (*sth)[TT][32] = reinterpret_cast<uint16_t (*)[TT][32]>(sa + 512);  // [head][slice]
  uint8_t (*stl)[TT][32] = reinterpret_cast<uint8_t (*)[TT][32]>(sb);
  constexpr int ES = DT == 0 ? 4 : 2;
  const size_t rowb = static_cast<size_t>(g.C_ch) * ES;
  const uint32_t lane_off = static_cast<uint32_t>(ch) * ES;
  auto ld = [&](const char *row) -> float {
    if constexpr (DT == 0)
      return *reinterpret_cast<const float *>(row + lane_off);
    else
      return bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(row + lane_off));
  };
  const float w0 = load_elem<DT>(w, static_cast<size_t>(ch) * 4 + 0);
  const float w1 = load_elem<DT>(w, static_cast<size_t>(ch) * 4 + 1);
  const float w2 = load_elem<DT>(w, static_cast<size_t>(ch) * 4 + 2);
  const float w3 = load_elem<DT>(w, static_cast<size_t>(ch) * 4 + 3);
  const char *xb = static_cast<const char *>(x) + static_cast<size_t>(b) * L.T * rowb;
  const char *hb = static_cast<const char *>(hist) + static_cast<size_t>(b) * 3 * rowb;
  // The chunk's rows and the three before it, all loads in flight at once.
  float xa[C + 3];
  if (tau0 >= 3 && tau0 + C <= L.T) {
    const char *r0 = xb + static_cast<size_t>(tau0 - 3) * rowb;
#pragma unroll
    for (int i = 0; i < C + 3; ++i) xa[i] = ld(r0 + i * rowb);
  } else {
#pragma unroll
    for (int i = 0; i < C + 3; ++i) {
      const int64_t tau = tau0 - 3 + i;  // uniform per block
      float v = 0.f;
      if (tau < 0)
        v = ld(hb + static_cast<size_t>(3 + tau) * rowb);
      else if (tau < L.T)
        v = ld(xb + static_cast<size_t>(tau) * rowb);
      xa[i] = v;
    }
  }
  // Slice 0 of the head: [b][kh][slice][T_pad][32] token-major rows.
  const size_t slice0 = (static_cast<size_t>(b) * g.H_k + kh) * (L.Dp / 32) * L.T_pad;
  const int pos = kslot(j & 31);
#pragma unroll
  for (int it = 0; it < C / TT; ++it) {
    const int64_t t0 = tau0 + it * TT;
    float val[TT], ss[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      val[t] = siluf_(conv4(w0, w1, w2, w3, xa[TT * it + t], xa[TT * it + t + 1], xa[TT * it + t + 2],
                            xa[TT * it + t + 3]));
      ss[t] = val[t] * val[t];
    }
    head_scale_128x16(ss, g.eps, sc, red + 2 * hp, bc + 2 * hp, (threadIdx.x >> 6) & 1);
#pragma unroll
    for (int t = 0; t < TT; ++t) val[t] *= ss[t];
    if (t0 + TT > L.T) {
#pragma unroll
      for (int t = 0; t < TT; ++t)
        if (t0 + t >= L.T) val[t] = 0.f;  // padding tokens of the prefill layout
    }
#pragma unroll
    for (int t = 0; t < TT; t += 2) {
      uint32_t h2;
      uint16_t l2;
      split2_lo8(val[t], val[t + 1], lo_scale, h2, l2);
      sth[4 * hp + (j >> 5)][t][pos] = static_cast<uint16_t>(h2);
      sth[4 * hp + (j >> 5)][t + 1][pos] = static_cast<uint16_t>(h2 >> 16);
      stl[4 * hp + (j >> 5)][t][pos] = static_cast<uint8_t>(l2);
      stl[4 * hp + (j >> 5)][t + 1][pos] = static_cast<uint8_t>(l2 >> 8);
    }
    __syncthreads();
    {
      // K rows 16 it .. 16 it + 15 of the Gram staging: thread (token tok,
      // piece p = 4 ks + gq) moves slots 8 gq .. 8 gq + 7 of slice ks.
      const int tok = threadIdx.x >> 4, p = threadIdx.x & 15, ks = p >> 2, gq = p & 3;
      const int off = 8 * (p ^ tok);
      *reinterpret_cast<u16x8 *>(&krows[16 * it + tok][off]) =
          *reinterpret_cast<const u16x8 *>(&sth[4 + ks][tok][8 * gq]);
      *reinterpret_cast<u16x8 *>(&krows[C + 16 * it + tok][off]) =
          lo8_to_bf16x8(*reinterpret_cast<const uint2 *>(&stl[4 + ks][tok][8 * gq]), L.k_lo_scale);
    }
    if ((threadIdx.x >> 6) == it) {
      // Wave `it`: the tile's Q operands (token c, slots 8 gq .. 8 gq + 7 of
      // each slice, the low halves widened).
      const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        qh_op[ks] = *reinterpret_cast<const u16x8 *>(&sth[ks][c][8 * gq]);
        ql_op[ks] = lo8_to_bf16x8(*reinterpret_cast<const uint2 *>(&stl[ks][c][8 * gq]), L.q_lo_scale);
      }
    }
    // Per head and tile: four 1 KB runs of hi and four 512-byte runs of lo
    // (one per 32-channel slice), written as 16-byte pieces.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int piece = threadIdx.x;  // of head u's 4 KB of hi
      const int sl = piece >> 6, tok = (piece >> 2) & 15, part = piece & 3;
      uint16_t *dst = reinterpret_cast<uint16_t *>(ws + (u == 0 ? L.q_hi : L.k_hi)) +
                      ((slice0 + sl * L.T_pad + t0 + tok) * 32 + 8 * part);
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(&sth[4 * u + sl][tok][8 * part]),
                                  reinterpret_cast<u32x4 *>(dst));
    }
    {
      const int u = threadIdx.x >> 7, piece = threadIdx.x & 127;  // of head u's 2 KB of lo
      const int sl = piece >> 5, tok = (piece >> 1) & 15, part = piece & 1;
      uint8_t *dst = reinterpret_cast<uint8_t *>(ws + (u == 0 ? L.q_lo : L.k_lo)) +
                     ((slice0 + sl * L.T_pad + t0 + tok) * 32 + 16 * part);
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(&stl[4 * u + sl][tok][16 * part]),
                                  reinterpret_cast<u32x4 *>(dst));
    }
    __syncthreads();  // the stages and sums are rewritten by the next tile
  }
}

// Gate table of one value head and chunk for the state pass (four-wave prep
// form; the per-wave form writes its own).
template <int D, int C>
__device__ __forceinline__ void store_gate_table(const Geom &g, const PrefillWs &L, char *ws, int b,
                                                 int h, int chunk, const float *Gs, const float *Bs) {
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

// Tm (bf16, from TI) and / or P (hi/lo, tril(D) * QK) of one value head and
// chunk as A operands of the state pass: row t, column s at its permuted K
// slot; zero above the diagonal and in the padding columns.  One item is the
// 16-byte piece of slots 8q..8q+7 of a 32-column step, which holds columns
// 4q..4q+3 and 16+4q..16+4q+3 of that step.  Streamed to the workspace with
// the nontemporal hint (read once, by the state pass).
template <int D, int C, bool TM, bool PP>
__device__ __forceinline__ void store_pieces(const Geom &g, const PrefillWs &L, char *ws, int b,
                                             int h, int chunk, const float *Gs,
                                             float (*TI)[256], float (*QK)[256]) {
  constexpr int Cp = C < 32 ? 32 : C;
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
        if constexpr (TM) tv = TI[tr][off];
        if constexpr (PP) pv[i] = __expf(Gs[t] - Gs[sc]) * QK[tr][off];
      }
      tv8[i] = f32_to_bf16_bits(tv);
    }
    const size_t o = static_cast<size_t>(t) * Cp + 32 * kk + 8 * q;
    if constexpr (TM) __builtin_nontemporal_store(tv8, reinterpret_cast<u16x8 *>(Tm + o));
    if constexpr (PP) {
      if constexpr (kLo8) {
        uint32_t hh[4];
        uint16_t ll[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split2_lo8(pv[2 * i], pv[2 * i + 1], L.q_lo_scale, hh[i], ll[i]);
        const u32x4 hv = {hh[0], hh[1], hh[2], hh[3]};
        __builtin_nontemporal_store(__builtin_bit_cast(u16x8, hv), reinterpret_cast<u16x8 *>(Ph + o));
        const u32x2 lv = {ll[0] | (static_cast<uint32_t>(ll[1]) << 16), ll[2] | (static_cast<uint32_t>(ll[3]) << 16)};
        __builtin_nontemporal_store(lv, reinterpret_cast<u32x2 *>(Pl8 + o));
      } else {
        u16x8 ph8, pl8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint16_t hi, lo;
          split_bf16(pv[i], hi, lo);
          ph8[i] = hi;
          pl8[i] = lo;
        }
        __builtin_nontemporal_store(ph8, reinterpret_cast<u16x8 *>(Ph + o));
        __builtin_nontemporal_store(pl8, reinterpret_cast<u16x8 *>(Pl + o));
      }
    }
  }
}

template <int D, int C, bool STAGE, bool PERWAVE, bool CONV = false>
__global__ __launch_bounds__(256, (C <= 64 ? (CONV ? 3 : 4) : 2)) void prep_kernel(Geom g, PrefillWs L,
                                                   const float *__restrict__ gl,
                                                   const float *__restrict__ beta,
                                                   char *__restrict__ ws,
                                                   const void *__restrict__ x,
                                                   const void *__restrict__ conv_w,
                                                   void *__restrict__ hist) {
  using Sh = PrepShape<D, C>;
  constexpr int NT = Sh::NT, NTRI = Sh::NTRI, Dp = Sh::Dp;
  // Gram tiles, row-major 16 x 16 (with CONV, first the conv's scratch)
  __shared__ __attribute__((aligned(16))) float KK[NTRI][256];
  __shared__ __attribute__((aligned(16))) float QK[NTRI][256];
  // A, then (I + A)^{-1} in place; before that (STAGE, chunks of at most 64
  // tokens), the chunk's K tiles as MFMA operands (hi and lo, bf16).
  constexpr bool kStageK = STAGE && C <= 64;
  // Chunks of 128 (four-wave form): P of every value head is formed and
  // stored right after the Gram products, so that each head's inverse then
  // works in QK's space; the block takes 74 instead of 111 KB of LDS and two
  // blocks share a compute unit.
  constexpr bool kPFirst = !STAGE && !PERWAVE && C > 64;
  constexpr size_t kTiBytes = kPFirst ? 16 : sizeof(float) * NTRI * 256 * (PERWAVE ? kHeadSlots : 1);
  constexpr size_t kStageBytes = kStageK ? size_t(2) * NT * 16 * Dp * 2 : 0;
  __shared__ __attribute__((aligned(16))) unsigned char ti_raw[kTiBytes > kStageBytes ? kTiBytes : kStageBytes];
  float (*TI)[256] = kPFirst ? QK : reinterpret_cast<float (*)[256]>(ti_raw);
  // the four-wave form's gate prefix and beta (the per-wave form keeps them in registers)
  __shared__ float Gs[PERWAVE ? 1 : C], Bs[PERWAVE ? 1 : C];

  const int chunk = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, gq = lane >> 4;
  const int64_t tau0 = static_cast<int64_t>(chunk) * C;
  const int n_valid = static_cast<int>((L.T - tau0) < C ? (L.T - tau0) : C);

  // 0. With CONV, this block first computes its chunk of q-hat and k-hat
  //    from x (the conv pass does not run); the first chunk's blocks then
  //    roll the history of exactly the channels they read (no other block
  //    reads them, and their own reads are done).
  // With CONV: wave w's Q operands of token tile w, from the conv.
  [[maybe_unused]] u16x8 cq_h[4], cq_l[4];
  if constexpr (CONV) {
    static_assert(D == 128 && C == 64 && STAGE && PERWAVE, "fused conv: split-role prefill, staged grids");
    static_assert(sizeof(KK) >= kPrepConvScratchA && sizeof(QK) >= kPrepConvScratchB &&
                      sizeof(ti_raw) >= size_t(2) * C * 128 * 2,
                  "conv scratch in the Gram tiles, K rows in the staging space");
    unsigned char *sa = reinterpret_cast<unsigned char *>(&KK[0][0]);
    unsigned char *sb = reinterpret_cast<unsigned char *>(&QK[0][0]);
    uint16_t (*krows)[128] = reinterpret_cast<uint16_t (*)[128]>(ti_raw);
    if (g.in_dt == 0)
      prep_conv_qk<0, C>(g, L, x, conv_w, hist, ws, b, kh, tau0, sa, sb, krows, cq_h, cq_l);
    else
      prep_conv_qk<1, C>(g, L, x, conv_w, hist, ws, b, kh, tau0, sa, sb, krows, cq_h, cq_l);
    if (chunk == 0) {
      const int nq = g.H_k * D;
#pragma unroll 1
      for (int part = 0; part < 2; ++part) {
        const int c0 = part * nq + kh * D;
        if (g.in_dt == 0)
          roll_history(g.C_ch, L.T, b, c0, c0 + D, static_cast<const uint32_t *>(x), static_cast<uint32_t *>(hist));
        else
          roll_history(g.C_ch, L.T, b, c0, c0 + D, static_cast<const uint16_t *>(x), static_cast<uint16_t *>(hist));
      }
    }
  }
  // Otherwise the conv history roll rides on the first chunk's blocks (one
  // slice of the channels per key head): the conv pass, its only reader, has
  // finished before this kernel starts.
  if (!CONV && chunk == 0) {
    // With the split-role state pass, that pass rolls the v channels itself.
    const int nroll = prefill_split_roles(g, L) ? 2 * g.H_k * g.D : g.C_ch;
    const int per = (nroll + g.H_k - 1) / g.H_k;
    const int c0 = kh * per, c1 = c0 + per < nroll ? c0 + per : nroll;
    if (g.in_dt == 0)
      roll_history(g.C_ch, L.T, b, c0, c1, static_cast<const uint32_t *>(x), static_cast<uint32_t *>(hist));
    else
      roll_history(g.C_ch, L.T, b, c0, c1, static_cast<const uint16_t *>(x), static_cast<uint16_t *>(hist));
  }

  // 1. K K^T and Q K^T, lower tiles only, split operands.  With STAGE, K is
  //    staged in LDS (each tile read from the workspace once; the grids of
  //    long sequences, which are bound by HBM traffic, take this form);
  //    otherwise the tiles go to the waves in contiguous runs of the
  //    column-major order (column nt, then row mt), so a wave loads each K
  //    column tile it needs (the B operand of both products) once, and each
  //    K and Q row tile once, and the smaller LDS footprint keeps four blocks
  //    on a compute unit.
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
    if constexpr (kStageK) {
      // Each wave loads token tile `wave` of K (hi, lo widened) and of Q once;
      // K goes to LDS for the other waves.  Wave w then computes the Gram tiles
      // of row tile w: K_w K_n^T and Q_w K_n^T for n <= w, with its own K_w
      // and Q_w from registers and K_n from LDS (the same operands, in the
      // same order, as tile-by-tile loads from the workspace would give).
      // Rows of Dp bf16; the 16-byte piece p of row t sits at piece p ^ (t mod
      // NP), so the 16 rows that one operand read touches land on distinct
      // banks without padding.
      typedef uint16_t KRow[Dp];
      constexpr int NP = Dp / 8;
      KRow *Kh = reinterpret_cast<KRow *>(ti_raw);            // [NT * 16][Dp]
      KRow *Kl = reinterpret_cast<KRow *>(ti_raw) + NT * 16;  // low halves, bf16
      const int sw = c & (NP - 1);
      u16x8 akh[KS], akl[KS], aqh[KS], aql[KS];
      if (wave < NT) {
        if constexpr (CONV) {
          // K's rows are already staged and Q's operands in registers.
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int off = 8 * ((4 * ks + gq) ^ sw);
            akh[ks] = *reinterpret_cast<const u16x8 *>(&Kh[16 * wave + c][off]);
            akl[ks] = *reinterpret_cast<const u16x8 *>(&Kl[16 * wave + c][off]);
            aqh[ks] = cq_h[ks];
            aql[ks] = cq_l[ks];
          }
        } else {
          load_tile(khi, klo, L.k_lo_scale, wave, akh, akl);
          load_tile(qhi, qlo, L.q_lo_scale, wave, aqh, aql);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int off = 8 * ((4 * ks + gq) ^ sw);
            *reinterpret_cast<u16x8 *>(&Kh[16 * wave + c][off]) = akh[ks];
            *reinterpret_cast<u16x8 *>(&Kl[16 * wave + c][off]) = akl[ks];
          }
        }
      }
      __syncthreads();
      if (wave < NT) {
        const int mt = wave;
        for (int nt = 0; nt <= mt; ++nt) {
          u16x8 bh[KS], bl[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int off = 8 * ((4 * ks + gq) ^ sw);
            bh[ks] = *reinterpret_cast<const u16x8 *>(&Kh[16 * nt + c][off]);
            bl[ks] = *reinterpret_cast<const u16x8 *>(&Kl[16 * nt + c][off]);
          }
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
    } else {
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
  }

  if constexpr (PERWAVE) {
    // Value heads in parallel, one per wave (wave w: heads w, w + 3, ...),
    // each in its own slot of TI.
    static_assert(C <= 64, "per-wave heads need C <= 64");
    __syncthreads();  // Gram tiles written; the K staging (aliased with TI) no longer read
    if (wave < kHeadSlots)
      for (int jv = wave; jv < g.G; jv += kHeadSlots)
        prep_head_wave<D, C>(g, L, gl, beta, ws, KK, QK, TI + wave * NTRI, b, kh * g.G + jv, chunk,
                             tau0, n_valid);
    return;
  } else {
  // Gate prefix G_t and beta_t of value head h into Gs, Bs (wave 0).
  auto head_prefix = [&](int h) {
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
  };
  if constexpr (kPFirst) {
    for (int jv = 0; jv < g.G; ++jv) {
      const int h = kh * g.G + jv;
      __syncthreads();  // Gram tiles written; previous head's readers done
      head_prefix(h);
      __syncthreads();
      store_gate_table<D, C>(g, L, ws, b, h, chunk, Gs, Bs);
      store_pieces<D, C, false, true>(g, L, ws, b, h, chunk, Gs, TI, QK);
    }
  }
  for (int jv = 0; jv < g.G; ++jv) {
    const int h = kh * g.G + jv;
    __syncthreads();  // Gram tiles (and with kPFirst, every head's P) done; previous head's readers done
    head_prefix(h);
    __syncthreads();

    // Gate factors of this chunk for the state pass.
    if constexpr (!kPFirst) store_gate_table<D, C>(g, L, ws, b, h, chunk, Gs, Bs);

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

    // 3. Store Tm (bf16) and P (hi/lo) as A operands (with kPFirst, P was
    //    stored before the inverses).
    store_pieces<D, C, true, !kPFirst>(g, L, ws, b, h, chunk, Gs, TI, QK);
  }
  }
}

// ---------------------------------------------------------------- launcher

// K staged in LDS once the grid spans more than kPrepStageBlocks (8 blocks
// per compute unit): a 4096-token prefill (1,024 blocks) then keeps every
// block resident at once (37 against 47 us staged), and 65,536 tokens
// (16,384 blocks, bound by HBM traffic) read 1.31 instead of 1.84 GB (535
// against 582 us).

template <int D, int C>
static void launch_prep_t(const Geom &g, const PrefillWs &L, const float *gl, const float *beta,
                          char *ws, const void *x, const void *conv_w, void *hist, hipStream_t s,
                          const KernelEvents *ev) {
  dim3 grid(L.NC, g.H_k, g.B);
  const bool stage = C <= 64 && static_cast<int64_t>(L.NC) * g.H_k * g.B > kPrepStageBlocks;
  if constexpr (D == 128 && C == 64) {
    if (prep_fuses_conv(g, L)) {
      launch_kernel(prep_kernel<D, C, true, true, true>, grid, dim3(256), s, ev, g, L, gl, beta, ws, x,
                    conv_w, hist);
      return;
    }
  }
  if constexpr (C <= 64) {
    if (stage && g.G >= 2) {
      // Value heads one per wave: 511-517 against 543-571 us at T = 65,536
      // (bitwise equal).  Smaller grids keep the four-wave form, whose
      // smaller LDS footprint keeps four blocks per compute unit (35 against
      // 41 us at T = 4096).
      launch_kernel(prep_kernel<D, C, true, true>, grid, dim3(256), s, ev, g, L, gl, beta, ws, x, conv_w,
                    hist);
      return;
    }
  }
  if (stage)
    launch_kernel(prep_kernel<D, C, true, false>, grid, dim3(256), s, ev, g, L, gl, beta, ws, x, conv_w, hist);
  else
    launch_kernel(prep_kernel<D, C, false, false>, grid, dim3(256), s, ev, g, L, gl, beta, ws, x, conv_w, hist);
}

hipError_t launch_prefill_prep(const Geom &g, const PrefillWs &L, const float *gl,
                               const float *beta, char *ws, const void *x, const void *conv_w,
                               void *hist, hipStream_t s, const KernelEvents *ev) {
#define GDN_PREP(Dv)                                                               \
  switch (L.C) {                                                                   \
    case 16: launch_prep_t<Dv, 16>(g, L, gl, beta, ws, x, conv_w, hist, s, ev); break;  \
    case 32: launch_prep_t<Dv, 32>(g, L, gl, beta, ws, x, conv_w, hist, s, ev); break;  \
    case 64: launch_prep_t<Dv, 64>(g, L, gl, beta, ws, x, conv_w, hist, s, ev); break;  \
    default: launch_prep_t<Dv, 128>(g, L, gl, beta, ws, x, conv_w, hist, s, ev); break; \
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
