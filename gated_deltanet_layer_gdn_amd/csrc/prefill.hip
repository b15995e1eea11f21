// prefill.hip -- state pass of the chunked gated delta rule (WY / UT form)
// on bf16 MFMA for gfx950, fused with the sigmoid output gate.
//
// For one value head, a chunk of C tokens with entry state S0 (d_v x d_k),
// G_t = sum_{r<=t} g_r, gamma_t = exp(G_t), D_ts = exp(G_t - G_s), and the
// chunk-local Tm = (I + A)^{-1} and P = tril(D) * (Q K^T) from the prep pass:
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
// Kernels (serial over chunks, parallel over sequences, value heads and row
// blocks of S; S^T stays in MFMA accumulator registers for the whole
// sequence):
//   state_kernel_ws (d = 128, C = 64): 32 rows of S per block, eight waves in
//         two roles.  Chain waves: K S^T over the full depth for one token
//         tile, R, U = Tm R, and one d_k quarter of the state update; they
//         also turn x into V (conv + SiLU) for the next chunk.  Output waves,
//         concurrently: Q S^T, P U, the gate and the y stores, and the staging
//         of x.  K^T for the update comes from an LDS copy of K through
//         transposing loads.
//   state_kernel (other chunk sizes, d = 16): 16 or 32 rows per block, four
//         waves splitting d_k; K S^T and Q S^T partials reduced through LDS.
// Precision: every product that carries the value path uses split bf16
// operands (hi + lo, 16 significant bits) with fp32 accumulation; only Tm
// (unit diagonal, small off-diagonal) is rounded to plain bf16.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// ---------------------------------------------------------------- state kernel

template <int D, int C>
struct StateShape {
  static constexpr int NWV = D >= 128 ? 4 : 1;   // waves; each owns a slice of d_k
  static constexpr int NDT = D >= 32 ? 2 : 1;    // 16-wide d_k tiles per wave
  // 16-row state tiles per block: two share every K / Q / K^T operand load
  // (for 128-token chunks only with U and DU in the partial sums' space).
  static constexpr int NB = D >= 128 ? 2 : 1;
  static constexpr int ROWS = 16 * NB;           // state rows per block
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

// Load through a block-uniform base and a 32-bit byte offset (lets the
// compiler use the scalar-base + vector-offset addressing form).
template <typename V>
__device__ __forceinline__ V ldb(const void *base, uint32_t byte_off) {
  return *reinterpret_cast<const V *>(static_cast<const char *>(base) + byte_off);
}

// Raw buffer resource over `bytes` bytes from `base` (stride 0, gfx9 word 3):
// loads take a wave-uniform base in scalar registers, a 32-bit vector
// offset and a scalar offset, so they need no 64-bit address arithmetic on
// the VALU; loads at or past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

template <typename V>
__device__ __forceinline__ V bld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(V) == 4)
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
  else if constexpr (sizeof(V) == 8)
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
  else
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

constexpr uint32_t kAllBytes = 0xffffffffu;

// A value at a wave-uniform address through a vector load.  A scalar load
// would share its wait counter with LDS, so every LDS wait issued while it
// is in flight would also wait for its L2 round trip.
__device__ __forceinline__ float ld_uniform_vec(const float *base, uint32_t byte_off) {
  asm volatile("" : "+v"(byte_off));
  return ldb<float>(base, byte_off);
}

// Per-chunk operands of one wave.  None of them depends on the state, so
// each is fetched for the next chunk as soon as this chunk has consumed it
// (into the same registers): every load has about one chunk of compute to
// arrive.  Wave w owns the output tokens of tiles w, w + NWV, ...
template <int NT, int MW, int KSC, int NDT, int NB, int ZK>
struct ChunkOps {
  u16x8 kh[NT], kl[NT], qh[NT], ql[NT];  // A operands of K S^T / Q S^T (all tiles, own d_k slice)
  float4 gam[MW], dl[MW], bt[MW];        // gate factors of the owned tiles (D-register order)
  float glast;                           // gamma of the chunk's last token
  float4 v[MW][NB];                      // V of the owned tiles (D-register order)
  u16x8 tm[MW][KSC], ph[MW][KSC], pl[MW][KSC];  // (I+A)^{-1} and P rows of owned tiles
  uint4 z[MW][ZK];                       // gate inputs of the owned tiles, token-major 16-byte pieces
  u16x8 th[NDT][KSC], tl[NDT][KSC];      // A operands of the state update (own d_k slice)
};

// Four bf16 values of one D-register tile, hi and lo halves.
struct Split4 {
  uint2 hi, lo;
};

template <int D, int C, int DTZ, int DTY>
struct StateKernel {
  using SS = StateShape<D, C>;
  static constexpr int NWV = SS::NWV, NDT = SS::NDT, Dp = SS::Dp, NB = SS::NB, ROWS = SS::ROWS;
  static constexpr int NT = C / 16, Cp = C < 32 ? 32 : C, KSC = Cp / 32;
  static constexpr int MW = (NT + NWV - 1) / NWV;  // output tiles per wave
  static constexpr int EZ = DTZ == 0 ? 4 : 2;      // bytes per z element
  static constexpr int ZL = ROWS * EZ / 16;        // 16-byte pieces per token row of z
  static constexpr int ZK = (16 * ZL + 63) / 64;   // pieces per lane per tile
  using Ops = ChunkOps<NT, MW, KSC, NDT, NB, ZK>;

  // Shared memory of one block.  Every tile is stored in D-register order
  // (one entry per lane), so writes and reads are lane-contiguous.
  struct SmemPlain {
    f32x4 part[NWV][2][NT][NB][64];  // K S^T / Q S^T partial sums of each wave's d_k slice
    Split4 R[NT][NB][64];            // R tiles, split
    Split4 U[NT][NB][64];            // U tiles, split (operand of P U)
    Split4 DU[NT][NB][64];           // exp(G_last - G_t) U tiles, split (operand of the update)
    uint4 z[NWV][16 * ZL];           // per wave: one token tile of z, token-major
  };
  // d = 128, chunk 128: U and DU share the partial sums' space (those are
  // consumed in step 2, before step 3 writes U), which brings the 32-row
  // block to 148 KB of LDS, so that 192 blocks (one per compute unit) cover
  // one sequence of 48 heads in one round; a barrier at the top of each
  // chunk keeps the next chunk's partial sums from overwriting U and DU
  // while steps 4 and 5 of other waves still read them.
  static constexpr bool kAliasUDU = D == 128 && C == 128;
  struct SmemAlias {
    union {
      f32x4 part[NWV][2][NT][NB][64];
      struct {
        Split4 U[NT][NB][64];
        Split4 DU[NT][NB][64];
      };
    };
    Split4 R[NT][NB][64];
    uint4 z[NWV][16 * ZL];
  };
  using Smem = typename std::conditional<kAliasUDU, SmemAlias, SmemPlain>::type;

  // Wave-uniform base pointers (advanced per chunk by uniform strides) and
  // per-lane byte offsets, so that every load is base + 32-bit offset.
  struct Ctx {
    const uint16_t *khi, *klo, *qhi, *qlo;  // this wave's 32-slice of the token-major rows
    const uint16_t *kThi, *kTlo;            // dim-major blocks of this key head
    const float *vT;                        // dim-major v of this value head
    const uint16_t *Tm, *Ph, *Pl;           // chunk matrices of this value head
    const float *gates;                     // gate table of this value head
    const void *z;                          // [.][T][H_v][D] at (b, 0, h, first row)
    void *y;
    int64_t T;
    int H_v, NC, wave, lane, gq;
    uint32_t o_tok, o_kT, o_v, o_mat, o_zy, o_gate;  // byte offsets (o_zy: elements)
  };

  static __device__ __forceinline__ int valid_of(const Ctx &x, int chunk) {
    const int64_t r = x.T - static_cast<int64_t>(chunk) * C;
    return static_cast<int>(r < C ? r : C);
  }

  static __device__ __forceinline__ Split4 split4(const f32x4 &v) {
    uint32_t h0, h1, l0, l1;
    split2(v[0], v[1], h0, l0);
    split2(v[2], v[3], h1, l1);
    return Split4{make_uint2(h0, h1), make_uint2(l0, l1)};
  }

  // B operand of one 32-wide K step from two split tiles (second may be absent).
  static __device__ __forceinline__ void operand(const Split4 &a, const Split4 &b, u16x8 &hi,
                                                 u16x8 &lo) {
    const u32x4 h = {a.hi.x, a.hi.y, b.hi.x, b.hi.y}, l = {a.lo.x, a.lo.y, b.lo.x, b.lo.y};
    hi = __builtin_bit_cast(u16x8, h);
    lo = __builtin_bit_cast(u16x8, l);
  }

  // The loads below are branch-free (indices are clamped instead, so a load
  // that is not needed re-reads a valid address): the compiler then knows
  // exactly which loads are outstanding and waits only for the ones a
  // product needs, keeping the next chunk's loads in flight.
  static __device__ __forceinline__ int own_tile(const Ctx &x, int i) {
    const int m = x.wave + i * NWV;
    return m < NT ? m : NT - 1;
  }

  static __device__ __forceinline__ void load_head(const Ctx &x, int chunk, Ops &o) {
    const size_t row = static_cast<size_t>(chunk) * C * 32 * 2;
    const char *kh = reinterpret_cast<const char *>(x.khi) + row;
    const char *kl = reinterpret_cast<const char *>(x.klo) + row;
    const char *qh = reinterpret_cast<const char *>(x.qhi) + row;
    const char *ql = reinterpret_cast<const char *>(x.qlo) + row;
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const uint32_t ao = x.o_tok + 16 * m * 32 * 2;
      o.kh[m] = ldb<u16x8>(kh, ao);
      o.kl[m] = ldb<u16x8>(kl, ao);
      o.qh[m] = ldb<u16x8>(qh, ao);
      o.ql[m] = ldb<u16x8>(ql, ao);
    }
  }

  // Gate factors are used in steps 2-5, so they are fetched after step 5.
  static __device__ __forceinline__ void load_gates(const Ctx &x, int chunk, Ops &o) {
    const float *gb = x.gates + static_cast<size_t>(chunk) * 3 * C;
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int m = own_tile(x, i);
      o.gam[i] = ldb<float4>(gb, x.o_gate + m * 64);
      o.dl[i] = ldb<float4>(gb, x.o_gate + m * 64 + C * 4);
      o.bt[i] = ldb<float4>(gb, x.o_gate + m * 64 + 2 * C * 4);
    }
    o.glast = ld_uniform_vec(gb, (C - 1) * 4);
  }

  static __device__ __forceinline__ void load_v(const Ctx &x, int chunk, Ops &o) {
    const float *base = x.vT + static_cast<size_t>(chunk) * C * D;
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int m = own_tile(x, i);
#pragma unroll
      for (int n = 0; n < NB; ++n) o.v[i][n] = ldb<float4>(base, x.o_v + (m * 16 * D + n * 16 * 16) * 4);
    }
  }

  static __device__ __forceinline__ void load_tm(const Ctx &x, int chunk, Ops &o) {
    const uint16_t *base = x.Tm + static_cast<size_t>(chunk) * C * Cp;
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int m = own_tile(x, i);
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        const int kk = ks <= m / 2 ? ks : m / 2;
        o.tm[i][ks] = ldb<u16x8>(base, x.o_mat + (16 * m * Cp + 32 * kk) * 2);
      }
    }
  }

  static __device__ __forceinline__ void load_pz(const Ctx &x, int chunk, Ops &o) {
    const size_t mo = static_cast<size_t>(chunk) * C * Cp;
    const uint16_t *ph = x.Ph + mo;
    const uint16_t *pl = x.Pl + mo;
    const int n_valid = valid_of(x, chunk);  // >= 1 for every chunk of the sequence
    const char *zb = static_cast<const char *>(x.z) + static_cast<size_t>(chunk) * C * x.H_v * D * EZ;
    const uint32_t tstride = x.H_v * D * EZ;
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int m = own_tile(x, i);
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        const int kk = ks <= m / 2 ? ks : m / 2;
        const uint32_t ao = x.o_mat + (16 * m * Cp + 32 * kk) * 2;
        o.ph[i][ks] = ldb<u16x8>(ph, ao);
        o.pl[i][ks] = ldb<u16x8>(pl, ao);
      }
      // z of this tile: 16 token rows of ROWS elements, one 16-byte piece per
      // lane; rows past the sequence end re-read its last row (their outputs
      // are not stored).
      if constexpr (out_gated(DTY)) {
#pragma unroll
        for (int k = 0; k < ZK; ++k) {
          int idx = x.lane + 64 * k;
          idx = idx < 16 * ZL ? idx : 16 * ZL - 1;
          int t = 16 * m + idx / ZL;
          t = t < n_valid ? t : n_valid - 1;
          o.z[i][k] = ldb<uint4>(zb, t * tstride + (idx % ZL) * 16);
        }
      }
    }
  }

  static __device__ __forceinline__ void load_kT(const Ctx &x, int chunk, Ops &o) {
    // The 32-token key block that holds the chunk (a 16-token chunk with an
    // odd index sits in the second half of its block).
    const size_t base = static_cast<size_t>((static_cast<int64_t>(chunk) * C) & ~int64_t(31)) * D;
    const uint16_t *th = x.kThi + base;
    const uint16_t *tl = x.kTlo + base;
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint32_t ao = x.o_kT + (ks * D + 16 * dt) * 32 * 2;
        o.th[dt][ks] = ldb<u16x8>(th, ao);
        o.tl[dt][ks] = ldb<u16x8>(tl, ao);
      }
  }

  // First chunk's operands, issued in the order the loop issues them (the
  // compiler barriers keep that order), so that the wait counts at the top of
  // the loop are the same on entry as on every later iteration.
  static __device__ __forceinline__ void load_all(const Ctx &x, int chunk, Ops &o) {
    load_head(x, chunk, o);
    asm volatile("" ::: "memory");
    load_v(x, chunk, o);
    asm volatile("" ::: "memory");
    load_tm(x, chunk, o);
    asm volatile("" ::: "memory");
    load_pz(x, chunk, o);
    asm volatile("" ::: "memory");
    load_kT(x, chunk, o);
    load_gates(x, chunk, o);
    asm volatile("" ::: "memory");
  }

  // One chunk.  On entry `o` holds this chunk's operands (loads possibly in
  // flight); on exit it holds the next chunk's.  Three barriers: after the
  // K S^T / Q S^T partials, after the R tiles, after the U tiles.  The gated
  // outputs are stored last, after every load for the next chunk is issued,
  // so that no later wait on those loads also waits for these stores.
  static __device__ __forceinline__ void chunk_step(const Ctx &x, int chunk, Ops &o,
                                                    f32x4 (&st)[NB][NDT], Smem &sm) {
    const int lane = x.lane, wave = x.wave, gq = x.gq, c = lane & 15;
    const int n_valid = valid_of(x, chunk);
    // The last chunk re-reads its own operands instead of branching.
    const int next = chunk + 1 < x.NC ? chunk + 1 : chunk;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const Split4 none = {make_uint2(0u, 0u), make_uint2(0u, 0u)};
    if constexpr (kAliasUDU) __syncthreads();

    // 1. Partial K S^T and Q S^T over this wave's d_k slice, all token tiles.
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      u16x8 bh, bl;
      pack_split(st[n][0], NDT > 1 ? st[n][NDT - 1] : zero, bh, bl);
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        sm.part[wave][0][m][n][lane] = mfma_split3(o.kh[m], o.kl[m], bh, bl, zero);
        sm.part[wave][1][m][n][lane] = mfma_split3(o.qh[m], o.ql[m], bh, bl, zero);
      }
    }
    load_head(x, next, o);
    __syncthreads();

    // 2. Owned tiles: R = beta (V - gamma K S^T), published split; Q S^T kept.
    f32x4 qs[MW][NB];
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int m = wave + i * NWV;
      if (m < NT) {
        const float4 g4 = o.gam[i], b4 = o.bt[i];
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          f32x4 ks = sm.part[0][0][m][n][lane];
          qs[i][n] = sm.part[0][1][m][n][lane];
#pragma unroll
          for (int w = 1; w < NWV; ++w) {
            ks += sm.part[w][0][m][n][lane];
            qs[i][n] += sm.part[w][1][m][n][lane];
          }
          const float4 vv = o.v[i][n];
          const f32x4 r = {b4.x * (vv.x - g4.x * ks[0]), b4.y * (vv.y - g4.y * ks[1]),
                           b4.z * (vv.z - g4.z * ks[2]), b4.w * (vv.w - g4.w * ks[3])};
          sm.R[m][n][lane] = split4(r);
        }
      }
    }
    load_v(x, next, o);
    __syncthreads();

    // 3. Owned tiles: U = Tm R, published split, also scaled by exp(G_last - G_t).
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int m = wave + i * NWV;
      if (m < NT) {
        const float4 d4 = o.dl[i];
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          f32x4 acc = zero;
#pragma unroll
          for (int ks = 0; ks < KSC; ++ks)
            if (ks <= m / 2) {
              u16x8 bh, bl;
              operand(sm.R[2 * ks][n][lane],
                      (2 * ks + 1 < NT) ? sm.R[(2 * ks + 1) % NT][n][lane] : none, bh, bl);
              acc = mfma_split2(o.tm[i][ks], bh, bl, acc);
            }
          sm.U[m][n][lane] = split4(acc);
          const f32x4 du = {d4.x * acc[0], d4.y * acc[1], d4.z * acc[2], d4.w * acc[3]};
          sm.DU[m][n][lane] = split4(du);
        }
      }
    }
    load_tm(x, next, o);
    __syncthreads();

    // 4. Owned tiles: O = gamma Q S^T + P U, gated (stored at the end).  z
    //    arrives token-major; this wave's LDS slot turns it into D-register order.
    f32x4 out[MW][NB];
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int m = wave + i * NWV;
      if (m < NT) {
        if constexpr (out_gated(DTY)) {
#pragma unroll
          for (int k = 0; k < ZK; ++k)
            if (lane + 64 * k < 16 * ZL) sm.z[wave][lane + 64 * k] = o.z[i][k];
        }
        // Other lanes of this wave read what was just written: keep the
        // compiler from moving those reads above the stores (LDS operations of
        // one wave execute in order).
        asm volatile("" ::: "memory");
        const char *zt = reinterpret_cast<const char *>(sm.z[wave]);
        const float4 g4 = o.gam[i];
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          f32x4 acc = {g4.x * qs[i][n][0], g4.y * qs[i][n][1], g4.z * qs[i][n][2], g4.w * qs[i][n][3]};
#pragma unroll
          for (int ks = 0; ks < KSC; ++ks)
            if (ks <= m / 2) {
              u16x8 bh, bl;
              operand(sm.U[2 * ks][n][lane],
                      (2 * ks + 1 < NT) ? sm.U[(2 * ks + 1) % NT][n][lane] : none, bh, bl);
              acc = mfma_split3(o.ph[i][ks], o.pl[i][ks], bh, bl, acc);
            }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (out_gated(DTY)) {
              const int off = ((4 * gq + r) * ROWS + 16 * n + c) * EZ;
              float zz;
              if constexpr (DTZ == 0)
                zz = *reinterpret_cast<const float *>(zt + off);
              else
                zz = bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(zt + off));
              out[i][n][r] = acc[r] * sigmoidf_(zz);
            } else {
              out[i][n][r] = acc[r];
            }
          }
        }
        asm volatile("" ::: "memory");
      }
    }
    load_pz(x, next, o);

    // 5. S^T <- gamma_last S^T + K^T (D_last * U) over this wave's d_k slice.
    {
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) st[n][dt] *= o.glast;
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
          Split4 a = sm.DU[2 * ks < NT ? 2 * ks : 0][n][lane];
          Split4 b = (2 * ks + 1 < NT) ? sm.DU[(2 * ks + 1) % NT][n][lane] : none;
          // A 16-token chunk fills one half of a 32-token key block.
          if (C == 16 && (chunk & 1)) {
            b = a;
            a = none;
          }
          u16x8 bh, bl;
          operand(a, b, bh, bl);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            st[n][dt] = mfma_split3(o.th[dt][ks], o.tl[dt][ks], bh, bl, st[n][dt]);
        }
      }
    }
    load_kT(x, next, o);
    load_gates(x, next, o);

    // 6. Gated outputs of the owned tiles.
    constexpr int ey = out_bytes(DTY);
    char *yb = static_cast<char *>(x.y) + static_cast<size_t>(chunk) * C * x.H_v * D * ey;
    const uint32_t tstride = x.H_v * D * ey;
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int m = wave + i * NWV;
      if (m < NT) {
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * m + 4 * gq + r;
            if (t < n_valid) {
              char *dst = yb + (x.o_zy + 16 * n) * ey + (16 * m + r) * tstride;
              if constexpr (out_type(DTY) == 0)
                *reinterpret_cast<float *>(dst) = out[i][n][r];
              else if constexpr (out_type(DTY) == 1)
                *reinterpret_cast<uint16_t *>(dst) = f32_to_bf16_bits(out[i][n][r]);
              else
                *reinterpret_cast<uint16_t *>(dst) = f32_to_f16_bits(out[i][n][r]);
            }
          }
      }
    }
  }
};

template <int D, int C, int DTZ, int DTY>
__global__ __launch_bounds__((StateShape<D, C>::NWV * 64)) void state_kernel(
    Geom g, PrefillWs L, const void *__restrict__ z, float *__restrict__ S, void *__restrict__ y,
    const char *__restrict__ ws) {
  using K = StateKernel<D, C, DTZ, DTY>;
  constexpr int NDT = K::NDT, NB = K::NB, Dp = K::Dp, Cp = K::Cp, ROWS = K::ROWS;
  __shared__ typename K::Smem sm;

  const int RB = D / ROWS;
  const int lid = xcd_remap(blockIdx.x, g.B * g.H_v * RB);
  const int rb = lid % RB;
  const int h = (lid / RB) % g.H_v;
  const int b = lid / (RB * g.H_v);
  const int kh = h / g.G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, gq = lane >> 4;

  typename K::Ctx x;
  // token-major slices: [b][kh][slice][T_pad][32]; this wave reads slice `wave`
  const size_t slice0 = ((static_cast<size_t>(b) * g.H_k + kh) * (Dp / 32) + wave) * L.T_pad * 32;
  x.khi = reinterpret_cast<const uint16_t *>(ws + L.k_hi) + slice0;
  x.klo = reinterpret_cast<const uint16_t *>(ws + L.k_lo) + slice0;
  x.qhi = reinterpret_cast<const uint16_t *>(ws + L.q_hi) + slice0;
  x.qlo = reinterpret_cast<const uint16_t *>(ws + L.q_lo) + slice0;
  const size_t kbase = (static_cast<size_t>(b) * g.H_k + kh) * L.T_pad;
  x.kThi = reinterpret_cast<const uint16_t *>(ws + L.kT_hi) + kbase * D;
  x.kTlo = reinterpret_cast<const uint16_t *>(ws + L.kT_lo) + kbase * D;
  x.vT = reinterpret_cast<const float *>(ws + L.vT) +
         (static_cast<size_t>(b) * g.H_v + h) * L.T_pad * D;
  const size_t mat = (static_cast<size_t>(b) * g.H_v + h) * L.NC * C * Cp;
  x.Tm = reinterpret_cast<const uint16_t *>(ws + L.Tm) + mat;
  x.Ph = reinterpret_cast<const uint16_t *>(ws + L.P_hi) + mat;
  x.Pl = reinterpret_cast<const uint16_t *>(ws + L.P_lo) + mat;
  x.gates = reinterpret_cast<const float *>(ws + L.gates) +
            (static_cast<size_t>(b) * g.H_v + h) * L.NC * 3 * C;
  const size_t zy = (static_cast<size_t>(b) * L.T * g.H_v + h) * D + ROWS * rb;
  x.z = static_cast<const char *>(z) + zy * K::EZ;
  x.y = static_cast<char *>(y) + zy * out_bytes(DTY);
  x.T = L.T;
  x.H_v = g.H_v;
  x.NC = L.NC;
  x.wave = wave;
  x.lane = lane;
  x.gq = gq;
  x.o_tok = (c * 32 + 8 * gq) * 2;
  x.o_kT = ((32 * wave + c) * 32 + 8 * gq) * 2;
  x.o_v = ((ROWS * rb + c) * 16 + 4 * gq) * 4;
  x.o_mat = (c * Cp + 8 * gq) * 2;
  x.o_zy = 4 * gq * g.H_v * D + c;
  x.o_gate = 4 * gq * 4;

  // S^T tiles: for state-row tile n, rows d_k = 32*wave + 16*dt + 4*gq + r,
  // column = state row ROWS*rb + 16*n + c.
  float *Sh = S + ((static_cast<size_t>(b) * g.H_v + h) * D + ROWS * rb + c) * D;
  f32x4 st[NB][NDT];
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const float4 v = *reinterpret_cast<const float4 *>(Sh + 16 * n * D + 32 * wave + 16 * dt + 4 * gq);
      st[n][dt] = f32x4{v.x, v.y, v.z, v.w};
    }

  typename K::Ops ops;
  K::load_all(x, 0, ops);
  for (int chunk = 0; chunk < L.NC; ++chunk) K::chunk_step(x, chunk, ops, st, sm);

#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<float4 *>(Sh + 16 * n * D + 32 * wave + 16 * dt + 4 * gq) =
          make_float4(st[n][dt][0], st[n][dt][1], st[n][dt][2], st[n][dt][3]);
}

// ---------------------------------------------------------------- state pass, split roles
//
// The state recurrence of a chunk is a chain (K S^T -> R -> U -> S update),
// while the outputs (Q S^T, P U, the gate and the stores) hang off it.  With
// d = 128 and 64-token chunks the block therefore runs eight waves, two per
// SIMD: chain waves 0-3 own token tile w for K S^T, R and U and d_k slice w
// of the state, output waves 4-7 own token tile w - 4 for Q S^T, P U and y.
// Both kinds of wave go through the same three barriers per chunk, so a
// SIMD always has the other wave's independent products to issue while one
// waits on a barrier, an LDS round trip or a dependent MFMA.  The state is
// shared as ready-made split B operands (one 32-wide d_k step per chain
// wave), so each wave forms its full-depth products itself and no partial
// sums cross waves.
//   phase 1: chain  KS = K_t S^T (full d_k), R = beta (V - gamma KS) -> LDS
//            output QS = Q_t S^T (kept in registers)
//   phase 2: chain  U = Tm R, DU = exp(G_last - G) U -> LDS
//            output z tile -> sigmoid, through the wave's LDS slot
//   phase 3: chain  S^T <- gamma_last S^T + K^T DU, new state operands -> LDS
//            output O = gamma QS + P U, y = O sigmoid(z) -> HBM
// K^T of the update comes from a token-major LDS copy of the chunk's K (the
// chain waves' A operand registers, stored as held) through transposing
// loads; V is SiLU(conv x) of the block's v channels, from x tiles the output
// waves stage; the low halves of q, k and P arrive as scaled e4m3 bytes and
// are widened to bf16 in registers.  Column c of the two 16-column tiles
// (n = 0, 1) is the block's state row 2c + n, so each lane's two channels
// sit side by side in x, z and y: one 4- or 8-byte access serves both.
template <int DTZ, int DTY>
struct StateKernelWS {
  static constexpr int D = 128, C = 64, NT = 4, NB = 2, ROWS = 32, NDT = 2, KSC = 2, Cp = 64;
  static constexpr int NS = D / 32;              // 32-wide d_k steps
  static constexpr int EZ = DTZ == 0 ? 4 : 2;    // bytes per z element
  static constexpr int ZL = ROWS * EZ / 16;      // 16-byte pieces per token row of z
  static constexpr int ZK = (16 * ZL + 63) / 64; // pieces per lane per tile
  static constexpr int kThreads = 512;


  // x as stored (raw input bits: fp32 or bf16), for V computed in the pass.
  using XE = typename std::conditional<DTZ == 0, uint32_t, uint16_t>::type;
  static constexpr int XR = C + 3;                        // tile rows: tokens -3 .. C-1 of a chunk
  static constexpr int XPR = ROWS * sizeof(XE) / 16;      // 16-byte pieces per tile row
  static constexpr int XPIECES = XR * XPR;
  static constexpr int XK = (XPIECES + 255) / 256;        // pieces per output-wave lane

  struct Smem {
    u16x8 Sh[NS][NB][64], Sl[NS][NB][64];  // state as split B operands, one d_k step each
    // K of the chunk, token-major as the chain waves hold it (d_k in the
    // permuted K order), hi and lo, 16-byte pieces swizzled per token (see
    // kq_piece).  The state update reads K^T from it with transposing loads.
    alignas(16) uint16_t KQ[2][C][D];
    // R, U and DU tiles, split, as B operands: entry [kk][n][lane] holds the
    // hi (or lo) halves of token tiles 2kk (first 8 bytes) and 2kk + 1.
    u16x8 Rh[NT / 2][NB][64], Rl[NT / 2][NB][64];
    u16x8 Uh[NT / 2][NB][64], Ul[NT / 2][NB][64];
    u16x8 DUh[NT / 2][NB][64], DUl[NT / 2][NB][64];
    uint4 z[NT][16 * ZL];                  // per output wave: one token tile of z
    // x of the block's 32 v channels for a chunk and the three tokens before
    // it, double-buffered by chunk parity (staged by the output waves).
    alignas(16) XE XT[2][XR][ROWS];
  };

  // Gate factors of the owned tile.  Lane (c, g) holds the factor of token
  // 4g + (c % 4); quad_bcast hands every lane the four of its own rows.
  struct Gates {
    float gam, bt, dl;
    float glast;  // gamma of the chunk's last token (same in every lane)
  };

  struct ChainOps {
    u16x8 kh[NS];                      // K of the owned tile, A operand per d_k step
    uint2 kl8[NS];                     // its low halves, e4m3
    Gates g;
    u16x8 tm[KSC];                     // (I+A)^{-1} rows of the owned tile
  };

  struct OutOps {
    u16x8 qh[NS];          // Q of the owned tile
    uint2 ql8[NS];         // its low halves, e4m3
    float gam;             // gamma of token 4g + (c % 4), as in Gates
    u16x8 ph[KSC];
    uint2 pl8[KSC];        // P's low halves, e4m3
    uint4 z[ZK];
  };

  struct Ctx {
    const char *ktok_hi, *ktok_lo, *qtok_hi, *qtok_lo;  // slice 0 of this key head
    size_t slice_bytes;                                  // T_pad * 32 * 2 (hi; lo: half)
    float k_lo_scale, q_lo_scale;                        // scales of the e4m3 low halves
    const char *xv;    // x at (b, token 0, the block's first v channel)
    const char *hv;    // conv history at (b, row 0, the block's first v channel)
    const void *w;     // conv weights at the block's first v channel
    size_t xrow;       // bytes per token row of x (and of the history)
    const uint16_t *Tm, *Ph;
    const uint8_t *Pl8;  // P's e4m3 low halves
    const float *gates;
    const void *z;
    void *y;
    int64_t T;
    int H_v, NC, m, lane, gq;
    uint32_t o_tok, o_mat, o_zy, o_gate;
  };

  static __device__ __forceinline__ int valid_of(const Ctx &x, int chunk) {
    const int64_t r = x.T - static_cast<int64_t>(chunk) * C;
    return static_cast<int>(r < C ? r : C);
  }

  static __device__ __forceinline__ Split4 split4(const f32x4 &v) {
    uint32_t h0, h1, l0, l1;
    split2(v[0], v[1], h0, l0);
    split2(v[2], v[3], h1, l1);
    return Split4{make_uint2(h0, h1), make_uint2(l0, l1)};
  }

  static __device__ __forceinline__ u16x8 pair(const u16x8 (&a)[NT / 2][NB][64], int kk, int n,
                                               int lane) {
    return a[kk][n][lane];
  }

  // Tile m's half of its K step's operands.
  static __device__ __forceinline__ void put(u16x8 (&h)[NT / 2][NB][64], u16x8 (&l)[NT / 2][NB][64],
                                             int m, int n, int lane, const Split4 &v) {
    reinterpret_cast<uint2 *>(&h[m / 2][n][lane])[m & 1] = v.hi;
    reinterpret_cast<uint2 *>(&l[m / 2][n][lane])[m & 1] = v.lo;
  }

  // Token-major rows of the owned tile, every d_k step (slice-major layout):
  // bf16 hi, and the e4m3 low halves (one byte per element) widened to bf16.
  // The low halves of the next chunk stay packed until it starts (lo8 holds
  // them), so only 8 bytes per lane and step are in flight for them.
  static __device__ __forceinline__ void load_tok(const char *hi, const char *lo, const Ctx &x,
                                                  int chunk, u16x8 (&h)[NS], uint2 (&l8)[NS]) {
    const size_t row = static_cast<size_t>(chunk) * C * 32 * 2;
    const __amdgpu_buffer_rsrc_t rh = buf_rsrc(hi + row, kAllBytes), rl = buf_rsrc(lo + row / 2, kAllBytes);
    const uint32_t sb = static_cast<uint32_t>(x.slice_bytes);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      h[s] = bld<u16x8>(rh, x.o_tok, s * sb);
      l8[s] = bld<uint2>(rl, x.o_tok / 2, s * sb / 2);
    }
  }

  static __device__ __forceinline__ void widen_lo(const uint2 (&l8)[NS], float scale,
                                                  u16x8 (&l)[NS]) {
#pragma unroll
    for (int s = 0; s < NS; ++s) l[s] = lo8_to_bf16x8(l8[s], scale);
  }

  // ---- V from x in the pass.  The output waves stage the x tile of chunk
  // c + 1 (tokens -3 .. C-1 relative to it, the block's 32 v channels) in
  // phase 2 of chunk c; the chain waves apply the width-4 conv and SiLU to it
  // in phase 3, beside the state update, with the same operations as the conv
  // pass (so V is the same to the bit), and carry it into chunk c + 1.
  static __device__ __forceinline__ float xval(XE r) {
    if constexpr (DTZ == 0)
      return __uint_as_float(r);
    else
      return bf16_bits_to_f32(r);
  }

  // Loads of the x tile of `chunk` (stored for chunks >= 1 only, whose rows
  // are all tokens >= 0); rows past the sequence end re-read its last row
  // (zeroed when stored), and token rows before 0 re-read row 0 (such a tile,
  // of the first chunk, is never stored: it comes from stage_first_xtile).
  static __device__ __forceinline__ void load_xtile(const Ctx &x, int chunk, int olane,
                                                    uint4 (&xr)[XK]) {
    const int64_t t0 = static_cast<int64_t>(chunk) * C - 3;
    if (t0 < 0) return;  // only a one-chunk sequence asks for it, and never stores it
    // Rows at or past the sequence end lie past the resource and read zero.
    const int64_t rows = x.T - t0 < XR ? x.T - t0 : XR;
    const __amdgpu_buffer_rsrc_t r =
        buf_rsrc(x.xv + static_cast<size_t>(t0) * x.xrow, static_cast<uint32_t>(rows * x.xrow));
#pragma unroll
    for (int k = 0; k < XK; ++k) {
      int piece = olane + 256 * k;
      piece = piece < XPIECES ? piece : XPIECES - 1;
      const int row = piece / XPR, part = piece % XPR;
      xr[k] = bld<uint4>(r, static_cast<uint32_t>(row * x.xrow + part * 16), 0);
    }
  }

  static __device__ __forceinline__ void store_xtile(const Ctx &x, Smem &sm, int chunk,
                                                     int olane, const uint4 (&xr)[XK]) {
#pragma unroll
    for (int k = 0; k < XK; ++k) {
      const int piece = olane + 256 * k;
      if (piece < XPIECES) {
        const int row = piece / XPR, part = piece % XPR;
        const int64_t tok = static_cast<int64_t>(chunk) * C - 3 + row;
        // A mask rather than a select of two vectors (which the compiler
        // lowers to a stack slot).
        const uint32_t keep = tok < x.T ? 0xffffffffu : 0u;
        const uint4 v = make_uint4(xr[k].x & keep, xr[k].y & keep, xr[k].z & keep, xr[k].w & keep);
        *reinterpret_cast<uint4 *>(&sm.XT[chunk & 1][row][part * 16 / sizeof(XE)]) = v;
      }
    }
  }

  // The first chunk's tile: its three leading rows come from the history.
  static __device__ __forceinline__ void stage_first_xtile(const Ctx &x, Smem &sm, int olane) {
    for (int piece = olane; piece < XPIECES; piece += 256) {
      const int row = piece / XPR, part = piece % XPR;
      const int tok = row - 3;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (tok < 0)
        v = ldb<uint4>(x.hv + static_cast<size_t>(3 + tok) * x.xrow, part * 16);
      else if (tok < x.T)
        v = ldb<uint4>(x.xv + static_cast<size_t>(tok) * x.xrow, part * 16);
      *reinterpret_cast<uint4 *>(&sm.XT[0][row][part * 16 / sizeof(XE)]) = v;
    }
  }

  // V of the owned tile for both of the lane's channels (2c and 2c + 1: tile
  // columns n = 0, 1 hold the block's even and odd rows), D-register order:
  // tokens 16 m + 4 g + r, r = 0..3 (tile rows 16 m + 4 g + r .. + 3).
  static __device__ __forceinline__ void v_tile2(const Smem &sm, int buf, int m, int gq, int c,
                                                 const float (&w)[NB][4], float4 (&v)[NB]) {
    const int t0 = 16 * m + 4 * gq;
    float xs[NB][7];
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      if constexpr (DTZ == 0) {
        const uint2 p = *reinterpret_cast<const uint2 *>(&sm.XT[buf][t0 + i][2 * c]);
        xs[0][i] = __uint_as_float(p.x);
        xs[1][i] = __uint_as_float(p.y);
      } else {
        const uint32_t p = *reinterpret_cast<const uint32_t *>(&sm.XT[buf][t0 + i][2 * c]);
        xs[0][i] = __uint_as_float(p << 16);
        xs[1][i] = __uint_as_float(p & 0xffff0000u);
      }
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const float *q = xs[n];
      v[n].x = siluf_(conv4(w[n][0], w[n][1], w[n][2], w[n][3], q[0], q[1], q[2], q[3]));
      v[n].y = siluf_(conv4(w[n][0], w[n][1], w[n][2], w[n][3], q[1], q[2], q[3], q[4]));
      v[n].z = siluf_(conv4(w[n][0], w[n][1], w[n][2], w[n][3], q[2], q[3], q[4], q[5]));
      v[n].w = siluf_(conv4(w[n][0], w[n][1], w[n][2], w[n][3], q[3], q[4], q[5], q[6]));
    }
  }



  // Element offset in a token row of KQ of the 16-byte piece `piece` (0..15,
  // d_k step piece / 4, lane group piece % 4).  The XOR spreads the sixteen
  // tokens that one store or one transposing load touches over all banks.
  static __device__ __forceinline__ int kq_piece(int tok, int piece) {
    return 8 * (piece ^ (((tok >> 2) & 3) | ((tok & 3) << 2)));
  }

  // A operand K^T of the state update for d_k rows 32w + 16dt .. + 15 and
  // tokens 32kk .. 32kk + 31 (permuted K order).  ds_read_b64_tr_b16 hands
  // lane 4a + b of each 16-lane group element b of the 8 bytes that lanes
  // a, a + 4, a + 8, a + 12 of the group address; so lane (a + 4j) of group
  // g addresses d_k 32w + 16dt + 4a .. + 3 of token 32kk + 4g + j (then + 16),
  // and lane (c, g) receives d_k row c for tokens 4g + j (then 16 + 4g + j),
  // slots 8g .. 8g + 7.
  static __device__ __forceinline__ u16x8 kt_operand(const uint16_t (&kq)[C][D], int kk, int w,
                                                     int dt, int lane) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const int grp = lane >> 4, a = lane & 3, j = (lane >> 2) & 3;
    const int t0 = 32 * kk + 4 * grp + j, t1 = t0 + 16;
    const uint16_t *p0 = &kq[t0][kq_piece(t0, 4 * w + a) + 4 * dt];
    const uint16_t *p1 = &kq[t1][kq_piece(t1, 4 * w + a) + 4 * dt];
    const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s *)(p0));
    const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s *)(p1));
    const uint2 d0 = __builtin_bit_cast(uint2, r0), d1 = __builtin_bit_cast(uint2, r1);
    const u32x4 v = {d0.x, d0.y, d1.x, d1.y};
    return __builtin_bit_cast(u16x8, v);
  }

  // Lane r of each group of four lanes to all four (DPP quad_perm r,r,r,r).
  template <int R>
  static __device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), R * 0x55, 0xf, 0xf, false));
  }

  static __device__ __forceinline__ float4 quad4(float v) {
    return make_float4(quad_bcast<0>(v), quad_bcast<1>(v), quad_bcast<2>(v), quad_bcast<3>(v));
  }

  // One dword per lane: sixteen lanes share each group's four values, so
  // the loads return a quarter of what per-lane float4 loads would.
  static __device__ __forceinline__ Gates load_gates(const Ctx &x, int chunk) {
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(x.gates + static_cast<size_t>(chunk) * 4 * C, kAllBytes);
    const float4 v = bld<float4>(r, 4 * x.o_gate, 0);
    Gates o;
    o.gam = v.x;
    o.dl = v.y;
    o.bt = v.z;
    o.glast = v.w;
    return o;
  }

  // Rows of a chunk matrix (Tm or P) for the owned tile; K steps past the
  // diagonal re-read the last needed one (they are not used).
  static __device__ __forceinline__ void load_rows(const uint16_t *mat, const Ctx &x, int chunk,
                                                   u16x8 (&r)[KSC]) {
    const __amdgpu_buffer_rsrc_t rr = buf_rsrc(mat + static_cast<size_t>(chunk) * C * Cp, kAllBytes);
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      const int kk = ks <= x.m / 2 ? ks : x.m / 2;
      r[ks] = bld<u16x8>(rr, x.o_mat, 32 * kk * 2);
    }
  }

  // The same rows of a matrix of e4m3 bytes (P's low halves).
  static __device__ __forceinline__ void load_rows8(const uint8_t *mat, const Ctx &x, int chunk,
                                                    uint2 (&r)[KSC]) {
    const __amdgpu_buffer_rsrc_t rr = buf_rsrc(mat + static_cast<size_t>(chunk) * C * Cp, kAllBytes);
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      const int kk = ks <= x.m / 2 ? ks : x.m / 2;
      r[ks] = bld<uint2>(rr, x.o_mat / 2, 32 * kk);
    }
  }



  static __device__ __forceinline__ void load_z(const Ctx &x, int chunk, OutOps &o) {
    if constexpr (!out_gated(DTY)) return;  // no gate: z is not read
    const int n_valid = valid_of(x, chunk);
    const char *zb = static_cast<const char *>(x.z) + static_cast<size_t>(chunk) * C * x.H_v * D * EZ;
    const uint32_t tstride = x.H_v * D * EZ;
    // Rows past the sequence end lie past the resource and read zero.
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(zb, n_valid * tstride);
#pragma unroll
    for (int k = 0; k < ZK; ++k) {
      int idx = x.lane + 64 * k;
      idx = idx < 16 * ZL ? idx : 16 * ZL - 1;
      const int t = 16 * x.m + idx / ZL;
      o.z[k] = bld<uint4>(r, t * tstride + (idx % ZL) * 16, 0);
    }
  }

  static __device__ __forceinline__ void load_gam(const Ctx &x, int chunk, OutOps &o) {
    o.gam = bld<float>(buf_rsrc(x.gates + static_cast<size_t>(chunk) * 4 * C, kAllBytes), 4 * x.o_gate, 0);
  }



  static __device__ void chain(const Ctx &x, Smem &sm, float *Sh, int w) {
    const int lane = x.lane, m = x.m;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // State slice d_k = 32w..32w+31 of the block's rows, as S^T tiles.
    f32x4 st[NB][NDT];
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const float4 v = *reinterpret_cast<const float4 *>(Sh + n * D + 32 * w + 16 * dt + 4 * x.gq);
        st[n][dt] = f32x4{v.x, v.y, v.z, v.w};
      }
#pragma unroll
    for (int n = 0; n < NB; ++n) pack_split(st[n][0], st[n][1], sm.Sh[w][n][lane], sm.Sl[w][n][lane]);
    // Conv weights of the two v channels this lane turns into V.
    float wv[NB][4];
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int k = 0; k < 4; ++k) wv[n][k] = load_elem<DTZ>(x.w, (2 * (lane & 15) + n) * 4 + k);
    ChainOps o;
    float4 vc[NB];  // V of the current chunk, from the staged x tile
    o.g = load_gates(x, 0);
    asm volatile("" ::: "memory");
    load_tok(x.ktok_hi, x.ktok_lo, x, 0, o.kh, o.kl8);
    asm volatile("" ::: "memory");
    load_rows(x.Tm, x, 0, o.tm);
    asm volatile("" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) st[n][dt] *= o.g.glast;
    v_tile2(sm, 0, m, x.gq, lane & 15, wv, vc);
    // The owned token's row of the token-major K copy.
    const int t_own = 16 * m + (lane & 15);

    for (int chunk = 0; chunk < x.NC; ++chunk) {
      const int next = chunk + 1 < x.NC ? chunk + 1 : chunk;
      // The next chunk's gate factors are needed first (phase 1) and fetched
      // first, a whole chunk ahead, into registers of their own.
      const Gates gn = load_gates(x, next);
      asm volatile("" ::: "memory");
      // 1. KS over the full depth, then R of the owned tile.
      u16x8 kl[NS];
      widen_lo(o.kl8, x.k_lo_scale, kl);
      u16x8 bh[NS][NB], bl[NS][NB];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          bh[s][n] = sm.Sh[s][n][lane];
          bl[s][n] = sm.Sl[s][n][lane];
        }
      f32x4 ks[NB] = {zero, zero};
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int n = 0; n < NB; ++n) ks[n] = mfma_split3(o.kh[s], kl[s], bh[s][n], bl[s][n], ks[n]);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const float4 vv = vc[n];
        const float4 bt = quad4(o.g.bt), ga = quad4(o.g.gam);
        const f32x4 r = {bt.x * (vv.x - ga.x * ks[n][0]), bt.y * (vv.y - ga.y * ks[n][1]),
                         bt.z * (vv.z - ga.z * ks[n][2]), bt.w * (vv.w - ga.w * ks[n][3])};
        put(sm.Rh, sm.Rl, m, n, lane, split4(r));
      }
      __syncthreads();

      // 2. U = Tm R for the owned tile, and its decayed copy for the update.
      //    The R operands are read first, every K step whether this tile
      //    needs it or not, so that they go out together ahead of the LDS
      //    stores below instead of one round trip per step behind them.
      //    Then the owned K tile into the token-major copy, as held (read in
      //    phase 3; phase 1 already carries the state-operand reads), and the
      //    next chunk's K in flight.
      u16x8 rh[KSC][NB], rl[KSC][NB];
#pragma unroll
      for (int kk = 0; kk < KSC; ++kk)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          rh[kk][n] = pair(sm.Rh, kk, n, lane);
          rl[kk][n] = pair(sm.Rl, kk, n, lane);
        }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int off = kq_piece(t_own, 4 * s + x.gq);
        *reinterpret_cast<u16x8 *>(&sm.KQ[0][t_own][off]) = o.kh[s];
        *reinterpret_cast<u16x8 *>(&sm.KQ[1][t_own][off]) = kl[s];
      }
      load_tok(x.ktok_hi, x.ktok_lo, x, next, o.kh, o.kl8);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        f32x4 acc = zero;
#pragma unroll
        for (int kk = 0; kk < KSC; ++kk)
          if (kk <= m / 2) {
            acc = mfma_split2(o.tm[kk], rh[kk][n], rl[kk][n], acc);
          }
        // DU first: the split overwrites what it splits.
        const float4 dl = quad4(o.g.dl);
        const f32x4 du = {dl.x * acc[0], dl.y * acc[1], dl.z * acc[2], dl.w * acc[3]};
        put(sm.DUh, sm.DUl, m, n, lane, split4(du));
        put(sm.Uh, sm.Ul, m, n, lane, split4(acc));
      }
      load_rows(x.Tm, x, next, o.tm);
      __syncthreads();

      // 3. S^T <- gamma_last S^T + K^T DU over the owned d_k slice, and V of
      //    the next chunk from its x tile (staged in phase 2).
      v_tile2(sm, next & 1, m, x.gq, lane & 15, wv, vc);
      u16x8 th[KSC][NDT], tl[KSC][NDT];
#pragma unroll
      for (int kk = 0; kk < KSC; ++kk)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          th[kk][dt] = kt_operand(sm.KQ[0], kk, w, dt, lane);
          tl[kk][dt] = kt_operand(sm.KQ[1], kk, w, dt, lane);
        }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int kk = 0; kk < KSC; ++kk) {
          const u16x8 bh = pair(sm.DUh, kk, n, lane), bl = pair(sm.DUl, kk, n, lane);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) st[n][dt] = mfma_split3(th[kk][dt], tl[kk][dt], bh, bl, st[n][dt]);
        }
      }
      // The state decayed for the next chunk's update, then the split of
      // this state in place (it overwrites what it splits).  After the last
      // chunk the factor is 1 and sc is the final state.
      const float gl = chunk + 1 < x.NC ? gn.glast : 1.f;
      f32x4 sc[NB][NDT];
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) sc[n][dt] = st[n][dt] * gl;
#pragma unroll
      for (int n = 0; n < NB; ++n) pack_split(st[n][0], st[n][1], sm.Sh[w][n][lane], sm.Sl[w][n][lane]);
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) st[n][dt] = sc[n][dt];
      o.g = gn;
      __syncthreads();
    }
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<float4 *>(Sh + n * D + 32 * w + 16 * dt + 4 * x.gq) =
            make_float4(st[n][dt][0], st[n][dt][1], st[n][dt][2], st[n][dt][3]);
  }

  static __device__ void output(const Ctx &x, Smem &sm) {
    const int lane = x.lane, m = x.m, gq = x.gq, c = lane & 15;
    const int olane = 64 * m + lane;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    stage_first_xtile(x, sm, olane);
    uint4 xr[XK];  // x tile of the chunk after next, in flight
    load_xtile(x, x.NC > 1 ? 1 : 0, olane, xr);
    OutOps o;
    load_tok(x.qtok_hi, x.qtok_lo, x, 0, o.qh, o.ql8);
    asm volatile("" ::: "memory");
    load_z(x, 0, o);
    asm volatile("" ::: "memory");
    load_rows(x.Ph, x, 0, o.ph);
    load_rows8(x.Pl8, x, 0, o.pl8);
    load_gam(x, 0, o);
    asm volatile("" ::: "memory");
    __syncthreads();
    constexpr int ey = out_bytes(DTY);
    const uint32_t ystride = x.H_v * D * ey;

    // One chunk; `last` (a compile-time flag) marks the final chunk, the only
    // one whose tokens may end early.  Every other chunk stores all of its
    // outputs unconditionally and after its loads, which keeps the stores out
    // of branches: the wait counts then see them, and a wait for a load never
    // waits for a store issued after it.
    auto step = [&](int chunk, auto last) {
      constexpr bool kLast = decltype(last)::value;
      const int next = kLast ? chunk : chunk + 1;
      // 1. QS over the full depth.
      u16x8 ql[NS];
      widen_lo(o.ql8, x.q_lo_scale, ql);
      u16x8 bh[NS][NB], bl[NS][NB];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          bh[s][n] = sm.Sh[s][n][lane];
          bl[s][n] = sm.Sl[s][n][lane];
        }
      f32x4 qs[NB] = {zero, zero};
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int n = 0; n < NB; ++n) qs[n] = mfma_split3(o.qh[s], ql[s], bh[s][n], bl[s][n], qs[n]);
      if (!kLast) load_tok(x.qtok_hi, x.qtok_lo, x, next, o.qh, o.ql8);
      __syncthreads();

      // 2. Gate of the owned tile: z arrives token-major; the wave's LDS slot
      //    turns it into D-register order.  Only this wave touches the slot,
      //    and LDS keeps one wave's accesses in order.
      float sg[NB][4];
      if constexpr (!out_gated(DTY)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sg[0][r] = sg[1][r] = 1.0f;
      } else {
#pragma unroll
        for (int k = 0; k < ZK; ++k)
          if (lane + 64 * k < 16 * ZL) sm.z[m][lane + 64 * k] = o.z[k];
        asm volatile("" ::: "memory");
        const char *zt = reinterpret_cast<const char *>(sm.z[m]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int off = ((4 * gq + r) * ROWS + 2 * c) * EZ;  // channels 2c, 2c + 1
          float z0, z1;
          if constexpr (DTZ == 0) {
            const uint2 p = *reinterpret_cast<const uint2 *>(zt + off);
            z0 = __uint_as_float(p.x);
            z1 = __uint_as_float(p.y);
          } else {
            const uint32_t p = *reinterpret_cast<const uint32_t *>(zt + off);
            z0 = __uint_as_float(p << 16);
            z1 = __uint_as_float(p & 0xffff0000u);
          }
          sg[0][r] = sigmoidf_(z0);
          sg[1][r] = sigmoidf_(z1);
        }
        asm volatile("" ::: "memory");
      }
      if (!kLast) {
        load_z(x, next, o);
        // The next chunk's x tile, for the chain waves' phase 3; then the
        // one after it (the last chunk's tile stands in past the end).
        store_xtile(x, sm, next, olane, xr);
        load_xtile(x, next + 1 < x.NC ? next + 1 : next, olane, xr);
      }
      __syncthreads();

      // 3. O = gamma QS + P U, gated, stored.
      const __amdgpu_buffer_rsrc_t ry =
          buf_rsrc(static_cast<char *>(x.y) + static_cast<size_t>(chunk) * C * x.H_v * D * ey, kAllBytes);
      const uint32_t yoff = x.o_zy * ey + 16 * m * ystride;
      f32x4 out[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const float4 ga = quad4(o.gam);
        f32x4 acc = {ga.x * qs[n][0], ga.y * qs[n][1], ga.z * qs[n][2], ga.w * qs[n][3]};
#pragma unroll
        for (int kk = 0; kk < KSC; ++kk)
          if (kk <= m / 2) {
            const u16x8 uh = pair(sm.Uh, kk, n, lane), ul = pair(sm.Ul, kk, n, lane);
            acc = mfma_split3(o.ph[kk], lo8_to_bf16x8(o.pl8[kk], x.q_lo_scale), uh, ul, acc);
          }
#pragma unroll
        for (int r = 0; r < 4; ++r) out[n][r] = acc[r] * sg[n][r];
      }
      if (!kLast) {
        load_rows(x.Ph, x, next, o.ph);
        load_rows8(x.Pl8, x, next, o.pl8);
        load_gam(x, next, o);
      }
      const int n_valid = valid_of(x, chunk);
      // Channels 2c and 2c + 1 side by side: one store per token.  y is
      // written once and not read here again: nontemporal stores (cache
      // policy bit 1) keep it from evicting the operands the blocks share
      // from L2 (measured: about 4 us faster at T = 4096).
      constexpr int kYNt = 2;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * m + 4 * gq + r;
        if (!kLast || t < n_valid) {
          const uint32_t so = r * ystride;
          if constexpr (out_type(DTY) == 0) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 v = {__float_as_uint(out[0][r]), __float_as_uint(out[1][r])};
            __builtin_amdgcn_raw_buffer_store_b64(v, ry, yoff, so, kYNt);
          } else if constexpr (out_type(DTY) == 1) {
            const uint32_t v = static_cast<uint32_t>(f32_to_bf16_bits(out[0][r])) |
                               (static_cast<uint32_t>(f32_to_bf16_bits(out[1][r])) << 16);
            __builtin_amdgcn_raw_buffer_store_b32(v, ry, yoff, so, kYNt);
          } else {
            const uint32_t v = static_cast<uint32_t>(f32_to_f16_bits(out[0][r])) |
                               (static_cast<uint32_t>(f32_to_f16_bits(out[1][r])) << 16);
            __builtin_amdgcn_raw_buffer_store_b32(v, ry, yoff, so, kYNt);
          }
        }
      }
      __syncthreads();
    };
    // The first chunk runs ahead of the loop so that the loop is entered with
    // the same memory operations in flight as on its back edge (loads of
    // the next chunk, then this chunk's stores): the wait counts inside the
    // loop are then exact instead of also covering the previous stores.
    if (x.NC > 1) {
      step(0, std::false_type{});
      for (int chunk = 1; chunk + 1 < x.NC; ++chunk) step(chunk, std::false_type{});
    }
    step(x.NC - 1, std::true_type{});
    // Conv history of the block's v channels after the sequence: the last
    // three rows of concat(history, x), still in the last chunk's tile.  This
    // block alone reads and writes these channels' history.
    if (m == 0 && lane < ROWS) {
      const int last = x.NC - 1;
      const int row0 = static_cast<int>(x.T - static_cast<int64_t>(last) * C);
#pragma unroll
      for (int r = 0; r < 3; ++r)
        *reinterpret_cast<XE *>(const_cast<char *>(x.hv) + r * x.xrow + lane * sizeof(XE)) =
            sm.XT[last & 1][row0 + r][lane];
    }
  }
};

template <int DTZ, int DTY>
__global__ __launch_bounds__(512) void state_kernel_ws(Geom g, PrefillWs L,
                                                       const void *__restrict__ z,
                                                       float *__restrict__ S,
                                                       void *__restrict__ y,
                                                       const char *__restrict__ ws,
                                                       const void *__restrict__ xin,
                                                       const void *__restrict__ conv_w,
                                                       void *__restrict__ hist) {
  using K = StateKernelWS<DTZ, DTY>;
  constexpr int D = K::D, C = K::C, Cp = K::Cp, ROWS = K::ROWS;
  __shared__ typename K::Smem sm;

  const int RB = D / ROWS;
  const int lid = xcd_remap(blockIdx.x, g.B * g.H_v * RB);
  const int rb = lid % RB;
  const int h = (lid / RB) % g.H_v;
  const int b = lid / (RB * g.H_v);
  const int kh = h / g.G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool is_chain = wave < 4;
  const int c = lane & 15, gq = lane >> 4;

  typename K::Ctx x;
  const size_t slice0 = (static_cast<size_t>(b) * g.H_k + kh) * (D / 32) * L.T_pad * 32 * 2;
  x.ktok_hi = ws + L.k_hi + slice0;
  x.ktok_lo = ws + L.k_lo + slice0 / 2;
  x.qtok_hi = ws + L.q_hi + slice0;
  x.qtok_lo = ws + L.q_lo + slice0 / 2;
  x.slice_bytes = static_cast<size_t>(L.T_pad) * 32 * 2;
  x.k_lo_scale = L.k_lo_scale;
  x.q_lo_scale = L.q_lo_scale;
  const int v_ch0 = 2 * g.H_k * D + h * D + ROWS * rb;  // first conv channel of the block's rows
  x.xrow = static_cast<size_t>(g.C_ch) * sizeof(typename K::XE);
  x.xv = static_cast<const char *>(xin) + (static_cast<size_t>(b) * L.T * g.C_ch + v_ch0) * sizeof(typename K::XE);
  x.hv = static_cast<const char *>(hist) + (static_cast<size_t>(b) * 3 * g.C_ch + v_ch0) * sizeof(typename K::XE);
  x.w = static_cast<const char *>(conv_w) + static_cast<size_t>(v_ch0) * 4 * sizeof(typename K::XE);
  const size_t mat = (static_cast<size_t>(b) * g.H_v + h) * L.NC * C * Cp;
  x.Tm = reinterpret_cast<const uint16_t *>(ws + L.Tm) + mat;
  x.Ph = reinterpret_cast<const uint16_t *>(ws + L.P_hi) + mat;
  x.Pl8 = reinterpret_cast<const uint8_t *>(ws + L.P_lo) + mat;
  x.gates = reinterpret_cast<const float *>(ws + L.gates) + (static_cast<size_t>(b) * g.H_v + h) * L.NC * 4 * C;
  const size_t zy = (static_cast<size_t>(b) * L.T * g.H_v + h) * D + ROWS * rb;
  x.z = static_cast<const char *>(z) + zy * K::EZ;
  x.y = static_cast<char *>(y) + zy * out_bytes(DTY);
  x.T = L.T;
  x.H_v = g.H_v;
  x.NC = L.NC;
  x.m = is_chain ? wave : wave - 4;
  x.lane = lane;
  x.gq = gq;
  x.o_tok = ((16 * x.m + c) * 32 + 8 * gq) * 2;
  x.o_mat = ((16 * x.m + c) * Cp + 8 * gq) * 2;
  x.o_zy = 4 * gq * g.H_v * D + 2 * c;  // tile columns n = 0, 1 are rows 2c, 2c + 1
  x.o_gate = (16 * x.m + 4 * gq + (lane & 3)) * 4;

  float *Sh = S + ((static_cast<size_t>(b) * g.H_v + h) * D + ROWS * rb + 2 * c) * D;
  if (is_chain)
    K::chain(x, sm, Sh, wave);
  else
    K::output(x, sm);
}

// ---------------------------------------------------------------- launchers

template <int D, int C>
static void launch_state_t(const Geom &g, const PrefillWs &L, const void *z, float *S, void *y,
                           const char *ws, const void *x, const void *cw, void *hist,
                           hipStream_t s, const KernelEvents *ev) {
  if constexpr (D == 128 && C == 64) {
    dim3 grid(g.B * g.H_v * (D / StateKernelWS<0, 0>::ROWS));
    dim3 block(StateKernelWS<0, 0>::kThreads);
#define GDN_WS(ZT, OC) launch_kernel(state_kernel_ws<ZT, OC>, grid, block, s, ev, g, L, z, S, y, ws, x, cw, hist)
    GDN_OUT_DISPATCH(g.in_dt, out_code(g.out_dt, z), GDN_WS);
#undef GDN_WS
    return;
  }
  (void)x;
  (void)cw;
  (void)hist;
  dim3 grid(g.B * g.H_v * (D / StateShape<D, C>::ROWS));
  dim3 block(StateShape<D, C>::NWV * 64);
#define GDN_ST(ZT, OC) launch_kernel(state_kernel<D, C, ZT, OC>, grid, block, s, ev, g, L, z, S, y, ws)
  GDN_OUT_DISPATCH(g.in_dt, out_code(g.out_dt, z), GDN_ST);
#undef GDN_ST
}

hipError_t launch_prefill_state(const Geom &g, const PrefillWs &L, const void *z, float *S,
                                void *y, const char *ws, const void *x, const void *conv_w,
                                void *hist, hipStream_t s, const KernelEvents *ev) {
#define GDN_STATE(Dv)                                                                   \
  switch (L.C) {                                                                        \
    case 16: launch_state_t<Dv, 16>(g, L, z, S, y, ws, x, conv_w, hist, s, ev); break;     \
    case 32: launch_state_t<Dv, 32>(g, L, z, S, y, ws, x, conv_w, hist, s, ev); break;     \
    case 64: launch_state_t<Dv, 64>(g, L, z, S, y, ws, x, conv_w, hist, s, ev); break;     \
    default: launch_state_t<Dv, 128>(g, L, z, S, y, ws, x, conv_w, hist, s, ev); break;    \
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
