// gdn_device.h -- device-side helpers shared by the GDN kernels (gfx950).
//
// MFMA operand layout of v_mfma_f32_16x16x32_bf16 on a 64-lane wave, with
// lane l, group g = l / 16 and column c = l % 16:
//   A (16 x 32, M x K): the lane supplies A[c][8g + i], i = 0..7
//   B (32 x 16, K x N): the lane supplies B[8g + i][c]
//   D (16 x 16):        the lane holds    D[4g + r][c], r = 0..3
// A 32-wide K step that spans two consecutive 16-row D tiles can therefore be
// fed straight from D registers if the K index is permuted: K slot 8g + i
// stands for index 4g + i (i < 4, first tile) or 16 + 4g + (i - 4) (second
// tile).  Every operand that is loaded from memory is stored in that permuted
// order, so no data ever moves between lanes to turn a result into the next
// product's operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A 16-byte store with the nontemporal hint: for workspace rows that the
// next pass streams back once, so they do not stay in the L2 in place of the
// operands that blocks share.
__device__ __forceinline__ void st_stream(uint4 *p, const uint4 &v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
}

constexpr int kWave = 64;

// ---------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// x - float(hi) for a pair and its bf16 rounding, one bf16 dot2 per element
// (x + (-1) hi_i + (-0) hi_j): the products are exact and the sum is rounded
// once, so this is the exact residual, as the two-step subtraction gives it.
// The zero weights are -0 so that neither weight pair is an inline constant:
// (-1, +0) was encoded as the inline constant -1.0, which the unit reads as
// the fp32 bits of -1.0, i.e. the pair (+0, -1).
__device__ __forceinline__ f32x2 residual2(f32x2 v, bf16x2 h) {
  const bf16x2 m0 = {static_cast<__bf16>(-1.0f), static_cast<__bf16>(-0.0f)};
  const bf16x2 m1 = {static_cast<__bf16>(-0.0f), static_cast<__bf16>(-1.0f)};
  const f32x2 r = {__builtin_amdgcn_fdot2_f32_bf16(h, m0, v[0], false),
                   __builtin_amdgcn_fdot2_f32_bf16(h, m1, v[1], false)};
  return r;
}

// Split a pair into hi + lo, both bf16 (round to nearest even, on gfx950's
// packed convert): hi = bf16(x), lo = bf16(x - hi), so hi + lo carries 16
// significant bits of x.  Returns each pair packed low element first.
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
  const f32x2 v = {a, b};
  const bf16x2 h = __builtin_convertvector(v, bf16x2);
  const f32x2 r = residual2(v, h);
  const bf16x2 l = __builtin_convertvector(r, bf16x2);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// The same split with the low half narrowed to fp8 (OCP e4m3): lo8 =
// e4m3((x - hi) / scale), two bytes per pair, low element first.  With
// |x| <= 2^e and scale = 2^(e - 15), |x - hi| / scale <= 128 stays inside
// e4m3's range (448); hi + lo8 * scale carries about 13 significant bits.
__device__ __forceinline__ void split2_lo8(float a, float b, float scale, uint32_t &hi,
                                           uint16_t &lo8) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  const bf16x2 h = __builtin_convertvector(v, bf16x2);
  const f32x2 r = residual2(v, h);
  const s16x2 zero = {0, 0};
  const s16x2 c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(zero, r[0], r[1], scale, false);
  hi = __builtin_bit_cast(uint32_t, h);
  lo8 = static_cast<uint16_t>(__builtin_bit_cast(uint32_t, c));
}

// Eight fp8 low halves (as stored by split2_lo8) back to a bf16 operand:
// element i = e4m3 byte i * scale, exact in bf16.
__device__ __forceinline__ u16x8 lo8_to_bf16x8(uint2 q, float scale) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, scale, false);
  const bf2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, scale, true);
  const bf2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, scale, false);
  const bf2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, scale, true);
  const u32x4 v = {__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1),
                   __builtin_bit_cast(uint32_t, a2), __builtin_bit_cast(uint32_t, a3)};
  return __builtin_bit_cast(u16x8, v);
}

__device__ __forceinline__ void split_bf16(float x, uint16_t &hi, uint16_t &lo) {
  uint32_t h, l;
  split2(x, 0.f, h, l);
  hi = static_cast<uint16_t>(h);
  lo = static_cast<uint16_t>(l);
}

// float -> fp16 bits, round to nearest even (the hardware convert).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

template <int DT>  // 0 = fp32, 1 = bf16, 2 = fp16 (outputs only)
__device__ __forceinline__ float load_elem(const void *p, size_t i) {
  if constexpr (DT == 0)
    return static_cast<const float *>(p)[i];
  else if constexpr (DT == 1)
    return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
  else
    return static_cast<float>(static_cast<const _Float16 *>(p)[i]);
}

template <int DT>
__device__ __forceinline__ void store_elem(void *p, size_t i, float v) {
  if constexpr (DT == 0)
    static_cast<float *>(p)[i] = v;
  else if constexpr (DT == 1)
    static_cast<uint16_t *>(p)[i] = f32_to_bf16_bits(v);
  else
    static_cast<uint16_t *>(p)[i] = f32_to_f16_bits(v);
}

// Output codes of the kernels' DTY template parameter: the low two bits are
// the element type of y (0 fp32, 1 bf16, 2 fp16); bit 2 set means no gate
// (y = o, the readout before the sigmoid gate; z is not read).
__host__ __device__ constexpr int out_type(int code) { return code & 3; }
__host__ __device__ constexpr bool out_gated(int code) { return (code & 4) == 0; }
__host__ __device__ constexpr int out_bytes(int code) { return (code & 3) == 0 ? 4 : 2; }

// e^{-x} as the hardware base-2 exponential of -x log2(e): one v_exp_f32
// without the library's denormal range handling.  A result that underflows
// becomes 0 and one that overflows +inf, and both ends give the right limit
// below (1 / (1 + inf) = 0, 1 / (1 + 0) = 1).
__device__ __forceinline__ float exp_neg(float x) {
  return __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
}

// Hardware reciprocal (1 ulp) instead of an IEEE division sequence.
__device__ __forceinline__ float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + exp_neg(z)); }
__device__ __forceinline__ float siluf_(float x) { return x * __builtin_amdgcn_rcpf(1.0f + exp_neg(x)); }

// Causal width-4 conv of one channel: taps w0..w3 meet x[t-3]..x[t].  The
// accumulation order is fixed so that every kernel gets the same bits.
__device__ __forceinline__ float conv4(float w0, float w1, float w2, float w3, float x0,
                                       float x1, float x2, float x3) {
  float acc = w0 * x0;
  acc = __builtin_fmaf(w1, x1, acc);
  acc = __builtin_fmaf(w2, x2, acc);
  acc = __builtin_fmaf(w3, x3, acc);
  return acc;
}

// ---------------------------------------------------------------- head sums of squares

// DPP lane exchange within a row of 16 lanes (gfx9 control codes):
// row_mirror (0x140) pairs lanes l and 15 - l, row_half_mirror (0x141) pairs
// l and 7 - l in each group of 8, quad_perm (2,3,0,1) (0x4E) pairs l and l ^ 2,
// quad_perm (1,0,3,2) (0xB1) pairs l and l ^ 1.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// One exchange of the transpose-reduce: N per-token values become N / 2.  The
// lane whose BIT is set keeps the upper half of the tokens, its partner (which
// has BIT clear and the same bits above) the lower half; each adds what the
// other sends for the half it keeps.
template <int N, int CTRL, int BIT>
__device__ __forceinline__ void tr_step(float *v, int lane) {
  const bool up = (lane & BIT) != 0;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float keep = up ? v[i + N / 2] : v[i];
    const float send = up ? v[i] : v[i + N / 2];
    v[i] = keep + dpp_f<CTRL>(send);
  }
}

// Per-token factor sc / sqrt(sum of squares + eps) of one 128-channel head
// held by two waves (w = 0, 1: the wave's place in the head; red and bc hold
// the head's two rows), for 16 tokens: 8 + 4 + 2 + 1 exchanges leave lane l with
// token l / 4, and two more DPP additions (partners l ^ 2, then l ^ 1) finish
// the lane sums.  Every token's sum runs through the same pairing tree, so a
// token's factor does not depend on its place in the tile.
__device__ __forceinline__ void head_scale_128x16(float (&ss)[16], float eps, float sc,
                                                  float (*red)[16], float (*bc)[16], int w) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss[i]),
                                                    __float_as_uint(ss[i + 8]), false, false);
    ss[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(ss[i]),
                                                    __float_as_uint(ss[i + 4]), false, false);
    ss[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  tr_step<4, 0x140, 8>(ss, lane);
  tr_step<2, 0x141, 4>(ss, lane);
  float s = ss[0] + dpp_f<0x4E>(ss[0]);
  s += dpp_f<0xB1>(s);
  const int t = lane >> 2;
  if ((lane & 3) == 0) red[w][t] = s;
  __syncthreads();
  const float f = __builtin_amdgcn_rsqf(red[0][t] + red[1][t] + eps) * sc;
  if ((lane & 3) == 0) bc[w][t] = f;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 16; ++i) ss[i] = bc[w][i];
}

// ---------------------------------------------------------------- wave ops

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Inclusive prefix sum over the 64 lanes (Hillis-Steele; fixed order).
__device__ __forceinline__ float wave_incl_scan(float v) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    float o = __shfl_up(v, d, kWave);
    if (l >= d) v += o;
  }
  return v;
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4 mfma16x16x32(const u16x8 &a, const u16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Split-precision product: (a_hi + a_lo)(b_hi + b_lo) without the lo*lo term.
__device__ __forceinline__ f32x4 mfma_split3(const u16x8 &ah, const u16x8 &al,
                                             const u16x8 &bh, const u16x8 &bl, f32x4 c) {
  c = mfma16x16x32(al, bh, c);
  c = mfma16x16x32(ah, bl, c);
  c = mfma16x16x32(ah, bh, c);
  return c;
}

// a plain bf16, b split.
__device__ __forceinline__ f32x4 mfma_split2(const u16x8 &a, const u16x8 &bh,
                                             const u16x8 &bl, f32x4 c) {
  c = mfma16x16x32(a, bl, c);
  c = mfma16x16x32(a, bh, c);
  return c;
}

// Pack the D registers of two stacked 16-row tiles (t0: K indices 0..15, t1:
// 16..31) into a split B (or A) operand with the permuted K order.
__device__ __forceinline__ void pack_split(const f32x4 &t0, const f32x4 &t1, u16x8 &hi,
                                           u16x8 &lo) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  split2(t0[0], t0[1], h0, l0);
  split2(t0[2], t0[3], h1, l1);
  split2(t1[0], t1[1], h2, l2);
  split2(t1[2], t1[3], h3, l3);
  const u32x4 h = {h0, h1, h2, h3}, l = {l0, l1, l2, l3};
  hi = __builtin_bit_cast(u16x8, h);
  lo = __builtin_bit_cast(u16x8, l);
}

// Position of index j (0..31) of a K step in the permuted slot order.
__host__ __device__ __forceinline__ int kslot(int j) {
  const int tile = j >> 4, within = j & 15;
  return 8 * (within >> 2) + 4 * tile + (within & 3);
}

}  // namespace gdn
