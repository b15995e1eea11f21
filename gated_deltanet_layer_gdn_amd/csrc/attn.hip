// attn.hip -- the full-attention layer of the hybrid schedule: Qwen RoPE,
// a bf16 KV cache and causal grouped-query attention ("Implement the Qwen3.8
// Flash Next Rust and Metal text core", section Implementation: Qwen RoPE and
// an exact dense 24Q/2KV causal attention; its implementation comment: BF16
// KV storage; "Add a performance-parity Qwen3.8-27B Q4 and Q8 text backend
// on Metal", section Model and reference contract: three Gated DeltaNet
// layers to one full-attention layer).
//
// Readings: RoPE rotates the pairs (i, i + r/2), i < r/2, of the first r
// dimensions of each head by pos * base^(-2i/r); query head h reads KV head
// h / (H_q / H_kv); o = softmax(scale q k^T over keys at positions <= the
// query's) v.
//
// Launches per call:
//   kv_cache_kernel    (calls of more than one token; a one-token call does
//                      this inside attn_kernel) the new keys, rotated, and
//                      values into the cache, and
//                      the cos and sin of the RoPE angles of the new
//                      positions into the workspace (T x r/2 pairs; the angle
//                      formed in double and reduced mod 2 pi before the fp32
//                      sin/cos, so long positions keep their accuracy);
//   attn_kernel        flash-style causal attention; each lane rotates its
//                      query operand while loading it (the rotated queries
//                      never go to memory).  A block of 8 waves owns
//                      128 (token, head) rows of one KV head's query group
//                      and walks 64-position KV tiles staged in LDS (V
//                      transposed on the way in).  S^T = K Q^T on the MFMA,
//                      so that each lane holds one query row's scores for
//                      positions 4g + r of every 16-position tile: that is
//                      exactly the A operand of O = P V in the permuted K
//                      order (no data moves between lanes), and the row
//                      statistics of the online softmax take two cross-lane
//                      steps;
//   attn_combine_kernel  only when few row blocks exist (decode, short
//                      chunks after a long context): the KV range is split
//                      over several blocks per row block and the partial
//                      results are merged here.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

// The new keys, rotated, and the new values into the cache at positions
// pos0 .. pos0 + T - 1, and the RoPE table of those positions for the
// attention pass.  One thread per pair of dimensions of one (b, t, KV head):
// thread p < r/2 turns the pair (p, p + r/2) by the angle (pos0 + t) *
// base^(-2p/r), formed in double and reduced mod 2 pi before the fp32
// sincos (positions of 10^5 and more keep their accuracy), and the blocks of
// sequence 0, KV head 0 store its cos and sin as cs[t][p]; the other threads
// copy two dimensions past r.  Every thread copies two dimensions of v.
// cos and sin of the RoPE angle of pair p at position pos: pos * base^(-2p/r)
// formed in double and reduced mod 2 pi, then the fp32 sincos.  One function
// for every kernel that needs them, so the angles agree bit for bit.
__device__ __forceinline__ float2 rope_cs(float base, int rot, int p, int64_t pos) {
  const double inv = pow(static_cast<double>(base), -2.0 * p / rot);
  double ang = static_cast<double>(pos) * inv;
  ang -= kTwoPi * floor(ang / kTwoPi);
  float sn, c;
  sincosf(static_cast<float>(ang), &sn, &c);
  return make_float2(c, sn);
}

// One key's rotation and its cache row (bf16 in, bf16 out): thread p < r/2
// turns the pair (p, p + r/2) by cs = (cos, sin); the other threads (p < D/2)
// copy two dimensions past r; every thread p < D/2 copies dimensions 2p and
// 2p + 1 of v.  Explicit fused operations, so that every caller gets the
// same bits.
template <int D>
__device__ __forceinline__ void rope_cache_row(int p, int rot, float2 cs, const uint16_t *src,
                                               const uint16_t *vs, uint16_t *kdst, uint16_t *vdst) {
  const int half = rot / 2;
  if (p < half) {
    const float x0 = bf16_bits_to_f32(src[p]), x1 = bf16_bits_to_f32(src[p + half]);
    kdst[p] = f32_to_bf16_bits(__builtin_fmaf(x0, cs.x, -(x1 * cs.y)));
    kdst[p + half] = f32_to_bf16_bits(__builtin_fmaf(x1, cs.x, x0 * cs.y));
  } else {
    const int j = rot + 2 * (p - half);
    kdst[j] = src[j];
    kdst[j + 1] = src[j + 1];
  }
  vdst[2 * p] = vs[2 * p];
  vdst[2 * p + 1] = vs[2 * p + 1];
}

template <int D>
__global__ __launch_bounds__(D / 2) void kv_cache_kernel(AttnGeom a, int64_t T, int64_t pos0,
                                                         int64_t T_max, const uint16_t *k,
                                                         const uint16_t *v, float2 *cs,
                                                         uint16_t *kc, uint16_t *vc) {
  const int p = threadIdx.x;
  int64_t idx = blockIdx.x;  // (b * T + t) * H_kv + head
  const int head = static_cast<int>(idx % a.H_kv);
  idx /= a.H_kv;
  const int64_t t = idx % T;
  const int b = static_cast<int>(idx / T);
  const uint16_t *src = k + ((b * T + t) * a.H_kv + head) * D;
  const uint16_t *vs = v + ((b * T + t) * a.H_kv + head) * D;
  const int64_t crow = ((b * T_max + pos0 + t) * a.H_kv + head) * D;
  const int half = a.rot / 2;
  float2 c = make_float2(1.f, 0.f);
  if (p < half) {
    c = rope_cs(a.base, a.rot, p, pos0 + t);
    if (b == 0 && head == 0) cs[t * half + p] = c;
  }
  rope_cache_row<D>(p, a.rot, c, src, vs, kc + crow, vc + crow);
}

// Geometry of the attention pass, fixed on the host per call.
struct AttnArgs {
  AttnGeom a;
  int64_t T, pos0, T_max;
  int G;             // query heads per KV head
  int n_fb;          // row blocks per (sequence, KV head)
  int64_t rows_pad;  // n_fb * rows per block
  int n_split, tps;  // KV splits and KV tiles per split (1, all: no split)
  const uint16_t *q, *kc, *vc;  // q as given (RoPE applied here, on load)
  const float2 *cs;             // RoPE cos / sin of the new positions [T][r/2]
  // T = 1 with the cache write fused in: the new key and value [B][1][H_kv][D]
  // and the cache again, writable.
  const uint16_t *k_new, *v_new;
  uint16_t *kc_w, *vc_w;
  void *o;
  float *part_o, *part_ml;  // partial results when n_split > 1
};

template <int D, int NW>
struct AttnCfg {
  static constexpr int NT = 64 * NW;            // threads
  static constexpr int R = 16 * NW;             // query rows per block (16 per wave)
  static constexpr int NS = D / 32;             // 32-wide dim steps of S^T
  static constexpr int NJ = D / 16;             // 16-wide dim tiles of O
  static constexpr int KPAD = D + 8;            // LDS row of the K tile (bank spread)
  static constexpr int VPAD = 64 + 8;           // LDS row of the V^T tile: 36 dwords, so
                                                // rows 8 apart fall 32 banks apart
  static constexpr int KP = 64 * (D / 8) / NT;  // 16-byte K pieces per thread
  static constexpr int VUNITS = 16 * (D / 8);   // V units: 4 tokens x 8 dims
  static constexpr int VU = (VUNITS + NT - 1) / NT;
  static_assert(KP >= 1 && 64 * (D / 8) % NT == 0, "K tile split");
  struct Smem {
    uint16_t K[64][KPAD];
    uint16_t V[D][VPAD];  // V^T, tokens in the MFMA slot order of each 32-block
  };
};

// Flash-style causal attention over (token, head) rows.  Block rows are R
// consecutive entries f of the flattened [T][G] index of one (sequence, KV
// head): row f is token f / G of query head kvh * G + f % G, so the G heads
// that read one KV head share every staged K/V tile (grouped-query reuse).
// The K/V tiles of 64 positions are loaded into registers one tile ahead
// (global latency hidden behind the current tile's products) and stored to
// LDS, V transposed on the way.  With n_split > 1 a block covers only the KV
// tiles [s tps, (s + 1) tps) and writes its unnormalised output with its row
// maximum and sum; attn_combine_kernel merges the splits.  FUSE (one new
// token, T = 1): the block forms the RoPE table of position pos0 itself, and
// the block of the last KV split of each (sequence, KV head) writes the new
// key, rotated, and value into cache row pos0 before it reads the cache,
// in place of kv_cache_kernel (one launch less per decode step).
template <int D, int NW, int OC, bool SPLIT, bool FUSE>
__global__ __launch_bounds__(64 * NW) void attn_kernel(AttnArgs p) {
  using C = AttnCfg<D, NW>;
  constexpr int NS = C::NS, NJ = C::NJ, R = C::R, NT = C::NT;
  __shared__ typename C::Smem sm;
  __shared__ __attribute__((aligned(16))) float2 cs_sm[FUSE ? D / 2 : 2];
  const AttnGeom &a = p.a;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  int64_t id = blockIdx.x;
  const int s_idx = SPLIT ? static_cast<int>(id % p.n_split) : 0;
  if (SPLIT) id /= p.n_split;
  const int n_bk = a.B * a.H_kv;
  const int bk = static_cast<int>(id % n_bk);
  const int fb = p.n_fb - 1 - static_cast<int>(id / n_bk);  // late rows (most keys) first
  const int b = bk / a.H_kv, kvh = bk % a.H_kv;
  const int64_t TG = p.T * p.G;
  const int64_t f0 = static_cast<int64_t>(fb) * R;
  const int64_t L = p.pos0 + p.T;

  // This lane's query row (the column c of S^T) and its operand of K Q^T.
  const int64_t f = f0 + 16 * w + c;
  const int64_t fc = f < TG ? f : TG - 1;
  const bool active = f0 + 16 * w < TG;  // a wave of padding rows only stages tiles
  const int64_t tq = fc / p.G;
  const int hq = kvh * p.G + static_cast<int>(fc % p.G);
  const int64_t qpos = p.pos0 + tq;
  if constexpr (FUSE) {
    const int half = a.rot / 2;
    if (tid < half) cs_sm[tid] = rope_cs(a.base, a.rot, tid, p.pos0);
    __syncthreads();
    if (s_idx == p.n_split - 1 && tid < D / 2) {
      const int64_t nrow = (static_cast<int64_t>(b) * a.H_kv + kvh) * D;
      const int64_t crow = ((static_cast<int64_t>(b) * p.T_max + p.pos0) * a.H_kv + kvh) * D;
      rope_cache_row<D>(tid, a.rot, tid < half ? cs_sm[tid] : make_float2(1.f, 0.f), p.k_new + nrow,
                        p.v_new + nrow, p.kc_w + crow, p.vc_w + crow);
    }
    __syncthreads();  // the new cache row written before any wave reads the cache
  }
  u16x8 qb[NS];
  {
    // The lane's eight dimensions 32 s + 8 g .. + 7 of each K step, turned by
    // RoPE in fp32 (dimension d < r/2 pairs with d + r/2) and rounded to bf16;
    // r is a multiple of 16, so an 8-dimension block lies wholly below r/2,
    // in [r/2, r) or past r.
    const uint16_t *qp = p.q + ((b * p.T + tq) * a.H_q + hq) * D;
    const int half = a.rot / 2;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int d0 = 32 * s + 8 * g;
      qb[s] = *reinterpret_cast<const u16x8 *>(qp + d0);
      if (d0 < a.rot) {
        const bool lo = d0 < half;
        const int i0 = lo ? d0 : d0 - half;
        const u16x8 pq = *reinterpret_cast<const u16x8 *>(qp + (lo ? d0 + half : d0 - half));
        const float4 *cp = reinterpret_cast<const float4 *>(p.cs + tq * half + i0);
        u16x8 r;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          // (cos, sin) of pairs i0 + 2 e2, i0 + 2 e2 + 1
          const float4 c2 = FUSE ? reinterpret_cast<const float4 *>(cs_sm)[i0 / 2 + e2] : cp[e2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int e = 2 * e2 + h2;
            const float cs_ = h2 ? c2.z : c2.x, sn_ = h2 ? c2.w : c2.y;
            const float x = bf16_bits_to_f32(qb[s][e]), y = bf16_bits_to_f32(pq[e]);
            r[e] = f32_to_bf16_bits(lo ? x * cs_ - y * sn_ : x * cs_ + y * sn_);
          }
        }
        qb[s] = r;
      }
    }
  }
  const float sl2 = a.scale * 1.4426950408889634f;  // scores in log2 units
  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;

  // KV tiles up to the block's last query position, this split's share.
  const int64_t f_last = f0 + R - 1 < TG ? f0 + R - 1 : TG - 1;
  const int64_t q_first = p.pos0 + f0 / p.G;  // the block's first query position
  const int n_kv = static_cast<int>((p.pos0 + f_last / p.G) / 64 + 1);
  const int kt0 = s_idx * p.tps;
  const int kt1 = kt0 + p.tps < n_kv ? kt0 + p.tps : n_kv;
  const int64_t row_stride = static_cast<int64_t>(a.H_kv) * D;
  const uint16_t *kbase = p.kc + static_cast<int64_t>(b) * p.T_max * row_stride + kvh * D;
  const uint16_t *vbase = p.vc + static_cast<int64_t>(b) * p.T_max * row_stride + kvh * D;

  u32x4 kreg[C::KP], vreg[C::VU][4];
  auto load_tile = [&](int kt) {
    const int64_t t0 = static_cast<int64_t>(kt) * 64;
#pragma unroll
    for (int i = 0; i < C::KP; ++i) {
      const int piece = tid + NT * i;
      const int row = piece / (D / 8), part = piece % (D / 8);
      kreg[i] = u32x4{0u, 0u, 0u, 0u};
      if (t0 + row < L)
        kreg[i] = *reinterpret_cast<const u32x4 *>(kbase + (t0 + row) * row_stride + part * 8);
    }
#pragma unroll
    for (int i = 0; i < C::VU; ++i) {
      const int unit = tid + NT * i;
      const int tg = unit % 16, dg = unit / 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t tok = t0 + 4 * tg + j;
        vreg[i][j] = u32x4{0u, 0u, 0u, 0u};
        if (unit < C::VUNITS && tok < L)
          vreg[i][j] = *reinterpret_cast<const u32x4 *>(vbase + tok * row_stride + dg * 8);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < C::KP; ++i) {
      const int piece = tid + NT * i;
      const int row = piece / (D / 8), part = piece % (D / 8);
      *reinterpret_cast<u32x4 *>(&sm.K[row][part * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::VU; ++i) {
      const int unit = tid + NT * i;
      if (unit >= C::VUNITS) continue;
      const int tg = unit % 16, dg = unit / 16;
      const int j0 = 4 * tg;  // four tokens in four consecutive slots
      const int slot = (j0 & 32) + kslot(j0 & 31);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        uint32_t t[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = (vreg[i][j][e >> 1] >> sh) & 0xffffu;
        const uint2 pr = make_uint2(t[0] | (t[1] << 16), t[2] | (t[3] << 16));
        *reinterpret_cast<uint2 *>(&sm.V[8 * dg + e][slot]) = pr;
      }
    }
  };

  if (kt0 < kt1) load_tile(kt0);
  for (int kt = kt0; kt < kt1; ++kt) {
    store_tile();
    __syncthreads();
    if (kt + 1 < kt1) load_tile(kt + 1);
    if (!active) {
      __syncthreads();
      continue;
    }
    const int64_t t0 = static_cast<int64_t>(kt) * 64;
    // S^T = K Q^T: four 16-token tiles; lane (g, c) holds tokens 16 m + 4 g + r of row c.
    f32x4 st[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      st[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u16x8 ka = *reinterpret_cast<const u16x8 *>(&sm.K[16 * m + c][32 * s + 8 * g]);
        st[m] = mfma16x16x32(ka, qb[s], st[m]);
      }
    }
    // Online softmax of row c (log2 units, causal mask).  A row with no
    // visible key yet (possible only in a split) keeps p = 0 and alpha = 0.
    // Tiles wholly at or before the block's first query position need no
    // mask (the test is the same for the whole block).
    float mx = -INFINITY;
    if (t0 + 63 <= q_first) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          st[m][r] *= sl2;
          mx = fmaxf(mx, st[m][r]);
        }
    } else {
      const int dk = static_cast<int>(qpos - t0) - 4 * g;  // key 16 m + r visible iff <= dk
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sv = 16 * m + r <= dk ? st[m][r] * sl2 : -INFINITY;
          st[m][r] = sv;
          mx = fmaxf(mx, sv);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    // Lazy rescaling: a row keeps its reference maximum until the tile's
    // exceeds it by more than 8 (log2 units), so its weights stay below 2^8
    // and most tiles skip the rescale of O; numerator and denominator use
    // the same reference, so the normalised result is unchanged.
    const bool grow = mx > m_run + 8.f;
    const float m_new = grow ? mx : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    if (__ballot(grow)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);  // 1 for rows that keep it
      l_lane *= alpha;
      // O's rows are 4 g + r, whose factors sit in lanes c = 4 g + r.
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * g + r, kWave);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] *= al[r];
    }
    m_run = m_new;
    // This lane's share of the row sum (reduced over the row's four lanes once, at the end).
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = __builtin_amdgcn_exp2f(st[m][r] - m_use);
        st[m][r] = pv;
        l_lane += pv;
      }
    // O += P V: P (bf16, the packed round-to-nearest-even convert) as the A
    // operand straight from the score registers.
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      uint32_t pw[4];
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const f32x2 a0 = {st[2 * s2][r], st[2 * s2][r + 1]};
        const f32x2 a1 = {st[2 * s2 + 1][r], st[2 * s2 + 1][r + 1]};
        pw[r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(a0, bf16x2));
        pw[2 + r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(a1, bf16x2));
      }
      const u32x4 pa = {pw[0], pw[1], pw[2], pw[3]};
      const u16x8 pop = __builtin_bit_cast(u16x8, pa);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u16x8 vb = *reinterpret_cast<const u16x8 *>(&sm.V[16 * j + c][32 * s2 + 8 * g]);
        acc[j] = mfma16x16x32(pop, vb, acc[j]);
      }
    }
    __syncthreads();
  }
  float l_run = l_lane + __shfl_xor(l_lane, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  if (SPLIT) {
    // Unnormalised rows 4 g + r with the row maximum (log2 units) and sum.
    const int64_t rows_total = static_cast<int64_t>(n_bk) * p.rows_pad;
    const int64_t base = static_cast<int64_t>(s_idx) * rows_total + bk * p.rows_pad + f0 + 16 * w;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (f0 + 16 * w + 4 * g + r >= TG) continue;
      float *po = p.part_o + (base + 4 * g + r) * D + c;
#pragma unroll
      for (int j = 0; j < NJ; ++j) po[16 * j] = acc[j][r];
    }
    if (g == 0 && f < TG) {
      p.part_ml[2 * (base + c)] = m_run;
      p.part_ml[2 * (base + c) + 1] = l_run;
    }
    return;
  }
  // Normalise rows 4 g + r and store.
  float inv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) inv[r] = 1.0f / __shfl(l_run, 4 * g + r, kWave);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t fr = f0 + 16 * w + 4 * g + r;
    if (fr >= TG) continue;
    const int64_t tr = fr / p.G;
    const int hr = kvh * p.G + static_cast<int>(fr % p.G);
    const size_t ob = ((static_cast<size_t>(b) * p.T + tr) * a.H_q + hr) * D + c;
#pragma unroll
    for (int j = 0; j < NJ; ++j) store_elem<out_type(OC)>(p.o, ob + 16 * j, acc[j][r] * inv[r]);
  }
}

constexpr int kAttnMaxSplit = 512;

// Merge the KV splits of each row: weights 2^(m_s - max m), normalised by the
// weighted sum of the splits' l_s.  One block per (sequence, token, query
// head), one thread per output dimension; the splits' maxima and sums are
// read once into LDS.
template <int D, int OC>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnArgs p) {
  __shared__ float msh[kAttnMaxSplit], lsh[kAttnMaxSplit];
  const int tid = threadIdx.x;
  int64_t id = blockIdx.x;  // (b * T + t) * H_q + h
  const int h = static_cast<int>(id % p.a.H_q);
  id /= p.a.H_q;
  const int64_t t = id % p.T;
  const int b = static_cast<int>(id / p.T);
  const int kvh = h / p.G;
  const int64_t rows_total = static_cast<int64_t>(p.a.B) * p.a.H_kv * p.rows_pad;
  const int64_t prow = (static_cast<int64_t>(b) * p.a.H_kv + kvh) * p.rows_pad + t * p.G + h % p.G;
  for (int s = tid; s < p.n_split; s += D) {
    msh[s] = p.part_ml[2 * (s * rows_total + prow)];
    lsh[s] = p.part_ml[2 * (s * rows_total + prow) + 1];
  }
  __syncthreads();
  float mmax = -INFINITY;
  for (int s = 0; s < p.n_split; ++s) mmax = fmaxf(mmax, msh[s]);
  float l = 0.f, o = 0.f;
#pragma unroll 8
  for (int s = 0; s < p.n_split; ++s) {
    const float ms = msh[s];
    const float wgt = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - mmax);
    l += wgt * lsh[s];
    o += wgt * p.part_o[(s * rows_total + prow) * D + tid];
  }
  const size_t ob = ((static_cast<size_t>(b) * p.T + t) * p.a.H_q + h) * D + tid;
  store_elem<out_type(OC)>(p.o, ob, o / l);
}

constexpr int kAttnWaves = 8;
constexpr int kAttnRows = 16 * kAttnWaves;
constexpr int kAttnTargetBlocks = 256;  // blocks to aim for when the KV range is split
constexpr int kAttnSplitBelow = 64;      // split only below this many row blocks: above it
                                         // the partial results cost more traffic than the
                                         // idle compute units

// Row blocks, KV splits and workspace pieces of one call (host).
struct AttnPlan {
  int G, n_fb, n_split, tps;
  int64_t rows_pad;
  size_t cs_bytes, part_o_bytes, part_ml_bytes;
};

AttnPlan attn_plan(const AttnGeom &a, int64_t T, int64_t pos0) {
  AttnPlan pl{};
  pl.G = a.H_q / a.H_kv;
  pl.n_fb = static_cast<int>((T * pl.G + kAttnRows - 1) / kAttnRows);
  pl.rows_pad = static_cast<int64_t>(pl.n_fb) * kAttnRows;
  const int64_t blocks = static_cast<int64_t>(pl.n_fb) * a.B * a.H_kv;
  const int n_kv = static_cast<int>((pos0 + T - 1) / 64 + 1);
  int split = 1;
  if (blocks < kAttnSplitBelow) {
    split = static_cast<int>((kAttnTargetBlocks + blocks - 1) / blocks);
    const int most = (n_kv + 1) / 2;  // two tiles a split at least: the second tile's
    split = split < most ? split : most;  // load overlaps the first one's products
    split = split < kAttnMaxSplit ? split : kAttnMaxSplit;
    split = split > 1 ? split : 1;
  }
  pl.tps = (n_kv + split - 1) / split;
  pl.n_split = (n_kv + pl.tps - 1) / pl.tps;
  // the RoPE table, at least 256 bytes: a valid call never reports a zero
  // workspace size (zero means invalid arguments), even without rotation
  // and without KV splits
  pl.cs_bytes = (static_cast<size_t>(T) * (a.rot / 2) * 8 + 255) / 256 * 256;
  if (pl.cs_bytes < 256) pl.cs_bytes = 256;
  const size_t rows = static_cast<size_t>(pl.n_split) * a.B * a.H_kv * pl.rows_pad;
  pl.part_o_bytes = pl.n_split > 1 ? (rows * a.D * 4 + 255) / 256 * 256 : 0;
  pl.part_ml_bytes = pl.n_split > 1 ? (rows * 2 * 4 + 255) / 256 * 256 : 0;
  return pl;
}

template <int D, int OC, bool FUSE>
void launch_attn_core(const AttnArgs &p, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(p.n_fb) * p.a.B * p.a.H_kv *
                                                p.n_split);
  if (p.n_split == 1) {
    hipLaunchKernelGGL((attn_kernel<D, kAttnWaves, OC, false, FUSE>), dim3(blocks),
                       dim3(64 * kAttnWaves), 0, s, p);
    return;
  }
  hipLaunchKernelGGL((attn_kernel<D, kAttnWaves, OC, true, FUSE>), dim3(blocks),
                     dim3(64 * kAttnWaves), 0, s, p);
  const int64_t rows = static_cast<int64_t>(p.a.B) * p.T * p.a.H_q;
  hipLaunchKernelGGL((attn_combine_kernel<D, OC>), dim3(static_cast<unsigned>(rows)), dim3(D), 0,
                     s, p);
}

}  // namespace

size_t attn_ws_bytes(const AttnGeom &a, int64_t T, int64_t pos0) {
  const AttnPlan pl = attn_plan(a, T, pos0);
  return pl.cs_bytes + pl.part_o_bytes + pl.part_ml_bytes;
}

hipError_t launch_attn_prefill(const AttnGeom &a, int64_t T, int64_t pos0, const void *q,
                               const void *k, const void *v, void *kc, void *vc, int64_t T_max,
                               void *o, void *ws, hipStream_t s) {
  const AttnPlan pl = attn_plan(a, T, pos0);
  char *wsb = static_cast<char *>(ws);
  AttnArgs p{};
  p.a = a;
  p.T = T;
  p.pos0 = pos0;
  p.T_max = T_max;
  p.G = pl.G;
  p.n_fb = pl.n_fb;
  p.rows_pad = pl.rows_pad;
  p.n_split = pl.n_split;
  p.tps = pl.tps;
  p.q = static_cast<const uint16_t *>(q);
  p.kc = static_cast<const uint16_t *>(kc);
  p.vc = static_cast<const uint16_t *>(vc);
  p.cs = reinterpret_cast<const float2 *>(wsb);
  p.o = o;
  p.part_o = reinterpret_cast<float *>(wsb + pl.cs_bytes);
  p.part_ml = reinterpret_cast<float *>(wsb + pl.cs_bytes + pl.part_o_bytes);
  const auto *k16 = static_cast<const uint16_t *>(k);
  const auto *v16 = static_cast<const uint16_t *>(v);
  auto *kc16 = static_cast<uint16_t *>(kc);
  auto *vc16 = static_cast<uint16_t *>(vc);
  float2 *cs = reinterpret_cast<float2 *>(wsb);
  const dim3 g1(static_cast<unsigned>(static_cast<int64_t>(a.B) * T * a.H_kv));
  // One new token (a decode step): the attention pass writes the cache row
  // itself.  Since T = 1 gives one row block per (sequence, KV head), exactly
  // one block (that of the last KV split) writes each row.
  const bool fuse = T == 1 && pl.n_fb == 1;
  p.k_new = k16;
  p.v_new = v16;
  p.kc_w = kc16;
  p.vc_w = vc16;
  if (a.D == 256) {
    if (fuse) {
      if (a.out_dt == 0)
        launch_attn_core<256, 0, true>(p, s);
      else
        launch_attn_core<256, 1, true>(p, s);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((kv_cache_kernel<256>), g1, dim3(128), 0, s, a, T, pos0, T_max, k16, v16, cs,
                       kc16, vc16);
    if (a.out_dt == 0)
      launch_attn_core<256, 0, false>(p, s);
    else
      launch_attn_core<256, 1, false>(p, s);
  } else {
    if (fuse) {
      if (a.out_dt == 0)
        launch_attn_core<128, 0, true>(p, s);
      else
        launch_attn_core<128, 1, true>(p, s);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((kv_cache_kernel<128>), g1, dim3(64), 0, s, a, T, pos0, T_max, k16, v16, cs,
                       kc16, vc16);
    if (a.out_dt == 0)
      launch_attn_core<128, 0, false>(p, s);
    else
      launch_attn_core<128, 1, false>(p, s);
  }
  return hipGetLastError();
}

}  // namespace gdn
