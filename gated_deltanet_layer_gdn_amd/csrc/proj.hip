// proj.hip -- the GDN input projections with the decay and beta
// parametrisation fused into the GEMM's epilogue ("Implement the Qwen3.8
// Flash Next Rust and Metal text core", section Verification: primitive
// vectors for the GDN projection; section Implementation: the GDN geometry
// these projections feed).
//
// One bf16 GEMM on the MFMA, Y = H W^T (fp32 accumulation), over the fused
// weight W [N_out][hidden] whose rows are, in order:
//   the C_ch conv inputs x ([q | k | v], head-major), the H_v d_v gate
//   inputs z, H_v rows b and H_v rows a;
// the epilogue writes x and z in bf16 and turns the last 2 H_v columns into
//   beta = sigmoid(b),   g = -exp(A_log[h]) * softplus(a + dt_bias[h])
// in fp32 (the gated delta rule's beta_t and log decay g_t = log a_t, with the
// decay parametrised as in Gated DeltaNet's Mamba2-style gate).
//
// Tiling.  Where C_ch and H_v d_v are multiples of 256 (the Qwen geometry:
// 10,240 and 6,144), x and z are computed in 256 x 256 output tiles by
// proj_dma_kernel: 512 threads as 2 x 4 waves of 128 x 64 (8 x 4 MFMA tiles of
// 16 x 16, v_mfma_f32_16x16x32_bf16), K in steps of 32 through a ring of five
// LDS stages (all 160 KB of the compute unit's LDS) filled by gfx950's
// direct-to-LDS loads four steps ahead, and each step's operand fragments
// read into registers while the previous step's MFMAs run.  Other
// geometries, and the last 2 H_v columns (b and a), use proj_kernel, which
// stages its tiles through registers: 256 x 256 tiles of 2 x 4 waves of
// 128 x 64, K steps of 64, the tiles of step kt + 2 loaded into registers
// while step kt computes (two register sets, double-buffered LDS rows padded
// by 16 bytes against bank conflicts, one barrier per step; the staging
// registers are native vectors, which the compiler keeps in registers:
// arrays of the struct-based uint4 went to scratch memory and made the
// kernel four times slower).  Both operands are K-contiguous in memory (H rows
// and W rows), which is the MFMA operand layout (lane (g, c) supplies row c,
// K indices 8g .. 8g + 7), so every operand read is one 16-byte LDS read.
// Blocks are numbered so that each XCD takes a contiguous range, walked in
// groups of 8 M tiles, so the blocks resident on an XCD at one time share
// their A and B tiles through its L2.
#include <utility>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kBK = 64;
constexpr int kPad = 8;                 // bf16 elements of padding per LDS row
constexpr int kLdsRow = kBK + kPad;     // 72 elements = 144 bytes
constexpr int kGroupM = 8;

struct ProjArgs {
  const uint16_t *h;   // [M][K] bf16
  const uint16_t *w;   // [N][K] bf16
  const float *A_log, *dt_bias;
  uint16_t *x, *z;     // [M][C_ch], [M][Z] bf16
  float *g, *beta;     // [M][H_v]
  int64_t M;
  int K, N, C_ch, Z, H_v;
  int n_begin, n_count;  // the columns this launch covers: [n_begin, n_begin + n_count)
};

__device__ __forceinline__ float softplus_f(float u) {
  // max(u, 0) + log(1 + exp(-|u|)): no overflow for large u, and log1p keeps
  // the relative precision of the small values that large negative u give
  return fmaxf(u, 0.f) + log1pf(expf(-fabsf(u)));
}

__device__ __forceinline__ int xcd_remap_p(int bid, int n) {
  if (n % 8) return bid;
  const int per = n / 8;
  return (bid % 8) * per + bid / 8;
}

// Block tile BM x BN, waves WGM x WGN, each wave (BM / WGM) x (BN / WGN).
template <int BM, int BN, int WGM, int WGN>
struct ProjShape {
  static constexpr int kThreads = 64 * WGM * WGN;
  static constexpr int MI = BM / WGM / 16, NJ = BN / WGN / 16;  // MFMA tiles per wave
  static constexpr int PA = BM * (kBK / 8) / kThreads;          // 16-byte pieces per thread
  static constexpr int PB = BN * (kBK / 8) / kThreads;
  static constexpr int ROWS = kThreads / (kBK / 8);             // rows one pass of pieces covers
};

// Global -> register staging of one K step (16-byte pieces, row-major tile
// rows of 64 K values: thread t takes part t % 8 of rows t / 8 + ROWS j).
template <int PA, int PB>
struct Stage {
  u32x4 a[PA], b[PB];
};

template <int PA, int PB>
__device__ __forceinline__ void gload(Stage<PA, PB> &st, const uint16_t *const (&hrow)[PA],
                                      const uint16_t *const (&wrow)[PB], int k0) {
#pragma unroll
  for (int j = 0; j < PA; ++j) st.a[j] = *reinterpret_cast<const u32x4 *>(hrow[j] + k0);
#pragma unroll
  for (int j = 0; j < PB; ++j) st.b[j] = *reinterpret_cast<const u32x4 *>(wrow[j] + k0);
}

template <int PA, int PB, int ROWS>
__device__ __forceinline__ void lstore(const Stage<PA, PB> &st, uint16_t (*As)[kLdsRow],
                                       uint16_t (*Bs)[kLdsRow], int row0, int part) {
#pragma unroll
  for (int j = 0; j < PA; ++j) *reinterpret_cast<u32x4 *>(&As[row0 + ROWS * j][part * 8]) = st.a[j];
#pragma unroll
  for (int j = 0; j < PB; ++j) *reinterpret_cast<u32x4 *>(&Bs[row0 + ROWS * j][part * 8]) = st.b[j];
}

// The wave's sub-tile over one K step: kBK / 32 rounds of MI x NJ MFMAs.
template <int MI, int NJ>
__device__ __forceinline__ void compute(const uint16_t (*As)[kLdsRow], const uint16_t (*Bs)[kLdsRow],
                                        f32x4 (&acc)[MI][NJ], int wm, int wn, int c, int gq) {
#pragma unroll
  for (int ks = 0; ks < kBK / 32; ++ks) {
    u16x8 av[MI], bv[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      av[i] = *reinterpret_cast<const u16x8 *>(&As[wm + 16 * i + c][32 * ks + 8 * gq]);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      bv[j] = *reinterpret_cast<const u16x8 *>(&Bs[wn + 16 * j + c][32 * ks + 8 * gq]);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16x16x32(av[i], bv[j], acc[i][j]);
  }
}

// Four rows (m, m + 1, m + 2, m + 3) of output column n from one
// accumulator.  Each 16-column tile lies in one output except around b and
// a (H_v columns each), so the column decides per lane.
__device__ __forceinline__ void store_out(const ProjArgs &a, const f32x4 &v, int64_t m, int n) {
  if (n >= a.N) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t mr = m + r;
    if (mr >= a.M) continue;
    if (n < a.C_ch) {
      a.x[mr * a.C_ch + n] = f32_to_bf16_bits(v[r]);
    } else if (n < a.C_ch + a.Z) {
      a.z[mr * a.Z + (n - a.C_ch)] = f32_to_bf16_bits(v[r]);
    } else if (n < a.C_ch + a.Z + a.H_v) {
      a.beta[mr * a.H_v + (n - a.C_ch - a.Z)] = sigmoidf_(v[r]);
    } else {
      const int hh = n - a.C_ch - a.Z - a.H_v;
      a.g[mr * a.H_v + hh] = -expf(a.A_log[hh]) * softplus_f(v[r] + a.dt_bias[hh]);
    }
  }
}

template <int MI, int NJ, size_t... Is>
__device__ __forceinline__ void epilogue_all(const ProjArgs &a, const f32x4 (&acc)[MI][NJ],
                                             int64_t m_base, int n_base,
                                             std::index_sequence<Is...>) {
  (store_out(a, acc[Is / NJ][Is % NJ], m_base + 16 * static_cast<int>(Is / NJ),
             n_base + 16 * static_cast<int>(Is % NJ)),
   ...);
}

template <int BM, int BN, int WGM, int WGN, int STAGES>
__global__ __launch_bounds__((ProjShape<BM, BN, WGM, WGN>::kThreads))
void proj_kernel(ProjArgs a) {
  using Sh = ProjShape<BM, BN, WGM, WGN>;
  constexpr int MI = Sh::MI, NJ = Sh::NJ, PA = Sh::PA, PB = Sh::PB, ROWS = Sh::ROWS;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][kLdsRow];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_mt = static_cast<int>((a.M + BM - 1) / BM);
  const int n_nt = (a.n_count + BN - 1) / BN;
  const int lid = xcd_remap_p(blockIdx.x, n_mt * n_nt);
  // grouped raster: kGroupM M tiles share each N tile in turn
  const int per_group = kGroupM * n_nt;
  const int grp = lid / per_group;
  const int first_mt = grp * kGroupM;
  const int gm = min(kGroupM, n_mt - first_mt);
  const int in_grp = lid % per_group;
  const int mt = first_mt + in_grp % gm;
  const int nt = in_grp / gm;
  const int64_t m0 = static_cast<int64_t>(mt) * BM;
  const int n0 = a.n_begin + nt * BN;

  // Rows past M or N re-read the last row (their products are not stored).
  const int row0 = tid >> 3, part = tid & 7;
  const uint16_t *hrow[PA], *wrow[PB];
#pragma unroll
  for (int j = 0; j < PA; ++j) {
    int64_t ma = m0 + row0 + ROWS * j;
    ma = ma < a.M ? ma : a.M - 1;
    hrow[j] = a.h + ma * a.K + part * 8;
  }
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    int nb = n0 + row0 + ROWS * j;
    nb = nb < a.N ? nb : a.N - 1;
    wrow[j] = a.w + static_cast<int64_t>(nb) * a.K + part * 8;
  }

  const int wm = (wave / WGN) * (BM / WGM), wn = (wave % WGN) * (BN / WGN);
  const int c = lane & 15, gq = lane >> 4;
  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = a.K / kBK;
  const int last = (nk - 1) * kBK;
  if constexpr (STAGES == 2) {
    // Two register sets: the tile of K step kt + 2 is requested while step
    // kt computes, so every load has two steps of MFMAs to arrive in; LDS is
    // double-buffered with one barrier per step.  Loads past the last K step
    // re-read it (branch-free, so both sets stay in registers); only the
    // stores to LDS are guarded.
    Stage<PA, PB> s0, s1;
    gload(s0, hrow, wrow, 0);
    gload(s1, hrow, wrow, min(kBK, last));
    lstore<PA, PB, ROWS>(s0, As[0], Bs[0], row0, part);
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      gload(s0, hrow, wrow, min((kt + 2) * kBK, last));
      compute<MI, NJ>(As[0], Bs[0], acc, wm, wn, c, gq);
      lstore<PA, PB, ROWS>(s1, As[1], Bs[1], row0, part);
      __syncthreads();
      gload(s1, hrow, wrow, min((kt + 3) * kBK, last));
      compute<MI, NJ>(As[1], Bs[1], acc, wm, wn, c, gq);
      if (kt + 2 < nk) lstore<PA, PB, ROWS>(s0, As[0], Bs[0], row0, part);
      __syncthreads();
    }
    if (kt < nk) compute<MI, NJ>(As[0], Bs[0], acc, wm, wn, c, gq);
  } else {
    // One register set: the next K step's tile is requested while this one
    // computes.
    Stage<PA, PB> st;
    gload(st, hrow, wrow, 0);
    lstore<PA, PB, ROWS>(st, As[0], Bs[0], row0, part);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      gload(st, hrow, wrow, min((kt + 1) * kBK, last));
      compute<MI, NJ>(As[buf], Bs[buf], acc, wm, wn, c, gq);
      if (kt + 1 < nk) lstore<PA, PB, ROWS>(st, As[buf ^ 1], Bs[buf ^ 1], row0, part);
      __syncthreads();
    }
  }

  // Epilogue: tile (i, j) holds rows m0 + wm + 16 i + 4 gq + r, column
  // n0 + wn + 16 j + c.  The tiles are walked by a fold over a compile-time
  // index sequence, so every accumulator is named statically (a runtime loop
  // index would put the accumulators in scratch memory).
  epilogue_all(a, acc, m0 + wm + 4 * gq, n0 + wn + c, std::make_index_sequence<MI * NJ>{});
}

// Four rows of one output column into a bf16 matrix with row stride ld.
__device__ __forceinline__ void store4_bf16(uint16_t *out, int64_t ld, int64_t M, const f32x4 &v,
                                            int64_t m, int n) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (m + r < M) out[(m + r) * ld + n] = f32_to_bf16_bits(v[r]);
}

template <int MI, int NJ, size_t... Is>
__device__ __forceinline__ void epilogue_bf16(uint16_t *out, int64_t ld, int64_t M,
                                              const f32x4 (&acc)[MI][NJ], int64_t m_base,
                                              int n_base, std::index_sequence<Is...>) {
  (store4_bf16(out, ld, M, acc[Is / NJ][Is % NJ], m_base + 16 * static_cast<int>(Is / NJ),
               n_base + 16 * static_cast<int>(Is % NJ)),
   ...);
}

// ---- direct-to-LDS tiles.  gfx950's global_load_lds_dwordx4 moves 16-byte
// pieces from memory into LDS without passing through registers, so loads can
// run several K steps ahead at no register cost.  One such load writes a
// wave's 64 pieces to 1 KB of consecutive LDS, lane by lane, so instead of
// padding rows, the layout permutes the pieces within a row: a row is 32 bf16
// (64 bytes, 4 pieces) and piece p of row r sits in slot p ^ ((r >> 2) & 3).
// An operand read (16 lanes of one K quarter over 16 consecutive rows) then
// touches 16 distinct 4-bank groups.  Measured side by side at M = 4096 /
// 16,384, hidden 5120, N = 16,480 (TFLOP/s, bitwise equal results): the
// register-staged kernel 816-896 / 1,010; direct-to-LDS with four stages
// 966-1,064 / 1,130 and with five 995-1,082 / 1,160; four waves of 128 x 128
// (256 accumulators each, in AGPRs) lost to the compiler's copies between
// accumulator registers (824-879 / 931).
constexpr int kDBK = 32;          // K per stage
constexpr int kDStages = 5;       // LDS ring (5 x 32 KB); loads run kDStages - 1 steps ahead
constexpr int kDRowBytes = kDBK * 2;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <int N>
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt vmcnt(N), other counters left at their maxima (gfx9 encoding:
  // vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <int BM, int BN, int WGM, int WGN>
struct DmaShape {
  static constexpr int kWaves = WGM * WGN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WM = BM / WGM, WN = BN / WGN;         // wave tile
  static constexpr int MI = WM / 16, NJ = WN / 16;
  static constexpr int kStageBytes = (BM + BN) * kDRowBytes;  // A rows, then B rows
  static constexpr int kLoads = (BM + BN) * kDRowBytes / 1024 / kWaves;  // 1 KB loads per wave and stage
};

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void proj_dma_kernel(ProjArgs a) {
  using Sh = DmaShape<BM, BN, WGM, WGN>;
  constexpr int MI = Sh::MI, NJ = Sh::NJ, NL = Sh::kLoads;
  __shared__ __attribute__((aligned(1024))) char lds[kDStages * Sh::kStageBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_mt = static_cast<int>((a.M + BM - 1) / BM);
  const int n_nt = (a.n_count + BN - 1) / BN;
  const int lid = xcd_remap_p(blockIdx.x, n_mt * n_nt);
  const int per_group = kGroupM * n_nt;
  const int grp = lid / per_group;
  const int first_mt = grp * kGroupM;
  const int gm = min(kGroupM, n_mt - first_mt);
  const int in_grp = lid % per_group;
  const int mt = first_mt + in_grp % gm;
  const int nt = in_grp / gm;
  const int64_t m0 = static_cast<int64_t>(mt) * BM;
  const int n0 = a.n_begin + nt * BN;

  // Load l of this wave covers tile rows 16 q .. 16 q + 15 (q = NL wave + l;
  // A rows first): lane i fills row 16 q + i / 4, slot i % 4, which holds
  // piece (i % 4) ^ ((i >> 4) & 3) of that row.  Rows past M or N re-read the
  // last row (their products are not stored).
  const uint16_t *src[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    const int q = NL * wave + l;
    const int r = 16 * q + (lane >> 2);
    const int piece = (lane & 3) ^ ((lane >> 4) & 3);
    if (r < BM) {
      int64_t ma = m0 + r;
      ma = ma < a.M ? ma : a.M - 1;
      src[l] = a.h + ma * a.K + piece * 8;
    } else {
      int nb = n0 + (r - BM);
      nb = nb < a.N ? nb : a.N - 1;
      src[l] = a.w + static_cast<int64_t>(nb) * a.K + piece * 8;
    }
  }
  auto issue = [&](int stage, int k0) {
    char *base = lds + stage * Sh::kStageBytes + NL * wave * 1024;
#pragma unroll
    for (int l = 0; l < NL; ++l)
      __builtin_amdgcn_global_load_lds((glb_void_t *)(src[l] + k0), (lds_void_t *)(base + 1024 * l),
                                       16, 0, 0);
  };

  const int wm = (wave / WGN) * Sh::WM, wn = (wave % WGN) * Sh::WN;
  const int c = lane & 15, gq = lane >> 4;
  const int slot_off = 16 * (gq ^ (c >> 2));  // this lane's piece within its row
  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = a.K / kDBK;
  // Fragments of one K step: the A operands of the wave's MI row tiles and the
  // B operands of its NJ column tiles.
  auto read_frags = [&](int stage, u16x8 (&av)[MI], u16x8 (&bv)[NJ]) {
    const char *A = lds + stage * Sh::kStageBytes;
    const char *B = A + BM * kDRowBytes;
#pragma unroll
    for (int i = 0; i < MI; ++i)
      av[i] = *reinterpret_cast<const u16x8 *>(A + (wm + 16 * i + c) * kDRowBytes + slot_off);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      bv[j] = *reinterpret_cast<const u16x8 *>(B + (wn + 16 * j + c) * kDRowBytes + slot_off);
  };
  auto mma = [&](const u16x8 (&av)[MI], const u16x8 (&bv)[NJ]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16x16x32(av[i], bv[j], acc[i][j]);
  };
  // Step kt: wait for stage kt + 1 and publish it; refill the slot of stage
  // kt, whose fragments are already in registers, with stage kt + S (S
  // stages in the ring); read stage kt + 1's fragments into the other
  // register set while the MFMAs of step kt run.  Steps of the main loop all
  // do the same (kt + S < nk); the last ones are peeled.
  auto publish_next = [&](int kt) {
    // loads still in flight after stage kt + 1's: stages kt + 2 .. min(nk - 1, kt + S - 1)
    const int ahead = min(nk - 1, kt + kDStages - 1) - (kt + 1);
    if (ahead >= 3) wait_vm<3 * NL>();
    else if (ahead == 2) wait_vm<2 * NL>();
    else if (ahead == 1) wait_vm<NL>();
    else wait_vm<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage kt are done
    __builtin_amdgcn_s_barrier();
  };
  auto step_full = [&](int kt, const u16x8 (&av)[MI], const u16x8 (&bv)[NJ], u16x8 (&an)[MI],
                       u16x8 (&bn)[NJ]) {
    wait_vm<(kDStages - 2) * NL>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    issue(kt % kDStages, (kt + kDStages) * kDBK);
    read_frags((kt + 1) % kDStages, an, bn);
    mma(av, bv);
  };
  auto step_tail = [&](int kt, const u16x8 (&av)[MI], const u16x8 (&bv)[NJ], u16x8 (&an)[MI],
                       u16x8 (&bn)[NJ]) {
    if (kt + 1 < nk) {
      publish_next(kt);
      if (kt + kDStages < nk) issue(kt % kDStages, (kt + kDStages) * kDBK);
      read_frags((kt + 1) % kDStages, an, bn);
    }
    mma(av, bv);
  };

#pragma unroll
  for (int st = 0; st < kDStages; ++st)
    if (st < nk) issue(st, st * kDBK);
  publish_next(-1);  // stage 0
  u16x8 a0[MI], b0[NJ], a1[MI], b1[NJ];
  read_frags(0, a0, b0);
  int kt = 0;
  for (; kt + kDStages + 1 < nk; kt += 2) {  // nk is even (K is a multiple of 64)
    step_full(kt, a0, b0, a1, b1);
    step_full(kt + 1, a1, b1, a0, b0);
  }
  for (; kt < nk; kt += 2) {
    step_tail(kt, a0, b0, a1, b1);
    step_tail(kt + 1, a1, b1, a0, b0);
  }

  // The launch covers whole tiles of x or of z only (C_ch and H_v d_v are
  // multiples of BN), so a tile stores bf16 to one output, chosen per block.
  const int64_t mb = m0 + wm + 4 * gq;
  constexpr auto seq = std::make_index_sequence<MI * NJ>{};
  if (n0 < a.C_ch)
    epilogue_bf16(a.x, a.C_ch, a.M, acc, mb, n0 + wn + c, seq);
  else
    epilogue_bf16(a.z, a.Z, a.M, acc, mb, n0 - a.C_ch + wn + c, seq);
}

template <int BM, int BN, int WGM, int WGN>
void launch_dma_tiles(const ProjArgs &a, hipStream_t s) {
  const int64_t n_mt = (a.M + BM - 1) / BM;
  const int64_t n_nt = (a.n_count + BN - 1) / BN;
  hipLaunchKernelGGL((proj_dma_kernel<BM, BN, WGM, WGN>), dim3(static_cast<unsigned>(n_mt * n_nt)),
                     dim3(DmaShape<BM, BN, WGM, WGN>::kThreads), 0, s, a);
}

template <int BM, int BN, int WGM, int WGN, int STAGES>
void launch_tiles(const ProjArgs &a, hipStream_t s) {
  const int64_t n_mt = (a.M + BM - 1) / BM;
  const int64_t n_nt = (a.n_count + BN - 1) / BN;
  hipLaunchKernelGGL((proj_kernel<BM, BN, WGM, WGN, STAGES>), dim3(static_cast<unsigned>(n_mt * n_nt)),
                     dim3(ProjShape<BM, BN, WGM, WGN>::kThreads), 0, s, a);
}

// 256 x 256 tiles of 8 waves, each 128 x 64, with two register stages: half
// the LDS and L2 traffic per flop of 128 x 128 tiles.  Measured side by side
// at M = 4096 / 16384, hidden 5120, N = 16480 (TFLOP/s): 128 x 128, 4 waves,
// two stages 794 / 792; 256 x 256, one stage 680 / 803; 256 x 256, two
// stages 828 / 970; 256 x 128 or 128 x 256, 8 waves of 64 x 64, two stages
// 801-817 / 877-882.
constexpr int kProjBM = 256, kProjBN = 256, kProjWGM = 2, kProjWGN = 4, kProjStages = 2;
// The columns after the last full 256-column tile (b and a: 2 H_v = 96 at the
// Qwen geometry) in 32 x 96 tiles of 4 waves (16 x 48 each): 128 blocks at M =
// 4096 with no padding columns.  Measured side by side (whole projection,
// bitwise equal): 1,117-1,131 TFLOP/s at M = 4096 and 1,152-1,167 at 16,384,
// against 1,073-1,084 / 1,142-1,153 with 64 x 256 tiles (62% of their columns
// padding) and 1,116-1,124 / 1,135-1,148 with 16 x 128.
constexpr int kProjRemBM = 32, kProjRemBN = 96, kProjRemWGM = 2, kProjRemWGN = 2;
constexpr int kDmaWGM = 2, kDmaWGN = 4;  // waves of the direct-to-LDS kernel (M x N)

}  // namespace

hipError_t launch_in_proj(const Geom &g, int64_t M, int hidden, const void *h, const void *w,
                          const float *A_log, const float *dt_bias, void *x, void *z, float *gl,
                          float *beta, hipStream_t s) {
  ProjArgs a;
  a.h = static_cast<const uint16_t *>(h);
  a.w = static_cast<const uint16_t *>(w);
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.x = static_cast<uint16_t *>(x);
  a.z = static_cast<uint16_t *>(z);
  a.g = gl;
  a.beta = beta;
  a.M = M;
  a.K = hidden;
  a.C_ch = g.C_ch;
  a.Z = g.H_v * g.D;
  a.H_v = g.H_v;
  a.N = g.C_ch + a.Z + 2 * g.H_v;
  // The full 256-column tiles, then the remaining columns (96 at the Qwen
  // geometry) in small tiles: as 256 x 256 tiles they would be a last round
  // of blocks at the cost of a full one for a third of the work (at M = 4096,
  // 16 such blocks after 1024 full ones on 256 compute units).
  int n_full = a.N / kProjBN * kProjBN;
  if (a.C_ch % kProjBN == 0 && a.Z % kProjBN == 0) {
    // x and z in whole 256-column tiles on the direct-to-LDS kernel; b and a
    // (2 H_v columns) below with the remainder.
    n_full = a.C_ch + a.Z;
    a.n_begin = 0;
    a.n_count = n_full;
    launch_dma_tiles<kProjBM, kProjBN, kDmaWGM, kDmaWGN>(a, s);
  } else if (n_full > 0) {
    a.n_begin = 0;
    a.n_count = n_full;
    launch_tiles<kProjBM, kProjBN, kProjWGM, kProjWGN, kProjStages>(a, s);
  }
  if (n_full < a.N) {
    a.n_begin = n_full;
    a.n_count = a.N - n_full;
    launch_tiles<kProjRemBM, kProjRemBN, kProjRemWGM, kProjRemWGN, kProjStages>(a, s);
  }
  return hipGetLastError();
}

}  // namespace gdn
