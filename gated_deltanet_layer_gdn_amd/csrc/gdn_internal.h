// gdn_internal.h -- host-side plumbing between the C ABI and the kernels.
#pragma once

#ifdef __HIPCC__
#include <hip/hip_ext.h>
#endif
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

// Events recorded at one kernel's own start and end (the timed entry points
// launch through hipExtLaunchKernelGGL with them; null: a plain launch).
struct KernelEvents {
  hipEvent_t start, stop;
};

// Output code of the kernels' DTY template parameter (see gdn_device.h):
// y's element type, plus 4 when z is null (no gate, y = o).
inline int out_code(int out_dt, const void *z) { return out_dt | (z ? 0 : 4); }

// LAUNCH(ZT, OC) with the input element type ZT (0 fp32, 1 bf16) and the
// output code OC as compile-time constants.
#define GDN_OUT_DISPATCH(IN_DT, OC, LAUNCH)                                       \
  do {                                                                            \
    const int oc_ = (OC);                                                         \
    if ((IN_DT) == 0) {                                                           \
      switch (oc_) {                                                              \
        case 0: LAUNCH(0, 0); break;                                              \
        case 1: LAUNCH(0, 1); break;                                              \
        case 2: LAUNCH(0, 2); break;                                              \
        case 4: LAUNCH(0, 4); break;                                              \
        case 5: LAUNCH(0, 5); break;                                              \
        default: LAUNCH(0, 6); break;                                             \
      }                                                                           \
    } else {                                                                      \
      switch (oc_) {                                                              \
        case 0: LAUNCH(1, 0); break;                                              \
        case 1: LAUNCH(1, 1); break;                                              \
        case 2: LAUNCH(1, 2); break;                                              \
        case 4: LAUNCH(1, 4); break;                                              \
        case 5: LAUNCH(1, 5); break;                                              \
        default: LAUNCH(1, 6); break;                                             \
      }                                                                           \
    }                                                                             \
  } while (0)

// Everything a kernel needs to know about the geometry, as plain values.
struct Geom {
  int B, H_k, H_v, D, W, G;  // D = d_k = d_v, G = H_v / H_k
  int C_ch;                  // 2*H_k*D + H_v*D
  int in_dt, out_dt;         // 0 = fp32, 1 = bf16 (, 2 = fp16 for out_dt)
  float eps, q_scale;
};

// Prefill workspace carve-up (byte offsets from the workspace base, each
// 256-byte aligned).  Dp = max(D, 32); Cp = max(C, 32); T_pad = T rounded up
// to a multiple of Cp; NC = ceil(T / C) chunks.
//   q/k token-major   [B][H_k][Dp/32][T_pad][32] bf16 hi and lo: each 32-wide
//                                               slice of the head dimension in
//                                               permuted K order, slice-major;
//                                               for the split-role pass the lo
//                                               halves are e4m3 bytes scaled by
//                                               q_lo_scale / k_lo_scale
//   k dim-major       [B][H_k][T_pad/32][D][32] bf16 hi and lo, tokens in
//                                               permuted K order
//   v dim-major       [B][H_v][T_pad/16][D][16] fp32
//   (both empty for the split-role pass)
//   T = (I + A)^{-1}  [B][H_v][NC][C][Cp]      bf16, columns permuted
//   P = tril(D) * QK^T [B][H_v][NC][C][Cp]     bf16 hi and lo, columns permuted
//   gates             [B][H_v][NC][3][C]       fp32: gamma_t = exp(G_t),
//                                               exp(G_last - G_t), beta_t;
//                     [B][H_v][NC][C][4]       for d = 128, chunk 64: per token
//                                               gamma_t, exp(G_last - G_t), beta_t,
//                                               gamma_last (room for 4C per chunk
//                                               is reserved either way)
struct PrefillWs {
  int64_t T, T_pad;
  int C, Cp, Dp, NC;
  size_t q_hi, q_lo, k_hi, k_lo, kT_hi, kT_lo, vT, Tm, P_hi, P_lo, gates;
  size_t total;
  // Split-role pass: scales of the fp8 low halves of q and k (0 otherwise).
  float q_lo_scale, k_lo_scale;
};

bool prefill_ws_layout(const Geom &g, int64_t T, int C, PrefillWs *ws);
// Whether prefill runs the split-role state pass (d = 128, 64-token chunks).
// That pass builds the dim-major copy of k in LDS, computes v from x itself
// and rolls the conv history of the v channels; the conv pass then writes
// neither k dim-major nor v, and the prep pass rolls the q and k channels only.
__host__ __device__ inline bool prefill_split_roles(const Geom &g, const PrefillWs &L) {
  return g.D == 128 && L.C == 64;
}
size_t decode_ws_bytes(const Geom &g, int T);

// Size of the fixed device array that serves as the decode workspace of
// gdn_decode_step_noalloc, and its device address on the GPU of stream `s`
// (looked up once per GPU).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(hipStream_t s, void **ptr);

// Kernel launchers (enqueue only; return the launch status).
hipError_t launch_conv_plain(const Geom &g, int64_t T, const void *x, const void *w,
                             void *hist, float *out, hipStream_t s);
hipError_t launch_conv_prefill(const Geom &g, const PrefillWs &L, const void *x,
                               const void *w, const void *hist, char *ws, hipStream_t s,
                               const KernelEvents *ev = nullptr);
hipError_t launch_conv_roll(const Geom &g, int64_t T, const void *x, void *hist,
                            hipStream_t s);
// Decode of T = 1..kMaxMultiTokens tokens per sequence in two launches: the
// conv step writes qkv [B][T][C_ch] fp32 and rolls the histories into their
// out slots; the state stream then reads qkv.  in_slots / out_slots may be
// null (sequence b in slot b, state after the last token back into it).
constexpr int kMaxMultiTokens = 4;
#ifdef __HIPCC__
// Launch of `kernel` on `s`; with `ev` (the timed entry points), through
// hipExtLaunchKernelGGL, which records ev->start and ev->stop at the kernel's
// own start and end, so the interval leaves out the launch latency that
// events recorded on the stream between launches would include.  The
// arguments are converted to the kernel's parameter types first (the
// extended launch passes them by address as given).
template <typename... P, typename... A>
inline void launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s,
                          const KernelEvents *ev, A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
  if (ev)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev->start, ev->stop, 0, static_cast<P>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, static_cast<P>(args)...);
}
#endif
hipError_t launch_conv_step(const Geom &g, int T, const void *x, const void *w, void *hist,
                            float *out, const int32_t *in_slots, const int32_t *out_slots,
                            int n_slots, hipStream_t s, const KernelEvents *ev = nullptr);
hipError_t launch_decode(const Geom &g, int T, const float *qkv, const void *z, const float *gl,
                         const float *beta, float *S, void *y, int n_slots,
                         const int32_t *in_slots, const int32_t *out_slots, hipStream_t s,
                         const KernelEvents *ev = nullptr);
// Full attention of the hybrid schedule (attn.hip): geometry of one call.
struct AttnGeom {
  int B, H_q, H_kv, D, rot;  // D = head dimension (128 or 256), rot = rotary width
  float base, scale;         // RoPE base, score scale
  int in_dt, out_dt;
};
size_t attn_ws_bytes(const AttnGeom &a, int64_t T, int64_t pos0);
hipError_t launch_attn_prefill(const AttnGeom &a, int64_t T, int64_t pos0, const void *q,
                               const void *k, const void *v, void *kc, void *vc, int64_t T_max,
                               void *o, void *ws, hipStream_t s);

// Input projections: Y = H W^T over M rows of `hidden` bf16 values, W
// [C_ch + H_v D + 2 H_v][hidden] bf16; x, z in bf16, beta and the log decay
// g in fp32 (see proj.hip).
hipError_t launch_in_proj(const Geom &g, int64_t M, int hidden, const void *h, const void *w,
                          const float *A_log, const float *dt_bias, void *x, void *z, float *gl,
                          float *beta, hipStream_t s);
// Zero-centred grouped RMS norm + sigmoid gate over rows * H_v groups of D
// values (z may be null: no gate; w may be null: unit scale).
hipError_t launch_gated_rmsnorm(const Geom &g, int64_t rows, const float *o, const void *z,
                                const float *w, float eps, void *y, hipStream_t s);
// Prep grids of more than this many blocks (chunks x key heads x sequences)
// stage K in LDS; with two or more value heads per key head they also take
// the value heads one per wave.
constexpr int64_t kPrepStageBlocks = 8 * 256;
// Whether the prep pass computes the q and k channels' conv, SiLU and L2 norm
// itself (and writes them to the workspace for the state pass) instead of
// reading them from a conv pass, which is then not launched: the split-role
// prefill on grids of more than kPrepFuseBlocks blocks (where prep stages K
// and takes the value heads one per wave).  There the fused pass moves less
// (x read once instead of the q/k rows written by one pass and read by the
// next) and hides its conv among the other blocks; on smaller grids each
// block's conv latency shows and the separate conv pass is faster (measured
// crossover between 3,072 and 6,144 blocks).
constexpr int64_t kPrepFuseBlocks = 16 * 256;
inline bool prep_fuses_conv(const Geom &g, const PrefillWs &L) {
  return prefill_split_roles(g, L) && g.G >= 2 &&
         static_cast<int64_t>(L.NC) * g.H_k * g.B > kPrepFuseBlocks;
}
// Also rolls the conv history (x, hist) after the sequence; conv_w is read
// when prep_fuses_conv.
hipError_t launch_prefill_prep(const Geom &g, const PrefillWs &L, const float *gl,
                               const float *beta, char *ws, const void *x, const void *conv_w,
                               void *hist, hipStream_t s, const KernelEvents *ev = nullptr);
// x, conv_w and hist are used by the split-role pass (v and its history).
hipError_t launch_prefill_state(const Geom &g, const PrefillWs &L, const void *z, float *S,
                                void *y, const char *ws, const void *x, const void *conv_w,
                                void *hist, hipStream_t s, const KernelEvents *ev = nullptr);

}  // namespace gdn
