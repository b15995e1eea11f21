// gdn_internal.h -- host-side plumbing between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

// Everything a kernel needs to know about the geometry, as plain values.
struct Geom {
  int B, H_k, H_v, D, W, G;  // D = d_k = d_v, G = H_v / H_k
  int C_ch;                  // 2*H_k*D + H_v*D
  int in_dt, out_dt;         // 0 = fp32, 1 = bf16
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
size_t decode_ws_bytes(const Geom &g);

// Kernel launchers (enqueue only; return the launch status).
hipError_t launch_conv_plain(const Geom &g, int64_t T, const void *x, const void *w,
                             void *hist, float *out, hipStream_t s);
hipError_t launch_conv_prefill(const Geom &g, const PrefillWs &L, const void *x,
                               const void *w, const void *hist, char *ws, hipStream_t s);
hipError_t launch_conv_roll(const Geom &g, int64_t T, const void *x, void *hist,
                            hipStream_t s);
hipError_t launch_decode(const Geom &g, const float *qkv, const void *z, const float *gl,
                         const float *beta, float *S, void *y, hipStream_t s);
// Also rolls the conv history (x, hist) after the sequence.
hipError_t launch_prefill_prep(const Geom &g, const PrefillWs &L, const float *gl,
                               const float *beta, char *ws, const void *x, void *hist,
                               hipStream_t s);
// x, conv_w and hist are used by the split-role pass (v and its history).
hipError_t launch_prefill_state(const Geom &g, const PrefillWs &L, const void *z, float *S,
                                void *y, const char *ws, const void *x, const void *conv_w,
                                void *hist, hipStream_t s);

}  // namespace gdn
