// epilogue.hip -- zero-centred grouped RMS norm before the sigmoid output
// gate, as its own pass over the layer's ungated readout ("Implement the
// Qwen3.8 Flash Next Rust and Metal text core", section Implementation:
// zero-centred norms; its implementation comment: zero-centred grouped RMS
// and the sigmoid output gate).  Reading taken: a group is the d_v values of
// one value head of one token;
//   y = o / sqrt(mean(o^2) + eps) * (1 + w) * sigmoid(z),
// with a per-channel weight w of d_v entries shared by the heads (zero-
// centred: w = 0 is the identity scale).
//
// The norm needs a whole group, which the state kernels split over several
// blocks (32 state rows each), so it runs after them: the layer writes the
// ungated readout o (z = NULL) and this pass reads it once.  HBM-bound: per
// group, d_v fp32 of o and d_v elements of z read, d_v elements of y written.
// D / 4 lanes hold one group, four channels each (16-byte o loads); the
// group's sum of squares is an xor-shuffle reduction over those lanes.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int D, int DTZ, int OC>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(int64_t groups, const float *__restrict__ o,
                                                            const void *__restrict__ z,
                                                            const float *__restrict__ w,
                                                            float eps, void *__restrict__ y) {
  constexpr int LPG = D / 4;  // lanes per group
  const int64_t gi = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / LPG;
  const int j = threadIdx.x % LPG;
  if (gi >= groups) return;  // whole groups only: the shuffles stay within live lanes
  const size_t base = static_cast<size_t>(gi) * D + 4 * j;
  const float4 v = *reinterpret_cast<const float4 *>(o + base);
  float ss = v.x * v.x;
  ss = __builtin_fmaf(v.y, v.y, ss);
  ss = __builtin_fmaf(v.z, v.z, ss);
  ss = __builtin_fmaf(v.w, v.w, ss);
#pragma unroll
  for (int m = LPG / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, kWave);
  const float r = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
  float4 sc = make_float4(1.f, 1.f, 1.f, 1.f);
  if (w) {
    const float4 ww = *reinterpret_cast<const float4 *>(w + 4 * j);
    sc = make_float4(1.f + ww.x, 1.f + ww.y, 1.f + ww.z, 1.f + ww.w);
  }
  float out[4] = {v.x * r * sc.x, v.y * r * sc.y, v.z * r * sc.z, v.w * r * sc.w};
  if constexpr (out_gated(OC)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] *= sigmoidf_(load_elem<DTZ>(z, base + k));
  }
  if constexpr (out_type(OC) == 0) {
    *reinterpret_cast<float4 *>(static_cast<float *>(y) + base) =
        make_float4(out[0], out[1], out[2], out[3]);
  } else {
    uint16_t h[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      h[k] = out_type(OC) == 1 ? f32_to_bf16_bits(out[k]) : f32_to_f16_bits(out[k]);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(y) + base) =
        make_uint2(h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16));
  }
}

hipError_t launch_gated_rmsnorm(const Geom &g, int64_t rows, const float *o, const void *z,
                                const float *w, float eps, void *y, hipStream_t s) {
  const int64_t groups = rows * g.H_v;
  if (groups == 0) return hipSuccess;
  const int64_t lanes = groups * (g.D / 4);
  const dim3 grid(static_cast<unsigned>((lanes + 255) / 256));
  if (g.D == 128) {
#define GDN_NORM(ZT, OC) hipLaunchKernelGGL((gated_rmsnorm_kernel<128, ZT, OC>), grid, dim3(256), 0, s, groups, o, z, w, eps, y)
    GDN_OUT_DISPATCH(g.in_dt, out_code(g.out_dt, z), GDN_NORM);
#undef GDN_NORM
  } else {
#define GDN_NORM(ZT, OC) hipLaunchKernelGGL((gated_rmsnorm_kernel<16, ZT, OC>), grid, dim3(256), 0, s, groups, o, z, w, eps, y)
    GDN_OUT_DISPATCH(g.in_dt, out_code(g.out_dt, z), GDN_NORM);
#undef GDN_NORM
  }
  return hipGetLastError();
}

}  // namespace gdn
