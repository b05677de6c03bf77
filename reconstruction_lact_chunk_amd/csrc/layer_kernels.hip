// Elementwise ends of the whole TTT layer (around update + apply):
//   k_eta_from_logits  the per-token rate from its linear-layer logits,
//                      eta = scale * sigmoid(z) (review of ZipMap, the note on
//                      the rate under Eq. (3): predicted from the token by a
//                      linear layer; the sigmoid keeps it positive and bounded);
//   k_rmsnorm_gate     the output gate o = RMSNorm(o') * SiLU(g), g = W_g o'
//                      (review Eq. (5)), RMSNorm over the whole width with a
//                      learnable scale gamma: o' / sqrt(mean(o'^2) + eps) * gamma.
// The dense products on either side are plain GEMMs (gemm_lt.cpp).
#include "layer_kernels.h"

namespace zm {

// One thread per (token, head): logits are bf16 columns col0 .. col0 + heads - 1
// of the projection rows (row stride ldy); eta is fp32 [n][heads].
__global__ __launch_bounds__(256) void k_eta_from_logits(const uint16_t* __restrict__ y,
                                                         int64_t ldy, int64_t col0, int heads,
                                                         float scale, float* __restrict__ eta,
                                                         int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * heads) return;
  const int64_t t = i / heads;
  const int hd = (int)(i - t * heads);
  const float z = __uint_as_float((unsigned)y[t * ldy + col0 + hd] << 16);
  eta[i] = scale / (1.f + __expf(-z));
}

// One wave per token: lane l holds the 16-byte pieces c = 8 l + 512 i
// (i < NC) of its row of o' and of g, loaded once into registers (NC 512-wide
// pieces cover the width).  The sum of squares adds the pieces in order and
// ends with a wave butterfly, so every lane holds the same bits.  op, g: bf16
// rows (strides ldo, ldg); o: bf16 rows (stride ldout).  width is a multiple
// of 8 and at most 512 NC.
template <int NC>
__global__ __launch_bounds__(256) void k_rmsnorm_gate(const uint16_t* __restrict__ op,
                                                      int64_t ldo, const uint16_t* __restrict__ g,
                                                      int64_t ldg, const float* __restrict__ gamma,
                                                      float eps, uint16_t* __restrict__ o,
                                                      int64_t ldout, int width, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;
  const int lane = threadIdx.x & 63;
  const uint16_t* orow = op + t * ldo;
  const uint16_t* grow = g + t * ldg;
  u32x4 ov[NC], gv[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = 8 * lane + 512 * i;
    if (c < width) {
      ov[i] = *(const u32x4*)(orow + c);
      gv[i] = *(const u32x4*)(grow + c);
    } else {
      ov[i] = u32x4{0u, 0u, 0u, 0u};
      gv[i] = ov[i];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = bf16lo(ov[i][q]), hi = bf16hi(ov[i][q]);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  const float r = 1.f / sqrtf(ss / (float)width + eps);
  uint16_t* out = o + t * ldout;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = 8 * lane + 512 * i;
    if (c >= width) break;
    const f32x4 ga = *(const f32x4*)(gamma + c), gb = *(const f32x4*)(gamma + c + 4);
    u32x4 res;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[2], gg[2];
      v[0] = bf16lo(ov[i][q]);
      v[1] = bf16hi(ov[i][q]);
      gg[0] = bf16lo(gv[i][q]);
      gg[1] = bf16hi(gv[i][q]);
      float out2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float gm = (2 * q + e) < 4 ? ga[2 * q + e] : gb[2 * q + e - 4];
        const float silu = gg[e] / (1.f + __expf(-gg[e]));
        out2[e] = v[e] * r * gm * silu;
      }
      res[q] = pack_bf16x2(out2[0], out2[1]);
    }
    *(u32x4*)(out + c) = res;
  }
}

hipError_t launch_eta_from_logits(const uint16_t* y, int64_t ldy, int64_t col0, int heads,
                                  float scale, float* eta, int64_t n, hipStream_t st) {
  const int64_t items = n * heads;
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(k_eta_from_logits, dim3((unsigned)ceil_div(items, 256)), dim3(256), 0, st, y,
                     ldy, col0, heads, scale, eta, n);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_gate(const uint16_t* op, int64_t ldo, const uint16_t* g, int64_t ldg,
                               const float* gamma, float eps, uint16_t* o, int64_t ldout,
                               int width, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(n, 4));
#define ZM_LAUNCH_GATE(NC)                                                                    \
  hipLaunchKernelGGL((k_rmsnorm_gate<NC>), grid, dim3(256), 0, st, op, ldo, g, ldg, gamma, eps, \
                     o, ldout, width, n)
  if (width <= 512) ZM_LAUNCH_GATE(1);
  else if (width <= 1024) ZM_LAUNCH_GATE(2);
  else if (width <= 2048) ZM_LAUNCH_GATE(4);
  else if (width <= 4096) ZM_LAUNCH_GATE(8);
  else if (width <= 8192) ZM_LAUNCH_GATE(16);
  else return hipErrorInvalidValue;
#undef ZM_LAUNCH_GATE
  return hipGetLastError();
}

}  // namespace zm
