// fp32 path of the TTT layer: the same update and apply as the bf16 kernels,
// with fp32 inputs, fp32 weights and fp32 arithmetic throughout (vector FMA,
// no matrix cores).  It serves fp32 callers and tight-tolerance validation.
//
// Update (review of ZipMap, kimjy99.github.io, Method 2, Eq. (1)-(3)): minus
// the chunk gradient of sum_i eta_i * (-f(k_i)^T v_i) is accumulated per
// chunk as
//   D1 += (eta e (*) b (*) SiLU'(a)) k^T,  D3 += (eta e (*) SiLU(a)) k^T,
//   D2 += v (eta SiLU(a) (*) b)^T,   a = W1 k, b = W3 k, e = W2^T v,
// into the same partial-sum layout the bf16 kernel writes, so the shared
// reduce kernel finishes the step.  Apply: Eq. (4), o = f_W(q).
#include "zm_internal.h"

namespace zm {

constexpr int kTokF32 = 16;

template <int D, int HID>
__global__ __launch_bounds__(256) void k_update_f32(const float* __restrict__ kp,
                                                    const float* __restrict__ vp,
                                                    const float* __restrict__ eta, int64_t n,
                                                    int64_t ld, int heads,
                                                    const float* __restrict__ w1,
                                                    const float* __restrict__ w2,
                                                    const float* __restrict__ w3,
                                                    float* __restrict__ part, int splits,
                                                    int64_t chunk) {
  constexpr int TF = kTokF32, HS = kHidPerWgF32, NSL = HID / HS, DR = D / 4;
  __shared__ float ks[TF][D], vs[TF][D], es[TF];
  __shared__ float gas[TF][HS], gbs[TF][HS], ugs[TF][HS];

  const int slice = blockIdx.x % NSL;
  const int pair = blockIdx.x / NSL;
  const int head = pair % heads, chunk_id = pair / heads;
  const int64_t t_begin = (int64_t)chunk_id * chunk;
  const int64_t t_end = (t_begin + chunk < n) ? t_begin + chunk : n;

  const int tid = threadIdx.x;
  const int hid = tid % HS, quarter = tid / HS;
  const int j = slice * HS + hid;
  const int d0 = quarter * DR;
  const float* w1r = w1 + ((int64_t)head * HID + j) * D;
  const float* w3r = w3 + ((int64_t)head * HID + j) * D;
  const float* w2c = w2 + (int64_t)head * D * HID + j;  // column j, stride HID

  float a1[DR], a3[DR], a2[DR];
#pragma unroll
  for (int i = 0; i < DR; ++i) a1[i] = a3[i] = a2[i] = 0.f;

  for (int64_t t0 = t_begin; t0 < t_end; t0 += TF) {
    for (int i = tid; i < TF * D; i += 256) {
      const int tok = i / D, dd = i - (i / D) * D;
      const int64_t t = t0 + tok;
      float kv = 0.f, vv = 0.f;
      if (t < t_end) {
        kv = kp[t * ld + (int64_t)head * D + dd];
        vv = vp[t * ld + (int64_t)head * D + dd];
      }
      ks[tok][dd] = kv;
      vs[tok][dd] = vv;
    }
    if (tid < TF) {
      const int64_t t = t0 + tid;
      es[tid] = t < t_end ? eta[t * heads + head] : 0.f;
    }
    __syncthreads();
    // forward for tokens quarter, quarter + 4, quarter + 8, quarter + 12
    float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f}, e[4] = {0.f, 0.f, 0.f, 0.f};
    for (int dd = 0; dd < D; ++dd) {
      const float x1 = w1r[dd], x3 = w3r[dd], x2 = w2c[(int64_t)dd * HID];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = quarter + 4 * r;
        a[r] = fmaf(x1, ks[tok][dd], a[r]);
        b[r] = fmaf(x3, ks[tok][dd], b[r]);
        e[r] = fmaf(x2, vs[tok][dd], e[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = quarter + 4 * r;
      const float sg = 1.f / (1.f + expf(-a[r]));
      const float s = a[r] * sg;
      const float ee = es[tok] * e[r];
      gas[tok][hid] = ee * b[r] * (sg + s * (1.f - sg));
      gbs[tok][hid] = ee * s;
      ugs[tok][hid] = es[tok] * s * b[r];
    }
    __syncthreads();
    for (int tok = 0; tok < TF; ++tok) {
      const float ga = gas[tok][hid], gb = gbs[tok][hid], u = ugs[tok][hid];
#pragma unroll
      for (int i = 0; i < DR; ++i) {
        const float kk = ks[tok][d0 + i];
        a1[i] = fmaf(ga, kk, a1[i]);
        a3[i] = fmaf(gb, kk, a3[i]);
        a2[i] = fmaf(u, vs[tok][d0 + i], a2[i]);
      }
    }
    __syncthreads();
  }
  const int64_t hd_elems = (int64_t)HID * D;
  float* P = part + ((int64_t)chunk_id * heads + head) * 3 * hd_elems;
#pragma unroll
  for (int i = 0; i < DR; ++i) {
    P[(int64_t)j * D + d0 + i] = a1[i];
    P[hd_elems + (int64_t)j * D + d0 + i] = a3[i];
    P[2 * hd_elems + (int64_t)(d0 + i) * HID + j] = a2[i];
  }
}

template <int D, int HID>
__global__ __launch_bounds__(256) void k_apply_f32(const float* __restrict__ qp,
                                                   float* __restrict__ op, int64_t n, int64_t ld,
                                                   int heads, const float* __restrict__ w1,
                                                   const float* __restrict__ w2,
                                                   const float* __restrict__ w3) {
  constexpr int TF = kTokF32;
  __shared__ float qs[TF][D];
  __shared__ float us[TF][HID];
  const int head = blockIdx.x % heads;
  const int64_t t0 = (int64_t)(blockIdx.x / heads) * TF;
  const int tid = threadIdx.x;
  for (int i = tid; i < TF * D; i += 256) {
    const int tok = i / D, dd = i - (i / D) * D;
    const int64_t t = t0 + tok;
    qs[tok][dd] = t < n ? qp[t * ld + (int64_t)head * D + dd] : 0.f;
  }
  __syncthreads();
  for (int j = tid; j < HID; j += 256) {
    float a[TF], b[TF];
#pragma unroll
    for (int t = 0; t < TF; ++t) a[t] = b[t] = 0.f;
    const float* w1r = w1 + ((int64_t)head * HID + j) * D;
    const float* w3r = w3 + ((int64_t)head * HID + j) * D;
    for (int dd = 0; dd < D; ++dd) {
      const float x1 = w1r[dd], x3 = w3r[dd];
#pragma unroll
      for (int t = 0; t < TF; ++t) {
        a[t] = fmaf(x1, qs[t][dd], a[t]);
        b[t] = fmaf(x3, qs[t][dd], b[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < TF; ++t) {
      const float sg = 1.f / (1.f + expf(-a[t]));
      us[t][j] = a[t] * sg * b[t];
    }
  }
  __syncthreads();
  for (int i = tid; i < TF * D; i += 256) {
    const int tok = i / D, dd = i - (i / D) * D;
    const int64_t t = t0 + tok;
    if (t >= n) continue;
    const float* w2r = w2 + ((int64_t)head * D + dd) * HID;
    float s = 0.f;
    for (int jj = 0; jj < HID; ++jj) s = fmaf(w2r[jj], us[tok][jj], s);
    op[t * ld + (int64_t)head * D + dd] = s;
  }
}

hipError_t launch_update_f32(const float* k, const float* v, const float* eta, int64_t n,
                             int64_t ld, int heads, int d, int h, const float* w1,
                             const float* w2, const float* w3, float* part, UpdatePlan plan,
                             hipStream_t st) {
  if (plan.splits <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((int64_t)heads * plan.splits * (h / kHidPerWgF32));
#define ZM_LAUNCH(DD, HH)                                                                     \
  hipLaunchKernelGGL((k_update_f32<DD, HH>), dim3(blocks), dim3(256), 0, st, k, v, eta, n, ld, \
                     heads, w1, w2, w3, part, plan.splits, plan.chunk)
  if (d == 128 && h == 256) ZM_LAUNCH(128, 256);
  else if (d == 128 && h == 128) ZM_LAUNCH(128, 128);
  else if (d == 64 && h == 256) ZM_LAUNCH(64, 256);
  else if (d == 64 && h == 128) ZM_LAUNCH(64, 128);
  else return hipErrorInvalidValue;
#undef ZM_LAUNCH
  return hipGetLastError();
}

hipError_t launch_apply_f32(const float* q, float* o, int64_t n, int64_t ld, int heads, int d,
                            int h, const float* w1, const float* w2, const float* w3,
                            hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((int64_t)heads * ceil_div(n, kTokF32));
#define ZM_LAUNCH(DD, HH)                                                                       \
  hipLaunchKernelGGL((k_apply_f32<DD, HH>), dim3(blocks), dim3(256), 0, st, q, o, n, ld, heads, \
                     w1, w2, w3)
  if (d == 128 && h == 256) ZM_LAUNCH(128, 256);
  else if (d == 128 && h == 128) ZM_LAUNCH(128, 128);
  else if (d == 64 && h == 256) ZM_LAUNCH(64, 256);
  else if (d == 64 && h == 128) ZM_LAUNCH(64, 128);
  else return hipErrorInvalidValue;
#undef ZM_LAUNCH
  return hipGetLastError();
}

}  // namespace zm
