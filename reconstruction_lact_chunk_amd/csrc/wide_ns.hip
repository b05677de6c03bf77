// Newton-Schulz step for the full-width head (d = 1024, h = 2048): the same
// iteration as newton_schulz.hip (review of ZipMap, the update display after
// Eq. (3); Muon's odd quintic, five steps of X <- a X + (b A + c A^2) X with
// A = X X^T, from X = G / max(||G||_F, 1e-12)), for matrices of 1024 x 2048
// that do not fit one compute unit.  Each product runs as library GEMMs over
// all 3 H matrices at once (strided batch), in split-bf16: every fp32 operand
// is stored as a bf16 high part and a bf16 low part, and a product is
// hi*hi + hi*lo + lo*hi accumulated in fp32 (three GEMMs, the second and
// third adding into the first's result).  Elementwise kernels do the
// transposes, the norm, the splits and the polynomial's combinations.
#include "gemm_lt.h"
#include "wide_path.h"

namespace zm {
namespace {

constexpr float kNsA = 3.4445f;
constexpr float kNsB = -4.7750f;
constexpr float kNsC = 2.0315f;
constexpr int kNsSteps = 5;
constexpr int kNormChunks = 64;  // first-stage partial sums per matrix

__device__ __forceinline__ void split2(float x, uint16_t& hi, uint16_t& lo) {
  hi = to_bf16(x);
  lo = to_bf16(x - __uint_as_float((unsigned)hi << 16));
}

// X [3 H][M][N] from the summed partials [H][3][h d]: W1 and W3 gradients are
// [h][d] = [N][M] and are transposed, the W2 gradient is [d][h] = [M][N].
// dir = 0 gathers into X, dir = 1 scatters X back.  32 x 32 tiles through LDS.
__global__ __launch_bounds__(256) void k_ns_move(float* __restrict__ part0,
                                                 float* __restrict__ x, int M, int N, int dir) {
  __shared__ float tile[32][33];
  const int mi = blockIdx.z, mat = mi % 3;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;  // X tile rows i (M), columns j (N)
  float* xm = x + (int64_t)mi * M * N;
  float* pm = part0 + (int64_t)mi * M * N;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  if (mat == 2) {  // same layout: a plain copy
    for (int r = ty; r < 32; r += 8) {
      const int64_t o = (int64_t)(i0 + r) * N + j0 + tx;
      if (dir == 0) xm[o] = pm[o];
      else pm[o] = xm[o];
    }
    return;
  }
  if (dir == 0) {  // X[i][j] = P[j][i]
    for (int r = ty; r < 32; r += 8) tile[r][tx] = pm[(int64_t)(j0 + r) * M + i0 + tx];
    __syncthreads();
    for (int r = ty; r < 32; r += 8) xm[(int64_t)(i0 + r) * N + j0 + tx] = tile[tx][r];
  } else {         // P[j][i] = X[i][j]
    for (int r = ty; r < 32; r += 8) tile[r][tx] = xm[(int64_t)(i0 + r) * N + j0 + tx];
    __syncthreads();
    for (int r = ty; r < 32; r += 8) pm[(int64_t)(j0 + r) * M + i0 + tx] = tile[tx][r];
  }
}

// First stage of ||X_m||_F^2: block (c, m) sums a contiguous slice in a fixed order.
__global__ __launch_bounds__(256) void k_ns_sumsq(const float* __restrict__ x, float* __restrict__ part,
                                                  int64_t per_mat) {
  __shared__ float red[4];
  const int mi = blockIdx.y, c = blockIdx.x;
  const int64_t len = per_mat / kNormChunks;
  const float* p = x + (int64_t)mi * per_mat + c * len;
  float s = 0.f;
  for (int64_t e = threadIdx.x; e < len; e += 256) s = fmaf(p[e], p[e], s);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) part[mi * kNormChunks + c] = (red[0] + red[1]) + (red[2] + red[3]);
}

// X_m <- X_m / max(||X_m||_F, 1e-12) and its bf16 planes.  One thread per 4
// elements; every thread adds the chunk sums in the same order.
__global__ __launch_bounds__(256) void k_ns_normalize_split(float* __restrict__ x,
                                                            uint16_t* __restrict__ hi,
                                                            uint16_t* __restrict__ lo,
                                                            const float* __restrict__ part,
                                                            int64_t per_mat) {
  const int mi = blockIdx.y;
  const int64_t e = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (e >= per_mat) return;
  float ss = 0.f;
  for (int c = 0; c < kNormChunks; ++c) ss += part[mi * kNormChunks + c];
  const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
  const int64_t o = (int64_t)mi * per_mat + e;
  f32x4 v = *(const f32x4*)(x + o);
  v *= inv;
  *(f32x4*)(x + o) = v;
  uint16_t h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) split2(v[q], h[q], l[q]);
  *(u32x2*)(hi + o) = u32x2{h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16)};
  *(u32x2*)(lo + o) = u32x2{l[0] | ((unsigned)l[1] << 16), l[2] | ((unsigned)l[3] << 16)};
}

// out = alpha * u + beta * v (v may be null), written back to u when
// write_u, and split into bf16 planes.  One thread per 4 elements.
__global__ __launch_bounds__(256) void k_ns_combine_split(float* __restrict__ u,
                                                          const float* __restrict__ v, float alpha,
                                                          float beta, int write_u,
                                                          uint16_t* __restrict__ hi,
                                                          uint16_t* __restrict__ lo, int64_t count) {
  const int64_t e = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (e >= count) return;
  f32x4 r = alpha * *(const f32x4*)(u + e);
  if (v) r += beta * *(const f32x4*)(v + e);
  if (write_u) *(f32x4*)(u + e) = r;
  uint16_t h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) split2(r[q], h[q], l[q]);
  *(u32x2*)(hi + e) = u32x2{h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16)};
  *(u32x2*)(lo + e) = u32x2{l[0] | ((unsigned)l[1] << 16), l[2] | ((unsigned)l[3] << 16)};
}

#define NS_HIP(expr)                                                      \
  do {                                                                    \
    const hipError_t _e = (expr);                                         \
    if (_e != hipSuccess) {                                               \
      set_last_error("%s: %s", #expr, hipGetErrorString(_e));             \
      return ZM_ERR_HIP;                                                  \
    }                                                                     \
  } while (0)

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct NsBufs {
  float *x, *a, *c, *p, *norm;
  uint16_t *xh, *xl, *ah, *al;
};

NsBufs carve(void* base, int nm, int64_t M, int64_t N) {
  char* q = (char*)base;
  NsBufs b;
  auto take = [&](size_t bytes) {
    char* r = q;
    q += align256(bytes);
    return r;
  };
  b.x = (float*)take(nm * M * N * 4);
  b.p = (float*)take(nm * M * N * 4);
  b.a = (float*)take(nm * M * M * 4);
  b.c = (float*)take(nm * M * M * 4);
  b.xh = (uint16_t*)take(nm * M * N * 2);
  b.xl = (uint16_t*)take(nm * M * N * 2);
  b.ah = (uint16_t*)take(nm * M * M * 2);
  b.al = (uint16_t*)take(nm * M * M * 2);
  b.norm = (float*)take(nm * kNormChunks * 4);
  return b;
}

// Split product sum: D = Ah Bh + Ah Bl + Al Bh through `prod` (a GEMM taking
// the two operands and beta).
template <class F>
bool split_product(F&& prod, const uint16_t* ah, const uint16_t* al, const uint16_t* bh,
                   const uint16_t* bl) {
  return prod(ah, bh, 0.f) && prod(ah, bl, 1.f) && prod(al, bh, 1.f);
}

}  // namespace

size_t wide_ns_bytes(int heads, int d, int h) {
  const int64_t nm = 3 * (int64_t)heads, M = d, N = h;
  return align256(nm * M * N * 4) * 2 + align256(nm * M * M * 4) * 2 + align256(nm * M * N * 2) * 2 +
         align256(nm * M * M * 2) * 2 + align256(nm * kNormChunks * 4);
}

int wide_newton_schulz(float* part0, int heads, int d, int h, void* ns_ws, void* lt_ws,
                       size_t lt_bytes, hipStream_t st) {
  const int nm = 3 * heads;
  const int64_t M = d, N = h, MN = M * N, MM = M * M;
  const NsBufs b = carve(ns_ws, nm, M, N);
  const LtWs lt{lt_ws, lt_bytes};
  hipLaunchKernelGGL(k_ns_move, dim3((unsigned)(N / 32), (unsigned)(M / 32), nm), dim3(256), 0, st,
                     part0, b.x, (int)M, (int)N, 0);
  NS_HIP(hipGetLastError());
  hipLaunchKernelGGL(k_ns_sumsq, dim3(kNormChunks, nm), dim3(256), 0, st, b.x, b.norm, MN);
  NS_HIP(hipGetLastError());
  hipLaunchKernelGGL(k_ns_normalize_split, dim3((unsigned)ceil_div(MN / 4, 256), nm), dim3(256), 0,
                     st, b.x, b.xh, b.xl, b.norm, MN);
  NS_HIP(hipGetLastError());
  const unsigned g_mm = (unsigned)ceil_div(nm * MM / 4, 256), g_mn = (unsigned)ceil_div(nm * MN / 4, 256);
  for (int step = 0; step < kNsSteps; ++step) {
    // A = X X^T  (M x M, contraction over N)
    auto pa = [&](const uint16_t* u, const uint16_t* v, float beta) {
      return lt_rm_nt(M, M, N, u, N, v, N, b.a, M, true, lt, st, nm, MN, MN, MM, beta);
    };
    if (!split_product(pa, b.xh, b.xl, b.xh, b.xl)) return ZM_ERR_HIP;
    hipLaunchKernelGGL(k_ns_combine_split, dim3(g_mm), dim3(256), 0, st, b.a, nullptr, 1.f, 0.f, 0,
                       b.ah, b.al, nm * MM);
    NS_HIP(hipGetLastError());
    // C = A A^T = A^2 (A symmetric)
    auto pc = [&](const uint16_t* u, const uint16_t* v, float beta) {
      return lt_rm_nt(M, M, M, u, M, v, M, b.c, M, true, lt, st, nm, MM, MM, MM, beta);
    };
    if (!split_product(pc, b.ah, b.al, b.ah, b.al)) return ZM_ERR_HIP;
    // B = b A + c C, its planes in place of A's
    hipLaunchKernelGGL(k_ns_combine_split, dim3(g_mm), dim3(256), 0, st, b.a, b.c, kNsB, kNsC, 0,
                       b.ah, b.al, nm * MM);
    NS_HIP(hipGetLastError());
    // P = B X (B symmetric, taken as B^T X)
    auto pp = [&](const uint16_t* u, const uint16_t* v, float beta) {
      return lt_rm_tn(M, N, M, u, M, v, N, b.p, N, true, lt, st, nm, MM, MN, MN, beta);
    };
    if (!split_product(pp, b.ah, b.al, b.xh, b.xl)) return ZM_ERR_HIP;
    // X = a X + P, and its planes
    hipLaunchKernelGGL(k_ns_combine_split, dim3(g_mn), dim3(256), 0, st, b.x, b.p, kNsA, 1.f, 1,
                       b.xh, b.xl, nm * MN);
    NS_HIP(hipGetLastError());
  }
  hipLaunchKernelGGL(k_ns_move, dim3((unsigned)(N / 32), (unsigned)(M / 32), nm), dim3(256), 0, st,
                     part0, b.x, (int)M, (int)N, 1);
  NS_HIP(hipGetLastError());
  return ZM_OK;
}

}  // namespace zm
