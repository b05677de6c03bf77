// Newton-Schulz orthonormalisation of the chunk gradient, the update rule of
// the review of ZipMap (kimjy99.github.io), Method 2, the update display after
// Eq. (3): Delta = NewtonSchulz(g), after the Muon optimizer, then
// W' = W - Delta and the norm-preserving renorm.  The pages give neither the
// polynomial nor the step count; this library uses Muon's published odd
// quintic (K. Jordan, "Muon: An optimizer for hidden layers in neural
// networks", 2024): five steps of
//     X <- a X + (b A + c A^2) X,   A = X X^T,   (a, b, c) = (3.4445, -4.7750, 2.0315)
// from X_0 = G / max(||G||_F, 1e-12).
//
// The step runs on the summed partials D = -g (the update kernels accumulate
// minus the gradient); the polynomial is odd, so NewtonSchulz(D) =
// -NewtonSchulz(g) and W + NewtonSchulz(D) is the step.
//
// One workgroup per (head, matrix): the matrix is small (at most 256 x 128)
// and every step needs all of it, so it stays on one compute unit for all
// five steps.  X is taken in the orientation with fewer rows (M = d rows,
// N = h columns; W1 and W3 gradients, [h][d], are transposed on the way in and
// out), so the Gram matrix A is M x M.  The X master copy lives in registers
// (fp32) in the output layout of the product B X; the three products of a
// step read their operands from LDS:
//   A = X X^T        operands: X row-major, contraction over N
//   C = A A^T        operands: A (stored transposed; A is symmetric)
//   X' = a X + B X   operands: B (stored transposed), X^T row-major
// X is staged in panels of 128 columns so that two LDS regions of about
// 70 KB each suffice.  Fragments are read conflict-free (row pitch = 32 bytes
// modulo 256).
//
// Two product policies:
//   Split3: bf16 matrix cores with each fp32 operand split into a bf16 high
//           part and a bf16 low part (x = hi + lo to about 2^-17); a product
//           takes hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_bf16 with fp32
//           accumulation (relative error about 1e-5 per product);
//   F32:    v_mfma_f32_16x16x4_f32, fp32 operands (the fp32 validation path).
#include "zm_internal.h"

namespace zm {

constexpr float kNsA = 3.4445f;
constexpr float kNsB = -4.7750f;
constexpr float kNsC = 2.0315f;
constexpr int kNsSteps = 5;

// ---- product policies ------------------------------------------------------
struct NsSplit3 {
  typedef uint16_t T;
  static constexpr int PLANES = 2;
  static constexpr int PAD = 16;   // elements: 32 bytes, pitch = 32 mod 256 bytes
  static constexpr int KB = 32;    // contraction per fragment step
  struct Frag {
    bf16x8 hi, lo;
  };
  // 8 consecutive elements at p (16-byte aligned) of each plane
  static __device__ __forceinline__ Frag load(const T* plane0, int plane_elems, int off) {
    return Frag{as_bf16x8(*(const u32x4*)(plane0 + off)),
                as_bf16x8(*(const u32x4*)(plane0 + plane_elems + off))};
  }
  static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b) {
    acc = mfma_bf16(a.lo, b.hi, acc);
    acc = mfma_bf16(a.hi, b.lo, acc);
    acc = mfma_bf16(a.hi, b.hi, acc);
  }
  static __device__ __forceinline__ void split(float x, uint16_t& hi, uint16_t& lo) {
    hi = to_bf16(x);
    lo = to_bf16(x - __uint_as_float((unsigned)hi << 16));
  }
  static __device__ __forceinline__ void store1(T* plane0, int plane_elems, int off, float x) {
    uint16_t h, l;
    split(x, h, l);
    plane0[off] = h;
    plane0[plane_elems + off] = l;
  }
  // 4 consecutive elements (8-byte aligned) as hi + lo (exact in fp32)
  static __device__ __forceinline__ f32x4 load4(const T* plane0, int plane_elems, int off) {
    const u32x2 h = *(const u32x2*)(plane0 + off);
    const u32x2 l = *(const u32x2*)(plane0 + plane_elems + off);
    return f32x4{bf16lo(h[0]) + bf16lo(l[0]), bf16hi(h[0]) + bf16hi(l[0]),
                 bf16lo(h[1]) + bf16lo(l[1]), bf16hi(h[1]) + bf16hi(l[1])};
  }
  // 4 consecutive elements (8-byte aligned)
  static __device__ __forceinline__ void store4(T* plane0, int plane_elems, int off,
                                                const f32x4& x) {
    uint16_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split(x[i], h[i], l[i]);
    *(u32x2*)(plane0 + off) = u32x2{h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16)};
    *(u32x2*)(plane0 + plane_elems + off) =
        u32x2{l[0] | ((unsigned)l[1] << 16), l[2] | ((unsigned)l[3] << 16)};
  }
};

struct NsF32 {
  typedef float T;
  static constexpr int PLANES = 1;
  static constexpr int PAD = 8;
  static constexpr int KB = 16;    // four 16x16x4 products per fragment step
  typedef f32x4 Frag;
  static __device__ __forceinline__ Frag load(const T* plane0, int, int off) {
    return *(const f32x4*)(plane0 + off);
  }
  // Lane group g supplies contraction index k0 + 4 g + s to product s, the
  // same for both operands, so the four products cover k0 .. k0 + 15.
  static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 load4(const T* plane0, int, int off) {
    return *(const f32x4*)(plane0 + off);
  }
  static __device__ __forceinline__ void store1(T* plane0, int, int off, float x) { plane0[off] = x; }
  static __device__ __forceinline__ void store4(T* plane0, int, int off, const f32x4& x) {
    *(f32x4*)(plane0 + off) = x;
  }
};

template <int M, int N, class P>
struct NsCfg {
  static constexpr int PW = N < 128 ? N : 128;      // X panel width (columns)
  static constexpr int NP = N / PW;                 // panels
  static constexpr int RB = M / 64;                 // 16-row blocks per wave tile
  static constexpr int CB1 = M / 32;                // 16-col blocks per wave tile of A, C
  static constexpr int CB3 = PW / 32;               // 16-col blocks per wave tile of X'
  // Region P holds X_p (M x PW) or X_p^T (PW x M); region Q holds A or B (M x M).
  static constexpr int PITCH_X = PW + P::PAD;       // X_p rows
  static constexpr int PITCH_XT = M + P::PAD;       // X_p^T rows and A / B rows
  static constexpr int PLANE_P = (M * PITCH_X > PW * PITCH_XT) ? M * PITCH_X : PW * PITCH_XT;
  static constexpr int PLANE_Q = M * PITCH_XT;
  static constexpr int LDS_ELEMS = P::PLANES * (PLANE_P + PLANE_Q);
  static_assert(M == 64 || M == 128, "M");
  static_assert(N % PW == 0 && PW % 64 == 0, "N");
  // 8 waves: 4 row tiles x 2 column tiles for every product
  static_assert((M / (16 * RB)) * (M / (16 * CB1)) == kWaves, "A tiling");
  static_assert((M / (16 * RB)) * (PW / (16 * CB3)) == kWaves, "X tiling");
};

// One product: acc[RB][CB] += S1[rows r0 + 16 rb ..] . S2[rows c0 + 16 cb ..]^T
// over a contraction of K; S1 and S2 are stored row-major (contraction index
// along the row), each as P::PLANES planes of pe elements with its own pitch.
template <class P, int RB, int CB, int K>
__device__ __forceinline__ void ns_product(f32x4 (&acc)[RB][CB], const typename P::T* s1,
                                           int pe1, int pitch1, const typename P::T* s2, int pe2,
                                           int pitch2, int r0, int c0, int lane) {
  const int c = lane & 15, g = lane >> 4;
  constexpr int KOFF = P::KB / 4;  // elements per lane group per fragment step
  const typename P::T* a0 = s1 + (r0 + c) * pitch1 + KOFF * g;
  const typename P::T* b0 = s2 + (c0 + c) * pitch2 + KOFF * g;
#pragma unroll 2
  for (int k0 = 0; k0 < K; k0 += P::KB) {
    typename P::Frag fa[RB], fb[CB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) fa[rb] = P::load(a0, pe1, 16 * rb * pitch1 + k0);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) fb[cb] = P::load(b0, pe2, 16 * cb * pitch2 + k0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) P::mma(acc[rb][cb], fa[rb], fb[cb]);
  }
}

// Stores an accumulator tile transposed: element (r0 + 16 rb + 4 g + i,
// c0 + 16 cb + c) goes to row c0 + 16 cb + c, column r0 + 16 rb + 4 g + i.
template <class P, int RB, int CB>
__device__ __forceinline__ void ns_store_t(typename P::T* dst, int plane_elems, int pitch,
                                           const f32x4 (&acc)[RB][CB], int r0, int c0, int lane) {
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      P::store4(dst, plane_elems, (c0 + 16 * cb + c) * pitch + r0 + 16 * rb + 4 * g, acc[rb][cb]);
}

// Reads back a tile stored by ns_store_t, in the accumulator layout.
template <class P, int RB, int CB>
__device__ __forceinline__ void ns_load_t(f32x4 (&acc)[RB][CB], const typename P::T* src,
                                          int plane_elems, int pitch, int r0, int c0, int lane) {
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      acc[rb][cb] = P::load4(src, plane_elems, (c0 + 16 * cb + c) * pitch + r0 + 16 * rb + 4 * g);
}

// Grid: heads * 3 workgroups, one per (head, matrix); 512 threads.
// g: [heads][3][h*d] fp32 (W1, W3 as [h][d], W2 as [d][h]), overwritten in
// place by NewtonSchulz of each matrix.
template <int D, int HID, class P>
__global__ __launch_bounds__(512) void k_newton_schulz(float* __restrict__ g) {
  constexpr int M = D, N = HID;
  using C = NsCfg<M, N, P>;
  constexpr int RB = C::RB, CB1 = C::CB1, CB3 = C::CB3, NP = C::NP, PW = C::PW;
  typedef typename P::T T;
  __shared__ __attribute__((aligned(16))) T lds[C::LDS_ELEMS];
  __shared__ float red[kWaves];
  T* const rp = lds;                             // region P
  T* const rq = lds + P::PLANES * C::PLANE_P;    // region Q

  const int mat = blockIdx.x % 3;
  float* const gm = g + (int64_t)blockIdx.x * M * N;
  // W1, W3 gradients are [h][d] = N x M: X = G^T.  W2's is [d][h] = M x N.
  const bool tr = (mat < 2) && (N > M);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, gq = l >> 4;
  const int r0 = (w >> 1) * 16 * RB;             // wave tile row (all products)
  const int c01 = (w & 1) * 16 * CB1;            // wave tile column of A, C
  const int c03 = (w & 1) * 16 * CB3;            // wave tile column of X' in a panel

  // X master: element (r0 + 16 rb + 4 gq + i, p PW + c03 + 16 cb + c)
  f32x4 xm[NP][RB][CB3];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB3; ++cb) {
        const int i0 = r0 + 16 * rb + 4 * gq, j = p * PW + c03 + 16 * cb + c;
        f32x4 x;
        if (tr) {
          x = *(const f32x4*)(gm + (int64_t)j * M + i0);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = gm[(int64_t)(i0 + i) * N + j];
        }
        xm[p][rb][cb] = x;
#pragma unroll
        for (int i = 0; i < 4; ++i) ss = fmaf(x[i], x[i], ss);
      }
  // Frobenius norm: butterfly within the wave, then the 8 wave sums in a
  // fixed order (every thread gets the same bits).
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if (l == 0) red[w] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) tot += red[i];
  const float inv = 1.f / fmaxf(sqrtf(tot), 1e-12f);
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB3; ++cb) xm[p][rb][cb] *= inv;

  for (int step = 0; step < kNsSteps; ++step) {
    // ---- A = X X^T, panel by panel
    f32x4 acc_a[RB][CB1];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB1; ++cb) acc_a[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      __syncthreads();  // earlier readers of region P are done
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB3; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            P::store1(rp, C::PLANE_P, (r0 + 16 * rb + 4 * gq + i) * C::PITCH_X + c03 + 16 * cb + c,
                      xm[p][rb][cb][i]);
      // X is stored again (transposed) for X'; pinning it here stops the
      // compiler from keeping this store's bf16 splits live until then
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB3; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float t = xm[p][rb][cb][i];
            pin(t);
            xm[p][rb][cb][i] = t;
          }
      __syncthreads();
      ns_product<P, RB, CB1, PW>(acc_a, rp, C::PLANE_P, C::PITCH_X, rp, C::PLANE_P, C::PITCH_X,
                                 r0, c01, l);
    }
    // ---- C = A A^T (A symmetric: its transposed store serves as A)
    __syncthreads();  // region Q free (last read by the previous step's X')
    ns_store_t<P, RB, CB1>(rq, C::PLANE_Q, C::PITCH_XT, acc_a, r0, c01, l);
    __syncthreads();
    f32x4 acc_b[RB][CB1];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB1; ++cb) acc_b[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    ns_product<P, RB, CB1, M>(acc_b, rq, C::PLANE_Q, C::PITCH_XT, rq, C::PLANE_Q, C::PITCH_XT,
                              r0, c01, l);
    // ---- B = b A + c A^2, A read back from its stored copy (hi + lo is A to
    // 2^-17 with split-bf16, exact with fp32) so that its accumulators need
    // not stay live across the product
    ns_load_t<P, RB, CB1>(acc_a, rq, C::PLANE_Q, C::PITCH_XT, r0, c01, l);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB1; ++cb) acc_b[rb][cb] = kNsB * acc_a[rb][cb] + kNsC * acc_b[rb][cb];
    __syncthreads();  // all reads of A done
    ns_store_t<P, RB, CB1>(rq, C::PLANE_Q, C::PITCH_XT, acc_b, r0, c01, l);
    // ---- X' = a X + B X, panel by panel
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (p > 0) __syncthreads();  // the previous panel's reads of region P are done
      ns_store_t<P, RB, CB3>(rp, C::PLANE_P, C::PITCH_XT, xm[p], r0, c03, l);
      __syncthreads();
      f32x4 acc[RB][CB3];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB3; ++cb) acc[rb][cb] = kNsA * xm[p][rb][cb];
      ns_product<P, RB, CB3, M>(acc, rq, C::PLANE_Q, C::PITCH_XT, rp, C::PLANE_P, C::PITCH_XT,
                                r0, c03, l);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB3; ++cb) xm[p][rb][cb] = acc[rb][cb];
    }
  }

  // ---- write back in the matrix's own orientation
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB3; ++cb) {
        const int i0 = r0 + 16 * rb + 4 * gq, j = p * PW + c03 + 16 * cb + c;
        if (tr) {
          *(f32x4*)(gm + (int64_t)j * M + i0) = xm[p][rb][cb];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) gm[(int64_t)(i0 + i) * N + j] = xm[p][rb][cb][i];
        }
      }
}

// Adds the S partial-sum slots of [heads][3][h*d] into slot 0, in slot
// order (fixed order: bitwise reproducible).  One thread per 4 elements.
__global__ __launch_bounds__(256) void k_sum_splits(float* __restrict__ part, int splits,
                                                    int64_t slot) {
  const int64_t e = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (e >= slot) return;
  *(f32x4*)(part + e) = sum_slots(part + e, slot, splits);
}

template <int D, int HID>
hipError_t launch_ns_shape(float* part, int heads, bool f32, hipStream_t st) {
  if (f32) {
    hipLaunchKernelGGL((k_newton_schulz<D, HID, NsF32>), dim3(3 * heads), dim3(512), 0, st, part);
  } else {
    hipLaunchKernelGGL((k_newton_schulz<D, HID, NsSplit3>), dim3(3 * heads), dim3(512), 0, st,
                       part);
  }
  return hipGetLastError();
}

hipError_t launch_sum_splits(float* part, int splits, int heads, int d, int h, hipStream_t st) {
  const int64_t slot = (int64_t)heads * 3 * h * d;
  if (splits <= 1) return hipSuccess;
  const unsigned blocks = (unsigned)ceil_div(slot / 4, 256);
  hipLaunchKernelGGL(k_sum_splits, dim3(blocks), dim3(256), 0, st, part, splits, slot);
  return hipGetLastError();
}

hipError_t launch_newton_schulz(float* part, int splits, int heads, int d, int h, bool f32,
                                hipStream_t st) {
  const hipError_t e = launch_sum_splits(part, splits, heads, d, h, st);
  if (e != hipSuccess) return e;
  if (d == 64 && h == 128) return launch_ns_shape<64, 128>(part, heads, f32, st);
  if (d == 64 && h == 256) return launch_ns_shape<64, 256>(part, heads, f32, st);
  if (d == 128 && h == 128) return launch_ns_shape<128, 128>(part, heads, f32, st);
  if (d == 128 && h == 256) return launch_ns_shape<128, 256>(part, heads, f32, st);
  return hipErrorInvalidValue;
}

}  // namespace zm
