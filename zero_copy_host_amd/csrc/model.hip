// Decode-step kernels around the attention layer, for a multi-layer decode loop: RMSNorm,
// a weight-streaming linear layer for a few rows (Y = X·Wᵀ, optionally + a residual), and
// the SwiGLU gate of the MLP.
//
// In a decode step these touch each weight once for a handful of rows (the batch), so they
// are bound by HBM: a layer of an 8B-shaped model streams ~0.4 GB of weights, ~70 us at
// ~6 TB/s, against ~19 ms of host-link-bound attention. The layouts follow the attention
// layer's conventions: activations [rows, features] row-major, weights [out, in] row-major.
#include "dkv_internal.h"

namespace dkv {

__device__ inline float wsum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// y[r, :] = x[r, :] / sqrt(mean(x[r, :]^2) + eps) * w, fp32 arithmetic, one rounding at the
// store. One 256-thread workgroup per row. y may be x (an in-place norm): x and y are not
// restrict-qualified, and each element is read, then written, by the same thread.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* x, const T* __restrict__ w, T* y, int D, float eps) {
  __shared__ float red[4];
  const T* xr = x + (size_t)blockIdx.x * D;
  T* yr = y + (size_t)blockIdx.x * D;
  float ss = 0.f;
  for (int i = threadIdx.x; i < D; i += 256) {
    const float v = Elem<T>::to_float(xr[i]);
    ss = fmaf(v, v, ss);
  }
  ss = wsum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float inv = 1.f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)D + eps);
  for (int i = threadIdx.x; i < D; i += 256)
    yr[i] = Elem<T>::from_float(Elem<T>::to_float(xr[i]) * inv * Elem<T>::to_float(w[i]));
}

// Y[b, n] = sum_k X[b, k] W[n, k] (+ Res[b, n]) for b < rows <= MB. Each wave owns R
// consecutive output features and streams their weight rows once, 16 bytes per lane per
// step, two steps in flight; the few X rows come from L2 beside them. fp32 accumulation,
// one rounding at the store. Y may alias Res (each element is read, then written, by one lane).
template <typename T, int R, int MB>
__global__ __launch_bounds__(256) void linear_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                     const T* res, T* y, int rows, int N, int K) {
  constexpr int VEC = Elem<T>::VEC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * 4 + wave) * R;
  if (n0 >= N) return;
  float acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[r][b] = 0.f;
  for (int k = lane * VEC; k < K; k += 64 * VEC) {
    uint4 wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      wr[r] = (n0 + r < N) ? *reinterpret_cast<const uint4*>(w + (size_t)(n0 + r) * K + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      if (b >= rows) break;
      float xf[VEC];
      Elem<T>::unpack(*reinterpret_cast<const uint4*>(x + (size_t)b * K + k), xf);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float wf[VEC];
        Elem<T>::unpack(wr[r], wf);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[r][b] = fmaf(wf[e], xf[e], acc[r][b]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      if (b >= rows) break;
      const float v = wsum(acc[r][b]);
      const int n = n0 + r;
      if (lane == 0 && n < N) {
        const size_t o = (size_t)b * N + n;
        y[o] = Elem<T>::from_float(res ? v + Elem<T>::to_float(res[o]) : v);
      }
    }
}

// y[b, j] = silu(gu[b, j]) * gu[b, F + j], silu(z) = z / (1 + exp(-z)); gu is [rows, 2F]
// (the gate projection, then the up projection).
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(const T* __restrict__ gu, T* __restrict__ y, int rows, int F) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)rows * F) return;
  const size_t b = i / F, j = i - b * F;
  const float g = Elem<T>::to_float(gu[b * 2 * F + j]);
  const float u = Elem<T>::to_float(gu[b * 2 * F + F + j]);
  y[i] = Elem<T>::from_float(g / (1.f + expf(-g)) * u);
}

template <typename T>
static hipError_t run_rmsnorm(const void* x, const void* w, void* y, int rows, int D, float eps, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel<T>, dim3(rows), dim3(256), 0, s, reinterpret_cast<const T*>(x),
                     reinterpret_cast<const T*>(w), reinterpret_cast<T*>(y), D, eps);
  return hipGetLastError();
}

template <typename T>
static hipError_t run_linear(const void* x, const void* w, const void* res, void* y, int rows, int N, int K,
                             hipStream_t s) {
  // row groups of at most 16; R = 4 outputs per wave for <= 8 rows, 2 for <= 16
  for (int r0 = 0; r0 < rows; r0 += 16) {
    const int nr = rows - r0 < 16 ? rows - r0 : 16;
    const T* xp = reinterpret_cast<const T*>(x) + (size_t)r0 * K;
    const T* rp = res ? reinterpret_cast<const T*>(res) + (size_t)r0 * N : nullptr;
    T* yp = reinterpret_cast<T*>(y) + (size_t)r0 * N;
    const T* wp = reinterpret_cast<const T*>(w);
    if (nr <= 8) {
      hipLaunchKernelGGL((linear_kernel<T, 4, 8>), dim3((N + 15) / 16), dim3(256), 0, s, xp, wp, rp, yp, nr, N, K);
    } else {
      hipLaunchKernelGGL((linear_kernel<T, 2, 16>), dim3((N + 7) / 8), dim3(256), 0, s, xp, wp, rp, yp, nr, N, K);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T>
static hipError_t run_swiglu(const void* gu, void* y, int rows, int F, hipStream_t s) {
  const size_t n = (size_t)rows * F;
  hipLaunchKernelGGL(swiglu_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const T*>(gu), reinterpret_cast<T*>(y), rows, F);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, const void* x, const void* w, void* y, int rows, int D, float eps,
                          hipStream_t s) {
  switch (dtype) {
    case 0: return run_rmsnorm<float>(x, w, y, rows, D, eps, s);
    case 1: return run_rmsnorm<_Float16>(x, w, y, rows, D, eps, s);
    default: return run_rmsnorm<__bf16>(x, w, y, rows, D, eps, s);
  }
}

hipError_t launch_linear(int dtype, const void* x, const void* w, const void* res, void* y, int rows, int N, int K,
                         hipStream_t s) {
  switch (dtype) {
    case 0: return run_linear<float>(x, w, res, y, rows, N, K, s);
    case 1: return run_linear<_Float16>(x, w, res, y, rows, N, K, s);
    default: return run_linear<__bf16>(x, w, res, y, rows, N, K, s);
  }
}

hipError_t launch_swiglu(int dtype, const void* gu, void* y, int rows, int F, hipStream_t s) {
  switch (dtype) {
    case 0: return run_swiglu<float>(gu, y, rows, F, s);
    case 1: return run_swiglu<_Float16>(gu, y, rows, F, s);
    default: return run_swiglu<__bf16>(gu, y, rows, F, s);
  }
}

}  // namespace dkv
