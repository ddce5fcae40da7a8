// Per-lane row kernels of the decode step on gfx950: embedding gather with the
// first RMSNorm and the lane's rotary table, RMSNorm of the residual stream,
// and the final argmax over the LM head's per-tile candidates.
#include "cbd_internal.h"

namespace cbd {

__device__ inline uint16_t f2bf_m(float f) {
  unsigned u = __builtin_bit_cast(unsigned, f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int ACT>
__device__ inline void put(void* base, size_t idx, float v) {
  if constexpr (ACT == WT_F32)
    ((float*)base)[idx] = v;
  else if constexpr (ACT == WT_BF16)
    ((uint16_t*)base)[idx] = f2bf_m(v);
  else
    ((_Float16*)base)[idx] = (_Float16)v;
}

// Block sum of per-thread partials (256 threads): a fixed shuffle tree, then
// the four waves in order.
__device__ inline float block_sum(float ss) {
  __shared__ float red[4];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float t = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return t;
}

// RMSNorm: out = (x * r) * g, r = 1 / sqrt(mean(x^2) + eps), in the activation format.
template <int ACT>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* x, const float* g, int d, float eps, void* xn) {
  const int b = blockIdx.x;
  const float* xr = x + (size_t)b * d;
  float part = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) part += xr[i] * xr[i];
  const float ss = block_sum(part);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += 256) put<ACT>(xn, (size_t)b * d + i, (xr[i] * r) * g[i]);
}

// x[b] = E[token_b] (exact upcast of bf16, q * scale of Q8_0), then the first
// RMSNorm, and the rotary (cos, sin) of the lane's position for every pair:
// theta_j = theta^(-2j/hd), angle = pos * theta_j, in double, rounded to f32.
template <int WT>
__global__ __launch_bounds__(256) void k_embed_norm(const void* E, const uint16_t* Es, const int* tokens,
                                                    const int* pos, int d, int hd, float theta, float eps,
                                                    const float* g, float* x, void* xn, float2* rope) {
  const int b = blockIdx.x;
  const int tok = tokens[b];
  float* xr = x + (size_t)b * d;
  auto row = [&](int i) -> float {
    if constexpr (WT == WT_F32) {
      return ((const float*)E)[(size_t)tok * d + i];
    } else if constexpr (WT == WT_BF16) {
      return __builtin_bit_cast(float, (unsigned)((const uint16_t*)E)[(size_t)tok * d + i] << 16);
    } else {
      const float q = (float)((const int8_t*)E)[(size_t)tok * d + i];
      const float s = (float)__builtin_bit_cast(_Float16, Es[(size_t)tok * (d / 32) + i / 32]);
      return q * s;
    }
  };
  float part = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) {
    const float v = row(i);
    xr[i] = v;
    part += v * v;
  }
  const float ss = block_sum(part);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += 256) put<WT>(xn, (size_t)b * d + i, (row(i) * r) * g[i]);
  const int p = pos[b];
  for (int j = threadIdx.x; j < hd / 2; j += 256) {
    const double th = pow((double)theta, -(2.0 * (double)j) / (double)hd);
    const double ang = (double)p * th;
    rope[(size_t)b * (hd / 2) + j] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

// argmax[b]: largest value over the LM head's per-row-block candidates, the
// lowest index on ties.  One wave per lane.
__global__ __launch_bounds__(64) void k_argmax(const float2* amax, int nRB, int B, int* out) {
  const int b = blockIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int rb = threadIdx.x; rb < nRB; rb += 64) {
    const float2 e = amax[(size_t)rb * B + b];
    const int i = __float_as_int(e.y);
    if (e.x > best || (e.x == best && i < bi)) {
      best = e.x;
      bi = i;
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float ov = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    if (ov > best || (ov == best && oi < bi)) {
      best = ov;
      bi = oi;
    }
  }
  if (threadIdx.x == 0) out[b] = bi;
}

__global__ void k_fill_u32(unsigned* p, size_t n, unsigned v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_embed_norm(int wt, const void* E, const uint16_t* Es, const int* tokens, const int* pos, int B,
                             int d, int hd, float theta, float eps, const float* g, float* x, void* xn,
                             float2* rope, hipStream_t st) {
  switch (wt) {
    case WT_F32:
      hipLaunchKernelGGL(k_embed_norm<WT_F32>, dim3(B), dim3(256), 0, st, E, Es, tokens, pos, d, hd, theta, eps, g,
                         x, xn, rope);
      break;
    case WT_BF16:
      hipLaunchKernelGGL(k_embed_norm<WT_BF16>, dim3(B), dim3(256), 0, st, E, Es, tokens, pos, d, hd, theta, eps,
                         g, x, xn, rope);
      break;
    default:
      hipLaunchKernelGGL(k_embed_norm<WT_Q8>, dim3(B), dim3(256), 0, st, E, Es, tokens, pos, d, hd, theta, eps, g,
                         x, xn, rope);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int wt, const float* x, const float* g, int B, int d, float eps, void* xn,
                          hipStream_t st) {
  switch (wt) {
    case WT_F32: hipLaunchKernelGGL(k_rmsnorm<WT_F32>, dim3(B), dim3(256), 0, st, x, g, d, eps, xn); break;
    case WT_BF16: hipLaunchKernelGGL(k_rmsnorm<WT_BF16>, dim3(B), dim3(256), 0, st, x, g, d, eps, xn); break;
    default: hipLaunchKernelGGL(k_rmsnorm<WT_Q8>, dim3(B), dim3(256), 0, st, x, g, d, eps, xn); break;
  }
  return hipGetLastError();
}

hipError_t launch_argmax(const float2* amax, int nRB, int B, int* argmax, hipStream_t st) {
  hipLaunchKernelGGL(k_argmax, dim3(B), dim3(64), 0, st, amax, nRB, B, argmax);
  return hipGetLastError();
}

hipError_t launch_fill_u32(unsigned* p, size_t n, unsigned v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace cbd
