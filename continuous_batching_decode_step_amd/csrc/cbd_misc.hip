// Per-lane row kernels of the decode step on gfx950: embedding gather with the
// first RMSNorm's sum of squares and the lane's rotary table, and the final
// argmax over the LM head's per-tile candidates.
#include "cbd_internal.h"

namespace cbd {

// x[b] = E[token_b] (exact upcast of bf16, q * scale of Q8_0), the sum of
// x[b]^2 for the first RMSNorm (the projections that consume x normalise it),
// and the rotary (cos, sin) of the lane's position for every pair:
// theta_j = theta^(-2j/hd), angle = pos * theta_j, in double, rounded to f32.
template <int WT>
__global__ __launch_bounds__(256) void k_embed(const void* E, const uint16_t* Es, const int* tokens, const int* pos,
                                               int d, int hd, float theta, float* x, float* ssq, float2* rope) {
  const int b = blockIdx.x;
  const int tok = tokens[b];
  float* xr = x + (size_t)b * d;
  float part = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) {
    float v;
    if constexpr (WT == WT_F32) {
      v = ((const float*)E)[(size_t)tok * d + i];
    } else if constexpr (WT == WT_BF16) {
      v = __builtin_bit_cast(float, (unsigned)((const uint16_t*)E)[(size_t)tok * d + i] << 16);
    } else {
      const float q = (float)((const int8_t*)E)[(size_t)tok * d + i];
      const float s = (float)__builtin_bit_cast(_Float16, Es[(size_t)tok * (d / 32) + i / 32]);
      v = q * s;
    }
    xr[i] = v;
    part += v * v;
  }
  const float ss = block_sum(part);
  if (threadIdx.x == 0) ssq[b] = ss;
  const int p = pos[b];
  for (int j = threadIdx.x; j < hd / 2; j += 256) {
    const double th = pow((double)theta, -(2.0 * (double)j) / (double)hd);
    const double ang = (double)p * th;
    rope[(size_t)b * (hd / 2) + j] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

__device__ inline uint16_t f2bf_m(float f) {
  unsigned u = __builtin_bit_cast(unsigned, f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// RMSNorm of the residual stream into the activation panel the next
// projection reads: xn = (x * r) * g with r = 1 / sqrt(mean(x^2) + eps).  The
// sum of x^2 of lane b is the producer's per-tile partials added in a fixed
// order (strided per thread, a shuffle tree, then the four waves in order), so
// every workgroup of the lane gets the same r.  Workgroup (chunk, b) handles
// 1024 elements of lane b, 4 per thread.
template <int ACT>
__global__ __launch_bounds__(256) void k_norm(const float* x, const float* ssq, int ssq_n, const float* g, int B,
                                              int d, float eps, void* xn) {
  const int b = blockIdx.y;
  // this thread's x and gain first, so their loads overlap the reduction
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  const bool live = i < d;
  const int ic = live ? i : 0;
  const float4 xv = *(const float4*)(x + (size_t)b * d + ic);
  const float4 gv = *(const float4*)(g + ic);
  float part = 0.f;
  for (int t = threadIdx.x; t < ssq_n; t += 256) part += ssq[(size_t)t * B + b];
  const float ss = block_sum(part);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  if (!live) return;
  const float v0 = (xv.x * r) * gv.x, v1 = (xv.y * r) * gv.y, v2 = (xv.z * r) * gv.z, v3 = (xv.w * r) * gv.w;
  const size_t o = (size_t)b * d + i;
  if constexpr (ACT == WT_F32) {
    *(float4*)((float*)xn + o) = make_float4(v0, v1, v2, v3);
  } else if constexpr (ACT == WT_BF16) {
    *(uint2*)((uint16_t*)xn + o) = make_uint2((unsigned)f2bf_m(v0) | ((unsigned)f2bf_m(v1) << 16),
                                              (unsigned)f2bf_m(v2) | ((unsigned)f2bf_m(v3) << 16));
  } else {
    _Float16* p = (_Float16*)xn + o;
    p[0] = (_Float16)v0;
    p[1] = (_Float16)v1;
    p[2] = (_Float16)v2;
    p[3] = (_Float16)v3;
  }
}

// argmax[b]: largest value over the LM head's per-row-block candidates, the
// lowest index on ties.  "Larger value, then lower index" is a total order on
// the (non-NaN) candidates, so the result does not depend on the order in
// which they are compared.  One 256-thread workgroup per lane; each thread
// keeps up to ARGMAX_PER candidates in flight (one memory round trip for the
// LM heads here), then a shuffle tree per wave and the four waves in LDS.
constexpr int ARGMAX_PER = 8;

__device__ inline void argmax_take(float v, int i, float& best, int& bi) {
  if (v > best || (v == best && i < bi)) {
    best = v;
    bi = i;
  }
}

__global__ __launch_bounds__(256) void k_argmax(const float2* amax, int nRB, int B, int* out) {
  const int b = blockIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int rb0 = 0; rb0 < nRB; rb0 += 256 * ARGMAX_PER) {
    float2 e[ARGMAX_PER];
#pragma unroll
    for (int u = 0; u < ARGMAX_PER; ++u) {
      const int rb = rb0 + u * 256 + threadIdx.x;
      e[u] = rb < nRB ? amax[(size_t)rb * B + b] : make_float2(-INFINITY, __int_as_float(0x7fffffff));
    }
#pragma unroll
    for (int u = 0; u < ARGMAX_PER; ++u) argmax_take(e[u].x, __float_as_int(e[u].y), best, bi);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) argmax_take(__shfl_xor(best, off), __shfl_xor(bi, off), best, bi);
  __shared__ float vb[4];
  __shared__ int ib[4];
  if ((threadIdx.x & 63) == 0) {
    vb[threadIdx.x >> 6] = best;
    ib[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) argmax_take(vb[w], ib[w], best, bi);
    out[b] = bi;
  }
}

__global__ void k_fill_u32(unsigned* p, size_t n, unsigned v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// Move positions [p0, p0 + len) of one lane's K or V between rows
// [n_rows = L * Hkv][len][hd] (contiguous, `rows`) and its blocks in a
// layer-major pool, 16 bytes per thread: position p of row (l, g) sits at
// l * lstride + blocks[p / 64] * bbytes + (g * 64 + p % 64) * row_bytes.
// row_bytes (hd * element size) is a multiple of 16.
__global__ __launch_bounds__(256) void k_kv_rows(char* pool, char* rows, const int* blocks, int p0, int len,
                                                 int n_rows, int Hkv, int row_bytes, long long lstride,
                                                 long long bbytes, int to_pool) {
  const int W = row_bytes / 16;
  const size_t n = (size_t)n_rows * len * W;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < n; u += (size_t)gridDim.x * blockDim.x) {
    const int w = (int)(u % W);
    const size_t tr = u / W;
    const int t = p0 + (int)(tr % len), r = (int)(tr / len);
    const int l = r / Hkv, g = r % Hkv;
    char* pp = pool + l * lstride + blocks[t >> 6] * bbytes + ((long long)g * 64 + (t & 63)) * row_bytes + w * 16;
    uint4* rp = (uint4*)(rows + u * 16);
    if (to_pool)
      *(uint4*)pp = *rp;
    else
      *rp = *(const uint4*)pp;
  }
}

hipError_t launch_kv_rows(char* pool, char* rows, const int* blocks, int p0, int len, int n_rows, int Hkv,
                          int row_bytes, long long lstride, long long bbytes, bool to_pool, hipStream_t st) {
  const size_t n = (size_t)n_rows * len * (row_bytes / 16);
  if (n == 0) return hipSuccess;
  size_t wgs = (n + 255) / 256;
  if (wgs > 8192) wgs = 8192;
  hipLaunchKernelGGL(k_kv_rows, dim3((unsigned)wgs), dim3(256), 0, st, pool, rows, blocks, p0, len, n_rows, Hkv,
                     row_bytes, lstride, bbytes, (int)to_pool);
  return hipGetLastError();
}

// Fragment-ordered bf16 chunks (kfrag_off / vfrag_off) to or from rows: one
// workgroup per (row (l, g), chunk c overlapping [p0, p0 + len)), through an
// LDS tile of the chunk in row-major order.  A chunk only partly in range is
// read first, so its other keys keep their contents.  Rows as in k_kv_rows.
__global__ __launch_bounds__(256) void k_kv_rows_frag(uint16_t* pool, uint16_t* rows, const int* blocks, int p0,
                                                      int len, int Hkv, int hd, long long lstride, long long bstride,
                                                      int to_pool, int frag) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * 128];
  const int r = blockIdx.x, l = r / Hkv, g = r % Hkv;
  const int c = p0 / 64 + (int)blockIdx.y;
  const int kb = c * 64, lo = max(p0, kb), hi = min(p0 + len, kb + 64);
  uint16_t* chunk = pool + l * lstride + (long long)blocks[c] * bstride + (long long)g * 64 * hd;
  const int n = 64 * hd;
  auto at = [&](int o, int* key, int* d) {
    if (frag == 1)
      kfrag_at(o, hd, key, d);
    else
      vfrag_at(o, hd, key, d);
  };
  if (!to_pool || lo > kb || hi < kb + 64) {
    for (int q = threadIdx.x; q < n / 8; q += blockDim.x) {
      const uint4 v = *(const uint4*)(chunk + 8 * q);
      const unsigned wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int key, d;
        at(8 * q + e, &key, &d);
        tile[key * hd + d] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
      }
    }
    __syncthreads();
  }
  const int pieces = (hi - lo) * (hd / 8);  // 16-byte pieces of the rows in range
  uint16_t* rrow = rows + ((long long)r * len + (lo - p0)) * hd;
  if (to_pool) {
    for (int q = threadIdx.x; q < pieces; q += blockDim.x)
      *(uint4*)(tile + (lo - kb) * hd + 8 * q) = *(const uint4*)(rrow + 8 * q);
    __syncthreads();
    for (int q = threadIdx.x; q < n / 8; q += blockDim.x) {
      unsigned wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int key, d;
        at(8 * q + e, &key, &d);
        wv[e >> 1] |= (unsigned)tile[key * hd + d] << (16 * (e & 1));
      }
      *(uint4*)(chunk + 8 * q) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
  } else {
    for (int q = threadIdx.x; q < pieces; q += blockDim.x)
      *(uint4*)(rrow + 8 * q) = *(const uint4*)(tile + (lo - kb) * hd + 8 * q);
  }
}

hipError_t launch_kv_rows_frag(char* pool, char* rows, const int* blocks, int p0, int len, int n_rows, int Hkv,
                               int hd, long long lstride, long long bbytes, bool to_pool, int frag, hipStream_t st) {
  if (len <= 0 || n_rows <= 0) return hipSuccess;
  if (hd > 128 || hd % 32 != 0 || (frag != 1 && frag != 2)) return hipErrorInvalidValue;
  const int nch = (p0 + len - 1) / 64 - p0 / 64 + 1;
  hipLaunchKernelGGL(k_kv_rows_frag, dim3(n_rows, nch), dim3(256), 0, st, (uint16_t*)pool, (uint16_t*)rows, blocks, p0,
                     len, Hkv, hd, lstride / 2, bbytes / 2, (int)to_pool, frag);
  return hipGetLastError();
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Rotate n_vec stored key vectors of hd elements in place by one rotary angle
// per pair (cs[j] = (cos, sin) for the pair (j, j + hd/2)): (a, b) ->
// (a c - b s, b c + a s), every product and sum rounded to f32 on its own (no
// fused multiply-add), then rounded to the KV format (bf16 round-to-nearest-
// even, or kept in f32).
__global__ __launch_bounds__(256) void k_kv_rot(char* rows, long long n_vec, int hd, const float2* cs, int bf16) {
#pragma clang fp contract(off)  // the products must round before the sum (the compiler fuses them otherwise)
  const int h = hd / 2;
  const long long n = n_vec * h;
  for (long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x; u < n; u += (long long)gridDim.x * blockDim.x) {
    const long long r = u / h;
    const int j = (int)(u % h);
    const float2 t = cs[j];
    float a, b;
    if (bf16) {
      const uint16_t* x = (const uint16_t*)rows + r * hd;
      a = __uint_as_float((unsigned)x[j] << 16);
      b = __uint_as_float((unsigned)x[j + h] << 16);
    } else {
      const float* x = (const float*)rows + r * hd;
      a = x[j];
      b = x[j + h];
    }
    const float ac = a * t.x, bs = b * t.y, bc = b * t.x, as = a * t.y;
    const float y0 = ac - bs, y1 = bc + as;
    if (bf16) {
      uint16_t* x = (uint16_t*)rows + r * hd;
      x[j] = f32_to_bf16_rne(y0);
      x[j + h] = f32_to_bf16_rne(y1);
    } else {
      float* x = (float*)rows + r * hd;
      x[j] = y0;
      x[j + h] = y1;
    }
  }
}

hipError_t launch_kv_rot(char* rows, long long n_vec, int hd, const float2* cs, bool bf16, hipStream_t st) {
  const long long n = n_vec * (hd / 2);
  if (n == 0) return hipSuccess;
  long long wgs = (n + 255) / 256;
  if (wgs > 8192) wgs = 8192;
  hipLaunchKernelGGL(k_kv_rot, dim3((unsigned)wgs), dim3(256), 0, st, rows, n_vec, hd, cs, (int)bf16);
  return hipGetLastError();
}

// Copy whole blocks of a layer-major pool, K and V: block src[j] to block
// dst[j] in every layer, 16 bytes per thread.  Unit u covers (pool half v,
// layer l, pair j, 16-byte word w) with w fastest.
__global__ __launch_bounds__(256) void k_kv_blocks(char* base, long long half, const int* src, const int* dst,
                                                   int n, int L, long long lstride, long long bbytes) {
  const long long W = bbytes / 16;
  const long long total = 2LL * L * n * W;
  for (long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x; u < total;
       u += (long long)gridDim.x * blockDim.x) {
    const long long w = u % W;
    const long long r = u / W;
    const int j = (int)(r % n);
    const int l = (int)((r / n) % L);
    const int v = (int)(r / ((long long)n * L));
    char* p = base + v * half + l * lstride;
    *(uint4*)(p + dst[j] * bbytes + w * 16) = *(const uint4*)(p + src[j] * bbytes + w * 16);
  }
}

hipError_t launch_kv_blocks(char* base, long long half, const int* src, const int* dst, int n, int L,
                            long long lstride, long long bbytes, hipStream_t st) {
  const long long total = 2LL * L * n * (bbytes / 16);
  if (total == 0) return hipSuccess;
  long long wgs = (total + 255) / 256;
  if (wgs > 16384) wgs = 16384;
  hipLaunchKernelGGL(k_kv_blocks, dim3((unsigned)wgs), dim3(256), 0, st, base, half, src, dst, n, L, lstride, bbytes);
  return hipGetLastError();
}

hipError_t launch_embed(int wt, const void* E, const uint16_t* Es, const int* tokens, const int* pos, int B, int d,
                        int hd, float theta, float* x, float* ssq, float2* rope, hipStream_t st) {
  switch (wt) {
    case WT_F32:
      hipLaunchKernelGGL(k_embed<WT_F32>, dim3(B), dim3(256), 0, st, E, Es, tokens, pos, d, hd, theta, x, ssq, rope);
      break;
    case WT_BF16:
      hipLaunchKernelGGL(k_embed<WT_BF16>, dim3(B), dim3(256), 0, st, E, Es, tokens, pos, d, hd, theta, x, ssq,
                         rope);
      break;
    default:
      hipLaunchKernelGGL(k_embed<WT_Q8>, dim3(B), dim3(256), 0, st, E, Es, tokens, pos, d, hd, theta, x, ssq, rope);
      break;
  }
  return hipGetLastError();
}

// The step's metadata from its pinned staging slot (host memory the device
// reads over the bus) to the workspace, by a kernel: for the ~140 KB of items
// of a 64-lane step the runtime's own copy goes through a DMA engine, whose
// hand-off with the kernel queue left ~25 us idle before each step.  Loads at
// system scope never see a stale cached copy of a slot written again by the
// host four steps later.
__global__ __launch_bounds__(256) void k_meta_copy(unsigned* dst, const unsigned* src, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

hipError_t launch_meta_copy(void* dst, const void* src_dev, size_t bytes, hipStream_t st) {
  if (bytes % 4 != 0 || bytes / 4 > 0x7fffffffu) return hipErrorInvalidValue;
  const int n = (int)(bytes / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_meta_copy, dim3((n + 255) / 256), dim3(256), 0, st, (unsigned*)dst, (const unsigned*)src_dev, n);
  return hipGetLastError();
}

hipError_t launch_norm(int wt, const float* x, const float* ssq, int ssq_n, const float* g, int B, int d, float eps,
                       void* xn, hipStream_t st) {
  const dim3 grid((d + 1023) / 1024, B);
  switch (wt) {
    case WT_F32: hipLaunchKernelGGL(k_norm<WT_F32>, grid, dim3(256), 0, st, x, ssq, ssq_n, g, B, d, eps, xn); break;
    case WT_BF16: hipLaunchKernelGGL(k_norm<WT_BF16>, grid, dim3(256), 0, st, x, ssq, ssq_n, g, B, d, eps, xn); break;
    default: hipLaunchKernelGGL(k_norm<WT_Q8>, grid, dim3(256), 0, st, x, ssq, ssq_n, g, B, d, eps, xn); break;
  }
  return hipGetLastError();
}

hipError_t launch_argmax(const float2* amax, int nRB, int B, int* argmax, hipStream_t st) {
  hipLaunchKernelGGL(k_argmax, dim3(B), dim3(256), 0, st, amax, nRB, B, argmax);
  return hipGetLastError();
}

// Packed tile layout of a bf16 matrix (the layout the header documents at
// cbd_pack_matrix): one thread per 16-byte slot of a tile, zeros for the
// padding rows of a half's last tile and for the gap tiles.
__global__ __launch_bounds__(256) void k_pack_bf16(const uint16_t* src, uint16_t* dst, int rows, int K, int T,
                                                   long long n_slots) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_slots) return;
  const int nks = K / 32, run = nks + PACK_GAP;
  const int L = (int)(i & 63);
  const long long tile = i >> 6;            // (h * T + ti) * run + t
  const int t = (int)(tile % run);
  const long long ht = tile / run;          // h * T + ti
  const int ti = (int)(ht % T), h = (int)(ht / T);
  const int row = ti * 16 + (L & 15);
  const int k = t * 32 + 8 * (L >> 4);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < rows && t < nks) v = *(const uint4*)(src + ((size_t)h * rows + row) * K + k);
  *(uint4*)(dst + (size_t)i * 8) = v;
}

size_t packed_bytes_bf16(int rows, int K, int halves) {
  if (rows <= 0 || halves <= 0 || K <= 0 || K % 32 != 0) return 0;
  return (size_t)halves * ((rows + 15) / 16) * (K / 32 + PACK_GAP) * 1024;
}

hipError_t launch_pack_bf16(const void* src, void* dst, int rows, int K, int halves, hipStream_t st) {
  const long long n_slots = (long long)(packed_bytes_bf16(rows, K, halves) / 16);
  if (n_slots == 0) return hipSuccess;
  const int T = (rows + 15) / 16;
  hipLaunchKernelGGL(k_pack_bf16, dim3((unsigned)((n_slots + 255) / 256)), dim3(256), 0, st, (const uint16_t*)src,
                     (uint16_t*)dst, rows, K, T, n_slots);
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
