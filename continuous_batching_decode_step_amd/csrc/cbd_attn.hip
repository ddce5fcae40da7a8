// Ragged per-lane grouped-query attention for one decode step on gfx950.
//
// "MODEL-BATCHING-RESULTS — multi-user batched decode, measured" (section
// "The lever") keeps attention per user: lane b's queries read only lane b's
// own cache, over its own length.  Each lane owns a contiguous slab per
// (layer, KV head) in the arena, so there is no padding and no mask: a lane at
// position p reads slots [0, p] and writes slot p.
//
// One workgroup handles (lane, KV head, split of ATTN_SPLIT keys) for the
// whole group of query heads sharing that KV head, so each K/V row is read
// once per group.  The workgroup that owns slot p rotates the new key at p
// (the same position as the queries, "parallel-slots.md", trap 2 of
// "S1b decode: design traps"), rounds it to the KV format, writes it into the
// slab in place and uses the rounded value.  Splits combine by the usual
// max-rescaled sum, done by the last workgroup of the lane/head to finish (an
// agent-scope counter) in split order, so the result is fixed by the lane's
// position alone.
#include "cbd_internal.h"

namespace cbd {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int MAXG = 8;

__device__ inline uint16_t f2bf_a(float f) {
  unsigned u = __builtin_bit_cast(unsigned, f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline float bf2f(uint16_t h) { return __builtin_bit_cast(float, (unsigned)h << 16); }

template <int ACT>
__device__ inline void put_act(void* base, size_t idx, float v) {
  if constexpr (ACT == WT_F32)
    ((float*)base)[idx] = v;
  else if constexpr (ACT == WT_BF16)
    ((uint16_t*)base)[idx] = f2bf_a(v);
  else
    ((_Float16*)base)[idx] = (_Float16)v;
}

// Block-wide reductions over 256 threads with a fixed combining tree.
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

template <int HD, bool KVBF16, int ACT>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  constexpr int NSUB = 256 / HD;  // key subsets in the value pass
  const int item = blockIdx.x;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int b = a.items[2 * item];
  const int s = a.items[2 * item + 1];
  const int p = a.pos[b];
  const int G = a.G;
  const int nk = p + 1;
  const int nsplit = (nk + ATTN_SPLIT - 1) / ATTN_SPLIT;
  const int kbeg = s * ATTN_SPLIT;
  const int kend = min(kbeg + ATTN_SPLIT, nk);
  const int n = kend - kbeg;

  __shared__ float q_s[MAXG][HD];
  __shared__ float knew[HD], vnew[HD];
  __shared__ float sc[MAXG][ATTN_SPLIT];
  __shared__ float red[MAXG][4];
  __shared__ float opart[NSUB][MAXG][HD];
  __shared__ float stat[2][MAXG];
  __shared__ unsigned last_flag;

  const long long base = (long long)a.lanes[b] * a.lane_stride + a.layer_off + (long long)g * a.max_seq * HD;
  const float* row = a.qkv + (size_t)b * a.Nqkv;
  const float2* cs = a.rope + (size_t)b * (HD / 2);

  // Rotate the group's queries at p.
  for (int e = tid; e < G * (HD / 2); e += 256) {
    const int j = e / (HD / 2), jj = e % (HD / 2);
    const float* qh = row + (size_t)(g * G + j) * HD;
    const float x0 = qh[jj], x1 = qh[jj + HD / 2];
    const float2 t = cs[jj];
    q_s[j][jj] = x0 * t.x - x1 * t.y;
    q_s[j][jj + HD / 2] = x1 * t.x + x0 * t.y;
  }
  // The split holding slot p rotates the new key, appends K and V in place.
  if (kend == nk) {
    const float* kr = row + (size_t)(a.Hq + g) * HD;
    const float* vr = row + (size_t)(a.Hq + a.Hkv + g) * HD;
    for (int jj = tid; jj < HD / 2; jj += 256) {
      const float x0 = kr[jj], x1 = kr[jj + HD / 2];
      const float2 t = cs[jj];
      float k0 = x0 * t.x - x1 * t.y, k1 = x1 * t.x + x0 * t.y;
      const long long o0 = base + (long long)p * HD + jj;
      if constexpr (KVBF16) {
        uint16_t h0 = f2bf_a(k0), h1 = f2bf_a(k1);
        ((uint16_t*)a.kslab)[o0] = h0;
        ((uint16_t*)a.kslab)[o0 + HD / 2] = h1;
        k0 = bf2f(h0);
        k1 = bf2f(h1);
      } else {
        ((float*)a.kslab)[o0] = k0;
        ((float*)a.kslab)[o0 + HD / 2] = k1;
      }
      knew[jj] = k0;
      knew[jj + HD / 2] = k1;
    }
    for (int d = tid; d < HD; d += 256) {
      float v = vr[d];
      const long long o = base + (long long)p * HD + d;
      if constexpr (KVBF16) {
        uint16_t h = f2bf_a(v);
        ((uint16_t*)a.vslab)[o] = h;
        v = bf2f(h);
      } else {
        ((float*)a.vslab)[o] = v;
      }
      vnew[d] = v;
    }
  }
  __syncthreads();

  // Scores: one key per thread.
  const float inv = 1.0f / sqrtf((float)HD);
  float dot[MAXG];
#pragma unroll
  for (int j = 0; j < MAXG; ++j) dot[j] = 0.f;
  const int key = kbeg + tid;
  const bool valid = tid < n;
  if (valid) {
    if (key == p) {
      for (int d = 0; d < HD; ++d) {
        const float kv = knew[d];
#pragma unroll
        for (int j = 0; j < MAXG; ++j)
          if (j < G) dot[j] += q_s[j][d] * kv;
      }
    } else {
      const long long kro = base + (long long)key * HD;
      if constexpr (KVBF16) {
        const u32x4* kp = (const u32x4*)((const uint16_t*)a.kslab + kro);
#pragma unroll 4
        for (int c = 0; c < HD / 8; ++c) {
          const u32x4 w = kp[c];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const unsigned word = w[e >> 1];
            const float kv = __builtin_bit_cast(float, (e & 1) ? (word & 0xffff0000u) : (word << 16));
#pragma unroll
            for (int j = 0; j < MAXG; ++j)
              if (j < G) dot[j] += q_s[j][c * 8 + e] * kv;
          }
        }
      } else {
        const u32x4* kp = (const u32x4*)((const float*)a.kslab + kro);
#pragma unroll 4
        for (int c = 0; c < HD / 4; ++c) {
          // bit-cast the whole vector: a bit-cast of one vector element reads element 0
          const f32x4 w = __builtin_bit_cast(f32x4, kp[c]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float kv = w[e];
#pragma unroll
            for (int j = 0; j < MAXG; ++j)
              if (j < G) dot[j] += q_s[j][c * 4 + e] * kv;
          }
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < MAXG; ++j) {
    if (j >= G) break;
    const float sj = valid ? dot[j] * inv : -INFINITY;
    sc[j][tid] = sj;
    const float m = wave_max(sj);
    if ((tid & 63) == 0) red[j][wid] = m;
  }
  __syncthreads();
  if (tid < G) {
    float m = red[tid][0];
    for (int w = 1; w < 4; ++w) m = fmaxf(m, red[tid][w]);
    stat[0][tid] = m;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < MAXG; ++j) {
    if (j >= G) break;
    const float e = valid ? expf(sc[j][tid] - stat[0][j]) : 0.f;
    sc[j][tid] = e;
    const float l = wave_sum(e);
    if ((tid & 63) == 0) red[j][wid] = l;
  }
  __syncthreads();
  if (tid < G) {
    float l = red[tid][0];
    for (int w = 1; w < 4; ++w) l += red[tid][w];
    stat[1][tid] = l;
  }

  // Values: thread (dim, key subset), then subsets summed in order.
  {
    const int dim = tid % HD, sub = tid / HD;
    float o[MAXG];
#pragma unroll
    for (int j = 0; j < MAXG; ++j) o[j] = 0.f;
    for (int tl = sub; tl < n; tl += NSUB) {
      const int kk = kbeg + tl;
      float v;
      if (kk == p) {
        v = vnew[dim];
      } else {
        const long long off = base + (long long)kk * HD + dim;
        if constexpr (KVBF16)
          v = bf2f(((const uint16_t*)a.vslab)[off]);
        else
          v = ((const float*)a.vslab)[off];
      }
#pragma unroll
      for (int j = 0; j < MAXG; ++j)
        if (j < G) o[j] += sc[j][tl] * v;
    }
#pragma unroll
    for (int j = 0; j < MAXG; ++j)
      if (j < G) opart[sub][j][dim] = o[j];
  }
  __syncthreads();

  const int Hqd = a.Hq * HD;
  if (nsplit == 1) {
    for (int e = tid; e < G * HD; e += 256) {
      const int j = e / HD, dim = e % HD;
      float acc = opart[0][j][dim];
      for (int u = 1; u < NSUB; ++u) acc += opart[u][j][dim];
      put_act<ACT>(a.out, (size_t)b * Hqd + (size_t)(g * G + j) * HD + dim, acc / stat[1][j]);
    }
    return;
  }

  // Several splits: publish (o, m, l), the last workgroup combines in split order.
  const size_t pstride = (size_t)G * (HD + 2);
  float* mine = a.part + (((size_t)b * a.max_splits + s) * a.Hkv + g) * pstride;
  for (int e = tid; e < G * HD; e += 256) {
    const int j = e / HD, dim = e % HD;
    float acc = opart[0][j][dim];
    for (int u = 1; u < NSUB; ++u) acc += opart[u][j][dim];
    mine[(size_t)j * (HD + 2) + dim] = acc;
  }
  if (tid < G) {
    mine[(size_t)tid * (HD + 2) + HD] = stat[0][tid];
    mine[(size_t)tid * (HD + 2) + HD + 1] = stat[1][tid];
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(a.cnt + (size_t)b * a.Hkv + g, 1u);
    last_flag = (prev == (unsigned)(nsplit - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  if (tid == 0) atomicExch(a.cnt + (size_t)b * a.Hkv + g, 0u);
  const float* P0 = a.part + ((size_t)b * a.max_splits * a.Hkv + g) * pstride;
  const size_t sstride = (size_t)a.Hkv * pstride;
  for (int e = tid; e < G * HD; e += 256) {
    const int j = e / HD, dim = e % HD;
    float M = -INFINITY;
    for (int u = 0; u < nsplit; ++u) M = fmaxf(M, P0[u * sstride + (size_t)j * (HD + 2) + HD]);
    float L = 0.f, O = 0.f;
    for (int u = 0; u < nsplit; ++u) {
      const float* P = P0 + u * sstride + (size_t)j * (HD + 2);
      const float w = expf(P[HD] - M);
      L += w * P[HD + 1];
      O += w * P[dim];
    }
    put_act<ACT>(a.out, (size_t)b * Hqd + (size_t)(g * G + j) * HD + dim, O / L);
  }
}

template <int HD>
static hipError_t launch_hd(int kv_bf16, int act, const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.n_items, a.Hkv), blk(256);
  if (kv_bf16) {
    hipLaunchKernelGGL((k_attn<HD, true, WT_BF16>), grid, blk, 0, st, a);
  } else if (act == WT_Q8) {
    hipLaunchKernelGGL((k_attn<HD, false, WT_Q8>), grid, blk, 0, st, a);
  } else {
    hipLaunchKernelGGL((k_attn<HD, false, WT_F32>), grid, blk, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn(int hd, int kv_bf16, int act, const AttnArgs& a, hipStream_t st) {
  if (a.n_items <= 0) return hipSuccess;
  switch (hd) {
    case 16: return launch_hd<16>(kv_bf16, act, a, st);
    case 32: return launch_hd<32>(kv_bf16, act, a, st);
    case 64: return launch_hd<64>(kv_bf16, act, a, st);
    case 128: return launch_hd<128>(kv_bf16, act, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cbd
