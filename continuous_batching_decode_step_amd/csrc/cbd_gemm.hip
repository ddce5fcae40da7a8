// Weight-streaming panel projection for gfx950: Y[b][n] = sum_k W[n][k] X[b][k].
//
// The method this serves ("MODEL-BATCHING-RESULTS — multi-user batched
// decode, measured", section "The lever") runs each projection once over the
// [B, d] panel of the step so each weight row is read once for all B lanes.
// Here a wave owns GEMM_R tiles of 16 weight rows, C groups of 16 lanes and
// one split of K: it streams its rows from HBM with 16-byte loads straight
// into MFMA A operands (rows = MFMA M), takes the lanes' activations as the B
// operand (lanes = MFMA N), and accumulates in f32 registers.  The same wave
// code serves B = 1 (15 of 16 columns idle: the MFMA pipe has ample headroom
// while HBM is the bound) and wide panels.
//
// Reduction contract (what makes lane b bit-identical to running alone, the
// structural invariant of "Correctness — proven, not asserted"): every output
// element is  ((P_0 + P_1) + ...) + P_{S-1}  where P_s is a chain of MFMAs
// over the ascending k-steps of split s starting from zero; S and the split
// bounds depend on (N, K) only.  MFMA computes each output element from its
// own row and column, so neither B nor the other lanes change a bit.
//
// Split partials go to the workspace; the last wave of a tile to arrive (an
// agent-scope counter, reset by that wave) sums them in split order and runs
// the epilogue: store, residual add, SwiGLU, or LM-head store + argmax
// candidates.  No float atomics, no second launch.
#include "cbd_internal.h"

namespace cbd {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int WT>
struct KStep;
template <>
struct KStep<WT_F32> {
  static constexpr int v = 16;  // 4 MFMA 16x16x4 f32; a lane holds 4 consecutive k
  static constexpr int per_lane = 4;
};
template <>
struct KStep<WT_BF16> {
  static constexpr int v = 32;  // one MFMA 16x16x32 bf16; a lane holds 8 consecutive k
  static constexpr int per_lane = 8;
};
template <>
struct KStep<WT_Q8> {
  static constexpr int v = 32;  // one MFMA 16x16x32 f16 = one Q8_0 block; 8 k per lane
  static constexpr int per_lane = 8;
};

__device__ inline u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// A operand: 16 bytes of weights of `row` at element k (a lane's share of one k-step).
template <int WT>
__device__ inline u32x4 load_a(const GemmArgs& a, int row, int k, bool ok) {
  if constexpr (WT == WT_F32) {
    const float* W = (const float*)a.W;
    size_t off = ok ? (size_t)row * a.K + k : 0;
    u32x4 v = *(const u32x4*)(W + off);
    return ok ? v : zero4();
  } else if constexpr (WT == WT_BF16) {
    const uint16_t* W = (const uint16_t*)a.W;
    size_t off = ok ? (size_t)row * a.K + k : 0;
    u32x4 v = *(const u32x4*)(W + off);
    return ok ? v : zero4();
  } else {
    // Q8_0: 8 int8 of one block, scaled into binary16 in registers.
    const int8_t* W = (const int8_t*)a.W;
    size_t off = ok ? (size_t)row * a.K + k : 0;
    size_t soff = ok ? (size_t)row * (a.K >> 5) + (k >> 5) : 0;
    u32x2 q = *(const u32x2*)(W + off);
    _Float16 sh = __builtin_bit_cast(_Float16, a.Ws[soff]);
    float s = ok ? (float)sh : 0.0f;
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      unsigned wd = i < 4 ? q.x : q.y;
      int qi = (int)(signed char)((wd >> (8 * (i & 3))) & 0xffu);
      r[i] = (_Float16)((float)qi * s);
    }
    return __builtin_bit_cast(u32x4, r);
  }
}

// B operand: 16 bytes of the activation panel of lane `col` at element k.
template <int WT>
__device__ inline u32x4 load_b(const GemmArgs& a, int col, int k, bool ok) {
  size_t off = ok ? (size_t)col * a.K + k : 0;
  u32x4 v;
  if constexpr (WT == WT_F32)
    v = *(const u32x4*)((const float*)a.X + off);
  else
    v = *(const u32x4*)((const uint16_t*)a.X + off);
  return ok ? v : zero4();
}

template <int WT>
__device__ inline f32x4 mma(u32x4 av, u32x4 bv, f32x4 c) {
  if constexpr (WT == WT_F32) {
    f32x4 af = __builtin_bit_cast(f32x4, av), bf = __builtin_bit_cast(f32x4, bv);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[0], bf[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[1], bf[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[2], bf[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[3], bf[3], c, 0, 0, 0);
    return c;
  } else if constexpr (WT == WT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv),
                                                   c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv), c,
                                                  0, 0, 0);
  }
}

__device__ inline uint16_t f2bf(float f) {
  unsigned u = __builtin_bit_cast(unsigned, f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int WT>
__device__ inline void store_act(void* base, size_t idx, float v) {
  if constexpr (WT == WT_F32)
    ((float*)base)[idx] = v;
  else if constexpr (WT == WT_BF16)
    ((uint16_t*)base)[idx] = f2bf(v);
  else
    ((_Float16*)base)[idx] = (_Float16)v;
}

template <int WT, int EPI, int C>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  constexpr int R = GEMM_R;
  constexpr int KS = KStep<WT>::v;
  constexpr int PL = KStep<WT>::per_lane;
  constexpr int U = 4;  // k-steps whose loads are issued together
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int total = a.nRB * a.S * a.nCG;
  if (wave >= total) return;
  const int rb = wave % a.nRB;
  const int s = (wave / a.nRB) % a.S;
  const int cg = wave / (a.nRB * a.S);
  const int r16 = lane & 15, g4 = lane >> 4;

  // Rows this lane loads (A operand row = lane % 16).
  int arow[R];
  bool aok[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int H = R / 2;
      int j = rb * TILE * H + TILE * (r % H) + r16;
      arow[r] = r < H ? j : a.N + j;
      aok[r] = j < a.N;
    } else {
      int n = rb * TILE * R + TILE * r + r16;
      arow[r] = n;
      aok[r] = n < a.N;
    }
  }
  int bcol[C];
  bool bok[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    bcol[c] = cg * TILE * C + TILE * c + r16;
    bok[c] = bcol[c] < a.B;
  }

  const int kb = s * a.Ks;
  const int ke = min(kb + a.Ks, a.K);
  const int koff = PL * g4;

  f32x4 acc[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  int k0 = kb;
  for (; k0 + U * KS <= ke; k0 += U * KS) {
    u32x4 av[U][R], bv[U][C];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) av[u][r] = load_a<WT>(a, arow[r], k0 + u * KS + koff, aok[r]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < C; ++c) bv[u][c] = load_b<WT>(a, bcol[c], k0 + u * KS + koff, bok[c]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[r][c] = mma<WT>(av[u][r], bv[u][c], acc[r][c]);
  }
  for (; k0 < ke; k0 += KS) {
    const int kk = k0 + koff;
    const bool kok = kk + PL <= a.K;  // K % PL == 0, so a lane's vector is all in or all out
    u32x4 av[R], bv[C];
#pragma unroll
    for (int r = 0; r < R; ++r) av[r] = load_a<WT>(a, arow[r], kk, aok[r] && kok);
#pragma unroll
    for (int c = 0; c < C; ++c) bv[c] = load_b<WT>(a, bcol[c], kk, bok[c] && kok);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) acc[r][c] = mma<WT>(av[r], bv[c], acc[r][c]);
  }

  // Output coordinates of acc[r][c][i]: row (or gate/up pair) and lane column.
  auto out_row = [&](int r, int i) -> int {
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int H = R / 2;
      return rb * TILE * H + TILE * (r % H) + 4 * g4 + i;
    } else {
      return rb * TILE * R + TILE * r + 4 * g4 + i;
    }
  };
  auto raw_row = [&](int r, int i) -> int {
    int n = out_row(r, i);
    if constexpr (EPI == EPI_SWIGLU) return r < R / 2 ? n : a.N + n;
    return n;
  };

  if (a.S > 1) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int col = cg * TILE * C + TILE * c + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (out_row(r, i) < a.N && col < a.B)
            a.part[((size_t)s * a.B + col) * a.Nraw + raw_row(r, i)] = acc[r][c][i];
      }
    __threadfence();
    const int tile = cg * a.nRB + rb;
    unsigned prev = 0;
    if (lane == 0) prev = atomicAdd(a.cnt + tile, 1u);
    prev = __shfl(prev, 0);
    if (prev != (unsigned)(a.S - 1)) return;
    __threadfence();
    if (lane == 0) atomicExch(a.cnt + tile, 0u);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int col = cg * TILE * C + TILE * c + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (!(out_row(r, i) < a.N && col < a.B)) continue;
          float v = 0.f;
          for (int s2 = 0; s2 < a.S; ++s2) {
            float p = (s2 == s) ? acc[r][c][i] : a.part[((size_t)s2 * a.B + col) * a.Nraw + raw_row(r, i)];
            v = (s2 == 0) ? p : v + p;
          }
          acc[r][c][i] = v;
        }
      }
  }

  // Epilogue.
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int col = cg * TILE * C + TILE * c + r16;
    const bool cok = col < a.B;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int r = 0; r < R / 2; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = out_row(r, i);
          if (cok && j < a.N) {
            float g = acc[r][c][i], u = acc[r + R / 2][c][i];
            float act = (g / (1.0f + expf(-g))) * u;
            store_act<WT>(a.act_out, (size_t)col * a.N + j, act);
          }
        }
    } else {
      float best = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = out_row(r, i);
          if (!(cok && n < a.N)) continue;
          const float v = acc[r][c][i];
          const size_t idx = (size_t)col * a.N + n;
          if constexpr (EPI == EPI_RESID) {
            a.out[idx] = a.out[idx] + v;
          } else {
            a.out[idx] = v;
          }
          if constexpr (EPI == EPI_HEAD) {
            if (v > best || (v == best && n < bi)) {
              best = v;
              bi = n;
            }
          }
        }
      if constexpr (EPI == EPI_HEAD) {
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
          float ov = __shfl_xor(best, off);
          int oi = __shfl_xor(bi, off);
          if (ov > best || (ov == best && oi < bi)) {
            best = ov;
            bi = oi;
          }
        }
        if (g4 == 0 && cok) a.amax[(size_t)rb * a.B + col] = make_float2(best, __int_as_float(bi));
      }
    }
  }
}

template <int WT, int EPI>
static hipError_t launch_c(int C, const GemmArgs& a, int blocks, hipStream_t st) {
  switch (C) {
    case 1: hipLaunchKernelGGL((k_gemm<WT, EPI, 1>), dim3(blocks), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_gemm<WT, EPI, 2>), dim3(blocks), dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((k_gemm<WT, EPI, 4>), dim3(blocks), dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

template <int WT>
static hipError_t launch_epi(int epi, int C, const GemmArgs& a, int blocks, hipStream_t st) {
  switch (epi) {
    case EPI_STORE: return launch_c<WT, EPI_STORE>(C, a, blocks, st);
    case EPI_RESID: return launch_c<WT, EPI_RESID>(C, a, blocks, st);
    case EPI_SWIGLU: return launch_c<WT, EPI_SWIGLU>(C, a, blocks, st);
    default: return launch_c<WT, EPI_HEAD>(C, a, blocks, st);
  }
}

hipError_t launch_gemm(int wt, int epi, int C, const GemmArgs& a, int n_waves, hipStream_t st) {
  const int blocks = (n_waves + 3) / 4;
  if (blocks <= 0) return hipSuccess;
  switch (wt) {
    case WT_F32: return launch_epi<WT_F32>(epi, C, a, blocks, st);
    case WT_BF16: return launch_epi<WT_BF16>(epi, C, a, blocks, st);
    default: return launch_epi<WT_Q8>(epi, C, a, blocks, st);
  }
}

}  // namespace cbd
