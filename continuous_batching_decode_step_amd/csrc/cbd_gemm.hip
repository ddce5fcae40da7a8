// Weight-streaming panel projection for gfx950: Y[b][n] = sum_k W[n][k] X[b][k].
//
// The method this serves ("MODEL-BATCHING-RESULTS — multi-user batched
// decode, measured", section "The lever") runs each projection once over the
// [B, d] panel of the step so each weight row is read once for all B lanes.
// A wave owns `rows` tiles of 16 weight rows, C groups of 16 lanes and one
// split of K: it streams its rows from HBM with 16-byte loads straight into
// MFMA A operands (rows = MFMA M), takes the lanes' activations as the B
// operand (lanes = MFMA N), and accumulates in f32 registers.  Loads run two
// pipeline stages ahead of the MFMAs.  The same wave code serves B = 1 (15 of
// 16 columns idle: the MFMA pipe has ample headroom while HBM is the bound)
// and wide panels.
//
// Reduction contract (what makes lane b bit-identical to running alone, the
// structural invariant of "Correctness — proven, not asserted"): every output
// element is  ((P_0 + P_1) + ...) + P_{S-1}  where P_s is a chain of MFMAs
// over the ascending k-steps of split s starting from zero; S and the split
// bounds depend on (N, K) only.  MFMA computes each output element from its
// own row and column, so neither B nor the other lanes change a bit.
//
// A workgroup owns one output tile and runs its S splits as S waves; the
// partials meet in LDS and wave 0 sums them in split order and runs the
// epilogue.  Nothing crosses workgroups, so no device-scope fence is needed
// (on MI355X those write back and invalidate an XCD's whole L2).
//
// Epilogues: store (QKV), residual add (O, down; also per-tile sums of x^2
// for the next RMSNorm), SwiGLU (gate|up), and the LM head (store + per-tile
// argmax candidates, lowest index on ties).
#include <algorithm>

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

// Unconditional fragment loads from byte pointers (rows and columns already
// clamped into range).
__device__ inline u32x4 ld16(const char* p) { return *(const u32x4*)p; }

// Q8_0: a lane's share of one block is 8 int8 plus the block's binary16 scale,
// carried raw through the load pipeline as {q[0..3], q[4..7], scale, 0} and
// scaled into binary16 MFMA operands when consumed.
__device__ inline u32x4 ld_q8(const char* q, const uint16_t* sp) {
  const u32x2 w = *(const u32x2*)q;
  return u32x4{w.x, w.y, (unsigned)*sp, 0u};
}

__device__ inline u32x4 q8_to_f16(u32x4 raw) {
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)raw.z);
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned wd = i < 4 ? raw.x : raw.y;
    const int qi = (int)(signed char)((wd >> (8 * (i & 3))) & 0xffu);
    r[i] = (_Float16)((float)qi * s);
  }
  return __builtin_bit_cast(u32x4, r);
}

// The epilogue of one wave's output tile: R row tiles x C column tiles of
// 16 x 16 results, the wave's row block rb and column group cg.
//
// A wave may own RM consecutive row blocks (rb is then the index of that group
// and R = RM x the row tiles of one block).  Per-row-block side outputs (sums
// of x^2, argmax candidates) are written per row block, exactly as a wave
// owning one block writes them.
// xpre (EPI_RESID, optional): the residual's values at the wave's outputs,
// loaded earlier (the wave owns them: nobody else writes them meanwhile).
template <int WT, int EPI, int R, int C, int RM = 1>
__device__ inline void epilogue(const GemmArgs& a, int rb, int cg, int lane, const f32x4 (&acc)[R][C],
                                const f32x4 (*xpre)[C] = nullptr) {
  constexpr int R0 = R / RM;  // row tiles of one row block
  const int r16 = lane & 15, g4 = lane >> 4;
  // Output coordinates of acc[r][c][i]: row (or gate/up pair) and lane column.
  auto out_row = [&](int r, int i) -> int {
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int H = R / 2;
      return rb * TILE * H + TILE * (r % H) + 4 * g4 + i;
    } else {
      return rb * TILE * R + TILE * r + 4 * g4 + i;
    }
  };

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
            const float g = acc[r][c][i], u = acc[r + R / 2][c][i];
            const float act = (g / (1.0f + expf(-g))) * u;
            store_act<WT>(a.act_out, (size_t)col * a.N + j, act);
          }
        }
    } else if constexpr (EPI == EPI_RESID) {
      // x += y, and each row block's sum of x^2 per lane for the next RMSNorm
#pragma unroll
      for (int m = 0; m < RM; ++m) {
        float ss = 0.f;
#pragma unroll
        for (int r = m * R0; r < (m + 1) * R0; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = out_row(r, i);
            if (!(cok && n < a.N)) continue;
            const size_t idx = (size_t)col * a.N + n;
            const float xn = (xpre ? xpre[r][c][i] : a.out[idx]) + acc[r][c][i];
            a.out[idx] = xn;
            ss = __builtin_fmaf(xn, xn, ss);  // the same operation in k_fold_norm
          }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const int ob = rb * RM + m;
        if (g4 == 0 && cok && ob < a.nRB) a.ssq_out[(size_t)ob * a.B + col] = ss;
      }
    } else {
#pragma unroll
      for (int m = 0; m < RM; ++m) {
        float best = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int r = m * R0; r < (m + 1) * R0; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = out_row(r, i);
            if (!(cok && n < a.N)) continue;
            const float v = acc[r][c][i];
            a.out[(size_t)col * a.N + n] = v;
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
            const float ov = __shfl_xor(best, off);
            const int oi = __shfl_xor(bi, off);
            if (ov > best || (ov == best && oi < bi)) {
              best = ov;
              bi = oi;
            }
          }
          const int ob = rb * RM + m;
          if (g4 == 0 && cok && ob < a.nRB) a.amax[(size_t)ob * a.B + col] = make_float2(best, __int_as_float(bi));
        }
      }
    }
  }
}

// NRM: the activations are the RMSNorm of a.in_x, computed by each wave for
// its own split and staged in LDS (one column group of at most 16 lanes).
template <int WT, int EPI, int C, bool NRM = false>
__global__ __launch_bounds__(GEMM_MAX_SPLIT * 64) void k_gemm(GemmArgs a) {
  static_assert(!NRM || C == 1, "normalising split-K tiles take one column group");
  extern __shared__ __attribute__((aligned(16))) char gsm[];  // [norm staging][split partials]
  constexpr int R = gemm_rows(EPI);
  constexpr int KS = KStep<WT>::v;
  constexpr int PL = KStep<WT>::per_lane;
  constexpr int U = C == 1 ? 4 : 2;  // k-steps per pipeline stage
  constexpr int EB = WT == WT_F32 ? 4 : (WT == WT_BF16 ? 2 : 1);  // weight bytes per element
  constexpr int XB = WT == WT_F32 ? 4 : 2;                        // activation bytes per element
  const int lane = threadIdx.x & 63;
  const int s = threadIdx.x >> 6;  // the split this wave computes
  const int rb = blockIdx.x % a.nRB;
  const int cg = blockIdx.x / a.nRB;
  const int r16 = lane & 15, g4 = lane >> 4;

  const int kb = s * a.Ks;
  const int ke = min(kb + a.Ks, a.K);
  const int koff = PL * g4;

  // Row pointers (A operand row = lane % 16).  A row past the end is clamped to
  // the last row: it only feeds output rows that are never stored.  Packed
  // bf16 weights: the lane's slot of the row tile's first k-step tile of the
  // split (a tile past the end is clamped to the half's last tile), one tile
  // (1 KB) per k-step.
  const char* ap[R];
  const uint16_t* sp[R];
  const bool packed = WT == WT_BF16 && a.wpack;
  const int wks = packed ? 1024 : KS * EB;  // weight bytes between k-steps
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int row, tile;
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int H = R / 2;
      const int j = min(rb * TILE * H + TILE * (r % H) + r16, a.N - 1);
      row = r < H ? j : a.N + j;
      tile = min(rb * H + r % H, a.wtiles - 1) + (r < H ? 0 : a.wtiles);
    } else {
      row = min(rb * TILE * R + TILE * r + r16, a.N - 1);
      tile = min(rb * R + r, a.wtiles - 1);
    }
    if (packed)
      ap[r] = (const char*)a.W + ((size_t)tile * (a.K / KS + PACK_GAP) + kb / KS) * 1024 + lane * 16;
    else
      ap[r] = (const char*)a.W + ((size_t)row * a.K + kb + koff) * EB;
    if constexpr (WT == WT_Q8) sp[r] = a.Ws + (size_t)row * (a.K >> 5) + (kb >> 5);
  }
  // Column pointers (B operand column = lane % 16), clamped the same way.
  // NRM: rows of this wave's LDS staging, one per lane of the step, Ks
  // activations + 16 bytes each.
  const int n_st = NRM ? a.B : 0;                    // staged lanes (B <= 16)
  const int st_row = NRM ? a.Ks * XB + 16 : 0;       // bytes per staged lane
  char* mine = gsm + (size_t)s * n_st * st_row;      // this wave's staging
  const char* bp[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int col = min(cg * TILE * C + TILE * c + r16, a.B - 1);
    if constexpr (NRM)
      bp[c] = mine + (size_t)col * st_row + koff * XB;
    else
      bp[c] = (const char*)a.X + ((size_t)col * a.K + kb + koff) * XB;
  }

  // NRM: rows [0, B) of this wave's staging get xn = (x * r) * g over k in
  // [kb, ke), as the norm kernel computes them: r from the sum of the
  // producer's partials in its order (thread t of its 256 adds partial t; a
  // shuffle tree per wave; then its four waves in order, three of them empty
  // here), rounded to the activation format.
  auto stage_norm = [&](char* dst, int row_bytes, int k0, int k1) {
    if constexpr (NRM) {
      float ssv[TILE];
#pragma unroll
      for (int j = 0; j < TILE; ++j) {
        ssv[j] = 0.f;
        if (j < a.B && lane < a.in_ssq_n) ssv[j] += a.in_ssq[(size_t)lane * a.B + j];
      }
      const int nq = (k1 - k0) / 4;  // float4 groups of the split
#pragma unroll
      for (int j = 0; j < TILE; ++j) {
        if (j >= a.B) break;
        float ss = ssv[j];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
        ss = ((ss + 0.f) + 0.f) + 0.f;
        const float r = 1.0f / sqrtf(ss / (float)a.K + a.in_eps);
        const float* xr = a.in_x + (size_t)j * a.K + k0;
        const float* gr = a.in_g + k0;
        char* row = dst + (size_t)j * row_bytes;
        for (int q0 = 0; q0 < nq; q0 += 128) {
          const int qa = q0 + lane, qb = q0 + 64 + lane;
          const bool oka = qa < nq, okb = qb < nq;
          const float4 xa = *(const float4*)(xr + 4 * (oka ? qa : 0));
          const float4 ga = *(const float4*)(gr + 4 * (oka ? qa : 0));
          const float4 xb = *(const float4*)(xr + 4 * (okb ? qb : 0));
          const float4 gb = *(const float4*)(gr + 4 * (okb ? qb : 0));
          auto put = [&](int q, const float4& xv, const float4& gv) {
            const float v0 = (xv.x * r) * gv.x, v1 = (xv.y * r) * gv.y, v2 = (xv.z * r) * gv.z,
                        v3 = (xv.w * r) * gv.w;
            if constexpr (WT == WT_F32) {
              *(float4*)(row + (size_t)q * 16) = make_float4(v0, v1, v2, v3);
            } else if constexpr (WT == WT_BF16) {
              *(u32x2*)(row + (size_t)q * 8) = u32x2{(unsigned)f2bf(v0) | ((unsigned)f2bf(v1) << 16),
                                                     (unsigned)f2bf(v2) | ((unsigned)f2bf(v3) << 16)};
            } else {
              _Float16 h[4] = {(_Float16)v0, (_Float16)v1, (_Float16)v2, (_Float16)v3};
              *(u32x2*)(row + (size_t)q * 8) = __builtin_bit_cast(u32x2, h);
            }
          };
          if (oka) put(qa, xa, ga);
          if (okb) put(qb, xb, gb);
        }
      }
    } else {
      (void)dst;
      (void)row_bytes;
      (void)k0;
      (void)k1;
    }
  };

  f32x4 acc[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Residual projections: wave 0, which runs the epilogue, loads the residual
  // at its outputs now, beside its first weights, rather than after the
  // reduction (one memory round trip less on the serial path).
  f32x4 xpre[R][C];
  if constexpr (EPI == EPI_RESID) {
    if (s == 0) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int col = min(cg * TILE * C + TILE * c + r16, a.B - 1);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = min(rb * TILE * R + TILE * r + 4 * g4 + i, a.N - 1);
            xpre[r][c][i] = a.out[(size_t)col * a.N + n];
          }
      }
    }
  }

  auto load_stage_w = [&](u32x4 (&A)[U][R], int step0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (step0 + u) * KS;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (WT == WT_Q8)
          A[u][r] = ld_q8(ap[r] + k, sp[r] + (k >> 5));
        else
          A[u][r] = ld16(ap[r] + (size_t)(step0 + u) * wks);
      }
    }
  };
  auto load_stage_x = [&](u32x4 (&Bv)[U][C], int step0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (step0 + u) * KS;
#pragma unroll
      for (int c = 0; c < C; ++c) Bv[u][c] = ld16(bp[c] + (size_t)k * XB);
    }
  };
  auto load_stage = [&](u32x4 (&A)[U][R], u32x4 (&Bv)[U][C], int step0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (step0 + u) * KS;  // offset from kb
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (WT == WT_Q8)
          A[u][r] = ld_q8(ap[r] + k, sp[r] + (k >> 5));
        else
          A[u][r] = ld16(ap[r] + (size_t)(step0 + u) * wks);
      }
#pragma unroll
      for (int c = 0; c < C; ++c) Bv[u][c] = ld16(bp[c] + (size_t)k * XB);
    }
  };
  auto compute_stage = [&](const u32x4 (&A)[U][R], const u32x4 (&Bv)[U][C]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        u32x4 av = A[u][r];
        if constexpr (WT == WT_Q8) av = q8_to_f16(av);
#pragma unroll
        for (int c = 0; c < C; ++c) acc[r][c] = mma<WT>(av, Bv[u][c], acc[r][c]);
      }
  };

  // Full k-steps of this split, in stages of U, two stages in flight.
  const int nfull = (ke - kb) / KS;
  const int nst = nfull / U;
  {
    u32x4 A0[U][R], B0[U][C], A1[U][R], B1[U][C];
    if constexpr (NRM) {
      // The first weights are in flight while the activations are normalised.
      if (nst > 0) load_stage_w(A0, 0);
      stage_norm(mine, st_row, kb, ke);
      __syncthreads();
      if (nst > 0) load_stage_x(B0, 0);
    } else {
      if (nst > 0) load_stage(A0, B0, 0);
    }
    int st = 0;
    // steady state, no branches inside: stage st+1 (and st+2) load while st (st+1) computes
    for (; st + 2 < nst; st += 2) {
      load_stage(A1, B1, (st + 1) * U);
      compute_stage(A0, B0);
      load_stage(A0, B0, (st + 2) * U);
      compute_stage(A1, B1);
    }
    if (st + 1 < nst) {
      load_stage(A1, B1, (st + 1) * U);
      compute_stage(A0, B0);
      compute_stage(A1, B1);
    } else if (st < nst) {
      compute_stage(A0, B0);
    }
  }
  // Leftover full steps, then the K tail (a lane's vector is all in or all out
  // because K % PL == 0; out-of-range vectors become zero).
  for (int st = nst * U; st * KS < ke - kb; ++st) {
    const int k = st * KS;
    const bool kok = kb + k + koff + PL <= a.K;
    u32x4 av[R], bv[C];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if constexpr (WT == WT_Q8)
        av[r] = q8_to_f16(ld_q8(ap[r] + (kok ? k : 0), sp[r] + (kok ? (k >> 5) : 0)));
      else
        av[r] = ld16(ap[r] + (size_t)(kok ? st : 0) * wks);
      if (!kok) av[r] = zero4();
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      bv[c] = ld16(bp[c] + (size_t)(kok ? k : 0) * XB);
      if (!kok) bv[c] = zero4();
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) acc[r][c] = mma<WT>(av[r], bv[c], acc[r][c]);
  }

  if (a.S > 1) {
    // Split partials through LDS, in rounds of `per_round` waves; wave 0 adds
    // them to its own partial P_0 in ascending split order.
    constexpr int E = R * C * 4;
    // [per_round][E][64], after the norm staging
    float* red = (float*)(gsm + (NRM ? (size_t)a.S * n_st * st_row : 0));
    const int per_round = a.red_waves;
    for (int r0 = 1; r0 < a.S; r0 += per_round) {
      const int r1 = min(r0 + per_round, a.S);
      if (s >= r0 && s < r1) {
        float* dst = red + (size_t)(s - r0) * E * 64 + lane;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int c = 0; c < C; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[((r * C + c) * 4 + i) * 64] = acc[r][c][i];
      }
      __syncthreads();
      if (s == 0) {
        for (int s2 = r0; s2 < r1; ++s2) {
          const float* src = red + (size_t)(s2 - r0) * E * 64 + lane;
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[r][c][i] = acc[r][c][i] + src[((r * C + c) * 4 + i) * 64];
        }
      }
      __syncthreads();
    }
    if (s != 0) return;
  }

  if constexpr (EPI == EPI_RESID)
    epilogue<WT, EPI, R, C>(a, rb, cg, lane, acc, xpre);
  else
    epilogue<WT, EPI, R, C>(a, rb, cg, lane, acc);
}


// ---- wide panels: the activation panel staged in LDS ---------------------------
//
// At wide B the per-wave re-reads of the activation panel, not the weight
// stream, bound the split-K kernel above.  Here a workgroup of PW waves owns
// PW row blocks (the same R row tiles per wave as above) and one column group
// of 16*C lanes; the waves walk K together, staging each chunk of U k-steps
// of the [16*C, K] panel into LDS once for all of them (double-buffered, one
// barrier per chunk), while each wave streams its own weight rows from HBM.
//
// Same reduction contract: a wave runs the S splits of its row block one after
// the other, each a chain of MFMAs over ascending k-steps from zero, and keeps
// the running total ((P_0 + P_1) + ...) in registers, so every output bit
// equals the split-K kernel's.  In split mode (for projections with few row
// blocks) a workgroup runs one split only and writes P_s to a partial buffer
// [S][B][row blocks][rows per block]; k_fold then adds the partials in split
// order and runs the epilogue.
//
// Workgroups are numbered so that the column groups of one (row group, split)
// are consecutive and land on the same XCD (workgroups are dealt to the 8 XCDs
// in turn), so that their shared weight rows are read from HBM once into that
// XCD's L2.
constexpr int PW = 4;  // waves per workgroup in the panel kernel

template <int WT, int C>
struct PanelShape {
  static constexpr int KS = KStep<WT>::v;
  static constexpr int XB = WT == WT_F32 ? 4 : 2;
  static constexpr int U = C >= 8 ? 2 : 4;                 // k-steps per chunk
  static constexpr int CHUNK_BYTES = U * KS * XB;          // bytes of one lane row per chunk
  static constexpr int ROW_BYTES = CHUNK_BYTES + 16;       // padded LDS row
  static constexpr int COLS = TILE * C;
  static constexpr int BUF_BYTES = COLS * ROW_BYTES;
  static constexpr int PIECES = COLS * CHUNK_BYTES / 16;   // 16-byte pieces per chunk
  static constexpr int PER_THREAD = PIECES / (PW * 64);
  static_assert(PIECES % (PW * 64) == 0, "chunk pieces must divide evenly over the workgroup");
};

__host__ __device__ constexpr size_t panel_lds_bytes(int wt, int C) {
  return 2 * (size_t)(TILE * C) * ((C >= 8 ? 2 : 4) * (wt == WT_F32 ? 16 * 4 : 32 * 2) + 16);
}

// Buffer-descriptor loads (raw buffer, 32-bit data format): per-lane byte
// offsets stay in registers across the K walk and the k-step's offset is a
// scalar, so a fragment load costs no vector instructions.  An offset at or past
// the buffer's size reads zeros without touching memory.
__device__ inline __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(unsigned)std::min<size_t>(bytes, 0xffffffffu), 0x00020000);
}
__device__ inline u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ inline u32x2 buf_ld8(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}
__device__ inline unsigned buf_ld2(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return (unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}

// At most 256 registers per lane (two waves per SIMD): the 128-lane full-mode
// panels otherwise take 294 with their accumulators in AGPRs, one wave per
// SIMD, and wait on memory with nothing to switch to.
template <int WT, int EPI, int C, int RM, bool SPLIT>
__global__ __launch_bounds__(PW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_panel(GemmArgs a) {
  using PS = PanelShape<WT, C>;
  constexpr int R0 = gemm_rows(EPI);  // row tiles of one row block
  constexpr int R = R0 * RM;          // row tiles of one wave: RM consecutive row blocks
  constexpr int KS = PS::KS;
  constexpr int PL = KStep<WT>::per_lane;
  constexpr int U = PS::U;
  constexpr int EB = WT == WT_F32 ? 4 : (WT == WT_BF16 ? 2 : 1);
  constexpr int XB = PS::XB;
  extern __shared__ __attribute__((aligned(16))) char xl[];  // [2][COLS][ROW_BYTES]

  // workgroup -> (row group, split, column group), XCD-aware
  const int nWB = (a.nRB + RM - 1) / RM;  // groups of RM row blocks, one per wave
  const int nRG = (nWB + PW - 1) / PW;
  const int nRGS = nRG * (SPLIT ? a.S : 1);
  const int bi = blockIdx.x;
  const int cg = (bi >> 3) % a.nCG;
  const int rgs = ((bi >> 3) / a.nCG) * 8 + (bi & 7);
  if (rgs >= nRGS) return;  // padding workgroup: the whole workgroup leaves together
  const int rg = SPLIT ? rgs / a.S : rgs;
  const int split = SPLIT ? rgs % a.S : 0;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int rb = rg * PW + w;  // this wave's group of row blocks (past the end: it only helps stage)
  const int koff = PL * g4;

  // k-steps this workgroup walks: all of K, or one split.  When K is not a
  // multiple of the k-step, the last k-step of K is partial; it runs after the
  // chunk loop with per-lane masks, so the loop itself needs none.
  const int nks = (a.K + KS - 1) / KS;
  const int kps = a.Ks / KS;  // k-steps per split
  const int t0 = SPLIT ? split * kps : 0;
  const int t1 = SPLIT ? min(t0 + kps, nks) : nks;
  const bool tail = t1 == nks && a.K % KS != 0;
  const int tm = tail ? t1 - 1 : t1;  // end of the full k-steps
  const int nst = (tm - t0 + U - 1) / U;

  // Packed bf16 weights: the lane's slot of the row tile's first tile, one
  // tile (1 KB) per k-step (a tile past the end is clamped to the half's last).
  const bool packed = WT == WT_BF16 && a.wpack;
  const unsigned wks = packed ? 1024u : (unsigned)(KS * EB);  // weight bytes between k-steps
  const size_t wbytes = packed ? (size_t)(EPI == EPI_SWIGLU ? 2 : 1) * a.wtiles * (a.K / KS + PACK_GAP) * 1024
                               : (size_t)a.Nraw * a.K * EB;
  const __amdgpu_buffer_rsrc_t wrs = buf_rsrc(a.W, wbytes);
  const __amdgpu_buffer_rsrc_t srs = buf_rsrc(a.Ws, WT == WT_Q8 ? (size_t)a.Nraw * (a.K >> 5) * 2 : 0);
  const __amdgpu_buffer_rsrc_t xrs = buf_rsrc(a.X, (size_t)a.B * a.K * XB);
  unsigned wv[R], sv[R];  // byte offsets of this lane's weight vector at k = 0 (and its Q8 scale)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int row, tile;
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int H = R / 2;
      const int j = min(rb * TILE * H + TILE * (r % H) + r16, a.N - 1);
      row = r < H ? j : a.N + j;
      tile = min(rb * H + r % H, a.wtiles - 1) + (r < H ? 0 : a.wtiles);
    } else {
      row = min(rb * TILE * R + TILE * r + r16, a.N - 1);
      tile = min(rb * R + r, a.wtiles - 1);
    }
    wv[r] = packed ? (unsigned)((size_t)tile * (a.K / KS + PACK_GAP) * 1024 + lane * 16)
                   : (unsigned)(((size_t)row * a.K + koff) * EB);
    sv[r] = (unsigned)((size_t)row * (a.K >> 5) * 2);
  }
  auto ld_w = [&](int r, int t) -> u32x4 {
    if constexpr (WT == WT_Q8) {
      const u32x2 q = buf_ld8(wrs, wv[r], (unsigned)t * KS);
      return u32x4{q.x, q.y, buf_ld2(srs, sv[r], (unsigned)t * 2), 0u};
    } else {
      return buf_ld16(wrs, wv[r], (unsigned)t * wks);
    }
  };

  // Weight fragments of chunk st: full k-steps t0 + st*U + u; steps past the
  // last full one reload it (an L1/L2 hit) and are never used.
  auto load_w = [&](u32x4 (&A)[U][R], int st) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = max(t0, min(t0 + st * U + u, tm - 1));
#pragma unroll
      for (int r = 0; r < R; ++r) A[u][r] = ld_w(r, t);
    }
  };
  // The panel's chunk st: PER_THREAD 16-byte pieces per thread.  Chunks past the
  // last reload it; pieces past K (in a last, partial chunk) are never read.
  constexpr int PPC = PS::CHUNK_BYTES / 16;  // pieces per lane row
  unsigned xv[PS::PER_THREAD];
#pragma unroll
  for (int j = 0; j < PS::PER_THREAD; ++j) {
    const int pc = j * PW * 64 + tid;
    const int col = min(cg * PS::COLS + pc / PPC, a.B - 1);
    xv[j] = (unsigned)(((size_t)col * a.K + (pc % PPC) * (16 / XB)) * XB);
  }
  auto load_x = [&](u32x4 (&xr)[PS::PER_THREAD], int st) {
    const unsigned kc = (unsigned)(t0 + min(st, max(nst - 1, 0)) * U) * KS * XB;
#pragma unroll
    for (int j = 0; j < PS::PER_THREAD; ++j) xr[j] = buf_ld16(xrs, xv[j] + kc, 0u);
  };
  auto store_x = [&](const u32x4 (&xr)[PS::PER_THREAD], int buf) {
    char* base = xl + (size_t)buf * PS::BUF_BYTES;
#pragma unroll
    for (int j = 0; j < PS::PER_THREAD; ++j) {
      const int pc = j * PW * 64 + tid;
      *(u32x4*)(base + (size_t)(pc / PPC) * PS::ROW_BYTES + (pc % PPC) * 16) = xr[j];
    }
  };

  // The running total starts at -0: (-0) + x is x bit for bit for every x
  // (-0 included), so adding P_0 to it gives exactly P_0.
  f32x4 acc[R][C], tot[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      tot[r][c] = f32x4{-0.f, -0.f, -0.f, -0.f};
    }
  int tf = t0 + kps;  // full mode: the first k-step of the next split
  // split boundary: fold the finished split's chain into the running total.
  // Split lengths are whole multiples of two chunks, so boundaries fall
  // between chunk pairs (or before the partial last k-step of K).
  auto fold = [&]() {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[r][c][i] = tot[r][c][i] + acc[r][c][i];
        acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  };
  // A uniform branch taken once per split: the volatile statement keeps it a
  // branch outside the MFMA stream.
  auto fold_at = [&](int t) {
    if constexpr (!SPLIT) {
      if (t == tf) {
        __asm__ volatile("");
        fold();
        tf += kps;
      }
    }
  };
  auto step = [&](u32x4 av0[R], const u32x4 (&bv)[C], int t) {
    (void)t;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      u32x4 av = av0[r];
      if constexpr (WT == WT_Q8) av = q8_to_f16(av);
#pragma unroll
      for (int c = 0; c < C; ++c) acc[r][c] = mma<WT>(av, bv[c], acc[r][c]);
    }
  };
  auto compute = [&](u32x4 (&A)[U][R], int buf, int st) {
    const char* base = xl + (size_t)buf * PS::BUF_BYTES + (size_t)r16 * PS::ROW_BYTES + g4 * 16;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + st * U + u;
      if (t >= tm) break;
      u32x4 bv[C];
#pragma unroll
      for (int c = 0; c < C; ++c) bv[c] = *(const u32x4*)(base + (size_t)c * TILE * PS::ROW_BYTES + u * KS * XB);
      step(A[u], bv, t);
    }
  };

  {
    // Two chunks of weights in flight.  The loop has no exit between its two
    // halves and the LDS stores are unconditional (a chunk past the end stores
    // data nobody reads), which keeps the compiler's waits on the loads exact.
    u32x4 A0[U][R], A1[U][R], xr[PS::PER_THREAD];
    load_x(xr, 0);
    load_w(A0, 0);
    store_x(xr, 0);
    load_x(xr, 1);
    load_w(A1, 1);
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
      fold_at(t0 + st * U);
      compute(A0, 0, st);
      store_x(xr, 1);
      if (st + 2 < nst) {
        load_x(xr, st + 2);
        load_w(A0, st + 2);
      }
      __syncthreads();
      compute(A1, 1, st + 1);  // nothing when st + 1 == nst
      store_x(xr, 0);
      if (st + 3 < nst) {
        load_x(xr, st + 3);
        load_w(A1, st + 3);
      }
      __syncthreads();
    }
  }
  if (tail) {
    // The partial last k-step: lane vectors past K are zero on both sides.
    const int t = tm;
    fold_at(t);
    const bool kok = t * KS + koff + PL <= a.K;
    u32x4 av[R], bv[C];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      av[r] = ld_w(r, kok ? t : 0);
      if (!kok) av[r] = zero4();
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int col = min(cg * PS::COLS + TILE * c + r16, a.B - 1);
      bv[c] = buf_ld16(xrs, (unsigned)(((size_t)col * a.K + (kok ? t * KS + koff : 0)) * XB), 0u);
      if (!kok) bv[c] = zero4();
    }
    step(av, bv, t);
  }
  if (rb >= nWB) return;
  if constexpr (SPLIT) {
    // P_s of this wave's row tiles for the lanes of the column group, as
    // [split][lane][row block][R0 tiles][16]; wave tile r belongs to row block
    // rb*RM + r % RM as its gate (r < RM) or up tile (SwiGLU), else to row
    // block rb*RM + r / R0 as its tile r % R0.
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int col = cg * PS::COLS + TILE * c + r16;
      if (col >= a.B) continue;
      float* dst = a.part + (size_t)split * a.B * a.nRB * (R0 * TILE) + (size_t)col * a.nRB * (R0 * TILE) + 4 * g4;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int ob = rb * RM + (EPI == EPI_SWIGLU ? r % RM : r / R0);
        const int t0r = EPI == EPI_SWIGLU ? r / RM : r % R0;
        if (ob < a.nRB) *(f32x4*)(dst + (size_t)ob * (R0 * TILE) + t0r * TILE) = acc[r][c];
      }
    }
  } else {
    fold();
    epilogue<WT, EPI, R, C, RM>(a, rb, cg, lane, tot);
  }
}

// Split mode's second half: out = ((P_0 + P_1) + ...) + P_{S-1}, then the
// epilogue, one wave per (row block, 16 lanes).
template <int WT, int EPI>
__global__ __launch_bounds__(64) void k_fold(GemmArgs a) {
  constexpr int R = gemm_rows(EPI);
  const int rb = blockIdx.x % a.nRB;
  const int ct = blockIdx.x / a.nRB;
  const int lane = threadIdx.x;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int col = min(ct * TILE + r16, a.B - 1);
  const size_t sstride = (size_t)a.B * a.nRB * (R * TILE);
  const float* src = a.part + ((size_t)col * a.nRB + rb) * (R * TILE) + 4 * g4;
  // All partials are loaded before the first add (one memory round trip; slots
  // past S reload the last split and are not added), then summed in split order.
  f32x4 pv[R][GEMM_MAX_SPLIT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < GEMM_MAX_SPLIT; ++s) pv[r][s] = *(const f32x4*)(src + min(s, a.S - 1) * sstride + r * TILE);
  f32x4 acc[R][1];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    f32x4 v = pv[r][0];
#pragma unroll
    for (int s = 1; s < GEMM_MAX_SPLIT; ++s)
      if (s < a.S) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = v[i] + pv[r][s][i];
      }
    acc[r][0] = v;
  }
  epilogue<WT, EPI, R, 1>(a, rb, ct, lane, acc);
}

// Split mode's second half for a residual projection followed by RMSNorm, one
// workgroup per lane: x += ((P_0 + P_1) + ...) + P_{S-1}, then the next
// norm's xn = (x * r) * g.  Every value is the one the separate kernels give:
// thread t owns row blocks t, t + 256 (16 rows each); a block's sum of squares
// is taken as the residual epilogue takes it (rows 4j..4j+3 in order with
// fused multiply-adds, then (s0 + s1) + (s2 + s3)), the lane's statistic as
// the norm kernel takes it (the row blocks strided over 256 threads, then
// block_sum), and r = 1 / sqrt(ss / N + eps).
template <int WT>
__global__ __launch_bounds__(256) void k_fold_norm(GemmArgs a) {
  constexpr int MAXRB = 2;  // row blocks per thread: N up to 8192
  const int b = blockIdx.x, t = threadIdx.x;
  const size_t sstride = (size_t)a.B * a.nRB * TILE;
  float xv[MAXRB][TILE];
  float part = 0.f;
#pragma unroll
  for (int k = 0; k < MAXRB; ++k) {
    const int rb = t + 256 * k;
    if (rb >= a.nRB) break;
    const float* src = a.part + ((size_t)b * a.nRB + rb) * TILE;
    f32x4 pv[GEMM_MAX_SPLIT][4];
#pragma unroll
    for (int s2 = 0; s2 < GEMM_MAX_SPLIT; ++s2)
#pragma unroll
      for (int q = 0; q < 4; ++q) pv[s2][q] = *(const f32x4*)(src + min(s2, a.S - 1) * sstride + 4 * q);
    float* xr = a.out + (size_t)b * a.N + rb * TILE;
    float sg[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 v = pv[0][q];
#pragma unroll
      for (int s2 = 1; s2 < GEMM_MAX_SPLIT; ++s2)
        if (s2 < a.S) {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = v[i] + pv[s2][q][i];
        }
      const f32x4 xo = *(const f32x4*)(xr + 4 * q);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = xo[i] + v[i];
        xv[k][4 * q + i] = x;
        ss = __builtin_fmaf(x, x, ss);
      }
      *(f32x4*)(xr + 4 * q) = f32x4{xv[k][4 * q], xv[k][4 * q + 1], xv[k][4 * q + 2], xv[k][4 * q + 3]};
      sg[q] = ss;
    }
    part += (sg[0] + sg[1]) + (sg[2] + sg[3]);
  }
  const float ss = block_sum(part);
  const float r = 1.0f / sqrtf(ss / (float)a.N + a.norm_eps);
  // xn of the thread's rows in 16-byte stores (its 16 rows are consecutive)
#pragma unroll
  for (int k = 0; k < MAXRB; ++k) {
    const int rb = t + 256 * k;
    if (rb >= a.nRB) break;
    const size_t o = (size_t)b * a.N + rb * TILE;
    float v[TILE];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 g = *(const f32x4*)(a.norm_g + rb * TILE + 4 * q);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * q + i] = (xv[k][4 * q + i] * r) * g[i];
    }
    if constexpr (WT == WT_F32) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4*)((float*)a.norm_out + o + 4 * q) = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = v[8 * h + 2 * e], hi = v[8 * h + 2 * e + 1];
          if constexpr (WT == WT_BF16) {
            w[e] = (unsigned)f2bf(lo) | ((unsigned)f2bf(hi) << 16);
          } else {
            w[e] = (unsigned)__builtin_bit_cast(uint16_t, (_Float16)lo) |
                   ((unsigned)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
          }
        }
        *(u32x4*)((uint16_t*)a.norm_out + o + 8 * h) = w;
      }
    }
  }
}

// ---- dense tiles: both operands staged in LDS (wide panels and prefill) ---------
//
// Once B makes the contraction dense ("MODEL-BATCHING-RESULTS — multi-user
// batched decode, measured", section "The honest ceiling": throughput is then
// capped by the matrix units, not by the weight stream), the matrix cores need
// operands reused from on-chip memory.  A workgroup of eight waves owns a tile
// of 256 weight rows (SwiGLU: 128 gate/up pairs) by 128 lanes, each wave a
// 64 x 64 part as 4 x 4 MFMA blocks (four wave rows by two wave columns), and
// walks K in stages of two k-steps (64 elements, 128 bytes of every row).  At
// full MFMA rate the tile draws 48 bytes per clock per compute unit through
// L2, against 64 for 128 x 128 tiles (4096-row prefill projections: 36% ->
// 42% of MFMA peak; 256 and 512 lanes: 10-20% faster, though 256 lanes give
// gate|up only 224 such workgroups).
//
// Loads go from memory straight into LDS (buffer loads with the LDS as
// destination: no registers, no LDS write instructions).  One load
// instruction fills a 1 KB block with 8 whole 128-byte row segments, eight
// consecutive lanes per row, so every instruction reads whole cache lines;
// the lanes of a row take its 16-byte pieces in the order p ^ (row % 16) / 2,
// which spreads the 16 rows of an MFMA operand over all LDS banks when a wave
// reads piece p of each of them (one 16-byte load per lane, no conflicts).
// Three slots of 48 KB (one workgroup per compute unit, two waves per SIMD):
// the loads run two stages ahead of the MFMAs.  Each stage starts with one
// barrier, after which every wave's loads of it have landed (each waits for
// its own first) and every wave has finished reading the slot the new loads
// overwrite.
//
// Same reduction contract: each 16 x 16 block is a chain of
// v_mfma_f32_16x16x32_bf16 over ascending k-steps from zero per split.
// Modes: DN_ONE, one split per workgroup whose partial goes straight to the
// epilogue (the projection has one split: (-0) + P_0 is P_0); DN_PART, one
// split per workgroup written as a partial for k_fold / k_fold_norm; DN_FULL,
// every split of K in one workgroup, KPS k-steps each, each split's chain
// folded in order into a running total ((P_0 + P_1) + ...) at the stage where
// the next split starts.  So every output bit equals the other families'.
constexpr int DN_ROWS = 256, DN_COLS = 128;
constexpr int DN_WAVES = 8;
constexpr int DN_BLOCK = 1024;             // 8 rows x 128 bytes
constexpr int DN_WBLK = DN_ROWS / 8;       // weight blocks of a stage, then 16 activation blocks
constexpr int DN_STAGE = (DN_WBLK + 16) * DN_BLOCK;
constexpr int DN_WPW = DN_WBLK / DN_WAVES;  // weight blocks loaded per wave
constexpr int DN_XPW = 16 / DN_WAVES;       // activation blocks loaded per wave
enum { DN_ONE = 0, DN_PART = 1, DN_FULL = 2 };

template <int EPI, int MODE, int KPS>
__global__ __launch_bounds__(DN_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_dense(GemmArgs a) {
  constexpr int R0 = gemm_rows(EPI);
  constexpr int RM = 4 / R0;  // row blocks of a wave's four row tiles
  constexpr int KS = 32;
  constexpr bool SPLIT = MODE == DN_PART;
  // stage slots, as separate objects so that the compiler can tell the slot
  // being read from the slots being loaded (else it waits for every load
  // before each LDS read)
  __shared__ __attribute__((aligned(16))) char sl0[DN_STAGE];
  __shared__ __attribute__((aligned(16))) char sl1[DN_STAGE];
  __shared__ __attribute__((aligned(16))) char sl2[DN_STAGE];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int wm = w >> 1, wn = w & 1;
  const int l16 = lane & 15, g4 = lane >> 4;

  // workgroup -> (row group with its split, lane group).  Workgroups are dealt
  // to the 8 XCDs in turn; XCD x takes the row groups x, x + 8, ... (its
  // weight rows come from HBM once, into its own L2), and walks them in blocks
  // of DN_RB row groups, all row groups of a block for one lane group, then
  // the next lane group: the workgroups an XCD holds at a time then share a
  // few weight and activation tiles instead of re-reading the activation
  // tiles from beyond L2 for every row group.
  const int outs = EPI == EPI_SWIGLU ? DN_ROWS / 2 : DN_ROWS;  // outputs (rows or pairs) per row group
  const int nRG = (a.N + outs - 1) / outs;
  const int nRGS = nRG * (SPLIT ? a.S : 1);
  constexpr int DN_RB = 8;
  const int bi = blockIdx.x;
  const int xcd = bi & 7, li = bi >> 3;
  const int rows_x = (nRGS - xcd + 7) / 8;  // row groups of this XCD
  const int blk = li / (DN_RB * a.nCG);
  const int within = li - blk * DN_RB * a.nCG;
  const int rows_b = min(DN_RB, rows_x - blk * DN_RB);  // row groups of this block
  if (rows_b <= 0) return;  // padding workgroup: the whole workgroup leaves together
  const int cg = within / rows_b;
  if (cg >= a.nCG) return;
  const int rgs = xcd + 8 * (blk * DN_RB + within % rows_b);
  const int rg = SPLIT ? rgs / a.S : rgs;
  const int split = SPLIT ? rgs % a.S : 0;

  const int nks = a.K / KS;  // K is a multiple of 128
  const int kps = a.Ks / KS;
  const int t0 = SPLIT ? split * kps : 0;
  const int ns = ((SPLIT ? min(t0 + kps, nks) : nks) - t0) / 2;  // stages walked: an even number

  // Weight row of tile row q: MFMA row tile q / 16 of the tile, row q % 16 in
  // it.  Row tiles 4 wm .. 4 wm + 3 are wave row wm's; SwiGLU row tiles are
  // [gate, gate, up, up] of 32 pairs.
  auto wrow = [&](int q) -> int {
    const int f = q >> 4, fm = f >> 2, r = f & 3, i = q & 15;
    if constexpr (EPI == EPI_SWIGLU) {
      const int j = min(rg * (DN_ROWS / 2) + fm * 32 + (r & 1) * 16 + i, a.N - 1);
      return r < 2 ? j : a.N + j;
    } else {
      return min(rg * DN_ROWS + q, a.N - 1);
    }
  };
  // Packed weights (1 KB tiles of 16 rows x one k-step): weight block j of a
  // stage is row tile j / 2 of the tile at its k-step j % 2, loaded whole.
  const bool packed = a.wpack != 0;
  auto wtile = [&](int f) -> int {  // global tile of the tile's row tile f (0..15)
    const int fm = f >> 2, r = f & 3;
    if constexpr (EPI == EPI_SWIGLU)
      return min(rg * (DN_ROWS / 32) + fm * 2 + (r & 1), a.wtiles - 1) + (r < 2 ? 0 : a.wtiles);
    else
      return min(rg * (DN_ROWS / 16) + f, a.wtiles - 1);
  };
  const size_t wbytes = packed ? (size_t)(EPI == EPI_SWIGLU ? 2 : 1) * a.wtiles * (a.K / KS + PACK_GAP) * 1024
                               : (size_t)a.Nraw * a.K * 2;
  const __amdgpu_buffer_rsrc_t wrs = buf_rsrc(a.W, wbytes);
  const __amdgpu_buffer_rsrc_t xrs = buf_rsrc(a.X, (size_t)a.B * a.K * 2);
  // this wave fills weight blocks DN_WPW w .. and activation blocks DN_XPW w ..;
  // row-major: lane row 8 j + lane / 8 of block j, its piece (lane % 8) ^ (row % 16) / 2
  unsigned wv[DN_WPW], xv[DN_XPW];
#pragma unroll
  for (int jj = 0; jj < DN_WPW; ++jj) {
    const int jb = DN_WPW * w + jj;
    const int q = 8 * jb + (lane >> 3);
    const unsigned piece = (unsigned)((lane & 7) ^ ((q & 15) >> 1)) * 16;
    wv[jj] = packed ? (unsigned)(((size_t)wtile(jb >> 1) * (a.K / KS + PACK_GAP) + (jb & 1)) * 1024 + lane * 16)
                    : (unsigned)((size_t)wrow(q) * a.K * 2) + piece;
  }
  const int wstep = packed ? 2048 : 128;  // weight bytes between stages
#pragma unroll
  for (int jj = 0; jj < DN_XPW; ++jj) {
    const int q = 8 * (DN_XPW * w + jj) + (lane >> 3);
    const unsigned piece = (unsigned)((lane & 7) ^ ((q & 15) >> 1)) * 16;
    const int col = min(cg * DN_COLS + q, a.B - 1);
    xv[jj] = (unsigned)((size_t)col * a.K * 2) + piece;
  }
  // stage st of the walk into a slot (a stage past the last reloads it into a
  // slot nobody reads, so every stage issues the same loads)
  auto load = [&](char* slot, int st) {
    const int s2 = t0 / 2 + min(st, ns - 1);  // the stage's pair of k-steps
    const int kb = s2 * 128, kbw = s2 * wstep;
#pragma unroll
    for (int jj = 0; jj < DN_WPW; ++jj)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, slot + (DN_WPW * w + jj) * DN_BLOCK, 16, (int)wv[jj], kbw, 0, 0);
#pragma unroll
    for (int jj = 0; jj < DN_XPW; ++jj)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, slot + (DN_WBLK + DN_XPW * w + jj) * DN_BLOCK, 16, (int)xv[jj],
                                               kb, 0, 0);
  };
  // Start of a stage: this wave's loads of it have landed (those of the next
  // stage, issued after them, may still be in flight), then the barrier.
  auto arrive = [&]() {
    __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(DN_WPW + DN_XPW) : "memory");
  };
  // Piece p of tile row 16 t + l16 sits at block 2 t + l16 / 8, row l16 % 8,
  // slot p ^ l16 / 2: per lane, the offsets of k-step 0 and 1 (p = 4 ks + g4).
  // Packed weights: the lane's slot of block 2 t + ks.
  unsigned ro[2], wo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    ro[ks] = (unsigned)((l16 >> 3) * DN_BLOCK + (l16 & 7) * 128 + (((4 * ks + g4) ^ (l16 >> 1)) << 4));
    wo[ks] = packed ? (unsigned)(ks * DN_BLOCK + lane * 16) : ro[ks];
  }
  auto compute = [&](f32x4 (&acc)[4][4], const char* slot) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 av[4], bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = *(const u32x4*)(slot + (2 * (4 * wm + r)) * DN_BLOCK + wo[ks]);
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = *(const u32x4*)(slot + (DN_WBLK + 2 * (4 * wn + c)) * DN_BLOCK + ro[ks]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = mma<WT_BF16>(av[r], bv[c], acc[r][c]);
    }
  };

  // The running total of DN_FULL starts at -0: (-0) + x is x bit for bit.
  f32x4 ch[4][4], tot[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ch[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      tot[r][c] = f32x4{-0.f, -0.f, -0.f, -0.f};
    }
  auto fold = [](f32x4 (&acc)[4][4], f32x4 (&sum)[4][4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[r][c][i] = sum[r][c][i] + acc[r][c][i];
        acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  };
  // Stage st sits in slot (st - r) % 3, r = ns % 3, so that the loop walks
  // whole triples of stages after r stages of prologue; at its start the
  // loads of st + 2 go into the slot of st - 1.  DN_FULL folds at each split
  // boundary (a uniform branch kept outside the MFMA stream).
  int nf = KPS / 2;  // stage at which the next split starts
  auto stage = [&](f32x4 (&acc)[4][4], f32x4 (&sum)[4][4], char* cur, char* nxt2, int st) {
    if constexpr (MODE == DN_FULL) {
      if (st == nf) {
        __asm__ volatile("");
        fold(acc, sum);
        nf += KPS / 2;
      }
    }
    arrive();
    load(nxt2, st + 2);
    compute(acc, cur);
  };
  const int r = ns % 3;
  if (r == 1) {
    load(sl2, 0);
    load(sl0, 1);
    stage(ch, tot, sl2, sl1, 0);
  } else if (r == 2) {
    load(sl1, 0);
    load(sl2, 1);
    stage(ch, tot, sl1, sl0, 0);
    stage(ch, tot, sl2, sl1, 1);
  } else {
    load(sl0, 0);
    load(sl1, 1);
  }
  for (int st = r; st < ns; st += 3) {
    stage(ch, tot, sl0, sl2, st);
    stage(ch, tot, sl1, sl0, st + 1);
    stage(ch, tot, sl2, sl1, st + 2);
  }
  if constexpr (MODE == DN_FULL) fold(ch, tot);
  // the loads past the end must land before the workgroup's LDS is released
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const int rb = rg * (DN_WAVES / 2) + wm;  // this wave's group of RM row blocks
  const int cgw = cg * 2 + wn;              // this wave's group of 64 lanes
  if constexpr (MODE == DN_PART) {
    // P_s as [split][lane][row block][R0 tiles][16], as the panels write it
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = cgw * 64 + TILE * c + l16;
      if (col >= a.B) continue;
      float* dst = a.part + (size_t)split * a.B * a.nRB * (R0 * TILE) + (size_t)col * a.nRB * (R0 * TILE) + 4 * g4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ob = rb * RM + (EPI == EPI_SWIGLU ? r % RM : r / R0);
        const int t0r = EPI == EPI_SWIGLU ? r / RM : r % R0;
        if (ob < a.nRB) *(f32x4*)(dst + (size_t)ob * (R0 * TILE) + t0r * TILE) = ch[r][c];
      }
    }
  } else if constexpr (MODE == DN_FULL) {
    epilogue<WT_BF16, EPI, 4, 4, RM>(a, rb, cgw, lane, tot);
  } else {
    epilogue<WT_BF16, EPI, 4, 4, RM>(a, rb, cgw, lane, ch);
  }
}

// K-steps per split of the DN_FULL instances built (per epilogue; the
// Mistral-7B shapes: QKV and O 512-element splits, gate|up and the head 1024,
// down 1792), or 0.
static int dense_full_kps(int epi, int Ks) {
  const int kps = Ks / 32;
  switch (epi) {
    case EPI_STORE: return kps == 16 ? 16 : 0;
    case EPI_RESID: return kps == 16 || kps == 56 ? kps : 0;
    default: return kps == 32 ? 32 : 0;
  }
}

int dense_mode_available(int epi, int K, int Ks, int S) {
  if (S == 1) return 1;
  return dense_full_kps(epi, Ks) && K % Ks == 0;
}

int dense_workgroups(const GemmArgs& a, int epi, int split) {
  const int outs = epi == EPI_SWIGLU ? DN_ROWS / 2 : DN_ROWS;
  const int nRGS = ((a.N + outs - 1) / outs) * (split ? a.S : 1);
  const int nCG = (a.B + DN_COLS - 1) / DN_COLS;
  return ((nRGS + 7) / 8) * 8 * nCG;
}

template <int EPI, int MODE, int KPS>
static hipError_t launch_dense_k(const GemmArgs& a, int split, hipStream_t st) {
  hipLaunchKernelGGL((k_dense<EPI, MODE, KPS>), dim3(dense_workgroups(a, EPI, split)), dim3(DN_WAVES * 64), 0, st, a);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_dense_epi(int split, const GemmArgs& a, hipStream_t st) {
  if (split) {
    hipError_t e = launch_dense_k<EPI, DN_PART, 0>(a, 1, st);
    if (e != hipSuccess) return e;
    if (EPI == EPI_RESID && a.norm_out) {
      if (!fold_norm_supported(a.N)) return hipErrorInvalidValue;
      hipLaunchKernelGGL((k_fold_norm<WT_BF16>), dim3(a.B), dim3(256), 0, st, a);
    } else if (EPI == EPI_STORE && a.fold_elsewhere) {
      // the consumer adds the partials
    } else {
      const int nct = (a.B + TILE - 1) / TILE;
      hipLaunchKernelGGL((k_fold<WT_BF16, EPI>), dim3(a.nRB * nct), dim3(64), 0, st, a);
    }
    return hipGetLastError();
  }
  if (a.S == 1) return launch_dense_k<EPI, DN_ONE, 0>(a, 0, st);
  switch (dense_full_kps(EPI, a.Ks)) {
    case 16:
      if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) return launch_dense_k<EPI, DN_FULL, 16>(a, 0, st);
      break;
    case 32:
      if constexpr (EPI == EPI_SWIGLU || EPI == EPI_HEAD) return launch_dense_k<EPI, DN_FULL, 32>(a, 0, st);
      break;
    case 56:
      if constexpr (EPI == EPI_RESID) return launch_dense_k<EPI, DN_FULL, 56>(a, 0, st);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dense(int epi, int split, const GemmArgs& a, hipStream_t st) {
  if (a.S < 1 || a.K % 128 != 0 || a.Ks % 256 != 0) return hipErrorInvalidValue;
  if (!split && !dense_mode_available(epi, a.K, a.Ks, a.S)) return hipErrorInvalidValue;
  if (a.nRB <= 0 || a.B <= 0) return hipSuccess;
  GemmArgs g = a;
  g.nCG = (a.B + DN_COLS - 1) / DN_COLS;
  switch (epi) {
    case EPI_STORE: return launch_dense_epi<EPI_STORE>(split, g, st);
    case EPI_RESID: return launch_dense_epi<EPI_RESID>(split, g, st);
    case EPI_SWIGLU: return launch_dense_epi<EPI_SWIGLU>(split, g, st);
    default: return launch_dense_epi<EPI_HEAD>(split, g, st);
  }
}

template <int WT, int EPI>
static hipError_t launch_c(int C, const GemmArgs& a, int blocks, hipStream_t st) {
  const dim3 blk(64 * a.S);
  size_t lds = a.S > 1 ? (size_t)a.red_waves * gemm_rows(EPI) * C * 4 * 64 * sizeof(float) : 0;
  if (a.in_x) {
    constexpr int XB = WT == WT_F32 ? 4 : 2;
    if (C != 1 || EPI == EPI_RESID || !gemm_norm_in_supported(a.B, a.K, a.S, a.Ks, XB, a.in_ssq_n))
      return hipErrorInvalidValue;
    lds += (size_t)a.S * a.B * (a.Ks * XB + 16);
    if constexpr (EPI != EPI_RESID) hipLaunchKernelGGL((k_gemm<WT, EPI, 1, true>), dim3(blocks), blk, lds, st, a);
    return hipGetLastError();
  }
  switch (C) {
    case 1: hipLaunchKernelGGL((k_gemm<WT, EPI, 1>), dim3(blocks), blk, lds, st, a); break;
    case 2: hipLaunchKernelGGL((k_gemm<WT, EPI, 2>), dim3(blocks), blk, lds, st, a); break;
    default: hipLaunchKernelGGL((k_gemm<WT, EPI, 4>), dim3(blocks), blk, lds, st, a); break;
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

hipError_t launch_gemm(int wt, int epi, int C, const GemmArgs& a, hipStream_t st) {
  if (a.S < 1 || a.S > GEMM_MAX_SPLIT) return hipErrorInvalidValue;
  GemmArgs g = a;
  // LDS per split round: at most 32 KB
  g.red_waves =
      (int)std::max<size_t>(1, (32768 / ((size_t)gemm_rows(epi) * C * 4 * 64 * sizeof(float))));
  const int blocks = a.nRB * a.nCG;
  if (blocks <= 0) return hipSuccess;
  switch (wt) {
    case WT_F32: return launch_epi<WT_F32>(epi, C, g, blocks, st);
    case WT_BF16: return launch_epi<WT_BF16>(epi, C, g, blocks, st);
    default: return launch_epi<WT_Q8>(epi, C, g, blocks, st);
  }
}

int panel_workgroups(const GemmArgs& a, int C, int rm, int split) {
  const int nRG = ((a.nRB + rm - 1) / rm + PW - 1) / PW;
  const int nRGS = nRG * (split ? a.S : 1);
  const int nCG = (a.B + TILE * C - 1) / (TILE * C);
  return ((nRGS + 7) / 8) * 8 * nCG;
}

template <int WT, int EPI, int C, int RM>
static hipError_t launch_panel_c(int split, const GemmArgs& a, hipStream_t st) {
  const size_t lds = panel_lds_bytes(WT, C);
  const int blocks = panel_workgroups(a, C, RM, split);
  if (split) {
    hipLaunchKernelGGL((k_panel<WT, EPI, C, RM, true>), dim3(blocks), dim3(PW * 64), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (EPI == EPI_RESID && a.norm_out) {
      if (!fold_norm_supported(a.N)) return hipErrorInvalidValue;
      hipLaunchKernelGGL((k_fold_norm<WT>), dim3(a.B), dim3(256), 0, st, a);
    } else if (EPI == EPI_STORE && a.fold_elsewhere) {
      // the consumer (attention) adds the partials
    } else {
      const int nct = (a.B + TILE - 1) / TILE;
      hipLaunchKernelGGL((k_fold<WT, EPI>), dim3(a.nRB * nct), dim3(64), 0, st, a);
    }
  } else {
    // full mode with one row block per wave only (two would not fit in 256
    // registers with the running total)
    if constexpr (RM == 1)
      hipLaunchKernelGGL((k_panel<WT, EPI, C, RM, false>), dim3(blocks), dim3(PW * 64), lds, st, a);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int WT, int EPI>
static hipError_t launch_panel_epi(int C, int rm, int split, const GemmArgs& a, hipStream_t st) {
  // Row blocks per wave: 1, or 2 in split mode.
  if (rm == 1) {
    switch (C) {
      case 2: return launch_panel_c<WT, EPI, 2, 1>(split, a, st);
      case 4: return launch_panel_c<WT, EPI, 4, 1>(split, a, st);
      case 8: return launch_panel_c<WT, EPI, 8, 1>(split, a, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (rm == 2) {
    switch (C) {
      case 4: return launch_panel_c<WT, EPI, 4, 2>(split, a, st);
      case 8: return launch_panel_c<WT, EPI, 8, 2>(split, a, st);
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}

template <int WT>
static hipError_t launch_panel_wt(int epi, int C, int rm, int split, const GemmArgs& a, hipStream_t st) {
  switch (epi) {
    case EPI_STORE: return launch_panel_epi<WT, EPI_STORE>(C, rm, split, a, st);
    case EPI_RESID: return launch_panel_epi<WT, EPI_RESID>(C, rm, split, a, st);
    case EPI_SWIGLU: return launch_panel_epi<WT, EPI_SWIGLU>(C, rm, split, a, st);
    default: return launch_panel_epi<WT, EPI_HEAD>(C, rm, split, a, st);
  }
}

hipError_t launch_panel(int wt, int epi, int C, int rm, int split, const GemmArgs& a, hipStream_t st) {
  if (a.S < 1) return hipErrorInvalidValue;
  if (a.nRB <= 0 || a.B <= 0) return hipSuccess;
  GemmArgs g = a;
  g.nCG = (a.B + TILE * C - 1) / (TILE * C);
  switch (wt) {
    case WT_F32: return launch_panel_wt<WT_F32>(epi, C, rm, split, g, st);
    case WT_BF16: return launch_panel_wt<WT_BF16>(epi, C, rm, split, g, st);
    default: return launch_panel_wt<WT_Q8>(epi, C, rm, split, g, st);
  }
}

}  // namespace cbd
