// Internal interface between the host runtime (cbd_runtime.hip) and the
// gfx950 kernels (cbd_gemm.hip, cbd_attn.hip, cbd_misc.hip).  Not installed.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cbd {

enum WType { WT_F32 = 0, WT_BF16 = 1, WT_Q8 = 2 };
enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_HEAD = 3 };

// Keys per attention split.  A constant of the design: the per-lane result
// never depends on B, on the lane's slot or on the other lanes.
constexpr int ATTN_SPLIT = 256;
// Rows of one MFMA tile, and 16-row tiles per wave in the projection kernels.
constexpr int TILE = 16;
constexpr int GEMM_R = 2;

// Projection over a panel: Y[b][n] = sum_k W[n][k] * X[b][k] for b < B.
// The reduction contract (identical in every kernel variant and batch width):
// K is cut into S splits of Ks elements (the last may be shorter); each
// split's partial is a chain of MFMAs over ascending k-steps starting from
// zero; the output is ((P_0 + P_1) + P_2) + ... in split order, then the
// epilogue.  So lane b's outputs are the same bits whatever B is.
struct GemmArgs {
  const void* W;        // data plane [Nraw, K]
  const uint16_t* Ws;   // Q8_0 scale plane [Nraw, K/32] (binary16), or null
  const void* X;        // activation panel [B, K] (f32 / bf16 / f16 by weight type)
  int N;                // output rows (EPI_SWIGLU: ffn, the number of gate/up pairs)
  int Nraw;             // rows of W (EPI_SWIGLU: 2 * ffn)
  int K;
  int B;
  int S;                // splits
  int Ks;               // elements per split (multiple of the k-step)
  int nRB;              // row blocks of TILE*GEMM_R rows (SWIGLU: TILE*GEMM_R/2 pairs)
  int nCG;              // column groups
  float* out;           // STORE/HEAD: [B, N] f32; RESID: residual [B, N] updated in place
  void* act_out;        // SWIGLU: [B, N] in the activation format
  float* part;          // split partials [S][B][Nraw]
  unsigned* cnt;        // per (row block, column group) arrival counters, zero between launches
  float2* amax;         // HEAD: per (row block, lane) (max value, index as float bits)
};

struct AttnArgs {
  const float* qkv;       // [B, Nqkv] f32, before rotation
  void* kslab;            // arena K region
  void* vslab;            // arena V region
  long long lane_stride;  // elements per lane per region: L * Hkv * max_seq * hd
  long long layer_off;    // l * Hkv * max_seq * hd
  int max_seq;
  int B;
  const int* lanes;       // [B] arena lane ids
  const int* pos;         // [B] positions (slot written this step)
  const int* items;       // [n_items][2] (b, split)
  int n_items;
  int max_splits;         // splits per lane the partial buffer is sized for
  int Hq, Hkv, G, Nqkv;
  const float2* rope;     // [B][hd/2] (cos, sin) of each lane's position
  float* part;            // [B][max_splits][Hkv][G][hd + 2]
  unsigned* cnt;          // [B][Hkv] arrival counters, zero between launches
  void* out;              // [B, Hq*hd] in the activation format
};

// ---- launchers (return hipError_t of the launch) -------------------------------
hipError_t launch_gemm(int wt, int epi, int C, const GemmArgs& a, int n_waves, hipStream_t st);
hipError_t launch_attn(int hd, int kv_bf16, int act, const AttnArgs& a, hipStream_t st);
// x[b] = E[token_b]; xn[b] = rmsnorm(x[b]) * g (act format); rope table of pos_b.
hipError_t launch_embed_norm(int wt, const void* E, const uint16_t* Es, const int* tokens, const int* pos, int B,
                             int d, int hd, float theta, float eps, const float* g, float* x, void* xn,
                             float2* rope, hipStream_t st);
hipError_t launch_rmsnorm(int wt, const float* x, const float* g, int B, int d, float eps, void* xn,
                          hipStream_t st);
hipError_t launch_argmax(const float2* amax, int nRB, int B, int* argmax, hipStream_t st);
hipError_t launch_fill_u32(unsigned* p, size_t n, unsigned v, hipStream_t st);

}  // namespace cbd
