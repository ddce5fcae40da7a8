// Internal interface between the host runtime (cbd_runtime.hip) and the
// gfx950 kernels (cbd_gemm.hip, cbd_attn.hip, cbd_misc.hip).  Not installed.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct cbd_arena;  // include/cbd.h
struct cbd_model;

namespace cbd {

enum WType { WT_F32 = 0, WT_BF16 = 1, WT_Q8 = 2 };
enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_HEAD = 3 };

// Keys per attention split.  A constant of the design: the per-lane result
// never depends on B, on the lane's slot or on the other lanes.
constexpr int ATTN_SPLIT = 64;
// Chunks per attention work item of the matrix-core kernel: aligned groups of
// a lane's chunks, merged in chunk order inside the wave into one partial.  A
// constant of the design, like ATTN_SPLIT.
constexpr int ATTN_GROUP = 4;
// ints per attention work item: lane index | chunk count << 24, first chunk,
// position, padding, then the arena block of each of up to ATTN_GROUP chunks.
constexpr int ITEM_INTS = 8;
// Attention modes: fused (a decode step: each lane's new K/V is written and
// used by the same launch) and attend only (several rows of a lane in one
// call: launch_kv_append writes every row's K/V first, then every key is read
// from the cache, so rows never read a slot another workgroup is writing).
constexpr int ATTN_FUSED = 0, ATTN_ATTEND = 2;
// Rows of one lane per work item of the batched-prefill attention kernel.
constexpr int ATTN_ROWS_MAX = 16;
// Rows of one MFMA tile; 16-row tiles per wave in the projection kernels, by
// epilogue (SwiGLU pairs a gate tile with an up tile; the LM head has the most
// rows; the others take one tile so that d-row projections fill the chip).
constexpr int TILE = 16;
__host__ __device__ constexpr int gemm_rows(int epi) { return (epi == 2 || epi == 3) ? 2 : 1; }
// Splits of K per projection tile: one wave each, in one workgroup.
constexpr int GEMM_MAX_SPLIT = 8;

// Projection over a panel: Y[b][n] = sum_k W[n][k] * X[b][k] for b < B.
// The reduction contract (identical in every kernel variant and batch width):
// K is cut into S splits of Ks elements (the last may be shorter); each
// split's partial is a chain of MFMAs over ascending k-steps starting from
// zero; the output is ((P_0 + P_1) + P_2) + ... in split order, then the
// epilogue.  So lane b's outputs are the same bits whatever B is.
//
// RMSNorm statistics come from the producer: a projection that updates the
// residual stream x (EPI_RESID) also writes, per row block, the partial sums
// of x^2 of each lane, which the norm kernel adds in row-block order.
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
  int nRB;              // row blocks of TILE*rows rows (SWIGLU: TILE*rows/2 pairs)
  int nCG;              // column groups
  float* out;           // STORE/HEAD: [B, N] f32; RESID: residual [B, N] updated in place
  void* act_out;        // SWIGLU: [B, N] in the activation format
  float2* amax;         // HEAD: per (row block, lane) (max value, index as float bits)
  int red_waves;        // split partials per LDS round (set by the launcher)
  float* ssq_out;       // EPI_RESID: [nRB][B] this tile's sum of x^2 per lane
  float* part;          // panel split mode: [S][B][nRB][rows per row block] split partials
  int fold_elsewhere;   // EPI_STORE split mode: leave the partials unfolded (the consumer adds them)
  // bf16 weights in the packed tile layout (cbd_pack_matrix): W holds
  // tiles of 16 rows x 32 k, 1 KB each, row tile i of half h from tile
  // (h * wtiles + i) * (K / 32 + PACK_GAP); wtiles = row tiles per half
  // (SWIGLU: the gate half, then the up half).  0: row-major.
  int wpack;
  int wtiles;
  // EPI_RESID in panel split mode only: if norm_out is set, the fold also runs
  // the next RMSNorm, xn = (x * r) * g into norm_out (activation format), and
  // writes no sums of squares.
  const float* norm_g;
  float norm_eps;
  void* norm_out;
  // Split-K tiles only (launch_gemm, one column group of at most 16 lanes):
  // if in_x is set, X is not read; each wave computes its split of the
  // RMSNorm output itself, (x * r) * in_g rounded to the activation format,
  // r = 1 / sqrt(sum of the in_ssq_n per-row-block sums of x^2 / K + in_eps)
  // with the norm kernel's additions, and stages it in LDS (the norm kernel's
  // bits, without its launch).  in_ssq_n at most NORM_IN_MAX_SSQ.
  const float* in_x;
  const float* in_ssq;
  int in_ssq_n;
  const float* in_g;
  float in_eps;
};
// Producer row blocks (sums of x^2 per lane) a split-K tile that normalises its
// own activations can add: one per lane of a wave.
constexpr int NORM_IN_MAX_SSQ = 64;
// Largest LDS staging of normalised activations per split-K workgroup.
constexpr size_t NORM_IN_MAX_LDS = 32 * 1024;
// Most lanes a split-K tile normalises for itself: a wave stages its lanes one
// after another (a memory round trip each), so beyond two lanes the norm's own
// launch costs less (SmolLM2-135M Q8_0 at 12 lanes: 1.37 ms per step with
// normalising tiles, 0.97 at 16 with the norm launched).
constexpr int NORM_IN_MAX_B = 2;
// Whether launch_gemm can normalise its own activations for a projection of K
// inputs, S splits of Ks, over B lanes whose activation format has xb bytes.
__host__ __device__ constexpr bool gemm_norm_in_supported(int B, int K, int S, int Ks, int xb, int ssq_n) {
  return B >= 1 && B <= NORM_IN_MAX_B && ssq_n >= 1 && ssq_n <= NORM_IN_MAX_SSQ && K % 4 == 0 &&
         (size_t)S * B * ((size_t)Ks * xb + 16) <= NORM_IN_MAX_LDS;
}

struct AttnArgs {
  const float* qkv;       // [B, Nqkv] f32, before rotation
  void* kpool;            // arena K block pool
  void* vpool;            // arena V block pool
  // A block holds ATTN_SPLIT positions of one lane for every layer and KV
  // head; the pools are layer-major, [L][n_blocks][Hkv][ATTN_SPLIT][hd]:
  // chunk c of a lane is the block the work item names for it, and (layer l,
  // head g) of block j sits at j * block_elems + layer_off + g * ATTN_SPLIT * hd.
  long long block_elems;  // Hkv * ATTN_SPLIT * hd
  long long layer_off;    // l * n_blocks * block_elems
  int B;
  int mode;               // ATTN_FUSED or ATTN_ATTEND
  const int* lanes;       // [B] arena lane ids
  const int* pos;         // [B] positions (slot written this step)
  const int* items;       // [n_items][ITEM_INTS] {b | chunks << 24, first chunk, position, 0, block of each chunk (up to 4)}, 16-byte aligned
  const int* n_items_dev; // number of items of this step (device)
  int max_items;          // grid size: the most items a step of B lanes can have
  int max_splits;         // partials per lane the partial buffer is sized for
  int per;                // chunks per partial: ATTN_GROUP (matrix-core kernel) or 1
  int Hq, Hkv, G, Nqkv;
  const float2* rope;     // [B][hd/2] (cos, sin) of each lane's position
  // Matrix-core kernel only: if qkv_S > 0 the QKV projection left its split
  // partials [qkv_S][B][Nqkv] unfolded in qkv_part, and attention adds them
  // (in split order) instead of reading qkv.
  const float* qkv_part;
  int qkv_S;
  float* part;            // [B][max_splits][Hkv][G][hd + 2] partials (o, m, l) per chunk or group
  void* out;              // [B, Hq*hd] in the activation format
  // A row whose keys fit one work item (one partial) gets out = o / l from the
  // attention kernel itself, in the activation format act, and the combine
  // skips it (the combine of a single partial gives exactly o / l).
  int act;                // WT_* of the activation format
  // Batched prefill (attend mode): rowmap lists the rows of each lane in
  // position order (work items of launch_attn_rows name a run of it);
  // rowblk[b] is the block holding slot pos[b] of row b's lane (launch_kv_append).
  const int* rowmap;
  const int* rowblk;
  int frag;               // chunks in fragment order (kfrag_off / vfrag_off)
};

// Block sum of per-thread partials (256 threads): a fixed shuffle tree, then
// the four waves in order.  The one reduction every RMSNorm statistic goes
// through, whichever kernel computes it.
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

// ---- launchers (return hipError_t of the launch) -------------------------------
hipError_t launch_gemm(int wt, int epi, int C, const GemmArgs& a, hipStream_t st);
// Wide-panel projection (activation panel staged in LDS, 16*C lanes per
// workgroup, C in {2, 4, 8}; rm row blocks per wave, 1, or 2 in split mode
// with C >= 4); split = 1 writes split partials to a.part and adds them in
// order in a second kernel.
// Same output bits as launch_gemm.
hipError_t launch_panel(int wt, int epi, int C, int rm, int split, const GemmArgs& a, hipStream_t st);
// Whether a split-mode EPI_RESID panel can fold and normalise in one kernel
// (a.norm_out set): N up to 8192, a multiple of 16.
__host__ __device__ constexpr bool fold_norm_supported(int N) { return N % 16 == 0 && N <= 8192; }
// workgroups of one panel launch (for sizing decisions)
int panel_workgroups(const GemmArgs& a, int C, int rm, int split);
// Dense-tile projection for bf16 weights (both operands staged in LDS, 256
// weight rows x 128 lanes per eight-wave workgroup); K a multiple of 128,
// split lengths a multiple of 256.  split = 1: one split per workgroup, partials folded in order by a
// second kernel (as launch_panel).  Same output bits as launch_gemm.
hipError_t launch_dense(int epi, int split, const GemmArgs& a, hipStream_t st);
int dense_workgroups(const GemmArgs& a, int epi, int split);
// Whether the dense tiles can run a projection of (K, Ks, S) without split
// partials: one split, or a split length built into a whole-K kernel.
int dense_mode_available(int epi, int K, int Ks, int S);
// Whether the MFMA attention kernel serves this shape (bf16 KV; head_dim 64
// with up to 8, or 128 with up to 4 query heads per KV head, the shapes that
// fit two waves per SIMD); otherwise items carry one chunk.
__host__ __device__ constexpr bool attn_mfma_supported(int hd, bool kv_bf16, int G) {
  return kv_bf16 && G >= 1 && ((hd == 64 && G <= 8) || (hd == 128 && G <= 4));
}
// chunk partials of every (lane, KV head, 64-key chunk) item; RoPE and KV append
hipError_t launch_attn(int hd, int kv_bf16, const AttnArgs& a, hipStream_t st);
// Chunk layout of bf16 caches on the matrix-core shapes: within one (layer,
// KV head) chunk of ATTN_SPLIT keys x hd dims, elements sit in the order the
// attention kernels load their MFMA operand fragments, 16 bytes per lane and
// 1 KB per wave-wide load:
//  K: fragment (t, kk) = keys 16t..16t+15 x dims 32kk..32kk+31 (the score
//     MFMA's A operand), lane 16*g4 + l16 holding key 16t + l16, dims
//     32kk + 8*g4 .. + 7;
//  V: fragment (dt, u) = keys 32u..32u+31 x dims 16dt..16dt+15 (the P.V
//     MFMA's B operand), lane 16*kg + n holding dim 16dt + n of keys
//     32u + 16*(e >> 2) + 4*kg + (e & 3), e = 0..7.
// Other shapes keep row-major chunks (key * hd + dim).
__host__ __device__ inline int kfrag_off(int key, int d, int hd) {
  const int t = key >> 4, l16 = key & 15, kk = d >> 5, g4 = (d >> 3) & 3, e = d & 7;
  return ((t * (hd / 32) + kk) * 64 + 16 * g4 + l16) * 8 + e;
}
__host__ __device__ inline int vfrag_off(int key, int d, int hd) {
  const int dt = d >> 4, n = d & 15, u = key >> 5, h = (key >> 4) & 1, kg = (key >> 2) & 3, i = key & 3;
  (void)hd;
  return ((dt * 2 + u) * 64 + 16 * kg + n) * 8 + 4 * h + i;
}
// (key, dim) of element o of a fragment-ordered chunk (the inverses)
__host__ __device__ inline void kfrag_at(int o, int hd, int* key, int* d) {
  const int e = o & 7, lane = (o >> 3) & 63, tk = o >> 9, kk = tk % (hd / 32), t = tk / (hd / 32);
  *key = 16 * t + (lane & 15);
  *d = 32 * kk + 8 * (lane >> 4) + e;
}
__host__ __device__ inline void vfrag_at(int o, int hd, int* key, int* d) {
  (void)hd;
  const int e = o & 7, lane = (o >> 3) & 63, du = o >> 9, u = du & 1, dt = du >> 1;
  *key = 32 * u + 16 * (e >> 2) + 4 * (lane >> 4) + (e & 3);
  *d = 16 * dt + (lane & 15);
}

// Batched-prefill attention (shapes attn_mfma_supported serves): a.max_items
// work items {first rowmap index | rows << 24, first chunk of the group,
// position of the first row, chunks of the group the last row reaches, block
// of each of the group's chunks}, each up to ATTN_ROWS_MAX rows of one lane at
// consecutive positions, all of which reach the group.
hipError_t launch_attn_rows(int hd, const AttnArgs& a, hipStream_t st);
// Every row's new K (rotated) and V into its slot (a.pos, a.rowblk), all heads.
hipError_t launch_kv_append(int hd, int kv_bf16, const AttnArgs& a, hipStream_t st);
// combine a lane's chunks into the attention output (activation format act)
hipError_t launch_attn_combine(int hd, int act, const AttnArgs& a, hipStream_t st);
// x[b] = E[token_b]; ssq[b] = sum x[b]^2; rope table of pos_b.
hipError_t launch_embed(int wt, const void* E, const uint16_t* Es, const int* tokens, const int* pos, int B, int d,
                        int hd, float theta, float* x, float* ssq, float2* rope, hipStream_t st);
// xn[b] = (x[b] * r_b) * g in the activation format, r_b = 1 / sqrt(sum_t ssq[t][b] / d + eps).
hipError_t launch_norm(int wt, const float* x, const float* ssq, int ssq_n, const float* g, int B, int d, float eps,
                       void* xn, hipStream_t st);
hipError_t launch_argmax(const float2* amax, int nRB, int B, int* argmax, hipStream_t st);
// Copy `bytes` (a multiple of 4) from device-visible pinned host memory
// (src_dev: its device address) to device memory, by a kernel.
hipError_t launch_meta_copy(void* dst, const void* src_dev, size_t bytes, hipStream_t st);
hipError_t launch_fill_u32(unsigned* p, size_t n, unsigned v, hipStream_t st);
// Copy blocks src[j] -> dst[j] (j < n) of a layer-major pool in every layer,
// K (at base) and V (at base + half); the block lists are on the device.
hipError_t launch_kv_blocks(char* base, long long half, const int* src, const int* dst, int n, int L,
                            long long lstride, long long bbytes, hipStream_t st);
// Record a formatted message as the calling thread's last error; returns code.
int report_error(int code, const char* fmt, ...);
// KV bytes of one position of one lane in an arena (K and V, every layer and head).
size_t arena_kv_bytes_per_token(const cbd_arena* a);
// Positions a lane of the arena can hold.
int arena_max_seq(const cbd_arena* a);
// Rows (lanes of a decode step, or prompt tokens of a prefill call) a workspace
// of `bytes` holds for arenas of max_seq positions per lane.
int workspace_rows(const cbd_model* m, int max_seq, size_t bytes);
// Copy one lane's K or V rows [L * Hkv][len][hd] (device, contiguous) into its
// blocks of a layer-major pool (to_pool), or back; blocks: the lane's block ids
// on the device, one per 64 positions.
// The packed tile layout of a bf16 matrix (cbd_pack_matrix): its size (0 if
// none) and the packing kernel.  Each row tile's run of K / 32 tiles is
// followed by PACK_GAP unused tiles, so that the runs the waves stream at
// once do not start 2^n kilobytes apart (two adjacent row tiles per wave, as
// the LM head reads them, streamed at 5.0 TB/s with runs 128 KB apart and
// at 5.85 TB/s with 136 KB).
constexpr int PACK_GAP = 8;
size_t packed_bytes_bf16(int rows, int K, int halves);
hipError_t launch_pack_bf16(const void* src, void* dst, int rows, int K, int halves, hipStream_t st);
hipError_t launch_kv_rows(char* pool, char* rows, const int* blocks, int p0, int len, int n_rows, int Hkv,
                          int row_bytes, long long lstride, long long bbytes, bool to_pool, hipStream_t st);
// The same for fragment-ordered bf16 chunks (frag: 1 = K order, 2 = V order),
// one workgroup per (row, chunk) through an LDS tile; chunks only partly in
// [p0, p0 + len) keep their other keys.
hipError_t launch_kv_rows_frag(char* pool, char* rows, const int* blocks, int p0, int len, int n_rows, int Hkv,
                               int hd, long long lstride, long long bbytes, bool to_pool, int frag, hipStream_t st);
// Rotate n_vec key vectors of hd elements (bf16 or f32, device) in place by the
// per-pair (cos, sin) table cs[hd/2] (rotate-half pairs; products and sums
// rounded to f32 one by one), rounding to the KV format.
hipError_t launch_kv_rot(char* rows, long long n_vec, int hd, const float2* cs, bool bf16, hipStream_t st);

}  // namespace cbd
