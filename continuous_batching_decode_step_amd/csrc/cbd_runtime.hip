// Host runtime of the C-ABI in include/cbd.h: model and arena objects,
// host-side validation (all of it before any GPU work, so a failed call
// changes nothing), the workspace layout and the per-step launch sequence.
//
// Step = embed + first RMSNorm, then per layer: QKV projection, attention
// (rotary, in-place KV append, ragged split-K), O projection + residual,
// RMSNorm, gate|up projection + SwiGLU, down projection + residual, RMSNorm;
// then the LM head with per-lane greedy argmax.  Every projection runs once
// over the [B, d] panel of the step ("MODEL-BATCHING-RESULTS — multi-user
// batched decode, measured", section "The lever").
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <string>
#include <vector>

#include "../../include/cbd.h"
#include "cbd_internal.h"

using namespace cbd;

namespace {

thread_local std::string g_err;

// Device and pinned-host allocations the library has made (a test hook: a
// decode step must make none).
std::atomic<long long> g_allocs{0};

hipError_t counted_malloc(void** p, size_t bytes) {
  g_allocs.fetch_add(1);
  return hipMalloc(p, bytes);
}

hipError_t counted_host_malloc(void** p, size_t bytes) {
  g_allocs.fetch_add(1);
  return hipHostMalloc(p, bytes, hipHostMallocDefault);
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) return fail(CBD_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr int TARGET_WAVES = 4096;  // split-K is chosen so a B=1 step has this many waves
constexpr int MIN_KS = 256;         // but no split shorter than this many elements
// Split lengths are whole multiples of this many elements, so that every split
// of a wide-panel walk covers an even number of LDS chunks (a chunk is at most
// 128 elements) and the running total is folded between chunk pairs only.
constexpr int KS_ALIGN = 256;
constexpr int NSLOT = 4;  // pinned staging slots for per-step metadata

struct Plan {
  int N, Nraw, K, S, Ks, nRB;
};

Plan make_plan(int N, int Nraw, int K, int kstep, int rows_per_rb) {
  Plan p;
  p.N = N;
  p.Nraw = Nraw;
  p.K = K;
  p.nRB = (N + rows_per_rb - 1) / rows_per_rb;
  int S = (TARGET_WAVES + p.nRB - 1) / p.nRB;
  S = std::max(1, std::min(std::min(S, K / MIN_KS), GEMM_MAX_SPLIT));
  int Ks = (K + S - 1) / S;
  Ks = (Ks + KS_ALIGN - 1) / KS_ALIGN * KS_ALIGN;
  (void)kstep;  // KS_ALIGN is a multiple of every k-step
  p.Ks = Ks;
  p.S = (K + Ks - 1) / Ks;
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

struct cbd_model {
  cbd_config c;
  int wt;
  int q_dim, kv_dim, n_qkv, G, actb, kvb, pl, kstep;
  cbd_matrix embed, head;
  const float* final_norm;
  std::vector<const float*> attn_norm, ffn_norm;
  std::vector<cbd_matrix> qkv, o, gu, down;
  Plan p_qkv, p_o, p_gu, p_down, p_head;
  int variant = 0;
  // captured step graphs, keyed by everything their kernel arguments depend on
  // (the arena object and its pool geometry: the pool base, the V region's
  // offset and the layer stride are baked into the attention arguments); an
  // arena's graphs are dropped when it is destroyed
  struct GraphKey {
    int B;
    const void *ws, *arena, *base, *logits, *argmax;
    size_t ws_bytes, region_bytes;
    int max_seq, n_lanes, n_blocks, variant;
    bool direct;  // attention finishes the rows itself (no combine launch)
    bool operator==(const GraphKey& o) const {
      return B == o.B && ws == o.ws && arena == o.arena && base == o.base && logits == o.logits &&
             argmax == o.argmax && ws_bytes == o.ws_bytes && region_bytes == o.region_bytes &&
             max_seq == o.max_seq && n_lanes == o.n_lanes && n_blocks == o.n_blocks && variant == o.variant &&
             direct == o.direct;
    }
  };
  std::vector<std::pair<GraphKey, hipGraphExec_t>> graphs;
  hipStream_t cap_stream = nullptr;
  bool use_graphs = false;
  // pinned staging for per-step metadata, sized when an arena is created for
  // a decode step over all of its lanes (a decode step never allocates; a
  // prefill call with more rows may grow them)
  void* slot[NSLOT] = {};
  void* slot_dev[NSLOT] = {};  // each slot's device address
  size_t slot_bytes[NSLOT] = {};
  hipEvent_t ev[NSLOT] = {};
  bool ev_live[NSLOT] = {};
  int next_slot = 0;
  // rows of a multi-row call sorted by (lane, position), reused across calls
  std::vector<int32_t> row_order;
  // per-kernel-class timing
  bool prof = false;
  std::vector<hipEvent_t> ev_pool;
  std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> pending;
  double prof_ms[16] = {};
  long long prof_n[16] = {};
};

// A pool of KV blocks over caller-owned memory: a block holds ATTN_SPLIT
// positions (one attention chunk) of one lane for every layer and KV head.
// The pool is layer-major, K [L][n_blocks][Hkv][ATTN_SPLIT][hd] then V alike:
// one layer's blocks are contiguous, which loads 13% faster in attention than
// a pool of whole blocks [n_blocks][L][...] (5.95 vs 5.26 TB/s for the same
// chunks, whatever the blocks' placement).  A lane
// holds the blocks of its chunks in order (any blocks of the pool); a step
// takes a free block when a lane's new slot opens a chunk, and clear, evict
// and truncate return blocks to the pool.
struct cbd_arena {
  cbd_model* m;
  int n_lanes, max_seq;
  char* base;
  size_t bytes;
  int n_blocks;
  long long block_elems;  // elements of one block of one layer: Hkv * ATTN_SPLIT * hd
  size_t region_bytes;    // bytes of the K pool (the V pool follows)
  std::vector<uint8_t> live;
  std::vector<int> len;
  std::vector<std::vector<int>> blocks;  // per lane, the block of each chunk
  std::vector<int> free_blocks;          // a stack; the lowest block on top
  // duplicate-lane check of a step without a per-step allocation: lane i is
  // taken in this step if mark[i] == epoch
  std::vector<uint32_t> mark;
  uint32_t epoch = 0;
  // device staging for kv import/export: one lane's K or V rows, then its block
  // ids; allocated on first use, grown as needed, freed with the arena
  char* stage = nullptr;
  size_t stage_bytes = 0;
};

namespace {

struct WsLayout {
  size_t meta, meta_bytes, x, xn, ssq, qkv, o, a, amax, rope, apart, gpart, gpart_bytes, total;
  int maxB, MS, parts;  // parts: attention partials per lane (chunks, or groups of chunks)
};

// 64-key chunks per attention work item (and per partial): 1 for the one-chunk
// kernel; aligned groups of ATTN_GROUP for the matrix-core kernel, which
// merges a group inside the wave.  Never a function of B.
int attn_chunks_per_item(const cbd_model* m) {
  return attn_mfma_supported(m->c.head_dim, m->wt == WT_BF16, m->G) ? ATTN_GROUP : 1;
}

// Whether the model's bf16 chunks are stored in the matrix-core kernels'
// fragment order (kfrag_off / vfrag_off): exactly the shapes they serve.
static bool kv_frag(const cbd_model* m) { return attn_chunks_per_item(m) == ATTN_GROUP; }

// Attention partials per lane for MS chunks: one per work item.
int attn_partials(const cbd_model* m, int MS) {
  const int per = attn_chunks_per_item(m);
  return (MS + per - 1) / per;
}

// Per-step metadata: lanes[B], positions[B], tokens[B], rowmap[B], rowblk[B]
// (multi-row calls: the rows in (lane, position) order, and the block holding
// each row's slot), n_items, padding to a multiple of 4 ints, then the
// attention work items (ITEM_INTS ints each), 16-byte aligned (B is at most
// 65536).
size_t meta_header(int B) { return ((size_t)5 * B + 1 + 3) & ~(size_t)3; }

// Bytes of the per-step metadata of B rows holding `chunks` 64-key chunks in all.
size_t meta_bytes_for(int B, long long items) { return 4 * (meta_header(B) + (size_t)ITEM_INTS * items); }

// Grow every pinned staging slot to at least `bytes` (each slot's last copy is
// waited for before it is freed).
int grow_slots(cbd_model* m, size_t bytes) {
  for (int i = 0; i < NSLOT; ++i) {
    if (m->slot_bytes[i] >= bytes) continue;
    if (m->ev_live[i]) HIP_TRY(hipEventSynchronize(m->ev[i]));
    if (m->slot[i]) HIP_TRY(hipHostFree(m->slot[i]));
    m->slot[i] = nullptr;
    m->slot_dev[i] = nullptr;
    m->slot_bytes[i] = 0;
    const size_t cap = std::max(bytes, (size_t)65536);
    HIP_TRY(counted_host_malloc(&m->slot[i], cap));
    HIP_TRY(hipHostGetDevicePointer(&m->slot_dev[i], m->slot[i], 0));
    m->slot_bytes[i] = cap;
    if (!m->ev[i]) HIP_TRY(hipEventCreateWithFlags(&m->ev[i], hipEventDisableTiming));
  }
  return CBD_OK;
}

WsLayout layout(const cbd_model* m, int maxB, int max_seq) {
  WsLayout L{};
  const cbd_config& c = m->c;
  L.maxB = maxB;
  L.MS = (max_seq + ATTN_SPLIT - 1) / ATTN_SPLIT;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.meta_bytes = 4 * (meta_header(maxB) + (size_t)ITEM_INTS * maxB * L.MS);
  L.meta = take(L.meta_bytes);
  L.x = take(4 * (size_t)maxB * c.d_model);
  L.xn = take((size_t)m->actb * maxB * c.d_model);
  const int ssq_rows = std::max(std::max(m->p_o.nRB, m->p_down.nRB), 1);
  L.ssq = take(4 * (size_t)ssq_rows * maxB);
  L.qkv = take(4 * (size_t)maxB * m->n_qkv);
  L.o = take((size_t)m->actb * maxB * m->q_dim);
  L.a = take((size_t)m->actb * maxB * c.ffn_dim);
  L.amax = take(8 * (size_t)m->p_head.nRB * maxB);
  L.rope = take(8 * (size_t)maxB * (c.head_dim / 2));
  L.parts = attn_partials(m, L.MS);
  L.apart = take(4 * (size_t)maxB * L.parts * c.n_kv_heads * m->G * (c.head_dim + 2));
  // split partials of the wide-panel projections that can run in split mode
  // (panel_shape: a two-tile projection splits only up to 64 lanes, and only
  // with fewer than 512 row blocks; a one-tile one may split at any width)
  size_t gp = 0;
  const Plan* plans[] = {&m->p_qkv, &m->p_o, &m->p_gu, &m->p_down, &m->p_head};
  const int epis[] = {EPI_STORE, EPI_RESID, EPI_SWIGLU, EPI_RESID, EPI_HEAD};
  for (int i = 0; i < 5; ++i) {
    const Plan& pl = *plans[i];
    if (pl.S < 2) continue;
    const bool one_tile = gemm_rows(epis[i]) == 1;
    if (!one_tile && pl.nRB >= 512) continue;
    const size_t lanes = one_tile ? (size_t)maxB : (size_t)std::min(maxB, 64);
    gp = std::max(gp, (size_t)pl.S * pl.nRB * TILE * gemm_rows(epis[i]) * lanes);
  }
  L.gpart_bytes = 4 * gp;
  L.gpart = take(L.gpart_bytes);
  L.total = off;
  return L;
}

int max_batch_for(const cbd_model* m, int max_seq, size_t bytes) {
  if (layout(m, 1, max_seq).total > bytes) return 0;
  int lo = 1, hi = 1 << 16;
  while (lo < hi) {
    int mid = lo + (hi - lo + 1) / 2;
    if (layout(m, mid, max_seq).total <= bytes)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_matrix(const cbd_matrix& mt, int wt, const char* name) {
  if (!mt.data) return fail(CBD_E_ARG, "weight %s: null data pointer", name);
  if (!aligned16(mt.data)) return fail(CBD_E_ARG, "weight %s: data not 16-byte aligned", name);
  if (wt == WT_Q8 && !mt.scale) return fail(CBD_E_ARG, "weight %s: Q8_0 needs a scale plane", name);
  return CBD_OK;
}

const char* const kClassNames[] = {"meta_copy", "embed",     "gemm_qkv",  "attention", "attn_combine", "gemm_o",
                                   "rmsnorm",   "gemm_gu",   "gemm_down", "gemm_head", "argmax"};
enum { P_META, P_EMBED, P_QKV, P_ATTN, P_COMB, P_O, P_NORM, P_GU, P_DOWN, P_HEAD, P_ARGMAX, P_N };

hipEvent_t take_event(cbd_model* m) {
  if (!m->ev_pool.empty()) {
    hipEvent_t e = m->ev_pool.back();
    m->ev_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Fold finished event pairs into the per-class totals (all of them if `all`).
int drain_profile(cbd_model* m, bool all) {
  size_t keep_from = 0;
  const size_t n = m->pending.size();
  const size_t upto = all ? n : (n > 2048 ? n - 1024 : 0);
  for (size_t i = 0; i < upto; ++i) {
    auto& pr = m->pending[i];
    HIP_TRY(hipEventSynchronize(pr.second.second));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, pr.second.first, pr.second.second));
    m->prof_ms[pr.first] += ms;
    m->prof_n[pr.first] += 1;
    m->ev_pool.push_back(pr.second.first);
    m->ev_pool.push_back(pr.second.second);
    keep_from = i + 1;
  }
  m->pending.erase(m->pending.begin(), m->pending.begin() + keep_from);
  return CBD_OK;
}

// Brackets one launch with events when profiling is on.
struct ProfScope {
  cbd_model* m;
  int cls;
  hipStream_t st;
  hipEvent_t a = nullptr;
  ProfScope(cbd_model* m_, int cls_, hipStream_t st_) : m(m_), cls(cls_), st(st_) {
    if (m->prof && (a = take_event(m))) (void)hipEventRecord(a, st);
  }
  ~ProfScope() {
    if (!a) return;
    hipEvent_t b = take_event(m);
    if (!b) return;
    (void)hipEventRecord(b, st);
    m->pending.push_back({cls, {a, b}});
  }
};

}  // namespace

extern "C" {

const char* cbd_version(void) { return "cbd 0.1 gfx950"; }

const char* cbd_last_error(void) { return g_err.c_str(); }

int cbd_model_create(const cbd_config* cfg, const cbd_weights* w, cbd_model** out) {
  if (!cfg || !w || !out) return fail(CBD_E_ARG, "null argument");
  const cbd_config& c = *cfg;
  if (c.d_model <= 0 || c.n_layers <= 0 || c.n_heads <= 0 || c.n_kv_heads <= 0 || c.ffn_dim <= 0 || c.vocab <= 0)
    return fail(CBD_E_ARG, "non-positive model dimension");
  if (c.wtype < CBD_F32 || c.wtype > CBD_Q8_0) return fail(CBD_E_ARG, "unknown wtype %d", c.wtype);
  if (!(c.rms_eps >= 0.f) || !(c.rope_theta > 0.f)) return fail(CBD_E_ARG, "bad rms_eps or rope_theta");
  if (c.n_heads % c.n_kv_heads != 0 || c.n_heads / c.n_kv_heads > 8)
    return fail(CBD_E_UNSUPPORTED, "n_heads / n_kv_heads must be an integer <= 8");
  if (c.head_dim != 16 && c.head_dim != 32 && c.head_dim != 64 && c.head_dim != 128)
    return fail(CBD_E_UNSUPPORTED, "head_dim %d not in {16, 32, 64, 128}", c.head_dim);
  const int pl = c.wtype == CBD_F32 ? 4 : (c.wtype == CBD_BF16 ? 8 : 32);
  const int qd = c.n_heads * c.head_dim;
  if (c.d_model % pl || c.ffn_dim % pl || qd % pl)
    return fail(CBD_E_UNSUPPORTED, "d_model, ffn_dim and n_heads*head_dim must be multiples of %d", pl);
  if (c.packed && (c.wtype != CBD_BF16 || c.d_model % 32 || c.ffn_dim % 32 || qd % 32))
    return fail(CBD_E_UNSUPPORTED, "packed weights need bf16 and d_model, ffn_dim, n_heads*head_dim multiples of 32");
  if (!w->final_norm || !w->attn_norm || !w->ffn_norm || !w->w_qkv || !w->w_o || !w->w_gu || !w->w_down)
    return fail(CBD_E_ARG, "null weight pointer array");
  int rc;
  if ((rc = check_matrix(w->embed, c.wtype, "embed"))) return rc;
  if (!c.tied_embeddings && (rc = check_matrix(w->lm_head, c.wtype, "lm_head"))) return rc;
  // the norm kernels load the gains 16 bytes at a time
  auto misaligned = [](const float* g) { return ((uintptr_t)g & 15) != 0; };
  if (misaligned(w->final_norm)) return fail(CBD_E_ARG, "final_norm: gains must be 16-byte aligned");
  for (int l = 0; l < c.n_layers; ++l) {
    if (!w->attn_norm[l] || !w->ffn_norm[l]) return fail(CBD_E_ARG, "layer %d: null norm gain", l);
    if (misaligned(w->attn_norm[l]) || misaligned(w->ffn_norm[l]))
      return fail(CBD_E_ARG, "layer %d: norm gains must be 16-byte aligned", l);
    if ((rc = check_matrix(w->w_qkv[l], c.wtype, "w_qkv"))) return rc;
    if ((rc = check_matrix(w->w_o[l], c.wtype, "w_o"))) return rc;
    if ((rc = check_matrix(w->w_gu[l], c.wtype, "w_gu"))) return rc;
    if ((rc = check_matrix(w->w_down[l], c.wtype, "w_down"))) return rc;
  }
  cbd_model* m = new cbd_model();
  m->c = c;
  m->wt = c.wtype;
  m->q_dim = qd;
  m->kv_dim = c.n_kv_heads * c.head_dim;
  m->n_qkv = qd + 2 * m->kv_dim;
  m->G = c.n_heads / c.n_kv_heads;
  m->actb = c.wtype == CBD_F32 ? 4 : 2;
  m->kvb = c.wtype == CBD_BF16 ? 2 : 4;
  m->pl = pl == 32 ? 8 : pl;
  m->kstep = c.wtype == CBD_F32 ? 16 : 32;
  m->embed = w->embed;
  m->head = c.tied_embeddings ? w->embed : w->lm_head;
  m->final_norm = w->final_norm;
  for (int l = 0; l < c.n_layers; ++l) {
    m->attn_norm.push_back(w->attn_norm[l]);
    m->ffn_norm.push_back(w->ffn_norm[l]);
    m->qkv.push_back(w->w_qkv[l]);
    m->o.push_back(w->w_o[l]);
    m->gu.push_back(w->w_gu[l]);
    m->down.push_back(w->w_down[l]);
  }
  m->p_qkv = make_plan(m->n_qkv, m->n_qkv, c.d_model, m->kstep, TILE * gemm_rows(EPI_STORE));
  m->p_o = make_plan(c.d_model, c.d_model, qd, m->kstep, TILE * gemm_rows(EPI_RESID));
  m->p_gu = make_plan(c.ffn_dim, 2 * c.ffn_dim, c.d_model, m->kstep, TILE * gemm_rows(EPI_SWIGLU) / 2);
  m->p_down = make_plan(c.d_model, c.d_model, c.ffn_dim, m->kstep, TILE * gemm_rows(EPI_RESID));
  m->p_head = make_plan(c.vocab, c.vocab, c.d_model, m->kstep, TILE * gemm_rows(EPI_HEAD));
  *out = m;
  return CBD_OK;
}

void cbd_model_destroy(cbd_model* m) {
  if (!m) return;
  (void)drain_profile(m, true);
  for (hipEvent_t e : m->ev_pool) (void)hipEventDestroy(e);
  for (auto& g : m->graphs) (void)hipGraphExecDestroy(g.second);
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  for (int i = 0; i < NSLOT; ++i) {
    if (m->ev[i]) {
      (void)hipEventSynchronize(m->ev[i]);
      (void)hipEventDestroy(m->ev[i]);
    }
    if (m->slot[i]) (void)hipHostFree(m->slot[i]);
  }
  delete m;
}

size_t cbd_packed_bytes(int wtype, int rows, int K, int halves) {
  return wtype == CBD_BF16 ? packed_bytes_bf16(rows, K, halves) : 0;
}

int cbd_pack_matrix(int wtype, const void* src, void* dst, int rows, int K, int halves, void* stream) {
  if (!src || !dst) return fail(CBD_E_ARG, "null matrix pointer");
  if (cbd_packed_bytes(wtype, rows, K, halves) == 0)
    return fail(CBD_E_UNSUPPORTED, "no packed layout for wtype %d, %d x %d rows, K %d", wtype, halves, rows, K);
  if (((uintptr_t)src | (uintptr_t)dst) & 15) return fail(CBD_E_ARG, "matrix pointers must be 16-byte aligned");
  HIP_TRY(launch_pack_bf16(src, dst, rows, K, halves, (hipStream_t)stream));
  return CBD_OK;
}

size_t cbd_arena_block_bytes(const cbd_config* cfg) {
  if (!cfg || cfg->n_layers <= 0 || cfg->n_kv_heads <= 0 || cfg->head_dim <= 0) return 0;
  const size_t kvb = cfg->wtype == CBD_BF16 ? 2 : 4;
  return 2 * (size_t)cfg->n_layers * cfg->n_kv_heads * ATTN_SPLIT * cfg->head_dim * kvb;
}

size_t cbd_arena_bytes(const cbd_config* cfg, int n_lanes, int max_seq) {
  if (!cfg || n_lanes <= 0 || max_seq <= 0 || cfg->n_layers <= 0 || cfg->n_kv_heads <= 0 || cfg->head_dim <= 0)
    return 0;
  const size_t kvb = cfg->wtype == CBD_BF16 ? 2 : 4;
  const size_t rounded = ((size_t)max_seq + ATTN_SPLIT - 1) / ATTN_SPLIT * ATTN_SPLIT;  // whole blocks
  return 2 * (size_t)n_lanes * cfg->n_layers * cfg->n_kv_heads * rounded * cfg->head_dim * kvb;
}

int cbd_arena_create(cbd_model* m, int n_lanes, int max_seq, void* dev_mem, size_t dev_bytes, cbd_arena** out) {
  if (!m || !out || !dev_mem) return fail(CBD_E_ARG, "null argument");
  if (n_lanes <= 0 || max_seq <= 0) return fail(CBD_E_ARG, "n_lanes and max_seq must be positive");
  if ((uintptr_t)dev_mem & 255u) return fail(CBD_E_ARG, "arena memory must be 256-byte aligned");
  const size_t bb = cbd_arena_block_bytes(&m->c);
  if (dev_bytes < bb) return fail(CBD_E_ARG, "arena needs at least one block of %zu bytes, got %zu", bb, dev_bytes);
  const size_t nb = dev_bytes / bb;
  if (nb > (size_t)INT32_MAX) return fail(CBD_E_ARG, "arena of %zu blocks is too large", nb);
  cbd_arena* a = new cbd_arena();
  a->m = m;
  a->n_lanes = n_lanes;
  a->max_seq = max_seq;
  a->base = (char*)dev_mem;
  a->bytes = dev_bytes;
  a->n_blocks = (int)nb;
  a->block_elems = (long long)m->c.n_kv_heads * ATTN_SPLIT * m->c.head_dim;
  a->region_bytes = nb * (bb / 2);
  a->live.assign(n_lanes, 0);
  a->len.assign(n_lanes, 0);
  a->blocks.assign(n_lanes, std::vector<int>());
  // every lane's block list at its longest, so that taking a block never
  // reallocates (a step allocates no host memory either)
  for (auto& bl : a->blocks) bl.reserve(((size_t)max_seq + ATTN_SPLIT - 1) / ATTN_SPLIT);
  a->free_blocks.resize(nb);
  for (size_t i = 0; i < nb; ++i) a->free_blocks[i] = (int)(nb - 1 - i);
  a->mark.assign(n_lanes, 0u);
  // Pinned staging for a decode step over every lane at up to max_seq
  // positions, so that steps allocate nothing.  Without a usable device (the
  // arena is host bookkeeping over caller memory, and is validated on hosts
  // without one) this fails quietly and the first step sizes the staging.
  const int per = attn_chunks_per_item(m);
  const long long chunks = (max_seq + ATTN_SPLIT - 1) / ATTN_SPLIT;
  if (grow_slots(m, meta_bytes_for(n_lanes, (long long)n_lanes * ((chunks + per - 1) / per))) != CBD_OK) {
    (void)hipGetLastError();
    g_err.clear();
  }
  *out = a;
  return CBD_OK;
}

void cbd_arena_destroy(cbd_arena* a) {
  if (!a) return;
  // graphs captured over this arena hold its pool addresses: drop them
  std::vector<std::pair<cbd_model::GraphKey, hipGraphExec_t>>& gs = a->m->graphs;
  for (size_t i = 0; i < gs.size();) {
    if (gs[i].first.arena == a) {
      (void)hipGraphExecDestroy(gs[i].second);
      gs.erase(gs.begin() + i);
    } else {
      ++i;
    }
  }
  if (a->stage) (void)hipFree(a->stage);
  delete a;
}

int cbd_lane_alloc(cbd_arena* a, int* lane) {
  if (!a || !lane) return fail(CBD_E_ARG, "null argument");
  for (int i = 0; i < a->n_lanes; ++i)
    if (!a->live[i]) {
      a->live[i] = 1;
      a->len[i] = 0;
      *lane = i;
      return CBD_OK;
    }
  return fail(CBD_E_NO_FREE_LANE, "all %d lanes are live", a->n_lanes);
}

static int check_lane(const cbd_arena* a, int lane) {
  if (!a) return fail(CBD_E_ARG, "null arena");
  if (lane < 0 || lane >= a->n_lanes) return fail(CBD_E_ARG, "lane %d outside [0, %d)", lane, a->n_lanes);
  if (!a->live[lane]) return fail(CBD_E_LANE_NOT_LIVE, "lane %d is not live", lane);
  return CBD_OK;
}

// Keep the blocks of a lane's first `length` positions, return the rest.
static void lane_keep(cbd_arena* a, int lane, int length) {
  std::vector<int>& bl = a->blocks[lane];
  const size_t keep = ((size_t)length + ATTN_SPLIT - 1) / ATTN_SPLIT;
  while (bl.size() > keep) {
    a->free_blocks.push_back(bl.back());
    bl.pop_back();
  }
  a->len[lane] = length;
}

int cbd_lane_clear(cbd_arena* a, int lane) {
  int rc = check_lane(a, lane);
  if (rc) return rc;
  lane_keep(a, lane, 0);
  return CBD_OK;
}

int cbd_lane_evict(cbd_arena* a, int lane) {
  int rc = check_lane(a, lane);
  if (rc) return rc;
  lane_keep(a, lane, 0);
  a->live[lane] = 0;
  return CBD_OK;
}

int cbd_arena_free_blocks(const cbd_arena* a) { return a ? (int)a->free_blocks.size() : -1; }
int cbd_arena_n_blocks(const cbd_arena* a) { return a ? a->n_blocks : -1; }

int cbd_lane_length(const cbd_arena* a, int lane) {
  int rc = check_lane(a, lane);
  if (rc) return rc;
  return a->len[lane];
}

size_t cbd_arena_used_bytes(const cbd_arena* a) {
  if (!a) return 0;
  const cbd_config& c = a->m->c;
  const size_t per_tok = 2 * (size_t)c.n_layers * c.n_kv_heads * c.head_dim * a->m->kvb;
  size_t n = 0;
  for (int i = 0; i < a->n_lanes; ++i)
    if (a->live[i]) n += (size_t)a->len[i] * per_tok;
  return n;
}

int cbd_arena_live_lanes(const cbd_arena* a) {
  if (!a) return 0;
  int n = 0;
  for (uint8_t v : a->live) n += v;
  return n;
}

size_t cbd_workspace_bytes(const cbd_model* m, int max_batch, int max_seq) {
  if (!m || max_batch <= 0 || max_seq <= 0) return 0;
  return layout(m, max_batch, max_seq).total;
}

int cbd_lane_truncate(cbd_arena* a, int lane, int length) {
  int rc = check_lane(a, lane);
  if (rc) return rc;
  if (length < 0 || length > a->len[lane])
    return fail(CBD_E_ARG, "length %d outside [0, %d] for lane %d", length, a->len[lane], lane);
  lane_keep(a, lane, length);
  return CBD_OK;
}

int cbd_profile_enable(cbd_model* m, int enable) {
  if (!m) return fail(CBD_E_ARG, "null model");
  m->prof = enable != 0;
  return CBD_OK;
}

int cbd_profile_reset(cbd_model* m) {
  if (!m) return fail(CBD_E_ARG, "null model");
  int rc = drain_profile(m, true);
  if (rc) return rc;
  for (int i = 0; i < 16; ++i) {
    m->prof_ms[i] = 0.0;
    m->prof_n[i] = 0;
  }
  return CBD_OK;
}

int cbd_profile_read(cbd_model* m, int cls, double* total_ms, long long* launches) {
  if (!m || !total_ms || !launches || cls < 0 || cls >= P_N) return fail(CBD_E_ARG, "bad argument");
  int rc = drain_profile(m, true);
  if (rc) return rc;
  *total_ms = m->prof_ms[cls];
  *launches = m->prof_n[cls];
  return CBD_OK;
}

int cbd_profile_classes(void) { return P_N; }

const char* cbd_profile_class_name(int cls) { return cls >= 0 && cls < P_N ? kClassNames[cls] : nullptr; }

long long cbd_debug_alloc_count(void) { return g_allocs.load(); }

int cbd_set_graph_replay(cbd_model* m, int enable) {
  if (!m) return fail(CBD_E_ARG, "null model");
  m->use_graphs = enable != 0;
  return CBD_OK;
}

int cbd_set_variant(cbd_model* m, int variant) {
  if (!m || variant < 0 || variant > 3) return fail(CBD_E_ARG, "variant must be 0, 1, 2 or 3");
  m->variant = variant;
  return CBD_OK;
}

// Automatic choice of the projection family: wide panels from this many
// lanes on, per projection (measured on the 7B shapes at 1-32 lanes, each
// projection alone): below these widths the split-K tiles are as fast or
// faster; above them their per-wave activation re-reads cost more than a
// mostly idle 32-lane panel (at 16 lanes the four layer projections take
// 116 us as split-K tiles, 97 us as panels).  QKV on bf16 models with the
// matrix-core attention shapes is a split-mode panel from one lane, its
// partials added by the attention kernel up to 32 lanes (QKV 15.9 -> 13.2 us
// at one lane, attention +0.6).  The residual projections (O, down) of those
// models keep the split-K tiles (their in-workgroup fold, then the norm
// kernel) up to 16 lanes, one column group: with the residual loaded at
// kernel start they beat the split-mode panels there (8 lanes 2036 -> 2148
// tok/s, 12 lanes 2900 -> 2993, 16 lanes 3680 -> 3718), and run as split-mode
// panels from 17, where the fold also runs the next RMSNorm (tiles of two
// column groups: 24 lanes -5%, 32 lanes -8%).  bf16 gate|up is a full-mode panel from one
// lane (packed weights: 292 -> 297 tok/s at one lane, 1096 -> 1120 at four;
// f32 and Q8_0 keep the split-K tiles up to 16 lanes, one column group).
// Other weight formats and attention shapes keep the split-K tiles for QKV
// and gate|up up to 16 lanes (the SmolLM2-135M shape, Q8_0: 4 lanes 1.065 ->
// about 0.98 ms per step, 8 lanes 1.26 -> 1.17, 16 lanes 1.29 -> 0.97,
// against split-mode panels from 4 and 8 lanes with their norm launches and
// folds) and for O below 24, and run the long reduction (down) as a panel at
// every width.
static int panel_min_b(const cbd_model* m, int epi, int K) {
  const bool bf16_mf = m->wt == WT_BF16 && attn_chunks_per_item(m) == ATTN_GROUP;
  switch (epi) {
    case EPI_STORE: return bf16_mf ? 1 : 17;                // QKV
    case EPI_SWIGLU: return m->wt == WT_BF16 ? 1 : 17;      // gate|up
    case EPI_HEAD: return 4;
    default: return bf16_mf ? 17 : (K > 4096 ? 1 : 24);     // down; O
  }
}

// Panel width C (lanes per workgroup / 16), row blocks per wave and mode for
// one projection at B lanes (measured per projection at 64-512 lanes on the
// 7B shapes). Up to 64 lanes C follows B and a projection splits when full mode
// would give fewer than 512 waves (gate|up and the head, 896 and 1000 waves,
// run 10-20% faster in full mode than split; QKV, O and down, 256-384 waves,
// need the split); a split with a long reduction (down) gives each wave two
// row blocks (10% faster at 64 lanes). Above 64 lanes: two-tile row blocks
// (gate|up, the head) run 128-lane panels in full mode; short one-tile
// projections (QKV, O) run 64-lane panels in full mode once those give 1024
// waves, else 128-lane panels split with two row blocks per wave, as does the
// long reduction (down). Neither width, row blocks per wave nor mode changes
// any output's reduction order.
static void panel_shape(int B, const Plan& p, int epi, int* C, int* rm, int* split) {
  auto units = [&](int c) { return (long long)p.nRB * ((B + TILE * c - 1) / (TILE * c)); };
  const bool one_tile = gemm_rows(epi) == 1;
  *rm = 1;
  if (B <= 64) {
    *C = B <= 32 ? 2 : 4;
    *split = p.S > 1 && units(*C) < 512;
    if (*split && B > 32 && one_tile && p.K > 4096) *rm = 2;
  } else if (!one_tile) {
    *C = 8;
    *split = 0;
  } else if (p.K <= 4096 && units(4) >= 1024) {
    *C = 4;
    *split = 0;
  } else {
    *C = 8;
    *split = p.S > 1;
    if (*split) *rm = 2;
  }
}

// Dense tiles (both operands in LDS) from this many rows on, for bf16 weights
// whose reductions fit them (K a multiple of 128).  Measured per projection on
// the 7B shapes: at 128 lanes the wide panels are faster; from 256 the dense
// tiles are for gate|up, the head and both residual projections (O and down:
// one split per workgroup, its partials folded by the kernel that also runs
// the next RMSNorm; O 38 -> 32 us at 256 lanes), while QKV, whose split
// partials would need a fold launch of their own, stays a panel unless
// whole-K dense workgroups cover the chip (a 4096-row prefill).
constexpr int DENSE_MIN_B = 256;

static bool dense_ok(const cbd_model* m, const Plan& p, int epi) {
  if (m->wt != WT_BF16 || p.K % 128 != 0 || p.Ks % 256 != 0) return false;
  return gemm_rows(epi) == 1 || dense_mode_available(epi, p.K, p.Ks, p.S);
}

// The automatic choice of dense tiles at B rows (see DENSE_MIN_B).
static bool dense_auto(const Plan& p, int epi, int B) {
  if (B < DENSE_MIN_B) return false;
  if (gemm_rows(epi) != 1 || p.K > 4096 || epi == EPI_RESID) return true;
  GemmArgs g{};
  g.N = p.N;
  g.B = B;
  g.S = p.S;
  return dense_mode_available(epi, p.K, p.Ks, p.S) && dense_workgroups(g, epi, 0) >= 256;
}

// Dense mode: a one-tile projection whose whole-K workgroups would not cover
// the 256 compute units, or whose split length has no whole-K kernel, runs one
// split per workgroup with partials; two-tile projections (gate|up, the head)
// have rows enough and never split (dense_ok requires their whole-K kernel).
static int dense_split(int B, const Plan& p, int epi) {
  if (p.S < 2 || gemm_rows(epi) != 1) return 0;
  if (!dense_mode_available(epi, p.K, p.Ks, p.S)) return 1;
  GemmArgs g{};
  g.N = p.N;
  g.B = B;
  g.S = p.S;
  return dense_workgroups(g, epi, 0) < 256 ? 1 : 0;
}

// The RMSNorm of the residual stream that produces a projection's input, not
// yet launched: its gain and the producer's row blocks of sums of x^2.
struct PendingNorm {
  const float* g;
  int ssq_n;
  int rows;  // rows of x (the step's B; the LM head reads only the first n_out)
};

// norm_g: for a residual projection, the gain of the RMSNorm that follows; if
// the projection runs as a split-mode panel its fold also normalises x into
// xn, and *normed says so (the caller then launches no norm).  unfolded: for
// QKV, the consumer can add split partials itself; if the projection runs as
// a split-mode panel its fold is skipped and *unfolded says so.
// pre: the RMSNorm that produces X (xn), if not yet run; split-K tiles of one
// column group run it themselves (no norm launch), otherwise it is launched
// here first.
static int run_gemm(cbd_model* m, int cls, const Plan& p, int epi, const cbd_matrix& W, const void* X, int B, float* out,
                    void* act_out, char* ws, const WsLayout& L, hipStream_t st, const float* norm_g = nullptr,
                    bool* normed = nullptr, bool* unfolded = nullptr, const PendingNorm* pre = nullptr) {
  GemmArgs g{};
  g.W = W.data;
  g.Ws = (const uint16_t*)W.scale;
  g.X = X;
  g.N = p.N;
  g.Nraw = p.Nraw;
  g.K = p.K;
  g.B = B;
  g.S = p.S;
  g.Ks = p.Ks;
  g.nRB = p.nRB;
  g.out = out;
  g.act_out = act_out;
  g.amax = (float2*)(ws + L.amax);
  g.ssq_out = (float*)(ws + L.ssq);
  g.part = (float*)(ws + L.gpart);
  // packed tile layout: the layer matrices and an untied head (a tied head is
  // the row-major embedding)
  g.wpack = m->c.packed && (epi != EPI_HEAD || !m->c.tied_embeddings) ? 1 : 0;
  g.wtiles = (p.N + TILE - 1) / TILE;
  const bool dense = dense_ok(m, p, epi) && (m->variant == 3 || (m->variant == 0 && dense_auto(p, epi, B)));
  const bool panel = !dense && (m->variant == 2 || m->variant == 3 || (m->variant == 0 && B >= panel_min_b(m, epi, p.K)));
  const int C1 = B <= 16 ? 1 : (B <= 32 ? 2 : 4);  // split-K tiles: column group width / 16
  if (pre) {
    if (!dense && !panel && C1 == 1 && epi != EPI_RESID && pre->rows == B &&
        gemm_norm_in_supported(B, p.K, p.S, p.Ks, m->actb, pre->ssq_n)) {
      g.in_x = (const float*)(ws + L.x);
      g.in_ssq = (const float*)(ws + L.ssq);
      g.in_ssq_n = pre->ssq_n;
      g.in_g = pre->g;
      g.in_eps = m->c.rms_eps;
    } else {
      ProfScope pn(m, P_NORM, st);
      HIP_TRY(launch_norm(m->wt, (const float*)(ws + L.x), (const float*)(ws + L.ssq), pre->ssq_n, pre->g,
                          pre->rows, m->c.d_model, m->c.rms_eps, ws + L.xn, st));
    }
  }
  ProfScope ps(m, cls, st);
  if (dense) {
    const int split = dense_split(B, p, epi);
    if (split && (size_t)4 * p.S * p.nRB * TILE * gemm_rows(epi) * B > L.gpart_bytes)
      return fail(CBD_E_WORKSPACE, "split partials of %d lanes exceed the workspace's %zu bytes", B, L.gpart_bytes);
    if (epi == EPI_RESID && split && norm_g && normed && fold_norm_supported(p.N)) {
      g.norm_g = norm_g;
      g.norm_eps = m->c.rms_eps;
      g.norm_out = ws + L.xn;
      *normed = true;
    }
    if (epi == EPI_STORE && split && unfolded) {
      g.fold_elsewhere = 1;
      *unfolded = true;
    }
    HIP_TRY(launch_dense(epi, split, g, st));
  } else if (panel) {
    int C, rm, split;
    panel_shape(B, p, epi, &C, &rm, &split);
    if (split && (size_t)4 * p.S * p.nRB * TILE * gemm_rows(epi) * B > L.gpart_bytes)
      return fail(CBD_E_WORKSPACE, "split partials of %d lanes exceed the workspace's %zu bytes", B, L.gpart_bytes);
    if (epi == EPI_RESID && split && norm_g && normed && fold_norm_supported(p.N)) {
      g.norm_g = norm_g;
      g.norm_eps = m->c.rms_eps;
      g.norm_out = ws + L.xn;
      *normed = true;
    }
    if (epi == EPI_STORE && split && unfolded) {
      g.fold_elsewhere = 1;
      *unfolded = true;
    }
    HIP_TRY(launch_panel(m->wt, epi, C, rm, split, g, st));
  } else {
    g.nCG = (B + TILE * C1 - 1) / (TILE * C1);
    HIP_TRY(launch_gemm(m->wt, epi, C1, g, st));
  }
  return CBD_OK;
}

// Every kernel of one step, in order, on `st` (plain launches or a capture),
// over B rows (a lane at a position with a token each); the first n_out rows
// produce logits and argmax.  multi: some lane has several rows, so attention
// appends every row's K/V first and then reads all keys from the cache.
// Arguments depend only on (B, n_out, multi, workspace layout, arena,
// outputs): the per-step data (lanes, positions, tokens, attention items) is
// read from the workspace.
static int enqueue_step(cbd_model* m, cbd_arena* a, int B, int n_out, bool multi, bool direct, int row_items,
                        char* ws, const WsLayout& L, float* logits, int32_t* argmax, hipStream_t st) {
  const cbd_config& c = m->c;
  const int32_t* dmeta = (const int32_t*)(ws + L.meta);
  const int* d_lanes = dmeta;
  const int* d_pos = dmeta + B;
  const int* d_tok = dmeta + 2 * B;
  const int* d_nitems = dmeta + 5 * B;
  const int* d_items = dmeta + meta_header(B);
  float* x = (float*)(ws + L.x);
  float* ssq = (float*)(ws + L.ssq);
  float* qkv = (float*)(ws + L.qkv);
  void* o = ws + L.o;
  void* act = ws + L.a;
  float2* rope = (float2*)(ws + L.rope);
  const int d = c.d_model;

  {
    ProfScope ps(m, P_EMBED, st);
    HIP_TRY(launch_embed(m->wt, m->embed.data, (const uint16_t*)m->embed.scale, d_tok, d_pos, B, d, c.head_dim,
                         c.rope_theta, x, ssq, rope, st));
  }
  AttnArgs at{};
  at.qkv = qkv;
  at.kpool = a->base;
  at.vpool = a->base + a->region_bytes;
  at.block_elems = a->block_elems;
  at.B = B;
  at.lanes = d_lanes;
  at.pos = d_pos;
  at.items = d_items;
  at.n_items_dev = d_nitems;
  at.per = attn_chunks_per_item(m);
  at.max_items = B * L.parts;
  at.max_splits = L.parts;
  at.Hq = c.n_heads;
  at.Hkv = c.n_kv_heads;
  at.G = m->G;
  at.Nqkv = m->n_qkv;
  at.rope = rope;
  at.part = (float*)(ws + L.apart);
  at.out = o;
  at.act = m->wt;
  at.rowmap = dmeta + 3 * B;
  at.rowblk = dmeta + 4 * B;
  at.frag = kv_frag(m) ? 1 : 0;
  int rc;
  void* xn = ws + L.xn;
  // The RMSNorm of x into xn that the next projection consumes, run by that
  // projection (or launched just before it); ssq_n = row blocks of the last
  // producer of x (the embedding: one).  None pending when a split-mode fold
  // has already normalised x.
  PendingNorm pn{m->attn_norm[0], 1, B};
  const PendingNorm* pending = &pn;
  for (int l = 0; l < c.n_layers; ++l) {
    // Up to 32 lanes the matrix-core attention kernel adds the QKV split
    // partials itself (no fold launch: QKV 18.8 -> 14.7 us at 32 lanes,
    // attention 51.9 -> 54.1); wider, each lane's partials are re-read by all
    // its attention workgroups (at 64 lanes QKV -6.2 us, attention +7.1).
    bool unfolded = false;
    const bool attn_folds = !multi && B <= 32 && attn_mfma_supported(c.head_dim, m->wt == WT_BF16, m->G);
    if ((rc = run_gemm(m, P_QKV, m->p_qkv, EPI_STORE, m->qkv[l], xn, B, qkv, nullptr, ws, L, st, nullptr, nullptr,
                       attn_folds ? &unfolded : nullptr, pending)))
      return rc;
    at.qkv_part = unfolded ? (const float*)(ws + L.gpart) : nullptr;
    at.qkv_S = unfolded ? m->p_qkv.S : 0;
    at.layer_off = (long long)l * a->n_blocks * a->block_elems;
    {
      ProfScope ps(m, P_ATTN, st);
      if (multi) {
        // every row's K/V first, then every row attends to its lane's cache:
        // runs of one lane's rows per work item on the matrix-core shapes
        HIP_TRY(launch_kv_append(c.head_dim, m->wt == WT_BF16, at, st));
        at.mode = ATTN_ATTEND;
        if (row_items >= 0) {
          AttnArgs ar = at;
          ar.max_items = row_items;
          HIP_TRY(launch_attn_rows(c.head_dim, ar, st));
        } else {
          HIP_TRY(launch_attn(c.head_dim, m->wt == WT_BF16, at, st));
        }
      } else {
        at.mode = ATTN_FUSED;
        HIP_TRY(launch_attn(c.head_dim, m->wt == WT_BF16, at, st));
      }
    }
    if (!direct) {
      ProfScope ps(m, P_COMB, st);
      HIP_TRY(launch_attn_combine(c.head_dim, m->wt, at, st));
    }
    bool normed = false;
    if ((rc = run_gemm(m, P_O, m->p_o, EPI_RESID, m->o[l], o, B, x, nullptr, ws, L, st, m->ffn_norm[l], &normed)))
      return rc;
    pn = PendingNorm{m->ffn_norm[l], m->p_o.nRB, B};
    pending = normed ? nullptr : &pn;
    if ((rc = run_gemm(m, P_GU, m->p_gu, EPI_SWIGLU, m->gu[l], xn, B, nullptr, act, ws, L, st, nullptr, nullptr,
                       nullptr, pending)))
      return rc;
    const float* gnext = l + 1 < c.n_layers ? m->attn_norm[l + 1] : m->final_norm;
    normed = false;
    if ((rc = run_gemm(m, P_DOWN, m->p_down, EPI_RESID, m->down[l], act, B, x, nullptr, ws, L, st, gnext, &normed)))
      return rc;
    pn = PendingNorm{gnext, m->p_down.nRB, B};
    pending = normed ? nullptr : &pn;
  }
  if ((rc = run_gemm(m, P_HEAD, m->p_head, EPI_HEAD, m->head, xn, n_out, logits, nullptr, ws, L, st, nullptr, nullptr,
                     nullptr, pending)))
    return rc;
  if (argmax) {
    ProfScope ps(m, P_ARGMAX, st);
    HIP_TRY(launch_argmax((const float2*)(ws + L.amax), m->p_head.nRB, n_out, argmax, st));
  }
  return CBD_OK;
}

// Copy B rows' metadata (lane, position, token) and their attention work
// items to the workspace and run the step over them; the first n_out rows
// produce logits and argmax.  Blocks for every row's slot are already taken.
static int submit_rows(cbd_model* m, cbd_arena* a, int B, int n_out, bool multi, const int32_t* lanes,
                       const int32_t* positions, const int32_t* tokens, char* ws, size_t workspace_bytes,
                       const WsLayout& L, float* logits, int32_t* argmax, hipStream_t st, bool noalloc = false) {
  // Per-step metadata: lanes, positions, tokens, item count, attention work
  // items {b | chunks << 24, first chunk, position, 0, block of each chunk}: a
  // workgroup of the attention kernel takes one aligned group of up to `per`
  // consecutive 64-key chunks of one lane, the same groups whatever B is.
  // Written straight into a pinned staging slot (sized when the arena was
  // created, so a decode step allocates nothing), then one copy to the workspace.
  const size_t hdr = meta_header(B);
  const int per = attn_chunks_per_item(m);
  // A multi-row call on the matrix-core shapes attends by runs of one lane's
  // rows at consecutive positions (k_attn_rows): sort the rows by (lane,
  // position); a run is cut where the lane changes or a position is skipped.
  const bool by_runs = multi && per == ATTN_GROUP;
  std::vector<int32_t>& ord = m->row_order;
  long long items = 0;
  if (by_runs) {
    ord.resize(B);
    for (int b = 0; b < B; ++b) ord[b] = b;
    std::sort(ord.begin(), ord.end(), [&](int x, int y) {
      return lanes[x] != lanes[y] ? lanes[x] < lanes[y] : positions[x] < positions[y];
    });
  }
  // visits each run [s, e) of ord with its first and last positions
  auto for_runs = [&](auto&& fn) {
    for (int s = 0; s < B;) {
      int e = s + 1;
      while (e < B && lanes[ord[e]] == lanes[ord[s]] && positions[ord[e]] == positions[ord[e - 1]] + 1) ++e;
      fn(s, e, positions[ord[s]], positions[ord[e - 1]]);
      s = e;
    }
  };
  const int GROUP_KEYS = ATTN_SPLIT * ATTN_GROUP;
  if (by_runs) {
    for_runs([&](int, int, int P0, int P1) {
      for (int k = 0; k * GROUP_KEYS <= P1; ++k) {
        const int lo = std::max(P0, k * GROUP_KEYS);
        items += (P1 - lo + ATTN_ROWS_MAX) / ATTN_ROWS_MAX;
      }
    });
  } else {
    for (int b = 0; b < B; ++b) items += ((positions[b] + ATTN_SPLIT) / ATTN_SPLIT + per - 1) / per;
  }
  const size_t meta_bytes = meta_bytes_for(B, items);
  if (meta_bytes > L.meta_bytes)
    return fail(CBD_E_WORKSPACE, "step metadata of %zu bytes exceeds the workspace's %zu", meta_bytes, L.meta_bytes);
  const int si = m->next_slot;
  m->next_slot = (si + 1) % NSLOT;
  if (m->slot_bytes[si] < meta_bytes) {
    if (noalloc)
      return fail(CBD_E_WORKSPACE, "pinned staging of %zu bytes is smaller than the step's %zu (the arena was "
                  "created without a usable device)", m->slot_bytes[si], meta_bytes);
    int rc = grow_slots(m, meta_bytes);  // a prefill call with more rows than any arena's lanes
    if (rc) return rc;
  } else if (m->ev_live[si]) {
    HIP_TRY(hipEventSynchronize(m->ev[si]));
  }
  int32_t* meta = (int32_t*)m->slot[si];
  memcpy(meta, lanes, sizeof(int32_t) * B);
  memcpy(meta + B, positions, sizeof(int32_t) * B);
  memcpy(meta + 2 * B, tokens, sizeof(int32_t) * B);
  for (size_t i = 3 * (size_t)B; i < hdr; ++i) meta[i] = 0;
  int32_t* it = meta + hdr;
  int n_items = 0;
  if (multi) {
    for (int b = 0; b < B; ++b) meta[4 * B + b] = a->blocks[lanes[b]][positions[b] / ATTN_SPLIT];
  }
  if (by_runs) {
    // items of a run: for each group k its rows reach (positions from
    // max(P0, first key of the group)), blocks of ATTN_ROWS_MAX rows
    for (int b = 0; b < B; ++b) meta[3 * B + b] = ord[b];
    for_runs([&](int s, int, int P0, int P1) {
      const std::vector<int>& bl = a->blocks[lanes[ord[s]]];
      const int nch = P1 / ATTN_SPLIT + 1;  // chunks the run's last row reaches
      for (int k = 0; k * GROUP_KEYS <= P1; ++k) {
        const int c0 = k * ATTN_GROUP;
        for (int pa = std::max(P0, k * GROUP_KEYS); pa <= P1; pa += ATTN_ROWS_MAX) {
          const int nr = std::min(ATTN_ROWS_MAX, P1 - pa + 1);
          it[0] = (s + (pa - P0)) | (nr << 24);
          it[1] = c0;
          it[2] = pa;
          it[3] = std::min(ATTN_GROUP, (pa + nr - 1) / ATTN_SPLIT + 1 - c0);
          for (int q = 0; q < ATTN_GROUP; ++q) it[4 + q] = bl[std::min(c0 + q, nch - 1)];
          it += ITEM_INTS;
          ++n_items;
        }
      }
    });
  }
  // Items by chunk count: groups of `per` chunks first (every lane's), then
  // the lanes' shorter last groups, longest first, so that the launch drains
  // on the cheapest items (the order changes no result).
  for (int want = per; !by_runs && want >= 1; --want)
    for (int b = 0; b < B; ++b) {
      const int ns = (positions[b] + ATTN_SPLIT) / ATTN_SPLIT;  // chunks holding slots 0..positions[b]
      const std::vector<int>& bl = a->blocks[lanes[b]];
      for (int s0 = 0; s0 < ns; s0 += per) {
        const int n = std::min(per, ns - s0);
        if (n != want) continue;
        it[0] = b | (n << 24);
        it[1] = s0;
        it[2] = positions[b];
        it[3] = 0;
        for (int k = 0; k < ATTN_GROUP; ++k) it[4 + k] = k < n ? bl[s0 + k] : bl[s0 + n - 1];
        it += ITEM_INTS;
        ++n_items;
      }
    }
  meta[5 * B] = n_items;
  int32_t* dmeta = (int32_t*)(ws + L.meta);
  {
    ProfScope ps(m, P_META, st);
    HIP_TRY(launch_meta_copy(dmeta, m->slot_dev[si], meta_bytes, st));
  }
  HIP_TRY(hipEventRecord(m->ev[si], st));
  m->ev_live[si] = true;

  // Every row's keys in one work item (one attention partial per lane): the
  // attention kernel finishes the rows itself and the combine is not launched.
  int max_pos = 0;
  for (int b = 0; b < B; ++b) max_pos = std::max(max_pos, positions[b]);
  const bool direct = max_pos < ATTN_SPLIT * per;
  int rc;
  const bool graph = m->use_graphs && !m->prof && !multi && !noalloc;  // instantiating a graph allocates
  if (!graph) {
    if ((rc = enqueue_step(m, a, B, n_out, multi, direct, by_runs ? n_items : -1, ws, L, logits, argmax, st)))
      return rc;
  } else {
    const cbd_model::GraphKey key{B,          ws,        a,           a->base,    logits,
                                  argmax,     workspace_bytes, a->region_bytes, a->max_seq, a->n_lanes,
                                  a->n_blocks, m->variant, direct};
    hipGraphExec_t exec = nullptr;
    for (auto& g : m->graphs)
      if (g.first == key) exec = g.second;
    if (!exec) {
      if (!m->cap_stream) HIP_TRY(hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking));
      hipGraph_t graph_def = nullptr;
      HIP_TRY(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal));
      rc = enqueue_step(m, a, B, n_out, multi, direct, -1, ws, L, logits, argmax, m->cap_stream);
      hipError_t e = hipStreamEndCapture(m->cap_stream, &graph_def);
      if (rc) {
        if (graph_def) (void)hipGraphDestroy(graph_def);
        return rc;
      }
      if (e != hipSuccess) return fail(CBD_E_HIP, "graph capture failed: %s", hipGetErrorString(e));
      e = hipGraphInstantiate(&exec, graph_def, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph_def);
      if (e != hipSuccess) return fail(CBD_E_HIP, "graph instantiate failed: %s", hipGetErrorString(e));
      if (m->graphs.size() >= 64) {
        (void)hipGraphExecDestroy(m->graphs.front().second);
        m->graphs.erase(m->graphs.begin());
      }
      m->graphs.push_back({key, exec});
    }
    HIP_TRY(hipGraphLaunch(exec, st));
  }
  if (m->prof && (rc = drain_profile(m, false))) return rc;
  return CBD_OK;
}

}  // extern "C"

// The decode step over a workspace; noalloc: the workspace is the device's
// static scratch, and nothing may allocate (no staging growth, no graph).
static int decode_step_impl(cbd_model* m, cbd_arena* a, int B, const int32_t* lanes, int32_t* positions,
                            const int32_t* tokens, float* logits, int32_t* argmax, void* workspace,
                            size_t workspace_bytes, void* stream, bool noalloc) {
  if (!m || !a || !lanes || !positions || !tokens || !logits) return fail(CBD_E_ARG, "null argument");
  if (a->m != m) return fail(CBD_E_ARG, "arena belongs to another model");
  if (B < 1) return fail(CBD_E_ARG, "B = %d < 1", B);
  const cbd_config& c = m->c;
  // lanes: range, liveness, distinctness; positions; tokens
  if (++a->epoch == 0) {
    std::fill(a->mark.begin(), a->mark.end(), 0u);
    a->epoch = 1;
  }
  for (int b = 0; b < B; ++b) {
    const int ln = lanes[b];
    if (ln < 0 || ln >= a->n_lanes) return fail(CBD_E_ARG, "lanes[%d] = %d outside [0, %d)", b, ln, a->n_lanes);
    if (a->mark[ln] == a->epoch) return fail(CBD_E_DUP_LANE, "lane %d appears twice", ln);
    a->mark[ln] = a->epoch;
    if (!a->live[ln]) return fail(CBD_E_LANE_NOT_LIVE, "lane %d is not live", ln);
    if (positions[b] != a->len[ln])
      return fail(CBD_E_POS_MISMATCH, "positions[%d] = %d but lane %d holds %d tokens", b, positions[b], ln,
                  a->len[ln]);
    if (positions[b] >= a->max_seq)
      return fail(CBD_E_KV_FULL, "lane %d is full (%d of %d slots)", ln, positions[b], a->max_seq);
    if (tokens[b] < 0 || tokens[b] >= c.vocab)
      return fail(CBD_E_TOKEN, "tokens[%d] = %d outside [0, %d)", b, tokens[b], c.vocab);
  }
  // slot positions[b] opens a new chunk for lanes whose blocks end there
  int new_blocks = 0;
  for (int b = 0; b < B; ++b)
    if ((size_t)positions[b] / ATTN_SPLIT >= a->blocks[lanes[b]].size()) ++new_blocks;
  if (new_blocks > (int)a->free_blocks.size())
    return fail(CBD_E_KV_FULL, "the step needs %d new KV blocks, %zu of %d are free", new_blocks,
                a->free_blocks.size(), a->n_blocks);
  if (!workspace) return fail(CBD_E_WORKSPACE, "null workspace");
  if ((uintptr_t)workspace & 255u) return fail(CBD_E_WORKSPACE, "workspace must be 256-byte aligned");
  const int maxB = max_batch_for(m, a->max_seq, workspace_bytes);
  if (maxB < B)
    return fail(CBD_E_WORKSPACE, "%s of %zu bytes holds %d lanes at max_seq %d, step has %d (need %zu)",
                noalloc ? "static scratch" : "workspace", workspace_bytes, maxB, a->max_seq, B,
                cbd_workspace_bytes(m, B, a->max_seq));
  const WsLayout L = layout(m, maxB, a->max_seq);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;

  // The step's new blocks (validated above: the pool has them).
  for (int b = 0; b < B; ++b) {
    std::vector<int>& bl = a->blocks[lanes[b]];
    if ((size_t)positions[b] / ATTN_SPLIT >= bl.size()) {
      bl.push_back(a->free_blocks.back());
      a->free_blocks.pop_back();
    }
  }
  int rc = submit_rows(m, a, B, B, false, lanes, positions, tokens, ws, workspace_bytes, L, logits, argmax, st,
                       noalloc);
  if (rc) return rc;

  for (int b = 0; b < B; ++b) {
    positions[b] += 1;
    a->len[lanes[b]] += 1;
  }
  return CBD_OK;
}

// Scratch of the allocation-free step: one copy per device, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (its
// host-side name is not a device address): it uses the address
// hipGetSymbolAddress gives on the current device.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
static std::atomic<void*> g_scratch[MAX_DEVICES];

static int scratch_address(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(CBD_E_UNSUPPORTED, "device %d beyond %d", dev, MAX_DEVICES);
  void* p = g_scratch[dev].load();
  if (!p) {
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(CBD_E_HIP, "no device address for the static scratch on device %d", dev);
    g_scratch[dev].store(p);  // the same address whichever thread stores it
  }
  *out = p;
  return CBD_OK;
}

extern "C" {

int cbd_decode_step_batch(cbd_model* m, cbd_arena* a, int B, const int32_t* lanes, int32_t* positions,
                          const int32_t* tokens, float* logits, int32_t* argmax, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_step_impl(m, a, B, lanes, positions, tokens, logits, argmax, workspace, workspace_bytes, stream,
                          false);
}

size_t cbd_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

int cbd_decode_step_batch_noalloc(cbd_model* m, cbd_arena* a, int B, const int32_t* lanes, int32_t* positions,
                                  const int32_t* tokens, float* logits, int32_t* argmax, void* stream) {
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  return decode_step_impl(m, a, B, lanes, positions, tokens, logits, argmax, ws, NOALLOC_SCRATCH_BYTES, stream,
                          true);
}

int cbd_prefill_batch(cbd_model* m, cbd_arena* a, int n_seq, const int32_t* lanes, int32_t* positions,
                      const int32_t* counts, const int32_t* tokens, float* logits, int32_t* argmax, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!m || !a || !lanes || !positions || !counts || !tokens || !logits) return fail(CBD_E_ARG, "null argument");
  if (a->m != m) return fail(CBD_E_ARG, "arena belongs to another model");
  if (n_seq < 1) return fail(CBD_E_ARG, "n_seq = %d < 1", n_seq);
  const cbd_config& c = m->c;
  // distinct lanes: the arena's per-call marks, as the decode step checks them
  // (no host allocation per call)
  if (++a->epoch == 0) {
    std::fill(a->mark.begin(), a->mark.end(), 0u);
    a->epoch = 1;
  }
  long long R = 0;
  int new_blocks = 0;
  bool multi = false;
  for (int i = 0; i < n_seq; ++i) {
    const int ln = lanes[i];
    if (ln < 0 || ln >= a->n_lanes) return fail(CBD_E_ARG, "lanes[%d] = %d outside [0, %d)", i, ln, a->n_lanes);
    if (a->mark[ln] == a->epoch) return fail(CBD_E_DUP_LANE, "lane %d appears twice", ln);
    a->mark[ln] = a->epoch;
    if (!a->live[ln]) return fail(CBD_E_LANE_NOT_LIVE, "lane %d is not live", ln);
    if (positions[i] != a->len[ln])
      return fail(CBD_E_POS_MISMATCH, "positions[%d] = %d but lane %d holds %d tokens", i, positions[i], ln,
                  a->len[ln]);
    if (counts[i] < 1) return fail(CBD_E_ARG, "counts[%d] = %d < 1", i, counts[i]);
    if ((long long)positions[i] + counts[i] > a->max_seq)
      return fail(CBD_E_KV_FULL, "lane %d: %d + %d positions exceed max_seq %d", ln, positions[i], counts[i],
                  a->max_seq);
    const long long need = ((long long)positions[i] + counts[i] + ATTN_SPLIT - 1) / ATTN_SPLIT;
    if (need > (long long)a->blocks[ln].size()) new_blocks += (int)(need - (long long)a->blocks[ln].size());
    multi = multi || counts[i] > 1;
    R += counts[i];
  }
  for (long long r = 0; r < R; ++r)
    if (tokens[r] < 0 || tokens[r] >= c.vocab)
      return fail(CBD_E_TOKEN, "tokens[%lld] = %d outside [0, %d)", r, tokens[r], c.vocab);
  if (new_blocks > (int)a->free_blocks.size())
    return fail(CBD_E_KV_FULL, "the call needs %d new KV blocks, %zu of %d are free", new_blocks,
                a->free_blocks.size(), a->n_blocks);
  if (!workspace) return fail(CBD_E_WORKSPACE, "null workspace");
  if ((uintptr_t)workspace & 255u) return fail(CBD_E_WORKSPACE, "workspace must be 256-byte aligned");
  const int maxB = max_batch_for(m, a->max_seq, workspace_bytes);
  if (maxB < R)
    return fail(CBD_E_WORKSPACE, "workspace of %zu bytes holds %d rows, the call has %lld", workspace_bytes, maxB, R);
  const WsLayout L = layout(m, maxB, a->max_seq);

  // Blocks for every new slot (validated above: the pool has them).
  for (int i = 0; i < n_seq; ++i) {
    std::vector<int>& bl = a->blocks[lanes[i]];
    const size_t need = ((size_t)positions[i] + counts[i] + ATTN_SPLIT - 1) / ATTN_SPLIT;
    while (bl.size() < need) {
      bl.push_back(a->free_blocks.back());
      a->free_blocks.pop_back();
    }
  }
  // Rows: each lane's last token first (rows 0..n_seq-1 give the logits), then
  // the lane's earlier tokens in order.
  std::vector<int32_t> rl, rp, rt;
  rl.reserve(R);
  rp.reserve(R);
  rt.reserve(R);
  std::vector<long long> off(n_seq + 1, 0);
  for (int i = 0; i < n_seq; ++i) off[i + 1] = off[i] + counts[i];
  for (int i = 0; i < n_seq; ++i) {
    rl.push_back(lanes[i]);
    rp.push_back(positions[i] + counts[i] - 1);
    rt.push_back(tokens[off[i + 1] - 1]);
  }
  for (int i = 0; i < n_seq; ++i)
    for (int t = 0; t + 1 < counts[i]; ++t) {
      rl.push_back(lanes[i]);
      rp.push_back(positions[i] + t);
      rt.push_back(tokens[off[i] + t]);
    }
  int rc = submit_rows(m, a, (int)R, n_seq, multi, rl.data(), rp.data(), rt.data(), (char*)workspace,
                       workspace_bytes, L, logits, argmax, (hipStream_t)stream);
  if (rc) return rc;
  for (int i = 0; i < n_seq; ++i) {
    positions[i] += counts[i];
    a->len[lanes[i]] += counts[i];
  }
  return CBD_OK;
}

int cbd_decode_step(cbd_model* m, cbd_arena* a, int lane, int32_t* position, int32_t token, float* logits,
                    int32_t* argmax, void* workspace, size_t workspace_bytes, void* stream) {
  if (!position) return fail(CBD_E_ARG, "null position");
  const int32_t ln = lane, tok = token;
  return cbd_decode_step_batch(m, a, 1, &ln, position, &tok, logits, argmax, workspace, workspace_bytes, stream);
}

// Rows [n_rows][len][hd] of positions [p0, p0 + len) of a lane (block list on
// the device) to or from the K (v = false) or V pool, in the pool's chunk order.
static hipError_t kv_rows(cbd_arena* a, char* pool, char* rows, const int* dblk, int p0, int len, bool v, bool to_pool,
                          hipStream_t st) {
  const cbd_config& c = a->m->c;
  const long long bbytes = a->block_elems * (long long)a->m->kvb;
  const long long lstride = (long long)a->n_blocks * bbytes;
  const int n_rows = c.n_layers * c.n_kv_heads;
  if (kv_frag(a->m))
    return launch_kv_rows_frag(pool, rows, dblk, p0, len, n_rows, c.n_kv_heads, c.head_dim, lstride, bbytes, to_pool,
                               v ? 2 : 1, st);
  return launch_kv_rows(pool, rows, dblk, p0, len, n_rows, c.n_kv_heads, c.head_dim * (int)a->m->kvb, lstride, bbytes,
                        to_pool, st);
}

// Copy a lane's K or V between rows [L][Hkv][len][hd] (host or device) and its
// blocks: one contiguous copy through the arena's device staging buffer, and
// one kernel that moves the rows to or from the blocks.
static int copy_lane(cbd_arena* a, int lane, int len, char* rows, bool to_pool, bool v, hipStream_t st) {
  const cbd_config& c = a->m->c;
  const size_t kvb = a->m->kvb;
  const int n_rows = c.n_layers * c.n_kv_heads;
  const int row_bytes = c.head_dim * (int)kvb;
  const size_t bytes = (size_t)n_rows * len * row_bytes;
  const size_t boff = (bytes + 255) & ~(size_t)255;
  const std::vector<int>& bl = a->blocks[lane];
  const size_t need = boff + bl.size() * sizeof(int);
  if (a->stage_bytes < need) {
    HIP_TRY(hipStreamSynchronize(st));
    if (a->stage) HIP_TRY(hipFree(a->stage));
    a->stage = nullptr;
    a->stage_bytes = 0;
    HIP_TRY(counted_malloc((void**)&a->stage, need));
    a->stage_bytes = need;
  }
  char* pool = a->base + (v ? a->region_bytes : 0);
  int* dblk = (int*)(a->stage + boff);
  HIP_TRY(hipMemcpyAsync(dblk, bl.data(), bl.size() * sizeof(int), hipMemcpyHostToDevice, st));
  if (to_pool) {
    HIP_TRY(hipMemcpyAsync(a->stage, rows, bytes, hipMemcpyDefault, st));
    HIP_TRY(kv_rows(a, pool, a->stage, dblk, 0, len, v, true, st));
  } else {
    HIP_TRY(kv_rows(a, pool, a->stage, dblk, 0, len, v, false, st));
    HIP_TRY(hipMemcpyAsync(rows, a->stage, bytes, hipMemcpyDefault, st));
  }
  // the staging buffer (and the block list) are reused by the next copy
  HIP_TRY(hipStreamSynchronize(st));
  return CBD_OK;
}

int cbd_lane_kv_export(cbd_arena* a, int lane, void* k_dst, void* v_dst, void* stream) {
  int rc = check_lane(a, lane);
  if (rc) return rc;
  if (!k_dst || !v_dst) return fail(CBD_E_ARG, "null destination");
  const int len = a->len[lane];
  hipStream_t st = (hipStream_t)stream;
  if (len > 0) {
    if ((rc = copy_lane(a, lane, len, (char*)k_dst, false, false, st))) return rc;
    if ((rc = copy_lane(a, lane, len, (char*)v_dst, false, true, st))) return rc;
  }
  HIP_TRY(hipStreamSynchronize(st));
  return CBD_OK;
}

int cbd_lane_clone(cbd_arena* a, int src, int dst, int n, void* stream) {
  int rc = check_lane(a, src);
  if (rc) return rc;
  if ((rc = check_lane(a, dst))) return rc;
  if (src == dst) return fail(CBD_E_ARG, "source and destination are the same lane %d", src);
  if (n < 0 || n > a->len[src]) return fail(CBD_E_ARG, "n = %d outside [0, %d] for lane %d", n, a->len[src], src);
  const size_t need = ((size_t)n + ATTN_SPLIT - 1) / ATTN_SPLIT;
  if (need > a->free_blocks.size() + a->blocks[dst].size())
    return fail(CBD_E_KV_FULL, "cloning %d positions needs %zu KV blocks, %zu are free", n, need,
                a->free_blocks.size() + a->blocks[dst].size());
  lane_keep(a, dst, 0);
  std::vector<int>& bl = a->blocks[dst];
  while (bl.size() < need) {
    bl.push_back(a->free_blocks.back());
    a->free_blocks.pop_back();
  }
  // whole blocks, every layer, K and V: one kernel over the block pairs, whose
  // lists go to the device through the arena's staging buffer
  hipStream_t st = (hipStream_t)stream;
  if (need > 0) {
    const size_t lb = need * sizeof(int);
    if (a->stage_bytes < 2 * lb) {
      HIP_TRY(hipStreamSynchronize(st));
      if (a->stage) HIP_TRY(hipFree(a->stage));
      a->stage = nullptr;
      a->stage_bytes = 0;
      HIP_TRY(counted_malloc((void**)&a->stage, 2 * lb));
      a->stage_bytes = 2 * lb;
    }
    std::vector<int> pairs(a->blocks[src].begin(), a->blocks[src].begin() + need);
    pairs.insert(pairs.end(), bl.begin(), bl.end());
    int* d = (int*)a->stage;
    HIP_TRY(hipMemcpyAsync(d, pairs.data(), 2 * lb, hipMemcpyHostToDevice, st));
    const long long bbytes = a->block_elems * (long long)a->m->kvb;
    HIP_TRY(launch_kv_blocks(a->base, (long long)a->region_bytes, d, d + need, (int)need, a->m->c.n_layers,
                             (long long)a->n_blocks * bbytes, bbytes, st));
    // the staging buffer and the host list are reused by the next call
    HIP_TRY(hipStreamSynchronize(st));
  }
  a->len[dst] = n;
  return CBD_OK;
}

int cbd_lane_evict_span(cbd_arena* a, int lane, int begin, int end, void* stream) {
  int rc = check_lane(a, lane);
  if (rc) return rc;
  const int len = a->len[lane];
  if (begin < 0 || end < begin || end > len)
    return fail(CBD_E_ARG, "span [%d, %d) outside [0, %d] for lane %d", begin, end, len, lane);
  const int d = end - begin, n = len - end;  // span length; entries that move
  hipStream_t st = (hipStream_t)stream;
  if (d > 0 && n > 0) {
    const cbd_config& c = a->m->c;
    const size_t kvb = a->m->kvb;
    const int n_rows = c.n_layers * c.n_kv_heads, row_bytes = c.head_dim * (int)kvb, h = c.head_dim / 2;
    const std::vector<int>& bl = a->blocks[lane];
    // rotary angle of -d positions per pair: theta_j = theta^(-2j/hd) in double, cos and sin rounded to f32
    std::vector<float> cs(2 * h);
    for (int j = 0; j < h; ++j) {
      const double th = pow((double)c.rope_theta, -(2.0 * (double)j) / (double)c.head_dim);
      const double ang = (double)(-d) * th;
      cs[2 * j] = (float)cos(ang);
      cs[2 * j + 1] = (float)sin(ang);
    }
    // staging: the moved rows, the lane's block ids, the angle table
    const size_t bytes = (size_t)n_rows * n * row_bytes;
    const size_t boff = (bytes + 255) & ~(size_t)255;
    const size_t coff = (boff + bl.size() * sizeof(int) + 255) & ~(size_t)255;
    const size_t need = coff + cs.size() * sizeof(float);
    if (a->stage_bytes < need) {
      HIP_TRY(hipStreamSynchronize(st));
      if (a->stage) HIP_TRY(hipFree(a->stage));
      a->stage = nullptr;
      a->stage_bytes = 0;
      HIP_TRY(counted_malloc((void**)&a->stage, need));
      a->stage_bytes = need;
    }
    int* dblk = (int*)(a->stage + boff);
    const float2* dcs = (const float2*)(a->stage + coff);
    HIP_TRY(hipMemcpyAsync(dblk, bl.data(), bl.size() * sizeof(int), hipMemcpyHostToDevice, st));
    HIP_TRY(hipMemcpyAsync(a->stage + coff, cs.data(), cs.size() * sizeof(float), hipMemcpyHostToDevice, st));
    for (int v = 0; v < 2; ++v) {
      char* pool = a->base + (v ? a->region_bytes : 0);
      HIP_TRY(kv_rows(a, pool, a->stage, dblk, end, n, v != 0, false, st));
      if (!v) HIP_TRY(launch_kv_rot(a->stage, (long long)n_rows * n, c.head_dim, dcs, kvb == 2, st));
      HIP_TRY(kv_rows(a, pool, a->stage, dblk, begin, n, v != 0, true, st));
    }
    HIP_TRY(hipStreamSynchronize(st));
  }
  lane_keep(a, lane, len - d);
  return CBD_OK;
}

int cbd_lane_kv_import(cbd_arena* a, int lane, int length, const void* k_src, const void* v_src, void* stream) {
  int rc = check_lane(a, lane);
  if (rc) return rc;
  if (length < 0) return fail(CBD_E_ARG, "negative length");
  if (length > a->max_seq) return fail(CBD_E_KV_FULL, "length %d exceeds max_seq %d", length, a->max_seq);
  if (length > 0 && (!k_src || !v_src)) return fail(CBD_E_ARG, "null source");
  const int need = (length + ATTN_SPLIT - 1) / ATTN_SPLIT;
  const int have = (int)a->blocks[lane].size();
  if (need - have > (int)a->free_blocks.size())
    return fail(CBD_E_KV_FULL, "importing %d positions needs %d more KV blocks, %zu are free", length, need - have,
                a->free_blocks.size());
  lane_keep(a, lane, std::min(a->len[lane], length));
  while ((int)a->blocks[lane].size() < need) {
    a->blocks[lane].push_back(a->free_blocks.back());
    a->free_blocks.pop_back();
  }
  hipStream_t st = (hipStream_t)stream;
  if (length > 0) {
    if ((rc = copy_lane(a, lane, length, (char*)k_src, true, false, st))) return rc;
    if ((rc = copy_lane(a, lane, length, (char*)v_src, true, true, st))) return rc;
  }
  HIP_TRY(hipStreamSynchronize(st));
  a->len[lane] = length;
  return CBD_OK;
}

}  // extern "C"

namespace cbd {

int report_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return fail(code, "%s", buf);
}

int workspace_rows(const cbd_model* m, int max_seq, size_t bytes) { return max_batch_for(m, max_seq, bytes); }

int arena_max_seq(const cbd_arena* a) { return a->max_seq; }

size_t arena_kv_bytes_per_token(const cbd_arena* a) {
  const cbd_config& c = a->m->c;
  return 2 * (size_t)c.n_layers * c.n_kv_heads * c.head_dim * a->m->kvb;
}

}  // namespace cbd
