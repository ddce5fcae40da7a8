/*
 * cbd — the batched decode step of a dense Llama decoder on one AMD Instinct
 * MI355X (gfx950).
 *
 * One call of cbd_decode_step_batch advances B independent sequences
 * ("lanes") by one token each.  The operation is the multi-user batched
 * decode of "MODEL-BATCHING-RESULTS — multi-user batched decode, measured"
 * (section "The lever"): one decode token per user is stacked into a [B, d]
 * panel, each of the seven projections (q, k, v, o, gate, up, down) and the
 * LM head runs once over that panel so every weight byte is read once for the
 * whole batch, and attention stays per user over that user's own KV cache and
 * length, with no mixing between users.  Its interface follows the primitive
 * of "Fat-station continuous batching" (section "The capture"): per-lane KV
 * caches, per-lane positions and one input token per lane in, logits for every
 * lane out, positions advanced.  Lanes live in a fixed arena allocated once at
 * capacity and bounded by a maximum sequence length (same page, "Components",
 * items 1 and 4); a lane is cleared for reuse by the next job and released
 * when its job completes, after which its KV usage is zero ("DGR-012",
 * section "Summary", bounded memory).
 *
 * Conventions
 *  - All functions return 0 (CBD_OK) on success or a negative CBD_E_* code;
 *    cbd_last_error() gives a message for the calling thread's last failure.
 *  - Every check runs on the host before any GPU work is enqueued, so a call
 *    that fails changes nothing (arena, positions and device memory untouched).
 *  - Device pointers are plain HIP device addresses (e.g. a torch tensor's
 *    data_ptr()).  The caller owns all device memory: weights, the arena, the
 *    workspace and the outputs.  The library borrows it and never frees it.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Steps are asynchronous on that stream; results are valid once it syncs.
 *  - One host thread drives a given model and arena at a time.
 *
 * Number formats: f32 is IEEE binary32; bf16 is the upper 16 bits of a
 * binary32 (round to nearest even when produced); Q8_0 stores a weight matrix
 * [N, K] as two planes: int8 q [N, K] and binary16 scales [N, K/32], one per
 * block of 32 consecutive elements along K, value = q * scale.
 */
#ifndef CBD_H
#define CBD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CBD_OK 0
#define CBD_E_ARG (-1)           /* bad argument: null pointer, size or config out of range */
#define CBD_E_DUP_LANE (-2)      /* the same lane appears twice in one step */
#define CBD_E_LANE_NOT_LIVE (-3) /* lane not allocated, or already evicted (a cache miss) */
#define CBD_E_POS_MISMATCH (-4)  /* positions[b] differs from the lane's KV length */
#define CBD_E_KV_FULL (-5)       /* positions[b] == max_seq: no slot left in the lane */
#define CBD_E_TOKEN (-6)         /* token id outside [0, vocab) */
#define CBD_E_NO_FREE_LANE (-7)  /* every lane of the arena is live */
#define CBD_E_HIP (-8)           /* a HIP runtime call failed */
#define CBD_E_WORKSPACE (-9)     /* workspace null or smaller than cbd_workspace_bytes() */
#define CBD_E_UNSUPPORTED (-10)  /* model shape outside what the kernels are built for */

/* Weight storage type; also fixes the activation and KV formats:
 *  CBD_F32  - f32 weights, f32 projection inputs, f32 KV.
 *  CBD_BF16 - bf16 weights, bf16 projection inputs and KV, f32 accumulation,
 *             f32 residual stream, norm statistics, softmax and logits.
 *  CBD_Q8_0 - Q8_0 weights, binary16 projection inputs, f32 KV.            */
typedef enum { CBD_F32 = 0, CBD_BF16 = 1, CBD_Q8_0 = 2 } cbd_wtype;

/* Model shape.  Requirements: n_heads % n_kv_heads == 0 and
 * n_heads / n_kv_heads <= 8; head_dim in {16, 32, 64, 128}; d_model and
 * ffn_dim multiples of 4 (f32), 8 (bf16) or 32 (Q8_0); n_heads*head_dim a
 * multiple of the same. */
typedef struct {
  int d_model, n_layers, n_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  float rms_eps;    /* RMSNorm epsilon, e.g. 1e-5 */
  float rope_theta; /* rotary base, e.g. 10000 */
  int tied_embeddings; /* nonzero: the LM head is the embedding matrix */
  int wtype;           /* cbd_wtype */
  int packed;          /* nonzero: w_qkv, w_o, w_gu, w_down and an untied lm_head are in
                          the packed tile layout of cbd_pack_matrix (CBD_BF16, d_model,
                          ffn_dim and n_heads*head_dim multiples of 32); the embedding
                          stays row-major */
} cbd_config;

/* One weight matrix [N, K], row-major, K contiguous, rows 16-byte aligned.
 * data: f32, bf16 or int8 (Q8_0) device pointer; scale: binary16 [N, K/32]
 * device pointer for Q8_0, NULL otherwise. */
typedef struct {
  const void* data;
  const void* scale;
} cbd_matrix;

/* Weights (device memory, borrowed for the model's lifetime).  The pointer
 * arrays themselves are host arrays of n_layers entries, copied at create.
 *  embed      [vocab, d]
 *  lm_head    [vocab, d] (ignored when tied_embeddings)
 *  final_norm, attn_norm[l], ffn_norm[l]  f32 [d] RMSNorm gains, 16-byte aligned
 *  w_qkv[l]   [(n_heads + 2 n_kv_heads) * head_dim, d]: query rows, key rows, value rows
 *  w_o[l]     [d, n_heads * head_dim]
 *  w_gu[l]    [2 ffn, d]: gate rows, then up rows
 *  w_down[l]  [d, ffn]                                                        */
typedef struct {
  cbd_matrix embed;
  cbd_matrix lm_head;
  const float* final_norm;
  const float* const* attn_norm;
  const float* const* ffn_norm;
  const cbd_matrix* w_qkv;
  const cbd_matrix* w_o;
  const cbd_matrix* w_gu;
  const cbd_matrix* w_down;
} cbd_weights;

typedef struct cbd_model cbd_model;
typedef struct cbd_arena cbd_arena;

/* Packed tile layout of a bf16 weight matrix.  The step reads every weight
 * byte once for all lanes ("MODEL-BATCHING-RESULTS — multi-user batched
 * decode, measured", section "The lever"); in this layout each 64-lane load
 * of the weight stream is one contiguous kilobyte that is already a matrix-
 * core operand, where row-major rows give 16 segments of 64 bytes (on
 * MI355X a plain stream of such loads reads 5.85 TB/s against 5.4; the
 * 7B gate|up projection at 64 lanes takes 46.5 us against 56.5).  The rows are
 * taken as `halves` consecutive halves of `rows` rows each (w_gu: 2, the
 * gate rows and the up rows; every other matrix 1); each half is cut into
 * T = ceil(rows / 16) row tiles (the last padded with zero rows) and K / 32
 * column steps; tile (h, i, t) is the 1024 bytes at offset
 * ((h * T + i) * (K / 32 + 8) + t) * 1024 and holds, for slot L = 0 .. 63,
 * the 8 elements of row 16 i + L % 16, columns 32 t + 8 (L / 16) .. + 7.
 * The 8 tiles after each row tile's run are zeros (unused: they keep the
 * runs the weight stream reads at once from starting 2^n kilobytes apart).
 * Returns the packed size in bytes, or 0 when the matrix has no packed form
 * (wtype other than CBD_BF16, K not a positive multiple of 32, rows or
 * halves not positive). */
size_t cbd_packed_bytes(int wtype, int rows, int K, int halves);

/* Write the packed layout of src (device, [halves * rows, K] row-major) into
 * dst (device, cbd_packed_bytes bytes, 16-byte aligned), on `stream` (a
 * hipStream_t; NULL: the default stream).  src and dst must not overlap.
 * Errors: CBD_E_ARG (null pointer), CBD_E_UNSUPPORTED (no packed form),
 * CBD_E_HIP. */
int cbd_pack_matrix(int wtype, const void* src, void* dst, int rows, int K, int halves, void* stream);

/* Library version string. */
const char* cbd_version(void);

/* Message of the calling thread's last failed call ("" if none). */
const char* cbd_last_error(void);

/* Validate the shape, copy the config and the weight pointer arrays.  No GPU
 * work happens here.  Errors: CBD_E_ARG (null or inconsistent), CBD_E_UNSUPPORTED. */
int cbd_model_create(const cbd_config* cfg, const cbd_weights* w, cbd_model** out);
void cbd_model_destroy(cbd_model* m);

/* The arena is a pool of KV blocks (paged KV): a block holds 64 positions (one
 * attention chunk) of one lane for every layer and KV head.  The pool is
 * layer-major: K [n_layers][n_blocks][n_kv_heads][64 * head_dim], then V
 * alike, in the KV format of the model's wtype, so that block j of every
 * layer belongs to the same lane and one layer's blocks are contiguous.  The
 * 64 x head_dim elements of one (layer, block, KV head) are row-major
 * [64][head_dim], except for bf16 caches whose attention runs on the matrix
 * cores (head_dim 128 with at most 4, or 64 with at most 8, query heads per KV
 * head): there they sit in the order the kernels load their matrix-core
 * operands, so the pool is opaque; cbd_lane_kv_import / _export always take
 * rows [len][head_dim].  A lane holds the blocks of its chunks, any
 * blocks of the pool in any order; a step takes a free block when a lane's new
 * slot opens a chunk (CBD_E_KV_FULL, changing nothing, if none is free), and
 * clear, evict and truncate return blocks to the pool.  Bytes of one block
 * (K and V), or 0 for an invalid config. */
size_t cbd_arena_block_bytes(const cbd_config* cfg);

/* Device bytes for every one of n_lanes lanes to reach max_seq positions at
 * once: n_lanes * ceil(max_seq / 64) blocks.  A smaller pool serves lanes of
 * mixed lengths (the blocks are shared).  Returns 0 for invalid arguments. */
size_t cbd_arena_bytes(const cbd_config* cfg, int n_lanes, int max_seq);

/* Create a lane arena of n_lanes lanes (each at most max_seq positions) over
 * caller-owned device memory dev_mem of dev_bytes bytes, 256-byte aligned:
 * floor(dev_bytes / cbd_arena_block_bytes) blocks, at least one.  All lanes
 * start free and all blocks unused.  Errors: CBD_E_ARG. */
int cbd_arena_create(cbd_model* m, int n_lanes, int max_seq, void* dev_mem, size_t dev_bytes,
                     cbd_arena** out);
void cbd_arena_destroy(cbd_arena* a);

/* Reserve the lowest free lane; its length is 0.  Errors: CBD_E_NO_FREE_LANE. */
int cbd_lane_alloc(cbd_arena* a, int* lane);
/* Length := 0, reservation kept (reuse by the next job).  Errors: CBD_E_ARG,
 * CBD_E_LANE_NOT_LIVE. */
int cbd_lane_clear(cbd_arena* a, int lane);
/* Release the lane: its usage drops to zero, and stepping it is an error
 * until it is allocated again.  Errors: CBD_E_ARG, CBD_E_LANE_NOT_LIVE. */
int cbd_lane_evict(cbd_arena* a, int lane);
/* KV length of a live lane (>= 0), or a negative error code. */
int cbd_lane_length(const cbd_arena* a, int lane);
/* Sum over live lanes of length * KV bytes per token (all layers, K and V). */
size_t cbd_arena_used_bytes(const cbd_arena* a);
/* Number of live lanes. */
int cbd_arena_live_lanes(const cbd_arena* a);
/* Blocks of the pool, and of them the free ones (or -1 for a null arena). */
int cbd_arena_n_blocks(const cbd_arena* a);
int cbd_arena_free_blocks(const cbd_arena* a);

/* Device bytes of the workspace a step of up to max_batch lanes of an arena
 * of max_seq positions needs (activations, split partials, attention partials,
 * per-step metadata).  Returns 0 for invalid arguments. */
size_t cbd_workspace_bytes(const cbd_model* m, int max_batch, int max_seq);

/* One decode step over B lanes (1 <= B <= the max_batch the workspace was
 * sized for).  Host inputs: lanes[B] (distinct live lanes), positions[B]
 * (in/out: must equal each lane's KV length on entry; each is incremented on
 * success), tokens[B] (ids in [0, vocab)).  Device outputs: logits [B, vocab]
 * f32 (required) and argmax [B] int32 (optional, NULL to skip; lowest index
 * wins ties).  Lane b's token is embedded, written into the lane's KV slot
 * positions[b] of every layer, attends over slots [0, positions[b]] of its own
 * lane only, and its logits land in row b.  workspace: device memory of
 * workspace_bytes >= cbd_workspace_bytes(m, B, arena max_seq), used by one
 * model at a time; nothing in it persists between steps (each step writes
 * what it reads).
 * Errors: CBD_E_ARG, CBD_E_DUP_LANE, CBD_E_LANE_NOT_LIVE, CBD_E_POS_MISMATCH,
 * CBD_E_KV_FULL, CBD_E_TOKEN, CBD_E_WORKSPACE, CBD_E_HIP. */
int cbd_decode_step_batch(cbd_model* m, cbd_arena* a, int B, const int32_t* lanes, int32_t* positions,
                          const int32_t* tokens, float* logits, int32_t* argmax, void* workspace,
                          size_t workspace_bytes, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same decode step with
 * no workspace argument and no allocation of any kind.  Its workspace is a
 * static device array of cbd_noalloc_scratch_bytes() (64 MiB), one copy per
 * device, which the library holds on every device it runs on until the
 * process ends; its device address is looked up once per device.  The step's
 * pinned staging must already be sized (cbd_arena_create does it on a
 * device), and graph replay does not apply.  Results are bitwise those of
 * cbd_decode_step_batch.  Every call on a device shares that device's scratch
 * and it keeps the last call's contents (nothing in it needs to start at
 * zero: each step writes what it reads); calls that overlap on one device
 * (other streams or threads) race and must not be issued.  Errors: as
 * cbd_decode_step_batch; CBD_E_WORKSPACE when B lanes at the arena's max_seq
 * need more than the scratch holds (the Mistral-7B shape: 64 lanes at 4097
 * positions fit). */
int cbd_decode_step_batch_noalloc(cbd_model* m, cbd_arena* a, int B, const int32_t* lanes, int32_t* positions,
                                  const int32_t* tokens, float* logits, int32_t* argmax, void* stream);
/* Bytes of that static scratch on each device. */
size_t cbd_noalloc_scratch_bytes(void);

/* The same step for one lane (B = 1): position in/out, logits [vocab]. */
int cbd_decode_step(cbd_model* m, cbd_arena* a, int lane, int32_t* position, int32_t token, float* logits,
                    int32_t* argmax, void* workspace, size_t workspace_bytes, void* stream);

/* Batched chunked prefill: several tokens for each of n_seq lanes in one
 * call.  The prompt of "Fat-station continuous batching" (section "The
 * capture") is prefilled in chunks into the lane's cache at consecutive
 * positions; "parallel-slots.md" (section "Reuse: batched PREFILL already
 * exists") batches prefill over rows under a causal mask that keeps each
 * row's result independent of the others.  Here lane i takes counts[i] >= 1
 * tokens, tokens[off_i .. off_i + counts[i]) with off_i = counts[0] + ... +
 * counts[i-1], at positions positions[i] .. positions[i] + counts[i] - 1:
 * each token is embedded, its K/V written at its slot, and it attends over
 * slots [0, its position] of its own lane (the tokens before it in the same
 * call included).  The result equals feeding the lane's tokens one decode step
 * at a time, bit for bit (logits and KV).  Host inputs: lanes[n_seq] (distinct
 * live lanes), positions[n_seq] (in/out: each lane's KV length on entry,
 * advanced by counts[i] on success), counts[n_seq], tokens[sum counts].
 * Device outputs: logits [n_seq, vocab] f32 of each lane's last token
 * (required) and argmax [n_seq] int32 (optional, NULL to skip).  The workspace
 * must hold sum(counts) rows: workspace_bytes >= cbd_workspace_bytes(m,
 * sum(counts), arena max_seq).  Errors: as cbd_decode_step_batch, plus
 * CBD_E_ARG for a count below 1 and CBD_E_KV_FULL for positions[i] +
 * counts[i] > max_seq or too few free blocks; a failed call changes nothing. */
int cbd_prefill_batch(cbd_model* m, cbd_arena* a, int n_seq, const int32_t* lanes, int32_t* positions,
                      const int32_t* counts, const int32_t* tokens, float* logits, int32_t* argmax, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Copy a live lane's KV out: k_dst, v_dst (host or device, hipMemcpy default
 * kind) receive [n_layers][n_kv_heads][length][head_dim] in the KV format.
 * Synchronous with respect to `stream`.  Import and export move the rows
 * through a device staging buffer of one lane's K (or V) that the arena
 * allocates on first use, grows as needed and frees in cbd_arena_destroy (not a
 * step-path call: the step allocates nothing).  Errors: CBD_E_ARG,
 * CBD_E_LANE_NOT_LIVE, CBD_E_HIP. */
int cbd_lane_kv_export(cbd_arena* a, int lane, void* k_dst, void* v_dst, void* stream);

/* Prefix reuse: live lane dst takes the first n positions (0 <= n <= the
 * length of live lane src) of src's cache, its own content dropped, and its
 * length becomes n; src is unchanged.  Each user of "MODEL-BATCHING-RESULTS —
 * multi-user batched decode, measured" (section "Why in-kernel batching, not
 * vLLM") keeps a cache of its own that can be cloned for prefix reuse while
 * decode steps are batched.  Keys are stored rotated at their own positions,
 * so a prefix at the same positions is a plain copy: dst takes ceil(n / 64)
 * blocks of the pool, copied by one kernel on `stream`; synchronous with
 * respect to `stream` (the block lists go through the arena's staging buffer,
 * as for import and export).  Errors: CBD_E_ARG (same lane, n out of range),
 * CBD_E_LANE_NOT_LIVE, CBD_E_KV_FULL (too few free blocks; nothing changes),
 * CBD_E_HIP. */
int cbd_lane_clone(cbd_arena* a, int src, int dst, int n, void* stream);

/* Span eviction: drop positions [begin, end) of live lane `lane` (0 <= begin
 * <= end <= its length).  The per-user Evict of "MODEL-BATCHING-RESULTS —
 * multi-user batched decode, measured" (section "Why in-kernel batching, not
 * vLLM") quarantines a poisoned span of a user's cache while decode steps
 * stay batched.  Entries after the span move down by d = end - begin, so the
 * lane's positions stay contiguous and its length drops by d; keys are stored
 * rotated at their positions, so each moved key is rotated by the rotary angle
 * of -d positions (theta^(-2j/hd) in double, cos and sin rounded to f32, each
 * product and sum rounded to f32, then to the KV format); values move
 * unchanged; blocks past the new length return to the pool.  Synchronous with
 * respect to `stream` (it moves the entries through the arena's staging
 * buffer).  Errors: CBD_E_ARG (span out of range), CBD_E_LANE_NOT_LIVE,
 * CBD_E_HIP. */
int cbd_lane_evict_span(cbd_arena* a, int lane, int begin, int end, void* stream);

/* Load a live lane's KV from k_src, v_src laid out as in export, with
 * `length` positions (<= max_seq), and set its length (taking or returning
 * blocks).  Keys are taken as already rotated.  Synchronous with respect to
 * `stream`.  Errors: CBD_E_ARG, CBD_E_LANE_NOT_LIVE, CBD_E_KV_FULL (too few free
 * blocks or length > max_seq; nothing changes), CBD_E_HIP. */
int cbd_lane_kv_import(cbd_arena* a, int lane, int length, const void* k_src, const void* v_src, void* stream);

/* Keep only the first `length` positions of a live lane (0 <= length <= its
 * current length); later slots become free and are rewritten by the next
 * steps, and blocks past the kept positions return to the pool.  Host
 * bookkeeping only, no GPU work.  Lets a caller roll a lane back
 * (e.g. replay the same step).  Errors: CBD_E_ARG, CBD_E_LANE_NOT_LIVE. */
int cbd_lane_truncate(cbd_arena* a, int lane, int length);

/* Per-kernel timing for measurement.  While enabled, every step brackets each
 * kernel launch with HIP events on the step's stream and attributes the
 * elapsed GPU time to a kernel class (see cbd_profile_class_name).  The event
 * records add small gaps between kernels, so time the throughput of a step
 * with profiling disabled.  cbd_profile_read synchronizes on the recorded
 * events and returns the accumulated milliseconds and launch count of one
 * class since the last reset.  Errors: CBD_E_ARG, CBD_E_HIP. */
int cbd_profile_enable(cbd_model* m, int enable);
int cbd_profile_reset(cbd_model* m);
int cbd_profile_read(cbd_model* m, int cls, double* total_ms, long long* launches);
/* Number of kernel classes, and the name of class `cls` (NULL if out of range). */
int cbd_profile_classes(void);
const char* cbd_profile_class_name(int cls);

/* Device and pinned host allocations this library has made so far, all models
 * and arenas together (a test hook).  A decode step makes none: its staging is
 * sized when the arena is created and its workspace is the caller's.  Arena
 * creation, KV import/export, clone, span eviction, a prefill call with more
 * rows than staged for, and graph capture may allocate.  Never fails. */
long long cbd_debug_alloc_count(void);

/* Step launch mode of this model: 0 (default) = plain kernel launches; 1 =
 * each decode step's kernel sequence is captured once per (B, workspace,
 * arena, outputs) into a HIP graph and replayed on the caller's stream (for
 * callers whose host thread cannot keep up with plain launches).  Both run the
 * same kernels with the same arguments, so results are bitwise identical.
 * While profiling is enabled, and for prefill, steps launch plainly.
 * Errors: CBD_E_ARG. */
int cbd_set_graph_replay(cbd_model* m, int enable);

/* Projection kernel family for steps of this model: 0 = automatic by batch
 * width and projection (wide panels from 4 lanes for QKV and the LM head, 8
 * for gate|up, 24 for the output projection, always for a reduction longer
 * than 4096; split-K tiles below; for bf16 weights, dense tiles from 256 rows
 * for gate|up, the head and the down projection, and for QKV and O once
 * whole-K dense tiles fill the chip), 1 = weight-streaming split-K tiles at
 * every width, 2 = wide panels (the activation panel staged in on-chip
 * memory) at every width, 3 = dense tiles (both operands staged in on-chip
 * memory; bf16 weights with K a multiple of 128, else wide panels) at every
 * width.  Every family computes each output with the same chunked reduction,
 * so the choice changes speed only, never a bit of the result.
 * Errors: CBD_E_ARG. */
int cbd_set_variant(cbd_model* m, int variant);

/* ---- Continuous-batching scheduler (host policy over the step) ----
 *
 * The node-local scheduler of "DGR-012" (section "Summary"): sessions are
 * admitted against weight, KV, scratch and queue budgets, with an explicit
 * reason when refused; every tick runs decode first (each decoding session
 * contributes its next token to one batched step) and then bounded prefill of
 * waiting sessions; finished sessions release their KV, so the total returns
 * to zero.  Tick rules:
 *   1. every decoding session (up to max_batch, least recently decoded
 *      first) decodes one token; its KV grows by one position;
 *   2. a session that has produced max_new tokens is released at the end of
 *      the tick (its lane evicted, its slot free from the next tick);
 *   3. if slots were free at the start of the tick, waiting sessions are
 *      prefilled in arrival order into at most that many slots, while their
 *      prompts fit max_prefill_tokens_per_tick (the first always does) and
 *      the KV reserved by active sessions plus theirs (prompt + max_new
 *      positions each) fits the KV budget; a prefill yields the session's
 *      first token;
 *   4. telemetry: KV bytes (positions held x kv_bytes_per_token) are taken
 *      after the releases; occupancy is sessions per decode step, averaged
 *      over ticks that decode.
 * The engine is either the decode path of a model and arena
 * (cbd_sched_create_device) or caller-supplied functions (cbd_sched_create).
 * Not thread-safe: one caller drives a scheduler. */
typedef struct cbd_sched cbd_sched;

#define CBD_SCHED_QUEUED 0             /* admitted: waits for a slot */
#define CBD_SCHED_REJECT_KV 1          /* prompt + max_new positions exceed the KV budget on their own,
                                          or (device engine) prompt + max_new - 1 exceed the arena's max_seq */
#define CBD_SCHED_REJECT_SCRATCH 2     /* one session's scratch exceeds the scratch envelope, or (device
                                          engine) the prompt has more tokens than the workspace has rows */
#define CBD_SCHED_REJECT_DUPLICATE 3   /* the job id is already known */
#define CBD_SCHED_REJECT_QUEUE_FULL 4  /* max_queue sessions are waiting (backpressure) */

typedef struct cbd_sched_budget {
  size_t weight_bytes;             /* resident weights (reported only) */
  size_t kv_budget_bytes;          /* KV all sessions may hold at once */
  size_t kv_bytes_per_token;       /* KV of one position of one session (> 0) */
  size_t scratch_per_session;      /* activation bytes of one active session */
  size_t scratch_budget_bytes;     /* activation envelope */
  int max_active;                  /* active sessions (slots, lanes) */
  int max_queue;                   /* waiting sessions */
  int max_batch;                   /* sessions per decode step */
  int max_prefill_tokens_per_tick; /* prompt tokens prefilled per tick (one session always may) */
} cbd_sched_budget;

/* Caller-supplied engine.  prefill: n sessions' prompts (tokens concatenated,
 * counts[i] each) into the given lanes at positions[i] (advanced in place);
 * next[i] = the session's next token.  decode: one token per lane, the same
 * contract as cbd_decode_step_batch, next[b] = the next token.  lane_alloc /
 * lane_evict: reserve and release a lane.  Each returns 0 or a negative
 * error, which the scheduler returns unchanged. */
typedef struct cbd_sched_engine {
  void* ctx;
  int (*prefill)(void* ctx, int n, const int32_t* lanes, int32_t* positions, const int32_t* counts,
                 const int32_t* tokens, int32_t* next);
  int (*decode)(void* ctx, int B, const int32_t* lanes, int32_t* positions, const int32_t* tokens,
                int32_t* next);
  int (*lane_alloc)(void* ctx, int32_t* lane);
  int (*lane_evict)(void* ctx, int32_t lane);
} cbd_sched_engine;

typedef struct cbd_sched_telemetry {
  long long ticks, decode_ticks;
  int active, queued, finished, effective_active_cap;
  int occupancy_last, occupancy_max;
  double occupancy_avg;
  size_t kv_bytes, kv_peak_bytes, kv_budget_bytes;
  size_t scratch_bytes, scratch_budget_bytes, weight_bytes;
  long long prefill_tokens, decode_tokens;
  long long rejected, rejected_kv, rejected_scratch, rejected_duplicate, rejected_queue_full;
} cbd_sched_telemetry;

/* A scheduler over caller-supplied engine functions (copied).  The
 * effective active cap is min(max_active, scratch_budget_bytes /
 * scratch_per_session).  Errors: CBD_E_ARG (null, kv_bytes_per_token 0,
 * max_active, max_queue, max_batch or max_prefill_tokens_per_tick below 1). */
int cbd_sched_create(const cbd_sched_budget* budget, const cbd_sched_engine* engine, cbd_sched** out);

/* A scheduler whose engine is the decode path: cbd_prefill_batch and
 * cbd_decode_step_batch on (m, a) with the caller's device workspace (sized for
 * the most rows a tick runs: the larger of max_batch and the prefill tokens
 * of one tick), logits [rows, vocab] and argmax [rows] buffers and stream;
 * greedy tokens are copied to the host after each call.  budget's
 * kv_bytes_per_token is replaced by the arena's (K and V of every layer).
 * The workspace's rows also bound every call: a decode step takes at most that
 * many sessions, a prefill call at most that many prompt tokens, and a prompt
 * longer than that is refused at submission (CBD_SCHED_REJECT_SCRATCH), as is
 * a session that would outgrow the arena's max_seq (CBD_SCHED_REJECT_KV).
 * Errors: as cbd_sched_create. */
int cbd_sched_create_device(const cbd_sched_budget* budget, cbd_model* m, cbd_arena* a, void* workspace,
                            size_t workspace_bytes, float* logits, int32_t* argmax, void* stream, cbd_sched** out);
void cbd_sched_destroy(cbd_sched* s);

/* Submit a job: prompt[n_prompt] (n_prompt >= 1, copied), max_new >= 1 tokens
 * to generate.  *decision = CBD_SCHED_QUEUED or a CBD_SCHED_REJECT_* reason
 * (a refusal is not an error).  Errors: CBD_E_ARG. */
int cbd_sched_submit(cbd_sched* s, long long job_id, const int32_t* prompt, int n_prompt, int max_new,
                     int* decision);

/* One tick (rules above).  *worked = 0 when there was nothing to do.
 * Errors: the engine's, unchanged.  If the prefill fails, its sessions wait
 * again at the head of the queue (their lanes released), and sessions the
 * tick's decode finished are still released. */
int cbd_sched_tick(cbd_sched* s, int* worked);

/* Ticks until no session is active or waiting; CBD_E_ARG if that takes more
 * than max_ticks (a guard against misconfiguration). */
int cbd_sched_run(cbd_sched* s, long long max_ticks);

int cbd_sched_get_telemetry(const cbd_sched* s, cbd_sched_telemetry* t);

/* Tokens generated so far for a job (up to cap into out), their count in *n,
 * and *done = 1 once the job has finished.  Errors: CBD_E_ARG (unknown job). */
int cbd_sched_job_tokens(const cbd_sched* s, long long job_id, int32_t* out, int cap, int* n, int* done);

#ifdef __cplusplus
}
#endif

#endif /* CBD_H */
