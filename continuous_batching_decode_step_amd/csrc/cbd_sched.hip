// Continuous-batching scheduler: the host policy of "DGR-012" (section
// "Summary": bounded admission, decode first then bounded prefill, KV released
// on completion, telemetry) over an engine, which is either the decode path of
// this library (cbd_prefill_batch / cbd_decode_step_batch on a model and
// arena) or caller-supplied functions.  Host code only.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <deque>
#include <unordered_map>
#include <vector>

#include "../../include/cbd.h"
#include "cbd_internal.h"

using namespace cbd;

namespace {

enum { WAITING = 0, DECODING = 1, FINISHED = 2 };

struct Session {
  long long id = 0;
  long long seq = 0;            // arrival order
  std::vector<int32_t> prompt;
  int max_new = 0;
  std::vector<int32_t> out;     // generated tokens
  int32_t lane = -1;
  int32_t pos = 0;              // KV positions held
  long long last_decoded = -1;  // tick of the last decode (or prefill)
  int state = WAITING;
  size_t reserve = 0;           // KV bytes reserved while active: (prompt + max_new) positions
};

// The decode path as an engine: greedy tokens come back through a host copy
// of the argmax buffer after each call.
struct DeviceEngine {
  cbd_model* m;
  cbd_arena* a;
  void* ws;
  size_t ws_bytes;
  float* logits;
  int32_t* argmax;
  hipStream_t st;
};

int copy_tokens(DeviceEngine* e, int n, int32_t* next) {
  hipError_t h = hipMemcpyAsync(next, e->argmax, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, e->st);
  if (h == hipSuccess) h = hipStreamSynchronize(e->st);
  return h == hipSuccess ? CBD_OK : report_error(CBD_E_HIP, hipGetErrorString(h));
}

int dev_prefill(void* ctx, int n, const int32_t* lanes, int32_t* positions, const int32_t* counts,
                const int32_t* tokens, int32_t* next) {
  DeviceEngine* e = (DeviceEngine*)ctx;
  const int rc = cbd_prefill_batch(e->m, e->a, n, lanes, positions, counts, tokens, e->logits, e->argmax, e->ws,
                                   e->ws_bytes, e->st);
  return rc ? rc : copy_tokens(e, n, next);
}

int dev_decode(void* ctx, int B, const int32_t* lanes, int32_t* positions, const int32_t* tokens, int32_t* next) {
  DeviceEngine* e = (DeviceEngine*)ctx;
  const int rc = cbd_decode_step_batch(e->m, e->a, B, lanes, positions, tokens, e->logits, e->argmax, e->ws,
                                       e->ws_bytes, e->st);
  return rc ? rc : copy_tokens(e, B, next);
}

int dev_lane_alloc(void* ctx, int32_t* lane) {
  int l = -1;
  const int rc = cbd_lane_alloc(((DeviceEngine*)ctx)->a, &l);
  *lane = l;
  return rc;
}

int dev_lane_evict(void* ctx, int32_t lane) { return cbd_lane_evict(((DeviceEngine*)ctx)->a, lane); }

}  // namespace

struct cbd_sched {
  cbd_sched_budget b{};
  cbd_sched_engine e{};
  DeviceEngine* dev = nullptr;
  int cap = 0;                 // effective active cap
  // device engine: rows its workspace holds per call (prompt tokens of one
  // prefill call, lanes of one decode step) and positions per lane; 0 = no limit
  int row_cap = 0, max_seq = 0;
  std::vector<Session> sessions;
  std::unordered_map<long long, size_t> index;
  std::deque<size_t> queue;    // waiting sessions, arrival order
  std::vector<size_t> active;  // decoding sessions
  size_t reserved = 0;         // KV bytes reserved by active sessions
  long long ticks = 0, decode_ticks = 0, occ_sum = 0, prefill_tokens = 0, decode_tokens = 0;
  int occ_last = 0, occ_max = 0, finished = 0;
  size_t kv_bytes = 0, kv_peak = 0;
  long long rej_kv = 0, rej_scratch = 0, rej_dup = 0, rej_queue = 0;
};

namespace {

// Release the finished sessions of this tick: lanes evicted, slots and KV
// reservations returned.
int release(cbd_sched* s, const std::vector<size_t>& done) {
  for (size_t i : done) {
    Session& x = s->sessions[i];
    const int rc = s->e.lane_evict(s->e.ctx, x.lane);
    if (rc) return rc;
    x.state = FINISHED;
    x.lane = -1;
    x.pos = 0;
    s->reserved -= x.reserve;
    s->active.erase(std::find(s->active.begin(), s->active.end(), i));
    ++s->finished;
  }
  return CBD_OK;
}

}  // namespace

extern "C" {

int cbd_sched_create(const cbd_sched_budget* budget, const cbd_sched_engine* engine, cbd_sched** out) {
  if (!budget || !engine || !out) return report_error(CBD_E_ARG, "null argument");
  if (!engine->prefill || !engine->decode || !engine->lane_alloc || !engine->lane_evict)
    return report_error(CBD_E_ARG, "engine function missing");
  const cbd_sched_budget& b = *budget;
  if (b.kv_bytes_per_token == 0 || b.max_active < 1 || b.max_queue < 1 || b.max_batch < 1 ||
      b.max_prefill_tokens_per_tick < 1)
    return report_error(CBD_E_ARG, "budget: kv_bytes_per_token, max_active, max_queue, max_batch and "
                                   "max_prefill_tokens_per_tick must be positive");
  cbd_sched* s = new cbd_sched();
  s->b = b;
  s->e = *engine;
  s->cap = b.max_active;
  if (b.scratch_per_session > 0)
    s->cap = (int)std::min<size_t>((size_t)b.max_active, b.scratch_budget_bytes / b.scratch_per_session);
  *out = s;
  return CBD_OK;
}

int cbd_sched_create_device(const cbd_sched_budget* budget, cbd_model* m, cbd_arena* a, void* workspace,
                            size_t workspace_bytes, float* logits, int32_t* argmax, void* stream, cbd_sched** out) {
  if (!budget || !m || !a || !workspace || !logits || !argmax || !out) return report_error(CBD_E_ARG, "null argument");
  DeviceEngine* d = new DeviceEngine{m, a, workspace, workspace_bytes, logits, argmax, (hipStream_t)stream};
  cbd_sched_budget b = *budget;
  b.kv_bytes_per_token = arena_kv_bytes_per_token(a);
  const cbd_sched_engine e{d, dev_prefill, dev_decode, dev_lane_alloc, dev_lane_evict};
  const int rc = cbd_sched_create(&b, &e, out);
  if (rc) {
    delete d;
    return rc;
  }
  (*out)->dev = d;
  (*out)->max_seq = arena_max_seq(a);
  (*out)->row_cap = workspace_rows(m, arena_max_seq(a), workspace_bytes);
  return CBD_OK;
}

void cbd_sched_destroy(cbd_sched* s) {
  if (!s) return;
  delete s->dev;
  delete s;
}

int cbd_sched_submit(cbd_sched* s, long long job_id, const int32_t* prompt, int n_prompt, int max_new,
                     int* decision) {
  if (!s || !prompt || !decision) return report_error(CBD_E_ARG, "null argument");
  if (n_prompt < 1 || max_new < 1) return report_error(CBD_E_ARG, "n_prompt = %d, max_new = %d", n_prompt, max_new);
  const cbd_sched_budget& b = s->b;
  const size_t need = ((size_t)n_prompt + (size_t)max_new) * b.kv_bytes_per_token;
  // A session ends holding n_prompt + max_new - 1 positions (its last token is
  // not fed back); its prompt is prefilled in one call.
  const bool too_long = s->max_seq > 0 && (long long)n_prompt + max_new - 1 > s->max_seq;
  const bool too_wide = s->row_cap > 0 && n_prompt > s->row_cap;
  if (s->index.count(job_id)) {
    ++s->rej_dup;
    *decision = CBD_SCHED_REJECT_DUPLICATE;
  } else if (need > b.kv_budget_bytes || too_long) {
    ++s->rej_kv;
    *decision = CBD_SCHED_REJECT_KV;
  } else if (s->cap < 1 || too_wide) {
    ++s->rej_scratch;
    *decision = CBD_SCHED_REJECT_SCRATCH;
  } else if ((int)s->queue.size() >= b.max_queue) {
    ++s->rej_queue;
    *decision = CBD_SCHED_REJECT_QUEUE_FULL;
  } else {
    Session x;
    x.id = job_id;
    x.seq = (long long)s->sessions.size();
    x.prompt.assign(prompt, prompt + n_prompt);
    x.max_new = max_new;
    x.reserve = need;
    s->index[job_id] = s->sessions.size();
    s->queue.push_back(s->sessions.size());
    s->sessions.push_back(std::move(x));
    *decision = CBD_SCHED_QUEUED;
  }
  return CBD_OK;
}

int cbd_sched_tick(cbd_sched* s, int* worked) {
  if (!s) return report_error(CBD_E_ARG, "null scheduler");
  const cbd_sched_budget& b = s->b;
  const int free_slots = s->cap - (int)s->active.size();  // slots free at the start of the tick
  bool work = false;
  std::vector<size_t> done;

  // 1. decode first: every decoding session, least recently decoded first,
  //    up to max_batch, one token each
  std::vector<size_t> dec(s->active);
  std::stable_sort(dec.begin(), dec.end(), [&](size_t x, size_t y) {
    const Session &p = s->sessions[x], &q = s->sessions[y];
    return p.last_decoded != q.last_decoded ? p.last_decoded < q.last_decoded : p.seq < q.seq;
  });
  const int max_b = s->row_cap > 0 ? std::min(b.max_batch, s->row_cap) : b.max_batch;
  if ((int)dec.size() > max_b) dec.resize(max_b);
  if (!dec.empty()) {
    const int B = (int)dec.size();
    std::vector<int32_t> lanes(B), pos(B), toks(B), next(B);
    for (int i = 0; i < B; ++i) {
      const Session& x = s->sessions[dec[i]];
      lanes[i] = x.lane;
      pos[i] = x.pos;
      toks[i] = x.out.back();
    }
    const int rc = s->e.decode(s->e.ctx, B, lanes.data(), pos.data(), toks.data(), next.data());
    if (rc) return rc;
    for (int i = 0; i < B; ++i) {
      Session& x = s->sessions[dec[i]];
      x.pos = pos[i];
      x.out.push_back(next[i]);
      x.last_decoded = s->ticks;
      if ((int)x.out.size() >= x.max_new) done.push_back(dec[i]);
    }
    ++s->decode_ticks;
    s->occ_sum += B;
    s->occ_last = B;
    s->occ_max = std::max(s->occ_max, B);
    s->decode_tokens += B;
    work = true;
  }

  // 2. then bounded prefill into the slots that were free at the start
  std::vector<size_t> pick;
  int used = 0;
  size_t reserved = s->reserved;
  while (!s->queue.empty() && (int)pick.size() < free_slots) {
    const Session& x = s->sessions[s->queue.front()];
    const int np = (int)x.prompt.size();
    if (!pick.empty() && used + np > b.max_prefill_tokens_per_tick) break;
    if (s->row_cap > 0 && used + np > s->row_cap) break;  // one prefill call's rows
    if (reserved + x.reserve > b.kv_budget_bytes) break;  // waits, in order, for KV to return
    reserved += x.reserve;
    used += np;
    pick.push_back(s->queue.front());
    s->queue.pop_front();
  }
  if (!pick.empty()) {
    const int n = (int)pick.size();
    std::vector<int32_t> lanes(n, -1), pos(n, 0), counts(n), toks, next(n);
    int rc = CBD_OK;
    for (int i = 0; i < n && !rc; ++i) rc = s->e.lane_alloc(s->e.ctx, &lanes[i]);
    if (!rc) {
      for (int i = 0; i < n; ++i) {
        const Session& x = s->sessions[pick[i]];
        counts[i] = (int32_t)x.prompt.size();
        toks.insert(toks.end(), x.prompt.begin(), x.prompt.end());
      }
      rc = s->e.prefill(s->e.ctx, n, lanes.data(), pos.data(), counts.data(), toks.data(), next.data());
    }
    if (rc) {  // the picked sessions wait again, at the head of the queue, and their lanes return
      for (int i = 0; i < n; ++i)
        if (lanes[i] >= 0) (void)s->e.lane_evict(s->e.ctx, lanes[i]);
      for (int i = n - 1; i >= 0; --i) s->queue.push_front(pick[i]);
      // sessions this tick's decode finished still release their lanes
      (void)release(s, done);
      if (work) ++s->ticks;
      if (worked) *worked = work ? 1 : 0;
      return rc;
    }
    s->reserved = reserved;
    for (int i = 0; i < n; ++i) {
      Session& x = s->sessions[pick[i]];
      x.lane = lanes[i];
      x.pos = pos[i];
      x.out.push_back(next[i]);
      x.state = DECODING;
      x.last_decoded = s->ticks;
      s->active.push_back(pick[i]);
      if (x.max_new == 1) done.push_back(pick[i]);
    }
    s->prefill_tokens += used;
    work = true;
  }

  // 3. finished sessions release their KV at the end of the tick
  const int rc = release(s, done);
  if (rc) return rc;

  // 4. KV held after the releases
  size_t kv = 0;
  for (size_t i : s->active) kv += (size_t)s->sessions[i].pos * b.kv_bytes_per_token;
  s->kv_bytes = kv;
  s->kv_peak = std::max(s->kv_peak, kv);
  if (work) ++s->ticks;
  if (worked) *worked = work ? 1 : 0;
  return CBD_OK;
}

int cbd_sched_run(cbd_sched* s, long long max_ticks) {
  if (!s) return report_error(CBD_E_ARG, "null scheduler");
  long long n = 0;
  while (!s->active.empty() || !s->queue.empty()) {
    if (n++ >= max_ticks) return report_error(CBD_E_ARG, "sessions remain after max_ticks ticks");
    int worked = 0;
    const int rc = cbd_sched_tick(s, &worked);
    if (rc) return rc;
    if (!worked) return report_error(CBD_E_ARG, "no session can make progress");
  }
  return CBD_OK;
}

int cbd_sched_get_telemetry(const cbd_sched* s, cbd_sched_telemetry* t) {
  if (!s || !t) return report_error(CBD_E_ARG, "null argument");
  cbd_sched_telemetry r{};
  r.ticks = s->ticks;
  r.decode_ticks = s->decode_ticks;
  r.active = (int)s->active.size();
  r.queued = (int)s->queue.size();
  r.finished = s->finished;
  r.effective_active_cap = s->cap;
  r.occupancy_last = s->occ_last;
  r.occupancy_max = s->occ_max;
  r.occupancy_avg = s->decode_ticks ? (double)s->occ_sum / (double)s->decode_ticks : 0.0;
  r.kv_bytes = s->kv_bytes;
  r.kv_peak_bytes = s->kv_peak;
  r.kv_budget_bytes = s->b.kv_budget_bytes;
  r.scratch_bytes = s->active.size() * s->b.scratch_per_session;
  r.scratch_budget_bytes = s->b.scratch_budget_bytes;
  r.weight_bytes = s->b.weight_bytes;
  r.prefill_tokens = s->prefill_tokens;
  r.decode_tokens = s->decode_tokens;
  r.rejected_kv = s->rej_kv;
  r.rejected_scratch = s->rej_scratch;
  r.rejected_duplicate = s->rej_dup;
  r.rejected_queue_full = s->rej_queue;
  r.rejected = s->rej_kv + s->rej_scratch + s->rej_dup + s->rej_queue;
  *t = r;
  return CBD_OK;
}

int cbd_sched_job_tokens(const cbd_sched* s, long long job_id, int32_t* out, int cap, int* n, int* done) {
  if (!s || !n || !done || (cap > 0 && !out)) return report_error(CBD_E_ARG, "null argument");
  const auto it = s->index.find(job_id);
  if (it == s->index.end()) return report_error(CBD_E_ARG, "unknown job %lld", job_id);
  const Session& x = s->sessions[it->second];
  const int m = std::min<int>(cap, (int)x.out.size());
  for (int i = 0; i < m; ++i) out[i] = x.out[i];
  *n = (int)x.out.size();
  *done = x.state == FINISHED ? 1 : 0;
  return CBD_OK;
}

}  // extern "C"
