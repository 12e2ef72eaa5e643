// Continuous-batching scheduler over a libkvc cache (host only).
//
// Iteration-level scheduling as "LLM推理优化实战：从KV-Cache到Continuous Batching的
// 技术演进与代码实现" §5.2 describes it: every iteration keeps the unfinished
// running requests, tops the batch up from the waiting queue, and frees a
// request's KV cache as soon as it finishes.  When the pool cannot hold an
// iteration, running sequences are preempted and recomputed later
// ("苦猿的大模型日记 · Day45" PART 05 lists waiting, preemption, dropping the cache
// and recomputing among what an engine does instead of failing); the
// allocator's all-or-nothing KVC_E_NO_BLOCKS (the out-of-blocks case of
// "大模型推理加速核心KV Cache 复用机制与内存布局优化" §三, which hands the decision to
// the scheduler) is what the plan avoids.
//
// Token accounting.  A request has a prompt of P tokens and produces up to M
// tokens.  Its K/V rows enter the cache in position order: the prompt in
// chunks of at most chunk_tokens (chunked prefill), then, after each emitted
// token, that token's row.  An iteration that brings the cache up to every
// known token (prompt plus tokens emitted so far) emits the next token; the
// request finishes when it has emitted M tokens (the last one's row is never
// written).  Preemption frees the request's blocks and requeues it at the
// front of the waiting queue; on readmission it re-prefills its prompt and
// every token it had emitted (recompute), so the K/V it writes are the same.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <deque>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "kvc_internal.h"

namespace {

struct Request {
  int64_t id;
  int32_t prompt;     // P
  int32_t max_new;    // M
  int32_t emitted = 0;
  int32_t cached = 0;  // rows in the cache (0 while waiting)
  int64_t admitted_at = -1;
};

}  // namespace

struct kvc_sched {
  kvc_cache* cache;
  kvc_sched_config cfg;
  int32_t block_size;
  std::mutex mu;
  std::deque<int64_t> waiting;          // front first
  std::vector<int64_t> running;         // admission order
  std::unordered_map<int64_t, Request> reqs;
  // the plan awaiting commit
  bool planned = false;
  std::vector<int64_t> plan_ids;
  std::vector<int32_t> plan_n;
  int64_t admissions = 0;
  kvc_sched_stats stats{};
};

namespace {

// Failures are reported through the library's per-thread message.
kvc_status sched_fail(kvc_status st, const char* what) {
  return kvc::host_fail(st, (std::string("scheduler: ") + what).c_str());
}

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

int32_t known_tokens(const Request& r) { return r.prompt + r.emitted; }

// Rows this request appends in the coming iteration (>= 1 for a running one).
int32_t rows_wanted(const Request& r, int32_t chunk) {
  return std::min(known_tokens(r) - r.cached, r.cached < r.prompt ? chunk : 1);
}

int64_t free_blocks(kvc_cache* c) {
  kvc_stats_t st;
  if (kvc_stats(c, &st) != KVC_OK) return 0;
  return st.free_blocks;
}

}  // namespace

extern "C" {

kvc_status kvc_sched_create(kvc_cache* cache, const kvc_sched_config* cfg, kvc_sched** out) {
  if (!cache || !cfg || !out) return sched_fail(KVC_E_INVALID, "cache, cfg and out must be non-NULL");
  *out = nullptr;
  if (cfg->max_batch < 1 || cfg->chunk_tokens < 1 || cfg->max_tokens < 1)
    return sched_fail(KVC_E_INVALID, "max_batch, chunk_tokens and max_tokens must be >= 1");
  kvc_stats_t st;
  kvc_status s = kvc_stats(cache, &st);
  if (s != KVC_OK) return s;
  kvc_sched* sc = new (std::nothrow) kvc_sched();
  if (!sc) return sched_fail(KVC_E_INVALID, "out of host memory");
  sc->cache = cache;
  sc->cfg = *cfg;
  sc->block_size = kvc::cache_block_size(cache);
  *out = sc;
  return KVC_OK;
}

void kvc_sched_destroy(kvc_sched* sc) { delete sc; }

kvc_status kvc_sched_submit(kvc_sched* sc, int64_t req_id, int32_t prompt_len, int32_t max_new_tokens) {
  if (!sc) return sched_fail(KVC_E_INVALID, "scheduler is NULL");
  std::lock_guard<std::mutex> lock(sc->mu);
  if (prompt_len < 1 || max_new_tokens < 1) return sched_fail(KVC_E_INVALID, "prompt_len and max_new_tokens must be >= 1");
  if (sc->reqs.count(req_id)) return sched_fail(KVC_E_SEQ_EXISTS, "request id already submitted");
  Request r;
  r.id = req_id;
  r.prompt = prompt_len;
  r.max_new = max_new_tokens;
  sc->reqs.emplace(req_id, r);
  sc->waiting.push_back(req_id);
  sc->stats.waiting = (int64_t)sc->waiting.size();
  ++sc->stats.submitted;
  return KVC_OK;
}

kvc_status kvc_sched_plan(kvc_sched* sc, int32_t capacity, int64_t* seq_ids, int32_t* n_new, int32_t* start,
                          int32_t* emits, int32_t* batch, int64_t* preempted, int32_t preempt_capacity,
                          int32_t* num_preempted) {
  if (!sc || !batch) return sched_fail(KVC_E_INVALID, "scheduler and batch must be non-NULL");
  std::lock_guard<std::mutex> lock(sc->mu);
  if (sc->planned) return sched_fail(KVC_E_INVALID, "the previous plan was not committed");
  if (capacity < sc->cfg.max_batch || !seq_ids || !n_new)
    return sched_fail(KVC_E_INVALID, "seq_ids / n_new must hold max_batch entries");
  const int32_t bs = sc->block_size;
  const int32_t chunk = sc->cfg.chunk_tokens;
  int64_t avail = free_blocks(sc->cache);
  int32_t npre = 0;
  // 1. running requests: one row for each decoding request (never deferred),
  //    then prefill chunks in admission order within the token budget.  If
  //    their blocks do not fit, the most recently admitted running request is
  //    preempted and the rows are planned again.
  std::vector<int64_t> order = sc->running;
  std::vector<int32_t> want(order.size());
  for (;;) {
    int64_t need = 0, tokens = 0;
    for (size_t i = 0; i < order.size(); ++i) {
      const Request& r = sc->reqs[order[i]];
      want[i] = r.cached < r.prompt ? 0 : rows_wanted(r, chunk);
      tokens += want[i];
    }
    for (size_t i = 0; i < order.size(); ++i) {
      const Request& r = sc->reqs[order[i]];
      if (r.cached < r.prompt) {
        want[i] = (int32_t)std::min<int64_t>(rows_wanted(r, chunk), std::max<int64_t>(0, sc->cfg.max_tokens - tokens));
        tokens += want[i];
      }
      need += blocks_for(r.cached + want[i], bs) - blocks_for(r.cached, bs);
    }
    if (need <= avail) break;
    // the oldest running request alone does not fit: the pool is too small for
    // it (preempting it would only start it over); requests preempted on the
    // way stay preempted
    if (order.size() <= 1) {
      sc->stats.running = (int64_t)sc->running.size();
      sc->stats.waiting = (int64_t)sc->waiting.size();
      if (num_preempted) *num_preempted = npre;
      return sched_fail(KVC_E_NO_BLOCKS, "the pool cannot hold the next rows of the oldest running request");
    }
    // preempt the newest running request: free its blocks, requeue it first
    const int64_t victim = order.back();
    Request& v = sc->reqs[victim];
    kvc_status st = kvc_free_seq(sc->cache, victim);
    if (st != KVC_OK) return st;
    avail = free_blocks(sc->cache);
    v.cached = 0;
    v.admitted_at = -1;
    sc->waiting.push_front(victim);
    order.pop_back();
    want.pop_back();
    sc->running.erase(std::find(sc->running.begin(), sc->running.end(), victim));
    if (preempted && npre < preempt_capacity) preempted[npre] = victim;
    ++npre;
    ++sc->stats.preemptions;
  }
  // blocks and tokens the running requests take
  int64_t need = 0, tokens = 0;
  for (size_t i = 0; i < order.size(); ++i) {
    const Request& r = sc->reqs[order[i]];
    need += blocks_for(r.cached + want[i], bs) - blocks_for(r.cached, bs);
    tokens += want[i];
  }
  avail -= need;
  // 2. admit waiting requests, front first, while the batch, the token budget
  //    and the pool allow (strict order: the first one that does not fit stops
  //    admission, so nobody is overtaken)
  while (!sc->waiting.empty() && (int32_t)order.size() < sc->cfg.max_batch && tokens < sc->cfg.max_tokens) {
    const int64_t id = sc->waiting.front();
    Request& r = sc->reqs[id];
    const int32_t w = (int32_t)std::min<int64_t>({(int64_t)chunk, (int64_t)known_tokens(r),
                                                  (int64_t)sc->cfg.max_tokens - tokens});
    const int64_t nb = blocks_for(w, bs);
    if (nb > avail) break;
    kvc_status st = kvc_add_seq(sc->cache, id, 0);
    if (st != KVC_OK) return st;
    sc->waiting.pop_front();
    r.admitted_at = sc->admissions++;
    sc->running.push_back(id);
    order.push_back(id);
    want.push_back(w);
    avail -= nb;
    tokens += w;
  }
  // drop running requests that get no rows this iteration (token budget spent)
  int32_t nb_out = 0;
  sc->plan_ids.clear();
  sc->plan_n.clear();
  for (size_t i = 0; i < order.size(); ++i) {
    if (want[i] <= 0) continue;
    const Request& r = sc->reqs[order[i]];
    seq_ids[nb_out] = order[i];
    n_new[nb_out] = want[i];
    if (start) start[nb_out] = r.cached;
    if (emits) emits[nb_out] = (r.cached + want[i] == known_tokens(r)) ? 1 : 0;
    sc->plan_ids.push_back(order[i]);
    sc->plan_n.push_back(want[i]);
    ++nb_out;
  }
  if (nb_out == 0 && !sc->running.empty())
    return sched_fail(KVC_E_NO_BLOCKS, "the pool cannot hold the next rows of even one request");
  if (nb_out == 0 && !sc->waiting.empty())
    return sched_fail(KVC_E_NO_BLOCKS, "the pool cannot hold the first chunk of the next waiting request");
  *batch = nb_out;
  if (num_preempted) *num_preempted = npre;
  sc->planned = true;
  sc->stats.running = (int64_t)sc->running.size();
  sc->stats.waiting = (int64_t)sc->waiting.size();
  return KVC_OK;
}

kvc_status kvc_sched_commit(kvc_sched* sc, int64_t* finished, int32_t capacity, int32_t* num_finished) {
  if (!sc) return sched_fail(KVC_E_INVALID, "scheduler is NULL");
  std::lock_guard<std::mutex> lock(sc->mu);
  if (!sc->planned) return sched_fail(KVC_E_INVALID, "no plan to commit");
  // the caller must have appended exactly the planned rows
  for (size_t i = 0; i < sc->plan_ids.size(); ++i) {
    const Request& r = sc->reqs[sc->plan_ids[i]];
    int32_t nblk = 0, len = 0;
    kvc_status st = kvc_get_table(sc->cache, r.id, nullptr, 0, &nblk, &len);
    if (st != KVC_OK) return st;
    if (len != r.cached + sc->plan_n[i]) return sched_fail(KVC_E_INVALID, "the planned rows were not appended");
  }
  int32_t nf = 0;
  for (size_t i = 0; i < sc->plan_ids.size(); ++i) {
    const int64_t id = sc->plan_ids[i];
    Request& r = sc->reqs[id];
    r.cached += sc->plan_n[i];
    sc->stats.tokens_scheduled += sc->plan_n[i];
    if (r.cached == known_tokens(r)) {
      ++r.emitted;
      if (r.emitted == r.max_new) {
        kvc_status st = kvc_free_seq(sc->cache, id);
        if (st != KVC_OK) return st;
        sc->running.erase(std::find(sc->running.begin(), sc->running.end(), id));
        if (finished && nf < capacity) finished[nf] = id;
        ++nf;
        ++sc->stats.finished;
        sc->reqs.erase(id);
      }
    }
  }
  if (num_finished) *num_finished = nf;
  sc->planned = false;
  ++sc->stats.iterations;
  sc->stats.running = (int64_t)sc->running.size();
  sc->stats.waiting = (int64_t)sc->waiting.size();
  return KVC_OK;
}

kvc_status kvc_sched_get_stats(const kvc_sched* csc, kvc_sched_stats* out) {
  kvc_sched* sc = const_cast<kvc_sched*>(csc);
  if (!sc || !out) return sched_fail(KVC_E_INVALID, "scheduler and out must be non-NULL");
  std::lock_guard<std::mutex> lock(sc->mu);
  *out = sc->stats;
  return KVC_OK;
}

}  // extern "C"
