// Continuous-batching scheduler (include/pa_sched.h) over the host block
// manager: four phases per step, look-ahead admission with a blocking
// fallback, lifetime reservation.
#include "pa_sched.h"

#include <algorithm>
#include <climits>
#include <deque>
#include <new>
#include <vector>

namespace {

struct Req {
  int32_t prompt = 0, want = 0;   // P, N
  int32_t tok0 = -1;              // first of its prompt tokens in the token store (-1: none)
  int32_t first_rows = 0;         // rows of its first step: P minus the cached prefix
  int32_t sid = -1;
  int32_t generated = 0;
  int32_t state = 0;              // 0 waiting, 1 running, 2 finished
};

int32_t blocks_for(int64_t tokens, int32_t bs) { return (int32_t)((tokens + bs - 1) / bs); }

}  // namespace

struct pa_sched {
  pa_mgr* m = nullptr;
  int32_t bs = 0, max_tokens = 0, max_seqs = 0, lookahead = 0, max_skips = 0;
  std::vector<Req> reqs;
  std::deque<int32_t> waiting;    // arrival order
  std::vector<int32_t> running;   // admission order
  bool blocking = false;
  int32_t head_skips = 0;
  int32_t max_width = 1;
  int32_t n_finished = 0;
  int64_t generated = 0, cached_tokens = 0;
  std::vector<int32_t> tokens;    // prompt tokens of the requests that carry them
  std::vector<int32_t> admitted, decode;   // per-step scratch

  int32_t lifetime(const Req& r) const { return blocks_for((int64_t)r.prompt + r.want - 1, bs); }
  int32_t held(const Req& r) const { return blocks_for(pa_mgr_seq_len(m, r.sid), bs); }
};

extern "C" {

pa_sched* pa_sched_create(pa_mgr* m, int32_t max_batch_tokens, int32_t max_seqs, int32_t lookahead,
                          int32_t max_skips) {
  if (!m || max_batch_tokens < 1 || max_seqs < 1 || lookahead < 1 || max_skips < 0) return nullptr;
  pa_sched* s = new (std::nothrow) pa_sched;
  if (!s) return nullptr;
  s->m = m;
  s->max_tokens = max_batch_tokens;
  s->max_seqs = max_seqs;
  s->lookahead = lookahead;
  s->max_skips = max_skips;
  s->bs = pa_mgr_block_size(m);
  if (s->bs <= 0) {
    delete s;
    return nullptr;
  }
  return s;
}

void pa_sched_destroy(pa_sched* s) { delete s; }

int32_t pa_sched_add(pa_sched* s, int32_t prompt_len, int32_t new_tokens, int32_t* rid) {
  if (!s || !rid || prompt_len < 1 || new_tokens < 1 || prompt_len > s->max_tokens) return PA_HOST_ERR_ARG;
  Req r;
  r.prompt = prompt_len;
  r.want = new_tokens;
  if ((int64_t)prompt_len + new_tokens - 1 > INT32_MAX / 2 || s->lifetime(r) > pa_mgr_num_blocks(s->m))
    return PA_HOST_ERR_ARG;
  try {
    s->reqs.push_back(r);
    s->waiting.push_back((int32_t)s->reqs.size() - 1);
  } catch (...) {
    return PA_HOST_ERR_ARG;
  }
  s->max_width = std::max(s->max_width, s->lifetime(r));
  *rid = (int32_t)s->reqs.size() - 1;
  return PA_HOST_OK;
}

int32_t pa_sched_add_tokens(pa_sched* s, const int32_t* tokens, int32_t n, int32_t new_tokens, int32_t* rid) {
  if (!s || !tokens || n < 1) return PA_HOST_ERR_ARG;
  const size_t at = s->tokens.size();
  try {
    s->tokens.insert(s->tokens.end(), tokens, tokens + n);
  } catch (...) {
    return PA_HOST_ERR_ARG;
  }
  const int32_t st = pa_sched_add(s, n, new_tokens, rid);
  if (st != PA_HOST_OK) {
    s->tokens.resize(at);
    return st;
  }
  s->reqs[*rid].tok0 = (int32_t)at;
  return PA_HOST_OK;
}

int64_t pa_sched_cached_tokens(const pa_sched* s) { return s ? s->cached_tokens : (int64_t)PA_HOST_ERR_ARG; }

int32_t pa_sched_max_width(const pa_sched* s) { return s ? s->max_width : PA_HOST_ERR_ARG; }

int32_t pa_sched_step(pa_sched* s, int32_t* rids, int32_t* sids, int32_t* q_lens, int32_t* num_rows,
                      int32_t* finished, int32_t cap_finished, int32_t* num_finished, int32_t width,
                      int32_t* slot_mapping, int32_t* block_tables, int32_t* seq_lens) {
  if (!s || !rids || !sids || !q_lens || !num_rows || !num_finished || cap_finished < 0 ||
      (cap_finished > 0 && !finished) || !slot_mapping)
    return PA_HOST_ERR_ARG;
  if (block_tables && width < s->max_width) return PA_HOST_ERR_CAPACITY;
  // 1. release the requests that finished in the last step
  int32_t nf = 0;
  for (int32_t rid : s->running)
    if (s->reqs[rid].generated == s->reqs[rid].want) ++nf;
  if (nf > cap_finished) return PA_HOST_ERR_CAPACITY;
  nf = 0;
  std::vector<int32_t> still;
  still.reserve(s->running.size());
  for (int32_t rid : s->running) {
    Req& r = s->reqs[rid];
    if (r.generated == r.want) {
      pa_mgr_finish(s->m, r.sid);
      r.state = 2;
      finished[nf++] = rid;
      ++s->n_finished;
    } else {
      still.push_back(rid);
    }
  }
  s->running.swap(still);
  *num_finished = nf;
  // 2. every running request decodes one token
  s->decode = s->running;
  // 3. admission
  int64_t owed = 0;
  for (int32_t rid : s->running) owed += s->lifetime(s->reqs[rid]) - s->held(s->reqs[rid]);
  int64_t avail = (int64_t)pa_mgr_num_free(s->m) + pa_mgr_num_cached(s->m) - owed;
  int64_t tokens = (int64_t)s->max_tokens - (int64_t)s->decode.size();
  int64_t seqs = (int64_t)s->max_seqs - (int64_t)s->decode.size();
  s->admitted.clear();
  auto fits = [&](const Req& r) { return s->lifetime(r) <= avail && r.prompt <= tokens && seqs >= 1; };
  if (s->blocking) {
    if (!s->waiting.empty() && fits(s->reqs[s->waiting.front()])) {
      s->admitted.push_back(s->waiting.front());
      s->blocking = false;
      s->head_skips = 0;
    }
  } else {
    const int32_t look = std::min<int32_t>(s->lookahead, (int32_t)s->waiting.size());
    for (int32_t i = 0; i < look; ++i) {
      const Req& r = s->reqs[s->waiting[i]];
      if (fits(r)) {
        s->admitted.push_back(s->waiting[i]);
        avail -= s->lifetime(r);
        tokens -= r.prompt;
        seqs -= 1;
      }
    }
    if (!s->waiting.empty()) {
      const int32_t head = s->waiting.front();
      if (!s->admitted.empty() && s->admitted.front() == head) {
        s->head_skips = 0;
      } else if (!s->admitted.empty()) {
        if (++s->head_skips > s->max_skips) s->blocking = true;
      }
    }
  }
  for (int32_t rid : s->admitted) {
    s->waiting.erase(std::find(s->waiting.begin(), s->waiting.end(), rid));
    Req& r = s->reqs[rid];
    int32_t sid = -1, cached = 0;
    // cannot fail: an empty sequence takes no block, a prefix match only takes references
    const int32_t st = r.tok0 >= 0 ? pa_mgr_add_sequence_prefix(s->m, &s->tokens[r.tok0], r.prompt, &sid, &cached)
                                   : pa_mgr_add_sequence(s->m, 0, -1, 0, &sid);
    if (st != PA_HOST_OK) return st;
    r.sid = sid;
    r.first_rows = r.prompt - cached;
    s->cached_tokens += cached;
    r.state = 1;
    s->running.push_back(rid);
  }
  // 4. the batch: running requests first, then the newly admitted ones
  int32_t n = 0;
  for (int32_t rid : s->decode) {
    rids[n] = rid;
    sids[n] = s->reqs[rid].sid;
    q_lens[n] = 1;
    ++n;
  }
  for (int32_t rid : s->admitted) {
    rids[n] = rid;
    sids[n] = s->reqs[rid].sid;
    q_lens[n] = s->reqs[rid].first_rows;
    ++n;
  }
  *num_rows = n;
  if (n == 0) return PA_HOST_OK;
  int32_t nc = 0;
  const int32_t st = pa_mgr_step(s->m, sids, q_lens, n, width, slot_mapping, nullptr, 0, &nc, block_tables,
                                 seq_lens);
  if (st != PA_HOST_OK) return st;   // cannot happen: admission reserved every request's lifetime
  for (int32_t i = 0; i < n; ++i) {
    ++s->reqs[rids[i]].generated;
    ++s->generated;
  }
  // the new requests' prompts enter the prefix cache (their K/V are written by this step's
  // device work, which every later step's reads follow)
  for (int32_t rid : s->admitted) {
    const Req& r = s->reqs[rid];
    if (r.tok0 >= 0) pa_mgr_publish(s->m, r.sid, &s->tokens[r.tok0], r.prompt);
  }
  return PA_HOST_OK;
}

int32_t pa_sched_counts(const pa_sched* s, int32_t* waiting, int32_t* running, int32_t* finished,
                        int32_t* blocking, int64_t* generated) {
  if (!s) return PA_HOST_ERR_ARG;
  if (waiting) *waiting = (int32_t)s->waiting.size();
  if (running) *running = (int32_t)s->running.size();
  if (finished) *finished = s->n_finished;
  if (blocking) *blocking = s->blocking ? 1 : 0;
  if (generated) *generated = s->generated;
  return PA_HOST_OK;
}

}  // extern "C"
