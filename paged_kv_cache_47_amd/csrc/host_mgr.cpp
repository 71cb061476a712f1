// Host-side block bookkeeping (include/pa_host.h): allocator, tables,
// reference counts, copy-on-write, sliding-window release, step metadata.
//
// A step is first run as a dry run that only counts (blocks popped and pushed,
// with reference-count changes kept in a scratch overlay), so a step that the
// pool cannot supply is refused before anything changes; the real pass then
// performs the same operations in the same order and cannot fail.
//
// Prefix cache: published full blocks are nodes of a tree whose edges are
// the blocks' token ids (one block per edge), kept as a hash map from
// (parent block, tokens) to block.  A published block whose reference count
// drops to zero is cached instead of freed; when the free stack is empty, the
// least recently released cached block is evicted together with its subtree
// (cached nodes are freed, nodes still in use only leave the tree).
#include "pa_host.h"

#include <algorithm>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

namespace {

struct Seq {
  std::vector<int32_t> blocks;   // table; released entries are -1 (always a prefix)
  int32_t len = 0;
  int32_t released = 0;          // entries [0, released) are -1
  bool live = true;
};

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

struct PrefixKey {
  int32_t parent;                // parent block, -1 for the root
  std::vector<int32_t> tokens;   // the block's token ids
  bool operator==(const PrefixKey& o) const { return parent == o.parent && tokens == o.tokens; }
};

struct PrefixKeyHash {
  size_t operator()(const PrefixKey& k) const {
    uint64_t h = 1469598103934665603ull ^ (uint32_t)k.parent;
    for (int32_t t : k.tokens) h = (h ^ (uint32_t)t) * 1099511628211ull;
    return (size_t)h;
  }
};

}  // namespace

struct pa_mgr {
  int32_t nb = 0, bs = 0, window = 0;
  std::vector<int32_t> stack;    // free stack; its top is the back
  std::vector<int32_t> refs;     // reference count per block (0 = free)
  std::vector<Seq> seqs;
  // prefix cache (sized on the first publish): tree nodes, their edges, and
  // the least-recently-released list of cached blocks (refcount 0, in the tree)
  std::unordered_map<PrefixKey, int32_t, PrefixKeyHash> index;
  std::vector<uint8_t> indexed;
  std::vector<int32_t> node_parent;
  std::vector<std::vector<int32_t>> children;
  std::vector<std::vector<int32_t>> node_tokens;
  std::vector<int32_t> lru_prev, lru_next;
  int32_t lru_head = -1, lru_tail = -1, cached = 0;
  // dry-run scratch: reference-count deltas of touched blocks, per-sequence stamps
  mutable std::vector<int32_t> delta;
  mutable std::vector<int32_t> touched;
  mutable std::vector<uint32_t> seen;
  mutable uint32_t epoch = 0;

  bool held(int32_t b) const { return b >= 0 && b < nb && refs[b] > 0; }
  bool valid_seq(int32_t s) const { return s >= 0 && s < (int32_t)seqs.size(); }

  int64_t available() const { return (int64_t)stack.size() + cached; }

  // the caller has checked available() >= 1
  int32_t pop() {
    if (stack.empty()) evict(lru_head);
    const int32_t b = stack.back();
    stack.pop_back();
    refs[b] = 1;
    return b;
  }
  void drop(int32_t b) {   // b is held
    if (--refs[b] == 0) {
      if (!indexed.empty() && indexed[b]) {
        lru_push(b);
      } else {
        stack.push_back(b);
      }
    }
  }
  // a cached block taken by a prefix match
  void revive(int32_t b) {
    if (refs[b] == 0) lru_remove(b);
    ++refs[b];
  }

  void lru_push(int32_t b) {
    lru_prev[b] = lru_tail;
    lru_next[b] = -1;
    if (lru_tail >= 0) lru_next[lru_tail] = b;
    else lru_head = b;
    lru_tail = b;
    ++cached;
  }
  void lru_remove(int32_t b) {
    if (lru_prev[b] >= 0) lru_next[lru_prev[b]] = lru_next[b];
    else lru_head = lru_next[b];
    if (lru_next[b] >= 0) lru_prev[lru_next[b]] = lru_prev[b];
    else lru_tail = lru_prev[b];
    --cached;
  }
  // Take node b and its subtree out of the tree: the subtree is listed
  // breadth first and handled in reverse (deepest first, b last); cached
  // nodes go back on the free stack, nodes in use only leave the tree (they
  // are freed normally when released).
  void evict(int32_t b) {
    std::vector<int32_t> pre{b};
    for (size_t i = 0; i < pre.size(); ++i)
      for (int32_t c : children[pre[i]]) pre.push_back(c);
    const int32_t parent = node_parent[b];
    if (parent >= 0) {
      auto& sib = children[parent];
      sib.erase(std::find(sib.begin(), sib.end(), b));
    }
    for (auto it = pre.rbegin(); it != pre.rend(); ++it) {
      const int32_t x = *it;
      index.erase(PrefixKey{node_parent[x], node_tokens[x]});
      children[x].clear();
      node_tokens[x].clear();
      node_parent[x] = -1;
      indexed[x] = 0;
      if (refs[x] == 0) {
        lru_remove(x);
        stack.push_back(x);
      }
    }
  }
  void enable_prefix() {
    if (!indexed.empty()) return;
    indexed.assign(nb, 0);
    node_parent.assign(nb, -1);
    children.assign(nb, {});
    node_tokens.assign(nb, {});
    lru_prev.assign(nb, -1);
    lru_next.assign(nb, -1);
  }

  // ---- dry run ----------------------------------------------------------
  struct Plan {
    int32_t copies = 0;
    int32_t width = 1;
  };

  void bump(int32_t b, int32_t d) const {
    if (delta[b] == 0) touched.push_back(b);
    delta[b] += d;
  }
  void reset_overlay() const {
    for (int32_t b : touched) delta[b] = 0;
    touched.clear();
  }

  // Count what appending n positions to s (and, with `release`, its window
  // release) needs; `avail` is the free-block count as the step proceeds.
  int32_t dry_one(const Seq& s, int32_t n, bool release, int64_t& avail, Plan& p) const {
    int32_t nblk = (int32_t)s.blocks.size();
    if (n > 0) {
      const int32_t i0 = s.len / bs, i1 = (int32_t)(((int64_t)s.len + n - 1) / bs);
      for (int32_t idx = i0; idx <= i1; ++idx) {
        if (idx >= nblk) {            // a fresh block
          if (--avail < 0) return PA_HOST_ERR_EXHAUSTED;
          ++nblk;
        } else {
          const int32_t b = s.blocks[idx];
          if (refs[b] + delta[b] > 1) {   // shared: copy into a fresh block, drop one reference
            if (--avail < 0) return PA_HOST_ERR_EXHAUSTED;
            bump(b, -1);
            ++p.copies;
          }
        }
      }
    }
    if (release && window > 0) {
      const int32_t lo = std::max(0, s.len - window + 1);   // length after the step minus n
      const int32_t upto = std::min(lo / bs, (int32_t)s.blocks.size());
      for (int32_t lb = s.released; lb < upto; ++lb) {
        const int32_t b = s.blocks[lb];
        if (b < 0) continue;
        bump(b, -1);
        if (refs[b] + delta[b] == 0) ++avail;
      }
    }
    p.width = std::max(p.width, nblk);
    return PA_HOST_OK;
  }

  int32_t dry_run(const int32_t* sids, const int32_t* q_lens, int32_t num, bool release, Plan& p) const {
    if (num < 0 || (num > 0 && (sids == nullptr || q_lens == nullptr))) return PA_HOST_ERR_ARG;
    if (delta.size() != (size_t)nb) delta.assign(nb, 0);
    if (seen.size() < seqs.size()) seen.resize(seqs.size(), 0);
    if (++epoch == 0) {   // stamps wrapped: clear them
      std::fill(seen.begin(), seen.end(), 0);
      epoch = 1;
    }
    int64_t avail = available();
    int32_t st = PA_HOST_OK;
    for (int32_t i = 0; i < num && st == PA_HOST_OK; ++i) {
      const int32_t s = sids[i], n = q_lens[i];
      if (!valid_seq(s) || !seqs[s].live || n < 0 || seen[s] == epoch ||
          (int64_t)seqs[s].len + n > INT32_MAX / 2) {
        st = PA_HOST_ERR_ARG;
        break;
      }
      seen[s] = epoch;
      st = dry_one(seqs[s], n, release, avail, p);
    }
    reset_overlay();
    return st;
  }

  // ---- real pass ----------------------------------------------------------
  void append(Seq& s, int32_t n, int32_t* slots, int32_t* copies, int32_t& nc) {
    for (int32_t k = 0; k < n; ++k) {
      const int32_t pos = s.len + k, idx = pos / bs, off = pos % bs;
      if (idx == (int32_t)s.blocks.size()) {
        s.blocks.push_back(pop());
      } else if (off == 0 || k == 0) {   // first write into an existing block of this call
        const int32_t b = s.blocks[idx];
        if (refs[b] > 1) {
          const int32_t fresh = pop();
          copies[2 * nc] = b;
          copies[2 * nc + 1] = fresh;
          ++nc;
          drop(b);
          s.blocks[idx] = fresh;
        }
      }
      slots[k] = s.blocks[idx] * bs + off;
    }
    s.len += n;
  }

  void release_window(Seq& s, int32_t q_len) {
    if (window <= 0) return;
    const int32_t lo = std::max(0, s.len - q_len - window + 1);
    const int32_t upto = std::min(lo / bs, (int32_t)s.blocks.size());
    for (int32_t lb = s.released; lb < upto; ++lb) {
      const int32_t b = s.blocks[lb];
      if (b >= 0) {
        drop(b);
        s.blocks[lb] = -1;
      }
    }
    s.released = std::max(s.released, upto);
  }

  void write_table(const Seq& s, int32_t width, int32_t* row) const {
    const int32_t n = (int32_t)s.blocks.size();
    if (n) std::memcpy(row, s.blocks.data(), sizeof(int32_t) * n);
    if (width > n) std::memset(row + n, 0, sizeof(int32_t) * (width - n));
  }
};

extern "C" {

const char* pa_host_status_str(int32_t s) {
  switch (s) {
    case PA_HOST_OK: return "ok";
    case PA_HOST_ERR_ARG: return "invalid argument";
    case PA_HOST_ERR_EXHAUSTED: return "the pool cannot supply the blocks";
    case PA_HOST_ERR_NOT_ALLOCATED: return "the block is not allocated";
    case PA_HOST_ERR_SHARED: return "the block has more than one reference";
    case PA_HOST_ERR_CAPACITY: return "an output array is too small";
    case PA_HOST_ERR_RELEASED: return "the positions are in blocks the sliding window released";
  }
  return "unknown status";
}

pa_mgr* pa_mgr_create(int32_t num_blocks, int32_t block_size, const int32_t* first_pops, int32_t window) {
  if (num_blocks <= 0 || block_size <= 0 || window < 0) return nullptr;
  if ((int64_t)num_blocks * block_size > INT32_MAX) return nullptr;
  pa_mgr* m = new (std::nothrow) pa_mgr;
  if (m == nullptr) return nullptr;
  try {
    m->nb = num_blocks;
    m->bs = block_size;
    m->window = window;
    m->refs.assign(num_blocks, 0);
    m->stack.resize(num_blocks);
    if (first_pops == nullptr) {
      for (int32_t i = 0; i < num_blocks; ++i) m->stack[i] = num_blocks - 1 - i;
    } else {
      std::vector<char> hit(num_blocks, 0);
      for (int32_t i = 0; i < num_blocks; ++i) {
        const int32_t b = first_pops[i];
        if (b < 0 || b >= num_blocks || hit[b]) {
          delete m;
          return nullptr;
        }
        hit[b] = 1;
        m->stack[num_blocks - 1 - i] = b;   // the first entry ends on top
      }
    }
  } catch (...) {
    delete m;
    return nullptr;
  }
  return m;
}

void pa_mgr_destroy(pa_mgr* m) { delete m; }

int32_t pa_mgr_num_blocks(const pa_mgr* m) { return m ? m->nb : PA_HOST_ERR_ARG; }
int32_t pa_mgr_block_size(const pa_mgr* m) { return m ? m->bs : PA_HOST_ERR_ARG; }
int32_t pa_mgr_num_free(const pa_mgr* m) { return m ? (int32_t)m->stack.size() : PA_HOST_ERR_ARG; }

int32_t pa_mgr_allocate(pa_mgr* m, int32_t n, int32_t* out) {
  if (!m || n < 0 || (n > 0 && !out)) return PA_HOST_ERR_ARG;
  if (n > m->available()) return PA_HOST_ERR_EXHAUSTED;
  for (int32_t i = 0; i < n; ++i) out[i] = m->pop();
  return PA_HOST_OK;
}

int32_t pa_mgr_refcount(const pa_mgr* m, int32_t b) {
  if (!m || b < 0 || b >= m->nb) return -1;
  return m->refs[b];
}

int32_t pa_mgr_retain(pa_mgr* m, int32_t b) {
  if (!m) return PA_HOST_ERR_ARG;
  if (!m->held(b)) return PA_HOST_ERR_NOT_ALLOCATED;
  ++m->refs[b];
  return PA_HOST_OK;
}

int32_t pa_mgr_release(pa_mgr* m, int32_t b, int32_t* freed) {
  if (!m) return PA_HOST_ERR_ARG;
  if (!m->held(b)) return PA_HOST_ERR_NOT_ALLOCATED;
  m->drop(b);
  if (freed) *freed = m->refs[b] == 0;
  return PA_HOST_OK;
}

int32_t pa_mgr_free(pa_mgr* m, int32_t b) {
  if (!m) return PA_HOST_ERR_ARG;
  if (!m->held(b)) return PA_HOST_ERR_NOT_ALLOCATED;
  if (m->refs[b] != 1) return PA_HOST_ERR_SHARED;
  m->drop(b);
  return PA_HOST_OK;
}

int32_t pa_mgr_free_all(pa_mgr* m, const int32_t* ids, int32_t n) {
  if (!m || n < 0 || (n > 0 && !ids)) return PA_HOST_ERR_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t st = pa_mgr_free(m, ids[i]);
    if (st != PA_HOST_OK) return st;
  }
  return PA_HOST_OK;
}

int32_t pa_mgr_free_ids(const pa_mgr* m, int32_t* out, int32_t cap) {
  if (!m || cap < 0 || (cap > 0 && !out)) return PA_HOST_ERR_ARG;
  const int32_t n = (int32_t)m->stack.size();
  if (cap < n) return PA_HOST_ERR_CAPACITY;
  if (n) std::memcpy(out, m->stack.data(), sizeof(int32_t) * n);
  return n;
}

int32_t pa_mgr_refcounts(const pa_mgr* m, int32_t* out, int32_t cap) {
  if (!m || cap < 0 || (cap > 0 && !out)) return PA_HOST_ERR_ARG;
  if (cap < m->nb) return PA_HOST_ERR_CAPACITY;
  std::memcpy(out, m->refs.data(), sizeof(int32_t) * m->nb);
  return m->nb;
}

int32_t pa_mgr_add_sequence(pa_mgr* m, int32_t num_tokens, int32_t shared_from, int32_t shared_tokens,
                            int32_t* sid) {
  if (!m || !sid || num_tokens < 0) return PA_HOST_ERR_ARG;
  int32_t nshared = 0;
  if (shared_from >= 0) {
    if (!m->valid_seq(shared_from) || !m->seqs[shared_from].live) return PA_HOST_ERR_ARG;
    const Seq& src = m->seqs[shared_from];
    if (shared_tokens < 0 || shared_tokens % m->bs != 0 || shared_tokens > src.len || shared_tokens > num_tokens)
      return PA_HOST_ERR_ARG;
    nshared = shared_tokens / m->bs;
    for (int32_t j = 0; j < nshared; ++j)
      if (src.blocks[j] < 0) return PA_HOST_ERR_RELEASED;
  } else if (shared_tokens != 0) {
    return PA_HOST_ERR_ARG;
  }
  const int32_t need = ceil_div((int64_t)num_tokens - (int64_t)nshared * m->bs, m->bs);
  if (need > m->available()) return PA_HOST_ERR_EXHAUSTED;
  try {
    Seq s;
    s.blocks.reserve(nshared + need);
    for (int32_t j = 0; j < nshared; ++j) s.blocks.push_back(m->seqs[shared_from].blocks[j]);
    s.len = num_tokens;
    m->seqs.push_back(std::move(s));
  } catch (...) {
    return PA_HOST_ERR_ARG;
  }
  Seq& s = m->seqs.back();
  for (int32_t i = 0; i < need; ++i) s.blocks.push_back(m->pop());
  for (int32_t j = 0; j < nshared; ++j) ++m->refs[s.blocks[j]];
  *sid = (int32_t)m->seqs.size() - 1;
  return PA_HOST_OK;
}

int32_t pa_mgr_num_cached(const pa_mgr* m) { return m ? m->cached : PA_HOST_ERR_ARG; }

int32_t pa_mgr_add_sequence_prefix(pa_mgr* m, const int32_t* tokens, int32_t n, int32_t* sid,
                                   int32_t* cached_tokens) {
  if (!m || !sid || !cached_tokens || n < 1 || !tokens) return PA_HOST_ERR_ARG;
  std::vector<int32_t> matched;
  if (!m->indexed.empty()) {
    const int32_t maxb = (n - 1) / m->bs;   // at least one prompt token is left to compute
    PrefixKey key{-1, {}};
    for (int32_t j = 0; j < maxb; ++j) {
      key.tokens.assign(tokens + (int64_t)j * m->bs, tokens + (int64_t)(j + 1) * m->bs);
      auto it = m->index.find(key);
      if (it == m->index.end()) break;
      matched.push_back(it->second);
      key.parent = it->second;
    }
  }
  try {
    Seq s;
    s.blocks = matched;
    s.len = (int32_t)matched.size() * m->bs;
    m->seqs.push_back(std::move(s));
  } catch (...) {
    return PA_HOST_ERR_ARG;
  }
  for (int32_t b : matched) m->revive(b);
  *sid = (int32_t)m->seqs.size() - 1;
  *cached_tokens = (int32_t)matched.size() * m->bs;
  return PA_HOST_OK;
}

int32_t pa_mgr_publish(pa_mgr* m, int32_t sid, const int32_t* tokens, int32_t n) {
  if (!m || !m->valid_seq(sid) || n < 0 || (n > 0 && !tokens)) return PA_HOST_ERR_ARG;
  const Seq& s = m->seqs[sid];
  if (!s.live) return PA_HOST_ERR_ARG;
  try {
    m->enable_prefix();
  } catch (...) {
    return PA_HOST_ERR_ARG;
  }
  const int32_t nfull = std::min(n, s.len) / m->bs;
  PrefixKey key{-1, {}};
  for (int32_t j = 0; j < nfull; ++j) {
    const int32_t b = s.blocks[j];
    if (b < 0) break;                                // released by a sliding window
    key.tokens.assign(tokens + (int64_t)j * m->bs, tokens + (int64_t)(j + 1) * m->bs);
    auto it = m->index.find(key);
    if (it != m->index.end()) {
      if (it->second != b) break;                    // another block already holds this path
      key.parent = b;
      continue;
    }
    if (m->indexed[b]) break;                        // this block is a node on another path
    try {
      m->index.emplace(key, b);
      if (key.parent >= 0) m->children[key.parent].push_back(b);
    } catch (...) {
      return PA_HOST_ERR_ARG;
    }
    m->indexed[b] = 1;
    m->node_parent[b] = key.parent;
    m->node_tokens[b] = key.tokens;
    key.parent = b;
  }
  return PA_HOST_OK;
}

int32_t pa_mgr_fork(pa_mgr* m, int32_t sid, int32_t* child) {
  if (!m || !child || !m->valid_seq(sid) || !m->seqs[sid].live) return PA_HOST_ERR_ARG;
  try {
    Seq c = m->seqs[sid];
    m->seqs.push_back(std::move(c));
  } catch (...) {
    return PA_HOST_ERR_ARG;
  }
  for (int32_t b : m->seqs.back().blocks)
    if (b >= 0) ++m->refs[b];
  *child = (int32_t)m->seqs.size() - 1;
  return PA_HOST_OK;
}

int32_t pa_mgr_finish(pa_mgr* m, int32_t sid) {
  if (!m || !m->valid_seq(sid)) return PA_HOST_ERR_ARG;
  Seq& s = m->seqs[sid];
  if (!s.live) return PA_HOST_OK;
  for (int32_t b : s.blocks)
    if (b >= 0) m->drop(b);
  s.blocks.clear();
  s.blocks.shrink_to_fit();
  s.released = 0;
  s.live = false;
  return PA_HOST_OK;
}

int32_t pa_mgr_num_seqs(const pa_mgr* m) { return m ? (int32_t)m->seqs.size() : PA_HOST_ERR_ARG; }

int32_t pa_mgr_seq_len(const pa_mgr* m, int32_t sid) {
  if (!m || !m->valid_seq(sid)) return -1;
  return m->seqs[sid].len;
}

int32_t pa_mgr_seq_blocks(const pa_mgr* m, int32_t sid, int32_t* out, int32_t cap) {
  if (!m || !m->valid_seq(sid) || cap < 0 || (cap > 0 && !out)) return PA_HOST_ERR_ARG;
  const Seq& s = m->seqs[sid];
  const int32_t n = (int32_t)s.blocks.size();
  if (cap < n) return PA_HOST_ERR_CAPACITY;
  if (n) std::memcpy(out, s.blocks.data(), sizeof(int32_t) * n);
  return n;
}

int32_t pa_mgr_slots(const pa_mgr* m, int32_t sid, int32_t start, int32_t n, int32_t* out) {
  if (!m || !m->valid_seq(sid) || start < 0 || n < 0 || (n > 0 && !out)) return PA_HOST_ERR_ARG;
  const Seq& s = m->seqs[sid];
  if ((int64_t)start + n > s.len || !s.live) return PA_HOST_ERR_ARG;
  if (n > 0 && s.blocks[start / m->bs] < 0) return PA_HOST_ERR_RELEASED;
  for (int32_t k = 0; k < n; ++k) {
    const int32_t pos = start + k;
    out[k] = s.blocks[pos / m->bs] * m->bs + pos % m->bs;
  }
  return PA_HOST_OK;
}

int32_t pa_mgr_append(pa_mgr* m, int32_t sid, int32_t n, int32_t* slots, int32_t* copies, int32_t cap_copies,
                      int32_t* n_copies) {
  if (!m || !n_copies || cap_copies < 0 || (n > 0 && !slots) || (cap_copies > 0 && !copies))
    return PA_HOST_ERR_ARG;
  pa_mgr::Plan p;
  const int32_t st = m->dry_run(&sid, &n, 1, false, p);
  if (st != PA_HOST_OK) return st;
  if (p.copies > cap_copies) return PA_HOST_ERR_CAPACITY;
  int32_t nc = 0;
  m->append(m->seqs[sid], n, slots, copies, nc);
  *n_copies = nc;
  return PA_HOST_OK;
}

int32_t pa_mgr_release_out_of_window(pa_mgr* m, int32_t sid, int32_t q_len) {
  if (!m || !m->valid_seq(sid) || q_len < 0 || q_len > m->seqs[sid].len) return PA_HOST_ERR_ARG;
  if (m->seqs[sid].live) m->release_window(m->seqs[sid], q_len);
  return PA_HOST_OK;
}

int32_t pa_mgr_step_width(const pa_mgr* m, const int32_t* sids, const int32_t* q_lens, int32_t num_seqs) {
  if (!m) return PA_HOST_ERR_ARG;
  pa_mgr::Plan p;
  // growth alone decides the width, but the dry run also validates the step
  const int32_t st = m->dry_run(sids, q_lens, num_seqs, true, p);
  if (st == PA_HOST_ERR_EXHAUSTED || st == PA_HOST_OK) {
    // an exhausted pool still has a well-defined width: the tables' final sizes
    int32_t w = 1;
    for (int32_t i = 0; i < num_seqs; ++i) {
      const Seq& s = m->seqs[sids[i]];
      w = std::max<int32_t>(w, std::max<int32_t>((int32_t)s.blocks.size(),
                                                 ceil_div((int64_t)s.len + q_lens[i], m->bs)));
    }
    return w;
  }
  return st;
}

int32_t pa_mgr_step(pa_mgr* m, const int32_t* sids, const int32_t* q_lens, int32_t num_seqs, int32_t width,
                    int32_t* slot_mapping, int32_t* copies, int32_t cap_copies, int32_t* n_copies,
                    int32_t* block_tables, int32_t* seq_lens) {
  if (!m || !n_copies || cap_copies < 0 || (cap_copies > 0 && !copies)) return PA_HOST_ERR_ARG;
  pa_mgr::Plan p;
  const int32_t st = m->dry_run(sids, q_lens, num_seqs, true, p);
  if (st != PA_HOST_OK) return st;
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) total += q_lens[i];
  if (total > 0 && !slot_mapping) return PA_HOST_ERR_ARG;
  if (p.copies > cap_copies) return PA_HOST_ERR_CAPACITY;
  if (block_tables && width < p.width) return PA_HOST_ERR_CAPACITY;
  int32_t nc = 0;
  int64_t off = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    Seq& s = m->seqs[sids[i]];
    m->append(s, q_lens[i], slot_mapping + off, copies, nc);
    m->release_window(s, q_lens[i]);
    off += q_lens[i];
  }
  *n_copies = nc;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = m->seqs[sids[i]];
    if (block_tables) m->write_table(s, width, block_tables + (int64_t)i * width);
    if (seq_lens) seq_lens[i] = s.len;
  }
  return PA_HOST_OK;
}

int32_t pa_mgr_block_tables(const pa_mgr* m, const int32_t* sids, int32_t num_seqs, int32_t width, int32_t* out) {
  if (!m || num_seqs < 0 || width < 0 || (num_seqs > 0 && (!sids || !out))) return PA_HOST_ERR_ARG;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (!m->valid_seq(sids[i])) return PA_HOST_ERR_ARG;
    if ((int32_t)m->seqs[sids[i]].blocks.size() > width) return PA_HOST_ERR_CAPACITY;
  }
  for (int32_t i = 0; i < num_seqs; ++i) m->write_table(m->seqs[sids[i]], width, out + (int64_t)i * width);
  return PA_HOST_OK;
}

}  // extern "C"
