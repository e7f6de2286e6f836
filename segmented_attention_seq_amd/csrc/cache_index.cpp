// KV cache index of the AKV server: an extended radix tree over token and cache-op
// histories, position versions per token, and drop-aware eviction.  Host code only.
//
// "Cache Engineering for Agents" review, AKV serving system (§4.2, App. A.1.2, Fig. 8)
// and the request-flow diagram; explainer (vibeprogramminglab), §3.4 / Fig. 5:
//   * rows are shared only where the token history and the op history agree: a drop
//     node records which logical entries a boundary removed, a repos node opens the
//     branch in which the surviving keys sit at new positions;
//   * a token's rows exist per position version: a version at the needed position is
//     copied as it is, any other is converted by rotating the key;
//   * storage goes back only when no running computation or restore uses it
//     (locks); among unused rows the dropped ones go before those of finished
//     requests; an emptied row leaves its tree node in place, so later rows stay
//     reachable; versions are evicted one by one.
//
// Readings (the pages leave these open):
//   canonical history  -- token items, one drop item per boundary holding the
//       logical ranges that boundary actually removed (merged, no-op drops
//       dropped), and a repos item only when the repos moves a position or the next
//       position;
//   finished requests  -- the final states of completed requests whose history is
//       not a strict prefix of another completed history (the latest round of each
//       conversation); a version held by such a state is "finished", every other
//       unlocked version is "dropped"; least recently used first within a class
//       (one clock tick per call), then the lower slot;
//   restore start      -- the largest s in [0, T] such that every key seen by a query
//       at or after s, and every final-state token below s, has a resident version;
//       a missing token j blocks exactly the starts s with j < s < D_j (D_j = the
//       boundary that drops it, infinity if none);
//   preferred version  -- the one at the needed position (final position for tokens
//       of the final state, else the append position), else the most recently used,
//       then the lowest position.
//
// Layout: nodes live in one vector and refer to each other by index; a token node
// holds a run of token ids and, per token, a tree-token id (tid) that survives node
// splits.  Versions hang off the tid.  Every slot of the caller's KV pool is free,
// allocated-and-empty (locked, no version) or holds one version.
#include <algorithm>
#include <climits>
#include <cstring>
#include <map>
#include <new>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "internal.h"

namespace {

enum { K_TOKEN = 0, K_DROP = 1, K_REPOS = 2, K_ROOT = -1 };

struct Node {
  int32_t parent = -1;
  int32_t kind = K_ROOT;
  std::vector<int32_t> tok, tid;        // K_TOKEN: the run and its tree-token ids
  std::vector<int64_t> drop;            // K_DROP: ranges [a, b) flattened
  std::map<std::vector<int64_t>, int32_t> child;
  int64_t marks_here = 0, marks_below = 0;  // below: this node's subtree, itself included
  std::vector<int32_t> state_tid, state_pos;  // final state of the mark here while frontier
};

struct Ver {
  int32_t pos, slot, held;   // slot -1: not resident (kept while held > 0)
};

struct Slot {
  int32_t lock = 0;
  int32_t tid = -1, pos = -1;   // the version held, tid -1 if none
  int64_t last = 0;
  bool held = false;
};

// Canonical history of one request (readings above).
struct History {
  std::vector<int32_t> kind;               // per item
  std::vector<int32_t> val;                // token id, or index into drops
  std::vector<std::vector<int64_t>> drops;
  std::vector<int64_t> tok_item;           // item index of each token
  std::vector<int32_t> tok_pos, tok_drop;
  std::vector<int32_t> final_tok, final_pos;
  int64_t p_next = 0;
};

struct R64 { int64_t a, b; };

int build_history(const int32_t* tok, int64_t n_tok, const akv_op* ops, int64_t n_ops, History& h,
                  const char* who) {
  const std::string w(who);
  if (n_tok < 0 || (n_tok > 0 && !tok)) return akv::fail(AKV_EINVAL, w + ": bad token array");
  if (n_ops < 0 || (n_ops > 0 && !ops)) return akv::fail(AKV_EINVAL, w + ": bad op array");
  if (n_tok > (int64_t)INT32_MAX - 1) return akv::fail(AKV_EINVAL, w + ": too many tokens");
  int64_t T = 0;
  for (int64_t n = 0; n < n_ops; ++n) {
    const akv_op& op = ops[n];
    if (op.kind == AKV_OP_APPEND) {
      if (op.a < 0) return akv::fail(AKV_EOPSEQ, w + ": op " + std::to_string(n) + ": negative append");
      T += op.a;
      if (T > n_tok) return akv::fail(AKV_EINVAL, w + ": ops append more tokens than given");
    } else if (op.kind == AKV_OP_DROP) {
      if (op.a < 0 || op.b < op.a || op.b > T)
        return akv::fail(AKV_EOPSEQ, w + ": op " + std::to_string(n) + ": drop range not yet appended");
    } else if (op.kind != AKV_OP_REPOS) {
      return akv::fail(AKV_EOPSEQ, w + ": op " + std::to_string(n) + ": unknown kind");
    }
  }
  if (T != n_tok) return akv::fail(AKV_EINVAL, w + ": ops append fewer tokens than given");

  h.tok_pos.assign(T, 0);
  h.tok_drop.assign(T, INT32_MAX);
  h.tok_item.assign(T, 0);
  std::vector<int32_t> pos(T, 0);     // current position of active tokens
  std::vector<R64> live;              // active tokens, ascending ranges
  std::vector<R64> pending;           // removed at the current boundary
  int64_t t = 0, p_next = 0, n_live = 0;

  auto flush = [&]() {
    if (pending.empty()) return;
    std::sort(pending.begin(), pending.end(), [](const R64& x, const R64& y) { return x.a < y.a; });
    std::vector<int64_t> flat;
    for (const R64& r : pending) {
      if (!flat.empty() && flat.back() == r.a) flat.back() = r.b;
      else { flat.push_back(r.a); flat.push_back(r.b); }
    }
    h.kind.push_back(K_DROP);
    h.val.push_back((int32_t)h.drops.size());
    h.drops.push_back(std::move(flat));
    pending.clear();
  };

  for (int64_t n = 0; n < n_ops; ++n) {
    const akv_op& op = ops[n];
    if (op.kind == AKV_OP_APPEND) {
      if (op.a == 0) continue;
      flush();
      for (int64_t m = 0; m < op.a; ++m) {
        h.tok_pos[t + m] = pos[t + m] = (int32_t)(p_next + m);
        h.tok_item[t + m] = (int64_t)h.kind.size();
        h.kind.push_back(K_TOKEN);
        h.val.push_back(tok[t + m]);
      }
      if (!live.empty() && live.back().b == t) live.back().b += op.a;
      else live.push_back({t, t + op.a});
      t += op.a;
      p_next += op.a;
      n_live += op.a;
    } else if (op.kind == AKV_OP_DROP) {
      std::vector<R64> kept;
      kept.reserve(live.size() + 1);
      for (const R64& r : live) {
        const int64_t lo = std::max(r.a, op.a), hi = std::min(r.b, op.b);
        if (lo >= hi) { kept.push_back(r); continue; }
        for (int64_t j = lo; j < hi; ++j) h.tok_drop[j] = (int32_t)t;
        pending.push_back({lo, hi});
        n_live -= hi - lo;
        if (r.a < lo) kept.push_back({r.a, lo});
        if (hi < r.b) kept.push_back({hi, r.b});
      }
      live.swap(kept);
    } else {  // REPOS: an event only if it moves a position or the next position
      bool moves = p_next != n_live;
      int64_t rank = 0;
      for (const R64& r : live) {
        for (int64_t j = r.a; j < r.b && !moves; ++j, ++rank) moves = pos[j] != rank;
        if (moves) break;
      }
      if (!moves) continue;
      flush();
      rank = 0;
      for (const R64& r : live)
        for (int64_t j = r.a; j < r.b; ++j) pos[j] = (int32_t)rank++;
      p_next = n_live;
      h.kind.push_back(K_REPOS);
      h.val.push_back(0);
    }
  }
  flush();
  h.p_next = p_next;
  h.final_tok.clear();
  h.final_pos.clear();
  h.final_tok.reserve(n_live);
  h.final_pos.reserve(n_live);
  for (const R64& r : live)
    for (int64_t j = r.a; j < r.b; ++j) {
      h.final_tok.push_back((int32_t)j);
      h.final_pos.push_back(pos[j]);
    }
  return AKV_OK;
}

std::vector<int64_t> child_key(const History& h, size_t item) {
  if (h.kind[item] == K_TOKEN) return {K_TOKEN, h.val[item]};
  if (h.kind[item] == K_REPOS) return {K_REPOS};
  std::vector<int64_t> k{K_DROP};
  const auto& d = h.drops[h.val[item]];
  k.insert(k.end(), d.begin(), d.end());
  return k;
}

}  // namespace

struct akv_cache {
  std::vector<Node> nodes;
  std::vector<std::vector<Ver>> vers;   // by tid
  std::vector<Slot> slots;
  std::set<int32_t> free;
  std::set<std::tuple<int, int64_t, int32_t>> evictable;   // (held, last, slot)
  int64_t clock = 0;

  // --- evictable-set upkeep: call ev_out before changing a slot, ev_in after ---
  std::tuple<int, int64_t, int32_t> ev_key(int32_t s) const {
    return {slots[s].held ? 1 : 0, slots[s].last, s};
  }
  void ev_out(int32_t s) {
    if (slots[s].tid >= 0 && slots[s].lock == 0) evictable.erase(ev_key(s));
  }
  void ev_in(int32_t s) {
    if (slots[s].tid >= 0 && slots[s].lock == 0) evictable.insert(ev_key(s));
  }

  Ver* find_ver(int32_t tid, int32_t pos) {
    for (Ver& v : vers[tid])
      if (v.pos == pos) return &v;
    return nullptr;
  }

  void held_inc(int32_t tid, int32_t pos) {
    Ver* v = find_ver(tid, pos);
    if (!v) {
      vers[tid].push_back({pos, -1, 0});
      v = &vers[tid].back();
    }
    if (v->held++ == 0 && v->slot >= 0) {
      ev_out(v->slot);
      slots[v->slot].held = true;
      ev_in(v->slot);
    }
  }

  void held_dec(int32_t tid, int32_t pos) {
    Ver* v = find_ver(tid, pos);
    if (!v || v->held == 0) return;   // cannot happen: states are counted once
    if (--v->held > 0) return;
    if (v->slot >= 0) {
      ev_out(v->slot);
      slots[v->slot].held = false;
      ev_in(v->slot);
    } else {
      auto& vs = vers[tid];
      vs.erase(vs.begin() + (v - vs.data()));
    }
  }

  int32_t new_tid() {
    vers.emplace_back();
    return (int32_t)vers.size() - 1;
  }

  // Split token node n before offset k (0 < k < size); returns the new prefix node.
  int32_t split(int32_t n, size_t k) {
    const int32_t p = (int32_t)nodes.size();
    nodes.emplace_back();
    Node& P = nodes[p];
    Node& N = nodes[n];
    P.parent = N.parent;
    P.kind = K_TOKEN;
    P.tok.assign(N.tok.begin(), N.tok.begin() + k);
    P.tid.assign(N.tid.begin(), N.tid.begin() + k);
    N.tok.erase(N.tok.begin(), N.tok.begin() + k);
    N.tid.erase(N.tid.begin(), N.tid.begin() + k);
    P.marks_below = N.marks_below;
    P.child[{K_TOKEN, N.tok[0]}] = n;
    nodes[P.parent].child[{K_TOKEN, P.tok[0]}] = p;
    N.parent = p;
    return p;
  }

  // Read-only walk: tid of each leading token whose history prefix is in the tree.
  int64_t walk(const History& h, std::vector<int32_t>& tid_of) const {
    const int64_t T = (int64_t)h.tok_item.size();
    tid_of.assign(T, -1);
    int32_t cur = 0;
    size_t off = 0;
    int64_t ti = 0;
    for (size_t it = 0; it < h.kind.size(); ++it) {
      const Node& N = nodes[cur];
      if (N.kind == K_TOKEN && off < N.tok.size()) {
        if (h.kind[it] != K_TOKEN || N.tok[off] != h.val[it]) break;
        tid_of[ti++] = N.tid[off++];
        continue;
      }
      auto c = N.child.find(child_key(h, it));
      if (c == N.child.end()) break;
      cur = c->second;
      off = 0;
      if (h.kind[it] == K_TOKEN) tid_of[ti++] = nodes[cur].tid[off++];
    }
    return ti;
  }

  // Walk creating and splitting nodes; returns the node where the history ends
  // (always at a node end) and the tid of every token.
  int32_t insert_path(const History& h, std::vector<int32_t>& tid_of) {
    tid_of.assign(h.tok_item.size(), -1);
    int32_t cur = 0, fresh = -1;
    size_t off = 0;
    int64_t ti = 0;
    for (size_t it = 0; it < h.kind.size(); ++it) {
      if (nodes[cur].kind == K_TOKEN && off < nodes[cur].tok.size()) {
        if (h.kind[it] == K_TOKEN && nodes[cur].tok[off] == h.val[it]) {
          tid_of[ti++] = nodes[cur].tid[off++];
          continue;
        }
        cur = split(cur, off);          // diverges inside the run: cut it here
        off = nodes[cur].tok.size();
      }
      if (h.kind[it] == K_TOKEN && cur == fresh) {   // extend the run made by this call
        const int32_t id = new_tid();
        nodes[cur].tok.push_back(h.val[it]);
        nodes[cur].tid.push_back(id);
        tid_of[ti++] = id;
        ++off;
        continue;
      }
      std::vector<int64_t> key = child_key(h, it);
      auto c = nodes[cur].child.find(key);
      if (c != nodes[cur].child.end()) {
        cur = c->second;
        off = 0;
        if (h.kind[it] == K_TOKEN) tid_of[ti++] = nodes[cur].tid[off++];
        continue;
      }
      const int32_t n = (int32_t)nodes.size();
      nodes.emplace_back();
      Node& M = nodes[n];
      M.parent = cur;
      M.kind = h.kind[it];
      if (M.kind == K_TOKEN) {
        const int32_t id = new_tid();
        M.tok.push_back(h.val[it]);
        M.tid.push_back(id);
        tid_of[ti++] = id;
        off = 1;
        fresh = n;
      } else {
        if (M.kind == K_DROP) M.drop = h.drops[h.val[it]];
        off = 0;
        fresh = -1;
      }
      nodes[cur].child.emplace(std::move(key), n);
      cur = n;
    }
    if (nodes[cur].kind == K_TOKEN && off < nodes[cur].tok.size()) cur = split(cur, off);
    return cur;
  }

  // Record a completed request ending at node x with final state (tid, pos).
  void add_mark(int32_t x, const std::vector<int32_t>& ftid, const std::vector<int32_t>& fpos) {
    if (nodes[x].marks_here == 0) {
      const bool frontier = nodes[x].marks_below == 0;
      for (int32_t a = nodes[x].parent; a >= 0; a = nodes[a].parent) {
        Node& A = nodes[a];
        if (A.marks_here > 0 && A.marks_below == A.marks_here) {   // was frontier
          for (size_t i = 0; i < A.state_tid.size(); ++i) held_dec(A.state_tid[i], A.state_pos[i]);
          std::vector<int32_t>().swap(A.state_tid);
          std::vector<int32_t>().swap(A.state_pos);
        }
      }
      if (frontier) {
        nodes[x].state_tid = ftid;
        nodes[x].state_pos = fpos;
        for (size_t i = 0; i < ftid.size(); ++i) held_inc(ftid[i], fpos[i]);
      }
    }
    nodes[x].marks_here += 1;
    for (int32_t a = x; a >= 0; a = nodes[a].parent) nodes[a].marks_below += 1;
  }
};

extern "C" {

int akv_cache_create(int32_t n_slots, akv_cache** out) {
  if (!out) return akv::fail(AKV_EINVAL, "akv_cache_create: out is NULL");
  *out = nullptr;
  if (n_slots < 1) return akv::fail(AKV_EINVAL, "akv_cache_create: n_slots must be positive");
  akv_cache* c = new (std::nothrow) akv_cache;
  if (!c) return akv::fail(AKV_ENOMEM, "akv_cache_create: allocation failed");
  try {
    c->nodes.emplace_back();   // root
    c->slots.resize(n_slots);
    for (int32_t s = 0; s < n_slots; ++s) c->free.insert(c->free.end(), s);
  } catch (const std::bad_alloc&) {
    delete c;
    return akv::fail(AKV_ENOMEM, "akv_cache_create: allocation failed");
  }
  *out = c;
  return AKV_OK;
}

void akv_cache_destroy(akv_cache* c) { delete c; }

int akv_cache_match(akv_cache* c, const int32_t* tok, int64_t n_tok, const akv_op* ops, int64_t n_ops,
                    int32_t lock, int32_t* slot_out, int32_t* pos_out, akv_cache_match_info* info) {
  if (!c) return akv::fail(AKV_EINVAL, "akv_cache_match: cache is NULL");
  if (n_tok > 0 && (!slot_out || !pos_out)) return akv::fail(AKV_EINVAL, "akv_cache_match: output is NULL");
  try {
    c->clock += 1;
    History h;
    if (int st = build_history(tok, n_tok, ops, n_ops, h, "akv_cache_match")) return st;
    std::vector<int32_t> tid;
    const int64_t n_matched = c->walk(h, tid);
    const int64_t T = n_tok;
    std::vector<int32_t> want(h.tok_pos.begin(), h.tok_pos.end());
    for (size_t i = 0; i < h.final_tok.size(); ++i) want[h.final_tok[i]] = h.final_pos[i];
    int64_t n_res = 0;
    for (int64_t i = 0; i < T; ++i) {
      slot_out[i] = -1;
      pos_out[i] = -1;
      if (tid[i] < 0) continue;
      const Ver* best = nullptr;
      for (const Ver& v : c->vers[tid[i]]) {
        if (v.slot < 0) continue;
        if (v.pos == want[i]) { best = &v; break; }
        if (!best) { best = &v; continue; }
        const int64_t lv = c->slots[v.slot].last, lb = c->slots[best->slot].last;
        if (lv > lb || (lv == lb && v.pos < best->pos)) best = &v;
      }
      if (!best) continue;
      slot_out[i] = best->slot;
      pos_out[i] = best->pos;
      ++n_res;
    }
    for (int64_t i = 0; i < T; ++i) {
      const int32_t s = slot_out[i];
      if (s < 0) continue;
      c->ev_out(s);
      c->slots[s].last = c->clock;
      if (lock) c->slots[s].lock += 1;
      c->ev_in(s);
    }
    // restore start: largest s with no missing j < s < D_j
    int64_t s0 = 0;
    {
      std::vector<int64_t> pm(T + 1);
      pm[0] = -1;
      for (int64_t j = 0; j < T; ++j)
        pm[j + 1] = std::max<int64_t>(pm[j], slot_out[j] < 0 ? (int64_t)h.tok_drop[j] : -1);
      for (int64_t s = T; s >= 0; --s)
        if (pm[s] <= s) { s0 = s; break; }
    }
    if (info) {
      info->n_tokens = T;
      info->n_matched = n_matched;
      info->n_resident = n_res;
      info->restore_from = s0;
      info->n_final = (int64_t)h.final_tok.size();
      info->p_next = h.p_next;
    }
  } catch (const std::bad_alloc&) {
    return akv::fail(AKV_ENOMEM, "akv_cache_match: allocation failed");
  }
  return AKV_OK;
}

int akv_cache_alloc(akv_cache* c, int32_t n, int32_t* slots_out) {
  if (!c) return akv::fail(AKV_EINVAL, "akv_cache_alloc: cache is NULL");
  c->clock += 1;
  if (n < 0 || (n > 0 && !slots_out)) return akv::fail(AKV_EINVAL, "akv_cache_alloc: bad count or output");
  if ((uint64_t)n > c->free.size() + c->evictable.size())
    return akv::fail(AKV_ENOSPACE, "akv_cache_alloc: " + std::to_string(n) + " rows asked, " +
                                       std::to_string(c->free.size() + c->evictable.size()) +
                                       " free or evictable (the rest are locked)");
  int32_t k = 0;
  while (k < n && !c->free.empty()) {
    slots_out[k++] = *c->free.begin();
    c->free.erase(c->free.begin());
  }
  while (k < n) {
    const int32_t s = std::get<2>(*c->evictable.begin());
    c->evictable.erase(c->evictable.begin());
    Slot& S = c->slots[s];
    auto& vs = c->vers[S.tid];
    for (size_t i = 0; i < vs.size(); ++i)
      if (vs[i].pos == S.pos) {
        if (vs[i].held > 0) vs[i].slot = -1;
        else vs.erase(vs.begin() + i);
        break;
      }
    S.tid = S.pos = -1;
    S.held = false;
    slots_out[k++] = s;
  }
  for (int32_t i = 0; i < n; ++i) {
    c->slots[slots_out[i]].lock = 1;
    c->slots[slots_out[i]].last = c->clock;
  }
  return AKV_OK;
}

int akv_cache_insert(akv_cache* c, const int32_t* tok, int64_t n_tok, const akv_op* ops, int64_t n_ops,
                     const int32_t* ver_token, const int32_t* ver_pos, const int32_t* ver_slot,
                     int64_t n_ver) {
  if (!c) return akv::fail(AKV_EINVAL, "akv_cache_insert: cache is NULL");
  try {
    c->clock += 1;
    History h;
    if (int st = build_history(tok, n_tok, ops, n_ops, h, "akv_cache_insert")) return st;
    if (n_ver < 0 || (n_ver > 0 && (!ver_token || !ver_pos || !ver_slot)))
      return akv::fail(AKV_EINVAL, "akv_cache_insert: bad version arrays");
    // validate everything before the tree changes
    std::vector<int32_t> tid;
    c->walk(h, tid);
    std::set<int32_t> used_slot;
    std::set<std::pair<int32_t, int32_t>> used_row;
    const int32_t n_slots = (int32_t)c->slots.size();
    for (int64_t v = 0; v < n_ver; ++v) {
      const int32_t i = ver_token[v], p = ver_pos[v], s = ver_slot[v];
      if (i < 0 || i >= n_tok || p < 0 || s < 0 || s >= n_slots)
        return akv::fail(AKV_EINVAL, "akv_cache_insert: version " + std::to_string(v) + " out of range");
      if (c->slots[s].tid >= 0 || c->slots[s].lock == 0 || !used_slot.insert(s).second)
        return akv::fail(AKV_EINVAL, "akv_cache_insert: slot " + std::to_string(s) +
                                         " is not an allocated empty slot");
      if (!used_row.insert({i, p}).second)
        return akv::fail(AKV_EINVAL, "akv_cache_insert: version given twice");
      if (tid[i] >= 0) {
        const Ver* e = c->find_ver(tid[i], p);
        if (e && e->slot >= 0) return akv::fail(AKV_EINVAL, "akv_cache_insert: version already resident");
      }
    }
    const int32_t end = c->insert_path(h, tid);
    for (int64_t v = 0; v < n_ver; ++v) {
      const int32_t t = tid[ver_token[v]], p = ver_pos[v], s = ver_slot[v];
      Ver* e = c->find_ver(t, p);
      if (!e) {
        c->vers[t].push_back({p, -1, 0});
        e = &c->vers[t].back();
      }
      e->slot = s;
      Slot& S = c->slots[s];   // locked: not in the evictable set
      S.tid = t;
      S.pos = p;
      S.last = c->clock;
      S.held = e->held > 0;
    }
    std::vector<int32_t> ftid(h.final_tok.size());
    for (size_t k = 0; k < ftid.size(); ++k) ftid[k] = tid[h.final_tok[k]];
    c->add_mark(end, ftid, h.final_pos);
  } catch (const std::bad_alloc&) {
    return akv::fail(AKV_ENOMEM, "akv_cache_insert: allocation failed");
  }
  return AKV_OK;
}

int akv_cache_unlock(akv_cache* c, const int32_t* slots, int64_t n) {
  if (!c) return akv::fail(AKV_EINVAL, "akv_cache_unlock: cache is NULL");
  if (n < 0 || (n > 0 && !slots)) return akv::fail(AKV_EINVAL, "akv_cache_unlock: bad slot array");
  std::map<int32_t, int32_t> count;
  for (int64_t i = 0; i < n; ++i) count[slots[i]] += 1;
  for (const auto& kv : count)
    if (kv.first < 0 || kv.first >= (int32_t)c->slots.size() || c->slots[kv.first].lock < kv.second)
      return akv::fail(AKV_EINVAL, "akv_cache_unlock: slot " + std::to_string(kv.first) + " is not locked");
  for (const auto& kv : count) {
    const int32_t s = kv.first;
    c->ev_out(s);
    c->slots[s].lock -= kv.second;
    if (c->slots[s].lock == 0 && c->slots[s].tid < 0) c->free.insert(s);
    else c->ev_in(s);
  }
  return AKV_OK;
}

int akv_cache_stats_get(const akv_cache* c, akv_cache_stats* out) {
  if (!c || !out) return akv::fail(AKV_EINVAL, "akv_cache_stats_get: NULL argument");
  std::memset(out, 0, sizeof(*out));
  out->n_slots = (int64_t)c->slots.size();
  out->n_free = (int64_t)c->free.size();
  for (const Slot& s : c->slots) {
    out->n_resident += s.tid >= 0;
    out->n_locked += s.lock > 0;
  }
  out->n_nodes = (int64_t)c->nodes.size();
  out->n_tree_tokens = (int64_t)c->vers.size();
  for (const Node& n : c->nodes) {
    out->n_marks += n.marks_here > 0;
    out->n_frontier += n.marks_here > 0 && n.marks_below == n.marks_here;
  }
  return AKV_OK;
}

}  // extern "C"
