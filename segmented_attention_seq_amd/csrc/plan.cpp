// Host plan compiler: canonical op list -> restore plan (tables T1..T7, work
// items, tile-class lists, device image).
//
// Semantics follow the "three cache operations" of the "Cache Engineering for
// Agents" review (§3.3): append gives the token the next position; drop removes
// entries from later attention without touching positions; repos renumbers the
// remaining keys 0..r-1 in logical order and restarts appends at r.  The
// segment-batch form follows the review's "single-prefill restore" section
// (§4.2, App. A.1.1): query i sees key j iff j <= i < drop boundary of j, and
// each repos stretch sees the keys active after its repos as version rows whose
// positions are their row indices.
//
// The live set is kept as a short list of token ranges (drops cut whole message
// ranges, so it stays small), which makes every op O(number of ranges) plus the
// tokens it touches.
#include <algorithm>
#include <climits>
#include <cstring>
#include <new>
#include <numeric>
#include <stdexcept>

#include "internal.h"

namespace akv {

namespace {

struct Range { int64_t a, b; };

struct Stretch { int64_t tb, te; std::vector<int32_t> src; };

// Per key-tile summary used to classify tiles in O(1): every key j of a stretch
// is visible exactly to the queries in [start_j, drop_j), where start_j is j for
// own tokens and the stretch's first token for version rows.  Within one key
// tile these intervals overlap into one interval [lo, max_drop): for own keys
// every j lies inside its own interval and the keys are consecutive tokens; for
// version rows every interval starts at the stretch's first query.
struct KeyTile {
  int64_t lo;        // first query index that can see some key of the tile
  int64_t max_drop;  // one past the last such query
  int64_t min_drop;  // every key visible to all queries in [hi_start, min_drop)
  int64_t hi_start;  // largest start over the tile's keys
  bool complete;     // tile holds bk keys
};

}  // namespace

int build_plan(const akv_op* ops, int64_t n_ops, int32_t bq, int32_t bk, akv_plan** out) {
  if (!out) return fail(AKV_EINVAL, "akv_build_visibility: out is NULL");
  *out = nullptr;
  if (n_ops < 0 || (n_ops > 0 && !ops)) return fail(AKV_EINVAL, "akv_build_visibility: bad op array");
  if (bq < 1 || bk < 1 || bq > (1 << 20) || bk > (1 << 20))
    return fail(AKV_EINVAL, "akv_build_visibility: tile sizes must be in [1, 2^20]");

  // Validate and count tokens.
  int64_t T = 0;
  for (int64_t n = 0; n < n_ops; ++n) {
    const akv_op& op = ops[n];
    if (op.kind == AKV_OP_APPEND) {
      if (op.a < 0) return fail(AKV_EOPSEQ, "op " + std::to_string(n) + ": negative append");
      T += op.a;
      if (T > (int64_t)INT32_MAX - 1) return fail(AKV_EINVAL, "more than 2^31-2 tokens");
    } else if (op.kind == AKV_OP_DROP) {
      if (op.a < 0 || op.b < op.a || op.b > T)
        return fail(AKV_EOPSEQ, "op " + std::to_string(n) + ": drop range not yet appended");
    } else if (op.kind != AKV_OP_REPOS) {
      return fail(AKV_EOPSEQ, "op " + std::to_string(n) + ": unknown kind");
    }
  }

  akv_plan* p = new (std::nothrow) akv_plan;
  if (!p) return fail(AKV_ENOMEM, "plan allocation failed");
  try {
    p->bq = bq;
    p->bk = bk;
    p->T = T;
    p->tok_pos.resize(T);
    p->tok_drop.assign(T, INT32_MAX);

    std::vector<Range> live;            // ascending, disjoint
    int64_t n_live = 0, t = 0, next_pos = 0;
    std::vector<int64_t> cuts;          // token indices of op boundaries
    std::vector<Stretch> stretches;
    Stretch cur{0, 0, {}};
    int64_t pairs = 0;

    auto live_tokens = [&](std::vector<int32_t>& dst) {
      dst.clear();
      dst.reserve(n_live);
      for (const Range& r : live)
        for (int64_t j = r.a; j < r.b; ++j) dst.push_back((int32_t)j);
    };

    for (int64_t n = 0; n < n_ops; ++n) {
      const akv_op& op = ops[n];
      if (op.kind == AKV_OP_APPEND) {
        const int64_t cnt = op.a;
        if (cnt == 0) continue;
        for (int64_t m = 0; m < cnt; ++m) p->tok_pos[t + m] = (int32_t)(next_pos + m);
        // the m-th new token (1-based) attends to the n_live earlier keys and to m tokens of its own run
        pairs += cnt * n_live + cnt * (cnt + 1) / 2;
        if (!live.empty() && live.back().b == t) live.back().b += cnt;
        else live.push_back({t, t + cnt});
        n_live += cnt;
        t += cnt;
        next_pos += cnt;
      } else if (op.kind == AKV_OP_DROP) {
        cuts.push_back(t);
        std::vector<Range> kept;
        kept.reserve(live.size() + 1);
        for (const Range& r : live) {
          const int64_t lo = std::max(r.a, op.a), hi = std::min(r.b, op.b);
          if (lo >= hi) { kept.push_back(r); continue; }
          for (int64_t j = lo; j < hi; ++j) p->tok_drop[j] = (int32_t)t;
          n_live -= hi - lo;
          if (r.a < lo) kept.push_back({r.a, lo});
          if (hi < r.b) kept.push_back({hi, r.b});
        }
        live.swap(kept);
      } else {  // REPOS
        cuts.push_back(t);
        if (t > cur.tb) { cur.te = t; stretches.push_back(std::move(cur)); }
        cur = Stretch{t, t, {}};
        live_tokens(cur.src);
        next_pos = n_live;
      }
    }
    if (t > cur.tb) { cur.te = t; stretches.push_back(cur); }
    p->visible_pairs = pairs;
    p->p_next = next_pos;

    // T7: final live tokens with their current positions.  Tokens appended after
    // the last repos keep their append position; older ones hold their rank in
    // that repos' renumbering (cur.src, ascending).
    live_tokens(p->final_tok);
    p->final_pos.resize(p->final_tok.size());
    for (size_t n = 0; n < p->final_tok.size(); ++n) {
      const int32_t j = p->final_tok[n];
      if (j >= cur.tb) {
        p->final_pos[n] = p->tok_pos[j];
      } else {
        auto it = std::lower_bound(cur.src.begin(), cur.src.end(), j);
        p->final_pos[n] = (int32_t)(it - cur.src.begin());
      }
    }

    // T3: segments between op boundaries; T4/T5: stretches and version rows.
    std::sort(cuts.begin(), cuts.end());
    cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
    {
      std::vector<int64_t> c{0};
      for (int64_t x : cuts) if (x > 0 && x < T) c.push_back(x);
      c.push_back(T);
      size_t s = 0;
      for (size_t n = 0; n + 1 < c.size(); ++n) {
        if (c[n + 1] <= c[n]) continue;
        while (s < stretches.size() && stretches[s].te <= c[n]) ++s;
        p->segments.insert(p->segments.end(), {(int32_t)c[n], (int32_t)c[n + 1], (int32_t)s});
      }
    }
    int64_t ver_total = 0;
    for (const Stretch& st : stretches) ver_total += (int64_t)st.src.size();
    if (ver_total > INT32_MAX) throw std::length_error("more than 2^31-1 version rows");
    p->versions.resize(3 * ver_total);
    {
      int64_t row = 0;
      for (const Stretch& st : stretches) {
        p->epochs.insert(p->epochs.end(), {(int32_t)st.tb, (int32_t)st.te, (int32_t)st.src.size(),
                                           (int32_t)row});
        int32_t* w = p->versions.data() + 3 * row;
        for (size_t v = 0; v < st.src.size(); ++v, w += 3) {
          w[0] = st.src[v];
          w[1] = p->tok_pos[st.src[v]];
          w[2] = (int32_t)v;
        }
        row += (int64_t)st.src.size();
      }
    }

    // T6: tile classes per (stretch, q-tile).
    std::vector<int32_t> desc;  // device item descriptors
    p->tile_ptr.push_back(0);
    std::vector<KeyTile> kts;
    int64_t ver_off = 0;
    for (size_t e = 0; e < stretches.size(); ++e) {
      const Stretch& st = stretches[e];
      const int64_t r = (int64_t)st.src.size();
      const int64_t own = st.te - st.tb;
      const int64_t nvt = (r + bk - 1) / bk, not_ = (own + bk - 1) / bk;
      kts.assign(nvt + not_, KeyTile{});
      for (int64_t kt = 0; kt < nvt + not_; ++kt) {
        KeyTile& K = kts[kt];
        K.max_drop = INT64_MIN;
        K.min_drop = INT64_MAX;
        int64_t k0, k1;
        if (kt < nvt) {
          k0 = kt * bk;
          k1 = std::min(r, k0 + bk);
          for (int64_t v = k0; v < k1; ++v) {
            const int64_t dd = p->tok_drop[st.src[v]];
            K.max_drop = std::max(K.max_drop, dd);
            K.min_drop = std::min(K.min_drop, dd);
          }
          K.lo = st.tb;
          K.hi_start = st.tb;
        } else {
          k0 = st.tb + (kt - nvt) * bk;
          k1 = std::min(st.te, k0 + bk);
          for (int64_t j = k0; j < k1; ++j) {
            const int64_t dd = p->tok_drop[j];
            K.max_drop = std::max(K.max_drop, dd);
            K.min_drop = std::min(K.min_drop, dd);
          }
          K.lo = k0;
          K.hi_start = k1 - 1;
        }
        K.complete = (k1 - k0) == bk;
      }
      const int64_t nqt = (own + bq - 1) / bq;
      for (int64_t qt = 0; qt < nqt; ++qt) {
        const int64_t i0 = st.tb + qt * bq, i1 = std::min(st.te, i0 + bq) - 1;
        const int64_t first = (int64_t)p->tiles.size();
        for (int64_t kt = 0; kt < nvt + not_; ++kt) {
          const KeyTile& K = kts[kt];
          if (K.lo > i1) break;                 // own tiles only grow from here on
          if (K.max_drop <= i0) continue;       // every key dropped before this q-tile
          const bool full = K.complete && K.hi_start <= i0 && K.min_drop > i1;
          p->tiles.push_back((int32_t)(kt * 4 + (full ? AKV_TILE_FULL : AKV_TILE_PARTIAL)));
          (full ? p->n_full : p->n_partial)++;
        }
        if ((int64_t)p->tiles.size() > INT32_MAX) throw std::length_error("too many tiles");
        p->items.insert(p->items.end(), {(int32_t)e, (int32_t)qt});
        p->tile_ptr.push_back((int32_t)p->tiles.size());
        desc.insert(desc.end(), {(int32_t)i0, (int32_t)(i1 + 1), (int32_t)st.tb, (int32_t)st.te,
                                 (int32_t)r, (int32_t)ver_off, (int32_t)first,
                                 (int32_t)p->tiles.size()});
      }
      ver_off += r;
    }
    const int64_t n_items = (int64_t)p->items.size() / 2;
    p->item_order.resize(n_items);
    std::iota(p->item_order.begin(), p->item_order.end(), 0);
    std::stable_sort(p->item_order.begin(), p->item_order.end(), [&](int32_t a, int32_t b) {
      return p->tile_ptr[a + 1] - p->tile_ptr[a] > p->tile_ptr[b + 1] - p->tile_ptr[b];
    });

    // Device image.  Version rows carry only (src, to); kernels read the source's
    // append position and drop boundary through tok_pos / tok_drop.
    const int64_t nv = ver_total;
    uint64_t off = 0;
    auto place = [&](uint64_t bytes) { uint64_t o = off; off += (bytes + 255) & ~uint64_t(255); return o; };
    p->off_tok_pos = place(4 * T);
    p->off_tok_drop = place(4 * T);
    p->off_ver_src = place(4 * nv);
    p->off_ver_to = place(4 * nv);
    p->off_item_desc = place(4 * desc.size());
    p->off_tiles = place(4 * p->tiles.size());
    p->off_order = place(4 * n_items);
    p->image_bytes = std::max<uint64_t>(off, 256);
    p->image.reset(new uint8_t[p->image_bytes]);   // padding between arrays is never read
    auto put = [&](uint64_t o, const std::vector<int32_t>& v) {
      if (!v.empty()) std::memcpy(p->image.get() + o, v.data(), 4 * v.size());
    };
    put(p->off_tok_pos, p->tok_pos);
    put(p->off_tok_drop, p->tok_drop);
    {
      int32_t* src = (int32_t*)(p->image.get() + p->off_ver_src);
      int32_t* to = (int32_t*)(p->image.get() + p->off_ver_to);
      for (int64_t v = 0; v < nv; ++v) {
        src[v] = p->versions[3 * v];
        to[v] = p->versions[3 * v + 2];
      }
    }
    put(p->off_item_desc, desc);
    put(p->off_tiles, p->tiles);
    put(p->off_order, p->item_order);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(AKV_ENOMEM, "host allocation failed while building the plan");
  } catch (const std::exception& ex) {
    delete p;
    return fail(AKV_EINVAL, ex.what());
  }
  *out = p;
  return AKV_OK;
}

}  // namespace akv
