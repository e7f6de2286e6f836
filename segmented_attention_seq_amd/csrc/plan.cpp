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
#include <thread>

#include "internal.h"

namespace akv {

namespace {

struct Range { int64_t a, b; };

// A repos stretch: its own tokens [tb, te) and the keys active after its repos,
// kept as the live range list (ascending) with their count r; version row v is
// the v-th token of those ranges.
struct Stretch {
  int64_t tb, te;
  std::vector<Range> src;
  int64_t r;
};

// Host threads for the plan build (the tables are filled at precomputed offsets,
// so the result does not depend on the split).
int plan_threads() {
  static const int n = [] {
    const unsigned h = std::thread::hardware_concurrency();
    return (int)std::max(1u, std::min(16u, h));
  }();
  return n;
}

// f(lo, hi) over [0, n) in contiguous chunks of at least `grain`, one per thread.
template <class F>
void par_for(int64_t n, int64_t grain, const F& f) {
  if (n <= 0) return;
  const int64_t P = std::min<int64_t>(plan_threads(), (n + grain - 1) / grain);
  if (P <= 1) { f(0, n); return; }
  std::vector<std::thread> th;
  th.reserve(P - 1);
  for (int64_t k = 1; k < P; ++k) th.emplace_back([&f, n, k, P] { f(n * k / P, n * (k + 1) / P); });
  f(0, n / P);
  for (auto& x : th) x.join();
}

// Source tokens of version rows [v0, v1) of a stretch, in order: cb(v, token).
template <class CB>
void for_version_rows(const Stretch& st, const std::vector<int64_t>& pre, int64_t v0, int64_t v1, const CB& cb) {
  // pre[i] = number of version rows before range i
  size_t i = std::upper_bound(pre.begin(), pre.end(), v0) - pre.begin() - 1;
  int64_t v = v0;
  while (v < v1) {
    const Range& rg = st.src[i];
    const int64_t end = std::min(v1, pre[i] + (rg.b - rg.a));
    for (int64_t j = rg.a + (v - pre[i]); v < end; ++v, ++j) cb(v, j);
    ++i;
  }
}

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
    Stretch cur{0, 0, {}, 0};
    int64_t pairs = 0;

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
        cur = Stretch{t, t, live, n_live};
        next_pos = n_live;
      }
    }
    if (t > cur.tb) { cur.te = t; stretches.push_back(cur); }
    p->visible_pairs = pairs;
    p->p_next = next_pos;

    // T7: final live tokens with their current positions.  Tokens appended after
    // the last repos keep their append position; older ones hold their rank in
    // that repos' renumbering (the ranges of cur.src, ascending).
    {
      p->final_tok.resize(n_live);
      p->final_pos.resize(n_live);
      std::vector<int64_t> pre(cur.src.size() + 1, 0);
      for (size_t i = 0; i < cur.src.size(); ++i) pre[i + 1] = pre[i] + (cur.src[i].b - cur.src[i].a);
      int64_t n = 0;
      size_t i = 0;
      for (const Range& r : live)
        for (int64_t j = r.a; j < r.b; ++j, ++n) {
          p->final_tok[n] = (int32_t)j;
          if (j >= cur.tb) {
            p->final_pos[n] = p->tok_pos[j];
          } else {
            while (cur.src[i].b <= j) ++i;  // live tokens are ascending, so is i
            p->final_pos[n] = (int32_t)(pre[i] + (j - cur.src[i].a));
          }
        }
    }

    // T3: segments between op boundaries.
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

    // Layout of everything per stretch: version rows, key tiles, items (q-tiles).
    const int64_t S = (int64_t)stretches.size();
    std::vector<int64_t> vrow(S + 1, 0), ktile(S + 1, 0), item(S + 1, 0);
    std::vector<std::vector<int64_t>> rpre(S);  // per stretch: version rows before each range
    for (int64_t e = 0; e < S; ++e) {
      const Stretch& st = stretches[e];
      rpre[e].assign(st.src.size() + 1, 0);
      for (size_t i = 0; i < st.src.size(); ++i) rpre[e][i + 1] = rpre[e][i] + (st.src[i].b - st.src[i].a);
      const int64_t own = st.te - st.tb;
      vrow[e + 1] = vrow[e] + st.r;
      ktile[e + 1] = ktile[e] + (st.r + bk - 1) / bk + (own + bk - 1) / bk;
      item[e + 1] = item[e] + (own + bq - 1) / bq;
    }
    const int64_t ver_total = vrow[S], n_ktiles = ktile[S], n_items = item[S];
    if (ver_total > INT32_MAX) throw std::length_error("more than 2^31-1 version rows");
    for (int64_t e = 0; e < S; ++e)
      p->epochs.insert(p->epochs.end(), {(int32_t)stretches[e].tb, (int32_t)stretches[e].te,
                                         (int32_t)stretches[e].r, (int32_t)vrow[e]});
    auto stretch_of = [](const std::vector<int64_t>& off, int64_t x) {
      return (int64_t)(std::upper_bound(off.begin(), off.end(), x) - off.begin()) - 1;
    };

    // T6, pass 1: per key tile, the interval summary (KeyTile).  Every key j of a
    // stretch is visible exactly to the queries in [start_j, drop_j).
    std::vector<KeyTile> kts(n_ktiles);
    par_for(n_ktiles, 256, [&](int64_t lo, int64_t hi) {
      int64_t e = stretch_of(ktile, lo);
      for (int64_t g = lo; g < hi; ++g) {
        while (ktile[e + 1] <= g) ++e;
        const Stretch& st = stretches[e];
        const int64_t nvt = (st.r + bk - 1) / bk, kt = g - ktile[e];
        KeyTile& K = kts[g];
        K.max_drop = INT64_MIN;
        K.min_drop = INT64_MAX;
        int64_t k0, k1;
        auto see = [&](int64_t, int64_t j) {
          const int64_t dd = p->tok_drop[j];
          K.max_drop = std::max(K.max_drop, dd);
          K.min_drop = std::min(K.min_drop, dd);
        };
        if (kt < nvt) {
          k0 = kt * bk;
          k1 = std::min(st.r, k0 + bk);
          for_version_rows(st, rpre[e], k0, k1, see);
          K.lo = st.tb;
          K.hi_start = st.tb;
        } else {
          k0 = st.tb + (kt - nvt) * bk;
          k1 = std::min(st.te, k0 + bk);
          for (int64_t j = k0; j < k1; ++j) see(0, j);
          K.lo = k0;
          K.hi_start = k1 - 1;
        }
        K.complete = (k1 - k0) == bk;
      }
    });

    // T6, pass 2: visit the non-empty key tiles of each item (stretch, q-tile);
    // emit(kt, full) is called in key-tile order.
    auto visit_item = [&](int64_t it, int64_t& e, const auto& emit) {
      while (item[e + 1] <= it) ++e;
      const Stretch& st = stretches[e];
      const int64_t nk = ktile[e + 1] - ktile[e];
      const int64_t qt = it - item[e];
      const int64_t i0 = st.tb + qt * bq, i1 = std::min(st.te, i0 + bq) - 1;
      const KeyTile* kk = kts.data() + ktile[e];
      for (int64_t kt = 0; kt < nk; ++kt) {
        const KeyTile& K = kk[kt];
        if (K.lo > i1) break;                 // own tiles only grow from here on
        if (K.max_drop <= i0) continue;       // every key dropped before this q-tile
        emit(kt, K.complete && K.hi_start <= i0 && K.min_drop > i1);
      }
    };
    std::vector<int64_t> cnt(n_items + 1, 0), nfull(n_items, 0);
    par_for(n_items, 16, [&](int64_t lo, int64_t hi) {
      int64_t e = stretch_of(item, lo);
      for (int64_t it = lo; it < hi; ++it) {
        int64_t c = 0, f = 0;
        visit_item(it, e, [&](int64_t, bool full) { ++c; f += full; });
        cnt[it + 1] = c;
        nfull[it] = f;
      }
    });
    p->n_full = 0;
    for (int64_t it = 0; it < n_items; ++it) {
      cnt[it + 1] += cnt[it];
      p->n_full += nfull[it];
    }
    const int64_t n_tiles = cnt[n_items];
    if (n_tiles > INT32_MAX) throw std::length_error("too many tiles");
    p->n_partial = n_tiles - p->n_full;

    // T5 version rows (src, its append position, row index).
    p->versions.resize(3 * ver_total);
    par_for(ver_total, 4096, [&](int64_t lo, int64_t hi) {
      int64_t e = stretch_of(vrow, lo);
      int64_t v = lo;
      while (v < hi) {
        while (vrow[e + 1] <= v) ++e;
        const int64_t b = vrow[e], end = std::min(hi, vrow[e + 1]);
        for_version_rows(stretches[e], rpre[e], v - b, end - b, [&](int64_t vv, int64_t j) {
          int32_t* w = p->versions.data() + 3 * (b + vv);
          w[0] = (int32_t)j;
          w[1] = p->tok_pos[j];
          w[2] = (int32_t)vv;
        });
        v = end;
      }
    });

    // Runs of version rows that move by one shift (row index - append position):
    // a run starts at a stretch's first version row and wherever the shift changes.
    // Consecutive surviving tokens of one append keep consecutive positions, so a
    // stretch has few runs (a table of per-run rotations serves all its rows).
    {
      auto shift = [&](int64_t v) { return p->versions[3 * v + 2] - p->versions[3 * v + 1]; };
      auto starts = [&](int64_t v) { return p->versions[3 * v + 2] == 0 || shift(v) != shift(v - 1); };
      const int64_t nch = std::max<int64_t>(1, std::min<int64_t>(256, (ver_total + 16383) / 16384));
      std::vector<int64_t> cbase(nch + 1, 0);
      par_for(nch, 1, [&](int64_t lo, int64_t hi) {
        for (int64_t c = lo; c < hi; ++c) {
          int64_t k = 0;
          for (int64_t v = ver_total * c / nch; v < ver_total * (c + 1) / nch; ++v) k += starts(v);
          cbase[c + 1] = k;
        }
      });
      for (int64_t c = 0; c < nch; ++c) cbase[c + 1] += cbase[c];
      p->n_runs = cbase[nch];
      if (p->n_runs > INT32_MAX) throw std::length_error("too many version runs");
      p->ver_run.resize(ver_total);
      p->run_delta.resize(p->n_runs);
      par_for(nch, 1, [&](int64_t lo, int64_t hi) {
        for (int64_t c = lo; c < hi; ++c) {
          int64_t id = cbase[c] - 1;
          for (int64_t v = ver_total * c / nch; v < ver_total * (c + 1) / nch; ++v) {
            if (starts(v)) p->run_delta[++id] = shift(v);
            p->ver_run[v] = (int32_t)id;
          }
        }
      });
    }

    // Device image layout.  Version rows carry only (src, to, run); kernels read the
    // source's append position and drop boundary through tok_pos / tok_drop.  The
    // src and run tables are followed by kVerPad zero entries: the fused attention
    // loads them eight rows at a time from a tile's first row, past a ragged last
    // tile's end.
    uint64_t off = 0;
    auto place = [&](uint64_t bytes) { uint64_t o = off; off += (bytes + 255) & ~uint64_t(255); return o; };
    p->off_tok_pos = place(4 * T);
    p->off_tok_drop = place(4 * T);
    constexpr uint64_t kVerPad = 64;
    p->off_ver_src = place(4 * ((uint64_t)ver_total + kVerPad));
    p->off_ver_to = place(4 * ver_total);
    p->off_ver_run = place(4 * ((uint64_t)ver_total + kVerPad));
    p->off_run_delta = place(4 * (uint64_t)p->n_runs);
    p->off_item_desc = place(4 * (uint64_t)n_items * ID_WORDS);
    p->off_tiles = place(4 * (uint64_t)n_tiles);
    p->off_order = place(4 * (uint64_t)n_items);
    p->image_bytes = std::max<uint64_t>(off, 256);
    p->image.reset(new uint8_t[p->image_bytes]);   // padding between arrays is never read
    int32_t* img_src = (int32_t*)(p->image.get() + p->off_ver_src);
    int32_t* img_to = (int32_t*)(p->image.get() + p->off_ver_to);
    int32_t* img_desc = (int32_t*)(p->image.get() + p->off_item_desc);
    int32_t* img_tiles = (int32_t*)(p->image.get() + p->off_tiles);
    par_for(ver_total, 1 << 15, [&](int64_t lo, int64_t hi) {
      for (int64_t v = lo; v < hi; ++v) {
        img_src[v] = p->versions[3 * v];
        img_to[v] = p->versions[3 * v + 2];
      }
      std::memcpy(p->image.get() + p->off_ver_run + 4 * lo, p->ver_run.data() + lo, 4 * (hi - lo));
    });
    if (p->n_runs) std::memcpy(p->image.get() + p->off_run_delta, p->run_delta.data(), 4 * p->n_runs);
    std::memset(p->image.get() + p->off_ver_src + 4 * ver_total, 0, 4 * kVerPad);
    std::memset(p->image.get() + p->off_ver_run + 4 * ver_total, 0, 4 * kVerPad);

    // T6 tile lists, items and item descriptors.
    p->tiles.resize(n_tiles);
    p->items.resize(2 * n_items);
    p->tile_ptr.resize(n_items + 1);
    par_for(n_items, 16, [&](int64_t lo, int64_t hi) {
      int64_t e = stretch_of(item, lo);
      for (int64_t it = lo; it < hi; ++it) {
        int64_t w = cnt[it];
        visit_item(it, e, [&](int64_t kt, bool f) {
          const int32_t x = (int32_t)(kt * 4 + (f ? AKV_TILE_FULL : AKV_TILE_PARTIAL));
          p->tiles[w] = x;
          img_tiles[w] = x;
          ++w;
        });
        const Stretch& st = stretches[e];
        const int64_t qt = it - item[e];
        const int64_t i0 = st.tb + qt * bq, i1 = std::min(st.te, i0 + bq);
        p->items[2 * it] = (int32_t)e;
        p->items[2 * it + 1] = (int32_t)qt;
        p->tile_ptr[it] = (int32_t)cnt[it];
        int32_t* d = img_desc + it * ID_WORDS;
        d[ID_QBEGIN] = (int32_t)i0;
        d[ID_QEND] = (int32_t)i1;
        d[ID_TB] = (int32_t)st.tb;
        d[ID_TE] = (int32_t)st.te;
        d[ID_R] = (int32_t)st.r;
        d[ID_VEROFF] = (int32_t)vrow[e];
        d[ID_TILE0] = (int32_t)cnt[it];
        d[ID_TILE1] = (int32_t)cnt[it + 1];
      }
    });
    p->tile_ptr[n_items] = (int32_t)n_tiles;

    // Work order: stretch by stretch, the stretch with the longest item first (ties
    // in stretch order), and within a stretch its items longest first (stable).  The
    // workgroups an XCD runs at once then mostly belong to one stretch and walk the
    // same K/V tiles, so more of those reads hit its L2; the order ends with the
    // shortest items of the stretch whose items are shortest, which keeps the tail
    // of the launch short.
    p->item_order.resize(n_items);
    std::iota(p->item_order.begin(), p->item_order.end(), 0);
    {
      std::vector<int64_t> work(S, 0);
      std::vector<int32_t> st_of(n_items);
      for (int64_t e = 0; e < S; ++e) {
        for (int64_t it = item[e]; it < item[e + 1]; ++it) {
          st_of[it] = (int32_t)e;
          work[e] = std::max<int64_t>(work[e], cnt[it + 1] - cnt[it]);
        }
      }
      std::stable_sort(p->item_order.begin(), p->item_order.end(), [&](int32_t a, int32_t b) {
        const int32_t ea = st_of[a], eb = st_of[b];
        if (ea != eb) return work[ea] != work[eb] ? work[ea] > work[eb] : ea < eb;
        return cnt[a + 1] - cnt[a] > cnt[b + 1] - cnt[b];
      });
    }

    // Remaining image arrays.
    par_for(T, 1 << 16, [&](int64_t lo, int64_t hi) {
      std::memcpy(p->image.get() + p->off_tok_pos + 4 * lo, p->tok_pos.data() + lo, 4 * (hi - lo));
      std::memcpy(p->image.get() + p->off_tok_drop + 4 * lo, p->tok_drop.data() + lo, 4 * (hi - lo));
    });
    if (n_items) std::memcpy(p->image.get() + p->off_order, p->item_order.data(), 4 * n_items);
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
