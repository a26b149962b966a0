// Split-KV work planner: chunk-size search + longest-first assignment.
//
// Cost model, in token-equivalents of KV traffic (one token = one 1152-byte
// latent row in bf16): a chunk of n tokens costs n + kFixed + H (loading the
// request's H query rows, 1152 B each) and, when the request is cut, another
// 4H for its partial output (written, read back by the merge launch: 1 KiB of
// fp16 per head each way) and its share of that launch.
// For each candidate chunk size C (a multiple of the granularity) every
// request is cut into ceil(L / C) near-equal chunks; the chunks are assigned
// longest-first to the least-loaded worker (ties to the lower index) and the
// candidate with the smallest largest-load wins, ties going to fewer cuts.
// Everything depends only on the lengths, so the plan is deterministic.
#include "planner.h"

#include <algorithm>
#include <limits>
#include <cstdint>
#include <queue>
#include <utility>
#include <vector>

namespace mla {
namespace {

constexpr int64_t kFixed = 64;  // per-chunk start-up (pipeline fill, epilogue)

struct Piece {
  int32_t request;
  int32_t begin;
  int32_t end;
  int32_t nsplit;  // chunks of its request
  int64_t cost;
};

// Chunks of a request of L tokens for chunk size `chunk` (or `force` chunks):
// near-equal, with boundaries on multiples of gran; returns the count and the
// step between boundaries.
std::pair<int64_t, int64_t> cut_of(int64_t L, int64_t chunk, int32_t gran, int32_t force,
                                   int32_t max_splits) {
  int64_t n = 1;
  if (L > 0) {
    if (force > 0)
      n = std::min<int64_t>(force, (L + gran - 1) / gran);
    else
      n = (L + chunk - 1) / chunk;
    if (n < 1) n = 1;
    if (n > max_splits) n = max_splits;
  }
  int64_t step = (L + n - 1) / n;
  step = ((step + gran - 1) / gran) * gran;
  if (step <= 0) step = gran;
  n = L > 0 ? (L + step - 1) / step : 1;
  return {n, step};
}

int64_t piece_cost(int64_t tokens, int64_t n, int32_t heads) {
  return tokens + kFixed + heads + (n > 1 ? 4 * (int64_t)heads : 0);
}

// Pieces, total cost and largest piece of a cut, without building it: the
// candidate search skips cuts whose bound cannot beat what it has.
struct CutSummary {
  int64_t pieces = 0, total = 0, largest = 0;
};
CutSummary summarize(const std::vector<int64_t>& len, int64_t chunk, int32_t gran, int32_t heads,
                     int32_t max_splits) {
  CutSummary c;
  for (int64_t L : len) {
    const std::pair<int64_t, int64_t> ns = cut_of(L, chunk, gran, 0, max_splits);
    c.pieces += ns.first;
    c.total += L + ns.first * piece_cost(0, ns.first, heads);
    c.largest = std::max(c.largest, piece_cost(std::min(L, ns.second), ns.first, heads));
  }
  return c;
}

void cut_requests(const std::vector<int64_t>& len, int64_t chunk, int32_t gran, int32_t heads,
                  int32_t force, int32_t max_splits, std::vector<Piece>* pieces) {
  pieces->clear();
  for (size_t b = 0; b < len.size(); ++b) {
    const int64_t L = len[b];
    const std::pair<int64_t, int64_t> ns = cut_of(L, chunk, gran, force, max_splits);
    const int64_t n = ns.first, step = ns.second;
    for (int64_t k = 0; k < n; ++k) {
      Piece p;
      p.request = (int32_t)b;
      p.begin = (int32_t)std::min<int64_t>(L, k * step);
      p.end = (int32_t)std::min<int64_t>(L, (k + 1) * step);
      p.nsplit = (int32_t)n;
      p.cost = piece_cost(p.end - p.begin, n, heads);
      pieces->push_back(p);
    }
  }
}

// Longest-first assignment; returns the largest worker load.
int64_t assign(const std::vector<Piece>& pieces, int32_t workers, std::vector<int32_t>* owner) {
  std::vector<int32_t> order(pieces.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int32_t)i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return pieces[a].cost > pieces[b].cost; });
  typedef std::pair<int64_t, int32_t> Load;  // (load, worker)
  std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
  for (int32_t w = 0; w < workers; ++w) heap.push(Load(0, w));
  owner->assign(pieces.size(), -1);
  int64_t worst = 0;
  for (int32_t i : order) {
    Load top = heap.top();
    heap.pop();
    (*owner)[i] = top.second;
    top.first += pieces[i].cost;
    worst = std::max(worst, top.first);
    heap.push(top);
  }
  return worst;
}

// Improve a longest-first assignment (which leaves the busiest worker some
// 10% above the mean when each worker gets a few requests of very different
// lengths): while it helps, the busiest worker moves one of its pieces to, or
// swaps one with, the partner and pieces that lower the larger of the two
// loads the most.  Every step lowers the busiest load, or leaves it to a worker
// with a higher index among equals; the scan orders are fixed, so the result is
// deterministic.  Returns the largest worker load.
int64_t refine(const std::vector<Piece>& pieces, int32_t workers, int64_t bound,
               std::vector<int32_t>* owner) {
  std::vector<int64_t> load((size_t)workers, 0);
  std::vector<std::vector<int32_t>> items((size_t)workers);
  for (size_t i = 0; i < pieces.size(); ++i) {
    load[(*owner)[i]] += pieces[i].cost;
    items[(*owner)[i]].push_back((int32_t)i);
  }
  // workers by (load, index), kept sorted: a step changes two loads
  auto before = [&](int32_t x, int32_t y) { return load[x] < load[y] || (load[x] == load[y] && x < y); };
  std::vector<int32_t> by_load((size_t)workers);
  for (int32_t w = 0; w < workers; ++w) by_load[w] = w;
  std::sort(by_load.begin(), by_load.end(), before);
  auto unlink = [&](int32_t w) {
    by_load.erase(std::lower_bound(by_load.begin(), by_load.end(), w, before));
  };
  auto relink = [&](int32_t w) {
    by_load.insert(std::lower_bound(by_load.begin(), by_load.end(), w, before), w);
  };
  const int64_t max_steps = 4 * (int64_t)workers;
  for (int64_t step = 0; step < max_steps; ++step) {
    const int32_t hi = by_load[workers - 1];
    if (load[hi] <= bound) break;  // no assignment does better
    int64_t best = load[hi];
    int32_t best_a = -1, best_b = -1, best_w = -1;
    for (int32_t k = 0; k < workers - 1; ++k) {
      const int32_t lo = by_load[k];
      const int64_t gap = load[hi] - load[lo];
      // no exchange with lo (or anyone heavier) can bring the pair below the
      // mean of their loads
      if (gap <= 0 || (load[hi] + load[lo] + 1) / 2 >= best) break;
      for (int32_t a : items[hi]) {
        const int64_t ca = pieces[a].cost;
        if (ca < gap) {  // move a
          const int64_t m = std::max(load[hi] - ca, load[lo] + ca);
          if (m < best) best = m, best_a = a, best_b = -1, best_w = lo;
        }
        for (int32_t b : items[lo]) {  // swap a and b
          const int64_t d = ca - pieces[b].cost;
          if (d <= 0 || d >= gap) continue;
          const int64_t m = std::max(load[hi] - d, load[lo] + d);
          if (m < best) best = m, best_a = a, best_b = b, best_w = lo;
        }
      }
    }
    if (best_a < 0) break;
    unlink(hi);
    unlink(best_w);
    auto take = [&](int32_t w, int32_t i) {
      items[w].erase(std::find(items[w].begin(), items[w].end(), i));
      load[w] -= pieces[i].cost;
    };
    auto put = [&](int32_t w, int32_t i) {
      items[w].push_back(i);
      load[w] += pieces[i].cost;
      (*owner)[i] = w;
    };
    take(hi, best_a);
    put(best_w, best_a);
    if (best_b >= 0) {
      take(best_w, best_b);
      put(hi, best_b);
    }
    relink(hi);
    relink(best_w);
  }
  return load[by_load[workers - 1]];
}

// Reorder workers so that the workers serving the hs rows of one request
// (the row groups that share its latent cache, with all their chunks) get
// launch positions congruent modulo the number of L2 domains: workgroups are
// dealt to XCDs round-robin in launch order, so they then share one L2.  The
// chunks of one row read the same query rows, which then cross HBM once per
// domain rather than once per chunk (the L2 merges the misses of the chunks'
// concurrent loads of Q; L2s of different domains do not share lines).
// Workers are sorted by the first row they serve and the domains are filled
// one after the other (domain d takes sorted workers d * per .. d * per + per - 1,
// per = used / xcds, at positions d, d + xcds, d + 2 xcds, ...), so a request
// is split over two domains only where it straddles such a boundary.  Only
// applied when the worker count divides evenly; it is a placement heuristic and
// never affects results.
void xcd_colocate(const std::vector<Piece>& pieces, const std::vector<int32_t>& owner,
                  int32_t xcds, int32_t used, std::vector<int32_t>* remap) {
  if (xcds < 2 || used % xcds != 0) return;
  std::vector<int32_t> first_row((size_t)used, std::numeric_limits<int32_t>::max());
  for (size_t i = 0; i < pieces.size(); ++i) {
    const int32_t w = (*remap)[owner[i]];
    first_row[w] = std::min(first_row[w], pieces[i].request);
  }
  std::vector<int32_t> order((size_t)used);
  for (int32_t w = 0; w < used; ++w) order[w] = w;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return first_row[x] < first_row[y]; });
  const int32_t per = used / xcds;
  std::vector<int32_t> pos((size_t)used);
  for (int32_t i = 0; i < used; ++i) pos[order[i]] = (i / per) + xcds * (i % per);
  for (auto& r : *remap)
    if (r >= 0) r = pos[r];
}

}  // namespace

int64_t max_segments(int32_t batch, const PlanParams& p) {
  const int64_t rows = (int64_t)batch * std::max(1, p.head_split);
  if (p.force_splits > 0) return rows * std::min(p.force_splits, p.max_splits);
  return rows + 2 * (int64_t)p.num_workers;
}

int64_t max_partials(int32_t batch, const PlanParams& p) { return max_segments(batch, p); }

int32_t build_plan(const int32_t* kv_indptr, const int32_t* kv_last_page_len, int32_t batch,
                   const PlanParams& p, Plan* out) {
  if (!kv_indptr || !kv_last_page_len || !out || batch < 0 || p.num_workers <= 0 ||
      p.granularity <= 0 || p.page_size <= 0 || p.num_heads <= 0 || p.max_splits < 1 ||
      p.head_split < 1)
    return -1;
  if (kv_indptr[0] != 0) return -1;
  const int32_t hs = p.head_split;
  std::vector<int64_t> len((size_t)batch * hs);
  int64_t max_len = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
    if (n < 0) return -1;
    if (n == 0) {
      len[b] = 0;
      continue;
    }
    const int32_t last = kv_last_page_len[b];
    if (last < 1 || last > p.page_size) return -1;
    len[b] = (n - 1) * p.page_size + last;
    if (len[b] > INT32_MAX) return -1;
    max_len = std::max(max_len, len[b]);
  }
  // sub-requests g of request b are rows b * hs + g (lengths copied, last first)
  for (int64_t r = (int64_t)batch * hs - 1; r >= 0; --r) len[r] = len[r / hs];
  const int32_t rows = batch * hs;

  const int32_t gran = p.granularity;
  const int64_t seg_cap = max_segments(batch, p);
  std::vector<Piece> pieces, best_pieces;
  std::vector<int32_t> owner, best_owner;
  int64_t best = -1;

  if (p.force_splits > 0) {
    cut_requests(len, 0, gran, p.num_heads, p.force_splits, p.max_splits, &best_pieces);
    assign(best_pieces, p.num_workers, &best_owner);
  } else {
    // candidate chunk sizes: gran * {1, 2, 3, 4, 6, 8, 12, 16, ...} up to max_len
    std::vector<int64_t> cands;
    for (int64_t m = 1;; m *= 2) {
      cands.push_back(m * gran);
      if (m * gran >= max_len) break;
      if (m >= 2) {
        cands.push_back(m * gran * 3 / 2);
      }
    }
    std::sort(cands.begin(), cands.end(), std::greater<int64_t>());  // fewest cuts first
    // longest-first for every candidate; the refinement (the costly part) for
    // the two best of those.  A candidate's longest-first load is at least its
    // bound (the mean load, or its largest piece), so one whose bound exceeds
    // the second best load found so far cannot be among the two and is not
    // assigned; candidates with more pieces than the workspace holds are
    // skipped before they are cut.
    struct Ranked {
      int64_t worst, k, bound;
      std::vector<Piece> pieces;
      std::vector<int32_t> owner;
    };
    std::vector<Ranked> top;  // the two best so far, by (worst, candidate order)
    for (size_t k = 0; k < cands.size(); ++k) {
      const CutSummary cs = summarize(len, cands[k], gran, p.num_heads, p.max_splits);
      if (cs.pieces > seg_cap) continue;
      const int64_t bound = std::max((cs.total + p.num_workers - 1) / p.num_workers, cs.largest);
      if (top.size() == 2 && bound > top[1].worst) continue;
      cut_requests(len, cands[k], gran, p.num_heads, 0, p.max_splits, &pieces);
      const int64_t worst = assign(pieces, p.num_workers, &owner);
      Ranked r{worst, (int64_t)k, bound, pieces, owner};
      auto pos = std::upper_bound(top.begin(), top.end(), r, [](const Ranked& x, const Ranked& y) {
        return x.worst < y.worst;
      });
      top.insert(pos, std::move(r));
      if (top.size() > 2) top.pop_back();
    }
    if (top.empty()) return -1;  // unreachable: the largest candidate never cuts
    std::sort(top.begin(), top.end(),
              [](const Ranked& x, const Ranked& y) { return x.k < y.k; });  // fewest cuts first
    for (Ranked& r : top) {
      // refining cannot go below the bound: skip a candidate that cannot win
      if (best >= 0 && r.bound >= best) continue;
      const int64_t worst = refine(r.pieces, p.num_workers, r.bound, &r.owner);
      if (best < 0 || worst < best) {
        best = worst;
        best_pieces.swap(r.pieces);
        best_owner.swap(r.owner);
      }
    }
  }

  // group by worker, keep assignment order within a worker stable (request order)
  std::vector<int32_t> count((size_t)p.num_workers, 0);
  for (int32_t w : best_owner) ++count[w];
  std::vector<int32_t> remap((size_t)p.num_workers, -1);
  int32_t used = 0;
  for (int32_t w = 0; w < p.num_workers; ++w)
    if (count[w] > 0) remap[w] = used++;
  bool cut = false;
  for (const Piece& pc : best_pieces) cut = cut || pc.nsplit > 1;
  if (hs > 1 || cut) xcd_colocate(best_pieces, best_owner, p.xcd_count, used, &remap);
  out->batch = batch;
  out->num_workers = used;
  out->worker_ptr.assign((size_t)used + 1, 0);
  for (int32_t w = 0; w < p.num_workers; ++w)
    if (remap[w] >= 0) out->worker_ptr[remap[w] + 1] = count[w];
  for (int32_t w = 0; w < used; ++w) out->worker_ptr[w + 1] += out->worker_ptr[w];
  out->segments.assign(best_pieces.size(), Segment());
  std::vector<int32_t> fill(out->worker_ptr.begin(), out->worker_ptr.end() - 1);

  // partial slots: consecutive per split request, in token order (cut_requests
  // emits the pieces of a request consecutively, in token order)
  std::vector<int32_t> first_slot((size_t)rows, -1), first_piece((size_t)rows, -1);
  std::vector<int32_t> split_index((size_t)rows, -1);
  out->combine.clear();
  int32_t slots = 0;
  for (size_t i = 0; i < best_pieces.size(); ++i) {
    const Piece& pc = best_pieces[i];
    if (first_piece[pc.request] < 0) first_piece[pc.request] = (int32_t)i;
    if (pc.nsplit > 1 && first_slot[pc.request] < 0) {
      first_slot[pc.request] = slots;
      split_index[pc.request] = (int32_t)(out->combine.size() / 4);
      out->combine.push_back(pc.request);
      out->combine.push_back(slots);
      out->combine.push_back(pc.nsplit);
      out->combine.push_back(0);
      slots += pc.nsplit;
    }
  }
  out->num_partials = slots;
  for (size_t i = 0; i < best_pieces.size(); ++i) {
    const Piece& pc = best_pieces[i];
    Segment s;
    s.request = pc.request;
    s.begin = pc.begin;
    s.end = pc.end;
    s.slot = pc.nsplit > 1 ? first_slot[pc.request] + ((int32_t)i - first_piece[pc.request]) : -1;
    s.split_request = split_index[pc.request];
    s.first_slot = first_slot[pc.request];
    s.num_splits = pc.nsplit;
    s.last = (i + 1 == best_pieces.size() || best_pieces[i + 1].request != pc.request) ? 1 : 0;
    const int32_t w = remap[best_owner[i]];
    out->segments[fill[w]++] = s;
  }
  return 0;
}

}  // namespace mla
