// Sharding planner of FlashCP (host only): Algorithm 1 of section 3.4, with
// Whole-Doc sharding (section 3.3) for most documents and Per-Doc sharding
// (section 2.3) for the longest ones when the workload ratio needs it.
//
// Quantities: a shard with prefix p and length s costs W = (2p + s + 1) s / 2
// (section 3.1); a worker's load is the sum over its shards, Per-Doc pieces
// included; the ratio is max load / mean load (1 without work).  The loop:
//   1. documents by decreasing length (ties: document order), empty ones skipped;
//   2. Whole-Doc plan from scratch: each remaining document whole to the
//      least-loaded worker (ties: lowest index);
//   3. equal tokens (Eq. 2): worker j's Whole-Doc target is its share of all
//      tokens (T div N, one more for the first T mod N workers) minus what its
//      Per-Doc pieces hold; if that is negative anywhere, the Whole-Doc tokens
//      are split evenly instead.  While a worker is above its target, the one
//      furthest above (ties: lowest index) gives back its most recently added
//      shards until it is not; each given-back shard goes to the least-loaded
//      worker below its target, its head as large as that worker lacks, the
//      rest onward to the next such worker;
//   4. if the ratio exceeds R and Whole-Doc documents remain, the longest of
//      them moves to Per-Doc sharding (pieces i and 2N-1-i, piece i = local
//      rows [floor(i L / 2N), floor((i+1) L / 2N))) and the loop repeats.
// Loads are exact 64-bit integers; the ratio is one rounding of an exact
// quotient's operands, so the comparison with R is reproducible.
#include "docmask.h"

#include <algorithm>
#include <cmath>
#include <vector>

namespace {

struct Shard {
  int32_t doc;
  int64_t p;
  int64_t s;
};

inline int64_t workload(int64_t p, int64_t s) { return (2 * p + s + 1) * s / 2; }

// pieces j and 2N-1-j of a document of length L: (p, s) pairs, empty ones dropped
void per_doc_pieces(int64_t L, int32_t n, int32_t j, std::vector<std::pair<int64_t, int64_t>>& out) {
  out.clear();
  const int64_t parts = 2 * (int64_t)n;
  for (int64_t i : {(int64_t)j, parts - 1 - j}) {
    const int64_t a = i * L / parts, b = (i + 1) * L / parts;
    if (b > a) out.emplace_back(a, b - a);
  }
}

double ratio_of(const std::vector<int64_t>& load) {
  int64_t mx = 0, tot = 0;
  for (int64_t x : load) {
    mx = std::max(mx, x);
    tot += x;
  }
  if (tot == 0) return 1.0;
  const unsigned __int128 num = (unsigned __int128)mx * (unsigned __int128)load.size();
  return (double)num / (double)tot;
}

struct Plan {
  std::vector<int32_t> per_doc;                 // document ids, in the order they left
  std::vector<std::vector<Shard>> whole;        // per worker, in the order shards were added
  double ratio = 1.0;
};

Plan make_plan(const int32_t* len, int32_t n_docs, int32_t n, double r_target) {
  std::vector<int32_t> order;
  for (int32_t i = 0; i < n_docs; ++i)
    if (len[i] > 0) order.push_back(i);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return len[a] > len[b]; });

  Plan plan;
  std::vector<int64_t> pd_load(n, 0), pd_tokens(n, 0);
  std::vector<std::pair<int64_t, int64_t>> pcs;
  int64_t pd_total = 0;
  size_t k = 0;                                 // order[0, k) are Per-Doc
  for (;;) {
    std::vector<std::vector<Shard>> tmp(n);
    std::vector<int64_t> load = pd_load, tokens(n, 0);
    for (size_t i = k; i < order.size(); ++i) {           // least-loaded worker takes the whole document
      int32_t w = 0;
      for (int32_t j = 1; j < n; ++j)
        if (load[j] < load[w]) w = j;
      tmp[w].push_back(Shard{order[i], 0, len[order[i]]});
      load[w] += workload(0, len[order[i]]);
      tokens[w] += len[order[i]];
    }
    int64_t tw = 0;
    for (int64_t t : tokens) tw += t;
    const int64_t total = tw + pd_total;
    std::vector<int64_t> target(n);
    bool feasible = true;
    for (int32_t j = 0; j < n; ++j) {
      target[j] = total / n + (j < total % n ? 1 : 0) - pd_tokens[j];
      feasible = feasible && target[j] >= 0;
    }
    if (!feasible)
      for (int32_t j = 0; j < n; ++j) target[j] = tw / n + (j < tw % n ? 1 : 0);
    for (;;) {                                            // equal tokens
      int32_t a = 0;
      for (int32_t j = 1; j < n; ++j)
        if (tokens[j] - target[j] > tokens[a] - target[a]) a = j;
      if (tokens[a] <= target[a]) break;                  // nobody above target: all equal (sums agree)
      std::vector<Shard> back;
      while (tokens[a] > target[a]) {
        const Shard sh = tmp[a].back();
        tmp[a].pop_back();
        tokens[a] -= sh.s;
        load[a] -= workload(sh.p, sh.s);
        back.push_back(sh);
      }
      for (Shard sh : back) {
        while (sh.s > 0) {
          int32_t b = -1;
          for (int32_t j = 0; j < n; ++j)
            if (tokens[j] < target[j] && (b < 0 || load[j] < load[b])) b = j;
          const int64_t take = std::min(sh.s, target[b] - tokens[b]);
          tmp[b].push_back(Shard{sh.doc, sh.p, take});
          tokens[b] += take;
          load[b] += workload(sh.p, take);
          sh.p += take;
          sh.s -= take;
        }
      }
    }
    const double r = ratio_of(load);
    if (r > r_target && k < order.size()) {               // the longest remaining document goes Per-Doc
      const int32_t d = order[k++];
      plan.per_doc.push_back(d);
      pd_total += len[d];
      for (int32_t j = 0; j < n; ++j) {
        per_doc_pieces(len[d], n, j, pcs);
        for (const auto& pc : pcs) {
          pd_load[j] += workload(pc.first, pc.second);
          pd_tokens[j] += pc.second;
        }
      }
      continue;
    }
    plan.whole = std::move(tmp);
    plan.ratio = r;
    return plan;
  }
}

}  // namespace

extern "C" {

int docmask_plan_shards(const int32_t* doc_lengths, int32_t n_docs, int32_t n_workers, double target_ratio,
                        docmask_chunk* chunks, int32_t max_chunks, int32_t* worker_n_chunks, int32_t* per_doc,
                        int32_t* n_per_doc, double* ratio) {
  if (n_docs < 0 || (n_docs > 0 && !doc_lengths) || n_workers < 1 || !worker_n_chunks || !n_per_doc || !ratio)
    return DOCMASK_EINVAL;
  if (!std::isfinite(target_ratio) || target_ratio < 1.0) return DOCMASK_EINVAL;
  int64_t total = 0;
  for (int32_t i = 0; i < n_docs; ++i) {
    if (doc_lengths[i] < 0) return DOCMASK_EINVAL;
    total += doc_lengths[i];
  }
  if (total > INT32_MAX) return DOCMASK_EINVAL;
  const Plan plan = make_plan(doc_lengths, n_docs, n_workers, target_ratio);

  std::vector<int64_t> start(n_docs + 1, 0);
  for (int32_t i = 0; i < n_docs; ++i) start[i + 1] = start[i] + doc_lengths[i];
  std::vector<std::pair<int64_t, int64_t>> pcs;
  std::vector<docmask_chunk> out;
  for (int32_t j = 0; j < n_workers; ++j) {
    std::vector<std::pair<int64_t, int64_t>> segs;
    for (const Shard& sh : plan.whole[j]) segs.emplace_back(start[sh.doc] + sh.p, sh.s);
    for (int32_t d : plan.per_doc) {
      per_doc_pieces(doc_lengths[d], n_workers, j, pcs);
      for (const auto& pc : pcs) segs.emplace_back(start[d] + pc.first, pc.second);
    }
    std::sort(segs.begin(), segs.end());
    int32_t cnt = 0;
    for (const auto& sg : segs) {
      if (cnt > 0 && (int64_t)out.back().g_start + out.back().len == sg.first) {
        out.back().len += (int32_t)sg.second;
      } else {
        out.push_back(docmask_chunk{(int32_t)sg.first, (int32_t)sg.second});
        ++cnt;
      }
    }
    worker_n_chunks[j] = cnt;
  }
  *n_per_doc = (int32_t)plan.per_doc.size();
  *ratio = plan.ratio;
  if (per_doc) {
    std::vector<int32_t> ids = plan.per_doc;
    std::sort(ids.begin(), ids.end());
    std::copy(ids.begin(), ids.end(), per_doc);
  }
  if (chunks) {
    if (max_chunks < (int32_t)out.size()) return DOCMASK_EINVAL;
    std::copy(out.begin(), out.end(), chunks);
  }
  return DOCMASK_OK;
}

}  // extern "C"
