"""Reference for FlashCP's heuristic sharding (Algorithm 1, section 3.4) with
Whole-Doc sharding (section 3.3) and Per-Doc sharding (section 2.3).

Test infrastructure only (see the package docstring).

The pages give the loop; the two plan operations it names are left open and
are read here as follows (every reading is also stated where it is used):

* workload of a shard with prefix p and length s: W = (2p + s + 1) s / 2
  (section 3.1), exact integers; a worker's load is the sum over its shards,
  Per-Doc shares included; imbalance ratio = max load / mean load (1 when
  there is no work);
* "Min Worker Add(d)": the whole document goes to the worker with the
  smallest load, ties to the lowest index;
* equal tokens (Eq. 2): worker j's share of all T tokens is T div N, plus one
  for the first (T mod N) workers; its Whole-Doc target is that share minus
  the tokens its Per-Doc pieces hold (pieces i and 2N-1-i of every Per-Doc
  document, piece i = local rows [floor(i L / 2N), floor((i+1) L / 2N))).
  When a target would be negative, the Whole-Doc tokens are instead split
  as evenly as integers allow, the first workers one more;
* "Max Token Worker Pop()": the worker furthest above its token target (ties
  to the lowest index) gives back its most recently added shards until it is
  at or below its target;
* "Whole Doc Shard and Add(docs)": each given-back shard goes, in the order
  given back, to the least-loaded worker still below its target (ties to the
  lowest index); if it does not fit there, its head (the first tokens, as many
  as that worker lacks) stays there as a shard and the rest continues to the
  next such worker.  Only heads are ever cut off, so only those travel (the
  pages' "lower segments", volume bounded by the largest cut);
* the longest remaining document leaves for Per-Doc sharding while the ratio
  exceeds R and Whole-Doc documents remain.
"""
from __future__ import annotations


def shard_workload(p: int, s: int) -> int:
    """W = (2p + s + 1) s / 2 (section 3.1)."""
    return (2 * p + s + 1) * s // 2


def per_doc_pieces(length: int, n: int, j: int):
    """[(p, s)] pieces j and 2N-1-j of a document of the given length."""
    b = [(i * length) // (2 * n) for i in range(2 * n + 1)]
    return [(b[i], b[i + 1] - b[i]) for i in (j, 2 * n - 1 - j) if b[i + 1] > b[i]]


def imbalance_ratio(loads) -> float:
    total = sum(loads)
    return 1.0 if total == 0 else float(max(loads) * len(loads)) / float(total)


def flashcp_plan(lengths, n: int, r_target: float):
    """Algorithm 1.  Returns (per_doc_docs, whole_doc_plan, ratio) where
    whole_doc_plan[j] = [(doc, p, s)] in the order shards were added."""
    # 1: sort D by decreasing length (ties: document order); empty documents carry nothing
    d_sorted = sorted((i for i, L in enumerate(lengths) if L > 0), key=lambda i: (-lengths[i], i))
    per_doc_p = []                                   # 2
    cur_r = float("inf")                             # 3
    while True:                                      # 4: while Cur R > R
        whole = [i for i in d_sorted if i not in per_doc_p]
        pd_load = [sum(shard_workload(p, s) for i in per_doc_p for p, s in per_doc_pieces(lengths[i], n, j))
                   for j in range(n)]
        tmp_p = [[] for _ in range(n)]               # 5
        load = list(pd_load)
        tokens = [0] * n
        for d in whole:                              # 6-9: Min Worker Add(d)
            w = min(range(n), key=lambda j: (load[j], j))
            tmp_p[w].append((d, 0, lengths[d]))
            load[w] += shard_workload(0, lengths[d])
            tokens[w] += lengths[d]
        tw = sum(tokens)
        total = tw + sum(lengths[i] for i in per_doc_p)
        pd_tokens = [sum(s for i in per_doc_p for _, s in per_doc_pieces(lengths[i], n, j)) for j in range(n)]
        target = [total // n + (1 if j < total % n else 0) - pd_tokens[j] for j in range(n)]
        if min(target) < 0:
            target = [tw // n + (1 if j < tw % n else 0) for j in range(n)]
        while any(tokens[j] != target[j] for j in range(n)):      # 10-16: equal tokens
            a = max(range(n), key=lambda j: (tokens[j] - target[j], -j))
            docs = []                                # Max Token Worker Pop()
            while tokens[a] > target[a]:
                d, p, s = tmp_p[a].pop()
                tokens[a] -= s
                load[a] -= shard_workload(p, s)
                docs.append((d, p, s))
            for d, p, s in docs:                     # Whole Doc Shard and Add(docs)
                while s > 0:
                    b = min((j for j in range(n) if tokens[j] < target[j]), key=lambda j: (load[j], j))
                    take = min(s, target[b] - tokens[b])
                    tmp_p[b].append((d, p, take))
                    tokens[b] += take
                    load[b] += shard_workload(p, take)
                    p, s = p + take, s - take
        cur_r = imbalance_ratio(load)                # 17-18
        if cur_r > r_target and whole:               # 19-23: longest remaining document -> Per-Doc
            per_doc_p.append(whole[0])
            continue
        return per_doc_p, tmp_p, cur_r               # 25-26


def plan_chunks(lengths, n: int, r_target: float):
    """Each worker's chunk list (global positions, ascending, adjacent shards
    joined) for the plan above, plus the per-doc documents and the ratio."""
    per_doc, whole, ratio = flashcp_plan(lengths, n, r_target)
    starts = [0]
    for L in lengths:
        starts.append(starts[-1] + L)
    out = []
    for j in range(n):
        segs = [(starts[d] + p, s) for d, p, s in whole[j]]
        segs += [(starts[d] + p, s) for d in per_doc for p, s in per_doc_pieces(lengths[d], n, j)]
        segs.sort()
        merged = []
        for g, s in segs:
            if merged and merged[-1][0] + merged[-1][1] == g:
                merged[-1] = (merged[-1][0], merged[-1][1] + s)
            else:
                merged.append((g, s))
        out.append(merged)
    return out, sorted(per_doc), ratio
