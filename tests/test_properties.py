"""Property tests of the oracle on random small inputs (hypothesis, CPU).

Each property is a fact the pages or the mathematics fix, checked without
re-running the oracle's own algorithm:

* tree ([DDTree] "방법론 자세히 보기"): the returned node set is prefix-
  closed and closed under "elder sibling"; every node's parent precedes it
  and its depth is its parent's plus one; sibling tokens are distinct; each
  score is the fp32 sum of its parent's score and its own log-prob; scores
  never increase in slot order; the ancestor mask holds exactly the path to
  the root; and the set is a top-B set, certified by its frontier: every
  prefix left out (the first child of a node, or the next sibling of a
  node) scores no higher than the lowest node taken, and the node count is
  min(B, number of prefixes) + 1.
* logit pass ([DDTree] "핵심 아이디어"): the k ids are distinct, ordered by
  (x desc, id asc), no token left out beats the k-th, and the log-probs
  are x - lse with sum_v exp(x_v - lse) = 1.
* acceptance ([DDTree] "방법론 자세히 보기"): the path follows parent links
  whose tokens equal the target at the previous node, it cannot be
  extended, the bonus is the target at its end, and the compacted rows are
  the path's rows in order."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle.accept import accept_compact
from oracle.logits import topk_logprobs
from oracle.tree import build_tree

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def tree_tables(draw):
    L = draw(st.integers(1, 6))
    K = draw(st.integers(1, 7))
    k_tree = draw(st.integers(1, K))
    B = draw(st.integers(0, 50))
    coarse = draw(st.booleans())       # coarse values force exact score ties
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    raw = rng.uniform(-6.0, 0.0, size=(L, K))
    if coarse:
        raw = np.round(raw * 2) / 2
    logp = -np.sort(-raw, axis=1).astype(np.float32)
    ids = np.stack([rng.choice(1000, K, replace=False) for _ in range(L)]).astype(np.int32)
    return logp, ids, k_tree, B


def _universe_size(L, k_tree, B):
    n, level = 0, 1
    for _ in range(L):
        level *= k_tree
        n += level
        if n >= B:
            return B
    return n


@SETTINGS
@given(tree_tables())
def test_tree_is_a_certified_top_b_prefix_set(case):
    logp, ids, k_tree, B = case
    L = logp.shape[0]
    t = build_tree(logp, ids, 7, k_tree, B)
    n = t["n_nodes"]
    assert n == min(B, _universe_size(L, k_tree, B)) + 1
    tok, par, dep, sc = t["token"], t["parent"], t["depth"], t["score"]
    # rank of every node within its position's row (tokens are distinct per row)
    rank = np.full(n, -1)
    for s in range(1, n):
        row = list(ids[dep[s] - 1])
        assert tok[s] in row[:k_tree]
        rank[s] = row.index(tok[s])
    children = {}
    for s in range(1, n):
        p = int(par[s])
        assert 0 <= p < s and dep[s] == dep[p] + 1 and dep[s] <= L
        assert sc[s] == np.float32(sc[p] + logp[dep[s] - 1, rank[s]])
        children.setdefault(p, []).append(s)
    for p, cs in children.items():
        ranks = sorted(int(rank[c]) for c in cs)
        assert ranks == list(range(len(ranks)))           # elder siblings present
        assert len({int(tok[c]) for c in cs}) == len(cs)  # distinct sibling tokens
    assert np.all(np.diff(sc[1:n]) <= 0)
    # frontier certificate of optimality
    low = sc[1:n].min() if n > 1 else np.float32(np.inf)
    frontier = []
    for s in range(0, n):
        d = int(dep[s])
        if d < L and 0 not in [int(rank[c]) for c in children.get(s, [])]:
            frontier.append(np.float32(sc[s] + logp[d, 0]))      # first child left out
        if s > 0:
            nxt = int(rank[s]) + 1
            sibs = [int(rank[c]) for c in children.get(int(par[s]), [])]
            if nxt < k_tree and nxt not in sibs:
                frontier.append(np.float32(sc[int(par[s])] + logp[d - 1, nxt]))
    if n - 1 == B:
        assert all(f <= low for f in frontier)
    # ancestor mask = the root path, self included
    for s in range(n):
        path, a = {s}, s
        while a > 0:
            a = int(par[a])
            path.add(a)
        bits = {j for j in range(B + 1) if (int(t["mask"][s, j // 64]) >> (j % 64)) & 1}
        assert bits == path


@st.composite
def logit_rows(draw):
    rows = draw(st.integers(1, 4))
    V = draw(st.integers(1, 300))
    k = draw(st.integers(1, min(V, 40)))
    coarse = draw(st.booleans())
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 3, size=(rows, V))
    if coarse:
        z = np.round(z)
    inv_t = draw(st.sampled_from([1.0, 0.5, 1.7]))
    return z.astype(np.float32), k, inv_t


@SETTINGS
@given(logit_rows())
def test_topk_is_the_ordered_k_best(case):
    z, k, inv_t = case
    ids, logp, lse = topk_logprobs(z, k, inv_t)
    x = (z * np.float32(inv_t)).astype(np.float32).astype(np.float64)
    for r in range(z.shape[0]):
        sel = ids[r].astype(np.int64)
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < z.shape[1]
        for a, b in zip(sel[:-1], sel[1:]):
            assert x[r, a] > x[r, b] or (x[r, a] == x[r, b] and a < b)
        rest = np.setdiff1d(np.arange(z.shape[1]), sel)
        last = sel[-1]
        assert np.all((x[r, rest] < x[r, last]) | ((x[r, rest] == x[r, last]) & (rest > last)))
        assert abs(np.exp(x[r] - lse[r]).sum() - 1.0) < 1e-12
        assert np.allclose(logp[r], (x[r, sel] - lse[r]).astype(np.float32), rtol=0, atol=0)


@st.composite
def accept_cases(draw):
    n = draw(st.integers(1, 40))
    L = draw(st.integers(1, 8))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    par = np.full(n, -1, np.int32)
    tok = np.zeros(n, np.int32)
    dep = np.zeros(n, np.int32)
    used = {}
    for s in range(1, n):
        cands = [p for p in range(s) if dep[p] < L]
        p = int(rng.choice(cands))
        par[s], dep[s] = p, dep[p] + 1
        t = int(rng.integers(0, 6))
        while t in used.setdefault(p, set()):   # sibling tokens distinct
            t += 1
        used[p].add(t)
        tok[s] = t
    tgt = rng.integers(0, 8, size=n).astype(np.int32)
    P = int(rng.integers(0, 5))
    return tok, par, tgt, L, P


@SETTINGS
@given(accept_cases())
def test_accept_path_is_the_longest_agreeing_walk(case):
    tok, par, tgt, L, P = case
    n = len(tok)
    rows = P + n
    rng = np.random.default_rng(0)
    k = rng.integers(0, 65536, size=(1, rows, 1, 4), dtype=np.uint16)
    v = rng.integers(0, 65536, size=(1, rows, 1, 4), dtype=np.uint16)
    acc, path, bonus, new_len, ko, vo = accept_compact(tok[None], par[None], [n], tgt[None], L,
                                                       k, v, [0], [P])
    m = int(acc[0])
    pth = [int(x) for x in path[0, :m + 1]]
    assert pth[0] == 0 and m <= L and all(x == -1 for x in path[0, m + 1:])
    for j in range(1, m + 1):
        assert par[pth[j]] == pth[j - 1] and tok[pth[j]] == tgt[pth[j - 1]]
    last = pth[-1]
    if m < L:
        assert not any(par[c] == last and tok[c] == tgt[last] for c in range(1, n))
    assert bonus[0] == tgt[last] and new_len[0] == P + m + 1
    for j, s in enumerate(pth):
        assert np.array_equal(ko[0, P + j], k[0, P + s]) and np.array_equal(vo[0, P + j], v[0, P + s])
    assert np.array_equal(ko[0, :P], k[0, :P])
