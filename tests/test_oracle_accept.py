"""Pins for the oracle's acceptance walk and KV compaction (CPU only).

* chain case: the standard greedy speculative-decoding rule (accept the
  longest prefix where draft and target agree, then the target's token);
* forced path: a target built to stop at a chosen node stops there;
* hazard case: path [0, 2, 5] moves rows in the right order;
* lossless (both DFlash pages: output identical to the target alone): a
  multi-step simulation with a deterministic target f(context) and drafted
  trees built by the oracle commits exactly the tokens that running f
  autoregressively produces, and the compacted cache holds exactly the rows
  a sequential writer would have written.
"""
import hashlib

import numpy as np
import pytest

import synth
from oracle.accept import accept_compact
from oracle.logits import topk_logprobs
from oracle.tree import build_tree


def _cache(rows, n_layers=2, hkv=1, D=4):
    c = np.zeros((n_layers, rows, hkv, D), dtype=np.int64)
    for l in range(n_layers):
        for r in range(rows):
            c[l, r] = 1000 * l + r
    return c


def test_chain_is_longest_agreeing_prefix():
    rng = np.random.default_rng(0)
    L = 8
    for trial in range(50):
        draft = rng.integers(0, 3, L)
        target_next = rng.integers(0, 3, L + 1)
        n = L + 1
        tok = np.concatenate([[99], draft]).astype(np.int32)
        par = np.arange(-1, L).astype(np.int32)
        t = target_next.astype(np.int32)
        k = _cache(n + 5)
        acc, path, bonus, new_len, _, _ = accept_compact(
            tok[None], par[None], [n], t[None], L, k, k, [0], [5])
        want = 0
        while want < L and draft[want] == target_next[want]:
            want += 1
        assert acc[0] == want
        assert bonus[0] == target_next[want]
        assert new_len[0] == 5 + want + 1
        assert path[0, :want + 1].tolist() == list(range(want + 1))


def test_forced_path_stops_at_chosen_node_and_compacts():
    cfg = synth.CONFIGS[1]
    case = synth.make_case(cfg)
    ids, logp, _ = topk_logprobs(case.logits, cfg.K)
    t = build_tree(logp, ids, int(case.root_token[0]), cfg.k_tree, cfg.B)
    n = t["n_nodes"]
    P = 10
    for stop in range(n):
        tgt = synth.force_path_target(t["token"], t["parent"], t["depth"], n, stop,
                                      case.off_path[0], cfg.vocab)
        k = _cache(P + n)
        v = -_cache(P + n)
        acc, path, bonus, new_len, k2, v2 = accept_compact(
            t["token"][None], t["parent"][None], [n], tgt[None], cfg.L, k, v, [0], [P])
        chain = [stop]
        while chain[-1] != 0:
            chain.append(int(t["parent"][chain[-1]]))
        chain.reverse()
        assert path[0, :len(chain)].tolist() == chain
        assert acc[0] == t["depth"][stop]
        assert bonus[0] == tgt[stop]
        for j, s in enumerate(chain):
            assert np.array_equal(k2[:, P + j], k[:, P + s])
            assert np.array_equal(v2[:, P + j], v[:, P + s])
        assert np.array_equal(k2[:, :P], k[:, :P])


def test_overlapping_rows_use_snapshot():
    # slots: 0 root, 1 (a), 2 (b child of 0), 3, 4, 5 (child of 2)
    tok = np.array([0, 10, 11, 12, 13, 14], dtype=np.int32)
    par = np.array([-1, 0, 0, 1, 1, 2], dtype=np.int32)
    tgt = np.array([11, 0, 14, 0, 0, 77], dtype=np.int32)
    k = _cache(3 + 6)
    acc, path, bonus, new_len, k2, _ = accept_compact(
        tok[None], par[None], [6], tgt[None], 4, k, k, [0], [3])
    assert path[0, :3].tolist() == [0, 2, 5] and acc[0] == 2 and bonus[0] == 77
    assert np.array_equal(k2[:, 3 + 1], k[:, 3 + 2])
    assert np.array_equal(k2[:, 3 + 2], k[:, 3 + 5])


def _f(context):
    """Deterministic synthetic target: next token is a hash of the context."""
    h = hashlib.sha256(np.asarray(context, dtype=np.int64).tobytes()).digest()
    return int.from_bytes(h[:4], "little") % 5


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_lossless_multi_step(seed):
    rng = np.random.default_rng(seed)
    L, K, B, V = 4, 3, 9, 5
    prompt = [1, 2, 3]
    steps = 12
    cap = len(prompt) + steps * (L + 1) + B + 2
    # cache rows encode (token, position): row value = token * 1000 + position
    kc = np.full((1, cap, 1, 1), -1, dtype=np.int64)
    for p, tkn in enumerate(prompt):
        kc[0, p, 0, 0] = tkn * 1000 + p
    committed = list(prompt)
    bonus = _f(committed)                  # first target token after the prompt
    for _ in range(steps):
        P = len(committed)                 # rows [0, P) hold committed tokens
        # the bonus token is the tree root, already produced by the target
        logp = np.sort(np.log(rng.dirichlet(np.ones(V), size=L)), axis=1)[:, ::-1][:, :K]
        ids = np.stack([rng.permutation(V)[:K] for _ in range(L)]).astype(np.int32)
        t = build_tree(logp.astype(np.float32), ids, bonus, K, B)
        n = t["n_nodes"]
        # target argmax at every slot, from the slot's own root-to-node context
        tgt = np.zeros(B + 1, dtype=np.int32)
        for s in range(n):
            chain = [s]
            while chain[-1] != 0:
                chain.append(int(t["parent"][chain[-1]]))
            toks = [int(t["token"][c]) for c in reversed(chain)]
            tgt[s] = _f(committed + toks)
        # verify pass writes each slot's row at P + slot
        for s in range(n):
            d = int(t["depth"][s])
            kc[0, P + s, 0, 0] = int(t["token"][s]) * 1000 + (P + d)
        acc, path, nb, new_len, kc, _ = accept_compact(
            t["token"][None], t["parent"][None], [n], tgt[None], L, kc, kc, [0], [P])
        new = [int(t["token"][s]) for s in path[0, :acc[0] + 1]]
        committed += new
        bonus = int(nb[0])
        assert new_len[0] == len(committed)
    # autoregressive rollout of f
    ref = list(prompt)
    ref.append(_f(ref))
    while len(ref) < len(committed) + 1:
        ref.append(_f(ref))
    assert committed == ref[:len(committed)]
    assert bonus == ref[len(committed)]
    for p, tkn in enumerate(committed):
        assert kc[0, p, 0, 0] == tkn * 1000 + p
