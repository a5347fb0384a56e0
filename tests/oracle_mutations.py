"""Planted-mistake check of the oracle's pins (CPU only; not collected by pytest).

Each entry plants one plausible mistake (a dropped term, a wrong sign or
index, a transposed operand, a missing snapshot) in a copy of oracle/ and
runs the oracle's pins and property tests against the copy; every mistake
must make at least one of them fail.  Run: python tests/oracle_mutations.py
[--dest DIR] [index ...]."""
import os, shutil, subprocess, sys, tempfile
REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MUTS = [
 ("logits", "oracle/logits.py", "x = (z * np.float32(inv_temperature))", "x = (z * np.float32(1.0))"),
 ("logits", "oracle/logits.py", "lse[r] = m + np.log(np.sum(np.exp(xr - m)))", "lse[r] = np.log(np.sum(np.exp(xr - m)))"),
 ("logits", "oracle/logits.py", "order = np.lexsort((token, -xr))", "order = np.lexsort((-token, -xr))"),
 ("logits", "oracle/logits.py", "logp[r] = (xr[top] - lse[r])", "logp[r] = (lse[r] - xr[top])"),
 ("argmax", "oracle/logits.py", "ids = np.argmax(z, axis=1)", "ids = (z.shape[1] - 1 - np.argmax(z[:, ::-1], axis=1))"),
 ("tree", "oracle/tree.py", "s = np.float32(score[par_slot] + y[d - 1, rank])", "s = np.float32(y[d - 1, rank])"),
 ("tree", "oracle/tree.py", "s = np.float32(score[par_slot] + y[d - 1, rank])", "s = np.float32(score[par_slot] + y[d - 1, 0])"),
 ("tree", "oracle/tree.py", "heapq.heappush(heap, (-float(s), d, par_slot, rank))", "heapq.heappush(heap, (-float(s), -d, par_slot, rank))"),
 ("tree", "oracle/tree.py", "if rank + 1 < k_tree:", "if rank + 1 < k_tree and d > 1:"),
 ("tree", "oracle/tree.py", "token.append(int(ids[d - 1, rank]))", "token.append(int(ids[d - 1, 0]))"),
 ("tree", "oracle/tree.py", "if d < L:", "if d < L - 1:"),
 ("tree", "oracle/tree.py", "sets[s] = (sets[p] if s > 0 else 0) | (1 << s)", "sets[s] = (sets[p] if s > 0 else 0)"),
 ("attn", "oracle/attention.py", "scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D"),
 ("attn", "oracle/attention.py", "kh = h // g", "kh = h % hkv"),
 ("attn", "oracle/attention.py", "visible[i, P:] = _mask_bits(own_mask[r, i], n)", "visible[:, P + i] = _mask_bits(own_mask[r, i], n)"),
 ("attn", "oracle/attention.py", "lse[r, :n, h] = (m + np.log(l))[:, 0]", "lse[r, :n, h] = (np.log(l))[:, 0]"),
 ("attn", "oracle/attention.py", "visible[i, P + j] = (i // block_len) == (j // block_len)", "visible[i, P + j] = abs(i - j) < block_len"),
 ("accept", "oracle/accept.py", "if node_parent[c] == cur and node_token[c] == target[cur]:", "if node_parent[c] == cur and node_token[c] == target[c]:"),
 ("accept", "oracle/accept.py", "return path, int(target[cur])", "return path, int(target[path[-2] if len(path) > 1 else cur])"),
 ("accept", "oracle/accept.py", "new_len[r] = P + n_acc + 1", "new_len[r] = P + n_acc"),
 ("accept", "oracle/accept.py", "rows = cache[:, src].copy()      # snapshot every source row first\n            cache[:, dst] = rows", "for a_, b_ in zip(reversed(src), reversed(dst)):\n                cache[:, b_] = cache[:, a_]"),
 ("accept", "oracle/accept.py", "while len(path) <= L:", "while len(path) < L:"),
 ("rope", "oracle/rope.py", "theta = float(base) ** (-2.0 * j / D)", "theta = float(base) ** (-1.0 * j / D)"),
 ("rope", "oracle/rope.py", "return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)", "return np.concatenate([lo * c + hi * s, hi * c - lo * s], axis=-1)"),
 ("rope", "oracle/rope.py", "pos[r, :n] = int(prefix_len[r]) + node_depth[r, :n]", "pos[r, :n] = int(prefix_len[r]) + np.arange(n)"),
 ("rope", "oracle/rope.py", "return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16)", "return ((u + 0x8000) >> 16)"),
 ("rope", "oracle/rope.py", "vc[rows] = v_new_bits[r, :n]", "vc[rows] = _f64_to_bf16_bits(rope_f64(_bf16_bits_to_f64(v_new_bits[r, :n]), p[:, None], base))"),
 ("lmhead", "oracle/lmhead.py", "z[:, v0:v0 + _BLOCK] = h @ _bf16_to_f64(w_bits[v0:v0 + _BLOCK]).T", "z[:, v0:v0 + _BLOCK] = h[:, ::-1] @ _bf16_to_f64(w_bits[v0:v0 + _BLOCK]).T"),
 ("lmhead", "oracle/lmhead.py", "return hidden * 2.0 ** -24 * m", "return 2.0 ** -24 * m"),
 ("lmhead", "oracle/lmhead.py", "ids, logp, lse = topk_logprobs(z64.astype(np.float32), k, inv_temperature)", "ids, logp, lse = topk_logprobs(z64.astype(np.float32), k, 1.0)"),
]
def main():
    args = sys.argv[1:]
    dest_root = None
    if args[:1] == ["--dest"]:
        dest_root, args = args[1], args[2:]
    sel = args
    DST = os.path.join(dest_root or tempfile.mkdtemp(prefix="oracle_mut_"), "repo")
    survived = 0
    for idx, (fam, f, old, new) in enumerate(MUTS):
        if sel and str(idx) not in sel: continue
        if os.path.exists(DST): shutil.rmtree(DST)
        shutil.copytree(REPO, DST, ignore=shutil.ignore_patterns('.git', 'gpurun_out', '_work', '_build', '__pycache__', '*.so', '.hypothesis'))
        p = os.path.join(DST, f); s = open(p).read()
        assert s.count(old) == 1, (idx, old)
        open(p, 'w').write(s.replace(old, new))
        r = subprocess.run([sys.executable, '-m', 'pytest', '-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider',
                            'tests/test_oracle_logits.py', 'tests/test_oracle_tree.py', 'tests/test_oracle_attention.py',
                            'tests/test_oracle_accept.py', 'tests/test_oracle_rope.py', 'tests/test_oracle_lmhead.py',
                            'tests/test_properties.py'], cwd=DST, capture_output=True, text=True, timeout=1200)
        tail = [l for l in r.stdout.splitlines() if l.startswith('FAILED') or 'passed' in l or 'failed' in l]
        survived += r.returncode == 0
        print(idx, fam, 'CAUGHT' if r.returncode else 'SURVIVED', '|', new.splitlines()[0][:60], '|',
              tail[-2:] if tail else '', flush=True)
    shutil.rmtree(DST, ignore_errors=True)
    print(f"{survived} of {len(sel) or len(MUTS)} planted mistakes survived", flush=True)
    return 1 if survived else 0


if __name__ == "__main__":
    sys.exit(main())
