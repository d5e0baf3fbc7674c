"""Mutation sweep of the oracle's pins (CPU only; run by hand, not collected by pytest).

Plants one plausible mistake at a time in a scratch copy of oracle/ (a temporary
directory; the repository is not touched), runs the oracle pins (tests/test_oracle_*.py)
against that copy, and prints whether some pin catches it.  A mistake that no pin
catches would leave the GPU parity tests comparing against an unchecked definition.

    python tests/oracle_mutation_sweep.py
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (oracle file, text, replacement, what the mistake is)
M = [
 ("masks.py", "<= wt)", "< wt)", "sta window off by one in t"),
 ("masks.py", "& (np.abs(cw[:, None] - cw[None, :]) <= ww))", "& (np.abs(cw[:, None] - cw[None, :]) <= wh))", "sta w-window uses wh"),
 ("masks.py", "return (d <= 1) | (ds * (np.int64(1) << r) < S)", "return (d <= 0) | (ds * (np.int64(1) << r) < S)", "radial token: dense band d<=0"),
 ("masks.py", "return (d <= 1) | (ds * (np.int64(1) << r) < S)", "return (d <= 1) | (ds * (np.int64(1) << r) <= S)", "radial token: <= S"),
 ("masks.py", "w = (S - 1) >> r", "w = S >> r", "radial block: window width"),
 ("masks.py", "int(x).bit_length() - 1 if x >= 2 else 0", "int(x).bit_length() if x >= 2 else 0", "radial block: r = ceil"),
 ("masks.py", "x[i * block:min((i + 1) * block, n)].mean(axis=0)", "x[i * block:min((i + 1) * block, n)].sum(axis=0) / block", "pool: ragged mean over block"),
 ("masks.py", 'k = int(np.searchsorted(c, thr, side="left"))', 'k = int(np.searchsorted(c, thr, side="right"))', "cut: C>thr instead of >="),
 ("masks.py", "return np.sort(order[:k + 1]), bool(flagged), bool(near_tie)", "return np.sort(order[:k]), bool(flagged), bool(near_tie)", "cut: crossing block dropped"),
 ("masks.py", '    order = np.argsort(-p, kind="stable")\n    ps = p[order]', '    order = np.lexsort((-np.arange(n), -p))\n    ps = p[order]', "cut: ties to higher index"),
 ("masks.py", "return [(0, -(-anchor_end // block)), (recent_start // block, nbk)]", "return [(0, anchor_end // block), (recent_start // block, nbk)]", "ar: anchor range floor"),
 ("masks.py", "return [(0, -(-anchor_end // block)), (recent_start // block, nbk)]", "return [(0, -(-anchor_end // block)), (-(-recent_start // block), nbk)]", "ar: recent range ceil"),
 ("masks.py", "m[order[:topk]] = True", "m[order[:topk - 1]] = True", "ar: top-(k-1)"),
 ("masks.py", 'order = cand[np.argsort(-z[cand], kind="stable")]', 'order = cand[np.lexsort((-cand, -z[cand]))]', "ar: ties to higher index"),
 ("masks.py", "rows.append(sorted(a | b))", "rows.append(sorted(a & b))", "union -> intersection"),
 ("masks.py", "rows = [parts[h] for _ in range(batch) for h in range(len(windows))]", "rows = [parts[h] for h in range(len(windows)) for _ in range(batch)]", "sta_heads slab order"),
 ("attention.py", "                s = (q[b, q0:q1, h] @ k[b, toks, h].T) * scale\n", "                s = (q[b, q0:q1, h] @ k[b, toks, h].T) * scale * scale\n", "attn: scale squared"),
 ("attention.py", "                lse[b, h, q0:q1] = (m + np.log(l))[:, 0]", "                lse[b, h, q0:q1] = (m + np.log2(l))[:, 0]", "attn: lse log2"),
 ("attention.py", "    return np.concatenate([np.arange(j * block_k, min((j + 1) * block_k, nk)) for j in cols])", "    return np.concatenate([np.arange(j * block_k, (j + 1) * block_k) % nk for j in cols])", "attn: ragged key tail wraps"),
 ("attention.py", "                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "                ds = p * (dp + (p * dp).sum(axis=1, keepdims=True))", "bwd: sign of D"),
 ("attention.py", "                dk[b, toks, h] += ds.T @ qi * scale", "                dk[b, toks, h] += ds.T @ qi", "bwd: dk missing scale"),
 ("attention.py", "                dv[b, toks, h] += p.T @ di", "                dv[b, toks, h] = p.T @ di", "bwd: dv overwritten not accumulated"),
 ("reorder.py", "    lt, lh, lw = r // (th * tw), (r // tw) % th, r % tw", "    lt, lh, lw = r // (th * tw), (r // th) % tw, r % th", "reorder: th/tw swapped inside tile"),
 ("reorder.py", "    it, ih, iw = tile_id // (NH * NW), (tile_id // NW) % NH, tile_id % NW", "    it, ih, iw = tile_id // (NH * NW), tile_id % NH, (tile_id // NH) % NW", "reorder: tile grid order"),
 ("sics.py", "                out[b, h, i] = (unit @ unit.T).sum()", "                out[b, h, i] = (unit @ unit.T).sum() - len(rows)", "sics: diagonal excluded"),
 ("sics.py", "                unit = np.divide(rows, norm[:, None], out=np.zeros_like(rows), where=norm[:, None] > 0)", "                unit = rows / max(norm.max(), 1e-300)", "sics: not per-row normalised"),
 ("kvcache.py", "            remap[s, tail] = n_full_max", "            remap[s, tail] = len(full)", "kv: tail slot per head not shared"),
 ("kvcache.py", "    return n_full_max * block_k + ((nk - (nk // block_k) * block_k) if has_tail else 0)", "    return n_full_max * block_k + (block_k if has_tail else 0)", "kv: tail counted as a full block"),
 ("kvcache.py", "        keeps.append(np.unique(np.asarray(col_idx[lo:hi], np.int64)))", "        keeps.append(np.unique(np.asarray(col_idx[lo:hi - 1], np.int64)))", "kv: last entry of a slab missed"),
 ("kvcache.py", "        s = 0 if remap.shape[0] == 1 else r // n_qblocks", "        s = 0 if remap.shape[0] == 1 else r % remap.shape[0]", "kv remap: wrong slab of a row"),
 ("attention.py", "        p = block_softmax(q_rows[n][None], kj, scale)[0]\n        dp = vj @ dout_rows[n]\n        ds = p * (dp - (p * dp).sum())", "        p = block_softmax(q_rows[n][None], kj, scale)[0]\n        dp = vj @ dout_rows[n]\n        ds = p * (dp - dp.sum())", "bwd rows: D without p"),
 ("attention.py", "        dk += ds[:, sel].T @ qi * scale\n", "        dk += ds[:, sel].T @ qi\n", "bwd key block: dk missing scale"),
 ("attention.py", "        dv += p[:, sel].T @ di\n", "        dv += p[:, sel].T @ di * scale\n", "bwd key block: dv scaled"),
 ("attention.py", "            r = row_base + int(t) // block_q", "            r = row_base + int(t) // block_k", "attn rows: CSR row from block_k"),
 ("attention.py", "                allowed[a, j * block_k:min((j + 1) * block_k, nk)] = True", "                allowed[a, j * block_k:min((j + 1) * block_k, nk) - 1] = True", "attn rows: last key of each block dropped"),
 ("masks.py", "    if mass < thr - tol or mass - smallest >= thr + tol:", "    if mass < thr - tol:", "admissible: minimality unchecked"),
 ("masks.py", "    return bool(hi - lo <= tol * max(abs(lo), 1e-300))", "    return True", "topk admissible: order unchecked"),
]


# a rewrite that changes nothing (at d = 1, r = 0 and the window spans the frame)
EQUIVALENT = {"radial token: dense band d<=0"}


def run(idx, scratch):
    f, old, new, name = M[idx]
    d = os.path.join(scratch, f"m{idx:02d}")
    for sub in ("oracle", "tests", "workloads"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(d, sub), ignore=shutil.ignore_patterns("__pycache__"))
    p = os.path.join(d, "oracle", f)
    s = open(p).read()
    if s.count(old) != 1:
        return name, f"PATTERN FOUND {s.count(old)} TIMES"
    open(p, "w").write(s.replace(old, new))
    tests = sorted(t for t in os.listdir(os.path.join(d, "tests")) if t.startswith("test_oracle"))
    r = subprocess.run([sys.executable, "-m", "pytest", *[f"tests/{t}" for t in tests], "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=d, capture_output=True, text=True, timeout=900)
    fail = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
    if r.returncode:
        return name, "caught by " + (fail[0].split(" - ")[0].replace("FAILED ", "") if fail else "a failing run")
    return name, "SURVIVED" + (" (equivalent rewrite)" if name in EQUIVALENT else "")


def main():
    scratch = tempfile.mkdtemp(prefix="oracle_mutants_")
    try:
        with ThreadPoolExecutor(min(6, os.cpu_count() or 1)) as ex:
            results = list(ex.map(lambda i: run(i, scratch), range(len(M))))
    finally:
        shutil.rmtree(scratch, ignore_errors=True)
    for name, res in results:
        print(f"{name:44s} {res}")
    bad = [n for n, r in results if not r.startswith("caught") and n not in EQUIVALENT]
    print(f"{len(results)} mistakes planted, {len(bad)} not caught")
    sys.exit(1 if bad else 0)


if __name__ == "__main__":
    main()
