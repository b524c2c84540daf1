"""Planted mistakes in copies of the oracle must fail its pins (CPU only).

Each case copies the oracle package to a temporary directory, changes one
line the way a plausible slip would (a dropped term, a wrong sign or index,
a max for a sum), imports the copy and runs the pin that should catch it.
"""

import importlib.util
import os
import shutil
import sys

import numpy as np
import pytest
import torch

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _mutant(tmp_path, name, fname, old, new):
    dst = tmp_path / name
    shutil.copytree(ORACLE_DIR, dst)
    path = dst / fname
    src = path.read_text()
    assert src.count(old) == 1, (fname, old)
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(name, dst / "__init__.py", submodule_search_locations=[str(dst)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


def _pin_budget(orc):
    return orc.budget(512, 1, 20, 16) == 26 and all(
        orc.budget(L, 1, 20, 64) * 20 >= L for L in range(0, 3000))


def _pin_select(orc):
    sc = np.array([0.5, 0.9, 0.9, 0.1, 0.0, 0.0], dtype=np.float32)
    ok = orc.select(sc, 6, 1, 2, 2).tolist() == [1, 4, 5]
    rng = np.random.default_rng(2)
    sc = rng.integers(0, 20, size=900).astype(np.float32) / 4
    cand = np.arange(900 - 64)
    order = np.lexsort((cand, -sc[:900 - 64].astype(np.float64)))
    ref = np.sort(np.concatenate([order[:orc.budget(900, 1, 20, 64) - 64], np.arange(900 - 64, 900)]))
    return ok and np.array_equal(orc.select(sc, 900, 1, 20, 64), ref)


def _pin_verify(orc):
    from s3r_inputs import get_config, make_batch
    cfg = get_config(1, B=1, Hq=4, Hkv=2, D=16, k=3, lengths=("fixed", 50))
    bt = make_batch(cfg, parts=("kv", "q"))
    S = int(bt.seq_len[0])
    o, lse, sc = orc.verify(bt.q_verify[0], bt.k_pages, bt.v_pages, bt.block_table[0], S, 3, float(bt.scale))
    K = np.stack([orc.gather(bt.k_pages, bt.block_table[0], kv, np.arange(S)) for kv in range(2)])
    V = np.stack([orc.gather(bt.v_pages, bt.block_table[0], kv, np.arange(S)) for kv in range(2)])
    q = torch.tensor(bt.q_verify[0].astype(np.float64)).permute(1, 0, 2)
    Kt, Vt = torch.tensor(K).repeat_interleave(2, 0), torch.tensor(V).repeat_interleave(2, 0)
    mask = torch.arange(S)[None, :] <= (torch.arange(4)[:, None] + S - 4)
    ref = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, attn_mask=mask, scale=float(bt.scale))
    ok_o = np.allclose(o.transpose(1, 0, 2), ref.numpy(), rtol=1e-10, atol=1e-12)
    ok_sum = np.allclose(sc.sum(axis=1), 2 * 4, rtol=1e-12)
    return ok_o and ok_sum


def _pin_decode(orc):
    from s3r_inputs import get_config, make_batch
    cfg = get_config(1, B=1, Hq=4, Hkv=2, D=16, k=2, lengths=("fixed", 40))
    bt = make_batch(cfg, parts=("kv", "q"))
    L = 40
    idx = [np.arange(L), np.arange(L)]
    o, lse = orc.sparse_decode(bt.q_draft[1, 0], bt.k_pages, bt.v_pages, bt.block_table[0], idx, L, L, L + 2, float(bt.scale))
    K = np.stack([orc.gather(bt.k_pages, bt.block_table[0], kv, np.arange(L + 2)) for kv in range(2)])
    V = np.stack([orc.gather(bt.v_pages, bt.block_table[0], kv, np.arange(L + 2)) for kv in range(2)])
    q = torch.tensor(bt.q_draft[1, 0].astype(np.float64))[:, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, torch.tensor(K).repeat_interleave(2, 0), torch.tensor(V).repeat_interleave(2, 0), scale=float(bt.scale))
    return np.allclose(o, ref[:, 0].numpy(), rtol=1e-10, atol=1e-12)


def _pin_sampling(orc):
    from tests.test_oracle_sampling import _chi2_run
    import importlib
    mod = importlib.import_module(orc.__name__ + ".sampling")
    return min(_chi2_run(mod.spec_decide, n=100_000)) > 1e-3


def _pin_append(orc):
    from tests.test_oracle_driver import pin_append_against_generator
    try:
        return pin_append_against_generator(orc)
    except IndexError:  # a slip that writes outside the cache fails the pin too
        return False


def _pin_pages(orc):
    from tests.test_oracle_select_variants import _brute_pages, _int_scores
    rng = np.random.default_rng(2)
    for L in (17, 200, 777):
        for (sn, sd, W) in ((1, 20, 64), (1, 5, 1), (1, 2, 30)):
            sc = _int_scores(rng, 3, L, hi=6)
            got = orc.select_grouped(sc, L, sn, sd, W, 16, False)
            for h in range(3):
                if got[h].tolist() != _brute_pages(sc[h].astype(np.int64), L, sn, sd, W):
                    return False
    return True


def _pin_all_heads(orc):
    rng = np.random.default_rng(1)
    sc = rng.integers(0, 50, size=(8, 333)).astype(np.float32)
    ref = orc.select(sc.astype(np.int64).sum(axis=0).astype(np.float32), 333, 1, 10, 16)
    return all(np.array_equal(g, ref) for g in orc.select_grouped(sc, 333, 1, 10, 16, 1, True))


def _pin_margins(orc):
    from tests.test_oracle_sampling import _flip_checks, _rows
    import importlib
    mod = importlib.import_module(orc.__name__ + ".sampling")
    p0 = np.array([0.5, 0.25, 0.125, 0.125])
    q0 = np.array([0.25, 0.5, 0.125, 0.125])
    if mod.decide_margins([p0, np.full(4, 0.25)], [q0], [1], [0.75, 0.375]) != (0.25, 0.375):
        return False
    rng = np.random.default_rng(8)
    try:
        for _ in range(60):
            zt, zd = _rows(12, 3, int(rng.integers(1 << 30)), noise=1.0)
            p_rows = [mod.softmax_t(zt[i], 1.0) for i in range(4)]
            q_rows = [mod.softmax_t(zd[i], 1.0) for i in range(3)]
            d = [int(rng.choice(12, p=q_rows[i])) for i in range(3)]
            _flip_checks(p_rows, q_rows, d, rng.random(4), S=mod)
    except AssertionError:
        return False
    return True


def _pin_commit(orc):
    from tests.test_oracle_driver import pin_commit
    try:
        return pin_commit(orc)
    except (AssertionError, IndexError):
        return False


def _pin_page_scores(orc):
    from tests.test_oracle_attention import test_page_scores_are_sums_of_position_scores as pin
    import tests.test_oracle_attention as ta
    saved = ta.oracle
    ta.oracle = orc
    try:
        pin()
    except AssertionError:
        return False
    finally:
        ta.oracle = saved
    return True


def _pin_page_select(orc):
    from tests.test_oracle_select_variants import _brute_pages, _int_scores
    rng = np.random.default_rng(4)
    for all_heads in (False, True):
        for L in (17, 300):
            sc = _int_scores(rng, 3, L + 7, hi=6)
            npg = -(-(L + 7) // 16)
            pages = np.stack([[sc[h, 16 * p:16 * p + 16].astype(np.int64).sum() for p in range(npg)]
                              for h in range(3)]).astype(np.float32)
            try:
                got = orc.select_by_page_scores(pages, L, 1, 5, 20, all_heads)
            except IndexError:  # a slip that reads past the candidates fails the pin too
                return False
            for h in range(3):
                key = sc.astype(np.int64).sum(axis=0) if all_heads else sc[h].astype(np.int64)
                if got[h].tolist() != _brute_pages(key, L, 1, 5, 20):
                    return False
    return True


MUTANTS = [
    ("budget.py", "frac = -((-s_num * L) // s_den)", "frac = (s_num * L) // s_den", _pin_budget),
    ("budget.py", "return min(L, max(newest, frac))", "return min(L, newest + frac)", _pin_budget),
    ("select.py", "key=lambda j: (-vals[j], j)", "key=lambda j: (-vals[j], -j)", _pin_select),
    ("select.py", "key=lambda j: (-vals[j], j)", "key=lambda j: (vals[j], j)", _pin_select),
    ("attention.py", "last = seq_len - (k + 1) + i", "last = seq_len - (k + 1) + i - 1", _pin_verify),
    ("attention.py", "scores[kv, :last + 1] += p", "scores[kv, :last + 1] = np.maximum(scores[kv, :last + 1], p)", _pin_verify),
    ("attention.py", "logits = float(scale) * (K @ q)", "logits = K @ q", _pin_verify),
    ("attention.py", "for h in range(kv * G, (kv + 1) * G):", "for h in range(kv, kv + G):", _pin_verify),
    ("attention.py", "kv = h // G\n        pos", "kv = h % Hkv\n        pos", _pin_decode),
    ("attention.py", "np.arange(L, cur, dtype=np.int64)])", "np.arange(L, cur - 1, dtype=np.int64)])", _pin_decode),
    ("sampling.py", "if p >= q or float(u[i]) * q < p:", "if p >= q or float(u[i]) * p < q:", _pin_sampling),
    ("sampling.py", "tokens[k] = invcdf(p_rows[k], u[k])", "tokens[k] = invcdf(p_rows[k - 1], u[k])", _pin_sampling),
    ("cache.py", "j = int(pos) + t", "j = int(pos) + t + 1", _pin_append),
    ("cache.py", "k_pages[page, :, j % P, :] = k_rows[t]", "k_pages[page, :, j % P, :] = k_rows[n - 1 - t]", _pin_append),
    ("cache.py", "v_pages[page, :, j % P, :] = v_rows[t]", "v_pages[page, :, j % P, :] = k_rows[t]", _pin_append),
    ("cache.py", "page = int(bt_row[j // P])", "page = int(bt_row[j % P])", _pin_append),
    ("sampling.py", "return float(min(t - lo, c[y] - t) / Z)", "return float((c[y] - t) / Z)", _pin_margins),
    ("sampling.py", "ratio = min(ratio, abs(float(u[i]) * q - p) / max(p, q))",
     "ratio = min(ratio, abs(float(u[i]) * q - p))", _pin_margins),
    ("sampling.py", "lo = c[y - 1] if y > 0 else 0.0", "lo = c[y - 1] if y > 1 else 0.0", _pin_margins),
    ("attention.py", "out[:, p] = scores[:, p * unit:min((p + 1) * unit, int(seq_len))].sum(axis=1)",
     "out[:, p] = scores[:, p * unit + 1:min((p + 1) * unit + 1, int(seq_len))].sum(axis=1)", _pin_page_scores),
    ("attention.py", "npg = -(-int(seq_len) // unit)", "npg = int(seq_len) // unit", _pin_page_scores),
    ("select_variants.py", "keys = [head_sum(page_rows, f)] if all_heads",
     "keys = [np.asarray(page_rows[0][:f], np.float32)] if all_heads", _pin_page_select),
    ("select_variants.py", "vals = [float(v) for v in np.asarray(sums, dtype=np.float32)[:f]]",
     "vals = [float(v) for v in np.asarray(sums, dtype=np.float32)[1:f + 1]]", _pin_page_select),
    ("round.py", "L1 = int(L) + n_out", "L1 = int(L) + n_out - 1", _pin_commit),
    ("round.py", "pending = int(np.asarray(tokens)[n_out - 1])", "pending = int(np.asarray(tokens)[n_out - 2])",
     _pin_commit),
    ("round.py", "return L1, pending, [L1 + j for j in range(1, k + 1)], L1 + k + 1",
     "return L1, pending, [L1 + j for j in range(1, k + 1)], L1 + k", _pin_commit),
    ("select_variants.py", "key=lambda p: (-vals[p], p))", "key=lambda p: (-vals[p], -p))", _pin_pages),
    ("select_variants.py", "n_top = min(f, -(-max(0, n - wc) // unit))", "n_top = min(f, max(0, n - wc) // unit)",
     _pin_pages),
    ("select_variants.py", "f = (L - w) // unit", "f = -(-(L - w) // unit)", _pin_pages),
    ("select_variants.py", "acc = (acc + np.asarray(scores_rows[h][:L], dtype=np.float32)).astype(np.float32)",
     "acc = np.maximum(acc, np.asarray(scores_rows[h][:L], dtype=np.float32))", _pin_all_heads),
]


def test_unmutated_oracle_passes_pins():
    import oracle
    assert _pin_budget(oracle) and _pin_select(oracle) and _pin_verify(oracle) and _pin_decode(oracle)
    assert _pin_append(oracle) and _pin_pages(oracle) and _pin_all_heads(oracle)
    assert _pin_margins(oracle) and _pin_commit(oracle) and _pin_page_scores(oracle) and _pin_page_select(oracle)


@pytest.mark.parametrize("case", range(len(MUTANTS)))
def test_mutant_is_caught(tmp_path, case):
    fname, old, new, pin = MUTANTS[case]
    mod = _mutant(tmp_path, f"oracle_mutant_{case}", fname, old, new)
    assert not pin(mod)
