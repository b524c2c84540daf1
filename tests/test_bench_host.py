"""Host-side logic of the benchmark: the unique-row count of the rollout workload
(shared prompt prefix read once per group), the rollout block tables, and the
single-GPU guard."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from s3r_inputs import get_config, make_batch  # noqa: E402


def brute_unique(seq_len, idx, n_sel, prefix, group, k):
    """Count distinct physical rows by naming each one: a prefix row belongs to the group,
    every other row to its sequence."""
    B, Hkv = idx.shape[0], idx.shape[1]

    def owner(b, pos):
        return ("g", b // group) if pos < prefix else ("s", b)

    ver = {(owner(b, p), h, p) for b in range(B) for h in range(Hkv) for p in range(int(seq_len[b]))}
    draft = []
    for j in range(1, k + 1):
        rows = set()
        for b in range(B):
            L = int(seq_len[b]) - k - 1
            for h in range(Hkv):
                for p in list(idx[b, h, :n_sel[b]]) + [L + i for i in range(j)]:
                    rows.add((owner(b, int(p)), h, int(p)))
        draft.append(len(rows))
    return len(ver), draft


def test_rollout_unique_rows_brute_force():
    rng = np.random.default_rng(5)
    prefix, group, k, Hkv = 32, 3, 2, 2
    B = 7  # two full groups and a ragged one
    L = rng.integers(prefix + 8, prefix + 40, size=B)
    seq_len = (L + k + 1).astype(np.int32)
    cap = 12
    idx = np.zeros((B, Hkv, cap), dtype=np.int32)
    n_sel = rng.integers(4, cap + 1, size=B).astype(np.int32)
    for b in range(B):
        for h in range(Hkv):
            # distinct positions, most of them inside the shared prefix so groups overlap
            idx[b, h, :n_sel[b]] = np.sort(rng.choice(prefix + 4, size=n_sel[b], replace=False))
    ver, draft = bench.rollout_unique_positions(seq_len, idx, n_sel, prefix, group, k)
    ref_ver, ref_draft = brute_unique(seq_len, idx, n_sel, prefix, group, k)
    assert ver == ref_ver
    assert draft == ref_draft


def test_rollout_block_table_aliases_prefix_pages():
    cfg = get_config(4, B=20)
    b = make_batch(cfg, parts=())
    prefix, group = cfg.lengths[1], cfg.lengths[5]
    shared = prefix // cfg.page
    bt = b.block_table
    npages = (b.seq_len.astype(np.int64) + cfg.page - 1) // cfg.page
    for s in range(cfg.B):
        assert np.array_equal(bt[s, :shared], bt[(s // group) * group, :shared])
    used = np.concatenate([bt[s, :npages[s]] for s in range(cfg.B)])
    # every physical page is used, and only the group prefixes are shared
    n_groups = (cfg.B + group - 1) // group
    assert len(np.unique(used)) == b.num_pages
    assert len(used) - b.num_pages == (cfg.B - n_groups) * shared


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_traffic_is_reported_only_for_the_profiled_source_and_shape(tmp_path, monkeypatch):
    import json

    import bench
    from s3r_inputs import get_config

    src = os.path.join(bench.ROOT, "self_sparse_speculative_amd", "csrc", "verify.hip")
    c5 = get_config(5)
    rec = {"source_sha": bench.source_sha(src), "bytes_per_launch": {"one_call": 123},
           "workload_shapes": {"one_call": bench.workload_shape(c5)}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "verify_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic(src, "one_call", c5) == 123
    assert bench.load_traffic(src, "one_call", get_config(5, Hq=16, Hkv=4)) is None   # another shape
    assert bench.load_traffic(src, "one_call", get_config(5, k=8)) is None
    assert bench.load_traffic(src, "pages", c5) is None                                # no record
    rec["source_sha"] = "0" * 16                                                       # another source
    (tmp_path / "profiles" / "verify_traffic.json").write_text(json.dumps(rec))
    assert bench.load_traffic(src, "one_call", c5) is None
