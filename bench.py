#!/usr/bin/env python3
"""Benchmark of one S3R round on one MI355X: select, k sparse draft steps,
dense block verification (with next-round scores) and exact speculative
sampling, all through the C ABI of libs3r.so, on one stream
(--overlap-scores: the next round's scores are formed on a second stream
while sampling runs).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]

Workload (default): Qwen3-8B attention shapes (Hq 32, Hkv 8, head_dim 128,
bf16 KV, page 16), batch 128, 24K committed context per sequence, budget
s = 0.05 with a 64-position window, k = 6 drafts, vocabulary 151936 with
N(0, 3) target logits and draft logits = target + N(0, 0.3). Inputs are
seeded synthetic data resident in HBM before timing starts.

A step is one round over the batch. Each round's selection reads the scores
the previous round's verification wrote. Prints one JSON line.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--s", type=str, default=None, help="budget as num/den, e.g. 1/20")
    ap.add_argument("--k", type=int, default=None)
    ap.add_argument("--sigma", type=float, default=None)
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seqs", type=int, default=64, help="sequences in the oracle's timed CPU sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline (profiling runs)")
    ap.add_argument("--sweep", action="store_true",
                    help="run all 48 points of the 24K sweep (s x k x draft noise), one JSON line per point")
    ap.add_argument("--overlap-scores", action="store_true",
                    help="verify as s3r_verify_attn_deferred + s3r_verify_scores on a side stream, concurrent "
                         "with sampling (default: one s3r_verify_attn call on the launch stream)")
    ap.add_argument("--copy-gib", type=float, default=2.0,
                    help="size of the device-to-device copy timed as the HBM reference (0 to skip)")
    return ap.parse_args()


def to_dev(batch, s3r, torch):
    def st(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    t = {
        "ctx_len": torch.from_numpy(batch.ctx_len).cuda(),
        "seq_len": torch.from_numpy(batch.seq_len).cuda(),
        "kv": s3r.PagedKV(st(batch.k_pages), st(batch.v_pages), torch.from_numpy(batch.block_table).cuda()),
        "q_draft": st(batch.q_draft),
        "q_verify": st(batch.q_verify),
        "scores": torch.from_numpy(batch.scores).cuda(),
        "zt": torch.from_numpy(batch.zt).cuda(),
        "zd": torch.from_numpy(batch.zd).cuda(),
        "u": torch.from_numpy(batch.u).cuda(),
        "d": torch.from_numpy(batch.d).cuda(),
    }
    return t


def source_sha(path):
    """Hash of the code in a source file, ignoring // comments and blank lines."""
    lines = []
    for ln in open(path).read().splitlines():
        code = ln.split("//", 1)[0].rstrip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def load_traffic(kernel_src, key):
    """Counter-measured HBM bytes per launch from the committed summary, if it is current.

    key: "rows" (split pass + output merge, the deferred call) or "one_call" (s3r_verify_attn)."""
    path = os.path.join(ROOT, "profiles", "verify_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != source_sha(kernel_src):
        return None
    per = rec.get("bytes_per_launch")
    return per.get(key) if isinstance(per, dict) else None


def cpu_baseline(cfg, nseq, seed):
    """The fp64 oracle, timed on a bounded sample of the same workload on the host cores."""
    import oracle
    from s3r_inputs import make_batch

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    batch = make_batch(cfg, seed=seed, B=nseq)
    t0 = time.perf_counter()
    tokens = 0
    for b in range(nseq):
        L = int(batch.ctx_len[b])
        idx = [oracle.select(batch.scores[b, kv], L, cfg.s_num, cfg.s_den, cfg.window) for kv in range(cfg.Hkv)]
        n = len(idx[0])
        for j in range(1, cfg.k + 1):
            oracle.sparse_decode(batch.q_draft[j - 1, b], batch.k_pages, batch.v_pages, batch.block_table[b], idx, n,
                                 L, L + j, float(batch.scale))
        oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b], int(batch.seq_len[b]),
                      cfg.k, float(batch.scale))
        _, n_out, _ = oracle.spec_sample(batch.zt[b], batch.zd[b], batch.d[b], batch.u[b], batch.temperature)
        tokens += int(n_out)
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "verified tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"full round (select, {cfg.k} draft steps, verify with scores, sampling) for the first {nseq} "
                      f"of {cfg.B} sequences of the same workload, fp64 numpy, {dt:.1f} s, {tokens} tokens",
            "seconds": dt, "host_cpus": len(os.sched_getaffinity(0))}


def measure_round(args, cfg, batch, t, s3r, torch):
    """Time args.steps rounds (after args.warmup) of the step over resident inputs."""
    B, k, Hq, Hkv, D = cfg.B, cfg.k, cfg.Hq, cfg.Hkv, cfg.D
    max_ctx = int(batch.ctx_len.max())
    max_seq = int(batch.seq_len.max())
    cap = s3r.budget(max_ctx, cfg.s_num, cfg.s_den, cfg.window)
    max_attend = cap + k
    scale = float(batch.scale)
    T = float(batch.temperature)
    ws = s3r.Workspace()
    idx = torch.empty((B, Hkv, cap), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((B,), dtype=torch.int32, device="cuda")
    cur = [t["ctx_len"] + j for j in range(1, k + 1)]
    dout = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    dlse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    vout = torch.empty((B, k + 1, Hq, D), dtype=torch.float32, device="cuda")
    vlse = torch.empty((B, k + 1, Hq), dtype=torch.float32, device="cuda")
    scores = t["scores"]  # verification rewrites it for the next round's selection
    tokens = torch.empty((B, k + 1), dtype=torch.int32, device="cuda")
    n_out = torch.empty((B,), dtype=torch.int32, device="cuda")
    accepted = torch.empty((B, k), dtype=torch.int8, device="cuda")

    # With --overlap-scores the next round's scores, which only the next select
    # reads, are formed on a side stream (default priority) while sampling
    # runs; the round ends when both streams are done.
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    rows_done = torch.cuda.Event()

    def step(ev=None, sev=None):
        if ev is not None:
            ev[0].record()
        s3r.select(scores, t["ctx_len"], max_ctx, cfg.s_num, cfg.s_den, cfg.window, idx=idx, n_sel=n_sel)
        if ev is not None:
            ev[1].record()
        for j in range(k):
            s3r.sparse_decode_attn(t["q_draft"][j], t["kv"], idx, n_sel, t["ctx_len"], cur[j], scale, max_attend,
                                   out=dout, lse=dlse, ws=ws)
        if ev is not None:
            ev[2].record()
        if not args.overlap_scores:
            s3r.verify_attn(t["q_verify"], t["kv"], t["seq_len"], k, scale, max_seq, out=vout, lse=vlse,
                            scores=scores, ws=ws)
            if ev is not None:
                ev[3].record()
        else:
            s3r.verify_attn_deferred(t["q_verify"], t["kv"], t["seq_len"], k, scale, max_seq, out=vout, lse=vlse,
                                     ws=ws)
            if ev is not None:
                ev[3].record()
            rows_done.record(main)
            side.wait_event(rows_done)
            if sev is not None:
                sev[0].record(side)
            s3r.verify_scores(t["kv"], t["seq_len"], B, k, Hq, D, max_seq, scores=scores, ws=ws, stream=side)
            if sev is not None:
                sev[1].record(side)
        s3r.spec_sample(t["zt"], t["zd"], t["d"], t["u"], T, tokens=tokens, n_out=n_out, accepted=accepted, ws=ws)
        if ev is not None:
            ev[4].record()
        if args.overlap_scores:
            main.wait_stream(side)  # the next select reads the scores

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    tok_a = n_out.clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(tok_a, n_out), "rounds over the same inputs must give the same token counts"
    verified = int(n_out.sum().item())
    nsel_np = n_sel.cpu().numpy()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    sevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(evs[i], sevs[i])
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    phase = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs])  # ms
    t_sel, t_draft, t_ver, t_smp = phase.mean(axis=0)
    t_scores = None if not args.overlap_scores else float(np.mean([e[0].elapsed_time(e[1]) for e in sevs]))
    round_median = float(np.median([e[0].elapsed_time(e[4]) for e in evs]))

    # algorithmic bytes per launch (per-unit figures: K and V rows, index / score words,
    # q and output rows once per (sequence, head, row))
    e = 2 if cfg.dtype == "bf16" else 4
    L = batch.ctx_len.astype(np.int64)
    S = batch.seq_len.astype(np.int64)
    kv_row = 2 * D * e  # one K row + one V row
    # the verify call on the launch stream: K and V rows, q, output rows and lse; in
    # the one-call form also the scores it writes
    ver_bytes = int(Hkv * S.sum() * (kv_row + (0 if args.overlap_scores else 4)) + B * (k + 1) * Hq * (D * e + D * 4 + 4))
    score_bytes = int(Hkv * S.sum() * 4)
    draft_bytes = int(sum(Hkv * (nsel_np.astype(np.int64) + j).sum() * (kv_row + 4) for j in range(1, k + 1))
                      + k * B * Hq * (D * e + D * 4 + 4))
    sel_bytes = int(Hkv * L.sum() * 4 + Hkv * nsel_np.astype(np.int64).sum() * 4)
    smp_bytes = int(B * (2 * k + 1) * cfg.V * 4)
    kv_bytes = ver_bytes + draft_bytes
    kv_ms = t_ver + t_draft
    ver_gbs = ver_bytes / (t_ver * 1e-3) / 1e9
    round_bytes = kv_bytes + sel_bytes + smp_bytes + (score_bytes if args.overlap_scores else 0)
    return {
        "value": verified / (ms_step * 1e-3), "ms_step": ms_step, "round_ms_median": round_median,
        "verified": verified, "B": B, "max_seq": max_seq, "ver_bytes": ver_bytes, "ver_gbs": ver_gbs,
        "t_ver": float(t_ver),
        "breakdown": {
            "verified_tokens_per_round": verified,
            "tokens_per_sequence": round(verified / B, 4),
            "ms": {"select": round(float(t_sel), 4), "draft_k_steps": round(float(t_draft), 4),
                   "verify": round(float(t_ver), 4), "spec_sample": round(float(t_smp), 4),
                   "verify_scores_side_stream": None if t_scores is None else round(t_scores, 4),
                   "round_median": round(round_median, 4)},
            "GBs": {"select": round(sel_bytes / (t_sel * 1e-3) / 1e9, 1),
                    "draft": round(draft_bytes / (t_draft * 1e-3) / 1e9, 1),
                    "verify": round(ver_gbs, 1),
                    "spec_sample": round(smp_bytes / (t_smp * 1e-3) / 1e9, 1),
                    "verify_scores_side_stream": None if t_scores is None else round(score_bytes / (t_scores * 1e-3) / 1e9, 1)},
            "draft_plus_verify_kv_GBs": round(kv_bytes / (kv_ms * 1e-3) / 1e9, 1),
            "draft_plus_verify_frac_of_hbm_peak": round(kv_bytes / (kv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "round_algorithmic_bytes": round_bytes,
            "round_frac_of_hbm_peak": round(round_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
    }


def reference_rates(args, torch):
    """Plain device copy and read of known size: the HBM references (the copy is also the
    calibration kernel of the byte counters)."""
    if args.copy_gib <= 0:
        return None, None
    n = int(args.copy_gib * (1 << 30)) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 4 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9  # read + write bytes per copy
    acc = src.sum()
    c0.record()
    for _ in range(5):
        acc = src.sum()
    c1.record()
    torch.cuda.synchronize()
    read_gbs = n * 4 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst, acc
    return copy_gbs, read_gbs


def run_sweep(args, torch, s3r):
    """All 48 points of the 24K sweep (s x k x draft noise), one JSON line each."""
    from dataclasses import replace

    from s3r_inputs import make_batch
    from s3r_inputs.configs import CONFIGS, SWEEP_K, SWEEP_S, SWEEP_SIGMA
    base = CONFIGS[5]
    for k in SWEEP_K:
        cfg_k = replace(base, k=k)
        batch = make_batch(cfg_k, seed=args.seed)
        t = to_dev(batch, s3r, torch)
        scores0 = t["scores"].clone()
        for sig in SWEEP_SIGMA:
            lb = make_batch(replace(cfg_k, noise_std=sig), seed=args.seed, parts=("logits",))
            for name in ("zt", "zd", "d", "u"):
                t[name] = torch.from_numpy(getattr(lb, name)).cuda()
            batch.zt, batch.zd, batch.d, batch.u = lb.zt, lb.zd, lb.d, lb.u
            for s_num, s_den in SWEEP_S:
                cfg = replace(cfg_k, s_num=s_num, s_den=s_den, noise_std=sig)
                t["scores"].copy_(scores0)  # every point starts from the same first-round scores
                r = measure_round(args, cfg, batch, t, s3r, torch)
                print(json.dumps({"sweep": "qwen3-8b-24k", "s": f"{s_num}/{s_den}", "k": k, "sigma": sig,
                                  "value": round(r["value"], 1), "unit": "verified tokens/s",
                                  "ms_per_step": round(r["ms_step"], 4), **r["breakdown"]}), flush=True)
        del t, batch
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the hot path is single-GPU; "
              "sharding is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch

    import self_sparse_speculative_amd as s3r
    from s3r_inputs import get_config, make_batch

    torch.cuda.set_device(0)
    if args.sweep:
        run_sweep(args, torch, s3r)
        return
    ov = {}
    if args.s:
        num, den = args.s.split("/")
        ov["s_num"], ov["s_den"] = int(num), int(den)
    if args.k is not None:
        ov["k"] = args.k
    if args.sigma is not None:
        ov["noise_std"] = args.sigma
    if args.batch is not None:
        ov["B"] = args.batch
    cfg = get_config(args.config, **ov)
    if cfg.layers != 1:
        cfg = get_config(args.config, layers=1, **ov)
    print(f"[bench] generating {cfg.name} B={cfg.B} k={cfg.k} s={cfg.s_num}/{cfg.s_den}", file=sys.stderr, flush=True)
    t0 = time.time()
    batch = make_batch(cfg, seed=args.seed)
    t = to_dev(batch, s3r, torch)
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    r = measure_round(args, cfg, batch, t, s3r, torch)
    traffic = load_traffic(os.path.join(ROOT, "self_sparse_speculative_amd", "csrc", "verify.hip"),
                           "rows" if args.overlap_scores else "one_call")
    copy_gbs, read_gbs = reference_rates(args, torch)
    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, min(args.cpu_seqs, cfg.B), args.seed)
    B, k, Hq, Hkv, D = cfg.B, cfg.k, cfg.Hq, cfg.Hkv, cfg.D
    breakdown = dict(r["breakdown"])
    breakdown["device_copy_GBs"] = None if copy_gbs is None else round(copy_gbs, 1)
    breakdown["device_read_GBs"] = None if read_gbs is None else round(read_gbs, 1)
    res = {
        "metric": "verified tokens/s per draft+verify round; KV-read GB/s as % of HBM peak",
        "value": round(r["value"], 1),
        "unit": "verified tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: one attention layer, B={B}, Hq={Hq}, Hkv={Hkv}, head_dim={D}, {cfg.dtype} paged KV "
                        f"(page 16), context {cfg.lengths}, s={cfg.s_num}/{cfg.s_den}, window {cfg.window}, k={k}, "
                        f"V={cfg.V}, target N(0,{cfg.target_std}), draft noise {cfg.noise_std}, T={cfg.temperature}",
            "global_batch": B,
            "seq_len": r["max_seq"],
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": ("s3r_verify_attn: verify_mfma_kernel (split pass) + verify_finalize_kernel (merge, scores)"
                       if not args.overlap_scores else
                       "s3r_verify_attn_deferred: verify_mfma_kernel (split pass) + verify_finalize_kernel (output merge)"),
            "bound": "hbm",
            "achieved": round(r["ver_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["ver_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": r["ver_bytes"],
            "ms_per_launch": round(r["t_ver"], 4),
        },
        "cpu_baseline": cpu,
        "breakdown": breakdown,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
