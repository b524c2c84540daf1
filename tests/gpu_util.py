"""Helpers for the GPU parity tests: move a seeded batch to the device and run
the library's four calls on it. Nothing here computes any step of the method."""

import numpy as np
import torch

import self_sparse_speculative_amd as s3r


def to_dev_storage(a: np.ndarray, device="cuda"):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_dev(batch, device="cuda"):
    t = {}
    t["ctx_len"] = torch.from_numpy(batch.ctx_len).to(device)
    t["seq_len"] = torch.from_numpy(batch.seq_len).to(device)
    if batch.k_pages is not None:
        t["kv"] = s3r.PagedKV(to_dev_storage(batch.k_pages, device), to_dev_storage(batch.v_pages, device),
                              torch.from_numpy(batch.block_table).to(device))
    if batch.q_draft is not None:
        t["q_draft"] = to_dev_storage(batch.q_draft, device)
        t["q_verify"] = to_dev_storage(batch.q_verify, device)
    if batch.scores is not None:
        t["scores"] = torch.from_numpy(batch.scores).to(device)
    if batch.zt is not None:
        t["zt"] = torch.from_numpy(batch.zt).to(device)
        t["zd"] = torch.from_numpy(batch.zd).to(device)
        t["u"] = torch.from_numpy(batch.u).to(device)
        t["d"] = torch.from_numpy(batch.d).to(device)
    return t


def nsel_cap(cfg, batch):
    return s3r.budget(int(batch.ctx_len.max()), cfg.s_num, cfg.s_den, cfg.window)


def run_select(cfg, batch, t, scores=None, order=None):
    sc = t["scores"] if scores is None else scores
    return s3r.select(sc, t["ctx_len"], int(batch.ctx_len.max()), cfg.s_num, cfg.s_den, cfg.window,
                      nsel_cap=nsel_cap(cfg, batch), order=order)


def run_draft_steps(cfg, batch, t, idx, n_sel, order=None):
    outs = []
    max_attend = nsel_cap(cfg, batch) + cfg.k
    for j in range(1, cfg.k + 1):
        cur = t["ctx_len"] + j
        o, lse = s3r.sparse_decode_attn(t["q_draft"][j - 1], t["kv"], idx, n_sel, t["ctx_len"], cur,
                                        float(batch.scale), max_attend, order=order)
        outs.append((o, lse))
    return outs


def run_verify(cfg, batch, t, want_scores=True):
    return s3r.verify_attn(t["q_verify"], t["kv"], t["seq_len"], cfg.k, float(batch.scale),
                           int(batch.seq_len.max()), want_scores=want_scores)


def run_sample(cfg, batch, t, temperature=None):
    T = float(batch.temperature) if temperature is None else temperature
    return s3r.spec_sample(t["zt"], t["zd"], t["d"], t["u"], T)


def rel_err_rows(got: np.ndarray, ref: np.ndarray) -> float:
    """max over output vectors of max|got - ref| / max(max|ref|, 1e-6) (last axis = vector)."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-6)
    return float((num / den).max())
