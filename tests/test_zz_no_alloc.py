"""s3r_spec_sample_noalloc (library-owned scratch, no workspace argument) against
s3r_spec_sample on the same inputs: bit-identical tokens, counts and decisions,
on two calls in a row, the second with a smaller batch (and a shorter draft),
and at temperature 0."""

import numpy as np
import pytest
import torch

import self_sparse_speculative_amd as s3r
from s3r_inputs import get_config, make_batch

pytestmark = pytest.mark.gpu


def _inputs(B, k, V, seed):
    cfg = get_config(2, B=B, k=k, V=V)
    b = make_batch(cfg, seed=seed, parts=("logits",))
    dev = torch.device("cuda")
    return {n: torch.from_numpy(getattr(b, n)).to(dev) for n in ("zt", "zd", "d", "u")}, float(b.temperature)


def _both(t, T):
    B, kp1, _ = t["zt"].shape
    k = kp1 - 1
    ref = s3r.spec_sample(t["zt"], t["zd"], t["d"], t["u"], T, ws=s3r.Workspace())
    tok = torch.full((B, kp1), -7, dtype=torch.int32, device="cuda")
    nout = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    acc = torch.full((B, k), 5, dtype=torch.int8, device="cuda") if k > 0 else None
    got = s3r.spec_sample_noalloc(t["zt"], t["zd"], t["d"], t["u"], T, tok, nout, acc)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("T", [None, 0.0])
def test_noalloc_matches_workspace_entry_point_twice(T):
    big, T1 = _inputs(96, 6, 151936, seed=1)
    small, _ = _inputs(20, 3, 151936, seed=2)
    TT = T1 if T is None else T
    for name, t in (("first call, B=96 k=6", big), ("second call, B=20 k=3", small)):
        print(f"[noalloc] {name} T={TT}", flush=True)
        (rt, rn, ra), (gt, gn, ga) = _both(t, TT)
        assert torch.equal(rt, gt), name
        assert torch.equal(rn, gn), name
        assert torch.equal(ra, ga), name


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    k, V = 6, 16
    B = 1
    while s3r.spec_sample_workspace_bytes(B, k, V) <= s3r.SAMPLE_SCRATCH_BYTES:
        B *= 2
    assert B <= 65535
    dev = torch.device("cuda")
    zt = torch.zeros((B, k + 1, V), device=dev)
    zd = torch.zeros((B, k, V), device=dev)
    d = torch.zeros((B, k), dtype=torch.int32, device=dev)
    u = torch.zeros((B, k + 1), device=dev)
    tok = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    nout = torch.empty((B,), dtype=torch.int32, device=dev)
    with pytest.raises(s3r.S3RError) as e:
        s3r.spec_sample_noalloc(zt, zd, d, u, 1.0, tok, nout)
    assert e.value.status == 3  # S3R_ERR_WORKSPACE
