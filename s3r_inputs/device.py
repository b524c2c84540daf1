"""K/V pages drawn on the GPU for workloads too large to draw on the host.

The 28-layer rollout workload holds about 7.7 GB of K/V per layer; drawing
all layers on the host would take far longer than the measured run, so the
benchmark draws each layer's pages N(0, 1) in bfloat16 on the device from a
torch generator seeded per (seed, config, layer). Everything else of that
workload (lengths, block tables, queries, scores, logits) comes from the
host generator. Tests copy pages drawn here back to the host to check the
same inputs the benchmark times. Like the rest of this package it draws
random numbers only.
"""


def layer_seed(seed: int, cid: int, layer: int) -> int:
    return ((seed * 1000003 + cid) * 1000003 + layer) & ((1 << 63) - 1)


def draw_pages_on_device(cfg, num_pages: int, layer: int, seed: int, torch, device="cuda"):
    """(k_pages, v_pages) [num_pages][Hkv][page][D] bfloat16 ~ N(0, 1), drawn on the device."""
    gen = torch.Generator(device=device)
    gen.manual_seed(layer_seed(seed, cfg.cid, layer))
    shape = (num_pages, cfg.Hkv, cfg.page, cfg.D)
    kp = torch.empty(shape, dtype=torch.bfloat16, device=device).normal_(generator=gen)
    vp = torch.empty(shape, dtype=torch.bfloat16, device=device).normal_(generator=gen)
    return kp, vp
