"""Back-to-back S3R rounds on one stream with every piece of state on the device.

A round is the library's calls in order (no computation here: this module
only sequences calls and owns the buffers they read and write):

    s3r_select                  on the scores the previous verification wrote (and the
                                draft steps' dispatch order, longest first);
    k x (s3r_kv_append          the draft token's K/V row at L + j - 1,
         s3r_sparse_decode_attn draft step j, attending up to L + j);
    s3r_kv_append               the k + 1 block rows at L .. L + k (they replace
                                the draft rows);
    s3r_verify_attn             the block against the whole cache, writing the
                                next round's scores;
    s3r_spec_sample             accept / resample;
    s3r_commit                  L += n_out, the pending token, the next round's
                                draft and verify lengths, the verified total.

Nothing crosses to the host between rounds, so a round can be captured once
in a HIP graph (torch.cuda.CUDAGraph) and replayed; every host-side bound
(selection capacity, draft attend bound, verification length) is the bound
over the whole run, given as ``max_len``.

[explainer] "S3R - Self-sparse speculative rollouts for RL - What does it
mean?", mechanism paragraph (k draft steps, one verification pass, a new
ranking of the cache after each round) and Jargon "Block efficiency (tau)"; [news] "Long-
context RL training stops waiting on autoregressive rollouts...",
Interpretation (verification recomputes the block against the full cache).
"""

import torch

from . import s3r


class RoundDriver:
    """Owns the device state of a run over one layer's paged cache.

    kv        PagedKV whose block table covers max_len positions per sequence
              (the pages are written by s3r_kv_append);
    ctx_len   int32 [B] device: committed lengths at the start (updated in place);
    scores    float32 [B][Hkv][stride >= max_len] device: first-round scores
              (rewritten by every verification); with page_scores, one score
              per page of 16 positions ([B][Hkv][stride >= ceil(max_len / 16)]),
              written by s3r_verify_attn_pages and read by s3r_select_pages;
    max_len   host bound on any sequence's cache length during the run
              (initial length + rounds * (k + 1)).
    """

    def __init__(self, kv: s3r.PagedKV, ctx_len: torch.Tensor, scores: torch.Tensor, *, k: int, Hq: int, V: int,
                 s_num: int, s_den: int, window: int, scale: float, temperature: float, max_len: int,
                 select_unit: int = 1, select_all_heads: bool = False, page_scores: bool = False):
        dev = ctx_len.device
        B = ctx_len.shape[0]
        Hkv, D = kv.num_kv_heads, kv.head_dim
        self.page_scores = bool(page_scores)
        if self.page_scores:
            select_unit = 16  # scores per page select whole pages
            if scores.shape[0] != B or scores.shape[1] != Hkv or scores.shape[2] < (max_len + 15) // 16:
                raise ValueError("page scores must be [B][Hkv][stride >= ceil(max_len / 16)]")
        elif scores.shape[0] != B or scores.shape[1] != Hkv or scores.shape[2] < max_len:
            raise ValueError("scores must be [B][Hkv][stride >= max_len]")
        if kv.block_table.shape[1] * 16 < max_len:
            raise ValueError("the block table must cover max_len positions")
        self.kv, self.ctx_len, self.scores = kv, ctx_len, scores
        self.B, self.k, self.Hq, self.Hkv, self.D, self.V = B, k, Hq, Hkv, D, V
        self.s_num, self.s_den, self.window = s_num, s_den, window
        self.scale, self.temperature, self.max_len = float(scale), float(temperature), int(max_len)
        i32 = dict(dtype=torch.int32, device=dev)
        self.select_unit, self.select_all_heads = int(select_unit), bool(select_all_heads)
        self.plain_select = self.select_unit == 1 and not self.select_all_heads
        self.cap = max(1, s3r.budget(self.max_len, s_num, s_den, window) if self.plain_select else
                       s3r.select_grouped_capacity(self.max_len, s_num, s_den, window, self.select_unit))
        self.max_attend = self.cap + k
        # lengths of the next round, derived once here; s3r_commit keeps them current
        self.cur_len = torch.stack([ctx_len + j for j in range(1, k + 1)]).to(torch.int32).contiguous() if k > 0 \
            else torch.empty((0, B), **i32)
        self.seq_len = (ctx_len + (k + 1)).to(torch.int32)
        self.pending = torch.full((B,), -1, **i32)
        self.verified = torch.zeros((1,), dtype=torch.int64, device=dev)
        self.idx = torch.empty((B, Hkv, self.cap), **i32)
        self.n_sel = torch.empty((B,), **i32)
        self.order = torch.empty((B,), **i32)
        self.draft_out = torch.empty((k, B, Hq, D), dtype=torch.float32, device=dev)
        self.draft_lse = torch.empty((k, B, Hq), dtype=torch.float32, device=dev)
        self.ver_out = torch.empty((B, k + 1, Hq, D), dtype=torch.float32, device=dev)
        self.ver_lse = torch.empty((B, k + 1, Hq), dtype=torch.float32, device=dev)
        self.tokens = torch.empty((B, k + 1), **i32)
        self.n_out = torch.empty((B,), **i32)
        self.accepted = torch.empty((B, max(k, 1)), dtype=torch.int8, device=dev)
        # the round's inputs (what the model hands the step), filled by set_inputs
        st = kv.k_pages.dtype
        self.q_draft = torch.empty((k, B, Hq, D), dtype=st, device=dev)
        self.k_draft = torch.empty((k, B, 1, Hkv, D), dtype=st, device=dev)
        self.v_draft = torch.empty((k, B, 1, Hkv, D), dtype=st, device=dev)
        self.q_verify = torch.empty((B, k + 1, Hq, D), dtype=st, device=dev)
        self.k_block = torch.empty((B, k + 1, Hkv, D), dtype=st, device=dev)
        self.v_block = torch.empty((B, k + 1, Hkv, D), dtype=st, device=dev)
        self.zt = torch.empty((B, k + 1, V), dtype=torch.float32, device=dev)
        self.zd = torch.empty((B, k, V), dtype=torch.float32, device=dev)
        self.d = torch.empty((B, k), **i32)
        self.u = torch.empty((B, k + 1), dtype=torch.float32, device=dev)
        self.ws = s3r.Workspace(dev)
        self.graph = None

    def set_inputs(self, q_draft, k_draft, v_draft, q_verify, k_block, v_block, zt, zd, d, u):
        """Copy one round's inputs (device tensors, generator layouts) into the driver's buffers."""
        self.q_draft.copy_(q_draft)
        self.k_draft.copy_(k_draft.reshape(self.k_draft.shape))
        self.v_draft.copy_(v_draft.reshape(self.v_draft.shape))
        self.q_verify.copy_(q_verify)
        self.k_block.copy_(k_block)
        self.v_block.copy_(v_block)
        self.zt.copy_(zt)
        self.zd.copy_(zd)
        self.d.copy_(d)
        self.u.copy_(u)

    def step(self):
        """Enqueue one round on the current stream."""
        k, ml = self.k, self.max_len
        if self.page_scores:
            s3r.select_pages(self.scores, self.ctx_len, ml, self.s_num, self.s_den, self.window,
                             all_heads=self.select_all_heads, idx=self.idx, n_sel=self.n_sel, ws=self.ws,
                             order=self.order)
        elif self.plain_select:
            s3r.select(self.scores, self.ctx_len, ml, self.s_num, self.s_den, self.window, idx=self.idx,
                       n_sel=self.n_sel, order=self.order)
        else:
            s3r.select_grouped(self.scores, self.ctx_len, ml, self.s_num, self.s_den, self.window,
                               unit=self.select_unit, all_heads=self.select_all_heads, idx=self.idx,
                               n_sel=self.n_sel, ws=self.ws, order=self.order)
        for j in range(1, k + 1):
            pos = self.ctx_len if j == 1 else self.cur_len[j - 2]
            s3r.kv_append(self.k_draft[j - 1], self.v_draft[j - 1], self.kv, pos, ml)
            s3r.sparse_decode_attn(self.q_draft[j - 1], self.kv, self.idx, self.n_sel, self.ctx_len,
                                   self.cur_len[j - 1], self.scale, self.max_attend, out=self.draft_out[j - 1],
                                   lse=self.draft_lse[j - 1], ws=self.ws, order=self.order)
        s3r.kv_append(self.k_block, self.v_block, self.kv, self.ctx_len, ml)
        if self.page_scores:
            s3r.verify_attn_pages(self.q_verify, self.kv, self.seq_len, k, self.scale, ml, out=self.ver_out,
                                  lse=self.ver_lse, page_scores=self.scores, ws=self.ws)
        else:
            s3r.verify_attn(self.q_verify, self.kv, self.seq_len, k, self.scale, ml, out=self.ver_out,
                            lse=self.ver_lse, scores=self.scores, ws=self.ws)
        s3r.spec_sample(self.zt, self.zd, self.d, self.u, self.temperature, tokens=self.tokens, n_out=self.n_out,
                        accepted=self.accepted if k > 0 else None, want_accepted=k > 0, ws=self.ws)
        s3r.commit(self.n_out, self.tokens, self.ctx_len, pending=self.pending,
                   cur_len=self.cur_len if k > 0 else None, seq_len=self.seq_len, verified=self.verified)

    def prepare(self):
        """Allocate the workspace of every call at the run's bounds (nothing is enqueued)."""
        B, k, Hq, D = self.B, self.k, self.Hq, self.D
        if not self.plain_select:
            lib = s3r.load()
            self.ws.get("select", max(1, int(lib.s3r_select_grouped_workspace_bytes(
                B, self.Hkv, self.max_len, self.s_num, self.s_den, self.window, self.select_unit,
                int(self.select_all_heads)))))
        self.ws.get("decode", s3r.sparse_decode_workspace_bytes(B, Hq, D, self.max_attend))
        wsb = s3r.verify_pages_workspace_bytes if self.page_scores else s3r.verify_workspace_bytes
        self.ws.get("verify", wsb(B, k, Hq, self.Hkv, D, self.kv.dtype_code, self.max_len))
        self.ws.get("sample", s3r.spec_sample_workspace_bytes(B, k, self.V))

    def capture(self):
        """Record one round in a HIP graph (replay() runs it; the driver's buffers are the graph's
        inputs and outputs)."""
        self.prepare()
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.step()
        return self.graph

    def replay(self):
        self.graph.replay()
