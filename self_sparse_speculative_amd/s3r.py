"""Thin ctypes binding of libs3r.so (argument marshalling only).

Every computation runs in the HIP kernels of libs3r.so; this module turns
torch device tensors into pointers, allocates output and workspace tensors
when the caller does not pass them, and raises on a non-OK status. It never
computes any step of the method itself and has no CPU fallback: if the
library is missing, loading it raises.

The functions mirror the C entry points of include/s3r.h:
``select``, ``sparse_decode_attn``, ``verify_attn``, ``spec_sample``, the
multi-round ``kv_append`` and ``commit``, plus the ``budget`` host helper and
the ``*_workspace_bytes`` queries.
"""

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libs3r.so")
_lib = None
_lock = threading.Lock()

S3R_OK, S3R_ERR_INVALID_ARG, S3R_ERR_UNSUPPORTED, S3R_ERR_WORKSPACE, S3R_ERR_HIP = range(5)
S3R_F32, S3R_BF16 = 0, 1

EXPORTED = (
    "s3r_status_string", "s3r_version", "s3r_budget", "s3r_select",
    "s3r_select_grouped_capacity", "s3r_select_grouped_workspace_bytes", "s3r_select_grouped",
    "s3r_sparse_decode_workspace_bytes", "s3r_sparse_decode_attn",
    "s3r_verify_workspace_bytes", "s3r_verify_attn", "s3r_verify_attn_deferred", "s3r_verify_scores",
    "s3r_spec_sample_workspace_bytes", "s3r_spec_sample", "s3r_kv_append", "s3r_commit",
    "s3r_length_order", "s3r_spec_sample_noalloc", "s3r_verify_pages_workspace_bytes", "s3r_verify_attn_pages",
    "s3r_select_pages", "s3r_read_pattern_sink_words", "s3r_read_verify_pattern", "s3r_read_draft_pattern",
)
SAMPLE_SCRATCH_BYTES = 8 << 20  # S3R_SAMPLE_SCRATCH_BYTES


class PagedKVStruct(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class S3RError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libs3r.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m self_sparse_speculative_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        L.s3r_status_string.restype = ctypes.c_char_p
        L.s3r_status_string.argtypes = [ctypes.c_int]
        L.s3r_version.restype = i32
        L.s3r_version.argtypes = []
        L.s3r_budget.restype = i32
        L.s3r_budget.argtypes = [i32, i32, i32, i32]
        L.s3r_select.restype = ctypes.c_int
        L.s3r_select.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, vp, i32, vp, vp, vp]
        L.s3r_select_grouped_capacity.restype = i32
        L.s3r_select_grouped_capacity.argtypes = [i32, i32, i32, i32, i32]
        L.s3r_select_grouped_workspace_bytes.restype = sz
        L.s3r_select_grouped_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
        L.s3r_select_grouped.restype = ctypes.c_int
        L.s3r_select_grouped.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, i32, vp, vp, vp,
                                         sz, vp]
        L.s3r_sparse_decode_workspace_bytes.restype = sz
        L.s3r_sparse_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.s3r_sparse_decode_attn.restype = ctypes.c_int
        L.s3r_sparse_decode_attn.argtypes = [vp, ctypes.POINTER(PagedKVStruct), vp, i32, vp, vp, vp, vp, i32,
                                             i32, f32, i32, vp, vp, vp, sz, vp]
        L.s3r_length_order.restype = ctypes.c_int
        L.s3r_length_order.argtypes = [vp, i32, vp, vp]
        L.s3r_verify_workspace_bytes.restype = sz
        L.s3r_verify_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.s3r_verify_attn.restype = ctypes.c_int
        L.s3r_verify_attn.argtypes = [vp, ctypes.POINTER(PagedKVStruct), vp, i32, i32, i32, f32, i32, vp,
                                      vp, vp, i32, vp, sz, vp]
        L.s3r_verify_pages_workspace_bytes.restype = sz
        L.s3r_verify_pages_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.s3r_verify_attn_pages.restype = ctypes.c_int
        L.s3r_verify_attn_pages.argtypes = [vp, ctypes.POINTER(PagedKVStruct), vp, i32, i32, i32, f32, i32, vp,
                                            vp, vp, i32, vp, sz, vp]
        L.s3r_select_pages.restype = ctypes.c_int
        L.s3r_select_pages.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, vp, i32, vp, vp, vp, sz, vp]
        L.s3r_verify_attn_deferred.restype = ctypes.c_int
        L.s3r_verify_attn_deferred.argtypes = [vp, ctypes.POINTER(PagedKVStruct), vp, i32, i32, i32, f32, i32,
                                               vp, vp, vp, sz, vp]
        L.s3r_verify_scores.restype = ctypes.c_int
        L.s3r_verify_scores.argtypes = [ctypes.POINTER(PagedKVStruct), vp, i32, i32, i32, i32, vp, i32, vp, sz,
                                        vp]
        L.s3r_spec_sample_workspace_bytes.restype = sz
        L.s3r_spec_sample_workspace_bytes.argtypes = [i32, i32, i32]
        L.s3r_spec_sample.restype = ctypes.c_int
        L.s3r_spec_sample.argtypes = [vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, vp, vp, sz, vp]
        L.s3r_spec_sample_noalloc.restype = ctypes.c_int
        L.s3r_spec_sample_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, vp, vp]
        L.s3r_read_pattern_sink_words.restype = sz
        L.s3r_read_pattern_sink_words.argtypes = [i32, i32, i32, i32]
        L.s3r_read_verify_pattern.restype = ctypes.c_int
        L.s3r_read_verify_pattern.argtypes = [ctypes.POINTER(PagedKVStruct), vp, i32, i32, vp, sz, vp]
        L.s3r_read_draft_pattern.restype = ctypes.c_int
        L.s3r_read_draft_pattern.argtypes = [ctypes.POINTER(PagedKVStruct), vp, i32, vp, vp, vp, i32, i32, vp, sz,
                                             vp]
        L.s3r_kv_append.restype = ctypes.c_int
        L.s3r_kv_append.argtypes = [vp, vp, ctypes.POINTER(PagedKVStruct), vp, i32, i32, i32, vp]
        L.s3r_commit.restype = ctypes.c_int
        L.s3r_commit.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp, vp, vp]
        _lib = L
        return L


def status_string(status: int) -> str:
    return load().s3r_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != S3R_OK:
        raise S3RError(status, where)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Workspace:
    """Caller-owned scratch memory for the library calls (one per stream)."""

    def __init__(self, device=None):
        self.device = torch.device("cuda") if device is None else torch.device(device)
        self._buf = {}

    def get(self, name: str, nbytes: int):
        buf = self._buf.get(name)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=self.device)
            self._buf[name] = buf
        return buf


_default_ws = {}


def _ws(ws, device):
    if ws is not None:
        return ws
    key = str(device)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


class PagedKV:
    """Device paged KV cache: k/v [num_pages][Hkv][16][D] (float32 or bfloat16), block_table [B][max_pages] int32."""

    def __init__(self, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor):
        if k_pages.shape != v_pages.shape or k_pages.dtype != v_pages.dtype or k_pages.dim() != 4:
            raise ValueError("k_pages and v_pages must share one [pages][Hkv][page][D] shape and dtype")
        if block_table.dtype != torch.int32 or block_table.dim() != 2:
            raise ValueError("block_table must be int32 [B][max_pages]")
        if k_pages.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("K/V dtype must be float32 or bfloat16")
        self.k_pages, self.v_pages, self.block_table = k_pages, v_pages, block_table
        n, hkv, page, d = k_pages.shape
        self.struct = PagedKVStruct(k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(), n,
                                    block_table.shape[1], hkv, d, page,
                                    S3R_BF16 if k_pages.dtype == torch.bfloat16 else S3R_F32)

    @property
    def num_kv_heads(self):
        return self.k_pages.shape[1]

    @property
    def head_dim(self):
        return self.k_pages.shape[3]

    @property
    def dtype_code(self):
        return self.struct.dtype


def budget(L: int, s_num: int, s_den: int, window: int) -> int:
    return int(load().s3r_budget(int(L), int(s_num), int(s_den), int(window)))


def select(scores, ctx_len, max_ctx_len, s_num, s_den, window, idx=None, n_sel=None, nsel_cap=None, stream=None,
           order=None):
    """s3r_select. scores f32 [B][Hkv][stride], ctx_len i32 [B]; order: i32 [B] written with the draft
    dispatch order when given. Returns (idx, n_sel)."""
    L = load()
    B, Hkv, stride = scores.shape
    if nsel_cap is None:
        nsel_cap = idx.shape[2] if idx is not None else max(1, budget(max_ctx_len, s_num, s_den, window))
    if idx is None:
        idx = torch.empty((B, Hkv, nsel_cap), dtype=torch.int32, device=scores.device)
    if n_sel is None:
        n_sel = torch.empty((B,), dtype=torch.int32, device=scores.device)
    _check(L.s3r_select(_ptr(scores), stride, _ptr(ctx_len), B, Hkv, int(max_ctx_len), int(s_num), int(s_den),
                        int(window), _ptr(idx), int(nsel_cap), _ptr(n_sel), _ptr(order), _stream(stream)),
           "s3r_select")
    return idx, n_sel


def select_grouped_capacity(max_ctx_len, s_num, s_den, window, unit) -> int:
    return int(load().s3r_select_grouped_capacity(int(max_ctx_len), int(s_num), int(s_den), int(window), int(unit)))


def select_grouped(scores, ctx_len, max_ctx_len, s_num, s_den, window, unit=16, all_heads=False, idx=None,
                   n_sel=None, nsel_cap=None, ws=None, stream=None, order=None):
    """s3r_select_grouped: whole pages (unit 16) and/or one kept set per sequence (all_heads).
    Returns (idx [B][Hkv][cap], n_sel [B])."""
    L = load()
    B, Hkv, stride = scores.shape
    if nsel_cap is None:
        nsel_cap = idx.shape[2] if idx is not None else max(1, select_grouped_capacity(max_ctx_len, s_num, s_den,
                                                                                        window, unit))
    if idx is None:
        idx = torch.empty((B, Hkv, nsel_cap), dtype=torch.int32, device=scores.device)
    if n_sel is None:
        n_sel = torch.empty((B,), dtype=torch.int32, device=scores.device)
    nb = int(L.s3r_select_grouped_workspace_bytes(B, Hkv, int(max_ctx_len), int(s_num), int(s_den), int(window),
                                                  int(unit), int(bool(all_heads))))
    buf = _ws(ws, scores.device).get("select", max(nb, 1))
    _check(L.s3r_select_grouped(_ptr(scores), stride, _ptr(ctx_len), B, Hkv, int(max_ctx_len), int(s_num),
                                int(s_den), int(window), int(unit), int(bool(all_heads)), _ptr(idx), int(nsel_cap),
                                _ptr(n_sel), _ptr(order), _ptr(buf), buf.numel(), _stream(stream)),
           "s3r_select_grouped")
    return idx, n_sel


def select_pages(page_scores, ctx_len, max_ctx_len, s_num, s_den, window, all_heads=False, idx=None, n_sel=None,
                 nsel_cap=None, ws=None, stream=None, order=None):
    """s3r_select_pages: whole pages chosen on scores given per page (page_scores [B][Hkv][page_stride]).
    Returns (idx [B][Hkv][cap], n_sel [B])."""
    L = load()
    B, Hkv, stride = page_scores.shape
    if nsel_cap is None:
        nsel_cap = idx.shape[2] if idx is not None else max(1, select_grouped_capacity(max_ctx_len, s_num, s_den,
                                                                                        window, 16))
    if idx is None:
        idx = torch.empty((B, Hkv, nsel_cap), dtype=torch.int32, device=page_scores.device)
    if n_sel is None:
        n_sel = torch.empty((B,), dtype=torch.int32, device=page_scores.device)
    nb = int(L.s3r_select_grouped_workspace_bytes(B, Hkv, int(max_ctx_len), int(s_num), int(s_den), int(window), 16,
                                                  int(bool(all_heads))))
    buf = _ws(ws, page_scores.device).get("select", max(nb, 1))
    _check(L.s3r_select_pages(_ptr(page_scores), stride, _ptr(ctx_len), B, Hkv, int(max_ctx_len), int(s_num),
                              int(s_den), int(window), int(bool(all_heads)), _ptr(idx), int(nsel_cap), _ptr(n_sel),
                              _ptr(order), _ptr(buf), buf.numel(), _stream(stream)), "s3r_select_pages")
    return idx, n_sel


def sparse_decode_workspace_bytes(B, Hq, head_dim, max_attend) -> int:
    return int(load().s3r_sparse_decode_workspace_bytes(B, Hq, head_dim, max_attend))


def length_order(lengths, out=None, stream=None):
    """s3r_length_order: int32 [B] device permutation, longest first (stable)."""
    L = load()
    B = lengths.shape[0]
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=lengths.device)
    _check(L.s3r_length_order(_ptr(lengths), B, _ptr(out), _stream(stream)), "s3r_length_order")
    return out


def sparse_decode_attn(q, kv: PagedKV, idx, n_sel, sel_len, cur_len, scale, max_attend, out=None, lse=None,
                       want_lse=True, ws=None, stream=None, order=None):
    """s3r_sparse_decode_attn. q [B][Hq][D]; order: int32 [B] dispatch permutation or None.
    Returns (out f32 [B][Hq][D], lse f32 [B][Hq] or None)."""
    L = load()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    nb = sparse_decode_workspace_bytes(B, Hq, D, int(max_attend))
    buf = _ws(ws, q.device).get("decode", nb)
    _check(L.s3r_sparse_decode_attn(_ptr(q), ctypes.byref(kv.struct), _ptr(idx), idx.shape[2], _ptr(n_sel),
                                    _ptr(sel_len), _ptr(cur_len), _ptr(order), B, Hq, float(scale), int(max_attend),
                                    _ptr(out), _ptr(lse), _ptr(buf), buf.numel(), _stream(stream)),
           "s3r_sparse_decode_attn")
    return out, lse


def verify_workspace_bytes(B, k, Hq, Hkv, head_dim, dtype_code, max_seq_len) -> int:
    return int(load().s3r_verify_workspace_bytes(B, k, Hq, Hkv, head_dim, dtype_code, max_seq_len))


def verify_attn(q, kv: PagedKV, seq_len, k, scale, max_seq_len, out=None, lse=None, scores=None,
                want_scores=True, want_lse=True, score_stride=None, ws=None, stream=None):
    """s3r_verify_attn. q [B][k+1][Hq][D]. Returns (out, lse, scores)."""
    L = load()
    B, kp1, Hq, D = q.shape
    assert kp1 == k + 1
    Hkv = kv.num_kv_heads
    if out is None:
        out = torch.empty((B, k + 1, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, k + 1, Hq), dtype=torch.float32, device=q.device)
    if scores is None and want_scores:
        stride = int(max_seq_len) if score_stride is None else int(score_stride)
        scores = torch.empty((B, Hkv, stride), dtype=torch.float32, device=q.device)
    stride = scores.shape[2] if scores is not None else 0
    nb = verify_workspace_bytes(B, k, Hq, Hkv, D, kv.dtype_code, int(max_seq_len))
    buf = _ws(ws, q.device).get("verify", nb)
    _check(L.s3r_verify_attn(_ptr(q), ctypes.byref(kv.struct), _ptr(seq_len), B, int(k), Hq, float(scale),
                             int(max_seq_len), _ptr(out), _ptr(lse), _ptr(scores), stride, _ptr(buf),
                             buf.numel(), _stream(stream)), "s3r_verify_attn")
    return out, lse, scores


def verify_pages_workspace_bytes(B, k, Hq, Hkv, D, dtype_code, max_seq_len) -> int:
    return int(load().s3r_verify_pages_workspace_bytes(B, k, Hq, Hkv, D, dtype_code, max_seq_len))


def verify_attn_pages(q, kv: PagedKV, seq_len, k, scale, max_seq_len, out=None, lse=None, page_scores=None,
                      want_lse=True, page_stride=None, ws=None, stream=None):
    """s3r_verify_attn_pages. q [B][k+1][Hq][D]. Returns (out, lse, page_scores [B][Hkv][page_stride])."""
    L = load()
    B, kp1, Hq, D = q.shape
    assert kp1 == k + 1
    Hkv = kv.num_kv_heads
    if out is None:
        out = torch.empty((B, k + 1, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, k + 1, Hq), dtype=torch.float32, device=q.device)
    if page_scores is None:
        stride = (int(max_seq_len) + 15) // 16 if page_stride is None else int(page_stride)
        page_scores = torch.empty((B, Hkv, stride), dtype=torch.float32, device=q.device)
    nb = verify_pages_workspace_bytes(B, k, Hq, Hkv, D, kv.dtype_code, int(max_seq_len))
    buf = _ws(ws, q.device).get("verify", nb)
    _check(L.s3r_verify_attn_pages(_ptr(q), ctypes.byref(kv.struct), _ptr(seq_len), B, int(k), Hq, float(scale),
                                   int(max_seq_len), _ptr(out), _ptr(lse), _ptr(page_scores), page_scores.shape[2],
                                   _ptr(buf), buf.numel(), _stream(stream)), "s3r_verify_attn_pages")
    return out, lse, page_scores


def verify_attn_deferred(q, kv: PagedKV, seq_len, k, scale, max_seq_len, out=None, lse=None, want_lse=True,
                         ws=None, stream=None):
    """s3r_verify_attn_deferred: output rows and lse now, score partials kept in the workspace for
    verify_scores. Returns (out, lse)."""
    L = load()
    B, kp1, Hq, D = q.shape
    assert kp1 == k + 1
    if out is None:
        out = torch.empty((B, k + 1, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, k + 1, Hq), dtype=torch.float32, device=q.device)
    nb = verify_workspace_bytes(B, k, Hq, kv.num_kv_heads, D, kv.dtype_code, int(max_seq_len))
    buf = _ws(ws, q.device).get("verify", nb)
    _check(L.s3r_verify_attn_deferred(_ptr(q), ctypes.byref(kv.struct), _ptr(seq_len), B, int(k), Hq,
                                      float(scale), int(max_seq_len), _ptr(out), _ptr(lse), _ptr(buf),
                                      buf.numel(), _stream(stream)), "s3r_verify_attn_deferred")
    return out, lse


def verify_scores(kv: PagedKV, seq_len, B, k, Hq, head_dim, max_seq_len, scores=None, score_stride=None, ws=None,
                  stream=None):
    """s3r_verify_scores: the scores of the preceding verify_attn_deferred on the same workspace."""
    L = load()
    Hkv = kv.num_kv_heads
    if scores is None:
        stride = int(max_seq_len) if score_stride is None else int(score_stride)
        scores = torch.empty((B, Hkv, stride), dtype=torch.float32, device=seq_len.device)
    nb = verify_workspace_bytes(B, k, Hq, Hkv, head_dim, kv.dtype_code, int(max_seq_len))
    buf = _ws(ws, seq_len.device).get("verify", nb)
    _check(L.s3r_verify_scores(ctypes.byref(kv.struct), _ptr(seq_len), int(B), int(k), int(Hq), int(max_seq_len),
                               _ptr(scores), scores.shape[2], _ptr(buf), buf.numel(), _stream(stream)),
           "s3r_verify_scores")
    return scores


def spec_sample_workspace_bytes(B, k, V) -> int:
    return int(load().s3r_spec_sample_workspace_bytes(B, k, V))


def spec_sample(target_logits, draft_logits, draft_tokens, uniforms, temperature, tokens=None, n_out=None,
                accepted=None, want_accepted=True, ws=None, stream=None):
    """s3r_spec_sample. target [B][k+1][V], draft [B][k][V] f32. Returns (tokens, n_out, accepted)."""
    L = load()
    B, kp1, V = target_logits.shape
    k = kp1 - 1
    dev = target_logits.device
    if tokens is None:
        tokens = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    if n_out is None:
        n_out = torch.empty((B,), dtype=torch.int32, device=dev)
    if accepted is None and want_accepted and k > 0:
        accepted = torch.empty((B, k), dtype=torch.int8, device=dev)
    nb = spec_sample_workspace_bytes(B, k, V)
    buf = _ws(ws, dev).get("sample", nb)
    _check(L.s3r_spec_sample(_ptr(target_logits), _ptr(draft_logits) if k > 0 else None,
                             _ptr(draft_tokens) if k > 0 else None, _ptr(uniforms), B, k, V,
                             float(temperature), _ptr(tokens), _ptr(n_out), _ptr(accepted), _ptr(buf),
                             buf.numel(), _stream(stream)), "s3r_spec_sample")
    return tokens, n_out, accepted


def spec_sample_noalloc(target_logits, draft_logits, draft_tokens, uniforms, temperature, tokens, n_out,
                        accepted=None, stream=None):
    """s3r_spec_sample_noalloc: as spec_sample with caller-given outputs and the library's own scratch
    (nothing is allocated, here or in the library)."""
    L = load()
    B, kp1, V = target_logits.shape
    k = kp1 - 1
    _check(L.s3r_spec_sample_noalloc(_ptr(target_logits), _ptr(draft_logits) if k > 0 else None,
                                     _ptr(draft_tokens) if k > 0 else None, _ptr(uniforms), B, k, V,
                                     float(temperature), _ptr(tokens), _ptr(n_out), _ptr(accepted),
                                     _stream(stream)), "s3r_spec_sample_noalloc")
    return tokens, n_out, accepted


def read_verify_pattern(kv: PagedKV, seq_len, max_seq_len, sink=None, stream=None):
    """s3r_read_verify_pattern (measurement): returns the checksum words."""
    L = load()
    B = seq_len.shape[0]
    n = int(L.s3r_read_pattern_sink_words(B, kv.num_kv_heads, int(max_seq_len), 0))
    if sink is None:
        sink = torch.empty((n,), dtype=torch.int32, device=seq_len.device)
    _check(L.s3r_read_verify_pattern(ctypes.byref(kv.struct), _ptr(seq_len), B, int(max_seq_len), _ptr(sink),
                                     sink.numel(), _stream(stream)), "s3r_read_verify_pattern")
    return sink


def read_draft_pattern(kv: PagedKV, idx, n_sel, sel_len, cur_len, max_attend, sink=None, stream=None):
    """s3r_read_draft_pattern (measurement): returns the checksum words."""
    L = load()
    B, _, cap = idx.shape
    n = int(L.s3r_read_pattern_sink_words(B, kv.num_kv_heads, int(max_attend), 1))
    if sink is None:
        sink = torch.empty((n,), dtype=torch.int32, device=idx.device)
    _check(L.s3r_read_draft_pattern(ctypes.byref(kv.struct), _ptr(idx), cap, _ptr(n_sel), _ptr(sel_len),
                                    _ptr(cur_len), B, int(max_attend), _ptr(sink), sink.numel(), _stream(stream)),
           "s3r_read_draft_pattern")
    return sink


def kv_append(k_rows, v_rows, kv: PagedKV, pos, max_pos, stream=None):
    """s3r_kv_append. k_rows, v_rows [B][n][Hkv][D] in the cache dtype; pos i32 [B] (device)."""
    L = load()
    B, n, hkv, d = k_rows.shape
    if v_rows.shape != k_rows.shape or k_rows.dtype != kv.k_pages.dtype or v_rows.dtype != kv.k_pages.dtype:
        raise ValueError("k_rows and v_rows must be [B][n][Hkv][D] in the cache dtype")
    if hkv != kv.num_kv_heads or d != kv.head_dim:
        raise ValueError("rows must have the cache's KV heads and head_dim")
    _check(L.s3r_kv_append(_ptr(k_rows), _ptr(v_rows), ctypes.byref(kv.struct), _ptr(pos), B, n, int(max_pos),
                           _stream(stream)), "s3r_kv_append")


def commit(n_out, tokens, ctx_len, pending=None, cur_len=None, seq_len=None, verified=None, stream=None):
    """s3r_commit: ctx_len += n_out in place; optional pending [B], cur_len [k][B], seq_len [B],
    verified int64 [1] (accumulated)."""
    L = load()
    B, kp1 = tokens.shape
    if cur_len is not None and tuple(cur_len.shape) != (kp1 - 1, B):
        raise ValueError("cur_len must be int32 [k][B]")
    if verified is not None and verified.dtype != torch.int64:
        raise ValueError("verified must be int64")
    _check(L.s3r_commit(_ptr(n_out), _ptr(tokens), B, kp1 - 1, _ptr(ctx_len), _ptr(pending), _ptr(cur_len),
                        _ptr(seq_len), _ptr(verified), _stream(stream)), "s3r_commit")
