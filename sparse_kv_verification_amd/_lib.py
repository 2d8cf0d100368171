"""ctypes binding of libdustin.so (include/dustin.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every computation runs in the library's gfx950 kernels.
There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DUSTIN_LIBRARY selects another build of the same library (the phase-trace
# build, libdustin_trace.so); by default the in-tree libdustin.so.
LIB_PATH = os.environ.get("DUSTIN_LIBRARY") or os.path.join(_HERE, "libdustin.so")

DUSTIN_F32 = 0
DUSTIN_BF16 = 1
STATUS = {0: "DUSTIN_OK", 1: "DUSTIN_ERR_INVALID_ARG", 2: "DUSTIN_ERR_UNSUPPORTED", 3: "DUSTIN_ERR_HIP"}

EXPORTS = [
    "dustin_score", "dustin_score_workspace_bytes", "dustin_draft_row_lse",
    "dustin_topk", "dustin_topk_workspace_bytes",
    "dustin_sparse_verify_attn", "dustin_attn_workspace_bytes", "dustin_sparse_verify_attn_noalloc",
    "dustin_verify_attn", "dustin_verify_attn_workspace_bytes", "dustin_verify_attn_append",
    "dustin_append_window_kv", "dustin_commit_window",
    "dustin_window_attn", "dustin_window_attn_workspace_bytes",
    "dustin_arr", "dustin_window_mean", "dustin_policy_sweep", "dustin_policy_sweep_workspace_bytes",
    "dustin_page_bounds", "dustin_page_scores", "dustin_page_scores_workspace_bytes",
    "dustin_head_scores", "dustin_head_scores_workspace_bytes", "dustin_candidate_arr",
    "dustin_candidate_arr_workspace_bytes", "dustin_greedy_select", "dustin_greedy_select_workspace_bytes",
    "dustin_probe_stream_read", "dustin_probe_gather_rows",
    "dustin_status_string", "dustin_last_error", "dustin_abi_version",
]


class DustinKV(ctypes.Structure):
    """Mirror of struct dustin_kv."""
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("H_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("N_max", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("page_table", ctypes.c_void_p),
        ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int32),
    ]


class DustinError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def lib():
    """Load libdustin.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(or python -m sparse_kv_verification_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        kvp = ctypes.POINTER(DustinKV)
        L.dustin_score.argtypes = [kvp, i32, vp, i32, i32, kvp, i32, vp, vp, i32, i32, f32, f32, vp, vp, vp, vp, sz,
                                   vp]
        L.dustin_draft_row_lse.argtypes = [kvp, i32, vp, i32, i32, f32, vp, vp, sz, vp]
        L.dustin_draft_row_lse.restype = ctypes.c_int
        L.dustin_score.restype = ctypes.c_int
        L.dustin_score_workspace_bytes.argtypes = [i32] * 6
        L.dustin_score_workspace_bytes.restype = sz
        L.dustin_topk.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.dustin_topk.restype = ctypes.c_int
        L.dustin_topk_workspace_bytes.argtypes = [i32, i32, i32]
        L.dustin_topk_workspace_bytes.restype = sz
        L.dustin_sparse_verify_attn.argtypes = [vp, i32, i32, kvp, vp, vp, i32, f32, vp, vp, vp, sz, vp]
        L.dustin_sparse_verify_attn.restype = ctypes.c_int
        L.dustin_sparse_verify_attn_noalloc.argtypes = [vp, i32, i32, kvp, vp, vp, i32, f32, vp, vp, vp]
        L.dustin_sparse_verify_attn_noalloc.restype = ctypes.c_int
        L.dustin_attn_workspace_bytes.argtypes = [i32] * 6
        L.dustin_attn_workspace_bytes.restype = sz
        L.dustin_verify_attn.argtypes = [vp, i32, i32, kvp, vp, vp, i32, f32, vp, vp, vp, sz, vp]
        L.dustin_verify_attn.restype = ctypes.c_int
        L.dustin_verify_attn_append.argtypes = [vp, i32, i32, kvp, vp, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp]
        L.dustin_verify_attn_append.restype = ctypes.c_int
        L.dustin_verify_attn_workspace_bytes.argtypes = [i32] * 6
        L.dustin_verify_attn_workspace_bytes.restype = sz
        L.dustin_append_window_kv.argtypes = [kvp, vp, vp, i32, vp]
        L.dustin_append_window_kv.restype = ctypes.c_int
        L.dustin_commit_window.argtypes = [vp, vp, i32, i32, vp]
        L.dustin_commit_window.restype = ctypes.c_int
        L.dustin_window_attn.argtypes = [vp, i32, i32, kvp, f32, vp, vp, sz, vp]
        L.dustin_window_attn.restype = ctypes.c_int
        L.dustin_window_attn_workspace_bytes.argtypes = [i32] * 6
        L.dustin_window_attn_workspace_bytes.restype = sz
        L.dustin_arr.argtypes = [vp, vp, i32, i32, i32, vp, vp, i32, vp, vp, vp]
        L.dustin_arr.restype = ctypes.c_int
        L.dustin_window_mean.argtypes = [vp, i32, i32, i32, vp, vp]
        L.dustin_window_mean.restype = ctypes.c_int
        L.dustin_policy_sweep.argtypes = [vp, i32, vp, i32, i32, kvp, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, sz,
                                          vp]
        L.dustin_policy_sweep.restype = ctypes.c_int
        L.dustin_policy_sweep_workspace_bytes.argtypes = [i32] * 8
        L.dustin_policy_sweep_workspace_bytes.restype = sz
        L.dustin_page_bounds.argtypes = [kvp, vp, vp, vp]
        L.dustin_page_bounds.restype = ctypes.c_int
        L.dustin_page_scores.argtypes = [vp, i32, i32, kvp, vp, vp, f32, vp, vp, sz, vp]
        L.dustin_page_scores_workspace_bytes.argtypes = [i32, i32, i32]
        L.dustin_page_scores_workspace_bytes.restype = sz
        i32p = ctypes.POINTER(ctypes.c_int32)
        f32p = ctypes.POINTER(ctypes.c_float)
        L.dustin_head_scores.argtypes = [vp, i32, vp, vp, i32, i32, f32, vp, vp, sz, vp]
        L.dustin_head_scores.restype = ctypes.c_int
        L.dustin_head_scores_workspace_bytes.argtypes = [i32, i32, i32]
        L.dustin_head_scores_workspace_bytes.restype = sz
        L.dustin_candidate_arr.argtypes = [vp, vp, vp, vp, i32, vp, i32, vp, vp, i32, i32, vp, i32, i32, i32, i32,
                                           vp, vp, vp, sz, vp]
        L.dustin_candidate_arr.restype = ctypes.c_int
        L.dustin_candidate_arr_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.dustin_candidate_arr_workspace_bytes.restype = sz
        L.dustin_greedy_select.argtypes = [vp, i32, vp, i32, i32, vp, vp, i32, i32, vp, i32, i32, i32, i32, i32,
                                           i32p, f32p, i32p, vp, vp, sz, vp]
        L.dustin_greedy_select.restype = ctypes.c_int
        L.dustin_greedy_select_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.dustin_greedy_select_workspace_bytes.restype = sz
        L.dustin_page_scores.restype = ctypes.c_int
        i64 = ctypes.c_int64
        L.dustin_probe_stream_read.argtypes = [vp, sz, i32, vp, vp]
        L.dustin_probe_stream_read.restype = ctypes.c_int
        L.dustin_probe_gather_rows.argtypes = [vp, vp, i64, i64, vp, i64, i32, vp]
        L.dustin_probe_gather_rows.restype = ctypes.c_int
        L.dustin_status_string.argtypes = [ctypes.c_int]
        L.dustin_status_string.restype = ctypes.c_char_p
        L.dustin_last_error.argtypes = []
        L.dustin_last_error.restype = ctypes.c_char_p
        L.dustin_abi_version.argtypes = []
        L.dustin_abi_version.restype = i32
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise DustinError(status, lib().dustin_last_error().decode())


def _ptr(t):
    """Device address of a GPU tensor (None for None).  A tensor in host
    memory is refused here: a kernel dereferencing a host address faults."""
    if t is None:
        return None
    if not t.is_cuda:
        raise TypeError(f"expected a GPU tensor, got one on {t.device}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t=None):
    if t is not None and t.is_cuda:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return ctypes.c_void_p(0)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return DUSTIN_F32
    if t.dtype == torch.bfloat16:
        return DUSTIN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


class KV:
    """One layer's cache descriptor; keeps the tensors it points to alive.

    Contiguous: k, v are [B][N_max][H_kv][head_dim].
    Paged: k, v are [num_pages][16][H_kv][head_dim] with page_table
    [B][max_pages] (int32); N_max defaults to max_pages * 16.
    """

    def __init__(self, k, v=None, seq_lens=None, page_table=None, N_max=None, B=None):
        self.k, self.v, self.seq_lens, self.page_table = k, v, seq_lens, page_table
        if seq_lens is None or seq_lens.dtype != torch.int32:
            raise TypeError("seq_lens must be an int32 tensor")
        for name, t in (("k", k), ("v", v), ("seq_lens", seq_lens), ("page_table", page_table)):
            if t is not None and not t.is_cuda:
                raise TypeError(f"KV: {name} must be a GPU tensor, got one on {t.device}")
        if page_table is None:
            Bk, N, H, D = k.shape
            ps, maxp, npages = 0, 0, 0
        else:
            npages, ps, H, D = k.shape
            Bk, maxp = page_table.shape
            N = N_max if N_max is not None else maxp * ps
        self.desc = DustinKV(
            k=k.data_ptr(), v=v.data_ptr() if v is not None else None, dtype=_dtype_code(k),
            B=B if B is not None else Bk, H_kv=H, head_dim=D, N_max=N,
            seq_lens=seq_lens.data_ptr(), page_size=ps,
            page_table=page_table.data_ptr() if page_table is not None else None,
            max_pages=maxp, num_pages=npages)

    @property
    def ref(self):
        return ctypes.byref(self.desc)


def _kv_array(kvs):
    arr = (DustinKV * len(kvs))(*[x.desc for x in kvs])
    return arr


class Workspace:
    """Zero-initialised device scratch, grown on demand.  One per entry point:
    the attention calls rely on the arrival counters at its start being zero
    (they leave them zero), so it must not be shared with other calls."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes, device):
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        return self.buf


_default_ws = {}


def _ws(name, ws, nbytes, device):
    if ws is None:
        ws = _default_ws.setdefault((name, str(device)), Workspace())
    return ws.get(nbytes, device)


# --------------------------------------------------------------------------

def dustin_sparse_verify_attn(q, kv: KV, idx=None, count=None, k=None, scale=0.0,
                              out=None, lse=None, ws: Workspace | None = None):
    """Sparse verification attention over the rows idx[b][:count[b]] (or dense
    over j < n_b when idx is None).  q: [B][w][H_q][d]."""
    B, w, Hq, D = q.shape
    kk = 0 if idx is None else (k if k is not None else idx.shape[1])
    if out is None:
        out = torch.empty_like(q)
    d = kv.desc
    nbytes = lib().dustin_attn_workspace_bytes(d.B, w, Hq, d.H_kv, d.head_dim, kk if idx is not None else d.N_max)
    wsb = _ws("attn", ws, nbytes, q.device)
    _check(lib().dustin_sparse_verify_attn(_ptr(q), w, Hq, kv.ref, _ptr(idx), _ptr(count), kk, float(scale),
                                           _ptr(out), _ptr(lse), _ptr(wsb), wsb.numel(), _stream(q)))
    return out


def dustin_sparse_verify_attn_noalloc(q, kv: KV, idx=None, count=None, k=None, scale=0.0, out=None, lse=None):
    """dustin_sparse_verify_attn without a workspace: the library's static
    per-GPU scratch holds the split state, and the call allocates nothing
    (pass `out` to keep the binding from allocating it either).  Calls that
    overlap on one GPU race."""
    B, w, Hq, D = q.shape
    kk = 0 if idx is None else (k if k is not None else idx.shape[1])
    if out is None:
        out = torch.empty_like(q)
    _check(lib().dustin_sparse_verify_attn_noalloc(_ptr(q), w, Hq, kv.ref, _ptr(idx), _ptr(count), kk, float(scale),
                                                   _ptr(out), _ptr(lse), _stream(q)))
    return out


def dustin_verify_attn(q, kv: KV, idx=None, count=None, k=None, scale=0.0,
                       out=None, lse=None, ws: Workspace | None = None):
    """Attention of one verification step: window query s attends the
    selected history rows idx[b][:count[b]] (all j < n_b when idx is None)
    and the window's own cache rows n_b .. n_b + s.  q: [B][w][H_q][d]."""
    B, w, Hq, D = q.shape
    kk = 0 if idx is None else (k if k is not None else idx.shape[1])
    if out is None:
        out = torch.empty_like(q)
    d = kv.desc
    nbytes = lib().dustin_verify_attn_workspace_bytes(d.B, w, Hq, d.H_kv, d.head_dim,
                                                      kk if idx is not None else d.N_max)
    wsb = _ws("verify", ws, nbytes, q.device)
    _check(lib().dustin_verify_attn(_ptr(q), w, Hq, kv.ref, _ptr(idx), _ptr(count), kk, float(scale),
                                    _ptr(out), _ptr(lse), _ptr(wsb), wsb.numel(), _stream(q)))
    return out


def dustin_verify_attn_append(q, kv: KV, k_win, v_win, idx=None, count=None, k=None, scale=0.0,
                              out=None, lse=None, ws: Workspace | None = None):
    """dustin_append_window_kv(kv, k_win, v_win) then dustin_verify_attn(q,
    kv, ...) in one call (one launch for a bfloat16 cache): the window's
    keys / values ([B][w][H_kv][d] each) go into cache rows n_b .. n_b + w - 1
    and window query s attends the selected history rows and rows
    n_b .. n_b + s."""
    B, w, Hq, D = q.shape
    kk = 0 if idx is None else (k if k is not None else idx.shape[1])
    if out is None:
        out = torch.empty_like(q)
    d = kv.desc
    nbytes = lib().dustin_verify_attn_workspace_bytes(d.B, w, Hq, d.H_kv, d.head_dim,
                                                      kk if idx is not None else d.N_max)
    wsb = _ws("verify", ws, nbytes, q.device)
    _check(lib().dustin_verify_attn_append(_ptr(q), w, Hq, kv.ref, _ptr(k_win), _ptr(v_win), _ptr(idx),
                                           _ptr(count), kk, float(scale), _ptr(out), _ptr(lse), _ptr(wsb),
                                           wsb.numel(), _stream(q)))
    return out


def dustin_append_window_kv(kv: KV, k_win, v_win):
    """Write the window's keys/values ([B][w][H_kv][d] each) into cache rows
    n_b .. n_b + w - 1; the sequence lengths are not changed."""
    w = k_win.shape[1]
    _check(lib().dustin_append_window_kv(kv.ref, _ptr(k_win), _ptr(v_win), w, _stream(k_win)))


def dustin_commit_window(seq_lens, accepted, w):
    """seq_lens[b] += clamp(accepted[b], 0, w), in place."""
    B = seq_lens.shape[0]
    _check(lib().dustin_commit_window(_ptr(seq_lens), _ptr(accepted), B, int(w), _stream(seq_lens)))
    return seq_lens


def dustin_score(draft_kvs, q_draft, target_kvs, q_hist, sub_heads, H_t, s_draft=None, s_target=None,
                 scale_draft=0.0, scale_target=0.0, ws: Workspace | None = None, want_draft=True,
                 want_target=True, draft_lse=None):
    """Hybrid importance vectors S_Draft, S_Target ([B][N_max] float32 each).
    q_draft: [B][L_d][gamma][H_d][d_d]; q_hist: [B][S][d]; sub_heads: S
    (layer, head) pairs into target_kvs.  draft_lse (optional, float32
    [B][L_d][gamma][H_d] on the device): the draft softmaxes' row normalisers
    (natural log), used as given: S_Draft then reads the draft keys once."""
    ref = (draft_kvs or target_kvs)[0]
    B, N = ref.desc.B, ref.desc.N_max
    dev = (q_draft if q_draft is not None else q_hist).device
    L_d = len(draft_kvs) if (draft_kvs and want_draft) else 0
    H_d = gamma = 0
    if L_d:
        _, L_chk, gamma, H_d, _ = q_draft.shape
        assert L_chk == L_d, "q_draft layer count differs from draft_kvs"
        if s_draft is None:
            s_draft = torch.empty((B, N), dtype=torch.float32, device=dev)
    S = len(sub_heads) if (sub_heads and want_target) else 0
    if S and s_target is None:
        s_target = torch.empty((B, N), dtype=torch.float32, device=dev)
    heads = (ctypes.c_int32 * (2 * max(S, 1)))(*[x for p in (sub_heads or [])[:S] for x in p])
    if L_d and draft_lse is not None:
        if not (draft_lse.is_cuda and draft_lse.dtype == torch.float32 and draft_lse.is_contiguous()
                and tuple(draft_lse.shape) == (B, L_d, gamma, H_d)):
            raise TypeError(f"draft_lse must be a contiguous float32 GPU tensor of shape {(B, L_d, gamma, H_d)}")
    darr = _kv_array(draft_kvs) if L_d else None
    tarr = _kv_array(target_kvs) if S else None
    nbytes = lib().dustin_score_workspace_bytes(B, N, L_d, H_d, gamma, S)
    wsb = _ws("score", ws, nbytes, dev)
    _check(lib().dustin_score(darr, L_d, _ptr(q_draft) if L_d else None, H_d, gamma,
                              tarr, len(target_kvs) if S else 0, _ptr(q_hist) if S else None,
                              heads if S else None, S, int(H_t), float(scale_draft), float(scale_target),
                              _ptr(draft_lse) if (L_d and draft_lse is not None) else None,
                              _ptr(s_draft) if L_d else None, _ptr(s_target) if S else None,
                              _ptr(wsb), wsb.numel(), _stream(wsb)))
    return s_draft, s_target


def dustin_draft_row_lse(draft_kvs, q_draft, scale_draft=0.0, out=None, ws: Workspace | None = None):
    """Row normalisers of S_Draft's softmaxes: float32 [B][L_d][gamma][H_d],
    ln sum_{j < n_b} exp(scale * q . k_j) (-inf for an empty history)."""
    B, N = draft_kvs[0].desc.B, draft_kvs[0].desc.N_max
    _, L_d, gamma, H_d, _ = q_draft.shape
    assert L_d == len(draft_kvs), "q_draft layer count differs from draft_kvs"
    if out is None:
        out = torch.empty((B, L_d, gamma, H_d), dtype=torch.float32, device=q_draft.device)
    nbytes = lib().dustin_score_workspace_bytes(B, N, L_d, H_d, gamma, 0)
    wsb = _ws("score", ws, nbytes, q_draft.device)
    _check(lib().dustin_draft_row_lse(_kv_array(draft_kvs), L_d, _ptr(q_draft), H_d, gamma, float(scale_draft),
                                      _ptr(out), _ptr(wsb), wsb.numel(), _stream(wsb)))
    return out


def dustin_topk(s_draft, s_target, seq_lens, k, m, n_sink, n_window, idx=None, count=None, tier=None,
                want_tier=True, ws: Workspace | None = None):
    """Per-sequence verification set; returns (idx [B][k] int32 ascending,
    count [B] int32, tier [B][k] int8 or None)."""
    ref = s_target if s_target is not None else s_draft
    B, N = ref.shape
    dev = ref.device
    if idx is None:
        idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((B,), dtype=torch.int32, device=dev)
    if tier is None and want_tier:
        tier = torch.empty((B, k), dtype=torch.int8, device=dev)
    nbytes = lib().dustin_topk_workspace_bytes(B, N, k)
    wsb = _ws("topk", ws, nbytes, dev)
    _check(lib().dustin_topk(_ptr(s_draft), _ptr(s_target), _ptr(seq_lens), B, N, k, m, n_sink, n_window,
                             _ptr(idx), _ptr(count), _ptr(tier), _ptr(wsb), wsb.numel(), _stream(ref)))
    return idx, count, tier


def dustin_window_attn(q, kv: KV, scale=0.0, A=None, ws: Workspace | None = None):
    """Head-mean full-cache attention weights A [B][w][N_max] (float32)."""
    B, w, Hq, D = q.shape
    d = kv.desc
    if A is None:
        A = torch.empty((B, w, d.N_max), dtype=torch.float32, device=q.device)
    nbytes = lib().dustin_window_attn_workspace_bytes(d.B, w, Hq, d.H_kv, d.head_dim, d.N_max)
    wsb = _ws("window", ws, nbytes, q.device)
    _check(lib().dustin_window_attn(_ptr(q), w, Hq, kv.ref, float(scale), _ptr(A), _ptr(wsb), wsb.numel(),
                                    _stream(q)))
    return A


def dustin_arr(A, seq_lens, idx, count, arr_step=None, arr_window=None):
    """ARR per window step (Eq. 1) and windowed ARR (Eq. 2)."""
    B, w, N = A.shape
    k = idx.shape[1]
    if arr_step is None:
        arr_step = torch.empty((B, w), dtype=torch.float32, device=A.device)
    if arr_window is None:
        arr_window = torch.empty((B,), dtype=torch.float32, device=A.device)
    _check(lib().dustin_arr(_ptr(A), _ptr(seq_lens), B, w, N, _ptr(idx), _ptr(count), k, _ptr(arr_step),
                            _ptr(arr_window), _stream(A)))
    return arr_step, arr_window


def dustin_window_mean(A, Abar=None):
    """Eq. (3)'s averaged future attention Abar [B][N_max] of A [B][w][N_max]."""
    B, w, N = A.shape
    if Abar is None:
        Abar = torch.empty((B, N), dtype=torch.float32, device=A.device)
    _check(lib().dustin_window_mean(_ptr(A), B, w, N, _ptr(Abar), _stream(A)))
    return Abar


POLICY_NAMES = ("oracle", "history", "draft", "dustin_T", "dustin_D", "dustin_H")


def dustin_policy_sweep(q_window, q_past, kv: KV, s_draft, s_target, ks, m_hybrid, n_sink, n_window, scale=0.0,
                        arr=None, ws: Workspace | None = None):
    """Windowed ARR of the compared selection policies at each budget:
    arr [n_past + 5][len(ks)][B]; rows: SD oracle, one history row per past
    query, draft lookahead, Dustin-T, Dustin-D, Dustin-H.
    q_window [B][w][H_q][d]; q_past [n_past][B][H_q][d] or None."""
    B, w, Hq, D = q_window.shape
    n_past = 0 if q_past is None else q_past.shape[0]
    nk = len(ks)
    d = kv.desc
    for t in (s_draft, s_target):
        if tuple(t.shape) != (d.B, d.N_max) or not t.is_contiguous():
            raise ValueError(f"score vectors must be contiguous [B][N_max] = [{d.B}][{d.N_max}], got {tuple(t.shape)}")
    if q_past is not None and tuple(q_past.shape[1:]) != (B, Hq, D):
        raise ValueError(f"q_past must be [n_past][B][H_q][d], got {tuple(q_past.shape)}")
    if arr is None:
        arr = torch.empty((n_past + 5, nk, B), dtype=torch.float32, device=q_window.device)
    kbuf = (ctypes.c_int32 * nk)(*[int(k) for k in ks])
    mbuf = (ctypes.c_int32 * nk)(*[int(m) for m in m_hybrid])
    nbytes = lib().dustin_policy_sweep_workspace_bytes(d.B, w, n_past, Hq, d.H_kv, d.head_dim, d.N_max, max(ks))
    wsb = _ws("sweep", ws, nbytes, q_window.device)
    _check(lib().dustin_policy_sweep(_ptr(q_window), w, _ptr(q_past), n_past, Hq, kv.ref, _ptr(s_draft),
                                     _ptr(s_target), kbuf, mbuf, nk, n_sink, n_window, float(scale), _ptr(arr),
                                     _ptr(wsb), wsb.numel(), _stream(q_window)))
    return arr


def dustin_page_bounds(kv: KV, kmin=None, kmax=None):
    """Page min/max key bounds [B][ceil(N_max/16)][H_kv][d] (kv dtype)."""
    d = kv.desc
    shape = (d.B, (d.N_max + 15) // 16, d.H_kv, d.head_dim)
    if kmin is None:
        kmin = torch.empty(shape, dtype=kv.k.dtype, device=kv.k.device)
    if kmax is None:
        kmax = torch.empty(shape, dtype=kv.k.dtype, device=kv.k.device)
    _check(lib().dustin_page_bounds(kv.ref, _ptr(kmin), _ptr(kmax), _stream(kv.k)))
    return kmin, kmax


def dustin_page_scores(q, kv: KV, kmin, kmax, scale=0.0, scores=None, ws: Workspace | None = None):
    """Page scores [B][ceil(N_max/16)] float32 from the bounds."""
    B, w, Hq, D = q.shape
    d = kv.desc
    if scores is None:
        scores = torch.empty((d.B, (d.N_max + 15) // 16), dtype=torch.float32, device=q.device)
    wsb = _ws("pages", ws, lib().dustin_page_scores_workspace_bytes(d.B, d.H_kv, d.head_dim), q.device)
    _check(lib().dustin_page_scores(_ptr(q), w, Hq, kv.ref, _ptr(kmin), _ptr(kmax), float(scale), _ptr(scores),
                                    _ptr(wsb), wsb.numel(), _stream(q)))
    return scores


def _host_i32(vals):
    if vals is None:
        return None
    vals = [int(v) for v in vals]
    return (ctypes.c_int32 * max(len(vals), 1))(*vals)


def dustin_head_scores(target_kvs, q_hist, sub_heads, H_t, scale=0.0, out=None, ws: Workspace | None = None):
    """Per-(layer, head) S_Target rows [S][B][N_max] float32 (not summed).
    q_hist: [B][S][d]; sub_heads: S (layer, head) pairs into target_kvs."""
    d = target_kvs[0].desc
    S = len(sub_heads)
    if out is None:
        out = torch.empty((S, d.B, d.N_max), dtype=torch.float32, device=q_hist.device)
    heads = (ctypes.c_int32 * (2 * S))(*[x for p in sub_heads for x in p])
    wsb = _ws("heads", ws, lib().dustin_head_scores_workspace_bytes(d.B, d.N_max, S), q_hist.device)
    _check(lib().dustin_head_scores(_kv_array(target_kvs), len(target_kvs), _ptr(q_hist), heads, S, int(H_t),
                                    float(scale), _ptr(out), _ptr(wsb), wsb.numel(), _stream(q_hist)))
    return out


def dustin_candidate_arr(seq_lens, abar, k, m, n_sink, n_window, s_draft=None, draft_units=None, s_target=None,
                         target_units=None, unit_ids=None, C=None, m_cand=None, arr=None, arr_mean=None,
                         want_mean=True, ws: Workspace | None = None):
    """Objective of C candidate configurations: arr [C][B] (and the batch
    means [C]); units [U][B][N_max] on one side, base vectors [B][N_max]."""
    B, N = abar.shape
    units = draft_units if draft_units is not None else target_units
    U = 0 if units is None else units.shape[0]
    if C is None:
        C = len(unit_ids) if unit_ids is not None else (len(m_cand) if m_cand is not None else U or 1)
    dev = abar.device
    if arr is None:
        arr = torch.empty((C, B), dtype=torch.float32, device=dev)
    if arr_mean is None and want_mean:
        arr_mean = torch.empty((C,), dtype=torch.float32, device=dev)
    base = s_draft if draft_units is not None else s_target
    mat = units is not None and (unit_ids is not None or base is not None)
    wsb = _ws("cand", ws, lib().dustin_candidate_arr_workspace_bytes(C, B, N, k, int(mat)), dev)
    _check(lib().dustin_candidate_arr(_ptr(s_draft), _ptr(draft_units), _ptr(s_target), _ptr(target_units), U,
                                      _host_i32(unit_ids), C, _host_i32(m_cand), _ptr(seq_lens), B, N, _ptr(abar),
                                      k, m, n_sink, n_window, _ptr(arr), _ptr(arr_mean), _ptr(wsb), wsb.numel(),
                                      _stream(abar)))
    return arr, arr_mean


def dustin_greedy_select(units, seq_lens, abar, k, m, n_sink, n_window, max_units, side, s_target_fixed=None,
                         unit_ids=None, sum_out=None, ws: Workspace | None = None):
    """Greedy forward selection over candidate units of one side (0 target,
    1 draft).  Returns (chosen candidate indices, objective curve, sum of the
    chosen units [B][N_max])."""
    U, B, N = units.shape
    C = len(unit_ids) if unit_ids is not None else U
    if sum_out is None:
        sum_out = torch.empty((B, N), dtype=torch.float32, device=units.device)
    chosen = (ctypes.c_int32 * max(max_units, 1))()
    curve = (ctypes.c_float * max(max_units, 1))()
    n_ch = ctypes.c_int32(0)
    wsb = _ws("greedy", ws, lib().dustin_greedy_select_workspace_bytes(C, B, N, k), units.device)
    _check(lib().dustin_greedy_select(_ptr(units), U, _host_i32(unit_ids), C, int(side), _ptr(s_target_fixed),
                                      _ptr(seq_lens), B, N, _ptr(abar), k, m, n_sink, n_window, max_units, chosen,
                                      curve, ctypes.byref(n_ch), _ptr(sum_out), _ptr(wsb), wsb.numel(),
                                      _stream(units)))
    n = n_ch.value
    return [chosen[i] for i in range(n)], [curve[i] for i in range(n)], sum_out


def dustin_probe_stream_read(buf, nontemporal=True, sink=None):
    """Measurement kernel: read every byte of `buf` once (returns sink)."""
    if sink is None:
        sink = torch.zeros(2048, dtype=torch.int32, device=buf.device)
    _check(lib().dustin_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), int(bool(nontemporal)),
                                          _ptr(sink), _stream(buf)))
    return sink


def dustin_probe_gather_rows(base, rows, row_bytes, row_stride, base2=None):
    """Measurement kernel: gather rows[i] (row numbers) of `row_bytes` bytes
    at `row_stride` from base (and base2) into LDS, as the attention does."""
    buf_rows = (base.numel() * base.element_size() - row_bytes) // row_stride + 1
    _check(lib().dustin_probe_gather_rows(_ptr(base), _ptr(base2), int(row_stride), int(buf_rows), _ptr(rows),
                                          rows.numel(), int(row_bytes), _stream(base)))
