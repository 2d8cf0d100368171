"""Seeded synthetic inputs for the sparse-verification step.

This module only draws random tensors with the shapes and structure of the
workloads the Dustin pages measure on (Qwen2.5-7B/32B/72B-shaped target
layers, a 0.5B-shaped draft, 16K-128K contexts, batch 4-16).  It holds none
of the method's arithmetic: no attention, no softmax, no scoring, no
selection.  Both the HIP library's tests/bench and the CPU oracle consume
what it produces, so the two sides see identical values.

Recipe (per config, master seed = config number unless given):
  keys      k_j = z_j + (3 * [j heavy] + lambda_j) * u_g    z ~ N(0, I_d)
            heavy set: ceil(rho * n_b) positions per sequence, no replacement
            lambda_j ~ LogNormal(0, sigma) per position (sigma = 0 disables)
            u_g: random unit direction per target KV head
  values    V ~ N(0, 1)
  queries   q_i^h = zeta_h + sqrt(d) * u_{g(h)};  window step s >= 1 adds
            N(0, 0.2^2); the most recent history query q_{i-1} likewise.
  draft     layer l, draft KV head c follows target KV head
            t = (l * Hkv_d + c) mod Hkv through a projection P_{l,c}
            (entries N(0, 1/d)):  k^d = P k^t + N(0, 0.3^2);
            draft query head h follows target head t*G + ((l + h) mod G):
            q^d_{l,h,g} = P q^{h_t}_{i+g} + N(0, 0.3^2).
  drift     (ragged config) 13 orthonormal directions u_{g,t} per KV head;
            0.1% of positions per group t get +3 u_{g,t}; the query of step
            s in [-1, w) carries sqrt(d) * sum_{t=s+1}^{s+5} u_{g,t}, so one
            fifth of the active heavy set changes per window step.
  ragged    n_b ~ UniformInt[lo, hi]; KV in 16-token pages with a seeded
            permutation of physical page ids; unused slots are NaN.
Storage dtype: float32 for the tiny config, bfloat16 (round-to-nearest-even
from float32) otherwise.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Shape", "PRESETS", "preset", "make", "tier_defaults", "spread_heads", "history_trajectory",
           "SearchInputs", "make_search"]


@dataclass(frozen=True)
class Shape:
    name: str
    B: int
    n: int                      # context length (max length when ragged)
    Hq: int
    Hkv: int
    d: int
    w: int
    k: int
    S: int                      # number of scored target heads
    L_d: int
    H_d: int
    Hkv_d: int
    d_d: int
    dtype: str = "bf16"         # "f32" | "bf16"
    heavy_frac: float = 0.01
    sigma: float = 0.0          # log-normal salience (0 = off)
    n_lo: int = 0               # ragged lower bound (0 = not ragged)
    page_size: int = 0          # 0 = contiguous, 16 = paged
    drift: bool = False
    layers: int = 1             # target layers in the timed step
    k_sweep: tuple = ()
    seed: int = 0               # master seed

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def gamma(self):
        return self.w

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


PRESETS = {
    "c1": Shape("c1-tiny-f32", B=1, n=1024, Hq=4, Hkv=1, d=64, w=4, k=128, S=4,
                L_d=1, H_d=2, Hkv_d=1, d_d=32, dtype="f32", heavy_frac=0.02, seed=1),
    "c2": Shape("c2-qwen7b-16k", B=4, n=16384, Hq=28, Hkv=4, d=128, w=4, k=512, S=4,
                L_d=24, H_d=14, Hkv_d=2, d_d=64, heavy_frac=0.01, sigma=0.5, seed=2),
    "c3": Shape("c3-qwen32b-32k", B=16, n=32768, Hq=40, Hkv=8, d=128, w=4, k=1024, S=8,
                L_d=24, H_d=14, Hkv_d=2, d_d=64, heavy_frac=0.01, sigma=0.5, seed=3),
    "c4": Shape("c4-qwen72b-32k", B=16, n=32768, Hq=64, Hkv=8, d=128, w=4, k=2048, S=8,
                L_d=24, H_d=14, Hkv_d=2, d_d=64, heavy_frac=0.01, sigma=0.5,
                layers=80, k_sweep=(512, 1024, 2048), seed=4),
    "c5": Shape("c5-ragged-paged", B=8, n=131072, Hq=64, Hkv=8, d=128, w=8, k=4096, S=8,
                L_d=24, H_d=14, Hkv_d=2, d_d=64, heavy_frac=0.005, n_lo=8192,
                page_size=16, drift=True, seed=5),
}


def preset(name, **overrides):
    return PRESETS[name].replace(**overrides)


def tier_defaults(k):
    """Sink, window and draft-share defaults (the pages leave them open)."""
    n_sink, n_window = 4, 32
    if n_sink + n_window > k:
        n_sink, n_window = min(4, k), 0
    m = max(0, (k - n_sink - n_window) // 2)
    return n_sink, n_window, m


def spread_heads(shape):
    """Scored target heads, all in layer 0: one per KV group when S <= Hkv
    (heads g*G), otherwise the first S heads."""
    if shape.S <= shape.Hkv:
        return [(0, g * shape.G) for g in range(shape.S)]
    return [(0, h) for h in range(shape.S)]


_STREAMS = ["K", "V", "heavy", "dirs", "salience", "q", "drift_q", "proj",
            "draft_k_noise", "draft_q_noise", "lens", "pages", "trajectory",
            "search_heavy", "search_layer", "search_rho", "search_draft"]


def _gen(master, stream, device):
    st = np.random.SeedSequence([int(master), _STREAMS.index(stream)]).generate_state(2)
    seed = (int(st[0]) << 31 ^ int(st[1])) & ((1 << 62) - 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _orthonormal(n_vec, d, gen, device):
    a = _randn((d, n_vec), gen, device).double()
    qm, _ = torch.linalg.qr(a.cpu())
    return qm.T.contiguous().float().to(device)   # [n_vec][d]


@dataclass
class Inputs:
    shape: Shape
    seq_lens: torch.Tensor          # [B] int32
    q: torch.Tensor                 # [B][w][Hq][d]
    q_hist: torch.Tensor            # [B][S][d]
    sub_heads: list
    q_draft: torch.Tensor           # [B][L_d][Gamma][H_d][d_d]
    K: torch.Tensor                 # [B][N][Hkv][d] or pool [P][ps][Hkv][d]
    V: torch.Tensor
    Kd: torch.Tensor                # [L_d][B][N][Hkv_d][d_d] or [L_d][P][ps][Hkv_d][d_d]
    page_table: torch.Tensor | None = None   # [B][max_pages] int32, -1 unused
    extra: dict = field(default_factory=dict)

    @property
    def N(self):
        return self.shape.n

    def logical(self, name, b):
        """Logical rows [0, n_b) of sequence b of K / V (contiguous view),
        or of every draft layer for Kd -> [L_d][n_b][Hkv_d][d_d]."""
        n = int(self.seq_lens[b])
        t = getattr(self, name)
        if self.page_table is None:
            if name == "Kd":
                return t[:, b, :n]
            return t[b, :n]
        ps = self.shape.page_size
        npg = (n + ps - 1) // ps
        pages = self.page_table[b, :npg].long()
        if name == "Kd":
            return t[:, pages].reshape(t.shape[0], npg * ps, *t.shape[3:])[:, :n]
        return t[pages].reshape(npg * ps, *t.shape[2:])[:n]


def make(shape: Shape, seed=None, device="cpu"):
    """Draw one batch of inputs for ``shape`` on ``device``."""
    dev = torch.device(device)
    master = shape.seed if seed is None else seed
    B, N, Hq, Hkv, d, w = shape.B, shape.n, shape.Hq, shape.Hkv, shape.d, shape.w
    G = shape.G
    store = torch.float32 if shape.dtype == "f32" else torch.bfloat16

    # ---- sequence lengths
    if shape.n_lo:
        gl = _gen(master, "lens", "cpu")
        lens = torch.randint(shape.n_lo, N + 1, (B,), generator=gl, dtype=torch.int64)
    else:
        lens = torch.full((B,), N, dtype=torch.int64)

    # ---- key directions
    gdir = _gen(master, "dirs", dev)
    if shape.drift:
        n_groups = w + 5
        U = torch.stack([_orthonormal(n_groups, d, gdir, dev) for _ in range(Hkv)])  # [Hkv][T][d]
    else:
        U = _randn((Hkv, d), gdir, dev)
        U = U / U.norm(dim=-1, keepdim=True)

    # ---- heavy sets and salience -> coefficient along u
    gh = _gen(master, "heavy", "cpu")
    if shape.drift:
        n_groups = w + 5
        coef = torch.zeros((B, N, n_groups), dtype=torch.float32)
        for b in range(B):
            nb = int(lens[b])
            per = max(1, math.ceil(0.001 * nb))
            perm = torch.randperm(nb, generator=gh)
            for t in range(n_groups):
                coef[b, perm[t * per:(t + 1) * per], t] = 3.0
    else:
        coef = torch.zeros((B, N), dtype=torch.float32)
        for b in range(B):
            nb = int(lens[b])
            cnt = max(1, math.ceil(shape.heavy_frac * nb))
            coef[b, torch.randperm(nb, generator=gh)[:cnt]] = 3.0
        if shape.sigma > 0:
            gs = _gen(master, "salience", "cpu")
            coef += torch.exp(shape.sigma * torch.randn((B, N), generator=gs))
    coef = coef.to(dev)

    # ---- keys / values (logical contiguous layout first)
    gk = _gen(master, "K", dev)
    K = _randn((B, N, Hkv, d), gk, dev)
    if shape.drift:
        K += torch.einsum("bnt,gtd->bngd", coef, U)
    else:
        K += coef[:, :, None, None] * U[None, None, :, :]
    gv = _gen(master, "V", dev)
    V = _randn((B, N, Hkv, d), gv, dev)

    # ---- queries: steps -1 (history) .. w-1 (window)
    gq = _gen(master, "q", dev)
    zeta = _randn((B, Hq, d), gq, dev)
    kv_of = torch.arange(Hq, device=dev) // G
    gdq = _gen(master, "drift_q", dev)
    steps = []
    for s in range(-1, w):
        if shape.drift:
            base = zeta + math.sqrt(d) * U[kv_of][:, s + 1:s + 6, :].sum(1)[None]
        else:
            base = zeta + math.sqrt(d) * U[kv_of][None]
        if s == 0:
            steps.append(base)
        else:
            steps.append(base + 0.2 * _randn((B, Hq, d), gdq, dev))
    q_all = torch.stack(steps, dim=1)           # [B][w+1][Hq][d], index 0 = history
    q_prev = q_all[:, 0].clone()                 # q_{i-1}, every head (float32)
    q = q_all[:, 1:]
    sub_heads = spread_heads(shape)
    q_hist = torch.stack([q_all[:, 0, h] for (_, h) in sub_heads], dim=1)   # [B][S][d]

    # ---- draft model
    L_d, H_d, Hkv_d, d_d = shape.L_d, shape.H_d, shape.Hkv_d, shape.d_d
    G_d = H_d // Hkv_d
    gp = _gen(master, "proj", dev)
    Pm = _randn((L_d, Hkv_d, d_d, d), gp, dev) / math.sqrt(d)
    gkn = _gen(master, "draft_k_noise", dev)
    gqn = _gen(master, "draft_q_noise", dev)
    Kd = torch.empty((L_d, B, N, Hkv_d, d_d), device=dev, dtype=torch.float32)
    q_draft = torch.empty((B, L_d, w, H_d, d_d), device=dev, dtype=torch.float32)
    for l in range(L_d):
        for c in range(Hkv_d):
            t = (l * Hkv_d + c) % Hkv
            Kd[l, :, :, c, :] = K[:, :, t, :] @ Pm[l, c].T + 0.3 * _randn((B, N, d_d), gkn, dev)
        for h in range(H_d):
            c = h // G_d
            t = (l * Hkv_d + c) % Hkv
            ht = t * G + ((l + h) % G)
            q_draft[:, l, :, h, :] = q[:, :, ht, :] @ Pm[l, c].T + 0.3 * _randn((B, w, d_d), gqn, dev)

    # ---- round to the storage dtype
    K = K.to(store)
    V = V.to(store)
    Kd = Kd.to(store)
    q = q.to(store).contiguous()
    q_hist = q_hist.to(store).contiguous()
    q_draft = q_draft.to(store).contiguous()

    # ---- poison rows beyond each sequence's length
    nan = float("nan")
    for b in range(B):
        nb = int(lens[b])
        if nb < N:
            K[b, nb:] = nan
            V[b, nb:] = nan
            Kd[:, b, nb:] = nan

    page_table = None
    if shape.page_size:
        ps = shape.page_size
        npg = [(int(lens[b]) + ps - 1) // ps for b in range(B)]
        total = sum(npg)
        maxp = (N + ps - 1) // ps
        gpg = _gen(master, "pages", "cpu")
        phys = torch.randperm(total, generator=gpg)
        page_table = torch.full((B, maxp), -1, dtype=torch.int32)
        Kp = torch.full((total, ps, Hkv, d), nan, dtype=store, device=dev)
        Vp = torch.full((total, ps, Hkv, d), nan, dtype=store, device=dev)
        Kdp = torch.full((L_d, total, ps, Hkv_d, d_d), nan, dtype=store, device=dev)
        off = 0
        for b in range(B):
            ids = phys[off:off + npg[b]]
            off += npg[b]
            page_table[b, :npg[b]] = ids.to(torch.int32)
            idd = ids.to(dev)
            span = npg[b] * ps
            kb = K[b, :span]
            vb = V[b, :span]
            kdb = Kd[:, b, :span]
            if kb.shape[0] < span:   # n_b == N with N not a page multiple
                extra = span - kb.shape[0]
                kb = torch.cat([kb, torch.full((extra, Hkv, d), nan, dtype=store, device=dev)])
                vb = torch.cat([vb, torch.full((extra, Hkv, d), nan, dtype=store, device=dev)])
                kdb = torch.cat([kdb, torch.full((L_d, extra, Hkv_d, d_d), nan, dtype=store, device=dev)], 1)
            Kp[idd] = kb.reshape(npg[b], ps, Hkv, d)
            Vp[idd] = vb.reshape(npg[b], ps, Hkv, d)
            Kdp[:, idd] = kdb.reshape(L_d, npg[b], ps, Hkv_d, d_d)
        K, V, Kd = Kp, Vp, Kdp
        page_table = page_table.to(dev)

    return Inputs(shape=shape, seq_lens=lens.to(torch.int32).to(dev), q=q, q_hist=q_hist,
                  sub_heads=sub_heads, q_draft=q_draft, K=K.contiguous(), V=V.contiguous(),
                  Kd=Kd.contiguous(), page_table=page_table, extra={"q_prev": q_prev, "master": master})


def history_trajectory(x: Inputs, deltas):
    """Past target queries q_{i-delta} for each delta in ``deltas`` (all >= 1),
    [len(deltas)][B][Hq][d] in the storage dtype: q_{i-1} is the generator's
    history query, and each earlier step adds an independent N(0, 0.2^2)
    drift, q_{i-t} = q_{i-t+1} + 0.2 * z_t (the same per-step drift the
    window queries carry), so a query further back has drifted further."""
    deltas = [int(t) for t in deltas]
    assert deltas and min(deltas) >= 1
    shape = x.shape
    dev = x.q.device
    g = _gen(x.extra["master"], "trajectory", dev)
    cur = x.extra["q_prev"].clone()
    want = {t: i for i, t in enumerate(deltas)}
    out = [None] * len(deltas)
    for t in range(1, max(deltas) + 1):
        if t > 1:
            cur = cur + 0.2 * _randn(tuple(cur.shape), g, dev)
        if t in want:
            out[want[t]] = cur.clone()
    store = x.q.dtype
    return torch.stack(out).to(store).contiguous()


@dataclass
class SearchInputs:
    """Profiling batch of the offline configuration search: several target
    layers, each with its own keys, window queries and previous query per
    head, plus the draft's layers.  Every sequence has length n."""
    shape: Shape
    L_t: int
    seq_lens: torch.Tensor          # [B] int32 (all n)
    K: torch.Tensor                 # [L_t][B][n][Hkv][d]
    q: torch.Tensor                 # [L_t][B][w][Hq][d] window queries
    q_prev: torch.Tensor            # [L_t][B][Hq][d] previous query of every head
    Kd: torch.Tensor                # [L_d][B][n][Hkv_d][d_d]
    q_draft: torch.Tensor           # [B][L_d][w][H_d][d_d]
    rho: torch.Tensor               # [L_t][Hq] retrieval quality of each head's previous query
    share: torch.Tensor             # [L_t] fraction of the shared salient set a layer attends
    draft_noise: torch.Tensor       # [L_d] noise level of each draft layer


def make_search(shape: Shape, L_t: int, seed=None, device="cpu"):
    """Synthetic multi-layer profiling data for the configuration search.

    The context has a shared set of salient positions.  Target layer l
    attends a fraction share[l] of it plus salient positions of its own
    (keys pushed along one direction per KV head, as in ``make``); its window
    queries point along that direction.  The previous query of head (l, h)
    points along it only with weight rho[l][h]: about a quarter of the heads
    are retrieval-like (rho in [0.8, 1.2]), the rest diffuse (rho in [0,
    0.4]).  Every draft layer is a random projection of the target layers'
    summed salient structure (keys: salience times direction; queries: the
    directions), so its attention weights a position by how many layers
    attend it, plus noise of the layer's own level: some draft layers are
    informative and some are not.  Lengths are all n (no padding)."""
    dev = torch.device(device)
    master = (shape.seed if seed is None else seed) + 7919 * L_t
    B, N, Hq, Hkv, d, w = shape.B, shape.n, shape.Hq, shape.Hkv, shape.d, shape.w
    G = Hq // Hkv
    store = torch.float32 if shape.dtype == "f32" else torch.bfloat16
    L_d, H_d, Hkv_d, d_d = shape.L_d, shape.H_d, shape.Hkv_d, shape.d_d
    G_d = H_d // Hkv_d

    gh = _gen(master, "search_heavy", "cpu")
    cnt = max(1, math.ceil(shape.heavy_frac * N))
    shared = [torch.randperm(N, generator=gh)[:cnt] for _ in range(B)]
    gl = _gen(master, "search_layer", "cpu")
    share = 0.3 + 0.7 * torch.rand(L_t, generator=gl)
    grho = _gen(master, "search_rho", "cpu")
    retr = torch.rand((L_t, Hq), generator=grho) < 0.25
    rho = torch.where(retr, 0.8 + 0.4 * torch.rand((L_t, Hq), generator=grho), 0.4 * torch.rand((L_t, Hq), generator=grho))
    gd = _gen(master, "search_draft", dev)
    draft_noise = 0.2 + 1.3 * torch.rand(L_d, generator=_gen(master, "search_draft", "cpu"))
    Pm = _randn((L_d, Hkv_d, d_d, d), gd, dev) / math.sqrt(d_d)   # keeps inner products in expectation

    K = torch.empty((L_t, B, N, Hkv, d), dtype=store, device=dev)
    q = torch.empty((L_t, B, w, Hq, d), dtype=store, device=dev)
    q_prev = torch.empty((L_t, B, Hq, d), dtype=store, device=dev)
    Kd = torch.empty((L_d, B, N, Hkv_d, d_d), dtype=store, device=dev)
    q_draft = torch.empty((B, L_d, w, H_d, d_d), dtype=store, device=dev)
    kv_of = torch.arange(Hq, device=dev) // G
    for l in range(L_t):
        gk = _gen(master * 131 + l, "K", dev)
        gq = _gen(master * 131 + l, "q", dev)
        gs = _gen(master * 131 + l, "salience", "cpu")
        coef = torch.zeros((B, N), dtype=torch.float32)
        keep = int(round(float(share[l]) * cnt))
        for b in range(B):
            coef[b, shared[b][torch.randperm(cnt, generator=gs)[:keep]]] = 3.0
            coef[b, torch.randperm(N, generator=gs)[:cnt - keep]] = 3.0
        if shape.sigma > 0:
            coef += torch.exp(shape.sigma * torch.randn((B, N), generator=gs))
        coef = coef.to(dev)
        U = _randn((Hkv, d), gk, dev)
        U = U / U.norm(dim=-1, keepdim=True)
        Kl = _randn((B, N, Hkv, d), gk, dev) + coef[:, :, None, None] * U[None, None]
        zeta = _randn((B, Hq, d), gq, dev)
        lead = math.sqrt(d) * U[kv_of][None]                              # [1][Hq][d]
        ql = torch.stack([zeta + lead + (0.2 * _randn((B, Hq, d), gq, dev) if s else 0.0) for s in range(w)], dim=1)
        r = rho[l].to(dev)[None, :, None]
        qp = zeta + r * lead + 0.2 * _randn((B, Hq, d), gq, dev)
        if l == 0:
            ksig = torch.zeros((B, N, Hkv, d), dtype=torch.float32, device=dev)
            qsig = torch.zeros((Hq, d), dtype=torch.float32, device=dev)
        ksig += coef[:, :, None, None] * U[None, None] / math.sqrt(L_t)    # the layers' salient structure
        qsig += lead[0] / math.sqrt(L_t)
        K[l] = Kl.to(store)
        q[l] = ql.to(store)
        q_prev[l] = qp.to(store)
        del Kl
    # draft layers: projections of the layers' summed salient structure, each with its own noise
    for ld in range(L_d):
        nz = float(draft_noise[ld])
        for c in range(Hkv_d):
            t = (ld * Hkv_d + c) % Hkv
            Kd[ld, :, :, c, :] = (ksig[:, :, t, :] @ Pm[ld, c].T + nz * _randn((B, N, d_d), gd, dev)).to(store)
        for h in range(H_d):
            c = h // G_d
            t = (ld * Hkv_d + c) % Hkv
            ht = t * G + ((ld + h) % G)
            qd = qsig[ht] @ Pm[ld, c].T                                       # [d_d]
            q_draft[:, ld, :, h, :] = (qd[None, None] + nz * _randn((B, w, d_d), gd, dev)).to(store)
    del ksig, qsig
    lens = torch.full((B,), N, dtype=torch.int32, device=dev)
    return SearchInputs(shape=shape, L_t=L_t, seq_lens=lens, K=K, q=q, q_prev=q_prev, Kd=Kd, q_draft=q_draft,
                        rho=rho, share=share, draft_noise=draft_noise)

