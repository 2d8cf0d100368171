"""The step captured in a HIP graph (as bench.py times it) and replayed:
score -> select -> sparse attention over two layers, plus the window
attention of the evaluator.  Every replay must reproduce the eager results
bit for bit (all these kernels are deterministic), with eager work on other
inputs and synchronisations between the replays: whatever state a call
leaves in its workspace (attention arrival counters, the chunked select's
counters) must be back where the next call, captured or not, expects it.
"""
import pytest
import torch

import synth
import sparse_kv_verification_amd as dk
from _util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # contiguous, register-resident select (n <= 32768), statistics items of 8192 positions
    ("contiguous", dict(base="c4", B=16, n=20000, L_d=3)),
    # longer rows: the chunked multi-work-group select; ragged lengths
    ("chunked-select", dict(base="c4", B=3, n=50000, n_lo=33000, L_d=2)),
    # paged, ragged, w = 8 (window attention in two slices), one KV head per draft item
    ("paged-ragged-w8", dict(base="c5", B=3, n=6000, n_lo=2000, L_d=2)),
]


class Step:
    """Preallocated buffers and workspaces for one configuration; run() issues
    the calls on the current stream."""

    def __init__(self, sh, x, layers=2):
        self.sh, self.x = sh, x
        self.k = min(sh.k, 2048)
        self.ns, self.nw, self.m = synth.tier_defaults(self.k)
        self.kvs = [dk.KV(x.K if l == 0 else x.K.clone(), x.V if l == 0 else x.V.clone(), x.seq_lens, x.page_table)
                    for l in range(layers)]
        self.dkv = [dk.KV(x.Kd[l], None, x.seq_lens, x.page_table) for l in range(sh.L_d)]
        N = self.kvs[0].desc.N_max
        f32 = dict(dtype=torch.float32, device=DEV)
        self.s_d = torch.empty((sh.B, N), **f32)
        self.s_t = torch.empty((sh.B, N), **f32)
        self.idx = torch.empty((sh.B, self.k), dtype=torch.int32, device=DEV)
        self.cnt = torch.empty((sh.B,), dtype=torch.int32, device=DEV)
        self.tier = torch.empty((sh.B, self.k), dtype=torch.int8, device=DEV)
        self.out = [torch.empty_like(x.q) for _ in range(layers)]
        self.A = torch.empty((sh.B, sh.w, N), **f32)
        self.ws = {nm: dk.Workspace() for nm in ("score", "topk", "attn", "win")}

    def run(self, q):
        x, sh = self.x, self.sh
        dk.dustin_score(self.dkv, x.q_draft, [self.kvs[0]], x.q_hist, x.sub_heads, sh.Hq, s_draft=self.s_d,
                        s_target=self.s_t, ws=self.ws["score"])
        dk.dustin_topk(self.s_d, self.s_t, x.seq_lens, self.k, self.m, self.ns, self.nw, idx=self.idx,
                       count=self.cnt, tier=self.tier, ws=self.ws["topk"])
        for l, kv in enumerate(self.kvs):
            dk.dustin_sparse_verify_attn(q, kv, self.idx, self.cnt, out=self.out[l], ws=self.ws["attn"])
        dk.dustin_window_attn(q, self.kvs[0], A=self.A, ws=self.ws["win"])

    def snapshot(self):
        return [t.clone() for t in (self.s_d, self.s_t, self.idx, self.cnt, self.tier, *self.out, self.A)]


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(name, over):
    say("graph replay", name)
    over = dict(over)
    sh = synth.preset(over.pop("base")).replace(**over)
    x = synth.make(sh, device=DEV)
    st = Step(sh, x)
    q_other = (x.q.float() * 0.5).to(x.q.dtype)          # eager work between the replays
    st.run(x.q)
    torch.cuda.synchronize()
    want = st.snapshot()
    st.run(q_other)
    torch.cuda.synchronize()
    other = st.snapshot()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run(x.q)                                       # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            st.run(x.q)
    torch.cuda.synchronize()
    names = ["s_draft", "s_target", "idx", "count", "tier"] + [f"out[{l}]" for l in range(len(st.out))] + ["A"]
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        got = st.snapshot()
        for nm, a, b in zip(names, got, want):
            assert torch.equal(a, b), f"replay {rep}: {nm} differs from the eager result"
        st.run(q_other)                                   # eager, other inputs, same workspaces
        torch.cuda.synchronize()
        got = st.snapshot()
        for nm, a, b in zip(names, got, other):
            assert torch.equal(a, b), f"eager call after replay {rep}: {nm} differs"
        say(f"  replay {rep}: bitwise equal to eager; eager call after it unchanged")
