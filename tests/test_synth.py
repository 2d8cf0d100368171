"""Seeded generator: determinism and the structure the recipe promises."""
import math

import torch

import synth


def _small(name, **kw):
    sh = synth.preset(name)
    base = dict(B=2, n=700, L_d=2)
    if name == "c5":
        base.update(n_lo=200)
    base.update(kw)
    return sh.replace(**base)


def test_same_seed_same_bytes():
    for name in ("c1", "c2", "c5"):
        sh = synth.preset("c1") if name == "c1" else _small(name)
        a, b = synth.make(sh), synth.make(sh)
        for f in ("q", "q_hist", "q_draft", "K", "V", "Kd", "seq_lens"):
            ta, tb = getattr(a, f), getattr(b, f)
            assert torch.equal(ta.view(torch.uint8) if ta.is_floating_point() else ta,
                               tb.view(torch.uint8) if tb.is_floating_point() else tb), (name, f)
    c = synth.make(_small("c2"), seed=99)
    assert not torch.equal(c.K, synth.make(_small("c2")).K)


def test_shapes_dtypes_and_poison():
    sh = _small("c2", n=300)
    x = synth.make(sh)
    assert x.K.dtype == torch.bfloat16 and x.K.shape == (2, 300, 4, 128)
    assert x.q.shape == (2, 4, 28, 128) and x.q_hist.shape == (2, 4, 128)
    assert x.q_draft.shape == (2, 2, 4, 14, 64) and x.Kd.shape == (2, 2, 300, 2, 64)
    assert x.sub_heads == [(0, 0), (0, 7), (0, 14), (0, 21)]
    p = synth.make(_small("c5"))
    assert p.page_table is not None and p.K.shape[1:] == (16, 8, 128)
    for b in range(2):
        n = int(p.seq_lens[b])
        assert 200 <= n <= 700
        assert not torch.isnan(p.logical("K", b).float()).any()
        npg = math.ceil(n / 16)
        last = p.K[int(p.page_table[b, npg - 1])]
        tail = n - (npg - 1) * 16
        assert torch.isnan(last[tail:].float()).all()
    ids = p.page_table[p.page_table >= 0]
    assert ids.unique().numel() == ids.numel() == p.K.shape[0]


def test_heavy_hitters_present():
    sh = synth.preset("c1")
    x = synth.make(sh)
    K = x.K[0, :, 0].double()
    # projection on the shared direction separates the +3 sigma heavy rows
    proj = K @ (x.q[0, 0, 0].double() - 0)  # query carries sqrt(d) u
    top = proj.topk(int(math.ceil(0.02 * 1024))).values.mean()
    assert top > proj.mean() + 3 * math.sqrt(64) * 0.8


def test_search_inputs_shapes_determinism_and_structure():
    """The multi-layer profiling batch: shapes and dtypes, the same bytes for
    the same seed, finite values (no padding), and retrieval-like heads whose
    previous query leans on the layer's salient direction more than the rest."""
    sh = synth.preset("c4").replace(B=2, n=1024, Hq=8, Hkv=2, d=64, L_d=4, H_d=4, Hkv_d=2, d_d=32)
    a = synth.make_search(sh, 3)
    b = synth.make_search(sh, 3)
    assert a.K.shape == (3, 2, 1024, 2, 64) and a.q.shape == (3, 2, 4, 8, 64) and a.q_prev.shape == (3, 2, 8, 64)
    assert a.Kd.shape == (4, 2, 1024, 2, 32) and a.q_draft.shape == (2, 4, 4, 4, 32)
    assert a.K.dtype == torch.bfloat16 and int(a.seq_lens.min()) == 1024
    for t in ("K", "q", "q_prev", "Kd", "q_draft"):
        assert torch.equal(getattr(a, t), getattr(b, t)), t
        assert torch.isfinite(getattr(a, t).float()).all(), t
    # cosine of the previous query with the window query's lead direction grows with rho
    lead = a.q[:, :, 0].float().mean(dim=1)                     # [L][Hq][d] (offsets average out less, still informative)
    cos = torch.nn.functional.cosine_similarity(a.q_prev.float().mean(dim=1), lead, dim=-1)
    hi, lo = cos[a.rho > 0.7].mean(), cos[a.rho < 0.2].mean()
    assert hi > lo
