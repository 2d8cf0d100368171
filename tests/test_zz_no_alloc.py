"""dustin_sparse_verify_attn_noalloc (static per-GPU scratch, no workspace)
against dustin_sparse_verify_attn with a workspace, through the C ABI: two
calls in a row, the second on a smaller input, each bitwise equal to the
workspace form and within the attention bar (max-abs 2e-2, bf16) of the
oracle on sampled sequences."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_kv_verification_amd as dk
from _util import f64, make_idx, oracle_kv, say, valid_set

pytestmark = pytest.mark.gpu
DEV = "cuda"

CALLS = [
    # the 72B-shaped headline workload at k = 2048 (what bench.py times), then a smaller one
    ("c4-full-k2048", "c4", dict(layers=1, L_d=1), 2048, (0, 15)),
    ("qwen32b-rows20-small", "c4", dict(B=2, n=3000, Hq=40, Hkv=8, k=300, L_d=1), 300, (0, 1)),
]


def _one(name, base, over, k, sample):
    say("no-alloc attention", name)
    x = synth.make(synth.preset(base).replace(**over), device=DEV)
    sh = x.shape
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    idx, cnt = make_idx(x.seq_lens, k, seed=zlib.crc32(name.encode()) % 1000, device=DEV, frac_invalid=0.01)
    lse_a = torch.empty((sh.B, sh.w, sh.Hq), dtype=torch.float32, device=DEV)
    lse_b = torch.empty_like(lse_a)
    out_a = dk.dustin_sparse_verify_attn_noalloc(x.q, kv, idx, cnt, lse=lse_a)
    out_b = dk.dustin_sparse_verify_attn(x.q, kv, idx, cnt, lse=lse_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.uint8), out_b.view(torch.uint8)), "output differs from the workspace form"
    assert torch.equal(lse_a, lse_b), "lse differs from the workspace form"
    for b in sample:
        n = int(x.seq_lens[b])
        I = valid_set(idx[b].cpu().numpy(), int(cnt[b]), n)
        O, L = oracle.sparse_attention(f64(x.q[b]), oracle_kv(x, "K", b), oracle_kv(x, "V", b), I)
        err, lerr = np.abs(f64(out_a[b]) - O).max(), np.abs(f64(lse_a[b]) - L).max()
        say(f"  b={b} |I|={len(I)} max|dO|={err:.2e} max|dlse|={lerr:.2e}")
        assert err <= 2e-2 and lerr <= 2e-3


def test_noalloc_matches_workspace_form_two_calls():
    for name, base, over, k, sample in CALLS:
        _one(name, base, over, k, sample)


def test_noalloc_dense_form():
    say("no-alloc attention, dense form")
    x = synth.make(synth.preset("c5").replace(B=2, n=3000, n_lo=900, L_d=1), device=DEV)
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    a = dk.dustin_sparse_verify_attn_noalloc(x.q, kv)
    b = dk.dustin_sparse_verify_attn(x.q, kv)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
