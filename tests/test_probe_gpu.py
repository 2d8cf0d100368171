"""The measurement kernels (achievable read and gather rates) run through
the C ABI: the read probe on a buffer whose size is not a multiple of its
grid stride, the gather probe with one and two tensors and a ragged last
work-group; their sink stays zero."""
import pytest
import torch

import sparse_kv_verification_amd as dk
from _util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_probe_stream_read():
    say("probe: stream read")
    buf = torch.randint(0, 1 << 30, ((1 << 22) + 12,), dtype=torch.int32, device=DEV)   # 16 MiB + 48 B
    for nt in (True, False):
        sink = dk.dustin_probe_stream_read(buf, nontemporal=nt)
        torch.cuda.synchronize()
        assert int(sink.abs().sum()) == 0


def test_probe_gather_rows():
    say("probe: gather rows")
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    K = torch.randn((4, 3000, 8, 128), device=DEV).to(torch.bfloat16)
    V = torch.randn_like(K)
    nrow = K.numel() * 2 // 256
    rows = torch.randint(0, nrow, (70001,), generator=g, device=DEV, dtype=torch.int32)
    dk.dustin_probe_gather_rows(K, rows, 256, 256)
    dk.dustin_probe_gather_rows(K, rows, 256, 256, base2=V)
    dk.dustin_probe_gather_rows(K, rows[:1000], 512, 2048, base2=V)
    torch.cuda.synchronize()
