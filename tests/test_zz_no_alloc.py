"""dl_moe_route_noalloc (the router with the library's static device scratch, for callers that cannot allocate)
against dl_moe_route on the same inputs: bit-identical experts, gates and logits, on two calls in a row, the second
with a smaller batch, so the second call runs on scratch the first one left behind.  Both go through the C ABI.
Also: a request above the scratch limit is refused on the host, before anything is enqueued."""
import ctypes as C
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_moe_amd as dl
from parity import expert_mismatch, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, E, D, seed):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, D, generator=g)
    w_r = torch.randn(E, D, generator=g) / math.sqrt(D)
    bias = torch.randn(E, generator=g) * 0.1
    return h.to(DEV), w_r.to(DEV), bias.to(DEV)


def _route(fn, h, w_r, bias, ke, **kw):
    B, E = h.shape[0], w_r.shape[0]
    ex = torch.full((B, ke), -7, dtype=torch.int32, device=DEV)
    gt = torch.full((B, ke), -7.0, dtype=torch.float32, device=DEV)
    lg = torch.full((B, E), -7.0, dtype=torch.float32, device=DEV)
    fn(h, w_r, bias, ke, ex, gt, logits=lg, **kw)
    return ex, gt, lg


def test_noalloc_router_matches_workspace_router_on_two_calls():
    cases = [(64, 256, 6144, 8, 21), (5, 256, 6144, 8, 22)]  # the second call smaller than the first
    for B, E, D, ke, seed in cases:
        h, w_r, bias = _inputs(B, E, D, seed)
        say(f"[gpu] moe_route vs moe_route_noalloc B={B} E={E} D={D} ke={ke}")
        ref = _route(dl.moe_route, h, w_r, bias, ke)
        got = _route(dl.moe_route_noalloc, h, w_r, bias, ke)
        torch.cuda.synchronize()
        for a, b, name in zip(got, ref, ("experts", "gates", "logits")):
            assert torch.equal(a, b), f"B={B}: {name} differ"
        # and both against the oracle (experts bit-exact up to the 1e-6 rule)
        ex = host(got[0])
        hh, wr, bs = h.cpu().double().numpy(), w_r.cpu().numpy(), bias.cpu().numpy()
        for b in range(B):
            ol, oe, og = oracle.router(hh[b], wr, bs, ke)
            assert expert_mismatch(ex[b], oe, ol) in (None, "near-tie"), f"row {b}"


def test_noalloc_router_refuses_sizes_above_its_scratch():
    L = dl.load()
    B, E, D = 1024, 1024, 16384  # 16 chunks x 1024 x 1024 x 8 B = 128 MiB > the scratch
    rc = L.dl_moe_route_noalloc(C.c_void_p(0x1000), B, D, C.c_void_p(0x2000), None, E, 8, C.c_void_p(0x3000),
                                C.c_void_p(0x4000), None, None)
    assert rc == -2 and b"scratch" in L.dl_last_error()
