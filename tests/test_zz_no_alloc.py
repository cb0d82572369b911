"""The allocation-free paged decode (dsa_forward_decode_paged_noalloc) against
the workspace call on the same inputs: two calls in a row, the second with a
smaller batch and shorter contexts, each bit-identical to the workspace call.
Collected last, so a failure here hides no other test."""
import numpy as np
import pytest
import torch

from dsa_inputs import configs, device
from dsa_run import ws_tensor

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _run(dsa, wl, inp, pt, ctx, noalloc):
    B, max_pages = pt.shape
    max_ctx = int(ctx.max().item())
    k = wl.k
    idx = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, wl.H, wl.D_v), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((B, wl.H), 7.0, dtype=torch.float32, device="cuda")
    args = (inp["q_idx"][:B], inp["w"][:B], inp["k_pool"], inp["q"][:B], inp["kv_pool"], inp["n_pages"], pt,
            max_pages, ctx, wl.page, B, max_ctx, wl.H_I, wl.d_I, wl.H, wl.D_qk, wl.D_v, k, wl.scale, idx, out, lse)
    if noalloc:
        dsa.dsa_forward_decode_paged_noalloc(*args)
    else:
        nb = dsa.dsa_forward_decode_paged_workspace_bytes(B, max_ctx, wl.H, wl.D_v, k)
        ws = ws_tensor(nb)
        dsa.dsa_forward_decode_paged(*args, ws, nb)
    torch.cuda.synchronize()
    return idx, out, lse


def test_noalloc_paged_decode_equals_workspace_call(dsa):
    wl = configs.WORKLOADS["paged_decode_b32_ctx4k_128k"]
    _case("noalloc paged decode: inputs")
    inp = device.make_paged_inputs(wl)
    pt, ctx = inp["page_table"], inp["ctx_len"]
    # the second call: the first 6 sequences, contexts cut to at most 5000
    # tokens (two of them shorter than k), their page-table rows unchanged
    ctx2 = torch.clamp(ctx[:6], max=5000).clone()
    ctx2[1] = 1500
    ctx2[4] = 64
    pt2 = pt[:6].contiguous()
    _case("noalloc paged decode: workspace calls")
    ref1 = _run(dsa, wl, inp, pt, ctx, False)
    ref2 = _run(dsa, wl, inp, pt2, ctx2, False)
    _case("noalloc paged decode: call 1 (32 sequences, 4K..128K)")
    got1 = _run(dsa, wl, inp, pt, ctx, True)
    _case("noalloc paged decode: call 2 (6 sequences, <= 5000 tokens)")
    got2 = _run(dsa, wl, inp, pt2, ctx2, True)
    for ref, got, name in ((ref1, got1, "first"), (ref2, got2, "second")):
        for r, g, what in zip(ref, got, ("idx", "out", "lse")):
            assert torch.equal(r, g), f"{name} call: {what} differs from the workspace call"
    assert int((got2[0][4] >= 0).sum().item()) == 64  # a 64-token context selects all 64 positions
