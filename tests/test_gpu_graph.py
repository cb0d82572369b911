"""The fused paged decode captured into a HIP graph (torch's CUDA-graph API
over HIP): the decode path records no memset nodes, and every replay must
give the eager call's outputs bit for bit.  Three replays, with eager work
on the same buffers between them and the outputs overwritten before each, so
a replay that left any output unwritten, or read a stale buffer, fails."""
import pytest
import torch

from dsa_inputs import configs, device
from dsa_run import ws_tensor

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def test_paged_decode_graph_replays_equal_eager(dsa):
    wl = configs.WORKLOADS["paged_decode_b32_ctx4k_128k"]
    _case("paged decode under HIP graph capture: inputs")
    inp = device.make_paged_inputs(wl)
    B, k = 8, wl.k  # the first 8 sequences
    pt = inp["page_table"][:B].contiguous()
    max_pages = pt.shape[1]
    ctx = inp["ctx_len"][:B].contiguous()
    max_ctx = int(ctx.max().item())
    nb = dsa.dsa_forward_decode_paged_workspace_bytes(B, max_ctx, wl.H, wl.D_v, k)
    ws = ws_tensor(nb)
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, wl.H, wl.D_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, wl.H), dtype=torch.float32, device="cuda")

    def call():
        dsa.dsa_forward_decode_paged(inp["q_idx"][:B], inp["w"][:B], inp["k_pool"], inp["q"][:B], inp["kv_pool"],
                                     inp["n_pages"], pt, max_pages, ctx, wl.page, B, max_ctx, wl.H_I, wl.d_I, wl.H,
                                     wl.D_qk, wl.D_v, k, wl.scale, idx, out, lse, ws, nb)

    def scribble():
        idx.fill_(-7)
        out.fill_(7.0)
        lse.fill_(7.0)

    _case("eager call")
    call()  # also sets the kernels' attributes before capture
    torch.cuda.synchronize()
    ref = (idx.clone(), out.clone(), lse.clone())
    _case("capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        _case(f"replay {rep}")
        scribble()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(out, ref[1]) and torch.equal(lse, ref[2]), f"replay {rep}"
        scribble()
        call()  # eager work on the same buffers between replays
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(out, ref[1]) and torch.equal(lse, ref[2])
