"""The decode and writer entry points captured in a HIP graph (torch.cuda.graph)
and replayed several times, with eager work and synchronisations between
replays, give bitwise the eager result every time."""
import numpy as np
import pytest
import torch

from compressed_cross_loop_amd import binding as B
from synth import gen

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    c = gen.decode_inputs(900, batch=4, heads=16, head_dim=128, groups=1, r_k=512, r_v=512,
                          positions=(700, 300, 129, 64), window=128, dtype="bf16",
                          rope_base=10000.0, rope_baked=1, loop=2, latent_std=np.sqrt(3.0),
                          exact_std=np.sqrt(3.0))
    desc = B.set_desc(n_heads=16, head_dim=128, groups=1, r_k=512, r_v=512, loop_first=2, loop_last=4,
                      page_size=64, rope_baked=1, rope_base=10000.0, dtype=B.LLA_BF16)
    dev = lambda t: t.cuda()
    pages, bt, pos = dev(c.pages), dev(c.block_table), dev(c.pos)
    q, kc, vc, rk, rv, A = map(dev, (c.q, c.k_cur, c.v_cur, c.ring_k, c.ring_v, c.A))
    Bv = dev(c.Bv.transpose(1, 2).contiguous())   # value decoder as B_t^T
    out = torch.empty_like(q)
    ws = torch.empty(B.lla_decode_workspace_bytes(desc, 4, 700, 128), dtype=torch.uint8, device="cuda")
    st = B.store(pages, bt)
    args = B.decode_args(loop=2, window=128, pos=pos, q=q, k_cur=kc, v_cur=vc, ring_k=rk, ring_v=rv, A=A,
                         B=Bv, out=out, workspace=ws, max_pos_hint=700)
    # latent write of the current tokens into a separate store
    wi = gen.writer_inputs(901, batch=4, n_tok=1, n_loops=3, groups=1, r_k=512, r_v=512, d_in=2048,
                           dtype="bf16", positions=[[700], [300], [129], [64]])
    wpages = torch.zeros_like(pages)
    wst = B.store(wpages, bt)
    wws = torch.empty(max(4, B.lla_write_workspace_bytes(desc, 4, 1, 2048)), dtype=torch.uint8, device="cuda")
    x, enc, wpos = dev(wi.x), dev(wi.enc), dev(wi.pos)

    def step():
        B.hla_decode_windowed(desc, st, 4, args)
        B.lla_write_latents(desc, wst, pos=wpos, x=x, enc=enc, workspace=wws)

    step()
    torch.cuda.synchronize()
    want_out, want_w = out.clone(), wpages.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        wpages.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_out), rep
        assert torch.equal(wpages, want_w), rep
        step()                      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, want_out)


@pytest.mark.parametrize("positions", [(300, 129, 7), (900,)])
def test_graph_replays_wide_absorbed(positions):
    """The two-pass absorbed read of a wide shared latent (query map, score,
    softmax and value passes, combine; at batch 1 the score pass is split
    along r_k) replays bitwise like the eager call."""
    nb = len(positions)
    c = gen.decode_inputs(910 + nb, batch=nb, heads=55, head_dim=96, groups=1, r_k=1056, r_v=1056,
                          positions=positions, window=4, dtype="bf16", loop=3, loop_first=1, loop_last=8,
                          latent_std=1.0, exact_std=1.0, paired=False, map_scale=float(np.sqrt(1056 / 96)))
    desc = B.set_desc(n_heads=55, head_dim=96, groups=1, r_k=1056, r_v=1056, loop_first=1, loop_last=8,
                      page_size=64, rope_baked=0, rope_base=0.0, dtype=B.LLA_BF16)
    assert B.lla_decode_scan_kernel(desc, 1) == "k_scan_absorbed_wide"
    dev = lambda t: t.cuda()
    pages, bt, pos = dev(c.pages), dev(c.block_table), dev(c.pos)
    q, kc, vc, rk, rv, A = map(dev, (c.q, c.k_cur, c.v_cur, c.ring_k, c.ring_v, c.A))
    Bv = dev(c.Bv.transpose(1, 2).contiguous())
    out = torch.empty_like(q)
    mp = max(positions)
    ws = torch.empty(B.lla_decode_workspace_bytes(desc, nb, mp, 4), dtype=torch.uint8, device="cuda")
    args = B.decode_args(loop=3, window=4, pos=pos, q=q, k_cur=kc, v_cur=vc, ring_k=rk, ring_v=rv, A=A,
                         B=Bv, out=out, workspace=ws, max_pos_hint=mp)
    st = B.store(pages, bt)

    def step():
        B.lla_decode_absorbed(desc, st, nb, args)

    step()
    torch.cuda.synchronize()
    want = out.clone()
    assert torch.isfinite(want.float()).all()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(255)               # stale workspace contents must not matter
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), rep
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, want)
