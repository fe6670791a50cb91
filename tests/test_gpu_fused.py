"""Parity of the fused single-launch decode (LLA_FLAG_FUSED: query map, scan,
window and value map in one kernel, splits merged by the last workgroup to
arrive) with the fp64 oracle, through the C ABI, with the same poisoned
inputs and checks (output, ring append, untouched ring slots) as the
three-kernel decode tests."""
import numpy as np
import pytest
import torch

from compressed_cross_loop_amd import binding as B
from synth import gen
from tests.gpu_cases import TOL, oracle_decode, poison_unread, run_decode
from tests.test_gpu_decode import check, hla_case
from tests.util import max_rel_err

pytestmark = pytest.mark.gpu
F = B.LLA_FLAG_FUSED


@pytest.mark.parametrize("r", [512, 256])
@pytest.mark.parametrize("splits", [0, 1, 3, 9])
def test_fused_hla(r, splits):
    c = hla_case(600 + r, r=r, loop=1 if r == 256 else 3)
    check(c, "hla", "absorbed", splits=splits, flags=F)


@pytest.mark.parametrize("W, positions", [(128, (4095, 700, 129, 128)), (16, (0, 1, 16, 17)), (0, (5, 64, 65))])
def test_fused_windows_and_edges(W, positions):
    """W = 128 over many slices, the first token, windows covering the whole
    context, W = 0 (only the current token exact)."""
    c = hla_case(620 + W, positions=positions, W=W)
    check(c, "hla", "absorbed", flags=F)


@pytest.mark.parametrize("r, d_h, H, G, rope", [(128, 64, 8, 2, False), (256, 128, 16, 4, True),
                                                (1024, 128, 4, 1, True), (512, 64, 6, 3, False)])
def test_fused_absorbed_groups_and_widths(r, d_h, H, G, rope):
    """Absorbed LLA-D reads: several latent groups, r up to 1024, d_h = 64."""
    c = gen.decode_inputs(640 + r + H, batch=3, heads=H, head_dim=d_h, groups=G, r_k=r, r_v=r,
                          positions=(777, 20, 300), window=9, dtype="bf16", page_size=32,
                          rope_base=10000.0 if rope else 0.0, rope_baked=1 if rope else 0, loop=2,
                          loop_first=1, loop_last=4, paired=rope)
    check(poison_unread(c), "absorbed", "absorbed", splits=2, flags=F)


def test_fused_reuses_one_workspace_and_matches_three_kernel_path():
    """Two fused calls in a row on one workspace (tickets left by the first
    call, the rest NaN at first): identical outputs, and both within bf16
    rounding of the three-kernel path."""
    from tests.gpu_cases import desc_of
    c = hla_case(660, positions=(2000, 1), W=128)
    out3, _, _ = run_decode("hla", c)
    dev = "cuda"
    desc = desc_of(c)
    mp = int(c.pos.max())
    ws = torch.full((B.lla_decode_workspace_bytes(desc, c.batch, mp, c.window) // 4,), float("nan"),
                    dtype=torch.float32, device=dev)
    st = B.store(c.pages.to(dev), c.block_table.to(dev))
    outs = []
    for call in range(2):
        print(f"[case] fused call {call} on a shared workspace", flush=True)
        out = torch.full(tuple(c.q.shape), float("nan"), dtype=torch.bfloat16, device=dev)
        args = B.decode_args(loop=c.loop, window=c.window, pos=c.pos.to(dev), q=c.q.to(dev), k_cur=c.k_cur.to(dev),
                             v_cur=c.v_cur.to(dev), ring_k=c.ring_k.to(dev), ring_v=c.ring_v.to(dev), A=c.A.to(dev),
                             B=c.Bv.transpose(1, 2).contiguous().to(dev), out=out, workspace=ws, max_pos_hint=mp,
                             flags=F)
        B.hla_decode_windowed(desc, st, c.batch, args)
        torch.cuda.synchronize()
        outs.append(out.float().cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])
    assert max_rel_err(outs[0], out3) < TOL["bf16"]
