"""The allocation-free decode entry point (hla_decode_windowed_noalloc):
its workspace is the library's per-GPU scratch array.  Checked against
hla_decode_windowed with a caller workspace on the same inputs (the same
kernels and plan, so the outputs and rings agree bit for bit) and against
the fp64 oracle, on two calls in a row, the second one smaller."""
import ctypes

import numpy as np
import pytest
import torch

from compressed_cross_loop_amd import binding as B
from synth import gen
from tests.gpu_cases import TOL, desc_of, oracle_decode, poison_unread
from tests.util import max_rel_err


def _case(seed, *, positions, r, W, loop):
    c = gen.decode_inputs(seed, batch=len(positions), heads=16, head_dim=128, groups=1, r_k=r, r_v=r,
                          positions=positions, window=W, dtype="bf16", rope_base=10000.0, rope_baked=1,
                          loop=loop, loop_first=1 if loop == 1 else 2, loop_last=1 if loop == 1 else 4,
                          latent_std=np.sqrt(3.0), exact_std=np.sqrt(3.0))
    return poison_unread(c)


def _run(c, noalloc, flags=0):
    dev = "cuda"
    desc = desc_of(c)
    rk, rv = c.ring_k.to(dev), c.ring_v.to(dev)
    out = torch.full(tuple(c.q.shape), float("nan"), dtype=torch.bfloat16, device=dev)
    mp = int(c.pos.max())
    ws = None
    if not noalloc:
        nbytes = B.lla_decode_workspace_bytes(desc, c.batch, mp, c.window)
        ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=dev)
    args = B.decode_args(loop=c.loop, window=c.window, pos=c.pos.to(dev), q=c.q.to(dev), k_cur=c.k_cur.to(dev),
                         v_cur=c.v_cur.to(dev), ring_k=rk, ring_v=rv, A=c.A.to(dev),
                         B=c.Bv.transpose(1, 2).contiguous().to(dev), out=out, workspace=ws, max_pos_hint=mp,
                         flags=flags)
    st = B.store(c.pages.to(dev), c.block_table.to(dev))
    (B.hla_decode_windowed_noalloc if noalloc else B.hla_decode_windowed)(desc, st, c.batch, args)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), rk.float().cpu().numpy(), rv.float().cpu().numpy()


@pytest.mark.gpu
@pytest.mark.parametrize("flags", [0, B.LLA_FLAG_FUSED])
def test_noalloc_matches_workspace_entry(flags):
    cases = [dict(seed=51, positions=(4095, 700, 129, 128), r=512, W=128, loop=3),   # 8.7 MiB of workspace
             dict(seed=52, positions=(300, 37), r=256, W=16, loop=1)]                # smaller, second
    for k in cases:
        c = _case(**k)
        print(f"[case] noalloc flags={flags} B={c.batch} r={c.r_k} W={c.window} pos={c.pos.tolist()}", flush=True)
        got = _run(c, True, flags)
        want = _run(c, False, flags)
        for g, w in zip(got, want):
            np.testing.assert_array_equal(g, w)
        ref, *_ = oracle_decode(c, "absorbed")
        assert max_rel_err(got[0], ref) < TOL["bf16"]


def _fake_args(**kw):
    FAKE = 0x10000   # aligned, never dereferenced: the calls below fail validation first
    base = dict(loop=2, window=128, max_pos_hint=4095, splits=0, flags=0, pos=FAKE, q=FAKE, k_cur=FAKE,
                v_cur=FAKE, ring_k=FAKE, ring_v=FAKE, A=FAKE, B=FAKE, out=FAKE, workspace=None,
                workspace_bytes=0, scan_events=None)
    base.update(kw)
    return B.LlaDecodeArgs(*base.values())


def test_noalloc_rejects_without_launching():
    """Host-side rejections, before any HIP call: a workspace passed in, sizes
    beyond the 32 MiB array, and the regular entry point's own checks."""
    st = B.LlaStore(0x10000, 0x10000, 64)
    hla = B.set_desc(n_heads=16, head_dim=128, groups=1, r_k=512, r_v=512, loop_first=2, loop_last=4,
                     page_size=64, rope_baked=1, rope_base=10000.0, dtype=B.LLA_BF16)
    f = B.lib.hla_decode_windowed_noalloc
    assert f(ctypes.byref(hla), ctypes.byref(st), 128, ctypes.byref(_fake_args(workspace=0x10000)), None) == \
        B.LLA_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(hla), ctypes.byref(st), 128, ctypes.byref(_fake_args(workspace_bytes=16)), None) == \
        B.LLA_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(hla), ctypes.byref(st), 128, None, None) == B.LLA_ERR_INVALID_ARGUMENT
    # batch 128 at 4k needs 16.1 MiB: fits; batch 512 needs more than 32 MiB
    assert B.lla_decode_workspace_bytes(hla, 128, 4095, 128) <= B.NOALLOC_SCRATCH_BYTES
    assert B.lla_decode_workspace_bytes(hla, 512, 4095, 128) > B.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(hla), ctypes.byref(st), 512, ctypes.byref(_fake_args()), None) == \
        B.LLA_ERR_WORKSPACE_TOO_SMALL
    # an invalid descriptor or loop: the regular entry point's status
    bad = B.set_desc(n_heads=16, head_dim=128, groups=2, r_k=512, r_v=512, loop_first=2, loop_last=4,
                     page_size=64, rope_baked=1, rope_base=10000.0, dtype=B.LLA_BF16)
    assert f(ctypes.byref(bad), ctypes.byref(st), 128, ctypes.byref(_fake_args()), None) == \
        B.LLA_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(hla), ctypes.byref(st), 128, ctypes.byref(_fake_args(loop=7)), None) == \
        B.LLA_ERR_INVALID_ARGUMENT
