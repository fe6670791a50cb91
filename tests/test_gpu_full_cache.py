"""Parity of the uncompressed (full-cache) decode baseline with the fp64
oracle, through the C ABI.  Every cache slot a call must not read is NaN, the
workspace and the output start NaN-filled, and the slot of position i must
receive R_i k_cur, v_cur while every other slot stays bit-identical."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_cross_loop_amd import binding as B
from synth import gen
from tests.gpu_cases import TOL
from tests.util import max_rel_err

pytestmark = pytest.mark.gpu


def run_full(c, dtype, *, rope_base, splits=0, max_pos_hint=None):
    H, dh = int(c.q.shape[1]), int(c.q.shape[2])
    Bsz = int(c.q.shape[0])
    mp = int(c.pos.max()) if max_pos_hint is None else max_pos_hint
    print(f"[case] full-cache B={Bsz} H={H} d_h={dh} P={c.page_size} pos={c.pos.tolist()} dtype={dtype} "
          f"rope={rope_base} splits={splits} hint={mp}", flush=True)
    desc = B.kv_desc(n_heads=H, head_dim=dh, page_size=c.page_size, rope_base=rope_base,
                     dtype=B.LLA_BF16 if dtype == "bf16" else B.LLA_F32)
    kp, vp = c.k_pages.cuda(), c.v_pages.cuda()
    cache = B.kv_cache(kp, vp, c.block_table.cuda())
    out = torch.full(tuple(c.q.shape), float("nan"), dtype=c.q.dtype, device="cuda")
    ws = torch.full((max(4, B.lla_full_decode_workspace_bytes(desc, Bsz, mp, splits)) // 4,), float("nan"),
                    dtype=torch.float32, device="cuda")
    args = B.full_decode_args(pos=c.pos.cuda(), q=c.q.cuda(), k_cur=c.k_cur.cuda(), v_cur=c.v_cur.cuda(),
                              out=out, workspace=ws, max_pos_hint=mp, splits=splits)
    B.lla_decode_full_cache(desc, cache, Bsz, args)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), kp.float().cpu().numpy(), vp.float().cpu().numpy()


def check_full(c, dtype, *, rope_base, **kw):
    out, kp, vp = run_full(c, dtype, rope_base=rope_base, **kw)
    f = lambda t: t.double().numpy()
    ref = O.full_cache_decode(f(c.k_pages), f(c.v_pages), c.block_table.numpy(), c.pos.numpy(), f(c.q),
                              f(c.k_cur), f(c.v_cur), page_size=c.page_size, rope_base=rope_base)
    err = max_rel_err(out, ref)
    assert err < TOL[dtype], err
    # the appended slot, and nothing else written
    page, slot, k_new, v_new = O.kv_cache_update(c.pos.numpy(), f(c.k_cur), f(c.v_cur), c.block_table.numpy(),
                                                 page_size=c.page_size, rope_base=rope_base)
    k0, v0 = c.k_pages.float().numpy(), c.v_pages.float().numpy()
    for b in range(len(page)):
        assert max_rel_err(kp[page[b], slot[b]], k_new[b]) < TOL[dtype]
        np.testing.assert_array_equal(vp[page[b], slot[b]], c.v_cur[b].float().numpy())
        k0[page[b], slot[b]] = kp[page[b], slot[b]]
        v0[page[b], slot[b]] = vp[page[b], slot[b]]
    np.testing.assert_array_equal(kp, k0)
    np.testing.assert_array_equal(vp, v0)
    return err


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
def test_full_cache_bf16_ouro_heads(splits, rope_base):
    """16 heads x 128 (the Ouro-1.4B attention); first token, page edges,
    ragged ends, a long context."""
    c = gen.kv_cache_inputs(700 + splits, batch=7, heads=16, head_dim=128,
                            positions=(0, 1, 63, 64, 65, 700, 4095), dtype="bf16", page_size=64)
    check_full(c, "bf16", rope_base=rope_base, splits=splits)


def test_full_cache_fp32_tiny():
    """Workload 1 attention shape (2 heads x 64, fp32), small pages."""
    c = gen.kv_cache_inputs(710, batch=3, heads=2, head_dim=64, positions=(255, 16, 0), dtype="f32",
                            page_size=16)
    check_full(c, "f32", rope_base=0.0)
    c = gen.kv_cache_inputs(711, batch=3, heads=2, head_dim=64, positions=(255, 16, 0), dtype="f32",
                            page_size=16)
    check_full(c, "f32", rope_base=10000.0, splits=4)


def test_full_cache_two_head_blocks():
    """40 heads of 64: two head blocks per sequence, the second partial."""
    c = gen.kv_cache_inputs(720, batch=2, heads=40, head_dim=64, positions=(333, 96), dtype="bf16",
                            page_size=32)
    check_full(c, "bf16", rope_base=10000.0)


def test_full_cache_position_beyond_hint():
    """The split plan from a smaller hint still covers every cached token."""
    c = gen.kv_cache_inputs(730, batch=2, heads=16, head_dim=128, positions=(1500, 900), dtype="bf16")
    check_full(c, "bf16", rope_base=10000.0, max_pos_hint=100)


def test_full_cache_full_size_sampled():
    """Batch 32 at context 4096 (i = 4095) in the automatic split plan; the
    oracle checks four sequences."""
    Bsz, H, dh, P, i = 32, 16, 128, 64, 4095
    g = gen.rng(740)
    pps = i // P + 1
    bt, n_pages = gen.block_table(g, Bsz, pps, 2)
    kp = gen.device_normal((n_pages, P, H, dh), "bf16", 741)
    vp = gen.device_normal((n_pages, P, H, dh), "bf16", 742)
    q = gen.device_normal((Bsz, H, dh), "bf16", 743)
    kc = gen.device_normal((Bsz, H, dh), "bf16", 744)
    vc = gen.device_normal((Bsz, H, dh), "bf16", 745)
    pos = torch.full((Bsz,), i, dtype=torch.int32, device="cuda")
    desc = B.kv_desc(n_heads=H, head_dim=dh, page_size=P, rope_base=10000.0, dtype=B.LLA_BF16)
    bt_d = torch.from_numpy(bt).cuda()
    k_before = kp.clone()
    v_before = vp.clone()
    out = torch.full((Bsz, H, dh), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(B.lla_full_decode_workspace_bytes(desc, Bsz, i), dtype=torch.uint8, device="cuda")
    args = B.full_decode_args(pos=pos, q=q, k_cur=kc, v_cur=vc, out=out, workspace=ws, max_pos_hint=i)
    print(f"[case] full-cache full size B={Bsz} N={i + 1}", flush=True)
    B.lla_decode_full_cache(desc, B.kv_cache(kp, vp, bt_d), Bsz, args)
    torch.cuda.synchronize()
    seqs = [0, 11, 20, 31]
    sub_bt = np.arange(len(seqs) * pps).reshape(len(seqs), pps)
    phys = torch.from_numpy(bt[seqs].reshape(-1).astype(np.int64)).cuda()
    f = lambda t: t.index_select(0, phys).double().cpu().numpy()
    idx = torch.tensor(seqs, device="cuda")
    s = lambda t: t.index_select(0, idx).double().cpu().numpy()
    ref = O.full_cache_decode(f(k_before), f(v_before), sub_bt, np.full(len(seqs), i), s(q), s(kc), s(vc),
                              page_size=P, rope_base=10000.0)
    err = max_rel_err(out[seqs].float().cpu().numpy(), ref)
    print(f"max_rel_err={err:.3e}")
    assert err < TOL["bf16"]
    assert torch.isfinite(out.float()).all()
