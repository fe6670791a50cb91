"""Parity of the parallel pass (HLA attention at every position of whole
sequences) with the fp64 oracle, through the C ABI.  Every store slot the
call must not read (tokens at or past n_tok - 1 - W, pages nobody owns) and
every q, k, v row at or past n_tok is NaN; the output starts NaN and rows at
or past n_tok must stay NaN."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_cross_loop_amd import binding as B
from synth import gen
from tests.gpu_cases import TOL
from tests.util import max_rel_err

pytestmark = pytest.mark.gpu


def poison(c: gen.ParallelInputs):
    kw = dict(groups=c.groups, page_size=c.page_size, r_k=c.r_k, r_v=c.r_v)
    pages = c.pages.clone()
    flat = pages.view(-1)
    bt = c.block_table.numpy()
    owned = set(bt.ravel().tolist())
    for pg in range(pages.shape[0]):
        if pg not in owned:
            pages[pg] = float("nan")
    for b in range(bt.shape[0]):
        n_lat = max(0, int(c.n_tok[b]) - 1 - c.window)
        j = np.arange(n_lat, bt.shape[1] * c.page_size)
        if j.size == 0:
            continue
        page, slot = bt[b, j // c.page_size].astype(np.int64), j % c.page_size
        for g in range(c.groups):
            ko = O.store_key_offset(page[:, None], g, slot[:, None], np.arange(c.r_k)[None], **kw)
            vo = O.store_value_offset(page[:, None], g, slot[:, None], np.arange(c.r_v)[None], **kw)
            flat[torch.from_numpy(ko.ravel())] = float("nan")
            flat[torch.from_numpy(vo.ravel())] = float("nan")
    q, k, v = c.q.clone(), c.k.clone(), c.v.clone()
    for b in range(q.shape[0]):
        n = int(c.n_tok[b])
        q[b, n:] = k[b, n:] = v[b, n:] = float("nan")
    c.pages, c.q, c.k, c.v = pages, q, k, v
    return c


def run_parallel(c: gen.ParallelInputs, loop=2):
    Bsz, n_max = int(c.q.shape[0]), int(c.q.shape[1])
    print(f"[case] parallel B={Bsz} n_max={n_max} n_tok={c.n_tok.tolist()} H={c.heads} d_h={c.head_dim} "
          f"G={c.groups} r={c.r_k}/{c.r_v} W={c.window} rope={c.rope_base}", flush=True)
    desc = B.set_desc(n_heads=c.heads, head_dim=c.head_dim, groups=c.groups, r_k=c.r_k, r_v=c.r_v,
                      loop_first=1, loop_last=4, page_size=c.page_size, rope_baked=c.rope_baked,
                      rope_base=c.rope_base, dtype=B.LLA_BF16)
    dev = "cuda"
    out = torch.full(tuple(c.q.shape), float("nan"), dtype=torch.bfloat16, device=dev)
    ws = torch.full((B.lla_parallel_workspace_bytes(desc, Bsz, n_max) // 2,), float("nan"), dtype=torch.bfloat16,
                    device=dev)
    st = B.store(c.pages.to(dev), c.block_table.to(dev))
    args = B.parallel_args(loop=loop, window=c.window, n_tok=c.n_tok.to(dev), q=c.q.to(dev), k=c.k.to(dev),
                           v=c.v.to(dev), A=c.A.to(dev), B=c.Bv.transpose(1, 2).contiguous().to(dev), out=out,
                           workspace=ws)
    B.hla_attention_parallel(desc, st, Bsz, args)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def oracle(c: gen.ParallelInputs, rows=None):
    kw = dict(groups=c.groups, page_size=c.page_size, r_k=c.r_k, r_v=c.r_v)
    pages = c.pages.double().numpy()
    bt = c.block_table.numpy()
    sK, sV = [], []
    for b in range(bt.shape[0]):
        n_lat = max(0, int(c.n_tok[b]) - 1 - c.window)
        k_, v_ = O.gather_latents(pages, bt, b, n_lat, **kw)
        sK.append(k_)
        sV.append(v_)
    f = lambda t: t.double().numpy()
    return O.parallel_attention(sK, sV, c.n_tok.numpy(), f(c.q), f(c.k), f(c.v), f(c.A), f(c.Bv),
                                window=c.window, rope_base=c.rope_base, rows=rows)


def check(c, **kw):
    c = poison(c)
    out = run_parallel(c, **kw)
    ref = oracle(c)
    for b in range(out.shape[0]):
        n = int(c.n_tok[b])
        if n:
            err = max_rel_err(out[b, :n], ref[b, :n])
            print(f"  seq {b}: max_rel_err={err:.3e}")
            assert err < TOL["bf16"], (b, err)
        assert np.isnan(out[b, n:]).all(), b
    return out


def test_parallel_hla_main_set_shape():
    """16 heads x 128, r = 512 (m = 4 rotary blocks), W = 16: two sequences,
    the longer one spanning two query tiles."""
    c = gen.parallel_inputs(900, batch=2, heads=16, head_dim=128, groups=1, r_k=512, r_v=512, n_max=300,
                            n_tok=(300, 129), window=16, rope_base=10000.0)
    check(c)


def test_parallel_window_128_band_tiles():
    """W = 128 as in the HLA set: the exact band spans several key tiles and
    three query tiles."""
    c = gen.parallel_inputs(901, batch=1, heads=16, head_dim=128, groups=1, r_k=512, r_v=512, n_max=700,
                            n_tok=(700,), window=128, rope_base=10000.0)
    check(c)


def test_parallel_loop1_width_and_odd_lengths():
    """r = 256 (the loop-1 set), lengths around tile and page edges."""
    c = gen.parallel_inputs(902, batch=4, heads=16, head_dim=128, groups=1, r_k=256, r_v=256, n_max=320,
                            n_tok=(64, 65, 257, 320), window=31, rope_base=10000.0)
    check(c, loop=1)


@pytest.mark.parametrize("rope", [0.0, 500.0])
def test_parallel_head_dim_64_groups(rope):
    """d_h = 64, two latent groups of 4 heads, ragged lengths including 1."""
    c = gen.parallel_inputs(903, batch=3, heads=8, head_dim=64, groups=2, r_k=128, r_v=64, n_max=260,
                            n_tok=(77, 1, 260), window=5, rope_base=rope)
    check(c)


def test_parallel_dense_decoders_without_rotation():
    """Dense (not frequency-paired) key decoders, no rotary embedding, W = 0
    (only the token itself is exact)."""
    c = gen.parallel_inputs(904, batch=2, heads=4, head_dim=128, groups=1, r_k=96, r_v=160, n_max=200,
                            n_tok=(200, 150), window=0, rope_base=0.0, paired=False)
    check(c)


def test_parallel_window_covers_sequence_and_empty_sequence():
    """W >= n - 1: no latent is read (the whole store is NaN); an empty
    sequence writes nothing."""
    c = gen.parallel_inputs(905, batch=3, heads=16, head_dim=128, groups=1, r_k=512, r_v=512, n_max=100,
                            n_tok=(100, 0, 37), window=99, rope_base=10000.0)
    c.pages[:] = float("nan")
    check(c)


def test_parallel_full_size_sampled():
    """8 sequences of 2048 positions (the pages' phase-1 sequence length) on
    the main-set shape, W = 128; the oracle checks sampled positions."""
    Bsz, n, H, dh, r, W, P = 8, 2048, 16, 128, 512, 128, 64
    g = gen.rng(910)
    bt, n_pages = gen.block_table(g, Bsz, n // P, 2)
    pages = gen.device_normal((n_pages, P * 2 * r), "bf16", 911)
    q = gen.device_normal((Bsz, n, H, dh), "bf16", 912)
    k = gen.device_normal((Bsz, n, H, dh), "bf16", 913)
    v = gen.device_normal((Bsz, n, H, dh), "bf16", 914)
    A = gen.as_stored(gen.frequency_paired_decoder(g, H, dh, r), "bf16")
    Bv = gen.as_stored(np.stack([gen.gaussian_orthonormal(g, r, dh) for _ in range(H)]), "bf16")
    n_tok = torch.full((Bsz,), n, dtype=torch.int32)
    desc = B.set_desc(n_heads=H, head_dim=dh, groups=1, r_k=r, r_v=r, loop_first=2, loop_last=4, page_size=P,
                      rope_baked=1, rope_base=10000.0, dtype=B.LLA_BF16)
    out = torch.full((Bsz, n, H, dh), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(B.lla_parallel_workspace_bytes(desc, Bsz, n), dtype=torch.uint8, device="cuda")
    print(f"[case] parallel full size B={Bsz} n={n}", flush=True)
    B.hla_attention_parallel(desc, B.store(pages, torch.from_numpy(bt).cuda()), Bsz,
                             B.parallel_args(loop=3, window=W, n_tok=n_tok.cuda(), q=q, k=k, v=v, A=A.cuda(),
                                             B=Bv.transpose(1, 2).contiguous().cuda(), out=out, workspace=ws))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    c = gen.ParallelInputs(heads=H, head_dim=dh, groups=1, r_k=r, r_v=r, page_size=P, window=W,
                           rope_base=10000.0, rope_baked=1, pages=pages.cpu(), block_table=torch.from_numpy(bt),
                           n_tok=n_tok, q=q.cpu(), k=k.cpu(), v=v.cpu(), A=A, Bv=Bv)
    rows = [(0, 0), (0, 128), (0, 129), (0, 130), (3, 255), (3, 256), (5, 1000), (7, 2046), (7, 2047)]
    ref = oracle(c, rows=rows)
    got = out.float().cpu().numpy()
    err = max(max_rel_err(got[b, i], ref[b, i]) for b, i in rows)
    print(f"max_rel_err={err:.3e}")
    assert err < TOL["bf16"]
