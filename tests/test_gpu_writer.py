"""Parity of the latent writer (Eq. 2 of the Hybrid Latent Attention summary)
with the fp64 oracle, through the C ABI, and writer -> decode end to end."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_cross_loop_amd import binding as B
from synth import gen
from tests.gpu_cases import TOL
from tests.util import max_rel_err

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def run_writer(*, batch, n_tok, n_loops, groups, r_k, r_v, d_in, dtype, positions, head_dim=128,
               rope_base=0.0, rope_baked=0, page_size=64, seed=0, max_pos=None):
    print(f"[case] writer B={batch} n_tok={n_tok} loops={n_loops} G={groups} r={r_k}/{r_v} "
          f"d_in={d_in} dtype={dtype} rope={rope_base}", flush=True)
    wi = gen.writer_inputs(seed, batch=batch, n_tok=n_tok, n_loops=n_loops, groups=groups, r_k=r_k,
                           r_v=r_v, d_in=d_in, dtype=dtype, positions=positions)
    max_pos = int(np.max(positions)) if max_pos is None else max_pos
    pps = -(-(max_pos + 1) // page_size)
    bt, n_pages = gen.block_table(gen.rng(seed, 5), batch, pps, 2)
    dt = gen.TORCH_DTYPE[dtype]
    pages = torch.full((n_pages, groups * page_size * (r_k + r_v)), SENTINEL, dtype=dt, device="cuda")
    bt_d = torch.from_numpy(bt).cuda()
    desc = B.set_desc(n_heads=groups, head_dim=head_dim, groups=groups, r_k=r_k, r_v=r_v,
                      loop_first=1, loop_last=n_loops, page_size=page_size, rope_baked=rope_baked,
                      rope_base=rope_base, dtype=B.LLA_BF16 if dtype == "bf16" else B.LLA_F32)
    nbytes = B.lla_write_workspace_bytes(desc, batch, n_tok, d_in)
    ws = torch.full((max(nbytes, 4) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    B.lla_write_latents(desc, B.store(pages, bt_d), pos=wi.pos.cuda(), x=wi.x.cuda(),
                        enc=wi.enc.cuda(), workspace=ws)
    torch.cuda.synchronize()
    want = O.write_latents(wi.x.double().numpy(), wi.enc.double().numpy(), wi.pos.numpy(), r_k=r_k,
                           rope_base=rope_base, rope_baked=rope_baked, head_dim=head_dim)
    got_pages = pages.double().cpu().numpy()
    kw = dict(groups=groups, page_size=page_size, r_k=r_k, r_v=r_v)
    touched = np.zeros(got_pages.size, dtype=bool)
    got = np.zeros_like(want)
    for b in range(batch):
        for n in range(n_tok):
            p = int(wi.pos[b, n])
            pg, sl = int(bt[b, p // page_size]), p % page_size
            for g in range(groups):
                ko = O.store_key_offset(pg, g, sl, np.arange(r_k), **kw)
                vo = O.store_value_offset(pg, g, sl, np.arange(r_v), **kw)
                got[b, n, g] = np.concatenate([got_pages.ravel()[ko], got_pages.ravel()[vo]])
                touched[ko] = touched[vo] = True
    # nothing outside the written slots changed
    assert np.all(got_pages.ravel()[~touched] == SENTINEL)
    return got, want


@pytest.mark.parametrize("set_key", [0, 1])
def test_writer_fp32_tiny(set_key):
    """Workload 1 shapes: loop-1 set (r_1 = 32) and main set (128 + 128), d = 128."""
    n_loops, r = (1, 32) if set_key == 0 else (3, 128)
    got, want = run_writer(batch=1, n_tok=5, n_loops=n_loops, groups=1, r_k=r, r_v=r, d_in=128,
                           dtype="f32", positions=[[0, 17, 100, 254, 255]], head_dim=64, seed=3)
    assert max_rel_err(got, want) < 1e-5


def test_writer_bf16_hla_rope_baked():
    """Main HLA set at the Ouro-1.4B shape: 3 loops x d = 2048 -> 512 + 512, RoPE baked."""
    got, want = run_writer(batch=3, n_tok=2, n_loops=3, groups=1, r_k=512, r_v=512, d_in=2048,
                           dtype="bf16", positions=[[5, 4095], [1000, 77], [64, 63]],
                           rope_base=10000.0, rope_baked=1, seed=4)
    assert max_rel_err(got, want) < TOL["bf16"]


def test_writer_bf16_per_head():
    """Per-head LLA set: 16 groups, [k; v] of 256 per loop -> 32 + 32, 4 loops."""
    got, want = run_writer(batch=2, n_tok=3, n_loops=4, groups=16, r_k=32, r_v=32, d_in=256,
                           dtype="bf16", positions=[[0, 1, 2], [300, 301, 302]], seed=5)
    assert max_rel_err(got, want) < TOL["bf16"]


def test_writer_bf16_generic_path():
    """d_in not a multiple of 32 takes the general kernel."""
    got, want = run_writer(batch=2, n_tok=2, n_loops=2, groups=2, r_k=64, r_v=48, d_in=48,
                           dtype="bf16", positions=[[3, 9], [70, 71]], head_dim=64,
                           rope_base=10000.0, rope_baked=1, seed=6)
    assert max_rel_err(got, want) < TOL["bf16"]


def test_writer_then_decode_end_to_end():
    """GPU writer fills the whole store, GPU decode reads it; the oracle writes
    fp64 latents and decodes them.  Same seeded inputs on both sides."""
    H, dh, r, W, n_loops, d_in, P = 16, 128, 256, 8, 3, 256, 64
    N = 150
    Bsz = 2
    base = 10000.0
    wi = gen.writer_inputs(7, batch=Bsz, n_tok=N, n_loops=n_loops, groups=1, r_k=r, r_v=r, d_in=d_in,
                           dtype="bf16", positions=np.tile(np.arange(N), (Bsz, 1)), enc_scale=1.0)
    dc = gen.decode_inputs(8, batch=Bsz, heads=H, head_dim=dh, groups=1, r_k=r, r_v=r,
                           positions=[N - 1, N - 1], window=W, dtype="bf16", page_size=P,
                           rope_base=base, rope_baked=1, loop=3, loop_first=2, loop_last=4,
                           exact_std=np.sqrt(3.0))
    desc = B.set_desc(n_heads=H, head_dim=dh, groups=1, r_k=r, r_v=r, loop_first=2, loop_last=4,
                      page_size=P, rope_baked=1, rope_base=base, dtype=B.LLA_BF16)
    pages = torch.full(tuple(dc.pages.shape), float("nan"), dtype=torch.bfloat16, device="cuda")
    bt = dc.block_table.cuda()
    st = B.store(pages, bt)
    ws = torch.empty(max(B.lla_write_workspace_bytes(desc, Bsz, N, d_in), 4), dtype=torch.uint8,
                     device="cuda")
    B.lla_write_latents(desc, st, pos=wi.pos.cuda(), x=wi.x.cuda(), enc=wi.enc.cuda(), workspace=ws)
    out = torch.empty(tuple(dc.q.shape), dtype=torch.bfloat16, device="cuda")
    dws = torch.empty(B.lla_decode_workspace_bytes(desc, Bsz, N - 1, W), dtype=torch.uint8, device="cuda")
    rk, rv = dc.ring_k.cuda(), dc.ring_v.cuda()
    args = B.decode_args(loop=3, window=W, pos=dc.pos.cuda(), q=dc.q.cuda(), k_cur=dc.k_cur.cuda(),
                         v_cur=dc.v_cur.cuda(), ring_k=rk, ring_v=rv, A=dc.A.cuda(), B=dc.Bv.transpose(1, 2).contiguous().cuda(),
                         out=out, workspace=dws, max_pos_hint=N - 1)
    B.hla_decode_windowed(desc, st, Bsz, args)
    torch.cuda.synchronize()
    c = O.write_latents(wi.x.double().numpy(), wi.enc.double().numpy(), wi.pos.numpy(), r_k=r,
                        rope_base=base, rope_baked=1, head_dim=dh)
    sK = [c[b, :, :, :r] for b in range(Bsz)]
    sV = [c[b, :, :, r:] for b in range(Bsz)]
    f = [t.double().numpy() for t in (dc.q, dc.k_cur, dc.v_cur, dc.ring_k, dc.ring_v, dc.A, dc.Bv)]
    ref = O.absorbed_decode(sK, sV, dc.pos.numpy(), *f, window=W, rope_base=base)
    ref_t = O.textbook_decode(sK, sV, dc.pos.numpy(), *f, window=W, rope_base=base)
    assert max_rel_err(ref, ref_t) < 1e-10
    assert max_rel_err(out.float().cpu().numpy(), ref) < TOL["bf16"]


@pytest.mark.parametrize("case", [
    # decode shape of the main HLA set: 128 tokens, 3 loops x 2048 -> 512 + 512, 16 K splits
    dict(batch=128, n_tok=1, n_loops=3, groups=1, r_k=512, r_v=512, d_in=2048, rope_base=10000.0,
         rope_baked=1, head_dim=128, positions="decode"),
    # 150 tokens (second 128-token tile ragged), R = 80 (64-wide output tile ragged), 2 groups
    dict(batch=3, n_tok=50, n_loops=2, groups=2, r_k=48, r_v=32, d_in=64, head_dim=64,
         positions="prefix"),
    # 256 output tiles -> one K split of 16 steps: two rounds, the second ragged
    dict(batch=1, n_tok=2, n_loops=1, groups=1, r_k=8192, r_v=8192, d_in=512, rope_base=500.0,
         rope_baked=1, head_dim=128, positions="prefix"),
    # tiny output, long K: 64 K splits, summed in eight batches of eight
    dict(batch=2, n_tok=1, n_loops=4, groups=1, r_k=32, r_v=32, d_in=4096, head_dim=64,
         positions="decode"),
    # bulk writes (1024 tokens or more) take the tiled GEMM: 1200 tokens (last
    # 128-token tile ragged), R = 80 (one ragged 128-wide tile), 2 groups, 2 loops
    dict(batch=3, n_tok=400, n_loops=2, groups=2, r_k=48, r_v=32, d_in=64, head_dim=64,
         positions="prefix"),
    # bulk write of the main HLA set with baked rotary embedding, 3 K segments
    dict(batch=2, n_tok=600, n_loops=3, groups=1, r_k=512, r_v=512, d_in=2048, rope_base=10000.0,
         rope_baked=1, head_dim=128, positions="prefix"),
], ids=["hla-decode-b128", "ragged-m-and-n", "two-rounds", "many-splits", "bulk-ragged",
        "bulk-hla"])
def test_writer_bf16_shapes(case):
    case = dict(case)
    kind = case.pop("positions")
    Bsz, n_tok = case["batch"], case["n_tok"]
    if kind == "decode":
        positions = gen.rng(11, 1).integers(0, 4096, size=(Bsz, 1))
    else:
        positions = np.tile(np.arange(n_tok), (Bsz, 1)) + 7 * np.arange(Bsz)[:, None]
    got, want = run_writer(dtype="bf16", positions=positions, seed=12, **case)
    assert max_rel_err(got, want) < TOL["bf16"]


def test_writer_lla2d_decode_shape():
    """The writer call the bench times on workload 5: 64 tokens (one per
    sequence, at positions anywhere in a 4k context), 32 loops x d_in 10560 ->
    5280 + 5280, one group; K = 32 x 10560 is cut into many splits of several
    rounds each.  Encoders and inputs are drawn on the device (E_t entries
    N(0, 1/d_in), x ~ N(0, 1), as the bench draws them); four sampled tokens
    are checked in full (all 10560 latent dims) against the oracle's Eq. 2, in
    chunks of encoder rows, and every other store element keeps its NaN."""
    from synth import configs
    w = configs.get(5)
    s = w.sets[0]
    Bsz, R, P = w.batch, s.r_k + s.r_v, w.page_size
    print(f"[case] writer workload 5 B={Bsz} loops={s.n_loops} d_in={s.d_in} R={R}", flush=True)
    enc = gen.device_normal((s.n_loops, 1, R, s.d_in), "bf16", 501, 1.0 / np.sqrt(s.d_in))
    x = gen.device_normal((Bsz, 1, s.n_loops, 1, s.d_in), "bf16", 502)
    positions = gen.rng(13, 1).integers(0, w.context, size=(Bsz, 1)).astype(np.int32)
    pps = -(-w.context // P)
    bt, n_pages = gen.block_table(gen.rng(13, 2), Bsz, pps, 2)
    pages = torch.full((n_pages, P * R), float("nan"), dtype=torch.bfloat16, device="cuda")
    desc = B.set_desc(n_heads=w.heads, head_dim=w.head_dim, groups=1, r_k=s.r_k, r_v=s.r_v, loop_first=1,
                      loop_last=s.n_loops, page_size=P, rope_baked=0, rope_base=0.0, dtype=B.LLA_BF16)
    nbytes = B.lla_write_workspace_bytes(desc, Bsz, 1, s.d_in)
    ws = torch.full((max(nbytes, 4) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    B.lla_write_latents(desc, B.store(pages, torch.from_numpy(bt).cuda()), pos=torch.from_numpy(positions).cuda(),
                        x=x, enc=enc, workspace=ws)
    torch.cuda.synchronize()
    # nothing but the 64 written rows changed
    assert int((~torch.isnan(pages)).sum()) == Bsz * R
    kw = dict(groups=1, page_size=P, r_k=s.r_k, r_v=s.r_v)
    flat = pages.view(-1)
    seqs = [0, 21, 42, 63]
    got = []
    for b in seqs:
        p = int(positions[b, 0])
        pg, sl = int(bt[b, p // P]), p % P
        ko = O.store_key_offset(pg, 0, sl, np.arange(s.r_k), **kw)
        vo = O.store_value_offset(pg, 0, sl, np.arange(s.r_v), **kw)
        got.append(flat[torch.from_numpy(np.concatenate([ko, vo])).cuda()].double().cpu().numpy())
    xs = x[seqs].double().cpu().numpy()
    want = np.concatenate([
        O.write_latents(xs, enc[:, :, r0:r0 + 1056].double().cpu().numpy(), positions[seqs], r_k=1056)[:, 0, 0]
        for r0 in range(0, R, 1056)], axis=-1)
    err = max_rel_err(np.stack(got), want)
    print(f"max_rel_err={err:.3e}", flush=True)
    assert err < TOL["bf16"]


@pytest.mark.parametrize("loop", [1, 2, 3, 4])
def test_tiny_fp32_writer_then_decode(loop):
    """Workload 1 end to end in fp32: h_j,t ~ N(0, 1) for every token and loop,
    E_t, A_t, B_t Gaussian-QR x 1/sqrt(d_h); the GPU writer fills both sets of
    the layer (loop 1: r_1 = 32; loops 2..4: 128 + 128) at positions 0..255, then
    the decode at i = 255 with W = 16 runs through every entry point that
    reads the loop's set (hla_decode_windowed, lla_decode_absorbed,
    lla_decode_reconstruct).  Exact window / current K and V ~ N(0, sigma^2),
    sigma the RMS of the latent keys the loop's decoder rebuilds.  The oracle
    writes its own fp64 latents from the same inputs; tolerance 1e-5."""
    from synth import configs
    w = configs.get(1)
    H, dh, W, P, N = w.heads, w.head_dim, w.window, w.page_size, w.context
    i = N - 1
    sc = 1.0 / np.sqrt(dh)
    k = w.set_for_loop(loop)
    s = w.sets[k]
    g = gen.rng(40 + loop)
    h = g.standard_normal((1, N, w.loops, 1, w.d_model))
    x = h[:, :, s.loop_first - 1:s.loop_last]                    # this set's loops
    enc = np.stack([gen.gaussian_orthonormal(g, s.r_k + s.r_v, s.d_in, sc)[None] for _ in range(s.n_loops)])
    A = np.stack([gen.gaussian_orthonormal(g, dh, s.r_k, sc) for _ in range(H)])
    Bv = np.stack([gen.gaussian_orthonormal(g, s.r_v, dh, sc) for _ in range(H)])
    q = g.standard_normal((1, H, dh))
    pos = np.arange(N)[None]
    lat = O.write_latents(x, enc, pos, r_k=s.r_k)[0]              # [N, 1, r_k + r_v] fp64
    sigma = float(np.sqrt(np.mean(np.einsum("hdr,nr->nhd", A, lat[:, 0, :s.r_k]) ** 2)))
    kc, vc = (g.standard_normal((1, H, dh)) * sigma for _ in range(2))
    ring_k, ring_v = (g.standard_normal((1, W + 1, H, dh)) * sigma for _ in range(2))
    pps = -(-N // P)
    bt, n_pages = gen.block_table(g, 1, pps, 1)
    desc = B.set_desc(n_heads=H, head_dim=dh, groups=1, r_k=s.r_k, r_v=s.r_v, loop_first=s.loop_first,
                      loop_last=s.loop_last, page_size=P, rope_baked=0, rope_base=0.0, dtype=B.LLA_F32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).float().cuda()
    pages = torch.full((n_pages, P * (s.r_k + s.r_v)), float("nan"), dtype=torch.float32, device="cuda")
    st = B.store(pages, torch.from_numpy(bt).cuda())
    ws = torch.empty(max(B.lla_write_workspace_bytes(desc, 1, N, s.d_in), 4), dtype=torch.uint8, device="cuda")
    B.lla_write_latents(desc, st, pos=torch.from_numpy(pos.astype(np.int32)).cuda(), x=dev(x), enc=dev(enc),
                        workspace=ws)
    sK, sV = [lat[:i - W, :, :s.r_k]], [lat[:i - W, :, s.r_k:]]
    ref = {f: fn(sK, sV, [i], q, kc, vc, ring_k, ring_v, A, Bv, window=W, rope_base=0.0)
           for f, fn in (("absorbed", O.absorbed_decode), ("textbook", O.textbook_decode))}
    entries = [("absorbed", "absorbed"), ("reconstruct", "textbook"), ("hla", "absorbed")]
    for entry, form in entries:
        print(f"[case] workload 1 writer -> {entry} loop={loop}", flush=True)
        out = torch.full((1, H, dh), float("nan"), dtype=torch.float32, device="cuda")
        dws = torch.full((B.lla_decode_workspace_bytes(desc, 1, i, W) // 4,), float("nan"), device="cuda")
        args = B.decode_args(loop=loop, window=W, pos=torch.tensor([i], dtype=torch.int32, device="cuda"),
                             q=dev(q), k_cur=dev(kc), v_cur=dev(vc), ring_k=dev(ring_k), ring_v=dev(ring_v),
                             A=dev(A), B=dev(Bv.transpose(0, 2, 1)), out=out, workspace=dws, max_pos_hint=i)
        {"absorbed": B.lla_decode_absorbed, "reconstruct": B.lla_decode_reconstruct,
         "hla": B.hla_decode_windowed}[entry](desc, st, 1, args)
        torch.cuda.synchronize()
        err = max_rel_err(out.cpu().numpy(), ref[form])
        print(f"max_rel_err={err:.3e}", flush=True)
        assert err < TOL["f32"]
