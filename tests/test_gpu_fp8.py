"""fp8 (OCP e4m3 + per-token scale) latent storage on the GPU: the absorbed /
HLA decode reading an fp8 store, against the fp64 oracle on the same bytes,
and the writer's quantization, against the oracle's quantizer.

The store content is drawn directly as codes and scales (synth), laid out with
the oracle's offset functions; every slot the call must not read holds NaN
codes and NaN scales."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_cross_loop_amd import binding as B
from synth import gen
from tests.gpu_cases import TOL, ENTRY, poison_unread
from tests.util import max_rel_err

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F


def fp8_store_bytes(codes, scales, bt, positions, window, *, groups, page_size, r_k, r_v, chunk=256):
    """Lay codes / scales into the fp8 page bytes with the oracle's offset
    functions; tokens a call must not read (at or past max(0, i-W) of their
    sequence, and pages nobody owns) get NaN codes and NaN scales.  Works over
    `chunk` pages at a time to bound host memory at full size."""
    n_pages = codes.shape[0]
    kw = dict(groups=groups, page_size=page_size, r_k=r_k, r_v=r_v)
    raw = np.zeros(n_pages * groups * (page_size // 16) * O.fp8_tile_bytes(r_k, r_v), dtype=np.uint8)
    readable = np.zeros((n_pages, page_size), dtype=bool)
    for b, i in enumerate(positions):
        n_lat = max(0, int(i) - window)
        j = np.arange(n_lat)
        readable[bt[b, j // page_size], j % page_size] = True
    for p0 in range(0, n_pages, chunk):
        p1 = min(n_pages, p0 + chunk)
        pg, sl = np.meshgrid(np.arange(p0, p1), np.arange(page_size), indexing="ij")
        rd = readable[p0:p1]
        for g in range(groups):
            c = codes[p0:p1, g].copy()
            s = scales[p0:p1, g].astype(np.float32)
            c[~rd] = NAN_CODE
            s[~rd] = np.nan
            raw[O.fp8_key_offset(pg[..., None], g, sl[..., None], np.arange(r_k), **kw)] = c[..., :r_k]
            raw[O.fp8_value_offset(pg[..., None], g, sl[..., None], np.arange(r_v), **kw)] = c[..., r_k:]
            for part in (0, 1):
                off = O.fp8_scale_offset(pg, g, sl, part, **kw)
                sb = np.ascontiguousarray(s[..., part]).view(np.uint8).reshape(off.shape + (4,))
                raw[off[..., None] + np.arange(4)] = sb
    return raw


def fp8_case(seed, *, r, positions, W, H=16, d_h=128, G=1, P=64, rope=True, loop=2):
    c = gen.decode_inputs(seed, batch=len(positions), heads=H, head_dim=d_h, groups=G, r_k=r, r_v=r,
                          positions=positions, window=W, dtype="bf16", page_size=P,
                          rope_base=10000.0 if rope else 0.0, rope_baked=1 if rope else 0, loop=loop,
                          loop_first=1, loop_last=4, paired=rope, exact_std=1.0)
    codes, scales = gen.fp8_latent_draws(seed, n_pages=c.n_pages, groups=G, page_size=P, r_k=r, r_v=r)
    raw = fp8_store_bytes(codes, scales, c.block_table.numpy(), c.pos.numpy(), W, groups=G, page_size=P,
                          r_k=r, r_v=r)
    return poison_unread(c), raw


def run_fp8(entry, c, raw, *, splits=0, flags=0):
    dev = "cuda"
    desc = B.set_desc(n_heads=c.heads, head_dim=c.head_dim, groups=c.groups, r_k=c.r_k, r_v=c.r_v,
                      loop_first=c.loop_first, loop_last=c.loop_last, page_size=c.page_size,
                      rope_baked=c.rope_baked, rope_base=c.rope_base, dtype=B.LLA_BF16, latent_fp8=1)
    print(f"[case] fp8 entry={entry} B={c.batch} H={c.heads} G={c.groups} r={c.r_k} W={c.window} "
          f"pos={c.pos.tolist()} splits={splits} flags={flags}", flush=True)
    pages = torch.from_numpy(raw).to(dev)
    out = torch.full(tuple(c.q.shape), float("nan"), dtype=torch.bfloat16, device=dev)
    mp = int(c.pos.max())
    ws = torch.full((B.lla_decode_workspace_bytes(desc, c.batch, mp, c.window, splits) // 4,), float("nan"),
                    dtype=torch.float32, device=dev)
    rk, rv = c.ring_k.to(dev), c.ring_v.to(dev)
    args = B.decode_args(loop=c.loop, window=c.window, pos=c.pos.to(dev), q=c.q.to(dev), k_cur=c.k_cur.to(dev),
                         v_cur=c.v_cur.to(dev), ring_k=rk, ring_v=rv, A=c.A.to(dev),
                         B=c.Bv.transpose(1, 2).contiguous().to(dev), out=out, workspace=ws, max_pos_hint=mp,
                         splits=splits, flags=flags)
    ENTRY[entry](desc, B.store(pages, c.block_table.to(dev)), c.batch, args)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def oracle_fp8(c, raw, form="absorbed"):
    kw = dict(groups=c.groups, page_size=c.page_size, r_k=c.r_k, r_v=c.r_v)
    sK, sV = [], []
    for b in range(c.batch):
        n_lat = max(0, int(c.pos[b]) - c.window)
        k, v = O.gather_latents_fp8(raw, c.block_table.numpy(), b, n_lat, **kw)
        sK.append(k)
        sV.append(v)
    fn = O.textbook_decode if form == "textbook" else O.absorbed_decode
    args = [t.double().numpy() for t in (c.q, c.k_cur, c.v_cur, c.ring_k, c.ring_v, c.A, c.Bv)]
    return fn(sK, sV, c.pos.numpy(), *args, window=c.window, rope_base=c.rope_base)


@pytest.mark.parametrize("r", [512, 256])
@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("generic", [False, True])
def test_fp8_hla_decode(r, splits, generic):
    c, raw = fp8_case(800 + r + splits, r=r, positions=(300, 37, 129, 1000), W=16)
    out = run_fp8("hla", c, raw, splits=splits, flags=1 if generic else 0)
    ref = oracle_fp8(c, raw)
    err = max_rel_err(out, ref)
    assert err < TOL["bf16"], err
    # the absorbed and textbook forms agree on the fp8 store too
    assert max_rel_err(oracle_fp8(c, raw, "textbook"), ref) < 1e-10


@pytest.mark.parametrize("r, d_h, H, G", [(64, 64, 4, 1), (128, 64, 8, 2), (64, 128, 6, 3)])
def test_fp8_absorbed_widths_and_groups(r, d_h, H, G):
    """Narrow latents, grouped heads, ragged tiles, no rotary (LLA-D style)."""
    c, raw = fp8_case(820 + r + d_h + H, r=r, positions=(613, 66, 9, 16), W=5, H=H, d_h=d_h, G=G,
                      rope=False, loop=3)
    err = max_rel_err(run_fp8("absorbed", c, raw, splits=2), oracle_fp8(c, raw))
    assert err < TOL["bf16"], err


def test_fp8_edges_and_window_slices():
    """First token, window covering the context, tile and page edges, W = 128
    over several slices."""
    c, raw = fp8_case(840, r=512, positions=(0, 5, 16, 17, 63, 64, 65, 4095), W=128)
    err = max_rel_err(run_fp8("hla", c, raw), oracle_fp8(c, raw))
    assert err < TOL["bf16"], err


def _run_writer_fp8(*, batch, n_tok, n_loops, r, d_in, positions, rope, seed, d_h=128):
    wi = gen.writer_inputs(seed, batch=batch, n_tok=n_tok, n_loops=n_loops, groups=1, r_k=r, r_v=r, d_in=d_in,
                           dtype="bf16", positions=positions)
    P = 64
    pps = int(np.max(positions)) // P + 1
    bt, n_pages = gen.block_table(gen.rng(seed, 5), batch, pps, 2)
    desc = B.set_desc(n_heads=1, head_dim=d_h, groups=1, r_k=r, r_v=r, loop_first=1, loop_last=n_loops,
                      page_size=P, rope_baked=1 if rope else 0, rope_base=10000.0 if rope else 0.0,
                      dtype=B.LLA_BF16, latent_fp8=1)
    print(f"[case] fp8 writer B={batch} n_tok={n_tok} loops={n_loops} r={r} d_in={d_in} rope={rope}", flush=True)
    pages = torch.full((B.store_bytes(desc, n_pages),), 0xAB, dtype=torch.uint8, device="cuda")
    ws = torch.full((max(4, B.lla_write_workspace_bytes(desc, batch, n_tok, d_in)) // 4,), float("nan"),
                    dtype=torch.float32, device="cuda")
    B.lla_write_latents(desc, B.store(pages, torch.from_numpy(bt).cuda()), pos=wi.pos.cuda(), x=wi.x.cuda(),
                        enc=wi.enc.cuda(), workspace=ws)
    torch.cuda.synchronize()
    raw = pages.cpu().numpy()
    c = O.write_latents(wi.x.double().numpy(), wi.enc.double().numpy(), wi.pos.numpy(), r_k=r,
                        rope_base=10000.0 if rope else 0.0, rope_baked=1 if rope else 0, head_dim=d_h)
    kw = dict(groups=1, page_size=P, r_k=r, r_v=r)
    touched = np.zeros(raw.size, dtype=bool)
    n_near = 0
    for b in range(batch):
        for n in range(n_tok):
            p = int(wi.pos[b, n])
            pg, sl = int(bt[b, p // P]), p % P
            for part, lo, hi, off_fn in ((0, 0, r, O.fp8_key_offset), (1, r, 2 * r, O.fp8_value_offset)):
                offs = off_fn(pg, 0, sl, np.arange(r), **kw)
                so = int(O.fp8_scale_offset(pg, 0, sl, part, **kw))
                touched[offs] = True
                touched[so:so + 4] = True
                got_codes = raw[offs]
                got_scale = float(raw[so:so + 4].view(np.float32)[0])
                want_codes, want_scale = O.fp8_quantize_rows(c[b, n, 0, lo:hi])
                # the scale: max |x| / 448 of an fp32 accumulation
                assert abs(got_scale - want_scale) <= 1e-5 * want_scale
                # codes: equal, except where the oracle's x / scale lies
                # within the fp32 accumulation's reach of a rounding tie (the
                # two roundings are one grid step apart there).  The kernel's
                # c carries an error below 1e-5 max|c|, i.e. below 448e-5 in
                # x / scale, plus a relative 1e-5 through the scale.
                y = np.abs(c[b, n, 0, lo:hi] / want_scale)
                step = 2.0 ** (np.clip(np.floor(np.log2(np.maximum(y, 2.0 ** -9))), -6, 8) - 3)
                tie = (np.floor(y / step) + 0.5) * step
                near = np.abs(y - tie) < 448e-5 + 1e-5 * y
                n_near += int(near.sum())
                np.testing.assert_array_equal(got_codes[~near], want_codes[~near])
                d = np.abs(O.e4m3_decode(got_codes[near]) - O.e4m3_decode(want_codes[near]))
                assert np.all(d <= step[near] * 1.0001)
    # nothing outside the written codes and scales changed
    assert np.all(raw[~touched] == 0xAB)
    return n_near


@pytest.mark.parametrize("rope", [True, False])
def test_fp8_writer_hla_shape(rope):
    """Main HLA set at the Ouro-1.4B shape: 3 loops x 2048 -> 512 + 512 codes per token."""
    _run_writer_fp8(batch=4, n_tok=2, n_loops=3, r=512, d_in=2048, positions=[[5, 4095], [1000, 77], [64, 63],
                                                                            [0, 1]], rope=rope, seed=850)


def test_fp8_writer_generic_and_decode_shapes():
    """d_in not a multiple of 32 takes the general writer; the loop-1 width."""
    _run_writer_fp8(batch=2, n_tok=3, n_loops=1, r=256, d_in=48, positions=[[3, 9, 200], [70, 71, 72]],
                    rope=True, seed=851)


def test_fp8_full_size_hla_sampled():
    """Batch 128 at context 4096 on an fp8 main-set store, automatic plan;
    the oracle checks three sequences."""
    Bsz, H, dh, r, W, P, i = 128, 16, 128, 512, 128, 64, 4095
    g = gen.rng(860)
    pps = i // P + 1
    bt, n_pages = gen.block_table(g, Bsz, pps, 2)
    codes, scales = gen.fp8_latent_draws(860, n_pages=n_pages, groups=1, page_size=P, r_k=r, r_v=r)
    pos = np.full(Bsz, i)
    raw = fp8_store_bytes(codes, scales, bt, pos, W, groups=1, page_size=P, r_k=r, r_v=r)
    A = gen.frequency_paired_decoder(g, H, dh, r, 1.0)
    Bv = np.stack([gen.gaussian_orthonormal(g, r, dh) for _ in range(H)])
    q = g.standard_normal((Bsz, H, dh))
    kc, vc = g.standard_normal((Bsz, H, dh)), g.standard_normal((Bsz, H, dh))
    rk, rv = g.standard_normal((Bsz, W + 1, H, dh)), g.standard_normal((Bsz, W + 1, H, dh))
    t = lambda a: gen.as_stored(a, "bf16")
    c = gen.DecodeInputs(heads=H, head_dim=dh, groups=1, r_k=r, r_v=r, page_size=P, window=W, loop=3,
                         loop_first=2, loop_last=4, rope_base=10000.0, rope_baked=1, dtype="bf16",
                         pages=None, block_table=torch.from_numpy(bt), pos=torch.from_numpy(pos.astype(np.int32)),
                         q=t(q), k_cur=t(kc), v_cur=t(vc), ring_k=t(rk), ring_v=t(rv), A=t(A), Bv=t(Bv))
    out = run_fp8("hla", c, raw)
    seqs = [0, 63, 127]
    sub = gen.DecodeInputs(heads=H, head_dim=dh, groups=1, r_k=r, r_v=r, page_size=P, window=W, loop=3,
                           loop_first=2, loop_last=4, rope_base=10000.0, rope_baked=1, dtype="bf16", pages=None,
                           block_table=torch.from_numpy(bt[seqs]), pos=torch.from_numpy(pos[seqs].astype(np.int32)),
                           q=c.q[seqs], k_cur=c.k_cur[seqs], v_cur=c.v_cur[seqs], ring_k=c.ring_k[seqs],
                           ring_v=c.ring_v[seqs], A=c.A, Bv=c.Bv)
    err = max_rel_err(out[seqs], oracle_fp8(sub, raw))
    print(f"max_rel_err={err:.3e}")
    assert err < TOL["bf16"]


def test_fp8_writer_then_decode_end_to_end():
    """The GPU writer fills an fp8 store, the GPU HLA decode reads it; the
    oracle writes fp64 latents, quantizes each token's key and value parts
    with its own e4m3 quantizer, and decodes the dequantized latents."""
    H, dh, r, W, n_loops, d_in, P = 16, 128, 512, 8, 3, 256, 64
    N, Bsz, base = 150, 2, 10000.0
    wi = gen.writer_inputs(870, batch=Bsz, n_tok=N, n_loops=n_loops, groups=1, r_k=r, r_v=r, d_in=d_in,
                           dtype="bf16", positions=np.tile(np.arange(N), (Bsz, 1)))
    dc = gen.decode_inputs(871, batch=Bsz, heads=H, head_dim=dh, groups=1, r_k=r, r_v=r, positions=[N - 1, N - 1],
                           window=W, dtype="bf16", page_size=P, rope_base=base, rope_baked=1, loop=3,
                           loop_first=2, loop_last=4, exact_std=np.sqrt(3.0))
    desc = B.set_desc(n_heads=H, head_dim=dh, groups=1, r_k=r, r_v=r, loop_first=2, loop_last=4, page_size=P,
                      rope_baked=1, rope_base=base, dtype=B.LLA_BF16, latent_fp8=1)
    print(f"[case] fp8 writer->decode B={Bsz} N={N} r={r}", flush=True)
    pages = torch.full((B.store_bytes(desc, dc.n_pages),), NAN_CODE, dtype=torch.uint8, device="cuda")
    st = B.store(pages, dc.block_table.cuda())
    ws = torch.empty(max(B.lla_write_workspace_bytes(desc, Bsz, N, d_in), 4), dtype=torch.uint8, device="cuda")
    B.lla_write_latents(desc, st, pos=wi.pos.cuda(), x=wi.x.cuda(), enc=wi.enc.cuda(), workspace=ws)
    out = torch.empty(tuple(dc.q.shape), dtype=torch.bfloat16, device="cuda")
    dws = torch.empty(B.lla_decode_workspace_bytes(desc, Bsz, N - 1, W), dtype=torch.uint8, device="cuda")
    args = B.decode_args(loop=3, window=W, pos=dc.pos.cuda(), q=dc.q.cuda(), k_cur=dc.k_cur.cuda(),
                         v_cur=dc.v_cur.cuda(), ring_k=dc.ring_k.cuda(), ring_v=dc.ring_v.cuda(), A=dc.A.cuda(),
                         B=dc.Bv.transpose(1, 2).contiguous().cuda(), out=out, workspace=dws, max_pos_hint=N - 1)
    B.hla_decode_windowed(desc, st, Bsz, args)
    torch.cuda.synchronize()
    c = O.write_latents(wi.x.double().numpy(), wi.enc.double().numpy(), wi.pos.numpy(), r_k=r, rope_base=base,
                        rope_baked=1, head_dim=dh)
    kc, ks = O.fp8_quantize_rows(c[..., :r])
    vc, vs = O.fp8_quantize_rows(c[..., r:])
    kq = O.e4m3_decode(kc) * ks[..., None]
    vq = O.e4m3_decode(vc) * vs[..., None]
    f = [t.double().numpy() for t in (dc.q, dc.k_cur, dc.v_cur, dc.ring_k, dc.ring_v, dc.A, dc.Bv)]
    ref = O.absorbed_decode([kq[b] for b in range(Bsz)], [vq[b] for b in range(Bsz)], dc.pos.numpy(), *f,
                            window=W, rope_base=base)
    exact = O.absorbed_decode([c[b, ..., :r] for b in range(Bsz)], [c[b, ..., r:] for b in range(Bsz)],
                              dc.pos.numpy(), *f, window=W, rope_base=base)
    got = out.float().cpu().numpy()
    err = max_rel_err(got, ref)
    print(f"max_rel_err vs quantized oracle={err:.3e}; fp8 storage error vs unquantized={max_rel_err(ref, exact):.3e}")
    assert err < TOL["bf16"], err
