"""Parity of the HIP decode paths with the fp64 oracle, through the C ABI.

Tolerance (max over output rows of max|gpu - oracle| / max|oracle|):
1e-5 for fp32 storage, 2e-2 for bf16 storage with fp32 accumulation.
Unread store slots and ring slots are NaN-poisoned, the workspace starts
NaN-filled, and the output starts NaN-filled."""
import numpy as np
import pytest
import torch

from synth import gen
from compressed_cross_loop_amd import binding as B
from tests.gpu_cases import TOL, desc_of, oracle_decode, poison_unread, run_decode, widen_block_table
from tests.util import max_rel_err

pytestmark = pytest.mark.gpu


def hla_case(seed, *, r=512, positions=(300, 37, 129), W=16, H=16, d_h=128, dtype="bf16",
             loop=2, P=64):
    c = gen.decode_inputs(seed, batch=len(positions), heads=H, head_dim=d_h, groups=1, r_k=r, r_v=r,
                          positions=positions, window=W, dtype=dtype, page_size=P,
                          rope_base=10000.0, rope_baked=1, loop=loop,
                          loop_first=1 if loop == 1 else 2, loop_last=1 if loop == 1 else 4,
                          latent_std=np.sqrt(3.0), exact_std=np.sqrt(3.0))
    return poison_unread(c)


def check(c, entry, form, **kw):
    print(f"[case] entry={entry} form={form} B={c.batch} H={c.heads} G={c.groups} r={c.r_k} "
          f"W={c.window} pos={c.pos.tolist()} dtype={c.dtype} kw={kw}", flush=True)
    out, rk, rv = run_decode(entry, c, **kw)
    ref, slot, nk, nv = oracle_decode(c, form)
    err = max_rel_err(out, ref)
    assert err < TOL[c.dtype], err
    # ring: the current token was appended, every other slot is untouched
    for b in range(c.batch):
        assert max_rel_err(rk[b, slot[b]], nk[b]) < TOL[c.dtype]
        np.testing.assert_array_equal(rv[b, slot[b]], c.v_cur[b].float().numpy())
        keep = [s for s in range(c.window + 1) if s != slot[b]]
        np.testing.assert_array_equal(rk[b, keep], c.ring_k[b, keep].float().numpy())
    return err, out


@pytest.mark.parametrize("r", [512, 256])
@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("generic", [False, True])
def test_hla_bf16(r, splits, generic):
    c = hla_case(100 + r, r=r, loop=1 if r == 256 else 3)
    check(c, "hla", "absorbed", splits=splits, flags=1 if generic else 0)


@pytest.mark.parametrize("W, positions", [(128, (4095, 700, 129, 128)), (40, (500, 41, 12))])
def test_hla_bf16_window_slices(W, positions):
    """Exact windows spanning several 32-token slices, ragged last slice."""
    c = hla_case(150 + W, positions=positions, W=W)
    check(c, "hla", "absorbed")
    check(hla_case(150 + W, positions=positions, W=W), "hla", "absorbed", flags=1)


@pytest.mark.parametrize("r, loop", [(512, 3), (256, 1)])
@pytest.mark.parametrize("positions", [(4095,), (16383,), (700,), (4095, 300, 2000, 77, 1500)])
def test_hla_small_batch_combine(r, loop, positions):
    """Batches below 16: the matrix-core combine's small-batch form requests
    the first sequence's split rows and window slices at entry; at 16k the
    plan's 80 splits and 80 window slices take a second round of both, and
    with five sequences the others load theirs after the merge."""
    c = hla_case(820 + sum(positions) % 97 + r, r=r, positions=positions, W=128, loop=loop)
    check(c, "hla", "absorbed")


def test_hla_bf16_many_splits():
    """More context splits than the fast combine takes: the general combine merges them."""
    c = hla_case(160, positions=(4700,), W=16)
    check(c, "hla", "absorbed", splits=40)


def test_hla_bf16_matches_textbook_form_too():
    c = hla_case(7)
    out, _, _ = run_decode("hla", c)
    ref, *_ = oracle_decode(c, "textbook")
    assert max_rel_err(out, ref) < 2e-2


@pytest.mark.parametrize("positions", [(0, 5, 16, 17), (15, 16, 31, 64), (1000, 1, 63, 80)])
def test_hla_bf16_edges(positions):
    """first token, window covering the whole context, tile/page edges."""
    c = hla_case(200 + positions[0], positions=positions)
    check(c, "hla", "absorbed")
    check(hla_case(200 + positions[0], positions=positions), "hla", "absorbed", flags=1)


def test_hla_pos_beyond_hint_and_split_determinism():
    c = hla_case(300, positions=(700, 650))
    # plan for a shorter context than the real one: still exact
    check(c, "hla", "absorbed", max_pos_hint=100)
    a, _, _ = run_decode("hla", hla_case(300, positions=(700, 650)), splits=4)
    b, _, _ = run_decode("hla", hla_case(300, positions=(700, 650)), splits=4)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("r, d_h, H, G", [(64, 64, 4, 1), (128, 64, 8, 2), (128, 128, 6, 3), (32, 64, 6, 2)])
@pytest.mark.parametrize("splits", [0, 3])
def test_absorbed_bf16_widths_and_groups(r, d_h, H, G, splits):
    """Matrix-core absorbed scan at the narrow latent widths (deeper prefetch
    than r = 256 / 512) and with several heads per latent group."""
    seed = 600 + r + d_h + H + G + splits
    baked = r % d_h == 0   # rotary needs whole d_h blocks in the key latent
    c = gen.decode_inputs(seed, batch=3, heads=H, head_dim=d_h, groups=G, r_k=r, r_v=r,
                          positions=(613, 66, 9), window=5, dtype="bf16", page_size=64,
                          rope_base=10000.0 if baked else 0.0, rope_baked=int(baked), loop=2,
                          loop_first=1, loop_last=3, latent_std=np.sqrt(3.0), exact_std=np.sqrt(3.0),
                          paired=baked)
    check(poison_unread(c), "absorbed", "absorbed", splits=splits)


def tiny_fp32_case(seed, set_key, loop):
    """Workload 1 shape: 2 heads x 64, fp32, N = 256, W = 16, RoPE off."""
    r = 32 if set_key == 0 else 128
    lf, ll = (1, 1) if set_key == 0 else (2, 4)
    s = 1.0 / np.sqrt(64)
    c = gen.decode_inputs(seed, batch=1, heads=2, head_dim=64, groups=1, r_k=r, r_v=r,
                          positions=[255], window=16, dtype="f32", loop=loop, loop_first=lf,
                          loop_last=ll, map_scale=s, latent_std=1.0, exact_std=s)
    return poison_unread(c)


@pytest.mark.parametrize("entry, form", [("hla", "absorbed"), ("absorbed", "absorbed"),
                                         ("reconstruct", "textbook")])
@pytest.mark.parametrize("set_key, loop", [(0, 1), (1, 2), (1, 4)])
def test_tiny_fp32(entry, form, set_key, loop):
    c = tiny_fp32_case(10 + loop, set_key, loop)
    err, _ = check(c, entry, form)
    assert err < 1e-5


def per_head_case(seed, *, positions=(200, 77), W=0, dtype="bf16", r=32, H=16, d_h=128):
    c = gen.decode_inputs(seed, batch=len(positions), heads=H, head_dim=d_h, groups=H, r_k=r, r_v=r,
                          positions=positions, window=W, dtype=dtype, loop=2, loop_first=1,
                          loop_last=4, latent_std=4.0, exact_std=1.0, paired=False)
    return poison_unread(c)


@pytest.mark.parametrize("W", [0, 5])
def test_reconstruct_per_head_bf16(W):
    check(per_head_case(400 + W, W=W), "reconstruct", "textbook")


@pytest.mark.parametrize("r, d_h, H", [(32, 128, 16), (64, 128, 6), (32, 64, 5), (64, 64, 8)])
@pytest.mark.parametrize("generic", [False, True])
def test_reconstruct_per_head_shapes(r, d_h, H, generic):
    """Matrix-core and general reconstruct kernels: latent widths, head dims,
    head counts that leave a partial workgroup, ragged contexts, splits."""
    c = per_head_case(440 + r + d_h + H, positions=(333, 17, 64, 1), W=3, r=r, H=H, d_h=d_h)
    check(c, "reconstruct", "textbook", flags=1 if generic else 0)
    c = per_head_case(441 + r + d_h + H, positions=(333, 17, 64, 1), W=3, r=r, H=H, d_h=d_h)
    check(c, "reconstruct", "textbook", splits=3, flags=1 if generic else 0)


@pytest.mark.parametrize("splits", [1, 2])
def test_reconstruct_per_head_long_window(splits):
    """Per-head reconstruct with a window of 100 exact tokens: a split's exact
    steps of 16 tokens are dealt to the four waves of its workgroup in turn
    (the current token's ring append included); position 64 < W leaves no
    latent token at all."""
    c = per_head_case(470 + splits, positions=(333, 120, 64), W=100)
    check(c, "reconstruct", "textbook", splits=splits)


@pytest.mark.parametrize("d_h, r, rope", [(64, 192, True), (128, 208, False)])
def test_qmap_partial_column_block(d_h, r, rope):
    """Matrix-core query map with latent widths that are not a whole number
    of its 128-column blocks (the last block partly past r_k; with rotary the
    partner columns stay inside it), two latent groups so that the one-pass
    general scan reads q~ (the HLA entry takes one group only, whose wide
    shapes have their own query map)."""
    c = gen.decode_inputs(480 + r, batch=3, heads=4, head_dim=d_h, groups=2, r_k=r, r_v=r,
                          positions=(400, 77, 5), window=5, dtype="bf16",
                          rope_base=10000.0 if rope else 0.0, rope_baked=int(rope), loop=2,
                          loop_first=1, loop_last=3, latent_std=np.sqrt(3.0), exact_std=np.sqrt(3.0),
                          paired=rope)
    check(poison_unread(c), "absorbed", "absorbed")


@pytest.mark.parametrize("generic", [False, True])
def test_lla_d_per_head_bf16(generic):
    check(per_head_case(410), "absorbed", "absorbed", flags=1 if generic else 0)


def test_absorbed_equals_reconstruct_on_gpu():
    """LLA-D and reconstruct read the same store (RoPE off): same result."""
    c = per_head_case(420, positions=(150, 64, 3))
    a, _, _ = run_decode("absorbed", c)
    r, _, _ = run_decode("reconstruct", per_head_case(420, positions=(150, 64, 3)))
    assert max_rel_err(a, r) < 2e-2


def test_reconstruct_shared_latent_bf16():
    """Reconstruct from one latent shared by all heads (G = 1, LLA-2D style)."""
    c = gen.decode_inputs(430, batch=2, heads=6, head_dim=96, groups=1, r_k=192, r_v=192,
                          positions=(130, 40), window=0, dtype="bf16", loop=3, loop_first=1,
                          loop_last=8, latent_std=1.0, exact_std=1.0, paired=False,
                          map_scale=np.sqrt(192 / 96))
    check(poison_unread(c), "reconstruct", "textbook")
    c = gen.decode_inputs(431, batch=2, heads=6, head_dim=96, groups=1, r_k=192, r_v=192,
                          positions=(130, 40), window=0, dtype="bf16", loop=3, loop_first=1,
                          loop_last=8, latent_std=1.0, exact_std=1.0, paired=False,
                          map_scale=np.sqrt(192 / 96))
    check(poison_unread(c), "absorbed", "absorbed")


@pytest.mark.parametrize("H, d_h, r_k, r_v", [(6, 96, 192, 192), (20, 64, 256, 256), (3, 64, 96, 32),
                                              (55, 96, 1056, 1056), (64, 64, 64, 64), (2, 96, 5280, 5280)])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_absorbed_wide_shared_latent(H, d_h, r_k, r_v, splits):
    """LLA-D over one latent shared by all heads, shapes the one-pass matrix-core
    scan does not take (r not a power of two, more than 16 heads, r_k != r_v,
    r in the thousands): the two-pass scan.  Ragged 16-token tiles, empty and
    forced splits, 256-dim value slabs with a ragged last slab."""
    c = gen.decode_inputs(700 + H + r_k + r_v + splits, batch=3, heads=H, head_dim=d_h, groups=1, r_k=r_k,
                          r_v=r_v, positions=(300, 129, 7), window=4, dtype="bf16", loop=3, loop_first=1,
                          loop_last=8, latent_std=1.0, exact_std=1.0, paired=False,
                          map_scale=float(np.sqrt(r_k / d_h)))
    assert B.lla_decode_scan_kernel(desc_of(c), 1) == "k_scan_absorbed_wide"
    check(poison_unread(c), "absorbed", "absorbed", splits=splits)


@pytest.mark.parametrize("batch", [8, 16])
@pytest.mark.parametrize("H, d_h, r_k, r_v, splits", [(6, 96, 192, 192, 0), (6, 96, 192, 192, 3),
                                                      (55, 96, 1056, 1056, 0)])
def test_absorbed_wide_xcd_grid(batch, H, d_h, r_k, r_v, splits):
    """Batches that are a multiple of 8: the two-pass scan's score and value
    passes run one-dimensional grids dealt so that a sequence's workgroups
    share an XCD.  Ragged positions (one sequence with no latent token at all,
    so all of its score workgroups return at once, one with a single latent
    tile), forced splits, and the 1056-wide latent split over parts of r_k."""
    positions = (1500, 700, 4, 1023, 1024, 20, 900, 1600, 64, 1300, 333, 1200, 2, 800, 1100, 450)[:batch]
    c = gen.decode_inputs(860 + batch + r_k + splits, batch=batch, heads=H, head_dim=d_h, groups=1, r_k=r_k,
                          r_v=r_v, positions=positions, window=4, dtype="bf16", loop=3, loop_first=1,
                          loop_last=8, latent_std=1.0, exact_std=1.0, paired=False,
                          map_scale=float(np.sqrt(r_k / d_h)))
    assert B.lla_decode_scan_kernel(desc_of(c), 1) == "k_scan_absorbed_wide"
    check(poison_unread(c), "absorbed", "absorbed", splits=splits)


@pytest.mark.parametrize("H, d_h, r", [(20, 64, 256), (6, 96, 192), (18, 128, 1024)])
@pytest.mark.parametrize("entry", ["absorbed", "hla"])
def test_absorbed_wide_rope(H, d_h, r, entry):
    """The two-pass scan with RoPE (frequency-paired decoders, rotation baked
    into the stored key latents, q~ rotated per d_h block by the query map) and
    an exact window, through both absorbed entry points."""
    c = gen.decode_inputs(780 + H + r, batch=3, heads=H, head_dim=d_h, groups=1, r_k=r, r_v=r,
                          positions=(300, 129, 17), window=16, dtype="bf16", rope_base=10000.0, rope_baked=1,
                          loop=2, loop_first=2, loop_last=4, latent_std=1.0, exact_std=1.0)
    assert B.lla_decode_scan_kernel(desc_of(c), 1) == "k_scan_absorbed_wide"
    check(poison_unread(c), entry, "absorbed")


@pytest.mark.parametrize("positions", [(300,), (4000,), (5,)])
def test_absorbed_wide_single_sequence(positions):
    """Batch 1: the score pass splits r_k into parts (here 9 of 128 dims, the
    last one 32) summed by the softmax pass; a context shorter than one tile."""
    c = gen.decode_inputs(800 + positions[0], batch=1, heads=55, head_dim=96, groups=1, r_k=1056, r_v=1056,
                          positions=positions, window=0, dtype="bf16", loop=3, loop_first=1, loop_last=8,
                          latent_std=1.0, exact_std=1.0, paired=False, map_scale=float(np.sqrt(1056 / 96)))
    check(poison_unread(c), "absorbed", "absorbed")


@pytest.mark.parametrize("hint, columns, kernel", [(100, 16, "k_scan_absorbed_generic"),
                                                   (2000, 5, "k_scan_absorbed_wide"),
                                                   (20000, 5, "k_scan_absorbed_wide")])
def test_absorbed_wide_hint(hint, columns, kernel):
    """max_pos_hint below the positions with a block table of 16 pages (1024
    tokens, more than the 512-token score rows planned from the hint: the
    one-pass general scan runs, between the matrix-core query map and combine),
    and far above them (longer score rows than needed; at 20000 longer than
    the softmax pass keeps in LDS): all stay exact."""
    c = gen.decode_inputs(760 + hint, batch=3, heads=6, head_dim=96, groups=1, r_k=192, r_v=192,
                          positions=(300, 129, 7), window=4, dtype="bf16", loop=3, loop_first=1,
                          loop_last=8, latent_std=1.0, exact_std=1.0, paired=False,
                          map_scale=float(np.sqrt(2.0)))
    c = widen_block_table(poison_unread(c), columns)
    assert B.lla_decode_scan_kernel_for_store(desc_of(c), 1, hint, columns) == kernel
    check(c, "absorbed", "absorbed", max_pos_hint=hint)


@pytest.mark.parametrize("entry, form, G, r, columns, kernel", [
    ("reconstruct", "textbook", 16, 32, 4097, "k_scan_reconstruct_generic"),
    ("reconstruct", "textbook", 16, 32, 4096, "k_scan_reconstruct_mfma"),
    ("absorbed", "absorbed", 16, 32, 8193, "k_scan_absorbed_generic"),
    ("hla", "absorbed", 1, 256, 8193, "k_scan_absorbed_generic"),
    ("hla", "absorbed", 1, 256, 8192, "k_scan_absorbed_mfma"),
])
def test_long_block_table(entry, form, G, r, columns, kernel):
    """16-token pages and a block table longer than the matrix-core scans
    stage in LDS (4096 page ids per split for the per-head reconstruct scan,
    8192 for the absorbed scan): the call takes the general scan and stays
    exact; at the limit the matrix-core scan runs."""
    H, d_h = 16, 128
    rope = G == 1
    c = gen.decode_inputs(900 + columns + r, batch=2, heads=H, head_dim=d_h, groups=G, r_k=r, r_v=r,
                          positions=(150, 41), window=5, dtype="bf16", page_size=16,
                          rope_base=10000.0 if rope else 0.0, rope_baked=int(rope), loop=2,
                          loop_first=1 if not rope else 2, loop_last=4, latent_std=2.0,
                          exact_std=1.0, paired=rope)
    c = widen_block_table(poison_unread(c), columns)
    assert B.lla_decode_scan_kernel_for_store(desc_of(c), {"reconstruct": 0, "absorbed": 1, "hla": 2}[entry],
                                              150, columns) == kernel
    check(c, entry, form)


@pytest.mark.parametrize("d_h", [96, 64])
@pytest.mark.parametrize("columns", [2048, 2049])
def test_reconstruct_shared_latent_long_block_table(d_h, columns):
    """16-token pages and a block table at, and one past, the 2048 page ids
    per split that the LDS-staged head-folded reconstruct holds: the staged
    form, then the register-streamed one; both exact."""
    r = 192
    c = gen.decode_inputs(1300 + columns + d_h, batch=2, heads=5, head_dim=d_h, groups=1, r_k=r, r_v=r,
                          positions=(150, 41), window=5, dtype="bf16", page_size=16, loop=3,
                          loop_first=1, loop_last=8, latent_std=1.0, exact_std=1.0, paired=False,
                          map_scale=float(np.sqrt(r / d_h)))
    c = widen_block_table(poison_unread(c), columns)
    assert B.lla_decode_scan_kernel_for_store(desc_of(c), 0, 150, columns) == "k_scan_reconstruct_gemm"
    check(c, "reconstruct", "textbook")


@pytest.mark.parametrize("H, d_h, r", [(5, 96, 192), (4, 128, 256), (3, 64, 96), (2, 96, 5280)])
@pytest.mark.parametrize("splits", [0, 2])
def test_reconstruct_shared_latent_shapes(H, d_h, r, splits):
    """Head-folded reconstruct (one latent shared by all heads): odd head
    counts, ragged 128-token tiles, an exact window, forced splits."""
    c = gen.decode_inputs(460 + H + r + splits, batch=3, heads=H, head_dim=d_h, groups=1, r_k=r, r_v=r,
                          positions=(300, 129, 7), window=4, dtype="bf16", loop=3, loop_first=1,
                          loop_last=8, latent_std=1.0, exact_std=1.0, paired=False,
                          map_scale=float(np.sqrt(r / d_h)))
    check(poison_unread(c), "reconstruct", "textbook", splits=splits)
