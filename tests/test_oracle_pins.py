"""Pins of the fp64 oracle to facts that do not come from the oracle itself:
numbers printed on the pages, closed forms, library routines on special cases,
algebraic identities, and brute force on tiny inputs.

Sources: "Hybrid Latent Attention" summary (picx.dev/p/a0K1YZ), sections
"Summary (Overview)", "Key Problem", "Latent Writer" (Eq. 2), "Latent Reader"
(Eqs. 3-4) and "Rotary Embedding Alignment"; "Looped Latent Attention" abstracts
(acceptodds.com/papers/iclr2027-34396, searcharxiv.org/abs/2607.15456).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from tests.util import golden_kv, golden_lines, max_rel_err


# ---------------------------------------------------------------- cache bytes
def test_cache_bytes_match_printed_values():
    """768 KiB -> 72 KiB per token, 10.7x ("Summary (Overview)", "Latent Writer")."""
    g = golden_kv("cache_bytes.txt")
    full = O.full_cache_bytes_per_token(int(g["layers"]), int(g["loops"]), int(g["d_model"]),
                                        int(g["elem_bytes"]))
    hla = O.hla_bytes_per_token(int(g["layers"]), int(g["r_k"]), int(g["r_v"]), int(g["r_1"]),
                                int(g["elem_bytes"]))
    assert full == g["full_cache_kib"] * 1024
    assert hla == g["hla_kib"] * 1024
    assert round(full / hla, 1) == g["ratio_1dp"]


def test_cache_bytes_other_workloads():
    # per-head LLA rank 32 on Ouro-1.4B: 16 heads x 64 numbers x 2 B x 24 layers = 48 KiB (16x)
    per_layer = O.set_bytes_per_token(16, 32, 32, 2)
    assert 24 * per_layer == 48 * 1024
    assert O.full_cache_bytes_per_token(24, 4, 2048, 2) // (24 * per_layer) == 16
    # LLA-2D, Huginn-like: one 5280 K + one 5280 V latent per token-layer vs 2*32*5280 (32x)
    assert O.set_bytes_per_token(1, 5280, 5280, 2) * 32 == O.full_cache_bytes_per_token(1, 32, 5280, 2)


# ---------------------------------------------------------------- rotary embedding
def test_rope_closed_form():
    theta = O.rope_theta(4, 10000.0)
    np.testing.assert_allclose(theta, [1.0, 0.01], rtol=0, atol=1e-15)
    for line in golden_lines("rope_closed_form.txt"):
        idx, vals = line.split(":")
        e = np.zeros(4)
        e[int(idx)] = 1.0
        want = np.array([float(v) for v in vals.split()])
        np.testing.assert_allclose(O.rope_head(e, 3, 10000.0), want, rtol=0, atol=1e-15)


def test_rope_group_properties():
    g = gen.rng(11)
    d_h, base = 16, 10000.0
    x = g.standard_normal((5, d_h))
    # R_0 = I, R_p orthogonal, R_p R_q = R_{p+q}
    np.testing.assert_allclose(O.rope_head(x, 0, base), x, atol=1e-15)
    np.testing.assert_allclose(np.linalg.norm(O.rope_head(x, 123, base), axis=1),
                               np.linalg.norm(x, axis=1), rtol=1e-14)
    np.testing.assert_allclose(O.rope_head(O.rope_head(x, 17, base), 40, base),
                               O.rope_head(x, 57, base), atol=1e-12)
    # inner product depends on the position difference only
    y = g.standard_normal(d_h)
    a = O.rope_head(x, 100, base) @ O.rope_head(y, 93, base)
    b = O.rope_head(x, 7, base) @ O.rope_head(y, 0, base)
    np.testing.assert_allclose(a, b, rtol=1e-12)
    # no rotary embedding
    np.testing.assert_array_equal(O.rope_head(x, 99, 0.0), x)


def test_rope_latent_rotates_every_block_alike():
    g = gen.rng(12)
    d_h, m = 8, 3
    c = g.standard_normal(d_h * m)
    out = O.rope_latent(c, 29, 10000.0, d_h)
    for b in range(m):
        np.testing.assert_allclose(out[b * d_h:(b + 1) * d_h],
                                   O.rope_head(c[b * d_h:(b + 1) * d_h], 29, 10000.0), atol=1e-15)


@pytest.mark.parametrize("complex_coeffs", [True, False])
def test_frequency_paired_decoders_commute(complex_coeffs):
    """"Rotary Embedding Alignment": rotation commutes with combinations of key
    pairs that share a frequency:  R_p A = A R~_p."""
    g = gen.rng(13)
    d_h, r_k, H = 8, 32, 3
    A = gen.frequency_paired_decoder(g, H, d_h, r_k, complex_coeffs=complex_coeffs)
    c = g.standard_normal(r_k)
    for h in range(H):
        for p in (0, 1, 77, 4095):
            lhs = O.rope_head(A[h] @ c, p, 10000.0)
            rhs = A[h] @ O.rope_latent(c, p, 10000.0, d_h)
            np.testing.assert_allclose(lhs, rhs, atol=1e-13)
        # orthonormal rows
        np.testing.assert_allclose(A[h] @ A[h].T, np.eye(d_h), atol=1e-13)


def test_dense_decoder_does_not_commute():
    """Negative control: a dense map does not commute with the rotation."""
    g = gen.rng(14)
    d_h, r_k = 8, 32
    A = gen.gaussian_orthonormal(g, d_h, r_k)
    c = g.standard_normal(r_k)
    lhs = O.rope_head(A @ c, 5, 10000.0)
    rhs = A @ O.rope_latent(c, 5, 10000.0, d_h)
    assert np.abs(lhs - rhs).max() > 1e-2


# ---------------------------------------------------------------- store layout
def test_store_layout_fixture():
    kw = dict(groups=2, page_size=32, r_k=16, r_v=32)
    for line in golden_lines("store_layout.txt"):
        if line.startswith("params"):
            g_, p_, rk_, rv_ = (int(x) for x in line.split()[1:])
            kw = dict(groups=g_, page_size=p_, r_k=rk_, r_v=rv_)
            continue
        lhs, want = line.split(":")
        kind, page, group, slot, dim = lhs.split()
        fn = O.store_key_offset if kind == "key" else O.store_value_offset
        assert int(fn(int(page), int(group), int(slot), int(dim), **kw)) == int(want)


def test_store_layout_is_a_bijection():
    kw = dict(groups=3, page_size=48, r_k=32, r_v=16)
    n_pages = 2
    R = kw["r_k"] + kw["r_v"]
    p, g, s = np.meshgrid(np.arange(n_pages), np.arange(3), np.arange(48), indexing="ij")
    ko = O.store_key_offset(p[..., None], g[..., None], s[..., None], np.arange(32), **kw)
    vo = O.store_value_offset(p[..., None], g[..., None], s[..., None], np.arange(16), **kw)
    allo = np.concatenate([ko.ravel(), vo.ravel()])
    assert np.array_equal(np.sort(allo), np.arange(n_pages * 3 * 48 * R))


@pytest.mark.parametrize("r_k, r_v", [(544, 16), (528, 48)])
def test_wide_key_layout_is_a_bijection(r_k, r_v):
    """Chunk-major wide key rows still tile the store exactly once."""
    kw = dict(groups=2, page_size=32, r_k=r_k, r_v=r_v)
    n_pages = 2
    p, g, s = np.meshgrid(np.arange(n_pages), np.arange(2), np.arange(32), indexing="ij")
    ko = O.store_key_offset(p[..., None], g[..., None], s[..., None], np.arange(r_k), **kw)
    vo = O.store_value_offset(p[..., None], g[..., None], s[..., None], np.arange(r_v), **kw)
    allo = np.concatenate([ko.ravel(), vo.ravel()])
    assert np.array_equal(np.sort(allo), np.arange(n_pages * 2 * 32 * (r_k + r_v)))


def test_wide_key_chunk_is_contiguous():
    """The 16 tokens x 32 dimensions of one key chunk of a tile are one
    contiguous run of 512 elements (what the wide readers rely on)."""
    kw = dict(groups=1, page_size=16, r_k=1024, r_v=32)
    s, d = np.meshgrid(np.arange(16), np.arange(64, 96), indexing="ij")
    o = np.sort(O.store_key_offset(0, 0, s, d, **kw).ravel())
    assert np.array_equal(o, np.arange(o[0], o[0] + 512)) and o[0] == 2 * 512


def test_gather_follows_block_table():
    kw = dict(groups=2, page_size=16, r_k=16, r_v=16)
    n_pages = 4
    pages = np.arange(n_pages * 2 * 16 * 32, dtype=np.float64).reshape(n_pages, -1)
    bt = np.array([[2, 0], [3, 1]])
    sK, sV = O.gather_latents(pages, bt, 1, 20, **kw)
    # token 17 of sequence 1 sits in physical page 1, slot 1
    assert sK[17, 1, 3] == O.store_key_offset(1, 1, 1, 3, **kw)
    assert sV[17, 0, 9] == O.store_value_offset(1, 0, 1, 9, **kw)
    assert sK[2, 0, 0] == O.store_key_offset(3, 0, 2, 0, **kw)


# ---------------------------------------------------------------- writer (Eq. 2)
def test_writer_placement_encoders_stack_inputs():
    """With encoders that place loop t's input in its own block, c is exactly
    the stack of the per-loop inputs (Eq. 2's sum of E_t h_t)."""
    g = gen.rng(21)
    B, n, T, G, d_in = 2, 3, 3, 2, 4
    x = g.standard_normal((B, n, T, G, d_in))
    R = T * d_in
    enc = np.zeros((T, G, R, d_in))
    for t in range(T):
        for gg in range(G):
            enc[t, gg, t * d_in:(t + 1) * d_in, :] = np.eye(d_in)
    c = O.write_latents(x, enc, np.zeros((B, n), dtype=np.int64), r_k=R // 2)
    np.testing.assert_array_equal(c, np.concatenate([x[:, :, t] for t in range(T)], axis=-1))


def test_writer_linear_and_brute_force():
    g = gen.rng(22)
    B, n, T, G, d_in, r_k, r_v, d_h = 1, 2, 2, 2, 5, 8, 4, 4
    x1 = g.standard_normal((B, n, T, G, d_in))
    x2 = g.standard_normal((B, n, T, G, d_in))
    enc = g.standard_normal((T, G, r_k + r_v, d_in))
    pos = np.array([[3, 9]])
    kw = dict(r_k=r_k, rope_base=10000.0, rope_baked=1, head_dim=d_h)
    c1 = O.write_latents(x1, enc, pos, **kw)
    c2 = O.write_latents(x2, enc, pos, **kw)
    np.testing.assert_allclose(O.write_latents(x1 + 2 * x2, enc, pos, **kw), c1 + 2 * c2, atol=1e-12)
    # brute force: explicit sums, then the rotation written with math.cos / math.sin
    for tok in range(n):
        p = int(pos[0, tok])
        for gg in range(G):
            raw = [sum(enc[t, gg, o, k] * x1[0, tok, t, gg, k] for t in range(T) for k in range(d_in))
                   for o in range(r_k + r_v)]
            want = list(raw)
            half = d_h // 2
            for blk in range(r_k // d_h):
                for f in range(half):
                    th = 10000.0 ** (-2.0 * f / d_h)
                    a, b = raw[blk * d_h + f], raw[blk * d_h + f + half]
                    want[blk * d_h + f] = a * math.cos(p * th) - b * math.sin(p * th)
                    want[blk * d_h + f + half] = a * math.sin(p * th) + b * math.cos(p * th)
            np.testing.assert_allclose(c1[0, tok, gg], want, atol=1e-12)


# ---------------------------------------------------------------- decode
def _complex_rope(x, p, base):
    """Independent rotation for the references: pairs as complex numbers
    z_f = x_f + i x_{f+d_h/2}, multiplied by exp(i p theta_f)."""
    d_h = x.shape[-1]
    half = d_h // 2
    th = base ** (-2.0 * np.arange(half) / d_h) if base else np.zeros(half)
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * np.asarray(p)[..., None] * th)
    return np.concatenate([z.real, z.imag], axis=-1)


def _identity_hla(seed, *, H=2, d_h=4, T=3, n_tok=12, base=10000.0):
    """Uncompressed looped K/V plus a full-rank identity HLA codec built from it."""
    g = gen.rng(seed)
    hd = H * d_h
    k = g.standard_normal((T, n_tok, H, d_h))   # pre-rotation keys per loop
    v = g.standard_normal((T, n_tok, H, d_h))
    q = g.standard_normal((T, H, d_h))
    # main set: loops 2..T, r_k = r_v = (T-1) H d_h ; loop-1 set: r_1 = H d_h
    r_main = (T - 1) * hd
    x_main = np.zeros((1, n_tok, T - 1, 1, 2 * hd))
    enc_main = np.zeros((T - 1, 1, 2 * r_main, 2 * hd))
    for t in range(2, T + 1):
        x_main[0, :, t - 2, 0, :hd] = k[t - 1].reshape(n_tok, hd)
        x_main[0, :, t - 2, 0, hd:] = v[t - 1].reshape(n_tok, hd)
        enc_main[t - 2, 0, (t - 2) * hd:(t - 1) * hd, :hd] = np.eye(hd)
        enc_main[t - 2, 0, r_main + (t - 2) * hd:r_main + (t - 1) * hd, hd:] = np.eye(hd)
    x1 = np.zeros((1, n_tok, 1, 1, 2 * hd))
    x1[0, :, 0, 0, :hd] = k[0].reshape(n_tok, hd)
    x1[0, :, 0, 0, hd:] = v[0].reshape(n_tok, hd)
    enc1 = np.zeros((1, 1, 2 * hd, 2 * hd))
    enc1[0, 0] = np.eye(2 * hd)
    pos = np.arange(n_tok)[None, :]
    c_main = O.write_latents(x_main, enc_main, pos, r_k=r_main, rope_base=base, rope_baked=1, head_dim=d_h)
    c_one = O.write_latents(x1, enc1, pos, r_k=hd, rope_base=base, rope_baked=1, head_dim=d_h)

    def maps(t):
        blk = 0 if t == 1 else t - 2
        r = hd if t == 1 else r_main
        A = np.zeros((H, d_h, r))
        Bv = np.zeros((H, r, d_h))
        for h in range(H):
            A[h, :, blk * hd + h * d_h: blk * hd + (h + 1) * d_h] = np.eye(d_h)
            Bv[h, blk * hd + h * d_h: blk * hd + (h + 1) * d_h, :] = np.eye(d_h)
        c = c_one if t == 1 else c_main
        return c[0, :, :, :r], c[0, :, :, r:], A, Bv

    return k, v, q, maps


def _ring(k_t, v_t, i, W, base):
    H, d_h = k_t.shape[1:]
    rk = np.full((1, W + 1, H, d_h), np.nan)
    rv = np.full((1, W + 1, H, d_h), np.nan)
    for j in range(max(0, i - W), i):
        rk[0, j % (W + 1)] = _complex_rope(k_t[j], j, base)
        rv[0, j % (W + 1)] = v_t[j]
    return rk, rv


def _sdpa_reference(k_t, v_t, q_t, i, base):
    """Uncompressed attention of loop t at position i: torch's scaled dot
    product attention in fp64 on the CPU over all tokens 0..i."""
    H, d_h = q_t.shape
    keys = np.stack([_complex_rope(k_t[j], j, base) for j in range(i + 1)])      # [i+1, H, d_h]
    qr = _complex_rope(q_t, i, base)                                                # [H, d_h]
    qq = torch.from_numpy(qr)[None, :, None, :]
    kk = torch.from_numpy(keys.transpose(1, 0, 2).copy())[None]
    vv = torch.from_numpy(v_t[: i + 1].transpose(1, 0, 2).copy())[None]
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[0, :, 0, :].numpy()


@pytest.mark.parametrize("form", ["textbook", "absorbed"])
@pytest.mark.parametrize("t", [1, 2, 3])
@pytest.mark.parametrize("W", [0, 1, 4, 9, 20])
def test_identity_codec_equals_uncompressed_attention(form, t, W):
    """A full-rank identity codec must reproduce uncompressed looped attention,
    for every window W (Eq. 4's single softmax makes the output W-independent)."""
    base = 10000.0
    k, v, q, maps = _identity_hla(31, base=base)
    i = 10
    sK, sV, A, Bv = maps(t)
    rk, rv = _ring(k[t - 1], v[t - 1], i, W, base)
    fn = O.textbook_decode if form == "textbook" else O.absorbed_decode
    out = fn([sK], [sV], [i], q[t - 1][None], k[t - 1][i][None], v[t - 1][i][None], rk, rv, A, Bv,
             window=W, rope_base=base)
    ref = _sdpa_reference(k[t - 1], v[t - 1], q[t - 1], i, base)
    np.testing.assert_allclose(out[0], ref, atol=1e-12)


@pytest.mark.parametrize("form", ["textbook", "absorbed"])
def test_identity_codec_per_head_lla(form):
    """Per-head LLA identity codec (G = H, one set for loops 1..T)."""
    g = gen.rng(32)
    H, d_h, T, n_tok, base, W, i = 3, 4, 2, 9, 10000.0, 2, 8
    k = g.standard_normal((T, n_tok, H, d_h))
    v = g.standard_normal((T, n_tok, H, d_h))
    q = g.standard_normal((H, d_h))
    r = T * d_h
    x = np.zeros((1, n_tok, T, H, 2 * d_h))
    enc = np.zeros((T, H, 2 * r, 2 * d_h))
    for t in range(T):
        x[0, :, t, :, :d_h] = k[t]
        x[0, :, t, :, d_h:] = v[t]
        for h in range(H):
            enc[t, h, t * d_h:(t + 1) * d_h, :d_h] = np.eye(d_h)
            enc[t, h, r + t * d_h: r + (t + 1) * d_h, d_h:] = np.eye(d_h)
    c = O.write_latents(x, enc, np.arange(n_tok)[None], r_k=r, rope_base=base, rope_baked=1, head_dim=d_h)
    for t in range(1, T + 1):
        A = np.zeros((H, d_h, r))
        Bv = np.zeros((H, r, d_h))
        for h in range(H):
            A[h, :, (t - 1) * d_h: t * d_h] = np.eye(d_h)
            Bv[h, (t - 1) * d_h: t * d_h, :] = np.eye(d_h)
        rk, rv = _ring(k[t - 1], v[t - 1], i, W, base)
        fn = O.textbook_decode if form == "textbook" else O.absorbed_decode
        out = fn([c[0, :, :, :r]], [c[0, :, :, r:]], [i], q[None], k[t - 1][i][None],
                 v[t - 1][i][None], rk, rv, A, Bv, window=W, rope_base=base)
        np.testing.assert_allclose(out[0], _sdpa_reference(k[t - 1], v[t - 1], q, i, base), atol=1e-12)


def test_sequential_steps_with_ring_update():
    """Three decode steps in a row, the window maintained only by ring_update
    and the latents only by the writer, still match uncompressed attention."""
    base, W, t = 10000.0, 3, 2
    k, v, q, maps = _identity_hla(33, n_tok=14, base=base)
    sK, sV, A, Bv = maps(t)
    i0 = 9
    rk, rv = _ring(k[t - 1], v[t - 1], i0, W, base)
    for i in range(i0, i0 + 3):
        out = O.textbook_decode([sK], [sV], [i], q[t - 1][None], k[t - 1][i][None], v[t - 1][i][None],
                                rk, rv, A, Bv, window=W, rope_base=base)
        np.testing.assert_allclose(out[0], _sdpa_reference(k[t - 1], v[t - 1], q[t - 1], i, base),
                                   atol=1e-12)
        slot, nk, nv = O.ring_update([i], k[t - 1][i][None], v[t - 1][i][None], window=W,
                                     rope_base=base)
        rk[0, slot[0]] = nk[0]
        rv[0, slot[0]] = nv[0]


def _random_case(seed, *, B=2, H=4, G=2, d_h=8, r_k=16, r_v=12, W=3, base=10000.0, n=30,
                 paired=True):
    g = gen.rng(seed)
    sK = [g.standard_normal((n, G, r_k)) for _ in range(B)]
    sV = [g.standard_normal((n, G, r_v)) for _ in range(B)]
    q = g.standard_normal((B, H, d_h))
    kc = g.standard_normal((B, H, d_h))
    vc = g.standard_normal((B, H, d_h))
    rk = g.standard_normal((B, W + 1, H, d_h))
    rv = g.standard_normal((B, W + 1, H, d_h))
    if paired:
        A = gen.frequency_paired_decoder(g, H, d_h, r_k)
    else:
        A = np.stack([gen.gaussian_orthonormal(g, d_h, r_k) for _ in range(H)])
    Bv = np.stack([gen.gaussian_orthonormal(g, r_v, d_h) for _ in range(H)])
    return sK, sV, q, kc, vc, rk, rv, A, Bv


@pytest.mark.parametrize("pos", [[0, 29], [3, 4], [17, 2], [29, 25]])
def test_absorbed_equals_textbook(pos):
    """Step-6 identity: the absorbed read (Eq. 3/4) equals reconstruct-then-attend
    when every key decoder is frequency-paired."""
    args = _random_case(41)
    kw = dict(window=3, rope_base=10000.0)
    a = O.absorbed_decode(*args[:2], pos, *args[2:], **kw)
    t = O.textbook_decode(*args[:2], pos, *args[2:], **kw)
    assert max_rel_err(a, t) < 1e-12


def test_absorbed_differs_from_textbook_for_dense_decoders():
    """Negative control: with rotary embedding on and dense key decoders the two
    forms disagree (so the previous test can fail)."""
    args = _random_case(42, paired=False)
    kw = dict(window=3, rope_base=10000.0)
    a = O.absorbed_decode(*args[:2], [29, 20], *args[2:], **kw)
    t = O.textbook_decode(*args[:2], [29, 20], *args[2:], **kw)
    assert max_rel_err(a, t) > 1e-3
    # ...and agree again without rotary embedding
    kw0 = dict(window=3, rope_base=0.0)
    assert max_rel_err(O.absorbed_decode(*args[:2], [29, 20], *args[2:], **kw0),
                       O.textbook_decode(*args[:2], [29, 20], *args[2:], **kw0)) < 1e-12


def test_first_token_returns_current_value():
    """i = 0: the only attended token is the current one, so o = v_cur."""
    sK, sV, q, kc, vc, rk, rv, A, Bv = _random_case(43)
    for fn in (O.textbook_decode, O.absorbed_decode):
        out = fn(sK, sV, [0, 0], q, kc, vc, rk, rv, A, Bv, window=3, rope_base=10000.0)
        np.testing.assert_allclose(out, vc, atol=1e-15)


def test_window_covering_context_ignores_latents():
    """W >= i: no latent token is read, so changing the store changes nothing."""
    sK, sV, q, kc, vc, rk, rv, A, Bv = _random_case(44)
    sK2 = [x + 5.0 for x in sK]
    sV2 = [x - 3.0 for x in sV]
    for fn in (O.textbook_decode, O.absorbed_decode):
        a = fn(sK, sV, [3, 2], q, kc, vc, rk, rv, A, Bv, window=3, rope_base=10000.0)
        b = fn(sK2, sV2, [3, 2], q, kc, vc, rk, rv, A, Bv, window=3, rope_base=10000.0)
        np.testing.assert_array_equal(a, b)


def test_relative_position_invariance():
    """Scores depend on positions only through i - j: with the query rotated at
    i + delta and latents baked by the writer at j + delta, every latent score
    of Eq. 3 is unchanged, and so is every exact-window score."""
    g = gen.rng(45)
    H, d_h, r, d_in, n, base = 2, 8, 16, 6, 20, 10000.0
    x = g.standard_normal((1, n, 2, 1, d_in))
    enc = g.standard_normal((2, 1, 2 * r, d_in))
    A = gen.frequency_paired_decoder(g, H, d_h, r)
    q = g.standard_normal(d_h)
    k_ex = g.standard_normal((n, d_h))
    i = n - 1
    ref = None
    for delta in (0, 37, 1000, 16000):
        pos = np.arange(n)[None] + delta
        c = O.write_latents(x, enc, pos, r_k=r, rope_base=base, rope_baked=1, head_dim=d_h)
        s_lat = np.stack([c[0, :, 0, :r] @ O.rope_latent(A[h].T @ q, i + delta, base, d_h)
                          for h in range(H)])
        s_ex = O.rope_head(k_ex, np.arange(n) + delta, base) @ O.rope_head(q, i + delta, base)
        if ref is None:
            ref = (s_lat, s_ex)
        else:
            np.testing.assert_allclose(s_lat, ref[0], atol=1e-9)
            np.testing.assert_allclose(s_ex, ref[1], atol=1e-9)


def test_brute_force_loops_match_textbook():
    """A pure-Python loop form (explicit sums, math.exp, math.cos/sin) on tiny
    shapes, with dense non-square decoders and several groups."""
    B, H, G, d_h, r_k, r_v, W, base = 2, 4, 2, 4, 6, 5, 2, 10000.0
    sK, sV, q, kc, vc, rk, rv, A, Bv = _random_case(46, B=B, H=H, G=G, d_h=d_h, r_k=r_k, r_v=r_v,
                                                    W=W, n=9, paired=False)
    pos = [8, 1]

    def rot(vec, p):
        half = d_h // 2
        out = list(vec)
        for f in range(half):
            th = base ** (-2.0 * f / d_h)
            a, b = vec[f], vec[f + half]
            out[f] = a * math.cos(p * th) - b * math.sin(p * th)
            out[f + half] = a * math.sin(p * th) + b * math.cos(p * th)
        return out

    want = np.zeros((B, H, d_h))
    for b in range(B):
        i = pos[b]
        for h in range(H):
            g = h // (H // G)
            keys, vals = [], []
            for j in range(i + 1):
                if j < i - W:
                    keys.append([sum(A[h, e, r] * sK[b][j, g, r] for r in range(r_k)) for e in range(d_h)])
                    vals.append([sum(Bv[h, r, e] * sV[b][j, g, r] for r in range(r_v)) for e in range(d_h)])
                elif j < i:
                    keys.append(list(rk[b, j % (W + 1), h]))
                    vals.append(list(rv[b, j % (W + 1), h]))
                else:
                    keys.append(rot(kc[b, h], i))
                    vals.append(list(vc[b, h]))
            qr = rot(q[b, h], i)
            logits = [sum(qr[e] * kk[e] for e in range(d_h)) / math.sqrt(d_h) for kk in keys]
            mx = max(logits)
            w = [math.exp(l - mx) for l in logits]
            s = sum(w)
            for e in range(d_h):
                want[b, h, e] = sum(w[j] * vals[j][e] for j in range(len(keys))) / s
    got = O.textbook_decode(sK, sV, pos, q, kc, vc, rk, rv, A, Bv, window=W, rope_base=base)
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_ring_update_slot_and_rotation():
    pos = np.array([0, 5, 130])
    kc = np.ones((3, 1, 4))
    slot, k, v = O.ring_update(pos, kc, 2 * kc, window=128, rope_base=10000.0)
    assert list(slot) == [0, 5, 1]
    np.testing.assert_allclose(k[2, 0], _complex_rope(np.ones(4), 130, 10000.0), atol=1e-14)
    np.testing.assert_array_equal(v, 2 * kc)


# ---------------------------------------------------------------- full-cache baseline
def _full_cache_case(seed, *, B=3, H=2, d_h=8, P=16, positions=(0, 17, 40), base=10000.0):
    """Random pre-rotation keys / values per sequence, laid into a paged exact
    cache through a permuted block table; unused pages are NaN."""
    g = gen.rng(seed)
    pos = np.asarray(positions)
    pps = int(pos.max()) // P + 1
    n_pages = B * pps + 2
    perm = g.permutation(n_pages)
    bt = perm[: B * pps].reshape(B, pps)
    kp = np.full((n_pages, P, H, d_h), np.nan)
    vp = np.full((n_pages, P, H, d_h), np.nan)
    k_raw = g.standard_normal((B, int(pos.max()) + 1, H, d_h))
    v_raw = g.standard_normal((B, int(pos.max()) + 1, H, d_h))
    for b in range(B):
        for j in range(int(pos[b])):
            kp[bt[b, j // P], j % P] = _complex_rope(k_raw[b, j], j, base)
            vp[bt[b, j // P], j % P] = v_raw[b, j]
    q = g.standard_normal((B, H, d_h))
    kc = g.standard_normal((B, H, d_h))
    vc = g.standard_normal((B, H, d_h))
    return pos, bt, kp, vp, k_raw, v_raw, q, kc, vc


@pytest.mark.parametrize("base", [0.0, 10000.0])
def test_full_cache_equals_sdpa(base):
    """The uncompressed baseline is ordinary attention over tokens 0..i (torch
    SDPA in fp64 on the CPU, keys rotated by the independent complex form)."""
    P = 16
    pos, bt, kp, vp, k_raw, v_raw, q, kc, vc = _full_cache_case(31, P=P, base=base)
    got = O.full_cache_decode(kp, vp, bt, pos, q, kc, vc, page_size=P, rope_base=base)
    for b, i in enumerate(pos):
        k_all = np.concatenate([k_raw[b, :i], kc[b][None]])
        v_all = np.concatenate([v_raw[b, :i], vc[b][None]])
        np.testing.assert_allclose(got[b], _sdpa_reference(k_all, v_all, q[b], int(i), base), atol=1e-12)


def test_full_cache_equals_window_over_whole_context():
    """With a window covering the whole context, the compressed path's exact
    part sees the same tokens: textbook_decode then equals the baseline."""
    P, base = 16, 10000.0
    pos, bt, kp, vp, k_raw, v_raw, q, kc, vc = _full_cache_case(32, P=P, base=base)
    W = int(pos.max())
    B, H, d_h = q.shape
    rk = np.full((B, W + 1, H, d_h), np.nan)
    rv = np.full((B, W + 1, H, d_h), np.nan)
    for b, i in enumerate(pos):
        K, V = O.gather_kv_cache(kp, vp, bt, b, int(i), page_size=P)
        rk[b, : int(i)] = K
        rv[b, : int(i)] = V
    sK = [np.zeros((0, 1, 4))] * B
    sV = [np.zeros((0, 1, 4))] * B
    A = np.zeros((H, d_h, 4))
    Bv = np.zeros((H, 4, d_h))
    want = O.textbook_decode(sK, sV, pos, q, kc, vc, rk, rv, A, Bv, window=W, rope_base=base)
    got = O.full_cache_decode(kp, vp, bt, pos, q, kc, vc, page_size=P, rope_base=base)
    np.testing.assert_allclose(got, want, atol=1e-13)


def test_full_cache_brute_force():
    """Pure-Python loops with math.exp on a tiny case (RoPE off)."""
    P = 4
    d_h = 4
    pos, bt, kp, vp, k_raw, v_raw, q, kc, vc = _full_cache_case(33, B=2, H=2, d_h=d_h, P=P, positions=(5, 2),
                                                               base=0.0)
    got = O.full_cache_decode(kp, vp, bt, pos, q, kc, vc, page_size=P)
    for b, i in enumerate(pos):
        for h in range(2):
            keys = [list(k_raw[b, j, h]) for j in range(i)] + [list(kc[b, h])]
            vals = [list(v_raw[b, j, h]) for j in range(i)] + [list(vc[b, h])]
            s = [sum(q[b, h, e] * k[e] for e in range(d_h)) / math.sqrt(d_h) for k in keys]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            want = [sum(w[j] * vals[j][e] for j in range(len(w))) / sum(w) for e in range(d_h)]
            np.testing.assert_allclose(got[b, h], want, atol=1e-12)


def test_kv_cache_update_page_slot_rotation():
    bt = np.array([[7, 3, 9], [1, 2, 0]])
    pos = np.array([20, 5])
    kc = np.ones((2, 1, 4))
    page, slot, k, v = O.kv_cache_update(pos, kc, 3 * kc, bt, page_size=16, rope_base=500.0)
    assert list(page) == [3, 1] and list(slot) == [4, 5]
    np.testing.assert_allclose(k[0, 0], _complex_rope(np.ones(4), 20, 500.0), atol=1e-14)
    np.testing.assert_array_equal(v, 3 * kc)


# ---------------------------------------------------------------- fp8 latent storage
def _e4m3_brute(x):
    """Nearest finite e4m3 value by exhaustive search over all codes, ties to
    the even mantissa; |x| > 448 saturates."""
    codes = [c for c in range(256) if not ((c >> 3) & 0xF == 15 and c & 7 == 7)]
    vals = O.e4m3_decode(codes)
    out = []
    for v in np.atleast_1d(x):
        v = float(np.clip(v, -448.0, 448.0))
        d = np.abs(vals - v)
        best = [codes[k] for k in np.flatnonzero(d == d.min())]
        if len(best) > 1:                       # a tie: the even mantissa wins
            best = [c for c in best if (c & 1) == 0] or best
        if len(best) > 1:                       # +0 / -0: keep the sign of v
            best = [c for c in best if bool(c & 0x80) == (math.copysign(1.0, v) < 0)]
        out.append(best[0])
    return np.array(out, dtype=np.uint8)


def test_e4m3_closed_forms():
    assert list(O.e4m3_decode([0x38, 0x7E, 0x08, 0x01, 0x07, 0xC0, 0x00])) == \
        [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, -2.0, 0.0]
    assert np.isnan(O.e4m3_decode([0x7F, 0xFF])).all()
    cases = {1.0: 0x38, 1.0625: 0x38, 1.1875: 0x3A, 500.0: 0x7E, -1e9: 0xFE, 2.0 ** -10: 0x00,
             3 * 2.0 ** -10: 0x02, 15.5: 0x58, 447.0: 0x7E, -2.0: 0xC0, 0.0: 0x00}
    for x, c in cases.items():
        assert int(O.e4m3_encode(x)) == c, (x, hex(int(O.e4m3_encode(x))), hex(c))


def test_e4m3_encode_is_nearest_even_by_brute_force():
    g = gen.rng(51)
    x = np.exp2(g.uniform(-12, 9.2, 4000)) * np.where(g.random(4000) < 0.5, -1, 1)
    vals = np.sort(O.e4m3_decode(np.arange(0, 0x7F)))
    mids = (vals[1:] + vals[:-1]) / 2          # every tie point between neighbours
    x = np.concatenate([x, mids, -mids, vals, [449.0, 463.9, 480.0, 1e6]])
    np.testing.assert_array_equal(O.e4m3_encode(x), _e4m3_brute(x))


def test_e4m3_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F and c != 0x80])
    np.testing.assert_array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)


def test_fp8_store_layout_is_a_bijection():
    G, P, r_k, r_v = 2, 32, 64, 128
    kw = dict(groups=G, page_size=P, r_k=r_k, r_v=r_v)
    pg, g, sl = np.meshgrid(np.arange(2), np.arange(G), np.arange(P), indexing="ij")
    pg, g, sl = pg[..., None], g[..., None], sl[..., None]
    k = O.fp8_key_offset(pg, g, sl, np.arange(r_k), **kw).ravel()
    v = O.fp8_value_offset(pg, g, sl, np.arange(r_v), **kw).ravel()
    sc = np.concatenate([O.fp8_scale_offset(pg, g, sl, part, **kw).ravel()[:, None] + np.arange(4)
                         for part in (0, 1)]).ravel()
    allb = np.sort(np.concatenate([k, v, sc]))
    np.testing.assert_array_equal(allb, np.arange(2 * G * (P // 16) * O.fp8_tile_bytes(r_k, r_v)))


def test_fp8_worked_offsets():
    """Offsets worked by hand for G = 1, P = 32, r_k = r_v = 64: a tile is
    16 * 128 code bytes + 64 bytes of key scales + 64 bytes of value scales =
    2176 bytes; slot 19 is token 3 of the page's second tile."""
    kw = dict(groups=1, page_size=32, r_k=64, r_v=64)
    assert O.fp8_tile_bytes(64, 64) == 2176
    assert int(O.fp8_key_offset(1, 0, 19, 10, **kw)) == 2 * 2176 + 2176 + 3 * 64 + 10
    assert int(O.fp8_scale_offset(1, 0, 19, 0, **kw)) == 2 * 2176 + 2176 + 2048 + 3 * 4
    assert int(O.fp8_scale_offset(1, 0, 19, 1, **kw)) == 2 * 2176 + 2176 + 2048 + 64 + 3 * 4
    # value dim 37 = quad 0, sub-block 2, row 5; token 3 = group 0, position 3
    assert int(O.fp8_value_offset(1, 0, 19, 37, **kw)) == 2 * 2176 + 2176 + 1024 + 5 * 64 + 0 * 16 + 2 * 4 + 3


def test_fp8_value_fragment_is_contiguous():
    """Worked offsets: dims 16 j + m of quad 0 for tokens 4 kg .. 4 kg + 3 are
    the 16 bytes at m * 64 + kg * 16 after the key rows (j = 0..3)."""
    kw = dict(groups=1, page_size=16, r_k=64, r_v=64)
    m, kg = 5, 2
    offs = [int(O.fp8_value_offset(0, 0, 4 * kg + t, 16 * j + m, **kw)) for j in range(4) for t in range(4)]
    assert offs == list(range(16 * 64 + m * 64 + kg * 16, 16 * 64 + m * 64 + kg * 16 + 16))


def test_fp8_quantize_rows_and_gather():
    """Scale = max|x| / 448; each element's error is at most half a grid step
    of its binade times the scale; gather decodes through the block table."""
    g = gen.rng(52)
    G, P, r_k, r_v = 2, 16, 64, 64
    n = 20
    c = g.standard_normal((n, G, r_k + r_v)) * 3
    c[3, 1, :r_k] = 0.0                                   # an all-zero part
    kq, ks = O.fp8_quantize_rows(c[..., :r_k])
    vq, vs = O.fp8_quantize_rows(c[..., r_k:])
    np.testing.assert_allclose(ks[0, 0], np.abs(c[0, 0, :r_k]).max() / 448.0, rtol=1e-15)
    assert ks[3, 1] == 1.0 and not kq[3, 1].any()
    for q, sc, x in ((kq, ks, c[..., :r_k]), (vq, vs, c[..., r_k:])):
        y = x / sc[..., None]
        step = 2.0 ** (np.clip(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -9))), -6, 8) - 3)
        assert np.all(np.abs(O.e4m3_decode(q) - y) <= step / 2 + 1e-12)
    bt = np.array([[1, 0]])
    nbytes = 2 * G * (P // 16) * O.fp8_tile_bytes(r_k, r_v)
    raw = np.zeros(nbytes, dtype=np.uint8)
    kw = dict(groups=G, page_size=P, r_k=r_k, r_v=r_v)
    for j in range(n):
        for gg in range(G):
            pg, sl = bt[0, j // P], j % P
            raw[O.fp8_key_offset(pg, gg, sl, np.arange(r_k), **kw)] = kq[j, gg]
            raw[O.fp8_value_offset(pg, gg, sl, np.arange(r_v), **kw)] = vq[j, gg]
            for part, sc in ((0, ks), (1, vs)):
                o = int(O.fp8_scale_offset(pg, gg, sl, part, **kw))
                raw[o:o + 4] = np.frombuffer(np.float32(sc[j, gg]).tobytes(), dtype=np.uint8)
    sK, sV = O.gather_latents_fp8(raw, bt, 0, n, **kw)
    np.testing.assert_allclose(sK, O.e4m3_decode(kq) * ks.astype(np.float32)[..., None], rtol=0, atol=0)
    np.testing.assert_allclose(sV, O.e4m3_decode(vq) * vs.astype(np.float32)[..., None], rtol=0, atol=0)


# ---------------------------------------------------------------- parallel pass
def _causal_sdpa(q, k, v, base):
    """Causal attention over whole sequences: torch's scaled dot product
    attention (fp64, CPU, is_causal) on R_i q_i and R_j k_j.  q, k, v [n, H, d_h]."""
    n = q.shape[0]
    qr = _complex_rope(q, np.arange(n)[:, None], base)
    kr = _complex_rope(k, np.arange(n)[:, None], base)
    t = lambda a: torch.from_numpy(a.transpose(1, 0, 2).copy())[None]
    o = torch.nn.functional.scaled_dot_product_attention(t(qr), t(kr), t(v), is_causal=True)
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("t", [1, 2, 3])
@pytest.mark.parametrize("W", [0, 2, 5, 20])
def test_parallel_identity_codec_equals_causal_attention(t, W):
    """Under a full-rank identity codec the parallel pass is causal attention
    over the loop's exact keys and values at every position, for every W."""
    base, n = 10000.0, 12
    k, v, _, maps = _identity_hla(61, n_tok=n, base=base)
    q = gen.rng(62).standard_normal((n,) + k.shape[2:])
    sK, sV, A, Bv = maps(t)
    out = O.parallel_attention([sK], [sV], [n], q[None], k[t - 1][None], v[t - 1][None], A, Bv, window=W,
                               rope_base=base)
    np.testing.assert_allclose(out[0], _causal_sdpa(q, k[t - 1], v[t - 1], base), atol=1e-12)


def _parallel_case(seed, *, B=2, n=20, H=4, G=2, d_h=8, r_k=16, r_v=12, base=10000.0):
    g = gen.rng(seed)
    sK = [g.standard_normal((n, G, r_k)) for _ in range(B)]
    sV = [g.standard_normal((n, G, r_v)) for _ in range(B)]
    q, k, v = (g.standard_normal((B, n, H, d_h)) for _ in range(3))
    A = gen.frequency_paired_decoder(g, H, d_h, r_k) if base else \
        np.stack([gen.gaussian_orthonormal(g, d_h, r_k) for _ in range(H)])
    Bv = np.stack([gen.gaussian_orthonormal(g, r_v, d_h) for _ in range(H)])
    return sK, sV, q, k, v, A, Bv


@pytest.mark.parametrize("W", [0, 3, 7])
def test_parallel_equals_decode_at_every_position(W):
    """Each position of the parallel pass is one decode call: the ring holds
    R_j k_j, v_j of the W tokens before i and the current token is k_i, v_i."""
    base = 10000.0
    sK, sV, q, k, v, A, Bv = _parallel_case(63, base=base)
    n_tok = [20, 13]
    out = O.parallel_attention(sK, sV, n_tok, q, k, v, A, Bv, window=W, rope_base=base)
    for b in range(2):
        for i in range(n_tok[b]):
            rk, rv = _ring(k[b], v[b], i, W, base)
            want = O.absorbed_decode([sK[b]], [sV[b]], [i], q[b, i][None], k[b, i][None], v[b, i][None],
                                     rk, rv, A, Bv, window=W, rope_base=base)
            np.testing.assert_allclose(out[b, i], want[0], atol=1e-12)
        assert np.all(out[b, n_tok[b]:] == 0)


def test_parallel_window_over_whole_sequence_ignores_latents():
    """W >= n-1: no position reads a latent (NaN latents stay unread) and the
    pass is causal attention over the exact keys and values."""
    base, n = 10000.0, 9
    sK, sV, q, k, v, A, Bv = _parallel_case(64, B=1, n=n, base=base)
    sK[0][:] = np.nan
    sV[0][:] = np.nan
    out = O.parallel_attention(sK, sV, [n], q, k, v, A, Bv, window=n - 1, rope_base=base)
    np.testing.assert_allclose(out[0], _causal_sdpa(q[0], k[0], v[0], base), atol=1e-12)


def test_parallel_rows_subset_and_ragged_lengths():
    """Evaluating a subset of rows gives the same rows as the whole pass."""
    sK, sV, q, k, v, A, Bv = _parallel_case(65)
    full = O.parallel_attention(sK, sV, [20, 7], q, k, v, A, Bv, window=3, rope_base=10000.0)
    sub = O.parallel_attention(sK, sV, [20, 7], q, k, v, A, Bv, window=3, rope_base=10000.0,
                               rows=[(0, 19), (1, 0), (1, 6)])
    for b, i in [(0, 19), (1, 0), (1, 6)]:
        np.testing.assert_array_equal(sub[b, i], full[b, i])
    assert np.all(sub[0, :19] == 0)


def test_parallel_brute_force():
    """Pure-Python loops (math.cos / sin / exp, explicit sums) on a tiny case:
    one group, d_h = 4, r_k = r_v = 8, W = 2, rotary on."""
    base, W, n, H, d_h, r = 10000.0, 2, 6, 2, 4, 8
    sK, sV, q, k, v, A, Bv = _parallel_case(66, B=1, n=n, H=H, G=1, d_h=d_h, r_k=r, r_v=r, base=base)
    out = O.parallel_attention(sK, sV, [n], q, k, v, A, Bv, window=W, rope_base=base)

    def rot(vec, p):   # rotate-half pairs (f, f + d/2), theta_f = base^(-2f/d)
        d = len(vec)
        res = list(vec)
        for f in range(d // 2):
            th = p * base ** (-2.0 * f / d)
            a, b2 = vec[f], vec[f + d // 2]
            res[f] = a * math.cos(th) - b2 * math.sin(th)
            res[f + d // 2] = a * math.sin(th) + b2 * math.cos(th)
        return res

    for h in range(H):
        for i in range(n):
            logits, vals = [], []
            # latent tokens: score (R~_i A^T q) . sK_j / sqrt(d), value B^T sV_j
            at_q = [sum(A[h][e][c] * q[0, i, h, e] for e in range(d_h)) for c in range(r)]
            qt = rot(at_q[:4], i) + rot(at_q[4:], i)
            for j in range(max(0, i - W)):
                logits.append(sum(qt[c] * sK[0][j, 0, c] for c in range(r)) / math.sqrt(d_h))
                vals.append([sum(Bv[h][c][e] * sV[0][j, 0, c] for c in range(r)) for e in range(d_h)])
            qr = rot(list(q[0, i, h]), i)
            for j in range(max(0, i - W), i + 1):
                kr = rot(list(k[0, j, h]), j)
                logits.append(sum(qr[e] * kr[e] for e in range(d_h)) / math.sqrt(d_h))
                vals.append(list(v[0, j, h]))
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            z = sum(w)
            want = [sum(w[u] * vals[u][e] for u in range(len(w))) / z for e in range(d_h)]
            np.testing.assert_allclose(out[0, i, h], want, atol=1e-12)
