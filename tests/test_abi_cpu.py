"""Host-only checks of the C-ABI library: it loads, exports every function
include/lla.h declares, and rejects invalid arguments with the documented
status before anything is enqueued (these calls never reach a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from compressed_cross_loop_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lla.h")

FAKE = 0x10000  # aligned, non-null, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:lla_status|size_t|int32_t|const char\s*\*)\s+(\w+)\s*\(",
                                 text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    assert B.lla_abi_version() == 5 == B.ABI_VERSION
    for s in range(5):
        assert B.lla_status_string(s)
    assert B.lla_status_string(99) == "unknown status"


def hla_main(**kw):
    d = dict(n_heads=16, head_dim=128, groups=1, r_k=512, r_v=512, loop_first=2, loop_last=4,
             page_size=64, rope_baked=1, rope_base=10000.0, dtype=B.LLA_BF16)
    d.update(kw)
    return B.set_desc(**d)


def test_bytes_per_token_matches_closed_form():
    main = hla_main()
    one = hla_main(r_k=256, r_v=256, loop_first=1, loop_last=1)
    per_layer = B.lla_bytes_per_token(main) + B.lla_bytes_per_token(one)
    assert 24 * per_layer == O.hla_bytes_per_token(24, 512, 512, 256, 2) == 72 * 1024
    lla = hla_main(groups=16, r_k=32, r_v=32, loop_first=1, loop_last=4, rope_baked=0, rope_base=0.0)
    assert B.lla_bytes_per_token(lla) == O.set_bytes_per_token(16, 32, 32, 2)
    f32 = hla_main(dtype=B.LLA_F32)
    assert B.lla_bytes_per_token(f32) == 2 * B.lla_bytes_per_token(main)


@pytest.mark.parametrize("bad", [
    dict(n_heads=0), dict(head_dim=127), dict(groups=3), dict(r_k=500), dict(r_v=0),
    dict(loop_first=0), dict(loop_first=3, loop_last=2), dict(page_size=40), dict(dtype=7),
    dict(rope_base=-1.0), dict(rope_baked=2), dict(rope_baked=1, rope_base=0.0),
])
def test_invalid_descriptor(bad):
    d = hla_main(**bad)
    assert B.lla_bytes_per_token(d) == 0
    assert B.lla_decode_workspace_bytes(d, 4, 100, 16) == 0


def test_unsupported_descriptor():
    # rope baked into a key latent that is not whole d_h blocks
    d = hla_main(r_k=96, r_v=96)
    st = B.LlaStore(FAKE, FAKE, 4)
    args = B.LlaDecodeArgs(2, 16, 100, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert B.lib.hla_decode_windowed(ctypes.byref(d), ctypes.byref(st), 4, ctypes.byref(args), None) \
        == B.LLA_ERR_UNSUPPORTED
    big = hla_main(head_dim=512, r_k=512)
    assert B.lib.hla_decode_windowed(ctypes.byref(big), ctypes.byref(st), 4, ctypes.byref(args), None) \
        == B.LLA_ERR_UNSUPPORTED


def _args(**kw):
    a = dict(loop=2, window=16, max_pos_hint=100, splits=0, flags=0, pos=FAKE, q=FAKE, k_cur=FAKE,
             v_cur=FAKE, ring_k=FAKE, ring_v=FAKE, A=FAKE, B=FAKE, out=FAKE, workspace=FAKE,
             workspace_bytes=1 << 40, scan_events=None)
    a.update(kw)
    return B.LlaDecodeArgs(*[a[f] for f, _ in B.LlaDecodeArgs._fields_])


ENTRIES = ["lla_decode_reconstruct", "lla_decode_absorbed", "hla_decode_windowed"]


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("bad, want", [
    (dict(loop=1), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(loop=5), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(window=-1), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(splits=-2), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(flags=8), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(q=None), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(ring_v=None), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(out=FAKE + 2), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(pos=None), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(window=100000), B.LLA_ERR_UNSUPPORTED),
    (dict(workspace=None), B.LLA_ERR_WORKSPACE_TOO_SMALL),
    (dict(workspace_bytes=1024), B.LLA_ERR_WORKSPACE_TOO_SMALL),
])
def test_decode_argument_errors(entry, bad, want):
    d = hla_main()
    st = B.LlaStore(FAKE, FAKE, 4)
    fn = getattr(B.lib, entry)
    assert fn(ctypes.byref(d), ctypes.byref(st), 4, ctypes.byref(_args(**bad)), None) == want


@pytest.mark.parametrize("entry", ENTRIES)
def test_decode_null_struct_and_store(entry):
    d = hla_main()
    fn = getattr(B.lib, entry)
    st = B.LlaStore(FAKE, FAKE, 4)
    a = _args(workspace_bytes=1024)
    assert fn(None, ctypes.byref(st), 4, ctypes.byref(a), None) == B.LLA_ERR_INVALID_ARGUMENT
    assert fn(ctypes.byref(d), None, 4, ctypes.byref(a), None) == B.LLA_ERR_INVALID_ARGUMENT
    assert fn(ctypes.byref(d), ctypes.byref(st), 4, None, None) == B.LLA_ERR_INVALID_ARGUMENT
    assert fn(ctypes.byref(d), ctypes.byref(st), 0, ctypes.byref(a), None) == B.LLA_ERR_INVALID_ARGUMENT
    for bad in (B.LlaStore(None, FAKE, 4), B.LlaStore(FAKE, None, 4), B.LlaStore(FAKE, FAKE, 0),
                B.LlaStore(FAKE + 8, FAKE, 4)):
        assert fn(ctypes.byref(d), ctypes.byref(bad), 4, ctypes.byref(a), None) == B.LLA_ERR_INVALID_ARGUMENT


def test_hla_requires_one_group_and_rotation_needs_baking():
    st = B.LlaStore(FAKE, FAKE, 4)
    per_head = hla_main(groups=16, r_k=32, r_v=32, rope_baked=0, rope_base=0.0, loop_first=1)
    a = _args()
    assert B.lib.hla_decode_windowed(ctypes.byref(per_head), ctypes.byref(st), 4, ctypes.byref(a), None) \
        == B.LLA_ERR_INVALID_ARGUMENT
    unbaked = hla_main(rope_baked=0)
    for entry in ("lla_decode_reconstruct", "lla_decode_absorbed"):
        assert getattr(B.lib, entry)(ctypes.byref(unbaked), ctypes.byref(st), 4, ctypes.byref(a), None) \
            == B.LLA_ERR_UNSUPPORTED


def test_writer_argument_errors():
    d = hla_main()
    st = B.LlaStore(FAKE, FAKE, 4)
    f = B.lib.lla_write_latents
    ok = (ctypes.byref(d), ctypes.byref(st), 4, 1, FAKE, FAKE, 2048, FAKE, None, 0, None)

    def call(**kw):
        a = list(ok)
        names = ["desc", "store", "batch", "n_tok", "pos", "x", "d_in", "enc", "ws", "wsb", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(batch=0) == B.LLA_ERR_INVALID_ARGUMENT
    assert call(n_tok=0) == B.LLA_ERR_INVALID_ARGUMENT
    assert call(d_in=0) == B.LLA_ERR_INVALID_ARGUMENT
    assert call(pos=None) == B.LLA_ERR_INVALID_ARGUMENT
    assert call(x=FAKE + 4) == B.LLA_ERR_INVALID_ARGUMENT
    assert call(enc=None) == B.LLA_ERR_INVALID_ARGUMENT
    assert call(desc=None) == B.LLA_ERR_INVALID_ARGUMENT
    assert call(store=None) == B.LLA_ERR_INVALID_ARGUMENT


def test_workspace_and_plan():
    d = hla_main()
    # workspace grows with batch and context; the plan never exceeds the tile count
    assert B.lla_decode_workspace_bytes(d, 128, 4095, 128) > B.lla_decode_workspace_bytes(d, 32, 4095, 128)
    assert B.lla_decode_plan_splits(d, 1, 10, 16) == 1          # no latent tokens: one empty split
    assert B.lla_decode_plan_splits(d, 1, 4095, 128, splits=1000) == (4095 - 128 + 63) // 64
    assert B.lla_decode_plan_splits(d, 128, 4095, 128, splits=3) == 3
    for b, ctx in ((128, 4096), (32, 16384), (1, 256)):
        s = B.lla_decode_plan_splits(d, b, ctx - 1, 128)
        assert 1 <= s <= max(1, (ctx - 1 - 128 + 63) // 64)


def test_scan_kernel_query():
    """The library names the latent-scan kernel family it would launch."""
    def desc(dtype, G, H, r, dh):
        return B.set_desc(n_heads=H, head_dim=dh, groups=G, r_k=r, r_v=r, loop_first=1, loop_last=4,
                          page_size=64, rope_baked=0, rope_base=0.0, dtype=dtype)
    hla = desc(B.LLA_BF16, 1, 16, 512, 128)
    assert B.lla_decode_scan_kernel(hla, 2) == "k_scan_absorbed_mfma"
    assert B.lla_decode_scan_kernel(hla, 1) == "k_scan_absorbed_mfma"
    assert B.lla_decode_scan_kernel(hla, 2, B.LLA_FLAG_GENERIC) == "k_scan_absorbed_generic"
    assert B.lla_decode_scan_kernel(hla, 0) == "k_scan_reconstruct_gemm"
    per_head = desc(B.LLA_BF16, 16, 16, 32, 128)
    assert B.lla_decode_scan_kernel(per_head, 0) == "k_scan_reconstruct_mfma"
    assert B.lla_decode_scan_kernel(per_head, 0, B.LLA_FLAG_GENERIC) == "k_scan_reconstruct_generic"
    tiny = desc(B.LLA_F32, 1, 2, 128, 64)   # fp32 storage: general kernels only
    assert B.lla_decode_scan_kernel(tiny, 1) == "k_scan_absorbed_generic"
    assert B.lla_decode_scan_kernel(tiny, 0) == "k_scan_reconstruct_generic"
    wide = desc(B.LLA_BF16, 1, 55, 5280, 96)
    assert B.lla_decode_scan_kernel(wide, 0) == "k_scan_reconstruct_gemm"
    assert B.lla_decode_scan_kernel(wide, 1) == "k_scan_absorbed_wide"
    assert B.lla_decode_scan_kernel(wide, 1, B.LLA_FLAG_GENERIC) == "k_scan_absorbed_generic"
    # the two-pass form takes shared latents only, up to 64 heads, r_k % 32 == 0
    assert B.lla_decode_scan_kernel(desc(B.LLA_BF16, 1, 65, 256, 64), 1) == "k_scan_absorbed_generic"
    assert B.lla_decode_scan_kernel(desc(B.LLA_BF16, 1, 64, 256, 64), 1) == "k_scan_absorbed_wide"
    assert B.lla_decode_scan_kernel(desc(B.LLA_BF16, 1, 4, 48, 64), 1) == "k_scan_absorbed_generic"
    assert B.lla_decode_scan_kernel(desc(B.LLA_BF16, 2, 4, 1024, 64), 1) == "k_scan_absorbed_generic"
    assert B.lla_decode_scan_kernel(desc(B.LLA_F32, 1, 55, 5280, 96), 1) == "k_scan_absorbed_generic"
    assert B.lla_decode_scan_kernel(hla, 3) is None
    assert B.lla_decode_scan_kernel(hla, 0, 2) is None
    bad = desc(B.LLA_BF16, 1, 16, 512, 128)
    bad.head_dim = 0
    assert B.lla_decode_scan_kernel(bad, 0) is None


def test_scan_kernel_query_for_store():
    """A block table longer than a matrix-core scan stages in LDS (8192 page ids
    for the absorbed scans, 4096 for the per-head reconstruct scan), or a store
    holding more tokens than the wide scan's score rows cover, takes the
    general scan; the store-free query names the matrix-core kernel."""
    def desc(G, H, r, dh, P=64):
        return B.set_desc(n_heads=H, head_dim=dh, groups=G, r_k=r, r_v=r, loop_first=1, loop_last=4,
                          page_size=P, rope_baked=0, rope_base=0.0, dtype=B.LLA_BF16)
    q = B.lla_decode_scan_kernel_for_store
    per_head = desc(16, 16, 32, 128, P=16)
    assert q(per_head, 0, 100, 4096) == "k_scan_reconstruct_mfma"
    assert q(per_head, 0, 100, 4097) == "k_scan_reconstruct_generic"
    assert q(per_head, 1, 100, 8192) == "k_scan_absorbed_mfma"
    assert q(per_head, 1, 100, 8193) == "k_scan_absorbed_generic"
    hla = desc(1, 16, 256, 128, P=16)
    assert q(hla, 2, 100, 8193) == "k_scan_absorbed_generic"
    assert q(hla, 2, 100, 8192) == "k_scan_absorbed_mfma"
    # the wide scan: score rows of max_pos_hint + 1 tokens rounded up to 512
    wide = desc(1, 6, 192, 96)
    assert q(wide, 1, 100, 8) == "k_scan_absorbed_wide"        # 512 tokens
    assert q(wide, 1, 100, 9) == "k_scan_absorbed_generic"     # 576 > 512
    assert q(wide, 1, 600, 16) == "k_scan_absorbed_wide"       # 1024 rows
    assert q(wide, 1, 100, 8, B.LLA_FLAG_GENERIC) == "k_scan_absorbed_generic"
    assert q(wide, 1, -1, 8) is None and q(wide, 1, 100, 0) is None


def _kv(**kw):
    base = dict(n_heads=16, head_dim=128, page_size=64, rope_base=10000.0, dtype=B.LLA_BF16)
    base.update(kw)
    return B.kv_desc(**base)


def _full_call(desc=None, cache="ok", batch=2, **kw):
    d = desc if desc is not None else _kv()
    c = B.LlaKvCache(FAKE, FAKE, FAKE, 4) if cache == "ok" else cache
    a = dict(max_pos_hint=100, splits=0, flags=0, pos=FAKE, q=FAKE, k_cur=FAKE, v_cur=FAKE, out=FAKE,
             workspace=FAKE, workspace_bytes=1 << 40, scan_events=None)
    a.update(kw)
    args = B.LlaFullDecodeArgs(*[a[f] for f, _ in B.LlaFullDecodeArgs._fields_])
    return B.lib.lla_decode_full_cache(ctypes.byref(d) if d is not None else None,
                                       ctypes.byref(c) if c is not None else None, batch,
                                       ctypes.byref(args), None)


@pytest.mark.parametrize("bad, want", [
    (dict(head_dim=96), B.LLA_ERR_UNSUPPORTED),
    (dict(head_dim=0), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(n_heads=0), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(page_size=12), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(rope_base=-1.0), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), B.LLA_ERR_INVALID_ARGUMENT),
])
def test_full_cache_descriptor_errors(bad, want):
    assert _full_call(desc=_kv(**bad)) == want
    assert B.lla_full_decode_workspace_bytes(_kv(**bad), 2, 100) == 0


@pytest.mark.parametrize("kw, want", [
    (dict(flags=1), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(q=None), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(out=FAKE + 4), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(splits=-1), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(workspace_bytes=16), B.LLA_ERR_WORKSPACE_TOO_SMALL),
    (dict(workspace=None), B.LLA_ERR_WORKSPACE_TOO_SMALL),
])
def test_full_cache_argument_errors(kw, want):
    assert _full_call(**kw) == want


def test_full_cache_null_structs_and_plan():
    assert _full_call(cache=None) == B.LLA_ERR_INVALID_ARGUMENT
    assert _full_call(cache=B.LlaKvCache(FAKE, None, FAKE, 4)) == B.LLA_ERR_INVALID_ARGUMENT
    assert _full_call(cache=B.LlaKvCache(FAKE, FAKE, FAKE, 0)) == B.LLA_ERR_INVALID_ARGUMENT
    assert _full_call(batch=0) == B.LLA_ERR_INVALID_ARGUMENT
    d = _kv()
    assert B.lla_full_decode_plan_splits(d, 1, 10) == 1
    assert B.lla_full_decode_plan_splits(d, 32, 4095, splits=5) == 5
    assert B.lla_full_decode_workspace_bytes(d, 32, 4095, 4) > B.lla_full_decode_workspace_bytes(d, 8, 4095, 4) > 0


def test_fp8_descriptor_rules_and_bytes_per_token():
    def d(**kw):
        base = dict(n_heads=16, head_dim=128, groups=1, r_k=512, r_v=512, loop_first=2, loop_last=4,
                    page_size=64, rope_baked=1, rope_base=10000.0, dtype=B.LLA_BF16, latent_fp8=1)
        base.update(kw)
        return B.set_desc(**base)
    assert B.lla_bytes_per_token(d()) == 512 + 512 + 8
    assert B.lla_bytes_per_token(d(groups=16, n_heads=16, r_k=64, r_v=64, rope_baked=0, rope_base=0.0)) == \
        16 * (64 + 64 + 8)
    assert B.store_bytes(d(), 3) == 3 * 4 * (16 * 1024 + 128)
    for bad, want in ((dict(latent_fp8=2), B.LLA_ERR_INVALID_ARGUMENT),
                      (dict(dtype=B.LLA_F32), B.LLA_ERR_INVALID_ARGUMENT),
                      (dict(r_k=96, r_v=96, rope_baked=0, rope_base=0.0), B.LLA_ERR_UNSUPPORTED)):
        assert B.lla_bytes_per_token(d(**bad)) == 0
        assert B.lla_decode_workspace_bytes(d(**bad), 2, 100, 16) == 0
    # fp8 latents are read by the absorbed entry points only
    assert B.lla_decode_scan_kernel(d(), 2) == "k_scan_absorbed_mfma"


def test_fp8_reconstruct_is_unsupported():
    d = hla_main()
    d.latent_fp8 = 1
    st = B.LlaStore(FAKE, FAKE, 4)
    assert B.lib.lla_decode_reconstruct(ctypes.byref(d), ctypes.byref(st), 4, ctypes.byref(_args()), None) \
        == B.LLA_ERR_UNSUPPORTED


def _par_call(desc="ok", store="ok", batch=2, **kw):
    d = hla_main() if isinstance(desc, str) else desc
    st = B.LlaStore(FAKE, FAKE, 64) if store == "ok" else store
    a = dict(loop=3, window=128, n_max=4096, flags=0, n_tok=FAKE, q=FAKE, k=FAKE, v=FAKE, A=FAKE, B=FAKE,
             out=FAKE, workspace=FAKE, workspace_bytes=1 << 40, attn_events=None)
    a.update(kw)
    args = B.LlaParallelArgs(*[a[f] for f, _ in B.LlaParallelArgs._fields_])
    return B.lib.hla_attention_parallel(ctypes.byref(d) if d is not None else None,
                                        ctypes.byref(st) if st is not None else None, batch,
                                        ctypes.byref(args), None)


@pytest.mark.parametrize("bad, want", [
    (dict(dtype=B.LLA_F32), B.LLA_ERR_UNSUPPORTED),
    (dict(latent_fp8=1), B.LLA_ERR_UNSUPPORTED),
    (dict(head_dim=96, r_k=480, r_v=480), B.LLA_ERR_UNSUPPORTED),
    (dict(r_k=496, rope_baked=0, rope_base=0.0), B.LLA_ERR_UNSUPPORTED),
    (dict(rope_baked=0), B.LLA_ERR_UNSUPPORTED),
    (dict(groups=3), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(page_size=8), B.LLA_ERR_INVALID_ARGUMENT),
])
def test_parallel_descriptor_errors(bad, want):
    assert _par_call(desc=hla_main(**bad)) == want
    assert B.lla_parallel_workspace_bytes(hla_main(**bad), 2, 100) == 0


@pytest.mark.parametrize("kw, want", [
    (dict(flags=1), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(loop=1), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(loop=5), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(window=-1), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(n_max=0), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(n_tok=None), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(v=FAKE + 2), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(B=None), B.LLA_ERR_INVALID_ARGUMENT),
    (dict(n_max=64 * 64 + 130), B.LLA_ERR_INVALID_ARGUMENT),       # block table covers 4096 latent tokens
    (dict(workspace_bytes=1 << 20), B.LLA_ERR_WORKSPACE_TOO_SMALL),
    (dict(workspace=None), B.LLA_ERR_WORKSPACE_TOO_SMALL),
    (dict(workspace=FAKE + 8), B.LLA_ERR_INVALID_ARGUMENT),
])
def test_parallel_argument_errors(kw, want):
    assert _par_call(**kw) == want


def test_parallel_null_structs_and_workspace():
    assert _par_call(desc=None) == B.LLA_ERR_INVALID_ARGUMENT
    assert _par_call(store=None) == B.LLA_ERR_INVALID_ARGUMENT
    assert _par_call(store=B.LlaStore(FAKE, FAKE, 0)) == B.LLA_ERR_INVALID_ARGUMENT
    assert _par_call(batch=0) == B.LLA_ERR_INVALID_ARGUMENT
    d = hla_main()
    # W + 1 >= n_max: no latent is read, so any block table will do
    assert _par_call(store=B.LlaStore(FAKE, FAKE, 1), n_max=129, workspace_bytes=16) == \
        B.LLA_ERR_WORKSPACE_TOO_SMALL
    w = B.lla_parallel_workspace_bytes
    assert w(d, 2, 100) == w(d, 2, 256) < w(d, 2, 257) < w(d, 4, 257)
    # rebuilt keys and values: 2 head-space rows of bf16 per padded position,
    # the gathered latents, and the (cos, sin) table (d_h / 2 fp32 pairs per
    # position)
    assert w(d, 1, 256) >= 256 * (2 * 16 * 128 + 1024) * 2 + 256 * 64 * 8
    assert w(d, 0, 256) == 0 and w(d, 1, 0) == 0


def test_fused_flag_rules():
    """LLA_FLAG_FUSED: absorbed / HLA entries on supported bf16 shapes only,
    never together with LLA_FLAG_GENERIC (all rejected before any launch)."""
    st = B.LlaStore(FAKE, FAKE, 4)
    F, Gn = B.LLA_FLAG_FUSED, B.LLA_FLAG_GENERIC

    def call(entry, d, flags):
        return getattr(B.lib, entry)(ctypes.byref(d), ctypes.byref(st), 4,
                                     ctypes.byref(_args(flags=flags, workspace_bytes=16)), None)
    d = hla_main()
    assert call("hla_decode_windowed", d, F | Gn) == B.LLA_ERR_INVALID_ARGUMENT
    assert call("lla_decode_reconstruct", d, F) == B.LLA_ERR_UNSUPPORTED
    for bad in (hla_main(dtype=B.LLA_F32), hla_main(latent_fp8=1), hla_main(r_k=512, r_v=256),
                hla_main(r_k=64, r_v=64, rope_baked=0, rope_base=0.0), hla_main(head_dim=256, r_k=512, r_v=512)):
        assert call("lla_decode_absorbed", bad, F) == B.LLA_ERR_UNSUPPORTED
    # a supported shape gets as far as the workspace check
    assert call("hla_decode_windowed", d, F) == B.LLA_ERR_WORKSPACE_TOO_SMALL
    assert B.lla_decode_scan_kernel(d, 2, F) == "k_fused_decode"
    assert B.lla_decode_scan_kernel(d, 0, F) is None
    assert B.lla_decode_scan_kernel(d, 2, F | Gn) is None
    assert B.lla_decode_scan_kernel(hla_main(r_k=64, r_v=64, rope_baked=0, rope_base=0.0), 1, F) is None


def test_decode_workspace_holds_regrouped_decoders():
    """Head-folded bf16 sets with d_h 64 or 96 reserve a copy of A_t and B_t^T
    (2 H d_h r_k bf16) in the decode workspace for the LDS-staged reconstruct;
    other shapes do not."""
    def desc(G, H, r, dh):
        return B.set_desc(n_heads=H, head_dim=dh, groups=G, r_k=r, r_v=r, loop_first=1, loop_last=4,
                          page_size=64, rope_baked=0, rope_base=0.0, dtype=B.LLA_BF16)
    w = B.lla_decode_workspace_bytes
    wide = desc(1, 55, 5280, 96)
    assert w(wide, 64, 4095, 0) >= 2 * 55 * 96 * 5280 * 2
    # the copy is the only region that grows with H d_h r_k alone: at batch 1
    # and a short context it dominates (the rest is mostly the split score
    # rows of the absorbed read: 42 parts x 55 heads x 512 tokens x 4 bytes)
    small = w(wide, 1, 200, 0)
    assert 2 * 55 * 96 * 5280 * 2 <= small < 2 * 55 * 96 * 5280 * 2 + 16 * 1024 * 1024
    # per-head latents (groups == heads) never take the head-folded path
    per_head = desc(16, 16, 32, 128)
    assert w(per_head, 1, 200, 0) < 2 * 16 * 128 * 32 * 2


def test_decode_workspace_holds_wide_scan_rows():
    """The two-pass absorbed scan of a wide shared latent keeps an fp32 score and
    a bf16 probability per (sequence, head, token) up to max_pos + 1 rounded up
    to 512 tokens; the one-pass shapes keep none."""
    def desc(G, H, r, dh):
        return B.set_desc(n_heads=H, head_dim=dh, groups=G, r_k=r, r_v=r, loop_first=1, loop_last=4,
                          page_size=64, rope_baked=0, rope_base=0.0, dtype=B.LLA_BF16)
    w = B.lla_decode_workspace_bytes
    wide = desc(1, 55, 5280, 96)
    rows = 64 * 55 * 4096 * 6
    assert w(wide, 64, 4095, 0) >= rows + 2 * 55 * 96 * 5280 * 2
    # and q~ as bf16 hi and lo parts (the lo part follows the hi part)
    assert w(wide, 64, 4095, 0) >= rows + 2 * 55 * 96 * 5280 * 2 + 2 * 64 * 55 * 5280 * 2
    assert w(wide, 64, 4096, 0) - w(wide, 64, 4095, 0) >= 64 * 55 * 256 * 6
    hla = desc(1, 16, 512, 128)   # one-pass matrix-core scan: nothing per token
    assert w(hla, 128, 4095, 128) < 128 * 16 * 4096 * 6


def test_check_indices_on_host_copies():
    """The host-side index check: positions inside the block table's reach and
    block-table entries of the pages in use inside the store; nothing beyond
    the current position's page is inspected."""
    bt = np.array([[3, 0, 7, -1], [1, 2, 4, 5]], dtype=np.int32)
    ok = B.LLA_OK
    assert B.lla_check_indices([130, 255], bt, n_pages=8, page_size=64) == ok
    assert B.lla_check_indices([256, 0], bt, n_pages=8, page_size=64) == B.LLA_ERR_INVALID_ARGUMENT   # past the table
    assert B.lla_check_indices([-1, 0], bt, n_pages=8, page_size=64) == B.LLA_ERR_INVALID_ARGUMENT
    assert B.lla_check_indices([192, 0], bt, n_pages=8, page_size=64) == B.LLA_ERR_INVALID_ARGUMENT   # page id -1
    assert B.lla_check_indices([130, 255], bt, n_pages=7, page_size=64) == B.LLA_ERR_INVALID_ARGUMENT  # id 7 of 7
    assert B.lla_check_indices([63, 0], bt, n_pages=4, page_size=64) == ok                           # only page 0 used
