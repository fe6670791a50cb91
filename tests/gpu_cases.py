"""Run one decode or writer call through the C ABI on the GPU, and compute the
oracle's expectation for the same seeded inputs."""
import numpy as np
import torch

import oracle as O
from compressed_cross_loop_amd import binding as B
from synth import gen

ENTRY = {
    "reconstruct": B.lla_decode_reconstruct,
    "absorbed": B.lla_decode_absorbed,
    "hla": B.hla_decode_windowed,
}
TOL = {"f32": 1e-5, "bf16": 2e-2}


def desc_of(c: gen.DecodeInputs):
    return B.set_desc(n_heads=c.heads, head_dim=c.head_dim, groups=c.groups, r_k=c.r_k, r_v=c.r_v,
                      loop_first=c.loop_first, loop_last=c.loop_last, page_size=c.page_size,
                      rope_baked=c.rope_baked, rope_base=c.rope_base,
                      dtype=B.LLA_BF16 if c.dtype == "bf16" else B.LLA_F32)


def poison_unread(c: gen.DecodeInputs):
    """NaN into every store element and ring slot the call must not read:
    tokens at or past max(0, i-W), pages no sequence owns, and the ring slot
    the call overwrites (plus slots of positions that do not exist yet)."""
    pages = c.pages.clone()
    flat = pages.view(-1)
    kw = dict(groups=c.groups, page_size=c.page_size, r_k=c.r_k, r_v=c.r_v)
    bt = c.block_table.numpy()
    owned = set(bt.ravel().tolist())
    for pg in range(c.n_pages):
        if pg not in owned:
            pages[pg] = float("nan")
    for b in range(c.batch):
        i = int(c.pos[b])
        n_lat = max(0, i - c.window)
        j = np.arange(n_lat, bt.shape[1] * c.page_size)
        if j.size == 0:
            continue
        page = bt[b, j // c.page_size].astype(np.int64)
        slot = j % c.page_size
        for gg in range(c.groups):
            ko = O.store_key_offset(page[:, None], gg, slot[:, None], np.arange(c.r_k)[None], **kw)
            vo = O.store_value_offset(page[:, None], gg, slot[:, None], np.arange(c.r_v)[None], **kw)
            flat[torch.from_numpy(ko.ravel())] = float("nan")
            flat[torch.from_numpy(vo.ravel())] = float("nan")
    ring_k, ring_v = c.ring_k.clone(), c.ring_v.clone()
    for b in range(c.batch):
        i = int(c.pos[b])
        live = {j % (c.window + 1) for j in range(max(0, i - c.window), i)}
        for sl in range(c.window + 1):
            if sl not in live:
                ring_k[b, sl] = float("nan")
                ring_v[b, sl] = float("nan")
    c.pages, c.ring_k, c.ring_v = pages, ring_k, ring_v
    return c


def widen_block_table(c: gen.DecodeInputs, columns: int):
    """Give every sequence a block table of `columns` columns: the extra
    columns name a page no sequence owns (poisoned by poison_unread, so a call
    that read one would return NaN).  Call after poison_unread."""
    bt = c.block_table.numpy()
    assert columns >= bt.shape[1]
    spare = sorted(set(range(c.n_pages)) - set(bt.ravel().tolist()))
    assert spare, "the store needs an unowned page"
    wide = np.full((bt.shape[0], columns), spare[0], dtype=np.int32)
    wide[:, :bt.shape[1]] = bt
    c.block_table = torch.from_numpy(wide)
    return c


def run_decode(entry, c: gen.DecodeInputs, *, splits=0, flags=0, max_pos_hint=None):
    dev = "cuda"
    desc = desc_of(c)
    dt = gen.TORCH_DTYPE[c.dtype]
    pages = c.pages.to(dev)
    bt = c.block_table.to(dev)
    pos = c.pos.to(dev)
    q, kc, vc = c.q.to(dev), c.k_cur.to(dev), c.v_cur.to(dev)
    rk, rv = c.ring_k.to(dev), c.ring_v.to(dev)
    # the library takes the value decoder as B_t^T [H][d_h][r_v]
    A, Bv = c.A.to(dev), c.Bv.transpose(1, 2).contiguous().to(dev)
    out = torch.full(tuple(c.q.shape), float("nan"), dtype=dt, device=dev)
    mp = int(c.pos.max()) if max_pos_hint is None else max_pos_hint
    nbytes = B.lla_decode_workspace_bytes(desc, c.batch, mp, c.window, splits)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=dev)
    st = B.store(pages, bt)
    args = B.decode_args(loop=c.loop, window=c.window, pos=pos, q=q, k_cur=kc, v_cur=vc, ring_k=rk,
                         ring_v=rv, A=A, B=Bv, out=out, workspace=ws, max_pos_hint=mp, splits=splits,
                         flags=flags)
    ENTRY[entry](desc, st, c.batch, args)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), rk.float().cpu().numpy(), rv.float().cpu().numpy()


def oracle_decode(c: gen.DecodeInputs, form: str):
    pages = c.pages.double().numpy()
    bt = c.block_table.numpy()
    kw = dict(groups=c.groups, page_size=c.page_size, r_k=c.r_k, r_v=c.r_v)
    sK, sV = [], []
    for b in range(c.batch):
        n_lat = max(0, int(c.pos[b]) - c.window)
        k, v = O.gather_latents(pages, bt, b, n_lat, **kw)
        sK.append(k)
        sV.append(v)
    fn = O.textbook_decode if form == "textbook" else O.absorbed_decode
    args = [t.double().numpy() for t in (c.q, c.k_cur, c.v_cur, c.ring_k, c.ring_v, c.A, c.Bv)]
    pos = c.pos.numpy()
    out = fn(sK, sV, pos, *args, window=c.window, rope_base=c.rope_base)
    slot, nk, nv = O.ring_update(pos, args[1], args[2], window=c.window, rope_base=c.rope_base)
    return out, slot, nk, nv
