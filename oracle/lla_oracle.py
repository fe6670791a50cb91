"""Plain fp64 CPU oracle for single-token decode attention over a compressed
cross-loop KV latent cache (Looped Latent Attention and its absorbed successor,
Hybrid Latent Attention).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline may import this module; the HIP library and its Python binding never
call it, and it shares no code with them.  Every function below is written
from the pages' description, in fp64, with numpy matrix products as the only
library steps.

Sources (cited by page title and section / equation):
  [HLA]  "Hybrid Latent Attention" summary, picx.dev/p/a0K1YZ: sections
         "Latent Writer" (Eq. 2), "Latent Reader" (Eqs. 3, 4), "Rotary
         Embedding Alignment", "Key Problem", "Summary (Overview)".
  [LLA-A] "Looped Latent Attention: Cross-Loop Key-Value Compression For
         Looped Transformers", abstract, acceptodds.com/papers/iclr2027-34396.
  [LLA-S] "Looped Latent Attention: Cross-Loop KV Compression for Looped
         Transformers", abstract, searcharxiv.org/abs/2607.15456.

Readings taken where the pages are silent (each also applies to the GPU path):
  R1  Window range: Eq. 4 literally -- latent tokens j < i-W, exact tokens
      i-W <= j <= i (W+1 tokens including the current one).
  R2  The current token is always exact (its latent needs every loop).
  R3  One joint softmax over latent, window and current token (Eq. 4 uses
      one attention weight a_ij,t in both sums).
  R4  Score scale 1/sqrt(d_h) for latent scores too (Eq. 3).
  R5  Loop-1 maps act on the loop-1 latent exactly as A_t, B_t act on the main
      latent (with r_1 in place of r_k, r_v).
  R6  The writer input h_j,t is any vector of width d_in (hidden state for
      HLA; the concatenated [k; v] of a group for LLA).
  R7  E_t has shape (r_k+r_v) x d_in and c = E_t x (Eq. 2 writes E_t h).
  R8  Rotary embedding, head space: pairs (f, f+d_h/2), angle p*theta_f with
      theta_f = base^(-2f/d_h), 0-based absolute positions; base 0 = none.
  R9  Latent space rotation: R~_p = I_m (x) R_p over m = r_k/d_h consecutive
      d_h-blocks of the key latent (m latent pairs per rotary frequency).
  R10 Key latents are stored already rotated ("baked"), R~_p c^K, when the set
      uses rotary embedding; the reader rotates the query by R~_i.
  (R11, R15, R17, R18 concern the synthetic maps, bf16 rounding, the error
  metric and unsupported argument forms; nothing here depends on them.)
  R12 LLA-2D / per-head LLA decoders are dense maps from the group's latent.
  R13 LLA has a single set serving loops 1..T (no separate loop-1 latent).
  R14 The exact window holds post-rotation keys and values for every loop.
  R16 context N = i+1; latent count max(0, i-W); exact count min(W+1, i+1).
  R19 The uncompressed (full-cache) baseline keeps one exact paged cache per
      (layer, loop), pages of [P][H][d_h] with rotated keys; a decode call
      appends the current token and attends to tokens 0..i.
  R20 fp8 latent storage: OCP e4m3 codes, round to nearest even, saturating
      at 448, one fp32 scale per token, group and part = max|x| / 448 of that
      part (1 when the part is all zero).
  R21 The parallel (second) pass of the two-pass procedure evaluates Eq. 4 at
      every position i of whole sequences at once: latents of j < i-W from
      the store (written by the first pass), this loop's exact keys and
      values of j = max(0, i-W) .. i, positions 0-based from the start of
      each sequence.
"""
import numpy as np

TILE = 16  # tokens per tile in the paged store layout
WIDE_KEY_ROWS = 512  # key rows wider than this are stored in chunks of KEY_CHUNK dimensions
KEY_CHUNK = 32


# ----------------------------------------------------------------------------
# Rotary embedding  ([HLA] "Rotary Embedding Alignment"; readings R8, R9)
# ----------------------------------------------------------------------------
def rope_theta(d_h: int, base: float) -> np.ndarray:
    """theta_f = base^(-2f/d_h), f = 0..d_h/2-1 (reading R8)."""
    f = np.arange(d_h // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * f / d_h)


def rope_head(x: np.ndarray, pos, base: float) -> np.ndarray:
    """R_p x for x [..., d_h]: pair (f, f+d_h/2) rotated by angle p*theta_f.
    base == 0 means no rotary embedding (identity)."""
    x = np.asarray(x, dtype=np.float64)
    if base == 0:
        return x.copy()
    d_h = x.shape[-1]
    half = d_h // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_theta(d_h, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_latent(c: np.ndarray, pos, base: float, d_h: int) -> np.ndarray:
    """R~_p c for a key latent c [..., r_k] made of m = r_k/d_h blocks of d_h:
    the same head-space rotation applied to every block (reading R9)."""
    c = np.asarray(c, dtype=np.float64)
    if base == 0:
        return c.copy()
    r_k = c.shape[-1]
    assert r_k % d_h == 0, "rotary latent needs whole d_h blocks"
    blocks = c.reshape(c.shape[:-1] + (r_k // d_h, d_h))
    out = rope_head(blocks, np.asarray(pos)[..., None], base)
    return out.reshape(c.shape)


# ----------------------------------------------------------------------------
# Paged store layout (the library's documented store format)
# ----------------------------------------------------------------------------
def store_key_offset(page, group, slot, dim, *, groups, page_size, r_k, r_v):
    """Flat element offset of key-latent element `dim` of the token in `slot`
    of physical page `page`, group `group`.  A page holds, for each group, P
    tokens as P/16 tiles; a tile is 16 token rows of r_k key numbers followed
    by the value block (see store_value_offset).  Key rows wider than
    WIDE_KEY_ROWS numbers are kept chunk-major instead: chunk c (dimensions
    32c .. 32c + 31, the last one narrower when r_k is not a multiple of 32)
    holds the 16 tokens' pieces one after another, so that a 16-token x
    32-dimension block is contiguous."""
    R = r_k + r_v
    page, group, slot, dim = (np.asarray(a, dtype=np.int64) for a in (page, group, slot, dim))
    base = (page * groups + group) * page_size * R + (slot // TILE) * TILE * R
    if r_k <= WIDE_KEY_ROWS:
        return base + (slot % TILE) * r_k + dim
    c = dim // KEY_CHUNK
    width = np.minimum(KEY_CHUNK, r_k - KEY_CHUNK * c)
    return base + c * (TILE * KEY_CHUNK) + (slot % TILE) * width + dim % KEY_CHUNK


def store_value_offset(page, group, slot, dim, *, groups, page_size, r_k, r_v):
    """Flat element offset of value-latent element `dim`: inside a tile, the
    value block is r_v/16 sub-blocks of 16 dimensions x 16 tokens, each stored
    dimension-major (16 consecutive tokens of one dimension are contiguous)."""
    R = r_k + r_v
    page, group, slot, dim = (np.asarray(a, dtype=np.int64) for a in (page, group, slot, dim))
    base = (page * groups + group) * page_size * R + (slot // TILE) * TILE * R
    return base + TILE * r_k + (dim // TILE) * TILE * TILE + (dim % TILE) * TILE + (slot % TILE)


def gather_latents(pages: np.ndarray, block_table: np.ndarray, b: int, n_tok: int, *,
                   groups, page_size, r_k, r_v):
    """Key and value latents of tokens 0..n_tok-1 of sequence b, read through
    the block table: returns (sK [n_tok, G, r_k], sV [n_tok, G, r_v]) in fp64."""
    flat = np.asarray(pages, dtype=np.float64).reshape(-1)
    j = np.arange(n_tok)
    page = np.asarray(block_table)[b, j // page_size].astype(np.int64)
    slot = j % page_size
    kw = dict(groups=groups, page_size=page_size, r_k=r_k, r_v=r_v)
    g = np.arange(groups)
    ko = store_key_offset(page[:, None, None], g[None, :, None], slot[:, None, None],
                          np.arange(r_k)[None, None, :], **kw)
    vo = store_value_offset(page[:, None, None], g[None, :, None], slot[:, None, None],
                            np.arange(r_v)[None, None, :], **kw)
    return flat[ko], flat[vo]


# ----------------------------------------------------------------------------
# fp8 latent storage ([HLA] "Summary (Overview)": the codec combines with
# quantization; reading R20): OCP e4m3 codes with one fp32 scale per token,
# group and part (key, value).  A stored latent element is decode(code) *
# scale.
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(code):
    """Values of OCP e4m3 codes: sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no
    infinities."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return sign * v


def e4m3_encode(x):
    """Round to nearest, ties to even, onto the e4m3 grid, saturating at
    +-448 (reading R20).  The grid spacing in the binade [2^e, 2^(e+1)) is
    2^(e-3) for e >= -6; below 2^-6 it is the subnormal spacing 2^-9."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    e = np.clip(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6, 8)
    quantum = 2.0 ** (e - 3)
    v = np.minimum(np.round(a / quantum) * quantum, E4M3_MAX)   # np.round: halves to even
    normal = v >= 2.0 ** -6
    ev = np.floor(np.log2(np.where(normal, v, 1.0)))
    code = np.where(normal, ((ev + 7) * 8 + (v / 2.0 ** ev * 8 - 8)), v / 2.0 ** -9)
    return (code.astype(np.int64) | np.where(neg, 0x80, 0)).astype(np.uint8)


def fp8_quantize_rows(rows):
    """Per row (last axis): scale = max|x| / 448 (1 for an all-zero row) and
    codes = e4m3_encode(x / scale).  Returns (codes uint8, scale)."""
    rows = np.asarray(rows, dtype=np.float64)
    amax = np.max(np.abs(rows), axis=-1)
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    return e4m3_encode(rows / scale[..., None]), scale


def fp8_tile_bytes(r_k: int, r_v: int) -> int:
    """Bytes of one fp8 tile (16 tokens, one group): key codes, value codes,
    16 key scales and 16 value scales (fp32)."""
    return TILE * (r_k + r_v) + 2 * TILE * 4


def _fp8_tile_base(page, group, slot, groups, page_size, r_k, r_v):
    tb = fp8_tile_bytes(r_k, r_v)
    return (page * groups + group) * (page_size // TILE) * tb + (slot // TILE) * tb


def fp8_key_offset(page, group, slot, dim, *, groups, page_size, r_k, r_v):
    """Byte offset of the key code of element `dim` (token-major rows of r_k
    codes, as in the 16-bit store)."""
    page, group, slot, dim = (np.asarray(a, dtype=np.int64) for a in (page, group, slot, dim))
    return _fp8_tile_base(page, group, slot, groups, page_size, r_k, r_v) + (slot % TILE) * r_k + dim


def fp8_value_offset(page, group, slot, dim, *, groups, page_size, r_k, r_v):
    """Byte offset of the value code of element `dim`: the value block is
    r_v/64 quads of four 16-dimension sub-blocks; inside a quad, dimension row
    m (dim % 16) holds, for each group of 4 tokens, the 4 tokens of each of the
    4 sub-blocks: [m][token // 4][sub-block][token % 4]."""
    page, group, slot, dim = (np.asarray(a, dtype=np.int64) for a in (page, group, slot, dim))
    t = slot % TILE
    return (_fp8_tile_base(page, group, slot, groups, page_size, r_k, r_v) + TILE * r_k + (dim // 64) * 1024
            + (dim % TILE) * 64 + (t // 4) * 16 + ((dim // TILE) % 4) * 4 + t % 4)


def fp8_scale_offset(page, group, slot, part, *, groups, page_size, r_k, r_v):
    """Byte offset of the fp32 scale of the token's key (part 0) or value
    (part 1) codes."""
    page, group, slot, part = (np.asarray(a, dtype=np.int64) for a in (page, group, slot, part))
    return (_fp8_tile_base(page, group, slot, groups, page_size, r_k, r_v) + TILE * (r_k + r_v)
            + part * TILE * 4 + (slot % TILE) * 4)


def gather_latents_fp8(pages: np.ndarray, block_table: np.ndarray, b: int, n_tok: int, *,
                       groups, page_size, r_k, r_v):
    """Decoded key and value latents (code value x scale, fp64) of tokens
    0..n_tok-1 of sequence b from an fp8 store given as raw bytes."""
    raw = np.asarray(pages).reshape(-1).view(np.uint8)
    j = np.arange(n_tok)
    page = np.asarray(block_table)[b, j // page_size].astype(np.int64)
    slot = j % page_size
    kw = dict(groups=groups, page_size=page_size, r_k=r_k, r_v=r_v)
    g = np.arange(groups)
    P3, G3, S3 = page[:, None, None], g[None, :, None], slot[:, None, None]
    kc = raw[fp8_key_offset(P3, G3, S3, np.arange(r_k)[None, None, :], **kw)]
    vc = raw[fp8_value_offset(P3, G3, S3, np.arange(r_v)[None, None, :], **kw)]

    def scale(part):
        off = fp8_scale_offset(page[:, None], g[None, :], slot[:, None], part, **kw)
        by = raw[off[..., None] + np.arange(4)].astype(np.uint8)
        return by.copy().view(np.float32)[..., 0].astype(np.float64)
    return e4m3_decode(kc) * scale(0)[..., None], e4m3_decode(vc) * scale(1)[..., None]


# ----------------------------------------------------------------------------
# Latent writer  ([HLA] "Latent Writer", Eq. 2; readings R6, R7, R10)
# ----------------------------------------------------------------------------
def write_latents(x: np.ndarray, enc: np.ndarray, pos: np.ndarray, *, r_k: int,
                  rope_base: float = 0.0, rope_baked: int = 0, head_dim: int = 0):
    """c = sum over the set's loops of E_t x_t, per token and group (Eq. 2).

    x   [B, n_tok, n_loops, G, d_in]   per-loop inputs h_j,t
    enc [n_loops, G, r_k+r_v, d_in]    encoders E_t
    pos [B, n_tok]                     absolute positions
    Returns c [B, n_tok, G, r_k+r_v] in fp64; with a baked rotary set the key
    part is replaced by R~_p c^K."""
    x = np.asarray(x, dtype=np.float64)
    enc = np.asarray(enc, dtype=np.float64)
    n_loops, G = enc.shape[0], enc.shape[1]
    c = np.zeros(x.shape[:2] + (G, enc.shape[2]))
    for t in range(n_loops):
        for g in range(G):
            c[:, :, g, :] += x[:, :, t, g, :] @ enc[t, g].T
    if rope_baked and rope_base != 0:
        c[..., :r_k] = rope_latent(c[..., :r_k], np.asarray(pos)[..., None], rope_base, head_dim)
    return c


# ----------------------------------------------------------------------------
# Decode: shared bookkeeping of Eq. 4's ranges (readings R1, R2, R16)
# ----------------------------------------------------------------------------
def ranges(i: int, window: int):
    """(n_lat, exact window positions j < i) for current position i."""
    n_lat = max(0, i - window)
    return n_lat, np.arange(n_lat, i)


def _softmax(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max()
    e = np.exp(z)
    return e / e.sum()


def _exact_part(b, h, i, window, ring_k, ring_v, k_cur, v_cur, rope_base):
    """Exact keys/values for positions max(0,i-W)..i: ring slots j mod (W+1)
    hold positions j < i (post-rotation keys, R14); the current token's key is
    R_i k_cur and its value v_cur (R2)."""
    _, win = ranges(i, window)
    slots = win % (window + 1)
    kw = np.asarray(ring_k[b, slots, h], dtype=np.float64)
    vw = np.asarray(ring_v[b, slots, h], dtype=np.float64)
    k_self = rope_head(np.asarray(k_cur[b, h], dtype=np.float64), i, rope_base)
    v_self = np.asarray(v_cur[b, h], dtype=np.float64)
    return np.vstack([kw, k_self[None]]), np.vstack([vw, v_self[None]])


def textbook_decode(sK, sV, pos, q, k_cur, v_cur, ring_k, ring_v, A, Bv, *,
                    window: int, rope_base: float = 0.0):
    """Reconstruct-then-attend (the primary oracle).

    For every sequence b and head h (group g = h // (H/G)), at position
    i = pos[b]: latent tokens j < i-W get k_j = A^(h) sK_j and
    v_j = B^(h)T sV_j (the decoders rebuild loop-specific keys and values, as
    Looped Latent Attention does on read; [LLA-A], [LLA-S]); exact tokens come
    from the ring and the current token; then ordinary softmax attention with
    q' = R_i q and scale 1/sqrt(d_h) ([HLA] "Latent Reader", R3, R4).

    sK[b] [n >= n_lat, G, r_k], sV[b] [n >= n_lat, G, r_v]   (lists over b)
    q, k_cur, v_cur [B, H, d_h]; ring_k, ring_v [B, W+1, H, d_h]
    A [H, d_h, r_k]; Bv [H, r_v, d_h]
    Returns out [B, H, d_h] (fp64)."""
    B, H, d_h = np.asarray(q).shape
    G = np.asarray(sK[0]).shape[1]
    hpg = H // G
    out = np.zeros((B, H, d_h))
    for b in range(B):
        i = int(pos[b])
        n_lat, _ = ranges(i, window)
        for h in range(H):
            g = h // hpg
            a_h = np.asarray(A[h], dtype=np.float64)
            b_h = np.asarray(Bv[h], dtype=np.float64)
            k_lat = np.asarray(sK[b][:n_lat, g], dtype=np.float64) @ a_h.T
            v_lat = np.asarray(sV[b][:n_lat, g], dtype=np.float64) @ b_h
            k_ex, v_ex = _exact_part(b, h, i, window, ring_k, ring_v, k_cur, v_cur, rope_base)
            keys = np.vstack([k_lat, k_ex])
            vals = np.vstack([v_lat, v_ex])
            qr = rope_head(np.asarray(q[b, h], dtype=np.float64), i, rope_base)
            a = _softmax(keys @ qr / np.sqrt(d_h))
            out[b, h] = a @ vals
    return out


def absorbed_decode(sK, sV, pos, q, k_cur, v_cur, ring_k, ring_v, A, Bv, *,
                    window: int, rope_base: float = 0.0):
    """Eq. 3 / Eq. 4 literally ([HLA] "Latent Reader"): the query is mapped
    into latent space, q~ = R~_i A_t^T q, latent scores are
    q~ . sK_j / sqrt(d_h) against the stored (already rotated, R10) key
    latents, exact scores are q' . k_j / sqrt(d_h) with q' = R_i q, one
    softmax spans all of them (R3), and
        o = B_t^T sum_{j<i-W} a_j sV_j + sum_{i-W<=j<=i} a_j v_j.
    Same arguments and result shape as textbook_decode."""
    B, H, d_h = np.asarray(q).shape
    G = np.asarray(sK[0]).shape[1]
    hpg = H // G
    out = np.zeros((B, H, d_h))
    for b in range(B):
        i = int(pos[b])
        n_lat, _ = ranges(i, window)
        for h in range(H):
            g = h // hpg
            qv = np.asarray(q[b, h], dtype=np.float64)
            a_h = np.asarray(A[h], dtype=np.float64)
            q_lat = rope_latent(a_h.T @ qv, i, rope_base, d_h)
            s_lat = np.asarray(sK[b][:n_lat, g], dtype=np.float64) @ q_lat / np.sqrt(d_h)
            k_ex, v_ex = _exact_part(b, h, i, window, ring_k, ring_v, k_cur, v_cur, rope_base)
            s_ex = k_ex @ rope_head(qv, i, rope_base) / np.sqrt(d_h)
            a = _softmax(np.concatenate([s_lat, s_ex]))
            a_lat, a_ex = a[:n_lat], a[n_lat:]
            o_lat_latent = a_lat @ np.asarray(sV[b][:n_lat, g], dtype=np.float64)
            out[b, h] = np.asarray(Bv[h], dtype=np.float64).T @ o_lat_latent + a_ex @ v_ex
    return out


def ring_update(pos, k_cur, v_cur, *, window: int, rope_base: float = 0.0):
    """What a decode call writes into the exact window: slot i mod (W+1) of
    sequence b receives R_i k_cur[b] and v_cur[b] (reading R14).
    Returns (slot [B], k [B, H, d_h], v [B, H, d_h])."""
    pos = np.asarray(pos, dtype=np.int64)
    k = rope_head(np.asarray(k_cur, dtype=np.float64), pos[:, None], rope_base)
    return pos % (window + 1), k, np.asarray(v_cur, dtype=np.float64).copy()


# ----------------------------------------------------------------------------
# Parallel HLA attention over whole sequences ([HLA] "Training Procedure": the
# two-pass fine-tuning writes every token's latents in a first pass, then runs
# HLA attention at all positions in parallel; reading R21)
# ----------------------------------------------------------------------------
def parallel_attention(sK, sV, n_tok, q, k, v, A, Bv, *, window: int, rope_base: float = 0.0,
                       rows=None):
    """Eq. 3 / Eq. 4 at every position i < n_tok[b] of every sequence b.

    sK[b] [>= n_tok[b], G, r_k], sV[b] [>= n_tok[b], G, r_v]   latents of the
        sequence's tokens (key latents stored rotated when the set bakes
        rotary embedding, R10)
    q, k, v [B, n_max, H, d_h]   this loop's query and exact key / value at
        every position (q, k before rotation)
    A [H, d_h, r_k]; Bv [H, r_v, d_h]
    Position i scores latent tokens j < i-W with q~ = R~_i A_t^T q_i (Eq. 3)
    and exact tokens max(0, i-W) <= j <= i with (R_i q_i).(R_j k_j), all
    over sqrt(d_h), in one softmax (R3); o_i = B_t^T sum_lat a_j sV_j +
    sum_exact a_j v_j.  `rows`: optional list of (b, i) to evaluate (the
    rest stay zero).  Returns out [B, n_max, H, d_h] (fp64); rows at or past
    n_tok[b] are zero."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, n_max, H, d_h = q.shape
    G = np.asarray(sK[0]).shape[1]
    hpg = H // G
    if rows is None:
        rows = [(b, i) for b in range(B) for i in range(int(n_tok[b]))]
    out = np.zeros((B, n_max, H, d_h))
    for b, i in rows:
        assert i < int(n_tok[b])
        n_lat = max(0, i - window)
        j_ex = np.arange(n_lat, i + 1)
        k_ex = rope_head(k[b, j_ex], j_ex[:, None], rope_base)        # [n_ex, H, d_h]
        for h in range(H):
            g = h // hpg
            a_h = np.asarray(A[h], dtype=np.float64)
            q_lat = rope_latent(a_h.T @ q[b, i, h], i, rope_base, d_h)
            s_lat = np.asarray(sK[b][:n_lat, g], dtype=np.float64) @ q_lat / np.sqrt(d_h)
            s_ex = k_ex[:, h] @ rope_head(q[b, i, h], i, rope_base) / np.sqrt(d_h)
            a = _softmax(np.concatenate([s_lat, s_ex]))
            o_lat = a[:n_lat] @ np.asarray(sV[b][:n_lat, g], dtype=np.float64)
            out[b, i, h] = np.asarray(Bv[h], dtype=np.float64).T @ o_lat + a[n_lat:] @ v[b, j_ex, h]
    return out


# ----------------------------------------------------------------------------
# Uncompressed (full-cache) looped decode: the teacher the codec replaces
# ([HLA] "Key Problem": every loop keeps and attends to its own exact keys and
# values, 2 T d numbers per token per layer).  Reading R19: the exact cache
# of one (layer, loop) is paged like the latent store, a page holding
# [P][H][d_h] (all heads of a token contiguous), keys stored rotated (R14).
# ----------------------------------------------------------------------------
def gather_kv_cache(k_pages, v_pages, block_table, b: int, n_tok: int, *, page_size: int):
    """Keys and values [n_tok, H, d_h] of tokens 0..n_tok-1 of sequence b:
    token j lives in page block_table[b][j // P], slot j % P."""
    j = np.arange(n_tok)
    pg = np.asarray(block_table)[b][j // page_size]
    sl = j % page_size
    return (np.asarray(k_pages, dtype=np.float64)[pg, sl],
            np.asarray(v_pages, dtype=np.float64)[pg, sl])


def full_cache_decode(k_pages, v_pages, block_table, pos, q, k_cur, v_cur, *, page_size: int,
                      rope_base: float = 0.0):
    """One decode call of the uncompressed model for one (layer, loop): at
    position i the query q' = R_i q attends with scale 1/sqrt(d_h) (R4) to
    the cached tokens 0..i-1 and to the current token R_i k_cur, v_cur, one
    softmax over all of them.

    k_pages, v_pages [n_pages, P, H, d_h]; block_table [B, max_pages];
    q, k_cur, v_cur [B, H, d_h].  Returns out [B, H, d_h] (fp64)."""
    B, H, d_h = np.asarray(q).shape
    out = np.zeros((B, H, d_h))
    for b in range(B):
        i = int(pos[b])
        K, V = gather_kv_cache(k_pages, v_pages, block_table, b, i, page_size=page_size)
        for h in range(H):
            k_self = rope_head(np.asarray(k_cur[b, h], dtype=np.float64), i, rope_base)
            keys = np.vstack([K[:, h], k_self[None]])
            vals = np.vstack([V[:, h], np.asarray(v_cur[b, h], dtype=np.float64)[None]])
            qr = rope_head(np.asarray(q[b, h], dtype=np.float64), i, rope_base)
            out[b, h] = _softmax(keys @ qr / np.sqrt(d_h)) @ vals
    return out


def kv_cache_update(pos, k_cur, v_cur, block_table, *, page_size: int, rope_base: float = 0.0):
    """What a full-cache decode call writes: page block_table[b][i // P], slot
    i % P of sequence b receives R_i k_cur[b] and v_cur[b].
    Returns (page [B], slot [B], k [B, H, d_h], v [B, H, d_h])."""
    pos = np.asarray(pos, dtype=np.int64)
    page = np.asarray(block_table)[np.arange(len(pos)), pos // page_size]
    k = rope_head(np.asarray(k_cur, dtype=np.float64), pos[:, None], rope_base)
    return page, pos % page_size, k, np.asarray(v_cur, dtype=np.float64).copy()


# ----------------------------------------------------------------------------
# Cache size closed form  ([HLA] "Latent Writer": r_k + r_v + 2 r_1 numbers per
# token per layer, vs 2 T d for the full per-loop cache ("Key Problem"))
# ----------------------------------------------------------------------------
def set_bytes_per_token(groups: int, r_k: int, r_v: int, elem_bytes: int) -> int:
    """Bytes one latent set stores per token per layer."""
    return groups * (r_k + r_v) * elem_bytes


def hla_bytes_per_token(layers: int, r_k: int, r_v: int, r_1: int, elem_bytes: int) -> int:
    """Hybrid Latent Attention: main latent [c^K; c^V] plus loop-1 latent
    [c^K,1; c^V,1] in every layer."""
    return layers * (set_bytes_per_token(1, r_k, r_v, elem_bytes)
                     + set_bytes_per_token(1, r_1, r_1, elem_bytes))


def full_cache_bytes_per_token(layers: int, loops: int, d_model: int, elem_bytes: int) -> int:
    """Uncompressed looped cache: each loop keeps its own K and V of width d."""
    return layers * 2 * loops * d_model * elem_bytes
