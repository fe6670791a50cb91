"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the attention or codec arithmetic: it only draws
random numbers with stated distributions and structure, and casts them to the
storage dtype.  Everything it returns is an input; expected values are
computed elsewhere from these same inputs.

Two flavours:
  * host (numpy, fp64 draws, cast to the storage dtype): small cases that the
    fp64 oracle checks exhaustively;
  * device (torch generator on the GPU): full-size buffers, for timing and for
    parity on sampled sequences (the sampled slices are copied to the host).
"""
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def as_stored(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Cast fp64 draws to the storage dtype (a CPU tensor)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DTYPE[dtype])


def gaussian_orthonormal(g: np.random.Generator, rows: int, cols: int,
                         scale: float = 1.0) -> np.ndarray:
    """Gaussian matrix orthonormalised by QR: orthonormal rows when wide,
    orthonormal columns when tall; times `scale`."""
    if rows >= cols:
        q, r = np.linalg.qr(g.standard_normal((rows, cols)))
        q = q * np.sign(np.diag(r))[None, :]
        return q * scale
    q, r = np.linalg.qr(g.standard_normal((cols, rows)))
    q = q * np.sign(np.diag(r))[None, :]
    return q.T * scale


def frequency_paired_decoder(g: np.random.Generator, heads: int, d_h: int, r_k: int,
                             scale: float = 1.0, complex_coeffs: bool = True) -> np.ndarray:
    """Key decoders A [heads, d_h, r_k] built only from same-frequency pair blocks.

    The key latent is m = r_k / d_h blocks of d_h numbers; in each block, as in
    head space, dimension f pairs with f + d_h/2 (one rotary frequency per pair).
    For head h and frequency f a coefficient vector alpha in C^m (unit norm)
    maps the m latent pairs of frequency f to head pair f:
        [a -c; c a] per block, with alpha_b = a + i c.
    With complex_coeffs=False the coefficients are real (c = 0).
    Rows of each A[h] are orthonormal (times `scale`)."""
    assert d_h % 2 == 0 and r_k % d_h == 0
    m, half = r_k // d_h, d_h // 2
    A = np.zeros((heads, d_h, r_k))
    for h in range(heads):
        for f in range(half):
            if complex_coeffs:
                v = g.standard_normal(m) + 1j * g.standard_normal(m)
            else:
                v = g.standard_normal(m).astype(complex)
            v = v / np.linalg.norm(v)
            for b in range(m):
                a, c = v[b].real, v[b].imag
                A[h, f, b * d_h + f] = a
                A[h, f, b * d_h + f + half] = -c
                A[h, f + half, b * d_h + f] = c
                A[h, f + half, b * d_h + f + half] = a
    return A * scale


def block_table(g: np.random.Generator, batch: int, pages_per_seq: int,
                spare: int = 0) -> (np.ndarray, int):
    """Each sequence gets `pages_per_seq` distinct physical pages drawn from a
    random permutation of batch*pages_per_seq + spare pages (fragmentation)."""
    n_pages = batch * pages_per_seq + spare
    perm = g.permutation(n_pages)[: batch * pages_per_seq]
    return perm.reshape(batch, pages_per_seq).astype(np.int32), n_pages


@dataclass
class DecodeInputs:
    """One decode call's inputs, all CPU tensors in the storage dtype (int32
    for indices).  Shapes: pages [n_pages, G*P*(r_k+r_v)], block_table
    [B, max_pages], pos [B], q/k_cur/v_cur [B, H, d_h], ring_k/ring_v
    [B, W+1, H, d_h], A [H, d_h, r_k], Bv [H, r_v, d_h]."""
    heads: int
    head_dim: int
    groups: int
    r_k: int
    r_v: int
    page_size: int
    window: int
    loop: int
    loop_first: int
    loop_last: int
    rope_base: float
    rope_baked: int
    dtype: str
    pages: torch.Tensor
    block_table: torch.Tensor
    pos: torch.Tensor
    q: torch.Tensor
    k_cur: torch.Tensor
    v_cur: torch.Tensor
    ring_k: torch.Tensor
    ring_v: torch.Tensor
    A: torch.Tensor
    Bv: torch.Tensor

    @property
    def batch(self) -> int:
        return int(self.pos.shape[0])

    @property
    def n_pages(self) -> int:
        return int(self.pages.shape[0])


def decode_inputs(seed: int, *, batch: int, heads: int, head_dim: int, groups: int,
                  r_k: int, r_v: int, positions, window: int, dtype: str,
                  page_size: int = 64, rope_base: float = 0.0, rope_baked: int = 0,
                  loop: int = 2, loop_first: int = 2, loop_last: int = 4,
                  latent_std: float = 1.0, exact_std: float = 1.0,
                  map_scale: float = 1.0, paired: Optional[bool] = None,
                  spare_pages: int = 3) -> DecodeInputs:
    """Random decode-call inputs with the given shapes.

    latents ~ N(0, latent_std^2); q ~ N(0, 1); exact window / current K and V
    ~ N(0, exact_std^2); A frequency-paired when the key latent holds whole
    d_h blocks and `paired` is not False (Gaussian-QR otherwise); B Gaussian-QR
    with orthonormal columns.  Maps are multiplied by `map_scale`."""
    g = rng(seed)
    positions = np.asarray(positions, dtype=np.int64).reshape(batch)
    max_pos = int(positions.max())
    pages_per_seq = max(1, -(-(max_pos + 1) // page_size))
    bt, n_pages = block_table(g, batch, pages_per_seq, spare_pages)
    row = groups * page_size * (r_k + r_v)
    pages = g.standard_normal((n_pages, row)) * latent_std
    q = g.standard_normal((batch, heads, head_dim))
    k_cur = g.standard_normal((batch, heads, head_dim)) * exact_std
    v_cur = g.standard_normal((batch, heads, head_dim)) * exact_std
    ring_k = g.standard_normal((batch, window + 1, heads, head_dim)) * exact_std
    ring_v = g.standard_normal((batch, window + 1, heads, head_dim)) * exact_std
    if paired is None:
        paired = r_k % head_dim == 0
    if paired:
        A = frequency_paired_decoder(g, heads, head_dim, r_k, map_scale)
    else:
        A = np.stack([gaussian_orthonormal(g, head_dim, r_k, map_scale) for _ in range(heads)])
    Bv = np.stack([gaussian_orthonormal(g, r_v, head_dim, map_scale) for _ in range(heads)])
    return DecodeInputs(
        heads=heads, head_dim=head_dim, groups=groups, r_k=r_k, r_v=r_v,
        page_size=page_size, window=window, loop=loop, loop_first=loop_first,
        loop_last=loop_last, rope_base=rope_base, rope_baked=rope_baked, dtype=dtype,
        pages=as_stored(pages, dtype), block_table=torch.from_numpy(bt),
        pos=torch.from_numpy(positions.astype(np.int32)),
        q=as_stored(q, dtype), k_cur=as_stored(k_cur, dtype), v_cur=as_stored(v_cur, dtype),
        ring_k=as_stored(ring_k, dtype), ring_v=as_stored(ring_v, dtype),
        A=as_stored(A, dtype), Bv=as_stored(Bv, dtype))


@dataclass
class WriterInputs:
    """Writer-call inputs: x [B, n_tok, n_loops, G, d_in], enc
    [n_loops, G, r_k+r_v, d_in], pos [B, n_tok] (CPU tensors)."""
    x: torch.Tensor
    enc: torch.Tensor
    pos: torch.Tensor


def writer_inputs(seed: int, *, batch: int, n_tok: int, n_loops: int, groups: int,
                  r_k: int, r_v: int, d_in: int, dtype: str, positions,
                  enc_scale: float = 1.0, x_std: float = 1.0) -> WriterInputs:
    """x ~ N(0, x_std^2); each encoder E_t (per group) Gaussian-QR with
    orthonormal rows (or columns when r_k+r_v > d_in), times enc_scale."""
    g = rng(seed)
    x = g.standard_normal((batch, n_tok, n_loops, groups, d_in)) * x_std
    enc = np.stack([np.stack([gaussian_orthonormal(g, r_k + r_v, d_in, enc_scale)
                              for _ in range(groups)]) for _ in range(n_loops)])
    pos = np.asarray(positions, dtype=np.int32).reshape(batch, n_tok)
    return WriterInputs(x=as_stored(x, dtype), enc=as_stored(enc, dtype),
                        pos=torch.from_numpy(pos))


def fp8_latent_draws(seed: int, *, n_pages: int, groups: int, page_size: int, r_k: int, r_v: int):
    """Synthetic content of an fp8 latent store, drawn directly as codes and
    scales: codes of finite e4m3 numbers with magnitudes in [1/8, 2) (exponent
    fields 4..7, any mantissa, random sign) and per-token scales uniform in
    [0.5, 1.5).  Returns codes uint8 [n_pages, G, P, r_k+r_v] and scales
    float32 [n_pages, G, P, 2] (key, value)."""
    g = rng(seed, 8)
    shape = (n_pages, groups, page_size, r_k + r_v)
    # six random bits per code: bit 5 the sign, bits 0..4 the low five bits
    # of an exponent field in 4..7 and the mantissa (uint8 throughout, so a
    # full-size store stays within a few bytes per element)
    v = g.integers(0, 64, size=shape, dtype=np.uint8)
    codes = ((v & 32) << 2) | 32 | (v & 31)
    scales = g.uniform(0.5, 1.5, size=(n_pages, groups, page_size, 2)).astype(np.float32)
    return codes, scales


@dataclass
class ParallelInputs:
    """One parallel-pass call's inputs (CPU tensors): latent store pages
    [n_pages, G*P*(r_k+r_v)] (the store layout), block_table [B, pages],
    n_tok [B], q, k, v [B, n_max, H, d_h], A [H, d_h, r_k], Bv [H, r_v, d_h]."""
    heads: int
    head_dim: int
    groups: int
    r_k: int
    r_v: int
    page_size: int
    window: int
    rope_base: float
    rope_baked: int
    pages: torch.Tensor
    block_table: torch.Tensor
    n_tok: torch.Tensor
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    A: torch.Tensor
    Bv: torch.Tensor


def parallel_inputs(seed: int, *, batch: int, heads: int, head_dim: int, groups: int, r_k: int, r_v: int,
                    n_max: int, n_tok, window: int, dtype: str = "bf16", page_size: int = 64,
                    rope_base: float = 0.0, paired: Optional[bool] = None, latent_std: float = 1.0,
                    exact_std: float = 1.0, spare_pages: int = 2) -> ParallelInputs:
    """Latents ~ N(0, latent_std^2) for every slot of every page; q ~ N(0, 1);
    k, v ~ N(0, exact_std^2); A frequency-paired (complex coefficients) when
    `paired` (default: with rotary embedding), Gaussian-QR otherwise; B
    Gaussian-QR.  Sequences own random pages covering n_max tokens."""
    g = rng(seed, 9)
    pps = max(1, -(-n_max // page_size))
    bt, n_pages = block_table(g, batch, pps, spare_pages)
    pages = g.standard_normal((n_pages, groups * page_size * (r_k + r_v))) * latent_std
    q = g.standard_normal((batch, n_max, heads, head_dim))
    k = g.standard_normal((batch, n_max, heads, head_dim)) * exact_std
    v = g.standard_normal((batch, n_max, heads, head_dim)) * exact_std
    if paired is None:
        paired = rope_base != 0
    if paired:
        A = frequency_paired_decoder(g, heads, head_dim, r_k)
    else:
        A = np.stack([gaussian_orthonormal(g, head_dim, r_k) for _ in range(heads)])
    Bv = np.stack([gaussian_orthonormal(g, r_v, head_dim) for _ in range(heads)])
    return ParallelInputs(heads=heads, head_dim=head_dim, groups=groups, r_k=r_k, r_v=r_v, page_size=page_size,
                          window=window, rope_base=rope_base, rope_baked=1 if rope_base else 0,
                          pages=as_stored(pages, dtype), block_table=torch.from_numpy(bt),
                          n_tok=torch.from_numpy(np.asarray(n_tok, dtype=np.int32).reshape(batch)),
                          q=as_stored(q, dtype), k=as_stored(k, dtype), v=as_stored(v, dtype),
                          A=as_stored(A, dtype), Bv=as_stored(Bv, dtype))


@dataclass
class KvCacheInputs:
    """One full-cache decode call's inputs (CPU tensors): k_pages, v_pages
    [n_pages, P, H, d_h] with every slot a call must not read (positions >= i
    of each sequence, spare pages) set to NaN; block_table [B, max_pages];
    pos [B]; q, k_cur, v_cur [B, H, d_h]."""
    page_size: int
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    block_table: torch.Tensor
    pos: torch.Tensor
    q: torch.Tensor
    k_cur: torch.Tensor
    v_cur: torch.Tensor


def kv_cache_inputs(seed: int, *, batch: int, heads: int, head_dim: int, positions, dtype: str,
                    page_size: int = 64, spare_pages: int = 2, kv_std: float = 1.0) -> KvCacheInputs:
    """Cached keys / values ~ N(0, kv_std^2), q, k_cur, v_cur ~ N(0, 1); the
    cache holds tokens 0..i-1 of each sequence; the page of position i exists."""
    g = rng(seed)
    pos = np.asarray(positions, dtype=np.int64).reshape(batch)
    pps = int(pos.max()) // page_size + 1
    bt, n_pages = block_table(g, batch, pps, spare_pages)
    kp = g.standard_normal((n_pages, page_size, heads, head_dim)) * kv_std
    vp = g.standard_normal((n_pages, page_size, heads, head_dim)) * kv_std
    valid = np.zeros((n_pages, page_size), dtype=bool)
    for b in range(batch):
        j = np.arange(int(pos[b]))
        valid[bt[b, j // page_size], j % page_size] = True
    kp[~valid] = np.nan
    vp[~valid] = np.nan
    q = g.standard_normal((batch, heads, head_dim))
    kc = g.standard_normal((batch, heads, head_dim)) * kv_std
    vc = g.standard_normal((batch, heads, head_dim)) * kv_std
    return KvCacheInputs(page_size=page_size, k_pages=as_stored(kp, dtype), v_pages=as_stored(vp, dtype),
                         block_table=torch.from_numpy(bt), pos=torch.from_numpy(pos.astype(np.int32)),
                         q=as_stored(q, dtype), k_cur=as_stored(kc, dtype), v_cur=as_stored(vc, dtype))


def device_normal(shape, dtype: str, seed: int, std: float = 1.0,
                  device: str = "cuda") -> torch.Tensor:
    """N(0, std^2) filled on the device from a seeded torch generator."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=gen)
    return t.to(TORCH_DTYPE[dtype])


@dataclass
class TrajectoryCodec:
    """A per-head LLA codec fit to synthetic loop trajectories.

    For every head h and part p (0 = keys, 1 = values) a token's trajectory
    over the T loops is one vector X in R^(T d_h) (loop t holds dims
    t d_h .. (t+1) d_h - 1), drawn as X = M alpha + noise eps with M [T d_h,
    rank] of orthonormal columns times sqrt(T d_h / rank) (so the elements of
    X have about unit variance), alpha ~ N(0, I_rank), eps ~ N(0, I).
    U [T d_h, r] holds the top-r left singular vectors of a calibration sample
    of n_cal such trajectories (fp64, from the symmetric eigendecomposition of
    X X^T).  Shapes: M [H, 2, T d_h, rank], U [H, 2, T d_h, r]."""
    loops: int
    head_dim: int
    noise: float
    M: np.ndarray
    U: np.ndarray

    @property
    def heads(self) -> int:
        return int(self.M.shape[0])

    @property
    def rank(self) -> int:
        return int(self.U.shape[3])

    def encoders(self) -> np.ndarray:
        """enc [T, H, 2r, 2 d_h]: E_t of head h = blockdiag(U^K_t^T, U^V_t^T),
        mapping a loop's [k_t; v_t] to its contribution to [s^K; s^V]."""
        T, dh, r, H = self.loops, self.head_dim, self.rank, self.heads
        enc = np.zeros((T, H, 2 * r, 2 * dh))
        for t in range(T):
            blk = self.U[:, :, t * dh:(t + 1) * dh, :]          # [H, 2, d_h, r]
            enc[t, :, :r, :dh] = blk[:, 0].transpose(0, 2, 1)
            enc[t, :, r:, dh:] = blk[:, 1].transpose(0, 2, 1)
        return enc

    def decoders(self, loop: int):
        """(A_t [H, d_h, r], Bv_t [H, r, d_h]) of loop t (1-based): the key
        decoder U^K_t and the value decoder B_t = U^V_t^T (v = B_t^T s^V)."""
        dh = self.head_dim
        blk = self.U[:, :, (loop - 1) * dh:loop * dh, :]
        return blk[:, 0].copy(), blk[:, 1].transpose(0, 2, 1).copy()


def trajectory_codec(seed: int, *, heads: int, head_dim: int, loops: int, rank: int = 8, r: int = 32,
                     noise: float = 0.05, n_cal: int = 2048) -> TrajectoryCodec:
    """Draw the trajectory bases M and fit U (see TrajectoryCodec)."""
    g = rng(seed, 31)
    D = loops * head_dim
    M = np.empty((heads, 2, D, rank))
    U = np.empty((heads, 2, D, r))
    for h in range(heads):
        for p in range(2):
            m = gaussian_orthonormal(g, D, rank, np.sqrt(D / rank))
            X = m @ g.standard_normal((rank, n_cal)) + noise * g.standard_normal((D, n_cal))
            _, vec = np.linalg.eigh(X @ X.T)      # ascending eigenvalues
            U[h, p] = vec[:, ::-1][:, :r]
            M[h, p] = m
    return TrajectoryCodec(loops=loops, head_dim=head_dim, noise=noise, M=M, U=U)


def trajectory_tokens(codec: TrajectoryCodec, *, batch: int, n_tok: int, seed: int, dtype: str = "bf16",
                      device: str = "cuda") -> torch.Tensor:
    """Fresh token trajectories of `batch` sequences x `n_tok` tokens, laid out
    as writer inputs x [B, n_tok, T, H, 2 d_h]: x[b, j, t, h] = [k; v] of
    token j, loop t, head h (the loop-t slices of X^K and X^V).  Drawn on
    `device` from a seeded torch generator."""
    H, T, dh, rank = codec.heads, codec.loops, codec.head_dim, codec.M.shape[3]
    D = T * dh
    gen_ = torch.Generator(device=device)
    gen_.manual_seed(int(seed))
    n = batch * n_tok
    Mt = torch.from_numpy(codec.M.reshape(H * 2, D, rank).transpose(0, 2, 1).copy()).float().to(device)
    alpha = torch.empty((H * 2, n, rank), dtype=torch.float32, device=device).normal_(generator=gen_)
    X = torch.bmm(alpha, Mt.contiguous())                   # [2H, n, D]
    del alpha
    X.add_(torch.empty_like(X).normal_(generator=gen_), alpha=codec.noise)
    X = X.view(H, 2, batch, n_tok, T, dh).permute(2, 3, 4, 0, 1, 5)
    return X.reshape(batch, n_tok, T, H, 2 * dh).to(TORCH_DTYPE[dtype]).contiguous()
