"""Properties of the seeded input generators that the workloads' recipes
state (CPU only; the generators hold no attention or codec arithmetic)."""
import numpy as np

from synth import gen


def test_trajectory_codec_shapes_and_bases():
    """Rank-8 trajectories of T d_h = 512 numbers per (head, part): M has
    orthonormal columns times sqrt(512 / 8), U orthonormal columns; the
    encoders are block-diagonal (keys feed only the key latent)."""
    c = gen.trajectory_codec(5, heads=3, head_dim=128, loops=4, rank=8, r=32, noise=0.05, n_cal=2048)
    assert c.M.shape == (3, 2, 512, 8) and c.U.shape == (3, 2, 512, 32)
    for h in range(3):
        for p in range(2):
            np.testing.assert_allclose(c.M[h, p].T @ c.M[h, p], 64.0 * np.eye(8), atol=1e-9)
            np.testing.assert_allclose(c.U[h, p].T @ c.U[h, p], np.eye(32), atol=1e-9)
    enc = c.encoders()
    assert enc.shape == (4, 3, 64, 256)
    assert np.all(enc[:, :, :32, 128:] == 0) and np.all(enc[:, :, 32:, :128] == 0)
    A, Bv = c.decoders(3)
    assert A.shape == (3, 128, 32) and Bv.shape == (3, 32, 128)
    np.testing.assert_array_equal(A, c.U[:, 0, 256:384, :])
    np.testing.assert_array_equal(Bv, c.U[:, 1, 256:384, :].transpose(0, 2, 1))


def test_trajectory_codec_captures_the_trajectory_subspace():
    """The top-8 singular directions of the calibration sample span M (the
    noise is 0.05 against unit signal), so the fitted rank-32 projection
    keeps every fresh token's trajectory up to the noise it cannot predict."""
    c = gen.trajectory_codec(6, heads=2, head_dim=64, loops=4, rank=8, r=32, noise=0.05, n_cal=2048)
    for h in range(2):
        for p in range(2):
            m = c.M[h, p] / np.sqrt(256 / 8)
            u8 = c.U[h, p, :, :8]
            s = np.linalg.svd(m.T @ u8, compute_uv=False)      # cosines of principal angles
            assert s.min() > 0.999
    x = gen.trajectory_tokens(c, batch=2, n_tok=500, seed=7, dtype="f32", device="cpu").double().numpy()
    assert x.shape == (2, 500, 4, 2, 128)
    assert abs(x.std() - 1.0) < 0.03                              # about unit variance
    # a fresh token's key trajectory, projected onto U: residual ~ noise level
    X = x[..., :64].transpose(0, 1, 3, 2, 4).reshape(2 * 500, 2, 256)   # [tokens, head, T d_h]
    U = c.U[:, 0]
    resid = X - np.einsum("hdr,hsr,nhs->nhd", U, U, X)
    rel = np.sqrt((resid ** 2).mean() / (X ** 2).mean())
    assert 0.02 < rel < 0.06


def test_trajectory_tokens_seeded():
    c = gen.trajectory_codec(8, heads=1, head_dim=64, loops=4, rank=8, r=32)
    a = gen.trajectory_tokens(c, batch=1, n_tok=10, seed=3, dtype="f32", device="cpu")
    b = gen.trajectory_tokens(c, batch=1, n_tok=10, seed=3, dtype="f32", device="cpu")
    d = gen.trajectory_tokens(c, batch=1, n_tok=10, seed=4, dtype="f32", device="cpu")
    assert (a == b).all() and not (a == d).all()
