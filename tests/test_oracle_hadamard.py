"""Pins for the oracle's Hadamard blocks (no GPU)."""
import numpy as np

from conftest import golden_rows
from oracle import hadamard


def _sylvester_recursive(n):
    """Independent textbook construction H_{2k} = [[H, H], [H, -H]] in +-1 form."""
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_order4_textbook():
    ref = np.array([[float(v) for v in row] for row in golden_rows("sylvester_h4.txt")])
    assert np.array_equal(hadamard.hadamard(4) * 2.0, ref)


def test_h128_properties():
    H = hadamard.hadamard(128)
    pm = np.rint(H * np.sqrt(128))
    assert set(np.unique(pm)) == {-1.0, 1.0}
    assert np.array_equal(pm @ pm.T, 128 * np.eye(128))          # H H^T = n I (+-1 form)
    assert np.allclose(H @ H.T, np.eye(128), atol=1e-14)         # normalised form
    assert np.array_equal(H, H.T)
    assert (pm[0] == 1).all() and (pm[:, 0] == 1).all()
    assert np.array_equal(pm, _sylvester_recursive(128))


def test_signs_unpacking():
    w = np.array([0b1011, 0x80000000], dtype=np.uint32)
    s = hadamard.signs(w, 64)
    assert list(s[:5]) == [-1, -1, 1, -1, 1]
    assert s[63] == -1 and (s[4:63] == 1).all()


def test_forward_inverse_identity_and_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 384))
    sw = rng.integers(0, 1 << 32, 12, dtype=np.uint32)
    xt = hadamard.rht_forward(x, sw)
    # blockwise orthogonal: norms preserved block by block
    assert np.allclose(np.linalg.norm(xt.reshape(3, 3, 128), axis=-1),
                       np.linalg.norm(x.reshape(3, 3, 128), axis=-1))
    # diag(s) H H diag(s) = I: inverse of forward with the same signs
    assert np.allclose(hadamard.rht_inverse(xt, sw), x, atol=1e-12)


def test_sign_order_on_each_side():
    """Input side applies the sign before H; output side after H (all-ones vector test)."""
    sw = np.array([0x1, 0, 0, 0], dtype=np.uint32)          # s_0 = -1, all other signs +1
    ones = np.ones(128)
    # input: H diag(s) 1 = H (1 - 2 e_0): entry 0 is (128 - 2)/sqrt(128)
    assert np.isclose(hadamard.rht_forward(ones, sw)[0], 126 / np.sqrt(128))
    # output: diag(s) H 1 = diag(s) sqrt(128) e_0 -> entry 0 is -sqrt(128), others 0
    y = hadamard.rht_inverse(ones, sw)
    assert np.isclose(y[0], -np.sqrt(128)) and np.allclose(y[1:], 0)
