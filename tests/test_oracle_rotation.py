"""Pins of the oracle's rotation R_n (blocked orthonormal Walsh-Hadamard transform).

128-point butterfly with scale 1/sqrt(128) = 0.088388347648: 'integrate EXL3 Trellis into
the fused W4A16 API' (sparkinfer PR #90), review of kernel.py (_had128_quad). Non-power-of-two
dimensions use 128-blocks plus a power-of-two remainder (stated reading)."""
import numpy as np
import pytest
import scipy.linalg

import oracle_np as O


def _blocked_reference(n):
    if n & (n - 1) == 0:
        sizes = [n]
    else:
        sizes = [128] * (n // 128) + ([n % 128] if n % 128 else [])
    return scipy.linalg.block_diag(*[scipy.linalg.hadamard(b) / np.sqrt(b) for b in sizes])


@pytest.mark.parametrize("n", [16, 64, 128, 256, 512, 1024])
def test_explicit_equals_scipy_sylvester(n):
    assert np.allclose(O.hadamard_explicit(n), scipy.linalg.hadamard(n) / np.sqrt(n), atol=0, rtol=1e-15)


@pytest.mark.parametrize("n", [320, 160, 2560, 384])
def test_explicit_blocked_non_power_of_two(n):
    assert np.allclose(O.hadamard_explicit(n), _blocked_reference(n), atol=0, rtol=1e-15)


@pytest.mark.parametrize("n", [128, 320, 1024])
def test_unnormalised_hadamard_orthogonality(n):
    R = O.hadamard_explicit(n)
    # H H^T = b I per block; with the normalisation R R^T = I.
    assert np.allclose(R @ R.T, np.eye(n), atol=1e-12)
    H128 = np.round(O.hadamard_explicit(128) * np.sqrt(128))
    assert np.array_equal(H128 @ H128.T, 128 * np.eye(128))


@pytest.mark.parametrize("n", [32, 64, 128, 256, 320, 512, 1024, 2560])
def test_butterfly_equals_explicit_matrix(n):
    rng = np.random.default_rng(n)
    v = rng.standard_normal((3, n))
    got = O.rotate_rows(v)
    want = v @ O.hadamard_explicit(n).T
    assert np.allclose(got, want, atol=1e-12, rtol=1e-12)


@pytest.mark.parametrize("n", [128, 320, 1024, 2560])
def test_involution(n):
    rng = np.random.default_rng(1 + n)
    v = rng.standard_normal((2, n))
    assert np.allclose(O.rotate_rows(O.rotate_rows(v)), v, atol=1e-12)


def test_scale_constant_128():
    e0 = np.zeros((1, 128))
    e0[0, 0] = 1.0
    r = O.rotate_rows(e0)
    assert np.allclose(r, 0.088388347648, atol=1e-12)


def test_identity_mode_is_identity():
    v = np.random.default_rng(3).standard_normal((2, 320))
    assert np.array_equal(O.rotate_rows(v, identity=True), v)


def test_unsupported_remainder_rejected():
    out = np.zeros((96 + 128) ** 2)
    rc = O.lib().orc_hadamard_explicit(224, out.ctypes.data_as(__import__("ctypes").c_void_p))
    assert rc != 0    # 224 = 128 + 96, remainder not a power of two
