"""Pins of the oracle's lattice tables against closed forms (CPU only).

The velocity set, weights and moment basis are not printed on the pages (the
lattice figure of the thermal-LBM page is lost); the oracle takes the textbook
D3Q19 set and the orthogonal moment basis of d'Humieres et al.  These tests pin
the tables to properties that fix them independently of how the oracle builds
them: completeness of the velocity set, isotropy of the weights up to fourth
order, mutual orthogonality of the moment rows with the published squared
norms, and the D3Q7 equilibrium weights implied by the anti-bounce-back
coefficient w = (6 + a_T)/21 that the thermal-LBM page prints (Sec. 2).
"""
import itertools

import numpy as np
import pytest

import oracle

# squared norms of the D3Q19 orthogonal moment rows (d'Humieres et al. 2002,
# Table of the D3Q19 basis), in the row order 1, e, eps, jx, qx, jy, qy, jz, qz,
# 3pxx, 3pixx, pww, piww, pxy, pyz, pxz, mx, my, mz.
PUBLISHED_NORMS = [19, 2394, 252, 10, 40, 10, 40, 10, 40, 36, 72, 12, 24, 4, 4, 4, 8, 8, 8]


@pytest.fixture(scope="module")
def tab():
    return oracle.tables()


def test_velocity_set_is_complete_d3q19(tab):
    c = tab["c19"]
    expect = {v for v in itertools.product((-1, 0, 1), repeat=3) if sum(a * a for a in v) <= 2}
    assert len(expect) == 19
    assert {tuple(int(a) for a in v) for v in c} == expect
    assert tuple(c[0]) == (0, 0, 0)


def test_opposites(tab):
    c, opp = tab["c19"], tab["opp19"]
    for q in range(19):
        assert np.array_equal(c[opp[q]], -c[q])
        assert opp[opp[q]] == q


def test_weights_isotropy(tab):
    c = tab["c19"].astype(float)
    w = tab["w19"]
    assert abs(w.sum() - 1) < 1e-15
    # odd moments vanish
    assert np.abs(w @ c).max() < 1e-16
    assert np.abs(np.einsum("q,qa,qb,qc->abc", w, c, c, c)).max() < 1e-16
    # second moment = cs^2 I with cs^2 = 1/3
    assert np.allclose(np.einsum("q,qa,qb->ab", w, c, c), np.eye(3) / 3, atol=1e-16)
    # fourth moment = cs^4 (d_ab d_cd + d_ac d_bd + d_ad d_bc)
    d = np.eye(3)
    iso = (np.einsum("ab,cd->abcd", d, d) + np.einsum("ac,bd->abcd", d, d) + np.einsum("ad,bc->abcd", d, d)) / 9
    assert np.allclose(np.einsum("q,qa,qb,qc,qd->abcd", w, c, c, c, c), iso, atol=1e-16)


def test_moment_rows_orthogonal_with_published_norms(tab):
    M = tab["M"]
    G = M @ M.T
    assert np.abs(G - np.diag(np.diag(G))).max() < 1e-12
    assert np.allclose(np.diag(G), PUBLISHED_NORMS, atol=1e-12)
    assert np.linalg.matrix_rank(M) == 19


def test_moment_rows_conserved_and_integer(tab):
    M, c = tab["M"], tab["c19"]
    assert np.array_equal(M[0], np.ones(19))
    assert np.array_equal(M[3], c[:, 0]) and np.array_equal(M[5], c[:, 1]) and np.array_equal(M[7], c[:, 2])
    assert np.array_equal(M, np.round(M))


def test_inverse(tab):
    M, Mi = tab["M"], tab["Minv"]
    assert np.abs(M @ Mi - np.eye(19)).max() < 1e-14
    assert np.abs(Mi @ M - np.eye(19)).max() < 1e-14
    # orthogonal rows: the inverse is M^T divided by the norms
    assert np.abs(Mi - M.T / np.array(PUBLISHED_NORMS)).max() < 1e-14


def test_d3q7_tables(tab):
    c7, N, Ni, opp = tab["c7"], tab["N"], tab["Ninv"], tab["opp7"]
    assert {tuple(v) for v in c7} == {(0, 0, 0), (1, 0, 0), (-1, 0, 0), (0, 1, 0), (0, -1, 0), (0, 0, 1), (0, 0, -1)}
    for k in range(7):
        assert np.array_equal(c7[opp[k]], -c7[k])
    assert np.abs(N @ Ni - np.eye(7)).max() < 1e-14
    assert np.array_equal(N[1:4], c7.T)


@pytest.mark.parametrize("a_T", [-0.75, 0.0, -2.0, 1.5])
def test_d3q7_equilibrium_matches_antibounceback_coefficient(a_T):
    """At rest the D3Q7 equilibrium has rest weight (1 - a_T)/7 and moving weight
    (6 + a_T)/42; the page's ABB coefficient (6 + a_T)/21 is twice the moving
    weight, i.e. 2 w_i T_w, which is what half-way anti-bounce-back needs."""
    p = dict(nx=1, ny=1, nz=1, thermal=1, s19=[1.0] * 19, s7=[1.0] * 7, a_T=a_T)
    T = 0.37
    _, geq = oracle.equilibrium(p, np.array([1.0]), np.zeros((1, 3)), np.array([T]))
    geq = geq[0]
    assert abs(geq[0] - (1 - a_T) / 7 * T) < 1e-15
    assert np.allclose(geq[1:], (6 + a_T) / 42 * T, atol=1e-15)
    omega_page = (6 + a_T) / 21
    assert np.allclose(2 * geq[1:] / T, omega_page, atol=1e-15)
