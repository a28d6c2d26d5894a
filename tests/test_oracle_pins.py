"""Pins of the fp64 oracle against facts fixed by the mathematics of the gated
delta rule (closed forms, special cases, an independent chunked form, finite
differences and invariants).  CPU only.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, a transposed state, an off-by-one in the decay) fails at least one.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import chunked

RTOL = 1e-12


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def rand_case(rng, B=1, T=37, H=2, dk=5, dv=4, h0=True, gscale=0.3):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -np.logaddexp(0, rng.standard_normal((B, T, H))) * gscale
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    N = B
    s0 = rng.standard_normal((N, H, dk, dv)) * 0.5 if h0 else None
    return q, k, v, g, beta, s0


# ---------------------------------------------------------------- closed forms

def test_beta_zero_forward_closed_form():
    """beta = 0: S_t = exp(G_t) S_0 with G_t = sum_{s<=t} g_s."""
    rng = np.random.default_rng(1)
    q, k, v, g, beta, s0 = rand_case(rng, T=29, dk=6, dv=3)
    beta[:] = 0.0
    o, ht = oracle.fwd(q, k, v, g, beta, s0, scale=0.7)
    G = np.cumsum(g[0], axis=0)                      # [T,H]
    for h in range(q.shape[2]):
        S0 = s0[0, h].T                              # d_v x d_k
        exp_o = 0.7 * np.exp(G[:, h])[:, None] * (q[0, :, h] @ S0.T)
        assert rel(o[0, :, h], exp_o) < RTOL
        assert rel(ht[0, h], np.exp(G[-1, h]) * s0[0, h]) < RTOL


def test_beta_zero_backward_closed_form():
    """beta = 0: every gradient has a closed form in G_t, S_0, q, do, dht."""
    rng = np.random.default_rng(2)
    q, k, v, g, beta, s0 = rand_case(rng, T=23, H=1, dk=4, dv=5)
    beta[:] = 0.0
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(s0.shape)
    sc = 0.9
    dq, dk, dv, dg, db, dh0 = oracle.bwd(q, k, v, g, beta, do, s0, dht, scale=sc)
    o, ht = oracle.fwd(q, k, v, g, beta, s0, scale=sc)
    G = np.cumsum(g[0, :, 0])
    S0 = s0[0, 0].T
    dST = dht[0, 0].T
    T = q.shape[1]
    Q, K, V, DO = q[0, :, 0], k[0, :, 0], v[0, :, 0], do[0, :, 0]
    # dq_t = sc e^{G_t} S0^T do_t
    assert rel(dq[0, :, 0], sc * np.exp(G)[:, None] * (DO @ S0)) < RTOL
    assert np.max(np.abs(dv)) == 0.0
    assert np.max(np.abs(dk)) == 0.0
    # dh0 (h-layout) = sum_t sc e^{G_t} q_t do_t^T + e^{G_T} dht
    exp_dh0 = sc * np.einsum("t,ti,tj->ij", np.exp(G), Q, DO) + np.exp(G[-1]) * dht[0, 0]
    assert rel(dh0[0, 0], exp_dh0) < RTOL
    # dg_s = sum_{t>=s} <do_t, o_t> + <dht, ht>
    per_t = np.sum(DO * o[0, :, 0], axis=1)
    exp_dg = np.cumsum(per_t[::-1])[::-1] + np.sum(dht * ht)
    assert rel(dg[0, :, 0], exp_dg) < RTOL
    # dbeta_t = (Y_t k_t) . (v_t - a_t S_{t-1} k_t), Y_t = dL/dS_t
    a = np.exp(g[0, :, 0])
    exp_db = np.zeros(T)
    for t in range(T):
        Y = np.exp(G[-1] - G[t]) * dST
        for u in range(t, T):
            Y = Y + sc * np.exp(G[u] - G[t]) * np.outer(DO[u], Q[u])
        Sprev = np.exp(G[t - 1]) * S0 if t > 0 else S0
        exp_db[t] = (Y @ K[t]) @ (V[t] - a[t] * (Sprev @ K[t]))
    assert rel(db[0, :, 0], exp_db) < 1e-11


def test_orthonormal_key_retrieval():
    """g = 0, beta = 1, orthonormal keys: S k_i = v_i exactly after the writes,
    so a query equal to an earlier key returns that key's value."""
    rng = np.random.default_rng(3)
    dk, dv, T = 8, 5, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T[:T]                                     # orthonormal rows
    k = keys[None, :, None, :].copy()
    v = rng.standard_normal((1, T, 1, dv))
    j = np.array([rng.integers(0, t + 1) for t in range(T)])   # j <= t
    q = keys[j][None, :, None, :].copy()
    g = np.zeros((1, T, 1))
    beta = np.ones((1, T, 1))
    s0 = rng.standard_normal((1, 1, dk, dv))            # any prior content is erased
    o, ht = oracle.fwd(q, k, v, g, beta, s0)
    assert rel(o[0, :, 0], v[0, j, 0]) < 1e-12
    # full-rank case: T = dk keys span the space, final S = V^T K exactly
    assert rel(ht[0, 0], keys.T @ v[0, :, 0]) < 1e-12


def test_single_token_closed_form():
    rng = np.random.default_rng(4)
    q, k, v, g, beta, s0 = rand_case(rng, T=1, H=3, dk=4, dv=6)
    o, ht = oracle.fwd(q, k, v, g, beta, s0, scale=1.3)
    for h in range(3):
        a, b = np.exp(g[0, 0, h]), beta[0, 0, h]
        S0 = s0[0, h].T
        kk, vv, qq = k[0, 0, h], v[0, 0, h], q[0, 0, h]
        S1 = a * S0 + b * np.outer(vv - a * S0 @ kk, kk)
        assert rel(o[0, 0, h], 1.3 * S1 @ qq) < RTOL
        assert rel(ht[0, h], S1.T) < RTOL


def test_strong_decay_limit():
    """g = -30: S_t ~ beta_t v_t k_t^T; nothing overflows."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta, s0 = rand_case(rng, T=40, dk=6, dv=6)
    g[:] = -30.0
    o, ht = oracle.fwd(q, k, v, g, beta, s0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    exp_o = beta[..., None] * v * np.sum(k * q, axis=-1, keepdims=True)
    assert rel(o, exp_o) < 1e-10
    o2, ht2 = chunked.fwd(q, k, v, g, beta, s0, chunk=16)
    assert np.all(np.isfinite(o2)) and rel(o2, o) < 1e-10


# ------------------------------------------------------ independent chunked form

@pytest.mark.parametrize("C", [1, 3, 16, 64])
def test_chunked_equals_recurrent_forward(C):
    rng = np.random.default_rng(10 + C)
    q, k, v, g, beta, s0 = rand_case(rng, B=2, T=47, H=3, dk=7, dv=5)
    o, ht = oracle.fwd(q, k, v, g, beta, s0, scale=0.8)
    o2, ht2 = chunked.fwd(q, k, v, g, beta, s0, scale=0.8, chunk=C)
    assert rel(o2, o) < RTOL and rel(ht2, ht) < RTOL


@pytest.mark.parametrize("C", [1, 3, 16, 64])
def test_chunked_equals_recurrent_backward(C):
    rng = np.random.default_rng(20 + C)
    q, k, v, g, beta, s0 = rand_case(rng, B=2, T=41, H=2, dk=6, dv=4)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(s0.shape)
    r1 = oracle.bwd(q, k, v, g, beta, do, s0, dht, scale=0.6)
    r2 = chunked.bwd(q, k, v, g, beta, do, s0, dht, scale=0.6, chunk=C)
    for name, a, b in zip("dq dk dv dg dbeta dh0".split(), r2, r1):
        assert rel(a, b) < 1e-11, name


def test_chunked_equals_recurrent_varlen():
    rng = np.random.default_rng(30)
    lens = [5, 0, 17, 1, 33]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = rand_case(rng, B=1, T=T, H=2, dk=5, dv=5)
    s0 = rng.standard_normal((len(lens), 2, 5, 5))
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(s0.shape)
    o, ht = oracle.fwd(q, k, v, g, beta, s0, cu_seqlens=cu)
    o2, ht2 = chunked.fwd(q, k, v, g, beta, s0, cu_seqlens=cu, chunk=16)
    assert rel(o2, o) < RTOL and rel(ht2, ht) < RTOL
    # an empty sequence passes its state through
    assert np.array_equal(ht[1], s0[1])
    r1 = oracle.bwd(q, k, v, g, beta, do, s0, dht, cu_seqlens=cu)
    r2 = chunked.bwd(q, k, v, g, beta, do, s0, dht, cu_seqlens=cu, chunk=16)
    for name, a, b in zip("dq dk dv dg dbeta dh0".split(), r2, r1):
        assert rel(a, b) < 1e-11, name
    assert np.array_equal(r1[5][1], dht[1])


def test_wy_identity():
    """Within one chunk, exp(gamma_L) I - Kt^T W equals the product of the
    per-token transition matrices a_r (I - beta_r k_r k_r^T) (rightmost first
    token), and Kt^T U is the chunk's end state from a zero state."""
    rng = np.random.default_rng(40)
    L, dk, dv = 11, 6, 4
    K = rng.standard_normal((L, dk))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.standard_normal((L, dv))
    g = -np.logaddexp(0, rng.standard_normal(L)) * 0.3
    b = 1 / (1 + np.exp(-rng.standard_normal(L)))
    p = chunked.chunk_prep(K, V, g, b)
    Kt = np.exp(p["gamma"][-1] - p["gamma"])[:, None] * K
    M = np.exp(p["gamma"][-1]) * np.eye(dk) - Kt.T @ p["W"]
    prod = np.eye(dk)
    for r in range(L):
        prod = np.exp(g[r]) * (np.eye(dk) - b[r] * np.outer(K[r], K[r])) @ prod
    assert rel(M, prod) < 1e-12
    bvec = np.zeros((dk, dv))
    for r in range(L):
        bvec = np.exp(g[r]) * (np.eye(dk) - b[r] * np.outer(K[r], K[r])) @ bvec \
            + b[r] * np.outer(K[r], V[r])
    assert rel(Kt.T @ p["U"], bvec) < 1e-12


def test_triangular_solve_matches_textbook_routine():
    rng = np.random.default_rng(41)
    L = 64
    K = rng.standard_normal((L, 16))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    g = -np.logaddexp(0, rng.standard_normal(L)) * 0.1
    b = 1 / (1 + np.exp(-rng.standard_normal(L)))
    p = chunked.chunk_prep(K, np.zeros((L, 1)), g, b)
    Tref = scipy.linalg.solve_triangular(np.eye(L) + p["A"], np.eye(L), lower=True,
                                         unit_diagonal=True)
    assert rel(p["T"], Tref) < 1e-12
    assert np.allclose(np.triu(p["T"], 1), 0.0) and np.allclose(np.diag(p["T"]), 1.0)


# ------------------------------------------------------------ finite differences

def test_backward_finite_differences():
    rng = np.random.default_rng(50)
    q, k, v, g, beta, s0 = rand_case(rng, B=1, T=19, H=2, dk=4, dv=3)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(s0.shape)
    sc = 0.75

    def loss(q, k, v, g, beta, s0):
        o, ht = oracle.fwd(q, k, v, g, beta, s0, scale=sc)
        return np.sum(o * do) + np.sum(ht * dht)

    grads = oracle.bwd(q, k, v, g, beta, do, s0, dht, scale=sc)
    args = [q, k, v, g, beta, s0]
    idx = [0, 1, 2, 3, 4, 5]
    gmap = [grads[0], grads[1], grads[2], grads[3], grads[4], grads[5]]
    eps = 1e-6
    for a_i, gr in zip(idx, gmap):
        for _ in range(3):
            d = rng.standard_normal(args[a_i].shape)
            plus = [x.copy() for x in args]
            minus = [x.copy() for x in args]
            plus[a_i] = plus[a_i] + eps * d
            minus[a_i] = minus[a_i] - eps * d
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            an = np.sum(gr * d)
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (a_i, fd, an)


# ------------------------------------------------------------------- invariants

def test_linearity_in_state_and_values():
    rng = np.random.default_rng(60)
    q, k, v, g, beta, s0 = rand_case(rng, T=25, dk=5, dv=4)
    v2 = rng.standard_normal(v.shape)
    s02 = rng.standard_normal(s0.shape)
    a, b = 0.7, -1.9
    o1, h1 = oracle.fwd(q, k, v, g, beta, s0)
    o2, h2 = oracle.fwd(q, k, v2, g, beta, s02)
    o3, h3 = oracle.fwd(q, k, a * v + b * v2, g, beta, a * s0 + b * s02)
    assert rel(o3, a * o1 + b * o2) < 1e-12 and rel(h3, a * h1 + b * h2) < 1e-12


def test_contraction_and_reflection():
    rng = np.random.default_rng(61)
    q, k, v, g, beta, s0 = rand_case(rng, T=30, H=1, dk=6, dv=6)
    v[:] = 0.0
    beta[:] = rng.uniform(0, 2, beta.shape)
    prev = np.linalg.norm(s0[0, 0])
    for t in range(1, 31):
        _, ht = oracle.fwd(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], s0)
        cur = np.linalg.norm(ht[0, 0])
        assert cur <= np.exp(g[0, t - 1, 0]) * prev * (1 + 1e-12)
        prev = cur
    # beta = 2, g = 0: a Householder reflection per token preserves the norm
    beta[:] = 2.0
    g[:] = 0.0
    _, ht = oracle.fwd(q, k, v, g, beta, s0)
    assert abs(np.linalg.norm(ht) - np.linalg.norm(s0)) < 1e-12 * np.linalg.norm(s0)


def test_split_resume_forward_and_backward():
    rng = np.random.default_rng(62)
    q, k, v, g, beta, s0 = rand_case(rng, T=50, H=2, dk=5, dv=4)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(s0.shape)
    T1 = 21
    o, ht = oracle.fwd(q, k, v, g, beta, s0)
    oa, ha = oracle.fwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], s0)
    ob, hb = oracle.fwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], ha)
    assert rel(np.concatenate([oa, ob], 1), o) < RTOL and rel(hb, ht) < RTOL
    full = oracle.bwd(q, k, v, g, beta, do, s0, dht)
    second = oracle.bwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], do[:, T1:],
                        ha, dht)
    first = oracle.bwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], do[:, :T1],
                       s0, second[5])
    for i in range(5):
        assert rel(np.concatenate([first[i], second[i]], 1), full[i]) < 1e-11
    assert rel(first[5], full[5]) < 1e-11


def test_varlen_equals_independent_dense_calls():
    rng = np.random.default_rng(63)
    lens = [9, 30, 2]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = rand_case(rng, T=sum(lens), H=2, dk=4, dv=4)
    s0 = rng.standard_normal((3, 2, 4, 4))
    do = rng.standard_normal(v.shape)
    o, ht = oracle.fwd(q, k, v, g, beta, s0, cu_seqlens=cu)
    gr = oracle.bwd(q, k, v, g, beta, do, s0, None, cu_seqlens=cu)
    for n in range(3):
        sl = slice(cu[n], cu[n + 1])
        on, hn = oracle.fwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], s0[n:n + 1])
        assert rel(o[:, sl], on) < RTOL and rel(ht[n:n + 1], hn) < RTOL
        gn = oracle.bwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], do[:, sl],
                        s0[n:n + 1])
        for i in range(5):
            assert rel(gr[i][:, sl], gn[i]) < RTOL


def test_head_and_batch_independence():
    rng = np.random.default_rng(64)
    q, k, v, g, beta, s0 = rand_case(rng, B=2, T=20, H=3, dk=4, dv=5)
    o, ht = oracle.fwd(q, k, v, g, beta, s0)
    perm = [2, 0, 1]
    op, hp = oracle.fwd(q[:, :, perm], k[:, :, perm], v[:, :, perm], g[:, :, perm],
                        beta[:, :, perm], s0[:, perm])
    assert np.array_equal(op, o[:, :, perm]) and np.array_equal(hp, ht[:, perm])
    ob, hb = oracle.fwd(q[1:], k[1:], v[1:], g[1:], beta[1:], s0[1:])
    assert np.array_equal(ob, o[1:]) and np.array_equal(hb, ht[1:])


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(65)
    q, k, v, g, beta, s0 = rand_case(rng, B=2, T=70, H=3, dk=4, dv=4)
    do = rng.standard_normal(v.shape)
    a = oracle.bwd(q, k, v, g, beta, do, s0, nthreads=1)
    b = oracle.bwd(q, k, v, g, beta, do, s0, nthreads=5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ------------------------------------------ in-operator L2 normalisation of q, k

def _raw_qk_case(rng, T=21, H=2, dk=5, dv=4):
    q, k, v, g, beta, s0 = rand_case(rng, T=T, H=H, dk=dk, dv=dv)
    k = k * rng.uniform(0.3, 3.0, k.shape[:-1] + (1,))   # rand_case's keys are unit rows
    return q, k, v, g, beta, s0


def test_l2norm_forward_is_scale_invariant():
    """Normalised rows do not depend on a positive rescaling of q or k rows."""
    rng = np.random.default_rng(61)
    q, k, v, g, beta, s0 = _raw_qk_case(rng)
    cq = rng.uniform(0.1, 10.0, q.shape[:-1] + (1,))
    ck = rng.uniform(0.1, 10.0, k.shape[:-1] + (1,))
    o1, h1 = oracle.fwd(q, k, v, g, beta, s0, scale=0.8, qk_l2norm=True)
    o2, h2 = oracle.fwd(q * cq, k * ck, v, g, beta, s0, scale=0.8, qk_l2norm=True)
    assert rel(o2, o1) < 1e-12 and rel(h2, h1) < 1e-12
    # and equals the plain recurrence on rows divided by their norms
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o3, h3 = oracle.fwd(qn, kn, v, g, beta, s0, scale=0.8)
    assert rel(o3, o1) < 1e-12 and rel(h3, h1) < 1e-12


def test_l2norm_gradients_orthogonal_and_scaled():
    """d/dx of f(x/||x||) is orthogonal to x, and scales as 1/c under x -> c x."""
    rng = np.random.default_rng(62)
    q, k, v, g, beta, s0 = _raw_qk_case(rng, T=17)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(s0.shape)
    dq, dk, dv, dg, db, dh0 = oracle.bwd(q, k, v, g, beta, do, s0, dht, scale=1.1, qk_l2norm=True)
    for x, dx in ((q, dq), (k, dk)):
        dots = np.sum(x * dx, axis=-1)
        assert np.max(np.abs(dots)) < 1e-10 * np.max(np.linalg.norm(x, axis=-1) * np.linalg.norm(dx, axis=-1))
    c = 3.5
    dq2, dk2, dv2, dg2, db2, dh02 = oracle.bwd(q * c, k, v, g, beta, do, s0, dht, scale=1.1, qk_l2norm=True)
    assert rel(dq2 * c, dq) < 1e-10 and rel(dk2, dk) < 1e-10 and rel(dv2, dv) < 1e-10
    # the other gradients do not see the normalisation
    dqh = oracle.bwd(q / np.linalg.norm(q, axis=-1, keepdims=True), k / np.linalg.norm(k, axis=-1, keepdims=True),
                     v, g, beta, do, s0, dht, scale=1.1)
    for a, b in zip((dv, dg, db, dh0), dqh[2:]):
        assert rel(a, b) < 1e-12


def test_l2norm_backward_finite_differences():
    """Central differences of L = <do, o> + <dht, ht> in raw q and k entries."""
    rng = np.random.default_rng(63)
    q, k, v, g, beta, s0 = _raw_qk_case(rng, T=9, H=1, dk=4, dv=3)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(s0.shape)

    def loss(qq, kk):
        o, ht = oracle.fwd(qq, kk, v, g, beta, s0, scale=0.6, qk_l2norm=True)
        return float(np.sum(o * do) + np.sum(ht * dht))

    dq, dk = oracle.bwd(q, k, v, g, beta, do, s0, dht, scale=0.6, qk_l2norm=True)[:2]
    eps = 1e-6
    for (which, x, dx) in (("q", q, dq), ("k", k, dk)):
        for idx in [(0, 0, 0, 0), (0, 3, 0, 2), (0, 8, 0, 3), (0, 5, 0, 1)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            num = (loss(xp, k) - loss(xm, k)) / (2 * eps) if which == "q" else (loss(q, xp) - loss(q, xm)) / (2 * eps)
            assert abs(num - dx[idx]) < 1e-6 * max(1.0, abs(num)), (which, idx, num, dx[idx])


def test_l2norm_rows_below_eps():
    """Rows shorter than the floor are divided by the floor (and differentiated so)."""
    x = np.zeros((1, 1, 1, 4))
    x[..., 0] = 1e-13
    y, d = oracle.l2norm_rows(x)
    assert d[..., 0] == oracle.L2_EPS and y[..., 0] == 1e-13 / oracle.L2_EPS
    dy = np.arange(1.0, 5.0).reshape(x.shape)
    assert np.array_equal(oracle.l2norm_rows_bwd(y, d, dy), dy / oracle.L2_EPS)
