"""Pins of the oracle's sampled acceptance (MTP K = 1) and inverse-CDF sampling.

[ORCH] module doc, "Non-greedy (Metropolis-Hastings)": the pages name stochastic
acceptance on the MTP K = 1 path without its rule. The oracle takes the standard
speculative-sampling rule (accept d with probability min(1, p0(d)/q(d)), else draw
from max(0, p0 - q) normalised; on acceptance the bonus token comes from p1). Its
defining property is that the emitted token is distributed exactly as p0 whatever
q is; these tests check that property, and each piece against closed forms
computed with scipy, by running the oracle's decisions over stratified grids of
uniforms (a grid of N points resolves every probability to within 1/N).
"""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import oracle as orc


def grid(n):
    return (np.arange(n) + 0.5) / n


def draw_counts(z, T, n):
    z2 = np.repeat(np.asarray(z, np.float32)[None, :], n, axis=0)
    tok, _ = orc.sample_tokens(z2, grid(n), T)
    return np.bincount(tok, minlength=len(z)) / n


@pytest.mark.parametrize("T", [0.5, 1.0, 2.5])
def test_inverse_cdf_draws_follow_softmax(T):
    z = np.random.default_rng(3).normal(0, 2, 7).astype(np.float32)
    n = 20000
    freq = draw_counts(z, T, n)
    want = softmax(z.astype(np.float64) / T)
    assert np.max(np.abs(freq - want)) <= 1.0 / n + 1e-12


def test_draw_reports_its_probability_and_orders_by_index():
    z = np.array([0.0, 1.0, 2.0, -1.0], np.float32)
    p = softmax(z.astype(np.float64))
    c = np.cumsum(p)
    for k, u in enumerate([0.0, c[0] * 0.999, c[0] * 1.001, c[2] * 1.0001, 0.999999]):
        tok, prob = orc.sample_tokens(z[None, :], [u])
        want = int(np.searchsorted(c, u, side="right"))
        assert tok[0] == want, (k, u)
        assert prob[0] == pytest.approx(p[want], rel=1e-12)


def test_dominant_logit_is_always_drawn():
    z = np.zeros(50, np.float32)
    z[17] = 60.0
    tok, _ = orc.sample_tokens(np.repeat(z[None, :], 5, 0), grid(5))
    assert (tok == 17).all()


def test_temperature_scales_the_logits():
    rng = np.random.default_rng(5)
    z = rng.normal(0, 3, 300).astype(np.float32)
    u = rng.random(40)
    for T in (0.5, 2.0):  # powers of two: z / T is exact in F32
        a, _ = orc.sample_tokens(np.repeat(z[None, :], 40, 0), u, T)
        b, _ = orc.sample_tokens(np.repeat((z / np.float32(T))[None, :], 40, 0), u, 1.0)
        assert (a == b).all()


def _case(seed, V=6, T=1.0):
    rng = np.random.default_rng(seed)
    zq = rng.normal(0, 1.5, V).astype(np.float32)
    zt = rng.normal(0, 1.5, (2, V)).astype(np.float32)
    q = softmax(zq.astype(np.float64) / T)
    p0 = softmax(zt[0].astype(np.float64) / T)
    p1 = softmax(zt[1].astype(np.float64) / T)
    return zq, zt, q, p0, p1


@pytest.mark.parametrize("seed,T", [(11, 1.0), (12, 0.8), (13, 1.7)])
def test_acceptance_rate_residual_and_bonus(seed, T):
    zq, zt, q, p0, p1 = _case(seed, T=T)
    V = q.size
    n = 1000
    r = np.maximum(p0 - q, 0.0)
    r /= r.sum()
    for d in range(V):
        acc = np.array([orc.accept_sampled(zq, zt, d, u, 0.5, T)["accept_count"] for u in grid(n)])
        assert abs(acc.mean() - min(1.0, p0[d] / q[d])) <= 1.0 / n + 1e-12
    # after a rejection (u0 -> 1- with a draft that p0 under-weights) the free token
    # follows the residual; after an acceptance (u0 = 0) the next position's p1
    d_rej = int(np.argmin(p0 / q))
    rej = [orc.accept_sampled(zq, zt, d_rej, 1.0 - 1e-15, u, T) for u in grid(n)]
    assert all(x["accept_count"] == 0 for x in rej)
    f = np.bincount([x["free_token"] for x in rej], minlength=V) / n
    assert np.max(np.abs(f - r)) <= 1.0 / n + 1e-12
    acc_runs = [orc.accept_sampled(zq, zt, d_rej, 0.0, u, T) for u in grid(n)]
    assert all(x["accept_count"] == 1 for x in acc_runs)
    f = np.bincount([x["free_token"] for x in acc_runs], minlength=V) / n
    assert np.max(np.abs(f - p1)) <= 1.0 / n + 1e-12


@pytest.mark.parametrize("seed", [21, 22])
def test_emitted_token_is_distributed_as_the_target(seed):
    """sum_d q(d) [a(d) 1{i = d} + (1 - a(d)) r(i)] = p0(i), with the acceptance
    rate a(d) and the rejection draw r taken from the oracle's own decisions over
    grids of uniforms (acceptance depends on u0 only, the draw on u1 only)."""
    zq, zt, q, p0, _ = _case(seed)
    V = q.size
    n = 1000
    out = np.zeros(V)
    for d in range(V):
        a = np.mean([orc.accept_sampled(zq, zt, d, u0, 0.5)["accept_count"] for u0 in grid(n)])
        out[d] += q[d] * a
        if a < 1.0:
            f = np.bincount([orc.accept_sampled(zq, zt, d, 1.0 - 1e-15, u)["free_token"]
                             for u in grid(n)], minlength=V) / n
            out += q[d] * (1.0 - a) * f
    assert np.max(np.abs(out - p0)) <= 2.0 / n


def test_identical_distributions_always_accept():
    zq, zt, *_ = _case(31)
    zt = zt.copy()
    zt[0] = zq
    for d in range(zq.size):
        assert all(orc.accept_sampled(zq, zt, d, u, 0.3)["accept_count"] == 1 for u in grid(200))


def test_rollback_commit_and_eos():
    zq, zt, q, p0, p1 = _case(41)
    d = int(np.argmax(p0 / q))  # p0(d) > q(d): always accepted
    acc = orc.accept_sampled(zq, zt, d, 0.99, 0.5)
    assert acc["accept_count"] == 1 and acc["rollback"] == 0
    assert acc["committed"] == [d, acc["free_token"]]
    assert orc.accept_sampled(zq, zt, d, 0.99, 0.5, eos=[d])["committed"] == [d]
    d2 = int(np.argmin(p0 / q))  # p0(d2) < q(d2): rejected for u0 -> 1
    rej = orc.accept_sampled(zq, zt, d2, 1.0 - 1e-15, 0.5)
    assert rej["accept_count"] == 0 and rej["rollback"] == 1
    assert rej["committed"] == [rej["free_token"]]
    e = orc.accept_sampled(zq, zt, d2, 1.0 - 1e-15, 0.5, eos=[rej["free_token"]])
    assert e["hit_eos"] and e["committed"] == [rej["free_token"]]
    assert rej["q_draft"] == pytest.approx(q[d2], rel=1e-12)
    assert rej["p_draft"] == pytest.approx(p0[d2], rel=1e-12)
