"""Parity of the sampling calls (sample_tokens, accept_sampled) with the oracle.

A draw is an integer decided by floating point: the HIP path forms probabilities
and running sums in F32, the oracle in F64, so the two can only disagree when the
uniform lies within rounding of a cumulative boundary. The HIP running sums chain
about 20 F32 additions of positive terms (segment trees, the segment scan, the
in-segment scan), so they sit within ~2e-6 of the exact cumulative probability;
MARGIN is five times that. Each comparison first computes, in F64, how far u is
from the ends of the oracle's chosen interval and compares exactly where that
margin is clear. Half of the random rows place u at the midpoint of the interval
of a token drawn from p (among tokens wider than 2 * MARGIN), so that every such
row is compared; the other half use raw uniforms, compared where clear. The
acceptance test is compared where |u0 q(d) - p0(d)| is clear in the same way.
"""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import oracle as orc
from tests.gpu_harness import torch

pytestmark = pytest.mark.gpu

MARGIN = 1e-5


def dev(a, dtype=None):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda") if dtype is None else \
        t.tensor(np.asarray(a), dtype=dtype, device="cuda")


def boundary_margin(p, tok, u):
    """Distance of u from the ends of token tok's interval of the CDF of p."""
    c = np.cumsum(p)
    lo = c[tok - 1] if tok > 0 else 0.0
    return min(u - lo, c[tok] - u)


def clear_uniform(p, rng):
    """u at the midpoint of the interval of a token drawn from p, among the tokens
    whose interval is wider than 2 * MARGIN."""
    w = np.where(p > 2 * MARGIN, p, 0.0)
    i = int(rng.choice(p.size, p=w / w.sum()))
    c = np.cumsum(p)
    lo = c[i - 1] if i > 0 else 0.0
    return float(np.float32(0.5 * (lo + c[i])))


def gpu_sample(z, u, T):
    from verifier_block_forward_amd import dbf
    t = torch()
    M, V = z.shape
    tok = t.empty(M, dtype=t.int32, device="cuda")
    prob = t.empty(M, dtype=t.float32, device="cuda")
    ws = t.empty(dbf.sample_tokens_workspace_bytes(M, V), dtype=t.uint8, device="cuda")
    dbf.sample_tokens(dev(z), dev(np.asarray(u, np.float32)), tok, prob, T, ws)
    t.cuda.synchronize()
    return tok.cpu().numpy(), prob.cpu().numpy()


def _random_vmt(n=8, seed=4242):
    """Seeded (V, M, T): V log-uniform over 2 .. 300,000 (segment counts 1 .. 256 and
    segments past 1024 values), M in 1 .. 16, T in 0.5 .. 2."""
    rng = np.random.default_rng(seed)
    return [(int(np.exp(rng.uniform(np.log(2), np.log(300000)))), int(rng.integers(1, 17)),
             round(float(rng.uniform(0.5, 2.0)), 3)) for _ in range(n)]


@pytest.mark.parametrize("V,M,T", [(1000, 5, 1.0), (1025, 16, 0.7), (5000, 3, 1.6), (248320, 16, 1.0),
                                   (262151, 4, 0.7), (1, 2, 1.0)] + _random_vmt())
def test_sample_tokens_match_the_oracle(V, M, T):
    print(f"\n[sample] V={V} M={M} T={T}", flush=True)
    rng = np.random.default_rng(V + M)
    z = rng.normal(0, 3, (M, V)).astype(np.float32)
    u = rng.random(M)
    u[0] = 0.0
    if M > 2:
        u[1] = 1.0 - 2.0 ** -24
    mid = set(range(2, M, 2)) if V > 1 else set()
    for m in mid:
        u[m] = clear_uniform(softmax(z[m].astype(np.float64) / T), rng)
    u = u.astype(np.float32).astype(np.float64)  # the GPU takes F32 uniforms
    got, prob = gpu_sample(z, u, T)
    want, pw = orc.sample_tokens(z, u, T)
    assert ((got >= 0) & (got < V)).all()
    # edge rows: u = 0 draws the first index; u -> 1 draws the last where its
    # probability is clear of rounding (both sit on a boundary by construction)
    assert got[0] == want[0] == 0
    if M > 2 and softmax(z[1].astype(np.float64) / T)[-1] > MARGIN:
        assert got[1] == want[1] == V - 1
    for m in range(2 if M > 2 else 1, M):
        p = softmax(z[m].astype(np.float64) / T)
        clear = boundary_margin(p, int(want[m]), u[m]) > MARGIN or V == 1
        assert clear or m not in mid
        if clear:
            assert got[m] == want[m], f"row {m}: token {got[m]} vs oracle {want[m]} (u={u[m]})"
            assert abs(prob[m] - pw[m]) <= 1e-6 + 1e-4 * pw[m]


def test_sample_tokens_dominant_and_edges():
    V = 70000
    z = np.full((4, V), -5.0, np.float32)
    z[0, 12345] = 40.0          # one token holds all the mass
    z[1, -1] = 40.0             # the last index
    z[2, 0] = 40.0              # the first index
    z[3] = np.linspace(-3, 3, V, dtype=np.float32)
    u = np.array([0.5, 0.999, 0.0, 0.5], np.float64)
    got, _ = gpu_sample(z, u, 1.0)
    want, _ = orc.sample_tokens(z, u, 1.0)
    assert got[0] == 12345 and got[1] == V - 1 and got[2] == 0
    p = softmax(z[3].astype(np.float64))
    assert boundary_margin(p, int(want[3]), u[3]) > MARGIN
    assert got[3] == want[3]


def gpu_accept(zq, zt, d, u0, u1, T=1.0, eos=None):
    from verifier_block_forward_amd import dbf
    t = torch()
    V = zq.size
    res = t.full((5,), -9, dtype=t.int32, device="cuda")
    com = t.full((2,), -9, dtype=t.int32, device="cuda")
    ws = t.empty(dbf.accept_sampled_workspace_bytes(V), dtype=t.uint8, device="cuda")
    dbf.accept_sampled(dev(zq), dev(zt), dev([d], t.int32), dev(np.array([u0, u1], np.float32)), res, T,
                       None if eos is None else dev(eos, t.int32), com, ws)
    t.cuda.synchronize()
    r = res.cpu().numpy()
    return r, com.cpu().numpy()[: max(int(r[4]), 0)].tolist()


def accept_margins(zq, zt, d, u0, u1, T, want):
    q = softmax(zq.astype(np.float64) / T)
    p0 = softmax(zt[0].astype(np.float64) / T)
    p1 = softmax(zt[1].astype(np.float64) / T)
    m_acc = abs(u0 * q[d] - p0[d])
    if want["accept_count"]:
        dist = p1
    else:
        r = np.maximum(p0 - q, 0.0)
        dist = r / r.sum() if r.sum() > 0 else p0
    return m_acc, boundary_margin(dist, want["free_token"], u1)


@pytest.mark.parametrize("V,T", [(5000, 1.0), (248320, 0.8), (1500, 1.3)])
def test_accept_sampled_matches_the_oracle(V, T):
    print(f"\n[accept] V={V} T={T}", flush=True)
    rng = np.random.default_rng(V)
    zq = rng.normal(0, 2, V).astype(np.float32)
    zt = rng.normal(0, 2, (2, V)).astype(np.float32)
    zt[0] = zq + rng.normal(0, 1, V).astype(np.float32)  # a drafter that tracks the target
    q = softmax(zq.astype(np.float64) / T)
    p0 = softmax(zt[0].astype(np.float64) / T)
    ratio = p0 / q
    top = np.argsort(-q)[:200]  # drafts the drafter would plausibly propose
    cases = [(int(top[np.argmax(ratio[top])]), 0.9), (int(top[np.argmin(ratio[top])]), 0.999)]
    cases += [(int(rng.choice(top)), float(rng.random())) for _ in range(14)]
    seen = {0: 0, 1: 0}
    checked = 0
    p1 = softmax(zt[1].astype(np.float64) / T)
    r = np.maximum(p0 - q, 0.0)
    r /= r.sum()
    for d, u0 in cases:
        u0 = float(np.float32(u0))
        # u1 at a clear point of the distribution the draw will come from
        u1 = clear_uniform(p1 if u0 * q[d] < p0[d] else r, rng)
        want = orc.accept_sampled(zq, zt, d, u0, u1, T)
        got, com = gpu_accept(zq, zt, d, u0, u1, T)
        m_acc, m_draw = accept_margins(zq, zt, d, u0, u1, T, want)
        if m_acc <= MARGIN * max(q[d], p0[d]):
            continue
        assert got[0] == want["accept_count"], f"d={d} u0={u0}: accept {got[0]} vs {want['accept_count']}"
        assert got[2] == want["rollback"]
        seen[int(got[0])] += 1
        if m_draw > MARGIN:
            assert got[1] == want["free_token"], f"d={d}: free token {got[1]} vs {want['free_token']}"
            assert com == want["committed"]
            checked += 1
    assert seen[0] > 0 and seen[1] > 0, seen
    assert checked >= sum(seen.values()) - 1


def test_accept_sampled_small_vocabulary_grid():
    """Every draft of an 8-token vocabulary against a grid of uniforms: both the
    acceptance decisions and the free tokens follow the oracle's."""
    rng = np.random.default_rng(77)
    V = 8
    zq = rng.normal(0, 1.5, V).astype(np.float32)
    zt = rng.normal(0, 1.5, (2, V)).astype(np.float32)
    grid = ((np.arange(16) + 0.5) / 16).astype(np.float32)
    n = 0
    for d in range(V):
        for u0 in grid:
            for u1 in grid[::3]:
                want = orc.accept_sampled(zq, zt, d, float(u0), float(u1))
                m_acc, m_draw = accept_margins(zq, zt, d, float(u0), float(u1), 1.0, want)
                if m_acc <= MARGIN or m_draw <= MARGIN:
                    continue
                got, com = gpu_accept(zq, zt, d, float(u0), float(u1))
                assert got[0] == want["accept_count"] and got[1] == want["free_token"], (d, u0, u1)
                assert com == want["committed"]
                n += 1
    assert n > 500


def test_accept_sampled_special_cases():
    rng = np.random.default_rng(5)
    V = 3000
    zq = rng.normal(0, 2, V).astype(np.float32)
    zt = rng.normal(0, 2, (2, V)).astype(np.float32)
    same = zt.copy()
    same[0] = zq
    for d in (0, 17, V - 1):  # identical distributions: always accepted
        got, _ = gpu_accept(zq, same, d, 0.999, 0.5)
        assert got[0] == 1 and got[2] == 0
    got, com = gpu_accept(zq, zt, V, 0.5, 0.5)  # not a token: nothing read at d
    assert got.tolist() == [-1, -1, -1, 0, 0] and com == []
    got, _ = gpu_accept(zq, zt, -1, 0.5, 0.5)
    assert got.tolist() == [-1, -1, -1, 0, 0]
    q = softmax(zq.astype(np.float64))
    p0 = softmax(zt[0].astype(np.float64))
    d = int(np.argmax(p0 / q))  # always accepted; EOS on the draft stops the commit
    got, com = gpu_accept(zq, zt, d, 0.5, 0.5, eos=np.array([d], np.int32))
    assert got[0] == 1 and got[3] == 1 and com == [d]
