"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks an oracle function against what the pages print (tests/golden),
a closed form, an invariant of the method, a library routine on a special case,
or brute force on tiny inputs. Chosen so that a dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

from verifier_block_forward_amd import configs, synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _dec(u16):
    """Independent BF16 decode for the tests: numpy bit reinterpretation."""
    return (np.asarray(u16, np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# BF16 (tensors.rs test module facts; RNE cases)
# ---------------------------------------------------------------------------

def test_bf16_canonical_round_trip(orc):
    g = _gold("bf16_facts.json")
    vals = np.array(g["canonical_values"], np.float32)
    raw = (vals.view(np.uint32) >> 16).astype("<u2").tobytes()
    out = orc.decode_bf16_bytes(raw)
    assert out.view(np.uint32).tolist() == vals.view(np.uint32).tolist()


def test_bf16_one_bytes_and_misread_signature(orc):
    g = _gold("bf16_facts.json")
    one = synth.bf16_rne(np.array([1.0], np.float32))
    assert list(one.astype("<u2").tobytes()) == g["one_le_bytes"]
    two = np.array([1.0, 1.0], np.float32)
    raw = synth.bf16_rne(two).astype("<u2").tobytes()
    misread = np.frombuffer(raw, "<u4")[0]
    assert misread == int(g["two_ones_read_as_f32_bits"], 16)
    assert np.frombuffer(raw, "<f4")[0] != 1.0
    # the oracle decodes the same bytes element-wise, not as F32 words
    assert orc.decode_bf16_bytes(raw).tolist() == [1.0, 1.0]


def test_bf16_odd_length_rejected(orc):
    g = _gold("bf16_facts.json")
    with pytest.raises(ValueError) as e:
        orc.decode_bf16_bytes(bytes(g["odd_length_bytes"]))
    assert g["odd_length_error_contains"] in str(e.value)


@pytest.mark.parametrize("case", _gold("bf16_rne_cases.json")["cases"])
def test_bf16_rne_cases(orc, case):
    src, want, _ = case
    f = np.array([int(src, 16)], np.uint32).view(np.float32)
    assert orc.f32_to_bf16(float(f[0])) == int(want, 16)
    assert int(synth.bf16_rne(f)[0]) == int(want, 16)


def test_bf16_encode_decode_identity_on_exact_values(orc):
    rng = np.random.default_rng(7)
    bits = (rng.integers(0, 0xFFFF, 4096).astype(np.uint32) << 16)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    enc = synth.bf16_rne(f)
    assert np.array_equal(_dec(enc), f.astype(np.float64))
    for x in f[:64]:
        assert orc.f32_to_bf16(float(x)) == int(np.array([x], np.float32).view(np.uint32)[0] >> 16)


def test_synth_chunking_independent_of_threads():
    a = synth.normal_f32(5, 3, (synth.CHUNK * 2 + 17,))
    b = synth.normal_f32(5, 3, (synth.CHUNK * 2 + 17,))
    assert np.array_equal(a, b)
    # first chunk equals a fresh single-chunk draw of the same stream
    c = synth.normal_f32(5, 3, (100,))
    assert np.array_equal(a[:100], c)


# ---------------------------------------------------------------------------
# RMSNorm: unit RMS, weight scaling, scale invariance, constant-vector closed form
# ---------------------------------------------------------------------------

def test_rmsnorm_unit_rms(orc):
    rng = np.random.default_rng(1)
    for n in (1, 7, 256, 2816):
        x = rng.standard_normal(n) * 3.0
        eps = 1e-6
        y = orc.rmsnorm(x, np.ones(n, np.float32), eps)
        ms = np.mean(x * x)
        assert np.isclose(np.mean(y * y), ms / (ms + eps), rtol=1e-12)


def test_rmsnorm_weight_scaling_and_x_scaling(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(64)
    w = (1 + 0.1 * rng.standard_normal(64)).astype(np.float32)
    y = orc.rmsnorm(x, w, 0.0)
    y2 = orc.rmsnorm(x, (2 * w).astype(np.float32), 0.0)
    assert np.allclose(y2, 2 * y, rtol=1e-14, atol=0)
    y3 = orc.rmsnorm(5.0 * x, w, 0.0)
    assert np.allclose(y3, y, rtol=1e-13, atol=0)
    # elementwise weight: each lane scales only its own output
    w2 = w.copy()
    w2[5] *= 3
    y4 = orc.rmsnorm(x, w2, 0.0)
    assert np.isclose(y4[5], 3 * y[5], rtol=1e-14) and np.array_equal(np.delete(y4, 5), np.delete(y, 5))


def test_rmsnorm_constant_vector_closed_form(orc):
    for a in (0.5, -2.0, 1e-3):
        eps = 1e-6
        w = np.linspace(0.5, 1.5, 10).astype(np.float32)
        y = orc.rmsnorm(np.full(10, a), w, eps)
        assert np.allclose(y, a / math.sqrt(a * a + eps) * w.astype(np.float64), rtol=1e-14)


# ---------------------------------------------------------------------------
# Linear over BF16 [out, in]
# ---------------------------------------------------------------------------

def test_linear_brute_force_non_square(orc):
    rng = np.random.default_rng(3)
    M, K, N = 3, 7, 5
    X = rng.standard_normal((M, K))
    W = synth.bf16_rne(rng.standard_normal((N, K)).astype(np.float32))
    Y = orc.linear(X, W)
    Wd = _dec(W)
    for m in range(M):
        for o in range(N):
            assert math.isclose(Y[m, o], math.fsum(X[m, k] * Wd[o, k] for k in range(K)),
                                rel_tol=1e-13, abs_tol=1e-15)


def test_linear_identity_and_one_hot(orc):
    K = 16
    eye = synth.bf16_rne(np.eye(K, dtype=np.float32))
    X = np.random.default_rng(4).standard_normal((2, K))
    assert np.array_equal(orc.linear(X, eye), X)
    W = synth.bf16_rne(np.random.default_rng(5).standard_normal((6, K)).astype(np.float32))
    onehot = np.zeros((1, K))
    onehot[0, 3] = 1.0
    assert np.array_equal(orc.linear(onehot, W)[0], _dec(W)[:, 3])


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def test_rope_position_zero_identity(orc):
    v = np.random.default_rng(6).standard_normal(64)
    assert np.array_equal(orc.rope(v, 64, 0.0, 1e6), v)


def test_rope_pair_zero_one_radian(orc):
    d = 8
    v = np.zeros(d)
    v[0] = 1.0
    r = orc.rope(v, d, 1.0, 1e6)
    assert np.allclose([r[0], r[d // 2]], [math.cos(1.0), math.sin(1.0)], atol=1e-15)
    v = np.zeros(d)
    v[d // 2] = 1.0
    r = orc.rope(v, d, 1.0, 1e6)
    assert np.allclose([r[0], r[d // 2]], [-math.sin(1.0), math.cos(1.0)], atol=1e-15)
    # only the rotate-half partner lanes mix
    assert np.count_nonzero(np.abs(r) > 1e-15) == 2


def test_rope_frequency_closed_form(orc):
    # d=4, j=1: inv_freq = theta^(-1/2) = 1e-3 for theta=1e6 -> position 1000 turns pair 1 by 1 rad
    v = np.array([0.0, 1.0, 0.0, 0.0])
    r = orc.rope(v, 4, 1000.0, 1e6)
    assert np.allclose(r, [0.0, math.cos(1.0), 0.0, math.sin(1.0)], atol=1e-12)


def test_rope_norm_preserved_and_relative(orc):
    rng = np.random.default_rng(7)
    d = 128
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n in ((5, 3), (40000, 39990), (17, 17)):
        rq, rk = orc.rope(q, d, m, 1e6), orc.rope(k, d, n, 1e6)
        half = d // 2
        assert np.allclose(rq[:half] ** 2 + rq[half:] ** 2, q[:half] ** 2 + q[half:] ** 2, rtol=1e-12)
        for delta in (1, 1000):
            sq, sk = orc.rope(q, d, m + delta, 1e6), orc.rope(k, d, n + delta, 1e6)
            assert math.isclose(rq @ rk, sq @ sk, rel_tol=1e-9, abs_tol=1e-9)


def test_rope_partial_rotary_passthrough(orc):
    v = np.random.default_rng(8).standard_normal(64)
    r = orc.rope(v, 32, 123.0, 1e6)
    assert np.array_equal(r[32:], v[32:])
    assert not np.allclose(r[:32], v[:32])


def test_rope_composes(orc):
    v = np.random.default_rng(9).standard_normal(64)
    assert np.allclose(orc.rope(orc.rope(v, 64, 7.0, 1e6), 64, 5.0, 1e6), orc.rope(v, 64, 12.0, 1e6),
                       atol=1e-12)


# ---------------------------------------------------------------------------
# SDPA
# ---------------------------------------------------------------------------

def test_sdpa_matches_full_matrix_brute_force(orc):
    rng = np.random.default_rng(10)
    n, d, nq = 9, 16, 4
    Q = rng.standard_normal((nq, d))
    Kc = rng.standard_normal((n, d))
    Vc = rng.standard_normal((n, d))
    # causal over the last nq keys: query i sees keys [0, n - nq + i]
    mask = np.full((nq, n), -np.inf)
    for i in range(nq):
        mask[i, : n - nq + i + 1] = 0.0
    P = softmax(Q @ Kc.T / math.sqrt(d) + mask, axis=1)
    ref = P @ Vc
    for i in range(nq):
        cnt = n - nq + i + 1
        o = orc.sdpa_one(Q[i], Kc[:cnt], Vc[:cnt])
        assert np.allclose(o, ref[i], rtol=1e-12, atol=1e-14)


def test_sdpa_special_cases(orc):
    rng = np.random.default_rng(11)
    d = 8
    q, k, v = rng.standard_normal(d), rng.standard_normal((1, d)), rng.standard_normal((1, d))
    assert np.allclose(orc.sdpa_one(q, k, v), v[0], rtol=0, atol=1e-15)
    keys = np.repeat(k, 5, axis=0)
    vals = rng.standard_normal((5, d))
    assert np.allclose(orc.sdpa_one(q, keys, vals), vals.mean(axis=0), rtol=1e-13)
    # a huge shift of all scores changes nothing (max subtraction)
    assert np.allclose(orc.sdpa_one(q * 1e3, keys, vals), vals.mean(axis=0), rtol=1e-13)


# ---------------------------------------------------------------------------
# MoE routing
# ---------------------------------------------------------------------------

def test_moe_route_full_topk_is_softmax(orc):
    z = np.random.default_rng(12).standard_normal(16)
    sel, w, gap = orc.moe_route(z, 16)
    p = softmax(z)
    assert sorted(sel.tolist()) == list(range(16))
    assert np.allclose(w, p[sel], rtol=1e-13)
    assert gap == math.inf


def test_moe_route_topk_properties(orc):
    rng = np.random.default_rng(13)
    z = rng.standard_normal(256)
    sel, w, gap = orc.moe_route(z, 8)
    assert np.isclose(w.sum(), 1.0, rtol=1e-14)
    order = np.argsort(-z, kind="stable")
    assert sel.tolist() == order[:8].tolist()
    assert np.isclose(gap, z[order[7]] - z[order[8]])
    p = softmax(z)
    assert np.allclose(w, p[sel] / p[sel].sum(), rtol=1e-13)
    sel1, w1, _ = orc.moe_route(z, 1)
    assert sel1[0] == int(np.argmax(z)) and w1[0] == 1.0


def test_moe_route_ties_lower_index(orc):
    z = np.zeros(6)
    z[[1, 3, 4]] = 2.0
    sel, _, gap = orc.moe_route(z, 2)
    assert sel.tolist() == [1, 3] and gap == 0.0


# ---------------------------------------------------------------------------
# lm_head argmax
# ---------------------------------------------------------------------------

def test_lm_head_argmax_brute_force_and_ties(orc):
    rng = np.random.default_rng(14)
    H, V = 24, 300
    W = synth.bf16_rne(rng.standard_normal((V, H)).astype(np.float32) * 0.1)
    W[[17, 250]] = W[40]  # three identical rows
    h = rng.standard_normal((3, H))
    logits, am, mg = orc.lm_head(h, W)
    ref = h @ _dec(W).T
    assert np.allclose(logits, ref, rtol=1e-12, atol=1e-14)
    for m in range(3):
        assert am[m] == int(np.argmax(logits[m]))
        s = np.sort(logits[m])
        assert np.isclose(mg[m], s[-1] - s[-2])
    # force a tie at the top: lowest index wins, margin 0
    hb = _dec(W)[40][None, :] * 50.0
    _, am2, mg2 = orc.lm_head(hb, W)
    assert am2[0] == 17 and mg2[0] == 0.0


# ---------------------------------------------------------------------------
# Accept walk (orchestrator greedy accept-prefix invariants), exhaustive K <= 10
# ---------------------------------------------------------------------------

def test_accept_walk_exhaustive(orc):
    for K in range(1, 11):
        for pattern in range(1 << K):
            d = np.arange(100, 100 + K, dtype=np.int32)
            t = np.concatenate([d, [7]]).astype(np.int32)
            for i in range(K):
                if not (pattern >> i) & 1:
                    t[i] = 5 + i
            r = orc.accept_prefix(d, t)
            a = r["accept_count"]
            assert all(d[i] == t[i] for i in range(a))
            assert a == K or d[a] != t[a]
            assert r["free_token"] == t[a]
            assert r["rollback"] == K - a
            assert r["committed"] == t[: a + 1].tolist()
            assert not r["hit_eos"]


def test_accept_walk_seeded_targets(orc):
    for K in (1, 3, 15):
        for s in range(20):
            d = np.random.default_rng(s).integers(0, 4096, K).astype(np.int32)
            t, j = synth.accept_targets(d, 4096, seed=s)
            r = orc.accept_prefix(d, t)
            assert r["accept_count"] == j and r["rollback"] == K - j


def test_accept_walk_eos(orc):
    d = np.array([1, 2, 3, 4], np.int32)
    t = np.array([1, 2, 3, 9, 8], np.int32)
    r = orc.accept_prefix(d, t, eos=[2])
    assert r["accept_count"] == 3 and r["rollback"] == 1 and r["hit_eos"]
    assert r["committed"] == [1, 2] and r["free_token"] == 9
    r = orc.accept_prefix(d, t, eos=[9])
    assert r["committed"] == [1, 2, 3, 9] and r["hit_eos"]
    r = orc.accept_prefix(d, t, eos=[77])
    assert r["committed"] == [1, 2, 3, 9] and not r["hit_eos"]


def test_kv_rollback_bounds(orc):
    assert orc.kv_rollback(10, 3) == 7
    assert orc.kv_rollback(10, 10) == 0
    with pytest.raises(ValueError):
        orc.kv_rollback(10, 11)
    with pytest.raises(ValueError):
        orc.kv_rollback(10, -1)
