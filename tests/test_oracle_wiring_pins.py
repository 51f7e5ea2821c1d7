"""Wiring pins of the oracle block: which weight meets which vector.

The building blocks (RMSNorm, Linear, RoPE, SDPA, routing) have their own pins.
These tests pin how the block composes them, on special cases whose result is
fixed by the method itself:

* the per-head q/k RMSNorm (qwen35/mtp.rs `forward_full_attention`, per-head
  q/k norm): each head normalised on its own, q with q_norm and k with k_norm;
* the DFlash context rows (dflash/tensors.rs `DFlashModelTensors`: fc and
  hidden_norm): h_ctx = RMSNorm(T fc^T; hidden_norm) feeds every layer's Wk/Wv,
  then k_norm and RoPE at P0 + r for keys, nothing for values, and no in_norm;
* the MoE expert indexing (qwen35/mtp.rs `MtpFfnWeightsGpu::Moe`): each row's
  routing weights multiply the SwiGLU of the experts the router picked.

Expected values are computed here in numpy from the definitions, on inputs
chosen so that they reduce to short closed forms (one-hot weights, constant
rows, a single cached key).
"""
import math

import numpy as np
from scipy.special import expit

from verifier_block_forward_amd import configs, synth

BF16_ONE = 0x3F80


def _dec(u16):
    return (np.asarray(u16, np.uint32) << 16).view(np.float32).astype(np.float64)


def _enc(x):
    return synth.bf16_rne(np.asarray(x, np.float32))


def _rope(v, pos, theta):
    """Rotate-half RoPE of one head vector (pair j, j + d/2 turns by pos * theta^(-2j/d));
    the sign convention is the one pinned by the RoPE pins."""
    d = v.size
    h = d // 2
    out = v.astype(np.float64).copy()
    for j in range(h):
        a = pos * theta ** (-2.0 * j / d)
        c, s = math.cos(a), math.sin(a)
        out[j] = v[j] * c - v[j + h] * s
        out[j + h] = v[j] * s + v[j + h] * c
    return out


def _rms_unit(v):
    return v / math.sqrt(float(np.mean(np.asarray(v, np.float64) ** 2)))


def tiny(**kw):
    base = dict(name="wiring", seed=21, kind="dflash", n_layers=1, hidden=32, n_q_heads=4,
                n_kv_heads=2, head_dim=8, vocab=64, M=3, R=2, C=4, kv_dtype="f32",
                intermediate=24, n_target_hidden=2, block_input="x0")
    base.update(kw)
    return configs.BlockConfig(**base)


def _scaled_rows(w, rows, c):
    """BF16 weight with `rows` multiplied by the power of two c (exact)."""
    out = w.copy()
    out[rows] = _enc(_dec(w[rows]) * c)
    assert np.array_equal(_dec(out[rows]), _dec(w[rows]) * c)
    return out


# ---------------------------------------------------------------------------
# per-head q/k RMSNorm
# ---------------------------------------------------------------------------

def test_per_head_norm_scale_invariance(orc):
    """With eps = 0 each head's RMSNorm is exactly invariant to scaling that head's
    projection rows by a power of two, so scaling the last q head's rows of Wq, or
    the last kv head's rows of Wk, changes nothing. A norm over the whole q (or k)
    vector, or over too few heads, is not invariant."""
    cfg = tiny(rms_eps=0.0, n_layers=2)
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    base = orc.block_forward(cfg, w, inp)
    hd, nq, nkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    for layer in range(cfg.n_layers):
        for name, head, c in (("wq", nq - 1, 2.0), ("wk", nkv - 1, 4.0), ("wq", 0, 0.5)):
            w2 = dict(w)
            key = f"layers.{layer}.{name}"
            w2[key] = _scaled_rows(w[key], slice(head * hd, (head + 1) * hd), c)
            out = orc.block_forward(cfg, w2, inp)
            assert np.array_equal(out["attn_out"], base["attn_out"]), (layer, name, head)
            assert np.array_equal(out["h_final"], base["h_final"]), (layer, name, head)
    # the value rows are not normalised: scaling them scales that head's output
    w2 = dict(w)
    w2["layers.0.wv"] = _scaled_rows(w["layers.0.wv"], slice(0, hd), 2.0)
    out = orc.block_forward(cfg, w2, inp)
    assert not np.allclose(out["attn_out"][0], base["attn_out"][0])


def test_q_norm_and_k_norm_roles_two_key_closed_form(orc):
    """One block row at position 1 over one cached key (position 0). Wk = 0 and
    Wv = 0 make the row's own key and value zero (score 0, value 0); the cached
    value is all ones. So each q head's output is sigma(s) in every lane, with
    s = RoPE_1(u_h / rms(u_h) * q_norm) . k0[kv(h)] / sqrt(hd), where u_h is the
    raw query of head h (one-hot Wq on a constant row). Swapping q_norm and k_norm,
    normalising q over all heads, a wrong position, or a wrong GQA group each
    change some head's sigma(s)."""
    H, nq, nkv, hd = 32, 4, 2, 8
    cfg = tiny(rms_eps=1e-30, M=1, R=0, C=1, hidden=H, n_q_heads=nq, n_kv_heads=nkv, head_dim=hd)
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    qt, kt = nq * hd, nkv * hd
    rng = np.random.default_rng(5)
    # raw queries: exact small BF16 values with a different RMS per head
    u = np.round(rng.uniform(-4, 4, qt) * 4) / 4
    u[u == 0] = 0.75
    u[hd:2 * hd] *= 3.0
    wq = np.zeros((qt, H), np.uint16)
    wq[:, 0] = _enc(u)
    assert np.array_equal(_dec(wq[:, 0]), u)
    w["layers.0.wq"] = wq
    w["layers.0.wk"] = np.zeros((kt, H), np.uint16)
    w["layers.0.wv"] = np.zeros((kt, H), np.uint16)
    w["layers.0.in_norm"] = np.ones(H, np.float32)
    q_norm = (1.0 + 0.5 * rng.standard_normal(hd)).astype(np.float32)
    k_norm = (1.0 + 0.5 * rng.standard_normal(hd)).astype(np.float32)
    w["layers.0.q_norm"] = q_norm
    w["layers.0.k_norm"] = k_norm
    inp["x0"] = np.ones((1, H), np.float32)  # x_hat = 1 in every lane
    k0 = rng.standard_normal((nkv, hd)).astype(np.float32)
    inp["cache_k"][0, :, 0, :] = k0
    inp["cache_v"][0, :, 0, :] = 1.0
    out = orc.block_forward(cfg, w, inp)
    o = out["attn_out"][0, 0].reshape(nq, hd)
    swapped = []
    for h in range(nq):
        kvh = h * nkv // nq
        uh = u[h * hd:(h + 1) * hd]
        q = _rope(_rms_unit(uh) * q_norm.astype(np.float64), 1.0, cfg.rope_theta)
        s = float(q @ k0[kvh].astype(np.float64)) / math.sqrt(hd)
        assert np.allclose(o[h], expit(s), rtol=1e-12, atol=1e-15), h
        qs = _rope(_rms_unit(uh) * k_norm.astype(np.float64), 1.0, cfg.rope_theta)
        swapped.append(expit(float(qs @ k0[kvh].astype(np.float64)) / math.sqrt(hd)))
    # the alternative readings really are distinguishable on these inputs
    assert not np.allclose(o[:, 0], swapped, rtol=1e-6)
    qall = u / math.sqrt(float(np.mean(u ** 2)))
    whole = [expit(float(_rope(qall[h * hd:(h + 1) * hd] * q_norm, 1.0, cfg.rope_theta)
                         @ k0[h * nkv // nq]) / math.sqrt(hd)) for h in range(nq)]
    assert not np.allclose(o[:, 0], whole, rtol=1e-6)


def test_own_value_is_unnormalised_projection(orc):
    """A block row with no cached prefix and no context rows attends only to itself,
    so its output is its own value row: v = x_hat Wv^T, with no norm and no RoPE,
    as stored in the F32 cache (rounded to F32 there)."""
    cfg = tiny(M=1, R=0, C=0)
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    out = orc.block_forward(cfg, w, inp)
    x_hat = orc.rmsnorm(inp["x0"][0].astype(np.float64), w["layers.0.in_norm"], cfg.rms_eps)
    v = _dec(w["layers.0.wv"]) @ x_hat
    hd, nq, nkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    o = out["attn_out"][0, 0].reshape(nq, hd)
    for h in range(nq):
        kvh = h * nkv // nq
        want = v[kvh * hd:(kvh + 1) * hd].astype(np.float32).astype(np.float64)
        assert np.allclose(o[h], want, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# DFlash context rows
# ---------------------------------------------------------------------------

def test_context_rows_absorb_fc_scale(orc):
    """hidden_norm normalises the fc output, so with eps = 0 scaling fc by a power of
    two leaves every output and every written cache row unchanged."""
    cfg = tiny(rms_eps=0.0, n_layers=2, R=3)
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    a = orc.block_forward(cfg, w, inp)
    w2 = dict(w, fc=_scaled_rows(w["fc"], slice(None), 4.0))
    b = orc.block_forward(cfg, w2, inp)
    assert np.array_equal(a["h_final"], b["h_final"])
    assert np.array_equal(a["cache_k"], b["cache_k"])
    assert np.array_equal(a["cache_v"], b["cache_v"])


def test_context_row_cache_closed_form(orc):
    """One context row, one-hot weights. fc picks the second target state
    (proj = T[H:2H]), so h_ctx = T[H:2H] / rms * hidden_norm. Layer 0's Wk picks
    h_ctx[0:kt] and layer 1's Wk picks it in reverse; Wv picks h_ctx[kt:2kt]. The
    key cached at P0 is then, per kv head, RoPE_P0(k_raw / rms * k_norm) and the
    value is v_raw itself, in both layers (the context rows bypass in_norm and the
    layer chain)."""
    H, nkv, hd, nt = 32, 2, 8, 2
    kt = nkv * hd
    cfg = tiny(n_layers=2, M=2, R=1, C=3, hidden=H, n_kv_heads=nkv, head_dim=hd, n_target_hidden=nt)
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    fc = np.zeros((H, nt * H), np.uint16)
    fc[np.arange(H), H + np.arange(H)] = BF16_ONE
    w["fc"] = fc
    picks_k = [np.arange(kt), kt - 1 - np.arange(kt)]
    for layer in range(2):
        wk = np.zeros((kt, H), np.uint16)
        wk[np.arange(kt), picks_k[layer]] = BF16_ONE
        wv = np.zeros((kt, H), np.uint16)
        wv[np.arange(kt), kt + np.arange(kt)] = BF16_ONE
        w[f"layers.{layer}.wk"] = wk
        w[f"layers.{layer}.wv"] = wv
    out = orc.block_forward(cfg, w, inp)
    P0 = cfg.C
    T = inp["ctx"][0].astype(np.float64)
    hn = w["hidden_norm"].astype(np.float64)
    r = T[H:2 * H]
    h_ctx = r / math.sqrt(float(np.mean(r ** 2)) + cfg.rms_eps) * hn
    for layer in range(2):
        k_norm = w[f"layers.{layer}.k_norm"].astype(np.float64)
        k_raw = h_ctx[picks_k[layer]]
        v_raw = h_ctx[kt:2 * kt]
        for h in range(nkv):
            seg = k_raw[h * hd:(h + 1) * hd]
            kn = seg / math.sqrt(float(np.mean(seg ** 2)) + cfg.rms_eps) * k_norm
            want_k = _rope(kn, float(P0), cfg.rope_theta)
            got_k = out["cache_k"][layer, h, P0]
            got_v = out["cache_v"][layer, h, P0]
            assert np.allclose(got_k, want_k.astype(np.float32), rtol=2e-7, atol=1e-8), (layer, h)
            assert np.allclose(got_v, v_raw[h * hd:(h + 1) * hd].astype(np.float32), rtol=2e-7,
                               atol=1e-8), (layer, h)
    # an in_norm applied to the context rows would be visible: in_norm is not all ones
    assert np.ptp(w["layers.0.in_norm"]) > 0.1


# ---------------------------------------------------------------------------
# MoE expert indexing
# ---------------------------------------------------------------------------

def _moe(**kw):
    base = dict(kind="mtp", R=0, M=4, n_layers=1, ffn_kind="moe", n_experts=8, top_k=1,
                expert_intermediate=6, shared_intermediate=6, intermediate=6, C=5)
    base.update(kw)
    return tiny(**base)


def _dense_runs(orc, cfg, w, inp):
    """hidden_out of the same block with a dense FFN equal to each expert in turn,
    and with a zero FFN (which gives x1, the FFN's residual input)."""
    dense = cfg.with_(ffn_kind="dense", intermediate=cfg.expert_intermediate)
    runs = []
    for e in range(cfg.n_experts):
        wd = dict(w)
        wd["layers.0.ffn_gate"] = w["layers.0.exp_gate"][e]
        wd["layers.0.ffn_up"] = w["layers.0.exp_up"][e]
        wd["layers.0.ffn_down"] = w["layers.0.exp_down"][e]
        runs.append(orc.block_forward(dense, wd, inp)["hidden_out"])
    wz = dict(w)
    wz["layers.0.ffn_gate"] = w["layers.0.exp_gate"][0]
    wz["layers.0.ffn_up"] = w["layers.0.exp_up"][0]
    wz["layers.0.ffn_down"] = np.zeros_like(w["layers.0.exp_down"][0])
    x1 = orc.block_forward(dense, wz, inp)["hidden_out"]
    return np.stack(runs), x1


def _router_logits(orc, cfg, w, x1):
    x2 = np.stack([orc.rmsnorm(x1[m], w["layers.0.post_norm"], cfg.rms_eps) for m in range(cfg.M)])
    return x2 @ _dec(w["layers.0.router"]).T


def test_moe_top1_is_the_argmax_expert(orc):
    """top_k = 1 with distinct experts and no shared branch: row m's output equals the
    dense SwiGLU of expert argmax_e(router logit), exactly (weight 1)."""
    cfg = _moe()
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    w["layers.0.sh_down"] = np.zeros_like(w["layers.0.sh_down"])
    moe = orc.block_forward(cfg, w, inp)
    dense, x1 = _dense_runs(orc, cfg, w, inp)
    z = _router_logits(orc, cfg, w, x1)
    picks = z.argmax(axis=1)
    assert len(set(picks.tolist())) > 1  # rows route to different experts
    for m in range(cfg.M):
        assert moe["moe_sel"][0, m, 0] == picks[m]
        assert np.allclose(moe["hidden_out"][m], dense[picks[m], m], rtol=1e-12, atol=1e-14), m
        others = [e for e in range(cfg.n_experts) if e != picks[m]]
        assert not any(np.allclose(moe["hidden_out"][m], dense[e, m], rtol=1e-6) for e in others)


def test_moe_top2_closed_form_weights(orc):
    """top_k = 2: the renormalised weight of the first expert is sigma(z_a - z_b), so
    y_m = x1 + sigma(d) (D_a - x1) + (1 - sigma(d)) (D_b - x1), with a, b the two
    largest router logits of row m and D_e the dense run of expert e."""
    cfg = _moe(top_k=2)
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    w["layers.0.sh_down"] = np.zeros_like(w["layers.0.sh_down"])
    moe = orc.block_forward(cfg, w, inp)
    dense, x1 = _dense_runs(orc, cfg, w, inp)
    z = _router_logits(orc, cfg, w, x1)
    for m in range(cfg.M):
        order = np.argsort(-z[m], kind="stable")
        a, b = int(order[0]), int(order[1])
        wa = expit(z[m, a] - z[m, b])
        want = x1[m] + wa * (dense[a, m] - x1[m]) + (1.0 - wa) * (dense[b, m] - x1[m])
        assert np.allclose(moe["hidden_out"][m], want, rtol=1e-11, atol=1e-13), m
        assert moe["moe_sel"][0, m].tolist() == [a, b]
