"""Block-level pins of the oracle: invariants the drafter block must satisfy.

The pages print no worked example of hidden states or logits, so the composed
block is pinned through properties of the method rather than through values:
the residual chain, the causal in-block mask and the row positions (a block of
M rows equals M single-row calls), incremental context plus rollback, GQA as
MHA over repeated K/V, the sigmoid gate, SwiGLU's operand order, the MTP eh
split, and the MoE reductions.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

from verifier_block_forward_amd import configs, synth


def _dec(u16):
    return (np.asarray(u16, np.uint32) << 16).view(np.float32).astype(np.float64)


def tiny(**kw):
    base = dict(name="tiny", seed=11, kind="dflash", n_layers=2, hidden=32, n_q_heads=4,
                n_kv_heads=2, head_dim=8, vocab=64, M=4, R=3, C=5, kv_dtype="f32",
                intermediate=24, n_target_hidden=2, block_input="x0")
    base.update(kw)
    return configs.BlockConfig(**base)


def data(cfg):
    return synth.make_weights(cfg), synth.make_inputs(cfg)


def run(orc, cfg, w, inp, **kw):
    return orc.block_forward(cfg, w, inp, **kw)


def test_residual_chain_zero_branches(orc):
    cfg = tiny()
    w, inp = data(cfg)
    for i in range(cfg.n_layers):
        w[f"layers.{i}.wo"][:] = 0
        w[f"layers.{i}.ffn_down"][:] = 0
    out = run(orc, cfg, w, inp)
    x0 = inp["x0"].astype(np.float64)
    assert np.array_equal(out["hidden_out"], x0)
    for m in range(cfg.M):
        assert np.allclose(out["h_final"][m], orc.rmsnorm(x0[m], w["final_norm"], cfg.rms_eps),
                           rtol=1e-15, atol=0)


def test_causal_chain_equals_single_row_calls(orc):
    """Row i of an M-row block == the i-th of M successive one-row calls: pins the
    causal mask (row i sees block rows <= i) and the row positions P0+R+i."""
    cfg = tiny()
    w, inp = data(cfg)
    full = run(orc, cfg, w, inp)
    ck, cv = inp["cache_k"].copy(), inp["cache_v"].copy()
    s = inp["seq_len"]
    for i in range(cfg.M):
        one = dict(inp)
        one["x0"] = inp["x0"][i: i + 1]
        one["ctx"] = inp["ctx"] if i == 0 else inp["ctx"][:0]
        o = run(orc, cfg, w, one, cache_k=ck, cache_v=cv, seq_len=s, M=1, R=cfg.R if i == 0 else 0)
        s = o["seq_len"]
        assert np.allclose(o["h_final"][0], full["h_final"][i], rtol=1e-12, atol=1e-13)
    assert s == full["seq_len"]
    assert np.allclose(ck, full["cache_k"], rtol=1e-6, atol=1e-7)
    assert np.array_equal(cv, full["cache_v"])


def test_causal_row0_ignores_later_rows(orc):
    cfg = tiny()
    w, inp = data(cfg)
    a = run(orc, cfg, w, inp)
    inp2 = dict(inp)
    inp2["x0"] = inp["x0"].copy()
    inp2["x0"][1:] += 1.0
    b = run(orc, cfg, w, inp2)
    assert np.array_equal(a["h_final"][0], b["h_final"][0])
    assert not np.allclose(a["h_final"][1], b["h_final"][1])


def test_incremental_context_with_rollback(orc):
    """R context rows in one call == two calls of R/2 rows with the block rows
    rolled back in between: pins context positions P0..P0+R-1, block positions
    after them, and that a rollback of M drops exactly the block rows."""
    cfg = tiny(R=6)
    w, inp = data(cfg)
    one = run(orc, cfg, w, inp)
    ck, cv = inp["cache_k"].copy(), inp["cache_v"].copy()
    a = dict(inp)
    a["ctx"] = inp["ctx"][:3]
    oa = run(orc, cfg, w, a, cache_k=ck, cache_v=cv, R=3)
    s = orc.kv_rollback(oa["seq_len"], cfg.M)
    b = dict(inp)
    b["ctx"] = inp["ctx"][3:]
    ob = run(orc, cfg, w, b, cache_k=ck, cache_v=cv, seq_len=s, R=3)
    assert ob["seq_len"] == one["seq_len"]
    assert np.allclose(ob["h_final"], one["h_final"], rtol=1e-12, atol=1e-13)
    assert np.allclose(ck, one["cache_k"], rtol=1e-6, atol=1e-7)


def test_rollback_then_rerun_is_deterministic(orc):
    cfg = tiny()
    w, inp = data(cfg)
    ck, cv = inp["cache_k"].copy(), inp["cache_v"].copy()
    a = run(orc, cfg, w, inp, cache_k=ck, cache_v=cv)
    s = orc.kv_rollback(a["seq_len"], cfg.R + cfg.M)
    b = run(orc, cfg, w, inp, cache_k=ck, cache_v=cv, seq_len=s)
    assert np.array_equal(a["h_final"], b["h_final"])


def test_gqa_equals_mha_on_repeated_kv(orc):
    cfg = tiny(n_q_heads=6, n_kv_heads=2)
    w, inp = data(cfg)
    rep = cfg.n_q_heads // cfg.n_kv_heads
    mha = cfg.with_(n_kv_heads=cfg.n_q_heads)
    w2 = dict(w)
    hd = cfg.head_dim
    for i in range(cfg.n_layers):
        for nm in ("wk", "wv"):
            t = w[f"layers.{i}.{nm}"].reshape(cfg.n_kv_heads, hd, -1)
            w2[f"layers.{i}.{nm}"] = np.repeat(t, rep, axis=0).reshape(mha.kv_total, -1)
    inp2 = dict(inp)
    for nm in ("cache_k", "cache_v"):
        inp2[nm] = np.repeat(inp[nm], rep, axis=1)
    a = run(orc, cfg, w, inp)
    b = run(orc, mha, w2, inp2)
    assert np.array_equal(a["h_final"], b["h_final"])


def test_sigmoid_gate(orc):
    cfg = tiny(kind="mtp", R=0, M=2, has_attn_gate=True, n_layers=1)
    w, inp = data(cfg)
    w["layers.0.attn_gate"][:] = 0
    gated = run(orc, cfg, w, inp)
    ungated = run(orc, cfg.with_(has_attn_gate=False), w, inp)
    assert np.array_equal(gated["attn_out"], 0.5 * ungated["attn_out"])
    # one-hot gate rows: g_j = xhat_j, so o_j scales by sigmoid(xhat_j)
    H = cfg.hidden
    inp["x0"][:] = 0.7  # constant embedding rows
    w["layers.0.attn_gate"][:] = 0
    for j in range(cfg.q_total):
        w["layers.0.attn_gate"][j, j % H] = 0x3F80  # BF16 1.0
    gated = run(orc, cfg, w, inp)
    ungated = run(orc, cfg.with_(has_attn_gate=False), w, inp)
    # recompute the layer input x of the MTP block with the pinned pieces
    e = np.full(H, 0.7)
    for m in range(cfg.M):
        x = orc.linear(orc.rmsnorm(e, w["enorm"], 1e-6)[None], w["eh_embed"])[0] + \
            orc.linear(orc.rmsnorm(inp["ctx"][m].astype(np.float64), w["hnorm"], 1e-6)[None],
                       w["eh_hidden"])[0]
        xh = orc.rmsnorm(x, w["layers.0.in_norm"], cfg.rms_eps)
        scale = expit(xh[np.arange(cfg.q_total) % H])
        assert np.allclose(gated["attn_out"][0, m], ungated["attn_out"][0, m] * scale, rtol=1e-12)


def test_mtp_eh_split_equals_concat_projection(orc):
    cfg = tiny(kind="mtp", R=0, M=3, n_layers=1)
    w, inp = data(cfg)
    w["layers.0.wo"][:] = 0
    w["layers.0.ffn_down"][:] = 0
    out = run(orc, cfg, w, inp)
    H = cfg.hidden
    Wfull = np.concatenate([_dec(w["eh_embed"]), _dec(w["eh_hidden"])], axis=1)  # [H, 2H]
    for m in range(cfg.M):
        cat = np.concatenate([orc.rmsnorm(inp["x0"][m].astype(np.float64), w["enorm"], 1e-6),
                              orc.rmsnorm(inp["ctx"][m].astype(np.float64), w["hnorm"], 1e-6)])
        assert np.allclose(out["hidden_out"][m], Wfull @ cat, rtol=1e-12, atol=1e-14)


def test_swiglu_operand_order(orc):
    cfg = tiny(n_layers=1, R=0, M=1, intermediate=4)
    w, inp = data(cfg)
    H = cfg.hidden
    w["layers.0.wo"][:] = 0
    for nm in ("ffn_gate", "ffn_up", "ffn_down"):
        w[f"layers.0.{nm}"][:] = 0
    w["layers.0.ffn_gate"][0, 0] = 0x3F80   # gate_0 = xhat_0
    w["layers.0.ffn_up"][0, 0] = 0x3F00     # up_0 = 0.5 * xhat_0
    w["layers.0.ffn_down"][1, 0] = 0x3F80   # y_1 = h_0
    c = float(np.float32(-1.3))
    inp["x0"][:] = c
    out = run(orc, cfg, w, inp)
    xh = orc.rmsnorm(np.full(H, c), w["layers.0.post_norm"], cfg.rms_eps)
    g, u = xh[0], 0.5 * xh[0]
    want = g * expit(g) * u
    swapped = u * expit(u) * g
    assert math.isclose(out["hidden_out"][0, 1] - c, want, rel_tol=1e-9)
    assert not math.isclose(want, swapped, rel_tol=1e-3)
    assert np.array_equal(np.delete(out["hidden_out"][0], 1), np.full(H - 1, c))


def _moe_cfg(**kw):
    base = dict(kind="mtp", R=0, M=2, n_layers=1, ffn_kind="moe", n_experts=8, top_k=3,
                expert_intermediate=6, shared_intermediate=6, intermediate=6)
    base.update(kw)
    return tiny(**base)


def test_moe_identical_experts_equal_dense(orc):
    """Identical experts + zero shared branch: renormalised top-k weights sum to 1,
    so the mixture equals one dense SwiGLU with those weights (any top_k)."""
    for top_k in (1, 3, 8):
        cfg = _moe_cfg(top_k=top_k)
        w, inp = data(cfg)
        for nm in ("exp_gate", "exp_up", "exp_down"):
            t = w[f"layers.0.{nm}"]
            t[:] = t[0][None]
        w["layers.0.sh_down"][:] = 0
        moe = run(orc, cfg, w, inp)
        dense = cfg.with_(ffn_kind="dense")
        wd = dict(w)
        wd["layers.0.ffn_gate"] = w["layers.0.exp_gate"][0]
        wd["layers.0.ffn_up"] = w["layers.0.exp_up"][0]
        wd["layers.0.ffn_down"] = w["layers.0.exp_down"][0]
        ref = run(orc, dense, wd, inp)
        assert np.allclose(moe["hidden_out"], ref["hidden_out"], rtol=1e-12, atol=1e-13)


def test_moe_shared_branch_sigmoid_scale(orc):
    cfg = _moe_cfg()
    w, inp = data(cfg)
    w["layers.0.wo"][:] = 0
    w["layers.0.exp_down"][:] = 0
    a = run(orc, cfg, w, inp)
    w0 = dict(w)
    w0["layers.0.sh_gate_inp"] = np.zeros_like(w["layers.0.sh_gate_inp"])
    b = run(orc, cfg, w0, inp)
    x = a["hidden_out"] * 0  # x1 == x (Wo = 0); recover x from the zero-FFN run below
    wz = dict(w)
    wz["layers.0.sh_down"] = np.zeros_like(w["layers.0.sh_down"])
    z = run(orc, cfg, wz, inp)
    x = z["hidden_out"]
    fa, fb = a["hidden_out"] - x, b["hidden_out"] - x
    for m in range(cfg.M):
        xh = orc.rmsnorm(x[m], w["layers.0.post_norm"], cfg.rms_eps)
        s = float(xh @ _dec(w["layers.0.sh_gate_inp"])[0])
        assert np.allclose(fa[m], fb[m] * expit(s) / 0.5, rtol=1e-11, atol=1e-14)


def test_moe_selection_reported(orc):
    cfg = _moe_cfg()
    w, inp = data(cfg)
    out = run(orc, cfg, w, inp)
    assert out["moe_sel"].shape == (1, cfg.M, cfg.top_k)
    for m in range(cfg.M):
        assert len(set(out["moe_sel"][0, m].tolist())) == cfg.top_k
        assert out["moe_gap"][0, m] >= 0


def test_bf16_cache_rows_are_rne_of_f32(orc):
    cfg = tiny(kv_dtype="bf16")
    w, inp = data(cfg)
    f = run(orc, cfg.with_(kv_dtype="f32"), w,
            dict(inp, cache_k=_dec(inp["cache_k"]).astype(np.float32),
                 cache_v=_dec(inp["cache_v"]).astype(np.float32)))
    b = run(orc, cfg, w, inp)
    lo, hi = cfg.C, cfg.C + cfg.R + cfg.M
    # layer 0 sees identical inputs, so its new rows are the RNE of the F32 rows
    assert np.array_equal(b["cache_k"][0, :, lo:hi], synth.bf16_rne(f["cache_k"][0, :, lo:hi]))
    assert np.array_equal(b["cache_v"][0, :, lo:hi], synth.bf16_rne(f["cache_v"][0, :, lo:hi]))


def test_capacity_overflow_rejected(orc):
    cfg = tiny()
    w, inp = data(cfg)
    with pytest.raises(RuntimeError):
        run(orc, cfg, w, inp, seq_len=cfg.C + 1)


def test_mtp_token_input_is_the_embedding_row(orc):
    """A chained MTP step takes embed_t as the embedding row of its token: the same
    block with tokens equals the block with x0 = decode(embed[tokens]) exactly, and
    differs from it once any token changes."""
    cfg = tiny(name="tiny_mtp_tok", kind="mtp", R=0, M=2, n_layers=1, n_target_hidden=0,
               has_attn_gate=True, block_input="tokens")
    w, inp = data(cfg)
    toks = np.array([5, 63], np.int32)
    by_tok = dict(inp, tokens=toks)
    by_x0 = {k: v for k, v in inp.items() if k != "tokens"}
    by_x0["x0"] = _dec(w["embed"][toks]).astype(np.float32)
    a = run(orc, cfg, w, by_tok)
    b = run(orc, cfg, w, by_x0)
    assert np.array_equal(a["h_final"], b["h_final"])
    assert np.array_equal(a["hidden_out"], b["hidden_out"])
    c = run(orc, cfg, w, dict(inp, tokens=np.array([6, 63], np.int32)))
    assert not np.allclose(c["h_final"][0], a["h_final"][0])


def test_bidirectional_block_mask(orc):
    """Block-diffusion reading of the in-block mask: every block row attends to all M
    block rows. With one row it equals the causal block exactly; in a one-layer block
    the last row sees the same keys under both masks (exactly equal) while earlier
    rows differ; and row 0 now depends on the later rows."""
    cfg = tiny(n_layers=1)
    bid = tiny(n_layers=1, block_mask="bidirectional")
    w, inp = data(cfg)
    c = run(orc, cfg, w, inp)
    b = run(orc, bid, w, inp)
    assert np.array_equal(b["h_final"][-1], c["h_final"][-1])
    for m in range(cfg.M - 1):
        assert not np.allclose(b["h_final"][m], c["h_final"][m])
    w2, inp2_ = data(tiny(n_layers=2, M=1))
    one_c = run(orc, tiny(n_layers=2, M=1), w2, inp2_)
    one_b = run(orc, tiny(n_layers=2, M=1, block_mask="bidirectional"), w2, inp2_)
    assert np.array_equal(one_c["h_final"], one_b["h_final"])
    inp2 = dict(inp, x0=inp["x0"].copy())
    inp2["x0"][-1] += 1.0
    b2 = run(orc, bid, w, inp2)
    c2 = run(orc, cfg, w, inp2)
    assert not np.allclose(b2["h_final"][0], b["h_final"][0])
    assert np.array_equal(c2["h_final"][0], c["h_final"][0])
