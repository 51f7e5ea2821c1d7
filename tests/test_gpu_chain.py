"""Multi-step use of the hot path on the GPU, against the oracle doing the same steps.

* Verify-shaped block: a target-shaped stack runs K+1 rows [last, d1..dK] with
  the block K/V kept; the greedy accept walk compares d1..dK with the argmax of
  rows 0..K-1, and kv_rollback(K - a) drops the rejected rows ([ORCH] per-round
  steps 7-8 and the rollback of K - a). The drafts are built from the oracle's own
  greedy choices up to row j and then break, so the accept count is known (j).
  A second verify pass then continues from the rolled-back cache.
* Chained MTP: step k+1 drafts from the argmax of step k (embed_t = embed[token],
  gathered on the device) and takes step k's pre-norm hidden as prev_hidden, with
  no host round trip between steps.

Argmax indices are compared exactly wherever the oracle's top-2 margin is above
1e-2 (the seeded cases are asserted to clear it); hidden states and cache rows
use the parity tolerance.
"""
import numpy as np
import pytest

from verifier_block_forward_amd import configs, synth
from tests.gpu_harness import Prepared, bf16_ulp, check_close, torch

pytestmark = pytest.mark.gpu

MARGIN = 1e-2


def small(**kw):
    base = dict(name="chain", seed=31, kind="dflash", n_layers=2, hidden=200, n_q_heads=4,
                n_kv_heads=2, head_dim=64, vocab=1000, M=5, R=0, C=30, kv_dtype="f32",
                intermediate=360, n_target_hidden=2, block_input="tokens")
    base.update(kw)
    return configs.BlockConfig(**base)


def padded_cache(inp, extra):
    """The seeded cache with `extra` more rows of capacity (zeros), host and device."""
    from tests.gpu_harness import to_dev
    pads = [((0, 0), (0, 0), (0, extra), (0, 0))]
    hk = np.pad(inp["cache_k"], *pads)
    hv = np.pad(inp["cache_v"], *pads)
    return hk, hv, to_dev(hk), to_dev(hv)


def oracle_step(orc, cfg, w, inp, tokens, ck, cv, seq_len, M, ctx=None):
    d = dict(inp, tokens=np.asarray(tokens, np.int32))
    if ctx is not None:
        d["ctx"] = ctx
    out = orc.block_forward(cfg, w, d, cache_k=ck, cache_v=cv, seq_len=seq_len, M=M, R=0)
    _, am, mg = orc.lm_head(out["h_final"], w["lm_head"])
    return out, am, mg


def greedy_drafts(orc, cfg, w, inp, j, rng):
    """tokens [last, d1..dK]: d_i = oracle argmax of row i-1 for i <= j, then a
    draft that differs from row j's argmax (rows only see earlier rows)."""
    K = cfg.M - 1
    s0 = inp["seq_len"]
    toks = [int(inp["tokens"][0])] + [int(t) for t in rng.integers(0, cfg.vocab, K)]
    for i in range(1, j + 2):
        if i > K:
            break
        hk, hv, _, _ = padded_cache(inp, 0)
        _, am, mg = oracle_step(orc, cfg, w, inp, toks, hk, hv, s0, cfg.M)
        assert mg[i - 1] > MARGIN, f"seeded row {i - 1} has a near tie; pick another seed"
        if i <= j:
            toks[i] = int(am[i - 1])
        elif toks[i] == am[i - 1]:
            toks[i] = (toks[i] + 1) % cfg.vocab
    return toks


@pytest.mark.parametrize("kv_dtype,j", [("f32", 2), ("bf16", 3), ("f32", 0), ("f32", 4)])
def test_verify_block_accept_and_rollback(orc, kv_dtype, j):
    from verifier_block_forward_amd import dbf
    t = torch()
    cfg = small(name=f"verify_{kv_dtype}_{j}", kv_dtype=kv_dtype)
    K, M, H, V = cfg.M - 1, cfg.M, cfg.hidden, cfg.vocab
    print(f"\n[verify] {cfg.name} K={K} expected accept {j}", flush=True)
    P = Prepared(cfg)
    w, inp = P.w_host, P.in_host
    s0 = inp["seq_len"]
    rng = np.random.default_rng(100 + j)
    toks = greedy_drafts(orc, cfg, w, inp, j, rng)

    # oracle round: verify, accept, rollback (capacity for a second pass)
    ck_o, cv_o, ck, cv = padded_cache(inp, M)
    out_o, am_o, mg_o = oracle_step(orc, cfg, w, inp, toks, ck_o, cv_o, s0, M)
    acc_o = orc.accept_prefix(np.array(toks[1:], np.int32), am_o)
    assert acc_o["accept_count"] == j
    s1 = orc.kv_rollback(s0 + M, acc_o["rollback"])
    assert s1 == s0 + 1 + j

    # GPU round through the C ABI, argmax and accept on the device
    kv = dbf.make_cache(ck, cv, s0)
    tok_dev = t.tensor(toks, dtype=t.int32, device="cuda")
    h_final = t.empty((M, H), dtype=t.float32, device="cuda")
    am = t.empty(M, dtype=t.int32, device="cuda")
    mg = t.empty(M, dtype=t.float32, device="cuda")
    res = t.zeros(5, dtype=t.int32, device="cuda")
    ws_head = t.empty(dbf.lm_head_argmax_workspace_bytes(M, H, V), dtype=t.uint8, device="cuda")
    io = dbf.make_io(M, 0, h_final, tokens=tok_dev)
    dbf.draft_block_forward(P.ccfg, P.bw, kv, io, P.ws)
    dbf.lm_head_argmax(h_final, P.w_dev["lm_head"], am, None, mg, ws_head)
    dbf.accept_prefix(tok_dev[1:], am, res)
    t.cuda.synchronize()
    r = res.cpu().numpy()
    check_close("verify h_final", h_final.cpu().numpy(), out_o["h_final"])
    for m in range(j + 1):
        assert mg_o[m] > MARGIN
        assert int(am[m]) == int(am_o[m]), f"row {m}: argmax {int(am[m])} vs oracle {int(am_o[m])}"
    assert r[0] == j and r[1] == acc_o["free_token"] and r[2] == K - j
    dbf.kv_rollback(kv, int(r[2]))
    assert kv.seq_len == s1

    # the kept rows [s0, s1) match the oracle's
    got_k, got_v = P.cache_host(ck, cv)
    dec = (lambda a: (np.asarray(a[:, :, s0:s1], np.uint32) << 16).view(np.float32)) \
        if kv_dtype == "bf16" else (lambda a: a[:, :, s0:s1])
    extra = None
    if kv_dtype == "bf16":
        extra = bf16_ulp(dec(ck_o))
    check_close("verify kept K rows", dec(got_k), dec(ck_o), extra=extra)
    if kv_dtype == "bf16":
        extra = bf16_ulp(dec(cv_o))
    check_close("verify kept V rows", dec(got_v), dec(cv_o), extra=extra)

    # second verify pass from the rolled-back cache: [free token, new drafts]
    toks2 = [int(r[1])] + [int(x) for x in rng.integers(0, V, K)]
    out2_o, _, _ = oracle_step(orc, cfg, w, inp, toks2, ck_o, cv_o, s1, M)
    tok2 = t.tensor(toks2, dtype=t.int32, device="cuda")
    io2 = dbf.make_io(M, 0, h_final, tokens=tok2)
    dbf.draft_block_forward(P.ccfg, P.bw, kv, io2, P.ws)
    t.cuda.synchronize()
    assert kv.seq_len == s1 + M
    check_close("second verify h_final", h_final.cpu().numpy(), out2_o["h_final"])
    got_k, got_v = P.cache_host(ck, cv)
    lo, hi = s1, s1 + M
    dec2 = (lambda a: (np.asarray(a[:, :, lo:hi], np.uint32) << 16).view(np.float32)) \
        if kv_dtype == "bf16" else (lambda a: a[:, :, lo:hi])
    extra = bf16_ulp(dec2(ck_o)) if kv_dtype == "bf16" else None
    check_close("second verify K rows", dec2(got_k), dec2(ck_o), extra=extra)


@pytest.mark.parametrize("ffn", ["dense", "moe"])
def test_chained_mtp_steps_on_device(orc, ffn):
    from verifier_block_forward_amd import dbf
    t = torch()
    kw = dict(name=f"mtp_chain_{ffn}", kind="mtp", M=1, R=0, n_layers=1, has_attn_gate=True,
              n_target_hidden=0, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, C=40,
              vocab=2000, seed=37)
    if ffn == "moe":
        kw.update(ffn_kind="moe", intermediate=0, n_experts=16, top_k=4, expert_intermediate=64,
                  shared_intermediate=96)
    cfg = small(**kw)
    H, V, N = cfg.hidden, cfg.vocab, 4
    print(f"\n[mtp chain] {cfg.name} steps={N}", flush=True)
    P = Prepared(cfg)
    w, inp = P.w_host, P.in_host
    s0 = inp["seq_len"]
    ck_o, cv_o, ck, cv = padded_cache(inp, N)
    kv = dbf.make_cache(ck, cv, s0)
    ws_head = t.empty(dbf.lm_head_argmax_workspace_bytes(1, H, V), dtype=t.uint8, device="cuda")
    tok = t.tensor(inp["tokens"][:1], dtype=t.int32, device="cuda")
    ctx = t.from_numpy(inp["ctx"]).cuda()
    steps = []
    for k in range(N):
        h_final = t.empty((1, H), dtype=t.float32, device="cuda")
        hid = t.empty((1, H), dtype=t.float32, device="cuda")
        am = t.empty(1, dtype=t.int32, device="cuda")
        mg = t.empty(1, dtype=t.float32, device="cuda")
        io = dbf.make_io(1, 0, h_final, tokens=tok, ctx=ctx, hidden_out=hid)
        dbf.draft_block_forward(P.ccfg, P.bw, kv, io, P.ws)
        dbf.lm_head_argmax(h_final, P.w_dev["lm_head"], am, None, mg, ws_head)
        steps.append((h_final, hid, am, mg))
        tok, ctx = am, hid  # the next step drafts from this step's token and hidden
    t.cuda.synchronize()
    assert kv.seq_len == s0 + N

    tok_o, ctx_o = [int(inp["tokens"][0])], inp["ctx"]
    for k, (h_final, hid, am, mg) in enumerate(steps):
        out, am_o, mg_o = oracle_step(orc, cfg, w, inp, tok_o, ck_o, cv_o, s0 + k, 1,
                                      ctx=np.asarray(ctx_o, np.float32))
        if cfg.ffn_kind == "moe":  # expert sets are unique only away from router ties
            assert out["moe_gap"].min() > 1e-4, f"seeded step {k} has a router near tie"
        check_close(f"step {k} h_final", h_final.cpu().numpy(), out["h_final"])
        check_close(f"step {k} hidden_out", hid.cpu().numpy(), out["hidden_out"])
        assert mg_o[0] > MARGIN, f"seeded step {k} has a near tie; pick another seed"
        assert int(am[0]) == int(am_o[0]), f"step {k}: argmax {int(am[0])} vs oracle {int(am_o[0])}"
        tok_o, ctx_o = [int(am_o[0])], out["hidden_out"].astype(np.float32)
    got_k, got_v = P.cache_host(ck, cv)
    check_close("chain K rows", got_k[:, :, s0:s0 + N], ck_o[:, :, s0:s0 + N])
    check_close("chain V rows", got_v[:, :, s0:s0 + N], cv_o[:, :, s0:s0 + N])
