"""HIP graph capture of one whole hot-path step: draft_block_forward, lm_head_argmax
and accept_prefix enqueue on one stream, with no host synchronisation and no
memsets, so the step can be captured and replayed. Every replay, with eager
device work and synchronisations between replays, must reproduce the eager step
bit for bit (the kernels are deterministic: fixed reduction orders, no float
atomics). A replay rewrites the same cache rows, which is what the eager step does
after kv_rollback(R + M).
"""
import numpy as np
import pytest

from verifier_block_forward_amd import configs, synth
from tests.gpu_harness import Prepared, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c0", "c4m4", "c1"])
def test_graph_replay_matches_eager(name):
    from verifier_block_forward_amd import dbf
    t = torch()
    cfg = configs.get(name)
    print(f"\n[graph] {name}", flush=True)
    P = Prepared(cfg, tiled=True)
    M, R, H, V = cfg.M, cfg.R, cfg.hidden, cfg.vocab
    ck, cv = P.fresh_cache()
    kv = dbf.make_cache(ck, cv, P.in_host["seq_len"])
    h_final = t.empty((M, H), dtype=t.float32, device="cuda")
    hidden_out = t.empty((M, H), dtype=t.float32, device="cuda")
    argmax = t.empty(M, dtype=t.int32, device="cuda")
    margin = t.empty(M, dtype=t.float32, device="cuda")
    result = t.zeros(5, dtype=t.int32, device="cuda")
    ws_head = t.empty(dbf.lm_head_argmax_workspace_bytes(M, H, V), dtype=t.uint8, device="cuda")
    io = dbf.make_io(M, R, h_final, tokens=P.inp.get("tokens"), x0=P.inp.get("x0"),
                     ctx=P.inp.get("ctx"), hidden_out=hidden_out)
    K = cfg.K
    drafts = argmax[1:] if cfg.kind == "dflash" else argmax[:1]
    target_np, _ = synth.accept_targets(np.arange(K, dtype=np.int32), V, cfg.seed)
    target = t.from_numpy(target_np).cuda()
    lm_head = P.w_dev["lm_head"]

    def step(stream):
        dbf.draft_block_forward(P.ccfg, P.bw, kv, io, P.ws, stream)
        dbf.lm_head_argmax(h_final, lm_head, argmax, None, margin, ws_head, stream)
        dbf.accept_prefix(drafts, target, result, stream=stream)

    outs = (h_final, hidden_out, argmax, margin, result, ck, cv)
    step(t.cuda.current_stream())
    dbf.kv_rollback(kv, R + M)
    t.cuda.synchronize()
    ref = [x.clone() for x in outs]

    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step(t.cuda.current_stream())
    dbf.kv_rollback(kv, R + M)  # capture advanced the host-side seq_len
    assert kv.seq_len == P.in_host["seq_len"]

    for rep in range(3):
        junk = t.randn(4096, device="cuda")
        float((junk * 2).sum().item())  # eager work and a sync between replays
        h_final.fill_(float("nan"))
        hidden_out.fill_(float("nan"))
        argmax.fill_(-1)
        margin.fill_(float("nan"))
        result.fill_(-7)
        g.replay()
        t.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert t.equal(got, want), f"{name}: replay {rep}, output {i} differs from the eager step"
        print(f"  replay {rep}: bitwise equal", flush=True)


def test_graph_replay_of_the_sampled_round():
    """sample_tokens and accept_sampled captured in a graph: every replay, with eager
    work between replays, reproduces the eager results bit for bit."""
    from verifier_block_forward_amd import dbf
    t = torch()
    print("\n[graph] sampled round", flush=True)
    rng = np.random.default_rng(9)
    V, M = 50000, 3
    z = t.from_numpy(rng.normal(0, 3, (M, V)).astype(np.float32)).cuda()
    zt = t.from_numpy(rng.normal(0, 3, (2, V)).astype(np.float32)).cuda()
    u = t.from_numpy(rng.random(M).astype(np.float32)).cuda()
    u2 = t.from_numpy(rng.random(2).astype(np.float32)).cuda()
    tok = t.empty(M, dtype=t.int32, device="cuda")
    prob = t.empty(M, dtype=t.float32, device="cuda")
    res = t.zeros(5, dtype=t.int32, device="cuda")
    com = t.zeros(2, dtype=t.int32, device="cuda")
    ws1 = t.empty(dbf.sample_tokens_workspace_bytes(M, V), dtype=t.uint8, device="cuda")
    ws2 = t.empty(dbf.accept_sampled_workspace_bytes(V), dtype=t.uint8, device="cuda")

    def step(stream):
        dbf.sample_tokens(z, u, tok, prob, 0.9, ws1, stream)
        dbf.accept_sampled(z[0], zt, tok[:1], u2, res, 0.9, committed=com, ws=ws2, stream=stream)

    outs = (tok, prob, res, com)
    step(t.cuda.current_stream())
    t.cuda.synchronize()
    ref = [x.clone() for x in outs]
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step(t.cuda.current_stream())
    for rep in range(3):
        float((t.randn(4096, device="cuda") * 2).sum().item())
        tok.fill_(-1)
        prob.fill_(float("nan"))
        res.fill_(-7)
        com.fill_(-7)
        g.replay()
        t.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert t.equal(got, want), f"replay {rep}, output {i} differs from the eager call"


@pytest.mark.parametrize("name", ["c0", "c4m4", "c1"])
def test_graph_replay_of_the_fused_call(name):
    """The single draft_block_forward call with the shared lm_head argmax and the
    accept walk fused in (the form the benchmark times), captured once and replayed
    three times with eager work in between: every replay equals the eager fused call
    bit for bit, including the accept result and the committed tokens (the first
    n_committed entries, the only ones the call writes)."""
    from verifier_block_forward_amd import dbf
    t = torch()
    cfg = configs.get(name)
    print(f"\n[graph fused] {name}", flush=True)
    P = Prepared(cfg, tiled=True)
    M, R, H, V = cfg.M, cfg.R, cfg.hidden, cfg.vocab
    K = M - 1 if cfg.kind == "dflash" else 1
    ck, cv = P.fresh_cache()
    kv = dbf.make_cache(ck, cv, P.in_host["seq_len"])
    outs = {"h_final": t.empty((M, H), dtype=t.float32, device="cuda"),
            "hidden_out": t.empty((M, H), dtype=t.float32, device="cuda"),
            "argmax": t.empty(M, dtype=t.int32, device="cuda"),
            "margin": t.empty(M, dtype=t.float32, device="cuda"),
            "result": t.zeros(5, dtype=t.int32, device="cuda"),
            "committed": t.zeros(K + 1, dtype=t.int32, device="cuda")}
    target_np, _ = synth.accept_targets(np.arange(K, dtype=np.int32), V, cfg.seed)
    target = t.from_numpy(target_np).cuda()
    io = dbf.make_io(M, R, outs["h_final"], tokens=P.inp.get("tokens"), x0=P.inp.get("x0"),
                     ctx=P.inp.get("ctx"), hidden_out=outs["hidden_out"], lm_head=P.w_dev["lm_head"],
                     argmax=outs["argmax"], top2_margin=outs["margin"], target=target,
                     accept_result=outs["result"], committed=outs["committed"])

    def step(stream):
        dbf.draft_block_forward(P.ccfg, P.bw, kv, io, P.ws, stream)

    tensors = list(outs.values()) + [ck, cv]
    step(t.cuda.current_stream())
    dbf.kv_rollback(kv, R + M)
    t.cuda.synchronize()
    ref = [x.clone() for x in tensors]

    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step(t.cuda.current_stream())
    dbf.kv_rollback(kv, R + M)
    assert kv.seq_len == P.in_host["seq_len"]

    for rep in range(3):
        junk = t.randn(4096, device="cuda")
        float((junk * 2).sum().item())  # eager work and a sync between replays
        for k, x in outs.items():
            x.fill_(float("nan") if x.is_floating_point() else -7)
        g.replay()
        t.cuda.synchronize()
        for i, (got, want) in enumerate(zip(tensors, ref)):
            if got is outs["committed"]:
                # only the committed prefix is written; the rest keeps the fill value
                n = int(outs["result"][4])
                assert t.equal(got[:n], want[:n]), f"{name}: replay {rep}, committed tokens differ"
                assert bool((got[n:] == -7).all()), f"{name}: replay {rep} wrote past the committed tokens"
                continue
            assert t.equal(got, want), f"{name}: replay {rep}, output {i} differs from the eager call"
        print(f"  replay {rep}: bitwise equal", flush=True)
