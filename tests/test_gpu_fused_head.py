"""The shared head and the accept walk fused into draft_block_forward against the
separate calls (draft_block_forward, lm_head_argmax, accept_prefix) on the same
inputs, through the C ABI: h_final, hidden_out, argmax, top-2 margin, the accept
result and the committed tokens bit for bit. The separate calls are parity-tested
against the oracle elsewhere; the accept targets are built from the drafts so that
a seeded number of them match."""
import numpy as np
import pytest

from verifier_block_forward_amd import configs, synth
from tests.gpu_harness import Prepared, to_dev, torch
from tests.test_gpu_block import small, small_moe

pytestmark = pytest.mark.gpu


def _outs(t, M, H):
    return {"h_final": t.empty((M, H), dtype=t.float32, device="cuda"),
            "hidden_out": t.empty((M, H), dtype=t.float32, device="cuda"),
            "argmax": t.full((M,), -1, dtype=t.int32, device="cuda"),
            "margin": t.full((M,), float("nan"), dtype=t.float32, device="cuda"),
            "result": t.full((5,), -9, dtype=t.int32, device="cuda"),
            "committed": t.full((M + 1,), -9, dtype=t.int32, device="cuda")}


def _host(o):
    return {k: v.cpu().numpy() for k, v in o.items()}


def run_pair(cfg, tiled=False, eos=None):
    from verifier_block_forward_amd import dbf
    t = torch()
    print(f"\n[fused head] {cfg.name} M={cfg.M} R={cfg.R} V={cfg.vocab} tiled={tiled}", flush=True)
    P = Prepared(cfg, tiled=tiled)
    M, R, H, V = cfg.M, cfg.R, cfg.hidden, cfg.vocab
    K = M - 1 if cfg.kind == "dflash" else 1
    lm = P.w_dev["lm_head"]
    common = dict(tokens=P.inp.get("tokens"), x0=P.inp.get("x0"), ctx=P.inp.get("ctx"))
    # separate calls
    a = _outs(t, M, H)
    ck, cv = P.fresh_cache()
    kv = dbf.make_cache(ck, cv, P.in_host["seq_len"])
    io = dbf.make_io(M, R, a["h_final"], hidden_out=a["hidden_out"], **common)
    dbf.draft_block_forward(P.ccfg, P.bw, kv, io, P.ws)
    ws_head = t.empty(dbf.lm_head_argmax_workspace_bytes(M, H, V), dtype=t.uint8, device="cuda")
    dbf.lm_head_argmax(a["h_final"], lm, a["argmax"], None, a["margin"], ws_head)
    t.cuda.synchronize()
    am = a["argmax"].cpu().numpy()
    drafts = am[1:] if cfg.kind == "dflash" else am[:1]
    target, j = synth.accept_targets(drafts, V, cfg.seed)
    tgt = to_dev(target)
    eos_d = to_dev(np.asarray(eos, np.int32)) if eos else None
    dr = a["argmax"][1:] if cfg.kind == "dflash" else a["argmax"][:1]
    dbf.accept_prefix(dr, tgt, a["result"], eos=eos_d, committed=a["committed"][:K + 1])
    t.cuda.synchronize()
    # one fused call on a fresh copy of the cache
    b = _outs(t, M, H)
    ck2, cv2 = P.fresh_cache()
    kv2 = dbf.make_cache(ck2, cv2, P.in_host["seq_len"])
    io2 = dbf.make_io(M, R, b["h_final"], hidden_out=b["hidden_out"], lm_head=lm, argmax=b["argmax"],
                      top2_margin=b["margin"], target=tgt, eos=eos_d, accept_result=b["result"],
                      committed=b["committed"][:K + 1], **common)
    dbf.draft_block_forward(P.ccfg, P.bw, kv2, io2, P.ws)
    t.cuda.synchronize()
    ha, hb = _host(a), _host(b)
    for k in ha:
        assert np.array_equal(ha[k], hb[k]), f"{cfg.name}: fused {k} differs"
    assert kv2.seq_len == kv.seq_len
    bits = (lambda c: c.view(t.int16)) if ck.dtype == t.bfloat16 else (lambda c: c)
    assert np.array_equal(bits(ck).cpu().numpy(), bits(ck2).cpu().numpy())
    assert np.array_equal(bits(cv).cpu().numpy(), bits(cv2).cpu().numpy())
    if not eos:
        assert int(hb["result"][0]) == j  # the seeded number of matching drafts
    return hb


@pytest.mark.parametrize("cfg", [
    small(),
    small(name="fh_tokens", block_input="tokens"),
    small(name="fh_mtp", kind="mtp", R=0, M=1, has_attn_gate=True, n_layers=1, n_target_hidden=0),
    small(name="fh_mtp_m4", kind="mtp", R=0, M=4, has_attn_gate=True, n_layers=1, n_target_hidden=0,
          hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, C=300),
    small_moe(name="fh_moe", M=4),
    configs.C0,
], ids=lambda c: c.name)
def test_fused_head_equals_separate_calls(cfg):
    run_pair(cfg)


def test_fused_head_tiled_and_eos():
    cfg = small(name="fh_tiled")
    out = run_pair(cfg, tiled=True)
    # an EOS among the target tokens cuts the committed list
    run_pair(cfg, tiled=True, eos=[int(out["committed"][0]), 7])


@pytest.mark.slow
@pytest.mark.parametrize("name", ["c1", "c4m4"])
def test_fused_head_full_size(name):
    run_pair(configs.get(name), tiled=True)
