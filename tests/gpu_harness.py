"""Helpers shared by the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, run the oracle on the same host arrays, compare.

Tolerance (hidden states, logits, F32 cache rows): |g - o| <= 1e-3 + 2e-3 |o|
elementwise. BF16 cache rows: the same bound plus one BF16 ulp of o, since both
sides round values that agree within the tolerance to the nearest BF16.
"""
from __future__ import annotations

import numpy as np

from verifier_block_forward_amd import synth

ATOL = 1e-3
RTOL = 2e-3


def torch():
    import torch as t
    return t


def to_dev(a: np.ndarray):
    t = torch()
    if a.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).cuda()
    return t.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_ulp(x):
    ax = np.abs(x).astype(np.float64)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_close(name, got, want, atol=ATOL, rtol=RTOL, extra=None):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    tol = atol + rtol * np.abs(want)
    if extra is not None:
        tol = tol + extra
    err = np.abs(got - want)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{bad.size} outside tolerance; worst at {i}: "
            f"got {got[i]!r} want {want[i]!r} (err {err[i]:.3g}, tol {tol[i]:.3g})")
    return float((err / tol).max()) if err.size else 0.0


def decode_bf16(u16):
    return (np.asarray(u16, np.uint32) << 16).view(np.float32)


class Prepared:
    """Device copies of one workload's weights and inputs."""

    def __init__(self, cfg, weights=None, inputs=None, tiled=False):
        """tiled: True (every projection + lm_head tiled), False, or a set of names."""
        from verifier_block_forward_amd import dbf
        t = torch()
        self.cfg = cfg
        self.w_host = weights if weights is not None else synth.make_weights(cfg)
        self.in_host = inputs if inputs is not None else synth.make_inputs(cfg)
        self.w_dev = {k: to_dev(v) for k, v in self.w_host.items()}
        if tiled:
            for k, v in list(self.w_dev.items()):
                if v.dtype == t.bfloat16 and k != "embed" and (tiled is True or k in tiled):
                    self.w_dev[k] = dbf.tile_weight(v)
            t.cuda.synchronize()
        self.bw = dbf.BlockWeights(cfg, self.w_dev)
        self.ccfg = dbf.make_config(cfg)
        self.inp = {k: to_dev(v) for k, v in self.in_host.items()
                    if isinstance(v, np.ndarray) and v.size > 0}
        self.ws = t.empty(dbf.draft_block_workspace_bytes(self.ccfg, dbf.MAX_M, dbf.MAX_R),
                          dtype=t.uint8, device="cuda")
        assert self.ws.numel() > 0, dbf.last_error()

    def fresh_cache(self):
        return self.inp["cache_k"].clone(), self.inp["cache_v"].clone()

    def run(self, M=None, R=None, seq_len=None, cache=None, x0=None, ctx=None, tokens=None,
            want_layers=True, ctx_layers=None, ctx_row0=0):
        """Returns the outputs as host arrays, the cache tensors and the dbf cache
        struct; MoE workloads also return moe_experts (distinct experts per layer)."""
        from verifier_block_forward_amd import dbf
        t = torch()
        cfg = self.cfg
        M = cfg.M if M is None else M
        R = cfg.R if R is None else R
        seq_len = self.in_host["seq_len"] if seq_len is None else seq_len
        ck, cv = cache if cache is not None else self.fresh_cache()
        H = cfg.hidden
        h_final = t.empty((M, H), dtype=t.float32, device="cuda")
        hidden_out = t.empty((M, H), dtype=t.float32, device="cuda")
        layers = t.empty((cfg.n_layers, M, H), dtype=t.float32, device="cuda") if want_layers else None
        if tokens is None and x0 is None:
            tokens = self.inp.get("tokens")
            x0 = self.inp.get("x0")
        if ctx is None and ctx_layers is None:
            ctx = self.inp.get("ctx")
        moe = t.full((cfg.n_layers,), -1, dtype=t.int32, device="cuda") if cfg.ffn_kind == "moe" else None
        io = dbf.make_io(M, R, h_final, tokens=tokens, x0=x0, ctx=ctx, hidden_out=hidden_out,
                         layer_hidden=layers, ctx_layers=ctx_layers, ctx_row0=ctx_row0,
                         moe_experts=moe)
        kv = dbf.make_cache(ck, cv, seq_len)
        dbf.draft_block_forward(self.ccfg, self.bw, kv, io, self.ws)
        t.cuda.synchronize()
        out = {"h_final": h_final.cpu().numpy(), "hidden_out": hidden_out.cpu().numpy(),
               "seq_len": kv.seq_len, "cache": (ck, cv), "kv": kv}
        if moe is not None:
            out["moe_experts"] = moe.cpu().numpy()
        if want_layers:
            out["layer_hidden"] = layers.cpu().numpy()
        return out

    def cache_host(self, ck, cv):
        t = torch()
        if ck.dtype == t.bfloat16:
            return ck.view(t.int16).cpu().numpy().view(np.uint16), cv.view(t.int16).cpu().numpy().view(np.uint16)
        return ck.cpu().numpy(), cv.cpu().numpy()


def compare_block(cfg, got, want, lo, hi, cache_got, cache_want, layers=True):
    """Compare GPU block outputs with the oracle's; returns worst err/tol ratio."""
    worst = 0.0
    if layers:
        for l in range(cfg.n_layers):
            worst = max(worst, check_close(f"{cfg.name} layer {l} hidden", got["layer_hidden"][l],
                                           want["layer_hidden"][l]))
    worst = max(worst, check_close(f"{cfg.name} hidden_out", got["hidden_out"], want["hidden_out"]))
    worst = max(worst, check_close(f"{cfg.name} h_final", got["h_final"], want["h_final"]))
    assert got["seq_len"] == want["seq_len"]
    gk, gv = cache_got
    wk, wv = cache_want
    for nm, g, w in (("K", gk, wk), ("V", gv, wv)):
        if g.dtype == np.uint16:
            gd = decode_bf16(g[:, :, lo:hi]).astype(np.float64)
            wd = decode_bf16(w[:, :, lo:hi]).astype(np.float64)
            worst = max(worst, check_close(f"{cfg.name} cache {nm}", gd, wd, extra=bf16_ulp(wd)))
            assert np.array_equal(g[:, :, :lo], w[:, :, :lo]), "cache prefix modified"
        else:
            worst = max(worst, check_close(f"{cfg.name} cache {nm}", g[:, :, lo:hi], w[:, :, lo:hi]))
            assert np.array_equal(g[:, :, :lo], w[:, :, :lo]), "cache prefix modified"
    return worst
