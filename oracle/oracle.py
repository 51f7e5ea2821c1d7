"""ctypes front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke entry point and the benchmark's
CPU-baseline leg use it; the product path never imports it. It takes numpy
arrays and any object carrying the block-shape attributes (name, kind,
n_layers, hidden, ...); it imports nothing from the GPU package.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b  # noqa: F401  (package-relative when imported as oracle.oracle)
            _b.build()
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


D = C.POINTER(C.c_double)
F = C.POINTER(C.c_float)
U16 = C.POINTER(C.c_uint16)
I32 = C.POINTER(C.c_int32)


class OrcCfg(C.Structure):
    _fields_ = [("kind", C.c_int32), ("n_layers", C.c_int32), ("hidden", C.c_int32),
                ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("rotary_dim", C.c_int32), ("intermediate", C.c_int32),
                ("n_target_hidden", C.c_int32), ("vocab", C.c_int32), ("ffn_moe", C.c_int32),
                ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("expert_intermediate", C.c_int32), ("shared_intermediate", C.c_int32),
                ("has_gate", C.c_int32), ("kv_bf16", C.c_int32), ("block_bidir", C.c_int32),
                ("eps", C.c_double), ("theta", C.c_double)]


class OrcLayer(C.Structure):
    _fields_ = [("in_norm", F), ("post_norm", F), ("wq", U16), ("wk", U16), ("wv", U16),
                ("wgate", U16), ("wo", U16), ("q_norm", F), ("k_norm", F),
                ("ffn_gate", U16), ("ffn_up", U16), ("ffn_down", U16),
                ("router", U16), ("exp_gate", U16), ("exp_up", U16), ("exp_down", U16),
                ("sh_gate", U16), ("sh_up", U16), ("sh_down", U16), ("sh_gate_inp", U16)]


class OrcWeights(C.Structure):
    _fields_ = [("fc", U16), ("hidden_norm", F), ("enorm", F), ("hnorm", F),
                ("eh_embed", U16), ("eh_hidden", U16), ("layers", C.POINTER(OrcLayer)),
                ("final_norm", F), ("embed", U16)]


class OrcCache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("capacity", C.c_int64),
                ("seq_len", C.c_int64)]


class OrcIO(C.Structure):
    _fields_ = [("tokens", I32), ("x0", F), ("ctx", F), ("M", C.c_int32), ("R", C.c_int32),
                ("layer_hidden", D), ("hidden_out", D), ("h_final", D), ("moe_sel", I32),
                ("moe_gap", D), ("attn_out", D)]


def _declare(L):
    L.orc_decode_bf16_bytes.argtypes = [C.POINTER(C.c_uint8), C.c_long, F]
    L.orc_decode_bf16_bytes.restype = C.c_long
    L.orc_f32_to_bf16.argtypes = [C.c_float]
    L.orc_f32_to_bf16.restype = C.c_uint16
    L.orc_rmsnorm.argtypes = [D, F, C.c_int, C.c_double, D]
    L.orc_linear.argtypes = [D, C.c_int, C.c_int, U16, C.c_int, D]
    L.orc_rope.argtypes = [D, C.c_int, C.c_int, C.c_double, C.c_double]
    L.orc_sdpa_one.argtypes = [D, D, D, C.c_int, C.c_int, D]
    L.orc_moe_route.argtypes = [D, C.c_int, C.c_int, I32, D]
    L.orc_moe_route.restype = C.c_double
    L.orc_block_forward.argtypes = [C.POINTER(OrcCfg), C.POINTER(OrcWeights),
                                    C.POINTER(OrcCache), C.POINTER(OrcIO)]
    L.orc_block_forward.restype = C.c_int
    L.orc_lm_head.argtypes = [D, C.c_int, C.c_int, U16, C.c_int, D, I32, D]
    L.orc_lm_head.restype = C.c_int
    L.orc_accept_prefix.argtypes = [I32, I32, C.c_int, I32, C.c_int, I32, I32]
    L.orc_accept_prefix.restype = C.c_int
    L.orc_sample_tokens.argtypes = [F, C.c_int, C.c_int, C.c_double, D, I32, D]
    L.orc_sample_tokens.restype = C.c_int
    L.orc_accept_sampled.argtypes = [F, F, C.c_int, C.c_double, C.c_int32, C.c_double,
                                     C.c_double, I32, C.c_int, I32, I32, D]
    L.orc_accept_sampled.restype = C.c_int
    L.orc_kv_rollback.argtypes = [C.POINTER(OrcCache), C.c_int]
    L.orc_kv_rollback.restype = C.c_int
    L.orc_threads.restype = C.c_int


def _p(a, t):
    if a is None:
        return C.cast(None, t)
    return a.ctypes.data_as(t)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------------------
# building blocks
# ---------------------------------------------------------------------------

def decode_bf16_bytes(data: bytes) -> np.ndarray:
    buf = np.frombuffer(bytes(data), dtype=np.uint8).copy()
    out = np.zeros(max(len(buf) // 2, 1), np.float32)
    n = lib().orc_decode_bf16_bytes(_p(buf, C.POINTER(C.c_uint8)), len(buf), _p(out, F))
    if n < 0:
        raise ValueError(f"decode_bf16_bytes: data len {len(buf)} not even (not BF16-aligned)")
    return out[:n]


def f32_to_bf16(x: float) -> int:
    return int(lib().orc_f32_to_bf16(C.c_float(x)))


def rmsnorm(x, w, eps):
    x = _c(x, np.float64)
    w = _c(w, np.float32)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_p(x, D), _p(w, F), x.size, eps, _p(y, D))
    return y


def linear(X, W):
    X = _c(np.atleast_2d(X), np.float64)
    W = _c(W, np.uint16)
    M, K = X.shape
    N = W.shape[0]
    assert W.shape[1] == K
    Y = np.empty((M, N), np.float64)
    lib().orc_linear(_p(X, D), M, K, _p(W, U16), N, _p(Y, D))
    return Y


def rope(v, rotary_dim, pos, theta):
    v = _c(v, np.float64).copy()
    lib().orc_rope(_p(v, D), v.size, rotary_dim, float(pos), float(theta))
    return v


def sdpa_one(q, keys, vals):
    q = _c(q, np.float64)
    keys = _c(keys, np.float64)
    vals = _c(vals, np.float64)
    n, hd = keys.shape
    o = np.empty(hd, np.float64)
    lib().orc_sdpa_one(_p(q, D), _p(keys, D), _p(vals, D), n, hd, _p(o, D))
    return o


def moe_route(logits, top_k):
    z = _c(logits, np.float64)
    sel = np.empty(top_k, np.int32)
    w = np.empty(top_k, np.float64)
    gap = lib().orc_moe_route(_p(z, D), z.size, top_k, _p(sel, I32), _p(w, D))
    return sel, w, gap


# ---------------------------------------------------------------------------
# block, head, accept walk
# ---------------------------------------------------------------------------

def make_cfg(cfg) -> OrcCfg:
    return OrcCfg(kind=0 if cfg.kind == "dflash" else 1, n_layers=cfg.n_layers, hidden=cfg.hidden,
                  n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                  rotary_dim=cfg.rotary_dim or cfg.head_dim, intermediate=cfg.intermediate,
                  n_target_hidden=cfg.n_target_hidden, vocab=cfg.vocab,
                  ffn_moe=1 if cfg.ffn_kind == "moe" else 0, n_experts=cfg.n_experts,
                  top_k=cfg.top_k, expert_intermediate=cfg.expert_intermediate,
                  shared_intermediate=cfg.shared_intermediate,
                  has_gate=1 if cfg.has_attn_gate else 0,
                  kv_bf16=1 if cfg.kv_dtype == "bf16" else 0,
                  block_bidir=1 if getattr(cfg, "block_mask", "causal") == "bidirectional" else 0,
                  eps=cfg.rms_eps, theta=cfg.rope_theta)


def block_forward(cfg, weights: dict, inputs: dict, cache_k=None, cache_v=None, seq_len=None,
                  M=None, R=None):
    """Run the oracle block. cache_k/cache_v are updated in place (copies of the
    inputs' cache are made when not given). Returns a dict of F64 outputs."""
    keep = []

    def P(name, t, dt):
        if name not in weights or weights[name] is None:
            return C.cast(None, t)
        a = _c(weights[name], dt)
        keep.append(a)
        return a.ctypes.data_as(t)

    L, H = cfg.n_layers, cfg.hidden
    M = cfg.M if M is None else M
    R = cfg.R if R is None else R
    layers = (OrcLayer * L)()
    for i in range(L):
        p = f"layers.{i}."
        lay = layers[i]
        for f, t in OrcLayer._fields_:
            key = {"wgate": "attn_gate"}.get(f, f)
            setattr(lay, f, P(p + key, t, np.uint16 if t is U16 else np.float32))
    w = OrcWeights(fc=P("fc", U16, np.uint16), hidden_norm=P("hidden_norm", F, np.float32),
                   enorm=P("enorm", F, np.float32), hnorm=P("hnorm", F, np.float32),
                   eh_embed=P("eh_embed", U16, np.uint16), eh_hidden=P("eh_hidden", U16, np.uint16),
                   layers=layers, final_norm=P("final_norm", F, np.float32),
                   embed=P("embed", U16, np.uint16))
    if cache_k is None:
        cache_k = inputs["cache_k"].copy()
        cache_v = inputs["cache_v"].copy()
    assert cache_k.flags.c_contiguous and cache_v.flags.c_contiguous
    cap = cache_k.shape[2]
    s0 = inputs["seq_len"] if seq_len is None else seq_len
    kv = OrcCache(k=cache_k.ctypes.data, v=cache_v.ctypes.data, capacity=cap, seq_len=s0)
    tokens = _c(inputs["tokens"], np.int32) if inputs.get("tokens") is not None else None
    x0 = _c(inputs["x0"], np.float32) if inputs.get("x0") is not None else None
    ctx = _c(inputs["ctx"], np.float32) if inputs.get("ctx") is not None else None
    out = {
        "layer_hidden": np.zeros((L, M, H), np.float64),
        "hidden_out": np.zeros((M, H), np.float64),
        "h_final": np.zeros((M, H), np.float64),
        "attn_out": np.zeros((L, M, cfg.q_total), np.float64),
    }
    if cfg.ffn_kind == "moe":
        out["moe_sel"] = np.zeros((L, M, cfg.top_k), np.int32)
        out["moe_gap"] = np.zeros((L, M), np.float64)
    io = OrcIO(tokens=_p(tokens, I32), x0=_p(x0, F), ctx=_p(ctx, F), M=M, R=R,
               layer_hidden=_p(out["layer_hidden"], D), hidden_out=_p(out["hidden_out"], D),
               h_final=_p(out["h_final"], D), moe_sel=_p(out.get("moe_sel"), I32),
               moe_gap=_p(out.get("moe_gap"), D), attn_out=_p(out["attn_out"], D))
    c = make_cfg(cfg)
    rc = lib().orc_block_forward(C.byref(c), C.byref(w), C.byref(kv), C.byref(io))
    if rc != 0:
        raise RuntimeError(f"oracle block forward failed: {rc}")
    out["cache_k"] = cache_k
    out["cache_v"] = cache_v
    out["seq_len"] = kv.seq_len
    return out


def lm_head(h, W, want_logits=True):
    h = _c(np.atleast_2d(h), np.float64)
    W = _c(W, np.uint16)
    M, H = h.shape
    V = W.shape[0]
    logits = np.empty((M, V), np.float64) if want_logits else None
    am = np.empty(M, np.int32)
    mg = np.empty(M, np.float64)
    rc = lib().orc_lm_head(_p(h, D), M, H, _p(W, U16), V, _p(logits, D), _p(am, I32), _p(mg, D))
    if rc != 0:
        raise RuntimeError(f"oracle lm_head failed: {rc}")
    return logits, am, mg


def accept_prefix(drafts, target, eos=()):
    d = _c(drafts, np.int32)
    t = _c(target, np.int32)
    e = _c(np.asarray(eos, dtype=np.int32).reshape(-1), np.int32)
    K = d.size
    assert t.size == K + 1
    res = np.zeros(5, np.int32)
    com = np.zeros(K + 1, np.int32)
    rc = lib().orc_accept_prefix(_p(d, I32), _p(t, I32), K, _p(e, I32) if e.size else C.cast(None, I32),
                                 e.size, _p(res, I32), _p(com, I32))
    if rc != 0:
        raise ValueError(f"oracle accept_prefix rejected its arguments: {rc}")
    return {"accept_count": int(res[0]), "free_token": int(res[1]), "rollback": int(res[2]),
            "hit_eos": bool(res[3]), "committed": com[: res[4]].tolist()}


def sample_tokens(logits, u, temperature=1.0):
    """One draw per row from softmax(logits[m] / T) by inverse CDF with uniform u[m]
    (oracle.c `orc_sample_tokens`). Returns (tokens [M] int32, probabilities [M])."""
    z = _c(np.atleast_2d(logits), np.float32)
    M, V = z.shape
    uu = _c(np.asarray(u, np.float64).reshape(-1), np.float64)
    assert uu.size == M
    tok = np.zeros(M, np.int32)
    prob = np.zeros(M, np.float64)
    rc = lib().orc_sample_tokens(_p(z, F), M, V, float(temperature), _p(uu, D), _p(tok, I32),
                                 _p(prob, D))
    if rc != 0:
        raise ValueError(f"oracle sample_tokens rejected its arguments: {rc}")
    return tok, prob


def accept_sampled(draft_logits, target_logits, draft, u0, u1, temperature=1.0, eos=()):
    """Sampled acceptance of one drafted token, MTP K = 1 (oracle.c
    `orc_accept_sampled`: the speculative-sampling reading)."""
    zq = _c(np.asarray(draft_logits).reshape(-1), np.float32)
    zt = _c(target_logits, np.float32)
    V = zq.size
    assert zt.shape == (2, V)
    e = _c(np.asarray(eos, dtype=np.int32).reshape(-1), np.int32)
    res = np.zeros(5, np.int32)
    com = np.zeros(2, np.int32)
    info = np.zeros(3, np.float64)
    rc = lib().orc_accept_sampled(_p(zq, F), _p(zt, F), V, float(temperature), int(draft), float(u0),
                                  float(u1), _p(e, I32) if e.size else C.cast(None, I32), e.size,
                                  _p(res, I32), _p(com, I32), _p(info, D))
    if rc != 0:
        raise ValueError(f"oracle accept_sampled rejected its arguments: {rc}")
    return {"accept_count": int(res[0]), "free_token": int(res[1]), "rollback": int(res[2]),
            "hit_eos": bool(res[3]), "committed": com[: res[4]].tolist(),
            "q_draft": float(info[0]), "p_draft": float(info[1]), "residual_sum": float(info[2])}


def kv_rollback(seq_len: int, n: int) -> int:
    kv = OrcCache(k=None, v=None, capacity=seq_len, seq_len=seq_len)
    rc = lib().orc_kv_rollback(C.byref(kv), n)
    if rc != 0:
        raise ValueError(f"rollback of {n} rows from {seq_len} refused")
    return kv.seq_len


def threads() -> int:
    return int(lib().orc_threads())
