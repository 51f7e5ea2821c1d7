"""Seeded synthetic inputs for the drafter block.

Every array is drawn from ``numpy.random.Generator(PCG64(SeedSequence([seed,
tensor_id, chunk])))`` in fixed chunks of ``CHUNK`` values, so the content of a
tensor depends only on (seed, tensor_id) and never on how many threads drew it.
``tensor_id`` is the tensor's index in a fixed manifest order (modelled on the
stable upload order of the DFlash drafter's tensors on the hf2q 0.1.1
``spec_decode/dflash/tensors.rs`` page, ``DFlashModelTensors::upload``).

Distributions (one recipe for every workload):

* projection weights (fc / eh halves, Q/K/V/gate/O, FFN, router, experts,
  shared expert and its gate, embed, lm_head): N(0, 0.02) drawn in F32, then
  rounded to BF16 with round-to-nearest-even;
* RMSNorm weights: 1 + N(0, 0.1), kept in F32 (the page's dtype policy stores
  every norm weight as F32);
* activations (x0 / embed_t, the context T or prev_hidden) and the cached K/V
  prefix: N(0, 1), the cache rounded to BF16 (RNE) when the cache is BF16;
* token ids: uniform in [0, vocab).

This module holds no step of the block's arithmetic: the oracle and the GPU
path both consume the arrays it returns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import BlockConfig

CHUNK = 1 << 22

WEIGHT_STD = 0.02
NORM_STD = 0.1


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, tid: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, chunk])))


def bf16_rne(a: np.ndarray) -> np.ndarray:
    """F32 -> BF16 bits with round-to-nearest-even (finite inputs only)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    r = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + r) >> np.uint32(16)).astype(np.uint16)


def _fill(seed: int, tid: int, n: int, fn) -> np.ndarray:
    """Run fn(rng, count) -> array over fixed chunks, in parallel, concatenated."""
    nch = (n + CHUNK - 1) // CHUNK
    if nch <= 1:
        return fn(_rng(seed, tid, 0), n)
    first = fn(_rng(seed, tid, 0), min(CHUNK, n))
    out = np.empty(n, dtype=first.dtype)
    out[: first.size] = first

    def work(c):
        lo = c * CHUNK
        cnt = min(CHUNK, n - lo)
        out[lo: lo + cnt] = fn(_rng(seed, tid, c), cnt)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(1, nch)))
    return out


def normal_f32(seed: int, tid: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))

    def fn(rng, cnt):
        a = rng.standard_normal(cnt, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        if mean != 0.0:
            a += np.float32(mean)
        return a

    return _fill(seed, tid, n, fn).reshape(shape)


def normal_bf16(seed: int, tid: int, shape, std: float = WEIGHT_STD) -> np.ndarray:
    n = int(np.prod(shape))

    def fn(rng, cnt):
        a = rng.standard_normal(cnt, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        return bf16_rne(a)

    return _fill(seed, tid, n, fn).reshape(shape)


def uniform_ids(seed: int, tid: int, n: int, hi: int) -> np.ndarray:
    return _rng(seed, tid, 0).integers(0, hi, size=n, dtype=np.int64).astype(np.int32)


# --------------------------------------------------------------------------
# manifest
# --------------------------------------------------------------------------

def manifest(cfg: BlockConfig):
    """Ordered list of (name, shape, kind) for every weight of the block.

    kind is "w" (BF16 projection), "norm" (F32 RMSNorm weight).
    """
    H, L = cfg.hidden, cfg.n_layers
    qt, kt, hd = cfg.q_total, cfg.kv_total, cfg.head_dim
    m = []
    if cfg.kind == "dflash":
        m += [("fc", (H, cfg.n_target_hidden * H), "w"), ("hidden_norm", (H,), "norm"),
              ("final_norm", (H,), "norm")]
    else:
        m += [("enorm", (H,), "norm"), ("hnorm", (H,), "norm"),
              ("eh_embed", (H, H), "w"), ("eh_hidden", (H, H), "w"), ("final_norm", (H,), "norm")]
    for i in range(L):
        p = f"layers.{i}."
        m += [(p + "in_norm", (H,), "norm"), (p + "post_norm", (H,), "norm"),
              (p + "wq", (qt, H), "w"), (p + "wk", (kt, H), "w"), (p + "wv", (kt, H), "w"),
              (p + "wo", (H, qt), "w"), (p + "q_norm", (hd,), "norm"), (p + "k_norm", (hd,), "norm")]
        if cfg.has_attn_gate:
            m += [(p + "attn_gate", (qt, H), "w")]
        if cfg.ffn_kind == "dense":
            I = cfg.intermediate
            m += [(p + "ffn_gate", (I, H), "w"), (p + "ffn_up", (I, H), "w"),
                  (p + "ffn_down", (H, I), "w")]
        else:
            E, Ie, Is = cfg.n_experts, cfg.expert_intermediate, cfg.shared_intermediate
            m += [(p + "router", (E, H), "w"), (p + "exp_gate", (E, Ie, H), "w"),
                  (p + "exp_up", (E, Ie, H), "w"), (p + "exp_down", (E, H, Ie), "w"),
                  (p + "sh_gate", (Is, H), "w"), (p + "sh_up", (Is, H), "w"),
                  (p + "sh_down", (H, Is), "w"), (p + "sh_gate_inp", (1, H), "w")]
    m += [("lm_head", (cfg.vocab, H), "w")]
    if cfg.block_input == "tokens":
        m += [("embed", (cfg.vocab, H), "w")]
    return m


# tensor ids of the per-call inputs follow the weights; fixed offsets keep them stable
_INPUT_BASE = 1000


def make_weights(cfg: BlockConfig) -> dict:
    out = {}
    for tid, (name, shape, kind) in enumerate(manifest(cfg)):
        if kind == "w":
            out[name] = normal_bf16(cfg.seed, tid, shape)
        else:
            out[name] = normal_f32(cfg.seed, tid, shape, mean=1.0, std=NORM_STD)
    return out


def make_inputs(cfg: BlockConfig) -> dict:
    """Per-call inputs: block rows, context rows, the cached K/V prefix."""
    s, H, M, R = cfg.seed, cfg.hidden, cfg.M, cfg.R
    b = _INPUT_BASE
    out = {}
    if cfg.block_input == "tokens":
        ids = uniform_ids(s, b + 0, 2, cfg.vocab)  # last_token, mask_token_id
        out["tokens"] = np.array([ids[0]] + [ids[1]] * (M - 1), dtype=np.int32)
    else:
        out["x0"] = normal_f32(s, b + 1, (M, H))
    if cfg.kind == "dflash":
        out["ctx"] = normal_f32(s, b + 2, (R, cfg.n_target_hidden * H)) if R > 0 else \
            np.zeros((0, cfg.n_target_hidden * H), np.float32)
    else:
        out["ctx"] = normal_f32(s, b + 2, (M, H))
    L, nkv, hd, cap, C = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim, cfg.capacity, cfg.C
    for j, nm in enumerate(("cache_k", "cache_v")):
        pre = normal_f32(s, b + 3 + j, (L, nkv, C, hd))
        if cfg.kv_dtype == "bf16":
            full = np.zeros((L, nkv, cap, hd), np.uint16)
            full[:, :, :C, :] = bf16_rne(pre).reshape(pre.shape)
        else:
            full = np.zeros((L, nkv, cap, hd), np.float32)
            full[:, :, :C, :] = pre
        out[nm] = full
    out["seq_len"] = C
    return out


def accept_targets(drafts: np.ndarray, vocab: int, seed: int, tid: int = _INPUT_BASE + 9):
    """Target argmaxes in which exactly the first j drafts match, j uniform in 0..K.

    Returns (targets[K+1], j).
    """
    d = np.asarray(drafts, dtype=np.int64)
    K = d.size
    rng = _rng(seed, tid, 0)
    j = int(rng.integers(0, K + 1))
    t = rng.integers(0, vocab, size=K + 1, dtype=np.int64)
    t[:j] = d[:j]
    if j < K:
        t[j] = (d[j] + 1 + int(rng.integers(0, vocab - 1))) % vocab
    return t.astype(np.int32), j
