"""ctypes binding of libdbf.so (include/dbf.h): argument marshalling only.

Every step of the drafter block runs in the library's HIP kernels; this module
only turns torch tensors (device memory) and the current HIP stream into the C
structs and pointers the ABI takes. Importing it fails loudly when the built
library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdbf.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "dbf.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libdbf.so is not built ({LIB_PATH}); run __graft_entry__.build()")
# torch first: its bundled HIP runtime has the same soname (libamdhip64.so.7) as the
# one libdbf.so links against, so the loader then binds libdbf.so to torch's copy and
# the process holds a single HIP runtime (two runtimes do not share devices/streams).
import torch  # noqa: E402,F401

_lib = C.CDLL(LIB_PATH)

OK, EINVAL, ESHAPE, EDTYPE, ERANGE, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5, -6
F32, BF16, I32, BF16_T16 = 0, 1, 2, 3
MASK_CAUSAL, MASK_BIDIR = 0, 1
KIND_DFLASH, KIND_MTP = 0, 1
FFN_DENSE, FFN_MOE = 0, 1
MAX_M = 16
MAX_R = 16
NOALLOC_MAX_VOCAB = 1 << 20


class DbfError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dbf error {code}: {msg}")
        self.code = code


class Tensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32), ("ndim", C.c_int32),
                ("shape", C.c_int64 * 4)]


class Config(C.Structure):
    _fields_ = [("kind", C.c_int32), ("n_layers", C.c_int32), ("hidden", C.c_int32),
                ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("rotary_dim", C.c_int32), ("intermediate", C.c_int32),
                ("n_target_hidden", C.c_int32), ("vocab", C.c_int32), ("ffn_kind", C.c_int32),
                ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("expert_intermediate", C.c_int32), ("shared_intermediate", C.c_int32),
                ("has_attn_gate", C.c_int32), ("block_mask", C.c_int32), ("reserved_", C.c_int32),
                ("rms_eps", C.c_double), ("rope_theta", C.c_double)]


LAYER_FIELDS = ["in_norm", "post_norm", "wq", "wk", "wv", "attn_gate", "wo", "q_norm", "k_norm",
                "ffn_gate", "ffn_up", "ffn_down", "router", "exp_gate", "exp_up", "exp_down",
                "sh_gate", "sh_up", "sh_down", "sh_gate_inp"]


class LayerWeights(C.Structure):
    _fields_ = [(f, Tensor) for f in LAYER_FIELDS]


class Weights(C.Structure):
    _fields_ = [("fc", Tensor), ("hidden_norm", Tensor), ("enorm", Tensor), ("hnorm", Tensor),
                ("eh_embed", Tensor), ("eh_hidden", Tensor), ("layers", C.POINTER(LayerWeights)),
                ("final_norm", Tensor), ("embed", Tensor)]


class KVCache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("dtype", C.c_int32),
                ("n_layers", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("capacity", C.c_int64), ("seq_len", C.c_int64)]


class BlockIO(C.Structure):
    _fields_ = [("tokens", C.c_void_p), ("x0", C.c_void_p), ("ctx", C.c_void_p),
                ("M", C.c_int32), ("R", C.c_int32), ("hidden_out", C.c_void_p),
                ("h_final", C.c_void_p), ("layer_hidden", C.c_void_p),
                ("ctx_layers", C.POINTER(C.c_void_p)), ("ctx_ld", C.c_int64), ("ctx_row0", C.c_int64),
                ("moe_experts", C.c_void_p), ("lm_head", C.POINTER(Tensor)), ("argmax", C.c_void_p),
                ("top2_margin", C.c_void_p), ("target", C.c_void_p), ("eos", C.c_void_p),
                ("n_eos", C.c_int32), ("accept_result", C.c_void_p), ("committed", C.c_void_p)]


_lib.draft_block_forward.argtypes = [C.POINTER(Config), C.POINTER(Weights), C.POINTER(KVCache),
                                     C.POINTER(BlockIO), C.c_void_p, C.c_size_t, C.c_void_p]
_lib.draft_block_forward.restype = C.c_int
_lib.draft_block_workspace_bytes.argtypes = [C.POINTER(Config), C.c_int32, C.c_int32]
_lib.draft_block_workspace_bytes.restype = C.c_size_t
_lib.lm_head_argmax.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.POINTER(Tensor), C.c_void_p,
                                C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
_lib.lm_head_argmax.restype = C.c_int
_lib.lm_head_argmax_noalloc.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.POINTER(Tensor), C.c_void_p,
                                        C.c_void_p, C.c_void_p, C.c_void_p]
_lib.lm_head_argmax_noalloc.restype = C.c_int
_lib.lm_head_argmax_workspace_bytes.argtypes = [C.c_int32, C.c_int32, C.c_int32]
_lib.lm_head_argmax_workspace_bytes.restype = C.c_size_t
_lib.accept_prefix.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_int32,
                               C.c_void_p, C.c_void_p, C.c_void_p]
_lib.accept_prefix.restype = C.c_int
_lib.sample_tokens.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_float, C.c_void_p, C.c_void_p,
                               C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
_lib.sample_tokens.restype = C.c_int
_lib.sample_tokens_workspace_bytes.argtypes = [C.c_int32, C.c_int32]
_lib.sample_tokens_workspace_bytes.restype = C.c_size_t
_lib.accept_sampled.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_float, C.c_void_p, C.c_void_p,
                                C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                C.c_void_p]
_lib.accept_sampled.restype = C.c_int
_lib.accept_sampled_workspace_bytes.argtypes = [C.c_int32]
_lib.accept_sampled_workspace_bytes.restype = C.c_size_t
_lib.kv_rollback.argtypes = [C.POINTER(KVCache), C.c_int32]
_lib.kv_rollback.restype = C.c_int
_lib.dbf_tiled_bytes.argtypes = [C.c_int64, C.c_int64]
_lib.dbf_tiled_bytes.restype = C.c_size_t
_lib.dbf_tile_weight.argtypes = [C.POINTER(Tensor), C.c_void_p, C.c_void_p]
_lib.dbf_tile_weight.restype = C.c_int


class ProfRecord(C.Structure):
    _fields_ = [("cls", C.c_int32), ("reserved_", C.c_int32), ("kernel", C.c_char_p),
                ("us", C.c_double)]


_lib.dbf_profile_start.argtypes = [C.c_int32]
_lib.dbf_profile_start.restype = C.c_int
_lib.dbf_profile_stop.argtypes = [C.POINTER(ProfRecord), C.c_int32, C.POINTER(C.c_int32)]
_lib.dbf_profile_stop.restype = C.c_int
_lib.dbf_last_error.restype = C.c_char_p
_lib.dbf_abi_version.restype = C.c_int


def lib():
    return _lib


def declared_functions() -> list[str]:
    """Names of every function include/dbf.h declares."""
    with open(HEADER) as f:
        txt = f.read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       txt, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "return")))


def _check(rc: int):
    if rc != 0:
        raise DbfError(rc, _lib.dbf_last_error().decode())


def last_error() -> str:
    return _lib.dbf_last_error().decode()


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _check_layout(t, name, dtype, min_numel=0, ndim=None):
    """Element type, contiguity, rank and length of a tensor the entry point reads or
    writes through a raw pointer."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got {t.dim()})")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {min_numel}")


def _need(t, name, dtype, min_numel=0, ndim=None, optional=False):
    """Checks the C ABI cannot make on a raw pointer: a device tensor of the element
    type the entry point reads, contiguous, holding at least min_numel elements."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    _check_layout(t, name, dtype, min_numel, ndim)
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be device memory (got {t.device})")


def _need_ws(ws, need, name="workspace"):
    torch = _torch()
    _need(ws, name, torch.uint8)
    if ws.numel() < need:
        raise ValueError(f"{name} holds {ws.numel()} bytes, needs {need}")


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


class Tiled:
    """A BF16 weight in the tiled matrix-core layout: device storage + logical shape."""

    def __init__(self, data, shape):
        self.data = data
        self.shape = tuple(int(x) for x in shape)


def tensor(t) -> Tensor:
    """dbf_tensor view of a contiguous torch tensor or a Tiled weight (empty for None)."""
    out = Tensor()
    if t is None:
        return out
    if isinstance(t, Tiled):
        out.data = t.data.data_ptr()
        out.dtype = BF16_T16
        out.ndim = len(t.shape)
        for i, s in enumerate(t.shape):
            out.shape[i] = s
        return out
    torch = _torch()
    if not t.is_contiguous():
        raise ValueError("dbf tensors must be contiguous")
    dt = {torch.float32: F32, torch.bfloat16: BF16, torch.int32: I32}.get(t.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {t.dtype}")
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    out.data = t.data_ptr()
    out.dtype = dt
    out.ndim = t.dim()
    for i, s in enumerate(t.shape):
        out.shape[i] = s
    return out


def make_config(bc) -> Config:
    """dbf_config from a configs.BlockConfig."""
    return Config(kind=KIND_DFLASH if bc.kind == "dflash" else KIND_MTP, n_layers=bc.n_layers,
                  hidden=bc.hidden, n_q_heads=bc.n_q_heads, n_kv_heads=bc.n_kv_heads,
                  head_dim=bc.head_dim, rotary_dim=bc.rotary_dim, intermediate=bc.intermediate,
                  n_target_hidden=bc.n_target_hidden, vocab=bc.vocab,
                  ffn_kind=FFN_MOE if bc.ffn_kind == "moe" else FFN_DENSE,
                  n_experts=bc.n_experts, top_k=bc.top_k,
                  expert_intermediate=bc.expert_intermediate,
                  shared_intermediate=bc.shared_intermediate,
                  has_attn_gate=1 if bc.has_attn_gate else 0,
                  block_mask=MASK_BIDIR if bc.block_mask == "bidirectional" else MASK_CAUSAL,
                  rms_eps=bc.rms_eps, rope_theta=bc.rope_theta)


class BlockWeights:
    """dbf_weights over a dict of device tensors named as in synth.manifest()."""

    def __init__(self, bc, t: dict):
        self.t = t  # keep the tensors alive
        L = bc.n_layers
        self.layers = (LayerWeights * L)()
        for i in range(L):
            for f in LAYER_FIELDS:
                setattr(self.layers[i], f, tensor(t.get(f"layers.{i}.{f}")))
        self.w = Weights(fc=tensor(t.get("fc")), hidden_norm=tensor(t.get("hidden_norm")),
                         enorm=tensor(t.get("enorm")), hnorm=tensor(t.get("hnorm")),
                         eh_embed=tensor(t.get("eh_embed")), eh_hidden=tensor(t.get("eh_hidden")),
                         layers=self.layers, final_norm=tensor(t.get("final_norm")),
                         embed=tensor(t.get("embed")))

    def resident_bytes(self) -> int:
        """Bytes of the block's own weights as uploaded ([TENS] page,
        `DFlashModelTensors::gpu_resident_bytes`: the sum of every tensor's byte
        length; projections BF16, norms F32). The embedding and lm_head belong to the
        target, are shared by reference, and are not counted. Tiled weights count
        their tiled storage."""
        total = 0
        for name, x in self.t.items():
            if x is None or name in ("embed", "lm_head"):
                continue
            d = x.data if isinstance(x, Tiled) else x
            total += d.numel() * d.element_size()
        return total


def make_cache(k, v, seq_len: int) -> KVCache:
    torch = _torch()
    if k.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"cache dtype {k.dtype}: F32 or BF16")
    _need(k, "cache k", k.dtype, ndim=4)
    _need(v, "cache v", k.dtype, ndim=4)
    if tuple(k.shape) != tuple(v.shape):
        raise ValueError(f"cache k {tuple(k.shape)} and v {tuple(v.shape)} differ in shape")
    dt = BF16 if k.dtype == torch.bfloat16 else F32
    L, nkv, cap, hd = k.shape
    return KVCache(k=k.data_ptr(), v=v.data_ptr(), dtype=dt, n_layers=L, n_kv_heads=nkv,
                   head_dim=hd, capacity=cap, seq_len=seq_len)


def make_io(M, R, h_final, tokens=None, x0=None, ctx=None, hidden_out=None,
            layer_hidden=None, ctx_layers=None, ctx_row0=0, moe_experts=None, lm_head=None,
            argmax=None, top2_margin=None, target=None, eos=None, accept_result=None,
            committed=None) -> BlockIO:
    """ctx_layers: list of n_t device tensors [positions, >= H] F32 (captured target
    layers); the R context rows are gathered from positions ctx_row0..
    lm_head (+ argmax, top2_margin) runs the shared head in the same call; target
    (+ eos, accept_result, committed) also runs the greedy accept walk of the drafts."""
    torch = _torch()
    _need(h_final, "h_final", torch.float32, ndim=2)
    H = h_final.shape[1]
    if h_final.shape[0] < M:
        raise ValueError(f"h_final has {h_final.shape[0]} rows, needs {M}")
    _need(tokens, "tokens", torch.int32, M, optional=True)
    _need(x0, "x0", torch.float32, M * H, optional=True)
    _need(ctx, "ctx", torch.float32, 0, optional=True)
    _need(hidden_out, "hidden_out", torch.float32, M * H, optional=True)
    _need(layer_hidden, "layer_hidden", torch.float32, M * H, optional=True)
    _need(moe_experts, "moe_experts", torch.int32, 1, optional=True)
    if ctx_layers is not None:
        for i, t in enumerate(ctx_layers):
            if t.device.type != "cuda" or t.dtype != torch.float32 or t.dim() != 2 or t.stride(1) != 1:
                raise ValueError(f"ctx_layers[{i}] must be a device F32 [positions, H] row-major tensor")
            if t.stride(0) != ctx_layers[0].stride(0):
                raise ValueError("ctx_layers must share one row stride")
    _need(argmax, "argmax", torch.int32, M, optional=True)
    _need(top2_margin, "top2_margin", torch.float32, M, optional=True)
    _need(target, "target", torch.int32, 2, optional=True)
    _need(eos, "eos", torch.int32, optional=True)
    _need(accept_result, "accept_result", torch.int32, 5, optional=True)
    _need(committed, "committed", torch.int32, 2, optional=True)
    io = BlockIO(tokens=_ptr(tokens), x0=_ptr(x0), ctx=_ptr(ctx), M=M, R=R,
                 hidden_out=_ptr(hidden_out), h_final=_ptr(h_final),
                 layer_hidden=_ptr(layer_hidden), moe_experts=_ptr(moe_experts),
                 argmax=_ptr(argmax), top2_margin=_ptr(top2_margin), target=_ptr(target),
                 eos=_ptr(eos), n_eos=0 if eos is None else eos.numel(),
                 accept_result=_ptr(accept_result), committed=_ptr(committed))
    if lm_head is not None:
        io._lm_head = tensor(lm_head)  # the struct must outlive the call
        io.lm_head = C.pointer(io._lm_head)
    if ctx_layers is not None:
        arr = (C.c_void_p * len(ctx_layers))(*[t.data_ptr() for t in ctx_layers])
        io._ctx_arr = arr  # the host pointer array must outlive the call
        io.ctx_layers = C.cast(arr, C.POINTER(C.c_void_p))
        io.ctx_ld = ctx_layers[0].stride(0)
        io.ctx_row0 = ctx_row0
    return io


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def draft_block_workspace_bytes(cfg: Config, M: int, R: int) -> int:
    return int(_lib.draft_block_workspace_bytes(C.byref(cfg), M, R))


def draft_block_forward(cfg: Config, w: BlockWeights, cache: KVCache, io: BlockIO, ws,
                        stream=None) -> None:
    _need_ws(ws, 0)
    _check(_lib.draft_block_forward(C.byref(cfg), C.byref(w.w), C.byref(cache), C.byref(io),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def lm_head_argmax_workspace_bytes(M: int, H: int, V: int) -> int:
    return int(_lib.lm_head_argmax_workspace_bytes(M, H, V))


def lm_head_argmax(h, lm_head, argmax, logits=None, top2_margin=None, ws=None, stream=None) -> None:
    torch = _torch()
    _need(h, "h", torch.float32, ndim=2)
    M, H = h.shape
    V = lm_head.shape[0]
    _need(argmax, "argmax", torch.int32, M)
    _need(logits, "logits", torch.float32, M * V, optional=True)
    _need(top2_margin, "top2_margin", torch.float32, M, optional=True)
    _need_ws(ws, lm_head_argmax_workspace_bytes(M, H, V))
    lt = tensor(lm_head)
    _check(_lib.lm_head_argmax(_ptr(h), M, H, C.byref(lt), _ptr(argmax), _ptr(logits),
                               _ptr(top2_margin), _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(),
                               _stream(stream)))


def lm_head_argmax_noalloc(h, lm_head, argmax, logits=None, top2_margin=None, stream=None) -> None:
    """lm_head_argmax on the library's static device scratch (no workspace argument)."""
    torch = _torch()
    _need(h, "h", torch.float32, ndim=2)
    M, H = h.shape
    V = lm_head.shape[0]
    _need(argmax, "argmax", torch.int32, M)
    _need(logits, "logits", torch.float32, M * V, optional=True)
    _need(top2_margin, "top2_margin", torch.float32, M, optional=True)
    lt = tensor(lm_head)
    _check(_lib.lm_head_argmax_noalloc(_ptr(h), M, H, C.byref(lt), _ptr(argmax), _ptr(logits),
                                       _ptr(top2_margin), _stream(stream)))


def accept_prefix(drafts, target, result, eos=None, committed=None, stream=None) -> None:
    torch = _torch()
    _need(drafts, "drafts", torch.int32)
    K = drafts.numel()
    _need(target, "target", torch.int32, K + 1)
    _need(result, "result", torch.int32, 5)
    _need(eos, "eos", torch.int32, optional=True)
    _need(committed, "committed", torch.int32, K + 1, optional=True)
    n_eos = 0 if eos is None else eos.numel()
    _check(_lib.accept_prefix(_ptr(drafts), _ptr(target), K, _ptr(eos), n_eos, _ptr(result),
                              _ptr(committed), _stream(stream)))


def sample_tokens_workspace_bytes(M: int, V: int) -> int:
    return int(_lib.sample_tokens_workspace_bytes(M, V))


def sample_tokens(logits, u, token, prob=None, temperature=1.0, ws=None, stream=None) -> None:
    """One draw per row of logits [M, V] from softmax(logits / T), uniforms u [M]."""
    torch = _torch()
    _need(logits, "logits", torch.float32, ndim=2)
    M, V = logits.shape
    _need(u, "u", torch.float32, M)
    _need(token, "token", torch.int32, M)
    _need(prob, "prob", torch.float32, M, optional=True)
    _need_ws(ws, sample_tokens_workspace_bytes(M, V))
    _check(_lib.sample_tokens(_ptr(logits), M, V, float(temperature), _ptr(u), _ptr(token), _ptr(prob),
                              _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(stream)))


def accept_sampled_workspace_bytes(V: int) -> int:
    return int(_lib.accept_sampled_workspace_bytes(V))


def accept_sampled(draft_logits, target_logits, draft, u, result, temperature=1.0, eos=None,
                   committed=None, ws=None, stream=None) -> None:
    """Sampled acceptance of one drafted token: draft_logits [V], target_logits [2, V],
    draft [1] int32, u [2] uniforms, result [5] int32."""
    torch = _torch()
    _need(draft_logits, "draft_logits", torch.float32)
    V = draft_logits.numel()
    _need(target_logits, "target_logits", torch.float32, 2 * V)
    _need(draft, "draft", torch.int32, 1)
    _need(u, "u", torch.float32, 2)
    _need(result, "result", torch.int32, 5)
    _need(eos, "eos", torch.int32, optional=True)
    _need(committed, "committed", torch.int32, 2, optional=True)
    _need_ws(ws, accept_sampled_workspace_bytes(V))
    n_eos = 0 if eos is None else eos.numel()
    _check(_lib.accept_sampled(_ptr(draft_logits), _ptr(target_logits), V, float(temperature),
                               _ptr(draft), _ptr(u), _ptr(eos), n_eos, _ptr(result), _ptr(committed),
                               _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                               _stream(stream)))


def tiled_bytes(N: int, K: int) -> int:
    return int(_lib.dbf_tiled_bytes(N, K))


def tile_weight(t, stream=None) -> Tiled:
    """Repack a row-major BF16 weight [N, K] or [B, N, K] into the tiled layout."""
    torch = _torch()
    B = t.shape[0] if t.dim() == 3 else 1
    N, K = t.shape[-2], t.shape[-1]
    nbytes = B * tiled_bytes(N, K)
    dst = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=t.device)
    src = tensor(t)
    _check(_lib.dbf_tile_weight(C.byref(src), C.c_void_p(dst.data_ptr()), _stream(stream)))
    return Tiled(dst, t.shape)


def kv_rollback(cache: KVCache, n: int) -> None:
    _check(_lib.kv_rollback(C.byref(cache), n))


PROF_CLASSES = ("projections", "attention", "row_kernels", "lm_head", "accept", "sampling", "other")


def profile_start(max_records: int = 4096) -> None:
    """Time the library's next max_records kernel launches (measurement only)."""
    rc = _lib.dbf_profile_start(max_records)
    if rc != 0:
        raise DbfError(rc, f"profile_start({max_records}) refused")


def profile_stop(max_records: int = 4096) -> list:
    """Stop timing; returns [(class name, kernel name, microseconds)] in launch order."""
    recs = (ProfRecord * max_records)()
    n = C.c_int32(0)
    rc = _lib.dbf_profile_stop(recs, max_records, C.byref(n))
    if rc != 0:
        raise DbfError(rc, "profile_stop: a timed kernel's events could not be read")
    return [(PROF_CLASSES[recs[i].cls], recs[i].kernel.decode(), recs[i].us)
            for i in range(min(n.value, max_records))]


def abi_version() -> int:
    return int(_lib.dbf_abi_version())
