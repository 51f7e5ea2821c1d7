"""CPU checks of the C-ABI library: it loads, exports every declared symbol, and
rejects bad arguments before anything touches the GPU (no device is used here:
every call below fails validation before the first HIP call)."""
import ctypes as C

import pytest

from verifier_block_forward_amd import configs, dbf


def test_exports_every_declared_symbol():
    names = dbf.declared_functions()
    assert set(names) >= {"draft_block_forward", "lm_head_argmax", "accept_prefix", "kv_rollback",
                          "draft_block_workspace_bytes", "lm_head_argmax_workspace_bytes",
                          "sample_tokens", "sample_tokens_workspace_bytes", "accept_sampled",
                          "accept_sampled_workspace_bytes", "dbf_last_error", "dbf_abi_version",
                          "dbf_profile_start", "dbf_profile_stop"}
    for n in names:
        assert hasattr(dbf.lib(), n), n
    assert dbf.abi_version() == 4


def _cfg(name="c0", **kw):
    c = dbf.make_config(configs.get(name))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_workspace_sizes():
    for name in ("c0", "c1", "c2", "c3"):
        bc = configs.get(name)
        n = dbf.draft_block_workspace_bytes(_cfg(name), bc.M, bc.R)
        assert n > 0 and n % 256 == 0
    assert dbf.draft_block_workspace_bytes(_cfg(), 0, 0) == 0
    assert dbf.draft_block_workspace_bytes(_cfg(), 17, 0) == 0
    assert dbf.draft_block_workspace_bytes(_cfg(head_dim=96), 4, 4) == 0
    assert dbf.lm_head_argmax_workspace_bytes(16, 2816, 262144) > 0
    assert dbf.lm_head_argmax_workspace_bytes(0, 2816, 262144) == 0


def _fake(n=0x1000):
    return C.c_void_p(n)


def _call_block(cfg, io, cache=None, w=None, ws=0x100000, ws_bytes=1 << 40):
    L = cfg.n_layers
    if w is None:
        w = dbf.Weights()
    cache = cache or dbf.KVCache(k=0x2000, v=0x3000, dtype=dbf.F32, n_layers=L,
                                 n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, capacity=100,
                                 seq_len=10)
    rc = dbf.lib().draft_block_forward(C.byref(cfg), C.byref(w), C.byref(cache), C.byref(io),
                                       C.c_void_p(ws), ws_bytes, None)
    return rc, cache


def test_block_argument_errors():
    cfg = _cfg()
    h = 0x4000
    assert _call_block(cfg, dbf.BlockIO(M=0, R=0, h_final=h, x0=h))[0] == dbf.EINVAL
    assert _call_block(cfg, dbf.BlockIO(M=17, R=0, h_final=h, x0=h))[0] == dbf.EINVAL
    assert _call_block(cfg, dbf.BlockIO(M=4, R=17, h_final=h, x0=h, ctx=h))[0] == dbf.EINVAL
    assert _call_block(cfg, dbf.BlockIO(M=4, R=0, h_final=None, x0=h))[0] == dbf.EINVAL
    assert _call_block(cfg, dbf.BlockIO(M=4, R=2, h_final=h, x0=h, ctx=None))[0] == dbf.EINVAL
    # weights missing -> EINVAL (null data), config problems first
    rc, cache = _call_block(cfg, dbf.BlockIO(M=4, R=0, h_final=h, x0=h))
    assert rc == dbf.EINVAL and "null" in dbf.last_error()
    assert cache.seq_len == 10
    bad = _cfg(kind=7)
    assert _call_block(bad, dbf.BlockIO(M=4, R=0, h_final=h, x0=h))[0] == dbf.EINVAL
    assert _call_block(_cfg(n_kv_heads=3), dbf.BlockIO(M=4, R=0, h_final=h, x0=h))[0] == dbf.ESHAPE
    assert _call_block(_cfg(hidden=260), dbf.BlockIO(M=4, R=0, h_final=h, x0=h))[0] == dbf.ESHAPE
    mtp = _cfg("c2")
    assert _call_block(mtp, dbf.BlockIO(M=1, R=1, h_final=h, x0=h, ctx=h))[0] == dbf.EINVAL
    assert _call_block(_cfg(block_mask=2), dbf.BlockIO(M=4, R=0, h_final=h, x0=h))[0] == dbf.EINVAL
    assert "block_mask" in dbf.last_error()
    # DFlash context rows: given (ctx) or gathered from captured target layers
    assert _call_block(cfg, dbf.BlockIO(M=4, R=2, h_final=h, x0=h))[0] == dbf.EINVAL
    import ctypes as C
    arr = (C.c_void_p * 2)(h, None)
    io = dbf.BlockIO(M=4, R=2, h_final=h, x0=h, ctx_ld=256)
    io.ctx_layers = C.cast(arr, C.POINTER(C.c_void_p))
    assert _call_block(cfg, io)[0] == dbf.EINVAL and "ctx_layers[1]" in dbf.last_error()
    arr[1] = h
    io.ctx_ld = 8  # shorter than a row
    assert _call_block(cfg, io)[0] == dbf.EINVAL and "ctx_ld" in dbf.last_error()
    # MTP needs embed_t as rows (x0) or as token ids to gather
    assert _call_block(mtp, dbf.BlockIO(M=1, R=0, h_final=h, ctx=h))[0] == dbf.EINVAL
    assert "neither tokens nor x0" in dbf.last_error()


def test_token_input_needs_the_embedding_table():
    """Token ids (DFlash block rows, or a chained MTP step's embed_t) are gathered
    from embed; without a valid embed tensor the call is refused before any launch."""
    bc = configs.C0
    cfg = dbf.make_config(bc)
    w, _ = _weights_for(bc)
    w.embed = dbf.Tensor()  # absent
    rc, cache = _call_block(cfg, dbf.BlockIO(M=4, R=0, h_final=0x4000, tokens=0x4000), w=w)
    assert rc in (dbf.EINVAL, dbf.ESHAPE) and "embed" in dbf.last_error()
    assert cache.seq_len == 10
    w, _ = _weights_for(bc)
    w.embed.dtype = dbf.BF16_T16  # the gather reads rows: row-major only
    rc, _ = _call_block(cfg, dbf.BlockIO(M=4, R=0, h_final=0x4000, tokens=0x4000), w=w)
    assert rc == dbf.EDTYPE and "embed" in dbf.last_error()


def _weights_for(bc, dtype_override=None):
    """Struct of fake device pointers with correct dtypes/shapes (never dereferenced)."""
    w = dbf.Weights()
    H = bc.hidden

    def T(shape, dt):
        t = dbf.Tensor()
        t.data = 0x10000
        t.dtype = dt
        t.ndim = len(shape)
        for i, s in enumerate(shape):
            t.shape[i] = s
        return t
    w.fc = T((H, bc.n_target_hidden * H), dbf.BF16)
    w.hidden_norm = T((H,), dbf.F32)
    w.final_norm = T((H,), dbf.F32)
    w.embed = T((bc.vocab, H), dbf.BF16)
    layers = (dbf.LayerWeights * bc.n_layers)()
    for i in range(bc.n_layers):
        L = layers[i]
        L.in_norm = T((H,), dbf.F32)
        L.post_norm = T((H,), dbf.F32)
        L.wq = T((bc.q_total, H), dbf.BF16)
        L.wk = T((bc.kv_total, H), dbf.BF16)
        L.wv = T((bc.kv_total, H), dbf.BF16)
        L.wo = T((H, bc.q_total), dbf.BF16)
        L.q_norm = T((bc.head_dim,), dbf.F32)
        L.k_norm = T((bc.head_dim,), dbf.F32)
        L.ffn_gate = T((bc.intermediate, H), dbf.BF16)
        L.ffn_up = T((bc.intermediate, H), dbf.BF16)
        L.ffn_down = T((H, bc.intermediate), dbf.BF16)
    w.layers = layers
    return w, layers


def test_dtype_policy_rejects_bf16_norm():
    """A BF16 norm weight is refused (the tensors.rs dtype policy: norms are F32)."""
    bc = configs.C0
    cfg = dbf.make_config(bc)
    w, layers = _weights_for(bc)
    layers[0].q_norm.dtype = dbf.BF16
    rc, cache = _call_block(cfg, dbf.BlockIO(M=4, R=0, h_final=0x4000, x0=0x4000), w=w)
    assert rc == dbf.EDTYPE and "q_norm" in dbf.last_error()
    layers[0].q_norm.dtype = dbf.F32
    layers[0].wq.dtype = dbf.F32
    assert _call_block(cfg, dbf.BlockIO(M=4, R=0, h_final=0x4000, x0=0x4000), w=w)[0] == dbf.EDTYPE
    layers[0].wq.dtype = dbf.BF16
    layers[0].wk.shape[0] = 7
    assert _call_block(cfg, dbf.BlockIO(M=4, R=0, h_final=0x4000, x0=0x4000), w=w)[0] == dbf.ESHAPE


def test_cache_and_workspace_errors():
    bc = configs.C0
    cfg = dbf.make_config(bc)
    w, layers = _weights_for(bc)
    io = dbf.BlockIO(M=4, R=4, h_final=0x4000, x0=0x4000, ctx=0x4000)
    full = dbf.KVCache(k=0x2000, v=0x3000, dtype=dbf.F32, n_layers=1, n_kv_heads=2, head_dim=64,
                       capacity=40, seq_len=33)
    rc, c = _call_block(cfg, io, cache=full, w=w)
    assert rc == dbf.ERANGE and c.seq_len == 33
    badt = dbf.KVCache(k=0x2000, v=0x3000, dtype=dbf.I32, n_layers=1, n_kv_heads=2, head_dim=64,
                       capacity=100, seq_len=3)
    assert _call_block(cfg, io, cache=badt, w=w)[0] == dbf.EDTYPE
    shp = dbf.KVCache(k=0x2000, v=0x3000, dtype=dbf.F32, n_layers=2, n_kv_heads=2, head_dim=64,
                      capacity=100, seq_len=3)
    assert _call_block(cfg, io, cache=shp, w=w)[0] == dbf.ESHAPE
    ok = dbf.KVCache(k=0x2000, v=0x3000, dtype=dbf.F32, n_layers=1, n_kv_heads=2, head_dim=64,
                     capacity=100, seq_len=3)
    assert _call_block(cfg, io, cache=ok, w=w, ws_bytes=16)[0] == dbf.EWORKSPACE
    assert _call_block(cfg, io, cache=ok, w=w, ws=0x100010)[0] == dbf.EWORKSPACE
    assert ok.seq_len == 3


def test_head_accept_rollback_errors():
    L = dbf.lib()
    t = dbf.Tensor()
    t.data = 0x1000
    t.dtype = dbf.F32
    t.ndim = 2
    t.shape[0], t.shape[1] = 100, 64
    rc = L.lm_head_argmax(C.c_void_p(0x2000), 4, 64, C.byref(t), C.c_void_p(0x3000), None, None,
                          C.c_void_p(0x100000), 1 << 30, None)
    assert rc == dbf.EDTYPE
    t.dtype = dbf.BF16
    t.shape[1] = 32
    assert L.lm_head_argmax(C.c_void_p(0x2000), 4, 64, C.byref(t), C.c_void_p(0x3000), None, None,
                            C.c_void_p(0x100000), 1 << 30, None) == dbf.ESHAPE
    t.shape[1] = 64
    assert L.lm_head_argmax(C.c_void_p(0x2000), 0, 64, C.byref(t), C.c_void_p(0x3000), None, None,
                            C.c_void_p(0x100000), 1 << 30, None) == dbf.EINVAL
    assert L.lm_head_argmax(C.c_void_p(0x2000), 4, 64, C.byref(t), C.c_void_p(0x3000), None, None,
                            C.c_void_p(0x100000), 8, None) == dbf.EWORKSPACE
    assert L.accept_prefix(C.c_void_p(1), C.c_void_p(1), 0, None, 0, C.c_void_p(1), None, None) == dbf.EINVAL
    assert L.accept_prefix(C.c_void_p(1), C.c_void_p(1), 1025, None, 0, C.c_void_p(1), None, None) == dbf.EINVAL
    assert L.accept_prefix(C.c_void_p(1), C.c_void_p(1), 4, None, 2, C.c_void_p(1), None, None) == dbf.EINVAL
    assert L.accept_prefix(None, C.c_void_p(1), 4, None, 0, C.c_void_p(1), None, None) == dbf.EINVAL
    kv = dbf.KVCache(seq_len=10, capacity=20)
    with pytest.raises(dbf.DbfError) as e:
        dbf.kv_rollback(kv, 11)
    assert e.value.code == dbf.ERANGE and kv.seq_len == 10
    with pytest.raises(dbf.DbfError):
        dbf.kv_rollback(kv, -1)
    dbf.kv_rollback(kv, 4)
    assert kv.seq_len == 6
    dbf.kv_rollback(kv, 6)
    assert kv.seq_len == 0


def test_workspace_sizing_every_workload_and_moe_bounds():
    """Sizing never divides by an empty FFN (MoE configs have no dense width) and
    MoE limits are enforced."""
    for name in configs.CONFIGS:
        c = dbf.make_config(configs.get(name))
        for M, R in ((1, 0), (16, 16), (4, 3)):
            assert dbf.draft_block_workspace_bytes(c, M, R) > 0, (name, M, R, dbf.last_error())
    c = dbf.make_config(configs.get("c4"))
    c.top_k = 0
    assert dbf.draft_block_workspace_bytes(c, 1, 0) == 0
    c.top_k = 17
    assert dbf.draft_block_workspace_bytes(c, 1, 0) == 0
    c = dbf.make_config(configs.get("c4"))
    c.n_experts = 2000
    assert dbf.draft_block_workspace_bytes(c, 1, 0) == 0


def test_sampling_workspace_sizes():
    for V in (1, 1000, 248320, 262144, 1 << 24):
        n = dbf.sample_tokens_workspace_bytes(16, V)
        assert n > 0 and n % 256 == 0
        m = dbf.accept_sampled_workspace_bytes(V)
        assert m > 0 and m % 256 == 0
    assert dbf.sample_tokens_workspace_bytes(0, 100) == 0
    assert dbf.sample_tokens_workspace_bytes(1025, 100) == 0
    assert dbf.sample_tokens_workspace_bytes(1, 0) == 0
    assert dbf.sample_tokens_workspace_bytes(1, (1 << 24) + 1) == 0
    assert dbf.accept_sampled_workspace_bytes(0) == 0


def _sample(M=4, V=1000, T=1.0, logits=0x1000, u=0x2000, token=0x3000, ws=0x100000, ws_bytes=1 << 20):
    return dbf.lib().sample_tokens(_fake(logits) if logits else None, M, V, T, _fake(u) if u else None,
                                   _fake(token) if token else None, None,
                                   _fake(ws) if ws else None, ws_bytes, None)


def test_sample_tokens_argument_errors():
    assert _sample(logits=0) == dbf.EINVAL
    assert _sample(u=0) == dbf.EINVAL
    assert _sample(token=0) == dbf.EINVAL
    assert _sample(M=0) == dbf.EINVAL
    assert _sample(M=1025) == dbf.EINVAL
    assert _sample(V=0) == dbf.ESHAPE
    for T in (0.0, -1.0, 1e-4, 2e3, float("nan"), float("inf")):
        assert _sample(T=T) == dbf.EINVAL, T
    assert _sample(ws=0) == dbf.EWORKSPACE
    assert _sample(ws=0x100010) == dbf.EWORKSPACE  # not 256-byte aligned
    assert _sample(ws_bytes=16) == dbf.EWORKSPACE
    assert "workspace" in dbf.last_error()


def _accept(V=1000, T=1.0, zq=0x1000, zt=0x2000, d=0x3000, u=0x4000, res=0x5000, eos=None, n_eos=0,
            ws=0x100000, ws_bytes=1 << 20):
    f = lambda p: _fake(p) if p else None
    return dbf.lib().accept_sampled(f(zq), f(zt), V, T, f(d), f(u), f(eos), n_eos, f(res), None, f(ws),
                                    ws_bytes, None)


def test_accept_sampled_argument_errors():
    for k in ("zq", "zt", "d", "u", "res"):
        assert _accept(**{k: 0}) == dbf.EINVAL, k
    assert _accept(V=0) == dbf.ESHAPE
    assert _accept(V=(1 << 24) + 1) == dbf.ESHAPE
    assert _accept(T=0.0) == dbf.EINVAL
    assert _accept(n_eos=1) == dbf.EINVAL  # eos list missing
    assert _accept(n_eos=-1) == dbf.EINVAL
    assert _accept(ws=0) == dbf.EWORKSPACE
    assert _accept(ws_bytes=dbf.accept_sampled_workspace_bytes(1000) - 1) == dbf.EWORKSPACE



def test_binding_checks_buffers_before_the_call():
    """The binding refuses what the C ABI cannot see through a raw pointer: host
    memory, non-contiguous views, wrong element types and buffers shorter than the
    entry point writes. Each case below fails in the binding; no library call runs."""
    import torch

    i32 = torch.zeros(8, dtype=torch.int32)
    f = torch.zeros((4, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="device memory"):
        dbf.accept_prefix(i32[:3], i32[:4], i32[:5])
    with pytest.raises(ValueError, match="device memory"):
        dbf.lm_head_argmax(f, f, i32)
    with pytest.raises(ValueError, match="device memory"):
        dbf.make_cache(torch.zeros((1, 2, 8, 64)), torch.zeros((1, 2, 8, 64)), 0)
    with pytest.raises(ValueError, match="required"):
        dbf._need(None, "target", torch.int32)
    dbf._need(None, "eos", torch.int32, optional=True)
    with pytest.raises(ValueError, match="contiguous"):
        dbf._check_layout(f.t(), "h", torch.float32)
    with pytest.raises(ValueError, match="must be torch.int32"):
        dbf._check_layout(torch.zeros(6, dtype=torch.int64), "target", torch.int32, 6)
    with pytest.raises(ValueError, match="needs at least 6"):
        dbf._check_layout(torch.zeros(5, dtype=torch.int32), "target", torch.int32, 6)
    with pytest.raises(ValueError, match="2 dimensions"):
        dbf._check_layout(torch.zeros(6, dtype=torch.float32), "h", torch.float32, ndim=2)
    dbf._check_layout(torch.zeros(6, dtype=torch.int32), "target", torch.int32, 6)


def test_profile_switch_host_side():
    """The profiling switch validates its bound and, with nothing launched, stops with
    no records (no device work is involved)."""
    assert dbf.lib().dbf_profile_start(0) == dbf.EINVAL
    assert dbf.lib().dbf_profile_start(70000) == dbf.EINVAL
    dbf.profile_start(16)
    assert dbf.profile_stop() == []


def test_noalloc_head_refuses_vocabulary_past_its_scratch():
    """lm_head_argmax_noalloc refuses, before any device work, a vocabulary whose
    records do not fit its static scratch (and takes the largest one that does)."""
    assert dbf.lm_head_argmax_workspace_bytes(16, 2816, dbf.NOALLOC_MAX_VOCAB) == 262144
    assert dbf.lm_head_argmax_workspace_bytes(16, 2816, dbf.NOALLOC_MAX_VOCAB + 1) > 262144
    lm = dbf.Tensor(data=0x1000, dtype=dbf.BF16, ndim=2)
    lm.shape[0], lm.shape[1] = dbf.NOALLOC_MAX_VOCAB + 1, 64
    rc = dbf.lib().lm_head_argmax_noalloc(C.c_void_p(0x2000), 4, 64, C.byref(lm), C.c_void_p(0x3000),
                                          None, None, None)
    assert rc == dbf.ERANGE
    assert "static" in dbf.last_error()


def test_fused_head_fields_validated_before_launch():
    """The optional shared head and accept walk of draft_block_forward are checked
    with everything else, before any launch: lm_head shape and dtype, the outputs
    each part needs, K >= 1 for the walk, and the EOS list."""
    bc = configs.C0
    cfg = dbf.make_config(bc)
    w, _ = _weights_for(bc)
    ok = dict(k=0x2000, v=0x3000, dtype=dbf.F32, n_layers=1, n_kv_heads=2, head_dim=64, capacity=100,
              seq_len=3)

    def lm(V, H, dt=dbf.BF16):
        t = dbf.Tensor()
        t.data, t.dtype, t.ndim = 0x10000, dt, 2
        t.shape[0], t.shape[1] = V, H
        return t

    def run(M=4, **kw):
        io = dbf.BlockIO(M=M, R=0, h_final=0x4000, x0=0x4000)
        keep = []
        for k, v in kw.items():
            if k == "lm_head":
                keep.append(v)
                io.lm_head = C.pointer(v)
            else:
                setattr(io, k, v)
        cache = dbf.KVCache(**ok)
        rc, c = _call_block(cfg, io, cache=cache, w=w)
        assert c.seq_len == 3  # nothing ran
        return rc, dbf.last_error()

    good = lm(bc.vocab, bc.hidden)
    assert run(lm_head=lm(bc.vocab - 1, bc.hidden), argmax=0x5000)[0] == dbf.ESHAPE
    assert run(lm_head=lm(bc.vocab, bc.hidden, dbf.F32), argmax=0x5000)[0] == dbf.EDTYPE
    rc, msg = run(lm_head=good)
    assert rc == dbf.EINVAL and "argmax" in msg
    rc, msg = run(argmax=0x5000)
    assert rc == dbf.EINVAL and "lm_head" in msg
    rc, msg = run(target=0x6000, accept_result=0x7000)
    assert rc == dbf.EINVAL and "lm_head" in msg
    rc, msg = run(lm_head=good, argmax=0x5000, target=0x6000)
    assert rc == dbf.EINVAL and "accept_result" in msg
    rc, msg = run(M=1, lm_head=good, argmax=0x5000, target=0x6000, accept_result=0x7000)
    assert rc == dbf.EINVAL and "M >= 2" in msg
    rc, msg = run(lm_head=good, argmax=0x5000, target=0x6000, accept_result=0x7000, n_eos=2)
    assert rc == dbf.EINVAL and "eos" in msg
    rc, msg = run(lm_head=good, argmax=0x5000, accept_result=0x7000)
    assert rc == dbf.EINVAL and "target" in msg
