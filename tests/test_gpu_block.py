"""GPU parity of draft_block_forward (through the C ABI) against the oracle.

Small shapes span several tiles and ragged tails (H not a multiple of 32, odd
intermediate sizes, M and R not multiples of 16); the full-size workloads run in
the launch configuration the benchmark times. Every layer's hidden state,
hidden_out, h_final and the written K/V rows are compared elementwise.
"""
import numpy as np
import pytest

from verifier_block_forward_amd import configs, synth
from tests.gpu_harness import Prepared, compare_block, to_dev

pytestmark = pytest.mark.gpu


def small(**kw):
    base = dict(name="small", seed=21, kind="dflash", n_layers=2, hidden=200, n_q_heads=4,
                n_kv_heads=2, head_dim=64, vocab=1000, M=5, R=3, C=37, kv_dtype="f32",
                intermediate=360, n_target_hidden=3, block_input="x0")
    base.update(kw)
    return configs.BlockConfig(**base)


def run_case(orc, cfg, prep=None, **kw):
    print(f"\n[block] {cfg.name} M={kw.get('M', cfg.M)} R={kw.get('R', cfg.R)} "
          f"seq_len={kw.get('seq_len', cfg.C)} kv={cfg.kv_dtype}", flush=True)
    prep = prep or Prepared(cfg)
    got = prep.run(**kw)
    M = kw.get("M", cfg.M)
    R = kw.get("R", cfg.R)
    s0 = kw.get("seq_len", prep.in_host["seq_len"])
    inp = dict(prep.in_host)
    if "x0" in kw:
        inp["x0"] = kw["x0"].cpu().numpy()
    want = orc.block_forward(cfg, prep.w_host, inp, seq_len=s0, M=M, R=R)
    gk, gv = prep.cache_host(*got["cache"])
    worst = compare_block(cfg, got, want, s0, s0 + R + M, (gk, gv), (want["cache_k"], want["cache_v"]))
    print(f"  worst err/tol = {worst:.3f}", flush=True)
    return got, want


@pytest.mark.parametrize("cfg", [
    small(),
    small(name="small_tokens", block_input="tokens"),
    small(name="small_bf16kv", kv_dtype="bf16"),
    small(name="small_m1_r0", M=1, R=0),
    small(name="small_m16_r16", M=16, R=16, C=100),
    small(name="small_empty_cache", C=0),
    small(name="small_hd128", hidden=264, n_q_heads=2, n_kv_heads=1, head_dim=128, M=7, R=9),
    small(name="small_hd256_gqa6", hidden=256, n_q_heads=6, n_kv_heads=1, head_dim=256, M=3, R=2,
          rotary_dim=64),
    small(name="small_mtp", kind="mtp", R=0, M=1, has_attn_gate=True, n_layers=1, n_target_hidden=0),
    small(name="small_mtp_m4", kind="mtp", R=0, M=4, has_attn_gate=True, n_layers=1,
          n_target_hidden=0, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, C=300),
], ids=lambda c: c.name)
def test_block_small(orc, cfg):
    run_case(orc, cfg)


# The chunk merge picks its block size and batch from the chunk count, and the chunk
# count follows the context length (one query group per kv head, 256 chunks at most).
# These contexts put each head dim into the ranges the other tests do not reach:
# 64-dim heads with 65-128 and 129-256 chunks, 128-dim heads with 33-64 and 65-256
# chunks, 256-dim heads with 17-32 and 129-256 chunks.
@pytest.mark.parametrize("cfg", [
    small(name="combine_hd128_63chunks", hidden=264, n_q_heads=2, n_kv_heads=1, head_dim=128,
          M=7, R=9, C=4000, n_layers=1),
    small(name="combine_hd128_125chunks", hidden=264, n_q_heads=2, n_kv_heads=1, head_dim=128,
          M=7, R=9, C=8000, n_layers=1),
    small(name="combine_hd256_24chunks", hidden=256, n_q_heads=6, n_kv_heads=1, head_dim=256,
          M=3, R=2, rotary_dim=64, C=1500, n_layers=1),
    small(name="combine_mtp_hd256_gate", kind="mtp", R=0, M=1, has_attn_gate=True, n_layers=1,
          n_target_hidden=0, hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=256, C=3000),
    small(name="combine_hd64_71chunks", C=9000, n_layers=1),
    small(name="combine_hd64_157chunks", n_q_heads=2, n_kv_heads=1, C=10000, n_layers=1),
    small(name="combine_mtp_hd256_141chunks", kind="mtp", R=0, M=1, has_attn_gate=True, n_layers=1,
          n_target_hidden=0, hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=256, C=9000),
], ids=lambda c: c.name)
def test_block_combine_chunk_counts(orc, cfg):
    run_case(orc, cfg)


# With 8 kv heads the planner makes about 32 chunks per head, so a 10,000-position
# context gives the waves of the first 31 chunks five 16-key sub-tiles each: the F32
# key loop runs four passes of its main loop (unconditional refills) and one tail
# pass, and the two-slot BF16 loop two full passes and a half one. In the last chunk
# one wave has two sub-tiles and two waves have none.
@pytest.mark.parametrize("cfg", [
    small(name="waves_5subtiles_f32", hidden=256, n_q_heads=16, n_kv_heads=8, head_dim=128,
          M=16, R=4, C=10000, n_layers=1),
    small(name="waves_5subtiles_bf16", hidden=256, n_q_heads=16, n_kv_heads=8, head_dim=128,
          M=16, R=4, C=10000, n_layers=1, kv_dtype="bf16"),
], ids=lambda c: c.name)
def test_block_long_wave_shares(orc, cfg):
    run_case(orc, cfg)


# The attention kernel takes 1, 2 or 4 query tiles (16 queries each) per workgroup,
# capped by head dim and cache type (F32: 4 at 64 dims, 2 at 128, 1 at 256; BF16: 2
# at 256 dims, else 4). These shapes reach the variants the other tests leave out:
# four tiles at 64 dims (F32 and BF16, 52 of 64 queries used), four at 128 dims with
# a BF16 cache (36 queries, and 72 queries over two query groups), one at 128 dims
# with a BF16 cache, and BF16 caches at 256 dims with one and two tiles.
@pytest.mark.parametrize("cfg", [
    small(name="qt4_hd64_f32", n_q_heads=8, n_kv_heads=2, M=13, R=3, C=700),
    small(name="qt4_hd64_bf16", n_q_heads=8, n_kv_heads=2, M=13, R=3, C=700, kv_dtype="bf16"),
    small(name="qt4_hd128_bf16", hidden=264, n_q_heads=4, n_kv_heads=1, head_dim=128, M=9, R=5,
          C=700, kv_dtype="bf16"),
    small(name="qt4x2_hd128_bf16", hidden=264, n_q_heads=8, n_kv_heads=1, head_dim=128, M=9, R=5,
          C=300, n_layers=1, kv_dtype="bf16"),
    small(name="qt1_hd128_bf16", hidden=264, n_q_heads=2, n_kv_heads=1, head_dim=128, M=7, R=9,
          C=700, kv_dtype="bf16"),
    small(name="qt2_hd256_bf16", hidden=256, n_q_heads=6, n_kv_heads=1, head_dim=256, M=3, R=2,
          rotary_dim=64, C=700, kv_dtype="bf16"),
    small(name="qt1_hd256_bf16_mtp", kind="mtp", R=0, M=1, has_attn_gate=True, n_layers=1,
          n_target_hidden=0, hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=256, C=900,
          kv_dtype="bf16"),
], ids=lambda c: c.name)
def test_block_query_tile_variants(orc, cfg):
    run_case(orc, cfg)


# A plain split-K launch whose k-slices reach 25 steps or more takes the two-stage
# ring with 8-wave workgroups. At H = 4096 with four target hidden states the fc
# projection (4096 x 16384) is planned as 128 row-tile pairs x 16 slices of 32 steps.
def test_block_long_plain_slices(orc):
    run_case(orc, small(name="fc_long_slices", hidden=4096, n_target_hidden=4, n_layers=1,
                        intermediate=512, n_q_heads=2, n_kv_heads=1, head_dim=64, M=3, R=2, C=40))


def test_block_c0(orc):
    run_case(orc, configs.C0)


def test_block_c0_all_m_r(orc):
    cfg = configs.C0
    prep = Prepared(cfg)
    for M, R in ((1, 0), (2, 1), (4, 4), (4, 0), (3, 2)):
        x0 = prep.inp["x0"][:M].contiguous()
        run_case(orc, cfg, prep=prep, M=M, R=R, x0=x0)


def test_block_rollback_rerun_bitwise(orc):
    """Roll back R+M rows and run again: bit-identical outputs (deterministic kernels)."""
    from verifier_block_forward_amd import dbf
    cfg = small()
    prep = Prepared(cfg)
    ck, cv = prep.fresh_cache()
    a = prep.run(cache=(ck, cv))
    kv = a["kv"]
    dbf.kv_rollback(kv, cfg.R + cfg.M)
    assert kv.seq_len == cfg.C
    b = prep.run(cache=(ck, cv), seq_len=kv.seq_len)
    assert np.array_equal(a["h_final"], b["h_final"])
    assert np.array_equal(a["layer_hidden"], b["layer_hidden"])


def test_block_incremental_context(orc):
    """Two calls (R/2 context rows each, block rolled back in between) match one
    call with all R rows, on the GPU as in the oracle."""
    from verifier_block_forward_amd import dbf
    cfg = small(R=6)
    prep = Prepared(cfg)
    one = prep.run()
    ck, cv = prep.fresh_cache()
    ctx = prep.inp["ctx"]
    a = prep.run(cache=(ck, cv), R=3, ctx=ctx[:3].contiguous())
    kv = a["kv"]
    dbf.kv_rollback(kv, cfg.M)
    b = prep.run(cache=(ck, cv), R=3, seq_len=kv.seq_len, ctx=ctx[3:].contiguous())
    from tests.gpu_harness import check_close
    check_close("incremental h_final", b["h_final"], one["h_final"])


@pytest.mark.slow
@pytest.mark.parametrize("name,layout", [
    ("c1", "rowmajor"), ("c1", "tiled"), ("c2", "rowmajor"), ("c2", "tiled"),
    ("c3", "rowmajor"), ("c3", "tiled"), ("c4", "rowmajor"),
], ids=lambda v: v)
def test_block_full_size(orc, name, layout):
    """Full-size workloads, in both weight layouts; "tiled" is the launch configuration
    the benchmark times (every projection tiled)."""
    cfg = configs.get(name)
    run_case(orc, cfg, prep=Prepared(cfg, tiled=layout == "tiled"))


# ---------------------------------------------------------------------------
# tiled weight layout
# ---------------------------------------------------------------------------

def tiled_reference(w: np.ndarray) -> np.ndarray:
    """The tiled layout written out element by element from its definition in dbf.h."""
    B = w.shape[0] if w.ndim == 3 else 1
    w3 = w.reshape(B, w.shape[-2], w.shape[-1])
    N, K = w3.shape[1:]
    T, S = (N + 15) // 16, (K + 31) // 32
    out = np.zeros((B, T * S * 512), np.uint16)
    n, k = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    off = ((n // 16 * S + k // 32) * 64 + ((k % 32) // 8) * 16 + n % 16) * 8 + k % 8
    for b in range(B):
        out[b, off.ravel()] = w3[b].ravel()
    return out.ravel()


@pytest.mark.parametrize("shape", [(37, 200), (16, 32), (1, 8), (3, 33, 72), (300, 2816)])
def test_tile_weight_layout(shape):
    from verifier_block_forward_amd import dbf
    from tests.gpu_harness import to_dev, torch
    w = synth.normal_bf16(9, len(shape), shape)
    tw = dbf.tile_weight(to_dev(w))
    torch().cuda.synchronize()
    got = tw.data.view(torch().int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, tiled_reference(w))


@pytest.mark.parametrize("cfg", [small(), small(name="small_mtp_t", kind="mtp", R=0, M=2,
                                                has_attn_gate=True, n_layers=1, n_target_hidden=0)],
                         ids=lambda c: c.name)
def test_block_tiled_weights(orc, cfg):
    prep = Prepared(cfg, tiled=True)
    got = prep.run()
    want = orc.block_forward(cfg, prep.w_host, prep.in_host)
    gk, gv = prep.cache_host(*got["cache"])
    s0 = cfg.C
    compare_block(cfg, got, want, s0, s0 + cfg.R + cfg.M, (gk, gv), (want["cache_k"], want["cache_v"]))


def test_block_mixed_layouts_bitwise():
    """Tiled and row-major weights give bit-identical block outputs (same sums)."""
    cfg = small()
    a = Prepared(cfg).run()
    b = Prepared(cfg, tiled={"layers.0.wq", "layers.1.ffn_down", "fc", "layers.0.wv"}).run()
    assert np.array_equal(a["h_final"], b["h_final"])


def scale_cached_keys(inp, kv_dtype, ramp):
    """Multiply cached key row p of every layer and head by ramp[p] (BF16 caches are
    decoded, scaled and re-rounded)."""
    k = inp["cache_k"]
    C = ramp.size
    if kv_dtype == "bf16":
        f = (k[:, :, :C].astype(np.uint32) << 16).view(np.float32) * ramp[None, None, :, None]
        k[:, :, :C] = synth.bf16_rne(f.astype(np.float32)).reshape(f.shape)
    else:
        k[:, :, :C] *= ramp[None, None, :, None].astype(np.float32)


@pytest.mark.parametrize("kv_dtype,order", [("f32", "growing"), ("bf16", "growing"),
                                            ("f32", "shrinking"), ("bf16", "shrinking")])
def test_block_attention_score_range(orc, kv_dtype, order):
    """Cached keys scaled by position (1 to 16 along 20,000 positions, several 16-key
    sub-tiles per wave): with rising scores a query's running max keeps passing its
    reference point, so the accumulator is rescaled many times inside one wave; with
    falling scores the first sub-tile sets it for good."""
    cfg = small(name=f"scores_{order}_{kv_dtype}", kv_dtype=kv_dtype, C=20000, M=5, R=3)
    inp = synth.make_inputs(cfg)
    ramp = np.linspace(1.0, 16.0, cfg.C)
    scale_cached_keys(inp, kv_dtype, ramp if order == "growing" else ramp[::-1].copy())
    run_case(orc, cfg, Prepared(cfg, inputs=inp))


# ---------------------------------------------------------------------------
# MoE FFN (MTP block with routed experts + shared expert)
# ---------------------------------------------------------------------------

def small_moe(**kw):
    base = dict(name="small_moe", seed=31, kind="mtp", n_layers=1, hidden=256, n_q_heads=4,
                n_kv_heads=2, head_dim=64, vocab=500, M=3, R=0, C=20, kv_dtype="f32",
                ffn_kind="moe", n_experts=16, top_k=4, expert_intermediate=64,
                shared_intermediate=96, has_attn_gate=True, block_input="x0")
    base.update(kw)
    return configs.BlockConfig(**base)


def run_moe_case(orc, cfg, tiled=False):
    print(f"\n[moe] {cfg.name} M={cfg.M} E={cfg.n_experts} top_k={cfg.top_k} tiled={tiled}", flush=True)
    prep = Prepared(cfg, tiled=tiled)
    got = prep.run()
    want = orc.block_forward(cfg, prep.w_host, prep.in_host)
    # the expert sets are unique only where the router's rank-k / rank-k+1 logit gap is
    # clear of rounding; the seeded inputs are checked to have no such near-tie
    if cfg.top_k < cfg.n_experts:
        assert want["moe_gap"].min() > 1e-4, f"near-tie in the router: gap {want['moe_gap'].min()}"
    gk, gv = prep.cache_host(*got["cache"])
    s0 = cfg.C
    worst = compare_block(cfg, got, want, s0, s0 + cfg.R + cfg.M, (gk, gv),
                          (want["cache_k"], want["cache_v"]))
    # the reported count of distinct experts is the size of the oracle's routed set
    for layer in range(cfg.n_layers):
        assert got["moe_experts"][layer] == len(np.unique(want["moe_sel"][layer])), layer
    print(f"  worst err/tol = {worst:.3f}, experts touched {got['moe_experts'].tolist()}", flush=True)


@pytest.mark.parametrize("cfg", [
    small_moe(),
    small_moe(name="moe_m1", M=1),
    small_moe(name="moe_top1", top_k=1, M=4),
    small_moe(name="moe_all", n_experts=8, top_k=8, M=2),
    small_moe(name="moe_m16", M=16, C=40),
    small_moe(name="moe_ragged", hidden=200, expert_intermediate=40, shared_intermediate=24, M=5),
    # E not a multiple of the wavefront; the largest E with M = 16 routes in two row passes
    small_moe(name="moe_e100", n_experts=100, top_k=5, M=7, seed=32),
    small_moe(name="moe_e1024_m16", n_experts=1024, top_k=16, M=16, C=40, seed=32),
    # 8 experts per lane in the routing (257-512 experts)
    small_moe(name="moe_e500", n_experts=500, top_k=8, M=5, seed=33),
    # a router width that is not a multiple of 4: the partial stores' scalar edge
    small_moe(name="moe_e101", n_experts=101, top_k=6, M=4, seed=34),
], ids=lambda c: c.name)
def test_block_moe_small(orc, cfg):
    run_moe_case(orc, cfg)


@pytest.mark.parametrize("E,top_k,M", [(16, 3, 3), (16, 1, 2), (100, 5, 4), (300, 7, 2)])
def test_block_moe_router_ties(orc, E, top_k, M):
    """Router rows duplicated in pairs (expert 2i+1 gets expert 2i's row): every
    logit comes in an exactly equal pair on both sides, so with an odd top_k the
    last pick is always a tie, which must go to the lower (even) index. The experts
    themselves differ, so a wrong pick shows in the block output."""
    cfg = small_moe(name=f"moe_ties_e{E}_k{top_k}", n_experts=E, top_k=top_k, M=M, seed=35)
    w = synth.make_weights(cfg)
    r = w["layers.0.router"]
    r[1::2] = r[0:E - 1:2]
    print(f"\n[moe ties] E={E} top_k={top_k} M={M}", flush=True)
    prep = Prepared(cfg, weights=w)
    got = prep.run()
    want = orc.block_forward(cfg, prep.w_host, prep.in_host)
    sel = want["moe_sel"][0]
    assert (sel[:, -1] % 2 == 0).all(), sel  # the oracle's tied pick is the even twin
    gk, gv = prep.cache_host(*got["cache"])
    compare_block(cfg, got, want, cfg.C, cfg.C + cfg.M, (gk, gv), (want["cache_k"], want["cache_v"]))
    assert got["moe_experts"][0] == len(np.unique(sel))


def test_block_moe_tiled(orc):
    run_moe_case(orc, small_moe(name="moe_tiled", M=4), tiled=True)


def test_block_moe_fewer_experts_after_more(orc):
    """A call that touches fewer experts than the previous call on the same workspace:
    the routing of the second call must not pick up the first call's coefficients
    or expert partials for the slots it does not use."""
    cfg = small_moe(name="moe_shrink", M=8)
    prep = Prepared(cfg)
    first = orc.block_forward(cfg, prep.w_host, prep.in_host)
    prep.run()  # many distinct experts (8 independent rows)
    # second call: every input row the same, so the rows (which still differ after
    # the causal attention) route to far fewer experts
    inp = dict(prep.in_host)
    inp["x0"] = np.repeat(prep.in_host["x0"][:1], cfg.M, axis=0)
    inp["ctx"] = np.repeat(prep.in_host["ctx"][:1], cfg.M, axis=0)
    want = orc.block_forward(cfg, prep.w_host, inp)
    n_first = len(np.unique(first["moe_sel"]))
    n_second = len(np.unique(want["moe_sel"]))
    assert n_second < n_first, (n_first, n_second)  # 6 after 16 with these seeds
    assert want["moe_gap"].min() > 1e-4, f"near-tie in the router: gap {want['moe_gap'].min()}"
    got = prep.run(x0=to_dev(inp["x0"]), ctx=to_dev(inp["ctx"]))
    gk, gv = prep.cache_host(*got["cache"])
    compare_block(cfg, got, want, cfg.C, cfg.C + cfg.M, (gk, gv), (want["cache_k"], want["cache_v"]))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["c4", "c4m4"])
def test_block_moe_full_size(orc, name):
    run_moe_case(orc, configs.get(name), tiled=True)


@pytest.mark.parametrize("cfg", [
    small(name="bidir", block_mask="bidirectional"),
    small(name="bidir_bf16kv", block_mask="bidirectional", kv_dtype="bf16", M=9, R=5),
    small(name="bidir_mtp_m4", kind="mtp", R=0, M=4, has_attn_gate=True, n_layers=1,
          n_target_hidden=0, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, C=300,
          block_mask="bidirectional"),
], ids=lambda c: c.name)
def test_block_bidirectional_mask(orc, cfg):
    run_case(orc, cfg)


def test_block_context_gathered_on_device(orc):
    """The R context rows gathered on the device from the captured target layers
    (row r = concat_t layer_t[row0 + r], the pages' extract_drafter_concat for the
    new rows) give bit for bit the block of the host-built context, and match the
    oracle fed the host-built rows."""
    from tests.gpu_harness import to_dev, torch
    cfg = small(name="gather", R=6, n_target_hidden=3)
    H, R, nt = cfg.hidden, cfg.R, cfg.n_target_hidden
    prep = Prepared(cfg)
    rng = np.random.default_rng(44)
    row0, P_cap, pitch = 17, 50, H + 8  # padded rows: the gather honours the stride
    layers = [rng.standard_normal((P_cap, pitch)).astype(np.float32) for _ in range(nt)]
    T = np.concatenate([L[row0:row0 + R, :H] for L in layers], axis=1)
    print(f"\n[gather] R={R} n_t={nt} row0={row0}", flush=True)
    by_ctx = prep.run(ctx=to_dev(T))
    got = prep.run(ctx_layers=[to_dev(L) for L in layers], ctx_row0=row0)
    for k in ("h_final", "hidden_out", "layer_hidden"):
        assert np.array_equal(got[k], by_ctx[k]), f"gathered context differs in {k}"
    gk, gv = prep.cache_host(*got["cache"])
    ck, cv = prep.cache_host(*by_ctx["cache"])
    assert np.array_equal(gk, ck) and np.array_equal(gv, cv)
    inp = dict(prep.in_host, ctx=T)
    s0 = prep.in_host["seq_len"]
    want = orc.block_forward(cfg, prep.w_host, inp, seq_len=s0)
    worst = compare_block(cfg, got, want, s0, s0 + R + cfg.M, (gk, gv), (want["cache_k"], want["cache_v"]))
    print(f"  worst err/tol = {worst:.3f}", flush=True)
