"""GPU parity of lm_head_argmax and accept_prefix against the oracle (via the C ABI)."""
import numpy as np
import pytest

from verifier_block_forward_amd import synth
from tests.gpu_harness import check_close, to_dev, torch

pytestmark = pytest.mark.gpu


def _dec(u16):
    return (np.asarray(u16, np.uint32) << 16).view(np.float32).astype(np.float64)


def run_head(h, W, want_logits=True, tiled=False):
    from verifier_block_forward_amd import dbf
    t = torch()
    M, H = h.shape
    V = W.shape[0]
    hd, Wd = to_dev(h.astype(np.float32)), to_dev(W)
    if tiled:
        Wd = dbf.tile_weight(Wd)
    am = t.empty(M, dtype=t.int32, device="cuda")
    mg = t.empty(M, dtype=t.float32, device="cuda")
    lg = t.empty((M, V), dtype=t.float32, device="cuda") if want_logits else None
    ws = t.empty(dbf.lm_head_argmax_workspace_bytes(M, H, V), dtype=t.uint8, device="cuda")
    dbf.lm_head_argmax(hd, Wd, am, lg, mg, ws)
    t.cuda.synchronize()
    return (lg.cpu().numpy() if want_logits else None), am.cpu().numpy(), mg.cpu().numpy()


def check_argmax(name, am, lg_oracle, am_o, mg_o):
    for m in range(len(am)):
        if mg_o[m] > 1e-2:
            assert am[m] == am_o[m], f"{name} row {m}: argmax {am[m]} vs oracle {am_o[m]} (margin {mg_o[m]})"
        else:
            z = lg_oracle[m]
            assert z[am[m]] >= z.max() - 1e-2, f"{name} row {m}: argmax {am[m]} not within 1e-2 of the max"


def _random_mhv(n=6, seed=5151):
    """Seeded (M, H, V): M in 1 .. 16, H a multiple of 8 in 8 .. 1024, V log-uniform
    over 1 .. 300,000."""
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 17)), 8 * int(rng.integers(1, 129)),
             int(np.exp(rng.uniform(0.0, np.log(300000))))) for _ in range(n)]


@pytest.mark.parametrize("M,H,V", [(3, 264, 1000), (4, 256, 4096), (16, 200, 777), (1, 8, 65),
                                   (16, 2816, 262144), (1, 5120, 248320), (4, 2048, 248320)]
                         + _random_mhv())
@pytest.mark.parametrize("tiled", [False, True], ids=["rowmajor", "tiled"])
def test_lm_head_argmax_parity(orc, M, H, V, tiled):
    print(f"\n[lm_head] M={M} H={H} V={V} tiled={tiled}", flush=True)
    rng = np.random.default_rng(M * 1000 + H)
    W = synth.normal_bf16(77, H, (V, H))
    h = rng.standard_normal((M, H)).astype(np.float32)
    # normed-hidden scale: logits ~ N(0, 0.02^2 H)
    lg_o, am_o, mg_o = orc.lm_head(h.astype(np.float64), W)
    lg, am, mg = run_head(h, W, tiled=tiled)
    check_close(f"logits M{M} H{H} V{V}", lg, lg_o)
    check_argmax(f"argmax M{M} V{V}", am, lg_o, am_o, mg_o)
    check_close(f"margin M{M} V{V}", mg, mg_o)


def test_lm_head_ties_take_lowest_index(orc):
    rng = np.random.default_rng(5)
    H, V, M = 64, 3000, 5
    W = synth.normal_bf16(5, 1, (V, H))
    for dup in (2999, 1500, 64, 65):
        W[dup] = W[10]
    # rows that make W[10] (and its copies) the clear winner
    h = np.repeat(_dec(W[10])[None, :] * 40.0, M, axis=0).astype(np.float32)
    h[1:] += 0.01 * rng.standard_normal((M - 1, H)).astype(np.float32)
    lg_o, am_o, mg_o = orc.lm_head(h.astype(np.float64), W)
    _, am, mg = run_head(h, W, want_logits=False)
    assert am.tolist() == [10] * M
    assert np.all(mg == 0.0)
    assert am_o.tolist() == [10] * M


def test_lm_head_without_optional_outputs():
    """Null logits/margin pointers give the same argmax as the full call."""
    from verifier_block_forward_amd import dbf
    t = torch()
    H, V, M = 256, 4096, 4
    Wh = synth.normal_bf16(3, 3, (V, H))
    h = np.random.default_rng(9).standard_normal((M, H)).astype(np.float32)
    _, am_full, _ = run_head(h, Wh)
    hd, Wd = to_dev(h), to_dev(Wh)
    am = t.empty(M, dtype=t.int32, device="cuda")
    ws = t.empty(dbf.lm_head_argmax_workspace_bytes(M, H, V), dtype=t.uint8, device="cuda")
    dbf.lm_head_argmax(hd, Wd, am, None, None, ws)
    t.cuda.synchronize()
    assert am.cpu().numpy().tolist() == am_full.tolist()


# ---------------------------------------------------------------------------
# accept_prefix
# ---------------------------------------------------------------------------

def run_accept_batch(cases):
    """cases: list of (drafts, target, eos). Returns list of (result[5], committed)."""
    from verifier_block_forward_amd import dbf
    t = torch()
    res = t.zeros((len(cases), 5), dtype=t.int32, device="cuda")
    outs = []
    keep = []
    for i, (d, tg, eos) in enumerate(cases):
        dd, td = to_dev(np.asarray(d, np.int32)), to_dev(np.asarray(tg, np.int32))
        ed = to_dev(np.asarray(eos, np.int32)) if len(eos) else None
        com = t.full((len(d) + 1,), -1, dtype=t.int32, device="cuda")
        dbf.accept_prefix(dd, td, res[i], eos=ed, committed=com)
        keep += [dd, td, ed]
        outs.append(com)
    t.cuda.synchronize()
    r = res.cpu().numpy()
    return [(r[i], outs[i].cpu().numpy()) for i in range(len(cases))]


def _cmp(orc, cases):
    got = run_accept_batch(cases)
    for (d, tg, eos), (r, com) in zip(cases, got):
        o = orc.accept_prefix(np.asarray(d, np.int32), np.asarray(tg, np.int32), eos)
        assert [int(r[0]), int(r[1]), int(r[2]), bool(r[3])] == \
            [o["accept_count"], o["free_token"], o["rollback"], o["hit_eos"]], (d, tg, eos, r, o)
        assert int(r[4]) == len(o["committed"])
        assert com[: r[4]].tolist() == o["committed"]
        assert np.all(com[r[4]:] == -1)


def test_accept_exhaustive_small_k(orc):
    cases = []
    for K in range(1, 9):
        for pattern in range(1 << K):
            d = list(range(100, 100 + K))
            tg = d + [7]
            for i in range(K):
                if not (pattern >> i) & 1:
                    tg[i] = 5 + i
            cases.append((d, tg, []))
    _cmp(orc, cases)


def test_accept_seeded_and_long(orc):
    cases = []
    for K in (1, 3, 15, 63, 64, 65, 200, 1024):
        for s in range(6):
            d = np.random.default_rng(s + K).integers(0, 262144, K).astype(np.int32)
            tg, j = synth.accept_targets(d, 262144, seed=s + K)
            cases.append((d.tolist(), tg.tolist(), []))
    _cmp(orc, cases)


def test_accept_eos(orc):
    d = [1, 2, 3, 4]
    tg = [1, 2, 3, 9, 8]
    cases = [(d, tg, [2]), (d, tg, [9]), (d, tg, [77, 3]), (d, tg, [77]), (d, tg, [1, 2, 3, 9])]
    long_d = list(range(1000, 1100))
    long_t = long_d + [5]
    cases.append((long_d, long_t, [1070]))
    cases.append((long_d, long_t, [5]))
    _cmp(orc, cases)
