"""lm_head_argmax_noalloc (the static-scratch variant of lm_head_argmax) against
lm_head_argmax on the same inputs, through the C ABI: argmax, top-2 margin and
logits bit for bit, on two calls in a row, the second with a smaller input (the
static array keeps the first call's records; the second call must not read them)."""
import numpy as np
import pytest

from verifier_block_forward_amd import synth
from tests.gpu_harness import to_dev, torch

pytestmark = pytest.mark.gpu


def _both(h, W, M, V):
    from verifier_block_forward_amd import dbf
    t = torch()
    H = h.shape[1]
    outs = []
    for kind in ("workspace", "noalloc"):
        am = t.full((M,), -1, dtype=t.int32, device="cuda")
        mg = t.full((M,), float("nan"), dtype=t.float32, device="cuda")
        lg = t.full((M, V), float("nan"), dtype=t.float32, device="cuda")
        if kind == "workspace":
            ws = t.empty(dbf.lm_head_argmax_workspace_bytes(M, H, V), dtype=t.uint8, device="cuda")
            dbf.lm_head_argmax(h, W, am, lg, mg, ws)
        else:
            dbf.lm_head_argmax_noalloc(h, W, am, lg, mg)
        t.cuda.synchronize()
        outs.append((am.cpu().numpy(), mg.cpu().numpy(), lg.cpu().numpy()))
    return outs


def _case(M, H, V, seed, tiled):
    from verifier_block_forward_amd import dbf
    rng = np.random.default_rng(seed)
    h = to_dev(rng.standard_normal((M, H)).astype(np.float32))
    W = to_dev(synth.normal_bf16(seed, 7, (V, H)))
    if tiled:
        W = dbf.tile_weight(W)
    print(f"\n[noalloc] M={M} H={H} V={V} tiled={tiled}", flush=True)
    (a0, m0, l0), (a1, m1, l1) = _both(h, W, M, V)
    assert np.array_equal(a0, a1)
    assert np.array_equal(m0, m1)
    assert np.array_equal(l0, l1)
    assert np.all((a1 >= 0) & (a1 < V))


def test_noalloc_matches_workspace_call_twice():
    # the benchmark's lm_head shape first, then a smaller, ragged one on the same array
    _case(16, 2816, 262144, 51, tiled=True)
    _case(3, 200, 5003, 52, tiled=False)


def test_noalloc_largest_vocabulary():
    from verifier_block_forward_amd import dbf
    _case(2, 64, dbf.NOALLOC_MAX_VOCAB, 53, tiled=True)
