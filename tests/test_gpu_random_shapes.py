"""GPU parity of draft_block_forward against the oracle on seeded random shapes.

The other block tests pick their shapes by hand, one code path at a time. These
draw every size the configuration allows from one fixed seed, so that paths meet in
combinations nobody chose: odd hidden and intermediate sizes (multiples of 8), every
head dim with GQA group sizes 1-8, 1-16 block rows, 0-16 context rows, empty and
longer caches, F32 and BF16 caches, the output gate, token or row input, causal or
bidirectional block masks, partial rotary dims, and MoE blocks with 1-40 experts.
The list is fixed: the same 24 configurations every run.
"""
import numpy as np
import pytest

from verifier_block_forward_amd import configs
from tests.test_gpu_block import run_case, run_moe_case

pytestmark = pytest.mark.gpu

N_CONFIGS = 24
SEED = 2026


def random_configs(n=N_CONFIGS, seed=SEED):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = "dflash" if i % 2 == 0 else "mtp"
        moe = kind == "mtp" and i % 6 == 1
        hd = int(rng.choice([64, 128, 256]))
        nkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 3, 4, 6, 8]))
        M = int(rng.integers(1, 17))
        kw = dict(
            name=f"rand{i:02d}_{kind}{'_moe' if moe else ''}_hd{hd}_g{G}_m{M}",
            seed=100 + i, kind=kind, n_layers=int(rng.integers(1, 3)),
            hidden=8 * int(rng.integers(1, 65)), n_q_heads=nkv * G, n_kv_heads=nkv,
            head_dim=hd, vocab=int(rng.integers(1, 3001)), M=M,
            R=int(rng.integers(0, 17)) if kind == "dflash" else 0,
            C=int(rng.choice([0, int(rng.integers(1, 64)), int(rng.integers(64, 700))])),
            kv_dtype=str(rng.choice(["f32", "bf16"])),
            has_attn_gate=bool(rng.integers(0, 2)),
            rotary_dim=int(rng.choice([0, 2 * int(rng.integers(1, hd // 2 + 1))])),
            block_input=str(rng.choice(["x0", "tokens"])),
            block_mask=str(rng.choice(["causal", "bidirectional"])),
        )
        if kind == "dflash":
            kw["n_target_hidden"] = int(rng.integers(1, 5))
        if moe:
            E = int(rng.integers(1, 41))
            kw.update(ffn_kind="moe", n_experts=E, top_k=int(rng.integers(1, min(E, 8) + 1)),
                      expert_intermediate=8 * int(rng.integers(1, 25)),
                      shared_intermediate=8 * int(rng.integers(1, 25)))
        else:
            kw["intermediate"] = 8 * int(rng.integers(1, 97))
        out.append(configs.BlockConfig(**kw))
    return out


CONFIGS = random_configs()


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_block_random_shape(orc, cfg):
    if cfg.ffn_kind == "moe":
        run_moe_case(orc, cfg)
    else:
        run_case(orc, cfg)


# The shared head and the accept walk fused into the block call, against the
# separate calls, bit for bit, on the first twelve of those shapes that have drafts
# to check (MTP, or DFlash with two or more block rows); every third in the tiled
# weight layout.
FUSED = [c for c in CONFIGS if c.kind == "mtp" or c.M >= 2][:12]


@pytest.mark.parametrize("cfg", FUSED, ids=lambda c: c.name)
def test_fused_head_random_shape(cfg):
    from tests.test_gpu_fused_head import run_pair
    run_pair(cfg, tiled=CONFIGS.index(cfg) % 3 == 0)
