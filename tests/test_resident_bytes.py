"""Resident-bytes accounting of the drafter's weights ([TENS] page,
`gpu_resident_bytes`, and the identity its integration test asserts: the bytes
resident after upload equal the BF16 file bytes plus the F32 cast expansion of the
norms, (L * (2 hd + 2 H) + 2 H) * 2 bytes, for q_norm, k_norm, input and
post-attention norms per layer and hidden_norm, final_norm per model). Checks the
upload dtype policy (projections BF16, norms F32) and the tensor set. CPU only:
host tensors stand in for device ones, nothing is launched."""
import numpy as np
import pytest

from verifier_block_forward_amd import configs, dbf, synth


def host_tensors(w):
    import torch
    out = {}
    for k, v in w.items():
        if v.dtype == np.uint16:
            out[k] = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16)
        else:
            out[k] = torch.from_numpy(v)
    return out


@pytest.mark.parametrize("cfg", [
    configs.get("c0"),
    configs.BlockConfig(name="dflash_3l", seed=5, kind="dflash", n_layers=3, hidden=192, n_q_heads=4,
                        n_kv_heads=2, head_dim=48, vocab=300, M=4, R=2, C=8, kv_dtype="f32",
                        intermediate=320, n_target_hidden=3, block_input="x0"),
], ids=lambda c: c.name)
def test_resident_bytes_equal_file_bytes_plus_norm_cast(cfg):
    w = synth.make_weights(cfg)
    bw = dbf.BlockWeights(cfg, host_tensors(w))
    own = {k: v for k, v in w.items() if k not in ("embed", "lm_head")}
    file_bytes = sum(v.size * 2 for v in own.values())  # every tensor is BF16 on disk
    H, hd, L = cfg.hidden, cfg.head_dim, cfg.n_layers
    cast_expansion = (L * (2 * hd + 2 * H) + 2 * H) * 2
    assert bw.resident_bytes() == file_bytes + cast_expansion
    # the page's tensor list: fc, hidden_norm, final_norm, and 11 tensors per layer
    assert set(own) == {"fc", "hidden_norm", "final_norm"} | {
        f"layers.{i}.{f}" for i in range(L)
        for f in ("in_norm", "post_norm", "wq", "wk", "wv", "wo", "q_norm", "k_norm",
                  "ffn_gate", "ffn_up", "ffn_down")}
