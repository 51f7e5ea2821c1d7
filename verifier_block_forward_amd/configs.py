"""Shape registry for the drafter-block workloads.

Each entry fixes the model shape, the block shape (M = K+1 rows, R new context
rows, C cached positions), the KV-cache dtype and the seed of its synthetic
inputs. The shapes follow the two block kinds on the hf2q 0.1.1 source pages:

* ``dflash`` -- the DFlash drafter of ``spec_decode/dflash/tensors.rs``
  (``DFlashModelTensors``: ``fc`` over n_t concatenated target hidden states,
  ``hidden_norm``, per-layer attention + SwiGLU tensors, ``final_norm``; embed
  and lm_head shared with the target), driven block-wise as in
  ``spec_decode/dflash/qwen35_orchestrator.rs`` (module doc, "Per-round loop").
* ``mtp`` -- the Qwen3.5 multi-token-prediction block of
  ``models/qwen35/mtp.rs`` (``MtpWeights``: enorm/hnorm, the split eh_proj
  halves, one full-attention layer with an optional sigmoid output gate, a
  dense or MoE FFN, ``shared_head_norm`` + lm_head).

Nothing in this module computes any part of the block.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class BlockConfig:
    name: str
    seed: int
    kind: str  # "dflash" | "mtp"
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    M: int  # block rows (K+1)
    R: int  # new context rows projected this call (DFlash only)
    C: int  # positions already in the KV cache
    kv_dtype: str  # "f32" | "bf16"
    ffn_kind: str = "dense"  # "dense" | "moe"
    intermediate: int = 0  # dense SwiGLU width
    n_target_hidden: int = 0  # DFlash: target hidden states concatenated into fc
    n_experts: int = 0
    top_k: int = 0
    expert_intermediate: int = 0
    shared_intermediate: int = 0
    has_attn_gate: bool = False
    rotary_dim: int = 0  # 0 -> head_dim
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    block_input: str = "x0"  # "x0" (F32 rows given) | "tokens" (gather from embed)
    block_mask: str = "causal"  # "causal" | "bidirectional" (every block row sees the block)
    description: str = ""

    @property
    def K(self) -> int:
        """Number of drafts checked by the accept walk."""
        return max(self.M - 1, 1) if self.kind == "dflash" else 1

    @property
    def rope_dim(self) -> int:
        return self.rotary_dim or self.head_dim

    @property
    def q_total(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_total(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def capacity(self) -> int:
        """KV rows allocated per (layer, kv head): the cached prefix plus one call."""
        return self.C + self.R + self.M

    def with_(self, **kw) -> "BlockConfig":
        return replace(self, **kw)


C0 = BlockConfig(
    name="c0", seed=0, kind="dflash", n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2,
    head_dim=64, vocab=4096, M=4, R=4, C=32, kv_dtype="f32", intermediate=768,
    n_target_hidden=2, block_input="x0",
    description="tiny DFlash drafter block, 1 layer, K+1=4, 32 cached positions",
)

C1 = BlockConfig(
    name="c1", seed=1, kind="dflash", n_layers=5, hidden=2816, n_q_heads=16, n_kv_heads=8,
    head_dim=128, vocab=262144, M=16, R=16, C=4096, kv_dtype="f32", intermediate=8448,
    n_target_hidden=5, block_input="tokens",
    description="DFlash-style drafter, 5 layers, K+1=16, context 4096",
)

C2 = BlockConfig(
    name="c2", seed=2, kind="mtp", n_layers=1, hidden=5120, n_q_heads=24, n_kv_heads=4,
    head_dim=256, vocab=248320, M=1, R=0, C=8192, kv_dtype="f32", intermediate=17408,
    has_attn_gate=True, block_input="x0",
    description="dense MTP draft block, M=1, context 8192, sigmoid output gate",
)

C3 = C1.with_(
    name="c3", seed=3, C=32768, kv_dtype="bf16",
    description="long-context verify-shaped block, K+1=16, context 32768, BF16 KV",
)

C4 = BlockConfig(
    name="c4", seed=4, kind="mtp", n_layers=1, hidden=2048, n_q_heads=16, n_kv_heads=2,
    head_dim=256, vocab=248320, M=1, R=0, C=8192, kv_dtype="f32", ffn_kind="moe",
    n_experts=256, top_k=8, expert_intermediate=512, shared_intermediate=512,
    has_attn_gate=True, block_input="x0",
    description="MoE MTP draft block, M=1, 256 experts top-8 + shared expert",
)

C4_M4 = C4.with_(name="c4m4", M=4, description="MoE MTP draft block, M=4")

CONFIGS = {c.name: c for c in (C0, C1, C2, C3, C4, C4_M4)}


def get(name: str) -> BlockConfig:
    return CONFIGS[name]
