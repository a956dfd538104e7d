"""Workload shapes.  Weights are N x K (output rows x reduction).

The shapes are those of public model configurations; the pages name the
models but print none of their dimensions.  Every tensor is synthetic
(see ``inputs.py``).
"""
from __future__ import annotations

GROUP = 64

# Single decode GEMV: K = 1024 -> N = 3072, Q4.
SINGLE_Q4 = {"name": "q4_single_3072x1024", "n": 3072, "k": 1024, "bits": 4}

# Qwen3-0.6B-shaped decode projection set, Q4: 28 layers + LM head.
QWEN3_06B_LAYERS = 28
QWEN3_06B_PROJ = [  # (name, N, K)
    ("q_proj", 2048, 1024),
    ("k_proj", 1024, 1024),
    ("v_proj", 1024, 1024),
    ("o_proj", 1024, 2048),
    ("gate_proj", 3072, 1024),
    ("up_proj", 3072, 1024),
    ("down_proj", 1024, 3072),
]
QWEN3_06B_LM_HEAD = ("lm_head", 151936, 1024)

# Llama-3.2-3B-shaped GEMVs for the bit-width sweep.
LLAMA32_3B_PROJ = [
    ("q_proj", 3072, 3072),
    ("k_proj", 1024, 3072),
    ("v_proj", 1024, 3072),
    ("o_proj", 3072, 3072),
    ("gate_proj", 8192, 3072),
    ("up_proj", 8192, 3072),
    ("down_proj", 3072, 8192),
    ("lm_head", 128256, 3072),
]
# Decoder layers of that model's public configuration (used only to add the
# per-launch times up to a per-token projection time).
LLAMA32_3B_LAYERS = 28
# Q5 and fp16 weights (16) are not among the pages' measured widths; they
# are swept beside them.
SWEEP_BITS = (2, 3, 4, 5, 6, 8, 16)

# Llama-3.2-1B-shaped prefill GEMMs, Q4, M tokens.
LLAMA32_1B_PROJ = [
    ("q_proj", 2048, 2048),
    ("k_proj", 512, 2048),
    ("v_proj", 512, 2048),
    ("o_proj", 2048, 2048),
    ("gate_proj", 8192, 2048),
    ("up_proj", 8192, 2048),
    ("down_proj", 2048, 8192),
]
PREFILL_M = (128, 512)
# Longer prefill (2048 tokens, the length vendor prefill figures use), timed
# with fp32 and with fp16 output.
PREFILL_M_LONG = 2048

# Qwen3-30B-A3B-shaped experts, Q4.
MOE = {"n_experts": 128, "top_k": 8, "hidden": 2048, "inter": 768,
       "tokens": (1, 16)}
MOE_PROJ = [  # (name, N, K)
    ("gate_proj", 768, 2048),
    ("up_proj", 768, 2048),
    ("down_proj", 2048, 768),
]

# Workload ids used as the first seed component.
CFG_SINGLE, CFG_DECODE_SET, CFG_SWEEP, CFG_PREFILL, CFG_MOE = 0, 1, 2, 3, 4


def decode_set():
    """[(layer, proj_index, name, N, K)] for the Qwen3-0.6B projection set."""
    out = []
    for layer in range(QWEN3_06B_LAYERS):
        for j, (name, n, k) in enumerate(QWEN3_06B_PROJ):
            out.append((layer, j, name, n, k))
    name, n, k = QWEN3_06B_LM_HEAD
    out.append((QWEN3_06B_LAYERS, 0, name, n, k))
    return out


def weight_bytes(n: int, k: int, bits: int, group: int = GROUP) -> int:
    """Compressed bytes of one N x K matrix: codes + fp16 scale + fp16 min
    (bits 16: the fp16 weights alone)."""
    if bits == 16:
        return 2 * n * k
    return n * k * bits // 8 + 4 * n * (k // group)


def gemv_bytes(n: int, k: int, bits: int, group: int = GROUP, m: int = 1) -> int:
    """Algorithmic bytes of Y[M][N] = X W^T: weights + fp16 x + fp32 y."""
    return weight_bytes(n, k, bits, group) + 2 * m * k + 4 * m * n
