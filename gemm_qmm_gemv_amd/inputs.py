"""Seeded synthetic inputs, shared by the HIP path's tests and the oracle's.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no unpacking, no dequantization, no dot products), and it
imports neither the oracle nor the native library.

Recipe (the pages give no values; the workloads are synthetic):
  * packed weights -- independent uniform 32-bit words.  Every b-bit field of
    the row bitstream is then an independent uniform code in [0, 2^b - 1], so
    the codes are exactly "uniform over the code range" without the generator
    having to know the bit layout;
  * scales  -- fp16(|z| * 0.02 + 1e-3), z ~ N(0, 1), rounded to nearest even;
  * mins    -- fp16(0.05 * z),           z ~ N(0, 1);
  * x       -- fp16(z),                  z ~ N(0, 1);
  * fp16 weights (bits 16, no scales or mins) -- fp16(0.1 * z), z ~ N(0, 1),
    stored two per uint32 word in k order (the low half holds the even k);
  * MoE routing -- logits ~ N(0, 1) per (token, expert); each token picks its
    top-k experts (equal logits: lower expert index first).  Softmax is
    monotone, so this is also the top-k of the softmax probabilities.
Every tensor has its own ``numpy.random.SeedSequence`` built from a tuple of
small integers (config, layer, projection, bit width, role), so any tensor
can be regenerated on its own.
"""
from __future__ import annotations

import numpy as np

ROLE_WEIGHTS = 0
ROLE_X = 1
ROLE_ROUTING = 2


def rng_for(*key: int) -> np.random.Generator:
    """A PCG64 generator seeded from a tuple of non-negative ints."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(v) for v in key])))


def packed_words(rng: np.random.Generator, n: int, k: int, bits: int) -> np.ndarray:
    """Uniform random packed rows, uint32 [n][k*bits/32]."""
    if (k * bits) % 32:
        raise ValueError("k*bits must be a multiple of 32")
    return rng.integers(0, 1 << 32, size=(n, k * bits // 32), dtype=np.uint32)


def scales_mins(rng: np.random.Generator, n: int, k: int, group: int):
    """(scales, mins) fp16 [n][k/group] with the distributions above."""
    if k % group:
        raise ValueError("k must be a multiple of group")
    g = k // group
    s = (np.abs(rng.standard_normal((n, g))) * 0.02 + 1e-3).astype(np.float16)
    m = (0.05 * rng.standard_normal((n, g))).astype(np.float16)
    return s, m


def activations(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    """fp16 [m][k] N(0, 1) activations."""
    return rng.standard_normal((m, k)).astype(np.float16)


def fp16_weight_words(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """fp16 [n][k] weights as uint32 words [n][k/2] (little-endian pairs)."""
    if k % 2:
        raise ValueError("k must be even")
    h = (0.1 * rng.standard_normal((n, k))).astype(np.float16)
    return np.ascontiguousarray(h).view(np.uint32)


def quantized_matrix(n: int, k: int, bits: int, group: int, key=(0,)):
    """dict(w, scales, mins) for one N x K weight matrix (bits 16: fp16
    weights, scales and mins None)."""
    rng = rng_for(*key, ROLE_WEIGHTS)
    if bits == 16:
        return {"w": fp16_weight_words(rng, n, k), "scales": None, "mins": None,
                "n": n, "k": k, "bits": bits, "group": group}
    w = packed_words(rng, n, k, bits)
    s, m = scales_mins(rng, n, k, group)
    return {"w": w, "scales": s, "mins": m, "n": n, "k": k, "bits": bits, "group": group}


def activation_rows(m: int, k: int, key=(0,)) -> np.ndarray:
    return activations(rng_for(*key, ROLE_X), m, k)


def stacked_experts(n_experts: int, n: int, k: int, bits: int, group: int, key=(0,)):
    """dict(w [E][N][K*b/32], scales [E][N][K/g], mins) -- one draw per expert."""
    ws, ss, ms = [], [], []
    for e in range(n_experts):
        q = quantized_matrix(n, k, bits, group, key=(*key, e))
        ws.append(q["w"])
        ss.append(q["scales"])
        ms.append(q["mins"])
    stack = (lambda v: None) if bits == 16 else np.stack
    return {"w": np.stack(ws), "scales": stack(ss), "mins": stack(ms),
            "n_experts": n_experts, "n": n, "k": k, "bits": bits, "group": group}


def routing(tokens: int, n_experts: int, top_k: int, key=(0,)):
    """Top-k routing of N(0,1) logits, rows sorted by expert.

    Returns dict with
      logits  float64 [T][E]
      experts int32 [T][top_k]   chosen experts per token, best first
      weights float64 [T][top_k] softmax probabilities of the chosen experts
      pair_token  int32 [P]      token of each (token, slot) pair, P = T*top_k,
      pair_expert int32 [P]      sorted by expert, ties by token
      pair_weight float32 [P]    routing weight of each pair (same order)
      offsets int32 [E+1]        pairs of expert e are [offsets[e], offsets[e+1])
    """
    rng = rng_for(*key, ROLE_ROUTING)
    logits = rng.standard_normal((tokens, n_experts))
    # Stable sort of -logit keeps the lower index first among equal logits.
    order = np.argsort(-logits, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    probs = z / z.sum(axis=1, keepdims=True)
    weights = np.take_along_axis(probs, order, axis=1)
    tok = np.repeat(np.arange(tokens, dtype=np.int32), top_k)
    exp = order.reshape(-1)
    perm = np.lexsort((tok, exp))  # by expert, then token
    pair_token = tok[perm].astype(np.int32)
    pair_expert = exp[perm].astype(np.int32)
    counts = np.bincount(pair_expert, minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    pair_weight = weights.reshape(-1)[perm].astype(np.float32)
    return {"logits": logits, "experts": order, "weights": weights,
            "pair_token": pair_token, "pair_expert": pair_expert, "pair_weight": pair_weight,
            "offsets": offsets}
