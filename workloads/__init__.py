"""Seeded synthetic workloads for the ConvRot int8 quantized linear.

This module only *makes inputs*: it draws seeded random numbers, shapes them
like the MiniMax H3 DiT's projections, and rounds them to bf16 with torch's
own float->bf16 conversion.  It holds none of the method's arithmetic (no
rotation, no quantization, no contraction, no epilogue).  Both the CPU oracle
and the GPU library consume the bytes it returns.

Shapes (the pages fix only the hidden size): the DiT is 33B dense, 50 blocks,
hidden 5376 (cloud-worker RESEARCH.md, "The model"); a 1344x768, 124-frame
canvas gives 32 latent frames of 42x24 tokens = 32256 video tokens (RESEARCH.md,
"The model": 16x spatial / 4x temporal VAE; h3-rs README, "Guides, masks,
ControlNet": 2x2 token grid), and 5.17 s of audio at 40 latent fps is about 208
audio tokens.  The QKV width 3*5376 and the FFN width 14336 are synthetic
choices (the pages do not state them).  Outlier channels stand in for the
activation outliers that the rotation spreads (RESEARCH.md, "Weight
families"); their count and magnitude are synthetic.

Draw order per workload is fixed below; numpy ``default_rng(seed)`` (PCG64).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

HIDDEN = 5376
FFN = 14336
QKV = 3 * HIDDEN
VIDEO_TOKENS = 32256
AUDIO_TOKENS = 208


@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    k: int
    n: int            # GEMM N (2*I for the SwiGLU layer)
    swiglu: bool
    seed: int
    desc: str


WORKLOADS = {
    "tiny": Workload("tiny", 64, 512, 256, False, 0,
                     "tiny ConvRot linear 64x512x256, 4 outlier channels x50"),
    "qkv": Workload("qkv", 4096, HIDDEN, QKV, False, 1,
                    "fused QKV projection 4096x5376x16128, 1% outlier channels x30"),
    "ffn_up": Workload("ffn_up", VIDEO_TOKENS, HIDDEN, 2 * FFN, True, 2,
                       "FFN up + fused SwiGLU 32256x5376x(2x14336), Laplace(0,1) activations"),
    "ffn_down": Workload("ffn_down", VIDEO_TOKENS, FFN, HIDDEN, False, 3,
                         "FFN down 32256x14336x5376, SwiGLU-like activations"),
    "block_chain": Workload("block_chain", VIDEO_TOKENS + AUDIO_TOKENS, HIDDEN, 0, False, 4,
                            "one block's linear chain, M=32464: QKV, attn-out, FFN up+SwiGLU, FFN down"),
}


# Attention: the DiT's 5376-wide hidden state split into 42 heads of 128 (the
# pages give neither the head count nor the head dimension; 128 x 42 = 5376).
ATTN_HEADS = 42
ATTN_HEAD_DIM = 128
ATTN_SEED = 5


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> raw bf16 bits (uint16) via torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_linear(name: str, m: int | None = None) -> dict:
    """Inputs of a single-linear workload: ``x`` raw bf16 [m, k] (uint16),
    ``w`` fp32 [n, k].

    ``m`` < the workload's M keeps the first m token rows of the same draw
    (rows are drawn first-to-last, so a prefix is a prefix); the full weight
    is always drawn."""
    c = WORKLOADS[name]
    assert name != "block_chain"
    rng = np.random.default_rng(c.seed)
    if name == "tiny":
        idx = rng.choice(c.k, 4, replace=False)
        x = _normal(rng, (c.m, c.k))
        x[:, idx] *= np.float32(50.0)
        w = _normal(rng, (c.n, c.k), 0.02)
    elif name == "qkv":
        idx = rng.choice(c.k, 54, replace=False)
        x = _normal(rng, (c.m, c.k))
        x[:, idx] *= np.float32(30.0)
        w = _normal(rng, (c.n, c.k), 0.02)
    elif name == "ffn_up":
        x = rng.laplace(0.0, 1.0, (c.m, c.k)).astype(np.float32)
        w = _normal(rng, (c.n, c.k), 0.02)
    elif name == "ffn_down":
        import torch
        a = torch.from_numpy(_normal(rng, (c.m, c.k)))
        b = torch.from_numpy(_normal(rng, (c.m, c.k)))
        x = (torch.nn.functional.silu(a) * b).numpy()
        del a, b
        w = _normal(rng, (c.n, c.k), 0.01)
    else:
        raise ValueError(name)
    if m is not None:
        x = x[:m]
    return {"x": to_bf16_bits(x), "w": w, "workload": c}


# ------------------------------------------------------------------ block chain

CHAIN_LAYERS = (
    # name, K, N (GEMM), swiglu, weight std
    ("qkv", HIDDEN, QKV, False, 0.02),
    ("attn_out", HIDDEN, HIDDEN, False, 0.02),
    ("ffn_up", HIDDEN, 2 * FFN, True, 0.02),
    ("ffn_down", FFN, HIDDEN, False, 0.01),
)
# the value third of the QKV output feeds the synthetic attention stand-in
V_COLS = (2 * HIDDEN, 3 * HIDDEN)


def make_chain(m: int | None = None) -> dict:
    """Block-chain inputs: x0 raw bf16 [M, 5376] (before its outlier scaling), the
    four fp32 weights, four outlier channel sets and two row permutations.

    Draw order: x0, W_qkv, W_o, W_up, W_down, idx_1..idx_4, perm_1, perm_2.
    ``m`` < 32464 keeps a prefix of x0 and draws the permutations over m rows
    (a smaller but complete chain)."""
    c = WORKLOADS["block_chain"]
    rng = np.random.default_rng(c.seed)
    x0 = _normal(rng, (c.m, HIDDEN))
    ws = [_normal(rng, (n, k), std) for (_, k, n, _, std) in CHAIN_LAYERS]
    idx = [np.sort(rng.choice(k, int(round(0.01 * k)), replace=False)).astype(np.int64)
           for (_, k, _, _, _) in CHAIN_LAYERS]
    mm = c.m if m is None else m
    perm1 = rng.permutation(mm).astype(np.int64)
    perm2 = rng.permutation(mm).astype(np.int64)
    return {"x0": to_bf16_bits(x0[:mm]), "w": ws, "idx": idx,
            "perm": (perm1, perm2), "m": mm}


def chain_outliers(x_bf16, idx):
    """Scale the outlier channels ``idx`` of a bf16 torch tensor by 30 in fp32
    and round back to bf16 (torch ops; runs on CPU or GPU tensors alike)."""
    import torch
    out = x_bf16.clone()
    ii = torch.as_tensor(idx, device=x_bf16.device)
    out[:, ii] = (x_bf16[:, ii].float() * 30.0).to(torch.bfloat16)
    return out


def chain_mix(v_a, v_b):
    """Synthetic stand-in for attention between the QKV and output
    projections: bf16(0.5 * (a + b)) in fp32, for two bf16 torch tensors of
    gathered value rows (torch ops; CPU or GPU)."""
    import torch
    return ((v_a.float() + v_b.float()) * 0.5).to(torch.bfloat16)


def sample_rows(m: int, seed: int, count: int = 64) -> np.ndarray:
    """Rows checked against the oracle at full size: the first two, the last
    two, the 208-row tail above 32256 when present, and ``count`` seeded random
    rows; sorted, unique."""
    rng = np.random.default_rng(1000 + seed)
    rows = {0, 1, m - 2, m - 1}
    if m > VIDEO_TOKENS:
        rows.update(range(VIDEO_TOKENS, m, 16))
    rows.update(rng.choice(m, min(count, m), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < m), dtype=np.int64)


# ------------------------------------------------------------------ attention

def make_attention(s: int = VIDEO_TOKENS, heads: int = ATTN_HEADS, seed: int = ATTN_SEED,
                   qk_std: float = 2.0, k_outlier: float = 0.0) -> dict:
    """Inputs of the attention: one fused QKV matrix, raw bf16 [s, 3 * heads *
    128] with Q, K, V in that order along the columns and head h at columns
    [128 h, 128 h + 128) of each third.

    Synthetic statistics (the pages give none for attention): Q and K are
    N(0, qk_std^2), so the logits q.k / sqrt(128) have standard deviation
    qk_std^2 (4 by default: peaked, not one-hot, over 32256 keys); V is
    N(0, 1).  ``k_outlier`` > 0 multiplies one seeded channel of every key
    head by that factor (a shared key offset direction that makes the
    per-token key scales coarse).  Draw order: Q, K, V, then the outlier
    channels."""
    rng = np.random.default_rng(seed)
    w = heads * ATTN_HEAD_DIM
    q = _normal(rng, (s, w), qk_std)
    k = _normal(rng, (s, w), qk_std)
    v = _normal(rng, (s, w))
    if k_outlier > 0:
        ch = rng.integers(0, ATTN_HEAD_DIM, size=heads)
        k[:, np.arange(heads) * ATTN_HEAD_DIM + ch] *= np.float32(k_outlier)
    bits = np.empty((s, 3 * w), np.uint16)
    for i, t in enumerate((q, k, v)):
        bits[:, i * w:(i + 1) * w] = to_bf16_bits(t)
    return {"qkv": bits, "s": s, "heads": heads}
