"""Closed-form multiply-accumulate counts of the DiT forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages' "Gflops" are 10^9 multiply-accumulates: counting a MAC as two
FLOPs would make DiT-XL/2 237 rather than the printed 118.6
([DiT-wiki] Conditioning methods table; Results / ImageNet notes).

Counted: every matrix product of the forward pass (patch embedding, timestep
MLP, per-block adaLN modulation, QKV, attention scores and weighted sum,
output projection, FFN, final modulation, linear decoder).  Not counted:
LayerNorm, softmax, activations, position embedding, class-table lookup.
"""
from __future__ import annotations


def gmac_per_image(N, d, T, p, C, Cout, freq_dim=256, pt=1, conditioning="adaLN-Zero",
                   mlp_ratio=4):
    """GMAC for one image/video row.

    conditioning:
      "adaLN" / "adaLN-Zero": per block 12 T d^2 (QKV 3, out 1, FFN 8 at
          ratio 4) + 2 T^2 d (scores + weighted sum) + 6 d^2 (modulation);
          final modulation 2 d^2.
      "in-context": t and c appended as two extra tokens, no modulation
          ([DiT-wiki] Conditioning methods table, first row).
      "cross-attention": no modulation; each block adds a cross-attention
          layer over the two conditioning tokens: Q and output projections
          2 T d^2, K/V projections of two tokens 4 d^2, scores and weighted sum
          4 T d.
    """
    f = 2 * mlp_ratio  # FFN MACs per token per d^2
    kin = pt * p * p * C
    kout = pt * p * p * Cout
    temb = freq_dim * d + d * d
    if conditioning in ("adaLN", "adaLN-Zero"):
        blocks = N * ((4 + f) * T * d * d + 2 * T * T * d + 6 * d * d)
        final = 2 * d * d
    elif conditioning == "in-context":
        T2 = T + 2
        blocks = N * ((4 + f) * T2 * d * d + 2 * T2 * T2 * d)
        final = 0
    elif conditioning == "cross-attention":
        blocks = N * ((4 + f) * T * d * d + 2 * T * T * d + 2 * T * d * d + 4 * d * d + 4 * T * d)
        final = 0
    else:
        raise ValueError(conditioning)
    embed = T * kin * d
    decode = T * d * kout
    return (blocks + embed + decode + temb + final) / 1e9


COND_NAMES = {0: "adaLN-Zero", 1: "in-context", 2: "cross-attention", 3: "MMDiT"}


def gmac_mmdit(N, d, T, L, ctx_dim, p, C, Cout, freq_dim=256, mlp_ratio=4):
    """GMAC for one row of the MMDiT model ([DiT-wiki] MMDiT section): per
    block each stream's QKV, output projection and FFN ((4 + 2 mlp_ratio) d^2
    per token; T image, L text tokens), joint attention over T + L tokens
    (2 (T + L)^2 d) and both streams' modulation (2 x 6 d^2); the text-token
    embedding L ctx_dim d; final modulation 2 d^2.  The pooled-vector
    projection is added by gmac_for."""
    f = 2 * mlp_ratio
    J = T + L
    blocks = N * ((4 + f) * J * d * d + 2 * J * J * d + 12 * d * d)
    embed = T * p * p * C * d + L * ctx_dim * d
    return (blocks + embed + T * d * p * p * Cout + freq_dim * d + d * d + 2 * d * d) / 1e9


def gmac_for(cfg, conditioning=None):
    """GMAC per row for a workload dict (keys N, d, F, H, W, p, pt, C, Cout,
    freq_dim, mlp_hidden, and the conditioning design code, 0 = adaLN-Zero,
    1 = in-context, 2 = cross-attention, 3 = MMDiT with ctx_len, ctx_dim).  Adds the pooled-vector projection
    when present."""
    if conditioning is None:
        conditioning = COND_NAMES[cfg.get("conditioning", 0)]
    T = (cfg["F"] // cfg["pt"]) * (cfg["H"] // cfg["p"]) * (cfg["W"] // cfg["p"])
    if conditioning == "MMDiT":
        return gmac_mmdit(cfg["N"], cfg["d"], T, cfg["ctx_len"], cfg["ctx_dim"], cfg["p"],
                          cfg["C"], cfg["Cout"], cfg["freq_dim"],
                          cfg["mlp_hidden"] // cfg["d"]) + cfg["cond_dim"] * cfg["d"] / 1e9
    g = gmac_per_image(cfg["N"], cfg["d"], T, cfg["p"], cfg["C"], cfg["Cout"],
                       cfg["freq_dim"], cfg["pt"], conditioning,
                       mlp_ratio=cfg["mlp_hidden"] // cfg["d"])
    g += cfg.get("cond_dim", 0) * cfg["d"] / 1e9
    return g


def params(N, d, p, C, Cout, num_classes=1000, freq_dim=256, pt=1, mlp_ratio=4):
    """Parameter count of the adaLN-Zero model (weights + biases + class
    table).  Used for the scaling-rule check: halving p leaves it almost
    unchanged."""
    kin, kout = pt * p * p * C, pt * p * p * Cout
    per_block = (3 * d * d + 3 * d) + (d * d + d) + 2 * (mlp_ratio * d * d) + mlp_ratio * d + d \
        + (6 * d * d + 6 * d)
    return (N * per_block + kin * d + d + freq_dim * d + d + d * d + d
            + (num_classes + 1) * d + 2 * d * d + 2 * d + d * kout + kout)
