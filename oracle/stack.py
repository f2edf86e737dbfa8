"""Block stack and token refiner in numpy fp64 (test infrastructure only; see
__init__).

Pages: "MiniMaxH3Transformer3DModel" (diffusers API page) -- constructor
parameters num_layers (the DiT block stack), num_refiner_layers (token refiner
blocks applied to the projected text stream), text_dim (width of the text
conditioning), final_norm_eps (epsilon of the refiner's output norm); forward
parameters (encoder_hidden_states are ordered as text_indices).  "MiniMax H3
Inference Engine voor Mac computers" -- scheduling notes: one activation arena
reused from block to block.

Readings (listed in the design doc):
  * stack: x_{l+1} = block_l(x_l) with every block's own weights and its own
    AdaLN table computed from the same timestep embedding; x is stored in
    bf16 between blocks (the residual stream is bf16).
  * refiner: text = text_in @ W_text^T (bf16 stack, no bias, like every
    projection inside the block stack), then num_refiner_layers blocks of the
    same structure over the text rows alone (all tagged text, their own
    positions and timestep indices), then LayerNorm without affine, eps =
    final_norm_eps, stored in bf16.
"""
from __future__ import annotations

import numpy as np

from . import bf16_round, bf16_to_f64
from .block import adaln_table, block_forward, layer_norm


def stack_forward(x_bits, temb_bits, blocks, layout, dims: dict, store_bf16: bool = True,
                  fused_qkv: bool = True, eps: float = 1e-5, pos_scale=None) -> np.ndarray:
    """x after len(blocks) blocks, as bf16 bits [L, hidden].

    blocks: list of dicts with w_ada, w_qkv, w_o, w_fc1, w_fc2 (bf16 bits).
    dims: L, hidden, heads, head_dim, ffn.  The residual stream handed from
    block to block is bf16 in either mode; store_bf16 only selects whether
    the tensors inside each block are rounded as the GPU stores them."""
    x = np.asarray(x_bits, dtype=np.uint16)
    for w in blocks:
        inp = dict(dims)
        inp.update(w)
        inp.update(layout=layout, x=x, temb=temb_bits)
        xv = block_forward(inp, store_bf16=store_bf16, eps=eps,
                           mod=adaln_table(temb_bits, w["w_ada"]), fused_qkv=fused_qkv,
                           pos_scale=pos_scale)
        x = bf16_round(xv)
    return x


def text_refiner(text_bits, w_text_bits, temb_bits, blocks, text_layout, dims: dict,
                 final_eps: float = 1e-5, store_bf16: bool = True, eps: float = 1e-5):
    """Refined text rows [n_text, hidden]: bf16 bits when store_bf16, else fp64
    (the output norm of the last bf16 residual stream)."""
    t = bf16_to_f64(text_bits) @ bf16_to_f64(w_text_bits).T
    x = bf16_round(t)
    if blocks:
        x = stack_forward(x, temb_bits, blocks, text_layout, dims, store_bf16=store_bf16, eps=eps)
    y = layer_norm(bf16_to_f64(x), final_eps)
    return bf16_round(y) if store_bf16 else y


def reduced_stack_forward(x_bits, temb_bits, blocks, layout, plan: dict, merge_after: int,
                          restore_before: int, dims: dict, store_bf16: bool = True,
                          eps: float = 1e-5) -> np.ndarray:
    """The stack with token reduction (engine page, token-reduction notes):
    blocks [0, merge_after) at full resolution, merge, blocks
    [merge_after, restore_before) on the reduced rows (plan["layout"], its
    positions scaled by plan["pos_scale"]), restore from the bypass, then the
    remaining blocks at full resolution.  dims' L is the full row count."""
    from .tokenred import merge, unmerge
    x = stack_forward(x_bits, temb_bits, blocks[:merge_after], layout, dims, store_bf16,
                      eps=eps) if merge_after else np.asarray(x_bits, np.uint16)
    bypass = x
    xr0 = merge(x, plan["src0"], plan["src1"])
    rdims = dict(dims)
    rdims["L"] = int(plan["layout"]["L"])
    xr1 = stack_forward(xr0, temb_bits, blocks[merge_after:restore_before], plan["layout"], rdims,
                        store_bf16, eps=eps, pos_scale=plan["pos_scale"])
    x = unmerge(bypass, xr0, xr1, plan["src0"], plan["src1"])
    if restore_before < len(blocks):
        x = stack_forward(x, temb_bits, blocks[restore_before:], layout, dims, store_bf16, eps=eps)
    return x
