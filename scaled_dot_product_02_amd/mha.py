"""The multi-head self-attention module of the page "flash attention的调用" (its
MultiHeadAttention example) on the HIP path: the weights live in two linear layers as there
(qkv_proj: embed -> 3 embed, out_proj: embed -> embed), and forward() is one call of the C
entry point mha_self_attn_fwd (rocBLAS projections around the attention kernel).

Differences from the page's module, both deliberate:
  * attn_mask follows the library's convention (uint8/bool [S, S], nonzero = the pair is
    masked out), the opposite of a boolean mask given to torch's SDPA;
  * dropout draws from the library's counter-based generator: `seed` is fixed per module
    and the offset advances by one per training-mode call.
"""
from __future__ import annotations

import torch

_DTYPE_NAMES = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}


class MultiHeadAttention(torch.nn.Module):
    def __init__(self, embed_dim: int = 512, num_heads: int = 8, dropout: float = 0.1,
                 bias: bool = True, dtype=torch.bfloat16, device="cuda", seed: int = 0):
        super().__init__()
        if dtype not in _DTYPE_NAMES:
            raise ValueError(f"dtype {dtype} not supported (bf16, fp16 or fp32)")
        self.embed_dim = embed_dim
        self.num_heads = num_heads
        self.qkv_proj = torch.nn.Linear(embed_dim, 3 * embed_dim, bias=bias, dtype=dtype, device=device)
        self.out_proj = torch.nn.Linear(embed_dim, embed_dim, bias=bias, dtype=dtype, device=device)
        self.dropout_p = dropout
        self.seed = seed
        self.calls = 0   # dropout offset of the next training-mode call

    def forward(self, query, key=None, value=None, attn_mask=None):
        from . import mha_self_attn_fwd, mha_workspace_bytes
        for other in (key, value):
            if other is not None and other is not query and not torch.equal(other, query):
                raise NotImplementedError("Cross-attention not implemented")
        B, S, E = query.shape
        if E != self.embed_dim:
            raise ValueError(f"embed dim {E} != {self.embed_dim}")
        dt = _DTYPE_NAMES[query.dtype]
        x = query.contiguous()
        out = torch.empty_like(x)
        nbytes = mha_workspace_bytes(B, S, E, dt)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
        p = self.dropout_p if self.training else 0.0
        offset = 0
        if p > 0.0:
            offset = self.calls
            self.calls += 1
        mask = None
        if attn_mask is not None:
            mask = attn_mask.to(device=x.device, dtype=torch.uint8).contiguous()
        mha_self_attn_fwd(x, self.qkv_proj.weight.contiguous(), self.qkv_proj.bias,
                          self.out_proj.weight.contiguous(), self.out_proj.bias, out, ws, nbytes,
                          B, S, E, self.num_heads, dt, atten_mask=mask, dropout_p=p,
                          seed=self.seed, offset=offset)
        return out
