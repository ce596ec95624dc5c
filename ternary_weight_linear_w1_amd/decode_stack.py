"""Decode through a stack of BitNet layers' BitLinears, one launch per BitLinear.

Each layer follows the standard Transformer block with every nn.Linear replaced by a
BitLinear ("BitNet b1.58 深度解析" s.2.4 block diagram; subln before O and down,
"微软AI大模型炸场" s.1; squared ReLU in the FFN, same page s.2):

    qkv = BitLinear_qkv(RMSNorm(h; g_in))                     fused input prologue
    o   = attention(qkv)                                       at context length 1: v of the head's KV group
    h   = h + BitLinear_o(RMSNorm(o; g_attn))                  fused subln prologue, residual epilogue
    u   = BitLinear_up(RMSNorm(h; g_post))                     gated: [gate | up] from one [2F][K] BitLinear
    h   = h + BitLinear_down(RMSNorm(act(u); g_ffn))           act = ReLU^2, or ReLU(gate)^2 * up

At context length 1 the softmax over a single key is 1 and rotary embedding at position 0
is the identity, so attention copies each query head's value vector (grouped-query
attention: heads / kv_heads query heads share one KV head). That copy is the only step
outside the library; it is one gather on the device.

All launches go to one stream in order; `capture()` records a whole pass in a HIP graph.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import bitlinear_forward_f32


@dataclass
class LayerWeights:
    """Packed weights (uint8 [N][K/4]) and gamma ([1]) of one layer, and its four gains."""
    qkv: tuple
    o: tuple
    up: tuple       # [F][K/4], or [2F][K/4] (gate rows, then up rows) when gated
    down: tuple
    g_in: object
    g_attn: object
    g_post: object
    g_ffn: object


class DecodeStack:
    def __init__(self, layers, hidden, heads, kv_heads, head_dim, ffn, gated, M=1, eps=1e-5, device="cuda"):
        import torch
        if heads % kv_heads or heads * head_dim != hidden:
            raise ValueError("hidden must equal heads * head_dim and heads a multiple of kv_heads")
        self.layers = list(layers)
        self.hidden, self.heads, self.kv_heads, self.head_dim = hidden, heads, kv_heads, head_dim
        self.ffn, self.gated, self.M, self.eps = ffn, bool(gated), M, eps
        nqkv = (heads + 2 * kv_heads) * head_dim
        self.h = torch.zeros((M, hidden), dtype=torch.float32, device=device)
        self.qkv = torch.empty((M, nqkv), dtype=torch.float32, device=device)
        self.o = torch.empty((M, hidden), dtype=torch.float32, device=device)
        self.u = torch.empty((M, (2 if gated else 1) * ffn), dtype=torch.float32, device=device)
        # column of qkv that feeds o[:, k]: value vector of the KV group of k's query head
        k = torch.arange(hidden, device=device)
        group = (k // head_dim) // (heads // kv_heads)
        self.gather = (heads + kv_heads) * head_dim + group * head_dim + k % head_dim
        for lw in self.layers:
            for name, n, kk in (("qkv", nqkv, hidden), ("o", hidden, hidden),
                                ("up", (2 if gated else 1) * ffn, hidden), ("down", hidden, ffn)):
                p, g = getattr(lw, name)
                if tuple(p.shape) != (n, kk // 4) or tuple(g.shape) != (1,):
                    raise ValueError("layer %s weights must be [%d][%d] packed with gamma [1]" % (name, n, kk // 4))

    def ops(self, i, stream=None):
        """The launches of layer i as (name, callable) in order."""
        import torch
        lw, e = self.layers[i], self.eps
        act = 2 if self.gated else 1
        return [
            ("qkv", lambda: bitlinear_forward_f32(self.h, lw.qkv[0], lw.qkv[1], lw.g_in, e, 0, y=self.qkv,
                                                  stream=stream)),
            ("attn", lambda: torch.index_select(self.qkv, 1, self.gather, out=self.o)),
            ("o", lambda: bitlinear_forward_f32(self.o, lw.o[0], lw.o[1], lw.g_attn, e, 0, y=self.h, stream=stream,
                                                residual=True)),
            ("up", lambda: bitlinear_forward_f32(self.h, lw.up[0], lw.up[1], lw.g_post, e, 0, y=self.u,
                                                 stream=stream)),
            ("down", lambda: bitlinear_forward_f32(self.u, lw.down[0], lw.down[1], lw.g_ffn, e, act, y=self.h,
                                                   stream=stream, residual=True)),
        ]

    def step(self, stream=None):
        """One decode pass through every layer (h is updated in place)."""
        for i in range(len(self.layers)):
            for _, op in self.ops(i, stream):
                op()

    def capture(self):
        """A CUDA/HIP graph of one pass; replay() runs it on the current stream."""
        import torch
        self.step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(stream=torch.cuda.current_stream())
        return g
