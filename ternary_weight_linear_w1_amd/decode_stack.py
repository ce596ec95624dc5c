"""Decode through a stack of BitNet layers: one token per sequence per step, every launch
a library call.

Each layer follows the standard Transformer block with every nn.Linear replaced by a
BitLinear ("BitNet b1.58 深度解析" s.2.4 block diagram; subln before O and down,
"微软AI大模型炸场" s.1; squared ReLU in the FFN, same page s.2; rotary positions, same
page s.2):

    qkv = BitLinear_qkv(RMSNorm(h; g_in))                     fused input prologue
    o   = attention(qkv, cache, pos)                           rotary, grouped-query, bf16 KV cache
    h   = h + BitLinear_o(RMSNorm(o; g_attn))                  fused subln prologue, residual epilogue
    u   = BitLinear_up(RMSNorm(h; g_post))                     gated: [gate | up] from one [2F][K] BitLinear
    h   = h + BitLinear_down(RMSNorm(act(u); g_ffn))           act = ReLU^2, or ReLU(gate)^2 * up

Each layer owns a key and a value cache, bf16 [M][kv_heads][capacity][head_dim]; a step
appends the new token's rotated key and value at `pos` (int32 [M] on the device, one
position per sequence) and attends over slots 0 .. pos. `step(advance=True)` also adds 1
to pos after the last layer, so replaying a captured step decodes successive tokens.

All launches go to one stream in order; `capture()` records a whole pass in a HIP graph.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import bitlinear_attention_decode, bitlinear_attention_workspace_bytes, bitlinear_forward_f32


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
    def __init__(self, layers, hidden, heads, kv_heads, head_dim, ffn, gated, M=1, eps=1e-5, device="cuda",
                 capacity=4096, theta=10000.0):
        import torch
        if heads % kv_heads or heads * head_dim != hidden:
            raise ValueError("hidden must equal heads * head_dim and heads a multiple of kv_heads")
        if head_dim != 128:
            raise ValueError("the attention kernels take head_dim 128")
        self.layers = list(layers)
        self.hidden, self.heads, self.kv_heads, self.head_dim = hidden, heads, kv_heads, head_dim
        self.ffn, self.gated, self.M, self.eps = ffn, bool(gated), M, eps
        self.capacity, self.theta = int(capacity), float(theta)
        nqkv = (heads + 2 * kv_heads) * head_dim
        self.h = torch.zeros((M, hidden), dtype=torch.float32, device=device)
        self.qkv = torch.empty((M, nqkv), dtype=torch.float32, device=device)
        self.o = torch.empty((M, hidden), dtype=torch.float32, device=device)
        self.u = torch.empty((M, (2 if gated else 1) * ffn), dtype=torch.float32, device=device)
        self.pos = torch.zeros((M,), dtype=torch.int32, device=device)
        shape = (M, kv_heads, self.capacity, head_dim)
        self.k_cache = [torch.zeros(shape, dtype=torch.bfloat16, device=device) for _ in self.layers]
        self.v_cache = [torch.zeros(shape, dtype=torch.bfloat16, device=device) for _ in self.layers]
        self.work = torch.empty((bitlinear_attention_workspace_bytes(M, heads, self.capacity),), dtype=torch.uint8,
                                device=device)
        for lw in self.layers:
            for name, n, kk in (("qkv", nqkv, hidden), ("o", hidden, hidden),
                                ("up", (2 if gated else 1) * ffn, hidden), ("down", hidden, ffn)):
                p, g = getattr(lw, name)
                if tuple(p.shape) != (n, kk // 4) or tuple(g.shape) != (1,):
                    raise ValueError("layer %s weights must be [%d][%d] packed with gamma [1]" % (name, n, kk // 4))

    def ops(self, i, stream=None):
        """The launches of layer i as (name, callable) in order."""
        lw, e = self.layers[i], self.eps
        act = 2 if self.gated else 1
        return [
            ("qkv", lambda: bitlinear_forward_f32(self.h, lw.qkv[0], lw.qkv[1], lw.g_in, e, 0, y=self.qkv,
                                                  stream=stream)),
            ("attn", lambda: bitlinear_attention_decode(self.qkv, self.k_cache[i], self.v_cache[i], self.pos,
                                                        self.heads, self.kv_heads, self.theta, out=self.o,
                                                        workspace=self.work, stream=stream)),
            ("o", lambda: bitlinear_forward_f32(self.o, lw.o[0], lw.o[1], lw.g_attn, e, 0, y=self.h, stream=stream,
                                                residual=True)),
            ("up", lambda: bitlinear_forward_f32(self.h, lw.up[0], lw.up[1], lw.g_post, e, 0, y=self.u,
                                                 stream=stream)),
            ("down", lambda: bitlinear_forward_f32(self.u, lw.down[0], lw.down[1], lw.g_ffn, e, act, y=self.h,
                                                   stream=stream, residual=True)),
        ]

    def step(self, stream=None, advance=False):
        """One decode pass through every layer at the current positions (h is updated in
        place); with advance, pos += 1 afterwards."""
        import torch
        for i in range(len(self.layers)):
            for _, op in self.ops(i, stream):
                op()
        if advance:
            if stream is None:
                self.pos.add_(1)
            else:
                with torch.cuda.stream(stream):
                    self.pos.add_(1)

    def capture(self, advance=False):
        """A CUDA/HIP graph of one pass; replay() runs it on the current stream. Capturing
        runs one eager pass first (which writes the caches at the current positions)."""
        import torch
        self.step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(stream=torch.cuda.current_stream(), advance=advance)
        return g
