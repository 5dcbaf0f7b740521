"""Transformer-block decompression overlapped with the forward pass.

The DF11 digest ("Descompressão por bloco de transformer") decompresses all
weight matrices of one transformer block together, just before the block
runs, and notes that the cost is amortised over the batch.  This module runs
a Llama-shaped forward pass whose block weights live only as compressed
containers in HBM: while block i computes on the caller's stream, block i+1
is decoded on a side stream into the other of two scratch buffers; events
order the reuse of each scratch buffer (decode waits for the compute that
last read it, compute waits for its decode).

The block itself is plain PyTorch in BF16 (RMSNorm, grouped-query attention
with rotary embeddings, SwiGLU MLP), weights random, norms at one.  Every
batched product takes contiguous operands.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import dfh


@dataclass(frozen=True)
class BlockShape:
    hidden: int = 4096
    heads: int = 32
    kv_heads: int = 8
    ffn: int = 14336
    rope_theta: float = 500000.0

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    def matrices(self):
        """(name, rows, cols) in the order the block's container concatenates them."""
        d, kv = self.hidden, self.kv_heads * self.head_dim
        return (("q", d, d), ("k", kv, d), ("v", kv, d), ("o", d, d),
                ("gate", self.ffn, d), ("up", self.ffn, d), ("down", d, self.ffn))

    def elements(self) -> int:
        return sum(r * c for _, r, c in self.matrices())


LLAMA3_8B = BlockShape()


def weight_views(flat: torch.Tensor, shape: BlockShape) -> dict:
    """Row-major matrix views into one block's flat BF16 weight buffer."""
    out, off = {}, 0
    for name, r, c in shape.matrices():
        out[name] = flat[off: off + r * c].view(r, c)
        off += r * c
    return out


def _rms_norm(x: torch.Tensor, eps: float = 1e-5) -> torch.Tensor:
    xf = x.float()
    return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps)).to(x.dtype)


def _rope(x: torch.Tensor, theta: float) -> torch.Tensor:
    # x: [heads, T, head_dim]; rotate pairs (i, i + head_dim / 2) in float32
    _, t, hd = x.shape
    half = hd // 2
    inv = 1.0 / (theta ** (torch.arange(0, half, device=x.device, dtype=torch.float32) / half))
    ang = torch.arange(t, device=x.device, dtype=torch.float32)[:, None] * inv[None, :]
    cos, sin = ang.cos(), ang.sin()
    xf = x.float()
    a, b = xf[..., :half], xf[..., half:]
    return torch.cat([a * cos - b * sin, a * sin + b * cos], dim=-1).to(x.dtype)


def block_forward(x: torch.Tensor, w: dict, shape: BlockShape) -> torch.Tensor:
    """One Llama block on activations x [T, hidden] (BF16), causal attention."""
    t = x.shape[0]
    hd, nh, nkv = shape.head_dim, shape.heads, shape.kv_heads
    h = _rms_norm(x)
    q = torch.nn.functional.linear(h, w["q"]).view(t, nh, hd).transpose(0, 1).contiguous()
    k = torch.nn.functional.linear(h, w["k"]).view(t, nkv, hd).transpose(0, 1).contiguous()
    v = torch.nn.functional.linear(h, w["v"]).view(t, nkv, hd).transpose(0, 1).contiguous()
    q, k = _rope(q, shape.rope_theta), _rope(k, shape.rope_theta)
    rep = nh // nkv
    k = k.repeat_interleave(rep, dim=0)
    v = v.repeat_interleave(rep, dim=0).contiguous()
    kt = k.transpose(1, 2).contiguous()                       # [heads, hd, T]
    scores = torch.bmm(q, kt).float() * (hd ** -0.5)           # [heads, T, T]
    mask = torch.ones(t, t, device=x.device, dtype=torch.bool).triu(1)
    scores.masked_fill_(mask, float("-inf"))
    probs = torch.softmax(scores, dim=-1).to(x.dtype).contiguous()
    att = torch.bmm(probs, v).transpose(0, 1).reshape(t, nh * hd)
    x = x + torch.nn.functional.linear(att, w["o"])
    h2 = _rms_norm(x)
    g = torch.nn.functional.linear(h2, w["gate"])
    u = torch.nn.functional.linear(h2, w["up"])
    return x + torch.nn.functional.linear(torch.nn.functional.silu(g) * u, w["down"])


class CompressedBlocks:
    """Blocks held as device-resident containers, decoded one block ahead.

    containers: one host container per block (BF16 kind, matrices in
    BlockShape.matrices() order).  Two scratch buffers of one block each are
    allocated up front; the side stream has the default priority.
    decode_workgroups caps the workgroups of a decode on the side stream
    (0: no cap), so that it runs beside the block's kernels on the CUs they
    leave rather than taking every CU."""

    def __init__(self, containers, shape: BlockShape, device, decode_workgroups: int = 0):
        self.shape = shape
        self.decode_workgroups = int(decode_workgroups)
        self.device = torch.device(device)
        n = shape.elements()
        for c in containers:
            if int(c.info()["n"]) != n or int(c.info()["kind"]) != dfh.KIND_BF16:
                raise ValueError("container does not hold one BF16 block of this shape")
        self.blocks = [dfh.to_device(c, self.device) for c in containers]
        self.scratch = [torch.empty(n, dtype=torch.bfloat16, device=self.device) for _ in range(2)]
        self.side = torch.cuda.Stream(device=self.device)
        self.decoded = [torch.cuda.Event() for _ in range(2)]  # scratch j holds its block
        self.released = [torch.cuda.Event() for _ in range(2)]  # compute done with scratch j

    def _decode(self, i: int, main: torch.cuda.Stream):
        j = i % 2
        self.side.wait_event(self.released[j])
        dfh.df_decompress(self.blocks[i], self.scratch[j], self.side, max_workgroups=self.decode_workgroups)
        self.decoded[j].record(self.side)

    def forward(self, x: torch.Tensor, overlap: bool = True) -> torch.Tensor:
        """All blocks in order.  overlap=False decodes each block on the
        caller's stream right before it runs (no overlap)."""
        main = torch.cuda.current_stream(self.device)
        for j in range(2):
            self.released[j].record(main)
        if overlap:
            self._decode(0, main)
        for i in range(len(self.blocks)):
            j = i % 2
            if overlap:
                if i + 1 < len(self.blocks):
                    self._decode(i + 1, main)
                main.wait_event(self.decoded[j])
            else:
                dfh.df_decompress(self.blocks[i], self.scratch[j], main)
            x = block_forward(x, weight_views(self.scratch[j], self.shape), self.shape)
            self.released[j].record(main)
        return x


def resident_forward(x: torch.Tensor, weights, shape: BlockShape) -> torch.Tensor:
    """The same blocks with every weight buffer resident (the reference)."""
    for flat in weights:
        x = block_forward(x, weight_views(flat, shape), shape)
    return x


def random_blocks(n_blocks: int, shape: BlockShape, seed: int = 0):
    """Host BF16 weights, one flat array per block: N(0, s^2) per matrix with
    s ~ U[0.01, 0.04], from the same generator family as the benchmark."""
    from . import synth
    return [synth.bf16_block(seed, config=synth.CONFIG_FORWARD, block=b, shapes=shape.matrices())[0]
            for b in range(n_blocks)]


def to_torch(host: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(host.view(np.int16)).to(device).view(torch.bfloat16)
