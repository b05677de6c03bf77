"""Seeded synthetic workloads for the large-chunk TTT layer.

This module holds shapes and random draws only: none of the layer's
arithmetic.  Both sides of every parity check (the HIP library and the fp64
oracle) take their inputs from here, and the benchmark times the same
workloads.

Shapes follow the ZipMap pages: every frame of H x W pixels gives
H*W / P^2 patch tokens (patch P = 14) plus one camera token and four register
tokens ("[논문리뷰] ZipMap ..." review, Method, 1. Input Tokenization), so a
518 x 518 frame gives 37*37 + 5 = 1374 tokens and a 70 x 70 frame gives 30.
The model width 1024 is split into 8 heads of 128, each with a SwiGLU hidden
width of 256; the tiny case uses one head of 64 with hidden width 128.

Value recipe (stand-ins for trained projections and real images):
  q, k, v ~ N(0, 1) / sqrt(d_head), rounded to bf16 (kept fp32 for f32 cases)
  eta     = eta_scale * 0.01 * sigmoid(N(0, 1)), fp32, one per token and head
  W1, W3  ~ N(0, 1 / d_head),  W2 ~ N(0, 1 / d_hidden), fp32
Every tensor has its own generator stream: seed * 1000 + stream id.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

PATCH = 14
SPECIAL_TOKENS = 5  # one camera token + four register tokens per frame


def tokens_per_frame(height: int, width: int, patch: int = PATCH) -> int:
    """Tokens one frame contributes: patches plus the five special tokens."""
    if height % patch or width % patch:
        raise ValueError("image size must be a multiple of the patch size")
    return (height // patch) * (width // patch) + SPECIAL_TOKENS


@dataclass(frozen=True)
class Workload:
    name: str
    frames: int
    image: int                  # square frame side in pixels
    heads: int
    d_head: int
    d_hidden: int
    io_dtype: str               # "bf16" or "f32"
    renorm: bool
    extra_queries: int = 0      # target-view ray queries read after the update
    layers: int = 1
    streaming: bool = False     # one frame at a time
    chunked: bool = False       # the frames as the chunks of one multi-chunk call
    description: str = field(default="", compare=False)

    @property
    def tokens_per_frame(self) -> int:
        return tokens_per_frame(self.image, self.image)

    @property
    def n_kv(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def n_q(self) -> int:
        return self.n_kv + self.extra_queries

    def flops_per_token_update(self) -> int:
        # six GEMM-shaped products of d x h per token and head, 2 flops each
        return 12 * self.d_head * self.d_hidden * self.heads

    def flops_per_token_apply(self) -> int:
        return 6 * self.d_head * self.d_hidden * self.heads

    def with_frames(self, frames: int) -> "Workload":
        return replace(self, frames=frames)


WORKLOADS = {
    "tiny": Workload("tiny", 4, 70, 1, 64, 128, "f32", False,
                     description="4 frames x 30 tokens, 1 head, d 64, hidden 128, fp32"),
    "f8": Workload("f8", 8, 518, 8, 128, 256, "bf16", True,
                   description="8 frames x 1374 tokens, 8 heads, d 128, hidden 256"),
    "f100": Workload("f100", 100, 518, 8, 128, 256, "bf16", True, extra_queries=1374,
                     description="100 frames + one 518x518 ray-map target view"),
    "f700": Workload("f700", 700, 518, 8, 128, 256, "bf16", True,
                     description="700 frames x 1374 tokens, one chunk"),
    "f700x24": Workload("f700x24", 700, 518, 8, 128, 256, "bf16", True, layers=24,
                        description="the 700-frame layer repeated 24 times"),
    "stream256": Workload("stream256", 256, 518, 8, 128, 256, "bf16", True, streaming=True,
                          description="256 frames fed one at a time"),
    "chunked256": Workload("chunked256", 256, 518, 8, 128, 256, "bf16", True, streaming=True,
                           chunked=True,
                           description="the 256 frames as 256 chunks of one multi-chunk call"),
    # the full-width fast weight: one head of the whole model width 1024 with
    # hidden 2048 (a 6 d^2 state, d = 1024)
    "fw8": Workload("fw8", 8, 518, 1, 1024, 2048, "bf16", True,
                    description="8 frames x 1374 tokens, one full-width head 1024 / 2048"),
    "fw100": Workload("fw100", 100, 518, 1, 1024, 2048, "bf16", True,
                      description="100 frames x 1374 tokens, one full-width head"),
    "fw700": Workload("fw700", 700, 518, 1, 1024, 2048, "bf16", True,
                      description="700 frames x 1374 tokens, one full-width head, one chunk"),
    # the whole layer around the TTT step: projections from 1024-wide tokens,
    # update + apply, output gate
    "layer700": Workload("layer700", 700, 518, 8, 128, 256, "bf16", True,
                         description="700 frames x 1374 tokens through the whole layer"),
}
CONFIG_IDS = {"tiny": 1, "f8": 2, "f100": 3, "f700": 4, "f700x24": 4, "stream256": 5,
              "chunked256": 5,
              "fw8": 6, "fw100": 7, "fw700": 8, "layer700": 9}

STREAM_Q, STREAM_K, STREAM_V, STREAM_ETA, STREAM_QX = 1, 2, 3, 4, 5
STREAM_W = 100  # + layer


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(stream))
    return g


def _normal(shape, scale, device, seed, stream, dtype):
    g = _gen(device, seed, stream)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(scale)
    return x.to(dtype)


def token_dtype(io_dtype: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[io_dtype]


def make_tokens(n: int, heads: int, d_head: int, io_dtype: str, seed: int,
                device="cpu", stream: int = STREAM_K) -> torch.Tensor:
    """[n, heads, d_head] tokens ~ N(0,1)/sqrt(d_head) in the io dtype."""
    return _normal((n, heads, d_head), 1.0 / math.sqrt(d_head), device, seed, stream,
                   token_dtype(io_dtype))


def make_eta(n: int, heads: int, seed: int, device="cpu", eta_scale: float = 1.0) -> torch.Tensor:
    """[n, heads] fp32 per-token rates: eta_scale * 0.01 * sigmoid(N(0,1))."""
    g = _gen(device, seed, STREAM_ETA)
    z = torch.randn((n, heads), generator=g, device=device, dtype=torch.float32)
    return torch.sigmoid(z).mul_(0.01 * eta_scale)


def make_weights(heads: int, d_head: int, d_hidden: int, seed: int, device="cpu", layer: int = 0):
    """Fast-weight initial state: W1, W3 [H, h, d] ~ N(0, 1/d); W2 [H, d, h] ~ N(0, 1/h)."""
    base = STREAM_W + 3 * layer
    w1 = _normal((heads, d_hidden, d_head), 1.0 / math.sqrt(d_head), device, seed, base, torch.float32)
    w2 = _normal((heads, d_head, d_hidden), 1.0 / math.sqrt(d_hidden), device, seed, base + 1, torch.float32)
    w3 = _normal((heads, d_hidden, d_head), 1.0 / math.sqrt(d_head), device, seed, base + 2, torch.float32)
    return w1, w2, w3


STREAM_X, STREAM_WIN, STREAM_WETA, STREAM_WG, STREAM_GAMMA = 6, 7, 8, 9, 10


def make_layer_tensors(n: int, heads: int, d_head: int, seed: int, device="cpu",
                       d_in: int | None = None):
    """Input tokens and slow weights of the whole layer (synthetic stand-ins for
    trained projections).  Scales follow the token recipe above: with
    x ~ N(0, 1) (bf16), W_Q, W_K, W_V rows ~ N(0, 1 / (d_in d_head)) give q, k, v
    of variance 1 / d_head; W_eta rows ~ N(0, 1 / d_in) give rate logits of
    variance 1 (so eta = 0.01 sigmoid(.) as above); W_g ~ N(0, 1 / (H d_head));
    gamma = 1 + 0.1 N(0, 1).  Returns x [n, d_in], w_in [3 H d + H, d_in] and
    w_gate [H d, H d] in bf16, gamma [H d] fp32."""
    width = heads * d_head
    d_in = width if d_in is None else d_in
    x = _normal((n, d_in), 1.0, device, seed, STREAM_X, torch.bfloat16)
    w_qkv = _normal((3 * width, d_in), 1.0 / math.sqrt(d_in * d_head), device, seed, STREAM_WIN,
                    torch.float32)
    w_eta = _normal((heads, d_in), 1.0 / math.sqrt(d_in), device, seed, STREAM_WETA, torch.float32)
    w_in = torch.cat([w_qkv, w_eta]).to(torch.bfloat16)
    w_gate = _normal((width, width), 1.0 / math.sqrt(width), device, seed, STREAM_WG,
                     torch.bfloat16)
    gamma = 1.0 + _normal((width,), 0.1, device, seed, STREAM_GAMMA, torch.float32)
    return x, w_in, w_gate, gamma


def make_inputs(wl: Workload, seed: int | None = None, device="cpu", eta_scale: float = 1.0,
                layer: int = 0, io_dtype: str | None = None):
    """All tensors of one layer invocation of ``wl``.

    Returns a dict with q [n_q, H, d], k, v [n_kv, H, d], eta [n_kv, H] and
    w1, w2, w3.  For workloads with extra target-view queries, those rows sit
    after the n_kv image queries in q.
    """
    if seed is None:
        seed = CONFIG_IDS.get(wl.name, 9)
    io = io_dtype or wl.io_dtype
    n, H, d = wl.n_kv, wl.heads, wl.d_head
    q = make_tokens(n, H, d, io, seed, device, STREAM_Q)
    if wl.extra_queries:
        qx = make_tokens(wl.extra_queries, H, d, io, seed, device, STREAM_QX)
        q = torch.cat([q, qx], dim=0)
    k = make_tokens(n, H, d, io, seed, device, STREAM_K)
    v = make_tokens(n, H, d, io, seed, device, STREAM_V)
    eta = make_eta(n, H, seed, device, eta_scale)
    w1, w2, w3 = make_weights(H, d, wl.d_hidden, seed, device, layer)
    return {"q": q, "k": k, "v": v, "eta": eta, "w1": w1, "w2": w2, "w3": w3}


def frame_slices(wl: Workload):
    """Token ranges [start, end) of the frames of a streaming workload."""
    p = wl.tokens_per_frame
    return [(t * p, (t + 1) * p) for t in range(wl.frames)]
