"""Seeded synthetic workloads for one rank's sharded mixed-precision Adam/AdamW step.

This module describes the five workloads (tensor lists, world size N, the rank
that is measured, dtypes, hyper-parameters, input distributions) and draws their
inputs from seeded torch generators.  It holds none of the step's arithmetic: no
slice reduction, no averaging or unscaling, no Adam update and no rounding of
the outputs.  The HIP path and the CPU oracle both receive the arrays it returns
and nothing else from it.

Where the inputs depend on the flat layout (which local shard element belongs to
which tensor, which elements are padding), the caller passes that layout in as
plain tables; this module does not compute it.

Tensor shapes follow the models the ZeRO pages train or size:
  * the toy MLP (Linear 64->256, GELU, Linear 256->10) of the handbook chapter
    "ZeRO 与 FSDP" (zero_check.py);
  * GPT-2 1.5B (48 layers, hidden 1600) of "ZeRO: 大模型训练的零冗余状态优化",
    Table 5;
  * the 7.5B flat vector of the same page's Figure 1 / Table 1 example;
  * Llama-7B-like and Llama-3-8B-like decoder lists (workload shapes named by
    the measured configuration, not by the pages).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

Shape = Tuple[int, ...]
Tensor = Tuple[str, Shape]


# ----------------------------------------------------------------------------
# tensor lists
# ----------------------------------------------------------------------------

def toy_mlp() -> List[Tensor]:
    """Parameters of Sequential(Linear(64,256), GELU(), Linear(256,10)) in
    module order: 256*64 + 256 + 10*256 + 10 = 19,210 elements."""
    return [("0.weight", (256, 64)), ("0.bias", (256,)),
            ("2.weight", (10, 256)), ("2.bias", (10,))]


def gpt2(n_layer: int = 48, d: int = 1600, vocab: int = 50257, n_ctx: int = 1024) -> List[Tensor]:
    """GPT-2 parameter list (tied output head, so no separate lm_head)."""
    t: List[Tensor] = [("wte", (vocab, d)), ("wpe", (n_ctx, d))]
    for i in range(n_layer):
        p = f"h.{i}."
        t += [(p + "ln_1.weight", (d,)), (p + "ln_1.bias", (d,)),
              (p + "attn.c_attn.weight", (d, 3 * d)), (p + "attn.c_attn.bias", (3 * d,)),
              (p + "attn.c_proj.weight", (d, d)), (p + "attn.c_proj.bias", (d,)),
              (p + "ln_2.weight", (d,)), (p + "ln_2.bias", (d,)),
              (p + "mlp.c_fc.weight", (d, 4 * d)), (p + "mlp.c_fc.bias", (4 * d,)),
              (p + "mlp.c_proj.weight", (4 * d, d)), (p + "mlp.c_proj.bias", (d,))]
    t += [("ln_f.weight", (d,)), ("ln_f.bias", (d,))]
    return t


def llama(n_layer: int, d: int, n_kv_heads: int, head_dim: int, ffn: int, vocab: int) -> List[Tensor]:
    """Llama-style decoder parameter list with an untied lm_head."""
    kv = n_kv_heads * head_dim
    t: List[Tensor] = [("embed_tokens.weight", (vocab, d))]
    for i in range(n_layer):
        p = f"layers.{i}."
        t += [(p + "self_attn.q_proj.weight", (d, d)),
              (p + "self_attn.k_proj.weight", (kv, d)),
              (p + "self_attn.v_proj.weight", (kv, d)),
              (p + "self_attn.o_proj.weight", (d, d)),
              (p + "mlp.gate_proj.weight", (ffn, d)),
              (p + "mlp.up_proj.weight", (ffn, d)),
              (p + "mlp.down_proj.weight", (d, ffn)),
              (p + "input_layernorm.weight", (d,)),
              (p + "post_attention_layernorm.weight", (d,))]
    t += [("norm.weight", (d,)), ("lm_head.weight", (vocab, d))]
    return t


def numels(tensors: Sequence[Tensor]) -> List[int]:
    return [int(math.prod(s)) for _, s in tensors]


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tensors: Tuple[Tensor, ...]
    world: int                     # N, data-parallel degree
    rank: int                      # the rank whose shard is stepped
    bucket_cap: int                # <= 0: one flat bucket (ignored by the dim0 layout)
    grad_dtype: str                # "f32" | "bf16" | "f16": dtype of the N slices
    param_dtype: str               # "f32" | "bf16" | "f16": dtype written to the gather slot
    lr: float
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    loss_scale: float = 1.0        # slices hold loss_scale * gradient
    max_norm: float = 0.0          # > 0: global-norm clip
    steps: int = 3                 # steps a multi-step parity run takes
    t0: int = 0                    # completed steps before the first one here
    grad_sigma: float = 1e-3       # std of each slice's entries (before loss scaling)
    grad_sigma_loguniform: Optional[Tuple[float, float]] = None  # per-tensor sigma range
    grad_zero_frac: float = 0.0    # fraction of positions exactly 0 in every slice
    grad_signed_zero_frac: float = 0.0  # fraction of positions that are +0 or -0 in every slice (sign per slice;
                                        # at a quarter of them -0 in all slices)
    master_sigma: float = 0.02
    m_sigma: float = 0.0           # 0: m starts at 0
    v_sigma: float = 0.0           # 0: v starts at 0; else v = |N(0, v_sigma)|
    inject_inf_step: Optional[int] = None  # 1-based step whose slices carry one +inf
    seed: int = 0
    plan_layout: str = "flat"      # "flat": flat buckets; "dim0": per-parameter dim-0 split

    @property
    def psi(self) -> int:
        return sum(numels(self.tensors))


def _mk(name, tensors, **kw) -> Workload:
    return Workload(name=name, tensors=tuple(tensors), **kw)


# The five measured configurations (full size).
TOY = _mk("toy_mlp_n4", toy_mlp(), world=4, rank=3, bucket_cap=0, grad_dtype="f32",
          param_dtype="f32", lr=1e-2, grad_sigma=1e-2, master_sigma=0.05, seed=11)
GPT2_1P5B = _mk("gpt2_1p5b_n8", gpt2(), world=8, rank=7, bucket_cap=0, grad_dtype="bf16",
                param_dtype="bf16", lr=3e-4, weight_decay=0.1, grad_sigma=1e-3,
                master_sigma=0.02, m_sigma=1e-4, v_sigma=1e-6, t0=100, seed=22)
FLAT_7P5B = _mk("flat_7p5b_n64", [("flat", (7_500_000_000,))], world=64, rank=63, bucket_cap=0,
                grad_dtype="f16", param_dtype="f16", lr=1e-2, loss_scale=65536.0,
                grad_sigma=1e-3, grad_zero_frac=0.01, master_sigma=0.05, seed=33)
LLAMA_7B = _mk("llama_7b_n8", llama(32, 4096, 32, 128, 11008, 32000), world=8, rank=7,
               bucket_cap=0, grad_dtype="bf16", param_dtype="bf16", lr=3e-4, weight_decay=0.1,
               grad_sigma_loguniform=(1e-5, 1e-2), master_sigma=0.02, inject_inf_step=2, seed=44)
LLAMA3_8B = _mk("llama3_8b_n16_buckets", llama(32, 4096, 8, 128, 14336, 128256), world=16,
                rank=15, bucket_cap=500_000_000, grad_dtype="bf16", param_dtype="bf16", lr=3e-4,
                weight_decay=0.1, max_norm=1.0, grad_sigma=1e-3, master_sigma=0.02, seed=55)

FULL: Dict[str, Workload] = {w.name: w for w in (TOY, GPT2_1P5B, FLAT_7P5B, LLAMA_7B, LLAMA3_8B)}
ORDER = [TOY.name, GPT2_1P5B.name, FLAT_7P5B.name, LLAMA_7B.name, LLAMA3_8B.name]

# Scaled-down versions: same recipe, dtypes, N, rank and structure (tensor
# kinds, padding, misaligned slots, several buckets), sized so the oracle
# finishes in seconds while the shard still spans several 2048-element tiles
# and ends in a ragged tail.
SMALL: Dict[str, Workload] = {
    TOY.name: TOY,
    GPT2_1P5B.name: dataclasses.replace(
        GPT2_1P5B, name="gpt2_small_n8", tensors=tuple(gpt2(n_layer=2, d=96, vocab=503, n_ctx=64))),
    FLAT_7P5B.name: dataclasses.replace(
        FLAT_7P5B, name="flat_750k_n64", tensors=(("flat", (750_000,)),)),
    LLAMA_7B.name: dataclasses.replace(
        LLAMA_7B, name="llama_small_n8", tensors=tuple(llama(2, 128, 4, 32, 344, 1000))),
    LLAMA3_8B.name: dataclasses.replace(
        LLAMA3_8B, name="llama3_small_n16_buckets", tensors=tuple(llama(3, 128, 2, 32, 448, 2000)),
        bucket_cap=150_000),
}


# ----------------------------------------------------------------------------
# seeded inputs
# ----------------------------------------------------------------------------

_TORCH_DTYPE = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def torch_dtype(name: str):
    import torch
    return getattr(torch, _TORCH_DTYPE[name])


def _gen(device, seed: int, stream: int):
    import torch
    g = torch.Generator(device=device)
    # one fixed sub-stream per input kind
    g.manual_seed((seed * 1_000_003 + stream * 7919) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


STREAM_MASTER, STREAM_M, STREAM_V, STREAM_SIGMA, STREAM_ZEROS, STREAM_INF = 1, 2, 3, 4, 5, 6
STREAM_SZEROS = 7                  # positions of the signed zeros; their signs use STREAM_SIGNS0 + 1000*s + k
STREAM_SIGNS0 = 20_000_000
STREAM_SLICE0 = 100  # slice k of step s uses STREAM_SLICE0 + 1000*s + k
STREAM_FULL0 = 10_000_000  # full gradient k of step s uses STREAM_FULL0 + 1000*s + k


def tensor_sigmas(w: Workload) -> List[float]:
    """Per-tensor gradient std: constant, or 10**U(log10 lo, log10 hi) per tensor."""
    import torch
    n = len(w.tensors)
    if w.grad_sigma_loguniform is None:
        return [w.grad_sigma] * n
    lo, hi = w.grad_sigma_loguniform
    u = torch.rand(n, generator=_gen("cpu", w.seed, STREAM_SIGMA), dtype=torch.float64)
    return [float(10.0 ** (math.log10(lo) + (math.log10(hi) - math.log10(lo)) * x)) for x in u]


@dataclasses.dataclass
class Layout:
    """The rank's view of the flat layout, as tables supplied by a planner.

    segments: (gather_off, local_off, seg_len, valid) per bucket, in bucket order;
              local elements [local_off + valid, local_off + seg_len) are padding.
    tensor_flat_off: flat (gather-buffer) offset of each tensor's first element.
    """
    S: int
    segments: List[Tuple[int, int, int, int]]
    tensor_flat_off: List[int]


def _elem_sigma(w: Workload, lay: Layout, device):
    """Per-local-element sigma (float32 [S]); 0 on padding."""
    import torch
    sig = tensor_sigmas(w)
    out = torch.zeros(lay.S, dtype=torch.float32, device=device)
    sizes = numels(w.tensors)
    offs = torch.tensor(lay.tensor_flat_off, dtype=torch.int64, device=device)
    ends = offs + torch.tensor(sizes, dtype=torch.int64, device=device)
    sig_t = torch.tensor(sig, dtype=torch.float32, device=device)
    for (goff, loff, seg_len, valid) in lay.segments:
        if valid == 0:
            continue
        if len(set(sig)) == 1:
            out[loff:loff + valid] = sig[0]
            continue
        chunk = 1 << 26
        for a in range(0, valid, chunk):
            b = min(valid, a + chunk)
            flat = torch.arange(goff + a, goff + b, dtype=torch.int64, device=device)
            ti = torch.searchsorted(ends, flat, right=True)
            ok = (ti < len(sizes))
            ti = ti.clamp(max=len(sizes) - 1)
            ok &= flat >= offs[ti]
            out[loff + a:loff + b] = torch.where(ok, sig_t[ti], torch.zeros_like(sig_t[ti]))
    return out


def pad_mask(lay: Layout, device):
    """Bool [S]: True on padding elements of the rank's shard."""
    import torch
    m = torch.zeros(lay.S, dtype=torch.bool, device=device)
    for (_goff, loff, seg_len, valid) in lay.segments:
        m[loff + valid:loff + seg_len] = True
    return m


def make_state(w: Workload, lay: Layout, device="cpu"):
    """fp32 master, m, v of the rank's shard (zeros on padding)."""
    import torch
    S = lay.S
    pad = pad_mask(lay, device)
    master = torch.randn(S, generator=_gen(device, w.seed, STREAM_MASTER), device=device,
                         dtype=torch.float32) * w.master_sigma
    if w.m_sigma > 0:
        m = torch.randn(S, generator=_gen(device, w.seed, STREAM_M), device=device,
                        dtype=torch.float32) * w.m_sigma
    else:
        m = torch.zeros(S, device=device, dtype=torch.float32)
    if w.v_sigma > 0:
        v = (torch.randn(S, generator=_gen(device, w.seed, STREAM_V), device=device,
                         dtype=torch.float32) * w.v_sigma).abs()
    else:
        v = torch.zeros(S, device=device, dtype=torch.float32)
    for x in (master, m, v):
        x.masked_fill_(pad, 0.0)
    return master, m, v


def zero_positions(w: Workload, S: int, device="cpu"):
    """Bool [S] of the seeded positions that are exactly 0 in every slice."""
    import torch
    if w.grad_zero_frac <= 0:
        return None
    u = torch.rand(S, generator=_gen(device, w.seed, STREAM_ZEROS), device=device)
    return u < w.grad_zero_frac


def signed_zero_positions(w: Workload, S: int, device="cpu"):
    """(Bool [S] of the positions holding a zero of either sign in every slice,
    Bool [S] of those where every slice holds -0), or None."""
    import torch
    if w.grad_signed_zero_frac <= 0:
        return None
    u = torch.rand(S, generator=_gen(device, w.seed, STREAM_SZEROS), device=device)
    return u < w.grad_signed_zero_frac, u < 0.25 * w.grad_signed_zero_frac


def inf_position(w: Workload, S: int) -> Tuple[int, int]:
    """(slice, element) of the injected +inf: slice = seed mod N, element ~ U[0, S)."""
    import torch
    j = int(torch.randint(0, S, (1,), generator=_gen("cpu", w.seed, STREAM_INF)).item())
    return w.seed % w.world, j


def make_slices(w: Workload, lay: Layout, step: int = 1, ld: Optional[int] = None, device="cpu",
                out=None):
    """N gradient slices [N, ld] in w.grad_dtype (columns >= S are 0).

    Slice k, element j ~ N(0, sigma_j) * loss_scale, rounded to the slice dtype by
    torch's own cast; padding, the seeded zero positions, and columns beyond S are
    0.  At w.inject_inf_step one element of one slice is +inf.
    """
    import torch
    S = lay.S
    ld = S if ld is None else ld
    assert ld >= S
    dt = torch_dtype(w.grad_dtype)
    if out is None:
        out = torch.zeros((w.world, ld), dtype=dt, device=device)
    else:
        assert out.shape == (w.world, ld) and out.dtype == dt
        out[:, S:].zero_()
    sig = _elem_sigma(w, lay, device) * w.loss_scale
    szeros = signed_zero_positions(w, S, device)
    zeros = zero_positions(w, S, device)
    pad = pad_mask(lay, device)
    if zeros is not None:
        pad |= zeros
    for k in range(w.world):
        g = _gen(device, w.seed, STREAM_SLICE0 + 1000 * step + k)
        x = torch.randn(S, generator=g, device=device, dtype=torch.float32)
        x.mul_(sig)
        x.masked_fill_(pad, 0.0)   # +0 exactly (a product with sigma 0 may be -0)
        if szeros is not None:
            sz, all_neg = szeros
            neg = torch.rand(S, generator=_gen(device, w.seed, STREAM_SIGNS0 + 1000 * step + k),
                             device=device) < 0.5
            x.masked_fill_(sz, 0.0)
            x.masked_fill_(sz & (neg | all_neg) & ~pad, -0.0)
        out[k, :S].copy_(x)
        del x
    if w.inject_inf_step is not None and step == w.inject_inf_step:
        k, j = inf_position(w, S)
        out[k, j] = float("inf")
    return out


def make_full_grads(w: Workload, padded: int, tensor_offsets: Sequence[int], count: int,
                    step: int = 1, ld: Optional[int] = None, device="cpu", inf_at: Optional[int] = None):
    """count whole flat gradients [count, ld] in w.grad_dtype, each laid out like
    the padded flat parameter vector (tensor i at tensor_offsets[i]): entries of
    tensor i ~ N(0, sigma_i) * loss_scale, padding and columns >= padded are +0.
    inf_at, if given, puts +inf at that flat index of buffer 0."""
    import torch
    ld = padded if ld is None else ld
    assert ld >= padded
    out = torch.zeros((count, ld), dtype=torch_dtype(w.grad_dtype), device=device)
    sig = tensor_sigmas(w)
    sizes = numels(w.tensors)
    for k in range(count):
        g = _gen(device, w.seed, STREAM_FULL0 + 1000 * step + k)
        x = torch.randn(padded, generator=g, device=device, dtype=torch.float32)
        y = torch.zeros(padded, dtype=torch.float32, device=device)
        for i, n in enumerate(sizes):
            o = tensor_offsets[i]
            y[o:o + n] = x[o:o + n] * (sig[i] * w.loss_scale)
        out[k, :padded].copy_(y)
    if inf_at is not None:
        out[0, inf_at] = float("inf")
    return out
