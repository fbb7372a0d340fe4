"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds input recipes only (random draws, the per-workload shape and value
distributions, dtype casts); none of the gated-delta-rule arithmetic lives here. Both the
GPU path and the CPU oracle receive the arrays it returns, unchanged.

All draws are on the CPU with an explicit ``torch.Generator`` so every consumer sees the
same values for the same seed. Value distributions follow the workloads the pages use:
keys/queries drawn from a normal and L2-normalised along the head dim, values normal, the
forget gate alpha = sigmoid(randn + 3) passed as its log g = log(alpha) = logsigmoid(x + 3),
write gate beta = sigmoid(randn).
"""
from dataclasses import dataclass, field
from typing import Optional

import torch

F32 = torch.float32
BF16 = torch.bfloat16


def _gen(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(int(seed))


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    """Recipe step: rescale each head-dim vector to unit L2 length (fp32)."""
    x = x.to(F32)
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def gate_from_normal(x: torch.Tensor) -> torch.Tensor:
    """log(alpha) with alpha = sigmoid(x + 3), computed in fp32."""
    return torch.nn.functional.logsigmoid(x.to(F32) + 3.0)


def beta_from_normal(x: torch.Tensor) -> torch.Tensor:
    return torch.sigmoid(x.to(F32))


@dataclass
class PrefillInputs:
    q: torch.Tensor             # [T, H, dk]  dtype
    k: torch.Tensor             # [T, H, dk]  dtype
    v: torch.Tensor             # [T, H, dv]  dtype
    g: torch.Tensor             # [T, H] or [T, H, dk]  fp32
    beta: torch.Tensor          # [T, H]  fp32
    cu_seqlens: torch.Tensor    # [n+1] int32
    scale: float
    qk_l2norm: bool
    chunk: int
    init_states: Optional[torch.Tensor] = None  # [n, H, dk, dv] fp32 or None
    extra: dict = field(default_factory=dict)

    @property
    def dtype(self):
        return self.q.dtype

    @property
    def n_seqs(self):
        return int(self.cu_seqlens.numel() - 1)

    @property
    def total_tokens(self):
        return int(self.q.shape[0])

    @property
    def perkey(self):
        return self.g.dim() == 3


def tiny_config(seed: int = 0) -> PrefillInputs:
    """Tiny GDN: one sequence, T=64, H=1, d_k=d_v=16, chunk 16, fp32, zero initial state.
    Draw order q, k, v, alpha-normal, then beta-normal, with q, k ~ randn/4 then unit rows
    (the handbook's recurrent-vs-chunked toy uses this draw order and scaling)."""
    g = _gen(seed)
    T, D = 64, 16
    q = torch.randn(T, D, generator=g) / 4
    k = torch.randn(T, D, generator=g) / 4
    v = torch.randn(T, D, generator=g)
    a = torch.randn(T, generator=g)
    b = torch.randn(T, generator=g)
    return PrefillInputs(
        q=_unit_rows(q)[:, None, :].contiguous(), k=_unit_rows(k)[:, None, :].contiguous(),
        v=v[:, None, :].contiguous(), g=gate_from_normal(a)[:, None].contiguous(),
        beta=beta_from_normal(b)[:, None].contiguous(),
        cu_seqlens=torch.tensor([0, T], dtype=torch.int32), scale=1.0, qk_l2norm=False,
        chunk=16)


def random_prefill(seed: int, lengths, H: int, dk: int, dv: int, dtype=BF16,
                   perkey: bool = False, chunk: int = 64, scale: Optional[float] = None,
                   prenorm: bool = True, with_init: bool = False,
                   gate_shift: float = 3.0) -> PrefillInputs:
    """Packed varlen prefill inputs. q, k ~ randn (unit rows if prenorm), v ~ randn,
    g = logsigmoid(randn + gate_shift) per head or per key channel, beta = sigmoid(randn).
    with_init draws fp32 initial states ~ randn / sqrt(dk)."""
    gen = _gen(seed)
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    q = torch.randn(T, H, dk, generator=gen)
    k = torch.randn(T, H, dk, generator=gen)
    v = torch.randn(T, H, dv, generator=gen)
    a = torch.randn(*((T, H, dk) if perkey else (T, H)), generator=gen)
    b = torch.randn(T, H, generator=gen)
    if prenorm:
        q, k = _unit_rows(q), _unit_rows(k)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    init = None
    if with_init:
        init = torch.randn(len(lengths), H, dk, dv, generator=gen) / dk ** 0.5
    return PrefillInputs(
        q=q.to(dtype).contiguous(), k=k.to(dtype).contiguous(), v=v.to(dtype).contiguous(),
        g=torch.nn.functional.logsigmoid(a + gate_shift).contiguous(),
        beta=beta_from_normal(b).contiguous(), cu_seqlens=cu,
        scale=(1.0 / dk ** 0.5) if scale is None else float(scale),
        qk_l2norm=not prenorm, chunk=chunk, init_states=init)


def prefill_config(seed: int = 0, T: int = 8192, H: int = 16, d: int = 128,
                   chunk: int = 64) -> PrefillInputs:
    """GDN chunked prefill: one sequence, T=8192, H=16, d=128, chunk 64, bf16 q/k/v with
    q, k unit rows (normalised in fp32, then cast), fp32 gates, zero initial state,
    scale 1/sqrt(d)."""
    gen = _gen(seed)
    q = torch.randn(T, H, d, generator=gen)
    k = torch.randn(T, H, d, generator=gen)
    v = torch.randn(T, H, d, generator=gen)
    a = torch.randn(T, H, generator=gen)
    b = torch.randn(T, H, generator=gen)
    return PrefillInputs(
        q=_unit_rows(q).to(BF16).contiguous(), k=_unit_rows(k).to(BF16).contiguous(),
        v=v.to(BF16).contiguous(), g=gate_from_normal(a).contiguous(),
        beta=beta_from_normal(b).contiguous(),
        cu_seqlens=torch.tensor([0, T], dtype=torch.int32), scale=1.0 / d ** 0.5,
        qk_l2norm=False, chunk=chunk)


def prefill_batch_config(seed: int = 0, n_seqs: int = 32, L: int = 2048, H: int = 16,
                         d: int = 128, chunk: int = 64) -> PrefillInputs:
    """A serving-style prefill batch: n_seqs sequences of L tokens (32 x 2048 = 65536 tokens),
    H=16, d=128, chunk 64, drawn as the single-sequence workload (bf16 q/k/v, q and k unit rows,
    fp32 gates logsigmoid(randn + 3), beta sigmoid(randn)), zero initial states."""
    gen = _gen(seed)
    T = n_seqs * L
    q = torch.randn(T, H, d, generator=gen)
    k = torch.randn(T, H, d, generator=gen)
    v = torch.randn(T, H, d, generator=gen)
    a = torch.randn(T, H, generator=gen)
    b = torch.randn(T, H, generator=gen)
    return PrefillInputs(
        q=_unit_rows(q).to(BF16).contiguous(), k=_unit_rows(k).to(BF16).contiguous(),
        v=v.to(BF16).contiguous(), g=gate_from_normal(a).contiguous(),
        beta=beta_from_normal(b).contiguous(),
        cu_seqlens=torch.arange(0, T + 1, L, dtype=torch.int32), scale=1.0 / d ** 0.5,
        qk_l2norm=False, chunk=chunk)


def decode_pool(seed: int, n_slots: int, H: int, dk: int, dv: int) -> torch.Tensor:
    """fp32 slot-indexed state pool [n_slots, H, dk, dv] ~ randn / sqrt(dk)."""
    gen = _gen(seed)
    return (torch.randn(n_slots, H, dk, dv, generator=gen) / dk ** 0.5).contiguous()


def decode_slots(seed: int, n_slots: int, batch: int) -> torch.Tensor:
    """Random slot map: the first `batch` entries of a permutation of the pool (unique)."""
    return torch.randperm(n_slots, generator=_gen(seed))[:batch].to(torch.int32).contiguous()


class DecodeStream:
    """Per-step one-token inputs for a batch of requests: q, k unit rows (fp32 then cast),
    v ~ randn, g = logsigmoid(randn + 3) (per head or per key channel), beta = sigmoid."""

    def __init__(self, seed: int, batch: int, H: int, dk: int, dv: int, dtype=BF16,
                 perkey: bool = False, prenorm: bool = True):
        self.gen = _gen(seed)
        self.B, self.H, self.dk, self.dv = batch, H, dk, dv
        self.dtype, self.perkey, self.prenorm = dtype, perkey, prenorm

    def next(self):
        B, H, dk, dv, gen = self.B, self.H, self.dk, self.dv, self.gen
        q = torch.randn(B, H, dk, generator=gen)
        k = torch.randn(B, H, dk, generator=gen)
        v = torch.randn(B, H, dv, generator=gen)
        a = torch.randn(*((B, H, dk) if self.perkey else (B, H)), generator=gen)
        b = torch.randn(B, H, generator=gen)
        if self.prenorm:
            q, k = _unit_rows(q), _unit_rows(k)
        return (q.to(self.dtype).contiguous(), k.to(self.dtype).contiguous(),
                v.to(self.dtype).contiguous(), gate_from_normal(a).contiguous(),
                beta_from_normal(b).contiguous())


def spec_round(seed: int, batch: int, n_pos: int, H: int, dk: int, dv: int, dtype=BF16,
               perkey: bool = False, prenorm: bool = True):
    """One verify round of speculative decoding: n_pos tokens per request, drawn as the
    one-token decode recipe for batch * n_pos rows and laid out [batch, n_pos, H, d]."""
    q, k, v, g, b = DecodeStream(seed, batch * n_pos, H, dk, dv, dtype=dtype, perkey=perkey,
                                 prenorm=prenorm).next()
    shp = (batch, n_pos)
    return (q.view(*shp, H, dk), k.view(*shp, H, dk), v.view(*shp, H, dv),
            g.view(*shp, *g.shape[1:]), b.view(*shp, H))


def spec_slot_table(seed: int, n_slots: int, batch: int, n_pos: int):
    """Distinct pool slots per (request, position) ([batch, n_pos] int32, a random
    permutation prefix) and num_accepted in [1, n_pos] per request."""
    gen = _gen(seed)
    table = torch.randperm(n_slots, generator=gen)[:batch * n_pos].view(batch, n_pos)
    acc = torch.randint(1, n_pos + 1, (batch,), generator=gen)
    return table.to(torch.int32).contiguous(), acc.to(torch.int32).contiguous()


@dataclass
class FusedDecodeInputs:
    x: torch.Tensor            # [B, 3 H d] dtype, q|k|v before the convolution
    conv_w: torch.Tensor       # [3 H d, W] fp32
    conv_state: torch.Tensor   # [n_slots, 3 H d, W - 1] dtype
    forget_b: torch.Tensor     # [B, H, d] fp32
    write_logit: torch.Tensor  # [B, H] fp32
    A_log: torch.Tensor        # [H] fp32
    dt_bias: torch.Tensor      # [H, d] fp32
    lower_bound: float


def fused_decode_step(seed: int, batch: int, n_slots: int, H: int, d: int, width: int = 4,
                      dtype=BF16) -> FusedDecodeInputs:
    """One fused KDA decode step: raw q|k|v ~ randn, conv weights randn/2 and a conv-state
    pool ~ randn (all as the KDA prefill recipe), gate projection forget_b ~ randn, write
    logits ~ randn, A_log = log(uniform(1, 16)) per head, dt_bias ~ randn/2 per (head,
    channel), lower_bound -5 (the page's value). No trained weights: all synthetic."""
    gen = _gen(seed)
    CH = 3 * H * d
    x = torch.randn(batch, CH, generator=gen).to(dtype)
    w = torch.randn(CH, width, generator=gen) / 2
    cs = torch.randn(n_slots, CH, width - 1, generator=gen).to(dtype)
    fb = torch.randn(batch, H, d, generator=gen)
    wl = torch.randn(batch, H, generator=gen)
    A_log = torch.log(1.0 + 15.0 * torch.rand(H, generator=gen))
    dt = torch.randn(H, d, generator=gen) / 2
    return FusedDecodeInputs(x=x.contiguous(), conv_w=w.contiguous(), conv_state=cs.contiguous(),
                             forget_b=fb.contiguous(), write_logit=wl.contiguous(),
                             A_log=A_log.contiguous(), dt_bias=dt.contiguous(), lower_bound=-5.0)


@dataclass
class ConvPrefillInputs:
    x: torch.Tensor           # [T, 3 H d] dtype, q|k|v before the convolution
    conv_w: torch.Tensor      # [3 H d, W] fp32
    g: torch.Tensor           # [T, H] or [T, H, d] fp32
    beta: torch.Tensor        # [T, H] fp32
    cu_seqlens: torch.Tensor  # [n + 1] int32
    conv_hist: torch.Tensor   # [n, 3 H d, W - 1] dtype, conv history per sequence
    init_states: torch.Tensor  # [n, H, d, d] fp32
    H: int
    d: int
    scale: float
    qk_l2norm: bool


def conv_prefill(seed: int, lengths, H: int, d: int, width: int = 4, dtype=BF16,
                 perkey: bool = True, gate_shift: float = 3.0) -> ConvPrefillInputs:
    """Packed varlen inputs of the conv-fused prefill, as the KDA recipe: raw q|k|v ~ randn,
    conv weights randn/2, gates logsigmoid(randn + gate_shift) (per key or per head), beta =
    sigmoid(randn), conv histories ~ randn and initial states ~ randn/sqrt(d); q and k are
    L2-normalised in the kernel after the convolution."""
    gen = _gen(seed)
    lengths = [int(x) for x in lengths]
    T, n, CH = sum(lengths), len(lengths), 3 * H * d
    x = torch.randn(T, CH, generator=gen).to(dtype)
    w = torch.randn(CH, width, generator=gen) / 2
    a = torch.randn(*((T, H, d) if perkey else (T, H)), generator=gen)
    b = torch.randn(T, H, generator=gen)
    hist = torch.randn(n, CH, width - 1, generator=gen).to(dtype)
    init = torch.randn(n, H, d, d, generator=gen) / d ** 0.5
    cu = torch.zeros(n + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return ConvPrefillInputs(
        x=x.contiguous(), conv_w=w.contiguous(),
        g=torch.nn.functional.logsigmoid(a + gate_shift).contiguous(),
        beta=beta_from_normal(b).contiguous(), cu_seqlens=cu, conv_hist=hist.contiguous(),
        init_states=init.contiguous(), H=H, d=d, scale=1.0 / d ** 0.5, qk_l2norm=True)


@dataclass
class KdaVarlenInputs:
    x: torch.Tensor           # [T, 3*H*d] bf16, raw fused q|k|v projection output
    conv_w: torch.Tensor      # [3*H*d, 4] fp32
    g: torch.Tensor           # [T, H, d] fp32 (per key channel)
    beta: torch.Tensor        # [T, H] fp32
    cu_seqlens: torch.Tensor  # [n+1] int32
    H: int
    d: int
    scale: float
    chunk: int


def kda_varlen_config(seed: int = 0, n_seqs: int = 8, H: int = 32, d: int = 128,
                      lo: int = 1024, hi: int = 8192, chunk: int = 64) -> KdaVarlenInputs:
    """KDA-style varlen prefill: 8 sequences with lengths uniform in [1024, 8192], H=32,
    d=128, raw q|k|v ~ randn in bf16 concatenated along channels, causal conv weights
    randn/2 (width 4, no bias), per-key gate logsigmoid(randn + 3), beta = sigmoid(randn);
    q, k are L2-normalised inside the kernel after the convolution."""
    gen = _gen(seed)
    lengths = torch.randint(lo, hi + 1, (n_seqs,), generator=gen)
    T = int(lengths.sum())
    cu = torch.zeros(n_seqs + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lengths, 0).to(torch.int32)
    HD = H * d
    q = torch.randn(T, HD, generator=gen).to(BF16)
    k = torch.randn(T, HD, generator=gen).to(BF16)
    v = torch.randn(T, HD, generator=gen).to(BF16)
    w = torch.randn(3 * HD, 4, generator=gen) / 2
    a = torch.randn(T, H, d, generator=gen)
    b = torch.randn(T, H, generator=gen)
    return KdaVarlenInputs(
        x=torch.cat([q, k, v], dim=1).contiguous(), conv_w=w.contiguous(),
        g=gate_from_normal(a).contiguous(), beta=beta_from_normal(b).contiguous(),
        cu_seqlens=cu, H=H, d=d, scale=1.0 / d ** 0.5, chunk=chunk)
