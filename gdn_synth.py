"""Seeded synthetic inputs for the Gated DeltaNet layer.

This module only draws random inputs and converts between float32 and bfloat16
bit patterns.  It holds none of the layer's arithmetic: the oracle (``oracle/``)
and the HIP library both receive exactly the arrays produced here.

Shapes follow the Qwen3-Next linear-attention configuration printed on the
model-atlas page for Qwen3-Coder-Next (raw config.json table:
``linear_num_key_heads`` 16, ``linear_num_value_heads`` 32, key/value head dim
128, ``linear_conv_kernel_dim`` 4).  Value distributions follow the stated
workload recipes: q, k, v, z ~ N(0, 1); beta = sigmoid(N(0, 1));
g = -softplus(N(0, 1)) (log-decay); conv weights ~ N(0, 0.5);
norm weight = 1 + N(0, 0.02); seeded states ~ N(0, 0.01).  The second argument
of N(., .) is read as the standard deviation.

Layouts (row-major, last index contiguous):
  q, k            [T_total, Hk, dk]        io dtype
  v, z            [T_total, Hv, dv]        io dtype
  g, beta         [T_total, Hv]            float32
  conv_w          [Cch, K]                 io dtype, Cch = 2*Hk*dk + Hv*dv,
                                           channels ordered q | k | v
  norm_w          [dv]                     io dtype
  state           [N, Hv, dv, dk]          float32 (or bf16 for decode)
  conv_state      [N, K-1, Cch]            io dtype, oldest token first
  cu_seqlens      [N+1]                    int32
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

BF16 = "bf16"
F32 = "f32"


# --------------------------------------------------------------------------
# bfloat16 bit conversions (round to nearest, ties to even)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, returned as uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # NaN stays NaN (quiet bit set); finite values round to nearest even.
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of an io-dtype array to float64."""
    if dtype == BF16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == BF16 else np.ascontiguousarray(x32, np.float32)


def _normal(rng: np.random.Generator, shape, std: float = 1.0, block: int = 1 << 24):
    """float32 normal draws, produced in blocks to bound host temporaries."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, block):
        e = min(n, s + block)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32) * np.float32(std)
    return out.reshape(shape)


def _normal_io(rng, shape, std, dtype, block: int = 1 << 24):
    """Normal draws stored directly in the io dtype, block by block."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    for s in range(0, n, block):
        e = min(n, s + block)
        x = rng.standard_normal(e - s, dtype=np.float32) * np.float32(std)
        out[s:e] = f32_to_bf16_bits(x) if dtype == BF16 else x
    return out.reshape(shape)


# --------------------------------------------------------------------------
# Problem description
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Problem:
    """One synthetic layer invocation (prefill or decode)."""
    name: str
    seq_lens: Sequence[int]
    Hk: int = 16
    Hv: int = 32
    dk: int = 128
    dv: int = 128
    K: int = 4
    io: str = BF16
    state_dtype: str = F32
    conv: bool = True
    gate: bool = True
    l2norm: bool = True
    prenormalize_qk: bool = False   # input recipe: q, k L2-normalised by the generator
    init_state_std: Optional[float] = None   # None: zero initial state
    conv_state_std: Optional[float] = None   # None: zero conv state
    g_scale: float = 1.0            # g = -g_scale * softplus(N(0,1)); 0 gives a = 1
    beta_fixed: Optional[float] = None       # override beta with a constant
    scale: float = 1.0
    l2_eps: float = 1e-6
    norm_eps: float = 1e-6
    seed: int = 0
    decode: bool = False

    @property
    def N(self) -> int:
        return len(self.seq_lens)

    @property
    def T(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def Cch(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv


def configs() -> dict:
    """The five workloads of the layer (seed = 1000 + index)."""
    c = {}
    c["C0"] = Problem("C0 fp32 T=512 1 head", [512], Hk=1, Hv=1, io=F32, conv=False,
                      gate=False, l2norm=False, prenormalize_qk=True, seed=1000)
    c["C1"] = Problem("C1 prefill T=4096 16k/32v", [4096], seed=1001)
    c["C2"] = Problem("C2 prefill T=65536", [65536], init_state_std=0.01,
                      conv_state_std=0.01, seed=1002)
    rng = np.random.default_rng(1003 + 7919)
    lens = rng.integers(512, 8192, size=16, endpoint=True).tolist()
    c["C3"] = Problem("C3 varlen 16 seqs", lens, init_state_std=0.01, seed=1003)
    c["C4"] = Problem("C4 decode 256 seqs fp32 state", [1] * 256, init_state_std=0.01,
                      conv_state_std=0.01, seed=1004, decode=True)
    c["C4b"] = dataclasses.replace(c["C4"], name="C4b decode 256 seqs bf16 state",
                                   state_dtype=BF16)
    return c


def serving() -> dict:
    """Stand-ins for the serving benchmark of the SGLang cookbook's Qwen3-Next
    page (ShareGPT prompts of about 300 tokens on average, about 93 requests in
    flight; the dataset itself is not used): a prefill of 93 new prompts packed
    with cu_seqlens, lengths uniform in [250, 350], zero initial states; and a
    decode step of 93 sequences against seeded fp32 states."""
    rng = np.random.default_rng(2001 + 7919)
    lens = rng.integers(250, 350, size=93, endpoint=True).tolist()
    return {"prefill": Problem("serving prefill, 93 prompts of 250-350 tokens", lens, seed=2001),
            "decode": Problem("serving decode, 93 sequences, fp32 state", [1] * 93, init_state_std=0.01,
                              conv_state_std=0.01, seed=2002, decode=True)}


def generate(p: Problem) -> dict:
    """Draw every input of problem ``p``; fixed draw order per seed."""
    rng = np.random.default_rng(p.seed)
    T, N = p.T, p.N
    d = {}
    if p.prenormalize_qk:
        for name in ("q", "k"):
            x = _normal(rng, (T, p.Hk, p.dk))
            x /= np.sqrt((x.astype(np.float64) ** 2).sum(-1, keepdims=True)).astype(np.float32)
            d[name] = _store(x, p.io)
    else:
        d["q"] = _normal_io(rng, (T, p.Hk, p.dk), 1.0, p.io)
        d["k"] = _normal_io(rng, (T, p.Hk, p.dk), 1.0, p.io)
    d["v"] = _normal_io(rng, (T, p.Hv, p.dv), 1.0, p.io)
    z = _normal_io(rng, (T, p.Hv, p.dv), 1.0, p.io)
    graw = _normal(rng, (T, p.Hv))
    # softplus(x) = log(1 + e^x), evaluated stably
    sp = np.maximum(graw, 0) + np.log1p(np.exp(-np.abs(graw)))
    d["g"] = (-np.float32(p.g_scale) * sp).astype(np.float32)
    braw = _normal(rng, (T, p.Hv))
    beta = (1.0 / (1.0 + np.exp(-braw.astype(np.float64)))).astype(np.float32)
    if p.beta_fixed is not None:
        beta[:] = np.float32(p.beta_fixed)
    d["beta"] = beta
    conv_w = _normal_io(rng, (p.Cch, p.K), 0.5, p.io)
    norm_w = _store((1.0 + _normal(rng, (p.dv,), 0.02)).astype(np.float32), p.io)
    d["z"] = z if p.gate else None
    d["norm_w"] = norm_w if p.gate else None
    d["conv_w"] = conv_w if p.conv else None
    if p.init_state_std is not None:
        st = _normal(rng, (N, p.Hv, p.dv, p.dk), p.init_state_std)
        d["state"] = f32_to_bf16_bits(st) if p.state_dtype == BF16 else st
    else:
        d["state"] = None
    if p.conv_state_std is not None:
        d["conv_state"] = _normal_io(rng, (N, p.K - 1, p.Cch), p.conv_state_std, p.io)
    else:
        d["conv_state"] = None
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(p.seq_lens, dtype=np.int64))
    d["cu_seqlens"] = cu
    return d


def orthonormal_rows(rng: np.random.Generator, n: int, d: int) -> np.ndarray:
    """n <= d orthonormal rows of length d (QR of a Gaussian matrix)."""
    a = rng.standard_normal((d, d))
    qm, _ = np.linalg.qr(a)
    return qm[:n].copy()
