"""Seeded synthetic inputs for the Gated DeltaNet token mixer.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the HIP path's tests and the CPU oracle can be fed
from it.  Every tensor is a CPU torch tensor; bf16 tensors are rounded from
float32 with round-to-nearest-even (torch's conversion).

Workloads (shapes follow the 0.8B hybrid model's linear-attention layer in
"7.6 Qwen3.5: the linear-attention hybrid", section 7.6.1: 16 key heads,
16 value heads, head dims 128, conv kernel 4):

  tiny_f32   T=64, H=2, dk=dv=16, fp32 core-only inputs
  layer_4k   T=4096, 16/16 heads, 128x128, bf16 pre-conv x (conv_dim 6144)
  varlen8    8 sequences with lengths ~U{512..8192} packed by cu_seqlens,
             random fp32 initial states N(0, 0.1) and conv caches N(0, 1)
  decode256  B=256 single-token rows, fp32 state N(0, 0.1), conv cache N(0, 1)
  long_64k   T=65536, 16 key heads / 32 value heads (2 value heads per key head)

Distributions: x ~ N(0,1); conv weights ~ N(0, 0.5) (second parameter is the
standard deviation); beta = sigmoid(N(0,1)); log-decay g = -softplus(N(0,1)),
or g = log(a) with a ~ U(0.9, 1.0) where the workload says so.  Gated RMSNorm
epilogue: gate z ~ N(0, 1), per-channel gain gamma = 1 + N(0, 0.1); standalone
norm rows y ~ N(0, 1) times a per-row scale 10^U(-3, 2).
Layer forward (input projection -> core -> gated RMSNorm -> output projection, at the
0.8B layer widths of section 7.6.1: hidden 1024): hidden ~ N(0, 1); input projection
weight ~ N(0, 1/E) and output projection weight ~ N(0, 1/(Hv dv)), so every projected
value is ~N(0, 1) like the pre-conv x and the gate pre-activations of the core
workloads; conv weights, gain and caches as above (the layer's conv caches in fp32).
Generator: numpy PCG64(1234 + index).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

WORKLOADS = ["tiny_f32", "layer_4k", "varlen8", "decode256", "long_64k"]
SEED_BASE = 1234
_BLOCK_ROWS = 4096


def _rng(index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(SEED_BASE + index))


def _normal_f32(rng, shape, std=1.0):
    """N(0, std^2) draws in float32, generated in row blocks (same stream as one draw)."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(shape[0], int(np.prod(shape[1:]))) if len(shape) > 1 else out.reshape(-1, 1)
    for r0 in range(0, flat.shape[0], _BLOCK_ROWS):
        r1 = min(r0 + _BLOCK_ROWS, flat.shape[0])
        flat[r0:r1] = rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def _sigmoid_normal(rng, shape):
    z = rng.standard_normal(shape)
    return 1.0 / (1.0 + np.exp(-z))


def _neg_softplus_normal(rng, shape):
    z = rng.standard_normal(shape)
    return -np.logaddexp(0.0, z)


def _log_uniform_decay(rng, shape, lo=0.9, hi=1.0):
    a = rng.uniform(lo, hi, shape)
    return np.log(a)


def _unit_rows(rng, shape):
    """Gaussian vectors scaled to unit length along the last axis (uniform on the sphere)."""
    z = rng.standard_normal(shape)
    return z / np.linalg.norm(z, axis=-1, keepdims=True)


@dataclass
class Workload:
    name: str
    T: int
    N: int
    Hk: int
    Hv: int
    dk: int
    dv: int
    dtype: str                      # "bf16" or "f32": element type of x / conv weights / conv caches
    cu_seqlens: torch.Tensor        # int32 [N+1]
    g: torch.Tensor                 # fp32 [T, Hv] (decode: [B, Hv])
    beta: torch.Tensor              # fp32 [T, Hv]
    x: torch.Tensor | None = None   # [T, conv_dim] pre-conv input
    conv_w: torch.Tensor | None = None
    conv_state: torch.Tensor | None = None    # [N, 3, conv_dim] or None (zeros)
    state: torch.Tensor | None = None         # fp32 [N, Hv, dk, dv] or None (zeros)
    q: torch.Tensor | None = None   # core-only inputs (already normalised)
    k: torch.Tensor | None = None
    v: torch.Tensor | None = None
    scale: float = 1.0
    decode: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def conv_dim(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv


def _cu(lengths) -> torch.Tensor:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return torch.from_numpy(cu.astype(np.int32))


def tiny_f32() -> Workload:
    rng = _rng(0)
    T, H, d = 64, 2, 16
    q = _unit_rows(rng, (T, H, d))
    k = _unit_rows(rng, (T, H, d))
    v = rng.standard_normal((T, H, d))
    beta = _sigmoid_normal(rng, (T, H))
    g = _log_uniform_decay(rng, (T, H))
    return Workload("tiny_f32", T, 1, H, H, d, d, "f32", _cu([T]), _f32(g), _f32(beta),
                    q=_f32(q), k=_f32(k), v=_f32(v))


def prefill_workload(name: str, index: int, lengths, Hk: int, Hv: int, d: int = 128,
                     random_states: bool = False, decay: str = "softplus") -> Workload:
    """bf16 pre-conv prefill workload with the given sequence lengths."""
    rng = _rng(index)
    lengths = [int(x) for x in lengths]
    T = int(sum(lengths))
    N = len(lengths)
    C = 2 * Hk * d + Hv * d
    x = _normal_f32(rng, (T, C))
    w = _normal_f32(rng, (C, 4), std=0.5)
    beta = _sigmoid_normal(rng, (T, Hv))
    g = _neg_softplus_normal(rng, (T, Hv)) if decay == "softplus" else _log_uniform_decay(rng, (T, Hv), 0.99, 1.0)
    wl = Workload(name, T, N, Hk, Hv, d, d, "bf16", _cu(lengths), _f32(g), _f32(beta),
                  x=_bf16(x), conv_w=_bf16(w))
    if random_states:
        wl.state = _f32(_normal_f32(rng, (N, Hv, d, d), std=0.1))
        wl.conv_state = _bf16(_normal_f32(rng, (N, 3, C)))
    return wl


def layer_4k() -> Workload:
    return prefill_workload("layer_4k", 1, [4096], 16, 16)


def varlen8_lengths() -> list[int]:
    rng = _rng(2)
    return [int(x) for x in rng.integers(512, 8192, size=8, endpoint=True)]


def varlen8() -> Workload:
    lengths = varlen8_lengths()
    # the lengths consume the head of stream 2; the tensors use a fresh stream of
    # the same seed offset by 100 so that T does not shift the tensor draws
    wl = prefill_workload("varlen8", 102, lengths, 16, 16, random_states=True)
    wl.meta["lengths"] = lengths
    return wl


def decode_workload(name: str, index: int, B: int, Hk: int, Hv: int, d: int = 128) -> Workload:
    rng = _rng(index)
    C = 2 * Hk * d + Hv * d
    x = _normal_f32(rng, (B, C))
    w = _normal_f32(rng, (C, 4), std=0.5)
    g = _log_uniform_decay(rng, (B, Hv))
    beta = _sigmoid_normal(rng, (B, Hv))
    state = _normal_f32(rng, (B, Hv, d, d), std=0.1)
    cs = _normal_f32(rng, (B, 3, C))
    return Workload(name, B, B, Hk, Hv, d, d, "bf16", _cu([1] * B), _f32(g), _f32(beta),
                    x=_bf16(x), conv_w=_bf16(w), conv_state=_bf16(cs), state=_f32(state), decode=True)


def decode256() -> Workload:
    return decode_workload("decode256", 3, 256, 16, 16)


def long_64k() -> Workload:
    return prefill_workload("long_64k", 4, [65536], 16, 32)


def core_workload(name: str, index: int, lengths, Hk: int, Hv: int, dk: int, dv: int,
                  random_states: bool = False, decay: str = "softplus", scale: float = 1.0) -> Workload:
    """Core-only fp32 inputs (unit-norm q, k; v ~ N(0,1)) for the chunked prefill."""
    rng = _rng(index)
    lengths = [int(x) for x in lengths]
    T = int(sum(lengths))
    N = len(lengths)
    q = _unit_rows(rng, (T, Hk, dk))
    k = _unit_rows(rng, (T, Hk, dk))
    v = rng.standard_normal((T, Hv, dv))
    beta = _sigmoid_normal(rng, (T, Hv))
    if decay == "softplus":
        g = _neg_softplus_normal(rng, (T, Hv))
    elif decay == "slow":
        g = _log_uniform_decay(rng, (T, Hv), 0.99, 1.0)
    else:
        g = _log_uniform_decay(rng, (T, Hv))
    wl = Workload(name, T, N, Hk, Hv, dk, dv, "f32", _cu(lengths), _f32(g), _f32(beta),
                  q=_f32(q), k=_f32(k), v=_f32(v), scale=scale)
    if random_states:
        wl.state = _f32(_normal_f32(rng, (N, Hv, dk, dv), std=0.1))
    return wl


def get(name: str) -> Workload:
    return {"tiny_f32": tiny_f32, "layer_4k": layer_4k, "varlen8": varlen8,
            "decode256": decode256, "long_64k": long_64k}[name]()


def gate_inputs(index: int, shape, dv: int, dtype: str = "bf16"):
    """Gate z ~ N(0, 1) of `shape` (last axis dv) and gain gamma = 1 + N(0, 0.1) [dv] for
    the gated RMSNorm epilogue, in the element type ("bf16" or "f32")."""
    rng = _rng(index)
    z = _normal_f32(rng, tuple(shape))
    gamma = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    cast = _bf16 if dtype == "bf16" else _f32
    return cast(z), cast(gamma)


def norm_rows(index: int, rows: int, dv: int) -> torch.Tensor:
    """fp32 rows [rows, dv] ~ N(0, 1) times a per-row scale 10^U(-3, 2)."""
    rng = _rng(index)
    y = rng.standard_normal((rows, dv)) * (10.0 ** rng.uniform(-3.0, 2.0, (rows, 1)))
    return _f32(y)


@dataclass
class LayerWeights:
    """bf16 weights of one linear-attention layer (stored as a linear layer stores them)."""
    w_in: torch.Tensor      # [conv_dim + Hv dv + 2 Hv, E]: rows q|k|v, z, a, b
    conv_w: torch.Tensor    # [conv_dim, 4]
    gamma: torch.Tensor     # [dv], the gain as applied
    w_out: torch.Tensor     # [E, Hv dv]


def _on_grid(a: np.ndarray, step: float, bound: float) -> np.ndarray:
    """Draws moved to the nearest multiple of `step` and clipped to [-bound, bound]."""
    return (np.clip(np.rint(a / step), -bound / step, bound / step) * step).astype(np.float32)


def layer_weights(index: int, E: int, Hk: int, Hv: int, dk: int, dv: int, exact: bool = False) -> LayerWeights:
    """exact: the input projection weight on multiples of 2^-6 in [-1/2, 1/2] (see
    layer_hidden), so that with a grid input every projected value is exact in fp32."""
    rng = _rng(index)
    C = 2 * Hk * dk + Hv * dv
    w_in = _normal_f32(rng, (C + Hv * dv + 2 * Hv, E), std=1.0 / np.sqrt(E))
    if exact:
        w_in = _on_grid(w_in, 2.0 ** -6, 0.5)
    conv_w = _normal_f32(rng, (C, 4), std=0.5)
    gamma = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    w_out = _normal_f32(rng, (E, Hv * dv), std=1.0 / np.sqrt(Hv * dv))
    return LayerWeights(_bf16(w_in), _bf16(conv_w), _bf16(gamma), _bf16(w_out))


def layer_hidden(index: int, T: int, E: int, exact: bool = False) -> torch.Tensor:
    """Layer input rows [T, E] ~ N(0, 1), bf16.  exact: on multiples of 1/8 in [-4, 4].
    With a grid weight every product is a multiple of 2^-9 of size <= 2 and every partial
    sum over E <= 2^13 terms stays below 2^14 in size, i.e. within 23 significant bits:
    any summation order in fp32 gives the exact value, so its bf16 rounding is one
    decision, whoever computes it."""
    h = _normal_f32(_rng(index), (T, E))
    return _bf16(_on_grid(h, 0.125, 4.0) if exact else h)


def layer_caches(index: int, N: int, Hk: int, Hv: int, dk: int, dv: int):
    """Incoming conv caches [N, 3, conv_dim] ~ N(0, 1) and states [N, Hv, dk, dv] ~
    N(0, 0.1), both fp32 (the layer keeps its pre-conv inputs in fp32)."""
    rng = _rng(index)
    C = 2 * Hk * dk + Hv * dv
    cs = _normal_f32(rng, (N, 3, C))
    st = _normal_f32(rng, (N, Hv, dk, dv), std=0.1)
    return _f32(cs), _f32(st)
