"""Seeded synthetic inputs shared by the tests, the oracle checks and the benchmark.

This module holds no arithmetic of the sparse-attention method.  It only turns
(seed, stream, element index) into numbers:

* ``splitmix64`` -- the counter-based mixer published by Steele, Lea and Flood
  ("Fast splittable pseudorandom number generators", OOPSLA 2014): the state
  advances by the golden-ratio increment 0x9E3779B97F4A7C15 and every output is
  the state passed through two xor-shift-multiply rounds.
* standard normals by the Box-Muller transform (one cosine output per pair of
  uniforms), evaluated in float64 and rounded once to float32;
* the logistic sigmoid of such normals for the importance scores and gates.

Element ``i`` of a stream depends only on ``(seed, stream, i)``, so any slice of
a large tensor can be regenerated on its own, on the CPU or on a GPU, with
identical bits (all integer steps are exact; the float steps are done in
float64 and rounded to float32, then optionally to bfloat16 round-to-nearest-
even by ``torch.Tensor.to``).
"""
from __future__ import annotations

import math

import torch

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _signed(v: int) -> int:
    v &= _MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def _mix_int(z: int) -> int:
    """splitmix64 output function on a Python int (mod 2**64)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def stream_base(seed: int, stream: int) -> int:
    """Starting state of one named stream of one seed (a plain Python int)."""
    return _mix_int(_mix_int(seed) + (stream + 1) * _GAMMA)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    # logical shift right on int64 two's-complement storage
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix_tensor(z: torch.Tensor) -> torch.Tensor:
    z = z ^ _lsr(z, 30)
    z = z * _signed(_M1)
    z = z ^ _lsr(z, 27)
    z = z * _signed(_M2)
    return z ^ _lsr(z, 31)


def u64_at(seed: int, stream: int, counters: torch.Tensor) -> torch.Tensor:
    """splitmix64 outputs (int64 storage of the uint64 value) at the counters."""
    base = _signed(stream_base(seed, stream))
    z = base + (counters.to(torch.int64) + 1) * _signed(_GAMMA)
    return _mix_tensor(z)


def u64_py(seed: int, stream: int, i: int) -> int:
    """Same value as ``u64_at`` for one counter, as an unsigned Python int."""
    return _mix_int(stream_base(seed, stream) + (i + 1) * _GAMMA)


_CHUNK = 1 << 24


def _normal_flat(seed: int, stream: int, start: int, n: int, device) -> torch.Tensor:
    out = torch.empty(n, dtype=torch.float32, device=device)
    two_m53 = 2.0 ** -53
    for off in range(0, n, _CHUNK):
        m = min(_CHUNK, n - off)
        idx = torch.arange(start + off, start + off + m, dtype=torch.int64, device=device)
        a = _lsr(u64_at(seed, stream, 2 * idx), 11).to(torch.float64)
        b = _lsr(u64_at(seed, stream, 2 * idx + 1), 11).to(torch.float64)
        u1 = (a + 1.0) * two_m53            # (0, 1]
        u2 = b * two_m53                    # [0, 1)
        z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
        out[off:off + m] = z.to(torch.float32)
    return out


def normal(seed: int, stream: int, shape, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """N(0,1) tensor of ``shape``; float32 values, then rounded to ``dtype``."""
    n = 1
    for s in shape:
        n *= int(s)
    z = _normal_flat(seed, stream, 0, n, device).reshape(tuple(int(s) for s in shape))
    return z if dtype == torch.float32 else z.to(dtype)


def sigmoid_normal(seed: int, stream: int, shape, device="cpu") -> torch.Tensor:
    """sigmoid(N(0,1)) in float32 (the logistic function evaluated in float64)."""
    z = normal(seed, stream, shape, device).to(torch.float64)
    return (1.0 / (1.0 + torch.exp(-z))).to(torch.float32)


def uniform_ints(seed: int, stream: int, n: int, lo: int, hi: int) -> list[int]:
    """``n`` integers uniform in [lo, hi] (64-bit draw modulo the range size)."""
    span = hi - lo + 1
    return [lo + u64_py(seed, stream, i) % span for i in range(n)]


def random_keys(seed: int, stream: int, shape, device="cpu") -> torch.Tensor:
    """Non-negative int64 sort keys (top 63 bits of the splitmix64 output)."""
    n = 1
    for s in shape:
        n *= int(s)
    idx = torch.arange(n, dtype=torch.int64, device=device)
    return _lsr(u64_at(seed, stream, idx), 1).reshape(tuple(int(s) for s in shape))
