"""Counter-based SplitMix64 generator.

Element ``i`` of stream ``(seed, tensor_id)`` is a pure function of those three
integers, so any slice of any tensor can be regenerated on any device without
generating what comes before it.

Definition (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014 — the SplitMix64 finaliser):

    mix(z):  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
             z ^= z >> 27; z *= 0x94D049BB133111EB;
             z ^= z >> 31                                 (all mod 2**64)
    key(seed, tid) = mix((seed mod 2**32) << 32 | (tid mod 2**32))
    bits(i)        = mix(key + (i + 1) * 0x9E3779B97F4A7C15)
    uniform(i)     = (bits(i) >> 11) * 2**-53                 in [0, 1)
    normal(i)      = sqrt(-2 ln(1 - uniform(2i))) * cos(2 pi uniform(2i+1))

Normals are fp64, rounded once to fp32 and then once to bf16, both
round-to-nearest-even (torch's conversions).

Tensors are torch int64 tensors carrying the 64-bit patterns in two's
complement; add and multiply wrap mod 2**64 and right shifts are made logical
with a mask.  ``tests/test_synth.py`` checks this against exact Python
integers.
"""
from __future__ import annotations

import math

import torch

GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1
CHUNK = 1 << 24


def _s64(c: int) -> int:
    c &= MASK64
    return c - (1 << 64) if c >= (1 << 63) else c


def mix64_int(z: int) -> int:
    """The SplitMix64 finaliser on an exact Python integer."""
    z &= MASK64
    z ^= z >> 30
    z = (z * M1) & MASK64
    z ^= z >> 27
    z = (z * M2) & MASK64
    z ^= z >> 31
    return z


def stream_key(seed: int, tensor_id: int) -> int:
    return mix64_int(((seed & 0xFFFFFFFF) << 32) | (tensor_id & 0xFFFFFFFF))


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = z ^ _srl(z, 30)
    z = z * _s64(M1)
    z = z ^ _srl(z, 27)
    z = z * _s64(M2)
    return z ^ _srl(z, 31)


def bits64(seed: int, tensor_id: int, start: int, n: int, device="cpu") -> torch.Tensor:
    """Raw 64-bit draws for counters start .. start+n-1, as int64 bit patterns."""
    key = _s64(stream_key(seed, tensor_id))
    idx = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix(idx * _s64(GAMMA) + key)


def _uniform_chunk(seed, tid, start, n, device):
    b = bits64(seed, tid, start, n, device)
    return _srl(b, 11).to(torch.float64) * (2.0 ** -53)


def uniform(seed: int, tensor_id: int, n: int, device="cpu", lo=0.0, hi=1.0, start: int = 0) -> torch.Tensor:
    """fp64 uniforms on [lo, hi) for counters start .. start+n-1."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        out[s:s + m] = _uniform_chunk(seed, tensor_id, start + s, m, device)
    if lo != 0.0 or hi != 1.0:
        out = lo + (hi - lo) * out
    return out


def _normal_chunk(seed, tid, start, n, device):
    u = _uniform_chunk(seed, tid, 2 * start, 2 * n, device).view(n, 2)
    r = torch.sqrt(-2.0 * torch.log1p(-u[:, 0]))
    return r * torch.cos((2.0 * math.pi) * u[:, 1])


def normal(seed: int, tensor_id: int, n: int, device="cpu", dtype=torch.float32, start: int = 0) -> torch.Tensor:
    """N(0,1) draws for counters start .. start+n-1, fp64 rounded to ``dtype`` (fp32 or fp64)."""
    out = torch.empty(n, dtype=dtype, device=device)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        out[s:s + m] = _normal_chunk(seed, tensor_id, start + s, m, device).to(dtype)
    return out


def normal_bf16(seed: int, tensor_id: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """N(0,1) draws for counters start .. start+n-1, rounded fp64 -> fp32 -> bf16 (RNE each time)."""
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        out[s:s + m] = _normal_chunk(seed, tensor_id, start + s, m, device).to(torch.float32).to(torch.bfloat16)
    return out


def permutation(seed: int, tensor_id: int, n: int) -> torch.Tensor:
    """A random permutation of 0..n-1 (argsort of n distinct 64-bit draws), int64 on the CPU."""
    b = bits64(seed, tensor_id, 0, n, "cpu")
    return torch.argsort(b, stable=True)
