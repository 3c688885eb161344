"""Helpers for the GPU parity tests: device upload of the seeded workloads'
bit arrays, guard-banded output buffers, and the comparison rules.

Comparison rules (the tolerances of the path, applied element by element):
- FP8 codes: signed e4m3 ordinals may differ by at most one step, on at most
  0.1 % of the elements of a tensor (exact e4m3 ties, where the kernel's fp32
  y and the oracle's fp64 y can fall on either side); everything else equal.
- producer output y (fp32): per row, ||y_gpu - y_ref||_inf / ||y_ref||_inf
  <= 1e-5 (an elementwise relative bound is ill-posed where the modulation
  cancels the normalised value).
- residual write-back, gate echo, packed weights and scales: bit-exact.
- GEMM from identical FP8 operands: fp32 outputs within 1e-3 * max|ref| of
  the exact oracle; bf16 outputs within one bf16 ulp plus that tolerance.
  (The matrix cores' fp32 accumulation is not exact: on random codes that
  span the whole e4m3 range it reaches ~1e-4 * max|ref|, an order of
  magnitude inside the bound.)
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import codecs

GUARD = 4096          # guard elements on each side of an output
GUARD_BYTE = 0x5A


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.cuda().view(torch.bfloat16)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def scalar(v) -> torch.Tensor:
    return torch.tensor([float(np.float32(v))], dtype=torch.float32, device="cuda")


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.uint8).cpu().numpy()


class Guarded:
    """A [rows, cols] output with row stride `ld`, surrounded by guard bytes
    so that any write outside the logical region is detected."""

    def __init__(self, rows, cols, dtype, ld=None):
        self.rows, self.cols = rows, cols
        self.ld = cols if ld is None else ld
        esz = torch.tensor([], dtype=dtype).element_size()
        n = (rows - 1) * self.ld + cols if rows > 0 else 0
        total = n + 2 * GUARD
        self.raw = torch.full((total * esz,), GUARD_BYTE, dtype=torch.uint8,
                              device="cuda")
        flat = self.raw.view(dtype)
        self.view = flat[GUARD:GUARD + max(n, 0)].as_strided(
            (rows, cols), (self.ld, 1)) if rows > 0 else flat[GUARD:GUARD].view(0, cols)
        self.dtype = dtype
        self.esz = esz

    def check_guards(self):
        raw = self.raw.cpu().numpy()
        g = GUARD * self.esz
        assert (raw[:g] == GUARD_BYTE).all(), "write before the output region"
        assert (raw[-g:] == GUARD_BYTE).all(), "write after the output region"
        if self.ld > self.cols and self.rows > 1:
            body = raw[g:-g].reshape(-1)
            n = (self.rows - 1) * self.ld + self.cols
            idx = np.arange(n)
            gap = (idx % self.ld) >= self.cols
            gb = body.reshape(n, self.esz)[gap]
            assert (gb == GUARD_BYTE).all(), "write into the row-stride gap"


def assert_codes_close(got: np.ndarray, ref: np.ndarray, what=""):
    assert got.shape == ref.shape
    d = np.abs(codecs.e4m3_ordinal(got) - codecs.e4m3_ordinal(ref))
    nbad = int((d > 0).sum())
    assert d.max(initial=0) <= 1, f"{what}: code off by {d.max()} steps"
    assert nbad <= 0.001 * d.size, f"{what}: {nbad} of {d.size} codes differ"
    return nbad


def assert_rows_close(y: np.ndarray, ref: np.ndarray, tol=1e-5, what=""):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(y - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    rel = num / np.where(den > 0, den, 1.0)
    assert rel.max(initial=0) <= tol, f"{what}: row rel err {rel.max():.3e}"
    return float(rel.max(initial=0))


def assert_codes_quantise_own_y(codes: np.ndarray, y: np.ndarray, s: float):
    """Property: the kernel's codes are the round-to-nearest-even e4m3 of
    clamp(fl32(y / s)) for its own fp32 y (torch's CPU cast as the codec)."""
    q = (torch.from_numpy(np.asarray(y, np.float32)) /
         torch.tensor(np.float32(s))).clamp(-448, 448)
    want = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # +0 / -0 are the same value
    same = (codes == want) | (((codes & 0x7F) == 0) & ((want & 0x7F) == 0))
    assert same.all(), f"{(~same).sum()} codes are not the quantised y"


def assert_gemm_f32(got: np.ndarray, ref: np.ndarray, what=""):
    got = np.asarray(got, np.float64)
    scale = np.max(np.abs(ref)) if ref.size else 1.0
    err = np.max(np.abs(got - ref)) if ref.size else 0.0
    assert err <= 1e-3 * scale, f"{what}: max|d| {err:.3e} > 1e-3 * {scale:.3e}"
    return err / scale if scale else 0.0


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** -126)))
    return 2.0 ** (np.maximum(e, -126) - 7)


def assert_gemm_bf16(got_bits: np.ndarray, ref: np.ndarray, what="",
                     scale=None):
    """bf16 output: one bf16 rounding of a value that is itself within the
    GEMM tolerance (1e-3 * max|ref|) of the exact result, so element by
    element |out - ref| <= ulp_bf16(ref) + 1e-3 * max|ref|."""
    got = codecs.bf16_to_f32(got_bits).astype(np.float64)
    ref = np.asarray(ref, np.float64)
    if scale is None:
        scale = np.max(np.abs(ref)) if ref.size else 0.0
    bound = bf16_ulp(ref) + 1e-3 * scale
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} bf16 outputs beyond one ulp; "
                           f"worst {err[bad].max():.3e} at |ref| {np.abs(ref[bad]).max():.3e}")


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between two bf16 bit arrays (same sign order)."""
    def ordv(b):
        b = b.astype(np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(ordv(a_bits) - ordv(b_bits))
