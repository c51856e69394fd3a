"""Test helpers: golden-file parsing, bf16/e4m3 views through torch (a library independent of
both the oracle and libpuro), and the GEMM acceptance rule."""
from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def parse_float(tok: str) -> float:
    tok = tok.strip()
    if "0x" in tok or "0X" in tok:
        return float.fromhex(tok)
    return float(tok)


def read_e4m3_hand():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_hand.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((parse_float(parts[0]), int(parts[1], 16), " ".join(parts[2:])))
    return rows


def read_quant_hand(name: str = "quant_hand.txt"):
    cases, cur = [], None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest, "values": {}, "codes": {}}
                cases.append(cur)
            elif key == "values":
                for item in rest.split():
                    i, v = item.split(":")
                    cur["values"][int(i)] = parse_float(v)
            elif key == "scale":
                cur["scale"] = parse_float(rest)
            elif key == "codes":
                for item in rest.split():
                    i, c = item.split(":")
                    cur["codes"][int(i)] = int(c, 16)
    return cases


def f32_to_bf16_bits(vals) -> np.ndarray:
    """Exact fp32 values -> bf16 bit patterns (the values must be bf16-representable)."""
    t = torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16)
    back = t.float().numpy()
    assert np.array_equal(back.view(np.uint32), np.asarray(vals, np.float32).view(np.uint32))
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def torch_e4m3_decode(codes) -> np.ndarray:
    """E4M3 bytes -> float64 via torch.float8_e4m3fn."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_e4m3_encode(vals) -> np.ndarray:
    """fp32 values (|v| <= 448) -> E4M3 bytes via torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_np(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def gemm_tolerance_violations(gpu: np.ndarray, ref: np.ndarray, rms_ref: float | None = None):
    """Acceptance: |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref), elementwise. Returns the number
    of violating elements and the worst ratio err / bound."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if rms_ref is None:
        rms_ref = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = 2.0 ** -7 * np.abs(ref) + 1e-3 * rms_ref
    err = np.abs(gpu - ref)
    bad = err > bound
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if ref.size else 0.0
    return int(bad.sum()), worst
