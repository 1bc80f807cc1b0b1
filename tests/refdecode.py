"""Independent decoders used only to pin the oracle.

They reach the same values by other routes than the oracle's C code:
E4M3FN through torch's float8_e4m3fn cast, bf16 through torch's bfloat16
cast, E2M1 through the OCP MX table stored in tests/golden/, nibble unpacking
through vectorised numpy.
"""
import os

import numpy as np
import torch

_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_table() -> np.ndarray:
    vals = np.zeros(16, np.float64)
    with open(os.path.join(_GOLDEN, "ocp_e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def e4m3_table() -> np.ndarray:
    b = torch.arange(256, dtype=torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_to_f64(bits) -> np.ndarray:
    t = torch.as_tensor(np.asarray(bits).astype(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def f32_to_bf16_bits(f32) -> np.ndarray:
    t = torch.as_tensor(np.asarray(f32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def _np(t):
    if hasattr(t, "detach"):
        return t.detach().cpu().numpy()
    return np.asarray(t)


def dequant(mat, e: int) -> np.ndarray:
    q = _np(mat["q"])[e].astype(np.uint8)
    s = _np(mat["s"])[e].astype(np.uint8)
    ts = float(_np(mat["ts"])[e])
    rows, half = q.shape
    codes = np.empty((rows, half * 2), np.uint8)
    codes[:, 0::2] = q & 0x0F
    codes[:, 1::2] = q >> 4
    vals = e2m1_table()[codes]
    scale = np.repeat(e4m3_table()[s], 16, axis=1)
    return vals * scale * ts


def silu(g):
    return g / (1.0 + np.exp(-g))


def swiglu_ffn(x64: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """Textbook SwiGLU MLP in float64 with numpy matmuls: x [.., H]."""
    g = x64 @ wg.T
    v = x64 @ wu.T
    return (silu(g) * v) @ wd.T
