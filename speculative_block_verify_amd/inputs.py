"""Seeded synthetic inputs for the MoE block-verify layer.

This module only *produces data*: bf16 activations and router weights, and
expert weights packed in NVFP4.  It holds none of the layer's arithmetic
(no routing, no dequantisation, no FFN).  The same bytes are handed both to
the HIP library and to the CPU oracle; neither side imports the other.

Shapes follow the Laguna XS 2.1 description on the mlxfast challenge README
("Why this challenge exists": hidden 2048, 256 routed experts + 1 shared,
top-8, MoE intermediate 512, NVFP4 group-16 on expert projections, bf16
routers), and the byte budget in PR #844 section 2 ("Where the time goes").

NVFP4 packing (the reading used throughout this repository):
  q  uint8 [E, rows, cols/2]   two E2M1 codes per byte, even column in the
                               low nibble, odd column in the high nibble;
  s  uint8 [E, rows, cols/16]  one E4M3FN scale per 16 consecutive input
                               columns of a row;
  ts fp32  [E]                 one tensor scale per expert matrix.

Quantisation recipe for synthetic weights (pages are silent; data shaping
only, both sides consume the resulting bytes):
  W ~ N(0, std^2) fp32;  ts = amax(|W|) / (6 * 448);
  s = e4m3_rne(amax_block / (6 * ts));  q = e2m1_rne(W / (s * ts)), ties to
  the even code, magnitudes clamped to 6;  all-zero blocks get s = q = 0.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional

import torch

# ---------------------------------------------------------------------------
# Workload shapes
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class MoEShape:
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int


TINY = MoEShape(hidden=256, n_experts=16, top_k=2, inter=128, shared_inter=0)
LAGUNA = MoEShape(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512)

WEIGHT_STD = 0.02      # expert and router weights ~ N(0, 0.02^2)
X_STD = 1.0            # activations ~ N(0, 1)
KSWEEP_LOGIT_NOISE = 0.01

# E2M1 magnitudes indexed by the 3-bit code (exponent bits 2..1, mantissa
# bit 0).  Used here only to *encode* synthetic data.
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_E4M3_MAX = 448.0
_E2M1_MAX = 6.0


def _seed(*parts) -> int:
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _randn(shape, device, *parts) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(device, *parts), device=device, dtype=torch.float32)


# ---------------------------------------------------------------------------
# Encoders (data shaping only)
# ---------------------------------------------------------------------------


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """Round fp32 to bf16 (torch's round-to-nearest-even) and return the raw
    16-bit patterns as int16."""
    return t.to(torch.bfloat16).view(torch.int16)


def _e2m1_encode(v: torch.Tensor) -> torch.Tensor:
    """Nearest E2M1 code (sign in bit 3), ties to the even code."""
    grid = torch.tensor(_E2M1_GRID, device=v.device, dtype=torch.float32)
    mag = v.abs().clamp(max=_E2M1_MAX)
    lo = torch.bucketize(mag, grid, right=True) - 1          # grid[lo] <= mag
    lo = lo.clamp(0, 7)
    hi = (lo + 1).clamp(max=7)
    d_lo = mag - grid[lo]
    d_hi = grid[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = torch.where(take_hi, hi, lo).to(torch.uint8)
    sign = ((v < 0) & (code != 0)).to(torch.uint8) << 3
    return code | sign


def quantize_nvfp4(w: torch.Tensor):
    """Pack fp32 weights [E, rows, cols] into (q, s, ts) as documented above."""
    E, rows, cols = w.shape
    assert cols % 16 == 0
    amax = w.abs().amax(dim=(1, 2))                                    # [E]
    ts = (amax / (6.0 * _E4M3_MAX)).to(torch.float32)
    ts = torch.where(ts > 0, ts, torch.ones_like(ts))
    blocks = w.view(E, rows, cols // 16, 16)
    bamax = blocks.abs().amax(dim=-1)                                  # [E, rows, cols/16]
    s_f = (bamax / (6.0 * ts[:, None, None])).clamp(max=_E4M3_MAX)
    s8 = s_f.to(torch.float8_e4m3fn)
    s_dec = s8.to(torch.float32)
    denom = (s_dec * ts[:, None, None])[..., None]
    scaled = torch.where(denom > 0, blocks / torch.where(denom > 0, denom, torch.ones_like(denom)),
                         torch.zeros_like(blocks))
    codes = _e2m1_encode(scaled).view(E, rows, cols)
    q = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return q.contiguous(), s8.view(torch.uint8).contiguous(), ts.contiguous()


# ---------------------------------------------------------------------------
# Layer / stack generators
# ---------------------------------------------------------------------------


def gen_nvfp4(E: int, rows: int, cols: int, device, *parts, std: float = WEIGHT_STD):
    # Generate expert by expert so a 256-expert matrix never needs more than
    # one expert's fp32 copy plus the packed result.
    qs, ss, tss = [], [], []
    chunk = max(1, min(E, (1 << 26) // (rows * cols)))
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        w = _randn((e1 - e0, rows, cols), device, *parts, e0) * std
        q, s, ts = quantize_nvfp4(w)
        qs.append(q); ss.append(s); tss.append(ts)
        del w
    return {"q": torch.cat(qs), "s": torch.cat(ss), "ts": torch.cat(tss)}


def gen_layer(shape: MoEShape, seed: int, layer: int = 0, device="cpu",
              with_bias: bool = False) -> Dict[str, object]:
    """One MoE layer's weights.  Router bf16 [E, H]; gate/up NVFP4 [E, I, H];
    down NVFP4 [E, H, I]; shared expert (if any) as E = 1 matrices."""
    H, E, I, Is = shape.hidden, shape.n_experts, shape.inter, shape.shared_inter
    out: Dict[str, object] = {}
    out["router_w"] = bf16_bits(_randn((E, H), device, seed, layer, "router") * WEIGHT_STD)
    out["router_bias"] = (_randn((E,), device, seed, layer, "bias") * 0.01) if with_bias else None
    out["gate"] = gen_nvfp4(E, I, H, device, seed, layer, "gate")
    out["up"] = gen_nvfp4(E, I, H, device, seed, layer, "up")
    out["down"] = gen_nvfp4(E, H, I, device, seed, layer, "down")
    if Is > 0:
        out["sh_gate"] = gen_nvfp4(1, Is, H, device, seed, layer, "sh_gate")
        out["sh_up"] = gen_nvfp4(1, Is, H, device, seed, layer, "sh_up")
        out["sh_down"] = gen_nvfp4(1, H, Is, device, seed, layer, "sh_down")
    else:
        out["sh_gate"] = out["sh_up"] = out["sh_down"] = None
    return out


def gen_x(K: int, H: int, seed: int, device="cpu", tag: str = "x") -> torch.Tensor:
    """bf16 activations [K, H] ~ N(0, 1), as int16 bit patterns."""
    return bf16_bits(_randn((K, H), device, seed, tag) * X_STD)


def gen_x_correlated(K: int, H: int, seed: int, device="cpu") -> torch.Tensor:
    """K-sweep rows: rows 1..floor(K/2) are row 0 plus N(0, sigma^2) noise with
    sigma chosen so the layer-0 router logits move by ~N(0, 0.01^2):
    sigma = 0.01 / (0.02 * sqrt(H))."""
    base = _randn((K, H), device, seed, "xk") * X_STD
    sigma = KSWEEP_LOGIT_NOISE / (WEIGHT_STD * (H ** 0.5))
    noise = _randn((K, H), device, seed, "xk-noise") * sigma
    for r in range(1, K // 2 + 1):
        base[r] = base[0] + noise[r]
    return bf16_bits(base)


def gen_logits(K: int, E: int, seed: int, device="cpu", std: float = 1.0) -> torch.Tensor:
    return _randn((K, E), device, seed, "logits") * std


def gen_stack(shape: MoEShape, n_layers: int, seed: int, device="cpu",
              with_bias: bool = False) -> List[Dict[str, object]]:
    return [gen_layer(shape, seed, l, device, with_bias) for l in range(n_layers)]



# ---------------------------------------------------------------------------
# The verify step's head: lm_head weights and draft tokens
# ---------------------------------------------------------------------------

VOCAB = 100352      # the pages' lm_head: bf16 [100352, 2048], 0.41 GB


DENSE_INTER = 8192    # the target's dense first layer (README "Why this challenge exists")


def gen_dense(hidden: int, inter: int, seed: int, device="cpu") -> Dict[str, object]:
    """The dense first layer's bf16 SwiGLU weights ~ N(0, 0.02^2) as int16 bit
    patterns: gate/up [inter, hidden], down [hidden, inter]; no norm weight."""
    return {"gate": bf16_bits(_randn((inter, hidden), device, seed, "dense_gate") * WEIGHT_STD),
            "up": bf16_bits(_randn((inter, hidden), device, seed, "dense_up") * WEIGHT_STD),
            "down": bf16_bits(_randn((hidden, inter), device, seed, "dense_down") * WEIGHT_STD),
            "norm_w": None}


def gen_lm_head(vocab: int, hidden: int, seed: int, device="cpu") -> torch.Tensor:
    """bf16 lm_head weights [vocab, hidden] ~ N(0, 0.02^2), as int16 bit
    patterns (generated in chunks of rows)."""
    out = torch.empty(vocab, hidden, dtype=torch.int16, device=device)
    step = max(1, (1 << 24) // hidden)
    for v0 in range(0, vocab, step):
        v1 = min(vocab, v0 + step)
        out[v0:v1] = bf16_bits(_randn((v1 - v0, hidden), device, seed, "lm_head", v0) * WEIGHT_STD)
    return out


def gen_tokens(n: int, vocab: int, seed: int, device="cpu") -> torch.Tensor:
    """n uniform token ids in [0, vocab) (int32)."""
    g = _gen(device, seed, "tokens")
    return torch.randint(0, vocab, (n,), generator=g, device=device, dtype=torch.int32)


def gen_norm_weights(n_layers: int, hidden: int, seed: int, device="cpu") -> List[torch.Tensor]:
    """bf16 RMSNorm weights per layer, ~ N(1, 0.1^2) (synthetic; the pages
    give no values), as int16 bit patterns."""
    return [bf16_bits(1.0 + 0.1 * _randn((hidden,), device, seed, l, "norm_w")) for l in range(n_layers)]
