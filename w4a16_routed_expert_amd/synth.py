"""Seeded synthetic inputs for the W4A16 routed-expert MoE layer.

This module only *makes inputs*: random tensors, the INT4 block quantizer that
turns them into qpacked bytes, and the byte packer. It holds none of the
layer's arithmetic (no dequantization, routing, FFN or combine), so the CPU
oracle and the HIP path can both be fed from it without sharing any code.

Sources (Horizon RunMap pages):
  * "Horizon RunMap - architecture", table "Representation and computation":
    routed experts are INT4 qpacked in 256-value blocks with FP16 scales,
    activations are FP16, non-routed weights are FP16.
  * "horizonrunmap.com/en", section "05 / Memory & speed" names the models
    whose shapes the configurations below stand in for (OLMoE-1B-7B, 64
    experts, top-8; Qwen1.5-MoE-A2.7B, 60 experts, top-4, one shared expert).
    The pages give no shapes; the hidden/intermediate sizes are those of the
    public model cards of the named checkpoints. No trained weights are used:
    every tensor is drawn from a seeded generator.

Quantizer (input preparation, not the hot path): per 256-value block along the
reduction axis, s = fp16(absmax / 7), code = clamp(rint(w / s), -7, 7) + 8
(round half to even), an all-zero block gets s = 0 and codes 8.

qpacked v1 byte layout of one matrix with R rows and K columns (row = output
feature, column = reduction index); R % 16 == 0 and K % 128 == 0:
  nibble plane, R*K/2 bytes, made of 1024-byte tiles.  Tile (rg, kt) covers
  rows 16*rg .. 16*rg+15 and columns 128*kt .. 128*kt+127 and sits at byte
  (rg * (K/128) + kt) * 1024.  Inside a tile, the 16-byte chunk number
  c = 16*g + r (g in 0..3, r in 0..15) holds row 16*rg + r, columns
  128*kt + 32*g .. +31; its byte i holds column 2i in bits 0-3 and column
  2i+1 in bits 4-7 (relative to the chunk's first column).
  scale plane, R * ceil(K/256) fp16 values: the scale of row 16*rg + r,
  block b (columns 256*b .. min(256*b+256, K)-1) is element
  (rg * ceil(K/256) + b) * 16 + r.
Expert row (the unit that is uploaded to the GPU): gate nibbles, up nibbles,
down nibbles, gate scales, up scales, down scales, each section starting on a
256-byte boundary.  gate/up are [I rows, H cols]; down is [H rows, I cols].
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SEED_ROOT = 0x57A16
BLOCK = 256
TILE_K = 128
TILE_R = 16
SECTION_ALIGN = 256


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_idx: int
    E: int            # routed experts
    k: int            # experts per token
    H: int            # hidden size
    I: int            # expert intermediate size
    batches: tuple    # token counts T exercised
    resident: int     # experts resident on the GPU (E = all)
    n_layers: int = 1
    zipf_s: float = 0.0       # per-layer Zipf expert bias exponent (0 = none)
    shared_I: int = 0         # FP16 shared-expert intermediate (0 = none)
    sigma_w: float = 0.02     # weight std before quantization
    sigma_r: float = 0.02     # router weight std
    sigma_x: float = 1.0      # activation std


CONFIGS = {
    "tiny": LayerConfig("tiny", 0, E=8, k=2, H=256, I=512, batches=(4,), resident=8),
    "olmoe": LayerConfig("olmoe", 1, E=64, k=8, H=2048, I=1024, batches=(1, 8, 32), resident=64),
    "olmoe_stack": LayerConfig("olmoe_stack", 2, E=64, k=8, H=2048, I=1024,
                               batches=(1, 2, 4, 8, 16, 32), resident=40, n_layers=16, zipf_s=1.1),
    "qwen": LayerConfig("qwen", 3, E=60, k=4, H=2048, I=1408, batches=(1, 16, 64), resident=39,
                        shared_I=5632),
    "prefill": LayerConfig("prefill", 4, E=64, k=8, H=2048, I=1024, batches=(4096,), resident=64),
}


def rng_for(cfg_idx: int, layer: int, tensor_idx: int, extra: int = 0) -> np.random.Generator:
    """Independent PCG64 stream per (config, layer, tensor[, extra])."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, cfg_idx, layer, tensor_idx, extra])))


# ---------------------------------------------------------------- fp16 helpers
def f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float16).view(np.uint16)


def bits_f16(b: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16)


# ---------------------------------------------------------------- quantizer
def n_blocks(K: int) -> int:
    return (K + BLOCK - 1) // BLOCK


def quantize_q4(w: np.ndarray):
    """w float32 [R, K] -> (codes uint8 [R, K] in 0..15, scales float16 [R, ceil(K/256)])."""
    w = np.asarray(w, dtype=np.float32)
    R, K = w.shape
    nb = n_blocks(K)
    codes = np.empty((R, K), dtype=np.uint8)
    scales = np.empty((R, nb), dtype=np.float16)
    for b in range(nb):
        blk = w[:, b * BLOCK:min((b + 1) * BLOCK, K)]
        amax = np.max(np.abs(blk), axis=1)
        s16 = (amax / np.float32(7.0)).astype(np.float16)
        s32 = s16.astype(np.float32)
        safe = np.where(s32 > 0, s32, np.float32(1.0))
        q = np.rint(blk / safe[:, None])
        q = np.clip(q, -7, 7)
        q = np.where(s32[:, None] > 0, q, 0.0)
        codes[:, b * BLOCK:min((b + 1) * BLOCK, K)] = (q + 8).astype(np.uint8)
        scales[:, b] = s16
    return codes, scales


# ---------------------------------------------------------------- packer
def check_matrix_shape(R: int, K: int) -> None:
    if R % TILE_R or K % TILE_K or R <= 0 or K <= 0:
        raise ValueError(f"qpacked v1 needs rows % 16 == 0 and cols % 128 == 0, got {R}x{K}")


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [R, K] (0..15) -> uint8 [R*K/2] in the tiled nibble-plane order."""
    R, K = codes.shape
    check_matrix_shape(R, K)
    c = codes.reshape(R // TILE_R, TILE_R, K // TILE_K, 4, 32)      # rg, r, kt, g, kk
    c = c.transpose(0, 2, 3, 1, 4)                                  # rg, kt, g, r, kk
    lo = c[..., 0::2].astype(np.uint8)
    hi = c[..., 1::2].astype(np.uint8)
    return np.ascontiguousarray((lo | (hi << 4)).reshape(-1))


def pack_scales(scales: np.ndarray) -> np.ndarray:
    """scales float16 [R, nb] -> uint16 [R*nb] in scale-plane order."""
    R, nb = scales.shape
    s = f16_bits(scales).reshape(R // TILE_R, TILE_R, nb).transpose(0, 2, 1)
    return np.ascontiguousarray(s.reshape(-1))


def _align(n: int) -> int:
    return (n + SECTION_ALIGN - 1) // SECTION_ALIGN * SECTION_ALIGN


def expert_row_layout(H: int, I: int) -> dict:
    """Byte offsets of the six sections of one expert row, and the row size."""
    check_matrix_shape(I, H)
    check_matrix_shape(H, I)
    sizes = [
        ("gate_q", I * H // 2), ("up_q", I * H // 2), ("down_q", H * I // 2),
        ("gate_s", I * n_blocks(H) * 2), ("up_s", I * n_blocks(H) * 2), ("down_s", H * n_blocks(I) * 2),
    ]
    off = 0
    out = {}
    for name, sz in sizes:
        out[name] = off
        off = _align(off + sz)
    out["row_bytes"] = off
    return out


def pack_expert_row(H: int, I: int, gate, up, down) -> np.ndarray:
    """Each of gate/up/down is (codes, scales).  Returns uint8 [row_bytes]."""
    lay = expert_row_layout(H, I)
    row = np.zeros(lay["row_bytes"], dtype=np.uint8)
    for name, (codes, scales) in (("gate", gate), ("up", up), ("down", down)):
        q = pack_nibbles(codes)
        s = pack_scales(scales).view(np.uint8)
        row[lay[name + "_q"]:lay[name + "_q"] + q.size] = q
        row[lay[name + "_s"]:lay[name + "_s"] + s.size] = s
    return row


# ---------------------------------------------------------------- layer inputs
def expert_codes(cfg: LayerConfig, layer: int, e: int):
    """Seeded float32 N(0, sigma_w) gate/up/down weights of one expert, quantized."""
    out = []
    for m, (R, K) in enumerate(((cfg.I, cfg.H), (cfg.I, cfg.H), (cfg.H, cfg.I))):
        g = rng_for(cfg.cfg_idx, layer, 100 + 3 * e + m)
        w = g.standard_normal((R, K), dtype=np.float32) * np.float32(cfg.sigma_w)
        out.append(quantize_q4(w))
    return out


def make_expert_rows(cfg: LayerConfig, layer: int = 0, experts=None) -> np.ndarray:
    """uint8 [E, row_bytes]: all expert rows of one layer (or the listed experts)."""
    experts = range(cfg.E) if experts is None else experts
    lay = expert_row_layout(cfg.H, cfg.I)
    rows = np.zeros((len(experts), lay["row_bytes"]), dtype=np.uint8)
    for i, e in enumerate(experts):
        g, u, d = expert_codes(cfg, layer, e)
        rows[i] = pack_expert_row(cfg.H, cfg.I, g, u, d)
    return rows


def make_router(cfg: LayerConfig, layer: int = 0) -> np.ndarray:
    """float16 [H, E] router weight, N(0, sigma_r) rounded to fp16."""
    g = rng_for(cfg.cfg_idx, layer, 1)
    return (g.standard_normal((cfg.H, cfg.E)) * cfg.sigma_r).astype(np.float16)


def make_zipf_bias(cfg: LayerConfig, layer: int = 0):
    """float32 [E] = -s * ln(rank), rank = 1 + a seeded permutation of 0..E-1; None if no skew."""
    if cfg.zipf_s == 0.0:
        return None
    g = rng_for(cfg.cfg_idx, layer, 2)
    rank = g.permutation(cfg.E).astype(np.float64) + 1.0
    return (-cfg.zipf_s * np.log(rank)).astype(np.float32)


def make_x(cfg: LayerConfig, T: int, step: int = 0, layer: int = 0) -> np.ndarray:
    """float16 [T, H] activations N(0, sigma_x), fresh per (step, layer)."""
    g = rng_for(cfg.cfg_idx, layer, 3, extra=step * 65536 + T)
    return (g.standard_normal((T, cfg.H)) * cfg.sigma_x).astype(np.float16)


def make_shared(cfg: LayerConfig, layer: int = 0):
    """FP16 shared expert: gate [Is, H], up [Is, H], down [H, Is], sigmoid-gate vector [H]."""
    if cfg.shared_I == 0:
        return None
    Is, H = cfg.shared_I, cfg.H
    out = []
    for m, shape in enumerate(((Is, H), (Is, H), (H, Is), (H,))):
        g = rng_for(cfg.cfg_idx, layer, 10 + m)
        out.append((g.standard_normal(shape, dtype=np.float32) * np.float32(cfg.sigma_w)).astype(np.float16))
    return tuple(out)


def pack_fp16_tile8(w: np.ndarray) -> np.ndarray:
    """The tile8 layout of an FP16 matrix [R][K] (R % 8 == 0, K % 128 == 0), as a flat float16
    array: tile (r8, kt) of 8 rows x 128 columns at element (r8 * K/128 + kt) * 1024, its piece s
    (256 values) at s * 256, and inside the piece element (8 g + r) * 8 + c = w[8 r8 + r][128 kt +
    32 s + 8 g + c].  A permutation of the values (no arithmetic)."""
    R, K = w.shape
    if R % 8 or K % 128:
        raise ValueError(f"tile8 needs R % 8 == 0 and K % 128 == 0, got {R}x{K}")
    a = np.ascontiguousarray(w, dtype=np.float16).reshape(R // 8, 8, K // 128, 4, 4, 8)   # r8 r kt s g c
    return np.ascontiguousarray(a.transpose(0, 2, 3, 4, 1, 5)).reshape(-1)             # r8 kt s g r c


def expected_active(E: int, k: int, T: int) -> float:
    """E * (1 - (1 - k/E)^T): expected number of distinct experts hit by T tokens (planning only)."""
    return E * (1.0 - math.pow(1.0 - k / E, T))
