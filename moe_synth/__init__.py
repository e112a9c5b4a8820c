"""Seeded synthetic inputs for MoE dispatch/combine, shared by tests, the smoke check and the bench.

This module makes inputs only.  It holds none of the routing, dispatch or combine arithmetic:
neither the HIP path nor the oracle imports anything else from the other, and both read the
arrays made here.

Workloads (shapes of the models the pages discuss; distributions are synthetic):
  tiny                     N=2  T=16   H=256  E=8   R=2  bf16, logits ~N(0,1)
  mixtral_8x7b_decode      N=8  T=128  H=4096 E=8   R=2  bf16, logits ~N(0,1)
  deepseek_v3_decode       N=32 T=128  H=7168 E=256 R=8  bf16, logits ~N(0,1) + Zipf(s=1) bias
  deepseek_v3_decode_fp8   same, payload e4m3 + fp32 scale per 128 elements
  qwen3_235b_prefill       N=4  T=4096 H=4096 E=128 R=8  bf16, logits ~N(0,1)
  kimi_k2_worst            N=64 T=128  H=7168 E=384 R=8  e4m3 + scales, +16 bias on experts 0..5
  deepseek_v3_decode_fp8q  DeepSeek-V3 decode, bf16 tokens quantised to e4m3 rows by the send pack
  deepseek_v3_decode_ragged DeepSeek-V3 decode (bf16) with a token count per rank, T_s ~ U{1..T}
  qwen3_235b_prefill_ep    N=4  T=4096 H=4096 E=128 R=8  bf16, the same T tokens on every rank
                           (prefill expert parallelism with replicated inputs), logits ~N(0,1)

Recipe (seed s, numpy PCG64 ``default_rng``): logits = rng(s).standard_normal((N*T, E), f32);
then x = rng(s) (same stream, next draw) .standard_normal((N, T, H), f32) rounded to bf16
(round-to-nearest-even).  fp8 payloads: per token and per 128-element block,
scale = amax / 448 (1 if amax == 0), codes = e4m3(clamp(x / scale, -448, 448)).
Zipf bias: bias[e] = -ln(1 + pi[e]) with pi a permutation of 0..E-1 drawn from
``default_rng(1)``, so expert popularity falls off as 1 / rank.
Kimi worst case: bias = +16 on experts 0..5 (rank 0's experts), 0 elsewhere: every token picks
all six, the other two slots go to the noise winners among experts 6..383.
Ragged token counts: T_s = default_rng(seed + 2).integers(1, T + 1, N) (uniform on 1..T); the
tokens past T_s of each rank still hold data but take no part.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

try:  # torch is used only for its bf16 / e4m3 conversions (vectorised, round-to-nearest-even)
    import torch
except ImportError:  # pragma: no cover
    torch = None

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Config:
    name: str
    N: int
    T: int
    H: int
    E: int
    R: int
    fp8: bool = False       # tokens arrive as e4m3 codes + scales
    bias: str = "none"      # "none" | "zipf" | "kimi"
    seed: int = 0
    desc: str = ""
    quant: bool = False     # tokens arrive as bf16; the send pack makes the e4m3 rows
    tokens: str = "full"    # "full" (T per rank) | "ragged" (T_s uniform on 1..T)
    layout: str = "decode"  # "decode" (T tokens per rank) | "prefill" (T tokens on every rank)

    @property
    def L(self) -> int:
        return self.E // self.N

    @property
    def B(self) -> int:
        """Receive rows per rank at the worst-case bound N*T*max(R, E/N)."""
        return self.N * self.T * max(self.R, self.L)

    @property
    def M(self) -> int:
        """Routed rows in total, N*T*R."""
        return self.N * self.T * self.R

    @property
    def rows_fp8(self) -> bool:
        """Dispatched rows are e4m3 codes + scales."""
        return self.fp8 or self.quant

    @property
    def dtype(self) -> str:
        return "bf16->fp8_e4m3" if self.quant else ("fp8_e4m3" if self.fp8 else "bf16")


CONFIGS = {
    c.name: c for c in [
        Config("tiny", 2, 16, 256, 8, 2, desc="N2 T16 H256 E8 R2 bf16"),
        Config("mixtral_8x7b_decode", 8, 128, 4096, 8, 2,
               desc="Mixtral-8x7B-shaped decode, N8 T128 H4096 E8 R2 bf16"),
        Config("deepseek_v3_decode", 32, 128, 7168, 256, 8, bias="zipf",
               desc="DeepSeek-V3-shaped decode, N32 T128 H7168 E256 R8 bf16, Zipf bias"),
        Config("deepseek_v3_decode_fp8", 32, 128, 7168, 256, 8, fp8=True, bias="zipf",
               desc="DeepSeek-V3-shaped decode, N32 T128 H7168 E256 R8 e4m3+scales, Zipf bias"),
        Config("qwen3_235b_prefill", 4, 4096, 4096, 128, 8,
               desc="Qwen3-235B-shaped prefill, N4 T4096 H4096 E128 R8 bf16"),
        Config("kimi_k2_worst", 64, 128, 7168, 384, 8, fp8=True, bias="kimi",
               desc="Kimi-K2-shaped worst case, N64 T128 H7168 E384 R8 e4m3+scales, "
                    "all tokens on rank 0's six experts"),
        Config("deepseek_v3_decode_fp8q", 32, 128, 7168, 256, 8, quant=True, bias="zipf",
               desc="DeepSeek-V3-shaped decode, N32 T128 H7168 E256 R8, bf16 tokens quantised "
                    "to e4m3+scales in the send pack, Zipf bias"),
        Config("deepseek_v3_decode_ragged", 32, 128, 7168, 256, 8, bias="zipf", tokens="ragged",
               desc="DeepSeek-V3-shaped decode, N32 T<=128 H7168 E256 R8 bf16, Zipf bias, "
                    "tokens per rank uniform on 1..128"),
        Config("qwen3_235b_prefill_ep", 4, 4096, 4096, 128, 8, layout="prefill",
               desc="Qwen3-235B-shaped prefill with replicated inputs (EP=4), T4096 H4096 E128 R8 "
                    "bf16"),
    ]
}


def make_tokens(kind: str, N: int, T: int, seed: int):
    """Per-rank token counts (int32[N]) or None for T on every rank."""
    if kind == "full":
        return None
    if kind == "ragged":
        return np.random.default_rng(seed + 2).integers(1, T + 1, N).astype(np.int32)
    raise ValueError(kind)


def config_tokens(cfg: "Config"):
    return make_tokens(cfg.tokens, cfg.N, cfg.T, cfg.seed)


def make_bias(kind: str, E: int):
    if kind == "none":
        return None
    if kind == "zipf":
        perm = np.random.default_rng(1).permutation(E)
        return (-np.log1p(perm.astype(np.float64))).astype(np.float32)
    if kind == "kimi":
        b = np.zeros(E, np.float32)
        b[:6] = 16.0
        return b
    raise ValueError(kind)


def to_bf16_bits(xf32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even), returned as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(xf32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def quantize_e4m3(xf32: np.ndarray):
    """Per-token, per-128-block e4m3 quantisation of [..., H] -> (codes uint8, scales f32)."""
    H = xf32.shape[-1]
    assert H % 128 == 0
    blk = xf32.reshape(*xf32.shape[:-1], H // 128, 128).astype(np.float32)
    amax = np.abs(blk).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = np.clip(blk / scale[..., None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn)
    codes = codes.view(torch.uint8).numpy().reshape(xf32.shape)
    return codes, scale


def make_inputs(N: int, T: int, H: int, E: int, R: int, fp8: bool = False, bias: str = "none",
                seed: int = 0) -> dict:
    """Seeded inputs: logits f32[N*T][E], bias f32[E] | None, x (bf16 bits uint16[N][T][H] or
    e4m3 codes uint8[N][T][H]), x_scale f32[N][T][H/128] | None, and xf (the fp32 values the
    payload was made from, after the bf16 rounding)."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((N * T, E), dtype=np.float32)
    xf = rng.standard_normal((N, T, H), dtype=np.float32)
    xb = to_bf16_bits(xf)
    xf = bf16_bits_to_f32(xb)
    out = dict(logits=logits, bias=make_bias(bias, E), xf=xf)
    if fp8:
        out["x"], out["x_scale"] = quantize_e4m3(xf)
    else:
        out["x"], out["x_scale"] = xb, None
    return out


def config_inputs(cfg: Config) -> dict:
    return make_inputs(cfg.N, cfg.T, cfg.H, cfg.E, cfg.R, cfg.fp8, cfg.bias, cfg.seed)


def random_y(N: int, B: int, H: int, seed: int) -> np.ndarray:
    """bf16 bit patterns ~N(0,1) for an arbitrary expert output tensor [N][B][H]."""
    rng = np.random.default_rng(seed + 7919)
    return to_bf16_bits(rng.standard_normal((N, B, H), dtype=np.float32))


TIE_KINDS = ("equal", "levels", "signed_zero", "bias_round")


def tie_logits(kind: str, n_tokens: int, E: int, seed: int):
    """Router scores made to tie, for the selection order's tie rule.  Returns (logits f32
    [n_tokens][E], bias f32[E] or None).
      equal        every expert of a row has the same score (one N(0,1) value per row)
      levels       N(0,1) rounded to multiples of 1/2: a handful of values, many ties per row,
                   equal scores spread over every lane and lane group
      signed_zero  negative scores with 2..E experts per row set to +0.0 or -0.0 (random sign),
                   so the largest scores are zeros of both signs; no bias
      bias_round   logits 1e-4 * N(0,1) and bias 1000 + (e % 4) * 2^-14 (2^-14 is one fp32 step
                   at 1000): the fp32 sums fall on a few neighbouring values, so experts whose
                   logits differ tie once the bias is added"""
    rng = np.random.default_rng(seed + 31337)
    if kind == "equal":
        v = rng.standard_normal((n_tokens, 1), dtype=np.float32)
        return np.repeat(v, E, axis=1), None
    if kind == "levels":
        v = rng.standard_normal((n_tokens, E), dtype=np.float32)
        return (np.round(v * 2.0) / 2.0).astype(np.float32), None
    if kind == "signed_zero":
        v = -np.abs(rng.standard_normal((n_tokens, E), dtype=np.float32)) - np.float32(0.5)
        nz = rng.integers(min(2, E), E + 1, n_tokens)
        keys = rng.random((n_tokens, E))
        ranks = np.argsort(np.argsort(keys, axis=1), axis=1)
        zero = ranks < nz[:, None]
        sign = rng.random((n_tokens, E)) < 0.5
        v[zero & sign] = np.float32(-0.0)
        v[zero & ~sign] = np.float32(0.0)
        return v.astype(np.float32), None
    if kind == "bias_round":
        v = (rng.standard_normal((n_tokens, E), dtype=np.float32) * np.float32(1e-4)).astype(np.float32)
        bias = (np.float32(1000.0) + (np.arange(E) % 4).astype(np.float32) * np.float32(2.0 ** -14))
        return v, bias.astype(np.float32)
    raise ValueError(kind)


def random_topk(N: int, T: int, E: int, R: int, seed: int) -> np.ndarray:
    """R distinct experts per token drawn uniformly: int32[N][T][R]."""
    rng = np.random.default_rng(seed + 104729)
    keys = rng.random((N * T, E))
    return np.argsort(keys, axis=1)[:, :R].astype(np.int32).reshape(N, T, R)
