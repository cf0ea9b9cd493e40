"""Seeded synthetic workloads for the Deja Vu sparse decode step.

This module holds shapes, keep counts and random inputs only.  It contains none
of the method's arithmetic: no products, no activation, no softmax, no top-k.
Both the HIP path (through its tests and the benchmark) and the CPU oracle (through
the tests) take their inputs from here, so that the two sides see identical data.

Shapes follow the OPT family used on the Deja Vu page ("Deja Vu: contextual
sparsity for efficient LLMs at inference time", section 2.3: a layer has
W1, W2 in R^{d x 4d}, h heads of width d_h, and a KV cache of n previous tokens).
The pages evaluate on OPT checkpoints with OpenBookQA / WikiText text
(section 3.1); neither is available here, so i.i.d. Gaussian tensors of the
same shapes stand in for them and prediction quality is not measured.

Storage layouts (all row-major; a "row" is one contiguous d-vector):
  y      [B][d]         fp32, the layer input of the current decode step
  W1t    [F][d]         row i is the column W1_i of W1 (neuron-major)
  W2t    [F][d]         row i is the column W2_i of W2 (neuron-major)
  Wq     [h][dh][d]     Wq[i][c] is column c of W_i^Q
  Wo     [h][dh][d]     Wo[i] is W_i^O (dh x d), unchanged
  K, V   [B][h][n][dh]  K[b][i] = X_b W_i^K, V[b][i] = X_b W_i^V
  A      [r][d]         low-rank predictor, first factor (one rank vector a row)
  Bm     [r][N]         low-rank predictor, second factor
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import torch

# Tensor order used to derive seeds; the position is part of the seed recipe.
TENSOR_IDS = {
    "y": 0, "W1t": 1, "W2t": 2, "Wq": 3, "Wk": 4, "Wv": 5, "Wo": 6,
    "K": 7, "V": 8, "A_M": 9, "B_M": 10, "A_A": 11, "B_A": 12,
}


@dataclass(frozen=True)
class LayerConfig:
    """One decode-layer workload.

    ``k_m``/``k_a`` are explicit per-token keep counts (neurons / heads).  The
    pages give keep fractions; the count is the fraction times N rounded to
    nearest (the only printed count, 154 of 1024 for 15 %, fixes that reading).
    """
    name: str
    cfg_id: int
    d: int
    F: int
    h: int
    dh: int
    batch: int
    n_ctx: int
    k_m: int
    k_a: int
    r: int
    wdtype: str = "bf16"          # "bf16" or "f32" for W1t, W2t, Wq, Wo, A, Bm
    kvdtype: str = "bf16"         # "bf16" or "f32" for K, V
    y_unit_rms: bool = True       # c2..c5 scale each token to unit RMS
    union: bool = False           # batch union of the per-token sets
    w_std: float = 0.02
    pred_std: float = 0.05
    kv_std: float = 1.0
    layers: int = 1
    scale: float = 1.0            # logit scale; the page's Eq. 2 has none

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def torch_wdtype(self) -> torch.dtype:
        return torch.bfloat16 if self.wdtype == "bf16" else torch.float32

    @property
    def torch_kvdtype(self) -> torch.dtype:
        return torch.bfloat16 if self.kvdtype == "bf16" else torch.float32


def keep_count(fraction: float, n: int) -> int:
    """Per-token keep count: fraction of n rounded half up."""
    return int(fraction * n + 0.5)


# The five workloads (tiny fp32, OPT-6.7B, OPT-30B, OPT-175B, 24-layer OPT-175B stack).
CONFIGS = {
    "c1": LayerConfig("tiny-fp32", 1, d=256, F=1024, h=4, dh=64, batch=1, n_ctx=32,
                      k_m=154, k_a=2, r=64, wdtype="f32", kvdtype="f32",
                      y_unit_rms=False),
    "c2": LayerConfig("opt-6.7b", 2, d=4096, F=16384, h=32, dh=128, batch=1, n_ctx=512,
                      k_m=keep_count(0.10, 16384), k_a=keep_count(0.25, 32), r=1000),
    "c3": LayerConfig("opt-30b", 3, d=7168, F=28672, h=56, dh=128, batch=4, n_ctx=1024,
                      k_m=keep_count(0.12, 28672), k_a=keep_count(0.20, 56), r=1000,
                      union=True),
    "c4": LayerConfig("opt-175b", 4, d=12288, F=49152, h=96, dh=128, batch=1, n_ctx=2048,
                      k_m=keep_count(0.10, 49152), k_a=keep_count(0.20, 96), r=1000,
                      union=True),
    "c5": LayerConfig("opt-175b-stack24", 5, d=12288, F=49152, h=96, dh=128, batch=32,
                      n_ctx=2048, k_m=keep_count(0.10, 49152), k_a=keep_count(0.20, 96),
                      r=1000, union=True, layers=24),
}
C4_BATCHES = (1, 2, 4, 8, 16)


def seed_of(cfg_id: int, layer: int, name: str) -> int:
    return 1000 * cfg_id + 16 * layer + TENSOR_IDS[name]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, seed, device, dtype) -> torch.Tensor:
    """i.i.d. N(0, std^2) drawn in fp32, then rounded to ``dtype`` (bf16: RNE)."""
    t = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype) if dtype != torch.float32 else t


def make_y(cfg: LayerConfig, device="cpu", layer: int = 0, batch: int | None = None) -> torch.Tensor:
    """Layer input [B][d] fp32; N(0,1) per element, optionally scaled to unit RMS per token."""
    B = cfg.batch if batch is None else batch
    y = _normal((B, cfg.d), 1.0, seed_of(cfg.cfg_id, layer, "y"), device, torch.float32)
    if cfg.y_unit_rms:
        rms = y.pow(2).mean(dim=1, keepdim=True).sqrt()
        y = y / rms
    return y.contiguous()


@dataclass
class LayerTensors:
    """Device- or host-resident tensors of one layer (inputs only)."""
    cfg: LayerConfig
    W1t: torch.Tensor
    W2t: torch.Tensor
    Wq: torch.Tensor
    Wo: torch.Tensor
    K: torch.Tensor
    V: torch.Tensor
    A_M: torch.Tensor
    B_M: torch.Tensor
    A_A: torch.Tensor
    B_A: torch.Tensor
    extra: dict = field(default_factory=dict)


def make_layer(cfg: LayerConfig, device="cpu", layer: int = 0, batch: int | None = None,
               with_kv: bool = True) -> LayerTensors:
    """Weights, KV cache and predictor factors of one layer, from the seed recipe."""
    B = cfg.batch if batch is None else batch
    wdt, kvdt = cfg.torch_wdtype, cfg.torch_kvdtype
    s = lambda name: seed_of(cfg.cfg_id, layer, name)  # noqa: E731
    W1t = _normal((cfg.F, cfg.d), cfg.w_std, s("W1t"), device, wdt)
    W2t = _normal((cfg.F, cfg.d), cfg.w_std, s("W2t"), device, wdt)
    Wq = _normal((cfg.h, cfg.dh, cfg.d), cfg.w_std, s("Wq"), device, wdt)
    Wo = _normal((cfg.h, cfg.dh, cfg.d), cfg.w_std, s("Wo"), device, wdt)
    if with_kv:
        K = _normal((B, cfg.h, cfg.n_ctx, cfg.dh), cfg.kv_std, s("K"), device, kvdt)
        V = _normal((B, cfg.h, cfg.n_ctx, cfg.dh), cfg.kv_std, s("V"), device, kvdt)
    else:
        K = V = None
    A_M = _normal((cfg.r, cfg.d), cfg.pred_std, s("A_M"), device, wdt)
    B_M = _normal((cfg.r, cfg.F), cfg.pred_std, s("B_M"), device, wdt)
    A_A = _normal((cfg.r, cfg.d), cfg.pred_std, s("A_A"), device, wdt)
    B_A = _normal((cfg.r, cfg.h), cfg.pred_std, s("B_A"), device, wdt)
    return LayerTensors(cfg, W1t, W2t, Wq, Wo, K, V, A_M, B_M, A_A, B_A)


def make_kv_weights(cfg: LayerConfig, device="cpu", layer: int = 0):
    """W^K and W^V of one layer, stored like W^Q as [h][d_h][d] (row c of head i is
    column c of W_i^K), from the seed recipe."""
    s = lambda name: seed_of(cfg.cfg_id, layer, name)  # noqa: E731
    return (_normal((cfg.h, cfg.dh, cfg.d), cfg.w_std, s("Wk"), device, cfg.torch_wdtype),
            _normal((cfg.h, cfg.dh, cfg.d), cfg.w_std, s("Wv"), device, cfg.torch_wdtype))


def make_kv_cache(cfg: LayerConfig, cap: int, device="cpu", layer: int = 0,
                  batch: int | None = None, fill: float = 1e4):
    """A KV cache with room for ``cap`` rows per (token, head), [B][h][cap][d_h]:
    rows 0..n_ctx-1 are the layer's seeded cache, the rest hold ``fill`` (a value no
    computed row takes, so a test can see which rows a step wrote)."""
    B = cfg.batch if batch is None else batch
    s = lambda name: seed_of(cfg.cfg_id, layer, name)  # noqa: E731
    out = []
    for name in ("K", "V"):
        t = torch.full((B, cfg.h, cap, cfg.dh), fill, dtype=cfg.torch_kvdtype, device=device)
        t[:, :, :cfg.n_ctx] = _normal((B, cfg.h, cfg.n_ctx, cfg.dh), cfg.kv_std, s(name), device,
                                      cfg.torch_kvdtype)
        out.append(t)
    return tuple(out)


def make_predictor(cfg: LayerConfig, device="cpu", layer: int = 0):
    """Only the predictor factors (A_M, B_M, A_A, B_A) of a layer, same seeds as make_layer."""
    wdt = cfg.torch_wdtype
    s = lambda name: seed_of(cfg.cfg_id, layer, name)  # noqa: E731
    return dict(A_M=_normal((cfg.r, cfg.d), cfg.pred_std, s("A_M"), device, wdt),
                B_M=_normal((cfg.r, cfg.F), cfg.pred_std, s("B_M"), device, wdt),
                A_A=_normal((cfg.r, cfg.d), cfg.pred_std, s("A_A"), device, wdt),
                B_A=_normal((cfg.r, cfg.h), cfg.pred_std, s("B_A"), device, wdt))


def random_index_set(N: int, count: int, seed: int) -> torch.Tensor:
    """A seeded ascending subset of [0, N) of the given size (int32), for tests that
    feed the sparse blocks a set directly rather than through the predictor."""
    g = _gen(seed, "cpu")
    perm = torch.randperm(N, generator=g)[:count]
    return torch.sort(perm).values.to(torch.int32)


E4M3_MAX = 448.0   # largest finite OCP fp8 E4M3 value


def quantize_rows_e4m3(W: torch.Tensor):
    """Weight-only fp8 input preparation: one float32 scale per row (last axis) so the
    row's largest magnitude maps to 448, then each element rounded to the nearest
    E4M3 value (ties to even, torch's float8_e4m3fn cast).  Returns (codes as uint8,
    scales as float32) on W's device; an all-zero row gets scale 1."""
    w = W.float()
    amax = w.abs().amax(dim=-1)
    scales = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (w / scales.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).contiguous(), scales.contiguous()


def to_f64_numpy(t: torch.Tensor):
    """Exact widening of a host or device tensor (fp32 or bf16) to a float64 NumPy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
