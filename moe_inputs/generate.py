"""Seeded synthetic inputs for one MoE-layer call.

Recipe (every tensor comes from its own torch.Generator, seeded from
``SeedSequence([seed, tensor_id, expert])`` so that experts can be drawn one
at a time and the draw does not depend on how many experts exist):

* ``x``     [T, H]   ~ N(0, 1), rounded to the activation dtype.
* ``wg``    [E, H]   gate weight ~ N(0, 1/H), activation dtype.
* ``bias``  [E]      selection bias ~ U(-0.1, 0.1), fp32.
* ``w13``   [E, 2I, H]  rows [0, I) are the gate projection W1, rows [I, 2I)
                        the up projection W3, both ~ N(0, 1/H).
* ``w2``    [E, H, I]   down projection ~ N(0, 1/I).
* ``ws13``, ``ws2``     the shared expert, same laws, [2Is, H] and [H, Is].

Weights are [out, in] row-major (the layout of a linear layer's weight).

Routing structure is injected through the data, so the layer itself stays a
plain gate:

* ``zipf``: expert e gets a logit offset ``-s * ln(rank_e)`` with ``rank`` a
  seeded permutation of 1..E; it is carried by the last hidden column
  (x[:, H-1] = 1, wg[e, H-1] = offset_e).  Expert popularity then follows a
  Zipf(s) law.
* ``clusters``: experts form ``n_clusters`` consecutive clusters; each token
  draws one cluster; the last ``n_clusters`` hidden columns carry a one-hot of
  the token's cluster in x and ``boost`` times a one-hot of the expert's cluster
  in wg, adding ``boost`` to the logits of the token's own cluster.

FP8 expert weights (``w_dtype == "fp8"``) are drawn as above in fp32 and then
stored as OCP E4M3 codes with one fp32 scale per row per 128 columns:
``scale = amax / 448`` (1 when the block is all zero) and
``code = e4m3(clamp(w / scale, -448, 448))`` through torch's float8 cast.
This is the static, offline weight preparation that the pages' block
quantisation assumes (weights quantised ahead of time, activations on the
fly; Perplexity, "Lower latency and higher throughput with multi-node
DeepSeek deployment", section "Quantization").  The layer consumes the codes
and scales as given.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import MoEConfig

_TID = dict(x=1, wg=2, bias=3, w13=4, w2=5, ws13=6, ws2=7, zipf=8, clusters=9)

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def sub_seed(seed: int, tensor: str, expert: int = 0) -> int:
    ss = np.random.SeedSequence([int(seed), _TID[tensor], int(expert)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def _gen(device, seed, tensor, expert=0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(sub_seed(seed, tensor, expert))
    return g


def _normal(shape, std, device, seed, tensor, expert=0) -> torch.Tensor:
    g = _gen(device, seed, tensor, expert)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def quantize_weight_fp8(w: torch.Tensor, block: int = 128, block_rows: int = 1):
    """Static fp8 E4M3 quantisation of a [N, K] fp32 weight in blocks of
    ``block_rows`` x ``block`` (1 x 128 or 128 x 128): scale = amax / 448 of
    the block (1 for an all-zero block), codes = e4m3(w / scale).

    Returns (codes uint8 [N, K], scales fp32 [N // block_rows, K // block]).
    """
    n, kdim = w.shape
    assert kdim % block == 0 and n % block_rows == 0
    wb = w.view(n // block_rows, block_rows, kdim // block, block)
    amax = wb.abs().amax(dim=(1, 3))                                   # [N/br, K/b]
    scale = amax / 448.0
    scale = torch.where(amax == 0, torch.ones_like(scale), scale)
    q = (wb / scale[:, None, :, None]).clamp_(-448.0, 448.0)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, kdim)
    return codes, scale.contiguous()


@dataclass
class MoEInputs:
    cfg: MoEConfig
    x: torch.Tensor
    wg: torch.Tensor
    bias: torch.Tensor
    w13: torch.Tensor
    w2: torch.Tensor
    ws13: Optional[torch.Tensor]
    ws2: Optional[torch.Tensor]
    w13_scale: Optional[torch.Tensor] = None
    w2_scale: Optional[torch.Tensor] = None
    ws13_scale: Optional[torch.Tensor] = None
    ws2_scale: Optional[torch.Tensor] = None

    @property
    def device(self):
        return self.x.device


def _expert_weights(cfg: MoEConfig, device, tensor: str, e: int, rows: int, cols: int,
                    fan_in: int, w_out: torch.Tensor, s_out: Optional[torch.Tensor]):
    w = _normal((rows, cols), fan_in ** -0.5, device, cfg.seed, tensor, e)
    if cfg.w_dtype == "fp8":
        codes, scale = quantize_weight_fp8(w, cfg.quant_block, cfg.w_block_rows)
        w_out.copy_(codes)
        s_out.copy_(scale)
    else:
        w_out.copy_(w.to(_TORCH_DT[cfg.w_dtype]))


def make_router_inputs(cfg: MoEConfig, device="cpu"):
    """x [T,H], wg [E,H] (activation dtype) and bias [E] fp32: the router's
    inputs, identical to the ones ``make_inputs`` draws for the same config."""
    device = torch.device(device)
    T, H, E = cfg.T, cfg.H, cfg.E
    adt = _TORCH_DT[cfg.act_dtype]
    seed = cfg.seed

    x = _normal((T, H), 1.0, device, seed, "x")
    wg = _normal((E, H), H ** -0.5, device, seed, "wg")
    gb = _gen(device, seed, "bias")
    bias = (torch.rand((E,), generator=gb, device=device, dtype=torch.float32) * 0.2 - 0.1)

    if cfg.routing == "zipf":
        gz = _gen(device, seed, "zipf")
        rank = torch.randperm(E, generator=gz, device=device).to(torch.float32) + 1.0
        x[:, H - 1] = 1.0
        wg[:, H - 1] = -cfg.zipf_s * torch.log(rank)
    elif cfg.routing == "clusters":
        nc = cfg.n_clusters
        assert E % nc == 0 and H > nc
        gc = _gen(device, seed, "clusters")
        ct = torch.randint(0, nc, (T,), generator=gc, device=device)
        x[:, H - nc:] = torch.nn.functional.one_hot(ct, nc).to(torch.float32)
        ce = torch.arange(E, device=device) // (E // nc)
        wg[:, H - nc:] = cfg.cluster_boost * torch.nn.functional.one_hot(ce, nc).to(torch.float32)
    elif cfg.routing != "random":
        raise ValueError(f"unknown routing structure {cfg.routing!r}")
    return x.to(adt).contiguous(), wg.to(adt).contiguous(), bias.contiguous()


def make_inputs(cfg: MoEConfig, device="cpu") -> MoEInputs:
    """Draw every input of one layer call for ``cfg`` directly on ``device``.

    Draws on different devices use different torch generators and therefore
    give different (equally distributed) values; a test always feeds both the
    oracle and the library from one draw.
    """
    device = torch.device(device)
    T, H, E, I, Is = cfg.T, cfg.H, cfg.E, cfg.I, cfg.I_shared
    x, wg, bias = make_router_inputs(cfg, device)

    fp8 = cfg.w_dtype == "fp8"
    wdt = torch.uint8 if fp8 else _TORCH_DT[cfg.w_dtype]
    qb = cfg.quant_block
    w13 = torch.empty((E, 2 * I, H), dtype=wdt, device=device)
    w2 = torch.empty((E, H, I), dtype=wdt, device=device)
    br = cfg.w_block_rows
    w13_s = torch.empty((E, 2 * I // br, H // qb), dtype=torch.float32, device=device) if fp8 else None
    w2_s = torch.empty((E, H // br, I // qb), dtype=torch.float32, device=device) if fp8 else None
    for e in range(E):
        _expert_weights(cfg, device, "w13", e, 2 * I, H, H, w13[e], w13_s[e] if fp8 else None)
        _expert_weights(cfg, device, "w2", e, H, I, I, w2[e], w2_s[e] if fp8 else None)

    ws13 = ws2 = ws13_s = ws2_s = None
    if Is > 0:
        ws13 = torch.empty((2 * Is, H), dtype=wdt, device=device)
        ws2 = torch.empty((H, Is), dtype=wdt, device=device)
        ws13_s = torch.empty((2 * Is // br, H // qb), dtype=torch.float32, device=device) if fp8 else None
        ws2_s = torch.empty((H // br, Is // qb), dtype=torch.float32, device=device) if fp8 else None
        _expert_weights(cfg, device, "ws13", 0, 2 * Is, H, H, ws13, ws13_s)
        _expert_weights(cfg, device, "ws2", 0, H, Is, Is, ws2, ws2_s)

    return MoEInputs(cfg, x, wg, bias, w13, w2, ws13, ws2, w13_s, w2_s, ws13_s, ws2_s)
