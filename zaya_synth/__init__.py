"""Seeded synthetic inputs for the ZAYA1 decoder block.

This module only draws random numbers and lays them out: it holds none of the
block's arithmetic. Both the HIP path (through its Python binding) and the CPU
oracle are fed from it.

Every tensor has its own PCG64 stream keyed by (seed, config name, block index,
tensor name). Draws are float32; for bfloat16 configurations the draw is rounded
once to bfloat16 by torch's conversion (round-to-nearest-even), so the GPU and
the oracle see identical values.

Shapes follow the ZAYA1-8B printout and config ("Printout" and "Config" on the
nnterp encyclopedia page for ``nnterp.families.zaya``); the initialisation recipe
(weights N(0, 0.02), residual scales 1 + N(0, 0.05), residual biases N(0, 0.01),
activations N(0, 1)) is the one the workload descriptions state.
"""
from __future__ import annotations

import dataclasses
import zlib
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class ZayaConfig:
    """Shape and workload of one block (or stack) call.

    Field names follow the HF config keys listed on the nnterp page ("Config").
    """

    name: str
    hidden_size: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    rope_dim: int
    rope_theta: float
    num_experts: int
    moe_intermediate_size: int
    router_hidden: int
    act_dtype: str  # "bf16" or "f32"
    batch: int
    seq: int
    conv_k: int = 3  # 3: one depthwise kernel-3 conv; 2: the printout's depthwise k2 then grouped k2
    rms_norm_eps: float = 1e-5
    sliding_window: int = -1  # < 0: off; else key visible iff p_q - p_k <= window
    window_layers: int = 0  # stacks: 0 all blocks windowed, 1 blocks 0, 2, ..., 2 blocks 1, 3, ...
    kv_len: int = 0  # tokens already in the cache before this call
    decode: bool = False
    num_layers: int = 1
    vocab_size: int = 0
    has_router_state: bool = True  # False: block-0 semantics (no carried state)
    temp_range: tuple = (0.8, 2.0)  # key temperature drawn U(lo, hi); (1, 1) = ones
    conv_std: float = 0.02  # std of the conv taps and bias
    conv2_std: float = 0.02  # std of the grouped conv stage's taps and bias (conv_k == 2)
    gain_std: float = 0.0  # RMSNorm gains: 1 + N(0, gain_std); 0 = ones
    bal_bias: str = "zeros"  # "zeros", "normal", "trained", "zipf"
    expert_format: str = "act"  # "act" or "fp8": expert weights stored as E4M3 bytes + fp32 row scales
    # "rows": the expert weights go to the block library row-major, as drawn; "packed": the
    # library lays them out in its packed form (zaya_pack_experts) before the runs
    expert_layout: str = "rows"

    @property
    def conv_channels(self) -> int:
        return (self.num_heads + self.num_kv_heads) * self.head_dim

    @property
    def qkv_rows(self) -> int:
        return self.num_heads * self.head_dim + 2 * self.num_kv_heads * self.head_dim

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.act_dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "ZayaConfig":
        return dataclasses.replace(self, **kw)


# --- the five workloads -------------------------------------------------------

def _full(**kw) -> dict:
    base = dict(hidden_size=2048, num_heads=8, num_kv_heads=2, head_dim=128, rope_dim=64,
                rope_theta=1e6, num_experts=16, moe_intermediate_size=2048, router_hidden=256,
                act_dtype="bf16", expert_layout="packed")
    base.update(kw)
    return base


CONFIGS: Dict[str, ZayaConfig] = {
    # tiny fp32 block, B1 S64 (hidden 256, 4 q / 1 kv heads of 64, rope 32 dims, theta 1e4,
    # 4 experts of width 512, router width 256), key temperature one, vocab 1000
    "tiny": ZayaConfig(name="tiny", hidden_size=256, num_heads=4, num_kv_heads=1, head_dim=64,
                       rope_dim=32, rope_theta=1e4, num_experts=4, moe_intermediate_size=512,
                       router_hidden=256, act_dtype="f32", batch=1, seq=64, vocab_size=1000,
                       temp_range=(1.0, 1.0)),
    # one full block prefill, bf16, B1 S4096, router state fed N(0, 1)
    "prefill": ZayaConfig(name="prefill", **_full(batch=1, seq=4096)),
    # block decode, bf16, B64, 8192 cached tokens, one new token each
    "decode": ZayaConfig(name="decode", **_full(batch=64, seq=1, kv_len=8192, decode=True)),
    # the same decode step with the expert weights stored as FP8 E4M3 + fp32 row scales
    "decode_fp8": ZayaConfig(name="decode_fp8", **_full(batch=64, seq=1, kv_len=8192, decode=True,
                                                        expert_format="fp8")),
    # the prefill workload with the printout's two-stage q/k convolution (depthwise k2, then
    # grouped k2 with one group per head)
    "prefill_conv2": ZayaConfig(name="prefill_conv2", **_full(batch=1, seq=4096, conv_k=2)),
    # 40-block stack prefill, bf16, B4 S2048, vocab 262144
    "stack": ZayaConfig(name="stack", **_full(batch=4, seq=2048, num_layers=40, vocab_size=262144)),
    # long-context prefill, bf16, B1 S32768, window 4096, Zipf(1.2) expert load + 15% skip
    "longctx": ZayaConfig(name="longctx", **_full(batch=1, seq=32768, sliding_window=4096,
                                                  bal_bias="zipf")),
}


# --- random streams ----------------------------------------------------------

def _stream(seed: int, cfg_name: str, block: int, tensor: str) -> np.random.Generator:
    key = [int(seed), zlib.crc32(cfg_name.encode()), int(block) + 1, zlib.crc32(tensor.encode())]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def normal(seed, cfg_name, block, tensor, shape, mean=0.0, std=1.0) -> np.ndarray:
    g = _stream(seed, cfg_name, block, tensor)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def uniform(seed, cfg_name, block, tensor, shape, lo, hi) -> np.ndarray:
    g = _stream(seed, cfg_name, block, tensor)
    return g.uniform(lo, hi, size=shape).astype(np.float32)


def integers(seed, cfg_name, block, tensor, shape, lo, hi) -> np.ndarray:
    g = _stream(seed, cfg_name, block, tensor)
    return g.integers(lo, hi, size=shape, dtype=np.int64).astype(np.int32)


def _act(a: np.ndarray, cfg: ZayaConfig) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(cfg.torch_dtype)


def _f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


# --- weights -----------------------------------------------------------------

BLOCK_TENSORS = (
    "ln1_g", "W_qkv", "conv_w", "conv_b", "temp", "W_o",
    "a_hsb", "a_hss", "a_rb", "a_rs", "ln2_g",
    "r_Wd", "r_bd", "r_rss", "r_norm_g", "r_W1", "r_b1", "r_W2", "r_b2", "r_Wout",
    "bal_bias", "W_gu", "W_dn", "m_hsb", "m_hss", "m_rb", "m_rs",
)


def block_weight_shapes(cfg: ZayaConfig) -> Dict[str, tuple]:
    """Shape of every tensor of one block (the ones ``block_weights`` draws)."""
    H, nh, nkv, d = cfg.hidden_size, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    E, I, R, C = cfg.num_experts, cfg.moe_intermediate_size, cfg.router_hidden, cfg.conv_channels
    return {
        "ln1_g": (H,), "W_qkv": (cfg.qkv_rows, H), "conv_w": (C, cfg.conv_k), "conv_b": (C,),
        "temp": (nkv,), "W_o": (H, nh * d),
        "a_hsb": (H,), "a_hss": (H,), "a_rb": (H,), "a_rs": (H,), "ln2_g": (H,),
        "r_Wd": (R, H), "r_bd": (R,), "r_rss": (R,), "r_norm_g": (R,), "r_W1": (R, R),
        "r_b1": (R,), "r_W2": (R, R), "r_b2": (R,), "r_Wout": (E + 1, R), "bal_bias": (E + 1,),
        "W_gu": (E, 2 * I, H), "W_dn": (E, H, I),
        "m_hsb": (H,), "m_hss": (H,), "m_rb": (H,), "m_rs": (H,),
        **({"conv2_w": (C, 2, d), "conv2_b": (C,)} if cfg.conv_k == 2 else {}),
    }


def block_weights(cfg: ZayaConfig, block: int = 0, seed: int = 0,
                  bal_bias: Optional[np.ndarray] = None) -> Dict[str, torch.Tensor]:
    """Random-init weights of one decoder block, as CPU tensors of the act dtype.

    ``bal_bias`` is fp32 [E+1]. ``W_gu`` is [E, 2I, H] (gate rows, then up rows) and
    ``W_dn`` is [E, H, I]: the pre-stacked expert layout the pages describe.
    """
    H, nh, nkv, d = cfg.hidden_size, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    E, I, R, C = cfg.num_experts, cfg.moe_intermediate_size, cfg.router_hidden, cfg.conv_channels
    n = cfg.name

    def N(t, shape, mean=0.0, std=0.02):
        return _act(normal(seed, n, block, t, shape, mean, std), cfg)

    def gain(t, shape):
        if cfg.gain_std == 0.0:
            return _act(np.ones(shape, np.float32), cfg)
        return N(t, shape, 1.0, cfg.gain_std)

    lo, hi = cfg.temp_range
    temp = np.full((nkv,), lo, np.float32) if lo == hi else uniform(seed, n, block, "temp", (nkv,), lo, hi)
    w = {
        "ln1_g": gain("ln1_g", (H,)),
        "W_qkv": N("W_qkv", (cfg.qkv_rows, H)),
        "conv_w": N("conv_w", (C, cfg.conv_k), std=cfg.conv_std),
        "conv_b": N("conv_b", (C,), std=cfg.conv_std),
        "temp": _act(temp, cfg),
        "W_o": N("W_o", (H, nh * d)),
        "a_hsb": N("a_hsb", (H,), std=0.01),
        "a_hss": N("a_hss", (H,), 1.0, 0.05),
        "a_rb": N("a_rb", (H,), std=0.01),
        "a_rs": N("a_rs", (H,), 1.0, 0.05),
        "ln2_g": gain("ln2_g", (H,)),
        "r_Wd": N("r_Wd", (R, H)),
        "r_bd": N("r_bd", (R,)),
        "r_rss": N("r_rss", (R,), 1.0, 0.05),
        "r_norm_g": gain("r_norm_g", (R,)),
        "r_W1": N("r_W1", (R, R)),
        "r_b1": N("r_b1", (R,)),
        "r_W2": N("r_W2", (R, R)),
        "r_b2": N("r_b2", (R,)),
        "r_Wout": N("r_Wout", (E + 1, R)),
        "W_gu": N("W_gu", (E, 2 * I, H)),
        "W_dn": N("W_dn", (E, H, I)),
        "m_hsb": N("m_hsb", (H,), std=0.01),
        "m_hss": N("m_hss", (H,), 1.0, 0.05),
        "m_rb": N("m_rb", (H,), std=0.01),
        "m_rs": N("m_rs", (H,), 1.0, 0.05),
    }
    if cfg.conv_k == 2:  # grouped stage: [C, tap, d] (output channel, tap, input channel of its head)
        w["conv2_w"] = N("conv2_w", (C, 2, d), std=cfg.conv2_std)
        w["conv2_b"] = N("conv2_b", (C,), std=cfg.conv2_std)
    if bal_bias is not None:
        bb = np.asarray(bal_bias, np.float32)
    elif cfg.bal_bias == "normal":
        bb = normal(seed, n, block, "bal_bias", (E + 1,), 0.0, 0.01)
    elif cfg.bal_bias == "trained":
        # the pattern the pages report for the trained model: -1 on skip, one expert above 0
        bb = np.zeros(E + 1, np.float32)
        bb[E] = -1.0
        bb[block % E] = 0.1
    else:
        bb = np.zeros(E + 1, np.float32)
    # the buffer holds bf16-representable values
    w["bal_bias"] = torch.from_numpy(bb).to(torch.bfloat16).float()
    if cfg.expert_format == "fp8":
        w.update(fp8_rows(w.pop("W_gu"), "W_gu"))
        w.update(fp8_rows(w.pop("W_dn"), "W_dn"))
    return w


def fp8_rows(W: torch.Tensor, name: str) -> Dict[str, torch.Tensor]:
    """Storage of a weight tensor as OCP FP8 E4M3 bytes with one fp32 scale per row
    (last dimension = row): scale = max|row| / 448 (448 is the largest E4M3 value), the
    bytes are torch's round-to-nearest conversion of row / scale. Returns
    {name: uint8 tensor of W's shape, name + "_scale": fp32 tensor of W.shape[:-1]}.
    This is how the synthetic weights are stored; the dequantization (byte value times
    scale) is the block's arithmetic and is not done here."""
    Wf = W.float()
    amax = Wf.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (Wf / scale.unsqueeze(-1)).to(torch.float8_e4m3fn)
    return {name: q.view(torch.uint8).contiguous(), name + "_scale": scale.contiguous()}


def _device_stream(seed: int, cfg_name: str, block: int, tensor: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    key = (int(seed) * 1000003 + zlib.crc32(cfg_name.encode()) * 8191 + (int(block) + 1) * 131
           + zlib.crc32(tensor.encode())) % (2 ** 63)
    g.manual_seed(key)
    return g


def block_weights_device(cfg: ZayaConfig, block: int = 0, seed: int = 0, device="cuda") -> Dict[str, torch.Tensor]:
    """The same recipe as ``block_weights`` drawn directly on the device (torch's own
    counter-based generator, one stream per tensor): for large stacks, where drawing
    40 blocks on the host takes minutes. Values differ from ``block_weights``; every
    consumer of a run reads the same tensors."""
    shapes = block_weight_shapes(cfg)
    dt = cfg.torch_dtype
    n = cfg.name

    def N(t, mean=0.0, std=0.02):
        x = torch.randn(shapes[t], generator=_device_stream(seed, n, block, t, device), device=device,
                        dtype=torch.float32)
        return (x * std + mean).to(dt)

    def gain(t):
        return torch.ones(shapes[t], device=device, dtype=dt) if cfg.gain_std == 0.0 else N(t, 1.0, cfg.gain_std)

    lo, hi = cfg.temp_range
    tg = _device_stream(seed, n, block, "temp", device)
    temp = torch.rand(shapes["temp"], generator=tg, device=device) * (hi - lo) + lo
    w = {
        "ln1_g": gain("ln1_g"), "W_qkv": N("W_qkv"), "conv_w": N("conv_w", std=cfg.conv_std),
        "conv_b": N("conv_b", std=cfg.conv_std), "temp": temp.to(dt), "W_o": N("W_o"),
        "a_hsb": N("a_hsb", std=0.01), "a_hss": N("a_hss", 1.0, 0.05), "a_rb": N("a_rb", std=0.01),
        "a_rs": N("a_rs", 1.0, 0.05), "ln2_g": gain("ln2_g"),
        "r_Wd": N("r_Wd"), "r_bd": N("r_bd"), "r_rss": N("r_rss", 1.0, 0.05), "r_norm_g": gain("r_norm_g"),
        "r_W1": N("r_W1"), "r_b1": N("r_b1"), "r_W2": N("r_W2"), "r_b2": N("r_b2"), "r_Wout": N("r_Wout"),
        "W_gu": N("W_gu"), "W_dn": N("W_dn"),
        "m_hsb": N("m_hsb", std=0.01), "m_hss": N("m_hss", 1.0, 0.05), "m_rb": N("m_rb", std=0.01),
        "m_rs": N("m_rs", 1.0, 0.05),
        "bal_bias": torch.zeros(shapes["bal_bias"], device=device, dtype=torch.float32),
    }
    if cfg.conv_k == 2:
        w["conv2_w"] = N("conv2_w", std=cfg.conv2_std)
        w["conv2_b"] = N("conv2_b", std=cfg.conv2_std)
    return w


def stack_weights_device(cfg: ZayaConfig, seed: int = 0, device="cuda") -> Dict[str, torch.Tensor]:
    """Embedding, shift/scale and final norm gain drawn on the device (see
    ``block_weights_device``)."""
    H, V, n, dt = cfg.hidden_size, cfg.vocab_size, cfg.name, cfg.torch_dtype

    def N(t, shape, mean, std):
        x = torch.randn(shape, generator=_device_stream(seed, n, -1, t, device), device=device, dtype=torch.float32)
        return (x * std + mean).to(dt)

    return {"embed": N("embed", (V, H), 0.0, 0.02), "emb_shift": N("emb_shift", (H,), 0.0, 0.01),
            "emb_scale": N("emb_scale", (H,), 1.0, 0.05), "final_g": torch.ones(H, device=device, dtype=dt)}


def stack_weights(cfg: ZayaConfig, seed: int = 0) -> Dict[str, torch.Tensor]:
    """Embedding (tied with lm_head), its shift/scale, and the final norm gain."""
    H, V, n = cfg.hidden_size, cfg.vocab_size, cfg.name
    out = {
        "embed": _act(normal(seed, n, -1, "embed", (V, H), 0.0, 0.02), cfg),
        "emb_shift": _act(normal(seed, n, -1, "emb_shift", (H,), 0.0, 0.01), cfg),
        "emb_scale": _act(normal(seed, n, -1, "emb_scale", (H,), 1.0, 0.05), cfg),
    }
    if cfg.gain_std == 0.0:
        out["final_g"] = _act(np.ones(H, np.float32), cfg)
    else:
        out["final_g"] = _act(normal(seed, n, -1, "final_g", (H,), 1.0, cfg.gain_std), cfg)
    return out


# --- activations and state ---------------------------------------------------

def block_inputs(cfg: ZayaConfig, block: int = 0, seed: int = 0) -> Dict[str, torch.Tensor]:
    """Stream input x (fp32), carried router state, and the decode cache state.

    Cache tensors are allocated with capacity ``kv_len + seq`` and filled N(0, 1)
    up to ``kv_len``; positions beyond hold zeros.
    """
    B, S, H, R = cfg.batch, cfg.seq, cfg.hidden_size, cfg.router_hidden
    nkv, d, C = cfg.num_kv_heads, cfg.head_dim, cfg.conv_channels
    n = cfg.name
    out = {"x": _f32(normal(seed, n, block, "x", (B, S, H)))}
    if cfg.has_router_state:
        out["s_in"] = _act(normal(seed, n, block, "s_in", (B, S, R)), cfg)
    cap = cfg.kv_len + S
    K = torch.zeros((B, nkv, cap, d), dtype=cfg.torch_dtype)
    V = torch.zeros((B, nkv, cap, d), dtype=cfg.torch_dtype)
    if cfg.kv_len > 0:
        K[:, :, :cfg.kv_len] = _act(normal(seed, n, block, "K_cache", (B, nkv, cfg.kv_len, d)), cfg)
        V[:, :, :cfg.kv_len] = _act(normal(seed, n, block, "V_cache", (B, nkv, cfg.kv_len, d)), cfg)
        conv = _act(normal(seed, n, block, "conv_state", (B, C, 2)), cfg)
        prev = _act(normal(seed, n, block, "prev_hs", (B, H)), cfg)
    else:
        conv = torch.zeros((B, C, 2), dtype=cfg.torch_dtype)
        prev = torch.zeros((B, H), dtype=cfg.torch_dtype)
    out.update(K=K, V=V, conv_state=conv, prev_hs=prev,
               cache_len=torch.full((B,), cfg.kv_len, dtype=torch.int32))
    return out


def token_ids(cfg: ZayaConfig, seed: int = 0) -> torch.Tensor:
    return torch.from_numpy(integers(seed, cfg.name, -1, "ids", (cfg.batch, cfg.seq), 0, cfg.vocab_size))
