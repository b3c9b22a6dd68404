"""Seeded synthetic workloads (inputs only: no step of the method lives here).

Llama-shaped K/V/q stand in for real activations, which are not available:
  K[t, h, j] = z * s[h, j], z ~ N(0, 1); s[h, j] = exp(0.5 * zeta), zeta ~ N(0, 1),
              fixed per (layer, KV head, channel); 4 outlier channels per
              (layer, head), drawn without replacement, get s * 10.
  V ~ N(0, 1), q ~ N(0, 1).
Values are drawn in fp32 and rounded to nearest-even bf16 unless the workload
is fp32. Paged caches use 16-token blocks; block tables are shuffled so that
logical neighbours are physically apart.

Both the oracle side and the GPU side of every test take their inputs from
here; the numbers the method itself draws (rotation, QJL matrix, WHT signs) are
not drawn here.
"""
from dataclasses import dataclass, field

import numpy as np

BLOCK = 16


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returned as fp32."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of fp32 values that are already bf16-exact."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@dataclass
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_lens: list
    capacity_tokens: int          # per sequence (block table width * 16)
    bits: int = 4
    dtype: str = "bf16"           # "f32" or "bf16" K/V/q
    rotation: str = "haar"
    num_splits: int = 0           # 0 = let the library choose
    layers: int = 1
    notes: str = ""
    extra: dict = field(default_factory=dict)


def workload(index: int, **over) -> Workload:
    """The five configurations (index 0..4)."""
    if index == 0:
        w = Workload("tiny-1head-256tok-f32", 1, 1, 1, 128, [256], 256, dtype="f32")
    elif index == 1:
        w = Workload("llama3-8b-layer-b1-ctx4096", 1, 32, 8, 128, [4096], 4096)
    elif index == 2:
        rs = np.random.default_rng(1002)
        lens = rs.integers(3072, 4096, size=32, endpoint=True).tolist()
        w = Workload("llama3-8b-layer-b32-ctx3072to4096", 32, 32, 8, 128, lens, 4096, num_splits=4)
    elif index == 3:
        w = Workload("llama3.1-70b-layer-b1-ctx32768", 1, 64, 8, 128, [32768], 32768)
    elif index == 4:
        w = Workload("70b-80layer-stream-ctx32768", 4, 64, 8, 128, [32768] * 4, 32768, layers=80)
    else:
        raise ValueError(index)
    for k, v in over.items():
        setattr(w, k, v)
    return w


def channel_scales(rng: np.random.Generator, num_kv_heads: int, d: int) -> np.ndarray:
    """Per-(head, channel) K scales: log-normal(0, 0.5) with 4 outlier channels x10."""
    s = np.exp(0.5 * rng.standard_normal((num_kv_heads, d))).astype(np.float32)
    for h in range(num_kv_heads):
        out = rng.choice(d, size=4, replace=False)
        s[h, out] *= 10.0
    return s


def kv_tensors(seed: int, tokens: int, num_kv_heads: int, d: int, dtype: str = "bf16"):
    """K, V [tokens, Hkv, d] (fp32 arrays holding bf16-exact values unless dtype == 'f32')."""
    rng = np.random.default_rng(seed)
    s = channel_scales(rng, num_kv_heads, d)
    k = (rng.standard_normal((tokens, num_kv_heads, d), dtype=np.float32) * s[None]).astype(np.float32)
    v = rng.standard_normal((tokens, num_kv_heads, d), dtype=np.float32)
    if dtype == "bf16":
        k, v = bf16_round(k), bf16_round(v)
    return k, v


def queries(seed: int, batch: int, num_q_heads: int, d: int, dtype: str = "bf16"):
    q = np.random.default_rng(seed).standard_normal((batch, num_q_heads, d), dtype=np.float32)
    return bf16_round(q) if dtype == "bf16" else q


def block_tables(seed: int, seq_lens, capacity_tokens: int, pool_blocks: int = None):
    """Non-contiguous block tables drawn from one shuffled pool.

    Every sequence gets capacity_tokens / 16 distinct physical blocks; the pool
    holds exactly batch * that many blocks unless pool_blocks is larger.
    Returns (block_tables int32 [B, max_blocks], num_blocks).
    """
    B = len(seq_lens)
    per = capacity_tokens // BLOCK
    total = B * per if pool_blocks is None else pool_blocks
    perm = np.random.default_rng(seed).permutation(total).astype(np.int32)
    return perm[: B * per].reshape(B, per).copy(), total


def slot_mapping_for(block_table_row: np.ndarray, seq_len: int) -> np.ndarray:
    """Slots (block * 16 + offset) of tokens 0..seq_len-1 of one sequence."""
    t = np.arange(seq_len)
    return block_table_row[t // BLOCK].astype(np.int64) * BLOCK + t % BLOCK


def layer_inputs(w: Workload, layer: int = 0, data_seed: int = None):
    """Everything one layer of a workload needs, on the host.

    Returns dict with k, v ([B, capacity, Hkv, d] fp32 arrays; tokens past a
    sequence's length are present but never written), q [B, Hq, d],
    block_tables [B, max_blocks] int32, seq_lens int32 [B], num_blocks,
    slot_mapping [B * capacity] int64 (-1 for tokens past a sequence's length).
    """
    seed = (1000 + layer * 7919) if data_seed is None else data_seed
    B, d = w.batch, w.head_dim
    cap = w.capacity_tokens
    k, v = kv_tensors(seed, B * cap, w.num_kv_heads, d, w.dtype)
    q = queries(seed + 1, B, w.num_q_heads, d, w.dtype)
    bt, nb = block_tables(seed + 2, w.seq_lens, cap)
    slots = np.full((B, cap), -1, dtype=np.int64)
    for b in range(B):
        L = int(w.seq_lens[b])
        slots[b, :L] = slot_mapping_for(bt[b], L)
    return {
        "k": k.reshape(B, cap, w.num_kv_heads, d),
        "v": v.reshape(B, cap, w.num_kv_heads, d),
        "q": q,
        "block_tables": bt,
        "seq_lens": np.asarray(w.seq_lens, dtype=np.int32),
        "num_blocks": nb,
        "slot_mapping": slots.reshape(-1),
    }


def kv_device(seed: int, tokens: int, num_kv_heads: int, d: int, device="cuda", dtype="bf16"):
    """Device-side K, V [tokens, Hkv, d] with the same recipe (torch generator on the device)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    s = torch.exp(0.5 * torch.randn((num_kv_heads, d), generator=g, device=device))
    out_idx = torch.argsort(torch.rand((num_kv_heads, d), generator=g, device=device), dim=1)[:, :4]
    s.scatter_(1, out_idx, s.gather(1, out_idx) * 10.0)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = (torch.randn((tokens, num_kv_heads, d), generator=g, device=device) * s[None]).to(tdt)
    v = torch.randn((tokens, num_kv_heads, d), generator=g, device=device).to(tdt)
    return k, v
