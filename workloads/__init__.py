"""Seeded synthetic inputs for the DeepSeek-V4 DSA indexer hot path.

This module only draws random numbers and lays them out; it holds none of the
indexer's arithmetic (no score, no selection, no mxfp4 decode).  The CPU oracle
and the HIP path both consume exactly the byte arrays produced here.

Shapes follow the indexer described on the pages:
  * "xkernels #27 -- DeepSeek-V4 DSA indexer + attention" (context paragraph):
    index_n_heads 64, index_head_dim 128, top-512 (Flash) / top-1024 (Pro).
  * "xkernels #28 -- DeepSeek-V4 serving support", comment shipping the mxfp4
    paged gather: block-table paged cache of E2M1 nibbles + E8M0 group scales.

Every tensor gets its own child stream of numpy's PCG64, spawned from the
config seed in a fixed order, so a config is reproducible byte for byte.
"""
from __future__ import annotations

import dataclasses
import functools
from typing import Optional

import numpy as np

H_INDEX = 64      # index_n_heads
D_INDEX = 128     # index_head_dim
BLOCK_SIZE = 64   # paged-cache tokens per block
FP8_E4M3_MAX = 448.0

# order in which child streams are spawned; never reorder (changes every input)
_STREAMS = ("q", "k", "w", "lens", "fp4", "scale", "table", "ff", "neg", "kc4", "kcs", "aq", "sink")


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int
    B: int                 # sequences
    T: int                 # queries per sequence
    K: int                 # keys per sequence (allocated row length)
    topk: int
    dtype: str = "bf16"    # "bf16" or "fp8" (OCP e4m3 + fp32 scales)
    causal_offset: Optional[int] = None   # limit[b,t] = offset + t  (prefill)
    len_range: Optional[tuple] = None     # decode: L_b ~ U{lo..hi}, limit = L_b-1
    scale_lo: int = 118
    scale_hi: int = 136
    n_ff: int = 0          # E8M0 0xFF bytes planted in the scale array
    n_neg: int = 0         # sel_pos slots forced to -1 per row
    kcache: Optional[str] = None   # indexer keys in a paged cache: "mxfp4" or "fp8"
    kscale_lo: int = 124   # E8M0 bytes of the mxfp4 key cache
    kscale_hi: int = 130
    description: str = ""

    @property
    def rows(self) -> int:
        return self.B * self.T


CONFIGS = {
    "tiny": Config(
        "tiny", seed=0, B=1, T=4, K=256, topk=16, causal_offset=252,
        scale_lo=120, scale_hi=134, n_ff=4, n_neg=3,
        description="1 seq, T=4, K=256, limit 252+t, top-16"),
    "flash_decode": Config(
        "flash_decode", seed=1, B=32, T=1, K=8192, topk=512,
        len_range=(8192, 8192),
        description="32 seqs x 1 query, 8192 keys, top-512"),
    "flash_prefill": Config(
        "flash_prefill", seed=2, B=1, T=4096, K=4096, topk=512,
        causal_offset=0,
        description="1 seq, T=K=4096 causal, top-512"),
    "pro_decode": Config(
        "pro_decode", seed=3, B=64, T=1, K=65536, topk=1024,
        len_range=(16384, 65536),
        description="64 seqs x 1 query, context U{16384..65536}, top-1024"),
    "long_fp8_prefill": Config(
        "long_fp8_prefill", seed=4, B=1, T=2048, K=98304, topk=1024,
        dtype="fp8", causal_offset=96256,
        description="1 seq, T=2048 at causal offset 96256, K=98304, OCP e4m3, top-1024"),
    # logits straight from a paged quantized key cache (fp8 q, mxfp4 keys
    # through the block table), then the same top-k and gather
    "flash_decode_fp4": Config(
        "flash_decode_fp4", seed=5, B=32, T=1, K=8192, topk=512, dtype="fp8",
        len_range=(8192, 8192), kcache="mxfp4", n_ff=8,
        description="32 seqs x 1 query, 8192 keys in a paged mxfp4 key cache, fp8 q, top-512"),
    "pro_decode_fp4": Config(
        "pro_decode_fp4", seed=6, B=64, T=1, K=65536, topk=1024, dtype="fp8",
        len_range=(16384, 65536), kcache="mxfp4",
        description="64 seqs x 1 query, context U{16384..65536} in a paged mxfp4 key cache, "
                    "fp8 q, top-1024"),
}


def _streams(seed: int):
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {n: np.random.Generator(np.random.PCG64(c)) for n, c in zip(_STREAMS, children)}


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 storage bits (round to nearest even), done by torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _to_e4m3_bytes(x32: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn bytes (round to nearest even, saturated to +-448)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    t = t.clamp(-FP8_E4M3_MAX, FP8_E4M3_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def seq_lengths(cfg: Config) -> np.ndarray:
    """Valid keys per sequence (decode) or the key count (prefill)."""
    if cfg.len_range is None:
        return np.full(cfg.B, cfg.K, dtype=np.int64)
    lo, hi = cfg.len_range
    if lo == hi:
        return np.full(cfg.B, lo, dtype=np.int64)
    rng = _streams(cfg.seed)["lens"]
    return rng.integers(lo, hi + 1, size=cfg.B, dtype=np.int64)


def limits(cfg: Config) -> np.ndarray:
    """limit[b,t]: inclusive last valid key index of each query."""
    if cfg.causal_offset is not None:
        lim = cfg.causal_offset + np.arange(cfg.T, dtype=np.int64)
        lim = np.broadcast_to(lim, (cfg.B, cfg.T))
    else:
        lim = np.broadcast_to((seq_lengths(cfg) - 1)[:, None], (cfg.B, cfg.T))
    return np.ascontiguousarray(np.minimum(lim, cfg.K - 1), dtype=np.int32)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_inputs(cfg: Config) -> dict:
    """All host arrays for one config (uncached)."""
    s = _streams(cfg.seed)
    B, T, K, H, D = cfg.B, cfg.T, cfg.K, H_INDEX, D_INDEX
    lens = seq_lengths(cfg)
    out = {"cfg": cfg, "limit": limits(cfg), "seq_len": lens}

    qx = _normal(s["q"], (B, T, H, D))
    # keys past a sequence's length are never read: keep them zero, draw only
    # the valid ones (none at all when the keys live in an mxfp4 cache)
    kx = np.zeros((B, K if cfg.kcache != "mxfp4" else 0, D), dtype=np.float32)
    if cfg.kcache != "mxfp4":
        for b in range(B):
            kx[b, : lens[b]] = _normal(s["k"], (int(lens[b]), D))
    out["w"] = (_normal(s["w"], (B, T, H)) / np.float32(8.0)).astype(np.float32)

    if cfg.dtype == "bf16":
        out["q"] = _to_bf16_bits(qx)
        out["k"] = _to_bf16_bits(kx)
        out["q_scale"] = None
        out["k_scale"] = None
    elif cfg.dtype == "fp8":
        # per-(token,head) q scale and per-token k scale: amax / 448
        sq = (np.abs(qx).max(axis=-1) / np.float32(FP8_E4M3_MAX)).astype(np.float32)
        sk = (np.abs(kx).max(axis=-1) / np.float32(FP8_E4M3_MAX)).astype(np.float32)
        sk = np.where(sk > 0, sk, np.float32(1.0)).astype(np.float32)  # all-zero pad rows
        out["q"] = _to_e4m3_bytes(qx / sq[..., None])
        out["k"] = _to_e4m3_bytes(kx / sk[..., None])
        out["q_scale"] = sq
        out["k_scale"] = sk
    else:
        raise ValueError(cfg.dtype)
    del qx, kx

    # mxfp4 paged cache: one physical pool, a shuffled block table per sequence
    nblk = (lens + BLOCK_SIZE - 1) // BLOCK_SIZE
    NB = int(nblk.sum())
    MB = (K + BLOCK_SIZE - 1) // BLOCK_SIZE
    perm = s["table"].permutation(NB).astype(np.int32)
    table = np.zeros((B, MB), dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += int(nblk[b])
    out["kv_fp4"] = s["fp4"].integers(0, 256, size=(NB, BLOCK_SIZE, D // 2), dtype=np.uint8)
    sc = s["scale"].integers(cfg.scale_lo, cfg.scale_hi + 1, size=(NB, BLOCK_SIZE, D // 32),
                             dtype=np.uint8)
    if cfg.n_ff:
        flat = sc.reshape(-1)
        pos = s["ff"].choice(flat.size, size=cfg.n_ff, replace=False)
        flat[pos] = 0xFF
        out["ff_positions"] = np.sort(pos)
    out["kv_scale"] = sc
    out["block_table"] = table
    if cfg.kcache == "mxfp4":
        # indexer keys in their own mxfp4 pages, same block table
        out["kc"] = s["kc4"].integers(0, 256, size=(NB, BLOCK_SIZE, D // 2), dtype=np.uint8)
        kcs = s["kcs"].integers(cfg.kscale_lo, cfg.kscale_hi + 1, size=(NB, BLOCK_SIZE, D // 32),
                                dtype=np.uint8)
        if cfg.n_ff:
            flat = kcs.reshape(-1)
            flat[s["kcs"].choice(flat.size, size=cfg.n_ff, replace=False)] = 0xFF
        out["kc_scale"] = kcs
        out["k"] = None
    elif cfg.kcache == "fp8":
        # the dense fp8 keys and scales, moved into pages through the table
        kc = np.zeros((NB, BLOCK_SIZE, D), dtype=np.uint8)
        kcs = np.ones((NB, BLOCK_SIZE), dtype=np.float32)
        for b in range(B):
            p = np.arange(int(lens[b]))
            kc[table[b, p // BLOCK_SIZE], p % BLOCK_SIZE] = out["k"][b, : lens[b]]
            kcs[table[b, p // BLOCK_SIZE], p % BLOCK_SIZE] = out["k_scale"][b, : lens[b]]
        out["kc"], out["kc_scale"] = kc, kcs
    elif cfg.kcache is not None:
        raise ValueError(cfg.kcache)
    out["row_seq"] = np.repeat(np.arange(B, dtype=np.int32), T)
    out["block_size"] = BLOCK_SIZE
    if cfg.n_neg:
        out["neg_slots"] = np.stack([
            np.sort(s["neg"].choice(cfg.topk, size=cfg.n_neg, replace=False))
            for _ in range(cfg.rows)]).astype(np.int64)
    else:
        out["neg_slots"] = None
    return out


@functools.lru_cache(maxsize=2)
def inputs(name: str) -> dict:
    """Cached inputs of a named config."""
    return make_inputs(CONFIGS[name])


def custom(name="custom", seed=123, B=1, T=4, K=300, topk=16, dtype="bf16",
           causal_offset=None, len_range=None, n_ff=0, n_neg=0,
           scale_lo=118, scale_hi=136, kcache=None, kscale_lo=124, kscale_hi=130) -> dict:
    """Small ad-hoc shapes for edge-case tests (ragged tails, short rows...)."""
    if causal_offset is None and len_range is None:
        len_range = (K, K)
    return make_inputs(Config(name, seed=seed, B=B, T=T, K=K, topk=topk, dtype=dtype,
                              causal_offset=causal_offset, len_range=len_range,
                              n_ff=n_ff, n_neg=n_neg, scale_lo=scale_lo, scale_hi=scale_hi,
                              kcache=kcache, kscale_lo=kscale_lo, kscale_hi=kscale_hi))


ATTN_HEADS = 64
ATTN_Q_SIGMA = 2.0 ** -7   # scores of a few units against the configs' mxfp4 rows


@functools.lru_cache(maxsize=2)
def attention_inputs(cfg: Config, heads: int = ATTN_HEADS, q_sigma: float = ATTN_Q_SIGMA) -> dict:
    """Inputs of the sparse attention that consumes a config's selection:
    q [rows, heads, 128] bf16 bits ~ N(0, q_sigma^2), a sink logit per head
    ~ N(0, 1), and the softmax scale 1/sqrt(128). With the configs' group
    scales (E8M0 bytes 118..136) a cache row has an rms of a few hundred, so
    q_sigma = 2^-7 gives scores of a few units."""
    s = _streams(cfg.seed)
    q = _to_bf16_bits(_normal(s["aq"], (cfg.rows, heads, D_INDEX)) * np.float32(q_sigma))
    sink = _normal(s["sink"], (heads,))
    return {"q": q, "sink": sink, "scale": float(1.0 / np.sqrt(D_INDEX))}


def apply_forced_negatives(idx: np.ndarray, neg_slots) -> np.ndarray:
    """sel_pos = top-k indices with the seeded slots forced to -1 (padded slots)."""
    sel = np.array(idx, dtype=np.int32, copy=True)
    if neg_slots is not None:
        for r in range(sel.shape[0]):
            sel[r, neg_slots[r]] = -1
    return sel


def to_device(x: dict, device="cuda") -> dict:
    """Device copies of a config's arrays, typed for the binding (bf16 / fp8 / int)."""
    import torch

    def dev(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return t.view(dtype) if dtype is not None else t

    cfg = x["cfg"]
    out = {}
    if cfg.dtype == "bf16":
        out["q"] = dev(x["q"].view(np.int16), torch.bfloat16)
        out["k"] = dev(x["k"].view(np.int16), torch.bfloat16)
        out["q_scale"] = out["k_scale"] = None
    else:
        out["q"] = dev(x["q"], torch.float8_e4m3fn)
        out["k"] = dev(x["k"], torch.float8_e4m3fn) if x["k"] is not None else None
        out["q_scale"] = dev(x["q_scale"])
        out["k_scale"] = dev(x["k_scale"]) if x["k"] is not None else None
    if cfg.kcache == "mxfp4":
        out["kc"] = dev(x["kc"])
        out["kc_scale"] = dev(x["kc_scale"])
    elif cfg.kcache == "fp8":
        out["kc"] = dev(x["kc"], torch.float8_e4m3fn)
        out["kc_scale"] = dev(x["kc_scale"])
    out["w"] = dev(x["w"])
    out["limit"] = dev(x["limit"])
    out["kv_fp4"] = dev(x["kv_fp4"])
    out["kv_scale"] = dev(x["kv_scale"])
    out["block_table"] = dev(x["block_table"])
    out["row_seq"] = dev(x["row_seq"])
    return out
