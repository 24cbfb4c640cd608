"""Seeded synthetic workloads for mixed retrieval/streaming KV attention.

This module holds the workload shapes and the seeded random-number recipe that
both the CPU oracle and the HIP path are fed from.  It contains none of the
attention arithmetic: no visibility rule, no softmax, no cache slot placement.

Recipe (every tensor):
  * values are drawn as float32 standard normals from numpy's PCG64, seeded by
    ``SeedSequence([241010819, cfg_index, layer, batch, head, tensor_id, block])``
    where tensor_id is 0=Q, 1=K, 2=V, 3=mask, 4=gate and ``block`` counts GEN_BLOCK-row
    slabs along the position axis, so any position range can be regenerated on
    its own;
  * for workloads that say so, the K rows of the first ``sink`` positions are
    multiplied by 4 (exact in binary) to mimic attention-sink tokens;
  * values are then rounded to the workload's storage dtype (bf16 by
    round-to-nearest-even through torch, or kept as float32).

The retrieval/streaming role of each KV head is drawn per layer with the same
seeding (tensor_id 3): a seeded permutation of the KV heads whose first
``n_ret`` entries are the retrieval heads.

Head gates (one per KV head and layer, for the gated full/streaming forward)
are float32 uniforms on [0, 1) from the same seeding (tensor_id 4).

The five cache workloads follow the shapes the DuoAttention pages use as examples
(a LLaMA-3-8B-like GQA layer, a 7B MHA model, a 70B GQA model at 128k context,
and a chunked prefill), plus one gated-forward workload on the LLaMA-3-8B layer
shape, with synthetic values standing in for model
activations: no weights or datasets are involved.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

SEED_ROOT = 241010819
GEN_BLOCK = 4096  # rows per independently seeded slab along the position axis
TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_MASK, TENSOR_GATE = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int              # cfg_index used in the seed
    L: int                  # layers
    B: int                  # batch
    n_q: int                # query heads
    n_kv: int               # KV heads
    d: int                  # head dim
    dtype: str              # "f32" or "bf16" (Q, K, V and output)
    T: int                  # context length at the measured step
    S: int                  # attention-sink tokens kept by streaming heads
    W: int                  # recent-window tokens kept by streaming heads
    n_ret: int              # retrieval KV heads per layer
    sink_scale: float       # multiplier on K rows at positions < S (1.0 = none)
    mode: str               # "decode" | "decode_append" | "prefill" | "gated"
    chunk: int = 0          # prefill chunk length
    fixed_mask: Optional[tuple] = None  # explicit per-layer mask rows, else seeded
    kv_format: Optional[str] = None     # "fp8" / "int4": K/V rows stored as low-bit codes + row scales
    page_rows: int = 0                  # > 0: retrieval rows in pages of this many rows
    rope_theta: float = 0.0             # > 0: rotary positions with this base
    forked: bool = False                # rows 1 .. B-1 forked from row 0's prefix (paged: its full pages shared)

    @property
    def g(self) -> int:
        return self.n_q // self.n_kv

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def kv_row_bytes(self) -> int:
        """Bytes of one stored K (or V) row: d elements, plus an fp32 scale for
        FP8 rows (one byte per element) and INT4 rows (two elements per byte)."""
        if self.kv_format == "fp8":
            return self.d + 4
        if self.kv_format == "int4":
            return self.d // 2 + 4
        return self.d * self.elem_bytes

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # 1 layer, GQA group 2, fp32, T=512; KV head 0 retrieval, KV head 1 streaming.
    "tiny_decode": Workload("tiny_decode", 0, L=1, B=1, n_q=4, n_kv=2, d=64, dtype="f32",
                            T=512, S=4, W=64, n_ret=1, sink_scale=4.0, mode="decode",
                            fixed_mask=((1, 0),)),
    # LLaMA-3-8B-shaped layer, batch 8, 32k context, 2 of 8 KV heads retrieval.
    "llama3_8b_decode_b8_32k": Workload("llama3_8b_decode_b8_32k", 1, L=1, B=8, n_q=32, n_kv=8,
                                        d=128, dtype="bf16", T=32768, S=32, W=1024, n_ret=2,
                                        sink_scale=4.0, mode="decode"),
    # 7B MHA-shaped model, 32 layers, 128k context, half the heads retrieval; one new token appended.
    "mha7b_decode_128k": Workload("mha7b_decode_128k", 2, L=32, B=1, n_q=32, n_kv=32, d=128,
                                  dtype="bf16", T=131072, S=64, W=1024, n_ret=16,
                                  sink_scale=1.0, mode="decode_append"),
    # 70B GQA shape, 80 layers, 128,000 context, 2 of 8 KV heads retrieval; one new token appended.
    "gqa70b_decode_128k": Workload("gqa70b_decode_128k", 3, L=80, B=1, n_q=64, n_kv=8, d=128,
                                   dtype="bf16", T=128000, S=64, W=1024, n_ret=2,
                                   sink_scale=1.0, mode="decode_append"),
    # Chunked prefill of one LLaMA-3-8B-shaped layer: 65,536 tokens in 4,096-token chunks.
    "llama3_8b_prefill_64k": Workload("llama3_8b_prefill_64k", 4, L=1, B=1, n_q=32, n_kv=8, d=128,
                                      dtype="bf16", T=65536, S=64, W=1024, n_ret=2,
                                      sink_scale=1.0, mode="prefill", chunk=4096),
    # Gated full/streaming forward over one 32,768-token sequence of a LLaMA-3-8B-shaped layer
    # (one gate per KV head; the retrieval mask does not apply).
    "llama3_8b_gated_32k": Workload("llama3_8b_gated_32k", 5, L=1, B=1, n_q=32, n_kv=8, d=128,
                                    dtype="bf16", T=32768, S=64, W=1024, n_ret=0,
                                    sink_scale=1.0, mode="gated"),
}
# The two 128k decode workloads again with the cache's K/V rows stored as FP8
# and as INT4 (same shapes and inputs).
for _n in ("gqa70b_decode_128k", "mha7b_decode_128k"):
    WORKLOADS[_n + "_fp8"] = WORKLOADS[_n].with_(name=_n + "_fp8", kv_format="fp8")
    WORKLOADS[_n + "_int4"] = WORKLOADS[_n].with_(name=_n + "_int4", kv_format="int4")
# The 70B decode again with the retrieval rows in 256-row pages (same shapes
# and inputs; the pool holds exactly the rows the batch needs).
WORKLOADS["gqa70b_decode_128k_paged"] = WORKLOADS["gqa70b_decode_128k"].with_(name="gqa70b_decode_128k_paged",
                                                                            page_rows=256)
# Two requests that share a 128k prefix (row 1 forked from row 0 in every
# layer, the prefix's full 256-row pages shared) against the same two rows
# held apart: the shared pages are read once per step for both rows.
WORKLOADS["gqa70b_decode_128k_b2_forked"] = WORKLOADS["gqa70b_decode_128k"].with_(
    name="gqa70b_decode_128k_b2_forked", B=2, page_rows=256, forked=True)
WORKLOADS["gqa70b_decode_128k_b2_paged"] = WORKLOADS["gqa70b_decode_128k"].with_(
    name="gqa70b_decode_128k_b2_paged", B=2, page_rows=256)
# ... and with rotary positions (base 500,000, as LLaMA-3 checkpoints use).
WORKLOADS["gqa70b_decode_128k_rope"] = WORKLOADS["gqa70b_decode_128k"].with_(name="gqa70b_decode_128k_rope",
                                                                           rope_theta=500000.0)
# The two 128k decodes with every KV head a retrieval head: full attention
# through the same kernels, the reference point of the decode speedup the
# DuoAttention guide claims.
for _n in ("gqa70b_decode_128k", "mha7b_decode_128k"):
    WORKLOADS[_n + "_full"] = WORKLOADS[_n].with_(name=_n + "_full", n_ret=WORKLOADS[_n].n_kv)
# Workloads that run on the mixed cache in the cache dtype, contiguous (the
# gated forward runs on none, the FP8 and paged variants repeat shapes
# already listed).
ORDER: List[str] = [n for n, w in WORKLOADS.items()
                    if w.mode != "gated" and w.kv_format is None and w.page_rows == 0 and w.rope_theta == 0
                    and not n.endswith("_full")]


def _rng(w: Workload, layer: int, b: int, head: int, tensor_id: int, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence([SEED_ROOT, w.index, layer, b, head, tensor_id, block])
    return np.random.Generator(np.random.PCG64(ss))


def retrieval_mask(w: Workload, layer: int) -> np.ndarray:
    """uint8 [n_kv], 1 = retrieval head, for one layer."""
    if w.fixed_mask is not None:
        return np.asarray(w.fixed_mask[layer % len(w.fixed_mask)], dtype=np.uint8)
    perm = _rng(w, layer, 0, 0, TENSOR_MASK, 0).permutation(w.n_kv)
    m = np.zeros(w.n_kv, dtype=np.uint8)
    m[perm[: w.n_ret]] = 1
    return m


def mask_table(w: Workload, layers: Optional[int] = None) -> np.ndarray:
    """uint8 [L][n_kv] retrieval mask."""
    L = w.L if layers is None else layers
    return np.stack([retrieval_mask(w, l) for l in range(L)])


def gate_values(w: Workload, layer: int) -> np.ndarray:
    """Seeded head gates for one layer: float32 uniforms on [0, 1), one per KV head."""
    return _rng(w, layer, 0, 0, TENSOR_GATE, 0).uniform(0.0, 1.0, w.n_kv).astype(np.float32)


def rows_f32(w: Workload, layer: int, b: int, head: int, tensor_id: int, p0: int, p1: int) -> np.ndarray:
    """float32 [p1-p0][d] rows for positions p0..p1-1 of one head's Q, K or V stream.

    Positions index the token sequence; the sink multiplier is applied to K rows
    at positions < S when the workload asks for it.  Values are not yet rounded.
    """
    out = np.empty((max(p1 - p0, 0), w.d), dtype=np.float32)
    if p1 <= p0:
        return out
    for blk in range(p0 // GEN_BLOCK, (p1 - 1) // GEN_BLOCK + 1):
        b0 = blk * GEN_BLOCK
        slab = _rng(w, layer, b, head, tensor_id, blk).standard_normal((GEN_BLOCK, w.d), dtype=np.float32)
        lo, hi = max(p0, b0), min(p1, b0 + GEN_BLOCK)
        out[lo - p0: hi - p0] = slab[lo - b0: hi - b0]
    if tensor_id == TENSOR_K and w.sink_scale != 1.0 and p0 < w.S:
        out[: min(w.S, p1) - p0] *= np.float32(w.sink_scale)
    return out


def round_to_dtype(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype and return them as float64
    (bf16 upcasts exactly).  bf16 rounding is torch's round-to-nearest-even."""
    if dtype == "f32":
        return x_f32.astype(np.float64)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def to_torch(x_f32: np.ndarray, dtype: str):
    """Storage tensor (CPU) in the workload dtype from float32 values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def head_rows(w: Workload, layer: int, b: int, head: int, tensor_id: int, p0: int, p1: int) -> np.ndarray:
    """Rows as the stored values, upcast to float64."""
    return round_to_dtype(rows_f32(w, layer, b, head, tensor_id, p0, p1), w.dtype)


def stacked_rows_f32(w: Workload, layer: int, tensor_id: int, heads: int, p0: int, p1: int,
                     batches: Optional[Sequence[int]] = None) -> np.ndarray:
    """float32 [B][heads][p1-p0][d] for one layer."""
    bs = range(w.B) if batches is None else batches
    return np.stack([np.stack([rows_f32(w, layer, b, h, tensor_id, p0, p1) for h in range(heads)])
                     for b in bs])


def normal_f32(shape, seed: int) -> np.ndarray:
    """float32 standard normals for ad-hoc test shapes, seeded like the
    workloads (SeedSequence([SEED_ROOT, 1000, seed]))."""
    ss = np.random.SeedSequence([SEED_ROOT, 1000, int(seed)])
    return np.random.Generator(np.random.PCG64(ss)).standard_normal(shape, dtype=np.float32)


def device_fill_normal(t, seed: int, sink_rows: int = 0, sink_scale: float = 1.0):
    """Fill a device tensor [..., positions, d] with seeded standard normals from
    torch's device generator (used where host generation would take minutes,
    e.g. filling a 32-layer 128k-context cache); optional sink multiplier on the
    first ``sink_rows`` positions."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    tmp = torch.randn(t.shape, generator=g, device=t.device, dtype=torch.float32)
    if sink_rows > 0 and sink_scale != 1.0:
        tmp[..., :sink_rows, :] *= sink_scale
    t.copy_(tmp)
    return t


def device_seed(w: Workload, layer: int, tensor_id: int, block: int = 0) -> int:
    """Integer seed for the device generator, keyed like the host recipe."""
    ss = np.random.SeedSequence([SEED_ROOT, w.index, layer, 0, 0, tensor_id, block, 1])
    return int(ss.generate_state(1, dtype=np.uint64)[0])
