"""Seeded synthetic inputs for the shard path, shared by tests and the benchmark.

This module holds shapes, distributions and random draws only: none of the
path's arithmetic.  Values come from a counter-based generator written in
plain C (inputs_gen.c, run on host threads): element (row, column) of a
tensor is SplitMix64 of its position under a key made from the seed, the
tensor and the source rank, turned into N(0, 1) by Box-Muller, then
mu + sigma * z rounded once to f32 (and f32 to bf16, nearest even).  Rows are
global token indices, so rank r's shard of partial q is rows [r*S, (r+1)*S)
of partial q's full tensor, and any rows can be drawn on any machine, with or
without a GPU; tensors for a device are drawn on the host and copied.

Workloads (one rank's shard each; shapes follow the pages' worked examples
where they give one -- vllm-ascend PR #18671 walkthrough §2: 3500 tokens
padded to 3504 over TP=16, 219 tokens per rank, hidden 8192):

  C1  tp=2,  64 tokens,          S=32,    H=512,  fp32 in, bias, replicated residual
  C2  tp=8,  1000 -> 1024 tokens, S=128,   H=4096, bf16, 24 padding rows on rank 7
  C3  tp=16, 3500 -> 3504 tokens, S=219,   H=8192, bf16, bias, 4 padding rows on rank 15
  C4  tp=8,  65536 tokens,       S=8192,  H=7168, bf16 in, e4m3 out, static scale
  C5  tp=4,  131072 tokens,      S=32768, H=5120, bf16 in + deepstack, e4m3 out, per-token scale
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np
import torch

QUANT_NONE, QUANT_STATIC_TENSOR, QUANT_DYNAMIC_TOKEN, QUANT_MX_BLOCK = 0, 1, 2, 4

BASE_SEED = 20261202

# tensor ids folded into the seed, one stream per tensor
_TID_PARTIALS, _TID_RESIDUAL, _TID_DEEPSTACK, _TID_WEIGHT, _TID_BIAS = 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    tp: int
    num_tokens: int          # valid tokens T over all ranks
    num_tokens_pad: int      # T_pad, a multiple of tp
    hidden: int
    partial_dtype: torch.dtype
    act_dtype: torch.dtype
    quant_mode: int
    out_dtype: torch.dtype   # bf16 / f32 for no quant, uint8 (e4m3 codes) otherwise
    residual_replicated: bool  # residual holds every rank's rows ([tp*S, H])
    deepstack: bool            # deepstack present, full [T_pad, H], chunked by rank
    bias: bool
    rank: int                  # rank whose shard is timed
    partial_sigma: float
    residual_sigma: float = 1.0
    deepstack_sigma: float = 0.3
    weight_mu: float = 1.0
    weight_sigma: float = 0.1
    bias_sigma: float = 0.02
    eps: float = 1e-6
    seed_index: int = 0
    fp4: bool = False          # block-scaled output with e2m1 elements (two per byte)

    @property
    def shard_rows(self) -> int:
        return self.num_tokens_pad // self.tp

    def valid_rows(self, rank: Optional[int] = None) -> int:
        r = self.rank if rank is None else rank
        return max(0, min(self.shard_rows, self.num_tokens - r * self.shard_rows))

    def algorithmic_bytes(self, rank: Optional[int] = None) -> int:
        """Bytes the method must move for one rank's shard: read the tp partials,
        the residual and deepstack rows of the valid rows, weight and bias once,
        the static scale once; write residual_out and out for all S rows and
        the per-token scales."""
        S, H, v = self.shard_rows, self.hidden, self.valid_rows(rank)
        pe = torch.tensor([], dtype=self.partial_dtype).element_size()
        ae = torch.tensor([], dtype=self.act_dtype).element_size()
        out_row = H // 2 if self.fp4 else H * torch.tensor([], dtype=self.out_dtype).element_size()
        reads = v * H * (self.tp * pe + ae + (ae if self.deepstack else 0))
        reads += H * ae * (2 if self.bias else 1)
        reads += 4 if self.quant_mode == QUANT_STATIC_TENSOR else 0
        scale_row = {QUANT_DYNAMIC_TOKEN: 4, QUANT_MX_BLOCK: H // 32}.get(self.quant_mode, 0)
        writes = S * (H * ae + out_row + scale_row)
        return reads + writes


WORKLOADS = {
    "C1": Workload("C1", "tp=2, 64 tokens (32/rank shard), hidden 512, fp32 partials and residual, "
                   "bias, bf16 out", tp=2, num_tokens=64, num_tokens_pad=64, hidden=512,
                   partial_dtype=torch.float32, act_dtype=torch.float32, quant_mode=QUANT_NONE,
                   out_dtype=torch.bfloat16, residual_replicated=True, deepstack=False, bias=True,
                   rank=1, partial_sigma=1.0, seed_index=0),
    "C2": Workload("C2", "dense SP threshold: 1000 tokens padded to 1024, tp=8 (128-token shard), "
                   "hidden 4096, bf16", tp=8, num_tokens=1000, num_tokens_pad=1024, hidden=4096,
                   partial_dtype=torch.bfloat16, act_dtype=torch.bfloat16, quant_mode=QUANT_NONE,
                   out_dtype=torch.bfloat16, residual_replicated=False, deepstack=False, bias=False,
                   rank=7, partial_sigma=0.5, seed_index=1),
    "C3": Workload("C3", "GLM-like: 3500 tokens padded to 3504, tp=16 (219-token shard), hidden "
                   "8192, bf16, bias", tp=16, num_tokens=3500, num_tokens_pad=3504, hidden=8192,
                   partial_dtype=torch.bfloat16, act_dtype=torch.bfloat16, quant_mode=QUANT_NONE,
                   out_dtype=torch.bfloat16, residual_replicated=False, deepstack=False, bias=True,
                   rank=15, partial_sigma=0.5, seed_index=2),
    "C4": Workload("C4", "FP8 static per-tensor: 65536 tokens, tp=8 (8192-token shard), hidden "
                   "7168, bf16 in, e4m3 out", tp=8, num_tokens=65536, num_tokens_pad=65536,
                   hidden=7168, partial_dtype=torch.bfloat16, act_dtype=torch.bfloat16,
                   quant_mode=QUANT_STATIC_TENSOR, out_dtype=torch.uint8,
                   residual_replicated=False, deepstack=False, bias=False, rank=7,
                   partial_sigma=0.5, seed_index=3),
    "C5": Workload("C5", "VL deepstack + per-token dynamic FP8: 131072 tokens, tp=4 (32768-token "
                   "shard), hidden 5120, bf16 in, e4m3 out + fp32 row scales", tp=4,
                   num_tokens=131072, num_tokens_pad=131072, hidden=5120,
                   partial_dtype=torch.bfloat16, act_dtype=torch.bfloat16,
                   quant_mode=QUANT_DYNAMIC_TOKEN, out_dtype=torch.uint8,
                   residual_replicated=False, deepstack=True, bias=False, rank=3,
                   partial_sigma=0.5, seed_index=4),
}


_HERE = os.path.dirname(os.path.abspath(__file__))
GEN_SRC = os.path.join(_HERE, "inputs_gen.c")
GEN_LIB = os.path.join(_HERE, "libsprms_inputs.so")
GEN_CMD = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread", "-o", GEN_LIB,
           GEN_SRC, "-lm"]
_gen = None


def build_generator() -> str:
    """Compile the input generator with gcc (always; part of the repository build)."""
    subprocess.run(GEN_CMD, check=True)
    return GEN_LIB


def _lib():
    global _gen
    if _gen is None:
        if not os.path.exists(GEN_LIB):
            build_generator()
        lib = ctypes.CDLL(GEN_LIB)
        lib.sprms_inputs_key.argtypes = [ctypes.c_uint64] * 3
        lib.sprms_inputs_key.restype = ctypes.c_uint64
        lib.sprms_inputs_normal.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_int]
        lib.sprms_inputs_normal.restype = ctypes.c_int
        _gen = lib
    return _gen


GEN_THREADS = max(1, min(16, os.cpu_count() or 1))


def draw(seed: int, tensor: int, source: int, row0: int, rows: int, cols: int, mu: float, sigma: float,
         dtype: torch.dtype, out: Optional[np.ndarray] = None) -> torch.Tensor:
    """Rows [row0, row0 + rows) of a [.][cols] tensor of the stream
    (seed, tensor, source), as a CPU tensor of dtype (float32 or bfloat16),
    drawn into `out` (a C-contiguous [rows][cols] array of the storage type)
    when given."""
    lib = _lib()
    bf16 = dtype == torch.bfloat16
    arr = np.empty((rows, cols), np.uint16 if bf16 else np.float32) if out is None else out
    assert arr.shape == (rows, cols) and arr.dtype == (np.uint16 if bf16 else np.float32)
    assert arr.flags["C_CONTIGUOUS"]
    key = lib.sprms_inputs_key(seed, tensor, source)
    rc = lib.sprms_inputs_normal(key, row0, rows, cols, float(mu), float(sigma), int(bf16),
                                 arr.ctypes.data_as(ctypes.c_void_p), GEN_THREADS)
    if rc != 0:
        raise ValueError(f"input draw failed for rows {row0}+{rows} x {cols}")
    if arr.size == 0:  # numpy gives empty arrays zero strides; keep torch's row-major ones
        return torch.empty((rows, cols), dtype=dtype)
    t = torch.from_numpy(arr)
    return t.view(torch.int16).view(torch.bfloat16) if bf16 else t


def make_inputs(w: Workload, rank: Optional[int] = None, device="cpu", base_seed=BASE_SEED,
                pad_fill: Optional[float] = None, shard_rows: Optional[int] = None,
                num_tokens: Optional[int] = None):
    """Seeded inputs for one rank's shard.

    Returns a dict of tensors: partials [tp, S, H], residual ([tp*S, H] when
    replicated else [S, H]), weight [H], bias [H] or None, deepstack
    [tp*S, H] or None.  ``pad_fill`` (e.g. NaN) overwrites every input row
    that belongs to a padding row of this shard, to show they are not read.
    ``shard_rows`` and ``num_tokens`` override S and T (smaller stand-ins of
    a workload's shape; T defaults to min(T, tp*S)).
    """
    r = w.rank if rank is None else rank
    S = w.shard_rows if shard_rows is None else shard_rows
    H, tp = w.hidden, w.tp
    seed = base_seed + w.seed_index
    # partial q of rank r: rows [r*S, (r+1)*S) of partial q's full tensor
    pbuf = np.empty((tp, S, H), np.uint16 if w.partial_dtype == torch.bfloat16 else np.float32)
    for q in range(tp):
        draw(seed, _TID_PARTIALS, q, r * S, S, H, 0.0, w.partial_sigma, w.partial_dtype, out=pbuf[q])
    parts = torch.from_numpy(pbuf)
    if w.partial_dtype == torch.bfloat16:
        parts = parts.view(torch.int16).view(torch.bfloat16)
    if S == 0:  # numpy gives empty arrays zero strides; keep torch's row-major ones
        parts = torch.empty((tp, 0, H), dtype=w.partial_dtype)
    res0, res_rows = (0, tp * S) if w.residual_replicated else (r * S, S)
    out = {
        "partials": parts,
        "residual": draw(seed, _TID_RESIDUAL, 0, res0, res_rows, H, 0.0, w.residual_sigma, w.act_dtype),
        # gain and bias are replicated on every rank: one row each, no rank in the stream
        "weight": draw(seed, _TID_WEIGHT, 0, 0, 1, H, w.weight_mu, w.weight_sigma, w.act_dtype)[0],
        "bias": (draw(seed, _TID_BIAS, 0, 0, 1, H, 0.0, w.bias_sigma, w.act_dtype)[0] if w.bias else None),
        "deepstack": (draw(seed, _TID_DEEPSTACK, 0, 0, tp * S, H, 0.0, w.deepstack_sigma, w.act_dtype)
                      if w.deepstack else None),
    }
    out = {k: (None if t is None else t.to(device)) for k, t in out.items()}
    if pad_fill is not None:
        T = min(w.num_tokens, tp * S) if num_tokens is None else num_tokens
        v = max(0, min(S, T - r * S))
        if v < S:
            out["partials"][:, v:, :] = pad_fill
            roff = r * S if w.residual_replicated else 0
            out["residual"][roff + v:roff + S] = pad_fill
            if out["deepstack"] is not None:
                out["deepstack"][r * S + v:r * S + S] = pad_fill
    return out
