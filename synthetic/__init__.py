"""Seeded synthetic inputs for attention, shared by the tests, smoke() and bench.py.

This module holds no attention arithmetic: it only draws i.i.d. N(0, 1) tensors
from seeded CPU generators, rounds them to the working dtype, and names the
workloads.  Both the HIP path and the CPU oracle consume what it returns (the
oracle upcasts the same rounded values to float64).

Seeds: tensor t of workload k uses seed 1000*k + t with t = 0 (Q), 1 (K), 2 (V),
3 (dO).  Point p of the throughput sweep uses 5000 + 10*p + t; the decoding
workloads (fewer queries than keys) use 6000, 6100 and 6200 + t, the masked ones 7000
and 7100 + t, the row workloads 8000, 8100 and 8200 + t.  The GQA workload
additionally scales ceil(1%) of all key rows by 8 (exact in bf16), rows picked by
a seed-4100 permutation over the flattened (batch, kv-head, position) rows, before
the dtype cast: those rows produce scores far above the rest and move the running
max late in the key loop.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    causal: bool
    backward: bool
    seed_base: int
    k_outlier_frac: float = 0.0
    k_outlier_scale: float = 8.0
    k_outlier_seed: int = 0
    notes: str = ""
    Nk: int = 0  # key/value rows; 0 means the same as N (queries)

    @property
    def nk(self) -> int:
        return self.Nk or self.N

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def shape_q(self):
        return (self.B, self.H, self.N, self.d)

    @property
    def shape_kv(self):
        return (self.B, self.Hkv, self.nk, self.d)

    def fwd_flop(self) -> float:
        """4*B*H*N^2*d for the two forward matmuls, halved under a causal mask.  With
        fewer queries than keys: 4*B*H*d per visible (query, key) pair, the causal
        mask being aligned bottom-right (query i sees keys 0 .. i + Nk - N)."""
        if self.nk == self.N:
            f = 4.0 * self.B * self.H * self.N * self.N * self.d
            return f / 2 if self.causal else f
        pairs = self.N * self.nk
        if self.causal:
            pairs -= self.N * (self.N - 1) // 2
        return 4.0 * self.B * self.H * pairs * self.d

    def kv_bytes(self) -> int:
        """Bytes of K and V: what a decoding step must read at least once."""
        e = DTYPES[self.dtype].itemsize
        return 2 * self.B * self.Hkv * self.nk * self.d * e

    def bwd_flop(self) -> float:
        """Five N^2*d matmuls (S recompute, dV, dP, dK, dQ): 2.5x the forward."""
        return 2.5 * self.fwd_flop()

    def describe(self) -> dict:
        out = {"workload": self.name, "dtype": self.dtype, "B": self.B, "H": self.H,
               "Hkv": self.Hkv, "N": self.N, "d": self.d, "causal": self.causal}
        if self.nk != self.N:
            out["Nq"], out["Nk"] = out.pop("N"), self.nk
        return out


SWEEP_N = (1024, 2048, 4096, 8192, 16384)
SWEEP_D = (64, 128)


def sweep_points():
    """Throughput sweep points, ordered by N ascending then d ascending."""
    pts = []
    for n in SWEEP_N:
        for d in SWEEP_D:
            p = len(pts)
            pts.append(Workload(f"sweep_bf16_B4_H16_N{n}_d{d}", "bf16", 4, 16, 16, n, d,
                                False, True, 5000 + 10 * p))
    return pts


WORKLOADS = {
    "fp32_single_head": Workload("fp32_single_head_B1_H1_N256_d64", "fp32", 1, 1, 1, 256, 64,
                                 False, True, 1000),
    "bf16_fwd": Workload("bf16_fwd_B4_H16_N2048_d128", "bf16", 4, 16, 16, 2048, 128,
                         False, False, 2000),
    "fp16_causal": Workload("fp16_causal_B2_H32_N8192_d64", "fp16", 2, 32, 32, 8192, 64,
                            True, True, 3000),
    "bf16_gqa_causal": Workload("bf16_gqa_causal_B1_H32_Hkv8_N16384_d128", "bf16", 1, 32, 8,
                                16384, 128, True, True, 4000, k_outlier_frac=0.01,
                                k_outlier_seed=4100),
}
for _w in sweep_points():
    WORKLOADS[_w.name] = _w

# Decoding with a long key/value history (split-KV forward): one new query per head,
# or a block of 16 (speculative / chunked decoding), against 16384 cached positions;
# causal with the queries at the end of the sequence.
DECODE = {
    "decode_bf16_gqa_q1": Workload("decode_bf16_gqa_B4_H32_Hkv8_Nq1_Nk16384_d128", "bf16", 4, 32,
                                   8, 1, 128, True, False, 6000, Nk=16384),
    "decode_bf16_gqa_q16": Workload("decode_bf16_gqa_B4_H32_Hkv8_Nq16_Nk16384_d128", "bf16", 4,
                                    32, 8, 16, 128, True, False, 6100, Nk=16384),
    "decode_fp16_mha_q1": Workload("decode_fp16_mha_B8_H16_Nq1_Nk8192_d64", "fp16", 8, 16, 16, 1,
                                   64, False, False, 6200, Nk=8192),
}
WORKLOADS.update(DECODE)

# The throughput headline: bf16, non-causal, B*H = 64, N = 8192, d = 128.
HEADLINE = WORKLOADS["sweep_bf16_B4_H16_N8192_d128"]


def randn(shape, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32)


def make_inputs(w: Workload, with_grad: bool | None = None) -> dict:
    """CPU tensors q, k, v (and do) in the workload's dtype, contiguous."""
    dt = DTYPES[w.dtype]
    q = randn(w.shape_q, w.seed_base + 0)
    k = randn(w.shape_kv, w.seed_base + 1)
    v = randn(w.shape_kv, w.seed_base + 2)
    if w.k_outlier_frac > 0:
        rows = w.B * w.Hkv * w.nk
        n_sel = math.ceil(w.k_outlier_frac * rows)
        g = torch.Generator(device="cpu").manual_seed(w.k_outlier_seed)
        sel = torch.randperm(rows, generator=g)[:n_sel]
        k = k.reshape(rows, w.d)
        k[sel] *= w.k_outlier_scale
        k = k.reshape(w.shape_kv)
    out = {"q": q.to(dt).contiguous(), "k": k.to(dt).contiguous(), "v": v.to(dt).contiguous()}
    if with_grad if with_grad is not None else w.backward:
        out["do"] = randn(w.shape_q, w.seed_base + 3).to(dt).contiguous()
    return out


def custom(dtype: str, B: int, H: int, Hkv: int, N: int, d: int, causal: bool,
           seed_base: int, **kw) -> Workload:
    """A small ad-hoc workload (edge cases in tests); Nk=... for fewer queries than keys."""
    nk = kw.get("Nk", 0)
    tag = f"N{N}" if not nk else f"Nq{N}_Nk{nk}"
    return Workload(f"case_{dtype}_B{B}_H{H}_Hkv{Hkv}_{tag}_d{d}_{'c' if causal else 'nc'}",
                    dtype, B, H, Hkv, N, d, causal, not nk, seed_base, **kw)


def with_dtype(w: Workload, dtype: str) -> Workload:
    return replace(w, dtype=dtype, name=w.name + "_as_" + dtype)


def mask_intervals(kind: str, B: int, Nq: int, Nk: int, seed: int = 0, **kw):
    """Per-row visible key intervals (kv_lo, kv_hi), int32 [B, Nq], inclusive.

    These are inputs (like q, k, v), the same for the oracle and the GPU:
      causal    query i sees keys 0 .. i + Nk - Nq (queries at the end of the sequence)
      sliding   keys i + off - left .. i + off + right (right = 0 with causal=True)
      document  doc_lens[b] splits the positions into documents (Nq == Nk); a row sees its
                own document (up to itself with causal=True)
      prefix    prefix-LM: keys 0 .. max(prefix - 1, i + off)
      random    seeded random intervals, some of them empty (lo > hi)
    """
    off = Nk - Nq
    i = torch.arange(Nq, dtype=torch.int64)
    if kind == "causal":
        lo = torch.zeros(Nq, dtype=torch.int64)
        hi = i + off
    elif kind == "sliding":
        left, right = kw.get("left", 128), kw.get("right", 0)
        lo = (i + off - left).clamp(min=0)
        hi = (i + off + (0 if kw.get("causal", True) else right)).clamp(max=Nk - 1)
    elif kind == "prefix":
        lo = torch.zeros(Nq, dtype=torch.int64)
        hi = torch.maximum(torch.full((Nq,), kw["prefix"] - 1), i + off).clamp(max=Nk - 1)
    elif kind == "document":
        if Nq != Nk:
            raise ValueError("document masks need Nq == Nk")
        los, his = [], []
        for b in range(B):
            lens = kw["doc_lens"][b]
            if sum(lens) != Nq:
                raise ValueError("document lengths must add up to N")
            start = torch.tensor([0] + list(lens[:-1])).cumsum(0)
            doc = torch.repeat_interleave(torch.arange(len(lens)), torch.tensor(lens))
            s_b = start[doc]
            e_b = s_b + torch.tensor(lens)[doc] - 1
            los.append(s_b)
            his.append(torch.minimum(e_b, i) if kw.get("causal", True) else e_b)
        return torch.stack(los).to(torch.int32).contiguous(), torch.stack(his).to(torch.int32).contiguous()
    elif kind == "random":
        g = torch.Generator(device="cpu").manual_seed(seed)
        a = torch.randint(0, Nk, (B, Nq), generator=g)
        w = torch.randint(0, max(1, Nk // 2), (B, Nq), generator=g)
        lo, hi = a, (a + w).clamp(max=Nk - 1)
        empty = torch.rand((B, Nq), generator=g) < kw.get("empty_frac", 0.05)
        lo = torch.where(empty, hi + 1, lo)
        return lo.to(torch.int32).contiguous(), hi.to(torch.int32).contiguous()
    else:
        raise ValueError(f"unknown mask kind {kind}")
    lo = lo.to(torch.int32).expand(B, Nq).contiguous()
    hi = hi.to(torch.int32).expand(B, Nq).contiguous()
    return lo, hi


# Masked workloads (interval masks): a 4096-key causal sliding window on the GQA shape,
# and packed documents of mixed lengths (causal within each document).
MASKED = {
    "sliding4096_bf16_gqa": (custom("bf16", 1, 32, 8, 16384, 128, False, seed_base=7000),
                             "sliding", {"left": 4095, "causal": True}),
    "documents_bf16": (custom("bf16", 4, 16, 16, 8192, 128, False, seed_base=7100), "document",
                       {"doc_lens": [[3000, 2000, 3192], [8192], [1, 4095, 4096], [100] * 81 + [92]],
                        "causal": True}),
}


# ---- fp8 (e4m3) inputs -----------------------------------------------------------------
def fp8_quantize(x: torch.Tensor):
    """e4m3 codes (uint8, same shape) of x / s and the per-tensor dequantisation factor
    s = max|x| / 448 (so the largest magnitude maps to the largest e4m3 value);
    torch's conversion rounds to nearest even."""
    amax = float(x.abs().max())
    descale = amax / 448.0 if amax > 0 else 1.0
    codes = (x.float() / descale).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return codes, descale


def make_fp8_inputs(w: Workload) -> dict:
    """The workload's Q, K, V (the same seeded N(0, 1) draws as make_inputs, before any
    rounding) quantised to e4m3 per tensor: codes q8, k8, v8 and factors dq, dk, dv."""
    out = {}
    for name, t in (("q", 0), ("k", 1), ("v", 2)):
        shape = w.shape_q if name == "q" else w.shape_kv
        codes, ds = fp8_quantize(randn(shape, w.seed_base + t))
        out[name + "8"] = codes
        out["d" + name] = ds
    return out


# ---- row softmax / log-softmax / cross-entropy workloads ------------------------------
@dataclass(frozen=True)
class RowWorkload:
    """Rows of `cols` logits.  op is "softmax", "log_softmax" or "xent"."""
    name: str
    op: str
    dtype: str
    rows: int
    cols: int
    seed: int
    std: float = 1.0          # logits are std * N(0, 1)
    ignore_frac: float = 0.0  # xent: fraction of rows whose target is -100 (ignored)

    def elem_bytes(self) -> int:
        return DTYPES[self.dtype].itemsize

    def describe(self) -> dict:
        return {"workload": self.name, "op": self.op, "rows": self.rows, "cols": self.cols,
                "dtype": self.dtype, "logit_std": self.std, "ignored_fraction": self.ignore_frac}


IGNORE_TARGET = -100


def row_inputs(w: RowWorkload, backward: bool = True) -> dict:
    """CPU tensors: x [rows, cols] in the dtype; softmax ops add dy (N(0, 1), seed + 1);
    xent adds int32 targets uniform over the classes (seed + 2), a seeded fraction of
    them set to -100 (seed + 3), and dloss = 1 / (rows not ignored) on every row, the
    gradient of the mean loss."""
    dt = DTYPES[w.dtype]
    out = {"x": (randn((w.rows, w.cols), w.seed) * w.std).to(dt).contiguous()}
    if w.op == "xent":
        g = torch.Generator(device="cpu").manual_seed(w.seed + 2)
        t = torch.randint(0, w.cols, (w.rows,), generator=g)
        if w.ignore_frac > 0:
            g3 = torch.Generator(device="cpu").manual_seed(w.seed + 3)
            t = torch.where(torch.rand((w.rows,), generator=g3) < w.ignore_frac,
                            torch.full_like(t, IGNORE_TARGET), t)
        out["targets"] = t.to(torch.int32).contiguous()
        live = int((out["targets"] >= 0).sum())
        out["dloss"] = torch.full((w.rows,), 1.0 / max(1, live), dtype=torch.float32)
    elif backward:
        out["dy"] = randn((w.rows, w.cols), w.seed + 1).to(dt).contiguous()
    return out


# Row workloads: cross-entropy over a 128256-class vocabulary for 8192 tokens (an LM
# head's logits), softmax over 65536 rows of 8192 attention scores (8 heads' full
# score matrices at N = 8192), and fp32 log-softmax over a 32000-class vocabulary.
ROWS = {
    "xent_bf16_T8192_V128256": RowWorkload("xent_bf16_T8192_V128256", "xent", "bf16", 8192,
                                           128256, 8000, std=2.0, ignore_frac=0.02),
    "softmax_bf16_R65536_C8192": RowWorkload("softmax_bf16_R65536_C8192", "softmax", "bf16",
                                             65536, 8192, 8100),
    "log_softmax_fp32_R8192_C32000": RowWorkload("log_softmax_fp32_R8192_C32000", "log_softmax",
                                                 "fp32", 8192, 32000, 8200, std=2.0),
}


def visible_pairs(kv_lo, kv_hi, Nk: int) -> int:
    """Number of (query, key) pairs an interval mask leaves visible, over the batch."""
    lo = kv_lo.to(torch.int64).clamp(min=0)
    hi = kv_hi.to(torch.int64).clamp(max=Nk - 1)
    return int((hi - lo + 1).clamp(min=0).sum())
