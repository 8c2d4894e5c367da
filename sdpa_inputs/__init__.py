"""Seeded synthetic inputs for the attention forward: shapes, seeds, value draws.

This module is shared by the GPU path's tests/bench and by the CPU oracle's tests, so it holds
no attention arithmetic at all: it only draws numbers and stores them in the dtype the kernel
receives. Both sides get the *same bytes*: bf16 inputs are produced once here (fp32 draw, then
round-to-nearest-even to bf16) and handed to the GPU as raw 16-bit words and to the oracle as
float64 upcasts of those same words.

The workloads take their shapes from the pages:
  * Mistral-7B attention (32 query heads, 8 KV heads, head dim 128, sliding window 4096,
    batch 4, seq 4096/8192) -- transformers issue "Slowdown in Training Speed Due to SDPA Mask
    Fix in Version 4.40.0" (the throughput table and the reproduction script);
  * T5-small encoder attention (12 heads, head dim 64) with bucketed relative-position bias or a
    full additive bias -- the FAT5 (flashT5) README, attention-bias list;
  * MHA / GQA / MQA head sharing -- "jax-gpu-05-attention-gpu" codelab, section 9.
Values are N(0,1) draws (the codelab draws Q, K, V with a normal generator, section 3). The
pages' own datasets (alpaca-cleaned, CulturaX, ...) are not used: these synthetic tensors
stand in for the activations those runs would produce.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

MASK_NONE, MASK_CAUSAL, MASK_SLIDING = 0, 1, 2
BIAS_NONE, BIAS_T5, BIAS_FULL, BIAS_ALIBI, BIAS_T5U = 0, 1, 2, 3, 4
MASK_NAMES = {MASK_NONE: "none", MASK_CAUSAL: "causal", MASK_SLIDING: "sliding"}
BIAS_NAMES = {BIAS_NONE: "none", BIAS_T5: "t5", BIAS_FULL: "full", BIAS_ALIBI: "alibi",
              BIAS_T5U: "t5u"}


def alibi_slopes(H: int) -> np.ndarray:
    """The ALiBi paper's head slopes for H heads (H a power of two): 2^(-8 h / H), h = 1..H;
    for other H the sequence of the next power of two, interleaved as the paper prescribes."""
    def pow2(n):
        return [2.0 ** (-8.0 * (i + 1) / n) for i in range(n)]
    p = 1 << (H - 1).bit_length()
    s = pow2(p) if p == H else pow2(p // 2) + pow2(p)[0::2][: H - p // 2]
    return np.asarray(s[:H], dtype=np.float32)

# T5 relative-position table geometry (fixed constants of the bias kind).
T5_NUM_BUCKETS = 32
T5_MAX_DISTANCE = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    dtype: str            # "bf16" or "f32": the dtype of q, k, v (and of a full bias)
    mask_kind: int
    window: int = 0
    bias_kind: int = BIAS_NONE
    seed: int = 0         # base seed; q = seed, k = seed+1, v = seed+2, t5 table = seed+3,
    #                       bias = seed+4, dO (backward) = seed+5
    kv_seed: Optional[int] = None   # overrides the k/v seed base (k = kv_seed+1, v = kv_seed+2)
    bias_std: float = 0.5
    scale_override: Optional[float] = None   # softmax scale; default 1/sqrt(D)

    @property
    def scale(self) -> float:
        if self.scale_override is not None:
            return float(np.float32(self.scale_override))
        return float(np.float32(1.0 / np.sqrt(self.D)))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def describe(self) -> dict:
        d = dict(workload=self.name, B=self.B, Hq=self.Hq, Hkv=self.Hkv, Sq=self.Sq, Sk=self.Sk,
                 D=self.D, dtype=self.dtype, mask=MASK_NAMES[self.mask_kind],
                 bias=BIAS_NAMES[self.bias_kind])
        if self.mask_kind == MASK_SLIDING:
            d["window"] = self.window
        return d


def _c5(hkv: int) -> Workload:
    return Workload(f"headshare_hkv{hkv}_b16_s4096", 16, 32, hkv, 4096, 4096, 128, "bf16",
                    MASK_CAUSAL, seed=5000, kv_seed=5000 + 10 * hkv)


# The five workloads (c1..c5); c3c is the full-causal comparison run of c3 and c2c the causal
# twin of c2 (window 4096 = S), c4full the full-bias variant of c4, c5 is swept over Hkv in
# {32, 8, 1}.
WORKLOADS = {
    "c1": Workload("tiny_causal_f32_b1_h2_s128_d64", 1, 2, 2, 128, 128, 64, "f32", MASK_CAUSAL,
                   seed=1000),
    "c2": Workload("mistral_gqa_sliding4096_b4_s4096", 4, 32, 8, 4096, 4096, 128, "bf16",
                   MASK_SLIDING, window=4096, seed=2000),
    "c3": Workload("mistral_gqa_sliding4096_b4_s8192", 4, 32, 8, 8192, 8192, 128, "bf16",
                   MASK_SLIDING, window=4096, seed=3000),
    "c3c": Workload("mistral_gqa_causal_b4_s8192", 4, 32, 8, 8192, 8192, 128, "bf16",
                    MASK_CAUSAL, seed=3000),
    "c2c": Workload("mistral_gqa_causal_b4_s4096", 4, 32, 8, 4096, 4096, 128, "bf16",
                    MASK_CAUSAL, seed=2000),
    "c4t5": Workload("t5_encoder_rpe_b8_h12_s2048_d64", 8, 12, 12, 2048, 2048, 64, "bf16",
                     MASK_NONE, bias_kind=BIAS_T5, seed=4000),
    "c4full": Workload("t5_encoder_fullbias_b8_h12_s2048_d64", 8, 12, 12, 2048, 2048, 64, "bf16",
                       MASK_NONE, bias_kind=BIAS_FULL, seed=4000),
    "c5mha": _c5(32),
    "c5gqa": _c5(8),
    "c5mqa": _c5(1),
    # KV-cache decode: one new query row per head against a long cache
    # (Mistral-7B heads), the MQA variant, and four new rows against a sliding-window cache
    "dec": Workload("mistral_gqa_decode_b16_q1_k16384", 16, 32, 8, 1, 16384, 128, "bf16",
                    MASK_CAUSAL, seed=6000),
    "decmqa": Workload("mqa_decode_b16_q1_k16384", 16, 32, 1, 1, 16384, 128, "bf16",
                       MASK_CAUSAL, seed=6100),
    "decsw": Workload("mistral_gqa_decode_b8_q4_k32768_sliding4096", 8, 32, 8, 4, 32768, 128,
                      "bf16", MASK_SLIDING, window=4096, seed=6200),
    "decd256": Workload("gqa_decode_d256_b16_q1_k16384", 16, 32, 8, 1, 16384, 256, "bf16",
                        MASK_CAUSAL, seed=6300),
    # more index-generated biases: ALiBi on the Mistral GQA shape, and the
    # T5 decoder's unidirectional buckets on T5-small decoder self-attention
    "c2alibi": Workload("mistral_gqa_causal_alibi_b4_s4096", 4, 32, 8, 4096, 4096, 128, "bf16",
                        MASK_CAUSAL, bias_kind=BIAS_ALIBI, seed=8000),
    "c4t5u": Workload("t5_decoder_rpe_b8_h12_s2048_d64", 8, 12, 12, 2048, 2048, 64, "bf16",
                      MASK_CAUSAL, bias_kind=BIAS_T5U, seed=8100),
    # the head-dim sweep at both ends (32 and 256) on the Mistral GQA causal shape
    "c2d32": Workload("gqa_causal_d32_b4_s4096", 4, 32, 8, 4096, 4096, 32, "bf16",
                      MASK_CAUSAL, seed=8200),
    "c2d256": Workload("gqa_causal_d256_b4_s4096", 4, 32, 8, 4096, 4096, 256, "bf16",
                       MASK_CAUSAL, seed=8300),
}


# ----------------------------------------------------------------------------------------------
# bf16 storage helpers (bit manipulation only)
# ----------------------------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return raw uint16 words.

    Inputs here are finite normal draws, so no NaN/Inf special-casing is needed (asserted).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert np.isfinite(x).all()
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 words to float32 (the bf16 word is the top half of the f32 word)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# Draws
# ----------------------------------------------------------------------------------------------
def normal_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


@dataclasses.dataclass
class Inputs:
    """One workload's inputs, in the storage the kernel receives.

    For bf16 workloads q/k/v (and a full bias) are uint16 bf16 words; for f32 they are float32.
    t5_table holds the float32 bias table: [Hq][32] for T5 buckets, [Hq] ALiBi slopes.
    """
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    t5_table: Optional[np.ndarray] = None
    bias: Optional[np.ndarray] = None

    def as_f64(self):
        """float64 views of the exact values the kernel sees: (q, k, v, bias-or-table)."""
        conv = bf16_bits_to_f64 if self.wl.dtype == "bf16" else (lambda a: a.astype(np.float64))
        extra = None
        if self.wl.bias_kind in (BIAS_T5, BIAS_T5U, BIAS_ALIBI):
            extra = self.t5_table.astype(np.float64)
        elif self.wl.bias_kind == BIAS_FULL:
            extra = conv(self.bias)
        return conv(self.q), conv(self.k), conv(self.v), extra


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def make_inputs(wl: Workload) -> Inputs:
    """Draw q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] (+ t5 table [Hq,32] or bias [B,Hq,Sq,Sk])."""
    kvs = wl.seed if wl.kv_seed is None else wl.kv_seed
    q = _store(normal_f32(wl.seed, (wl.B, wl.Sq, wl.Hq, wl.D)), wl.dtype)
    k = _store(normal_f32(kvs + 1, (wl.B, wl.Sk, wl.Hkv, wl.D)), wl.dtype)
    v = _store(normal_f32(kvs + 2, (wl.B, wl.Sk, wl.Hkv, wl.D)), wl.dtype)
    inp = Inputs(wl, q, k, v)
    if wl.bias_kind in (BIAS_T5, BIAS_T5U):
        inp.t5_table = normal_f32(wl.seed + 3, (wl.Hq, T5_NUM_BUCKETS))
    elif wl.bias_kind == BIAS_ALIBI:
        inp.t5_table = alibi_slopes(wl.Hq)
    elif wl.bias_kind == BIAS_FULL:
        inp.bias = _store(normal_f32(wl.seed + 4, (wl.B, wl.Hq, wl.Sq, wl.Sk), wl.bias_std),
                          wl.dtype)
    return inp


def make_dout(wl: Workload) -> np.ndarray:
    """The output gradient dL/dO [B, Sq, Hq, D] for the backward, in the workload's dtype:
    N(0, 1) draws from seed + 5 (the weights of an arbitrary linear loss sum(dO * O))."""
    return _store(normal_f32(wl.seed + 5, (wl.B, wl.Sq, wl.Hq, wl.D)), wl.dtype)


# ----------------------------------------------------------------------------------------------
# Packed variable-length sequences
# ----------------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """Sequences packed back to back: lengths drawn from a seeded log-normal (median `median`,
    log-sd `sigma`, clipped to [lo, hi]) until they fill `total` tokens (the last one cut)."""
    name: str
    total: int
    Hq: int
    Hkv: int
    D: int
    mask_kind: int
    window: int = 0
    bias_kind: int = BIAS_NONE
    seed: int = 0
    median: float = 1024.0
    sigma: float = 0.8
    lo: int = 16
    hi: int = 8192
    scale_override: Optional[float] = None
    lengths_override: Optional[tuple] = None

    @property
    def scale(self) -> float:
        if self.scale_override is not None:
            return float(np.float32(self.scale_override))
        return float(np.float32(1.0 / np.sqrt(self.D)))

    def lengths(self) -> list:
        if self.lengths_override is not None:
            return list(self.lengths_override)
        rng = np.random.default_rng(self.seed + 9)
        out, left = [], self.total
        while left > 0:
            n = int(np.clip(round(self.median * np.exp(self.sigma * rng.standard_normal())),
                            self.lo, self.hi))
            n = min(n, left)
            out.append(n)
            left -= n
        return out

    def replace(self, **kw) -> "VarlenWorkload":
        return dataclasses.replace(self, **kw)

    def describe(self) -> dict:
        ls = self.lengths()
        d = dict(workload=self.name, packed_tokens=sum(ls), sequences=len(ls),
                 max_len=max(ls), Hq=self.Hq, Hkv=self.Hkv, D=self.D, dtype="bf16",
                 mask=MASK_NAMES[self.mask_kind], bias=BIAS_NAMES[self.bias_kind])
        if self.mask_kind == MASK_SLIDING:
            d["window"] = self.window
        return d


# Mistral-7B heads, 32768 packed tokens (one training micro-batch's worth, like B4 x S8192),
# causal inside each sequence; lengths stand in for packed instruction-tuning examples
VARLEN_WORKLOADS = {
    "vl": VarlenWorkload("mistral_gqa_packed_32768_causal", 32768, 32, 8, 128, MASK_CAUSAL,
                         seed=7000),
}


@dataclasses.dataclass
class VarlenInputs:
    wl: VarlenWorkload
    q: np.ndarray          # bf16 words [total, Hq, D]
    k: np.ndarray          # bf16 words [total_k, Hkv, D]
    v: np.ndarray
    cu_q: np.ndarray       # int32 [n + 1]
    cu_k: np.ndarray
    t5_table: Optional[np.ndarray] = None

    def as_f64(self):
        return (bf16_bits_to_f64(self.q), bf16_bits_to_f64(self.k), bf16_bits_to_f64(self.v),
                None if self.t5_table is None else self.t5_table.astype(np.float64))


def make_varlen_inputs(wl: VarlenWorkload, key_lengths: Optional[list] = None) -> VarlenInputs:
    """q [total_q, Hq, D], k/v [total_k, Hkv, D] bf16 from seeds seed, seed+1, seed+2 (T5 table
    seed+3); key lengths equal the query lengths unless given."""
    lq = wl.lengths()
    lk = list(key_lengths) if key_lengths is not None else lq
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = f32_to_bf16_bits(normal_f32(wl.seed, (int(cu_q[-1]), wl.Hq, wl.D)))
    k = f32_to_bf16_bits(normal_f32(wl.seed + 1, (int(cu_k[-1]), wl.Hkv, wl.D)))
    v = f32_to_bf16_bits(normal_f32(wl.seed + 2, (int(cu_k[-1]), wl.Hkv, wl.D)))
    inp = VarlenInputs(wl, q, k, v, cu_q, cu_k)
    if wl.bias_kind in (BIAS_T5, BIAS_T5U):
        inp.t5_table = normal_f32(wl.seed + 3, (wl.Hq, T5_NUM_BUCKETS))
    elif wl.bias_kind == BIAS_ALIBI:
        inp.t5_table = alibi_slopes(wl.Hq)
    return inp


def varlen_visible_pairs(wl: VarlenWorkload, key_lengths: Optional[list] = None) -> int:
    """Visible (query, key) pairs of one head summed over the sequences."""
    lq = wl.lengths()
    lk = list(key_lengths) if key_lengths is not None else lq
    return sum(visible_pairs(a, b, wl.mask_kind, wl.window) for a, b in zip(lq, lk) if a and b)


def small(wl: Workload, *, B=None, Hq=None, Hkv=None, Sq=None, Sk=None, window=None,
          name_suffix="small") -> Workload:
    """A reduced copy of a workload with the same kinds (for element-by-element parity)."""
    kw = {}
    for key, val in dict(B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, window=window).items():
        if val is not None:
            kw[key] = val
    return wl.replace(name=f"{wl.name}_{name_suffix}", **kw)


# ----------------------------------------------------------------------------------------------
# Work counts (index arithmetic only; used to price the run in FLOP and bytes)
# ----------------------------------------------------------------------------------------------
def visible_pairs(Sq: int, Sk: int, mask_kind: int, window: int = 0) -> int:
    """Number of (query, key) pairs the mask leaves visible in one (batch, head).

    Query i sits at absolute position i + (Sk - Sq) (bottom-right alignment). Pure counting.
    """
    off = Sk - Sq
    total = 0
    for i in range(Sq):
        p = i + off
        if mask_kind == MASK_NONE:
            total += Sk
            continue
        hi = min(p, Sk - 1)            # last visible key
        if hi < 0:
            continue
        lo = 0 if mask_kind == MASK_CAUSAL else max(0, p - window + 1)
        total += max(0, hi - lo + 1)
    return total


def effective_flops(wl: Workload) -> float:
    """4*D flop per visible pair (Q.K^T and P.V, 2 flop per multiply-add); exps not counted."""
    return 4.0 * wl.D * visible_pairs(wl.Sq, wl.Sk, wl.mask_kind, wl.window) * wl.B * wl.Hq


def algorithmic_bytes(wl: Workload) -> float:
    """Read q, k, v (and a full bias) once, write out and lse once."""
    es = 2 if wl.dtype == "bf16" else 4
    b = es * wl.B * wl.D * (2 * wl.Sq * wl.Hq + 2 * wl.Sk * wl.Hkv)
    b += 4 * wl.B * wl.Hq * wl.Sq
    if wl.bias_kind == BIAS_FULL:
        b += es * wl.B * wl.Hq * wl.Sq * wl.Sk
    elif wl.bias_kind == BIAS_T5:
        b += 4 * wl.Hq * T5_NUM_BUCKETS
    return float(b)


def decode_key_range(wl: Workload) -> int:
    """Keys of one (batch, KV head) that some query row may see (bottom-right alignment)."""
    off = wl.Sk - wl.Sq
    pmin, pmax = off, wl.Sq - 1 + off
    lo, hi = 0, wl.Sk - 1
    if wl.mask_kind != MASK_NONE:
        hi = min(hi, pmax)
    if wl.mask_kind == MASK_SLIDING:
        lo = max(0, pmin - wl.window + 1)
    return max(0, hi - lo + 1)


def algorithmic_bytes_decode(wl: Workload) -> float:
    """Decode (bf16): read the visible range of the K/V cache and q once, write out and lse
    once (plus a full bias, read once)."""
    es = 2
    b = es * wl.B * wl.Hkv * wl.D * 2 * decode_key_range(wl)
    b += es * wl.B * wl.D * 2 * wl.Sq * wl.Hq + 4 * wl.B * wl.Hq * wl.Sq
    if wl.bias_kind == BIAS_FULL:
        b += es * wl.B * wl.Hq * wl.Sq * wl.Sk
    elif wl.bias_kind == BIAS_T5:
        b += 4 * wl.Hq * T5_NUM_BUCKETS
    return float(b)


def algorithmic_bytes_bwd(wl: Workload) -> float:
    """One gradient call (bf16): read q, k, v, out, dout, lse (and a full bias) once, write dq,
    dk, dv once, and write then read the fp32 row sums rowsum(dout * out) once."""
    es = 2
    b = es * wl.B * wl.D * (4 * wl.Sq * wl.Hq + 4 * wl.Sk * wl.Hkv)
    b += (4 + 8) * wl.B * wl.Hq * wl.Sq
    if wl.bias_kind == BIAS_FULL:
        b += es * wl.B * wl.Hq * wl.Sq * wl.Sk
    elif wl.bias_kind == BIAS_T5:
        b += 4 * wl.Hq * T5_NUM_BUCKETS
    return float(b)
