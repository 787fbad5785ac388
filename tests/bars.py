"""Parity bars for attention outputs, shared by the GPU parity tests and the
CPU tests that show the bars can fail.

Contract bars (the path's stated tolerances): max |device - oracle| within
2e-2 on bf16 K/V and 6e-2 on fp8 K/V, both on the device's own table.

Detector bar (tighter, elementwise, derived from the device's arithmetic):

    |device - oracle| <= 5e-4 + 2^-8 (|oracle| + A),   A = sum_u p_u |V-hat_u| / sum_u p_u

with p the softmax weights of the oracle's attention (no sinks). The device
rounds the output to bf16 (at most 2^-9 |out|) and feeds each probability to
the PV products as one bf16 value (with a per-token V scale folded in first),
so the numerator is off by at most 2^-9 sum p |V-hat| = 2^-9 A times the
denominator; block partials kept in fp16 add at most about 2^-11 A. The
factor 2^-8 doubles that. The 5e-4 covers fp32 accumulation and fp16
subnormal floors. It is a detector, not a change of contract: an output
missing one selected block or holding one twice falls outside it
(tests/test_bars_cpu.py), while the contract bar can miss that on long rows.
"""
from __future__ import annotations

import numpy as np

from oracle import msa_oracle as O

ATOL_BF16 = 2e-2
ATOL_FP8 = 6e-2
DETECT_ATOL = 5e-4
DETECT_RTOL = 2.0 ** -8


def contract_atol(kv_dtype: int) -> float:
    return ATOL_FP8 if kv_dtype == 1 else ATOL_BF16


def oracle_and_abs_mean(b, table, ctx, rows):
    """The oracle's attention on a page-16 table (as attention_from_table) and,
    with the same weights, A = sum p |V-hat| / sum p for every (row, head,
    dim). Returns (ref, A), both [len(rows)][Hq][128]."""
    hq = b.num_q_heads
    ref = np.zeros((len(rows), hq, 128))
    amean = np.zeros((len(rows), hq, 128))
    hkv_n = b.k_cache.shape[1]
    group = hq // hkv_n
    for i, n in enumerate(rows):
        c = int(ctx[n])
        if c == 0:
            continue
        q = O.bf16_to_f64(b.q[n])
        for g in range(hkv_n):
            kh, vh = O._table_keys_values(b, table, n, c, g)
            hs = slice(g * group, (g + 1) * group)
            ref[i, hs] = O.softmax_attention(q[hs], kh, vh, b.sm_scale)
            amean[i, hs] = O.softmax_attention(q[hs], kh, np.abs(vh), b.sm_scale)
    return ref, amean


def detect_excess(out: np.ndarray, ref: np.ndarray, amean: np.ndarray) -> float:
    """Largest amount by which |out - ref| exceeds the detector bar (<= 0:
    within it)."""
    bar = DETECT_ATOL + DETECT_RTOL * (np.abs(ref) + amean)
    return float(np.max(np.abs(out - ref) - bar, initial=-np.inf))


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values at |x| (8 significant bits); the
    smallest normal spacing below 2^-126."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


# Zero-query coverage bar: |out - mean of V-hat| <= 1e-4 + bf16 half-ulp of
# the mean. With every logit 0 the probabilities are exactly 1 (bf16 too) and
# the sum is the exact integer ctx, so what remains is fp32 accumulation of at
# most a few thousand values of magnitude < 10 (below 1e-5 after the division
# by ctx), fp16 block partials on the block-major path (below 1e-5 here), and
# the output's bf16 rounding.
COVER_ATOL = 1e-4


def cover_excess(out: np.ndarray, mean: np.ndarray) -> float:
    return float(np.max(np.abs(out - mean) - (COVER_ATOL + bf16_half_ulp(mean)), initial=-np.inf))
