"""The parity bars of the GPU tests, in one place, and a record of every comparison.

Bars (attention outputs against the float64 oracle):

* float32 inputs: row-normwise relative error ||o - r||_inf / ||r||_inf <= 1e-5
  per (row, head).
* bfloat16 inputs: max |o - r| <= 2e-2 (unit-variance values, float32
  accumulation), AND the row-normwise relative error <= 5 * 2^-9.  The
  absolute bar alone is as large as the whole output at long contexts (a
  64k-token row's outputs are ~0.02), where it would pass a result that
  skipped a 2048-token partition.  The relative bar is what the bf16 kernels'
  own roundings cost: the output is rounded to bf16 (at most one half-ulp,
  2^-9 of the row's largest entry) and the softmax weights are rounded to bf16
  before the value product (each weight's relative error is at most 2^-9 and
  the errors of different tokens are independent with zero mean, so they add
  up like a random walk against the row norm; four half-ulps cover it on the
  configs' own inputs, where a rounding model of both steps reaches 2.7).
  tests/test_parity_gates.py shows, on the CPU, that this bar accepts that
  rounding model and rejects a dropped partition or a dropped newest token.
* fp8 (E4M3) caches: |o - r| <= 2^-6 * max|V| of the (sequence, kv head)'s
  context (tests/test_gpu_fp8.py), AND a row-normwise relative error <= 2^-6.
  The roundings are the bf16 ones (weights times the per-token V scale, and
  the output, rounded to bf16), but the dequantised values are far from unit
  variance (codes uniform over the E4M3 bytes, scales spread over 2^-12..2^-6),
  so a few tokens carry most of a row and the weights' rounding errors add up
  less evenly: the rounding model reaches 3.8 half-ulps on the fp8 test cases,
  so the bar is eight.

Every attention comparison of the GPU tests is kept in RECORDS (`record`);
the test session prints them at its end (tests/conftest.py), so a quiet run still
shows each workload's absolute and relative error.
"""
from __future__ import annotations

import numpy as np

import oracle

F32_REL = 1e-5
BF16_ABS = 2e-2
BF16_REL = 5 * 2.0 ** -9
FP8_REL = 8 * 2.0 ** -9

RECORDS: list = []


def attn_errors(got, ref):
    """(max abs error, max row-normwise relative error) of got against ref (rows = last axis)."""
    return oracle.max_abs_err(got, ref), oracle.max_rownorm_rel_err(got, ref)


def within_bar(got, ref, dtype) -> bool:
    """True when got meets the bar for its input dtype (NaN never does)."""
    a, r = attn_errors(got, ref)
    if dtype == "f32":
        return r <= F32_REL
    return a <= BF16_ABS and r <= BF16_REL


def record(what, dtype, abs_err, rel_err):
    RECORDS.append((what, dtype, abs_err, rel_err))
