"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each case swaps one oracle helper for a plausible wrong version -- a wrong
index, a dropped term, a wrong sign, a wrong operand -- and re-runs a pin from
test_oracle_pins, expecting it to fail.
"""
import numpy as np
import pytest

import oracle.paged_attention as pa
from tests import test_oracle_pins as pins


def _bad_attend_no_normalise(qg, keys, values, sigma, key_counts=None):
    x = sigma * (qg @ keys.T)
    if key_counts is not None:
        x = np.where(np.arange(keys.shape[0])[None, :] < np.asarray(key_counts)[:, None], x, -np.inf)
    w = np.exp(x - x.max(axis=1, keepdims=True))
    return w @ values  # dropped the division by the sum of weights


def _bad_attend_keys_as_values(qg, keys, values, sigma, key_counts=None):
    return pa.__dict__["_orig_attend"](qg, keys, keys, sigma, key_counts)


def _bad_attend_unscaled(qg, keys, values, sigma, key_counts=None):
    return pa.__dict__["_orig_attend"](qg, keys, values, 1.0, key_counts)


def _bad_lse_merge(parts):
    ms = np.stack([p[0] for p in parts])
    M = ms.max(axis=0)
    sc = np.exp(M[None, :] - ms)  # wrong sign
    lam = sum(sc[i] * parts[i][1] for i in range(len(parts)))
    num = sum(sc[i][:, None] * parts[i][2] for i in range(len(parts)))
    return num / lam[:, None]


MUTATIONS = {
    "gqa_mapping_modulo": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "token_offset_off_by_one": ("token_location", lambda row, t: (int(row[t // 16]), (t + 1) % 16)),
    "token_block_index_swapped": ("token_location", lambda row, t: (int(row[t % len(row)]), t // 16 % 16)),
    "slot_fields_swapped": ("slot_location", lambda s: (s % 16, s // 16)),
    "causal_exclusive": ("causal_key_count", lambda p0, i: p0 + i),
    "scale_dropped": ("exact_scale", lambda s: 1.0),
    "no_normalisation": ("attend", _bad_attend_no_normalise),
    "keys_as_values": ("attend", _bad_attend_keys_as_values),
    "attend_unscaled": ("attend", _bad_attend_unscaled),
    "lse_sign": ("lse_merge", _bad_lse_merge),
    "gather_fast_wrong_transpose": ("gather_fast", lambda c, row, L: pa.gather(c, row[::-1], L)),
}

# The pins run against each mutation; at least one of them must fail.
PINS = [
    lambda: pins.test_single_token_returns_value_exactly("f32"),
    lambda: pins.test_uniform_keys_give_mean_of_values(),
    lambda: pins.test_two_tokens_logistic(),
    lambda: pins.test_toykv_code_semantics(),
    lambda: [pins.test_decode_matches_naive_recompute(s) for s in range(6)],
    lambda: [pins.test_prefill_matches_naive_recompute(s) for s in range(4)],
    lambda: pins.test_gqa_equals_mha_with_replicated_kv_heads(),
    lambda: [pins.test_partitioned_lse_merge_equals_plain(p) for p in (16, 48)],
    lambda: pins.test_write_round_trip_and_untouched_slots(),
    lambda: pins.test_write_then_gather_returns_rows(),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setitem(pa.__dict__, "_orig_attend", pa.attend)
    monkeypatch.setattr(pa, attr, bad)
    caught = []
    for i, pin in enumerate(PINS):
        try:
            pin()
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            caught.append(i)
    assert caught, f"mutation {name} passed every pin"
