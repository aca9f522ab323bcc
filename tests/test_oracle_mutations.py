"""Mistakes planted in the oracle are caught by its pins.

Each case below replaces one oracle function (for that test only, on the
CPU) with a plausible mistake: a dropped term, a wrong sign, index or axis,
a transposed or swapped operand, a wrong rounding, an off-by-one.  Then it
runs the oracle's own pin tests unchanged and requires at least one of them
to fail.  A mutant no pin catches would mean that part of the oracle is not
really pinned."""
import heapq
import importlib.util
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import planner as P
from oracle import quant as Q
from oracle import splitzip as Z

HERE = os.path.dirname(os.path.abspath(__file__))


def _load(name):
    spec = importlib.util.spec_from_file_location(f"_pins_{name}", os.path.join(HERE, name + ".py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


TA = _load("test_oracle_attention")
TQ = _load("test_oracle_quant")
TP = _load("test_oracle_planner")
TZ = _load("test_oracle_splitzip")

ATTENTION_PINS = [
    lambda: TA.test_uniform_budgets_equal_dense_sdpa(
        "llama8b", dict(B=2, ctx=("uniform", 200, 500), ratio_ppm=(1_000_000, 1_000_000), n_clusters=1)),
    TA.test_single_row_returns_its_value_row,
    TA.test_closed_forms,
    TA.test_matches_pure_python_brute_force,
    TA.test_lse_merge_split_invariance,
    TA.test_int8_rows_equal_attention_over_same_bf16_values,
    TA.test_workload_tier_rows_oldest_quantised_newest_exact,
    TA.test_gqa_mapping_and_scale_default,
]
QUANT_PINS = [TQ.test_error_bounded_by_half_step_and_absmax_hits_127,
              TQ.test_integer_multiples_of_power_of_two_step_round_trip_exactly,
              TQ.test_ties_round_to_even, TQ.test_zero_block_and_sign_symmetry_and_saturation,
              TQ.test_rows_are_quantised_block_by_block]
PLANNER_PINS = [TP.test_hand_worked_budgets_clusters_tables_plan, TP.test_hand_worked_tier_split,
                TP.test_hand_worked_rounding_directions,
                TP.test_tiered_128k_split_matches_workload_statement, TP.test_hand_worked_sharing_and_release,
                TP.test_radix_lesson_block_counts, TP.test_hand_worked_group_items]


def _caught(pins) -> bool:
    for pin in pins:
        try:
            pin()
        except Exception:  # an assertion, or the mutant breaking a shape
            return True
    return False


# ------------------------------------------------------------------ attention mutants
def _attend_no_scale(q, K, V, scale):
    s = np.asarray(K, np.float64) @ np.asarray(q, np.float64).T
    p = np.exp(s - s.max(axis=0))
    return (p.T @ np.asarray(V, np.float64)) / p.sum(axis=0)[:, None]


def _attend_wrong_axis(q, K, V, scale):  # softmax over the heads instead of the rows
    s = (np.asarray(K, np.float64) @ np.asarray(q, np.float64).T) * scale
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    return p.T @ np.asarray(V, np.float64)


def _attend_keys_as_values(q, K, V, scale):
    return TA_ORIG_ATTEND(q, K, K, scale)


def _attend_no_normaliser(q, K, V, scale):
    s = (np.asarray(K, np.float64) @ np.asarray(q, np.float64).T) * scale
    p = np.exp(s - s.max(axis=0))
    return p.T @ np.asarray(V, np.float64)


def _merge_sign(m, l, acc):
    m = np.asarray(m, np.float64)
    w = np.exp(m.max(axis=0) - m)
    return (w[:, :, None] * np.asarray(acc, np.float64)).sum(axis=0) / (w * np.asarray(l, np.float64)).sum(axis=0)[:, None]


def _merge_unweighted_l(m, l, acc):
    m = np.asarray(m, np.float64)
    w = np.exp(m - m.max(axis=0))
    return (w[:, :, None] * np.asarray(acc, np.float64)).sum(axis=0) / np.asarray(l, np.float64).sum(axis=0)[:, None]


def _rows_off_by_one(K16, V16, n_i8, qb, bits=8):
    return TA_ORIG_ROWS(K16, V16, max(n_i8 - 1, 0), qb, bits)


def _rows_k_only(K16, V16, n_i8, qb, bits=8):
    K, _ = TA_ORIG_ROWS(K16, V16, n_i8, qb, bits)
    return K, A.bf16_to_f64(V16)


TA_ORIG_ATTEND = A.attend
TA_ORIG_ROWS = A.rows_f64


# ------------------------------------------------------------------ bf16 decoder mutants
def _bf16_shift_15(u):  # the pattern moved one bit short of the fp32 high half
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)


def _bf16_as_fp16(u):  # the bits read as IEEE half precision
    return np.asarray(u, dtype=np.uint16).view(np.float16).astype(np.float64)


def _bf16_sign_dropped(u):  # the sign bit masked off
    return (((np.asarray(u, dtype=np.uint16) & np.uint16(0x7FFF)).astype(np.uint32)) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def _bf16_fraction_truncated(u):  # the lowest fraction bit lost
    return (((np.asarray(u, dtype=np.uint16) & np.uint16(0xFFFE)).astype(np.uint32)) << np.uint32(16)).view(
        np.float32).astype(np.float64)


BF16_PINS = [TA.test_bf16_decoder_on_fixed_patterns, TA.test_bf16_decoder_on_every_pattern,
             lambda: TA.test_q_f64_decodes_the_query_bits("llama8b"),
             lambda: TA.test_uniform_budgets_equal_dense_sdpa(
                 "llama8b", dict(B=2, ctx=("uniform", 200, 500), ratio_ppm=(1_000_000, 1_000_000), n_clusters=1))]


@pytest.mark.parametrize("mutant", [_bf16_shift_15, _bf16_as_fp16, _bf16_sign_dropped, _bf16_fraction_truncated],
                         ids=["shift-15", "read-as-fp16", "sign-dropped", "fraction-bit-lost"])
def test_bf16_decoder_mutants_are_caught(monkeypatch, mutant):
    """A wrong bf16 decoder is caught by its own pins and, through q_f64 and
    the row decoding, by the dense-SDPA pin (whose rows are decoded from the
    format's fields, not by this function)."""
    monkeypatch.setattr(A, "bf16_to_f64", mutant)
    with np.errstate(all="ignore"):
        assert _caught(BF16_PINS), f"no pin catches the {mutant.__name__} mutant of bf16_to_f64"
        # the end-to-end pin alone must catch it too: it never calls the decoder under test for its reference
        assert _caught(BF16_PINS[3:]), f"the dense-SDPA pin misses the {mutant.__name__} mutant"


def test_q_f64_mutant_is_caught(monkeypatch):
    """q_f64 reading bf16 queries as fp16 is caught by the query pin and by
    the dense-SDPA pin."""
    monkeypatch.setattr(A, "q_f64", lambda w: np.asarray(w.q(), np.float64) if w.q_dtype == "f32"
                        else _bf16_as_fp16(w.q()))
    with np.errstate(all="ignore"):
        assert _caught(BF16_PINS[2:3]) and _caught(BF16_PINS[3:])


@pytest.mark.parametrize("target,mutant", [
    ("attend", _attend_no_scale), ("attend", _attend_wrong_axis), ("attend", _attend_keys_as_values),
    ("attend", _attend_no_normaliser), ("lse_merge", _merge_sign), ("lse_merge", _merge_unweighted_l),
    ("rows_f64", _rows_off_by_one), ("rows_f64", _rows_k_only),
], ids=["no-scale", "softmax-over-heads", "keys-as-values", "no-normaliser", "merge-sign", "merge-unweighted-l",
        "int8-rows-off-by-one", "int8-values-not-dequantised"])
def test_attention_mutants_are_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(A, target, mutant)
    assert _caught(ATTENTION_PINS), f"no pin catches the {mutant.__name__} mutant of {target}"


# ------------------------------------------------------------------ quantiser mutants
QB_ORIG = Q.quantize_block
BS_ORIG = Q.block_scale


def _scale_over_128(x, bits=8):
    x = np.asarray(x, np.float32)
    return (np.max(np.abs(x), axis=0) / np.float32(128 if bits == 8 else 8)).astype(np.float16)


def _scale_not_fp16(x, bits=8):  # the scale kept in fp32, so a code is not the stored scale's
    s = np.max(np.abs(np.asarray(x, np.float32)), axis=0) / np.float32(Q.qmax_of(bits))
    return s.astype(np.float32).view(np.float32)


def _round_half_up(x, bits=8):
    x = np.asarray(x, np.float32)
    qm = Q.qmax_of(bits)
    s = Q.block_scale(x, bits)
    sf = s.astype(np.float32)
    safe = np.where(sf > 0, sf, np.float32(1))
    y = np.floor(x / safe + np.float32(0.5))
    return np.where(sf > 0, np.clip(y, -qm, qm), 0).astype(np.int8), s


def _clamp_128(x, bits=8):
    x = np.asarray(x, np.float32)
    s = Q.block_scale(x, bits)
    sf = s.astype(np.float32)
    safe = np.where(sf > 0, sf, np.float32(1))
    y = np.rint(x / safe * np.float32(1.004))  # saturates just past the code range
    return np.where(sf > 0, np.clip(y, -128, 127), 0).astype(np.int8), s


def _qmax_int4_as_8(bits):  # a 4-bit code taken as 0..15 magnitude 8
    return 127 if bits == 8 else 8


INT4_PINS = [TQ.test_int4_error_bounded_and_absmax_hits_7, TQ.test_int4_exact_round_trip_and_ties,
             TQ.test_int4_is_coarser_than_int8_on_the_same_block,
             TA.test_int4_workload_rows_within_half_a_step_and_exact_multiples]


def test_int4_code_range_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(Q, "qmax_of", _qmax_int4_as_8)
    assert _caught(INT4_PINS), "no pin catches an INT4 code range of +-8"


@pytest.mark.parametrize("target,mutant", [
    ("block_scale", _scale_over_128), ("block_scale", _scale_not_fp16),
    ("quantize_block", _round_half_up), ("quantize_block", _clamp_128),
], ids=["scale-over-128", "scale-not-fp16", "round-half-up", "overshoot-and-clamp-128"])
def test_quantiser_mutants_are_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(Q, target, mutant)
    assert _caught(QUANT_PINS), f"no pin catches the {mutant.__name__} mutant of {target}"


# ------------------------------------------------------------------ planner mutants
RATIO_ORIG = P.ratio_ppm
ALLOC_ORIG = P.Pool.alloc


def _ratio_reversed_rank(k, H, hi, lo):
    return RATIO_ORIG(H - 1 - k, H, hi, lo)


def _ratio_rounds_up(k, H, hi, lo):
    return hi if H == 1 else hi - (-((-(hi - lo) * k) // (H - 1)))


def _tier_floor(L, recent_ppm, quant_block):
    old = L - (L * recent_ppm) // P.PPM
    i8 = (old // quant_block) * quant_block
    return i8, L - i8


def _tier_unaligned(L, recent_ppm, quant_block):
    i8 = L - P._ceil_div(L * recent_ppm, P.PPM)
    return i8, L - i8


def _alloc_reversed(self, c, t):
    # hand out the highest page id first instead of the lowest
    free = [p for p in range(self.cap[c][t]) if self.ref[c][t].get(p, 0) == 0]
    if not free:
        raise P.OracleError("ENOMEM", "exhausted")
    pid = free[-1]
    self.ref[c][t][pid] = 1
    if pid >= self.top[c][t]:
        self.top[c][t] = pid + 1
    h = self.heap[c][t]
    if pid in h:
        h.remove(pid)
        heapq.heapify(h)
    return pid


@pytest.mark.parametrize("target,mutant", [
    ("ratio_ppm", _ratio_reversed_rank), ("ratio_ppm", _ratio_rounds_up),
    ("tier_split", _tier_floor), ("tier_split", _tier_unaligned),
], ids=["rank-reversed", "ratio-rounded-up", "tier-floor", "tier-not-block-aligned"])
def test_planner_mutants_are_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(P, target, mutant)
    assert _caught(PLANNER_PINS), f"no pin catches the {mutant.__name__} mutant of {target}"


def test_allocation_order_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(P.Pool, "alloc", _alloc_reversed)
    assert _caught(PLANNER_PINS), "no pin catches highest-free-first allocation"


def test_pins_pass_on_the_oracle_as_it_is():
    """The control: unmutated, every pin used above passes."""
    for pins in (ATTENTION_PINS, QUANT_PINS, INT4_PINS, PLANNER_PINS, BF16_PINS):
        assert not _caught(pins)


# ------------------------------------------------------------------ plan, growth and codec mutants
PLAN_PINS = [TP.test_hand_worked_budgets_clusters_tables_plan, TP.test_hand_worked_group_items,
             lambda: TP.test_invariants("llama8b"), lambda: TP.test_invariants("radix"),
             lambda: TP.test_longest_first_order_follows_bytes_read(8, (64, 128)),
             lambda: TP.test_longest_first_order_follows_bytes_read(4, (128, 192))]
GROWTH_PINS = [lambda: TP.test_append_steps_follow_the_tier_split(125_000, 64),
               lambda: TP.test_append_steps_follow_the_tier_split(300_000, 64),
               TP.test_capacity_is_the_largest_split_on_the_way,
               TP.test_incremental_blocks_equal_blocks_of_the_whole_sequence,
               lambda: TP.test_growth_plan_item_counts_follow_the_live_rows(128, (512, 1792)),
               TP.test_growth_tables_cover_capacity_and_keep_live_lengths]
CODEC_PINS = [TZ.test_hand_worked_buffer, TZ.test_round_trips_bit_exact, TZ.test_codebook_is_the_sixteen_most_frequent]
SPLIT_ORIG = P.split_range
CODEBOOK_ORIG = Z.codebook


def _split_one_more(lo, hi, unit, chunk, hi_live=None):  # one item too many
    u = P._ceil_div(hi - lo, unit)
    if u <= 0:
        return []
    k = P._ceil_div(u, chunk // unit) + 1
    k = min(k, u)
    return [(lo + (i * u // k) * unit, min(lo + ((i + 1) * u // k) * unit, hi)) for i in range(k)]


def _split_ceil_starts(lo, hi, unit, chunk, hi_live=None):  # item i starts at ceil(i u / k)
    u = P._ceil_div(hi - lo, unit)
    if u <= 0:
        return []
    k = P._ceil_div(u, chunk // unit) if hi_live is None else max(
        1, P._ceil_div(P._ceil_div(max(hi_live - lo, 0), unit), chunk // unit), P._ceil_div(u, 2 * (chunk // unit)))
    st = [lo + P._ceil_div(i * u, k) * unit for i in range(k)] + [hi]
    return [(st[i], min(st[i + 1], hi)) for i in range(k)]


def _lpt_swapped(tier, quant_block, old_bits):
    return old_bits * quant_block + 16 if tier == P.TIER_BF else 16 * quant_block


def _append_ages_a_row(n_i8, n_bf, recent_ppm, quant_block):  # ages when the boundary passes a row, not a block
    n_bf += 1
    old = n_i8 + n_bf - P._ceil_div((n_i8 + n_bf) * recent_ppm, P.PPM)
    if old - n_i8 >= 1 and n_bf > quant_block:
        return n_i8 + quant_block, n_bf - quant_block, True
    return n_i8, n_bf, False


def _codebook_ties_to_larger(x):
    counts = np.bincount(Z.exponents(x), minlength=256)
    order = sorted(range(256), key=lambda e: (-counts[e], -e))
    return np.array(order[:16], dtype=np.uint8)


def _codebook_least_frequent(x):
    counts = np.bincount(Z.exponents(x), minlength=256)
    seen = [e for e in range(256) if counts[e] > 0]
    order = sorted(seen, key=lambda e: (counts[e], e)) + [e for e in range(256) if counts[e] == 0]
    return np.array(order[:16], dtype=np.uint8)


@pytest.mark.parametrize("module,target,mutant,pins", [
    (P, "split_range", _split_one_more, PLAN_PINS), (P, "split_range", _split_ceil_starts, PLAN_PINS),
    (P, "lpt_weight", _lpt_swapped, PLAN_PINS), (P, "append_step", _append_ages_a_row, GROWTH_PINS),
    (Z, "codebook", _codebook_ties_to_larger, CODEC_PINS), (Z, "codebook", _codebook_least_frequent, CODEC_PINS),
], ids=["plan-one-item-too-many", "plan-starts-rounded-up", "lpt-weights-swapped", "ageing-by-row",
        "codebook-ties-to-larger", "codebook-least-frequent"])
def test_plan_growth_codec_mutants_are_caught(monkeypatch, module, target, mutant, pins):
    monkeypatch.setattr(module, target, mutant)
    assert _caught(pins), f"no pin catches the {mutant.__name__} mutant of {target}"


def test_plan_growth_codec_pins_pass_unmutated():
    for pins in (PLAN_PINS, GROWTH_PINS, CODEC_PINS):
        assert not _caught(pins)
