"""Planted mistakes in the oracle: each one must fail at least one pin.

A pin that no plausible mistake can fail pins nothing, so each mistake below
is planted into the oracle (monkeypatched, on the CPU) and the pins of that
part -- the test functions of tests/test_oracle_route.py,
test_oracle_dispatch.py, test_oracle_layer.py and test_oracle_fp8.py, run
unchanged -- must reject it.  The real oracle passes all of them.

Sources of the rules the mistakes break: sparse-activation page §3.2 stage 2
(rank the logits, keep the top k), §2.3 (per-expert load and capacity); NCCL
EP page §2.1 (LL combine: the gate-weighted sum; FP8 expert compute with a
scale tensor), §2.2 (compact expert-major layout); DWDP page, key
optimisations (W1 and W3 as the fused first-layer operand, SwiGLU).
"""
import numpy as np
import pytest

import test_oracle_dispatch as PD
import test_oracle_fp8 as PF
import test_oracle_layer as PL
import test_oracle_route as PR
from oracle import fp8_oracle as F
from oracle import moe_oracle as O

_REAL_ROUTE = O.route
_REAL_GATES = O.gate_values
_REAL_DISPATCH = O.dispatch


def _fails(pins):
    """Names of the pins that reject the oracle as currently patched."""
    failed = []
    for name, fn in pins:
        try:
            fn()
        except (AssertionError, pytest.fail.Exception):
            failed.append(name)
    return failed


# ----------------------------------------------------------------- routing
ROUTE_PINS = [
    ("brute force, coarse ties E=8 k=2", lambda: PR.test_topk_matches_brute_force(8, 2)),
    ("brute force, coarse ties E=64 k=8", lambda: PR.test_topk_matches_brute_force(64, 8)),
    ("brute force, tiny workload", PR.test_topk_brute_force_on_tiny_workload),
    ("all-equal rows, softmax k=2", lambda: PR.test_all_equal_rows(2, O.GATE_SOFTMAX)),
    ("all-equal rows, sigmoid k=8", lambda: PR.test_all_equal_rows(8, O.GATE_SIGMOID)),
    ("signed zeros", PR.test_signed_zero_ties_lower_index_wins),
    ("dominant logit first", PR.test_dominant_logit_first),
    ("textbook softmax", PR.test_softmax_then_topk_then_renorm_equals_oracle),
    ("sigmoid closed form", PR.test_sigmoid_pair_closed_form),
    ("sigmoid vs softmax", PR.test_sigmoid_gates_differ_from_softmax_gates),
    ("invariants, tiny workload", lambda: PR.test_invariants_on_workloads("tiny_fp32")),
    ("invariants, DeepSeek decode", lambda: PR.test_invariants_on_workloads("dsv3_decode")),
]


def _route_variant(ties_high=False, zero_by_sign=False, worst_first=False):
    """The oracle's route with one selection mistake."""
    def route(logits_f32, k, gate):
        l32 = np.asarray(logits_f32, dtype=np.float32)
        T, E = l32.shape
        if not (1 <= k <= E):
            raise ValueError("k")
        if not np.all(np.isfinite(l32)):
            raise ValueError("logits")
        if not zero_by_sign:
            l32 = l32 + np.float32(0.0)
        l64 = l32.astype(np.float64)
        e_key = np.broadcast_to(np.arange(E), (T, E))
        if ties_high:
            order = np.lexsort((-e_key, -l64), axis=-1)[:, :k]
        elif zero_by_sign:      # +0.0 ranked above -0.0 whatever the indices
            order = np.lexsort((e_key, np.signbit(l32), -l64), axis=-1)[:, :k]
        else:
            order = np.lexsort((e_key, -l64), axis=-1)[:, :k]
        if worst_first:
            order = order[:, ::-1]
        sel = np.take_along_axis(l64, order, axis=-1)
        return order.astype(np.int32), O.gate_values(sel, gate)
    return route


def _gates_full_softmax(sel, gate):
    """Softmax gates scaled by the k chosen logits' share of a softmax over
    the chosen logits plus the next-best one: not renormalised over the k."""
    sel = np.asarray(sel, np.float64)
    if gate == O.GATE_SOFTMAX:
        z = np.exp(sel - sel[:, :1])
        return z / (z.sum(axis=1, keepdims=True) + np.exp(sel[:, -1:] - sel[:, :1]))
    return _REAL_GATES(sel, gate)


def _gates_sigmoid_unnormalised(sel, gate):
    sel = np.asarray(sel, np.float64)
    if gate == O.GATE_SIGMOID:
        return 1.0 / (1.0 + np.exp(-sel))
    return _REAL_GATES(sel, gate)


def _gates_swapped(sel, gate):
    other = O.GATE_SIGMOID if gate == O.GATE_SOFTMAX else O.GATE_SOFTMAX
    return _REAL_GATES(sel, other)


def _gates_no_shift_sign(sel, gate):
    """softmax taken of the negated logits (a sign slip)."""
    if gate == O.GATE_SOFTMAX:
        return _REAL_GATES(-np.asarray(sel, np.float64), gate)
    return _REAL_GATES(sel, gate)


def test_real_route_passes_every_pin():
    assert _fails(ROUTE_PINS) == []


@pytest.mark.parametrize("mistake", [
    ("ties to the higher index", dict(route=_route_variant(ties_high=True))),
    ("-0.0 ranked below +0.0", dict(route=_route_variant(zero_by_sign=True))),
    ("worst first", dict(route=_route_variant(worst_first=True))),
    ("softmax not renormalised over k", dict(gate_values=_gates_full_softmax)),
    ("sigmoid gates not normalised", dict(gate_values=_gates_sigmoid_unnormalised)),
    ("gate rules swapped", dict(gate_values=_gates_swapped)),
    ("softmax of negated logits", dict(gate_values=_gates_no_shift_sign)),
], ids=lambda m: m[0])
def test_planted_route_mistake_fails_a_pin(mistake, monkeypatch):
    name, patch = mistake
    for attr, fn in patch.items():
        monkeypatch.setattr(O, attr, fn)
    assert _fails(ROUTE_PINS), f"planted mistake '{name}' passes every routing pin"


# ----------------------------------------------------------------- dispatch
DISPATCH_PINS = [
    ("capacity rounding", PD.test_capacity_rounding_and_none),
    ("page's worked capacity example", PD.test_capacity_worked_example_from_page),
    ("stable argsort", lambda: PD.test_uncapped_full_range_is_stable_argsort(64, 8, 2)),
    ("position = earlier tokens", PD.test_position_is_count_of_earlier_tokens),
    ("hand-worked plan", PD.test_hand_worked_plan),
    ("invariants, capacity 5", lambda: PD.test_plan_invariants(5, 0, 16)),
    ("invariants, local range", lambda: PD.test_plan_invariants(5, 4, 9)),
    ("latest tokens drop", PD.test_dropped_pairs_are_the_latest_tokens),
    ("permute copies rows", PD.test_permute_is_row_copy),
]


def _dispatch_capacity_off_by_one(topk_idx, E, capacity=-1, e_begin=0, e_end=None):
    return _REAL_DISPATCH(topk_idx, E, capacity + 1 if capacity >= 0 else capacity, e_begin, e_end)


def _dispatch_remote_as_dropped(topk_idx, E, capacity=-1, e_begin=0, e_end=None):
    p = _REAL_DISPATCH(topk_idx, E, capacity, e_begin, e_end)
    pp = p["pair_pos"].copy()
    pp[pp == O.REMOTE] = O.DROPPED
    return dict(p, pair_pos=pp)


def _dispatch_segments_descending(topk_idx, E, capacity=-1, e_begin=0, e_end=None):
    p = _REAL_DISPATCH(topk_idx, E, capacity, e_begin, e_end)
    sp, off = p["sorted_pair"].copy(), p["offsets"]
    for i in range(len(off) - 1):
        sp[off[i]:off[i + 1]] = sp[off[i]:off[i + 1]][::-1]
    pp = p["pair_pos"].copy()
    pp[sp] = np.arange(len(sp), dtype=pp.dtype)
    return dict(p, sorted_pair=sp, pair_pos=pp)


def _dispatch_offsets_inclusive(topk_idx, E, capacity=-1, e_begin=0, e_end=None):
    p = _REAL_DISPATCH(topk_idx, E, capacity, e_begin, e_end)
    off = p["offsets"]
    return dict(p, offsets=np.concatenate([off[1:], off[-1:]]).astype(off.dtype))


def _dispatch_pos_from_one(topk_idx, E, capacity=-1, e_begin=0, e_end=None):
    p = _REAL_DISPATCH(topk_idx, E, capacity, e_begin, e_end)
    return dict(p, pos=p["pos"] + 1)


def _capacity_floor(T, k, E, capacity_factor):
    if capacity_factor is None:
        return -1
    from fractions import Fraction
    return int(Fraction(str(capacity_factor)) * T * k / E)


def _permute_by_pair(x, sorted_pair, k):       # forgot the // k
    return np.asarray(x)[np.asarray(sorted_pair, np.int64) % len(x)]


def test_real_dispatch_passes_every_pin():
    assert _fails(DISPATCH_PINS) == []


@pytest.mark.parametrize("mistake", [
    ("capacity off by one", dict(dispatch=_dispatch_capacity_off_by_one)),
    ("remote pairs marked dropped", dict(dispatch=_dispatch_remote_as_dropped)),
    ("segments in descending token order", dict(dispatch=_dispatch_segments_descending)),
    ("inclusive offsets", dict(dispatch=_dispatch_offsets_inclusive)),
    ("positions counted from one", dict(dispatch=_dispatch_pos_from_one)),
    ("capacity rounded down", dict(capacity=_capacity_floor)),
    ("permute by pair index", dict(permute=_permute_by_pair)),
], ids=lambda m: m[0])
def test_planted_dispatch_mistake_fails_a_pin(mistake, monkeypatch):
    name, patch = mistake
    for attr, fn in patch.items():
        monkeypatch.setattr(O, attr, fn)
    assert _fails(DISPATCH_PINS), f"planted mistake '{name}' passes every dispatch pin"


# ----------------------------------------------------------------- expert FFN and combine
LAYER_PINS = [
    ("single expert = textbook SwiGLU", PL.test_single_expert_reduces_to_plain_swiglu),
    ("dense masked brute force", lambda: PL.test_layer_equals_dense_masked_brute_force(
        dict(T=64, d=32, f=48, E=8, k=2, dtype="f32"))),
    ("identical experts", PL.test_identical_experts_give_plain_ffn),
    ("W2 = 0", PL.test_zero_down_projection_gives_zero),
    ("one-hot rows reproduce gates", PL.test_combine_one_hot_rows_reproduce_gates),
    ("dropped and remote skipped", PL.test_combine_skips_dropped_and_remote),
    ("silu against torch", PL.test_silu_against_library),
    ("token outputs", PL.test_token_outputs_match_layer),
]

_REAL_COMBINE = O.combine
_REAL_HIDDEN = O.swiglu_hidden


def _silu_no_product(a):
    return 1.0 / (1.0 + np.exp(-a))


def _hidden_w1_w3_swapped(x64, w1, w3):
    return _REAL_HIDDEN(x64, w3, w1)


def _combine_unweighted(y_perm64, pair_pos, topk_w):
    return _REAL_COMBINE(y_perm64, pair_pos, np.ones_like(np.asarray(topk_w, np.float64)))


def _combine_keeps_remote(y_perm64, pair_pos, topk_w):
    """remote pairs (-2) read a row from the end of y_perm (a negative index)."""
    w = np.asarray(topk_w, np.float64)
    T, k = w.shape
    y = np.zeros((T, y_perm64.shape[1] if y_perm64.ndim == 2 else 0))
    pp = np.asarray(pair_pos).reshape(T, k)
    for t in range(T):
        for j in range(k):
            if pp[t, j] != O.DROPPED and len(y_perm64):
                y[t] += w[t, j] * y_perm64[pp[t, j]]
    return y


def _combine_slot_order_swapped(y_perm64, pair_pos, topk_w):
    return _REAL_COMBINE(y_perm64, pair_pos, np.asarray(topk_w, np.float64)[:, ::-1])


def test_real_layer_passes_every_pin():
    assert _fails(LAYER_PINS) == []


@pytest.mark.parametrize("mistake", [
    ("silu without the product", dict(silu=_silu_no_product)),
    ("W1 and W3 swapped", dict(swiglu_hidden=_hidden_w1_w3_swapped)),
    ("unweighted combine", dict(combine=_combine_unweighted)),
    ("remote pairs combined", dict(combine=_combine_keeps_remote)),
    ("gate slots swapped", dict(combine=_combine_slot_order_swapped)),
], ids=lambda m: m[0])
def test_planted_layer_mistake_fails_a_pin(mistake, monkeypatch):
    name, patch = mistake
    for attr, fn in patch.items():
        monkeypatch.setattr(O, attr, fn)
    assert _fails(LAYER_PINS), f"planted mistake '{name}' passes every layer pin"


# ----------------------------------------------------------------- FP8 weights
FP8_PINS = [
    ("defining code values", PF.test_defining_values),
    ("codes ascending", PF.test_positive_codes_are_ascending_and_distinct),
    ("brute-force nearest code", PF.test_encode_matches_brute_force_nearest),
    ("round trip", PF.test_round_trip_of_every_finite_code),
    ("hand block", PF.test_block_scale_hand_example),
    ("power-of-two hand blocks", PF.test_power_of_two_scale_hand_example),
    ("zero block, independence", PF.test_zero_block_and_block_independence),
    ("scale property, error bound", PF.test_block_scale_property_and_error_bound),
    ("representable weights", PF.test_representable_weights_reduce_to_the_bf16_ffn),
]

_REAL_DECODE = F.e4m3_decode
_REAL_QUANT = F.quantize_blocks
_REAL_EW = F.expert_weights


def _encode_variant(ties_away=False, saturate=True, min_exp=-6):
    """The oracle's encoder with one rounding mistake."""
    def enc(x):
        x = np.asarray(x, dtype=np.float32)
        a = np.abs(x.astype(np.float64))
        neg = np.signbit(x)
        _, ex = np.frexp(np.where(a > 0, a, 1.0))
        e = np.maximum(ex - 1, min_exp)
        quantum = np.ldexp(1.0, e - 3)
        q = np.floor(a / quantum + 0.5) if ties_away else np.rint(a / quantum)
        v = q * quantum
        if saturate:
            v = np.minimum(v, F.E4M3_MAX)
        code = np.minimum(np.searchsorted(F._POS, v), 0x7F).astype(np.int64)
        return (code | np.where(neg, 0x80, 0)).astype(np.uint8)
    return enc


def _decode_variant(bias=7, sub_exp=-9):
    def dec(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0)
        e = (c >> 3) & 0xF
        m = c & 0x7
        v = sign * np.where(e == 0, np.ldexp(m.astype(np.float64), sub_exp),
                            np.ldexp(1.0 + m / 8.0, e - bias))
        return np.where((c & 0x7F) == 0x7F, np.nan, v)
    return dec


def _quantize_with_scale(scale_of):
    """The oracle's quantiser with another block-scale rule (scale_of(amax))."""
    def quant(w_bits):
        w_bits = np.asarray(w_bits, dtype=np.uint16)
        E, R, K = w_bits.shape
        w = (w_bits.astype(np.uint32) << 16).view(np.float32)
        blocks = w.reshape(E, R // 128, 128, K // 128, 128)
        amax = np.abs(blocks).max(axis=(2, 4)).astype(np.float64)
        scale = np.where(amax > 0, scale_of(np.where(amax > 0, amax, 1.0)), 1.0).astype(np.float32)
        ratio = (blocks / scale[:, :, None, :, None]).astype(np.float32)
        return F.e4m3_encode(ratio).reshape(E, R, K), scale
    return quant


def _mx_floor_scale(amax):
    # the microscaling rule 2^(floor(log2 amax) - 8): its top binade saturates
    _, ex = np.frexp(amax)
    return np.ldexp(1.0, ex - 1 - 8)


def _expert_weights_swapped(w13_codes, w13_scale, w2_codes, w2_scale, f):
    real = _REAL_EW(w13_codes, w13_scale, w2_codes, w2_scale, f)

    def weights(i):
        w1, w3, w2 = real(i)
        return w3, w1, w2
    return weights


def test_real_fp8_oracle_passes_every_pin():
    assert _fails(FP8_PINS) == []


@pytest.mark.parametrize("mistake", [
    ("ties away from zero", dict(e4m3_encode=_encode_variant(ties_away=True))),
    ("no saturation at 448", dict(e4m3_encode=_encode_variant(saturate=False))),
    ("subnormal quantum 2^-10 in the encoder", dict(e4m3_encode=_encode_variant(min_exp=-7))),
    ("exponent bias 8", dict(e4m3_decode=_decode_variant(bias=8))),
    ("subnormal scale 2^-10 in the decoder", dict(e4m3_decode=_decode_variant(sub_exp=-10))),
    ("scale = amax / 448 (not a power of two)",
     dict(quantize_blocks=_quantize_with_scale(lambda a: (a.astype(np.float32) / np.float32(448.0))))),
    ("scale = 2^(floor(log2 amax) - 8)", dict(quantize_blocks=_quantize_with_scale(_mx_floor_scale))),
    ("scale one power of two too large",
     dict(quantize_blocks=_quantize_with_scale(lambda a: np.ldexp(1.0, F.scale_exponent(a) + 1)))),
    ("W1 and W3 swapped", dict(expert_weights=_expert_weights_swapped)),
], ids=lambda m: m[0])
def test_planted_fp8_mistake_fails_a_pin(mistake, monkeypatch):
    name, patch = mistake
    for attr, fn in patch.items():
        monkeypatch.setattr(F, attr, fn)
    assert _fails(FP8_PINS), f"planted mistake '{name}' passes every FP8 pin"
