"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case patches one oracle routine with a plausible bug (wrong tie rule,
dropped term, swapped axis, wrong sign, missing saturation, wrong GQA index)
and checks that the corresponding pin test then fails.
"""
import numpy as np
import pytest

import oracle.attention as A
import oracle.cache as C
import oracle.quant as Q
from tests import test_oracle_pins as P


def _all_assertions(e):
    """True when e is an AssertionError, or a group of them (hypothesis raises
    an exception group when it finds several distinct failing examples)."""
    if isinstance(e, AssertionError):
        return True
    subs = getattr(e, "exceptions", None)
    return bool(subs) and all(_all_assertions(x) for x in subs)


def _fails(fn, *args):
    try:
        fn(*args)
    except Exception as e:  # noqa: BLE001  (only assertion failures count)
        if _all_assertions(e):
            return True
        raise
    return False


def test_round_half_away_is_caught(monkeypatch):
    monkeypatch.setattr(Q.np, "rint", lambda x: np.trunc(x + np.copysign(0.5, x)))
    assert _fails(P.test_asym_ties_round_to_even)


def test_dropped_zero_point_is_caught(monkeypatch):
    monkeypatch.setattr(Q, "asym_dequantize", lambda c, s, z: (c.astype(np.float32) * s).astype(np.float32))
    assert _fails(P.test_asym_codes_range_error_bound_and_brute_force)


def test_swapped_grouping_axis_is_caught(monkeypatch):
    orig = C.quantize_part

    def swapped(x, spec, fp8_scale=None):
        if spec.axis == C.PER_CHANNEL:
            spec = C.Spec(spec.scheme, spec.bits, C.PER_TOKEN, 0)
        elif spec.axis == C.PER_TOKEN:
            spec = C.Spec(spec.scheme, spec.bits, C.PER_CHANNEL, 0)
        return orig(x, spec, fp8_scale)

    monkeypatch.setattr(C, "quantize_part", swapped)
    assert _fails(P.test_int8_table_reproduces_printed_digits)
    assert _fails(P.test_int4_per_channel_beats_per_token)


def test_symmetric_scale_off_by_one_level_is_caught(monkeypatch):
    def sym128(x, axis, meta16=False):
        x = np.asarray(x, dtype=np.float32)
        a = np.abs(x).max(axis=axis, keepdims=True)
        s = (np.maximum(a, Q.EPS) / np.float32(128.0)).astype(np.float32)
        return np.clip(np.rint(x / s), -127, 127).astype(np.int8), s

    monkeypatch.setattr(Q, "sym_quantize", sym128)
    assert _fails(P.test_int8_table_reproduces_printed_digits)


def test_missing_fp8_saturation_is_caught(monkeypatch):
    orig = Q.e4m3_encode

    def nosat(y):
        y = np.asarray(y, dtype=np.float32)
        out = orig(y)
        return np.where(np.abs(y) > 464, np.uint8(0x7F) | (out & 0x80), out).astype(np.uint8)

    monkeypatch.setattr(Q, "e4m3_encode", nosat)
    assert _fails(P.test_e4m3_page_facts)


def test_fp8_ties_away_is_caught(monkeypatch):
    def away(y):
        y = np.asarray(y, dtype=np.float32)
        a = np.minimum(np.abs(y).astype(np.float64), 448.0)
        d = np.abs(Q._GRID_VALS[None, :] - a[:, None])
        best = d.min(axis=1, keepdims=True)
        idx = np.where(d == best, np.arange(d.shape[1])[None, :], -1).max(axis=1)  # larger on ties
        return (Q._GRID_CODES[idx] | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)

    monkeypatch.setattr(Q, "e4m3_encode", away)
    assert _fails(P.test_e4m3_encode_matches_library_cast_after_clamp)


def test_rope_sign_flip_is_caught(monkeypatch):
    orig = A.rope
    monkeypatch.setattr(A, "rope", lambda x, pos, base: orig(x, -np.asarray(pos), base))
    assert _fails(P.test_rope_closed_forms)


def test_rope_pairing_halves_is_caught(monkeypatch):
    def halves(x, positions, base):
        x = np.asarray(x, dtype=np.float64)
        D = x.shape[-1]
        th = np.power(float(base), -2.0 * np.arange(D // 2) / D)
        ang = np.asarray(positions, dtype=np.float64)[:, None] * th[None]
        c, s = np.cos(ang), np.sin(ang)
        a, b = x[..., :D // 2], x[..., D // 2:]
        return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)

    monkeypatch.setattr(A, "rope", halves)
    assert _fails(P.test_rope_closed_forms)


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    orig = A.decode_attention

    def interleaved(q, K, V, sm, pre_rope_base=None, heads=None):
        B, Hq, D = q.shape
        Hkv = K.shape[1]
        # query head h -> kv head h % Hkv instead of h // n_rep
        perm = np.array([(h % Hkv) * (Hq // Hkv) + h // Hkv for h in range(Hq)])
        out = orig(q[:, np.argsort(perm)], K, V, sm, pre_rope_base)
        return out[:, perm]

    monkeypatch.setattr(A, "decode_attention", interleaved)
    assert _fails(P.test_attention_matches_library_sdpa_fp64)


def test_transposed_attention_operand_is_caught(monkeypatch):
    def bad(q, K, V, sm):
        q = np.asarray(q, dtype=np.float64)
        K = np.asarray(K, dtype=np.float64)
        V = np.asarray(V, dtype=np.float64)
        lg = (K @ q) * sm
        p = np.exp(lg - lg.max())
        p /= p.sum()
        return (V.T[:, :len(p)] @ p) if V.shape[0] == V.shape[1] else p @ V[::-1], lg

    monkeypatch.setattr(A, "single_head", bad)
    assert _fails(P.test_attention_matches_library_sdpa_fp64)


@pytest.mark.parametrize("bug", ["window_off_by_one", "no_fp16_staging"])
def test_residual_bugs_are_caught(monkeypatch, bug):
    if bug == "window_off_by_one":
        orig = C.quantized_tokens
        monkeypatch.setattr(C, "quantized_tokens",
                            lambda cfg, T: (orig(cfg, T + 1) if not C.one_shot(cfg) else T))
        assert _fails(P.test_residual_split_properties, 32, 32)
    else:
        monkeypatch.setattr(C, "has_window", lambda cfg: False)
        assert _fails(P.test_window_holds_fp16_values)


def test_e5m2_missing_saturation_is_caught(monkeypatch):
    orig = Q.e5m2_encode

    def nosat(y):
        y = np.asarray(y, dtype=np.float32)
        c = orig(y)
        return np.where(np.abs(y) > 57344, c | 0x7C, c).astype(np.uint8)   # overflow to infinity
    monkeypatch.setattr(Q, "e5m2_encode", nosat)
    assert _fails(P.test_e5m2_page_facts)


def test_e5m2_wrong_bias_is_caught(monkeypatch):
    orig = Q.e5m2_value_of_code
    monkeypatch.setattr(Q, "e5m2_value_of_code", lambda c: orig(c) * 2.0)   # bias 14
    assert _fails(P.test_e5m2_grid_matches_library_decode)


def test_fp16_metadata_rounded_to_nearest_is_caught(monkeypatch):
    """Storing the fp16 zero-point / scale rounded to nearest (not toward the
    side that keeps the group covered) must fail the fp16-metadata pins."""
    from tests import test_meta16_oracle as M16
    monkeypatch.setattr(Q, "f16_toward", lambda x, up: np.asarray(x, np.float32).astype(np.float16).astype(np.float32))
    assert _fails(M16.test_directed_fp16_rounding_matches_brute_force)
    assert _fails(M16.test_asym_fp16_metadata_rule_and_bound, 2)


def test_fp16_metadata_codes_against_the_unrounded_range_are_caught(monkeypatch):
    """Codes taken against the fp32 minimum while the fp16 zero-point is
    stored must fail the reconstruction bound."""
    from tests import test_meta16_oracle as M16
    orig = Q.asym_quantize

    def mixed(x, bits, axis, meta16=False):
        c, s, z = orig(x, bits, axis, meta16)
        if meta16:
            x = np.asarray(x, np.float32)
            mn = x.min(axis=axis, keepdims=True)
            t = ((x - mn).astype(np.float32) / s).astype(np.float32)
            c = np.clip(np.rint(t), 0, 2 ** bits - 1).astype(np.uint8)
        return c, s, z
    monkeypatch.setattr(Q, "asym_quantize", mixed)
    assert _fails(M16.test_asym_fp16_metadata_rule_and_bound, 8)


# ---------------------------------------------------------------------------
# the parity checker itself: every GPU attention assertion goes through it
# ---------------------------------------------------------------------------

def _checker(reduce_fn):
    def mutated(out, ref, heads=None):
        B, Hq = ref.shape[0], ref.shape[1]
        todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
        return reduce_fn([A.rel_l2(out[b, h], ref[b, h]) for b, h in todo])
    return mutated


def _checker_nan_skipping(out, ref, heads=None):
    """The old form: Python's max() over the heads, whose comparisons skip a
    NaN that is not the first element, and rel_l2 without a finiteness check."""
    B, Hq = ref.shape[0], ref.shape[1]
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    return max(float(np.linalg.norm(out[b, h] - ref[b, h]) / np.linalg.norm(ref[b, h])) for b, h in todo)


def _checker_ignores_heads(out, ref, heads=None):
    return max(A.rel_l2(out[b, h], ref[b, h]) for b in range(ref.shape[0]) for h in range(ref.shape[1]))


@pytest.mark.parametrize("bug", ["min", "mean", "median", "first"])
def test_checker_wrong_reduction_is_caught(monkeypatch, bug):
    fn = {"min": min, "mean": lambda v: float(np.mean(v)), "median": lambda v: float(np.median(v)),
          "first": lambda v: v[0]}[bug]
    monkeypatch.setattr(A, "max_rel_l2_per_head", _checker(fn))
    assert _fails(P.test_max_rel_l2_per_head_hand_values)


def test_checker_skipping_nan_is_caught(monkeypatch):
    monkeypatch.setattr(A, "max_rel_l2_per_head", _checker_nan_skipping)
    assert _fails(P.test_max_rel_l2_per_head_non_finite_is_infinite, 0, 1)


def test_checker_ignoring_the_head_list_is_caught(monkeypatch):
    monkeypatch.setattr(A, "max_rel_l2_per_head", _checker_ignores_heads)
    assert _fails(P.test_max_rel_l2_per_head_hand_values)


def test_dequantize_part_bugs_are_caught(monkeypatch):
    """A zero-point dropped from the stored-code rebuild, or per-channel scales
    taken from the wrong group row, fail the hand-value pin."""
    orig = C.dequantize_part

    def no_zero(part, spec):
        if spec.scheme == C.INT_ASYM:
            part = dict(part, zero=np.zeros_like(part["zero"]))
        return orig(part, spec)

    monkeypatch.setattr(C, "dequantize_part", no_zero)
    assert _fails(P.test_dequantize_part_hand_values)

    def first_group_only(part, spec):
        if spec.scheme == C.INT_ASYM and spec.axis == C.PER_CHANNEL:
            s, z = part["scale"].copy(), part["zero"].copy()
            s[:, :, 1:] = s[:, :, :1]
            z[:, :, 1:] = z[:, :, :1]
            part = dict(part, scale=s, zero=z)
        return orig(part, spec)

    monkeypatch.setattr(C, "dequantize_part", first_group_only)
    assert _fails(P.test_dequantize_part_hand_values)


def test_window_slot_bugs_are_caught(monkeypatch):
    orig = C.ring_slots
    monkeypatch.setattr(C, "ring_slots", lambda cfg: max(orig(cfg) - 32, 0))
    assert _fails(P.test_window_slots_hand_values_and_no_collisions)
    monkeypatch.setattr(C, "ring_slots", orig)
    monkeypatch.setattr(C, "window_slots", lambda cfg, Tq, T: (np.arange(Tq, T) % max(orig(cfg), 1)) if
                        orig(cfg) == 0 else (np.arange(Tq, T) - Tq) % orig(cfg))
    assert _fails(P.test_window_slots_hand_values_and_no_collisions)


def test_gather_pages_bugs_are_caught(monkeypatch):
    """Pages taken in table order but from the wrong sequence's row, or the
    table read column-major, fail the hand-value pin."""
    import oracle.paged as OP
    orig = OP.gather_pages
    monkeypatch.setattr(OP, "gather_pages", lambda sec, bt, b, P, T: orig(sec, bt[::-1], b, P, T))
    assert _fails(P.test_gather_pages_hand_values)
    monkeypatch.setattr(OP, "gather_pages",
                        lambda sec, bt, b, P, T: np.concatenate([sec[int(bt.T.reshape(-1)[b * OP.blocks_of(T, P) + j])]
                                                                 for j in range(OP.blocks_of(T, P))], axis=1)
                        if OP.blocks_of(T, P) else orig(sec, bt, b, P, T))
    assert _fails(P.test_gather_pages_hand_values)
