"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a closed form,
an invariant of the mathematics, a hand-worked example, or the pure-Python brute
force on a dense key list.  Together they are chosen so that a plausible slip in
the oracle (a dropped rope term, the wrong 512 columns as V, a page/offset mix-up,
an off-by-one in the causal rule, a missing max shift, a wrong log base) fails at
least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from mla_inputs import (D_QK, D_V, PAGE, SCALE_192, bf16_bits_to_f32, f32_to_bf16_bits,
                        make_case)

HERE = os.path.dirname(os.path.abspath(__file__))


def _f32_case(B, T, H, lens, seed, causal=False, permute=True, scale=SCALE_192):
    return make_case(batch=B, q_len=T, num_heads=H, seqlens=lens, dtype="f32", causal=causal,
                     permute_pages=permute, seed=seed, scale=scale)


def _logical_keys(case, b):
    """Keys of sequence b in logical order, gathered with plain indexing (float64)."""
    L = int(case.cache_seqlens[b])
    out = []
    for p in range(L):
        page = case.block_table[b, p // PAGE]
        out.append(case.kv[page, p % PAGE].astype(np.float64))
    return out


def test_hand_worked_two_keys():
    g = json.load(open(os.path.join(HERE, "golden", "hand_two_keys.json")))
    q = np.array(g["q"], dtype=np.float32).reshape(1, 1, 1, 2)
    kv = np.array(g["keys"], dtype=np.float32).reshape(1, 2, 2)   # one page of 2 tokens
    bt = np.zeros((1, 1), dtype=np.int32)
    out, lse = oracle.decode(q, kv, bt, np.array([2], np.int32), scale=g["scale"], d_v=g["d_v"])
    # inputs are float32 roundings of ln 3; allow that rounding (2^-24 relative)
    assert abs(out[0, 0] - g["out"][0]) < 1e-7
    assert abs(lse[0] - g["lse"]) < 1e-7


def test_single_token_returns_its_value_row():
    case = _f32_case(2, 1, 4, [1, 1], seed=1)
    out, lse = oracle.decode_case(case)
    for b in range(2):
        k = case.kv[case.block_table[b, 0], 0].astype(np.float64)
        for h in range(4):
            r = b * 4 + h
            assert np.array_equal(out[r], k[:D_V])            # weight is exactly 1
            s = case.scale * float(np.dot(case.q[b, 0, h].astype(np.float64), k))
            assert abs(lse[r] - s) <= 1e-12 * max(1.0, abs(s))


def test_zero_query_gives_mean_of_values_and_log_n():
    case = _f32_case(2, 1, 3, [70, 129], seed=2)
    case.q[:] = 0.0
    out, lse = oracle.decode_case(case)
    for b in range(2):
        keys = np.array(_logical_keys(case, b))
        n = keys.shape[0]
        mean = keys[:, :D_V].mean(axis=0)
        for h in range(3):
            r = b * 3 + h
            np.testing.assert_allclose(out[r], mean, rtol=0, atol=1e-12)
            assert abs(lse[r] - math.log(n)) < 1e-12


def test_one_hot_query_picks_one_row_without_overflow():
    """q = 10 * k_j: s_j ~ 0.072*10*576 ~ 416 overflows exp() without a max shift; every
    other score is far below, so out = v_j and lse = s_j up to e^-40."""
    case = _f32_case(1, 1, 2, [200], seed=3)
    keys = _logical_keys(case, 0)
    j = 137
    case.q[0, 0, 0] = (10.0 * keys[j]).astype(np.float32)
    case.q[0, 0, 1] = (10.0 * keys[5]).astype(np.float32)
    out, lse = oracle.decode_case(case)
    for h, jj in ((0, j), (1, 5)):
        qv = case.q[0, 0, h].astype(np.float64)
        s = np.array([case.scale * float(np.dot(qv, k)) for k in keys])
        assert s[jj] > 300 and np.sort(s)[-2] < s[jj] - 40     # the premise of the pin
        assert np.all(np.isfinite(out[h]))
        np.testing.assert_allclose(out[h], keys[jj][:D_V], rtol=0, atol=1e-12)
        assert abs(lse[h] - s[jj]) < 1e-9


def test_page_permutation_invariance_is_bit_exact():
    case = _f32_case(3, 1, 4, [65, 200, 3], seed=4)
    out0, lse0 = oracle.decode_case(case)
    rng = np.random.default_rng(99)
    perm = rng.permutation(case.num_pages)          # new physical slot of each old page
    kv2 = np.empty_like(case.kv)
    kv2[perm] = case.kv
    bt2 = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    out1, lse1 = oracle.decode(case.q, kv2, bt2, case.cache_seqlens, scale=case.scale)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_rope_dims_only_enter_scores():
    case = _f32_case(2, 1, 4, [100, 64], seed=5)
    case.q[..., D_V:] = 0.0                            # q_rope = 0
    out0, lse0 = oracle.decode_case(case)
    case.kv[..., D_V:] = np.random.default_rng(7).standard_normal(case.kv[..., D_V:].shape)
    out1, lse1 = oracle.decode_case(case)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)
    # and with q_nope = 0 the rope dims alone decide the scores
    case.q[..., :D_V] = 0.0
    case.q[..., D_V:] = np.random.default_rng(8).standard_normal(case.q[..., D_V:].shape)
    out2, lse2 = oracle.decode_case(case)
    keys = _logical_keys(case, 0)
    qv = case.q[0, 0, 1].astype(np.float64)
    ref, ref_lse = brute.attend_row(list(qv), [list(k) for k in keys], case.scale, D_V)
    np.testing.assert_allclose(out2[1], ref, rtol=0, atol=1e-12)
    assert abs(lse2[1] - ref_lse) < 1e-12


def test_causal_first_query_equals_shorter_decode():
    """Query 0 of a q_len=2 causal step sees L-1 keys: it equals a q_len=1 decode
    of the same row over cache_seqlens - 1; query 1 equals a q_len=1 decode over L."""
    case = _f32_case(2, 2, 3, [65, 130], seed=6, causal=True)
    out, lse = oracle.decode_case(case)
    for t, delta in ((0, 1), (1, 0)):
        q1 = np.ascontiguousarray(case.q[:, t:t + 1])
        o1, l1 = oracle.decode(q1, case.kv, case.block_table, case.cache_seqlens - delta,
                               scale=case.scale)
        for b in range(2):
            for h in range(3):
                r2 = (b * 2 + t) * 3 + h
                r1 = b * 3 + h
                assert np.array_equal(out[r2], o1[r1]) and lse[r2] == l1[r1]


@pytest.mark.parametrize("causal,T", [(False, 1), (True, 2), (False, 2)])
def test_brute_force_tiny(causal, T):
    """Real 576/512 dims, lengths crossing a page boundary, permuted pages: the C oracle
    against the pure-Python fsum brute force on the dense logical key list."""
    lens = [70, 1] if T == 1 else [66, 2]
    case = _f32_case(2, T, 2, lens, seed=10 + T + int(causal), causal=causal)
    out, lse = oracle.decode_case(case)
    for b in range(2):
        keys = [list(k) for k in _logical_keys(case, b)]
        L = len(keys)
        for t in range(T):
            # the causal reading: query t sees positions p <= L - T + t
            n = L - T + 1 + t if causal else L
            for h in range(2):
                r = (b * T + t) * 2 + h
                ref, ref_lse = brute.attend_row(list(case.q[b, t, h].astype(np.float64)),
                                                keys[:max(n, 0)], case.scale, D_V)
                np.testing.assert_allclose(out[r], ref, rtol=0, atol=1e-12)
                assert abs(lse[r] - ref_lse) < 1e-12


def test_bf16_inputs_are_widened_exactly():
    case = make_case(batch=1, q_len=1, num_heads=2, seqlens=67, dtype="bf16", seed=12)
    out_b, lse_b = oracle.decode_case(case)
    # the float32 values of the same bits must give the identical float64 result
    out_f, lse_f = oracle.decode(case.q, case.kv, case.block_table, case.cache_seqlens,
                                 scale=case.scale, dtype="f32")
    assert np.array_equal(out_b, out_f) and np.array_equal(lse_b, lse_f)
    # round trip of the generator's bf16 rounding: ties go to even
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], dtype=np.float32)
    assert list(bf16_bits_to_f32(f32_to_bf16_bits(x))) == [1.0, 1.0 + 4 * 2 ** -8, -2.5, 0.0]


def test_batch_independence_and_row_subset():
    case = _f32_case(3, 1, 2, [90, 10, 64], seed=13)
    out, lse = oracle.decode_case(case)
    for b in range(3):
        o1, l1 = oracle.decode(case.q[b:b + 1], case.kv, case.block_table[b:b + 1],
                               case.cache_seqlens[b:b + 1], scale=case.scale)
        assert np.array_equal(out[b * 2:(b + 1) * 2], o1) and np.array_equal(lse[b * 2:(b + 1) * 2], l1)
    rows = np.array([5, 0, 3])
    o2, l2 = oracle.decode_case(case, rows=rows)
    assert np.array_equal(o2, out[rows]) and np.array_equal(l2, lse[rows])


def test_empty_rows_give_zero_and_minus_inf():
    case = _f32_case(2, 2, 2, [1, 0], seed=14, causal=True)
    out, lse = oracle.decode_case(case)
    # b=0: L=1, T=2 -> query 0 sees 0 keys, query 1 sees 1 key; b=1: no keys at all
    for r in (0, 1, 4, 5, 6, 7):
        assert np.all(out[r] == 0.0) and lse[r] == -np.inf
    for r in (2, 3):
        assert np.isfinite(lse[r])


def test_split_keys_then_combine_equals_whole():
    """decode over [0, L) == combine(decode over [0, 64k), decode over [64k, L)).
    The second part is expressed as its own sequence whose block table starts at
    block k, so both parts go through the paged oracle."""
    case = _f32_case(1, 1, 4, [300], seed=15)
    whole, whole_lse = oracle.decode_case(case)
    parts_o, parts_l = [], []
    bounds = [0, 64, 192, 300]
    for a, e in zip(bounds[:-1], bounds[1:]):
        bt = np.ascontiguousarray(case.block_table[:, a // PAGE:])
        q = case.q
        # keys [a, e) = the first (e - a) tokens of the shifted table
        o, l = oracle.decode(q, case.kv, bt, np.array([e - a], np.int32), scale=case.scale)
        parts_o.append(o)
        parts_l.append(l)
    out, lse = oracle.combine(np.stack(parts_o), np.stack(parts_l))
    np.testing.assert_allclose(out, whole, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, whole_lse, rtol=0, atol=1e-13)
    # equal-LSE closed form: two identical parts average to themselves, lse + ln 2
    o2, l2 = oracle.combine(np.stack([whole, whole]), np.stack([whole_lse, whole_lse]))
    np.testing.assert_allclose(o2, whole, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l2, whole_lse + math.log(2.0), rtol=0, atol=1e-13)
    # an empty part (-inf) has weight 0; all-empty gives zeros and -inf
    o3, l3 = oracle.combine(np.stack([whole, np.full_like(whole, 7.0)]),
                            np.stack([whole_lse, np.full_like(whole_lse, -np.inf)]))
    assert np.array_equal(o3, whole) and np.array_equal(l3, whole_lse)
    o4, l4 = oracle.combine(np.zeros((2, 1, 3)), np.full((2, 1), -np.inf))
    assert np.all(o4 == 0) and l4[0] == -np.inf


def test_generator_sanity_mean_lse():
    """Not a gate on the oracle's arithmetic: with N(0,1) data, scores have variance
    576/192 = 3, so E[exp(s)] = e^1.5 and the mean lse is about ln L + 1.5."""
    case = make_case(batch=1, q_len=1, num_heads=16, seqlens=256, dtype="f32",
                     permute_pages=False, seed=1000)
    _, lse = oracle.decode_case(case)
    assert abs(lse.mean() - (math.log(256) + 1.5)) < 0.35


def test_bad_page_is_reported():
    case = _f32_case(1, 1, 1, [70], seed=16)
    case.block_table[0, 1] = case.num_pages + 5
    with pytest.raises(RuntimeError):
        oracle.decode_case(case)


# ---- attention sinks: one more softmax term per head, with a zero value row -------------

def test_sink_hand_worked_two_keys():
    g = json.load(open(os.path.join(HERE, "golden", "hand_two_keys_sink.json")))
    q = np.array(g["q"], dtype=np.float32).reshape(1, 1, 1, 2)
    kv = np.array(g["keys"], dtype=np.float32).reshape(1, 2, 2)
    bt = np.zeros((1, 1), dtype=np.int32)
    out, lse = oracle.decode(q, kv, bt, np.array([2], np.int32), scale=g["scale"], d_v=g["d_v"],
                             sinks=[g["sink"]])
    assert abs(out[0, 0] - g["out"][0]) < 1e-7
    assert abs(lse[0] - g["lse"]) < 1e-7


@pytest.mark.parametrize("causal,T", [(False, 1), (True, 2)])
def test_sink_brute_force_tiny(causal, T):
    """The C oracle with sinks against the pure-Python brute force (the sink appended to
    the score list), real dims, a page crossing, permuted pages, an empty causal row."""
    lens = [70, 1] if T == 1 else [66, 1]
    H = 3
    case = _f32_case(2, T, H, lens, seed=80 + T, causal=causal)
    sinks = np.array([0.75, -2.0, 40.0])          # the last one outweighs every key
    out, lse = oracle.decode_case(case, sinks=sinks)
    for b in range(2):
        keys = [list(k) for k in _logical_keys(case, b)]
        L = len(keys)
        for t in range(T):
            n = L - T + 1 + t if causal else L
            for h in range(H):
                r = (b * T + t) * H + h
                ref, ref_lse = brute.attend_row(list(case.q[b, t, h].astype(np.float64)),
                                                keys[:max(n, 0)], case.scale, D_V, sink=float(sinks[h]))
                np.testing.assert_allclose(out[r], ref, rtol=0, atol=1e-12)
                assert abs(lse[r] - ref_lse) < 1e-12 * max(1.0, abs(ref_lse))


def test_sink_rescales_the_plain_result():
    """Identity of the reading: adding a term e^sigma to the denominator scales every
    weight by Z / (Z + e^sigma) with Z = e^lse, so out_sink = out / (1 + e^(sigma - lse))
    and lse_sink = ln(e^lse + e^sigma).  A sink that leaked into the values, or that was
    left out of lse, fails this."""
    case = _f32_case(2, 2, 4, [130, 9], seed=82, causal=True)
    plain_o, plain_l = oracle.decode_case(case)
    sinks = np.array([-1.0, 0.5, 3.0, 12.0])
    o, l = oracle.decode_case(case, sinks=sinks)
    h = np.arange(plain_l.size) % 4
    sig = sinks[h]
    np.testing.assert_allclose(l, np.logaddexp(plain_l, sig), rtol=1e-14, atol=1e-14)
    factor = 1.0 / (1.0 + np.exp(sig - plain_l))
    np.testing.assert_allclose(o, plain_o * factor[:, None], rtol=1e-12, atol=1e-15)


def test_sink_minus_inf_is_the_plain_decode_and_empty_rows_take_the_sink():
    case = _f32_case(2, 2, 2, [1, 40], seed=83, causal=True)
    o0, l0 = oracle.decode_case(case)
    o1, l1 = oracle.decode_case(case, sinks=[-np.inf, -np.inf])
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    o2, l2 = oracle.decode_case(case, sinks=[1.5, -3.0])
    # b=0, t=0 sees no key: out 0, lse = its head's sink
    assert np.all(o2[0] == 0.0) and l2[0] == 1.5
    assert np.all(o2[1] == 0.0) and l2[1] == -3.0


# ---- sparse (top-k) decode: each (b, t) attends to exactly its listed tokens ------------

def _sparse_case(B, T, H, lens, seed):
    return _f32_case(B, T, H, lens, seed=seed)


def test_sparse_full_list_is_the_dense_decode():
    """Listing every position 0 .. L-1 in order (unused entries -1) gathers the same keys
    in the same order as the dense decode: bit-identical."""
    case = _sparse_case(3, 2, 2, [70, 5, 128], seed=90)
    topk = 130
    idx = np.full((3, 2, topk), -1, np.int32)
    for b, L in enumerate(case.cache_seqlens):
        idx[b, :, :L] = np.arange(L)
    o0, l0 = oracle.decode_case(case)
    o1, l1 = oracle.decode_case(case, indices=idx)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_sparse_brute_force_tiny():
    """Random lists with unused entries and repeats, against the brute force over the
    listed keys gathered by plain indexing."""
    from mla_inputs import make_topk_indices
    case = _sparse_case(2, 2, 2, [150, 40], seed=91)
    idx = make_topk_indices(case.cache_seqlens, 2, 70, seed=5, pad_frac=0.2, dup_frac=0.1)
    out, lse = oracle.decode_case(case, indices=idx)
    for b in range(2):
        keys = _logical_keys(case, b)
        for t in range(2):
            sel = [list(keys[p]) for p in idx[b, t] if p != -1]
            for h in range(2):
                r = (b * 2 + t) * 2 + h
                ref, ref_lse = brute.attend_row(list(case.q[b, t, h].astype(np.float64)), sel, case.scale, D_V)
                np.testing.assert_allclose(out[r], ref, rtol=0, atol=1e-12)
                assert abs(lse[r] - ref_lse) < 1e-12


def test_sparse_unused_entries_order_and_repeats():
    case = _sparse_case(1, 1, 3, [200], seed=92)
    rng = np.random.default_rng(3)
    base = rng.choice(200, size=50, replace=False).astype(np.int32)
    o0, l0 = oracle.decode_case(case, indices=base.reshape(1, 1, -1))
    # -1 entries anywhere change nothing, bit for bit
    padded = np.insert(base, [0, 10, 10, 50], -1).reshape(1, 1, -1)
    o1, l1 = oracle.decode_case(case, indices=padded)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # the list is a set of keys up to rounding order
    o2, l2 = oracle.decode_case(case, indices=rng.permutation(base).reshape(1, 1, -1))
    np.testing.assert_allclose(o2, o0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l0, rtol=0, atol=1e-13)
    # listing every entry twice doubles every weight: same output, lse + ln 2
    o3, l3 = oracle.decode_case(case, indices=np.concatenate([base, base]).reshape(1, 1, -1))
    np.testing.assert_allclose(o3, o0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l3, l0 + math.log(2.0), rtol=0, atol=1e-13)
    # an all-unused list is an empty row
    o4, l4 = oracle.decode_case(case, indices=np.full((1, 1, 8), -1, np.int32))
    assert np.all(o4 == 0.0) and np.all(l4 == -np.inf)


def test_sparse_bad_entries_are_reported():
    case = _sparse_case(2, 1, 1, [10, 64], seed=93)
    for bad in (10, 64 + 5, -2):
        idx = np.array([[[0, 1, 2]], [[3, 4, 5]]], np.int32)
        idx[0, 0, 1] = bad                     # sequence 0 holds 10 tokens
        with pytest.raises(RuntimeError, match="code 2"):
            oracle.decode_case(case, indices=idx)
    with pytest.raises(RuntimeError, match="code 1"):   # sparse lists replace the causal rule
        c2 = _f32_case(1, 2, 1, [10], seed=94, causal=True)
        oracle.decode_case(c2, indices=np.zeros((1, 2, 2), np.int32))


def test_sink_far_above_every_score_keeps_the_max_shift():
    """A sink 800 above the scores: the softmax is all sink.  Without the sink in the
    max shift, exp(800 - max score) overflows float64 and lse comes out infinite."""
    case = _f32_case(1, 1, 2, [70], seed=84)
    o, l = oracle.decode_case(case, sinks=[800.0, -800.0])
    plain_o, plain_l = oracle.decode_case(case)
    assert abs(l[0] - 800.0) < 1e-12 and np.all(np.abs(o[0]) < 1e-300)
    # a sink far below changes nothing measurable
    np.testing.assert_allclose(o[1], plain_o[1], rtol=1e-15, atol=0)
    assert l[1] == plain_l[1]
