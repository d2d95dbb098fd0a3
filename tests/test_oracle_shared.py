"""Pins of the split-context partial, the log-sum-exp merge and the grouped
(shared-prefix) decode evaluation, against what the mathematics fixes: the
merge of partials over any split of a row's keys is the attention over all of
them (closed forms for two keys, brute-force agreement with decode_ref at
every split point), and the grouped evaluation equals the plain definition
whenever the grouped sequences really share their prefix. Planted mistakes
in the oracle must fail one of them."""

import numpy as np
import pytest

import oracle
import oracle.paged_ref as pr
from oracle.numerics import to_f64
from oracle_helpers import lay_out


def _rows(rng, n, d):
    return rng.standard_normal((n, d)), rng.standard_normal((n, d))


def test_merge_of_two_single_key_partials_is_the_logistic_closed_form():
    # one key per partial: partial i = (v_i, s_i, 1); their merge is
    # (e^s0 v0 + e^s1 v1) / (e^s0 + e^s1) = sigma(s0 - s1) v0 + sigma(s1 - s0) v1
    v0, v1 = np.array([1.0, -2.0, 0.5]), np.array([-3.0, 4.0, 2.0])
    for s0, s1 in [(0.3, -1.2), (800.0, 799.0), (-5.0, 7.5)]:
        a = 1.0 / (1.0 + np.exp(s1 - s0))
        want = a * v0 + (1.0 - a) * v1
        got = pr.merge_partials_ref([(v0, s0, 1.0), (v1, s1, 1.0)])
        assert np.allclose(got, want, rtol=1e-14, atol=1e-14)


def test_partial_closed_form_and_empty_partials():
    q = np.array([1.0, 0.0])
    keys = np.array([[2.0, 0.0], [0.0, 1.0]])
    vals = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, m, l = pr.attention_partial_ref(q, keys, vals, 0.5)
    # scores 1 and 0: m = 1, l = 1 + e^-1, o = (v0 + e^-1 v1) / l
    assert m == 1.0 and np.isclose(l, 1.0 + np.exp(-1.0), rtol=1e-15)
    assert np.allclose(o, np.array([1.0, np.exp(-1.0)]) / l, rtol=1e-15)
    o_e, m_e, l_e = pr.attention_partial_ref(q, keys[:0], vals[:0], 0.5)
    assert m_e == -np.inf and l_e == 0.0 and np.all(o_e == 0)
    # empty partials contribute nothing; all empty gives zeros
    assert np.array_equal(pr.merge_partials_ref([(o, m, l), (o_e, m_e, l_e)]), o)
    assert np.array_equal(pr.merge_partials_ref([(o_e, m_e, l_e), (o_e, m_e, l_e)]),
                          np.zeros(2))


def test_merge_at_every_split_point_equals_decode():
    # a row's keys cut into two or three consecutive ranges at every position:
    # the merged partials equal decode_ref over the whole context
    rng = np.random.default_rng(3)
    n, d, bs = 37, 8, 4
    k, v = _rows(rng, n, d)
    q = rng.standard_normal(d)
    kc, vc, bt = lay_out([k.astype(np.float32)[:, None, :]], [v.astype(np.float32)[:, None, :]],
                         bs, rng)
    want = oracle.decode_ref(q.astype(np.float32)[None, None, :], kc, vc, bt, np.array([n]),
                             0.4)[0, 0]
    kk, vv = to_f64(k.astype(np.float32)), to_f64(v.astype(np.float32))
    qq = to_f64(q.astype(np.float32))
    for a in range(n + 1):
        got = pr.merge_partials_ref([pr.attention_partial_ref(qq, kk[:a], vv[:a], 0.4),
                                     pr.attention_partial_ref(qq, kk[a:], vv[a:], 0.4)])
        assert np.max(np.abs(got - want)) < 1e-13
    for a, b in [(5, 9), (0, 30), (12, 37), (36, 37)]:
        got = pr.merge_partials_ref([pr.attention_partial_ref(qq, kk[:a], vv[:a], 0.4),
                                     pr.attention_partial_ref(qq, kk[a:b], vv[a:b], 0.4),
                                     pr.attention_partial_ref(qq, kk[b:], vv[b:], 0.4)])
        assert np.max(np.abs(got - want)) < 1e-13


def _cow_case(rng, bs, prompt, tails, hkv=2, d=16, extra=()):
    """Sequences forked from one prompt (tables share its full blocks), plus
    `extra` unrelated lengths after them. Returns (q, kc, vc, bt, lens)."""
    pk = rng.standard_normal((prompt, hkv, d)).astype(np.float32)
    pv = rng.standard_normal((prompt, hkv, d)).astype(np.float32)
    ks, vs = [], []
    for t in tails:
        n = prompt + t  # t < 0: a member shorter than the prompt
        ks.append(np.concatenate([pk, rng.standard_normal((max(t, 0), hkv, d)).astype(np.float32)])[:n])
        vs.append(np.concatenate([pv, rng.standard_normal((max(t, 0), hkv, d)).astype(np.float32)])[:n])
    for n in extra:
        ks.append(rng.standard_normal((n, hkv, d)).astype(np.float32))
        vs.append(rng.standard_normal((n, hkv, d)).astype(np.float32))
    full = prompt // bs
    shared = [(i, 0, min(full, -(-ks[i].shape[0] // bs))) for i in range(1, len(tails))]
    kc, vc, bt = lay_out(ks, vs, bs, rng, shared=shared)
    lens = np.array([k.shape[0] for k in ks])
    q = rng.standard_normal((len(ks), 4 * hkv // 2, d)).astype(np.float32)
    return q, kc, vc, bt, lens


@pytest.mark.parametrize("bs", [4, 16])
@pytest.mark.parametrize("prefix", ["full_blocks", "mid_block", "zero", "whole_prompt_plus"])
def test_grouped_equals_plain_decode_when_the_prefix_is_shared(bs, prefix):
    rng = np.random.default_rng(bs + len(prefix))
    prompt = 3 * bs + (bs // 2)              # a partly filled last prompt block
    tails = [0, 5, 2 * bs + 1, -3, 1]        # -3: a member shorter than the prompt
    q, kc, vc, bt, lens = _cow_case(rng, bs, prompt, tails, extra=(9, 2 * bs))
    p = {"full_blocks": 3 * bs, "mid_block": prompt - 1, "zero": 0,
         "whole_prompt_plus": prompt}[prefix]
    # group 0: the five forks; the two unrelated sequences stay ungrouped
    cu = np.array([0, len(tails)])
    want = oracle.decode_ref(q, kc, vc, bt, lens, 0.3)
    got = oracle.decode_shared_prefix_ref(q, kc, vc, bt, lens, cu, np.array([p]), 0.3)
    assert np.max(np.abs(got - want)) < 1e-12
    # singleton groups, and groups that cover the unrelated sequences too
    cu2 = np.array([0, 2, 5, 6, 7])
    got2 = oracle.decode_shared_prefix_ref(q, kc, vc, bt, lens, cu2, np.array([p, p, 0, 0]), 0.3)
    assert np.max(np.abs(got2 - want)) < 1e-12


def test_grouped_reads_the_prefix_through_the_first_member():
    # member 1 is given its own, different prefix blocks: the grouped result
    # is the plain decode with member 1's prefix entries pointing at member 0's
    rng = np.random.default_rng(17)
    bs, hkv, d = 4, 1, 8
    ks = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in (14, 11)]
    vs = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in (14, 11)]
    kc, vc, bt = lay_out(ks, vs, bs, rng)
    q = rng.standard_normal((2, 2, d)).astype(np.float32)
    lens = np.array([14, 11])
    got = oracle.decode_shared_prefix_ref(q, kc, vc, bt, lens, np.array([0, 2]), np.array([8]),
                                          0.5)
    bt2 = bt.copy()
    bt2[1, :2] = bt[0, :2]
    want = oracle.decode_ref(q, kc, vc, bt2, lens, 0.5)
    assert np.max(np.abs(got - want)) < 1e-12
    assert np.max(np.abs(got[1] - oracle.decode_ref(q, kc, vc, bt, lens, 0.5)[1])) > 1e-3


# ---- sensitivity: plausible mistakes planted in the oracle must fail a pin ----------------

PINS = [
    test_merge_of_two_single_key_partials_is_the_logistic_closed_form,
    test_partial_closed_form_and_empty_partials,
    test_merge_at_every_split_point_equals_decode,
    lambda: test_grouped_equals_plain_decode_when_the_prefix_is_shared(4, "full_blocks"),
    lambda: test_grouped_equals_plain_decode_when_the_prefix_is_shared(16, "mid_block"),
    test_grouped_reads_the_prefix_through_the_first_member,
]


def _fails():
    for fn in PINS:
        try:
            with np.errstate(all="ignore"):
                fn()
        except (AssertionError, ValueError, IndexError, ZeroDivisionError, FloatingPointError):
            return True
    return False


def _merge_unweighted(partials):
    live = [(o, m, l) for o, m, l in partials if l > 0]
    if not live:
        return np.zeros_like(partials[0][0])
    big_m = max(m for _, m, _ in live)
    w = [np.exp(m - big_m) for _, m, _ in live]
    return sum(wi * o for wi, (o, _, _) in zip(w, live)) / sum(w)


def _merge_no_max(partials):
    live = [(o, m, l) for o, m, l in partials if l > 0]
    if not live:
        return np.zeros_like(partials[0][0])
    w = [l * np.exp(m) for _, m, l in live]
    return sum(wi * o for wi, (o, _, _) in zip(w, live)) / sum(w)


def _partial_no_normalise(query_row, keys, values, scale):
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1]), -np.inf, 0.0
    s = scale * (keys @ query_row)
    m = np.max(s)
    p = np.exp(s - m)
    return p @ values, m, float(np.sum(p))


def _grouped_variant(tail_skip=0, own_table=False):
    def grouped(query, key_cache, value_cache, block_tables, context_lens, cu_groups,
                prefix_lens, scale):
        q_all = to_f64(query)
        S, Hq, d = q_all.shape
        Hkv = key_cache.shape[1]
        G = Hq // Hkv
        out = np.zeros((S, Hq, d))
        cu = np.asarray(cu_groups)
        owner = {}
        for g in range(len(cu) - 1):
            for b in range(int(cu[g]), int(cu[g + 1])):
                owner[b] = (int(cu[g]), int(prefix_lens[g]))
        for b in range(S):
            n = int(context_lens[b])
            first, p_len = owner.get(b, (b, 0))
            if own_table:
                first = b
            sh = min(p_len, n)
            for kv in range(Hkv):
                kp = pr._gather_sequence(key_cache, block_tables[first], sh, kv)
                vp = pr._gather_sequence(value_cache, block_tables[first], sh, kv)
                ka = pr._gather_sequence(key_cache, block_tables[b], n, kv)
                va = pr._gather_sequence(value_cache, block_tables[b], n, kv)
                for h in range(kv * G, (kv + 1) * G):
                    parts = [pr.attention_partial_ref(q_all[b, h], kp, vp, scale),
                             pr.attention_partial_ref(q_all[b, h], ka[sh + tail_skip:],
                                                      va[sh + tail_skip:], scale)]
                    out[b, h] = pr.merge_partials_ref(parts)
        return out
    return grouped


@pytest.mark.parametrize("mutation", ["unweighted_merge", "merge_without_max", "unnormalised_partial",
                                      "tail_drops_a_token", "prefix_through_own_table"])
def test_planted_mistake_fails_a_pin(monkeypatch, mutation):
    if mutation == "unweighted_merge":
        monkeypatch.setattr(pr, "merge_partials_ref", _merge_unweighted)
    elif mutation == "merge_without_max":
        monkeypatch.setattr(pr, "merge_partials_ref", _merge_no_max)
    elif mutation == "unnormalised_partial":
        monkeypatch.setattr(pr, "attention_partial_ref", _partial_no_normalise)
    elif mutation == "tail_drops_a_token":
        monkeypatch.setattr(oracle, "decode_shared_prefix_ref", _grouped_variant(tail_skip=1))
    else:
        monkeypatch.setattr(oracle, "decode_shared_prefix_ref", _grouped_variant(own_table=True))
    assert _fails()
