"""Pins of the float64 oracle against facts that do not come from the oracle itself.

Each test names the passage or the mathematical fact it pins. Together they are
chosen so that a plausible slip in the oracle (a dropped max subtraction, a
wrong causal offset, a transposed operand, a missing normalisation, a sign
error in the log-sum-exp, a missing scale) fails at least one of them; the
mutation test in test_oracle_mutants.py checks exactly that.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import tiled_model as tm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _num(x):
    return math.log(2.0) if x == "ln2" else float(x)


def _golden():
    with open(GOLDEN) as f:
        return {e["id"]: e for e in json.load(f)["examples"]}


def _d1(scores, values, scale=1.0):
    """d=1 construction: q=[1], k_j=[s_j], v_j=[value_j] gives scores s_j*scale."""
    q = np.ones((1, 1, 1, 1), np.float32)
    k = np.asarray(scores, np.float32).reshape(1, 1, -1, 1)
    v = np.asarray(values, np.float32).reshape(1, 1, -1, 1)
    return q, k, v, scale


def _rand(shape, rng, mult=1.0):
    return (rng.standard_normal(shape) * mult).astype(np.float32)


def _heads(q, k, v):
    return [(q[b, h].astype(np.float64), k[b, h].astype(np.float64), v[b, h].astype(np.float64))
            for b in range(q.shape[0]) for h in range(q.shape[1])]


# ---------------------------------------------------------------- worked examples

def test_worked_example_block_of_two():
    """Flash Attention Optimization: 'Worked example: online softmax by hand' and the
    printed output of 'Tracing the algorithm as code'."""
    ex = _golden()["fa_optimization_worked_example"]
    q, k, v, sc = _d1(ex["scores"], ex["values"])
    o, lse, p = oracle.attention(q, k, v, sc, want_p=True)
    val, tol = ex["O_program_output"]
    assert abs(o[0, 0] - val) <= tol
    val, tol = ex["direct"]["O"]
    assert abs(o[0, 0] - val) <= tol
    w, tol = ex["direct"]["weights"]
    assert np.max(np.abs(p[0] - np.array(w))) <= tol
    # log-sum-exp is m + ln(sum exp(s - m)) with the printed sum 1.20345 and m = 5
    val, tol = ex["direct"]["exp_sum"]
    assert abs(lse[0] - (5.0 + math.log(val))) <= tol / (val - tol)


def test_worked_example_block_states():
    """The per-block running states printed in the same worked example, reproduced by the
    tiled model (which the oracle is then compared with below)."""
    g = _golden()
    for key in ("fa_optimization_worked_example", "fa_optimization_active_recall_1"):
        ex = g[key]
        s = np.array(ex["scores"], np.float64)
        vals = np.array(ex["values"], np.float64)[:, None]
        B = ex["block_size"]
        st = tm.empty(1, 1)
        for bi, blk in enumerate(ex["blocks"]):
            lo, hi = bi * B, (bi + 1) * B
            loc = tm.of_keys(s[None, lo:hi], vals[lo:hi])
            if "local_l" in blk:
                for name, got in (("local_m", loc.m[0]), ("local_l", loc.l[0]),
                                  ("local_acc", loc.o[0, 0])):
                    val, tol = blk[name]
                    assert abs(got - val) <= tol + 1e-12, (key, name, got, val)
                _, f_old, f_new = tm.factors(st, loc)
                for name, got in (("scale_old", f_old[0]), ("scale_new", f_new[0])):
                    val, tol = blk[name]
                    assert abs(got - val) <= tol + 1e-12, (key, name, got, val)
            st = tm.combine(st, loc)
            for name, got in (("m", st.m[0]), ("l", st.l[0]), ("acc", st.o[0, 0])):
                if name not in blk:
                    continue
                val, tol = blk[name]
                assert abs(got - val) <= tol + 1e-12, (key, name, got, val)
        q, k, v, sc = _d1(ex["scores"], ex["values"])
        o, _ = oracle.attention(q, k, v, sc)
        if "O" in ex:
            val, tol = ex["O"]
            assert abs(o[0, 0] - val) <= tol
        assert abs(o[0, 0] - tm.finish(st)[0][0]) <= 1e-12


def test_worked_example_two_tiles_interview():
    """Explain FlashAttention ...: 'Keep only the state needed ...' (scores 0 and ln 2 over
    values 10 and 20 give 16 2/3). The score ln 2 is carried by the float64 scale, k=[0,1]."""
    ex = _golden()["io_aware_interview_two_tiles"]
    q = np.ones((1, 1, 1, 1), np.float32)
    k = np.array([0.0, 1.0], np.float32).reshape(1, 1, 2, 1)
    v = np.array(ex["values"], np.float32).reshape(1, 1, 2, 1)
    o, lse = oracle.attention(q, k, v, math.log(2.0))
    val, tol = ex["O"]
    assert abs(o[0, 0] - val) <= tol
    assert abs(o[0, 0] - 50.0 / 3.0) <= 1e-13
    assert abs(lse[0] - math.log(3.0)) <= 1e-15   # closed form: ln(e^0 + e^ln2) = ln 3
    # block states of the example, tile size 1
    s = np.array([_num(x) for x in ex["scores"]])
    vals = np.array(ex["values"])[:, None]
    st = tm.empty(1, 1)
    for bi, blk in enumerate(ex["blocks"]):
        loc = tm.of_keys(s[None, bi:bi + 1], vals[bi:bi + 1])
        _, alpha, _ = tm.factors(st, loc)
        st = tm.combine(st, loc)
        for name, got in (("m", st.m[0]), ("l", st.l[0]), ("o", st.o[0, 0])):
            val, tol = blk[name]
            assert abs(got - _num(val)) <= tol + 1e-15, (name, got, val)
        if "alpha" in blk:
            val, tol = blk["alpha"]
            assert abs(alpha[0] - val) <= tol


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True, 2])
@pytest.mark.parametrize("nq,nk", [(7, 7), (5, 9), (9, 5), (1, 33)])
def test_uniform_scores_give_mean_of_visible_values(causal, nq, nk):
    """q = 0 makes every visible score 0, so softmax is uniform over visible keys: O is the
    mean of the visible value rows and LSE = ln(count). With causal masking query i sees
    keys 0..i+(Nk-Nq) (bottom-right, causal = 1) or 0..i (top-left, causal = 2), which pins
    the absolute-position offset of each alignment."""
    rng = np.random.default_rng(3)
    d = 6
    q = np.zeros((2, 3, nq, d), np.float32)
    k = _rand((2, 3, nk, d), rng)
    v = _rand((2, 3, nk, d), rng)
    o, lse = oracle.attention(q, k, v, 0.37, causal)
    o = o.reshape(2, 3, nq, d)
    lse = lse.reshape(2, 3, nq)
    for b in range(2):
        for h in range(3):
            for i in range(nq):
                n = nk
                if causal == 2:
                    n = min(nk, i + 1)
                elif causal:
                    n = min(nk, i + (nk - nq) + 1)
                if n <= 0:
                    assert np.all(o[b, h, i] == 0.0) and lse[b, h, i] == -math.inf
                    continue
                want = v[b, h, :n].astype(np.float64).mean(axis=0)
                assert np.max(np.abs(o[b, h, i] - want)) <= 1e-14
                assert abs(lse[b, h, i] - math.log(n)) <= 1e-14


def test_rows_of_p_sum_to_one_and_are_nonnegative():
    rng = np.random.default_rng(4)
    q, k, v = _rand((2, 2, 9, 5), rng, 2.0), _rand((2, 2, 13, 5), rng, 2.0), _rand((2, 2, 13, 5), rng)
    for causal in (False, True):
        _, _, p = oracle.attention(q, k, v, 0.5, causal, want_p=True)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-15 * 16


def test_key_permutation_invariance():
    """Non-causal attention is a sum over keys: permuting K and V rows jointly only changes
    the summation order ('Correcting a common misconception': rounding only)."""
    rng = np.random.default_rng(5)
    q, k, v = _rand((1, 2, 11, 8), rng), _rand((1, 2, 40, 8), rng), _rand((1, 2, 40, 8), rng)
    perm = rng.permutation(40)
    o1, l1 = oracle.attention(q, k, v, 0.3)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.3)
    assert np.max(np.abs(o1 - o2)) <= 1e-13
    assert np.max(np.abs(l1 - l2)) <= 1e-13


@pytest.mark.parametrize("c", [0.75, 1e4, -1e4])
def test_common_shift_cancels_and_guards_overflow(c):
    """Adding one constant c to every score of a row leaves O unchanged and adds c to LSE
    (the local max cancels: 'Handwritten Notes on Flash Attention', 'Merging two blocks').
    With c = 1e4 an implementation without max subtraction overflows exp."""
    rng = np.random.default_rng(6)
    d = 8
    scale = 0.125
    q, k, v = _rand((1, 2, 6, d), rng), _rand((1, 2, 10, d), rng), _rand((1, 2, 10, d), rng)
    q2 = np.concatenate([q, np.ones((1, 2, 6, 1), np.float32)], axis=3)
    extra = np.full((1, 2, 10, 1), c / scale, np.float32)
    assert float(extra[0, 0, 0, 0]) * scale == c          # exactly representable
    k2 = np.concatenate([k, extra], axis=3)
    v2 = np.concatenate([v, np.zeros((1, 2, 10, 1), np.float32)], axis=3)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, scale, causal)
        o2, l2 = oracle.attention(q2, k2, v2, scale, causal)
        assert np.all(np.isfinite(o2))
        assert np.max(np.abs(o1 - o2[:, :d])) <= 1e-11
        assert np.max(np.abs((l1 + c) - l2)) <= 1e-11


def test_special_cases():
    """Nk = 1: the only key gets weight 1. Causal row 0 (Nq = Nk): sees only key 0.
    Causal Nq > Nk: the first Nq - Nk rows see nothing and follow the empty-row policy
    ('Explain FlashAttention ...', 'Executable recurrence, with an empty-state policy')."""
    rng = np.random.default_rng(7)
    d = 5
    q, k, v = _rand((2, 2, 4, d), rng), _rand((2, 2, 1, d), rng), _rand((2, 2, 1, d), rng)
    o, lse = oracle.attention(q, k, v, 0.7)
    o = o.reshape(2, 2, 4, d)
    lse = lse.reshape(2, 2, 4)
    for b in range(2):
        for h in range(2):
            for i in range(4):
                assert np.array_equal(o[b, h, i], v[b, h, 0].astype(np.float64))
                s0 = 0.7 * sum(float(q[b, h, i, t]) * float(k[b, h, 0, t]) for t in range(d))
                assert abs(lse[b, h, i] - s0) <= 1e-14
    q, k, v = _rand((1, 2, 12, d), rng), _rand((1, 2, 12, d), rng), _rand((1, 2, 12, d), rng)
    o, lse = oracle.attention(q, k, v, 0.7, causal=True)
    o = o.reshape(1, 2, 12, d)
    for h in range(2):
        assert np.array_equal(o[0, h, 0], v[0, h, 0].astype(np.float64))
    q, k, v = _rand((1, 1, 10, d), rng), _rand((1, 1, 4, d), rng), _rand((1, 1, 4, d), rng)
    o, lse = oracle.attention(q, k, v, 0.7, causal=True)
    assert np.all(o[:6] == 0.0) and np.all(lse[:6] == -math.inf)
    assert np.all(np.isfinite(lse[6:]))
    assert np.array_equal(o[6], v[0, 0, 0].astype(np.float64))   # row 6 sits at position 0


# ---------------------------------------------------------------- brute force, library

def _brute_row(qi, kk, vv, scale, last):
    """Direct softmax of one row with no max subtraction (scores kept small), math.fsum."""
    w = [math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(qi, kk[j])))
         for j in range(last + 1)]
    if not w:
        return [0.0] * len(vv[0]), -math.inf
    tot = math.fsum(w)
    out = [math.fsum(w[j] * float(vv[j][t]) for j in range(len(w))) / tot for t in range(len(vv[0]))]
    return out, math.log(tot)


@pytest.mark.parametrize("causal", [False, True, 2])
@pytest.mark.parametrize("nq,nk,d", [(5, 5, 3), (3, 11, 8), (13, 4, 2), (16, 16, 7), (1, 9, 4)])
def test_brute_force_tiny(causal, nq, nk, d):
    rng = np.random.default_rng(100 + nq * 7 + nk + d)
    B, H = 2, 2
    q, k, v = _rand((B, H, nq, d), rng), _rand((B, H, nk, d), rng), _rand((B, H, nk, d), rng)
    scale = 0.61
    o, lse = oracle.attention(q, k, v, scale, causal)
    o = o.reshape(B, H, nq, d)
    lse = lse.reshape(B, H, nq)
    for b in range(B):
        for h in range(H):
            for i in range(nq):
                last = nk - 1
                if causal == 2:
                    last = min(nk - 1, i)
                elif causal:
                    last = min(nk - 1, i + nk - nq)
                want, wl = _brute_row(q[b, h, i], k[b, h], v[b, h], scale, last)
                assert np.max(np.abs(o[b, h, i] - np.array(want))) <= 1e-13
                if wl == -math.inf:
                    assert lse[b, h, i] == -math.inf
                else:
                    assert abs(lse[b, h, i] - wl) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_torch_sdpa_float64(causal):
    """PyTorch's scaled_dot_product_attention in float64 on the CPU; the page's 'Try it'
    section compares a tiled loop with this routine and reports ~6e-16."""
    rng = np.random.default_rng(8)
    q, k, v = _rand((2, 3, 70, 16), rng), _rand((2, 3, 70, 16), rng), _rand((2, 3, 70, 16), rng)
    scale = 0.25
    o, lse = oracle.attention(q, k, v, scale, causal)
    t = [torch.from_numpy(x).double() for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=scale)
    assert np.max(np.abs(o - ref.reshape(-1, 16).numpy())) <= 1e-13
    # log-sum-exp via torch.logsumexp of the materialised scores
    s = (t[0] @ t[1].transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(torch.ones(70, 70, dtype=torch.bool).triu(1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, -1).reshape(-1).numpy())) <= 1e-13


def test_sdpa_example_size_from_try_it():
    """The 'Try it' workload itself: one head, n=1000, d=64, scale 1/sqrt(d), non-causal."""
    rng = np.random.default_rng(0)
    q, k, v = (_rand((1, 1, 1000, 64), rng) for _ in range(3))
    o, _ = oracle.attention(q, k, v, 0.125)
    t = [torch.from_numpy(x).double() for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t)
    assert np.max(np.abs(o - ref.reshape(-1, 64).numpy())) <= 1e-14


# ---------------------------------------------------------------- tiled model agreement

@pytest.mark.parametrize("tile", [1, 2, 3, 7, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_recurrence_matches_definition(tile, causal):
    rng = np.random.default_rng(9 + tile)
    nq, nk, d = 37, 150, 8
    q, k, v = _rand((1, 2, nq, d), rng, 3.0), _rand((1, 2, nk, d), rng, 3.0), _rand((1, 2, nk, d), rng)
    o, lse = oracle.attention(q, k, v, 0.35, causal)
    o = o.reshape(2, nq, d)
    lse = lse.reshape(2, nq)
    for h, (qh, kh, vh) in enumerate(_heads(q, k, v)):
        to, tl = tm.tiled_head(qh, kh, vh, 0.35, causal, tile)
        assert np.max(np.abs(to - o[h])) <= 1e-13
        assert np.max(np.abs(tl - lse[h])) <= 1e-13


def test_prefix_property():
    """After j tiles the finished running state equals attention over the first j*T keys
    ('Handwritten Notes on Flash Attention', 'Green + yellow': correct after every step)."""
    rng = np.random.default_rng(10)
    d, nk, T = 6, 50, 8
    q, k, v = _rand((1, 1, 3, d), rng), _rand((1, 1, nk, d), rng), _rand((1, 1, nk, d), rng)
    qh, kh, vh = _heads(q, k, v)[0]
    s = tm.scores(qh, kh, 0.4, False)
    st = tm.empty(3, d)
    for lo, hi in tm.bounds(nk, T):
        st = tm.combine(st, tm.of_keys(s[:, lo:hi], vh[lo:hi]))
        o, lse = oracle.attention(q, k[:, :, :hi], v[:, :, :hi], 0.4)
        fo, fl = tm.finish(st)
        assert np.max(np.abs(fo - o)) <= 1e-13 and np.max(np.abs(fl - lse)) <= 1e-13


@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_split_and_merge_matches_definition(splits):
    """Split the keys into chunks of ceil(Nk/S) (trailing chunks short or empty), keep a
    state per chunk relative to its own max, merge with the two-sided rule."""
    rng = np.random.default_rng(11 + splits)
    nk, d = 100, 8
    q, k, v = _rand((1, 2, 3, d), rng, 2.0), _rand((1, 2, nk, d), rng, 2.0), _rand((1, 2, nk, d), rng)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.3, causal)
        o = o.reshape(2, 3, d)
        lse = lse.reshape(2, 3)
        for h, (qh, kh, vh) in enumerate(_heads(q, k, v)):
            so, sl = tm.split_merge_head(qh, kh, vh, 0.3, causal, splits)
            assert np.max(np.abs(so - o[h])) <= 1e-13
            assert np.max(np.abs(sl - lse[h])) <= 1e-13


def test_bf16_inputs_are_widened_exactly():
    """bfloat16 inputs are read as their exact values (the bytes the GPU receives)."""
    rng = np.random.default_rng(12)
    q, k, v = (torch.from_numpy(_rand((1, 2, 9, 16), rng)).bfloat16() for _ in range(3))
    o1, l1 = oracle.attention(q, k, v, 0.25, True)
    o2, l2 = oracle.attention(q.float(), k.float(), v.float(), 0.25, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_row_subset_matches_full():
    rng = np.random.default_rng(13)
    q, k, v = _rand((2, 3, 20, 8), rng), _rand((2, 3, 25, 8), rng), _rand((2, 3, 25, 8), rng)
    o, lse = oracle.attention(q, k, v, 0.3, True)
    rows = [0, 5, 19, 20, 77, 119]
    os_, ls_ = oracle.attention(q, k, v, 0.3, True, rows=rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls_, lse[rows])


def test_rejects_bad_arguments():
    q = np.zeros((1, 1, 2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.attention(q, np.zeros((1, 1, 3, 5), np.float32), np.zeros((1, 1, 3, 5), np.float32), 1.0)
    with pytest.raises(ValueError):
        oracle.attention(q, q, q, 1.0, rows=[2])
    with pytest.raises(TypeError):
        oracle.attention(q.astype(np.float64), q, q, 1.0)
