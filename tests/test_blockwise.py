"""The pages' online-softmax recurrence (fp64 models) reaches the oracle's result.

Runs on the CPU. The recurrence is the method; the oracle is the definition. On the
same inputs they must agree to fp64 rounding (1e-12), for the tile shapes and the
ragged, causal and wide-logit cases the workloads use.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import blockwise
import pins
from workloads import WORKLOADS, make_qkv


def _f64(t):
    return t.double().numpy()


def test_online_softmax_matches_two_block_example():
    exp_scores, l1, l2, rows = pins.load_two_block_golden()
    x = np.log(np.array(exp_scores, dtype=np.float64))
    for bs in (1, 2, 3, 4):
        p = blockwise.online_softmax(x, bs)
        np.testing.assert_allclose(p, [0.1, 0.2, 0.3, 0.4], rtol=0, atol=1e-15)


@pytest.mark.parametrize("bs", [1, 2, 3, 5, 64])
def test_online_softmax_matches_oracle_row(bs):
    r = np.random.default_rng(3)
    n = 23
    Q = r.normal(size=(n, n)) * 3.0
    K = r.normal(size=(n, n))
    P, _ = oracle.attention(Q, K, np.eye(n), False, 1.0)  # V = I: output rows are P
    S = Q @ K.T
    for i in (0, 11, 22):
        np.testing.assert_allclose(blockwise.online_softmax(S[i], bs), P[i], rtol=0, atol=1e-14)


@pytest.mark.parametrize("bs", [1, 4, 7, 32])
def test_one_query_attention_matches_oracle(bs):
    r = np.random.default_rng(4)
    n, d, scale = 40, 8, 1 / math.sqrt(8)
    Q, K, V = r.normal(size=(n, d)), r.normal(size=(n, d)), r.normal(size=(n, d))
    O, L = oracle.attention(Q, K, V, False, scale)
    for i in (0, 19, 39):
        o, lse = blockwise.one_query_attention(Q[i], K, V, bs, scale)
        np.testing.assert_allclose(o, O[i], rtol=0, atol=1e-13)
        assert abs(lse - L[i]) < 1e-13


def test_tiled_16x16_on_single_head_workload():
    """The 16 x 16 tiling of the single-head fp32 workload (N = 128, d = 64)."""
    w = WORKLOADS["single_head_f32"]
    q, k, v = w.make()
    O, L = oracle.attention(_f64(q), _f64(k), _f64(v), w.causal, w.scale)
    Ob, Lb = blockwise.blockwise_attention(_f64(q[0, 0]), _f64(k[0, 0]), _f64(v[0, 0]),
                                           16, 16, w.causal, w.scale)
    np.testing.assert_allclose(Ob, O[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lb, L[0, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("blocks", [(16, 16), (128, 64), (64, 128), (32, 48)])
@pytest.mark.parametrize("variant", ["plain", "base2", "base2_slack8", "base2_slack8_lead64"])
def test_recurrence_on_ragged_wide_logits(causal, blocks, variant):
    """N = 1000 (not a multiple of any block), Q, K ~ N(0, 16): frequent max rescales."""
    w = WORKLOADS["ragged_wide_logits_bf16_n1000"]
    q, k, v = make_qkv(1, 1, w.N, w.d, "bf16", w.seed, w.sigma_qk, w.sigma_v)
    Q, K, V = _f64(q[0, 0]), _f64(k[0, 0]), _f64(v[0, 0])
    O, L = oracle.attention(Q, K, V, causal, w.scale)
    base2 = variant != "plain"
    slack = 8.0 if variant.startswith("base2_slack8") else 0.0
    lead = 64.0 if variant.endswith("lead64") else 0.0
    Ob, Lb = blockwise.blockwise_attention(Q, K, V, blocks[0], blocks[1], causal, w.scale,
                                           base2=base2, rescale_slack=slack, reference_lead=lead)
    np.testing.assert_allclose(Ob, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lb, L, rtol=0, atol=1e-11)


def test_slack_keeps_probabilities_exact():
    """With a rescale slack of 8 (base 2) the probability rows are still exact."""
    r = np.random.default_rng(7)
    n, d = 300, 16
    Q, K, V = r.normal(size=(n, d)) * 4, r.normal(size=(n, d)) * 4, np.eye(n)[:, :d]
    # V's first columns pick out probabilities; O = P[:, :d] stays exact
    O, L = oracle.attention(Q, K, V, False, 0.25)
    Ob, Lb = blockwise.blockwise_attention(Q, K, V, 32, 32, False, 0.25, base2=True,
                                           rescale_slack=8.0)
    np.testing.assert_allclose(Ob, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Lb, L, rtol=0, atol=1e-11)


@pytest.mark.parametrize("lead", [0.0, 64.0])
def test_lead_keeps_probabilities_exact(lead):
    """A reference set 64 (base 2) above the row maximum when it moves, with slack 8:
    the probability rows are still exact, and so is L."""
    r = np.random.default_rng(9)
    n, d = 300, 16
    Q, K, V = r.normal(size=(n, d)) * 4, r.normal(size=(n, d)) * 4, np.eye(n)[:, :d]
    O, L = oracle.attention(Q, K, V, True, 0.25)
    Ob, Lb = blockwise.blockwise_attention(Q, K, V, 32, 32, True, 0.25, base2=True,
                                           rescale_slack=8.0, reference_lead=lead)
    np.testing.assert_allclose(Ob, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Lb, L, rtol=0, atol=1e-11)


def test_lead_moves_the_reference_less_often():
    """On wide logits (Q, K ~ N(0, 16), d = 128) most 32-key blocks raise some row's
    maximum past a reference at the maximum plus 8, and almost none past one set 64
    above it: counted with the model's own grow rule, block by block."""
    w = WORKLOADS["ragged_wide_logits_bf16_n1000"]
    q, k, _ = make_qkv(1, 1, w.N, w.d, "bf16", w.seed, w.sigma_qk, w.sigma_v)
    Q, K = _f64(q[0, 0]), _f64(k[0, 0])
    s = (Q[:32] @ K.T) * w.scale * blockwise.LOG2E
    moves = {}
    for lead in (0.0, 64.0):
        m = np.full(32, -np.inf)
        count = 0
        for k0 in range(32, w.N, 32):  # blocks after the first, which always moves it
            if not np.isfinite(m).all():
                m = s[:, :32].max(axis=1) + lead
            bmax = s[:, k0:k0 + 32].max(axis=1)
            grow = bmax > m + 8.0
            count += int(grow.any())
            m = np.where(grow, bmax + lead, m)
        moves[lead] = count
    assert moves[0.0] >= 10 and moves[64.0] <= 1, moves


def test_causal_early_exit_equals_masking_every_block():
    """Ending the key loop at the first block after the query block (first page) gives
    the definition's result, which masks every later key individually."""
    r = np.random.default_rng(8)
    n, d = 100, 8
    Q, K, V = r.normal(size=(n, d)), r.normal(size=(n, d)), r.normal(size=(n, d))
    O, L = oracle.attention(Q, K, V, True, 0.5)
    Ob, Lb = blockwise.blockwise_attention(Q, K, V, 16, 16, True, 0.5)
    np.testing.assert_allclose(Ob, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Lb, L, rtol=0, atol=1e-13)
