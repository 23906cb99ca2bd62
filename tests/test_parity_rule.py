"""The allocation comparison rule of the GPU parity tests, checked on the
CPU: a schedule that breaks exact ties against the lowest-index rule must
fail, while a swap of two refinements whose oracle gains differ inside the
1e-6 window is a near tie."""
import numpy as np

import oracle as O
from query_adaptive_decode_amd import synth
from tests.parity_util import alloc_mismatch


def _highest_index_ties(w, W, B):
    """ChooseDepths with ties broken toward the highest index: the oracle run
    on the reversed item order, reversed back."""
    return O.choose_depths(w[::-1], O.gain_table(W), W, B)[::-1]


def test_tie_order_reversal_fails_on_depth0_keys():
    # R_K = 0: every key is read at depth 0, so the 32 tokens of a group have
    # identical reconstructed keys, logits and value weights
    cfg = synth.workload(2, B=1, H=8, G=2, T0=300)
    K, V = synth.kv_unit(cfg, 0, 1, 300)
    q = synth.q_step(cfg, 0, 0)[4:8]
    for rv in (1.3, 2.1, 2.7, 3.3):
        res = O.decode_unit(q, K, V, R_K=0.0, R_V=rv)
        assert res["tK"].sum() == 0
        wrong = _highest_index_ties(res["wv"], 8, res["BV"])
        assert wrong.sum() == res["tV"].sum()
        assert not np.array_equal(wrong, res["tV"]), rv   # the ties straddle the threshold
        near, bad, det = alloc_mismatch(wrong, res["tV"], res["wv"], 8)
        assert bad > 0, (rv, near, det)
        assert "exact-tie swaps" in det
        assert alloc_mismatch(res["tV"], res["tV"], res["wv"], 8) == (0, 0, "")


def test_key_tie_order_reversal_fails():
    # two channels with equal weights at the threshold (duplicated key and
    # query channel), with a budget that splits the pair
    w = np.array([5.0, 3.0, 3.0, 1.0])
    # gains in order: 5/4, 3/4, 3/4, 5/16, 1/4, then the tie 3/16 (items 1, 2)
    B = 6
    good = O.choose_depths(w, O.gain_table(8), 8, B)
    wrong = _highest_index_ties(w, 8, B)
    assert not np.array_equal(good, wrong)
    near, bad, det = alloc_mismatch(wrong, good, w, 8)
    assert bad > 0 and "exact-tie swaps 1" in det, det


def test_swap_of_unequal_gains_inside_window_is_near():
    # item 1 is larger by 1e-9 relative and wins the last refinement; a GPU
    # that rounded the other way takes item 0 instead
    w = np.array([1.0, 1.0 + 1e-9, 10.0])
    gains = O.gain_table(8)
    B = 3
    good = O.choose_depths(w, gains, 8, B)
    assert good.tolist() == [0, 1, 2]
    gpu = np.array([1, 0, 2])
    assert alloc_mismatch(gpu, good, w, 8)[:2] == (2, 0)


def test_far_mismatch_and_total_mismatch_fail():
    w = np.array([1.0, 2.0, 10.0])
    good = O.choose_depths(w, O.gain_table(8), 8, 3)
    assert good.tolist() == [0, 1, 2]
    assert alloc_mismatch(np.array([1, 0, 2]), good, w, 8)[1] >= 1
    assert alloc_mismatch(np.array([0, 1, 3]), good, w, 8)[1] == 1
