"""Expert placement rules (moe_place_experts, host only, through the C ABI).

hipfire expert-offload explainer, section "放置算法：auto 自动放置…": fixed
weights first, then whole layers of routed experts while the budget lasts
(the default), or single experts by decode heat (the hot set); a
configuration that does not fit is refused, naming the bytes short.  The
expected placements below are worked out by hand from those rules.
"""

import numpy as np
import pytest


@pytest.fixture(scope="module")
def q():
    import quantized_moe_decode_amd as q
    return q


def test_layers_mode_fills_whole_layers_in_order(q):
    # 4 layers x 3 experts of 10 bytes, fixed 7, budget 7 + 65: two whole
    # layers (60 bytes) fit, the third (30 more) does not
    res, placed = q.moe_place_experts(q.HFQ4_PLACE_LAYERS, 4, 3, 10, 7, 72)
    assert res.tolist() == [[1, 1, 1], [1, 1, 1], [0, 0, 0], [0, 0, 0]]
    assert placed == 60
    res, placed = q.moe_place_experts(q.HFQ4_PLACE_LAYERS, 4, 3, 10, 7, 7 + 29)
    assert res.sum() == 0 and placed == 0


def test_hotset_mode_takes_the_hottest_with_lower_index_ties(q):
    heat = np.array([[5, 9, 0], [9, 1, 7], [2, 9, 3]], dtype=np.uint64)
    # room for 4 experts of 10 bytes: the three 9s (in index order) and the 7
    res, placed = q.moe_place_experts(q.HFQ4_PLACE_HOTSET, 3, 3, 10, 0, 45, heat=heat)
    assert res.tolist() == [[0, 1, 0], [1, 0, 1], [0, 1, 0]]
    assert placed == 40
    # room for 2: the first two 9s by (layer, expert) index
    res, _ = q.moe_place_experts(q.HFQ4_PLACE_HOTSET, 3, 3, 10, 0, 29, heat=heat)
    assert res.tolist() == [[0, 1, 0], [1, 0, 0], [0, 0, 0]]
    # everything fits
    res, placed = q.moe_place_experts(q.HFQ4_PLACE_HOTSET, 3, 3, 10, 5, 1000, heat=heat)
    assert res.sum() == 9 and placed == 90


def test_refusal_names_the_bytes_short(q):
    with pytest.raises(q.Hfq4Error) as ex:
        q.moe_place_experts(q.HFQ4_PLACE_LAYERS, 2, 2, 10, 1000, 900)
    assert ex.value.code == q.HFQ4_E_NOFIT
    assert "short by 100 bytes" in str(ex.value) and "DOES NOT FIT" in str(ex.value)


def test_bad_arguments_refused(q):
    with pytest.raises(q.Hfq4Error):
        q.moe_place_experts(q.HFQ4_PLACE_HOTSET, 2, 2, 10, 0, 100)        # no heat
    with pytest.raises(q.Hfq4Error):
        q.moe_place_experts(7, 2, 2, 10, 0, 100)
    with pytest.raises(q.Hfq4Error):
        q.moe_place_experts(q.HFQ4_PLACE_LAYERS, 2, 2, 0, 0, 100)
