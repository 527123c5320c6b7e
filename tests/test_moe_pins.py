"""Pin of the MoE FFN core oracle (oracle.moe) against the closed form of
``moe_cases.structured`` (every step exact: sigmoid is 1, quantisation is
lossless, W2 is a per-expert permutation).  Swapping the gate and up halves,
dropping the multiplication, using another expert's W2 or transposing W2 all
break it."""
import numpy as np

import oracle
from oracle import moe
import moe_cases


def test_moe_ffn_closed_form(orc):
    c = moe_cases.structured(hidden=256, inter=128, counts=[3, 0, 5], seed=4, align=1)
    pk = lambda s: np.stack([oracle.pack_scales(x) for x in s])
    rows = np.arange(c["offsets"][-1])
    res = moe.moe_ffn(c["A"], oracle.pack_scales(c["sfa"]), c["W13"], pk(c["sfw13"]), c["W2"],
                      pk(c["sfw2"]), c["offsets"], rows)
    assert np.array_equal(res["D"], c["D"])
    assert np.array_equal(res["expert"], [0, 0, 0, 2, 2, 2, 2, 2])
