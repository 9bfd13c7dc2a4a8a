"""GPU checks of the index-list validator (sla_validate_lists) and of the
clamping every compute entry point applies to list entries.

The validator's verdicts are compared with what the lists are by
construction (routing output is valid; each planted fault names its row).
The clamping contract (an entry outside [0, nkb) is used as the nearest
valid block) is checked by comparing the forward on a list with planted
out-of-range entries with the forward on the same list with those entries
clamped by hand: both must agree bit for bit.
"""
import re

import pytest
import torch

import block_sparse_linear_route_amd as s
from block_sparse_linear_route_amd import SlaError
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _routed(name):
    w = make_workload(name)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    r = s.route(q, k, w.k_crit, w.k_marg)
    return w, q, k, v, r


@pytest.mark.parametrize("name", ["tiny", "seq8k"])
def test_routing_output_is_valid(name):
    w, q, k, v, r = _routed(name)
    s.validate_lists(q, r["crit_idx"], r["marg_idx"])
    s.validate_lists(q, r["crit_idx"], None)
    s.validate_lists(q, None, r["marg_idx"])


def _first(err):
    m = re.search(r"(\d+) of \d+ rows.*batch (\d+), head (\d+), query block (\d+)", str(err))
    assert m, str(err)
    return tuple(int(x) for x in m.groups())


@pytest.mark.parametrize("fault", ["past_end", "negative", "repeat_crit", "repeat_marg", "both_lists"])
def test_planted_faults_are_reported_at_their_row(fault):
    w, q, k, v, r = _routed("seq8k")
    nkb = (w.shape[2] + 63) // 64
    crit, marg = r["crit_idx"].clone(), r["marg_idx"].clone()
    rows = [(0, 7, 100), (0, 3, 5)]           # (b, h, i): planted in both, first is (0, 3, 5)
    for b, h, i in rows:
        if fault == "past_end":
            crit[b, h, i, 1] = nkb
        elif fault == "negative":
            marg[b, h, i, 2] = -1
        elif fault == "repeat_crit":
            crit[b, h, i, 1] = crit[b, h, i, 0]
        elif fault == "repeat_marg":
            marg[b, h, i, -1] = marg[b, h, i, 0]
        else:
            marg[b, h, i, 3] = crit[b, h, i, 2]
    with pytest.raises(SlaError) as e:
        s.validate_lists(q, crit, marg)
    assert _first(e.value) == (2, 0, 3, 5)
    # the untouched lists still pass
    s.validate_lists(q, r["crit_idx"], r["marg_idx"])


def test_out_of_range_entries_are_clamped_by_the_forward():
    w, q, k, v, r = _routed("seq8k")
    nkb = (w.shape[2] + 63) // 64
    crit, marg = r["crit_idx"].clone(), r["marg_idx"].clone()
    crit[0, 1, 10, 0] = -5
    crit[0, 4, 60, -1] = nkb + 1000
    marg[0, 2, 33, 4] = 1 << 30
    marg[0, 9, 0, 0] = -(1 << 30)
    Hs, zs = s.linear_states(k, v)
    alpha = w.alpha.to(q.device)
    o_bad = s.forward(q, k, v, crit, marg, Hs, zs, alpha)
    o_ref = s.forward(q, k, v, crit.clamp(0, nkb - 1), marg.clamp(0, nkb - 1), Hs, zs, alpha)
    torch.cuda.synchronize()
    assert torch.equal(o_bad, o_ref)
    assert torch.isfinite(o_bad.float()).all()
