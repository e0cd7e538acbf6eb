"""CPU check of tests/parity_table.py: records of one workload merge by element counts and
sums (the RMSE of the union, not the mean of the parts' RMSEs), and a repeated label keeps
its last record."""

import json
import math

from tests import parity_table as P


def _rec(wl, label, n, sabs, ssq, refsq, mx, lse):
    return json.dumps({"workload": wl, "label": label, "n": n, "o_sum_abs": sabs, "o_sum_sq": ssq,
                       "o_ref_sum_sq": refsq, "o_max_abs": mx, "lse_max_abs": lse})


def test_merge_by_sums():
    lines = [_rec("w", "a", 4, 0.4, 0.04, 4.0, 0.2, 1e-4),
             _rec("w", "b", 12, 1.2, 0.36, 12.0, 0.1, 3e-4),
             _rec("w", "a", 4, 0.8, 0.16, 4.0, 0.3, 2e-4)]      # replaces the first "a"
    m = P.merge(lines)["w"]
    assert m["n"] == 16 and m["parts"] == 2
    assert math.isclose(m["sum_abs"], 2.0) and math.isclose(m["sum_sq"], 0.52)
    assert m["max_abs"] == 0.3 and m["lse_max"] == 3e-4
    t = P.table(P.merge(lines))
    assert f"{math.sqrt(0.52 / 16):.3e}" in t and f"{math.sqrt(0.52 / 16.0):.3e}" in t
    assert f"{2.0 / 16:.3e}" in t
