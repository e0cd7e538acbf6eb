"""Per-workload numerical-error table from the parity log the GPU tests write.

Usage:
    ATTN_PARITY_LOG=/tmp/parity.jsonl python -m pytest tests -m gpu
    python tests/parity_table.py /tmp/parity.jsonl

Each line of the log is one check_parity call (tests/helpers.py) that named a workload: the GPU
output against the fp64 oracle on the same seeded inputs. Calls of one workload (the 128K
block-sparse check runs as four groups of heads) are merged from their element counts and
sums; the last run of each label wins when the log holds several runs."""

from __future__ import annotations

import json
import math
import sys

ORDER = ["tiny_causal", "gqa_prefill_8k", "gqa_decode_4k", "mla_decode_64k", "blocksparse_128k"]


def merge(lines):
    by_label = {}
    for ln in lines:
        rec = json.loads(ln)
        by_label[(rec["workload"], rec["label"])] = rec
    out = {}
    for (wl, _), r in by_label.items():
        m = out.setdefault(wl, {"n": 0, "sum_abs": 0.0, "sum_sq": 0.0, "ref_sq": 0.0,
                                "max_abs": 0.0, "lse_max": 0.0, "parts": 0})
        m["n"] += r["n"]
        m["sum_abs"] += r["o_sum_abs"]
        m["sum_sq"] += r["o_sum_sq"]
        m["ref_sq"] += r["o_ref_sum_sq"]
        m["max_abs"] = max(m["max_abs"], r["o_max_abs"])
        m["lse_max"] = max(m["lse_max"], r.get("lse_max_abs", 0.0))
        m["parts"] += 1
    return out


def table(merged) -> str:
    rows = ["| workload | O elements compared | O max-abs | O mean-abs | O RMSE | O relative RMSE "
            "| LSE max-abs |", "|---|---|---|---|---|---|---|"]
    for wl in ORDER + sorted(set(merged) - set(ORDER)):
        if wl not in merged:
            continue
        m = merged[wl]
        rmse = math.sqrt(m["sum_sq"] / m["n"])
        rel = math.sqrt(m["sum_sq"] / m["ref_sq"]) if m["ref_sq"] > 0 else 0.0
        rows.append(f"| {wl} | {m['n']:,} | {m['max_abs']:.3e} | {m['sum_abs'] / m['n']:.3e} | "
                    f"{rmse:.3e} | {rel:.3e} | {m['lse_max']:.3e} |")
    return "\n".join(rows)


if __name__ == "__main__":
    with open(sys.argv[1]) as f:
        print(table(merge([ln for ln in f if ln.strip()])))
