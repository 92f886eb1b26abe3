"""Calibrate the skewed expert bias of the c2, c3 and c4 workloads (test data).

The c2 workload asks for an expert bias that sends about half of all routes
to 16 of the 128 experts.  Its literal recipe (+1.0 on those experts) sends
every route there, because the bias is added to scores in (0, 1) after the
sigmoid / softmax ([muse_moe_runner] MuseSpark1xRouter: the bias is added to
the normalised scores, for selection only).  This script keeps the stated
intent: it bisects the hot-expert bias delta (0 on the other experts) on the
workload's own seeded routing inputs, using only the oracle's routing, until
the hot share of routes is closest to 0.5, and writes the result to
synth/skew_calibration.json.

Run: python -m oracle.calibrate_skew
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import synth  # noqa: E402
from oracle import steps as ob  # noqa: E402


def hot_share(logits, name, delta):
    d = synth.CONFIGS[name]
    hot = synth.hot_experts(synth.inputs.SEEDS[name], d.experts)
    bias = np.zeros(d.experts, dtype=np.float32)
    bias[hot] = np.float32(delta)
    s = ob.score(logits, d.scoring, d.multiplier)
    ids, _ = ob.select_topk(s, bias, d.top_k)
    return float(np.isin(ids, hot).mean())


def calibrate(name):
    x, w, _ = synth.routing_inputs(name)
    logits = ob.router_logits(x, w)
    lo, hi = 0.0, 1.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if hot_share(logits, name, mid) < 0.5:
            lo = mid
        else:
            hi = mid
    # The share is a step function of delta; take the side closest to 0.5.
    cands = [(abs(hot_share(logits, name, v) - 0.5), v) for v in (lo, hi)]
    delta = float(np.float32(min(cands)[1]))
    return {"delta": delta, "hot_share": hot_share(logits, name, delta),
            "rows": int(x.shape[0])}


def main():
    out = {name: calibrate(name) for name in ("c2", "c3", "c4")}
    path = os.path.join(os.path.dirname(synth.__file__), "skew_calibration.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
