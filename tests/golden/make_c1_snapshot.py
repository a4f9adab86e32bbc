"""Write c1_oracle_snapshot.json: the oracle's decode step on the seeded tiny
fp32 workload (1 sequence, 2 query heads on 1 KV head, d = 64, context 512,
B = 64, 4 dominant FCs per head).

Only the oracle computes the stored values; the inputs come from the seeded
generators.  Run from the repository root:  python tests/golden/make_c1_snapshot.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads as W  # noqa: E402


def snapshot():
    w = W.get("c1")
    x = W.generate(w)
    st = oracle.OracleState(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim,
                            w.rope_theta, w.dtype, x["dom"], w.capacity)
    n0 = int(x["ctx"][0])
    st.append(0, x["k_prefill"][0][:, :n0 - 1], x["v_prefill"][0][:, :n0 - 1])
    r = st.step(x["q"][0], x["k_new"][0], x["v_new"][0], w.budget)
    return {
        "workload": w.name,
        "note": "oracle output on seeded inputs; regression guard, not a pin",
        "idx": r["idx"][0].tolist(),
        "tau": r["tau"][0].tolist(),
        "out": [[float(v) for v in row] for row in r["out"][0]],
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "c1_oracle_snapshot.json"), "w") as f:
        json.dump(snapshot(), f, indent=1)
