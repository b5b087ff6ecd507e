"""Write tests/golden/config1_oracle.json: the CPU oracle's outputs on the
100 seeded steps of the tiny workload (C=1, L=4, V=1000, fp32, T=1).

Calls only ``oracle/`` and the seeded input generators; run from the repo root:
    python tests/golden/make_golden.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from isd_inputs import CONFIGS, gen_step  # noqa: E402
from oracle import isd_oracle as O  # noqa: E402


def main():
    cfg = CONFIGS[1]
    steps = []
    for step in range(cfg["steps"]):
        d = gen_step(1, step)
        p = O.decode_logits(d["p"], "f32")
        q = O.decode_logits(d["q"], "f32")
        qn = O.decode_logits(d["qn"], "f32")
        v = O.verify_sample(p, q, d["x"], d["ua"], d["ur"], cfg["T"])
        tok, prob, margin, _ = O.propose_sample(qn, d["up"], cfg["T"])
        steps.append(dict(
            step=step,
            accept_len=v["accept_len"].tolist(),
            out_tokens=v["out_tokens"].tolist(),
            n_emitted=v["n_emitted"].tolist(),
            alpha=v["alpha"].tolist(),
            p_x=v["p_x"].tolist(),
            q_x=v["q_x"].tolist(),
            flagged=v["flagged"].tolist(),
            resid_flagged=v["resid_flagged"].tolist(),
            next_tokens=tok.tolist(),
            next_prob=prob.tolist(),
            next_margin=margin.tolist(),
        ))
    out = dict(about="CPU oracle outputs for the tiny ISD workload (C=1, L=4, V=1000, fp32, "
                     "T=1), 100 seeded steps; written by tests/golden/make_golden.py",
               steps=steps)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "config1_oracle.json")
    with open(path, "w") as f:
        f.write('{"about": %s,\n "steps": [\n' % json.dumps(out["about"]))
        f.write(",\n".join("  " + json.dumps(s) for s in steps))
        f.write("\n]}\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
