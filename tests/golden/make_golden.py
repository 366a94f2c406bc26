"""Write tests/golden/tiny.json: oracle outputs on the 4-row tiny workload.

This script calls only the oracle and the input generator. The pages print no
worked numerical example for the log-probability path, so these stored values
are an oracle snapshot (a regression fixture), not printed values. Each case
names the passage it exercises: the full-vocabulary reference logprob follows
page "Configurable H100 consistency runs" (mode/KL paragraph), the policy
support follows the same page's sampling paragraph and its commands section
(top-k independent of top-p and temperature).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import datagen  # noqa: E402
from oracle import logp as O  # noqa: E402

SUPPORT_CASES = [(0.9, -1), (0.95, 50), (1.0, 10), (0.5, 3)]


def main():
    w = datagen.tiny()
    logits, targets = w.generate()
    rows = []
    for i in range(w.n_rows):
        t = int(targets[i])
        ref, lse = O.ref_logp_row(logits[i], w.vocab_real, 1.0, t)
        cases = []
        for p, k in SUPPORT_CASES:
            # the target for each support case: the row's argmax (always kept)
            am = int(np.argmax(O.decode_bf16(logits[i, :w.vocab_real])))
            pol, ref2, info = O.nucleus_row(logits[i], w.vocab_real, 1.0, p, k, am)
            cases.append({"top_p": p, "top_k": k, "target": am, "policy_logp": pol,
                          "ref_logp": ref2, "support_size": info.support_size})
        rows.append({"row": i, "target": t, "ref_logp": ref, "lse": lse, "support": cases})
    out = {
        "workload": "tiny: 4 rows x vocab 1024 (real 1000), N(0, 3^2) BF16, seed 1001, T = 1.0",
        "source": "oracle snapshot written by tests/golden/make_golden.py",
        "cite": "RL-Kernel page 'Configurable H100 consistency runs', sampling and mode/KL paragraphs",
        "rows": rows,
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
