"""Write oracle_tiny.json: oracle outputs on tiny seeded inputs.

Calls only the oracle and the seeded workload generator. The pages print no
worked numeric example, so this fixture is a regression pin on the oracle
itself (it must not drift), not an independent truth; the independent pins
are the brute-force, library and closed-form tests.

Run from the repository root:  python tests/golden/make_oracle_fixture.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

CASES = [
    ("decoder_causal_bf16", dict(B=1, H=2, N=9, d=4)),
    ("encoder_padded_bf16", dict(B=2, H=1, N=7, d=4, key_len_range=(2, 7))),
    ("single_head_fp32", dict(N=5, d=3)),
    ("long_causal_fp8", dict(H=1, N=6, d=4)),
]


def main():
    out = []
    for name, shape in CASES:
        spec = W.SPECS[name].with_shape(**shape)
        w = W.draw(spec)
        q, k, v = w.exact()
        s = spec.scale
        o, lse = oracle.attention_forward(q, k, v, s, spec.causal, w.key_len_or_none())
        out.append(dict(name=name, shape=shape, seed=spec.seed,
                        key_len=None if w.key_len is None else w.key_len.tolist(),
                        o=[float(x).hex() for x in o.reshape(-1)],
                        lse=[float(x).hex() for x in lse.reshape(-1)]))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
