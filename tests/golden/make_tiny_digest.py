"""Write tests/golden/tiny_oracle_digest.txt: SHA-256 digests of the CPU
oracle's results on the tiny workload (64 x 512 x 256, seed 0).

It calls only the oracle and the seeded input generator.  The digests lock the
oracle's arithmetic: any later change to it must come with a new digest and a
commit message naming the passage (or the reading of it) that justifies it.

Run from the repository root:  python tests/golden/make_tiny_digest.py
"""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def digests():
    d = workloads.make_linear("tiny")
    qw, sw = oracle.quantize_weight(d["w"])
    qx, sx = oracle.rotate_quant_act(d["x"])
    acc = oracle.gemm_s32(qx, qw)
    y = oracle.dequant_bf16(acc, sx, sw)
    ysw = oracle.swiglu_bf16(acc, sx, sw)
    out = {}
    for name, a in [("x", d["x"]), ("w", d["w"]), ("q_w", qw), ("s_w", sw), ("q_x", qx),
                    ("s_x", sx), ("acc", acc), ("y", y), ("y_swiglu", ysw)]:
        out[name] = hashlib.sha256(a.tobytes()).hexdigest()
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_digest.txt")
    with open(path, "w") as f:
        f.write("# SHA-256 of the oracle's arrays on the tiny workload (written by make_tiny_digest.py)\n")
        for k, v in digests().items():
            f.write("%s %s\n" % (k, v))
    print(open(path).read())
