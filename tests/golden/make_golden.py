"""Write the stored expected values under tests/golden/.

The pages print no worked example with numbers, so every stored value here is the oracle's
output on a seeded workload (this script calls only the oracle and the input generators).
Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from tests._util import bits, oracle_cache  # noqa: E402
from workloads import make_named  # noqa: E402


def main():
    wl = make_named("tiny_d64_n1024", device="cpu")
    cache = oracle_cache(wl)
    qb = bits(wl.q)
    idx = oracle.decode_topk(qb, cache, wl.k_per_req.numpy(), wl.k_max)
    o_s, l_s = oracle.decode_sparse(qb, cache, idx)
    o_d, l_d = oracle.decode_dense(qb, cache)
    rec = {
        "workload": "tiny_d64_n1024 (B1 T1 Hq4 Hkv1 d64 N1024 k32, one needle per query head, seed 1001)",
        "source": "oracle output (the pages print no worked example)",
        "needles": wl.needles.tolist(),
        "topk_indices": idx.tolist(),
        "sparse_out": o_s.tolist(),
        "sparse_lse": l_s.tolist(),
        "dense_out": o_d.tolist(),
        "dense_lse": l_d.tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_d64_n1024.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=None, separators=(",", ":"))
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
