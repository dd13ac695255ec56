"""Write the stored expected values under tests/golden/.

Calls only ``oracle`` (and the seeded input generators in ``workloads``); no
value here comes from the HIP implementation.  Run from the repository root:

    python tests/golden/make_golden.py

Fixture ``tiny_seed0.json``: the tiny workload (N=16, H=128 fp32, E=8,
topk=2, seed 0).  The small integer outputs are stored in full; the float
arrays are stored as SHA-256 digests of their little-endian bytes, so the
file stays small while a single flipped bit anywhere still fails.
"""

import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as W  # noqa: E402


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def tiny_fixture() -> dict:
    w = W.WORKLOADS["tiny"]
    inp = W.make_all(w, seed=0, device="cpu")
    ids = inp["topk_ids"].numpy()
    wts = inp["topk_weights"].numpy()
    x = inp["hidden_states"].numpy()
    y = inp["expert_output"].numpy()
    p = oracle.permute(x, ids, w.num_experts)
    out = oracle.unpermute(y, wts, p["inv_permuted_idx"], "f32")
    return {
        "about": "tiny workload, seed 0; expected values from oracle/ (moe_oracle.c) only",
        "workload": {"num_tokens": w.num_tokens, "hidden_size": w.hidden_size,
                     "num_experts": w.num_experts, "topk": w.topk, "dtype": "f32", "seed": 0},
        "inputs": {
            "topk_ids": ids.tolist(),
            "topk_weights_f32_hex": [[float(v).hex() for v in row] for row in wts],
            "hidden_states_sha256": sha(x),
            "expert_output_sha256": sha(y),
        },
        "expected": {
            "expert_first_token_offset": p["expert_first_token_offset"].tolist(),
            "permuted_idx": p["permuted_idx"].tolist(),
            "inv_permuted_idx": p["inv_permuted_idx"].tolist(),
            "permuted_hidden_states_sha256": sha(p["permuted_hidden_states"]),
            "output_sha256": sha(out),
        },
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_seed0.json"), "w") as f:
        json.dump(tiny_fixture(), f, indent=1)
        f.write("\n")
    print("wrote", os.path.join(HERE, "tiny_seed0.json"))
