"""Write the oracle's results for a full-size verify workload (default: the
8B-shaped batch-1 step, seeds 0..4) to verify_<workload>.json: the draft tokens planted against the
oracle's argmax (by the workload's planting rule), the oracle's per-node argmax and top-2 gap, and
the accepted path. The stored files: llama8b-b1 (5 seeds), llama8b-b64 (2), llama70b-b8 (5), and
the chain-vs-tree workloads chain60-b64, tree60-b64, chain40-b64, tree40-b64 (1 seed each). The benchmark reads the planted tokens from here (so no planting ever
uses the GPU's own argmax) and the GPU tests compare against the rest.

Calls only the oracle and the seeded generators. Usage:
    python tests/golden/make_verify_golden.py [workload [number of seeds]]
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402


def main(name="llama8b-b1", seeds=range(5)):
    shape = synth.VERIFY_SHAPES[name]
    W = synth.lm_head_weight(shape, shape.V, shape.K)
    out = {"workload": name, "generator": "synth.verify_inputs(shape, seed); synth.lm_head_weight(shape, V, K)",
           "oracle": "oracle.verify_step", "seeds": {}}
    for seed in seeds:
        inp = synth.verify_inputs(shape, seed)
        r = oracle.verify_step(inp, W)
        out["seeds"][str(seed)] = {
            "tokens": r["tokens"].tolist(), "idx": r["idx"].tolist(), "gap": r["gap"].tolist(),
            "accept_len": r["accept_len"].tolist(), "path": r["path"].tolist(),
            "out_tokens": r["out_tokens"].tolist(), "flagged": r["flagged"].tolist(),
        }
        print(seed, "accept_len", r["accept_len"].tolist(), "flagged", r["flagged"].tolist(), flush=True)
    path = os.path.join(HERE, f"verify_{name}.json")
    with open(path, "w") as f:
        json.dump(out, f, separators=(",", ":"))
    print("wrote", path)


if __name__ == "__main__":
    name = sys.argv[1] if len(sys.argv) > 1 else "llama8b-b1"
    n = int(sys.argv[2]) if len(sys.argv) > 2 else 5
    main(name, range(n))
