"""Write tests/golden/c4_static_scale.json: the calibrated static FP8 scale of
the C4 workload (65536 tokens, tp=8, shard 8192 x 7168, rank 7).

The scale is max |y| over the rank's shard divided by 448, y being the
normalised output before quantisation, computed by the CPU oracle on the
seeded inputs.  The inputs come from the counter-based generator the tests
and the benchmark use (drawn on the host, so no GPU is needed); only the
oracle does arithmetic here.

    python tests/golden/make_static_scale.py [OUT.json]
"""

import json
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from reduce_add_rmsnorm_amd.inputs import WORKLOADS, make_inputs  # noqa: E402


def bits(t):
    t = t.contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def main():
    w = WORKLOADS["C4"]
    t0 = time.time()
    x = make_inputs(w, rank=w.rank)
    h = {k: (None if v is None else bits(v)) for k, v in x.items()}
    del x
    S = w.shard_rows
    amax = 0.0
    step = 512
    for r0 in range(0, S, step):
        rows = np.arange(r0, min(S, r0 + step))
        ref = oracle.reduce_add_rmsnorm(h["partials"], h["residual"], h["weight"], h["bias"],
                                        w.eps, oracle.QUANT_NONE, h["deepstack"], tp_rank=w.rank,
                                        num_tokens=w.num_tokens, out_dtype=oracle.ORC_F32,
                                        rows=rows)
        amax = max(amax, float(np.abs(ref["y"]).max()))
        print(f"rows {r0}..{rows[-1]}: running max |y| = {amax!r}", flush=True)
    scale = float(np.float32(amax / 448.0))
    out = {
        "workload": "C4: 65536 tokens, tp=8, shard 8192 x 7168, rank 7, bf16 inputs",
        "definition": "float32(max over the shard of |y| / 448), y = oracle's normalised output",
        "amax": amax,
        "scale": scale,
        "command": "python tests/golden/make_static_scale.py",
        "seconds": round(time.time() - t0, 1),
    }
    path = sys.argv[1] if len(sys.argv) > 1 else os.path.join(HERE, "c4_static_scale.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
