"""Writes train_8k_lambda_grads.json: the oracle's dL/dlambda and the four
lambda-vector gradients for the full training workload (batch 2, 8192 causal
tokens, 16 heads, d 64, dv 128, seeded inputs and upstream gradient of
workloads.make_attn_inputs("train_8k"), lambda_init at layer 12), for both
RMSNorm eps values.  Only oracle.diff_attn_lambda_grad does arithmetic; the
32 (batch, head) slices run in worker processes and their contributions are
summed (lambda is shared by every head).  Takes a few minutes.
Run: python tests/golden/make_train_8k_lambda_grads.py"""
import json
import os
import sys
from concurrent.futures import ProcessPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from differential_attention_02_amd import workloads  # noqa: E402

NAMES = ("q1", "k1", "q2", "k2", "v")
_INP = None


def _slice(args):
    b, h, eps = args
    global _INP
    if _INP is None:
        _INP = workloads.make_attn_inputs("train_8k")
    x = [_INP[k][b:b + 1, :, h:h + 1].double().numpy() for k in NAMES]
    dy = _INP["dy"][b:b + 1, :, h:h + 1].double().numpy()
    vecs = [t.double().numpy() for t in _INP["lambda_vecs"]]
    g = oracle.diff_attn_lambda_grad(*x, dy, lam_init=oracle.lambda_init(12), lam_vectors=vecs, causal=True,
                                     norm=True, eps=eps)
    return {k: np.asarray(g[k], dtype=np.float64).tolist() for k in ("dlambda", "dlq1", "dlk1", "dlq2", "dlk2")}


def main():
    cfg = workloads.CONFIGS["train_8k"]
    rec = {"workload": "train_8k: batch 2, 8192 causal tokens, 16 heads, d 64, dv 128, bf16 inputs from "
                       "workloads.make_attn_inputs('train_8k') (seed 0), lambda_init at layer 12",
           "source": "oracle.diff_attn_lambda_grad summed over the 32 (batch, head) slices",
           "eps": {}}
    jobs = int(os.environ.get("JOBS", "8"))
    for eps in (1e-5, 1e-8):
        work = [(b, h, eps) for b in range(cfg.batch) for h in range(cfg.heads)]
        with ProcessPoolExecutor(max_workers=jobs) as ex:
            parts = list(ex.map(_slice, work))
        tot = {k: np.sum([np.asarray(p[k]) for p in parts], axis=0) for k in parts[0]}
        rec["eps"][repr(eps)] = {k: np.asarray(v).tolist() for k, v in tot.items()}
        print(f"eps {eps}: dlambda {float(tot['dlambda']):.10g}", flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "train_8k_lambda_grads.json")
    with open(path, "w") as f:
        json.dump(rec, f)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
