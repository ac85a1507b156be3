"""Helpers for the GPU tests: run a round through the C ABI and compare it
with the oracle request by request, every request to its last node.

When the environment names a file in DTREE_PARITY_LOG, one JSON line per
checked request is appended to it (workload, seed, request, tolerated ties
with their stage, the number of the oracle's ambiguous decisions, nodes
compared), from which the committed tie table is written."""
import json
import os
import sys

import numpy as np

import synth
from oracle import dtree_oracle as O
from checker import compare_request, compare_heap_request


def caps_for(cfg, **over):
    c = dict(max_batch=cfg.batch, max_D=cfg.D, max_M=cfg.M, max_K=cfg.K, max_W=cfg.W,
             max_B=cfg.B)
    c.update(over)
    return (c["max_batch"], c["max_D"], c["max_M"], c["max_K"], c["max_W"], c["max_B"])


def gpu_round(inputs, cfg, caps=None, beta=None, runs=1, scoring="conditional",
              builder="depthwise"):
    from conditional_draft_tree_depth_amd import runner
    import torch
    wd, H, root = runner.to_device(inputs)
    rnd = runner.Round(wd, cfg.wtype, caps or caps_for(cfg), cfg.batch, cfg.D, cfg.M, cfg.K,
                       cfg.W, cfg.B, cfg.beta if beta is None else beta, scoring=scoring,
                       builder=builder)
    try:
        outs = []
        for _ in range(runs):
            rnd.run(H, root)
            torch.cuda.synchronize()
            outs.append(rnd.outputs())
        traces = [rnd.trace(q) for q in range(cfg.batch)]
    finally:
        rnd.close()
    return outs if runs > 1 else outs[0], traces


def _log(rec):
    path = os.environ.get("DTREE_PARITY_LOG")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def check_outputs(inputs, cfg, gouts, gtrs, label, max_ties_per_request=0,
                  scoring="conditional", seed=None, builder="depthwise"):
    """Every request of a GPU round against the oracle (checker.py);
    returns the per-request results."""
    prep = O.prepare_round(inputs, cfg.D)
    prm = dict(D=cfg.D, M=cfg.M, K=cfg.K, W=cfg.W, B=cfg.B, beta=cfg.beta)
    cmp = compare_heap_request if builder == "heap" else compare_request
    res = []
    for q in range(cfg.batch):
        r = cmp(gouts[q], gtrs[q], prep, q, prm, where=f"{label} req {q}: ", scoring=scoring)
        res.append(r)
        _log({"label": label, "workload": cfg.name, "seed": seed, "req": q,
              "scoring": scoring, "builder": builder, "ties": r["ties"],
              "ambiguous": r["ambiguous"],
              "nodes": r["nodes"], "superarbol": r["superarbol"]})
    ties = [(q, t) for q, r in enumerate(res) for t in r["ties"]]
    if ties:
        print(f"[gpu] {label}: tolerated near-ties (all requests compared to the last node): "
              f"{ties}", flush=True)
    worst = max(len(r["ties"]) for r in res)
    assert worst <= max_ties_per_request, ties
    sys.stdout.flush()
    return res


def check_config(inputs, cfg, label, max_ties_per_request=0, caps=None,
                 scoring="conditional", seed=None, builder="depthwise"):
    """GPU round vs oracle on every request."""
    print(f"[gpu] {label}: batch={cfg.batch} D={cfg.D} M={cfg.M} K={cfg.K} W={cfg.W} "
          f"B={cfg.B} beta={cfg.beta} wtype={cfg.wtype} scoring={scoring} builder={builder}",
          flush=True)
    gouts, gtrs = gpu_round(inputs, cfg, caps, scoring=scoring, builder=builder)
    return check_outputs(inputs, cfg, gouts, gtrs, label, max_ties_per_request, scoring, seed,
                         builder)
