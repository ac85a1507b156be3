"""Helpers for the GPU tests: run a round through the C ABI and compare it
with the oracle request by request."""
import sys

import numpy as np

import synth
from oracle import dtree_oracle as O
from checker import compare_request


def caps_for(cfg, **over):
    c = dict(max_batch=cfg.batch, max_D=cfg.D, max_M=cfg.M, max_K=cfg.K, max_W=cfg.W,
             max_B=cfg.B)
    c.update(over)
    return (c["max_batch"], c["max_D"], c["max_M"], c["max_K"], c["max_W"], c["max_B"])


def gpu_round(inputs, cfg, caps=None, beta=None, runs=1, scoring="conditional"):
    from conditional_draft_tree_depth_amd import runner
    import torch
    wd, H, root = runner.to_device(inputs)
    rnd = runner.Round(wd, cfg.wtype, caps or caps_for(cfg), cfg.batch, cfg.D, cfg.M, cfg.K,
                       cfg.W, cfg.B, cfg.beta if beta is None else beta, scoring=scoring)
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


def check_config(inputs, cfg, label, max_tie_frac=0.0, caps=None, scoring="conditional"):
    """GPU round vs oracle on every request; returns the tie descriptions."""
    print(f"[gpu] {label}: batch={cfg.batch} D={cfg.D} M={cfg.M} K={cfg.K} W={cfg.W} "
          f"B={cfg.B} beta={cfg.beta} wtype={cfg.wtype} scoring={scoring}", flush=True)
    gouts, gtrs = gpu_round(inputs, cfg, caps, scoring=scoring)
    orcs = O.build_round(inputs, cfg.D, cfg.M, cfg.K, cfg.W, cfg.B, cfg.beta, scoring=scoring)
    prm = dict(D=cfg.D, M=cfg.M, K=cfg.K, W=cfg.W, B=cfg.B, beta=cfg.beta)
    ties = []
    for q in range(cfg.batch):
        res = compare_request(gouts[q], gtrs[q], orcs[q], prm, where=f"{label} req {q}: ")
        if not res["exact"]:
            ties.append(f"req {q}: {res['tie']}")
    if ties:
        print(f"[gpu] {label}: tolerated near-ties: {ties}", flush=True)
    assert len(ties) <= max_tie_frac * cfg.batch, ties
    sys.stdout.flush()
    return ties
