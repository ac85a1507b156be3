"""Writes the committed parity tie table from the per-request records the
GPU tests append to $DTREE_PARITY_LOG (tests/gpu_util.py):

    python tests/tie_table.py gpurun_out/parity_ties.jsonl profiles/parity_ties.md

Per workload group: requests compared with the oracle to their last node,
tolerated ties (selections where the GPU kept another admissible set, by
stage), the oracle's ambiguous decisions (values within 1e-4 of a cutoff,
where an admissible alternative existed), emitted nodes and superarbol
nodes compared."""
import collections
import json
import sys


def group(rec):
    if rec["workload"] != "custom":
        return rec["workload"] + (" (marginal)" if rec["scoring"] == "marginal" else "")
    return rec["label"].split(" ")[0] + " shapes" + (
        " (marginal)" if rec["scoring"] == "marginal" else "")


def main(src, dst, cmd):
    recs = [json.loads(line) for line in open(src)]
    rows = collections.OrderedDict()
    for r in recs:
        g = rows.setdefault(group(r), dict(req=0, ties=collections.Counter(), amb=0, nodes=0,
                                           sa=0, seeds=set()))
        g["req"] += 1
        g["amb"] += r["ambiguous"]
        g["nodes"] += r["nodes"]
        g["sa"] += r["superarbol"]
        g["seeds"].add(r["seed"])
        for t in r["ties"]:
            g["ties"][t["stage"]] += 1
    out = ["# Parity: tolerated near-ties per workload", "",
           "Every request is compared with the oracle to its last node. A tolerated tie is a",
           "selection (Top-M `M`, Top-K `K`, Top-W `W`, Top-B `B`) where the GPU kept a different set",
           "that is an admissible alternative of the oracle's own decision (values within 1e-4 of the",
           "cutoff); the oracle then builds the rest of the tree along it. Ambiguous decisions are",
           "the oracle's decisions where such an alternative existed at all.", "",
           f"Command: `{cmd}`", "",
           "| group | requests | tolerated ties | ambiguous decisions (oracle) | emitted nodes compared | superarbol nodes compared |",
           "|---|---:|---|---:|---:|---:|"]
    tot = collections.Counter()
    for name, g in rows.items():
        ties = ", ".join(f"{k}: {v}" for k, v in sorted(g["ties"].items())) or "0"
        out.append(f"| {name} | {g['req']} | {ties} | {g['amb']} | {g['nodes']} | {g['sa']} |")
        tot["req"] += g["req"]; tot["amb"] += g["amb"]; tot["nodes"] += g["nodes"]
        tot["sa"] += g["sa"]; tot["ties"] += sum(g["ties"].values())
    out.append(f"| **all** | {tot['req']} | {tot['ties']} | {tot['amb']} | {tot['nodes']} | {tot['sa']} |")
    with open(dst, "w") as f:
        f.write("\n".join(out) + "\n")


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2],
         "DTREE_PARITY_LOG=gpurun_out/parity_ties.jsonl python -m pytest tests -m gpu")
