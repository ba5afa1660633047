"""GPU: a propose -> verify step captured in a HIP graph.

The calls only enqueue kernels (no allocation, synchronisation or memset
inside a call), so a step of all four entry points can be captured once and
replayed.  Every replay must reproduce the eager outputs exactly; the
outputs are poisoned before each replay, and other eager library work and
synchronisations run between replays."""
import numpy as np
import pytest
import torch

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import check_rejection, dev, host, say, to_dev

pytestmark = pytest.mark.gpu


def _step_inputs():
    ng = W.ngram_workload(8, 2048, seed=41)
    rj = W.rejection_workload(8, 3, 5000, seed=42)
    gr = W.greedy_workload(8, 4, 32000, "f32", 1.0, (0.7,), seed=43)
    tr = W.tree_workload(4, 16, 3000, seed=44)
    return ng, rj, gr, tr


def _prepare(ng, rj, gr, tr):
    return [
        ("ngram", sv.prepare_ngram(to_dev(ng["tokens"]), to_dev(ng["lengths"]), 2, 5, 8)),
        ("rejection", sv.prepare_rejection(to_dev(rj["target"]), to_dev(rj["draft_logits"]),
                                           to_dev(rj["draft"]), to_dev(rj["uniforms"]), 1.0)),
        ("greedy", sv.prepare_greedy(to_dev(gr["logits"]), to_dev(gr["drafts"][0.7]))),
        ("tree", sv.prepare_tree(to_dev(tr["logits"]), to_dev(tr["parent"]), to_dev(tr["token"]))),
    ]


def test_graph_replay_matches_eager_and_oracle(orc):
    ng, rj, gr, tr = _step_inputs()
    s = torch.cuda.Stream(device=dev())
    with torch.cuda.stream(s):
        calls = _prepare(ng, rj, gr, tr)
        for _, c in calls:
            c()
    torch.cuda.synchronize()
    eager = {name: {k: host(v).copy() for k, v in c.out.items()} for name, c in calls}

    # the eager step itself against the oracle
    r = orc.ngram_propose(ng["tokens"], ng["lengths"], 2, 5, 8)
    for k in ("proposal", "proposal_len", "match_n", "match_pos"):
        np.testing.assert_array_equal(eager["ngram"][k], r[k], err_msg="ngram " + k)
    r = orc.verify_greedy(gr["logits"], gr["drafts"][0.7])
    for k in ("accepted", "emitted", "argmax"):
        np.testing.assert_array_equal(eager["greedy"][k], r[k], err_msg="greedy " + k)
    r = orc.verify_tree(tr["logits"], tr["parent"], tr["token"])
    for k in ("accepted", "path", "emitted"):
        np.testing.assert_array_equal(eager["tree"][k], r[k], err_msg="tree " + k)
    r = orc.verify_rejection(rj["target"], rj["draft_logits"], rj["draft"], rj["uniforms"])
    flagged, mism = check_rejection({k: torch.from_numpy(v) for k, v in eager["rejection"].items()},
                                    r, "graph eager", max_flagged=2)

    say("graph capture of the four calls")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _, c in calls:
            c()
    torch.cuda.synchronize()

    other = W.greedy_workload(3, 2, 777, "bf16", 2.0, (0.5,), seed=45)
    other_ref = orc.verify_greedy(other["logits"], other["drafts"][0.5])
    for rep in range(5):
        for _, c in calls:                       # poison every output
            for v in c.out.values():
                v.fill_(-7)
        # unrelated eager library work on the default stream between replays
        o = sv.verify_greedy(to_dev(other["logits"]), to_dev(other["drafts"][0.5]))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(o["emitted"]), other_ref["emitted"])
        say("graph replay", rep)
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for name, c in calls:
            for k, v in c.out.items():
                np.testing.assert_array_equal(host(v), eager[name][k],
                                              err_msg="replay %d %s %s" % (rep, name, k))
