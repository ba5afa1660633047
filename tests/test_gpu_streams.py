"""GPU: calls are reentrant and keep no hidden state.  Two streams (default
priority) each run their own calls, with their own inputs, outputs and
workspaces, back to back and interleaved; every result must equal the
oracle's (bit-exact for greedy, tree and n-gram; decisions except
oracle-flagged ties for rejection sampling)."""
import numpy as np
import pytest
import torch

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import check_rejection, dev, host, say, to_dev

pytestmark = pytest.mark.gpu


def test_two_streams_same_and_different_calls(orc):
    sa, sb = torch.cuda.Stream(device=dev()), torch.cuda.Stream(device=dev())
    ga = W.greedy_workload(16, 6, 50000, "bf16", 2.0, (0.6,), seed=61)
    gb = W.greedy_workload(9, 3, 70001, "f32", 2.0, (0.8,), seed=62)
    rj = W.rejection_workload(12, 4, 40000, seed=63)
    tr = W.tree_workload(6, 32, 30000, seed=64)
    ng = W.ngram_workload(40, 4096, seed=65)
    inputs = [to_dev(a) for a in (ga["logits"], ga["drafts"][0.6], gb["logits"], gb["drafts"][0.8],
                                  rj["target"], rj["draft_logits"], rj["draft"], rj["uniforms"],
                                  tr["logits"], tr["parent"], tr["token"], ng["tokens"], ng["lengths"])]
    torch.cuda.synchronize()
    (gal, gad, gbl, gbd, rjt, rjd, rjx, rju, trl, trp, trt, ngt, ngl) = inputs
    with torch.cuda.stream(sa):                  # stream A: greedy (bf16) and rejection
        a_calls = [sv.prepare_greedy(gal, gad), sv.prepare_rejection(rjt, rjd, rjx, rju)]
    with torch.cuda.stream(sb):                  # stream B: greedy (fp32), tree and n-gram
        b_calls = [sv.prepare_greedy(gbl, gbd), sv.prepare_tree(trl, trp, trt),
                   sv.prepare_ngram(ngt, ngl, 2, 5, 8)]
    refs = [orc.verify_greedy(ga["logits"], ga["drafts"][0.6]),
            orc.verify_rejection(rj["target"], rj["draft_logits"], rj["draft"], rj["uniforms"]),
            orc.verify_greedy(gb["logits"], gb["drafts"][0.8]),
            orc.verify_tree(tr["logits"], tr["parent"], tr["token"]),
            orc.ngram_propose(ng["tokens"], ng["lengths"], 2, 5, 8)]
    for rep in range(4):
        say("two streams, round", rep)
        for c in a_calls + b_calls:              # poison every output first
            for v in c.out.values():
                v.fill_(-5)
        torch.cuda.synchronize()
        for k in range(3):                       # interleave the two streams' launches
            with torch.cuda.stream(sa):
                a_calls[k % 2]()
            with torch.cuda.stream(sb):
                b_calls[k % 3]()
        with torch.cuda.stream(sa):
            for c in a_calls:
                c()
        with torch.cuda.stream(sb):
            for c in b_calls:
                c()
        torch.cuda.synchronize()
        outs = [c.out for c in a_calls + b_calls]
        for k in ("accepted", "emitted", "argmax"):
            np.testing.assert_array_equal(host(outs[0][k]), refs[0][k], err_msg="greedy A " + k)
            np.testing.assert_array_equal(host(outs[2][k]), refs[2][k], err_msg="greedy B " + k)
        f, m = check_rejection(outs[1], refs[1], "rejection A")
        assert m <= f
        for k in ("accepted", "path", "emitted", "argmax"):
            np.testing.assert_array_equal(host(outs[3][k]), refs[3][k], err_msg="tree " + k)
        for k in ("proposal", "proposal_len", "match_n", "match_pos"):
            np.testing.assert_array_equal(host(outs[4][k]), refs[4][k], err_msg="ngram " + k)
