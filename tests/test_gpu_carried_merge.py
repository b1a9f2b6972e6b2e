"""sgqa_forward on decode-shaped calls runs the merge of the blocks a call
completes (page "Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache",
section "Eight tokens become one search key, coordinate by coordinate": a
block's summary appears when its last token arrives) inside the index step's
scoring launch, which is valid because no query of such a call has a block
the call completes among its candidates (query t sees blocks below t / B).

Edge shapes of that path, each checked bit for bit against the three
separate calls and against the oracle:

* B = 16: one query completing its block, one not, three queries inside one
  block whose last completes it, two inside one block not completing it,
  and an empty sequence;
* B = 1: every single-query sequence completes its own block;
* B = 16 with one sequence whose 20 queries span blocks: the merge cannot
  ride in the scoring launch and runs as its own launch first.

The rows each call completes hold NaN codes before the forward call, so a
merge that did not run (or wrote elsewhere) shows.
"""
import numpy as np
import pytest
import torch

from synth import workloads as W

from .gpu_checks import Checker, log, prepare, run_steps
from .gpu_setup import poison_store

pytestmark = pytest.mark.gpu

# (block size, per-sequence allocation in tokens, [(n_q, pos0), ...])
CASES = {
    "b16": (16, 8192, [(1, 16 * 200 + 15), (1, 16 * 150 + 7), (3, 16 * 250 + 13), (2, 16 * 180 + 4),
                       (0, 16 * 100 + 15)]),
    "b1": (1, 4096, [(1, 3000), (1, 2000), (1, 1500)]),
    "b16_spanning": (16, 8192, [(1, 16 * 200 + 15), (20, 16 * 150 + 7)]),
}


def _workload(name, B, cap, spec, K=64):
    seqs, q = [], 0
    for i, (nq, pos0) in enumerate(spec):
        seqs.append(W.SeqLayout(q, nq, pos0, i * cap, cap, i * (cap // B), cap // B))
        q += nq
    return W.Workload("carried_merge_" + name, B, K, seqs, prebuilt=True)


@pytest.mark.parametrize("name", list(CASES))
def test_forward_merge_in_scoring_launch(name):
    B, cap, spec = CASES[name]
    wl = _workload(name, B, cap, spec)
    done = [s for s in wl.seqs if s.cache_len // B > s.pos0 // B]
    log("case", wl.name, "sequences", [(s.n_q, s.pos0) for s in wl.seqs], "completing a block:", len(done))
    assert done
    di, cfg = prepare(wl)
    run_steps(wl, di, cfg)
    keys = ("store", "sel", "sel_scores", "out", "lse")
    ref = {k: di[k].clone() for k in keys}
    for s in done:
        poison_store(di["store"][s.store_offset + s.pos0 // B:s.store_offset + s.cache_len // B])
    for k in keys[1:]:
        di[k].zero_()
    run_steps(wl, di, cfg, use_forward=True)
    for k, v in ref.items():
        assert torch.equal(di[k], v), k

    ck = Checker(wl, di, cfg)
    n_rows = 0
    for si, s in enumerate(wl.seqs):
        if s.n_q == 0:
            continue
        stored, exact = ck.oracle_store(s, s.cache_len // B)
        if s in done:
            ck.check_store(s, stored, exact, np.arange(s.pos0 // B, s.cache_len // B))
        ck.check_seq(si, np.arange(s.n_q), store_exact=(stored, exact))
        n_rows += s.n_q
    stats = ck.finish()
    log(" ", stats)
    assert stats["rows"] == n_rows
