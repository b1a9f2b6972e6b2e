"""sgqa_forward in pieces: calls whose index step is tiled and whose gather
attention takes queries run each piece's index step on the caller's stream
and its attention on the library's second stream, when every query keeps
its attention kernel and the gather its ranges.  Checked against the same
three steps as separate calls on one stream (bit-identical sel, sel_scores,
out and lse), the shared diagnostics block at sgqa_forward_diag_offset, and
the oracle on sampled rows.  The cases cover the unsplit gather over long
caches, and prefills whose leading queries take the tiled attention kernel
and the rest the gather with range splits."""
import time

import numpy as np
import pytest
import torch

import sparse_long_context_block_amd as sg
from synth import workloads as W

from .gpu_checks import Checker, lib_seqs, log, prepare, run_steps, stratified_rows

pytestmark = pytest.mark.gpu

OUTS = ("sel", "sel_scores", "out", "lse")

CASES = {
    # one sequence: 4,600 queries from t = 262,144 -> pieces of 1,136 x 3 and 1,192
    "one sequence": lambda: W.make("chunk_262144_4600"),
    # three sequences: pieces of 1,232, 1,232 and 1,236 queries cut inside
    # the first and second sequences
    "three sequences": lambda: W._multi("pieces_multi", [(1500, 200_000), (1300, 150_003), (900, 140_000)],
                                        B=8, K=512),
    # B = 1, k = 2048: listed rows of 150,000+ candidates, pieces of 1,040 and
    # 1,060 queries (k above 1024: four-wavefront rescue select)
    "one sequence, B = 1": lambda: W.make("chunk_150000_2100_b1_k2048"),
    # a prefill from t = 0: queries below t = 16,384 take the tiled attention
    # kernel, the rest the gather with four range splits; 16 pieces of 1,248
    "prefill, tiled and range-split gather": lambda: W.make("prefill_20000"),
    # the same at B = 1, k = 2048 (tiled below t = 8,192); 11 pieces of 1,088
    "prefill, tiled and range-split gather, B = 1": lambda: W.make("prefill_12000_b1_k2048"),
}


def _aligned_ws(n):
    buf = torch.empty(max(n, 1) + 256, dtype=torch.uint8, device="cuda")
    return buf[(-buf.data_ptr()) % 256:][:max(n, 1)]


def _zero(di):
    for k in OUTS:
        di.t[k].zero_()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", list(CASES))
def test_forward_pieces_match_separate_calls(case):
    t0 = time.time()
    wl = CASES[case]()
    log("case forward pieces:", case, [(s.n_q, s.pos0) for s in wl.seqs])
    di, cfg = prepare(wl)
    seqs = lib_seqs(wl)
    fwd = sg.workspace_size(cfg, seqs, sg.OP_FORWARD)
    # the call is run in pieces: its workspace is the pieces' layout (not the
    # larger of the single-stream index and attention workspaces), with the
    # diagnostics block at its end
    single = max(sg.workspace_size(cfg, seqs, sg.OP_INDEX_TOPK), sg.workspace_size(cfg, seqs, sg.OP_SPARSE_ATTN))
    assert 0 < fwd != single
    off = sg.forward_diag_offset(cfg, seqs)
    assert off == fwd - 256
    ws = _aligned_ws(fwd)
    ws[off:off + 256].fill_(0xFF)               # the call must clear it
    _zero(di)
    run_steps(wl, di, cfg, use_forward=True, ws=ws)
    diag = sg.index_diagnostics(ws, off)
    n_rows = sum(s.n_q for s in wl.seqs)
    assert 0 <= diag["rescored_rows"] <= 4 * n_rows
    q_rows = set(r for s in wl.seqs for r in range(s.q_offset, s.q_offset + s.n_q))
    for r, g in diag["rows"]:
        assert r in q_rows and 0 <= g < 4
    got = {k: di[k].clone() for k in OUTS}
    _zero(di)
    run_steps(wl, di, cfg, use_forward=False)
    for k in OUTS:
        assert torch.equal(got[k].view(torch.uint8), di[k].view(torch.uint8)), f"{case}: {k} differs"
    log("  identical to the separate calls;", "rescored rows", diag["rescored_rows"],
        round(time.time() - t0, 1), "s")
    # the oracle on a few rows of every sequence (the separate calls' q_hat)
    ck = Checker(wl, di, cfg)
    rng = np.random.default_rng(5)
    for si, s in enumerate(wl.seqs):
        qs = stratified_rows(s, wl.block_size, wl.topk, 6, rng)
        stored, exact = ck.oracle_store(s, s.cache_len // wl.block_size)
        ck.check_seq(si, qs, store_exact=(stored, exact))
    st = ck.finish()
    log(" ", case, st, round(time.time() - t0, 1), "s")
