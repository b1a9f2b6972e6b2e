"""sgqa_forward captured into a HIP graph (torch.cuda.CUDAGraph over the
caller's stream) and replayed: on a call that runs in pieces over the
library's second stream (the fork and join events pull that stream into the
capture), on a decode-sized call on one stream, and on the same decode call
through sgqa_forward_noalloc (its static scratch).  Every replay, with eager
work and synchronisations between them, must equal the eager call bit for
bit (sel, sel_scores, out, lse)."""
import time

import pytest
import torch

import sparse_long_context_block_amd as sg
from synth import workloads as W

from .gpu_checks import lib_seqs, log, prepare

pytestmark = pytest.mark.gpu

OUTS = ("sel", "sel_scores", "out", "lse")

CASES = {
    # 4,600 queries from t = 262,144: four pieces, two streams
    "pieces": ("chunk_262144_4600", False),
    # 8 sequences of one query over 8K-40K tokens: one stream
    "decode": ("decode_small", False),
    "decode, static scratch": ("decode_small", True),
}


def _aligned_ws(n):
    buf = torch.empty(max(n, 1) + 256, dtype=torch.uint8, device="cuda")
    return buf[(-buf.data_ptr()) % 256:][:max(n, 1)]


def _poison(di):
    for k in OUTS:
        t = di.t[k]
        if t.dtype == torch.int32:
            t.fill_(-7)
        else:
            t.view(torch.uint8).fill_(0xFF)


def _forward(di, cfg, seqs, ws, noalloc):
    args = (cfg, seqs, di["proxy_k"], di["logits"], di["store"], di["q_idx"], di["w"], di["sel"],
            di["q"], di["k"], di["v"], di["out"])
    if noalloc:
        sg.forward_noalloc(*args, lse=di["lse"], sel_scores=di["sel_scores"])
    else:
        sg.forward(*args, lse=di["lse"], sel_scores=di["sel_scores"], ws=ws)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", list(CASES))
def test_forward_graph_replays_match_eager(case):
    t0 = time.time()
    name, noalloc = CASES[case]
    wl = W.make(name)
    log("case forward graph:", case, [(s.n_q, s.pos0) for s in wl.seqs])
    di, cfg = prepare(wl)
    seqs = lib_seqs(wl)
    ws = _aligned_ws(sg.workspace_size(cfg, seqs, sg.OP_FORWARD))
    # eager call first (on poisoned outputs, as every replay): it also
    # creates the library's second stream, outside the capture
    _poison(di)
    call = lambda: _forward(di, cfg, seqs, ws, noalloc)
    call()
    torch.cuda.synchronize()
    ref = {k: di[k].clone() for k in OUTS}
    _poison(di)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    log("  captured", round(time.time() - t0, 1), "s")
    scratch = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for rep in range(3):
        _poison(di)
        scratch.normal_()
        torch.cuda.synchronize()
        g.replay()
        scratch.mul_(2.0)                    # eager work behind the replay
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(ref[k].view(torch.uint8), di[k].view(torch.uint8)), \
                f"{case}: replay {rep}: {k} differs from the eager call"
        log("  replay", rep, "identical", round(time.time() - t0, 1), "s")
    del g
    torch.cuda.synchronize()
