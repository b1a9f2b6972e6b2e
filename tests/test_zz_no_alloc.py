"""sgqa_forward_noalloc (the static-scratch forward for callers that cannot
allocate) against sgqa_forward with a caller workspace: the same kernels and
launch shapes, so the outputs must be bit-identical.  Two calls in a row, the
second smaller than the first (the scratch keeps the first call's contents),
then the first again."""
import numpy as np
import pytest
import torch

import sparse_long_context_block_amd as sg
from synth import workloads as W

from .gpu_setup import lib_seqs, log, prepare

pytestmark = pytest.mark.gpu

OUTS = ("sel", "sel_scores", "out", "lse", "store")


def _zero_outputs(di):
    for k in ("sel", "sel_scores", "out", "lse"):
        di.t[k].zero_()


def _run(di, cfg, seqs, noalloc):
    args = (cfg, seqs, di["proxy_k"], di["logits"], di["store"], di["q_idx"], di["w"], di["sel"],
            di["q"], di["k"], di["v"], di["out"])
    if noalloc:
        sg.forward_noalloc(*args, lse=di["lse"], sel_scores=di["sel_scores"])
    else:
        sg.forward(*args, lse=di["lse"], sel_scores=di["sel_scores"])
    torch.cuda.synchronize()
    return {k: di[k].clone() for k in OUTS}


def _compare(a, b, what):
    for k in OUTS:
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), f"{what}: {k} differs"


def test_noalloc_forward_matches_forward():
    wl = W.make("decode_small")
    log("case noalloc decode_small (8 sequences), then 3 of them, then all 8 again")
    di, cfg = prepare(wl)
    full = lib_seqs(wl)
    small = full[:3]
    need = sg.workspace_size(cfg, full, sg.OP_FORWARD)
    assert 0 < need <= 64 << 20
    for seqs, what in ((full, "8 sequences"), (small, "3 sequences"), (full, "8 sequences again")):
        _zero_outputs(di)
        ref = _run(di, cfg, seqs, noalloc=False)
        _zero_outputs(di)
        got = _run(di, cfg, seqs, noalloc=True)
        _compare(ref, got, what)
        rows = np.concatenate([np.arange(s.q_offset, s.q_offset + s.n_q) for s in seqs])
        assert torch.isfinite(got["out"][rows].float()).all()
        log("  identical:", what, "workspace", sg.workspace_size(cfg, seqs, sg.OP_FORWARD), "bytes")


def test_noalloc_rejects_calls_beyond_the_scratch():
    wl = W.make("prefill_8k")
    cfg = sg.config()
    seqs = lib_seqs(wl)
    assert sg.workspace_size(cfg, seqs, sg.OP_FORWARD) > 64 << 20
    di, cfg = prepare(wl)
    with pytest.raises(sg.SgqaError, match="static"):
        _run(di, cfg, seqs, noalloc=True)
