"""A prefill split into consecutive calls, each one sgqa_forward over the
cache the calls before it built (page "Step-5-Preview: Sparse Reads Are Not
a Compressed KV Cache": the store grows block by block as tokens arrive, and
a chunk's queries select among every completed block before their own; the
long-context comparison of B = 8 against B = 1 on the second page runs a
1M-token prefill this way).

Nothing is compressed before the first call: every store block is written
by the compression step of the call whose chunk holds its tokens, and store
rows are NaN until then, so a call that read a block not yet built would
turn its outputs NaN or change its selections.  After the chain every
call's sampled rows and the whole store are checked against the oracle."""
import numpy as np
import pytest
import torch

import sparse_long_context_block_amd as sg
from synth import workloads as W

from .gpu_checks import Checker, lib_config, lib_seq, log, stratified_rows
from .gpu_setup import poison_store, store_values

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["chained_small", "chained_small_b1"])
def test_chained_prefill_builds_its_own_store(name):
    wl = W.make(name)
    B, K, n_calls = wl.block_size, wl.topk, wl.loop_steps
    log("case", name, n_calls, "calls of", wl.seqs[0].n_q, "B", B, "K", K)
    di = W.device_inputs(wl)
    cfg = lib_config(wl)
    poison_store(di["store"])
    torch.cuda.synchronize()
    for c in range(n_calls):
        sg.forward(cfg, [lib_seq(s) for s in wl.step_seqs(c)], di["proxy_k"], di["logits"],
                   di["store"], di["q_idx"], di["w"], di["sel"], di["q"], di["k"], di["v"],
                   di["out"], lse=di["lse"], sel_scores=di["sel_scores"])
    torch.cuda.synchronize()
    assert torch.isfinite(di["out"].float()).all() and torch.isfinite(di["lse"]).all()
    assert torch.isfinite(store_values(di["store"])).all()

    # the indexer once more per call, only to expose q_hat (the store is
    # complete now, but a call only ever reads blocks before its queries)
    sel_fwd, ssc_fwd = di["sel"].clone(), di["sel_scores"].clone()
    for c in range(n_calls):
        sg.index_topk(cfg, [lib_seq(s) for s in wl.step_seqs(c)], di["q_idx"], di["w"],
                      di["store"], di["sel"], sel_scores=di["sel_scores"], q_hat_out=di["q_hat"])
    torch.cuda.synchronize()
    assert torch.equal(sel_fwd, di["sel"]) and torch.equal(ssc_fwd, di["sel_scores"])

    ck = Checker(wl, di, cfg)
    last = wl.seqs[-1]
    n_blocks = last.cache_len // B
    stored, exact = ck.oracle_store(last, n_blocks)
    ck.check_store(last, stored, exact)
    rng = np.random.default_rng(11)
    for c in range(n_calls):
        qs = stratified_rows(wl.seqs[c], B, K, 12, rng)
        ck.check_seq(c, qs, store_exact=(stored, exact))
    stats = ck.finish()
    log(" ", stats)
    assert stats["rows"] == 12 * n_calls
    assert stats["store"]["n"] == n_blocks * 128
