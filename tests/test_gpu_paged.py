"""Paged caches (page "Step-5-Preview: Sparse Reads Are Not a Compressed KV
Cache", section "Cache capacity: 4,104 reads do not mean 4,104 stored
tokens": capacity rounded to 16-token pages, page tables).

The per-token tensors of a workload (K, V, proxy keys, compression logits)
are scattered into pools of 16-position pages through a random page table
with spare pages; every pool slot that holds no position below a sequence's
capacity is NaN, so a read outside the valid rows would show.  The paged
forward must give bit-identical selections, store rows, outputs and LSE to
the contiguous forward on the same logical contents (same arithmetic, only
the row addresses differ), and sampled rows are checked against the oracle.
"""
import numpy as np
import pytest
import torch

import sparse_long_context_block_amd as sg
from synth import workloads as W

from .gpu_checks import Checker, lib_seq, lib_seqs, log, prepare, stratified_rows
from .gpu_setup import poison_store

pytestmark = pytest.mark.gpu

# chunk_150000_2100: 2,100 queries over a 152,100-token cache, which both
# forward calls run in two pieces over the second stream
@pytest.mark.parametrize("name", ["chunk_1003_997_b8_k64", "decode_small", "decode_64_small", "prefill_2000_b1_k64",
                                  "prefill_1003_b16_k8", "chunk_150000_2100"])
def test_paged_forward_matches_contiguous(name):
    wl = W.make(name)
    log("case paged", name)
    di, cfg = prepare(wl)
    seqs = lib_seqs(wl)
    sg.forward(cfg, seqs, di["proxy_k"], di["logits"], di["store"], di["q_idx"], di["w"], di["sel"],
               di["q"], di["k"], di["v"], di["out"], lse=di["lse"], sel_scores=di["sel_scores"])
    torch.cuda.synchronize()
    ref = {k: di[k].clone() for k in ("store", "sel", "sel_scores", "out", "lse")}

    pools, table, players = W.paginate(wl, di, np.random.default_rng(3))
    pseqs = [lib_seq(p) for p in players]
    # the history's store rows through the paged merge too
    pre = [sg.Seq(q_offset=0, n_q=s.pos0, pos0=0, cache_len=s.pos0, kv_offset=p.kv_offset,
                  kv_capacity=s.kv_capacity, store_offset=s.store_offset, store_capacity=s.store_capacity)
           for s, p in zip(wl.seqs, pseqs) if s.pos0 > 0]
    poison_store(di["store"])
    if pre:
        sg.compress_paged(cfg, pre, pools["proxy_k"], pools["logits"], table, di["store"])
    for k in ("sel", "sel_scores", "out", "lse"):
        di[k].zero_()
    sg.forward_paged(cfg, pseqs, pools["proxy_k"], pools["logits"], di["store"], di["q_idx"], di["w"],
                     di["sel"], di["q"], pools["k"], pools["v"], table, di["out"], lse=di["lse"],
                     sel_scores=di["sel_scores"])
    torch.cuda.synchronize()
    n_blocks = [s.cache_len // wl.block_size for s in wl.seqs]
    for s, nb in zip(wl.seqs, n_blocks):
        rows = slice(s.store_offset, s.store_offset + nb)
        assert torch.equal(di["store"][rows].view(torch.int16), ref["store"][rows].view(torch.int16))
    for k in ("sel", "sel_scores", "lse"):
        assert torch.equal(di[k], ref[k]), k
    assert torch.equal(di["out"].view(torch.int16), ref["out"].view(torch.int16))

    # oracle parity of the paged outputs on sampled rows (q_hat from the split call)
    sg.index_topk(cfg, seqs, di["q_idx"], di["w"], di["store"], di["sel"], sel_scores=di["sel_scores"],
                  q_hat_out=di["q_hat"])
    torch.cuda.synchronize()
    assert torch.equal(di["sel"], ref["sel"])
    ck = Checker(wl, di, cfg)
    rng = np.random.default_rng(0)
    for si, s in enumerate(wl.seqs[:4]):
        stored, exact = ck.oracle_store(s, s.cache_len // wl.block_size)
        ck.check_seq(si, stratified_rows(s, wl.block_size, wl.topk, 8, rng), store_exact=(stored, exact))
    log(" ", ck.finish())
