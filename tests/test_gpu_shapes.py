"""Shapes the other parity tests leave out (page "Step-5-Preview: Sparse Reads
Are Not a Compressed KV Cache": block size B, k selected blocks, sequences
batched into one call):

* block sizes 2 and 4 (every kernel is specialised per block size);
* the largest k the library takes, 3072 blocks, at B = 1 (selections and
  attention over up to 3,073 tokens per query);
* a call whose sequence list holds empty sequences (n_q = 0) among real
  ones: the outputs are bit for bit those of the call without them.
"""
import numpy as np
import pytest
import torch

import sparse_long_context_block_amd as sg
from synth import workloads as W

from .gpu_checks import Checker, lib_seqs, log, prepare, run_steps, stratified_rows

pytestmark = pytest.mark.gpu


def _parity(name, n_rows):
    wl = W.make(name)
    log("case", wl.name)
    di, cfg = prepare(wl)
    run_steps(wl, di, cfg)
    ck = Checker(wl, di, cfg)
    rng = np.random.default_rng(11)
    for si, s in enumerate(wl.seqs):
        stored, exact = ck.oracle_store(s, s.cache_len // wl.block_size)
        ck.check_store(s, stored, exact)
        ck.check_seq(si, stratified_rows(s, wl.block_size, wl.topk, n_rows, rng), store_exact=(stored, exact))
    log(" ", ck.finish())


@pytest.mark.parametrize("name", ["prefill_1500_b2_k160", "prefill_1300_b4_k96"])
def test_block_sizes_two_and_four(name):
    _parity(name, 48)


def test_largest_topk():
    _parity("prefill_3400_b1_k3072", 40)


def test_empty_sequences_change_nothing():
    wl = W.make("multi_b1_passes")
    log("case empty sequences", wl.name)
    di, cfg = prepare(wl)
    seqs = lib_seqs(wl)
    outs = {}
    for with_empty in (False, True):
        for k in ("sel", "sel_scores", "out", "lse"):      # outputs; the store keeps its history
            di[k].zero_()
        call = list(seqs)
        if with_empty:
            s0 = seqs[0]
            empty = [sg.Seq(q_offset=0, n_q=0, pos0=s0.pos0, cache_len=s0.pos0, kv_offset=s0.kv_offset,
                            kv_capacity=s0.kv_capacity, store_offset=s0.store_offset,
                            store_capacity=s0.store_capacity),
                     sg.Seq(q_offset=0, n_q=0, pos0=0, cache_len=0, kv_offset=0, kv_capacity=0,
                            store_offset=0, store_capacity=0)]
            call = [empty[0]] + call[:1] + [empty[1]] + call[1:]
        sg.forward(cfg, call, di["proxy_k"], di["logits"], di["store"], di["q_idx"], di["w"], di["sel"],
                   di["q"], di["k"], di["v"], di["out"], lse=di["lse"], sel_scores=di["sel_scores"])
        torch.cuda.synchronize()
        outs[with_empty] = {k: di[k].clone() for k in ("store", "sel", "sel_scores", "out", "lse")}
    for k in outs[False]:
        a, b = outs[False][k], outs[True][k]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), k
