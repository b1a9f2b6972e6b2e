"""Multi-step decode: eight sequences decoded for twelve consecutive tokens,
each step one sgqa_forward after the caller appends the new token's K/V,
proxy key and compression logits to its caches (page "Step-5-Preview: Sparse
Reads Are Not a Compressed KV Cache", section "Eight tokens become one search
key, coordinate by coordinate": the summary of a block appears when its
eighth token arrives; the tokens of the incomplete block wait in the
caller's buffers).

Every cache row from the first new token on, and every store row not yet
built, is NaN until the loop appends or compresses it, so a kernel that read
past cache_len or an unbuilt block would turn its outputs NaN or change its
selections.  After the loop every (sequence, step) query and the store
blocks compressed during the loop are checked against the oracle."""
import numpy as np
import pytest
import torch

import sparse_long_context_block_amd as sg
from synth import workloads as W

from .gpu_checks import Checker, lib_config, log
from .gpu_setup import poison_store

pytestmark = pytest.mark.gpu

_CACHE_TENSORS = ("k", "v", "proxy_k", "logits")


def _lib_seq(s: W.SeqLayout) -> sg.Seq:
    return sg.Seq(q_offset=s.q_offset, n_q=s.n_q, pos0=s.pos0, cache_len=s.cache_len,
                  kv_offset=s.kv_offset, kv_capacity=s.kv_capacity,
                  store_offset=s.store_offset, store_capacity=s.store_capacity)


@pytest.mark.timeout(600)
def test_decode_loop_appends_and_compresses():
    wl = W.make("decode_loop_small")
    n, S, B = wl.loop_seqs, wl.loop_steps, wl.block_size
    log("case", wl.name, n, "sequences x", S, "steps")
    di = W.device_inputs(wl)
    cfg = lib_config(wl)
    first = wl.step_seqs(0)
    # the history before the loop: blocks entirely inside [0, L_i - 1)
    pre = [sg.Seq(q_offset=0, n_q=s.pos0, pos0=0, cache_len=s.pos0, kv_offset=s.kv_offset,
                  kv_capacity=s.kv_capacity, store_offset=s.store_offset,
                  store_capacity=s.store_capacity) for s in first]
    sg.compress(cfg, pre, di["proxy_k"], di["logits"], di["store"])
    # keep the rows the loop will append, then poison every row from the
    # first new token on and every store row not built yet
    saved = []
    for s in first:
        app = torch.arange(s.kv_offset + s.pos0, s.kv_offset + s.pos0 + S, device="cuda")
        saved.append({name: di[name][app].clone() for name in _CACHE_TENSORS})
        tail = slice(s.kv_offset + s.pos0, s.kv_offset + s.kv_capacity)
        for name in _CACHE_TENSORS:
            di[name][tail] = float("nan")
        poison_store(di["store"][s.store_offset + s.pos0 // B:s.store_offset + s.store_capacity])
    torch.cuda.synchronize()

    completed = 0
    for st in range(S):
        seqs = wl.step_seqs(st)
        for i, s in enumerate(seqs):
            row = s.kv_offset + s.pos0                       # the appended token
            for name in _CACHE_TENSORS:
                di[name][row] = saved[i][name][st]
            completed += int((s.pos0 + 1) % B == 0)
        sg.forward(cfg, [_lib_seq(s) for s in seqs], di["proxy_k"], di["logits"], di["store"],
                   di["q_idx"], di["w"], di["sel"], di["q"], di["k"], di["v"], di["out"],
                   lse=di["lse"], sel_scores=di["sel_scores"])
    torch.cuda.synchronize()
    log("  blocks completed during the loop:", completed)
    assert completed >= n                                   # 12 steps cross a boundary
    assert torch.isfinite(di["out"].float()).all() and torch.isfinite(di["lse"]).all()

    # the indexer once more per step, only to expose q_hat (the blocks a step
    # reads were complete at that step, so the selections are the same)
    sel_fwd, ssc_fwd = di["sel"].clone(), di["sel_scores"].clone()
    for st in range(S):
        sg.index_topk(cfg, [_lib_seq(s) for s in wl.step_seqs(st)], di["q_idx"], di["w"],
                      di["store"], di["sel"], sel_scores=di["sel_scores"], q_hat_out=di["q_hat"])
    torch.cuda.synchronize()
    assert torch.equal(sel_fwd, di["sel"]) and torch.equal(ssc_fwd, di["sel_scores"])

    ck = Checker(wl, di, cfg)
    last = wl.step_seqs(S - 1)
    for i in range(n):
        s_last = last[i]
        n_blocks = s_last.cache_len // B
        stored, exact = ck.oracle_store(s_last, n_blocks)
        first_new = first[i].pos0 // B
        ck.check_store(s_last, stored, exact, np.arange(first_new, n_blocks))   # built by the loop
        for st in range(S):
            ck.check_seq(st * n + i, np.array([0]), store_exact=(stored, exact))
    stats = ck.finish()
    log(" ", stats)
    assert stats["rows"] == n * S
