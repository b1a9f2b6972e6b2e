"""Full-size workloads through sgqa_forward (the launch configuration the
benchmark times), checked against the oracle on sampled rows: the 8K prefill,
the 64K prefill at B=8 and its B=1 ablation, 64-sequence decode at up to 256K
tokens, and the 8K-query chunk over a 1M-token cache."""
import time

import numpy as np
import pytest
import torch

from synth import workloads as W

from .gpu_checks import Checker, log, prepare, run_steps, stratified_rows

pytestmark = pytest.mark.gpu


def _forward_then_index(wl, di, cfg):
    # the timed path: one sgqa_forward; then the split index call once more
    # only to expose q_hat for the check (same store, same selections)
    run_steps(wl, di, cfg, use_forward=True)
    out = di["out"].clone()
    sel = di["sel"].clone()
    run_steps(wl, di, cfg, use_forward=False)
    assert torch.equal(out, di["out"]) and torch.equal(sel, di["sel"])


def _check(name, rows_per_seq, seqs=None, store_blocks=None, seed=3):
    t0 = time.time()
    wl = W.make(name)
    log("case", name, "preparing")
    di, cfg = prepare(wl)
    _forward_then_index(wl, di, cfg)
    log("  gpu done", round(time.time() - t0, 1), "s")
    ck = Checker(wl, di, cfg)
    rng = np.random.default_rng(seed)
    seq_ids = range(len(wl.seqs)) if seqs is None else seqs
    for si in seq_ids:
        s = wl.seqs[si]
        qs = stratified_rows(s, wl.block_size, wl.topk, rows_per_seq, rng)
        t_max = s.pos0 + int(qs.max())
        stored, exact = ck.oracle_store(s, max(t_max // wl.block_size, s.cache_len // wl.block_size))
        n_st = stored.shape[0]
        blocks = np.arange(n_st) if store_blocks is None or n_st <= store_blocks else \
            np.unique(np.concatenate([rng.choice(n_st, store_blocks, replace=False),
                                      np.arange(max(0, n_st - 64), n_st)]))
        ck.check_store(s, stored, exact, blocks)
        ck.check_seq(si, qs, store_exact=(stored, exact))
    st = ck.finish()
    log(" ", name, st, round(time.time() - t0, 1), "s")
    return st


@pytest.mark.timeout(900)
def test_prefill_8k_bench_configuration():
    _check("prefill_8k", 48)


@pytest.mark.timeout(900)
def test_prefill_64k():
    st = _check("prefill_64k", 40, store_blocks=2048)
    assert st["sel_rows"] == 160


@pytest.mark.timeout(900)
def test_prefill_64k_block_size_one():
    _check("prefill_64k_b1", 24, store_blocks=4096)


@pytest.mark.timeout(900)
def test_decode_64_sequences():
    st = _check("decode_64x256k", 1, store_blocks=1024)
    assert st["rows"] == 64


@pytest.mark.timeout(900)
def test_chunk_over_1m_cache():
    _check("chunk_1m", 24, store_blocks=4096)
