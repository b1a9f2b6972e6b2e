"""First GPU parity checks: generator twin, the tiny prefill in full, forward
vs the three calls (also a decode call whose merge rides in the scoring
launch), determinism."""
import numpy as np
import pytest
import torch

import synth
from synth import workloads as W

from .gpu_checks import Checker, log, prepare, run_steps
from .gpu_setup import poison_store

pytestmark = pytest.mark.gpu


def test_device_generator_matches_host():
    from synth import device as dv
    n = 1 << 16
    for tid, idx0 in [(synth.TID_V, 0), (synth.TID_QIDX, 12345), (synth.TID_V, (1 << 34) + 7)]:
        t = dv.fill_bf16(torch.empty(n, dtype=torch.bfloat16, device="cuda"), 0, tid, idx0)
        host = synth.normal_bf16_bits(0, tid, np.arange(idx0, idx0 + n, dtype=np.uint64))
        assert np.array_equal(t.cpu().view(torch.int16).numpy().view(np.uint16), host)
    f = dv.fill_f32(torch.empty(n, dtype=torch.float32, device="cuda"), 3, synth.TID_W, 99, synth.C_W)
    assert np.array_equal(f.cpu().numpy(), synth.normal_f32(3, synth.TID_W, np.arange(99, 99 + n, dtype=np.uint64), synth.C_W))
    r = dv.fill_rms_rows(torch.empty((512, 192), dtype=torch.bfloat16, device="cuda"), 0, synth.TID_K, 1000)
    host = synth.rms_rows_bf16_bits(0, synth.TID_K, np.arange(1000, 1512), 192)
    assert np.array_equal(r.cpu().view(torch.int16).numpy().view(np.uint16), host)
    # correlated rows (indexer queries and weights of the correlated variant)
    c = dv.fill_corr_rows(torch.empty((300, 4, 4, 128), dtype=torch.bfloat16, device="cuda"), 0,
                          synth.TID_QIDX, 64, row0=777)
    host = synth.f32_to_bf16_bits(synth.corr_rows_f32(0, synth.TID_QIDX, np.arange(777, 1077), 2048, 64))
    assert np.array_equal(c.cpu().view(torch.int16).numpy().view(np.uint16).reshape(300, -1), host)
    cw = dv.fill_corr_rows(torch.empty((300, 4, 4), dtype=torch.float32, device="cuda"), 0, synth.TID_W, 64,
                           scale=synth.C_W)
    assert np.array_equal(cw.cpu().numpy().reshape(300, -1),
                          synth.corr_rows_f32(0, synth.TID_W, np.arange(300), 16, 64, synth.C_W))


def test_tiny_prefill_all_rows():
    wl = W.make("tiny_prefill_256")
    log("case", wl.name)
    di, cfg = prepare(wl)
    run_steps(wl, di, cfg)
    ck = Checker(wl, di, cfg)
    s = wl.seqs[0]
    stored, exact = ck.oracle_store(s, s.cache_len // wl.block_size)
    ck.check_store(s, stored, exact)
    ck.check_seq(0, np.arange(s.n_q), store_exact=(stored, exact))
    st = ck.finish()
    log(st)
    assert st["rows"] == 256


def test_forward_equals_steps_and_is_deterministic():
    wl = W.make("tiny_prefill_256")
    di, cfg = prepare(wl)
    run_steps(wl, di, cfg)
    a = {k: di[k].clone() for k in ("store", "sel", "sel_scores", "out", "lse")}
    for k in ("store", "sel", "sel_scores", "out", "lse"):
        di[k].zero_()
    run_steps(wl, di, cfg, use_forward=True)
    for k, v in a.items():
        assert torch.equal(di[k], v), k
    run_steps(wl, di, cfg, use_forward=True)
    for k, v in a.items():
        assert torch.equal(di[k], v), k


def test_decode_forward_carries_the_merge():
    """A decode call (one new token per sequence) reads none of the blocks it
    completes, so sgqa_forward merges them inside the scoring launch.  The
    store rows it completes (NaN codes before the call), the selections and
    the outputs equal those of the three separate calls bit for bit."""
    wl = W.make("decode_64_small")
    B = wl.block_size
    done = [s for s in wl.seqs if (s.pos0 + 1) % B == 0]
    log("case decode_64_small: sequences completing a block:", len(done))
    assert len(done) >= 8
    di, cfg = prepare(wl)
    run_steps(wl, di, cfg)
    keys = ("store", "sel", "sel_scores", "out", "lse")
    ref = {k: di[k].clone() for k in keys}
    for s in done:
        r = s.store_offset + s.pos0 // B
        poison_store(di["store"][r:r + 1])
    for k in keys[1:]:
        di[k].zero_()
    run_steps(wl, di, cfg, use_forward=True)
    for k, v in ref.items():
        assert torch.equal(di[k], v), k
