"""bench.py's host-side rules, without a GPU: it measures one GPU only and
refuses more before touching one, refuses contradictory store options, and
sizes one workspace for the timed forward calls and the separate stage calls
that follow them."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_store_options_exclude_each_other():
    r = _run("--store-bf16", "--store-e4m3-bf16")
    assert r.returncode == 2
    assert "exclude each other" in r.stderr and r.stdout == ""


def test_workspace_covers_the_forward_and_the_stage_calls():
    sg = pytest.importorskip("sparse_long_context_block_amd")
    try:
        sg.lib()
    except Exception as e:          # the library is built by __graft_entry__.build()
        pytest.skip(f"libsgqa.so not loadable here: {e}")
    sys.path.insert(0, ROOT)
    import bench
    from synth import workloads as W
    from synth.library import lib_config, lib_seqs
    for name in ("chunk_1m", "prefill_64k", "decode_64x256k"):
        wl = W.make(name)
        cfg, seqs = lib_config(wl), lib_seqs(wl)
        sizes = [sg.workspace_size(cfg, seqs, op) for op in (sg.OP_FORWARD, sg.OP_INDEX_TOPK, sg.OP_SPARSE_ATTN)]
        assert bench._ws_need(sg, cfg, seqs) == max(sizes) > 0
    # the 1M chunk's forward call runs in pieces: it needs less than its
    # index step alone, so the separate index call sizes the workspace
    wl = W.make("chunk_1m")
    cfg, seqs = lib_config(wl), lib_seqs(wl)
    assert sg.workspace_size(cfg, seqs, sg.OP_FORWARD) < sg.workspace_size(cfg, seqs, sg.OP_INDEX_TOPK)
