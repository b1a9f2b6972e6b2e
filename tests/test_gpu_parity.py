"""GPU parity against the oracle across block sizes, top-k sizes, ragged
tails, chunked prefill on an existing cache and the split (decode) paths."""
import numpy as np
import pytest
import torch

from synth import workloads as W

from .gpu_checks import Checker, log, prepare, run_steps

pytestmark = pytest.mark.gpu


def _run_and_check(name, n_rows=64, store_q8=2, check_all_store=True, seed_rows=0):
    wl = W.make(name, store_q8=store_q8)
    log("case", wl.name, "q8" if store_q8 else "bf16")
    di, cfg = prepare(wl)
    run_steps(wl, di, cfg)
    ck = Checker(wl, di, cfg)
    rng = np.random.default_rng(seed_rows)
    from .gpu_checks import stratified_rows
    for si, s in enumerate(wl.seqs):
        qs = stratified_rows(s, wl.block_size, wl.topk, n_rows, rng)
        b_need = max((s.cache_len - 1) // wl.block_size, s.cache_len // wl.block_size)
        stored, exact = ck.oracle_store(s, s.cache_len // wl.block_size)
        if check_all_store:
            ck.check_store(s, stored, exact)
        ck.check_seq(si, qs, store_exact=(stored, exact))
    st = ck.finish()
    log(st)
    return st


def test_topk_compaction_heavy():
    # K=16 over up to 499 candidates: the streaming buffer compacts many times
    _run_and_check("prefill_4000_b8_k16", n_rows=96)


def test_prefill_8k_stratified():
    _run_and_check("prefill_8k", n_rows=64)


def test_block_size_one():
    _run_and_check("prefill_2000_b1_k64", n_rows=64)


def test_block_size_sixteen_ragged():
    _run_and_check("prefill_1003_b16_k8", n_rows=64)


def test_bf16_store():
    _run_and_check("prefill_1000_b8_k32", n_rows=64, store_q8=False)


def test_chunk_on_existing_cache_unaligned():
    # pos0 = 1003 is inside block 125: the block mixes earlier and new tokens
    _run_and_check("chunk_1003_997_b8_k64", n_rows=64)


def test_tiled_index_passes_over_ragged_sequences():
    # 2533 queries at B = 1 over histories up to 180K tokens: the tiled
    # indexer runs in two launches of at most 1472 queries (one pass over
    # its 4 GiB key workspace each) that cut through the sequences
    _run_and_check("multi_b1_passes", n_rows=24, check_all_store=False)


def test_tiled_index_rows_out_of_call_order():
    # the same sequences with 1000 unused rows between them, listed in the
    # call in another order than their rows: key-workspace rows follow the
    # call order, output rows follow q_offset
    _run_and_check("multi_b1_shuffled", n_rows=24, check_all_store=False)


@pytest.mark.parametrize("name", ["chunk_40000_1024_b1_k64", "chunk_65536_1024_b1_k2048",
                                  "chunk_300000_1040_b8_k512"])
def test_listed_long_rows(name):
    # tiled calls whose tiles start at 32768+ candidate blocks: their rows
    # select from the candidates at or above a sampled threshold (the last
    # case with a ragged 16-query tile)
    _run_and_check(name, n_rows=24, check_all_store=False)


def test_decode_one_workgroup_per_cu():
    # 64 sequences x 4 groups = 256 (sequence, group) units, enough to fill
    # the CUs, so the gather runs unsplit (no partials, no merge kernel)
    st = _run_and_check("decode_64_small", n_rows=1, check_all_store=False)
    assert st["rows"] >= 64


def test_decode_split_paths():
    st = _run_and_check("decode_small", n_rows=1, check_all_store=True)
    assert st["rows"] == 8
