"""Device-side set-up of a synthetic workload for the library: descriptors,
configuration and the inputs in HBM, with the cached history's store blocks
written by the library's own merge.  Shared by the GPU tests and bench.py;
imports nothing from the oracle.
"""
from __future__ import annotations

import sys

import torch

import sparse_long_context_block_amd as sg
from synth import workloads as W


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def lib_config(wl: W.Workload) -> sg.Config:
    return sg.config(block_size=wl.block_size, topk_blocks=wl.topk, store_q8=wl.store_q8)


def lib_seqs(wl: W.Workload):
    return [sg.Seq(q_offset=s.q_offset, n_q=s.n_q, pos0=s.pos0, cache_len=s.cache_len,
                   kv_offset=s.kv_offset, kv_capacity=s.kv_capacity,
                   store_offset=s.store_offset, store_capacity=s.store_capacity)
            for s in wl.seqs]


def setup_seqs(wl: W.Workload):
    """Descriptors that write the store blocks of the cached history (before
    the measured step's new tokens; for a decode loop, before its first step)."""
    seqs = wl.step_seqs(0) if wl.loop_steps else wl.seqs
    return [sg.Seq(q_offset=0, n_q=s.pos0, pos0=0, cache_len=s.pos0, kv_offset=s.kv_offset,
                   kv_capacity=s.kv_capacity, store_offset=s.store_offset,
                   store_capacity=s.store_capacity)
            for s in seqs if s.pos0 > 0]


def lib_seq(s: W.SeqLayout) -> sg.Seq:
    return sg.Seq(q_offset=s.q_offset, n_q=s.n_q, pos0=s.pos0, cache_len=s.cache_len,
                  kv_offset=s.kv_offset, kv_capacity=s.kv_capacity,
                  store_offset=s.store_offset, store_capacity=s.store_capacity)


def poison_store(rows):
    """Mark store rows as unwritten: NaN, or the E4M3FN NaN code (0x7F) in a
    code store, which widens to NaN."""
    rows.fill_(0x7F if rows.dtype == torch.uint8 else float("nan"))


def store_values(store):
    """The store's values as float32 (codes widened)."""
    if store.dtype == torch.uint8:
        store = store.view(torch.float8_e4m3fn)
    return store.float()


def prepare(wl: W.Workload):
    di = W.device_inputs(wl)
    cfg = lib_config(wl)
    pre = setup_seqs(wl)
    if pre:
        sg.compress(cfg, pre, di["proxy_k"], di["logits"], di["store"])
    torch.cuda.synchronize()
    return di, cfg
