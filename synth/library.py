"""Library descriptors and device set-up of a synthetic workload.

Turns a :class:`synth.workloads.Workload` into the library's configuration
and per-sequence descriptors, and puts its inputs in HBM with the store blocks
of the cached history written by the library's own merge.  Shared by the GPU
tests and ``bench.py``.  It holds none of the method's arithmetic (the merge
it triggers runs in the library) and the CPU oracle never imports it.
"""
from __future__ import annotations

import torch

import sparse_long_context_block_amd as sg

from . import workloads as W


def lib_config(wl: W.Workload) -> sg.Config:
    return sg.config(block_size=wl.block_size, topk_blocks=wl.topk, store_q8=wl.store_q8)


def lib_seq(s: W.SeqLayout) -> sg.Seq:
    return sg.Seq(q_offset=s.q_offset, n_q=s.n_q, pos0=s.pos0, cache_len=s.cache_len,
                  kv_offset=s.kv_offset, kv_capacity=s.kv_capacity,
                  store_offset=s.store_offset, store_capacity=s.store_capacity)


def lib_seqs(wl: W.Workload, seqs=None):
    return [lib_seq(s) for s in (wl.seqs if seqs is None else seqs)]


def setup_seqs(wl: W.Workload):
    """Descriptors that write the store blocks of the cached history (before
    the measured step's new tokens; for a loop of calls, before its first)."""
    seqs = wl.step_seqs(0) if wl.loop_steps else wl.seqs
    return [sg.Seq(q_offset=0, n_q=s.pos0, pos0=0, cache_len=s.pos0, kv_offset=s.kv_offset,
                   kv_capacity=s.kv_capacity, store_offset=s.store_offset,
                   store_capacity=s.store_capacity)
            for s in seqs if s.pos0 > 0]


def prepare(wl: W.Workload):
    """Device inputs of `wl` and its library config; the cached history's
    store blocks are merged by the library before returning."""
    di = W.device_inputs(wl)
    cfg = lib_config(wl)
    pre = setup_seqs(wl)
    if pre:
        sg.compress(cfg, pre, di["proxy_k"], di["logits"], di["store"])
    torch.cuda.synchronize()
    return di, cfg


__all__ = ["lib_config", "lib_seq", "lib_seqs", "setup_seqs", "prepare"]
