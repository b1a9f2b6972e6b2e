"""Device-side set-up of a synthetic workload for the GPU tests: the
library descriptors and inputs come from :mod:`synth.library`; this module
adds the tests' own helpers (progress log, poisoned store rows).  Imports
nothing from the oracle.
"""
from __future__ import annotations

import sys

import torch

from synth.library import lib_config, lib_seq, lib_seqs, prepare, setup_seqs  # noqa: F401


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def poison_store(rows):
    """Mark store rows as unwritten: NaN, or the E4M3FN NaN code (0x7F) in a
    code store, which widens to NaN."""
    rows.fill_(0x7F if rows.dtype == torch.uint8 else float("nan"))


def store_values(store):
    """The store's values as float32 (codes widened)."""
    if store.dtype == torch.uint8:
        store = store.view(torch.float8_e4m3fn)
    return store.float()
