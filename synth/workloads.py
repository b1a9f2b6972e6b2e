"""The synthetic workloads: shapes, sequence layout and seeded contents.

Input infrastructure shared by the tests, the smoke check and the benchmark.
It holds none of the method's arithmetic: it only lays sequences out in the
caches and fills tensors from the counter-based generator, on the device
(:mod:`synth.device`) or, for any slice the CPU oracle needs, on the host.

Workloads (one attention layer each, 64 heads / 4 KV groups / head_dim 192,
indexer 4 heads x 128 per group with a 32-dim rotary span, seed 0):

=====================  ==========================================  ======  =====
name                   queries / cache                             B       K
=====================  ==========================================  ======  =====
tiny_prefill_256       prefill N=256                               8       16
prefill_8k             prefill N=8,192                             8       512
prefill_64k            prefill N=65,536                            8       512
prefill_64k_b1         prefill N=65,536 (ablation)                 1       2,048
decode_64x256k         64 sequences x 1 new token, lengths U[131072,262144],
                       262,144-token allocation each               8       512
decode_loop_64x256k    the same 64 sequences decoded for 80 consecutive
                       tokens (lengths U[131072,262064])           8       512
chunk_1m               8,192 queries at 1,040,384..1,048,575 over a
                       1,048,576-token cache                       8       512
prefill_1m_chained     a 1,048,576-token prefill as 128 calls of
                       8,192 queries, each on the cache and store
                       the calls before it built                   8       512
prefill_1m_chained_b1  the same                                    1       2,048
=====================  ==========================================  ======  =====

Distributions: main Q and K bf16 unit normal then RMS-normalised per
(token, head / group) row; V, indexer queries and proxy keys bf16 unit
normal; compression logits fp32 unit normal; indexer weights fp32 normal with
standard deviation 1/sqrt(512).  All i.i.d.; the draws are Irwin-Hall(4)
(bounded tails, see :mod:`synth`).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np

from . import (C_W, TID_K, TID_LOGITS, TID_PROXY, TID_Q, TID_QIDX, TID_V, TID_W, corr_rows_f32,
               f32_to_bf16_bits, normal_bf16_bits, normal_f32, rms_rows_bf16_bits, seq_lengths)

H, G, D, HI, DI = 64, 4, 192, 4, 128


@dataclass
class SeqLayout:
    q_offset: int
    n_q: int
    pos0: int
    kv_offset: int
    kv_capacity: int
    store_offset: int
    store_capacity: int

    @property
    def cache_len(self) -> int:
        return self.pos0 + self.n_q


@dataclass
class Workload:
    name: str
    block_size: int
    topk: int
    seqs: List[SeqLayout]
    # store rows written before the measured step: (pos0=0, n_q=pos0) per seq
    prebuilt: bool = False
    # proxy-key store: 2 E4M3 codes (uint8), 1 the same values held in
    # bf16, 0 bf16 values
    store_q8: int = 2
    seed: int = 0
    notes: str = ""
    # loops of calls (decode loops, chained prefills): seqs holds
    # loop_steps x loop_seqs entries, step-major; entry (s, i) is sequence
    # i's part of call s
    loop_steps: int = 0
    loop_seqs: int = 0
    # > 0: the indexer queries and weights of neighbouring query rows are
    # correlated (a moving sum of this many draws along the row index, see
    # synth item 6), so neighbouring queries select overlapping blocks
    corr_window: int = 0

    def step_seqs(self, s: int) -> List[SeqLayout]:
        return self.seqs[s * self.loop_seqs:(s + 1) * self.loop_seqs]

    @property
    def n_q_total(self) -> int:
        return sum(s.n_q for s in self.seqs)

    @property
    def q_rows(self) -> int:
        return max(s.q_offset + s.n_q for s in self.seqs)

    @property
    def kv_rows(self) -> int:
        return max(s.kv_offset + s.kv_capacity for s in self.seqs)

    @property
    def store_rows(self) -> int:
        return max(s.store_offset + s.store_capacity for s in self.seqs)


def _prefill(name, n, B, K, pos0=0, **kw) -> Workload:
    T = pos0 + n
    return Workload(name, B, K, [SeqLayout(0, n, pos0, 0, T, 0, T // B)], prebuilt=pos0 > 0, **kw)


def _decode(name, n_seqs=64, lo=131072, hi=262144, cap=262144, B=8, K=512, seed=0) -> Workload:
    L = seq_lengths(seed, n_seqs, lo, hi)
    seqs = [SeqLayout(i, 1, int(L[i]) - 1, i * cap, cap, i * (cap // B), cap // B)
            for i in range(n_seqs)]
    return Workload(name, B, K, seqs, prebuilt=True, seed=seed)


def _decode_loop(name, n_seqs, lo, hi, cap, steps, B=8, K=512, seed=0) -> Workload:
    """n_seqs sequences decoded for `steps` consecutive tokens: sequence i
    starts with a cache of L_i - 1 tokens (L_i uniform in [lo, hi]) and its
    step s appends position L_i - 1 + s; query rows i * steps + s."""
    assert hi + steps <= cap
    L = seq_lengths(seed, n_seqs, lo, hi)
    seqs = [SeqLayout(i * steps + st, 1, int(L[i]) - 1 + st, i * cap, cap, i * (cap // B), cap // B)
            for st in range(steps) for i in range(n_seqs)]
    w = Workload(name, B, K, seqs, prebuilt=True, seed=seed)
    w.loop_steps, w.loop_seqs = steps, n_seqs
    return w


def _chained(name, n_chunks, chunk, B, K) -> Workload:
    """One sequence prefilled in n_chunks consecutive calls of `chunk`
    queries: call c covers positions c*chunk .. (c+1)*chunk - 1 and finds
    the store blocks of everything before it written by the earlier calls'
    compression step; query rows = positions."""
    T = n_chunks * chunk
    seqs = [SeqLayout(c * chunk, chunk, c * chunk, 0, T, 0, T // B) for c in range(n_chunks)]
    w = Workload(name, B, K, seqs)
    w.loop_steps, w.loop_seqs = n_chunks, 1
    return w


def _multi(name, parts, B, K, row_gap=0, order=None) -> Workload:
    """Sequences (n_q, pos0) back to back in caches and store; their query
    rows `row_gap` rows apart; listed in the call in `order` (default: as
    given)."""
    seqs, row, kv, st = [], 0, 0, 0
    for n, pos0 in parts:
        T = pos0 + n
        seqs.append(SeqLayout(row, n, pos0, kv, T, st, T // B))
        row, kv, st = row + n + row_gap, kv + T, st + T // B
    if order is not None:
        seqs = [seqs[j] for j in order]
    return Workload(name, B, K, seqs, prebuilt=True)


def make(name: str, seed: int = 0, store_q8: int = 2) -> Workload:
    if "_corr" in name:
        # <workload>_corr<W>: the same workload with correlated indexer
        # queries and weights along the query rows (a variant outside the
        # benchmark configurations)
        base, _, win = name.rpartition("_corr")
        w = make(base, seed=seed, store_q8=store_q8)
        w.name = name
        w.corr_window = int(win)
        return w
    if name == "tiny_prefill_256":
        w = _prefill(name, 256, 8, 16)
    elif name == "prefill_8k":
        w = _prefill(name, 8192, 8, 512)
    elif name == "prefill_64k":
        w = _prefill(name, 65536, 8, 512)
    elif name == "prefill_64k_b1":
        w = _prefill(name, 65536, 1, 2048)
    elif name == "decode_64x256k":
        w = _decode(name, seed=seed)
    elif name == "chunk_1m":
        w = _prefill(name, 8192, 8, 512, pos0=1_040_384)
    elif name == "multi_b1_passes":              # ragged sequences, tiled index in passes (tests)
        w = _multi(name, [(700, 180_000), (1500, 0), (333, 120_003)], B=1, K=64)
    elif name == "multi_b1_shuffled":            # the same, rows apart and out of call order (tests)
        w = _multi(name, [(700, 180_000), (1500, 0), (333, 120_003)], B=1, K=64,
                   row_gap=1000, order=[2, 0, 1])
    elif name == "decode_loop_small":            # 8 sequences x 12 decode steps (tests)
        w = _decode_loop(name, 8, 8192, 40960 - 16, 40960, 12, seed=seed)
    elif name == "decode_loop_64x256k":          # 64 sequences x 80 decode steps
        w = _decode_loop(name, 64, 131072, 262144 - 80, 262144, 80, seed=seed)
    elif name == "prefill_1m_chained":           # 1M-token prefill, 128 calls of 8192
        w = _chained(name, 128, 8192, 8, 512)
    elif name == "prefill_1m_chained_b1":        # the same at B = 1, k = 2048 blocks
        w = _chained(name, 128, 8192, 1, 2048)
    elif name == "chained_small":                # 6 calls of 1024 (tests)
        w = _chained(name, 6, 1024, 8, 32)
    elif name == "chained_small_b1":             # 4 calls of 1024 at B = 1 (tests)
        w = _chained(name, 4, 1024, 1, 256)
    elif name == "decode_small":                 # 8 sequences, split paths (tests)
        w = _decode(name, n_seqs=8, lo=8192, hi=40000, cap=40960, seed=seed)
    elif name == "decode_64_small":              # 64 sequences: one attention workgroup per CU (tests)
        w = _decode(name, n_seqs=64, lo=4100, hi=12000, cap=12288, seed=seed)
    elif name.startswith("chunk_"):              # chunk_<pos0>_<n>[_b<B>_k<K>] (tests)
        parts = name.split("_")
        pos0, n = int(parts[1]), int(parts[2])
        B = int(parts[3][1:]) if len(parts) > 3 else 8
        K = int(parts[4][1:]) if len(parts) > 4 else 512
        w = _prefill(name, n, B, K, pos0=pos0)
    elif name.startswith("prefill_"):          # prefill_<n>[_b<B>_k<K>] for tests
        parts = name.split("_")
        n = int(parts[1])
        B = int(parts[2][1:]) if len(parts) > 2 else 8
        K = int(parts[3][1:]) if len(parts) > 3 else 512
        w = _prefill(name, n, B, K)
    else:
        raise KeyError(name)
    w.seed = seed
    w.store_q8 = int(store_q8)
    return w


NAMES = ["tiny_prefill_256", "prefill_8k", "prefill_64k", "prefill_64k_b1", "decode_64x256k",
         "chunk_1m"]


# ---------------------------------------------------------------------------
# device tensors
# ---------------------------------------------------------------------------

@dataclass
class DeviceInputs:
    wl: Workload
    t: Dict[str, "object"] = field(default_factory=dict)

    def __getitem__(self, k):
        return self.t[k]


def device_inputs(wl: Workload, device="cuda") -> DeviceInputs:
    """Allocate and fill every tensor of the workload on the device; outputs
    (store, sel, sel_scores, q_hat, out, lse) are allocated and zero-filled."""
    import torch

    from . import device as dv

    Nq, R, S = wl.q_rows, wl.kv_rows, wl.store_rows
    bf, f32 = torch.bfloat16, torch.float32
    t = {}
    t["q"] = dv.fill_rms_rows(torch.empty((Nq, H, D), dtype=bf, device=device), wl.seed, TID_Q)
    t["k"] = dv.fill_rms_rows(torch.empty((R, G, D), dtype=bf, device=device), wl.seed, TID_K)
    t["v"] = dv.fill_bf16(torch.empty((R, G, D), dtype=bf, device=device), wl.seed, TID_V)
    if wl.corr_window:
        t["q_idx"] = dv.fill_corr_rows(torch.empty((Nq, G, HI, DI), dtype=bf, device=device), wl.seed,
                                       TID_QIDX, wl.corr_window)
        t["w"] = dv.fill_corr_rows(torch.empty((Nq, G, HI), dtype=f32, device=device), wl.seed, TID_W,
                                   wl.corr_window, scale=C_W)
    else:
        t["q_idx"] = dv.fill_bf16(torch.empty((Nq, G, HI, DI), dtype=bf, device=device), wl.seed,
                                  TID_QIDX)
        t["w"] = dv.fill_f32(torch.empty((Nq, G, HI), dtype=f32, device=device), wl.seed, TID_W,
                             scale=C_W)
    t["proxy_k"] = dv.fill_bf16(torch.empty((R, DI), dtype=bf, device=device), wl.seed, TID_PROXY)
    t["logits"] = dv.fill_f32(torch.empty((R, DI), dtype=f32, device=device), wl.seed, TID_LOGITS)
    t["store"] = torch.zeros((S, DI), dtype=torch.uint8 if wl.store_q8 == 2 else bf, device=device)
    t["sel"] = torch.zeros((Nq, G, wl.topk), dtype=torch.int32, device=device)
    t["sel_scores"] = torch.zeros((Nq, G, wl.topk), dtype=f32, device=device)
    t["q_hat"] = torch.zeros((Nq, G, HI, DI), dtype=bf, device=device)
    t["out"] = torch.zeros((Nq, H, D), dtype=bf, device=device)
    t["lse"] = torch.zeros((Nq, H), dtype=f32, device=device)
    return DeviceInputs(wl, t)


# ---------------------------------------------------------------------------
# host slices for the oracle (regenerated, never copied from the device)
# ---------------------------------------------------------------------------

def host_q(wl: Workload, qrows) -> np.ndarray:
    qrows = np.asarray(qrows, dtype=np.int64).reshape(-1)
    rows = (qrows[:, None] * H + np.arange(H)[None, :]).reshape(-1)
    return rms_rows_bf16_bits(wl.seed, TID_Q, rows, D).reshape(-1, H, D)


def host_k(wl: Workload, kv_rows) -> np.ndarray:
    kv_rows = np.asarray(kv_rows, dtype=np.int64).reshape(-1)
    rows = (kv_rows[:, None] * G + np.arange(G)[None, :]).reshape(-1)
    return rms_rows_bf16_bits(wl.seed, TID_K, rows, D).reshape(-1, G, D)


def host_k_group(wl: Workload, kv_rows, g: int) -> np.ndarray:
    """K cache rows of one group: [n, D] bits (the same values as host_k[:, g])."""
    kv_rows = np.asarray(kv_rows, dtype=np.int64).reshape(-1)
    return rms_rows_bf16_bits(wl.seed, TID_K, kv_rows * G + g, D)


def host_v_group(wl: Workload, kv_rows, g: int) -> np.ndarray:
    """V cache rows of one group: [n, D] bits (the same values as host_v[:, g])."""
    kv_rows = np.asarray(kv_rows, dtype=np.int64).reshape(-1)
    idx = (kv_rows[:, None] * (G * D) + g * D + np.arange(D)[None, :]).astype(np.uint64)
    return normal_bf16_bits(wl.seed, TID_V, idx)


def _flat(rows, width):
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    return (rows[:, None] * width + np.arange(width)[None, :]).astype(np.uint64)


def host_v(wl: Workload, kv_rows) -> np.ndarray:
    return normal_bf16_bits(wl.seed, TID_V, _flat(kv_rows, G * D)).reshape(-1, G, D)


def host_q_idx(wl: Workload, qrows) -> np.ndarray:
    if wl.corr_window:
        x = corr_rows_f32(wl.seed, TID_QIDX, qrows, G * HI * DI, wl.corr_window)
        return f32_to_bf16_bits(x).reshape(-1, G, HI, DI)
    return normal_bf16_bits(wl.seed, TID_QIDX, _flat(qrows, G * HI * DI)).reshape(-1, G, HI, DI)


def host_w(wl: Workload, qrows) -> np.ndarray:
    if wl.corr_window:
        return corr_rows_f32(wl.seed, TID_W, qrows, G * HI, wl.corr_window, C_W).reshape(-1, G, HI)
    return normal_f32(wl.seed, TID_W, _flat(qrows, G * HI), C_W).reshape(-1, G, HI)


def host_proxy(wl: Workload, kv_rows) -> np.ndarray:
    return normal_bf16_bits(wl.seed, TID_PROXY, _flat(kv_rows, DI)).reshape(-1, DI)


def host_logits(wl: Workload, kv_rows) -> np.ndarray:
    return normal_f32(wl.seed, TID_LOGITS, _flat(kv_rows, DI)).reshape(-1, DI)


# ---------------------------------------------------------------------------
# paged layout of the per-token tensors
# ---------------------------------------------------------------------------
PAGE_TOKENS = 16


def paginate(wl: Workload, di, rng):
    """The per-token tensors of ``di`` (K, V, proxy keys, logits) scattered
    into pools of 16-position pages through a random page table with seven
    spare pages; every pool slot that holds no position below a sequence's
    capacity is NaN.  Returns (pools by name, int32 page table on the device,
    per-sequence layouts whose kv_offset is the first page-table entry)."""
    import torch
    P = PAGE_TOKENS
    n_log = [(s.kv_capacity + P - 1) // P for s in wl.seqs]
    total = sum(n_log)
    n_pages = total + 7
    phys = rng.permutation(n_pages)[:total]
    table = np.zeros(total + 3, dtype=np.int32)          # trailing entries unused
    pools = {}
    for name in ("k", "v", "proxy_k", "logits"):
        t = di[name]
        pools[name] = torch.full((n_pages, P) + tuple(t.shape[1:]), float("nan"), dtype=t.dtype,
                                 device=t.device)
    seqs, off = [], 0
    for s, n in zip(wl.seqs, n_log):
        ids = phys[off:off + n]
        table[off:off + n] = ids
        pos = torch.arange(s.kv_capacity, device=di["k"].device)
        prow = torch.as_tensor(ids, device=pos.device).long()[pos // P]
        for name in pools:
            pools[name][prow, pos % P] = di[name][s.kv_offset:s.kv_offset + s.kv_capacity]
        seqs.append(SeqLayout(s.q_offset, s.n_q, s.pos0, off, s.kv_capacity, s.store_offset,
                              s.store_capacity))
        off += n
    return pools, torch.as_tensor(table, device=di["k"].device), seqs
