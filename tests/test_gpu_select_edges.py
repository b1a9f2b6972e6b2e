"""Selection edge cases whose exact answer follows from the selection rule
alone (page "Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache",
section "Selection is a weighted ReLU score, not attention softmax": the k
highest scores among blocks r < floor(t/B), equal scores to the lower block
id), so no oracle run is needed:

* every score equal (indexer weights zero): every row keeps blocks
  0..min(n, k)-1 -- rows of up to 1024 candidates in the one-wavefront
  select, longer ones in the sampled select, which then starts from a
  threshold every key passes, so the candidate list overflows and is cut to
  its top k, repeatedly -- the compaction path, with all keys tied;
* a row whose only positive scores sit at positions the long-row select
  samples (1008 blocks at k = 3072, 512 at k = 1024): the sampled threshold
  admits fewer than k keys, so the select must fall back to a radix over
  the whole row; the answer is those blocks plus the lowest-numbered others
  (score 0, ties to the lower id);
* the same two situations for the candidate lists of prefill calls whose
  rows have 32768+ candidates: all scores equal overflow every segment's
  list, and hot blocks placed on the positions the list threshold is
  sampled from leave fewer than k candidates; both rows are scored again in
  full and selected from their keys.

Inputs are seeded random tensors (or constructed exactly), written straight
into the indexer's inputs as a bf16-held store (store_q8 = 1, so the tied-mass
case can use values E4M3 does not hold); only the index step runs.
"""
import numpy as np
import pytest
import torch

import sparse_long_context_block_amd as sg

from .gpu_checks import log

pytestmark = pytest.mark.gpu


def _run_index(cfg, seqs, n_rows, q_idx, w, store):
    K = cfg.topk_blocks
    sel = torch.full((n_rows, 4, K), -7, dtype=torch.int32, device="cuda")
    ssc = torch.full((n_rows, 4, K), 7.0, dtype=torch.float32, device="cuda")
    sg.index_topk(cfg, seqs, q_idx, w, store, sel, sel_scores=ssc)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), ssc.cpu().numpy()


@pytest.mark.parametrize("n_q,pos0,B,K", [
    (1, 20000, 1, 3072),          # decode-sized call: split scoring, long row
    (1100, 16000, 1, 512),        # tiled call, long rows
    (1100, 160000, 8, 512),       # tiled call at B = 8, 20000+ candidates per row
    (3, 300000, 8, 2048),         # decode-sized, several queries, k = 2048
    (2, 40000, 1, 512),           # decode-sized, k <= 1024: 16-wavefront select
    (1100, 300000, 8, 512),       # tiled call, listed rows: every segment's list overflows
    (1100, 4000, 8, 64),          # tiled call, rows of 500..637 candidates: one wavefront per row
    (1100, 0, 1, 64),             # rows of 0..1099 candidates: per-wavefront rows, then sampled
])
def test_equal_scores_keep_lowest_block_ids(n_q, pos0, B, K):
    log("case equal scores", n_q, pos0, B, K)
    gen = torch.Generator(device="cuda").manual_seed(5)
    cache = pos0 + n_q
    q_idx = torch.randn(n_q, 4, 4, 128, generator=gen, device="cuda").to(torch.bfloat16)
    w = torch.zeros(n_q, 4, 4, dtype=torch.float32, device="cuda")
    store = torch.randn(cache // B, 128, generator=gen, device="cuda").to(torch.bfloat16)
    cfg = sg.config(block_size=B, topk_blocks=K, store_q8=1)
    sel, ssc = _run_index(cfg, [sg.seq(n_q, pos0=pos0, block_size=B)], n_q, q_idx, w, store)
    n = (pos0 + np.arange(n_q)) // B                       # candidates per row
    m = np.minimum(n, K)
    j = np.arange(K)[None, :]
    exp = np.where(j < m[:, None], j, -1).astype(np.int32)  # [n_q, K]
    assert (sel == exp[:, None, :]).all()
    assert (ssc == 0.0).all()


@pytest.mark.parametrize("K,hot_groups", [(3072, 63), (1024, 32)])
def test_sample_overestimate_falls_back_exactly(K, hot_groups):
    B = 1
    t = 16383                        # one query; n = 16383 candidate blocks
    n = t // B
    # the long-row select's sample: S keys (a sixteenth of the row, at most
    # 2048) in S/16 groups of 16 consecutive keys, group g starting at
    # g * (n - 16) // (S/16 - 1); the first hot_groups groups hold the only
    # positive scores, fewer than k of them but more than the sample rank the
    # threshold is taken at
    S = min(2048, n // 16) // 16 * 16
    ngrp = S // 16
    hot = sorted({(g * (n - 16)) // (ngrp - 1) + i for g in range(hot_groups) for i in range(16)})
    assert hot_groups <= ngrp and len(hot) == 16 * hot_groups < K and hot[-1] < n
    assert len(hot) >= -(-3 * K * S // n)
    log("case sampled-threshold fallback", n, K, len(hot))
    # u: zero on the rotary span (dims 0..31), one elsewhere, so q_hat . u
    # does not depend on positions; hot store rows are u, all others zero
    u = torch.zeros(128, dtype=torch.float32)
    u[32:] = 1.0
    store = torch.zeros(t + 1, 128, dtype=torch.float32)
    store[hot] = u
    q_idx = torch.zeros(1, 4, 4, 128, dtype=torch.float32)
    q_idx[0, :, 0] = u               # head 0 of every group
    w = torch.zeros(1, 4, 4, dtype=torch.float32)
    w[0, :, 0] = 1.0
    cfg = sg.config(block_size=B, topk_blocks=K, store_q8=1)
    sel, ssc = _run_index(cfg, [sg.seq(1, pos0=t, block_size=B)], 1,
                          q_idx.to(torch.bfloat16).cuda(), w.cuda(),
                          store.to(torch.bfloat16).cuda())
    hot_set = set(hot)
    cold = [r for r in range(n) if r not in hot_set][:K - len(hot)]
    exp = np.array(sorted(hot + cold), dtype=np.int32)
    is_hot = np.isin(exp, hot)
    for g in range(4):
        assert (sel[0, g] == exp).all()
        assert (ssc[0, g][~is_hot] == 0.0).all()
        hs = ssc[0, g][is_hot]
        assert (hs > 100.0).all() and (hs == hs[0]).all()


@pytest.mark.parametrize("K,hot_groups", [(512, 4), (2048, 10)])
def test_listed_threshold_above_kth_falls_back_exactly(K, hot_groups):
    # 1024 queries at B = 1 from t = 40960: tiles start at 40960+ candidates,
    # so their rows are listed.  The list threshold is the j-th largest of a
    # sample of 2048 scores taken as 128 groups of 16 consecutive blocks, group
    # g starting at g * (n0 - 16) // 127 (n0 = the tile's first position);
    # j = ceil(m k S / n0) (51 at k = 512, 153 at k = 2048).  The blocks of the
    # first hot_groups groups of the first tile are the only positive scores:
    # at least j of them, fewer than k, so the threshold admits fewer than k
    # candidates and the row must be scored again (later tiles sample other
    # blocks: their lists overflow instead); every row's answer is still the
    # hot blocks plus the lowest-numbered others.  k = 512 takes the failed
    # rows' sixteen-wavefront select, k = 2048 the four-wavefront one.
    B, n_q, pos0 = 1, 1024, 40960
    S, ngrp = 2048, 128
    n0 = pos0 // B
    hot = sorted({(g * (n0 - 16)) // (ngrp - 1) + i for g in range(hot_groups) for i in range(16)})
    m = 1.0 + 5.0 / np.sqrt(K * S / n0)
    j = int(np.ceil(m * K * S / n0))
    assert j <= len(hot) < K
    log("case listed-threshold fallback", n_q, pos0, K, len(hot), "j", j)
    u = torch.zeros(128, dtype=torch.float32)
    u[32:] = 1.0
    cache = pos0 + n_q
    store = torch.zeros(cache // B, 128, dtype=torch.float32)
    store[hot] = u
    q_idx = torch.zeros(n_q, 4, 4, 128, dtype=torch.float32)
    q_idx[:, :, 0] = u
    w = torch.zeros(n_q, 4, 4, dtype=torch.float32)
    w[:, :, 0] = 1.0
    cfg = sg.config(block_size=B, topk_blocks=K, store_q8=1)
    sel, ssc = _run_index(cfg, [sg.seq(n_q, pos0=pos0, block_size=B)], n_q,
                          q_idx.to(torch.bfloat16).cuda(), w.cuda(), store.to(torch.bfloat16).cuda())
    hot_set = set(hot)
    cold = [r for r in range(K) if r not in hot_set][:K - len(hot)]
    exp = np.array(sorted(hot + cold), dtype=np.int32)
    is_hot = np.isin(exp, hot)
    assert (sel == exp[None, None, :]).all()
    assert (ssc[:, :, ~is_hot] == 0.0).all()
    hs = ssc[:, :, is_hot]
    assert (hs > 100.0).all() and (hs == hs[0, 0, 0]).all()


@pytest.mark.parametrize("w0", [-1.0, 1.0])
def test_listed_rows_with_tied_mass_above_the_pool(w0):
    """Listed rows whose entries at the threshold outnumber the LDS pool.

    Every query's indexer heads are one-hot on dims 40..43 (past the rotary
    span), so a block's score is sum_i w_i * c * relu(store[r, 40 + i]) with
    c = bf16(RMSNorm(one-hot)).  Blocks r with r % 256 < 40 have all four
    dims <= 0 (score exactly 0: 40 per segment, about 9,400 per row, more
    than the 8,192-entry pool, none of the 256-block segment lists
    overflowing); 300 blocks carry a distinct positive value on dim 40 and
    the rest a positive value on dim 41.  With w = (-1, -1, -1, -1) no score
    is positive and the answer is the first k zero-score blocks (the tie
    rule); with w = (+1, -1, -1, -1) the 300 positive scores are the only
    ones above the zero threshold and the answer is the k largest of them.
    """
    n_q, pos0, B, K = 1100, 60000, 1, 256
    log("case tied mass", w0)
    rng = np.random.default_rng(17)
    cache = pos0 + n_q
    n_blocks = cache // B
    store = -np.abs(rng.standard_normal((n_blocks, 128))).astype(np.float32)
    store[:, :40] = rng.standard_normal((n_blocks, 40))
    store[:, 44:] = rng.standard_normal((n_blocks, 84))
    r = np.arange(n_blocks)
    zero = r % 256 < 40
    cand = np.flatnonzero(~zero & (r < pos0))
    pos = np.sort(rng.choice(cand, 300, replace=False))
    # distinct bf16 values: consecutive bit patterns from 1.0 upwards
    vals = (np.uint32(0x3F80) + rng.permutation(300).astype(np.uint32)) << 16
    store[pos, 40] = vals.view(np.float32)
    neg = ~zero
    neg[pos] = False
    store[neg, 41] = np.abs(rng.standard_normal(int(neg.sum()))) + 0.25
    store_d = torch.from_numpy(store).to(torch.bfloat16).cuda()
    q = np.zeros((n_q, 4, 4, 128), dtype=np.float32)
    for i in range(4):
        q[:, :, i, 40 + i] = 1.0
    q_idx = torch.from_numpy(q).to(torch.bfloat16).cuda()
    w = torch.tensor([w0, -1.0, -1.0, -1.0], dtype=torch.float32).repeat(n_q, 4, 1).cuda()
    cfg = sg.config(block_size=B, topk_blocks=K, store_q8=1)
    seqs = [sg.seq(n_q, pos0=pos0, kv_capacity=cache, store_capacity=n_blocks)]
    sel, ssc = _run_index(cfg, seqs, n_q, q_idx, w, store_d)
    c = float(torch.tensor(1.0 / np.sqrt(1.0 / 128 + 1e-6)).to(torch.bfloat16))
    if w0 < 0:
        want = np.flatnonzero(zero)[:K]
        want_s = np.zeros(K)
    else:
        v = store_d[pos, 40].float().cpu().numpy()
        top = np.sort(pos[np.argsort(-v, kind="stable")[:K]])
        want = top
        want_s = c * store_d[top, 40].float().cpu().numpy()
    for row in (0, 1, 517, n_q - 1):
        for g in range(4):
            assert np.array_equal(sel[row, g], want), (row, g)
            assert np.allclose(ssc[row, g], want_s, rtol=1e-6, atol=0.0), (row, g)
    assert (sel == want[None, None, :]).all()
