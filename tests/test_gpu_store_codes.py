"""The proxy-key store held as E4M3 codes (store_q8 = 2; page "Step-5-Preview:
Sparse Reads Are Not a Compressed KV Cache", section "Eight tokens become one
search key, coordinate by coordinate": the summaries are stored in E4M3 and
widened to BF16 for the score matmul).

Every store value is an E4M3 value either way, so a run over a uint8 code
store must give the same bits as the run over the bf16-held store
(store_q8 = 1): the codes widen to the very bf16 values, and every score
kernel sees identical MFMA operands.  Checked on workloads that take each
index path (fused streaming top-k, split scoring, tiled keyed and listed
tiles, the list select's rescue) and through the oracle on one of them; every
finite code is scored once through the fused and the decode scorer, and written
once by the merge step (B = 1, gamma 0, beta set to the codes' values).
"""
import numpy as np
import pytest
import torch

import sparse_long_context_block_amd as sg
from synth import workloads as W

from .gpu_checks import Checker, log, prepare, run_steps, stratified_rows
from .gpu_setup import lib_seqs

pytestmark = pytest.mark.gpu


def _forward(wl):
    di, cfg = prepare(wl)
    sg.forward(cfg, lib_seqs(wl), di["proxy_k"], di["logits"], di["store"], di["q_idx"], di["w"], di["sel"],
               di["q"], di["k"], di["v"], di["out"], lse=di["lse"], sel_scores=di["sel_scores"])
    torch.cuda.synchronize()
    return di


@pytest.mark.parametrize("name", [
    "prefill_300_b8_k64",            # every row has <= k candidates: fused kernel
    "tiny_prefill_256",              # split scoring, short rows
    "decode_small",                  # split scoring, long rows, split attention
    "prefill_2000_b1_k64",           # tiled keyed scoring, wave and sampled selects
    "chunk_40000_1024_b1_k64",       # listed tiles: sample, threshold, candidate lists
    "chunk_1003_1997_b8_k64",        # a chunk over an existing cache
])
def test_code_store_gives_identical_bits(name):
    log("case store codes", name)
    ref = _forward(W.make(name, store_q8=1))
    got = _forward(W.make(name, store_q8=2))
    assert got["store"].dtype == torch.uint8
    widened = got["store"].view(torch.float8_e4m3fn).to(torch.bfloat16)
    assert torch.equal(widened.view(torch.int16), ref["store"].view(torch.int16))
    for k in ("sel", "sel_scores", "lse"):
        assert torch.equal(got[k], ref[k]), k
    assert torch.equal(got["out"].view(torch.int16), ref["out"].view(torch.int16))


def test_code_store_against_the_oracle():
    wl = W.make("decode_small", store_q8=2)
    log("case store codes, oracle", wl.name)
    di, cfg = prepare(wl)
    run_steps(wl, di, cfg)
    ck = Checker(wl, di, cfg)
    rng = np.random.default_rng(3)
    for si, s in enumerate(wl.seqs[:4]):
        stored, exact = ck.oracle_store(s, s.cache_len // wl.block_size)
        ck.check_store(s, stored, exact)
        ck.check_seq(si, stratified_rows(s, wl.block_size, wl.topk, 8, rng), store_exact=(stored, exact))
    log(" ", ck.finish())


def test_code_store_rescue_path():
    # a listed tile whose sampled threshold admits fewer than k candidates
    # (hot blocks only on sampled positions): the rows are scored again from
    # the code store by the rescore kernel and selected from their keys
    B, K, n_q, pos0 = 1, 512, 1024, 40960
    n0 = pos0 // B
    hot = sorted({(g * (n0 - 16)) // 127 + i for g in range(4) for i in range(16)})
    log("case store codes, rescue", len(hot))
    u = torch.zeros(128, dtype=torch.float32)
    u[32:] = 1.0
    store = torch.zeros((pos0 + n_q) // B, 128, dtype=torch.float32)
    store[hot] = u
    q_idx = torch.zeros(n_q, 4, 4, 128, dtype=torch.float32)
    q_idx[:, :, 0] = u
    w = torch.zeros(n_q, 4, 4, dtype=torch.float32)
    w[:, :, 0] = 1.0
    seqs = [sg.seq(n_q, pos0=pos0, block_size=B)]
    q_idx, w = q_idx.to(torch.bfloat16).cuda(), w.cuda()
    outs = []
    for q8, st in ((1, store.to(torch.bfloat16).cuda()),
                   (2, store.to(torch.float8_e4m3fn).view(torch.uint8).cuda())):
        cfg = sg.config(block_size=B, topk_blocks=K, store_q8=q8)
        sel = torch.full((n_q, 4, K), -7, dtype=torch.int32, device="cuda")
        ssc = torch.full((n_q, 4, K), 7.0, dtype=torch.float32, device="cuda")
        sg.index_topk(cfg, seqs, q_idx, w, st, sel, sel_scores=ssc)
        torch.cuda.synchronize()
        outs.append((sel.cpu(), ssc.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    hot_set = set(hot)
    exp = np.array(sorted(hot + [r for r in range(K) if r not in hot_set][:K - len(hot)]), dtype=np.int32)
    assert (outs[1][0].numpy() == exp[None, None, :]).all()


@pytest.mark.parametrize("K", [256, 64])
def test_every_code_widens_exactly(K):
    # block r of the store holds code r on coordinate 40 (past the rotary
    # span; the two NaN codes replaced by zero) and zeros elsewhere; indexer
    # head 0 of every group is +e_40 for the first query and -e_40 for the
    # second, weight 1, so block r scores c * max(+-value(r), 0) exactly
    # (c = bf16 of the RMSNorm of a one-hot row; a bf16 x E4M3 product is
    # exact in fp32).  K = 256 keeps every block (fused kernel); K = 64 keeps
    # the 64 largest of each sign (decode-sized scoring kernel).
    log("case every code", K)
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    rows = 257
    store = np.zeros((2 * rows, 128), dtype=np.uint8)
    store[:256, 40] = codes
    store[rows:rows + 256, 40] = codes
    q = np.zeros((2, 4, 4, 128), dtype=np.float32)
    q[0, :, 0, 40] = 1.0
    q[1, :, 0, 40] = -1.0
    w = np.zeros((2, 4, 4), dtype=np.float32)
    w[:, :, 0] = 1.0
    seqs = [sg.Seq(q_offset=i, n_q=1, pos0=256, cache_len=257, kv_offset=0, kv_capacity=257,
                   store_offset=i * rows, store_capacity=rows) for i in range(2)]
    cfg = sg.config(block_size=1, topk_blocks=K)
    sel = torch.full((2, 4, K), -7, dtype=torch.int32, device="cuda")
    ssc = torch.full((2, 4, K), 7.0, dtype=torch.float32, device="cuda")
    sg.index_topk(cfg, seqs, torch.from_numpy(q).to(torch.bfloat16).cuda(), torch.from_numpy(w).cuda(),
                  torch.from_numpy(store).cuda(), sel, sel_scores=ssc)
    torch.cuda.synchronize()
    sel, ssc = sel.cpu().numpy(), ssc.cpu().numpy()
    c = np.float32(float(torch.tensor(1.0 / np.sqrt(1.0 / 128 + 1e-6)).to(torch.bfloat16)))
    for i, sign in enumerate((1.0, -1.0)):
        s = (c * np.maximum(np.float32(sign) * vals, 0)).astype(np.float32)
        want = np.sort(np.argsort(-s, kind="stable")[:K]).astype(np.int32)
        for g in range(4):
            assert np.array_equal(sel[i, g], want), (sign, g)
            assert np.array_equal(ssc[i, g], s[want]), (sign, g)


def test_compress_writes_every_code():
    # B = 1 and ln_gamma = 0: a block's summary is ln_beta exactly (softmax
    # over one token is 1; LayerNorm times 0 plus beta), so with beta set to
    # E4M3 values on the coordinates past the rotary span (32..127) the store
    # codes must be those values' codes.  Three calls cover the 253 nonzero
    # finite codes (0x80, negative zero, is left out: beta = -0 stores +0).
    codes = np.array([c for c in range(256) if c not in (0x00, 0x7F, 0x80, 0xFF)], dtype=np.uint8)
    log("case compress codes", len(codes))
    n = 3
    cfg = sg.config(block_size=1, topk_blocks=8)
    seqs = [sg.Seq(q_offset=0, n_q=n, pos0=0, cache_len=n, kv_offset=0, kv_capacity=n, store_offset=0,
                   store_capacity=n)]
    rng = np.random.default_rng(11)
    proxy = torch.from_numpy(rng.standard_normal((n, 128)).astype(np.float32)).to(torch.bfloat16).cuda()
    logits = torch.from_numpy(rng.standard_normal((n, 128)).astype(np.float32)).cuda()
    gamma = torch.zeros(128, dtype=torch.bfloat16, device="cuda")
    for part in range(0, len(codes), 96):
        chunk = codes[part:part + 96]
        c96 = np.zeros(96, dtype=np.uint8)
        c96[:len(chunk)] = chunk
        beta = np.zeros(128, dtype=np.float32)
        beta[32:] = torch.from_numpy(c96).view(torch.float8_e4m3fn).float().numpy()
        store = torch.full((n, 128), 0x7F, dtype=torch.uint8, device="cuda")
        sg.compress(cfg, seqs, proxy, logits, store, ln_gamma=gamma,
                    ln_beta=torch.from_numpy(beta).to(torch.bfloat16).cuda())
        torch.cuda.synchronize()
        st = store.cpu().numpy()
        for r in range(n):
            assert np.array_equal(st[r, 32:], c96), (part, r)
            assert np.isin(st[r, :32], (0x00, 0x80)).all(), (part, r)     # zeros on the rotary span
