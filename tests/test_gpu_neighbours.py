"""The path's neighbours, fused into it (page "Step-5-Preview: Sparse Reads
Are Not a Compressed KV Cache": "Two paths leave the same hidden state" --
the main path normalizes Q/K and applies the layer's partial RoPE; "Main
attention still reads original K/V" -- each head's output vector is
sigmoid-gated before concatenation).

* sgqa_qk_prep against the oracle's main_qk (admissible bf16 rounding of the
  exact value), V copied bit for bit, the paged producer equal to the
  contiguous one;
* the gated attention: a gate of +30 (sigmoid 1 in fp32) reproduces the
  ungated output bit for bit; random gates are checked against the oracle's
  gated output on the tiled and gather paths and the split decode; the
  paged gated forward equals the contiguous one.
Raw Q/K/V, gammas and gate logits are seeded host arrays copied to the
device, so the oracle reads the same bits.
"""
import numpy as np
import pytest
import torch

import sparse_long_context_block_amd as sg
from oracle import sgqa as O
from synth import workloads as W

from . import parity as P
from .gpu_checks import Checker, lib_seq, lib_seqs, log, prepare, stratified_rows

pytestmark = pytest.mark.gpu


def _bf16_host(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("span,base", [(64, 10000.0), (192, 1e6), (0, 10000.0)])
def test_qk_prep_matches_oracle(span, base):
    log("case qk_prep", span, base)
    rng = np.random.default_rng(span + 7)
    # a prefill chunk and a decode token far into its cache
    layouts = [W.SeqLayout(0, 37, 1000, 0, 1100, 0, 137), W.SeqLayout(37, 1, 70000, 1100, 70001, 137, 8750)]
    nq, rows = 38, 1100 + 70001
    q_raw = _bf16_host(rng.standard_normal((nq, 64, 192)))
    k_raw = _bf16_host(rng.standard_normal((nq, 4, 192)) * 3)
    v_raw = _bf16_host(rng.standard_normal((nq, 4, 192)))
    qg = _bf16_host(rng.uniform(0.5, 1.5, 192))
    kg = _bf16_host(rng.uniform(0.5, 1.5, 192))
    cfg = sg.config()
    qk = sg.qk_config(rope_dim=span, rope_base=base, eps=1e-6)
    seqs = [lib_seq(s) for s in layouts]
    dev = {n: t.cuda() for n, t in dict(q_raw=q_raw, k_raw=k_raw, v_raw=v_raw, qg=qg, kg=kg).items()}
    q_out = torch.zeros(nq, 64, 192, dtype=torch.bfloat16, device="cuda")
    k_cache = torch.full((rows, 4, 192), float("nan"), dtype=torch.bfloat16, device="cuda")
    v_cache = torch.full((rows, 4, 192), float("nan"), dtype=torch.bfloat16, device="cuda")
    sg.qk_prep(cfg, qk, seqs, dev["q_raw"], dev["k_raw"], q_out, k_cache, v_raw=dev["v_raw"],
               v_cache=v_cache, q_gamma=dev["qg"], k_gamma=dev["kg"])
    torch.cuda.synchronize()
    pos = np.concatenate([s.pos0 + np.arange(s.n_q) for s in layouts])
    crow = np.concatenate([s.kv_offset + s.pos0 + np.arange(s.n_q) for s in layouts])
    q_ex = O.main_qk(_bits(q_raw), pos, span, base, 1e-6, _bits(qg))
    k_ex = O.main_qk(_bits(k_raw), pos, span, base, 1e-6, _bits(kg))
    st_q = P.check_rounded(P.bits_to_f64(_bits(q_out.cpu())), q_ex, False, P.REL_QHAT, "main q")
    kc = k_cache.cpu()[torch.as_tensor(crow)]
    st_k = P.check_rounded(P.bits_to_f64(_bits(kc)), k_ex, False, P.REL_QHAT, "main k")
    assert torch.equal(v_cache.cpu()[torch.as_tensor(crow)].view(torch.int16), v_raw.view(torch.int16))
    log("  q", st_q, "k", st_k)
    # only the new tokens' cache rows are written
    written = torch.zeros(rows, dtype=torch.bool)
    written[torch.as_tensor(crow)] = True
    assert torch.isnan(k_cache.cpu()[~written].float()).all()

    # paged caches: the same rows through a page table
    n_pages = rows // 16 + 9
    ids = np.random.default_rng(1).permutation(n_pages)
    table = torch.as_tensor(ids[:(1100 + 15) // 16 + (70001 + 15) // 16].astype(np.int32), device="cuda")
    players = [W.SeqLayout(0, 37, 1000, 0, 1100, 0, 137),
               W.SeqLayout(37, 1, 70000, (1100 + 15) // 16, 70001, 137, 8750)]
    kp = torch.full((n_pages, 16, 4, 192), float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    q_out2 = torch.zeros_like(q_out)
    sg.qk_prep(cfg, qk, [lib_seq(s) for s in players], dev["q_raw"], dev["k_raw"], q_out2, kp,
               v_raw=dev["v_raw"], v_cache=vp, q_gamma=dev["qg"], k_gamma=dev["kg"], page_table=table)
    torch.cuda.synchronize()
    assert torch.equal(q_out2.view(torch.int16), q_out.view(torch.int16))
    tab = table.cpu().numpy()
    for s, p in zip(layouts, players):
        for i in range(s.n_q):
            t = s.pos0 + i
            prow = int(tab[p.kv_offset + t // 16]) * 16 + t % 16
            assert torch.equal(kp.view(-1, 4, 192)[prow].view(torch.int16),
                               k_cache[s.kv_offset + t].view(torch.int16))
            assert torch.equal(vp.view(-1, 4, 192)[prow].view(torch.int16),
                               v_cache[s.kv_offset + t].view(torch.int16))


@pytest.mark.parametrize("name", ["chunk_1003_1997_b8_k64", "decode_small", "chunk_150000_2100"])
def test_gated_attention(name):
    # the chunk's queries t < 2048 take the tiled kernel, the rest the
    # gather kernel; the decode is split and merged; the forward calls over
    # the 152K-token cache run in two pieces over the second stream
    wl = W.make(name)
    log("case gated", name)
    di, cfg = prepare(wl)
    seqs = lib_seqs(wl)
    sg.forward(cfg, seqs, di["proxy_k"], di["logits"], di["store"], di["q_idx"], di["w"], di["sel"],
               di["q"], di["k"], di["v"], di["out"], lse=di["lse"], sel_scores=di["sel_scores"])
    torch.cuda.synchronize()
    out0, lse0, sel0 = di["out"].clone(), di["lse"].clone(), di["sel"].clone()
    nq = di["out"].shape[0]

    # sigmoid(30) is 1 in fp32: the gated kernels then give the ungated output
    ones = torch.full((nq, 64, 192), 30.0, dtype=torch.bfloat16, device="cuda")
    sg.sparse_attn_gated(cfg, seqs, di["q"], di["k"], di["v"], di["sel"], di["out"], ones, lse=di["lse"])
    torch.cuda.synchronize()
    assert torch.equal(di["out"].view(torch.int16), out0.view(torch.int16))
    assert torch.equal(di["lse"], lse0)

    gate = _bf16_host(np.random.default_rng(9).standard_normal((nq, 64, 192)) * 3)
    gate_d = gate.cuda()
    sg.forward_gated(cfg, seqs, di["proxy_k"], di["logits"], di["store"], di["q_idx"], di["w"], di["sel"],
                     di["q"], di["k"], di["v"], di["out"], gate_d, lse=di["lse"], sel_scores=di["sel_scores"])
    torch.cuda.synchronize()
    assert torch.equal(di["sel"], sel0) and torch.equal(di["lse"], lse0)
    gated = di["out"].clone()

    # paged + gated: the same bits
    pools, table, players = W.paginate(wl, di, np.random.default_rng(4))
    sg.forward_paged(cfg, [lib_seq(p) for p in players], pools["proxy_k"], pools["logits"], di["store"],
                     di["q_idx"], di["w"], di["sel"], di["q"], pools["k"], pools["v"], table, di["out"],
                     lse=di["lse"], gate=gate_d)
    torch.cuda.synchronize()
    assert torch.equal(di["out"].view(torch.int16), gated.view(torch.int16))

    # oracle: the gated head vectors on sampled rows (q_hat from the split call)
    sg.index_topk(cfg, seqs, di["q_idx"], di["w"], di["store"], di["sel"], sel_scores=di["sel_scores"],
                  q_hat_out=di["q_hat"])
    torch.cuda.synchronize()
    ck = Checker(wl, di, cfg)
    rng = np.random.default_rng(0)
    gb = _bits(gate)
    for si, s in enumerate(wl.seqs[:4]):
        stored, exact = ck.oracle_store(s, s.cache_len // wl.block_size)
        ck.check_seq(si, stratified_rows(s, wl.block_size, wl.topk, 12, rng), store_exact=(stored, exact),
                     gate_bits=gb)
    log(" ", ck.finish())
