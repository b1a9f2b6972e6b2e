"""sparse_attn alone on constructed selections, and the all-blocks case
against dense causal attention (torch, float32 on the CPU)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import sparse_long_context_block_amd as sg
from oracle import numerics as nu
from oracle import sgqa as O
from synth import workloads as W

from . import parity as P
from .gpu_checks import lib_seqs, log, oracle_config, prepare

pytestmark = pytest.mark.gpu


def _host_sel(rng, n_q, pos0, B, K, mode):
    sel = np.full((n_q, 4, K), -1, dtype=np.int32)
    for i in range(n_q):
        b = (pos0 + i) // B
        for g in range(4):
            if mode == "empty" or b == 0:
                continue
            if mode == "all":
                ids = np.arange(min(b, K))
            else:
                cnt = int(rng.integers(0, min(b, K) + 1))
                ids = np.sort(rng.choice(b, size=cnt, replace=False))
            sel[i, g, :ids.size] = ids
    return sel


@pytest.mark.parametrize("name,mode", [("prefill_600_b8_k40", "random"),
                                       ("prefill_600_b8_k40", "empty"),
                                       ("prefill_300_b1_k100", "random"),
                                       ("prefill_500_b16_k4", "all"),
                                       ("decode_small", "random")])
def test_attention_on_constructed_selection(name, mode):
    wl = W.make(name)
    log("case", name, mode)
    di, cfg = prepare(wl)
    rng = np.random.default_rng(5)
    ocfg = oracle_config(wl)
    o_gpu, o_ref, l_gpu, l_ref = [], [], [], []
    sel_all = np.full((wl.q_rows, 4, wl.topk), -1, dtype=np.int32)
    for s in wl.seqs:
        sel_all[s.q_offset:s.q_offset + s.n_q] = _host_sel(rng, s.n_q, s.pos0, wl.block_size, wl.topk, mode)
    di.t["sel"].copy_(torch.from_numpy(sel_all))
    sg.sparse_attn(cfg, lib_seqs(wl), di["q"], di["k"], di["v"], di["sel"], di["out"], lse=di["lse"])
    torch.cuda.synchronize()
    out = di["out"].float().cpu().numpy()
    lse = di["lse"].cpu().numpy()
    for s in wl.seqs:
        qs = np.arange(s.n_q) if s.n_q <= 64 else np.sort(rng.choice(s.n_q, 64, replace=False))
        qrows = s.q_offset + qs
        q = nu.bf16_bits_to_f64(W.host_q(wl, qrows))
        for n_i, qi in enumerate(qs):
            t = s.pos0 + int(qi)
            row = s.q_offset + int(qi)
            for g in range(4):
                u = O.token_set(sel_all[row, g], t, wl.block_size)
                kk = nu.bf16_bits_to_f64(W.host_k(wl, s.kv_offset + u))[:, g]
                vv = nu.bf16_bits_to_f64(W.host_v(wl, s.kv_offset + u))[:, g]
                o, l = O.attend(q[n_i, 16 * g:16 * g + 16], kk, vv, ocfg.softmax_scale)
                o_ref.append(o); l_ref.append(l)
                o_gpu.append(out[row, 16 * g:16 * g + 16]); l_gpu.append(lse[row, 16 * g:16 * g + 16])
    st = P.check_attention(np.stack(o_gpu), np.stack(o_ref), np.stack(l_gpu), np.stack(l_ref), name)
    log(st)


def test_all_blocks_selected_equals_dense_causal():
    # K >= floor(t/B) for every t: sparse attention over all history is dense
    # causal GQA attention (torch SDPA in float32 on the CPU)
    wl = W.make("prefill_512_b8_k64")
    di, cfg = prepare(wl)
    seqs = lib_seqs(wl)
    sg.forward(cfg, seqs, di["proxy_k"], di["logits"], di["store"], di["q_idx"], di["w"],
               di["sel"], di["q"], di["k"], di["v"], di["out"], lse=di["lse"])
    torch.cuda.synchronize()
    T = 512
    q = torch.from_numpy(nu.bf16_bits_to_f64(W.host_q(wl, np.arange(T))).astype(np.float32))
    k = torch.from_numpy(nu.bf16_bits_to_f64(W.host_k(wl, np.arange(T))).astype(np.float32))
    v = torch.from_numpy(nu.bf16_bits_to_f64(W.host_v(wl, np.arange(T))).astype(np.float32))
    qt = q.permute(1, 0, 2)[None]
    kt = k.permute(1, 0, 2).repeat_interleave(16, 0)[None].contiguous()
    vt = v.permute(1, 0, 2).repeat_interleave(16, 0)[None].contiguous()
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=cfg.softmax_scale)
    ref = ref[0].permute(1, 0, 2).double().numpy()
    got = di["out"].float().cpu().numpy().astype(np.float64)
    st = P.check_attention(got, ref, what="dense equivalence")
    log(st)
    sel = di["sel"].cpu().numpy()
    for t in range(T):
        b = t // 8
        assert np.array_equal(sel[t, :, :b], np.tile(np.arange(b), (4, 1)))
        assert np.all(sel[t, :, b:] == -1)
