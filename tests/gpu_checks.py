"""Run the HIP path on a synthetic workload and check it against the oracle.

The oracle side regenerates every input slice it needs from the seeded
generator on the host (synth.workloads.host_*); nothing it reads comes from
the GPU.  See tests/parity.py for the comparison rules.
"""
from __future__ import annotations

import numpy as np
import torch

import sparse_long_context_block_amd as sg
from oracle import numerics as nu
from oracle import sgqa as O
from synth import workloads as W

from . import parity as P
from .gpu_setup import lib_config, lib_seq, lib_seqs, log, prepare, setup_seqs  # noqa: F401


def oracle_config(wl: W.Workload) -> O.Config:
    return O.Config(block_size=wl.block_size, topk_blocks=wl.topk, store_q8=bool(wl.store_q8),
                    softmax_scale=float(np.float32(1.0 / np.sqrt(192.0))))


def run_steps(wl: W.Workload, di, cfg, use_forward: bool = False, ws=None):
    seqs = lib_seqs(wl)
    if use_forward:
        sg.forward(cfg, seqs, di["proxy_k"], di["logits"], di["store"], di["q_idx"], di["w"],
                   di["sel"], di["q"], di["k"], di["v"], di["out"], lse=di["lse"],
                   sel_scores=di["sel_scores"], ws=ws)
    else:
        sg.compress(cfg, seqs, di["proxy_k"], di["logits"], di["store"])
        sg.index_topk(cfg, seqs, di["q_idx"], di["w"], di["store"], di["sel"],
                      sel_scores=di["sel_scores"], q_hat_out=di["q_hat"], ws=ws)
        sg.sparse_attn(cfg, seqs, di["q"], di["k"], di["v"], di["sel"], di["out"], lse=di["lse"])
    torch.cuda.synchronize()


def stratified_rows(s: W.SeqLayout, B: int, K: int, n: int, rng) -> np.ndarray:
    """Query indices (0-based within the sequence) covering t < B, the first
    and last token of blocks, the k*B threshold, the last query, random."""
    nq = s.n_q
    if nq <= n:
        return np.arange(nq)
    t0 = s.pos0
    cand = set()
    for t in [t0, t0 + 1, t0 + nq - 1, t0 + nq - 2]:
        cand.add(t)
    for t in range(t0, min(t0 + nq, B + 2)):
        cand.add(t)
    thr = K * B
    for t in (thr - 1, thr, thr + 1, thr + B - 1, thr + B, 2 * thr, 2 * thr + B - 1):
        if t0 <= t < t0 + nq:
            cand.add(t)
    while len(cand) < n:
        t = int(rng.integers(t0, t0 + nq))
        cand.add(t)
        if len(cand) < n and (t // B) * B >= t0:
            cand.add((t // B) * B)                 # first token of a block
        if len(cand) < n and (t // B) * B + B - 1 < t0 + nq:
            cand.add((t // B) * B + B - 1)         # last token of a block
    return np.array(sorted(cand))[:max(n, 0)] - t0


class Checker:
    """Holds the GPU results of one run and checks sampled rows."""

    def __init__(self, wl: W.Workload, di, cfg):
        self.wl, self.di, self.cfg = wl, di, cfg
        self.ocfg = oracle_config(wl)
        st = di["store"].cpu()
        if st.dtype == torch.uint8:            # E4M3 codes: widened exactly to bf16
            st = st.view(torch.float8_e4m3fn).to(torch.bfloat16)
        self.store = st.view(torch.int16).numpy().view(np.uint16)
        self.sel = di["sel"].cpu().numpy()
        self.sel_scores = di["sel_scores"].cpu().numpy()
        self.q_hat = di["q_hat"].cpu().view(torch.int16).numpy().view(np.uint16)
        self.out = di["out"].float().cpu().numpy().astype(np.float64)
        self.lse = di["lse"].cpu().numpy().astype(np.float64)
        self.stats = {"rows": 0, "sel_identical": 0, "sel_valid_other": 0, "store": None,
                      "q_hat": None, "score_max_rel": 0.0, "attn": None, "sel_rows": 0}
        self._o_gpu, self._o_ref, self._l_gpu, self._l_ref = [], [], [], []

    # -- store ----------------------------------------------------------------
    def oracle_store(self, s: W.SeqLayout, n_blocks: int):
        B = self.wl.block_size
        rows = s.kv_offset + np.arange(n_blocks * B)
        kp = W.host_proxy(self.wl, rows)
        lg = W.host_logits(self.wl, rows)
        return O.compress(kp, lg, np.arange(n_blocks), self.ocfg)

    def check_store(self, s: W.SeqLayout, stored, exact, blocks=None):
        n = stored.shape[0]
        blocks = np.arange(n) if blocks is None else np.asarray(blocks)
        gpu = P.bits_to_f64(self.store[s.store_offset + blocks])
        st = P.check_rounded(gpu, exact[blocks], self.wl.store_q8, P.REL_STORE, "store")
        prev = self.stats["store"] or {"n": 0, "boundary_cases": 0, "max_abs": 0.0}
        self.stats["store"] = {"n": prev["n"] + st["n"],
                               "boundary_cases": prev["boundary_cases"] + st["boundary_cases"],
                               "max_abs": max(prev["max_abs"], st["max_abs"])}
        return st

    # -- one sequence ----------------------------------------------------------
    def check_seq(self, si: int, qs: np.ndarray, store_exact=None, check_attn: bool = True,
                  gate_bits=None):
        """Check query rows qs (0-based in sequence si): scores, selection
        and, unless check_attn is False, attention; gate_bits (bf16 bits
        [Nq, H, D]) makes the reference the sigmoid-gated output."""
        wl, ocfg = self.wl, self.ocfg
        s = wl.seqs[si]
        B, K = wl.block_size, wl.topk
        if qs.size == 0:
            return
        t_all = s.pos0 + qs
        b_max = int(t_all.max()) // B
        if store_exact is None:
            stored, exact = self.oracle_store(s, max(b_max, 0))
        else:
            stored, exact = store_exact
        s_lo_all, s_hi_all = P.rounding_interval(exact[:b_max], wl.store_q8, P.REL_STORE)
        sb = P.StoreBounds(s_lo_all, s_hi_all)
        qrows = s.q_offset + qs
        qi_bits = W.host_q_idx(wl, qrows)
        w = W.host_w(wl, qrows).astype(np.float64)
        qh_exact = O.index_queries(qi_bits, t_all, ocfg, exact=True)
        qh = nu.round_bf16(qh_exact)
        # q_hat parity (admissible rounding)
        qh_gpu = P.bits_to_f64(self.q_hat[qrows])
        st = P.check_rounded(qh_gpu, qh_exact, False, P.REL_QHAT, "q_hat")
        prev = self.stats["q_hat"] or {"n": 0, "boundary_cases": 0, "max_abs": 0.0}
        self.stats["q_hat"] = {"n": prev["n"] + st["n"],
                               "boundary_cases": prev["boundary_cases"] + st["boundary_cases"],
                               "max_abs": max(prev["max_abs"], st["max_abs"])}
        q_lo, q_hi = P.rounding_interval(qh_exact, False, P.REL_QHAT)
        q_main = W.host_q(wl, qrows) if check_attn else None
        for n_i, (qi, t) in enumerate(zip(qs, t_all)):
            t = int(t)
            row = int(s.q_offset + qi)
            b = t // B
            sel_ref_all = []
            for g in range(4):
                where = f"{wl.name} seq {si} t={t} g={g}"
                s_ref = O.block_scores(qh[n_i, g], w[n_i, g], stored[:b])
                lo, hi = P.score_bounds(q_lo[n_i, g], q_hi[n_i, g], None, None, w[n_i, g],
                                        sb=sb, b=b)
                sel_gpu = self.sel[row, g]
                P.check_selection(sel_gpu, b, K, s_ref, lo, hi, where)
                r = P.check_scores(self.sel_scores[row, g], sel_gpu, s_ref, lo, hi, where)
                self.stats["score_max_rel"] = max(self.stats["score_max_rel"], r)
                sel_ref = O.select_blocks(s_ref, K)
                same = np.array_equal(sel_ref, sel_gpu)
                self.stats["sel_rows"] += 1
                self.stats["sel_identical"] += int(same)
                self.stats["sel_valid_other"] += int(not same)
                sel_ref_all.append(sel_ref if same else sel_gpu.astype(np.int64))
            if not check_attn:
                continue
            # attention of row t for the 4 groups over the (validated) selections
            q = nu.bf16_bits_to_f64(q_main[n_i])
            for g in range(4):
                u = O.token_set(sel_ref_all[g], t, B)
                kk = nu.bf16_bits_to_f64(W.host_k_group(wl, s.kv_offset + u, g))
                vv = nu.bf16_bits_to_f64(W.host_v_group(wl, s.kv_offset + u, g))
                heads = slice(16 * g, 16 * g + 16)
                o, l = O.attend(q[heads], kk, vv, ocfg.softmax_scale)
                if gate_bits is not None:
                    o = O.gate(o, gate_bits[row, heads])
                self._o_ref.append(o)
                self._l_ref.append(l)
                self._o_gpu.append(self.out[row, heads])
                self._l_gpu.append(self.lse[row, heads])
            self.stats["rows"] += 1

    def finish(self):
        if self._o_ref:
            self.stats["attn"] = P.check_attention(np.stack(self._o_gpu), np.stack(self._o_ref),
                                                   np.stack(self._l_gpu), np.stack(self._l_ref),
                                                   f"{self.wl.name} attention")
        return self.stats
