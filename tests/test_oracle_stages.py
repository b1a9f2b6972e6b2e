"""Pins of the oracle's four steps (CPU only).

Each test ties an oracle function to something other than itself: a library
routine (torch norms, torch attention), a closed-form property the pages
state, brute force on tiny inputs, a hand-worked example under
tests/golden/, or a count the pages print.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import numerics as nu
from oracle import sgqa as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _rope_complex(y, pos, rope_dim, base):
    """Rotary span as a complex multiplication of z_j = y_j + i*y_{j+half}."""
    half = rope_dim // 2
    z = y[..., :half] + 1j * y[..., half:rope_dim]
    freqs = np.exp(-np.log(base) * (2.0 * np.arange(half) / rope_dim))
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * freqs)
    out = np.array(y, dtype=np.float64, copy=True)
    out[..., :half] = z.real
    out[..., half:rope_dim] = z.imag
    return out


# --------------------------------------------------------------------------
# norms and rotary span
# --------------------------------------------------------------------------

def test_layer_norm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 128)) * 3 + 1
    g, b = rng.standard_normal(128), rng.standard_normal(128)
    ref = F.layer_norm(torch.from_numpy(x), (128,), torch.from_numpy(g), torch.from_numpy(b), eps=1e-6)
    assert np.allclose(O.layer_norm(x, 1e-6, g, b), ref.numpy(), rtol=1e-12, atol=1e-12)
    ref0 = F.layer_norm(torch.from_numpy(x), (128,), eps=1e-6)
    assert np.allclose(O.layer_norm(x, 1e-6), ref0.numpy(), rtol=1e-12, atol=1e-12)


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 4, 128)) * 2
    g = rng.standard_normal(128)
    ref = F.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(g), eps=1e-6)
    assert np.allclose(O.rms_norm(x, 1e-6, g), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_rope_is_complex_rotation_of_half_split_pairs():
    # reading: half-split pairs, base**(-2j/d) frequencies (parity unpinned
    # against the real model); this pins the rotation direction and pairing
    rng = np.random.default_rng(2)
    y = rng.standard_normal((20, 128))
    pos = rng.integers(0, 1 << 20, 20)
    # angles near 1e6 rad carry ~1e-10 rad of float64 noise from the two
    # frequency evaluations; a pairing or sign mistake is an O(1) difference
    assert np.allclose(O.rope(y, pos, 32, 10000.0), _rope_complex(y, pos, 32, 10000.0),
                       rtol=0, atol=1e-8)
    small = np.arange(20)
    assert np.allclose(O.rope(y, small, 32, 10000.0), _rope_complex(y, small, 32, 10000.0),
                       rtol=0, atol=1e-13)


def test_rope_relative_position_norm_passthrough():
    rng = np.random.default_rng(3)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    for t, s, d in [(5, 3, 100), (1000, 17, 999_000), (70, 70, 123_456)]:
        a = O.rope(q, t, 32, 1e4) @ O.rope(k, s, 32, 1e4)
        b = O.rope(q, t + d, 32, 1e4) @ O.rope(k, s + d, 32, 1e4)
        assert abs(a - b) < 1e-9
    y = O.rope(q, 12345, 32, 1e4)
    assert abs(np.linalg.norm(y) - np.linalg.norm(q)) < 1e-12
    assert np.array_equal(y[32:], q[32:])
    assert np.array_equal(O.rope(q, 0, 32, 1e4), q)


# --------------------------------------------------------------------------
# step 1: merging
# --------------------------------------------------------------------------

def test_merge_weights_sum_to_one_per_coordinate():
    rng = np.random.default_rng(4)
    c = rng.standard_normal((8, 128)) * 5
    assert np.allclose(O.merge(np.ones((8, 128)), c), 1.0, rtol=0, atol=1e-15)
    const = np.tile(rng.standard_normal(128), (8, 1))
    assert np.allclose(O.merge(const, c), const[0], rtol=1e-14, atol=1e-15)


def test_merge_coordinatewise_range_and_not_mean():
    rng = np.random.default_rng(5)
    for _ in range(50):
        k = rng.standard_normal((8, 128))
        c = rng.standard_normal((8, 128)) * 3
        m = O.merge(k, c)
        assert np.all(m >= k.min(axis=0) - 1e-12) and np.all(m <= k.max(axis=0) + 1e-12)
        assert not np.allclose(m, k.mean(axis=0))


def test_merge_block_of_one_is_the_key():
    rng = np.random.default_rng(6)
    k = rng.standard_normal((1, 128))
    assert np.array_equal(O.merge(k, rng.standard_normal((1, 128))), k[0])


def test_merge_shift_invariance_and_equal_logits_mean():
    rng = np.random.default_rng(7)
    k = rng.standard_normal((8, 128))
    c = rng.standard_normal((8, 128))
    shift = rng.standard_normal(128) * 50
    assert np.allclose(O.merge(k, c + shift), O.merge(k, c), rtol=1e-12, atol=1e-13)
    same = np.tile(rng.standard_normal(128), (8, 1))
    assert np.allclose(O.merge(k, same), k.mean(axis=0), rtol=1e-13, atol=1e-14)


def test_merge_huge_gap_is_finite_selection():
    # max subtraction: a 1e4 logit gap must not overflow
    rng = np.random.default_rng(8)
    k = rng.standard_normal((8, 128))
    c = np.zeros((8, 128))
    winner = rng.integers(0, 8, 128)
    c[winner, np.arange(128)] = 1e4
    m = O.merge(k, c + 700.0)
    assert np.all(np.isfinite(m))
    assert np.array_equal(m, k[winner, np.arange(128)])


def test_merge_summary_outside_hull():
    ex = _golden("worked_examples.json")["merge_not_in_hull"]
    m = O.merge(np.array(ex["keys"]), np.array(ex["logits"]))
    expect = 1.0 / (1.0 + math.exp(-20.0))
    assert np.allclose(m, [expect, expect], rtol=1e-15, atol=0)
    # any convex combination of the two keys has coordinate sum 1
    assert m.sum() > ex["hull_coordinate_sum"] + 0.5


def test_compress_rounding_and_block_size_one():
    rng = np.random.default_rng(9)
    T = 64
    kp = _bf16_bits(rng.standard_normal((T, 128)))
    lg = rng.standard_normal((T, 128)).astype(np.float32)
    cfg8 = O.Config(block_size=8, store_q8=True)
    stored, exact = O.compress(kp, lg, np.arange(8), cfg8)
    assert np.array_equal(stored, nu.q8(exact))
    cfg8b = O.Config(block_size=8, store_q8=False)
    stored_b, exact_b = O.compress(kp, lg, np.arange(8), cfg8b)
    assert np.array_equal(exact_b, exact)
    assert np.array_equal(stored_b, nu.round_bf16(exact))
    # block size 1: each summary is the token's own normalised, rotated key
    cfg1 = O.Config(block_size=1, store_q8=False)
    s1, e1 = O.compress(kp, lg, np.arange(T), cfg1)
    x = torch.from_numpy(nu.bf16_bits_to_f64(kp))
    ln = F.layer_norm(x, (128,), eps=1e-6).numpy()
    ref = _rope_complex(ln, np.arange(T), 32, 10000.0)
    assert np.allclose(e1, ref, rtol=1e-12, atol=1e-12)


def test_compress_uses_each_tokens_own_position():
    # identical raw tokens at different positions give different summaries
    rng = np.random.default_rng(10)
    row = _bf16_bits(rng.standard_normal(128))
    kp = np.tile(row, (16, 1))
    lg = np.tile(rng.standard_normal(128).astype(np.float32), (16, 1))
    st, ex = O.compress(kp, lg, [0, 1], O.Config(block_size=8, store_q8=False))
    assert not np.allclose(ex[0, :32], ex[1, :32])
    assert np.array_equal(ex[0, 32:], ex[1, 32:])


# --------------------------------------------------------------------------
# step 2: indexer scores
# --------------------------------------------------------------------------

def test_index_queries_match_library_norm_and_cast():
    rng = np.random.default_rng(11)
    qi = _bf16_bits(rng.standard_normal((6, 4, 4, 128)))
    pos = np.array([0, 1, 7, 8, 1000, 1_048_575])
    got = O.index_queries(qi, pos, O.Config())
    x = torch.from_numpy(nu.bf16_bits_to_f64(qi))
    y = F.rms_norm(x, (128,), eps=1e-6).numpy()
    y = _rope_complex(y, pos[:, None, None], 32, 10000.0)
    ref = torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    # a float64 value within rounding noise of a bf16 midpoint may land on
    # either side; every element must agree to within one bf16 ulp and almost all exactly
    ulp = np.exp2(np.floor(np.log2(np.abs(ref) + 1e-300)) - 7)
    assert np.all(np.abs(got - ref) <= ulp)
    assert np.mean(got == ref) > 0.999


def test_scores_worked_example_relu_inside_sum():
    ex = _golden("worked_examples.json")["relu_inside_sum"]
    qh = np.zeros((4, 128))
    qh[:, :3] = ex["q_hat"]
    st = np.zeros((4, 128))
    st[:, :3] = ex["store"]
    s = O.block_scores(qh, np.array(ex["w"]), st)
    assert np.array_equal(s, np.array(ex["scores"]))
    assert not np.array_equal(s, np.array(ex["relu_outside_would_give"]))
    sel = ex["select"]
    for k in (1, 2, 3, 4):
        got = O.select_blocks(s, k)
        assert got.tolist() == sel[f"k{k}"]


def test_scores_can_be_negative():
    ex = _golden("worked_examples.json")["negative_scores"]
    qh = np.zeros((4, 128))
    qh[:, :3] = ex["q_hat"]
    st = np.zeros((len(ex["store"]), 128))
    st[:, :3] = ex["store"]
    s = O.block_scores(qh, np.array(ex["w"]), st)
    assert np.array_equal(s, np.array(ex["scores"]))
    assert O.select_blocks(s, 1).tolist() == ex["select_k1"]
    assert O.select_blocks(s, 2).tolist() == ex["select_k2"]


def test_scores_special_cases_and_linearity():
    rng = np.random.default_rng(12)
    qh = np.abs(rng.standard_normal((4, 128)))
    st = np.abs(rng.standard_normal((40, 128)))
    w1 = np.array([1.0, 0, 0, 0])
    assert np.allclose(O.block_scores(qh, w1, st), st @ qh[0], rtol=1e-14)
    assert np.array_equal(O.block_scores(qh, np.zeros(4), st), np.zeros(40))
    qh = rng.standard_normal((4, 128))
    st = rng.standard_normal((40, 128))
    wa, wb = rng.standard_normal(4), rng.standard_normal(4)
    sa, sb = O.block_scores(qh, wa, st), O.block_scores(qh, wb, st)
    assert np.allclose(O.block_scores(qh, wa + wb, st), sa + sb, rtol=1e-12, atol=1e-12)
    assert np.allclose(O.block_scores(qh, 3.5 * wa, st), 3.5 * sa, rtol=1e-12, atol=1e-12)
    assert np.all(O.block_scores(qh, np.abs(wa), st) >= 0)
    # per-head brute force
    s = O.block_scores(qh, wa, st)
    for r in range(40):
        ref = sum(wa[i] * max(0.0, float(np.dot(qh[i], st[r]))) for i in range(4))
        assert abs(s[r] - ref) < 1e-12


# --------------------------------------------------------------------------
# step 3: selection
# --------------------------------------------------------------------------

def _brute_force_select(s, k):
    """The unique size-k subset whose every member beats every non-member
    under (score desc, block id asc); -1 padded."""
    b = len(s)
    if b <= k:
        return list(range(b)) + [-1] * (k - b)
    found = []
    for sub in itertools.combinations(range(b), k):
        inside = set(sub)
        if all((s[a] > s[c]) or (s[a] == s[c] and a < c)
               for a in inside for c in range(b) if c not in inside):
            found.append(list(sub))
    assert len(found) == 1
    return found[0]


def test_select_matches_brute_force_with_ties():
    rng = np.random.default_rng(13)
    for _ in range(300):
        b = int(rng.integers(0, 10))
        k = int(rng.integers(1, 6))
        s = rng.integers(-2, 3, b).astype(np.float64) * 0.5
        # mix in negative zeros: IEEE-equal to +0
        z = rng.random(b) < 0.3
        s[z] = -0.0 if rng.random() < 0.5 else 0.0
        got = O.select_blocks(s, k).tolist()
        assert got == _brute_force_select(s, k)


def test_select_all_ties_takes_lowest_ids_and_covers_small_rows():
    assert O.select_blocks(np.zeros(100), 16).tolist() == list(range(16))
    assert O.select_blocks(-np.zeros(100), 16).tolist() == list(range(16))
    s = np.random.default_rng(14).standard_normal(10)
    assert O.select_blocks(s, 16).tolist() == list(range(10)) + [-1] * 6
    assert O.select_blocks(np.zeros(0), 4).tolist() == [-1] * 4


def test_candidates_are_strictly_past_blocks():
    for t in range(0, 200):
        b = O.num_candidates(t, 8)
        assert 8 * b <= t < 8 * (b + 1)
        u = O.token_set(np.arange(b), t, 8)
        assert u.max() == t and np.array_equal(u, np.arange(t + 1))


# --------------------------------------------------------------------------
# step 4: attention
# --------------------------------------------------------------------------

def test_token_set_size_bound():
    pc = _golden("page_counts.json")
    sel = np.arange(600)[:512]
    for t in [8 * 600 + 7, 8 * 100_000 + 7]:
        assert O.token_set(sel, t, 8).size == pc["max_reads_per_query_group"]["value"]
    for j in range(8):
        assert O.token_set(sel, 8 * 600 + j, 8).size == 512 * 8 + j + 1


def _small_inputs(T, cfg, seed=0):
    rng = np.random.default_rng(seed)
    H, G, D, Hi, Di = cfg.num_q_heads, cfg.num_kv_groups, cfg.head_dim, cfg.idx_heads, cfg.idx_dim
    q = _bf16_bits(rng.standard_normal((T, H, D)))
    k = _bf16_bits(rng.standard_normal((T, G, D)))
    v = _bf16_bits(rng.standard_normal((T, G, D)))
    qi = _bf16_bits(rng.standard_normal((T, G, Hi, Di)))
    w = (rng.standard_normal((T, G, Hi)) / np.sqrt(512)).astype(np.float32)
    kp = _bf16_bits(rng.standard_normal((T, Di)))
    lg = rng.standard_normal((T, Di)).astype(np.float32)
    return q, k, v, qi, w, kp, lg


def _sdpa_causal_gqa(q, k, v, cfg):
    hg = cfg.heads_per_group
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]                       # [1,H,T,D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hg, 0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hg, 0)[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=cfg.softmax_scale)
    return o[0].permute(1, 0, 2).numpy()


def test_all_blocks_selected_equals_dense_causal_attention():
    cfg = O.Config(num_q_heads=8, num_kv_groups=2, head_dim=16, idx_dim=128,
                   block_size=4, topk_blocks=1000, store_q8=True)
    T = 48
    q, k, v, qi, w, kp, lg = _small_inputs(T, cfg)
    out = O.forward(cfg, q, k, v, qi, w, kp, lg)
    ref = _sdpa_causal_gqa(nu.bf16_bits_to_f64(q), nu.bf16_bits_to_f64(k), nu.bf16_bits_to_f64(v), cfg)
    assert np.allclose(out["o"], ref, rtol=1e-12, atol=1e-12)


def test_gather_equals_dense_mask_formulation():
    cfg = O.Config(num_q_heads=8, num_kv_groups=2, head_dim=16, block_size=4, topk_blocks=3)
    T = 64
    q, k, v, qi, w, kp, lg = _small_inputs(T, cfg, seed=1)
    out = O.forward(cfg, q, k, v, qi, w, kp, lg)
    qf, kf, vf = (nu.bf16_bits_to_f64(a) for a in (q, k, v))
    hg = cfg.heads_per_group
    for g in range(cfg.num_kv_groups):
        mask = np.zeros((T, T), dtype=bool)
        for t in range(T):
            for r in out["sel"][t, g]:
                if r >= 0:
                    mask[t, 4 * r:4 * r + 4] = True
            mask[t, 4 * (t // 4):t + 1] = True
        assert not np.any(np.triu(mask, 1))                 # never a future position
        qt = torch.from_numpy(qf[:, g * hg:(g + 1) * hg]).permute(1, 0, 2)[None]
        kt = torch.from_numpy(kf[:, g])[None, None].expand(1, hg, T, cfg.head_dim)
        vt = torch.from_numpy(vf[:, g])[None, None].expand(1, hg, T, cfg.head_dim)
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                           scale=cfg.softmax_scale)[0].permute(1, 0, 2).numpy()
        assert np.allclose(out["o"][:, g * hg:(g + 1) * hg], o, rtol=1e-12, atol=1e-12)


def test_attend_lse_closed_forms():
    # equal logits (q = 0): the normaliser over n tokens is ln(n) exactly;
    # one token: the logit itself; two tokens at z and z - ln 3 with z = 1000
    # (exp(z) overflows): z + ln(4/3), which needs the maximum term
    rng = np.random.default_rng(11)
    for n in (1, 7, 4104):
        k = rng.standard_normal((n, 16))
        v = rng.standard_normal((n, 16))
        o, lse = O.attend(np.zeros((3, 16)), k, v, 0.25)
        assert np.allclose(lse, math.log(n), rtol=0, atol=1e-12)
        assert np.allclose(o, v.mean(axis=0)[None, :], rtol=1e-12, atol=1e-12)
    q = rng.standard_normal((2, 8))
    k = rng.standard_normal((1, 8))
    _, lse = O.attend(q, k, rng.standard_normal((1, 8)), 0.5)
    assert np.allclose(lse, 0.5 * (q @ k[0]), rtol=1e-14, atol=1e-14)
    q = np.zeros((1, 2))
    q[0, 0] = 1.0
    k = np.array([[1000.0, 0.0], [1000.0 - math.log(3.0), 0.0]])
    o, lse = O.attend(q, k, np.eye(2), 1.0)
    assert np.isfinite(lse).all()
    assert abs(lse[0] - (1000.0 + math.log(4.0 / 3.0))) < 1e-9
    assert np.allclose(o[0], [0.75, 0.25], rtol=0, atol=1e-12)


def _masked_logsumexp(q, k, mask, scale):
    """torch.logsumexp over the scaled float64 logits of the allowed keys:
    q [T, h, D] against k [T, D] with mask [T, T] (query, key)."""
    z = torch.einsum("thd,ud->thu", torch.from_numpy(q), torch.from_numpy(k)) * scale
    z = z.masked_fill(~torch.from_numpy(mask)[:, None, :], float("-inf"))
    return torch.logsumexp(z, dim=-1).numpy()


def test_attend_lse_matches_library_logsumexp():
    # every block selected (dense causal, the t < B rows included) and a
    # sparse selection: the oracle's lse is the natural-log normaliser of
    # exactly the attended keys
    for topk, seed in ((1000, 4), (3, 5)):
        cfg = O.Config(num_q_heads=8, num_kv_groups=2, head_dim=16, block_size=4, topk_blocks=topk)
        T = 48
        q, k, v, qi, w, kp, lg = _small_inputs(T, cfg, seed=seed)
        out = O.forward(cfg, q, k, v, qi, w, kp, lg)
        qf, kf = nu.bf16_bits_to_f64(q), nu.bf16_bits_to_f64(k)
        hg = cfg.heads_per_group
        for g in range(cfg.num_kv_groups):
            mask = np.zeros((T, T), dtype=bool)
            for t in range(T):
                for r in out["sel"][t, g]:
                    if r >= 0:
                        mask[t, 4 * r:4 * r + 4] = True
                mask[t, 4 * (t // 4):t + 1] = True
            if topk == 1000:
                assert np.array_equal(mask, np.tril(np.ones((T, T), dtype=bool)))
            ref = _masked_logsumexp(qf[:, g * hg:(g + 1) * hg], kf[:, g], mask, cfg.softmax_scale)
            assert np.allclose(out["lse"][:, g * hg:(g + 1) * hg], ref, rtol=1e-13, atol=1e-13)
        # row 0 attends to itself only
        z0 = (qf[0, 0] @ kf[0, 0]) * cfg.softmax_scale
        assert abs(out["lse"][0, 0] - z0) < 1e-13


def test_future_tokens_do_not_change_a_query():
    cfg = O.Config(num_q_heads=8, num_kv_groups=2, head_dim=16, block_size=4, topk_blocks=2)
    T = 40
    a = _small_inputs(T, cfg, seed=2)
    out_a = O.forward(cfg, *a)
    t0 = 21                                     # inside block 5, which completes at 23
    rng = np.random.default_rng(99)
    b = [x.copy() for x in a]
    for x in b:                                 # perturb every input at positions > t0
        flat = x[t0 + 1:]
        if x.dtype == np.uint16:
            flat[...] = _bf16_bits(rng.standard_normal(flat.shape))
        else:
            flat[...] = rng.standard_normal(flat.shape).astype(np.float32)
    out_b = O.forward(cfg, *b)
    assert np.array_equal(out_a["o"][:t0 + 1], out_b["o"][:t0 + 1])
    assert np.array_equal(out_a["sel"][:t0 + 1], out_b["sel"][:t0 + 1])


def test_forward_internal_consistency():
    cfg = O.Config(num_q_heads=16, num_kv_groups=1, head_dim=8, block_size=2, topk_blocks=3,
                   store_q8=False)
    T = 30
    q, k, v, qi, w, kp, lg = _small_inputs(T, cfg, seed=3)
    out = O.forward(cfg, q, k, v, qi, w, kp, lg)
    for t in range(T):
        s = out["scores"][t][0]
        assert s.shape == (t // 2,)
        assert np.array_equal(out["sel"][t, 0], O.select_blocks(s, 3))
        assert np.all(out["sel"][t, 0][out["sel"][t, 0] >= 0] < t // 2)


# --------------------------------------------------------------------------
# counts the pages print
# --------------------------------------------------------------------------

def test_page_counts():
    pc = _golden("page_counts.json")
    cfg = O.Config()
    T = 1 << 20
    assert T // cfg.block_size == pc["summaries_at_1m"]["value"]
    assert round(T / pc["max_reads_per_query_group"]["value"], 1) == pc["read_ratio_at_1m"]["value"]
    R = O.num_candidates(T - 1, cfg.block_size)
    assert R == pc["score_matrix_candidates_R"]["value"]
    gib = 1 * T * R * 4 / 2 ** 30
    assert round(gib, 6) == pc["score_matrix_gib"]["value"]
    kv_bytes = 2 * cfg.num_kv_groups * cfg.head_dim * 2
    assert kv_bytes == pc["kv_bytes_per_token_layer"]["value"]
    n_global, n_local, ring = 23, 69, 512
    global_kv = n_global * T * kv_bytes
    local_kv = n_local * ring * kv_bytes
    store = n_global * (T // cfg.block_size) * cfg.idx_dim * 2     # bf16 containers of E4M3 values
    assert global_kv == pc["global_kv_gib"]["value"] * 2 ** 30
    assert local_kv == pc["local_ring_mib"]["value"] * 2 ** 20
    assert store == pc["summary_store_mib"]["value"] * 2 ** 20
    total = (2 * (global_kv + local_kv) + 8 * store) / 2 ** 30
    assert round(total, 6) == pc["payload_tp8_gib"]["value"]


# ---------------------------------------------------------------------------
# the path's neighbours: main Q/K norm + partial rotary span, sigmoid gate
# ---------------------------------------------------------------------------

def test_main_qk_is_library_rms_norm_then_rotation():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((5, 7, 192)).astype(np.float32)
    xb = _bf16_bits(x)
    gam = _bf16_bits(rng.uniform(0.5, 1.5, 192))
    pos = np.array([0, 3, 100, 4095, 262143])
    xf = torch.from_numpy(nu.bf16_bits_to_f64(xb))
    gf = torch.from_numpy(nu.bf16_bits_to_f64(gam))
    normed = F.rms_norm(xf, (192,), weight=gf, eps=1e-6).numpy()
    # span 0: the library norm alone
    plain = O.main_qk(xb, pos, 0, 10000.0, 1e-6, gam)
    assert np.allclose(plain, normed, rtol=1e-13, atol=1e-13)
    for span, base in [(64, 10000.0), (96, 1e6), (192, 500.0)]:
        out = O.main_qk(xb, pos, span, base, 1e-6, gam)
        ref = _rope_complex(normed, np.broadcast_to(pos[:, None], normed.shape[:2]), span, base)
        # the two frequency formulas differ by an ulp of theta: a phase error
        # of about pos * 2.2e-16 (6e-11 rad at position 262143)
        assert np.allclose(out, ref, rtol=0, atol=1e-9)
        assert np.array_equal(out[..., span:], plain[..., span:])        # dims past the span pass through
        assert np.allclose(np.linalg.norm(out[..., :span], axis=-1),
                           np.linalg.norm(normed[..., :span], axis=-1), rtol=1e-12)


def test_main_qk_scores_depend_on_relative_position():
    rng = np.random.default_rng(22)
    q = _bf16_bits(rng.standard_normal((1, 1, 192)))
    k = _bf16_bits(rng.standard_normal((1, 1, 192)))
    span = 64
    dots = []
    for t, s in [(10, 3), (1007, 1000), (65543, 65536)]:
        qa = O.main_qk(q, np.array([t]), span, 10000.0, 1e-6)
        ka = O.main_qk(k, np.array([s]), span, 10000.0, 1e-6)
        dots.append(float((qa[0, 0, :span] * ka[0, 0, :span]).sum()))
    assert np.allclose(dots, dots[0], rtol=1e-9, atol=1e-9)


def test_gate_is_library_sigmoid_and_exact_at_zero():
    rng = np.random.default_rng(23)
    o = rng.standard_normal((3, 16, 192))
    g = _bf16_bits(rng.standard_normal((3, 16, 192)) * 4)
    ref = o * torch.sigmoid(torch.from_numpy(nu.bf16_bits_to_f64(g))).numpy()
    assert np.allclose(O.gate(o, g), ref, rtol=1e-13, atol=1e-15)
    zero = np.zeros((3, 16, 192), dtype=np.uint16)
    assert np.array_equal(O.gate(o, zero), o / 2)                        # sigmoid(0) = 1/2 exactly
    big = _bf16_bits(np.full((3, 16, 192), 64.0))
    assert np.allclose(O.gate(o, big), o, rtol=1e-27)
    assert np.allclose(O.gate(o, _bf16_bits(np.full((3, 16, 192), -64.0))), 0.0, atol=1e-27)
