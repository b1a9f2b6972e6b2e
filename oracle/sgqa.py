"""Float64 definition of the sparse GQA global-attention path.

Sources (the pages, by title and section):

* P1 = "Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache"
  - "Two paths leave the same hidden state": Q is N x 64 x 192, K/V are
    N x 4 x 192; four provider groups share one compressed proxy-key store and
    score it separately; group g serves the 16 query heads of KV group g;
    indexer queries use RMSNorm, proxy keys LayerNorm, both a 32-dim rotary
    span; compression logits are a separate projection.
  - "Eight tokens become one search key, coordinate by coordinate": per
    completed 8-token block and per proxy coordinate d, a max-subtracted
    softmax of that coordinate's compression logits over the 8 tokens weights
    the tokens' coordinate d; FP32 accumulation, stored through BF16 into
    E4M3.
  - "Selection is a weighted ReLU score, not attention softmax": the score of
    block r for query t and group g sums, over the group's four indexer heads,
    a signed weight times ReLU of the query/summary dot product (ReLU inside
    the sum, no softmax, summaries E4M3-rounded then widened to BF16 for a
    BF16 matmul); only blocks r < floor(t/8) compete for the 512 historical
    slots; equal scores go to the lower block ID; the current block is
    appended, restricted to positions <= t.
  - "Main attention still reads original K/V": head h uses group
    g(h) = floor(h/16) and an ordinary scaled-dot-product softmax over the
    selected original tokens.
  - "What gets cheaper, and what stays length-dependent?": at most
    512*8 + 8 = 4,104 original positions per query and group.
* P2 = the Step 5 Preview architecture-blog summary: block size 8, final
  setting B=8 with k=4096 tokens, ablation B=1 with k=2048 tokens.

Readings where the pages are silent (each listed in the design notes):

* LayerNorm, then RoPE at the token's own position, then the merge (the lost
  compression equation; the coordinate-wise range statement refers to the
  keys being merged).  Parity unpinned against the real model.
* RoPE on dims [0, rope_dim), half-split pairs (j, j + rope_dim/2), angle
  pos * base**(-2j/rope_dim); llama3 scaling with factor 1.0 is the identity.
  Parity unpinned against the real model (the relative-position property is
  pinned).
* Population variance in LayerNorm; epsilons from the config; affine
  parameters optional (identity when absent).
* Selection emitted in ascending block ID, padded with -1; "equal" is IEEE
  equality (-0 == +0).
* A token in block 0 (t < B) has no historical candidates.
* Neighbours of the path: the main Q/K RMSNorm is per head over D with one
  gamma shared by the heads, epsilon eps_rms; the main rotary span uses the
  indexer's convention (half-split pairs, base**(-2j/span)) with span and
  base as parameters; the gate is elementwise over the head vector with
  caller-supplied logits.  Parity unpinned against the real model (span,
  gate shape); the norm, rotation and sigmoid are pinned.

Conventions: bf16 tensors arrive as uint16 bit arrays, fp32 tensors as
float32 arrays; everything is widened exactly to float64 and computed in
float64.  Only the two roundings the pages fix are applied: the store
rounding and the BF16 indexer query of the BF16 score matmul.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import bf16_bits_to_f64, q8, round_bf16, to_f32


@dataclass(frozen=True)
class Config:
    num_q_heads: int = 64
    num_kv_groups: int = 4
    head_dim: int = 192
    idx_heads: int = 4
    idx_dim: int = 128
    rope_dim: int = 32
    rope_base: float = 10000.0
    block_size: int = 8
    topk_blocks: int = 512
    softmax_scale: float = float(np.float32(1.0 / np.sqrt(192.0)))
    eps_rms: float = 1e-6
    eps_ln: float = 1e-6
    store_q8: bool = True

    @property
    def heads_per_group(self) -> int:
        return self.num_q_heads // self.num_kv_groups


# --------------------------------------------------------------------------
# norms and rotary span (P1, "Two paths leave the same hidden state")
# --------------------------------------------------------------------------

def layer_norm(x: np.ndarray, eps: float, gamma=None, beta=None) -> np.ndarray:
    """LayerNorm over the last axis with population variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * gamma
    if beta is not None:
        y = y + beta
    return y


def rms_norm(x: np.ndarray, eps: float, gamma=None) -> np.ndarray:
    """RMSNorm over the last axis."""
    y = x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    if gamma is not None:
        y = y * gamma
    return y


def rope(y: np.ndarray, pos, rope_dim: int, base: float) -> np.ndarray:
    """Rotate pairs (j, j + rope_dim/2), j < rope_dim/2, of the last axis by
    pos * base**(-2j/rope_dim); dims >= rope_dim pass through."""
    half = rope_dim // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / rope_dim)
    phi = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(phi), np.sin(phi)
    a = y[..., :half]
    b = y[..., half:rope_dim]
    out = np.array(y, dtype=np.float64, copy=True)
    out[..., :half] = a * c - b * s
    out[..., half:rope_dim] = a * s + b * c
    return out


# --------------------------------------------------------------------------
# step 1: block-wise token merging (P1, "Eight tokens become one search key")
# --------------------------------------------------------------------------

def proxy_keys(kp_bits: np.ndarray, positions: np.ndarray, cfg: Config,
               ln_gamma=None, ln_beta=None) -> np.ndarray:
    """k_hat[s] = RoPE_s(LayerNorm(kp[s])) for raw bf16 proxy keys [n, Di]."""
    x = bf16_bits_to_f64(kp_bits)
    y = layer_norm(x, cfg.eps_ln, ln_gamma, ln_beta)
    return rope(y, positions, cfg.rope_dim, cfg.rope_base)


def merge(k_hat: np.ndarray, logits: np.ndarray) -> np.ndarray:
    """Blocks [..., B, Di] -> summaries [..., Di]: for every coordinate d, the
    softmax over the block's B tokens of logits[..., :, d] (the common
    maximum subtracted first) weights k_hat[..., :, d]."""
    m = logits.max(axis=-2, keepdims=True)
    a = np.exp(logits - m)
    return (a * k_hat).sum(axis=-2) / a.sum(axis=-2)


def compress(kp_bits: np.ndarray, logits: np.ndarray, blocks, cfg: Config,
             ln_gamma=None, ln_beta=None, chunk: int = 8192):
    """Store rows for the listed blocks of one sequence.

    ``kp_bits`` [T, Di] (bf16 bits) and ``logits`` [T, Di] (fp32) hold the
    sequence's tokens from position 0.  Returns ``(stored, exact)``: the
    stored values (fp32 result rounded to bf16, then to E4M3 when
    ``store_q8``) and the unrounded float64 summaries, both [len(blocks), Di].
    Blocks are processed ``chunk`` at a time only to bound memory.
    """
    B = cfg.block_size
    blocks = np.asarray(blocks, dtype=np.int64).reshape(-1)
    exact = np.empty((blocks.size, cfg.idx_dim), dtype=np.float64)
    for c0 in range(0, blocks.size, chunk):
        r = blocks[c0:c0 + chunk]
        pos = (r[:, None] * B + np.arange(B)[None, :])               # [n, B]
        k_hat = proxy_keys(kp_bits[pos.reshape(-1)], pos.reshape(-1), cfg, ln_gamma, ln_beta)
        lg = np.asarray(logits[pos.reshape(-1)], dtype=np.float64)
        exact[c0:c0 + chunk] = merge(k_hat.reshape(r.size, B, -1), lg.reshape(r.size, B, -1))
    stored = q8(exact) if cfg.store_q8 else round_bf16(exact)
    return stored, exact


# --------------------------------------------------------------------------
# step 2: indexer scoring (P1, "Selection is a weighted ReLU score")
# --------------------------------------------------------------------------

def index_queries(qi_bits: np.ndarray, positions: np.ndarray, cfg: Config,
                  rms_gamma=None, exact: bool = False) -> np.ndarray:
    """q_hat = bf16(RoPE_t(RMSNorm(qi))) for raw queries [n, G, Hi, Di].
    With ``exact`` the float64 value before the bf16 rounding is returned."""
    x = bf16_bits_to_f64(qi_bits)
    y = rms_norm(x, cfg.eps_rms, rms_gamma)
    pos = np.asarray(positions, dtype=np.float64).reshape((-1,) + (1,) * (x.ndim - 2))
    y = rope(y, pos, cfg.rope_dim, cfg.rope_base)
    return y if exact else round_bf16(y)


def block_scores(q_hat: np.ndarray, w: np.ndarray, store: np.ndarray) -> np.ndarray:
    """s[r] = sum_i w[i] * max(0, q_hat[i] . store[r]) for one (query, group):
    q_hat [Hi, Di], w [Hi], store [b, Di] (the candidate blocks)."""
    dots = store @ q_hat.T                       # [b, Hi]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


# --------------------------------------------------------------------------
# step 3: causal top-k block selection (P1, "Selection is a weighted ReLU score")
# --------------------------------------------------------------------------

def num_candidates(t: int, block_size: int) -> int:
    """Historical blocks that may compete for query position t: r < floor(t/B)."""
    return int(t) // int(block_size)


def select_blocks(scores: np.ndarray, k: int) -> np.ndarray:
    """The k candidates with the largest score, equal scores to the lower
    block ID; all candidates when there are at most k.  Ascending IDs, -1 pad."""
    b = scores.shape[0]
    out = np.full(k, -1, dtype=np.int64)
    if b <= k:
        out[:b] = np.arange(b)
        return out
    s = np.asarray(scores, dtype=np.float64) + 0.0      # -0.0 -> +0.0
    order = np.lexsort((np.arange(b), -s))              # score desc, then id asc
    out[:] = np.sort(order[:k])
    return out


# --------------------------------------------------------------------------
# step 4: sparse GQA attention (P1, "Main attention still reads original K/V")
# --------------------------------------------------------------------------

def token_set(sel_row: np.ndarray, t: int, block_size: int) -> np.ndarray:
    """Original positions attended by query t: every token of the selected
    blocks plus the current block's tokens up to t, ascending."""
    B = int(block_size)
    blocks = np.asarray(sel_row, dtype=np.int64)
    blocks = blocks[blocks >= 0]
    hist = (blocks[:, None] * B + np.arange(B)[None, :]).reshape(-1)
    cur = np.arange(B * (int(t) // B), int(t) + 1)
    return np.concatenate([hist, cur])


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Exact softmax attention of the rows of q [h, D] over k, v [u, D].
    Returns (o [h, D], lse [h]) with lse the natural-log normaliser."""
    z = (q @ k.T) * scale
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ v) / l
    return o, (m + np.log(l))[:, 0]


# --------------------------------------------------------------------------
# the path's neighbours.  P1 "Two paths leave the same hidden state": the
# main path normalizes Q and K and applies the layer's partial RoPE (its
# span is head_dim times a partial-rotary factor the pages do not give, so
# it is a parameter).  P1 "Main attention still reads original K/V": each
# head's output vector is sigmoid-gated before concatenation and the output
# projection.
# --------------------------------------------------------------------------

def main_qk(x_bits: np.ndarray, positions: np.ndarray, rope_dim: int, rope_base: float,
            eps: float, gamma_bits=None) -> np.ndarray:
    """Main-path Q (or K) rows: x [n, heads, D] bf16 bits at token positions
    [n]; RMSNorm over each head's D dims (one gamma [D] shared by the heads),
    then the rotary span [0, rope_dim) at the token's position.  Exact
    (float64, not rounded)."""
    x = bf16_bits_to_f64(x_bits)
    g = bf16_bits_to_f64(gamma_bits) if gamma_bits is not None else None
    y = rms_norm(x, eps, g)
    pos = np.broadcast_to(np.asarray(positions, dtype=np.float64)[:, None], y.shape[:2])
    return rope(y, pos, rope_dim, rope_base)


def gate(o: np.ndarray, gate_bits: np.ndarray) -> np.ndarray:
    """A head's output vector times sigmoid of its gate logits, elementwise."""
    g = bf16_bits_to_f64(gate_bits)
    return o / (1.0 + np.exp(-g))


# --------------------------------------------------------------------------
# one query row through steps 2-4, and a whole small sequence
# --------------------------------------------------------------------------

def query_row(cfg: Config, t: int, q_hat_t: np.ndarray, w_t: np.ndarray,
              store: np.ndarray, q_t: np.ndarray, k_seq: np.ndarray,
              v_seq: np.ndarray):
    """Steps 2-4 for query position t of one sequence.

    q_hat_t [G, Hi, Di] (bf16-valued float64), w_t [G, Hi], store [>=b(t), Di]
    (stored values), q_t [H, D], k_seq / v_seq [>t, G, D] (float64 values of
    the caches from position 0).  Returns dict with per-group ``scores``
    (list of [b(t)] arrays), ``sel`` [G, K], ``o`` [H, D], ``lse`` [H].
    """
    G, hg = cfg.num_kv_groups, cfg.heads_per_group
    b = num_candidates(t, cfg.block_size)
    sel = np.empty((G, cfg.topk_blocks), dtype=np.int64)
    o = np.empty((cfg.num_q_heads, cfg.head_dim))
    lse = np.empty(cfg.num_q_heads)
    scores = []
    for g in range(G):
        s = block_scores(q_hat_t[g], w_t[g], store[:b])
        scores.append(s)
        sel[g] = select_blocks(s, cfg.topk_blocks)
        u = token_set(sel[g], t, cfg.block_size)
        heads = slice(g * hg, (g + 1) * hg)
        o[heads], lse[heads] = attend(q_t[heads], k_seq[u, g], v_seq[u, g], cfg.softmax_scale)
    return {"scores": scores, "sel": sel, "o": o, "lse": lse}


def forward(cfg: Config, q_bits, k_bits, v_bits, qi_bits, w, kp_bits, logits,
            pos0: int = 0, ln_gamma=None, ln_beta=None, rms_gamma=None):
    """All four steps for one sequence whose caches start at position 0.

    Shapes: q_bits [n, H, D], qi_bits [n, G, Hi, Di], w [n, G, Hi] for the n
    new queries at positions pos0..pos0+n-1; k_bits / v_bits [T, G, D],
    kp_bits / logits [T, Di] for T = pos0 + n cached tokens.
    Returns dict: store, store_exact, q_hat, scores, sel, o, lse.
    """
    n = q_bits.shape[0]
    T = pos0 + n
    B = cfg.block_size
    store, store_exact = compress(kp_bits, logits, np.arange(T // B), cfg, ln_gamma, ln_beta)
    positions = np.arange(pos0, T)
    q_hat = index_queries(qi_bits, positions, cfg, rms_gamma)
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    wf = np.asarray(w, dtype=np.float64)
    sel = np.empty((n, cfg.num_kv_groups, cfg.topk_blocks), dtype=np.int64)
    o = np.empty((n, cfg.num_q_heads, cfg.head_dim))
    lse = np.empty((n, cfg.num_q_heads))
    scores = []
    for i, t in enumerate(positions):
        r = query_row(cfg, int(t), q_hat[i], wf[i], store, q[i], k, v)
        sel[i], o[i], lse[i] = r["sel"], r["o"], r["lse"]
        scores.append(r["scores"])
    return {"store": store, "store_exact": store_exact, "q_hat": q_hat,
            "scores": scores, "sel": sel, "o": o, "lse": lse}


__all__ = [
    "Config", "layer_norm", "rms_norm", "rope", "proxy_keys", "merge", "compress",
    "index_queries", "block_scores", "num_candidates", "select_blocks", "token_set",
    "attend", "query_row", "forward", "to_f32",
]
