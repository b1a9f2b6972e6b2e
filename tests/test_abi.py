"""The C ABI without a GPU: every symbol include/sgqa.h declares is exported,
and every rejected call returns its status before any HIP call.

Every call here is invalid by construction (a NULL or inconsistent argument
that validation rejects first), so none of them can reach a kernel launch.
"""
import ctypes
import math
import os
import re

import pytest

import sparse_long_context_block_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgqa.h")

OK, E_NULL, E_CONFIG, E_SHAPE, E_CAUSAL, E_CAPACITY, E_WS, E_UNSUP, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8
FAKE = 0x100000          # a non-NULL pointer value; never dereferenced (calls fail validation)


@pytest.fixture(scope="module")
def L():
    return sg.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgqa_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported(L):
    names = declared_functions()
    assert set(names) >= {"sgqa_compress", "sgqa_index_topk", "sgqa_sparse_attn", "sgqa_forward",
                          "sgqa_workspace_size", "sgqa_status_string", "sgqa_last_error",
                          "sgqa_abi_version"}
    for n in names:
        assert hasattr(L, n), f"{n} not exported by libsgqa.so"


def test_version_and_status_strings(L):
    assert L.sgqa_abi_version() == 1
    for code, name in [(OK, b"SGQA_OK"), (E_NULL, b"SGQA_ERR_NULL"), (E_CONFIG, b"SGQA_ERR_CONFIG"),
                       (E_SHAPE, b"SGQA_ERR_SHAPE"), (E_CAUSAL, b"SGQA_ERR_CAUSAL"),
                       (E_CAPACITY, b"SGQA_ERR_CAPACITY"), (E_WS, b"SGQA_ERR_WORKSPACE"),
                       (E_UNSUP, b"SGQA_ERR_UNSUPPORTED"), (E_HIP, b"SGQA_ERR_HIP")]:
        assert L.sgqa_status_string(code) == name
    assert L.sgqa_status_string(12345) == b"SGQA_UNKNOWN_STATUS"


def _seqs(*seqs):
    arr = (sg.Seq * len(seqs))(*seqs)
    return arr, len(seqs)


def _call_attn(L, cfg, seqs, n=None, q=None, k=None, v=None, sel=None, out=None, ws=None, ws_bytes=0):
    arr, m = _seqs(*seqs) if seqs else (None, 0)
    return L.sgqa_sparse_attn(ctypes.byref(cfg) if cfg is not None else None, arr,
                              m if n is None else n, q, k, v, sel, out, None, ws, ws_bytes, None)


def _good_seq(n_q=8, pos0=0):
    return sg.seq(n_q, pos0=pos0)


# config and sequence errors are reported before pointers are looked at, so
# all tensor pointers below are NULL

@pytest.mark.parametrize("field,value,code", [
    ("num_q_heads", 0, E_CONFIG), ("num_q_heads", 65, E_CONFIG), ("rope_dim", 31, E_CONFIG),
    ("rope_dim", 256, E_CONFIG), ("store_q8", 3, E_CONFIG), ("store_q8", -1, E_CONFIG), ("softmax_scale", math.nan, E_CONFIG),
    ("softmax_scale", -1.0, E_CONFIG), ("eps_rms", -1.0, E_CONFIG), ("rope_base", 0.0, E_CONFIG),
    ("topk_blocks", 0, E_CONFIG), ("block_size", 0, E_CONFIG),
    ("head_dim", 128, E_UNSUP), ("idx_dim", 64, E_UNSUP), ("num_kv_groups", 8, E_UNSUP),
    ("idx_heads", 2, E_UNSUP), ("rope_dim", 64, E_UNSUP), ("block_size", 3, E_UNSUP),
    ("block_size", 32, E_UNSUP), ("topk_blocks", 3073, E_UNSUP),
])
def test_config_errors(L, field, value, code):
    cfg = sg.config()
    setattr(cfg, field, value)
    assert _call_attn(L, cfg, [_good_seq()]) == code
    assert field.split("_")[0] in L.sgqa_last_error().decode() or code in (E_UNSUP, E_CONFIG)


def test_null_config_and_seqs(L):
    assert _call_attn(L, None, [_good_seq()]) == E_NULL
    cfg = sg.config()
    assert L.sgqa_sparse_attn(ctypes.byref(cfg), None, 1, None, None, None, None, None, None,
                              None, 0, None) == E_NULL
    assert _call_attn(L, cfg, [_good_seq()], n=0) == E_SHAPE


@pytest.mark.parametrize("mutate,code", [
    (lambda s: setattr(s, "n_q", -1), E_SHAPE),
    (lambda s: setattr(s, "kv_offset", -5), E_SHAPE),
    (lambda s: setattr(s, "q_offset", 1 << 41), E_SHAPE),
    (lambda s: setattr(s, "cache_len", s.cache_len + 1), E_CAUSAL),
    (lambda s: setattr(s, "kv_capacity", s.cache_len - 1), E_CAPACITY),
    (lambda s: setattr(s, "store_capacity", s.cache_len // 8 - 1), E_CAPACITY),
])
def test_sequence_errors(L, mutate, code):
    s = sg.seq(64, pos0=100)
    mutate(s)
    assert _call_attn(L, sg.config(), [sg.seq(8), s]) == code
    assert "seqs[1]" in L.sgqa_last_error().decode()


def test_null_tensors(L):
    cfg = sg.config()
    arr, n = _seqs(_good_seq())
    P = ctypes.c_void_p(FAKE)
    # compress: proxy_k, comp_logits, store required
    assert L.sgqa_compress(ctypes.byref(cfg), arr, n, None, P, None, None, P, None, 0, None) == E_NULL
    assert L.sgqa_compress(ctypes.byref(cfg), arr, n, P, None, None, None, P, None, 0, None) == E_NULL
    assert L.sgqa_compress(ctypes.byref(cfg), arr, n, P, P, None, None, None, None, 0, None) == E_NULL
    # index_topk: q_idx, w, store, sel required
    for missing in range(4):
        a = [P, P, P, P]
        a[missing] = None
        assert L.sgqa_index_topk(ctypes.byref(cfg), arr, n, a[0], a[1], None, a[2], a[3], None,
                                 None, None, 0, None) == E_NULL
    # sparse_attn: q, k, v, sel, out required
    for missing in range(5):
        a = [P] * 5
        a[missing] = None
        assert L.sgqa_sparse_attn(ctypes.byref(cfg), arr, n, *a, None, None, 0, None) == E_NULL
    # forward: ten required pointers
    req = [3, 4, 7, 8, 9, 11, 13, 14, 15, 16]     # proxy_k, logits, store, q_idx, w, sel, q, k, v, out
    for missing in req:
        args = [ctypes.byref(cfg), arr, n] + [None] * 18
        for i in req:
            args[i] = P
        args[19] = 0                              # ws_bytes
        args[missing] = None
        assert L.sgqa_forward(*args) == E_NULL


def test_workspace_errors(L):
    # one decode query over a long cache needs split workspace
    cfg = sg.config()
    seqs = [sg.seq(1, pos0=200_000)]
    need = sg.workspace_size(cfg, seqs, sg.OP_SPARSE_ATTN)
    need_i = sg.workspace_size(cfg, seqs, sg.OP_INDEX_TOPK)
    need_f = sg.workspace_size(cfg, seqs, sg.OP_FORWARD)
    assert need > 0 and need_i > 0 and need_f >= max(need, need_i)
    P = ctypes.c_void_p(FAKE)
    arr, n = _seqs(*seqs)
    assert L.sgqa_sparse_attn(ctypes.byref(cfg), arr, n, P, P, P, P, P, None, None, need, None) == E_WS
    assert L.sgqa_sparse_attn(ctypes.byref(cfg), arr, n, P, P, P, P, P, None, P, need - 1, None) == E_WS
    assert L.sgqa_sparse_attn(ctypes.byref(cfg), arr, n, P, P, P, P, P, None,
                              ctypes.c_void_p(FAKE + 8), need, None) == E_WS
    assert L.sgqa_index_topk(ctypes.byref(cfg), arr, n, P, P, None, P, P, None, None, P, need_i - 1,
                             None) == E_WS
    assert "workspace" in L.sgqa_last_error().decode()


def test_workspace_size_invalid_args_is_zero(L):
    cfg = sg.config(block_size=3)
    assert sg.workspace_size(cfg, [_good_seq()], sg.OP_FORWARD) == 0
    assert "block_size" in L.sgqa_last_error().decode()
    assert sg.workspace_size(sg.config(), [_good_seq()], 7) == 0


def test_prefill_key_workspace(L):
    # prefills of 1024+ queries keep 4-byte score keys per (row, group,
    # candidate), each query's 16 x 128 bf16 indexer rows, a list of rows
    # to score again (a count and one word per row and group, rounded up to
    # 256 B) and the 256-byte diagnostics block in the workspace; compression
    # and attention need none
    cfg = sg.config()
    # key rows: 1023 candidates padded to 1088 (64 x an odd count)
    diag = 8192 * 4 * 1088 * 4 + 8192 * 16 * 128 * 2 + (1 + 8192 * 4) * 4 // 256 * 256 + 256
    need = diag + 256
    assert sg.workspace_size(cfg, [sg.seq(8192)], sg.OP_INDEX_TOPK) == need
    assert sg.workspace_size(cfg, [sg.seq(8192)], sg.OP_FORWARD) == need
    assert sg.index_diag_offset(cfg, [sg.seq(8192)]) == diag
    # decode-sized calls keep no diagnostics block
    assert sg.index_diag_offset(cfg, [sg.seq(1, pos0=200_000)]) is None
    assert sg.index_diag_offset(sg.config(block_size=3), [sg.seq(8192)]) is None
    assert sg.workspace_size(cfg, [sg.seq(8192)], sg.OP_COMPRESS) == 0
    assert sg.workspace_size(cfg, [sg.seq(8192)], sg.OP_SPARSE_ATTN) == 0
    # long prefills run in passes over query rows: the keys stay within 4 GiB
    cfg1 = sg.config(block_size=1, topk_blocks=2048)
    seqs1 = [sg.seq(65536, block_size=1)]
    ws_idx = sg.workspace_size(cfg1, seqs1, sg.OP_INDEX_TOPK)
    assert (1 << 20) * 16 <= ws_idx <= (1 << 32) + (1 << 25)
    # the forward call runs in pieces: a piece's keys, then the gather's
    # partial results, then the diagnostics block
    ws = sg.workspace_size(cfg1, seqs1, sg.OP_FORWARD)
    assert ws_idx <= ws <= ws_idx + sg.workspace_size(cfg1, seqs1, sg.OP_SPARSE_ATTN) + (1 << 20)
    assert sg.forward_diag_offset(cfg1, seqs1) == ws - 256


def test_forward_pieces_workspace(L):
    # a chunk of 8,192 queries over a 1M-token cache runs in pieces: its
    # forward workspace holds the pieces' index region (a piece's key rows,
    # not the whole call's), their attention region (none: no split) and one
    # diagnostics block at the end, apart from the index call's layout
    cfg = sg.config()
    chunk = [sg.seq(8192, pos0=1_040_384)]
    fwd = sg.workspace_size(cfg, chunk, sg.OP_FORWARD)
    idx = sg.workspace_size(cfg, chunk, sg.OP_INDEX_TOPK)
    assert sg.workspace_size(cfg, chunk, sg.OP_SPARSE_ATTN) == 0
    assert 0 < fwd < idx
    assert sg.forward_diag_offset(cfg, chunk) == fwd - 256
    assert sg.index_diag_offset(cfg, chunk) == idx - 256
    # the last (longest) piece of 1,024 queries: keys of 131,071 candidates
    # in rows of 131,136 (64 x an odd count), its indexer rows, the failed-row
    # list
    piece = 1024 * 4 * 131136 * 4 + 1024 * 16 * 128 * 2 + (1 + 1024 * 4) * 4 // 256 * 256 + 256 + 256
    assert fwd == piece + 256
    # calls that are not split (dense-ish queries, or too few queries) keep
    # the index call's layout
    for seqs in ([sg.seq(8192)], [sg.seq(2047, pos0=1_040_384)], [sg.seq(1, pos0=200_000)]):
        assert sg.forward_diag_offset(cfg, seqs) == sg.index_diag_offset(cfg, seqs)
        assert sg.workspace_size(cfg, seqs, sg.OP_FORWARD) == max(
            sg.workspace_size(cfg, seqs, sg.OP_INDEX_TOPK), sg.workspace_size(cfg, seqs, sg.OP_SPARSE_ATTN))


def test_workspace_ignores_query_row_offsets(L):
    # workspace rows are numbered per launch, so the size follows the queries
    # a launch holds, not where their rows sit in the caller's tensors (a
    # decode loop keeps every step's rows in one output buffer)
    cfg = sg.config()
    for op in (sg.OP_INDEX_TOPK, sg.OP_SPARSE_ATTN, sg.OP_FORWARD):
        for n_seq, n_q, pos0 in [(64, 1, 200_000), (2, 1, 200_000), (3, 600, 20_000)]:
            packed = [sg.seq(n_q, pos0=pos0, q_offset=n_q * i) for i in range(n_seq)]
            spread = [sg.seq(n_q, pos0=pos0, q_offset=5000 * n_q + 80 * n_q * i) for i in range(n_seq)]
            assert sg.workspace_size(cfg, packed, op) == sg.workspace_size(cfg, spread, op)
    # 64 decode queries: keys of 64 rows x 4 groups x 25024 candidates (25000
    # blocks padded to 64 x an odd count)
    spread = [sg.seq(1, pos0=200_000, q_offset=4000 + 80 * i) for i in range(64)]
    assert sg.workspace_size(cfg, spread, sg.OP_INDEX_TOPK) == 64 * 4 * 25024 * 4


def test_paged_calls_validate_the_page_table(L):
    # kv_offset indexes the sequence's first page-table entry; its
    # ceil(kv_capacity / 16) entries must lie inside the table
    cfg = sg.config()
    P = ctypes.c_void_p(FAKE)
    s = sg.seq(100, pos0=900, kv_offset=10, kv_capacity=1000)   # 63 pages: entries 10..72
    arr, n = _seqs(s)
    attn = lambda pt, ln, npg: L.sgqa_sparse_attn_paged(ctypes.byref(cfg), arr, n, P, P, P, pt, ln,
                                                        npg, P, P, None, None, None, 0, None)
    assert attn(None, 73, 8) == E_NULL
    assert attn(P, 72, 8) == E_CAPACITY
    assert "page-table entries 10 .. 72" in L.sgqa_last_error().decode()
    assert attn(P, 73, 0) == E_SHAPE
    assert attn(P, 0, 8) == E_SHAPE
    assert attn(P, 73, (1 << 27) + 1) == E_SHAPE
    comp = lambda pt, ln: L.sgqa_compress_paged(ctypes.byref(cfg), arr, n, P, P, pt, ln, 8, None, None,
                                                P, None, 0, None)
    assert comp(None, 73) == E_NULL
    assert comp(P, 72) == E_CAPACITY
    args = [ctypes.byref(cfg), arr, n] + [P] * 13 + [P, 72, 8, P, None, None, None, 0, None]
    assert L.sgqa_forward_paged(*args) == E_CAPACITY
    args[16] = None
    assert L.sgqa_forward_paged(*args) == E_NULL


def test_neighbour_calls_validate(L):
    cfg = sg.config()
    P = ctypes.c_void_p(FAKE)
    arr, n = _seqs(sg.seq(16, pos0=48))
    qk = sg.qk_config(rope_dim=64)
    prep = lambda qkc, *ptrs: L.sgqa_qk_prep(ctypes.byref(cfg), ctypes.byref(qkc) if qkc else None, arr, n,
                                             *ptrs, None, 0, 0, None)
    full = [P, P, P, None, None, P, P, P]
    assert prep(None, *full) == E_NULL
    assert prep(sg.qk_config(rope_dim=63), *full) == E_CONFIG
    assert prep(sg.qk_config(rope_dim=194), *full) == E_CONFIG
    assert prep(sg.qk_config(rope_base=0.0), *full) == E_CONFIG
    assert prep(sg.qk_config(eps=-1.0), *full) == E_CONFIG
    assert prep(qk, None, P, P, None, None, P, P, P) == E_NULL                    # q_raw
    assert prep(qk, P, P, None, None, None, P, P, P) == E_NULL                    # v_raw without v_cache's pair
    assert "together" in L.sgqa_last_error().decode()
    # a paged producer checks the table like the other paged calls
    assert L.sgqa_qk_prep(ctypes.byref(cfg), ctypes.byref(qk), arr, n, P, P, None, None, None, P, P, None,
                          P, 3, 8, None) == E_CAPACITY
    # the gate is required by the gated calls
    assert L.sgqa_sparse_attn_gated(ctypes.byref(cfg), arr, n, P, P, P, P, P, None, None, None, 0,
                                    None) == E_NULL
    args = [ctypes.byref(cfg), arr, n] + [P] * 15 + [None, None, 0, None]     # gate NULL
    assert L.sgqa_forward_gated(*args) == E_NULL
    assert "gate" in L.sgqa_last_error().decode()


def test_misaligned_tensors(L):
    # every tensor pointer must be 16-byte aligned; the message names the tensor
    cfg = sg.config()
    P, M = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 8)
    arr, n = _seqs(sg.seq(16, pos0=48))
    err = lambda: L.sgqa_last_error().decode()
    assert L.sgqa_compress(ctypes.byref(cfg), arr, n, P, P, None, None, M, None, 0, None) == E_SHAPE
    assert "store" in err() and "aligned" in err()
    assert L.sgqa_index_topk(ctypes.byref(cfg), arr, n, P, P, None, P, P, M, None, None, 0,
                             None) == E_SHAPE
    assert "sel_scores" in err()
    assert L.sgqa_sparse_attn(ctypes.byref(cfg), arr, n, P, P, P, P, P, ctypes.c_void_p(FAKE + 4),
                              None, 0, None) == E_SHAPE
    assert "lse" in err()
    assert L.sgqa_sparse_attn_gated(ctypes.byref(cfg), arr, n, P, P, P, P, P, None, M, None, 0,
                                    None) == E_SHAPE
    assert "gate" in err()
    req = [3, 4, 7, 8, 9, 11, 13, 14, 15, 16]
    args = [ctypes.byref(cfg), arr, n] + [None] * 18
    for i in req:
        args[i] = P
    args[19] = 0
    args[13] = M                                  # q
    assert L.sgqa_forward(*args) == E_SHAPE
    assert "q is" in err()
    qk = sg.qk_config()
    assert L.sgqa_qk_prep(ctypes.byref(cfg), ctypes.byref(qk), arr, n, P, M, None, None, None, P, P, None,
                          None, 0, 0, None) == E_SHAPE
    assert "k_raw" in err()


def test_binding_rejects_wrong_tensors():
    import torch
    cfg = sg.config()
    with pytest.raises((TypeError, ValueError)):
        sg.sparse_attn(cfg, [_good_seq()], torch.zeros(4), torch.zeros(4), torch.zeros(4),
                       torch.zeros(4, dtype=torch.int32), torch.zeros(4))


def test_binding_store_format():
    # store_q8 = 2 (the default) takes E4M3 codes in a uint8 store; the dtype is checked
    # before any call (CPU tensors and a bf16 store are both refused)
    import torch
    with pytest.raises(ValueError):
        sg.config(store_q8=3)
    cfg = sg.config()
    assert cfg.store_q8 == 2
    with pytest.raises(TypeError):
        sg._store_ptr(cfg, torch.zeros(4, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError):                                   # not a device tensor
        sg._addrs([sg._store_ptr(cfg, torch.zeros(4, 128, dtype=torch.uint8))])
    with pytest.raises(TypeError):
        sg._store_ptr(sg.config(store_q8=1), torch.zeros(4, 128, dtype=torch.uint8))


# ---------------------------------------------------------------------------
# the binding checks every tensor's extents against the config and the
# sequences before it calls the library (the C ABI sees bare pointers); the
# checks run before the device check, so CPU tensors exercise them here
# ---------------------------------------------------------------------------

def _bf(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16)


def _f32(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.float32)


def _i32(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.int32)


def _attn_args(nq=40, rows=64, K=512):
    return dict(q=_bf(nq, 64, 192), k_cache=_bf(rows, 4, 192), v_cache=_bf(rows, 4, 192),
                sel=_i32(nq, 4, K), out=_bf(nq, 64, 192), lse=_f32(nq, 64))


def _seqs_for_shapes():
    # two sequences: query rows up to 40, cache rows up to 64, store rows up to 8
    return [sg.Seq(q_offset=0, n_q=8, pos0=24, cache_len=32, kv_offset=0, kv_capacity=32,
                   store_offset=0, store_capacity=4),
            sg.Seq(q_offset=32, n_q=8, pos0=0, cache_len=8, kv_offset=32, kv_capacity=32,
                   store_offset=4, store_capacity=4)]


def test_binding_accepts_exact_shapes_up_to_the_device_check():
    cfg = sg.config()
    with pytest.raises(ValueError, match="device"):
        sg.sparse_attn(cfg, _seqs_for_shapes(), **_attn_args())


@pytest.mark.parametrize("name,bad", [
    ("q", _bf(39, 64, 192)),              # fewer rows than the last query row
    ("q", _bf(40, 64, 128)),              # head_dim
    ("q", _bf(40, 60, 192)),              # heads
    ("k_cache", _bf(63, 4, 192)),         # fewer rows than kv_offset + kv_capacity
    ("v_cache", _bf(64, 8, 192)),         # groups
    ("sel", _i32(40, 4, 256)),            # last dim is not topk_blocks
    ("sel", _i32(39, 4, 512)),
    ("out", _bf(40, 64 * 192)),           # rank
    ("lse", _f32(40, 32)),
])
def test_binding_rejects_wrong_attention_extents(name, bad):
    args = _attn_args()
    args[name] = bad
    with pytest.raises(ValueError, match=name):
        sg.sparse_attn(sg.config(), _seqs_for_shapes(), **args)


@pytest.mark.parametrize("name,bad", [
    ("q_idx", _bf(40, 4, 4, 64)), ("q_idx", _bf(39, 4, 4, 128)), ("w", _f32(40, 4, 2)),
    ("store", __import__("torch").zeros((7, 128), dtype=__import__("torch").uint8)),
    ("sel_scores", _f32(40, 4, 100)), ("q_hat_out", _bf(40, 4, 4, 127)),
    ("rms_gamma", _bf(64)),
])
def test_binding_rejects_wrong_index_extents(name, bad):
    import torch
    args = dict(q_idx=_bf(40, 4, 4, 128), w=_f32(40, 4, 4),
                store=torch.zeros((8, 128), dtype=torch.uint8), sel=_i32(40, 4, 512))
    args[name] = bad
    with pytest.raises(ValueError, match=name):
        sg.index_topk(sg.config(), _seqs_for_shapes(), **args)


@pytest.mark.parametrize("name,bad", [
    ("proxy_k", _bf(63, 128)), ("comp_logits", _f32(64, 64)), ("ln_gamma", _bf(127)),
    ("store", __import__("torch").zeros((8, 64), dtype=__import__("torch").uint8)),
])
def test_binding_rejects_wrong_compress_extents(name, bad):
    import torch
    args = dict(proxy_k=_bf(64, 128), comp_logits=_f32(64, 128),
                store=torch.zeros((8, 128), dtype=torch.uint8))
    args[name] = bad
    with pytest.raises(ValueError, match=name):
        sg.compress(sg.config(), _seqs_for_shapes(), **args)


def test_binding_checks_store_dtype_against_the_config():
    import torch
    args = dict(proxy_k=_bf(64, 128), comp_logits=_f32(64, 128),
                store=torch.zeros((8, 128), dtype=torch.uint8))
    with pytest.raises(TypeError, match="store"):
        sg.compress(sg.config(store_q8=1), _seqs_for_shapes(), **args)


def test_binding_rejects_wrong_page_pools():
    import torch
    seqs = [sg.Seq(q_offset=0, n_q=8, pos0=0, cache_len=8, kv_offset=0, kv_capacity=32,
                   store_offset=0, store_capacity=4)]
    table = _i32(2)
    base = dict(q=_bf(8, 64, 192), k_pages=_bf(5, 16, 4, 192), v_pages=_bf(5, 16, 4, 192),
                page_table=table, sel=_i32(8, 4, 512), out=_bf(8, 64, 192))
    bad = dict(base, k_pages=_bf(5, 8, 4, 192))          # pages of 8 tokens
    with pytest.raises(ValueError, match="k_pages"):
        sg.sparse_attn_paged(sg.config(), seqs, **bad)
    bad = dict(base, v_pages=_bf(4, 16, 4, 192))         # pools of different sizes
    with pytest.raises(ValueError, match="v_pages"):
        sg.sparse_attn_paged(sg.config(), seqs, **bad)
    with pytest.raises(ValueError, match="device"):
        sg.sparse_attn_paged(sg.config(), seqs, **base)
    del torch


def test_contiguous_gather_row_limit(L):
    # contiguous caches are addressed with 32-bit offsets per sequence
    cfg = sg.config()
    big = sg.Seq(q_offset=0, n_q=1, pos0=100, cache_len=101, kv_offset=0, kv_capacity=2_796_203,
                 store_offset=0, store_capacity=12)
    arr, n = _seqs(big)
    P = ctypes.c_void_p(FAKE)
    assert L.sgqa_sparse_attn(ctypes.byref(cfg), arr, n, P, P, P, P, P, None, None, 0, None) == E_UNSUP
    assert "2796202" in L.sgqa_last_error().decode()
    ok = sg.Seq(q_offset=0, n_q=1, pos0=100, cache_len=101, kv_offset=0, kv_capacity=2_796_202,
                store_offset=0, store_capacity=12)
    arr, n = _seqs(ok)
    # passes the limit; fails later only for the missing workspace-free NULL out
    assert L.sgqa_sparse_attn(ctypes.byref(cfg), arr, n, P, P, P, P, None, None, None, 0, None) == E_NULL


def test_noalloc_forward_rejects_oversized_calls_before_any_hip_call(L):
    # an 8K-token prefill needs ~142 MB of index keys: beyond the 64 MiB static
    # scratch, so the call fails during validation (no device is touched)
    cfg = sg.config()
    arr, n = _seqs(sg.seq(8192))
    P = ctypes.c_void_p(FAKE)
    assert sg.workspace_size(cfg, [sg.seq(8192)], sg.OP_FORWARD) > 64 << 20
    rc = L.sgqa_forward_noalloc(ctypes.byref(cfg), arr, n, P, P, None, None, P, P, P, None, P, None,
                                P, P, P, P, None, None)
    assert rc == E_WS
    assert "static scratch" in L.sgqa_last_error().decode()
    # invalid arguments are reported first, as for sgqa_forward
    assert L.sgqa_forward_noalloc(ctypes.byref(cfg), arr, n, None, P, None, None, P, P, P, None, P,
                                  None, P, P, P, P, None, None) == E_NULL
