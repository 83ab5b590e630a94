"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, sizes workspaces, and rejects bad arguments on the host before any
HIP call (each call here fails validation, so nothing is launched)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_pool_amd as sda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sda.h")

OK, NULL, SHAPE, UNSUP, WS, ALIGN, HIP = range(7)
P = 0x10000          # a 16-byte aligned stand-in address; never dereferenced
P_ODD = 0x10004


@pytest.fixture(scope="module")
def L():
    # these calls pass stand-in addresses that must be rejected on the host;
    # keep them off machines with a GPU so a validation slip can never launch
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-validation tests run only where no GPU is visible")
    if not os.path.exists(sda.LIB_PATH):
        from block_sparse_attention_pool_amd import _build
        _build.build()
    return sda.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sda_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound(L):
    names = header_functions()
    assert len(names) == 31
    for n in names:
        assert hasattr(L, n), n
        assert n in sda.exported_symbols(), n
    assert set(sda.exported_symbols()) == set(names)


def test_status_strings(L):
    assert sda.status_string(0) == "SDA_OK"
    assert sda.status_string(4) == "SDA_ERR_WORKSPACE"
    assert sda.version().startswith("sda ")


def test_workspace_sizes(L):
    # scores + per-chunk candidate keys (top_k <= 64, NB_cap <= 4096 only), each
    # padded to 256 B, + one arrival counter per (b, kv head, vector tile)
    assert L.sda_score_select_workspace(8, 1, 8, 2048, 32) == 8 * 8 * 2048 * 4 + 64 * 8 * 32 * 8 + 8 * 8 * 4
    # (several query vectors: one counter per vector tile; tiles shrink to one
    # vector each while the grid holds fewer than 512 workgroups)
    assert L.sda_score_select_workspace(1, 3, 1, 3, 1) == 256 + 256 + 1 * 1 * 3 * 4
    assert L.sda_score_select_workspace(2, 20, 1, 64, 1) == 2 * 20 * 64 * 4 + 512 + 2 * 1 * 20 * 4
    assert L.sda_score_select_workspace(4, 16, 8, 1024, 16) == 4 * 16 * 8 * 1024 * 4 + 4 * 16 * 8 * 4 * 16 * 8 + \
        4 * 8 * 4 * 4                                                      # 4 chunks x 32 rows x 4 tiles of 4
    assert L.sda_score_select_workspace(1, 1, 1, 2048, 65) == 2048 * 4 + 4       # lists too long: no candidates
    assert L.sda_score_select_workspace(1, 1, 1, 4097, 8) == 16640 + 4            # too many chunks
    assert L.sda_score_select_workspace(0, 1, 8, 2048, 32) == 0
    # multihead: per-head logits plus the summed scores
    # multihead: per-head logits and per-chunk softmax statistics, the summed
    # scores, candidate keys and arrival counters
    assert L.sda_score_select_multihead_workspace(8, 1, 64, 8, 2048, 32) == \
        (8 * 64 * 2048 + 8 * 64 * 8 * 2) * 4 + 8 * 8 * 2048 * 4 + 64 * 8 * 32 * 8 + 8 * 8 * 4
    # decode: 256-byte padded arrival counters, then (m, l) + d floats per padded row per split
    def dec(tasks, splits, rows=16, d=128):
        return (tasks * 4 + 255) // 256 * 256 + tasks * splits * rows * (d + 2) * 4
    n = L.sda_sparse_decode_workspace(8, 1, 64, 8, 35, 128, 0)
    assert n in {dec(64, s) for s in range(2, 36)}
    assert L.sda_sparse_decode_workspace(8, 1, 64, 8, 35, 128, 7) == dec(64, 7)
    assert L.sda_sparse_decode_workspace(8, 1, 64, 8, 35, 128, 1) == 0
    # exact groups of 4 at G = 4: tiles of all 16 queries (64 rows), one per (b, KV head)
    assert L.sda_grouped_decode_workspace(4, 16, 32, 8, 16, 128, 1024, 4, 0, 3) == dec(4 * 8, 3, rows=64)
    assert L.sda_grouped_decode_workspace(4, 16, 32, 8, 16, 128, 0, 4, 0, 3) == 0      # NB_cap < 1
    # exact groups on the row-tiled engine: a tile holds as many whole groups
    # as fit in 128 rows and 32 queries; partials per split for the tile's
    # rows (16 per row wave); the library's split count fills the compute
    # units once (one workgroup each), or twice with two-slot workgroups when
    # that gives fewer than four splits
    assert L.sda_grouped_decode_workspace(4, 16, 32, 8, 16, 128, 1024, 16, 0, 0) == dec(32, 8, rows=64)
    assert L.sda_grouped_decode_workspace(4, 16, 32, 8, 16, 128, 1024, 4, 0, 0) == dec(32, 8, rows=64)
    assert L.sda_grouped_decode_workspace(4, 16, 64, 8, 16, 128, 1024, 2, 0, 0) == dec(32, 8, rows=128)
    assert L.sda_grouped_decode_workspace(4, 16, 32, 8, 16, 128, 1024, 8, 0, 0) == dec(32, 8, rows=64)
    # groups of 3: tiles of 18 queries (six groups, the last holding one query; 72 rows on 8 row waves)
    assert L.sda_grouped_decode_workspace(4, 16, 32, 8, 16, 128, 1024, 3, 0, 0) == dec(32, 8, rows=128)
    assert L.sda_grouped_decode_workspace(4, 16, 32, 8, 16, 128, 1024, 4, 1, 0) > 0  # shared mode: grouped engine


def _last():
    return sda.last_error()


def test_update_validation(L):
    f = L.sda_update_compressed_keys
    assert f(None, P, P, P, 64, 1, 2, 64, 4096, 64, None) == NULL
    assert f(P, P, P, P, 64, 1, 2, 96, 4096, 64, None) == UNSUP
    assert "96" in _last()
    assert f(P, P, P, P, 64, 1, 2, 64, 4096, 63, None) == SHAPE          # NB_cap too small
    assert f(P_ODD, P, P, P, 64, 1, 2, 64, 4096, 64, None) == ALIGN
    assert f(P, P, P, P, -1, 1, 2, 64, 4096, 64, None) == SHAPE
    assert f(P, P, P, P, 0, 1, 2, 64, 4096, 64, None) == OK               # nothing to do, nothing launched


def test_strided_update_validation(L):
    f = L.sda_update_compressed_keys_strided
    # k, k_tilde, len_old, len_new, max_new, B, H_kv, d, T_cap, NC_cap, window, stride, stream
    ok = [P, P, P, P, 0, 1, 2, 64, 4096, 256, 32, 16, None]
    assert f(*ok) == OK                                                  # nothing to do, nothing launched
    bad = list(ok); bad[0] = None
    assert f(*bad) == NULL
    bad = list(ok); bad[11] = 12                                         # stride not supported
    assert f(*bad) == UNSUP
    bad = list(ok); bad[10] = 24                                         # window not a multiple of the stride
    assert f(*bad) == UNSUP
    bad = list(ok); bad[10] = 128; bad[11] = 64                          # window beyond 64 tokens
    assert f(*bad) == UNSUP
    bad = list(ok); bad[10] = 8                                          # window shorter than the stride
    assert f(*bad) == UNSUP
    bad = list(ok); bad[9] = 255                                         # NC_cap < ceil(T_cap / stride)
    assert f(*bad) == SHAPE
    bad = list(ok); bad[1] = P_ODD
    assert f(*bad) == ALIGN
    bad = list(ok); bad[4] = -1
    assert f(*bad) == SHAPE


def test_pooled_workspace_and_validation(L):
    # [block scores over ceil(NC_cap*stride/64) blocks][candidate keys][counters per (b, q, kv head)]
    assert L.sda_score_select_pooled_workspace(8, 1, 8, 8192, 16, 32) == \
        8 * 8 * 2048 * 4 + 64 * 8 * 32 * 8 + 8 * 8 * 4
    # NC_cap 100 at stride 16 = 25 blocks: 600 B of scores (768 padded), 192 B of keys (256), 24 B
    assert L.sda_score_select_pooled_workspace(2, 3, 1, 100, 16, 4) == 768 + 256 + 2 * 3 * 4
    assert L.sda_score_select_pooled_workspace(1, 1, 1, 0, 16, 4) == 0
    f = L.sda_score_select_pooled
    # f, k_tilde, seq_len, B, NQ, H_kv, d, NC_cap, window, stride, n_init, n_local, top_k, n_sel_max,
    # block_idx, n_sel, scores, ws, ws_bytes, stream
    args = [P, P, P, 1, 1, 2, 64, 256, 32, 16, 1, 2, 8, 11, P, P, None, P, 1 << 20, None]
    bad = list(args); bad[0] = None
    assert f(*bad) == NULL
    bad = list(args); bad[9] = 24
    assert f(*bad) == UNSUP
    bad = list(args); bad[8] = 16; bad[9] = 32                           # window shorter than the stride
    assert f(*bad) == UNSUP
    bad = list(args); bad[13] = 10                                       # n_sel_max < 1 + 2 + 8
    assert f(*bad) == SHAPE
    bad = list(args); bad[18] = 100
    assert f(*bad) == WS
    bad = list(args); bad[7] = 0
    assert f(*bad) == SHAPE
    bad = list(args); bad[7] = 90000                                     # beyond the block limit of the select launch
    assert f(*bad) == UNSUP
    bad = list(args); bad[1] = P_ODD
    assert f(*bad) == ALIGN


def test_nsa_workspace_and_validation(L):
    # 64 row groups x 9 splits (4 listed, 4 compressed at 2048 keys, 1 window) of 16 padded rows
    def dec(tasks, splits, rows=16, d=128):
        return (tasks * 4 + 255) // 256 * 256 + tasks * splits * rows * (d + 2) * 4
    n = L.sda_nsa_decode_workspace(8, 1, 64, 8, 35, 128, 131072, 2048, 512, 1, 0)
    assert n in {dec(64, s) for s in range(3, 80)}
    assert L.sda_nsa_decode_workspace(8, 1, 64, 8, 35, 128, 131072, 2048, -1, 1, 0) == 0
    # exact verification of 16 queries in groups of 4 (G = 4): one tile of all 16 queries (64 rows) per
    # (batch, KV head), 32 tiles x 8 splits, the same as grouped verification's split-K workspace
    n16 = L.sda_nsa_decode_workspace(4, 16, 32, 8, 16, 128, 65536, 1024, 512, 4, 0)
    assert n16 == dec(32, 8, rows=64)
    assert n16 == L.sda_grouped_decode_workspace(4, 1, 32, 8, 16, 128, 1024, 16, 0, 0)
    # shared-representative mode runs on the same tiles
    assert L.sda_nsa_decode_workspace(4, 16, 32, 8, 16, 128, 65536, 1024, 512, 4, 1) == n16
    # one query per KV head in groups of one keeps the per-group launch (16 padded rows)
    assert L.sda_nsa_decode_workspace(4, 1, 32, 8, 16, 128, 65536, 1024, 512, 1, 1) in \
        {dec(32, s) for s in range(3, 80)}
    f = L.sda_nsa_decode
    # q, k, v, k_cmp, v_cmp, seq_len, block_idx, n_sel, n_sel_max, T_cap, NC_cap, cmp_stride, window,
    # gates, B, NQ, H_q, H_kv, d, scale, group_C, mode, out, lse, union_count, ws, ws_bytes, stream
    args = [P, P, P, P, P, P, P, P, 11, 4096, 64, 64, 512, P, 1, 1, 8, 2, 64, 0.125, 1, 0, P, None, None,
            P, 1 << 24, None]
    bad = list(args); bad[3] = None
    assert f(*bad) == NULL
    bad = list(args); bad[13] = None                                     # gates
    assert f(*bad) == NULL
    bad = list(args); bad[10] = 63                                       # NC_cap < ceil(T_cap / stride)
    assert f(*bad) == SHAPE
    bad = list(args); bad[11] = 0
    assert f(*bad) == UNSUP
    bad = list(args); bad[12] = -1
    assert f(*bad) == SHAPE
    bad = list(args); bad[20] = 33; bad[21] = 1                          # group_C <= 32 in either mode
    assert f(*bad) == UNSUP
    bad = list(args); bad[16] = 128                                      # one query of G = 64 heads: no
    assert f(*bad) == UNSUP                                              # tile, and beyond 32 rows
    bad = list(args); bad[20] = 33                                       # exact mode: group_C <= 32
    assert f(*bad) == UNSUP
    bad = list(args); bad[20] = 8; bad[15] = 8; bad[16] = 64             # exact: 8 x G = 32 > 128 rows
    assert f(*bad) == UNSUP
    bad = list(args); bad[26] = 64
    assert f(*bad) == WS
    bad = list(args); bad[4] = P_ODD
    assert f(*bad) == ALIGN
    bad = list(args); bad[13] = P + 2
    assert f(*bad) == ALIGN


def test_score_select_validation(L):
    f = L.sda_score_select
    args = [P, P, P, 1, 1, 2, 64, 64, 1, 2, 8, 11, P, P, None, P, 1 << 20, None]
    bad = list(args); bad[0] = None
    assert f(*bad) == NULL
    bad = list(args); bad[11] = 10                                        # n_sel_max < 1 + 2 + 8
    assert f(*bad) == SHAPE
    bad = list(args); bad[16] = 100                                       # workspace too small
    assert f(*bad) == WS
    bad = list(args); bad[15] = None
    assert f(*bad) == WS
    bad = list(args); bad[14] = P; bad[15] = None                        # counters live in the workspace
    assert f(*bad) == WS
    bad = list(args); bad[6] = 32
    assert f(*bad) == UNSUP
    bad = list(args); bad[7] = 20000                                      # NB_cap beyond the select kernel
    assert f(*bad) == UNSUP
    bad = list(args); bad[10] = -1
    assert f(*bad) == SHAPE
    bad = list(args); bad[1] = P_ODD
    assert f(*bad) == ALIGN


def test_multihead_validation(L):
    f = L.sda_score_select_multihead
    base = [P, P, P, 1, 1, 8, 2, 64, 64, 1, 2, 8, 11, 8.0, P, P, None, P, 1 << 24, None]
    bad = list(base); bad[5] = 7                                          # H_q not a multiple of H_kv
    assert f(*bad) == SHAPE
    bad = list(base); bad[13] = 0.0
    assert f(*bad) == SHAPE
    bad = list(base); bad[18] = 16
    assert f(*bad) == WS


def test_decode_validation(L):
    f = L.sda_sparse_decode
    base = [P, P, P, P, P, P, 11, None, 4096, 1, 1, 8, 2, 64, 0.125, P, None, 0, P, 1 << 24, None]
    bad = list(base); bad[1] = None
    assert f(*bad) == NULL
    bad = list(base); bad[13] = 80
    assert f(*bad) == UNSUP
    bad = list(base); bad[11] = 6; bad[12] = 4                            # 6 heads over 4 KV heads
    assert f(*bad) == SHAPE
    bad = list(base); bad[11] = 128; bad[12] = 2                          # G = 64
    assert f(*bad) == UNSUP
    bad = list(base); bad[14] = float("nan")
    assert f(*bad) == SHAPE
    bad = list(base); bad[17] = -1
    assert f(*bad) == SHAPE
    bad = list(base); bad[18] = None; bad[19] = 0                         # auto split needs a workspace
    assert f(*bad) == WS
    bad = list(base); bad[2] = P_ODD
    assert f(*bad) == ALIGN


def test_grouped_validation(L):
    f = L.sda_grouped_decode
    base = [P, P, P, P, P, P, 16, 65536, 1024, 4, 16, 32, 8, 128, 0.088, 4, 0, P, None, None, 0, P,
            1 << 28, None]
    bad = list(base); bad[15] = 9; bad[16] = 1                            # shared mode: C > 8
    assert f(*bad) == UNSUP
    bad = list(base); bad[15] = 33                                        # C > 32
    assert f(*bad) == UNSUP
    bad = list(base); bad[16] = 2
    assert f(*bad) == SHAPE
    bad = list(base); bad[11] = 64; bad[15] = 8; bad[16] = 1              # shared mode: C*G = 64 rows
    assert f(*bad) == UNSUP
    bad = list(base); bad[11] = 256; bad[15] = 8                          # exact mode: C*G = 256 rows
    assert f(*bad) == UNSUP
    bad = list(base); bad[15] = 16; bad[22] = 16                          # exact, C*G = 64: the tiled
    assert f(*bad) == WS                                                  # engine's split workspace
    bad = list(base); bad[8] = 10                                         # NB_cap below T_cap/64
    assert f(*bad) == SHAPE


def test_gather_validation(L):
    f = L.sda_gather_blocks
    base = [P, P, P, P, 35, 4, 8, 128, 262144, P, P, P, 0, None]
    bad = list(base); bad[0] = None
    assert f(*bad) == NULL
    bad = list(base); bad[7] = 32
    assert f(*bad) == UNSUP
    bad = list(base); bad[12] = -3
    assert f(*bad) == SHAPE
    bad = list(base); bad[9] = P_ODD
    assert f(*bad) == ALIGN


def test_decode_step_workspace_and_validation(L):
    # the decode's partials + the score/select workspace of the next layer;
    # aliasing lists are refused
    n = L.sda_decode_step_workspace(8, 64, 8, 128, 35, 0, 2048, 32)
    assert n >= L.sda_score_select_workspace(8, 1, 8, 2048, 32)
    assert L.sda_decode_step_workspace(0, 64, 8, 128, 35, 0, 2048, 32) == 0
    # one launch at the 128K shape; two calls when the lists are too long for
    # the in-launch merge or a workgroup would have fewer than four waves
    assert L.sda_decode_step_is_fused(8, 64, 8, 128, 35, 0, 2048, 32) == 1
    assert L.sda_decode_step_is_fused(8, 64, 8, 128, 100, 0, 2048, 97) == 0      # top_k > 64
    assert L.sda_decode_step_is_fused(8, 64, 8, 128, 35, 0, 5000, 32) == 0       # 20 chunks
    assert L.sda_decode_step_is_fused(1, 8, 2, 64, 3, 0, 64, 1) == 0             # 3 entries: one wave
    assert L.sda_decode_step_is_fused(1, 8, 2, 64, 11, 0, 64, 8) == 1
    assert L.sda_decode_step_is_fused(8, 64, 8, 128, 35, 0, 2048, 0) == 0        # no top-k: two calls
    assert L.sda_decode_step_is_fused(8, 64, 8, 96, 35, 0, 2048, 32) == 0        # unsupported head dim
    f = L.sda_decode_step
    base = [P, P, P, P, P, P, 35, 4096, 1, 8, 2, 64, 0.125, P, None, 0,
            P, P, P, 64, 1, 2, 8, 11, P + 256, P + 512, None, None, 1, 0, P, 1 << 24, None]
    bad = list(base); bad[16] = None                                     # f_next
    assert f(*bad) == NULL
    bad = list(base); bad[24] = P                                        # block_idx_next aliases block_idx
    assert f(*bad) == SHAPE
    bad = list(base); bad[31] = 16                                       # workspace too small
    assert f(*bad) == WS
    bad = list(base); bad[23] = 10                                       # n_sel_max_next < 1 + 2 + 8
    assert f(*bad) == SHAPE
    # this layer's compressed-key refresh: k_tilde_cur, len_old_cur, max_new_tokens_cur, NB_cap_cur
    bad = list(base); bad[26] = P + 1024; bad[29] = 64                   # no len_old_cur
    assert f(*bad) == NULL
    bad = list(base); bad[26] = P; bad[27] = P; bad[29] = 64             # aliases k_tilde_next
    assert f(*bad) == SHAPE
    bad = list(base); bad[26] = P + 1024; bad[27] = P; bad[29] = 63      # NB_cap_cur < ceil(T_cap / 64)
    assert f(*bad) == SHAPE
    bad = list(base); bad[26] = P + 1024; bad[27] = P; bad[28] = -1; bad[29] = 64
    assert f(*bad) == SHAPE
    bad = list(base); bad[26] = P + 1032; bad[27] = P; bad[29] = 64      # k_tilde_cur not 16-byte aligned
    assert f(*bad) == ALIGN


def test_python_binding_rejects_bad_tensors():
    import torch
    k = torch.zeros((1, 2, 64, 64), dtype=torch.float32)
    with pytest.raises(TypeError):
        sda.sda_update_compressed_keys(k, k, torch.zeros(1, dtype=torch.int32),
                                       torch.zeros(1, dtype=torch.int32), 64)
    kb = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):                                        # CPU tensors are refused
        sda.sda_update_compressed_keys(kb, torch.zeros((1, 2, 1, 64), dtype=torch.bfloat16),
                                       torch.zeros(1, dtype=torch.int32),
                                       torch.zeros(1, dtype=torch.int32), 64)


# ---------------------------------------------------------------------------
# The binding checks the shape of every tensor argument (defaults and caller
# outputs alike) before the foreign call: the C ABI cannot see buffer sizes,
# so a wrong shape would otherwise become an out-of-bounds device access.
# Here every tensor is a host tensor: with all shapes right, the binding gets
# as far as its placement check and refuses the host tensors; with one shape
# wrong it names that argument first.  Nothing reaches the library's calls.
# ---------------------------------------------------------------------------

def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def _cases():
    import torch
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    B, NQ, H_q, H_kv, d, T_cap, nsm = 2, 1, 8, 2, 64, 256, 5
    dec = dict(q=_t((B, NQ, H_q, d), bf), k=_t((B, H_kv, T_cap, d), bf), v=_t((B, H_kv, T_cap, d), bf),
               seq_len=_t((B,), i32), block_idx=_t((B, NQ, H_kv, nsm), i32), n_sel=_t((B, NQ, H_kv), i32))
    cases = []
    # (binding, positional names, fixed kwargs, tensors, the wrong shape of each checked argument)
    cases.append((sda.sda_sparse_decode, dict(dec),
                  dict(out=_t((B, NQ, H_q, d), f32), lse=_t((B, NQ, H_q), f32), slot=_t((B, NQ, H_kv, nsm), i32)),
                  {}, dict(k=(B, H_kv, T_cap, 2 * d), v=(B, H_kv, T_cap + 64, d),
                           seq_len=(B + 1,), block_idx=(B, NQ + 1, H_kv, nsm), n_sel=(B, NQ, H_kv + 1),
                           out=(B, NQ, H_q, d - 1), lse=(B, NQ, H_q + 1), slot=(B, NQ, H_kv, nsm + 1))))
    step = dict(dec, f_next=_t((B, 1, H_kv, d), bf), k_tilde_next=_t((B, H_kv, 8, d), bf),
                seq_len_next=_t((B,), i32), n_init=1, n_local=1, top_k=3)
    cases.append((sda.sda_decode_step, step,
                  dict(block_idx_next=_t((B, 1, H_kv, 5), i32), n_sel_next=_t((B, 1, H_kv), i32),
                       out=_t((B, 1, H_q, d), f32), lse=_t((B, 1, H_q), f32),
                       k_tilde_cur=_t((B, H_kv, 4, d), bf), len_old_cur=_t((B,), i32)),
                  {}, dict(f_next=(B, 1, H_kv + 1, d), k_tilde_next=(B, H_kv, 8, d + 1), seq_len_next=(B - 1,),
                           block_idx_next=(B, 1, H_kv - 1, 5), n_sel_next=(B, 2, H_kv), out=(B, 1, H_q - 1, d),
                           lse=(B, 1, H_q, 2), k_tilde_cur=(B + 1, H_kv, 4, d), len_old_cur=(B + 1,),
                           n_sel=(B, 1, 1))))
    sel = dict(f=_t((B, NQ, H_kv, d), bf), k_tilde=_t((B, H_kv, 8, d), bf), seq_len=_t((B,), i32),
               n_init=1, n_local=1, top_k=3)
    cases.append((sda.sda_score_select, sel,
                  dict(block_idx=_t((B, NQ, H_kv, 5), i32), n_sel=_t((B, NQ, H_kv), i32),
                       scores=_t((B, NQ, H_kv, 8), f32)),
                  {}, dict(k_tilde=(B, H_kv + 1, 8, d), seq_len=(2 * B,), block_idx=(B, NQ, H_kv + 1, 5),
                           n_sel=(B, NQ + 1, H_kv), scores=(B, NQ, H_kv, 7))))
    cases.append((sda.sda_score_select_pooled, dict(sel, window=32, stride=16),
                  dict(block_idx=_t((B, NQ, H_kv, 5), i32), n_sel=_t((B, NQ, H_kv), i32),
                       scores=_t((B, NQ, H_kv, 2), f32)),
                  {}, dict(k_tilde=(B, H_kv, 8, d * 2), scores=(B, NQ, H_kv, 8), n_sel=(B, NQ, 1))))
    cases.append((sda.sda_score_select_multihead,
                  dict(q=_t((B, NQ, H_q, d), bf), k_tilde=_t((B, H_kv, 8, d), bf), seq_len=_t((B,), i32),
                       n_init=1, n_local=1, top_k=3, tau=8.0),
                  dict(block_idx=_t((B, NQ, H_kv, 5), i32), n_sel=_t((B, NQ, H_kv), i32)),
                  {}, dict(k_tilde=(B + 1, H_kv, 8, d), block_idx=(B, NQ, H_kv + 1, 5), n_sel=(B, NQ))))
    NQg, C = 4, 2
    grp = dict(q=_t((B, NQg, H_q, d), bf), k=dec["k"], v=dec["v"], seq_len=dec["seq_len"],
               block_idx=_t((B, NQg, H_kv, nsm), i32), n_sel=_t((B, NQg, H_kv), i32), group_C=C)
    cases.append((sda.sda_grouped_decode, grp,
                  dict(out=_t((B, NQg, H_q, d), f32), lse=_t((B, NQg, H_q), f32),
                       union_count=_t((B, NQg // C, H_kv), i32)),
                  {}, dict(block_idx=(B, NQg - 1, H_kv, nsm), union_count=(B, NQg, H_kv),
                           lse=(B, NQg, H_q, 1), out=(B, NQg, H_q + 8, d))))
    nsa = dict(grp, k_cmp=_t((B, H_kv, 16, d), bf), v_cmp=_t((B, H_kv, 16, d), bf),
               gates=_t((B, NQg, H_q, 3), f32), cmp_stride=16, window=64)
    cases.append((sda.sda_nsa_decode, nsa,
                  dict(out=_t((B, NQg, H_q, d), f32), lse=_t((B, NQg, H_q, 3), f32),
                       union_count=_t((B, NQg // C, H_kv), i32)),
                  {}, dict(k_cmp=(B, H_kv, 16, d + 64), v_cmp=(B, H_kv, 15, d), gates=(B, NQg, H_q, 2),
                           lse=(B, NQg, H_q), union_count=(B, 1, H_kv))))
    upd = dict(k=dec["k"], k_tilde=_t((B, H_kv, 4, d), bf), len_old=_t((B,), i32), len_new=_t((B,), i32),
               max_new_tokens=1)
    cases.append((sda.sda_update_compressed_keys, upd, {}, {},
                  dict(k_tilde=(B, H_kv, 4, d // 2), len_old=(B + 1,), len_new=(1,))))
    cases.append((sda.sda_update_compressed_keys_strided, dict(upd, window=32, stride=16), {}, {},
                  dict(k_tilde=(B, 1, 4, d), len_new=(B, 1))))
    return cases


def _call(fn, args, kw):
    return fn(**args, **kw)


def test_binding_checks_every_tensor_shape(L):
    import torch
    for fn, args, kw, _, wrong in _cases():
        with pytest.raises(ValueError, match="must be a GPU tensor"):       # every shape right
            _call(fn, args, kw)
        for name, shape in wrong.items():
            a2, kw2 = dict(args), dict(kw)
            tgt = a2 if name in a2 else kw2
            tgt[name] = torch.zeros(shape, dtype=tgt[name].dtype)
            with pytest.raises(ValueError, match=f"^{name} must have shape"):
                _call(fn, a2, kw2)


def test_binding_checks_workspace_and_gather_shapes(L):
    import torch
    fn, args, kw, _, _ = _cases()[0]
    with pytest.raises(ValueError, match="ws holds 16 bytes"):
        _call(fn, args, dict(kw, split_k=3, ws=torch.zeros(16, dtype=torch.uint8)))
    B, H_kv, T_cap, d = 2, 2, 256, 64
    kh = torch.zeros((B, H_kv, T_cap, d), dtype=torch.bfloat16)
    bi = torch.zeros((B, H_kv, 3), dtype=torch.int32)
    ns = torch.zeros((B, H_kv), dtype=torch.int32)
    with pytest.raises(ValueError, match="^v_host must have shape"):
        sda.sda_gather_blocks(kh, kh[:, :1].contiguous(), bi, ns)
    with pytest.raises(ValueError, match="^n_sel must have shape"):
        sda.sda_gather_blocks(kh, kh, bi, ns[:1])
    with pytest.raises(ValueError, match="^k_stage must have shape"):
        sda.sda_gather_blocks(kh, kh, bi, ns, k_stage=torch.zeros((B, H_kv, 2 * 64, d), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="^slot must have shape"):
        sda.sda_gather_blocks(kh, kh, bi, ns, slot=torch.zeros((B, H_kv, 4), dtype=torch.int32))
    with pytest.raises(ValueError, match="pinned"):                        # shapes right, not pinned
        sda.sda_gather_blocks(kh, kh, bi, ns)


def test_noalloc_step_rejects_sizes_beyond_its_scratch(L):
    # 512 rows x 8 splits of partials (34 MB) exceed the 8 MiB static
    # scratch: refused on the host, nothing launched
    f = L.sda_decode_step_noalloc
    args = [P, P, P, P, P, P, 35, 4096, 64, 64, 8, 128, ctypes.c_float(128 ** -0.5), P, P, 8,
            P, P, P, 64, 1, 2, 32, 35, P + 4096, P + 8192, None, None, 0, 0, None]
    assert f(*args) == WS
    assert "static scratch" in _last()
    bad = list(args); bad[0] = None                                        # null q: refused first
    assert f(*bad) == NULL


def _header_params():
    """name -> list of parameter types, from include/sda.h."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(sda_[a-z_]+)\s*\(([^)]*)\)\s*;", text):
        params = [p.strip() for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
        out[m.group(1)] = params
    return out


def test_binding_signatures_match_the_header(L):
    # every bound function takes as many arguments as the header declares,
    # with floats, 64-bit sizes and pointers where the header has them
    import ctypes as C
    params = _header_params()
    for name, (_, argtypes) in sda._SIGNATURES.items():
        decl = params[name]
        assert len(decl) == len(argtypes), (name, len(decl), len(argtypes))
        for p, t in zip(decl, argtypes):
            if "*" in p:
                assert t is C.c_void_p, (name, p)
            elif p.startswith("float"):
                assert t is C.c_float, (name, p)
            elif p.startswith("size_t"):
                assert t is C.c_size_t, (name, p)
            else:
                assert t is C.c_int, (name, p)
