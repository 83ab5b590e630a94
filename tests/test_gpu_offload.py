"""GPU parity of the offloaded decode chain with the persistent prefetch pool
(sda_offload_chain): K/V of every layer in pinned host memory, layer 0's
blocks chosen by its own indexer vectors, layer l+1's by layer l's
([SparDA] §4.2 steps 2-4 and 6, §4.5, §4.6), the pool copying each layer's
blocks into a device stage while the stream runs the previous layer.
Checked per layer: the block lists against the oracle's selection (tie-free
vectors), the outputs against the oracle's attention over them (2e-3), and
bit-equality with sda_sparse_decode on the same K/V resident in HBM; no
transfer wait gave up.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_pool_amd as sda
import oracle as O
import synth
from synth import inputs
from tests.parity_util import DEV, TOL, bits, oracle_kt, tie_free_indexer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sda.lib()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _f64(t):
    return O.bf16_to_f64(bits(t))


def _run(cfg, L, wgs, sample):
    T = cfg.T
    seq = torch.full((cfg.B,), T, dtype=torch.int32, device=DEV)
    layers, dev_kv, kts = [], [], []
    for l in range(L):
        K, V, _ = inputs.kv_layer(cfg, l, device=DEV)
        kt = torch.zeros((cfg.B, cfg.H_kv, cfg.NB, cfg.d), dtype=torch.bfloat16, device=DEV)
        sda.sda_update_compressed_keys(K, kt, torch.zeros(cfg.B, dtype=torch.int32, device=DEV), seq, T)
        Kh = torch.empty(K.shape, dtype=torch.bfloat16, pin_memory=True)
        Vh = torch.empty(V.shape, dtype=torch.bfloat16, pin_memory=True)
        Kh.copy_(K)
        Vh.copy_(V)
        kt_o = oracle_kt(K, T, [(b, g) for (b, _, g) in sample])
        kts.append(kt_o)
        dev_kv.append((K, V))
        layers.append(dict(k_host=Kh, v_host=Vh, k_tilde=kt,
                           q=inputs.to_bf16(inputs.attention_queries(cfg, l), DEV)))
    # indexer vectors: f_first scores layer 0, layer l's vectors score layer l+1
    f_first, _ = tie_free_indexer(cfg, 100, kts[0], sample)
    fs = []
    for l in range(L):
        F, _ = tie_free_indexer(cfg, l, kts[l + 1], sample) if l + 1 < L else \
            (inputs.to_bf16(inputs.indexer_vectors(cfg, l)), None)
        fs.append(F)
        layers[l]["f"] = F.to(DEV)
    outs, bi, ws = sda.sda_offload_chain(layers, seq, cfg.n_init, cfg.n_local, cfg.top_k, f_first.to(DEV),
                                         prefetch_workgroups=wgs)
    torch.cuda.synchronize()
    err_word = int(ws[8:12].view(torch.int32).item())
    assert err_word == 0, f"a transfer wait gave up (error word {err_word})"
    bi_h = bi.cpu().numpy()
    worst = 0.0
    for l in range(L):
        f_sel = f_first if l == 0 else fs[l - 1]
        Fd = _f64(f_sel)
        K, V = dev_kv[l]
        ns_l = (bi[l] >= 0).sum(-1).to(torch.int32)
        ref, _ = sda.sda_sparse_decode(layers[l]["q"], K, V, seq, bi[l].contiguous(), ns_l.contiguous())
        assert torch.equal(outs[l][0], ref), l                       # staged = resident, bit for bit
        Qd = _f64(layers[l]["q"])
        for (b, q, g) in sample:
            want, _ = O.select_row(Fd[b, q, g], kts[l][(b, g)], cfg.n_init, cfg.n_local, cfg.top_k)
            got = bi_h[l, b, q, g]
            assert list(got[got >= 0]) == list(want), (l, b, g)
            kk, vv = _f64(K[b, g, :T]), _f64(V[b, g, :T])
            o, _ = O.decode_row(Qd[b, q, g * cfg.G:(g + 1) * cfg.G], kk, vv, want, T, cfg.d ** -0.5)
            worst = max(worst, float(np.abs(outs[l][0][b, q, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
                                            - o).max()))
    _say(f"  chain of {L} layers, {wgs} pool workgroups: max abs err {worst:.2e}")
    assert worst <= TOL


@pytest.mark.parametrize("wgs", [64, 1])
def test_offload_chain_small(wgs):
    cfg = dataclasses.replace(synth.get_config(5), B=2, H_q=16, H_kv=4, T=8192)
    _say("offload chain small", wgs)
    _run(cfg, 4, wgs, [(b, 0, g) for b in range(cfg.B) for g in range(cfg.H_kv)])


def test_offload_chain_256k_sampled():
    cfg = synth.get_config(5)
    _say("offload chain 256K")
    _run(cfg, 3, 64, [(b, 0, (3 * b + 1) % cfg.H_kv) for b in range(cfg.B)])
