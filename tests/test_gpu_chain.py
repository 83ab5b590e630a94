"""GPU parity of the refresh/reuse NSA layer chain (sda_nsa_chain) against
the oracle's chain_lists and grouped_nsa_row, through the C ABI: a refresh
layer routes (top-n of f . K~ per row) and caches; every layer's output is
the gated three-branch NSA output over the cached lists ([SSV] core
mechanism 2 and its scheduling algorithm).  Refresh every r in {1, 2, 3}
layers, exact and shared-representative modes; routing vectors re-drawn per
row until the refresh layers' top-n cut gap clears the float32 score error.
"""
import math
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_pool_amd as sda
import oracle as O
from tests.parity_util import DELTA, DEV, TOL, bits, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sda.lib()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def _compressed(X, T):
    B, H, Tc, d = X.shape
    out = torch.zeros((B, H, -(-Tc // 64), d), dtype=torch.bfloat16, device=DEV)
    sda.sda_update_compressed_keys(X, out, torch.zeros(B, dtype=torch.int32, device=DEV),
                                   torch.full((B,), T, dtype=torch.int32, device=DEV), T)
    return out


@pytest.mark.parametrize("r,mode", [(1, 0), (2, 0), (3, 0), (2, 1)])
def test_chain_matches_oracle_layer_by_layer(r, mode):
    B, NQ, C, H, G, d, T, n, window, L = 2, 8, 4, 2, 4, 128, 4096, 8, 200, 5
    H_q = H * G
    rng = np.random.default_rng(100 + r + 10 * mode)
    sched = O.refresh_schedule(L, r)
    layers, ora = [], []
    nb = T // 64
    cand = O.candidates(nb, 0, 0)
    for j in range(L):
        K = _bf(rng.standard_normal((B, H, T, d)))
        V = _bf(rng.standard_normal((B, H, T, d)))
        Kg, Vg = K.to(DEV), V.to(DEV)
        kc, vc = _compressed(Kg, T), _compressed(Vg, T)
        kd = {(b, g): f64(K[b, g]) for b in range(B) for g in range(H)}
        vd = {(b, g): f64(V[b, g]) for b in range(B) for g in range(H)}
        kcd = {bg: O.store_bf16(O.compressed_keys(kd[bg], T)) for bg in kd}
        vcd = {bg: O.store_bf16(O.compressed_keys(vd[bg], T)) for bg in vd}
        F = rng.standard_normal((B, NQ, H, d)) / math.sqrt(d)
        for _ in range(100):                           # tie-free routing rows
            Fd = O.bf16_to_f64(bits(_bf(F)))
            bad = [(b, q, g) for b in range(B) for q in range(NQ) for g in range(H)
                   if O.cut_gap(O.decision_scores(O.indexer_scores(Fd[b, q, g], kcd[(b, g)])), cand, n) < DELTA]
            if not bad:
                break
            for x in bad:
                F[x] = rng.standard_normal(d) / math.sqrt(d)
        Q = _bf(rng.standard_normal((B, NQ, H_q, d)))
        gates = torch.from_numpy(rng.uniform(0.0, 1.0, (B, NQ, H_q, 3)).astype(np.float32))
        layers.append(dict(q=Q.to(DEV), k=Kg, v=Vg, k_cmp=kc, v_cmp=vc, k_route=kc, f_route=_bf(F).to(DEV),
                           gates=gates.to(DEV)))
        ora.append(dict(Qd=O.bf16_to_f64(bits(Q)), kd=kd, vd=vd, kcd=kcd, vcd=vcd, Fd=Fd, gd=gates.double().numpy()))
    seq = torch.full((B,), T, dtype=torch.int32, device=DEV)
    outs, bi, ns = sda.sda_nsa_chain(layers, sched, seq, n, 64, window, group_C=C, mode=mode)
    torch.cuda.synchronize()

    def route(j):
        o = ora[j]
        return {(b, q, g): O.select_row(o["Fd"][b, q, g], o["kcd"][(b, g)], 0, 0, n)[0]
                for b in range(B) for q in range(NQ) for g in range(H)}
    lists = O.chain_lists(sched, route)
    last = max(j for j in range(L) if sched[j])
    bi_h, ns_h = bi.cpu().numpy(), ns.cpu().numpy()
    for (b, q, g), want in lists[last].items():
        assert list(bi_h[b, q, g, :ns_h[b, q, g]]) == list(want)
    scale = 1.0 / math.sqrt(d)
    for j in range(L):
        o = ora[j]
        out = outs[j][0].double().cpu().numpy()
        err = 0.0
        for b in range(B):
            for g in range(H):
                for q0 in range(0, NQ, C):
                    qs = list(range(q0, q0 + C))
                    want, _ = O.grouped_nsa_row(
                        np.stack([o["Qd"][b, q, g * G:(g + 1) * G] for q in qs]), o["kd"][(b, g)], o["vd"][(b, g)],
                        o["kcd"][(b, g)], o["vcd"][(b, g)], [lists[j][(b, q, g)] for q in qs], T, nb, window,
                        np.stack([o["gd"][b, q, g * G:(g + 1) * G] for q in qs]), scale, mode)
                    for c, q in enumerate(qs):
                        err = max(err, float(np.abs(out[b, q, g * G:(g + 1) * G] - want[c]).max()))
        _say(f"r={r} mode={mode} layer {j} ({'refresh' if sched[j] else 'reuse'}): max abs err {err:.2e}")
        assert err <= TOL


def test_chain_refuses_a_first_reuse_layer():
    d, B, H = 64, 1, 1
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=DEV)
    y = dict(q=z(B, 1, 4, d), k=z(B, H, 128, d), v=z(B, H, 128, d), k_cmp=z(B, H, 2, d), v_cmp=z(B, H, 2, d),
             gates=torch.zeros((B, 1, 4, 3), dtype=torch.float32, device=DEV))
    with pytest.raises(sda.SdaError, match="first layer must refresh"):
        sda.sda_nsa_chain([y], [False], torch.full((B,), 128, dtype=torch.int32, device=DEV), 1, 64, 64)
