"""GPU parity of exact grouped verification on the row-tiled engine (every
group of two or more queries, C * G up to 128 rows) against the oracle's
grouped_row in exact mode ([SSV] core mechanism 1: each query attends to its
own list, the union of the group's lists is fetched once).

Drawn ascending lists with ragged lengths, empty lists, a last group smaller
than C, every row-wave count (16, 32, 64, 96 and 128 rows, and groups of
fewer rows than a wave), both slot plans (four slots with one workgroup per
compute unit, two slots and twice the splits when there are many groups),
split-K from one workgroup per group to more splits than union blocks, and
the union counts.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_pool_amd as sda
import oracle as O
from tests.parity_util import DEV, TOL, bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sda.lib()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    # (B, H_kv, G, d, lens, NQ, C, n_sel_max, split_k)
    (2, 2, 8, 128, [3000, 1234], 16, 16, 12, 0),     # 128 rows, the planner's split count
    (1, 2, 8, 128, [5000], 16, 16, 16, 1),           # one workgroup per group
    (1, 1, 8, 64, [700], 20, 8, 9, 3),               # 64 rows, NQ not a multiple of C
    (2, 1, 4, 128, [2500, 2500], 32, 32, 10, 40),    # 128 rows of 32 queries; more splits than blocks
    (1, 2, 8, 64, [900], 12, 12, 7, 5),              # 96 rows: 8 waves, two of them idle
    (2, 4, 4, 128, [3000, 2000], 16, 4, 12, 0),      # 16 rows: one row wave (two token-half waves)
    (4, 8, 4, 128, [2048, 1500, 2048, 777], 16, 4, 19, 0),   # 128 groups: two slots, twice the splits
    (1, 2, 16, 128, [4000], 6, 2, 11, 0),            # 32 rows: two row waves, NQ not a multiple of C
    (2, 2, 1, 64, [1500, 900], 7, 3, 8, 2),          # 3 rows in a 16-row wave
    (1, 4, 8, 64, [3100], 8, 2, 13, 64),             # 16 rows, the most splits
]


@pytest.mark.parametrize("case", CASES)
def test_grouped_exact_on_tiles(case):
    B, H, G, d, lens, NQ, C, nsm, split_k = case
    _say("grouped tiles", case)
    T_cap = max(lens)
    gen = torch.Generator().manual_seed(77 + G + d + C)
    K = torch.randn((B, H, T_cap, d), generator=gen).to(torch.bfloat16)
    V = torch.randn((B, H, T_cap, d), generator=gen).to(torch.bfloat16)
    Q = torch.randn((B, NQ, H * G, d), generator=gen).to(torch.bfloat16)
    rng = np.random.default_rng(C * 31 + G)
    bi = np.full((B, NQ, H, nsm), -1, dtype=np.int32)
    ns = np.zeros((B, NQ, H), dtype=np.int32)
    for b in range(B):
        nb = -(-lens[b] // 64)
        for q in range(NQ):
            for g in range(H):
                if rng.random() < 0.05:
                    continue                                    # an empty list
                n = int(rng.integers(1, min(nsm, nb) + 1))
                # draft queries share blocks: draw from a window of the sequence
                lo = int(rng.integers(0, max(1, nb - 3 * nsm)))
                pool = np.arange(lo, min(nb, lo + 3 * nsm))
                bi[b, q, g, :n] = np.sort(rng.choice(pool, size=min(n, len(pool)), replace=False))
                ns[b, q, g] = min(n, len(pool))
    seq = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    out, lse, uc = sda.sda_grouped_decode(Q.to(DEV), K.to(DEV), V.to(DEV), seq, torch.as_tensor(bi, device=DEV),
                                          torch.as_tensor(ns, device=DEV), C, sda.SDA_GROUP_EXACT, split_k=split_k)
    torch.cuda.synchronize()
    Kd, Vd, Qd = O.bf16_to_f64(bits(K)), O.bf16_to_f64(bits(V)), O.bf16_to_f64(bits(Q))
    o, l, uc = out.double().cpu().numpy(), lse.double().cpu().numpy(), uc.cpu().numpy()
    err = lerr = 0.0
    for b in range(B):
        for gi, grp in enumerate(O.groups(NQ, C)):
            for g in range(H):
                lists = [bi[b, q, g, :ns[b, q, g]] for q in grp]
                # exact mode: every query attends to its own list (the oracle's
                # grouped_row on the queries with a list), the union is counted
                # over all of them
                live = [ci for ci in range(len(grp)) if len(lists[ci])]
                assert uc[b, gi, g] == len(O.union_blocks(lists)), (b, gi, g)
                if live:
                    qrows = np.stack([Qd[b, grp[ci], g * G:(g + 1) * G] for ci in live])
                    want, wl, _ = O.grouped_row(qrows, Kd[b, g], Vd[b, g], [lists[ci] for ci in live], lens[b],
                                                d ** -0.5, O.MODE_EXACT)
                for ci, q in enumerate(grp):
                    sl = slice(g * G, (g + 1) * G)
                    if ci not in live:
                        assert np.all(o[b, q, sl] == 0) and np.all(np.isneginf(l[b, q, sl]))
                        continue
                    k = live.index(ci)
                    err = max(err, float(np.abs(o[b, q, sl] - want[k]).max()))
                    lerr = max(lerr, float(np.abs(l[b, q, sl] - wl[k]).max()))
    _say(f"  max abs err {err:.2e}, lse {lerr:.2e}, mean union {uc.mean():.1f}")
    assert err <= TOL and lerr <= 1e-3


@pytest.mark.parametrize("B,H,G,C", [(2, 4, 8, 16), (4, 8, 4, 4)])
def test_grouped_tiles_repeat_bit_identically(B, H, G, C):
    # the split merge's arrival counters are left at zero: calls in a row on
    # one workspace give identical results
    d, T, NQ = 128, 4096, 16
    _say("grouped tiles repeat", B, H, G, C)
    gen = torch.Generator().manual_seed(5)
    K = torch.randn((B, H, T, d), generator=gen).to(torch.bfloat16).to(DEV)
    V = torch.randn((B, H, T, d), generator=gen).to(torch.bfloat16).to(DEV)
    Q = torch.randn((B, NQ, H * G, d), generator=gen).to(torch.bfloat16).to(DEV)
    bi = torch.sort(torch.randint(0, T // 64, (B, NQ, H, 16), generator=gen), dim=-1).values
    bi = torch.where(torch.cat([torch.ones_like(bi[..., :1], dtype=torch.bool), bi[..., 1:] != bi[..., :-1]], -1),
                     bi, -1)
    bi = torch.sort(torch.where(bi < 0, 1 << 30, bi), dim=-1).values
    ns = (bi < (1 << 30)).sum(-1).to(torch.int32)
    bi = torch.where(bi >= (1 << 30), -1, bi).to(torch.int32)
    seq = torch.full((B,), T, dtype=torch.int32, device=DEV)
    nbytes = sda.lib().sda_grouped_decode_workspace(B, NQ, H * G, H, 16, d, T // 64, C, sda.SDA_GROUP_EXACT, 0)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    first = None
    for _ in range(5):
        out, lse, _ = sda.sda_grouped_decode(Q, K, V, seq, bi.to(DEV), ns.to(DEV), C, sda.SDA_GROUP_EXACT, ws=ws)
        if first is None:
            first = (out.clone(), lse.clone())
        else:
            assert torch.equal(out, first[0]) and torch.equal(lse, first[1])
    # one arrival counter per tile: a tile holds as many whole groups as fit
    # in 128 rows and 32 queries
    tile_q = min((min(32, 128 // G) // C) * C, -(-NQ // C) * C)
    assert int(ws[:4 * B * H * (-(-NQ // tile_q))].view(torch.int32).abs().sum().item()) == 0
