"""The allocation-free decode step (sda_decode_step_noalloc) against
sda_decode_step with its own workspace, through the C ABI: identical block
sets, outputs within 1e-5 (the same kernels and launch plan, so in practice
identical bits), on calls in a row whose shapes shrink and then grow again
(the static scratch keeps the previous call's partials; its counters must
be back at zero)."""
import sys

import pytest
import torch

import block_sparse_attention_pool_amd as sda
import synth
from synth import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sda.lib()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _ktilde(K, lens, NB_cap):
    B, H, _, d = K.shape
    kt = torch.zeros((B, H, NB_cap, d), dtype=torch.bfloat16, device=DEV)
    sda.sda_update_compressed_keys(K, kt, torch.zeros(B, dtype=torch.int32, device=DEV), lens, K.shape[2])
    return kt


def _case_config(cid):
    cfg = synth.get_config(cid)
    K0, V0, _ = inputs.kv_layer(cfg, 0, device=DEV)
    K1, _, _ = inputs.kv_layer(cfg, 1, device=DEV)
    seq = torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=DEV)
    kt0, kt1 = _ktilde(K0, seq, cfg.NB), _ktilde(K1, seq, cfg.NB)
    del K1
    F0 = inputs.to_bf16(inputs.indexer_vectors(cfg, 0)).to(DEV)
    F1 = inputs.to_bf16(inputs.indexer_vectors(cfg, 1)).to(DEV)
    Q = inputs.to_bf16(inputs.attention_queries(cfg, 0)).to(DEV)
    sel = (cfg.n_init, cfg.n_local, cfg.top_k)
    bi0, ns0 = sda.sda_score_select(F0, kt0, seq, *sel)
    return (Q, K0, V0, seq, bi0, ns0, F1, kt1, seq) + sel, dict(k_tilde_cur=None)


def _case_ragged(top_k):
    B, H_kv, G, d, T_cap, NBn = 3, 2, 4, 128, 5000, 300
    gen = torch.Generator(device=DEV).manual_seed(11 + top_k)

    def rnd(*shape, scale=1.0):
        return (torch.randn(*shape, generator=gen, device=DEV) * scale).to(torch.bfloat16)
    K, V, Kn = rnd(B, H_kv, T_cap, d), rnd(B, H_kv, T_cap, d), rnd(B, H_kv, NBn * 64, d)
    Q, F0, F1 = rnd(B, 1, H_kv * G, d), rnd(B, 1, H_kv, d, scale=d ** -0.5), rnd(B, 1, H_kv, d, scale=d ** -0.5)
    seq0 = torch.tensor([5000, 3000, 65], dtype=torch.int32, device=DEV)
    seq1 = torch.tensor([NBn * 64 - 5, 64 * 3, 1], dtype=torch.int32, device=DEV)
    kt0 = _ktilde(K, seq0, -(-T_cap // 64))
    kt1 = _ktilde(Kn, seq1, NBn)
    sel = (1, 2, top_k)
    bi0, ns0 = sda.sda_score_select(F0, kt0, seq0, *sel)
    old0 = seq0 - torch.tensor([70, 1, 1], dtype=torch.int32, device=DEV)
    kt0r = _ktilde(K, old0, -(-T_cap // 64))
    return (Q, K, V, seq0, bi0, ns0, F1, kt1, seq1) + sel, dict(k_tilde_cur=kt0r, len_old_cur=old0,
                                                               max_new_tokens_cur=70)


def _compare(tag, args, kw):
    kt_cur = kw.get("k_tilde_cur")
    kw_ref = dict(kw)
    if kt_cur is not None:
        kw_ref["k_tilde_cur"] = kt_cur.clone()
    ref = sda.sda_decode_step(*args, **kw_ref)
    got = sda.sda_decode_step_noalloc(*args, **kw)
    torch.cuda.synchronize()
    out, lse, bi, ns = got
    r_out, r_lse, r_bi, r_ns = ref
    _say(f"{tag}: max |noalloc - workspace| out {(out - r_out).abs().max().item():.2e}")
    assert torch.equal(bi, r_bi) and torch.equal(ns, r_ns), tag
    assert (out - r_out).abs().max().item() <= 1e-5, tag
    assert ((lse - r_lse).abs().nan_to_num(0.0)).max().item() <= 1e-5, tag
    if kt_cur is not None:
        assert torch.equal(kt_cur, kw_ref["k_tilde_cur"]), tag


def test_noalloc_step_matches_workspace_step_as_shapes_change():
    big = _case_config(3)                 # 128K, 8 sequences: one launch, 2 splits
    small = _case_ragged(32)              # ragged lengths, refresh: one launch
    unfused = _case_ragged(80)            # top_k past the in-launch selection: the calls
    _compare("128K", *big)
    _compare("ragged, smaller", *small)
    _compare("ragged, two calls", *unfused)
    _compare("128K again", *big)
    _compare("ragged again", *small)


def test_noalloc_step_replays_in_a_graph():
    # the callers this entry point serves capture it: a prepared call
    # captured in a HIP graph (after one eager call, which sets the scratch
    # up), replayed with eager work in between, equals the workspace step
    args, kw = _case_ragged(32)
    kw = dict(kw)
    kw["k_tilde_cur"] = None
    kw.pop("len_old_cur", None)
    kw.pop("max_new_tokens_cur", None)
    ref = [t.clone() for t in sda.sda_decode_step(*args, **kw)]
    call, outs = sda.prepare(sda.sda_decode_step_noalloc, *args, **kw)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call.run()
    for r in range(4):
        for o in outs:
            o.fill_(-7) if o.dtype == torch.int32 else o.zero_()
        g.replay()
        torch.cuda.synchronize()
        out, lse, bi, ns = outs
        assert torch.equal(bi, ref[2]) and torch.equal(ns, ref[3]), r
        assert (out - ref[0]).abs().max().item() <= 1e-5, r
        # eager work between replays: the workspace step on the other buffers
        sda.sda_decode_step(*args, **kw)
        torch.cuda.synchronize()


def test_noalloc_rejects_a_call_beyond_its_scratch():
    B, H_kv, G, d, T = 64, 8, 8, 128, 4096
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device=DEV)
    seq = torch.full((B,), T, dtype=torch.int32, device=DEV)
    bi = torch.zeros((B, 1, H_kv, 35), dtype=torch.int32, device=DEV)
    ns = torch.zeros((B, 1, H_kv), dtype=torch.int32, device=DEV)
    with pytest.raises(sda.SdaError, match="static scratch"):
        sda.sda_decode_step_noalloc(z(B, 1, H_kv * G, d), z(B, H_kv, T, d), z(B, H_kv, T, d), seq, bi, ns,
                                    z(B, 1, H_kv, d), z(B, H_kv, T // 64, d), seq, 1, 2, 32, split_k=8)
