"""Host-side helpers for the GPU parity tests: run the CPU oracle on the
inputs a test drew, build tie-free indexer inputs, and call the HIP path.

Nothing the oracle sees comes from the HIP path: K, V, Q and F come from the
seeded generators; block lists handed to the oracle are the oracle's own,
except where a test checks sparse_decode alone on a given list.
"""
import math

import numpy as np
import torch

import block_sparse_attention_pool_amd as sda
import oracle as O
from synth import inputs

DELTA = 1e-4          # minimum top-k cut gap (float32 decision scores) of a tie-free row
DELTA_REL_MH = 1e-4   # relative cut gap for the G-head comparator's summed softmax
TOL = 2e-3            # max-abs output tolerance (bf16 inputs, fp32 accumulation)

DEV = "cuda"


def bits(t):
    return inputs.bf16_bits(t)


def f64(t):
    return O.bf16_to_f64(bits(t))


# ---------------------------------------------------------------------------
# oracle side
# ---------------------------------------------------------------------------

def oracle_kt(K, T, rows):
    """Oracle compressed keys (as stored: bf16, held in float64) per (b, g)."""
    out = {}
    for (b, g) in rows:
        out[(b, g)] = O.store_bf16(O.compressed_keys(f64(K[b, g, :T]), T))
    return out


def tie_free_indexer(cfg, layer, kt, rows, sigma=None, delta=DELTA, max_iter=200):
    """bf16 F (CPU tensor) whose listed rows (b, q, g) have a top-k cut gap
    of at least delta in float32 decision scores; failing rows are re-drawn."""
    attempts = np.zeros((cfg.B, cfg.NQ, cfg.H_kv), dtype=np.int64)
    nb = O.num_blocks(cfg.T)
    cand = O.candidates(nb, cfg.n_init, cfg.n_local)
    for _ in range(max_iter):
        F = inputs.to_bf16(inputs.indexer_vectors(cfg, layer, attempts, sigma))
        Fd = O.bf16_to_f64(bits(F))
        bad = []
        for (b, q, g) in rows:
            s = O.decision_scores(O.indexer_scores(Fd[b, q, g], kt[(b, g)]))
            if O.cut_gap(s, cand, cfg.top_k) < delta:
                bad.append((b, q, g))
        if not bad:
            return F, attempts
        for r in bad:
            attempts[r] += 1
    raise RuntimeError("could not draw tie-free indexer vectors")


def tie_free_queries_mh(cfg, layer, kt, rows, tau, delta_rel=DELTA_REL_MH, max_iter=200):
    """bf16 Q (CPU tensor) whose listed rows have a relative cut gap of the
    G-head comparator's scores of at least delta_rel."""
    attempts = np.zeros((cfg.B, cfg.NQ, cfg.H_kv), dtype=np.int64)
    nb = O.num_blocks(cfg.T)
    cand = O.candidates(nb, cfg.n_init, cfg.n_local)
    G = cfg.G
    for _ in range(max_iter):
        Q = inputs.to_bf16(inputs.attention_queries(cfg, layer, attempts=attempts))
        Qd = O.bf16_to_f64(bits(Q))
        bad = []
        for (b, q, g) in rows:
            s = O.decision_scores(O.multihead_scores(Qd[b, q, g * G:(g + 1) * G], kt[(b, g)], tau))
            top = np.sort(s[cand])[::-1][cfg.top_k - 1]
            if O.cut_gap(s, cand, cfg.top_k) < delta_rel * abs(top):
                bad.append((b, q, g))
        if not bad:
            return Q, attempts
        for r in bad:
            attempts[r] += 1
    raise RuntimeError("could not draw tie-free queries")


def oracle_select(cfg, Fd, kt, rows):
    return {r: O.select_row(Fd[r], kt[(r[0], r[2])], cfg.n_init, cfg.n_local, cfg.top_k)[0] for r in rows}


class SparseRows:
    """Host float64 views of K/V rows holding only the tokens a test reads
    (zero-filled arrays are allocated lazily by the OS, so untouched tokens
    cost nothing)."""

    def __init__(self, K, V, T):
        self.K, self.V, self.T = K, V, T
        self.cache = {}

    def get(self, b, g, blocks):
        key = (b, g)
        if key not in self.cache:
            d = self.K.shape[-1]
            self.cache[key] = (np.zeros((self.T, d)), np.zeros((self.T, d)), set())
        kf, vf, have = self.cache[key]
        need = [int(j) for j in blocks if int(j) not in have and 0 <= int(j) * 64 < self.T]
        if need:
            toks = O.block_tokens(sorted(need), self.T)
            idx = torch.as_tensor(toks, device=self.K.device)
            kf[toks] = f64(self.K[b, g].index_select(0, idx))
            vf[toks] = f64(self.V[b, g].index_select(0, idx))
            have.update(need)
        return kf, vf


def oracle_decode(Qd, rows_kv, b, q, g, G, blocks, T, scale):
    kf, vf = rows_kv.get(b, g, blocks)
    return O.decode_row(Qd[b, q, g * G:(g + 1) * G], kf, vf, blocks, T, scale)


# ---------------------------------------------------------------------------
# GPU side (HIP path through the C ABI)
# ---------------------------------------------------------------------------

def gpu_ktilde(K, T, NB_cap=None):
    B, H, Tc, d = K.shape
    NB_cap = NB_cap or -(-Tc // 64)
    kt = torch.zeros((B, H, NB_cap, d), dtype=torch.bfloat16, device=K.device)
    lo = torch.zeros(B, dtype=torch.int32, device=K.device)
    hi = torch.full((B,), T, dtype=torch.int32, device=K.device)
    sda.sda_update_compressed_keys(K, kt, lo, hi, T)
    return kt


def seq(cfg, T=None):
    return torch.full((cfg.B,), cfg.T if T is None else T, dtype=torch.int32, device=DEV)


def rows_of(cfg):
    return [(b, q, g) for b in range(cfg.B) for q in range(cfg.NQ) for g in range(cfg.H_kv)]


def scale_of(cfg):
    return 1.0 / math.sqrt(cfg.d)
