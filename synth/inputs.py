"""Seeded draws for the decode workloads.

Every tensor is drawn from its own seed, derived from (base seed, config id,
tensor name, indices) with numpy's SeedSequence, so any tensor can be re-drawn
alone on any device.  Large K/V tensors use torch's generator on the device
they are wanted on (Philox on the GPU, MT on the CPU); the small indexer and
query vectors always come from numpy PCG64 on the host, so they are identical
wherever they are used.  Values are drawn in float32 and rounded to bfloat16
with round-to-nearest-even by torch's dtype conversion.

Nothing here pools, scores, selects or attends: the structure a workload needs
(which blocks carry a key bias, how noisy a draft query is) is expressed as
plain random draws and additions.
"""
import zlib

import numpy as np
import torch

from .configs import BLOCK

BASE_SEED = 20260624

# relative scale of the perturbation used when a row's indexer vector is
# re-drawn (attempt >= 1); a fraction of the row's own noise scale keeps the
# row's structure (bias alignment, draft-query similarity) intact
REDRAW_SCALE = 0.25


def derive_seed(cid, name, *idx):
    words = [BASE_SEED + int(cid), zlib.crc32(name.encode())] + [int(i) for i in idx]
    state = np.random.SeedSequence(words).generate_state(2, dtype=np.uint32)
    return int((int(state[0]) << 31) ^ int(state[1])) & 0x7FFF_FFFF_FFFF_FFFF


def _torch_gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def bf16_bits(t):
    """bfloat16 tensor -> numpy uint16 array of its bit patterns (host copy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# keys and values
# --------------------------------------------------------------------------

def kv_layer(cfg, layer, device="cpu", t_cap=None, bias_dirs=None, out=None, gen_device=None):
    """K and V caches of one layer, bf16 [B, H_kv, t_cap, d], N(0,1).

    Tokens at or beyond cfg.T (when t_cap > T) are drawn too; they are never
    read by a correct kernel.  ``bias_dirs`` (config 2) is a float32 tensor
    [B, H_kv, d] of unit directions and a boolean block mask
    ``bias_blocks`` [B, H_kv, NB] is drawn here: every key in a biased block
    gets ``cfg.bias_beta * dir`` added before rounding.
    ``out`` may supply preallocated (K, V) tensors (e.g. pinned host memory);
    ``gen_device`` is where the draws are made (default: ``device``).  The
    same seed gives different values on a CPU and a GPU generator, so both
    sides of a comparison must take their copy of one draw.
    """
    t_cap = cfg.T if t_cap is None else t_cap
    shape = (cfg.B, cfg.H_kv, t_cap, cfg.d)
    if out is None:
        K = torch.empty(shape, dtype=torch.bfloat16, device=device)
        V = torch.empty(shape, dtype=torch.bfloat16, device=device)
    else:
        K, V = out
    gen_dev = device if gen_device is None else gen_device
    bias_blocks = None
    if bias_dirs is not None:
        bias_blocks = biased_block_mask(cfg, layer)
    for name, dst in (("K", K), ("V", V)):
        g = _torch_gen(derive_seed(cfg.cid, name, layer), gen_dev)
        for b in range(cfg.B):
            slab = torch.randn((cfg.H_kv, t_cap, cfg.d), generator=g, device=gen_dev,
                               dtype=torch.float32)
            if name == "K" and bias_blocks is not None:
                nb = bias_blocks.shape[-1]
                m = torch.zeros((cfg.H_kv, t_cap), dtype=torch.float32, device=gen_dev)
                mb = torch.as_tensor(bias_blocks[b], device=gen_dev).to(torch.float32)
                m[:, : nb * BLOCK] = mb.repeat_interleave(BLOCK, dim=1)[:, : min(t_cap, nb * BLOCK)]
                dirs = bias_dirs[b].to(gen_dev, torch.float32)
                slab += cfg.bias_beta * m[:, :, None] * dirs[:, None, :]
            dst[b].copy_(slab.to(torch.bfloat16))
            del slab
    return K, V, bias_blocks


def biased_block_mask(cfg, layer):
    """Boolean [B, H_kv, NB]: round(bias_frac * NB) blocks per (b, kv head),
    drawn without replacement from the blocks that are neither initial nor local."""
    nb = cfg.NB
    lo, hi = cfg.n_init, nb - cfg.n_local
    n_b = int(round(cfg.bias_frac * nb))
    mask = np.zeros((cfg.B, cfg.H_kv, nb), dtype=bool)
    for b in range(cfg.B):
        for g in range(cfg.H_kv):
            rng = np.random.Generator(np.random.PCG64(derive_seed(cfg.cid, "bias_blocks", layer, b, g)))
            pick = rng.choice(np.arange(lo, hi), size=min(n_b, hi - lo), replace=False)
            mask[b, g, pick] = True
    return mask


# --------------------------------------------------------------------------
# indexer (Forecast) vectors and attention queries
# --------------------------------------------------------------------------

def _row_rng(cid, name, *idx):
    return np.random.Generator(np.random.PCG64(derive_seed(cid, name, *idx)))


def indexer_vectors(cfg, layer, attempts=None, sigma=None):
    """Indexer vectors F, float32 numpy [B, NQ, H_kv, d] (round with to_bf16).

    Plain configs: F ~ N(0, 1/d) per row.  Draft-query configs (NQ > 1, a
    given ``sigma``): f = f0 + sigma * eps with f0, eps ~ N(0, 1/d) and f0
    shared by all queries of a sequence and KV head.  ``attempts`` [B, NQ, H_kv]
    (int) re-draws a row: attempt a >= 1 adds REDRAW_SCALE * (row noise scale)
    * N(0, 1/d) from a seed that includes a.
    """
    B, NQ, H, d = cfg.B, cfg.NQ, cfg.H_kv, cfg.d
    s = 1.0 / np.sqrt(d)
    F = np.empty((B, NQ, H, d), dtype=np.float64)
    for b in range(B):
        for g in range(H):
            base = _row_rng(cfg.cid, "F0", layer, b, g).standard_normal(d) * s
            for q in range(NQ):
                if sigma is None:
                    f = base if NQ == 1 else _row_rng(cfg.cid, "Fq", layer, b, q, g).standard_normal(d) * s
                    scale = s
                else:
                    eps = _row_rng(cfg.cid, "Feps", layer, b, q, g).standard_normal(d) * s
                    f = base + sigma * eps
                    scale = sigma * s
                a = 0 if attempts is None else int(attempts[b, q, g])
                if a > 0:
                    f = f + REDRAW_SCALE * scale * _row_rng(cfg.cid, "Fredraw", layer, b, q, g, a).standard_normal(d)
                F[b, q, g] = f
    return F.astype(np.float32)


def bias_directions(F):
    """Unit directions F/|F| per (b, kv head) from the first query's vector,
    float32 torch [B, H_kv, d]; the config-2 key bias is drawn along them."""
    f = F[:, 0].astype(np.float64)
    u = f / np.linalg.norm(f, axis=-1, keepdims=True)
    return torch.from_numpy(u.astype(np.float32))


def attention_queries(cfg, layer, sigma=None, attempts=None):
    """Attention queries Q, float32 numpy [B, NQ, H_q, d], N(0,1).

    Draft-query configs: q = q0 + sigma * eps with q0 shared across the
    sequence's queries.  ``attempts`` [B, NQ, H_kv] re-draws the G heads of a
    KV group: attempt a >= 1 adds REDRAW_SCALE * N(0,1) from a seed that
    includes a."""
    B, NQ, H, d = cfg.B, cfg.NQ, cfg.H_q, cfg.d
    G = H // cfg.H_kv
    Q = np.empty((B, NQ, H, d), dtype=np.float64)
    for b in range(B):
        base = _row_rng(cfg.cid, "Q0", layer, b).standard_normal((H, d))
        for q in range(NQ):
            if NQ == 1:
                Q[b, q] = base
            elif sigma is None:
                Q[b, q] = _row_rng(cfg.cid, "Qq", layer, b, q).standard_normal((H, d))
            else:
                Q[b, q] = base + sigma * _row_rng(cfg.cid, "Qeps", layer, b, q).standard_normal((H, d))
            if attempts is not None:
                for g in range(cfg.H_kv):
                    a = int(attempts[b, q, g])
                    if a > 0:
                        Q[b, q, g * G:(g + 1) * G] += REDRAW_SCALE * _row_rng(
                            cfg.cid, "Qredraw", layer, b, q, g, a).standard_normal((G, d))
    return Q.astype(np.float32)


def to_bf16(x, device="cpu"):
    """float32 numpy/torch -> bf16 torch tensor (round to nearest even)."""
    t = torch.as_tensor(x, dtype=torch.float32)
    return t.to(torch.bfloat16).to(device)


def seq_lens(cfg, device="cpu"):
    return torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=device)


# --------------------------------------------------------------------------
# prefill: indexer vectors and queries of every position of a sequence
# --------------------------------------------------------------------------

PREFILL_RHO = 0.96     # correlation of consecutive positions' indexer vectors


def prefill_indexer_vectors(cfg, layer, nq, pos0=0, rho=PREFILL_RHO):
    """Indexer vectors of nq consecutive positions, float32 numpy
    [B, nq, H_kv, d]: per (b, KV head) a stationary first-order
    autoregressive sequence with N(0, 1/d) marginals, f_t = rho f_{t-1} +
    sqrt(1 - rho^2) e_t (consecutive positions' vectors correlate by rho, so
    their selections overlap as neighbouring queries' do); positions
    pos0 .. pos0 + nq - 1 of the sequence drawn from position 0."""
    from scipy.signal import lfilter
    B, H, d = cfg.B, cfg.H_kv, cfg.d
    n = int(pos0) + int(nq)
    out = np.empty((B, nq, H, d), dtype=np.float32)
    c = np.sqrt(1.0 - rho * rho)
    for b in range(B):
        e = _row_rng(cfg.cid, "Fprefill", layer, b).standard_normal((n, H, d)) / np.sqrt(d)
        e[0] /= c                                       # stationary start: f_0 = e_0
        f = lfilter([c], [1.0, -rho], e, axis=0)
        out[b] = f[pos0:].astype(np.float32)
    return out


def prefill_queries(cfg, layer, nq, device="cpu"):
    """Attention queries of nq positions, bf16 [B, nq, H_q, d], N(0,1), drawn
    by torch's generator on `device` (one seed per (config, layer))."""
    g = _torch_gen(derive_seed(cfg.cid, "Qprefill", layer), device)
    Q = torch.empty((cfg.B, nq, cfg.H_q, cfg.d), dtype=torch.bfloat16, device=device)
    for b in range(cfg.B):
        Q[b].copy_(torch.randn((nq, cfg.H_q, cfg.d), generator=g, device=device, dtype=torch.float32)
                   .to(torch.bfloat16))
    return Q
