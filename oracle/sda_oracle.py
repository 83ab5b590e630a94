"""CPU oracle for top-k block-sparse decode attention (test infrastructure).

This module is the plain, slow, float64 statement of what the decode path
computes.  It is test infrastructure: only the test suite, the package smoke
check and the benchmark's CPU-baseline leg may import it.  The HIP library
never calls it, and it shares no code, table or helper with the HIP library.

Sources (cited by page title and section/equation):
  [SparDA]  reading note "SparDA：稀疏解耦注意力，让长上下文推理又快又准"
            (zhongzhuzhou.org, 2026-06-24) on SparDA: Sparse Decoupled
            Attention (arXiv 2606.04511).
  [SSV]     reading note "SSV：稀疏投机验证——在动态稀疏注意力中做投机解码"
            (zhongzhuzhou.org, 2026-07-01) on SSV: Sparse Speculative
            Verification (arXiv 2605.19893).

Arithmetic is float64 throughout.  bf16 inputs arrive as uint16 bit patterns
and are decoded exactly.  Two places store or decide in a narrower format,
because the kernel's stored tensor or decision is narrower and an integer
result must be decided in the same precision on both sides:
  * the compressed key cache is stored in bf16, the KV cache's format: the
    float64 block mean rounded once to the nearest bf16, ties to even
    (``store_bf16``).  A block mean of bf16 keys is exact in float64 when the
    block's non-zero magnitudes lie within a factor 2^39 of each other, so
    the stored bits are then a function of the keys alone;
  * top-k ranks block scores after rounding them to float32
    (``decision_scores``); equal float32 scores go to the lower block index.

Readings of points the pages leave open (numbered as in the design notes):
  block = pooling kernel = stride = 64 tokens; a partial last block is the
  mean of the tokens present; the local window is the last n_local blocks;
  init/local blocks do not compete in top-k; output block lists ascend;
  query head h reads KV head floor(h / G); attention scale 1/sqrt(d);
  the G-head comparator sums per-head softmax over all blocks with tau = sqrt(d);
  with overlapping compression (kernel l, stride s) a block's score is the
  max over the compressed windows that share a token with it; NSA's
  compressed branch attends to every compressed entry present at length T,
  its window branch to the last w cached tokens, and the branch gates are
  inputs (one triple per query head); in prefill every query position p
  selects and attends as a decode step at length p + 1 would (per-token
  selection, causal), with at least one local block so that every scored
  block is complete; in a refresh/reuse layer chain a reuse layer takes the
  block lists of the latest refresh layer unchanged.

Parity pins: every function here is pinned by tests under tests/ against
closed forms, brute force or an independent library routine, except the
comparator's temperature tau, which the pages never give ("parity unpinned"
for the value of tau only; its ranking with G = 1 is pinned).
"""
import numpy as np

BLOCK = 64


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def bf16_to_f64(bits):
    """Exact decode of bf16 bit patterns (uint16 array) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def store_bf16(x):
    """Round float64 values to the nearest bf16 (8 significant bits, 8-bit
    exponent), ties to even, returned as float64: the compressed-key cache's
    stored values.  Below the normal range the grid stays at 2^-133 (bf16
    subnormals); beyond the largest finite bf16 the result is +-inf."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # |x| = m * 2^e, 0.5 <= m < 1
    e = np.maximum(e, -125)                 # the grid of the smallest binade
    r = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)   # rint: ties to even
    big = np.abs(r) >= 2.0 ** 128
    return np.where(big, np.copysign(np.inf, x), r)


def decision_scores(s):
    """Scores as ranked by top-k: float64 values rounded to float32."""
    return np.asarray(s, dtype=np.float64).astype(np.float32).astype(np.float64)


def num_blocks(T, block=BLOCK):
    return -(-int(T) // block)


# ---------------------------------------------------------------------------
# O1  compressed keys  ([SparDA] prerequisites §3, eq. (4); §4.2 step 1; §4.6)
# ---------------------------------------------------------------------------

def compressed_keys(k, T, block=BLOCK):
    """Mean-pooled keys over non-overlapping blocks.

    k: float64 [>=T, d] keys of one (sequence, KV head); T cached tokens.
    Returns float64 [ceil(T/block), d]; block j is the mean of tokens
    j*block .. min(j*block+block, T)-1 (eq. (4) with kernel = stride = block;
    a partial last block averages the tokens it has).
    """
    T = int(T)
    nb = num_blocks(T, block)
    out = np.empty((nb, k.shape[-1]), dtype=np.float64)
    for j in range(nb):
        lo, hi = j * block, min(j * block + block, T)
        out[j] = np.mean(k[lo:hi], axis=0)
    return out


def append_token(kt, T_old, k_new, block=BLOCK):
    """Per-token incremental update of the compressed keys, O(d) work.

    The decode step appends one key and refreshes the pooled cache
    incrementally ([SparDA] §4.2 step 1, §4.6).  kt: float64 [>=ceil(T_old/block), d]
    (rows past the last block are ignored); returns the array for T_old + 1
    tokens.  A key that opens a new block becomes that block's mean; otherwise
    the running mean of the last block moves by (k_new - mean) / (n + 1).
    """
    T_old = int(T_old)
    nb_old = num_blocks(T_old, block)
    n_in_last = T_old - (nb_old - 1) * block if T_old > 0 else 0
    if T_old % block == 0:
        out = np.zeros((nb_old + 1, k_new.shape[-1]), dtype=np.float64)
        out[:nb_old] = kt[:nb_old]
        out[nb_old] = k_new
        return out
    out = np.array(kt[:nb_old], dtype=np.float64, copy=True)
    out[nb_old - 1] = out[nb_old - 1] + (k_new - out[nb_old - 1]) / (n_in_last + 1)
    return out


# ---------------------------------------------------------------------------
# O2-O6  block selection  ([SparDA] eq. (3), eq. (6), eq. (9), §4.2 step 2;
#        [SSV] NSA selection branch, steps 1-2)
# ---------------------------------------------------------------------------

def init_local(nb, n_init, n_local):
    """Initial blocks {0..n_init-1} and local blocks {nb-n_local..nb-1},
    both clipped to [0, nb) (eq. (3)): returns (init_set, local_set)."""
    init = set(range(0, min(n_init, nb)))
    local = set(range(max(0, nb - n_local), nb))
    return init, local


def candidates(nb, n_init, n_local):
    """Blocks that compete in top-k: all blocks minus the initial and local
    ones (§4.2 step 2 excludes the fixed blocks before top-k).  Ascending."""
    init, local = init_local(nb, n_init, n_local)
    return np.array([j for j in range(nb) if j not in init and j not in local], dtype=np.int64)


def indexer_scores(f, kt):
    """Raw block scores s_j = f . K~_j for every block (eq. (6) and (9)).

    The softmax over blocks with temperature in eq. (9) is monotone, so it
    does not change which blocks are chosen; the raw dot product is what the
    decode-time indexer ranks.  f: float64 [d]; kt: float64 [nb, d].
    """
    return kt @ np.asarray(f, dtype=np.float64)


def top_k(scores, cand, k):
    """The k candidates of largest score, ties to the lower block index
    (f_top in eq. (6)).  scores: [nb] (decision precision); cand: ascending
    candidate block ids.  Returns the chosen ids in rank order."""
    cand = np.asarray(cand, dtype=np.int64)
    if k <= 0 or cand.size == 0:
        return np.zeros(0, dtype=np.int64)
    s = np.asarray(scores, dtype=np.float64)[cand]
    order = np.lexsort((cand, -s))          # primary: -score, secondary: index
    return cand[order[: min(int(k), cand.size)]]


def block_set(nb, n_init, n_local, chosen):
    """B = B_init U B_local U B_topk as an ascending list without repeats (eq. (3))."""
    init, local = init_local(nb, n_init, n_local)
    return np.array(sorted(init | local | set(int(j) for j in chosen)), dtype=np.int64)


def select_row(f, kt_stored, n_init, n_local, k):
    """Steps O2-O6 for one row: returns (ascending block ids, decision scores)."""
    nb = kt_stored.shape[0]
    s = decision_scores(indexer_scores(f, kt_stored))
    cand = candidates(nb, n_init, n_local)
    return block_set(nb, n_init, n_local, top_k(s, cand, k)), s


def cut_gap(scores, cand, k):
    """Gap between the k-th and (k+1)-th best candidate scores (inf when
    every candidate or none is chosen).  Used to build inputs without
    near-ties at the top-k cut."""
    cand = np.asarray(cand, dtype=np.int64)
    if k <= 0 or k >= cand.size:
        return np.inf
    s = np.sort(np.asarray(scores, dtype=np.float64)[cand])[::-1]
    return float(s[k - 1] - s[k])


# ---------------------------------------------------------------------------
# O10  G-head comparator  ([SparDA] §4.3 eq. (8); §4.4 eq. (10))
# ---------------------------------------------------------------------------

def multihead_scores(q_heads, kt, tau):
    """InfLLM-V2-style block importance from all G query heads of a group:
    s_j = sum_h softmax_j(q_h . K~_j / tau), softmax over all nb blocks.
    q_heads: float64 [G, d]; kt: float64 [nb, d].  With kernel = stride =
    block the max-pool onto the block grid is the identity."""
    z = (np.asarray(q_heads, dtype=np.float64) @ kt.T) / float(tau)   # [G, nb]
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    p = e / e.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


def select_row_multihead(q_heads, kt_stored, n_init, n_local, k, tau):
    nb = kt_stored.shape[0]
    s = decision_scores(multihead_scores(q_heads, kt_stored, tau))
    cand = candidates(nb, n_init, n_local)
    return block_set(nb, n_init, n_local, top_k(s, cand, k)), s


# ---------------------------------------------------------------------------
# O12  overlapping compression and max-pool onto the block grid
#      ([SparDA] prerequisites §3 eq. (4) with general kernel l and stride s;
#      §4.4: inference compression l = 32, s = 16; §4.3 and fig. 3: the
#      compressed scores are max-pooled onto the block grid)
# ---------------------------------------------------------------------------

def num_entries(T, stride):
    """Compressed entries of a T-token sequence: the windows that start
    before T, i.e. ceil(T / stride)."""
    return -(-int(T) // int(stride))


def compressed_keys_strided(k, T, window, stride):
    """eq. (4) with kernel l = window and stride s: entry j is the mean of
    tokens j*s .. min(j*s + l, T) - 1, for every j with j*s < T.  The last
    windows are cut at T (Python-slice semantics, as for a partial block).
    With window = stride = 64 this is compressed_keys.
    k: float64 [>=T, d].  Returns float64 [ceil(T/s), d]."""
    T = int(T)
    n = num_entries(T, stride)
    out = np.empty((n, k.shape[-1]), dtype=np.float64)
    for j in range(n):
        lo, hi = j * stride, min(j * stride + window, T)
        out[j] = np.mean(k[lo:hi], axis=0)
    return out


def pool_range(J, window, stride, n_entries, block=BLOCK):
    """Entries whose windows share at least one token with block J (reading:
    the max-pool window of a block is every compressed window that overlaps
    it): j*s < (J+1)*block and j*s + l > J*block, clipped to the entries
    that exist.  Returns the inclusive range (lo, hi)."""
    lo = max(0, -(-(J * block - window + 1) // stride))
    hi = min(n_entries - 1, ((J + 1) * block - 1) // stride)
    return lo, hi


def max_pool_blocks(entry_scores, T, window, stride, block=BLOCK):
    """Block score = max of the scores of the compressed windows that overlap
    the block.  entry_scores: [ceil(T/s)]; returns [ceil(T/block)]."""
    e = np.asarray(entry_scores, dtype=np.float64)
    nb = num_blocks(T, block)
    out = np.empty(nb, dtype=np.float64)
    for J in range(nb):
        lo, hi = pool_range(J, window, stride, e.size, block)
        out[J] = e[lo:hi + 1].max()
    return out


def select_row_pooled(f, kt_stored, T, window, stride, n_init, n_local, k):
    """O2-O6 on max-pooled block scores: the indexer scores every compressed
    entry (ranked in float32, as the kernel decides), the scores are pooled
    onto the 64-token blocks, then init U local U top-k as in select_row.
    kt_stored: stored compressed keys [ceil(T/s), d].  Returns (ascending
    block ids, pooled decision scores)."""
    s_entries = decision_scores(indexer_scores(f, kt_stored))
    s = max_pool_blocks(s_entries, T, window, stride)
    nb = num_blocks(T)
    cand = candidates(nb, n_init, n_local)
    return block_set(nb, n_init, n_local, top_k(s, cand, k)), s


def select_row_multihead_pooled(q_heads, kt_stored, T, window, stride, n_init, n_local, k, tau):
    """InfLLM-V2's selector on overlapping compressed keys ([SparDA] §4.3
    eq. (8) and fig. 3: per-head softmax over the compressed entries, sum over
    the heads, max-pool onto the block grid; §4.4: l = 32, s = 16): the
    summed softmax weight of every entry (ranked in float32, as the kernel
    decides), max-pooled over the windows that share a token with each
    block, then init U local U top-k.  kt_stored: [ceil(T/s), d].  Returns
    (ascending block ids, pooled decision scores)."""
    s_entries = decision_scores(multihead_scores(q_heads, kt_stored, tau))
    s = max_pool_blocks(s_entries, T, window, stride)
    nb = num_blocks(T)
    cand = candidates(nb, n_init, n_local)
    return block_set(nb, n_init, n_local, top_k(s, cand, k)), s


# ---------------------------------------------------------------------------
# O7  attention over the selected blocks  ([SparDA] eq. (7); [SSV] NSA
#     selection-branch attention, step 3)
# ---------------------------------------------------------------------------

def block_tokens(blocks, T, block=BLOCK):
    """Token positions covered by the blocks, clipped at T, in block order."""
    T = int(T)
    parts = [np.arange(j * block, min(j * block + block, T)) for j in blocks if j * block < T]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def attend(q, k, v, blocks, T, scale):
    """softmax(q K_B^T * scale) V_B for one query head; two-pass softmax.

    q: float64 [d]; k, v: float64 [>=T, d]; returns (o [d], lse) with lse the
    natural-log sum of exp of the scaled scores."""
    tok = block_tokens(blocks, T)
    z = (k[tok] @ np.asarray(q, dtype=np.float64)) * float(scale)
    m = z.max()
    p = np.exp(z - m)
    l = p.sum()
    return (p @ v[tok]) / l, float(m + np.log(l))


def decode_row(q_heads, k, v, blocks, T, scale):
    """O7 for every query head that shares one KV head: q_heads [G, d]."""
    outs, lses = [], []
    for h in range(q_heads.shape[0]):
        o, lse = attend(q_heads[h], k, v, blocks, T, scale)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.array(lses)


# ---------------------------------------------------------------------------
# O8-O9  grouped verification  ([SSV] core mechanism 1: grouping, mode A
#        exact merge, mode B shared representative, bandwidth-saving formula;
#        verification-kernel algorithm steps 2-3)
# ---------------------------------------------------------------------------

MODE_EXACT = 0
MODE_SHARED_REP = 1


def groups(nq, C):
    """Consecutive groups of C queries; the last one may be smaller."""
    return [list(range(s, min(s + C, nq))) for s in range(0, nq, C)]


def union_blocks(lists):
    """I_merged = union of the group's block lists, ascending."""
    u = set()
    for lst in lists:
        u |= set(int(j) for j in lst)
    return np.array(sorted(u), dtype=np.int64)


def load_counts(lists):
    """How many times each block would be loaded if every query loaded its own list."""
    c = {}
    for lst in lists:
        for j in lst:
            c[int(j)] = c.get(int(j), 0) + 1
    return c


def grouped_row(q_rows, k, v, lists, T, scale, mode):
    """Grouped attention for one (sequence, group, KV head).

    q_rows: float64 [C, G, d] (query c, head h); lists: the C block lists.
    Mode A: query c attends to its own list (the merged set is only what is
    loaded).  Mode B: every query attends to the first query's list.
    Returns (out [C, G, d], lse [C, G], union_count)."""
    C = len(lists)
    if mode == MODE_EXACT:
        active = list(lists)
        ucount = len(union_blocks(lists))
    else:
        active = [lists[0]] * C
        ucount = len(union_blocks([lists[0]]))
    outs, lses = [], []
    for c in range(C):
        o, l = decode_row(q_rows[c], k, v, active[c], T, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses), ucount


def union_size_formula(n, C, gamma):
    """Approximate merged-set size n * (1 + (C-1)(1-gamma)) ([SSV] bandwidth-saving formula)."""
    return n * (1.0 + (C - 1) * (1.0 - gamma))


def saving_formula(C, gamma):
    """Fraction of block loads saved by merging: (C-1) * gamma / C."""
    return (C - 1) * gamma / C


# ---------------------------------------------------------------------------
# O13  NSA's three branches and their gated sum, as the SSV verification
#      kernel outputs them ([SSV] NSA three-branch derivation, steps 3-6;
#      verification-kernel algorithm step 3c)
# ---------------------------------------------------------------------------

def attend_tokens(q, k, v, tokens, scale):
    """softmax(q K_tok^T * scale) V_tok over the listed token rows; two-pass
    softmax.  Returns (o [d], lse); an empty token list gives (0, -inf)."""
    tok = np.asarray(tokens, dtype=np.int64)
    if tok.size == 0:
        return np.zeros(k.shape[-1]), -np.inf
    z = (k[tok] @ np.asarray(q, dtype=np.float64)) * float(scale)
    m = z.max()
    p = np.exp(z - m)
    l = p.sum()
    return (p @ v[tok]) / l, float(m + np.log(l))


def window_tokens(T, window):
    """The sliding-window branch's tokens: the last `window` cached tokens,
    [max(0, T - window), T) (the token being decoded is cached, reading 21)."""
    return np.arange(max(0, int(T) - int(window)), int(T), dtype=np.int64)


def nsa_row(q_heads, k, v, kc, vc, blocks, T, n_cmp, window, gates, scale):
    """Gated NSA output of the G query heads that share one KV head:
    o_h = g_c * Attn(q_h, K~, V~) + g_s * Attn(q_h, K_B, V_B) + g_w * Attn(q_h, K_win, V_win)
    with the compressed branch over the n_cmp compressed keys and values
    (kc, vc: [>= n_cmp, d]), the selection branch over the tokens of the
    listed blocks, the window branch over the last `window` tokens.
    gates: [G, 3] (g_c, g_s, g_w) per head.  Returns (out [G, d],
    branch outputs [3, G, d], branch lse [3, G])."""
    G = q_heads.shape[0]
    sel_tok = block_tokens(blocks, T)
    win_tok = window_tokens(T, window)
    cmp_tok = np.arange(int(n_cmp), dtype=np.int64)
    out = np.zeros((G, k.shape[-1]))
    br = np.zeros((3, G, k.shape[-1]))
    lse = np.zeros((3, G))
    for h in range(G):
        for b, (kk, vv, tok) in enumerate(((kc, vc, cmp_tok), (k, v, sel_tok), (k, v, win_tok))):
            br[b, h], lse[b, h] = attend_tokens(q_heads[h], kk, vv, tok, scale)
        out[h] = gates[h, 0] * br[0, h] + gates[h, 1] * br[1, h] + gates[h, 2] * br[2, h]
    return out, br, lse


def grouped_nsa_row(q_rows, k, v, kc, vc, lists, T, n_cmp, window, gates, scale, mode):
    """The verification kernel's output for one group of C draft queries of
    one KV head: the selection branch attends to each query's own list
    (mode A) or the first query's (mode B); the compressed and window
    branches see the same committed prefix for every query (reading 14).
    q_rows: [C, G, d]; gates: [C, G, 3].  Returns (out [C, G, d], union_count)."""
    C = len(lists)
    active = list(lists) if mode == MODE_EXACT else [lists[0]] * C
    ucount = len(union_blocks(lists if mode == MODE_EXACT else [lists[0]]))
    out = np.stack([nsa_row(q_rows[c], k, v, kc, vc, active[c], T, n_cmp, window, gates[c], scale)[0]
                    for c in range(C)])
    return out, ucount


# ---------------------------------------------------------------------------
# O14  prefill: block-sparse attention for every query position of a chunk
#      ([SparDA] eq. (3): the block set B(i) is a function of the query
#      position i, with the local window next to i; the complexity section's
#      eq. (13), (15) and (16) count one selection over the N_b compressed
#      blocks and one top-k attention per query token)
# ---------------------------------------------------------------------------

def prefill_lengths(pos0, nq):
    """Tokens visible to each of the nq queries of a prefill chunk whose
    first query sits at position pos0: query r (position pos0 + r) sees
    tokens 0 .. pos0 + r, i.e. pos0 + r + 1 of them (causal)."""
    return np.arange(int(pos0) + 1, int(pos0) + int(nq) + 1, dtype=np.int64)


def prefill_select_rows(f_rows, kt_stored, pos0, n_init, n_local, k):
    """Block sets of the nq query positions of one (sequence, KV head).

    Query r at position p = pos0 + r chooses exactly as a decode step at
    length p + 1: the blocks present are 0 .. p // 64, the local window is
    the last n_local of them (the block holding p among them), and top-k
    ranks the other blocks by f_r . K~_j.  With n_local >= 1 every block that
    competes in top-k is complete at position p, so the compressed keys of
    the whole sequence are the ones the query could have seen.
    f_rows: float64 [nq, d]; kt_stored: [>= (pos0 + nq - 1) // 64 + 1, d].
    Returns the list of ascending block-id arrays, one per query."""
    if n_local < 1:
        raise ValueError("prefill selection needs n_local >= 1 (the block holding the query is local)")
    out = []
    for r, T in enumerate(prefill_lengths(pos0, len(f_rows))):
        nb = num_blocks(T)
        blocks, _ = select_row(f_rows[r], kt_stored[:nb], n_init, n_local, k)
        out.append(blocks)
    return out


def prefill_rows(q_rows, k, v, lists, pos0, scale):
    """Causal block-sparse attention of every query of a prefill chunk:
    query r (heads q_rows[r], [G, d]) attends to the tokens of its blocks
    that lie at or before its position pos0 + r.  Returns (out [nq, G, d],
    lse [nq, G])."""
    outs, lses = [], []
    for r, T in enumerate(prefill_lengths(pos0, len(q_rows))):
        o, l = decode_row(q_rows[r], k, v, lists[r], T, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------------
# O15  refresh/reuse across layers  ([SSV] core mechanism 2 and its
#      scheduling algorithm: refresh layers route and cache the selected
#      block indices, reuse layers skip routing and take the cache;
#      T_total = R T_refresh + (L - R) T_reuse)
# ---------------------------------------------------------------------------

def refresh_schedule(L, r):
    """Refresh every r-th layer, starting with the first: layer j refreshes
    when j % r == 0 (r = 1: every layer routes)."""
    return [j % int(r) == 0 for j in range(int(L))]


def chain_lists(schedule, route):
    """The block lists each layer of the chain attends with: a refresh layer
    j routes (route(j) returns its lists) and replaces the cache; a reuse
    layer takes the cache as it stands.  The first layer must refresh."""
    cache = None
    out = []
    for j, refresh in enumerate(schedule):
        if refresh:
            cache = route(j)
        elif cache is None:
            raise ValueError("the first layer of a chain must refresh")
        out.append(cache)
    return out


def chain_time(schedule, t_refresh, t_reuse):
    """Verification time of one chain: R refresh layers and L - R reuse layers."""
    R = sum(1 for x in schedule if x)
    return R * t_refresh + (len(schedule) - R) * t_reuse
