"""Exact attention, written out in float64 on the CPU (test infrastructure).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Plain numpy; every
array is widened to float64 before any arithmetic, so bf16 inputs are exact.

What is computed (the sources are web pages; each is cited by title and
section):

* Standard attention is softmax(Q K^T) V: two matrix products with an N x N
  score matrix between them, re-reading the whole KV cache (plus the newest
  entry) when one new token is generated.  -- forum comment on SRAM and GEMM
  tiling (item 45450456), the paragraph on KV caching.
* The tiled method is exact: it yields the standard attention result.
  -- "11.4d FlashAttention", comparison table in "How
  FlashAttention Fixes This"; "How Does Flash Attention Reduce Memory Traffic
  During Local Inference?", section "Flash Attention Tiles the Problem Into
  On-Chip Working Sets".
* Softmax normalises each row by the sum over all of its scores.  -- "11.4d
  FlashAttention", "Online Softmax".
* Scaling and masking sit between score and normalisation.  -- "How Does
  Flash Attention Reduce Memory Traffic ...", section "Kernel Fusion Keeps More
  of the Attention Chain in One Execution Path".  Scale multiplies Q K^T before
  the mask; a causal mask lets query i see keys 0..i (square problems only).
* Grouped-query attention: fewer key/value heads than query heads; query head
  h reads key/value head h // (Hq / Hkv).  -- "Optimizing memory requirements
  for inference in large language models", the GQA paragraph.  The head map
  itself is not given on the page; consecutive grouping is the reading taken.

Because the fast method is exact, the reference for it is the plain
definition (score_matrix / attention / attention_rows / decode /
decode_paged / attention_varlen), and its gradients (attention_backward)
are the chain rule through that definition.  The running
softmax (tiled_attention) and the log-sum-exp merge (merge_partials) are
second, independent derivations used only to pin the exactness claim and the
split-KV merge.

Layouts: prefill q [B,Hq,N,d], k/v [B,Hkv,N,d], o [B,Hq,N,d], lse [B,Hq,N];
decode q [B,Hq,d], caches [B,Hkv,maxlen,d], seqlens [B], o [B,Hq,d],
lse [B,Hq].  lse is the natural log of the row's sum of exp(scaled score).
"""

import math

import numpy as np


def _f64(x):
    """Widen an array-like (numpy, or a torch CPU tensor of any dtype) to fp64."""
    if hasattr(x, "detach"):  # torch tensor: go through its own float64 cast
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _kv_head(h, hq, hkv):
    """Key/value head read by query head h (consecutive groups of Hq/Hkv)."""
    if hq % hkv != 0:
        raise ValueError(f"Hq={hq} is not a multiple of Hkv={hkv}")
    return h // (hq // hkv)


def score_matrix(q_bh, k_bh, scale, causal):
    """Materialised scaled score matrix S = scale * q k^T for one head.

    q_bh [Nq, d], k_bh [Nk, d].  When causal (square only) entries with key
    index j > query index i are set to -inf, which removes them from the
    softmax.  Returns an Nq x Nk float64 array -- the N^2-entry intermediate
    that the tiled method never writes out.
    """
    q_bh = _f64(q_bh)
    k_bh = _f64(k_bh)
    s = float(scale) * (q_bh @ k_bh.T)
    if causal:
        nq, nk = s.shape
        if nq != nk:
            raise ValueError("causal mask is defined for square problems")
        s[np.triu(np.ones((nq, nk), dtype=bool), k=1)] = -np.inf
    return s


def _softmax_rows_times_v(s, v_bh):
    """Row softmax of s applied to v: returns (o [Nq,d], lse [Nq])."""
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v_bh) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def attention(q, k, v, causal, scale):
    """softmax(scale * Q K^T + mask) V for every batch, head and row.

    Materialises each head's N x N score matrix.  Memory is N^2 * 8 bytes
    per head, so this is for small N; attention_rows covers large N.
    Returns (o, lse) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    bsz, hq, n, d = q.shape
    hkv = k.shape[1]
    o = np.empty((bsz, hq, n, d))
    lse = np.empty((bsz, hq, n))
    for b in range(bsz):
        for h in range(hq):
            g = _kv_head(h, hq, hkv)
            s = score_matrix(q[b, h], k[b, g], scale, causal)
            o[b, h], lse[b, h] = _softmax_rows_times_v(s, v[b, g])
    return o, lse


def attention_rows(q, k, v, causal, scale, rows, heads=None, rows_per_block=256):
    """The same definition evaluated only at query rows `rows` (and heads).

    Softmax is per row, so the requested rows are independent of the others:
    for a group of up to `rows_per_block` of them the score rows
    S[rows, :] = scale * q[rows] k^T are materialised (against keys
    0 .. the group's last row when causal, all keys otherwise), entries with
    key index j > i are set to -inf under the causal mask, and each row takes
    its max, exp, sum and weighted sum of V -- `attention` restricted to those
    rows.  q/k/v may be torch CPU tensors (converted head by head to keep
    memory bounded).  `heads` is a list of (b, h) pairs; default all.
    Returns (o [len(heads), len(rows), d], lse [len(heads), len(rows)]).
    """
    bsz, hq, n, d = q.shape
    hkv = k.shape[1]
    rows = np.asarray(rows, dtype=np.int64)
    if heads is None:
        heads = [(b, h) for b in range(bsz) for h in range(hq)]
    o = np.empty((len(heads), len(rows), d))
    lse = np.empty((len(heads), len(rows)))
    kv_cache = {}
    for t, (b, h) in enumerate(heads):
        g = _kv_head(h, hq, hkv)
        if (b, g) not in kv_cache:
            kv_cache.clear()
            kv_cache[(b, g)] = (_f64(k[b, g]), _f64(v[b, g]))
        kb, vb = kv_cache[(b, g)]
        qb = _f64(q[b, h][rows])
        for r0 in range(0, len(rows), rows_per_block):
            ri = rows[r0:r0 + rows_per_block]
            nk = int(ri.max()) + 1 if causal else n
            s = float(scale) * (qb[r0:r0 + len(ri)] @ kb[:nk].T)
            if causal:
                s[np.arange(nk)[None, :] > ri[:, None]] = -np.inf
            o[t, r0:r0 + len(ri)], lse[t, r0:r0 + len(ri)] = _softmax_rows_times_v(s, vb[:nk])
    return o, lse


def varlen_visible(i, n_q, n_k, causal, window_left):
    """Keys query row i of a sequence (n_q queries, n_k keys) may see: [lo, hi].

    The queries are the last n_q positions of the sequence, so with
    off = n_k - n_q, causal row i sees keys up to i + off (bottom-right
    alignment: a chunk of new queries sees the cached prefix and itself).
    A left window W >= 0 also drops keys before i + off - W.  The range may
    be empty (hi < lo), e.g. causal rows with i + off < 0.
    """
    off = n_k - n_q
    hi = min(i + off, n_k - 1) if causal else n_k - 1
    lo = max(0, i + off - window_left) if window_left >= 0 else 0
    return lo, hi


def attention_varlen(q, k, v, cu_q, cu_k, causal, scale, window_left=-1, rows=None, heads=None):
    """Packed variable-length attention (chunked prefill, sliding window).

    q [total_q, Hq, d], k/v [total_k, Hkv, d]; sequence b owns query rows
    cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1.  Row i of a
    sequence attends to the keys varlen_visible gives, with the scale,
    mask and softmax of `attention`.  The retained cache a chunk of new
    queries attends to, and windowing as one of the ways a runtime may limit
    it, follow "How Does Flash Attention Reduce Memory Traffic During Local
    Inference?", section "Reduced IO Is Not the Same as Eliminating KV
    Cache"; the masked softmax, its section "Kernel Fusion Keeps More of the
    Attention Chain in One Execution Path".  A row that sees no key gets
    o = 0 and lse = -inf.  `rows` (packed query rows) and `heads` restrict
    the evaluation to those entries (the rest stay 0 / -inf).  Returns
    (o [total_q, Hq, d], lse [Hq, total_q]).
    """
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    total_q, hq, d = qf.shape
    hkv = kf.shape[1]
    cu_q = [int(x) for x in np.asarray(cu_q).reshape(-1)]
    cu_k = [int(x) for x in np.asarray(cu_k).reshape(-1)]
    o = np.zeros((total_q, hq, d))
    lse = np.full((hq, total_q), -np.inf)
    want_rows = None if rows is None else set(int(r) for r in rows)
    for b in range(len(cu_q) - 1):
        q0, n_q = cu_q[b], cu_q[b + 1] - cu_q[b]
        k0, n_k = cu_k[b], cu_k[b + 1] - cu_k[b]
        for h in (range(hq) if heads is None else heads):
            g = _kv_head(h, hq, hkv)
            kb = kf[k0:k0 + n_k, g]
            vb = vf[k0:k0 + n_k, g]
            for i in range(n_q):
                if want_rows is not None and q0 + i not in want_rows:
                    continue
                lo, hi = varlen_visible(i, n_q, n_k, causal, window_left)
                if hi < lo:
                    continue
                s = float(scale) * (kb[lo:hi + 1] @ qf[q0 + i, h])
                m = s.max()
                p = np.exp(s - m)
                l = p.sum()
                o[q0 + i, h] = (p @ vb[lo:hi + 1]) / l
                lse[h, q0 + i] = m + math.log(l)
    return o, lse


def attention_backward(q, k, v, do, causal, scale):
    """Gradients of sum(o * do) with respect to q, k and v for o = attention(q, k, v).

    The probabilities are recomputed from q and k instead of being stored
    ("11.4d FlashAttention", section "Recomputation").  For each row, with
    p = softmax(s) over the visible keys and s = scale * q k^T:
        dv_j += p_j do           (per visible key j)
        dp_j  = do . v_j
        ds_j  = p_j (dp_j - sum_j' p_j' dp_j')
        dq   += scale * ds_j k_j,   dk_j += scale * ds_j q
    sum_j' p_j' dp_j' equals do . o, the row's output dotted with its
    upstream gradient.  Under GQA a key/value head's gradients sum over the
    query heads that share it.  Returns (dq, dk, dv) in float64, shaped like
    q, k, v.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    bsz, hq, n, d = q.shape
    hkv = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(bsz):
        for h in range(hq):
            g = _kv_head(h, hq, hkv)
            s = score_matrix(q[b, h], k[b, g], scale, causal)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            p /= p.sum(axis=1, keepdims=True)
            dv[b, g] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, g].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, h] = float(scale) * (ds @ k[b, g])
            dk[b, g] += float(scale) * (ds.T @ q[b, h])
    return dq, dk, dv


def decode(q, kcache, vcache, seqlens, scale):
    """One new token per sequence against its KV cache.

    Query b attends to cache entries 0 .. seqlens[b]-1 (the newest entry is
    already appended at index seqlens[b]-1).  Entries at or past seqlens[b]
    are never read.  An empty sequence gives o = 0 and lse = -inf.
    q [B,Hq,d]; caches [B,Hkv,maxlen,d]; returns (o [B,Hq,d], lse [B,Hq]).
    """
    qf = _f64(q)
    bsz, hq, d = qf.shape
    hkv = kcache.shape[1]
    seqlens = [int(x) for x in np.asarray(_f64(seqlens)).reshape(-1)]
    o = np.zeros((bsz, hq, d))
    lse = np.full((bsz, hq), -np.inf)
    for b in range(bsz):
        n = seqlens[b]
        if n == 0:
            continue
        for g in range(hkv):
            kb = _f64(kcache[b, g, :n])
            vb = _f64(vcache[b, g, :n])
            for h in range(hq):
                if _kv_head(h, hq, hkv) != g:
                    continue
                s = float(scale) * (kb @ qf[b, h])
                m = s.max()
                p = np.exp(s - m)
                l = p.sum()
                o[b, h] = (p @ vb) / l
                lse[b, h] = m + math.log(l)
    return o, lse


def decode_paged(q, kpages, vpages, block_table, seqlens, scale):
    """Decode against a paged KV cache: the same attention as `decode` over
    the logical cache the block table describes.

    The retained keys and values stay available to later tokens unless the
    runtime evicts, compresses, windows or offloads them ("How Does Flash
    Attention Reduce Memory Traffic During Local Inference?", section
    "Reduced IO Is Not the Same as Eliminating KV Cache"); a paged cache is
    storage such a runtime manages.  Pool layout [num_pages, Hkv, page_size,
    d]; block_table[b, i] is the pool page holding entries
    i*page_size .. (i+1)*page_size - 1 of sequence b.  Only the pages that
    hold entries 0 .. seqlens[b]-1 are read (an id past the pool raises).
    Returns (o [B,Hq,d], lse [B,Hq]).
    """
    kp, vp = _f64(kpages), _f64(vpages)
    table = np.asarray(block_table)
    num_pages, hkv, page, d = kp.shape
    bsz = table.shape[0]
    lens = [int(x) for x in np.asarray(seqlens).reshape(-1)]
    maxlen = max([1] + lens)
    kc = np.zeros((bsz, hkv, maxlen, d))
    vc = np.zeros((bsz, hkv, maxlen, d))
    for b in range(bsz):
        for i in range(-(-lens[b] // page)):  # pages holding entries 0 .. L-1
            pid = int(table[b, i])
            if not 0 <= pid < num_pages:
                raise IndexError(f"block_table[{b}, {i}] = {pid} is outside the pool")
            rows = min(page, lens[b] - i * page)
            kc[b, :, i * page:i * page + rows] = kp[pid, :, :rows]
            vc[b, :, i * page:i * page + rows] = vp[pid, :, :rows]
    return decode(q, kc, vc, lens, scale)


def tiled_attention(q, k, v, causal, scale, block_q, block_k):
    """The running-softmax form: key/value tiles consumed one at a time.

    For each block of `block_q` query rows, key/value tiles of `block_k`
    rows are visited in order.  Per row a running maximum m and running sum
    l of exp(score - m) are kept; when a tile raises the maximum, the sum and
    the partial output are first multiplied by exp(m_old - m_new), then the
    tile's exp(score - m_new) are added to l and their weighted V rows to the
    output.  After the last tile the output is divided by l.  -- "11.4d
    FlashAttention", "Online Softmax"; "How Does Flash Attention Reduce Memory
    Traffic ...", section "Online Softmax Avoids Storing the Full Score
    Matrix".  No score matrix larger than block_q x block_k ever exists.
    Returns (o, lse) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    bsz, hq, n, d = q.shape
    hkv = k.shape[1]
    o = np.empty((bsz, hq, n, d))
    lse = np.empty((bsz, hq, n))
    for b in range(bsz):
        for h in range(hq):
            g = _kv_head(h, hq, hkv)
            for i0 in range(0, n, block_q):
                qi = q[b, h, i0:i0 + block_q]
                rows = np.arange(i0, i0 + qi.shape[0])
                m = np.full(qi.shape[0], -np.inf)
                l = np.zeros(qi.shape[0])
                acc = np.zeros((qi.shape[0], d))
                for j0 in range(0, n, block_k):
                    if causal and j0 > rows[-1]:
                        break  # every key of this tile is after every query
                    kj = k[b, g, j0:j0 + block_k]
                    vj = v[b, g, j0:j0 + block_k]
                    s = float(scale) * (qi @ kj.T)
                    if causal:
                        cols = np.arange(j0, j0 + kj.shape[0])
                        s[cols[None, :] > rows[:, None]] = -np.inf
                    m_new = np.maximum(m, s.max(axis=1))
                    # rows that have seen no visible key yet keep m = -inf;
                    # their correction factor is irrelevant (l = acc = 0)
                    alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
                    p = np.where(np.isfinite(m_new)[:, None],
                                 np.exp(s - m_new[:, None]), 0.0)
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ vj
                    m = m_new
                o[b, h, i0:i0 + block_q] = acc / l[:, None]
                lse[b, h, i0:i0 + block_q] = m + np.log(l)
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Merge results computed over disjoint key subsets into the full result.

    Each part s holds o_s (its own softmax-weighted mean of V over its keys)
    and lse_s (log of its own sum of exp scores).  The full sum of exps is
    sum_s exp(lse_s), so the full output is the exp(lse_s)-weighted average of
    the o_s and the full lse is log sum_s exp(lse_s).  This is the running
    softmax of "Online Softmax" applied to whole key subsets at once; it is
    how split-KV decode partials are combined.  Parts with lse = -inf (no
    keys) carry zero weight.  o_parts [S,...,d], lse_parts [S,...].
    """
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    mx = lse_parts.max(axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lse_parts - safe)  # exp(-inf) = 0 for empty parts
    tot = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (w[..., None] * o_parts).sum(axis=0) / tot[..., None]
        lse = safe + np.log(tot)
    o = np.where(np.isfinite(mx)[..., None], o, 0.0)
    lse = np.where(np.isfinite(mx), lse, -np.inf)
    return o, lse
