"""fp64 reference for O = softmax(scale * Q K^T) V with per-row logsumexp.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and plain on
purpose: it materialises every score row and never uses online softmax.

Sources (three web pages on FlashAttention, cited by title and section):

* [P1] "FlashAttention: IO-aware attention kernel" (inference-learning-path
  course, part 2): §3.1 gives the attention formula and the three
  materialised tensors S, P, O; §3.2 the running-max / normaliser / output
  recurrence and its block-merge form; §4 the CPU proof program with a fully
  worked example whose output it prints.
* [P2] FlashAttention exam notes (omica.com.cn news item 1422242): §一 the
  formula and shapes, §二.3 the merge rule for (m, l, o) between K/V blocks
  (its extracted formulas lost their "=" and "+" signs), §三 the claim that
  the tiled result carries no approximation error.
* [P3] "FlashAttention" walkthrough (kyonqi.github.io, nano-vllm series):
  the three-step standard attention, the "Safe Softmax" section (subtract
  the row maximum), the "online softmax" section and its proof by induction
  that the running sum equals the sum of exponentials taken against the
  running maximum, and "Flash Attention Backward" (what the forward keeps).

Tensor conventions (the plainest reading where the pages are silent):

* q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nkv, D]; o: [B, Hq, Nq, D]; lse: [B, Hq, Nq].
* Query head h reads key/value head floor(h / (Hq / Hkv)) (consecutive
  grouping; the pages only use Hq == Hkv).
* causal: key j is allowed for query i iff j <= i (literal indices, top-left
  alignment when Nq != Nkv).  Key 0 is always allowed, so no row is empty.
* scale is taken as the float32 value the GPU receives, widened exactly to
  float64 (1/sqrt(128) is not exact in float32).
* lse_i = m_i + ln(l_i): natural log over the scaled scores of the allowed
  keys.  [P3] "Flash Attention Backward" keeps the row max m and the row sum
  l for the backward pass; one fp32 number per row carries both.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Key/value head read by query head ``h`` (consecutive grouping)."""
    return h // (Hq // Hkv)


def allowed_keys(i: int, Nkv: int, causal: bool) -> range:
    """Key indices query row ``i`` attends to ([P1] §5 uses is_causal=True)."""
    if causal:
        return range(0, min(i, Nkv - 1) + 1)
    return range(Nkv)


def _sigma(scale: float) -> float:
    return float(np.float32(scale))


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, D]")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nkv, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} must be a multiple of Hkv={Hkv}")
    if min(B, Hq, Nq, Nkv, D) < 1:
        raise ValueError("every dimension must be >= 1")
    return B, Hq, Hkv, Nq, Nkv, D


def _default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, n)


def attention_fp64(q, k, v, scale: float, causal: bool = False,
                   row_chunk: int = 256, threads: int | None = None, rows=None):
    """Exact attention by definition, in float64, materialising full rows.

    For each (b, h) and a chunk of query rows it forms the whole score block
    S = sigma * Q_chunk K^T ([P1] §3.1, [P3] standard attention step 1),
    applies the causal mask, then takes the safe softmax of each row: subtract
    the row maximum, exponentiate, divide by the row sum ([P3] "Safe
    Softmax"; [P1] §3.1, P = softmax(S) row by row), and forms O = P V
    ([P3] step 3).
    lse = m + ln(l).

    Chunking over query rows only bounds memory (a 32768-key row block is
    256 MiB in fp64); each row is still computed whole.  For causal rows the
    keys beyond the chunk's last row are never allowed, so they are not
    formed at all; this drops only terms that are exactly zero.

    ``rows`` (optional) lists absolute query indices to evaluate; the result
    then has len(rows) rows in that order (causal masking still uses the
    absolute index).  Used to check single rows of workloads too large to
    evaluate whole.

    Returns (o, lse) as float64 arrays.  Work units (b, h, chunk) run on a
    thread pool (numpy releases the GIL); BLAS is held to one thread meanwhile.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v)
    sigma = _sigma(scale)
    idx_all = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    if idx_all.size and (idx_all.min() < 0 or idx_all.max() >= Nq):
        raise ValueError("rows out of range")
    R = idx_all.size
    o = np.empty((B, Hq, R, D), dtype=np.float64)
    lse = np.empty((B, Hq, R), dtype=np.float64)

    def work(unit):
        b, h, r0 = unit
        r1 = min(r0 + row_chunk, R)
        idx = idx_all[r0:r1]
        g = kv_head_of(h, Hq, Hkv)
        kend = min(Nkv, int(idx.max()) + 1) if causal else Nkv
        kb = k[b, g, :kend]
        vb = v[b, g, :kend]
        s = sigma * (q[b, h, idx] @ kb.T)                    # [R, kend]
        if causal:
            s = np.where(np.arange(kend)[None, :] <= idx[:, None], s, -np.inf)
        m = s.max(axis=1)                                    # row maximum
        e = np.exp(s - m[:, None])                           # masked -> 0
        l = e.sum(axis=1)                                    # row sum
        p = e / l[:, None]                                   # probabilities
        o[b, h, r0:r1] = p @ vb
        lse[b, h, r0:r1] = m + np.log(l)

    units = [(b, h, r0) for b in range(B) for h in range(Hq)
             for r0 in range(0, R, row_chunk)]
    nthr = threads or _default_threads()
    if nthr <= 1 or len(units) == 1:
        for u in units:
            work(u)
    else:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=nthr) as ex:
            list(ex.map(work, units))
    return o, lse


def attention_fp64_keys(q, k, v, scale: float, causal: bool, keys):
    """Exact attention of every row over its allowed keys that belong to ``keys``.

    The same definition as ``attention_fp64`` with the key set J_i replaced by
    J_i intersected with the given key indices (causal masking keeps absolute
    indices).  A row whose restricted key set is empty has no softmax; it gets
    O = 0 and lse = -inf, the values that contribute nothing to the block
    merge rule ([P2] §二.3).  This is the partial result one split-KV chunk
    stands for.  Plain and unthreaded: meant for small cases.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v)
    sigma = _sigma(scale)
    keys = np.unique(np.asarray(keys, dtype=np.int64).reshape(-1))
    keys = keys[(keys >= 0) & (keys < Nkv)]
    o = np.zeros((B, Hq, Nq, D), dtype=np.float64)
    lse = np.full((B, Hq, Nq), -np.inf, dtype=np.float64)
    if keys.size == 0:
        return o, lse
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            s = sigma * (q[b, h] @ k[b, g, keys].T)           # [Nq, len(keys)]
            if causal:
                s = np.where(keys[None, :] <= np.arange(Nq)[:, None], s, -np.inf)
            for i in range(Nq):
                row = s[i]
                if not np.any(np.isfinite(row)):
                    continue                                   # empty: (0, -inf)
                m = row.max()
                e = np.exp(row - m)
                l = e.sum()
                o[b, h, i] = (e / l) @ v[b, g, keys]
                lse[b, h, i] = m + np.log(l)
    return o, lse


def attention_fp64_key_range(q, k, v, scale: float, causal: bool, lo: int, hi: int):
    """``attention_fp64_keys`` over the contiguous key range [lo, hi)."""
    return attention_fp64_keys(q, k, v, scale, causal, np.arange(max(0, int(lo)), int(hi)))


def attention_bwd_fp64(q, k, v, do, scale: float, causal: bool = False):
    """Gradients of the attention output, by definition, in float64.

    The pages give the backward pass as recomputation: the forward keeps O
    and the row statistics, and the backward forms S and P again from Q, K
    and those statistics instead of storing them ([P3] "Flash Attention
    Backward"; [P2] §二.5, §四.4).  The gradients themselves are the plain
    calculus of O = softmax(S) V with S = sigma Q K^T (masked keys have
    P = 0), for the scalar L = sum(O * dO):

        dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(P * dP)),
        dQ = sigma dS K,   dK = sigma dS^T Q.

    Here P is formed whole from S (safe softmax), not from saved statistics.
    With grouped heads, dK and dV of a key/value head sum the contributions
    of every query head that reads it.  Returns (dq, dk, dv) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have the shape of Q")
    sigma = _sigma(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            s = sigma * (q[b, h] @ k[b, g].T)                  # [Nq, Nkv]
            if causal:
                s = np.where(np.arange(Nkv)[None, :] <= np.arange(Nq)[:, None], s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)               # P
            dv[b, g] += p.T @ do[b, h]                         # dV = P^T dO
            dp = do[b, h] @ v[b, g].T                          # dP = dO V^T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[b, h] = sigma * (ds @ k[b, g])                  # dQ = sigma dS K
            dk[b, g] += sigma * (ds.T @ q[b, h])               # dK = sigma dS^T Q
    return dq, dk, dv


def attention_bwd_fp64_rows(q, k, v, do, scale: float, causal: bool, q_rows, key_rows):
    """Selected rows of dQ (query rows ``q_rows``) and of dK, dV (key rows
    ``key_rows``), by the same definition as ``attention_bwd_fp64``.

    For sequences too long to form every gradient: lse and O come from
    ``attention_fp64`` (exact, row by row), so P[i, j] = exp(s_ij - lse_i) is
    available for any single row or column.  A dQ row needs its own P and dP
    rows; a dK/dV row needs the P and dP columns of its key over every query:

        dQ[i] = sigma sum_j P[i,j] (dP[i,j] - D_i) K[j]
        dV[j] = sum_i P[i,j] dO[i],   dK[j] = sigma sum_i P[i,j] (dP[i,j] - D_i) Q[i]

    with D_i = sum_t dO[i,t] O[i,t] = sum_j P[i,j] dP[i,j].  Key rows sum over
    the query heads of their group.  Returns (dq[:, :, q_rows], dk[:, :, key_rows],
    dv[:, :, key_rows]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v)
    sigma = _sigma(scale)
    qr = np.asarray(q_rows, dtype=np.int64).reshape(-1)
    kr = np.asarray(key_rows, dtype=np.int64).reshape(-1)
    o, lse = attention_fp64(q, k, v, scale, causal)
    dvec = np.sum(do * o, axis=-1)                            # D_i
    dq = np.zeros((B, Hq, qr.size, D))
    dk = np.zeros((B, Hkv, kr.size, D))
    dv = np.zeros((B, Hkv, kr.size, D))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            # query rows: full rows of P and dP
            s = sigma * (q[b, h, qr] @ k[b, g].T)             # [len(qr), Nkv]
            if causal:
                s = np.where(np.arange(Nkv)[None, :] <= qr[:, None], s, -np.inf)
            p = np.exp(s - lse[b, h, qr][:, None])
            dp = do[b, h, qr] @ v[b, g].T
            dq[b, h] = sigma * ((p * (dp - dvec[b, h, qr][:, None])) @ k[b, g])
            # key rows: full columns of P and dP
            s = sigma * (q[b, h] @ k[b, g, kr].T)             # [Nq, len(kr)]
            if causal:
                s = np.where(kr[None, :] <= np.arange(Nq)[:, None], s, -np.inf)
            p = np.exp(s - lse[b, h][:, None])
            dp = do[b, h] @ v[b, g, kr].T
            ds = p * (dp - dvec[b, h][:, None])
            dv[b, g] += p.T @ do[b, h]
            dk[b, g] += sigma * (ds.T @ q[b, h])
    return dq, dk, dv


def probabilities_fp64(q, k, scale: float, causal: bool = False):
    """Full probability tensor P [B, Hq, Nq, Nkv] (masked entries are 0).

    Same definition as ``attention_fp64`` ([P3] standard attention step 2),
    for small shapes only; used by tests that read P back through V.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, k)
    sigma = _sigma(scale)
    P = np.zeros((B, Hq, Nq, Nkv), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            s = sigma * (q[b, h] @ k[b, g].T)
            if causal:
                s = np.where(np.arange(Nkv)[None, :] <= np.arange(Nq)[:, None],
                             s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            P[b, h] = e / e.sum(axis=1, keepdims=True)
    return P


def attention_bruteforce(q, k, v, scale: float, causal: bool = False):
    """Pure-Python element-by-element attention, straight from the softmax definition.

    [P1] §3.1 defines P = softmax(S) row by row, p_ij = e^(s_ij) / sum_k e^(s_ik),
    and O = P V.  Dividing numerator and denominator by e^(s_ij) gives
    p_ij = 1 / sum_k e^(s_ik - s_ij), which is evaluated here for every pair
    (O(N^2) exponentials per row, no running or row maximum, no separate
    normaliser); a term e^(s_ik - s_ij) beyond the float range makes p_ij
    smaller than 1e-300, taken as 0.  Then o_i = sum_j p_ij v_j and, since
    lse_i = ln sum_k e^(s_ik) = s_ij - ln p_ij for any j, lse_i is read off the
    key with the largest score.  Every sum is a ``math.fsum`` over Python
    floats.  Intended for N <= 16; used only to check ``attention_fp64``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v)
    sigma = _sigma(scale)
    o = np.empty((B, Hq, Nq, D), dtype=np.float64)
    lse = np.empty((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            for i in range(Nq):
                qi = [float(x) for x in q[b, h, i]]
                keys = list(allowed_keys(i, Nkv, causal))
                s = [sigma * math.fsum(qi[t] * float(k[b, g, j, t]) for t in range(D))
                     for j in keys]
                p = []
                for sj in s:
                    gaps = [sk - sj for sk in s]
                    p.append(0.0 if max(gaps) > 700.0
                             else 1.0 / math.fsum(math.exp(x) for x in gaps))
                for t in range(D):
                    o[b, h, i, t] = math.fsum(p[n] * float(v[b, g, j, t])
                                              for n, j in enumerate(keys))
                top = max(range(len(keys)), key=lambda n: s[n])
                lse[b, h, i] = s[top] - math.log(p[top])
    return o, lse


def attention_online_blocked(q, k, v, scale: float, causal: bool = False,
                             block: int = 64, on_step=None):
    """Tiled online-softmax attention in float64 (self-test companion only).

    Streams keys in blocks of ``block``.  For each block it takes the block's
    own row maximum m~, exponential sum l~ and unnormalised weighted sum o~,
    then merges with the running (m, l, o) by rescaling both sides to the new
    maximum ([P1] §3.2; [P2] §二.3, read with the lost "=" and "+" restored:
    m_new = max(m_old, m_j), l_new = l_old e^(m_old - m_new) + l_j e^(m_j - m_new),
    o_new likewise with o unnormalised).  A factor whose exponent base is -inf
    is 0 ([P1] §4 sets the correction to 0 while the running max is -inf).
    O = o / l once after the last block; lse = m + ln(l).

    ``on_step(b, h, j1, m, l)`` is called after each block with the running
    row statistics for keys [0, j1), so a test can check the induction
    invariant of [P3] "online softmax": l equals the sum of e^(s - m) over
    the keys seen so far.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v)
    if block < 1:
        raise ValueError("block must be >= 1")
    sigma = _sigma(scale)
    o_out = np.empty((B, Hq, Nq, D), dtype=np.float64)
    lse = np.empty((B, Hq, Nq), dtype=np.float64)
    rows = np.arange(Nq)[:, None]
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            m = np.full(Nq, -np.inf)
            l = np.zeros(Nq)
            acc = np.zeros((Nq, D))
            for j0 in range(0, Nkv, block):
                j1 = min(j0 + block, Nkv)
                s = sigma * (q[b, h] @ k[b, g, j0:j1].T)      # [Nq, blk]
                if causal:
                    s = np.where(np.arange(j0, j1)[None, :] <= rows, s, -np.inf)
                m_t = s.max(axis=1)
                live_t = np.isfinite(m_t)
                e = np.where(live_t[:, None],
                             np.exp(s - np.where(live_t, m_t, 0.0)[:, None]), 0.0)
                l_t = e.sum(axis=1)
                o_t = e @ v[b, g, j0:j1]
                m_new = np.maximum(m, m_t)
                live_new = np.isfinite(m_new)
                base = np.where(live_new, m_new, 0.0)
                a_old = np.where(np.isfinite(m), np.exp(m - base), 0.0)
                a_t = np.where(live_t, np.exp(m_t - base), 0.0)
                l = a_old * l + a_t * l_t
                acc = a_old[:, None] * acc + a_t[:, None] * o_t
                m = m_new
                if on_step is not None:
                    on_step(b, h, j1, m.copy(), l.copy())
            o_out[b, h] = acc / l[:, None]
            lse[b, h] = m + np.log(l)
    return o_out, lse


def attention_fp64_kv_cache(q, k, v, scale: float, causal: bool = False):
    """Exact attention of N_q new queries against a cache of N keys, in float64.

    q: [Hq, N_q, D]; k, v: [Hkv, N, D] (one sequence).  The queries are the
    last N_q positions of the sequence, so with ``causal`` query i sees key j
    iff j <= N - N_q + i (the cache's bottom-right alignment; it equals the
    top-left rule of ``attention_fp64`` when N_q == N).  [P1]'s vLLM reading
    (§4) hands the kernel this kind of cache together with its block tables.
    A row with no allowed key gets O = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, Nq, D = q.shape
    Hkv, N = k.shape[0], k.shape[1]
    sigma = _sigma(scale)
    o = np.zeros((Hq, Nq, D))
    lse = np.full((Hq, Nq), -np.inf)
    if N == 0:
        return o, lse
    allowed = np.ones((Nq, N), dtype=bool)
    if causal:
        allowed = np.arange(N)[None, :] <= (N - Nq) + np.arange(Nq)[:, None]
    live = allowed.any(axis=1)
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        s = np.where(allowed, sigma * (q[h] @ k[g].T), -np.inf)[live]
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        o[h, live] = (e / l[:, None]) @ v[g]
        lse[h, live] = m + np.log(l)
    return o, lse


def gather_paged(cache, block_table_row, n: int):
    """Keys 0..n-1 of one sequence from a paged cache, as [Hkv, n, D].

    cache: [num_blocks, block_size, Hkv, D]; key j lives in block
    block_table_row[j // block_size], slot j % block_size.
    """
    cache = np.asarray(cache)
    bs = cache.shape[1]
    j = np.arange(n)
    rows = cache[np.asarray(block_table_row)[j // bs], j % bs]     # [n, Hkv, D]
    return np.ascontiguousarray(rows.transpose(1, 0, 2))


def attention_fp64_paged(q, k_cache, v_cache, block_table, seqlens, scale: float,
                         causal: bool = False):
    """Exact attention over paged K/V caches, in float64.

    q: [B, Hq, N_q, D]; k_cache, v_cache: [num_blocks, block_size, Hkv, D];
    block_table: [B, max_blocks]; seqlens: [B].  Sequence b is gathered
    through its block-table row and attended with ``attention_fp64_kv_cache``.
    Returns (o [B, Hq, N_q, D], lse [B, Hq, N_q]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Nq, D = q.shape
    o = np.zeros((B, Hq, Nq, D))
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        n = int(seqlens[b])
        k = gather_paged(k_cache, block_table[b], n).astype(np.float64)
        v = gather_paged(v_cache, block_table[b], n).astype(np.float64)
        o[b], lse[b] = attention_fp64_kv_cache(q[b], k, v, scale, causal)
    return o, lse
