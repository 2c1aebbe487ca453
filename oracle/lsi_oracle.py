"""Plain, slow CPU oracle for the sparse-attention decode step.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package's smoke check and
the CPU-baseline leg of the benchmark may import this module.  The product
path (the HIP library and its Python binding) never calls it, and this module
imports nothing from the product path.

Everything is numpy float64 on exactly decoded inputs.  Each function states
the passage it follows:

* "LeanSparse: Shrinking GPU Memory for Sparse-Attention LLM Serving"
  (radioguide.fm episode notes), the episode summary: the indexer keys stay on
  the GPU; decode searches compact indexer keys and fetches a short list of
  original keys to rank exactly; prefill streams each layer's history through
  two alternating GPU buffers.
* "Multi-layer Indexer" abstract (zhuanzhiai.com), first paragraph: in DSA a
  lightning indexer scores the whole cache of every layer and keeps the k=2048
  highest-scoring tokens, which the layer then attends.

The pages print neither the score formula nor any dtype.  The formula used
here, I_s = sum_j w_j * ReLU(q_j . k_s) with k_s = sigma_s * dec(code_s), is
the DSA lightning-indexer definition this library implements; fp8 is OCP
E4M3FN; compact keys are symmetric int4 with a per-token fp32 scale.

Parity status per function
  decode_e4m3fn, decode_bf16, decode_int4     pinned (full code tables)
  index_scores                                 pinned (closed forms, invariants,
                                               hand-constructed cases)
  topk                                         pinned (defining property,
                                               planted recovery, hand cases)
  attention / mla_decode                       pinned (dense library attention,
                                               closed forms)
  two_stage_topk                               pinned (reduction to exact top-k,
                                               recall ordering); its recall on
                                               real data is unpinned (the pages
                                               publish no figure)
  prefill_index_topk                           pinned (reduces to decode on the
                                               visible prefix; causality)
  selection_source, multilayer_decode          pinned (hand tables of the layer
                                               schedule; reductions to
                                               decode_step; identical adjacent
                                               selections make MLI a no-op)
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode_e4m3fn", "decode_bf16", "decode_int4",
    "request_rows", "index_scores", "score_magnitude", "topk", "band",
    "attention", "mla_decode", "decode_step", "two_stage_topk",
    "prefill_index_topk", "selection_source", "multilayer_decode",
]


# ----------------------------------------------------------------------------
# Exact decoders
# ----------------------------------------------------------------------------

def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN byte -> float64.

    Sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.  Exponent
    field 0 is subnormal, value m/8 * 2^-6.  0x7F / 0xFF are NaN; there is no
    infinity, so exponent field 15 with mantissa < 7 is an ordinary number
    (largest 448).
    """
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = np.where(sign == 1, -mag, mag)
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return val


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern (uint16) -> float64: the high half of an IEEE
    binary32 word."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_int4(packed: np.ndarray, dim: int) -> np.ndarray:
    """Packed int4 rows -> int64 values in [-7, 7].

    packed has shape [..., dim/2] uint8; element 2i is the low nibble of byte i,
    element 2i+1 the high nibble.  Nibbles are two's complement; -8 (0x8) is
    not a valid code and decodes to NaN so that a test notices it.
    """
    p = np.asarray(packed).astype(np.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    nib = np.stack([lo, hi], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])
    assert nib.shape[-1] == dim
    val = np.where(nib >= 8, nib - 16, nib).astype(np.float64)
    val = np.where(nib == 8, np.nan, val)
    return val


# ----------------------------------------------------------------------------
# Paged cache access
# ----------------------------------------------------------------------------

def request_rows(pool: np.ndarray, page_table_row: np.ndarray, seq_len: int,
                 page_size: int) -> np.ndarray:
    """Rows of one request, in logical order 0..seq_len-1.

    pool is [num_pages][page_size][...]; logical token s of the request lives
    in physical page page_table_row[s // page_size], slot s % page_size.
    """
    n_pages = -(-seq_len // page_size)
    pages = np.asarray(page_table_row[:n_pages]).astype(np.int64)
    rows = pool[pages].reshape(n_pages * page_size, *pool.shape[2:])
    return rows[:seq_len]


# ----------------------------------------------------------------------------
# Indexer scan
# ----------------------------------------------------------------------------

def index_scores(q: np.ndarray, w: np.ndarray, keys: np.ndarray,
                 scale: np.ndarray | None = None) -> np.ndarray:
    """Lightning-indexer score of every cached token (MLI abstract: the
    indexer scores the whole cache).

    q [H][d] query of each indexer head, w [H] head weights, keys [L][d]
    decoded key codes, scale [L] per-token scale or None.
    Returns I [L] float64 with I_s = sum_j w_j * max(0, q_j . (sigma_s k_s)).
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    if scale is not None:
        k = k * np.asarray(scale, dtype=np.float64)[:, None]
    dots = q @ k.T                       # [H][L]
    return (w[:, None] * np.maximum(dots, 0.0)).sum(axis=0)


def score_magnitude(q: np.ndarray, w: np.ndarray, keys: np.ndarray,
                    scale: np.ndarray | None = None) -> np.ndarray:
    """A_s = sum_j |w_j| * sum_i |q_ji * k_si|: the size of the terms that
    make up I_s, used as the rounding floor when I_s cancels to near zero."""
    q = np.abs(np.asarray(q, dtype=np.float64))
    w = np.abs(np.asarray(w, dtype=np.float64))
    k = np.abs(np.asarray(keys, dtype=np.float64))
    if scale is not None:
        k = k * np.abs(np.asarray(scale, dtype=np.float64))[:, None]
    return (w[:, None] * (q @ k.T)).sum(axis=0)


# ----------------------------------------------------------------------------
# Top-k selection
# ----------------------------------------------------------------------------

def topk(scores: np.ndarray, k: int):
    """The k highest-scoring tokens (MLI abstract: keep the k highest-scoring
    tokens; every token is kept when fewer than k exist).

    Order is (score descending, position ascending); equal scores keep the
    lower position.  -0.0 compares equal to +0.0.  Returns (positions, tau)
    where positions are the first min(k, L) of that order and tau is the k-th
    score (None when L < k).
    """
    s = np.asarray(scores, dtype=np.float64)
    L = s.shape[0]
    order = np.lexsort((np.arange(L), -s))
    n = min(k, L)
    tau = float(s[order[k - 1]]) if L >= k else None
    return order[:n].astype(np.int64), tau


def band(scores: np.ndarray, tau: float | None, rel: float) -> np.ndarray:
    """Positions whose score lies within rel*|tau| of the threshold tau: the
    tokens whose membership in the top-k a rounding difference may flip."""
    s = np.asarray(scores, dtype=np.float64)
    if tau is None:
        return np.zeros(0, dtype=np.int64)
    return np.nonzero(np.abs(s - tau) <= rel * abs(tau))[0]


# ----------------------------------------------------------------------------
# Sparse attention over the selection
# ----------------------------------------------------------------------------

def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """Softmax attention of every query head over the given rows, all heads
    sharing one key/value head (MLI abstract: the layer attends only the
    selected tokens).

    q [H][dk], K [n][dk], V [n][dv].  Two-pass softmax: row max, then
    exp/sum.  Returns (out [H][dv], lse [H]) with lse the natural-log
    sum of exp of the scaled logits.  With n = 0 the output is zero and lse
    is -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    H = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, V.shape[1])), np.full(H, -np.inf)
    logits = sm_scale * (q @ K.T)                       # [H][n]
    m = logits.max(axis=1)
    p = np.exp(logits - m[:, None])
    l = p.sum(axis=1)
    out = (p @ V) / l[:, None]
    lse = m + np.log(l)
    return out, lse


def mla_decode(q: np.ndarray, kv: np.ndarray, dv: int, sm_scale: float):
    """Latent-KV (MLA) decode attention: every query head dots the whole
    latent row (latent + rope part) and reads back the first dv entries of
    the same row as its value."""
    kv = np.asarray(kv, dtype=np.float64)
    return attention(q, kv, kv[:, :dv], sm_scale)


# ----------------------------------------------------------------------------
# Whole decode step and its variants
# ----------------------------------------------------------------------------

def decode_step(q_idx, w, ikeys, iscale, q_attn, kv, v, k, sm_scale, dv):
    """One request of a DSA decode step (MLI abstract): score every cached
    token, keep the top k, attend them.

    ikeys [L][d] decoded indexer keys, iscale [L] or None; kv [L][dk] decoded
    keys of attention (latent rows for MLA); v [L][dv] separate values or
    None (then the first dv entries of kv).  Returns (positions, tau, scores,
    out, lse).
    """
    scores = index_scores(q_idx, w, ikeys, iscale)
    sel, tau = topk(scores, k)
    sel_sorted = np.sort(sel)
    K = np.asarray(kv, dtype=np.float64)[sel_sorted]
    V = (np.asarray(v, dtype=np.float64)[sel_sorted] if v is not None
         else K[:, :dv])
    out, lse = attention(q_attn, K, V, sm_scale)
    return sel, tau, scores, out, lse


def two_stage_topk(q, w, keys4, scale4, keys8, scale8, n_cand: int, k: int):
    """Compact-key search with exact rerank (LeanSparse episode notes: decode
    searches compact indexer keys, then fetches a short list of the original
    keys and ranks them exactly).

    Stage 1 scores every token with the compact keys and keeps the n_cand
    best; stage 2 re-scores only those candidates with the original keys and
    keeps the k best.  Ties in either stage keep the lower position.
    Returns (final positions, candidate positions).
    """
    s4 = index_scores(q, w, keys4, scale4)
    cand, _ = topk(s4, n_cand)
    cand = np.sort(cand)                 # slot order == position order
    s8 = index_scores(q, w, np.asarray(keys8)[cand],
                      np.asarray(scale8)[cand] if scale8 is not None else None)
    fin, _ = topk(s8, k)
    return cand[fin], cand


def prefill_index_topk(q, w, keys, scale, hist_len: int, k: int,
                       rows=None):
    """Indexer of a prefill chunk with a causal mask (LeanSparse episode
    notes: prefill streams each layer's history through the GPU; here only
    what is computed matters, not how it is streamed).

    q [T][H][d], w [T][H]; keys [hist_len+T][d] decoded, scale likewise.
    Query i sits at position hist_len+i and sees positions 0..hist_len+i
    inclusive.  rows optionally limits the work to some query indices.
    Returns {i: (positions, tau, scores)}.
    """
    T = q.shape[0]
    rows = range(T) if rows is None else rows
    res = {}
    for i in rows:
        p = hist_len + int(i)
        vis = p + 1
        s = index_scores(q[i], w[i], keys[:vis],
                         None if scale is None else scale[:vis])
        sel, tau = topk(s, k)
        res[int(i)] = (sel, tau, s)
    return res


def selection_source(layer: int, retention: int, schedule: str) -> int:
    """Which layer's selection layer `layer` attends ("Multi-layer Indexer"
    abstract, first paragraph).

    Indexer layers are the multiples of `retention`: IndexCache keeps an
    indexer in one layer out of every `retention` and the rest reuse the
    latest selection.  "serial": the latest indexer layer at or before
    `layer` (its own selection when it has an indexer).  "mli": a layer
    attends the selection of the previous indexer layer instead of its own,
    i.e. the latest indexer layer strictly before it; layer 0 has none and
    attends its own (a reading: the abstract does not treat the first layer).
    """
    if schedule == "serial" or layer == 0:
        return (layer // retention) * retention
    if schedule == "mli":
        return ((layer - 1) // retention) * retention
    raise ValueError(schedule)


def multilayer_decode(layers, retention: int, schedule: str, k: int,
                      sm_scale: float, dv: int):
    """Several layers of one decode step for one request, each attending the
    selection selection_source() names.

    layers: list of dicts with q_idx, w, ikeys, iscale (indexer inputs, read
    on indexer layers only), q_attn and kv (latent rows, MLA).  Returns
    ({indexer layer: positions}, [(out, lse) per layer]).  Only what is
    computed matters here; which kernels overlap is not visible in it.
    """
    sel = {}
    for l, L in enumerate(layers):
        if l % retention == 0:
            s = index_scores(L["q_idx"], L["w"], L["ikeys"], L["iscale"])
            sel[l], _ = topk(s, k)
    outs = []
    for l, L in enumerate(layers):
        rows = np.sort(sel[selection_source(l, retention, schedule)])
        outs.append(mla_decode(L["q_attn"], np.asarray(L["kv"])[rows], dv, sm_scale))
    return sel, outs


def lse_merge(parts):
    """Combine (out, lse) partials of disjoint row sets into the attention
    over their union (exact identity of the softmax normaliser)."""
    lses = np.stack([p[1] for p in parts])            # [S][H]
    m = lses.max(axis=0)
    wts = np.exp(lses - m)
    tot = wts.sum(axis=0)
    out = sum(wts[i][:, None] * parts[i][0] for i in range(len(parts))) / tot[:, None]
    return out, m + np.log(tot)


def recall(found, exact) -> float:
    """Fraction of the exact selection recovered."""
    e = set(int(x) for x in exact)
    if not e:
        return 1.0
    return len(e & set(int(x) for x in found)) / len(e)

