"""Acceptance rules of GPU results against the CPU oracle, and oracle-side
views of generated inputs.

Scores: |I_gpu - I_ref| <= 1e-3*|I_ref| + 1e-6*A_s, with A_s the magnitude of
        the terms that make up I_s (the floor only matters where I_s cancels
        to near zero; how many elements pass only through it is reported).
Top-k:  the GPU set has min(k, L) distinct valid positions, and every element
        of its symmetric difference with the oracle set scores within 1e-3
        relative of the oracle's k-th score (the band); |band| and |diff| are
        reported.
Attention: per head, max_i |o_gpu - o_ref| / max(|o_ref_i|, rms(o_ref_h)) <= 2e-2.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from lightning_indexer_top_04_amd import synth

SCORE_REL = 1e-3
SCORE_FLOOR = 1e-6
BAND_REL = 1e-3
ATTN_REL = 2e-2


def check_scores(gpu, ref, mag, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    tol = SCORE_REL * np.abs(ref) + SCORE_FLOOR * np.asarray(mag)
    bad = np.nonzero(~(err <= tol))[0]
    assert bad.size == 0, (f"{what}: {bad.size} scores out of tolerance, first {bad[:5]}: "
                           f"gpu {gpu[bad[:5]]} ref {ref[bad[:5]]}")
    floor_only = int(np.sum(err > SCORE_REL * np.abs(ref)))
    rel = err / np.maximum(np.abs(ref), 1e-30)
    return {"n": int(ref.size), "floor_only": floor_only,
            "max_rel": float(np.max(rel[np.abs(ref) > 0])) if np.any(np.abs(ref) > 0) else 0.0}


def check_topk(gpu_idx, gpu_count, ref_scores, k, what=""):
    """gpu_idx: int array [k] (-1 padded); ref_scores: oracle scores [L]."""
    L = len(ref_scores)
    n = min(k, L)
    g = np.asarray(gpu_idx)
    assert int(gpu_count) == n, f"{what}: count {gpu_count} != {n}"
    sel = g[:n]
    assert np.all(sel >= 0) and np.all(sel < L), f"{what}: invalid positions in the selection"
    assert np.all(g[n:] == -1), f"{what}: padding is not -1"
    assert len(np.unique(sel)) == n, f"{what}: duplicate positions"
    ref_sel, tau = O.topk(ref_scores, k)
    diff = np.setxor1d(sel, ref_sel)
    bnd = O.band(ref_scores, tau, BAND_REL)
    outside = np.setdiff1d(diff, bnd)
    assert outside.size == 0, (f"{what}: {outside.size} selection differences outside the "
                               f"band, e.g. {outside[:5]} (tau={tau})")
    return {"band": int(bnd.size), "diff": int(diff.size)}


def exact_topk_f32(scores, k):
    """Positions of the k best of float32 scores (fewer when there are fewer),
    ranked as the kernels rank them: by the order-preserving integer key of
    the float (-0 folded onto +0, NaN below -inf), equal keys by position
    ascending.  Sorted."""
    s = np.ascontiguousarray(np.asarray(scores, dtype=np.float32))
    b = s.view(np.uint32).astype(np.uint64)
    b = np.where(b == 0x80000000, 0, b)
    key = np.where(b >> 31 == 1, b ^ 0xFFFFFFFF, b | 0x80000000)
    key = np.where(np.isnan(s), 0, key)
    order = np.lexsort((np.arange(s.size), -key.astype(np.int64)))
    return np.sort(order[:min(k, s.size)])


def check_attention(out, ref, what=""):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den > 0, den, 1.0)
    rel = np.abs(out - ref) / den
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= ATTN_REL, f"{what}: attention rel err {worst:.3e} > {ATTN_REL}"
    return {"max_rel": worst}


# ----------------------------------------------------------------------------
# Oracle views of generated decode inputs
# ----------------------------------------------------------------------------

class OracleView:
    """Per-request float64 arrays of a DecodeInputs for the oracle (copies
    the needed device data to the host once)."""

    def __init__(self, di: synth.DecodeInputs):
        self.di = di
        self.wl = di.wl
        self.seq = di.seq_lens.cpu().numpy()
        self.pt = di.page_table.cpu().numpy()
        self.f32_keys = di.wl.key_dtype == "f32"
        self.ikeys = synth.u8_bits(di.ikeys) if not self.f32_keys else di.ikeys.cpu().numpy()
        self.iscale = None if di.iscale is None else di.iscale.cpu().numpy()
        self.ikeys4 = None if di.ikeys4 is None else synth.u8_bits(di.ikeys4)
        self.iscale4 = None if di.iscale4 is None else di.iscale4.cpu().numpy()
        if self.f32_keys:
            self.q_idx = di.q_idx.cpu().double().numpy()
        else:
            self.q_idx = O.decode_bf16(synth.bf16_bits(di.q_idx))
        self.w = di.w.cpu().double().numpy()
        self._kv = None

    def L(self, b):
        return int(self.seq[b])

    def keys(self, b):
        L = self.L(b)
        rows = O.request_rows(self.ikeys, self.pt[b], L, synth.PAGE)
        if self.f32_keys:
            return rows.astype(np.float64), None
        sc = O.request_rows(self.iscale, self.pt[b], L, synth.PAGE)
        return O.decode_e4m3fn(rows), sc.astype(np.float64)

    def keys4(self, b):
        L = self.L(b)
        rows = O.request_rows(self.ikeys4, self.pt[b], L, synth.PAGE)
        sc = O.request_rows(self.iscale4, self.pt[b], L, synth.PAGE)
        return O.decode_int4(rows, self.wl.idx_dim), sc.astype(np.float64)

    def scores(self, b):
        K, sc = self.keys(b)
        return (O.index_scores(self.q_idx[b], self.w[b], K, sc),
                O.score_magnitude(self.q_idx[b], self.w[b], K, sc))

    def attn_q(self, b):
        q = self.di.q_attn[b]
        if q.dtype == torch.float32:
            return q.cpu().double().numpy()
        return O.decode_bf16(synth.bf16_bits(q))

    def attn_rows(self, b, positions):
        """Decoded K rows (and V rows for the f32 case) of logical positions."""
        positions = np.asarray(positions, dtype=np.int64)
        pt = self.pt[b]
        phys = pt[positions // synth.PAGE].astype(np.int64) * synth.PAGE + positions % synth.PAGE
        P = self.di.kv.shape[0]
        kvflat = self.di.kv.view(P * synth.PAGE, -1)
        ph = torch.from_numpy(phys).to(kvflat.device)
        rows = kvflat.index_select(0, ph)
        if rows.dtype == torch.float32:
            K = rows.cpu().double().numpy()
            V = self.di.v.view(P * synth.PAGE, -1).index_select(0, ph).cpu().double().numpy()
            return K, V
        return O.decode_bf16(synth.bf16_bits(rows)), None

    def attention(self, b, positions):
        K, V = self.attn_rows(b, positions)
        q = self.attn_q(b)
        if V is None:
            return O.mla_decode(q, K, self.wl.dv, self.wl.sm_scale)
        return O.attention(q, K, V, self.wl.sm_scale)
