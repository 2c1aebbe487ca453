"""GPU vs oracle at the full workload sizes:

* dsa-decode-L131072: one request of 131072 tokens, planted and un-planted;
  every score, the whole selection and the attention output are checked.
* ragged-decode-B64: 64 requests of 10K..195K tokens in one launch; every
  request's selection and attention against the oracle.
* two-stage-L524288: int4 stage (8192 candidates) then exact fp8 rerank
  (2048); both stages against the oracle, recall against the exact fp8 scan
  reported.
* prefill-T4096-H65536: 4096 queries, 65536 history tokens streamed from pinned
  host memory through two 8192-token buffers, causal; 256 query rows (the
  first and last 32, rows at block and 1024-row boundaries, random rows).
"""
import numpy as np
import pytest
import torch

import oracle as O
from acceptance import OracleView, check_attention, check_scores, check_topk, exact_topk_f32
from lightning_indexer_top_04_amd import lsi, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _objs(di, max_len):
    ik = lsi.Cache(di.ikeys, di.iscale, "fp8", 128)
    kv = lsi.Cache(di.kv, None, "bf16", 576)
    req = lsi.Requests(di.seq_lens, di.page_table, max_len)
    return ik, kv, req


@pytest.mark.parametrize("planted", [True, False])
def test_dsa_128k_decode_step(planted):
    wl = synth.DSA_128K
    di = synth.make_decode_inputs(wl, device=DEV, planted=planted)
    ov = OracleView(di)
    ik, kv, req = _objs(di, 131072)
    scores = lsi.index_scores(ik, req, di.q_idx, di.w)
    idx, cnt, out, lse = lsi.decode_step(ik, kv, None, req, di.q_idx, di.w, di.q_attn, 2048,
                                         wl.sm_scale, 512)
    torch.cuda.synchronize()
    I, A = ov.scores(0)
    st = check_scores(scores[0].cpu().numpy(), I, A, "scan 128K")
    st.update(check_topk(idx[0].cpu().numpy(), cnt[0].item(), I, 2048, "topk 128K"))
    sel = idx[0, :cnt[0]].cpu().numpy()
    ro, rl = ov.attention(0, sel)
    st.update(check_attention(out[0].float().cpu().numpy(), ro, "mla 128K"))
    assert np.allclose(lse[0].cpu().numpy(), rl, rtol=1e-4, atol=1e-4)
    if planted:
        assert O.recall(sel, di.planted[0]) == 1.0
    # distance of the step's output from the oracle's attention over the
    # oracle's own selection (equal sets when the threshold sits in a gap)
    ref_sel, _ = O.topk(I, 2048)
    ro_ref, _ = ov.attention(0, ref_sel)
    og = out[0].float().cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(ro_ref * ro_ref, axis=-1, keepdims=True))
    st["dist_from_oracle_set"] = float(np.max(np.abs(og - ro_ref) / np.maximum(np.abs(ro_ref), rms)))
    st["set_diff"] = int(np.setxor1d(sel, ref_sel).size)
    if st["set_diff"] == 0:
        assert st["dist_from_oracle_set"] <= 2e-2
    print("128K", "planted" if planted else "unplanted", st)


def test_ragged_batch_64_decode_step():
    wl = synth.BATCH_RAGGED
    di = synth.make_decode_inputs(wl, device=DEV)
    seq = di.seq_lens.cpu().numpy()
    ik, kv, req = _objs(di, int(seq.max()))
    idx, cnt, out, lse = lsi.decode_step(ik, kv, None, req, di.q_idx, di.w, di.q_attn, 2048,
                                         wl.sm_scale, 512)
    torch.cuda.synchronize()
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(len(seq)):
        n = min(2048, seq[b])
        assert cnt_h[b] == n
        s = idx_h[b, :n]
        assert np.all((s >= 0) & (s < seq[b])) and len(np.unique(s)) == n
        assert np.all(idx_h[b, n:] == -1)
        assert np.all(np.isfinite(out[b].float().cpu().numpy()))
    ov = OracleView(di)
    for b in range(len(seq)):
        I, _ = ov.scores(b)
        st = check_topk(idx_h[b], cnt_h[b], I, 2048, f"req {b}")
        ro, _ = ov.attention(b, idx_h[b, :cnt_h[b]])
        st.update(check_attention(out[b].float().cpu().numpy(), ro, f"req {b}"))
        assert O.recall(idx_h[b, :cnt_h[b]], di.planted[b]) == 1.0
        print("ragged req", b, "L", seq[b], st)


@pytest.mark.parametrize("planted", [True, False])
def test_two_stage_512k(planted):
    wl = synth.TWO_STAGE_512K
    di = synth.make_decode_inputs(wl, device=DEV, planted=planted, with_int4=True)
    ov = OracleView(di)
    ik8 = lsi.Cache(di.ikeys, di.iscale, "fp8", 128)
    ik4 = lsi.Cache(di.ikeys4, di.iscale4, "int4", 128)
    req = lsi.Requests(di.seq_lens, di.page_table, 524288)
    idx, cnt, cand = lsi.two_stage_topk(ik4, ik8, req, di.q_idx, di.w, 8192, 2048, want_cand=True)
    torch.cuda.synchronize()
    cand_h = cand[0].cpu().numpy()
    K4, s4 = ov.keys4(0)
    I4 = O.index_scores(ov.q_idx[0], ov.w[0], K4, s4)
    st1 = check_topk(cand_h, 8192, I4, 8192, "stage 1")
    # stage 2 given the GPU's candidates: exact fp8 scores of exactly those
    K8, s8 = ov.keys(0)
    I8 = O.index_scores(ov.q_idx[0], ov.w[0], K8, s8)
    fin = idx[0, :cnt[0]].cpu().numpy()
    assert cnt[0].item() == 2048 and set(fin.tolist()) <= set(cand_h.tolist())
    c_sorted = np.sort(cand_h)
    pos_in = np.searchsorted(c_sorted, fin)
    fake_idx = np.full(2048, -1)
    fake_idx[:len(fin)] = pos_in
    st2 = check_topk(fake_idx, len(fin), I8[c_sorted], 2048, "stage 2")
    exact, _ = O.topk(I8, 2048)
    rec = O.recall(fin, exact)
    rec4 = O.recall(O.topk(I4, 2048)[0], exact)
    print("two-stage", "planted" if planted else "unplanted", st1, st2,
          f"recall {rec:.4f} (int4-only {rec4:.4f})")
    assert rec >= rec4 - 1e-9
    if planted:
        assert rec == 1.0
    # the sparse attention over the two-stage selection
    kv = lsi.Cache(di.kv, None, "bf16", 576)
    out, lse = lsi.sparse_mla_decode(kv, None, req, di.q_attn, idx, wl.sm_scale, 512)
    torch.cuda.synchronize()
    ro, rl = ov.attention(0, fin)
    check_attention(out[0].float().cpu().numpy(), ro, "attention over the two-stage selection")
    assert np.allclose(lse[0].cpu().numpy(), rl, rtol=1e-4, atol=1e-4)


def test_prefill_chunk_4096_over_65536():
    wl = synth.PREFILL_CHUNK
    pi = synth.make_prefill_inputs(wl, device=DEV)
    H = pi.hist_len
    hist_k = pi.keys[:H].cpu().pin_memory()
    hist_s = pi.scale[:H].cpu().pin_memory()
    chunk_k = pi.keys[H:].contiguous()
    chunk_s = pi.scale[H:].contiguous()
    copy_stream = torch.cuda.Stream()
    idx, cnt, sc = lsi.prefill_index_topk(hist_k, hist_s, chunk_k, chunk_s, pi.q, pi.w, 2048,
                                          8192, want_scores=True, copy_stream=copy_stream)
    torch.cuda.synchronize()
    cnt_h = cnt.cpu().numpy()
    assert np.all(cnt_h == 2048)
    keys = O.decode_e4m3fn(synth.u8_bits(pi.keys))
    scale = pi.scale.cpu().double().numpy()
    q = O.decode_bf16(synth.bf16_bits(pi.q))
    w = pi.w.cpu().double().numpy()
    rng = np.random.default_rng(12)
    edges = [i for i in range(wl.chunk) if (H + i) % 1024 in (0, 1, 1023)]
    rows = sorted(set(list(range(32)) + list(range(wl.chunk - 32, wl.chunk)) + edges))
    rest = np.setdiff1d(np.arange(wl.chunk), rows)
    rows = sorted(rows + rng.choice(rest, size=256 - len(rows), replace=False).tolist())
    assert len(rows) == 256
    res = O.prefill_index_topk(q, w, keys, scale, H, 2048, rows=rows)
    for i in rows:
        sel_ref, tau, s_ref = res[i]
        vis = H + i + 1
        mag = O.score_magnitude(q[i], w[i], keys[:vis], scale[:vis])
        st = check_scores(sc[i, :vis].cpu().numpy(), s_ref, mag, f"prefill row {i}")
        st.update(check_topk(idx[i].cpu().numpy(), cnt_h[i], s_ref, 2048, f"prefill row {i}"))
        # the running candidate selection is exactly the top-k of its own scores
        own = exact_topk_f32(sc[i, :vis].cpu().numpy(), 2048)
        assert np.array_equal(np.sort(idx[i].cpu().numpy()), own), f"prefill row {i}"
        print("prefill row", i, st)
    # history streamed from the host equals history read from the device
    idx2, cnt2 = lsi.prefill_index_topk(pi.keys[:H], pi.scale[:H], chunk_k, chunk_s, pi.q, pi.w,
                                        2048, 8192)
    torch.cuda.synchronize()
    assert torch.equal(cnt, cnt2)
    a = torch.sort(idx, dim=1).values
    b = torch.sort(idx2, dim=1).values
    assert torch.equal(a, b)


def test_prefill_small_history_and_partial_blocks():
    """hist_len not a multiple of the block, T not a multiple of 4, k above
    the visible count for the first queries."""
    wl = synth.scaled(synth.PREFILL_CHUNK, seq_lens=(1000,), chunk=37, block_tokens=256, seed=9)
    pi = synth.make_prefill_inputs(wl, device=DEV)
    H = pi.hist_len
    k = 1010
    idx, cnt, sc = lsi.prefill_index_topk(pi.keys[:H].cpu().pin_memory(),
                                          pi.scale[:H].cpu().pin_memory(), pi.keys[H:],
                                          pi.scale[H:], pi.q, pi.w, k, 256, want_scores=True)
    torch.cuda.synchronize()
    keys = O.decode_e4m3fn(synth.u8_bits(pi.keys))
    scale = pi.scale.cpu().double().numpy()
    q = O.decode_bf16(synth.bf16_bits(pi.q))
    w = pi.w.cpu().double().numpy()
    res = O.prefill_index_topk(q, w, keys, scale, H, k)
    for i in range(37):
        sel_ref, tau, s_ref = res[i]
        vis = H + i + 1
        mag = O.score_magnitude(q[i], w[i], keys[:vis], scale[:vis])
        check_scores(sc[i, :vis].cpu().numpy(), s_ref, mag, f"row {i}")
        check_topk(idx[i].cpu().numpy(), cnt[i].item(), s_ref, k, f"row {i}")
        n = min(k, vis)
        got = idx[i].cpu().numpy()
        assert np.array_equal(np.sort(got[:n]), exact_topk_f32(sc[i, :vis].cpu().numpy(), k))


def test_prefill_chunk_without_history():
    """hist_len = 0: only the chunk's own keys, causal; every row's selection
    against the oracle and exactly the top-k of the kernel's own scores."""
    wl = synth.scaled(synth.PREFILL_CHUNK, seq_lens=(0,), chunk=100, block_tokens=256, seed=17)
    pi = synth.make_prefill_inputs(wl, device=DEV)
    k = 64
    empty_k = pi.keys[:0]
    empty_s = pi.scale[:0]
    idx, cnt, sc = lsi.prefill_index_topk(empty_k, empty_s, pi.keys, pi.scale, pi.q, pi.w, k, 256,
                                          want_scores=True)
    torch.cuda.synchronize()
    keys = O.decode_e4m3fn(synth.u8_bits(pi.keys))
    scale = pi.scale.cpu().double().numpy()
    q = O.decode_bf16(synth.bf16_bits(pi.q))
    w = pi.w.cpu().double().numpy()
    res = O.prefill_index_topk(q, w, keys, scale, 0, k)
    for i in range(100):
        sel_ref, tau, s_ref = res[i]
        vis = i + 1
        got = idx[i].cpu().numpy()
        check_topk(got, cnt[i].item(), s_ref, k, f"row {i}")
        n = min(k, vis)
        assert np.array_equal(got[:n], exact_topk_f32(sc[i, :vis].cpu().numpy(), k))


@pytest.mark.parametrize("pattern,k", [("equal", 700), ("rising", 700), ("falling", 700),
                                       ("equal", 1), ("rising", 1), ("rising", 37), ("falling", 37)])
def test_prefill_running_selection_under_ties_and_monotone_scores(pattern, k):
    """Every key the same code: a query's scores are one constant times the
    token scale.  equal: all scores tie, the first positions win and after
    the first pruning nothing enters; rising / falling: the scale grows or
    shrinks with the position, so every token (or none) beats the entry
    threshold and the buffers are pruned as often as they can be."""
    wl = synth.scaled(synth.PREFILL_CHUNK, seq_lens=(9000,), chunk=43, block_tokens=1024, seed=5)
    pi = synth.make_prefill_inputs(wl, device=DEV)
    H = pi.hist_len
    n = H + 43
    keys = pi.keys[:1].expand(n, -1).contiguous()
    pos = torch.arange(n, dtype=torch.float64, device=DEV)
    scale = {"equal": torch.full((n,), 0.5, dtype=torch.float64, device=DEV),
             "rising": 0.25 + pos * 1e-4,
             "falling": 2.0 - pos * 1e-4}[pattern].float()
    idx, cnt, sc = lsi.prefill_index_topk(keys[:H], scale[:H].contiguous(), keys[H:],
                                          scale[H:].contiguous(), pi.q, pi.w, k, 1024,
                                          want_scores=True)
    torch.cuda.synchronize()
    for i in range(43):
        vis = H + i + 1
        row = sc[i, :vis].cpu().numpy()
        got = idx[i].cpu().numpy()
        assert cnt[i].item() == k and np.all(got[k:] == -1)
        assert np.all(np.diff(got[:k]) > 0), "positions in ascending order"
        assert np.array_equal(got[:k], exact_topk_f32(row, k)), f"{pattern} row {i}"
        if pattern == "equal":
            assert np.array_equal(got[:k], np.arange(k))
