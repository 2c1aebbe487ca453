"""GPU (HIP) vs CPU oracle, element by element, at sizes the oracle finishes
in seconds: several tiles and pages, ragged tails, edge cases.  Every call
goes through the C ABI (liblsi.so) via the ctypes binding."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from acceptance import OracleView, check_attention, check_scores, check_topk, exact_topk_f32
from lightning_indexer_top_04_amd import lsi, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def objs(di):
    wl = di.wl
    ik = lsi.Cache(di.ikeys, di.iscale, "f32" if wl.key_dtype == "f32" else "fp8", wl.idx_dim)
    req = lsi.Requests(di.seq_lens, di.page_table, int(di.seq_lens.max().item()))
    kv = v = None
    if di.kv is not None:
        kv = lsi.Cache(di.kv, None, "f32" if wl.attn_dtype == "f32" else "bf16", wl.dk)
        if di.v is not None:
            v = lsi.Cache(di.v, None, "f32", wl.dv)
    return ik, req, kv, v


def small_dsa(seq_lens, seed=11, n_planted=64, k=256, attn=True):
    wl = synth.scaled(synth.DSA_128K, seed=seed, seq_lens=tuple(seq_lens),
                      num_req=len(seq_lens), n_planted=n_planted, k=k)
    return synth.make_decode_inputs(wl, device=DEV, with_attn=attn)


# ----------------------------------------------------------------------------
# Indexer scan
# ----------------------------------------------------------------------------

def test_scan_fp8_every_code_and_subnormals():
    """Keys that walk through every finite E4M3FN code (subnormals included)."""
    di = small_dsa([300], n_planted=0, attn=False)
    P = di.ikeys.shape[0]
    codes = torch.arange(P * 64 * 128, dtype=torch.int64) % 256
    codes = torch.where((codes & 0x7F) == 0x7F, torch.zeros_like(codes), codes)
    di.ikeys.copy_(codes.to(torch.uint8).view(P, 64, 128).to(DEV))
    ov = OracleView(di)
    ik, req, _, _ = objs(di)
    s = lsi.index_scores(ik, req, di.q_idx, di.w)
    torch.cuda.synchronize()
    ref, mag = ov.scores(0)
    check_scores(s[0, :300].cpu().numpy(), ref, mag, "every-code")


def test_scan_fp8_ragged_batch():
    di = small_dsa([5000, 37, 4097, 64, 1])
    ov = OracleView(di)
    ik, req, _, _ = objs(di)
    s = lsi.index_scores(ik, req, di.q_idx, di.w)
    torch.cuda.synchronize()
    for b in range(req.num_req):
        L = ov.L(b)
        ref, mag = ov.scores(b)
        st = check_scores(s[b, :L].cpu().numpy(), ref, mag, f"req {b}")
        print(f"req {b} L={L} {st}")


@pytest.mark.parametrize("lens", [
    [60000, 0, 1, 40000, 777, 65, 12345, 30000],      # ragged, empty and one-token requests
    [50000, 50000, 50000],                            # uniform
    [0, 0, 131072, 0],                                # one request holds every token
])
def test_scan_fp8_balanced_slices(lens):
    """Batches large enough for the one-wave grid of balanced slices sized on
    the device: every score of every request, nothing past a request's end."""
    di = small_dsa(lens, n_planted=16, attn=False)
    ov = OracleView(di)
    ik, req, _, _ = objs(di)
    s = torch.full((len(lens), max(lens) + 64), float("nan"), device=DEV)
    lsi.index_scores(ik, req, di.q_idx, di.w, scores=s)
    torch.cuda.synchronize()
    sc = s.cpu().numpy()
    for b in range(len(lens)):
        L = ov.L(b)
        assert np.isnan(sc[b, L:]).all(), f"req {b}: written past its length"
        if L:
            ref, mag = ov.scores(b)
            check_scores(sc[b, :L], ref, mag, f"req {b}")


@pytest.mark.parametrize("R", [192, 193])
def test_scan_fp8_balanced_slices_at_the_request_limit(R):
    """Many short ragged requests: 192 take the balanced grid (at most a
    quarter of the 768 resident workgroups), 193 the grid of one row per
    request.  Every score of every request either way."""
    rng = np.random.default_rng(R)
    lens = [int(x) for x in rng.integers(1, 1300, size=R)]
    lens[0] = 1300
    di = small_dsa(lens, n_planted=4, attn=False)
    ov = OracleView(di)
    ik, req, _, _ = objs(di)
    s = lsi.index_scores(ik, req, di.q_idx, di.w)
    torch.cuda.synchronize()
    sc = s.cpu().numpy()
    for b in range(R):
        L = ov.L(b)
        ref, mag = ov.scores(b)
        check_scores(sc[b, :L], ref, mag, f"req {b}")


def test_scan_f32_tiny_case():
    di = synth.make_decode_inputs(synth.TINY_F32, device=DEV, with_attn=False)
    ov = OracleView(di)
    ik, req, _, _ = objs(di)
    s = lsi.index_scores(ik, req, di.q_idx, di.w)
    torch.cuda.synchronize()
    ref, mag = ov.scores(0)
    print(check_scores(s[0].cpu().numpy(), ref, mag, "tiny f32"))


def test_scan_is_bitwise_invariant_to_page_placement_and_repeatable():
    di = small_dsa([3000], n_planted=0, attn=False)
    ik, req, _, _ = objs(di)
    s1 = lsi.index_scores(ik, req, di.q_idx, di.w).clone()
    s1b = lsi.index_scores(ik, req, di.q_idx, di.w).clone()
    # move every page to a new physical slot
    P = di.ikeys.shape[0]
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(5))
    inv = torch.empty_like(perm); inv[perm] = torch.arange(P)
    keys2 = torch.empty_like(di.ikeys); keys2[perm.to(DEV)] = di.ikeys
    sc2 = torch.empty_like(di.iscale); sc2[perm.to(DEV)] = di.iscale
    pt2 = di.page_table.clone()
    valid = pt2 >= 0
    pt2[valid] = perm.to(DEV)[pt2[valid].long()].to(torch.int32)
    ik2 = lsi.Cache(keys2, sc2, "fp8", 128)
    req2 = lsi.Requests(di.seq_lens, pt2, req.max_seq_len)
    s2 = lsi.index_scores(ik2, req2, di.q_idx, di.w)
    torch.cuda.synchronize()
    assert torch.equal(s1[:, :3000], s1b[:, :3000])
    assert torch.equal(s1[:, :3000], s2[:, :3000])


def test_scan_repeatable_over_many_launches_into_poisoned_outputs():
    # every launch writes every score, and equal inputs give bitwise equal
    # scores: the key ring in LDS is refilled only after each slot's reads
    # (tiles and scales) are complete; NaN-filled outputs expose any score a
    # launch leaves unwritten or computes from a refilled slot
    di1 = small_dsa([131072], seed=19, attn=False)
    di8 = small_dsa([131072] * 4 + [70000, 50001, 8192, 33], seed=23, attn=False)
    cases = []
    for di in (di1, di8):
        ik, req, _, _ = objs(di)
        B = di.seq_lens.numel()
        ld = 131072
        cases.append((ik, req, di, B, ld))
    refs = []
    for ik, req, di, B, ld in cases:
        s = torch.full((B, ld), float("nan"), device=DEV)
        lsi.index_scores(ik, req, di.q_idx, di.w, scores=s)
        refs.append(s.cpu())
    for it in range(60):
        ik, req, di, B, ld = cases[it % 2]
        s = torch.full((B, ld), float("nan"), device=DEV)
        lsi.index_scores(ik, req, di.q_idx, di.w, scores=s)
        got = s.cpu()
        ref = refs[it % 2]
        for b in range(B):
            L = int(di.seq_lens[b])
            assert not torch.isnan(got[b, :L]).any(), (it, b)
            assert torch.equal(got[b, :L], ref[b, :L]), (it, b)


def test_scan_out_of_range_page_scores_minus_inf():
    di = small_dsa([640], n_planted=0, attn=False)
    pt = di.page_table.clone()
    pt[0, 3] = 10 ** 6          # page 3 points outside the pool
    ik, _, _, _ = objs(di)
    req = lsi.Requests(di.seq_lens, pt, 640)
    s = lsi.index_scores(ik, req, di.q_idx, di.w)
    torch.cuda.synchronize()
    s = s[0, :640].cpu()
    assert torch.all(torch.isneginf(s[192:256]))
    assert torch.all(torch.isfinite(s[:192])) and torch.all(torch.isfinite(s[256:]))


# ----------------------------------------------------------------------------
# Top-k
# ----------------------------------------------------------------------------

def _topk_case(scores_np, k, lens):
    B = len(lens)
    ld = scores_np.shape[1]
    sc = torch.from_numpy(scores_np.astype(np.float32)).to(DEV)
    req = lsi.Requests(torch.tensor(lens, dtype=torch.int32, device=DEV), None, ld)
    idx, cnt = lsi.topk(sc, req, k)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    out = []
    for b in range(B):
        ref = scores_np[b, :lens[b]].astype(np.float32).astype(np.float64)
        out.append(check_topk(idx[b], cnt[b], ref, k, f"row {b}"))
    return idx, cnt, out


# Batches of 16 rows or more, and rows of at most 32768 scores, run one
# workgroup per row; fewer, longer rows run the multi-workgroup kernels.  The
# cases below cover both.

@pytest.mark.parametrize("seed,reps", [(0, 1), (1, 1), (2, 3)])
def test_topk_random_rows_against_full_sort(seed, reps):
    rng = np.random.default_rng(seed)
    lens = [131072, 5000, 2049, 2048, 100, 0, 1, 77777] * reps
    sc = rng.standard_normal((len(lens), max(lens))) * 3
    _, _, st = _topk_case(sc, 2048, lens)
    # fp32 inputs: the oracle sees the same values, so the sets are equal
    assert all(s["diff"] == 0 for s in st), st


@pytest.mark.parametrize("ld,offset", [(50001, 0), (50004, 1), (50004, 0)])
def test_topk_row_alignment_and_ragged_tails(ld, offset):
    """Rows that do not start on 16-byte boundaries (odd leading dimension or
    a pointer one score in) take one score per load; aligned rows take four.
    Lengths end mid-run so that the last loads are partial."""
    rng = np.random.default_rng(17)
    lens = [50001 - offset, 45003, 33333, 40000]
    base = torch.from_numpy(rng.standard_normal((len(lens), ld)).astype(np.float32)).to(DEV)
    sc = base[:, offset:offset + max(lens)]
    req = lsi.Requests(torch.tensor(lens, dtype=torch.int32, device=DEV), None, max(lens))
    idx, cnt = lsi.topk(sc, req, 2048)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    host = sc.cpu().numpy().astype(np.float64)
    for b, L in enumerate(lens):
        st = check_topk(idx[b], cnt[b], host[b, :L], 2048, f"row {b}")
        assert st["diff"] == 0, st


@pytest.mark.parametrize("L", [20000, 70000])
def test_topk_exact_ties_keep_lowest_positions(L):
    rng = np.random.default_rng(3)
    sc = np.round(rng.standard_normal((2, L)) * 2) / 2     # heavy ties
    sc[1] = 1.5                                            # every score equal
    sc[0, 123] = -0.0
    idx, cnt, _ = _topk_case(sc, 1000, [L, L])
    for b in range(2):
        ref, _ = O.topk(sc[b].astype(np.float32).astype(np.float64), 1000)
        assert set(idx[b][:cnt[b]].tolist()) == set(ref.tolist())


def test_topk_crowded_threshold_bins():
    """Rows whose k-th score shares its top 12 key bits with a whole row's
    worth of others: one row inside one binade eighth (the members span many
    batches of the second-digit pass), one whose scores differ only in the
    low 8 bits (the second digit keeps them all, more than fit in LDS), and
    a narrow normal row."""
    rng = np.random.default_rng(29)
    L = 131072
    a = (2.0 + rng.uniform(0.0, 0.2499, L)).astype(np.float32)
    bits = np.full(L, 0x40000000, dtype=np.uint32) + rng.integers(0, 256, L).astype(np.uint32)
    b = bits.view(np.float32)
    c = (1.4 + 0.3 * rng.standard_normal(L)).astype(np.float32)
    sc = np.stack([a, b, c, a[::-1].copy()])
    _, _, st = _topk_case(sc, 2048, [L, L, L, 40000])
    assert all(x["diff"] == 0 for x in st), st
    _, _, st = _topk_case(sc, 20000, [L, L, 50000, 20001])
    assert all(x["diff"] == 0 for x in st), st


@pytest.mark.parametrize("L", [64, 40000])
def test_topk_negative_scores_signed_zero_and_infinities(L):
    sc = np.array([[-3.0, -0.0, 0.0, -np.inf, np.inf, -1e-30, 2.0, -2.0] + [-5.0] * (L - 8)])
    idx, cnt, _ = _topk_case(sc, 4, [L])
    assert sorted(idx[0][:4].tolist()) == [1, 2, 4, 6]


@pytest.mark.parametrize("reps", [1, 6])
def test_topk_small_k_and_large_k(reps):
    rng = np.random.default_rng(9)
    sc = rng.standard_normal((3 * reps, 70000))
    _topk_case(sc, 1, [70000, 10, 0] * reps)
    _topk_case(sc, 65536, [70000, 65536, 65535] * reps)


# ----------------------------------------------------------------------------
# Two-stage compact-key search
# ----------------------------------------------------------------------------

def _two_stage_case(host, lens, n_cand, k, seed):
    wl = synth.scaled(synth.TWO_STAGE_512K, seq_lens=tuple(lens), num_req=len(lens),
                      n_planted=64, seed=seed)
    di = synth.make_decode_inputs(wl, device=DEV, with_int4=True, with_attn=False)
    ik4 = lsi.Cache(di.ikeys4, di.iscale4, "int4", 128)
    if host:   # the originals in pinned host memory, read across the bus
        ik8 = lsi.Cache(di.ikeys.cpu().pin_memory(), di.iscale.cpu().pin_memory(), "fp8", 128)
    else:
        ik8 = lsi.Cache(di.ikeys, di.iscale, "fp8", 128)
    req = lsi.Requests(di.seq_lens, di.page_table, max(lens))
    idx, cnt, cand = lsi.two_stage_topk(ik4, ik8, req, di.q_idx, di.w, n_cand, k, want_cand=True)
    torch.cuda.synchronize()
    return di, idx.cpu().numpy(), cnt.cpu().numpy(), cand.cpu().numpy()


@pytest.mark.parametrize("host", [False, True])
def test_two_stage_ragged_against_oracle(host):
    """Both stages per request against the oracle: the compact scan's
    candidates, then the exact rescoring of exactly those; with the original
    keys on the device or in pinned host memory."""
    lens, n_cand, k = [30000, 9000, 3000], 4096, 512
    di, idx, cnt, cand = _two_stage_case(host, lens, n_cand, k, 13)
    ov = OracleView(di)
    for b, L in enumerate(lens):
        nc = min(n_cand, L)
        K4, s4 = ov.keys4(b)
        I4 = O.index_scores(ov.q_idx[b], ov.w[b], K4, s4)
        check_topk(cand[b], nc, I4, n_cand, f"stage 1 req {b}")
        c_sorted = np.sort(cand[b, :nc])
        K8, s8 = ov.keys(b)
        I8 = O.index_scores(ov.q_idx[b], ov.w[b], K8[c_sorted], s8[c_sorted])
        fin = idx[b, :cnt[b]]
        assert set(fin.tolist()) <= set(c_sorted.tolist())
        pos = np.full(k, -1)
        pos[:len(fin)] = np.searchsorted(c_sorted, fin)
        check_topk(pos, cnt[b], I8, k, f"stage 2 req {b}")


def test_two_stage_long_ragged_rows_against_oracle():
    """Rows longer than 32768 take the multi-workgroup first top-k with
    digits over each row's key range (reduced from the int4 scan's
    per-workgroup slots, here from the balanced multi-request grid); a row
    shorter than n_cand keeps everything.  Stage 1 equals the exact top
    n_cand of the scan's own int4 scores; both stages against the oracle."""
    lens, n_cand, k = [70000, 40000, 5000], 8192, 2048
    di, idx, cnt, cand = _two_stage_case(False, lens, n_cand, k, 23)
    ik4 = lsi.Cache(di.ikeys4, di.iscale4, "int4", 128)
    req = lsi.Requests(di.seq_lens, di.page_table, max(lens))
    s4 = lsi.index_scores(ik4, req, di.q_idx, di.w).cpu().numpy()
    ov = OracleView(di)
    for b, L in enumerate(lens):
        nc = min(n_cand, L)
        assert np.array_equal(np.sort(cand[b, :nc]), exact_topk_f32(s4[b, :L], n_cand)), b
        K4, sc4 = ov.keys4(b)
        I4 = O.index_scores(ov.q_idx[b], ov.w[b], K4, sc4)
        check_topk(cand[b], nc, I4, n_cand, f"stage 1 req {b}")
        c_sorted = np.sort(cand[b, :nc])
        K8, s8 = ov.keys(b)
        I8 = O.index_scores(ov.q_idx[b], ov.w[b], K8[c_sorted], s8[c_sorted])
        fin = idx[b, :cnt[b]]
        assert set(fin.tolist()) <= set(c_sorted.tolist())
        pos = np.full(k, -1)
        pos[:len(fin)] = np.searchsorted(c_sorted, fin)
        check_topk(pos, cnt[b], I8, k, f"stage 2 req {b}")


def test_two_stage_key_range_digits_with_a_tie_across_the_threshold():
    """20000 tokens share one compact key (and scale) whose score ranks near
    the 4000th: the threshold of the 8192 candidates falls inside that tie,
    which the key-range digits cannot split, so positions decide (the lowest
    kept).  Stage 1 must equal the exact top-8192 of the scan's own scores."""
    wl = synth.scaled(synth.TWO_STAGE_512K, seq_lens=(70001,), num_req=1, n_planted=0, seed=29)
    di = synth.make_decode_inputs(wl, device=DEV, with_int4=True, with_attn=False, planted=False)
    ik4 = lsi.Cache(di.ikeys4, di.iscale4, "int4", 128)
    ik8 = lsi.Cache(di.ikeys, di.iscale, "fp8", 128)
    req = lsi.Requests(di.seq_lens, di.page_table, 70001)
    s4 = lsi.index_scores(ik4, req, di.q_idx, di.w)[0, :70001].cpu().numpy()
    src = int(np.argsort(-s4.astype(np.float64), kind="stable")[4000])
    pt = di.page_table[0].cpu().numpy()
    pos = np.arange(10000, 30000)
    pages = torch.from_numpy(pt[pos // synth.PAGE].astype(np.int64)).to(DEV)
    slots = torch.from_numpy(pos % synth.PAGE).to(DEV)
    sp, ss = int(pt[src // synth.PAGE]), src % synth.PAGE
    di.ikeys4[pages, slots] = di.ikeys4[sp, ss].clone()
    di.iscale4[pages, slots] = di.iscale4[sp, ss].clone()
    s4 = lsi.index_scores(ik4, req, di.q_idx, di.w)[0, :70001].cpu().numpy()
    idx, cnt, cand = lsi.two_stage_topk(ik4, ik8, req, di.q_idx, di.w, 8192, 2048, want_cand=True)
    torch.cuda.synchronize()
    got = np.sort(cand[0].cpu().numpy())
    want = exact_topk_f32(s4, 8192)
    assert np.array_equal(got, want)
    tied = np.isin(want, pos)
    assert 0 < tied.sum() < 20000   # the threshold lies inside the tie


@pytest.mark.parametrize("planted,L_max", [(True, 100000), (False, 100000), (False, 20000)])
def test_two_stage_one_request_reuses_its_workspace(planted, L_max):
    """One long request: the compact scan builds the first top-k's histograms
    in the workspace's state words (fixed key digits, the threshold bin then
    holds a few percent of the row) and the exact scan clears them again.
    Three calls on one workspace, the second over a shorter row: each stage
    against the oracle, the state words zero after every call, and the
    repeated call equal to the first."""
    state = int(lsi.lib().lsi_decode_step_state_bytes(1))
    wl = synth.scaled(synth.TWO_STAGE_512K, seq_lens=(L_max,), n_planted=256, seed=23)
    di = synth.make_decode_inputs(wl, device=DEV, with_int4=True, with_attn=False, planted=planted)
    ov = OracleView(di)
    ik4 = lsi.Cache(di.ikeys4, di.iscale4, "int4", 128)
    ik8 = lsi.Cache(di.ikeys, di.iscale, "fp8", 128)
    n_cand, k = 4096, 1024
    ws = lsi.two_stage_workspace(1, L_max, n_cand, k, DEV)
    K4, s4 = ov.keys4(0)
    I4 = O.index_scores(ov.q_idx[0], ov.w[0], K4, s4)
    K8, s8 = ov.keys(0)
    I8 = O.index_scores(ov.q_idx[0], ov.w[0], K8, s8)
    first = None
    for L in (L_max, (L_max * 3) // 5, L_max):
        req = lsi.Requests(di.seq_lens.clamp(max=L), di.page_table, L_max)
        idx, cnt, cand = lsi.two_stage_topk(ik4, ik8, req, di.q_idx, di.w, n_cand, k,
                                            want_cand=True, ws=ws)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws[:state])) == 0, "state words left non-zero"
        cand_h = cand[0].cpu().numpy()
        check_topk(cand_h, n_cand, I4[:L], n_cand, f"stage 1 L={L}")
        c_sorted = np.sort(cand_h)
        fin = idx[0, :cnt[0]].cpu().numpy()
        assert cnt[0].item() == k and set(fin.tolist()) <= set(c_sorted.tolist())
        pos = np.searchsorted(c_sorted, fin)
        check_topk(pos, k, I8[c_sorted], k, f"stage 2 L={L}")
        if first is None:
            first = (np.sort(cand_h), np.sort(fin))
        elif L == L_max:
            assert np.array_equal(first[0], np.sort(cand_h)) and np.array_equal(first[1], np.sort(fin))


def test_two_stage_long_candidate_list_against_oracle():
    """More than 32768 candidates: the second top-k takes the multi-workgroup
    path with the slot map (candidate -> position), including the
    refinement's lookups; both stages against the oracle."""
    lens, n_cand, k = [200000], 40000, 2048
    di, idx, cnt, cand = _two_stage_case(False, lens, n_cand, k, 29)
    ov = OracleView(di)
    K4, s4 = ov.keys4(0)
    I4 = O.index_scores(ov.q_idx[0], ov.w[0], K4, s4)
    check_topk(cand[0], n_cand, I4, n_cand, "stage 1")
    c_sorted = np.sort(cand[0, :n_cand])
    K8, s8 = ov.keys(0)
    I8 = O.index_scores(ov.q_idx[0], ov.w[0], K8[c_sorted], s8[c_sorted])
    fin = idx[0, :cnt[0]]
    assert cnt[0] == k and set(fin.tolist()) <= set(c_sorted.tolist())
    check_topk(np.searchsorted(c_sorted, fin), k, I8, k, "stage 2")


def test_two_stage_host_originals_equal_device_and_pageable_is_rejected():
    lens = [70000, 20000]
    _, i_d, c_d, cd_d = _two_stage_case(False, lens, 8192, 2048, 19)
    _, i_h, c_h, cd_h = _two_stage_case(True, lens, 8192, 2048, 19)
    assert np.array_equal(c_d, c_h)
    assert np.array_equal(np.sort(cd_d, axis=1), np.sort(cd_h, axis=1))
    assert np.array_equal(np.sort(i_d, axis=1), np.sort(i_h, axis=1))
    di = small_dsa([5000], attn=False)
    ik4 = lsi.Cache(torch.zeros(di.ikeys.shape[0], 64, 64, dtype=torch.uint8, device=DEV),
                    torch.ones(di.ikeys.shape[0], 64, device=DEV), "int4", 128)
    pageable = lsi.Cache(di.ikeys.cpu(), di.iscale.cpu(), "fp8", 128)
    req = lsi.Requests(di.seq_lens, di.page_table, 5000)
    with pytest.raises(lsi.LsiError) as e:
        lsi.two_stage_topk(ik4, pageable, req, di.q_idx, di.w, 1024, 256)
    assert e.value.status == lsi.ERR_INVALID_ARG


# ----------------------------------------------------------------------------
# Sparse attention
# ----------------------------------------------------------------------------

# batches of 8 or more requests take the 32-head, double-buffered kernel
@pytest.mark.parametrize("reps", [1, 3])
def test_mla_on_oracle_selection_with_padding_and_splits(reps):
    lens = [6000, 1500, 2048] * reps
    B = len(lens)
    di = small_dsa(lens, k=2048)
    ov = OracleView(di)
    ik, req, kv, _ = objs(di)
    k = 2048
    idx = torch.full((B, k), -1, dtype=torch.int32)
    for b in range(B):
        I, _ = ov.scores(b)
        sel, _ = O.topk(I, k)
        idx[b, :len(sel)] = torch.from_numpy(sel.astype(np.int32))
    idx_d = idx.to(DEV)
    out, lse = lsi.sparse_mla_decode(kv, None, req, di.q_attn, idx_d, di.wl.sm_scale, 512)
    torch.cuda.synchronize()
    for b in range(B):
        sel = idx[b][idx[b] >= 0].numpy()
        ro, rl = ov.attention(b, sel)
        print(b, check_attention(out[b].float().cpu().numpy(), ro, f"mla {b}"))
        assert np.allclose(lse[b].cpu().numpy(), rl, rtol=1e-4, atol=1e-4)


def test_mla_single_row_and_empty_selection():
    di = small_dsa([500])
    ov = OracleView(di)
    _, req, kv, _ = objs(di)
    idx = torch.full((1, 64), -1, dtype=torch.int32)
    idx[0, 17] = 321
    out, lse = lsi.sparse_mla_decode(kv, None, req, di.q_attn, idx.to(DEV), di.wl.sm_scale, 512)
    K, _ = ov.attn_rows(0, [321])
    torch.cuda.synchronize()
    # one selected row: every head outputs that row's value part
    assert np.allclose(out[0].float().cpu().numpy(), np.broadcast_to(K[0, :512], (128, 512)),
                       rtol=1e-2, atol=1e-2)
    idx.fill_(-1)
    out, lse = lsi.sparse_mla_decode(kv, None, req, di.q_attn, idx.to(DEV), di.wl.sm_scale, 512)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("heads,reps", [(48, 1), (64, 3), (96, 3)])
def test_mla_head_counts_and_partial_blocks(heads, reps):
    # 48 heads (three 16-head groups; the 16-head kernel at any batch), 64 and
    # 96 heads over 9 requests (two and three 32-head groups); k = 1000 (a
    # partial 64-row block), -1 padding
    lens = (3000, 900, 2500) * reps
    B = len(lens)
    wl = synth.scaled(synth.DSA_128K, seed=13, seq_lens=lens, num_req=B, n_planted=32, k=1000,
                      n_heads=heads)
    di = synth.make_decode_inputs(wl, device=DEV, with_attn=True)
    ov = OracleView(di)
    _, req, kv, _ = objs(di)
    rng = np.random.default_rng(5)
    k = 1000
    idx = torch.full((B, k), -1, dtype=torch.int32)
    for b, L in enumerate(lens):
        n = min(L, k) - 7 * b
        idx[b, :n] = torch.from_numpy(rng.choice(L, size=n, replace=False).astype(np.int32))
    out, lse = lsi.sparse_mla_decode(kv, None, req, di.q_attn, idx.to(DEV), di.wl.sm_scale, 512)
    torch.cuda.synchronize()
    for b in range(B):
        sel = idx[b][idx[b] >= 0].numpy()
        ro, rl = ov.attention(b, sel)
        print(b, check_attention(out[b].float().cpu().numpy(), ro, f"mla48 {b}"))
        assert np.allclose(lse[b].cpu().numpy(), rl, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("B", [4, 8])
def test_mla_late_dominant_rows_rescale_the_running_softmax(B):
    # 16-head kernel (4 requests): each workgroup takes two 64-row blocks of
    # its slice; the rows in the second half of every 128-entry slice get 6x
    # larger latent rows, so their logits exceed the first block's maximum by
    # far.  32-head kernel (8 requests): slices of 256 rows, four blocks, the
    # same rows scaled.
    lens = (3000,) * B
    di = small_dsa(lens, seed=17, k=2048)
    _, req, kv, _ = objs(di)
    rng = np.random.default_rng(6)
    k = 2048
    idx = np.stack([rng.choice(3000, size=k, replace=False) for _ in lens]).astype(np.int32)
    pt = di.page_table.cpu().numpy()
    kvflat = di.kv.view(-1, di.kv.shape[-1])
    for b in range(len(lens)):
        late = idx[b][(np.arange(k) % 128) >= 96]
        phys = torch.from_numpy(pt[b][late // synth.PAGE].astype(np.int64) * synth.PAGE
                                + late % synth.PAGE).to(DEV)
        kvflat[phys] = (kvflat[phys].float() * 6.0).to(kvflat.dtype)
    ov = OracleView(di)
    out, lse = lsi.sparse_mla_decode(kv, None, req, di.q_attn, torch.from_numpy(idx).to(DEV),
                                     di.wl.sm_scale, 512)
    torch.cuda.synchronize()
    for b in range(len(lens)):
        ro, rl = ov.attention(b, idx[b])
        print(b, check_attention(out[b].float().cpu().numpy(), ro, f"mla rescale {b}"))
        assert np.allclose(lse[b].cpu().numpy(), rl, rtol=1e-4, atol=1e-4)


def test_attention_f32_tiny_case():
    di = synth.make_decode_inputs(synth.TINY_F32, device=DEV)
    ov = OracleView(di)
    _, req, kv, v = objs(di)
    I, _ = ov.scores(0)
    sel, _ = O.topk(I, 256)
    idx = torch.from_numpy(sel.astype(np.int32)).view(1, -1).to(DEV)
    out, lse = lsi.sparse_mla_decode(kv, v, req, di.q_attn, idx, di.wl.sm_scale, 64)
    torch.cuda.synchronize()
    ro, rl = ov.attention(0, sel)
    check_attention(out[0].cpu().numpy(), ro, "f32 attention")
    assert np.allclose(lse[0].cpu().numpy(), rl, rtol=1e-5, atol=1e-5)


# ----------------------------------------------------------------------------
# Fused decode step
# ----------------------------------------------------------------------------

def _check_step(di, k):
    ov = OracleView(di)
    ik, req, kv, v = objs(di)
    idx, cnt, out, lse = lsi.decode_step(ik, kv, v, req, di.q_idx, di.w, di.q_attn, k,
                                         di.wl.sm_scale, di.wl.dv)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    stats = []
    for b in range(req.num_req):
        I, _ = ov.scores(b)
        st = check_topk(idx[b], cnt[b], I, k, f"step req {b}")
        sel = idx[b][:cnt[b]]
        ro, rl = ov.attention(b, sel)           # oracle attention on the GPU's set
        st.update(check_attention(out[b].float().cpu().numpy(), ro, f"step attn {b}"))
        stats.append(st)
    return stats


def test_decode_step_tiny_f32_case():
    di = synth.make_decode_inputs(synth.TINY_F32, device=DEV)
    print(_check_step(di, 256))


@pytest.mark.parametrize("reps", [1, 2])
def test_decode_step_fp8_ragged(reps):
    di = small_dsa([9000, 2047, 2048, 130, 4500] * reps, k=2048)
    print(_check_step(di, 2048))


def test_decode_step_unplanted():
    wl = synth.scaled(synth.DSA_128K, seed=21, seq_lens=(20000,), n_planted=0)
    di = synth.make_decode_inputs(wl, device=DEV, planted=False)
    print(_check_step(di, 2048))


@pytest.mark.parametrize("lens", [(9000, 3000, 700), (70001,)])
def test_decode_step_graph_replays_match_eager(lens):
    """The fused step captured in a HIP graph: every replay (with eager work
    and synchronisations in between) reproduces the eager result.  One long
    request takes the path whose scan builds the top-k histograms in the
    workspace's state words, which every call must leave cleared."""
    di = small_dsa(list(lens), k=2048)
    ik, req, kv, _ = objs(di)
    B, k, H, dv = len(lens), 2048, 128, 512
    idx = torch.empty(B, k, dtype=torch.int32, device=DEV)
    cnt = torch.empty(B, dtype=torch.int32, device=DEV)
    out = torch.empty(B, H, dv, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, H, dtype=torch.float32, device=DEV)
    ws = lsi.decode_step_workspace(B, req.max_seq_len, k, H, dv, DEV)

    def run():
        lsi.decode_step(ik, kv, None, req, di.q_idx, di.w, di.q_attn, k, di.wl.sm_scale, dv,
                        out=out, lse=lse, idx=idx, count=cnt, ws=ws)

    run()
    torch.cuda.synchronize()
    e_idx = torch.sort(idx, dim=1).values.clone()
    e_cnt = cnt.clone()
    e_out = out.float().clone()
    e_lse = lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        out.zero_()
        idx.fill_(-7)
        lse.fill_(123.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cnt, e_cnt), rep
        assert torch.equal(torch.sort(idx, dim=1).values, e_idx), rep
        for b in range(B):
            check_attention(out[b].float().cpu().numpy(), e_out[b].cpu().numpy().astype(np.float64),
                            f"replay {rep} req {b}")
        assert torch.allclose(lse, e_lse, rtol=1e-5, atol=1e-5), rep
    st = lsi.lib().lsi_decode_step_state_bytes(B)
    assert torch.count_nonzero(ws[:st]).item() == 0


# ----------------------------------------------------------------------------
# Fused step with the threshold bin left to the attention kernel (rows longer
# than 32768 positions, few requests): the selection must be exactly the
# top-k of the step's own scores (same float decisions), ties to the lower
# positions, whatever depth of the radix the threshold needs.
# ----------------------------------------------------------------------------

def _exact_topk_of(scores, L, k):
    s = scores[:L].astype(np.float64)
    order = np.lexsort((np.arange(L), -s))
    return np.sort(order[:min(k, L)])


def _set_key(di, b, positions, codes_row, scales):
    pt = di.page_table[b].cpu().numpy()
    pos = np.asarray(positions, dtype=np.int64)
    pages = torch.from_numpy(pt[pos // synth.PAGE].astype(np.int64)).to(DEV)
    slots = torch.from_numpy(pos % synth.PAGE).to(DEV)
    di.ikeys[pages, slots] = codes_row.to(DEV)
    di.iscale[pages, slots] = torch.as_tensor(scales, dtype=torch.float32).to(DEV)


@pytest.mark.parametrize("case", ["unplanted", "ties", "near_ties", "two_requests"])
def test_decode_step_threshold_bin_resolved_by_attention(case):
    lens = (70001,) if case != "two_requests" else (40000, 1500)
    k = 2048
    wl = synth.scaled(synth.DSA_128K, seed=31, seq_lens=lens, num_req=len(lens), n_planted=0, k=k)
    di = synth.make_decode_inputs(wl, device=DEV, planted=False)
    ik, req, kv, _ = objs(di)
    if case in ("ties", "near_ties"):
        s0 = lsi.index_scores(ik, req, di.q_idx, di.w)[0, :lens[0]]
        top = int(torch.argmax(s0).item())
        rng = np.random.default_rng(41)
        pos = rng.choice(lens[0], size=3000, replace=False)
        pt = di.page_table[0].cpu().numpy()
        page, slot = int(pt[top // synth.PAGE]), top % synth.PAGE
        row = di.ikeys[page, slot].clone()
        sc = float(di.iscale[page, slot].item())
        if case == "ties":
            scales = np.full(3000, sc, dtype=np.float32)
        else:
            scales = (np.float32(sc) * (1.0 + np.arange(3000) * 2.0 ** -22)).astype(np.float32)
        _set_key(di, 0, pos, row, scales)
    scores = lsi.index_scores(ik, req, di.q_idx, di.w)
    idx, cnt, out, lse = lsi.decode_step(ik, kv, None, req, di.q_idx, di.w, di.q_attn, k,
                                         di.wl.sm_scale, di.wl.dv)
    torch.cuda.synchronize()
    sc_h, idx_h, cnt_h = scores.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    ov = OracleView(di)
    for b, L in enumerate(lens):
        n = min(k, L)
        assert cnt_h[b] == n
        assert np.all(idx_h[b, n:] == -1)
        got = np.sort(idx_h[b, :n])
        assert np.array_equal(got, _exact_topk_of(sc_h[b], L, k)), f"{case} req {b}"
        I, _ = ov.scores(b)
        st = check_topk(idx_h[b], cnt_h[b], I, k, f"{case} req {b}")
        ro, _ = ov.attention(b, idx_h[b, :n])
        st.update(check_attention(out[b].float().cpu().numpy(), ro, f"{case} attn {b}"))
        print(case, b, st)


def test_calls_on_a_side_stream_match_the_current_stream():
    """Entry points given a stream that is not the current one allocate their
    outputs and scratch on that stream and give the same results."""
    di = small_dsa([9000, 40000], k=2048)
    ik, req, kv, _ = objs(di)
    ref = lsi.decode_step(ik, kv, None, req, di.q_idx, di.w, di.q_attn, 2048, di.wl.sm_scale, 512)
    ref_sc = lsi.index_scores(ik, req, di.q_idx, di.w)
    ref_tk = lsi.topk(ref_sc, req, 2048)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    got = lsi.decode_step(ik, kv, None, req, di.q_idx, di.w, di.q_attn, 2048, di.wl.sm_scale, 512,
                          stream=s)
    sc = lsi.index_scores(ik, req, di.q_idx, di.w, stream=s)
    tk = lsi.topk(sc, req, 2048, stream=s)
    s.synchronize()
    for b, n in enumerate((9000, 40000)):   # positions past a row's length are not written
        assert torch.equal(sc[b, :n], ref_sc[b, :n])
    assert torch.equal(got[1], ref[1]) and torch.equal(tk[1], ref_tk[1])
    assert torch.equal(torch.sort(got[0], 1).values, torch.sort(ref[0], 1).values)
    assert torch.equal(torch.sort(tk[0], 1).values, torch.sort(ref_tk[0], 1).values)
    for b in range(2):
        check_attention(got[2][b].float().cpu().numpy(), ref[2][b].float().cpu().numpy().astype(np.float64),
                        f"side stream {b}")
