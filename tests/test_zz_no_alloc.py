"""lsi_decode_step_noalloc (the fused step with the library's own scratch)
against lsi_decode_step (the same step with a caller workspace), through the
C ABI: two calls in a row on one stream, the second with a smaller input, each
compared element by element with the workspace entry point on the same
inputs.  The selection (count and index set) must be identical; its order is
unspecified (one workgroup per row hands out output slots by LDS atomics), so
the attention, which sums the rows in selection order, is held to the
attention tolerance of the oracle comparisons and the log-sum-exp to fp32
summation-order differences."""
import numpy as np
import pytest
import torch

from acceptance import check_attention
from lightning_indexer_top_04_amd import lsi, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_both(wl, planted=True):
    di = synth.make_decode_inputs(wl, device=DEV, planted=planted)
    seq = di.seq_lens.cpu()
    maxL = int(seq.max())
    ik = lsi.Cache(di.ikeys, di.iscale, "fp8", 128)
    kv = lsi.Cache(di.kv, None, "bf16", 576)
    req = lsi.Requests(di.seq_lens, di.page_table, maxL)
    B, k, H, dv = seq.numel(), wl.k, wl.n_heads, wl.dv
    assert lsi.decode_step_workspace_bytes(B, maxL, k, H, dv) <= lsi.NOALLOC_SCRATCH_BYTES
    ref = lsi.decode_step(ik, kv, None, req, di.q_idx, di.w, di.q_attn, k, wl.sm_scale, dv)
    idx = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    out = torch.full((B, H, dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=DEV)
    got = lsi.decode_step_noalloc(ik, kv, None, req, di.q_idx, di.w, di.q_attn, k, wl.sm_scale, dv,
                                  out=out, lse=lse, idx=idx, count=cnt)
    torch.cuda.synchronize()
    r_idx, r_cnt, r_out, r_lse = ref
    g_idx, g_cnt, g_out, g_lse = got
    assert torch.equal(g_cnt, r_cnt)
    assert torch.equal(torch.sort(g_idx, dim=1).values, torch.sort(r_idx, dim=1).values)
    for b in range(B):
        check_attention(g_out[b].float().cpu().numpy(), r_out[b].float().cpu().numpy(), f"req {b}")
    assert np.allclose(g_lse.cpu().numpy(), r_lse.cpu().numpy(), rtol=1e-5, atol=1e-6)
    return seq.tolist()


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    # first call: one 131072-token request of the DSA-shaped workload
    big = _run_both(synth.DSA_128K)
    print("first call", big)
    # second call, smaller, right after: two ragged requests, un-planted, so
    # the top-k state the first call left in the shared scratch differs
    small = synth.scaled(synth.DSA_128K, seed=21, seq_lens=(20000, 5001), num_req=2)
    print("second call", _run_both(small, planted=False))


def test_noalloc_rejects_a_call_beyond_its_scratch():
    wl = synth.scaled(synth.DSA_128K, seed=5, seq_lens=(3000,) * 64, num_req=64, n_planted=16)
    di = synth.make_decode_inputs(wl, device=DEV)
    ik = lsi.Cache(di.ikeys, di.iscale, "fp8", 128)
    kv = lsi.Cache(di.kv, None, "bf16", 576)
    # a 64-request batch whose max length makes the step's scratch too large
    L = 300000
    pt = torch.zeros(64, (L + 63) // 64, dtype=torch.int32, device=DEV)
    req = lsi.Requests(di.seq_lens, pt, L)
    assert lsi.decode_step_workspace_bytes(64, L, 2048, 128, 512) > lsi.NOALLOC_SCRATCH_BYTES
    out = torch.empty(64, 128, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(64, 128, dtype=torch.float32, device=DEV)
    idx = torch.empty(64, 2048, dtype=torch.int32, device=DEV)
    cnt = torch.empty(64, dtype=torch.int32, device=DEV)
    with pytest.raises(lsi.LsiError) as e:
        lsi.decode_step_noalloc(ik, kv, None, req, di.q_idx, di.w, di.q_attn, 2048, wl.sm_scale,
                                512, out=out, lse=lse, idx=idx, count=cnt)
    assert e.value.status == lsi.ERR_WORKSPACE
