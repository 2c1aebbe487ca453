"""Seeded synthetic inputs for the decode step, the two-stage search and the
prefill chunk.

This module only draws and encodes inputs: random queries, weights, keys and
latent rows, page tables, and the fp8 / int4 encodings of keys that a serving
system would have stored.  It holds none of the scoring, selection or
attention arithmetic, and it serves both the CPU oracle's tests and the GPU
path.  Everything is drawn with a seeded ``torch.Generator`` on the requested
device (CPU for small cases, the GPU for the large pools), so a given
(config, seed, device type) always yields the same bytes.

Shapes and value laws (none is printed on the pages; these are the plainest
readings of the workloads they describe):

* tiny fp32 case: L=4096, 4 indexer heads of dim 64, q and k ~ N(0,1)/8,
  w ~ U(0,1), 256 planted tokens k_s = mean_j q_j + 0.1 * N(0,1)/8; 8 query
  heads over one K/V head of dim 64, K,V ~ N(0,1).
* DSA-shaped cases: 64 indexer heads of dim 128; keys ~ N(0,1) stored as
  E4M3FN codes with a per-token fp32 scale amax/448; q bf16 ~ N(0,1)/sqrt(128);
  w ~ U(0,1)/8; planted tokens k_s = rho*sqrt(128)*u + sqrt(1-rho^2)*n_s with
  u the unit vector along sum_j w_j q_j, rho = 0.8; MLA q [128][576] bf16 and
  latent rows [576] bf16 ~ N(0,1).
* compact keys: symmetric int4 of the dequantised fp8 key, scale amax/7,
  round-half-even, two nibbles per byte (low nibble = even element).
* pages of 64 tokens; every request's pages come from one global random
  permutation of the physical pool.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

PAGE = 64
FP8_MAX = 448.0


# ----------------------------------------------------------------------------
# Workload descriptions
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    seq_lens: tuple = ()            # explicit lengths, or empty to draw
    num_req: int = 1
    len_range: tuple = (0, 0)       # inclusive range for drawn lengths
    n_idx_heads: int = 64
    idx_dim: int = 128
    key_dtype: str = "fp8"          # "fp8" | "f32"
    k: int = 2048
    n_planted: int = 2048
    # attention
    n_heads: int = 128
    dk: int = 576
    dv: int = 512
    attn_dtype: str = "bf16"        # "bf16" (latent MLA) | "f32" (separate K/V)
    sm_scale: float = 1.0 / math.sqrt(576.0)
    # two-stage search
    n_cand: int = 0
    # prefill
    chunk: int = 0
    block_tokens: int = 0
    extra: dict = field(default_factory=dict)


TINY_F32 = Workload(
    name="tiny-fp32-L4096", seed=0, seq_lens=(4096,), n_idx_heads=4,
    idx_dim=64, key_dtype="f32", k=256, n_planted=256, n_heads=8, dk=64,
    dv=64, attn_dtype="f32", sm_scale=1.0 / 8.0)
DSA_128K = Workload(name="dsa-decode-L131072", seed=1, seq_lens=(131072,))
BATCH_RAGGED = Workload(name="ragged-decode-B64", seed=2, num_req=64,
                        len_range=(10000, 195000))
TWO_STAGE_512K = Workload(name="two-stage-L524288", seed=3,
                          seq_lens=(524288,), n_cand=8192)
PREFILL_CHUNK = Workload(name="prefill-T4096-H65536", seed=4,
                         seq_lens=(65536,), chunk=4096, block_tokens=8192)

WORKLOADS = {w.name: w for w in (TINY_F32, DSA_128K, BATCH_RAGGED,
                                 TWO_STAGE_512K, PREFILL_CHUNK)}


def scaled(wl: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller test shapes)."""
    d = dict(wl.__dict__)
    d.update(kw)
    return Workload(**d)


# ----------------------------------------------------------------------------
# Encoders (how a serving system stores keys; not part of the scored method)
# ----------------------------------------------------------------------------

def encode_fp8_rows(x: torch.Tensor):
    """Per-row E4M3FN encoding: scale = amax/448 (fp32), codes = RNE of
    x/scale clamped to +-448; an all-zero row gets scale 1 and zero codes.
    Returns (codes uint8 [..., d], scale float32 [...])."""
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.float()


def fp8_codes_to_float(codes: torch.Tensor) -> torch.Tensor:
    """Library cast of E4M3FN codes to float32 (used only to derive the
    compact keys from the stored fp8 keys)."""
    return codes.view(torch.float8_e4m3fn).float()


def encode_int4_rows(x: torch.Tensor):
    """Symmetric int4 per row: scale = amax/7 (fp32), n = RNE(x/scale)
    clamped to [-7, 7]; packed two per byte, low nibble = even element.
    Returns (packed uint8 [..., d/2], scale float32 [...])."""
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 7.0, torch.ones_like(amax))
    n = torch.round(x / scale.unsqueeze(-1)).clamp(-7, 7).to(torch.int32)
    nib = n & 0xF
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).to(torch.uint8)
    return packed, scale.float()


def to_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


# ----------------------------------------------------------------------------
# Draws
# ----------------------------------------------------------------------------

def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def draw_seq_lens(wl: Workload, g_cpu: torch.Generator) -> list:
    if wl.seq_lens:
        return list(wl.seq_lens)
    lo, hi = wl.len_range
    return [int(v) for v in torch.randint(lo, hi + 1, (wl.num_req,),
                                          generator=g_cpu)]


def make_page_table(seq_lens, g_cpu: torch.Generator, page: int = PAGE,
                    extra_pages: int = 0):
    """One global random permutation of the physical pool; request r takes
    the next ceil(L_r/page) entries.  Unused table slots are -1."""
    n_pages = [-(-L // page) for L in seq_lens]
    total = sum(n_pages) + extra_pages
    perm = torch.randperm(total, generator=g_cpu).to(torch.int32)
    max_pages = max(n_pages)
    pt = torch.full((len(seq_lens), max_pages), -1, dtype=torch.int32)
    off = 0
    for r, n in enumerate(n_pages):
        pt[r, :n] = perm[off:off + n]
        off += n
    return pt, total


@dataclass
class DecodeInputs:
    wl: Workload
    seq_lens: torch.Tensor          # int32 [B]
    page_table: torch.Tensor        # int32 [B][max_pages]
    num_pages: int
    q_idx: torch.Tensor             # bf16 [B][H_I][d] (f32 for the tiny case)
    w: torch.Tensor                 # f32 [B][H_I]
    ikeys: torch.Tensor             # uint8 [P][page][d] (f32 [P][page][d])
    iscale: torch.Tensor | None     # f32 [P][page]
    ikeys4: torch.Tensor | None     # uint8 [P][page][d/2]
    iscale4: torch.Tensor | None    # f32 [P][page]
    q_attn: torch.Tensor            # bf16 [B][H][dk] (f32 tiny)
    kv: torch.Tensor                # bf16 [P][page][dk] (f32 tiny: K)
    v: torch.Tensor | None          # f32 [P][page][dv] tiny only
    planted: list                   # per request, logical positions


def _planted_positions(L, n, g_cpu):
    n = min(n, L)
    return torch.randperm(L, generator=g_cpu)[:n].sort().values


def make_decode_inputs(wl: Workload, device="cpu", planted: bool = True,
                       with_int4: bool = False,
                       with_attn: bool = True, layer: int = 0) -> DecodeInputs:
    """Draw one decode step's inputs for workload wl.

    Small per-request tensors (q, w, page tables, planted positions) are
    drawn on the CPU and moved; the large pools are drawn on `device`.
    `layer` > 0 draws another layer of the same batch: the same lengths and
    page table (the layers of a model share them), its own queries, weights,
    keys and planted positions.
    """
    g_cpu = _gen(wl.seed, "cpu")
    g_dev = _gen(wl.seed + 1000, device)
    seq = draw_seq_lens(wl, g_cpu)
    B = len(seq)
    pt, P = make_page_table(seq, g_cpu)
    if layer:
        g_cpu = _gen(wl.seed + 7919 * layer, "cpu")
        g_dev = _gen(wl.seed + 1000 + 7919 * layer, device)
    H, d = wl.n_idx_heads, wl.idx_dim

    if wl.key_dtype == "f32":
        q = torch.randn(B, H, d, generator=g_cpu) / math.sqrt(d)
        w = torch.rand(B, H, generator=g_cpu)
    else:
        q = (torch.randn(B, H, d, generator=g_cpu) / math.sqrt(d)).to(torch.bfloat16)
        w = torch.rand(B, H, generator=g_cpu) / 8.0

    # logical keys of every physical slot, drawn on device
    keys = torch.randn(P * PAGE, d, generator=g_dev, device=device)
    if wl.key_dtype == "f32":
        keys = keys / math.sqrt(d)
    planted_pos = []
    if planted and wl.n_planted > 0:
        for r in range(B):
            pos = _planted_positions(seq[r], wl.n_planted, g_cpu)
            planted_pos.append(pos.tolist())
            phys = (pt[r, pos // PAGE].long() * PAGE + pos % PAGE).to(device)
            noise = torch.randn(len(pos), d, generator=g_cpu).to(device)
            if wl.key_dtype == "f32":
                qm = q[r].float().mean(0).to(device)
                keys[phys] = qm + 0.1 * noise / math.sqrt(d)
            else:
                u = (w[r].unsqueeze(1) * q[r].float()).sum(0)
                u = (u / u.norm()).to(device)
                rho = 0.8
                keys[phys] = rho * math.sqrt(d) * u + math.sqrt(1 - rho * rho) * noise
    else:
        planted_pos = [[] for _ in range(B)]

    if wl.key_dtype == "f32":
        ikeys = keys.view(P, PAGE, d).contiguous()
        iscale = None
        ikeys4 = iscale4 = None
    else:
        codes, scale = encode_fp8_rows(keys)
        ikeys = codes.view(P, PAGE, d).contiguous()
        iscale = scale.view(P, PAGE).contiguous()
        ikeys4 = iscale4 = None
        if with_int4:
            deq = fp8_codes_to_float(codes) * scale.unsqueeze(1)
            p4, s4 = encode_int4_rows(deq)
            ikeys4 = p4.view(P, PAGE, d // 2).contiguous()
            iscale4 = s4.view(P, PAGE).contiguous()
            del deq
    del keys

    q_attn = kv = v = None
    if with_attn:
        if wl.attn_dtype == "f32":
            q_attn = torch.randn(B, wl.n_heads, wl.dk, generator=g_cpu)
            kv = torch.randn(P, PAGE, wl.dk, generator=g_dev, device=device)
            v = torch.randn(P, PAGE, wl.dv, generator=g_dev, device=device)
        else:
            q_attn = torch.randn(B, wl.n_heads, wl.dk, generator=g_cpu).to(torch.bfloat16)
            kv = torch.empty(P, PAGE, wl.dk, dtype=torch.bfloat16, device=device)
            # draw in slabs to bound the fp32 temporary
            slab = 4096
            for p0 in range(0, P, slab):
                p1 = min(P, p0 + slab)
                kv[p0:p1] = torch.randn(p1 - p0, PAGE, wl.dk, generator=g_dev,
                                        device=device).to(torch.bfloat16)

    return DecodeInputs(
        wl=wl, seq_lens=torch.tensor(seq, dtype=torch.int32).to(device),
        page_table=pt.to(device), num_pages=P, q_idx=q.to(device),
        w=w.float().to(device), ikeys=ikeys, iscale=iscale, ikeys4=ikeys4,
        iscale4=iscale4,
        q_attn=None if q_attn is None else q_attn.to(device),
        kv=kv, v=v, planted=planted_pos)


@dataclass
class PrefillInputs:
    wl: Workload
    hist_len: int
    T: int
    q: torch.Tensor          # bf16 [T][H][d]
    w: torch.Tensor          # f32 [T][H]
    keys: torch.Tensor       # uint8 [hist_len+T][d]  (history then chunk)
    scale: torch.Tensor      # f32 [hist_len+T]


def make_prefill_inputs(wl: Workload, device="cpu") -> PrefillInputs:
    """Queries of a prefill chunk and the fp8 keys of history + chunk, laid
    out contiguously by position."""
    g_cpu = _gen(wl.seed, "cpu")
    g_dev = _gen(wl.seed + 1000, device)
    hist = wl.seq_lens[0]
    T = wl.chunk
    H, d = wl.n_idx_heads, wl.idx_dim
    q = (torch.randn(T, H, d, generator=g_dev, device=device) / math.sqrt(d)).to(torch.bfloat16)
    w = torch.rand(T, H, generator=g_dev, device=device) / 8.0
    keys = torch.randn(hist + T, d, generator=g_dev, device=device)
    codes, scale = encode_fp8_rows(keys)
    return PrefillInputs(wl=wl, hist_len=hist, T=T, q=q, w=w.float(),
                         keys=codes.contiguous(), scale=scale.contiguous())


# ----------------------------------------------------------------------------
# Views for the oracle (numpy), by request
# ----------------------------------------------------------------------------

def u8_bits(t: torch.Tensor):
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def bf16_bits(t: torch.Tensor):
    """uint16 bit patterns of a bf16 tensor."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
