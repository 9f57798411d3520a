"""Seeded synthetic inputs for page-selected sparse decode.

This module only draws inputs: shapes, random values, lengths, page tables,
needle pages and sink logits. It holds none of the method's arithmetic and is
the one module that both the HIP path's callers and the oracle's callers use.

Recipe (the same for every workload, see each Workload for its sizes):

* q [B, Hq, D] fp32 ~ N(0, 1); K and V pools [P_phys, Hkv, page, D] ~ N(0, 1)
  rounded to the KV dtype (bf16 round-to-nearest-even, or kept fp32). Bulk
  values come from ``torch.Generator(device).manual_seed(seed)``, so the same
  seed gives different (but fixed) values on CPU and on the GPU; small draws
  (lengths, needle pages, the pool permutation, sink logits) come from numpy
  PCG64(seed) and are identical on every device.
* Context lengths are fixed, uniform integers in an inclusive range, or
  listed explicitly (edge cases).
* The page table maps logical page p of request b to a physical page. Pools
  are laid out request-major, or (``permuted_pool``) through a seeded random
  permutation of one shared pool. Table entries past a request's last page
  are 0 and must be ignored by any consumer.
* Needles: per (request, KV head) ``needles`` distinct full, non-forced
  pages get keys 0.5*z + 2*qhat, z ~ N(0,1), qhat = sqrt(D) * mean(q of the
  group) / ||mean(q of the group)||, so the group's attention is peaked.
* Slots past the end of a partial last page hold the sentinel 1.0e4 in K and
  V, so a consumer that does not mask them produces visibly wrong results.
* Sink logits (``sink_logits``) ~ N(0, 1), one per query head, fp32.
* ``sink_page_needle``: the first page of every (request, KV head) gets the
  needle recipe too, so that the first (sink) page holds the keys the
  queries align with, as an attention sink does; with a forced sink page this
  gives the top-delta threshold (the pseudo-max over the forced pages) a high
  value.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

SENTINEL = 1.0e4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    budget_pages: int
    context: Optional[int] = None          # fixed context length
    ctx_range: Optional[tuple] = None      # (lo, hi) inclusive, for ragged batches
    lengths: Optional[tuple] = None        # explicit per-request lengths (edge cases)
    page_size: int = 16
    n_sink: int = 0
    n_local: int = 0
    needles: int = 0
    kv_dtype: str = "bf16"                 # "bf16" | "f32"
    sink_logits: bool = False
    permuted_pool: bool = False
    max_pages: Optional[int] = None        # page-table row stride (default: max pages)
    sink_page_needle: bool = False         # page 0 of every (b, g) follows the needle recipe
    seed: int = 0
    n_splits: int = 8                      # split-KV count of the sparse decode
    dense_splits: int = 32                 # split-KV count of the dense decode
    # metadata layout the workload is run with ("physical" | "logical"),
    # like the split counts a measured choice, not part of the inputs
    meta_layout: str = "physical"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five measured workloads. Seeds are 1000 + the workload's ordinal.
TINY = Workload("tiny", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64, context=1024,
                budget_pages=8, kv_dtype="f32", seed=1001, n_splits=1, dense_splits=4)
TINY_DENSE = TINY.replace(name="tiny_dense", budget_pages=64, n_splits=8)
B8_16K = Workload("b8_16k_needles_sink_page", batch=8, num_q_heads=12, num_kv_heads=2,
                  head_dim=128, context=16384, budget_pages=128, n_sink=1, needles=4,
                  seed=1002, n_splits=8, dense_splits=32, meta_layout="logical")
B32_64K = Workload("b32_64k_needles_local4", batch=32, num_q_heads=12, num_kv_heads=2,
                    head_dim=128, context=65536, budget_pages=128, n_local=4, needles=8,
                    seed=1003, n_splits=4, dense_splits=64, meta_layout="logical")
SINK = Workload("b16_32k_learned_sink", batch=16, num_q_heads=64, num_kv_heads=8, head_dim=64,
                context=32768, budget_pages=64, sink_logits=True, seed=1004, n_splits=1,
                dense_splits=32)
RAGGED = Workload("b64_ragged_4k_128k_shared_pool", batch=64, num_q_heads=28, num_kv_heads=4,
                  head_dim=128, ctx_range=(4096, 131072), budget_pages=128, needles=8,
                  permuted_pool=True, max_pages=8192, seed=1005, n_splits=1, dense_splits=64,
                  meta_layout="logical")

# The headline shape with one query head per KV head, a forced sink page whose
# keys follow the needle recipe and the last 4 pages forced: the top-delta
# threshold (pseudo-max over the forced pages' tokens, minus delta) then
# removes the random pages and keeps the needles (used for the top-delta
# measurement where the threshold binds).
TOPDELTA_BINDS = Workload("b32_64k_g1_sink_needle_topdelta", batch=32, num_q_heads=2,
                          num_kv_heads=2, head_dim=128, context=65536, budget_pages=128,
                          n_sink=1, n_local=4, needles=8, sink_page_needle=True, seed=1006,
                          n_splits=4, dense_splits=64, meta_layout="logical")

WORKLOADS = {w.name: w for w in (TINY, TINY_DENSE, B8_16K, B32_64K, SINK, RAGGED,
                                 TOPDELTA_BINDS)}


def _pages(n_tokens: int, page: int) -> int:
    return -(-n_tokens // page)


def _randn_into(dst: torch.Tensor, gen: torch.Generator, chunk_rows: int = 1 << 14):
    """Fill dst (first dim chunked) with N(0,1) rounded to dst's dtype."""
    rows = dst.shape[0]
    for lo in range(0, rows, chunk_rows):
        hi = min(rows, lo + chunk_rows)
        tmp = torch.randn((hi - lo,) + tuple(dst.shape[1:]), generator=gen,
                          device=dst.device, dtype=torch.float32)
        dst[lo:hi].copy_(tmp)
        del tmp


def make_inputs(w: Workload, device="cpu", seed: Optional[int] = None):
    """Draw one batch of inputs for workload w on `device`.

    Returns a dict of tensors on `device` (q, k_pool, v_pool, page_table,
    seq_lens, sink or None) plus host-side facts: seq_lens_host, n_pages_host,
    needle_pages {(b, g): [logical pages]}, scale (fp32 value), and the
    workload itself.
    """
    seed = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    b_, hq, hkv, d, ps = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if w.lengths is not None:
        if len(w.lengths) != b_:
            raise ValueError("lengths must give one length per request")
        lens = np.array(w.lengths, dtype=np.int64)
    elif w.context is not None:
        lens = np.full(b_, w.context, dtype=np.int64)
    else:
        lo, hi = w.ctx_range
        lens = rng.integers(lo, hi + 1, size=b_, dtype=np.int64)
    npages = np.array([_pages(int(x), ps) for x in lens], dtype=np.int64)
    max_pages = int(w.max_pages) if w.max_pages is not None else int(npages.max())
    if npages.max() > max_pages:
        raise ValueError("a context needs more pages than max_pages")
    p_phys = int(npages.sum())

    offsets = np.concatenate([[0], np.cumsum(npages)[:-1]])
    ids = rng.permutation(p_phys) if w.permuted_pool else np.arange(p_phys)
    table = np.zeros((b_, max_pages), dtype=np.int32)
    for b in range(b_):
        table[b, :npages[b]] = ids[offsets[b]:offsets[b] + npages[b]]

    kv_torch = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    q = torch.randn((b_, hq, d), generator=gen, device=dev, dtype=torch.float32)
    k_pool = torch.empty((p_phys, hkv, ps, d), device=dev, dtype=kv_torch)
    v_pool = torch.empty((p_phys, hkv, ps, d), device=dev, dtype=kv_torch)
    _randn_into(k_pool, gen)
    _randn_into(v_pool, gen)

    # Needle pages: full pages outside the forced sink/local ranges.
    needle_pages = {}
    if w.needles:
        grp = hq // hkv
        sites = []
        for b in range(b_):
            n = int(npages[b])
            full = int(lens[b]) // ps
            lo_p, hi_p = w.n_sink, min(full, n - w.n_local)
            pool = np.arange(lo_p, max(lo_p, hi_p))
            for g in range(hkv):
                k = min(w.needles, len(pool))
                chosen = sorted(int(x) for x in rng.choice(pool, size=k, replace=False))
                needle_pages[(b, g)] = chosen
                sites += [(b, g, p) for p in chosen]
                if w.sink_page_needle and n >= 1 and int(lens[b]) >= ps:
                    sites.append((b, g, 0))
        if sites:
            qbar = q.view(b_, hkv, grp, d).mean(dim=2)                      # [B, Hkv, D]
            qhat = math.sqrt(d) * qbar / qbar.norm(dim=-1, keepdim=True)
            z = torch.randn((len(sites), ps, d), generator=gen, device=dev, dtype=torch.float32)
            bs = torch.tensor([s[0] for s in sites], device=dev)
            gs = torch.tensor([s[1] for s in sites], device=dev)
            phys = torch.tensor([int(table[s[0], s[2]]) for s in sites], device=dev)
            vals = 0.5 * z + 2.0 * qhat[bs, gs][:, None, :]
            k_pool[phys, gs] = vals.to(kv_torch)

    # Sentinel in the unused slots of partial last pages.
    for b in range(b_):
        cnt = int(lens[b]) - (int(npages[b]) - 1) * ps
        if cnt < ps:
            phys = int(table[b, npages[b] - 1])
            k_pool[phys, :, cnt:, :] = SENTINEL
            v_pool[phys, :, cnt:, :] = SENTINEL

    sink = None
    if w.sink_logits:
        sink = torch.from_numpy(rng.standard_normal(hq).astype(np.float32)).to(dev)

    return {
        "workload": w,
        "q": q,
        "k_pool": k_pool,
        "v_pool": v_pool,
        "page_table": torch.from_numpy(table).to(dev),
        "seq_lens": torch.from_numpy(lens.astype(np.int32)).to(dev),
        "sink": sink,
        "seq_lens_host": lens,
        "n_pages_host": npages,
        "max_pages": max_pages,
        "num_phys_pages": p_phys,
        "needle_pages": needle_pages,
        "scale": float(np.float32(1.0 / math.sqrt(d))),
    }


def tighten_pages(inp, spread: float = 0.05, center_std: float = 0.6, seed: int = 77):
    """Replace the keys of every physical page by a per-(page, KV head) centre
    drawn N(0, center_std^2) plus N(0, spread^2) noise per token, in place,
    keeping the sentinel of unused slots. The page bounds then sit close to
    the keys, so a threshold on them separates pages (used by the threshold
    selection tests; input drawing only)."""
    k = inp["k_pool"]
    gen = torch.Generator(device=k.device).manual_seed(seed)
    p, h, t, d = k.shape
    centre = torch.randn((p, h, 1, d), generator=gen, device=k.device) * center_std
    noise = torch.randn((p, h, t, d), generator=gen, device=k.device) * spread
    keep = k == SENTINEL
    k.copy_(torch.where(keep, k, (centre + noise).to(k.dtype)))
    return inp


def kv_bits_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy of a K/V/meta tensor as the oracle takes it (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_inputs(inp) -> dict:
    """The oracle's view of an input batch: host numpy arrays."""
    w = inp["workload"]
    return {
        "q": inp["q"].detach().cpu().numpy(),
        "k_pool": kv_bits_numpy(inp["k_pool"]),
        "v_pool": kv_bits_numpy(inp["v_pool"]),
        "kv_dtype": w.kv_dtype,
        "page_table": inp["page_table"].cpu().numpy(),
        "seq_lens": inp["seq_lens"].cpu().numpy(),
        "page_size": w.page_size,
        "scale": inp["scale"],
        "sink": None if inp["sink"] is None else inp["sink"].cpu().numpy(),
    }
