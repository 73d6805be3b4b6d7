"""Seeded synthetic decode batches for block top-k sparse decode attention.

This module draws inputs only: random tensors, lengths and page tables.  It holds
none of the method's arithmetic (no means, no scores, no selection, no softmax),
so the CPU oracle and the HIP library can both be fed from it without sharing
any computation.

Every tensor is drawn on the CPU from one ``torch.Generator`` seeded with
``1000 * config + variant`` in a fixed order (lengths, page permutation,
per-block key offsets, heavy-block mask and directions, key noise, values,
queries, then filler for unused slots), in float32, then cast to the cache dtype
with round-to-nearest-even.  Both sides therefore read identical bytes.

Value model (workload descriptions of the five decode shapes):
  K_t = z_t + o_block + [heavy] * 2.0 * u_block,  z ~ N(0,1)^D, o ~ N(0, 0.5^2)^D,
  u a unit vector (normalised Gaussian); V, Q ~ N(0,1).
The per-block offset belongs to the physical page, so a page shared by several
sequences (a common prompt prefix) has one offset.  Slots past a sequence's last
token, and pages no sequence references, hold large filler values (|x| ~ 100)
so that a kernel reading them gives visibly wrong results.

Layouts: q [B,Hq,D]; k_cache [pages,Hkv,P,D]; v_cache [pages,Hkv,D,P];
block_table [B,max_blocks] int32 (entries past a sequence's blocks point at a
filler page, never at an invalid id); seq_lens [B] int32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

PAGE = 16
FILLER_SCALE = 100.0


@dataclass
class Batch:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    max_blocks: int
    top_k: int
    dtype: torch.dtype
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    notes: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def n_blocks(self) -> torch.Tensor:
        return (self.seq_lens + self.page_size - 1) // self.page_size

    def to(self, device) -> "Batch":
        kw = dict(self.__dict__)
        for key in ("q", "k_cache", "v_cache", "block_table", "seq_lens"):
            kw[key] = getattr(self, key).to(device)
        return Batch(**kw)


def make_batch(*, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
               seq_lens: Sequence[int] | torch.Tensor | None = None,
               len_range: Optional[tuple[int, int]] = None,
               top_k: int, dtype: torch.dtype = torch.bfloat16, seed: int = 0,
               table: str = "shuffled", shared_prefix: int = 0, heavy_frac: float = 0.0,
               offset_std: float = 0.5, page_size: int = PAGE, spare_pages: int = 2,
               max_blocks: Optional[int] = None, name: str = "custom") -> Batch:
    """Draw one decode batch.

    table: "identity" (sequence b owns pages b*max_blocks + j), "shuffled"
    (a random permutation of all used pages) or "shared" (the first
    shared_prefix tokens' pages are the same physical pages for every sequence,
    private pages shuffled).  seq_lens count the newest token.
    """
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    g = torch.Generator().manual_seed(int(seed))
    P = page_size
    # 1. lengths
    if seq_lens is not None:
        lens = torch.as_tensor(list(seq_lens) if not torch.is_tensor(seq_lens) else seq_lens,
                               dtype=torch.int64).reshape(batch)
    else:
        lo, hi = len_range
        lens = torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64)
    if int(lens.min()) < 1:
        raise ValueError("every sequence holds at least its newest token")
    nblk = (lens + P - 1) // P
    if max_blocks is None:
        max_blocks = int(nblk.max()) + 1
    if int(nblk.max()) > max_blocks:
        raise ValueError("max_blocks too small")

    # 2. page assignment
    bt = torch.empty((batch, max_blocks), dtype=torch.int64)
    if table == "identity":
        used = batch * max_blocks
        for b in range(batch):
            bt[b] = torch.arange(b * max_blocks, (b + 1) * max_blocks)
        num_pages = used + spare_pages
        filler_page = used  # spare page
        for b in range(batch):
            bt[b, int(nblk[b]):] = filler_page
        perm_used = None
    else:
        n_shared = (shared_prefix // P) if table == "shared" else 0
        if table == "shared" and shared_prefix % P:
            raise ValueError("shared prefix must be a whole number of pages")
        if table not in ("shuffled", "shared"):
            raise ValueError(f"unknown table kind {table}")
        private = int((nblk - n_shared).clamp(min=0).sum())
        used = n_shared + private
        num_pages = used + spare_pages
        perm = torch.randperm(num_pages, generator=g)
        shared_ids = perm[:n_shared]
        priv_ids = perm[n_shared:used]
        filler_page = int(perm[used]) if spare_pages > 0 else int(perm[0])
        cur = 0
        for b in range(batch):
            nb = int(nblk[b])
            if n_shared:
                if nb < n_shared:
                    raise ValueError("sequence shorter than the shared prefix")
                bt[b, :n_shared] = shared_ids
            cnt = nb - n_shared
            bt[b, n_shared:nb] = priv_ids[cur:cur + cnt]
            cur += cnt
            bt[b, nb:] = filler_page
        perm_used = perm[:used]

    hkv, D = num_kv_heads, head_dim
    # 3. per-block key offsets, one per (physical page, KV head)
    offset = torch.randn((num_pages, hkv, D), generator=g) * offset_std
    # 4. heavy blocks: +2.0 along a random unit direction
    heavy = torch.rand((num_pages, hkv), generator=g) < heavy_frac
    direc = torch.randn((num_pages, hkv, D), generator=g)
    direc = direc / direc.norm(dim=-1, keepdim=True)
    offset = offset + heavy.unsqueeze(-1).to(torch.float32) * 2.0 * direc
    # 5. key noise, 6. values, 7. queries
    k = torch.randn((num_pages, hkv, P, D), generator=g)
    k += offset.unsqueeze(2)
    v = torch.randn((num_pages, hkv, D, P), generator=g)
    q = torch.randn((batch, num_q_heads, D), generator=g)

    # 8. filler for slots no sequence uses: pages not referenced, and the tail of
    #    each sequence's last page
    valid = torch.zeros((num_pages, P), dtype=torch.bool)
    for b in range(batch):
        nb, L = int(nblk[b]), int(lens[b])
        pages = bt[b, :nb]
        valid[pages[:-1]] = True
        last_valid = L - (nb - 1) * P
        valid[pages[-1], :last_valid] = True
    invalid = ~valid
    if bool(invalid.any()):
        n_inv = int(invalid.sum())
        fk = torch.randn((n_inv, hkv, D), generator=g) * FILLER_SCALE
        fv = torch.randn((n_inv, hkv, D), generator=g) * FILLER_SCALE
        pi, ti = invalid.nonzero(as_tuple=True)
        k[pi, :, ti, :] = fk
        v[pi, :, :, ti] = fv

    batch_obj = Batch(name=name, seed=int(seed), batch=batch, num_q_heads=num_q_heads,
                      num_kv_heads=hkv, head_dim=D, page_size=P, num_pages=num_pages,
                      max_blocks=max_blocks, top_k=int(top_k), dtype=dtype,
                      q=q.to(dtype), k_cache=k.to(dtype), v_cache=v.to(dtype),
                      block_table=bt.to(torch.int32), seq_lens=lens.to(torch.int32),
                      notes={"table": table, "shared_prefix": shared_prefix,
                             "heavy_frac": heavy_frac, "filler_page": filler_page})
    return batch_obj


def make_tie_batch(*, seq_lens: Sequence[int], num_q_heads: int = 8, num_kv_heads: int = 2,
                   head_dim: int = 128, top_k: int = 32, seed: int = 0,
                   name: str = "ties") -> Batch:
    """A batch whose block scores tie exactly, in runs.

    Every token of a (page, KV head) tile holds one of four class vectors
    alpha_c * u_h (alpha = 2, 1, 1/2, -1, exact in bf16; u_h a bf16 direction per
    KV head) and every query head of group h is u_h, so a block's centroid is
    its class vector exactly and blocks of one class score exactly alike, with
    the classes far apart.  Per (sequence, KV head) a random number in
    [0, 2 * top_k] of blocks takes the top class and about half of the rest the
    second, so the k-th largest score is usually shared by many blocks, and
    sometimes the top class is kept whole.  Tables, lengths and values as in
    make_batch (shuffled pages).
    """
    bt = make_batch(batch=len(seq_lens), num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, seq_lens=seq_lens, top_k=top_k, seed=seed, name=name)
    g = torch.Generator().manual_seed(int(seed) + 7919)
    hkv, D, P = num_kv_heads, head_dim, bt.page_size
    u = torch.randn((hkv, D), generator=g).to(torch.bfloat16).to(torch.float32)
    alphas = torch.tensor([2.0, 1.0, 0.5, -1.0])
    cls = torch.randint(2, 4, (bt.num_pages, hkv), generator=g)  # the lower classes
    second = torch.rand((bt.num_pages, hkv), generator=g) < 0.5
    cls[second] = 1
    nblk = (bt.seq_lens.to(torch.int64) + P - 1) // P
    for b in range(bt.batch):
        nb = int(nblk[b])
        pages = bt.block_table[b, :nb].to(torch.int64)
        for h in range(hkv):
            n_top = int(torch.randint(0, 2 * top_k + 1, (1,), generator=g))
            pick = torch.randperm(nb, generator=g)[:min(n_top, nb)]
            cls[pages[pick], h] = 0
    vec = alphas[cls].unsqueeze(-1) * u.unsqueeze(0)  # [pages, hkv, D], exact in bf16
    k = vec.unsqueeze(2).expand(bt.num_pages, hkv, P, D).contiguous()
    r = num_q_heads // num_kv_heads
    q = u.repeat_interleave(r, dim=0).unsqueeze(0).expand(bt.batch, num_q_heads, D).contiguous()
    bt.k_cache = k.to(bt.dtype)
    bt.q = q.to(bt.dtype)
    bt.notes["ties"] = "four key classes"
    return bt


# The five decode workloads.  seed = 1000 * config + variant.
CONFIGS = {
    1: dict(name="tiny-fp32", batch=1, num_q_heads=2, num_kv_heads=1, head_dim=64,
            seq_lens=[1024], top_k=8, dtype=torch.float32, table="identity"),
    2: dict(name="qwen3-0.6b", batch=64, num_q_heads=16, num_kv_heads=8, head_dim=128,
            seq_lens=[8192] * 64, top_k=16, dtype=torch.bfloat16, table="identity",
            heavy_frac=0.05),
    3: dict(name="qwen3-8b", batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
            len_range=(4096, 32768), top_k=32, dtype=torch.bfloat16, table="shuffled"),
    4: dict(name="qwen3-30b-a3b", batch=16, num_q_heads=32, num_kv_heads=4, head_dim=128,
            seq_lens=[2048 + 30720] * 16, top_k=64, dtype=torch.bfloat16, table="shared",
            shared_prefix=2048),
    5: dict(name="qwen3-32b", batch=8, num_q_heads=64, num_kv_heads=8, head_dim=128,
            seq_lens=[32768] * 8, top_k=64, dtype=torch.bfloat16, table="shuffled"),
}
SWEEP_LENS = (8192, 16384, 32768, 65536)


def make_config(config: int, variant: int = 0, *, context: Optional[int] = None,
                table: Optional[str] = None, top_k: Optional[int] = None,
                heavy_frac: Optional[float] = None, batch: Optional[int] = None) -> Batch:
    """One of the five workloads, with optional overrides.

    config 5 takes ``context`` from its sweep (default 32768).  ``batch``
    truncates the batch (for quick checks); lengths are drawn for the full batch
    first so the leading sequences are the same as in the full workload.
    """
    spec = dict(CONFIGS[config])
    name = spec.pop("name")
    if context is not None:
        spec["seq_lens"] = [context] * spec["batch"]
        spec.pop("len_range", None)
    if table is not None:
        spec["table"] = table
    if top_k is not None:
        spec["top_k"] = top_k
    if heavy_frac is not None:
        spec["heavy_frac"] = heavy_frac
    if batch is not None and batch != spec["batch"]:
        if "len_range" in spec:
            g = torch.Generator().manual_seed(1000 * config + variant)
            lo, hi = spec.pop("len_range")
            lens = torch.randint(lo, hi + 1, (spec["batch"],), generator=g, dtype=torch.int64)
            spec["seq_lens"] = lens[:batch].tolist()
        else:
            spec["seq_lens"] = spec["seq_lens"][:batch]
        spec["batch"] = batch
    return make_batch(seed=1000 * config + variant, name=name, **spec)


def make_device_batch(*, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      context: int, top_k: int, seed: int, device, dtype=torch.bfloat16,
                      offset_std: float = 0.5, spare_pages: int = 2, chunk_pages: int = 1 << 16,
                      name: str = "device") -> Batch:
    """A batch of equal-length sequences drawn directly in device memory, for shapes
    whose caches do not fit in host memory (the one-GPU share of a large serving
    batch).  Same value model and layouts as ``make_batch`` with the shuffled table
    (no heavy blocks), drawn from a device ``torch.Generator`` seeded with ``seed``
    in page chunks (so the values differ from ``make_batch``'s for the same seed):
    per-page key offsets, key noise, values, then queries, then filler for the
    spare pages and the unused slots of each sequence's last page.  A checker reads
    the same bytes by copying the pages it needs to the host (``extract``)."""
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    P, hkv, D = PAGE, num_kv_heads, head_dim
    g = torch.Generator(device=device).manual_seed(int(seed))
    nb = (context + P - 1) // P
    used = batch * nb
    num_pages = used + spare_pages
    perm = torch.randperm(num_pages, generator=g, device=device)
    max_blocks = nb + 1
    bt = torch.empty((batch, max_blocks), dtype=torch.int64, device=device)
    bt[:, :nb] = perm[:used].view(batch, nb)
    filler_page = perm[used:used + 1] if spare_pages > 0 else perm[:1]
    bt[:, nb:] = filler_page
    k = torch.empty((num_pages, hkv, P, D), dtype=dtype, device=device)
    v = torch.empty((num_pages, hkv, D, P), dtype=dtype, device=device)
    for c0 in range(0, num_pages, chunk_pages):
        c1 = min(num_pages, c0 + chunk_pages)
        off = torch.randn((c1 - c0, hkv, 1, D), generator=g, device=device) * offset_std
        kc = torch.randn((c1 - c0, hkv, P, D), generator=g, device=device)
        kc += off
        k[c0:c1] = kc.to(dtype)
        v[c0:c1] = torch.randn((c1 - c0, hkv, D, P), generator=g, device=device).to(dtype)
        del off, kc
    q = torch.randn((batch, num_q_heads, D), generator=g, device=device).to(dtype)
    spare = perm[used:]
    if spare.numel():
        k[spare] = (torch.randn((spare.numel(), hkv, P, D), generator=g, device=device)
                    * FILLER_SCALE).to(dtype)
        v[spare] = (torch.randn((spare.numel(), hkv, D, P), generator=g, device=device)
                    * FILLER_SCALE).to(dtype)
    last_valid = context - (nb - 1) * P
    if last_valid < P:
        last = bt[:, nb - 1]
        n_inv = P - last_valid
        k[last, :, last_valid:, :] = (torch.randn((batch, hkv, n_inv, D), generator=g,
                                                  device=device) * FILLER_SCALE).to(dtype)
        v[last, :, :, last_valid:] = (torch.randn((batch, hkv, D, n_inv), generator=g,
                                                  device=device) * FILLER_SCALE).to(dtype)
    lens = torch.full((batch,), context, dtype=torch.int32, device=device)
    return Batch(name=name, seed=int(seed), batch=batch, num_q_heads=num_q_heads,
                 num_kv_heads=hkv, head_dim=D, page_size=P, num_pages=num_pages,
                 max_blocks=max_blocks, top_k=int(top_k), dtype=dtype, q=q, k_cache=k,
                 v_cache=v, block_table=bt.to(torch.int32), seq_lens=lens,
                 notes={"table": "shuffled", "device": str(device),
                        "filler_page": int(filler_page[0])})


def extract(bt: Batch, seqs: Sequence[int]) -> tuple[Batch, torch.Tensor]:
    """The sub-batch of sequences ``seqs`` of ``bt`` (any device) on the host, with
    their pages renumbered 0 .. n-1 in table order plus one filler page, and the
    original page id of each new page.  Pure indexing and copies."""
    sel = torch.as_tensor(list(seqs), dtype=torch.int64, device=bt.block_table.device)
    lens = bt.seq_lens[sel].to(torch.int64)
    nbs = (lens + bt.page_size - 1) // bt.page_size
    table = bt.block_table[sel].to(torch.int64)
    pages = torch.cat([table[i, :int(nbs[i])] for i in range(len(seqs))])
    filler = int(bt.notes.get("filler_page", int(table[0, -1])))
    pages = torch.cat([pages, torch.tensor([filler], device=pages.device)])
    n = pages.numel()
    new_bt = torch.full((len(seqs), bt.max_blocks), n - 1, dtype=torch.int32)
    cur = 0
    for i in range(len(seqs)):
        m = int(nbs[i])
        new_bt[i, :m] = torch.arange(cur, cur + m, dtype=torch.int32)
        cur += m
    sub = Batch(name=bt.name + "-extract", seed=bt.seed, batch=len(seqs),
                num_q_heads=bt.num_q_heads, num_kv_heads=bt.num_kv_heads, head_dim=bt.head_dim,
                page_size=bt.page_size, num_pages=n, max_blocks=bt.max_blocks, top_k=bt.top_k,
                dtype=bt.dtype, q=bt.q[sel].cpu(), k_cache=bt.k_cache[pages].cpu(),
                v_cache=bt.v_cache[pages].cpu(), block_table=new_bt, seq_lens=lens.to(torch.int32).cpu(),
                notes=dict(bt.notes, extracted=list(seqs)))
    return sub, pages.cpu()


def make_new_tokens(bt: Batch, seed: int, scale: float = 1.0) -> tuple[torch.Tensor, torch.Tensor]:
    """A fresh key and value per (sequence, KV head), [B, Hkv, D] in the batch's dtype:
    the token a decode step appends at position seq_lens - 1.  Keys carry the same
    per-page offset model as the cache (an offset drawn here, N(0, 0.5^2)), values
    are N(0, 1); ``scale`` multiplies both."""
    g = torch.Generator().manual_seed(int(seed))
    shape = (bt.batch, bt.num_kv_heads, bt.head_dim)
    k = torch.randn(shape, generator=g) + 0.5 * torch.randn(shape, generator=g)
    v = torch.randn(shape, generator=g)
    return (scale * k).to(bt.dtype), (scale * v).to(bt.dtype)


def write_tokens(bt: Batch, k_new: torch.Tensor, v_new: torch.Tensor) -> Batch:
    """A copy of ``bt`` (CPU) whose caches hold k_new / v_new at each sequence's
    position seq_lens - 1 (slot (L - 1) % P of page block_table[b][(L - 1) // P]),
    for every KV head.  Pure indexing, no arithmetic."""
    kw = dict(bt.__dict__)
    kc, vc = bt.k_cache.clone(), bt.v_cache.clone()
    L = bt.seq_lens.to(torch.int64)
    page = bt.block_table[torch.arange(bt.batch), (L - 1) // bt.page_size].to(torch.int64)
    slot = (L - 1) % bt.page_size
    heads = torch.arange(bt.num_kv_heads)
    kc[page[:, None], heads[None, :], slot[:, None], :] = k_new.to(kc.dtype)
    vc[page[:, None], heads[None, :], :, slot[:, None]] = v_new.to(vc.dtype)
    kw["k_cache"], kw["v_cache"] = kc, vc
    return Batch(**kw)
