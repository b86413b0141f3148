"""Seeded synthetic inputs for paged-KV decode attention.

This module builds the tensors a decode-attention call consumes: the query
block, the paged K/V cache, block tables and sequence lengths.  It is shared
by the tests, the benchmark and the smoke check, and it holds none of the
attention arithmetic: no dot products, no softmax, no merge.  The oracle and
the HIP path both read what it produces; neither imports the other.

Cache layouts (the packed K+V slot of the octave backend page,
`RocmOctaveAttentionBackend.customize_spec`: one slot of 2*D elements per
(token, kv head), K in elements 0..D-1 and V in D..2D-1):

* HND: ``[num_blocks, num_kv_heads, page_size, 2, head_size]`` -- the
  block/head/token stride order of ``expected_kv_cache_strides`` on the
  rocm_rdna_hip docs page.
* NHD: ``[num_blocks, page_size, num_kv_heads, 2, head_size]``.

The five named workloads follow the benchmark configurations of the
decode-attention pull request (its "Performance" section describes the
harness: batch 1, HND, KV working set kept out of the last-level cache).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Sequence

import torch

NHD = 0
HND = 1

_DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Spec:
    """Shape and distribution of one workload family."""

    dtype: str
    head_size: int
    num_q_heads: int
    num_kv_heads: int
    page_size: int
    layout: int
    window: int = 0
    q_std: float = 1.0
    kv_std: float = 1.0
    table: str = "shuffled"  # "contiguous" | "shuffled"
    window_table_only: bool = False  # table entries only for pages the window reaches

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    @property
    def slot_bytes(self) -> int:
        return 2 * self.head_size * torch.tensor([], dtype=self.torch_dtype).element_size()

    @property
    def block_bytes(self) -> int:
        return self.page_size * self.num_kv_heads * self.slot_bytes


# The five benchmark configurations.  Context lengths and query counts are
# chosen per call; these are the fixed parts.
CONFIGS: dict[int, Spec] = {
    1: Spec("fp16", 64, 4, 1, 16, HND, table="contiguous"),
    2: Spec("bf16", 128, 32, 8, 16, HND),
    3: Spec("fp16", 256, 8, 2, 32, NHD, window=512, window_table_only=True),
    4: Spec("bf16", 512, 16, 2, 32, HND, kv_std=0.5),
    5: Spec("bf16", 256, 16, 2, 1056, HND),
}

# Context lengths / query counts each configuration is exercised at.
CONFIG_POINTS: dict[int, dict] = {
    1: {"contexts": [256], "queries": [1]},
    2: {"contexts": [128 << i for i in range(9)], "queries": [1, 2, 4]},
    3: {"contexts": [16384], "queries": [1, 4]},
    4: {"contexts": [1024 << i for i in range(6)], "queries": list(range(1, 9))},
    5: {"contexts": [16384], "queries": [4]},  # 16384 = the upper bound of the length mix
}

# Configuration 5: 64 live sequences with lengths uniform in [512, 16384]
# plus one padded sequence (length 0) at the end of the batch.
BATCH5_LIVE = 64
BATCH5_MIN_LEN = 512


def seed_for(cfg: int, context: int, queries: int) -> int:
    """Deterministic seed of one (configuration, context, query count) point."""
    return 20261202 + 1000 * cfg + 10 * int(math.log2(max(context, 1))) + queries


@dataclasses.dataclass
class Case:
    """One decode-attention call's inputs (possibly several pool instances).

    ``block_tables[i]`` addresses instance ``i``: the instances use disjoint
    physical blocks of the same pool, so rotating through them keeps the
    K/V bytes of consecutive calls distinct.
    """

    spec: Spec
    q: torch.Tensor  # [S, M, Hq, D]
    kv_cache: torch.Tensor  # layout-dependent 5-d tensor
    block_tables: list[torch.Tensor]  # int32 [S, max_blocks] each
    seq_lens: torch.Tensor  # int32 [S]
    scale: float
    window: int
    poison_block: int  # block id filled with NaN (never to be read)
    seed: int

    @property
    def num_seqs(self) -> int:
        return self.q.shape[0]

    @property
    def query_len(self) -> int:
        return self.q.shape[1]

    @property
    def max_blocks(self) -> int:
        return self.block_tables[0].shape[1]

    @property
    def layout(self) -> int:
        return self.spec.layout


def _fill_normal(t: torch.Tensor, std: float, gen: torch.Generator, chunk: int = 1 << 26) -> None:
    """Fill ``t`` (fp16/bf16) with N(0, std) drawn in fp32, chunk by chunk."""
    flat = t.view(-1)
    n = flat.numel()
    for start in range(0, n, chunk):
        stop = min(n, start + chunk)
        x = torch.randn(stop - start, generator=gen, device=t.device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[start:stop].copy_(x)


def _cache_shape(spec: Spec, num_blocks: int) -> tuple[int, ...]:
    if spec.layout == HND:
        return (num_blocks, spec.num_kv_heads, spec.page_size, 2, spec.head_size)
    return (num_blocks, spec.page_size, spec.num_kv_heads, 2, spec.head_size)


def window_first_page(seq_len: int, query_len: int, window: int, page_size: int) -> int:
    """First page a windowed sequence's block table must map.

    Query token m sits at position seq_len - query_len + m and sees at most
    ``window`` keys ending at itself (the window start of ``plan_prefill`` on
    the rocm_rdna_hip docs page), so the earliest key any of the query tokens
    needs is seq_len - query_len - window + 1.  Pages before it are never
    read; the generator points them at the poisoned block.
    """
    first_key = max(0, seq_len - query_len - window + 1)
    return first_key // page_size


def make_case(
    spec: Spec,
    seq_lens: Sequence[int],
    query_len: int,
    *,
    seed: int,
    device: str | torch.device = "cpu",
    instances: int = 1,
    pool_blocks: int | None = None,
    max_blocks: int | None = None,
    scale: float | None = None,
    window: int | None = None,
    poison_tail: bool = True,
    padded: Sequence[bool] | None = None,
) -> Case:
    """Build a seeded case.

    ``seq_lens`` are per sequence (0 = padded sequence).  ``pool_blocks``
    sizes the physical pool (default: exactly what the instances need, plus
    the poisoned block); the instances' blocks are a random permutation of
    the pool (or consecutive ids for ``spec.table == "contiguous"``).
    ``poison_tail`` fills the unused slots of each partial last page with
    NaN, so a kernel that reads past a sequence's length is caught.
    """
    device = torch.device(device)
    gen_cpu = torch.Generator(device="cpu").manual_seed(seed)
    gen_dev = gen_cpu if device.type == "cpu" else torch.Generator(device=device).manual_seed(seed)
    P = spec.page_size
    S = len(seq_lens)
    window = spec.window if window is None else window
    lens = [int(x) for x in seq_lens]
    need = [-(-L // P) for L in lens]  # pages per sequence
    if max_blocks is None:
        max_blocks = max(1, max(need))
    if any(n > max_blocks for n in need):
        raise ValueError("a sequence needs more blocks than max_blocks")
    first_page = [0] * S
    if spec.window_table_only and window > 0:
        first_page = [window_first_page(L, query_len, window, P) if L else 0 for L in lens]
    live_pages = [need[s] - first_page[s] for s in range(S)]
    per_instance = sum(live_pages)
    min_pool = per_instance * instances + 1
    if pool_blocks is None:
        pool_blocks = min_pool
    if pool_blocks < min_pool:
        raise ValueError(f"pool of {pool_blocks} blocks is too small for {instances} instances")
    poison = pool_blocks - 1

    if spec.table == "contiguous":
        order = torch.arange(pool_blocks - 1, dtype=torch.int64)
    else:
        order = torch.randperm(pool_blocks - 1, generator=gen_cpu)
    tables = []
    cursor = 0
    for _ in range(instances):
        bt = torch.full((S, max_blocks), poison, dtype=torch.int32)
        for s in range(S):
            n = live_pages[s]
            bt[s, first_page[s] : first_page[s] + n] = order[cursor : cursor + n].to(torch.int32)
            cursor += n
        tables.append(bt.to(device))

    Hq, D = spec.num_q_heads, spec.head_size
    q = torch.empty((S, query_len, Hq, D), dtype=spec.torch_dtype, device=device)
    _fill_normal(q, spec.q_std, gen_dev)
    kv = torch.empty(_cache_shape(spec, pool_blocks), dtype=spec.torch_dtype, device=device)
    _fill_normal(kv, spec.kv_std, gen_dev)
    kv[poison].fill_(float("nan"))
    if poison_tail:
        for bt in tables:
            for s in range(S):
                L = lens[s]
                if L % P:
                    blk = int(bt[s, need[s] - 1])
                    if spec.layout == HND:
                        kv[blk, :, L % P :].fill_(float("nan"))
                    else:
                        kv[blk, L % P :].fill_(float("nan"))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Case(
        spec=spec,
        q=q,
        kv_cache=kv,
        block_tables=tables,
        seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
        scale=float(scale),
        window=int(window),
        poison_block=poison,
        seed=seed,
    )


def config_case(
    cfg: int,
    context: int,
    query_len: int,
    *,
    device: str | torch.device = "cpu",
    instances: int = 1,
    pool_bytes: int = 0,
    seed: int | None = None,
) -> Case:
    """A case of named configuration ``cfg`` at one (context, query count).

    For configuration 5, ``context`` is the upper bound of the length mix:
    64 sequences draw lengths uniformly from [512, context] and a 65th,
    padded sequence has length 0.  ``pool_bytes`` grows the pool (the
    benchmark keeps it at 512 MiB or more so rotating instances stay out of
    the last-level cache).
    """
    spec = CONFIGS[cfg]
    if seed is None:
        seed = seed_for(cfg, context, query_len)
    if cfg == 5:
        gen = torch.Generator().manual_seed(seed ^ 0x5EED)
        lo = min(BATCH5_MIN_LEN, context)
        lens = torch.randint(lo, context + 1, (BATCH5_LIVE,), generator=gen).tolist() + [0]
        max_blocks = -(-context // spec.page_size)
    else:
        lens = [context]
        max_blocks = None
    per_instance_blocks = sum(-(-L // spec.page_size) for L in lens)
    pool_blocks = None
    if pool_bytes:
        need = -(-pool_bytes // spec.block_bytes)
        pool_blocks = max(need, per_instance_blocks * instances) + 1
    return make_case(
        spec,
        lens,
        query_len,
        seed=seed,
        device=device,
        instances=instances,
        pool_blocks=pool_blocks,
        max_blocks=max_blocks,
    )


def as_f64(t: torch.Tensor):
    """Exact fp64 numpy copy of a (device) tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def compact(case: Case, instance: int = 0, seqs: Sequence[int] | None = None):
    """Host copy of the blocks ``seqs`` reference, renumbered densely.

    Returns ``(kv64, table, seq_lens)``: an fp64 numpy cache holding only the
    referenced blocks (the poisoned block kept as id 0 if referenced), the
    block table rewritten to the new ids, and the sequence lengths.  The
    mapping is a pure renumbering of physical blocks.
    """
    import numpy as np

    bt = case.block_tables[instance].to("cpu").numpy()
    lens = case.seq_lens.to("cpu").numpy()
    if seqs is None:
        seqs = range(bt.shape[0])
    seqs = list(seqs)
    sub = bt[seqs]
    used = np.unique(sub)
    remap = {int(b): i for i, b in enumerate(used)}
    table = np.vectorize(lambda b: remap[int(b)], otypes=[np.int64])(sub) if sub.size else sub.astype(np.int64)
    idx = torch.as_tensor(used, dtype=torch.int64, device=case.kv_cache.device)
    kv64 = as_f64(case.kv_cache.index_select(0, idx))
    return kv64, table, lens[seqs].astype(np.int64)


def sign_words(seed: int, head_size: int = 256) -> torch.Tensor:
    """Seeded sign bits of a rotation, ``head_size // 32`` 32-bit words as an
    int32 tensor (the random draw of the octave page's ``sign_bits``, handed
    to both sides as an input; bit i % 32 of word i // 32 set = element i
    negated)."""
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-(1 << 31), 1 << 31, (head_size // 32,), generator=g, dtype=torch.int64).to(torch.int32)
