"""Seeded synthetic inputs for MLA chunked-context prefill.

This module is shared by both sides of every comparison (the CPU oracle and the
HIP library) and by the benchmark.  It holds no arithmetic of the method: only
problem sizes, seeded random draws and the buffer layouts the draws are written
into.  The oracle and the library never import each other; both receive the
arrays built here.

Layouts (token-major, as in the merge kernel's test on the vLLM PR #49294
digest, section 关键源码片段, where the output is [tokens, heads, head_dim]
and the LSE is [heads, tokens]):
  q, k_new        [T, H, 192]   bf16   (192 = 128 no-rope + 64 rope dims)
  v_new           [T, H, 128]   bf16
  k_cache         [NB, B, H, 192] bf16 paged cache, B rows per block
  v_cache         [NB, B, H, 128] bf16
  block_table     [N, max_blocks] int32, physical block of each logical block

Unused cache slots (spare blocks, and the slots of a request's last block past
its context length) hold NaN when ``canary=True``, so any read of a row that
is not part of a request's context shows up as NaN downstream.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DK = 192  # query/key head dim: 128 no-rope + 64 rope
DV = 128  # value head dim


@dataclass(frozen=True)
class Workload:
    """One problem instance: request lengths plus kernel-shape parameters."""

    name: str
    context_lens: tuple
    query_lens: tuple
    num_heads: int
    workspace_rows: int
    split_alignment: int
    block_size: int
    std: float = 1.0
    seed: int = 0

    @property
    def num_requests(self) -> int:
        return len(self.context_lens)

    @property
    def num_tokens(self) -> int:
        return int(sum(self.query_lens))

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(DK)


def _config4_lens(seed: int = 4):
    """Heterogeneous batch: 32 requests, context log-uniform in [1, 131072],
    four of them set to zero, query lens uniform in [1, 2048].  Draw order:
    context, zeroed indices, query lens."""
    rng = np.random.default_rng(seed)
    n = 32
    ctx = np.clip(np.round(np.exp(rng.uniform(0.0, math.log(131072), size=n))), 1, 131072).astype(np.int64)
    zero_idx = rng.choice(n, size=4, replace=False)
    ctx[zero_idx] = 0
    ql = rng.integers(1, 2048, size=n, endpoint=True)
    return tuple(int(x) for x in ctx), tuple(int(x) for x in ql)


def named_workloads():
    """The five named workloads, indexed 1..5."""
    c4, q4 = _config4_lens(4)
    return {
        1: Workload("tiny", (768, 512, 512, 0), (3, 5, 7, 4), 8, 1024, 64, 64, 1.0, 1),
        2: Workload("empty_context_stress", tuple([4] * 32 + [0, 3]), tuple([2] + [1] * 31 + [131, 1]),
                    16, 256, 16, 16, 1.0, 2),
        3: Workload("homogeneous", tuple([4096] * 16), tuple([512] * 16), 128, 65536, 64, 64, 1.0, 3),
        4: Workload("heterogeneous", c4, q4, 128, 131072, 64, 64, 1.0, 4),
        5: Workload("long_context", tuple([131072] * 4), tuple([8192] * 4), 128, 65536, 64, 64, 0.5, 5),
    }


def extra_workloads():
    """Batches beyond the five named ones, for scheduler comparisons.

    skewed: one request with a 131072-row context among 63 with 64 rows, 512
    new tokens each (T = 32768), H = 128, workspace 131072 rows, A = B = 64.
    The equal-window scheduler gives every request with context a 2048-row
    window and needs 64 iterations over the whole batch for the long request;
    per-request packing needs 2 chunks.

    heterogeneous_h16: the heterogeneous batch (seed-4 lengths) at 16 heads,
    one GPU's share when its 128 heads are split over 8 GPUs; most of its
    chunk-attention launches then have fewer workgroups than the GPU has CUs."""
    c4, q4 = _config4_lens(4)
    return {
        "skewed": Workload("skewed", tuple([131072] + [64] * 63), tuple([512] * 64), 128, 131072, 64, 64, 1.0, 6),
        "heterogeneous_h16": Workload("heterogeneous_h16", c4, q4, 16, 131072, 64, 64, 1.0, 4),
    }


def workload_by_name(name: str) -> Workload:
    for w in list(named_workloads().values()) + list(extra_workloads().values()):
        if w.name == name:
            return w
    raise KeyError(name)


def random_workload(seed: int, max_requests=6, max_ctx=300, max_q=40, heads=(1, 2, 4),
                    alignments=(1, 2, 4, 8, 16), zero_frac=0.25) -> Workload:
    """A small random instance for property tests (seeded)."""
    rng = np.random.default_rng(10_000 + seed)
    n = int(rng.integers(1, max_requests + 1))
    ctx = [0 if rng.random() < zero_frac else int(rng.integers(1, max_ctx + 1)) for _ in range(n)]
    ql = [int(rng.integers(0 if rng.random() < 0.1 else 1, max_q + 1)) for _ in range(n)]
    a = int(rng.choice(alignments))
    b = a if rng.random() < 0.7 else int(rng.choice([x for x in (1, 2, 4, 8, 16, 32) if x >= 1]))
    w = int(rng.integers(a, max(a, 2 * max_ctx) + 1))
    w = max(a, (w // a) * a) if rng.random() < 0.5 else max(a, w)
    return Workload(f"random{seed}", tuple(ctx), tuple(ql), int(rng.choice(heads)), w, a, b, 1.0, 10_000 + seed)


# ----------------------------------------------------------------------------
# buffers


@dataclass
class Batch:
    """Device (or host) tensors of one workload, plus the host-side lens."""

    wl: Workload
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    num_blocks: int
    spare_blocks: list = field(default_factory=list)

    @property
    def context_lens(self):
        return np.asarray(self.wl.context_lens, dtype=np.int32)

    @property
    def query_lens(self):
        return np.asarray(self.wl.query_lens, dtype=np.int32)

    @property
    def query_start_loc(self):
        return np.concatenate([[0], np.cumsum(self.query_lens, dtype=np.int64)]).astype(np.int64)


def block_table_for(context_lens, block_size: int, seed: int, spare_frac: float = 0.05):
    """Each request gets ceil(ctx/B) distinct physical blocks, taken in order
    from a seeded permutation of a pool with ~5% spare blocks.  Table padding
    points at a spare block so that a stray read lands on canary rows."""
    rng = np.random.default_rng(seed * 7919 + 17)
    need = [(int(c) + block_size - 1) // block_size for c in context_lens]
    used = sum(need)
    spare = max(1, int(math.ceil(used * spare_frac)))
    pool = used + spare
    perm = rng.permutation(pool).astype(np.int32)
    width = max(1, max(need) if need else 1)
    spare_ids = perm[used:]
    table = np.full((len(need), width), spare_ids[0], dtype=np.int32)
    pos = 0
    for r, nb in enumerate(need):
        table[r, :nb] = perm[pos:pos + nb]
        pos += nb
    return table, pool, [int(x) for x in spare_ids]


_PIECE = 1 << 24  # elements generated per seeded piece


def _fill_normal(t: torch.Tensor, seed: int, tensor_id: int, std: float, gen_device: str):
    """Fill a bf16 tensor with N(0, std) values drawn in fp32 and rounded to
    bf16 (round-to-nearest-even).  Pieces are seeded independently so the
    result does not depend on the piece processing order."""
    flat = t.view(-1)
    n = flat.numel()
    g = torch.Generator(device=gen_device)
    for i, off in enumerate(range(0, n, _PIECE)):
        m = min(_PIECE, n - off)
        g.manual_seed((seed * 1_000_003 + tensor_id * 10_007 + i) & 0x7FFF_FFFF_FFFF)
        x = torch.randn(m, generator=g, device=gen_device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[off:off + m].copy_(x.to(torch.bfloat16))


def make_batch(wl: Workload, device="cpu", gen_device=None, canary=True) -> Batch:
    """Build the input tensors of ``wl`` on ``device``.

    Values are drawn on ``gen_device`` (default: ``device``); the CPU generator
    gives identical values on every machine, so small cases are drawn on the
    CPU and then moved."""
    gen_device = gen_device or (device if isinstance(device, str) else str(device))
    if gen_device.startswith("cuda"):
        gen_device = "cuda"
    H, B, T = wl.num_heads, wl.block_size, wl.num_tokens
    table, pool, spare = block_table_for(wl.context_lens, B, wl.seed)
    bf = torch.bfloat16

    def alloc(*shape):
        return torch.empty(*shape, dtype=bf, device=gen_device)

    q, k_new, v_new = alloc(T, H, DK), alloc(T, H, DK), alloc(T, H, DV)
    k_cache, v_cache = alloc(pool, B, H, DK), alloc(pool, B, H, DV)
    for tid, t in enumerate((q, k_new, v_new, k_cache, v_cache)):
        _fill_normal(t, wl.seed, tid, wl.std, gen_device)
    if canary:
        nan = float("nan")
        for blk in spare:
            k_cache[blk].fill_(nan)
            v_cache[blk].fill_(nan)
        for r, c in enumerate(wl.context_lens):
            tail = c % B
            if c > 0 and tail:
                last = int(table[r, (c - 1) // B])
                k_cache[last, tail:].fill_(nan)
                v_cache[last, tail:].fill_(nan)
    tensors = [q, k_new, v_new, k_cache, v_cache]
    if str(device) != gen_device:
        tensors = [t.to(device) for t in tensors]
    bt = torch.from_numpy(table).to(device)
    return Batch(wl, *tensors, block_table=bt, num_blocks=pool, spare_blocks=spare)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a bf16 tensor (every bf16 value is an fp64 value)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


# ----------------------------------------------------------------------------
# context sharded over emulated ranks


@dataclass
class RankCache:
    """One rank's share of the paged context cache (its positions, in order)."""

    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    num_blocks: int
    context_lens: list


def shard_context(b: Batch, world: int, interleave: int = 1, canary=True, seed: int = 0):
    """Split ``b``'s paged cache over ``world`` ranks: runs of ``interleave``
    consecutive context positions go to ranks in turn (run k to rank k % world),
    and each rank stores its positions of a request in order in blocks of its
    own (taken from a seeded permutation, with spare NaN blocks that table
    padding points at).  Returns a list of RankCache on b's device."""
    wl = b.wl
    B = wl.block_size
    dev = b.k_cache.device
    table = b.block_table.cpu().numpy()
    ranks = []
    for rank in range(world):
        positions = []
        for r, c in enumerate(wl.context_lens):
            p = np.arange(int(c), dtype=np.int64)
            positions.append(p[(p // interleave) % world == rank])
        lens = [len(p) for p in positions]
        ltable, pool, spare = block_table_for(lens, B, 1000 * (seed + 1) + 31 * rank + world)
        k = torch.full((pool, B) + tuple(b.k_cache.shape[2:]), float("nan") if canary else 0.0,
                       dtype=b.k_cache.dtype, device=dev)
        v = torch.full((pool, B) + tuple(b.v_cache.shape[2:]), float("nan") if canary else 0.0,
                       dtype=b.v_cache.dtype, device=dev)
        src, dst = [], []
        for r, p in enumerate(positions):
            if len(p) == 0:
                continue
            src.append(table[r][p // B].astype(np.int64) * B + p % B)
            li = np.arange(len(p), dtype=np.int64)
            dst.append(ltable[r][li // B].astype(np.int64) * B + li % B)
        if src:
            s = torch.from_numpy(np.concatenate(src)).to(dev)
            d = torch.from_numpy(np.concatenate(dst)).to(dev)
            k.view(pool * B, -1).index_copy_(0, d, b.k_cache.view(-1, k.shape[2] * k.shape[3]).index_select(0, s))
            v.view(pool * B, -1).index_copy_(0, d, b.v_cache.view(-1, v.shape[2] * v.shape[3]).index_select(0, s))
        ranks.append(RankCache(k, v, torch.from_numpy(ltable).to(dev), pool, lens))
    return ranks
