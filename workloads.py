"""Seeded synthetic workloads for the paged KV cache path.

This module only draws random numbers and lays out allocation bookkeeping (how
many pages each sequence owns and which physical ids they get). It contains
none of the path's arithmetic (no slot formula, no attention), so both the CPU
oracle and the HIP library can be fed from it.

Each workload is one layer of a decode batch shaped after the pages:

* ``tiny``      fp32, bs=4, Hq=4, Hkv=2, d=8, 12 pages pre-filled with N(0,1)
                garbage, context lengths [1, 4, 11], pages popped from a seeded
                permutation of the pool (the worked test of "Paged KV Cache · AI
                infra interview lesson", Step 2); ``tiny16``/``tiny256`` are the
                same at bs=16/256 with lengths [1, bs, 2bs+3]. All tokens are
                written through the store step before decoding.
* ``llama7b``   Llama-2-7B-shaped layer (Hq=Hkv=32, d=128, bs=16), 64 sequences,
                ctx ~ U{512..4096}, pool = exact need + 10 %, random pages.
* ``gqa``       Hq=32, Hkv=8, d=128, bs=16, 256 sequences, ctx log-uniform in
                [128, 8192].
* ``qwen3``     Qwen3-0.6B-shaped layer with 256-token pages: Hq=16, Hkv=8,
                d=128, 128 sequences, ctx ~ U{1..16384}; ~5 % of the new-token
                slots are dropped (set to -1) before the store.
* ``prefix``    512 sequences in 32 groups of 16 that share a 2048-token prefix
                (the same 128 page ids in every table of a group) followed by
                private tails of U{64..1024} tokens written by chunked prefill
                whose chunks start mid-page; u64 indices.

The decode step of every workload first stores one new token per sequence at
position ctx-1 (except ``tiny*`` and ``prefix``, which store their listed
tokens), then decodes with context length ctx.

Index structures are drawn on the host with numpy's PCG64 (independent of the
device); value tensors are drawn with a seeded ``torch.Generator`` on the
requested device.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
INDEX_NP = {"u32": np.uint32, "u64": np.uint64}


@dataclass
class Workload:
    name: str
    dtype: str
    index: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    context_lens: np.ndarray            # int32 [B]
    seq_ptr: np.ndarray                 # u32/u64 [B+1]
    block_table: np.ndarray             # u32/u64 [nnz]
    scale: float
    # store step: list of chunks; a chunk is (start_pos int32 [B], cu_new int64 [B+1])
    chunks: List[Tuple[np.ndarray, np.ndarray]] = field(default_factory=list)
    # new-token rows whose slot is replaced by -1 before the store (bool [N]) or None
    drop_mask: Optional[np.ndarray] = None
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return len(self.context_lens)

    @property
    def num_new_tokens(self) -> int:
        return int(sum(int(cu[-1]) for _, cu in self.chunks))

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    def kv_bytes_logical(self) -> int:
        """K+V bytes one decode pass must read: sum(ctx) * 2 * Hkv * d * b."""
        b = torch.tensor([], dtype=self.torch_dtype).element_size()
        return int(self.context_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * b

    def kv_bytes_unique(self) -> int:
        """K+V bytes of the distinct pages referenced (aliased pages counted once)."""
        b = torch.tensor([], dtype=self.torch_dtype).element_size()
        used = set()
        sp = self.seq_ptr.astype(np.int64)
        for s in range(self.num_seqs):
            n_pages = -(-int(self.context_lens[s]) // self.page_size)
            used.update(self.block_table[sp[s]:sp[s] + n_pages].tolist())
        return len(used) * self.page_size * 2 * self.num_kv_heads * self.head_dim * b

    def kv_bytes_unique_rows(self) -> int:
        """K+V bytes of the distinct pool rows a decode pass reads (rows t < ctx of every
        sequence's pages; a row shared by aliased pages counted once)."""
        b = torch.tensor([], dtype=self.torch_dtype).element_size()
        rows = {}
        sp = self.seq_ptr.astype(np.int64)
        for s in range(self.num_seqs):
            n = int(self.context_lens[s])
            for k in range(-(-n // self.page_size)):
                page = int(self.block_table[sp[s] + k])
                rows[page] = max(rows.get(page, 0), min(self.page_size, n - k * self.page_size))
        return sum(rows.values()) * 2 * self.num_kv_heads * self.head_dim * b

    def with_dtype(self, dtype: str) -> "Workload":
        w = Workload(**{**self.__dict__})
        w.dtype = dtype
        return w

    def with_index(self, index: str) -> "Workload":
        w = Workload(**{**self.__dict__})
        w.index = index
        w.seq_ptr = self.seq_ptr.astype(INDEX_NP[index])
        w.block_table = self.block_table.astype(INDEX_NP[index])
        return w


def _pages_needed(ctx: int, bs: int) -> int:
    # allocation bookkeeping: a sequence of ctx tokens owns ceil(ctx/bs) pages
    return -(-int(ctx) // bs)


def _csr(tables: List[List[int]], index: str):
    lens = [len(t) for t in tables]
    seq_ptr = np.zeros(len(tables) + 1, dtype=np.int64)
    seq_ptr[1:] = np.cumsum(lens)
    flat = np.array([p for t in tables for p in t], dtype=np.int64)
    return seq_ptr.astype(INDEX_NP[index]), flat.astype(INDEX_NP[index])


def _decode_step_chunks(ctx: np.ndarray):
    """One new token per sequence at position ctx-1 (the token being decoded)."""
    B = len(ctx)
    start = (ctx.astype(np.int64) - 1).clip(min=0).astype(np.int32)
    cu = np.arange(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum((ctx > 0).astype(np.int64))
    return [(start, cu)]


def _random_pool_tables(rng, ctx, bs, index, slack=0.10):
    """Tables drawn from a random permutation of a pool of need*(1+slack) pages."""
    need = [_pages_needed(c, bs) for c in ctx]
    total = int(sum(need))
    num_pages = max(1, int(np.ceil(total * (1.0 + slack))))
    perm = rng.permutation(num_pages)
    tables, k = [], 0
    for n in need:
        tables.append(perm[k:k + n].tolist())
        k += n
    seq_ptr, bt = _csr(tables, index)
    return num_pages, seq_ptr, bt


def tiny(bs: int = 4, dtype: str = "f32", index: str = "u32", seed: int = 1) -> Workload:
    rng = np.random.default_rng(seed)
    Hq, Hkv, d, nb = 4, 2, 8, 12
    lens = [1, 4, 11] if bs == 4 else [1, bs, 2 * bs + 3]
    free = rng.permutation(nb).tolist()
    tables = []
    for L in lens:
        tables.append([free.pop() for _ in range(_pages_needed(L, bs))])
    seq_ptr, bt = _csr(tables, index)
    ctx = np.array(lens, dtype=np.int32)
    start = np.zeros(len(lens), dtype=np.int32)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    name = "tiny" if bs == 4 else f"tiny{bs}"
    return Workload(name, dtype, index, Hq, Hkv, d, bs, nb, ctx, seq_ptr, bt, d ** -0.5,
                    chunks=[(start, cu)], seed=seed)


def llama7b(dtype: str = "bf16", index: str = "u32", seed: int = 2, batch: int = 64) -> Workload:
    rng = np.random.default_rng(seed)
    ctx = rng.integers(512, 4096, size=batch, endpoint=True).astype(np.int32)
    num_pages, seq_ptr, bt = _random_pool_tables(rng, ctx, 16, index)
    return Workload("llama7b", dtype, index, 32, 32, 128, 16, num_pages, ctx, seq_ptr, bt,
                    128 ** -0.5, chunks=_decode_step_chunks(ctx), seed=seed)


def gqa(dtype: str = "bf16", index: str = "u32", seed: int = 3, batch: int = 256) -> Workload:
    rng = np.random.default_rng(seed)
    ctx = np.rint(np.exp(rng.uniform(np.log(128), np.log(8192), size=batch))).astype(np.int32)
    num_pages, seq_ptr, bt = _random_pool_tables(rng, ctx, 16, index)
    return Workload("gqa", dtype, index, 32, 8, 128, 16, num_pages, ctx, seq_ptr, bt,
                    128 ** -0.5, chunks=_decode_step_chunks(ctx), seed=seed)


def qwen3(dtype: str = "bf16", index: str = "u32", seed: int = 4, batch: int = 128) -> Workload:
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, 16384, size=batch, endpoint=True).astype(np.int32)
    num_pages, seq_ptr, bt = _random_pool_tables(rng, ctx, 256, index)
    chunks = _decode_step_chunks(ctx)
    drop = rng.random(int(chunks[0][1][-1])) < 0.05
    return Workload("qwen3", dtype, index, 16, 8, 128, 256, num_pages, ctx, seq_ptr, bt,
                    128 ** -0.5, chunks=chunks, drop_mask=drop, seed=seed)


def chunked_prefill(name: str = "prefix", dtype: str = "bf16", index: str = "u64", seed: int = 5,
                    groups: int = 32, group_size: int = 16, prefix_tokens: int = 2048,
                    n_chunks: int = 3, num_q_heads: int = 32, num_kv_heads: int = 8,
                    head_dim: int = 128, bs: int = 16, tail_lo: int = 64,
                    tail_hi: int = 1024) -> Workload:
    """Groups of sequences aliasing a common prefix of prefix_tokens (whole pages,
    the same page ids in every table of the group), each followed by a private
    tail of U{tail_lo..tail_hi} tokens written in n_chunks chunks cut at seeded
    points (some chunk starts mid-page)."""
    assert prefix_tokens % bs == 0, "an aliased prefix covers whole pages"
    rng = np.random.default_rng(seed)
    B = groups * group_size
    tails = rng.integers(tail_lo, tail_hi, size=B, endpoint=True)
    prefix_pages = _pages_needed(prefix_tokens, bs)
    need = groups * prefix_pages + int(sum(_pages_needed(t, bs) for t in tails))
    num_pages = max(1, int(np.ceil(need * 1.10)))
    perm = rng.permutation(num_pages).tolist()
    tables = []
    k = 0
    for g in range(groups):
        shared = perm[k:k + prefix_pages]
        k += prefix_pages
        for j in range(group_size):
            t = tails[g * group_size + j]
            own = perm[k:k + _pages_needed(t, bs)]
            k += len(own)
            tables.append(shared + own)
    seq_ptr, bt = _csr(tables, index)
    ctx = (prefix_tokens + tails).astype(np.int32)
    # chunked prefill of the tails: cut [prefix, prefix+T) into n_chunks pieces
    cuts = np.zeros((B, n_chunks + 1), dtype=np.int64)
    for s in range(B):
        inner = np.sort(rng.choice(np.arange(1, tails[s]), size=n_chunks - 1, replace=False))
        cuts[s] = np.concatenate([[0], inner, [tails[s]]]) + prefix_tokens
    if n_chunks > 1 and np.all(cuts[:, 1:-1] % bs == 0):  # make sure some chunk starts mid-page
        cuts[0, 1] += 1
    chunks = []
    for c in range(n_chunks):
        start = cuts[:, c].astype(np.int32)
        n = cuts[:, c + 1] - cuts[:, c]
        cu = np.zeros(B + 1, dtype=np.int64)
        cu[1:] = np.cumsum(n)
        chunks.append((start, cu))
    return Workload(name, dtype, index, num_q_heads, num_kv_heads, head_dim, bs, num_pages, ctx,
                    seq_ptr, bt, head_dim ** -0.5, chunks=chunks, seed=seed)


def prefix(dtype: str = "bf16", index: str = "u64", seed: int = 5, groups: int = 32,
           group_size: int = 16, prefix_tokens: int = 2048, n_chunks: int = 3) -> Workload:
    return chunked_prefill("prefix", dtype, index, seed, groups, group_size, prefix_tokens,
                           n_chunks)


WORKLOADS = {"tiny": tiny, "llama7b": llama7b, "gqa": gqa, "qwen3": qwen3, "prefix": prefix}


@dataclass
class Tensors:
    q: torch.Tensor          # [B, Hq, d]
    k_cache: torch.Tensor    # [num_pages, bs, Hkv, d]
    v_cache: torch.Tensor
    new_keys: List[torch.Tensor]    # per chunk [N_c, Hkv, d]
    new_values: List[torch.Tensor]


def _randn(shape, dtype, device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, dtype=dtype, device=device, generator=g)


def make_tensors(w: Workload, device="cpu") -> Tensors:
    """N(0,1) pools (garbage everywhere), queries and new K/V rows."""
    dt = w.torch_dtype
    base = 1000 * w.seed
    pool_shape = (w.num_pages, w.page_size, w.num_kv_heads, w.head_dim)
    k_cache = _randn(pool_shape, dt, device, base + 1)
    v_cache = _randn(pool_shape, dt, device, base + 2)
    q = _randn((w.num_seqs, w.num_q_heads, w.head_dim), dt, device, base + 3)
    nk, nv = [], []
    for c, (_, cu) in enumerate(w.chunks):
        n = int(cu[-1])
        nk.append(_randn((n, w.num_kv_heads, w.head_dim), dt, device, base + 10 + 2 * c))
        nv.append(_randn((n, w.num_kv_heads, w.head_dim), dt, device, base + 11 + 2 * c))
    return Tensors(q, k_cache, v_cache, nk, nv)


def make_prefill_queries(w: Workload, device="cpu") -> List[torch.Tensor]:
    """N(0,1) queries of every chunk: [N_c, Hq, d] per chunk."""
    base = 1000 * w.seed
    return [_randn((int(cu[-1]), w.num_q_heads, w.head_dim), w.torch_dtype, device,
                   base + 50 + c) for c, (_, cu) in enumerate(w.chunks)]


@dataclass
class QuantTensors:
    k_codes: torch.Tensor    # uint8 [num_pages, bs, Hkv, d]
    v_codes: torch.Tensor
    k_scale: torch.Tensor    # fp32 [num_pages, Hkv]
    k_zero: torch.Tensor
    v_scale: torch.Tensor
    v_zero: torch.Tensor


def make_quant_tensors(w: Workload, kv_type: str, device="cpu",
                       fp8_full_range: bool = False) -> QuantTensors:
    """Random codes for quantized pools and per (page, KV head) scales and zero points:
    int8 scales U(0.005, 0.02) with integer zero points in [-8, 8], fp8 scales U(0.25, 1)
    with zero points U(-0.5, 0.5) and codes whose exponent field is at most 7 (magnitudes
    below 2, never a NaN code), so dequantized values stay below ~2.7 in magnitude, the
    O(1) range of N(0,1) K/V data.

    fp8_full_range: fp8 codes drawn from all 254 non-NaN codes (every exponent field,
    magnitudes up to 448) with power-of-two scales 2^-8 or 2^-9 and zero points that are
    integers in [-32, 32] on even pages and U(-32, 32) on odd ones, so values still
    dequantize to O(1); new N(0,1) rows stored with such scales land far beyond +-448
    (saturation) and, being 8-bit-mantissa numbers scaled by a power of two, often exactly
    halfway between two codes (ties)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * w.seed + 77)
    shape = (w.num_pages, w.page_size, w.num_kv_heads, w.head_dim)
    k = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
    v = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
    ps = (w.num_pages, w.num_kv_heads)
    if kv_type == "fp8" and fp8_full_range:
        for c in (k, v):  # the two NaN codes become +-0
            c[(c & 0x7F) == 0x7F] &= 0x80
        ks = torch.exp2(-8.0 - torch.randint(0, 2, ps, generator=g).float())
        vs = torch.exp2(-8.0 - torch.randint(0, 2, ps, generator=g).float())
        kz = torch.randint(-32, 33, ps, generator=g).float()
        vz = torch.randint(-32, 33, ps, generator=g).float()
        odd = torch.arange(w.num_pages) % 2 == 1
        kz[odd] = 64.0 * torch.rand((int(odd.sum()), w.num_kv_heads), generator=g) - 32.0
        vz[odd] = 64.0 * torch.rand((int(odd.sum()), w.num_kv_heads), generator=g) - 32.0
        return QuantTensors(*[x.contiguous().to(device) for x in (k, v, ks, kz, vs, vz)])
    if kv_type == "fp8":  # exponent field <= 7: magnitudes below 2, never a NaN code
        k &= 0xBF
        v &= 0xBF
    if kv_type == "i8":
        ks = 0.005 + 0.015 * torch.rand(ps, generator=g)
        vs = 0.005 + 0.015 * torch.rand(ps, generator=g)
        kz = torch.randint(-8, 9, ps, generator=g).float()
        vz = torch.randint(-8, 9, ps, generator=g).float()
    else:
        ks = 0.25 + 0.75 * torch.rand(ps, generator=g)
        vs = 0.25 + 0.75 * torch.rand(ps, generator=g)
        kz = torch.rand(ps, generator=g) - 0.5
        vz = torch.rand(ps, generator=g) - 0.5
    return QuantTensors(*[x.contiguous().to(device) for x in (k, v, ks, kz, vs, vz)])
