"""Seeded synthetic decode-attention inputs, shared by the tests, the bench and
the oracle's callers.

This module only draws random numbers and lays them out; it holds none of the
attention, scoring or selection arithmetic.  It produces

* logical arrays -- q [B, H_q, d], K and V [B, H_kv, n_alloc, d] and the
  valid lengths seq_lens [B] -- which the oracle reads, and
* a paged copy of the same K and V -- pools [num_pages, H_kv, P, d] in a
  shuffled physical order plus a block table [B, max_pages] -- which the GPU
  library reads.

Stored values are float32 for dtype "f32" and bfloat16 bit patterns (uint16,
rounded to nearest even from the float32 draw) for dtype "bf16".

Workload recipes (one per decode-attention configuration):

* ``tiny``    B=1, H_q=4, H_kv=1, d=64, n=1024, f32, token unit, r_KV=0.25;
              q, K, V ~ N(0, 1); 32 salient keys per query head, each set to
              3 * q_hat + noise with noise ~ N(0, 0.5^2) per channel.
* ``l8b``     Llama-3.1-8B-shaped layer: B=1, H_q=32, H_kv=8, d=128, bf16,
              page 16, n=32768, page unit, r_KV=0.3; K, V ~ N(0,1) times a
              per-channel scale ~ U(0.5, 2) (independent per KV head and for
              K and V); 1% of positions per KV head are salient keys as above,
              assigned round-robin to the group's query heads.
* ``sweep``   the same shape and values at n in {2K, 8K, 32K, 64K, 128K},
              token unit, r_KV in {1.0, 0.3, 0.2}.
* ``batch``   16 sequences with lengths uniform on [49152, 65536], each drawn
              independently like ``l8b``, page unit, r_KV=0.2.
* ``l70b``    Llama-3.1-70B-shaped layer on one GPU: H_q=64, H_kv=8, d=128,
              bf16, page 64, n in {128K, 1M}, page unit, r_KV=0.05; values as
              ``l8b`` plus 1% planted salient pages per KV head (every valid
              token of such a page is salient, round-robin over the group).

Draw order per sequence, from the recipe's generator: channel scales, q, then
per KV head the salient positions followed by their noise.  The bulk K and V
draws of each (sequence, KV head) come from their own PCG64 streams keyed by
(seed, sequence, KV head, K or V), so they can be drawn in parallel threads
and do not depend on the thread count.  The physical page permutation comes
from a second generator seeded from the recipe's seed.  "N(0, 0.5)" is read as
standard deviation 0.5.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

KTOK = 1024  # "K" tokens
_THREADS = max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------
# recipes
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Recipe:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str                    # "f32" | "bf16"
    seq_len: int                  # fixed length, or the upper end of a range
    seq_len_min: int | None       # lower end of an integer-uniform range
    unit: str                     # "token" | "page"
    r_kv: float
    seed: int
    channel_scale: tuple | None   # (lo, hi) of U(lo, hi) per channel, or None
    salient: str                  # "per_head" | "fraction" | "pages"
    salient_count: float          # keys per query head / fraction of positions / fraction of pages

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def with_(self, **kw) -> "Recipe":
        return replace(self, **kw)


RECIPES = {
    "tiny": Recipe("tiny", 1, 4, 1, 64, 16, "f32", 1024, None, "token", 0.25, 1,
                   None, "per_head", 32),
    "l8b": Recipe("l8b", 1, 32, 8, 128, 16, "bf16", 32 * KTOK, None, "page", 0.3, 2,
                  (0.5, 2.0), "fraction", 0.01),
    "sweep": Recipe("sweep", 1, 32, 8, 128, 16, "bf16", 32 * KTOK, None, "token", 0.3, 3,
                    (0.5, 2.0), "fraction", 0.01),
    "batch": Recipe("batch", 16, 32, 8, 128, 16, "bf16", 64 * KTOK, 48 * KTOK, "page", 0.2, 4,
                    (0.5, 2.0), "fraction", 0.01),
    "l70b": Recipe("l70b", 1, 64, 8, 128, 64, "bf16", 128 * KTOK, None, "page", 0.05, 5,
                   (0.5, 2.0), "pages", 0.01),
}

SWEEP_CONTEXTS = (2 * KTOK, 8 * KTOK, 32 * KTOK, 64 * KTOK, 128 * KTOK)
L70B_CONTEXTS = (128 * KTOK, 1024 * KTOK)


def sweep_recipe(context: int, r_kv: float) -> Recipe:
    """``sweep`` at one context; the seed is 3 + the context's index."""
    i = SWEEP_CONTEXTS.index(context) if context in SWEEP_CONTEXTS else 0
    return RECIPES["sweep"].with_(seq_len=context, seed=3 + i, r_kv=r_kv)


def l70b_recipe(context: int) -> Recipe:
    i = L70B_CONTEXTS.index(context) if context in L70B_CONTEXTS else 0
    return RECIPES["l70b"].with_(seq_len=context, seed=5 + i)


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even
    (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    recipe: Recipe
    seq_lens: np.ndarray          # [B] int32
    q: np.ndarray                 # [B, H_q, d] stored
    K: np.ndarray                 # [B, H_kv, n_alloc, d] stored (zeros past seq_lens)
    V: np.ndarray
    salient: dict = field(default_factory=dict)   # (b, g) -> salient positions (token ids)
    salient_pages: dict = field(default_factory=dict)  # (b, g) -> planted page ids

    @property
    def n_alloc(self) -> int:
        return self.K.shape[2]

    def max_pages(self) -> int:
        return self.n_alloc // self.recipe.page_size

    def paged(self, seed_offset: int = 0, block_table=None) -> "PagedCache":
        """Scatter K and V into a shuffled physical page pool.

        Pages are numbered per sequence, u = 0 .. ceil(n_b / P) - 1; the pool
        holds sum_b ceil(n_b / P) pages in a random order, and block_table[b, u]
        names the physical page of logical page u.  Entries past a sequence's
        last page hold -1.  Rows past n_b inside a last page are zeros.  A
        given ``block_table`` (from another workload with the same lengths,
        e.g. another layer of the same sequences) is reused as is.
        """
        r = self.recipe
        P, B, H_kv, d = r.page_size, r.batch, r.num_kv_heads, r.head_dim
        U = [-(-int(n) // P) for n in self.seq_lens]
        num_pages = int(sum(U))
        if block_table is None:
            rng = np.random.Generator(np.random.PCG64(r.seed * 1000 + 7 + seed_offset))
            perm = rng.permutation(num_pages).astype(np.int32)
            block_table = np.full((B, self.max_pages()), -1, dtype=np.int32)
            off = 0
            for b in range(B):
                block_table[b, :U[b]] = perm[off:off + U[b]]
                off += U[b]
        k_pool = np.zeros((num_pages, H_kv, P, d), dtype=self.K.dtype)
        v_pool = np.zeros((num_pages, H_kv, P, d), dtype=self.V.dtype)

        def scatter(job):
            b, g = job
            ids = block_table[b, :U[b]]
            k_pool[ids, g] = self.K[b, g, :U[b] * P].reshape(U[b], P, d)
            v_pool[ids, g] = self.V[b, g, :U[b] * P].reshape(U[b], P, d)

        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(scatter, [(b, g) for b in range(B) for g in range(H_kv)]))
        return PagedCache(k_pool, v_pool, block_table, num_pages)


@dataclass
class PagedCache:
    k_pool: np.ndarray       # [num_pages, H_kv, P, d]
    v_pool: np.ndarray
    block_table: np.ndarray  # [B, max_pages] int32
    num_pages: int


def _salient_key(rng, qhat, d, count):
    """``count`` salient keys along unit vector qhat: 3 * qhat + N(0, 0.5^2)."""
    return (3.0 * qhat[None, :] + 0.5 * rng.standard_normal((count, d))).astype(np.float32)


def generate(recipe: Recipe, *, seq_lens=None) -> Workload:
    """Draw one workload from ``recipe`` (seeded by ``recipe.seed``)."""
    r = recipe
    rng = np.random.Generator(np.random.PCG64(r.seed))
    B, H_q, H_kv, d, P, G = r.batch, r.num_q_heads, r.num_kv_heads, r.head_dim, r.page_size, r.group
    if seq_lens is None:
        if r.seq_len_min is None:
            seq_lens = np.full(B, r.seq_len, dtype=np.int32)
        else:
            seq_lens = rng.integers(r.seq_len_min, r.seq_len, endpoint=True, size=B).astype(np.int32)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    n_max = int(seq_lens.max())
    n_alloc = -(-n_max // P) * P
    store_dt = np.float32 if r.dtype == "f32" else np.uint16
    q_all = np.empty((B, H_q, d), dtype=store_dt)
    K_all = np.zeros((B, H_kv, n_alloc, d), dtype=store_dt)
    V_all = np.zeros((B, H_kv, n_alloc, d), dtype=store_dt)
    salient, salient_pages = {}, {}
    scales, qs = [], []
    for b in range(B):
        if r.channel_scale is not None:
            lo, hi = r.channel_scale
            sk = rng.uniform(lo, hi, size=(H_kv, d)).astype(np.float32)
            sv = rng.uniform(lo, hi, size=(H_kv, d)).astype(np.float32)
        else:
            sk = sv = np.ones((H_kv, d), dtype=np.float32)
        scales.append((sk, sv))
        qs.append(rng.standard_normal((H_q, d), dtype=np.float32))

    def bulk(job):
        b, g, which = job
        n = int(seq_lens[b])
        stream = np.random.Generator(np.random.PCG64(np.random.SeedSequence([r.seed, b, g, which])))
        dst = K_all if which == 0 else V_all
        dst[b, g, :n] = _store(stream.standard_normal((n, d), dtype=np.float32) * scales[b][which][g],
                               r.dtype)

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(bulk, [(b, g, w) for b in range(B) for g in range(H_kv) for w in (0, 1)]))

    for b in range(B):
        n = int(seq_lens[b])
        q = qs[b]
        qhat = q / np.linalg.norm(q, axis=1, keepdims=True)
        # salient positions, then their noise
        for g in range(H_kv):
            heads = [g * G + i for i in range(G)]
            if r.salient == "per_head":
                cnt = int(r.salient_count)
                pos = rng.choice(n, size=cnt * G, replace=False).astype(np.int64)
                owner = np.repeat(np.arange(G), cnt)
            elif r.salient == "fraction":
                cnt = math.ceil(r.salient_count * n)
                pos = rng.choice(n, size=cnt, replace=False).astype(np.int64)
                owner = np.arange(cnt) % G
            elif r.salient == "pages":
                U = -(-n // P)
                cntp = math.ceil(r.salient_count * U)
                pages = np.sort(rng.choice(U, size=cntp, replace=False).astype(np.int64))
                salient_pages[(b, g)] = pages
                pos_l, own_l = [], []
                for i, u in enumerate(pages):
                    toks = np.arange(u * P, min((u + 1) * P, n))
                    pos_l.append(toks)
                    own_l.append(np.full(toks.size, i % G))
                pos = np.concatenate(pos_l)
                owner = np.concatenate(own_l)
            else:
                raise ValueError(r.salient)
            for i in range(G):
                sel = pos[owner == i]
                if sel.size:
                    K_all[b, g, sel] = _store(_salient_key(rng, qhat[heads[i]], d, sel.size), r.dtype)
            salient[(b, g)] = np.sort(pos)
        q_all[b] = _store(q, r.dtype)
    return Workload(r, seq_lens, q_all, K_all, V_all, salient, salient_pages)
