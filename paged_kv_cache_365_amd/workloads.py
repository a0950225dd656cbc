"""Seeded synthetic inputs for paged decode attention.

This module only *draws inputs*: query vectors, K/V pool contents, block tables
and context lengths.  It holds none of the attention arithmetic, so both the
fp64 CPU oracle and the HIP library read the very same bytes from it.

Layouts (they are the library's ABI, stated in ``include/pa.h``):

* ``q``            ``[B][H_q][d]``            element dtype of the pool
* ``k_pool``       ``[num_blocks][H_kv][d / x][16][x]``, x = 16 / element bytes:
                    each token row is cut into 16-byte chunks and a tile stores
                    chunk 0 of its 16 tokens, then chunk 1, ...
* ``v_pool``       ``[num_blocks][H_kv][d][16]``: a tile stores column 0 of its
                    16 tokens, then column 1, ...
                    Either way one (block, kv-head) tile is 16 * d elements,
                    contiguous.
* ``block_tables`` ``int32 [B][max_blocks_per_seq]``; entry ``j`` of row ``s``
                    is the physical block holding tokens ``16j .. 16j+15`` of
                    sequence ``s``; entries past the live range are ``-1``
* ``context_lens`` ``int32 [B]``

Element storage: ``f32`` arrays are ``np.float32``, ``f16`` arrays are
``np.float16``, ``bf16`` arrays are ``np.uint16`` holding the raw bfloat16 bits.

Value recipe: every value is N(0,1), drawn by inverse CDF over 65,536
equiprobable levels (a uniform 16-bit draw indexes a table of standard-normal
quantiles at (i + 0.5) / 65536, so tails stop at about +-4.2 sigma), then rounded
to nearest-even into the element dtype.  A plain ``standard_normal`` draw is about
a hundred times slower on the host and would dominate every run at the 1 GB pool
sizes used here.

The five workload shapes follow the cases the pages discuss: 16-token blocks
(the default block size stated on both PagedAttention pages), 7B-style MHA,
70B-style GQA with 8 KV heads, a shared system-prompt prefix referenced by
every block table, and a 32K long-context batch split into 512-token
partitions.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
from scipy.special import ndtri

BLOCK_SIZE = 16
DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
# numpy storage type per element dtype (bf16 is carried as raw bits)
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
NAN_BITS = {"f32": np.uint32(0x7FC00000), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}


def chunk_elems(dtype: str) -> int:
    """Elements per 16-byte chunk of a K row."""
    return 16 // ELEM_BYTES[dtype]


def pool_shapes(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str,
                block_size: int = BLOCK_SIZE):
    """(K pool shape, V pool shape) of the library's layout."""
    x = chunk_elems(dtype)
    return ((num_blocks, num_kv_heads, head_dim // x, block_size, x),
            (num_blocks, num_kv_heads, head_dim, block_size))


# --------------------------------------------------------------------------
# element encoding (input preparation only)
# --------------------------------------------------------------------------
def f64_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage form of ``dtype`` (nearest-even)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        f = x.astype(np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        nan = np.isnan(f)
        if nan.any():
            rounded = np.where(nan, np.uint16(0x7FC0), rounded)
        return rounded
    raise ValueError(f"unknown dtype {dtype!r}")


_QUANTILES = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0)
_TABLE_CACHE: dict = {}


def _normal_table(dtype: str, gain: float = 1.0) -> np.ndarray:
    key = (dtype, gain)
    if key not in _TABLE_CACHE:
        _TABLE_CACHE[key] = f64_to_storage(_QUANTILES * gain, dtype)
    return _TABLE_CACHE[key]


def normal(rng: np.random.Generator, shape, dtype: str, gain: float = 1.0) -> np.ndarray:
    """N(0, gain^2) values in the storage form of ``dtype``."""
    idx = rng.integers(0, 65536, size=shape, dtype=np.uint16)
    return _normal_table(dtype, gain)[idx]


def nan_fill(shape, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.full(shape, NAN_BITS["f32"], dtype=np.uint32).view(np.float32)
    if dtype == "f16":
        return np.full(shape, NAN_BITS["f16"], dtype=np.uint16).view(np.float16)
    return np.full(shape, NAN_BITS["bf16"], dtype=np.uint16)


def const_fill(shape, dtype: str, value: float) -> np.ndarray:
    return np.full(shape, f64_to_storage(np.array(value), dtype), dtype=STORAGE[dtype])


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q: np.ndarray             # [B][H_q][d] storage dtype
    k_pool: np.ndarray        # [NB][H_kv][d/x][16][x]
    v_pool: np.ndarray        # [NB][H_kv][d][16]
    block_tables: np.ndarray  # int32 [B][max_blocks_per_seq]
    context_lens: np.ndarray  # int32 [B]
    scale: float              # float32 value carried as a Python float
    partition_size: int = 0   # 0 = single phase
    prefix_blocks: int = 0    # number of leading table entries shared by all rows
    free_blocks: np.ndarray | None = None  # physical ids not referenced by any table

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def block_size(self) -> int:
        return int(self.k_pool.shape[3])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def kv_bytes_logical(self, key_bytes: int | None = None) -> int:
        """K+V bytes one decode call reads, counting shared blocks once per reference
        (``key_bytes``: bytes per key element when keys are stored narrower than
        values, e.g. 1 for int8 keys)."""
        e = ELEM_BYTES[self.dtype]
        kb = e if key_bytes is None else key_bytes
        per_token = self.num_kv_heads * self.head_dim * (kb + e)
        return int(self.context_lens.astype(np.int64).sum()) * per_token

    def kv_bytes_unique(self) -> int:
        """K+V bytes of the distinct live token slots (shared prefix counted once)."""
        per_token = 2 * self.num_kv_heads * self.head_dim * ELEM_BYTES[self.dtype]
        lens = self.context_lens.astype(np.int64)
        shared = self.prefix_blocks * self.block_size
        if shared and len(lens):
            return int(shared + (lens - shared).sum()) * per_token
        return int(lens.sum()) * per_token

    def algorithmic_bytes(self, unique: bool = False, query_tokens: int = 1,
                          key_bytes: int | None = None) -> int:
        """KV + q + out + live block-table entries + context_lens (q and out hold
        ``query_tokens`` rows per sequence and head: 1 for decode, T for a verify
        call over a T-token draft).  With int8 keys (``key_bytes`` = 1) the
        float32 channel scales are read too, with 2-bit keys (``key_bytes`` =
        0.25) the float32 channel steps and zero points."""
        e = ELEM_BYTES[self.dtype]
        qo = 2 * query_tokens * self.num_seqs * self.num_q_heads * self.head_dim * e
        bs = self.block_size
        live_entries = int(((self.context_lens.astype(np.int64) + bs - 1) // bs).sum())
        if unique:
            kv = self.kv_bytes_unique()
        else:
            kv = self.kv_bytes_logical(key_bytes)
        scales = {1: 4, 0.25: 8}.get(key_bytes, 0) * self.num_kv_heads * self.head_dim
        return kv + qo + 4 * live_entries + 4 * self.num_seqs + scales


# --------------------------------------------------------------------------
# quantised keys: an int8 key cache over a workload's tables
# --------------------------------------------------------------------------
K8_POISON = -128           # a code no quantised write produces: marks unwritten slots
K8_CODE_SPREAD = 30.0      # codes ~ N(0, 30^2): N(0,1) keys at scale 4.2 / 127
K8_BASE_SCALE = 4.2 / 127.0


def k8_inputs(w: "Workload", seed: int, outlier_columns: int = 0, outlier_gain: float = 10.0):
    """An int8 key cache for ``w``'s pool, tables and shapes (``w``'s V pool, q
    and tables are used with it): codes [NB][H_kv][d/16][16][16] drawn as integers
    near N(0, 30^2) (rounded draws, clamped to +-127), and float32 channel scales
    [H_kv][d] of 4.2/127, times ``outlier_gain`` on ``outlier_columns`` random
    (KV head, channel) columns -- the per-channel key outliers.  Free blocks and
    the slots past each context in its last block hold -128.  Returns
    (k8_pool int8, k_scale float32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    NB, Hkv, d, bs = w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size
    shape = (NB, Hkv, d // 16, bs, 16)
    draws = normal(rng, shape, "f32", gain=K8_CODE_SPREAD)
    codes = np.clip(np.rint(draws), -127, 127).astype(np.int8)
    k_scale = np.full((Hkv, d), K8_BASE_SCALE, dtype=np.float32)
    if outlier_columns:
        cols = rng.choice(Hkv * d, size=outlier_columns, replace=False)
        k_scale.reshape(-1)[cols] *= np.float32(outlier_gain)
    if w.free_blocks is not None and len(w.free_blocks):
        codes[w.free_blocks] = K8_POISON
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        o = L % bs
        if L and o:
            codes[w.block_tables[s, L // bs], :, :, o:, :] = K8_POISON
    return codes, k_scale


K2_BASE_STEP = 1.4         # 2-bit codes 0..3 at -2.1, -0.7, 0.7, 2.1: a coarse N(0,1) key
K2_BASE_ZERO = -2.1


def k2_inputs(w: "Workload", seed: int, outlier_columns: int = 0, outlier_gain: float = 10.0):
    """A 2-bit key cache for ``w``'s pool, tables and shapes (``w``'s V pool, q
    and tables are used with it): key words [NB][H_kv][4][bs][d/64] of uniform
    random bits (every 2-bit code equally likely, free blocks and tail slots
    included: every pattern is a code, so unread slots are shown unread by the
    NaN V pool), float32 channel steps [H_kv][d] of 1.4 and zero points of
    -2.1, both times ``outlier_gain`` on ``outlier_columns`` random (KV head,
    channel) columns -- the per-channel key outliers.  Returns (k2_pool uint32,
    k_scale float32, k_zero float32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    NB, Hkv, d, bs = w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size
    words = rng.integers(0, 2 ** 32, size=(NB, Hkv, 4, bs, d // 64), dtype=np.uint32)
    k_scale = np.full((Hkv, d), K2_BASE_STEP, dtype=np.float32)
    k_zero = np.full((Hkv, d), K2_BASE_ZERO, dtype=np.float32)
    if outlier_columns:
        cols = rng.choice(Hkv * d, size=outlier_columns, replace=False)
        k_scale.reshape(-1)[cols] *= np.float32(outlier_gain)
        k_zero.reshape(-1)[cols] *= np.float32(outlier_gain)
    return words, k_scale, k_zero


def _scale_for(head_dim: int) -> float:
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def build_workload(
    name: str,
    rng: np.random.Generator,
    *,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    context_lens,
    max_blocks_per_seq: int | None = None,
    pool_blocks: int | None = None,
    free_fraction: float = 0.10,
    prefix_tokens: int = 0,
    k_outlier_columns: int = 0,
    outlier_gain: float = 10.0,
    poison: bool = True,
    tail_fill: str = "nan",
    partition_size: int = 0,
    scale: float | None = None,
    block_size: int = BLOCK_SIZE,
) -> Workload:
    """Draw one workload.

    Physical ids come from a seeded permutation of the pool and are handed out
    in (sequence, logical block) order; shared prefix blocks are handed out
    first.  With ``poison`` the blocks no table references are NaN, the slots
    past a sequence's length inside its last block hold ``tail_fill``
    ("nan" or "sentinel" = +-1e3), and table entries past the live range are -1.
    """
    lens = np.asarray(context_lens, dtype=np.int32)
    B = len(lens)
    bs = block_size
    if prefix_tokens % bs:
        raise ValueError("shared prefix must be a whole number of blocks")
    prefix_blocks = prefix_tokens // bs
    need = [(int(L) + bs - 1) // bs for L in lens]
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(need) if need else 1
    max_blocks_per_seq = max(max_blocks_per_seq, 1)
    private = [n - prefix_blocks for n in need]
    if prefix_blocks and min(private) < 0:
        raise ValueError("every context must cover the shared prefix")
    used = prefix_blocks + sum(private)
    if pool_blocks is None:
        pool_blocks = max(int(math.ceil(used * (1.0 + free_fraction))), used + 1)
    if pool_blocks < used:
        raise ValueError("pool too small")

    perm = rng.permutation(pool_blocks).astype(np.int32)
    tables = np.full((B, max_blocks_per_seq), -1, dtype=np.int32)
    cursor = prefix_blocks
    for s in range(B):
        tables[s, :prefix_blocks] = perm[:prefix_blocks]
        n = private[s]
        tables[s, prefix_blocks:prefix_blocks + n] = perm[cursor:cursor + n]
        cursor += n
    free = perm[used:]

    kshape, vshape = pool_shapes(pool_blocks, num_kv_heads, head_dim, dtype, bs)
    x = chunk_elems(dtype)
    k_pool = normal(rng, kshape, dtype)
    v_pool = normal(rng, vshape, dtype)
    if k_outlier_columns:
        # a few (kv-head, channel) columns of K carry x10 values: the per-channel
        # key outliers that motivate per-channel K quantisation on the pages
        cols = rng.choice(num_kv_heads * head_dim, size=k_outlier_columns, replace=False)
        for c in np.sort(cols):
            g, ch = divmod(int(c), head_dim)
            k_pool[:, g, ch // x, :, ch % x] = normal(rng, (pool_blocks, bs), dtype,
                                                      gain=outlier_gain)
    q = normal(rng, (B, num_q_heads, head_dim), dtype)

    if poison:
        if len(free):
            k_pool[free] = nan_fill((len(free),) + kshape[1:], dtype)
            v_pool[free] = nan_fill((len(free),) + vshape[1:], dtype)
        for s in range(B):
            L = int(lens[s])
            o = L % bs
            if L == 0 or o == 0:
                continue
            b = tables[s, L // bs]
            kt = (num_kv_heads, head_dim // x, bs - o, x)
            vt = (num_kv_heads, head_dim, bs - o)
            if tail_fill == "nan":
                k_pool[b, :, :, o:, :] = nan_fill(kt, dtype)
                v_pool[b, :, :, o:] = nan_fill(vt, dtype)
            elif tail_fill == "sentinel":
                k_pool[b, :, :, o:, :] = const_fill(kt, dtype, 1e3)
                v_pool[b, :, :, o:] = const_fill(vt, dtype, -1e3)
            else:
                raise ValueError(tail_fill)

    return Workload(
        name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, q=q, k_pool=k_pool, v_pool=v_pool, block_tables=tables,
        context_lens=lens, scale=_scale_for(head_dim) if scale is None else float(np.float32(scale)),
        partition_size=partition_size, prefix_blocks=prefix_blocks, free_blocks=free,
    )


# --------------------------------------------------------------------------
# the five workload shapes
# --------------------------------------------------------------------------
CONFIG_NAMES = (
    "tiny-mha-f32",          # B2, H4/4, d64, fp32, lens 17 and 40, pool of 8 blocks
    "7b-mha-f16",            # B32, H32/32, d128, fp16, lens U[512, 4096]
    "70b-gqa8-bf16-4k",      # B64, H64/8, d128, bf16, lens 4096, 1% x10 K channels
    "shared-prefix-gqa4",    # B128, H32/8, d128, bf16, 1024 shared + U[16, 1024]
    "long-32k-split512",     # B4, H64/8, d128, bf16, lens 32768, 512-token partitions
)


def make_config(index: int, seed: int | None = None, *, poison: bool = True,
                tail_fill: str = "nan", block_size: int = BLOCK_SIZE) -> Workload:
    """Workload ``index`` (0..4) drawn with ``seed`` (default 1000 + index).  With
    ``block_size`` 8 the same shapes are cut into 8-token blocks (named with a
    "-bs8" suffix); the table width doubles."""
    if seed is None:
        seed = 1000 + index
    rng = np.random.Generator(np.random.PCG64(seed))
    name = CONFIG_NAMES[index] + ("" if block_size == BLOCK_SIZE else f"-bs{block_size}")
    per16 = BLOCK_SIZE // block_size   # table entries per 16 tokens
    kw = dict(poison=poison, tail_fill=tail_fill, block_size=block_size)
    if index == 0:
        return build_workload(name, rng, dtype="f32", num_q_heads=4, num_kv_heads=4,
                              head_dim=64, context_lens=[17, 40], pool_blocks=8 * per16, **kw)
    if index == 1:
        lens = rng.integers(512, 4096, size=32, endpoint=True)
        return build_workload(name, rng, dtype="f16", num_q_heads=32, num_kv_heads=32,
                              head_dim=128, context_lens=lens, max_blocks_per_seq=256 * per16,
                              **kw)
    if index == 2:
        return build_workload(name, rng, dtype="bf16", num_q_heads=64, num_kv_heads=8,
                              head_dim=128, context_lens=[4096] * 64,
                              max_blocks_per_seq=256 * per16, k_outlier_columns=10, **kw)
    if index == 3:
        lens = 1024 + rng.integers(16, 1024, size=128, endpoint=True)
        return build_workload(name, rng, dtype="bf16", num_q_heads=32, num_kv_heads=8,
                              head_dim=128, context_lens=lens, max_blocks_per_seq=128 * per16,
                              prefix_tokens=1024, **kw)
    if index == 4:
        return build_workload(name, rng, dtype="bf16", num_q_heads=64, num_kv_heads=8,
                              head_dim=128, context_lens=[32768] * 4,
                              max_blocks_per_seq=2048 * per16, partition_size=512, **kw)
    raise IndexError(index)


def make_random_case(seed: int, *, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                     head_dim: int, dtype: str, lens=None, max_len: int = 80,
                     partition_size: int = 0, poison: bool = True, tail_fill: str = "nan",
                     free_fraction: float = 0.25, prefix_tokens: int = 0,
                     block_size: int = BLOCK_SIZE) -> Workload:
    """A small random case for parity sweeps (ragged lengths, several tiles)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if lens is None:
        lens = rng.integers(max(prefix_tokens, 1), max_len, size=num_seqs, endpoint=True)
    return build_workload(f"random-{seed}", rng, dtype=dtype, num_q_heads=num_q_heads,
                          num_kv_heads=num_kv_heads, head_dim=head_dim, context_lens=lens,
                          free_fraction=free_fraction, poison=poison, tail_fill=tail_fill,
                          partition_size=partition_size, prefix_tokens=prefix_tokens,
                          block_size=block_size)
