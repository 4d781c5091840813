"""Seeded synthetic workloads for paged-KV attention.

This module only makes inputs: context lengths, the assignment of physical
blocks, block tables, slot mappings and the Q/K/V values.  It holds none of
the attention or quantisation arithmetic, and it imports neither the HIP
binding nor the reference implementation, so both can be fed from it.

Shapes follow the serving workloads on the pages:

* 16-token blocks, addressed through a block-id table per sequence
  ("PyTorch LLM Serving Engine", §What is implemented; "llminfer",
  §Paged KV Cache And Continuous Batching, page_size_tokens = 16);
* right-skewed, clipped log-normal context lengths ("PyTorch LLM Serving
  Engine", §Measured results and §What is implemented, benchmark harness);
* grouped-query head sharing ("MicroGen", §Key Features).

Every value is a pure function of (seed, tag, element index) through an
integer counter-based hash: the 32-bit finaliser of MurmurHash3
(Appleby).  No floating-point operation is involved before the final
exact integer-to-float conversion, so an element is bit-identical whether
it is made on the CPU or on a GPU, and any subset of a large case (one
sequence out of 256) can be generated on its own.

Normal variates use the Irwin-Hall construction: the sum of twelve
independent 16-bit uniforms, centred, is exactly representable in fp32,
has mean 0 and variance 1 (to 1 part in 2^32) and is bounded by +-6.
Context lengths use Box-Muller on the host (numpy, float64), which only
ever runs on the CPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

M32 = 0xFFFFFFFF

TAG_Q = 1
TAG_K = 2
TAG_V = 3
TAG_K_OUTLIER = 4
TAG_V_OUTLIER = 5
TAG_LENS = 6
TAG_PERM = 7
TAG_MISC = 8

_CHUNK = 1 << 24  # elements per generation sub-call on the CPU (bounds temporaries)
_CHUNK_GPU = 1 << 26


# ---------------------------------------------------------------- hashing
def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 tensors holding values in [0, 2^32).

    Split into 16-bit halves so no intermediate leaves the int64 range."""
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + (((hi * c) & 0xFFFF) << 16)) & M32


def _fmix32(h: torch.Tensor) -> torch.Tensor:
    """MurmurHash3 32-bit finaliser (a bijection on [0, 2^32))."""
    h = h ^ (h >> 16)
    h = _mul32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = _mul32(h, 0xC2B2AE35)
    h = h ^ (h >> 16)
    return h


def _key(seed: int, tag: int) -> int:
    k = (seed * 0x9E3779B9 + tag * 0x7F4A7C15 + 0x632BE5AB) & M32
    return int(_fmix32(torch.tensor([k], dtype=torch.int64)).item())


def hash_u32(seed: int, tag: int, counter: torch.Tensor) -> torch.Tensor:
    """Uniform 32-bit words for int64 counters (any device)."""
    key = _key(seed, tag)
    lo = counter & M32
    hi = counter >> 32
    return _fmix32(_fmix32(lo ^ key) ^ hi)


def _normal_of(seed: int, tag: int, counters: torch.Tensor) -> torch.Tensor:
    idx = counters * 6
    acc = torch.zeros(counters.shape, dtype=torch.int64, device=counters.device)
    for j in range(6):
        h = hash_u32(seed, tag, idx + j)
        acc += (h & 0xFFFF) + (h >> 16)
    # sum of 12 uniforms on {0..65535} has mean 12 * 32767.5 = 393210
    return (acc - 393210).to(torch.float32) * (1.0 / 65536.0)


def _normal_chunk(seed: int, tag: int, start: int, count: int, device) -> torch.Tensor:
    return _normal_of(seed, tag, torch.arange(start, start + count, dtype=torch.int64, device=device))


def normal_f32(seed: int, tag: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Approximately N(0,1) fp32 values for element counters [start, start+count)."""
    out = torch.empty(count, dtype=torch.float32, device=device)
    step = _CHUNK if torch.device(device).type == "cpu" else _CHUNK_GPU
    for c0 in range(0, count, step):
        n = min(step, count - c0)
        out[c0:c0 + n] = _normal_chunk(seed, tag, start + c0, n, device)
    return out


def bernoulli_mask(seed: int, tag: int, start: int, count: int, prob: float, device="cpu") -> torch.Tensor:
    thresh = int(math.ceil(prob * 2.0 ** 32))
    out = torch.empty(count, dtype=torch.bool, device=device)
    for c0 in range(0, count, _CHUNK):
        n = min(_CHUNK, count - c0)
        idx = torch.arange(start + c0, start + c0 + n, dtype=torch.int64, device=device)
        out[c0:c0 + n] = hash_u32(seed, tag, idx) < thresh
    return out


def f32_to_bf16_rne(x: torch.Tensor) -> torch.Tensor:
    """Round fp32 to bf16, nearest-even, in integer arithmetic (finite inputs)."""
    bits = x.contiguous().view(torch.int32).to(torch.int64) & M32
    r = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) & 0xFFFF
    r = torch.where(r >= 0x8000, r - 0x10000, r)
    return r.to(torch.int16).view(torch.bfloat16)


def uniform_u32_host(seed: int, tag: int, count: int, start: int = 0) -> np.ndarray:
    idx = torch.arange(start, start + count, dtype=torch.int64)
    return hash_u32(seed, tag, idx).numpy().astype(np.uint64)


# ---------------------------------------------------------------- lengths and blocks
def lognormal_lengths(seed: int, n: int, median: int, lo: int, hi: int, sigma: float = 1.0) -> np.ndarray:
    """Clipped log-normal lengths: clamp(rint(median * exp(sigma * z)), lo, hi)."""
    u = uniform_u32_host(seed, TAG_LENS, 2 * n).astype(np.float64)
    u1 = (u[0::2] + 0.5) / 2.0 ** 32
    u2 = (u[1::2] + 0.5) / 2.0 ** 32
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    lens = np.rint(median * np.exp(sigma * z))
    return np.clip(lens, lo, hi).astype(np.int32)


def uniform_ints(seed: int, n: int, lo: int, hi: int, tag: int = TAG_LENS) -> np.ndarray:
    """n integers uniform on {lo..hi} (inclusive)."""
    u = uniform_u32_host(seed, tag, n)
    return (lo + (u % np.uint64(hi - lo + 1))).astype(np.int32)


def shuffled_blocks(seed: int, num_blocks: int) -> np.ndarray:
    """Fisher-Yates permutation of 0..num_blocks-1."""
    perm = np.arange(num_blocks, dtype=np.int64)
    u = uniform_u32_host(seed, TAG_PERM, num_blocks)
    for i in range(num_blocks - 1, 0, -1):
        j = int(u[i] % np.uint64(i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return perm.astype(np.int32)


# ---------------------------------------------------------------- cases
@dataclass
class PagedCase:
    """One batch of paged-KV attention work.

    ``seq_lens[s]`` counts every token of sequence s after this step's write;
    ``new_lens[s]`` is how many of its last tokens are written (and queried)
    by this step: 1 for decode, the chunk length for chunked prefill.
    K/V element (s, p, h, d) has counter ((tok_base[s] + p) * Hkv + h) * D + d;
    query element (i, h, d) of sequence s has counter (r * Hq + h) * D + d with
    r = q_base[s] + i (rows are the step's new tokens in sequence order).
    """
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    in_dtype: str                 # 'f32' | 'bf16' : Q and the K/V handed to the cache write
    kv_dtype: str                 # 'f32' | 'bf16' | 'i8' : pool element type
    seq_lens: np.ndarray
    new_lens: np.ndarray
    block_tables: np.ndarray      # int32 [B][max_blocks_per_seq]
    softmax_scale: float
    window: int = 0
    partition_size: int = 512
    outliers: float = 0.0         # probability of an x8 K/V entry
    poison_block: int = -1
    kind: str = "decode"          # 'decode' | 'prefill'
    tok_base: np.ndarray | None = None   # int64 [B]: K/V counter base token of each sequence
    q_base: np.ndarray | None = None     # int64 [B]: first query row of each sequence

    def __post_init__(self):
        if self.tok_base is None:
            self.tok_base = np.concatenate([[0], np.cumsum(self.seq_lens.astype(np.int64))[:-1]]).astype(np.int64)
        if self.q_base is None:
            self.q_base = np.concatenate([[0], np.cumsum(self.new_lens.astype(np.int64))[:-1]]).astype(np.int64)

    # -- derived
    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def cu_q_lens(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.new_lens.astype(np.int64))
        return cu

    @property
    def total_q(self) -> int:
        return int(self.new_lens.astype(np.int64).sum())

    @property
    def max_q_len(self) -> int:
        return int(self.new_lens.max()) if self.num_seqs else 0

    @property
    def torch_in_dtype(self):
        return torch.float32 if self.in_dtype == "f32" else torch.bfloat16

    # -- values
    def _convert(self, x: torch.Tensor) -> torch.Tensor:
        return x if self.in_dtype == "f32" else f32_to_bf16_rne(x)

    def kv(self, which: str, s: int, p0: int, p1: int, device="cpu") -> torch.Tensor:
        """K or V of sequence s, tokens [p0, p1): [p1-p0][Hkv][D] in ``in_dtype``."""
        hd = self.num_kv_heads * self.head_dim
        n = max(p1 - p0, 0) * hd
        start = (int(self.tok_base[s]) + p0) * hd
        tag = TAG_K if which == "k" else TAG_V
        x = normal_f32(self.seed, tag, start, n, device)
        if self.outliers > 0.0:
            otag = TAG_K_OUTLIER if which == "k" else TAG_V_OUTLIER
            m = bernoulli_mask(self.seed, otag, start, n, self.outliers, device)
            x = torch.where(m, x * 8.0, x)
        return self._convert(x).view(max(p1 - p0, 0), self.num_kv_heads, self.head_dim)

    def q_rows(self, r0: int, r1: int, device="cpu") -> torch.Tensor:
        """Query rows [r0, r1) of this step: [r1-r0][Hq][D] in ``in_dtype``."""
        hd = self.num_q_heads * self.head_dim
        x = normal_f32(self.seed, TAG_Q, r0 * hd, (r1 - r0) * hd, device)
        return self._convert(x).view(r1 - r0, self.num_q_heads, self.head_dim)

    def contiguous_counters(self) -> bool:
        """True when the sequences' tokens are one run of counters (a fresh case)."""
        lens = self.seq_lens.astype(np.int64)
        return bool(np.array_equal(self.tok_base, np.concatenate([[0], np.cumsum(lens)[:-1]])))

    def all_slots(self) -> np.ndarray:
        """Slots of every token of every sequence, in counter order."""
        if self.num_seqs == 0:
            return np.zeros(0, np.int32)
        return np.concatenate([self.slots(s, 0, int(self.seq_lens[s])) for s in range(self.num_seqs)])

    def kv_tokens(self, which: str, t0: int, t1: int, device="cpu") -> torch.Tensor:
        """K or V of global tokens [t0, t1) of a case with contiguous counters
        (token t of sequence s is tok_base[s] + p): [t1-t0][Hkv][D]."""
        hd = self.num_kv_heads * self.head_dim
        n = (t1 - t0) * hd
        tag = TAG_K if which == "k" else TAG_V
        x = normal_f32(self.seed, tag, t0 * hd, n, device)
        if self.outliers > 0.0:
            otag = TAG_K_OUTLIER if which == "k" else TAG_V_OUTLIER
            m = bernoulli_mask(self.seed, otag, t0 * hd, n, self.outliers, device)
            x = torch.where(m, x * 8.0, x)
        return self._convert(x).view(t1 - t0, self.num_kv_heads, self.head_dim)

    def kv_at(self, which: str, tokens, device="cpu") -> torch.Tensor:
        """K or V of arbitrary global token counters (tok_base[s] + p): [n][Hkv][D]."""
        hd = self.num_kv_heads * self.head_dim
        t = torch.as_tensor(np.asarray(tokens, dtype=np.int64)).to(device)
        counters = (t.view(-1, 1) * hd + torch.arange(hd, dtype=torch.int64, device=device)).view(-1)
        tag = TAG_K if which == "k" else TAG_V
        x = _normal_of(self.seed, tag, counters)
        if self.outliers > 0.0:
            otag = TAG_K_OUTLIER if which == "k" else TAG_V_OUTLIER
            thresh = int(math.ceil(self.outliers * 2.0 ** 32))
            x = torch.where(hash_u32(self.seed, otag, counters) < thresh, x * 8.0, x)
        return self._convert(x).view(-1, self.num_kv_heads, self.head_dim)

    def new_tokens(self) -> np.ndarray:
        """Global token counters of this step's new tokens, in sequence order."""
        if self.num_seqs == 0:
            return np.zeros(0, np.int64)
        return np.concatenate([self.tok_base[s] + np.arange(*self.new_range(s), dtype=np.int64)
                               for s in range(self.num_seqs)])

    def new_slots(self) -> np.ndarray:
        if self.num_seqs == 0:
            return np.zeros(0, np.int32)
        return np.concatenate([self.slots(s, *self.new_range(s)) for s in range(self.num_seqs)])

    def q(self, device="cpu") -> torch.Tensor:
        """All query rows of this step, in sequence order: [total_q][Hq][D]."""
        qb = self.q_base
        if self.num_seqs and np.array_equal(qb, np.concatenate([[0], np.cumsum(self.new_lens.astype(np.int64))[:-1]])):
            return self.q_rows(0, self.total_q, device)
        return torch.cat([self.q_seq(s, device) for s in range(self.num_seqs)]) if self.num_seqs \
            else self.q_rows(0, 0, device)

    def q_seq(self, s: int, device="cpu") -> torch.Tensor:
        """Query rows of sequence s: [new_lens[s]][Hq][D]."""
        r0 = int(self.q_base[s])
        return self.q_rows(r0, r0 + int(self.new_lens[s]), device)

    # -- addressing of the inputs (slot = physical block * block_size + offset)
    def slots(self, s: int, p0: int, p1: int) -> np.ndarray:
        p = np.arange(p0, p1, dtype=np.int64)
        blk = self.block_tables[s, p // self.block_size].astype(np.int64)
        return (blk * self.block_size + p % self.block_size).astype(np.int32)

    def context_range(self, s: int) -> tuple[int, int]:
        """Tokens already in the cache before this step."""
        return 0, int(self.seq_lens[s] - self.new_lens[s])

    def new_range(self, s: int) -> tuple[int, int]:
        """Tokens written by this step."""
        return int(self.seq_lens[s] - self.new_lens[s]), int(self.seq_lens[s])

    def subset(self, seqs) -> "PagedCase":
        """The same work restricted to some sequences, with a compact pool.

        Values are unchanged (counter bases are kept); each kept sequence gets
        consecutive physical blocks in a new pool, plus one trailing poison
        block that the unused table entries point at."""
        seqs = [int(s) for s in seqs]
        bs = self.block_size
        nblk = [-(-int(self.seq_lens[s]) // bs) for s in seqs]
        need = sum(nblk)
        tables = np.full((len(seqs), max([1] + nblk)), need, dtype=np.int32)
        base = 0
        for i, n in enumerate(nblk):
            tables[i, :n] = np.arange(base, base + n, dtype=np.int32)
            base += n
        return PagedCase(
            name=f"{self.name}[{len(seqs)} seqs]", seed=self.seed, num_q_heads=self.num_q_heads,
            num_kv_heads=self.num_kv_heads, head_dim=self.head_dim, block_size=bs,
            num_blocks=need + 1, in_dtype=self.in_dtype, kv_dtype=self.kv_dtype,
            seq_lens=self.seq_lens[seqs].copy(), new_lens=self.new_lens[seqs].copy(),
            block_tables=tables, softmax_scale=self.softmax_scale, window=self.window,
            partition_size=self.partition_size, outliers=self.outliers, poison_block=need,
            kind=self.kind, tok_base=self.tok_base[seqs].copy(), q_base=self.q_base[seqs].copy())


def _assign(seed: int, seq_lens: np.ndarray, block_size: int, num_blocks: int, max_blocks: int):
    nblk = -(-seq_lens.astype(np.int64) // block_size)
    need = int(nblk.sum())
    if num_blocks < need + 1:
        raise ValueError("pool must hold every sequence's blocks plus one spare block")
    perm = shuffled_blocks(seed, num_blocks)
    poison = int(perm[need])
    tables = np.full((len(seq_lens), max_blocks), poison, dtype=np.int32)
    off = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = perm[off:off + n]
        off += int(n)
    return tables, poison


def make_case(name: str, seed: int, seq_lens, new_lens, num_q_heads: int, num_kv_heads: int,
              head_dim: int, in_dtype: str = "bf16", kv_dtype: str | None = None,
              block_size: int = 16, num_blocks: int | None = None, max_blocks: int | None = None,
              softmax_scale: float | None = None, window: int = 0, partition_size: int = 512,
              outliers: float = 0.0, kind: str = "decode") -> PagedCase:
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    new_lens = np.asarray(new_lens, dtype=np.int32)
    nblk = -(-seq_lens.astype(np.int64) // block_size)
    need = int(nblk.sum())
    if num_blocks is None:
        num_blocks = max(int(math.ceil(1.2 * need)), need + 1)
    if max_blocks is None:
        max_blocks = max(1, int(nblk.max()) if len(nblk) else 1)
    if softmax_scale is None:
        softmax_scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    tables, poison = _assign(seed, seq_lens, block_size, num_blocks, max_blocks)
    return PagedCase(name=name, seed=seed, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                     head_dim=head_dim, block_size=block_size, num_blocks=num_blocks,
                     in_dtype=in_dtype, kv_dtype=kv_dtype or in_dtype, seq_lens=seq_lens,
                     new_lens=new_lens, block_tables=tables, softmax_scale=softmax_scale,
                     window=window, partition_size=partition_size, outliers=outliers,
                     poison_block=poison, kind=kind)


# ---------------------------------------------------------------- the five workloads
def tiny_fp32_decode() -> PagedCase:
    """fp32 decode: 4 sequences of 7/16/33/50 tokens, 4 q heads on 2 kv heads,
    head_dim 64, a 32-block pool assigned by a seeded permutation."""
    lens = np.array([7, 16, 33, 50], dtype=np.int32)
    return make_case("tiny-fp32-decode", 1, lens, np.ones(4, np.int32), 4, 2, 64,
                     in_dtype="f32", num_blocks=32, max_blocks=4, softmax_scale=0.125)


def qwen_decode(batch: int = 8, seed: int = 2, kv_dtype: str = "bf16", outliers: float = 0.0,
                name: str = "qwen2.5-1.5b-decode") -> PagedCase:
    """Qwen2.5-1.5B-shaped decode: 12 q / 2 kv heads, head_dim 128, lengths
    clipped log-normal (median 512, 64..4096)."""
    lens = lognormal_lengths(seed, batch, 512, 64, 4096)
    return make_case(name, seed, lens, np.ones(batch, np.int32), 12, 2, 128,
                     kv_dtype=kv_dtype, max_blocks=4096 // 16, outliers=outliers)


def llama_decode(batch: int = 256, seed: int = 3) -> PagedCase:
    """Llama-3-8B-shaped large-batch decode: 32 q / 8 kv heads, head_dim 128,
    lengths clipped log-normal (median 2048, 128..32768), pool 1.2x the need,
    split over 512-token partitions."""
    lens = lognormal_lengths(seed, batch, 2048, 128, 32768)
    return make_case("llama3-8b-decode", seed, lens, np.ones(batch, np.int32), 32, 8, 128,
                     max_blocks=32768 // 16, partition_size=512)


def int8_decode() -> PagedCase:
    """INT8-KV decode: the Qwen2.5-1.5B shapes at batch 64, K/V with 1% of
    entries scaled x8, written through the quantising cache write."""
    return qwen_decode(batch=64, seed=4, kv_dtype="i8", outliers=0.01, name="int8-kv-decode")


def prefill_window(num_seqs: int = 16, chunk: int = 256, seed: int = 5) -> PagedCase:
    """Chunked prefill with a sliding window: 16 sequences each appending a
    256-token chunk to a paged context of 1024..16384 tokens (uniform),
    32 q / 8 kv heads, head_dim 128, causal mask plus a 4096-token window."""
    ctx = uniform_ints(seed, num_seqs, 1024, 16384)
    lens = ctx + chunk
    return make_case("prefill-window", seed, lens, np.full(num_seqs, chunk, np.int32), 32, 8, 128,
                     max_blocks=(16384 + chunk) // 16, window=4096, kind="prefill")


def mixed_step(num_prefill: int = 16, chunk: int = 256, num_decode: int = 240, seed: int = 6) -> PagedCase:
    """One serving step that mixes chunked prefill with decode: 16 sequences
    appending a 256-token chunk to contexts of 1024..16384 tokens (uniform) and
    240 sequences decoding one token after clipped log-normal contexts (median
    2048, 128..32768), 32 q / 8 kv heads, head_dim 128, window 4096."""
    ctx = uniform_ints(seed, num_prefill, 1024, 16384)
    dec = lognormal_lengths(seed + 100, num_decode, 2048, 128, 32768)
    lens = np.concatenate([ctx + chunk, dec]).astype(np.int32)
    new = np.concatenate([np.full(num_prefill, chunk, np.int32), np.ones(num_decode, np.int32)])
    return make_case("mixed-step", seed, lens, new, 32, 8, 128, max_blocks=32768 // 16, window=4096,
                     kind="prefill")


WORKLOADS = {
    "tiny-fp32-decode": tiny_fp32_decode,
    "qwen2.5-1.5b-decode": qwen_decode,
    "llama3-8b-decode": llama_decode,
    "int8-kv-decode": int8_decode,
    "prefill-window": prefill_window,
    "mixed-step": mixed_step,
}


# ---------------------------------------------------------------- explicit and planted inputs
class ExplicitCase(PagedCase):
    """A PagedCase whose K, V and Q values are given as tensors instead of being
    generated from the seed: ``K``, ``V`` are fp32 [num_counter_tokens][Hkv][D]
    indexed by global token counter (tok_base[s] + p) and ``Q`` is fp32
    [total_q][Hq][D]; each is rounded to ``in_dtype`` when handed out.  Tables,
    lengths and pool come from the wrapped case."""

    K: torch.Tensor = None
    V: torch.Tensor = None
    Q: torch.Tensor = None

    @classmethod
    def wrap(cls, case: PagedCase, K: torch.Tensor, V: torch.Tensor, Q: torch.Tensor) -> "ExplicitCase":
        fields = {f: getattr(case, f) for f in case.__dataclass_fields__}
        out = cls(**fields)
        out.K, out.V, out.Q = K.float().contiguous(), V.float().contiguous(), Q.float().contiguous()
        return out

    def _pick(self, which):
        return self.K if which == "k" else self.V

    def kv(self, which, s, p0, p1, device="cpu"):
        t0 = int(self.tok_base[s]) + p0
        return self._convert(self._pick(which)[t0:t0 + max(p1 - p0, 0)].clone()).to(device)

    def kv_tokens(self, which, t0, t1, device="cpu"):
        return self._convert(self._pick(which)[t0:t1].clone()).to(device)

    def kv_at(self, which, tokens, device="cpu"):
        idx = torch.as_tensor(np.asarray(tokens, dtype=np.int64))
        return self._convert(self._pick(which)[idx].clone()).to(device)

    def q_rows(self, r0, r1, device="cpu"):
        return self._convert(self.Q[r0:r1].clone()).to(device)

    def subset(self, seqs) -> "ExplicitCase":
        return ExplicitCase.wrap(super().subset(seqs), self.K, self.V, self.Q)


def rising_scores(case: PagedCase, jump_log2: float = 12.0, stair: int = 128, c: float = 4.0,
                  period: int = 0, seed_tag: int = TAG_MISC) -> ExplicitCase:
    """Inputs whose attention scores rise along the context in steps.

    For every (sequence, KV head) a unit direction u is drawn.  Each query row
    of that head group becomes its generated value with the component along u
    replaced by c * u, and each key at position j becomes its generated value
    with the component along u replaced by r_j * u, where
        r_j = jump_log2 * n_j / (c * softmax_scale * log2(e)),
        n_j = floor(j / stair)  (or floor(j / stair) mod period, period > 0).
    So every query of the group sees scores (in log2 units, softmax scale and
    log2 e applied) equal to its random part plus jump_log2 * n_j: each step
    of keys outscores everything before it (in its period) by jump_log2, and
    an online softmax that meets the steps in order must rescale what it has
    accumulated.  A period keeps the scores' range bounded over long contexts
    (fp32 rounding of a score grows with its size).  V keeps its generated
    values.  The result is an ExplicitCase with the same tables, lengths and
    pool."""
    hkv, hq, d = case.num_kv_heads, case.num_q_heads, case.head_dim
    G = hq // hkv
    ntok = int(case.tok_base[-1] + case.seq_lens[-1]) if case.num_seqs else 0
    K = normal_f32(case.seed, TAG_K, 0, ntok * hkv * d).view(ntok, hkv, d)
    V = normal_f32(case.seed, TAG_V, 0, ntok * hkv * d).view(ntok, hkv, d)
    Q = normal_f32(case.seed, TAG_Q, 0, case.total_q * hq * d).view(case.total_q, hq, d)
    K, Q = K.double(), Q.double()
    dirs = normal_f32(case.seed, seed_tag, 0, case.num_seqs * hkv * d).view(case.num_seqs, hkv, d).double()
    dirs = dirs / dirs.norm(dim=-1, keepdim=True)
    unit = float(case.softmax_scale) * math.log2(math.e)
    for s in range(case.num_seqs):
        L = int(case.seq_lens[s])
        t0 = int(case.tok_base[s])
        r0, r1 = int(case.q_base[s]), int(case.q_base[s]) + int(case.new_lens[s])
        steps = torch.div(torch.arange(L, dtype=torch.float64), stair, rounding_mode="floor")
        if period > 0:
            steps = torch.remainder(steps, period)
        r = jump_log2 * steps / (c * unit)
        for g in range(hkv):
            u = dirs[s, g]
            ks = K[t0:t0 + L, g]
            K[t0:t0 + L, g] = ks - (ks @ u)[:, None] * u[None, :] + r[:, None] * u[None, :]
            qs = Q[r0:r1, g * G:(g + 1) * G]
            Q[r0:r1, g * G:(g + 1) * G] = qs - (qs @ u)[..., None] * u + c * u
    return ExplicitCase.wrap(case, K.float(), V, Q.float())
