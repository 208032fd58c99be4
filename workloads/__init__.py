"""Seeded synthetic inputs for paged KV-cache attention.

This module only draws random inputs and lays them out: sequence lengths,
a random assignment of physical pages to each sequence's logical pages
(the block tables), and bf16 K/V/q values.  It holds no attention or
addressing arithmetic, so both the oracle side and the HIP side can use it
without sharing any of the computation under test.

Recipe (every draw is seeded; see ``Workload``):

* lengths and the page permutation come from ``numpy.random.default_rng(seed)``,
  in that order (decode sequences first, then prefill sequences);
* the K and V values of sequence ``s`` come from their own stream,
  ``default_rng([seed, 1, s])``: K of shape ``[L_s, Hkv, D]`` first, then V;
* the query values of layer ``j`` come from ``default_rng([seed, 2, j])``:
  the decode rows ``[n_decode, Hq, D]`` first, then the packed prefill rows
  ``[Tq, Hq, D]``;
* every value is a float32 standard normal rounded to bf16 with
  round-to-nearest-even and stored as its 16-bit pattern (``uint16``).

Per-sequence streams let a test regenerate only the sequences it samples,
which keeps full-size checks cheap.

"Uniform in [a, b]" means integers with both ends included.  "Context
length" is the number of tokens already cached before the step; a decoding
sequence appends one token in the step.  The configurations are the
workloads the rollout-engine pages benchmark: a Qwen3-4B head shape
(32 query heads, 8 KV heads, head_dim 128), a Gemma-4 sliding-window shape
(8/1/256, window 512, a second layer sharing the pool) and a tiny case.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

__all__ = [
    "BF16_NAN",
    "CONFIGS",
    "Workload",
    "bf16_bits",
    "bf16_to_f32",
    "make",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass
class Workload:
    """One synthetic paged-attention step.

    Sequences ``0 .. n_decode-1`` decode one token; sequences
    ``n_decode .. n_decode+n_prefill-1`` run a (possibly chunked) prefill.
    Sequence ``s`` holds ``prefix_lens[s]`` cached tokens before the step
    and appends ``new_lens[s]`` tokens in it.
    """

    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    window: int
    num_layers: int
    n_decode: int
    n_prefill: int
    prefix_lens: np.ndarray          # int64 [S]
    new_lens: np.ndarray             # int64 [S]
    num_pages: int
    block_tables: np.ndarray         # int32 [S, max_pages]; padding entries = pad_page
    pad_page: int                    # a physical page no sequence uses
    _kv_cache: dict = field(default_factory=dict, repr=False)

    # ---- shapes -------------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return self.n_decode + self.n_prefill

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))

    @property
    def total_lens(self) -> np.ndarray:
        return self.prefix_lens + self.new_lens

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size

    @property
    def max_seq_len(self) -> int:
        return int(self.total_lens.max()) if self.num_seqs else 0

    def decode_ids(self) -> np.ndarray:
        return np.arange(self.n_decode)

    def prefill_ids(self) -> np.ndarray:
        return np.arange(self.n_decode, self.num_seqs)

    def decode_seq_lens(self) -> np.ndarray:
        """KV length of each decoding sequence after this step's append (int32)."""
        return self.total_lens[: self.n_decode].astype(np.int32)

    def cu_lens(self, lens: np.ndarray) -> np.ndarray:
        out = np.zeros(len(lens) + 1, dtype=np.int32)
        out[1:] = np.cumsum(lens)
        return out

    def prefill_cu_q(self) -> np.ndarray:
        return self.cu_lens(self.new_lens[self.n_decode:])

    def prefill_cu_k(self) -> np.ndarray:
        return self.cu_lens(self.total_lens[self.n_decode:])

    def total_q(self) -> int:
        return int(self.new_lens[self.n_decode:].sum())

    # ---- values -------------------------------------------------------
    def kv_seq(self, s: int):
        """K and V of every token of sequence ``s``: two uint16 ``[L_s, Hkv, D]``."""
        hit = self._kv_cache.get(s)
        if hit is not None:
            return hit
        rng = np.random.default_rng([self.seed, 1, int(s)])
        shape = (int(self.total_lens[s]), self.num_kv_heads, self.head_dim)
        k = _normal_bf16(rng, shape)
        v = _normal_bf16(rng, shape)
        return k, v

    def cache_all_kv(self, seqs=None) -> None:
        """Generate (in threads) and keep the K/V of ``seqs`` (default: all)."""
        seqs = list(range(self.num_seqs)) if seqs is None else list(seqs)
        todo = [s for s in seqs if s not in self._kv_cache]
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            for s, kv in zip(todo, ex.map(self.kv_seq, todo)):
                self._kv_cache[s] = kv

    def drop_kv(self) -> None:
        self._kv_cache.clear()

    def queries(self, layer: int = 0):
        """(q_decode ``[n_decode, Hq, D]``, q_prefill ``[Tq, Hq, D]``) as uint16."""
        rng = np.random.default_rng([self.seed, 2, int(layer)])
        qd = _normal_bf16(rng, (self.n_decode, self.num_q_heads, self.head_dim))
        qp = _normal_bf16(rng, (self.total_q(), self.num_q_heads, self.head_dim))
        return qd, qp

    def packed_tokens(self, part: str, seqs=None):
        """Pack K/V of the ``part`` tokens ("prefix" or "new") of ``seqs``.

        Returns ``(k [T, Hkv, D], v [T, Hkv, D], lens_q, lens_k)`` where the
        tokens of each sequence are consecutive, ``lens_q`` is how many
        tokens each sequence contributes and ``lens_k`` its KV length once
        they are in the cache.
        """
        seqs = np.arange(self.num_seqs) if seqs is None else np.asarray(seqs)
        ks, vs, lq, lk = [], [], [], []
        for s in seqs:
            k, v = self.kv_seq(int(s))
            p, n = int(self.prefix_lens[s]), int(self.new_lens[s])
            if part == "prefix":
                ks.append(k[:p]); vs.append(v[:p]); lq.append(p); lk.append(p)
            elif part == "new":
                ks.append(k[p:p + n]); vs.append(v[p:p + n]); lq.append(n); lk.append(p + n)
            else:
                raise ValueError(part)
        shape = (0, self.num_kv_heads, self.head_dim)
        k = np.concatenate(ks) if ks else np.zeros(shape, np.uint16)
        v = np.concatenate(vs) if vs else np.zeros(shape, np.uint16)
        return k, v, np.asarray(lq, np.int64), np.asarray(lk, np.int64)


# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    window: int = 0
    num_layers: int = 1
    decode_ctx: tuple | None = None      # ("fixed", values) or ("uniform", n, lo, hi)
    prefill_new: tuple | None = None     # ("uniform", n, lo, hi): fresh prompts
    chunk: tuple | None = None           # ("uniform", n, lo, hi, chunk): cached prefix + chunk
    pool_pages: int | None = None        # stated pool size, else used + spare
    spare_pages: int = 16


CONFIGS = {
    # 4 sequences, contexts {5,17,32,63}, 2/1/64, page 16, a 32-page pool.
    "tiny_decode": Config("tiny_decode", 20260001, 2, 1, 64, 16,
                          decode_ctx=("fixed", (5, 17, 32, 63)), pool_pages=32),
    # 32 sequences, context U[128,1024], Qwen3-4B heads, page 32.
    "qwen3_decode": Config("qwen3_decode", 20260002, 32, 8, 128, 32,
                           decode_ctx=("uniform", 32, 128, 1024)),
    # 8 fresh prompts U[64,256] + 56 decoders with context U[256,2048].
    "mixed_step": Config("mixed_step", 20260003, 32, 8, 128, 32,
                         decode_ctx=("uniform", 56, 256, 2048),
                         prefill_new=("uniform", 8, 64, 256)),
    # 256 sequences, context U[1024,8192]: the bandwidth-bound decode.
    "large_decode": Config("large_decode", 20260004, 32, 8, 128, 32,
                           decode_ctx=("uniform", 256, 1024, 8192)),
    # Gemma-4 sliding regime: 64 decoders + 4 sequences with a cached prefix
    # U[512,4096] and a 128-token chunk; window 512; two layers, shared pool.
    "window_shared": Config("window_shared", 20260005, 8, 1, 256, 32, window=512,
                            num_layers=2, decode_ctx=("uniform", 64, 512, 4096),
                            chunk=("uniform", 4, 512, 4096, 128)),
    # 16 fresh prompts U[1024,4096] with the Qwen3-4B heads: a prefill large
    # enough that the matrix cores, not launch latency, bound it.
    "long_prefill": Config("long_prefill", 20260006, 32, 8, 128, 32,
                           prefill_new=("uniform", 16, 1024, 4096)),
    # the same model's full-attention layers: head_dim 512, no window; the
    # 64 decoders of the windowed case, and 8 prompts for the prefill side
    "full512_decode": Config("full512_decode", 20260007, 8, 1, 512, 32,
                             decode_ctx=("uniform", 64, 512, 4096)),
    "full512_prefill": Config("full512_prefill", 20260008, 8, 1, 512, 32,
                              prefill_new=("uniform", 8, 1024, 4096)),
}


def _draw_lengths(rng, spec):
    if spec is None:
        return np.zeros(0, np.int64)
    if spec[0] == "fixed":
        return np.asarray(spec[1], np.int64)
    _, n, lo, hi = spec[:4]
    return rng.integers(lo, hi, size=n, endpoint=True).astype(np.int64)


def build(cfg: Config, *, seed: int | None = None, decode_ctx=None, prefill_new=None,
          chunk=None, name: str | None = None) -> Workload:
    """Draw the lengths and block tables of ``cfg`` (values are drawn lazily)."""
    seed = cfg.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    dctx = _draw_lengths(rng, cfg.decode_ctx if decode_ctx is None else decode_ctx)
    pnew = _draw_lengths(rng, cfg.prefill_new if prefill_new is None else prefill_new)
    chunk = cfg.chunk if chunk is None else chunk
    cpre = _draw_lengths(rng, chunk)
    clen = np.full(len(cpre), chunk[4] if chunk else 0, np.int64)

    prefix = np.concatenate([dctx, np.zeros(len(pnew), np.int64), cpre])
    new = np.concatenate([np.ones(len(dctx), np.int64), pnew, clen])
    total = prefix + new
    ps = cfg.page_size
    npages_seq = (total + ps - 1) // ps
    used = int(npages_seq.sum())
    num_pages = cfg.pool_pages if cfg.pool_pages is not None else used + cfg.spare_pages
    if num_pages <= used:
        raise ValueError("pool too small for the drawn lengths")
    perm = rng.permutation(num_pages).astype(np.int32)
    pad_page = int(perm[used])
    max_pages = max(1, int(npages_seq.max()) if len(npages_seq) else 1)
    bt = np.full((len(total), max_pages), pad_page, np.int32)
    off = 0
    for s, n in enumerate(npages_seq):
        bt[s, :n] = perm[off:off + n]
        off += int(n)
    return Workload(name or cfg.name, seed, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                    ps, cfg.window, cfg.num_layers, len(dctx), len(pnew) + len(cpre),
                    prefix, new, int(num_pages), bt, pad_page)


def make(config: str, **kw) -> Workload:
    return build(CONFIGS[config], **kw)
