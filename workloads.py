"""Seeded synthetic packed batches shared by the tests, the bench and the smoke check.

This module only draws inputs: document lengths, their alignment padding, empty
padding slots, token ids and row payloads.  It holds no step of the layout
transform itself, so both the CPU oracle and the HIP library can be fed from it
without sharing any of the method.

Recipes (base seed 1234, the seed of the Relax PR #273 training harness, §3/§4):

* ``tiny``      cp 2, lengths [8, 12, 4] (real = padded), rows [T, 2, 8] bf16,
                ids in [0, 32000), label shift only.
* ``gdn128k``   cp 4, T = 131072, real lengths log-uniform in 256..32768, each
                padded to a multiple of 8, rows [T, 16, 128] bf16.
* ``sft``       cp 8, T = 131072, real lengths uniform in 64..1024, each padded
                to a multiple of 16, plus 8 empty slots (repeated boundaries) at
                seeded places, one of them trailing, rows [T, 4096] bf16.
* ``sft512``    as ``sft`` but with exactly 512 documents (lengths uniform in
                64..448, rescaled to fill T in multiples of 16): the
                "about 512 documents" reading, used for route-build latency.
* ``long1m``    cp 4, T = 1048576 from 6 lengths uniform in 65536..409600,
                rescaled to T in multiples of 8, rows [T, 32, 128] bf16.
* ``full``      cp 16 (tp 2 only enters the alignment), T = 262144, real
                lengths log-uniform in 128..65536, each padded to a multiple of
                tp*cp*16 = 512, rows [T, 2048] bf16, ids, 48 layers x 2 swaps,
                label shift plus MTP depths 1..3.

Fill rule for a fixed T: draw a real length, pad it up to the alignment; when
the padded length would reach or pass the room left, the last document takes
all of the remaining room as its padded length (its real length is capped at
that room).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 1234
VOCAB = 32000
K = 1024


def pad_to_multiple(lengths, align: int) -> np.ndarray:
    """Pad every length up to the next multiple of ``align`` (0 stays 0).

    The per-sub-sequence alignment padding of "Packed Sequence 与上下文并行"
    §2.2 (``pad = (-len) mod align``).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    return lengths + (-lengths) % align


def cumulative(lengths) -> np.ndarray:
    """Boundary list ``[0, l0, l0 + l1, ...]`` as int32."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    assert out[-1] <= np.iinfo(np.int32).max
    return out.astype(np.int32)


@dataclass
class Workload:
    name: str
    index: int
    cp: int
    cu_padded: np.ndarray           # int32 [n_slots + 1]
    cu_real: np.ndarray             # int32 [n_slots + 1]
    row_shape: tuple                # shape of one row
    row_dtype: str = "bfloat16"
    max_shift: int = 0              # 0: no roll in this workload
    layers: int = 1                 # each layer does one z->c and one c->z swap
    notes: dict = field(default_factory=dict)
    seed_extra: tuple = ()

    @property
    def total(self) -> int:
        return int(self.cu_padded[-1])

    @property
    def n_slots(self) -> int:
        return int(len(self.cu_padded) - 1)

    @property
    def row_elems(self) -> int:
        return int(math.prod(self.row_shape))

    @property
    def row_bytes(self) -> int:
        return self.row_elems * np.dtype(_np_dtype(self.row_dtype)).itemsize

    def rng(self, stream: int) -> np.random.Generator:
        return np.random.default_rng([BASE_SEED, self.index, *self.seed_extra, stream])

    def ids(self) -> np.ndarray:
        """int64 token ids, uniform in [0, 32000)."""
        return self.rng(2).integers(0, VOCAB, size=self.total, dtype=np.int64)

    def rows_host(self) -> np.ndarray:
        """Row payload on the host: bf16 bit patterns (uint16) of N(0, 1) draws."""
        return random_rows(self.rng(3), self.total, self.row_shape, self.row_dtype)


def _np_dtype(name: str):
    return {"bfloat16": np.uint16, "float16": np.uint16, "float32": np.float32,
            "uint8": np.uint8, "int64": np.int64, "int32": np.int32}[name]


def random_rows(rng: np.random.Generator, total: int, row_shape, row_dtype="bfloat16") -> np.ndarray:
    """Seeded payload rows.  bf16 is returned as its uint16 bit pattern
    (N(0, 1) draws rounded to nearest even)."""
    shape = (total,) + tuple(row_shape)
    if row_dtype in ("bfloat16",):
        f = rng.standard_normal(shape, dtype=np.float32)
        bits = f.view(np.uint32)
        rounded = bits + 0x7FFF + ((bits >> 16) & 1)
        return (rounded >> 16).astype(np.uint16)
    if row_dtype == "float32":
        return rng.standard_normal(shape, dtype=np.float32)
    info = np.iinfo(_np_dtype(row_dtype))
    return rng.integers(info.min, info.max, size=shape, dtype=_np_dtype(row_dtype), endpoint=True)


def stamp_rows(rows_u8: np.ndarray) -> np.ndarray:
    """Diagnostic variant: write each row's index into its first 8 bytes."""
    t = rows_u8.shape[0]
    flat = rows_u8.reshape(t, -1).view(np.uint8)
    assert flat.shape[1] >= 8
    flat[:, :8] = np.arange(t, dtype=np.int64).view(np.uint8).reshape(t, 8)
    return rows_u8


def _fill_fixed_total(total: int, align: int, draw) -> tuple[list[int], list[int]]:
    real, padded = [], []
    room = total
    while room > 0:
        d = int(draw())
        p = int(pad_to_multiple([d], align)[0])
        if p >= room:
            padded.append(room)
            real.append(min(d, room))
            room = 0
        else:
            padded.append(p)
            real.append(d)
            room -= p
    return real, padded


def _log_uniform(rng: np.random.Generator, lo: int, hi: int):
    return lambda: int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))


def _insert_empty_slots(real, padded, n_empty: int, rng: np.random.Generator):
    """Insert ``n_empty`` zero-length slots: one at the end, the rest at seeded
    positions (possibly the front, possibly next to each other)."""
    real, padded = list(real), list(padded)
    positions = sorted(int(x) for x in rng.integers(0, len(real) + 1, size=n_empty - 1))
    for pos in reversed(positions):
        real.insert(pos, 0)
        padded.insert(pos, 0)
    real.append(0)
    padded.append(0)
    return real, padded


def _rescale(draws, total: int, align: int) -> list[int]:
    draws = np.asarray(draws, dtype=np.float64)
    scaled = draws * total / draws.sum()
    out = [int(x // align) * align for x in scaled[:-1]]
    out.append(total - sum(out))
    assert out[-1] > 0 and out[-1] % align == 0
    return out


def make(name: str) -> Workload:
    """Build one of the named workloads (see the module docstring)."""
    if name == "tiny":
        lens = [8, 12, 4]
        return Workload("tiny", 0, 2, cumulative(lens), cumulative(lens), (2, 8),
                        max_shift=1, layers=1)
    if name == "gdn128k":
        rng = np.random.default_rng([BASE_SEED, 1, 0])
        real, padded = _fill_fixed_total(128 * K, 8, _log_uniform(rng, 256, 32 * K))
        return Workload("gdn128k", 1, 4, cumulative(padded), cumulative(real), (16, 128),
                        max_shift=1, layers=1)
    if name == "sft":
        rng = np.random.default_rng([BASE_SEED, 2, 0])
        real, padded = _fill_fixed_total(128 * K, 16, lambda: rng.integers(64, 1024, endpoint=True))
        real, padded = _insert_empty_slots(real, padded, 8, np.random.default_rng([BASE_SEED, 2, 1]))
        return Workload("sft", 2, 8, cumulative(padded), cumulative(real), (4096,),
                        max_shift=1, layers=1)
    if name == "sft512":
        rng = np.random.default_rng([BASE_SEED, 2, 4])
        padded = _rescale(rng.integers(64, 448, size=512, endpoint=True), 128 * K, 16)
        real, padded = _insert_empty_slots(padded, padded, 8, np.random.default_rng([BASE_SEED, 2, 5]))
        return Workload("sft512", 2, 8, cumulative(padded), cumulative(real), (4096,),
                        max_shift=1, layers=1)
    if name == "long1m":
        rng = np.random.default_rng([BASE_SEED, 3, 0])
        padded = _rescale(rng.integers(64 * K, 400 * K, size=6, endpoint=True), 1024 * K, 8)
        return Workload("long1m", 3, 4, cumulative(padded), cumulative(padded), (32, 128),
                        max_shift=1, layers=1)
    if name == "full":
        rng = np.random.default_rng([BASE_SEED, 4, 0])
        real, padded = _fill_fixed_total(256 * K, 2 * 16 * 16, _log_uniform(rng, 128, 64 * K))
        return Workload("full", 4, 16, cumulative(padded), cumulative(real), (2048,),
                        max_shift=4, layers=48, notes={"tp": 2, "mtp_depths": 3})
    raise KeyError(name)


NAMES = ("tiny", "gdn128k", "sft", "long1m", "full")


def random_packed(seed, cp: int, n_docs: int, max_chunk: int, n_empty: int = 0,
                  pad_max: int = 0, row_shape=(8,), row_dtype="bfloat16") -> Workload:
    """Small ragged batch for parity tests: ``n_docs`` documents whose padded
    lengths are 2*cp times a chunk in 1..max_chunk, real lengths up to
    ``pad_max`` tokens shorter, and ``n_empty`` empty slots anywhere."""
    rng = np.random.default_rng([BASE_SEED, 100, *np.atleast_1d(seed).tolist()])
    padded = [2 * cp * int(rng.integers(1, max_chunk, endpoint=True)) for _ in range(n_docs)]
    real = [max(0, p - int(rng.integers(0, pad_max, endpoint=True))) if pad_max else p for p in padded]
    if n_empty:
        pos = sorted(int(x) for x in rng.integers(0, len(padded) + 1, size=n_empty))
        for p in reversed(pos):
            padded.insert(p, 0)
            real.insert(p, 0)
    return Workload(f"random{seed}", 100, cp, cumulative(padded), cumulative(real), tuple(row_shape),
                    row_dtype=row_dtype, max_shift=1,
                    seed_extra=tuple(np.atleast_1d(seed).tolist()))


def token_rows(seed, batch: int, seq: int, pad_id: int = 0, eod_id: int = 1, eod_rate: float = 0.01,
               pad_tail_max: int | None = None, inner_pad_rate: float = 0.0) -> np.ndarray:
    """Seeded [batch, seq] int64 token rows for packing tests: ids drawn from
    [2, 32000), EOD tokens at rate ``eod_rate``, a PAD tail of up to
    ``pad_tail_max`` tokens per row (whole rows of PAD possible), and PAD
    tokens inside the valid part at rate ``inner_pad_rate``."""
    rng = np.random.default_rng([BASE_SEED, 200, *np.atleast_1d(seed).tolist()])
    rows = rng.integers(2, VOCAB, size=(batch, seq), dtype=np.int64)
    rows[rng.random((batch, seq)) < eod_rate] = eod_id
    if inner_pad_rate:
        rows[rng.random((batch, seq)) < inner_pad_rate] = pad_id
    tail_max = seq if pad_tail_max is None else pad_tail_max
    for b in range(batch):
        tail = int(rng.integers(0, tail_max, endpoint=True))
        if tail:
            rows[b, seq - tail:] = pad_id
    return rows
