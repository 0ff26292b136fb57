"""Per-token CPU definition of the THD zigzag <-> contiguous layout transform.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may call it).

Sources, cited by page title and section:

* Relax PR #273 "[Task32] feat: fla mcore chunkwise cp stage 3" (github
  redai-infra/Relax): §1 (the per-token index route of the first stage and its
  validation), §2.1 (both layouts are unions of global token intervals; the
  route is send rows / receive rows / split sizes), §2.2 (repeated boundaries
  are empty padding slots; identity is a zero-copy special case), §2.6 (cp=1
  short-circuits the swap), §5 (fail-fast cases; all ranks emulated locally).
* "Packed Sequence 与上下文并行" (lizn-zn scholia-log, training-infra):
  §1.3 and §1.6 (labels and MTP targets must not cross a document), §2.2
  (padding per sub-sequence; valid-token mask is zero at pads), §2.4 (ring
  zigzag slice: 2*cp chunks per sequence, rank r takes chunks r and
  2*cp-1-r), §2.5 (Ulysses contiguous slice), §3 (worked example).

Everything here is integer index work; rows are moved as raw bytes, never as
floating point values.
"""

from __future__ import annotations

import numpy as np

ZIGZAG = "zigzag"
CONTIGUOUS = "contiguous"


class OracleInputError(ValueError):
    """Malformed boundaries.  ``kind`` names which rule failed.

    Kinds, in the order they are checked (the first failing rule wins):
    ``CU_START``, ``CU_MONOTONE``, ``CU_TOTAL``, ``CU_DIVISIBLE`` for the route,
    and ``CU_START``, ``CU_MONOTONE``, ``CU_TOTAL``, ``REAL_GT_PADDED`` for the
    label roll.  ``ARG`` covers arguments that are not boundary data.
    """

    def __init__(self, kind: str, detail: str):
        super().__init__(f"{kind}: {detail}")
        self.kind = kind


def _as_int_list(cu) -> list[int]:
    return [int(v) for v in np.asarray(cu).reshape(-1).tolist()]


# ---------------------------------------------------------------------------
# Validation (Relax PR #273, §5 fail-fast list; §1 the first stage's checks of
# cu[0] and cu[-1]; "Packed Sequence 与上下文并行" §1.7 divisibility by 2*cp and
# the b*s == cu_seqlens_padded[-1] total check).
# ---------------------------------------------------------------------------

def check_route_boundaries(cu, cp: int, total: int) -> list[int]:
    """Raise OracleInputError unless ``cu`` is a valid padded boundary list.

    Rules, each checked over every slot before the next rule is looked at:
    the first boundary is 0; boundaries never decrease; the last boundary is
    the total token count; every slot length is a multiple of 2*cp.
    """
    if cp < 1:
        raise OracleInputError("ARG", f"cp_size must be >= 1, got {cp}")
    if total < 0:
        raise OracleInputError("ARG", f"total tokens must be >= 0, got {total}")
    b = _as_int_list(cu)
    if len(b) < 1:
        raise OracleInputError("ARG", "cu_seqlens needs at least one entry")
    if b[0] != 0:
        raise OracleInputError("CU_START", f"cu_seqlens[0] = {b[0]}")
    for i in range(len(b) - 1):
        if b[i + 1] < b[i]:
            raise OracleInputError("CU_MONOTONE", f"cu_seqlens[{i + 1}] < cu_seqlens[{i}]")
    if b[-1] != total:
        raise OracleInputError("CU_TOTAL", f"cu_seqlens[-1] = {b[-1]} != {total}")
    for i in range(len(b) - 1):
        if (b[i + 1] - b[i]) % (2 * cp) != 0:
            raise OracleInputError(
                "CU_DIVISIBLE", f"slot {i} length {b[i + 1] - b[i]} not a multiple of {2 * cp}")
    return b


# ---------------------------------------------------------------------------
# Per-rank token lists.
# ---------------------------------------------------------------------------

def zigzag_rank_tokens(cu, cp: int, rank: int) -> np.ndarray:
    """Global token ids owned by ``rank`` under the ring (zigzag) slice.

    "Packed Sequence 与上下文并行" §2.4: each slot of length L is cut into 2*cp
    equal chunks of L/(2*cp) tokens; the rank keeps chunk ``rank`` and chunk
    ``2*cp-1-rank``, slot after slot, the earlier chunk first.  An empty slot
    (a repeated boundary, Relax PR #273 §2.2) has zero-length chunks and adds
    nothing.
    """
    b = _as_int_list(cu)
    owned_chunks = (rank, 2 * cp - 1 - rank)
    tokens: list[int] = []
    for s in range(len(b) - 1):
        slot_start = b[s]
        chunk = (b[s + 1] - b[s]) // (2 * cp)
        for c in owned_chunks:
            first = slot_start + c * chunk
            tokens.extend(range(first, first + chunk))
    return np.asarray(tokens, dtype=np.int64)


def zigzag_position(cu, cp: int, total: int, token: int) -> int:
    """Emulated zigzag row of one token, for checking huge batches one token
    at a time.

    The same definition as ``zigzag_rank_tokens`` ("Packed Sequence 与上下文并行"
    §2.4), read for a single token: in its slot the token sits in chunk q;
    the rank owning q is the r with q in {r, 2*cp-1-r}; on that rank every
    earlier slot contributed two chunks, and within the slot chunk r comes
    before chunk 2*cp-1-r.
    """
    b = _as_int_list(cu)
    before = 0                                    # rows each rank holds from earlier slots
    for s in range(len(b) - 1):
        start, end = b[s], b[s + 1]
        chunk = (end - start) // (2 * cp)
        if start <= token < end:
            q = (token - start) // chunk
            rank = q if q < cp else 2 * cp - 1 - q
            local = before + (0 if q == rank else chunk) + (token - start - q * chunk)
            return rank * (total // cp) + local
        before += 2 * chunk
    raise OracleInputError("ARG", f"token {token} outside the batch")


def contiguous_rank_tokens(total: int, cp: int, rank: int) -> np.ndarray:
    """Global token ids owned by ``rank`` under the contiguous (Ulysses) slice.

    "Packed Sequence 与上下文并行" §2.5: the packed stream is split into cp equal
    consecutive pieces and rank r keeps piece r.
    """
    share = total // cp
    return np.arange(rank * share, (rank + 1) * share, dtype=np.int64)


def layout_tokens(cu, cp: int, total: int, layout: str) -> np.ndarray:
    """The emulated global buffer: every rank's share, rank 0 first.

    Row ``rank * (total // cp) + local`` of the buffer holds the token that rank
    ``rank`` keeps at local position ``local``.
    """
    if layout == ZIGZAG:
        parts = [zigzag_rank_tokens(cu, cp, r) for r in range(cp)]
    elif layout == CONTIGUOUS:
        parts = [contiguous_rank_tokens(total, cp, r) for r in range(cp)]
    else:
        raise OracleInputError("DIRECTION", f"unknown layout {layout!r}")
    out = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    if out.shape[0] != total:
        raise OracleInputError("ARG", f"layout {layout} covers {out.shape[0]} of {total} tokens")
    return out


def _positions(tokens: np.ndarray) -> np.ndarray:
    """Inverse of a token list: ``pos[g]`` is the row that holds token ``g``."""
    pos = np.full(tokens.shape[0], -1, dtype=np.int64)
    pos[tokens] = np.arange(tokens.shape[0], dtype=np.int64)
    if tokens.shape[0] and (pos < 0).any():
        raise AssertionError("layout is not a permutation of the tokens")
    return pos


# ---------------------------------------------------------------------------
# Route (Relax PR #273 §2.1): for source layout zigzag and target layout
# contiguous, which rows each rank sends to each other rank.
# ---------------------------------------------------------------------------

def build_route(cu, cp: int, total: int) -> dict:
    """Per-token zigzag -> contiguous route over all cp emulated ranks.

    Returns a dict with

    * ``identity``: True when cp == 1 (the swap short-circuits before reading
      the boundaries, Relax PR #273 §2.6) or the batch is empty;
    * ``zigzag`` / ``contiguous``: the emulated buffers' token lists;
    * ``src_row`` / ``dst_row``: for each global token, its row in the zigzag
      buffer and in the contiguous buffer;
    * ``split``: ``split[s][d]`` tokens go from rank s (zigzag) to rank d
      (contiguous);
    * ``send_rows[s]`` (local rows of rank s, grouped by destination rank, each
      group in ascending token order), ``recv_rows[d]`` (local rows on rank d,
      grouped by source rank, ascending token order), ``input_split_sizes[s]``
      = split[s, :] and ``output_split_sizes[d]`` = split[:, d].

    The reverse direction uses the same route with the roles of the two
    layouts exchanged (its split matrix is the transpose).
    """
    if cp < 1:
        raise OracleInputError("ARG", f"cp_size must be >= 1, got {cp}")
    if cp == 1:
        return {"identity": True, "cp": 1, "total": total}
    check_route_boundaries(cu, cp, total)
    share = total // cp
    z = layout_tokens(cu, cp, total, ZIGZAG)
    c = layout_tokens(cu, cp, total, CONTIGUOUS)
    src_row = _positions(z)
    dst_row = _positions(c)
    tokens = np.arange(total, dtype=np.int64)
    src_rank = src_row // share if share else src_row
    dst_rank = dst_row // share if share else dst_row
    split = np.zeros((cp, cp), dtype=np.int64)
    np.add.at(split, (src_rank, dst_rank), 1)

    send_rows, recv_rows = [], []
    for s in range(cp):
        mine = tokens[src_rank == s]
        order = np.lexsort((mine, dst_rank[mine]))          # by destination, then token
        send_rows.append(src_row[mine[order]] - s * share)
    for d in range(cp):
        mine = tokens[dst_rank == d]
        order = np.lexsort((mine, src_rank[mine]))          # by source, then token
        recv_rows.append(dst_row[mine[order]] - d * share)
    return {
        "identity": total == 0,
        "cp": cp,
        "total": total,
        "zigzag": z,
        "contiguous": c,
        "src_row": src_row,
        "dst_row": dst_row,
        "split": split,
        "send_rows": send_rows,
        "recv_rows": recv_rows,
        "input_split_sizes": [split[s, :].copy() for s in range(cp)],
        "output_split_sizes": [split[:, d].copy() for d in range(cp)],
    }


def canonical_runs(route: dict) -> np.ndarray:
    """Maximal runs of the route, ordered by zigzag row.

    A run ``(src_row, dst_row, length)`` maps ``length`` consecutive zigzag
    rows onto ``length`` consecutive contiguous rows and stays inside one
    (source rank, destination rank) group.  Runs are listed in zigzag-row
    order, which is also (source rank, destination rank, token) order.  The
    run list is a compact way of writing the per-token route, nothing more: it
    is what the interval form of the route on the Relax PR #273 page (§2.1)
    reaches, with adjacent intervals merged.
    """
    if route["cp"] == 1 or route["total"] == 0:
        return np.zeros((0, 3), dtype=np.int64)
    total, cp = route["total"], route["cp"]
    share = total // cp
    z = route["zigzag"]
    dst_of_row = route["dst_row"][z]                 # zigzag row i -> contiguous row
    rows = np.arange(total, dtype=np.int64)
    starts = np.ones(total, dtype=bool)
    starts[1:] = ((dst_of_row[1:] != dst_of_row[:-1] + 1)
                  | (rows[1:] % share == 0)
                  | (dst_of_row[1:] % share == 0))
    first = np.flatnonzero(starts)
    lengths = np.diff(np.append(first, total))
    return np.stack([first, dst_of_row[first], lengths], axis=1).astype(np.int64)


# ---------------------------------------------------------------------------
# Swap: apply the route to rows (Relax PR #273 §2.1 pack -> all-to-all ->
# scatter, emulated over all ranks at once).
# ---------------------------------------------------------------------------

def swap_rows(x: np.ndarray, cu, cp: int, total: int, direction: str) -> np.ndarray:
    """Move the rows of ``x`` (shape [total, ...], any dtype) between layouts.

    ``direction`` is ``"z2c"`` (zigzag buffer in, contiguous buffer out) or
    ``"c2z"``.  Row ``j`` of the output holds the token that the target layout
    puts there, copied bit for bit from the row that holds it in the source
    layout.  cp == 1 returns ``x`` itself (the identity, Relax PR #273 §2.2).
    The route is built, then applied: ``build_route`` followed by
    ``apply_route``.
    """
    if direction not in ("z2c", "c2z"):
        raise OracleInputError("DIRECTION", f"unknown direction {direction!r}")
    x = np.asarray(x)
    if x.shape[0] != total:
        raise OracleInputError("SHAPE", f"x has {x.shape[0]} rows, route has {total}")
    return apply_route(x, build_route(cu, cp, total), direction)


def apply_route(x: np.ndarray, route: dict, direction: str, out_rows=None) -> np.ndarray:
    """Apply a route from ``build_route`` to the rows of ``x`` (the swap
    alone, without building the route).

    ``out_rows`` (a ``slice`` of output rows, default all) produces only those
    rows of the output, so a batch too large to gather at once can be checked
    piece by piece; the result then has ``len(range(total)[out_rows])`` rows.
    An identity route returns ``x`` (or its rows ``out_rows``) itself.
    """
    if direction not in ("z2c", "c2z"):
        raise OracleInputError("DIRECTION", f"unknown direction {direction!r}")
    x = np.asarray(x)
    total = route["total"]
    if x.shape[0] != total:
        raise OracleInputError("SHAPE", f"x has {x.shape[0]} rows, route has {total}")
    if route["cp"] == 1 or total == 0:
        return x if out_rows is None else x[out_rows]
    raw = x.reshape(total, -1).view(np.uint8) if x.size else x.reshape(total, 0).view(np.uint8)
    if direction == "z2c":
        source_of_out = route["src_row"][route["contiguous"]]
    else:
        source_of_out = route["dst_row"][route["zigzag"]]
    if out_rows is not None:
        source_of_out = source_of_out[out_rows]
    out = np.take(raw, source_of_out, axis=0)
    return out.view(x.dtype).reshape((out.shape[0],) + x.shape[1:])


# ---------------------------------------------------------------------------
# Label shift / MTP roll / valid-token mask ("Packed Sequence 与上下文并行"
# §1.3, §1.6, §2.2, §3.4).
# ---------------------------------------------------------------------------

def check_roll_boundaries(cu_padded, cu_real, total: int) -> tuple[list[int], list[int]]:
    """Validate padded and real boundaries for the roll.

    Order: first boundary 0 (either list), non-decreasing (either list), last
    padded boundary equals the token count, each real length at most its
    padded length.  ``cu_real=None`` means no slot has pads.
    """
    if total < 0:
        raise OracleInputError("ARG", f"total tokens must be >= 0, got {total}")
    p = _as_int_list(cu_padded)
    r = p if cu_real is None else _as_int_list(cu_real)
    if len(p) < 1 or len(r) != len(p):
        raise OracleInputError("ARG", "boundary lists must be non-empty and equally long")
    if p[0] != 0 or r[0] != 0:
        raise OracleInputError("CU_START", "first boundary is not 0")
    for i in range(len(p) - 1):
        if p[i + 1] < p[i] or r[i + 1] < r[i]:
            raise OracleInputError("CU_MONOTONE", f"boundary {i + 1} decreases")
    if p[-1] != total:
        raise OracleInputError("CU_TOTAL", f"cu_seqlens_padded[-1] = {p[-1]} != {total}")
    for i in range(len(p) - 1):
        if r[i + 1] - r[i] > p[i + 1] - p[i]:
            raise OracleInputError("REAL_GT_PADDED", f"slot {i} real length exceeds padded length")
    return p, r


def roll_labels(ids, cu_padded, cu_real, total: int, max_shift: int, fill: int = 0):
    """Document-aware shifted streams and validity masks.

    For position t in padded slot s (``cu_padded[s] <= t < cu_padded[s+1]``),
    the document's real tokens end at ``e = cu_padded[s] + real_len[s]``; the
    rest of the slot is alignment padding (§2.2).

    * ``mask[0][t] = t < e`` is the valid-token mask (zero at pads, §2.2/§3.4);
    * for shift j in 1..max_shift: ``shifted[j-1][t] = ids[t+j]`` and
      ``mask[j][t] = 1`` when ``t + j < e``, else ``fill`` and 0.

    Shift 1 is the next-token label; shift k+1 is the target of MTP depth k.
    A target never comes from another document (§1.3, §1.6).  Returns
    ``(shifted int64 [max_shift, total], mask uint8 [max_shift + 1, total])``.
    """
    if not 1 <= max_shift <= 8:
        raise OracleInputError("ARG", f"max_shift must be in 1..8, got {max_shift}")
    p, r = check_roll_boundaries(cu_padded, cu_real, total)
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    if ids.shape[0] != total:
        raise OracleInputError("SHAPE", f"ids has {ids.shape[0]} entries, expected {total}")
    shifted = np.full((max_shift, total), fill, dtype=np.int64)
    mask = np.zeros((max_shift + 1, total), dtype=np.uint8)
    for s in range(len(p) - 1):
        begin, end_padded = p[s], p[s + 1]
        if begin == end_padded:
            continue                                   # empty slot: no positions
        end_real = begin + (r[s + 1] - r[s])
        mask[0, begin:end_real] = 1
        for j in range(1, max_shift + 1):
            last = end_real - j                         # positions t < last have t + j < e
            if last > begin:
                shifted[j - 1, begin:last] = ids[begin + j:end_real]
                mask[j, begin:last] = 1
    return shifted, mask


def roll_valid_at(cu_padded, cu_real, token: int, shift: int) -> bool:
    """Whether shift ``shift`` of one position is a real label, for checking
    huge batches one position at a time.

    The same definition as ``roll_labels`` read for a single position: the
    padded slot holding ``token`` ends its real tokens at
    ``e = cu_padded[s] + (cu_real[s+1] - cu_real[s])``, and shift j is valid
    when ``token + j < e`` (shift 0 is the valid-token mask).  The shifted
    value is then ``ids[token + j]``, else the fill value.
    """
    p = _as_int_list(cu_padded)
    r = p if cu_real is None else _as_int_list(cu_real)
    for s in range(len(p) - 1):
        if p[s] <= token < p[s + 1]:
            return token + shift < p[s] + (r[s + 1] - r[s])
    raise OracleInputError("ARG", f"position {token} outside the batch")


# ---------------------------------------------------------------------------
# Packing ("Packed Sequence 与上下文并行" §2.2 steps (1)-(3), §3.2-§3.4).
# ---------------------------------------------------------------------------

def pack_batch(tokens, pad_id: int, eod_id: int, align: int, capacity: int, max_docs: int, pad_value: int):
    """Pack a [batch, seq] token matrix into one padded THD stream.

    Steps of §2.2, in order:

    1. documents: in each row the valid part ends after the last non-PAD
       token; inside it every EOD token closes a document (the EOD belongs to
       the document it closes) and whatever follows the last EOD is one more
       document.  PAD tokens before the end of the valid part stay inside
       their document.  Rows are taken in order, documents left to right.
    2. alignment: each document is padded at its end to a multiple of
       ``align`` (the page's TP*CP*2, or TP*CP*16 with FP8);
    3. flattening: documents are laid end to end at their padded offsets and
       every position that holds no token gets ``pad_value``.

    A fixed token budget keeps the output shape independent of the data: the
    stream is ``capacity`` long, the space after the last document is one
    trailing pad-only slot, and the document slots not used are empty (a
    repeated boundary).  Returns ``(packed int64 [capacity], cu_seqlens int32
    [max_docs + 2], cu_seqlens_padded int32 [max_docs + 2])``: slot k < n_docs
    is document k, slot n_docs the trailing pad slot, later slots are empty.
    Raises PACK_DOCS when there are more than ``max_docs`` documents and
    PACK_CAPACITY when the padded documents do not fit in ``capacity``.
    """
    if align < 1 or capacity < 0 or max_docs < 0 or capacity % align != 0 or pad_id == eod_id:
        raise OracleInputError("ARG", "bad pack arguments")
    rows = np.asarray(tokens, dtype=np.int64)
    rows = rows.reshape(-1, rows.shape[-1]) if rows.size else rows.reshape(-1, max(rows.shape[-1:] or [0]))
    docs = []                                           # (row, start, end) in row coordinates
    for b in range(rows.shape[0]):
        row = rows[b]
        non_pad = [s for s in range(row.shape[0]) if row[s] != pad_id]
        valid_end = non_pad[-1] + 1 if non_pad else 0
        start = 0
        for s in range(valid_end):
            if row[s] == eod_id:
                docs.append((b, start, s + 1))
                start = s + 1
        if start < valid_end:
            docs.append((b, start, valid_end))
    lengths = [e - s for _, s, e in docs]
    padded = [n + (-n) % align for n in lengths]
    if len(docs) > max_docs:
        raise OracleInputError("PACK_DOCS", f"{len(docs)} documents, room for {max_docs}")
    if sum(padded) > capacity:
        raise OracleInputError("PACK_CAPACITY", f"{sum(padded)} padded tokens, room for {capacity}")
    cu_real = np.zeros(max_docs + 2, dtype=np.int64)
    cu_pad = np.zeros(max_docs + 2, dtype=np.int64)
    for k, (n, p) in enumerate(zip(lengths, padded)):
        cu_real[k + 1] = cu_real[k] + n
        cu_pad[k + 1] = cu_pad[k] + p
    n_docs = len(docs)
    cu_real[n_docs + 1:] = cu_real[n_docs]              # trailing pad slot and empty slots: no real tokens
    cu_pad[n_docs + 1:] = capacity                      # trailing pad slot ends at the budget; the rest are empty
    packed = np.full(capacity, pad_value, dtype=np.int64)
    for k, (b, s, e) in enumerate(docs):
        packed[cu_pad[k]:cu_pad[k] + (e - s)] = rows[b, s:e]
    return packed, cu_real.astype(np.int32), cu_pad.astype(np.int32)
