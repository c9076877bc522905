"""Seeded synthetic inputs for the FP4 paged-MQA indexer with exact TopK.

This module only draws random data in the operator's input layout. It holds
none of the method's arithmetic (no decoding, no dot products, no selection),
so that both the HIP path and the CPU oracle can be fed from it.

Workload shapes follow the pages:
- "[FlyDSL] Add FP4 LiteTopK prefill operator" (ROCm/aiter PR 5309), Summary,
  model table: Q=8192 rows, H=64 heads, D=128, K=512 (V4-Flash) or 1024
  (V4-Pro), C4 context = raw / 4; Validation table: C4 widths 65,536,
  131,072 and 196,608; the pages benchmark fixed synthetic tensors shaped like
  the released models.
- "[FlyDSL][DSv4] Prototype FP4 MQA streaming TopK" (ROCm/aiter PR 5282),
  Scope: 64-position KV pages, 256-position score blocks, ragged prefill
  windows, shuffled page tables; runtime update: 1024-row production grid at
  C4 widths 196,608 and 262,144.

Layout of one input set (all numpy, C-contiguous):
  q          uint8   [Q, 64, 64]   E2M1 codes, two per byte; element 2j is the
                                   low nibble of byte j
  q_scale    uint8   [Q, 64, 4]    UE8M0 exponent byte per 32 elements along D
  k_pages    uint8   [P_phys, 64, 64]  paged C4 key cache, same packing
  k_scale    uint8   [P_phys, 64, 4]
  weights    float32 [Q, 64]
  page_table int32   [P_log]       logical page -> physical page, S = 64 * P_log
  row_start  int32   [Q]           window [start, end) in C4 positions
  row_end    int32   [Q]

Value recipe: codes uniform over all 16 E2M1 codes,
scale bytes 127 + U{-2..2}, weights N(0, 1/64) rounded to float32, page table a
seeded permutation, 5% of key positions duplicated (codes and scales) from a
seeded earlier, non-duplicated position.
"""
from __future__ import annotations

import dataclasses

import numpy as np

H = 64
D = 128
PAGE = 64
ROW_BYTES = D // 2          # 64 bytes of codes per head / key
SCALES = D // 32            # 4 scale bytes per head / key

BASE_SEED = 20261202


@dataclasses.dataclass
class Inputs:
    q: np.ndarray
    q_scale: np.ndarray
    k_pages: np.ndarray
    k_scale: np.ndarray
    weights: np.ndarray
    page_table: np.ndarray
    row_start: np.ndarray
    row_end: np.ndarray
    K: int
    name: str = ""
    tie_rows: np.ndarray = dataclasses.field(default_factory=lambda: np.zeros(0, np.int64))

    @property
    def Q(self) -> int:
        return int(self.q.shape[0])

    @property
    def P_log(self) -> int:
        return int(self.page_table.shape[0])

    @property
    def P_phys(self) -> int:
        return int(self.k_pages.shape[0])

    @property
    def S(self) -> int:
        return PAGE * self.P_log

    def lengths(self) -> np.ndarray:
        return self.row_end.astype(np.int64) - self.row_start.astype(np.int64)

    def scored_pairs(self) -> int:
        """Scored (row, position) pairs of the long rows (length > K)."""
        n = self.lengths()
        return int(n[n > self.K].sum())


def _codes(rng: np.random.Generator, shape) -> np.ndarray:
    # one byte = two independent uniform 4-bit codes
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def _scales(rng: np.random.Generator, shape) -> np.ndarray:
    return (127 + rng.integers(-2, 3, size=shape)).astype(np.uint8)


def causal_windows(Q: int, S: int) -> tuple[np.ndarray, np.ndarray]:
    """Ragged causal prefill windows: start 0, end_i = S - floor((Q-1-i)/4)."""
    i = np.arange(Q, dtype=np.int64)
    end = S - (Q - 1 - i) // 4
    return np.zeros(Q, np.int32), end.astype(np.int32)


def make_inputs(Q: int, S: int, K: int, seed: int, *, row_start=None, row_end=None,
                dup_frac: float = 0.05, tie_rows: int = 0, P_phys: int | None = None,
                name: str = "") -> Inputs:
    """Draw one seeded input set. S must be a multiple of the page size 64.

    row_start/row_end default to the ragged causal windows. ``tie_rows`` rows
    (seeded) get all-zero query codes, which makes every score in their window
    equal. ``P_phys`` > P_log leaves unused physical pages (filled with random
    data) so that slot numbers differ from identity mappings.
    """
    if S % PAGE:
        raise ValueError("S must be a multiple of 64")
    rng = np.random.Generator(np.random.PCG64(seed))
    P_log = S // PAGE
    P_phys = P_log if P_phys is None else int(P_phys)
    if P_phys < P_log:
        raise ValueError("need P_phys >= P_log for a permutation table")

    q = _codes(rng, (Q, H, ROW_BYTES))
    q_scale = _scales(rng, (Q, H, SCALES))
    weights = rng.standard_normal((Q, H)) * (1.0 / 8.0)
    weights = weights.astype(np.float32)

    k_log = _codes(rng, (S, ROW_BYTES))
    ks_log = _scales(rng, (S, SCALES))
    n_dup = int(round(dup_frac * S))
    if n_dup > 0 and S > 1:
        dup = np.sort(rng.choice(np.arange(1, S), size=min(n_dup, S - 1), replace=False))
        keep = np.setdiff1d(np.arange(S), dup, assume_unique=True)
        # pick, for each duplicated position, a uniform non-duplicated earlier one
        n_before = np.searchsorted(keep, dup, side="left")
        pick = (rng.random(dup.shape[0]) * n_before).astype(np.int64)
        src = keep[np.minimum(pick, n_before - 1)]
        k_log[dup] = k_log[src]
        ks_log[dup] = ks_log[src]

    perm = rng.permutation(P_phys)[:P_log].astype(np.int32)
    k_pages = _codes(rng, (P_phys, PAGE, ROW_BYTES))
    k_scale = _scales(rng, (P_phys, PAGE, SCALES))
    k_pages[perm] = k_log.reshape(P_log, PAGE, ROW_BYTES)
    k_scale[perm] = ks_log.reshape(P_log, PAGE, SCALES)

    if row_start is None or row_end is None:
        row_start, row_end = causal_windows(Q, S)
    row_start = np.ascontiguousarray(row_start, dtype=np.int32)
    row_end = np.ascontiguousarray(row_end, dtype=np.int32)

    ties = np.zeros(0, np.int64)
    if tie_rows > 0:
        ties = np.sort(rng.choice(Q, size=tie_rows, replace=False)).astype(np.int64)
        q[ties] = 0
    return Inputs(q=q, q_scale=q_scale, k_pages=k_pages, k_scale=k_scale, weights=weights,
                  page_table=perm, row_start=row_start, row_end=row_end, K=int(K),
                  name=name, tie_rows=ties)


# --- the five workloads and the headline shape -------------------------------------

TINY_SHORT_LENGTHS = [0, 1, 2, 63, 64, 65, 127, 128, 255, 256, 300, 400, 500, 510, 511, 512]
TINY_LONG_LENGTHS = [513, 514, 600, 1000, 1024, 1025, 1500, 2000, 2047, 2048]


def tiny_windows(seed: int, Q: int = 32, S: int = 2048, K: int = 512):
    """Windows of the tiny workload: rows 0-15 short (row 0 empty at start 100),
    rows 16-31 long; rows 1-3 and the full-length row start at 0, the rest at
    seeded, mostly non-page-aligned starts."""
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    lens = list(TINY_SHORT_LENGTHS) + list(TINY_LONG_LENGTHS)
    lens += [int(x) for x in rng.integers(K + 1, S + 1, size=Q - len(lens))]
    start = np.zeros(Q, np.int64)
    for i, n in enumerate(lens):
        if i == 0:
            start[i] = 100
        elif i in (1, 2, 3) or n == S:
            start[i] = 0
        else:
            start[i] = int(rng.integers(0, S - n + 1))
    lens = np.asarray(lens, np.int64)
    return start.astype(np.int32), (start + lens).astype(np.int32)


CONFIGS = {
    1: dict(Q=32, S=2048, K=512, name="tiny Q=32 C4=2048 K=512"),
    2: dict(Q=1024, S=65536, K=512, name="V4-Flash-shaped Q=1024 C4=65536 K=512"),
    3: dict(Q=1024, S=196608, K=1024, name="V4-Pro-shaped Q=1024 C4=196608 K=1024"),
    4: dict(Q=8192, S=131072, K=512, name="V4-Flash long prefill Q=8192 C4=131072 K=512"),
    5: dict(Q=8192, S=262144, K=1024, name="V4-Pro long prefill Q=8192 C4=262144 K=1024"),
    # headline shape of the pages' Validation table (V4-Pro, 786,432 raw tokens)
    "H": dict(Q=8192, S=196608, K=1024, name="V4-Pro headline Q=8192 C4=196608 K=1024"),
    # the table's other shapes ("[FlyDSL] Add FP4 LiteTopK prefill operator",
    # Validation): V4-Flash (K=512) and V4-Pro (K=1024) at 262,144 / 524,288 /
    # 786,432 raw tokens, i.e. C4 65,536 / 131,072 / 196,608, Q = 8192
    "F65": dict(Q=8192, S=65536, K=512, name="V4-Flash Q=8192 C4=65536 K=512"),
    "F131": dict(Q=8192, S=131072, K=512, name="V4-Flash Q=8192 C4=131072 K=512"),
    "F196": dict(Q=8192, S=196608, K=512, name="V4-Flash Q=8192 C4=196608 K=512"),
    "P65": dict(Q=8192, S=65536, K=1024, name="V4-Pro Q=8192 C4=65536 K=1024"),
    "P131": dict(Q=8192, S=131072, K=1024, name="V4-Pro Q=8192 C4=131072 K=1024"),
}
_NAMED_IDS = {"H": 6, "F65": 7, "F131": 8, "F196": 9, "P65": 10, "P131": 11}


def config_seed(cfg) -> int:
    cid = _NAMED_IDS[cfg] if isinstance(cfg, str) else int(cfg)
    return BASE_SEED + 1000 * cid


def make_config(cfg) -> Inputs:
    c = CONFIGS[cfg]
    seed = config_seed(cfg)
    kw = {}
    if cfg == 1:
        kw["row_start"], kw["row_end"] = tiny_windows(seed, c["Q"], c["S"], c["K"])
    if cfg == 5:
        kw["tie_rows"] = int(round(0.01 * c["Q"]))
    return make_inputs(c["Q"], c["S"], c["K"], seed, name=c["name"], **kw)


def sample_rows(inp: Inputs, n: int, seed: int) -> np.ndarray:
    """Seeded sample of n long rows including the first and last row; at least
    n // 8 of them tie rows when the input has any."""
    rng = np.random.Generator(np.random.PCG64(seed + 99))
    Q = inp.Q
    chosen = {0, Q - 1}
    if inp.tie_rows.size:
        m = min(inp.tie_rows.size, max(1, n // 8))
        chosen.update(int(x) for x in rng.choice(inp.tie_rows, size=m, replace=False))
    while len(chosen) < min(n, Q):
        chosen.add(int(rng.integers(0, Q)))
    return np.array(sorted(chosen), dtype=np.int64)


# --- decode / multi-sequence workloads ---------------------------------------------

@dataclasses.dataclass
class DecodeInputs:
    """Several sequences in one shared physical page pool. Row r belongs to
    sequence seq_of_row[r]; its window is in that sequence's logical positions;
    block_table[s, p] is the physical page of logical page p of sequence s
    (-1 past the sequence's pages)."""
    q: np.ndarray
    q_scale: np.ndarray
    k_pages: np.ndarray
    k_scale: np.ndarray
    weights: np.ndarray
    block_table: np.ndarray
    seq_of_row: np.ndarray
    row_start: np.ndarray
    row_end: np.ndarray
    seq_len: np.ndarray
    K: int
    name: str = ""

    @property
    def Q(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def lengths(self) -> np.ndarray:
        return self.row_end.astype(np.int64) - self.row_start.astype(np.int64)

    def scored_pairs(self) -> int:
        n = self.lengths()
        return int(n[n > self.K].sum())

    def view(self, seq: int) -> Inputs:
        """The single-table view of one sequence (every row shares its page table)."""
        return Inputs(self.q, self.q_scale, self.k_pages, self.k_scale, self.weights,
                      np.ascontiguousarray(self.block_table[seq]), self.row_start, self.row_end, self.K,
                      name=f"{self.name} seq {seq}")


def make_decode_inputs(n_seq: int, rows_per_seq: int, min_len: int, max_len: int, K: int, seed: int, *,
                       spare_pages: int = 3, dup_frac: float = 0.05, name: str = "") -> DecodeInputs:
    """Seeded decode-shaped inputs: n_seq sequences with C4 lengths uniform in
    [min_len, max_len], their pages scattered over one shuffled physical pool,
    rows_per_seq query rows per sequence with causal windows ending at the
    sequence's last positions (row j of a sequence: [0, len - (rows_per_seq-1-j)))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(min_len, max_len + 1, n_seq)
    pages = (lens + PAGE - 1) // PAGE
    max_pages = int(pages.max())
    P_phys = int(pages.sum()) + spare_pages
    phys = rng.permutation(P_phys).astype(np.int32)
    block_table = np.full((n_seq, max_pages), -1, np.int32)
    at = 0
    for s in range(n_seq):
        block_table[s, :pages[s]] = phys[at:at + pages[s]]
        at += pages[s]
    Q = n_seq * rows_per_seq
    base = make_inputs(Q, PAGE * P_phys, K, seed + 1, dup_frac=dup_frac, P_phys=P_phys)
    seq_of_row = np.repeat(np.arange(n_seq, dtype=np.int32), rows_per_seq)
    j = np.tile(np.arange(rows_per_seq), n_seq)
    row_end = (lens[seq_of_row] - (rows_per_seq - 1 - j)).clip(min=0).astype(np.int32)
    row_start = np.zeros(Q, np.int32)
    return DecodeInputs(base.q, base.q_scale, base.k_pages, base.k_scale, base.weights, block_table, seq_of_row,
                        row_start, row_end, lens.astype(np.int64), K, name=name)
