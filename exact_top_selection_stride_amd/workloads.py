"""Seeded synthetic score matrices for the Top-K workloads.

This module only draws inputs; it holds none of the selection arithmetic, so the
CPU oracle and the HIP path can both be fed from it.

Shapes follow the operator matrix of the HPC-Ops Top-K evaluation (page
"几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K", section "20 个形状都最快"):
each width keeps the last 8192-row causal window, in which window row r has
valid length N_alloc - 8192 + r + 1, cut into non-overlapping groups of M rows;
the invalid suffix is -inf. The width crossover sweep (same page, section
"采样不是处处都该开") covers 16K to 64K widths.

The captured indexer scores those pages used are not available, so values are
synthetic, shaped after the score concentration that the LiteTopK review
(page "LiteTopK: Exploiting the Curse of Dimensionality for a Fused
Indexer-TopK Kernel ...", section 六, score distribution) reports: a dense body
around 25-35 and a rare upper tail at 45 and above. Recipe per row, in this
draw order: body ~ Normal(30, 2.5); tail mask = Uniform(0,1) < p per position;
tail = 45 + Exponential(mean 3) replaces the body where masked; optionally
rounded to bfloat16 (round-to-nearest-even) and widened back to float32;
positions at or past the row's length set to -inf.
"""
from dataclasses import dataclass, field
from typing import Optional

import torch

WINDOW = 8192
BASE_SEED = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    n_alloc: int
    M: int                      # rows per call (group size)
    groups: int                 # groups rotated between calls
    tail_p: float
    lengths: str                # "uniform" (C0) or "causal"
    bf16: bool = False
    seed: int = BASE_SEED
    note: str = field(default="", compare=False)

    @property
    def window_rows(self) -> int:
        return self.M * self.groups


def _c4(n_alloc: int, M: int) -> Workload:
    groups = WINDOW // M if M <= WINDOW else 1
    return Workload(f"c4_n{n_alloc}_m{M}", n_alloc, M, groups, 0.01, "causal", bf16=True,
                    seed=BASE_SEED + 4,
                    note="bf16-rounded ties; rows past 8192 repeat the causal window lengths")


WORKLOADS = {
    "c0": Workload("c0", 8192, 256, 1, 0.01, "uniform", seed=BASE_SEED + 0,
                   note="lengths uniform in [1, 8192]; some rows <= K"),
    "c1": Workload("c1", 131072, 512, 16, 0.01, "causal", seed=BASE_SEED + 1),
    "c2": Workload("c2", 524288, 4096, 2, 0.005, "causal", seed=BASE_SEED + 2),
    "c3a": Workload("c3a", 1048576, 512, 16, 0.01, "causal", seed=BASE_SEED + 3),
    "c3b": Workload("c3b", 1048576, 8192, 1, 0.01, "causal", seed=BASE_SEED + 3),
}
C4_WIDTHS = (16384, 32768, 65536)
C4_ROWS = (512, 1024, 2048, 4096, 8192, 16384, 32768)
for _n in C4_WIDTHS:
    for _m in C4_ROWS:
        WORKLOADS[f"c4_n{_n}_m{_m}"] = _c4(_n, _m)

# Decode-shaped calls: a few long rows (the first M rows of the causal window,
# lengths N - 8191 onwards) at 128K and 1M widths, with the C1/C3 value recipe.
DECODE_ROWS = (1, 4, 16, 64)
DECODE_WIDTHS = (131072, 1048576)
for _n in DECODE_WIDTHS:
    for _m in DECODE_ROWS:
        WORKLOADS[f"dec_n{_n}_m{_m}"] = Workload(
            f"dec_n{_n}_m{_m}", _n, _m, 1, 0.01, "causal", seed=BASE_SEED + 5,
            note="decode shape: few long rows, row-split execution")


def get(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None


def causal_lengths(n_alloc: int, rows: torch.Tensor) -> torch.Tensor:
    """Valid length of window row r: n_alloc - 8192 + (r mod 8192) + 1 (at least 1)."""
    L = n_alloc - WINDOW + (rows % WINDOW) + 1
    return L.clamp(min=1, max=n_alloc).to(torch.int32)


def make_lengths(w: Workload, row_start: int, n_rows: int, device, gen: torch.Generator):
    if w.lengths == "uniform":
        # Drawn first from the generator, for the whole window at once.
        full = torch.randint(1, w.n_alloc + 1, (w.window_rows,), generator=gen, device=device,
                             dtype=torch.int64)
        return full[row_start:row_start + n_rows].to(torch.int32).contiguous()
    rows = torch.arange(row_start, row_start + n_rows, device=device, dtype=torch.int64)
    return causal_lengths(w.n_alloc, rows)


def fill_rows(out: torch.Tensor, lengths: torch.Tensor, tail_p: float, bf16: bool,
              gen: torch.Generator, chunk_rows: Optional[int] = None) -> torch.Tensor:
    """Fills out[R, N] in place with the body/tail recipe and a -inf suffix."""
    R, N = out.shape
    device = out.device
    if chunk_rows is None:
        chunk_rows = max(1, (1 << 27) // max(N, 1))  # ~512 MiB of float32 per temporary
    cols = torch.arange(N, device=device, dtype=torch.int32)
    for r0 in range(0, R, chunk_rows):
        r1 = min(R, r0 + chunk_rows)
        n = r1 - r0
        body = torch.randn((n, N), generator=gen, device=device, dtype=torch.float32)
        body.mul_(2.5).add_(30.0)
        mask = torch.rand((n, N), generator=gen, device=device, dtype=torch.float32) < tail_p
        tail = torch.empty((n, N), device=device, dtype=torch.float32)
        tail.exponential_(1.0 / 3.0, generator=gen).add_(45.0)
        x = torch.where(mask, tail, body)
        del body, mask, tail
        if bf16:
            x = x.to(torch.bfloat16).to(torch.float32)
        x.masked_fill_(cols[None, :] >= lengths[r0:r1, None], float("-inf"))
        out[r0:r1].copy_(x)
        del x
    return out


def make_window(w: Workload, device="cpu", row_start: int = 0, n_rows: Optional[int] = None,
                seed: Optional[int] = None):
    """Returns (scores [n_rows, n_alloc] float32, row_len [n_rows] int32) for window rows
    [row_start, row_start + n_rows). Deterministic in (workload, seed, device, row range)."""
    if n_rows is None:
        n_rows = w.window_rows - row_start
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    lengths = make_lengths(w, row_start, n_rows, device, gen)
    scores = torch.empty((n_rows, w.n_alloc), device=device, dtype=torch.float32)
    fill_rows(scores, lengths, w.tail_p, w.bf16, gen)
    return scores, lengths


def make_rows(n_rows: int, n_alloc: int, lengths, tail_p: float = 0.01, bf16: bool = False,
              seed: int = BASE_SEED, device="cpu"):
    """Free-form variant: explicit lengths (list or tensor) and the same value recipe."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    lengths = torch.as_tensor(lengths, dtype=torch.int32, device=device).reshape(n_rows)
    scores = torch.empty((n_rows, n_alloc), device=device, dtype=torch.float32)
    fill_rows(scores, lengths.clamp(min=0, max=n_alloc), tail_p, bf16, gen)
    return scores, lengths


def valid_score_bytes(lengths: torch.Tensor, K: int) -> int:
    """Bytes of valid FP32 scores a selector must read: 4 * sum of L over rows with L > K."""
    L = lengths.to(torch.int64)
    return int(4 * L[L > K].sum().item())


# ---------------------------------------------------------------------------
# Indexer inputs for the score + select chain.
#
# The selector's scores come from a DSA-style indexer (page "LiteTopK: Exploiting
# the Curse of Dimensionality for a Fused Indexer-TopK Kernel ...", section
# 核心公式, Eq. (1)) computed by an FP8 multi-query score kernel (page
# "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K", section "框架轨迹").
# Neither the model nor its weights are available, so q, k and w are drawn here.
# Recipe, in this draw order from one generator:
#   g  ~ Normal(0, 1)^D                         one shared "topic" direction
#   q[t, h, :] = 0.25 * g + Normal(0, 1)^D      rounded to FP8 E4M3
#   hot[s]     = Uniform(0, 1) < hot_p          (1% of keys)
#   k[s, :]    = Normal(0, 1)^D + hot[s] * g    rounded to FP8 E4M3
#   w[t, h]    ~ (0.5 + 0.5 * Normal(0, 1)) / sqrt(H)   float32, mostly positive
# Hot keys align with every query's shared component and form the upper tail of
# each score row; the cold keys form a dense body (the concentration the LiteTopK
# review reports for real indexer scores). Lengths are the causal window
# lengths of the selector workloads. Only the input draw lives here; the score
# arithmetic is the HIP kernel's (product path) and the oracle's (tests).
# ---------------------------------------------------------------------------

INDEXER_HEADS = 64
INDEXER_DIM = 128


@dataclass(frozen=True)
class ChainWorkload:
    name: str
    n_alloc: int        # keys S (= the selector's N_alloc)
    M: int              # query rows per call
    heads: int = INDEXER_HEADS
    dim: int = INDEXER_DIM
    hot_p: float = 0.01
    seed: int = BASE_SEED + 7


CHAINS = {
    "chain_c1": ChainWorkload("chain_c1", 131072, 512),
    "chain_n512k_m1024": ChainWorkload("chain_n512k_m1024", 524288, 1024),
}


def get_chain(name: str) -> ChainWorkload:
    try:
        return CHAINS[name]
    except KeyError:
        raise KeyError(f"unknown chain workload {name!r}; known: {sorted(CHAINS)}") from None


def to_e4m3_codes(x: torch.Tensor) -> torch.Tensor:
    """Rounds float32 values to OCP FP8 E4M3 (torch's float8_e4m3fn, saturating at
    +-448 first) and returns the raw bytes as uint8."""
    return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def make_indexer_inputs(T: int, S: int, H: int = INDEXER_HEADS, D: int = INDEXER_DIM,
                        row_len=None, hot_p: float = 0.01, seed: int = BASE_SEED + 7,
                        device="cpu", row_start: int = 0):
    """Returns (q [T, H, D] uint8, k [S, D] uint8, w [T, H] float32, row_len [T] int32).

    row_len defaults to the causal window lengths of rows row_start.. (S - 8192 + r + 1)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    g = torch.randn((D,), generator=gen, device=device, dtype=torch.float32)
    q = torch.randn((T, H, D), generator=gen, device=device, dtype=torch.float32)
    q.add_(0.25 * g)
    hot = torch.rand((S, 1), generator=gen, device=device, dtype=torch.float32) < hot_p
    k = torch.randn((S, D), generator=gen, device=device, dtype=torch.float32)
    k.add_(hot.to(torch.float32) * g)
    w = torch.randn((T, H), generator=gen, device=device, dtype=torch.float32)
    w.mul_(0.5).add_(0.5).div_(H ** 0.5)
    if row_len is None:
        rows = torch.arange(row_start, row_start + T, device=device, dtype=torch.int64)
        row_len = causal_lengths(S, rows)
    else:
        row_len = torch.as_tensor(row_len, dtype=torch.int32, device=device).reshape(T)
    return to_e4m3_codes(q).contiguous(), to_e4m3_codes(k).contiguous(), w.contiguous(), row_len


def make_chain(c: ChainWorkload, device="cpu", row_start: int = None, n_rows: int = None):
    """Indexer inputs of a chain workload: the last M rows of the causal window by default."""
    if n_rows is None:
        n_rows = c.M
    if row_start is None:
        row_start = WINDOW - c.M
    return make_indexer_inputs(n_rows, c.n_alloc, c.heads, c.dim, hot_p=c.hot_p, seed=c.seed,
                               device=device, row_start=row_start)
