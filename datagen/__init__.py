"""Seeded synthetic inputs for fused linear cross-entropy.

This module only draws and encodes inputs; it holds none of the loss
arithmetic.  Both the fp64 oracle (``oracle/``) and the HIP path take their
inputs from here, so every comparison runs on identical bits.

Workloads follow the LM-head shapes the Liger Kernel pages name: the
low-level API example of the project overview page ("Método de API de Baixo
Nível": ``nn.Linear(128, 256)`` weight, ``randn`` input, ``randint`` targets),
the LLaMA-3-8B benchmark setting of the same page ("Benchmarks de
Desempenho"), and the Qwen-7B SFT comparison of the ms-swift blog page (its
benchmark table).  Only the head shapes (hidden size H, vocabulary V, tokens
N) enter; no text, tokenizer or trained weight is used.

Recipe (all draws from numpy PCG64, seed = 20260 + workload id unless given):
  * X  ~ N(0, 1) in fp32, or its row-RMS-normalised form
        x = g / sqrt(mean(g^2) + 1e-6) (computed in fp32);
  * W  ~ N(0, 0.02^2) in fp32, drawn in fixed blocks of 4096 rows, each block
        from its own spawned child stream (so the values do not depend on
        how many threads draw them);
  * labels: uniform in [0, V), or truncated Zipf with P(id = k-1) ~ k^-s;
  * ignored positions: exactly round(p*N) of them, chosen by a seeded
        permutation, or a contiguous prefix;
  * bf16 workloads round the fp32 draws to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

IGNORE_INDEX = -100
W_BLOCK_ROWS = 4096
_THREADS = 8


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic FLCE workload."""
    name: str
    N: int
    H: int
    V: int
    dtype: str                 # "f32" or "bf16"
    chunk_tokens: int          # chunk size the workload is run with
    x_dist: str = "normal"     # "normal" | "rmsnorm"
    label_dist: str = "uniform"  # "uniform" | "zipf"
    zipf_s: float = 1.1
    ignore_mode: str = "random"  # "random" | "prefix" | "none"
    ignore_frac: float = 0.05
    w_std: float = 0.02


# The five workloads.  Sizes and recipes: see the module docstring.
WORKLOADS = {
    0: Workload("tiny-fp32", 512, 128, 256, "f32", 128, ignore_frac=0.10),
    1: Workload("llama3-8b-head", 8192, 4096, 128256, "bf16", 1024),
    2: Workload("qwen2-7b-head", 16384, 3584, 152064, "bf16", 2048,
                x_dist="rmsnorm", label_dist="zipf"),
    3: Workload("llama3-8b-head-longctx", 16384, 4096, 128256, "bf16", 1024,
                ignore_mode="prefix", ignore_frac=0.25),
    4: Workload("large-vocab-head", 8192, 2304, 256000, "bf16", 0),
}

# chunk sizes swept for the long-context workload
LONGCTX_CHUNKS = (512, 1024, 4096)


@dataclasses.dataclass
class Inputs:
    """One drawn workload.

    For bf16 workloads ``X`` and ``W`` hold the bf16 bit patterns as uint16;
    for fp32 workloads they are float32.  ``labels`` is int64 [N].
    """
    wl: Workload
    X: np.ndarray
    W: np.ndarray
    labels: np.ndarray
    seed: int

    def X_f64(self) -> np.ndarray:
        return as_f64(self.X)

    def W_f64(self) -> np.ndarray:
        return as_f64(self.W)


# ---------------------------------------------------------------- encodings

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite by construction (no NaN handling)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    r = b >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(a: np.ndarray) -> np.ndarray:
    """Exact fp64 copy of an fp32 array or of a bf16 bit-pattern array."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------- drawing

def _encode(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else a32


def _draw_W(ss: np.random.SeedSequence, V: int, H: int, std: float, dtype: str) -> np.ndarray:
    nblk = max(1, math.ceil(V / W_BLOCK_ROWS))
    kids = ss.spawn(nblk)
    out = np.empty((V, H), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(b):
        r0, r1 = b * W_BLOCK_ROWS, min(V, (b + 1) * W_BLOCK_ROWS)
        g = np.random.default_rng(kids[b]).standard_normal((r1 - r0, H), dtype=np.float32)
        g *= np.float32(std)
        out[r0:r1] = _encode(g, dtype)

    if nblk == 1:
        one(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(one, range(nblk)))
    return out


def _draw_X(rng: np.random.Generator, N: int, H: int, dist: str, dtype: str) -> np.ndarray:
    g = rng.standard_normal((N, H), dtype=np.float32)
    if dist == "rmsnorm":
        ms = np.mean(g * g, axis=1, dtype=np.float32, keepdims=True)
        g = g / np.sqrt(ms + np.float32(1e-6))
    elif dist != "normal":
        raise ValueError(dist)
    return _encode(g.astype(np.float32), dtype)


def zipf_probs(V: int, s: float) -> np.ndarray:
    """P(id = k-1) proportional to k^-s for k = 1..V (fp64)."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def _draw_labels(rng: np.random.Generator, N: int, V: int, dist: str, s: float) -> np.ndarray:
    if dist == "uniform":
        return rng.integers(0, V, size=N, dtype=np.int64)
    if dist == "zipf":
        cdf = np.cumsum(zipf_probs(V, s))
        u = rng.random(N)
        return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int64)
    raise ValueError(dist)


def _ignore_positions(rng: np.random.Generator, N: int, mode: str, frac: float) -> np.ndarray:
    k = int(round(frac * N))
    if mode == "none" or k == 0:
        return np.zeros(0, dtype=np.int64)
    if mode == "random":
        return np.sort(rng.permutation(N)[:k]).astype(np.int64)
    if mode == "prefix":
        return np.arange(k, dtype=np.int64)
    raise ValueError(mode)


def draw(wl: Workload, seed: int) -> Inputs:
    """Draw one workload: X, then W, then labels, then ignored positions."""
    ss = np.random.SeedSequence(seed)
    s_x, s_w, s_y, s_i = ss.spawn(4)
    X = _draw_X(np.random.default_rng(s_x), wl.N, wl.H, wl.x_dist, wl.dtype)
    W = _draw_W(s_w, wl.V, wl.H, wl.w_std, wl.dtype)
    y = _draw_labels(np.random.default_rng(s_y), wl.N, wl.V, wl.label_dist, wl.zipf_s)
    ign = _ignore_positions(np.random.default_rng(s_i), wl.N, wl.ignore_mode, wl.ignore_frac)
    y[ign] = IGNORE_INDEX
    return Inputs(wl, X, W, y, seed)


def make(workload_id: int, seed: int | None = None) -> Inputs:
    """Draw one of the five named workloads (seed defaults to 20260 + id)."""
    wl = WORKLOADS[workload_id]
    return draw(wl, 20260 + workload_id if seed is None else seed)


def make_custom(N: int, H: int, V: int, dtype: str = "bf16", seed: int = 1,
                chunk_tokens: int = 0, **kw) -> Inputs:
    """Draw an ad-hoc workload (ragged shapes, edge cases)."""
    return draw(Workload("custom", N, H, V, dtype, chunk_tokens, **kw), seed)


def make_logits(N: int, V: int, dtype: str = "bf16", seed: int = 1, std: float = 1.28,
                ignore_frac: float = 0.05) -> tuple[np.ndarray, np.ndarray]:
    """Logits and labels for cross-entropy on given logits.

    Z ~ N(0, std^2) in fp32 (the default 1.28 = sqrt(4096) * 0.02 is the
    spread of x.w for x ~ N(0, 1), w ~ N(0, 0.02^2) at H = 4096, i.e. the
    Llama-3-8B head's logits at initialisation), bf16 rounded to nearest even
    (returned as uint16 bits); labels uniform with exactly round(p N) ignored.
    Draw order: Z, labels, ignored positions."""
    ss = np.random.SeedSequence(seed)
    s_z, s_y, s_i = ss.spawn(3)
    Z = np.random.default_rng(s_z).standard_normal((N, V), dtype=np.float32)
    Z *= np.float32(std)
    y = _draw_labels(np.random.default_rng(s_y), N, V, "uniform", 0.0)
    y[_ignore_positions(np.random.default_rng(s_i), N, "random", ignore_frac)] = IGNORE_INDEX
    return (f32_to_bf16_bits(Z) if dtype == "bf16" else Z), y


def _prompt_lengths(rng: np.random.Generator, T: int, n: int) -> np.ndarray:
    """U{ceil(T/8) .. floor(T/2)} unscored prompt tokens; none when T < 2."""
    lo, hi = -(-T // 8), T // 2
    if hi < lo:
        return np.zeros(n, dtype=np.int64)
    return rng.integers(lo, hi + 1, size=n)


def make_pairs(n_pairs: int, T: int, H: int, V: int, dtype: str = "bf16", seed: int = 1,
               w_std: float = 0.02) -> Inputs:
    """Preference batch: 2 n_pairs sequences of T tokens as rows of X (the
    n_pairs chosen sequences first, then the rejected ones; pair i is
    sequence i and sequence n_pairs + i).

    Each pair shares a prompt of P ~ U{ceil(T/8) .. floor(T/2)} tokens, and
    each sequence ends with D ~ U{0 .. floor(T/4)} padding tokens; prompt and
    padding are ignore_index, the response tokens between them get uniform
    labels.  X ~ N(0, 1), W ~ N(0, w_std^2) as in the other workloads.  Draw
    order: X, W, labels, prompt lengths, padding lengths."""
    N = 2 * n_pairs * T
    wl = Workload("pairs", N, H, V, dtype, 0, ignore_mode="none", w_std=w_std)
    ss = np.random.SeedSequence(seed)
    s_x, s_w, s_y, s_p, s_d = ss.spawn(5)
    X = _draw_X(np.random.default_rng(s_x), N, H, "normal", dtype)
    W = _draw_W(s_w, V, H, w_std, dtype)
    y = _draw_labels(np.random.default_rng(s_y), N, V, "uniform", 0.0).reshape(2 * n_pairs, T)
    P = _prompt_lengths(np.random.default_rng(s_p), T, n_pairs)
    D = np.random.default_rng(s_d).integers(0, T // 4 + 1, size=2 * n_pairs)
    for s_ in range(2 * n_pairs):
        y[s_, :P[s_ % n_pairs]] = IGNORE_INDEX
        if D[s_]:
            y[s_, T - D[s_]:] = IGNORE_INDEX
    return Inputs(wl, X, W, y.reshape(-1), seed)


def make_unpaired(n_seq: int, T: int, H: int, V: int, dtype: str = "bf16", seed: int = 1,
                  w_std: float = 0.02):
    """Unpaired preference batch: n_seq sequences of T tokens as rows of X,
    each with its own prompt of U{ceil(T/8) .. floor(T/2)} and padding of
    U{0 .. floor(T/4)} unscored tokens (labels as make_pairs), a desirability
    flag (half of the sequences, by a seeded permutation) and a reference
    log-probability sum R ~ N(-n_s (ln V + w_std^2 H / 2), (2 sqrt(n_s))^2)
    for its n_s scored tokens: centred on what a head drawn this way gives
    (logits of variance w_std^2 H), so rewards are of order sqrt(n_s).  Returns (Inputs, desirable int32 [n_seq], R float32 [n_seq]).
    Draw order: X, W, labels, prompt lengths, padding lengths, flags, R."""
    N = n_seq * T
    wl = Workload("unpaired", N, H, V, dtype, 0, ignore_mode="none", w_std=w_std)
    ss = np.random.SeedSequence(seed)
    s_x, s_w, s_y, s_p, s_d, s_f, s_r = ss.spawn(7)
    X = _draw_X(np.random.default_rng(s_x), N, H, "normal", dtype)
    W = _draw_W(s_w, V, H, w_std, dtype)
    y = _draw_labels(np.random.default_rng(s_y), N, V, "uniform", 0.0).reshape(n_seq, T)
    P = _prompt_lengths(np.random.default_rng(s_p), T, n_seq)
    D = np.random.default_rng(s_d).integers(0, T // 4 + 1, size=n_seq)
    for s_ in range(n_seq):
        y[s_, :P[s_]] = IGNORE_INDEX
        if D[s_]:
            y[s_, T - D[s_]:] = IGNORE_INDEX
    des = np.zeros(n_seq, dtype=np.int32)
    des[np.random.default_rng(s_f).permutation(n_seq)[: n_seq // 2]] = 1
    n_s = (y != IGNORE_INDEX).sum(axis=1)
    R = (-(np.log(V) + 0.5 * w_std * w_std * H) * n_s + 2.0 * np.sqrt(n_s) *
         np.random.default_rng(s_r).standard_normal(n_seq)).astype(np.float32)
    return Inputs(wl, X, W, y.reshape(-1), seed), des, R


def share_of(inp: Inputs, share: str) -> Inputs:
    """One GPU's share of a workload sharded over 8 GPUs: "dp8" keeps the
    first N/8 tokens with the whole head; "tp8" keeps every token against the
    first ceil(V/8) vocabulary rows, with labels reduced modulo that count so
    that the call is a valid loss on the shard (its work is the shard's)."""
    wl = inp.wl
    if share == "dp8":
        n = wl.N // 8
        return dataclasses.replace(inp, wl=dataclasses.replace(wl, name=f"{wl.name}-dp8-share",
                                                               N=n),
                                   X=inp.X[:n], labels=inp.labels[:n].copy())
    if share != "tp8":
        raise ValueError(f"unknown share {share!r}")
    v = (wl.V + 7) // 8
    y = inp.labels.copy()
    y[y != IGNORE_INDEX] %= v
    return dataclasses.replace(inp, wl=dataclasses.replace(wl, name=f"{wl.name}-tp8-share", V=v),
                               W=np.ascontiguousarray(inp.W[:v]), labels=y)


def sample_rows(n_total: int, k: int, seed: int, must: tuple = ()) -> np.ndarray:
    """Seeded sorted sample of k distinct row indices, always holding ``must``."""
    rng = np.random.default_rng(seed)
    k = min(k, n_total)
    pick = set(int(m) for m in must if 0 <= m < n_total)
    rest = rng.permutation(n_total)
    for r in rest:
        if len(pick) >= k:
            break
        pick.add(int(r))
    return np.array(sorted(pick), dtype=np.int64)
