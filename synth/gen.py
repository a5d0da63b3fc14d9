"""Seeded generators for expert blobs, router logits and activations.

Every stream is keyed by a numpy SeedSequence built from (workload seed, purpose,
index), so that any single expert, layer or step can be regenerated on its own
(the oracle recomputes a sampled step without replaying the whole run).

Value recipes:
  * FP4 codes: uniform over the 16 nibbles (uniform random bytes).
  * Block scales: |N(0, 0.02)| rounded to nearest-even into FP8 E4M3 (OCP "FN"
    variant; subnormals and zero allowed, never the NaN code).
  * Global scales: 1.0 ("unit") or U[0.5, 2] rounded to fp32 ("uniform").
  * Activations: N(0, 1) rounded to nearest-even bf16 (stored as uint16 bits).
  * Router logits: i.i.d. N(0, 1) ("normal"), or Zipf(1.1) popularity over a
    seeded expert permutation plus an AR(1) drift with coefficient 0.99 plus
    per-row Gumbel noise ("zipf"); Gumbel-top-k of those logits is
    Plackett-Luce sampling without replacement from the drifting popularity.
  * Drafted rows: rows 1..M-1 add +20 to three experts drawn from the eight
    largest logits of row 0, so that draft rows share about half their picks.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .configs import WorkloadConfig, blob_parts, blob_bytes, rows_at_step

_BLOB = 3000
_GS = 4000
_ROUTE = 1000
_ACT = 2000


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def e4m3_bits_rne(v):
    """Encode floats to OCP E4M3FN bytes, round-to-nearest-even, saturating at 448."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(v), 448.0)
    out = np.zeros(a.shape, dtype=np.uint8)
    sub = a < 2.0 ** -6
    # subnormal grid: multiples of 2^-9; a quotient of 8 lands on the smallest normal (0x08)
    out[sub] = np.rint(a[sub] * 512.0).astype(np.uint8)
    an = a[~sub]
    mant, ex = np.frexp(an)                      # an = mant * 2^ex, mant in [0.5, 1)
    e = ex.astype(np.int64) - 1                  # unbiased exponent
    m = np.rint((mant * 2.0 - 1.0) * 8.0).astype(np.int64)   # exact product, half-even
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code = ((e + 7) << 3) | m
    code = np.minimum(code, 0x7E)
    out[~sub] = code.astype(np.uint8)
    return out | sign


def bf16_bits_from_f32(x):
    """Round float32 values to bf16 (nearest-even), returned as uint16 bit patterns."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def expert_blob(cfg: WorkloadConfig, bank: int, expert: int, out=None) -> np.ndarray:
    """One expert's blob: [w13 codes | w13 scales | w2 codes | w2 scales] (uint8)."""
    nb = blob_bytes(cfg.hidden, cfg.inter)
    if out is None:
        out = np.empty(nb, dtype=np.uint8)
    rng = _rng(cfg.seed, _BLOB + bank, expert)
    off = 0
    for name, n in blob_parts(cfg.hidden, cfg.inter):
        if name.endswith("codes"):
            out[off:off + n] = rng.integers(0, 256, size=n, dtype=np.uint8)
        else:
            s = np.abs(rng.standard_normal(n, dtype=np.float32)) * np.float32(0.02)
            out[off:off + n] = e4m3_bits_rne(s)
        off += n
    return out


def expert_blobs(cfg: WorkloadConfig, bank: int, experts=None, out=None, threads=None) -> np.ndarray:
    """Blobs of several experts as a [len(experts), B_e] uint8 array (filled in place if `out`)."""
    if experts is None:
        experts = range(cfg.n_experts)
    experts = list(experts)
    nb = blob_bytes(cfg.hidden, cfg.inter)
    if out is None:
        out = np.empty((len(experts), nb), dtype=np.uint8)
    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda i: expert_blob(cfg, bank, experts[i], out=out[i]), range(len(experts))))
    return out


def global_scales(cfg: WorkloadConfig, bank: int, mode: str = "unit") -> np.ndarray:
    """Per-(expert, matrix) fp32 global scales, shape [E, 2] = (w13, w2)."""
    if mode == "unit":
        return np.ones((cfg.n_experts, 2), dtype=np.float32)
    if mode == "uniform":
        rng = _rng(cfg.seed, _GS + bank)
        return rng.uniform(0.5, 2.0, size=(cfg.n_experts, 2)).astype(np.float32)
    raise ValueError(mode)


def activations(cfg: WorkloadConfig, layer: int, step: int, rows: int) -> np.ndarray:
    """bf16 bit patterns [rows, hidden] of N(0,1) activations for one step."""
    rng = _rng(cfg.seed, _ACT + layer, step)
    return bf16_bits_from_f32(rng.standard_normal((rows, cfg.hidden), dtype=np.float32))


def routing_trace(cfg: WorkloadConfig, layer: int = 0, steps=None):
    """Router logits for a whole run of one layer.

    Returns (logits float32 [T, Mmax, E], rows int32 [T]); row m of step t is
    meaningful for m < rows[t] (the rest is zero).
    """
    T = cfg.steps if steps is None else steps
    E = cfg.n_experts
    rows = np.array([rows_at_step(cfg, t) for t in range(T)], dtype=np.int32)
    mmax = int(rows.max())
    out = np.zeros((T, mmax, E), dtype=np.float32)
    rng = _rng(cfg.seed, _ROUTE + layer)
    if cfg.routing == "normal":
        for t in range(T):
            out[t, :rows[t]] = rng.standard_normal((rows[t], E), dtype=np.float32)
        return out, rows
    if cfg.routing != "zipf":
        raise ValueError(cfg.routing)
    perm = rng.permutation(E)
    rank = np.empty(E, dtype=np.float64)
    rank[perm] = np.arange(1, E + 1)
    logp = -1.1 * np.log(rank)
    logp -= np.log(np.exp(logp).sum())
    rho = 0.99
    drift = rng.standard_normal(E)
    for t in range(T):
        drift = rho * drift + np.sqrt(1.0 - rho * rho) * rng.standard_normal(E)
        M = int(rows[t])
        u = rng.random((M, E))
        gumbel = -np.log(-np.log(np.clip(u, 1e-300, 1.0)))
        z = logp[None, :] + drift[None, :] + gumbel
        if cfg.drafted and 1 < M <= 16:
            top8 = np.argsort(-z[0], kind="stable")[:8]
            for m in range(1, M):
                share = rng.choice(top8, size=3, replace=False)
                z[m, share] += 20.0
        out[t, :M] = z.astype(np.float32)
    return out, rows


# E2M1 code of 1.0 (exponent field 1, mantissa 0) and E4M3 byte of 1.0 (exponent field 7).
_E2M1_ONE = 0x2
_E4M3_ONE = 0x38


def probe_column(cfg: WorkloadConfig, expert: int) -> int:
    """The intermediate index that a "one_column" probe blob of `expert` keeps."""
    return (expert * 37 + 5) % cfg.inter


def probe_blob(cfg: WorkloadConfig, bank: int, expert: int, mode: str) -> np.ndarray:
    """A seeded random blob with one matrix replaced by a structured one, so that a
    step's output exposes single weights instead of a long dot product.

    "select_h": the down matrix is a selection matrix: row r holds 1.0 at column
      r mod I and zero elsewhere (every block scale 1.0).  With one pick per row
      and a unit global scale the output row repeats the expert's intermediate
      vector.
    "one_column": every up row is zero except row probe_column(cfg, expert), so
      the intermediate vector is zero except at that index and the output is one
      column of the down matrix times one intermediate value.
    """
    out = expert_blob(cfg, bank, expert)
    H, I = cfg.hidden, cfg.inter
    parts = dict()
    off = 0
    for name, n in blob_parts(H, I):
        parts[name] = (off, n)
        off += n
    if mode == "select_h":
        o, n = parts["w2_codes"]
        codes = np.zeros((H, I), dtype=np.uint8)
        codes[np.arange(H), np.arange(H) % I] = _E2M1_ONE
        out[o:o + n] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).reshape(-1)
        o, n = parts["w2_scales"]
        out[o:o + n] = _E4M3_ONE
    elif mode == "one_column":
        o, n = parts["w13_codes"]
        w13 = out[o:o + n].reshape(2 * I, H // 2)
        keep = I + probe_column(cfg, expert)
        row = w13[keep].copy()
        w13[I:] = 0
        w13[keep] = row
    else:
        raise ValueError(mode)
    return out
