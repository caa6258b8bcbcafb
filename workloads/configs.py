"""The five decode workloads of the EntmaxKV benchmark, as seeded generators.

Every random stream is keyed by (seed, tag, b, g) through numpy's
SeedSequence/PCG64, so any (sequence, KV head) slice can be regenerated on
its own: the CPU oracle regenerates one slice while the GPU side uploads all
of them, and both see the same bytes.

Recipes (shapes follow the decode regimes the EntmaxKV pages describe:
long contexts, small KV budgets; the benchmarks they use are not available,
these synthetic inputs stand in for them):
  c1  tiny: B=1, 1/1 heads, d=64, L=4096, P=16, fp32 K/V ~ N(0,1), q ~ 2N(0,1),
      16 needles k = 3 q/|q| + 0.1 N(0,I), alpha=1.5, bbox top-32.
  c2  B=1, 32/8 heads, d=128, L=32768, P=16, bf16 K/V ~ N(0,1),
      64 needles per KV head aligned round-robin to the group's query heads,
      alpha=1.5, bbox top-64.
  c3  B=4, 32/8, d=128, L=131072, P=32, bf16 keys from 64 Gaussian clusters
      (centres ~ N(0,I), sigma 0.3, runs of 256 tokens), V ~ N(0,1),
      alpha=2, Gaussian selector with margin 0.5.
  c4  B=1, 32/8, d=128, L=2^20, P=64, bf16, 256 needles per KV head,
      alpha=1.5, bbox top-328 (2% of 16384 pages).
  c5  B=16, 32/8, d=128, L_b ~ U{16384..65536}, P=16, randomly permuted
      physical pages, clustered keys as c3, alpha=1.5, Gaussian selector,
      64 decode steps each appending one token per sequence.
  c4g the million-token shape of c4 with c3's clustered keys and the
      Gaussian selector (margin 0.5), alpha=1.5: the selector the pages
      report their million-token speedups for, on keys it can separate
      (on isotropic keys it keeps almost nothing).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np

CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5", "c4g")

# stream tags
_T_Q, _T_K, _T_V, _T_NEEDLE_POS, _T_NEEDLE_NOISE, _T_CENTRES, _T_RUNS, _T_LENS, _T_PERM = range(9)


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: str            # "f32" or "bf16"
    alpha: float
    policy: str              # "bbox" or "gauss"
    top_k: int = 0
    delta: float = 0.5
    min_pages: int = 1       # Gaussian selector: fewest pages kept per unit
    key_kind: str = "needles"  # "needles" or "clusters"
    n_needles: int = 0       # per KV head
    needle_amp: float = 3.0
    needle_noise: float = 0.1
    n_centres: int = 64
    cluster_sigma: float = 0.3
    run_len: int = 256
    q_scale: float = 2.0
    context: int = 0         # fixed initial length when > 0
    ctx_lo: int = 0          # otherwise uniform integer in [ctx_lo, ctx_hi]
    ctx_hi: int = 0
    permute_pages: bool = False
    steps: int = 0           # tokens appended per sequence (one per decode step)
    seed: int = 1000

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.kv_dtype == "f32" else 2

    def with_(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)


_BASE = {
    "c1": WorkloadSpec("c1", 1, 1, 1, 64, 16, "f32", 1.5, "bbox", top_k=32,
                       key_kind="needles", n_needles=16, context=4096, seed=1000),
    "c2": WorkloadSpec("c2", 1, 32, 8, 128, 16, "bf16", 1.5, "bbox", top_k=64,
                       key_kind="needles", n_needles=64, context=32768, seed=1001),
    "c3": WorkloadSpec("c3", 4, 32, 8, 128, 32, "bf16", 2.0, "gauss", delta=0.5,
                       key_kind="clusters", context=131072, seed=1002),
    "c4": WorkloadSpec("c4", 1, 32, 8, 128, 64, "bf16", 1.5, "bbox", top_k=328,
                       key_kind="needles", n_needles=256, context=1 << 20, seed=1003),
    "c5": WorkloadSpec("c5", 16, 32, 8, 128, 16, "bf16", 1.5, "gauss", delta=0.5,
                       key_kind="clusters", ctx_lo=16384, ctx_hi=65536,
                       permute_pages=True, steps=64, seed=1004),
    "c4g": WorkloadSpec("c4g", 1, 32, 8, 128, 64, "bf16", 1.5, "gauss", delta=0.5,
                        key_kind="clusters", context=1 << 20, seed=1005),
}


def make_spec(name: str, **overrides) -> WorkloadSpec:
    """Full-size spec of a workload, optionally with fields overridden
    (shorter contexts or fewer heads for quick parity cases)."""
    return _BASE[name].with_(**overrides)


def _rng(spec: WorkloadSpec, tag: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([spec.seed, tag, *ids])))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (storage format only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _store(x: np.ndarray, spec: WorkloadSpec) -> np.ndarray:
    if spec.kv_dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    return round_to_bf16_bits(x)


def seq_lens(spec: WorkloadSpec) -> np.ndarray:
    """Initial (pre-decode) sequence lengths, int32 [B]."""
    if spec.context > 0:
        return np.full(spec.batch, spec.context, dtype=np.int32)
    r = _rng(spec, _T_LENS)
    return r.integers(spec.ctx_lo, spec.ctx_hi + 1, size=spec.batch).astype(np.int32)


def total_lens(spec: WorkloadSpec) -> np.ndarray:
    return seq_lens(spec) + np.int32(spec.steps)


def max_pages(spec: WorkloadSpec) -> int:
    tl = total_lens(spec)
    return int(max(-(-int(t) // spec.page_size) for t in tl))


def page_table(spec: WorkloadSpec) -> tuple[np.ndarray, int]:
    """Logical->physical page table int32 [B][max_pages] (-1 where unused)
    and the physical pool size.  Identity-blocked layout unless the spec asks
    for a seeded random permutation of the pool."""
    P = spec.page_size
    mp = max_pages(spec)
    tl = total_lens(spec)
    need = [-(-int(t) // P) for t in tl]
    table = np.full((spec.batch, mp), -1, dtype=np.int32)
    if not spec.permute_pages:
        for b in range(spec.batch):
            table[b, : need[b]] = b * mp + np.arange(need[b], dtype=np.int32)
        return table, spec.batch * mp
    n_phys = int(sum(need))
    perm = _rng(spec, _T_PERM).permutation(n_phys).astype(np.int32)
    off = 0
    for b in range(spec.batch):
        table[b, : need[b]] = perm[off : off + need[b]]
        off += need[b]
    return table, n_phys


def queries(spec: WorkloadSpec, step: int = 0) -> np.ndarray:
    """Decode queries, fp32 [B][Hq][d]: q = q_scale * N(0, I)."""
    r = _rng(spec, _T_Q, step)
    q = r.standard_normal((spec.batch, spec.n_q_heads, spec.head_dim), dtype=np.float32)
    return (q * np.float32(spec.q_scale)).astype(np.float32)


def _keys_f32(spec: WorkloadSpec, b: int, g: int) -> np.ndarray:
    L0 = int(seq_lens(spec)[b])
    n = L0 + spec.steps
    d = spec.head_dim
    if spec.key_kind == "clusters":
        centres = _rng(spec, _T_CENTRES, b, g).standard_normal((spec.n_centres, d), dtype=np.float32)
        n_runs = -(-n // spec.run_len)
        run_c = _rng(spec, _T_RUNS, b, g).integers(0, spec.n_centres, size=n_runs)
        k = _rng(spec, _T_K, b, g).standard_normal((n, d), dtype=np.float32)
        k *= np.float32(spec.cluster_sigma)
        k += centres[np.repeat(run_c, spec.run_len)[:n]]
        return k
    k = _rng(spec, _T_K, b, g).standard_normal((n, d), dtype=np.float32)
    if spec.n_needles > 0:
        q = queries(spec, 0)[b]
        pos = _rng(spec, _T_NEEDLE_POS, b, g).choice(L0, size=spec.n_needles, replace=False)
        noise = _rng(spec, _T_NEEDLE_NOISE, b, g).standard_normal((spec.n_needles, d), dtype=np.float32)
        G = spec.group
        for i in range(spec.n_needles):
            qh = q[g * G + (i % G)].astype(np.float64)
            dirn = qh / np.linalg.norm(qh)
            k[pos[i]] = (spec.needle_amp * dirn + spec.needle_noise * noise[i]).astype(np.float32)
    return k


def needle_positions(spec: WorkloadSpec, b: int, g: int) -> np.ndarray:
    if spec.key_kind != "needles" or spec.n_needles == 0:
        return np.zeros(0, dtype=np.int64)
    L0 = int(seq_lens(spec)[b])
    return np.sort(_rng(spec, _T_NEEDLE_POS, b, g).choice(L0, size=spec.n_needles, replace=False))


def keys(spec: WorkloadSpec, b: int, g: int) -> np.ndarray:
    """Keys of sequence b, KV head g, all L_b + steps tokens, in storage
    format ([n][d] float32, or uint16 bf16 bit patterns)."""
    return _store(_keys_f32(spec, b, g), spec)


def values(spec: WorkloadSpec, b: int, g: int) -> np.ndarray:
    L0 = int(seq_lens(spec)[b])
    n = L0 + spec.steps
    v = _rng(spec, _T_V, b, g).standard_normal((n, spec.head_dim), dtype=np.float32)
    return _store(v, spec)
