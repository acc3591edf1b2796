"""Seeded synthetic inputs for the SPLA decode step.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no block statistics, scores, selection, attention or
linear-attention state).  Both the fp64 oracle (``oracle/``) and the HIP
library are fed from here, so the two sides see bit-identical inputs.

Every array is returned as float32.  For bf16 workloads the values are
rounded to bf16 (round to nearest, ties to even) once, here, so a float32
array holds exactly the bf16 value the GPU stores and the oracle widens the
same value to fp64.

Streams: every draw comes from ``numpy.random.default_rng([seed, stream,
i, j])`` with a fixed stream id per purpose, so a chunk of a prefill can be
regenerated on its own and the recipe does not depend on how the caller
iterates.

The five named workloads stand in for the long-context decode settings the
SPLA pages discuss (contexts 4K..1M around their 256K RULER setting,
Llama-style GQA 32/8 x 128).  No benchmark-suite item is reproduced; the
inputs are random numbers with the shapes and structure listed per preset.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

__all__ = [
    "round_bf16",
    "bf16_bits",
    "Workload",
    "WORKLOADS",
    "make_workload",
]

# stream ids (fixed; changing one changes the recipe)
_S_PREFILL_K = 1
_S_PREFILL_V = 2
_S_STEP_Q = 3
_S_STEP_KV = 4
_S_PLANT = 5
_S_GATE = 6
_S_LENS = 7
_S_CHUNK_PICK = 8
_S_CHUNK_KV = 9
_S_OUTLIER = 10
_S_MIXTURE = 11
_S_QBASE = 12
_S_RLA_GAMMA = 13
_S_PREFILL_Q = 14


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return float32.

    Finite inputs only (the generators never produce inf/nan)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    u = ((u + bias) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _rng(seed: int, stream: int, *idx: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)] + [int(i) for i in idx])


@dataclass(frozen=True)
class Workload:
    """Shape + distribution recipe of one synthetic decode workload.

    kind:
      ``normal``   K, V ~ N(0, 1)
      ``outlier``  K, V ~ N(0, 1), then per KV head ``n_outlier`` seeded
                   channels scaled by ``outlier_scale`` in both K and V
      ``planted``  K, V ~ N(0, 1) plus ``n_plant`` planted blocks per sequence
                   whose keys are 3*u + plant_noise*N(0, I) (plant_noise 0.1
                   by default), u the unit direction of the sequence/KV
                   head's base query q0; step queries are q0 + 0.25*N(0, I)
      ``mixture``  keys c_m(i) + 0.3*N(0, I) with 64 centres c_m ~ N(0, I) per
                   KV head and m(i) constant over runs of length
                   round(exp(U[ln 16, ln 2048])), centre uniform per run;
                   V ~ N(0, 1)
    """

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    top_k: int
    kv_dtype: str  # "f32" | "bf16"
    t0: Tuple[int, ...]  # prefill length per sequence
    steps: int
    kind: str = "normal"
    seed: int = 1000
    # planted
    n_plant: int = 0
    plant_shared_heads: bool = True
    plant_noise: float = 0.1  # 0: every planted block of a head holds the same keys (tied scores)
    # outlier
    n_outlier: int = 0
    outlier_scale: float = 4.0
    # gate
    gate_ones: bool = False
    # chunked appends per step (ragged serving preset)
    chunk_seqs: int = 0
    chunk_len: int = 0
    prefill_chunk: int = 4096
    extra_capacity_tokens: int = 0

    # ---------------------------------------------------------------- shape
    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def max_tokens(self, steps: Optional[int] = None) -> int:
        steps = self.steps if steps is None else steps
        per_step = 1 + (self.chunk_len if self.chunk_seqs else 0)
        return max(self.t0) + steps * per_step + self.extra_capacity_tokens

    def max_blocks_per_seq(self, steps: Optional[int] = None) -> int:
        return -(-self.max_tokens(steps) // self.block_size)

    def round(self, x: np.ndarray) -> np.ndarray:
        x = np.asarray(x, dtype=np.float32)
        return round_bf16(x) if self.kv_dtype == "bf16" else np.ascontiguousarray(x)

    # ------------------------------------------------------------- helpers
    def _outlier_scale_vec(self) -> np.ndarray:
        """[G][d] per-channel multiplier (1 or outlier_scale)."""
        s = np.ones((self.n_kv_heads, self.head_dim), np.float32)
        if self.n_outlier:
            r = _rng(self.seed, _S_OUTLIER)
            for g in range(self.n_kv_heads):
                ch = r.choice(self.head_dim, self.n_outlier, replace=False)
                s[g, ch] = self.outlier_scale
        return s

    def q_base(self) -> np.ndarray:
        """[B][G][d] base query directions of the planted preset (float32)."""
        r = _rng(self.seed, _S_QBASE)
        return r.standard_normal((self.batch, self.n_kv_heads, self.head_dim)).astype(np.float32)

    def planted_blocks(self) -> np.ndarray:
        """[B][G][n_plant] planted block ids (distinct, in 1..t0/Bk - 1)."""
        out = np.zeros((self.batch, self.n_kv_heads, self.n_plant), np.int64)
        for b in range(self.batch):
            nfull = self.t0[b] // self.block_size
            r = _rng(self.seed, _S_PLANT, b)
            if self.plant_shared_heads:
                ids = np.sort(r.choice(np.arange(1, nfull), self.n_plant, replace=False))
                out[b, :, :] = ids[None, :]
            else:
                for g in range(self.n_kv_heads):
                    out[b, g] = np.sort(r.choice(np.arange(1, nfull), self.n_plant, replace=False))
        return out

    def _mixture(self) -> Tuple[np.ndarray, List[np.ndarray]]:
        """centres [G][64][d] and, per KV head, the centre id of every token."""
        r = _rng(self.seed, _S_MIXTURE)
        centres = r.standard_normal((self.n_kv_heads, 64, self.head_dim)).astype(np.float32)
        total = self.max_tokens()
        ids = []
        for g in range(self.n_kv_heads):
            rg = _rng(self.seed, _S_MIXTURE, g)
            m = np.empty(total, np.int32)
            pos = 0
            while pos < total:
                run = int(round(math.exp(rg.uniform(math.log(16.0), math.log(2048.0)))))
                m[pos:pos + run] = rg.integers(0, 64)
                pos += run
            ids.append(m)
        return centres, ids

    # ---------------------------------------------------------------- draws
    def gate(self) -> np.ndarray:
        """[H] per-query-head gate g_h (float32)."""
        if self.gate_ones:
            return np.ones(self.n_q_heads, np.float32)
        return _rng(self.seed, _S_GATE).uniform(0.0, 1.0, self.n_q_heads).astype(np.float32)

    def prefill_queries(self, b: int, pos0: int, n: int) -> np.ndarray:
        """[n][H][d] queries of prefill positions pos0 .. pos0 + n - 1 of sequence
        b, distributed like the decode steps' queries; drawn per prefill_chunk
        unit so any split regenerates the same values."""
        unit = self.prefill_chunk
        out = []
        p = pos0
        while p < pos0 + n:
            ui = p // unit
            lo = p - ui * unit
            take = min(unit - lo, pos0 + n - p)
            noise = _rng(self.seed, _S_PREFILL_Q, b, ui).standard_normal(
                (unit, self.n_q_heads, self.head_dim)).astype(np.float32)[lo:lo + take]
            if self.kind == "planted":
                gidx = np.arange(self.n_q_heads) // self.group
                noise = self.q_base()[b][gidx][None] + np.float32(0.25) * noise
            out.append(noise)
            p += take
        return self.round(np.concatenate(out, 0))

    def rla_gamma(self) -> np.ndarray:
        """[H][d] scale of the RMS-normalised RLA branch (float32, U(0.5, 1.5));
        a stand-in for trained norm weights, which are not available."""
        return _rng(self.seed, _S_RLA_GAMMA).uniform(0.5, 1.5, (self.n_q_heads, self.head_dim)).astype(np.float32)

    def _keys(self, r: np.random.Generator, b: int, pos0: int, n: int, mix=None) -> np.ndarray:
        G, d = self.n_kv_heads, self.head_dim
        if self.kind == "mixture":
            centres, ids = mix
            noise = r.standard_normal((n, G, d)).astype(np.float32)
            k = np.empty((n, G, d), np.float32)
            for g in range(G):
                k[:, g, :] = centres[g][ids[g][pos0:pos0 + n]] + np.float32(0.3) * noise[:, g, :]
            return k
        return r.standard_normal((n, G, d)).astype(np.float32)

    def prefill_chunks(self, b: int, chunk: Optional[int] = None) -> Iterator[Tuple[int, np.ndarray, np.ndarray]]:
        """Yield (pos0, K [n][G][d], V [n][G][d]) covering sequence b's prefill."""
        chunk = chunk or self.prefill_chunk
        mix = self._mixture() if self.kind == "mixture" else None
        scale = self._outlier_scale_vec() if self.kind == "outlier" else None
        if self.kind == "planted":
            u = self.q_base()[b]
            u = u / np.linalg.norm(u, axis=-1, keepdims=True)
            plant = self.planted_blocks()[b]
        # chunks are drawn in units of prefill_chunk tokens so any chunking
        # of the caller regenerates the same values
        unit = self.prefill_chunk
        t0 = self.t0[b]
        for pos0 in range(0, t0, chunk):
            n = min(chunk, t0 - pos0)
            ks, vs = [], []
            p = pos0
            while p < pos0 + n:
                ui = p // unit
                lo = p - ui * unit
                take = min(unit - lo, pos0 + n - p)
                un = min(unit, t0 - ui * unit)
                rk = _rng(self.seed, _S_PREFILL_K, b, ui)
                rv = _rng(self.seed, _S_PREFILL_V, b, ui)
                kk = self._keys(rk, b, ui * unit, un, mix)
                vv = rv.standard_normal((un, self.n_kv_heads, self.head_dim)).astype(np.float32)
                ks.append(kk[lo:lo + take])
                vs.append(vv[lo:lo + take])
                p += take
            k = np.concatenate(ks, 0)
            v = np.concatenate(vs, 0)
            if scale is not None:
                k = k * scale[None]
                v = v * scale[None]
            if self.kind == "planted":
                bk = self.block_size
                for g in range(self.n_kv_heads):
                    for j in plant[g]:
                        a, e = max(j * bk, pos0), min((j + 1) * bk, pos0 + n)
                        if a >= e:
                            continue
                        rp = _rng(self.seed, _S_PLANT, b, g, int(j))
                        noise = rp.standard_normal((bk, self.head_dim)).astype(np.float32)
                        k[a - pos0:e - pos0, g, :] = (np.float32(3.0) * u[g][None, :]
                                                      + np.float32(self.plant_noise) * noise[a - j * bk:e - j * bk])
            yield pos0, self.round(k), self.round(v)

    def prefill(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        ks, vs = [], []
        for _, k, v in self.prefill_chunks(b):
            ks.append(k)
            vs.append(v)
        if not ks:
            z = np.zeros((0, self.n_kv_heads, self.head_dim), np.float32)
            return z, z.copy()
        return np.concatenate(ks, 0), np.concatenate(vs, 0)

    def chunk_plan(self, s: int) -> np.ndarray:
        """Sequence ids that get a chunk append at step s (sorted, distinct)."""
        if not self.chunk_seqs:
            return np.zeros(0, np.int64)
        r = _rng(self.seed, _S_CHUNK_PICK, s)
        return np.sort(r.choice(self.batch, self.chunk_seqs, replace=False))

    def step(self, s: int, mix=None) -> Dict[str, np.ndarray]:
        """Inputs of decode step s.

        Returns a dict with
          chunk_seqs [c]              sequences getting a chunk append first
          chunk_k, chunk_v [c*L][G][d] their chunk rows, sequence-major
          k, v [B][G][d]              the decoded token of every sequence
          q [B][H][d]                 the queries
        """
        B, H, G, d = self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim
        out: Dict[str, np.ndarray] = {}
        cs = self.chunk_plan(s)
        out["chunk_seqs"] = cs
        if len(cs):
            rc = _rng(self.seed, _S_CHUNK_KV, s)
            out["chunk_k"] = self.round(rc.standard_normal((len(cs) * self.chunk_len, G, d)).astype(np.float32))
            out["chunk_v"] = self.round(rc.standard_normal((len(cs) * self.chunk_len, G, d)).astype(np.float32))
        else:
            out["chunk_k"] = np.zeros((0, G, d), np.float32)
            out["chunk_v"] = np.zeros((0, G, d), np.float32)
        rkv = _rng(self.seed, _S_STEP_KV, s)
        if self.kind == "mixture":
            if mix is None:
                mix = self._mixture()
            centres, ids = mix
            noise = rkv.standard_normal((B, G, d)).astype(np.float32)
            k = np.empty((B, G, d), np.float32)
            for b in range(B):
                pos = self.t0[b] + s
                for g in range(G):
                    k[b, g] = centres[g][ids[g][pos]] + np.float32(0.3) * noise[b, g]
        else:
            k = rkv.standard_normal((B, G, d)).astype(np.float32)
        v = rkv.standard_normal((B, G, d)).astype(np.float32)
        if self.kind == "outlier":
            sc = self._outlier_scale_vec()
            k = k * sc[None]
            v = v * sc[None]
        out["k"] = self.round(k)
        out["v"] = self.round(v)
        rq = _rng(self.seed, _S_STEP_Q, s)
        noise = rq.standard_normal((B, H, d)).astype(np.float32)
        if self.kind == "planted":
            q0 = self.q_base()  # [B][G][d]
            gidx = np.arange(H) // self.group
            q = q0[:, gidx, :] + np.float32(0.25) * noise
        else:
            q = noise
        out["q"] = self.round(q)
        return out

    def mixture_state(self):
        return self._mixture() if self.kind == "mixture" else None

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


def _ragged_lens(seed: int, batch: int) -> Tuple[int, ...]:
    r = _rng(seed, _S_LENS)
    u = r.uniform(math.log(2048.0), math.log(65536.0), batch)
    return tuple(int(math.floor(math.exp(x))) for x in u)


def _presets() -> Dict[str, Workload]:
    w = {}
    w["tiny_fp32"] = Workload(
        name="tiny_fp32", batch=1, n_q_heads=2, n_kv_heads=2, head_dim=64, block_size=64,
        top_k=8, kv_dtype="f32", t0=(4096,), steps=16, kind="planted", seed=1001,
        n_plant=4, plant_shared_heads=False, gate_ones=True)
    w["llama_gqa_128k"] = Workload(
        name="llama_gqa_128k", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=64,
        top_k=32, kv_dtype="bf16", t0=(131072,), steps=256, kind="outlier", seed=1002,
        n_outlier=8, outlier_scale=4.0)
    w["batched_32k"] = Workload(
        name="batched_32k", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=64,
        top_k=32, kv_dtype="bf16", t0=(32768,) * 16, steps=128, kind="planted", seed=1003,
        n_plant=16, plant_shared_heads=True)
    w["million_1m"] = Workload(
        name="million_1m", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=128,
        top_k=64, kv_dtype="bf16", t0=(1048576,), steps=64, kind="mixture", seed=1004)
    w["ragged_chunked"] = Workload(
        name="ragged_chunked", batch=64, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=64,
        top_k=16, kv_dtype="bf16", t0=_ragged_lens(1005, 64), steps=64, kind="normal", seed=1005,
        chunk_seqs=8, chunk_len=256)
    return w


WORKLOADS: Dict[str, Workload] = _presets()


def make_workload(name: str, **overrides) -> Workload:
    """A named preset, optionally with fields overridden (smaller contexts for tests)."""
    return replace(WORKLOADS[name], **overrides)
