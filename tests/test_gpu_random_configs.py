"""GPU parity over seeded random configurations (decode and chunked prefill).

The fixed cases of the other GPU tests pick shapes by hand; these draw them
from the whole supported space with one fixed seed, so that a combination no
one thought of (three KV heads with eight query heads each, fp32 pages with
128-token blocks and an odd top_k, a ragged batch where some sequences are
shorter than top_k blocks ...) is still compared with the oracle.  Every
draw is printed before it runs, and the list is the same on every run.

Decode cases: batch 1-5 with ragged lengths (1 .. 12000 tokens, some below
top_k blocks so that every block is selected), query heads per KV head
1/2/4/8, 1-3 KV heads, head dim 64/128, block 64/128, top_k 2-48, bf16 or
fp32 pages, the four input kinds, identity or shuffled pages, the plain and
the fused decode step, fused or split selection, sometimes chunk appends.
Prefill cases: 1-600 tokens through one spla_prefill call after a random
prefix, in groups of 16-256 tokens.
Long cases: one per keys-per-thread size of the selectors from 2 to 32
(each a template instance of its own): a single sequence whose candidate
count falls well inside that size's range (up to 8192 candidates, about 1M
tokens), one KV head of head dim 64, top_k 2-256, the fused and the split
selection in turn.
"""
import random

import pytest

from tests.test_gpu_parity import _needs_gpu
from workloads import Workload

pytestmark = pytest.mark.gpu

N_DECODE = 40
N_PREFILL = 20


def _draw_workload(rnd: random.Random, i: int, max_len: int, prefill: bool) -> Workload:
    r = rnd.choice([1, 2, 4, 8])
    g = rnd.choice([1, 2, 3])
    d = rnd.choice([64, 128])
    bk = rnd.choice([64, 128])
    top_k = rnd.randint(2, 48)
    dtype = rnd.choice(["bf16", "bf16", "f32"])
    batch = rnd.choice([1, 2]) if prefill else rnd.choice([1, 1, 2, 3, 5])
    kind = rnd.choice(["normal", "outlier", "planted", "mixture"])
    lens = []
    for _ in range(batch):
        if rnd.random() < 0.25:
            lens.append(rnd.randint(1, top_k * bk))  # every block selected
        else:
            lens.append(rnd.randint(1, max_len))
    kw = {}
    if kind == "planted":
        n_plant = rnd.randint(1, 4)
        lens = [max(t, (n_plant + 2) * bk + 1) for t in lens]
        kw = dict(n_plant=n_plant, plant_shared_heads=rnd.random() < 0.5)
    elif kind == "outlier":
        kw = dict(n_outlier=rnd.randint(1, 8), outlier_scale=4.0)
    chunk_seqs = rnd.choice([0, 0, 1, min(2, batch)]) if not prefill else 0
    return Workload(name=f"rand{'p' if prefill else 'd'}{i}", batch=batch, n_q_heads=r * g, n_kv_heads=g,
                    head_dim=d, block_size=bk, top_k=top_k, kv_dtype=dtype, t0=tuple(lens), steps=3,
                    kind=kind, seed=5000 + i, chunk_seqs=chunk_seqs,
                    chunk_len=rnd.randint(1, 200) if chunk_seqs else 0, **kw)


def _decode_cases():
    rnd = random.Random(20261203)
    out = []
    for i in range(N_DECODE):
        w = _draw_workload(rnd, i, 12000, prefill=False)
        out.append((w, rnd.choice(["identity", "shuffled"]), rnd.random() < 0.5, rnd.choice([-1, 0, 1])))
    return out


def _prefill_cases():
    rnd = random.Random(20261204)
    out = []
    for i in range(N_PREFILL):
        w = _draw_workload(rnd, i, 6000, prefill=True)
        seq = rnd.randrange(w.batch)
        n = rnd.randint(1, min(600, w.t0[seq]))
        out.append((w, seq, w.t0[seq] - n, rnd.choice([16, 17, 64, 100, 256])))
    return out


# keys-per-thread sizes of the selectors, in order; a selection of nc
# candidates runs the smallest size K with 256 K >= nc
SEL_SIZES = [1, 2, 3, 4, 6, 8, 9, 10, 12, 16, 20, 24, 32]


def _long_cases():
    rnd = random.Random(20261205)
    out = []
    for i in range(1, len(SEL_SIZES)):
        lo, hi = 256 * SEL_SIZES[i - 1], 256 * SEL_SIZES[i]
        nc = rnd.randint(lo + 32, hi - 32)  # candidates after the steps' appends stay inside (lo, hi]
        bk = 64 if SEL_SIZES[i] <= 12 else 128
        t0 = (nc + 2) * bk - rnd.randint(8, bk - 1) - 3
        w = Workload(name=f"randl{SEL_SIZES[i]}", batch=1, n_q_heads=rnd.choice([1, 2, 4, 8]), n_kv_heads=1,
                     head_dim=64, block_size=bk, top_k=rnd.randint(2, 256),
                     kv_dtype=rnd.choice(["bf16", "f32"]), t0=(t0,), steps=2,
                     kind=rnd.choice(["normal", "mixture"]), seed=7000 + i)
        out.append((w, rnd.choice(["identity", "shuffled"]), rnd.random() < 0.5, i % 2))
    return out


DECODE = _decode_cases()
PREFILL = _prefill_cases()
LONG = _long_cases()


@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode_config(i):
    _needs_gpu()
    from tests.spla_parity import ParityRun
    w, pages, use_step, fused = DECODE[i]
    print(f"[case] {w.name} B={w.batch} H={w.n_q_heads} G={w.n_kv_heads} d={w.head_dim} Bk={w.block_size} "
          f"k={w.top_k} {w.kv_dtype} kind={w.kind} t0={w.t0} chunks={w.chunk_seqs}x{w.chunk_len} "
          f"pages={pages} step={use_step} fused={fused}", flush=True)
    run = ParityRun(w, page_order=pages, prefill_chunk=1000, use_step=use_step, fused_select=fused)
    failures = run.run(verbose=True)
    assert not failures, "\n".join(failures[:20])


@pytest.mark.parametrize("i", range(N_PREFILL))
def test_random_prefill_config(i):
    from tests.test_gpu_prefill import _prefill_case
    w, seq, split, chunk = PREFILL[i]
    _prefill_case(w, seq, split, chunk=chunk)


@pytest.mark.parametrize("i", range(len(SEL_SIZES) - 1))
def test_random_long_config(i):
    _needs_gpu()
    from tests.spla_parity import ParityRun
    w, pages, use_step, fused = LONG[i]
    nb = -(-w.t0[0] // w.block_size)
    print(f"[case] {w.name} H={w.n_q_heads} G=1 d={w.head_dim} Bk={w.block_size} k={w.top_k} {w.kv_dtype} "
          f"kind={w.kind} t0={w.t0[0]} candidates={nb - 2}.. pages={pages} step={use_step} fused={fused}", flush=True)
    run = ParityRun(w, page_order=pages, prefill_chunk=65536, use_step=use_step, fused_select=fused)
    failures = run.run(verbose=True)
    assert not failures, "\n".join(failures[:20])
