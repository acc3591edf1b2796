"""GPU parity of the selection-fidelity pieces against the fp64 oracle,
through the C ABI: the exact attention mass of every candidate block
(spla_block_mass: bf16 on the matrix cores, fp32 on the VALU; every group
ratio, both block sizes and head dims, a ragged batch whose short sequences
have no candidates), and the decode with the first-order mean-pooling score
(sets under the same tie rule, outputs, at small and full size)."""
import numpy as np
import pytest

from workloads import make_workload
from tests.test_gpu_parity import _needs_gpu, small

pytestmark = pytest.mark.gpu

MASS_ABS = 2e-5  # log domain: fp32 exp / log sums of 64-128 exact bf16 products
SENTINEL = -123.0


def _mass_case(w, kv_heads=None, seqs=None, steps=1, page_order="shuffled"):
    _needs_gpu()
    import torch
    from tests.spla_parity import ParityRun
    print(f"[case] block mass {w.name} B={w.batch} H={w.n_q_heads} G={w.n_kv_heads} d={w.head_dim} "
          f"Bk={w.block_size} dtype={w.kv_dtype} t0={w.t0[:4]} kv_heads={kv_heads} seqs={seqs}", flush=True)
    run = ParityRun(w, steps=steps, page_order=page_order, seqs=seqs, kv_heads=kv_heads, prefill_chunk=4096)
    run.prefill()
    L = run.layer
    worst = 0.0
    for s in range(steps):
        st = run.append_step(s)
        q = run.dev(st["q"])
        lgx = torch.full((L.B, L.G, L.mb), SENTINEL, dtype=torch.float32, device=L.device)
        L.block_mass(q, lgx)
        torch.cuda.synchronize()
        got = lgx.cpu().numpy()
        for ob, b in enumerate(run.bs):
            nb = -(-L.lens[b] // w.block_size)
            for og, g in enumerate(run.gs):
                ref = run.oracle.block_exact_scores(ob, og, st["q"][b][run.hs])
                assert sorted(ref) == list(range(1, max(nb - 1, 1)))
                if ref:
                    js = np.array(sorted(ref))
                    err = np.abs(got[b, g, js] - np.array([ref[j] for j in js])).max()
                    worst = max(worst, float(err))
                    assert err <= MASS_ABS, (s, b, g, err)
                untouched = np.ones(L.mb, bool)
                untouched[1:max(nb - 1, 1)] = False
                assert np.all(got[b, g, untouched] == SENTINEL), (b, g)
    assert L.error_word() == 0
    print(f"[mass] {w.name} worst abs err {worst:.3g}", flush=True)


def test_block_mass_gqa4_ragged_tail():
    _mass_case(small(name="mass", t0=(64 * 150 + 37,), steps=2), steps=2)


@pytest.mark.parametrize("r", [1, 8])
def test_block_mass_group_ratios(r):
    _mass_case(small(name=f"mass_r{r}", n_q_heads=2 * r, t0=(64 * 70 + 5,)))


def test_block_mass_block128_d64():
    _mass_case(small(name="mass_bk128", head_dim=64, block_size=128, t0=(128 * 90 + 100,), top_k=12))


def test_block_mass_fp32():
    _mass_case(make_workload("tiny_fp32"))
    _mass_case(small(name="mass_f32_bk128", kv_dtype="f32", block_size=128, n_q_heads=16, t0=(128 * 20 + 1,)))


def test_block_mass_ragged_batch():
    # sequences of 1 and 2 blocks have no candidates: their rows stay untouched
    _mass_case(small(name="mass_ragged", batch=5, t0=(1, 127, 64 * 40 + 13, 64 * 9, 3000), top_k=6))


@pytest.mark.timeout(600)
def test_block_mass_llama_gqa_128k():
    _mass_case(make_workload("llama_gqa_128k"), kv_heads=[1, 6])


def _mean_pool_run(w, steps, **kw):
    _needs_gpu()
    from tests.spla_parity import ParityRun
    print(f"[case] mean-pool score {w.name} t0={w.t0[:4]} {kw}", flush=True)
    run = ParityRun(w, steps=steps, score_form=1, **kw)
    failures = run.run(verbose=True)
    assert not failures, "\n".join(failures[:20])


@pytest.mark.parametrize("fused", [0, 1])
def test_mean_pool_selection_small(fused):
    _mean_pool_run(small(name="meanpool", t0=(64 * 150 + 37,), steps=3), 3, page_order="shuffled",
                   fused_select=fused, prefill_chunk=1000)


def test_mean_pool_selection_step_ragged():
    w = small(name="meanpool_ragged", batch=5, t0=(1, 700, 64 * 40 + 13, 64 * 9, 3000), steps=3, chunk_seqs=2,
              chunk_len=100, top_k=6)
    _mean_pool_run(w, 3, page_order="shuffled", use_step=True, prefill_chunk=1000)


@pytest.mark.timeout(600)
def test_mean_pool_selection_llama_gqa_128k():
    _mean_pool_run(make_workload("llama_gqa_128k"), 2, page_order="shuffled", use_step=True, kv_heads=[2, 5])
