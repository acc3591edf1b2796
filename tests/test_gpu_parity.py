"""GPU parity of the HIP decode path against the fp64 oracle (through the C ABI).

Small shapes that still span several score tiles, a ragged tail, both block
sizes, both head dims, every GQA ratio, shuffled pages, chunked appends that
are not block aligned, a ragged batch, the degenerate lengths (one partial
block, exactly one block, every block selected) and the selection hook.
"""
import numpy as np
import pytest

from workloads import Workload, make_workload

pytestmark = pytest.mark.gpu


def _needs_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(w, steps=None, page_order="identity", verbose=True, use_step=False):
    _needs_gpu()
    from tests.spla_parity import ParityRun
    print(f"[case] {w.name} B={w.batch} H={w.n_q_heads} G={w.n_kv_heads} d={w.head_dim} "
          f"Bk={w.block_size} k={w.top_k} t0={w.t0[:4]} pages={page_order} step={use_step}", flush=True)
    run = ParityRun(w, page_order=page_order, steps=steps, prefill_chunk=1000, use_step=use_step)
    failures = run.run(verbose=verbose)
    assert not failures, "\n".join(failures[:20])


def small(name="small", **kw):
    base = dict(name=name, batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=64, top_k=8,
                kv_dtype="bf16", t0=(64 * 150 + 37,), steps=4, kind="normal", seed=77)
    base.update(kw)
    return Workload(**base)


def test_tiny_fp32_config():
    _run(make_workload("tiny_fp32"))


def test_small_gqa4_bf16_ragged_tail():
    _run(small(steps=6), page_order="shuffled")


@pytest.mark.parametrize("r", [1, 2, 8])
def test_group_ratios(r):
    _run(small(name=f"r{r}", n_q_heads=2 * r, t0=(64 * 70 + 5,), steps=3))


def test_block128_d64():
    _run(small(name="bk128_d64", head_dim=64, block_size=128, t0=(128 * 90 + 100,), top_k=12, steps=3))


@pytest.mark.parametrize("bk", [64, 128])
def test_split_plan_odd_top_k(bk):
    # 8 sequences x 8 KV heads = 64 (sequence, KV head) pairs: the stand-alone
    # selector and attend kernels; an odd top_k, ragged lengths, a sequence
    # with every block selected
    t0 = tuple(bk * n + e for n, e in ((40, 5), (3, 0), (61, 17), (25, 1), (50, 0), (33, 9), (12, 3), (70, 2)))
    _run(small(name=f"split_odd_k_bk{bk}", batch=8, n_q_heads=32, n_kv_heads=8, block_size=bk, top_k=7, t0=t0, steps=2),
         page_order="shuffled")


def test_fp32_d128_outliers():
    _run(small(name="f32_outlier", kv_dtype="f32", kind="outlier", n_outlier=8, t0=(64 * 80,), steps=3))


@pytest.mark.parametrize("t0", [1, 30, 63, 64, 65, 64 * 7, 64 * 7 + 1])
def test_short_sequences_all_selected(t0):
    # nb <= top_k: every block selected, o_rla == 0, output = dense attention
    _run(small(name=f"short{t0}", t0=(t0,), steps=2))


@pytest.mark.parametrize("bk", [64, 128])
def test_one_unselected_block(bk):
    # nb = top_k + 1 after the append: a single unselected block, so D and
    # o_rla are differences of sums several times larger than themselves
    # (the case that needs w = phi(q).phi(k) to ~2^-16 on the matrix cores)
    _run(small(name=f"one_out_bk{bk}", block_size=bk, head_dim=128 if bk == 64 else 64, t0=(bk * 8,), steps=3))


def test_ragged_batch_with_chunks():
    w = small(name="ragged", batch=5, t0=(1, 700, 64 * 40 + 13, 64 * 9, 3000), steps=3, chunk_seqs=2,
              chunk_len=100, top_k=6)
    _run(w, page_order="shuffled")


def test_planted_batched_small():
    _run(make_workload("batched_32k", batch=3, t0=(4096,) * 3, steps=3))


def test_mixture_block128_small():
    _run(make_workload("million_1m", t0=(128 * 200 + 77,), steps=3))


def test_selection_hook():
    _needs_gpu()
    from tests.spla_parity import ParityRun
    w = small(name="hook", t0=(64 * 40 + 9,), steps=1)
    run = ParityRun(w, steps=1, prefill_chunk=512)
    run.prefill()
    st = run.append_step(0)
    nb = -(-int(run.oracle.lens[0]) // 64)
    rng = np.random.default_rng(3)
    sel = np.full((1, 2, w.top_k), -1, np.int32)
    for g in range(2):
        ids = sorted(set([0, nb - 1]) | set(rng.choice(np.arange(1, nb - 1), 4, replace=False).tolist()))
        sel[0, g, :len(ids)] = ids
    rep = run.check_decode(0, st["q"], sel_in=sel)
    assert not rep.failures, rep.failures


# ---- fused decode step (spla_decode_step) -------------------------------------
def test_step_small_gqa4_crossing_block_boundaries():
    # 70 steps from t0 = 64 * 150 - 3: the appends complete blocks along the way
    _run(small(name="step", t0=(64 * 150 - 3,), steps=70), page_order="shuffled", use_step=True)


def test_step_ragged_batch_with_chunks():
    w = small(name="step_ragged", batch=5, t0=(1, 700, 64 * 40 + 13, 64 * 9 - 1, 3000), steps=4, chunk_seqs=2,
              chunk_len=100, top_k=6)
    _run(w, page_order="shuffled", use_step=True)


@pytest.mark.parametrize("d, G", [(128, 8), (64, 4)])
def test_step_many_pairs_state_groups(d, G):
    # at least 512 (sequence, KV head) pairs: the first kernel updates S_all
    # four row chunks per workgroup (d = 64: all four chunks of a pair in one);
    # ragged lengths, block ends crossed, sampled pairs against the oracle
    _needs_gpu()
    from tests.spla_parity import ParityRun
    B = 512 // G
    rng = np.random.default_rng(5)
    t0 = tuple(int(x) for x in rng.integers(1, 64 * 12, size=B))
    t0 = (64 * 20 - 2, 63, 64) + t0[3:]
    w = Workload(name=f"pairs{B}x{G}", batch=B, n_q_heads=2 * G, n_kv_heads=G, head_dim=d, block_size=64, top_k=6,
                 kv_dtype="bf16", t0=t0, steps=3, kind="normal", seed=57)
    seqs = [0, 1, 2, 5, B // 2, B - 1]
    print(f"[case] {w.name} d={d} seqs={seqs}", flush=True)
    run = ParityRun(w, steps=3, page_order="shuffled", prefill_chunk=1000, use_step=True, seqs=seqs,
                    kv_heads=[0, G - 1])
    failures = run.run(verbose=True)
    assert not failures, "\n".join(failures[:20])
    assert run.layer.error_word() == 0


def test_step_fp32_and_block128():
    _run(make_workload("tiny_fp32", steps=4), use_step=True)
    _run(small(name="step_bk128", head_dim=64, block_size=128, t0=(128 * 40 + 126,), top_k=12, steps=4),
         use_step=True)


def test_step_matches_two_calls_bitwise():
    """spla_decode_step == spla_append_kv + spla_decode, bit for bit."""
    _needs_gpu()
    import torch
    from tests.spla_parity import ParityRun
    w = small(name="bitwise", batch=3, t0=(64 * 30 - 2, 500, 64 * 12), steps=5, kind="outlier", n_outlier=8)
    a = ParityRun(w, steps=5, prefill_chunk=700)
    b = ParityRun(w, steps=5, prefill_chunk=700)
    a.prefill()
    b.prefill()
    for s in range(5):
        st = w.step(s)
        k, v, q = a.dev(st["k"]), a.dev(st["v"]), a.dev(st["q"])
        a.layer.append(list(range(3)), [1] * 3, k, v)
        oa = a.layer.decode(q, a.gate)
        ob = b.layer.decode_step(k, v, q, b.gate)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"step {s}"
    for x, y in zip(a.layer.state_tensors(), b.layer.state_tensors()):
        assert torch.equal(x, y)


# ---- selector placement ---------------------------------------------------------
def _placements_bitwise(w, steps):
    import torch
    from tests.spla_parity import ParityRun
    print(f"[gpu-test] {w.name}: B={w.batch} G={w.n_kv_heads} k={w.top_k} t0={w.t0}", flush=True)
    runs = [ParityRun(w, steps=steps, prefill_chunk=1000, page_order="shuffled", fused_select=m, step_kernel=sk,
                      fused_merge=fm)
            for m, sk, fm in ((0, -1, -1), (1, -1, -1), (1, 1, -1), (1, -1, 1))]
    assert runs[0].layer.launch_plan() == ["step_score", "select", "attend", "combine"]
    assert runs[1].layer.launch_plan() == ["step_score", "select_attend", "combine"]
    assert runs[2].layer.launch_plan() == ["step_fused", "combine"]
    assert runs[3].layer.launch_plan() == ["step_score", "select_attend"]  # merges the records itself
    for r in runs:
        r.prefill()
    for s in range(steps):
        st = w.step(s)
        res = [r.gpu_decode(st["q"], kv=(st["k"], st["v"])) for r in runs]
        for key in ("o", "sel_idx", "o_sparse", "o_rla", "d_rla", "lg"):
            for i in (1, 2, 3):
                assert np.array_equal(res[0][key], res[i][key]), f"step {s}: {key}, plan {i}"
        print(f"[gpu-test] step {s}: lens {runs[2].layer.lens[:4]}, error words {[r.layer.error_word() for r in runs]}",
              flush=True)
    errs = [r.layer.error_word() for r in runs]
    assert errs == [0, 0, 0, 0]
    for x, y in zip(runs[0].layer.state_tensors(), runs[2].layer.state_tensors()):
        assert torch.equal(x, y)


def test_fused_select_matches_split_bitwise():
    """The stand-alone selector, the fused select + attend kernel (with the
    combine kernel, and merging the records itself) and the one-kernel step
    give the same outputs and selections, bit for bit (every placement runs
    the same selection, attend and merge arithmetic).  The
    steps cross a block end, so the one-kernel step's append completes a
    block whose statistics the next step scores."""
    _needs_gpu()
    # ragged: one sequence with every block selected, others crossing block ends
    w = small(name="fused_vs_split", batch=4, t0=(64 * 300 - 3, 64 * 5, 64 * 40 + 1, 3000), steps=6,
              kind="outlier", n_outlier=8, top_k=12)
    _placements_bitwise(w, 6)


def test_step_kernel_three_pairs_per_xcd_bitwise():
    """The one-kernel step with 24 (sequence, KV head) pairs: three pairs on
    each XCD, whose producers all come before any of their attend
    workgroups; short sequences (every block selected) among long ones, a
    block end crossed, d = 64 and four query heads per KV head."""
    _needs_gpu()
    w = Workload(name="step3pp", batch=6, n_q_heads=16, n_kv_heads=4, head_dim=64, block_size=64, top_k=16,
                 kv_dtype="bf16", t0=(64 * 90 - 2, 100, 64 * 16, 5000, 64 * 33 + 7, 900), steps=5,
                 kind="normal", seed=83)
    _placements_bitwise(w, 5)


# ---- ties: equal group scores go to the smaller block id -------------------------
def _tied(n_plant, fused, steps=2):
    """Planted blocks with identical keys (noise 0): equal statistics, equal
    scores, all above the random blocks.  The selection must be exactly the
    oracle's: the smallest planted ids."""
    from tests.spla_parity import ParityRun
    w = Workload(name=f"tied{n_plant}", batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=64,
                 top_k=32, kv_dtype="bf16", t0=(64 * 1500 + 17,), steps=steps, kind="planted", seed=91,
                 n_plant=n_plant, plant_shared_heads=False, plant_noise=0.0)
    print(f"[gpu-test] {w.name} fused={fused}", flush=True)
    run = ParityRun(w, steps=steps, page_order="shuffled", fused_select=fused)
    run.prefill()
    for s in range(steps):
        st = run.append_step(s)
        rep = run.check_decode(s, st["q"])
        assert not rep.failures, rep.failures[:5]
        assert rep.sel_equal, "tied scores: the selection must be the smallest ids"
    assert run.layer.error_word() == 0


@pytest.mark.parametrize("fused", [0, 1])
def test_tied_scores_ranked_exactly(fused):
    # 100 tied blocks: fewer than the 256 ranked exactly in the last bucket
    _needs_gpu()
    _tied(100, fused)


@pytest.mark.parametrize("fused", [0, 1])
def test_tied_scores_taken_by_id(fused):
    # 600 tied blocks: the top bucket cannot be split by score, ids decide
    _needs_gpu()
    _tied(600, fused)


@pytest.mark.parametrize("fused", [0, 1])
def test_zero_query_every_score_equal(fused):
    # q = 0: every candidate has the same score; sink, current and the
    # smallest ids are selected, attention is uniform
    _needs_gpu()
    from tests.spla_parity import ParityRun
    w = small(name="zero_q", t0=(64 * 700 + 5,), steps=2)
    run = ParityRun(w, steps=2, page_order="shuffled", fused_select=fused)
    run.prefill()
    for s in range(2):
        st = run.append_step(s)
        rep = run.check_decode(s, np.zeros_like(st["q"]))
        assert not rep.failures, rep.failures[:5]
        assert rep.sel_equal
