"""Parity at the five workloads' full sizes, in the launch configuration the
benchmark times (spla_decode_step: the one-token append fused into the
scorer's launch, then select / attend / combine; pages in shuffled order).

Each workload runs its stated number of decode steps (16 / 256 / 128 / 64 /
64), or more where those steps would not complete a block: the tiny and the
1M workloads start block-aligned, so they run on until their own token
completes one (the path that appends a block's mean and variance inside the
scorer's launch and grows the candidate range by a block).  Every step is
checked.

The GPU runs the whole batch and every head; the oracle checks sampled
(sequence, KV head) pairs: the method treats each pair on its own, so the
oracle run on their slices of the same inputs gives exactly the values the
full oracle would.  Each case prints its name, shapes and samples before the
GPU work starts.
"""
import pytest

from spla_parity import ParityRun
from workloads import Workload, make_workload

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _completions(w, steps):
    """(step, sequence) pairs whose token completes a block within `steps`."""
    lens, out = list(w.t0), []
    for s in range(steps):
        for b in w.chunk_plan(s):
            lens[int(b)] += w.chunk_len
        lens = [t + 1 for t in lens]
        out += [(s, b) for b, t in enumerate(lens) if t % w.block_size == 0]
    return out


def _run(w, steps, seqs=None, kv_heads=None, page_order="shuffled", fused_select=-1, rla_form=0,
         need_completion=False):
    if need_completion:
        done = [c for c in _completions(w, steps) if seqs is None or c[1] in seqs]
        assert done, "the checked steps must complete a block"
        print(f"[fullsize] block completions (step, seq): {done[:8]}", flush=True)
    print(f"[fullsize] {w.name}: B={w.batch} H={w.n_q_heads} G={w.n_kv_heads} d={w.head_dim} "
          f"Bk={w.block_size} k={w.top_k} t0={w.t0[:4]}{'...' if w.batch > 4 else ''} steps={steps} "
          f"seqs={seqs} kv_heads={kv_heads} fused_select={fused_select} rla_form={rla_form}", flush=True)
    run = ParityRun(w, page_order=page_order, steps=steps, use_step=True, seqs=seqs, kv_heads=kv_heads,
                    fused_select=fused_select, rla_form=rla_form)
    print(f"[fullsize] kernels: {run.layer.launch_plan()}", flush=True)
    failures = run.run(verbose=True)
    assert not failures, "\n".join(failures[:20])


@pytest.mark.timeout(300)
def test_tiny_fp32_full():
    # B=1, 2/2 x 64, 4K context, fp32: the 16 stated steps and on to step 80,
    # past the first block its own tokens complete (step 63)
    _run(make_workload("tiny_fp32"), steps=80, need_completion=True)


@pytest.mark.timeout(600)
def test_llama_gqa_128k_full():
    # B=1, 128K context, GQA 32/8 x 128, Bk=64, k=32, 256 steps (4 blocks
    # completed): every head checked
    _run(make_workload("llama_gqa_128k"), steps=256, need_completion=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("form", [1, 2], ids=["normalized", "rmsnorm"])
def test_llama_gqa_128k_rla_forms(form):
    # the output forms of the RLA branch at the benchmark's workload: 2 KV heads
    _run(make_workload("llama_gqa_128k"), steps=2, kv_heads=[0, 6], rla_form=form)


@pytest.mark.timeout(600)
def test_batched_32k_full():
    # B=16 x 32K, planted blocks, 128 steps (2 blocks completed): 3 sequences x
    # 2 KV heads sampled
    _run(make_workload("batched_32k"), steps=128, seqs=[0, 7, 15], kv_heads=[0, 5], need_completion=True)


@pytest.mark.timeout(900)
def test_million_1m_full():
    # B=1, 1M context, Bk=128, k=64 (8192 blocks): the 64 stated steps and on
    # to step 128, whose token completes block 8192; 2 KV heads sampled
    _run(make_workload("million_1m", steps=128), steps=128, kv_heads=[2, 7], need_completion=True)


@pytest.mark.timeout(900)
def test_ragged_chunked_full():
    # B=64 ragged contexts with 8 x 256-token chunk appends per step: the
    # shortest, the longest and sequences that get chunks, 1 KV head each
    w = make_workload("ragged_chunked")
    lens = list(w.t0)
    chunked = sorted(set(int(b) for s in range(3) for b in w.chunk_plan(s)))
    seqs = sorted({lens.index(min(lens)), lens.index(max(lens))} | set(chunked[:3]))
    # 64 steps (the survey's reading of this workload's length)
    _run(w, steps=64, seqs=seqs, kv_heads=[3], need_completion=True)


# the selector holds KPT candidates per thread in registers, with one compiled
# size per entry below; a sequence whose candidate count just exceeds the next
# smaller size runs each of them (single KV head, d = 64 keeps the data small).
# Both placements: the stand-alone selector (fused_select = 0) and the fused
# select + attend kernel (1; its sizes are 1, 2, 4, 6, 9, 12, 16 and it is not
# used past 16).
SELECT_SIZES = [2, 3, 4, 6, 8, 9, 10, 12, 16, 20, 24, 32, 40, 48, 64]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("fused", [0, 1])
@pytest.mark.parametrize("kpt", SELECT_SIZES)
def test_selector_sizes(kpt, fused):
    if fused and kpt > 16:
        pytest.skip("the fused kernel is not used past 16 keys per thread")
    prev = SELECT_SIZES[SELECT_SIZES.index(kpt) - 1] if kpt > 2 else 1
    nb = prev * 256 + 2 + 37  # candidates = nb - 2 > prev * 256
    w = Workload(name=f"sel_kpt{kpt}", batch=1, n_q_heads=2, n_kv_heads=1, head_dim=64, block_size=64,
                 top_k=24, kv_dtype="bf16", t0=(nb * 64 - 9,), steps=2, kind="outlier", seed=500 + kpt,
                 n_outlier=4, prefill_chunk=16384)
    _run(w, steps=2, page_order="shuffled", fused_select=fused)


@pytest.mark.timeout(300)
def test_selector_max_blocks():
    # the largest supported table: 16386 blocks per sequence, 16384 candidates
    w = Workload(name="sel_max", batch=1, n_q_heads=2, n_kv_heads=1, head_dim=64, block_size=64,
                 top_k=256, kv_dtype="bf16", t0=(16386 * 64 - 5,), steps=2, kind="normal", seed=599,
                 prefill_chunk=16384)
    assert w.max_blocks_per_seq(2) == 16386
    _run(w, steps=2, page_order="shuffled")
