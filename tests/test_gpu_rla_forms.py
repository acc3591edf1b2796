"""GPU parity of the output forms of the RLA branch (normalised o_rla / D and
RMS-normalised gamma * o_rla / rms(o_rla)) against the fp64 oracle, through
the C ABI.  Several score tiles with a ragged tail, both head dims (the RMS
form reduces over the whole head in one workgroup), every block selected
(the branch vanishes), a ragged batch with chunk appends, the fused step,
an eps large enough to matter, and switching the form back to plain."""
import numpy as np
import pytest

from workloads import make_workload
from tests.test_gpu_parity import _needs_gpu, small

pytestmark = pytest.mark.gpu

NORMALIZED, RMSNORM = 1, 2


def _run(w, form, steps=None, page_order="identity", use_step=False, eps=1e-6):
    _needs_gpu()
    from tests.spla_parity import ParityRun
    print(f"[case] {w.name} form={form} eps={eps} B={w.batch} H={w.n_q_heads} G={w.n_kv_heads} d={w.head_dim} "
          f"Bk={w.block_size} k={w.top_k} t0={w.t0[:4]} pages={page_order} step={use_step}", flush=True)
    run = ParityRun(w, page_order=page_order, steps=steps, prefill_chunk=1000, use_step=use_step,
                    rla_form=form, rla_eps=eps)
    failures = run.run(verbose=True)
    assert not failures, "\n".join(failures[:20])


@pytest.mark.parametrize("form", [NORMALIZED, RMSNORM])
@pytest.mark.parametrize("use_step", [False, True])
def test_forms_gqa4_ragged_tail(form, use_step):
    _run(small(name="forms", steps=4), form, page_order="shuffled", use_step=use_step)


@pytest.mark.parametrize("form", [NORMALIZED, RMSNORM])
def test_forms_d64_block128_r8(form):
    _run(small(name="forms_d64", head_dim=64, block_size=128, n_q_heads=16, t0=(128 * 60 + 3,), top_k=10,
               steps=3), form)


@pytest.mark.parametrize("form", [NORMALIZED, RMSNORM])
@pytest.mark.parametrize("t0", [1, 64 * 7])
def test_forms_vanish_when_all_selected(form, t0):
    # after each step's append nb <= top_k = 8: every block selected
    _run(small(name=f"forms_short{t0}", t0=(t0,), steps=2), form)


@pytest.mark.parametrize("form", [NORMALIZED, RMSNORM])
def test_forms_one_unselected_block(form):
    # nb = top_k + 1 after the append: one block of 64 tokens is unselected,
    # so D and o_rla are differences of sums ~8x larger than themselves
    _run(small(name="forms_one_out", t0=(64 * 8,), steps=3), form)


@pytest.mark.parametrize("form", [NORMALIZED, RMSNORM])
def test_forms_ragged_batch_with_chunks(form):
    w = small(name="forms_ragged", batch=5, t0=(1, 700, 64 * 40 + 13, 64 * 9, 3000), steps=3, chunk_seqs=2,
              chunk_len=100, top_k=6)
    _run(w, form, page_order="shuffled", use_step=True)


def test_rmsnorm_fp32_r1():
    _run(small(name="forms_f32", kv_dtype="f32", n_q_heads=2, t0=(64 * 50 + 9,), steps=3), RMSNORM)


def test_rmsnorm_eps_matters():
    # eps of the order of the mean square of o_rla at this length (about 6e7
    # to 9e7 per head in the oracle), so where it enters the norm matters
    _run(small(name="forms_eps", t0=(64 * 40 + 21,), steps=3), RMSNORM, eps=5e7)


def test_switching_back_to_plain_is_bitwise_default():
    _needs_gpu()
    import torch
    from tests.spla_parity import ParityRun
    w = small(name="forms_switch", t0=(64 * 90 + 11,), steps=2)
    outs = []
    for forms in ((0,), (2, 1, 0)):
        run = ParityRun(w, steps=2)
        run.prefill()
        st = run.append_step(0)
        for f in forms:
            run.layer.set_rla_output(f, torch.from_numpy(w.rla_gamma()), 1e-6)
        outs.append(run.gpu_decode(st["q"]))
    for k in ("o", "o_sparse", "o_rla", "d_rla", "sel_idx"):
        assert np.array_equal(outs[0][k], outs[1][k]), k
