"""GPU parity of chunked prefill (spla_prefill) against the fp64 oracle's
per-token append + decode, through the C ABI.  The first part of one
sequence's tokens is appended as usual, the rest goes through one prefill
call; every new token's output is compared with the oracle's decode at that
token's position (on the GPU's selection when a near-tie picked another legal
set), then the state.  Cases: an empty sequence prefilled from its first
token, a prefix that ends inside a block, groups of launches smaller than the
call (the workspace sized for fewer tokens), every group ratio, Bk = 128 with
d = 64, fp32, the output forms, the mean-pooling score, a batch whose other
sequences must stay untouched, and 128K of prefix with 512 prefilled tokens."""
import numpy as np
import pytest

from tests.spla_parity import LG_ABS, OUT_REL, S_REL, STAT_REL, check_selection, rel_err
from tests.test_gpu_parity import _needs_gpu, small
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _prefill_case(w, seq, split, chunk=256, kv_heads=None, rla_form=0, score_form=0, eps=1e-6):
    """Tokens [0, split) of sequence seq appended in ordinary chunks, then
    tokens [split, t0[seq]) through one spla_prefill call."""
    _needs_gpu()
    import torch
    from block_sparse_linear_amd import SplaLayer
    from oracle import SplaOracle
    t0 = w.t0[seq]
    n = t0 - split
    print(f"[case] prefill {w.name} B={w.batch} H={w.n_q_heads} G={w.n_kv_heads} d={w.head_dim} Bk={w.block_size} "
          f"k={w.top_k} {w.kv_dtype} seq={seq} prefix={split} n={n} chunk={chunk} kv_heads={kv_heads} "
          f"rla_form={rla_form} score_form={score_form}", flush=True)
    dev = torch.device("cuda")
    tdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    mb = w.max_blocks_per_seq(1)
    L = SplaLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k, mb,
                  kv_dtype=w.kv_dtype, page_order="shuffled", seed=w.seed)
    gamma = torch.from_numpy(w.rla_gamma()) if rla_form == 2 else None
    L.set_rla_output(rla_form, gamma, eps)
    L.set_score_form(score_form)
    gs = list(range(w.n_kv_heads)) if kv_heads is None else kv_heads
    r = w.group
    hs = [g * r + i for g in gs for i in range(r)]
    o = SplaOracle(1, len(hs), len(gs), w.head_dim, w.block_size, w.top_k, t0 + 1)
    K, V = w.prefill(seq)
    dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(tdt)
    # every other sequence gets its prefill too: the call must leave them alone
    for b in range(w.batch):
        if b != seq:
            for _, k, v in w.prefill_chunks(b, 1000):
                L.append([b], [k.shape[0]], dv(k), dv(v))
    for p0 in range(0, split, 1000):
        p1 = min(split, p0 + 1000)
        L.append([seq], [p1 - p0], dv(K[p0:p1]), dv(V[p0:p1]))
    if split:
        o.append([0], [split], K[:split][:, gs], V[:split][:, gs])
    others = [(L.s_all[b].clone(), L.z_all[b].clone()) for b in range(w.batch) if b != seq]
    Q = w.prefill_queries(seq, split, n)
    gate_np = w.gate()
    ws = torch.empty(L.handle.prefill_workspace_bytes(chunk) // 4 + 64, dtype=torch.int32, device=dev)
    sel = torch.full((n, w.n_kv_heads, w.top_k), -7, dtype=torch.int32, device=dev)
    lg = torch.zeros((n, w.n_kv_heads, L.mb), dtype=torch.float32, device=dev)
    out = L.prefill(seq, dv(K[split:]), dv(V[split:]), dv(Q), torch.from_numpy(gate_np).to(dev), workspace=ws,
                    sel_idx=sel, lg=lg)
    torch.cuda.synchronize()
    assert L.lens[seq] == t0 and all(L.lens[b] == w.t0[b] for b in range(w.batch))
    got = out.cpu().numpy()[:, hs]
    sel_g = sel.cpu().numpy()[:, gs]
    lg_g = lg.cpu().numpy()[:, gs]
    form = dict(rla_mode=rla_form, eps=eps, score_form=score_form,
                gamma=None if gamma is None else w.rla_gamma()[hs])
    snap = (o.K[0].copy(), o.V[0].copy(), o.mean.copy(), o.var.copy(), o.S.copy(), o.z.copy(), o.lens.copy())
    ref = o.prefill_sequence(0, K[split:][:, gs], V[split:][:, gs], Q[:, hs], gate_np[hs], **form)
    failures, ties = [], 0
    lg_worst = 0.0
    for t in range(n):
        nb = -(-(split + t + 1) // w.block_size)
        for gg in range(len(gs)):
            msg = check_selection(sel_g[t, gg], ref["lg"][t][gg], nb, w.top_k)
            if msg:
                failures.append(f"token {t} g {gs[gg]}: {msg}")
            # group log scores of the candidate blocks: absolute in the log
            # domain, relative past |LG| = 1 (the decode's bar)
            if nb > w.top_k:
                js = np.arange(1, nb - 1)
                lg_ref = np.array([ref["lg"][t][gg][int(j)] for j in js])
                dlg = np.abs(lg_g[t, gg, js].astype(np.float64) - lg_ref) / np.maximum(1.0, np.abs(lg_ref))
                lg_worst = max(lg_worst, float(dlg.max()))
                if dlg.max() > LG_ABS:
                    i = int(np.argmax(dlg))
                    failures.append(f"token {t} g {gs[gg]}: group log score of block {int(js[i])} off by "
                                    f"{dlg[i]:.3g} (oracle {lg_ref[i]:.6g})")
            if not np.array_equal(sel_g[t, gg], ref["sel"][t, gg]):
                ties += 1
    if ties:
        # re-run the oracle from the same prefix on the GPU's (legal) sets
        o.K[0], o.V[0], o.mean, o.var, o.S, o.z, o.lens = (x.copy() for x in snap)
        ref = o.prefill_sequence(0, K[split:][:, gs], V[split:][:, gs], Q[:, hs], gate_np[hs],
                                 sel_per_token=sel_g, **form)
    worst = 0.0
    for t in range(n):
        e = rel_err(got[t], ref["o"][t])
        worst = max(worst, e)
        if e > OUT_REL:
            failures.append(f"token {t}: o rel err {e:.3g}")
    # state after the call: S_all / z_all, statistics of every complete block
    S = L.s_all.cpu().numpy()[seq][gs]
    z = L.z_all.cpu().numpy()[seq][gs]
    mean, var = (x.cpu().numpy()[seq][gs] for x in L.stats())
    nfull = t0 // w.block_size
    for gg in range(len(gs)):
        if rel_err(S[gg], o.S[0, gg]) > S_REL or rel_err(z[gg], o.z[0, gg]) > S_REL:
            failures.append(f"state g {gs[gg]}")
        for gv, ov in ((mean, o.mean), (var, o.var)):
            dd = np.abs(gv[gg, :nfull].astype(np.float64) - ov[0, gg, :nfull])
            if nfull and float((dd / (np.abs(ov[0, gg, :nfull]) + 1e-6 / STAT_REL)).max()) > STAT_REL:
                failures.append(f"block statistics g {gs[gg]}")
    for i, b in enumerate([b for b in range(w.batch) if b != seq]):
        if not (torch.equal(L.s_all[b], others[i][0]) and torch.equal(L.z_all[b], others[i][1])):
            failures.append(f"sequence {b} changed")
    if L.error_word():
        failures.append(f"error word {L.error_word():#x}")
    print(f"[prefill] {w.name} n={n} worst o rel err {worst:.3g} worst lg err {lg_worst:.3g} near-tie tokens {ties}",
          flush=True)
    assert not failures, "\n".join(failures[:20])


def test_prefill_from_empty_sequence():
    # the first tokens select every block; groups of 100 tokens
    _prefill_case(small(name="pf_empty", t0=(64 * 20 + 9,)), 0, 0, chunk=100)


def test_prefill_gqa4_prefix_inside_block():
    _prefill_case(small(name="pf_gqa4", t0=(64 * 150 + 37,)), 0, 64 * 140 + 21)


@pytest.mark.parametrize("r", [1, 8])
def test_prefill_group_ratios(r):
    _prefill_case(small(name=f"pf_r{r}", n_q_heads=2 * r, t0=(64 * 70 + 5,)), 0, 64 * 60 + 63, chunk=64)


@pytest.mark.parametrize("r", [2, 8])
def test_prefill_group_ratios_d64(r):
    # head dim 64 with two and eight query heads per KV head; groups of 130
    # tokens leave a partly filled last token tile of the matrix-core scorer
    _prefill_case(small(name=f"pf_r{r}_d64", n_q_heads=2 * r, head_dim=64, t0=(64 * 70 + 5,)), 0,
                  64 * 58 + 3, chunk=130)


def test_prefill_block128_d64():
    _prefill_case(small(name="pf_bk128", head_dim=64, block_size=128, top_k=12, t0=(128 * 90 + 100,)), 0,
                  128 * 87 + 5)


def test_prefill_fp32():
    _prefill_case(small(name="pf_f32", kv_dtype="f32", t0=(64 * 40 + 3,)), 0, 64 * 36 + 10, chunk=50)


@pytest.mark.parametrize("n,chunk", [(1, 256), (3, 256), (40, 17)])
def test_prefill_tiny_groups(n, chunk):
    # one token, three tokens, and groups of 17: partial 16-token tiles of the
    # linear-attention state, partial 4-token k-steps of the state append, a
    # score tile of a handful of queries; the prefix ends inside a block
    _prefill_case(small(name=f"pf_tiny_{n}_{chunk}", t0=(64 * 90 + 11 + n,)), 0, 64 * 90 + 11, chunk=chunk)


@pytest.mark.parametrize("form", [1, 2])
def test_prefill_rla_forms(form):
    _prefill_case(small(name=f"pf_form{form}", t0=(64 * 90 + 11,)), 0, 64 * 85, rla_form=form)


def test_prefill_mean_pool_score():
    _prefill_case(small(name="pf_meanpool", t0=(64 * 90 + 11,)), 0, 64 * 85 + 40, score_form=1)


def test_prefill_one_sequence_of_a_batch():
    w = small(name="pf_batch", batch=3, t0=(3000, 64 * 50 + 17, 700), top_k=6)
    _prefill_case(w, 1, 64 * 45 + 3)


@pytest.mark.timeout(900)
def test_prefill_llama_gqa_128k():
    w = make_workload("llama_gqa_128k")
    _prefill_case(w, 0, w.t0[0] - 512, kv_heads=[0, 5])
