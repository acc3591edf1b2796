"""Pins of the fp64 oracle against things other than itself: closed forms,
library special cases (torch SDPA / elu / matmul on the CPU in fp64) and
brute force on tiny inputs.  Each pin is also run against deliberately
broken copies of the oracle (``test_mutants_are_caught``) to show that a
plausible mistake anywhere in it fails at least one pin.

CPU only (no GPU, no HIP library).
"""
import math

import numpy as np
import pytest
import torch

import oracle.spla_oracle as so
from oracle import SplaOracle
from workloads import WORKLOADS, make_workload, round_bf16

F64 = np.float64


# ------------------------------------------------------------------ helpers
def factorial_block(kbar, t, axes):
    """Keys kbar + sum_c s_c t_c e_c over the full 2^m sign design on the
    given axes (m = len(axes)); every channel's values are exactly
    kbar_c +- t_c, half each, and all cross moments vanish."""
    m = len(axes)
    rows = []
    for code in range(2 ** m):
        k = np.array(kbar, F64).copy()
        for bit, (c, tc) in enumerate(zip(axes, t)):
            k[c] += tc if (code >> bit) & 1 else -tc
        rows.append(k)
    return np.array(rows)


def fresh_oracle(B=1, H=4, G=1, d=8, bk=4, top_k=3, cap=256):
    return SplaOracle(B, H, G, d, bk, top_k, cap)


def fill(o, b, K, V):
    o.append([b], [K.shape[0]], K.astype(np.float32), V.astype(np.float32))


def dyadic_normal(rng, shape, scale=8.0):
    """Random values on a 1/scale grid (exactly representable, exact sums)."""
    return np.round(rng.standard_normal(shape) * scale) / scale


# ---------------------------------------------------------------- the pins
def pin_phi():
    x = torch.linspace(-20, 20, 4001, dtype=torch.float64)
    ref = (torch.nn.functional.elu(x) + 1.0).numpy()
    # torch forms elu+1 as expm1(x)+1, exact only to ~1 ulp of 1 for x<0
    assert np.allclose(so.phi(x.numpy()), ref, rtol=1e-15, atol=1e-15), "phi != elu+1"


def pin_block_stats_factorial():
    kbar = [0.5, -1.25, 2.0, 0.0, 3.5, -0.75, 1.0, -2.0]
    t = [0.5, 0.25, 1.0, 0.125, 2.0, 0.75]
    axes = [0, 1, 2, 4, 5, 7]
    keys = factorial_block(kbar, t, axes)  # 64 keys
    mean, var = so.block_stats(keys)
    assert np.array_equal(mean, np.array(kbar)), "mean"
    want = np.zeros(8)
    for c, tc in zip(axes, t):
        want[c] = tc * tc  # population variance of {kbar-t, kbar+t}
    assert np.array_equal(var, want), ("var", var, want)


def pin_score_identical_keys():
    rng = np.random.default_rng(1)
    d = 16
    q = rng.standard_normal((3, d))
    k = dyadic_normal(rng, d)  # exact sums: the two-pass variance is exactly 0
    keys = np.repeat(k[None, :], 64, axis=0)
    mean, var = so.block_stats(keys)
    assert np.all(var == 0.0)
    ls = so.taylor_log_score(q, mean[None], var[None])[:, 0]
    want = np.array([sum(q[h, c] * k[c] for c in range(d)) / math.sqrt(d) for h in range(3)])
    assert np.allclose(ls, want, rtol=1e-14, atol=1e-14), (ls, want)


def pin_score_factorial_closed_form():
    """Second-order Taylor of the block's mean exp mass is
    exp(qh.kbar)(1 + 1/2 sum (qh_c t_c)^2); the exact mean mass of the sign
    design is exp(qh.kbar) prod cosh(qh_c t_c)."""
    d = 8
    kbar = np.array([0.25, -0.5, 1.0, 0.0, -1.5, 0.75, 0.5, -0.25])
    axes = [0, 1, 3, 4, 6, 7]
    t = np.array([0.3, 0.2, 0.1, 0.25, 0.15, 0.05])
    keys = factorial_block(kbar, t, axes)
    mean, var = so.block_stats(keys)
    rng = np.random.default_rng(7)
    for trial in range(20):
        q = rng.standard_normal(d) * (0.5 + trial / 10)
        qh = q / math.sqrt(d)
        ls = so.taylor_log_score(q[None], mean[None], var[None])[0, 0]
        x = qh[axes] * t
        taylor = math.exp(float(qh @ kbar)) * (1.0 + 0.5 * float((x * x).sum()))
        assert abs(math.exp(ls) / taylor - 1.0) < 1e-13, ("taylor form", trial)
        exact = math.exp(float(qh @ kbar)) * float(np.prod(np.cosh(x)))
        brute = float(np.mean(np.exp(keys @ qh)))
        assert abs(brute / exact - 1.0) < 1e-13  # closed form of the design
        # 0 <= prod cosh(x) - (1 + a) <= e^a - 1 - a <= a^2/2 e^a with
        # a = 1/2 sum x^2 (cosh x <= exp(x^2/2)); the fourth-order terms
        # sum x^4/24 + sum_{c<c'} x_c^2 x_c'^2 / 4 are a lower bound
        base = math.exp(float(qh @ kbar))
        gap = (exact - math.exp(ls)) / base
        a = 0.5 * float((x * x).sum())
        lower = a * a / 2 - float((x ** 4).sum()) / 12
        upper = a * a / 2 * math.exp(a)
        assert lower * (1 - 1e-9) - 1e-14 <= gap <= upper + 1e-14, ("truncation", trial, gap, lower, upper)


def pin_score_vs_bruteforce_low_variance():
    rng = np.random.default_rng(3)
    d = 16
    for trial in range(30):
        sigma = rng.uniform(0.005, 0.05, d)
        keys = rng.standard_normal(d)[None, :] + rng.standard_normal((64, d)) * sigma
        q = rng.standard_normal(d) * 2
        qh = q / math.sqrt(d)
        mean, var = so.block_stats(keys)
        score = math.exp(so.taylor_log_score(q[None], mean[None], var[None])[0, 0])
        brute = float(np.mean(np.exp(keys @ qh)))
        # error budget: off-diagonal covariance the diagonal score drops, plus
        # third and higher central moments of x = qh.(k - kbar)
        dev = keys - keys.mean(0)
        cov = dev.T @ dev / 64
        off = 0.5 * abs(float(qh @ (cov - np.diag(np.diag(cov))) @ qh))
        xm = np.abs(dev @ qh)
        tail = float(np.mean(xm ** 3)) / 6 * math.exp(float(xm.max()))
        base = math.exp(float(qh @ keys.mean(0)))
        assert abs(score - brute) / base <= off + tail + 1e-12, (trial, abs(score - brute) / base, off, tail)


def pin_group_score():
    rng = np.random.default_rng(4)
    ls = rng.standard_normal((1, 50))
    assert np.allclose(so.group_log_score(ls), ls[0], rtol=0, atol=1e-15)
    ls4 = np.repeat(ls, 4, axis=0)
    assert np.allclose(so.group_log_score(ls4), ls[0] + math.log(4), rtol=0, atol=1e-14)
    # two heads, closed form log(e^a + e^b)
    a, b = 0.3, -1.7
    got = so.group_log_score(np.array([[a], [b]]))[0]
    assert abs(got - math.log(math.exp(a) + math.exp(b))) < 1e-15


def pin_selection_properties():
    rng = np.random.default_rng(5)
    for trial in range(200):
        nb = int(rng.integers(1, 40))
        k = int(rng.integers(2, 12))
        vals = rng.integers(0, 6, size=nb)  # many exact ties
        lg = {j: float(vals[j]) for j in range(1, nb - 1)}
        sel = so.select_blocks(lg, nb, k)
        assert sel == sorted(set(sel))
        assert len(sel) == min(k, nb)
        assert 0 in sel and (nb - 1) in sel
        cand_in = [j for j in sel if 0 < j < nb - 1]
        cand_out = [j for j in range(1, nb - 1) if j not in sel]
        for a in cand_in:
            for b in cand_out:
                assert lg[a] > lg[b] or (lg[a] == lg[b] and a < b), (trial, a, b)


def _sdpa(q, K, V, mask=None):
    qt = torch.tensor(q, dtype=torch.float64)[None, None, None, :]
    kt = torch.tensor(K, dtype=torch.float64)[None, None]
    vt = torch.tensor(V, dtype=torch.float64)[None, None]
    m = None if mask is None else torch.tensor(mask)[None, None, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)[0, 0, 0].numpy()


def _random_state(rng, B=2, H=4, G=2, d=8, bk=4, top_k=3, T=(37, 9)):
    o = SplaOracle(B, H, G, d, bk, top_k, 64)
    KV = []
    for b in range(B):
        K = dyadic_normal(rng, (T[b], G, d))
        V = dyadic_normal(rng, (T[b], G, d))
        # mixed-size appends: chunked prefill of the same rows
        p = 0
        while p < T[b]:
            n = min(int(rng.integers(1, 9)), T[b] - p)
            o.append([b], [n], K[p:p + n].astype(np.float32), V[p:p + n].astype(np.float32))
            p += n
        KV.append((K, V))
    return o, KV


def pin_all_selected_is_dense_attention():
    rng = np.random.default_rng(6)
    o, KV = _random_state(rng, top_k=64)
    q = rng.standard_normal((2, 4, 8))
    gate = rng.uniform(size=4)
    res = o.decode(q, gate)
    for b in range(2):
        K, V = KV[b]
        for h in range(4):
            g = h // 2
            ref = _sdpa(q[b, h], K[:, g], V[:, g])
            assert np.allclose(res["o_sparse"][b, h], ref, rtol=1e-12, atol=1e-13)
            assert np.all(res["o_rla"][b, h] == 0.0) and res["d_rla"][b, h] == 0.0
            assert np.array_equal(res["o"][b, h], res["o_sparse"][b, h])


def pin_sparse_is_masked_attention_and_rla_is_direct():
    rng = np.random.default_rng(8)
    o, KV = _random_state(rng, T=(45, 30), top_k=4)
    q = rng.standard_normal((2, 4, 8))
    gate = rng.uniform(size=4)
    res = o.decode(q, gate, brute_rla=True)
    for b in range(2):
        K, V = KV[b]
        T = K.shape[0]
        for h in range(4):
            g = h // 2
            sel = [j for j in res["sel"][b, g] if j >= 0]
            mask = np.zeros(T, bool)
            for j in sel:
                mask[j * 4:min((j + 1) * 4, T)] = True
            ref = _sdpa(q[b, h], K[:, g], V[:, g], mask)
            assert np.allclose(res["o_sparse"][b, h], ref, rtol=1e-12, atol=1e-13)
            # o_rla = o_bar - o_tilde equals linear attention over the rest
            direct = np.zeros(8)
            dsum = 0.0
            f = (torch.nn.functional.elu(torch.tensor(q[b, h])) + 1).numpy()
            for i in range(T):
                if not mask[i]:
                    w = float(f @ (torch.nn.functional.elu(torch.tensor(K[i, g])) + 1).numpy())
                    direct += w * V[i, g]
                    dsum += w
            scale = max(1.0, np.abs(direct).max())
            assert np.abs(res["o_rla"][b, h] - direct).max() <= 1e-11 * scale
            assert abs(res["d_rla"][b, h] - dsum) <= 1e-11 * max(1.0, abs(dsum))
            assert np.allclose(res["o"][b, h], res["o_sparse"][b, h] + gate[h] * res["o_rla"][b, h],
                               rtol=1e-14, atol=1e-14)


def pin_global_state_is_phiK_T_V():
    rng = np.random.default_rng(9)
    o, KV = _random_state(rng)
    for b in range(2):
        K, V = KV[b]
        for g in range(2):
            kt = torch.tensor(K[:, g], dtype=torch.float64)
            fk = torch.nn.functional.elu(kt) + 1
            S = (fk.T @ torch.tensor(V[:, g], dtype=torch.float64)).numpy()
            z = fk.sum(0).numpy()
            assert np.allclose(o.S[b, g], S, rtol=1e-12, atol=1e-12)
            assert np.allclose(o.z[b, g], z, rtol=1e-13, atol=1e-13)
            nfull = K.shape[0] // 4
            for j in range(nfull):
                blk = K[j * 4:(j + 1) * 4, g]
                m = np.array([math.fsum(blk[:, c]) / 4 for c in range(8)])
                assert np.array_equal(o.mean[b, g, j], m)


def pin_gqa_head_map():
    """Query head h reads KV head h // r: with KV heads made of constant
    distinct values the sparse output identifies the head."""
    o = SplaOracle(1, 6, 3, 4, 4, 8, 64)
    T = 12
    K = np.zeros((T, 3, 4), np.float32)
    V = np.zeros((T, 3, 4), np.float32)
    for g in range(3):
        V[:, g, :] = g + 1
    o.append([0], [T], K, V)
    res = o.decode(np.zeros((1, 6, 4)), np.zeros(6))
    for h in range(6):
        assert np.allclose(res["o_sparse"][0, h], h // 2 + 1)


def pin_edge_lengths():
    rng = np.random.default_rng(10)
    for T, want in [(1, [0]), (3, [0]), (4, [0]), (5, [0, 1]), (8, [0, 1]), (9, [0, 1, 2])]:
        o = fresh_oracle(top_k=3)
        fill(o, 0, dyadic_normal(rng, (T, 1, 8)), dyadic_normal(rng, (T, 1, 8)))
        res = o.decode(rng.standard_normal((1, 4, 8)), np.ones(4))
        assert [int(j) for j in res["sel"][0, 0] if j >= 0] == want, (T, res["sel"])
        assert np.all(res["o_rla"] == 0)


def pin_planted_blocks_selected():
    w = make_workload("tiny_fp32", t0=(1024,), steps=2)
    o = SplaOracle(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k, w.max_tokens())
    K, V = w.prefill(0)
    o.append([0], [K.shape[0]], K, V)
    st = w.step(0)
    o.append([0], [1], st["k"], st["v"])
    res = o.decode(st["q"], w.gate())
    plant = w.planted_blocks()[0]
    for g in range(w.n_kv_heads):
        assert set(plant[g]).issubset(set(res["sel"][0, g])), (plant[g], res["sel"][0, g])


def _rla_setup(rng, K_unsel=None, V_unsel=None):
    """T = 24 tokens (6 blocks of 4) of one KV head, selection fixed to
    {0, 2, 5} by override, so tokens 4..7 and 12..19 are the unselected
    ones; their K or V rows can be set."""
    T, d = 24, 8
    K = dyadic_normal(rng, (T, 1, d))
    V = dyadic_normal(rng, (T, 1, d))
    unsel = np.r_[4:8, 12:20]
    if K_unsel is not None:
        K[unsel, 0] = K_unsel
    if V_unsel is not None:
        V[unsel, 0] = V_unsel
    o = fresh_oracle(B=1, H=2, G=1, d=d, bk=4, top_k=3)
    fill(o, 0, K, V)
    sel = np.array([[[0, 2, 5]]])
    return o, K, V, unsel, sel


def pin_rla_normalized_is_unselected_mean():
    """Normalised form = linear attention over the unselected tokens with
    weights normalised to 1: equal unselected keys give equal weights, so
    the branch is the plain mean of their value rows; equal unselected
    values give that value whatever the keys."""
    rng = np.random.default_rng(21)
    gate = np.array([0.75, -0.5])
    kc = dyadic_normal(rng, (8,))
    o, K, V, unsel, sel = _rla_setup(rng, K_unsel=kc)
    q = rng.standard_normal((1, 2, 8))
    res = o.decode(q, gate, sel_override=sel, rla_mode=so.RLA_NORMALIZED)
    want = V[unsel, 0].mean(axis=0)
    for h in range(2):
        assert np.allclose(res["rla_out"][0, h], want, rtol=1e-12, atol=1e-12)
        assert np.allclose(res["o"][0, h], res["o_sparse"][0, h] + gate[h] * want, rtol=1e-12, atol=1e-12)
    c = dyadic_normal(rng, (8,))
    o, K, V, unsel, sel = _rla_setup(rng, V_unsel=c)
    res = o.decode(q, gate, sel_override=sel, rla_mode=so.RLA_NORMALIZED)
    for h in range(2):
        assert np.allclose(res["rla_out"][0, h], c, rtol=1e-12, atol=1e-12)


def pin_rla_rmsnorm_is_torch_rms_norm():
    """RMS-normalised form = torch's rms_norm over the head's d channels
    with weight gamma[h] (a library special case), and it is scale-free:
    values scaled by 8 give the same branch."""
    rng = np.random.default_rng(22)
    gate = np.array([0.25, 1.5])
    gamma = rng.uniform(0.5, 2.0, (2, 8))
    q = rng.standard_normal((1, 2, 8))
    for eps in (1e-3, 1e-6):
        o, K, V, unsel, sel = _rla_setup(rng)
        res = o.decode(q, gate, sel_override=sel, rla_mode=so.RLA_RMSNORM, gamma=gamma, eps=eps)
        for h in range(2):
            x = torch.tensor(res["o_rla"][0, h], dtype=torch.float64)
            ref = torch.nn.functional.rms_norm(x, (8,), weight=torch.tensor(gamma[h]), eps=eps).numpy()
            assert np.allclose(res["rla_out"][0, h], ref, rtol=1e-12, atol=1e-12)
            assert np.allclose(res["o"][0, h], res["o_sparse"][0, h] + gate[h] * ref, rtol=1e-12, atol=1e-12)
    o2 = fresh_oracle(B=1, H=2, G=1, d=8, bk=4, top_k=3)
    fill(o2, 0, K, 8 * V)
    res2 = o2.decode(q, gate, sel_override=sel, rla_mode=so.RLA_RMSNORM, gamma=gamma, eps=1e-12)
    res1 = o.decode(q, gate, sel_override=sel, rla_mode=so.RLA_RMSNORM, gamma=gamma, eps=1e-12)
    assert np.allclose(res2["rla_out"], res1["rla_out"], rtol=1e-9, atol=1e-12)


def pin_rla_forms_vanish_when_all_selected():
    """Every form of the branch is 0 when the selection covers every token,
    so o is the exact attention output."""
    rng = np.random.default_rng(23)
    o = fresh_oracle(B=1, H=2, G=1, d=8, bk=4, top_k=3)
    fill(o, 0, dyadic_normal(rng, (10, 1, 8)), dyadic_normal(rng, (10, 1, 8)))
    q = rng.standard_normal((1, 2, 8))
    for mode in (so.RLA_PLAIN, so.RLA_NORMALIZED, so.RLA_RMSNORM):
        res = o.decode(q, np.array([0.5, 2.0]), rla_mode=mode, gamma=np.ones((2, 8)))
        assert np.all(res["rla_out"] == 0) and np.array_equal(res["o"], res["o_sparse"])


def pin_exact_mass_factorial_closed_form():
    """Over the full 2^m sign design around k_bar the mean of exp(q_hat . k)
    factorises: exp(q_hat . k_bar) * prod_c cosh(q_hat_c t_c), exactly.  The
    Taylor score sits below it (cosh x >= 1 + x^2/2) and the mean-pooling
    score below both (Jensen)."""
    rng = np.random.default_rng(31)
    d = 8
    kbar = dyadic_normal(rng, (d,))
    axes = [0, 2, 3, 5, 6, 7]
    t = rng.uniform(0.2, 1.5, len(axes))
    keys = factorial_block(kbar, t, axes)
    for _ in range(5):
        q = rng.standard_normal((3, d)) * 2.0
        qh = q / math.sqrt(d)
        got = so.exact_block_log_mass(q, keys)
        want = qh @ kbar + sum(np.log(np.cosh(qh[:, c] * tc)) for c, tc in zip(axes, t))
        assert np.allclose(got, want, rtol=0, atol=1e-12), (got, want)
        mean, var = keys.mean(0), keys.var(0)
        tay = so.taylor_log_score(q, mean[None], var[None])[:, 0]
        mp = so.mean_pool_log_score(q, mean[None])[:, 0]
        assert np.all(mp <= tay + 1e-15) and np.all(tay <= got + 1e-15)
        assert np.allclose(mp, qh @ kbar, rtol=0, atol=1e-13)


def pin_exact_mass_identical_and_jensen():
    """Identical keys: exact mass = Taylor = mean pooling = q_hat . k.  Any
    keys: the exact mass is never below the mean-pooling score (Jensen), with
    the gap growing with the spread of q_hat . k."""
    rng = np.random.default_rng(32)
    d = 16
    k = dyadic_normal(rng, (d,))
    keys = np.repeat(k[None], 64, axis=0)
    q = rng.standard_normal((4, d))
    qh = q / math.sqrt(d)
    assert np.allclose(so.exact_block_log_mass(q, keys), qh @ k, rtol=0, atol=1e-13)
    for scale in (0.1, 1.0, 3.0):
        keys = k[None] + scale * rng.standard_normal((64, d))
        ex = so.exact_block_log_mass(q, keys)
        mp = so.mean_pool_log_score(q, keys.mean(0)[None])[:, 0]
        assert np.all(ex >= mp - 1e-13)
    # group exact mass of the oracle state = sum over heads of the per-token mean mass
    o = fresh_oracle(B=1, H=4, G=2, d=8, bk=4, top_k=3)
    K = dyadic_normal(rng, (20, 2, 8))
    fill(o, 0, K, dyadic_normal(rng, (20, 2, 8)))
    qq = rng.standard_normal((4, 8))
    ex = o.block_exact_scores(0, 1, qq)
    assert sorted(ex) == [1, 2, 3]
    for j, x in ex.items():
        s = K[4 * j:4 * j + 4, 1].astype(F64) @ (qq[2:4] / math.sqrt(8)).T
        assert abs(math.exp(x) - np.exp(s).mean(axis=0).sum()) <= 1e-12 * math.exp(x)


def pin_score_forms_select_differently():
    """Blocks with the same mean but a larger spread along the query have a
    larger exact mass; the Taylor score ranks them first, mean pooling ties
    them with the others (then ids decide)."""
    rng = np.random.default_rng(33)
    d, bk = 8, 16
    u = np.zeros(d); u[0] = 1.0
    nblk = 10
    K = np.zeros((nblk * bk, 1, d))
    spread = {7: 2.0, 8: 2.0}  # wide blocks along u
    for j in range(nblk):
        sgn = np.where(np.arange(bk) % 2 == 0, 1.0, -1.0)
        K[j * bk:(j + 1) * bk, 0] = np.outer(sgn * spread.get(j, 0.25), u)
    o = SplaOracle(1, 1, 1, d, bk, 4, 256)
    fill(o, 0, K, dyadic_normal(rng, (nblk * bk, 1, d)))
    q = (3.0 * u)[None, None]
    r_t = o.decode(q, np.ones(1))
    r_m = o.decode(q, np.ones(1), score_form=so.SCORE_MEAN)
    assert [int(j) for j in r_t["sel"][0, 0]] == [0, 7, 8, 9]
    assert [int(j) for j in r_m["sel"][0, 0]] == [0, 1, 2, 9]
    ex = o.block_exact_scores(0, 0, q[0])
    assert sorted(ex, key=lambda j: (-ex[j], j))[:2] == [7, 8]


def pin_prefill_all_selected_is_causal_sdpa():
    """While every block of a token's prefix is selected, its prefill output
    is causal softmax attention over its prefix (torch SDPA with a causal
    mask, fp64 on the CPU) and its RLA branch is 0; the first token of an
    empty sequence returns its own value."""
    rng = np.random.default_rng(41)
    G, H, d, bk, k = 2, 4, 8, 4, 3
    n = bk * k  # every prefix fits in top_k blocks
    o = SplaOracle(2, H, G, d, bk, k, 64)
    K = dyadic_normal(rng, (n, G, d))
    V = dyadic_normal(rng, (n, G, d))
    Q = rng.standard_normal((n, H, d))
    res = o.prefill_sequence(1, K.astype(np.float32), V.astype(np.float32), Q, np.full(H, 0.7))
    assert np.all(res["o_rla"] == 0) and np.allclose(res["o"], res["o_sparse"], rtol=0, atol=0)
    for h in range(H):
        g = h // (H // G)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(Q[None, :, h]), torch.tensor(K[None, :, g]), torch.tensor(V[None, :, g]),
            is_causal=True)[0].numpy()
        assert np.allclose(res["o"][:, h], ref, rtol=1e-12, atol=1e-12), h
    assert np.allclose(res["o"][0, 0], V[0, 0], rtol=0, atol=1e-15)
    assert list(o.lens) == [0, n]


def pin_prefill_rla_is_direct_over_each_prefix():
    """Past the selection's reach, each prefill token's RLA branch equals the
    direct sum over the unselected tokens of its own prefix (brute force), so
    the linear-attention state is the prefix state of that token; a chunk
    split in two gives the same outputs."""
    rng = np.random.default_rng(42)
    G, H, d, bk, k = 1, 2, 8, 4, 3
    T0, n = 21, 14
    K = dyadic_normal(rng, (T0 + n, G, d))
    V = dyadic_normal(rng, (T0 + n, G, d))
    Q = rng.standard_normal((n, H, d))
    gate = np.array([0.5, 1.5])
    o = SplaOracle(1, H, G, d, bk, k, 64)
    fill(o, 0, K[:T0], V[:T0])
    res = o.prefill_sequence(0, K[T0:].astype(np.float32), V[T0:].astype(np.float32), Q, gate, brute_rla=True)
    assert np.abs(res["o_rla"]).max() > 0
    scale = np.abs(res["o_rla_direct"]).max()
    assert np.abs(res["o_rla"] - res["o_rla_direct"]).max() <= 1e-11 * scale
    assert np.abs(res["d_rla"] - res["d_rla_direct"]).max() <= 1e-11 * np.abs(res["d_rla_direct"]).max()
    o2 = SplaOracle(1, H, G, d, bk, k, 64)
    fill(o2, 0, K[:T0], V[:T0])
    a = o2.prefill_sequence(0, K[T0:T0 + 5].astype(np.float32), V[T0:T0 + 5].astype(np.float32), Q[:5], gate)
    b2 = o2.prefill_sequence(0, K[T0 + 5:].astype(np.float32), V[T0 + 5:].astype(np.float32), Q[5:], gate)
    assert np.allclose(np.concatenate([a["o"], b2["o"]]), res["o"], rtol=1e-12, atol=1e-12)


ALL_PINS = [
    pin_phi, pin_block_stats_factorial, pin_score_identical_keys, pin_score_factorial_closed_form,
    pin_score_vs_bruteforce_low_variance, pin_group_score, pin_selection_properties,
    pin_all_selected_is_dense_attention, pin_sparse_is_masked_attention_and_rla_is_direct,
    pin_global_state_is_phiK_T_V, pin_gqa_head_map, pin_edge_lengths, pin_planted_blocks_selected,
    pin_rla_normalized_is_unselected_mean, pin_rla_rmsnorm_is_torch_rms_norm, pin_rla_forms_vanish_when_all_selected,
    pin_exact_mass_factorial_closed_form, pin_exact_mass_identical_and_jensen, pin_score_forms_select_differently,
    pin_prefill_all_selected_is_causal_sdpa, pin_prefill_rla_is_direct_over_each_prefix,
]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_chunk_invariance():
    rng = np.random.default_rng(11)
    T = 77
    K = dyadic_normal(rng, (T, 2, 8)).astype(np.float32)
    V = dyadic_normal(rng, (T, 2, 8)).astype(np.float32)
    a = SplaOracle(1, 2, 2, 8, 8, 4, 128)
    a.append([0], [T], K, V)
    b = SplaOracle(1, 2, 2, 8, 8, 4, 128)
    for p in range(T):
        b.append([0], [1], K[p:p + 1], V[p:p + 1])
    assert np.allclose(a.S, b.S, rtol=1e-13, atol=1e-13)
    assert np.array_equal(a.mean, b.mean) and np.array_equal(a.var, b.var)
    q = rng.standard_normal((1, 2, 8))
    ra, rb = a.decode(q, np.ones(2)), b.decode(q, np.ones(2))
    assert np.array_equal(ra["sel"], rb["sel"])
    assert np.allclose(ra["o"], rb["o"], rtol=1e-12, atol=1e-12)


def test_bf16_generator_rounding_is_rne():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * 37
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(round_bf16(x), ref)


def test_workload_chunking_invariant():
    w = make_workload("million_1m", t0=(3000,), steps=2, prefill_chunk=1024)
    a = np.concatenate([k for _, k, _ in w.prefill_chunks(0, 1024)])
    b = np.concatenate([k for _, k, _ in w.prefill_chunks(0, 700)])
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ mutants
def _mut_sample_var(keys):
    keys = np.asarray(keys, F64)
    n = keys.shape[0]
    m = keys.sum(0) / n
    return m, ((keys - m) ** 2).sum(0) / (n - 1)


def _mut_no_half(q, mean, var):
    qh = np.asarray(q, F64) / math.sqrt(q.shape[-1])
    return qh @ np.asarray(mean).T + np.log1p((qh * qh) @ np.asarray(var).T)


def _mut_no_temperature(q, mean, var):
    q = np.asarray(q, F64)
    return q @ np.asarray(mean).T + np.log1p(0.5 * (q * q) @ np.asarray(var).T)


def _mut_first_order_sign(q, mean, var):
    qh = np.asarray(q, F64) / math.sqrt(q.shape[-1])
    return -(qh @ np.asarray(mean).T) + np.log1p(0.5 * (qh * qh) @ np.asarray(var).T)


def _mut_var_as_std(q, mean, var):
    qh = np.asarray(q, F64) / math.sqrt(q.shape[-1])
    return qh @ np.asarray(mean).T + np.log1p(0.5 * (qh * qh) @ np.sqrt(np.asarray(var)).T)


def _mut_phi_elu(x):
    x = np.asarray(x, F64)
    return np.where(x > 0, x, np.exp(np.minimum(x, 0)) - 1)


def _mut_phi_exp(x):
    return np.exp(np.asarray(x, F64))


def _mut_group_max(ls):
    return np.asarray(ls, F64).max(axis=0)


def _mut_select_no_sink(lg, nb, top_k):
    if nb <= top_k:
        return list(range(nb))
    order = sorted(range(1, nb - 1), key=lambda j: (-lg[j], j))
    return sorted(set(order[: top_k - 1]) | {nb - 1})


def _mut_select_ascending(lg, nb, top_k):
    if nb <= top_k:
        return list(range(nb))
    order = sorted(range(1, nb - 1), key=lambda j: (lg[j], j))
    return sorted(set(order[: top_k - 2]) | {0, nb - 1})


def _mut_softmax_no_scale(q, k, v):
    s = np.asarray(k, F64) @ np.asarray(q, F64)
    p = np.exp(s - s.max())
    return (p / p.sum()) @ np.asarray(v, F64)


def _mut_la_transposed(f, k, v):
    # phi applied to v instead of k: a swapped operand
    w = so.phi(v) @ np.asarray(f, F64)
    return w @ np.asarray(k, F64), w.sum()


def _mut_rla_no_divide(o_rla, d_rla, mode, gamma=None, eps=1e-6, covers_all=False):
    if mode == so.RLA_NORMALIZED and not covers_all:
        return np.asarray(o_rla, F64)
    return _ORIG_RLA_BRANCH(o_rla, d_rla, mode, gamma, eps, covers_all)


def _mut_rla_rms_sum(o_rla, d_rla, mode, gamma=None, eps=1e-6, covers_all=False):
    if mode == so.RLA_RMSNORM and not covers_all:
        x = np.asarray(o_rla, F64)
        return np.asarray(gamma) * x / math.sqrt(float(np.sum(x * x)) + eps)
    return _ORIG_RLA_BRANCH(o_rla, d_rla, mode, gamma, eps, covers_all)


def _mut_rla_rms_eps_outside(o_rla, d_rla, mode, gamma=None, eps=1e-6, covers_all=False):
    if mode == so.RLA_RMSNORM and not covers_all:
        x = np.asarray(o_rla, F64)
        return np.asarray(gamma) * x / (math.sqrt(float(np.mean(x * x))) + eps)
    return _ORIG_RLA_BRANCH(o_rla, d_rla, mode, gamma, eps, covers_all)


def _mut_rla_rms_no_gamma(o_rla, d_rla, mode, gamma=None, eps=1e-6, covers_all=False):
    return _ORIG_RLA_BRANCH(o_rla, d_rla, mode, None if gamma is None else np.ones_like(gamma), eps, covers_all)


def _mut_rla_no_zero_when_covered(o_rla, d_rla, mode, gamma=None, eps=1e-6, covers_all=False):
    x = np.asarray(o_rla, F64) + 1.0
    return _ORIG_RLA_BRANCH(x, d_rla, mode, gamma, eps, False) if covers_all else \
        _ORIG_RLA_BRANCH(o_rla, d_rla, mode, gamma, eps, covers_all)


_ORIG_RLA_BRANCH = so.rla_branch


def _mut_mass_sum_not_mean(q, keys):
    return _ORIG_EXACT_MASS(q, keys) + math.log(np.asarray(keys).shape[0])


def _mut_mass_no_temperature(q, keys):
    q = np.asarray(q, F64)
    return _ORIG_EXACT_MASS(q * math.sqrt(q.shape[-1]), keys)


def _mut_mass_max_token(q, keys):
    q = np.asarray(q, F64)
    return (np.asarray(keys, F64) @ (q / math.sqrt(q.shape[-1])).T).max(axis=0)


def _mut_mean_pool_with_var(q, mean):
    return _ORIG_MEAN_POOL(q, mean) + 0.01


def _mut_mean_pool_raw_q(q, mean):
    return np.asarray(q, F64) @ np.asarray(mean, F64).T


_ORIG_EXACT_MASS = so.exact_block_log_mass
_ORIG_MEAN_POOL = so.mean_pool_log_score


class _MutOracleChunkFirst(SplaOracle):
    """prefill that appends the whole chunk before decoding its tokens"""
    def prefill_sequence(self, b, k_new, v_new, q_new, gate, **kw):
        n = k_new.shape[0]
        self.append([b], [n], k_new, v_new)
        keys = ["o", "o_sparse", "o_rla", "rla_out", "d_rla", "sel"] + (
            ["o_rla_direct", "d_rla_direct"] if kw.get("brute_rla") else [])
        res = {k: [] for k in keys}
        q = np.zeros((self.B, self.H, self.d))
        for t in range(n):
            q[b] = q_new[t]
            r = self.decode(q, gate, seqs=[b], **kw)
            for k in keys:
                res[k].append(np.array(r[k][b]))
        return {k: np.stack(v) for k, v in res.items()}

    # (lg is not needed by the pins)


class _MutOracleStateAfterToken(SplaOracle):
    """prefill whose linear-attention state lags one token behind"""
    def prefill_sequence(self, b, k_new, v_new, q_new, gate, **kw):
        res = super().prefill_sequence(b, k_new, v_new, q_new, gate, **kw)
        res["o_rla"] = np.concatenate([np.zeros_like(res["o_rla"][:1]), res["o_rla"][:-1]])
        return res


class _MutOracleSTransposed(SplaOracle):
    def append(self, seq_ids, n_new, k_new, v_new):
        super().append(seq_ids, n_new, k_new, v_new)
        self.S = np.swapaxes(self.S, -1, -2).copy()


MUTANTS = {
    "sample_variance": ("block_stats", _mut_sample_var),
    "no_half": ("taylor_log_score", _mut_no_half),
    "no_temperature": ("taylor_log_score", _mut_no_temperature),
    "first_order_sign": ("taylor_log_score", _mut_first_order_sign),
    "var_as_std": ("taylor_log_score", _mut_var_as_std),
    "phi_elu_without_1": ("phi", _mut_phi_elu),
    "phi_exp": ("phi", _mut_phi_exp),
    "group_max": ("group_log_score", _mut_group_max),
    "no_sink": ("select_blocks", _mut_select_no_sink),
    "ascending": ("select_blocks", _mut_select_ascending),
    "softmax_no_scale": ("softmax_attention", _mut_softmax_no_scale),
    "la_swapped": ("linear_attention_numerator", _mut_la_transposed),
    "rla_normalized_no_divide": ("rla_branch", _mut_rla_no_divide),
    "rla_rms_over_sum": ("rla_branch", _mut_rla_rms_sum),
    "rla_rms_eps_outside_sqrt": ("rla_branch", _mut_rla_rms_eps_outside),
    "rla_rms_without_gamma": ("rla_branch", _mut_rla_rms_no_gamma),
    "rla_not_zero_when_covered": ("rla_branch", _mut_rla_no_zero_when_covered),
    "mass_sum_not_mean": ("exact_block_log_mass", _mut_mass_sum_not_mean),
    "mass_no_temperature": ("exact_block_log_mass", _mut_mass_no_temperature),
    "mass_max_token": ("exact_block_log_mass", _mut_mass_max_token),
    "mean_pool_offset": ("mean_pool_log_score", _mut_mean_pool_with_var),
    "mean_pool_raw_q": ("mean_pool_log_score", _mut_mean_pool_raw_q),
}


def _any_pin_fails():
    for pin in ALL_PINS + [test_chunk_invariance]:
        try:
            pin()
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(so, attr, fn)
    assert _any_pin_fails(), f"mutant {name} passes every pin"


def test_mutant_transposed_state_is_caught(monkeypatch):
    monkeypatch.setitem(globals(), "SplaOracle", _MutOracleSTransposed)
    assert _any_pin_fails()


@pytest.mark.parametrize("cls", [_MutOracleChunkFirst, _MutOracleStateAfterToken], ids=lambda c: c.__name__)
def test_mutant_prefill_is_caught(cls, monkeypatch):
    monkeypatch.setitem(globals(), "SplaOracle", cls)
    assert _any_pin_fails()


def test_mutant_rla_sign_is_caught(monkeypatch):
    orig = so.SplaOracle.decode

    def bad(self, q, gate, sel_override=None, brute_rla=False, **kw):
        r = orig(self, q, gate, sel_override, brute_rla, **kw)
        r["o_rla"] = r["o_bar"] + r["o_tilde"]
        return r

    monkeypatch.setattr(so.SplaOracle, "decode", bad)
    assert _any_pin_fails()
