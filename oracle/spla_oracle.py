"""fp64 CPU oracle of the SPLA decode step (block statistics, Taylor block
score, top-k block selection, exact sparse attention, subtraction-form
Residual Linear Attention, gated combine) and of the state append that feeds
it.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (``block_sparse_linear_amd``) never does; it fails loudly when
its HIP library is missing instead of falling back to this code.  It shares
no code with the HIP path: plain NumPy in float64, written from the SPLA
pages, one step after another in the order the pages give them.

Sources (web pages about arXiv 2601.22379, "SPLA: Block Sparse Plus Linear
Attention for Long Context Modeling"):
  [TS]   gist.science "Technical Summary: SPLA - Block Sparse Plus Linear
         Attention for Long Context Modeling" (English), sections 1-2.3.
  [TS-de] the German translation of the same summary on gist.science/de.
  [SA]   Baidu Cloud, "Sparse Attention for Long-Context LLMs: Implementation
         and Trade-off Design", section 1 (softmax(QK^T/sqrt(d))V) and
         section 7 (kernelised linear attention phi(Q)(phi(K)^T V)).
The step's fixed parameters that the pages leave open are those of the
decode specification this library implements: phi(x) = elu(x) + 1,
o = o_sparse + g_h * o_rla with a per-query-head gate g_h, block 0 (sink)
and the current block always selected, q.k scaled by 1/sqrt(d), fp32 block
mean/variance and S_all / z_all per KV head on the GPU side.

Readings taken where the pages are silent or loose (each one is also listed
with its reason in the design notes):
  R1  the score uses q_hat = q / sqrt(d) in both the exponent and the
      variance term (it is the expansion of E[exp(q_hat . k)], the same
      exponent the softmax uses);
  R2  Cov(k) is the population (divide by Bk) diagonal covariance of the
      block's keys;
  R3  the score is computed in the log domain: ls = q_hat.mu + log1p(1/2 *
      sum_c q_hat_c^2 var_c);
  R4  GQA: one selection per (sequence, KV head).  The group score of a block
      is the sum over the group's query heads of their Taylor masses, i.e.
      LG = logsumexp_h ls_h;
  R5  top_k counts the sink and the current block; the candidates are blocks
      1 .. nb-2 and k' = top_k - 2 of them are kept; when nb <= top_k every
      block is kept;
  R6  ties in LG go to the smaller block id;
  R7  phi is applied to raw q and k (elementwise, alpha = 1);
  R8  o_bar and o_tilde are the unnormalised linear-attention numerators
      phi(q)^T S_all and phi(q)^T sum_sel phi(k) v^T; the normaliser
      difference D = phi(q).(z_all - z_sel) is reported beside them;
  R9  o_rla (and D) is exactly 0 when the selection covers every token;
  R10 a decode step first appends the new token to the state, then decodes
      (the token attends to itself);
  R11 output forms of the RLA branch (the specification's combine uses o_rla
      as it is; the two others are options): "normalised" divides o_rla by
      D, which makes it the standard normalised linear attention over the
      unselected tokens; "RMS-normalised" is gamma * o_rla / sqrt(mean_c
      o_rla_c^2 + eps) over the d channels of one query head, with a scale
      gamma per (query head, channel) and eps > 0 given by the caller.  The
      gate multiplies the branch in every form, and the branch is 0 in every
      form when the selection covers every token;
  R12 selection fidelity: a block's exact mass is the per-token mean of
      exp(q_hat . k) over its keys (the form of the score formula, R1),
      summed over the group's query heads as in R4; the mean-pooling
      baseline keeps only the first-order term q_hat . k_bar;
  R13 chunked prefill of one sequence: every new token gets the decode result
      at its own position, as if the chunk were appended and decoded one
      token at a time (the token attends to itself and to every earlier
      token, R10; its selection, exact attention and linear-attention state
      are those of its own prefix).

Parity of this module is pinned by ``tests/test_oracle_pins.py`` against
closed forms, library special cases and brute force; the readings R4, R7 and
R8 are choices of the specification, not statements of the pages, so
agreement with the pages is unpinned for them beyond their definitions.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

F64 = np.float64


# --------------------------------------------------------------- feature map
def phi(x: np.ndarray) -> np.ndarray:
    """phi(x) = elu(x) + 1 = x + 1 for x > 0, exp(x) otherwise (R7).

    [TS] 2.3 asks for a parameter-free feature map close to exp; the
    decode specification fixes it to elu + 1."""
    x = np.asarray(x, dtype=F64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


# ---------------------------------------------------------- block statistics
def block_stats(keys: np.ndarray):
    """First and second order statistics of one block's keys ([TS] 2.1,
    implementation paragraph: diagonal covariance instead of O(d^2)).

    keys: [n][d].  Returns (mean [d], var [d]); var is the population
    variance (R2), computed in two passes."""
    keys = np.asarray(keys, dtype=F64)
    n = keys.shape[0]
    mean = keys.sum(axis=0) / n
    dev = keys - mean
    var = (dev * dev).sum(axis=0) / n
    return mean, var


# ------------------------------------------------------------- block score
def taylor_log_score(q: np.ndarray, mean: np.ndarray, var: np.ndarray) -> np.ndarray:
    """Log of the second-order Taylor block score ([TS] 2.1, score formula
    exp(q.k_bar)(1 + 1/2 q^T Cov(k) q), with the diagonal covariance of the
    implementation paragraph and the 1/sqrt(d) temperature, R1 and R3).

    q: [h][d] query heads, mean/var: [j][d].  Returns ls [h][j]."""
    q = np.asarray(q, dtype=F64)
    d = q.shape[-1]
    qh = q / math.sqrt(d)
    first = qh @ np.asarray(mean, dtype=F64).T
    second = 0.5 * ((qh * qh) @ np.asarray(var, dtype=F64).T)
    return first + np.log1p(second)


def mean_pool_log_score(q: np.ndarray, mean: np.ndarray) -> np.ndarray:
    """Log of the first-order (mean-pooling) block score exp(q_hat.k_bar):
    the Taylor score with its variance term left out, the heuristic pooling
    baseline [TS] 3 contrasts the second-order selection with.

    q: [h][d], mean: [j][d].  Returns ls [h][j]."""
    q = np.asarray(q, dtype=F64)
    qh = q / math.sqrt(q.shape[-1])
    return qh @ np.asarray(mean, dtype=F64).T


def exact_block_log_mass(q: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Log of the exact mean attention mass of one block, log (1/n) sum_i
    exp(q_hat . k_i), per query head: the quantity the Taylor score
    approximates ([TS] 2.1 objective: the block's integrated probability
    mass, in the per-token mean form of its score formula).

    q: [h][d], keys: [n][d].  Returns [h]."""
    q = np.asarray(q, dtype=F64)
    qh = q / math.sqrt(q.shape[-1])
    s = np.asarray(keys, dtype=F64) @ qh.T  # [n][h]
    m = s.max(axis=0)
    return m + np.log(np.exp(s - m[None, :]).sum(axis=0)) - math.log(s.shape[0])


def group_log_score(ls: np.ndarray) -> np.ndarray:
    """LG[j] = log sum_h exp(ls[h][j]) (R4): the summed Taylor mass of a
    block over the query heads sharing one KV head."""
    ls = np.asarray(ls, dtype=F64)
    m = ls.max(axis=0)
    return m + np.log(np.exp(ls - m[None, :]).sum(axis=0))


# --------------------------------------------------------------- selection
def select_blocks(lg: Dict[int, float], nb: int, top_k: int) -> List[int]:
    """Top-k block selection ([TS] 1 and 2.1: load only the most relevant
    blocks; [SA] 5: sort by score and keep the top K), with the sink and the
    current block always kept (R5) and ties to the smaller id (R6).

    lg maps candidate block id -> group log score.  Returns the selected
    block ids in ascending order."""
    cur = nb - 1
    if nb <= top_k:
        return list(range(nb))
    cand = list(range(1, nb - 1))
    order = sorted(cand, key=lambda j: (-lg[j], j))
    kept = set(order[: top_k - 2]) | {0, cur}
    return sorted(kept)


# ---------------------------------------------------- exact sparse attention
def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v over the given token rows ([SA] 1;
    [TS] 2: exact attention over the selected blocks).  q: [d], k, v: [n][d]."""
    q = np.asarray(q, dtype=F64)
    d = q.shape[-1]
    s = np.asarray(k, dtype=F64) @ q / math.sqrt(d)
    p = np.exp(s - s.max())
    p = p / p.sum()
    return p @ np.asarray(v, dtype=F64)


# ------------------------------------------------- residual linear attention
def linear_attention_numerator(f: np.ndarray, k: np.ndarray, v: np.ndarray):
    """Unnormalised linear attention of feature query f over token rows k, v
    ([SA] 7, numerator phi(Q)(phi(K)^T V); R8).  Returns (sum_i w_i v_i,
    sum_i w_i) with w_i = f . phi(k_i)."""
    w = phi(k) @ np.asarray(f, dtype=F64)
    return w @ np.asarray(v, dtype=F64), w.sum()


# ------------------------------------------- output forms of the RLA branch
RLA_PLAIN, RLA_NORMALIZED, RLA_RMSNORM = 0, 1, 2
# block scores for the selection: second-order Taylor (the method) or the
# first-order mean-pooling baseline
SCORE_TAYLOR, SCORE_MEAN = 0, 1


def rla_branch(o_rla: np.ndarray, d_rla: float, mode: int, gamma: Optional[np.ndarray] = None,
               eps: float = 1e-6, covers_all: bool = False) -> np.ndarray:
    """The RLA branch of one query head as it enters the gated sum (R11).

    RLA_PLAIN       o_rla (the specification's combine).
    RLA_NORMALIZED  o_rla / D.  By the subtraction form of [TS] 2.2, o_rla
                    and D are the numerator phi(q)^T sum phi(k) v^T and the
                    denominator phi(q) . sum phi(k) of linear attention over
                    the unselected tokens, so the ratio is the normalised
                    kernel form phi(Q)(phi(K)^T V) / phi(Q)(phi(K)^T 1) of
                    [SA] 7 restricted to them.
    RLA_RMSNORM     gamma * o_rla / sqrt(mean_c o_rla_c^2 + eps): [TS] 2.3
                    normalises the RLA output with an RMS norm whose scale
                    parameters are the method's only added weights.
    Zero in every form when the selection covers every token (R9)."""
    o_rla = np.asarray(o_rla, dtype=F64)
    if covers_all:
        return np.zeros_like(o_rla)
    if mode == RLA_PLAIN:
        return o_rla
    if mode == RLA_NORMALIZED:
        return o_rla / float(d_rla)
    if mode == RLA_RMSNORM:
        ms = float(np.mean(o_rla * o_rla))
        return np.asarray(gamma, dtype=F64) * o_rla / math.sqrt(ms + float(eps))
    raise ValueError(f"unknown RLA output form {mode}")


class SplaOracle:
    """The decode state of one SPLA attention layer and its two operations.

    State per sequence b and KV head g ([TS] 2.1 and 2.2):
      K, V            every key / value row so far (stored as float32, which
                      holds the bf16 or f32 inputs exactly; widened to fp64
                      at every use)
      mean, var       statistics of every complete block
      S = sum phi(k) v^T (d x d) and z = sum phi(k) (d): the running global
                      linear-attention state ([TS] 2.2, o_bar over all blocks)
    """

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 block_size: int, top_k: int, capacity_tokens: int):
        if n_q_heads % n_kv_heads:
            raise ValueError("n_q_heads must be a multiple of n_kv_heads")
        self.B, self.H, self.G, self.d = batch, n_q_heads, n_kv_heads, head_dim
        self.r = n_q_heads // n_kv_heads
        self.bk, self.top_k = block_size, top_k
        self.cap = capacity_tokens
        nbc = -(-capacity_tokens // block_size)
        self.K = [np.zeros((capacity_tokens, n_kv_heads, head_dim), np.float32) for _ in range(batch)]
        self.V = [np.zeros((capacity_tokens, n_kv_heads, head_dim), np.float32) for _ in range(batch)]
        self.mean = np.zeros((batch, n_kv_heads, nbc, head_dim), F64)
        self.var = np.zeros((batch, n_kv_heads, nbc, head_dim), F64)
        self.S = np.zeros((batch, n_kv_heads, head_dim, head_dim), F64)
        self.z = np.zeros((batch, n_kv_heads, head_dim), F64)
        self.lens = np.zeros(batch, np.int64)

    # ------------------------------------------------------------- append
    def append(self, seq_ids: Sequence[int], n_new: Sequence[int],
               k_new: np.ndarray, v_new: np.ndarray) -> None:
        """Append n_new[i] rows of k_new / v_new ([sum n][G][d], sequence-major)
        to sequence seq_ids[i]: store them, add phi(k) v^T and phi(k) to S and
        z, and compute the statistics of every block this append completes."""
        row = 0
        for b, n in zip(seq_ids, n_new):
            b, n = int(b), int(n)
            kb = np.asarray(k_new[row:row + n], np.float32)
            vb = np.asarray(v_new[row:row + n], np.float32)
            row += n
            t0 = int(self.lens[b])
            t1 = t0 + n
            if t1 > self.cap:
                raise ValueError("capacity exceeded")
            self.K[b][t0:t1] = kb
            self.V[b][t0:t1] = vb
            for g in range(self.G):
                fk = phi(kb[:, g, :])
                self.S[b, g] += fk.T @ vb[:, g, :].astype(F64)
                self.z[b, g] += fk.sum(axis=0)
            for j in range(t0 // self.bk, t1 // self.bk):
                for g in range(self.G):
                    keys = self.K[b][j * self.bk:(j + 1) * self.bk, g, :]
                    self.mean[b, g, j], self.var[b, g, j] = block_stats(keys)
            self.lens[b] = t1

    def append_bulk(self, b: int, k: np.ndarray, v: np.ndarray) -> None:
        """Same result as append([b], [n], k, v) (up to fp64 rounding order)
        for a long prefill: S by one matrix product per KV head, the block
        statistics block by block."""
        self.append([b], [k.shape[0]], k, v)

    # ------------------------------------------------------------- decode
    def block_group_scores(self, b: int, g: int, q: np.ndarray,
                           score_form: int = SCORE_TAYLOR) -> Dict[int, float]:
        """LG of every candidate block 1..nb-2 of (b, g) for queries q [H][d],
        from the second-order Taylor score (default) or the first-order
        mean-pooling score."""
        T = int(self.lens[b])
        nb = -(-T // self.bk)
        cand = np.arange(1, max(nb - 1, 1))
        if len(cand) == 0:
            return {}
        heads = q[g * self.r:(g + 1) * self.r]
        if score_form == SCORE_TAYLOR:
            ls = taylor_log_score(heads, self.mean[b, g, cand], self.var[b, g, cand])
        elif score_form == SCORE_MEAN:
            ls = mean_pool_log_score(heads, self.mean[b, g, cand])
        else:
            raise ValueError(f"unknown score form {score_form}")
        lg = group_log_score(ls)
        return {int(j): float(x) for j, x in zip(cand, lg)}

    def block_exact_scores(self, b: int, g: int, q: np.ndarray) -> Dict[int, float]:
        """Exact group log mass of every candidate block 1..nb-2 of (b, g):
        log sum_h (1/Bk) sum_{i in j} exp(q_hat_h . k_i), from the stored keys."""
        T = int(self.lens[b])
        nb = -(-T // self.bk)
        heads = np.asarray(q, dtype=F64)[g * self.r:(g + 1) * self.r]
        out = {}
        for j in range(1, max(nb - 1, 1)):
            keys = self.K[b][j * self.bk:(j + 1) * self.bk, g, :]
            out[j] = float(group_log_score(exact_block_log_mass(heads, keys)[:, None])[0])
        return out

    def prefill_sequence(self, b: int, k_new: np.ndarray, v_new: np.ndarray, q_new: np.ndarray,
                         gate: np.ndarray, sel_per_token: Optional[np.ndarray] = None,
                         **decode_kw) -> Dict[str, object]:
        """Chunked prefill of sequence b (R13): for each new token t in order,
        append k_new[t], v_new[t] ([n][G][d]) and decode q_new[t] ([n][H][d])
        for sequence b alone.  sel_per_token: optional [n][G][k] selections to
        use instead of the oracle's own (per token).  decode_kw go to decode
        (output form, score form, brute_rla).  Returns o, o_sparse, o_rla,
        rla_out [n][H][d], d_rla [n][H], sel [n][G][top_k], lg (per token, per
        KV head {block: LG}) (and o_rla_direct / d_rla_direct with brute_rla)."""
        n = int(k_new.shape[0])
        keys = ["o", "o_sparse", "o_rla", "rla_out", "d_rla", "sel", "lg"]
        if decode_kw.get("brute_rla"):
            keys += ["o_rla_direct", "d_rla_direct"]
        res = {k: [] for k in keys}
        q = np.zeros((self.B, self.H, self.d), F64)
        for t in range(n):
            self.append([b], [1], k_new[t:t + 1], v_new[t:t + 1])
            q[b] = q_new[t]
            ov = None
            if sel_per_token is not None:
                ov = np.full((self.B, self.G, self.top_k), -1, np.int64)
                ov[b] = sel_per_token[t]
            r = self.decode(q, gate, sel_override=ov, seqs=[b], **decode_kw)
            for k in keys:
                res[k].append(r[k][b] if k == "lg" else np.array(r[k][b]))
        return {k: (v if k == "lg" else (np.stack(v) if v else np.zeros((0,)))) for k, v in res.items()}

    def decode(self, q: np.ndarray, gate: np.ndarray,
               sel_override: Optional[np.ndarray] = None,
               brute_rla: bool = False, rla_mode: int = RLA_PLAIN,
               gamma: Optional[np.ndarray] = None, eps: float = 1e-6,
               score_form: int = SCORE_TAYLOR,
               seqs: Optional[Sequence[int]] = None) -> Dict[str, object]:
        """One decode step for every sequence (after that step's append).

        q: [B][H][d] queries, gate: [H].  sel_override: optional [B][G][k]
        block ids (-1 padded) used instead of the oracle's own selection
        (the scores are still computed and returned).  rla_mode, gamma
        ([H][d]) and eps choose the output form of the RLA branch
        (rla_branch); o = o_sparse + gate * branch.  score_form chooses the
        block score the selection ranks (SCORE_TAYLOR or SCORE_MEAN).  seqs:
        decode only these sequences (the other rows of the results stay 0).

        Returns a dict with o, o_sparse, o_rla, o_bar, o_tilde, rla_out
        (the branch in the chosen form) ([B][H][d]),
        d_rla [B][H], sel [B][G][top_k] (ascending, -1 padded), lg (list per
        b of list per g of {block: LG}), and, with brute_rla, o_rla_direct /
        d_rla_direct summed directly over the unselected tokens."""
        B, H, G, d, r, bk = self.B, self.H, self.G, self.d, self.r, self.bk
        q = np.asarray(q, dtype=F64)
        gate = np.asarray(gate, dtype=F64)
        out = {k: np.zeros((B, H, d), F64) for k in
               ("o", "o_sparse", "o_rla", "o_bar", "o_tilde", "rla_out")}
        if rla_mode == RLA_RMSNORM and gamma is None:
            raise ValueError("the RMS-normalised form needs gamma")
        out["d_rla"] = np.zeros((B, H), F64)
        out["sel"] = np.full((B, G, self.top_k), -1, np.int64)
        out["lg"] = [[None] * G for _ in range(B)]
        if brute_rla:
            out["o_rla_direct"] = np.zeros((B, H, d), F64)
            out["d_rla_direct"] = np.zeros((B, H), F64)
        for b in (range(B) if seqs is None else [int(x) for x in seqs]):
            T = int(self.lens[b])
            if T == 0:
                raise ValueError("decode on an empty sequence")
            nb = -(-T // bk)
            for g in range(G):
                # (1) block scores and (2) selection
                lg = self.block_group_scores(b, g, q[b], score_form)
                out["lg"][b][g] = lg
                if sel_override is not None:
                    sel = sorted(int(j) for j in sel_override[b][g] if j >= 0)
                else:
                    sel = select_blocks(lg, nb, self.top_k)
                out["sel"][b, g, :len(sel)] = sel
                tok = np.concatenate([np.arange(j * bk, min((j + 1) * bk, T)) for j in sel])
                ku = self.K[b][tok, g, :].astype(F64)
                vu = self.V[b][tok, g, :].astype(F64)
                covers_all = len(tok) == T
                if brute_rla:
                    mask = np.ones(T, bool)
                    mask[tok] = False
                    kn = self.K[b][:T][mask, g, :].astype(F64)
                    vn = self.V[b][:T][mask, g, :].astype(F64)
                for i in range(r):
                    h = g * r + i
                    # (3) exact attention over the selected tokens
                    o_sp = softmax_attention(q[b, h], ku, vu)
                    # (4) residual linear attention, subtraction form
                    f = phi(q[b, h])
                    o_bar = f @ self.S[b, g]
                    o_til, w_sum = linear_attention_numerator(f, ku, vu)
                    if covers_all:
                        o_rla = np.zeros(d, F64)
                        d_rla = 0.0
                    else:
                        o_rla = o_bar - o_til
                        d_rla = float(f @ self.z[b, g] - w_sum)
                    # (5) gated combine
                    out["o_sparse"][b, h] = o_sp
                    out["o_bar"][b, h] = o_bar
                    out["o_tilde"][b, h] = o_til
                    out["o_rla"][b, h] = o_rla
                    out["d_rla"][b, h] = d_rla
                    branch = rla_branch(o_rla, d_rla, rla_mode,
                                        None if gamma is None else gamma[h], eps, covers_all)
                    out["rla_out"][b, h] = branch
                    out["o"][b, h] = o_sp + gate[h] * branch
                    if brute_rla:
                        num, den = linear_attention_numerator(f, kn, vn)
                        out["o_rla_direct"][b, h] = num
                        out["d_rla_direct"][b, h] = den
        return out
