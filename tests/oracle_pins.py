"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``check_*`` takes the oracle module (or a stand-in with the same
functions) and returns a list of failure strings.  The normal tests call them
on the real oracle and expect no failure; the mutation tests call them on
copies with a planted mistake and expect at least one failure, which shows
that the pin would catch that mistake.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def f2bits(vals) -> np.ndarray:
    """Exact float -> bf16 bits for values that are bf16-representable (asserted)."""
    a = np.asarray(vals, dtype=np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, a), "value not exact in bf16"
    return bits


def torch_bf16_bits(vals_f32) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(vals_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _fail(out, cond, msg):
    if not cond:
        out.append(msg)


# --------------------------------------------------------------------------
def check_bf16_round(o) -> list:
    """bf16_round against torch's float32 -> bfloat16 conversion (RNE), on
    structured edge cases and a large random sample of float32 patterns."""
    out = []
    rng = np.random.default_rng(7)
    pats = [rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)]
    # every exponent, with mantissa tails just below / at / above the tie
    exps = np.arange(256, dtype=np.uint32) << 23
    mants = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x10000, 0x18000, 0x7F7FFF,
                      0x7F8000, 0x7FFFFF, 0x7E8000, 0x3F8000], dtype=np.uint32)
    grid = (exps[:, None] | mants[None, :]).reshape(-1)
    pats += [grid, grid | np.uint32(0x80000000)]
    p = np.concatenate(pats)
    f = p.view(np.float32)
    finite = np.isfinite(f)
    got = o.bf16_round(f[finite].astype(np.float64))
    ref = torch_bf16_bits(f[finite])
    bad = np.nonzero(got != ref)[0]
    _fail(out, bad.size == 0, f"bf16_round differs from torch on {bad.size} finite patterns "
          f"(first {[hex(int(x)) for x in p[finite][bad[:4]]]})")
    # infinities and NaN
    spec = o.bf16_round(np.array([np.inf, -np.inf, np.nan, 0.0, -0.0]))
    _fail(out, [int(x) for x in spec[[0, 1, 3, 4]]] == [0x7F80, 0xFF80, 0x0000, 0x8000],
          f"bf16_round special values wrong: {[hex(int(x)) for x in spec]}")
    _fail(out, (int(spec[2]) & 0x7F80) == 0x7F80 and (int(spec[2]) & 0x7F) != 0, "NaN not kept NaN")
    # decode is exact: bf16 value -> float64 -> same pattern
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    dec = o.bf16_decode(allb)
    fin = np.isfinite(dec)
    _fail(out, np.array_equal(o.bf16_round(dec[fin]), allb[fin]), "decode/round do not round-trip")
    ref_dec = torch.from_numpy(allb.view(np.int16)).view(torch.bfloat16).double().numpy()
    _fail(out, np.array_equal(dec[fin], ref_dec[fin]), "bf16_decode differs from torch")
    return out


def check_bf16_add(o) -> list:
    """Scatter arithmetic: the oracle's correctly rounded bf16 sum against the
    float32-add-then-RNE route done by torch, on a random sample of bf16 pairs
    (including large exponent gaps) plus the hand-computed cases of E4."""
    out = []
    rng = np.random.default_rng(11)
    a = rng.integers(0, 1 << 16, size=1 << 21, dtype=np.uint32).astype(np.uint16)
    b = rng.integers(0, 1 << 16, size=1 << 21, dtype=np.uint32).astype(np.uint16)
    # near-equal magnitudes (cancellation and ties) as well
    b2 = (a.astype(np.int32) + rng.integers(-300, 300, size=a.size)).clip(0, 0xFFFF).astype(np.uint16)
    b2 ^= np.uint16(0x8000) * (rng.random(a.size) < 0.5).astype(np.uint16)
    A = np.concatenate([a, a])
    B = np.concatenate([b, b2])
    da, db = o.bf16_decode(A), o.bf16_decode(B)
    ok = np.isfinite(da) & np.isfinite(db)
    got = o.bf16_round(da[ok] + db[ok])
    ta = torch.from_numpy(A[ok].view(np.int16)).view(torch.bfloat16).float()
    tb = torch.from_numpy(B[ok].view(np.int16)).view(torch.bfloat16).float()
    ref = (ta + tb).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan_ref = np.isnan((ta + tb).numpy())
    bad = np.nonzero((got != ref) & ~nan_ref)[0]
    _fail(out, bad.size == 0, f"bf16 add differs from float32 route on {bad.size} pairs")
    for case in golden()["E4_movement"]["adds"]:
        s = o.bf16_round(o.bf16_decode(np.array([int(case["a"], 16)], np.uint16))
                         + o.bf16_decode(np.array([int(case["b"], 16)], np.uint16)))
        _fail(out, int(s[0]) == int(case["sum"], 16), f"E4 add {case['a']}+{case['b']} -> {hex(int(s[0]))}")
    return out


# --------------------------------------------------------------------------
def _heads_to_bits(heads):
    """[H][N] per-head values (head_dim 1) -> bf16 bits [N][H]."""
    return f2bits(np.asarray(heads, dtype=np.float32).T.copy())


def check_exact_hand(o) -> list:
    out = []
    g = golden()
    e1 = g["E1_diagonal_exclusion"]
    q = f2bits(np.array(e1["q"])[:, None])
    k = f2bits(np.array(e1["k"])[:, None])
    for mode, key in ((o.REDUCE_PAPER, "M_paper"), (o.REDUCE_HEADMAX, "M_headmax")):
        M, I = o.exact_block_scores(q, k, 1, 1, 2, mode)
        _fail(out, np.array_equal(M, np.array(e1[key])), f"E1 M mode {mode}: {M.tolist()}")
        _fail(out, np.array_equal(I, np.array(e1["I"])), f"E1 I mode {mode}: {I.tolist()}")
    mask, kept, nk, th = o.select_mask(np.array(e1["I"], np.float32), o.SELECT_MEAN)
    _fail(out, mask.tolist() == e1["mean_mask"] and float(th) == e1["mean_threshold"],
          f"E1 mean select: {mask.tolist()} {th}")
    e2 = g["E2_head_reduction_order"]
    q = _heads_to_bits(e2["q_heads"])
    k = _heads_to_bits(e2["k_heads"])
    M, I = o.exact_block_scores(q, k, 2, 1, 2, o.REDUCE_PAPER)
    _fail(out, np.array_equal(M, np.array(e2["M_paper"])) and np.array_equal(I, np.array(e2["I_paper"])),
          f"E2 paper: {M.tolist()} {I.tolist()}")
    M, I = o.exact_block_scores(q, k, 2, 1, 2, o.REDUCE_HEADMAX)
    _fail(out, np.array_equal(M, np.array(e2["M_headmax"])) and np.array_equal(I, np.array(e2["I_headmax"])),
          f"E2 headmax: {M.tolist()} {I.tolist()}")
    # causal variant on the same tokens
    e7 = g["E7_causal"]
    one = e7["one_head"]
    q = f2bits(np.array(one["q"])[:, None])
    k = f2bits(np.array(one["k"])[:, None])
    for mode in (o.REDUCE_PAPER, o.REDUCE_HEADMAX):
        M, I = o.exact_block_scores(q, k, 1, 1, 2, mode, causal=True)
        _fail(out, np.array_equal(M, np.array(one["M"])) and np.array_equal(I, np.array(one["I"])),
              f"E7 one head mode {mode}: {M.tolist()} {I.tolist()}")
    mask, kept, nk, th = o.select_mask(np.array(one["I"], np.float32), o.SELECT_MEAN)
    _fail(out, mask.tolist() == one["mean_mask"] and float(th) == one["mean_threshold"],
          f"E7 mean select: {mask.tolist()} {th}")
    two = e7["two_heads"]
    q = _heads_to_bits(two["q_heads"])
    k = _heads_to_bits(two["k_heads"])
    for mode, mk, ik in ((o.REDUCE_PAPER, "M_paper", "I_paper"), (o.REDUCE_HEADMAX, "M_headmax", "I_headmax")):
        M, I = o.exact_block_scores(q, k, 2, 1, 2, mode, causal=True)
        _fail(out, np.array_equal(M, np.array(two[mk])) and np.array_equal(I, np.array(two[ik])),
              f"E7 two heads mode {mode}: {M.tolist()} {I.tolist()}")
    # a ragged last block
    e8 = g["E8_tail_block"]
    q = f2bits(np.array(e8["q"])[:, None])
    k = f2bits(np.array(e8["k"])[:, None])
    for causal, mk, ik in ((False, "M", "I"), (True, "M_causal", "I_causal")):
        for mode in (o.REDUCE_PAPER, o.REDUCE_HEADMAX):
            M, I = o.exact_block_scores(q, k, 1, 1, 2, mode, causal=causal)
            _fail(out, np.array_equal(M, np.array(e8[mk])) and np.array_equal(I, np.array(e8[ik])),
                  f"E8 causal={causal} mode {mode}: {M.tolist()} {I.tolist()}")
    return out


def brute_exact(qf, kf, H, hd, b, mode, causal=False):
    """Pure-Python scalar enumeration of Eq. 1/2 (tiny inputs only).  Blocks
    are consecutive runs of b tokens, the last one possibly shorter; a pair
    (i, j) takes part unless i == j, or j > i in the causal variant; a block
    pair with no pair taking part scores 0."""
    N = len(qf)
    nb = (N + b - 1) // b
    c = 1.0 / math.sqrt(hd)

    def S(h, i, j):
        return sum(qf[i][h * hd + t] * kf[j][h * hd + t] for t in range(hd)) * c

    M = [[0.0] * nb for _ in range(nb)]
    for n in range(nb):
        for m in range(nb):
            pairs = [(i, j) for i in range(n * b, min(n * b + b, N)) for j in range(m * b, min(m * b + b, N))
                     if (j < i if causal else i != j)]
            if not pairs:
                continue
            if mode == 0:
                M[n][m] = max(0.0, max(sum(max(0.0, S(h, i, j)) for h in range(H)) / H for i, j in pairs))
            else:
                M[n][m] = sum(max(0.0, max(S(h, i, j) for i, j in pairs)) for h in range(H))
    I = [sum(M[n][m] for n in range(nb)) for m in range(nb)]
    return np.array(M), np.array(I)


def check_exact_bruteforce(o, seeds=range(6)) -> list:
    out = []
    for s in seeds:
        rng = np.random.default_rng(100 + s)
        H = int(rng.integers(1, 4))
        hd = int(rng.choice([1, 2, 4]))
        b = int(rng.choice([2, 4]))
        nb = int(rng.integers(1, 4))
        qf32 = rng.standard_normal((nb * b + b - 1, H * hd)).astype(np.float32)
        kf32 = rng.standard_normal((nb * b + b - 1, H * hd)).astype(np.float32)
        tail = int(rng.integers(1, b))
        for N, causal in ((nb * b, False), (nb * b, True), (nb * b - b + tail, False), (nb * b - b + tail, True)):
            q, k = torch_bf16_bits(qf32[:N]), torch_bf16_bits(kf32[:N])
            qf = o.bf16_decode(q).tolist()
            kf = o.bf16_decode(k).tolist()
            for mode in (0, 1):
                Mb, Ib = brute_exact(qf, kf, H, hd, b, mode, causal)
                M, I = o.exact_block_scores(q, k, H, hd, b, mode, causal=causal)
                _fail(out, M.shape == Mb.shape and np.allclose(M, Mb, rtol=1e-12, atol=1e-12)
                      and np.allclose(I, Ib, rtol=1e-12, atol=1e-12),
                      f"bruteforce seed {s} mode {mode} causal {causal} H{H} hd{hd} b{b} N{N}")
    return out


def check_exact_closed_form(o) -> list:
    """Rank-one scores: Q_i = a e, K_j = beta_j e along one coordinate of every
    head.  Then every block score of key block m equals
    a*max_{j in m} beta_j/sqrt(hd) (mode PAPER) or H times that (HEADMAX), for
    every query block, so I[m] = nb times it."""
    out = []
    rng = np.random.default_rng(3)
    H, hd, b, nb = 3, 8, 4, 5
    N = nb * b
    a = 1.5
    beta = o.bf16_decode(torch_bf16_bits(np.abs(rng.standard_normal(N)).astype(np.float32)))
    qv = np.zeros((N, H * hd), np.float32)
    kv = np.zeros((N, H * hd), np.float32)
    for h in range(H):
        qv[:, h * hd + 3] = a
        kv[:, h * hd + 3] = beta
    q, k = f2bits(qv), f2bits(kv)
    bm = beta.reshape(nb, b).max(axis=1) * a / math.sqrt(hd)
    for mode, mult in ((o.REDUCE_PAPER, 1.0), (o.REDUCE_HEADMAX, float(H))):
        M, I = o.exact_block_scores(q, k, H, hd, b, mode)
        _fail(out, np.allclose(M, np.tile(bm * mult, (nb, 1)), rtol=1e-13, atol=0),
              f"closed form M mode {mode}")
        _fail(out, np.allclose(I, nb * bm * mult, rtol=1e-13, atol=0), f"closed form I mode {mode}")
    # constant heads of mixed sign: S^h_ij = s_h for every pair, so a head with
    # negative scores adds nothing; PAPER gives sum_h max(0, s_h) / H and
    # HEADMAX gives sum_h max(0, s_h), for every block
    s_h = np.array([1.0, -2.0, 0.5, -0.25])
    H2, hd2, b2, nb2 = 4, 4, 2, 3
    qv = np.zeros((nb2 * b2, H2 * hd2), np.float32)
    kv = np.zeros((nb2 * b2, H2 * hd2), np.float32)
    for h in range(H2):
        qv[:, h * hd2] = 2.0
        kv[:, h * hd2] = s_h[h]       # S = 2 * s_h / sqrt(4) = s_h
    pos = np.maximum(s_h, 0).sum()
    for mode, val in ((o.REDUCE_PAPER, pos / H2), (o.REDUCE_HEADMAX, pos)):
        M, I = o.exact_block_scores(f2bits(qv), f2bits(kv), H2, hd2, b2, mode)
        _fail(out, np.allclose(M, val, rtol=1e-14, atol=0) and np.allclose(I, nb2 * val, rtol=1e-14, atol=0),
              f"constant mixed-sign heads, mode {mode}: {M.tolist()}")
    return out


def check_exact_invariants(o) -> list:
    out = []
    rng = np.random.default_rng(5)
    H, hd, b, nb = 3, 16, 8, 6
    N = nb * b
    q = torch_bf16_bits(rng.standard_normal((N, H * hd)).astype(np.float32))
    k = torch_bf16_bits(rng.standard_normal((N, H * hd)).astype(np.float32))
    Mp, Ip = o.exact_block_scores(q, k, H, hd, b, o.REDUCE_PAPER)
    Mh, Ih = o.exact_block_scores(q, k, H, hd, b, o.REDUCE_HEADMAX)
    _fail(out, np.all(H * Mp <= Mh * (1 + 1e-12)), "H*M_paper <= M_headmax violated")
    _fail(out, np.all(Mp >= 0) and np.all(Mh >= 0), "negative block score")
    _fail(out, np.any(H * Mp < Mh * (1 - 1e-6)), "the two reductions never differ on random data")
    # Q -> 2Q is exact in bf16 and doubles every score
    q2 = torch_bf16_bits(2.0 * o.bf16_decode(q).astype(np.float32))
    for mode, M0, I0 in ((o.REDUCE_PAPER, Mp, Ip), (o.REDUCE_HEADMAX, Mh, Ih)):
        M2, I2 = o.exact_block_scores(q2, k, H, hd, b, mode)
        _fail(out, np.allclose(M2, 2 * M0, rtol=1e-13, atol=0) and np.allclose(I2, 2 * I0, rtol=1e-13, atol=0),
              f"scaling Q by 2 does not double scores (mode {mode})")
    # one head: both reductions agree
    M1p, _ = o.exact_block_scores(q[:, :hd], k[:, :hd], 1, hd, b, o.REDUCE_PAPER)
    M1h, _ = o.exact_block_scores(q[:, :hd], k[:, :hd], 1, hd, b, o.REDUCE_HEADMAX)
    _fail(out, np.allclose(M1p, M1h, rtol=1e-13, atol=0), "H=1 reductions differ")
    # permuting whole blocks of tokens permutes rows and columns of M
    perm = rng.permutation(nb)
    rows = (perm[:, None] * b + np.arange(b)[None, :]).reshape(-1)
    for mode, M0 in ((o.REDUCE_PAPER, Mp), (o.REDUCE_HEADMAX, Mh)):
        Mq, _ = o.exact_block_scores(q[rows], k[rows], H, hd, b, mode)
        _fail(out, np.allclose(Mq, M0[np.ix_(perm, perm)], rtol=1e-12, atol=0),
              f"block permutation not equivariant (mode {mode})")
    # zero queries: every score is zero
    Mz, Iz = o.exact_block_scores(np.zeros_like(q), k, H, hd, b, o.REDUCE_PAPER)
    _fail(out, not Mz.any() and not Iz.any(), "Q = 0 gives non-zero scores")
    # sub-matrix evaluation agrees with the full matrix
    Ms, _ = o.exact_block_scores(q, k, H, hd, b, o.REDUCE_PAPER, query_blocks=[4, 1], key_blocks=[2, 4, 0])
    _fail(out, np.array_equal(Ms, Mp[np.ix_([4, 1], [2, 4, 0])]), "sub-matrix evaluation differs")
    for mode, M0 in ((o.REDUCE_PAPER, Mp), (o.REDUCE_HEADMAX, Mh)):
        Mc, _ = o.exact_block_scores(q, k, H, hd, b, mode, causal=True)
        lower = np.tril(np.ones((nb, nb), dtype=bool), -1)
        # causal: nothing above the block diagonal; below it every pair has
        # j < i, so those blocks equal the full-attention ones
        _fail(out, not Mc[np.triu_indices(nb, 1)].any(), f"causal scores above the block diagonal (mode {mode})")
        _fail(out, np.array_equal(Mc[lower], M0[lower]), f"causal lower blocks differ from full attention (mode {mode})")
        _fail(out, np.all(Mc.diagonal() <= M0.diagonal()) and np.any(Mc.diagonal() < M0.diagonal()),
              f"causal diagonal blocks not a strict subset of pairs (mode {mode})")
        # causal: later tokens change nothing for earlier queries, whatever the
        # length of the prefix (a ragged last block included)
        for n_pre in (5 * b, 4 * b + 3, b + 1):
            Mpre, _ = o.exact_block_scores(q[:n_pre], k[:n_pre], H, hd, b, mode, causal=True)
            full_q = n_pre // b
            _fail(out, np.array_equal(Mpre[:full_q], Mc[:full_q, :Mpre.shape[1]]),
                  f"causal prefix of {n_pre} tokens changes earlier scores (mode {mode})")
        # full attention on a ragged sequence: pairs of whole blocks are those
        # of the sequence cut back to whole blocks
        Mr, Ir = o.exact_block_scores(q[:4 * b + 3], k[:4 * b + 3], H, hd, b, mode)
        Mw, _ = o.exact_block_scores(q[:4 * b], k[:4 * b], H, hd, b, mode)
        _fail(out, Mr.shape == (5, 5) and np.array_equal(Mr[:4, :4], Mw) and np.array_equal(Ir, Mr.sum(axis=0)),
              f"ragged tail changes whole-block scores (mode {mode})")
    # a batch is its sequences scored one by one
    qb = np.stack([q, k, q[::-1].copy()])
    kb = np.stack([k, q, k])
    for causal in (False, True):
        MB, IB = o.exact_block_scores_batched(qb, kb, H, hd, b, o.REDUCE_PAPER, causal=causal)
        for i in range(3):
            Mi, Ii = o.exact_block_scores(qb[i], kb[i], H, hd, b, o.REDUCE_PAPER, causal=causal)
            _fail(out, np.array_equal(MB[i], Mi) and np.array_equal(IB[i], Ii), f"batch item {i} causal={causal}")
    return out


# --------------------------------------------------------------------------
def check_predictor(o) -> list:
    out = []
    e3 = golden()["E3_predictor"]
    x = f2bits(e3["x"])
    args = [f2bits(e3[n]) for n in ("u_q", "v_q", "u_k", "v_k")]
    xbar = o.pool_blocks(x, 2)
    _fail(out, np.array_equal(o.bf16_decode(xbar), np.array(e3["xbar"])), "E3 xbar")
    M, I, qh, kh = o.predict_scores(x, *args, 2)
    _fail(out, np.array_equal(qh, np.array(e3["q_hat"])), f"E3 q_hat {qh.tolist()}")
    _fail(out, np.array_equal(kh, np.array(e3["k_hat"])), f"E3 k_hat {kh.tolist()}")
    _fail(out, np.array_equal(M, np.array(e3["M_hat"])), f"E3 M_hat {M.tolist()}")
    _fail(out, np.array_equal(I, np.array(e3["I_hat"])), f"E3 I_hat {I.tolist()}")
    # pooling is the block mean: small integers add exactly in float32, and
    # the mean of 8 integers is exact in bf16 when it is a multiple of 1/8 < 2^5
    rng = np.random.default_rng(9)
    b, nb, d = 8, 6, 40
    xi = rng.integers(-4, 5, size=(nb * b, d)).astype(np.float32)
    pooled = o.bf16_decode(o.pool_blocks(f2bits(xi), b))
    _fail(out, np.array_equal(pooled, xi.reshape(nb, b, d).mean(axis=1)), "pooling is not the block mean")
    # pooled value rounding: an inexact mean is the bf16 rounding of the fp32 mean
    xr = torch_bf16_bits(rng.standard_normal((nb * b, d)).astype(np.float32))
    fm = o.bf16_decode(xr).reshape(nb, b, d).astype(np.float32).sum(axis=1, dtype=np.float32)
    pooled = o.pool_blocks(xr, b)
    ref = torch_bf16_bits(fm / np.float32(b))
    _fail(out, np.mean(pooled == ref) > 0.999, "pooled bf16 values disagree with a rounded mean")
    # X -> 2X: every rounding point scales exactly, so M_hat and I_hat grow 4x
    r = 16
    w = [torch_bf16_bits(rng.standard_normal(s).astype(np.float32) / np.sqrt(s[0]))
         for s in ((d, r), (r, r), (d, r), (r, r))]
    M1, I1, _, _ = o.predict_scores(xr, *w, b)
    x2 = torch_bf16_bits(2.0 * o.bf16_decode(xr).astype(np.float32))
    M2, I2, _, _ = o.predict_scores(x2, *w, b)
    _fail(out, np.allclose(M2, 4 * M1, rtol=1e-12, atol=0) and np.allclose(I2, 4 * I1, rtol=1e-12, atol=0),
          "X -> 2X does not scale predicted scores by 4")
    _fail(out, np.all(M1 >= 0) and np.all(I1 >= 0), "negative predicted score")
    # a block's predicted column only depends on that block's rows: swapping two
    # blocks of X swaps the corresponding rows and columns of M_hat
    rows = np.arange(nb * b).reshape(nb, b)
    rows[[1, 4]] = rows[[4, 1]]
    Ms, _, _, _ = o.predict_scores(xr[rows.reshape(-1)], *w, b)
    p = np.arange(nb)
    p[[1, 4]] = p[[4, 1]]
    _fail(out, np.array_equal(Ms, M1[np.ix_(p, p)]), "block swap not equivariant")
    # brute force on a tiny case
    bq = _brute_predict(o.bf16_decode(xr[:16, :6]), [o.bf16_decode(a) for a in
                         (w[0][:6, :4], w[1][:4, :4], w[2][:6, :4], w[3][:4, :4])], 4, o)
    Mt, It, _, _ = o.predict_scores(xr[:16, :6], w[0][:6, :4], w[1][:4, :4], w[2][:6, :4], w[3][:4, :4], 4)
    _fail(out, np.allclose(Mt, bq[0], rtol=1e-12, atol=1e-12) and np.allclose(It, bq[1], rtol=1e-12, atol=1e-12),
          "predictor brute force")
    return out


def _brute_predict(X, W, b, o):
    """Scalar loops of Eq. 3 with mean pooling; bf16 rounding of the pooled
    mean and of the hidden ReLU output through torch's conversion."""
    Uq, Vq, Uk, Vk = W
    N, d = X.shape
    nb = N // b
    r = Uq.shape[1]

    def bf(v):
        return float(torch.tensor(float(v), dtype=torch.float32).to(torch.bfloat16).float())

    xbar = []
    for m in range(nb):
        row = []
        for c in range(d):
            acc = np.float32(0)
            for i in range(b):
                acc = np.float32(acc + np.float32(X[m * b + i][c]))
            row.append(bf(np.float32(acc / np.float32(b))))
        xbar.append(row)

    def pred(U, V):
        res = []
        for m in range(nb):
            hid = [bf(np.float32(max(0.0, sum(xbar[m][c] * U[c][t] for c in range(d))))) for t in range(r)]
            res.append([sum(hid[t] * V[t][v] for t in range(r)) for v in range(r)])
        return res

    qh, kh = pred(Uq, Vq), pred(Uk, Vk)
    M = np.array([[max(0.0, sum(qh[m][v] * kh[n][v] for v in range(r))) for n in range(nb)] for m in range(nb)])
    return M, M.sum(axis=0)


def check_token_predictor(o) -> list:
    """Per-token predictor embeddings: the hand example, agreement with the
    block predictor on blocks of identical rows, exact doubling, and brute
    force."""
    out = []
    e5 = golden()["E5_token_predictor"]
    x = f2bits(e5["x"])
    uq, vq, uk, vk = (f2bits(e5[n]) for n in ("u_q", "v_q", "u_k", "v_k"))
    qt = o.token_embeddings(x, uq, vq)
    kt = o.token_embeddings(x, uk, vk)
    _fail(out, np.array_equal(o.bf16_decode(qt), np.array(e5["q_tok"])), f"E5 q_tok {o.bf16_decode(qt).tolist()}")
    _fail(out, np.array_equal(o.bf16_decode(kt), np.array(e5["k_tok"])), f"E5 k_tok {o.bf16_decode(kt).tolist()}")
    M, I = o.exact_block_scores(qt, kt, 1, 2, e5["block"], o.REDUCE_PAPER)
    s2 = math.sqrt(2.0)
    _fail(out, np.allclose(M * s2, np.array(e5["M_unscaled"]), rtol=1e-12, atol=1e-12), f"E5 M {M.tolist()}")
    _fail(out, np.allclose(I * s2, np.array(e5["I_unscaled"]), rtol=1e-12, atol=1e-12), f"E5 I {I.tolist()}")
    # a block whose rows are all equal has that row as its mean, so the token
    # embedding of each row is the block predictor's output, rounded to bf16
    rng = np.random.default_rng(11)
    d, r, b, nb = 48, 16, 4, 5
    base = torch_bf16_bits(rng.standard_normal((nb, d)).astype(np.float32))
    xb = np.repeat(base, b, axis=0)
    w = [torch_bf16_bits(rng.standard_normal(sh).astype(np.float32) / np.sqrt(sh[0])) for sh in ((d, r), (r, r))]
    _, _, qh, _ = o.predict_scores(xb, w[0], w[1], w[0], w[1], b)
    tok = o.token_embeddings(xb, w[0], w[1])
    ref = torch_bf16_bits(np.repeat(qh, b, axis=0).astype(np.float32))
    _fail(out, np.array_equal(tok, ref), "token embeddings disagree with the block predictor on constant blocks")
    # X -> 2X doubles every embedding exactly (all rounding points scale by 2)
    xr = torch_bf16_bits(rng.standard_normal((24, d)).astype(np.float32))
    x2 = torch_bf16_bits(2.0 * o.bf16_decode(xr).astype(np.float32))
    t1 = o.bf16_decode(o.token_embeddings(xr, w[0], w[1]))
    t2 = o.bf16_decode(o.token_embeddings(x2, w[0], w[1]))
    _fail(out, np.array_equal(t2, 2.0 * t1), "X -> 2X does not double the token embeddings")
    # brute force: scalar loops, bf16 rounding through torch's conversion
    X = o.bf16_decode(xr[:6, :8])
    U = o.bf16_decode(w[0][:8, :4])
    V = o.bf16_decode(w[1][:4, :4])

    def bf(v):
        return float(torch.tensor(float(v), dtype=torch.float32).to(torch.bfloat16).float())

    brute = np.array([[bf(np.float32(sum(bf(np.float32(max(0.0, sum(X[i][c] * U[c][t] for c in range(8)))))
                                         * V[t][v] for t in range(4)))) for v in range(4)] for i in range(6)])
    got = o.bf16_decode(o.token_embeddings(xr[:6, :8], w[0][:8, :4], w[1][:4, :4]))
    _fail(out, np.array_equal(got, brute), "token embeddings brute force")
    return out


def check_fused_movement(o) -> list:
    """Selective load fused into a product and in-place addition fused into a
    product: the hand example, the identity weight reducing them to the plain
    gather and scatter, and brute force of the product's rounding."""
    out = []
    e6 = golden()["E6_fused_movement"]
    x = f2bits(e6["x"])
    w = f2bits(e6["weight"])
    kept = np.array(e6["kept"], np.int32)
    b, pad, cap = e6["block"], e6["pad_multiple"], e6["cap_rows"]
    dst0 = np.full((cap, 2), 0x5A5A, np.uint16)
    dst, over = o.gather_linear(x, b, kept, kept.size, w, dst0, pad)
    rows = np.array(e6["gather_linear_rows"])
    _fail(out, not over and np.array_equal(o.bf16_decode(dst[:4]), rows), f"E6 gathered product {dst[:4].tolist()}")
    _fail(out, np.all(dst[4:8] == 0) and np.all(dst[8:] == 0x5A5A), "E6 padding / untouched rows")
    res = o.linear_scatter(f2bits(e6["a"]), w, x, b, kept, kept.size)
    _fail(out, np.array_equal(o.bf16_decode(res), np.array(e6["residual_after"])), f"E6 residual {o.bf16_decode(res).tolist()}")
    # the identity weight reduces both to the plain movement, bit for bit
    rng = np.random.default_rng(13)
    n, d, blk = 96, 24, 8
    xr = torch_bf16_bits(rng.standard_normal((n, d)).astype(np.float32))
    eye = f2bits(np.eye(d))
    kp = np.array([1, 4, 5, 9], np.int32)
    init = np.full((48, d), 0x1357, np.uint16)
    g1, o1 = o.gather_linear(xr, blk, kp, kp.size, eye, init, 16)
    g2, o2 = o.gather_pad(xr, blk, kp, kp.size, init, 16)
    _fail(out, np.array_equal(g1, g2) and o1 == o2, "identity weight: gather_linear != gather_pad")
    ar = torch_bf16_bits(rng.standard_normal((kp.size * blk, d)).astype(np.float32))
    s1 = o.linear_scatter(ar, eye, xr, blk, kp, kp.size)
    s2 = o.scatter_residual(xr, blk, kp, kp.size, ar)
    _fail(out, np.array_equal(s1, s2), "identity weight: linear_scatter != scatter_residual")
    # rows of dropped blocks are untouched
    dropped = np.setdiff1d(np.arange(n // blk), kp)
    drows = (dropped[:, None] * blk + np.arange(blk)[None, :]).reshape(-1)
    _fail(out, np.array_equal(s1[drows], xr[drows]), "linear_scatter touched a dropped row")
    # brute force of the product's rounding on a tiny case
    A = torch_bf16_bits(rng.standard_normal((5, 7)).astype(np.float32))
    W = torch_bf16_bits(rng.standard_normal((3, 7)).astype(np.float32))
    Ad, Wd = o.bf16_decode(A), o.bf16_decode(W)
    brute = np.array([[float(torch.tensor(float(np.float32(sum(Ad[i][k] * Wd[j][k] for k in range(7)))),
                                          dtype=torch.float32).to(torch.bfloat16).float()) for j in range(3)]
                      for i in range(5)])
    _fail(out, np.array_equal(o.bf16_decode(o.linear_bf16(A, W)), brute), "linear_bf16 brute force")
    return out


# --------------------------------------------------------------------------
def check_select(o) -> list:
    out = []
    rng = np.random.default_rng(13)
    s = rng.random(37).astype(np.float32)
    for kk in (0, 1, 5, 36, 37):
        mask, kept, nk, th = o.select_mask(s, o.SELECT_TOPK, keep_blocks=kk)
        ref = np.sort(np.argsort(-s, kind="stable")[:kk])
        _fail(out, np.array_equal(kept, ref) and nk == kk and int(mask.sum()) == kk, f"topk {kk}")
        if kk:
            _fail(out, th == np.sort(s)[::-1][kk - 1], f"topk threshold {kk}")
    # ties go to the lower block index
    t = np.array([1, 3, 3, 2, 3, 0], np.float32)
    _, kept, _, th = o.select_mask(t, o.SELECT_TOPK, keep_blocks=2)
    _fail(out, kept.tolist() == [1, 2] and th == 3, f"topk ties: {kept.tolist()}")
    _, kept, _, _ = o.select_mask(t, o.SELECT_TOPK, keep_blocks=4)
    _fail(out, kept.tolist() == [1, 2, 3, 4], f"topk ties 4: {kept.tolist()}")
    # NaN sorts last and fails every threshold compare
    tn = np.array([np.nan, 1, 2, np.nan], np.float32)
    _, kept, _, _ = o.select_mask(tn, o.SELECT_TOPK, keep_blocks=3)
    _fail(out, kept.tolist() == [0, 1, 2], f"topk NaN: {kept.tolist()}")
    mask, _, _, _ = o.select_mask(tn, o.SELECT_THRESHOLD, threshold=0.5)
    _fail(out, mask.tolist() == [0, 1, 1, 0], "threshold NaN")
    # threshold: >= keeps ties; extremes keep all / nothing
    mask, kept, nk, th = o.select_mask(t, o.SELECT_THRESHOLD, threshold=2.0)
    _fail(out, mask.tolist() == [0, 1, 1, 1, 1, 0] and th == 2.0, "threshold >=")
    _fail(out, o.select_mask(s, o.SELECT_THRESHOLD, threshold=-1.0)[2] == s.size, "keep-all threshold")
    _fail(out, o.select_mask(s, o.SELECT_THRESHOLD, threshold=2.0)[2] == 0, "drop-all threshold")
    # mean: the threshold is the arithmetic mean (exact here: 1/8 multiples)
    m8 = (rng.integers(0, 64, size=40) / 8.0).astype(np.float32)
    mask, kept, nk, th = o.select_mask(m8, o.SELECT_MEAN)
    _fail(out, th == np.float32(np.mean(m8.astype(np.float64))), "mean threshold")
    _fail(out, np.array_equal(mask.astype(bool), m8 >= th), "mean mask")
    # mean: the float64 sum runs in block order (the reading both sides take).
    # 2^60 + 1 rounds to 2^60 in float64, so [2^60, 1, -2^60] averages to 0,
    # while [2^60, -2^60, 1] averages to 1/3; an exact or reordered sum would
    # give one value for both
    big = 2.0 ** 60
    th0 = o.select_mask(np.array([big, 1, -big], np.float32), o.SELECT_MEAN)[3]
    th1 = o.select_mask(np.array([big, -big, 1], np.float32), o.SELECT_MEAN)[3]
    _fail(out, th0 == 0.0 and th1 == np.float32(1.0 / 3.0), f"mean in block order: {th0} {th1}")
    # mean of scores that are not exact: the correctly rounded sum (math.fsum)
    # over nb, rounded to float32
    mask, kept, nk, th = o.select_mask(s, o.SELECT_MEAN)
    _fail(out, th == np.float32(math.fsum(float(v) for v in s) / s.size), "mean threshold (fsum)")
    _fail(out, np.array_equal(mask.astype(bool), s >= th), "mean mask (fsum)")
    # random: kept list ascending, counts add up, every kept >= every dropped (topk)
    mask, kept, nk, th = o.select_mask(s, o.SELECT_TOPK, keep_blocks=11)
    _fail(out, np.all(np.diff(kept) > 0) and nk + int((mask == 0).sum()) == s.size, "kept list shape")
    _fail(out, s[mask == 1].min() >= s[mask == 0].max(), "topk order")
    return out


def check_movement(o) -> list:
    out = []
    e4 = golden()["E4_movement"]
    N, b = e4["n_tokens"], e4["block"]
    mask = np.array(e4["mask"], np.uint8)
    kept = np.nonzero(mask)[0].astype(np.int32)
    _fail(out, kept.tolist() == e4["kept_blocks"], "E4 kept list")
    rng = np.random.default_rng(17)
    w = 8
    src = rng.integers(1, 0x7F00, size=(N, w)).astype(np.uint16)
    sentinel = np.full((10, w), 0xABCD, np.uint16)
    dst, over = o.gather_pad(src, b, kept, 2, sentinel, e4["pad_multiple"])
    _fail(out, np.array_equal(dst[:4], src[e4["gathered_rows"]]), "E4 gather rows")
    _fail(out, not dst[4:8].any(), "E4 pad rows not zero")
    _fail(out, np.all(dst[8:] == 0xABCD) and not over, "E4 rows past the pad touched")
    # gather = torch.index_select over the kept token rows
    N2, b2, w2 = 64, 4, 24
    src2 = rng.integers(0, 1 << 16, size=(N2, w2)).astype(np.uint16)
    m2 = (rng.random(N2 // b2) < 0.4).astype(np.uint8)
    k2 = np.nonzero(m2)[0].astype(np.int32)
    tok = torch.arange(N2).view(N2 // b2, b2)[torch.from_numpy(k2).long()].reshape(-1)
    ref = torch.index_select(torch.from_numpy(src2.view(np.int16)), 0, tok).numpy().view(np.uint16)
    dst2, _ = o.gather_pad(src2, b2, k2, k2.size, np.zeros((N2, w2), np.uint16), 1)
    _fail(out, np.array_equal(dst2[:tok.numel()], ref) and not dst2[tok.numel():].any(), "gather vs index_select")
    # capacity: copies past the buffer are dropped and reported
    small, over = o.gather_pad(src2, b2, k2, k2.size, np.zeros((3, w2), np.uint16), 1)
    _fail(out, over and np.array_equal(small, ref[:3]) if k2.size * b2 > 3 else True, "capacity overflow")
    # scatter: keep-all equals the dense bf16 add; drop-all leaves the residual;
    # only kept rows change; E4 tie rounding
    res = torch_bf16_bits(rng.standard_normal((N2, w2)).astype(np.float32))
    yf = torch_bf16_bits(rng.standard_normal((N2, w2)).astype(np.float32))
    allk = np.arange(N2 // b2, dtype=np.int32)
    dense = (torch.from_numpy(res.view(np.int16)).view(torch.bfloat16).float()
             + torch.from_numpy(yf.view(np.int16)).view(torch.bfloat16).float()).to(torch.bfloat16)
    got = o.scatter_residual(res, b2, allk, allk.size, yf)
    _fail(out, np.array_equal(got, dense.view(torch.int16).numpy().view(np.uint16)), "keep-all != dense add")
    _fail(out, np.array_equal(o.scatter_residual(res, b2, allk, 0, yf), res), "drop-all changed the residual")
    yk = yf[tok.numpy()]
    got = o.scatter_residual(res, b2, k2, k2.size, yk)
    dropped = np.ones(N2, bool)
    dropped[tok.numpy()] = False
    _fail(out, np.array_equal(got[dropped], res[dropped]), "dropped rows touched")
    refk = torch.from_numpy(res.view(np.int16)).view(torch.bfloat16).float()
    refk.index_add_(0, tok, torch.from_numpy(yk.view(np.int16)).view(torch.bfloat16).float())
    _fail(out, np.array_equal(got, refk.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)),
          "scatter vs index_add")
    r0 = np.full((N, 1), 0x3F80, np.uint16)
    y0 = np.array([[0x3B80], [0x3BC0], [0x3B80], [0x3BC0]], np.uint16)
    got = o.scatter_residual(r0, b, kept, 2, y0)
    _fail(out, got[:, 0].tolist() == [0x3F80, 0x3F81, 0x3F80, 0x3F80, 0x3F80, 0x3F81], f"E4 scatter {got[:, 0]}")
    rc = e4["recompute_by_subtraction"]
    back = o.bf16_round(o.bf16_decode(np.array([int(rc["stored"], 16)], np.uint16))
                        - o.bf16_decode(np.array([int(rc["minus"], 16)], np.uint16)))
    _fail(out, int(back[0]) == int(rc["gives"], 16), "E4 recompute example")
    return out


def check_mlp_scores(o) -> list:
    """MLP block scores: the hand example, a pure-Python brute force of the
    plain and the SiLU-gated form (math.exp), closed forms of the gate, and
    invariants (row order inside a block, channel order, sign, exact
    doubling, a ragged last block)."""
    out = []
    e9 = golden()["E9_mlp_scores"]
    a = f2bits(np.array(e9["act"]))
    I = o.mlp_block_scores(a, e9["block"])
    _fail(out, np.array_equal(I, np.array(e9["I"])), f"E9: {I.tolist()}")
    I3 = o.mlp_block_scores(a[:3], e9["block"])
    _fail(out, np.array_equal(I3, np.array(e9["I_first_three_rows"])), f"E9 ragged: {I3.tolist()}")
    rng = np.random.default_rng(31)
    for s in range(4):
        n, w, b = int(rng.integers(1, 12)), int(rng.integers(1, 6)), int(rng.choice([2, 4]))
        A = torch_bf16_bits(rng.standard_normal((n, w)).astype(np.float32))
        G = torch_bf16_bits(3 * rng.standard_normal((n, w)).astype(np.float32))
        Af, Gf = o.bf16_decode(A).tolist(), o.bf16_decode(G).tolist()
        nb = (n + b - 1) // b
        brute = [sum(max(abs(Af[i][c]) for i in range(m * b, min(m * b + b, n))) for c in range(w)) for m in range(nb)]
        _fail(out, np.allclose(o.mlp_block_scores(A, b), brute, rtol=1e-14, atol=0), f"mlp brute force case {s}")
        gated = [sum(max(abs(Gf[i][c] / (1.0 + math.exp(-Gf[i][c])) * Af[i][c]) for i in range(m * b, min(m * b + b, n)))
                     for c in range(w)) for m in range(nb)]
        _fail(out, np.allclose(o.mlp_block_scores_gated(G, A, b), gated, rtol=1e-13, atol=0),
              f"gated brute force case {s}")
    # invariants
    n, w, b = 24, 10, 4
    A = torch_bf16_bits(rng.standard_normal((n, w)).astype(np.float32))
    I0 = o.mlp_block_scores(A, b)
    perm_rows = np.concatenate([m * b + rng.permutation(b) for m in range(n // b)])
    _fail(out, np.array_equal(o.mlp_block_scores(A[perm_rows], b), I0), "row order inside a block matters")
    _fail(out, np.allclose(o.mlp_block_scores(A[:, rng.permutation(w)], b), I0, rtol=1e-14, atol=0),
          "channel order matters")
    _fail(out, np.array_equal(o.mlp_block_scores(A ^ np.uint16(0x8000), b), I0), "sign of the activation matters")
    A2 = torch_bf16_bits(2 * o.bf16_decode(A).astype(np.float32))
    _fail(out, np.allclose(o.mlp_block_scores(A2, b), 2 * I0, rtol=1e-14, atol=0), "doubling A does not double I")
    _fail(out, np.array_equal(o.mlp_block_scores(A[:22], b)[:5], I0[:5]), "a ragged tail changes whole blocks")
    # the gate: SiLU(0) = 0; SiLU(64) = 64 (1 + e^-64)^-1, within 2e-28 of 64; SiLU(-64) ~ -64 e^-64
    zero = np.zeros((n, w), np.uint16)
    _fail(out, not o.mlp_block_scores_gated(zero, A, b).any(), "SiLU(0) is not 0")
    g64 = np.full((n, w), f2bits(np.array([64.0]))[0], np.uint16)
    _fail(out, np.allclose(o.mlp_block_scores_gated(g64, A, b), 64 * I0, rtol=1e-15, atol=0), "SiLU(64) != 64")
    gm64 = g64 | np.uint16(0x8000)
    _fail(out, np.all(o.mlp_block_scores_gated(gm64, A, b) <= 64 * math.exp(-64) * I0 * (1 + 1e-12)),
          "SiLU(-64) is not ~0")
    return out


def check_recompute(o) -> list:
    """Backward recompute: the hand example (a forward tie that loses 2^-8),
    torch's bf16 subtraction on random and structured pairs, dropped rows
    untouched, y = 0 is the identity, exact forward additions come back
    exactly, and every recomputed element lies within half a spacing at the
    output plus half a spacing at the result of the original input."""
    out = []
    e = golden()["E10_recompute"]
    x = f2bits(np.array(e["residual_in"]))
    y = f2bits(np.array(e["y"]))
    kept = np.array(e["kept"], np.int32)
    fwd = o.scatter_residual(x, e["block"], kept, 1, y)
    _fail(out, np.array_equal(o.bf16_decode(fwd), np.array(e["residual_out"])), f"E10 forward {fwd}")
    rec = o.residual_recompute(fwd, e["block"], kept, 1, y)
    _fail(out, np.array_equal(o.bf16_decode(rec), np.array(e["recomputed"])), f"E10 recompute {o.bf16_decode(rec)}")
    rng = np.random.default_rng(8)
    N, w, b = 64, 48, 8
    x = torch_bf16_bits(rng.standard_normal((N, w)).astype(np.float32))
    y = torch_bf16_bits((rng.standard_normal((N, w)) * np.exp2(rng.integers(-12, 4, (N, w)))).astype(np.float32))
    kept = np.array([1, 4, 6, 7], np.int32)
    rows = (kept[:, None] * b + np.arange(b)[None, :]).reshape(-1)
    fwd = o.scatter_residual(x, b, kept, 4, y)
    rec = o.residual_recompute(fwd, b, kept, 4, y)
    # torch: bf16 - bf16 is the float32 difference rounded to nearest even
    tr = (torch.from_numpy(o.bf16_decode(fwd[rows]).astype(np.float32)).bfloat16()
          - torch.from_numpy(o.bf16_decode(y[:rows.size]).astype(np.float32)).bfloat16())
    _fail(out, np.array_equal(rec[rows], tr.view(torch.int16).numpy().view(np.uint16)), "differs from torch's bf16 subtraction")
    dropped = np.setdiff1d(np.arange(N), rows)
    _fail(out, np.array_equal(rec[dropped], x[dropped]), "dropped rows changed")
    _fail(out, np.array_equal(o.residual_recompute(x, b, kept, 4, np.zeros_like(y)), x), "y = 0 is not the identity")

    def spacing(v):
        _, ex = np.frexp(np.abs(v))
        return np.ldexp(1.0, np.maximum(ex - 8, -133))
    xv, fv, rv = o.bf16_decode(x[rows]), o.bf16_decode(fwd[rows]), o.bf16_decode(rec[rows])
    _fail(out, np.all(np.abs(rv - xv) <= 0.5 * spacing(fv) + 0.5 * spacing(rv)), "recompute outside its bound")
    _fail(out, np.any(rv != xv), "no rounding loss on random data (test too weak)")
    exact = o.bf16_decode(fwd[rows]) == xv + o.bf16_decode(y[:rows.size])
    _fail(out, np.array_equal(rv[exact], xv[exact]) and exact.any(), "exact additions do not come back exactly")
    return out


def check_ragged_tail(o) -> list:
    """A last block shorter than the others: hand example E11 (its mean,
    gather with padding, in-place addition, and the position map when the
    short block is listed before the end); a block of identical rows pools to
    that row whatever its length; whole blocks are unchanged by a ragged
    tail."""
    out = []
    e = golden()["E11_ragged_tail"]
    b = e["block"]
    x = f2bits(np.array(e["x"]))
    _fail(out, np.array_equal(o.bf16_decode(o.pool_blocks(x, b)), np.array(e["xbar"])), "E11 pooled means")
    kept = np.array(e["kept"], np.int32)
    dst, over = o.gather_pad(x, b, kept, 2, np.full((6, 2), 0x7777, np.uint16), e["gather_pad_multiple"])
    _fail(out, np.array_equal(o.bf16_decode(dst[:4]), np.array(e["gathered"])) and np.all(dst[4:] == 0x7777)
          and not over, f"E11 gather {dst.tolist()}")
    res = o.scatter_residual(x, b, kept, 2, f2bits(np.array(e["y"])))
    _fail(out, np.array_equal(o.bf16_decode(res), np.array(e["residual_after"])), f"E11 scatter {o.bf16_decode(res)}")
    back = o.residual_recompute(res, b, kept, 2, f2bits(np.array(e["y"])))
    _fail(out, np.array_equal(back, x), "E11 recompute of exact additions")
    rows = o.kept_token_rows(np.array(e["kept_misplaced"], np.int32), 2, b, 5)
    _fail(out, rows.tolist() == e["rows_misplaced"], f"E11 misplaced short block rows {rows.tolist()}")
    dstm, _ = o.gather_pad(x, b, np.array(e["kept_misplaced"], np.int32), 2, np.full((4, 2), 0x7777, np.uint16), 1)
    _fail(out, np.all(dstm[1] == 0x7777) and np.array_equal(dstm[0], x[4]) and np.array_equal(dstm[2:], x[:2]),
          "E11 misplaced short block: position 1 must be left untouched")
    # identical rows in every block, the short one included, pool to the row
    rng = np.random.default_rng(17)
    for n, blk in ((7, 4), (13, 8), (9, 2)):
        base = torch_bf16_bits(rng.standard_normal((-(-n // blk), 6)).astype(np.float32))
        xs = np.repeat(base, blk, axis=0)[:n]
        _fail(out, np.array_equal(o.pool_blocks(xs, blk), base), f"identical rows do not pool to the row (n={n} b={blk})")
    # whole blocks do not see the ragged tail
    xr = torch_bf16_bits(rng.standard_normal((21, 8)).astype(np.float32))
    _fail(out, np.array_equal(o.pool_blocks(xr, 4)[:5], o.pool_blocks(xr[:20], 4)), "ragged tail changes whole blocks")
    return out


def check_exact_column(o) -> list:
    """exact_column_score(m), the one-column form used by the sampled checks at
    full size, against the hand examples' column m (E1, E2, E7 and E8, both
    modes, with and without the causal mask) and against the pure-Python brute
    force on random tiny full, causal and ragged inputs: I[m] and the column
    M[:, m] must both match."""
    out = []
    g = golden()

    def cmp(q, k, H, hd, b, mode, causal, M_ref, I_ref, what):
        M_ref, I_ref = np.asarray(M_ref, np.float64), np.asarray(I_ref, np.float64)
        for m in range(I_ref.shape[0]):
            val, col = o.exact_column_score(q, k, H, hd, b, mode, m, causal=causal)
            _fail(out, np.shape(col) == (M_ref.shape[0],) and np.allclose(col, M_ref[:, m], rtol=1e-12, atol=1e-12)
                  and math.isclose(val, I_ref[m], rel_tol=1e-12, abs_tol=1e-12),
                  f"column {m} of {what} mode {mode} causal {causal}: {val} {np.asarray(col).tolist()}")

    e1 = g["E1_diagonal_exclusion"]
    q, k = f2bits(np.array(e1["q"])[:, None]), f2bits(np.array(e1["k"])[:, None])
    for mode, key in ((o.REDUCE_PAPER, "M_paper"), (o.REDUCE_HEADMAX, "M_headmax")):
        cmp(q, k, 1, 1, 2, mode, False, e1[key], e1["I"], "E1")
    e2 = g["E2_head_reduction_order"]
    q, k = _heads_to_bits(e2["q_heads"]), _heads_to_bits(e2["k_heads"])
    cmp(q, k, 2, 1, 2, o.REDUCE_PAPER, False, e2["M_paper"], e2["I_paper"], "E2")
    cmp(q, k, 2, 1, 2, o.REDUCE_HEADMAX, False, e2["M_headmax"], e2["I_headmax"], "E2")
    e7 = g["E7_causal"]
    one = e7["one_head"]
    q, k = f2bits(np.array(one["q"])[:, None]), f2bits(np.array(one["k"])[:, None])
    for mode in (o.REDUCE_PAPER, o.REDUCE_HEADMAX):
        cmp(q, k, 1, 1, 2, mode, True, one["M"], one["I"], "E7 one head")
    two = e7["two_heads"]
    q, k = _heads_to_bits(two["q_heads"]), _heads_to_bits(two["k_heads"])
    cmp(q, k, 2, 1, 2, o.REDUCE_PAPER, True, two["M_paper"], two["I_paper"], "E7 two heads")
    cmp(q, k, 2, 1, 2, o.REDUCE_HEADMAX, True, two["M_headmax"], two["I_headmax"], "E7 two heads")
    e8 = g["E8_tail_block"]
    q, k = f2bits(np.array(e8["q"])[:, None]), f2bits(np.array(e8["k"])[:, None])
    for causal, mk, ik in ((False, "M", "I"), (True, "M_causal", "I_causal")):
        for mode in (o.REDUCE_PAPER, o.REDUCE_HEADMAX):
            cmp(q, k, 1, 1, 2, mode, causal, e8[mk], e8[ik], "E8")
    for s in range(4):
        rng = np.random.default_rng(500 + s)
        H = int(rng.integers(1, 4))
        hd = int(rng.choice([1, 2, 4]))
        b = int(rng.choice([2, 4]))
        nb = int(rng.integers(2, 5))
        tail = int(rng.integers(1, b))
        for N, causal in ((nb * b, False), (nb * b, True), (nb * b - b + tail, False), (nb * b - b + tail, True)):
            qf32 = rng.standard_normal((N, H * hd)).astype(np.float32)
            kf32 = rng.standard_normal((N, H * hd)).astype(np.float32)
            q, k = torch_bf16_bits(qf32), torch_bf16_bits(kf32)
            for mode in (0, 1):
                Mb, Ib = brute_exact(o.bf16_decode(q).tolist(), o.bf16_decode(k).tolist(), H, hd, b, mode, causal)
                cmp(q, k, H, hd, b, mode, causal, Mb, Ib, f"random seed {s} H{H} hd{hd} b{b} N{N}")
    return out


ALL_CHECKS = [check_bf16_round, check_bf16_add, check_exact_hand, check_exact_bruteforce, check_exact_column,
              check_exact_closed_form, check_exact_invariants, check_predictor, check_token_predictor,
              check_select, check_movement, check_fused_movement, check_mlp_scores, check_recompute,
              check_ragged_tail]
