"""CPU oracle for contextual-token-sparsity token elimination.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(no headers, helpers, tables or constants) and imports nothing from it.

It is a plain, slow, obviously-correct restatement of what the pages define,
written with numpy.  Real-valued results are computed in float64.  Where a
floating-point value is quantised (a bf16 rounding point, a threshold compare)
the decision is taken in the precision the HIP kernels take it in (float32),
so that both sides round the same value.

Sources (the pages, cited by title and section):
  [Jenga]  "Jenga: Enhancing LLM Long-Context Fine-tuning with Contextual Token
           Sparsity", USENIX ATC'25 (structured summary page), section 4.2.
  [LeMo]   "LeMo: Enabling LEss Token Involvement for MOre Context
           Fine-tuning", arXiv 2501.09767 (review page: reading notes,
           figure captions).

Readings where the pages are silent or garbled (each is repeated at the
function that takes it):
  * scores are pre-softmax and scaled by 1/sqrt(head_dim) before clamping;
  * the i != j exclusion of Eq. 1 is carried into the block max of Eq. 2;
  * two head reductions are provided: the pages' order (mean over heads of
    positive scores, then block max) and the per-head block max, clamped, then
    summed over heads;
  * the column aggregate sums the block score over every query block;
  * causal variant: only pairs j < i take part; a ragged last block holds the
    N mod b remaining tokens; a block pair with no pair taking part scores 0;
    a batch is its sequences scored one by one;
  * a block's representative embedding is the mean of its rows;
  * the predictor is two matrices, ReLU(x U) V; x-bar and the hidden ReLU
    output are rounded to bf16, everything after stays real-valued; the block
    product is clamped at zero;
  * a block is kept when its score is >= the threshold; top-k ties go to the
    lower block index; NaN scores compare false and sort last;
  * the residual add is the correctly rounded bf16 sum, and the backward
    recompute of the input the correctly rounded bf16 difference;
  * the MLP block's token score sums over channels the largest magnitude of
    the intermediate activation over the block's tokens; the SiLU-gated
    activation is real-valued (not rounded) when formed from gate and up.

Parity pins: every function here is pinned in tests/ by hand-computed
examples (tests/golden), closed forms, invariants, brute force on tiny inputs
or library routines (torch's bf16 conversion, numpy sorting / indexing).
"""
from __future__ import annotations

import math

import numpy as np

REDUCE_PAPER = 0     # Eq. 2: block max of the head-mean of positive scores
REDUCE_HEADMAX = 1   # per-head block max, clamped at zero, summed over heads

SELECT_THRESHOLD = 0
SELECT_TOPK = 1
SELECT_MEAN = 2


# --------------------------------------------------------------------------
# bf16 values (stored as uint16 bit patterns)
# --------------------------------------------------------------------------
def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 values.  A bf16 pattern is the upper half
    of the binary32 pattern of the same value, so widening is exact."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return ((b.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round real values to the nearest bf16 value, ties to even, and return
    the bit patterns.

    Written from the format's definition, not from a bit trick: bf16 has an
    8-bit significand and binary32's exponent range, so the spacing of
    representable values in the binade [2^(e-1), 2^e) is 2^(e-8), never finer
    than the subnormal quantum 2^-133.  Values at or beyond the midpoint
    between the largest finite value (2 - 2^-7) * 2^127 and 2^128 overflow to
    infinity; NaN maps to the quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(ax)                      # ax = m * 2^e, 0.5 <= m < 1
        qexp = np.maximum(e - 8, -133)           # spacing exponent of ax's binade
        r = np.rint(np.ldexp(ax, -qexp))         # np.rint rounds half to even
        val = np.ldexp(r, qexp)
        val = np.where(np.isinf(ax) | (val >= 2.0 ** 128), np.inf, val)
        val = np.copysign(val, x)
    bits = (val.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits)


# --------------------------------------------------------------------------
# a1: exact block-wise informativeness
# --------------------------------------------------------------------------
def exact_block_scores(q, k, n_heads: int, head_dim: int, block: int,
                       head_reduce: int = REDUCE_PAPER,
                       query_blocks=None, key_blocks=None, causal: bool = False):
    """Score blocks B^S_nm of the attention scores and their column aggregate.

    [Jenga] 4.2.1, Eq. 1: the interaction of tokens i and j is S_ij = Q_i K_j;
    Eq. 2: the block score keeps only positive values, averages over the heads
    (1/N_head) and takes the maximum over the block; Figure 6 caption: the
    block matrix is aggregated along each column, I[m] = sum_n M[n][m];
    [LeMo] reading notes: the scores are the raw pre-softmax ones.

    Readings: S^h_ij = Q^h_i . K^h_j / sqrt(head_dim) (the scale of the
    attention formula; it does not change any ranking); pairs i == j are
    left out of the block max as in Eq. 1; the column aggregate runs over all
    query blocks (no causal mask).  With ``causal`` (a variant for decoder
    models, whose attention never pairs a query with a later key), only pairs
    j < i take part.  When N is not a multiple of the block size the last
    block holds the N mod b remaining tokens.  A block pair with no pair
    taking part scores 0.  ``head_reduce``:
      REDUCE_PAPER   M[n,m] = max_{i in n, j in m, i != j} (1/H) sum_h max(0, S^h_ij)
      REDUCE_HEADMAX M[n,m] = sum_h max(0, max_{i in n, j in m, i != j} S^h_ij)
    I[m] = sum_n M[n,m].

    q, k: bf16 bits [N][n_heads*head_dim], head h in columns h*head_dim...
    Returns (M float64 [len(query_blocks)][len(key_blocks)], I or None).
    I (float64 [nb]) is returned only when every query block is scored.
    """
    q = np.asarray(q)
    n_tok = q.shape[0]
    nb = -(-n_tok // block)
    Q = bf16_decode(q).reshape(n_tok, n_heads, head_dim)
    K = bf16_decode(k).reshape(n_tok, n_heads, head_dim)
    qb = list(range(nb)) if query_blocks is None else list(query_blocks)
    kb = list(range(nb)) if key_blocks is None else list(key_blocks)
    rows_of = [np.arange(m * block, min((m + 1) * block, n_tok)) for m in kb]
    j_abs = np.concatenate(rows_of)                               # key token index of each column
    seg_start = np.cumsum([0] + [len(r) for r in rows_of])[:-1]   # first column of each key block
    Kt = np.ascontiguousarray(K[j_abs].transpose(1, 2, 0))        # [H][hd][columns]
    scale = 1.0 / math.sqrt(head_dim)
    M = np.empty((len(qb), len(kb)), dtype=np.float64)
    for a, n in enumerate(qb):
        i_abs = np.arange(n * block, min((n + 1) * block, n_tok))
        Qn = np.ascontiguousarray(Q[i_abs].transpose(1, 0, 2))    # [H][rows][hd]
        S = np.matmul(Qn, Kt) * scale                             # S^h_ij
        # pairs that take no part: i == j, and every j > i in the causal variant
        out = (j_abs[None, :] >= i_abs[:, None]) if causal else (j_abs[None, :] == i_abs[:, None])
        if head_reduce == REDUCE_PAPER:
            Sbar = np.maximum(S, 0.0).sum(axis=0) / n_heads      # [rows][columns]
            Sbar[out] = -np.inf
            best = np.maximum.reduceat(Sbar.max(axis=0), seg_start)
            M[a] = np.maximum(best, 0.0)
        elif head_reduce == REDUCE_HEADMAX:
            S[:, out] = -np.inf
            per_head = np.maximum.reduceat(S.max(axis=1), seg_start, axis=1)   # [H][len(kb)]
            M[a] = np.maximum(per_head, 0.0).sum(axis=0)
        else:
            raise ValueError("unknown head reduction")
    I = M.sum(axis=0) if query_blocks is None else None
    return M, I


def exact_block_scores_batched(q, k, n_heads: int, head_dim: int, block: int,
                               head_reduce: int = REDUCE_PAPER, causal: bool = False):
    """A batch of independent sequences, q and k bf16 bits [B][N][n_heads*head_dim]:
    the scores of each sequence on its own (no pair crosses sequences).
    Returns M float64 [B][nb][nb] and I float64 [B][nb]."""
    res = [exact_block_scores(q[b], k[b], n_heads, head_dim, block, head_reduce, causal=causal)
           for b in range(len(q))]
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])


def exact_column_score(q, k, n_heads, head_dim, block, head_reduce, key_block, causal: bool = False):
    """I[m] of one key block, for sampled checks at sizes where the whole
    block matrix is too slow on the host ([Jenga] 4.2.1, Eq. 2 / Fig. 6)."""
    M, _ = exact_block_scores(q, k, n_heads, head_dim, block, head_reduce,
                              key_blocks=[key_block], query_blocks=None, causal=causal)
    return float(M[:, 0].sum()), M[:, 0]


# --------------------------------------------------------------------------
# a2-a4: predictor scores
# --------------------------------------------------------------------------
def pool_blocks(x, block: int) -> np.ndarray:
    """Representative embedding of each token block ([Jenga] 4.2.2: "extracting
    a representative embedding from each block"; the pages do not define it).

    Reading: the mean of the block's rows.  The sum is taken in float32, row by
    row in token order, divided by the number of rows in float32 (for a whole
    block of a power-of-two size that is the exact multiplication by 1/block),
    then rounded to bf16, because the result feeds a bf16 product.  When N is
    not a multiple of the block size the last block holds the N mod b
    remaining rows and is averaged over those.  Returns bf16 bits [nb][d]."""
    if block & (block - 1):
        raise ValueError("block must be a power of two")
    X = bf16_decode(x).astype(np.float32)
    n_tok, d = X.shape
    nb = -(-n_tok // block)
    mean = np.empty((nb, d), dtype=np.float32)
    for m in range(nb):
        rows = X[m * block:min((m + 1) * block, n_tok)]
        acc = np.zeros(d, dtype=np.float32)
        for row in rows:
            acc = acc + row                      # float32 add, rows in order
        mean[m] = acc / np.float32(len(rows))
    return bf16_round(mean.astype(np.float64))


def predictor_embeddings(xbar, u, v) -> np.ndarray:
    """One predictor of [Jenga] 4.2.2 / Figure 8 (low-rank matrices with a ReLU
    between them), read as two matrices: est = ReLU(xbar U) V.

    The hidden activation feeds a bf16 product, so it is rounded to bf16 from
    its float32 value (the precision the kernels accumulate in); the output is
    real-valued.  Returns float64 [nb][r]."""
    hid = np.maximum(bf16_decode(xbar) @ bf16_decode(u), 0.0)
    hid_bf16 = bf16_round(hid.astype(np.float32).astype(np.float64))
    return bf16_decode(hid_bf16) @ bf16_decode(v)


def predict_scores(x, u_q, v_q, u_k, v_k, block: int):
    """Predicted block scores ([Jenga] 4.2.2, Eq. 3): the score of block pair
    (m, n) is the product of the query predictor's output for block m and the
    key predictor's output for block n.  Reading: the product is clamped at
    zero, as positive scores are what Eq. 2 keeps, and aggregated along the
    column as in Figure 6.  Returns (M_hat [nb][nb], I_hat [nb], q_hat, k_hat),
    all float64."""
    xbar = pool_blocks(x, block)
    q_hat = predictor_embeddings(xbar, u_q, v_q)
    k_hat = predictor_embeddings(xbar, u_k, v_k)
    M = np.maximum(q_hat @ k_hat.T, 0.0)
    return M, M.sum(axis=0), q_hat, k_hat


def token_embeddings(x, u, v) -> np.ndarray:
    """Per-token predictor output ([Jenga] 4.2.2, Figure 8 and the complexity
    analysis: the query and key predictors cost O(s h^2), one pass per token of
    the sequence).  Reading: the predictor of `predictor_embeddings` applied to
    every token row instead of a block representative, ReLU(x U) V, and the
    result rounded to bf16 (to nearest even, from its float32 value) because it
    feeds the bf16 score product of Eq. 1 - 2 with one head of width r.
    Returns bf16 bits [N][r]."""
    est = predictor_embeddings(x, u, v)
    return bf16_round(est.astype(np.float32).astype(np.float64))


# --------------------------------------------------------------------------
# a5: layer threshold -> keep mask -> ascending kept-block list
# --------------------------------------------------------------------------
def select_mask(scores, mode: int, threshold: float = 0.0, keep_blocks: int = 0):
    """Compare token-block scores against a layer threshold ([Jenga] 4.2.1,
    "Layer-specific Threshold" and Algorithm 1, step 1).

    Comparisons are made on the float32 scores the kernels produce.
      SELECT_THRESHOLD: keep iff score >= threshold (float32).
      SELECT_MEAN:      threshold = the average block score (Algorithm 1's
                        initial threshold): float64 sum in block order, divided
                        by nb, rounded to float32; keep iff score >= it.
      SELECT_TOPK:      keep the keep_blocks best blocks, ordered by score
                        (descending, NaN last), ties to the lower index; the
                        threshold reported is the last kept score (+inf when
                        none is kept).
    Returns (mask uint8 [nb], kept int32 ascending [n_kept], n_kept, theta f32).
    """
    s = np.asarray(scores, dtype=np.float32)
    nb = s.shape[0]
    if mode == SELECT_THRESHOLD:
        theta = np.float32(threshold)
        keep = s >= theta
    elif mode == SELECT_MEAN:
        total = 0.0
        for v in s:
            total += float(v)
        theta = np.float32(total / nb) if nb else np.float32(np.nan)
        keep = s >= theta
    elif mode == SELECT_TOPK:
        if not 0 <= keep_blocks <= nb:
            raise ValueError("keep_blocks out of range")
        order = sorted(range(nb), key=lambda c: (bool(np.isnan(s[c])),
                                                 -float(s[c]) if not np.isnan(s[c]) else 0.0, c))
        keep = np.zeros(nb, dtype=bool)
        keep[order[:keep_blocks]] = True
        theta = s[order[keep_blocks - 1]] if keep_blocks else np.float32(np.inf)
    else:
        raise ValueError("unknown select mode")
    kept = np.nonzero(keep)[0].astype(np.int32)
    return keep.astype(np.uint8), kept, int(kept.size), np.float32(theta)


# --------------------------------------------------------------------------
# a6 / a7: permutation-free movement
# --------------------------------------------------------------------------
def kept_token_rows(kept, n_kept: int, block: int, n_tokens: int = None) -> np.ndarray:
    """Original row of every kept token, in kept-block order: packed row
    p = j * block + i is token kept[j] * block + i.  With n_tokens given and
    not a multiple of the block size, the last block has only the remaining
    rows: the packed rows end after the last kept block's rows (an ascending
    kept list, as select_mask gives, holds that short block last), and a
    position whose token lies past the sequence (the short block listed
    before the end) is -1: no row is read or written for it."""
    kept = np.asarray(kept[:n_kept], dtype=np.int64)
    rows = (kept[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    if n_tokens is None or n_kept == 0:
        return rows
    R = (n_kept - 1) * block + min(block, n_tokens - int(kept[-1]) * block)
    rows = rows[:R].copy()
    rows[rows >= n_tokens] = -1
    return rows


def gather_pad(src, block: int, kept, n_kept: int, dst_init, pad_multiple: int):
    """Selective load ([Jenga] 4.2.3, "Permutation-free Token Movement"): the
    kept tokens are read from their original rows.  Here they are copied, in
    kept-block order, into a dense buffer; rows from the last kept row up to
    the next multiple of pad_multiple are zero; rows past that keep their old
    contents.  Copies beyond the buffer's capacity are dropped and reported.
    Returns (dst bits, overflowed)."""
    dst = np.array(dst_init, dtype=np.uint16, copy=True)
    cap = dst.shape[0]
    rows = kept_token_rows(kept, n_kept, block, np.asarray(src).shape[0])
    n_rows = rows.size
    n_pad = -(-n_rows // pad_multiple) * pad_multiple
    width = min(dst.shape[1], np.asarray(src).shape[1])
    for p in range(min(n_rows, cap)):
        if rows[p] >= 0:
            dst[p, :width] = src[rows[p], :width]
    for p in range(n_rows, min(n_pad, cap)):
        dst[p, :width] = 0
    return dst, n_pad > cap


def linear_bf16(a, weight) -> np.ndarray:
    """A layer's linear map on bf16 rows: a weightᵀ with weight stored
    [out][in] (the usual Linear layout), the real product rounded to bf16
    from its float32 value.  Returns bf16 bits [rows][out]."""
    prod = bf16_decode(a) @ bf16_decode(weight).T
    return bf16_round(prod.astype(np.float32).astype(np.float64))


def gather_linear(x, block: int, kept, n_kept: int, weight, dst_init, pad_multiple: int):
    """Selective load fused into the layer's first product ([Jenga] 4.2.3:
    the kept tokens are read from their original rows inside the computation,
    Figure 18).  Reading: the same rows, order and zero padding as
    `gather_pad`, each row multiplied by weightᵀ and rounded to bf16; rows of
    dst past the padding keep their contents, rows past its capacity are
    dropped and reported.  Returns (dst bits, overflowed)."""
    dst = np.array(dst_init, dtype=np.uint16, copy=True)
    cap = dst.shape[0]
    rows = kept_token_rows(kept, n_kept, block, np.asarray(x).shape[0])
    n_rows = rows.size
    n_pad = -(-n_rows // pad_multiple) * pad_multiple
    take = min(n_rows, cap)
    width = np.asarray(weight).shape[0]
    live = np.nonzero(rows[:take] >= 0)[0]
    if live.size:
        dst[live, :width] = linear_bf16(np.asarray(x)[rows[live]], weight)
    for p in range(n_rows, min(n_pad, cap)):
        dst[p, :width] = 0
    return dst, n_pad > cap


def linear_scatter(a, weight, residual, block: int, kept, n_kept: int):
    """In-place addition fused into the layer's last product ([Jenga] 4.2.3,
    Figure 18).  Reading: row p of a (the dense kept rows) times weightᵀ,
    rounded to bf16, then added to the original row of kept token p exactly as
    `scatter_residual` adds it.  Returns new residual bits."""
    rows = kept_token_rows(kept, n_kept, block, np.asarray(residual).shape[0])
    y = linear_bf16(np.asarray(a)[:rows.size], weight) if rows.size else np.zeros((0, 0), np.uint16)
    return scatter_residual(residual, block, kept, n_kept, y)


def scatter_residual(residual, block: int, kept, n_kept: int, y):
    """In-place addition ([Jenga] 4.2.3): the layer output of each kept token
    (row p of y, in kept-block order) is added to that token's original row of
    the residual; eliminated tokens are left untouched.  Reading: the sum is
    the correctly rounded bf16 sum of the two bf16 values (the exact sum is
    formed in float64, where two bf16 values add exactly unless one is
    negligible, then rounded once).  Returns new residual bits."""
    out = np.array(residual, dtype=np.uint16, copy=True)
    rows = kept_token_rows(kept, n_kept, block, out.shape[0])
    width = out.shape[1]
    y = np.asarray(y)
    for p, t in enumerate(rows):
        if t >= 0:
            out[t] = bf16_round(bf16_decode(out[t]) + bf16_decode(y[p, :width]))
    return out


def residual_recompute(residual_out, block: int, kept, n_kept: int, y):
    """Backward recompute of a layer's input ([Jenga] 4.2.3, in-place
    addition: during backpropagation the original input is recovered by
    subtracting the block's output from the output embeddings).  For each kept
    token the layer output (row p of y, in kept-block order) is subtracted from
    that token's row; eliminated rows were never changed by the addition and
    stay as they are.  Reading: the correctly rounded bf16 difference (formed
    in float64, then rounded once).  When the forward addition rounded, this
    is not the input bit for bit: per element it is off by at most half a bf16
    spacing at the output value plus half a spacing at the result.
    Returns new residual bits."""
    out = np.array(residual_out, dtype=np.uint16, copy=True)
    rows = kept_token_rows(kept, n_kept, block, out.shape[0])
    width = out.shape[1]
    y = np.asarray(y)
    for p, t in enumerate(rows):
        if t >= 0:
            out[t] = bf16_round(bf16_decode(out[t]) - bf16_decode(y[p, :width]))
    return out


# --------------------------------------------------------------------------
def _block_channel_max_sum(mag, block: int) -> np.ndarray:
    """I[m] = sum over channels c of max over the tokens i of block m of
    mag[i, c]; the last block holds the N mod b remaining tokens."""
    n = mag.shape[0]
    nb = -(-n // block)
    return np.array([mag[m * block:min((m + 1) * block, n)].max(axis=0).sum() for m in range(nb)])


def mlp_block_scores(act, block: int) -> np.ndarray:
    """Token-block informativeness from the MLP block's intermediate
    activations ([Jenga] 4.2.1, "Extend to MLP Block": the output of the ReLU
    layer, or for SiLU-gated MLPs the element-wise product of the gate
    projection after SiLU and the up projection).

    The pages state no aggregation.  Reading, mirroring Eq. 2 (keep the
    magnitude that matters, take the maximum over the block's tokens) and the
    Figure 6 caption (aggregate along the other axis):
        I[m] = sum over channels c of max over tokens i in block m of |A[i, c]|.
    A ReLU output is >= 0, so its magnitude is the value itself.

    act: bf16 bits [N][w] (the activation tensor as the layer holds it).
    Returns I float64 [ceil(N / b)]."""
    return _block_channel_max_sum(np.abs(bf16_decode(act)), block)


def silu_gated(gate, up) -> np.ndarray:
    """SiLU(g) * u = g * u / (1 + e^-g) of bf16 gate and up projections,
    real-valued (float64, not rounded)."""
    g = bf16_decode(gate)
    u = bf16_decode(up)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def mlp_block_scores_gated(gate, up, block: int) -> np.ndarray:
    """mlp_block_scores of the SiLU-gated activation, formed from the gate
    and up projections (bf16 bits [N][w] each) without rounding it to bf16
    first (the activation is never stored)."""
    return _block_channel_max_sum(np.abs(silu_gated(gate, up)), block)
