"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs (and never on inputs produced by the HIP path).

Bars: scores within relative 1e-2 (floor 1e-6 of the largest score); masks
equal except on blocks whose oracle score is within 1e-2 of the oracle
threshold; select, gather and scatter bit-exact given the same inputs.
"""
import math
import sys

import numpy as np
import pytest
import torch

from contextual_token_sparsity_amd import lemo
from contextual_token_sparsity_amd import synth
from oracle import lemo_oracle as O
from tests.gpu_helpers import dev, host_bits, mask_acceptable, padded, scores_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lemo.lib()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rand_qk(seed, n, h, hd, std=1.0):
    rng = np.random.default_rng(seed)
    return synth.random_bf16(rng, (n, h * hd), std), synth.random_bf16(rng, (n, h * hd), std)


# ----------------------------------------------------------- exact scores
EXACT_SMALL = [
    # (N, H, hd, block)
    (256, 2, 128, 64),
    (320, 3, 64, 64),     # N not a multiple of the 128-row tile: ragged last tile
    (224, 2, 128, 32),    # ragged, 32-row blocks (one block per MFMA tile)
    (384, 2, 64, 128),    # 128-row blocks span the four waves of a tile
    (96, 1, 64, 32),      # smaller than one tile
    (64, 1, 128, 64),     # a single block: only diagonal pairs to exclude
    (1024, 5, 128, 64),
    # head_dim 64 with several heads (PAPER runs its chain from the running
    # sum there, two heads per loop turn): 32-row blocks, and an odd head
    # count with 128-row blocks
    (256, 4, 64, 32),
    (384, 3, 64, 128),
]


@pytest.mark.parametrize("mode", [O.REDUCE_PAPER, O.REDUCE_HEADMAX], ids=["paper", "headmax"])
@pytest.mark.parametrize("shape", EXACT_SMALL, ids=lambda s: "N%d_H%d_hd%d_b%d" % s)
def test_exact_small(shape, mode):
    n, h, hd, b = shape
    say("exact", shape, mode)
    q, k = rand_qk(1000 + n + h, n, h, hd)
    M_ref, I_ref = O.exact_block_scores(q, k, h, hd, b, mode)
    nb = n // b
    M = torch.full((nb, nb), -1.0, device="cuda")
    I, _ = lemo.lemo_block_scores(dev(q), dev(k), h, hd, b, mode, block_scores=M)
    torch.cuda.synchronize()
    ok, worst = scores_close(I.cpu().numpy(), I_ref)
    assert ok, worst
    okm, worstm = scores_close(M.cpu().numpy(), M_ref)
    assert okm, worstm
    assert worst < 1e-4 and worstm < 1e-4, (worst, worstm)   # fp32 accumulation, not 1e-2


@pytest.mark.parametrize("block", [32, 64, 128])
def test_headmax_most_heads(block):
    """HEADMAX at its largest head count (128): with 128-row blocks every
    head's per-wave maxima are kept in LDS and summed in head order at the end
    of the tile; 32- and 64-row blocks sum in registers."""
    n, h, hd = 384, 128, 64
    say("headmax most heads", n, h, hd, block)
    q, k = rand_qk(5100 + block, n, h, hd)
    M_ref, I_ref = O.exact_block_scores(q, k, h, hd, block, O.REDUCE_HEADMAX)
    nb = n // block
    M = torch.full((nb, nb), -1.0, device="cuda")
    I, _ = lemo.lemo_block_scores(dev(q), dev(k), h, hd, block, O.REDUCE_HEADMAX, block_scores=M)
    torch.cuda.synchronize()
    okm, worstm = scores_close(M.cpu().numpy(), M_ref)
    ok, worst = scores_close(I.cpu().numpy(), I_ref)
    assert okm and ok and worstm < 1e-4 and worst < 1e-4, (worstm, worst)


@pytest.mark.parametrize("mode", [O.REDUCE_PAPER, O.REDUCE_HEADMAX], ids=["paper", "headmax"])
@pytest.mark.parametrize("wname", ["tiny", "opt1.3b-n4k"])
def test_exact_workload(wname, mode):
    w = synth.WORKLOADS[wname]
    say("exact workload", wname, mode)
    L = synth.make_workload(w, with_y=False)
    M_ref, I_ref = O.exact_block_scores(L.q, L.k, w.n_heads, w.head_dim, w.block, mode)
    I, _ = lemo.lemo_block_scores(dev(L.q), dev(L.k), w.n_heads, w.head_dim, w.block, mode)
    ok, worst = scores_close(I.cpu().numpy(), I_ref)
    assert ok and worst < 1e-4, worst


def _sampled_check(q, k, h, hd, b, mode, entries, columns, M_gpu, I_gpu):
    for (r, c) in entries:
        M_ref, _ = O.exact_block_scores(q, k, h, hd, b, mode, query_blocks=[r], key_blocks=[c])
        ok, worst = scores_close([M_gpu[r, c]], M_ref[0])
        assert ok and worst < 1e-4, (r, c, M_gpu[r, c], M_ref[0, 0])
    for c in columns:
        I_ref, col = O.exact_column_score(q, k, h, hd, b, mode, c)
        ok, worst = scores_close(M_gpu[:, c], col)
        assert ok, (c, worst)
        ok, worst = scores_close([I_gpu[c]], [I_ref])
        assert ok and worst < 1e-4, (c, I_gpu[c], I_ref)


@pytest.mark.parametrize("wname", ["llama2-7b-n8k-exact", "llama2-7b-n16k"])
def test_exact_full_size_sampled(wname):
    """Full-size exact scoring in the benchmark's launch configuration; the
    oracle recomputes sampled block scores and whole columns one by one."""
    w = synth.WORKLOADS[wname]
    say("exact full size", wname)
    L = synth.make_layer(w.n_tokens, w.d_model, w.block, w.seed, n_heads=w.n_heads, head_dim=w.head_dim,
                         planted_frac=w.planted_frac, with_y=False, proj_device="cuda")
    nb = w.n_blocks
    rng = np.random.default_rng(5)
    entries = [(0, 0), (nb - 1, nb - 1), (nb // 2, nb // 2)] + [tuple(rng.integers(0, nb, 2)) for _ in range(5)]
    columns = [int(L.planted_blocks[0]) if L.planted_blocks.size else 1, nb - 1]
    qd, kd = dev(L.q), dev(L.k)
    for mode in (O.REDUCE_PAPER, O.REDUCE_HEADMAX):
        M = torch.empty((nb, nb), device="cuda")
        I, _ = lemo.lemo_block_scores(qd, kd, w.n_heads, w.head_dim, w.block, mode, block_scores=M)
        _sampled_check(L.q, L.k, w.n_heads, w.head_dim, w.block, mode, entries, columns,
                       M.cpu().numpy(), I.cpu().numpy())


@pytest.mark.parametrize("mode", [O.REDUCE_PAPER, O.REDUCE_HEADMAX], ids=["paper", "headmax"])
def test_exact_closed_form_full_size(mode):
    """Q_i = a e and K_j = beta_j e in every head (e one coordinate): every
    block score of key block m is a max_{j in m} beta_j / sqrt(hd), times H
    for HEADMAX, so I[m] is nb times that -- at N = 16384, no oracle needed."""
    n, h, hd, b = 16384, 32, 128, 64
    nb = n // b
    rng = np.random.default_rng(21)
    a = 0.75
    beta = synth.to_bf16_bits(np.abs(rng.standard_normal(n)).astype(np.float32))
    bf = synth.bf16_bits_to_f32(beta).astype(np.float64)
    q = np.zeros((n, h * hd), np.uint16)
    k = np.zeros((n, h * hd), np.uint16)
    q[:, 3::hd] = synth.to_bf16_bits(np.full((1,), a, np.float32))[0]
    k[:, 3::hd] = beta[:, None]
    I, _ = lemo.lemo_block_scores(dev(q), dev(k), h, hd, b, mode)
    expect = nb * a * bf.reshape(nb, b).max(axis=1) / math.sqrt(hd) * (h if mode == O.REDUCE_HEADMAX else 1)
    ok, worst = scores_close(I.cpu().numpy(), expect, rel=1e-5)
    assert ok, worst


@pytest.mark.parametrize("h,n", [(2, 2896 * 128), (1, 1 << 22)], ids=["two_heads", "one_head"])
def test_exact_max_tokens_closed_form(h, n):
    """The largest accepted sequences against the rank-one closed form
    I[m] = nb a max_{j in m} beta_j / sqrt(hd): with two heads 370688 tokens
    (2896^2 tiles, just under the 2^23 workgroups of one launch), with one
    head 2^22 tokens (a 32768 x 32768 block matrix of 4 GiB, the one-head
    kernel's workgroups walking ranges of 2^30 tiles).  Rows of h x 64
    elements, blocks of 128; checks every column score and sampled block
    pairs, one of them past 2^31 entries of M when N = 2^22."""
    hd, b = 64, 128
    nb = n // b
    say("exact max tokens", h)
    rng = np.random.default_rng(23)
    a = 0.5
    beta = synth.to_bf16_bits((np.abs(rng.standard_normal(n)) + 0.01).astype(np.float32))
    bf = synth.bf16_bits_to_f32(beta).astype(np.float64)
    q = np.zeros((n, h * hd), np.uint16)
    k = np.zeros((n, h * hd), np.uint16)
    q[:, 7::hd] = synth.to_bf16_bits(np.full((1,), a, np.float32))[0]
    k[:, 7::hd] = beta[:, None]
    M = torch.empty((nb, nb), device="cuda")
    I, _ = lemo.lemo_block_scores(dev(q), dev(k), h, hd, b, O.REDUCE_PAPER, block_scores=M)
    col = a * bf.reshape(nb, b).max(axis=1) / math.sqrt(hd)
    ok, worst = scores_close(I.cpu().numpy(), nb * col, rel=1e-5)
    assert ok, worst
    for (r, c) in ((nb - 1, nb - 1), (nb - 1, 5), (nb * 5 // 8, nb * 7 // 8)):
        assert abs(float(M[r, c]) - col[c]) <= 1e-5 * col[c], (r, c, float(M[r, c]), col[c])
    del M


def test_exact_deterministic():
    q, k = rand_qk(77, 1024, 4, 128)
    outs = []
    for _ in range(2):
        M = torch.empty((16, 16), device="cuda")
        I, _ = lemo.lemo_block_scores(dev(q), dev(k), 4, 128, 64, O.REDUCE_PAPER, block_scores=M)
        outs.append((I.cpu().numpy().tobytes(), M.cpu().numpy().tobytes()))
    assert outs[0] == outs[1]


def test_exact_strided_operands():
    """Q and K read from wider rows (ld > H*hd), e.g. slices of a fused QKV."""
    n, h, hd, b = 256, 2, 64, 64
    q, k = rand_qk(9, n, h, hd)
    _, I_ref = O.exact_block_scores(q, k, h, hd, b, O.REDUCE_PAPER)
    qp, kp = padded(q, 200, 0x7FC0), padded(k, 136, 0x7FC0)   # NaN in the unused columns
    I, _ = lemo.lemo_block_scores(qp[:, :h * hd], kp[:, :h * hd], h, hd, b, O.REDUCE_PAPER)
    ok, worst = scores_close(I.cpu().numpy(), I_ref)
    assert ok and worst < 1e-4


EIGHT_WAVE = [
    # (B, N, H, hd, block): launches the eight-wave kernel takes (no mask,
    # whole blocks, an even head count, >= 16 chunks per tile, >= 512 of its
    # 256 x 128 tiles)
    (1, 4096, 8, 128, 32),     # 32-row blocks: four per wave
    (1, 4096, 8, 128, 128),    # 128-row blocks span a group's four waves
    (1, 4096, 16, 64, 64),     # head_dim 64: every chunk ends a head
    (2, 3072, 8, 128, 64),     # a batch of two
    (1, 4160, 8, 128, 64),     # rows past N in the last query and key tiles (65 whole blocks)
    (1, 4224, 16, 64, 128),    # half of the last query tile past N (33 blocks of 128)
    (1, 4096, 128, 64, 128),   # the most heads HEADMAX takes: per-head maxima in LDS
]


@pytest.mark.parametrize("mode", [O.REDUCE_PAPER, O.REDUCE_HEADMAX], ids=["paper", "headmax"])
@pytest.mark.parametrize("shape", EIGHT_WAVE, ids=lambda s: "B%d_N%d_H%d_hd%d_b%d" % s)
def test_exact_eight_wave_sampled(shape, mode):
    """The eight-wave exact-score kernel against the oracle: sampled block
    pairs (the diagonal ones, whose i == j pairs are excluded, the last
    blocks, pairs in every wave group's rows, random ones) and two whole
    columns with their column scores, in every sequence of the batch."""
    B, n, h, hd, b = shape
    say("eight-wave exact", shape, mode)
    q, k = rand_batch(6000 + n + h + b, B, n, h, hd)
    nb = n // b
    M = torch.full((B, nb, nb), -1.0, device="cuda")
    I, _ = lemo.lemo_block_scores_batched(dev(q), dev(k), h, hd, b, mode, block_scores=M)
    torch.cuda.synchronize()
    Mg, Ig = M.cpu().numpy(), I.cpu().numpy()
    assert (Mg >= 0).all()                          # every entry written
    rng = np.random.default_rng(n + b)
    entries = [(0, 0), (1, 1), (nb - 1, nb - 1), (nb - 1, 0), (0, nb - 1), (nb // 2, nb // 2 + 1)]
    entries += [tuple(int(x) for x in rng.integers(0, nb, 2)) for _ in range(10)]
    for s in range(B):
        _sampled_check(q[s], k[s], h, hd, b, mode, entries, [int(rng.integers(0, nb)), nb - 1], Mg[s], Ig[s])


EIGHT_WAVE_CAUSAL = [
    # (B, N, H, hd, block): causal launches the eight-wave kernel takes (N a
    # multiple of 256, >= 512 of its tiles on or below the diagonal)
    (2, 4096, 8, 128, 64),     # 2 x 272 tiles
    (1, 6144, 16, 64, 32),     # 600 tiles, 32-row blocks, head_dim 64
    (1, 6144, 8, 128, 128),    # 128-row blocks span a group's four waves
    (1, 6144, 128, 64, 128),   # HEADMAX's most heads: per-head maxima in LDS
]


@pytest.mark.parametrize("mode", [O.REDUCE_PAPER, O.REDUCE_HEADMAX], ids=["paper", "headmax"])
@pytest.mark.parametrize("shape", EIGHT_WAVE_CAUSAL, ids=lambda s: "B%d_N%d_H%d_hd%d_b%d" % s)
def test_exact_eight_wave_causal_sampled(shape, mode):
    """The eight-wave kernel's causal launches against the oracle's causal
    scores: every entry written (M pre-filled with -1), every block above the
    diagonal 0, sampled blocks on, next to and below the diagonal, and two
    whole columns with their column scores."""
    B, n, h, hd, b = shape
    say("eight-wave causal", shape, mode)
    q, k = rand_batch(6500 + n + h + b, B, n, h, hd)
    nb = n // b
    M = torch.full((B, nb, nb), -1.0, device="cuda")
    I, _ = lemo.lemo_block_scores_batched(dev(q), dev(k), h, hd, b, mode, causal=True, block_scores=M)
    torch.cuda.synchronize()
    Mg, Ig = M.cpu().numpy(), I.cpu().numpy()
    assert (Mg >= 0).all()
    upper = np.triu_indices(nb, 1)
    rng = np.random.default_rng(n + b + 1)
    entries = [(0, 0), (1, 1), (1, 0), (nb - 1, nb - 1), (nb - 1, nb - 2), (nb - 1, 0), (nb // 2, nb // 2)]
    entries += [tuple(sorted(int(x) for x in rng.integers(0, nb, 2))[::-1]) for _ in range(8)]
    for s in range(B):
        assert not Mg[s][upper].any()
        for (r, c) in entries:
            M_ref, _ = O.exact_block_scores(q[s], k[s], h, hd, b, mode, query_blocks=[r], key_blocks=[c], causal=True)
            ok, worst = scores_close([Mg[s, r, c]], M_ref[0])
            assert ok and worst < 1e-4, (s, r, c, Mg[s, r, c], M_ref[0, 0])
        for c in (int(rng.integers(0, nb)), 0):
            I_ref, col = O.exact_column_score(q[s], k[s], h, hd, b, mode, c, causal=True)
            ok, worst = scores_close(Mg[s][:, c], col)
            assert ok, (s, c, worst)
            ok, worst = scores_close([Ig[s, c]], [I_ref])
            assert ok and worst < 1e-4, (s, c, Ig[s, c], I_ref)


DISPATCH_EDGES = [
    # (B, N, H, hd, block, causal): on either side of the eight-wave kernel's
    # launch conditions (even head count, >= 16 chunks per tile, >= 512 of
    # its tiles, causal N a multiple of 256); each side against the oracle
    (1, 4096, 9, 128, 64, False),    # odd head count: four-wave kernel
    (1, 4096, 14, 64, 64, False),    # 14 chunks per tile: four-wave kernel
    (1, 3840, 8, 128, 64, False),    # 450 tiles: four-wave kernel
    (1, 4096, 8, 128, 64, False),    # 512 tiles: eight-wave kernel
    (1, 5632, 8, 128, 64, True),     # 506 causal tiles: four-wave kernel
    (1, 5888, 8, 128, 64, True),     # 552 causal tiles: eight-wave kernel
    (1, 6016, 8, 128, 64, True),     # N not a multiple of 256: four-wave kernel
]


@pytest.mark.parametrize("mode", [O.REDUCE_PAPER, O.REDUCE_HEADMAX], ids=["paper", "headmax"])
@pytest.mark.parametrize("shape", DISPATCH_EDGES,
                         ids=lambda s: "B%d_N%d_H%d_hd%d_b%d_%s" % (*s[:5], "causal" if s[5] else "full"))
def test_exact_dispatch_edges_sampled(shape, mode):
    B, n, h, hd, b, causal = shape
    say("dispatch edge", shape, mode)
    q, k = rand_batch(6900 + n + h, B, n, h, hd)
    nb = n // b
    M = torch.full((B, nb, nb), -1.0, device="cuda")
    I, _ = lemo.lemo_block_scores_batched(dev(q), dev(k), h, hd, b, mode, causal=causal, block_scores=M)
    torch.cuda.synchronize()
    Mg, Ig = M.cpu().numpy()[0], I.cpu().numpy()[0]
    assert (Mg >= 0).all()
    if causal:
        assert not Mg[np.triu_indices(nb, 1)].any()
    rng = np.random.default_rng(n + h)
    entries = [(0, 0), (nb - 1, nb - 1), (nb - 1, 0), (nb // 2, nb // 2 - 1)]
    entries += [tuple(sorted(int(x) for x in rng.integers(0, nb, 2))[::-1]) for _ in range(4)]
    for (r, c) in entries:
        M_ref, _ = O.exact_block_scores(q[0], k[0], h, hd, b, mode, query_blocks=[r], key_blocks=[c], causal=causal)
        ok, worst = scores_close([Mg[r, c]], M_ref[0])
        assert ok and worst < 1e-4, (r, c, Mg[r, c], M_ref[0, 0])
    c = int(rng.integers(0, nb))
    I_ref, col = O.exact_column_score(q[0], k[0], h, hd, b, mode, c, causal=causal)
    ok, worst = scores_close(Mg[:, c], col)
    assert ok, (c, worst)
    ok, worst = scores_close([Ig[c]], [I_ref])
    assert ok and worst < 1e-4, (c, Ig[c], I_ref)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_exact_eight_wave_strided(causal):
    """The eight-wave kernel on Q and K read from wider rows (ld > H*hd, e.g.
    slices of a fused QKV) with NaN in every column it must not read:
    bit-equal to the same call on dense copies, and sampled blocks against the
    oracle."""
    n, h, hd, b = 6144, 8, 128, 64
    say("eight-wave strided", causal)
    q, k = rand_qk(6950, n, h, hd)
    nb = n // b
    Md = torch.empty((1, nb, nb), device="cuda")
    lemo.lemo_block_scores_batched(dev(q), dev(k), h, hd, b, O.REDUCE_PAPER, causal=causal, block_scores=Md)
    qp, kp = padded(q, 1160, 0x7FC0), padded(k, 1096, 0x7FC0)   # NaN in the unused columns
    Ms = torch.empty((1, nb, nb), device="cuda")
    lemo.lemo_block_scores_batched(qp[:, :h * hd], kp[:, :h * hd], h, hd, b, O.REDUCE_PAPER, causal=causal,
                                   block_scores=Ms)
    torch.cuda.synchronize()
    assert torch.equal(Md, Ms)
    Mg = Ms.cpu().numpy()[0]
    for (r, c) in ((0, 0), (nb - 1, nb - 1), (nb - 1, 3), (40, 17)):
        M_ref, _ = O.exact_block_scores(q, k, h, hd, b, O.REDUCE_PAPER, query_blocks=[r], key_blocks=[c],
                                        causal=causal)
        ok, worst = scores_close([Mg[r, c]], M_ref[0])
        assert ok and worst < 1e-4, (r, c, Mg[r, c], M_ref[0, 0])


def test_exact_eight_wave_deterministic():
    """Two launches of the eight-wave kernel give the same bits."""
    q, k = rand_qk(78, 4096, 8, 128)
    outs = []
    for _ in range(2):
        M = torch.empty((64, 64), device="cuda")
        I, _ = lemo.lemo_block_scores(dev(q), dev(k), 8, 128, 64, O.REDUCE_PAPER, block_scores=M)
        outs.append((I.cpu().numpy().tobytes(), M.cpu().numpy().tobytes()))
    assert outs[0] == outs[1]


# ---------------------------------- batches, causal masking, ragged last block
BATCHED_SMALL = [
    # (B, N, H, hd, block)
    (1, 256, 2, 128, 64),
    (2, 1000, 3, 64, 64),     # ragged: 15 whole blocks + 40 tokens
    (3, 200, 2, 128, 32),     # ragged 32-row blocks
    (1, 300, 1, 64, 128),     # ragged 128-row block spanning the tile's four waves
    (2, 1, 1, 64, 64),        # one token: its only pair is excluded
    (1, 65, 2, 64, 64),       # a last block of one token
    (2, 1536, 4, 128, 64),    # 78 causal tiles: not a multiple of 8 (no XCD split)
    (1, 2048, 4, 128, 64),    # 136 causal tiles: XCD split, groups of 8 query tiles
    (2, 200, 5, 64, 32),      # head_dim 64, an odd head count, ragged 32-row blocks
]


def rand_batch(seed, B, n, h, hd):
    rng = np.random.default_rng(seed)
    return (np.stack([synth.random_bf16(rng, (n, h * hd), 1.0) for _ in range(B)]),
            np.stack([synth.random_bf16(rng, (n, h * hd), 1.0) for _ in range(B)]))


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("mode", [O.REDUCE_PAPER, O.REDUCE_HEADMAX], ids=["paper", "headmax"])
@pytest.mark.parametrize("shape", BATCHED_SMALL, ids=lambda s: "B%d_N%d_H%d_hd%d_b%d" % s)
def test_scores_batched_small(shape, mode, causal):
    B, n, h, hd, b = shape
    say("batched scores", shape, mode, causal)
    q, k = rand_batch(3000 + n + B, B, n, h, hd)
    M_ref, I_ref = O.exact_block_scores_batched(q, k, h, hd, b, mode, causal=causal)
    nb = -(-n // b)
    M = torch.full((B, nb, nb), -1.0, device="cuda")        # every entry must be written
    I, _ = lemo.lemo_block_scores_batched(dev(q), dev(k), h, hd, b, mode, causal=causal, block_scores=M)
    torch.cuda.synchronize()
    Mg, Ig = M.cpu().numpy(), I.cpu().numpy()
    assert (Mg >= 0).all()
    okm, worstm = scores_close(Mg, M_ref)
    ok, worst = scores_close(Ig, I_ref)
    assert okm and ok and worstm < 1e-4 and worst < 1e-4, (worstm, worst)
    if causal:
        assert not Mg[:, np.triu_indices(nb, 1)[0], np.triu_indices(nb, 1)[1]].any()


ONE_HEAD_WALK = [
    # (B, N, hd, block, causal): one head, more than 2048 tiles in the launch,
    # so each workgroup walks a range of several tiles (the next tile's first
    # chunk loading under the current tile's last)
    (1, 6144, 64, 128, False),     # 128-row blocks: the four waves' maxima meet in LDS per tile
    (1, 6016, 128, 32, False),     # 32-row blocks: each wave writes its own four blocks
    (2, 6000, 128, 64, False),     # batch of two ragged sequences
    (1, 8190, 64, 64, True),       # causal, ragged: 2080 tiles on or below the diagonal
    # the eight-wave form (one sequence, no mask, blocks of 32 or 64, N a
    # multiple of 1024, >= 512 tiles of 256 x 128): each workgroup walks
    # tiles 256 apart, loads running on across tile boundaries
    (1, 4096, 128, 64, False),     # 512 tiles: two per workgroup
    (1, 4096, 64, 32, False),      # head_dim 64 (a tile is one chunk), 32-row blocks
    (1, 8192, 128, 32, False),     # 2048 tiles, 32-row blocks
]


@pytest.mark.parametrize("shape", ONE_HEAD_WALK, ids=lambda s: "B%d_N%d_hd%d_b%d_%s" % (*s[:4], "causal" if s[4] else "full"))
def test_one_head_range_walk(shape):
    """The one-head kernel (the per-token predictor's scoring) when every
    workgroup walks several consecutive tiles: the whole block matrix against
    the oracle."""
    B, n, hd, b, causal = shape
    say("one-head range walk", shape)
    q, k = rand_batch(4000 + n + hd, B, n, 1, hd)
    M_ref, I_ref = O.exact_block_scores_batched(q, k, 1, hd, b, O.REDUCE_PAPER, causal=causal)
    nb = -(-n // b)
    M = torch.full((B, nb, nb), -1.0, device="cuda")
    I, _ = lemo.lemo_block_scores_batched(dev(q), dev(k), 1, hd, b, O.REDUCE_PAPER, causal=causal, block_scores=M)
    torch.cuda.synchronize()
    Mg, Ig = M.cpu().numpy(), I.cpu().numpy()
    assert (Mg >= 0).all()
    okm, worstm = scores_close(Mg, M_ref)
    ok, worst = scores_close(Ig, I_ref)
    assert okm and ok and worstm < 1e-4 and worst < 1e-4, (worstm, worst)


def test_scores_batched_equals_single_call():
    """One sequence, whole blocks, no mask: the same kernel as lemo_block_scores, bit for bit."""
    q, k = rand_qk(41, 1024, 4, 128)
    for mode in (O.REDUCE_PAPER, O.REDUCE_HEADMAX):
        M1 = torch.empty((16, 16), device="cuda")
        M2 = torch.empty((1, 16, 16), device="cuda")
        I1, _ = lemo.lemo_block_scores(dev(q), dev(k), 4, 128, 64, mode, block_scores=M1)
        I2, _ = lemo.lemo_block_scores_batched(dev(q), dev(k), 4, 128, 64, mode, block_scores=M2)
        assert torch.equal(I1, I2[0]) and torch.equal(M1, M2[0])


def test_scores_batched_strided():
    """Sequences inside a larger buffer: wide rows (ld > H*hd) and a gap
    between sequences, NaN everywhere the call must not read."""
    B, n, h, hd, b = 3, 320, 2, 64, 64
    q, k = rand_batch(44, B, n, h, hd)
    ld, gap_rows = 200, 5
    buf_q = np.full((B, n + gap_rows, ld), 0x7FC0, np.uint16)
    buf_k = np.full((B, n + gap_rows, ld), 0x7FC0, np.uint16)
    buf_q[:, :n, :h * hd] = q
    buf_k[:, :n, :h * hd] = k
    qd, kd = dev(buf_q)[:, :n, :h * hd], dev(buf_k)[:, :n, :h * hd]
    assert qd.stride() == ((n + gap_rows) * ld, ld, 1)
    for causal in (False, True):
        _, I_ref = O.exact_block_scores_batched(q, k, h, hd, b, O.REDUCE_HEADMAX, causal=causal)
        I, _ = lemo.lemo_block_scores_batched(qd, kd, h, hd, b, O.REDUCE_HEADMAX, causal=causal)
        ok, worst = scores_close(I.cpu().numpy(), I_ref)
        assert ok and worst < 1e-4, (causal, worst)


@pytest.mark.parametrize("n", [16384, 16384 - 40], ids=["N16384", "N16344_ragged"])
@pytest.mark.parametrize("mode", [O.REDUCE_PAPER, O.REDUCE_HEADMAX], ids=["paper", "headmax"])
def test_causal_closed_form_full_size(mode, n):
    """Q_i = a e and K_j = beta_j e in every head, 32 heads of 128, blocks of
    64 (the 7B shape).  Causal: block pair (n, m) is a * max of beta_j over the
    keys of block m that precede some query of block n, over sqrt(hd) (times
    H for HEADMAX): all of block m below the diagonal, all but its last token
    on it, nothing above.  So I[m] = (nb - 1 - m) * full[m] + diag[m]."""
    h, hd, b = 32, 128, 64
    nb = -(-n // b)
    rng = np.random.default_rng(22)
    a = 0.75
    beta = synth.to_bf16_bits(np.abs(rng.standard_normal(n)).astype(np.float32) + 0.01)
    bf = synth.bf16_bits_to_f32(beta).astype(np.float64)
    q = np.zeros((n, h * hd), np.uint16)
    k = np.zeros((n, h * hd), np.uint16)
    q[:, 3::hd] = synth.to_bf16_bits(np.full((1,), a, np.float32))[0]
    k[:, 3::hd] = beta[:, None]
    c = a / math.sqrt(hd) * (h if mode == O.REDUCE_HEADMAX else 1)
    full = np.array([bf[m * b:min((m + 1) * b, n)].max() for m in range(nb)]) * c
    diag = np.array([bf[m * b:min((m + 1) * b, n) - 1].max() if min((m + 1) * b, n) - m * b > 1 else 0.0
                     for m in range(nb)]) * c
    expect = (nb - 1 - np.arange(nb)) * full + diag
    M = torch.empty((1, nb, nb), device="cuda")
    I, _ = lemo.lemo_block_scores_batched(dev(q), dev(k), h, hd, b, mode, causal=True, block_scores=M)
    ok, worst = scores_close(I.cpu().numpy()[0], expect, rel=1e-5)
    assert ok, worst
    Mg = M.cpu().numpy()[0]
    assert not Mg[np.triu_indices(nb, 1)].any()
    ok, worst = scores_close(Mg.diagonal(), diag, rel=1e-5)
    assert ok, worst


def test_causal_full_size_sampled():
    """The 7B N=16K exact workload, causal, in the benchmark's launch
    configuration: sampled block scores and whole columns from the oracle;
    below the block diagonal the causal launch runs the same MFMA chains as
    the full one (the eight-wave kernel in both), so those entries equal the
    full-attention call bit for bit."""
    w = synth.WORKLOADS["llama2-7b-n16k"]
    say("causal full size")
    L = synth.make_layer(w.n_tokens, w.d_model, w.block, w.seed, n_heads=w.n_heads, head_dim=w.head_dim,
                         planted_frac=w.planted_frac, with_y=False, proj_device="cuda")
    nb = w.n_blocks
    rng = np.random.default_rng(6)
    entries = [(0, 0), (nb - 1, nb - 1), (nb - 1, 0), (5, 200)] + \
        [tuple(sorted(rng.integers(0, nb, 2))[::-1]) for _ in range(4)]
    qd, kd = dev(L.q), dev(L.k)
    lower = np.tril(np.ones((nb, nb), dtype=bool), -1)
    for mode in (O.REDUCE_PAPER, O.REDUCE_HEADMAX):
        M = torch.empty((1, nb, nb), device="cuda")
        I, _ = lemo.lemo_block_scores_batched(qd, kd, w.n_heads, w.head_dim, w.block, mode, causal=True,
                                              block_scores=M)
        Mg, Ig = M.cpu().numpy()[0], I.cpu().numpy()[0]
        for (r, c) in entries:
            M_ref, _ = O.exact_block_scores(L.q, L.k, w.n_heads, w.head_dim, w.block, mode, query_blocks=[r],
                                            key_blocks=[c], causal=True)
            ok, worst = scores_close([Mg[r, c]], M_ref[0])
            assert ok and worst < 1e-4, (r, c, Mg[r, c], M_ref[0, 0])
        for c in (nb - 1, 7):
            I_ref, col = O.exact_column_score(L.q, L.k, w.n_heads, w.head_dim, w.block, mode, c, causal=True)
            ok, worst = scores_close(Mg[:, c], col)
            assert ok, (c, worst)
            ok, worst = scores_close([Ig[c]], [I_ref])
            assert ok and worst < 1e-4, (c, Ig[c], I_ref)
        Mf = torch.empty((nb, nb), device="cuda")
        lemo.lemo_block_scores(qd, kd, w.n_heads, w.head_dim, w.block, mode, block_scores=Mf)
        assert np.array_equal(Mg[lower], Mf.cpu().numpy()[lower])
        assert not Mg[np.triu_indices(nb, 1)].any()


# ------------------------------- ragged last block: predictor and movement calls
PRED_RAGGED = [
    # (N, d, block, rank): the last block holds N mod block rows
    (1000, 256, 64, 64),
    (200, 128, 32, 32),
    (130, 512, 64, 128),
    (4000, 192, 256, 96),
    (3001, 128, 2, 32),       # 1501 blocks, the last of one row: two key blocks per pair workgroup, one left over
]


@pytest.mark.parametrize("shape", PRED_RAGGED, ids=lambda s: "N%d_d%d_b%d_r%d" % s)
def test_predict_ragged(shape):
    n, d, b, r = shape
    say("predict ragged", shape)
    x, w = _pred_inputs(n + d + r + 1, n, d, r)
    nb = -(-n // b)
    M_ref, I_ref, _, _ = O.predict_scores(x, *w, b)
    assert M_ref.shape == (nb, nb)
    M = torch.full((nb, nb), -1.0, device="cuda")
    I, _ = lemo.lemo_predict_scores(dev(x), *[dev(a) for a in w], b, block_scores=M)
    Ig, Mg = I.cpu().numpy(), M.cpu().numpy()
    ok, worst = scores_close(Ig, I_ref)
    assert ok and worst < 1e-3, worst
    merr = np.abs(Mg - M_ref) <= 1e-2 * np.abs(M_ref) + 1e-3 * np.abs(M_ref).max()
    assert merr.all(), float(np.abs(Mg - M_ref).max())


MOVE_RAGGED = [
    # (N, width, block, kept blocks, pad_multiple): kept lists as select gives them
    # (ascending), with and without the short last block, and one that lists the
    # short block first (its missing rows are skipped and flagged)
    (1000, 256, 64, [1, 4, 5, 9, 15], 64),          # short last block (40 rows) kept
    (1000, 256, 64, [0, 3, 8, 14], 64),             # short block dropped
    (200, 64, 32, list(range(7)), 1),               # keep all: 6 x 32 + 8 rows = N
    (1000, 128, 64, [15, 2, 9], 32),                # short block listed first
]


@pytest.mark.parametrize("case", MOVE_RAGGED,
                         ids=lambda c: "N%d_w%d_b%d_%s" % (c[0], c[1], c[2], "-".join(map(str, c[3]))))
def test_movement_ragged(case):
    n, w, b, kept_l, pad = case
    say("movement ragged", case)
    rng = np.random.default_rng(n + w + len(kept_l))
    nb = -(-n // b)
    kept = np.array(kept_l, np.int32)
    nk = kept.size
    misplaced = nk and kept[:-1].max(initial=-1) == nb - 1 and n % b
    rows = O.kept_token_rows(kept, nk, b, n)
    R = rows.size
    cap = -(-R // pad) * pad + 3
    src = synth.random_bf16(rng, (n, w))
    kept_d = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    kept_d[:nk] = torch.from_numpy(kept).cuda()
    nk_d = torch.tensor([nk], dtype=torch.int32, device="cuda")
    expect_status = lemo.DEV_BAD_KEPT if misplaced else 0
    # gather with padding
    sentinel = np.full((cap, w), 0x5A5A, np.uint16)
    dst_ref, over = O.gather_pad(src, b, kept, nk, sentinel, pad)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dstd = dev(sentinel)
    lemo.lemo_gather_pad(dev(src), b, kept_d, nk_d, dstd, pad_multiple=pad, dev_status=status)
    assert np.array_equal(host_bits(dstd), dst_ref) and not over
    assert int(status.item()) == expect_status
    # in-place addition, then its backward recompute
    res = synth.random_bf16(rng, (n, w))
    y = synth.random_bf16(rng, (max(R, 1), w), 0.1)
    ref = O.scatter_residual(res, b, kept, nk, y)
    resd = dev(res)
    status.zero_()
    lemo.lemo_scatter_residual(resd, b, kept_d, nk_d, dev(y), dev_status=status)
    assert np.array_equal(host_bits(resd), ref)
    assert int(status.item()) == expect_status
    back_ref = O.residual_recompute(ref, b, kept, nk, y)
    lemo.lemo_residual_recompute(resd, b, kept_d, nk_d, dev(y))
    assert np.array_equal(host_bits(resd), back_ref)
    # the same movement fused into products (d_in = width, a multiple of 64)
    wt = synth.random_bf16(rng, (72, w), 1.0 / math.sqrt(w))
    ysent = np.full((cap, 72), 0x5A5A, np.uint16)
    yref, _ = O.gather_linear(src, b, kept, nk, wt, ysent, pad)
    yd = dev(ysent)
    status.zero_()
    lemo.lemo_gather_linear(dev(src), b, kept_d, nk_d, dev(wt), yd, pad_multiple=pad, dev_status=status)
    got = host_bits(yd)
    live = rows >= 0
    ok, same = _embeddings_close(got[:R][live], yref[:R][live])
    assert ok, same
    assert np.array_equal(got[:R][~live], yref[:R][~live]) and np.array_equal(got[R:], yref[R:])
    assert int(status.item()) == expect_status
    a = synth.random_bf16(rng, (max(R, 1), w))
    w2 = synth.random_bf16(rng, (w, w), 1.0 / math.sqrt(w))
    sref = O.linear_scatter(a, w2, res, b, kept, nk)
    r2 = dev(res)
    lemo.lemo_linear_scatter(dev(a), dev(w2), r2, b, kept_d, nk_d)
    got2 = host_bits(r2)
    touched = np.zeros(n, bool)
    touched[rows[rows >= 0]] = True
    assert np.array_equal(got2[~touched], res[~touched])
    ok, same = _embeddings_close(got2[touched], sref[touched])
    assert ok, same


# ------------------------------------------------------------- predictor
PRED_SMALL = [
    # (N, d, block, rank)
    (256, 128, 4, 32),
    (512, 256, 2, 64),
    (1024, 512, 64, 32),
    (2048, 192, 8, 96),
    (4096, 320, 256, 256),
    (4096, 256, 2, 64),       # 2048 blocks: two key blocks per pair workgroup
    (2048, 1280, 32, 32),     # five slices of d_model in the hidden product
    (1024, 512, 8, 160),      # a rank above 128 that is not a power of two
]


def _pred_inputs(seed, n, d, r, planted=0.2, b=64):
    rng = np.random.default_rng(seed)
    x = synth.random_bf16(rng, (n, d))
    w = [synth.random_bf16(rng, s, 1.0 / math.sqrt(s[0])) for s in ((d, r), (r, r), (d, r), (r, r))]
    return x, w


def _check_pred(x, w, b, d_model=None, xdev=None):
    n = x.shape[0]
    nb = n // b
    M_ref, I_ref, _, _ = O.predict_scores(x, *w, b)
    M = torch.full((nb, nb), -1.0, device="cuda")
    xd = dev(x) if xdev is None else xdev
    I, _ = lemo.lemo_predict_scores(xd, *[dev(a) for a in w], b, d_model=d_model, block_scores=M)
    Ig, Mg = I.cpu().numpy(), M.cpu().numpy()
    ok, worst = scores_close(Ig, I_ref)
    assert ok, worst
    merr = np.abs(Mg - M_ref) <= 1e-2 * np.abs(M_ref) + 1e-3 * np.abs(M_ref).max()
    assert merr.all(), float(np.abs(Mg - M_ref).max())
    return worst


@pytest.mark.parametrize("shape", PRED_SMALL, ids=lambda s: "N%d_d%d_b%d_r%d" % s)
def test_predict_small(shape):
    n, d, b, r = shape
    say("predict", shape)
    x, w = _pred_inputs(n + d + r, n, d, r)
    worst = _check_pred(x, w, b)
    assert worst < 1e-3, worst


@pytest.mark.parametrize("wname", ["llama2-7b-n16k", "llama2-13b-n32k-4layer"])
def test_predict_workload(wname):
    w = synth.WORKLOADS[wname]
    say("predict workload", wname)
    L = synth.make_layer(w.n_tokens, w.d_model, w.block, w.seed, rank=w.rank, planted_frac=w.planted_frac,
                         with_y=False)
    worst = _check_pred(L.x, [L.u_q, L.v_q, L.u_k, L.v_k], w.block)
    assert worst < 1e-3, worst


def test_predict_strided_x():
    n, d, b, r = 512, 128, 8, 32
    x, w = _pred_inputs(3, n, d, r)
    xp = padded(x, 200 + 0, 0x7FC0)
    _check_pred(x, w, b, xdev=xp[:, :d])


# ---------------------------------------------------------------- select
def _select_case(scores_f32, mode, threshold=0.0, keep=0):
    s = np.asarray(scores_f32, np.float32)
    nb = s.size
    mask_r, kept_r, nk_r, th_r = O.select_mask(s, mode, threshold, keep)
    kept = torch.full((nb,), -7, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    mask, kept, nk, th = lemo.lemo_select_mask(dev(s), mode, threshold, keep, kept_blocks=kept, dev_status=status)
    nk = int(nk.item())
    kept = kept.cpu().numpy()
    assert nk == nk_r
    assert np.array_equal(mask.cpu().numpy(), mask_r)
    assert np.array_equal(kept[:nk], kept_r)
    assert np.all(kept[nk:] == -7)
    thg = th.cpu().numpy()[0]
    assert (np.isnan(thg) and np.isnan(th_r)) or thg.tobytes() == np.float32(th_r).tobytes(), (thg, th_r)
    st = int(status.item())
    assert bool(st & lemo.DEV_NONFINITE) == (not np.isfinite(s).all())


@pytest.mark.parametrize("nb", [1, 5, 64, 256, 1000, 1025, 4097, 8192])
@pytest.mark.parametrize("mode", ["threshold", "mean", "topk"])
def test_select_random(nb, mode):
    rng = np.random.default_rng(nb)
    s = (rng.random(nb) * 10).astype(np.float32)
    if mode == "threshold":
        _select_case(s, O.SELECT_THRESHOLD, threshold=float(np.median(s)))
    elif mode == "mean":
        _select_case(s, O.SELECT_MEAN)
    else:
        for k in sorted({0, 1, nb // 3, nb - 1, nb} - {-1}):
            if 0 <= k <= nb:
                _select_case(s, O.SELECT_TOPK, keep=k)


def test_select_edge_values():
    ties = np.array([3, 1, 3, 3, 2, 3, 0, 3], np.float32)
    for k in range(9):
        _select_case(ties, O.SELECT_TOPK, keep=k)
    _select_case(ties, O.SELECT_THRESHOLD, threshold=3.0)
    _select_case(ties, O.SELECT_MEAN)
    zeros = np.array([0.0, -0.0, 0.0, 1.0, -0.0], np.float32)
    for k in range(6):
        _select_case(zeros, O.SELECT_TOPK, keep=k)
    _select_case(zeros, O.SELECT_THRESHOLD, threshold=-0.0)
    nan = np.array([np.nan, 2, np.inf, 1, np.nan, -np.inf], np.float32)
    for k in range(7):
        _select_case(nan, O.SELECT_TOPK, keep=k)
    _select_case(nan, O.SELECT_THRESHOLD, threshold=1.5)
    _select_case(nan, O.SELECT_MEAN)
    same = np.full(300, 0.25, np.float32)
    _select_case(same, O.SELECT_TOPK, keep=77)
    _select_case(same, O.SELECT_MEAN)


def test_select_mean_sum_paths():
    """The mean's float64 sum: exact inputs (every partial sum representable,
    summed as a tree) and inputs whose sum in block order rounds (summed by one
    lane in that order) both give the oracle's threshold bit for bit."""
    rng = np.random.default_rng(11)
    for nb in (3, 256, 1024, 1025, 8192):   # one wave reduces up to 1024 blocks, 16 beyond
        # multiples of 2^-8 below 64, either sign: a span of at most 27 bits
        s = (rng.integers(-2 ** 14, 2 ** 14, nb) / 256.0).astype(np.float32)
        _select_case(s, O.SELECT_MEAN)
        # a 2^60 term beside small ones: the sum in block order rounds
        w = (rng.random(nb) * 4).astype(np.float32)
        w[nb // 3] = np.float32(2.0 ** 60)
        w[(2 * nb) // 3] = np.float32(-(2.0 ** 60))
        _select_case(w, O.SELECT_MEAN)
    # rounding decides the threshold: 2^60 + 1 - 2^60 is 0 in block order, 1 exactly
    _select_case(np.array([2.0 ** 60, 1.0, -(2.0 ** 60)], np.float32), O.SELECT_MEAN)
    # float32 subnormals beside normal scores, and zeros of both signs only
    _select_case(np.array([1e-45, 3e-39, 0.5, 2.0], np.float32), O.SELECT_MEAN)
    _select_case(np.array([-0.0, 0.0, -0.0], np.float32), O.SELECT_MEAN)


@pytest.mark.parametrize("nb", [511, 512, 513])
def test_select_topk_ties_mid_sizes(nb):
    """Top-k at mid sizes with many ties (40 distinct scores)."""
    rng = np.random.default_rng(nb)
    s = rng.integers(0, 40, nb).astype(np.float32) / 4
    for k in (1, nb // 5, nb // 2, nb - 1, nb):
        _select_case(s, O.SELECT_TOPK, keep=k)


def test_select_on_oracle_scores():
    """The realistic case: scores of a real workload (oracle's, rounded to fp32)."""
    w = synth.WORKLOADS["tiny"]
    L = synth.make_workload(w, with_y=False)
    _, I_ref = O.exact_block_scores(L.q, L.k, w.n_heads, w.head_dim, w.block, O.REDUCE_PAPER)
    s = I_ref.astype(np.float32)
    _select_case(s, O.SELECT_MEAN)
    _select_case(s, O.SELECT_TOPK, keep=synth.keep_count(50, w.n_blocks))


# ------------------------------------------------------- gather / scatter
MOVE = [
    # (N, width, ld_src, ld_dst, block, keep fraction, pad_multiple, cap extra rows)
    (256, 64, 64, 64, 4, 0.5, 1, 0),
    (1024, 512, 520, 512, 64, 0.5, 256, 8),
    (2048, 8, 16, 8, 16, 0.3, 7, 3),
    (4096, 2048, 2048, 2056, 64, 0.4, 256, 0),
    (1024, 1376, 1376, 1376, 32, 1.0, 64, 0),     # keep all
    (1024, 256, 256, 256, 64, 0.0, 256, 5),       # keep none
    (16384, 11008, 11008, 11008, 64, 0.35, 256, 0),  # MLP activation width
]


def _kept_from_mask(rng, nb, frac):
    m = rng.random(nb) < frac
    if frac >= 1.0:
        m[:] = True
    return np.nonzero(m)[0].astype(np.int32)


@pytest.mark.parametrize("case", MOVE, ids=lambda c: "N%d_w%d_b%d_keep%.2f_pad%d" % (c[0], c[1], c[4], c[5], c[6]))
def test_gather_scatter(case):
    n, w, lds, ldd, b, frac, pad, extra = case
    say("move", case)
    rng = np.random.default_rng(n + w)
    nb = n // b
    kept = _kept_from_mask(rng, nb, frac)
    nk = kept.size
    src = synth.random_bf16(rng, (n, w))
    R = nk * b
    cap = max(1, -(-R // pad) * pad + extra)
    sentinel = np.full((cap, w), 0x5A5A, np.uint16)
    dst_ref, over_ref = O.gather_pad(src, b, kept, nk, sentinel, pad)
    kept_d = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    kept_d[:nk] = torch.from_numpy(kept).cuda()
    nk_d = torch.tensor([nk], dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    srcd = padded(src, lds, 0x7FC0)
    dstd = padded(sentinel, ldd, 0x1234)
    lemo.lemo_gather_pad(srcd[:, :w], b, kept_d, nk_d, dstd[:, :w], pad_multiple=pad, dev_status=status)
    got = host_bits(dstd)
    assert np.array_equal(got[:, :w], dst_ref)
    assert np.all(got[:, w:] == 0x1234)
    assert int(status.item()) == 0 and not over_ref
    # scatter: y rows in kept order, residual updated in place
    res = synth.random_bf16(rng, (n, w))
    y = synth.random_bf16(rng, (max(R, 1), w))
    res_ref = O.scatter_residual(res, b, kept, nk, y)
    resd = padded(res, lds, 0x4321)
    yd = padded(y, ldd, 0x7FC0)
    lemo.lemo_scatter_residual(resd[:, :w], b, kept_d, nk_d, yd[:, :w], dev_status=status)
    got = host_bits(resd)
    assert np.array_equal(got[:, :w], res_ref)
    assert np.all(got[:, w:] == 0x4321)
    assert int(status.item()) == 0


GATHER_MULTI = [
    # (N, block, keep fraction, pad_multiple, extra cap rows, [(width, ld_src, ld_dst), ...])
    (1024, 64, 0.5, 256, 8, [(512, 520, 512), (64, 64, 72)]),
    (2048, 16, 0.3, 7, 3, [(8, 16, 8), (2056, 2056, 2064), (1376, 1376, 1376)]),
    (1000, 64, 1.0, 64, 0, [(256, 256, 256), (4096, 4096, 4096), (8, 8, 8), (11008, 11008, 11008)]),  # ragged N
    (1024, 64, 0.0, 256, 5, [(128, 128, 128), (64, 64, 64)]),                                       # keep none
]


@pytest.mark.parametrize("case", GATHER_MULTI, ids=lambda c: "N%d_b%d_keep%.2f_src%d" % (c[0], c[1], c[2], len(c[5])))
def test_gather_multi(case):
    """Several matrices gathered on one kept list in one launch: each
    destination bit-exact against the oracle's gather of that source
    (padding, rows past it left as they were, a ragged last block)."""
    n, b, frac, pad, extra, mats = case
    say("gather multi", case)
    rng = np.random.default_rng(n + len(mats))
    nb = -(-n // b)
    kept = _kept_from_mask(rng, nb, frac)
    nk = kept.size
    R = O.kept_token_rows(kept, nk, b, n).size
    cap = max(1, -(-R // pad) * pad + extra)
    kept_d = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    kept_d[:nk] = torch.from_numpy(kept).cuda()
    nk_d = torch.tensor([nk], dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    srcs, dsts, refs = [], [], []
    for w, lds, ldd in mats:
        src = synth.random_bf16(rng, (n, w))
        sentinel = np.full((cap, w), 0x5A5A, np.uint16)
        ref, over = O.gather_pad(src, b, kept, nk, sentinel, pad)
        assert not over
        srcs.append(padded(src, lds, 0x7FC0))
        dsts.append(padded(sentinel, ldd, 0x1234))
        refs.append(ref)
    lemo.lemo_gather_pad_multi([sd[:, :w] for sd, (w, _, _) in zip(srcs, mats)],
                               [dd[:, :w] for dd, (w, _, _) in zip(dsts, mats)], b, kept_d, nk_d, pad_multiple=pad,
                               n_tokens=n, dev_status=status)
    for dd, ref, (w, _, _) in zip(dsts, refs, mats):
        got = host_bits(dd)
        assert np.array_equal(got[:, :w], ref)
        assert np.all(got[:, w:] == 0x1234)
    assert int(status.item()) == 0


def test_gather_multi_full_size_oracle_mask():
    """X and the MLP activation of the 7B N=16K layer gathered in one launch
    on the oracle's predicted mask (MEAN), padded to 256 rows: bit-exact."""
    w = synth.WORKLOADS["llama2-7b-n16k"]
    say("gather multi full size")
    L = synth.make_layer(w.n_tokens, w.d_model, w.block, w.seed, rank=w.rank, mlp_width=w.mlp_width,
                         planted_frac=w.planted_frac, with_y=False)
    _, I_ref, _, _ = O.predict_scores(L.x, L.u_q, L.v_q, L.u_k, L.v_k, w.block)
    _, kept, nk, _ = O.select_mask(I_ref.astype(np.float32), O.SELECT_MEAN)
    cap = -(-(nk * w.block) // 256) * 256
    dx = torch.empty((cap, w.d_model), dtype=torch.int16, device="cuda")
    da = torch.empty((cap, w.mlp_width), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    lemo.lemo_gather_pad_multi([dev(L.x), dev(L.act)], [dx, da], w.block, dev(kept), dev(np.array([nk], np.int32)),
                               pad_multiple=256, dev_status=status)
    for src, dd, width in ((L.x, dx, w.d_model), (L.act, da, w.mlp_width)):
        ref, _ = O.gather_pad(src, w.block, kept, nk, np.zeros((cap, width), np.uint16), 256)
        assert np.array_equal(host_bits(dd), ref)
    assert int(status.item()) == 0


@pytest.mark.parametrize("case", MOVE, ids=lambda c: "N%d_w%d_b%d_keep%.2f" % (c[0], c[1], c[4], c[5]))
def test_residual_recompute(case):
    """Backward recompute, bit for bit against the oracle on an independent
    random residual; then the forward addition followed by the recompute on
    the GPU comes back within the rounding bound of the input (and exactly
    where the addition was exact)."""
    n, w, lds, ldd, b, frac, pad, extra = case
    say("recompute", case)
    rng = np.random.default_rng(n + w + 7)
    nb = n // b
    kept = _kept_from_mask(rng, nb, frac)
    nk = kept.size
    R = nk * b
    res = synth.random_bf16(rng, (n, w))
    y = synth.random_bf16(rng, (max(R, 1), w), 0.05)
    kept_d = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    kept_d[:nk] = torch.from_numpy(kept).cuda()
    nk_d = torch.tensor([nk], dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref = O.residual_recompute(res, b, kept, nk, y)
    resd = padded(res, lds, 0x4321)
    yd = padded(y, ldd, 0x7FC0)
    lemo.lemo_residual_recompute(resd[:, :w], b, kept_d, nk_d, yd[:, :w], dev_status=status)
    got = host_bits(resd)
    assert np.array_equal(got[:, :w], ref)
    assert np.all(got[:, w:] == 0x4321) and int(status.item()) == 0
    # round trip on the GPU: x -> x + y -> (x + y) - y
    xd = padded(res, lds, 0x4321)
    lemo.lemo_scatter_residual(xd[:, :w], b, kept_d, nk_d, yd[:, :w])
    fwd = host_bits(xd)[:, :w]
    lemo.lemo_residual_recompute(xd[:, :w], b, kept_d, nk_d, yd[:, :w])
    back = host_bits(xd)[:, :w]
    assert np.array_equal(back, O.residual_recompute(O.scatter_residual(res, b, kept, nk, y), b, kept, nk, y))
    rows = (kept[:, None] * b + np.arange(b)[None, :]).reshape(-1)
    xv, fv, bv = (O.bf16_decode(a[rows]) for a in (res, fwd, back))
    spacing = lambda v: np.ldexp(1.0, np.maximum(np.frexp(np.abs(v))[1] - 8, -133))
    assert np.all(np.abs(bv - xv) <= 0.5 * spacing(fv) + 0.5 * spacing(bv))
    exact = fv == xv + O.bf16_decode(y[:rows.size])
    assert np.array_equal(bv[exact], xv[exact])
    dropped = np.setdiff1d(np.arange(n), rows)
    assert np.array_equal(back[dropped], res[dropped])


MLP_SMALL = [
    # (N, width, block, ld)
    (256, 64, 64, 64),
    (1000, 200, 64, 208),       # ragged last block (40 tokens), ld > width
    (200, 2056, 32, 2056),      # two channel chunks, the second 8 wide; ragged (8 tokens)
    (1, 8, 64, 8),              # one token
    (130, 11008, 64, 11008),    # the MLP width of the 7B shape; a 2-token last block
    (4096, 4104, 128, 4104),
    (96, 16, 1, 16),            # blocks of one token
]


@pytest.mark.parametrize("gated", [False, True], ids=["act", "gated"])
@pytest.mark.parametrize("case", MLP_SMALL, ids=lambda c: "N%d_w%d_b%d" % c[:3])
def test_mlp_scores_small(case, gated):
    n, w, b, ld = case
    say("mlp scores", case, gated)
    rng = np.random.default_rng(n + w + b)
    a = synth.random_bf16(rng, (n, w))
    if gated:
        u = synth.random_bf16(rng, (n, w))
        ref = O.mlp_block_scores_gated(a, u, b)
        got = lemo.lemo_mlp_block_scores_gated(padded(a, ld, 0x7FC0)[:, :w], padded(u, ld, 0x7FC0)[:, :w], b)
    else:
        ref = O.mlp_block_scores(a, b)
        got = lemo.lemo_mlp_block_scores(padded(a, ld, 0x7FC0)[:, :w], b)
    got = got.cpu().numpy()
    assert got.shape == ref.shape
    ok, worst = scores_close(got, ref)
    assert ok and worst < 1e-5, worst


def test_mlp_scores_relu_output_and_determinism():
    """A ReLU output (non-negative, many zeros) at the 7B shape's width; two
    calls give the same bits."""
    rng = np.random.default_rng(12)
    a = synth.random_bf16(rng, (2048, 11008))
    a[(a & 0x8000) != 0] = 0                      # ReLU: negatives to +0
    ref = O.mlp_block_scores(a, 64)
    ad = dev(a)
    g1 = lemo.lemo_mlp_block_scores(ad, 64).cpu().numpy()
    g2 = lemo.lemo_mlp_block_scores(ad, 64).cpu().numpy()
    assert g1.tobytes() == g2.tobytes()
    ok, worst = scores_close(g1, ref)
    assert ok and worst < 1e-5, worst


def test_mlp_scores_full_size():
    """The 7B N=16K MLP activation (16384 x 11008) in the benchmark's launch
    configuration, against the full oracle, plain and gated."""
    w = synth.WORKLOADS["llama2-7b-n16k"]
    say("mlp scores full size")
    rng = np.random.default_rng(13)
    a = synth.random_bf16(rng, (w.n_tokens, w.mlp_width))
    ok, worst = scores_close(lemo.lemo_mlp_block_scores(dev(a), w.block).cpu().numpy(), O.mlp_block_scores(a, w.block))
    assert ok and worst < 1e-5, worst
    u = synth.random_bf16(rng, (w.n_tokens, w.mlp_width))
    ok, worst = scores_close(lemo.lemo_mlp_block_scores_gated(dev(a), dev(u), w.block).cpu().numpy(),
                             O.mlp_block_scores_gated(a, u, w.block))
    assert ok and worst < 1e-5, worst


def test_gather_capacity_overflow():
    n, w, b = 512, 64, 16
    rng = np.random.default_rng(2)
    kept = np.arange(0, 32, 2, dtype=np.int32)          # 16 blocks = 256 rows
    src = synth.random_bf16(rng, (n, w))
    cap = 200                                            # < 256 rows, pad 64 -> 256
    dst_ref, over = O.gather_pad(src, b, kept, kept.size, np.full((cap, w), 0x5A5A, np.uint16), 64)
    assert over
    dstd = dev(np.full((cap, w), 0x5A5A, np.uint16))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    lemo.lemo_gather_pad(dev(src), b, dev(kept), dev(np.array([kept.size], np.int32)), dstd, pad_multiple=64,
                         dev_status=status)
    assert np.array_equal(host_bits(dstd), dst_ref)
    assert int(status.item()) & lemo.DEV_CAP_OVERFLOW


def test_bad_kept_indices_are_skipped_and_flagged():
    n, w, b = 256, 32, 8
    nb = n // b
    rng = np.random.default_rng(4)
    src = synth.random_bf16(rng, (n, w))
    kept = np.array([1, 40, 3, -2], np.int32)            # 40 and -2 are out of range
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dstd = dev(np.full((32, w), 0x5A5A, np.uint16))
    lemo.lemo_gather_pad(dev(src), b, dev(kept), dev(np.array([4], np.int32)), dstd, dev_status=status)
    got = host_bits(dstd)
    assert np.array_equal(got[0:8], src[8:16]) and np.array_equal(got[16:24], src[24:32])
    assert np.all(got[8:16] == 0x5A5A) and np.all(got[24:32] == 0x5A5A)
    assert int(status.item()) & lemo.DEV_BAD_KEPT
    status.zero_()
    res = synth.random_bf16(rng, (n, w))
    resd = dev(res)
    lemo.lemo_scatter_residual(resd, b, dev(kept), dev(np.array([nb + 1], np.int32)), dev(src), dev_status=status)
    assert np.array_equal(host_bits(resd), res) and int(status.item()) & lemo.DEV_BAD_KEPT


@pytest.mark.parametrize("recompute", [False, True], ids=["scatter", "recompute"])
def test_scatter_capped_short_layer_output(recompute):
    """A layer output with fewer rows than the kept rows (built from a gather
    that hit its capacity): the binding passes y's row count, the kept rows
    past it are left out (their residual rows untouched, y never read past its
    end) and the capacity flag is set; an explicit smaller count and a count
    of 0 behave the same way."""
    n, w, b = 512, 64, 16
    rng = np.random.default_rng(21 + recompute)
    kept = np.arange(0, 32, 2, dtype=np.int32)          # 16 blocks = 256 kept rows
    nk = kept.size
    rows = O.kept_token_rows(kept, nk, b)
    res = synth.random_bf16(rng, (n, w))
    kd, nkd = dev(kept), dev(np.array([nk], np.int32))
    oracle = O.residual_recompute if recompute else O.scatter_residual
    call = lemo.lemo_residual_recompute if recompute else lemo.lemo_scatter_residual
    call_capped = lemo.lemo_residual_recompute_capped if recompute else lemo.lemo_scatter_residual_capped
    y_short = synth.random_bf16(rng, (200, w))
    for y_rows, use_capped in ((200, False), (120, True), (0, True)):
        say("scatter capped", recompute, y_rows)
        y_ext = np.zeros((rows.size, w), np.uint16)
        y_ext[:y_rows] = y_short[:y_rows]
        ref = oracle(res, b, kept, nk, y_ext)
        ref[rows[y_rows:]] = res[rows[y_rows:]]           # rows past the layer output: untouched
        resd = dev(res)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        if use_capped:
            call_capped(resd, b, kd, nkd, dev(y_short), y_rows=y_rows, dev_status=status)
        else:
            call(resd, b, kd, nkd, dev(y_short), dev_status=status)
        assert np.array_equal(host_bits(resd), ref)
        assert int(status.item()) == lemo.DEV_CAP_OVERFLOW
    # enough rows: no flag, same as the plain call
    y_full = synth.random_bf16(rng, (rows.size, w))
    resd = dev(res)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    call_capped(resd, b, kd, nkd, dev(y_full), dev_status=status)
    assert np.array_equal(host_bits(resd), oracle(res, b, kept, nk, y_full)) and int(status.item()) == 0


def test_movement_full_size_oracle_mask():
    """The benchmark's Llama2-7B N=16K movement with the oracle's predicted
    mask (MEAN threshold): gather of X and of the MLP activation padded to
    256 rows, then the in-place residual add, all bit-exact."""
    w = synth.WORKLOADS["llama2-7b-n16k"]
    say("movement full size")
    L = synth.make_layer(w.n_tokens, w.d_model, w.block, w.seed, rank=w.rank, mlp_width=w.mlp_width,
                         planted_frac=w.planted_frac)
    _, I_ref, _, _ = O.predict_scores(L.x, L.u_q, L.v_q, L.u_k, L.v_k, w.block)
    _, kept, nk, _ = O.select_mask(I_ref.astype(np.float32), O.SELECT_MEAN)
    R = nk * w.block
    cap = -(-R // 256) * 256
    kd, nkd = dev(kept), dev(np.array([nk], np.int32))
    xd = dev(L.x)
    for src, width in ((L.x, w.d_model), (L.act, w.mlp_width)):
        ref, _ = O.gather_pad(src, w.block, kept, nk, np.zeros((cap, width), np.uint16), 256)
        dstd = torch.empty((cap, width), dtype=torch.int16, device="cuda")
        lemo.lemo_gather_pad(xd if src is L.x else dev(src), w.block, kd, nkd, dstd, pad_multiple=256)
        assert np.array_equal(host_bits(dstd), ref)
    rows = O.kept_token_rows(kept, nk, w.block)
    y = L.y[rows]
    res_ref = O.scatter_residual(L.x, w.block, kept, nk, y)
    lemo.lemo_scatter_residual(xd, w.block, kd, nkd, dev(y))
    assert np.array_equal(host_bits(xd), res_ref)


# -------------------------------------------------------------- pipeline
@pytest.mark.parametrize("path", ["exact", "predictor"])
def test_pipeline_tiny(path):
    """Scores -> select (top-k 50%) -> gather -> scatter on the GPU, chained
    on one stream with no host round trip, against the oracle's own chain."""
    w = synth.WORKLOADS["tiny"]
    L = synth.make_layer(w.n_tokens, w.d_model, w.block, w.seed, n_heads=w.n_heads, head_dim=w.head_dim, rank=64,
                         planted_frac=w.planted_frac)
    k = synth.keep_count(50, w.n_blocks)
    if path == "exact":
        _, I_ref = O.exact_block_scores(L.q, L.k, w.n_heads, w.head_dim, w.block, O.REDUCE_PAPER)
        I, _ = lemo.lemo_block_scores(dev(L.q), dev(L.k), w.n_heads, w.head_dim, w.block, O.REDUCE_PAPER)
    else:
        _, I_ref, _, _ = O.predict_scores(L.x, L.u_q, L.v_q, L.u_k, L.v_k, w.block)
        I, _ = lemo.lemo_predict_scores(dev(L.x), dev(L.u_q), dev(L.v_q), dev(L.u_k), dev(L.v_k), w.block)
    mask_r, kept_r, nk_r, th_r = O.select_mask(I_ref.astype(np.float32), O.SELECT_TOPK, keep_blocks=k)
    mask, kept, nk, th = lemo.lemo_select_mask(I, O.SELECT_TOPK, keep_blocks=k)
    xd = dev(L.x)
    cap = w.n_tokens
    dst = torch.zeros((cap, w.d_model), dtype=torch.int16, device="cuda")
    lemo.lemo_gather_pad(xd, w.block, kept, nk, dst, pad_multiple=256)
    y_full = dev(L.y)
    # the stand-in layer output of dense row p is Y_full[token(p)]: gather it too
    yk = torch.zeros((cap, w.d_model), dtype=torch.int16, device="cuda")
    lemo.lemo_gather_pad(y_full, w.block, kept, nk, yk)
    lemo.lemo_scatter_residual(xd, w.block, kept, nk, yk)
    torch.cuda.synchronize()
    ok, diff = mask_acceptable(mask.cpu().numpy(), mask_r, I_ref, th_r)
    assert ok, diff
    if diff.size == 0:
        ref_dst, _ = O.gather_pad(L.x, w.block, kept_r, nk_r, np.zeros((cap, w.d_model), np.uint16), 256)
        assert np.array_equal(host_bits(dst), ref_dst)
        rows = O.kept_token_rows(kept_r, nk_r, w.block)
        ref_res = O.scatter_residual(L.x, w.block, kept_r, nk_r, L.y[rows])
        assert np.array_equal(host_bits(xd), ref_res)


def test_headline_step_chain():
    """The benchmark's step at the Llama2-7B N=16K shape, chained on the GPU
    exactly as bench.py runs it (predicted scores -> MEAN select -> one
    gather launch for X and the MLP activation, padded to 256 -> in-place
    addition), against the oracle's own chain: scores within the tolerance,
    the mask equal to the oracle's except on near-threshold blocks, and the
    movement bit-exact against the oracle's movement on the GPU's kept list
    (which is the oracle's list whenever the masks agree)."""
    w = synth.WORKLOADS["llama2-7b-n16k"]
    N, d, b, wm = w.n_tokens, w.d_model, w.block, w.mlp_width
    say("headline step chain")
    L = synth.make_layer(N, d, b, w.seed, rank=w.rank, mlp_width=wm, planted_frac=w.planted_frac)
    _, I_ref, _, _ = O.predict_scores(L.x, L.u_q, L.v_q, L.u_k, L.v_k, b)
    mask_r, kept_r, nk_r, th_r = O.select_mask(I_ref.astype(np.float32), O.SELECT_MEAN)
    xd, ad, yd = dev(L.x), dev(L.act), dev(L.y)
    resd = xd.clone()
    cap = N
    xk = torch.empty((cap, d), dtype=torch.int16, device="cuda")
    ak = torch.empty((cap, wm), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    I, _ = lemo.lemo_predict_scores(xd, dev(L.u_q), dev(L.v_q), dev(L.u_k), dev(L.v_k), b)
    mask, kept, nk, th = lemo.lemo_select_mask(I, lemo.SELECT_MEAN, dev_status=status)
    lemo.lemo_gather_pad_multi([xd, ad], [xk, ak], b, kept, nk, pad_multiple=256, dev_status=status)
    lemo.lemo_scatter_residual(resd, b, kept, nk, yd, dev_status=status)
    torch.cuda.synchronize()
    ok, worst = scores_close(I.cpu().numpy(), I_ref)
    assert ok, worst
    ok, diff = mask_acceptable(mask.cpu().numpy(), mask_r, I_ref, th_r)
    assert ok, diff
    assert abs(float(th.item()) - float(th_r)) <= 1e-2 * abs(float(th_r))
    assert int(status.item()) == 0
    nkg = int(nk.item())
    kg = kept.cpu().numpy()[:nkg]
    if diff.size == 0:
        assert nkg == nk_r and np.array_equal(kg, kept_r)
    else:
        say("near-threshold mask difference on blocks", diff)
    R = nkg * b
    Rp = -(-R // 256) * 256
    for src, dst, width in ((L.x, xk, d), (L.act, ak, wm)):
        ref, _ = O.gather_pad(src, b, kg, nkg, np.zeros((Rp, width), np.uint16), 256)
        assert np.array_equal(host_bits(dst)[:Rp], ref)
    assert np.array_equal(host_bits(resd), O.scatter_residual(L.x, b, kg, nkg, L.y[:R]))


def test_pipeline_13b_four_layer_chain():
    """Llama2-13B-shaped stack (N=32768, d=5120, block 128, rank 256), four
    layers chained on the GPU with no host round trip: predicted scores of the
    current residual stream -> top-k select (keep 60/45/35/25 %) -> gather of
    the kept rows (the layer's input) -> in-place add of a fresh stand-in
    layer output.  Each layer is compared with the oracle's own chain; when a
    layer's mask differs only on near-threshold blocks (allowed), both chains
    continue from the oracle's residual."""
    w = synth.WORKLOADS["llama2-13b-n32k-4layer"]
    N, d, b = w.n_tokens, w.d_model, w.block
    nb = N // b
    L0 = synth.make_workload(w, 0)
    res_ref = L0.x.copy()
    resd = dev(L0.x)
    cap = N
    xin = torch.empty((cap, d), dtype=torch.int16, device="cuda")
    yk = torch.empty((cap, d), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for layer, pct in enumerate(w.keep_pct):
        say("13b chain layer", layer, "keep", pct)
        L = L0 if layer == 0 else synth.make_workload(w, layer)
        wts = [L.u_q, L.v_q, L.u_k, L.v_k]
        k = synth.keep_count(pct, nb)
        # oracle chain
        _, I_ref, _, _ = O.predict_scores(res_ref, *wts, b)
        mask_r, kept_r, nk_r, th_r = O.select_mask(I_ref.astype(np.float32), O.SELECT_TOPK, keep_blocks=k)
        rows = O.kept_token_rows(kept_r, nk_r, b)
        xin_ref, _ = O.gather_pad(res_ref, b, kept_r, nk_r, np.zeros((cap, d), np.uint16), 256)
        res_next = O.scatter_residual(res_ref, b, kept_r, nk_r, L.y[rows])
        # GPU chain
        I, _ = lemo.lemo_predict_scores(resd, *[dev(a) for a in wts], b)
        mask, kept, nk, _ = lemo.lemo_select_mask(I, O.SELECT_TOPK, keep_blocks=k, dev_status=status)
        xin.zero_()
        lemo.lemo_gather_pad(resd, b, kept, nk, xin, pad_multiple=256, dev_status=status)
        lemo.lemo_gather_pad(dev(L.y), b, kept, nk, yk, dev_status=status)
        lemo.lemo_scatter_residual(resd, b, kept, nk, yk, dev_status=status)
        torch.cuda.synchronize()
        ok, worst = scores_close(I.cpu().numpy(), I_ref)
        assert ok, (layer, worst)
        assert int(nk.item()) == k == nk_r
        ok, diff = mask_acceptable(mask.cpu().numpy(), mask_r, I_ref, th_r)
        assert ok, (layer, diff)
        assert int(status.item()) == 0
        if diff.size == 0:
            assert np.array_equal(host_bits(xin), xin_ref), layer
            assert np.array_equal(host_bits(resd), res_next), layer
        else:
            say("layer", layer, "near-threshold mask difference on blocks", diff, "- resyncing")
            resd.copy_(dev(res_next))
        res_ref = res_next


def test_scatter_every_bf16_pair():
    """The scatter's arithmetic on all 2^32 pairs of bf16 bit patterns, against
    torch's float32 add followed by its round-to-nearest-even conversion to
    bfloat16 (for finite inputs that is the correctly rounded bf16 sum: two
    bf16 values add exactly in float32 unless one is below half an ulp of the
    other).  NaN results are compared as NaN, whatever their payload."""
    rows, width = 256, 65536
    a = torch.arange(width, dtype=torch.int32, device="cuda").to(torch.int16)
    res = torch.empty((rows, width), dtype=torch.int16, device="cuda")
    y = torch.empty_like(res)
    kept = torch.zeros(1, dtype=torch.int32, device="cuda")
    nk = torch.ones(1, dtype=torch.int32, device="cuda")
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for c in range(0, 65536, rows):
        res.copy_(a.expand(rows, width))
        bvals = torch.arange(c, c + rows, dtype=torch.int32, device="cuda").to(torch.int16)
        y.copy_(bvals[:, None].expand(rows, width))
        ref = (res.view(torch.bfloat16).float() + y.view(torch.bfloat16).float()).to(torch.bfloat16)
        lemo.lemo_scatter_residual(res, rows, kept, nk, y)
        got = res.view(torch.bfloat16)
        both_nan = torch.isnan(got) & torch.isnan(ref)
        bad += ((res != ref.view(torch.int16)) & ~both_nan).sum()
    torch.cuda.synchronize()
    assert int(bad.item()) == 0


# ------------------------------------------------- per-token predictor
def _embeddings_close(got_bits, ref_bits):
    """Both sides round the hidden layer and the output to bf16 from fp32
    values summed in different orders, so an element may land one bf16 step
    away where a value sits near a rounding tie.  Accept: at least 99% of the
    elements bit-identical, every element within 2^-7 of (|ref| + mean |ref|)."""
    got = O.bf16_decode(got_bits)
    ref = O.bf16_decode(ref_bits)
    same = float(np.mean(got_bits == ref_bits))
    tol = 2.0 ** -7 * (np.abs(ref) + np.abs(ref).mean())
    return same >= 0.99 and bool(np.all(np.abs(got - ref) <= tol)), same


TOKEN_SMALL = [
    # (N, d, r)
    (256, 128, 64),
    (320, 192, 128),      # N not a multiple of the 128-row tile
    (200, 256, 256),      # rank 256: two column tiles per product
    (64, 64, 64),         # a single partial tile
    # rank 128, d_model % 256 == 0: the fused one-launch path
    (320, 256, 128),      # 2.5 row tiles, one round of four chunks
    (64, 512, 128),       # a single partial row tile
    (1000, 768, 128),     # 8 row tiles (query/key pairs on one XCD), ragged last tile
    (2048, 1280, 128),    # 16 row tiles, 20 chunks
    (4096, 5120, 128),    # the 13B model width: 80 chunks, 32 row tiles
]


@pytest.mark.parametrize("shape", TOKEN_SMALL, ids=lambda s: "N%d_d%d_r%d" % s)
def test_token_embeddings_small(shape):
    n, d, r = shape
    say("token embeddings", shape)
    x, w = _pred_inputs(n * 7 + d + r, n, d, r)
    ref_q = O.token_embeddings(x, w[0], w[1])
    ref_k = O.token_embeddings(x, w[2], w[3])
    qd, kd = lemo.lemo_token_embeddings(dev(x), *[dev(a) for a in w])
    ok, same = _embeddings_close(host_bits(qd), ref_q)
    assert ok, same
    ok, same = _embeddings_close(host_bits(kd), ref_k)
    assert ok, same


def test_token_embeddings_strided():
    n, d, r = 384, 128, 64
    x, w = _pred_inputs(17, n, d, r)
    xp = padded(x, 200, 0x7FC0)
    out = padded(np.zeros((n, r), np.uint16), 72, 0x1234)
    out2 = padded(np.zeros((n, r), np.uint16), 72, 0x1234)
    lemo.lemo_token_embeddings(xp[:, :d], *[dev(a) for a in w], q_hat=out[:, :r], k_hat=out2[:, :r])
    ok, _ = _embeddings_close(host_bits(out)[:, :r], O.token_embeddings(x, w[0], w[1]))
    assert ok
    assert np.all(host_bits(out)[:, r:] == 0x1234) and np.all(host_bits(out2)[:, r:] == 0x1234)


def test_token_embeddings_fused_strided_no_workspace():
    """The fused path on row strides past the used columns, without a
    workspace (it needs none)."""
    n, d, r = 384, 256, 128
    assert lemo.lemo_token_embeddings_workspace(n, d, r) == 0
    x, w = _pred_inputs(29, n, d, r)
    xp = padded(x, 304, 0x7FC0)
    out = padded(np.zeros((n, r), np.uint16), 136, 0x1234)
    out2 = padded(np.zeros((n, r), np.uint16), 136, 0x1234)
    empty = torch.empty(0, dtype=torch.uint8, device="cuda")
    lemo.lemo_token_embeddings(xp[:, :d], *[dev(a) for a in w], q_hat=out[:, :r], k_hat=out2[:, :r],
                               workspace=empty)
    ok, _ = _embeddings_close(host_bits(out)[:, :r], O.token_embeddings(x, w[0], w[1]))
    assert ok
    ok, _ = _embeddings_close(host_bits(out2)[:, :r], O.token_embeddings(x, w[2], w[3]))
    assert ok
    assert np.all(host_bits(out)[:, r:] == 0x1234) and np.all(host_bits(out2)[:, r:] == 0x1234)


@pytest.mark.parametrize("mode", [O.REDUCE_PAPER, O.REDUCE_HEADMAX], ids=["paper", "headmax"])
def test_token_predictor_scores_small(mode):
    """Per-token embeddings -> exact-score kernel with one head of width r,
    against the oracle's scores of the oracle's embeddings."""
    n, d, r, b = 1024, 256, 128, 64
    x, w = _pred_inputs(5, n, d, r)
    rq, rk = O.token_embeddings(x, w[0], w[1]), O.token_embeddings(x, w[2], w[3])
    M_ref, I_ref = O.exact_block_scores(rq, rk, 1, r, b, mode)
    qd, kd = lemo.lemo_token_embeddings(dev(x), *[dev(a) for a in w])
    M = torch.empty((n // b, n // b), device="cuda")
    I, _ = lemo.lemo_block_scores(qd, kd, 1, r, b, mode, block_scores=M)
    ok, worst = scores_close(I.cpu().numpy(), I_ref)
    assert ok, worst
    ok, worst = scores_close(M.cpu().numpy(), M_ref)
    assert ok, worst


def test_token_predictor_full_size():
    """Llama2-7B shape (N=16384, d=4096, r=128): embeddings against the
    oracle's everywhere, block scores on sampled key-block columns."""
    w = synth.WORKLOADS["llama2-7b-n16k"]
    say("token predictor full size")
    L = synth.make_layer(w.n_tokens, w.d_model, w.block, w.seed, rank=w.rank, planted_frac=w.planted_frac,
                         with_y=False)
    rq = O.token_embeddings(L.x, L.u_q, L.v_q)
    rk = O.token_embeddings(L.x, L.u_k, L.v_k)
    qd, kd = lemo.lemo_token_embeddings(dev(L.x), dev(L.u_q), dev(L.v_q), dev(L.u_k), dev(L.v_k))
    ok, same = _embeddings_close(host_bits(qd), rq)
    assert ok, same
    ok, same = _embeddings_close(host_bits(kd), rk)
    assert ok, same
    I, _ = lemo.lemo_block_scores(qd, kd, 1, w.rank, w.block, O.REDUCE_PAPER)
    Ig = I.cpu().numpy()
    nb = w.n_blocks
    for c in (0, 1, nb // 3, nb - 1):
        ref, _ = O.exact_column_score(rq, rk, 1, w.rank, w.block, O.REDUCE_PAPER, c)
        assert abs(Ig[c] - ref) <= 1e-2 * abs(ref), (c, Ig[c], ref)


def test_token_embeddings_deterministic():
    n, d, r = 512, 256, 128
    x, w = _pred_inputs(23, n, d, r)
    a = lemo.lemo_token_embeddings(dev(x), *[dev(t) for t in w])
    b = lemo.lemo_token_embeddings(dev(x), *[dev(t) for t in w])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------- movement fused into the products
FUSED = [
    # (N, d_in, d_out, block, keep fraction, pad_multiple, cap extra rows)
    (512, 128, 96, 16, 0.5, 64, 8),
    (1024, 256, 256, 64, 0.4, 256, 0),
    (640, 64, 200, 32, 1.0, 1, 0),        # keep all, ragged d_out
    (512, 128, 128, 64, 0.0, 64, 3),      # keep none
    # output widths that are a multiple of 256 run the ping-pong form
    (1024, 512, 512, 32, 0.3, 64, 5),
    (768, 256, 256, 64, 0.0, 64, 3),      # keep none
    (2048, 128, 768, 16, 0.7, 256, 0),    # three column tiles, two reduction chunks
]


def _fused_case(case, seed):
    n, din, dout, b, frac, pad, extra = case
    rng = np.random.default_rng(seed)
    nb = n // b
    kept = _kept_from_mask(rng, nb, frac)
    x = synth.random_bf16(rng, (n, din))
    w = synth.random_bf16(rng, (dout, din), 1.0 / math.sqrt(din))
    R = kept.size * b
    cap = max(1, -(-R // pad) * pad + extra)
    return n, din, dout, b, pad, kept, x, w, R, cap, rng


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "N%d_in%d_out%d_b%d_keep%.1f" % c[:5])
def test_gather_linear(case):
    n, din, dout, b, pad, kept, x, w, R, cap, rng = _fused_case(case, 31)
    say("gather_linear", case)
    sentinel = np.full((cap, dout), 0x5A5A, np.uint16)
    ref, over = O.gather_linear(x, b, kept, kept.size, w, sentinel, pad)
    kd = dev(kept) if kept.size else torch.zeros(1, dtype=torch.int32, device="cuda")
    nkd = dev(np.array([kept.size], np.int32))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    yd = dev(sentinel)
    lemo.lemo_gather_linear(dev(x), b, kd, nkd, dev(w), yd, pad_multiple=pad, dev_status=status)
    got = host_bits(yd)
    if R:
        ok, same = _embeddings_close(got[:R], ref[:R])
        assert ok, same
    assert np.array_equal(got[R:], ref[R:])          # zero padding and untouched rows, bit-exact
    assert int(status.item()) == 0 and not over
    # the gather in the operand prologue equals gathering first (same product)
    if R:
        xg = torch.zeros((cap, din), dtype=torch.int16, device="cuda")
        lemo.lemo_gather_pad(dev(x), b, kd, nkd, xg)
        ident = dev(np.arange(cap // b + 1, dtype=np.int32))
        y2 = dev(sentinel)
        lemo.lemo_gather_linear(xg, b, ident, nkd, dev(w), y2, pad_multiple=pad, n_tokens=(cap // b) * b)
        assert torch.equal(y2[:R], yd[:R])


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "N%d_in%d_out%d_b%d_keep%.1f" % c[:5])
def test_linear_scatter(case):
    n, din, dout, b, pad, kept, x, w, R, cap, rng = _fused_case(case, 37)
    say("linear_scatter", case)
    a = synth.random_bf16(rng, (max(R, 1), din))
    res = synth.random_bf16(rng, (n, dout))
    ref = O.linear_scatter(a, w, res, b, kept, kept.size)
    kd = dev(kept) if kept.size else torch.zeros(1, dtype=torch.int32, device="cuda")
    nkd = dev(np.array([kept.size], np.int32))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rd = dev(res)
    lemo.lemo_linear_scatter(dev(a), dev(w), rd, b, kd, nkd, dev_status=status)
    got = host_bits(rd)
    rows = O.kept_token_rows(kept, kept.size, b)
    dropped = np.setdiff1d(np.arange(n), rows)
    assert np.array_equal(got[dropped], res[dropped])     # untouched rows, bit-exact
    if R:
        ok, same = _embeddings_close(got[rows], ref[rows])
        assert ok, same
    assert int(status.item()) == 0
    # the addition in the epilogue equals the product followed by the plain scatter
    if R:
        ident = dev(np.arange(R // b, dtype=np.int32))
        y = torch.zeros((R, dout), dtype=torch.int16, device="cuda")
        lemo.lemo_gather_linear(dev(a[:R]), b, ident, nkd, dev(w), y)
        r2 = dev(res)
        lemo.lemo_scatter_residual(r2, b, kd, nkd, y)
        assert torch.equal(r2, rd)


@pytest.mark.parametrize("din,dout", [(64, 64), (128, 256)], ids=["tile", "pingpong"])
def test_fused_bad_kept_and_capacity(din, dout):
    n, b = 256, 16
    rng = np.random.default_rng(41)
    x = synth.random_bf16(rng, (n, din))
    w = synth.random_bf16(rng, (dout, din), 0.125)
    kept = np.array([1, 40, 3], np.int32)                  # 40 is out of range
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = dev(np.full((48, dout), 0x5A5A, np.uint16))
    lemo.lemo_gather_linear(dev(x), b, dev(kept), dev(np.array([3], np.int32)), dev(w), y, dev_status=status)
    got = host_bits(y)
    assert np.all(got[16:32] == 0x5A5A)                     # the invalid block's rows are skipped
    ref = O.linear_bf16(x[16:32], w)
    ok, _ = _embeddings_close(got[0:16], ref)
    assert ok and int(status.item()) & lemo.DEV_BAD_KEPT
    status.zero_()
    y = dev(np.full((20, dout), 0x5A5A, np.uint16))          # 2 kept blocks = 32 rows > 20
    lemo.lemo_gather_linear(dev(x), b, dev(np.array([2, 5], np.int32)), dev(np.array([2], np.int32)), dev(w), y,
                            pad_multiple=1, dev_status=status)
    assert int(status.item()) & lemo.DEV_CAP_OVERFLOW
    ok, _ = _embeddings_close(host_bits(y), O.linear_bf16(np.concatenate([x[32:48], x[80:84]]), w))
    assert ok


def test_fused_full_size_sampled():
    """Llama2-7B shape: the query projection (4096 x 4096) on the kept rows of
    the oracle's mask with the gather fused in, and the output projection
    added back into the residual stream; rows checked on a sample."""
    w = synth.WORKLOADS["llama2-7b-n16k"]
    say("fused full size")
    L = synth.make_layer(w.n_tokens, w.d_model, w.block, w.seed, rank=w.rank, planted_frac=w.planted_frac)
    _, I_ref, _, _ = O.predict_scores(L.x, L.u_q, L.v_q, L.u_k, L.v_k, w.block)
    _, kept, nk, _ = O.select_mask(I_ref.astype(np.float32), O.SELECT_MEAN)
    R = nk * w.block
    rng = np.random.default_rng(43)
    wq = synth.random_bf16(rng, (w.d_model, w.d_model), 1.0 / math.sqrt(w.d_model))
    kd, nkd = dev(kept), dev(np.array([nk], np.int32))
    cap = -(-R // 256) * 256
    y = torch.empty((cap, w.d_model), dtype=torch.int16, device="cuda")
    lemo.lemo_gather_linear(dev(L.x), w.block, kd, nkd, dev(wq), y, pad_multiple=256)
    rows = O.kept_token_rows(kept, nk, w.block)
    sample = np.sort(rng.choice(R, size=64, replace=False))
    got = host_bits(y)
    ok, same = _embeddings_close(got[sample], O.linear_bf16(L.x[rows[sample]], wq))
    assert ok, same
    assert np.all(got[R:] == 0)
    # the output projection of a stand-in attention output (seeded, R rows)
    a = synth.random_bf16(rng, (R, w.d_model))
    resd = dev(L.x)
    lemo.lemo_linear_scatter(dev(a), dev(wq), resd, w.block, kd, nkd)
    res = host_bits(resd)
    dropped = np.setdiff1d(np.arange(w.n_tokens), rows)
    assert np.array_equal(res[dropped], L.x[dropped])
    ref = O.scatter_residual(L.x[rows[sample]], 1, np.arange(sample.size, dtype=np.int32), sample.size,
                             O.linear_bf16(a[sample], wq))
    ok, same = _embeddings_close(res[rows[sample]], ref)
    assert ok, same


def test_binding_rejects_bad_buffers():
    """Buffers the library would write through blindly are refused before any
    launch: host memory, a wrong dtype, too few elements.  A float32
    workspace is counted in bytes."""
    n, h, hd, b = 256, 2, 64, 64
    rng = np.random.default_rng(11)
    qn, kn = synth.random_bf16(rng, (n, h * hd)), synth.random_bf16(rng, (n, h * hd))
    q, k = dev(qn), dev(kn)
    nb = n // b
    with pytest.raises(ValueError, match="tensor on"):
        lemo.lemo_block_scores(q, k, h, hd, b, scores=torch.zeros(nb))
    with pytest.raises(TypeError):
        lemo.lemo_block_scores(q, k, h, hd, b, scores=torch.zeros(nb, dtype=torch.float64, device="cuda"))
    with pytest.raises(ValueError, match="needed"):
        lemo.lemo_block_scores(q, k, h, hd, b, block_scores=torch.zeros(nb, nb - 1, device="cuda"))
    with pytest.raises(ValueError, match="needed"):
        lemo.lemo_select_mask(torch.zeros(nb, device="cuda"), lemo.SELECT_MEAN,
                              kept_blocks=torch.zeros(nb - 1, dtype=torch.int32, device="cuda"))
    # the heads must lie inside each operand's columns: a view of the last
    # half of a wider matrix has a row stride that covers them, its columns do not
    wide = dev(synth.random_bf16(rng, (n, 2 * h * hd)))
    with pytest.raises(ValueError, match="needed"):
        lemo.lemo_block_scores(wide[:, h * hd + 8:], wide[:, :h * hd], h, hd, b)
    with pytest.raises(ValueError, match="columns needed"):
        lemo.lemo_block_scores_batched(wide[:, h * hd + 8:], wide[:, :h * hd], h, hd, b)
    # the workspace holds nb*nb floats: a float32 tensor of that many elements suffices
    ws = torch.empty(lemo.lemo_block_scores_workspace(n, b) // 4, dtype=torch.float32, device="cuda")
    I, _ = lemo.lemo_block_scores(q, k, h, hd, b, workspace=ws)
    M_ref, I_ref = O.exact_block_scores(qn, kn, h, hd, b, O.REDUCE_PAPER)
    ok, worst = scores_close(I.cpu().numpy(), I_ref)
    assert ok, worst


def test_concurrent_streams_match_sequential():
    """Calls are thread-safe: two host threads, each on its own stream, run the
    exact scores, the predictor, select and gather on their own buffers while
    the other does the same; every output equals, bit for bit, the output of
    the same calls made one after the other."""
    import threading
    n, h, hd, b, d, r = 1024, 4, 128, 64, 512, 64
    nb = n // b

    def inputs(seed):
        q, k = rand_qk(seed, n, h, hd)
        x, w = _pred_inputs(seed + 1, n, d, r)
        return [dev(q), dev(k), dev(x)] + [dev(a) for a in w]

    def run(t):
        q, k, x, uq, vq, uk, vk = t
        I, _ = lemo.lemo_block_scores(q, k, h, hd, b)
        Ip, _ = lemo.lemo_predict_scores(x, uq, vq, uk, vk, b)
        mask, kept, nk, _ = lemo.lemo_select_mask(Ip, lemo.SELECT_TOPK, keep_blocks=nb // 2)
        dst = torch.zeros((n, d), dtype=torch.int16, device="cuda")
        lemo.lemo_gather_pad(x, b, kept, nk, dst, pad_multiple=64)
        return [I, Ip, mask, kept, dst]

    ins = [inputs(101), inputs(202)]
    ref = [run(t) for t in ins]
    torch.cuda.synchronize()
    ref = [[a.cpu() for a in r_] for r_ in ref]

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    barrier = threading.Barrier(2)

    def worker(i):
        with torch.cuda.stream(streams[i]):
            barrier.wait()
            out = None
            for _ in range(4):
                out = run(ins[i])
            streams[i].synchronize()
            got[i] = [a.cpu() for a in out]

    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    for i in range(2):
        for a, r_ in zip(got[i], ref[i]):
            assert torch.equal(a, r_)


def test_step_in_hip_graph_replays_bit_exact():
    """One step of the path (exact scores, predictor, mean select, gather of
    two tensors, in-place residual add) captured in a HIP graph: the library
    only launches kernels (no allocation, memset or synchronisation inside a
    call), so each replay, with eager work and a synchronisation between
    replays (the in-place residual is restored), equals the eager step bit for
    bit."""
    n, h, hd, b, d, r, wa = 1024, 4, 128, 64, 512, 64, 1024
    nb = n // b
    q, k = rand_qk(303, n, h, hd)
    x, w = _pred_inputs(304, n, d, r)
    rng = np.random.default_rng(305)
    act = synth.random_bf16(rng, (n, wa))
    y = synth.random_bf16(rng, (n, d))
    qd, kd, xd, actd, yd = dev(q), dev(k), dev(x), dev(act), dev(y)
    wd = [dev(a) for a in w]
    res0 = dev(x)
    bufs = dict(
        I=torch.empty(nb, device="cuda"), Ip=torch.empty(nb, device="cuda"),
        ws=torch.empty(lemo.lemo_block_scores_workspace(n, b), dtype=torch.uint8, device="cuda"),
        wsp=torch.empty(lemo.lemo_predict_scores_workspace(n, d, b, r), dtype=torch.uint8, device="cuda"),
        mask=torch.empty(nb, dtype=torch.uint8, device="cuda"), kept=torch.empty(nb, dtype=torch.int32, device="cuda"),
        nk=torch.empty(1, dtype=torch.int32, device="cuda"), th=torch.empty(1, device="cuda"),
        xk=torch.zeros((n, d), dtype=torch.int16, device="cuda"),
        ak=torch.zeros((n, wa), dtype=torch.int16, device="cuda"),
        res=res0.clone())

    def step(B):
        lemo.lemo_block_scores(qd, kd, h, hd, b, scores=B["I"], workspace=B["ws"])
        lemo.lemo_predict_scores(xd, *wd, b, scores=B["Ip"], workspace=B["wsp"])
        lemo.lemo_select_mask(B["Ip"], lemo.SELECT_MEAN, mask=B["mask"], kept_blocks=B["kept"], n_kept=B["nk"],
                              threshold_used=B["th"])
        lemo.lemo_gather_pad(xd, b, B["kept"], B["nk"], B["xk"], pad_multiple=64)
        lemo.lemo_gather_pad(actd, b, B["kept"], B["nk"], B["ak"], pad_multiple=64)
        lemo.lemo_scatter_residual(B["res"], b, B["kept"], B["nk"], yd)

    eager = {kk: v.clone() for kk, v in bufs.items()}
    eager["res"] = res0.clone()
    step(eager)
    torch.cuda.synchronize()
    names = ("I", "Ip", "mask", "kept", "nk", "th", "xk", "ak", "res")
    want = {kk: eager[kk].cpu() for kk in names}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):               # warm the binding's code paths off the capture
        step(bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    bufs["res"].copy_(res0)
    with torch.cuda.graph(g):
        step(bufs)
    for rep in range(3):
        bufs["res"].copy_(res0)                 # eager work between replays
        for kk in ("I", "Ip", "xk", "ak"):
            bufs[kk].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for kk in names:
            assert torch.equal(bufs[kk].cpu(), want[kk]), (rep, kk)
