"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any launch (so these run without a GPU: the
pointers below are never dereferenced)."""
import ctypes

import pytest

from contextual_token_sparsity_amd import lemo

OK, INVALID, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4
P = ctypes.c_void_p(0x100000)      # fake, 16-byte aligned, never touched
P2 = ctypes.c_void_p(0x100002)     # misaligned
NULL = None


@pytest.fixture(scope="module")
def L():
    return lemo.lib()


def test_exports_every_declared_symbol(L):
    names = lemo.declared_symbols()
    assert len(names) == 24
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings(L):
    assert L.lemo_version() == 100
    for s, text in ((0, "ok"), (1, "invalid argument"), (4, "workspace missing or too small")):
        assert lemo.lemo_status_string(s) == text
    assert lemo.lemo_status_string(99) == "unknown status"


def test_workspace_queries(L):
    assert L.lemo_block_scores_workspace(16384, 64) == 256 * 256 * 4
    assert L.lemo_block_scores_workspace(100, 64) == 0
    ws = L.lemo_predict_scores_workspace(16384, 4096, 64, 128)
    # xbar (2 MiB) + split-K partials of the hidden layer + q_hat/k_hat; M_hat is not stored
    assert ws >= 256 * 4096 * 2 + 256 * 256 * 4 + 2 * 256 * 128 * 4
    assert ws < 256 * 4096 * 2 + 16 * 256 * 256 * 4 + 2 * 256 * 128 * 4
    assert L.lemo_predict_scores_workspace(0, 4096, 64, 128) == 0


def bs(L, q=P, k=P, n=1024, h=4, hd=128, ldq=512, ldk=512, b=64, mode=0, M=NULL, I=P, ws=NULL, wsb=0):
    return L.lemo_block_scores(q, k, n, h, hd, ldq, ldk, b, mode, M, I, ws, wsb, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(I=NULL), INVALID), (dict(q=NULL), INVALID), (dict(n=1000), INVALID), (dict(n=0), INVALID),
    (dict(h=0), INVALID), (dict(mode=2), INVALID), (dict(ldq=256), INVALID),
    (dict(hd=96, ldq=384, ldk=384), UNSUP), (dict(b=16), UNSUP), (dict(b=256), UNSUP),
    (dict(mode=1, h=200, hd=64, ldq=12800, ldk=12800), UNSUP),
    (dict(q=P2), ALIGN), (dict(ldk=516), ALIGN),
    (dict(M=NULL, ws=NULL), WS), (dict(M=NULL, ws=P, wsb=100), WS),
])
def test_block_scores_rejects(L, kw, status):
    assert bs(L, **kw) == status
    assert lemo.lemo_last_error()


def test_block_scores_caps_tokens(L):
    assert bs(L, n=(1 << 22) + 64) == UNSUP


def bsb(L, q=P, k=P, B=2, n=1000, h=4, hd=128, ldq=512, ldk=512, sq=1000 * 512, sk=1000 * 512, b=64, mode=0,
        flags=1, M=P, I=P, ws=NULL, wsb=0):
    return L.lemo_block_scores_batched(q, k, B, n, h, hd, ldq, ldk, sq, sk, b, mode, flags, M, I, ws, wsb, NULL)


def test_batched_workspace_query(L):
    # ragged: 1000 tokens in blocks of 64 -> 16 blocks
    assert L.lemo_block_scores_batched_workspace(3, 1000, 64) == 3 * 16 * 16 * 4
    assert L.lemo_block_scores_batched_workspace(1, 16384, 64) == L.lemo_block_scores_workspace(16384, 64)
    assert L.lemo_block_scores_batched_workspace(0, 1000, 64) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(I=NULL), INVALID), (dict(q=NULL), INVALID), (dict(B=0), INVALID), (dict(n=0), INVALID),
    (dict(flags=2), INVALID), (dict(flags=-1), INVALID), (dict(mode=3), INVALID), (dict(ldq=256), INVALID),
    (dict(sq=999 * 512), INVALID), (dict(sk=-512), INVALID),
    (dict(B=65536), UNSUP), (dict(hd=96, ldq=384, ldk=384, sq=384000, sk=384000), UNSUP), (dict(b=256), UNSUP),
    (dict(n=(1 << 22) + 1, sq=1 << 32, sk=1 << 32), UNSUP),
    (dict(B=3, n=1 << 22, sq=1 << 32, sk=1 << 32, flags=0), UNSUP),   # 3 x 2^30 tiles in one launch
    (dict(q=P2), ALIGN), (dict(sq=1000 * 512 + 4), ALIGN),
    (dict(M=NULL), WS), (dict(M=NULL, ws=P, wsb=100), WS),
])
def test_block_scores_batched_rejects(L, kw, status):
    assert bsb(L, **kw) == status
    assert lemo.lemo_last_error()


def test_block_scores_batched_one_sequence_ignores_strides(L):
    # n_batch == 1: strides that would be rejected for a batch are not looked
    # at, so validation runs on to the (missing) workspace
    assert bsb(L, B=1, sq=3, sk=-5, M=NULL) == WS
    assert bsb(L, B=2, sq=3, sk=-5, M=NULL) == ALIGN


def ps(L, x=P, n=1024, d=512, ldx=512, b=64, r=64, M=NULL, I=P, ws=P, wsb=1 << 30):
    return L.lemo_predict_scores(x, n, d, ldx, b, P, P, P, P, r, M, I, ws, wsb, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(I=NULL), INVALID), (dict(x=NULL), INVALID), (dict(r=0), INVALID),
    (dict(ldx=256), INVALID), (dict(b=3, n=999), UNSUP), (dict(b=512, n=1024), UNSUP), (dict(b=1), UNSUP),
    (dict(d=100, ldx=104), UNSUP), (dict(r=48), UNSUP), (dict(r=288), UNSUP),
    (dict(x=P2), ALIGN), (dict(ldx=520 + 4), ALIGN),
    (dict(ws=NULL), WS), (dict(wsb=1000), WS),
])
def test_predict_rejects(L, kw, status):
    assert ps(L, **kw) == status


def te(L, x=P, n=1024, d=512, ldx=512, uq=P, r=128, q=P, k=P, ldo=128, ws=P, wsb=1 << 30):
    return L.lemo_token_embeddings(x, n, d, ldx, uq, P, P, P, r, q, k, ldo, ws, wsb, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(x=NULL), INVALID), (dict(uq=NULL), INVALID), (dict(q=NULL), INVALID), (dict(k=NULL), INVALID),
    (dict(n=0), INVALID), (dict(r=0), INVALID), (dict(ldx=256), INVALID), (dict(ldo=64), INVALID),
    (dict(d=100, ldx=104), UNSUP), (dict(r=96, ldo=96), UNSUP), (dict(r=320, ldo=320), UNSUP),
    (dict(x=P2), ALIGN), (dict(uq=P2), ALIGN), (dict(q=P2), ALIGN), (dict(ldo=132), ALIGN),
    # rank 64 needs a workspace (rank 128 at d_model 512 runs fused, without one)
    (dict(ws=NULL, r=64, ldo=64), WS), (dict(wsb=1000, r=64, ldo=64), WS), (dict(ws=P2, r=64, ldo=64), ALIGN),
])
def test_token_embeddings_rejects(L, kw, status):
    assert te(L, **kw) == status
    assert lemo.lemo_last_error()


def test_token_embeddings_workspace(L):
    # rank 128 with d_model % 256 == 0: the fused launch needs no workspace
    assert L.lemo_token_embeddings_workspace(16384, 4096, 128) == 0
    assert L.lemo_token_embeddings_workspace(32768, 5120, 128) == 0
    # otherwise [U_q | U_k]^T + V_q^T, V_k^T + hidden [N][2r], each 256-byte aligned
    assert L.lemo_token_embeddings_workspace(16384, 4096, 256) == 512 * 4096 * 2 + 2 * 256 * 256 * 2 + 16384 * 512 * 2
    assert L.lemo_token_embeddings_workspace(16384, 4160, 128) == 256 * 4160 * 2 + 2 * 128 * 128 * 2 + 16384 * 256 * 2
    assert L.lemo_token_embeddings_workspace(0, 4096, 128) == 0


def gl(L, x=P, n=1024, din=512, ldx=512, b=64, kept=P, nk=P, w=P, dout=256, ldw=512, y=P, ldy=256, cap=1024,
       pad=256):
    return L.lemo_gather_linear(x, n, din, ldx, b, kept, nk, w, dout, ldw, y, ldy, cap, pad, NULL, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(kept=NULL), INVALID), (dict(nk=NULL), INVALID), (dict(x=NULL), INVALID), (dict(w=NULL), INVALID),
    (dict(y=NULL), INVALID), (dict(cap=0), INVALID), (dict(pad=0), INVALID),
    (dict(dout=0), INVALID), (dict(ldw=256), INVALID), (dict(ldy=128), INVALID),
    (dict(din=96, ldx=96, ldw=96), UNSUP), (dict(x=P2), ALIGN), (dict(w=P2), ALIGN), (dict(ldy=260), ALIGN),
    (dict(dout=12), ALIGN),
])
def test_gather_linear_rejects(L, kw, status):
    assert gl(L, **kw) == status
    assert lemo.lemo_last_error()


def ls(L, a=P, din=512, lda=512, cap=1024, w=P, dout=256, ldw=512, res=P, n=1024, ldr=256, b=64, kept=P, nk=P):
    return L.lemo_linear_scatter(a, din, lda, cap, w, dout, ldw, res, n, ldr, b, kept, nk, NULL, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(kept=NULL), INVALID), (dict(nk=NULL), INVALID), (dict(a=NULL), INVALID), (dict(w=NULL), INVALID),
    (dict(res=NULL), INVALID), (dict(cap=0), INVALID), (dict(b=0), INVALID),
    (dict(lda=256), INVALID), (dict(ldr=128), INVALID),
    (dict(din=96, lda=96, ldw=96), UNSUP), (dict(a=P2), ALIGN), (dict(res=P2), ALIGN), (dict(ldr=260), ALIGN),
    (dict(dout=12), ALIGN),
])
def test_linear_scatter_rejects(L, kw, status):
    assert ls(L, **kw) == status
    assert lemo.lemo_last_error()


def sel(L, s=P, nb=256, mode=1, th=0.0, k=10, mask=P, kept=P, nk=P):
    return L.lemo_select_mask(s, nb, mode, th, k, mask, kept, nk, NULL, NULL, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(s=NULL), INVALID), (dict(mask=NULL), INVALID), (dict(kept=NULL), INVALID), (dict(nk=NULL), INVALID),
    (dict(nb=0), INVALID), (dict(nb=8193), UNSUP), (dict(mode=3), INVALID), (dict(k=257), INVALID),
    (dict(k=-1), INVALID),
])
def test_select_rejects(L, kw, status):
    assert sel(L, **kw) == status


def ga(L, src=P, n=1024, w=512, lds=512, b=64, kept=P, nk=P, dst=P, ldd=512, cap=1024, pad=256):
    return L.lemo_gather_pad(src, n, w, lds, b, kept, nk, dst, ldd, cap, pad, NULL, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(kept=NULL), INVALID), (dict(nk=NULL), INVALID), (dict(src=NULL), INVALID), (dict(dst=NULL), INVALID),
    (dict(cap=0), INVALID), (dict(pad=0), INVALID), (dict(ldd=256), INVALID),
    (dict(w=12, lds=16, ldd=16), ALIGN), (dict(dst=P2), ALIGN), (dict(lds=520 + 2), ALIGN),
])
def test_gather_rejects(L, kw, status):
    assert ga(L, **kw) == status


def sc(L, res=P, n=1024, w=512, ldr=512, b=64, kept=P, nk=P, y=P, ldy=512):
    return L.lemo_scatter_residual(res, n, w, ldr, b, kept, nk, y, ldy, NULL, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(kept=NULL), INVALID), (dict(res=NULL), INVALID), (dict(y=NULL), INVALID),
    (dict(b=0), INVALID), (dict(ldy=256), INVALID), (dict(w=4, ldr=8, ldy=8), ALIGN), (dict(y=P2), ALIGN),
])
def test_scatter_rejects(L, kw, status):
    assert sc(L, **kw) == status


def rc(L, res=P, n=1024, w=64, ldr=64, b=64, kept=P, nk=P, y=P, ldy=64):
    return L.lemo_residual_recompute(res, n, w, ldr, b, kept, nk, y, ldy, NULL, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(kept=NULL), INVALID), (dict(nk=NULL), INVALID), (dict(res=NULL), INVALID), (dict(y=NULL), INVALID),
    (dict(n=0), INVALID), (dict(ldr=32), INVALID),
    (dict(w=60, ldr=64, ldy=64), ALIGN), (dict(res=P2), ALIGN), (dict(ldy=68), ALIGN),
])
def test_residual_recompute_rejects(L, kw, status):
    assert rc(L, **kw) == status
    assert lemo.lemo_last_error()


def scc(L, res=P, n=1024, w=512, ldr=512, b=64, kept=P, nk=P, y=P, ldy=512, rows=64, recompute=False):
    fn = L.lemo_residual_recompute_capped if recompute else L.lemo_scatter_residual_capped
    return fn(res, n, w, ldr, b, kept, nk, y, ldy, rows, NULL, NULL)


@pytest.mark.parametrize("recompute", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(kept=NULL), INVALID), (dict(nk=NULL), INVALID), (dict(res=NULL), INVALID), (dict(y=NULL), INVALID),
    (dict(rows=-1), INVALID), (dict(b=0), INVALID), (dict(ldy=256), INVALID),
    (dict(w=4, ldr=8, ldy=8), ALIGN), (dict(y=P2), ALIGN), (dict(res=P2), ALIGN),
])
def test_scatter_capped_rejects(L, kw, status, recompute):
    """The capped scatter and recompute (y's row count as an argument) check
    what the plain calls check, and refuse a negative row count."""
    assert scc(L, recompute=recompute, **kw) == status
    assert lemo.lemo_last_error()
    if kw == dict(rows=-1):
        assert "y_rows" in lemo.lemo_last_error()


def gm(L, n_src=2, srcs=(P, P), widths=(512, 64), lds=(512, 64), dsts=(P, P), ldd=(512, 64), n=1024, b=64,
       kept=P, nk=P, cap=256, pad=1):
    k = 2
    arr = lambda t, vals: (t * k)(*vals) if vals is not None else None
    return L.lemo_gather_pad_multi(n_src, arr(ctypes.c_void_p, srcs), arr(ctypes.c_int, widths),
                                   arr(ctypes.c_int, lds), arr(ctypes.c_void_p, dsts), arr(ctypes.c_int, ldd), n, b,
                                   kept, nk, cap, pad, NULL, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(n_src=0), INVALID), (dict(n_src=5), INVALID), (dict(srcs=None), INVALID), (dict(kept=NULL), INVALID),
    (dict(cap=0), INVALID), (dict(pad=0), INVALID), (dict(srcs=(P, NULL)), INVALID), (dict(dsts=(NULL, P)), INVALID),
    (dict(widths=(512, 0)), INVALID), (dict(ldd=(512, 32)), INVALID),
    (dict(widths=(512, 60), lds=(512, 64), ldd=(512, 64)), ALIGN), (dict(dsts=(P, P2)), ALIGN),
    (dict(lds=(516, 64)), ALIGN),
])
def test_gather_multi_rejects(L, kw, status):
    """The multi-source gather checks every source and destination as the
    single gather does, and its source count (1..4)."""
    assert gm(L, **kw) == status
    assert lemo.lemo_last_error()


def test_predict_noalloc_checks(L):
    """The no-allocation predictor checks what lemo_predict_scores checks and
    refuses shapes whose scratch would exceed its fixed 16 MiB, before any
    device call."""
    call = lambda n=16384, d=4096, b=64, r=128, x=P, I=P: L.lemo_predict_scores_noalloc(
        x, n, d, d, b, P, P, P, P, r, NULL, I, NULL)
    assert call(x=NULL) == INVALID
    assert call(I=NULL) == INVALID
    assert call(r=48) == UNSUP
    assert call(b=3) == UNSUP
    assert call(n=4096 * 64, d=4096) == UNSUP               # 4096 blocks: x-bar alone is 32 MiB
    assert "16777216" in lemo.lemo_last_error()
    assert L.lemo_predict_scores_workspace(16384, 4096, 64, 128) <= 16 << 20
    assert L.lemo_predict_scores_workspace(32768, 5120, 128, 256) <= 16 << 20


def test_fused_tile_limit(L):
    """The fused products launch one 512-thread workgroup per 256 x 256 output
    tile, at most (2^31 - 1) / 512 of them.  Just past that is refused; just
    inside it passes the tile check (and these calls stop at the NULL output
    checked next), although the old 128 x 128 count refused it."""
    lim = ((1 << 31) - 1) // 512
    assert lim == 4194303
    ok_cap, bad_cap = lim * 256, (lim + 1) * 256
    assert L.lemo_gather_linear(P, 1024, 64, 64, 64, P, P, P, 256, 64, P, 256, bad_cap, 1, NULL, NULL) == UNSUP
    assert "256 x 256" in lemo.lemo_last_error()
    assert L.lemo_gather_linear(P, 1024, 64, 64, 64, P, P, P, 256, 64, NULL, 256, ok_cap, 1, NULL, NULL) == INVALID
    assert "y is NULL" in lemo.lemo_last_error()
    # the scatter's product covers min(cap_rows, n_tokens) rows
    rows = (1 << 25) - 1                      # ceil(rows / 256) = 131072 row tiles
    assert L.lemo_linear_scatter(P, 64, 64, rows, P, 8192, 64, P, rows, 8192, 64, P, P, NULL, NULL) == UNSUP
    assert L.lemo_linear_scatter(P, 64, 64, rows, P, 7936, 64, NULL, rows, 8192, 64, P, P, NULL, NULL) == INVALID
    assert "residual is NULL" in lemo.lemo_last_error()
    assert L.lemo_linear_scatter(P, 64, 64, rows, P, 8192, 64, NULL, 1024, 8192, 64, P, P, NULL, NULL) == INVALID


def test_mlp_workspace_query(L):
    # 16384 tokens in blocks of 64 -> 256 blocks; 11008 channels -> 6 chunks of 2048
    assert L.lemo_mlp_block_scores_workspace(16384, 11008, 64) == 256 * 6 * 4
    assert L.lemo_mlp_block_scores_workspace(1000, 200, 64) == 256      # 16 x 1 x 4 B, rounded up to 256
    assert L.lemo_mlp_block_scores_workspace(0, 200, 64) == 0


def ms(L, a=P, n=1000, w=200, lda=200, b=64, I=P, ws=P, wsb=1 << 20, up=None, ldu=200):
    if up is None:
        return L.lemo_mlp_block_scores(a, n, w, lda, b, I, ws, wsb, NULL)
    return L.lemo_mlp_block_scores_gated(a, up, n, w, lda, ldu, b, I, ws, wsb, NULL)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(I=NULL), INVALID), (dict(a=NULL), INVALID), (dict(n=0), INVALID), (dict(b=0), INVALID),
    (dict(w=0), INVALID), (dict(lda=192), INVALID),
    (dict(w=196, lda=200), ALIGN), (dict(a=P2), ALIGN), (dict(lda=204), ALIGN), (dict(ws=P2), ALIGN),
    (dict(ws=NULL), WS), (dict(wsb=100), WS),
])
def test_mlp_scores_rejects(L, kw, status, gated):
    kw = dict(kw)
    if gated:
        kw.setdefault("up", P)
    assert ms(L, **kw) == status
    assert lemo.lemo_last_error()


def test_mlp_gated_rejects_bad_up(L):
    assert L.lemo_mlp_block_scores_gated(P, NULL, 1000, 200, 200, 200, 64, P, P, 1 << 20, NULL) == INVALID
    assert ms(L, up=P2) == ALIGN
    assert ms(L, up=P, ldu=100) == INVALID


def test_ragged_sequences_pass_validation(L):
    """n_tokens need not be a multiple of block on the predictor and movement
    calls (the last block is short): such calls get past every check and stop
    at the first deliberately missing argument."""
    assert ps(L, n=1000, ws=NULL) == WS
    assert L.lemo_predict_scores_workspace(1000, 512, 64, 64) == L.lemo_predict_scores_workspace(1024, 512, 64, 64)
    assert L.lemo_gather_pad(P, 1000, 64, 64, 64, P, P, NULL, 64, 100, 1, NULL, NULL) == INVALID   # dst NULL
    assert L.lemo_scatter_residual(P, 1000, 64, 64, 64, P, P, NULL, 64, NULL, NULL) == INVALID      # y NULL
    assert L.lemo_residual_recompute(P, 1000, 64, 64, 64, P, P, NULL, 64, NULL, NULL) == INVALID    # y NULL
    assert "multiple of block" not in lemo.lemo_last_error()


def test_row_offsets_must_fit_32_bits(L):
    """The matrix-core kernels address rows with 32-bit byte offsets: rows x ld
    must stay below 2^31 elements, else the call is refused (never wraps)."""
    # exact scores (one head: no tile limit): 2^21 tokens in rows of 4096 elements is 2^33 elements
    assert bs(L, n=1 << 21, h=1, hd=128, ldq=4096, ldk=4096) == UNSUP
    assert "32-bit" in lemo.lemo_last_error()
    assert bsb(L, B=1, n=1 << 21, h=1, hd=128, ldq=4096, ldk=4096) == UNSUP
    assert "32-bit" in lemo.lemo_last_error()
    # per-token predictor embeddings: wide x
    assert te(L, n=1 << 20, d=4096, ldx=4096) == UNSUP
    # fused products: token rows of x, and the weight
    big = 1 << 20
    assert L.lemo_gather_linear(P, big, 4096, 4096, 64, P, P, P, 64, 4096, P, 64, 256, 1, NULL, NULL) == UNSUP
    assert L.lemo_linear_scatter(P, 64, 64, 16, P, 1 << 22, 1024, P, 1024, 1 << 22, 64, P, P, NULL, NULL) == UNSUP
    # just below the limit passes these checks (and stops at the missing workspace)
    assert bs(L, n=(1 << 19), h=1, hd=128, ldq=4096, ldk=4096, M=NULL, ws=NULL) == WS


def test_launch_grid_limits(L):
    """A launch holds at most 2^23 workgroups in x: more than one head takes at
    most 2^23 tiles of 128 x 128 (one head walks ranges of tiles, so any size
    up to 2^22 tokens passes); the predictor's pooling takes at most 65535
    blocks."""
    assert bs(L, n=1 << 22, h=2, hd=64, ldq=128, ldk=128) == UNSUP
    assert "tiles" in lemo.lemo_last_error()
    assert bs(L, n=2896 * 128, h=2, hd=64, ldq=128, ldk=128, M=NULL, ws=NULL) == WS
    assert bs(L, n=1 << 22, h=1, hd=64, ldq=64, ldk=64, M=NULL, ws=NULL) == WS
    assert bsb(L, B=2, n=2896 * 128, h=2, hd=64, ldq=128, ldk=128, sq=2896 * 128 * 128, sk=2896 * 128 * 128,
               flags=0) == UNSUP
    assert ps(L, n=65536 * 2 + 2, b=2, ws=NULL) == UNSUP
    assert ps(L, n=65535 * 2, b=2, ws=NULL) == WS


def test_binding_buffer_checks():
    """The binding refuses buffers the C side could not tell apart from good
    ones (it sees only an address): wrong dtype, host memory, non-contiguous,
    too small.  Host-side checks only; no call reaches the library."""
    import torch
    t = torch.zeros(8, dtype=torch.float32)
    gpu = torch.device("cuda", 0)
    with pytest.raises(TypeError):
        lemo._buf(torch.zeros(8, dtype=torch.float64), torch.float32, 8, "scores", gpu)
    with pytest.raises(ValueError, match="contiguous"):
        lemo._buf(torch.zeros(4, 4)[:, 1], torch.float32, 4, "scores", gpu)
    with pytest.raises(ValueError, match="9 needed"):
        lemo._buf(t, torch.float32, 9, "scores", gpu)
    with pytest.raises(ValueError, match="tensor on"):      # host memory
        lemo._buf(t, torch.float32, 8, "scores", gpu)
    assert lemo._buf(None, torch.float32, 9, "scores", gpu) is None
    with pytest.raises(ValueError, match="contiguous"):
        lemo._ws_bytes(torch.zeros(4, 4)[:, 1], gpu)
    with pytest.raises(ValueError, match="tensor on"):
        lemo._ws_bytes(t, gpu)
    assert lemo._ws_bytes(None, gpu) == 0
    with pytest.raises(ValueError, match="16 x 4 needed"):
        lemo._rows_within(torch.zeros(8, 4), 16, 4, "x")
    with pytest.raises(ValueError, match="required"):
        lemo._kept_bufs(None, None, None, t.device)


def test_last_error_is_per_thread(L):
    """The detail text of a failed call belongs to the calling thread: two
    threads that fail differently each read back their own message."""
    import threading
    barrier = threading.Barrier(2)
    seen = {}

    def run(name, kw):
        st = bs(L, **kw)
        barrier.wait()                      # both calls have failed before either reads
        seen[name] = (st, lemo.lemo_last_error())

    t1 = threading.Thread(target=run, args=("n", dict(n=1000)))
    t2 = threading.Thread(target=run, args=("mode", dict(mode=2)))
    t1.start(), t2.start()
    t1.join(), t2.join()
    assert seen["n"][0] == INVALID and "not a multiple" in seen["n"][1]
    assert seen["mode"][0] == INVALID and "head_reduce" in seen["mode"][1]


def test_headmax_head_limit(L):
    """HEADMAX keeps per-head maxima for at most 128 heads: 129 are refused;
    PAPER has no such limit (this call stops at the missing workspace)."""
    assert bs(L, h=129, hd=64, ldq=129 * 64, ldk=129 * 64, mode=1) == UNSUP
    assert "128 heads" in lemo.lemo_last_error()
    assert bs(L, h=128, hd=64, ldq=128 * 64, ldk=128 * 64, mode=1, M=NULL, ws=NULL) == WS
    assert bs(L, h=129, hd=64, ldq=129 * 64, ldk=129 * 64, mode=0, M=NULL, ws=NULL) == WS


def test_block_counts_near_int_max(L):
    """Block and tile counts are formed without int overflow: sizes near
    2^31 are refused as too large instead of wrapping to a negative count
    that would pass the limits."""
    big = (1 << 31) - 1
    assert ps(L, n=big, b=256, ws=NULL) == UNSUP           # 8388608 blocks (at most 65535)
    assert "8388608 blocks" in lemo.lemo_last_error()
    assert L.lemo_mlp_block_scores(P, big, 8, 8, 2, P, P, 1 << 40, NULL) == UNSUP   # 2^30 blocks
    assert L.lemo_mlp_block_scores_workspace(big, 8, 2) == (1 << 30) * 4
    d_out = big - 7                                        # a multiple of 8: 8388608 column tiles
    assert L.lemo_gather_linear(P, 1024, 64, 64, 64, P, P, P, d_out, 64, P, d_out, 256, 1, NULL, NULL) == UNSUP
    assert "256 x 256" in lemo.lemo_last_error()
