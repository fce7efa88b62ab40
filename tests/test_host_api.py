"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function the
header declares, and rejects bad arguments before any HIP call."""
import ctypes
import os

import pytest

from block_sparse_video_reblock_amd import _lib


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_video_reblock_amd import build
        build.build()
    return _lib.lib()


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails before any device work
FAKE2 = ctypes.c_void_p(0x2000)


def desc(h=2, n=4096, d=128, dt=_lib.BSA_BF16):
    return ctypes.byref(_lib.BsaDesc(h, n, d, dt))


def test_exports_every_declared_function(L):
    names = _lib.header_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(L, name), name


def test_topk_count(L):
    assert L.bsa_topk_count(1134, 0.1) == 113
    assert L.bsa_topk_count(256, 0.2) == 51
    assert L.bsa_topk_count(256, 0.3) == 76
    assert L.bsa_topk_count(64, 0.25) == 16
    assert L.bsa_topk_count(256, 1.0) == 256
    assert L.bsa_topk_count(10, 0.7) == 7
    assert L.bsa_topk_count(100, 1e-6) == 1
    assert L.bsa_topk_count(100, 0.0) == -1
    assert L.bsa_topk_count(100, 1.5) == -1
    assert L.bsa_topk_count(0, 0.5) == -1


def test_topk_count_matches_oracle(L):
    import oracle
    for nb in (1, 2, 7, 64, 256, 1134, 1620):
        for r in (0.05, 0.1, 0.2, 0.25, 0.3, 0.7, 1.0):
            assert L.bsa_topk_count(nb, r) == oracle.topk_count(nb, r)


def test_workspace_bytes(L):
    assert L.bsa_workspace_bytes(desc()) > 0
    assert L.bsa_workspace_bytes(desc(n=100)) == 0
    assert L.bsa_workspace_bytes(desc(d=64)) == 0                 # bf16 needs head_dim 128
    assert L.bsa_workspace_bytes(desc(d=64, dt=_lib.BSA_F32)) > 0
    assert L.bsa_workspace_bytes(None) == 0


@pytest.mark.parametrize("d,code", [
    ((0, 4096, 128, _lib.BSA_BF16), _lib.BSA_E_ARG),
    ((2, 4000, 128, _lib.BSA_BF16), _lib.BSA_E_ARG),
    ((2, 0, 128, _lib.BSA_BF16), _lib.BSA_E_ARG),
    ((2, 4096, 64, _lib.BSA_BF16), _lib.BSA_E_UNSUPPORTED),
    ((2, 4096, 128, _lib.BSA_F32), _lib.BSA_E_UNSUPPORTED),
    ((2, 4096, 128, 7), _lib.BSA_E_UNSUPPORTED),
    ((2, 1 << 23, 128, _lib.BSA_BF16), _lib.BSA_E_ARG),
])
def test_descriptor_errors(L, d, code):
    st = L.bsa_sparse_attn(ctypes.byref(_lib.BsaDesc(*d)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           4, 0, 0.0, FAKE, None, FAKE, 1 << 40, None)
    assert st == code
    assert L.bsa_last_error()


def test_sparse_attn_argument_errors(L):
    big = 1 << 40
    args = [FAKE] * 6
    # null tensor
    assert L.bsa_sparse_attn(desc(), None, *args[1:], 4, 0, 0.0, FAKE, None, FAKE, big,
                             None) == _lib.BSA_E_ARG
    # topk out of range (nb = 64)
    for k in (0, 65):
        assert L.bsa_sparse_attn(desc(), *args, k, 0, 0.0, FAKE, None, FAKE, big,
                                 None) == _lib.BSA_E_ARG
    # unknown and exclusive flags (BSA_TAIL_BLOCK = 8 combines with the others)
    for fl in (32, 1 << 31, 6, 6 | _lib.BSA_TAIL_BLOCK):
        assert L.bsa_sparse_attn(desc(), *args, 4, fl, 0.0, FAKE, None, FAKE, big,
                                 None) == _lib.BSA_E_ARG
    # bad scale
    for sc in (-1.0, float("nan"), float("inf")):
        assert L.bsa_sparse_attn(desc(), *args, 4, 0, sc, FAKE, None, FAKE, big,
                                 None) == _lib.BSA_E_ARG
    # workspace too small / null
    assert L.bsa_sparse_attn(desc(), *args, 4, 0, 0.0, FAKE, None, FAKE, 16,
                             None) == _lib.BSA_E_WORKSPACE
    assert L.bsa_sparse_attn(desc(), *args, 4, 0, 0.0, FAKE, None, None, big,
                             None) == _lib.BSA_E_ARG


def test_mixed_sequence_argument_errors(L):
    big = 1 << 40
    v3, c3 = [FAKE] * 3, [FAKE2] * 3
    perms = [FAKE] * 3

    def call(n_ctx, ctx=c3, o_ctx=FAKE2, ws=big, flags=0):
        return L.bsa_sparse_attn_ctx(desc(), n_ctx, *v3, *ctx, *perms, 4, flags, 0.0, FAKE,
                                     o_ctx, None, None, FAKE, ws, None)
    for n in (-1, (1 << 19) + 1):
        assert call(n) == _lib.BSA_E_ARG
    assert call(10, ctx=[FAKE2, None, FAKE2]) == _lib.BSA_E_ARG
    assert call(10, o_ctx=None) == _lib.BSA_E_ARG
    assert call(10, flags=32) == _lib.BSA_E_ARG
    # the context tiles need room beyond the plain layer's workspace once they outgrow it
    plain = L.bsa_workspace_bytes(desc())
    assert L.bsa_workspace_bytes_ctx(desc(), 0) == plain
    assert L.bsa_workspace_bytes_ctx(desc(), 1000) >= plain
    need = L.bsa_workspace_bytes_ctx(desc(), 200000)
    assert need > plain
    assert L.bsa_workspace_bytes_ctx(desc(), -1) == 0
    assert call(200000, ws=need - 1) == _lib.BSA_E_WORKSPACE
    # the two-phase form checks the same things (prepare needs no query or output pointers)
    assert L.bsa_prepare_kv_ctx(desc(), 10, *v3, FAKE2, None, FAKE, 0, 0.0, FAKE, big,
                                None) == _lib.BSA_E_ARG
    assert L.bsa_prepare_kv_ctx(desc(), -1, *v3, FAKE2, FAKE2, FAKE, 0, 0.0, FAKE, big,
                                None) == _lib.BSA_E_ARG
    assert L.bsa_prepare_kv_ctx(desc(), 200000, *v3, FAKE2, FAKE2, FAKE, 0, 0.0, FAKE, need - 1,
                                None) == _lib.BSA_E_WORKSPACE
    assert L.bsa_attend_ctx(desc(), 10, *v3, *c3, *perms, 4, 0, 0.0, FAKE, None, None, None,
                            FAKE, big, None) == _lib.BSA_E_ARG
    assert L.bsa_attend_ctx(desc(), 10, *v3, *c3, *perms, 0, 0, 0.0, FAKE, FAKE2, None, None,
                            FAKE, big, None) == _lib.BSA_E_ARG


def test_select_argument_errors(L):
    big = 1 << 40
    a = [FAKE] * 4
    assert L.bsa_select(desc(), *a, 0.0, 0, FAKE, None, FAKE, big, None) == _lib.BSA_E_ARG
    assert L.bsa_select(desc(), *a, 1.5, 0, FAKE, None, FAKE, big, None) == _lib.BSA_E_ARG
    assert L.bsa_select(desc(), *a, 0.1, 65, FAKE, None, FAKE, big, None) == _lib.BSA_E_ARG
    assert L.bsa_select(desc(), *a, 0.1, -2, FAKE, None, FAKE, big, None) == _lib.BSA_E_ARG
    assert L.bsa_select(desc(), *a, 0.1, 0, None, None, FAKE, big, None) == _lib.BSA_E_ARG
    assert L.bsa_select(desc(), *a, 0.1, 0, FAKE, None, FAKE, 8, None) == _lib.BSA_E_WORKSPACE


def test_reblock_and_hook_argument_errors(L):
    big = 1 << 40
    assert L.bsa_reblock(desc(), None, FAKE, FAKE, FAKE, None, FAKE, big, None) == _lib.BSA_E_ARG
    assert L.bsa_reblock(desc(), FAKE, FAKE, FAKE, FAKE2, None, FAKE, 8,
                         None) == _lib.BSA_E_WORKSPACE
    # separate layouts need two permutation buffers
    assert L.bsa_reblock(desc(), FAKE, FAKE, FAKE, FAKE, None, FAKE, big, None) == _lib.BSA_E_ARG
    # one-sided reblock: side must be 0 or 1
    for side in (-1, 2):
        assert L.bsa_reblock_side(desc(), FAKE, FAKE, side, 8, 0, FAKE, None, FAKE, big,
                                  None) == _lib.BSA_E_ARG
    assert L.bsa_reblock_side(desc(), FAKE, FAKE, 0, 0, 0, FAKE, None, FAKE, big,
                              None) == _lib.BSA_E_ARG
    assert L.bsa_reblock_side(desc(), FAKE, FAKE, 0, 8, 2, FAKE, None, FAKE, big,
                              None) == _lib.BSA_E_ARG
    assert L.bsa_reblock_side(desc(), FAKE, FAKE, 1, 8, 0, None, None, FAKE, big,
                              None) == _lib.BSA_E_ARG
    assert L.bsa_reblock_side(desc(), FAKE, FAKE, 1, 8, 1, FAKE, None, FAKE, 8,
                              None) == _lib.BSA_E_WORKSPACE
    # power steps per split outside [1, 64]; unknown tree flags; a shared subtree size outside
    # [2, 64] or without the shared-subtree flag
    for it, fl in ((0, 0), (-1, 0), (65, 0), (8, 2), (2, 1 << 31), (2, 1 | (1 << 8)),
                   (2, 1 | (65 << 8)), (2, 1 | (255 << 8)), (2, 32 << 8)):
        assert L.bsa_reblock_ex(desc(), FAKE, FAKE, 0, it, fl, FAKE, FAKE2, None, FAKE, big,
                                None) == _lib.BSA_E_ARG
        assert L.bsa_reblock_side(desc(), FAKE, FAKE, 0, it, fl, FAKE, None, FAKE, big,
                                  None) == _lib.BSA_E_ARG
    # valid sizes pass the flag checks and stop at the workspace check
    for fl in (1, 1 | (2 << 8), 1 | (32 << 8), 1 | (64 << 8)):
        assert L.bsa_reblock_ex(desc(), FAKE, FAKE, 0, 2, fl, FAKE, FAKE2, None, FAKE, 8,
                                None) == _lib.BSA_E_WORKSPACE
    assert _lib.tree_flags(True, _lib.BSA_LITE_SUBTREE_BLOCKS) == 1 | (64 << 8)
    # layout choice: unknown value, then the key-reuse layout, whose one buffer may serve both
    for bad in (-1, 2):
        assert L.bsa_reblock_layout(desc(), FAKE, FAKE, bad, FAKE, FAKE2, None, FAKE, big,
                                    None) == _lib.BSA_E_ARG
    assert L.bsa_reblock_layout(desc(), FAKE, FAKE, _lib.BSA_LAYOUT_Q_REUSE_K, FAKE, FAKE, None,
                                FAKE, 8, None) == _lib.BSA_E_WORKSPACE
    assert L.bsa_reblock_layout(desc(), FAKE, FAKE, _lib.BSA_LAYOUT_Q_REUSE_K, None, FAKE, None,
                                FAKE, big, None) == _lib.BSA_E_ARG
    assert L.bsa_reblock_from_projections(0, 128, FAKE, FAKE, FAKE, big, None) == _lib.BSA_E_ARG
    assert L.bsa_reblock_from_projections(2, 100, FAKE, FAKE, FAKE, big, None) == _lib.BSA_E_ARG
    assert L.bsa_reblock_from_projections(2, 128, None, FAKE, FAKE, big, None) == _lib.BSA_E_ARG
    assert L.bsa_reblock_from_projections(2, 128, FAKE, FAKE, FAKE, 4,
                                          None) == _lib.BSA_E_WORKSPACE
    assert L.bsa_topk_from_scores(4, 10, 0, FAKE, FAKE, None) == _lib.BSA_E_ARG
    assert L.bsa_topk_from_scores(4, 10, 11, FAKE, FAKE, None) == _lib.BSA_E_ARG
    assert L.bsa_topk_from_scores(0, 10, 1, FAKE, FAKE, None) == _lib.BSA_E_ARG
    assert L.bsa_topk_from_scores(4, 10, 3, None, FAKE, None) == _lib.BSA_E_ARG
    assert L.bsa_summaries(desc(), FAKE, FAKE, FAKE, FAKE, 2, 0.0, FAKE, FAKE, FAKE, FAKE, big,
                           None) == _lib.BSA_E_ARG


def test_tile_layout_argument_errors(L):
    ok = (2, 16, 32, 32, 4, 4, 4)
    assert L.bsa_tile_layout(*ok, None, None) == _lib.BSA_E_ARG            # null perm
    for bad in ((0, 16, 32, 32, 4, 4, 4),       # no heads
                (2, 16, 32, 32, 4, 4, 2),       # 32-token tile
                (2, 16, 32, 30, 4, 4, 4),       # 4 does not divide 30
                (2, 21, 48, 72, 4, 4, 4),       # 4 does not divide 21
                (2, 0, 32, 32, 4, 4, 4),
                (2, 512, 512, 512, 4, 4, 4)):   # too many tokens
        assert L.bsa_tile_layout(*bad, FAKE, None) == _lib.BSA_E_ARG, bad
        assert L.bsa_last_error()


def test_architecture_is_checked(L, monkeypatch):
    monkeypatch.setenv("BSATTN_ARCH_OVERRIDE", "gfx942")
    st = L.bsa_topk_from_scores(4, 10, 3, FAKE, FAKE, None)
    assert st == _lib.BSA_E_UNSUPPORTED
    assert b"gfx942" in L.bsa_last_error()


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4):
        assert L.bsa_status_str(code)


def test_summaries_noalloc_rejects_sizes_beyond_its_scratch(L):
    """The allocation-free summaries call checks its fixed scratch size on the host: within the
    limit it reports the bytes it needs, beyond it BSA_E_ARG before any HIP call."""
    limit = 16 << 20
    need = L.bsa_summaries_noalloc_bytes(desc(h=24, n=72576))
    assert 0 < need <= limit
    assert L.bsa_summaries_noalloc_bytes(desc(h=24, n=1 << 19)) <= limit
    big = _lib.BsaDesc(64, 1 << 19, 128, _lib.BSA_BF16)
    assert L.bsa_summaries_noalloc_bytes(ctypes.byref(big)) > limit
    st = L.bsa_summaries_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 0, 0.0, FAKE, FAKE,
                                 FAKE, None)
    assert st == _lib.BSA_E_ARG and b"scratch" in L.bsa_last_error()
    st = L.bsa_summaries_noalloc(desc(), FAKE, FAKE, FAKE, FAKE, 2, 0.0, FAKE, FAKE, FAKE, None)
    assert st == _lib.BSA_E_ARG


def test_list_check_argument_errors(L):
    assert L.bsa_check_lists(0, 10, 1, FAKE, FAKE, None) == _lib.BSA_E_ARG
    assert L.bsa_check_lists(4, 0, 1, FAKE, FAKE, None) == _lib.BSA_E_ARG
    assert L.bsa_check_lists(4, 10, 0, FAKE, FAKE, None) == _lib.BSA_E_ARG
    assert L.bsa_check_lists(4, 10, 11, FAKE, FAKE, None) == _lib.BSA_E_ARG
    assert L.bsa_check_lists(4, 10, 3, None, FAKE, None) == _lib.BSA_E_ARG
    assert L.bsa_check_lists(4, 10, 3, FAKE, None, None) == _lib.BSA_E_ARG
    out = (ctypes.c_int32 * 2)()
    assert L.bsa_list_status(None, 1 << 20, out, None) == _lib.BSA_E_ARG
    assert L.bsa_list_status(FAKE, 4, out, None) == _lib.BSA_E_WORKSPACE
    assert L.bsa_list_status(FAKE, 1 << 20, None, None) == _lib.BSA_E_ARG
    # the strict-list flag is a known flag: the call gets past the flag check to the workspace
    st = L.bsa_sparse_attn(desc(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, _lib.BSA_CHECK_LISTS,
                           0.0, FAKE, None, FAKE, 8, None)
    assert st == _lib.BSA_E_WORKSPACE
    st = L.bsa_sparse_attn(desc(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 0.0, FAKE, None,
                           FAKE, 1 << 40, None)
    assert st == _lib.BSA_E_ARG
