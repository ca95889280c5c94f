"""The C-ABI library loads, exports every symbol include/flowcache.h declares,
and rejects bad arguments on the host (no GPU work is queued on these paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flowcache.h")
LIB = os.path.join(ROOT, "kv_cache_compression_fc_amd", "libflowcache.so")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return sorted(set(re.findall(r"\b(fc_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def fc():
    from conftest import ensure_library
    ensure_library()
    from kv_cache_compression_fc_amd import binding
    return binding


def test_header_declares_the_path():
    names = declared_functions()
    for want in ("fc_kv_compress", "fc_chunk_rel_l1_decide", "fc_kv_compress_workspace_bytes",
                 "fc_chunk_rel_l1_workspace_bytes", "fc_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol(fc):
    lib = ctypes.CDLL(LIB)
    names = declared_functions()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(fc.EXPORTS) == set(names)


def test_status_strings(fc):
    assert fc.fc_status_string(fc.FC_OK) == "ok"
    assert "workspace" in fc.fc_status_string(fc.FC_ERR_WORKSPACE)
    assert fc.fc_status_string(99) == "unknown status"


def _params(fc, **kw):
    base = dict(H=24, d=128, L_q=3600, L_k=18000, B_budget=7200, lambda_=0.5, pool_window=7, softmax_scale=0.0,
                dtype=fc.FC_BF16)
    base.update(kw)
    return fc.fc_kv_params(**base)


def test_kv_workspace_query(fc):
    n = fc.fc_kv_compress_workspace_bytes(_params(fc))
    # at least imp, r and keys (3 x 4 B per key-head) plus the lse partials
    assert n >= 3 * 4 * 24 * 18000 + 8 * 24 * 3600
    assert n % 256 == 0
    for bad in (dict(H=0), dict(L_k=0), dict(B_budget=0), dict(lambda_=1.5), dict(lambda_=float("nan")),
                dict(pool_window=4), dict(pool_window=0), dict(softmax_scale=-1.0), dict(d=96), dict(dtype=7)):
        assert fc.fc_kv_compress_workspace_bytes(_params(fc, **bad)) == 0, bad
    # more work-items than one dispatch can count (65535 heads of 8M queries)
    assert fc.fc_kv_compress_workspace_bytes(_params(fc, H=65535, L_q=8_000_000, L_k=64, B_budget=8)) == 0


def test_kv_argument_errors(fc):
    lib = fc._lib
    p = _params(fc)
    dummy = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(4096)
    need = fc.fc_kv_compress_workspace_bytes(p)
    # null required pointer
    st = lib.fc_kv_compress(ctypes.byref(p), None, dummy, dummy, dummy, dummy, dummy, None, None, None, ws, need, None)
    assert st == fc.FC_ERR_INVALID_ARG
    # misaligned tensor
    st = lib.fc_kv_compress(ctypes.byref(p), ctypes.c_void_p(4098), dummy, dummy, dummy, dummy, dummy, None, None,
                            None, ws, need, None)
    assert st == fc.FC_ERR_INVALID_ARG
    # short workspace
    st = lib.fc_kv_compress(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, dummy, None, None, None, ws,
                            need - 1, None)
    assert st == fc.FC_ERR_WORKSPACE
    # misaligned workspace
    st = lib.fc_kv_compress(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, dummy, None, None, None,
                            ctypes.c_void_p(4096 + 128), need, None)
    assert st == fc.FC_ERR_WORKSPACE
    # unsupported head dim / dtype
    st = lib.fc_kv_compress(ctypes.byref(_params(fc, d=96)), dummy, dummy, dummy, dummy, dummy, dummy, None, None,
                            None, ws, need, None)
    assert st == fc.FC_ERR_UNSUPPORTED
    st = lib.fc_kv_compress(ctypes.byref(_params(fc, pool_window=8)), dummy, dummy, dummy, dummy, dummy, dummy,
                            None, None, None, ws, need, None)
    assert st == fc.FC_ERR_INVALID_ARG
    # select: partial gather pointers
    st = lib.fc_kv_select(ctypes.byref(p), dummy, dummy, dummy, None, None, None, dummy, None, None, None, ws, need,
                          None)
    assert st == fc.FC_ERR_INVALID_ARG
    assert lib.fc_topb_select(2, 10, 0, dummy, dummy, ws, 1 << 20, None) == fc.FC_ERR_INVALID_ARG
    assert lib.fc_topb_select(2, 10, 3, dummy, dummy, ws, 16, None) == fc.FC_ERR_WORKSPACE


def test_chunk_workspace_and_errors(fc):
    lib = fc._lib
    p = fc.fc_l1_params(16, 5, 0.01, fc.FC_BF16)
    e = 64 * 8 * 90 * 160
    offs = [i * e for i in range(17)]
    n = fc.fc_chunk_rel_l1_workspace_bytes(p, offs)
    assert n > 16 * 4
    assert fc.fc_chunk_rel_l1_workspace_bytes(fc.fc_l1_params(0, 5, 0.01, fc.FC_BF16), [0]) == 0
    assert fc.fc_chunk_rel_l1_workspace_bytes(fc.fc_l1_params(2, 5, 0.01, fc.FC_BF16), [0, 5, 3]) == 0
    assert fc.fc_chunk_rel_l1_workspace_bytes(fc.fc_l1_params(2, -1, 0.01, fc.FC_BF16), [0, 5, 9]) == 0
    assert fc.fc_chunk_rel_l1_workspace_bytes(fc.fc_l1_params(2, 1, float("nan"), fc.FC_BF16), [0, 5, 9]) == 0
    assert fc.fc_chunk_rel_l1_workspace_bytes(fc.fc_l1_params(200, 1, 0.1, fc.FC_BF16), list(range(201))) == 0
    dummy = ctypes.c_void_p(4096)
    arr = fc._offsets(offs)
    st = lib.fc_chunk_rel_l1_decide(ctypes.byref(p), arr, dummy, dummy, dummy, dummy, None, None, dummy, n, None)
    assert st == fc.FC_ERR_INVALID_ARG
    st = lib.fc_chunk_rel_l1_decide(ctypes.byref(p), arr, dummy, dummy, dummy, dummy, dummy, None, dummy, n - 1,
                                    None)
    assert st == fc.FC_ERR_WORKSPACE
    st = lib.fc_chunk_rel_l1_decide(ctypes.byref(p), arr, ctypes.c_void_p(4100), dummy, dummy, dummy, dummy, None,
                                    dummy, n, None)
    assert st == fc.FC_ERR_INVALID_ARG


def _cache_params(fc, **kw):
    base = dict(H=24, d=128, B_budget=7200, B_active=3600, lambda_=0.5, pool_window=7, softmax_scale=0.0,
                dtype=fc.FC_BF16)
    base.update(kw)
    return fc.fc_cache_params(**base)


def test_cache_workspace_query(fc):
    c = _cache_params(fc)
    n = fc.fc_cache_commit_workspace_bytes(c, 3600)
    # the kept indices plus the compression's workspace for every merged
    # length B_budget < L <= B_total (no merged copy of K and V)
    idx = 24 * 7200 * 4
    comp = [fc.fc_kv_compress_workspace_bytes(fc.fc_kv_params(24, 128, 3600, L, 7200, 0.5, 7, 0.0, fc.FC_BF16))
            for L in range(7201, 10801)]
    assert n == (idx + 255) // 256 * 256 + max(comp)
    assert n % 256 == 0
    for bad in (dict(H=0), dict(B_budget=0), dict(B_active=0), dict(lambda_=-0.1), dict(pool_window=2),
                dict(d=80), dict(dtype=5), dict(B_budget=2 ** 31 - 10, B_active=100)):
        assert fc.fc_cache_commit_workspace_bytes(_cache_params(fc, **bad), 3600) == 0, bad
    assert fc.fc_cache_commit_workspace_bytes(c, 0) == 0


def test_cache_argument_errors(fc):
    lib = fc._lib
    c = _cache_params(fc)
    dummy = ctypes.c_void_p(4096)
    need = fc.fc_cache_commit_workspace_bytes(c, 3600)

    # distinct (never dereferenced) addresses for the two regions
    K_cur, V_cur, pos_cur0 = ctypes.c_void_p(1 << 16), ctypes.c_void_p(2 << 16), ctypes.c_void_p(3 << 16)
    K_sp, V_sp, pos_sp0 = ctypes.c_void_p(4 << 16), ctypes.c_void_p(5 << 16), ctypes.c_void_p(6 << 16)

    def commit(L_clean, L_c, pos0=0, Q=dummy, ws_bytes=need, p=c, K_chunk=dummy, V_chunk=dummy, K_spare=K_sp,
               pos_cur=pos_cur0, pos_spare=pos_sp0):
        n = ctypes.c_int32(L_clean)
        sw = ctypes.c_int32(-7)
        st = lib.fc_cache_commit(ctypes.byref(p), ctypes.byref(n), K_chunk, V_chunk, L_c, pos0, Q, 3600, K_cur,
                                 V_cur, pos_cur, K_spare, V_sp, pos_spare, ctypes.byref(sw), dummy, ws_bytes, None)
        assert sw.value == -7  # untouched on error
        return st, n.value

    assert commit(-1, 100) == (fc.FC_ERR_INVALID_ARG, -1)
    assert commit(7201, 100) == (fc.FC_ERR_INVALID_ARG, 7201)
    assert commit(0, 0) == (fc.FC_ERR_INVALID_ARG, 0)
    assert commit(0, 3601) == (fc.FC_ERR_INVALID_ARG, 0)
    assert commit(0, 100, pos0=-5) == (fc.FC_ERR_INVALID_ARG, 0)
    assert commit(0, 100, pos0=2 ** 31 - 99) == (fc.FC_ERR_INVALID_ARG, 0)   # last position would be 2^31
    assert commit(0, 100, pos0=2 ** 31 - 50) == (fc.FC_ERR_INVALID_ARG, 0)
    assert commit(0, 100, K_chunk=ctypes.c_void_p(4104)) == (fc.FC_ERR_INVALID_ARG, 0)
    assert commit(0, 100, p=_cache_params(fc, d=96)) == (fc.FC_ERR_UNSUPPORTED, 0)
    # a commit that overflows the budget needs queries and the workspace
    assert commit(7200, 100, Q=None) == (fc.FC_ERR_INVALID_ARG, 7200)
    assert commit(7200, 100, ws_bytes=need // 2) == (fc.FC_ERR_WORKSPACE, 7200)
    # ... and the spare region, with positions on both sides or neither
    assert commit(7200, 100, K_spare=None) == (fc.FC_ERR_INVALID_ARG, 7200)
    assert commit(7200, 100, pos_spare=None) == (fc.FC_ERR_INVALID_ARG, 7200)
    assert commit(7200, 100, K_spare=ctypes.c_void_p(4100)) == (fc.FC_ERR_INVALID_ARG, 7200)
    # the spare region at the current region's address
    n = ctypes.c_int32(7200)
    sw = ctypes.c_int32(-7)
    cur, spare = ctypes.c_void_p(8192), ctypes.c_void_p(1 << 20)
    assert lib.fc_cache_commit(ctypes.byref(c), ctypes.byref(n), dummy, dummy, 100, 0, dummy, 3600, cur, spare,
                               None, cur, ctypes.c_void_p(1 << 21), None, ctypes.byref(sw), dummy, need,
                               None) == fc.FC_ERR_INVALID_ARG
    assert n.value == 7200 and sw.value == -7
    # a chunk given by one pointer only
    assert commit(0, 100, V_chunk=None) == (fc.FC_ERR_INVALID_ARG, 0)
    assert lib.fc_cache_commit(ctypes.byref(c), None, dummy, dummy, 10, 0, dummy, 3600, dummy, dummy, dummy, dummy,
                               dummy, dummy, None, dummy, need, None) == fc.FC_ERR_INVALID_ARG


def test_binding_refuses_mismatched_tensors(fc):
    # The library trusts the extents its arguments imply; the binding refuses
    # a tensor of another shape or dtype before any pointer is passed (these
    # CPU tensors would otherwise only be refused for living on the host).
    import torch
    bf = torch.bfloat16
    Q, K = torch.zeros(2, 8, 64, dtype=bf), torch.zeros(2, 16, 64, dtype=bf)
    with pytest.raises(ValueError, match="V: shape"):
        fc.fc_kv_compress(Q, K, torch.zeros(2, 15, 64, dtype=bf), 4, 0.5, 3)
    with pytest.raises(ValueError, match="V: dtype"):
        fc.fc_kv_compress(Q, K, torch.zeros(2, 16, 64), 4, 0.5, 3)
    with pytest.raises(ValueError, match="K: dtype"):
        fc.fc_kv_compress(Q, K.float(), K.float(), 4, 0.5, 3)
    with pytest.raises(ValueError, match="K: shape"):
        fc.fc_kv_compress(Q, torch.zeros(3, 16, 64, dtype=bf), torch.zeros(3, 16, 64, dtype=bf), 4, 0.5, 3)
    with pytest.raises(ValueError, match="idx: dtype"):
        fc.fc_kv_compress(Q, K, K, 4, 0.5, 3, out={"idx": torch.zeros(2, 4, dtype=torch.int64)})
    with pytest.raises(ValueError, match="K_out: shape"):
        fc.fc_kv_compress(Q, K, K, 4, 0.5, 3, out={"K_out": torch.zeros(2, 5, 64, dtype=bf)})
    with pytest.raises(ValueError, match="lse: shape"):
        fc.fc_kv_importance_colsum(Q, K, torch.zeros(2, 7))
    with pytest.raises(ValueError, match="r: shape"):
        fc.fc_kv_select(torch.zeros(2, 16), torch.zeros(2, 15), 4, 0.5, 3)
    with pytest.raises(ValueError, match="given together"):
        fc.fc_kv_select(torch.zeros(2, 16), torch.zeros(2, 16), 4, 0.5, 3, K=K)
    with pytest.raises(ValueError, match="scores: dtype"):
        fc.fc_topb_select(torch.zeros(2, 16, dtype=torch.float64), 4)

    offs = [0, 100, 250]
    p = fc.fc_l1_params(2, 1, 0.01, fc.FC_BF16)
    st, f, rec = torch.zeros(2, dtype=torch.int32), torch.zeros(2), torch.zeros(2, dtype=torch.uint8)
    ws = torch.zeros(4096, dtype=torch.uint8)
    with pytest.raises(ValueError, match="X_tm1: 249 elements"):
        fc.fc_chunk_rel_l1_decide(p, offs, torch.zeros(250, dtype=bf), torch.zeros(249, dtype=bf), st, f, rec,
                                  workspace=ws)
    with pytest.raises(ValueError, match="X_t: dtype"):
        fc.fc_chunk_rel_l1_decide(p, offs, torch.zeros(250), torch.zeros(250, dtype=bf), st, f, rec, workspace=ws)
    with pytest.raises(ValueError, match="step: dtype"):
        fc.fc_chunk_rel_l1_decide(p, offs, torch.zeros(250, dtype=bf), torch.zeros(250, dtype=bf), st.long(), f,
                                  rec, workspace=ws)
    with pytest.raises(ValueError, match="offsets for 2 chunks"):
        fc.fc_chunk_rel_l1_decide(p, offs[:2], torch.zeros(250, dtype=bf), torch.zeros(250, dtype=bf), st, f, rec,
                                  workspace=ws)
    with pytest.raises(ValueError, match="dt: shape"):
        x = torch.zeros(250, dtype=bf)
        fc.fc_euler_step_l1_decide(p, offs, x, x, torch.zeros(3), x, st, f, rec, workspace=ws)
    with pytest.raises(ValueError, match="f: shape"):
        x = torch.zeros(250, dtype=bf)
        fc.fc_uniform_rel_l1_decide(p, offs, x, x, st, st[:1], f, rec, workspace=ws)

    c = fc.fc_cache_params(2, 64, 32, 16, 0.5, 3, 0.0, fc.FC_BF16)
    Kc = torch.zeros(2, 48, 64, dtype=bf)
    pos = torch.zeros(2, 48, dtype=torch.int32)
    K8 = torch.zeros(2, 8, 64, dtype=bf)
    with pytest.raises(ValueError, match="K_chunk: shape"):
        fc.fc_cache_commit(c, 0, torch.zeros(2, 8, 128, dtype=bf), torch.zeros(2, 8, 128, dtype=bf), 0, None, Kc,
                           Kc, pos, Kc, Kc, pos, ws)
    with pytest.raises(ValueError, match="K_cur: shape"):   # regions hold B_budget + B_active rows
        fc.fc_cache_commit(c, 0, K8, K8, 0, None, Kc[:, :32], Kc, pos, Kc, Kc, pos, ws)
    with pytest.raises(ValueError, match="pos_spare: dtype"):
        fc.fc_cache_commit(c, 0, K8, K8, 0, None, Kc, Kc, pos, Kc, Kc, pos.long(), ws)
    with pytest.raises(fc.FlowCacheError):   # an in-place chunk needs its length
        fc.fc_cache_commit(c, 0, None, None, 0, None, Kc, Kc, pos, Kc, Kc, pos, ws)
    with pytest.raises(ValueError, match="on the GPU"):  # consistent arguments reach the device check
        fc.fc_cache_commit(c, 0, K8, K8, 0, None, Kc, Kc, pos, Kc, Kc, pos, ws)


def test_pool_window_cap_and_alignment_rule(fc):
    """The contract's limits: 1 <= pool_window <= 129 and odd; row tensors and
    chunk states 16-byte aligned (FC_ERR_INVALID_ARG otherwise)."""
    assert fc.fc_kv_compress_workspace_bytes(_params(fc, pool_window=129)) > 0
    assert fc.fc_kv_compress_workspace_bytes(_params(fc, pool_window=131)) == 0
    lib = fc._lib
    p = _params(fc)
    need = fc.fc_kv_compress_workspace_bytes(p)
    ws = ctypes.c_void_p(1 << 20)
    a = ctypes.c_void_p(4096)
    for bad in range(5):  # Q, K, V, K_out, V_out each 8 bytes off a 16-byte boundary
        ptrs = [a] * 5
        ptrs[bad] = ctypes.c_void_p(4096 + 8)
        st = lib.fc_kv_compress(ctypes.byref(p), *ptrs, a, None, None, None, ws, need, None)
        assert st == fc.FC_ERR_INVALID_ARG, bad
    st = lib.fc_kv_compress(ctypes.byref(_params(fc, pool_window=131)), a, a, a, a, a, a, None, None, None, ws,
                            need, None)
    assert st == fc.FC_ERR_INVALID_ARG
    # chunk states: the fused Euler step checks X_t, v and X_next
    pl = fc.fc_l1_params(2, 1, 0.01, fc.FC_BF16)
    offs = fc._offsets([0, 64, 128])
    n = fc.fc_chunk_rel_l1_workspace_bytes(pl, [0, 64, 128])
    for bad in range(3):
        ptrs = [a] * 3
        ptrs[bad] = ctypes.c_void_p(4096 + 8)
        st = lib.fc_euler_step_l1_decide(ctypes.byref(pl), offs, ptrs[0], ptrs[1], a, ptrs[2], a, a, a, None, ws, n,
                                         None)
        assert st == fc.FC_ERR_INVALID_ARG, bad
    # no workspace at all is a workspace error, not a crash
    st = lib.fc_chunk_rel_l1_decide(ctypes.byref(pl), offs, a, a, a, a, a, None, None, 0, None)
    assert st == fc.FC_ERR_WORKSPACE


def test_binding_workspace_sizes(fc):
    """Workspace sizes cross the boundary in bytes whatever the tensor's
    dtype, and the chunk-decision wrappers size their own workspace when none
    is given (here the CPU tensors then stop at the device check, not at an
    AttributeError)."""
    import torch
    assert fc._nbytes(None) == 0
    assert fc._nbytes(torch.zeros(10, dtype=torch.float32)) == 40
    assert fc._nbytes(torch.zeros(10, dtype=torch.uint8)) == 10
    bf = torch.bfloat16
    offs = [0, 100, 250]
    p = fc.fc_l1_params(2, 1, 0.01, fc.FC_BF16)
    st, f, rec = torch.zeros(2, dtype=torch.int32), torch.zeros(2), torch.zeros(2, dtype=torch.uint8)
    x = torch.zeros(250, dtype=bf)
    for call in (lambda: fc.fc_chunk_rel_l1_decide(p, offs, x, x, st, f, rec),
                 lambda: fc.fc_euler_step_l1_decide(p, offs, x, x, torch.zeros(2), x, st, f, rec),
                 lambda: fc.fc_uniform_rel_l1_decide(p, offs, x, x, st, st[:1], f[:1], rec),
                 lambda: fc.fc_history_rel_l1_decide(p, offs, x, x, st, f, rec)):
        with pytest.raises(ValueError, match="on the GPU"):
            call()


def test_noalloc_decision_limits(fc):
    """The allocation-free decision refuses, on the host, states whose slabs
    exceed its static scratch, and checks its arguments as the workspace form
    does (no device is touched on these paths)."""
    lib = fc._lib
    a = ctypes.c_void_p(4096)
    assert fc.FC_NOALLOC_SCRATCH_BYTES == 256 * 1024
    # bf16 slabs hold 32768 elements: 8192 slabs (64 KiB of partials) fit,
    # 2 x 2^30 elements (65536 slabs, 512 KiB) do not
    p = fc.fc_l1_params(2, 1, 0.01, fc.FC_BF16)
    big = fc._offsets([0, 1 << 30, 1 << 31])
    assert lib.fc_chunk_rel_l1_decide_noalloc(ctypes.byref(p), big, a, a, a, a, a, None, None) == fc.FC_ERR_UNSUPPORTED
    assert fc.fc_chunk_rel_l1_workspace_bytes(p, [0, 1 << 30, 1 << 31]) > fc.FC_NOALLOC_SCRATCH_BYTES
    small = fc._offsets([0, 64, 128])
    assert lib.fc_chunk_rel_l1_decide_noalloc(ctypes.byref(p), small, None, a, a, a, a, None, None) == \
        fc.FC_ERR_INVALID_ARG
    assert lib.fc_chunk_rel_l1_decide_noalloc(ctypes.byref(p), small, ctypes.c_void_p(4104), a, a, a, a, None,
                                              None) == fc.FC_ERR_INVALID_ARG
    assert lib.fc_chunk_rel_l1_decide_noalloc(ctypes.byref(fc.fc_l1_params(0, 1, 0.01, fc.FC_BF16)), small, a, a, a,
                                              a, a, None, None) == fc.FC_ERR_INVALID_ARG


def test_decision_presets(fc):
    """The page's settings (FlowCache page, Key designs item 2): m = 5 for
    MAGI-1 and 4 for SkyReels-V2; eps 0.01 / 0.015 (MAGI slow / fast) and
    0.1 / 0.15 (SkyReels slow / fast)."""
    import torch
    want = {"magi-slow": (5, 0.01), "magi-fast": (5, 0.015), "skyreels-slow": (4, 0.1), "skyreels-fast": (4, 0.15)}
    assert fc.DECISION_PRESETS == want
    for name, (m, eps) in want.items():
        dec = fc.ChunkDecider.preset(name, [0, 100, 250], torch.bfloat16, device="cpu")
        assert dec.p.m == m and dec.p.eps == pytest.approx(eps, rel=1e-7) and dec.p.n_chunks == 2
    with pytest.raises(ValueError, match="unknown preset"):
        fc.ChunkDecider.preset("magi-medium", [0, 100], torch.bfloat16, device="cpu")
