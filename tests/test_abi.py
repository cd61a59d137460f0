"""The C-ABI library loads and exports every symbol include/kvevict.h declares (CPU only).

No kernel is launched here: besides kv_version/kv_status_string, only calls
that the host-side validation rejects before any launch are made.
"""
import ctypes
import os
import re

import pytest

WS = ctypes.c_void_p(0x7000000)   # a workspace pointer: never dereferenced, validation fails first

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvevict.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from eviction_long_reasoning_amd import _lib
    from eviction_long_reasoning_amd.build import build, LIB_PATH
    if not os.path.exists(LIB_PATH):
        build()
    return _lib.load()


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("tri_score", "kv_score_workspace_bytes", "tri_score_rotated", "tri_score_gqa",
              "kv_score_gqa_workspace_bytes", "kv_select_topk", "kv_select_workspace_bytes", "kv_select_random",
              "kv_compact", "kv_version", "kv_status_string", "kv_device_checks"):
        assert n in names, names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.kv_version() >> 16 == 2
    assert lib.kv_device_checks() == 0
    assert lib.kv_status_string(0).decode() == "ok"
    assert "invalid" in lib.kv_status_string(-1).decode()
    assert lib.kv_status_string(12345).decode() == "unknown status"


def test_host_validation_rejects_bad_arguments(lib):
    from eviction_long_reasoning_amd import _lib as L
    dummy = ctypes.c_void_p(0x1000)        # never dereferenced: validation fails first
    seq = ctypes.c_void_p(0x2000)
    arr = (ctypes.c_int32 * 1)(1)
    # null shape
    assert lib.tri_score(None, dummy, None, dummy, None, dummy, 1e4, arr, 1, dummy, WS, 1 << 20, None) == L.KV_EINVAL
    # odd head_dim / bad dtype / misaligned K
    sh = L.KvShape(1, 1, 1, 7, 16, L.KV_F32, seq)
    assert lib.tri_score(ctypes.byref(sh), dummy, None, dummy, None, dummy, 1e4, arr, 1, dummy, WS, 1 << 20, None) == L.KV_ESHAPE
    sh = L.KvShape(1, 1, 1, 8, 16, 9, seq)
    assert lib.tri_score(ctypes.byref(sh), dummy, None, dummy, None, dummy, 1e4, arr, 1, dummy, WS, 1 << 20, None) == L.KV_EDTYPE
    sh = L.KvShape(1, 1, 1, 8, 16, L.KV_BF16, seq)
    assert lib.tri_score(ctypes.byref(sh), ctypes.c_void_p(0x1008), None, dummy, None, dummy, 1e4, arr, 1, dummy, WS, 1 << 20, None) == L.KV_EINVAL
    # no offsets, non-positive theta
    assert lib.tri_score(ctypes.byref(sh), dummy, None, dummy, None, dummy, 1e4, arr, 0, dummy, WS, 1 << 20, None) == L.KV_EINVAL
    assert lib.tri_score(ctypes.byref(sh), dummy, None, dummy, None, dummy, -1.0, arr, 1, dummy, WS, 1 << 20, None) == L.KV_EINVAL
    # rotated keys: unknown style, half-split rows that do not split into whole lanes, bad paging
    assert lib.tri_score_rotated(ctypes.byref(sh), dummy, None, 7, dummy, None, dummy, 1e4, arr, 1, dummy,
                                 None) == L.KV_EINVAL
    sh96 = L.KvShape(1, 1, 1, 96, 16, L.KV_BF16, seq)
    assert lib.tri_score_rotated(ctypes.byref(sh96), dummy, None, L.KV_ROPE_HALF, dummy, None, dummy, 1e4, arr, 1,
                                 dummy, None) == L.KV_ESHAPE
    pg = L.KvPaged(dummy, 1, 12, 4)       # block size not a power of two
    assert lib.tri_score_rotated(ctypes.byref(sh), dummy, ctypes.byref(pg), 0, dummy, None, dummy, 1e4, arr, 1,
                                 dummy, None) == L.KV_EINVAL
    pg = L.KvPaged(dummy, 2, 8, 4, 2)     # unknown pool layout
    assert lib.tri_score_rotated(ctypes.byref(sh), dummy, ctypes.byref(pg), 0, dummy, None, dummy, 1e4, arr, 1,
                                 dummy, None) == L.KV_EINVAL
    pg = L.KvPaged(dummy, 1, 8, 4)        # 1 block of 8 cannot hold t_cap = 16 slots
    assert lib.tri_score_rotated(ctypes.byref(sh), dummy, ctypes.byref(pg), 0, dummy, None, dummy, 1e4, arr, 1,
                                 dummy, None) == L.KV_ESHAPE
    # one head's bf16 d = 128 rows beyond 32-bit byte offsets
    huge = L.KvShape(1, 1, 1, 128, ((1 << 31) - (64 << 9)) // 256, L.KV_BF16, seq)
    assert lib.tri_score(ctypes.byref(huge), dummy, None, dummy, None, dummy, 1e4, arr, 1, dummy, WS, 1 << 20, None) == L.KV_ESHAPE
    big = L.KvShape(1, 1, 1, 8, (1 << 18) + 1, L.KV_BF16, seq)   # past the union selector's LDS bits
    huge_sel = L.KvShape(1, 1, 1, 8, (1 << 26) + 1, L.KV_BF16, seq)  # past every selector
    # grouped-query scores: group outside 1..16, workspace too small, fp32 head_dim beyond 128
    shg = L.KvShape(2, 3, 4, 128, 1000, L.KV_BF16, None)
    need = lib.kv_score_gqa_workspace_bytes(ctypes.byref(shg), 4)
    # the header, then (L*S*H) heads x 1 chunk of 1024 keys x G x (sum, sum of squares) in fp64
    assert need == L.KV_WORKSPACE_HEADER + 2 * 3 * 4 * 1 * 4 * 2 * 8
    shg2 = L.KvShape(2, 3, 4, 128, 1025, L.KV_BF16, None)
    assert lib.kv_score_gqa_workspace_bytes(ctypes.byref(shg2), 4) == 2 * need - L.KV_WORKSPACE_HEADER
    assert lib.kv_score_gqa_workspace_bytes(ctypes.byref(shg), 17) == 0
    assert lib.kv_score_gqa_workspace_bytes(ctypes.byref(shg), 0) == 0
    assert lib.kv_score_gqa_workspace_bytes(None, 4) == 0
    shg.seq_len = seq
    ws, hs, sc = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x400000)
    for grp in (0, 17):
        assert lib.tri_score_gqa(ctypes.byref(shg), dummy, None, grp, dummy, None, dummy, 1e4, arr, 1, hs, sc, ws,
                                 1 << 20, None) == L.KV_EINVAL
    assert lib.tri_score_gqa(ctypes.byref(shg), dummy, None, 4, dummy, None, dummy, 1e4, arr, 1, hs, sc, ws,
                             need - 8, None) == L.KV_EWORKSPACE
    assert lib.tri_score_gqa(ctypes.byref(shg), dummy, None, 4, dummy, None, dummy, 1e4, arr, 1, hs, sc,
                             ctypes.c_void_p(0x100004), need, None) == L.KV_EWORKSPACE  # misaligned workspace
    assert lib.tri_score_gqa(ctypes.byref(shg), dummy, None, 4, dummy, None, dummy, 1e4, arr, 1, hs, hs, ws,
                             need, None) == L.KV_EINVAL      # scores alias the per-query-head scores
    shbig = L.KvShape(1, 1, 1, 16, 1 << 26, L.KV_BF16, seq)  # 16 query heads x 2^26 slots overflow 2^31 bytes
    needbig = lib.kv_score_gqa_workspace_bytes(ctypes.byref(shbig), 16)
    assert lib.tri_score_gqa(ctypes.byref(shbig), dummy, None, 16, dummy, None, dummy, 1e4, arr, 1, hs, sc, ws,
                             needbig, None) == L.KV_ESHAPE
    sh256 = L.KvShape(1, 1, 1, 256, 16, L.KV_F32, seq)       # fp32 rows beyond 128 elements
    need256 = lib.kv_score_gqa_workspace_bytes(ctypes.byref(sh256), 2)
    assert lib.tri_score_gqa(ctypes.byref(sh256), dummy, None, 2, dummy, None, dummy, 1e4, arr, 1, hs, sc, ws,
                             need256, None) == L.KV_ESHAPE
    # policy variants: the recency selector and the shared draw validate like the others;
    # in-place compaction refuses K and V that overlap, and positions overlapping either
    pol = L.KvPolicy(8, 2, 4, seq)
    assert lib.kv_select_recent(ctypes.byref(sh), ctypes.byref(pol), dummy, 7, dummy, None) == L.KV_ESHAPE
    assert lib.kv_select_recent(ctypes.byref(sh), None, dummy, 8, dummy, None) == L.KV_EINVAL
    assert lib.kv_select_random_shared(ctypes.byref(huge_sel), ctypes.byref(pol), None, 1, 0, dummy, 8, dummy, WS, 1 << 20, None) == L.KV_ESHAPE
    assert lib.kv_select_union(ctypes.byref(sh), ctypes.byref(pol), 4, 0, None, dummy, dummy, 8, dummy,
                               None) == L.KV_EINVAL
    assert lib.kv_select_union(ctypes.byref(sh), ctypes.byref(pol), 0, 0, dummy, dummy, dummy, 8, dummy,
                               None) == L.KV_EINVAL
    assert lib.kv_select_union(ctypes.byref(big), ctypes.byref(pol), 2, 0, dummy, dummy, dummy, 8, dummy,
                               None) == L.KV_ESHAPE
    assert lib.kv_audit_kept(ctypes.byref(sh), ctypes.byref(pol), dummy, 8, dummy, None, None) == L.KV_EINVAL
    assert lib.kv_audit_kept(ctypes.byref(sh), ctypes.byref(pol), dummy, 7, dummy, dummy, None) == L.KV_ESHAPE
    a = ctypes.c_void_p(0x100000)
    assert lib.kv_compact_inplace(ctypes.byref(sh), a, ctypes.c_void_p(0x100010), None, dummy, 8, dummy,
                                  None) == L.KV_EINVAL
    assert lib.kv_compact_inplace(ctypes.byref(sh), a, ctypes.c_void_p(0x200000), ctypes.c_void_p(0x100000), dummy, 8,
                                  dummy, None) == L.KV_EINVAL
    assert lib.kv_compact_inplace(ctypes.byref(sh), a, ctypes.c_void_p(0x200008), None, dummy, 8, dummy,
                                  None) == L.KV_EINVAL       # V not 16-byte aligned
    # selector: b_cap below budget or prompt cap, t_cap above the supported maximum, budget < 1
    pol = L.KvPolicy(8, 2, 4, seq)
    assert lib.kv_select_topk(ctypes.byref(sh), ctypes.byref(pol), dummy, dummy, 7, dummy, WS, 1 << 20, None) == L.KV_ESHAPE
    pol = L.KvPolicy(8, 2, 12, seq)
    assert lib.kv_select_topk(ctypes.byref(sh), ctypes.byref(pol), dummy, dummy, 8, dummy, WS, 1 << 20, None) == L.KV_ESHAPE
    pol = L.KvPolicy(8, 2, 4, seq)
    assert lib.kv_select_random(ctypes.byref(huge_sel), ctypes.byref(pol), None, 1, 0, 0, dummy, 8, dummy, WS, 1 << 20, None) == L.KV_ESHAPE
    assert lib.kv_select_topk(ctypes.byref(huge_sel), ctypes.byref(pol), dummy, dummy, 8, dummy, WS, 1 << 20, None) == L.KV_ESHAPE
    assert lib.kv_select_recent(ctypes.byref(huge_sel), ctypes.byref(pol), dummy, 8, dummy, None) == L.KV_ESHAPE
    pol = L.KvPolicy(0, 2, 4, seq)
    assert lib.kv_select_topk(ctypes.byref(sh), ctypes.byref(pol), dummy, dummy, 8, dummy, WS, 1 << 20, None) == L.KV_EINVAL
    # compact: aliasing in/out is rejected
    a = ctypes.c_void_p(0x100000)
    assert lib.kv_compact(ctypes.byref(sh), a, ctypes.c_void_p(0x200000), None, dummy, 8, dummy, a,
                          ctypes.c_void_p(0x300000), None, 8, None) == L.KV_EINVAL


def test_stream_ceiling_validation(lib):
    from eviction_long_reasoning_amd import _lib as L
    a, o = ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x5000)   # never dereferenced
    assert lib.kv_stream_ceiling(None, 131072, o, 1, None) == L.KV_EINVAL
    assert lib.kv_stream_ceiling(a, 131072, None, 0, None) == L.KV_EINVAL
    assert lib.kv_stream_ceiling(ctypes.c_void_p(0x1000008), 131072, o, 1, None) == L.KV_EINVAL   # misaligned
    assert lib.kv_stream_ceiling(a, 131072, ctypes.c_void_p(0x5002), 1, None) == L.KV_EINVAL
    assert lib.kv_stream_ceiling(a, 0, o, 1, None) == L.KV_EINVAL
    assert lib.kv_stream_ceiling(a, 131072 + 4096, o, 1, None) == L.KV_EINVAL                  # not whole 128 KB
    assert lib.kv_stream_ceiling(a, 1 << 48, o, 1, None) == L.KV_ESHAPE


def test_workspace_queries_and_rejections(lib):
    # tri_score and the top-k / random selectors take a caller workspace sized by their queries;
    # a missing, misaligned or short one is rejected before any launch
    from eviction_long_reasoning_amd import _lib as L
    ok = ctypes.c_void_p(0x1000)
    arr = (ctypes.c_int32 * 17)(*[1 << i for i in range(17)])
    sh = L.KvShape(36, 8, 8, 128, 32768, L.KV_BF16, None)
    need_s = lib.kv_score_workspace_bytes(ctypes.byref(sh), 17)
    assert need_s == L.KV_WORKSPACE_HEADER                    # the score stream needs no scratch of its own
    assert lib.kv_score_workspace_bytes(ctypes.byref(sh), 0) == 0
    assert lib.kv_score_workspace_bytes(ctypes.byref(sh), 65) == 0
    assert lib.kv_score_workspace_bytes(None, 17) == 0
    bad = L.KvShape(36, 8, 8, 7, 32768, L.KV_BF16, None)
    assert lib.kv_score_workspace_bytes(ctypes.byref(bad), 17) == 0
    need_k = lib.kv_select_workspace_bytes(ctypes.byref(sh), 3072)
    assert need_k >= L.KV_WORKSPACE_HEADER and need_k % 8 == 0
    assert lib.kv_select_workspace_bytes(ctypes.byref(sh), 0) == 0
    huge = L.KvShape(1, 1, 1, 8, (1 << 26) + 1, L.KV_BF16, None)
    assert lib.kv_select_workspace_bytes(ctypes.byref(huge), 8) == 0
    sh.seq_len = ok
    for ws, nbytes in ((None, 1 << 20), (ctypes.c_void_p(0x7000004), 1 << 20), (WS, need_s - 1)):
        assert lib.tri_score(ctypes.byref(sh), ok, None, ok, None, ok, 1e6, arr, 17, ok, ws, nbytes,
                             None) == L.KV_EWORKSPACE
    pol = L.KvPolicy(3072, 128, 1024, ok)
    for ws, nbytes in ((None, 1 << 30), (ctypes.c_void_p(0x7000004), 1 << 30), (WS, need_k - 1)):
        assert lib.kv_select_topk(ctypes.byref(sh), ctypes.byref(pol), ok, ok, 3072, ok, ws, nbytes,
                                  None) == L.KV_EWORKSPACE
        assert lib.kv_select_random(ctypes.byref(sh), ctypes.byref(pol), None, 1, 0, 0, ok, 3072, ok, ws, nbytes,
                                    None) == L.KV_EWORKSPACE
        assert lib.kv_select_random_shared(ctypes.byref(sh), ctypes.byref(pol), None, 1, 0, ok, 3072, ok, ws,
                                           nbytes, None) == L.KV_EWORKSPACE
    assert "workspace" in lib.kv_status_string(L.KV_EWORKSPACE).decode()
    # the draw's layer index is packed into 16 bits: layer_base + n_layers must stay within it
    for base in (-1, 65536 - 36 + 1):
        assert lib.kv_select_random(ctypes.byref(sh), ctypes.byref(pol), None, 1, 0, base, ok, 3072, ok, WS,
                                    need_k, None) == L.KV_EINVAL


def test_device_check_build_loads_and_reports_itself():
    # the build with device-side precondition checks exports the same entry points and says so
    from eviction_long_reasoning_amd import _lib as L
    from eviction_long_reasoning_amd.build import DEBUG_LIB_PATH, build, build_debug, LIB_PATH
    if not os.path.exists(LIB_PATH):
        build()
    if not os.path.exists(DEBUG_LIB_PATH):
        build_debug()
    dbg = L.open_library(DEBUG_LIB_PATH)
    assert dbg.kv_device_checks() == 1
    assert dbg.kv_version() >> 16 == 2
    for name in _declared_functions():
        assert hasattr(dbg, name), name


def test_gqa_rotated_validation(lib):
    from eviction_long_reasoning_amd import _lib as L
    ok = ctypes.c_void_p(0x1000)
    arr = (ctypes.c_int32 * 1)(1)
    hs, sc, ws = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x900000), ctypes.c_void_p(0xA00000)
    sh = L.KvShape(1, 1, 1, 128, 4096, L.KV_BF16, ok)
    need = lib.kv_score_gqa_workspace_bytes(ctypes.byref(sh), 4)

    def call(shape, paged=None, style=0, group=4, workspace_bytes=None, qbar=ok):
        return lib.tri_score_gqa_rotated(ctypes.byref(shape), ok, None if paged is None else ctypes.byref(paged), style,
                                         group, qbar, None, ok, 1e4, arr, 1, hs, sc, ws,
                                         need if workspace_bytes is None else workspace_bytes, None)
    assert call(sh, group=9) == L.KV_EINVAL                     # groups of at most 8
    assert call(sh, group=0) == L.KV_EINVAL
    assert call(sh, style=5) == L.KV_EINVAL
    assert call(sh, workspace_bytes=need - 8) == L.KV_EWORKSPACE
    assert call(sh, qbar=ctypes.c_void_p(0x1002)) == L.KV_EINVAL
    sh256 = L.KvShape(1, 1, 1, 256, 4096, L.KV_BF16, ok)       # 32 pieces: more than 16 lanes per key
    assert call(sh256, workspace_bytes=1 << 20) == L.KV_ESHAPE
    sh96 = L.KvShape(1, 1, 1, 96, 4096, L.KV_BF16, ok)         # half-split rows must fill whole lanes
    assert call(sh96, style=1) == L.KV_ESHAPE
    assert call(sh, paged=L.KvPaged(ok, 256, 16, 8, 3)) == L.KV_EINVAL     # unknown pool layout
    assert call(sh, paged=L.KvPaged(ok, 2, 16, 8, 0)) == L.KV_ESHAPE       # table shorter than t_cap


def test_misaligned_word_arrays_are_rejected(lib):
    # int32 / fp32 arrays must be 4-byte aligned: one misaligned pointer per entry point
    from eviction_long_reasoning_amd import _lib as L
    ok, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1002)
    arr = (ctypes.c_int32 * 1)(1)
    sh = L.KvShape(1, 1, 1, 128, 4096, L.KV_BF16, ok)
    sh_odd = L.KvShape(1, 1, 1, 128, 4096, L.KV_BF16, odd)
    assert lib.tri_score(ctypes.byref(sh), ok, None, ok, None, ok, 1e4, arr, 1, odd, WS, 1 << 20, None) == L.KV_EINVAL
    assert lib.tri_score(ctypes.byref(sh_odd), ok, None, ok, None, ok, 1e4, arr, 1, ok, WS, 1 << 20, None) == L.KV_EINVAL
    assert lib.tri_score(ctypes.byref(sh), ok, odd, ok, None, ok, 1e4, arr, 1, ok, WS, 1 << 20, None) == L.KV_EINVAL
    assert lib.tri_score_rotated(ctypes.byref(sh), ok, None, 0, ok, None, odd, 1e4, arr, 1, ok, None) == L.KV_EINVAL
    ws = ctypes.c_void_p(0x100000)
    need = lib.kv_score_gqa_workspace_bytes(ctypes.byref(sh), 4)
    assert lib.tri_score_gqa(ctypes.byref(sh), ok, None, 4, ok, None, ok, 1e4, arr, 1, ctypes.c_void_p(0x200002),
                             ctypes.c_void_p(0x300000), ws, need, None) == L.KV_EINVAL
    pol = L.KvPolicy(1024, 64, 128, ok)
    pol_odd = L.KvPolicy(1024, 64, 128, odd)
    assert lib.kv_select_topk(ctypes.byref(sh), ctypes.byref(pol), odd, ok, 1024, ok, WS, 1 << 20, None) == L.KV_EINVAL
    assert lib.kv_select_topk(ctypes.byref(sh), ctypes.byref(pol_odd), ok, ok, 1024, ok, WS, 1 << 20, None) == L.KV_EINVAL
    assert lib.kv_select_random(ctypes.byref(sh), ctypes.byref(pol), None, 1, 0, 0, odd, 1024, ok, WS, 1 << 20, None) == L.KV_EINVAL
    assert lib.kv_select_random(ctypes.byref(sh), ctypes.byref(pol), odd, 1, 0, 0, ok, 1024, ok, WS, 1 << 20, None) == L.KV_EINVAL
    assert lib.kv_select_random_shared(ctypes.byref(sh), ctypes.byref(pol), None, 1, 0, ok, 1024, odd, WS, 1 << 20, None) == L.KV_EINVAL
    assert lib.kv_select_union(ctypes.byref(sh), ctypes.byref(pol), 2, 0, odd, ok, ok, 1024, ok, None) == L.KV_EINVAL
    assert lib.kv_select_recent(ctypes.byref(sh_odd), ctypes.byref(pol), ok, 1024, ok, None) == L.KV_EINVAL
    assert lib.kv_audit_kept(ctypes.byref(sh), ctypes.byref(pol), ok, 1024, ok, odd, None) == L.KV_EINVAL
    assert lib.kv_compact(ctypes.byref(sh), ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000), None, odd, 1024,
                          ok, ctypes.c_void_p(0x3000000), ctypes.c_void_p(0x4000000), None, 1024,
                          None) == L.KV_EINVAL
    assert lib.kv_compact_inplace(ctypes.byref(sh), ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000), odd, ok,
                                  1024, ok, None) == L.KV_EINVAL


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    import eviction_long_reasoning_amd as kv
    with pytest.raises(ValueError):
        kv.tri_score(torch.zeros(1, 1, 1, 4, 8), torch.zeros(1, 1, 8), torch.zeros(1, dtype=torch.int32),
                     torch.zeros(1, dtype=torch.int32), 1e4, [1])


def test_missing_library_raises_instead_of_falling_back():
    # with no built library every call fails loudly; nothing computes on the CPU instead
    import subprocess
    import sys
    code = ("import eviction_long_reasoning_amd._lib as L\n"
            "try:\n    L.load()\nexcept RuntimeError as e:\n    print('raised', 'missing' in str(e))\n")
    env = dict(os.environ, KVEVICT_LIB=os.path.join(ROOT, "no_such_library.so"))
    out = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert out.stdout.strip() == "raised True", out.stdout + out.stderr


def test_product_package_never_imports_the_oracle():
    # the oracle is test infrastructure: no module of the product package may import it
    pkg = os.path.join(ROOT, "eviction_long_reasoning_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            src = open(os.path.join(pkg, name)).read()
            assert not re.search(r"^\s*(from|import)\s+oracle\b", src, flags=re.M), name
