"""The build with device-side precondition checks (libkvevict_debug.so) reports broken device data in
the workspace status word, and computes the same results as the release build; the release build
never touches the word. Every kernel clamps lengths into the validated ranges, so the broken inputs
below are safe to run: they only set bits."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _libs():
    from eviction_long_reasoning_amd import _lib as L
    from eviction_long_reasoning_amd.build import DEBUG_LIB_PATH
    if not os.path.exists(DEBUG_LIB_PATH):
        pytest.fail("libkvevict_debug.so is not built")
    return L, L.load(), L.open_library(DEBUG_LIB_PATH)


P_ = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
STREAM = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _score(L, lib, K, qbar, tcur, seq, pos, ws):
    Lq, S, H, T, d = K.shape
    sh = L.KvShape(Lq, S, H, d, T, L.KV_F32, P_(seq))
    out = torch.full((Lq, S, H, T), float("nan"), device=DEV)
    arr = (ctypes.c_int32 * 3)(1, 4, 16)
    st = lib.tri_score(ctypes.byref(sh), P_(K), P_(pos), P_(qbar), None, P_(tcur), 1e4, arr, 3, P_(out), P_(ws),
                       ws.numel(), STREAM())
    assert st == L.KV_OK, st
    return out


def _topk(L, lib, scores, seq, plen, pcap, ws):
    Lq, S, H, T = scores.shape
    sh = L.KvShape(Lq, S, H, 0, T, 0, P_(seq))
    po = L.KvPolicy(64, 8, pcap, P_(plen))
    b_cap = max(64, pcap)
    kept = torch.empty((Lq, S, H, b_cap), dtype=torch.int32, device=DEV)
    nk = torch.empty((S,), dtype=torch.int32, device=DEV)
    st = lib.kv_select_topk(ctypes.byref(sh), ctypes.byref(po), P_(scores), P_(kept), b_cap, P_(nk), P_(ws),
                            ws.numel(), STREAM())
    assert st == L.KV_OK, st
    return kept, nk


def _random(L, lib, shape4, seq, plen, pcap, pos, ws):
    Lq, S, H, T = shape4
    sh = L.KvShape(Lq, S, H, 0, T, 0, P_(seq))
    po = L.KvPolicy(64, 8, pcap, P_(plen))
    b_cap = max(64, pcap)
    kept = torch.empty((Lq, S, H, b_cap), dtype=torch.int32, device=DEV)
    nk = torch.empty((S,), dtype=torch.int32, device=DEV)
    st = lib.kv_select_random(ctypes.byref(sh), ctypes.byref(po), P_(pos), 9, 2, 0, P_(kept), b_cap, P_(nk),
                              P_(ws), ws.numel(), STREAM())
    assert st == L.KV_OK, st
    return kept, nk


def _status(ws):
    torch.cuda.synchronize()
    return int(ws[:4].view(torch.int32).item())


def test_status_word_flags_and_results():
    L, rel, dbg = _libs()
    assert rel.kv_device_checks() == 0 and dbg.kv_device_checks() == 1
    g = torch.Generator(device="cpu")
    g.manual_seed(3)
    Lq, S, H, T, d = 2, 3, 2, 300, 64
    K = torch.randn((Lq, S, H, T, d), generator=g).to(DEV)
    qbar = torch.randn((Lq, H, d), generator=g).to(DEV)
    seq = torch.tensor([300, 250, 120], dtype=torch.int32, device=DEV)
    plen = torch.tensor([16, 40, 8], dtype=torch.int32, device=DEV)
    tcur = torch.tensor([300, 250, 120], dtype=torch.int32, device=DEV)
    pos = torch.arange(T, dtype=torch.int32, device=DEV).mul(2).expand(Lq, S, H, T).contiguous()
    ws = torch.zeros((4096,), dtype=torch.uint8, device=DEV)

    # valid data: no bit set, and both builds compute the same scores and keep-sets
    print("device checks: valid inputs", flush=True)
    s_dbg = _score(L, dbg, K, qbar, tcur, seq, pos, ws)
    k_dbg, n_dbg = _topk(L, dbg, s_dbg, seq, plen, 40, ws)
    r_dbg, rn_dbg = _random(L, dbg, (Lq, S, H, T), seq, plen, 40, pos, ws)
    assert _status(ws) == 0
    s_rel = _score(L, rel, K, qbar, tcur, seq, pos, ws)
    k_rel, n_rel = _topk(L, rel, s_rel, seq, plen, 40, ws)
    r_rel, rn_rel = _random(L, rel, (Lq, S, H, T), seq, plen, 40, pos, ws)
    torch.cuda.synchronize()
    for s in range(S):
        Ts = int(seq[s])
        assert torch.equal(s_dbg[:, s, :, :Ts], s_rel[:, s, :, :Ts])
    assert torch.equal(k_dbg, k_rel) and torch.equal(n_dbg, n_rel)
    assert torch.equal(r_dbg, r_rel) and torch.equal(rn_dbg, rn_rel)

    # a length past t_cap (clamped by the kernels)
    print("device checks: length past t_cap", flush=True)
    bad_seq = torch.tensor([300, 301 + 50, 120], dtype=torch.int32, device=DEV)
    _score(L, dbg, K, qbar, tcur, bad_seq, None, ws)
    assert _status(ws) == L.KV_DEV_SEQ_LEN
    ws.zero_()
    _topk(L, dbg, s_dbg, bad_seq, plen, 40, ws)
    assert _status(ws) == L.KV_DEV_SEQ_LEN
    ws.zero_()

    # a prompt length past the prompt cap, and a negative one (selectors)
    print("device checks: prompt length outside [0, prompt_cap]", flush=True)
    for bad in ([16, 41, 8], [16, 40, -3]):
        _topk(L, dbg, s_dbg, seq, torch.tensor(bad, dtype=torch.int32, device=DEV), 40, ws)
        assert _status(ws) == L.KV_DEV_PROMPT_LEN
        ws.zero_()

    # positions that do not ascend over one head's valid slots
    print("device checks: positions out of order", flush=True)
    bad_pos = pos.clone()
    bad_pos[1, 2, 1, 50] = bad_pos[1, 2, 1, 49]
    _score(L, dbg, K, qbar, tcur, seq, bad_pos, ws)
    assert _status(ws) == L.KV_DEV_POS_ORDER
    ws.zero_()
    _random(L, dbg, (Lq, S, H, T), seq, plen, 40, bad_pos, ws)
    assert _status(ws) == L.KV_DEV_POS_ORDER
    ws.zero_()
    # past the head's valid slots the order does not matter
    late = pos.clone()
    late[1, 2, 1, 200] = 0    # sequence 2 holds 120 valid slots
    _score(L, dbg, K, qbar, tcur, seq, late, ws)
    assert _status(ws) == 0

    # several flags accumulate; the release build never writes the word
    print("device checks: accumulation and the release build", flush=True)
    _topk(L, dbg, s_dbg, bad_seq, torch.tensor([16, 41, 8], dtype=torch.int32, device=DEV), 40, ws)
    assert _status(ws) == (L.KV_DEV_SEQ_LEN | L.KV_DEV_PROMPT_LEN)
    ws.zero_()
    _score(L, rel, K, qbar, tcur, bad_seq, bad_pos, ws)
    _topk(L, rel, s_rel, bad_seq, torch.tensor([16, 41, 8], dtype=torch.int32, device=DEV), 40, ws)
    assert _status(ws) == 0
