"""tri_score_gqa_noalloc: the grouped-query score without a caller workspace, called through the C
ABI, must give tri_score_gqa's results bit for bit (the same kernels, partial sums in the library's
own device array instead of a workspace) -- on two calls in a row, the second with a smaller input,
so the second call reuses the array the first one filled."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _inputs(seed, L, S, H, G, t_cap, d, dtype, with_pos):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dev = torch.device("cuda:0")
    K = (torch.randn((L, S, H, t_cap, d), generator=g) * 0.3 + 1.0).to(dtype).to(dev)
    qbar = torch.randn((L, H, G, d), generator=g).to(dev)
    seq = torch.randint(1, t_cap + 1, (S,), generator=g, dtype=torch.int32)
    seq[0] = t_cap
    tcur = (seq + torch.randint(0, 50, (S,), generator=g, dtype=torch.int32)).to(dev)
    pos = None
    if with_pos:   # gappy ascending positions
        steps = torch.randint(1, 4, (L, S, H, t_cap), generator=g, dtype=torch.int32)
        pos = torch.cumsum(steps, dim=-1, dtype=torch.int32).to(dev)
        tcur = (pos[0, :, 0, -1] + 7).to(torch.int32).contiguous()
    return K, qbar, tcur, seq.to(dev), pos


def _call_noalloc(lib, K, qbar, tcur, seq, theta, deltas, pos, out, head_out):
    from eviction_long_reasoning_amd import _lib as L
    Lq, S, H, t_cap, d = K.shape
    G = qbar.shape[2]
    shape = L.KvShape(Lq, S, H, d, t_cap, L.KV_BF16 if K.dtype == torch.bfloat16 else L.KV_F32,
                      ctypes.c_void_p(seq.data_ptr()))
    arr = (ctypes.c_int32 * len(deltas))(*deltas)
    st = lib.tri_score_gqa_noalloc(ctypes.byref(shape), ctypes.c_void_p(K.data_ptr()),
                                   None if pos is None else ctypes.c_void_p(pos.data_ptr()), G,
                                   ctypes.c_void_p(qbar.data_ptr()), None, ctypes.c_void_p(tcur.data_ptr()),
                                   float(theta), arr, len(deltas), ctypes.c_void_p(head_out.data_ptr()),
                                   ctypes.c_void_p(out.data_ptr()),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_matches_workspace_form_on_two_calls():
    import eviction_long_reasoning_amd as kv
    from eviction_long_reasoning_amd import _lib as L
    lib = kv.load_library()
    cases = [  # the second call is smaller than the first
        dict(seed=11, L=2, S=3, H=4, G=4, t_cap=5000, d=128, dtype=torch.bfloat16, with_pos=False, theta=1e6),
        dict(seed=12, L=1, S=2, H=2, G=8, t_cap=1500, d=64, dtype=torch.bfloat16, with_pos=True, theta=1e4),
    ]
    deltas = [1 << i for i in range(17)]
    for c in cases:
        K, qbar, tcur, seq, pos = _inputs(c["seed"], c["L"], c["S"], c["H"], c["G"], c["t_cap"], c["d"], c["dtype"],
                                          c["with_pos"])
        print(f"noalloc case seed={c['seed']} L={c['L']} S={c['S']} H={c['H']} G={c['G']} t_cap={c['t_cap']}",
              flush=True)
        need = kv.gqa_workspace_bytes(c["L"], c["S"], c["H"], c["t_cap"], c["d"], c["dtype"], c["G"])
        assert 0 < need <= lib.kv_score_gqa_noalloc_max_bytes()
        z_ref, raw_ref = kv.tri_score_gqa(K, qbar, tcur, seq, c["theta"], deltas, pos=pos)
        out = torch.full_like(z_ref, float("nan"))
        head_out = torch.full_like(raw_ref, float("nan"))
        st = _call_noalloc(lib, K, qbar, tcur, seq, c["theta"], deltas, pos, out, head_out)
        assert st == L.KV_OK, lib.kv_status_string(st)
        torch.cuda.synchronize()
        T = seq.cpu().numpy()
        for s in range(c["S"]):   # slots past T_s are not written by either form
            assert torch.equal(out[:, s, :, :T[s]], z_ref[:, s, :, :T[s]]), f"z, seq {s}"
            assert torch.equal(head_out[:, s, :, :, :T[s]], raw_ref[:, s, :, :, :T[s]]), f"raw, seq {s}"


def test_noalloc_rejects_shapes_beyond_its_array():
    import eviction_long_reasoning_amd as kv
    from eviction_long_reasoning_amd import _lib as L
    lib = kv.load_library()
    big = L.KvShape(36, 8, 8, 128, 32768, L.KV_BF16, ctypes.c_void_p(0x1000))   # 18.9 MB of partial sums at G=16
    assert lib.kv_score_gqa_workspace_bytes(ctypes.byref(big), 16) > lib.kv_score_gqa_noalloc_max_bytes()
    arr = (ctypes.c_int32 * 1)(1)
    d = ctypes.c_void_p(0x100000)
    st = lib.tri_score_gqa_noalloc(ctypes.byref(big), d, None, 16, d, None, d, 1e6, arr, 1, ctypes.c_void_p(0x200000),
                                   ctypes.c_void_p(0x300000), None)
    assert st == L.KV_EWORKSPACE
