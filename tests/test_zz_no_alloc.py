"""rax_decode_attention_noalloc (the decode attention that allocates nothing) against
rax_decode_attention with a caller workspace, through the C ABI: two calls in a row, the
second smaller, outputs equal element by element and within the bf16 tolerance of fp64
attention over each request's keys (oracle.attention.attend)."""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(seed, B, h_q, h_kv, P, own_max, S=1 << 17, d=128):
    gen = torch.Generator().manual_seed(seed)
    perm = torch.randperm(S, generator=gen).numpy().astype(np.int32)
    own = [int(x) for x in torch.randint(0, own_max + 1, (B,), generator=gen)]
    lens = np.array([P + n + 1 for n in own], dtype=np.int32)
    rtt = np.full((B + 1, int(lens.max()) + 1), -1, dtype=np.int32)
    rows = np.arange(B, dtype=np.int32)[::-1].copy() + 1
    used = P
    for i in range(B):
        rtt[rows[i], :P] = perm[:P]
        rtt[rows[i], P:lens[i]] = perm[used: used + lens[i] - P]
        used += lens[i] - P
    assert used <= S
    hints = np.full(B, P, dtype=np.int32)
    k_pool = torch.randn((S, h_kv, d), generator=gen).to(torch.bfloat16)
    v_pool = torch.randn((S, h_kv, d), generator=gen).to(torch.bfloat16)
    q = torch.randn((B, h_q, d), generator=gen).to(torch.bfloat16)
    return q, k_pool, v_pool, rtt, rows, lens, hints


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_decode_equals_workspace_decode(order):
    from oracle.attention import attend
    from prefix_shared_kv_extend_amd import _lib
    cases = [(5, 120, 32, 8, 700, 1500), (6, 37, 8, 8, 90, 300)]
    for seed, B, h_q, h_kv, P, own_max in cases:
        say(f"noalloc decode: {B} requests, {h_q}/{h_kv} heads, {P}-key shared prefix, own up to {own_max}")
        q, k_pool, v_pool, rtt, rows, lens, hints = _case(seed, B, h_q, h_kv, P, own_max)
        dev = lambda x: torch.as_tensor(x).cuda()
        args = [dev(q), dev(k_pool), dev(v_pool), dev(rtt), dev(rows), dev(lens), int(lens.max())]
        need = _lib.attention_workspace_bytes(True, B, h_q, h_kv, 128, int(lens.max()))
        assert 0 < need <= 64 << 20
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        o_ws = torch.empty((B, h_q, 128), dtype=torch.float32, device="cuda")
        o_na = torch.full_like(o_ws, float("nan"))
        _lib.decode_attention(*args, o_ws, workspace=ws, shared_len=dev(hints))
        _lib.decode_attention_noalloc(*args, o_na, shared_len=dev(hints))
        torch.cuda.synchronize()
        assert _lib.device_errors() == 0
        a, b = o_ws.cpu().numpy(), o_na.cpu().numpy()
        assert np.array_equal(a, b), f"max diff {np.abs(a - b).max()}"
        kf, vf, qf = k_pool.float().numpy(), v_pool.float().numpy(), q.float().numpy()
        worst = 0.0
        for i in range(0, B, max(1, B // 40)):
            sl = rtt[rows[i], : lens[i]]
            err = float(np.abs(b[i] - attend(qf[i], kf[sl], vf[sl])).max())
            worst = max(worst, err)
            assert err <= 1e-2, f"request {i}: max abs err {err:.3g}"
        say(f"  identical to the workspace call; worst max-abs vs fp64 {worst:.3g}")


def test_noalloc_rejects_layouts_beyond_its_array():
    """A layout larger than the 64 MiB array is refused before anything runs."""
    from prefix_shared_kv_extend_amd import _lib
    say("noalloc decode: a 60000-key, 256-request layout is refused")
    B, h_q, h_kv, d, L = 256, 32, 8, 128, 60000
    assert _lib.attention_workspace_bytes(True, B, h_q, h_kv, d, L) > 64 << 20
    q = torch.zeros((B, h_q, d), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((16, h_kv, d), dtype=torch.bfloat16, device="cuda")
    rtt = torch.zeros((B, 16), dtype=torch.int32, device="cuda")
    idx = torch.zeros(B, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(_lib.RaxError):
        _lib.decode_attention_noalloc(q, pool, pool, rtt, idx, idx, L, o)
    torch.cuda.synchronize()
    assert _lib.device_errors() == 0
