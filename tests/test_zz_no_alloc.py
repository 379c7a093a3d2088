"""GPU check of the allocation-free entry point sparse_attn_windowed_static
(its scratch in the library's static device array) against
sparse_attn_windowed (the caller's workspace), through the C ABI.

Both run the same kernels in the same order, so the outputs must agree bit
for bit, which is inside the bf16 output bar (2e-3 max abs). Calls come in a
row on one GPU, the second on a smaller layer, with and without lse_sparse
(without it the running LSE lives in the static array), and with token and
64-token key-block supports; a second round repeats them after the larger
layer has left its contents in the array.
"""
import numpy as np
import pytest

from synth import random_inputs
from tests.gpu_helpers import TOL_OUT, upload
from tests.test_gpu_windowed import _token_supports

pytestmark = pytest.mark.gpu


def _block_supports(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.full((n, k), -1, dtype=np.int32)
    cnt = np.zeros(n, dtype=np.int32)
    for i in range(n):
        nb = i // 64 + 1
        ids = np.sort(rng.choice(nb, min(k, nb), replace=False))
        idx[i, : ids.size] = ids
        cnt[i] = ids.size
    return idx, cnt


def _case(amtk, n, seed, key_block, want_lse):
    import torch
    x = random_inputs(n, 32, 8, 128, "bf16", seed=seed, sink=True)
    d = upload(x, "bf16")
    idx, cnt = (_token_supports(n, 96, seed + 1) if key_block == 1
                else _block_supports(n, 12, seed + 1))
    ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    o_ref, l_ref = amtk.sparse_attn_windowed(d["q"], d["k"], d["v"], ti, tc, key_block,
                                             want_lse=want_lse)
    o_st, l_st = amtk.sparse_attn_windowed_static(d["q"], d["k"], d["v"], ti, tc, key_block,
                                                  want_lse=want_lse)
    torch.cuda.synchronize()
    err = float((o_st - o_ref).abs().max())
    assert err <= TOL_OUT["bf16"], f"n={n} kb={key_block}: max abs {err}"
    assert torch.equal(o_st, o_ref), f"n={n} kb={key_block}: outputs differ (max abs {err})"
    if want_lse:
        assert torch.equal(l_st, l_ref), f"n={n} kb={key_block}: lse differs"


@pytest.mark.parametrize("rnd", [0, 1])
def test_static_scratch_matches_the_workspace_form(gpu_lib, rnd):
    # 20000 tokens: three key windows; 9000: two (a smaller call right after)
    for n, seed, kb, want_lse in ((20000, 101, 1, False), (9000, 103, 1, False),
                                  (20000, 105, 64, True), (9000, 107, 1, True)):
        print(f"[no_alloc] round {rnd}: n={n} key_block={kb} want_lse={want_lse}", flush=True)
        _case(gpu_lib, n, seed + rnd, kb, want_lse)


def test_static_scratch_rejects_layers_beyond_its_size(gpu_lib):
    import ctypes
    import torch
    from sparse_long_context_causal_amd import _abi
    n = 400000                      # needs more scratch than the static array holds
    q = torch.zeros((8, 32, 128), dtype=torch.bfloat16, device="cuda")
    ad = _abi.AttnDesc(n, 32, 8, 128, _abi.AMTK_BF16, 1, 0.0)
    lib = gpu_lib.load()
    p = q.data_ptr()
    rc = lib.sparse_attn_windowed_static(ctypes.byref(ad), 1, 16, p, p, p, p, p, p, None, None)
    assert rc == _abi.AMTK_E_WORKSPACE
