"""fa_bwd_noalloc (the backward pass on the library's static workspace) against fa_bwd
(the caller's workspace), through the C ABI: two calls in a row, the second on a smaller
problem, so the second runs on a workspace holding the first call's values. The kernels
are the same, so the gradients must be bitwise equal."""

import pytest
import torch

from workloads import default_scale, make_qkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def fa():
    import tiled_online_softmax_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return tiled_online_softmax_amd


def _case(fa, B, H, N, d, causal, dtype, seed, side_stream=False):
    q, k, v = make_qkv(B, H, N, d, dtype, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn((B, H, N, d), generator=g).to(q.dtype)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    scale = default_scale(d)
    O, L = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    ref = [torch.empty_like(qd) for _ in range(3)]
    work = torch.empty(2 * B * H * N, dtype=torch.float32, device=DEV)
    fa.fa_bwd(qd, kd, vd, O, L, dod, *ref, work, B, H, N, d, causal, scale)
    got = [torch.full_like(qd, float("nan")) for _ in range(3)]
    # On a stream of its own (a non-null handle: the library takes the GPU from the
    # stream), ordered after the work above.
    side = torch.cuda.Stream(DEV) if side_stream else None
    if side is not None:
        side.wait_stream(torch.cuda.current_stream(DEV))
    stream = (side or torch.cuda.current_stream(DEV)).cuda_stream
    st = fa.raw_fa_bwd_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), O.data_ptr(), L.data_ptr(),
                               dod.data_ptr(), *(t.data_ptr() for t in got), B, H, N, d, int(causal), scale,
                               stream, fa.FA_DTYPE_BF16 if dtype == "bf16" else fa.FA_DTYPE_F32)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"{name}: fa_bwd_noalloc differs from fa_bwd"


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_fa_bwd(fa, dtype, d, causal):
    print(f"[no-alloc] {dtype} d={d} causal={causal}", flush=True)
    _case(fa, 2, 4, 1000, d, causal, dtype, seed=5100 + d)   # fills 16000 workspace floats
    _case(fa, 1, 2, 129, d, causal, dtype, seed=5200 + d)    # then a smaller problem on the same workspace


def test_noalloc_on_side_stream(fa):
    print("[no-alloc] bf16 d=128 causal on a side stream", flush=True)
    _case(fa, 1, 4, 300, 128, True, "bf16", seed=5300, side_stream=True)


def test_noalloc_size_limit(fa):
    """2 * B * H * N floats must fit in the 2^21-float workspace: one row more is refused
    before anything is enqueued."""
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device=DEV)
    L = torch.zeros(1, 1, 8, dtype=torch.float32, device=DEV)
    p = [x.data_ptr()] * 4 + [L.data_ptr(), x.data_ptr()]
    outs = [torch.empty_like(x) for _ in range(3)]
    st = fa.raw_fa_bwd_noalloc(*p, *(t.data_ptr() for t in outs), 1, 1, (1 << 20) + 1, 64, 0, 0.125,
                               torch.cuda.current_stream(DEV).cuda_stream, fa.FA_DTYPE_BF16)
    assert st == fa.FA_ERR_SCRATCH_LIMIT
