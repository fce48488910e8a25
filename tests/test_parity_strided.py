"""GPU parity of the general forward interface (fa_fwd_strided through the C ABI, and
fa_fwd at d = 16, 32) against the fp64 oracles.

Tolerances as for fa_fwd (max abs error): O 1e-5 / L 1e-4 for fp32, O 2e-2 / L 1e-2
for bf16. Cross-attention (Nq != Nk) is compared with ``oracle.attention_cross``
(top-left causal alignment); strided layouts are compared on contiguous copies of
the same values.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import default_scale, make_qkv, make_qkv_cross, sample_rows

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-2, 1e-2)}
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def fa():
    import tiled_online_softmax_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return tiled_online_softmax_amd


def _compare(O, L, Oref, Lref, dtype, label):
    o = O.double().cpu().numpy()
    lse = L.double().cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{label}: non-finite output"
    eo = float(np.abs(o - Oref).max())
    el = float(np.abs(lse - Lref).max())
    otol, ltol = TOL[dtype]
    print(f"[parity-strided] {label} max|dO|={eo:.3e} (tol {otol}) max|dL|={el:.3e} (tol {ltol})", flush=True)
    assert eo <= otol and el <= ltol, f"{label}: O error {eo} (tol {otol}), L error {el} (tol {ltol})"


def _oracle_cross(q, k, v, causal, scale):
    return oracle.attention_cross(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)


CROSS = [(100, 300), (300, 100), (1, 257), (257, 1), (33, 65), (128, 64), (64, 200)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", CROSS)
def test_cross_attention(fa, Nq, Nk, causal, d, dtype):
    q, k, v = make_qkv_cross(1, 2, Nq, Nk, d, dtype, seed=Nq * 7 + Nk + d)
    scale = default_scale(d)
    O, L = fa.forward_strided(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    Oref, Lref = _oracle_cross(q, k, v, causal, scale)
    _compare(O, L, Oref, Lref, dtype, f"{dtype} d={d} {Nq}x{Nk} causal={causal}")


@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(100, 300), (300, 100), (1, 257), (257, 1), (65, 65)])
def test_cross_attention_large_grid_bf16(fa, Nq, Nk, causal, d):
    """The bf16 kernel that gives each wave all keys of its 32 rows (grids above 192
    workgroups of 128 rows, 384 when causal), through fa_fwd_strided with [B, N, H, d]
    storage: two heads repeated to 400 in one launch, compared with the oracle on the
    first two and bitwise among the repeats."""
    q, k, v = make_qkv_cross(1, 2, Nq, Nk, d, "bf16", seed=5000 + Nq * 7 + Nk + d)
    scale = default_scale(d)
    Oref, Lref = _oracle_cross(q, k, v, causal, scale)
    qd, kd, vd = (t.repeat(1, 200, 1, 1).transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for t in (q, k, v))
    O, L = fa.forward_strided(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    _compare(O[:, :2], L[:, :2], Oref, Lref, "bf16", f"x200 bshd d={d} {Nq}x{Nk} causal={causal}")
    for j in range(1, 200):
        assert torch.equal(O[:, 2 * j:2 * j + 2], O[:, :2]) and torch.equal(L[:, 2 * j:2 * j + 2], L[:, :2])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [16, 32])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 31, 64, 65, 200, 513])
def test_small_head_dims(fa, N, causal, d, dtype):
    """fa_fwd (contiguous) at d = 16 and 32, including ragged lengths."""
    q, k, v = make_qkv(2, 2, N, d, dtype, seed=N + d)
    scale = default_scale(d)
    O, L = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
    _compare(O, L, Oref, Lref, dtype, f"{dtype} d={d} N={N} causal={causal}")


def _layouts(B, H, Nq, Nk, d, dtype, seed):
    """(label, q, k, v) device views of the same values in several strided layouts,
    plus the contiguous CPU tensors they hold."""
    q, k, v = make_qkv_cross(B, H, Nq, Nk, d, dtype, seed=seed)
    out = []
    # [B, N, H, d] storage viewed as [B, H, N, d] (row stride H d, head stride d)
    bshd = [t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for t in (q, k, v)]
    out.append(("bshd", *bshd))
    # rows padded to d + 16 elements (a slice of a wider array)
    def padded(t):
        w = torch.zeros(t.shape[:-1] + (d + 16,), dtype=t.dtype)
        w[..., :d] = t
        return w.to(DEV)[..., :d]
    out.append(("padded_rows", *(padded(t) for t in (q, k, v))))
    # heads of every batch stored with a gap after each head
    def head_gap(t):
        n = t.shape[2]
        w = torch.zeros((t.shape[0], t.shape[1], n + 3, d), dtype=t.dtype)
        w[:, :, :n] = t
        return w.to(DEV)[:, :, :n]
    out.append(("head_gap", *(head_gap(t) for t in (q, k, v))))
    return (q, k, v), out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_strided_layouts(fa, d, causal, dtype):
    (q, k, v), layouts = _layouts(2, 3, 150, 230, d, dtype, seed=900 + d)
    scale = default_scale(d)
    Oref, Lref = _oracle_cross(q, k, v, causal, scale)
    for label, qd, kd, vd in layouts:
        assert not (qd.is_contiguous() and kd.is_contiguous())
        O, L = fa.forward_strided(qd, kd, vd, causal=causal, scale=scale)
        torch.cuda.synchronize()
        _compare(O, L, Oref, Lref, dtype, f"{label} {dtype} d={d} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_broadcast_kv_heads(fa, dtype):
    """One K, V head shared by all 4 query heads (head stride 0) equals the oracle on
    the repeated heads."""
    B, H, Nq, Nk, d = 2, 4, 120, 333, 64
    q, _, _ = make_qkv_cross(B, H, Nq, Nk, d, dtype, seed=77)
    _, k1, v1 = make_qkv_cross(B, 1, Nq, Nk, d, dtype, seed=78)
    scale = default_scale(d)
    kd = k1.to(DEV).expand(B, H, Nk, d)
    vd = v1.to(DEV).expand(B, H, Nk, d)
    assert kd.stride(1) == 0
    O, L = fa.forward_strided(q.to(DEV), kd, vd, causal=True, scale=scale)
    torch.cuda.synchronize()
    Oref, Lref = _oracle_cross(q, k1.expand(B, H, Nk, d), v1.expand(B, H, Nk, d), True, scale)
    _compare(O, L, Oref, Lref, dtype, f"broadcast {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_contiguous_strided_equals_fa_fwd(fa, causal, dtype):
    """Contiguous strides and Nq = Nk: the same kernel, bitwise the same results."""
    q, k, v = (t.to(DEV) for t in make_qkv(2, 4, 777, 128, dtype, seed=5))
    O1, L1 = fa.forward(q, k, v, causal=causal)
    O2, L2 = fa.forward_strided(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_strided_rejects_bad_layout(fa):
    """A non-unit stride along d is refused by the binding; an overlapping O by the library."""
    q, k, v = (t.to(DEV) for t in make_qkv(1, 2, 64, 64, "bf16", seed=1))
    with pytest.raises(ValueError):
        fa.forward_strided(q.transpose(2, 3), k, v)
    O = torch.empty((1, 2, 64, 64), dtype=q.dtype, device=DEV)
    L = torch.empty((1, 2, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_strided(q, k, v, O.expand(1, 2, 64, 64)[:, :1].expand(1, 2, 64, 64), L, False, 0.125)
    assert e.value.status == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("layout", ["contiguous", "bshd"])
def test_cross_workload_full_size(fa, layout):
    """The benchmarked cross-attention workload at full size (B=4, H=16, 1024 queries,
    4096 keys, d=128), in the launch the benchmark times; two heads against the oracle."""
    from workloads import WORKLOADS

    w = WORKLOADS["cross_bf16_b4h16q1024k4096d128"]
    q, k, v = w.make()
    if layout == "bshd":
        qd, kd, vd = (t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for t in (q, k, v))
    else:
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    O, L = fa.forward_strided(qd, kd, vd, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (3, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        Oref, Lref = _oracle_cross(q[sl], k[sl], v[sl], w.causal, w.scale)
        _compare(O[sl], L[sl], Oref, Lref, "bf16", f"cross workload {layout} head ({b},{h})")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [16, 128])
def test_strided_outputs_and_lse(fa, d, dtype):
    """O written into a [B, N, H, d] view and L into every other float of a wider buffer,
    with Nq > Nk, causal (queries past Nk see every key)."""
    B, H, Nq, Nk = 2, 3, 190, 70
    q, k, v = make_qkv_cross(B, H, Nq, Nk, d, dtype, seed=4000 + d)
    scale = default_scale(d)
    O = torch.full((B, Nq, H, d), float("nan"), dtype=q.dtype, device=DEV).transpose(1, 2)
    Lbuf = torch.full((B, H, 2 * Nq), float("nan"), dtype=torch.float32, device=DEV)
    L = Lbuf[:, :, ::2]
    fa.fa_fwd_strided(q.to(DEV), k.to(DEV), v.to(DEV), O, L, True, scale)
    torch.cuda.synchronize()
    Oref, Lref = _oracle_cross(q, k, v, True, scale)
    _compare(O, L, Oref, Lref, dtype, f"strided O/L {dtype} d={d}")
    assert torch.isnan(Lbuf[:, :, 1::2]).all(), "L stride: the skipped floats were written"


def test_strided_zero_batch_stride_inputs(fa):
    """K and V shared by both batches (batch stride 0) and Q heads broadcast from one head."""
    B, H, Nq, Nk, d = 2, 4, 96, 160, 64
    q1, k1, v1 = make_qkv_cross(1, 1, Nq, Nk, d, "bf16", seed=4100)
    qd = q1.to(DEV).expand(B, H, Nq, d)
    kd = k1.to(DEV).expand(B, H, Nk, d)
    vd = v1.to(DEV).expand(B, H, Nk, d)
    O = torch.empty((B, H, Nq, d), dtype=q1.dtype, device=DEV)
    L = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
    fa.fa_fwd_strided(qd, kd, vd, O, L, False, default_scale(d))
    torch.cuda.synchronize()
    Oref, Lref = _oracle_cross(q1, k1, v1, False, default_scale(d))
    for b in range(B):
        for h in range(H):
            _compare(O[b:b + 1, h:h + 1], L[b:b + 1, h:h + 1], Oref, Lref, "bf16", f"broadcast ({b},{h})")


# The largest sequence lengths the entry points accept (row indices stay in 32 bits; byte
# offsets of rows past 2^24 x 64 elements do not).
MAX_ROWS = 1 << 24


def _max_rows_check(fa, Nq, Nk, causal, seed, n_sample):
    d = 64
    label = f"bf16 d={d} Nq={Nq} Nk={Nk} causal={causal}"
    print(f"[parity-strided] generating {label}", flush=True)
    q, k, v = make_qkv_cross(1, 1, Nq, Nk, d, "bf16", seed=seed)
    scale = default_scale(d)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    O = torch.full_like(qd, float("nan"))
    L = torch.full((1, 1, Nq), float("nan"), dtype=torch.float32, device=DEV)
    print(f"[parity-strided] running {label}", flush=True)
    fa.fa_fwd_strided(qd, kd, vd, O, L, causal, scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(L).all()), f"{label}: rows no workgroup wrote"
    rows = sorted(set(sample_rows(Nq, n_sample, seed)) | {Nq - 1, Nq - 2, max(Nq - 129, 0), Nq // 2})
    o, lse = O[:, :, rows].cpu(), L[:, :, rows].cpu()
    del qd, kd, vd, O, L
    # Rows are independent: the oracle takes the sampled query rows against every key. With the
    # top-left causal mask, row i >= Nk - 1 sees every key; rows below Nk are compared as a
    # causal prefix (local and global row indices agree there).
    head = [r for r in rows if causal and r < Nk]
    tail = [r for r in rows if r not in head]
    Oref = np.empty((1, 1, len(rows), d))
    Lref = np.empty((1, 1, len(rows)))
    if tail:
        ot, lt = oracle.attention_cross(q[:, :, tail].double().numpy(), k.double().numpy(), v.double().numpy(),
                                        False, scale)
        for j, r in enumerate(tail):
            Oref[:, :, rows.index(r)], Lref[:, :, rows.index(r)] = ot[:, :, j], lt[:, :, j]
    if head:
        n = head[-1] + 1
        oh, lh = oracle.attention_cross(q[:, :, :n].double().numpy(), k[:, :, :n].double().numpy(),
                                        v[:, :, :n].double().numpy(), True, scale)
        for r in head:
            Oref[:, :, rows.index(r)], Lref[:, :, rows.index(r)] = oh[:, :, r], lh[:, :, r]
    _compare(o, lse, Oref, Lref, "bf16", f"{label}, {len(rows)} sampled rows")


@pytest.mark.parametrize("causal", [False, True])
def test_max_query_rows(fa, causal):
    """2^24 query rows (the largest Nq accepted) against 64 keys: every row is written, and
    sampled rows up to the last one match the oracle."""
    _max_rows_check(fa, MAX_ROWS, 64, causal, seed=77, n_sample=24)


@pytest.mark.parametrize("causal", [False, True])
def test_max_key_rows(fa, causal):
    """256 query rows against 2^24 keys (the largest Nk accepted): sampled rows match the
    oracle (non-causal: every key; causal: the top-left prefix)."""
    _max_rows_check(fa, 256, MAX_ROWS, causal, seed=78, n_sample=8)
