"""HIP path vs the fp64 oracle, element by element (needs an MI355X).

Tolerances (max abs error): O 1e-5 / L 1e-4 for fp32, O 2e-2 / L 1e-2 for bf16.
Every workload is compared with the oracle on every row of every head; the two large
causal workloads run at full size in the launch configuration the benchmark times (the
oracle evaluates them head by head), and their outputs are also checked for properties
that hold at every row.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, default_scale, make_qkv

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-2, 1e-2)}


@pytest.fixture(scope="module")
def fa():
    import tiled_online_softmax_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return tiled_online_softmax_amd


def _run(fa, q, k, v, causal, scale, stream=None):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    O, L = fa.forward(qd, kd, vd, causal=causal, scale=scale, stream=stream)
    torch.cuda.synchronize()
    return O, L


def _errors(O, L, Oref, Lref, rows=None):
    o = O.double().cpu().numpy()
    l = L.double().cpu().numpy()
    if rows is not None:
        o = o[:, :, rows]
        l = l[:, :, rows]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), "non-finite output"
    return float(np.max(np.abs(o - Oref))), float(np.max(np.abs(l - Lref)))


def _check(fa, q, k, v, causal, scale, dtype, rows=None, label="", tol=None):
    O, L = _run(fa, q, k, v, causal, scale)
    Oref, Lref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                  causal, scale, rows=rows)
    eo, el = _errors(O, L, Oref, Lref, rows)
    otol, ltol = tol or TOL[dtype]
    print(f"[parity] {label} max|dO|={eo:.3e} (tol {otol}) max|dL|={el:.3e} (tol {ltol})", flush=True)
    assert eo <= otol, f"{label}: O error {eo} > {otol}"
    assert el <= ltol, f"{label}: L error {el} > {ltol}"
    return O, L


@pytest.mark.parametrize("name", ["single_head_f32", "batch8_f32", "ragged_wide_logits_bf16_n1000"])
def test_workload_full(fa, name):
    w = WORKLOADS[name]
    q, k, v = w.make()
    _check(fa, q, k, v, w.causal, w.scale, w.dtype, label=name)


def _convex_hull_check(O, v, causal):
    """Each output row is a convex combination of the admissible value rows, so every
    coordinate lies between their minimum and maximum (prefix extrema when causal)."""
    vd = v.to(O.device).float()
    if causal:
        lo = torch.cummin(vd, dim=2).values
        hi = torch.cummax(vd, dim=2).values
    else:
        lo = vd.amin(dim=2, keepdim=True)
        hi = vd.amax(dim=2, keepdim=True)
    slack = 1e-2  # bf16 output rounding
    Of = O.float()
    assert bool(((Of >= lo - slack) & (Of <= hi + slack)).all()), "output outside the value hull"


def _errors_by_head(O, L, q, k, v, causal, scale, label):
    """Max |O - O_ref| and |L - L_ref| over every row of every head, the oracle run one
    head at a time (its S and P for one head are N x N fp64)."""
    o = O.double().cpu().numpy()
    lse = L.double().cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "non-finite output"
    qn, kn, vn = q.double().numpy(), k.double().numpy(), v.double().numpy()
    B, H = q.shape[0], q.shape[1]
    eo = el = 0.0
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            Oref, Lref = oracle.attention(qn[sl], kn[sl], vn[sl], causal, scale)
            eo = max(eo, float(np.max(np.abs(o[sl] - Oref))))
            el = max(el, float(np.max(np.abs(lse[sl] - Lref))))
        print(f"[parity] {label} heads {(b + 1) * H}/{B * H} max|dO|={eo:.3e} max|dL|={el:.3e}", flush=True)
    return eo, el


@pytest.mark.parametrize("name", ["causal_bf16_b4h16n4096d128", "long_causal_bf16_h32n16384d64"])
def test_workload_full_size_every_row(fa, name):
    w = WORKLOADS[name]
    q, k, v = w.make()
    O, L = _run(fa, q, k, v, w.causal, w.scale)
    eo, el = _errors_by_head(O, L, q, k, v, w.causal, w.scale, name)
    otol, ltol = TOL[w.dtype]
    print(f"[parity] {name} every row: max|dO|={eo:.3e} (tol {otol}) max|dL|={el:.3e} (tol {ltol})", flush=True)
    assert eo <= otol, f"{name}: O error {eo} > {otol}"
    assert el <= ltol, f"{name}: L error {el} > {ltol}"
    # Properties of every row: inside the value hull, and L >= the diagonal score (the
    # diagonal key is always admissible) and <= max score + log(#admissible keys).
    _convex_hull_check(O, v, w.causal)
    qd, kd = q.to(O.device).float(), k.to(O.device).float()
    diag = (qd * kd).sum(-1) * w.scale
    assert bool((L >= diag - 1e-2).all()), "L below the diagonal score"
    row_bound = (qd.norm(dim=-1) * kd.norm(dim=-1).cummax(dim=2).values) * w.scale
    logn = torch.log(torch.arange(1, w.N + 1, device=O.device, dtype=torch.float32))
    assert bool((L <= row_bound + logn + 1e-2).all()), "L above its Cauchy-Schwarz bound"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_f32_long(fa, causal, d):
    """fp32 at N = 4100: 129 key tiles spread over the waves of a workgroup (uneven
    shares, a ragged last tile), every row."""
    q, k, v = make_qkv(2, 4, 4100, d, "f32", seed=51 + d)
    _check(fa, q, k, v, causal, default_scale(d), "f32", label=f"fp32 N=4100 d={d} causal={causal}")


EDGE_N = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", EDGE_N)
def test_edge_sizes(fa, N, causal, d, dtype):
    q, k, v = make_qkv(1, 2, N, d, dtype, seed=1000 + N + d)
    _check(fa, q, k, v, causal, default_scale(d), dtype, label=f"N={N} d={d} causal={causal} {dtype}")


def _check_repeated(fa, q, k, v, causal, reps, label):
    """The heads of q, k, v, and the same heads repeated `reps` times in one launch: both
    match the oracle (computed once, on the distinct heads), and every repeat of a head is
    bitwise identical to its first copy."""
    dev = torch.device("cuda:0")
    scale = default_scale(q.shape[-1])
    H = q.shape[1]
    Oref, Lref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
    otol, ltol = TOL["bf16"]
    for r in (1, reps):
        qd, kd, vd = (t.repeat(1, r, 1, 1).to(dev) for t in (q, k, v))
        O, L = fa.forward(qd, kd, vd, causal=causal, scale=scale)
        torch.cuda.synchronize()
        eo, el = _errors(O[:, :H], L[:, :H], Oref, Lref)
        print(f"[parity] {label} x{r} max|dO|={eo:.3e} max|dL|={el:.3e}", flush=True)
        assert eo <= otol and el <= ltol, f"{label} x{r}: O error {eo}, L error {el}"
        for j in range(1, r):
            assert torch.equal(O[:, j * H:(j + 1) * H], O[:, :H]) and torch.equal(L[:, j * H:(j + 1) * H], L[:, :H])


KS_N = [1, 17, 33, 63, 64, 65, 127, 129, 255, 1000]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("N", KS_N)
def test_bf16_small_and_large_grid(fa, N, causal, d):
    """bf16 launches of at most 192 workgroups of 128 query rows (B*H*ceil(N/128) <= 192;
    384 when causal) pair the waves of a workgroup over the keys of each tile; larger ones
    give every wave all keys of its 32 rows. Two heads run alone (the paired form) and
    repeated to 400 heads (the other form, at least 400 workgroups)."""
    q, k, v = make_qkv(1, 2, N, d, "bf16", seed=3000 + N + d)
    _check_repeated(fa, q, k, v, causal, 200, f"N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_grid_size_threshold(fa, causal):
    """One head repeated to the largest head count with paired waves (192 workgroups of 128
    rows, 384 when causal) and to one more (one wave per 32 rows over all keys), at N = 100
    and N = 128 (one tile)."""
    limit = 384 if causal else 192
    for N in (100, 128):
        q, k, v = make_qkv(1, 1, N, 128, "bf16", seed=3100 + N)
        for reps in (limit, limit + 1):
            _check_repeated(fa, q, k, v, causal, reps, f"N={N} heads={reps} causal={causal}")


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 16, 2048, 128, True), (1, 24, 2048, 64, True),
                                             (1, 8, 2048, 128, False), (1, 32, 2048, 128, True)])
def test_bf16_long_rows_both_forms(fa, B, H, N, d, causal):
    """Long rows on either side of the key-split switch (causal: 256 and 384 workgroups of
    128 rows use the split, 512 do not; non-causal: 128 use it), every row of every head."""
    q, k, v = make_qkv(B, H, N, d, "bf16", seed=3200 + H + d)
    O, L = _run(fa, q, k, v, causal, default_scale(d))
    label = f"B{B} H{H} N{N} d{d} causal={causal}"
    eo, el = _errors_by_head(O, L, q, k, v, causal, default_scale(d), label)
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1], f"{label}: O error {eo}, L error {el}"


@pytest.mark.parametrize("causal", [False, True])
def test_grid_not_multiple_of_xcds(fa, causal):
    """B*H*tiles = 3*37*2 = 222 workgroups: the XCD renumbering must stay a bijection."""
    q, k, v = make_qkv(3, 37, 200, 64, "bf16", seed=42)
    _check(fa, q, k, v, causal, default_scale(64), "bf16", label=f"B3 H37 N200 causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_head_groups_per_xcd(fa, causal):
    """48 heads of N=4096, d=128 (2 MiB of K and V each): six heads per XCD, which each XCD
    takes three at a time (the largest divisor of 6 whose K and V fit in 8 MiB), so every
    XCD runs two head groups. O and L start as NaN, so a tile the mapping skips shows as a
    non-finite row; every row of every head is compared with the oracle."""
    B, H, N, d = 3, 16, 4096, 128
    q, k, v = make_qkv(B, H, N, d, "bf16", seed=48)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    O = torch.full_like(qd, float("nan"))
    L = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_fwd(qd, kd, vd, O, L, B, H, N, d, causal, default_scale(d))
    torch.cuda.synchronize()
    label = f"B{B} H{H} N{N} d{d} causal={causal}"
    eo, el = _errors_by_head(O, L, q, k, v, causal, default_scale(d), label)
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1], f"{label}: O error {eo}, L error {el}"


@pytest.mark.parametrize("B,H,N,d,causal,group", [
    (2, 32, 2304, 128, True, 4),    # 8 heads per XCD, 1.2 MB of K/V each: two groups of 4
    (1, 40, 4096, 64, False, 5),    # 5 heads per XCD, 1 MiB each: one group of all 5
    (1, 40, 8192, 128, True, 1),    # 4 MiB each: one head at a time, 5 groups
    (3, 8, 3000, 128, False, 3),    # 3 heads per XCD, 1.5 MB each: one group of 3
    (1, 72, 2048, 128, True, 3),    # 9 heads per XCD, 1 MiB each: 8 would fit, 3 divides 9
])
def test_head_group_sizes(fa, B, H, N, d, causal, group):
    """The per-XCD head groups over a range of group sizes (the largest divisor of the XCD's
    head count whose K and V fit in 8 MiB; the comment gives it). O and L start as NaN, so a
    tile the mapping skips shows as a non-finite row; 24 rows of every head against the
    oracle."""
    q, k, v = make_qkv(B, H, N, d, "bf16", seed=49 + H + N)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    O = torch.full_like(qd, float("nan"))
    L = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_fwd(qd, kd, vd, O, L, B, H, N, d, causal, default_scale(d))
    torch.cuda.synchronize()
    assert torch.isfinite(O).all() and torch.isfinite(L).all(), "rows no workgroup wrote"
    rows = np.unique(np.concatenate([np.linspace(0, N - 1, 20).astype(int), [1, 127, 128, N - 2]]))
    Oref, Lref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                  causal, default_scale(d), rows=rows)
    eo, el = _errors(O, L, Oref, Lref, rows)
    label = f"B{B} H{H} N{N} d{d} causal={causal} (groups of {group})"
    print(f"[parity] {label} max|dO|={eo:.3e} max|dL|={el:.3e}", flush=True)
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1], f"{label}: O error {eo}, L error {el}"


@pytest.mark.parametrize("causal", [False, True])
def test_scale_other_than_default(fa, causal):
    q, k, v = make_qkv(1, 2, 300, 128, "bf16", seed=43)
    _check(fa, q, k, v, causal, 0.3, "bf16", label=f"scale 0.3 causal={causal}")
    q, k, v = make_qkv(1, 2, 300, 64, "f32", seed=44)
    _check(fa, q, k, v, causal, 0.01, "f32", label=f"fp32 scale 0.01 causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_very_wide_logits(fa, causal):
    """Q, K ~ N(0, 8^2): scaled logits with a spread of ~64, many rescales per row."""
    q, k, v = make_qkv(1, 4, 700, 128, "bf16", seed=45, sigma_qk=8.0)
    _check(fa, q, k, v, causal, default_scale(128), "bf16", label=f"sigma 8 causal={causal}")
    # fp32: a score is a d-term fp32 dot product, so its rounding error grows with
    # |q||k| ~ sigma^2 (here ~25x the N(0,1) case: |s| reaches ~100, whose fp32 ulp
    # alone is 7.6e-6). The weights' relative error follows, so the N(0,1) bounds
    # are scaled by sigma^2.
    sigma = 5.0
    q, k, v = make_qkv(1, 2, 700, 64, "f32", seed=46, sigma_qk=sigma)
    otol, ltol = TOL["f32"]
    _check(fa, q, k, v, causal, default_scale(64), "f32", label=f"fp32 sigma 5 causal={causal}",
           tol=(otol * sigma ** 2, ltol * sigma ** 2))


@pytest.mark.parametrize("e", [-60, -30, 30, 60])
@pytest.mark.parametrize("H", [2, 160])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_value_scale_range(fa, e, H, d, causal):
    """V scaled by 2^e (exact in bf16), Q and K ~ N(0, 4^2): O scales by 2^e and L does not.
    The bf16 kernel's accumulators hold about 2^-64 |v| after a reference move (the
    reference sits 64 above the row maximum) and at most 2^8 N |v|, so V from 2^-60 to 2^60
    keeps the unscaled case's relative precision. H = 2 runs the key-split grid, H = 160
    the unsplit one."""
    q, k, v = make_qkv(1, H, 300, d, "bf16", seed=48, sigma_qk=4.0)
    vs = (v.double() * 2.0 ** e).to(torch.bfloat16)
    assert torch.equal(vs.double() * 2.0 ** -e, v.double()), "power-of-two scaling is exact"
    scale = default_scale(d)
    O, L = _run(fa, q, k, vs, causal, scale)
    Oref, Lref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
    Ob = O.double().cpu() * 2.0 ** -e
    eo, el = _errors(Ob, L, Oref, Lref)
    otol, ltol = TOL["bf16"]
    print(f"[parity] V x 2^{e} H={H} d={d} causal={causal} max|dO|/2^{e}={eo:.3e} max|dL|={el:.3e}", flush=True)
    assert eo <= otol and el <= ltol, (eo, el)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H", [2, 160])
@pytest.mark.parametrize("causal", [False, True])
def test_score_jumps(fa, dtype, H, causal):
    """Scores that jump by hundreds (base 2) between key tiles: 0 for keys < 64, 362
    (natural log) for keys 64..199, 724 from key 200 on. Against the reference kept
    from the earlier keys the new weights overflow to infinity, so the kernels must move
    the reference before those weights enter O and l (the bf16 kernel forms the tile's
    weights again once their sum is not finite). H = 2 runs the key-split grid."""
    N, d = 300, 128
    _, _, v = make_qkv(1, H, N, d, dtype, seed=49)
    q = torch.zeros(1, H, N, d, dtype=v.dtype)
    k = torch.zeros(1, H, N, d, dtype=v.dtype)
    q[..., 0] = 64.0
    k[..., 64:200, 0] = 64.0
    k[..., 200:, 0] = 128.0
    _check(fa, q, k, v, causal, default_scale(d), dtype, label=f"score jumps {dtype} H={H} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_uniform_closed_form(fa, dtype):
    """Q = 0: causal row i is the mean of value rows 0..i and L = log(i+1)."""
    N, d = 333, 64
    _, k, v = make_qkv(1, 1, N, d, dtype, seed=47)
    q = torch.zeros_like(k)
    O, L = _run(fa, q, k, v, True, default_scale(d))
    mean = torch.cumsum(v.double(), dim=2) / torch.arange(1, N + 1, dtype=torch.float64)[:, None]
    otol, ltol = TOL[dtype]
    assert float((O.double().cpu() - mean).abs().max()) <= otol
    assert float((L.double().cpu() - torch.log(torch.arange(1, N + 1, dtype=torch.float64))).abs().max()) <= ltol


@pytest.mark.parametrize("B,H,N,d,causal,dtype", [(2, 4, 777, 128, True, "bf16"), (1, 2, 255, 128, True, "bf16"),
                                                   (1, 8, 1000, 64, False, "bf16"), (4, 16, 4096, 128, True, "bf16"),
                                                   (8, 1, 1024, 64, False, "f32"), (2, 3, 777, 128, True, "f32")])
def test_deterministic(fa, B, H, N, d, causal, dtype):
    """Each output element is reduced in a fixed order (the fp32 kernel merges its waves'
    partial results in wave order), so repeated launches on the same inputs are bitwise
    identical. A K/V tile landing in the wrong LDS slot (a DMA issued before its LDS
    address took effect) or read before it landed shows up here as launch-to-launch
    differences."""
    q, k, v = make_qkv(B, H, N, d, dtype, seed=48)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    O1, L1 = fa.forward(qd, kd, vd, causal=causal, scale=default_scale(d))
    for _ in range(5):
        O2, L2 = fa.forward(qd, kd, vd, causal=causal, scale=default_scale(d))
        torch.cuda.synchronize()
        assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_non_default_stream(fa):
    q, k, v = make_qkv(1, 2, 512, 128, "bf16", seed=49)
    s = torch.cuda.Stream()
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        O, L = fa.forward(qd, kd, vd, causal=True, scale=default_scale(128), stream=s)
    s.synchronize()
    Oref, Lref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                  True, default_scale(128))
    eo, el = _errors(O, L, Oref, Lref)
    assert eo <= 2e-2 and el <= 1e-2


def test_bf16_close_to_fp32(fa):
    """The same bf16-representable inputs through both element types agree."""
    q, k, v = make_qkv(1, 2, 400, 64, "bf16", seed=50)
    Ob, Lb = _run(fa, q, k, v, True, default_scale(64))
    Of, Lf = _run(fa, q.float(), k.float(), v.float(), True, default_scale(64))
    assert float((Ob.float() - Of).abs().max()) <= 2e-2
    # The bf16 kernel's row sum adds the bf16-rounded weights (relative error <= u = 2^-8
    # each), so its L may differ by up to log(1 + 2^-8) = 3.9e-3 from the fp32 sum.
    assert float((Lb - Lf).abs().max()) <= 4e-3


def test_errors_raise(fa):
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device=dev)
    with pytest.raises(fa.FaError) as e:
        fa.forward(q, q.clone(), q.clone())
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
