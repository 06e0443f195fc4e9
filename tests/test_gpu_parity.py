"""Parity of the HIP path against the CPU oracle (needs an MI355X).

Every call goes through the C ABI via the ctypes binding.  The bar:

* integer-valued inputs: bit-exact (every fp32 partial sum is an exact
  integer, so any summation order gives the oracle's C16);
* Gaussian inputs with unit-variance outputs: max |C_gpu - C64| <= 1e-2, the
  tolerance the pages use for fp32-accumulating kernels ("6. Four Consumers,
  FP16 Accumulation, and a TMA Epilogue", "The Register Budget Problem");
  and, tighter, per element |C_gpu - C64| <= ulp16(C64) / 2 + e_acc, with at
  least 99% of outputs bit-equal to C16 = rne(C64).  The fp16 cast alone
  contributes at most half an fp16 ulp of the result.  e_acc bounds the fp32
  accumulation: partial sums have magnitude ~1, each fp32 addition rounds by
  at most 2^-24 of that, and the roundings add like a random walk over K
  terms, giving ~2^-24 * sqrt(K); e_acc = 64 * 2^-24 * sqrt(K) leaves a wide
  margin (3.4e-4 at K = 8192) yet still catches a truncating cast, which
  errs by up to a whole ulp (3.9e-3 for |C| in [4, 8)).
"""
from __future__ import annotations

import functools

import numpy as np
import pytest

import _errstats
import oracle
from dense_fp16_gemm_04_amd import binding, workloads

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _torch():
    import torch
    return torch


@pytest.fixture(scope="module", autouse=True)
def _lib():
    lib = binding.load()  # raises if the HIP library is missing
    return lib


def dev():
    return _torch().device("cuda:0")


def run(a, b, variant=None, out=None):
    torch = _torch()
    ta = torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    tb = torch.from_numpy(np.ascontiguousarray(b)).to(dev())
    if variant is None:
        c = binding.gemm_nt_f16(ta, tb, out=out)
    else:
        c = binding.gemm_nt_f16_ex(ta, tb, out=out, variant=variant)
    torch.cuda.synchronize()
    return c.cpu().numpy()


def fp16_ulp(x):
    """Spacing of fp16 values at |x| (2^-24 in the subnormal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(ax)) - 10)


def assert_close(got16, c64, c16, K, label=""):
    got = got16.astype(np.float64)
    assert np.all(np.isfinite(got)), label + ": non-finite output"
    err = np.abs(got - c64)
    assert err.max() <= TOL, "%s: max err %g" % (label, err.max())
    bound = fp16_ulp(c64) / 2 + 64 * 2.0 ** -24 * np.sqrt(max(K, 1))
    worst = np.max(err - bound)
    assert worst <= 0, "%s: error exceeds half an fp16 ulp + fp32 bound by %g" % (label, worst)
    same = np.mean(got16.view(np.uint16) == c16.view(np.uint16))
    assert same >= 0.99, "%s: only %.4f bit-equal to rne(C64)" % (label, same)
    return err


def variant_ids():
    names = binding.variants()
    return {n: i for i, n in enumerate(names)}


# ------------------------------------------------------------ workloads --

@functools.lru_cache(maxsize=None)
def workload_data(name):
    w = workloads.by_name(name)
    a, b = workloads.workload_inputs(w)
    return w, a, b


@functools.lru_cache(maxsize=None)
def workload_oracle(name):
    _, a, b = workload_data(name)
    return oracle.gemm_nt(a, b)


FULL = ["square_256", "square_1024", "square_4096", "ragged_5000x3000x6000",
        "share_m_1024x8192x8192", "share_n_8192x1024x8192"]


@pytest.mark.parametrize("name", FULL)
def test_workload_full_parity(name):
    w, a, b = workload_data(name)
    print("case", name, binding.gemm_nt_f16_config_name(w.M, w.N, w.K), flush=True)
    got = run(a, b)
    c64, c16 = workload_oracle(name)
    assert_close(got, c64, c16, w.K, name)
    _errstats.record(name, got, c64, c16, w.K)


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 2048), (256, 8192, 4096), (4352, 4352, 2048)])
def test_plan_shapes_gaussian(M, N, K):
    """Unit-variance outputs through gemm_nt_f16 on shapes whose plan uses
    the 128x128 hand-ordered kernel (2048^3; the 256-row product) or splits
    the rows of C (4352 x 4352 x 2048), against the oracle at the same bar
    as the workloads."""
    v, rows, rest = binding.gemm_nt_f16_plan(M, N, K)
    names = binding.variants()
    print("case plan", M, N, K, names[v], rows, names[rest] if rest >= 0 else "-", flush=True)
    a, b = workloads.gaussian(M, N, K, seed=M + 3 * N + 7 * K)
    c64, c16 = oracle.gemm_nt(a, b)
    err = assert_close(run(a, b), c64, c16, K, "%dx%dx%d" % (M, N, K))
    print("max %.3g mean %.3g" % (err.max(), err.mean()))


def test_headline_full_parity_and_error_figures():
    """M = N = K = 8192 through gemm_nt_f16, the launch the benchmark times,
    compared with the oracle on all 67,108,864 outputs.

    Beyond the bar of every workload, the error distribution must be the
    fp16 rounding of the exact result and nothing more: the pages report
    mean 0.00014 and max 0.0020 for their fp32-accumulating kernel at this K
    against an fp32 reference ("6. Four Consumers, FP16 Accumulation, and a
    TMA Epilogue", "The Register Budget Problem"); half an fp16 ulp in the
    [4, 8) binade is 0.00195, and a round-to-nearest cast has no bias.
    """
    name = "square_8192"
    w, a, b = workload_data(name)
    print("case", name, binding.gemm_nt_f16_config_name(w.M, w.N, w.K), flush=True)
    got = run(a, b)
    c64, c16 = workload_oracle(name)
    assert_close(got, c64, c16, w.K, name)
    rec = _errstats.record(name, got, c64, c16, w.K)
    assert abs(rec["mean"] - 1.4e-4) < 0.3e-4, rec
    assert rec["max"] <= 2.0e-3 + 1e-5, rec
    assert abs(rec["signed_mean"]) < 2e-5, rec  # round to nearest: no bias toward zero
    assert abs(rec["var_c64"] - 1.0) < 0.02, rec
    assert abs(float(got.astype(np.float64).var()) - 1.0) < 0.02


# ------------------------------------------------------ exact / invariants --

@pytest.mark.parametrize("name", [w.name for w in workloads.WORKLOADS])
def test_integer_inputs_bit_exact(name):
    """Integer inputs in {-1, 0, 1} at every workload's full size: every
    fp32 partial sum is an exact integer, so all outputs must equal the
    oracle's rne(C64) bit for bit."""
    w = workloads.by_name(name)
    a, b = workloads.small_integers(w.M, w.N, w.K, seed=w.seed)
    print("case int", name, flush=True)
    got = run(a, b)
    _, c16 = oracle.gemm_nt(a, b)
    assert np.array_equal(got.view(np.uint16), c16.view(np.uint16))


def test_identity_b_gives_a():
    a, _ = workloads.gaussian(512, 1, 512, seed=31)
    eye = np.eye(512, dtype=np.float16)
    got = run(a, eye)
    assert np.array_equal(got.astype(np.float64), a.astype(np.float64))


def test_scaling_by_two_is_exact():
    # doubling A doubles every product and every fp32 partial sum exactly;
    # the fp16 cast commutes with doubling wherever the result is a normal
    # fp16 value (the subnormal grid below 2^-14 is fixed, so there a
    # doubled value can round differently)
    a, b = workloads.gaussian(384, 320, 512, seed=32)
    c1 = run(a, b).astype(np.float64)
    c2 = run((a.astype(np.float32) * 2).astype(np.float16), b).astype(np.float64)
    normal = np.abs(c1) >= 2.0 ** -14
    assert normal.mean() > 0.99
    assert np.array_equal(c2[normal], 2.0 * c1[normal])
    assert np.all(np.abs(c2[~normal] - 2.0 * c1[~normal]) <= 2.0 ** -23)


def test_transpose_symmetry():
    a, b = workloads.small_integers(700, 300, 264, seed=33)
    assert np.array_equal(run(b, a).view(np.uint16), run(a, b).T.view(np.uint16))
    a, b = workloads.gaussian(700, 300, 264, seed=34)
    c_ab, c_ba = run(a, b), run(b, a)
    assert np.max(np.abs(c_ab.astype(np.float64) - c_ba.T.astype(np.float64))) <= 2 * TOL


def test_zero_k_padding():
    a, b = workloads.small_integers(257, 129, 200, seed=35)
    pad = 56
    ap = np.concatenate([a, np.zeros((257, pad), np.float16)], axis=1)
    bp = np.concatenate([b, np.zeros((129, pad), np.float16)], axis=1)
    assert np.array_equal(run(ap, bp).view(np.uint16), run(a, b).view(np.uint16))


def test_linearity_in_a():
    a1, b = workloads.small_integers(300, 260, 320, seed=36)
    a2, _ = workloads.small_integers(300, 260, 320, seed=37)
    s = (a1.astype(np.float32) + a2).astype(np.float16)
    lhs = run(s, b).astype(np.float64)
    rhs = run(a1, b).astype(np.float64) + run(a2, b).astype(np.float64)
    assert np.array_equal(lhs, rhs)


def test_subnormal_inputs():
    # every product a*b is a multiple of 2^-48 and every sum exact in fp32
    # until the last fp16 rounding, which lands in the subnormal range
    g = np.random.Generator(np.random.PCG64(38))
    a = (g.integers(-8, 9, (130, 96)) * 2.0 ** -20).astype(np.float16)
    b = (g.integers(-8, 9, (70, 96)) * 2.0 ** -8).astype(np.float16)
    assert np.any(np.abs(a.astype(np.float64)) < 2.0 ** -14)
    got = run(a, b)
    _, c16 = oracle.gemm_nt(a, b)
    assert np.array_equal(got.view(np.uint16), c16.view(np.uint16))


# --------------------------------------------------------- special values --
#
# The pages fix only the one fp16 cast of the fp32 accumulator ("0. A Minimal
# Hopper Matmul", "Walkthrough", "Epilogue").  Read by IEEE 754 rules: a NaN
# input, Inf * 0 and Inf - Inf give NaN, an Inf term otherwise gives an Inf of
# its sign, and a finite sum of magnitude >= 65520 rounds to Inf (65520 lies
# halfway between the largest fp16 value, 65504, and 2^16, and ties go to the
# even neighbour, 2^16, which overflows).  Products of fp16 values are exact
# in fp32, and with integer operands every partial sum below 2^24 is exact in
# any order, so the GPU must match the oracle's rne(C64) bit for bit (NaN by
# class: its payload and sign are not specified).

SPECIAL_SHAPE = (300, 264, 136)  # partial tiles in M and N, a K tail of 8


def assert_same_or_both_nan(got16, c16, label):
    g, c = got16.view(np.uint16), c16.view(np.uint16)
    gn, cn = np.isnan(got16.astype(np.float32)), np.isnan(c16.astype(np.float32))
    assert np.array_equal(gn, cn), "%s: NaN at %d outputs, oracle %d" % (label, gn.sum(), cn.sum())
    bad = (g != c) & ~gn
    assert not bad.any(), "%s: %d outputs differ, first at %s" % (label, bad.sum(), np.argwhere(bad)[0])


def special_value_inputs():
    """Integer inputs in {-1, 0, 1} with Inf and NaN planted in A and B: in
    full K steps, in the K tail, in the last row of B, and pairs that give
    Inf * 0 and Inf - Inf."""
    M, N, K = SPECIAL_SHAPE
    a, b = workloads.small_integers(M, N, K, seed=71)
    inf, nan = np.float16(np.inf), np.float16(np.nan)
    a[5, 17] = inf
    a[9, 100] = -inf
    a[13, 3] = nan
    a[40, 130] = inf      # in the K tail (k >= 128)
    a[299, 0] = -inf      # the last row, in the partial tile row
    a[30, 10] = inf       # Inf - Inf wherever B[n, 10] = -B[n, 11] != 0
    a[30, 11] = inf
    b[7, 17] = 0          # Inf * 0 = NaN at C[5, 7]
    b[20, 50] = inf       # column 20: +-Inf or NaN by A[m, 50]
    b[263, 135] = nan     # the last row of B, the last k
    b[100, 64] = -inf     # the first k of the second K step
    return a, b


def overflow_inputs():
    """Integer sums that land on and around the fp16 overflow edge and on
    rounding ties: rows 0 .. 7 of A hold 1 (rows 8 .. 15: -1) at k = 0 .. 3
    and 0 elsewhere, so C[m, n] = +-(B[n, 0] + .. + B[n, 3]) exactly, with
    B's first four entries in rows n < 18 fp16 integers that sum to each
    target; the other rows of A are random in {-1, 0, 1} against those large
    entries."""
    M, N, K = SPECIAL_SHAPE
    a, b = workloads.small_integers(M, N, K, seed=72)
    targets = [65504, 65505, 65519, 65520, 65521, 65536, 100000, 2049, 2051, 4097, 4098, 4099,
               32768, 65488, 65496, 65503, 131000, 200000]
    for n, t in enumerate(targets):
        parts, r = [], t
        while r > 0:  # greedy: the largest fp16 integer not above what is left
            f = np.float16(min(r, 65504))
            if float(f) > r:
                f = np.nextafter(f, np.float16(0))
            parts.append(float(f))
            r -= float(f)
        assert len(parts) <= 4 and sum(parts) == t, (t, parts)
        b[n, :4] = 0
        b[n, :len(parts)] = np.array(parts, dtype=np.float16)
    a[:16, :] = 0
    a[:8, :4] = 1
    a[8:16, :4] = -1
    return a, b


def test_special_values_every_variant():
    a, b = special_value_inputs()
    _, c16 = oracle.gemm_nt(a, b)
    assert np.isnan(c16.astype(np.float32)).any() and np.isinf(c16.astype(np.float32)).any()
    print("case special plan", *SPECIAL_SHAPE, flush=True)
    assert_same_or_both_nan(run(a, b), c16, "plan")
    for name, vid in variant_ids().items():
        print("case special", name, flush=True)
        assert_same_or_both_nan(run(a, b, variant=vid), c16, name)


def test_overflow_to_inf_every_variant():
    a, b = overflow_inputs()
    _, c16 = oracle.gemm_nt(a, b)
    c = c16.astype(np.float64)
    # the edge itself: 65504 stays, 65519 rounds down, 65520 (a tie) overflows
    assert c[0, 0] == 65504 and c[0, 2] == 65504 and np.isinf(c[0, 3]) and c[8, 0] == -65504
    assert c[0, 7] == 2048 and c[0, 8] == 2052  # ties to even
    assert np.isinf(c).sum() > 100 and not np.isnan(c).any()
    print("case overflow plan", *SPECIAL_SHAPE, flush=True)
    assert_same_or_both_nan(run(a, b), c16, "plan")
    for name, vid in variant_ids().items():
        print("case overflow", name, flush=True)
        got = run(a, b, variant=vid)
        assert np.array_equal(got.view(np.uint16), c16.view(np.uint16)), name


# ------------------------------------------------------------ edge shapes --

EDGE = [1, 7, 8, 15, 16, 17, 31, 33, 63, 65, 127, 129, 255, 257]


def _edge_shapes():
    g = np.random.Generator(np.random.PCG64(40))
    shapes = set()
    for m in EDGE:
        shapes.add((m, int(g.choice(EDGE)), int(g.choice([8, 16, 24, 56, 64, 72, 136, 200]))))
    for n in EDGE:
        shapes.add((int(g.choice(EDGE)), n, int(g.choice([8, 64, 120, 128, 264]))))
    shapes.update({(1, 1, 8), (257, 255, 8), (129, 513, 64), (600, 40, 1000)})
    return sorted(shapes)


def test_edge_shapes_every_variant():
    ids = variant_ids()
    for (M, N, K) in _edge_shapes():
        a, b = workloads.small_integers(M, N, K, seed=M * 1000003 + N * 1009 + K)
        _, c16 = oracle.gemm_nt(a, b)
        for name, vid in ids.items():
            print("case edge", M, N, K, name, flush=True)
            got = run(a, b, variant=vid)
            assert np.array_equal(got.view(np.uint16), c16.view(np.uint16)), (M, N, K, name)


@pytest.mark.parametrize("M,N,K", [(5000, 6000, 72), (8192, 8192, 128), (2304, 9000, 8),
                                   (4100, 4100, 72), (4097, 4097, 16), (4200, 4104, 200),
                                   (2560, 8200, 328)])
def test_many_tiles_per_workgroup_every_variant(M, N, K):
    """Shapes with more tiles than compute units, so the persistent kernels
    stream several tiles (and their K tails) through one workgroup; N = 4100
    and 4097 take the 8-byte and single-element stores.  4200 x 4104 x 200 and
    2560 x 8200 x 328 give the persistent 5-slot kernel one or two tiles per
    workgroup, K loops of 4 and 6 steps with a K tail, and partial tiles at
    both M and N (N % 256 = 8: the last tile column has one 16-byte chunk per
    row)."""
    a, b = workloads.small_integers(M, N, K, seed=M + N + K)
    _, c16 = oracle.gemm_nt(a, b)
    for name, vid in variant_ids().items():
        if name.startswith("simple") and M * N * K > 2 ** 32:
            continue
        print("case many-tiles", M, N, K, name, flush=True)
        got = run(a, b, variant=vid)
        assert np.array_equal(got.view(np.uint16), c16.view(np.uint16)), (M, N, K, name)


@pytest.mark.parametrize("K", [960, 1024, 1088, 1152, 1216, 1000, 1208])
def test_persistent_ring_positions(K):
    """The persistent kernels rotate a five-slot ring across tiles, and the
    lean one runs its whole-K-range steps as a cycle of five from slot 0
    after up to four general steps.  544 tiles of 256 x 256 give every
    workgroup two or three tiles; a tile of nk steps moves the ring by 2 nk
    slots, so nk = 15 .. 19 (K = 960 .. 1216) starts the second tile at each
    of the five positions, and K = 1000 and 1208 add a K tail (a last step
    of 40 and 56 columns).  Integer inputs, bit-exact."""
    M, N = 4352, 8192
    a, b = workloads.small_integers(M, N, K, seed=K * 31 + 5)
    _, c16 = oracle.gemm_nt(a, b)
    for name, vid in variant_ids().items():
        if "persistent" not in name:
            continue
        print("case ring", M, N, K, name, flush=True)
        got = run(a, b, variant=vid)
        assert np.array_equal(got.view(np.uint16), c16.view(np.uint16)), (M, N, K, name)


@pytest.mark.parametrize("M,N,K", [(4200, 4352, 1024), (4104, 4096, 2048), (4352, 4360, 2048)])
def test_split_launch_plan(M, N, K):
    """Shapes whose 256x256 tiles leave a small last wave: gemm_nt_f16 runs
    whole waves over the first rows and the remaining rows (with an M tail,
    an N tail, or only 8 rows) as a second kernel.  Bit-exact on integer
    inputs through the whole product."""
    v, rows, rest = binding.gemm_nt_f16_plan(M, N, K)
    assert 0 < rows < M and rows % 256 == 0 and rest >= 0
    a, b = workloads.small_integers(M, N, K, seed=M * 7 + N + K)
    _, c16 = oracle.gemm_nt(a, b)
    print("case split", M, N, K, rows, binding.variants()[v], binding.variants()[rest], flush=True)
    got = run(a, b)
    assert np.array_equal(got.view(np.uint16), c16.view(np.uint16)), (M, N, K)


def _random_plan_shapes():
    """16 seeded random shapes, 8 whose plan splits the rows of C and 8 run
    as one kernel, each at most 3e10 multiply-adds (a few seconds of the
    oracle)."""
    g = np.random.Generator(np.random.PCG64(77))
    split, single = [], []
    while len(split) < 8 or len(single) < 8:
        M, N = (int(x) for x in g.integers(1, 7000, size=2))
        K = int(g.choice([8, 72, 136, 520, 1032, 2056]))
        if M * N * K > 3e10:
            continue
        _, rows, rest = binding.gemm_nt_f16_plan(M, N, K)
        (split if rest >= 0 else single).append((M, N, K))
    return split[:8] + single[:8]


def test_random_shapes_through_the_launch_plan():
    """Integer inputs, bit-exact, through gemm_nt_f16 (the plan the library
    makes for each shape, split or not)."""
    for i, (M, N, K) in enumerate(_random_plan_shapes()):
        v, rows, rest = binding.gemm_nt_f16_plan(M, N, K)
        print("case random", M, N, K, binding.variants()[v], rows, rest, flush=True)
        a, b = workloads.small_integers(M, N, K, seed=5000 + i)
        _, c16 = oracle.gemm_nt(a, b)
        got = run(a, b)
        assert np.array_equal(got.view(np.uint16), c16.view(np.uint16)), (M, N, K, v, rows, rest)


def test_k_zero_many_tiles_every_variant():
    torch = _torch()
    a = torch.zeros((4096, 0), dtype=torch.float16, device=dev())
    b = torch.zeros((4352, 0), dtype=torch.float16, device=dev())
    for name, vid in variant_ids().items():
        out = torch.full((4096, 4352), 5.0, dtype=torch.float16, device=dev())
        binding.gemm_nt_f16_ex(a, b, out=out, variant=vid)
        torch.cuda.synchronize()
        assert torch.all(out == 0).item(), name


def test_k_not_multiple_of_8_uses_simple_path():
    for (M, N, K) in [(33, 17, 7), (64, 64, 1), (100, 90, 13), (5, 300, 999)]:
        a, b = workloads.gaussian(M, N, K, seed=K)
        print("case k%8", M, N, K, binding.gemm_nt_f16_config_name(M, N, K), flush=True)
        c64, c16 = oracle.gemm_nt(a, b)
        assert_close(run(a, b), c64, c16, K, "K=%d" % K)


def test_unaligned_pointers_use_simple_path():
    torch = _torch()
    M, N, K = 70, 50, 64
    a, b = workloads.gaussian(M, N, K, seed=41)
    c64, c16 = oracle.gemm_nt(a, b)
    # views that start one element into a buffer: 2-byte but not 16-byte aligned
    ba = torch.zeros(M * K + 1, dtype=torch.float16, device=dev())
    ba[1:] = torch.from_numpy(a.ravel()).to(dev())
    bb = torch.zeros(N * K + 1, dtype=torch.float16, device=dev())
    bb[1:] = torch.from_numpy(b.ravel()).to(dev())
    ta, tb = ba[1:].view(M, K), bb[1:].view(N, K)
    c = binding.gemm_nt_f16(ta, tb)
    torch.cuda.synchronize()
    assert_close(c.cpu().numpy(), c64, c16, K, "unaligned")
    with pytest.raises(binding.GemmError):
        binding.gemm_nt_f16_ex(ta, tb, variant=0)


def test_k_zero_writes_zeros_and_empty_is_no_op():
    torch = _torch()
    a = torch.zeros((37, 0), dtype=torch.float16, device=dev())
    b = torch.zeros((45, 0), dtype=torch.float16, device=dev())
    out = torch.full((37, 45), 7.0, dtype=torch.float16, device=dev())
    binding.gemm_nt_f16(a, b, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0).item() and not torch.any(torch.signbit(out)).item()
    a = torch.zeros((0, 16), dtype=torch.float16, device=dev())
    b = torch.ones((5, 16), dtype=torch.float16, device=dev())
    assert binding.gemm_nt_f16(a, b).shape == (0, 5)


def test_no_writes_outside_c():
    torch = _torch()
    M, N, K = 300, 264, 128
    a, b = workloads.small_integers(M, N, K, seed=42)
    _, c16 = oracle.gemm_nt(a, b)
    guard = 4096
    ids = variant_ids()
    for name, vid in ids.items():
        buf = torch.full((guard + M * N + guard,), -3.0, dtype=torch.float16, device=dev())
        out = buf[guard:guard + M * N].view(M, N)
        ta = torch.from_numpy(a).to(dev())
        tb = torch.from_numpy(b).to(dev())
        binding.gemm_nt_f16_ex(ta, tb, out=out, variant=vid)
        torch.cuda.synchronize()
        host = buf.cpu().numpy()
        assert np.all(host[:guard] == -3.0) and np.all(host[-guard:] == -3.0), name
        assert np.array_equal(host[guard:-guard].reshape(M, N).view(np.uint16),
                              c16.view(np.uint16)), name


@pytest.mark.parametrize("N,offset", [(264, 0), (264, 4), (264, 1), (260, 0), (262, 0)])
def test_every_store_path_every_variant(N, offset):
    """C rows taking 16-byte stores (through LDS), 8-byte stores, or single
    elements, chosen by N and by C's alignment (offset in elements from a
    16-byte boundary); guard bands on both sides must stay untouched."""
    torch = _torch()
    M, K = 300, 136
    a, b = workloads.small_integers(M, N, K, seed=N * 31 + offset)
    _, c16 = oracle.gemm_nt(a, b)
    guard = 4096
    ta = torch.from_numpy(a).to(dev())
    tb = torch.from_numpy(b).to(dev())
    for name, vid in variant_ids().items():
        print("case stores", N, offset, name, flush=True)
        buf = torch.full((guard + offset + M * N + guard,), -3.0, dtype=torch.float16, device=dev())
        out = buf[guard + offset:guard + offset + M * N].view(M, N)
        binding.gemm_nt_f16_ex(ta, tb, out=out, variant=vid)
        torch.cuda.synchronize()
        host = buf.cpu().numpy()
        assert np.all(host[:guard + offset] == -3.0) and np.all(host[-guard:] == -3.0), name
        assert np.array_equal(host[guard + offset:-guard].reshape(M, N).view(np.uint16),
                              c16.view(np.uint16)), name


def test_repeated_launches_are_deterministic_and_finite():
    torch = _torch()
    _, a, b = workload_data("square_4096")
    ta = torch.from_numpy(a).to(dev())
    tb = torch.from_numpy(b).to(dev())
    first = binding.gemm_nt_f16(ta, tb).clone()
    outs = [binding.gemm_nt_f16(ta, tb) for _ in range(30)]
    torch.cuda.synchronize()
    assert torch.isfinite(first.float()).all().item()
    for o in outs:
        assert torch.equal(o.view(torch.int16), first.view(torch.int16))


def test_graph_replays_match_eager_calls():
    """gemm_nt_f16 captured in a HIP graph (through torch.cuda.graph), one
    launch and a split plan of two: before each replay new inputs are copied
    in eagerly and an eager call computes the reference; every replay must
    equal it bit for bit, and the oracle on integer inputs."""
    torch = _torch()
    for (M, N, K) in [(1000, 520, 264), (4352, 4352, 2048)]:
        ta = torch.empty((M, K), dtype=torch.float16, device=dev())
        tb = torch.empty((N, K), dtype=torch.float16, device=dev())
        out = torch.empty((M, N), dtype=torch.float16, device=dev())
        ref = torch.empty_like(out)
        binding.gemm_nt_f16(ta.zero_(), tb.zero_(), out=out)  # eager first: the plan's CU count is cached
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            binding.gemm_nt_f16(ta, tb, out=out)
        for r in range(4):
            print("case graph", M, N, K, "replay", r, flush=True)
            a, b = workloads.small_integers(M, N, K, seed=9000 + 10 * r + (M > 2000))
            ta.copy_(torch.from_numpy(a))
            tb.copy_(torch.from_numpy(b))
            out.fill_(float("nan"))
            binding.gemm_nt_f16(ta, tb, out=ref)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (M, N, K, r)
            if M * N * K <= 1 << 28:
                _, c16 = oracle.gemm_nt(a, b)
                assert np.array_equal(out.cpu().numpy().view(np.uint16), c16.view(np.uint16)), (M, N, K, r)
        del g


def test_non_default_stream():
    torch = _torch()
    a, b = workloads.gaussian(520, 390, 264, seed=43)
    c64, c16 = oracle.gemm_nt(a, b)
    s = torch.cuda.Stream()
    ta = torch.from_numpy(a).to(dev())
    tb = torch.from_numpy(b).to(dev())
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c = binding.gemm_nt_f16(ta, tb)
    s.synchronize()
    assert_close(c.cpu().numpy(), c64, c16, 264, "side stream")


def test_binding_makes_a_device_current_when_another_is(monkeypatch):
    """The binding calls the library with a's device current: when torch
    reports another current device it enters a's device for the call.  On
    one GPU the other device is simulated; the result is bit-identical to
    the ordinary call and to the oracle."""
    torch = _torch()
    a, b = workloads.gaussian(300, 200, 136, seed=47)
    c64, c16 = oracle.gemm_nt(a, b)
    ta = torch.from_numpy(a).to(dev())
    tb = torch.from_numpy(b).to(dev())
    ref = binding.gemm_nt_f16(ta, tb)
    entered = []
    real_device = torch.cuda.device

    class Tracking(real_device):
        def __enter__(self):
            entered.append(self.idx)
            return super().__enter__()

    # patched for the binding's call only: nothing else may see the simulated device
    with monkeypatch.context() as m:
        m.setattr(torch.cuda, "current_device", lambda: ta.get_device() + 1)
        m.setattr(torch.cuda, "device", Tracking)
        c = binding.gemm_nt_f16(ta, tb)
    torch.cuda.synchronize()
    assert entered == [ta.get_device()]
    assert torch.equal(c.view(torch.int16), ref.view(torch.int16))
    assert_close(c.cpu().numpy(), c64, c16, 136, "device switch")
