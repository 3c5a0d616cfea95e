"""Parity of the HIP path (through the C ABI) with the CPU oracle, on an MI355X.

* packed streams and unpacked codes: bit-exact;
* fp16 products: max|Y_gpu - Y_ref| / max|Y_ref| <= 4e-3, Y_ref the oracle's
  unrounded fp64 result; exactly zero when every code equals its zero-point;
* int8-activation product: the int32 per-group sums bit-exact, Y within 4e-3.
Small shapes cover several tiles, ragged tails and every k; the full
workload shapes are checked on outputs the oracle computes one by one.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu
TOL = 4e-3


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_weight_quantized_qmm_amd as qmm
    return qmm


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\nCASE {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def stream_bytes(wq):
    return wq.cpu().numpy().view(np.uint8).reshape(wq.shape[0], -1)


def rel_err(y_gpu, y_ref):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    den = np.abs(y_ref).max()
    return np.abs(y - y_ref).max() / den


def gpu_pack(q, codes, bits):
    return q.pack(dev(codes), bits)


def guarded(shape, dtype, guard=256):
    """Output tensor followed by a guard region filled with a canary pattern."""
    n = int(np.prod(shape))
    buf = torch.full((n + guard,), 0x5A if dtype == torch.uint8 else -7, dtype=dtype, device=DEV)
    return buf, buf[:n].view(*shape)


def guard_intact(buf, n):
    tail = buf[n:].cpu()
    return bool((tail == tail[0]).all()) and int(tail[0]) in (0x5A, -7)


# ------------------------------------------------------------- pack/unpack --
@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("K,N", [(32, 1), (96, 37), (256, 256), (4096, 300)])
def test_pack_unpack_bit_exact(q, orc, bits, K, N):
    c = synthetic.make_case(1, K, N, bits, 32, synthetic.seed_for(90, bits, K + N))
    wq = gpu_pack(q, c["codes"], bits)
    assert np.array_equal(stream_bytes(wq), orc.pack(c["codes"], bits))
    buf, out = guarded((K, N), torch.uint8)
    q.unpack(wq, K, N, bits, out=out)
    assert np.array_equal(out.cpu().numpy(), orc.unpack(orc.pack(c["codes"], bits), K, N, bits))
    assert guard_intact(buf, K * N)


def test_pack_masks_wide_codes(q, orc):
    g = synthetic.rng(5)
    wide = g.integers(0, 256, size=(128, 40), dtype=np.uint8)
    for bits in range(1, 8):
        assert np.array_equal(stream_bytes(gpu_pack(q, wide, bits)), orc.pack(wide, bits))


# ------------------------------------------------------------ fp16 products --
def run_product(q, fn, c):
    wq = gpu_pack(q, c["codes"], c["bits"])
    z = None if c["z"] is None else dev(c["z"])
    return fn(dev(c["X"]), wq, dev(c["s"]), z, c["bits"], c["G"])


GEMV_SHAPES = [(256, 40, 64), (96, 19, 32), (1024, 130, 128), (4096, 33, 32), (2048, 50, 256), (8192, 17, 128),
               (384, 70, 128), (1152, 33, 128)]


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("pgz", [False, True])
@pytest.mark.parametrize("K,N,G", GEMV_SHAPES, ids=lambda v: str(v))
def test_gemv_small(q, orc, bits, M, pgz, K, N, G):
    c = synthetic.make_case(M, K, N, bits, G, synthetic.seed_for(91, bits, M + K + N), per_group_z=pgz)
    Y = run_product(q, q.gemv, c)
    ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, G)
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("K,N,G,pgz", [(16416, 300, 32, False), (20480, 77, 128, True), (28672, 130, 128, False)],
                         ids=lambda v: str(v))
def test_gemv_m1_runs_in_lds(q, orc, bits, K, N, G, pgz):
    """M = 1 beyond 8 runs per lane (K > 16384): the decode kernel with 16 runs
    per lane, X read from LDS for every column; a ragged run count (K 16416,
    513 runs), the 70B MLP-down K, and both zero-point forms."""
    c = synthetic.make_case(1, K, N, bits, G, synthetic.seed_for(101, bits, K // 32), per_group_z=pgz)
    Y = run_product(q, q.gemv, c)
    ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, G)
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("M,K,N,pgz", [(2, 12288, 70, True), (8, 28672, 300, False), (16, 9216, 33, True)],
                         ids=lambda v: str(v))
def test_gemv_batched_long_k(q, orc, bits, M, K, N, pgz):
    """2 <= M <= 16 past K = 8192: the MFMA GEMV in passes of 4096 rows, each
    with its own s | z table and row exponents (K 9216: a last pass of one
    step per wave; K 28672: the 70B MLP-down)."""
    c = synthetic.make_case(M, K, N, bits, 128, synthetic.seed_for(102, bits, M * 100 + K // 1024), per_group_z=pgz)
    Y = run_product(q, q.gemv, c)
    ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, 128)
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", range(1, 9))
def test_gemv_m1_long_k(q, orc, bits):
    """K = 32768 (1024 runs, 16 per lane): the decode kernel's largest K, with
    X read from LDS for every column."""
    c = synthetic.make_case(1, 32768, 24, bits, 128, synthetic.seed_for(92, bits), per_group_z=True)
    Y = run_product(q, q.gemv, c)
    ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, 128)
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("M", [1, 7, 257])
def test_gemm_small(q, orc, bits, M):
    for (K, N, G, pgz) in ((384, 200, 128, False), (96, 37, 32, True), (512, 130, 64, True)):
        c = synthetic.make_case(M, K, N, bits, G, synthetic.seed_for(93, bits, M + K), per_group_z=pgz)
        Y = run_product(q, q.gemm, c)
        ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, G)
        assert rel_err(Y, ref) <= TOL, (K, N, G, pgz)


@pytest.mark.parametrize("pgz", [False, True])
@pytest.mark.parametrize("K,N,G", [(32, 5, 32), (256, 300, 64), (4096, 1000, 128), (8192, 257, 128), (2080, 70, 32),
                                   (8192, 28672, 128)], ids=lambda v: str(v))
def test_gemv_lut(q, orc, K, N, G, pgz):
    """The table-lookup product (1-bit codes, M = 1): one run, ragged run counts
    (2080 = 65 runs), the longest K its tables hold, and the 70B MLP-up shape
    (checked on sampled outputs)."""
    c = synthetic.make_case(1, K, N, 1, G, synthetic.seed_for(86, 1, K + N), per_group_z=pgz)
    Y = run_product(q, q.gemv_lut, c)
    if N > 4096:
        assert sampled_check(orc, Y, c, count=3000, seed=N) <= TOL
    else:
        ref = orc.qmm(c["X"], orc.pack(c["codes"], 1), c["s"], c["z"], 1, G)
        assert rel_err(Y, ref) <= TOL


def test_gemv_lut_reads_every_nibble(q, orc):
    """One-hot X at each of the 32 positions of a run (every nibble and every
    bit of it), all 16 nibble values present across the columns: the lookup
    returns s (q - z) exactly for each code."""
    K, N, G = 64, 64, 32
    codes = np.zeros((K, N), dtype=np.uint8)
    for n in range(N):
        codes[:, n] = (np.arange(K) * 7 + n) % 2
    s = synthetic.fp16_uniform(synthetic.rng(85), 0.5, 2.0, (N, K // G))
    z = synthetic.zeros_uniform(synthetic.rng(84), 1, N, K // G)
    wq = gpu_pack(q, codes, 1)
    for i in range(K):
        X = np.zeros((1, K), dtype=np.float16)
        X[0, i] = 1.0
        Y = q.gemv_lut(dev(X), wq, dev(s), dev(z), 1, G).cpu().numpy()
        expect = ((codes[i].astype(np.float64) - z[:, i // G]) * s[:, i // G]).astype(np.float16)
        assert np.array_equal(Y[0].astype(np.float64), expect.astype(np.float64)), i


def test_gemv_lut_rejects_unsupported(q):
    c = synthetic.make_case(2, 256, 8, 1, 64, 9)
    wq = gpu_pack(q, c["codes"], 1)
    with pytest.raises(q.QmmError):
        q.gemv_lut(dev(c["X"]), wq, dev(c["s"]), None, 1, 64)       # M = 2


@pytest.mark.parametrize("K,G", [(256, 64), (4096, 128), (8192, 128), (2080, 32)])
def test_gemv_grouped(q, orc, K, G):
    """Several decode products in one launch: every code width, ragged and
    tiny N, zero-points on some problems.  Each output equals the
    single-product qmm_gemv result bit for bit (same kernel body) and the
    oracle within the tolerance."""
    probs, cases = [], []
    for i, bits in enumerate([3, 4, 6, 1, 2, 5, 7, 8]):
        N = [300, 1000, 37, 2048, 5, 777, 64, 129][i]
        c = synthetic.make_case(1, K, N, bits, G, synthetic.seed_for(83, bits, K + i), per_group_z=(i % 3 == 1))
        wq = gpu_pack(q, c["codes"], bits)
        z = None if c["z"] is None else dev(c["z"])
        probs.append((dev(c["X"]), wq, dev(c["s"]), z, bits))
        cases.append(c)
    Ys = q.gemv_grouped(probs, G)
    for (X, wq, s, z, bits), c, Y in zip(probs, cases, Ys):
        assert torch.equal(Y.cpu(), q.gemv(X, wq, s, z, bits, G).cpu()), bits
        ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, G)
        assert rel_err(Y, ref) <= TOL, bits


def test_gemv_grouped_decode_step(q, orc):
    """The 7B MLP decode shapes at k = 3, 4 and 6 as one grouped launch (the
    launch the benchmark times), and a single-problem group."""
    w = synthetic.DECODE_7B
    probs, cases = [], []
    for bits in w["bits"]:
        c = synthetic.make_case(1, w["K"], w["N"], bits, w["G"], synthetic.seed_for(2, bits), s_range=w["s_range"])
        probs.append((dev(c["X"]), gpu_pack(q, c["codes"], bits), dev(c["s"]), None, bits))
        cases.append(c)
    for group in (probs, probs[1:2]):
        Ys = q.gemv_grouped(group, w["G"])
        for (X, wq, s, z, bits), Y in zip(group, Ys):
            c = cases[w["bits"].index(bits)]
            ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], None, bits, w["G"])
            assert rel_err(Y, ref) <= TOL, bits
            assert torch.equal(Y.cpu(), q.gemv(X, wq, s, z, bits, w["G"]).cpu()), bits


def test_gemv_grouped_sixteen_problems(q, orc):
    K, G = 512, 128
    probs, cases = [], []
    for i in range(16):
        bits = 1 + i % 8
        c = synthetic.make_case(1, K, 50 + 13 * i, bits, G, synthetic.seed_for(82, bits, i), per_group_z=(i % 2 == 0))
        probs.append((dev(c["X"]), gpu_pack(q, c["codes"], bits), dev(c["s"]), None if c["z"] is None else dev(c["z"]),
                      bits))
        cases.append(c)
    for (X, wq, s, z, bits), c, Y in zip(probs, cases, q.gemv_grouped(probs, G)):
        ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, G)
        assert rel_err(Y, ref) <= TOL


def _codes_at_zero_point(bits, M):
    K, N, G = 512, 70, 128
    g = synthetic.rng(99 + bits)
    z = synthetic.zeros_uniform(g, bits, N, K // G)
    codes = np.repeat(z.astype(np.uint8).T, G, axis=0)
    c = dict(bits=bits, G=G, X=synthetic.fp16_normal(g, (M, K)), codes=codes,
             s=synthetic.fp16_uniform(g, 0.002, 0.02, (N, K // G)), z=z)
    mid = dict(c, codes=np.full((K, N), 1 << (bits - 1), dtype=np.uint8), z=None)
    return c, mid


@pytest.mark.parametrize("bits", [1, 3, 4, 8])
def test_codes_equal_zero_point_give_exact_zero(q, bits):
    """q == z everywhere makes W == 0, so Y == 0.  The GEMM subtracts the
    zero-point bias from every weight in fp16 before any rounding (an exact
    difference), so it must return exact zeros."""
    for c in _codes_at_zero_point(bits, 5):
        Y = run_product(q, q.gemm, c)
        assert not Y.float().abs().max().item()


@pytest.mark.parametrize("bits", [1, 3, 4, 8])
@pytest.mark.parametrize("M", [1, 3, 5])
def test_codes_equal_zero_point_gemv_bounded(q, orc, bits, M):
    """Same invariant on the GEMV paths, which remove the zero-point bias from
    fp32 sums (per 32-code run at M = 1; as 1024 S1 + z S2 per 128-row step at
    M >= 2), so q == z leaves rounding residue there instead of exact zeros.
    The bound is the product tolerance itself: every |Y| must stay within
    4e-3 max|Y_ref| of the product with the same X, s and z and uniformly
    random codes (computed by the oracle), i.e. the residue is invisible at the
    stated tolerance.  M = 3 with G = 128 reaches the row-tile kernel too."""
    for c in _codes_at_zero_point(bits, M):
        Y = run_product(q, q.gemv, c).float().cpu().numpy()
        g = synthetic.rng(500 + bits + M)
        codes = synthetic.codes_uniform(g, bits, *c["codes"].shape)
        ref = orc.qmm(c["X"], orc.pack(codes, bits), c["s"], c["z"], bits, c["G"])
        bound = TOL * np.abs(ref).max()
        resid = float(np.abs(Y).max())
        print(f"zero-point residue: max|Y| = {resid:.3e} = {resid / np.abs(ref).max():.2e} max|Y_ref|", file=sys.stderr)
        assert resid <= bound, (resid, bound)


def _scaled_case(M, K, N, bits, G, seed, factor, pgz):
    c = synthetic.make_case(M, K, N, bits, G, seed, per_group_z=pgz)
    c["X"] = (c["X"].astype(np.float32) * factor).astype(np.float16)
    return c


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("factor", [1e-3, 1e-4])
@pytest.mark.parametrize("M,K,N,G,fn", [(1, 4096, 300, 128, "gemv"), (5, 2048, 70, 128, "gemv"),
                                        (3, 1024, 70, 64, "gemv"), (1, 32768, 24, 128, "gemv"),
                                        (9, 1024, 70, 64, "gemv"), (40, 512, 130, 128, "gemm")],
                         ids=lambda v: str(v))
def test_small_activations(q, orc, bits, factor, M, K, N, G, fn):
    """Activations of 1e-3 / 1e-4 (fp16 normal numbers whose products with
    2^-p would be fp16 subnormals): every path keeps the stated precision
    (M = 1 decode, M = 5 MFMA GEMV, M = 3 row tiles, long K, M = 9 with G = 64,
    the GEMM)."""
    c = _scaled_case(M, K, N, bits, G, synthetic.seed_for(88, bits, M + K), factor, pgz=(bits % 2 == 0))
    Y = run_product(q, getattr(q, fn), c)
    ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, G)
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", [1, 4, 8])
@pytest.mark.parametrize("M,fn", [(2, "gemv"), (16, "gemv"), (1, "gemv"), (64, "gemm")])
def test_large_same_sign_activations(q, orc, bits, M, fn):
    """Activations near 600, all of one sign: 128-row sums reach 7.7e4 (past the
    fp16 range), which the per-row normalisation must keep finite; s is scaled
    so that Y itself stays inside fp16."""
    K, N, G = 2048, 70, 128
    c = synthetic.make_case(M, K, N, bits, G, synthetic.seed_for(89, bits, M), per_group_z=True)
    c["X"] = (600.0 + c["X"].astype(np.float32)).astype(np.float16)
    c["s"] = (c["s"].astype(np.float32) * 2.0 ** -6).astype(np.float16)
    Y = run_product(q, getattr(q, fn), c)
    ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, G)
    assert np.isfinite(Y.float().cpu().numpy()).all()
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", [1, 4, 7, 8])
@pytest.mark.parametrize("pgz", [False, True])
def test_gemv_m1_wide_n(q, orc, bits, pgz):
    """M = 1 with more than 65536 columns (an LM-head shape): past the decode
    kernel's 64 columns per wave, the row-tile kernel with G % 128 == 0 runs."""
    c = synthetic.make_case(1, 256, 70001, bits, 128, synthetic.seed_for(87, bits), per_group_z=pgz)
    Y = run_product(q, q.gemv, c)
    ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, 128)
    assert rel_err(Y, ref) <= TOL


def test_deterministic(q):
    c = synthetic.make_case(16, 2048, 300, 5, 128, 7, per_group_z=True)
    wq = gpu_pack(q, c["codes"], 5)
    args = (dev(c["X"]), wq, dev(c["s"]), dev(c["z"]), 5, 128)
    for fn in (q.gemv, q.gemm):
        outs = [fn(*args).cpu() for _ in range(3)]
        assert all(torch.equal(outs[0], o) for o in outs[1:])
    x1 = dev(c["X"][:1])
    outs = [q.gemv(x1, *args[1:]).cpu() for _ in range(3)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_outputs_stay_in_bounds(q):
    c = synthetic.make_case(3, 256, 45, 4, 64, 8)
    wq = gpu_pack(q, c["codes"], 4)
    for fn in (q.gemv, q.gemm):
        buf, out = guarded((3, 45), torch.float16)
        fn(dev(c["X"]), wq, dev(c["s"]), None, 4, 64, out=out)
        torch.cuda.synchronize()
        assert guard_intact(buf, 3 * 45)


def test_invalid_arguments_raise(q):
    c = synthetic.make_case(17, 256, 16, 4, 64, 9)
    wq = gpu_pack(q, c["codes"], 4)
    with pytest.raises(q.QmmError):
        q.gemv(dev(c["X"]), wq, dev(c["s"]), None, 4, 64)          # M = 17 > 16


# ---------------------------------------------------------- full workloads --
def sampled_check(orc, Y, c, count=3000, seed=0, st=None):
    g = synthetic.rng(seed)
    M, N = Y.shape
    ms = g.integers(0, M, size=count)
    ns = g.integers(0, N, size=count)
    ms[:4] = [0, M - 1, 0, M - 1]
    ns[:4] = [0, N - 1, N - 1, 0]
    st = orc.pack(c["codes"], c["bits"]) if st is None else st
    ref = orc.qmm_sampled(c["X"], st, c["s"], c["z"], c["bits"], c["G"], ms, ns)
    y = Y.float().cpu().numpy()[ms, ns].astype(np.float64)
    return np.abs(y - ref).max() / np.abs(ref).max()


def test_tiny_workload(q, orc):
    w = synthetic.TINY
    c = synthetic.make_case(1, w["K"], w["N"], 4, w["G"], synthetic.seed_for(1, 4), s_range=w["s_range"])
    Y = run_product(q, q.gemv, c)
    ref = orc.qmm(c["X"], orc.pack(c["codes"], 4), c["s"], None, 4, w["G"])
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", synthetic.DECODE_7B["bits"])
def test_decode_7b_workload(q, orc, bits):
    w = synthetic.DECODE_7B
    c = synthetic.make_case(1, w["K"], w["N"], bits, w["G"], synthetic.seed_for(2, bits), s_range=w["s_range"])
    wq = gpu_pack(q, c["codes"], bits)
    st = orc.pack(c["codes"], bits)
    assert np.array_equal(stream_bytes(wq), st)
    assert np.array_equal(q.unpack(wq, w["K"], w["N"], bits).cpu().numpy(), orc.unpack(st, w["K"], w["N"], bits))
    Y = q.gemv(dev(c["X"]), wq, dev(c["s"]), None, bits, w["G"])
    ref = orc.qmm(c["X"], st, c["s"], None, bits, w["G"])
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", synthetic.BATCHED_70B["bits"])
def test_batched_70b_workload(q, orc, bits):
    w = synthetic.BATCHED_70B
    c = synthetic.make_case(16, w["K"], w["N"], bits, w["G"], synthetic.seed_for(3, bits), per_group_z=True,
                            s_range=w["s_range"])
    wq = gpu_pack(q, c["codes"], bits)
    st = orc.pack(c["codes"], bits)
    assert np.array_equal(stream_bytes(wq), st)
    assert np.array_equal(q.unpack(wq, w["K"], w["N"], bits).cpu().numpy(), c["codes"])
    s, z = dev(c["s"]), dev(c["z"])
    for M in w["Ms"]:
        cm = dict(c, X=c["X"][:M])
        Y = q.gemv(dev(cm["X"]), wq, s, z, bits, w["G"])
        assert sampled_check(orc, Y, cm, seed=M, st=st) <= TOL, M


@pytest.mark.parametrize("M,K,N,bits", [(2048, 256, 4096, 4), (1024, 512, 4056, 3), (1000, 1152, 4000, 3),
                                         (512, 512, 4096, 5), (500, 256, 4000, 8), (256, 512, 4096, 4),
                                         (130, 512, 4000, 4), (130, 1152, 3000, 6), (130, 512, 300, 4),
                                         (17, 1024, 2000, 6), (100, 1152, 1000, 7)])
def test_gemm_tile_shapes(q, orc, M, K, N, bits):
    """Shapes that select each GEMM tile on a 256-CU part: 128 x 256 (M 2048),
    128 x 128 in 2 K parts (M 1000, 1024), 64 x 128 (M 500, 512), 64 x 64 in 2
    parts (M 256), 64 x 32 in 4 parts (M 130, N 3000-4000), 32 x 16 in 8 parts
    (the small products); ragged M and N edges, and K = 1152 (9 steps) so the
    K parts are uneven and some get no step at all.  All checked against the
    oracle in full."""
    c = synthetic.make_case(M, K, N, bits, 128, 560 + M + N + bits, per_group_z=(bits == 5))
    Y = run_product(q, q.gemm, c)
    ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, 128)
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", [1, 3, 4, 8])
@pytest.mark.parametrize("M,fn", [(1, "gemv"), (5, "gemv"), (16, "gemv"), (130, "gemm"), (300, "gemm")])
@pytest.mark.parametrize("K,G", [(480, 96), (1600, 160), (2240, 224), (3328, 416)])
def test_group_sizes_not_power_of_two(q, orc, bits, M, fn, K, G):
    """Groups of 3, 5, 7 and 13 runs of 32: the kernels find a run's group as
    r / (G / 32) through a rounded reciprocal, which is inexact for these, and
    the groups straddle the 128-row K steps."""
    N = 70 if fn == "gemv" else 300
    c = synthetic.make_case(M, K, N, bits, G, synthetic.seed_for(100, bits, M * 1000 + G), per_group_z=(bits != 4))
    Y = run_product(q, getattr(q, fn), c)
    ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, G)
    assert rel_err(Y, ref) <= TOL


def test_prefill_workload(q, orc):
    """The prefill shape: 4000 sampled outputs, plus 16 whole rows (one in every
    128-row tile, at varying offsets inside the tile) against the oracle."""
    w = synthetic.PREFILL
    c = synthetic.make_case(w["M"], w["K"], w["N"], 4, w["G"], synthetic.seed_for(4, 4), s_range=w["s_range"])
    Y = run_product(q, q.gemm, c)
    assert sampled_check(orc, Y, c, count=4000) <= TOL
    rows = [128 * t + (37 * t) % 128 for t in range(16)]
    ref = orc.qmm(c["X"][rows], orc.pack(c["codes"], 4), c["s"], None, 4, w["G"])
    assert rel_err(Y[rows], ref) <= TOL


# ------------------------------------------------------------------ W4A8 ---
def run_w4a8(q, c, with_acc=True):
    wq = gpu_pack(q, c["codes"], 4)
    M, K = c["Xq"].shape
    N = c["codes"].shape[1]
    acc = torch.full((M, K // c["G"], N), -12345, dtype=torch.int32, device=DEV) if with_acc else None
    z = None if c["z"] is None else dev(c["z"])
    Y = q.gemm_w4a8(dev(c["Xq"]), dev(c["sx"]), wq, dev(c["s"]), z, c["G"], acc_out=acc)
    return Y, acc


def same_without_dump(Y, Y2):
    """The kernels are compiled with and without the dump of the int32 sums;
    both must produce the same Y bit for bit."""
    assert torch.equal(Y.cpu().view(torch.int16), Y2.cpu().view(torch.int16))


@pytest.mark.parametrize("M", [1, 5, 16, 17, 33])
@pytest.mark.parametrize("G,pgz", [(128, False), (128, True), (256, True)])
def test_w4a8_small(q, orc, M, G, pgz):
    K, N = 1024, 70
    c = synthetic.make_w4a8_case(M, K, N, G, synthetic.seed_for(95, M, G), per_group_z=pgz)
    Y, acc = run_w4a8(q, c)
    A, ref = orc.w4a8(c["Xq"], c["sx"], orc.pack(c["codes"], 4), c["s"], c["z"], G)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), A)
    assert rel_err(Y, ref) <= TOL
    same_without_dump(Y, run_w4a8(q, c, with_acc=False)[0])


@pytest.mark.parametrize("M,K,N,G,pgz", [(3, 2048, 50, 512, True), (16, 2048, 33, 1024, False),
                                          (8, 8192, 40, 128, True), (2, 16384, 20, 256, False),
                                          (40, 3072, 65, 128, True)])
def test_w4a8_shapes(q, orc, M, K, N, G, pgz):
    """Groups spanning several 128-row steps, K slices that leave waves idle, and
    K beyond the streaming kernel's register slice (the tiled kernel)."""
    c = synthetic.make_w4a8_case(M, K, N, G, synthetic.seed_for(96, M, K // 128), per_group_z=pgz)
    Y, acc = run_w4a8(q, c)
    A, ref = orc.w4a8(c["Xq"], c["sx"], orc.pack(c["codes"], 4), c["s"], c["z"], G)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), A)
    assert rel_err(Y, ref) <= TOL
    same_without_dump(Y, run_w4a8(q, c, with_acc=False)[0])


def test_w4a8_extreme_activations(q, orc):
    """-128 everywhere and codes at the ends of their range: int32 sums still exact."""
    M, K, N, G = 16, 512, 40, 128
    c = synthetic.make_w4a8_case(M, K, N, G, 11, per_group_z=True)
    c["Xq"][:] = -128
    c["codes"][:, ::2] = 15
    Y, acc = run_w4a8(q, c)
    A, ref = orc.w4a8(c["Xq"], c["sx"], orc.pack(c["codes"], 4), c["s"], c["z"], G)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), A)
    assert rel_err(Y, ref) <= TOL


def test_w4a8_workload(q, orc):
    w = synthetic.W4A8_8B
    c = synthetic.make_w4a8_case(w["M"], w["K"], w["N"], w["G"], synthetic.seed_for(5, 4))
    Y, acc = run_w4a8(q, c)
    A, ref = orc.w4a8(c["Xq"], c["sx"], orc.pack(c["codes"], 4), c["s"], None, w["G"])
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), A)
    assert rel_err(Y, ref) <= TOL
    Y2, _ = run_w4a8(q, c, with_acc=False)
    assert torch.equal(Y.cpu(), Y2.cpu())


# ------------------------------------------------- WkA8 (any code width) ---
def run_wka8(q, c, bits, with_acc=True):
    wq = gpu_pack(q, c["codes"], bits)
    M, K = c["Xq"].shape
    N = c["codes"].shape[1]
    acc = torch.full((M, K // c["G"], N), -12345, dtype=torch.int32, device=DEV) if with_acc else None
    z = None if c["z"] is None else dev(c["z"])
    Y = q.gemm_wka8(dev(c["Xq"]), dev(c["sx"]), wq, dev(c["s"]), z, bits, c["G"], acc_out=acc)
    return Y, acc


def check_wka8(orc, c, bits, Y, acc):
    A, ref = orc.w4a8(c["Xq"], c["sx"], orc.pack(c["codes"], bits), c["s"], c["z"], c["G"], bits=bits)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), A)
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("M", [1, 5, 17])
@pytest.mark.parametrize("G,pgz", [(128, False), (256, True)])
def test_wka8_small(q, orc, bits, M, G, pgz):
    """Every code width through the streaming kernel: several column tiles, a
    ragged column tail and a ragged M tile."""
    K, N = 1024, 70
    c = synthetic.make_w4a8_case(M, K, N, G, synthetic.seed_for(97, bits, M + G), bits=bits, per_group_z=pgz)
    Y, acc = run_wka8(q, c, bits)
    check_wka8(orc, c, bits, Y, acc)
    same_without_dump(Y, run_wka8(q, c, bits, with_acc=False)[0])


@pytest.mark.parametrize("bits,M,K,N,G,pgz", [(8, 3, 2048, 50, 512, True), (3, 16, 2048, 33, 1024, False),
                                               (7, 8, 8192, 40, 128, True), (1, 2, 16384, 20, 256, False),
                                               (5, 40, 3072, 65, 128, True), (6, 4, 16384, 24, 128, True),
                                               (2, 9, 4096, 300, 128, False)])
def test_wka8_shapes(q, orc, bits, M, K, N, G, pgz):
    """Groups spanning several steps, K slices that leave waves idle, and K past
    the streaming kernel's register slice (the tiled kernel)."""
    c = synthetic.make_w4a8_case(M, K, N, G, synthetic.seed_for(98, bits, M), bits=bits, per_group_z=pgz)
    Y, acc = run_wka8(q, c, bits)
    check_wka8(orc, c, bits, Y, acc)
    same_without_dump(Y, run_wka8(q, c, bits, with_acc=False)[0])


@pytest.mark.parametrize("bits", [2, 5, 8])
@pytest.mark.parametrize("K,G", [(512, 128), (16384, 1024)])
def test_wka8_extreme(q, orc, bits, K, G):
    """-128 activations against the largest and smallest codes with zero-points
    at both ends: the int32 sums reach their largest magnitudes and stay exact."""
    M, N = 16, 40
    c = synthetic.make_w4a8_case(M, K, N, G, 12 + bits, bits=bits, per_group_z=True)
    c["Xq"][:] = -128
    c["codes"][:, ::2] = (1 << bits) - 1
    c["codes"][:, 1::2] = 0
    c["z"][::2, :] = 0
    c["z"][1::2, :] = (1 << bits) - 1
    # scale s by a power of two (exact; A does not depend on s) so that Y stays
    # inside the fp16 range
    _, ref = orc.w4a8(c["Xq"], c["sx"], orc.pack(c["codes"], bits), c["s"], c["z"], G, bits=bits)
    e = max(0, int(np.ceil(np.log2(np.abs(ref).max() / 16384.0))))
    c["s"] = (c["s"].astype(np.float32) / (1 << e)).astype(np.float16)
    Y, acc = run_wka8(q, c, bits)
    check_wka8(orc, c, bits, Y, acc)
    same_without_dump(Y, run_wka8(q, c, bits, with_acc=False)[0])


def test_wka8_four_bits_is_w4a8(q):
    """The general entry point at k = 4 is the W4A8 product, bit for bit."""
    c = synthetic.make_w4a8_case(16, 2048, 100, 128, 31, per_group_z=True)
    Y4, acc4 = run_w4a8(q, c)
    Yk, acck = run_wka8(q, c, 4)
    assert torch.equal(Y4.cpu(), Yk.cpu()) and torch.equal(acc4.cpu(), acck.cpu())


def test_w8a8_workload(q, orc):
    """The 8B MLP shape with 8-bit weights (the W8A8 setting), checked whole."""
    w = synthetic.W4A8_8B
    c = synthetic.make_w4a8_case(w["M"], w["K"], w["N"], w["G"], synthetic.seed_for(5, 8), bits=8)
    Y, acc = run_wka8(q, c, 8)
    check_wka8(orc, c, 8, Y, acc)
    Y2, _ = run_wka8(q, c, 8, with_acc=False)
    assert torch.equal(Y.cpu(), Y2.cpu())


# ------------------------------------------------------------- quantiser ---
def check_quantize(q, orc, W, bits, G):
    codes, s, z = q.quantize(dev(W), bits, G)
    cx, sx, zx = orc.quantize(W, bits, G)
    assert np.array_equal(codes.cpu().numpy(), cx)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), sx.view(np.uint16))
    assert np.array_equal(z.cpu().numpy().view(np.uint16), zx.view(np.uint16))
    return codes, s, z


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("K,N,G", [(256, 300, 64), (1024, 70, 128), (1024, 196, 128), (96, 513, 32), (480, 132, 96),
                                   (1600, 77, 160), (512, 260, 256), (1024, 68, 512), (2048, 33, 1024)])
def test_quantize_small(q, orc, bits, K, N, G):
    """Codes, s and z bit-exact on LLM-like weights: several column blocks and
    a ragged column tail; groups of 2 to 16 rows per lane in the one-pass
    kernel (G 32 .. 256, odd counts at G 96 and 160; G 128 with N a multiple
    of 4 takes its form compiled for 8 rows per lane) and the two-pass kernel
    beyond (G 512, 1024)."""
    rng = np.random.default_rng(synthetic.seed_for(99, bits, K + N))
    W = rng.normal(0.0, 0.02, (K, N)).astype(np.float16)
    W[:, ::7] *= np.float16(8.0)                   # a few wide columns
    check_quantize(q, orc, W, bits, G)


@pytest.mark.parametrize("G", [32, 128])
@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_quantize_special_groups(q, orc, bits, G):
    """Constant groups (zero, positive, negative), a range past the fp16 scale, a
    scale that underflows, exact rounding ties, and the largest fp16 values
    (at G 128 a column's special rows share one group)."""
    K, N = 128, 260
    rng = np.random.default_rng(41 + bits)
    W = rng.normal(0.0, 0.05, (K, N)).astype(np.float16)
    W[0:32, 1] = 0
    W[32:64, 1] = np.float16(0.75)
    W[64:96, 1] = np.float16(-3.0)
    W[0:32, 2] = np.float16(-60000.0)
    W[1, 2] = np.float16(60000.0)
    W[32:64, 2] = np.float16(2.0 ** -24)
    W[64:96, 2] = np.tile(np.array([0, 3, 0.5, 1.5, 2.5, 0.5, 1.5, 2.5, 1, 2, 0, 3, 2.5, 0.5, 1.5, 3],
                                   dtype=np.float16), 2)
    W[0:32, 3] = np.float16(65504.0)
    W[0:32, 4] = np.float16(-65504.0)
    W[:, 259] = np.arange(K, dtype=np.float16) * np.float16(0.25)
    check_quantize(q, orc, W, bits, G)


def test_quantize_feeds_the_product(q, orc):
    """quantize -> pack -> qmm_gemv on the 7B decode shape: codes, s, z bit-exact,
    and the product of the quantised weights within tolerance of the oracle."""
    w = synthetic.DECODE_7B
    K, N, G = w["K"], w["N"], w["G"]
    rng = np.random.default_rng(synthetic.seed_for(2, 4, 77))
    W = rng.normal(0.0, 0.02, (K, N)).astype(np.float16)
    codes, s, z = check_quantize(q, orc, W, 4, G)
    X = synthetic.fp16_normal(synthetic.rng(5), (1, K))
    wq = q.pack(codes, 4)
    Y = q.gemv(dev(X), wq, s, z, 4, G)
    cx, sx, zx = orc.quantize(W, 4, G)
    ref = orc.qmm(X, orc.pack(cx, 4), sx, zx, 4, G)
    assert rel_err(Y, ref) <= TOL


# ------------------------------------- more column tiles than one round ---
@pytest.mark.parametrize("bits,M,pgz", [(3, 8, True), (8, 2, False), (5, 16, True)])
def test_gemv_many_tiles(q, orc, bits, M, pgz):
    """More 16-column tiles than 8 per CU: the M >= 2 kernel's workgroups run in
    several rounds, the last one ragged (N not a multiple of 16)."""
    K, N, G = 1024, 40003, 128
    c = synthetic.make_case(M, K, N, bits, G, synthetic.seed_for(93, bits, M), per_group_z=pgz)
    Y = run_product(q, q.gemv, c)
    ref = orc.qmm(c["X"], orc.pack(c["codes"], bits), c["s"], c["z"], bits, G)
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", [4, 8, 3])
def test_wka8_many_tiles(q, orc, bits):
    """The int8-activation streaming kernel past one round of workgroups, two M
    tiles, a ragged column tail; int32 group sums bit-exact."""
    M, K, N, G = 20, 1024, 40003, 256
    c = synthetic.make_w4a8_case(M, K, N, G, synthetic.seed_for(94, bits), bits=bits, per_group_z=True)
    Y, acc = run_wka8(q, c, bits)
    check_wka8(orc, c, bits, Y, acc)


# ------------------------------ int8 activations at prefill size (tiled) ---
# Products whose M x N passes about 1.9 M (one round of 128 x 256 tiles costs
# less than the streaming kernel's pass per 16 rows) take the tiled i8-MFMA
# kernel for k <= 7; 1100 x 1800 is just past that, with ragged M and N tiles.
GEMM8_M, GEMM8_N = 1100, 1800


@pytest.mark.parametrize("bits", range(1, 8))
@pytest.mark.parametrize("K,G,pgz", [(512, 128, False), (1024, 256, True), (1024, 512, False), (2048, 1024, True),
                                     (1152, 128, True), (640, 128, False), (128, 128, True), (256, 256, False)])
def test_wka8_gemm_shapes(q, orc, bits, K, G, pgz):
    """The tiled int8 kernel: ragged M and N tiles, groups of 1, 2, 4 and 8 K
    steps, an odd number of one-step groups (the loop's unpaired last step), a
    single group (K = G: no group before it, its sums added after the loop),
    the default and per-group zero-points; int32 group sums bit-exact."""
    c = synthetic.make_w4a8_case(GEMM8_M, K, GEMM8_N, G, synthetic.seed_for(99, bits, K // G), bits=bits,
                                 per_group_z=pgz)
    Y, acc = run_wka8(q, c, bits)
    check_wka8(orc, c, bits, Y, acc)
    Y2, _ = run_wka8(q, c, bits, with_acc=False)
    assert torch.equal(Y.cpu(), Y2.cpu())


@pytest.mark.parametrize("bits", [1, 4, 7])
def test_wka8_gemm_extreme(q, orc, bits):
    """-128 activations against the end codes, zero-points at both ends: the
    byte-wise q - z of the tiled kernel at its extremes, sums exact."""
    M, K, N, G = GEMM8_M, 512, GEMM8_N, 128
    c = synthetic.make_w4a8_case(M, K, N, G, 40 + bits, bits=bits, per_group_z=True)
    c["Xq"][::3] = -128
    c["codes"][:, ::2] = (1 << bits) - 1
    c["codes"][:, 1::2] = 0
    c["z"][::2, :] = 0
    c["z"][1::2, :] = (1 << bits) - 1
    _, ref = orc.w4a8(c["Xq"], c["sx"], orc.pack(c["codes"], bits), c["s"], c["z"], G, bits=bits)
    e = max(0, int(np.ceil(np.log2(np.abs(ref).max() / 16384.0))))
    c["s"] = (c["s"].astype(np.float32) / (1 << e)).astype(np.float16)
    Y, acc = run_wka8(q, c, bits)
    check_wka8(orc, c, bits, Y, acc)


def test_w4a8_prefill_workload(q, orc):
    """W4A8 at prefill size (M 2048, K = N = 4096, k 4, G 128), the shape the
    benchmark times: 16 whole rows of Y and of the int32 sums against the oracle."""
    M, K, N, G = 2048, 4096, 4096, 128
    c = synthetic.make_w4a8_case(M, K, N, G, synthetic.seed_for(5, 4, 7))
    Y, acc = run_w4a8(q, c)
    rows = [128 * t + (53 * t) % 128 for t in range(16)]
    A, ref = orc.w4a8(c["Xq"][rows], c["sx"][rows], orc.pack(c["codes"], 4), c["s"], None, G)
    assert np.array_equal(acc[rows].cpu().numpy().astype(np.int64), A)
    assert rel_err(Y[rows], ref) <= TOL
    del acc


# ---------------------------------------------------------- signed codes ---
def signed_codes(bits, K, N, seed):
    g = synthetic.rng(seed)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    q = g.integers(lo, hi + 1, (K, N))
    q[0, :], q[1, :] = lo, hi
    return q.astype(np.int8)


@pytest.mark.parametrize("bits", range(1, 9))
def test_pack_signed(q, orc, bits):
    K, N = 256, 37
    qs = signed_codes(bits, K, N, 300 + bits)
    wq = q.pack_signed(dev(qs), bits)
    assert np.array_equal(stream_bytes(wq), orc.pack_signed(qs, bits))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("M", [1, 5, 40])
def test_signed_codes_product(q, orc, bits, M):
    """Signed codes with the default zero-point through qmm_gemv (M <= 16) or
    qmm_gemm: Y = X (q s), checked against the oracle and against the numpy
    closed form of the signed definition."""
    K, N, G = 512, 70, 128
    qs = signed_codes(bits, K, N, 310 + bits + M)
    c = synthetic.make_case(M, K, N, bits, G, 320 + bits + M)
    wq = q.pack_signed(dev(qs), bits)
    fn = q.gemv if M <= 16 else q.gemm
    Y = fn(dev(c["X"]), wq, dev(c["s"]), None, bits, G)
    ref = orc.qmm(c["X"], orc.pack_signed(qs, bits), c["s"], None, bits, G)
    direct = c["X"].astype(np.float64) @ (qs.astype(np.float64) * np.repeat(c["s"].astype(np.float64).T, G, axis=0))
    assert np.abs(ref - direct).max() <= 1e-9 * np.abs(direct).max()
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_signed_codes_int8_activations(q, orc, bits):
    """Signed codes on the int8-activation path: int32 group sums exact."""
    M, K, N, G = 16, 1024, 50, 128
    qs = signed_codes(bits, K, N, 330 + bits)
    c = synthetic.make_w4a8_case(M, K, N, G, 340 + bits, bits=bits)
    wq = q.pack_signed(dev(qs), bits)
    acc = torch.zeros((M, K // G, N), dtype=torch.int32, device=DEV)
    Y = q.gemm_wka8(dev(c["Xq"]), dev(c["sx"]), wq, dev(c["s"]), None, bits, G, acc_out=acc)
    A, ref = orc.w4a8(c["Xq"], c["sx"], orc.pack_signed(qs, bits), c["s"], None, G, bits=bits)
    direct = np.stack([c["Xq"][:, g * G:(g + 1) * G].astype(np.int64) @ qs[g * G:(g + 1) * G].astype(np.int64)
                       for g in range(K // G)], axis=1)
    assert np.array_equal(A, direct)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), A)
    assert rel_err(Y, ref) <= TOL


# ------------------------------------------------------ smallest shapes ---
@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("M", [1, 2, 16, 17])
@pytest.mark.parametrize("K,N,G", [(32, 1, 32), (128, 1, 128), (128, 3, 32)])
def test_smallest_products(q, orc, bits, M, K, N, G):
    """One run or one 128-row step, one to three columns: every product entry
    point that takes the shape (qmm_gemv for M <= 16, qmm_gemm always).

    With one or three outputs, max|Y| can be a small residue of cancelling
    terms, and max|dY| / max|Y| is then ill-conditioned (the GEMM's one
    rounding per weight is 2^-11 of each |x w| term).  The error is bounded
    instead by 4e-3 of max(|X| |W|), which any indexing mistake (an error of
    the size of the terms) still exceeds."""
    c = synthetic.make_case(M, K, N, bits, G, synthetic.seed_for(92, bits, M + K + N), per_group_z=True)
    st = orc.pack(c["codes"], bits)
    ref = orc.qmm(c["X"], st, c["s"], c["z"], bits, G)
    scale = (np.abs(c["X"].astype(np.float64)) @ np.abs(orc.dequant(st, c["s"], c["z"], K, N, bits, G))).max()
    fns = [q.gemm] + ([q.gemv] if M <= 16 else [])
    for fn in fns:
        Y = run_product(q, fn, c)
        err = np.abs(Y.float().cpu().numpy().astype(np.float64) - ref).max()
        assert err <= TOL * scale, (fn.__name__, err, scale)


@pytest.mark.parametrize("bits", [1, 4, 8])
@pytest.mark.parametrize("M,N", [(1, 1), (17, 3)])
def test_smallest_int8_products(q, orc, bits, M, N):
    """One 128-row group, one to three columns, on the int8-activation path."""
    K, G = 128, 128
    c = synthetic.make_w4a8_case(M, K, N, G, synthetic.seed_for(95, bits, M + N), bits=bits, per_group_z=True)
    Y, acc = run_wka8(q, c, bits)
    check_wka8(orc, c, bits, Y, acc)


@pytest.mark.parametrize("bits", [1, 4, 8])
def test_smallest_quantize(q, orc, bits):
    W = synthetic.fp16_normal(synthetic.rng(96 + bits), (32, 1))
    check_quantize(q, orc, W, bits, 32)


# ------------------------------------------------- floating-point codes ---
FP_FORMATS = [0, 1, 2, 3, 4, 5, 6]   # E2M1, E4M3, E3M2, E2M3, E1M1, E2M2, E3M3
FP_WIDTH = {0: 4, 1: 8, 2: 6, 3: 6, 4: 3, 5: 5, 6: 7}


def fp_codes(fmt, K, N, seed):
    g = synthetic.rng(seed)
    q = g.integers(0, 1 << FP_WIDTH[fmt], (K, N))
    if fmt == 1:
        q[(q & 0x7F) == 0x7F] = 0x30        # NaN patterns are not weights
    return q.astype(np.uint8)


def all_fp_codes(fmt):
    """Every valid code of a format (E4M3 without its two NaN patterns)."""
    allq = np.arange(1 << FP_WIDTH[fmt])
    return allq[(allq & 0x7F) != 0x7F] if fmt == 1 else allq


@pytest.mark.parametrize("fmt", FP_FORMATS)
@pytest.mark.parametrize("M", [1, 5, 130])
@pytest.mark.parametrize("G", [64, 128])
def test_gemm_fp_codes(q, orc, fmt, M, G):
    """Float codes of every format through qmm_gemm_fp: several tiles, ragged M and N."""
    K, N = 512, 300
    bits = orc.FP_BITS[fmt]
    codes = fp_codes(fmt, K, N, 400 + fmt + M + G)
    c = synthetic.make_case(M, K, N, bits, G, 410 + fmt + M + G)
    wq = q.pack(dev(codes), bits)
    Y = q.gemm_fp(dev(c["X"]), wq, dev(c["s"]), fmt, G)
    ref = orc.qmm_fp(c["X"], orc.pack(codes, bits), c["s"], fmt, G)
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("fmt", FP_FORMATS)
@pytest.mark.parametrize("K,N,G", [(32, 7, 32), (1056, 301, 32), (4096, 11008, 128), (8192, 1000, 128),
                                   (16384, 515, 256), (16416, 64, 32)])
def test_gemm_fp_decode_shapes(q, orc, fmt, K, N, G):
    """M = 1 float-code products: one run, a ragged run count, the 7B MLP decode
    shape (2 runs per lane), 4 and 8 runs per lane (the longest K the decode
    kernel takes) and one run past it (the GEMM kernel)."""
    bits = orc.FP_BITS[fmt]
    codes = fp_codes(fmt, K, N, 430 + fmt + K)
    c = synthetic.make_case(1, K, N, bits, G, 440 + fmt + K)
    wq = q.pack(dev(codes), bits)
    Y = q.gemm_fp(dev(c["X"]), wq, dev(c["s"]), fmt, G)
    ref = orc.qmm_fp(c["X"], orc.pack(codes, bits), c["s"], fmt, G)
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("fmt", FP_FORMATS)
def test_gemm_fp_decode_reads_every_code_exactly(q, orc, fmt):
    """M = 1, X one-hot at row i: Y[n] = fp16(value(q[i, n]) s) for every code,
    each in its own column, at a row in the middle of a run and of a group."""
    bits = orc.FP_BITS[fmt]
    allq = all_fp_codes(fmt)
    K, G = 512, 128
    N = len(allq)
    s = synthetic.fp16_uniform(synthetic.rng(450 + fmt), 0.5, 2.0, (N, K // G))
    for i in (0, 45, 511):
        codes = np.asarray(synthetic.rng(460 + i).integers(0, 16, (K, N)), dtype=np.uint8)
        codes[i, :] = allq
        X = np.zeros((1, K), dtype=np.float16)
        X[0, i] = 1.0
        Y = q.gemm_fp(dev(X), q.pack(dev(codes), bits), dev(s), fmt, G).cpu().numpy()
        vals = np.array([orc.float_code_value(int(v), fmt) for v in allq])
        expect = (vals * s[:, i // G].astype(np.float64)).astype(np.float16)
        assert np.array_equal(Y[0].astype(np.float64), expect.astype(np.float64)), i


@pytest.mark.parametrize("fmt", FP_FORMATS)
@pytest.mark.parametrize("M,K,N,G", [(2, 128, 17, 128), (8, 4096, 11008, 128), (16, 4096, 11008, 128),
                                     (16, 8192, 1000, 256),
                                     (3, 1024, 300, 1024), (16, 8320, 40, 128), (4, 12288, 70, 128)])
def test_gemm_fp_batched_shapes(q, orc, fmt, M, K, N, G):
    """2 <= M <= 16 float-code products: one 128-row step with a ragged tile,
    the 7B MLP shape at M 8, the longest one-pass K of the MFMA GEMV, one
    group per column, and K past it (passes of 4096 rows: a last pass of one
    step per wave at K 8320, three passes at K 12288)."""
    bits = orc.FP_BITS[fmt]
    codes = fp_codes(fmt, K, N, 470 + fmt + K + M)
    c = synthetic.make_case(M, K, N, bits, G, 480 + fmt + K + M)
    wq = q.pack(dev(codes), bits)
    Y = q.gemm_fp(dev(c["X"]), wq, dev(c["s"]), fmt, G)
    ref = orc.qmm_fp(c["X"], orc.pack(codes, bits), c["s"], fmt, G)
    assert rel_err(Y, ref) <= TOL


@pytest.mark.parametrize("fmt", FP_FORMATS)
def test_gemm_fp_batched_reads_every_code_exactly(q, orc, fmt):
    """M = 16, row m of X one-hot at a different row i_m (even and odd code
    positions, run and group boundaries): Y[m][n] = fp16(value(q[i_m][n]) s)."""
    bits = orc.FP_BITS[fmt]
    allq = all_fp_codes(fmt)
    K, G = 512, 128
    N = len(allq)
    rows = [0, 1, 13, 31, 32, 45, 127, 128, 255, 256, 300, 383, 400, 450, 500, 511]
    codes = np.asarray(synthetic.rng(490 + fmt).integers(0, 16, (K, N)), dtype=np.uint8)
    X = np.zeros((16, K), dtype=np.float16)
    for m, i in enumerate(rows):
        codes[i, :] = np.roll(allq, 3 * m)
        X[m, i] = 1.0
    s = synthetic.fp16_uniform(synthetic.rng(495 + fmt), 0.5, 2.0, (N, K // G))
    Y = q.gemm_fp(dev(X), q.pack(dev(codes), bits), dev(s), fmt, G).cpu().numpy()
    for m, i in enumerate(rows):
        vals = np.array([orc.float_code_value(int(v), fmt) for v in codes[i]])
        expect = (vals * s[:, i // G].astype(np.float64)).astype(np.float16)
        assert np.array_equal(Y[m].astype(np.float64), expect.astype(np.float64)), (m, i)


@pytest.mark.parametrize("fmt", FP_FORMATS)
def test_gemm_fp_prefill_workload(q, orc, fmt):
    """The prefill shape (M 2048, K = N = 4096, G 128) in the launch the bench
    times; the oracle checks 16 rows of Y (first, last, tile edges, random) in
    full, since rows of Y are independent."""
    w = synthetic.PREFILL
    M, K, N, G = w["M"], w["K"], w["N"], w["G"]
    bits = orc.FP_BITS[fmt]
    codes = fp_codes(fmt, K, N, 520 + fmt)
    c = synthetic.make_case(M, K, N, bits, G, 530 + fmt, s_range=w["s_range"])
    wq = q.pack(dev(codes), bits)
    Y = q.gemm_fp(dev(c["X"]), wq, dev(c["s"]), fmt, G)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 1023, 1024, 2046, 2047],
                                     synthetic.rng(540 + fmt).integers(0, M, 8)]))
    ref = orc.qmm_fp(c["X"][rows], orc.pack(codes, bits), c["s"], fmt, G)
    assert rel_err(Y[torch.as_tensor(rows, device=Y.device)], ref) <= TOL


@pytest.mark.parametrize("fmt", FP_FORMATS)
def test_gemm_fp_decodes_every_code_exactly(q, orc, fmt):
    """One-hot rows of X read single weights back: Y = fp16(value(q) s) bit for bit
    for every code (both signs, subnormals, the largest values)."""
    bits = orc.FP_BITS[fmt]
    allq = all_fp_codes(fmt)
    K, G = 256, 128
    N = 64
    codes = np.zeros((K, N), dtype=np.uint8)
    for idx, v in enumerate(allq):
        codes[idx % K, idx // K * 8 + idx % 8] = v      # spread over rows and columns
    M = K
    X = np.eye(K, dtype=np.float16)
    s = synthetic.fp16_uniform(synthetic.rng(420 + fmt), 0.5, 2.0, (N, K // G))
    wq = q.pack(dev(codes), bits)
    Y = q.gemm_fp(dev(X), wq, dev(s), fmt, G).cpu().numpy()
    vals = np.array([[orc.float_code_value(int(codes[i, n]), fmt) for n in range(N)] for i in range(K)])
    expect = (vals * np.repeat(s.astype(np.float64).T, G, axis=0)).astype(np.float16)
    # values, not bit patterns: -0 (E2M1 code 8) times one, plus +0 products, sums to +0
    assert np.array_equal(Y.astype(np.float64), expect.astype(np.float64))
