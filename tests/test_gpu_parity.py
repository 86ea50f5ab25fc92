"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: bit-exact on codes, packed bytes, scales, zero points, int8 activations,
int32 accumulators and W4A8 outputs (the W4A8 output is a fixed sequence of
fp32 roundings, so it must match bit for bit, which is stricter than the
1e-5 relative bound).  W4A16 outputs: fp32 accumulation in hardware order is
one of several correct results, so they are checked norm-wise
(||y - y_ref||_2 <= 1e-5 ||y_ref||_2) and element-wise against the fp32
summation bound |y - y_ref| <= gamma_K * sum_k |x_k w'_k| with
gamma_K = K u / (1 - K u), u = 2^-24.

Small cases run the oracle on the whole problem; full-size workloads run the
HIP path on the whole problem (in the launch configuration the benchmark
uses) and compare sampled rows / channels the oracle computes one by one
(rows of the W4A8 layer and channels of both layers are independent).
Output buffers sit between canary guard regions.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

W4 = None


@pytest.fixture(scope="module", autouse=True)
def w4():
    global W4
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_weight_quantized_amd as pkg
    pkg.lib()
    W4 = pkg
    return pkg


DEV = "cuda"
CANARY = {torch.uint8: 0xA5, torch.int8: -91, torch.float32: -12345.5, torch.int32: -0x5A5A5A5A}


def guarded(shape, dtype):
    """A contiguous output tensor with 256-byte canary regions on both sides."""
    n = int(np.prod(shape))
    pad = 256 // torch.tensor([], dtype=dtype).element_size()
    buf = torch.full((pad + n + pad,), CANARY[dtype], dtype=dtype, device=DEV)
    return buf, buf[pad:pad + n].view(*shape), pad


def guards_intact(buf, pad):
    c = CANARY[buf.dtype]
    head, tail = buf[:pad].cpu(), buf[-pad:].cpu()
    return bool((head == c).all()) and bool((tail == c).all())


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    if a.dtype == np.float32:
        return np.array_equal(a.view(np.uint32), b.astype(np.float32).view(np.uint32))
    return np.array_equal(a, b)


def report(name, got, want):
    bad = np.argwhere(~(got == want))
    return f"{name}: {len(bad)} mismatches, first {bad[:5].tolist()}"


# ---------------------------------------------------------- weight quantization
SYM_SHAPES = [(1, 1), (10, 32), (32, 1), (7, 5), (33, 70), (128, 64), (300, 129), (1152, 6912)]


@pytest.mark.parametrize("K,N", SYM_SHAPES)
def test_quantize_weight_sym(K, N):
    d = workloads.random_case(K * 13 + N, 1, K, N, sigma=0.02)
    W = d["W"]
    if N > 3:
        W[:, 3] = 0.0                            # all-zero channel
    if K >= 7 and N > 1:                         # exact ties at scale 1
        W[:7, 1] = [7, 2.5, -2.5, 0.5, -0.5, 1.5, -3.5]
        W[7:, 1] = 0
    pref, sref = oracle.quantize_weight_sym(W)
    bufp, packed, pp = guarded((N, (K + 1) // 2), torch.uint8)
    bufs, sw, ps = guarded((N,), torch.float32)
    W4.w4_quantize_weight(dev(W), "sym", 0, packed=packed, scales=sw)
    assert bits_equal(host(sw), sref)
    assert np.array_equal(host(packed), pref), report("packed", host(packed), pref)
    assert guards_intact(bufp, pp) and guards_intact(bufs, ps)


def test_quantize_weight_sym_full_7b():
    d = workloads.generate("mlp7b", M=1)
    pref, sref = oracle.quantize_weight_sym(d["W"])
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    assert bits_equal(host(sw), sref)
    assert np.array_equal(host(packed), pref)


ASYM_CASES = [(8, 3, 4), (64, 9, 32), (256, 70, 128), (384, 5, 128), (512, 33, 256), (1024, 130, 64)]


@pytest.mark.parametrize("K,N,g", ASYM_CASES)
def test_quantize_weight_asym(K, N, g):
    rng = np.random.default_rng(K + N + g)
    W = (rng.standard_normal((K, N)) * 0.015).astype(np.float32)
    W[:, 0] += 0.05                              # all-positive channel: zero point < 0
    if N > 2:
        W[:g, 2] = 0.25                          # degenerate (constant) group
    pref, sref, zref = oracle.quantize_weight_asym(W, g)
    bufp, packed, pp = guarded((N, K // 2), torch.uint8)
    packed_, s, z = W4.w4_quantize_weight(dev(W), "asym", g, packed=packed)
    assert np.array_equal(host(packed), pref), report("packed", host(packed), pref)
    assert bits_equal(host(s), sref) and bits_equal(host(z), zref)
    assert guards_intact(bufp, pp)


def test_quantize_weight_asym_full_70b_slice():
    """The 70B-class layer's weights, first 2048 channels (all of K)."""
    d = workloads.w4a16_inputs(N=2048)
    pref, sref, zref = oracle.quantize_weight_asym(d["W"], d["group"])
    packed, s, z = W4.w4_quantize_weight(dev(d["W"]), "asym", d["group"])
    assert np.array_equal(host(packed), pref)
    assert bits_equal(host(s), sref) and bits_equal(host(z), zref)


# ------------------------------------------------------------ activations
# K % 8 == 0 up to 16384 takes the register-resident quantizer (1, 2, 4 or 8
# groups of 8 per thread); other K, and K > 16384, the two-pass one
ACT_SHAPES = [(1, 1), (32, 10), (3, 33), (1, 1152), (8, 1152), (16, 4096), (64, 4096), (5, 1000),
              (4, 2056), (3, 8192), (2, 12296), (2, 16384), (2, 16392)]


@pytest.mark.parametrize("M,K", ACT_SHAPES)
def test_quantize_act(M, K):
    d = workloads.random_case(M * 7 + K, M, K, 1, outliers=min(6, K))
    X = d["x"]
    if M > 2:
        X[1] = 0.0                               # all-zero row
        X[2, : min(K, 6)] = [127, 0.5, 1.5, -2.5, -0.5, 126.5][: min(K, 6)]
    xq_ref, sx_ref = oracle.quantize_act(X)
    bufq, xq, pq = guarded((M, K), torch.int8)
    xq_, sx = W4.a8_quantize_act(dev(X), Xq=xq)
    assert np.array_equal(host(xq), xq_ref), report("xq", host(xq), xq_ref)
    assert bits_equal(host(sx), sx_ref)
    assert guards_intact(bufq, pq)


@pytest.mark.parametrize("M,K", [(3, 4096), (2, 1152)])
def test_quantize_act_misaligned(M, K):
    """fp32 rows starting 4 bytes past a 16-byte boundary and codes starting at
    an odd address (the two-pass quantizer): same bytes as the oracle."""
    d = workloads.random_case(M + K, M, K, 1, outliers=3)
    xref, sref = oracle.quantize_act(d["x"])
    xb = torch.zeros(M * K + 4, dtype=torch.float32, device=DEV)
    X = xb[1:1 + M * K].view(M, K)
    X.copy_(dev(d["x"]))
    qb = torch.zeros(M * K + 1, dtype=torch.int8, device=DEV)
    xq = qb[1:].view(M, K)
    _, sx = W4.a8_quantize_act(X, Xq=xq)
    assert np.array_equal(host(xq), xref) and bits_equal(host(sx), sref)


def _tiny_rows(M, K, seed):
    """Rows whose scales lie below 2^-64 (about 8e-33 and, subnormal, 8e-40),
    an all-zero row, and rows of ordinary magnitude, with subnormal values
    scattered in."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float32)
    for m in range(M):
        kind = m % 4
        if kind == 0:
            X[m] *= np.float32(1e-30)
        elif kind == 1:
            X[m] *= np.float32(1e-37)
        elif kind == 2:
            X[m] = 0.0
        X[m, rng.integers(0, K, 3)] = np.float32(1e-44)
    return X


@pytest.mark.parametrize("M,K,N,path", [(1, 1152, 64, "gemv_dot4"), (2, 4096, 40, "gemv_dot4"),
                                        (3, 4096, 40, "gemv_mfma_fused"),
                                        (4, 1152, 48, "gemv_mfma_fused"), (4, 4224, 48, "gemv_dot4"),
                                        (16, 512, 64, "gemv_mfma_fused"),
                                        (24, 512, 64, "gemv_mfma"),
                                        (100, 384, 260, "gemm_mfma")])
def test_tiny_activation_scales(M, K, N, path):
    """Row scales below 2^-64 take the rescaled division-free quotient: codes,
    scales and outputs still match the oracle's IEEE divisions bit for bit."""
    X = _tiny_rows(M, K, M + K)
    xq_ref, sx_ref = oracle.quantize_act(X)
    assert (sx_ref[1::4] < 2.0 ** -126).all() and (sx_ref[0::4] < 2.0 ** -64).all()
    xq, sx = W4.a8_quantize_act(dev(X))
    assert np.array_equal(host(xq), xq_ref) and bits_equal(host(sx), sx_ref)
    xb = torch.zeros(M * K + 1, dtype=torch.float32, device=DEV)   # misaligned rows
    xm = xb[1:].view(M, K)
    xm.copy_(dev(X))
    xq2, sx2 = W4.a8_quantize_act(xm)
    assert np.array_equal(host(xq2), xq_ref) and bits_equal(host(sx2), sx_ref)
    W = workloads.random_case(K + N, 1, K, N)["W"]
    pref, sref = oracle.quantize_weight_sym(W)
    yref = oracle.w4a8_linear(X, pref, sref)
    y = W4.w4a8_linear(dev(X), dev(pref), dev(sref))
    assert W4.w4_last_path() == path
    assert bits_equal(host(y), yref), report(f"y path={path}", host(y), yref)


def _tie_rows(M, K, seed):
    """Activation rows whose values sit on, and one ulp either side of, the
    rounding ties (k + 1/2) * sx of the int8 grid.  Even rows use a power-of-two
    scale (exact ties); odd rows a random scale (ties rounded to fp32)."""
    rng = np.random.default_rng(seed)
    X = np.empty((M, K), np.float32)
    for m in range(M):
        if m % 2 == 0:
            am = np.float32(127.0) * np.float32(2.0) ** np.float32(rng.integers(-8, 4))
        else:
            am = np.float32(rng.uniform(0.5, 60.0))
        s = np.float32(am / np.float32(127.0))
        k = rng.integers(-128, 127, K).astype(np.float32)
        tie = (k + np.float32(0.5)) * s
        kind = rng.integers(0, 3, K)
        up = np.nextafter(tie, np.float32(np.inf), dtype=np.float32)
        dn = np.nextafter(tie, np.float32(-np.inf), dtype=np.float32)
        row = np.where(kind == 0, tie, np.where(kind == 1, up, dn)).astype(np.float32)
        row = np.clip(row, -am, am)
        row[rng.integers(0, K)] = am if m % 3 else -am
        X[m] = row
    return X


@pytest.mark.parametrize("M,K", [(1, 1152), (2, 256), (4, 4096), (8, 1152), (1, 10), (100, 256)])
def test_activation_ties(M, K):
    """Values on and next to rounding ties: the standalone quantizer and the
    linear layer (whose decode path quantizes inside the product kernel)."""
    X = _tie_rows(M, K, M * 1000 + K)
    xq_ref, sx_ref = oracle.quantize_act(X)
    xq, sx = W4.a8_quantize_act(dev(X))
    assert np.array_equal(host(xq), xq_ref), report("xq", host(xq), xq_ref)
    assert bits_equal(host(sx), sx_ref)
    N = 64
    W = workloads.random_case(K, 1, K, N)["W"]
    pref, sref = oracle.quantize_weight_sym(W)
    yref = oracle.w4a8_linear(X, pref, sref)
    y = W4.w4a8_linear(dev(X), dev(pref), dev(sref))
    got = host(y)
    assert bits_equal(got, yref), report(f"y path={W4.w4_last_path()}", got, yref)


def test_quantize_act_prefill_full():
    d = workloads.generate("prefill", with_w=False)
    xq_ref, sx_ref = oracle.quantize_act(d["x"])
    xq, sx = W4.a8_quantize_act(dev(d["x"]))
    assert np.array_equal(host(xq), xq_ref)
    assert bits_equal(host(sx), sx_ref)


# ------------------------------------------------------- integer products
# (M, K, N): dot4 GEMV (M<=4, K%32==0), MFMA GEMV (M<=64, K%128==0),
# MFMA GEMM (M>64, K%128==0) and the generic kernel, with ragged edges.
I32_CASES = [
    (1, 128, 16), (1, 1152, 100), (2, 4096, 33), (3, 96, 17), (4, 1152, 257),
    (5, 128, 16), (8, 1152, 130), (16, 4096, 96), (17, 256, 65), (33, 512, 31), (64, 1152, 200),
    (65, 128, 130), (130, 256, 129), (256, 1152, 384), (300, 512, 1000),
    (1, 10, 32), (32, 10, 32), (32, 32, 1), (6, 96, 20), (3, 7, 5), (70, 200, 9),
]


@pytest.mark.parametrize("M,K,N", I32_CASES)
def test_matmul_i32(M, K, N):
    xq = workloads.random_int8(M * 31 + K, (M, K))
    packed = workloads.random_bytes(K * 17 + N, (N, (K + 1) // 2))  # every nibble incl. -8
    if K % 2:
        packed[:, -1] &= 0x0F
    ref = oracle.matmul_i32(xq, packed, K)
    bufa, acc, pa = guarded((M, N), torch.int32)
    W4.w4a8_matmul_i32(dev(xq), dev(packed), acc=acc)
    got = host(acc)
    assert np.array_equal(got, ref), report(f"acc path={W4.w4_last_path()}", got, ref)
    assert guards_intact(bufa, pa)


def test_matmul_i32_extremes():
    """Code -8 times -128 everywhere: the largest accumulator magnitude."""
    for M in (1, 8, 128):
        K, N = 4096, 48
        xq = np.full((M, K), -128, np.int8)
        packed = np.full((N, K // 2), 0x88, np.uint8)
        acc = W4.w4a8_matmul_i32(dev(xq), dev(packed))
        assert np.all(host(acc) == 1024 * K), W4.w4_last_path()


# ----------------------------------------------------------- W4A8 linear
LIN_CASES = [(1, 1152, 200), (4, 256, 70), (8, 1152, 130), (16, 512, 64), (64, 256, 33),
             (100, 384, 260), (300, 256, 516), (32, 10, 32), (9, 40, 7)]


@pytest.mark.parametrize("M,K,N", LIN_CASES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_linear(M, K, N, with_bias):
    d = workloads.random_case(M + K + N, M, K, N, outliers=min(6, K), bias=with_bias)
    pref, sref = oracle.quantize_weight_sym(d["W"])
    b = d.get("bias")
    yref = oracle.w4a8_linear(d["x"], pref, sref, b)
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    bufy, y, py = guarded((M, N), torch.float32)
    W4.w4a8_linear(dev(d["x"]), packed, sw, bias=None if b is None else dev(b), Y=y)
    got = host(y)
    assert bits_equal(got, yref), report(f"y path={W4.w4_last_path()}", got, yref)
    assert np.all(np.abs(got - yref) <= 1e-5 * np.abs(yref))
    assert guards_intact(bufy, py)
    # same product from pre-quantized activations
    xq, sx = oracle.quantize_act(d["x"])
    y2 = W4.w4a8_linear_q(dev(xq), dev(sx), packed, sw, bias=None if b is None else dev(b))
    assert bits_equal(host(y2), yref), W4.w4_last_path()


def test_gemm_epilogue_signed_zero():
    """Scales whose product underflows to zero: y = float(acc) * 0 is -0.0 for a
    negative sum, and with no bias the output keeps that sign, on the GEMM's
    interior and edge tiles alike."""
    M, K, N = 300, 256, 516
    d = workloads.random_case(77, M, K, N)
    X = (d["x"] * np.float32(1e-34)).astype(np.float32)
    W = (d["W"] * np.float32(1e-11)).astype(np.float32)
    pref, sref = oracle.quantize_weight_sym(W)
    yref = oracle.w4a8_linear(X, pref, sref)
    negzero = (yref == 0) & np.signbit(yref)
    assert negzero.any() and (~negzero).any()
    packed, sw, _ = W4.w4_quantize_weight(dev(W), "sym")
    y = W4.w4a8_linear(dev(X), packed, sw)
    assert W4.w4_last_path() == "gemm_mfma"
    assert bits_equal(host(y), yref)


# decode-batch MFMA GEMV launch widths: the channel blocks per workgroup follow
# N (4 for N >= 12288, 3 from 9216, 2 from 6144, else 1 on a 256-CU device);
# ragged N leaves the last workgroup partly outside the layer
MFMA_WIDTHS = [(16, 256, 12304), (40, 128, 9232), (64, 256, 6160), (9, 128, 3000)]


@pytest.mark.parametrize("M,K,N", MFMA_WIDTHS)
def test_gemv_mfma_widths(M, K, N):
    d = workloads.random_case(M * 3 + K + N, M, K, N, outliers=4, bias=True)
    pref, sref = oracle.quantize_weight_sym(d["W"])
    yref = oracle.w4a8_linear(d["x"], pref, sref, d["bias"])
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    bufy, y, py = guarded((M, N), torch.float32)
    W4.w4a8_linear(dev(d["x"]), packed, sw, bias=dev(d["bias"]), Y=y)
    assert W4.w4_last_path() == ("gemv_mfma_fused" if M <= 16 else "gemv_mfma")
    got = host(y)
    assert bits_equal(got, yref), report("y", got, yref)
    assert guards_intact(bufy, py)
    xq, _ = oracle.quantize_act(d["x"])
    acc = W4.w4a8_matmul_i32(dev(xq), packed)
    assert W4.w4_last_path() == "gemv_mfma"
    assert np.array_equal(host(acc), oracle.matmul_i32(xq, pref, K))


# whole-line weight loads of the MFMA GEMV: for int4 codes with K % 256 = 0
# and up to two row blocks (M <= 32) the loop runs over pairs of 128-k steps
# (waves with no pair, a ragged split of the pairs over the 8 waves, a ragged
# last channel block); three row blocks and K % 256 = 128 take per-step loads;
# int8 codes always load whole lines, one step per unit
LINE_CASES = [(17, 256, 100), (24, 768, 130), (32, 3840, 70), (20, 1280, 9300),
              (32, 640, 48), (33, 512, 50), (48, 1024, 40)]


@pytest.mark.parametrize("M,K,N", LINE_CASES)
def test_gemv_mfma_line_loads(M, K, N):
    d = workloads.random_case(M * 7 + K + N, M, K, N, outliers=4, bias=True)
    pref, sref = oracle.quantize_weight_sym(d["W"])
    yref = oracle.w4a8_linear(d["x"], pref, sref, d["bias"])
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    bufy, y, py = guarded((M, N), torch.float32)
    W4.w4a8_linear(dev(d["x"]), packed, sw, bias=dev(d["bias"]), Y=y)
    assert W4.w4_last_path() == "gemv_mfma"
    got = host(y)
    assert bits_equal(got, yref), report("y", got, yref)
    assert guards_intact(bufy, py)
    xq, _ = oracle.quantize_act(d["x"])
    acc = W4.w4a8_matmul_i32(dev(xq), packed)
    assert W4.w4_last_path() == "gemv_mfma"
    assert np.array_equal(host(acc), oracle.matmul_i32(xq, pref, K))
    qref, s8 = oracle.quantize_weight_w8(d["W"])
    Wq, sw8 = W4.w8_quantize_weight(dev(d["W"]))
    y8 = host(W4.w8a8_linear(dev(d["x"]), Wq, sw8, bias=dev(d["bias"])))
    assert W4.w4_last_path() == "w8_gemv_mfma"
    assert bits_equal(y8, oracle.w8a8_linear(d["x"], qref, s8, d["bias"]))
    acc8 = W4.w8a8_matmul_i32(dev(xq), Wq)
    assert W4.w4_last_path() == "w8_gemv_mfma"
    assert np.array_equal(host(acc8), oracle.matmul_w8_i32(xq, qref))


# the MFMA GEMV with the activation quantization in its prologue: M <= 16 and
# K <= 4096 on the canonical int4 layout (8 waves up to 8 rows with half-line
# loads and up to 7 rows with whole-line loads, 16 waves, one row each, above),
# and also ceil(M / 8) * K <= 4096 for shuffled tiles and int8 weights; rows
# past M padded to 16 (LDS rows of up to 2048 k, and of up to 4096 k); at the
# bounds and just outside them (the two-launch path runs there).
# (M, K, N, fused on the canonical layout, fused with shuffled tiles / int8)
FUSED_CASES = [(5, 128, 33, True, True), (8, 1152, 130, True, True),
               (8, 2048, 70, True, True), (16, 1152, 260, True, True),
               (9, 1536, 64, True, True), (16, 1536, 50, True, True),
               (7, 2176, 50, True, True), (9, 2048, 40, True, True),
               (16, 1664, 40, True, True), (8, 4096, 48, True, True),
               (4, 4096, 40, True, True), (9, 2176, 40, True, False),
               (16, 2176, 40, True, False), (12, 4096, 70, True, False),
               (10, 2688, 50, True, False), (16, 3968, 33, True, False),
               (16, 4096, 48, True, False), (5, 4224, 40, False, False)]


@pytest.mark.parametrize("M,K,N,fused,fused8", FUSED_CASES)
def test_gemv_mfma_fused(M, K, N, fused, fused8):
    path = "gemv_mfma_fused" if fused else "gemv_mfma"
    d = workloads.random_case(M * 11 + K + N, M, K, N, outliers=min(6, K), bias=True)
    X = d["x"]
    if M > 6:
        X[2] = 0.0                                   # all-zero row
        X[5] *= np.float32(1e-37)                    # scale below 2^-64 (subnormal)
    pref, sref = oracle.quantize_weight_sym(d["W"])
    yref = oracle.w4a8_linear(X, pref, sref, d["bias"])
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    bufy, y, py = guarded((M, N), torch.float32)
    W4.w4a8_linear(dev(X), packed, sw, bias=dev(d["bias"]), Y=y)
    assert W4.w4_last_path() == path
    got = host(y)
    assert bits_equal(got, yref), report(f"y path={path}", got, yref)
    assert guards_intact(bufy, py)
    yr = host(W4.w4a8_linear_act(dev(X), packed, sw, bias=dev(d["bias"]), activation="relu"))
    assert bits_equal(yr, oracle.relu(yref))
    if K % 128 == 0:
        wpp = W4.w4_prepack_weights(packed)
        y2 = host(W4.w4a8_linear_prepacked(dev(X), wpp, sw, bias=dev(d["bias"])))
        want = "gemv_mfma_fused_prepacked" if fused8 else "gemv_mfma_prepacked"
        assert W4.w4_last_path() == want
        assert bits_equal(y2, yref)
    qref, s8 = oracle.quantize_weight_w8(d["W"])
    Wq, sw8 = W4.w8_quantize_weight(dev(d["W"]))
    y8 = host(W4.w8a8_linear(dev(X), Wq, sw8, bias=dev(d["bias"])))
    assert W4.w4_last_path() == ("w8_gemv_mfma_fused" if fused8 else "w8_gemv_mfma")
    assert bits_equal(y8, oracle.w8a8_linear(X, qref, s8, d["bias"]))


def _sample(n, k, seed):
    if n <= k:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, min(n, k) - 2, replace=False)]))


@pytest.mark.parametrize("name,M", [("gemma", 1), ("gemma", 8), ("mlp7b", 1), ("mlp7b", 16),
                                    ("mlp7b", 64), ("prefill", None)])
def test_linear_full_workloads(name, M):
    """Full-size layers as benchmarked; sampled rows x channels against the oracle."""
    d = workloads.generate(name, M=M)
    W, X = d["W"], d["x"]
    packed, sw, _ = W4.w4_quantize_weight(dev(W), "sym")
    y = W4.w4a8_linear(dev(X), packed, sw)
    path = W4.w4_last_path()
    got = host(y)
    rows = _sample(X.shape[0], 64, 1)
    cols = _sample(W.shape[1], 256, 2)
    pref, sref = oracle.quantize_weight_sym(np.ascontiguousarray(W[:, cols]))
    assert np.array_equal(host(packed)[cols], pref) and bits_equal(host(sw)[cols], sref)
    yref = oracle.w4a8_linear(np.ascontiguousarray(X[rows]), pref, sref)
    sub = got[np.ix_(rows, cols)]
    assert bits_equal(sub, yref), report(f"{name} M={M} path={path}", sub, yref)
    assert np.all(np.isfinite(got))


def test_toy_model_end_to_end():
    """The Keras guide's toy model: Dense 10->32 (ReLU) -> Dense 32->1, W4A8."""
    t = workloads.toy_model()
    p1, s1 = oracle.quantize_weight_sym(t["W1"])
    p2, s2 = oracle.quantize_weight_sym(t["W2"])
    h = np.maximum(oracle.w4a8_linear(t["x"], p1, s1, t["b1"]), 0).astype(np.float32)
    yref = oracle.w4a8_linear(h, p2, s2, t["b2"])
    gp1, gs1, _ = W4.w4_quantize_weight(dev(t["W1"]), "sym")
    gp2, gs2, _ = W4.w4_quantize_weight(dev(t["W2"]), "sym")
    gh = torch.relu(W4.w4a8_linear(dev(t["x"]), gp1, gs1, bias=dev(t["b1"])))
    gy = W4.w4a8_linear(gh.contiguous(), gp2, gs2, bias=dev(t["b2"]))
    assert bits_equal(host(gy), yref)


# ----------------------------------------------------------------- W4A16
def _w4a16_check(got, yref, absy, K):
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    diff = np.abs(got.astype(np.float64) - yref)
    assert np.linalg.norm(diff) <= 1e-5 * np.linalg.norm(yref)
    assert np.all(diff <= gamma * absy + 1e-30)


W4A16_CASES = [(1, 128, 16, 128), (16, 256, 70, 128), (5, 512, 33, 64), (16, 1024, 130, 32),
               (20, 384, 48, 128), (3, 96, 10, 32), (2, 40, 6, 4), (64, 256, 64, 128),
               # LDS-staged kernel (group 128, K % 512 == 0): ragged N and M
               (16, 512, 70, 128), (33, 1024, 130, 128), (1, 2048, 64, 128)]


@pytest.mark.parametrize("M,K,N,g", W4A16_CASES)
def test_w4a16_linear(M, K, N, g):
    rng = np.random.default_rng(M * K + N + g)
    W = (rng.standard_normal((K, N)) * 0.015).astype(np.float32)
    W[:, 0] += 0.05
    xb = workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    pref, sref, zref = oracle.quantize_weight_asym(W, g)
    yref, absy = oracle.w4a16_linear(xb, pref, sref, zref, g)
    packed, s, z = W4.w4_quantize_weight(dev(W), "asym", g)
    bufy, y, py = guarded((M, N), torch.float32)
    W4.w4a16_linear(dev(xb.view(np.int16)), packed, s, z, g, Y=y)
    _w4a16_check(host(y), yref, absy, K)
    assert guards_intact(bufy, py)


@pytest.mark.parametrize("K", [256, 1024])
def test_w4a16_zero_point_outside_fast_range(K):
    """Groups whose zero point leaves [-112, 128] take the direct dequantization."""
    N, M, g = 32, 4, 128
    rng = np.random.default_rng(77)
    W = (rng.standard_normal((K, N)) * 0.01).astype(np.float32)
    W[:, :8] += 3.0       # far-positive groups: zero point about -4000
    W[:, 8:12] -= 3.0     # far-negative groups: zero point about +4000
    xb = workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    pref, sref, zref = oracle.quantize_weight_asym(W, g)
    assert zref.min() < -112 and zref.max() > 128
    yref, absy = oracle.w4a16_linear(xb, pref, sref, zref, g)
    packed, s, z = W4.w4_quantize_weight(dev(W), "asym", g)
    assert np.array_equal(host(packed), pref)
    y = W4.w4a16_linear(dev(xb.view(np.int16)), packed, s, z, g)
    _w4a16_check(host(y), yref, absy, K)


def test_w4a16_full_workload():
    """The 70B-class layer (16 x 8192 x 28672, group 128), sampled channels."""
    d = workloads.w4a16_inputs()
    W, xb, g = d["W"], d["x_bf16"], d["group"]
    packed, s, z = W4.w4_quantize_weight(dev(W), "asym", g)
    y = W4.w4a16_linear(dev(xb.view(np.int16)), packed, s, z, g)
    assert W4.w4_last_path() == "w4a16_lds"
    got = host(y)
    cols = _sample(W.shape[1], 384, 3)
    pref, sref, zref = oracle.quantize_weight_asym(np.ascontiguousarray(W[:, cols]), g)
    assert np.array_equal(host(packed)[cols], pref)
    yref, absy = oracle.w4a16_linear(xb, pref, sref, zref, g)
    _w4a16_check(got[:, cols], yref, absy, W.shape[0])
