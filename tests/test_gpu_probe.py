"""The measurement helpers and the kernel-name diagnostic, on the GPU."""
import pytest
import torch

import int4_weight_quantized_amd as W4
import workloads

pytestmark = pytest.mark.gpu


def test_last_kernel_names_the_kernel_that_ran():
    d = workloads.random_case(3, 1, 1152, 64)
    dev = torch.device("cuda:0")
    p, s, _ = W4.w4_quantize_weight(torch.from_numpy(d["W"]).to(dev), "sym")
    W4.w4a8_linear(torch.from_numpy(d["x"]).to(dev), p, s)
    assert W4.w4_last_path() == "gemv_dot4"
    assert "k_gemv_dot4" in W4.w4_last_kernel()
    x16 = torch.from_numpy(workloads.random_case(4, 300, 1024, 256)["x"]).to(dev)
    p2, s2, _ = W4.w4_quantize_weight(torch.randn(1024, 256, device=dev) * 0.02, "sym")
    W4.w4a8_linear(x16, p2, s2)
    assert "k_gemm_mfma" in W4.w4_last_kernel()
    torch.cuda.synchronize()


def test_probes_run():
    src = torch.ones(4041216, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    W4.w4_probe_read(src, sink)
    assert W4.w4_last_path() == "probe_read" and "k_probe_read" in W4.w4_last_kernel()
    W4.w4_probe_empty(432)
    assert W4.w4_last_path() == "probe_empty"
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0  # XOR of all-ones data is 0: no store
    with pytest.raises(W4.W4Error):
        W4.w4_probe_read(src[:15], sink)


def test_write_probe_writes_exactly_its_bytes():
    # 3 blocks of 16 KB plus 48 bytes: the last block's stores past the range
    # are dropped by the descriptor, so the guard words after it stay zero
    n = 3 * 16384 + 48
    buf = torch.zeros(n + 4096, dtype=torch.uint8, device="cuda:0")
    W4.w4_probe_write(buf[:n], 0x01020304)
    torch.cuda.synchronize()
    words = buf.view(torch.int32).cpu()
    assert (words[: n // 4] == 0x01020304).all()
    assert (words[n // 4:] == 0).all()
    assert W4.w4_last_path() == "probe_write" and "k_probe_write" in W4.w4_last_kernel()
    with pytest.raises(W4.W4Error):
        W4.w4_probe_write(buf[:24])


def test_mfma_probe_reports_a_clock():
    times = torch.zeros((8, 4), dtype=torch.int64, device="cuda:0")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    ops = torch.randint(-2 ** 31, 2 ** 31 - 1, (8 * 512 * 32,), dtype=torch.int32,
                        device="cuda:0")
    for o in (None, ops):
        times.zero_()
        W4.w4_probe_mfma(8, 200, times, sink, o)
        torch.cuda.synchronize()
        t = times.cpu().numpy().astype("float64")
        assert (t[:, 1] > t[:, 0]).all() and (t[:, 3] > t[:, 2]).all()
        ghz = (t[:, 1] - t[:, 0]) / ((t[:, 3] - t[:, 2]) / 1e8) / 1e9
        assert ((ghz > 0.3) & (ghz < 5.0)).all(), ghz
    with pytest.raises(W4.W4Error):
        W4.w4_probe_mfma(8, 202, times, sink)  # iterations come in fours
    with pytest.raises(ValueError):
        W4.w4_probe_mfma(8, 200, times, sink, ops[:100])
