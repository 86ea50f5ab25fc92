"""Host-side logic of bench.py, without a GPU: the algorithmic byte counts
that the reported rates divide by, the one-GPU guard, the rule that attaches
counter traffic only to the kernel source it was measured on, and the small
helpers of the CPU baseline."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (standard library only at import time)


def test_w4a8_bytes_of_the_workloads():
    # Gemma3-1B-like up-projection at M = 1: packed int4 weights 1152/2 x 6912,
    # fp32 scales, the fp32 activation row and the fp32 output row
    assert bench.w4a8_bytes(1, 1152, 6912) == 3_981_312 + 27_648 + 4_608 + 27_648 == 4_041_216
    # 7B-class MLP layer at M = 1
    assert bench.w4a8_bytes(1, 4096, 11008) == 22_544_384 + 44_032 + 16_384 + 44_032
    # odd K: the last byte of a row carries one code
    assert bench.w4a8_bytes(1, 3, 1) == 2 + 4 + 12 + 4


def test_w8a8_and_w4a16_bytes():
    assert bench.w8a8_bytes(1, 4096, 11008) == 45_088_768 + 44_032 + 16_384 + 44_032
    # 70B-class W4A16 layer: packed codes, fp32 scale and zero point per group
    # of 128, bf16 activations, fp32 output
    assert bench.w4a16_bytes(16, 8192, 28672, 128) == (
        117_440_512 + 2 * 7_340_032 + 262_144 + 1_835_008) == 134_217_728


def test_plain_read_probes_read_the_layers_bytes():
    # the --only read* probes stand for kernels that read a layer's bytes once
    src = open(os.path.join(ROOT, "bench.py")).read()
    sizes = {"read4m": bench.w4a8_bytes(1, 1152, 6912),
             "read22m": bench.w4a8_bytes(1, 4096, 11008),
             "read134m": bench.w4a16_bytes(16, 8192, 28672, 128)}
    for name, n in sizes.items():
        assert f'"{name}": {n}' in src, name


def test_plain_write_probe_writes_the_prefill_output():
    # the --only write67m probe stands for the prefill product's fp32 output
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert f'"write67m": {4 * 4096 * 4096}' in src


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def _traffic_file(tmp_path, digest, bytes_per_launch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "gemv_dot4_gemma_m1_traffic.json").write_text(json.dumps(
        {"src_digest": digest, "traffic_bytes_per_launch": bytes_per_launch}))


def test_traffic_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("abc") is None  # no counter summary
    _traffic_file(tmp_path, "abc", 4_155_222)
    assert bench.load_traffic("abc") == 4_155_222
    assert bench.load_traffic("abd") is None  # the kernel changed since


def test_src_digest_covers_the_headline_kernel_sources(tmp_path, monkeypatch):
    d0 = bench.src_digest()
    assert len(d0) == 16
    csrc = tmp_path / "int4_weight_quantized_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("gemv.hip", "common.h", "kernels.h"):
        (csrc / f).write_bytes(open(os.path.join(ROOT, "int4_weight_quantized_amd", "csrc", f),
                                    "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.src_digest() == d0
    for f in ("gemv.hip", "common.h", "kernels.h"):
        p = csrc / f
        orig = p.read_bytes()
        p.write_bytes(orig + b"\n")
        assert bench.src_digest() != d0, f
        p.write_bytes(orig)


@pytest.mark.parametrize("n,parts", [(10, 3), (6912, 16), (2, 4), (1, 1), (28672, 7)])
def test_slices_partition_the_range(n, parts):
    s = bench._slices(n, parts)
    assert s[0][0] == 0 and s[-1][1] == n
    assert all(a < b for a, b in s)
    assert all(s[i][1] == s[i + 1][0] for i in range(len(s) - 1))
    assert len(s) == min(n, parts)
    sizes = [b - a for a, b in s]
    assert max(sizes) - min(sizes) <= 1


def test_host_cores_is_bounded():
    assert 1 <= bench._host_cores() <= 16


def test_demangle():
    assert bench.demangle("k_plain") == "k_plain"
    name = "_ZN2w411k_gemv_dot4ILi1ELi16ELi3ELb1ELNS_3OutE0ELb0ELb0ELb0EEEvNS_8W4A8ArgsE"
    out = bench.demangle(name)
    assert out == name or out.startswith("void w4::k_gemv_dot4<1, 16, 3, true")


@pytest.mark.parametrize("est_s, true_s", [(3.7e-6, 2.8e-6), (2.8e-6, 2.8e-6), (1e-5, 2e-7),
                                           (1e-7, 5e-6)])
def test_timed_region_spans_two_ms(monkeypatch, est_s, true_s):
    # the graph is sized from an estimate; when replays run faster than it,
    # the region is captured again, sized by the measured rate
    sizes = []

    def replay(torch, hip, step, L):
        sizes.append(L)
        return true_s

    monkeypatch.setattr(bench, "region_replay", replay)
    sec, L = bench.region_time(None, None, None, est_s, 20)
    assert sec == true_s and L == sizes[-1] and L >= 20
    assert L * sec >= 2e-3
    assert len(sizes) == (1 if sizes[0] * true_s >= 2e-3 else 2)
