"""Host-side model of the direct-to-LDS loads of the two LDS-staged kernels.

The prefill GEMM (`k_gemm_mfma`) and the group-128 weight-only kernel
(`k_w4a16_lds`) fill LDS with raw buffer loads whose range check covers the
per-lane offset (voffset) only: the scalar offset (soffset) is added to the
address unchecked.  A lane is safe when either its voffset lies outside the
descriptor's range (the load returns zeros and touches no memory) or the whole
16-byte access, voffset + soffset included, lies inside the allocation.

This file restates each load's offsets as the kernels compute them and checks
that rule for every workgroup, wave, lane, load and k-tile of ragged shapes.
It runs on the CPU only; the GPU parity tests run the same shapes through the
kernels themselves.
"""
import numpy as np
import pytest

LANES = np.arange(64)


def _check(name, alloc, desc_base, desc_range, voff, soff):
    """voff, soff: broadcastable integer arrays of one load's lanes."""
    voff, soff = np.broadcast_arrays(np.asarray(voff, np.int64), np.asarray(soff, np.int64))
    inside = voff < desc_range
    # a load that starts inside the range stays inside it (no partial lanes)
    assert np.all(~inside | (voff + 16 <= desc_range)), f"{name}: partial range"
    end = desc_base + voff + soff + 16
    bad = inside & ((end > alloc) | (desc_base + voff + soff < 0))
    assert not np.any(bad), f"{name}: {int(bad.sum())} lanes leave the allocation of {alloc} B"


def gemm_loads(M, K, N, w8=False, pp=False, row_term_in_soffset=False):
    """Every direct load of k_gemm_mfma at M x K x N (256 x 256 x 128 tiles, 8 waves).

    `row_term_in_soffset` rebuilds the former offsets (row / channel term in the
    scalar offset) so that the model shows it would catch them.
    """
    KB = K if w8 else K // 2
    ST = K // 128
    KT = K // 128
    tiles_m, tiles_n = -(-M // 256), -(-N // 256)
    kt = np.arange(KT)[:, None]
    a_alloc = M * K
    b_alloc = (-(-N // 16)) * ST * 1024 if pp else N * KB
    for tm in range(tiles_m):
        m0 = tm * 256
        a_base, a_range = m0 * K, min(256, M - m0) * K
        for wave in range(8):
            for i in range(4):
                v = (LANES % 16) ^ (LANES // 16 + 4 * (i % 2))
                if row_term_in_soffset:
                    voff = (32 * wave + 2 * (LANES // 16) + (v >> 3)) * K + (v & 7) * 16
                    soff = 8 * i * K + kt * 128
                else:
                    voff = (32 * wave + 8 * i + 2 * (LANES // 16) + (v >> 3)) * K + (v & 7) * 16
                    soff = kt * 128
                _check(f"A tile {tm} wave {wave} load {i}", a_alloc, a_base, a_range, voff, soff)
    for tn in range(tiles_n):
        n0 = tn * 256
        if pp:
            b_base = (n0 // 16) * ST * 1024
            b_range = (-(-min(256, N - n0) // 16)) * ST * 1024
        else:
            b_base, b_range = n0 * KB, min(256, N - n0) * KB
        for wave in range(8):
            if w8:
                for i in range(4):
                    v = (LANES % 16) ^ (LANES // 16 + 4 * (i % 2))
                    row = 32 * wave + 2 * (LANES // 16) + (v >> 3)
                    if row_term_in_soffset:
                        voff, soff = row * K + (v & 7) * 16, 8 * i * K + kt * 128
                    else:
                        voff, soff = (row + 8 * i) * K + (v & 7) * 16, kt * 128
                    _check(f"B8 tile {tn} wave {wave} load {i}", b_alloc, b_base, b_range,
                           voff, soff)
            elif pp:
                for i in range(2):
                    voff = (2 * wave + i) * ST * 1024 + LANES * 16
                    _check(f"Bpp tile {tn} wave {wave} load {i}", b_alloc, b_base, b_range,
                           voff, kt * 1024)
            else:
                chunk = ((LANES % 4) ^ ((LANES // 8) % 4)) * 16
                for i in range(2):
                    ch = 32 * wave + LANES // 4
                    if row_term_in_soffset:
                        voff, soff = ch * KB + chunk, 16 * i * KB + kt * 64
                    else:
                        voff, soff = (ch + 16 * i) * KB + chunk, kt * 64
                    _check(f"B tile {tn} wave {wave} load {i}", b_alloc, b_base, b_range,
                           voff, soff)


def w4a16_lds_loads(M, K, N, WPH, pp=False):
    """Every direct load of k_w4a16_lds<WPH, PP> (group 128, K % 512 == 0)."""
    assert K % 512 == 0
    KB, G = K // 2, K // 128
    LSTEPS, CH = 2, 16 * WPH
    kW, kX = CH * 64 * LSTEPS, 4096 * LSTEPS
    kSZ = ((WPH + 3) // 4) * 1024 if pp else ((CH * 16 + 1023) // 1024) * 1024
    tabs = 1 if pp else 2
    loads_w, loads_x, loads_sz = kW // 1024, kX // 1024, kSZ // 1024
    loads = loads_w + loads_x + tabs * loads_sz
    per_wave = -(-loads // WPH)
    T = G // (2 * LSTEPS)
    nb16 = -(-N // 16)
    x_alloc = M * K * 2
    w_alloc = nb16 * G * 1024 if pp else N * KB
    t_alloc = nb16 * (G // 2) * 256 if pp else N * G * 4
    sw4 = (LANES % 4) ^ ((LANES // 8) % 4)
    for by in range(-(-M // 16)):
        m0 = by * 16
        rowsm = min(16, M - m0)
        x_base, x_range = m0 * K * 2, rowsm * K * 2
        for bx in range(-(-N // CH)):
            n0 = bx * CH
            cols = min(CH, N - n0)
            blk0 = bx * WPH
            nblk = min(WPH, nb16 - blk0)
            if pp:
                w_base, w_range = blk0 * G * 1024, nblk * G * 1024
                t_base, t_range = blk0 * (G // 2) * 256, nblk * (G // 2) * 256
            else:
                w_base, w_range = n0 * KB, cols * KB
                t_base, t_range = n0 * G * 4, cols * G * 4
            for half in range(2):
                s0 = half * T * LSTEPS
                step = (s0 + LSTEPS * np.arange(T))[:, None]
                for wl in range(WPH):
                    for i in range(per_wave):
                        q = min(wl + WPH * i, loads - 1)
                        if q < loads_w:
                            j = q // WPH
                            if pp:
                                voff = (q % WPH) * G * 1024 + LANES * 16
                                soff = (step + j) * 1024
                            else:  # whole 128-byte lines of channels 8q .. 8q + 7
                                c = 8 * q + LANES // 8
                                voff = c * KB + 16 * ((LANES % 8) ^ ((c // 2) % 8))
                                soff = step * 64
                            _check("W", w_alloc, w_base, w_range, voff, soff)
                        elif q < loads_w + loads_x:
                            qq = q - loads_w
                            j, pk, r = qq // 4, qq % 4, LANES // 4
                            voff = r * K * 2 + 64 * pk + 16 * (sw4 ^ pk)
                            _check("X", x_alloc, x_base, x_range, voff, (step + j) * 256)
                        elif pp:
                            qq = q - loads_w - loads_x
                            bq = 4 * qq + LANES // 16
                            voff = bq * (G // 2) * 256 + (LANES % 16) * 16
                            _check("SZ", t_alloc, t_base, t_range, voff, (step // 2) * 256)
                        else:
                            # the first stage of each pair of stages loads the
                            # quads; the second one's loads are out of range
                            qq = q - loads_w - loads_x
                            part = qq % loads_sz
                            first = (step % 4 == 0) | (np.arange(T)[:, None] == 0)
                            voff = np.where(first, (64 * part + LANES) * G * 4, 0x7FFF0000)
                            soff = np.where(first, (step // 4) * 16, 0)
                            _check("S/Z", t_alloc, t_base, t_range, voff, soff)


GEMM_SHAPES = [(300, 512, 1000), (130, 256, 129), (65, 128, 17), (257, 384, 300), (512, 256, 512),
               (4096 + 7, 128, 256 + 3)]


@pytest.mark.parametrize("shape", GEMM_SHAPES)
@pytest.mark.parametrize("kind", ["int4", "w8", "pp"])
def test_gemm_loads_in_bounds(shape, kind):
    M, K, N = shape
    gemm_loads(M, K, N, w8=(kind == "w8"), pp=(kind == "pp"))


@pytest.mark.parametrize("kind", ["int4", "w8"])
def test_model_catches_row_term_in_scalar_offset(kind):
    # the former offsets read up to 24*K bytes past the activation codes of a
    # ragged last row tile (and 16 channel rows past the packed weights)
    with pytest.raises(AssertionError, match="leave the allocation"):
        gemm_loads(300, 512, 1000, w8=(kind == "w8"), row_term_in_soffset=True)


W4A16_SHAPES = [(16, 512, 64), (5, 1024, 100), (17, 512, 4100), (33, 2048, 1000)]


@pytest.mark.parametrize("shape", W4A16_SHAPES)
@pytest.mark.parametrize("wph", [1, 2, 4, 7])
@pytest.mark.parametrize("pp", [False, True])
def test_w4a16_lds_loads_in_bounds(shape, wph, pp):
    M, K, N = shape
    w4a16_lds_loads(M, K, N, wph, pp=pp)
