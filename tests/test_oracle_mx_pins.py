"""Pins for the oracle's MXFP4 decode and the FP8 re-encoding of MXFP4 gate/up matrices (page "Kimi
K3's TPU megakernel: 92 layers in one Pallas call, and what 709 tokens a second measures", section "How
it maps onto a TPU v7": experts ship in MXFP4; the loader re-encodes gate/up into FP8 E4M3 with a bf16
scale per 256, checks bit for bit that it decodes to the same values, and raises if not; down stays
MXFP4). The formats are the OCP Microscaling ones: E2M1 elements, an E8M0 scale per 32. CPU only."""
import math

import numpy as np
import pytest
import torch

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP MX v1.0, FP4 E2M1 magnitudes


def test_e8m0_all_codes_match_torch(oracle):
    L = oracle.lib()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().numpy()
    ours = np.array([L.orc_e8m0_value(c) for c in range(256)], dtype=np.float32)
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127


def _mx(codes, scales):
    from persistent_megakernel_mk_amd.synth import MXFP4Tensor

    return MXFP4Tensor(np.ascontiguousarray(codes, np.uint8), np.ascontiguousarray(scales, np.uint8))


def test_mxfp4_row_nibble_order_and_block_scales(oracle):
    K = 64
    rng = np.random.default_rng(40)
    nib = rng.integers(0, 16, K)
    codes = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None]
    scales = np.array([[127 + 3, 127 - 5]], np.uint8)  # 2^3 for elements 0..31, 2^-5 for 32..63
    out = np.empty(K, np.float32)
    oracle.lib().orc_mxfp4_dequant_row(codes.ctypes.data, scales.ctypes.data, K, out.ctypes.data)
    ref = np.array([(-1 if n & 8 else 1) * E2M1[n & 7] * (2.0 ** 3 if j < 32 else 2.0 ** -5) for j, n in enumerate(nib)])
    assert np.array_equal(out, ref.astype(np.float32))


def test_mxfp4_and_fp8_products_match_float64(oracle, synth):
    rng = np.random.default_rng(41)
    W = synth.mxfp4_encode((rng.standard_normal((48, 512)) * 0.02).astype(np.float32))
    X = rng.standard_normal((3, 512)).astype(np.float32)
    deq = np.empty((48, 512), np.float32)
    for n in range(48):
        oracle.lib().orc_mxfp4_dequant_row(W.codes[n].ctypes.data, W.scales[n].ctypes.data, 512, deq[n].ctypes.data)
    ref = X.astype(np.float64) @ deq.astype(np.float64).T
    bound = 512 * 2.0 ** -24 * (np.abs(X).astype(np.float64) @ np.abs(deq).astype(np.float64).T)
    assert np.all(np.abs(oracle.gemv(W, X) - ref) <= bound)
    assert np.all(np.abs(oracle.gemv(oracle.fp8_reencode(W), X) - ref) <= bound)


def test_fp8_reencode_is_lossless_on_seeded_experts(oracle, synth):
    rng = np.random.default_rng(42)
    W = synth.mxfp4_encode((rng.standard_normal((64, 1024)) * 0.02).astype(np.float32))
    R = oracle.fp8_reencode(W)
    assert R.fp8.shape == (64, 1024) and R.bscale.shape == (64, 4)
    # every bf16 scale is a power of two (no mantissa bits)
    assert np.all((R.bscale & 0x7F) == 0)
    # the FP8 codes read by torch's float8_e4m3fn, times the scales, give the MXFP4 values bit for bit
    f8 = torch.from_numpy(R.fp8).view(torch.float8_e4m3fn).float().numpy()
    s = torch.from_numpy(R.bscale.view(np.int16)).view(torch.bfloat16).float().numpy()
    back = (f8 * np.repeat(s, 256, axis=1)).astype(np.float32)
    deq = np.empty((64, 1024), np.float32)
    for n in range(64):
        oracle.lib().orc_mxfp4_dequant_row(W.codes[n].ctypes.data, W.scales[n].ctypes.data, 1024, deq[n].ctypes.data)
    assert np.array_equal(back.view(np.uint32), deq.view(np.uint32))


def _one_block(exps, nibs):
    """One row of 256 elements: eight 32-blocks with the given E8M0 exponents; element j takes code nibs[j]."""
    nib = np.asarray(nibs, np.int64)
    codes = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None]
    return _mx(codes, np.asarray(exps, np.uint8)[None])


def test_fp8_reencode_closed_form(oracle):
    # all blocks at exponent 127 (scale 1): the block scale is 2^(127 - 133) = 2^-6, so the E2M1 value 6
    # becomes 6 * 2^6 = 384 = 1.5 * 2^8 (E4M3 exponent field 15, mantissa 4: code 0x7C), 0.5 becomes
    # 32 = 2^5 (exponent field 12: code 0x60), and -1 becomes -64 (0x80 | 13 << 3 = 0xE8)
    nibs = [0] * 256
    nibs[0], nibs[1], nibs[2] = 7, 1, 8 | 2
    R = oracle.fp8_reencode(_one_block([127] * 8, nibs))
    assert R.bscale[0, 0] == 0x3C80  # bf16 bits of 2^-6
    assert R.fp8[0, 0] == 0x7C and R.fp8[0, 1] == 0x60 and R.fp8[0, 2] == 0xE8
    assert np.all(R.fp8[0, 3:] == 0)


def test_fp8_reencode_raises_beyond_fourteen_exponents(oracle):
    # a nonzero 0.5 in a 32-block 14 exponents below the block maximum lands on 2^-9, the smallest E4M3
    # subnormal: still exact; 15 below it would need 2^-10: the re-encoding is not lossless and raises
    nibs = [0] * 256
    nibs[0], nibs[255] = 7, 1  # 6 in the first 32-block, 0.5 in the last
    R = oracle.fp8_reencode(_one_block([127] + [120] * 6 + [127 - 14], nibs))
    assert R.fp8[0, 255] == 0x01
    with pytest.raises(ValueError):
        oracle.fp8_reencode(_one_block([127] + [120] * 6 + [127 - 15], nibs))
    # an all-zero 32-block does not take part in the block maximum
    nibs2 = [0] * 256
    nibs2[40] = 1
    R2 = oracle.fp8_reencode(_one_block([200, 100] + [100] * 6, nibs2))
    assert R2.bscale[0, 0] == np.frombuffer(np.float32(2.0 ** (100 - 133)).tobytes(), np.uint16)[1]
