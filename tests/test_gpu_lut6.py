"""GPU parity for the per-row LUT 6-bit path ("Qwen3.8-27B - BenQ 6-bit"):
pack / unpack / dequant bit-exact, GEMV within the output tolerance."""
import numpy as np
import pytest
import torch

import dequant_matmul_amd as fqm
import oracle
import synth
from gpu_common import (DEV, assert_close, bf16_dev, canaries_intact, guarded, lut6_case,
                        lut6_weights, to_f64)

pytestmark = pytest.mark.gpu

SHAPES = [(256, 512, 1), (1000, 1088, 7), (17408, 5120, 2), (5120, 17408, 3)]


@pytest.mark.parametrize("rows,cols,seed", SHAPES)
def test_pack_is_bit_exact(rows, cols, seed):
    inp, ref = lut6_case(rows, cols, seed)
    codes = torch.from_numpy(inp.codes).to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    p = fqm.pack(codes, err=err)
    nb = cols * 3 // 4
    assert np.array_equal(p[:, :nb].cpu().numpy(), ref)
    assert (p[:, nb:] == 0).all()
    assert int(err.item()) == 0
    back = fqm.unpack(p, cols)
    assert torch.equal(back, codes)


def test_pack_flags_codes_out_of_range():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(33, 192), dtype=np.uint8)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    p = fqm.pack(torch.from_numpy(codes).to(DEV), err=err)
    assert int(err.item()) == 1
    assert np.array_equal(p[:, :144].cpu().numpy(), oracle.lut6.pack_codes(codes & 63))


@pytest.mark.parametrize("bits", [1, 4, 6])
@pytest.mark.parametrize("rows,cols", [(7, 24), (65, 2000), (3, 4096)])
def test_pack_bits_matches_oracle(bits, rows, cols):
    if (cols * bits) % 8:
        pytest.skip("row does not end on a byte")
    rng = np.random.default_rng(rows + cols + bits)
    vals = rng.integers(0, 1 << bits, size=(rows, cols), dtype=np.uint8)
    ld = ((cols * bits + 7) // 8 + 15) // 16 * 16
    p = fqm.pack_bits(torch.from_numpy(vals).to(DEV), bits, ld=ld)
    assert np.array_equal(p.cpu().numpy(), oracle.bits.pack(vals, bits, ld))


@pytest.mark.parametrize("rows,cols,seed", SHAPES[:3])
def test_dequant_is_bit_exact(rows, cols, seed):
    inp, _ = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    W = fqm.dequant(w).view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.numerics.bf16_bits_from_f64_rne(oracle.lut6.decode(inp.codes, inp.lut))
    assert np.array_equal(W, ref)


@pytest.mark.parametrize("batch", list(range(1, 17)))
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemv_ragged(batch, out):
    rows, cols, seed = 1000, 1088, 7
    inp, packed = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    x = synth.activations(batch, cols, seed)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    buf, y = guarded((batch, rows), dt)
    fqm.gemv(w, bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.lut6.gemv(packed, inp.lut, x, cols), out, f"b{batch} {out}")


def test_gemv_tiny_config_fp32():
    inp, packed = lut6_case(256, 512, 1)
    w = lut6_weights(256, 512, 1)
    x = synth.activations(1, 512, 1)
    y = fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32)
    m = assert_close(to_f64(y), oracle.lut6.gemv(packed, inp.lut, x, 512), "f32")
    assert m["rel_l2"] < 1e-5


@pytest.mark.parametrize("rows,cols,seed", SHAPES[2:])
@pytest.mark.parametrize("batch", [1, 8])
def test_gemv_full_size(rows, cols, seed, batch):
    inp, packed = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    x = synth.activations(batch, cols, seed)
    y = fqm.gemv(w, bf16_dev(x))
    assert_close(to_f64(y), oracle.lut6.gemv(packed, inp.lut, x, cols), "bf16", f"{rows}x{cols} b{batch}")


def test_gemv_exact_invariants():
    rows, cols, seed = 1000, 1088, 7
    inp, _ = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    lv = oracle.numerics.bf16_to_f64(inp.lut)
    # one-hot x returns a decoded column exactly
    for k in (0, 517, cols - 1):
        x = np.zeros((1, cols), np.uint16)
        x[0, k] = 0x3F80
        y = fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32)
        assert np.array_equal(to_f64(y)[0], lv[np.arange(rows), inp.codes[:, k]])
    x = synth.activations(3, cols, seed)
    y = to_f64(fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32))
    # mirrored codes negate y exactly (the tables are mirror-symmetric)
    wm = fqm.Lut6Weights.from_codes(63 - inp.codes, inp.lut, device=DEV)
    assert np.array_equal(to_f64(fqm.gemv(wm, bf16_dev(x), out_dtype=torch.float32)), -y)
    # scaling x by 4 scales y by 4 exactly
    x4 = x.astype(np.uint32) + (2 << 7)
    x4 = np.where((x & 0x7FFF) == 0, x, x4).astype(np.uint16)
    assert np.array_equal(to_f64(fqm.gemv(w, bf16_dev(x4), out_dtype=torch.float32)), 4 * y)


def test_gemv_zero_cols_and_padded_rows():
    # cols = 0 writes zeros
    w0 = fqm.Lut6Weights(torch.zeros((5, 16), dtype=torch.uint8, device=DEV),
                         torch.zeros((5, 64), dtype=torch.bfloat16, device=DEV), 5, 0)
    y = torch.full((2, 5), 7.0, device=DEV)
    fqm.gemv(w0, torch.zeros((2, 0), dtype=torch.bfloat16, device=DEV), y=y)
    assert (y == 0).all()
    # and through the GEMM entry point with more rows than the GEMV takes
    Y = torch.full((300, 5), 7.0, dtype=torch.bfloat16, device=DEV)
    fqm.gemm(w0, torch.zeros((300, 0), dtype=torch.bfloat16, device=DEV), Y=Y)
    assert (Y == 0).all()
    # a row stride larger than the packed row
    inp, packed = lut6_case(1000, 1088, 7)
    w = fqm.Lut6Weights.from_codes(inp.codes, inp.lut, device=DEV, ld=1024)
    x = synth.activations(2, 1088, 7)
    y = fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32)
    assert_close(to_f64(y), oracle.lut6.gemv(packed, inp.lut, x, 1088), "f32")


# Batch-1 shapes with cols a multiple of 1024 (the cell-streaming kernel):
# one 1024-weight chunk per row, rows not a multiple of the workgroup size,
# 16 and 17 chunks per row (the 10-wave workgroup variants), and a row count
# that leaves a partial last workgroup.
B1_SHAPES = [(77, 1024, 9), (1000, 3072, 8), (513, 2048, 12), (600, 16384, 10), (5200, 17408, 13),
             (130, 7168, 14), (301, 11264, 15), (97, 31744, 16)]  # 7, 11 and 31 cells: the widest


def test_gemv_b1_past_the_widest_cells():
    """32 cells (32768 columns) and a width that is not a whole number of
    cells take the generic batch-1 kernel."""
    for rows, cols, seed in ((65, 32768, 17), (70, 3136, 18)):
        inp, packed = lut6_case(rows, cols, seed)
        w = lut6_weights(rows, cols, seed)
        x = synth.activations(1, cols, seed)
        y = fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32)
        assert_close(to_f64(y), oracle.lut6.gemv(packed, inp.lut, x, cols), "f32", f"{rows}x{cols}")


@pytest.mark.parametrize("rows,cols,seed", B1_SHAPES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemv_b1_cells(rows, cols, seed, out):
    inp, packed = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    x = synth.activations(1, cols, seed)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    buf, y = guarded((1, rows), dt)
    fqm.gemv(w, bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.lut6.gemv(packed, inp.lut, x, cols), out, f"{rows}x{cols} {out}")


def test_gemv_b1_exact_invariants():
    rows, cols, seed = 1000, 3072, 8
    inp, _ = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    lv = oracle.numerics.bf16_to_f64(inp.lut)
    for k in (0, 1023, 1024, 2047 + 17, cols - 1):
        x = np.zeros((1, cols), np.uint16)
        x[0, k] = 0x3F80
        y = fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32)
        assert np.array_equal(to_f64(y)[0], lv[np.arange(rows), inp.codes[:, k]]), k
    x = synth.activations(1, cols, seed)
    y = to_f64(fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32))
    # Mirrored codes negate every weight.  This path accumulates with
    # v_dot2_f32_bf16, whose rounding is not symmetric under negation, so the
    # negation holds to within accumulated rounding (a few fp32 ulps per
    # step), not bit for bit.
    wm = fqm.Lut6Weights.from_codes(63 - inp.codes, inp.lut, device=DEV)
    ym = to_f64(fqm.gemv(wm, bf16_dev(x), out_dtype=torch.float32))
    assert np.linalg.norm(ym + y) <= 1e-5 * np.linalg.norm(y)
    x4 = x.astype(np.uint32) + (2 << 7)
    x4 = np.where((x & 0x7FFF) == 0, x, x4).astype(np.uint16)
    assert np.array_equal(to_f64(fqm.gemv(w, bf16_dev(x4), out_dtype=torch.float32)), 4 * y)
    # the same call twice gives the same bits (partial rows combine in a fixed order)
    y2 = to_f64(fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32))
    assert np.array_equal(y, y2)
