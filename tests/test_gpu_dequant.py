"""Nibble unpack and dequantisation, bit-exact: the library's device dequant (the same
function the GEMM kernels use, exported for tests) against the oracle's exact s*q + b and its
bf16 rounding."""
import numpy as np
import pytest

import synth
from gpu_common import DEV, device_layer, host_layer, log
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu


def gpu_dequant(w4_dev, n_rows, kin, mat, row):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    f = torch.full((kin,), float("nan"), dtype=torch.float32, device=DEV)
    b = torch.zeros((kin,), dtype=torch.int16, device=DEV)
    M.moe_debug_dequant_w4(w4_dev, n_rows, kin, mat, row, f, b)
    torch.cuda.synchronize()
    return f.cpu().numpy().astype(np.float64), b.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name,proj", [("tiny", "gate"), ("tiny", "down"), ("odd", "up"),
                                       ("full", "gate"), ("full", "down"), ("full", "sh_up"),
                                       ("full", "sh_down")])
def test_dequant_bit_exact(name, proj):
    host = host_layer(name)
    dev = device_layer(name).tensors[proj]
    q, s, b = host[proj]
    n_mat, N, kw = q.shape
    kin = kw * 8
    rng = np.random.default_rng(len(name) + len(proj))
    picks = {(0, 0), (n_mat - 1, N - 1)} | {(int(rng.integers(n_mat)), int(rng.integers(N)))
                                             for _ in range(6)}
    for mat, row in sorted(picks):
        f, bits = gpu_dequant(dev, N, kin, mat, row)
        ref = O.dequant(q[mat, row:row + 1], s[mat, row:row + 1], b[mat, row:row + 1])[0]
        assert np.array_equal(f, ref), (mat, row)                       # fp32 value == exact
        assert np.array_equal(O.bf16_to_f64(bits), O.round_to_bf16(ref)), (mat, row)
    log(f"[dequant] {name}.{proj}: {len(picks)} rows bit-exact")


def test_dequant_golden_words():
    """Words from the nibble-order fixture with scale 1 and bias 0 give the nibbles themselves;
    scale 1/2 and bias -4 give q/2 - 4."""
    import torch
    words = np.array([0x76543210, 0xfedcba98, 0x0000000f, 0xf0000000, 0x12345678, 0x88888888,
                      0xa5a5a5a5, 0x00000000], dtype=np.uint32)
    q = np.tile(words, 16).reshape(2, 64)                  # 2 rows x 512 inputs
    s = synth.f32_to_bf16_bits(np.array([[1.0] * 8, [0.5] * 8], np.float32))
    b = synth.f32_to_bf16_bits(np.array([[0.0] * 8, [-4.0] * 8], np.float32))
    w4 = tuple(torch.from_numpy(a.view(v)).to(DEV) for a, v in ((q, np.int32), (s, np.int16),
                                                                 (b, np.int16)))
    nibbles = O.unpack_nibbles(q)
    for row in range(2):
        f, bits = gpu_dequant(w4, 2, 512, 0, row)
        want = nibbles[row].astype(np.float64) * (1.0 if row == 0 else 0.5) - (0 if row == 0 else 4)
        assert np.array_equal(f, want)
        assert np.array_equal(O.bf16_to_f64(bits), want)
