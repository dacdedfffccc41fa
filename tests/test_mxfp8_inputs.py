"""The MXFP8 input encoding of synth.to_mxfp8 (input preparation for the
MXFP8 entry point), against hand-worked values of the OCP microscaling rule:
shared exponent E = floor(log2 amax) - 8 per block of 32, e4m3 elements
x / 2^E saturated to +-448, round to nearest even."""
import torch

import synth


def test_hand_worked_blocks():
    x = torch.zeros(3, 32)
    x[0, 0] = 1.0               # amax 1: E = -8, 1 * 2^8 = 256 = 1.0 * 2^8 -> 0x78
    x[1, 0], x[1, 1:] = 1792.0, 0.5  # amax 1792: E = 2; 448 -> 0x7E; 0.125 -> 0x20
    x[2, 0], x[2, 1] = -3.3, 0.001   # amax 3.3: E = -7; -422.4 -> -416 (0xFD); 0.128 -> 0.125 (0x20)
    b, sc, dec = synth.to_mxfp8(x)
    assert sc.flatten().tolist() == [119, 129, 120]
    assert b[0, :2].tolist() == [0x78, 0x00]
    assert b[1, :2].tolist() == [0x7E, 0x20]
    assert b[2, :2].tolist() == [0xFD, 0x20]
    assert dec[0, 0].item() == 1.0 and dec[1, 0].item() == 1792.0 and dec[1, 1].item() == 0.5
    assert dec[2, 0].item() == -3.25 and dec[2, 1].item() == 0.125 / 128


def test_saturation_and_zero_block():
    x = torch.zeros(2, 32)
    x[0, 0] = 511.0              # E = 0: 511 saturates to 448
    b, sc, dec = synth.to_mxfp8(x)
    assert sc[0, 0].item() == 127 and dec[0, 0].item() == 448.0
    assert sc[1, 0].item() == 0 and not dec[1].any() and not b[1].any()   # all-zero block: E = -127, zeros


def test_decoded_values_are_the_bytes():
    # decoded = e4m3(byte) * 2^(s - 127), element by element
    y = torch.randn(5, 7, 128)
    b, sc, dec = synth.to_mxfp8(y)
    f = b.view(torch.float8_e4m3fn).float()
    scale = torch.exp2(sc.float() - 127).repeat_interleave(32, dim=-1)
    assert torch.equal(f * scale, dec)
