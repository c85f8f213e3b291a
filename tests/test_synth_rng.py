"""Known-answer pins of the input generator's counter-based RNG.

Threefry-2x32 with 20 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11): the three known-answer vectors its
authors publish with the Random123 library (counter, key → output) for this
variant. The generator draws the inputs of both sides of every parity test,
so a wrong rotation, key-schedule word or round count would still give
matching (but different from the published) streams; these vectors pin it.
"""
import torch

import synth

KAT_2x32_20 = [
    # (counter c0, c1), (key k0, k1), (output x0, x1)
    ((0x00000000, 0x00000000), (0x00000000, 0x00000000), (0x6b200159, 0x99ba4efe)),
    ((0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff), (0x1cb996fc, 0xbb002be7)),
    ((0x243f6a88, 0x85a308d3), (0x13198a2e, 0x03707344), (0xc4923a9c, 0x483df7a0)),
]


def test_threefry2x32_20_known_answers():
    for (c0, c1), (k0, k1), (x0, x1) in KAT_2x32_20:
        y0, y1 = synth.threefry2x32(k0, k1, torch.tensor([c0], dtype=torch.int64),
                                    torch.tensor([c1], dtype=torch.int64))
        assert (int(y0), int(y1)) == (x0, x1)


def test_threefry_counter_chunking():
    """Element i of a long counter range equals the same counter drawn alone."""
    idx = torch.arange(1000, dtype=torch.int64) * 7919 + (3 << 32)
    full = synth.normal(0, synth.STREAM_K, idx)
    for i in (0, 1, 499, 999):
        assert float(synth.normal(0, synth.STREAM_K, idx[i:i + 1])[0]) == float(full[i])


def test_head_selection_is_a_slice():
    """Drawing only some KV heads gives exactly those heads' slices."""
    k = synth.make_k(2, 8, 5, 40, 128, b0=3)
    v = synth.make_v(2, 8, 5, 40, 128, b0=3)
    assert torch.equal(synth.make_k(1, 8, 5, 40, 128, b0=4, heads=[6, 2])[0], k[1, [6, 2]])
    assert torch.equal(synth.make_v(1, 8, 5, 40, 128, b0=4, heads=[7])[0], v[1, [7]])
