"""The mask-comparison protocol itself (tests/support.compare_masks), on the CPU.

The pages fix top-k selection but no tie rule (Light Forcing summary, execution flow,
stage 3), so where the oracle's fp64 score gap at a cut is below 1e-4 another choice is
also correct. The protocol accepts such a choice only if it is a valid one. Here an exact
tie is planted at both a frame cut and a block cut, and hand-made "GPU" lists are fed in:
valid alternatives pass (and are counted), lists that swap in an id outside the tie band,
drop an always-kept frame or differ at a clear cut fail.

Input (d = 2, 2 tokens per frame, 1-token blocks, key frames 0..4; sink 0, current 4,
memory set {1, 2, 3}, k_f = k_b = 1; both query tokens [1, 0]):
  frame 0 tokens [2, 0], [0, 0]     block scores 2, 0
  frame 1 tokens [1, 1], [1, -1]    frame score 1, block scores 1, 1  (block tie)
  frame 2 tokens [1, 5], [1, 5]     frame score 1 (ties frame 1), block scores 1, 1
  frame 3 tokens [.5, 0], [.5, 0]   frame score 0.5
  frame 4 tokens [3, 0], [1, 0]     block scores 3, 1
The oracle keeps frame 1 (lower id at the tie) and block 0 of each frame: T_r = {0, 1, 4},
list [0, 2, 8].
"""
import numpy as np
import pytest

import oracle
from support import compare_masks

K_TOKENS = [[2, 0], [0, 0], [1, 1], [1, -1], [1, 5], [1, 5], [0.5, 0], [0.5, 0], [3, 0], [1, 0]]


def _ref(frame2_shift=0.0):
    k = np.array(K_TOKENS, dtype=np.float64)
    k[4:6, 0] -= frame2_shift                      # moves frame 2's score off the tie
    k = k[None, None]
    q = np.array([[1.0, 0.0], [1.0, 0.0]])[None, None]
    ref = oracle.hsa(q, k, k, tpf=2, bs=1, n_kframes=5, mem=[1, 2, 3], forced=[0, 4], k_f=1, k_b=1,
                     scale=1.0, with_attn=False)
    ref["mem"], ref["forced"] = [1, 2, 3], [0, 4]
    return ref


def _gpu(ref, frames0, blocks0):
    f, b = ref["frames"].copy(), ref["blocks"].copy()
    f[0, 0, 0] = frames0
    b[0, 0, 0] = blocks0
    return dict(frames=f, blocks=b)


def test_planted_ties_in_the_oracle():
    ref = _ref()
    assert ref["frames"][0, 0].tolist() == [[0, 1, 4], [0, 1, 4]]
    assert ref["blocks"][0, 0].tolist() == [[0, 2, 8], [0, 2, 8]]
    assert ref["frame_gaps"][0, 0].tolist() == [0.0, 0.0]
    assert ref["block_gaps"][0, 0, 0].tolist() == [2.0, 0.0, 2.0]


def test_identical_lists_pass_uncounted():
    ref = _ref()
    assert compare_masks(dict(frames=ref["frames"], blocks=ref["blocks"]), ref, 1) == \
        dict(rows=2, frame_ties=0, block_ties=0)


@pytest.mark.parametrize("frames0,blocks0,frame_ties,block_ties", [
    ([0, 2, 4], [0, 4, 8], 1, 0),     # the tied frame 2 instead of 1, its own top block
    ([0, 2, 4], [0, 5, 8], 1, 1),     # ... and the other tied block of frame 2
    ([0, 1, 4], [0, 3, 8], 0, 1),     # frame 1's other tied block
])
def test_valid_alternatives_pass_and_are_counted(frames0, blocks0, frame_ties, block_ties):
    ref = _ref()
    st = compare_masks(_gpu(ref, frames0, blocks0), ref, 1)
    assert (st["frame_ties"], st["block_ties"]) == (frame_ties, block_ties)


def test_alternative_inside_the_band_passes():
    # frame 2 scores 5e-5 below the cut: still inside the 1e-4 band
    ref = _ref(frame2_shift=5e-5)
    assert ref["frames"][0, 0, 0].tolist() == [0, 1, 4] and ref["frame_gaps"][0, 0, 0] == pytest.approx(5e-5)
    assert compare_masks(_gpu(ref, [0, 2, 4], [0, 4, 8]), ref, 1)["frame_ties"] == 1


@pytest.mark.parametrize("frames0,blocks0,shift", [
    ([0, 3, 4], [0, 6, 8], 0.0),      # frame 3 scores 0.5 below the tied cut
    ([0, 1, 4], [1, 2, 8], 0.0),      # frame 0's cut has a gap of 2
    ([1, 2, 4], [2, 4, 8], 0.0),      # the sink frame 0 dropped
    ([0, 2, 4], [0, 4, 8], 2e-4),     # frame 2 now 2e-4 below the cut: not a near-tie
    ([0, 1, 4], [0, 2, 9], 0.0),      # frame 4's cut has a gap of 2
])
def test_invalid_alternatives_fail(frames0, blocks0, shift):
    ref = _ref(frame2_shift=shift)
    with pytest.raises(AssertionError):
        compare_masks(_gpu(ref, frames0, blocks0), ref, 1)
