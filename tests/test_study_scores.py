"""The accuracy study's scoring against a hand-built case (no GPU)."""
import numpy as np

from dense_grounded_image_amd import study_accuracy as st


def test_planted_scores_closed_form():
    src = np.array([2, 0, -1, 2, 1], np.int32)        # sources of image-2 pixels 0..4
    pairs = [[2, 0], [1, 4], [0, 3]]                   # correct, correct, wrong
    m, c, prec, rec = st.planted_scores(pairs, src)
    assert (m, c) == (3, 2) and prec == 2 / 3 and rec == 2 / 3   # recoverable: {0, 1, 2}
