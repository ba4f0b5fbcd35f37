"""Pins of the oracle's integer host logic against facts printed on the pages.

Page citations live in tests/golden/page_facts.json next to each case.
"""
import itertools

import numpy as np
import pytest

from oracle import host


def test_frame_alignment_page_cases(page_facts):
    for req, want in page_facts["frame_alignment"]["cases"]:
        assert host.align_frames(req) == want


def test_aligned_shapes_are_fixed_points_with_page_durations(page_facts):
    for frames, secs in page_facts["aligned_shapes_seconds"]["cases"]:
        assert host.align_frames(frames) == frames
        assert round(frames / host.FPS, 3) == pytest.approx(secs, abs=1e-9)
        assert (frames - 5) % 17 == 0


def test_alignment_brute_force():
    # brute force: enumerate 5+17n and take the first one >= request
    shapes = [5 + 17 * n for n in range(60)]
    for req in range(1, 900):
        assert host.align_frames(req) == next(s for s in shapes if s >= req)


def test_seconds_to_frames(page_facts):
    for secs, frames in page_facts["seconds_to_frames"]["cases"]:
        assert host.frames_for_seconds(secs) == frames
    with pytest.raises(ValueError):
        host.frames_for_seconds(0.0)


def test_token_grid_page_cases(page_facts):
    for w, h, gh, gw in page_facts["token_grid"]["cases"]:
        got = host.token_grid(w, h)
        assert got[:2] == (gh, gw)
    for w, h in page_facts["token_grid"]["invalid"]:
        with pytest.raises(ValueError):
            host.token_grid(w, h)


def test_rope_halving(page_facts):
    for w, h, ref, scale in page_facts["rope_halving"]["cases"]:
        assert host.token_grid(w, h, ref)[2] == scale
    # only the 8x8 grid halves
    for w, h in [(288, 256), (256, 288), (224, 224), (128, 128), (1344, 768)]:
        assert host.token_grid(w, h)[2] == 1.0


def test_workload_tokens(page_facts):
    for w, h, frames, flat, n in page_facts["workload_tokens"]["cases"]:
        f = host.align_frames(frames)
        assert f == frames
        assert host.latent_frames(f) == flat
        gh, gw, _ = host.token_grid(w, h)
        assert host.n_tokens(flat, gh, gw) == n


def test_latent_frames_ceil_on_aligned_counts():
    for n in range(40):
        f = 5 + 17 * n
        assert host.latent_frames(f) == -(-f // 4)


def test_fresh_counts(page_facts):
    for steps, reuse, want in page_facts["fresh_evaluations"]["cases"]:
        sig, fresh = host.schedule(steps, reuse)
        assert len(fresh) == steps and len(sig) == steps + 1
        assert int(fresh.sum()) == want


def test_sigma_grid_linear_with_endpoint():
    for steps in (1, 2, 4, 7, 20, 50):
        sig, fresh = host.schedule(steps)
        assert sig.dtype == np.float32
        assert sig[0] == 1.0 and sig[-1] == 0.0
        assert np.all(np.diff(sig.astype(np.float64)) < 0)
        np.testing.assert_allclose(np.diff(sig.astype(np.float64)), -1.0 / steps, rtol=0, atol=1.2e-7)
        np.testing.assert_array_equal(sig, np.array([(steps - i) / steps for i in range(steps + 1)], np.float32))
        assert fresh.all()  # --reuse 1: every pass runs the model


def test_reuse_fresh_positions_and_last_step():
    sig, fresh = host.schedule(20, 2)
    assert list(np.nonzero(fresh)[0]) == [0, 2, 4, 6, 8, 10, 12, 14, 16, 18, 19]
    sig, fresh = host.schedule(20, 3)
    assert list(np.nonzero(fresh)[0]) == [0, 3, 6, 9, 12, 15, 18, 19]


def test_reuse_and_core_reuse_exclusive():
    with pytest.raises(ValueError):
        host.schedule(20, 2, 4)
    with pytest.raises(ValueError):
        host.schedule(20, 1, 7)   # core-reuse values above 6 are not offered
    with pytest.raises(ValueError):
        host.schedule(0)


def test_core_reuse_marks_core_fresh_steps_like_reuse():
    # the same rule as --reuse: step i runs the core iff i mod k == 0 or it is the last step
    for k in range(2, 7):
        _, fresh_c = host.schedule(20, 1, k)
        _, fresh_r = host.schedule(20, k, 1)
        np.testing.assert_array_equal(fresh_c, fresh_r)
    _, fresh = host.schedule(20, 1, 4)
    assert list(np.nonzero(fresh)[0]) == [0, 4, 8, 12, 16, 19]


def _table_with_scores(scores, d=3):
    # gates g1 = score/(2d) in every channel, g2 the same, so the key is exactly the score
    t = np.zeros((len(scores), 6, d))
    for b, s in enumerate(scores):
        t[b, 2, :] = s / (2 * d)
        t[b, 5, :] = -s / (2 * d)
    return t


def test_select_layers_brute_force():
    # brute force over every dropped subset: the dropped middle blocks must all rank below
    # every kept middle block under the key (score, -index); exactly one subset qualifies
    rng = np.random.default_rng(3)
    for nb in (2, 3, 5, 8):
        t = rng.normal(size=(nb, 6, 4))
        scores = host.gate_scores(t)
        key = {b: (scores[b], -b) for b in range(nb)}
        middle = range(1, nb - 1)
        for L in range(2, nb + 1):
            got = host.select_layers(t, L)
            valid = []
            for dropped in itertools.combinations(middle, nb - L):
                kept = [b for b in middle if b not in dropped]
                if not dropped or not kept or max(key[b] for b in dropped) < min(key[b] for b in kept):
                    valid.append(sorted(set(range(nb)) - set(dropped)))
            assert len(valid) == 1
            assert got == valid[0]
            assert got[0] == 0 and got[-1] == nb - 1 and len(got) == L
    # the score is the float64 sum of |gate1| + |gate2| over channels
    t = rng.normal(size=(3, 6, 5))
    want = [float(np.abs(t[b, 2]).sum() + np.abs(t[b, 5]).sum()) for b in range(3)]
    np.testing.assert_allclose(host.gate_scores(t), want, rtol=1e-15)


def test_select_layers_known_scores_and_ties():
    t = _table_with_scores([9, 1, 5, 1, 7, 0.5])
    # middle blocks 1..4 with scores 1,5,1,7; drop two lowest: scores 1 (blocks 1 and 3)
    assert host.select_layers(t, 4) == [0, 2, 4, 5]
    # drop one: tie at score 1 -> the higher index (3) goes first
    assert host.select_layers(t, 5) == [0, 1, 2, 4, 5]
    # first and last are protected even with the smallest scores
    t2 = _table_with_scores([0, 3, 2, 0])
    assert host.select_layers(t2, 2) == [0, 3]
    assert host.select_layers(t2, 4) == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        host.select_layers(t2, 1)
    with pytest.raises(ValueError):
        host.select_layers(t2, 5)


def test_token_plan_pairs_by_reshape(page_facts):
    facts = page_facts["token_reduction_positions"]
    for f, gh, gw in [(2, 8, 8), (6, 16, 16), (2, 3, 5), (1, 15, 27), (1, 1, 1)]:
        n_active = 45
        idx = np.arange(f * gh * gw).reshape(f, gh, gw)
        if gw % 2:
            idx = np.concatenate([idx, idx[:, :, -1:]], axis=2)
        want = np.stack([idx[:, :, 0::2].ravel(), idx[:, :, 1::2].ravel()], axis=1)
        for ev, restore in [(0, facts["restore_before_first10"]), (9, facts["restore_before_first10"]),
                            (10, facts["restore_before_later"]), (15, facts["restore_before_later"])]:
            p = host.token_plan(f, gh, gw, ev, n_active)
            assert p["merge_after"] == facts["merge_after"]
            assert p["restore_before"] == restore
            np.testing.assert_array_equal(p["pairs"], want)
            assert p["n_reduced"] == f * gh * ((gw + 1) // 2)


def test_token_plan_short_lists():
    p = host.token_plan(6, 16, 16, 0, 20)
    assert p["restore_before"] == 21  # head
    assert p["n_reduced"] == 768
    with pytest.raises(ValueError):
        host.token_plan(6, 16, 16, 0, 3)
