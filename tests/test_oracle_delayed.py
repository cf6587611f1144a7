"""Pins of the oracle's delayed scaling (ROCm 7.0 FP8/MXFP8/MXFP4 article,
training part: "Delayed Scaling" -- quantise with the scale from earlier
steps, next scale = amax / 400, initial scale 1; its pitfall section: an amax
history window and the "max" compute algorithm)."""
import os

import numpy as np
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "delayed_scaling_case.txt")


def _bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def test_hand_worked_steps():
    rows = [ln for ln in open(GOLD) if ln[:1].isdigit()]
    x = np.array([[float(v) for v in r.split("|")[0].split()[1:]] for r in rows], np.float32)
    codes = np.array([[int(c, 16) for c in r.split("|")[1].split()] for r in rows], np.uint8)
    s_max = np.array([float(r.split("|")[2].split()[0]) for r in rows], np.float32)
    s_lat = np.array([float(r.split("|")[2].split()[1]) for r in rows], np.float32)
    q, s = O.delayed_scaling(_bits(x), 2, 0)
    np.testing.assert_array_equal(q, codes)
    np.testing.assert_array_equal(s, s_max)
    _, s = O.delayed_scaling(_bits(x), 2, 1)
    np.testing.assert_array_equal(s, s_lat)


def _steps(S=12, n=256, seed=0):
    rng = np.random.default_rng(seed)
    mag = 2.0 ** rng.uniform(-6, 6, size=(S, 1))
    x = (rng.standard_normal((S, n)) * mag).astype(np.float32)
    x[4] = 0.0                                             # an all-zero step
    return _bits(x)


def test_scale_follows_the_history_rule():
    bits = _steps()
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    amax = np.abs(x).max(axis=1)
    for L in (1, 3, 100):
        _, s_lat = O.delayed_scaling(bits, L, 1)
        _, s_max = O.delayed_scaling(bits, L, 0)
        assert s_lat[0] == 1 and s_max[0] == 1
        for t in range(1, len(amax)):
            h = amax[t - 1]
            want = np.float32(1.0) if h == 0 else np.float32(h) / np.float32(400.0)
            assert s_lat[t] == want
            h = amax[max(0, t - L):t].max()
            want = np.float32(1.0) if h == 0 else np.float32(h) / np.float32(400.0)
            assert s_max[t] == want, (L, t)


def test_codes_are_the_clamped_quotient_by_the_step_scale():
    bits = _steps(seed=1)
    q, s = O.delayed_scaling(bits, 4, 0)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    t = (x / torch.from_numpy(s)[:, None]).clamp(-448, 448)           # fp32 quotient (torch)
    want = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q, want)
