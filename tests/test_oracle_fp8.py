"""Pins of the FP8 oracle (CPU only): the E4M3 decode against torch's own
float8_e4m3fn conversion and the format's fixed values; the FP8 forward as
exact attention of the descaled values; and the output bound checked by brute
force, rounding P to E4M3 with torch's conversion at many reference points,
including adversarial rows (rounding ties, many weights in the subnormal
range) that a weaker bound misses."""

import inspect

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import fp8 as o8
from workloads import fp8_exact_weight_inputs, fp8_random_inputs


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def pin_decode_table():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = o8.e4m3_decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])
    # fixed points of the format: 1, 448, smallest normal and subnormal, -1
    fixed = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0xB8: -1.0, 0x44: 3.0, 0xFE: -448.0}
    for c, val in fixed.items():
        assert o8.e4m3_decode(np.array([c]))[0] == val, hex(c)
    assert np.isnan(o8.e4m3_decode(np.array([0x7F, 0xFF]))).all()


def pin_forward_is_attention_of_values():
    d = fp8_random_inputs(2, 9, 13, 3, 64, 11)
    for causal in (False, True):
        O, LSE = o8.attention_forward_fp8(d["q"], d["k"], d["v"], d["descale_q"],
                                          d["descale_k"], d["descale_v"], causal=causal)
        vals = {n: _torch_decode(d[n].numpy()) * d["descale_" + n].double().numpy()[:, None, :, None]
                for n in "qkv"}
        O2, LSE2 = oa.attention_forward(vals["q"], vals["k"], vals["v"], causal=causal)
        assert np.allclose(O, O2, rtol=0, atol=1e-14) and np.allclose(LSE, LSE2, rtol=0, atol=1e-14)


def _simulated_kernel_outputs(d, causal, scale, lags):
    """O^ = sum p^ v / sum p^ with p^ the E4M3 rounding (torch) of the weights
    taken against reference points `lag` (log2 units) below each row max."""
    Q = o8._descaled(d["q"], d["descale_q"])
    K = o8._descaled(d["k"], d["descale_k"])
    V = o8._descaled(d["v"], d["descale_v"])
    if scale is None:
        scale = 1.0 / np.sqrt(Q.shape[-1])
    P = oa.attention_probs(Q, K, causal=causal, scale=scale)
    p = P / P.max(-1, keepdims=True)
    Vh = np.transpose(V, (0, 2, 1, 3))
    outs = []
    for lag in lags:
        w = p * 2.0 ** lag
        w_hat = torch.from_numpy(w).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        oh = (w_hat @ Vh) / w_hat.sum(-1, keepdims=True)
        outs.append(np.transpose(oh, (0, 2, 1, 3)))
    return outs


def _check_bound(d, causal=False, scale=None, lags=(0.0, 0.37, 1.0, 3.6, 7.99)):
    O, _ = o8.attention_forward_fp8(d["q"], d["k"], d["v"], d["descale_q"], d["descale_k"],
                                    d["descale_v"], causal=causal, scale=scale)
    E = o8.fp8_output_bound(d["q"], d["k"], d["v"], d["descale_q"], d["descale_k"],
                            d["descale_v"], causal=causal, scale=scale)
    # the 2^-8 |O| output-rounding and 1e-4 accumulation terms are not in
    # the simulation; take them out so the P-rounding part is checked alone
    vmax = np.abs(o8._descaled(d["v"], d["descale_v"])).max(axis=(1, 3))
    E_p = E - 2.0 ** -8 * np.abs(O) - 1e-4 * vmax[:, None, :, None]
    worst = 0.0
    for oh in _simulated_kernel_outputs(d, causal, scale, lags):
        err = np.abs(oh - O)
        assert np.all(err <= E_p + 1e-12), float(np.max(err - E_p))
        worst = max(worst, float(np.max(err / np.maximum(E_p, 1e-300))))
    return worst


def pin_bound_random_rows():
    for causal in (False, True):
        d = fp8_random_inputs(1, 40, 40, 2, 64, 21)
        _check_bound(d, causal)
        _check_bound(d, causal, scale=1.0)   # peaked rows


def _tie_inputs(n=4):
    """Rows whose keys all sit on E4M3 rounding ties in opposite directions:
    keys of type A (code k = 1.0, value +1) and type B (k = 0, value -1) with
    exp(score_A - score_B) = 1.1875 / 1.0625.  Against a reference point
    log2(1.1875) below the row max, A weighs 1.1875 (rounds up to 1.25) and B
    1.0625 (rounds down to 1.0), so every rounding moves the output the same
    way."""
    D, nk = 64, 2 * n
    codes_q = np.zeros((1, 1, 1, D), np.uint8); codes_q[..., 0] = 0x38
    codes_k = np.zeros((1, nk, 1, D), np.uint8); codes_k[0, 0::2, 0, 0] = 0x38
    codes_v = np.full((1, nk, 1, D), 0xB8, np.uint8); codes_v[0, 0::2] = 0x38
    one = torch.ones((1, 1))
    return ({"q": torch.from_numpy(codes_q), "k": torch.from_numpy(codes_k),
             "v": torch.from_numpy(codes_v), "descale_q": one, "descale_k": one,
             "descale_v": one}, float(np.log(1.1875 / 1.0625)))


def pin_bound_rounding_tie():
    d, scale = _tie_inputs()
    worst = _check_bound(d, scale=scale, lags=(float(np.log2(1.1875)),))
    assert worst > 0.8, worst   # the bound is nearly attained


def _tiny_weight_inputs():
    """One key at the row max and many keys whose weight (about 0.9 * 2^-10)
    rounds to zero in E4M3, all with value +1 against -1 at the max key."""
    D, nk = 64, 600
    codes_q = np.zeros((1, 1, 1, D), np.uint8); codes_q[..., 0] = 0x38
    codes_k = np.zeros((1, nk, 1, D), np.uint8); codes_k[0, 0, 0, 0] = 0x38
    codes_v = np.full((1, nk, 1, D), 0x38, np.uint8); codes_v[0, 0] = 0xB8
    one = torch.ones((1, 1))
    scale = float(-np.log(0.9 * 2.0 ** -10))   # key 0 score = scale, others 0
    return ({"q": torch.from_numpy(codes_q), "k": torch.from_numpy(codes_k),
             "v": torch.from_numpy(codes_v), "descale_q": one, "descale_k": one,
             "descale_v": one}, scale)


def pin_bound_subnormal_floor():
    d, scale = _tiny_weight_inputs()
    worst = _check_bound(d, scale=scale, lags=(0.0,))
    assert worst > 0.5, worst


def pin_rows_match_full():
    """The row-sampled bound and forward equal the full ones at those rows."""
    for causal, (nq, nk) in ((False, (30, 30)), (True, (30, 30)), (True, (40, 25))):
        d = fp8_random_inputs(2, nq, nk, 2, 64, 41)
        args = (d["q"], d["k"], d["v"], d["descale_q"], d["descale_k"], d["descale_v"])
        O, LSE = o8.attention_forward_fp8(*args, causal=causal)
        E = o8.fp8_output_bound(*args, causal=causal)
        rows = [0, 7, nq - 1]
        r = o8.fp8_rows(*args, 1, 1, rows, causal=causal)
        assert np.allclose(r["O"], O[1, rows, 1], rtol=0, atol=1e-14)
        assert np.array_equal(np.isneginf(r["LSE"]), np.isneginf(LSE[1, 1, rows]))
        fin = np.isfinite(r["LSE"])
        assert np.allclose(r["LSE"][fin], LSE[1, 1, rows][fin], rtol=0, atol=1e-14)
        assert np.allclose(r["bound"], E[1, rows, 1], rtol=0, atol=1e-14)


def pin_exact_weight_inputs():
    """The exact-weight recipe: every weight a power of two in [2^-8, 2^8]."""
    d = fp8_exact_weight_inputs(1, 30, 50, 2, 64, 31)
    Q = o8._descaled(d["q"], d["descale_q"])
    K = o8._descaled(d["k"], d["descale_k"])
    S = np.einsum("bnhd,bmhd->bhnm", Q, K) * d["scale"] / np.log(2.0)   # log2 weights
    assert np.allclose(S, np.round(S), atol=1e-9) and np.abs(S).max() <= 4 + 1e-9
    for oh in _simulated_kernel_outputs(d, False, d["scale"], (0.0, 1.0, 4.0)):
        O, _ = o8.attention_forward_fp8(d["q"], d["k"], d["v"], d["descale_q"],
                                        d["descale_k"], d["descale_v"], scale=d["scale"])
        assert np.allclose(oh, O, rtol=0, atol=1e-12)


ALL_PINS = [pin_decode_table, pin_forward_is_attention_of_values, pin_bound_random_rows,
            pin_bound_rounding_tie, pin_bound_subnormal_floor, pin_rows_match_full,
            pin_exact_weight_inputs]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


# Planted mistakes in the decode and the bound.
MUTANTS = {
    "decode_bias_8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "decode_subnormal_as_normal": ("np.where(e == 0, (m / 8.0) * 2.0 ** -6,",
                                   "np.where(e == -1, (m / 8.0) * 2.0 ** -6,"),
    "decode_sign_ignored": ("np.where(c & 0x80, -1.0, 1.0)", "np.where(c & 0x80, 1.0, 1.0)"),
    "bound_half_relative": ("np.maximum(2.0 ** -4 * p, 2.0 ** -10)",
                            "np.maximum(2.0 ** -5 * p, 2.0 ** -10)"),
    "bound_no_subnormal_floor": ("np.maximum(2.0 ** -4 * p, 2.0 ** -10)",
                                 "np.maximum(2.0 ** -4 * p, 0.0)"),
    "bound_unrounded_denominator": ("p.sum(1) - e.sum(1)", "p.sum(1) + e.sum(1)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    old, new = MUTANTS[name]
    fn = o8.e4m3_decode if name.startswith("decode") else o8._bound_rows
    src = inspect.getsource(fn)
    assert src.count(old) == 1, f"mutation site for {name} not found"
    ns = dict(vars(o8))
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(o8, fn.__name__, ns[fn.__name__])
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
