"""Planted controls for the parity checkers (no GPU).

The TensorFold page (section "핵심 메커니즘 3 — 커널 계약") pairs every kernel
gate with deliberately wrong results that the gate must reject; a control that
passes means the gate has no teeth.  Here the wrong results are computed on the
host from the oracle's own inputs with one plausible kernel slip planted each:
swapped nibbles, the last group dropped, a neighbouring group's scale, the bias
term dropped or negated, bf16 accumulation, rows exchanged, a single output off
by more than the tolerance, bf16-rounded fp32 logits, an argmax that drops NaN,
the last NaN or the highest index of a tie winning, the runner-up chosen where
the top-2 gap is wide.  Each must make the checker used by the GPU tests fail,
and the correct result must pass it.
"""
import numpy as np
import pytest

import oracle
from bit_quantized_decode_group_amd import synth
from tests.gpu_util import assert_close, assert_close_f32, assert_ids, rows_identical

M, N, K = 8, 64, 1024


def _bf16_round(a):
    """fp64 -> bf16 -> fp64, nearest even (through fp32, as a bf16-storing kernel would)."""
    b = np.asarray(a, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


@pytest.fixture(scope="module")
def proj():
    d = synth.single_projection(M=M, N=N, K=K, seed=4242)
    ref = oracle.qgemv_affine4(d["x"], d["codes"], d["scales"], d["biases"])
    return d, ref


def _oracle_y(d, codes=None, scales=None, biases=None, x=None):
    return oracle.qgemv_affine4(d["x"] if x is None else x, d["codes"] if codes is None else codes,
                                d["scales"] if scales is None else scales, d["biases"] if biases is None else biases)


def _bf16_accumulate(d):
    """What a kernel that keeps its running sum in bf16 would output."""
    x = oracle.bf16_array_to_f64(d["x"]).reshape(M, K)
    w = oracle.dequant_affine4(d["codes"], d["scales"], d["biases"])
    acc = np.zeros((M, N))
    for k in range(K):
        acc = _bf16_round(acc + np.outer(x[:, k], w[:, k]))
    return acc


def _controls(d, ref):
    c = d["codes"]
    swapped = ((c & 0x0F0F0F0F) << 4) | ((c >> 4) & 0x0F0F0F0F)
    s_drop, b_drop = d["scales"].copy(), d["biases"].copy()
    s_drop[:, -1] = 0
    b_drop[:, -1] = 0
    s_nb = d["scales"][:, np.arange(K // 64) ^ 1]
    b_neg = d["biases"] ^ np.uint16(0x8000)
    x_rows = d["x"][[1, 0, 2, 3, 4, 5, 6, 7]]
    one_off = _bf16_round(ref).copy()
    rms = float(np.sqrt(np.mean(ref ** 2)))
    one_off[3, 17] += 3e-2 * rms
    return {
        "swapped nibbles": _oracle_y(d, codes=swapped),
        "last group dropped": _oracle_y(d, scales=s_drop, biases=b_drop),
        "neighbouring group's scale": _oracle_y(d, scales=s_nb),
        "bias term dropped": _oracle_y(d, biases=np.zeros_like(d["biases"])),
        "bias negated": _oracle_y(d, biases=b_neg),
        "rows exchanged": _oracle_y(d, x=x_rows),
        "bf16 accumulation": _bf16_accumulate(d),
        "one output off by 3e-2 rms": one_off,
    }


def test_correct_projection_passes(proj):
    d, ref = proj
    assert_close(_bf16_round(ref), ref, what="control: correct")


@pytest.mark.parametrize("name", ["swapped nibbles", "last group dropped", "neighbouring group's scale",
                                  "bias term dropped", "bias negated", "rows exchanged", "bf16 accumulation",
                                  "one output off by 3e-2 rms"])
def test_planted_projection_slip_is_rejected(proj, name):
    d, ref = proj
    wrong = _bf16_round(_controls(d, ref)[name])
    with pytest.raises(AssertionError):
        assert_close(wrong, ref, what=f"control: {name}")


def test_fp32_logits_bar_has_no_rounding_allowance():
    d = synth.lm_head(M=4, V=600, K=512, seed=4243)
    logits, _, _, _ = oracle.lmhead(d["x"], d["codes"], d["scales"], d["biases"])
    assert_close_f32(logits.astype(np.float32), logits, what="control: fp32 logits")
    with pytest.raises(AssertionError):
        assert_close_f32(_bf16_round(logits), logits, what="control: bf16-rounded logits")


def _lm_rows(V, K, bias_bits):
    codes = np.zeros((V, K // 8), np.uint32)
    scales = np.full((V, K // 64), 0x3F80, np.uint16)
    biases = np.repeat(np.asarray(bias_bits, np.uint16).reshape(V, 1), K // 64, axis=1)
    return codes, scales, biases


def test_argmax_checker_rejects_nan_drop_last_nan_and_high_tie():
    V, Kl = 300, 64
    x = np.full((1, Kl), 0x3F80, np.uint16)
    bias = np.full(V, 0x3F00, np.uint16)  # logits 0.5 * 64 = 32
    bias[200] = 0x3F80                     # 64: the strict maximum
    bias[40] = 0x3F80                      # an exact tie at a lower index
    logits, ids, gap, _ = oracle.lmhead(x, *_lm_rows(V, Kl, bias))
    assert ids[0] == 40 and gap[0] == 0.0
    assert_ids([40], ids, gap, logits, what="control: tie, lowest index")
    with pytest.raises(AssertionError):
        assert_ids([200], ids, gap, logits, what="control: tie to the highest index")
    bias[120] = 0x7FC0  # NaN logits: the first NaN wins
    bias[250] = 0x7FC0
    logits, ids, gap, _ = oracle.lmhead(x, *_lm_rows(V, Kl, bias))
    assert ids[0] == 120
    assert_ids([120], ids, gap, logits, what="control: first NaN")
    for wrong, why in ((40, "fmax-style argmax dropping NaN"), (250, "last NaN wins")):
        with pytest.raises(AssertionError):
            assert_ids([wrong], ids, gap, logits, what=f"control: {why}")


def test_argmax_checker_wide_and_narrow_gaps():
    d = synth.lm_head(M=8, V=2000, K=256, seed=4244)
    logits, ids, gap, _ = oracle.lmhead(d["x"], d["codes"], d["scales"], d["biases"])
    runner_up = np.argsort(-logits, axis=1, kind="stable")[:, 1]
    assert_ids(ids, ids, gap, logits, what="control: oracle ids")
    wide = [m for m in range(8) if gap[m] > 1e-2]
    assert wide
    for m in wide:
        bad = ids.copy()
        bad[m] = runner_up[m]
        with pytest.raises(AssertionError):
            assert_ids(bad, ids, gap, logits, what=f"control: runner-up in row {m}")
    # a near tie (0 < gap <= 1e-2): either of the two is a correct greedy id (reading R16)
    lg = logits.copy()
    lg[0, runner_up[0]] = lg[0, ids[0]] - 5e-3
    assert_ids([runner_up[0]] + list(ids[1:]), ids, np.r_[5e-3, gap[1:]], lg, what="control: near tie")


def test_rows_identical_helper():
    y = np.arange(24, dtype=np.uint16).reshape(3, 8)
    assert rows_identical(y, [y[0], y[1], y[2]]) == []
    z = y[2].copy()
    z[5] ^= 1
    assert rows_identical(y, [y[0], y[1], z]) == [2]
