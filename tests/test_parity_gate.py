"""The parity gate itself, on the CPU: a plausible kernel mistake confined to late causal
queries must fail it.

Causal attention outputs of late queries average many values and are about 1/40 of the
outputs of the first queries, so the per-tensor ratio max|err| / max|ref| lets a large error
on them through; the per-row ratio of helpers.assert_close does not.  The outputs are the
oracle's causal attention ([NeMo-MLA] forward with a causal attention_mask) on N(0,1) inputs
at the V3 prefill length and head width."""
import numpy as np
import pytest

import synth
from oracle import mla_oracle as O
from helpers import TOL, assert_close, rel_err, row_rel_err

T, H = 8192, 8


@pytest.fixture(scope="module")
def late_rows():
    w = synth.custom(synth.WORKLOADS[4], 150, "gate-check", n_heads=H)
    q = O.decode_tensor("bf16", synth.make_normal(w, "gate.q", (T, H, 192)).data)
    k = O.decode_tensor("bf16", synth.make_normal(w, "gate.k", (T, H, 192)).data)
    v = O.decode_tensor("bf16", synth.make_normal(w, "gate.v", (T, H, 128)).data)
    rows = np.array(sorted({0, 1, 2, 63, 64, 65, 127, 128, T // 2, T // 2 + 1, 5000, 6000, 7000, T - 2, T - 1}))
    ref = O.attention(q[rows], k, v, O.softmax_scale(128, 64), rows)
    return rows, ref


def test_late_row_error_fails_the_row_gate(late_rows):
    rows, ref = late_rows
    got = ref.copy()
    got[rows >= T // 2] *= 1.5
    # the tensor-wide ratio alone would pass this output
    assert rel_err(got, ref) < TOL["bf16"]
    err, i = row_rel_err(got, ref)
    assert err == pytest.approx(0.5, rel=1e-9) and rows[i] >= T // 2
    with pytest.raises(AssertionError):
        assert_close(got, ref, "bf16", "o (planted 1.5x on late rows)", rows)


def test_dropped_late_rows_fail(late_rows):
    rows, ref = late_rows
    got = ref.copy()
    got[rows >= T // 2] = 0.0
    with pytest.raises(AssertionError):
        assert_close(got, ref, "bf16", "o (late rows zero)", rows)


def test_bf16_rounding_passes(late_rows):
    """The output's own storage rounding (bf16, relative 2^-9) is far inside both gates."""
    rows, ref = late_rows
    got = O.bf16_round(ref)
    assert_close(got, ref, "bf16", "o rounded to bf16", rows)
    assert row_rel_err(got, ref)[0] < 4e-3
