"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one.

A pin set that passes a wrong oracle pins nothing; every mutant below must make
at least one pin of test_oracle_pins.py fail.
"""
import numpy as np
import pytest

import oracle.svg_oracle as O
from tests import test_oracle_pins as pins


def _mut_spatial_strict(q_t, k_t, P, w_f):
    fq = np.asarray(q_t)[:, None] // P
    fk = np.asarray(k_t)[None, :] // P
    return np.abs(fq - fk) < w_f + (w_f == 0)          # off-by-one window


def _mut_temporal_frame(q_t, k_t, P, w_p):
    return np.abs(np.asarray(q_t)[:, None] // P - np.asarray(k_t)[None, :] // P) <= w_p   # frame, not location


def _mut_temporal_stride_rows(q_t, k_t, P, w_p):
    return np.abs(np.asarray(q_t)[:, None] - np.asarray(k_t)[None, :]) % P <= w_p       # wraps across rows


def _mut_perm_wrong_axes(F, P):
    return np.arange(F * P).reshape(P, F).T.ravel()                                    # reshaped the wrong way


def _mut_attention_no_scale(q, k, v, mask, scale):
    return ORIG["attention"](q, k, v, mask, 1.0)


def _mut_attention_no_max_guard(q, k, v, mask, scale):
    logits = scale * (np.asarray(q) @ np.asarray(k).T)
    w = np.exp(logits) * mask                                                          # ignores row normalisation
    return w @ np.asarray(v)


def _mut_attention_transposed_v(q, k, v, mask, scale):
    out = ORIG["attention"](q, k, v, mask, scale)
    return out[:, ::-1]                                                                # channel order flipped


def _mut_profile_vs_spatial(q, k, v, idx, F, P, w_f, w_p, scale):
    idx = np.asarray(idx)
    o_sp = O.head_attention_rows(q, k, v, idx, O.SPATIAL, F, P, w_f, w_p, scale)
    o_tp = O.head_attention_rows(q, k, v, idx, O.TEMPORAL, F, P, w_f, w_p, scale)
    mse_sp = 0.0
    mse_tp = float(np.mean((o_tp - o_sp) ** 2))                                        # compares against the wrong reference
    return mse_sp, mse_tp, O.SPATIAL if mse_sp <= mse_tp else O.TEMPORAL


def _mut_profile_tie_temporal(q, k, v, idx, F, P, w_f, w_p, scale):
    a, c, _ = ORIG["profile_head"](q, k, v, idx, F, P, w_f, w_p, scale)
    return a, c, O.SPATIAL if a < c else O.TEMPORAL                                    # tie goes the other way


def _mut_profile_argmax(q, k, v, idx, F, P, w_f, w_p, scale):
    a, c, _ = ORIG["profile_head"](q, k, v, idx, F, P, w_f, w_p, scale)
    return a, c, O.SPATIAL if a >= c else O.TEMPORAL                                   # picks the larger error


def _mut_rms_no_eps(x, w, eps):
    return ORIG["rms_norm"](x, w, 0.0)


def _mut_rms_mean_abs(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.mean(np.abs(x), axis=-1, keepdims=True) + eps) * w


def _mut_rope_sign(x, F, HH, WW, base, dims=None):
    xc = np.array(x, dtype=np.float64)
    xc[..., 1::2] *= -1                                                                # conj -> rotate -> conj:
    y = ORIG["rope_3d"](xc, F, HH, WW, base, dims)                                     # turns by -theta
    y[..., 1::2] *= -1
    return y


def _mut_rope_freq(x, F, HH, WW, base, dims=None):
    return ORIG["rope_3d"](x, F, HH, WW, base ** 0.5, dims)                            # half the exponent


def _mut_rope_axes(x, F, HH, WW, base, dims=None):
    return ORIG["rope_3d"](x, F, WW, HH, base, dims)                                   # rows and columns swapped


def _mut_block_mask_floor(kind, F, P, w_f, w_p, bm, bn, q_blocks=None):
    out = ORIG["block_mask"](kind, F, P, w_f, w_p, bm, bn, q_blocks)
    S = F * P
    if S % bm:
        out = out[:-1]                                                                 # drops the ragged last row block
    return out


def _mut_block_mask_layout(kind, F, P, w_f, w_p, bm, bn, q_blocks=None):
    S = F * P
    nqb, nkb = -(-S // bm), -(-S // bn)
    out = np.zeros((nqb, nkb), dtype=np.uint8)
    for i in range(nqb):
        rows = np.arange(i * bm, min(S, (i + 1) * bm))
        m = O.mask_rows(kind, rows, S, P, w_f, w_p).any(axis=0)                        # forgets the token-major layout
        m = np.concatenate([m, np.zeros(nkb * bn - S, dtype=bool)])
        out[i] = m.reshape(nkb, bn).any(axis=1)
    return out


def _mut_qknorm_swap_weights(q, k, wq, wk, eps, F, HH, WW, base, dims=None):
    return ORIG["qknorm_rope"](q, k, wk, wq, eps, F, HH, WW, base, dims)                  # weights exchanged


def _mut_qknorm_rope_first(q, k, wq, wk, eps, F, HH, WW, base, dims=None):
    return (O.rms_norm(O.rope_3d(q, F, HH, WW, base, dims), wq, eps),                   # RoPE before the norm
            O.rms_norm(O.rope_3d(k, F, HH, WW, base, dims), wk, eps))


def _mut_qknorm_q_only(q, k, wq, wk, eps, F, HH, WW, base, dims=None):
    qo, _ = ORIG["qknorm_rope"](q, k, wq, wk, eps, F, HH, WW, base, dims)
    return qo, O.rope_3d(k, F, HH, WW, base, dims)                                     # K not normalised


def _mut_agree_always(kind_a, kind_b, mse_ref, rel_tie=1e-6):
    return np.ones(np.shape(kind_a), dtype=bool)                                       # vacuous checker


def _mut_agree_min_ref(kind_a, kind_b, mse_ref, rel_tie=1e-6):
    a, c = mse_ref[..., 0], mse_ref[..., 1]
    near = np.abs(a - c) <= rel_tie * np.maximum(np.minimum(a, c), 1e-300)             # gap relative to the smaller
    return (kind_a == kind_b) | near


def _mut_agree_absolute(kind_a, kind_b, mse_ref, rel_tie=1e-6):
    a, c = mse_ref[..., 0], mse_ref[..., 1]
    return (kind_a == kind_b) | (np.abs(a - c) <= rel_tie)                             # absolute, not relative


ORIG = {n: getattr(O, n) for n in ("attention", "profile_head", "rms_norm", "rope_3d", "block_mask",
                                  "qknorm_rope", "choices_agree")}

MUTANTS = [
    ("mask_spatial", _mut_spatial_strict),
    ("mask_temporal", _mut_temporal_frame),
    ("mask_temporal", _mut_temporal_stride_rows),
    ("perm_indices", _mut_perm_wrong_axes),
    ("attention", _mut_attention_no_scale),
    ("attention", _mut_attention_no_max_guard),
    ("attention", _mut_attention_transposed_v),
    ("profile_head", _mut_profile_vs_spatial),
    ("profile_head", _mut_profile_tie_temporal),
    ("profile_head", _mut_profile_argmax),
    ("rms_norm", _mut_rms_no_eps),
    ("rms_norm", _mut_rms_mean_abs),
    ("rope_3d", _mut_rope_sign),
    ("rope_3d", _mut_rope_freq),
    ("rope_3d", _mut_rope_axes),
    ("block_mask", _mut_block_mask_floor),
    ("block_mask", _mut_block_mask_layout),
    ("qknorm_rope", _mut_qknorm_swap_weights),
    ("qknorm_rope", _mut_qknorm_rope_first),
    ("qknorm_rope", _mut_qknorm_q_only),
    ("choices_agree", _mut_agree_always),
    ("choices_agree", _mut_agree_min_ref),
    ("choices_agree", _mut_agree_absolute),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[f"{n}:{m.__name__}" for n, m in MUTANTS])
def test_pins_catch_mutant(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as exc:  # an assertion, or the mutant breaking a shape
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught mutant {mutant.__name__} of {name}"
