"""The pins catch plausible mistakes: each test compiles a copy of oracle.c
with one planted mistake (on the CPU, in a temporary directory), points the
oracle module at that build, and requires that at least one pin fails.  The
steps oracle.py itself orders (dec_in_proj, windowed decode and stitching,
the alias-free Snake and its filter) get the same treatment: a method of
its Model, or a function of the module, is recompiled from its source with
one planted mistake and patched in for the test.

A mutation that no pin notices would mean the pins leave that part of the
oracle unchecked.
"""
import inspect
import os
import textwrap

import pytest

from oracle import oracle as O

import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("snake_no_square", "yr[t] = xr[t] + s * s / den;", "yr[t] = xr[t] + s / den;"),
    ("snake_no_alpha", "const REAL s = SIN(a * xr[t]);", "const REAL s = SIN(xr[t]);"),
    ("snakebeta_uses_alpha", "const REAL den = (beta ? beta[c] : alpha[c]) + (REAL)1e-9;",
     "const REAL den = alpha[c] + (REAL)1e-9;"),
    ("snake_channel_as_time", "const REAL a = alpha[c];", "const REAL a = alpha[r % C];"),
    ("fold_no_sqrt", "const REAL n = SQRT(ss);", "const REAL n = ss;"),
    ("fold_no_g", "w[i * rest + j] = g[i] * v[i * rest + j] / n;", "w[i * rest + j] = v[i * rest + j] / n;"),
    ("conv_flipped_taps", "const REAL wv = w[(o * Cin + i) * K + j];",
     "const REAL wv = w[(o * Cin + i) * K + (K - 1 - j)];"),
    ("conv_no_dilation", "const int64_t sh = j * dil - P;", "const int64_t sh = j - P;"),
    ("conv_no_bias", "for (int64_t t = 0; t < T; ++t) yr[t] += bias[o];",
     "for (int64_t t = 0; t < T; ++t) yr[t] += 0;"),
    ("convt_crop_off_by_one", "const int64_t n = m * s + k - p;", "const int64_t n = m * s + k - p - 1;"),
    ("convt_transposed_weight", "const REAL *wr = w + (i * Cout + o) * K;",
     "const REAL *wr = w + ((o % Cin) * Cout + (i % Cout)) * K;"),
    ("convt_no_bias", "for (int64_t n = 0; n < Tout; ++n) yr[n] += bias[o];",
     "for (int64_t n = 0; n < Tout; ++n) yr[n] += 0;"),
    ("no_tanh", "y[k] = TANH(x[k]);", "y[k] = x[k];"),
    ("residual_sign", "y[k] = a[k] + b[k];", "y[k] = a[k] - b[k];"),
    ("strided_conv_no_stride", "const int64_t src = t * s + j - P;", "const int64_t src = t + j - P;"),
    ("strided_conv_pad_off_by_one", "const int64_t src = t * s + j - P;",
     "const int64_t src = t * s + j - P + 1;"),
]


def _pins(orc):
    """The oracle pins, run against whatever build `orc` currently loads."""
    P.test_snake_closed_form_points(orc)
    P.test_snake_double_angle_identity_and_bounds(orc)
    P.test_snake_periodicity(orc)
    P.test_snakebeta(orc)
    P.test_snake_channel_indexing(orc)
    P.test_weight_norm_invariants(orc)
    P.test_weight_norm_axis0_of_transposed_layout(orc)
    for d in (1, 3):
        P.test_conv1d_brute_force(orc, d)
        P.test_conv1d_torch_float64(orc, d)
    P.test_conv1d_k1_is_matrix_product(orc)
    P.test_conv1d_impulse_orientation(orc)
    for s in (3, 4):
        P.test_convt_equals_zero_stuffed_conv(orc, s)
        P.test_convt_torch_float64(orc, s)
        P.test_convt_polyphase_identity(orc, s)
    P.test_convt_impulse_response(orc)
    P.test_residual_unit_zero_conv2_is_identity(orc)
    P.test_decode_matches_torch_composition(orc, (2, 2), "snake", 0, 0)
    P.test_decode_matches_torch_composition(orc, (3, 2), "snakebeta", 0, 0)
    P.test_golden_lengths_and_vocoder_gate(orc)
    for s in (2, 8):
        P.test_strided_conv_brute_force_and_torch(orc, s)
    P.test_encoder_matches_torch_composition(orc, (8, 4))


def test_pins_pass_on_the_real_oracle():
    _pins(O)


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, orig, bad, tmp_path, monkeypatch):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation site not unique: {name}"
    mutant = tmp_path / f"{name}.c"
    mutant.write_text(src.replace(orig, bad))
    so = tmp_path / f"{name}.so"
    O.compile_library(str(mutant), str(so), "f64")
    lib = O.load_library(str(so), "f64")
    monkeypatch.setitem(O._loaded, "f64", lib)
    with pytest.raises(AssertionError):
        _pins(O)


# (name, Model method / "Class.method" / "fn:function", original text, planted mistake)
PY_MUTANTS = [
    ("af_up_crop_off_by_one", "fn:upsample2", "lo = 2 * pad + (k - 2) // 2", "lo = 2 * pad + (k - 2) // 2 + 1"),
    ("af_up_gain_missing_2", "fn:upsample2", "+= 2.0 * f[j] * z", "+= f[j] * z"),
    ("af_up_zero_pad", "fn:upsample2", "np.repeat(x[:, :, :1], pad, 2), x,",
     "np.zeros(x.shape[:2] + (pad,)), x,"),
    ("af_down_pads_swapped", "fn:downsample2",
     "np.repeat(v[:, :, :1], k // 2 - 1, 2), v, np.repeat(v[:, :, -1:], k // 2, 2)",
     "np.repeat(v[:, :, :1], k // 2, 2), v, np.repeat(v[:, :, -1:], k // 2 - 1, 2)"),
    ("af_down_zero_pad", "fn:downsample2", "np.repeat(v[:, :, :1], k // 2 - 1, 2)",
     "np.zeros(v.shape[:2] + (k // 2 - 1,))"),
    ("af_filter_no_window", "fn:af_filter", "f = 2.0 * cutoff * window * np.sinc(2.0 * cutoff * t)",
     "f = 2.0 * cutoff * np.sinc(2.0 * cutoff * t)"),
    ("af_filter_not_normalised", "fn:af_filter", "return f / f.sum()", "return f"),
    ("af_filter_centred_on_a_tap", "fn:af_filter", "t = np.arange(-half, half) + 0.5",
     "t = np.arange(-half, half) + 1.0"),
    ("kaiser_beta_wrong_branch", "fn:kaiser_beta", "return 0.1102 * (atten_db - 8.7)",
     "return 0.5842 * (atten_db - 21.0) ** 0.4 + 0.07886 * (atten_db - 21.0)"),
    ("af_snake_is_plain", "fn:af_snake", 'return _c(downsample2(snake(u, alpha, beta, "f64")), prec)',
     'return _c(snake(x, alpha, beta, "f64"), prec)'),
    ("model_ignores_af", "_snake", "y = af_snake(x, a[0], a[1], self.prec) if self.af else",
     "y = snake(x, a[0], a[1], self.prec) if self.af else"),
    ("log_params_not_exponentiated", "__init__", "return _c(np.exp(v) if log_params else v, prec)",
     "return _c(v, prec)"),
    ("window_first_cropped", "decode_windows", "lo = crop_left if k > 0 else 0", "lo = crop_left"),
    ("window_last_cropped", "decode_windows", "hi = length - (crop_right if k < n - 1 else 0)",
     "hi = length - crop_right"),
    ("window_right_off_by_one", "decode_windows", "hi = length - (crop_right if k < n - 1 else 0)",
     "hi = length - (crop_right + 1 if k < n - 1 else 0)"),
    ("window_last_full_length", "decode_windows", "length = last_frames if k == n - 1 else L",
     "length = L"),
    ("window_sides_interleaved", "decode_windows",
     "x = windows[k, :, :length].reshape(sides, c, length)",
     "x = windows[k, :, :length].reshape(c, sides, length).transpose(1, 0, 2)"),
    ("in_proj_no_bias", "stage_conv_in", "x = conv1d(x, self.in_proj[0], self.in_proj[1], 1, self.prec)",
     "x = conv1d(x, self.in_proj[0], None, 1, self.prec)"),
    ("in_proj_weight_normed", "__init__", 'w = np.asarray(t["dec_in_proj.weight"], dtype=np.float32)',
     'w = np.asarray(t["dec_in_proj.weight"], dtype=np.float32); '
     'w = (w / np.linalg.norm(w, axis=(1, 2), keepdims=True)).astype(np.float32)'),
    ("causal_conv1_centered", "stage_res_unit",
     'u["d"], self.prec, self.causal)', 'u["d"], self.prec, False)'),
    ("causal_convt_centered", "stage_upsample", "pad_left=convt_crop(blk[\"s\"], self.causal)",
     "pad_left=convt_crop(blk[\"s\"], False)"),
    ("causal_head_centered", "stage_head_pre", "w, b, 1, self.prec, self.causal)",
     "w, b, 1, self.prec, False)"),
    ("causal_conv_in_centered", "stage_conv_in", "return conv1d(x, w, b, 1, self.prec, self.causal)",
     "return conv1d(x, w, b, 1, self.prec, False)"),
    ("encoder_strides_not_reversed", "Encoder.__init__", "enumerate(reversed(cfg[\"strides\"]))",
     "enumerate(cfg[\"strides\"])"),
    ("encoder_no_snake_before_down", "Encoder.encode",
     "h = conv1d_strided(self._snake(h, blk[\"act\"]), blk[\"wd\"]",
     "h = conv1d_strided(h, blk[\"wd\"]"),
    ("encoder_proj_no_bias", "Encoder.encode", "self.proj[0], self.proj[1], 1, self.prec)",
     "self.proj[0], None, 1, self.prec)"),
    ("in_proj_after_snake", "stage_conv_in", "x = conv1d(x, self.in_proj[0], self.in_proj[1], 1, self.prec)",
     "x = conv1d(x, self.in_proj[0], self.in_proj[1], 1, self.prec); "
     "x = snake(x, np.ones(x.shape[1]), None, self.prec)"),
]


def _py_pins(orc):
    P.test_encoder_matches_torch_composition(orc, (8, 4))
    P.test_decode_matches_torch_composition(orc, (2, 2), "snake", 5, 0)
    P.test_decode_matches_torch_composition(orc, (3, 2), "snakebeta", 0, 1)
    P.test_causal_decode_of_a_prefix_is_a_prefix(orc, (8, 5))
    P.test_in_proj_composes_with_conv_in(orc)
    P.test_window_stitch_bookkeeping_at_the_pages_sizes(orc)
    P.test_windows_cut_from_one_track_equal_its_decode(orc)
    P.test_windows_planar_sides_and_single_window(orc)
    P.test_af_filter_is_the_kaiser_windowed_sinc(orc)
    P.test_af_resamplers_match_torch_routines(orc)
    P.test_af_upsampler_delay_and_gain(orc)
    P.test_af_snake_reach_is_five_frames(orc)
    P.test_alias_free_decode_matches_torch_composition(orc, (5, 2), "snakebeta")
    P.test_log_stored_snake_parameters_are_exponentiated(orc)


def test_python_pins_pass_on_the_real_oracle():
    _py_pins(O)


@pytest.mark.parametrize("name,method,orig,bad", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_planted_python_mistake_is_caught(name, method, orig, bad, monkeypatch):
    if method.startswith("fn:"):
        owner, meth = O, method[3:]
    else:
        cls, meth = method.split(".") if "." in method else ("Model", method)
        owner = getattr(O, cls)
    src = textwrap.dedent(inspect.getsource(getattr(owner, meth)))
    assert src.count(orig) == 1, f"mutation site not unique: {name}"
    ns = dict(vars(O))
    exec(compile(src.replace(orig, bad), f"<mutant {name}>", "exec"), ns)
    monkeypatch.setattr(owner, meth, ns[meth])
    with pytest.raises(AssertionError):
        _py_pins(O)


# Planted mistakes in the two-term operand rounding, against its own pins
# (kept apart from the list above: the end-to-end pin decodes a full-width
# stack, too slow to repeat for every mutant there).
TT_MUTANTS = [
    ("two_term_drops_low_term", "fn:round_bf16_two_term", "return hi + lo", "return hi"),
    ("two_term_low_term_sign", "fn:round_bf16_two_term", "lo = round_bf16((x32 - hi).astype(np.float32))",
     "lo = round_bf16((hi - x32).astype(np.float32))"),
    ("two_term_low_term_unrounded", "fn:round_bf16_two_term", "lo = round_bf16((x32 - hi).astype(np.float32))",
     "lo = (x32 - hi).astype(np.float32).astype(np.float64)"),
    ("operand_terms_ignored", "__init__",
     "self._round_op = round_bf16_two_term if operand_terms == 2 else round_bf16",
     "self._round_op = round_bf16"),
]


def _tt_pins(orc):
    P.test_two_term_bf16_rounding(orc)
    P.test_two_term_operands_meet_the_bf16_bound_end_to_end(orc)


@pytest.mark.parametrize("name,method,orig,bad", TT_MUTANTS, ids=[m[0] for m in TT_MUTANTS])
def test_planted_two_term_mistake_is_caught(name, method, orig, bad, monkeypatch):
    owner, meth = (O, method[3:]) if method.startswith("fn:") else (O.Model, method)
    src = textwrap.dedent(inspect.getsource(getattr(owner, meth)))
    assert src.count(orig) == 1, f"mutation site not unique: {name}"
    ns = dict(vars(O))
    exec(compile(src.replace(orig, bad), f"<mutant {name}>", "exec"), ns)
    monkeypatch.setattr(owner, meth, ns[meth])
    with pytest.raises(AssertionError):
        _tt_pins(O)
