"""Planted mistakes in the CPU oracle, for test_oracle_mutants.py.

Each entry names one oracle function and a one-place edit of its source text
that a plausible slip would produce: a dropped term, a wrong sign, an
off-by-one, another rounding mode, a wrong index or a transposed operand. The
edit must match the source exactly once, so a change to the oracle that moves
the target makes the test fail loudly rather than test nothing. ``apply``
compiles the edited function into the oracle module's namespace (every other
oracle function then calls the planted version) and rebinds the package-level
name where the package re-exports it. Nothing is written to disk; only a pytest process started with
AR_ORACLE_MUTANT set loads this (through conftest.py).
"""
import inspect

MUTANTS = {
    # bf16 rounding: truncation instead of round-to-nearest-even
    "bf16_truncate": ("bf16", "upper = upper + up.astype(np.uint32)", "upper = upper"),
    # group min/max over strided instead of contiguous channels
    "strided_groups": ("group_minmax",
                       "Wg = np.asarray(W, dtype=F32).reshape(N, K // g, g)",
                       "Wg = np.asarray(W, dtype=F32).reshape(N, g, K // g).transpose(0, 2, 1)"),
    # scale and zero-point
    "zp_sign": ("qparams", "np.rint(-lo / s)", "np.rint(lo / s)"),
    "scale_off_by_one": ("qparams", "s = (hi - lo) / maxq", "s = (hi - lo) / (maxq + F32(1.0))"),
    "range_not_anchored_at_zero": ("qparams", "lo = np.minimum(alpha * wmin, F32(0.0))",
                                   "lo = alpha * wmin"),
    "sym_scale_halved": ("qparams", "s = (F32(2.0) * amax) / maxq", "s = amax / maxq"),
    "sym_zero_point": ("qparams", "F32(2 ** (bits - 1))", "F32(2 ** (bits - 1) - 1)"),
    "hi_not_anchored": ("qparams", "hi = np.maximum(beta * wmax, F32(0.0))", "hi = beta * wmax"),
    # fake-quantization
    "round_half_up": ("fake_quant", "r = np.rint(u)", "r = np.floor(u + F32(0.5))"),
    "offset_after_rounding": ("fake_quant", "    u = t + V\n    r = np.rint(u)\n",
                              "    u = t\n    r = np.rint(u) + V\n"),
    "mask_from_clamped_code": ("fake_quant", "m = (c >= 0) & (c <= maxq)",
                               "m = (q >= 0) & (q <= maxq)"),
    "dequant_drops_zero_point": ("fake_quant", "what = s_e * (q - zp_e)", "what = s_e * q"),
    # loss and weight gradient
    "grad_factor_half": ("forward_backward", "G = (2.0 / (T * Nn))", "G = (1.0 / (T * Nn))"),
    "loss_mean_over_tokens_only": ("forward_backward",
                                   "return loss_sum / (T * Nn), G, loss_sum",
                                   "return loss_sum / T, G, loss_sum"),
    "residual_sign": ("forward_backward", "R = Yp - np.asarray(Yb, F64)",
                      "R = np.asarray(Yb, F64) - Yp"),
    "grad_transposed": ("forward_backward", "(dY.T @ X64)", "(X64.T @ dY)"),
    "dY_not_rounded": ("forward_backward",
                       "dY = bf16(R.astype(F32)).astype(F64) if amp else R", "dY = R"),
    # straight-through gradients
    "ste_no_mask": ("ste_grads", "gV = G64 * fq.s_e.astype(F64) * m", "gV = G64 * fq.s_e.astype(F64)"),
    "ste_scale_term_drops_t": ("ste_grads", "(qz - m * fq.t.astype(F64))", "qz"),
    "ste_zero_point_sign": ("ste_grads", "B = -s64 * Bsum", "B = s64 * Bsum"),
    "ste_dlo_drops_zp_term": ("ste_grads", "dlo = -D / maxq - B / s64", "dlo = -D / maxq"),
    "ste_sym_routed_wrong": ("ste_grads", "        ga = np.where(to_alpha, damax",
                             "        to_alpha = ~to_alpha\n        ga = np.where(to_alpha, damax"),
    "sym_tie_to_alpha": ("ste_grads", "np.asarray(wmin, F32)) > \\", "np.asarray(wmin, F32)) >= \\"),
    # SignSGD
    "sgn_of_zero_is_one": ("sgn", "(x > 0).astype(F32)", "(x >= 0).astype(F32)"),
    "offset_clamp_too_wide": ("signsgd_update", "F32(-0.5), F32(0.5)", "F32(-1.0), F32(1.0)"),
    "minmax_lr_ignored": ("signsgd_update", "mlr = F32(cfg.mlr)", "mlr = F32(cfg.lr)"),
    "offset_step_ascends": ("signsgd_update", "np.asarray(V, F32) - lr * sgn(gV)",
                            "np.asarray(V, F32) + lr * sgn(gV)"),
    # the loop's best-loss snapshot
    "snapshot_after_update": ("tune_linear", "            best = (V.copy(), alpha.copy(), beta.copy())",
                              "            best = (r.V.copy(), r.alpha.copy(), r.beta.copy())"),
    "snapshot_on_ties": ("tune_linear", "if r.loss < best_loss:", "if r.loss <= best_loss:"),
    "last_state_kept": ("tune_linear", "        V, alpha, beta = best\n", "        pass\n"),
    "one_minibatch_only": ("tune_linear", "Xb, Yb = minibatch(i % nb)", "Xb, Yb = minibatch(0)"),
    # Gram form
    "gram_cross_term_sign": ("forward_backward_gram", "2.0 * np.sum(D * st.Cn)",
                             "-2.0 * np.sum(D * st.Cn)"),
    "gram_drops_e2": ("forward_backward_gram", " + st.e2)", ")"),
    # MSE initial scale
    "mse_grid_skips_one": ("mse_grid_points", "p = F32(1.0 - j / cfg.mse_grid)",
                           "p = F32(1.0 - (j + 1) / cfg.mse_grid)"),
    "mse_picks_largest_error": ("mse_shrink", "best = np.argmin(np.stack(errs), axis=0)",
                                "best = np.argmax(np.stack(errs), axis=0)"),
    # packing
    "pack_drops_straddling_bits": ("_pack_axis0",
                                   "            out[w + 1] |= v[k] >> np.uint64(32 - off)\n",
                                   "            pass\n"),
    "pack_field_order_reversed": ("_pack_axis0", "out[w] |= (v[k] << np.uint64(off))",
                                  "out[w] |= (v[L - 1 - k] << np.uint64(off))"),
    "unpack_drops_straddling_bits": ("_unpack_axis0",
                                     "            val |= w64[w + 1] << np.uint64(32 - off)\n",
                                     "            pass\n"),
    # packed-format dequantization and product
    "dequant_sym_zero_point": ("dequantize", "zp = np.full((N, K // g), 2 ** (bits - 1), np.int64)",
                               "zp = np.full((N, K // g), 2 ** (bits - 1) - 1, np.int64)"),
    "dequant_ignores_zero_points": ("dequantize", "(codes.astype(F32) - zp_e)", "codes.astype(F32)"),
    "dequant_product_not_bf16": ("dequant_matmul", "bf16(what).astype(F64).T", "what.astype(F64).T"),
    # Gram statistics and initial clip factors
    "gram_residual_sign": ("gram_stats", "E = X64 @ np.asarray(W, F64).T - np.asarray(Yb, F64)",
                           "E = np.asarray(Yb, F64) - X64 @ np.asarray(W, F64).T"),
    "init_clip_ignores_shrink": ("init_clip", "a = np.full((N, Gn), F32(cfg.minmax_shrink), F32)",
                                 "a = np.full((N, Gn), F32(1.0), F32)"),
    # per-layer configuration
    "layer_pattern_prefix_match": ("_whole_name_match", "re.compile(key).fullmatch(name)",
                                   "re.compile(key).match(name)"),
    "layer_exact_key_defaults_outside_set": ("resolve_layer_config",
                                             "return _merge(by_key[name], fallback)",
                                             "return _merge(by_key[name], tuple(defaults))"),
    "layer_plain_keys_as_patterns": ("_whole_name_match",
                                     "    if REGEX_SPECIAL_CHARS.isdisjoint(key):\n        return False\n",
                                     ""),
    "fused_configs_not_compared": ("resolve_fused_config", "if len(resolved) != 1:", "if False:"),
    "fused_experts_not_collected": ("resolve_fused_config",
                                    "members = [key for key, _ in rules if key.startswith(layer_name)]",
                                    "members = []"),
    # block forward (oracle/block_ref.py)
    "rmsnorm_sum_not_mean": ("block_ref.rmsnorm", "np.mean(x.astype(F64) ** 2", "np.sum(x.astype(F64) ** 2"),
    "rmsnorm_weight_dropped": ("block_ref.rmsnorm", " * np.asarray(w, F32))", ")"),
    "rope_rotation_sign": ("block_ref.rope", "(a * c).astype(F32) - (b * s).astype(F32)",
                           "(a * c).astype(F32) + (b * s).astype(F32)"),
    "rope_global_positions": ("block_ref.rope", "pos = np.arange(M) % seqlen", "pos = np.arange(M)"),
    "rope_frequency_exponent": ("block_ref.rope_table", "inv = theta ** (-2.0 * j / Dh)",
                                "inv = theta ** (-1.0 * j / Dh)"),
    "attention_not_causal": ("block_ref.attention", "S[mask] = -np.inf", "pass"),
    "attention_scale": ("block_ref.attention", "/ np.sqrt(Dh)", "/ Dh"),
    "attention_keys_of_first_sequence": ("block_ref.attention", "k[s0:s0 + seqlen, sl].T",
                                         "k[0:seqlen, sl].T"),
    "silu_sign": ("block_ref.silu_mul", "np.exp(-g)", "np.exp(g)"),
    "attention_residual_dropped": ("block_ref.block_forward", 't["h1"] = add(t["h"], t["o_proj"])',
                                   't["h1"] = t["o_proj"]'),
    "mlp_norm_of_block_input": ("block_ref.block_forward", 't["m"] = rmsnorm(t["h1"], norms[1]',
                                't["m"] = rmsnorm(t["h"], norms[1]'),
    "tuning_ignores_quantized_inputs": ("block_ref.tune_block",
                                        "X = q[LINEAR_INPUT[name]] if quanted_input else fp[LINEAR_INPUT[name]]",
                                        "X = fp[LINEAR_INPUT[name]]"),
    "tuning_targets_quantized_pipeline": ("block_ref.tune_block", "Y = fp[name]", "Y = q[name]"),
    "tuned_linear_not_substituted": ("block_ref.tune_block", "Wq[name] = b16(res.what)", "pass"),
}


def target(name: str):
    """(module, function name) of a mutant: "block_ref.f" lives in
    oracle/block_ref.py, a bare name in oracle/autoround_ref.py."""
    import importlib
    fn = MUTANTS[name][0]
    mod, _, fname = fn.rpartition(".")
    return importlib.import_module("oracle." + (mod or "autoround_ref")), fname


def apply(name: str) -> None:
    import oracle
    fn, old, new = MUTANTS[name]
    mod, fname = target(name)
    src = inspect.getsource(getattr(mod, fname))
    n = src.count(old)
    if n != 1:
        raise RuntimeError(f"mutant {name}: target occurs {n} times in {fn}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    if mod.__name__ == "oracle.autoround_ref" and hasattr(oracle, fname):
        setattr(oracle, fname, mod.__dict__[fname])
