"""Planted mistakes in copies of the oracle must each fail some pin.

Every mutant below is a plausible slip (dropped term, wrong sign, wrong
index, transposed operand, wrong tie rule, missing renormalisation, ...).
The mutated copy is compiled to a temporary library and run against the
whole pin battery of ``oracle_pins``; the real oracle source is untouched.
All mutants keep memory accesses in bounds.  (A wrong softmax normaliser
is not a mutant: it cancels in the renormalisation of the top-k weights.)
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

MUTANTS = [
    ("bf16_shift", "uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    ("nibble_high_first", "(q[i / 8] >> (4 * (i % 8)))", "(q[i / 8] >> (4 * (7 - i % 8)))"),
    ("dequant_no_bias", "dst[i] = s * (float)nib + b;", "dst[i] = s * (float)nib;"),
    ("dequant_bias_sign", "dst[i] = s * (float)nib + b;", "dst[i] = s * (float)nib - b;"),
    ("group_scale_index", "float s = moe_oracle_bf16_to_f32(sc[i / group]);",
     "float s = moe_oracle_bf16_to_f32(sc[0]);"),
    ("group_bias_index", "float b = moe_oracle_bf16_to_f32(bi[i / group]);",
     "float b = moe_oracle_bf16_to_f32(bi[(i / group + 1) % groups]);"),
    ("router_no_bias", "if (L->router_b) acc += (double)L->router_b[e];", ""),
    ("softplus_no_sqrt", "w[r] = 0.5 * log_softplus(logits[sel[r]]);", "w[r] = log_softplus(logits[sel[r]]);"),
    ("softplus_relu", "if (z > -30.0) return log(fmax(z, 0.0) + log1p(exp(-fabs(z))));",
     "if (z > -30.0) return log(fmax(z, 0.0) + 1e-300);"),
    ("softplus_tail_sign", "return z + log1p(-0.5 * exp(z));", "return -z + log1p(-0.5 * exp(z));"),
    ("softplus_underflows", "w[r] = 0.5 * log_softplus(logits[sel[r]]);",
     "w[r] = 0.5 * log(fmax(logits[sel[r]], 0.0) + log1p(exp(-fabs(logits[sel[r]]))));"),
    ("softplus_not_renormalised", "for (int64_t r = 0; r < k; r++) w[r] /= s;", ";"),
    ("gating_ignored", "if (L->gating == 1) sqrt_softplus_weights(lg, sel, k, ww);", ";"),
    ("weights_scale_ignored", "ww[r] *= weights_scale(L);", "ww[r] *= 1.0;"),
    ("weights_scale_no_default", "L->weights_scale == 0.0 ? 1.0 : L->weights_scale", "L->weights_scale"),
    ("weights_scale_squared", "ww[r] *= weights_scale(L);", "ww[r] *= weights_scale(L) * weights_scale(L);"),
    ("hash_ignored", "if (L->tid2eid) {", "if (0) {"),
    ("hash_table_transposed", "sel[r] = L->tid2eid[r * L->n_vocab + L->token_ids[t]];",
     "sel[r] = L->tid2eid[L->token_ids[t] * d->top_k + r];"),
    ("hash_rank_reversed", "sel[r] = L->tid2eid[r * L->n_vocab + L->token_ids[t]];",
     "sel[r] = L->tid2eid[(k - 1 - r) * L->n_vocab + L->token_ids[t]];"),
    ("hash_weights_by_rank", "for (int64_t r = 0; r < k; r++) w[r] = (exp(logits[sel[r]] - top) / norm) / chosen;",
     "for (int64_t r = 0; r < k; r++) w[r] = (exp(logits[r] - top) / norm) / chosen;"),
    ("hash_not_renormalised", "for (int64_t r = 0; r < k; r++) w[r] = (exp(logits[sel[r]] - top) / norm) / chosen;",
     "for (int64_t r = 0; r < k; r++) w[r] = exp(logits[sel[r]] - top) / norm;"),
    ("router_transposed", "L->router_w[e * d->d_model + i]", "L->router_w[i * d->n_experts + e]"),
    ("tie_upper_index", "if (!taken[e] && (best < 0 || logits[e] > logits[best])) best = e;",
     "if (!taken[e] && (best < 0 || logits[e] >= logits[best])) best = e;"),
    ("no_renormalise", "w[r] = (exp(logits[sel[r]] - mx) / z) / ps;", "w[r] = exp(logits[sel[r]] - mx) / z;"),
    ("weights_reversed", "w[r] = (exp(logits[sel[r]] - mx) / z) / ps;",
     "w[r] = (exp(logits[sel[k - 1 - r]] - mx) / z) / ps;"),
    ("margin_first", "logits[sel[k - 1]] - logits[next]", "logits[sel[0]] - logits[next]"),
    ("silu_sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("gate_reads_up", "moe_oracle_dequant_row(&L->gate, e, F, D, g, j, row);",
     "moe_oracle_dequant_row(&L->up, e, F, D, g, j, row);"),
    ("swiglu_drop_up", "h[j] = silu(gj) * uj;", "h[j] = silu(gj);"),
    ("swiglu_swapped", "h[j] = silu(gj) * uj;", "h[j] = silu(uj) * gj;"),
    ("expert_x_reversed", "for (int64_t i = 0; i < D; i++) gj += (double)row[i] * xd[i];",
     "for (int64_t i = 0; i < D; i++) gj += (double)row[i] * xd[D - 1 - i];"),
    ("down_row_offset", "moe_oracle_dequant_row(&L->down, e, D, F, g, o, row);",
     "moe_oracle_dequant_row(&L->down, e, D, F, g, (o + 1) % D, row);"),
    ("shared_down_transposed", "L->sh_down[o * Fs + j]", "L->sh_down[j * D + o]"),
    ("shared_gate_reads_up", "gj += (double)moe_oracle_bf16_to_f32(L->sh_gate[j * D + i]) * xd[i];",
     "gj += (double)moe_oracle_bf16_to_f32(L->sh_up[j * D + i]) * xd[i];"),
    ("sgate_missing", "*sgate = 1.0 / (1.0 + exp(-z));", "*sgate = 1.0;"),
    ("sgate_sign", "*sgate = 1.0 / (1.0 + exp(-z));", "*sgate = 1.0 / (1.0 + exp(z));"),
    ("combine_unweighted", "for (int64_t o = 0; o < D; o++) yr[o] += ww[r] * eo[o];",
     "for (int64_t o = 0; o < D; o++) yr[o] += eo[o];"),
    ("shared_ungated", "for (int64_t o = 0; o < D; o++) yr[o] += sg * eo[o];",
     "for (int64_t o = 0; o < D; o++) yr[o] += eo[o];"),
    ("renorm_wrong_set", "for (int64_t r = 0; r < k; r++) ps += exp(logits[sel[r]] - mx) / z;",
     "for (int64_t r = 0; r < k; r++) ps += exp(logits[r] - mx) / z;"),
    ("rms_sum_not_mean", "1.0 / sqrt(ss / (double)n + eps)", "1.0 / sqrt(ss + eps)"),
    ("rms_no_eps", "1.0 / sqrt(ss / (double)n + eps)", "1.0 / sqrt(ss / (double)n)"),
    ("rms_no_sqrt", "1.0 / sqrt(ss / (double)n + eps)", "1.0 / (ss / (double)n + eps)"),
    ("rms_weight_shifted", "* scale * (double)weight[i]);", "* scale * (double)weight[(i + 1) % n]);"),
    ("bf16_round_down", "r = ldexp(rint(ldexp(m, 8)), e - 8);", "r = ldexp(floor(ldexp(m, 8)), e - 8);"),
    ("residual_missing", "y[n * D + o] += (double)moe_oracle_bf16_to_f32(h[t * D + o]);", ";"),
    ("residual_of_normed", "y[n * D + o] += (double)moe_oracle_bf16_to_f32(h[t * D + o]);",
     "y[n * D + o] += (double)moe_oracle_bf16_to_f32(xr[t * D + o]);"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,needle,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, needle, repl):
    n = source.count(needle)
    assert n >= 1, f"mutation site for {name} not found in the oracle source"
    src = os.path.join(tmp_path, "moe_oracle.c")
    with open(src, "w") as f:
        f.write(source.replace(needle, repl))
    lib = os.path.join(tmp_path, f"libmut_{name}.so")
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-I", os.path.dirname(oracle.SRC), "-o", lib, src,
                           "-lm", "-lpthread"])
    O = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(O)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(exc).__name__))
    assert failed, f"mutant {name} passed every pin"
