"""Planted mistakes in the CPU reference must be caught by its pins.

Each mutation is a textual edit of a copy of oracle/oracle.c (a dropped term, a
wrong sign, index or operand), built with gcc into a temporary library.  The pin
checks of oracle_pins.py run against that build in a child process; at least one
must fail.  The committed reference is never modified.  CPU only.
"""
import concurrent.futures
import json
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "rmsnorm_no_eps": ("ss / (float)n + eps", "ss / (float)n"),
    "rmsnorm_no_mean": ("ss / (float)n + eps", "ss + eps"),
    "rmsnorm_no_gamma": ("v[i] * inv * orc_bf16_to_f32(gamma[i])", "v[i] * inv"),
    "matvec_transposed": ("acc += orc_bf16_to_f32(w[c]) * x[c]",
                          "acc += orc_bf16_to_f32(W[(int64_t)c * rows + r]) * x[c]"),
    "rope_sign": ("v[i] = a * c - b * s", "v[i] = a * c + b * s"),
    "rope_frequency": ("-2.0 * (double)i / (double)head_dim", "-1.0 * (double)i / (double)head_dim"),
    "rope_fp32_angle": ("const double ang = (double)pos * theta;",
                        "const double ang = (double)((float)pos * (float)theta);"),
    "rope_position_off_by_one": ("orc_rope(hd, d->rope_base, pos, k + g * hd)",
                                 "orc_rope(hd, d->rope_base, pos + 1, k + g * hd)"),
    "attn_no_scale": ("s[i] = dot * scale;", "s[i] = dot;"),
    "attn_gqa_modulo": ("const int32_t g = j / group;", "const int32_t g = j % d->n_kv_heads;"),
    "attn_excludes_new_token": ("const int64_t n = pos + 1 - t0;", "const int64_t n = pos - t0 > 0 ? pos - t0 : 1;"),
    "attn_window_one_longer": ("? pos + 1 - d->attn_window : 0;", "? pos - d->attn_window : 0;"),
    "attn_window_ignored": ("const int64_t t0 = (d->attn_window > 0", "const int64_t t0 = 0 * (d->attn_window > 0"),
    "step_window_on_every_layer": ("(d->full_every < 1 || (l + 1) % d->full_every != 0)", "(1)"),
    "attn_no_normalise": ("for (int64_t t = 0; t < n; ++t) s[t] /= sum;", ""),
    "attn_page_index": ("const int32_t page = page_row[t / P], tt = (int32_t)(t % P);\n      for (int32_t e = 0; e < hd; ++e)\n        oj[e]",
                        "const int32_t page = page_row[(t / P) % 2], tt = (int32_t)(t % P);\n      for (int32_t e = 0; e < hd; ++e)\n        oj[e]"),
    "kv_v_layout_as_k": ("base + (int64_t)dim * P + t", "base + (int64_t)t * D + dim"),
    "kv_write_wrong_slot": ("const int32_t t = (int32_t)(pos % d->page_size);",
                            "const int32_t t = (int32_t)((pos + 1) % d->page_size);"),
    "bf16_truncate": ("return (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);",
                      "return (uint16_t)(v.u >> 16);"),
    "topk_tie_high_index": ("logits[e] > logits[best]", "logits[e] >= logits[best]"),
    "topk_no_renormalise": ("for (int32_t j = 0; j < k; ++j) w[j] /= sum;", ""),
    "swiglu_on_up": ("const float g = gu[i];", "const float g = gu[inter + i];"),
    "swiglu_no_up": ("gu[i] = silu * gu[inter + i];", "gu[i] = silu;"),
    "moe_unweighted": ("m[i] += w[j] * y[i];", "m[i] += y[i];"),
    "residual_dropped": ("hb[i] = hb[i] + a[i] + m[i];", "hb[i] = a[i] + m[i];"),
    "attention_branch_dropped": ("hb[i] = hb[i] + a[i] + m[i];", "hb[i] = hb[i] + m[i];"),
    "oproj_reads_q": ("orc_matvec_bf16(H, nq * hd, w_o, o, a);", "orc_matvec_bf16(H, nq * hd, w_o, q, a);"),
    "router_reads_h": ("orc_matvec_bf16(E, H, w_router, x, r);", "orc_matvec_bf16(E, H, w_router, hb, r);"),
    "layer_gamma_fixed": ("norm + l * H, w_qkv", "norm, w_qkv"),
    "final_gamma_first": ("orc_lm_head(d, batch, h, norm + (int64_t)d->n_layers * H",
                          "orc_lm_head(d, batch, h, norm"),
    "layer_weights_fixed": ("w_o + l * H * nq * hd,", "w_o,"),
    "qkv_q_no_rope": ("for (int32_t j = 0; j < nq; ++j) orc_rope(hd, d->rope_base, pos, y + j * hd);", ""),
    "qkv_q_pos_plus_one": ("orc_rope(hd, d->rope_base, pos, y + j * hd)",
                           "orc_rope(hd, d->rope_base, pos + 1, y + j * hd)"),
    "qkv_rope_on_v": ("memcpy(q, y, sizeof(float) * (size_t)nq * hd);",
                      "for (int32_t g = 0; g < nkv; ++g) orc_rope(hd, d->rope_base, pos, v + g * hd);\n"
                      "  memcpy(q, y, sizeof(float) * (size_t)nq * hd);"),
    "qkv_v_from_k_rows": ("float* v = y + (nq + nkv) * hd;", "float* v = y + nq * hd;"),
}

RUNNER = r"""
import json, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
oracle._lib = oracle.load({so!r})
import oracle_pins
failed = []
for check in oracle_pins.ALL_CHECKS:
    try:
        check()
    except Exception as exc:  # AssertionError or a crash-free error
        failed.append(check.__name__)
        break
print(json.dumps(failed))
"""


def _run_mutation(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    if src.count(old) != 1:
        return name, "pattern-not-unique", []
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "oracle.c")
        with open(c, "w") as f:
            f.write(src.replace(old, new))
        import shutil
        shutil.copy(os.path.join(ROOT, "oracle", "oracle.h"), tmp)
        so = os.path.join(tmp, "liboracle_mut.so")
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", c, "-o", so, "-lm"],
                       check=True, capture_output=True)
        code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), so=so)
        env = dict(os.environ, OMP_NUM_THREADS="2")
        p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                           timeout=300)
        if p.returncode != 0:
            return name, "crashed", []          # a crash is also a caught mistake
        return name, "ran", json.loads(p.stdout.strip().splitlines()[-1])


@pytest.fixture(scope="module")
def mutation_results():
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        return dict((n, (s, f)) for n, s, f in ex.map(_run_mutation, sorted(MUTATIONS)))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, mutation_results):
    status, failed = mutation_results[name]
    assert status != "pattern-not-unique", f"mutation {name} no longer matches oracle.c"
    assert status == "crashed" or failed, f"planted mistake {name} passed every pin"
