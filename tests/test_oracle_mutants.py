"""Plant plausible mistakes in copies of the oracle; the pins must catch each.

Every mutant is one exact text substitution in oracle/hikv_ref.cpp, compiled
into a temporary library.  The real oracle source is never modified.
"""
import os
import subprocess
import tempfile

import pytest

import pins
from oracle import ref

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTANTS = [
    ("drop_logit_scale", "            s[n] = d.scale * acc;", "            s[n] = acc;"),
    ("new_token_not_attended", "      *x.len = slot + 1;\n      const int L = *x.len;",
     "      *x.len = slot + 1;\n      const int L = *x.len - 1;"),
    ("tie_keeps_newer", "        return x.pos[a] < x.pos[b];\n      });",
     "        return x.pos[a] > x.pos[b];\n      });"),
    ("window_off_by_one", "(x.pos[n] > newest - W)", "(x.pos[n] >= newest - W)"),
    ("importance_from_logits", "added[n] += by_logit ? s[n] : p[n];", "added[n] += s[n];"),
    ("gqa_group_strided", "        const int h = j * d.G + g;\n        std::vector<double> qh",
     "        const int h = g * d.Hkv + j;\n        std::vector<double> qh"),
    ("stage2_smallest_channels", "if (fa != fb) return fa > fb;", "if (fa != fb) return fa < fb;"),
    ("prefill_window_in_softmax", "if ((int64_t)qp - x.pos[n] >= 0) vis.push_back(n);",
     "if ((int64_t)qp - x.pos[n] >= 0 && (window == 0 || (int64_t)qp - x.pos[n] < window)) "
     "vis.push_back(n);"),
    ("evict_highest", "if (x.imp[a] != x.imp[b]) return x.imp[a] > x.imp[b];",
     "if (x.imp[a] != x.imp[b]) return x.imp[a] < x.imp[b];"),
    ("compaction_forgets_importance", "        x.imp[w] = x.imp[n];\n", "\n"),
    ("sinks_by_slot", "prot[n] = (x.pos[n] < S)", "prot[n] = (n < S)"),
    ("stage2_approx_probs_for_output", "o[c] += p[i] * val_elem(d, x, T[i], c);",
     "o[c] += pt[T[i]] * val_elem(d, x, T[i], c);"),
    ("budget_off_by_one", "int keep_n = std::max(0, beta - n_prot);",
     "int keep_n = std::max(0, beta - n_prot - 1);"),
    ("value_rows_from_keys", "  return elem(x.v, d.dtype, (size_t)n * d.D + c);",
     "  return elem(x.k, d.dtype, (size_t)n * d.D + c);"),
    ("stage2_tokens_tie_by_higher_pos",
     "if (st[a] != st[bb]) return st[a] > st[bb];\n            return x.pos[a] < x.pos[bb];",
     "if (st[a] != st[bb]) return st[a] > st[bb];\n            return x.pos[a] > x.pos[bb];"),
    ("dual_bank_accumulates_everywhere",
     "if (pol->accumulate == HIKV_REF_ACC_RECENT && !(x.pos[n] > new_pos[b] - Wacc)) continue;", ""),
    ("dual_bank_window_off_by_one", "!(x.pos[n] > new_pos[b] - Wacc)", "!(x.pos[n] >= new_pos[b] - Wacc)"),
    ("dual_bank_window_not_capped_by_budget",
     "const int Wacc = std::min(pol->n_recent, beta - pol->n_sink);", "const int Wacc = pol->n_recent;"),
    ("dual_bank_freezes_the_window",
     "if (pol->accumulate == HIKV_REF_ACC_RECENT && !(x.pos[n] > new_pos[b] - Wacc)) continue;",
     "if (pol->accumulate == HIKV_REF_ACC_RECENT && (x.pos[n] > new_pos[b] - Wacc)) continue;"),
    ("chunks_by_slot", "std::sort(byp.begin(), byp.end(), [&](int a, int bb) { return x.pos[a] < x.pos[bb]; });",
     ""),
    ("chunks_keep_smallest", "if (pt[a] != pt[bb]) return pt[a] > pt[bb];", "if (pt[a] != pt[bb]) return pt[a] < pt[bb];"),
    ("chunks_of_r_tokens", "for (int c0 = 0; c0 < L; c0 += d.D) {", "for (int c0 = 0; c0 < L; c0 += r) {"),
    ("chunks_keep_one_more", "const int keep = std::min(r, m);", "const int keep = std::min(r + 1, m);"),
    ("logit_acc_uses_probabilities", "added[n] += by_logit ? s[n] : p[n];", "added[n] += p[n];"),
    ("logit_acc_stage2_uses_probabilities", "added[n] += by_logit ? st[n] : pt[n];", "added[n] += pt[n];"),
    ("pool_window_one_longer", "if (dp >= 0 && dp < pool)", "if (dp >= 0 && dp <= pool)"),
    ("pool_looks_backward", "if (dp >= 0 && dp < pool)", "if (dp <= 0 && dp > -pool)"),
    ("chunks_use_exact_logits", "            st[n] = d.scale * acc;\n          }\n          std::vector<double> pt = softmax(st);",
     "            st[n] = d.scale * acc;\n          }\n          std::vector<double> pt = softmax(st);\n"
     "          if (pol->stage2_v == HIKV_REF_S2V_CHUNK) {\n"
     "            for (int n = 0; n < L; ++n) {\n              double a2 = 0.0;\n"
     "              for (int c = 0; c < d.D; ++c) a2 += qh[c] * key_elem(d, x, n, c);\n"
     "              st[n] = d.scale * a2;\n            }\n            pt = softmax(st);\n          }"),
    ("blocks_evict_highest", "if (blk[a].score != blk[b].score) return blk[a].score < blk[b].score;",
     "if (blk[a].score != blk[b].score) return blk[a].score > blk[b].score;"),
    ("blocks_tie_evicts_older", "    return blk[a].id > blk[b].id;", "    return blk[a].id < blk[b].id;"),
    ("blocks_protected_by_last_token_only", "blk[k].prot = blk[k].prot || prot[n];", "blk[k].prot = prot[n];"),
    ("blocks_evict_one_too_many", "    if (live <= beta) break;", "    if (live < beta) break;"),
    ("blocks_by_slot", "const int64_t p = x.pos[n];", "const int64_t p = n;"),
    ("blocks_score_by_max", "blk[k].score += (double)x.imp[n];",
     "blk[k].score = std::max(blk[k].score, (double)x.imp[n]);"),
]


def _build(tmp, name, old, new):
    src = open(os.path.join(SRC, "hikv_ref.cpp")).read()
    assert src.count(old) >= 1, f"mutant {name}: pattern not found"
    src = src.replace(old, new, 1)
    path = os.path.join(tmp, name + ".cpp")
    with open(path, "w") as f:
        f.write(src)
    so = os.path.join(tmp, name + ".so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-fPIC", "-shared", "-I", SRC, path, "-o", so],
                   check=True)
    return so


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new):
    with tempfile.TemporaryDirectory() as tmp:
        so = _build(tmp, name, old, new)
        prev = ref.use_library(so)
        caught = None
        try:
            for check in pins.ALL:
                try:
                    check()
                except (AssertionError, ValueError, IndexError) as e:  # noqa: PERF203
                    caught = (check.__name__, repr(e)[:200])
                    break
        finally:
            ref.use_library(prev)
        assert caught is not None, f"no pin caught mutant {name}"
