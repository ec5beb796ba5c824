"""The oracle's pins reject plausible mistakes (CPU only).

Each case below plants one mistake in a copy of ``oracle/moe_oracle.c`` -- a
dropped term, a wrong sign, index, order, rounding or tie rule, a transposed
operand -- builds it with the oracle's own flags and runs the pin suite
(``test_oracle_pins.py``) against that build.  The pins must fail for every
mutant, and pass for an unmodified copy built the same way.  The mistakes are
planted in the oracle only, on the CPU; nothing here touches the GPU library.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared"]

# (name, text in moe_oracle.c, replacement): the text must occur exactly once
MUTANTS = [
    # c1 top-k and gate weights
    ("tie_break_highest_id",
     "if (best < 0 || score[e] > score[best]) best = e;",
     "if (best < 0 || score[e] >= score[best]) best = e;"),
    ("bias_dropped",
     "score[e] = orc_load(logits, t * E + e, logits_bf16) + b;",
     "score[e] = orc_load(logits, t * E + e, logits_bf16) + 0.0f * b;"),
    ("softmax_sign",
     "v[j] = exp(s - (double)chosen[0]);",
     "v[j] = exp((double)chosen[0] - s);"),
    ("sigmoid_not_normalised",
     "for (int j = 0; j < k; ++j) topk_w[t * k + j] = v[j] / acc;",
     "for (int j = 0; j < k; ++j) topk_w[t * k + j] = gating ? v[j] : v[j] / acc;"),
    ("sigmoid_sign",
     "v[j] = 1.0 / (1.0 + exp(-s));",
     "v[j] = 1.0 / (1.0 + exp(s));"),
    # c2 replica map
    ("eplb_global_position",
     "int64_t b = t % LB;",
     "int64_t b = t;"),
    ("eplb_replica_off_by_one",
     "replica_slots[replica_offsets[e] + (int)(b % n)]",
     "replica_slots[replica_offsets[e] + (int)((b + 1) % n)]"),
    # c3 token quantization
    ("quant_scale_128",
     "float s = amax / 127.0f;\n  *scale = s;",
     "float s = amax / 128.0f;\n  *scale = s;"),
    ("quant_round_half_away",
     "float r = rintf(orc_load(x, row * H + h, is_bf16) / s);",
     "float r = roundf(orc_load(x, row * H + h, is_bf16) / s);"),
    ("quant_multiply_by_reciprocal",
     "float r = rintf(orc_load(x, row * H + h, is_bf16) / s);",
     "float r = rintf(orc_load(x, row * H + h, is_bf16) * (127.0f / amax));"),
    ("quant_clamp_128",
     "if (r < -127.0f) r = -127.0f;",
     "if (r < -128.0f) r = -128.0f;"),
    # c4 dispatch layout and messages
    ("region_order_slot_major",
     "    for (int64_t b = 0; b < LB; ++b)\n      for (int64_t j = 0; j < k; ++j) {\n        int64_t t = s * LB + b;",
     "    for (int64_t j = 0; j < k; ++j)\n      for (int64_t b = 0; b < LB; ++b) {\n        int64_t t = s * LB + b;"),
    ("meta_offset_inclusive",
     "m[1] = (int32_t)off;",
     "m[1] = (int32_t)(off + count[d * S + s]);"),
    ("slot_local_counts_itself",
     "for (int64_t p2 = 0; p2 < p; ++p2) n += (slot_partition[p2] == slot_partition[p]);",
     "for (int64_t p2 = 0; p2 <= p; ++p2) n += (slot_partition[p2] == slot_partition[p]);"),
    ("trailer_route_slot_reversed",
     "row[H + 12] = (uint8_t)j;",
     "row[H + 12] = (uint8_t)(k - 1 - j);"),
    ("capacity_unchecked",
     "if (r >= cap) status = ORC_ECAPACITY;",
     "if (r > cap) status = ORC_ECAPACITY;"),
    # c5 / c6 expert
    ("gate_up_interleaved_rows",
     "const int8_t *wg = w_gateup + c * H, *wu = w_gateup + (I + c) * H;",
     "const int8_t *wg = w_gateup + 2 * c * H, *wu = w_gateup + (2 * c + 1) * H;"),
    ("silu_on_up",
     "float e = (float)exp(-(double)g);\n      h[c] = (g / (1.0f + e)) * u;",
     "float e = (float)exp(-(double)u);\n      h[c] = (u / (1.0f + e)) * g;"),
    ("gate_scale_of_up",
     "float g = ((float)ag * s_rows[r]) * s_gateup[c];",
     "float g = ((float)ag * s_rows[r]) * s_gateup[I + c];"),
    ("requant_signed_max",
     "float a = fabsf(h[c]);",
     "float a = h[c];"),
    ("down_scale_dropped",
     "y[r * H + c] = orc_f32_to_bf16(((float)a * s) * s_down[c]);",
     "y[r * H + c] = orc_f32_to_bf16((float)a * s_down[c]);"),
    ("down_weight_transposed",
     "const int8_t *wd = w_down + c * I;\n      for (int64_t x = 0; x < I; ++x) a += (int32_t)hqr[x] * (int32_t)wd[x];",
     "const int8_t *wd = w_down + c;\n      for (int64_t x = 0; x < I; ++x) a += (int32_t)hqr[x] * (int32_t)wd[x * H];"),
    # c7 combine
    ("combine_weights_reversed",
     "float prod = w[t * k + j] * v;",
     "float prod = w[t * k + (k - 1 - j)] * v;"),
    ("combine_scale_dropped",
     "v = (float)((const int8_t *)row)[c] * sc;",
     "v = (float)((const int8_t *)row)[c];"),
    ("combine_block_scale_index",
     "const int64_t so = scale_offset + (mode == 2 ? 4 * (c / scale_block) : 0);",
     "const int64_t so = scale_offset + (mode == 2 ? 4 * (c % scale_block) : 0);"),
    # c6' INT8 returns
    ("block_quant_scale_slot",
     "scale[r * nblk + b] = sb;",
     "scale[r * nblk + (nblk - 1 - b)] = sb;"),
    # c2' EPLB plan
    ("plan_split_compounded",
     "#define SIM(t, e, extra) ((double)token_count[(t) * E + (e)] / (double)(copies[e] + (extra)))",
     "#define SIM(t, e, extra) ((double)token_count[(t) * E + (e)] / (double)(1 << (copies[e] + (extra) - 1)))"),
    ("plan_placement_tie_highest",
     "if (target < 0 || load[d] < load[target]) target = d;",
     "if (target < 0 || load[d] <= load[target]) target = d;"),
    ("plan_replica_order_ascending",
     "while (m > 0 && total[order[m - 1]] < total[v]) {",
     "while (m > 0 && total[order[m - 1]] > total[v]) {"),
    # c4' static sizes
    ("static_buffer_max",
     "int64_t m = topk < experts_per_die ? topk : experts_per_die;",
     "int64_t m = topk > experts_per_die ? topk : experts_per_die;"),
    # bf16 conversions
    ("bf16_round_toward_zero",
     "  u += 0x7fffu + lsb;\n  return (uint16_t)(u >> 16);",
     "  (void)lsb;\n  return (uint16_t)(u >> 16);"),
    ("bf16_round_half_up",
     "  u += 0x7fffu + lsb;",
     "  u += 0x8000u + 0u * lsb;"),
    # more of c1-c7
    ("topk_slots_reversed",
     "      topk_ids[t * k + j] = best;\n      chosen[j] = score[best];",
     "      topk_ids[t * k + (k - 1 - j)] = best;\n      chosen[j] = score[best];"),
    ("quant_amax_skips_last",
     "  for (int h = 0; h < H; ++h) {\n    float a = fabsf(orc_load(x, row * H + h, is_bf16));",
     "  for (int h = 0; h < H - 1; ++h) {\n    float a = fabsf(orc_load(x, row * H + h, is_bf16));"),
    ("trailer_batch_slot_global",
     "int32_t s = (int32_t)(t / LB), b = (int32_t)(t % LB);",
     "int32_t s = (int32_t)(t / LB), b = (int32_t)t;"),
    ("trailer_event_high_half",
     "uint16_t ev = (uint16_t)(event_id & 0xffffu);",
     "uint16_t ev = (uint16_t)(event_id >> 16);"),
    ("ret_rows_not_stable",
     "      int64_t rr = slot_offset[p] + fill[p]++;",
     "      int64_t rr = slot_offset[p + 1] - 1 - fill[p]++;"),
    ("block_quant_last_block_short",
     "const int32_t c0 = b * block, c1 = c0 + block < H ? c0 + block : H;",
     "const int32_t c0 = b * block, c1 = c0 + block < H ? c0 + block : H - 1;"),
    ("requant_scale_of_token",
     "    float s = amax / 127.0f;\n    hs[r] = s;",
     "    float s = amax / 127.0f;\n    hs[r] = s_rows[r];"),
    ("combine_fp32_out_truncated",
     "        ((float *)out)[t * H + c] = acc;",
     "        ((float *)out)[t * H + c] = orc_bf16_to_f32(orc_f32_to_bf16(acc));"),
    ("plan_candidate_tie_highest",
     "        if (SIM(t, e, 0) > SIM(t, best, 0)) best = e;",
     "        if (SIM(t, e, 0) >= SIM(t, best, 0)) best = e;"),
    ("plan_primary_share_undivided",
     "    load[d] += total[e] / (double)copies[e];\n    slot_partition[e] = d;",
     "    load[d] += total[e];\n    slot_partition[e] = d;"),
    ("plan_all_experts_candidates",
     "      if (!cand[c]) continue;",
     "      (void)cand;"),
    # gate logits
    ("router_single_precision",
     "      double acc = 0.0;\n      for (int64_t h = 0; h < H; ++h)",
     "      float acc = 0.0f;\n      for (int64_t h = 0; h < H; ++h)"),
    ("router_weight_transposed",
     "acc += (double)orc_bf16_to_f32(x[t * H + h]) * (double)orc_bf16_to_f32(w[e * H + h]);",
     "acc += (double)orc_bf16_to_f32(x[t * H + h]) * (double)orc_bf16_to_f32(w[h * E + e]);"),
]


def _build(src_text: str, out_dir: str) -> str:
    c = os.path.join(out_dir, "moe_oracle.c")
    with open(c, "w") as f:
        f.write(src_text)
    lib = os.path.join(out_dir, "libmoe_oracle.so")
    subprocess.run(["gcc", *CFLAGS, "-o", lib, c, "-lm"], check=True, capture_output=True)
    return lib


def _pins_pass(lib: str) -> bool:
    env = dict(os.environ, MOE_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, timeout=600)
    return r.returncode == 0


@pytest.fixture(scope="module")
def verdicts():
    with open(SRC) as f:
        base = f.read()
    work = tempfile.mkdtemp(prefix="oracle_mutants_")
    try:
        jobs = {"unmodified": base}
        for name, old, new in MUTANTS:
            assert base.count(old) == 1, f"{name}: the text to mutate must occur once"
            jobs[name] = base.replace(old, new)

        def run(item):
            name, text = item
            d = os.path.join(work, name)
            os.makedirs(d)
            return name, _pins_pass(_build(text, d))

        with concurrent.futures.ThreadPoolExecutor(4) as ex:
            return dict(ex.map(run, jobs.items()))
    finally:
        shutil.rmtree(work, ignore_errors=True)


def test_unmodified_copy_passes_the_pins(verdicts):
    assert verdicts["unmodified"], "the pins fail on an unmodified build: the harness is broken"


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_reject_mutant(verdicts, name):
    assert not verdicts[name], f"no pin catches the planted mistake '{name}'"
