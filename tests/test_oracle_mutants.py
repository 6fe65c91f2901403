"""The oracle's pins catch planted mistakes (CPU only).

Each case copies the oracle's C source, plants one plausible mistake (a
rounding instead of a truncating conversion, a dropped scale, a wrong index, a
sign flip, a missing rescale, ...), builds it with the oracle's own flags into
a temporary directory and runs a compact battery of the pins from
test_oracle_quant.py and test_oracle_decode.py against it.  Every mutant must
fail at least one pin; the real oracle must pass them all.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from cases import build, small
from test_oracle_quant import F, exact_quant
from test_oracle_decode import _decimal_reference

MUTANTS = {
    "round_not_truncate": ("return (int8_t)(int)v;", "return (int8_t)(int)lrintf(v);"),
    "no_guard": ("if (a < ORC_TINY) a = 1.0f;", ""),
    "scale_divides": ("*scale_out = a * ORC_INV127;", "*scale_out = a / 127.0f;"),
    "drop_qsc": ("s = s + (float)orc_block_dot(qi, k, blk) * qsc[blk];",
                 "s = s + (float)orc_block_dot(qi, k, blk);"),
    "drop_ks": ("return (s * ks) * scale;", "return s * scale;"),
    "no_acc_rescale": ("    for (int i = 0; i < st->hd; ++i) st->acc[i] = st->acc[i] * m;\n", ""),
    "no_sum_rescale": ("    st->S = st->S * m;\n", ""),
    "exp_sign": ("w = expf(s - st->M);", "w = expf(st->M - s);"),
    "drop_vs": ("float f = w * vs;", "float f = w;"),
    "no_final_divide": ("for (int i = 0; i < hd; ++i) out[i] = acc[i] / st.S;",
                        "for (int i = 0; i < hd; ++i) out[i] = acc[i];"),
    "kv_head_modulo": ("int G = a->n_q / a->n_kv, kh = h / G, nb = a->hd / ORC_QBLOCK;\n    for (int t = t0;",
                       "int G = a->n_q / a->n_kv, kh = h % a->n_kv, nb = a->hd / ORC_QBLOCK; (void)G;\n"
                       "    for (int t = t0;"),
    "row_index": ("(size_t)(t % a->kv_bs);", "(size_t)((t + 1) % a->kv_bs);"),
    "transposed_dot": ("d += (int32_t)qi[blk * ORC_QBLOCK + i] * (int32_t)k[blk * ORC_QBLOCK + i];",
                       "d += (int32_t)qi[blk * ORC_QBLOCK + i] * (int32_t)k[i * 4 % 128 + blk];"),
    "merge_unweighted": ("St = St + Sp[p] * e;", "St = St + Sp[p];"),
    "max_hysteresis": ("if (s > st->M) {", "if (s > st->M - 0.5f) {"),
    "max_not_updated": ("    st->M = s;\n", ""),
}


def battery():
    """Run the pins; return the list of names that failed."""
    failed = []

    def check(name, ok):
        if not ok:
            failed.append(name)

    rng = np.random.default_rng(1)
    bad = False
    for _ in range(30):
        x = rng.standard_normal(32).astype(np.float32)
        x[0] = 0.5 * np.abs(x).max()
        qv, sc = oracle.quantize(x)
        want_q, want_sc = exact_quant(x)
        bad |= list(qv.astype(int)) != want_q or F(sc) != want_sc
    xt = np.full(32, 5e-7, np.float32)
    qv, sc = oracle.quantize(xt)
    bad |= list(qv.astype(int)) != exact_quant(xt)[0] or F(sc) != exact_quant(xt)[1]
    check("quant_exact", not bad)

    for w in (small("long_gqa", n_q=8, n_kv=2, seq_len=300),
              small("ragged", batch=3, n_q=4, n_kv=2, seq_len=200)):
        c = build(w)
        ref = oracle.three_pass_f64(c.q, c.cache, c.table, c.lens, c.scale)
        sp32 = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
        check("c1_fp32", np.all(np.isfinite(sp32)) and np.abs(sp32 - ref).max() <= 2e-4)
        sp64 = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, use_f64=True)
        check("c1_fp64", np.abs(sp64 - ref).max() <= 1e-6 * np.abs(ref).max())
        split = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, part_tokens=64)
        check("split", np.all(np.isfinite(split)) and np.abs(split - ref).max() <= 2e-4)
        dots = oracle.block_dots(c.q, c.cache, c.table, c.lens)
        qi, _ = oracle.quantize_q(c.q)
        kk, _, _, _ = oracle.gather_rows(c.cache, c.table, 0, 1, int(c.lens[0]))
        want = np.einsum("tbi,bi->tb", kk.astype(np.int64).reshape(len(kk), -1, 32),
                         qi[0, w.group].astype(np.int64).reshape(-1, 32))
        check("dots", np.array_equal(dots[0, w.group, :len(kk)], want))

    w = small("long_gqa", n_q=4, n_kv=2, seq_len=200)
    c = build(w)
    out, (sc_t, m_t, s_t, w_t) = oracle.decode_trace(c.q, c.cache, c.table, c.lens, c.scale, 0, 1)
    total = np.exp(sc_t.astype(np.float64) - float(m_t[-1])).sum()
    check("c3", len(sc_t) == 200 and np.all(np.diff(m_t.astype(np.float64)) >= 0)
          and abs(total / float(s_t[-1]) - 1.0) <= 200 * 2.0 ** -23)

    w = workloads_tiny = small("gqa_batch", batch=2, n_q=4, n_kv=2, seq_len=1)
    c = build(workloads_tiny)
    out = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    _, v, _, vs = oracle.gather_rows(c.cache, c.table, 1, 1, 1)
    check("c2", np.array_equal(out[1, 3], v[0].astype(np.float32) * np.float32(vs[0])))

    import workloads
    w = workloads.Workload("bf", 2, 4, 2, 32, 4, 6, key=977)
    c = build(w)
    out = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    worst = max(np.abs(out[b, h] - _decimal_reference(c, b, h)).max()
                for b in range(2) for h in range(4))
    check("c6", worst <= 2e-6)
    return failed


@pytest.fixture(scope="module")
def tmpdir_mod():
    with tempfile.TemporaryDirectory() as d:
        yield d


def test_real_oracle_passes_battery():
    assert battery() == []


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, tmpdir_mod):
    src = open(obuild.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path_c = os.path.join(tmpdir_mod, f"{name}.c")
    path_so = os.path.join(tmpdir_mod, f"{name}.so")
    open(path_c, "w").write(src.replace(old, new))
    subprocess.run(["gcc"] + obuild.FLAGS + [path_c, "-o", path_so, "-lm"], check=True,
                   stderr=subprocess.DEVNULL)
    prev = oracle._use_library(path_so)
    try:
        with np.errstate(all="ignore"):
            failed = battery()
    finally:
        oracle._use_library(None)
        del prev
    assert failed, f"mutant {name} passed every pin"
