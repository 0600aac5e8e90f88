"""Plant one mistake at a time in a scratch copy of the oracle and count the
oracle pin tests (tests/test_oracle_*.py, CPU) that fail on it.

Each entry is a single-point slip in oracle/ (a sign, an index, a dropped
term, a swapped pair, an off-by-one, a wrong rounding rule), applied by exact
text replacement to a copy of the committed tree (git archive HEAD) in a
temporary directory; the oracle is rebuilt there and its pins run.  Every
entry must fail at least one pin.  Usage (from the repository root):
    python tests/pins/plant_mistakes.py [substring of a mistake's name ...]
Not a pytest module: it rebuilds the oracle once per mistake (about 15 s each).
"""
import os, re, shutil, subprocess, sys, tempfile
REPO = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
WORK = tempfile.mkdtemp(prefix="plant_mistakes_")
BASE = os.path.join(WORK, "base")
M = [
 ("decay sign", "double a = exp(dtv * (double)A_h);", "double a = exp(-dtv * (double)A_h);"),
 ("dt dropped from the update", "s = a * s + dtv * xv * bv;", "s = a * s + xv * bv;"),
 ("decay after the update", "s = a * s + dtv * xv * bv;", "s = a * (s + dtv * xv * bv);"),
 ("ring entry off by one", "int32_t e = (ring_start + j) % R;", "int32_t e = (ring_start + j + 1) % R;"),
 ("ring start ignored", "int32_t e = (ring_start + j) % R;", "int32_t e = j % R;"),
 ("group map h mod G", "const int32_t g = head / p->heads_per_group;", "const int32_t g = head % G;"),
 ("x indexed by column", "((int64_t)e * H + head) * dim + r);", "((int64_t)e * H + head) * dim + (c % dim));"),
 ("B indexed by row", "((int64_t)e * G + g) * ds + c);", "((int64_t)e * G + g) * ds + (r % ds));"),
 ("dt of head 0", "double dtv = (double)dt_slot[(int64_t)e * H + head];", "double dtv = (double)dt_slot[(int64_t)e * H];"),
 ("scale divisor qmax+1", "*scale = rowmax / qmax;", "*scale = rowmax / (qmax + 1.0f);"),
 ("row max without abs", "rowmax = fmaxf(rowmax, fabsf(row[c]));", "rowmax = fmaxf(rowmax, row[c]);"),
 ("Philox counter word 0 /2", "ctr[0] = (uint32_t)(((int64_t)r * p->dstate + c) >> 2);", "ctr[0] = (uint32_t)(((int64_t)r * p->dstate + c) >> 1);"),
 ("Philox output word 0", "return o[c & 3];", "return o[0];"),
 ("Philox key words swapped", "key[0] = (uint32_t)(p->seed & 0xFFFFFFFFu);\n  key[1] = (uint32_t)(p->seed >> 32);", "key[1] = (uint32_t)(p->seed & 0xFFFFFFFFu);\n  key[0] = (uint32_t)(p->seed >> 32);"),
 ("Philox request/layer words swapped", "ctr[2] = (uint32_t)b;\n  ctr[3] = (uint32_t)l;", "ctr[2] = (uint32_t)l;\n  ctr[3] = (uint32_t)b;"),
 ("k = 0 copy without scales", "if (one_byte && scale) memcpy(scale, src_scale, (size_t)dim * sizeof(float));", ";"),
 ("pad destination not skipped", "if (s == p->pad_slot_id || d == p->pad_slot_id) continue;", "if (s == p->pad_slot_id) continue;"),
 ("active list not ended at -1", "if (b == -1) break;", "if (b == -1) continue;"),
 ("RNE ties to odd", "else out = (c % 2u == 0u) ? c : c + 1u;", "else out = (c % 2u == 1u) ? c : c + 1u;"),
 ("RNE ties away from zero", "else out = (c % 2u == 0u) ? c : c + 1u;", "else out = c + 1u;"),
 ("SR compare <=", "out = ((double)u < f * 4294967296.0) ? c + 1u : c;", "out = ((double)u <= f * 4294967296.0) ? c + 1u : c;"),
 ("SR direction flipped", "out = ((double)u < f * 4294967296.0) ? c + 1u : c;", "out = ((double)u < f * 4294967296.0) ? c : c + 1u;"),
 ("bf16/f16 overflow saturates", "if (stochastic || dtype == ORC_I8 || dtype == ORC_F8E4M3 || a == maxv)", "if (1)"),
 ("e4m3 overflow to NaN code", "if (stochastic || dtype == ORC_I8 || dtype == ORC_F8E4M3 || a == maxv)", "if (stochastic || dtype == ORC_I8 || a == maxv)"),
 ("subnormal exponent off by one", "return ldexp((double)m, 1 - f->bias - f->mbits);", "return ldexp((double)m, -f->bias - f->mbits);"),
 ("e4m3 bias 8", "static const fmt_t FMT_E4M3 = {4, 3, 7, 0, 0x7Eu};", "static const fmt_t FMT_E4M3 = {4, 3, 8, 0, 0x7Eu};"),
 ("int8 range to 128", "if (dtype == ORC_I8) return 127u;", "if (dtype == ORC_I8) return 128u;"),
 ("NaN sign dropped (f16)", "case ORC_F16: return (negative ? 0x8000u : 0u) | 0x7E00u;", "case ORC_F16: return 0x7E00u;"),
 ("int8 NaN to 127", "default: return 0u; /* int8: NaN encodes as 0 */", "default: return 127u;"),
 ("Philox multiplier swapped", "uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;\n    uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;", "uint64_t p0 = (uint64_t)M1 * (uint64_t)c0;\n    uint64_t p1 = (uint64_t)M0 * (uint64_t)c2;"),
 ("Philox key bump before the first Philox round", "if (i > 0) { k0 += W0; k1 += W1; }", "{ k0 += W0; k1 += W1; }"),
 ("ssu: append ignores pending count", "const int32_t e = (r0 + n + t) % R;", "const int32_t e = (r0 + t) % R;", "ssu_oracle.c"),
 ("ssu: pending entry off by one", "const int32_t e = (r0 + j) % R;", "const int32_t e = (r0 + j + 1) % R;", "ssu_oracle.c"),
 ("ssu: no dt bias on replayed new tokens", "          if (in->dt_bias) dt += (double)in->dt_bias[h];\n          if (p->dt_softplus) dt = softplus(dt);\n          xb = in->x_new;", "          if (p->dt_softplus) dt = softplus(dt);\n          xb = in->x_new;", "ssu_oracle.c"),
 ("ssu: decay sign", "const double a = exp(dt * A);", "const double a = exp(-dt * A);", "ssu_oracle.c"),
 ("ssu: D term dropped", "            y += dx;", "            (void)dx;", "ssu_oracle.c"),
 ("ssu: sigmoid gate instead of silu", "const double gate = zv / (1.0 + exp(-zv));", "const double gate = 1.0 / (1.0 + exp(-zv));", "ssu_oracle.c"),
 ("checkpoints: no pre-call snapshot", "ins = _Inputs(state=_ptr_array(state_in), state_stride=_i64(meta.state_stride),\n                      scale=_ptr_array(scale_in) if scale_in else None,", "ins = _Inputs(state=_ptr_array(state_out), state_stride=_i64(meta.state_stride),\n                      scale=_ptr_array(scale_out) if scale_out else None,", "__init__.py"),
 ("checkpoints: first prefix table for all", "pf = np.ascontiguousarray(pref, np.int32)", "pf = np.ascontiguousarray(prefix_list[0], np.int32)", "__init__.py"),
 ("checkpoints: first destination table for all", "dst_arr = np.ascontiguousarray(dst, np.int32)", "dst_arr = np.ascontiguousarray(dst_list[0], np.int32)", "__init__.py"),
 ("gdn: decay after the update",
  ("    for (int i = 0; i < dv * dk; ++i) S[i] *= alpha;\n", "    if (t == track_step) {"),
  ("", "    for (int i = 0; i < dv * dk; ++i) S[i] *= alpha;\n    if (t == track_step) {"), "gdn_oracle.c"),
 ("gdn: wrong key-head map", "(((int64_t)l * p->slots + s) * H + hv / group);", "(((int64_t)l * p->slots + s) * H + hv % H);", "gdn_oracle.c"),
 ("gdn: keys not normalised", "if (p->use_l2norm) {", "if (0) {", "gdn_oracle.c"),
 ("gdn: tracked step off by one", "if (t == track_step) {", "if (t == track_step + 1) {", "gdn_oracle.c"),
 ("gdn: update sign", "const double u = beta * (v - Sk[i]);", "const double u = beta * (Sk[i] - v);", "gdn_oracle.c"),
 ("gdn: epsilon outside the root", "const double nrm = sqrt(ss + 1e-6);", "const double nrm = sqrt(ss) + 1e-6;", "gdn_oracle.c"),
 ("gdn: transposed product S k", "acc += S[(size_t)i * dk + j] * k[j];", "acc += S[(size_t)j * dk + i] * k[j];", "gdn_oracle.c"),
 ("gdn: beta inside the bracket", "const double u = beta * (v - Sk[i]);", "const double u = beta * v - Sk[i];", "gdn_oracle.c"),
 ("ssu: C of the wrong group", "const int64_t cbase = (((int64_t)b * T + t) * G + g) * ds;", "const int64_t cbase = (((int64_t)b * T + t) * G + (G - 1 - g)) * ds;", "ssu_oracle.c"),
]
def run(name, old, new, fname="rssm_oracle.c"):
    d = os.path.join(WORK, "case")
    shutil.rmtree(d, ignore_errors=True)
    shutil.copytree(BASE, d)
    if old is not None:
        p = os.path.join(d, "oracle", fname)
        s = open(p).read()
        pairs = zip(old, new) if isinstance(old, tuple) else [(old, new)]
        for o, n in pairs:
            assert s.count(o) == 1, (name, s.count(o))
            s = s.replace(o, n)
        open(p, "w").write(s)
    subprocess.check_call([sys.executable, "-c", "import oracle; oracle.build()"], cwd=d)
    tests = sorted(f"tests/{f}" for f in os.listdir(os.path.join(d, "tests")) if f.startswith("test_oracle_"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *tests], cwd=d,
                       capture_output=True, text=True, timeout=1200)
    last = r.stdout.strip().splitlines()[-1]
    failed = int(re.search(r"(\d+) failed", last).group(1)) if "failed" in last else 0
    passed = int(re.search(r"(\d+) passed", last).group(1)) if "passed" in last else 0
    names = sorted(set(l.split("::")[1].split(" ")[0].split("[")[0] for l in r.stdout.splitlines() if l.startswith("FAILED")))
    print(f"{name} | {failed} failed, {passed} passed | {', '.join(names[:6])}", flush=True)
    return failed
os.makedirs(BASE)
subprocess.check_call(f"git -C {REPO} archive HEAD | tar -x -C {BASE}", shell=True)
baseline = run("none (baseline)", None, None)
sel = sys.argv[1:]
missed = [m[0] for m in M if (not sel or any(s in m[0] for s in sel)) and run(*m) == 0]
shutil.rmtree(WORK, ignore_errors=True)
if baseline or missed:
    sys.exit(f"baseline failures: {baseline}; mistakes no pin caught: {missed}")
print("every planted mistake fails at least one pin")
