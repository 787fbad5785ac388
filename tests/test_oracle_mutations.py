"""The oracle's pins catch plausible mistakes: each case below plants one (an
off-by-one, a wrong operator, a dropped term, a swapped index or operand) in a
copy of oracle/msa_oracle.py, and the pin tests of tests/test_oracle_pins.py
run against that copy (MSA_ORACLE_UNDER_TEST names it); at least one pin must
fail on every copy. The committed oracle is never modified. An unmodified copy
must pass, so that a failure means a pin failed, not that the copy did not
load."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "msa_oracle.py")

# (what the mistake is, text in the oracle, its replacement)
MUTATIONS = [
    ("a row does not see its own key", "return int(row_pos) + 1", "return int(row_pos)"),
    ("block count rounded down", "return (int(v) + PAGE - 1) // PAGE", "return int(v) // PAGE"),
    ("row position without the prior context", "row_pos.append(context_len + i)", "row_pos.append(i)"),
    ("cu_seqlens_k sums query rows", "cu_k[r + 1] = cu_k[r] + L[r]", "cu_k[r + 1] = cu_k[r] + ql[r]"),
    ("index tile read with chunk and group swapped", "rows = page.transpose(0, 3, 1, 2, 4)",
     "rows = page.transpose(0, 3, 2, 1, 4)"),
    ("index dot product drops a dimension", "return keys[:v] @ qi", "return keys[:v, 1:] @ qi[1:]"),
    ("mean instead of max pooling", "out[b] = np.max(tok_scores[b * PAGE:(b + 1) * PAGE])",
     "out[b] = np.mean(tok_scores[b * PAGE:(b + 1) * PAGE])"),
    ("ties go to the higher block id", "key=lambda sb: (-sb[0], sb[1])", "key=lambda sb: (-sb[0], -sb[1])"),
    ("lowest scores kept", "key=lambda sb: (-sb[0], sb[1])", "key=lambda sb: (sb[0], sb[1])"),
    ("selection not listed by block id", "return np.array(sorted(b for _, b in keep), dtype=np.int64)",
     "return np.array([b for _, b in keep], dtype=np.int64)"),
    ("sub-page id with page and index swapped", "SUBS_PER_PAGE * int(bt_row[int(b)]) + i",
     "SUBS_PER_PAGE * i + int(bt_row[int(b)])"),
    ("table padded with -1", "out = np.zeros(SUBS_PER_PAGE * topk, dtype=np.int64)",
     "out = np.full(SUBS_PER_PAGE * topk, -1, dtype=np.int64)"),
    ("partial last block counted whole", "min(PAGE, int(v) - PAGE * int(b))", "PAGE"),
    ("e4m3 exponent bias 8", "(e - 7).astype(np.int64)", "(e - 8).astype(np.int64)"),
    ("e4m3 subnormals scaled by 2^-7", "np.ldexp(m / 8.0, -6)", "np.ldexp(m / 8.0, -7)"),
    ("softmax scale dropped", "    z = sm_scale * (q @ k.T)                       # [H][T]\n    m = z.max(axis=1, keepdims=True)",
     "    z = (q @ k.T)                       # [H][T]\n    m = z.max(axis=1, keepdims=True)"),
    ("LSE in log2", "lse = m + np.log(den)", "lse = m + np.log2(den)"),
    ("sink not shifted by the max", "den = den + np.exp(np.asarray(sinks, dtype=np.float64) - m)",
     "den = den + np.exp(np.asarray(sinks, dtype=np.float64))"),
    ("per-token-head scale from the sub-page slot", "return float(s[page, t % PAGE, hkv])",
     "return float(s[page, t % SUB, hkv])"),
    ("K/V token read from the next slot", "    slot = t % SUB\n    raw =", "    slot = (t + 1) % SUB\n    raw ="),
    ("attention walks one key past the visible ones", "min(PAGE * (int(b) + 1), v)",
     "min(PAGE * (int(b) + 1), v + 1)"),
    ("table walk reads entry u // 8", "sub = int(table[n][u // SUB])", "sub = int(table[n][u // SUBS_PER_PAGE])"),
    ("V scaled by the K scale in the table walk", "vh[u] = vs * dec(", "vh[u] = ks * dec("),
    ("quantiser scale from 240", "s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0",
     "s = np.float32(amax / np.float32(240.0)) if amax > 0"),
    ("insert skips slot 0", "        if slot < 0 or slot >= num_slots:\n            continue\n        page, off = divmod",
     "        if slot <= 0 or slot >= num_slots:\n            continue\n        page, off = divmod"),
    ("fp8 codes not clamped to 448", "        y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))\n", ""),
]


def _run_pins(path):
    env = dict(os.environ, MSA_ORACLE_UNDER_TEST=path)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x",
                        "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(ORACLE).read()
    clean = tmp_path / "clean.py"
    clean.write_text(src)
    code, out = _run_pins(str(clean))
    assert code == 0, "the unmodified copy does not pass its pins:\n" + out
    paths = []
    for i, (what, old, new) in enumerate(MUTATIONS):
        assert src.count(old) == 1, f"mutation '{what}': its text is not found once in the oracle"
        p = tmp_path / f"mutant_{i}.py"
        p.write_text(src.replace(old, new))
        paths.append(str(p))
    with ThreadPoolExecutor(max_workers=6) as pool:
        results = list(pool.map(_run_pins, paths))
    survived = [what for (what, _, _), (code, _) in zip(MUTATIONS, results) if code == 0]
    broken = [(what, out) for (what, _, _), (code, out) in zip(MUTATIONS, results) if code not in (0, 1)]
    assert not broken, f"copies that did not run as tests: {broken[:2]}"
    assert not survived, f"planted mistakes no pin caught: {survived}"
