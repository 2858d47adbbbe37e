"""Each plausible mistake planted in a copy of the oracle must fail a pin.

The mutants are textual edits of ``oracle/attn_oracle.c`` compiled into a
temporary directory (CPU only); the pin battery of ``tests/oracle_pins.py`` runs
against each one in a child process.  The real oracle source is never changed.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text to find, replacement, which occurrence (0 = all))
MUTANTS = [
    ("scale dropped", "s[j] = scale * dot;", "s[j] = dot;", 0),
    ("max subtracted with wrong sign", "exp(s[j] - m)", "exp(m - s[j])", 0),
    ("normalisation dropped", "p[j] /= l;", "p[j] /= 1.0;", 0),
    ("max missing from LSE", "*lse = m + log(l);", "*lse = log(l);", 0),
    ("log2 instead of ln in LSE", "*lse = m + log(l);", "*lse = m + log2(l);", 0),
    ("GQA head taken modulo", "int hk = h / G;", "int hk = h % A_kv;", 1),
    ("causal diagonal excluded", "(int64_t)j > (int64_t)i + (S_k - S_q)", "(int64_t)j >= (int64_t)i + (S_k - S_q)", 0),
    ("causal aligned top-left", "(int64_t)j > (int64_t)i + (S_k - S_q)", "(int64_t)j > (int64_t)i", 0),
    ("V read from K", "acc += p[j] * ld(v, kv_off[j] + e, dt);", "acc += p[j] * ld(k, kv_off[j] + e, dt);", 0),
    ("q_keep ignored (dense)", "int row_masked = q_keep && !q_keep[(int64_t)b * S_q + i];", "int row_masked = 0;", 0),
    ("k_keep ignored (dense)", "if (k_keep && !k_keep[(int64_t)b * S_k + j])", "if (0)", 0),
    ("k_keep ignored (varlen)", "if (k_keep && !k_keep[start + j])", "if (0)", 0),
    ("decode window excludes its left edge", "(int64_t)t >= (int64_t)n - 1 - win_left", "(int64_t)t > (int64_t)n - 1 - win_left",
     0),
    ("decode window ignored", "w.vis[t] = win_left < 0 ||", "w.vis[t] = 1 ||", 0),
    ("decode window anchored at the first token", "(int64_t)t >= (int64_t)n - 1 - win_left", "(int64_t)t <= (int64_t)win_left",
     0),
    ("varlen causal diagonal excluded", "if (causal && j > i)", "if (causal && j >= i)", 0),
    ("varlen keys not offset to sequence", "int64_t kv_base = ((int64_t)(h / G) * T + start) * d;",
     "int64_t kv_base = ((int64_t)(h / G) * T) * d;", 0),
    ("paged head stride dropped", "w.off[t] = ((page * page_size + off) * A_kv + hk) * (int64_t)d;",
     "w.off[t] = ((page * page_size + off) * A_kv) * (int64_t)d;", 0),
    ("paged offset uses page index", "int off = t % page_size;", "int off = (t / page_size) % page_size;", 0),
    ("bf16 widened with wrong shift", "<< 16;", "<< 15;", 0),
    ("last head-dim term dropped", "for (int e = 0; e < d; ++e)\n                dot +=", "for (int e = 0; e < d - 1; ++e)\n                dot +=", 0),
    ("fully masked row not guarded", "if (m == -INFINITY) {", "if (0) {", 0),
    ("row max taken as first score", "if (s[j] > m)\n            m = s[j];", "if (j == 0)\n            m = s[j];", 0),
    ("gradient: D term dropped", "double ds = w.p[j] * (dp[j] - D);", "double ds = w.p[j] * dp[j];", 0),
    ("gradient: dK scale dropped", "dkg[(int64_t)j * d + e] += sc * ds", "dkg[(int64_t)j * d + e] += ds", 0),
    ("gradient: dV weighted by dS", "dvg[(int64_t)j * d + e] += w.p[j] *", "dvg[(int64_t)j * d + e] += ds *", 0),
    ("gradient: dQ built from V", "dqi[e] += sc * ds * ld(k,", "dqi[e] += sc * ds * ld(v,", 0),
    ("gradient: dP built from K", "acc += ld(do_, id * d + e, dt) * ld(v, w.off[j] + e, dt);",
     "acc += ld(do_, id * d + e, dt) * ld(k, w.off[j] + e, dt);", 0),
    ("keep matrix ignored (dense)", "if (m_keep && !m_keep[((int64_t)b * S_q + i) * S_k + j])", "if (0)", 1),
    ("keep matrix transposed (dense)", "m_keep[((int64_t)b * S_q + i) * S_k + j]",
     "m_keep[((int64_t)b * S_k + j) * S_q + i]", 1),
    ("gradient: keep matrix ignored", "if (m_keep && !m_keep[((int64_t)b * S_q + i) * S_k + j])", "if (0)", 2),
    ("additive term scaled by the softmax scale", "s[j] += (double)bias_row[j];",
     "s[j] += scale * (double)bias_row[j];", 0),
    ("additive term subtracted", "s[j] += (double)bias_row[j];", "s[j] -= (double)bias_row[j];", 0),
    ("additive term: head ignored", "(bias_heads == 1 ? 0 : h)", "0", 0),
    ("additive term: row ignored", "* S_q + i) * S_k : NULL;", "* S_q + 0) * S_k : NULL;", 0),
    ("additive term: fill value kept finite", "if ((double)bias_row[j] < fill_limit(scale))", "if (0)", 0),
    ("additive term: fill limit without the scale", "return -flt_max * (scale < ln2 ? scale : ln2);",
     "return -flt_max;", 0),
    ("block mask: 64-wide blocks", "i / 128) * nkb + j / 128]", "i / 64) * nkb + j / 64]", 1),
    ("block mask: index transposed", "* nqb + i / 128) * nkb + j / 128]", "* nkb + j / 128) * nqb + i / 128]", 1),
    ("block mask: head ignored", "int hm = block_heads == 1 ? 0 : h;", "int hm = 0;", 0),
    ("block mask ignored (dense)", "if (!block_kept(block_keep, block_heads, b, h, S_q, S_k, i, j))", "if (0)", 1),
    ("gradient: block mask ignored", "if (!block_kept(block_keep, block_heads, b, h, S_q, S_k, i, j))", "if (0)", 2),
    ("gradient: additive term ignored", "w.vis, bias_row, S_k, d, sc, w.s, w.p, o, &lse);",
     "w.vis, NULL, S_k, d, sc, w.s, w.p, o, &lse);", 0),
    ("block mask of a bias: 64-wide blocks", "out[(bh * nqb + i / 128) * nkb + j / 128] = 1;",
     "out[(bh * nqb + i / 64) * nkb + j / 64] = 1;", 0),
    ("block mask of a bias: finite negatives ignored", "if (row[j] > -INFINITY)", "if (row[j] > -1e30f)", 0),
    ("block mask of a bias: row stride S_q", "const float *row = bias + (bh * S_q + i) * (int64_t)S_k;",
     "const float *row = bias + (bh * S_q + i) * (int64_t)S_q;", 0),
    ("paged prefill: page offset uses page index", "int off = t % page_size;", "int off = (t / page_size) % page_size;", 2),
    ("paged prefill: chunk aligned top-left", "int pos = L - q_len + (x - cu_q[s]);", "int pos = x - cu_q[s];", 0),
    ("paged prefill: causal diagonal excluded", "if (causal && t > pos)", "if (causal && t >= pos)", 0),
    ("paged prefill: window left edge ignored", "if (win_left >= 0 && t < pos - win_left)", "if (0)", 0),
    ("paged prefill: window right edge ignored", "if (win_right >= 0 && t > pos + win_right)", "if (0)", 0),
    ("paged prefill: GQA head taken modulo", "int hk = h / G;", "int hk = h % A_kv;", 3),
    ("varlen gradient: keys not offset to sequence", "int64_t kv_base = ((int64_t)hk * T + start) * d;",
     "int64_t kv_base = ((int64_t)hk * T) * d;", 0),
    ("varlen gradient: window left edge ignored", "if (win_left >= 0 && j < i - win_left)", "if (0)", 0),
    ("varlen gradient: window right edge off by one", "if (win_right >= 0 && j > i + win_right)",
     "if (win_right >= 0 && j >= i + win_right)", 0),
    ("varlen gradient: D term dropped", "double ds = w.p[j] * (dp[j] - D);", "double ds = w.p[j] * dp[j];", 2),
    ("varlen gradient: key flags ignored", "if (k_keep && !k_keep[start + j])\n                            visible = 0;",
     "if (0)\n                            visible = 0;", 0),
]

# Mutants of the package's Python side (oracle/__init__.py): the E4M3 code
# values, the FP8 block scales, the window keep matrix.  (name, text to find,
# replacement, which occurrence (0 = all))
PY_MUTANTS = [
    ("E4M3 exponent bias 8", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)", 0),
    ("E4M3 sign bit ignored", "sign = np.where(c & 0x80, -1.0, 1.0)", "sign = 1.0", 0),
    ("E4M3 subnormals without the 2^-6 factor", "(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7", 0),
    ("FP8 prefill: 64-token query scale blocks", "np.repeat(qs, 128, axis=2)", "np.repeat(qs, 64, axis=2)", 0),
    ("FP8 prefill: key scales ignored", "kv = fp8_e4m3_value(kc) * np.repeat(ks, 128, axis=2)[:, :, :S_k, None]",
     "kv = fp8_e4m3_value(kc) * 1.0", 0),
    ("FP8 decode: window ignored", "window_left=window_left, alibi_slopes=alibi_slopes)",
     "window_left=None, alibi_slopes=alibi_slopes)", 0),
    ("FP8 decode: value scale of the key", "vc = fp8_e4m3_value(v_codes[pages]) * np.asarray(v_scale",
     "vc = fp8_e4m3_value(v_codes[pages]) * np.asarray(k_scale", 0),
    ("FP8 paged prefill: value scale of the key", "vc = fp8_e4m3_value(v_codes) * np.asarray(v_scale",
     "vc = fp8_e4m3_value(v_codes) * np.asarray(k_scale", 0),
    ("window: left edge off by one", "keep &= j >= i - left", "keep &= j > i - left", 0),
    ("window: aligned top-left", "off = S_k - S_q\n    i = np.arange(S_q, dtype=np.int64)[:, None] + off",
     "off = 0\n    i = np.arange(S_q, dtype=np.int64)[:, None] + off", 0),
    ("varlen term rows not offset to the sequence", 'kw["bias"] = bias[:, s0:s1, :L][None]',
     'kw["bias"] = bias[:, 0:L, :L][None]', 0),
    ("varlen term columns offset to the sequence", 'kw["bias"] = bias[:, s0:s1, :L][None]',
     'kw["bias"] = bias[:, s0:s1, s0:s0 + L][None]', 0),
    ("varlen block mask of the first sequence", 'kw["block_keep"] = block_keep[s][None, :, :nbs, :nbs]',
     'kw["block_keep"] = block_keep[0][None, :, :nbs, :nbs]', 0),
    ("packed gradient: term rows not offset to the sequence", 'kw["bias"] = bias[:, s0:s1, :L][None]',
     'kw["bias"] = bias[:, 0:L, :L][None]', 1),
    ("packed gradient: block mask of the first sequence", 'kw["block_keep"] = block_keep[s][None, :, :nbs, :nbs]',
     'kw["block_keep"] = block_keep[0][None, :, :nbs, :nbs]', 1),
    ("paged term rows not offset to the chunk", 'kw["bias"] = bias[:, s0:s1, :L][None]', 'kw["bias"] = bias[:, 0:ql, :L][None]',
     2),
    ("paged block mask of the first sequence",
     'kw["block_keep"] = block_keep[s][None, :, :(ql + 127) // 128, :(L + 127) // 128]',
     'kw["block_keep"] = block_keep[0][None, :, :(ql + 127) // 128, :(L + 127) // 128]', 0),
    ("paged keys gathered page-major (t // ps as the row)", "offs = np.arange(L) % page_size",
     "offs = (np.arange(L) // page_size) % page_size", 0),
    ("paged causal diagonal aligned top-left", 'kw["m_keep"] = window_keep(1, ql, L, int(window[0]), int(window[1]))',
     'kw["m_keep"] = window_keep(1, ql, ql, int(window[0]), int(window[1]))', 0),
    ("key range: last key excluded", "(j <= r[..., 1:2])", "(j < r[..., 1:2])", 0),
    ("key range: first key excluded", "(j >= r[..., 0:1])", "(j > r[..., 0:1])", 0),
    ("key range: last key ignored", "((j >= r[..., 0:1]) & (j <= r[..., 1:2]))", "(j >= r[..., 0:1])", 0),
    ("key ranges ignored beside a keep matrix", "mk = rk if mk is None else mk & rk", "mk = rk if mk is None else mk", 0),
    ("key ranges ignored", "mk = rk if mk is None else mk & rk", "mk = mk", 0),
    ("varlen key ranges of the first tokens", 'kw["key_range"] = np.asarray(key_range).reshape(T, 2)[s0:s1][None]',
     'kw["key_range"] = np.asarray(key_range).reshape(T, 2)[0:L][None]', 0),
    ("paged key ranges of the first tokens", 'kw["key_range"] = np.asarray(key_range).reshape(T_q, 2)[s0:s1][None]',
     'kw["key_range"] = np.asarray(key_range).reshape(T_q, 2)[0:ql][None]', 0),
    ("ALiBi: penalty sign flipped", "m = -sl[:, None, None] * dist[None]", "m = sl[:, None, None] * dist[None]", 0),
    ("ALiBi: signed distance", "dist = np.abs(p[:, None] - np.arange(S_k, dtype=np.int64)[None, :])",
     "dist = (p[:, None] - np.arange(S_k, dtype=np.int64)[None, :])", 0),
    ("ALiBi: queries aligned top-left", "(np.arange(S_q, dtype=np.int64) + (S_k - S_q))",
     "np.arange(S_q, dtype=np.int64)", 0),
    ("ALiBi: the first head's slope for every head", "m = -sl[:, None, None] * dist[None]",
     "m = -sl[:1, None, None] * dist[None]", 0),
    ("ALiBi ignored in packed and paged calls", 'kw["alibi_slopes"] = alibi_slopes', 'kw["alibi_slopes"] = None', 0),
    ("ALiBi ignored", "return a if bias is None else", "return bias if bias is None else", 0),
    ("decode ALiBi: window dropped", "window = None if window_left is None else (int(window_left), 0)",
     "window = None", 0),
    ("decode ALiBi: sequences' rows shifted", "o[live] = oc.transpose(1, 0, 2)", "o[live] = oc.transpose(1, 0, 2)[::-1]", 0),
    ("FP8 decode: ALiBi ignored", "window_left=window_left, alibi_slopes=alibi_slopes)",
     "window_left=window_left, alibi_slopes=None)", 0),
    ("varlen block mask transposed", 'kw["block_keep"] = block_keep[s][None, :, :nbs, :nbs]',
     'kw["block_keep"] = np.ascontiguousarray(block_keep[s][None, :, :nbs, :nbs].transpose(0, 1, 3, 2))', 0),
]

BATTERY = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins
orc = oracle.Oracle({lib!r})
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(orc)
    except Exception as e:  # a pin that fails or cannot run counts
        failed.append(pin.__name__)
print("FAILED_PINS", ",".join(failed))
"""


def _mutate(src, old, new, which):
    assert old in src, f"mutation anchor not found: {old!r}"
    if which == 0:
        return src.replace(old, new)
    parts = src.split(old)
    assert len(parts) > which
    return old.join(parts[:which]) + new + old.join(parts[which:])


def test_mutants_fail_a_pin(tmp_path):
    src = open(oracle.SRC).read()
    # the unmutated source must pass every pin (control)
    results = {}
    for name, old, new, which in [("control", "", "", -1)] + MUTANTS:
        msrc = src if which == -1 else _mutate(src, old, new, which)
        c = tmp_path / f"m{len(results)}.c"
        c.write_text(msrc)
        lib = str(tmp_path / f"m{len(results)}.so")
        oracle.build(str(c), lib, werror=False)
        r = subprocess.run([sys.executable, "-c", BATTERY.format(root=ROOT, lib=lib)],
                           capture_output=True, text=True, timeout=300, cwd=ROOT)
        line = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED_PINS")]
        failed = line[0].split(" ", 1)[1].split(",") if line and line[0].strip() != "FAILED_PINS" else []
        crashed = r.returncode != 0
        results[name] = (failed, crashed)
    assert results["control"] == ([], False), results["control"]
    undetected = [n for n, (f, crashed) in results.items() if n != "control" and not f and not crashed]
    for n, (f, crashed) in results.items():
        print(f"{n:40s} caught by {len(f):2d} pins{' (crashed)' if crashed else ''}: {','.join(f)}")
    assert not undetected, f"mutants no pin catches: {undetected}"


def test_python_mutants_fail_a_pin(tmp_path):
    """The same for the package's Python side: each mutant is a copy of the
    oracle package whose __init__.py carries the mistake, imported ahead of the
    real one by the pin battery's child process."""
    import shutil
    src = open(os.path.join(os.path.dirname(oracle.SRC), "__init__.py")).read()
    undetected = []
    for n, (name, old, new, which) in enumerate([("control", "", "", -1)] + PY_MUTANTS):
        root = tmp_path / f"p{n}"
        pkg = root / "oracle"
        pkg.mkdir(parents=True)
        for f in ("attn_oracle.c", "blockwise.py", "liboracle.so"):
            shutil.copy(os.path.join(os.path.dirname(oracle.SRC), f), pkg / f)
        (pkg / "__init__.py").write_text(src if which == -1 else _mutate(src, old, new, which))
        code = BATTERY.format(root=ROOT, lib=str(pkg / "liboracle.so")).replace(
            "sys.path.insert(0, {!r})".format(ROOT), "sys.path.insert(0, {!r}); sys.path.insert(0, {!r})".format(
                ROOT, str(root)))
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=str(root))
        line = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED_PINS")]
        failed = line[0].split(" ", 1)[1].split(",") if line and line[0].strip() != "FAILED_PINS" else []
        print(f"{name:45s} caught by {len(failed):2d} pins{' (crashed)' if r.returncode else ''}: {','.join(failed)}")
        if which == -1:
            assert failed == [] and r.returncode == 0, (failed, r.stderr[-2000:])
        elif not failed and r.returncode == 0:
            undetected.append(name)
    assert not undetected, f"Python mutants no pin catches: {undetected}"
