"""The benchmark's command line and pure helpers (no GPU)."""

from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_percentiles_nearest_rank():
    xs = [float(i) for i in range(1, 11)]          # 1 .. 10
    assert bench.percentiles(xs) == [2.0, 6.0, 9.0]  # indexes floor(p (n - 1) + 1/2): 1, 5, 8
    assert bench.percentiles([]) is None
    assert bench.percentiles([3.5]) == [3.5, 3.5, 3.5]


class _Shape:
    def __init__(self, Hq, Hkv, D, dtype):
        self.Hq, self.Hkv, self.D, self.dtype = Hq, Hkv, D, dtype


def test_side_bytes_of_a_decode():
    # beam shape: 32 layers, 8 branches, Hq 32, Hkv 8, D 128, bf16; 64 partial rows per plane
    sh = _Shape(32, 8, 128, "bf16")
    info = {"partial_rows": 64, "workspace_bytes": 64 * 32 * 8 * (128 + 2) * 4 + 1792,
            "plan_bytes": 1632}
    b = bench.side_bytes(sh, 32, 8, info)
    assert b["q"] == 32 * 8 * 32 * 128 * 2
    assert b["out"] == 32 * 8 * 32 * 128 * 4
    assert b["partials"] == 2 * 64 * 32 * 8 * 130 * 4
    assert b["plan"] == 1632 and b["plan_in_launch_args"]
    info["plan_bytes"] = 12288
    assert bench.side_bytes(sh, 32, 8, info)["plan_in_launch_args"]
    info["plan_bytes"] = 12304
    assert not bench.side_bytes(sh, 32, 8, info)["plan_in_launch_args"]


def test_compare_applies_the_parity_bar():
    import numpy as np
    want = np.linspace(-1, 1, 64).reshape(4, 16)
    assert bench.compare(want + 1e-4, want)["ok"]
    assert not bench.compare(want + 3e-3, want)["ok"]          # max-abs above 2e-3
    small = want * 1e-3
    assert not bench.compare(small * 1.05, small)["ok"]        # relative L2 above 1e-2
    bad = want.copy()
    bad[0, 0] = np.nan
    assert not bench.compare(bad, want)["ok"]


def test_parity_legs_on_the_tiny_trees():
    """The bench's parity legs, fed the oracle's own output (passes) and the
    same output with one row moved by 4e-3 (fails)."""
    import numpy as np
    import oracle
    from workloads import generate, get, scaled
    w = get("tiny_b")
    inp = generate(w)
    pool = bench.oracle_pool(w, inp)
    want = oracle.decode(pool, list(w.query_sids), inp.q.f32(), w.softmax_scale)
    assert bench.parity_decode(pool, w, inp, want, 0)["ok"]
    off = want.copy()
    off[0, 1, 2] += 4e-3
    assert not bench.parity_decode(pool, w, inp, off, 0)["ok"]
    v = scaled("verify", "verify_tiny", n_req=2, ctx_len=40, n_nodes=9, max_depth=4,
               shape=get("tiny_a").shape)
    vin = generate(v)
    vpool = bench.oracle_pool(v, vin)
    vwant = oracle.verify(vpool, list(v.query_sids), vin.parents, vin.q.f32(), v.softmax_scale)
    assert bench.parity_verify(vpool, v, vin, vwant, 1, [0, 3, 8])["ok"]
    vwant[1, 3, 0, 0] += 4e-3
    assert not bench.parity_verify(vpool, v, vin, vwant, 1, [0, 3, 8])["ok"]


def test_nested_records_keep_the_measured_fields():
    rec = {"config": {"workload": "x"}, "value": 1.0, "unit": "GB/s", "roofline": {"frac": 0.5},
           "parity": {"ok": True}, "metric": "m", "n_gpus": 1, "commit": None}
    out = bench.nested(rec)
    assert out == {"workload": "x", "value": 1.0, "unit": "GB/s", "roofline": {"frac": 0.5},
                   "parity": {"ok": True}}


def test_kernel_hash_ignores_comments_only():
    """The stored HBM counters are keyed by the kernels' code: a comment or
    layout edit keeps the key, a code edit (also inside an asm string)
    changes it."""
    src = {name: bench.code_only("") for name in bench.KERNEL_SOURCES}
    text = ('// header\nint f(int a) { /* sum */ return a + 1; }  // tail\n'
            'void g() { asm("s_nop 7\\n\\t// not a comment" : : ); }\n')
    src[bench.KERNEL_SOURCES[0]] = text
    base = bench.kernel_source_hash(lambda n: src[n])
    commented = text.replace("int f(int a) {", "/* a new\n   comment */ int  f(int a)\n{")
    src[bench.KERNEL_SOURCES[0]] = commented
    assert bench.kernel_source_hash(lambda n: src[n]) == base
    for edit in (text.replace("a + 1", "a + 2"), text.replace("s_nop 7", "s_nop 6"),
                 text.replace("// not a comment", "// other text")):
        src[bench.KERNEL_SOURCES[0]] = edit
        assert bench.kernel_source_hash(lambda n: src[n]) != base
    assert bench.code_only('x = "/* kept */"; // gone\ny;') == 'x = "/* kept */"; y;'


def test_pool_options_from_the_command_line():
    """--option key=value (repeatable) reaches every pool the bench makes."""
    class _Pool:
        def __init__(self):
            self.set = []

        def set_option(self, key, value):
            self.set.append((key, value))

    saved = list(bench.OPTIONS)
    try:
        bench.OPTIONS[:] = ["wide_spec=1", "chunk_tokens=64"]
        c = _Pool()
        bench.apply_options(c)
        assert c.set == [("wide_spec", 1), ("chunk_tokens", 64)]
    finally:
        bench.OPTIONS[:] = saved
