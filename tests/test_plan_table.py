"""The tuned plan table (nvfp4_plan_table_load): JSON reading, entry checks,
the lookup rule, and the table shipped with the package.  Host-only."""
from __future__ import annotations

import json
import os

import pytest

import block_scaled_fp4_04_amd as nv
import plan_cases


def write(tmp_path, doc, name="t.json"):
    p = tmp_path / name
    p.write_text(doc if isinstance(doc, str) else json.dumps(doc))
    return str(p)


def table(entries, **head):
    d = {"format": "nvfp4-plan-table", "version": 1, "arch": "gfx950", "build": "x",
         "entries": entries}
    d.update(head)
    return d


def entry(M, N, K, path, tile=0, split_k=1, **extra):
    e = {"M": M, "N": N, "K": K, "path": path, "tile": tile, "split_k": split_k}
    e.update(extra)
    return e


def load(path):
    n, same = nv._i64(), nv.ctypes.c_int()
    st = nv.lib().nvfp4_plan_table_load(os.fsencode(path), nv.ctypes.byref(n),
                                        nv.ctypes.byref(same))
    return st, n.value, same.value


@pytest.fixture
def base(tmp_path, no_table):
    """A small table loaded; yields its path."""
    path = write(tmp_path, table([
        entry(4096, 2048, 6144, "tile", 128, 1, us=107.9),
        entry(2048, 2048, 6144, "tile", 128, 2),
        entry(512, 768, 6144, "wsplit", 128, 3),
        entry(16, 256, 6144, "skinny", 0, 2),
        entry(4, 768, 6144, "gemv"),
        entry(256, 768, 8192, "wsplit", 16, 1),
        entry(512, 768, 8192, "wsplit", 32, 2),
    ]), "base.json")
    assert load(path)[:2] == (nv.OK, 7)
    yield path


def test_exact_and_nearby_shapes(base):
    p = nv.plan(4096, 2048, 6144)
    assert (p["path"], p["tile_m"], p["split_k"], p["source"]) == (nv.PATH_TILE, 128, 1, nv.PLAN_TABLE)
    # same N and K: the smallest tuned M' >= M, if M' <= 2 M
    assert nv.plan(3000, 2048, 6144)["split_k"] == 1          # -> 4096
    assert nv.plan(2049, 2048, 6144)["split_k"] == 1          # -> 4096
    assert nv.plan(2048, 2048, 6144)["split_k"] == 2          # exact
    assert nv.plan(1024, 2048, 6144)["split_k"] == 2          # -> 2048 (= 2 M)
    assert nv.plan(1023, 2048, 6144)["source"] == nv.PLAN_HEURISTIC  # 2048 > 2 M
    assert nv.plan(4097, 2048, 6144)["source"] == nv.PLAN_HEURISTIC  # nothing above
    assert nv.plan(4096, 2048, 8192)["source"] == nv.PLAN_HEURISTIC  # other K
    assert nv.plan(4096, 2304, 6144)["source"] == nv.PLAN_HEURISTIC  # other N
    w = nv.plan(300, 768, 6144)
    assert (w["path"], w["tile_m"], w["tile_n"], w["split_k"]) == (nv.PATH_WSPLIT, 128, 64, 3)
    s = nv.plan(9, 256, 6144)
    assert (s["path"], s["split_k"], s["source"]) == (nv.PATH_SKINNY, 2, nv.PLAN_TABLE)
    # the mid-size kernel's small tiles: codes 16 (32 x 32) and 32 (64 x 32)
    w = nv.plan(256, 768, 8192)
    assert (w["path"], w["tile_m"], w["tile_n"], w["tile"], w["source"]) == \
        (nv.PATH_WSPLIT, 32, 32, 16, nv.PLAN_TABLE)
    w = nv.plan(512, 768, 8192)
    assert (w["tile_m"], w["tile_n"], w["tile"], w["split_k"]) == (64, 32, 32, 2)
    g = nv.plan(3, 768, 6144)
    assert (g["path"], g["source"]) == (nv.PATH_GEMV, nv.PLAN_TABLE)


def test_clear_gives_the_rules_back(base):
    nv.clear_plan_table()
    assert nv.plan(4096, 2048, 6144)["source"] == nv.PLAN_HEURISTIC


def test_tile_zero_means_the_paths_default(tmp_path, no_table):
    assert load(write(tmp_path, table([entry(16384, 8192, 8192, "tile", 0, 1),
                                       entry(600, 4096, 4096, "wsplit", 0, 1)])))[0] == nv.OK
    assert nv.plan(16384, 8192, 8192)["tile_m"] == 256
    assert nv.plan(600, 4096, 4096)["tile_m"] == 64


def test_later_entry_replaces_earlier(tmp_path, no_table):
    path = write(tmp_path, table([entry(64, 64, 1024, "wsplit", 64, 1),
                                  entry(64, 64, 1024, "tile", 64, 2)]))
    assert load(path)[0] == nv.OK
    p = nv.plan(64, 64, 1024)
    assert (p["path"], p["split_k"]) == (nv.PATH_TILE, 2)


def test_build_id_is_compared(tmp_path, no_table):
    assert len(nv.build_id()) == 16
    st, _, same = load(write(tmp_path, table([], build=nv.build_id())))
    assert (st, same) == (nv.OK, 1)
    st, _, same = load(write(tmp_path, table([], build="0123456789abcdef")))
    assert (st, same) == (nv.OK, 0)
    st, _, same = load(write(tmp_path, {k: v for k, v in table([]).items() if k != "build"}))
    assert (st, same) == (nv.OK, 0)


def test_json_details_are_accepted(tmp_path, no_table):
    doc = ('{"format":"nvfp4-plan-table","version":1.0,"arch":"gfx\\u0039\\u00350",'
           '"note":"caf\\u00e9 \\"x\\" \\/ \\\\","nested":{"a":[1,-2.5e3,true,false,null,{}]},'
           '"entries":[ {"M":64,"N":64,"K":128,"path":"tile","tile":64,"split_k":2E0,'
           '"us":1.25e-1} ] }\n')
    assert load(write(tmp_path, doc))[:2] == (nv.OK, 1)
    assert nv.plan(64, 64, 128)["source"] == nv.PLAN_TABLE


BAD_DOCS = {
    "empty file": "",
    "not an object": "[]",
    "trailing comma": '{"format":"nvfp4-plan-table","version":1,"arch":"gfx950","entries":[],}',
    "missing brace": '{"format":"nvfp4-plan-table","version":1,"arch":"gfx950","entries":[]',
    "leading zero": '{"format":"nvfp4-plan-table","version":01,"arch":"gfx950","entries":[]}',
    "bare word": '{"format":nvfp4,"version":1,"arch":"gfx950","entries":[]}',
    "unterminated string": '{"format":"nvfp4-plan-table',
    "raw newline in string": '{"format":"nvfp4-plan\ntable","version":1,"arch":"gfx950","entries":[]}',
    "bad escape": '{"format":"nvfp4\\q","version":1,"arch":"gfx950","entries":[]}',
    "text after the value": '{"format":"nvfp4-plan-table","version":1,"arch":"gfx950","entries":[]} x',
    "too deep": '{"format":"nvfp4-plan-table","version":1,"arch":"gfx950","entries":[],"x":'
                + "[" * 40 + "]" * 40 + "}",
}
BAD_TABLES = {
    "other format": table([], format="something-else"),
    "version 2": table([], version=2),
    "no entries": {k: v for k, v in table([]).items() if k != "entries"},
    "entries not a list": table({}),
    "unknown path": [entry(64, 64, 128, "simd")],
    "tile the path lacks": [entry(64, 64, 128, "tile", 96)],
    "wsplit tile 256": [entry(64, 64, 128, "wsplit", 256)],
    "wsplit tile 48": [entry(64, 64, 128, "wsplit", 48)],
    "skinny tile": [entry(8, 64, 128, "skinny", 16)],
    "skinny above 64 rows": [entry(65, 64, 128, "skinny")],
    "gemv above 4 rows": [entry(5, 64, 128, "gemv")],
    "split_k 0": [entry(64, 64, 128, "tile", 64, 0)],
    "split_k missing": [{"M": 64, "N": 64, "K": 128, "path": "tile", "tile": 64}],
    "K not a multiple of 16": [entry(64, 64, 120, "tile", 64)],
    "fractional M": [entry(64.5, 64, 128, "tile", 64)],
    "M zero": [entry(0, 64, 128, "tile", 64)],
    "N too large": [entry(64, 2 ** 31, 128, "tile", 64)],
    "path not a string": [entry(64, 64, 128, 1)],
    "entry not an object": [[64, 64, 128]],
}


@pytest.mark.parametrize("name", sorted(BAD_DOCS) + sorted(BAD_TABLES))
def test_bad_files_are_rejected_and_keep_the_old_table(base, tmp_path, name):
    if name in BAD_DOCS:
        doc = BAD_DOCS[name]
    else:
        t = BAD_TABLES[name]
        doc = table(t) if isinstance(t, list) else t
    assert load(write(tmp_path, doc, "bad.json"))[0] == nv.ERR_INVALID_VALUE, name
    assert nv.plan(4096, 2048, 6144)["source"] == nv.PLAN_TABLE


def test_other_arch_and_missing_file(base, tmp_path):
    assert load(write(tmp_path, table([], arch="gfx942")))[0] == nv.ERR_UNSUPPORTED
    assert load(str(tmp_path / "missing.json"))[0] == nv.ERR_INVALID_VALUE
    assert nv.lib().nvfp4_plan_table_load(None, None, None) == nv.ERR_INVALID_VALUE
    assert nv.plan(4096, 2048, 6144)["source"] == nv.PLAN_TABLE


def test_python_loader_raises_and_warns(tmp_path, no_table):
    with pytest.raises(nv.Nvfp4Error):
        nv.load_plan_table(write(tmp_path, "{", "broken.json"))
    with pytest.warns(UserWarning, match="other kernels"):
        assert nv.load_plan_table(write(tmp_path, table([entry(64, 64, 128, "tile", 64)]))) \
            == (1, False)


def test_environment_selects_the_table(tmp_path, monkeypatch, no_table):
    path = write(tmp_path, table([entry(64, 64, 1024, "tile", 64, 3)], build=nv.build_id()))
    monkeypatch.setenv("NVFP4_PLAN_TABLE", path)
    assert nv.load_default_plan_table() == 1
    assert nv.plan(64, 64, 1024)["split_k"] == 3
    nv.clear_plan_table()
    monkeypatch.setenv("NVFP4_PLAN_TABLE", "off")
    assert nv.load_default_plan_table() == 0
    assert nv.plan(64, 64, 1024)["source"] == nv.PLAN_HEURISTIC


def test_shipped_table_is_valid():
    """The table written by the tuner: it loads, covers the benchmark
    workloads, and every entry names a plan the library accepts."""
    if not os.path.exists(nv.PLAN_TABLE_PATH):
        pytest.skip("no tuned table shipped")
    doc = json.load(open(nv.PLAN_TABLE_PATH))
    st, n, _ = load(nv.PLAN_TABLE_PATH)
    assert st == nv.OK and n == len(doc["entries"]) > 0
    for e in doc["entries"]:
        p = nv.plan(e["M"], e["N"], e["K"])
        assert p["source"] == nv.PLAN_TABLE
        assert nv.PATH_NAMES[p["path"]] == e["path"]
        # only plans whose parity the GPU tests check
        assert plan_cases.tested(e["path"], e["tile"], e["split_k"]), e
    for M, N, K in [(1, 768, 6144), (16, 256, 6144), (512, 768, 6144), (512, 2048, 6144),
                    (16384, 8192, 8192)]:
        assert nv.plan(M, N, K)["source"] == nv.PLAN_TABLE, (M, N, K)
