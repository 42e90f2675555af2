"""Host-side pieces of bench.py that decide what its JSON line reports: the
source hash that ties a committed counter summary to the kernel code it was
taken on (comments and layout do not count, code does)."""
import os
import shutil

import pytest

import bench


@pytest.fixture()
def csrc_copy(tmp_path, monkeypatch):
    dst = tmp_path / "csrc"
    shutil.copytree(bench.CSRC, dst)
    monkeypatch.setattr(bench, "CSRC", str(dst))
    return dst


def _edit(path, fn):
    text = open(path, encoding="utf-8").read()
    open(path, "w", encoding="utf-8").write(fn(text))


def test_source_hash_ignores_comments_and_layout(csrc_copy):
    before = {k: bench.source_hash(k) for k in ("select_kernel", "pair_kernel", "pair_hist_kernel", None)}
    f = os.path.join(csrc_copy, "sv_finish.h")
    _edit(f, lambda t: t.replace("// Per-sequence finisher", "// A reworded comment:\n//   per-sequence finisher", 1))
    _edit(f, lambda t: t + "\n/* a block\n   comment */\n\n   \n")
    _edit(os.path.join(csrc_copy, "sv_wave.h"), lambda t: t.replace("{\n", "{  \n", 3))
    after = {k: bench.source_hash(k) for k in before}
    assert after == before


def test_source_hash_follows_code(csrc_copy):
    before = bench.source_hash("select_kernel")
    _edit(os.path.join(csrc_copy, "sv_wave.h"), lambda t: t.replace("constexpr int SCAP = 128;", "constexpr int SCAP = 96;", 1))
    assert bench.source_hash("select_kernel") != before


def test_traffic_needs_a_matching_hash(csrc_copy, tmp_path, monkeypatch):
    # A counter summary stamped with the tree's hash gives the traffic field;
    # after a code change the same summary gives null rather than stale bytes.
    w = "B256-V152064-g7-T0.7-topk64"
    name = bench.PMC_SUMMARIES[("select_kernel", w)]
    root = tmp_path / "root"
    (root / "profiles").mkdir(parents=True)
    (root / "profiles" / name).write_text(
        "# synthetic summary\n"
        f"source_hash = {bench.source_hash('select_kernel')}\n"
        "hbm_read_bytes_per_launch = 1000\n"
        "hbm_write_bytes_per_launch = 24\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.traffic_from_profile("select_kernel", w) == 1024
    _edit(os.path.join(csrc_copy, "sv_wave.h"), lambda t: t.replace("constexpr int SCAP = 128;", "constexpr int SCAP = 96;", 1))
    assert bench.traffic_from_profile("select_kernel", w) is None
