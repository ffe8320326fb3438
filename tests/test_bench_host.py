"""bench.py's host logic (no GPU needed):
* more than one GPU is refused with exit status 2 and a message;
* the kernel-source digest ignores comments and whitespace but not code;
* the committed traffic summary is read only while its digest is current.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8"],
                                  ["--op", "ce", "--gpus", "2"]])
def test_more_than_one_gpu_is_refused(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _with_sources(monkeypatch, tmp_path, texts):
    csrc = tmp_path / "linear_cross_entropy_06_amd" / "csrc"
    csrc.mkdir(parents=True, exist_ok=True)
    names = []
    for i, t in enumerate(texts):
        (csrc / f"k{i}.hip").write_text(t)
        names.append(f"k{i}.hip")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", tuple(names))
    return bench.sources_digest()


def test_digest_ignores_comments_and_whitespace(monkeypatch, tmp_path):
    code = "int f(int x) {\n  return x + 1;\n}\n"
    d0 = _with_sources(monkeypatch, tmp_path / "a", [code])
    d1 = _with_sources(monkeypatch, tmp_path / "b",
                       ["// a comment\nint f(int x) {  /* inline */\n\n  return x + 1;  // why\n}\n"])
    d2 = _with_sources(monkeypatch, tmp_path / "c", [code.replace("+ 1", "+ 2")])
    assert d0 == d1
    assert d0 != d2


def test_traffic_is_read_only_for_current_sources(monkeypatch):
    text = open(bench.TRAFFIC_FILE).read()
    digest = text.split("sources_digest:")[1].split()[0]
    monkeypatch.setattr(bench, "sources_digest", lambda: digest)
    for step in ("logits_gemm", "ce_rows", "grad_h_gemm", "grad_W_gemm"):
        v = bench.read_traffic(step, "llama3_8b_head")
        assert v is not None and v > 1e9, (step, v)
    assert bench.read_traffic("loss_sum", "llama3_8b_head") is None   # not listed
    assert bench.read_traffic("grad_W_gemm", "other_workload") is None
    monkeypatch.setattr(bench, "sources_digest", lambda: "0" * 16)
    assert bench.read_traffic("grad_W_gemm", "llama3_8b_head") is None

