"""Host-side parts of bench.py's measurement contract (no GPU): the one-GPU
refusal, the kernel-source hash that ties committed counter summaries to the
sources they were taken on, and the summaries' machine-readable blocks."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_code_only_drops_comments_and_blank_lines_only():
    src = 'int a = 1;  // note\n\n/* block\n comment */ int b = 2;\nconst char* s = "// kept";\n'
    assert bench._code_only(src) == 'int a = 1;\n int b = 2;\nconst char* s = "// kept";'
    # a comment edit leaves the code text as it is; a code edit does not
    assert bench._code_only(src.replace("note", "other note")) == bench._code_only(src)
    assert bench._code_only(src.replace("= 2", "= 3")) != bench._code_only(src)


def test_kernel_sources_cover_every_kernel_file():
    csrc = os.path.join(ROOT, "bit_weight_only_q4g64_amd", "csrc")
    on_disk = sorted(f for f in os.listdir(csrc) if f.endswith((".h", ".hip")))
    assert [os.path.basename(p) for p in bench.KERNEL_SOURCES] == on_disk
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_source_hash() == h


def test_traffic_is_reported_only_for_matching_sources(monkeypatch):
    data = bench.summary_json("traffic_ffn_flow_step.md")
    assert data is not None and data["hbm_bytes_per_launch"] > 0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: data["kernel_source_hash"])
    assert bench.traffic_per_launch("ffn_flow_step") == data["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.traffic_per_launch("ffn_flow_step") is None
    assert bench.traffic_per_launch("no_such_kernel") is None


def test_profile_summaries_parse_and_name_their_command():
    names = sorted(f for f in os.listdir(bench.PROFILES) if f.endswith(".md"))
    assert names
    for name in names:
        with open(os.path.join(bench.PROFILES, name), encoding="utf-8") as f:
            text = f.read()
        assert "rocprofv3" in text, name
        if "```json" in text:
            data = bench.summary_json(name)
            assert isinstance(data, dict), name
            assert len(data.get("kernel_source_hash", "")) == 16, name
