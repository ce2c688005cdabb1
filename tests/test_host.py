"""Host-side logic of the measurement tools (no GPU): the code digest that
keys stored traffic measurements, and the markdown formatting of bench
output lines."""

import json

from io_aware_softmax_02_amd.profile_summary import code_digest, configs_md


def test_code_digest_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {  // one\n  return x + 1;  /* two\n lines */\n}\n")
    b.write_text("int f(int x) {\n\treturn x + 1; // another comment\n}")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert code_digest(str(a)) == code_digest(str(b))
    assert code_digest(str(a)) != code_digest(str(c))


def test_code_digest_sees_every_kernel_source_change(tmp_path):
    # a one-character change of code in a real kernel source changes the digest
    import io_aware_softmax_02_amd.profile_summary as ps
    import os
    src = os.path.join(ps.ROOT, "io_aware_softmax_02_amd", "csrc", "attn_fwd_bf16.hip")
    text = open(src, encoding="utf-8").read()
    p = tmp_path / "k.hip"
    p.write_text(text)
    d0 = code_digest(str(p))
    p.write_text(text.replace("constexpr float kSlack = 8.0f;", "constexpr float kSlack = 7.0f;"))
    assert code_digest(str(p)) != d0
    p.write_text(text + "\n// trailing comment\n")
    assert code_digest(str(p)) == d0


def test_configs_markdown(tmp_path):
    line = {"workload": "w", "B": 1, "H": 2, "N": 3, "d": 64, "dtype": "bf16", "launches": 1,
            "ms_fwd": 0.5, "ms_bwd": 1.5, "fwd_tflops": 100.0, "fwdbwd_tflops": 250.0,
            "peak_tflops": 2500.0}
    log = tmp_path / "log"
    log.write_text("noise\n" + json.dumps(line) + "\n")
    md = configs_md(str(log))
    row = [r for r in md.splitlines() if r.startswith("| `w`")]
    assert row == ["| `w` | 1, 2, 3, 64 | bf16 | 500.0 | 100.0 | 1500.0 | 250.0 | 10.0 |"]
