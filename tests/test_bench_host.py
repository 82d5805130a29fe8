"""CPU: host-side logic of bench.py: whether a profile summary applies, and the parity sample.

A committed rocprofv3 summary carries the sha256 of the forward's code it was
taken on; bench.py reports its traffic only while the code is unchanged.
Comments and layout do not change the code, so they must not change the hash;
any change to the code itself must.
"""

import bench


def test_comments_and_layout_are_ignored():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    b = "/* doc */ int f(int x) { return x + 1; }"
    assert bench._code_tokens(a) == bench._code_tokens(b)


def test_code_changes_are_seen():
    a = "int f(int x) { return x + 1; }"
    for b in ("int f(int x) { return x + 2; }", "int f(int y) { return y + 1; }",
              "int f(int x) { return x - 1; }"):
        assert bench._code_tokens(a) != bench._code_tokens(b)


def test_string_literals_are_code():
    a = 'const char* s = "a // not a comment";'
    assert "not a comment" in bench._code_tokens(a)
    assert bench._code_tokens(a) != bench._code_tokens('const char* s = "a";')


def test_traffic_is_reported_only_for_the_current_code(tmp_path):
    """A summary's traffic figure is used only while the forward's code is the one it was taken on."""
    sha = bench.kernel_source_sha256()
    (tmp_path / "attn_fwd_w1.md").write_text(
        f"# x\n\ntraffic_bytes_per_launch: 12345\nkernel_source_sha256: {sha}\n")
    (tmp_path / "attn_fwd_w2.md").write_text(
        "# x\n\ntraffic_bytes_per_launch: 12345\nkernel_source_sha256: " + "0" * 64 + "\n")
    assert bench.measured_traffic("w1", str(tmp_path)) == 12345.0
    assert bench.measured_traffic("w2", str(tmp_path)) is None
    assert bench.measured_traffic("w3", str(tmp_path)) is None


def test_committed_summaries_record_their_code_and_traffic():
    """Every forward summary in profiles/ names the code hash it was taken on and its traffic."""
    import glob
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    files = glob.glob(os.path.join(root, "profiles", "attn_fwd_*.md"))
    assert files
    for f in files:
        text = open(f).read()
        assert re.search(r"^kernel_source_sha256: [0-9a-f]{64}$", text, re.M), os.path.basename(f)
        assert re.search(r"^traffic_bytes_per_launch: \d+$", text, re.M), os.path.basename(f)


def test_committed_summaries_describe_the_current_code():
    """The forward summaries were taken on the kernel code as it stands, so the bench reports traffic."""
    import glob
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sha = bench.kernel_source_sha256()
    for f in glob.glob(os.path.join(root, "profiles", "attn_fwd_*.md")):
        m = re.search(r"^kernel_source_sha256: ([0-9a-f]{64})$", open(f).read(), re.M)
        assert m and m.group(1) == sha, os.path.basename(f)
        w = os.path.basename(f)[len("attn_fwd_"):-len(".md")]
        assert bench.measured_traffic(w) is not None, w


def test_parity_sample_compares_the_heads_the_oracle_sample_computes():
    """cpu_baseline's comparison with the GPU's outputs: zero against the oracle's
    own result, and a planted error in one element is reported at its size."""
    import numpy as np

    import oracle
    from exact_attention_18_amd import inputs

    w = inputs.WORKLOADS["single_head_n256_d64"]
    x = inputs.workload_inputs(w)
    f64 = lambda t: t.float().numpy().astype(np.float64)
    o, lse = oracle.attention_forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), w.scale, w.causal)
    base, parity = bench.cpu_baseline(w, x, 5.0, got=(o, lse))
    assert base["kind"] == "oracle" and parity["heads"] == 1
    assert parity["o_max_abs"] == 0.0 and parity["lse_max_abs"] == 0.0
    o2 = o.copy()
    o2[0, 17, 0, 3] += 0.25
    lse2 = lse.copy()
    lse2[0, 0, 5] -= 0.125
    _, parity = bench.cpu_baseline(w, x, 5.0, got=(o2, lse2))
    assert abs(parity["o_max_abs"] - 0.25) < 1e-12 and abs(parity["lse_max_abs"] - 0.125) < 1e-12
    assert abs(parity["o_mean_abs"] - 0.25 / o.size) < 1e-12
    assert bench.cpu_baseline(w, x, 5.0)[1] is None
