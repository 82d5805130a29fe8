"""CPU: host-side logic of bench.py that decides whether a profile summary applies.

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


def test_committed_summaries_match_the_current_code():
    """The forward summaries in profiles/ were taken on the code as it stands."""
    import glob
    import os
    sha = bench.kernel_source_sha256()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    files = glob.glob(os.path.join(root, "profiles", "attn_fwd_*.md"))
    assert files
    for f in files:
        assert f"kernel_source_sha256: {sha}" in open(f).read(), os.path.basename(f)
