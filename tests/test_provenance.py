"""The identity under which stored counter measurements are kept: it follows the kernel
code and ignores comments and layout."""
from exact_tiled_attention_08_amd import provenance as P


def test_comments_and_layout_do_not_change_the_code_text():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    b = "/* header */\nint f(int x)\n{\n    return x + 1; /* one\n more */\n}"
    assert P.code_text(a) == P.code_text(b)


def test_a_code_change_changes_the_code_text():
    a = "int f(int x) { return x + 1; }"
    assert P.code_text(a) != P.code_text(a.replace("+ 1", "+ 2"))
    assert P.code_text(a) != P.code_text(a.replace("int f", "intf"))


def test_every_kind_hashes_its_sources():
    for kind, files in P.KERNEL_SOURCES.items():
        assert files and len(P.source_hash(kind)) == 16
