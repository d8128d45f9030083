"""Host-side checks of the profile summariser: the source hash that tells
bench.py whether the committed counters still describe the kernels."""
from gated_delta_rule_prep_amd import prof_summary as ps


def test_code_only_drops_comments_and_layout():
    src = 'int a = 1;  // one\n/* block\n comment */ const char* s = "//kept /* too */";\nchar c = \'/\';\n\tint  b;'
    assert ps.code_only(src) == 'int a = 1; const char* s = "//kept /* too */"; char c = \'/\'; int b;'


def test_code_only_keeps_code_changes():
    assert ps.code_only("x = a / b; // c") != ps.code_only("x = a * b; // c")
    assert ps.code_only("x = a/b;") == ps.code_only("x = a/b; /* same code */")


def test_source_hash_is_stable_and_covers_every_kernel_source():
    import os
    h = ps.source_hash()
    assert h == ps.source_hash() and len(h) == 16
    for rel in ps.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ps.HERE, rel)), rel


def test_stats_name_keeps_template_arguments():
    assert ps.stats_name("void kda::(anonymous namespace)::recur_kernel<4, 4, 0>(kda::RecurArgs)") == \
        "recur_kernel<4,4,0>"
    assert ps.stats_name("kda::(anonymous namespace)::prep_kernel(kda::PrepArgs)") == "prep_kernel"
