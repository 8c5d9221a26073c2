"""Host-side checks of the build helpers (no GPU): the fingerprint that keys recorded profiler figures to a
build ignores comments and layout, and nothing else."""
from exact_blockwise_attention_fwd_amd.build import code_text, fingerprint


def test_code_text_drops_comments_and_layout_only():
    src = 'int a = 1; // note "x"\n/* block\n note */ const char* s = "http://x // kept";\nchar c = \'"\'; // end\nint  b;'
    assert code_text(src) == 'int a = 1; const char* s = "http://x // kept"; char c = \'"\'; int b;'
    assert code_text("x = 1; // one") == code_text("x  =  1;\n// two\n")
    assert code_text("x = 1;") != code_text("x = 2;")
    assert code_text('s = "a\\"b"; // c') == 's = "a\\"b";'


def test_fingerprint_is_stable():
    a = fingerprint("attn_fwd_bf16.hip")
    assert len(a) == 64 and a == fingerprint("attn_fwd_bf16.hip")
    assert a != fingerprint("attn_merge.hip")
