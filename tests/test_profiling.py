"""Host checks of the profile-summary helpers (no GPU)."""
from dense_fp16_gemm_nt_amd import profiling


def test_code_only_drops_comments_and_blank_lines():
    src = "int a;  // trailing\n\n/* block\n comment */ int b;\n// whole line\nint c; /* x */\n"
    assert profiling._code_only(src) == "int a;\n int b;\nint c;"


def test_source_hash_is_stable_and_short():
    h = profiling.kernel_source_hash()
    assert h == profiling.kernel_source_hash() and len(h) == 16 and int(h, 16) >= 0
