"""Host-side helpers of bench.py (no GPU): the code hash that decides whether a committed counter
summary still describes the current kernels."""

import bench


def test_code_only_drops_comments_and_layout_but_keeps_literals():
    src = ('int a;  // tail "quoted"\n/* block\n   comment */ const char* s = "//kept /* kept */";\n'
           "char q = '\"'; char e = '\\''; x  =\t1;")
    assert bench.code_only(src) == ('int a; const char* s = "//kept /* kept */"; '
                                    "char q = '\"'; char e = '\\''; x = 1;")


def test_kernel_hash_ignores_comments_and_follows_code(tmp_path, monkeypatch):
    f = tmp_path / "k.hip"
    monkeypatch.setitem(bench.KERNEL_SRCS, "k_probe", [str(f)])
    f.write_text("__global__ void k(float* p) { p[0] = 1.0f; }\n")
    h0 = bench.kernel_hash("k_probe")
    f.write_text("// what k does\n__global__ void k(float* p) {\n  p[0] = 1.0f;  /* one */\n}\n")
    assert bench.kernel_hash("k_probe") == h0
    f.write_text("__global__ void k(float* p) { p[0] = 2.0f; }\n")
    assert bench.kernel_hash("k_probe") != h0


def test_every_kernel_has_a_hash_over_existing_sources():
    import os
    for k, files in bench.KERNEL_SRCS.items():
        assert files and all(os.path.exists(f) for f in files), k
        assert len(bench.kernel_hash(k)) == 16
