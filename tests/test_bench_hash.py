"""The hash that ties the recorded HBM counters (profiles/hbm_traffic.txt) to
the tiled kernel's code: comments and layout do not change it, code does, and
the committed record matches the current sources."""
import bench

SRC = """// kernel
int f(int x) {   /* block
                    comment */
    return x + 1;   // trailing
}
"""


def test_comments_and_whitespace_do_not_change_the_hash():
    edited = SRC.replace("// kernel", "// the kernel, reworded").replace("/* block", "/* other").replace(
        "x + 1;", "x  +  1;")
    assert bench.code_hash([SRC]) == bench.code_hash([edited])


def test_code_changes_change_the_hash():
    assert bench.code_hash([SRC]) != bench.code_hash([SRC.replace("x + 1", "x + 2")])
    assert bench.code_hash([SRC]) != bench.code_hash([SRC.replace("return", "return -")])
    # file order matters: the sources are hashed in sequence
    assert bench.code_hash([SRC, "int g;"]) != bench.code_hash(["int g;", SRC])


def test_committed_traffic_record_matches_the_sources():
    assert bench.recorded_traffic("i8_4096x4096x4096") is not None
