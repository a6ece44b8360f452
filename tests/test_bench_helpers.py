"""Host-side checks of bench.py's bookkeeping (no GPU): the forward GEMM's
committed HBM-traffic counters belong to the GEMM code as it stands, and the
code hash ignores comments and whitespace but not code."""
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_committed_traffic_counters_match_the_gemm_code():
    """The profile under profiles/ was taken on this ar_gemm.hip (code hash),
    so the bench line reports its traffic instead of null. A change to the
    GEMM's code needs the FETCH_SIZE / WRITE_SIZE passes taken again."""
    t = bench._measured_traffic("llama7b_q_proj")
    assert t is not None and t > 0
    assert bench._measured_traffic("llama7b_down_proj") is None


def test_code_hash_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) {  // one\n  return x + 1; /* two */ }\n")
    b = tmp_path / "b.hip"
    b.write_text("int f(int x) {\n  // a different comment\n  return x + 1;\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.gemm_code_hash(str(a)) == bench.gemm_code_hash(str(b))
    assert bench.gemm_code_hash(str(a)) != bench.gemm_code_hash(str(c))
