"""The rocprofv3 summary helpers (CPU): per-kernel classification and the
per-layer span / idle-time summary, on hand-made launch sequences."""
from sparse_moe_decode_gemv_amd import profiling as P


def test_gateup_launches_are_classed_by_predecessor():
    seq = ["k1_router", "k2_gateup", "k3_slab", "k2_gateup", "k1_topk", "k2_gateup"]
    keys = P._classify(seq)
    assert keys[1] == "k2_gateup (in layer)"
    assert keys[3] == "k2_gateup (stand-alone)"
    assert keys[5] == "k2_gateup (stand-alone)"


def test_layer_spans_of_two_batch1_layers():
    names = ["k1_router", "k2_gateup", "k3_slab"] * 2
    # (name, start ns, end ns): 100 ns idle inside layer 1, 500 ns between layers
    rows = [("", 0, 4000), ("", 4100, 50000), ("", 50000, 80000),
            ("", 80500, 84000), ("", 84000, 130000), ("", 130000, 160000)]
    out = P.layer_spans(names, rows)
    assert "decode layers in the trace: 2; kernels per layer: 3 (2 layers)" in out
    assert "mean 79.75" in out          # spans 80.0 and 79.5 us
    assert "idle between a layer's kernels us: mean 0.05" in out
    assert "gap to the next layer us: mean 0.50" in out


def test_layer_spans_batched_layer_with_rmsnorm_and_foreign_kernel():
    names = ["kb_rmsnorm", "kb_router", "kb_topk", "kb_group", "kb_gateup", "kb_down_flat",
             "kb_combine", "copyBuffer", "kb_router", "kb_topk"]
    rows = [("", 1000 * i, 1000 * i + 900) for i in range(len(names))]
    out = P.layer_spans(names, rows)
    # one complete 7-kernel layer; the trailing partial layer is not counted
    assert "decode layers in the trace: 1; kernels per layer: 7 (1 layers)" in out
    assert "kb_rmsnorm > kb_router > kb_topk > kb_group > kb_gateup > kb_down_flat > kb_combine" in out


def test_no_layer_in_trace():
    assert P.layer_spans(["copyBuffer"], [("", 0, 10)]) == "no complete decode layer in the trace"


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n")
        for d, name, grid, v in rows:
            f.write(f'{d},"{name}",{grid},{counter},{v}\n')


def test_counter_calibration_uses_the_largest_copy(tmp_path):
    """Two copies with the same (capped) grid: the 1 GiB calibration copy and
    a small one.  The scale comes from the 1 GiB copy alone."""
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    rows_f = [(1, "copyBuffer", 131072, 524288.0), (2, "copyBuffer", 131072, 7000.0),
              (3, "kb_gateup", 768, 1000.0), (4, "kb_gateup", 768, 3000.0)]
    rows_w = [(1, "copyBuffer", 131072, 1048576.0), (2, "copyBuffer", 131072, 14000.0),
              (3, "kb_gateup", 768, 10.0), (4, "kb_gateup", 768, 30.0)]
    _counter_csv(fetch, "FETCH_SIZE", rows_f)
    _counter_csv(write, "WRITE_SIZE", rows_w)
    out = P.counters(str(fetch), str(write))
    assert "fetch_scale: 2.0000" in out and "write_scale: 1.0000" in out
    # mean of the two launches: 2000 KiB fetched x 2 + 20 KiB written
    line = [l for l in out.splitlines() if l.startswith("kb_gateup")][0]
    assert line.split()[-1] == str((2000 * 2 + 20) * 1024)


def test_source_digest_follows_code_not_comments(tmp_path, monkeypatch):
    """The digest that ties a profile summary to the kernels changes with the
    code of the source or of a header it compiles with, not with comments or
    blank space."""
    from sparse_moe_decode_gemv_amd import profiling as P
    src, hdr = tmp_path / "k.hip", tmp_path / "h.h"
    hdr.write_text("int f();\n")
    monkeypatch.setattr(P, "KERNEL_HEADERS", [str(hdr)])
    src.write_text("__global__ void k(int* p) { p[0] = 1; }  // store one\n")
    d0 = P.source_digest(str(src))
    src.write_text("/* a kernel */\n__global__ void k(int* p) {\n  p[0] = 1;\n}\n")
    assert P.source_digest(str(src)) == d0
    src.write_text("__global__ void k(int* p) { p[0] = 2; }\n")
    assert P.source_digest(str(src)) != d0
    src.write_text("__global__ void k(int* p) { p[0] = 1; }\n")
    hdr.write_text("int f(int);\n")
    assert P.source_digest(str(src)) != d0
