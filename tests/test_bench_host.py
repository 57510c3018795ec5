"""Host-side checks of bench.py's accounting (no GPU): the algorithmic flop and byte counts per
token-head against a tile-by-tile enumeration of the chunked form, the counter calibration that
turns rocprofv3 FETCH_SIZE / WRITE_SIZE readings into HBM bytes, the source-hash gate on stored
counters, and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _enumerated_flops(dk, dv, C):
    """Flops of one chunk of C tokens, product by product, divided by C.  Every product whose
    left factor is lower triangular over the chunk (M, A, T and their uses) runs over the causal
    16x16 sub-tiles only; the state products are dense; the triangular solve is counted as
    C^3 / 3 (forward substitution)."""
    nt = C // 16
    causal_tiles = nt * (nt + 1) // 2
    tile_elems = 16 * 16
    m = causal_tiles * tile_elems * dk * 2        # M = (Q Gamma)(K Gamma^-1)^T
    a = causal_tiles * tile_elems * dk * 2        # A = diag(beta) (K Gamma)(K Gamma^-1)^T
    solve = C ** 3 / 3.0                          # T = (I + A)^-1
    w = causal_tiles * tile_elems * dk * 2        # W = T diag(beta) K~
    u_tilde = causal_tiles * tile_elems * dv * 2  # U~ = T diag(beta) V
    w_s = C * dk * dv * 2                         # W S
    k_u = C * dk * dv * 2                         # K^T U
    q_s = C * dk * dv * 2                         # Q~ S
    m_u = causal_tiles * tile_elems * dv * 2      # M U
    return (m + a + solve + w + u_tilde + w_s + k_u + q_s + m_u) / C


@pytest.mark.parametrize("dk,dv,C", [(128, 128, 64), (64, 64, 16), (128, 64, 32), (64, 128, 64)])
def test_flops_per_token_head_matches_the_enumeration(dk, dv, C):
    assert bench.flops_per_token_head(dk, dv, C) == pytest.approx(_enumerated_flops(dk, dv, C), rel=1e-12)


def test_flops_and_bytes_at_the_64k_workload():
    # 150,869 flop and 1,282 B per token-head (d = 128, chunk 64, bf16): intensity about 118 flop/B
    assert bench.flops_per_token_head(128, 128, 64) == pytest.approx(9655637.333333334 / 64)
    tensors_read = {"q": 128, "k": 128, "a": 128, "v": 128, "beta": 1}
    tensors_written = {"out": 128}
    elems = sum(tensors_read.values()) + sum(tensors_written.values())
    assert bench.path_bytes_per_token_head(128, 128, 2) == 2 * elems == 1282
    assert bench.path_bytes_per_token_head(64, 64, 4) == 4 * (3 * 64 + 64 + 64 + 1)


def _write_counters(d, rows):
    os.makedirs(os.path.join(d, "vm"), exist_ok=True)
    with open(os.path.join(d, "vm", "1_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, c, v) in enumerate(rows):
            wr.writerow([i, k, c, v])


def test_record_traffic_calibrates_each_counter_by_the_copy(tmp_path, monkeypatch):
    copy = 1 << 30
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>"
    intra = "void kda::kda_intra_kernel<64, 128, 128, false, false, 0>(...)"
    pass0 = "void kda::kda_seg_state_kernel<64, 128, 128, false, 0>(...)"
    pass1 = "void kda::kda_seg_state_kernel<64, 128, 128, false, 1>(...)"
    scan = "void kda::kda_seg_scan_kernel<128, 128>(...)"
    # the copy's FETCH_SIZE reads half its true bytes (factor 2), its WRITE_SIZE all of them; the
    # state stage is three kernels per step, each averaged over its own dispatches
    _write_counters(fetch, [(neg, "FETCH_SIZE", copy / 2048.0), (intra, "FETCH_SIZE", 1000.0),
                            (intra, "FETCH_SIZE", 1100.0), (pass0, "FETCH_SIZE", 200.0), (pass0, "FETCH_SIZE", 220.0),
                            (scan, "FETCH_SIZE", 10.0), (pass1, "FETCH_SIZE", 500.0)])
    _write_counters(write, [(neg, "WRITE_SIZE", copy / 1024.0), (intra, "WRITE_SIZE", 2000.0),
                            (intra, "WRITE_SIZE", 2000.0), (pass0, "WRITE_SIZE", 5.0), (scan, "WRITE_SIZE", 4.0),
                            (pass1, "WRITE_SIZE", 300.0)])
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_src_sha", lambda: "feedface")
    bench.record_traffic(fetch, write, "64k", copy)
    rec = json.load(open(tmp_path / "profiles" / "traffic.json"))
    i, s = rec["kda_intra_kernel@64k"], rec["state_stage@64k"]
    assert i["fetch_size_factor"] == pytest.approx(2.0) and i["write_size_factor"] == pytest.approx(1.0)
    assert i["bytes_per_launch"] == pytest.approx(1050.0 * 1024 * 2 + 2000.0 * 1024)
    assert s["bytes_per_launch"] == pytest.approx((210.0 + 10.0 + 500.0) * 1024 * 2 + (5.0 + 4.0 + 300.0) * 1024)
    assert i["kernels"] == 1 and s["kernels"] == 3 and i["src_sha"] == "feedface"
    # the stored figure is reported only for the sources it was taken on
    assert bench._traffic("state_stage", "64k") == pytest.approx(s["bytes_per_launch"])
    monkeypatch.setattr(bench, "_src_sha", lambda: "0ddba11")
    assert bench._traffic("state_stage", "64k") is None


def test_record_traffic_needs_the_calibration_copy(tmp_path, monkeypatch):
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    _write_counters(fetch, [("kda_intra_kernel", "FETCH_SIZE", 1.0), ("kda_seg_state_kernel", "FETCH_SIZE", 1.0)])
    _write_counters(write, [("kda_intra_kernel", "WRITE_SIZE", 1.0), ("kda_seg_state_kernel", "WRITE_SIZE", 1.0)])
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    with pytest.raises(SystemExit):
        bench.record_traffic(fetch, write, "64k", 1 << 30)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("B,H,T,d,C,es", [(1, 32, 65536, 128, 64, 2), (1, 8, 1048576, 128, 64, 2),
                                          (1, 16, 262144, 128, 64, 2), (4, 16, 8192, 128, 64, 2),
                                          (1, 2, 256, 64, 16, 4), (1, 3, 512, 64, 32, 2), (4, 64, 8192, 128, 64, 2),
                                          (1, 16, 65536, 128, 64, 4), (1, 31, 2048, 128, 64, 2)])
def test_record_layout_and_segments_match_the_library(B, H, T, d, C, es):
    # the workspace is the records plus, with several segments, two float32 maps per segment and head
    import torch
    import chunked_gated_linear_bounded_amd as kda
    L = bench.record_layout(d, d, C, es)
    units, nc = B * H, T // C
    nseg = bench.seg_count(units, nc) if bench.use_segmented(units, d, d, C, es) else 1
    extra = 0 if nseg == 1 else units * (nseg + nseg - 1) * d * d * 4
    want = units * nc * L["stride"] + extra
    assert kda.workspace_bytes(B, H, T, d, d, C, torch.float32 if es == 4 else torch.bfloat16) == want
    assert nseg * units <= max(256, units) and (nseg == 1 or -(-nc // nseg) >= 8)


def test_segment_counts_of_the_workloads():
    # 256 (head, segment) work-groups for the large workloads, one segment at 256 heads or more
    assert [bench.seg_count(u, nc) for (u, nc) in ((32, 1024), (16, 4096), (8, 16384), (64, 128), (256, 128))] == \
        [8, 16, 32, 4, 1]
    assert bench.seg_count(2, 16) == 2 and bench.seg_count(2, 15) == 1 and bench.seg_count(3, 100) == 12


def test_state_stage_choice():
    # per-slice where its (head, value slice) work-groups fill 256 compute units (64k: 32 x 8; 8k:
    # 64 x 8), segmented below that (256k: 16 heads, 1m: 8) and from 256 heads on; fp32 records of
    # 64-token chunks at d = 128 do not fit the segmented stage's ring twice
    assert [bench.use_segmented(u, 128, 128, 64, 2) for u in (32, 64, 16, 8, 31, 255, 256)] == \
        [False, False, True, True, True, False, True]
    assert not bench.use_segmented(16, 128, 128, 64, 4)
    assert bench.use_segmented(2, 64, 64, 16, 4) and bench.use_segmented(16, 128, 128, 32, 4)
