"""Host logic of bench.py that feeds its JSON line: the unique K/V bytes of
shared-prefix tables, the keys of the HBM counter records, and the choice of
the calibration copy in a counter CSV.  CPU only."""
import argparse
import csv

import numpy as np

import bench
import workloads


def test_unique_bytes_count_shared_prefix_blocks_once():
    bs, pre = 16, 64
    c = workloads.make_case("unique", 3, [pre + 5, pre + 20, pre + 1], 4, 2, 64, bs,
                            q_dtype="bf16", cache_dtype="bf16", prefix_len=pre)
    per_slot = c.Hkv * c.D * 2 * 2                     # K and V, 2-byte elements
    tails = int((c.seq_lens - pre).sum())
    assert bench.unique_kv_bytes(c) == (pre + tails) * per_slot
    assert bench.decode_bytes(c, 0)["kv"] == int(c.seq_lens.sum()) * per_slot


def test_unique_bytes_equal_logical_bytes_without_sharing():
    c = workloads.make_case("plain", 4, [7, 16, 33], 4, 4, 64, 16, q_dtype="f32",
                            cache_dtype="f32")
    assert bench.unique_kv_bytes(c) == bench.decode_bytes(c, 0)["kv"]


def test_traffic_keys():
    ns = argparse.Namespace
    assert bench.traffic_key(ns(workload="llama3-8b-gqa", partition=None), 16) == "llama3-8b-gqa"
    assert bench.traffic_key(ns(workload="shared-prefix-fp8", partition=None), 8) == \
        "shared-prefix-fp8-bs8"
    assert bench.traffic_key(ns(workload="long-context-gqa", partition=512), 32) == \
        "long-context-gqa-P512"
    assert bench.traffic_key(ns(workload="shared-prefix-fp8", partition=-1), 16) == \
        "shared-prefix-fp8-bs16-P-1"
    assert bench.decode_kernel_name(-1) == "decode_balanced_kernel"
    assert bench.decode_kernel_name(512) == "decode_mfma_kernel"


def test_chunk_floor_is_two_rounds_of_the_ring():
    """The floor bench.py replays the balanced split with: two rounds of the
    decode's tile ring (10 tiles for fp8, 6 for 16-bit D = 128, 8 for D = 64,
    half of that with 8-token blocks)."""
    assert bench.chunk_floor("bf16", 16, 128) == 12
    assert bench.chunk_floor("f16", 32, 64) == 16
    assert bench.chunk_floor("fp8", 16, 128) == 20
    assert bench.chunk_floor("fp8", 8, 128) == 10
    assert bench.chunk_floor("bf16", 8, 128) == 8


def test_balanced_split_replay_counts_split_streams():
    """Two streams of 10 tiles on 2 waves: T = 20, A = 10, C1 = 8, so the
    schedule cuts at 8 and 16.  Both cuts separate fixed first-phase chunks,
    which move only within an eighth of the smaller neighbour (1 tile and
    0): the cut at 8 lies 2 tiles before stream 0's end and stays.  Stream 0
    spans chunks 0-1, stream 1 chunks 1-2: 2 split streams, 4 entries,
    whatever the floor (the last chunk is the 4 tiles left)."""
    lens = np.array([160], np.int64)                 # 10 tiles per stream
    assert bench.balanced_split(lens, 2, 2, 4) == (2, 4)
    assert bench.balanced_split(lens, 2, 2, 20) == (2, 4)
    assert bench.balanced_split(np.array([0], np.int64), 2, 2, 12) == (0, 0)


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Value": v})


def test_calibration_copy_is_the_last_copy_before_the_kernel(tmp_path):
    """Pool uploads and clones can be larger than the calibration copy; the
    copy made right before the first decode dispatch is the calibration."""
    p = tmp_path / "c.csv"
    k = "void pkv::decode_balanced_kernel<pkv::BF16>(pkv::DecodeParams)"
    _write_csv(p, [("__amd_rocclr_copyBuffer", 1500.0),      # a pool clone
                   ("__amd_rocclr_copyBuffer", 1000.0),      # the calibration copy
                   (k, 10.0), ("__amd_rocclr_copyBuffer", 9999.0), (k, 14.0)])
    mean, calib, n = bench._counter_means(str(p), "decode_balanced_kernel")
    assert (mean, calib, n) == (12.0, 1000.0, 2)
