"""HBM context measurements for the decode kernels' roofline (not the decode path).

    python -m gqa_kv_cache_attn_amd.hbm_probe [--mode read|copy|both] [--gib 2] [--iters 20]

read: streaming reads of a buffer far larger than the caches (grid-stride,
      contiguous chunks, and the decode kernels' persistent split through
      bounded buffer descriptors), over several grid sizes and load depths;
      the best average is the device's practical read ceiling.
copy: a plain copy of known size (``--gib`` read + ``--gib`` written); under
      ``rocprofv3 --pmc FETCH_SIZE`` / ``WRITE_SIZE`` its counter readings
      give the scale between counter units and bytes.
Prints one JSON line.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics

import torch

from .build import PKG_DIR

PROBE_LIB = os.path.join(PKG_DIR, "libgqa_hbm_probe.so")


def _lib():
    if not os.path.exists(PROBE_LIB):
        raise ImportError(f"{PROBE_LIB} is not built; run python -m gqa_kv_cache_attn_amd.build")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.gqa_probe_read.restype = ctypes.c_int
    lib.gqa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.gqa_probe_read_chunks.restype = ctypes.c_int
    lib.gqa_probe_read_chunks.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32,
                                          ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.gqa_probe_read_split.restype = ctypes.c_int
    lib.gqa_probe_read_split.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.gqa_probe_copy.restype = ctypes.c_int
    lib.gqa_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                   ctypes.c_void_p]
    return lib


def _time(fn, iters, stream):
    evs = []
    for _ in range(iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mode", choices=["read", "copy", "both"], default="both")
    ap.add_argument("--gib", type=float, default=2.0)
    ap.add_argument("--iters", type=int, default=20)
    args = ap.parse_args()
    lib = _lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    nbytes = int(args.gib * (1 << 30)) // 16 * 16
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {"probe": "hbm", "bytes": nbytes, "device": torch.cuda.get_device_properties(dev).gcnArchName}
    if args.mode in ("read", "both"):
        best = None
        per_grid = {}
        for wgs in (1024, 2048, 4096, 8192, 16384):
            def run():
                assert lib.gqa_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), wgs, stream.cuda_stream) == 0
            run()
            ms = _time(run, args.iters, stream)
            gbps = nbytes / (statistics.fmean(ms) * 1e-3) / 1e9
            per_grid[wgs] = round(gbps, 1)
            best = max(best or 0.0, gbps)
        res["read_GBps_by_workgroups"] = per_grid
        per_chunk = {}
        for chunk_kib in (64, 256, 1024):
            for wgs in (512, 1024, 2048):
                def runk():
                    assert lib.gqa_probe_read_chunks(src.data_ptr(), nbytes, chunk_kib << 10,
                                                     sink.data_ptr(), wgs, stream.cuda_stream) == 0
                runk()
                ms = _time(runk, args.iters, stream)
                gbps = nbytes / (statistics.fmean(ms) * 1e-3) / 1e9
                per_chunk[f"{chunk_kib}KiB/{wgs}wg"] = round(gbps, 1)
                best = max(best, gbps)
        res["read_chunks_GBps"] = per_chunk
        per_split = {}
        for depth in (8, 16):
            for wgs in (256, 512, 768, 1024, 2048):
                def runs():
                    assert lib.gqa_probe_read_split(src.data_ptr(), nbytes, depth, sink.data_ptr(),
                                                    wgs, stream.cuda_stream) == 0
                runs()
                ms = _time(runs, args.iters, stream)
                gbps = nbytes / (statistics.fmean(ms) * 1e-3) / 1e9
                per_split[f"depth{depth}/{wgs}wg"] = round(gbps, 1)
                best = max(best, gbps)
        res["read_split_GBps"] = per_split
        res["read_ceiling_GBps"] = round(best, 1)
    if args.mode in ("copy", "both"):
        dst = torch.empty_like(src)

        def runc():
            assert lib.gqa_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, 8192, stream.cuda_stream) == 0
        runc()
        ms = _time(runc, args.iters, stream)
        res["copy_bytes_read_per_launch"] = nbytes
        res["copy_bytes_written_per_launch"] = nbytes
        res["copy_GBps_read_plus_write"] = round(2 * nbytes / (statistics.fmean(ms) * 1e-3) / 1e9, 1)
        res["copy_us_avg"] = round(statistics.fmean(ms) * 1e3, 2)
        torch.cuda.synchronize()
        assert torch.equal(dst[:4096], src[:4096])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
