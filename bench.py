"""Benchmark of the THD layout-transform hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gdn128k] [--also long1m,full]

One step is one pass of the whole hot path over one micro-batch already
resident in HBM: build the route from the padded boundaries, swap the
activations zigzag -> contiguous and back (layers x 2 swaps), and write the
document-aware label shift / MTP roll / valid mask (on a second stream of the
same priority: the roll reads only the token ids and the boundaries).  The
default workload is the GDN-style 128K batch (cp 4, T = 131072, rows
[T, 16, 128] bf16); the 1M-token batch and the 48-layer micro-batch follow
under ``workloads``, each measured the same way.

Before any timing the swap runs back to back for at least 0.25 s: the chip
raises its clocks only under sustained load, and from idle the swap needs
about 100 launches to reach its steady time.  The in-run ceilings (plain
copy, pure read and pure write streams) are measured next, then W warm-up
steps, then K timed steps.

Prints one JSON line.  ``value`` is the step's algorithmic HBM bytes (every
swap reads and writes each row once; the roll reads the ids and writes its
streams and masks) divided by the step time, in GB/s.  ``roofline`` prices the
swap kernel (the dominant kernel) against the MI355X HBM peak; its duration is
the mean, over the steps of the timed region, of the time between two HIP
timing events recorded on the swap's stream just before the step's first swap
and just after its last, divided by the step's swap count.  ``cpu_baseline``
times the CPU oracle on the host: route and swap apart, whole steps over a
bounded sample of the main workload, and the 1M-token batch on 256 MiB chunks
compared with the GPU's output.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E peak, 8 TB/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="gdn128k")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--also", default="long1m,full",
                   help="other workloads measured after the main one and reported under 'workloads' "
                        "(comma-separated, empty for none)")
    p.add_argument("--row-sweep", action="store_true",
                   help="instead of the step benchmark: swap and plain-copy bandwidth for a range of row sizes, "
                        "one JSON line per size")
    return p.parse_args()


ROW_SWEEP_BYTES = (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 40, 48, 64, 100, 112, 128, 256, 272, 400, 512, 720, 1008,
                   1024, 1536, 2048, 2560, 3072, 4000, 4096, 5120, 6144, 8192, 10240, 12288, 14336, 16384, 65536)


def row_sweep(workloads):
    """Swap bandwidth against row size: the 128K workload's document mix
    scaled so that one swap moves about 1 GiB, every row size through the
    same route shape; a plain copy of the same bytes alongside.  Each size
    first runs its swaps back to back for 0.15 s (the clocks rise only under
    sustained load), then swap pairs and copies are timed in interleaved
    samples of about 3 ms of back-to-back launches."""
    import numpy as np
    import torch

    import context_packed_sequence_amd as thd

    base = workloads.make("gdn128k")
    lens = np.diff(base.cu_padded).astype(np.int64)
    cp = base.cp
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    for rb in ROW_SWEEP_BYTES:
        scale = ((1 << 29) // rb) / lens.sum()
        new = [int(v * scale) // (2 * cp) * (2 * cp) for v in lens]
        cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
        total = int(cu[-1])
        route = thd.Route(len(new), cp, total).build(torch.from_numpy(cu).cuda(), cp, total, sh)
        g = torch.Generator(device="cuda").manual_seed(workloads.BASE_SEED + rb)
        x = torch.randint(0, 256, (total, rb), dtype=torch.uint8, device="cuda", generator=g)
        a = torch.empty_like(x)
        b = torch.empty_like(x)
        nbytes = total * rb

        def pair():
            thd.thd_swap(route.handle, thd.Z2C, x, a, total, rb, sh)
            thd.thd_swap(route.handle, thd.C2Z, a, b, total, rb, sh)

        pair()
        torch.cuda.synchronize()
        assert torch.equal(b, x), rb
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.15:
            for _ in range(10):
                pair()
            torch.cuda.synchronize()
        t_swap, t_copy = [], []
        for _ in range(8):
            t_swap += [t / 20 for t in _event_samples(torch, stream, lambda: [pair() for _ in range(10)], 1)]
            t_copy += [t / 20 for t in _event_samples(torch, stream, lambda: [thd.thd_copy(x, a, nbytes, sh)
                                                                           for _ in range(20)], 1)]
        t_swap, t_copy = float(np.median(t_swap)), float(np.median(t_copy))
        swap_gbps = 2 * nbytes / (t_swap * 1e-3) / 1e9
        copy_gbps = 2 * nbytes / (t_copy * 1e-3) / 1e9
        print(json.dumps({"row_bytes": rb, "tokens": total, "cp_size": cp, "swap_us": round(t_swap * 1e3, 2),
                          "swap_gbps": round(swap_gbps, 1), "frac_of_peak": round(swap_gbps / HBM_PEAK_GBPS, 4),
                          "copy_gbps": round(copy_gbps, 1), "swap_over_copy": round(swap_gbps / copy_gbps, 4)}),
              flush=True)
        route.close()
        del x, a, b
        torch.cuda.empty_cache()


def step_bytes(w, layers):
    swap = 2 * w.total * w.row_bytes
    roll = 0
    if w.max_shift:
        j = w.max_shift
        roll = 8 * w.total + 8 * j * w.total + (j + 1) * w.total
    return swap, roll, 2 * layers * swap + roll


def measured_traffic(workload):
    """HBM bytes per swap launch from the committed counter summary of this
    workload, or None when there is none or the swap kernel's source has
    changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"swap_traffic_{workload}.txt")
    src = os.path.join(ROOT, "context_packed_sequence_amd", "csrc", "thd_swap.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != digest:
        return None
    return int(fields["traffic_bytes_per_launch"])


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence


class TimingEvent:
    """A HIP event used only for timing, with torch.cuda.Event's record /
    elapsed_time interface.

    Created with hipEventDisableSystemFence: recording it skips the
    system-scope release (cache write-back and invalidate) that a default
    event performs, which on this runtime leaves the device idle for about
    3 us between the two kernels it separates (the flag is meant for events
    that only time work).  The HIP runtime functions are resolved through
    the library's handle, i.e. from the runtime the library and torch share.
    """

    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes

            from context_packed_sequence_amd.binding import library

            hip = library()
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes

        self._ctypes = ctypes
        self._hip_rt = self._runtime()
        self._ev = ctypes.c_void_p()
        rc = self._hip_rt.hipEventCreateWithFlags(ctypes.byref(self._ev), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            self._ev = None
            raise RuntimeError(f"hipEventCreateWithFlags failed (HIP error {rc})")

    def record(self, stream):
        rc = self._hip_rt.hipEventRecord(self._ev, self._ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed (HIP error {rc})")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end`; both must have completed."""
        ms = self._ctypes.c_float()
        rc = self._hip_rt.hipEventElapsedTime(self._ctypes.byref(ms), self._ev, end._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed (HIP error {rc})")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "_ev", None) is not None:
            try:
                self._hip_rt.hipEventDestroy(self._ev)
            except Exception:
                pass


def _event_samples(torch, stream, fn, reps):
    """Device time of fn() in ms, one sample per call, from timing events on the launch stream."""
    evs = []
    for _ in range(reps):
        a, b = TimingEvent(), TimingEvent()
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def _queued_event_samples(torch, stream, fn, reps, hold_cycles=400000):
    """Device time of fn() in ms when the stream is busy as fn is enqueued,
    one sample per call: a spin kernel of about 0.2 ms holds the stream while
    the host records the start event, enqueues fn (which may be several
    calls, or a graph replay) and records the end event, so the span holds
    the kernels' dispatch and run, not the host's time to enqueue them."""
    evs = []
    for _ in range(reps):
        a, b = TimingEvent(), TimingEvent()
        torch.cuda._sleep(hold_cycles)
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def _median_event_ms(torch, stream, fn, reps):
    """Median device time of fn() queued behind a spin kernel."""
    ts = sorted(_queued_event_samples(torch, stream, fn, reps))
    return ts[len(ts) // 2]


def _capture(torch, stream, launch_on):
    """A HIP graph of launch_on(stream handle), after one eager run of it on a side stream."""
    side = torch.cuda.Stream(device=stream.device)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        launch_on(side.cuda_stream)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch_on(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    return graph


def measure_next(thd, torch, workloads, w, route, x, stream, step_on, reps=20):
    """The widened rows on the same batch: one-launch multi-key slice, roll
    written in zigzag order, device packing, and a graph-captured step."""
    T, dev, sh = w.total, x.device, stream.cuda_stream
    out = {}
    g = torch.Generator(device=dev).manual_seed(workloads.BASE_SEED + 77)
    keys = [torch.randint(0, 32000, (T,), dtype=torch.int64, device=dev, generator=g) for _ in range(3)]
    keys += [torch.randint(0, 2, (T,), dtype=torch.uint8, device=dev, generator=g) for _ in range(2)]
    outs = [torch.empty_like(k) for k in keys]
    rbs = [k.element_size() for k in keys]
    for _ in range(3):
        thd.thd_swap_batch(route.handle, thd.C2Z, keys, outs, rbs, T, sh)
    t_batch = _median_event_ms(torch, stream, lambda: thd.thd_swap_batch(route.handle, thd.C2Z, keys, outs, rbs, T, sh),
                               reps)

    def separate():
        for k, o, r in zip(keys, outs, rbs):
            thd.thd_swap(route.handle, thd.C2Z, k, o, T, r, sh)
    t_sep = _median_event_ms(torch, stream, separate, reps)

    def separate_on(s):
        for k, o, r in zip(keys, outs, rbs):
            thd.thd_swap(route.handle, thd.C2Z, k, o, T, r, s)
    g_sep = _capture(torch, stream, separate_on)
    t_sep_graph = _median_event_ms(torch, stream, g_sep.replay, reps)
    moved = 2 * T * sum(rbs)
    out["multi_key_swap"] = {"keys": "3 x int64 + 2 x uint8 per token", "us": round(t_batch * 1e3, 2),
                             "gbps": round(moved / (t_batch * 1e-3) / 1e9, 1),
                             "five_thd_swap_calls_us": round(t_sep * 1e3, 2),
                             "five_thd_swap_calls_graph_us": round(t_sep_graph * 1e3, 2)}

    # the tensors of one gated-delta-net layer (q, k, v with the activation's
    # row shape, then the decay gate g in fp32 and beta in bf16 per head)
    # through the route in one launch, against one thd_swap per tensor
    heads = 16
    layer_in = [torch.empty_like(x) for _ in range(3)]
    layer_in += [torch.empty((T, heads), dtype=torch.float32, device=dev),
                 torch.empty((T, heads), dtype=torch.bfloat16, device=dev)]
    for t in layer_in:
        t.view(torch.uint8).random_(0, 256, generator=g)
    layer_out = [torch.empty_like(t) for t in layer_in]
    layer_rb = [t.numel() // T * t.element_size() for t in layer_in]
    for _ in range(3):
        thd.thd_swap_batch(route.handle, thd.Z2C, layer_in, layer_out, layer_rb, T, sh)
    t_layer = _median_event_ms(torch, stream, lambda: thd.thd_swap_batch(route.handle, thd.Z2C, layer_in,
                                                                          layer_out, layer_rb, T, sh), reps)

    def layer_separate():
        for i_, o_, r_ in zip(layer_in, layer_out, layer_rb):
            thd.thd_swap(route.handle, thd.Z2C, i_, o_, T, r_, sh)
    t_layer_sep = _median_event_ms(torch, stream, layer_separate, reps)
    layer_moved = 2 * T * sum(layer_rb)
    out["layer_batch_swap"] = {"tensors": f"q,k,v {list(x.shape[1:])} bf16 + g [{heads}] fp32 + beta [{heads}] bf16",
                               "row_bytes": layer_rb, "us": round(t_layer * 1e3, 2),
                               "gbps": round(layer_moved / (t_layer * 1e-3) / 1e9, 1),
                               "separate_calls_us": round(t_layer_sep * 1e3, 2),
                               "separate_gbps": round(layer_moved / (t_layer_sep * 1e-3) / 1e9, 1)}
    del layer_in, layer_out

    cu = torch.from_numpy(w.cu_padded).to(dev)
    cu_real = torch.from_numpy(w.cu_real).to(dev)
    j = max(w.max_shift, 1)
    shifted = torch.empty((j, T), dtype=torch.int64, device=dev)
    mask = torch.empty((j + 1, T), dtype=torch.uint8, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    ids = keys[0]
    t_rz = _median_event_ms(torch, stream, lambda: thd.thd_roll_labels_zigzag(
        route.handle, ids, cu, cu_real, w.n_slots, T, j, 0, shifted, mask, status, sh), reps)
    t_rn = _median_event_ms(torch, stream, lambda: thd.thd_roll_labels(
        ids, cu, cu_real, w.n_slots, T, j, 0, shifted, mask, status, sh), reps)
    out["roll_zigzag_us"] = round(t_rz * 1e3, 2)
    out["roll_natural_us"] = round(t_rn * 1e3, 2)

    batch = 16
    seq = T // batch
    align = 2 * w.cp
    max_docs = 256
    rows = torch.from_numpy(workloads.token_rows(7, batch, seq, 0, 1, 1.0 / 4096, 512)).to(dev)
    capacity = ((batch * seq) // align + max_docs + 1) * align
    nbytes = thd.thd_pack_workspace_bytes(batch, seq)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    packed = torch.empty(capacity, dtype=torch.int64, device=dev)
    pcu = torch.empty(max_docs + 2, dtype=torch.int32, device=dev)
    pcup = torch.empty(max_docs + 2, dtype=torch.int32, device=dev)
    pst = torch.empty(1, dtype=torch.int32, device=dev)

    def do_pack():
        thd.thd_pack(rows, batch, seq, 0, 1, align, capacity, max_docs, 0, ws, nbytes, packed, pcu, pcup, pst, sh)
    do_pack()
    t_pack = _median_event_ms(torch, stream, do_pack, reps)
    assert int(pst.item()) == 0
    pack_bytes = 8 * batch * seq + 8 * capacity
    out["pack"] = {"rows": f"[{batch},{seq}] int64", "capacity": capacity, "us": round(t_pack * 1e3, 2),
                   "gbps": round(pack_bytes / (t_pack * 1e-3) / 1e9, 1)}

    graph = _capture(torch, stream, step_on)
    t_graph = _median_event_ms(torch, stream, graph.replay, reps)
    t_eager = _median_event_ms(torch, stream, lambda: step_on(sh), reps)
    out["graph_step_ms"] = round(t_graph, 4)
    out["eager_step_ms"] = round(t_eager, 4)
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def device_peak():
    """The memory clock and bus width the device reports.  MI355X reports a
    2 GHz clock on an 8192-bit bus; its HBM3E moves 8 Gb/s per pin, four
    transfers per reported clock, which gives 8.19 TB/s, AMD's published
    8 TB/s.  The published figure stays the peak the line is priced against
    (the lower of the two)."""
    import ctypes

    from context_packed_sequence_amd.binding import library

    hip = library()
    hip.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    clock, width = ctypes.c_int(), ctypes.c_int()
    # hipDeviceAttributeMemoryBusWidth = 59, hipDeviceAttributeMemoryClockRate = 60 (kHz)
    if hip.hipDeviceGetAttribute(ctypes.byref(width), 59, 0) or hip.hipDeviceGetAttribute(ctypes.byref(clock), 60, 0):
        return None
    return {"memory_clock_khz": clock.value, "bus_width_bits": width.value,
            "gbps_at_4_transfers_per_clock": round(4 * clock.value * 1e3 * width.value / 8 / 1e9, 1)}


def oracle_baseline(w, layers, budget_s):
    """The CPU oracle as it stands on the primary workload: route (steps 1-5,
    ``build_route``) and swap (step 6, ``apply_route``) timed apart, then
    whole steps (route, layers x both swaps, roll) until the budget is used."""
    import numpy as np

    import oracle

    x = w.rows_host()
    ids = w.ids()
    cu = w.cu_padded.tolist()
    swap_bytes, _, total_bytes = step_bytes(w, layers)
    t = time.perf_counter()
    route = oracle.build_route(cu, w.cp, w.total)
    t_route = [time.perf_counter() - t]
    t_swap = {"z2c": [], "c2z": []}
    t_roll = []
    t0 = time.perf_counter()
    steps = 0
    while True:
        t = time.perf_counter()
        route = oracle.build_route(cu, w.cp, w.total)
        t_route.append(time.perf_counter() - t)
        cur = x
        for _ in range(layers):
            t = time.perf_counter()
            a = oracle.apply_route(cur, route, "z2c")
            t_swap["z2c"].append(time.perf_counter() - t)
            t = time.perf_counter()
            cur = oracle.apply_route(a, route, "c2z")
            t_swap["c2z"].append(time.perf_counter() - t)
        if w.max_shift:
            t = time.perf_counter()
            oracle.roll_labels(ids, w.cu_padded, w.cu_real, w.total, w.max_shift, 0)
            t_roll.append(time.perf_counter() - t)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    assert np.array_equal(cur, x)
    route_ms = float(np.median(t_route)) * 1e3
    swap_ms = {d: float(np.median(v)) * 1e3 for d, v in t_swap.items()}
    return {
        "value": round(total_bytes * steps / el / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{steps} whole step(s) of the {w.name} workload ({layers} layer(s): route, z2c, c2z, roll), "
                  f"{el:.1f} s; single-threaded NumPy on 1 of {os.cpu_count()} host threads ({cpu_model()})",
        "cpu": cpu_model(),
        "host_threads": os.cpu_count(),
        "ms_per_step": round(el / steps * 1e3, 1),
        "step_tokens_per_s": round(w.total * steps / el),
        "route_ms": round(route_ms, 2),
        "route_tokens_per_s": round(w.total / (route_ms * 1e-3)),
        "swap_ms": {d: round(v, 2) for d, v in swap_ms.items()},
        "swap_gbps": round(swap_bytes / (np.mean(list(swap_ms.values())) * 1e-3) / 1e9, 3),
        "roll_ms": round(float(np.median(t_roll)) * 1e3, 2) if t_roll else None,
    }


def oracle_chunked(w, x_dev, out_dev, direction, chunk_bytes=256 << 20, n_chunks=4):
    """The oracle on a batch too large to gather at once: the route (steps
    1-5) built whole, the swap (step 6) applied to chunks of output rows of
    ``chunk_bytes``, each timed and compared byte for byte with the same rows
    of the GPU's output.  Chunks are spread evenly over the buffer."""
    import numpy as np

    import oracle

    cu = w.cu_padded.tolist()
    t = time.perf_counter()
    route = oracle.build_route(cu, w.cp, w.total)
    route_s = time.perf_counter() - t
    x_host = x_dev.view(-1).view(torch_uint8()).cpu().numpy().reshape(w.total, w.row_bytes)
    rows = max(1, chunk_bytes // w.row_bytes)
    starts = np.linspace(0, w.total - rows, n_chunks).astype(np.int64)
    times, same = [], True
    for a in starts:
        sl = slice(int(a), int(a) + rows)
        t = time.perf_counter()
        got = oracle.apply_route(x_host, route, direction, sl)
        times.append(time.perf_counter() - t)
        dev = out_dev.view(-1).view(torch_uint8())[int(a) * w.row_bytes:(int(a) + rows) * w.row_bytes].cpu().numpy()
        same = same and np.array_equal(got.reshape(-1), dev)
    del x_host
    sec = float(np.median(times))
    return {
        "route_ms": round(route_s * 1e3, 1),
        "route_tokens_per_s": round(w.total / route_s),
        "swap_chunk_ms": round(sec * 1e3, 1),
        "swap_gbps": round(2 * rows * w.row_bytes / sec / 1e9, 3),
        "chunks_compared": len(starts),
        "chunk_mib": rows * w.row_bytes >> 20,
        "direction": direction,
        "match": bool(same),
    }


def torch_uint8():
    import torch
    return torch.uint8


def measure(thd, torch, workloads, w, steps, warmup):
    """One workload: device warm-up, in-run ceilings, W warm-up steps, K timed
    steps, then per-direction swap times, route build and roll latency and the
    no-host-wait check.  Returns the figures and the buffers' handles."""
    import numpy as np

    layers = w.layers
    total, cp, rb, n_slots = w.total, w.cp, w.row_bytes, w.n_slots
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    # the roll does not read the activations: it runs on a second stream of
    # the same (default) priority, beside the swaps, and the step joins it
    side = torch.cuda.Stream(device=dev)
    roll_done = torch.cuda.Event()

    cu = torch.from_numpy(w.cu_padded).to(dev)
    cu_real = torch.from_numpy(w.cu_real).to(dev)
    ids = torch.from_numpy(w.ids()).to(dev)
    g = torch.Generator(device=dev).manual_seed(workloads.BASE_SEED + w.index)
    x = torch.randn((total,) + tuple(w.row_shape), dtype=torch.bfloat16, device=dev, generator=g)
    a = torch.empty_like(x)
    b = torch.empty_like(x)
    j = max(w.max_shift, 1)
    shifted = torch.empty((j, total), dtype=torch.int64, device=dev)
    mask = torch.empty((j + 1, total), dtype=torch.uint8, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    route = thd.Route(n_slots, cp, total)
    h = route.handle
    torch.cuda.synchronize()

    def roll_on(s):
        thd.thd_roll_labels(ids, cu, cu_real, n_slots, total, j, 0, shifted, mask, status, s)

    def step(e=None):
        # e: two timing events, recorded on the swaps' stream just before the
        # first swap and just after the last; the swaps of all layers run back
        # to back with no event between them
        thd.thd_build_route(h, cu, n_slots, cp, total, sh)
        roll_on(side.cuda_stream)
        roll_done.record(side)
        if e is not None:
            e[0].record(stream)
        for _ in range(layers):
            thd.thd_swap(h, thd.Z2C, x, a, total, rb, sh)
            thd.thd_swap(h, thd.C2Z, a, b, total, rb, sh)
        if e is not None:
            e[1].record(stream)
        stream.wait_event(roll_done)

    # correctness guard (not timed): one step, then the round trip must be exact
    step()
    torch.cuda.synchronize()
    assert route.status() == 0 and int(status.item()) == 0
    assert torch.equal(b.view(torch.int16), x.view(torch.int16))

    # device warm-up: the chip's clocks rise only under sustained load (from
    # idle the swap needs about 100 back-to-back launches, ~20 ms, to reach
    # its steady time), so swaps run back to back for at least 0.25 s first
    swap_bytes, roll_bytes, total_bytes = step_bytes(w, layers)
    warm_launches, t0 = 0, time.perf_counter()
    while warm_launches < 200 or time.perf_counter() - t0 < 0.25:
        for _ in range(20):
            thd.thd_swap(h, thd.Z2C, x, a, total, rb, sh)
            thd.thd_swap(h, thd.C2Z, a, b, total, rb, sh)
        warm_launches += 40
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - t0

    # ceilings in the same run, right after the warm-up: the runtime's
    # device-to-device copy (torch copy_ of the same activation), the
    # library's plain streaming copy (the swap's units and workgroup shape
    # without the route) and the two pure streams over the bytes one swap
    # moves (a swap or a copy mixes reads and writes on the same HBM channels
    # and cannot move bytes faster than either pure stream)
    nbytes = total * rb
    per = max(1, int(round(0.003 / (swap_bytes / 6.5e12))))  # launches per sample: about 3 ms

    def batch_ms(fn, samples=8):
        ts = _event_samples(torch, stream, lambda: [fn() for _ in range(per)], samples)
        return float(np.median(ts)) / per

    copy_dtod_ms = batch_ms(lambda: a.copy_(x))
    copy_stream_ms = batch_ms(lambda: thd.thd_copy(x, a, nbytes, sh))
    scratch = torch.empty(2 * nbytes, dtype=torch.uint8, device=dev)
    hits = torch.zeros(1, dtype=torch.int32, device=dev)
    write_ms = batch_ms(lambda: thd.thd_write_stream(scratch, 2 * nbytes, 1, sh))
    key = struct.pack("<4I", 1, 2, 3, 4)  # never written: every written word repeats one value
    read_ms = batch_ms(lambda: thd.thd_read_stream(scratch, 2 * nbytes, key, hits, sh))
    assert int(hits.item()) == 0
    del scratch, hits

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    launches_before = 2 * layers * (1 + warmup) + warm_launches  # guard step, warm-up swaps, warm-up steps

    # timed region: K steps, two events per step on the swaps' stream
    events = [[TimingEvent(), TimingEvent()] for _ in range(steps)]
    t_start, t_end = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for e in events:
        step(e)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = t_start.elapsed_time(t_end)
    ms_per_step = max(wall * 1e3, gpu_ms) / steps
    swap_ms = [e[0].elapsed_time(e[1]) / (2 * layers) for e in events]
    swap_avg_ms = float(np.mean(swap_ms))

    # each direction alone, right after the timed region: samples of about
    # 3 ms of back-to-back launches of one direction, directions interleaved
    by_dir = {"z2c": [], "c2z": []}
    fns = {"z2c": lambda: thd.thd_swap(h, thd.Z2C, x, a, total, rb, sh),
           "c2z": lambda: thd.thd_swap(h, thd.C2Z, a, b, total, rb, sh)}
    for _ in range(10):
        for d, fn in fns.items():
            by_dir[d] += [t / per for t in _event_samples(torch, stream, lambda: [fn() for _ in range(per)], 1)]
    by_dir = {d: {"median_us": round(float(np.median(v)) * 1e3, 2), "min_us": round(float(np.min(v)) * 1e3, 2),
                  "gbps": round(swap_bytes / (float(np.median(v)) * 1e-3) / 1e9, 1),
                  "frac": round(swap_bytes / (float(np.median(v)) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
              for d, v in by_dir.items()}

    # route build and roll device times: events around single launches
    build_ms = _event_samples(torch, stream, lambda: thd.thd_build_route(h, cu, n_slots, cp, total, sh), 100)
    roll_ms = _event_samples(torch, stream, lambda: roll_on(sh), 100)
    # the floor those figures sit on: the same events around one launch of a
    # one-workgroup kernel that moves 16 bytes
    floor_ms = _event_samples(torch, stream, lambda: thd.thd_copy(x, a, 16, sh), 100)
    # route build: host enqueue time of the build call alone
    torch.cuda.synchronize()
    enq = []
    for _ in range(100):
        t0 = time.perf_counter()
        thd.thd_build_route(h, cu, n_slots, cp, total, sh)
        enq.append(time.perf_counter() - t0)
        torch.cuda.synchronize()

    # no call waits for the GPU: hold the stream with a spin kernel, enqueue a
    # whole step (build, every swap, the roll), and the spin must still run
    torch.cuda.synchronize()
    gate = torch.cuda.Event()
    torch.cuda._sleep(int(5e8))
    gate.record(stream)
    thd.thd_build_route(h, cu, n_slots, cp, total, sh)
    for _ in range(layers):
        thd.thd_swap(h, thd.Z2C, x, a, total, rb, sh)
        thd.thd_swap(h, thd.C2Z, a, b, total, rb, sh)
    roll_on(sh)
    host_syncs = 0 if not gate.query() else None
    torch.cuda.synchronize()
    assert route.status() == 0 and int(status.item()) == 0
    assert torch.equal(b.view(torch.int16), x.view(torch.int16))

    swap_gbps = swap_bytes / (swap_avg_ms * 1e-3) / 1e9
    res = {
        "workload": w.name,
        "cp_size": cp,
        "tokens": total,
        "slots": n_slots,
        "row_bytes": rb,
        "step": f"build + {layers}x(z2c + c2z) + roll(max_shift={j}) on a second stream",
        "steps": steps,
        "ms_per_step": round(ms_per_step, 4),
        "step_gbps": round(total_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "swap_us": round(swap_avg_ms * 1e3, 2),
        "swap_gbps": round(swap_gbps, 1),
        "swap_frac": round(swap_gbps / HBM_PEAK_GBPS, 4),
        "swap_tokens_per_s": round(total / (swap_avg_ms * 1e-3)),
        "step_tokens_per_s": round(total / (ms_per_step * 1e-3)),
        "swap_us_by_direction": by_dir,
        "route_build_us": round(float(np.median(build_ms)) * 1e3, 2),
        "route_build_enqueue_us": round(float(np.median(enq)) * 1e6, 2),
        "roll_us": round(float(np.median(roll_ms)) * 1e3, 2),
        "launch_floor_us": round(float(np.median(floor_ms)) * 1e3, 2),
        "host_syncs": host_syncs,
        "copy_ceiling_gbps": {"dtod_copy": round(swap_bytes / (copy_dtod_ms * 1e-3) / 1e9, 1),
                              "stream_copy": round(swap_bytes / (copy_stream_ms * 1e-3) / 1e9, 1)},
        "swap_over_stream_copy": round(copy_stream_ms / swap_avg_ms, 4),
        "stream_gbps": {"read_only": round(swap_bytes / (read_ms * 1e-3) / 1e9, 1),
                        "write_only": round(swap_bytes / (write_ms * 1e-3) / 1e9, 1)},
        "warm_up": {"swap_launches_before_timing": launches_before, "sustained_swaps_s": round(warm_s, 3)},
    }

    def step_on(s):
        thd.thd_build_route(h, cu, n_slots, cp, total, s)
        for _ in range(layers):
            thd.thd_swap(h, thd.Z2C, x, a, total, rb, s)
            thd.thd_swap(h, thd.C2Z, a, b, total, rb, s)
        roll_on(s)

    ctx = {"route": route, "x": x, "a": a, "b": b, "stream": stream, "step_on": step_on}
    return res, ctx


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the cross-rank exchange is "
              "emulated as one global permutation on a single device; on several GPUs each rank would build "
              "the same route locally and exchange its rows in one all-to-all-v, which is not built here.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import context_packed_sequence_amd as thd
    import workloads

    if args.row_sweep:
        row_sweep(workloads)
        return
    torch.cuda.set_device(torch.device("cuda", 0))
    w = workloads.make(args.workload)
    head, ctx = measure(thd, torch, workloads, w, args.steps, args.warmup)
    print(json.dumps({"progress": f"{w.name} measured", "swap_us": head["swap_us"]}), file=sys.stderr, flush=True)
    next_rows = measure_next(thd, torch, workloads, w, ctx["route"], ctx["x"], ctx["stream"], ctx["step_on"])

    cpu = None
    if not args.no_cpu_baseline:
        cpu = oracle_baseline(w, w.layers, args.cpu_seconds)
        cpu["by_config"] = {w.name: {k: cpu[k] for k in ("route_ms", "route_tokens_per_s", "swap_ms", "swap_gbps")}}
    ctx["route"].close()
    del ctx
    torch.cuda.empty_cache()

    # the other configured workloads, each on its own, same step structure
    others = {}
    for name in args.also.split(",") if args.also else []:
        if name == w.name:
            continue
        wo = workloads.make(name)
        res, octx = measure(thd, torch, workloads, wo, args.steps, args.warmup)
        if cpu is not None and name == "long1m":
            # a batch of 16 GiB per swap: the oracle is compared and timed on
            # 256 MiB chunks of the GPU's z->c output
            thd.thd_swap(octx["route"].handle, thd.Z2C, octx["x"], octx["a"], wo.total, wo.row_bytes,
                         octx["stream"].cuda_stream)
            torch.cuda.synchronize()
            cpu["by_config"][name] = oracle_chunked(wo, octx["x"], octx["a"], "z2c")
        elif cpu is not None:
            import oracle
            t = time.perf_counter()
            oracle.build_route(wo.cu_padded.tolist(), wo.cp, wo.total)
            route_s = time.perf_counter() - t
            cpu["by_config"][name] = {"route_ms": round(route_s * 1e3, 2),
                                      "route_tokens_per_s": round(wo.total / route_s)}
        others[name] = res
        print(json.dumps({"progress": f"{name} measured", "swap_us": res["swap_us"]}), file=sys.stderr, flush=True)
        octx["route"].close()
        del octx
        torch.cuda.empty_cache()

    swap_bytes = 2 * w.total * w.row_bytes
    out = {
        "metric": "thd_swap GB/s (% HBM peak) + tokens/s; route-build latency, host syncs=0",
        "value": head["step_gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "cp_size": w.cp,
            "tokens": w.total,
            "slots": w.n_slots,
            "rows": f"[{w.total},{','.join(str(s) for s in w.row_shape)}] bf16 (moved as bytes)",
            "row_bytes": w.row_bytes,
            "step": head["step"],
            "value_is": "step GB/s: algorithmic bytes of the whole step (route build, every swap, roll) "
                        "over the step time; the swap kernel alone is in roofline",
        },
    }
    for k in ("swap_us", "swap_gbps", "swap_tokens_per_s", "step_tokens_per_s", "route_build_us",
              "route_build_enqueue_us", "roll_us", "launch_floor_us", "host_syncs",
              "swap_us_by_direction", "copy_ceiling_gbps",
              "swap_over_stream_copy", "stream_gbps", "warm_up"):
        out[k] = head[k]
    out["roofline"] = {
        "bound": "hbm",
        "achieved": head["swap_gbps"],
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(head["swap_gbps"] / HBM_PEAK_GBPS, 4),
        "traffic": measured_traffic(w.name),
        "per_launch_bytes": swap_bytes,
        "device_reported": device_peak(),
    }
    out["cpu_baseline"] = cpu
    out["workloads"] = others
    out["next"] = next_rows
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
