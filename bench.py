"""Throughput of the masked second-order HLA forward on one MI355X.

Workload: B=4, H=8, n=2048, d=dv=64, bf16 q/k/v ~ N(0,1)/sqrt(d), chunk 64,
unnormalised, no decay or ridge.  One step = one ``hla_forward_chunked``
call over the whole batch (all of its kernels), with inputs resident in HBM.

Timing: the K timed steps are captured once into a HIP graph (torch.cuda.graph
on a side stream; the library allocates nothing and never synchronises, so
the launches capture as they are) and replayed once between two HIP events
recorded on the capture stream.  Consecutive steps rotate over several
copies of the inputs and outputs whose total exceeds twice the 256 MB
Infinity Cache, so each step reads its inputs from HBM rather than from the
previous step's cached lines.  The graph replay is checked bit-for-bit
against the eager result of the same calls.

Printed: one JSON line with tokens/s (B*n per second), the roofline of the
path (algorithmic q/k/v/out bytes per step over the measured step time,
against 8 TB/s), and the fp64 CPU oracle timed on the host on a bounded
sample of the same workload.  The line also carries ``workloads``: the
other parts of the hot path (the ratio-normalised forward with decay and
ridge, the long d=128 forward with and without states, the streaming decode
step, packed and multi-query decode, state composition, AHLA and third order,
the small fp32 forward), and at the headline shape the forward that also
returns its final state or also starts from an initial state (the calls a
sequence shard makes) and the backward (plain, and as a sequence shard runs
it: from an initial state, with a final-state gradient in and the
initial-state gradient out), each timed with HIP events on its launch stream
and set against its own HBM roofline (``--headline-only`` skips them).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20


SECONDARY = ("ratio", "long", "decode", "decode_mq", "compose", "small", "state", "backward", "ahla", "third")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--seed", type=int, default=1001)
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the secondary workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device copies of 256 MiB (for scaling HBM counters)")
    ap.add_argument("--only", choices=SECONDARY,
                    help="only time this secondary workload and print its record (for profiling)")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="only time plain device copies of the headline's size and of 1 GiB")
    ap.add_argument("--calls", type=int, default=100,
                    help="event-timed single calls per mode for the p10/p50/p90 figures")
    return ap.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "k_fast64_B4_H8_n2048_d64_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "associative_scan_sequence_amd", "csrc", f)
                  for f in ("fwd_fast64.hip", "fast64_common.h", "bf16_split.h")]


def kernel_source_hash():
    """sha256 over the headline kernel's sources, in order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the d=64 kernel from the committed counter
    summary, or None when the kernel source changed since it was taken."""
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    src = kernel_source_hash()
    m_hash = re.search(r"kernel source sha256: ([0-9a-f]{64})", text)
    m_bytes = re.search(r"HBM bytes per launch: ([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != src:
        return None
    return float(m_bytes.group(1))


def copy_calibration():
    """Plain 256 MiB device-to-device copies: the counters FETCH_SIZE and
    WRITE_SIZE of these dispatches give the scale from counter KiB to bytes."""
    import torch

    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "copies": 5}))


def copy_ceiling(dev):
    """What a plain device copy sustains at the headline's byte count
    (25.2 MB read + 16.8 MB written -> one 21 MB copy each way, 42 MB moved)
    and at 1 GiB: p50 of HIP-event-timed copies, cold (a 1 GiB scratch write
    between copies) and warm."""
    import torch

    out = []
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    for nbytes in (41943040 // 2, 1 << 30):
        a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        rec = {"bytes_moved": 2 * nbytes}
        for mode in ("cold", "warm"):
            ts = event_times(lambda i: b.copy_(a), stream, 30, scratch if mode == "cold" else None)
            p50 = percentiles(ts)["p50"]
            rec[mode] = {"p50_us": p50, "GB_per_s": 2 * nbytes / (p50 * 1e-6) / 1e9}
        out.append(rec)
        del a, b
    return {"copy_ceiling": out}


def event_times(fn, stream, calls, flush=None, warmup=3):
    """Microseconds of each of ``calls`` calls fn(i), each bracketed by its
    own pair of HIP events on ``stream``.  flush: a buffer written in full
    before every call, outside the events (cold mode: evicts the caches);
    without it the calls run back to back (warm mode).  The device is held
    busy first (torch.cuda._sleep) so the host enqueues ahead of it and no
    launch gap falls inside a pair of events."""
    import torch

    with torch.cuda.stream(stream):
        for i in range(warmup):
            fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    with torch.cuda.stream(stream):
        torch.cuda._sleep(50_000_000)  # ~20 ms of device time for the host to run ahead
        for i in range(calls):
            if flush is not None:
                flush.fill_(i & 0xFF)
            ev[i][0].record(stream)
            fn(i)
            ev[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def percentiles(ts):
    import numpy as np

    a = np.asarray(ts, dtype=np.float64)
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def algorithmic_bytes(w) -> int:
    # q, k (d each) and v (dv) in bf16 read once, out (dv) in fp32 written once
    per_token = 2 * (2 * w.d + w.dv) + 4 * w.dv
    return w.B * w.H * w.n * per_token


_LAST_PCT = {}


def time_calls(fn, stream, reps, warmup=3):
    """Mean microseconds per call of fn(i) over ``reps`` calls bracketed by
    one pair of HIP events on ``stream``; the p10/p50/p90 of the same calls
    timed one by one (each between its own events, see event_times) are kept
    for the record that follows (``single_call_us``)."""
    import torch

    with torch.cuda.stream(stream):
        for i in range(warmup):
            fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
    e1.synchronize()
    _LAST_PCT.clear()
    _LAST_PCT.update(percentiles(event_times(fn, stream, reps, warmup=0)))
    return e0.elapsed_time(e1) * 1e3 / reps


def roof(bytes_per_call, us):
    gbs = bytes_per_call / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_call": bytes_per_call}


def secondary_workloads(dev, stream, only=None):
    """The other parts of the hot path at their workload sizes (all, or the
    one named by ``only``)."""
    import torch

    import associative_scan_sequence_amd as hla
    import hla_inputs as inputs

    res = []
    if only not in (None, "ratio"):
        return res + secondary_rest(dev, stream, only)
    # ratio-normalised forward with per-head decay and ridge (out and den)
    w = inputs.RATIO_DECAY_D64
    per_tok = 2 * (2 * w.d + w.dv) + 4 * w.dv + 4
    copies = max(2, math.ceil(2 * MALL_BYTES / (w.B * w.H * w.n * per_tok)))
    sets = []
    for c in range(copies):
        q, k, v = inputs.qkv_on_device(w.B, w.H, w.n, w.d, w.dv, w.dtype, 5000 + c, dev)
        out = torch.empty(w.B, w.H, w.n, w.dv, dtype=torch.float32, device=dev)
        den = torch.empty(w.B, w.H, w.n, dtype=torch.float32, device=dev)
        ws = torch.zeros(hla.workspace_size(w.B, w.H, w.n, w.d, w.dv, chunk=w.chunk, gamma=w.gamma,
                                            ridge=w.ridge, normalize=True), dtype=torch.uint8, device=dev)
        sets.append((q, k, v, out, den, ws))

    def ratio_call(i):
        q, k, v, out, den, ws = sets[i % copies]
        hla.forward_chunked(q, k, v, gamma=w.gamma, ridge=w.ridge, normalize=True, chunk=w.chunk,
                            out=out, den=den, workspace=ws)
    us = time_calls(ratio_call, stream, 20)
    tok = w.B * w.H * w.n
    res.append({"workload": w.name, "entry": "hla_forward_chunked (out + den)", "us_per_call": us, "single_call_us": dict(_LAST_PCT),
                "tokens_per_s": w.B * w.n / (us * 1e-6), "roofline": roof(tok * per_tok, us)})
    del sets
    if only is not None:
        return res
    return res + secondary_rest(dev, stream, None)


def secondary_rest(dev, stream, only):
    import torch

    import associative_scan_sequence_amd as hla
    import hla_inputs as inputs

    res = []
    if only not in (None, "long"):
        return res + secondary_states(dev, stream, only)
    # long d = 128 forward with decay
    w = inputs.LONG_D128
    per_tok = 2 * (2 * w.d + w.dv) + 4 * w.dv
    q, k, v = inputs.qkv_on_device(w.B, w.H, w.n, w.d, w.dv, w.dtype, 5100, dev)
    out = torch.empty(w.B, w.H, w.n, w.dv, dtype=torch.float32, device=dev)
    ws = torch.zeros(hla.workspace_size(w.B, w.H, w.n, w.d, w.dv, chunk=w.chunk, gamma=w.gamma),
                     dtype=torch.uint8, device=dev)
    us = time_calls(lambda i: hla.forward_chunked(q, k, v, gamma=w.gamma, chunk=w.chunk, out=out,
                                                  workspace=ws), stream, 5, warmup=2)
    tok = w.B * w.H * w.n
    res.append({"workload": w.name, "entry": "hla_forward_chunked", "us_per_call": us, "single_call_us": dict(_LAST_PCT),
                "tokens_per_s": w.B * w.n / (us * 1e-6), "roofline": roof(tok * per_tok, us)})
    # the same call returning its final state, and starting from an initial one
    # (a long-context shard): the one-launch kernel's state variant
    fin = hla.State.empty(w.B * w.H, w.d, w.dv, dev)
    init = hla.State(*(t.to(dev) for t in inputs.random_state_fp32(w.B * w.H, w.d, w.dv, 5101, scale=0.05)))
    state_b = 4 * (w.d * w.d + 2 * w.d * w.dv + 2 * w.d + 1)
    for tag, ini, nstates in (("final_state", None, 1), ("init_and_final_state", init, 2)):
        us = time_calls(lambda i, ini=ini: hla.forward_chunked(q, k, v, gamma=w.gamma, chunk=w.chunk, out=out,
                                                               workspace=ws, init=ini, final_state=fin),
                        stream, 5, warmup=2)
        res.append({"workload": w.name.replace("masked_hla_fwd", f"masked_hla_fwd_{tag}"),
                    "entry": f"hla_forward_chunked (out + {tag.replace('_', ' ')}, one-launch kernel)",
                    "us_per_call": us, "single_call_us": dict(_LAST_PCT),
                    "tokens_per_s": w.B * w.n / (us * 1e-6),
                    "roofline": roof(tok * per_tok + nstates * w.B * w.H * state_b, us)})
    del q, k, v, out, ws, fin, init
    if only is not None:
        return res
    return res + secondary_states(dev, stream, None)


def secondary_states(dev, stream, only):
    import torch

    import associative_scan_sequence_amd as hla
    import hla_inputs as inputs

    res = []
    if only in ("small", "state", "backward", "ahla", "third"):
        return res + secondary_small(dev, stream, only)
    # streaming decode: 4096 states seeded from a 512-token prefix
    w = inputs.DECODE_D128
    q, k, v = inputs.qkv_on_device(w.B, w.H, w.n, w.d, w.dv, w.dtype, 5200, dev)
    _, _, st = hla.forward_chunked(q, k, v, return_state=True)
    del q, k, v
    q1, k1, v1 = (x[:, :, 0] .contiguous() for x in
                  inputs.qkv_on_device(w.B, w.H, 1, w.d, w.dv, w.dtype, 5201, dev))
    o1 = torch.empty(w.B, w.H, w.dv, dtype=torch.float32, device=dev)
    N = w.B * w.H
    state_b = 4 * (w.d * w.d + 2 * w.d * w.dv + 2 * w.d)
    if only in (None, "decode"):
        us = time_calls(lambda i: hla.decode_step(q1, k1, v1, st, out=o1), stream, 30)
        per_state = 2 * state_b + 2 * (2 * w.d + w.dv) + 4 * w.dv
        res.append({"workload": w.name, "entry": "hla_decode_step", "us_per_call": us, "single_call_us": dict(_LAST_PCT),
                    "states_per_s": N / (us * 1e-6), "roofline": roof(N * per_state, us)})
    if only in (None, "decode_mq"):
        res += decode_mq_workloads(st, q1, k1, v1, w, stream)
    if only in ("decode", "decode_mq"):
        return res
    # state composition of 4096 segment pairs at d = dv = 128
    b = hla.State.empty(N, w.d, w.dv, dev)
    for name in ("S", "C", "m", "G", "h", "rho"):
        getattr(b, name).copy_(getattr(st, name))
    r = hla.State.empty(N, w.d, w.dv, dev)
    us = time_calls(lambda i: hla.state_compose(st, b, r), stream, 30)
    per_pair = 3 * (state_b + 4)
    res.append({"workload": "masked_hla_compose_4096_pairs_d128", "entry": "hla_state_compose",
                "us_per_call": us, "single_call_us": dict(_LAST_PCT), "pairs_per_s": N / (us * 1e-6), "roofline": roof(N * per_pair, us)})
    del st, b, r
    if only is not None:
        return res
    return res + secondary_small(dev, stream, None)


def decode_mq_workloads(st, q1, k1, v1, w, stream):
    """The decode step with the key moment packed (hla_decode_step_mq): the
    4096 states unshared (each of S packed, C, G read once and written once),
    then as multi-query attention, the 16 query heads of each batch row
    sharing k, v and one packed S."""
    import torch

    import associative_scan_sequence_amd as hla

    res = []
    d, dv, B, H = w.d, w.dv, w.B, w.H
    N = B * H
    o1 = torch.empty(B, H, dv, dtype=torch.float32, device=q1.device)
    sp = 4 * hla.packed_size(d)                  # packed S bytes
    per_head = 4 * (2 * d * dv + 2 * d)          # C, G, m, h bytes
    mq = hla.MqState(hla.key_moment_pack(st.S), st.C, st.m, st.G, st.h, st.rho)
    us = time_calls(lambda i: hla.decode_step_mq(q1, k1, v1, mq, out=o1), stream, 30)
    per_state = 2 * (sp + per_head) + 2 * (2 * d + dv) + 4 * dv
    res.append({"workload": "masked_hla_decode_packed_S_4096_states_d128", "entry": "hla_decode_step_mq (kv_heads = H)",
                "us_per_call": us, "single_call_us": dict(_LAST_PCT), "states_per_s": N / (us * 1e-6), "bytes_per_state": per_state,
                "roofline": roof(N * per_state, us)})
    k1g, v1g = k1[:, :1].contiguous(), v1[:, :1].contiguous()
    Sg = mq.S.view(B, H, -1)[:, 0].contiguous()
    mqa = hla.MqState(Sg, st.C, st.m, st.G, st.h, st.rho.view(B, H)[:, 0].contiguous())
    us = time_calls(lambda i: hla.decode_step_mq(q1, k1g, v1g, mqa, out=o1), stream, 30)
    total = B * (2 * sp + H * (2 * per_head + 2 * d + 4 * dv) + 2 * (d + dv))
    res.append({"workload": "masked_hla_decode_multi_query_B256_H16_kv1_d128", "entry": "hla_decode_step_mq (kv_heads = 1)",
                "us_per_call": us, "single_call_us": dict(_LAST_PCT), "states_per_s": N / (us * 1e-6), "bytes_per_call": total,
                "roofline": roof(total, us)})
    return res


def higher_workloads(dev, stream, which):
    """The asymmetric variant (AHLA, per-head decay g_h = 1 - 2^-(5+h)) and
    masked third order at B4 H8 n2048 d = dv = 64 bf16, chunk 64: q, k, v in
    and out, 640 algorithmic bytes per head-token; inputs rotated over copies
    that exceed the Infinity Cache twice."""
    import torch

    import associative_scan_sequence_amd as hla
    import hla_inputs as inputs

    w = inputs.FWD_D64
    tok = w.B * w.H * w.n
    per_tok = 2 * (2 * w.d + w.dv) + 4 * w.dv
    res = []
    for name in which:
        third = name == "third"
        g = None if third else inputs.gamma_list_fp32([1 - 2.0 ** -(5 + h) for h in range(w.H)])
        size_fn = hla._binding.load().hla_third_workspace_size if third else hla._binding.load().hla_ahla_workspace_size
        p, _keep = hla._binding._params(w.B, w.H, w.n, w.d, w.dv, w.chunk, w.dtype, g, 0.0, False)
        need = int(size_fn(hla._binding.ctypes.byref(p)))
        copies = max(2, math.ceil(2 * MALL_BYTES / (tok * per_tok + need)))
        sets = []
        for c in range(copies):
            q, k, v = inputs.qkv_on_device(w.B, w.H, w.n, w.d, w.dv, w.dtype, 5700 + c, dev)
            sets.append((q, k, v, torch.empty(w.B, w.H, w.n, w.dv, dtype=torch.float32, device=dev),
                         torch.zeros(need, dtype=torch.uint8, device=dev)))

        def call(i, third=third, g=g, sets=sets):
            q, k, v, out, ws = sets[i % len(sets)]
            if third:
                hla.third_forward(q, k, v, chunk=w.chunk, out=out, workspace=ws)
            else:
                hla.ahla_forward(q, k, v, gamma=g, chunk=w.chunk, out=out, workspace=ws)
        us = time_calls(call, stream, 20)
        res.append({"workload": ("masked_third_order_fwd" if third else "ahla_fwd_decay") + "_B4_H8_n2048_d64_bf16_w64",
                    "entry": "hla_third_forward" if third else "hla_ahla_forward", "us_per_call": us,
                    "single_call_us": dict(_LAST_PCT), "tokens_per_s": w.B * w.n / (us * 1e-6),
                    "roofline": roof(tok * per_tok, us)})
        del sets
    return res


def secondary_small(dev, stream, only):
    res = []
    if only in (None, "ahla", "third"):
        res += higher_workloads(dev, stream, ("ahla", "third") if only is None else (only,))
    if only in (None, "small"):
        res += small_forward(dev, stream)
    if only in (None, "state"):
        res += forward_with_state(dev, stream)
    if only in (None, "backward"):
        res += backward_headline_shape(dev, stream)
    return res


def forward_with_state(dev, stream):
    """hla_forward_chunked at B4 H8 n2048 d64 bf16 returning the final state
    (the per-head summary a sequence shard hands on), and the same call that
    also starts from an initial state (a shard in the middle of a sequence):
    the one-launch kernel's state variant.  Algorithmic bytes: q, k, v in and
    out per head-token, plus each state read or written per head."""
    import torch

    import associative_scan_sequence_amd as hla
    import hla_inputs as inputs

    w = inputs.FWD_D64
    tok = w.B * w.H * w.n
    per_tok = 2 * (2 * w.d + w.dv) + 4 * w.dv
    state_b = 4 * (w.d * w.d + 2 * w.d * w.dv + 2 * w.d + 1)
    need = hla.workspace_size(w.B, w.H, w.n, w.d, w.dv, chunk=w.chunk)
    copies = max(2, math.ceil(2 * MALL_BYTES / (tok * per_tok + need)))
    sets = []
    for c in range(copies):
        q, k, v = inputs.qkv_on_device(w.B, w.H, w.n, w.d, w.dv, w.dtype, 5600 + c, dev)
        out = torch.empty(w.B, w.H, w.n, w.dv, dtype=torch.float32, device=dev)
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        sets.append((q, k, v, out, ws))
    fin = hla.State.empty(w.B * w.H, w.d, w.dv, dev)
    init = hla.State(*(t.to(dev) for t in inputs.random_state_fp32(w.B * w.H, w.d, w.dv, 5700, scale=0.1)))
    res = []
    for tag, ini, nstates in (("final_state", None, 1), ("init_and_final_state", init, 2)):
        def call_state(i, ini=ini):
            q, k, v, out, ws = sets[i % copies]
            hla.forward_chunked(q, k, v, chunk=w.chunk, out=out, workspace=ws, init=ini, final_state=fin)
        us = time_calls(call_state, stream, 20)
        res.append({"workload": f"masked_hla_fwd_{tag}_B4_H8_n2048_d64_bf16_w64",
                    "entry": f"hla_forward_chunked (out + {tag.replace('_', ' ')}, one-launch kernel)",
                    "us_per_call": us, "single_call_us": dict(_LAST_PCT),
                    "tokens_per_s": w.B * w.n / (us * 1e-6),
                    "roofline": roof(tok * per_tok + nstates * w.B * w.H * state_b, us)})
    return res


def backward_headline_shape(dev, stream):
    """hla_backward_chunked at B4 H8 n2048 d64 bf16: read q, k, v (bf16) and
    dout (fp32), write dq, dk, dv (fp32): 1408 B per head-token.  The plain
    call takes the one-launch backward (seven first-order maps in three
    launches); the shard's call (initial state, final-state gradient,
    initial-state gradient) the same maps with carries in and out."""
    import torch

    import associative_scan_sequence_amd as hla
    import hla_inputs as inputs

    w = inputs.FWD_D64
    per_tok = 2 * (2 * w.d + w.dv) + 4 * w.dv + 4 * (2 * w.d + w.dv)
    tok = w.B * w.H * w.n
    need = hla.backward_workspace_size(w.B, w.H, w.n, w.d, w.dv, chunk=w.chunk)
    copies = max(2, math.ceil(2 * MALL_BYTES / (tok * per_tok + need)))
    sets = []
    for c in range(copies):
        q, k, v = inputs.qkv_on_device(w.B, w.H, w.n, w.d, w.dv, w.dtype, 5400 + c, dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(5500 + c)
        dout = torch.randn(w.B, w.H, w.n, w.dv, generator=gen, dtype=torch.float32, device=dev)
        grads = (torch.empty(w.B, w.H, w.n, w.d, dtype=torch.float32, device=dev),
                 torch.empty(w.B, w.H, w.n, w.d, dtype=torch.float32, device=dev),
                 torch.empty(w.B, w.H, w.n, w.dv, dtype=torch.float32, device=dev))
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        sets.append((q, k, v, dout, grads, ws))

    def call(i):
        q, k, v, dout, grads, ws = sets[i % copies]
        hla.backward_chunked(q, k, v, dout, chunk=w.chunk, workspace=ws, grads=grads)
    us = time_calls(call, stream, 10, warmup=2)
    res = [{"workload": "masked_hla_bwd_B4_H8_n2048_d64_bf16_w64",
            "entry": "hla_backward_chunked (seven first-order maps in three launches)",
            "us_per_call": us, "single_call_us": dict(_LAST_PCT), "tokens_per_s": w.B * w.n / (us * 1e-6),
            "roofline": roof(tok * per_tok, us)}]

    # the backward of a sequence shard: from an initial state (the previous
    # shard's final state), with a gradient flowing into its own final state,
    # returning the gradient of its initial state; three states more per head
    N = w.B * w.H
    state_b = 4 * (w.d * w.d + 2 * w.d * w.dv + 2 * w.d)
    q0, k0, v0 = sets[0][:3]
    _, _, ini = hla.forward_chunked(q0, k0, v0, chunk=w.chunk, return_state=True)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5590)
    dfin = hla.State(*(0.1 * torch.randn(t.shape, generator=gen, dtype=torch.float32, device=dev)
                       for t in ini.tensors()[:5]))
    dini = hla.State.empty(N, w.d, w.dv, dev)

    def call_shard(i):
        q, k, v, dout, grads, ws = sets[i % copies]
        hla.backward_chunked(q, k, v, dout, chunk=w.chunk, workspace=ws, grads=grads, init=ini,
                             dfinal=dfin, dinit=dini)
    us = time_calls(call_shard, stream, 10, warmup=2)
    res.append({"workload": "masked_hla_bwd_shard_B4_H8_n2048_d64_bf16_w64",
                "entry": "hla_backward_chunked (init, dfinal in; dinit out; first-order maps with carries)",
                "us_per_call": us, "single_call_us": dict(_LAST_PCT), "tokens_per_s": w.B * w.n / (us * 1e-6),
                "roofline": roof(tok * per_tok + 3 * N * state_b, us)})
    return res


def small_forward(dev, stream):
    import torch

    import associative_scan_sequence_amd as hla
    import hla_inputs as inputs

    res = []
    # small fp32 forward (launch-bound: a correctness workload)
    w = inputs.SMALL_FP32
    q, k, v = inputs.qkv_on_device(w.B, w.H, w.n, w.d, w.dv, w.dtype, 5300, dev)
    out = torch.empty(w.B, w.H, w.n, w.dv, dtype=torch.float32, device=dev)
    ws = torch.zeros(hla.workspace_size(w.B, w.H, w.n, w.d, w.dv, dtype=w.dtype), dtype=torch.uint8,
                     device=dev)
    us = time_calls(lambda i: hla.forward_chunked(q, k, v, out=out, workspace=ws), stream, 50)
    pct = dict(_LAST_PCT)
    # the same calls replayed from a HIP graph: the launch cost without the host's
    reps = 50
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(reps):
            hla.forward_chunked(q, k, v, out=out, workspace=ws)
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "graph replay differs from the eager result"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        g.replay()
        e1.record(stream)
    e1.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / reps
    per_tok = 4 * (2 * w.d + 2 * w.dv)
    res.append({"workload": w.name, "entry": "hla_forward_chunked", "us_per_call": us, "single_call_us": pct,
                "graph_us_per_call": graph_us, "tokens_per_s": w.B * w.n / (us * 1e-6),
                "roofline": roof(w.B * w.H * w.n * per_tok, us)})
    return res


def cpu_baseline(w, q, k, v):
    """The fp64 oracle on the host: one head per thread, as many threads as
    the process may use, at most the heads (B*H) and at most the CPU share
    of one GPU on these hosts (16 threads, the limit the hosts set through
    OMP_NUM_THREADS)."""
    import oracle

    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    share = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    threads = max(1, min(nproc, w.B * w.H, share))
    oracle.forward(q[:, :1, :64], k[:, :1, :64], v[:, :1, :64], want_state=False)  # load/build
    reps, t_total = 0, 0.0
    while t_total < 10.0 and reps < 2000:
        t0 = time.perf_counter()
        oracle.forward(q, k, v, want_state=False, threads=threads)
        t_total += time.perf_counter() - t0
        reps += 1
    tokens = w.B * w.n * reps
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(), "nproc": nproc, "thread_cap": share,
            "sample": f"the full {w.name} workload ({w.B * w.H} heads), {reps} repetition(s), "
                      f"{t_total:.1f} s; fp64 serial recurrence, one head per thread, "
                      f"{threads} threads = min(nproc {nproc}, heads {w.B * w.H}, CPU share {share})"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the heads shard across GPUs with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import associative_scan_sequence_amd as hla
    import hla_inputs as inputs

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    if args.copy_calibration:
        copy_calibration()
        return
    dev = torch.device("cuda:0")
    if args.copy_ceiling:
        print(json.dumps(copy_ceiling(dev)))
        return
    if args.only:
        for rec in secondary_workloads(dev, torch.cuda.Stream(device=dev), only=args.only):
            print(json.dumps(rec))
        return
    w = inputs.FWD_D64
    q, k, v = inputs.workload_qkv(w, args.seed)
    alg = algorithmic_bytes(w)
    nsets = max(2, math.ceil(2 * MALL_BYTES / alg))
    sets = []
    for _ in range(nsets):
        qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
        out = torch.empty(w.B, w.H, w.n, w.dv, dtype=torch.float32, device=dev)
        ws = torch.zeros(hla.workspace_size(w.B, w.H, w.n, w.d, w.dv, chunk=w.chunk),
                         dtype=torch.uint8, device=dev)
        sets.append((qg, kg, vg, out, ws))

    def step(i):
        qg, kg, vg, out, ws = sets[i % nsets]
        hla.forward_chunked(qg, kg, vg, chunk=w.chunk, out=out, workspace=ws)

    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    # quick sampled parity guard (two heads) against the oracle
    import oracle
    ro, _, _ = oracle.forward(q[:1, :2], k[:1, :2], v[:1, :2], want_state=False)
    o = sets[0][3][:1, :2].cpu().double().numpy()
    err = float((abs(o - ro).max(axis=-1) / abs(ro).max(axis=-1)).max())
    assert err <= 2e-3, f"parity guard failed: row error {err:.3e}"

    K = args.steps
    eager_ms = None
    if not args.eager:
        with torch.cuda.stream(stream):
            for i in range(nsets):  # every output buffer gets its eager result
                step(i)
        torch.cuda.synchronize()
        ref = [s[3].clone() for s in sets]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(K):
                step(i)
        for rep in range(2):  # replays with eager work and syncs between them
            for s in sets:
                s[3].fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for s, r in zip(sets, ref):
                assert torch.equal(s[3], r), "graph replay differs from the eager result"
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        e1.synchronize()
        ms_total = e0.elapsed_time(e1)
    # eager timing (for reference, or as the headline with --eager)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(K):
            step(i)
        e1.record(stream)
    e1.synchronize()
    eager_ms = e0.elapsed_time(e1) / K
    if args.eager:
        ms_total = eager_ms * K
    torch.cuda.synchronize()
    # single calls, each between its own events: cold (caches evicted before
    # every call by a 1 GiB write) and warm (one input set, back to back)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = percentiles(event_times(step, stream, args.calls, flush=scratch))
    warm = percentiles(event_times(lambda i: step(0), stream, args.calls))
    del scratch
    for s in sets:
        assert hla.give_ups(s[4]) == 0, "a cross-workgroup wait gave up"

    ms = ms_total / K
    tokens = w.B * w.n
    value = tokens / (ms * 1e-3)
    achieved = alg / (ms * 1e-3) / 1e9
    rec = {
        "metric": "tokens/sec masked 2nd-order HLA fwd (d=dv=64, n=2048) + % of roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "n": w.n, "d": w.d, "dv": w.dv,
                   "chunk": w.chunk, "normalize": False, "gamma": None, "ridge": 0.0,
                   "timing": "eager" if args.eager else "hip_graph",
                   "input_copies_rotated": nsets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "k_fast64 (the whole hla_forward_chunked call is one launch)",
                     "algorithmic_bytes_per_step": alg},
        "eager_ms_per_step": eager_ms,
        "single_call_us": {"cold": cold, "warm": warm,
                           "how": "HIP events around each eager call on the launch stream; cold: a 1 GiB "
                                  "scratch write before every call (outside the events) evicts L2 and "
                                  "the 256 MB Infinity Cache; warm: one input set, calls back to back"},
        "roofline_single_call_p50_cold": {"frac": alg / (cold["p50"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                          "achieved_GBps": alg / (cold["p50"] * 1e-6) / 1e9},
        "parity_guard_row_error": err,
    }
    if not args.headline_only:
        del sets
        torch.cuda.empty_cache()
        rec["workloads"] = secondary_workloads(dev, stream)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
