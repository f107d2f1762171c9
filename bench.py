"""Benchmark of the WKV7 hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * prefill: the 2.9B-model shape, B=8, T=4096, H=40, N=64, bf16 inputs, fp32
    state, with the fused per-head GroupNorm + bonus epilogue (one layer);
  * decode: 32 layers x B=256 x H=40 resident fp32 states (5.4 GB), 64
    sequential single-token steps, each step calling every layer in order,
    with fresh bf16 inputs for every (token, layer).
Throughput is token*heads per second over both parts (decode counts every
layer's heads).  Inputs are resident in HBM before the timed region.

Prints ONE JSON line.  Extra options (--only, --copy-probe, --steps,
--prefill-shape) exist for profiling runs; "--only prefill --prefill-shape long"
times the long-context prefill instead (B=1, T=65536, H=40, slow decay, no
epilogue), which the chunked path splits into parallel time segments, and
"--only prefill --prefill-shape 0.19b" the 0.19B-model shape (B=4, T=1024,
H=12, initial states ~ N(0, 0.1), no epilogue).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

NAMES = ("r", "w", "k", "v", "kappa", "a")
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
N = 64
PREFILL = dict(B=8, T=4096, H=40)
# prefill shapes: (synthetic config index, shape, fused epilogue)
PREFILL_SHAPES = {"2.9b": (2, PREFILL, True), "long": (4, dict(B=1, T=65536, H=40), False),
                  "0.19b": (1, dict(B=4, T=1024, H=12), False)}
DECODE = dict(layers=32, B=256, H=40, steps=64)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "train"], default="all",
                    help="'train': the training step (forward with stored states + backward) "
                         "on the 2.9B prefill shape, printed as its own line")
    ap.add_argument("--decode-steps", type=int, default=DECODE["steps"],
                    help="tokens per decode run (default 64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=32,
                    help="decode layers (all sequences and heads) the oracle replays")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 4 GiB device copy (counter calibration)")
    ap.add_argument("--prefill-algo", default="auto", choices=["auto", "scan", "chunked"])
    ap.add_argument("--bwd-algo", default="auto", choices=["auto", "scan", "chunked"],
                    help="backward algorithm of --only train (auto: chunked for bf16)")
    ap.add_argument("--prefill-shape", default="2.9b", choices=sorted(PREFILL_SHAPES),
                    help="'long' and '0.19b' need --only prefill")
    ap.add_argument("--prefill-head", type=int, default=64, choices=[64, 128],
                    help="prefill (or training) head size; 128 keeps the model width of the "
                         "2.9B shape (H = 20) and needs --only prefill or --only train")
    ap.add_argument("--decode-head", type=int, default=64, choices=[64, 128],
                    help="decode head size; 128 keeps the state bytes (H = 20) and needs "
                         "--only decode")
    ap.add_argument("--fused", action="store_true",
                    help="prefill or decode from raw keys through the fused prologue, with "
                         "the output gate (needs --only prefill or --only decode)")
    ap.add_argument("--bidir", action="store_true",
                    help="time the bidirectional forward (needs --only prefill)")
    ap.add_argument("--decay-f32", action="store_true",
                    help="the decay w in float32, other vectors bf16 (--only prefill: "
                         "long context; --only train: the training step, dw float32)")
    return ap.parse_args()


SPIN_UP_S = 0.5


def spin_up(torch, step):
    """Untimed repetitions of a short step until about SPIN_UP_S seconds of GPU
    work have run.  A timed run of a few sub-millisecond steps right after start
    would otherwise be measured partly before the GPU's clocks have settled
    under sustained load (the default run's 110 ms decode steps do not need it)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SPIN_UP_S:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


def source_hash(*names):
    """Hash of the kernel sources' code: comments and whitespace are removed
    first, so a profile summary stays attached to the code it measured."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "linear_rnn_sequence_amd", "csrc", n)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(profile_name, src_hash):
    """Per-launch HBM bytes from a committed counter summary, if it was taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_profile_value(profile_name, key, src_hash):
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != src_hash:
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def copy_ceiling(torch, wkv, stream, launch_bytes):
    """Measured HBM ceiling for traffic that reads and writes each byte once: the
    library's streaming copy (rwkv7_stream_copy) over one 4 GiB buffer, and in
    launches that each copy `launch_bytes` (cycling through 4 GiB so that no
    launch finds its data in the caches).  HIP events on `stream`; GB/s count the
    bytes read plus the bytes written."""
    total = 4 << 30
    n_pieces = max(1, total // launch_bytes)
    src = torch.empty(total // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            a, b = ev(), ev()
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    def whole():
        wkv.stream_copy(src, dst, stream=stream)

    n_el = launch_bytes // 4

    def pieces():
        for i in range(n_pieces):
            wkv.stream_copy(src[i * n_el:(i + 1) * n_el], dst[i * n_el:(i + 1) * n_el],
                            stream=stream)

    timed(whole, 3)
    whole_ms = timed(whole, 10)
    timed(pieces, 1)
    piece_ms = timed(pieces, 5) / n_pieces
    del src, dst
    return {"kernel": "rwkv7_stream_copy (non-temporal, 1 KiB per wave access)",
            "GBps_4GiB_one_launch": 2 * total / (whole_ms / 1e3) / 1e9,
            "GBps_at_launch_size": 2 * launch_bytes / (piece_ms / 1e3) / 1e9,
            "launch_bytes_copied": launch_bytes}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# fp32 VALU peak without packed math (the kernels are built with packed fp32
# disabled): 256 CUs x 4 SIMDs x 16 lanes x 2 flop (FMA) x 2.4 GHz
FP32_VALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
# backward flops per token-head: the gradient recurrence (G += dy r^T, the
# column sums dr, dk, db, dw, S^T du, the row sums dv, du: 2N^2 each; the
# cotangent update G diag(w) + du kappa^T: 3N^2) plus one forward recompute of
# the states (probe 2N^2, update 5N^2)
def bwd_flops_per_token_head(n):
    return (19 + 7) * n * n


def workload_name(args, long_shape, do_prefill, do_decode):
    if args.prefill_head == 128:
        return ("2.9B-width WKV7 prefill at head size 128: B8 T4096 H20 N128 with fused "
                "GroupNorm+bonus epilogue")
    if args.prefill_shape == "0.19b":
        return ("0.19B-shape WKV7 prefill B4 T1024 H12 N64 from initial states ~ N(0, 0.1) "
                "(no epilogue)")
    if long_shape:
        return ("long-context WKV7 prefill B1 T65536 H40 N64 (slow decay, no epilogue"
                + (", decay w in float32)" if args.decay_f32 else ")"))
    pre = ("2.9B-shape WKV7 prefill B8 T4096 H40 N64 with fused GroupNorm+bonus epilogue"
           + (" (bidirectional: epilogue on the sum of both passes)" if args.bidir else "")
           + (" and the fused prologue (kappa, k-tilde from raw keys) and output gate"
              if args.fused else ""))
    dec = ("decode of 64 tokens through 32 layers x B256 x H40 resident fp32 states"
           if args.decode_head == 64 else
           "decode of 64 tokens through 32 layers x B256 x H20 resident fp32 states of head "
           "size 128")
    if args.fused and do_decode and not do_prefill:
        dec += ", fed from raw keys through the fused prologue, with the output gate"
    if do_prefill and do_decode:
        return "2.9B-shape WKV7: " + pre.replace("2.9B-shape WKV7 ", "") + ", then " + dec
    return pre if do_prefill else "2.9B-shape WKV7 " + dec


def _slow_decay_f32(px):
    """The long-context draw's decay before its bf16 rounding: the same recipe and
    seed with dtype 'bf16_w32' keeps w in float32 (all other vectors identical)."""
    import synth

    m = px["meta"]
    x = synth.draw(m["B"], m["T"], m["H"], m["N"], seed=m["seed"], dtype="bf16_w32",
                   w_recipe="slow", a_mean=2.0)
    for n in NAMES:
        if n != "w":
            assert np.array_equal(x[n], px[n])
    return x["w"]


def bench_train(args, torch, wkv, synth, dev):
    """Training step on the 2.9B prefill shape (no epilogue): forward with stored
    states + backward, inputs and cotangents resident before timing.  At head size
    128 the model width is kept (H = 20)."""
    N = args.prefill_head
    B, T, H = PREFILL["B"], PREFILL["T"], PREFILL["H"] * 64 // N
    if N == 64:
        px = synth.config_inputs(2)
    else:  # the 2.9B-shape recipe at head size 128, without the epilogue
        c = synth.CONFIGS[2]
        px = synth.draw(B, T, H, N, seed=2, dtype=c["dtype"], s0=c["s0"],
                        w_recipe=c["w_recipe"], a_mean=c["a_mean"])
    bf = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    ins = [bf(px[n]) for n in NAMES]
    if args.decay_f32:  # the same decays held in float32 (dtype RWKV7_DT_BF16_W32)
        ins[1] = ins[1].float()
    dy_bits, ds_T = synth.cotangents(B, T, H, N, seed=102, dtype="bf16")
    dy, dst = bf(dy_bits), torch.from_numpy(ds_T).to(dev)
    ws_bytes = wkv.forward_workspace_bytes(B, T, H, N, dtype="bf16", algo=args.prefill_algo)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    y = torch.empty_like(ins[0])
    s_out = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    ck = torch.empty((B, H, (T + 15) // 16, N, N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty_like(ins[1] if i == 1 else ins[0]) for i in range(6))
    ds0 = torch.empty_like(s_out)
    bws = wkv.backward_workspace_bytes(B, T, H, N, dtype="bf16", algo=args.bwd_algo)
    bwork = torch.empty(max(bws, 16), dtype=torch.uint8, device=dev)
    chunked_bwd = N == 64 and bws > 0
    stream = torch.cuda.current_stream()

    def fwd():
        wkv.forward_train(*ins, algo=args.prefill_algo, y=y, s_out=s_out, s_ckpt=ck,
                          workspace=ws)

    def bwd():
        wkv.backward(*ins, dy, ck, dst, grads=grads, ds0=ds0, algo=args.bwd_algo,
                     workspace=bwork)

    for wi in range(args.warmup):
        fwd()
        bwd()
        if wi == 0:
            torch.cuda.synchronize()
            g_first = [g.float().cpu().numpy() for g in grads] + [ds0.cpu().numpy()]
    torch.cuda.synchronize()
    spin_up(torch, lambda: (fwd(), bwd()))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        fwd()
        bwd()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / max(args.steps, 1)
    # each half alone, events on the launch stream around single calls
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(3)]
    for e in ev:
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        e[2].record(stream)
        bwd()
        e[3].record(stream)
    torch.cuda.synchronize()
    fwd_ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.median([e[2].elapsed_time(e[3]) for e in ev]))

    work = B * T * H
    bwd_flops = work * bwd_flops_per_token_head(N)
    tf = bwd_flops / (bwd_ms / 1e3) / 1e12
    nck = (T + 15) // 16
    wx = 2 if args.decay_f32 else 0  # extra bytes per decay element (w in, dw out)
    fwd_bytes = work * (7 * 2 + wx) * N + B * H * N * N * 4 * (1 + nck)
    bwd_bytes = work * (13 * 2 + 2 * wx) * N + B * H * N * N * 4 * (2 + nck)
    src = (source_hash("wkv7_backward_chunked.hip", "wkv7_device.h", "wkv7_mfma.h")
           if chunked_bwd else source_hash("wkv7_backward.hip", "wkv7_device.h"))
    out = {
        "metric": "WKV7 training tokens x heads per second (forward with stored states + backward)",
        "value": work / (ms_per_step / 1e3),
        "unit": "token*heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; recipes of the pages' parameterisations)",
        "config": {"workload": ("2.9B-shape WKV7 training step: forward with fp32 states stored "
                                "every 16 tokens, then backward to r, w, k, v, kappa, a, S0; "
                                + ("B8 T4096 H40 N64, no epilogue" if N == 64 else
                                   "2.9B width at head size 128: B8 T4096 H20 N128, "
                                   "no epilogue")),
                   "B": B, "T": T, "H": H, "N": N, "forward_algo": args.prefill_algo,
                   "backward_algo": "chunked" if chunked_bwd else "scan",
                   "decay_dtype": "f32" if args.decay_f32 else "bf16",
                   "state_dtype": "f32"},
        "roofline": ({"kernel": "wkv7 chunked backward (reverse chain + per-chunk gradients)",
                      "bound": "hbm", "achieved": bwd_bytes / (bwd_ms / 1e3) / 1e9,
                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": bwd_bytes / (bwd_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                      "traffic": (None if args.decay_f32 else
                                  read_traffic("backward_chunked_traffic_b8_t4096_h40.txt", src)),
                      "bytes_per_launch": bwd_bytes, "avg_launch_us": bwd_ms * 1e3,
                      "workspace_bytes": bws,
                      "valu_tflops_equivalent": tf}
                     if chunked_bwd else
                     {"kernel": ("wkv7 backward_kernel<bf16>" if N == 64 else
                                 "wkv7 backward_kernel<bf16, 128> + partial-sum combine"),
                      "bound": "alu",
                      "achieved": tf, "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": tf / FP32_VALU_PEAK_TFLOPS,
                      "traffic": (read_traffic("backward_kernel_traffic_b8_t4096_h40.txt", src)
                                  if N == 64 else None),
                      "workspace_bytes": bws,
                      "flops_per_launch": bwd_flops, "avg_launch_us": bwd_ms * 1e3,
                      "hbm_GBps_algorithmic": bwd_bytes / (bwd_ms / 1e3) / 1e9}),
        "forward_train": {"ms": fwd_ms, "bytes_per_launch": fwd_bytes,
                          "hbm_GBps": fwd_bytes / (fwd_ms / 1e3) / 1e9},
        "backward_ms": bwd_ms,
    }
    if not args.no_cpu_baseline:
        from oracle import grad as og

        b_idx, h_idx = [0, 7], [3, H - 1]
        dy64 = synth.bf16_bits_to_f32(dy_bits).astype(np.float64)
        t0 = time.perf_counter()
        ref = og.backward(*(px.as_f64(n) for n in NAMES), dy64, s0=None,
                          ds_T=ds_T.astype(np.float64), b_idx=b_idx, h_idx=h_idx)
        cpu_s = time.perf_counter() - t0
        errs = {}
        for n, g in zip(NAMES + ("s0",), g_first):
            got = g[np.asarray(b_idx)]
            got = got[:, :, h_idx] if n != "s0" else got[:, h_idx]
            errs["d" + n] = float(np.abs(got - ref[n]).max() / np.abs(ref[n]).max())
        out["parity_sampled"] = dict(errs, bound=2e-2, checked=(
            f"every gradient element of (b, h) in {{0, 7}} x {{3, {H - 1}}}, all 4096 tokens"))
        cpu_work = len(b_idx) * len(h_idx) * T
        out["cpu_baseline"] = {
            "value": cpu_work / cpu_s, "unit": "token*heads/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": (f"float64 autograd gradient oracle ({cpu_model()}, torch CPU, "
                       f"{torch.get_num_threads()} threads) on 4 (b, h) pairs x 4096 tokens "
                       f"({cpu_work} token*heads, forward + backward) in {cpu_s:.2f} s"),
        }
    print(json.dumps(out))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU; the WKV7 path is not sharded "
              "across GPUs (see the sharding notes in the design document). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    cfg_idx, PREFILL, p_with_epi = PREFILL_SHAPES[args.prefill_shape]
    if args.decode_head != 64 and args.only != "decode":
        print("bench.py: --decode-head 128 is a decode-only measurement (--only decode)",
              file=sys.stderr)
        sys.exit(2)
    if args.fused and args.only not in ("prefill", "decode"):
        print("bench.py: --fused needs --only prefill or --only decode", file=sys.stderr)
        sys.exit(2)
    if (args.prefill_shape != "2.9b" or args.bidir) and args.only != "prefill":
        print("bench.py: --prefill-shape long / 0.19b and --bidir are prefill-only "
              "measurements (--only prefill)", file=sys.stderr)
        sys.exit(2)
    if args.prefill_head != 64 and (args.only not in ("prefill", "train")
                                    or args.prefill_shape != "2.9b" or args.fused or args.bidir
                                    or (args.decay_f32 and args.only == "prefill")):
        print("bench.py: --prefill-head 128 times the 2.9B-width prefill alone (--only prefill) "
              "or the training step at that width (--only train)", file=sys.stderr)
        sys.exit(2)
    if args.decay_f32 and args.only not in ("prefill", "train"):
        print("bench.py: --decay-f32 needs --only prefill (long context) or --only train",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_rnn_sequence_amd as wkv
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wkv.lib()

    if args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                          "launches": 3}))
        return

    if args.only == "train":
        bench_train(args, torch, wkv, synth, dev)
        return

    do_prefill = args.only in ("all", "prefill")
    do_decode = args.only in ("all", "decode")
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------------ prefill
    if do_prefill:
        t0 = time.time()
        PN = args.prefill_head
        if PN == 128:  # the 2.9B-shape recipe at head size 128, model width kept (H = 20)
            c = synth.CONFIGS[2]
            PREFILL = dict(PREFILL, H=PREFILL["H"] * 64 // PN)
            px = synth.draw(PREFILL["B"], PREFILL["T"], PREFILL["H"], PN, seed=2,
                            dtype=c["dtype"], s0=c["s0"], w_recipe=c["w_recipe"],
                            a_mean=c["a_mean"], epilogue=c["epilogue"])
        else:
            px = synth.config_inputs(cfg_idx)
        pd = {}
        for n in NAMES:
            pd[n] = torch.from_numpy(px[n].view(np.int16)).to(dev).view(torch.bfloat16)
        if args.decay_f32:  # the decay in float32, from the same draw's values
            if cfg_idx != 4:
                raise SystemExit("--decay-f32 is defined for the long-context shape")
            pd["w"] = torch.from_numpy(_slow_decay_f32(px)).to(dev)
        p_s0 = None if px["s0"] is None else torch.from_numpy(px["s0"]).to(dev)
        e = px["epi"]
        p_epi = None
        if p_with_epi:
            p_epi = {"ln_w": torch.from_numpy(e["ln_w"]).to(dev),
                     "ln_b": torch.from_numpy(e["ln_b"]).to(dev),
                     "r_k": torch.from_numpy(e["r_k"]).to(dev), "eps": e["eps"]}
        B, T, H = PREFILL["B"], PREFILL["T"], PREFILL["H"]
        p_y = torch.empty((B, T, H, PN), dtype=torch.bfloat16, device=dev)
        p_s = torch.empty(((2,) if args.bidir else ()) + (B, H, PN, PN), dtype=torch.float32,
                          device=dev)
        ws_bytes = (wkv.forward_bidir_workspace_bytes if args.bidir else
                    wkv.forward_workspace_bytes)(B, T, H, PN, dtype="bf16",
                                                 algo=args.prefill_algo)
        p_ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        p_gen_s = time.time() - t0

        if args.fused:  # raw keys (the draw's k), prologue parameters and the gate
            pk_k, pk_a, pg = synth.prologue_extras(B, T, H, seed=1000 + cfg_idx)
            f_kk, f_ka = torch.from_numpy(pk_k).to(dev), torch.from_numpy(pk_a).to(dev)
            f_g = torch.from_numpy(pg.view(np.int16)).to(dev).view(torch.bfloat16)

        def prefill():
            if args.fused:
                wkv.forward_fused(*(pd[n] for n in ("r", "w", "k", "v", "a")), f_kk, f_ka,
                                  g=f_g, algo=args.prefill_algo, epilogue=p_epi, y=p_y,
                                  s_out=p_s, workspace=p_ws)
                return
            (wkv.forward_bidir if args.bidir else wkv.forward)(
                *(pd[n] for n in NAMES), s0=p_s0, algo=args.prefill_algo, epilogue=p_epi,
                y=p_y, s_out=p_s, workspace=p_ws)

    # ------------------------------------------------------------------- decode
    if do_decode:
        t0 = time.time()
        L, DB, DS = DECODE["layers"], DECODE["B"], args.decode_steps
        DN = args.decode_head
        DH = DECODE["H"] * 64 // DN  # head size 128: 20 heads, the same state bytes
        pool = synth.decode_states_device(torch, dev, layers=L, B=DB, H=DH, N=DN, seed=3)
        # host copies of the initial states of the layers the oracle replays (parity and
        # CPU baseline), taken before any step
        samp_l = list(range(min(args.cpu_layers, L)))
        s_init = pool[samp_l].cpu().numpy() if not args.no_cpu_baseline else None
        d_in = {n: [] for n in NAMES}
        for t in range(DS):
            one = synth.decode_step_inputs_device(torch, dev, B=DB, H=DH, N=DN, seed=1000 + t,
                                                  count=L)
            for n in NAMES:
                d_in[n].append(one[n])
        d_in = {n: torch.stack(v) for n, v in d_in.items()}  # [DS, L, B, H, N]
        if args.fused:  # raw keys = the draws' k; prologue parameters and gates
            gg = torch.Generator(device=dev)
            gg.manual_seed(77)
            dk_k = 1.0 + 0.1 * torch.randn(DH * DN, device=dev, generator=gg)
            dk_a = 1.0 + 0.1 * torch.randn(DH * DN, device=dev, generator=gg)
            d_g = torch.randn(d_in["r"].shape, device=dev, generator=gg).to(torch.bfloat16)
        d_y = torch.empty((DS, L, DB, DH, DN), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        d_gen_s = time.time() - t0
        n_launch = DS * L
        # The 64 x 32 launches of one decode run are captured once in a HIP graph
        # (argument marshalling happens at capture) and replayed per step.
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        cap_stream = torch.cuda.Stream()
        with torch.cuda.graph(graph, stream=cap_stream):
            for t in range(DS):
                for l in range(L):
                    if args.fused:
                        wkv.decode_fused(*(d_in[n][t, l] for n in ("r", "w", "k", "v", "a")),
                                         dk_k, dk_a, pool[l], g=d_g[t, l], y=d_y[t, l])
                    else:
                        wkv.decode(*(d_in[n][t, l] for n in NAMES), pool[l], y=d_y[t, l])
        torch.cuda.synchronize()
        ev_steps = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in range(args.steps)]

        def decode(events=None):
            if events is not None:
                events[0].record(stream)
            graph.replay()
            if events is not None:
                events[1].record(stream)

    # -------------------------------------------------------- warmup + parity
    for wi in range(args.warmup):
        if do_prefill:
            prefill()
        if do_decode:
            decode()
        if wi == 0:
            torch.cuda.synchronize()
            if do_decode and not args.no_cpu_baseline:
                d_y_first = d_y[:, samp_l].cpu()
                # final states of the first and last layer after one 64-token run
                d_s_first = {l: pool[l].cpu().numpy() for l in (0, L - 1) if l in samp_l}
            if do_prefill:
                p_y_first = p_y.float().cpu().numpy()
                p_s_first = p_s.cpu().numpy()
    torch.cuda.synchronize()
    if not do_decode:
        spin_up(torch, prefill)

    # ------------------------------------------------------------- timed region
    launch_ms = []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        if do_prefill:
            prefill()
        if do_decode:
            # duration of this step's 2048 decode launches, read after the final sync
            decode(ev_steps[len(launch_ms)])
            launch_ms.append(ev_steps[len(launch_ms)])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / max(args.steps, 1)

    # prefill kernel time alone (events around each prefill call, outside the timed loop)
    prefill_ms = None
    if do_prefill:
        pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(3)]
        for a, b in pe:
            a.record(stream)
            prefill()
            b.record(stream)
        torch.cuda.synchronize()
        prefill_ms = float(np.median([a.elapsed_time(b) for a, b in pe]))

    work = 0
    if do_prefill:
        work += PREFILL["B"] * PREFILL["T"] * PREFILL["H"]
    if do_decode:
        work += DS * L * DB * DH
    value = work / (ms_per_step / 1e3)

    long_shape = args.prefill_shape == "long"
    out = {
        "metric": ("WKV7 tokens x heads per second (long-context prefill)" if long_shape else
                   "WKV7 tokens x heads per second (0.19B-shape prefill)"
                   if args.prefill_shape == "0.19b" else
                   "WKV7 tokens x heads per second (bidirectional 2.9B-shape prefill)"
                   if args.bidir else
                   "WKV7 tokens x heads per second (2.9B-width prefill, head size 128)"
                   if do_prefill and args.prefill_head == 128 else
                   "WKV7 tokens x heads per second (2.9B-shape prefill)"
                   if do_prefill and not do_decode else
                   "WKV7 tokens x heads per second (B=256 decode)"
                   if do_decode and not do_prefill else
                   # the default run: the headline metric of the workload
                   "WKV7 tokens\u00d7heads/s and % HBM roofline (2.9B-shape prefill + B=256 "
                   "decode)"),
        "value": value,
        "unit": "token*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; recipes of the pages' parameterisations)",
        "config": {
            "workload": workload_name(args, long_shape, do_prefill, do_decode),
            "prefill": dict(PREFILL, N=PN, algo=args.prefill_algo, epilogue=p_with_epi,
                            workspace_bytes=ws_bytes, bidirectional=args.bidir,
                            fused_prologue=args.fused,
                            decay_dtype="f32" if args.decay_f32 else "bf16")
            if do_prefill else None,
            "decode": dict(DECODE, N=DN, H=DH, steps=args.decode_steps) if do_decode else None,
            "state_dtype": "f32",
        },
    }

    copy_cc = None
    if do_decode:
        run_ms = np.array([a.elapsed_time(b) for a, b in launch_ms])
        avg_ms = float(run_ms.sum() / (len(run_ms) * n_launch))  # per launch, gaps included
        # state in and out, six vectors in and y out (fused: r, w, k, v, a and g in)
        bytes_per_launch = DB * DH * (2 * DN * DN * 4 + 7 * DN * 2)
        achieved = bytes_per_launch / (avg_ms / 1e3) / 1e9
        traffic = (read_traffic("decode_kernel_traffic.txt",
                                source_hash("wkv7_decode.hip", "wkv7_device.h"))
                   if DN == 64 and not args.fused else None)
        out["roofline"] = {
            "kernel": f"wkv7 decode_kernel<bf16, N={DN}> (one layer, B256 x H{DH})",
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "bytes_per_launch": bytes_per_launch, "avg_launch_us": avg_ms * 1e3,
            "launches_timed": int(len(run_ms) * n_launch),
            "timing": "HIP events around each replay of the 2048-launch decode graph / 2048",
        }
        out["decode_ms_per_step"] = float(run_ms.mean())
        # the same achieved rate against a copy that moves each launch's state bytes
        cc = copy_ceiling(torch, wkv, stream, DB * DH * DN * DN * 4)
        copy_cc = cc
        out["roofline"]["copy_ceiling"] = cc
        out["roofline"]["frac_of_copy"] = achieved / cc["GBps_at_launch_size"]
    if do_prefill:
        B, T, H = PREFILL["B"], PREFILL["T"], PREFILL["H"]
        # six inputs + y, the final state (and the initial one when given), and the
        # epilogue parameters when fused
        p_bytes = (B * T * H * (7 + (1 if args.decay_f32 else 0)) * PN * 2
                   + B * H * PN * PN * 4 * (1 if p_s0 is None else 2))
        if p_with_epi:
            p_bytes += 2 * H * PN * 4 + H * PN * 4
        ach = p_bytes / (prefill_ms / 1e3) / 1e9
        chunked = args.prefill_algo in ("auto", "chunked")
        src = source_hash("wkv7_chunked.hip", "wkv7_device.h", "wkv7_mfma.h")
        plain_29b = (chunked and args.prefill_shape == "2.9b" and not args.fused
                     and not args.bidir and PN == 64)
        traffic = (read_traffic("chunked_kernel_traffic_b8_t4096_h40_epilogue.txt", src)
                   if plain_29b else None)
        out["prefill"] = {
            "ms": prefill_ms, "token_heads_per_s": B * T * H / (prefill_ms / 1e3),
            "algo": args.prefill_algo,
            "roofline": {"kernel": ("wkv7 chunked prefill (all its launches)" if chunked else
                                    "wkv7 scan_kernel<bf16>"),
                         "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBS, "traffic": traffic,
                         "bytes_per_launch": p_bytes},
        }
        if copy_cc is None:
            copy_cc = copy_ceiling(torch, wkv, stream, 256 << 20)
        out["prefill"]["roofline"]["frac_of_copy"] = ach / copy_cc["GBps_4GiB_one_launch"]
        if not do_decode:
            out["prefill"]["roofline"]["copy_ceiling"] = copy_cc
        if plain_29b:
            # executed MFMA work per launch is fixed by the kernel (counted once with
            # SQ_INSTS_VALU_MFMA_MOPS_BF16); divided by the live duration it gives the
            # MFMA utilisation against the 2.5 PFLOP/s dense bf16 peak
            mf = read_profile_value("chunked_kernel_mfma_b8_t4096_h40_epilogue.txt",
                                    "mfma_bf16_flops_per_launch", src)
            if mf is not None:
                tf = mf / (prefill_ms / 1e3) / 1e12
                out["prefill"]["mfma"] = {"achieved": tf, "peak": BF16_MFMA_PEAK_TFLOPS,
                                          "unit": "TFLOP/s", "frac": tf / BF16_MFMA_PEAK_TFLOPS,
                                          "flops_per_launch": mf}

    # ------------------------- parity against the oracle, timed as the CPU baseline
    # The oracle runs on the full prefill batch (every head, every token) and on the
    # sampled decode chains (layers 0 and 31 x sequences 0, 1, 255 x 40 heads x all
    # tokens, replayed from their initial states).  Its wall time over that sample is the
    # CPU baseline; the GPU outputs of the first warmup step are compared with it.
    import oracle

    threads = len(os.sched_getaffinity(0))
    par, cpu_work, cpu_s = {}, 0, 0.0
    if do_prefill and not args.no_cpu_baseline:
        sub = [px.as_f64(n) for n in NAMES]
        if args.decay_f32:
            sub[1] = pd["w"].cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        if args.fused:
            g64 = synth.bf16_bits_to_f32(pg).astype(np.float64)
            y_ref, s_ref = oracle.forward_fused(
                *(px.as_f64(n) for n in ("r", "w", "k", "v", "a")), pk_k, pk_a, g=g64, s0=None,
                epilogue=px["epi"] if p_with_epi else None, threads=threads)
        else:
            y_ref, s_ref = (oracle.forward_bidir if args.bidir else oracle.forward)(
                *sub, s0=px["s0"], epilogue=px["epi"] if p_with_epi else None, threads=threads)
        cpu_s += time.perf_counter() - t0
        cpu_work += PREFILL["B"] * PREFILL["T"] * PREFILL["H"]
        del sub
        par["prefill_y_rel_err"] = float(np.abs(p_y_first - y_ref).max() / np.abs(y_ref).max())
        par["prefill_state_rel_err"] = float(np.abs(p_s_first - s_ref).max()
                                             / np.abs(s_ref).max())
        par["prefill_checked"] = "all outputs"
        if long_shape and not args.fused and not args.bidir:
            # the same sequence as 32 chained calls of 2048 tokens (each split into
            # shorter segments of its own), the state passed between them: against the
            # oracle and against the single call
            seg_T = 2048
            st = torch.zeros((PREFILL["B"], PREFILL["H"], N, N), dtype=torch.float32, device=dev)
            ys = []
            for s_i in range(PREFILL["T"] // seg_T):
                sl = slice(s_i * seg_T, (s_i + 1) * seg_T)
                ys.append(wkv.forward(*(pd[n][:, sl].contiguous() for n in NAMES), s0=st,
                                      s_out=st, algo=args.prefill_algo)[0])
            torch.cuda.synchronize()
            y_chain = torch.cat(ys, 1).float().cpu().numpy()
            par["prefill_chained_y_rel_err"] = float(np.abs(y_chain - y_ref).max()
                                                     / np.abs(y_ref).max())
            par["prefill_chained_state_rel_err"] = float(
                np.abs(st.cpu().numpy() - s_ref).max() / np.abs(s_ref).max())
            par["prefill_drift_single_vs_chained"] = float(np.abs(p_y_first - y_chain).max()
                                                           / np.abs(y_chain).max())
            par["prefill_chained"] = f"{PREFILL['T'] // seg_T} calls of {seg_T} tokens"
            del y_chain, ys
        del y_ref, s_ref
    if do_decode and not args.no_cpu_baseline:
        errs, s_errs = [], []
        for li, l in enumerate(samp_l):
            # inputs of layer l for every token: [DS, B, H, N] -> [B, DS, H, N]
            seq = [np.ascontiguousarray(np.moveaxis(d_in[n][:, l].cpu().double().numpy(), 0, 1))
                   for n in NAMES]
            t0 = time.perf_counter()
            if args.fused:
                gseq = np.ascontiguousarray(
                    np.moveaxis(d_g[:, l].cpu().double().numpy(), 0, 1))
                y_ref, _ = oracle.forward_fused(seq[0], seq[1], seq[2], seq[3], seq[5],
                                                dk_k.cpu().double().numpy(),
                                                dk_a.cpu().double().numpy(), g=gseq,
                                                s0=s_init[li], threads=threads)
            else:
                y_ref, s_ref = oracle.forward(*seq, s0=s_init[li], threads=threads)
                if l in d_s_first:
                    s_errs.append(np.abs(d_s_first[l] - s_ref).max() / np.abs(s_ref).max())
                del s_ref
            cpu_s += time.perf_counter() - t0
            cpu_work += seq[0].shape[0] * seq[0].shape[1] * seq[0].shape[2]
            del seq
            y_got = np.moveaxis(d_y_first[:, li].double().numpy(), 0, 1)
            errs.append(np.abs(y_got - y_ref).max() / np.abs(y_ref).max())
            del y_ref, y_got
        par["decode_y_rel_err"] = float(max(errs))
        if s_errs:
            par["decode_state_rel_err"] = float(max(s_errs))
            par["decode_state_checked"] = (f"final states of layers {sorted(d_s_first)} after "
                                           f"one {DS}-token run (all {DB} sequences x {DH} "
                                           "heads)")
        par["decode_checked"] = (f"every output of layers 0..{len(samp_l) - 1} (all {DB} "
                                 f"sequences x {DH} heads x {DS} tokens)")
    if par:
        par["bound"] = 2e-2
        out["parity_sampled"] = par
    if cpu_work:
        out["cpu_baseline"] = {
            "value": cpu_work / cpu_s, "unit": "token*heads/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"fp64 C oracle ({cpu_model()}, {threads} threads) over {cpu_work} "
                       f"token*heads in {cpu_s:.2f} s: "
                       + (f"the whole prefill batch (B{PREFILL['B']} T{PREFILL['T']} "
                          f"H{PREFILL['H']}{' with epilogue' if p_with_epi else ''})"
                          if do_prefill else "")
                       + (" and " if do_prefill and do_decode else "")
                       + (f"the full decode runs of {len(samp_l)} layers" if do_decode else "")),
        }

        # the same oracle on one host core, over a bounded sample of the same work
        t0 = time.perf_counter()
        if do_prefill and not args.fused and not args.bidir:
            one = [px.as_f64(n)[:1] for n in NAMES]
            if args.decay_f32:
                one[1] = pd["w"][:1].cpu().numpy().astype(np.float64)
            s0_one = None if px["s0"] is None else px["s0"][:1]
            t0 = time.perf_counter()
            oracle.forward(*one, s0=s0_one, epilogue=px["epi"] if p_with_epi else None,
                           threads=1)
            one_work, one_what = one[0].shape[1] * one[0].shape[2], "batch 0 of the prefill"
        elif do_decode and not args.fused:
            seq = [np.ascontiguousarray(np.moveaxis(d_in[n][:, 0].cpu().double().numpy(), 0, 1))
                   for n in NAMES]
            t0 = time.perf_counter()
            oracle.forward(*seq, s0=s_init[0], threads=1)
            one_work = seq[0].shape[0] * seq[0].shape[1] * seq[0].shape[2]
            one_what = "the decode run of layer 0"
        else:
            one_work = 0
        one_s = time.perf_counter() - t0
        if one_work:
            out["cpu_baseline_1core"] = {
                "value": one_work / one_s, "unit": "token*heads/s", "cores": 1,
                "kind": "oracle",
                "sample": f"fp64 C oracle on 1 thread over {one_work} token*heads "
                          f"({one_what}) in {one_s:.2f} s"}

    print(json.dumps(out))


if __name__ == "__main__":
    main()
