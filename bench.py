#!/usr/bin/env python3
"""Benchmark of the FlashAttention forward (libfa.so) on one MI355X.

One step = one fa_fwd launch over the whole workload (every row tile, every head and
batch), inputs already resident in device memory.  Default workload: non-causal MHA prefill,
bf16, head dim 128, 16 heads, batch 4 x 8192 tokens (the 32768-token prefill grid of
https://yetianai.com/news/16520, section "七天跑出的成绩单").  The causal variant of the same
shape, every other workload of the grid (other sequence lengths, GQA, the short random-mask
cases), the default workload through fa_fwd_lse (O plus the per-row log-sum-exp) and the mask
kernels (byte-mask packing and the tile summary, on the B16 H16 S1000 shape) and a packed-document
mask on that shape and a sliding-window mask at S32768 (dense walk vs the tile-summary walk), and
split-KV on small grids (one sequence with one or two heads), and launch time against sequence
length on grids of at most one workgroup per CU (the cost of one key-tile iteration), are timed
alongside and reported under "also".

Prints ONE JSON line.  FLOPs are counted dense, 4*B*Hq*S^2*d, half of that for causal.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s + % of MI355X bf16 MFMA peak (hdim128, causal/non-causal)"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0


def flops(B, H, S, D, mode):
    f = 4.0 * B * H * S * S * D
    return f / 2 if mode == "causal" else f


def time_launches(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps   # ms per launch, HIP events on the launch stream


def launch_spread(fn, n):
    """Per-launch durations, after the timed region: HIP events around each call on the launch
    stream (p10, median and p90 in ms), and, inside each call, the pair the library records
    around its attention kernel alone (fa_set_kernel_events: mean, p10, median and p90 in ms)."""
    import torch
    from attention_forward_fwd_amd import set_kernel_events
    stream = torch.cuda.current_stream()
    mk = lambda: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(n)]
    ev, kev = mk(), mk()
    for a, b in kev:  # (torch creates an event when it is first recorded)
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for (a, b), (ka, kb) in zip(ev, kev):
        a.record(stream)
        set_kernel_events(ka, kb)
        fn()
        b.record(stream)
    set_kernel_events(None, None)
    torch.cuda.synchronize()
    pick = lambda t, f: t[min(n - 1, int(f * n))]
    t = sorted(a.elapsed_time(b) for a, b in ev)
    tk = sorted(a.elapsed_time(b) for a, b in kev)
    return ({"p10": pick(t, 0.1), "median": pick(t, 0.5), "p90": pick(t, 0.9), "n": n},
            {"mean": sum(tk) / n, "p10": pick(tk, 0.1), "median": pick(tk, 0.5),
             "p90": pick(tk, 0.9), "n": n})


def _sysfs_dir(dev_index=0):
    """sysfs directory of the amdgpu device that HIP device `dev_index` is (matched by PCI bus),
    or None.  Only plain file reads follow: no helper program is started."""
    import glob
    import torch
    try:
        p = torch.cuda.get_device_properties(dev_index)
        want = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}."
    except Exception:
        want = None
    cards = sorted(glob.glob("/sys/class/drm/card*/device"))
    for c in cards:
        if want is None or os.path.basename(os.path.realpath(c)).startswith(want):
            return c
    return None


def _read_clock_power(d):
    """(current GFX clock in MHz, socket power in W) from sysfs: the "S:" (current) line of
    pp_dpm_sclk and hwmon power1_input (microwatts); either may be None."""
    import glob
    clk = pw = None
    try:
        for line in open(os.path.join(d, "pp_dpm_sclk")):
            if line.startswith("S:") or line.rstrip().endswith("*"):
                clk = float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
                break
    except (OSError, ValueError, IndexError):
        pass
    for f in glob.glob(os.path.join(d, "hwmon", "hwmon*", "power1_input")) + \
            glob.glob(os.path.join(d, "hwmon", "hwmon*", "power1_average")):
        try:
            pw = int(open(f).read().strip()) / 1e6
            break
        except (OSError, ValueError):
            pass
    return clk, pw


def clock_under_load(fn, seconds=2.0):
    """GFX clock and socket power sampled about every 0.1 s from sysfs (pp_dpm_sclk's current
    line, hwmon power1_input), by a thread of this process reading files, while `fn` runs back to
    back for `seconds` after the timed region: the kernels run at the board's power cap, so the
    clock they get differs from box to box.  None if the files are not readable."""
    import threading
    import torch
    d = _sysfs_dir(torch.cuda.current_device())
    if d is None or _read_clock_power(d) == (None, None):
        return None
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            clk, pw = _read_clock_power(d)
            if clk is not None:
                samples.append((clk, pw))
            stop.wait(0.1)

    th = threading.Thread(target=poll, daemon=True)
    for _ in range(50):   # the GPU is busy before the first reading
        fn()
    t0 = time.time()
    th.start()
    while time.time() - t0 < seconds:
        for _ in range(50):   # enough queued work that the GPU never idles between batches
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=5)
    if not samples:
        return None
    clk = sorted(c for c, _ in samples)
    pws = [w for _, w in samples if w is not None]
    return {"gfx_mhz_median": clk[len(clk) // 2], "gfx_mhz_min": clk[0], "gfx_mhz_max": clk[-1],
            "socket_w_median": sorted(pws)[len(pws) // 2] if pws else None,
            "socket_w_max": max(pws) if pws else None, "n_samples": len(samples),
            "max_clk_mhz": 2400, "source": d,
            "note": "instantaneous sysfs readings: pp_dpm_sclk current line, hwmon power1_input"}


MALL_BYTES = 256 << 20   # MI355X Infinity Cache: inputs rotated past it for HBM-bound timings


def rotation_sets(w, draw):
    """Enough independent input sets (at least 4) that one pass over them exceeds the Infinity
    Cache, so an HBM-bound timing reads its inputs from HBM rather than from the cache."""
    n = max(4, -(-2 * MALL_BYTES // max(1, alg_bytes(w))))
    return [draw(i) for i in range(n)]


def draw_set(inputs, w, i, dev):
    """Input set i of a rotation: Q, K, V (and random mask words) drawn on the device with their
    own seed."""
    import dataclasses
    wi = dataclasses.replace(w, seed=w.seed + 100 + i)
    q, k, v = inputs.make_qkv_device(wi, dev)
    return q, k, v, (inputs.make_bitmask_device(wi, dev) if w.mode == "bitmask" else None)


def alg_bytes(w):
    """Q, K, V (and the mask words) read once, O written once."""
    qo = 2 * w.batch * w.seq_len * w.n_q_heads * w.head_dim * 2
    kv = 2 * w.batch * w.seq_len * w.n_kv_heads * w.head_dim * 2
    mk = w.batch * w.n_q_heads * w.seq_len * ((w.seq_len + 31) // 32) * 4 if w.mode == "bitmask" else 0
    return qo + kv + mk


def time_grid(fa_fwd, inputs, dev, main, steps):
    """Time every other workload of the grid once (inputs drawn on the device): the prefill
    shapes causal and non-causal, the GQA groupings, and the short random-mask cases (the
    latter with algorithmic HBM bytes per second, since they sit below the ridge point)."""
    import torch
    grid = []
    for B, S in inputs.PREFILL_SHAPES:
        for causal in (False, True):
            grid.append(inputs.mha_prefill(B, S, causal))
    for B, S in inputs.PREFILL_SHAPES:
        for hkv in (4, 8):
            for causal in (False, True):
                grid.append(inputs.gqa_prefill(B, S, hkv, causal))
    grid += [inputs.short_masked(512), inputs.short_masked(1000), inputs.tiny_masked()]
    out = {}
    for w in grid:
        if (w.mode, w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads) == (
                main.mode, main.batch, main.seq_len, main.n_q_heads, main.n_kv_heads):
            continue
        q, k, v = inputs.make_qkv_device(w, dev)
        mask = None
        if w.mode == "bitmask":
            mask = inputs.make_bitmask(w).to(dev)
        o = torch.empty_like(q)
        small = w.seq_len <= 1024
        ms = time_launches(lambda: fa_fwd(q, k, v, mode=w.mode, scale=w.scale, mask=mask, out=o),
                           steps * (20 if small else 1), 3)
        f = flops(w.batch, w.n_q_heads, w.seq_len, w.head_dim, w.mode)
        rec = {"ms": ms, "tflops": f / (ms * 1e-3) / 1e12,
               "frac_of_peak": f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        if small:
            if w.n_q_heads > 1:
                # HBM-bound shape: launches cycle through input sets larger than the Infinity
                # Cache together, so Q, K, V and the mask come from HBM; the single-set time
                # above (inputs cache-resident after the first launch) is kept beside it.
                sets = rotation_sets(w, lambda i: draw_set(inputs, w, i, dev))
                outs = [torch.empty_like(q) for _ in sets]
                ctr = [0]

                def rot():
                    i = ctr[0] % len(sets)
                    ctr[0] += 1
                    qq, kk, vv, mm = sets[i]
                    fa_fwd(qq, kk, vv, mode=w.mode, scale=w.scale, mask=mm, out=outs[i])
                ms_cached = ms
                ms = time_launches(rot, steps * 20, len(sets))
                rec.update({"ms": ms, "tflops": f / (ms * 1e-3) / 1e12,
                            "frac_of_peak": f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                            "input_sets": len(sets), "us_one_input_set": ms_cached * 1e3})
                del sets, outs
            gbs = alg_bytes(w) / (ms * 1e-3) / 1e9
            rec.update({"us": ms * 1e3, "alg_bytes": alg_bytes(w), "hbm_gbs": gbs,
                        "frac_of_hbm": gbs / PEAK_HBM_GBS})
        out[w.label] = rec
        del q, k, v, o, mask
    return out


def time_mask_kernels(inputs, dev, steps):
    """fa_pack_mask and fa_mask_tiles on the short random-mask shape (B16 H16 S1000): HBM-bound,
    reported as algorithmic bytes per second (bytes read once + words written once)."""
    import torch
    from attention_forward_fwd_amd import mask_tiles, pack_mask
    w = inputs.short_masked(1000)
    B, H, S = w.batch, w.n_q_heads, w.seq_len
    W, R = (S + 31) // 32, (S + 63) // 64
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 90)
    mbytes = (torch.rand((B, H, S, S), generator=g, device=dev) < 0.5).to(torch.uint8)
    words = torch.empty((B, H, S, W), dtype=torch.int32, device=dev)
    tiles = torch.empty((B, H, R, (R + 31) // 32), dtype=torch.int32, device=dev)
    out = {}
    for name, fn, nbytes in (
            ("fa_pack_mask", lambda: pack_mask(mbytes, out=words), B * H * S * S + words.numel() * 4),
            ("fa_mask_tiles", lambda: mask_tiles(words, out=tiles), words.numel() * 4 + tiles.numel() * 4)):
        ms = time_launches(fn, steps, 3)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"{name} B{B} H{H} S{S}"] = {"us": ms * 1e3, "alg_bytes": nbytes, "hbm_gbs": gbs,
                                         "frac_of_hbm": gbs / PEAK_HBM_GBS}
    del mbytes, words, tiles
    return out


def time_document_mask(inputs, dev, steps):
    """Packed documents (4 per sequence) on the short random-mask shape: the dense walk (every
    key tile loaded, dead ones skipped by the wave ballot) against the walk over the tiles the
    mask's summary marks live (dead tiles neither loaded nor visited).  The summary itself is
    made once per mask (fa_mask_tiles, timed with the mask kernels)."""
    import torch
    from attention_forward_fwd_amd import fa_fwd, mask_tiles
    w = inputs.document_masked(1000, 4)
    q, k, v = inputs.make_qkv_device(w, dev)
    m = inputs.document_mask(inputs.make_bitmask(w), w.extra["n_docs"], seed=w.seed + 1).to(dev)
    tiles = mask_tiles(m)
    o = torch.empty_like(q)
    f = flops(w.batch, w.n_q_heads, w.seq_len, w.head_dim, w.mode)
    out = {}
    for name, kw in (("dense walk", {}), ("tile walk", {"tiles": tiles})):
        ms = time_launches(lambda: fa_fwd(q, k, v, mode="bitmask", scale=w.scale, mask=m, out=o, **kw),
                           steps, 3)
        out[f"{w.label} {name}"] = {"us": ms * 1e3, "dense_equivalent_tflops": f / (ms * 1e-3) / 1e12,
                                     "live_tile_fraction": None}
    # fraction of (row block, key tile) pairs the summary marks live
    t = tiles.cpu().numpy().view("uint32")
    R = (w.seq_len + 63) // 64
    bits = sum(bin(int(x)).count("1") for x in t.ravel())
    for rec in out.values():
        rec["live_tile_fraction"] = bits / (w.batch * w.n_q_heads * R * R)
    del q, k, v, m, tiles, o
    return out


def time_sliding_window(inputs, dev, steps):
    """A sliding-window mask (keys within 1024 positions of the query, random bits inside) at
    B1 H16 S32768 fp16 d64: the dense walk against the walk over the tiles its summary marks live."""
    import torch
    from attention_forward_fwd_amd import fa_fwd, mask_tiles
    w = inputs.Workload("sliding-window", "f16", "bitmask", 1, 32768, 16, 16, 64, seed=2200)
    q, k, v = inputs.make_qkv_device(w, dev)
    m = inputs.band_mask(inputs.make_bitmask_device(w, dev), 1024)
    tiles = mask_tiles(m)
    o = torch.empty_like(q)
    f = flops(w.batch, w.n_q_heads, w.seq_len, w.head_dim, w.mode)
    R = (w.seq_len + 63) // 64
    live = int(sum(bin(int(x)).count("1") for x in tiles.cpu().numpy().view("uint32").ravel()))
    rec = {"live_tile_fraction": live / (w.n_q_heads * R * R)}
    for name, kw in (("dense walk", {}), ("tile walk", {"tiles": tiles})):
        ms = time_launches(lambda: fa_fwd(q, k, v, mode="bitmask", scale=w.scale, mask=m, out=o, **kw),
                           steps, 3)
        rec[name] = {"ms": ms, "dense_equivalent_tflops": f / (ms * 1e-3) / 1e12}
    del q, k, v, m, tiles, o
    return {w.label: rec}


def time_split_kv(inputs, dev, steps):
    """Split-KV on small grids (one sequence, one or two heads, so few workgroups): the call
    without splitting against the automatic split (kv_splits=0)."""
    import torch
    from attention_forward_fwd_amd import fa_fwd
    out = {}
    for H, S, causal in ((1, 32768, False), (1, 32768, True), (2, 16384, False), (1, 4096, False)):
        w = inputs.Workload("small-grid", "bf16", "causal" if causal else "none", 1, S, H, H, 128,
                            seed=6000 + H * 10 + (1 if causal else 0))
        q, k, v = inputs.make_qkv_device(w, dev)
        o = torch.empty_like(q)
        f = flops(1, H, S, 128, w.mode)
        rec = {}
        for name, splits in (("no split", 1), ("auto split", 0)):
            ms = time_launches(lambda: fa_fwd(q, k, v, mode=w.mode, scale=w.scale, out=o,
                                              kv_splits=splits), steps, 3)
            rec[name] = {"ms": ms, "tflops": f / (ms * 1e-3) / 1e12}
        out[w.label] = rec
        del q, k, v, o
    return out


def time_key_tile_chain(inputs, dev, steps):
    """Launch time against sequence length on grids of at most one workgroup per CU (B1 H16,
    inputs resident after the first launch), so the slope is the cost of one 64-key tile
    iteration with nothing else on the CU to hide its load round trip; the d64 shapes also at
    B16 (several workgroups per CU) beside them."""
    import torch
    from attention_forward_fwd_amd import fa_fwd
    out = {}
    for D, dtype, mode, batches in ((64, "f16", "none", (1, 16)), (64, "f16", "bitmask", (1, 16)),
                                    (128, "bf16", "none", (1,))):
        for B in batches:
            us = {}
            for S in (256, 512, 1024, 2048):
                w = inputs.Workload("key-tile-chain", dtype, mode, B, S, 16, 16, D,
                                    seed=6100 + S // 256 + (100 if mode == "bitmask" else 0) + D)
                q, k, v = inputs.make_qkv_device(w, dev)
                mask = inputs.make_bitmask_device(w, dev) if mode == "bitmask" else None
                o = torch.empty_like(q)
                us[S] = 1e3 * time_launches(lambda: fa_fwd(q, k, v, mode=mode, scale=w.scale,
                                                           mask=mask, out=o), steps, 5)
                del q, k, v, o, mask
            rec = {f"S{S}_us": t for S, t in us.items()}
            if B == 1:
                rec["us_per_key_tile_S256_to_S512"] = (us[512] - us[256]) / 4
                rec["us_per_key_tile_S1024_to_S2048"] = (us[2048] - us[1024]) / 16
            out[f"d{D} {mode} B{B} H16"] = rec
    return out


def cpu_baseline(w, q, k, v, mask, o_gpu, budget_s):
    """Time the fp64 oracle on a bounded sample of the same workload (row blocks of one head
    at full key length, as many as fit in budget_s) and check the GPU rows it covers."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    S, H = w.seq_len, w.n_q_heads
    rng = np.random.default_rng(w.seed)
    done_rows, t_used, max_err, sum_err, n_el = 0, 0.0, 0.0, 0.0, 0
    blocks = []
    while t_used < budget_s:
        b, h = int(rng.integers(0, w.batch)), int(rng.integers(0, H))
        r0 = int(rng.integers(0, max(1, S - 256)))
        rows = np.arange(r0, min(S, r0 + 256))
        t0 = time.perf_counter()
        # the (batch, head) slice the rows read, so a call converts only that slice to fp64
        g = h // (w.n_q_heads // w.n_kv_heads)
        ref = oracle.attention_rows(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, g:g + 1],
                                    v[b:b + 1, :, g:g + 1], w.mode, w.scale,
                                    None if mask is None else mask[b:b + 1, h:h + 1], rows=rows)
        t_used += time.perf_counter() - t0
        got = o_gpu[b, rows[0]:rows[-1] + 1, h].float().cpu().numpy().astype(np.float64)
        err = np.abs(got - ref[0, :, 0, :])
        max_err = max(max_err, float(err.max()))
        sum_err += float(err.sum())
        n_el += err.size
        done_rows += len(rows)
        blocks.append((b, h, int(rows[0])))
    per_row = 4.0 * S * w.head_dim * (0.5 if w.mode == "causal" else 1.0)
    tflops = done_rows * per_row / t_used / 1e12
    return {
        "value": tflops, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
        "sample": f"{done_rows} query rows ({len(blocks)} blocks of 256 rows, one head each) at "
                  f"full key length {S}, fp64 numpy, {t_used:.1f} s; dense-equivalent FLOPs",
        "gpu_vs_oracle_on_sample": {"max_abs": max_err, "mean_abs": sum_err / max(1, n_el)},
    }


WORKLOADS = ("mha", "gqa4", "gqa8", "short-masked", "document-masked", "tiny-masked")


def pick_workload(inputs, name, batch, seq_len, causal):
    if name == "mha":
        return inputs.mha_prefill(batch, seq_len, causal)
    if name in ("gqa4", "gqa8"):
        return inputs.gqa_prefill(batch, seq_len, 4 if name == "gqa4" else 8, causal)
    if name == "short-masked":
        return inputs.short_masked(seq_len)
    if name == "document-masked":
        return inputs.document_masked(seq_len)
    return inputs.tiny_masked()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=WORKLOADS, default="mha",
                    help="timed workload: MHA or GQA prefill (bf16, d128; --batch, --seq-len, "
                         "--causal), the short random-mask case (fp16, d64, B16 H16; --seq-len 512 "
                         "or 1000), the same shape with the mask confined to 4 packed documents per "
                         "sequence (--seq-len, default 1000; --tile-walk), or the tiny masked case")
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--seq-len", type=int, default=None,
                    help="default 8192 for prefill, 512 for short-masked")
    ap.add_argument("--causal", action="store_true")
    ap.add_argument("--tile-walk", action="store_true",
                    help="masked workloads: pass the mask's tile summary, so each workgroup walks only "
                         "the key tiles it keeps a key in")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--clock-seconds", type=float, default=2.0,
                    help="after the timed region, run the workload this long while a thread samples "
                         "the GFX clock and socket power from sysfs (0 = skip)")
    ap.add_argument("--no-also", action="store_true",
                    help="skip the timings of the rest of the grid (other shapes, causal, GQA, masked)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain elementwise kernel (512 MiB read, 512 MiB written) three "
                         "times, so hardware byte counters can be scaled by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the forward shards over independent (batch, KV head) groups with no "
              f"communication, so aggregate throughput is N x the one-GPU value).", file=sys.stderr)
        sys.exit(2)

    import torch
    from attention_forward_fwd_amd import fa_fwd, fa_fwd_lse, inputs

    dev = torch.device("cuda:0")
    seq_len = args.seq_len or {"short-masked": 512, "document-masked": 1000}.get(args.workload, 8192)
    w = pick_workload(inputs, args.workload, args.batch, seq_len, args.causal)
    q, k, v = inputs.make_qkv(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    mask = inputs.make_bitmask(w) if w.mode == "bitmask" else None
    if args.workload == "document-masked":
        mask = inputs.document_mask(mask, w.extra["n_docs"], seed=w.seed + 1)
    maskd = mask.to(dev) if mask is not None else None
    out = torch.empty_like(qd)

    if args.copy_calibration:
        # A plain elementwise kernel of known traffic: reads 512 MiB, writes 512 MiB.
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1, out=dst)
        torch.cuda.synchronize()
        del src, dst

    tiles = None
    if args.tile_walk:
        if w.mode != "bitmask":
            print("--tile-walk applies to the masked workloads only", file=sys.stderr)
            sys.exit(2)
        from attention_forward_fwd_amd import mask_tiles
        tiles = mask_tiles(maskd)

    def step():
        fa_fwd(qd, kd, vd, mode=w.mode, scale=w.scale, mask=maskd, out=out, tiles=tiles)

    main_step = step
    if args.workload == "short-masked" and tiles is None:
        # HBM-bound main workload: cycle through input sets larger than the Infinity Cache.
        # (Not with a tile summary, which belongs to one mask; the packed-document workload
        # keeps its one structured mask.)
        sets = [(qd, kd, vd, maskd)] + rotation_sets(w, lambda i: draw_set(inputs, w, i, dev))[1:]
        ctr = [0]

        def main_step():
            i = ctr[0] % len(sets)
            ctr[0] += 1
            qq, kk, vv, mm = sets[i]
            fa_fwd(qq, kk, vv, mode=w.mode, scale=w.scale, mask=mm, out=out, tiles=tiles)
    ms = time_launches(main_step, args.steps, args.warmup)
    spread, kernel_ms = launch_spread(main_step, args.steps)
    clock = clock_under_load(main_step, args.clock_seconds) if args.clock_seconds > 0 else None
    if main_step is not step:
        step()   # the output checked against the oracle below is that of the seeded set
        torch.cuda.synchronize()
    f = flops(w.batch, w.n_q_heads, w.seq_len, w.head_dim, w.mode)
    tflops = f / (ms * 1e-3) / 1e12
    o_main = out.clone()

    also = {}
    if not args.no_also:
        # The same workload through fa_fwd_lse (O plus each row's log-sum-exp), right after the
        # main timing so that both see the same clock.
        lse = torch.empty((w.batch, w.n_q_heads, w.seq_len), dtype=torch.float32, device=dev)
        ms_lse = time_launches(lambda: fa_fwd_lse(qd, kd, vd, mode=w.mode, scale=w.scale,
                                                  mask=maskd, out=out, lse=lse),
                               max(5, args.steps // 2), 3)
        lse_entry = {"ms": ms_lse, "tflops": f / (ms_lse * 1e-3) / 1e12,
                     "frac_of_peak": f / (ms_lse * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        del lse
        also = time_grid(fa_fwd, inputs, dev, w, max(5, args.steps // 2))
        also["fa_fwd_lse " + w.label] = lse_entry
        also.update(time_mask_kernels(inputs, dev, 50))
        also.update(time_document_mask(inputs, dev, 100))
        also["split-kv"] = time_split_kv(inputs, dev, 10)
        also.update(time_sliding_window(inputs, dev, 10))
        also["key-tile chain"] = time_key_tile_chain(inputs, dev, 100)

    bytes_alg = alg_bytes(w)   # Q, K, V (and mask) read + O written
    # HBM bytes per launch measured with rocprofv3 byte counters (profiles/traffic.json); only
    # reported while the kernel source is the one the counters were taken on.
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        import hashlib
        src = os.path.join(ROOT, "attention_forward_fwd_amd", "csrc", "fa_fwd.hip")
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        tr = json.load(open(tfile))
        if tr.get("kernel_source_sha256") == sha:
            traffic = tr.get("per_launch_bytes", {}).get(w.label)
    dname = {"bf16": "bf16", "f16": "fp16"}[w.dtype]
    kname = f"fa_fwd_kernel<{dname}, d{w.head_dim}, {w.mode}>"
    # The roofline divides the attention kernel's own work by its own average duration: the
    # events the library records around it in each call of the spread pass (the V pre-pass,
    # when there is one, is outside them; `value` is the whole call).
    kms = kernel_ms["mean"]
    if w.mode == "bitmask":
        # Below the ridge point (short sequences, d=64): HBM is the roofline.
        gbs = bytes_alg / (kms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS, "traffic": traffic, "algorithmic_bytes": bytes_alg,
                "kernel": kname, "kernel_ms": kernel_ms, "tflops": f / (kms * 1e-3) / 1e12}
    else:
        kt = f / (kms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": kt, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": kt / PEAK_BF16_TFLOPS, "traffic": traffic,
                "algorithmic_bytes": bytes_alg, "kernel": kname, "kernel_ms": kernel_ms}
    desc = {"mha": "MHA prefill", "gqa4": "GQA prefill", "gqa8": "GQA prefill",
            "short-masked": "short random-mask", "document-masked": "packed-document mask",
            "tiny-masked": "tiny random-mask"}[args.workload]
    mode_desc = {"none": "non-causal", "causal": "causal", "bitmask": "bitmask"}[w.mode]
    rec = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "launch_ms": spread,
        "clock_under_load": clock,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{mode_desc} {desc} {w.dtype} d{w.head_dim} "
                               f"H{w.n_q_heads}/{w.n_kv_heads} B{w.batch} S{w.seq_len}",
                   "batch": w.batch, "seq_len": w.seq_len, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "mask_mode": w.mode},
        "roofline": roof,
        "also": also,
    }
    if args.cpu_budget > 0:
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, mask, o_main, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
