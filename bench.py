"""Benchmark: key-switches/s at N=2^16, 36+12 x 32-bit primes, on one MI355X.

One step = one ckks_keyswitch call on a batch of 8 ciphertexts at level 36 with
one rotation key (Galois element 5), i.e. the whole hot path (INTT, ModUp,
inner product with the a-half regenerated in-kernel by ChaCha12, ModDown).
Inputs are synthetic and seeded (rns_ckks_key_amd.synth, workload 2), resident
in HBM before timing; R copies of the ciphertexts and keys are rotated so that
repeated steps cannot be served from the 256 MB Infinity Cache.

Output: one JSON line (rank 0).  Besides the headline (regenerated a-half) it
carries the stored-key variant, limb-NTTs/s, the roofline of the dominant
kernel (algorithmic work per launch over its event-timed duration) and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

LOG_N, L, K, DNUM, BITS = 16, 36, 12, 3, 32
N = 1 << LOG_N
BATCH, LEVEL, GALOIS = 8, 36, 5
SMALL_RING = (15, 20, 7, 3)           # log N, ciphertext primes, special primes, dnum of the smaller-ring workload
ROTATE = 4

# ---------------------------------------------------------------- work model
# Algorithmic work in 32-bit VALU lane-op slots (one full-rate op on one lane),
# with gfx950's measured full-rate 32-bit multiplies: a butterfly is one
# Montgomery constant multiply (3 multiplies + 3 adds) plus a modular add and a
# modular subtract; a MAC is a 32x32->64 product accumulated into 96 bits; a
# reduction is the two-word REDC; ChaCha12 is 12 rounds x 4 quarter rounds x 12
# ops / 16 words + feed-forward and rejection.
SLOT = {"bfly": 13, "cmul": 6, "mac": 5, "red": 9, "chacha_word": 42}
VALU_PEAK = 256 * 4 * 16 * 2.4e9      # lane-op slots/s: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz
HBM_PEAK = 8.0e12                      # bytes/s


def digits(level: int, alpha: int) -> list[int]:
    return [min(alpha, level - j * alpha) for j in range((level + alpha - 1) // alpha)]


def work_model(level: int, batch: int, regen: bool, n_keys: int = 1) -> dict:
    """Slots per launch of each kernel class of one key-switch call (batch ct, one key each group)."""
    alpha = -(-L // DNUM)
    dg = digits(level, alpha)
    d = len(dg)
    logc = LOG_N - 10
    col = N // 2 * logc           # butterflies of one column pass over a limb
    row = N // 2 * 10             # butterflies of one row pass over a limb
    e = level + K
    items = batch * n_keys
    w = {}
    w["row"] = batch * level * row * SLOT["bfly"]
    mu = 0
    for a in dg:
        mu += a * col * SLOT["bfly"] + a * N * SLOT["cmul"]
        mu += (e - a) * N * (a * SLOT["mac"] + SLOT["red"]) + (e - a) * col * SLOT["bfly"]
    w["modup_conv"] = batch * mu
    rej = 0.0075  # mean rejection rate over the chain's 48 primes
    words_special = d * K * N * (1 + rej) if regen else 0
    words_final = d * level * N * (1 + rej) if regen else 0
    w["ip_special"] = items * K * (d * row * SLOT["bfly"] + 2 * d * N * SLOT["mac"] + 2 * N * SLOT["red"]
                                   + 2 * row * SLOT["bfly"]) + n_keys * words_special * SLOT["chacha_word"]
    w["moddown_conv"] = items * 2 * (K * col * SLOT["bfly"] + K * N * SLOT["cmul"]
                                     + level * N * (K * SLOT["mac"] + SLOT["red"]) + level * col * SLOT["bfly"])
    w["ip_final"] = items * level * ((d - 1) * row * SLOT["bfly"] + 2 * row * SLOT["bfly"] + 2 * d * N * SLOT["mac"]
                                     + 2 * N * SLOT["red"] + 2 * N * SLOT["cmul"] + 4 * N) \
        + n_keys * words_final * SLOT["chacha_word"]
    return w


def hbm_bytes(level: int, batch: int, regen: bool, n_keys: int = 1) -> float:
    """Compulsory bytes of one call: ciphertexts in and out, and the key rows it must read once."""
    d = len(digits(level, -(-L // DNUM)))
    ct = batch * 2 * level * N * 4
    out = batch * n_keys * 2 * level * N * 4
    key_rows = d * (level + K) * N * 4
    return ct + out + n_keys * key_rows * (1 if regen else 2)


# ---------------------------------------------------------------- helpers

def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("kernels.hip", "modarith.h", "ckks_internal.h"):
        with open(os.path.join(ROOT, "rns_ckks_key_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str) -> dict | None:
    """Per-launch HBM bytes of `kernel` from the committed rocprofv3 counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_keyswitch_batch8_l36.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel-source-hash:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(rf"^\|\s*{kernel}\s*\|\s*([0-9.e+]+)\s*\|\s*([0-9.e+]+)\s*\|", text, re.M)
    if not m:
        return None
    return {"fetch_bytes": float(m.group(1)), "write_bytes": float(m.group(2))}


def time_calls(fn, steps: int, warmup: int, torch) -> float:
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for i in range(steps):
        fn(i)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per call


def cpu_baseline(primes, draw, budget_s: float) -> dict:
    """The oracle as it stands, on host cores, on ciphertexts of the same workload."""
    import numpy as np

    from oracle import ks as oks
    from oracle.params import Params

    pr = Params.make(LOG_N, L, K, DNUM, BITS)
    assert pr.primes == list(primes), "library and oracle chains differ"
    key_b = np.asarray(draw["key_b"], dtype=np.uint64)
    done, t0 = 0, time.perf_counter()
    for b in range(BATCH):
        ct = draw["cts"][b].astype(np.uint64)
        oks.keyswitch(pr, ct, LEVEL, key_b, GALOIS, seed=draw["seed"])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "key-switches/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of the 8 ciphertexts at level 36, g=5, a-half regenerated from the seed "
                      f"(numpy, single-threaded elementwise); {dt:.1f} s on {len(os.sched_getaffinity(0))} "
                      f"available host cores"}


# ---------------------------------------------------------------- main

def make_context(primes, max_batch: int, args):
    from rns_ckks_key_amd.api import Context
    ctx = Context(LOG_N, L, K, DNUM, primes, max_batch=max_batch)
    ctx.set_conv_mfma(args.conv == "matrix")
    return ctx


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--conv", choices=["vector", "matrix"], default="vector",
                    help="base conversion on the vector unit or the matrix cores")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--workload", type=int, choices=[2, 3, 4, 5, 6, 7, 8], default=2,
                    help="2 (default, the headline): batch 8 at level 36; 3: level sweep; 4: hoisted 16 keys; "
                         "5: mixed 64-ciphertext stream; 6: multiply + relinearise + rescale, batch 8 at level 36; "
                         "7: 4 x 4 baby-step/giant-step linear transform at level 36; "
                         "8: smaller ring N=2^15 (20+7 primes, dnum 3), batch 8 at level 20")
    ap.add_argument("--variant", choices=["both", "regen", "stored"], default="both",
                    help="which key variants to time (the headline is always the regenerated one when timed)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (xor with 0) three times, to calibrate HBM counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: key-switching is not sharded across GPUs in this library "
              "(see the design notes); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.randint(0, 2**31 - 1, (128 << 20,), dtype=torch.int32, device="cuda")  # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.bitwise_xor(src, 0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4, "launches": 3}))
        return 0

    from rns_ckks_key_amd import synth
    from rns_ckks_key_amd.api import Context, chain_primes, to_device

    torch.cuda.set_device(0)
    if args.workload != 2:
        return other_workload(args)
    primes = chain_primes(LOG_N, BITS, L + K)
    ctx = make_context(primes, BATCH, args)
    d = synth.draw(2, primes)
    seed = d.keys[0].seed
    cts = np.stack(d.cts)                                   # [8][2][36][N]
    kb_host = synth.uniform_key_rows(2000 + 2, primes, DNUM, N)
    dev_ct = [to_device(cts)]
    dev_kb = [to_device(kb_host)]
    for r in range(1, ROTATE):  # distinct copies: the next step's inputs are not in the Infinity Cache
        dev_ct.append(dev_ct[0].clone())
        dev_kb.append(dev_kb[0].clone())
    dev_ka = [ctx.expand_a(seed) for _ in range(ROTATE)]
    outs = [torch.empty((BATCH, 2, LEVEL, N), dtype=torch.int32, device="cuda") for _ in range(ROTATE)]
    torch.cuda.synchronize()

    def step(i, regen):
        r = i % ROTATE
        ctx.keyswitch(dev_ct[r], LEVEL, dev_kb[r], GALOIS, key_seed=seed if regen else None,
                      key_a=None if regen else dev_ka[r], out=outs[r])

    res = {}
    variants = [v for v in (("regen", True), ("stored", False)) if args.variant in ("both", v[0])]
    for variant, regen in variants:
        ms = time_calls(lambda i: step(i, regen), args.steps, args.warmup, torch)
        ctx.profile(True)
        for i in range(args.steps):
            step(i, regen)
        ctx.profile(False)
        prof = ctx.profile_read()
        res[variant] = {"ms_per_step": ms, "key_switches_per_s": BATCH / (ms * 1e-3), "prof": prof}
        print(f"[bench] {variant}: {ms:.3f} ms per batch of {BATCH}", file=sys.stderr, flush=True)

    # limb-NTTs/s on [8][72][N]
    x = torch.randint(0, 2**31 - 1, (BATCH, 2 * LEVEL, N), dtype=torch.int32, device="cuda")
    xr = x.view(BATCH * 2, LEVEL, N)
    ms_f = time_calls(lambda i: ctx.ntt_fwd(xr, 0), args.steps, args.warmup, torch)
    ms_i = time_calls(lambda i: ctx.ntt_inv(xr, 0), args.steps, args.warmup, torch)
    limbs = BATCH * 2 * LEVEL

    head_name = "regen" if "regen" in res else "stored"
    head = res[head_name]
    wm = work_model(LEVEL, BATCH, head_name == "regen")
    prof = head["prof"]
    per_launch = {k: prof[k][0] / prof[k][1] for k in prof if prof[k][1]}
    dominant = max(per_launch, key=lambda k: prof[k][0])
    t_dom = per_launch[dominant] * 1e-3
    achieved = wm[dominant] / t_dom
    traffic = read_traffic(dominant)
    total_slots = sum(wm.values())
    t_call = head["ms_per_step"] * 1e-3
    out = {
        "metric": "key-switches/sec at N=2^16, 36+12 x 32-bit primes; % of HBM roofline",
        "value": round(head["key_switches_per_s"], 1),
        "unit": "key-switches/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": "single key-switch at bootstrapping scale: batch 8 ciphertexts, level 36, "
                               "one rotation key g=5, a-half regenerated in-kernel by ChaCha12",
                   "N": N, "L": L, "K": K, "dnum": DNUM, "batch": BATCH, "level": LEVEL, "galois": GALOIS,
                   "variant": "regen", "input_copies_rotated": ROTATE},
        "roofline": {"bound": "alu", "kernel": dominant, "achieved": round(achieved / 1e12, 3),
                     "peak": round(VALU_PEAK / 1e12, 3), "unit": "T lane-op slots/s",
                     "frac": round(achieved / VALU_PEAK, 4),
                     "work_per_launch_slots": wm[dominant], "avg_launch_ms": round(per_launch[dominant], 4),
                     "traffic": None if traffic is None else traffic["fetch_bytes"] + traffic["write_bytes"]},
        "hbm_roofline_frac": round(hbm_bytes(LEVEL, BATCH, head_name == "regen") / t_call / HBM_PEAK, 4),
        "valu_frac_whole_call": round(total_slots / t_call / VALU_PEAK, 4),
        "kernel_ms_per_call": {k: round(prof[k][0] / args.steps, 4) for k in prof if prof[k][1]},
        "ntt_limbs_per_s": {"forward": round(limbs / (ms_f * 1e-3)), "inverse": round(limbs / (ms_i * 1e-3)),
                            "shape": [BATCH * 2, LEVEL, N]},
    }
    out["config"]["variant"] = head_name
    out["config"]["conversion"] = "matrix cores (int8 MFMA)" if args.conv == "matrix" else "vector unit"
    if "stored" in res and head_name != "stored":
        st = res["stored"]
        sp = st["prof"]
        out["stored_key"] = {"value": round(st["key_switches_per_s"], 1), "ms_per_step": round(st["ms_per_step"], 4),
                             "hbm_roofline_frac": round(hbm_bytes(LEVEL, BATCH, False) / (st["ms_per_step"] * 1e-3)
                                                        / HBM_PEAK, 4),
                             "kernel_ms_per_call": {k: round(sp[k][0] / args.steps, 4) for k in sp if sp[k][1]}}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(primes, {"cts": cts, "key_b": kb_host, "seed": seed}, args.cpu_budget)
    print(json.dumps(out))
    ctx.close()
    return 0


def other_workload(args) -> int:
    """Workloads 3-8: one JSON line each (not the headline); kernel times from the event timer."""
    import numpy as np
    import torch

    from rns_ckks_key_amd import synth
    from rns_ckks_key_amd.api import Context, chain_primes, to_device

    primes = chain_primes(LOG_N, BITS, L + K)
    variants = [v for v in ("regen", "stored") if args.variant in ("both", v)]
    if args.workload == 6:
        name, unit = "multiply + relinearise (s^2 key) + rescale, N=2^16, batch 8 at level 36 -> 35", "products/s"
    elif args.workload == 7:
        name, unit = ("double-hoisted baby-step/giant-step linear transform, N=2^16, level 36, n1 = n2 = 4 "
                      "(16 diagonals, 3 baby + 3 giant rotation keys g = 5^k)", "transforms/s")
    elif args.workload == 8:
        name, unit = ("smaller ring: N=2^15, 20+7 x 32-bit primes, dnum 3, batch 8 ciphertexts at level 20, "
                      "one rotation key g=5", "key-switches/s")
    else:
        wl = synth.WORKLOADS[args.workload]
        d = synth.draw(args.workload, primes)
        name, unit = wl.name, "key-switches/s"
    res = {"metric": f"workload {args.workload}: {name}", "unit": unit, "n_gpus": 1,
           "dtype": "u32", "data": "synthetic", "steps": args.steps, "warmup": args.warmup}
    if args.workload == 3:
        ctx = make_context(primes, 16, args)
        kb = to_device(synth.uniform_key_rows(3003, primes, DNUM, N))
        seed = d.keys[0].seed
        ka = ctx.expand_a(seed)
        per = {}
        for li, level in enumerate(wl.levels):
            cts = to_device(np.stack(d.cts[16 * li:16 * li + 16]))
            out = torch.empty((16, 2, level, N), dtype=torch.int32, device="cuda")
            for v in variants:
                fn = (lambda i, lv=level, c=cts, o=out, v=v: ctx.keyswitch(c, lv, kb, 5, key_seed=seed if v == "regen"
                                                                           else None, key_a=ka if v == "stored"
                                                                           else None, out=o))
                ms = time_calls(fn, args.steps, args.warmup, torch)
                ctx.profile(True)
                for i in range(args.steps):
                    fn(i)
                ctx.profile(False)
                prof = ctx.profile_read()
                per[f"l{level}_{v}"] = {"key_switches_per_s": round(16 / (ms * 1e-3), 1), "ms_per_call": round(ms, 4),
                                        "kernel_ms": {k: round(prof[k][0] / args.steps, 4) for k in prof if prof[k][1]}}
        res["levels"] = per
    elif args.workload == 4:
        ctx = make_context(primes, 16, args)
        ct = to_device(d.cts[0])
        kbs = [to_device(synth.uniform_key_rows(4000 + k, primes, DNUM, N)) for k in range(len(d.keys))]
        kas = [ctx.expand_a(kd.seed) for kd in d.keys]
        out = torch.empty((16, 2, LEVEL, N), dtype=torch.int32, device="cuda")
        for v in variants:
            keys = [(kbs[k], kd.galois, kd.seed if v == "regen" else None, kas[k] if v == "stored" else None)
                    for k, kd in enumerate(d.keys)]
            fn = lambda i, keys=keys: ctx.keyswitch_hoisted(ct, LEVEL, keys, out=out)
            ms = time_calls(fn, args.steps, args.warmup, torch)
            ctx.profile(True)
            for i in range(args.steps):
                fn(i)
            ctx.profile(False)
            prof = ctx.profile_read()
            res[v] = {"key_switches_per_s": round(16 / (ms * 1e-3), 1), "ms_per_call": round(ms, 4),
                      "hbm_roofline_frac": round(hbm_bytes(LEVEL, 1, v == "regen", 16) / (ms * 1e-3) / HBM_PEAK, 4),
                      "kernel_ms": {k: round(prof[k][0] / args.steps, 4) for k in prof if prof[k][1]}}
    elif args.workload == 6:
        # batch 8 at level 36: x (x) y, relinearisation with the s^2 key, rescale to level 35
        ctx = make_context(primes, BATCH, args)
        rng = np.random.default_rng(6006)
        xs = [to_device(np.stack([np.stack([synth.residues(rng, primes[:LEVEL], N) for _ in range(2)])
                                  for _ in range(BATCH)])) for _ in range(2)]
        kb = to_device(synth.uniform_key_rows(6000, primes, DNUM, N))
        seed = rng.bytes(32)
        ka = ctx.expand_a(seed)
        out = torch.empty((BATCH, 2, LEVEL - 1, N), dtype=torch.int32, device="cuda")
        for v in variants:
            fn = lambda i, v=v: ctx.mul_relin_rescale(xs[0], xs[1], LEVEL, kb, key_seed=seed if v == "regen" else None,
                                                       key_a=ka if v == "stored" else None, out=out)
            ms = time_calls(fn, args.steps, args.warmup, torch)
            ctx.profile(True)
            for i in range(args.steps):
                fn(i)
            ctx.profile(False)
            prof = ctx.profile_read()
            res[v] = {"mul_relin_rescale_per_s": round(BATCH / (ms * 1e-3), 1), "ms_per_call": round(ms, 4),
                      "kernel_ms": {k: round(prof[k][0] / args.steps, 4) for k in prof if prof[k][1]}}
        ms_r = time_calls(lambda i: ctx.rescale(xs[0], LEVEL, out=out), args.steps, args.warmup, torch)
        ctx.profile(True)
        for i in range(args.steps):
            ctx.rescale(xs[0], LEVEL, out=out)
        ctx.profile(False)
        prof = ctx.profile_read()
        res["rescale"] = {"ciphertexts_per_s": round(BATCH / (ms_r * 1e-3), 1), "ms_per_call": round(ms_r, 4),
                          "kernel_ms": {k: round(prof[k][0] / args.steps, 4) for k in prof if prof[k][1]}}
    elif args.workload == 7:
        n1 = n2 = 4
        ctx = make_context(primes, BATCH, args)
        rng = np.random.default_rng(7007)
        ct = to_device(np.stack([synth.residues(rng, primes[:LEVEL], N) for _ in range(2)]))
        ext = primes[:LEVEL] + primes[L:]
        diags = to_device(np.stack([np.stack([synth.residues(rng, ext, N) for _ in range(n1)]) for _ in range(n2)]))
        gs = [pow(5, k, 2 * N) for k in range(1, n1)] + [pow(5, n1 * j, 2 * N) for j in range(1, n2)]
        kbs = [to_device(synth.uniform_key_rows(7000 + i, primes, DNUM, N)) for i in range(len(gs))]
        seeds = [rng.bytes(32) for _ in gs]
        kas = [ctx.expand_a(sd) for sd in seeds]
        out = torch.empty((2, LEVEL, N), dtype=torch.int32, device="cuda")
        for v in variants:
            keys = [(kbs[i], gs[i], seeds[i] if v == "regen" else None, kas[i] if v == "stored" else None)
                    for i in range(len(gs))]
            fn = lambda i, keys=keys: ctx.linear_transform_bsgs(ct, LEVEL, diags, keys[:n1 - 1], keys[n1 - 1:], out=out)
            ms = time_calls(fn, args.steps, args.warmup, torch)
            ctx.profile(True)
            for i in range(args.steps):
                fn(i)
            ctx.profile(False)
            prof = ctx.profile_read()
            res[v] = {"transforms_per_s": round(1 / (ms * 1e-3), 1), "ms_per_call": round(ms, 4),
                      "rotations_per_s": round((n1 * n2) / (ms * 1e-3), 1),
                      "kernel_ms": {k: round(prof[k][0] / args.steps, 4) for k in prof if prof[k][1]}}
        t_diag = res[variants[0]]["kernel_ms"]["diag"] * 1e-3
        # the diagonal sums read the diagonals and the baby steps and write the sums: n1*n2 + 2*(n1-1) + 2*n2
        # extended limbs; the giant-step sum (same timer class) reads n2 ciphertexts and writes one
        diag_bytes = ((n1 * n2 + 2 * (n1 - 1) + 2 * n2) * (LEVEL + K) + (n2 + 1) * 2 * LEVEL) * N * 4
        res["diag_roofline"] = {"bound": "hbm", "achieved_gbs": round(diag_bytes / t_diag / 1e9, 1),
                                "peak_gbs": HBM_PEAK / 1e9, "frac": round(diag_bytes / t_diag / HBM_PEAK, 4)}
    elif args.workload == 8:
        log_n8, l8, k8, d8 = SMALL_RING
        n8 = 1 << log_n8
        primes8 = chain_primes(log_n8, BITS, l8 + k8)
        ctx = Context(log_n8, l8, k8, d8, primes8, max_batch=BATCH)
        rng = np.random.default_rng(8008)
        cts = to_device(np.stack([np.stack([synth.residues(rng, primes8[:l8], n8) for _ in range(2)])
                                  for _ in range(BATCH)]))
        kb = to_device(synth.uniform_key_rows(8000, primes8, d8, n8))
        seed = rng.bytes(32)
        ka = ctx.expand_a(seed)
        out = torch.empty((BATCH, 2, l8, n8), dtype=torch.int32, device="cuda")
        for v in variants:
            fn = (lambda i, v=v: ctx.keyswitch(cts, l8, kb, GALOIS, key_seed=seed if v == "regen" else None,
                                               key_a=ka if v == "stored" else None, out=out))
            ms = time_calls(fn, args.steps, args.warmup, torch)
            ctx.profile(True)
            for i in range(args.steps):
                fn(i)
            ctx.profile(False)
            prof = ctx.profile_read()
            res[v] = {"key_switches_per_s": round(BATCH / (ms * 1e-3), 1), "ms_per_call": round(ms, 4),
                      "kernel_ms": {k: round(prof[k][0] / args.steps, 4) for k in prof if prof[k][1]}}
    else:
        ctx = make_context(primes, 16, args)
        kbs = [to_device(synth.uniform_key_rows(5000 + k, primes, DNUM, N)) for k in range(len(d.keys))]
        kas = [ctx.expand_a(kd.seed) for kd in d.keys] if "stored" in variants else None
        cts = [to_device(c) for c in d.cts]
        outs = [torch.empty((2, lv, N), dtype=torch.int32, device="cuda") for lv in d.levels]
        for v in variants:
            items = []
            for c in range(len(cts)):
                k = d.key_index[c]
                items.append((cts[c], d.levels[c], kbs[k], wl.galois[k], d.keys[k].seed if v == "regen" else None,
                              kas[k] if v == "stored" else None, outs[c]))
            # one multi-item call: ciphertexts of equal level share launches, and the launch
            # sequences of different levels run concurrently on the library's four streams
            ms = time_calls(lambda i, items=items: ctx.keyswitch_multi(items), args.steps, args.warmup, torch)
            # one call per ciphertext, for comparison
            ms1 = time_calls(lambda i, items=items: [ctx.keyswitch(it[0][None], it[1], it[2], it[3], key_seed=it[4],
                                                                   key_a=None if it[5] is None else it[5],
                                                                   out=it[6][None]) for it in items],
                             args.steps, args.warmup, torch)
            byts = sum(hbm_bytes(lv, 1, v == "regen") for lv in d.levels)
            res[v] = {"key_switches_per_s": round(len(cts) / (ms * 1e-3), 1), "ms_per_stream": round(ms, 4),
                      "hbm_roofline_frac": round(byts / (ms * 1e-3) / HBM_PEAK, 4),
                      "one_call_per_ciphertext": {"key_switches_per_s": round(len(cts) / (ms1 * 1e-3), 1),
                                                  "ms_per_stream": round(ms1, 4)}}
        res["key_set_bytes"] = {"regen": len(d.keys) * DNUM * (L + K) * N * 4,
                                "stored": 2 * len(d.keys) * DNUM * (L + K) * N * 4}
    print(json.dumps(res))
    ctx.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
