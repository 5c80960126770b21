"""Benchmark: key-switches/s at N=2^16, 36+12 x 32-bit primes, on one MI355X.

One step = one ckks_keyswitch call on a batch of 8 ciphertexts at level 36 with
one rotation key (Galois element 5), i.e. the whole hot path (INTT, ModUp,
inner product with the a-half regenerated in-kernel by ChaCha12, ModDown).
Inputs are synthetic and seeded (rns_ckks_key_amd.synth, workload 2), resident
in HBM before timing; R copies of the ciphertexts and keys are rotated so that
repeated steps cannot be served from the 256 MB Infinity Cache.

Timing.  Before anything is timed, both key variants run alternately for a fixed
wall time (--prewarm seconds, whatever --warmup says), so the GPU's clocks have
settled for both; then --warmup calls of each.  The headline is exactly --steps
calls of the regenerated variant, bracketed by device synchronisations and HIP
events on the stream the library launches on, with an event between calls.
Then --rounds more blocks of --steps calls of each variant alternate (the order
flips every round); the per-call samples of all blocks give the median, p10 and
p90 of each variant.  Per-kernel times come from the library's per-launch event
timer in separate, also alternating, blocks.

Output: one JSON line.  Besides the headline it carries the stored-key variant,
limb-NTTs/s (ring 2^16 batch and the 2^12 ciphertext), workloads 3-5 in both
variants (unless --no-extra), the roofline of the dominant kernel and the CPU
oracle timed on a bounded sample of the same workload (unless --no-cpu).

Parity gate.  The oracle switches of that sample (every ciphertext of the batch
with the stored a-half, one with the regenerated one) are compared bit for bit
with the timed call's outputs on the same inputs, in both variants; the line
carries the result under "parity", and a mismatch withholds "value" (null) and
makes the exit status 1.  With --no-cpu nothing is compared.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

LOG_N, L, K, DNUM, BITS = 16, 36, 12, 3, 32
N = 1 << LOG_N
BATCH, LEVEL, GALOIS = 8, 36, 5
SMALL_RING = (15, 20, 7, 3)           # log N, ciphertext primes, special primes, dnum of the smaller-ring workload
TINY = (12, 4, 2, 2, 30)              # log N, L, K, dnum, bits of the small workload
ROTATE = 4

# ---------------------------------------------------------------- work model
# Algorithmic work in 32-bit VALU lane-op slots (one full-rate op on one lane):
# per-unit costs that assume full-rate 32-bit multiplies
# (measured on gfx950): a butterfly is one Montgomery constant multiply (3
# multiplies + 3 adds) plus a modular add and a modular subtract; a MAC is a
# 32x32->64 product accumulated into 96 bits; a reduction is the two-word REDC;
# ChaCha12 is 12 rounds x 4 quarter rounds x 12 ops / 16 words + feed-forward and
# rejection.  These count the method's work, not the compiled instructions (the
# counter table under profiles/ gives those).
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


# ---------------------------------------------------------------- committed counter summaries

def code_text(src: str) -> str:
    """Source text without comments and with whitespace collapsed: what the compiler sees."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash(texts: list[str] | None = None) -> str:
    """Hash of the device sources' code (comments and layout ignored), first 16 hex digits."""
    h = hashlib.sha256()
    for i, f in enumerate(("kernels.hip", "modarith.h", "ckks_internal.h")):
        if texts is None:
            with open(os.path.join(ROOT, "rns_ckks_key_amd", "csrc", f)) as fh:
                src = fh.read()
        else:
            src = texts[i]
        h.update(code_text(src).encode())
    return h.hexdigest()[:16]


def _current_profile(name: str) -> str | None:
    """Text of profiles/<name> if its kernel-source-hash matches the sources (else None)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel-source-hash:\s*([0-9a-f]+)", text)
    return text if m and m.group(1) == kernel_source_hash() else None


def read_traffic(kernel: str) -> dict | None:
    """Per-launch HBM bytes of `kernel` from the committed rocprofv3 counter summary, if still current."""
    text = _current_profile("hbm_traffic_keyswitch_batch8_l36.md")
    m = text and re.search(rf"^\|\s*{kernel}\s*\|\s*([0-9.e+]+)\s*\|\s*([0-9.e+]+)\s*\|", text, re.M)
    return {"fetch_bytes": float(m.group(1)), "write_bytes": float(m.group(2))} if m else None


def read_issue(kernel: str) -> dict | None:
    """VALU instructions and issue fraction of `kernel` from the committed SQ counter summary, if current."""
    text = _current_profile("valu_issue_keyswitch_batch8_l36.md")
    m = text and re.search(rf"^\|\s*{kernel}\s*\|\s*([0-9.e+]+)\s*\|\s*([0-9.e+]+)\s*\|\s*([0-9.]+)\s*\|"
                           rf"\s*([0-9.]+)\s*\|", text, re.M)
    if not m:
        return None
    return {"valu_insts": float(m.group(1)), "cycles": float(m.group(2)), "cycles_per_valu_inst": float(m.group(3)),
            "issue_frac": float(m.group(4))}


def read_valu_rates() -> dict | None:
    """Measured lane-op rates (T/s) of gfx950 integer instructions from the committed microbenchmark summary."""
    path = os.path.join(ROOT, "profiles", "valu_rates_gfx950.md")
    if not os.path.exists(path):
        return None
    rates = {}
    text = open(path).read()
    for m in re.finditer(r"^\|\s*(v_[a-z0-9_]+)\s*\|\s*([0-9.]+)\s*\|", text, re.M):
        rates[m.group(1)] = float(m.group(2))
    m = re.search(r"^\|\s*lazy forward butterfly \(T butterflies/s\)\s*\|\s*([0-9.]+)\s*\|", text, re.M)
    if m:
        rates["butterfly"] = float(m.group(1))
    return rates or None


def ntt_roofline(limbs_per_s: float, log_n: int, inverse: bool, rates: dict | None) -> dict:
    """A limb-NTT rate against both ceilings.  One limb-NTT is (N/2) log N butterflies (the
    inverse also multiplies every coefficient by N^-1) and reads and writes its N words once."""
    n = 1 << log_n
    bfly = n // 2 * log_n
    slots = bfly * SLOT["bfly"] + (n * SLOT["cmul"] if inverse else 0)
    nbytes = 2 * n * 4
    out = {"bound": "alu" if slots / VALU_PEAK >= nbytes / HBM_PEAK else "hbm",
           "valu_frac": round(limbs_per_s * slots / VALU_PEAK, 4),
           "hbm_frac": round(limbs_per_s * nbytes / HBM_PEAK, 4),
           "slots_per_limb": slots, "bytes_per_limb": nbytes}
    if rates and "butterfly" in rates:
        # against the measured butterfly throughput, the ceiling of every transform stage
        out["frac_vs_butterfly_rate"] = round(limbs_per_s * bfly / (rates["butterfly"] * 1e12), 4)
    return out


# ---------------------------------------------------------------- timing

def timed_block(fn, steps: int, torch) -> list[float]:
    """Exactly `steps` calls on torch's current stream (the library launches there), bracketed by
    device synchronisations; returns the per-call ms from events recorded between calls."""
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(s)
    for i in range(steps):
        fn(i)
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def prewarm(fns: list, seconds: float, torch) -> float:
    """Runs the calls alternately for at least `seconds` of wall time; returns the time spent."""
    t0 = time.perf_counter()
    i = 0
    while True:
        for fn in fns:
            fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return time.perf_counter() - t0


def stats(samples: list[float], blocks: list[float], items: float, unit: str) -> dict:
    q = statistics.quantiles(samples, n=10, method="inclusive") if len(samples) > 1 else samples * 9
    mean = sum(samples) / len(samples)
    return {unit: round(items / (mean * 1e-3), 1), "ms_per_call": round(mean, 4),
            "ms_median": round(statistics.median(samples), 4), "ms_p10": round(q[0], 4), "ms_p90": round(q[-1], 4),
            f"{unit}_at_median": round(items / (statistics.median(samples) * 1e-3), 1),
            "block_means_ms": [round(b, 4) for b in blocks], "calls_timed": len(samples)}


def interleaved(fns: dict, steps: int, warmup: int, rounds: int, torch, ctx=None, items: float = 1,
                unit: str = "per_s", first: dict | None = None) -> dict:
    """Warm-up, then `rounds` alternating blocks of `steps` calls of each variant (order flipped every
    round), then two alternating profiled blocks each for per-kernel times.  `first` holds per-call
    samples already timed for a variant (the headline block)."""
    for fn in fns.values():
        for i in range(warmup):
            fn(i)
    names = list(fns)
    samples = {k: list((first or {}).get(k, [])) for k in names}
    blocks = {k: ([sum(samples[k]) / len(samples[k])] if samples[k] else []) for k in names}
    for r in range(rounds):
        for k in (names if r % 2 == 0 else names[::-1]):
            t = timed_block(fns[k], steps, torch)
            samples[k] += t
            blocks[k].append(sum(t) / steps)
    out = {k: stats(samples[k], blocks[k], items, unit) for k in names}
    if ctx is not None:
        acc = {k: {} for k in names}
        for r in range(2):
            for k in (names if r % 2 == 0 else names[::-1]):
                ctx.profile(True)
                for i in range(steps):
                    fns[k](i)
                ctx.profile(False)
                for c, (ms, n) in ctx.profile_read().items():
                    if n:
                        a = acc[k].setdefault(c, [0.0, 0])
                        a[0] += ms
                        a[1] += n
        for k in names:
            out[k]["kernel_ms_per_call"] = {c: round(v[0] / (2 * steps), 4) for c, v in acc[k].items()}
            out[k]["kernel_ms_per_launch"] = {c: round(v[0] / v[1], 4) for c, v in acc[k].items()}
    return out


# ---------------------------------------------------------------- CPU baseline (the oracle)

def host_cpu() -> dict:
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    import numpy as np
    return {"cpu_model": model, "available_cores": len(os.sched_getaffinity(0)), "numpy": np.__version__}


def cpu_baseline(primes, cts, key_b, seed: bytes) -> tuple[dict, list]:
    """The oracle as it stands, on the host's cores, on ciphertexts of the headline workload.

    One core: one regenerated-key and one stored-key switch at level 36, and the forward and
    inverse transform of 36 limbs.  All cores: one stored-key switch per worker process at once.
    Also returns the oracle's outputs as (ciphertext index, key variant, [2][36][N]) for the
    parity gate."""
    import numpy as np

    from oracle import ks as oks, pool
    from oracle.chacha import expand_key_a
    from oracle.ntt import intt, ntt
    from oracle.params import Params

    pr = Params.make(LOG_N, L, K, DNUM, BITS)
    assert pr.primes == list(primes), "library and oracle chains differ"
    kb = np.asarray(key_b, dtype=np.uint64)
    ka = expand_key_a(seed, pr.primes, pr.dnum, pr.n)
    t0 = time.perf_counter()
    y_regen = oks.keyswitch(pr, cts[0].astype(np.uint64), LEVEL, kb, GALOIS, seed=seed)
    t_regen = time.perf_counter() - t0
    t0 = time.perf_counter()
    y_stored = oks.keyswitch(pr, cts[1].astype(np.uint64), LEVEL, kb, GALOIS, key_a=ka)
    t_stored = time.perf_counter() - t0
    x = cts[2][0].astype(np.uint64)
    t0 = time.perf_counter()
    y = ntt(x, pr.primes[:LEVEL], pr.psis[:LEVEL])
    t_fwd = time.perf_counter() - t0
    t0 = time.perf_counter()
    intt(y, pr.primes[:LEVEL], pr.psis[:LEVEL])
    t_inv = time.perf_counter() - t0
    n_w = pool.workers(16)
    ex = pool.start_pool((LOG_N, L, K, DNUM, BITS), kb, ka, n_w)
    try:
        jobs = [(cts[i % len(cts)], LEVEL, GALOIS) for i in range(n_w)]
        t0 = time.perf_counter()
        ys = pool.run_jobs(ex, jobs)
        t_all = time.perf_counter() - t0
    finally:
        ex.shutdown()
    outputs = [(0, "regen", y_regen), (1, "stored", y_stored)]
    outputs += [(i % len(cts), "stored", y) for i, y in enumerate(ys)]
    return {"value": round(n_w / t_all, 4), "unit": "key-switches/s", "cores": n_w, "kind": "oracle",
            "sample": f"{n_w} ciphertexts of the batch-8, level-36, g=5 workload, one per worker process "
                      f"(stored a-half), switched at once on {n_w} cores in {t_all:.1f} s; one core: one "
                      f"regenerated ({t_regen:.1f} s) and one stored ({t_stored:.1f} s) switch, and the "
                      f"forward and inverse NTT of 36 limbs",
            "single_core": {"regen_key_switches_per_s": round(1 / t_regen, 4),
                            "stored_key_switches_per_s": round(1 / t_stored, 4),
                            "ntt_limbs_per_s": {"forward": round(LEVEL / t_fwd, 1), "inverse": round(LEVEL / t_inv, 1)}},
            "host": host_cpu()}, outputs


def parity_check(gpu_out: dict, oracle_out: list) -> dict:
    """The timed call's outputs (per key variant, [batch][2][level][N]) against the oracle's outputs
    for the same ciphertexts.  The regenerated a-half equals the stored one, so every oracle output
    is compared with the output of every variant."""
    import numpy as np

    bad, cts = [], set()
    for ci, how, y in oracle_out:
        cts.add(int(ci))
        for v, g in gpu_out.items():
            if not np.array_equal(np.asarray(g[ci], dtype=np.uint64), np.asarray(y, dtype=np.uint64)):
                bad.append({"ciphertext": int(ci), "gpu_variant": v, "oracle_key": how})
    return {"bit_exact": not bad and bool(oracle_out), "ciphertexts": sorted(cts), "variants": sorted(gpu_out),
            "outputs_compared": len(oracle_out) * len(gpu_out), "mismatches": bad,
            "against": "the CPU oracle's switches of the cpu_baseline leg (same inputs and key)"}


# ---------------------------------------------------------------- headline

def make_context(primes, max_batch: int, args):
    from rns_ckks_key_amd.api import Context
    ctx = Context(LOG_N, L, K, DNUM, primes, max_batch=max_batch)
    ctx.set_conv_mfma(args.conv == "matrix")
    return ctx


def headline(args, primes, torch):
    import numpy as np

    from rns_ckks_key_amd import synth
    from rns_ckks_key_amd.api import to_device

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

    fns = {v: (lambda i, rg=(v == "regen"): step(i, rg)) for v in ("regen", "stored")
           if args.variant in ("both", v)}
    head_name = "regen" if "regen" in fns else "stored"
    warmed = prewarm(list(fns.values()), args.prewarm, torch)
    for fn in fns.values():
        for i in range(args.warmup):
            fn(i)
    # the headline: exactly --steps calls of one variant
    head_samples = timed_block(fns[head_name], args.steps, torch)
    head_ms = sum(head_samples) / args.steps
    res = interleaved(fns, args.steps, 0, args.rounds, torch, ctx=ctx, items=BATCH, unit="key_switches_per_s",
                      first={head_name: head_samples})
    for v in res:
        print(f"[bench] {v}: median {res[v]['ms_median']:.4f} ms per batch of {BATCH}", file=sys.stderr, flush=True)

    # limb-NTTs/s on [16][36][N], and on the small workload's ciphertext [2][4][2^12]
    x = torch.randint(0, 2**31 - 1, (BATCH * 2, LEVEL, N), dtype=torch.int32, device="cuda")
    nt = interleaved({"forward": lambda i: ctx.ntt_fwd(x, 0), "inverse": lambda i: ctx.ntt_inv(x, 0)},
                     args.steps, args.warmup, 2, torch, items=BATCH * 2 * LEVEL, unit="limb_ntts_per_s")
    from rns_ckks_key_amd.api import Context
    tiny = Context(TINY[0], TINY[1], TINY[2], TINY[3], synth_chain(TINY), max_batch=1)
    y = torch.randint(0, 2**29, (2, TINY[1], 1 << TINY[0]), dtype=torch.int32, device="cuda")
    nt1 = interleaved({"forward": lambda i: tiny.ntt_fwd(y, 0), "inverse": lambda i: tiny.ntt_inv(y, 0)},
                      args.steps, args.warmup, 2, torch, items=2 * TINY[1], unit="limb_ntts_per_s")
    tiny.close()
    # the timed call's outputs on the first input copy, per variant, for the parity gate (untimed)
    gpu_out = {}
    for v, fn in fns.items():
        outs[0].zero_()
        fn(0)
        torch.cuda.synchronize()
        gpu_out[v] = outs[0].cpu().numpy().view(np.uint32).copy()
    rates = read_valu_rates()
    for st, log_n in ((nt, LOG_N), (nt1, TINY[0])):
        for d in st:
            st[d]["roofline"] = ntt_roofline(st[d]["limb_ntts_per_s_at_median"], log_n, d == "inverse", rates)

    head = res[head_name]
    wm = work_model(LEVEL, BATCH, head_name == "regen")
    per_launch = head["kernel_ms_per_launch"]
    per_call = head["kernel_ms_per_call"]
    dominant = max(per_call, key=per_call.get)
    t_dom = per_launch[dominant] * 1e-3
    achieved = wm[dominant] / t_dom
    # the committed counter summaries were taken on the vector-unit conversion
    traffic = read_traffic(dominant) if args.conv == "vector" else None
    issue = read_issue(dominant) if args.conv == "vector" else None
    total_slots = sum(wm.values())
    t_call = head_ms * 1e-3
    roof = {"bound": "alu", "kernel": dominant, "achieved": round(achieved / 1e12, 3),
            "peak": round(VALU_PEAK / 1e12, 3), "unit": "T lane-op slots/s", "frac": round(achieved / VALU_PEAK, 4),
            "work_per_launch_slots": wm[dominant], "avg_launch_ms": round(per_launch[dominant], 4),
            "traffic": None if traffic is None else traffic["fetch_bytes"] + traffic["write_bytes"],
            "counters": issue}
    if rates and "v_add_u32" in rates:
        # the same work priced at the measured rate of the cheapest (add-class) instruction: a lower bound
        roof["frac_vs_add_rate"] = round(achieved / (rates["v_add_u32"] * 1e12), 4)
        roof["add_rate_T_per_s"] = rates["v_add_u32"]
    out = {
        "metric": "key-switches/sec at N=2^16, 36+12 x 32-bit primes; % of HBM roofline",
        "value": round(BATCH / t_call, 1),
        "unit": "key-switches/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": "single key-switch at bootstrapping scale: batch 8 ciphertexts, level 36, "
                               "one rotation key g=5, a-half regenerated in-kernel by ChaCha12",
                   "N": N, "L": L, "K": K, "dnum": DNUM, "batch": BATCH, "level": LEVEL, "galois": GALOIS,
                   "variant": head_name, "input_copies_rotated": ROTATE,
                   "conversion": "matrix cores (int8 MFMA)" if args.conv == "matrix" else "vector unit"},
        "timing": {"prewarm_s": round(warmed, 2), "prewarm": "both variants alternately before any timing",
                   "headline_block": "exactly `steps` calls after the pre-warm and `warmup` calls of each variant",
                   "interleaved_rounds": args.rounds},
        "roofline": roof,
        "hbm_roofline_frac": round(hbm_bytes(LEVEL, BATCH, head_name == "regen") / t_call / HBM_PEAK, 4),
        "valu_frac_whole_call": round(total_slots / t_call / VALU_PEAK, 4),
        "variants": res,
        "ntt_limbs_per_s": {"ring_2^16_batch": {"shape": [BATCH * 2, LEVEL, N], **nt},
                            "ring_2^12_one_ciphertext": {"shape": [2, TINY[1], 1 << TINY[0]], **nt1}},
        "key_bytes": {"stored": 2 * DNUM * (L + K) * N * 4, "regen": DNUM * (L + K) * N * 4 + 32},
    }
    ctx.close()
    return out, {"cts": cts, "key_b": kb_host, "seed": seed, "gpu_out": gpu_out}


def synth_chain(t) -> list[int]:
    from rns_ckks_key_amd.api import chain_primes
    return chain_primes(t[0], t[4], t[1] + t[2])


# ---------------------------------------------------------------- other workloads

def run_workload(w: int, args, primes, torch) -> dict:
    """Workloads 3-8 in the requested variants; kernel times from the event timer."""
    import numpy as np

    from rns_ckks_key_amd import synth
    from rns_ckks_key_amd.api import Context, chain_primes, to_device

    variants = [v for v in ("regen", "stored") if args.variant in ("both", v)]
    steps, warmup, rounds = args.steps, args.warmup, max(1, args.rounds // 2)

    def both(make_fn, items, unit, ctx):
        return interleaved({v: make_fn(v) for v in variants}, steps, warmup, rounds, torch, ctx=ctx, items=items,
                           unit=unit)

    if w == 6:
        name = "multiply + relinearise (s^2 key) + rescale, N=2^16, batch 8 at level 36 -> 35"
    elif w == 7:
        name = ("double-hoisted baby-step/giant-step linear transform, N=2^16, level 36, n1 = n2 = 4 "
                "(16 diagonals, 3 baby + 3 giant rotation keys g = 5^k)")
    elif w == 8:
        name = "smaller ring: N=2^15, 20+7 x 32-bit primes, dnum 3, batch 8 ciphertexts at level 20, one rotation key g=5"
    else:
        wl = synth.WORKLOADS[w]
        d = synth.draw(w, primes)
        name = wl.name
    res = {"metric": f"workload {w}: {name}", "n_gpus": 1, "dtype": "u32", "data": "synthetic", "steps": steps,
           "warmup": warmup, "rounds": rounds}
    if w == 3:
        ctx = make_context(primes, 16, args)
        kb = to_device(synth.uniform_key_rows(3003, primes, DNUM, N))
        seed = d.keys[0].seed
        ka = ctx.expand_a(seed)
        res["levels"] = {}
        for li, level in enumerate(wl.levels):
            cts = to_device(np.stack(d.cts[16 * li:16 * li + 16]))
            out = torch.empty((16, 2, level, N), dtype=torch.int32, device="cuda")
            mk = (lambda v, lv=level, c=cts, o=out: lambda i: ctx.keyswitch(
                c, lv, kb, 5, key_seed=seed if v == "regen" else None, key_a=ka if v == "stored" else None, out=o))
            r = both(mk, 16, "key_switches_per_s", ctx)
            for v in r:
                r[v]["hbm_roofline_frac"] = round(hbm_bytes(level, 16, v == "regen") / (r[v]["ms_per_call"] * 1e-3)
                                                  / HBM_PEAK, 4)
            res["levels"][str(level)] = r
        # the same calls with the inner product and ModDown as separate launches, once, for the
        # per-step split the fused kernels hide: NTT = every row pass (the column halves are fused
        # into the conversions), ModUp = its conversion, inner product alone, ModDown = its
        # conversion and its final row NTT with the subtraction and P^-1
        ctx.set_fused(False)
        res["unfused_split"] = {}
        steps_of = {"ntt": ("row", "digit_ntt", "moddown_row"), "modup": ("modup_conv",),
                    "inner_product": ("ip_ext",), "moddown": ("moddown_conv", "moddown_final")}
        for li, level in enumerate(wl.levels):
            cts = to_device(np.stack(d.cts[16 * li:16 * li + 16]))
            out = torch.empty((16, 2, level, N), dtype=torch.int32, device="cuda")
            mk = (lambda v, lv=level, c=cts, o=out: lambda i: ctx.keyswitch(
                c, lv, kb, 5, key_seed=seed if v == "regen" else None, key_a=ka if v == "stored" else None, out=o))
            r = both(mk, 16, "key_switches_per_s", ctx)
            for v in r:
                k = r[v]["kernel_ms_per_call"]
                r[v] = {"ms_per_call": r[v]["ms_per_call"], "ms_median": r[v]["ms_median"],
                        "step_ms_per_call": {st: round(sum(k.get(c, 0.0) for c in cs), 4)
                                             for st, cs in steps_of.items()},
                        "kernel_ms_per_call": k}
            res["unfused_split"][str(level)] = r
        ctx.set_fused(True)
    elif w == 4:
        ctx = make_context(primes, 16, args)
        ct = to_device(d.cts[0])
        kbs = [to_device(synth.uniform_key_rows(4000 + k, primes, DNUM, N)) for k in range(len(d.keys))]
        kas = [ctx.expand_a(kd.seed) for kd in d.keys]
        out = torch.empty((16, 2, LEVEL, N), dtype=torch.int32, device="cuda")

        def mk(v):
            keys = [(kbs[k], kd.galois, kd.seed if v == "regen" else None, kas[k] if v == "stored" else None)
                    for k, kd in enumerate(d.keys)]
            return lambda i: ctx.keyswitch_hoisted(ct, LEVEL, keys, out=out)
        res.update(both(mk, 16, "key_switches_per_s", ctx))
        for v in variants:
            res[v]["hbm_roofline_frac"] = round(hbm_bytes(LEVEL, 1, v == "regen", 16) / (res[v]["ms_per_call"] * 1e-3)
                                                / HBM_PEAK, 4)
    elif w == 5:
        ctx = make_context(primes, 16, args)
        kbs = [to_device(synth.uniform_key_rows(5000 + k, primes, DNUM, N)) for k in range(len(d.keys))]
        kas = [ctx.expand_a(kd.seed) for kd in d.keys] if "stored" in variants else None
        cts = [to_device(c) for c in d.cts]
        outs = [torch.empty((2, lv, N), dtype=torch.int32, device="cuda") for lv in d.levels]

        def items_of(v):
            return [(cts[c], d.levels[c], kbs[d.key_index[c]], wl.galois[d.key_index[c]],
                     d.keys[d.key_index[c]].seed if v == "regen" else None,
                     kas[d.key_index[c]] if v == "stored" else None, outs[c]) for c in range(len(cts))]
        # one multi-item call: ciphertexts of equal level share launches, and the launch
        # sequences of different levels run concurrently on the library's four streams
        res.update(both(lambda v: (lambda i, it=items_of(v): ctx.keyswitch_multi(it)), len(cts),
                        "key_switches_per_s", None))

        def single(v):
            it = items_of(v)
            return lambda i: [ctx.keyswitch(x[0][None], x[1], x[2], x[3], key_seed=x[4], key_a=x[5], out=x[6][None])
                              for x in it]
        one = both(single, len(cts), "key_switches_per_s", None)
        for v in variants:
            byts = sum(hbm_bytes(lv, 1, v == "regen") for lv in d.levels)
            res[v]["hbm_roofline_frac"] = round(byts / (res[v]["ms_per_call"] * 1e-3) / HBM_PEAK, 4)
            res[v]["one_call_per_ciphertext"] = {k: one[v][k] for k in ("key_switches_per_s", "ms_per_call",
                                                                        "ms_median")}
        res["key_set_bytes"] = {"regen": len(d.keys) * (DNUM * (L + K) * N * 4 + 32),
                                "stored": 2 * len(d.keys) * DNUM * (L + K) * N * 4}
    elif w == 6:
        # batch 8 at level 36: x (x) y, relinearisation with the s^2 key, rescale to level 35
        ctx = make_context(primes, BATCH, args)
        rng = np.random.default_rng(6006)
        xs = [to_device(np.stack([np.stack([synth.residues(rng, primes[:LEVEL], N) for _ in range(2)])
                                  for _ in range(BATCH)])) for _ in range(2)]
        kb = to_device(synth.uniform_key_rows(6000, primes, DNUM, N))
        seed = rng.bytes(32)
        ka = ctx.expand_a(seed)
        out = torch.empty((BATCH, 2, LEVEL - 1, N), dtype=torch.int32, device="cuda")
        res.update(both(lambda v: (lambda i: ctx.mul_relin_rescale(
            xs[0], xs[1], LEVEL, kb, key_seed=seed if v == "regen" else None, key_a=ka if v == "stored" else None,
            out=out)), BATCH, "mul_relin_rescale_per_s", ctx))
        res["rescale"] = interleaved({"rescale": lambda i: ctx.rescale(xs[0], LEVEL, out=out)}, steps, warmup,
                                     rounds, torch, ctx=ctx, items=BATCH, unit="ciphertexts_per_s")["rescale"]
    elif w == 7:
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

        def mk(v):
            keys = [(kbs[i], gs[i], seeds[i] if v == "regen" else None, kas[i] if v == "stored" else None)
                    for i in range(len(gs))]
            return lambda i: ctx.linear_transform_bsgs(ct, LEVEL, diags, keys[:n1 - 1], keys[n1 - 1:], out=out)
        res.update(both(mk, 1, "transforms_per_s", ctx))
        for v in variants:
            res[v]["rotations_per_s"] = round(n1 * n2 / (res[v]["ms_per_call"] * 1e-3), 1)
        t_diag = res[variants[0]]["kernel_ms_per_call"]["diag"] * 1e-3
        # the diagonal sums read the diagonals and the baby steps and write the sums: n1*n2 + 2*(n1-1) + 2*n2
        # extended limbs; the giant-step sum (same timer class) reads n2 ciphertexts and writes one
        diag_bytes = ((n1 * n2 + 2 * (n1 - 1) + 2 * n2) * (LEVEL + K) + (n2 + 1) * 2 * LEVEL) * N * 4
        res["diag_roofline"] = {"bound": "hbm", "achieved_gbs": round(diag_bytes / t_diag / 1e9, 1),
                                "peak_gbs": HBM_PEAK / 1e9, "frac": round(diag_bytes / t_diag / HBM_PEAK, 4)}
    elif w == 8:
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
        res.update(both(lambda v: (lambda i: ctx.keyswitch(cts, l8, kb, GALOIS, key_seed=seed if v == "regen" else None,
                                                           key_a=ka if v == "stored" else None, out=out)),
                        BATCH, "key_switches_per_s", ctx))
    ctx.close()
    return res


def valu_rates(torch) -> dict:
    """Lane-op throughput (T/s) of each instruction kind of the microbenchmark library."""
    import ctypes

    torch.cuda.set_device(0)
    torch.zeros(1, device="cuda")  # the HIP runtime torch loaded is the one the library binds to
    lib = ctypes.CDLL(os.path.join(ROOT, "rns_ckks_key_amd", "libckks_valu_rates.so"))
    lib.ckks_valu_rate_name.restype = ctypes.c_char_p
    lib.ckks_valu_rate.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_double)]
    blocks, iters = 2048, 4096   # 8 waves on each of the 1,024 SIMDs; ~128 instructions x 4096 per thread
    out = {"grid": {"workgroups": blocks, "threads_per_workgroup": 256, "iterations": iters,
                    "instructions_per_iteration": 128, "independent_chains_per_lane": 8},
           "peak_model_T_per_s": round(VALU_PEAK / 1e12, 3), "T_lane_ops_per_s": {}}
    for op in range(lib.ckks_valu_rate_ops()):
        v = ctypes.c_double()
        rc = lib.ckks_valu_rate(op, blocks, iters, 5, ctypes.byref(v))
        name = lib.ckks_valu_rate_name(op).decode()
        out["T_lane_ops_per_s"][name] = round(v.value, 2) if rc == 0 else f"error {rc}"
        print(f"[valu] {name}: {out['T_lane_ops_per_s'][name]}", file=sys.stderr, flush=True)
    return out


# ---------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--prewarm", type=float, default=2.0,
                    help="seconds of alternating calls of both variants before any timing (clock settling)")
    ap.add_argument("--rounds", type=int, default=4, help="alternating timed blocks of each variant after the headline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip workloads 3-5 in the default line")
    ap.add_argument("--conv", choices=["vector", "matrix"], default="vector",
                    help="base conversion on the vector unit or the matrix cores")
    ap.add_argument("--workload", type=int, choices=[2, 3, 4, 5, 6, 7, 8], default=2,
                    help="2 (default, the headline): batch 8 at level 36; 3: level sweep; 4: hoisted 16 keys; "
                         "5: mixed 64-ciphertext stream; 6: multiply + relinearise + rescale, batch 8 at level 36; "
                         "7: 4 x 4 baby-step/giant-step linear transform at level 36; "
                         "8: smaller ring N=2^15 (20+7 primes, dnum 3), batch 8 at level 20")
    ap.add_argument("--variant", choices=["both", "regen", "stored"], default="both",
                    help="which key variants to time (the headline is the regenerated one when it is timed)")
    ap.add_argument("--valu-rates", action="store_true",
                    help="only measure the lane-op throughput of the vector integer instructions the kernels use")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (xor with 0) three times, to calibrate HBM counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: key-switching is not sharded across GPUs in this library "
              "(see the design notes); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        src = torch.randint(0, 2**31 - 1, (128 << 20,), dtype=torch.int32, device="cuda")  # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.bitwise_xor(src, 0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4, "launches": 3}))
        return 0

    if args.valu_rates:
        print(json.dumps(valu_rates(torch)))
        return 0

    from rns_ckks_key_amd.api import chain_primes

    torch.cuda.set_device(0)
    primes = chain_primes(LOG_N, BITS, L + K)
    if args.workload != 2:
        print(json.dumps(run_workload(args.workload, args, primes, torch)))
        return 0
    out, host_inputs = headline(args, primes, torch)
    if not args.no_extra:
        out["workloads"] = {}
        for w in (3, 4, 5):
            r = run_workload(w, args, primes, torch)
            print(f"[bench] workload {w} done", file=sys.stderr, flush=True)
            out["workloads"][str(w)] = {k: v for k, v in r.items() if k not in ("n_gpus", "dtype", "data")}
    out["parity"] = {"bit_exact": None, "reason": "--no-cpu: the oracle did not run"}
    if not args.no_cpu:
        try:
            out["cpu_baseline"], oracle_out = cpu_baseline(primes, host_inputs["cts"], host_inputs["key_b"],
                                                           host_inputs["seed"])
            out["parity"] = parity_check(host_inputs["gpu_out"], oracle_out)
        except Exception as e:  # the GPU line stands on its own; say why the baseline is missing
            out["cpu_baseline"] = {"value": None, "unit": "key-switches/s", "kind": "oracle", "error": repr(e)}
            out["parity"] = {"bit_exact": None, "reason": f"the oracle failed: {e!r}"}
    if out["parity"]["bit_exact"] is False:
        # no throughput is reported for a path that computes something else
        print(f"bench.py: the timed key-switch differs from the oracle: {out['parity']['mismatches']}",
              file=sys.stderr)
        out["value"] = None
        print(json.dumps(out))
        return 1
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
