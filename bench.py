"""Benchmark of the paged-KV attention hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  1. store 256 new K/V rows + decode (Qwen3-0.6B shapes: 16 q / 8 kv heads,
     head_dim 128, bf16, block 256, 256 sequences of 100..2048 tokens);
  2. store + varlen causal prefill (same heads, prompts of 100..1024 tokens
     packed up to 16384);
  3. store + prefix-cache prefill (64 sequences sharing a 1024-token cached
     prefix, 64..512 new tokens each).
HIP events on the launch stream time every stage of every timed step.  The
JSON line reports decode HBM GB/s as the headline value (algorithmic bytes:
K/V of every valid token once, q, out, tables) and the prefill TFLOP/s
(visible query-key pairs only) beside it, each with its roofline fraction,
and the fp64 CPU oracle timed on this host's cores for comparison.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_bytes(case) -> int:
    """Algorithmic bytes of one decode call: K and V of every valid token,
    q and out, block-table entries in use and context lengths."""
    e = 2 if case.dtype == "bf16" else 4
    L = case.context_lens.astype(int)
    kv = 2 * int(L.sum()) * case.num_kv_heads * case.head_dim * e
    qo = 2 * case.num_seqs * case.num_q_heads * case.head_dim * e
    idx = 4 * (int(sum(math.ceil(x / case.block_size) for x in L)) + case.num_seqs)
    return kv + qo + idx


def store_bytes(num_rows: int, case) -> int:
    e = 2 if case.dtype == "bf16" else 4
    return 2 * 2 * num_rows * case.num_kv_heads * case.head_dim * e + 4 * num_rows


def prefill_flops(case) -> int:
    """4 * D * Hq per visible (query, key) pair: QK^T and PV, 2 FLOP per MAC."""
    ql, kl = case.q_lens.astype(int), case.k_lens.astype(int)
    pairs = sum(int(q) * (int(k) - int(q)) + int(q) * (int(q) + 1) // 2 for q, k in zip(ql, kl))
    return 4 * case.head_dim * case.num_q_heads * pairs


def prefill_bytes(case) -> int:
    """Q and O once, K and V of every distinct key once (a shared prefix once)."""
    e = 2
    qo = 2 * case.total_q * case.num_q_heads * case.head_dim * e
    if case.shared_prefix:
        keys = int(case.prefix_k.shape[0]) + case.total_q
    else:
        keys = int(case.k_lens.sum())
    return qo + 2 * keys * case.num_kv_heads * case.head_dim * e


def _code_only(src: str) -> str:
    """C/C++ source without comments and whitespace: what the compiler sees,
    so that an edit to comments alone keeps a measurement's digest."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return re.sub(r"\s+", "", src)


def kernel_sources_digest(files=None) -> str:
    """Digest of the kernel sources a measurement depends on (all of csrc/ by
    default; comments and whitespace ignored), so that a counter summary
    taken on other code is not used."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_85_amd", "csrc")
    for f in sorted(files if files else os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current sources of the kernels it covers; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k.strip()] = v.strip()
    files = [x.strip() for x in kv.get("sources", "").split(",") if x.strip()]
    try:
        if kv.get("kernel_sources") != kernel_sources_digest(files or None):
            return None
        return int(float(kv["bytes_per_launch"]))
    except (KeyError, ValueError, OSError):
        return None


def cpu_oracle_baseline(dec, pre4, threads=None):
    """The fp64 oracle, untuned, on this host: decode over the whole decode
    workload and prefill over the varlen workload (input generation not
    timed)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    if threads is None:
        threads = max(1, min(os.cpu_count() or 1, 16))
    with threadpool_limits(limits=threads):
        used = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
        kc, vc = oracle.store_kv(dec.k_cache, dec.v_cache, dec.k_new, dec.v_new,
                                 dec.slot_mapping)
        t = time.perf_counter()
        oracle.decode(dec.q, kc, vc, dec.block_tables, dec.context_lens, dec.scale, dec.dtype)
        t_dec = time.perf_counter() - t
        del kc, vc
        kc, vc = oracle.store_kv(pre4.k_cache, pre4.v_cache, pre4.k_new, pre4.v_new,
                                 pre4.slot_mapping)
        t = time.perf_counter()
        oracle.prefill_varlen(pre4.q, kc, vc, pre4.block_tables, pre4.cu_seqlens_q,
                              pre4.cu_seqlens_k, pre4.scale, pre4.dtype)
        t_pre = time.perf_counter() - t
    return {
        "decode": {"value": decode_bytes(dec) / t_dec / 1e9, "unit": "GB/s", "cores": used,
                   "kind": "oracle", "seconds": t_dec,
                   "sample": f"whole decode workload: {dec.num_seqs} sequences, "
                             f"{int(dec.context_lens.sum())} cached tokens (fp64 numpy)"},
        "prefill": {"value": prefill_flops(pre4) / t_pre / 1e12, "unit": "TFLOP/s",
                    "cores": used, "kind": "oracle", "seconds": t_pre,
                    "sample": f"whole varlen prefill workload: {pre4.num_seqs} prompts, "
                              f"{pre4.total_q} tokens (fp64 numpy)"},
    }


COPY_PROBE_BYTES = 1 << 30
FLUSH_BYTES = 512 << 20


def copy_probe(torch, dev, pa=None, up=None, dec=None, stream=None) -> None:
    """Known-size kernels run under the same counters as the path, so that
    the counters' bytes can be scaled: a plain elementwise copy (1 GiB read,
    1 GiB written per launch), and -- for the prefill kernel's
    direct-to-LDS tile loads -- the decode workload served as varlen rows of
    one query each, where every key/value tile is read exactly once (bytes
    in the log line)."""
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"copy probe: 3 x {COPY_PROBE_BYTES} B read + written")
    del src, dst
    if dec is None:
        return
    c = decode_rows_case(dec)
    kc, vc = up(c.k_cache), up(c.v_cache)
    pa.pa_store_kv(up(c.k_new), up(c.v_new), kc, vc, up(c.slot_mapping), stream=stream)
    q = up(c.q)
    out = torch.empty_like(q)
    bt, cq, ck = up(c.block_tables), up(c.cu_seqlens_q), up(c.cu_seqlens_k)
    torch.cuda.synchronize()
    for _ in range(3):
        pa.pa_prefill_varlen(out, q, kc, vc, bt, cq, ck, c.max_seqlen_q, c.max_seqlen_k,
                             float(c.scale), stream=stream)
    torch.cuda.synchronize()
    log(f"LDS-load probe: 3 x pa_prefill_varlen over {c.num_seqs} one-row sequences, "
        f"{prefill_bytes(c)} algorithmic bytes each (every key/value tile read once)")


def decode_rows_case(dec):
    """The decode workload's sequences as varlen rows of one query each (the
    same lengths, heads and block size; fresh seeded contents)."""
    from synth import PrefillSpec, make_prefill
    L = dec.context_lens.astype(int)
    spec = PrefillSpec("decode-rows", dec.num_q_heads, dec.num_kv_heads, dec.head_dim, "bf16",
                       dec.block_size, q_len_range=(1, 1))
    return make_prefill(spec, 95, q_lens=(1,) * len(L), prefix_lens=tuple(int(x) - 1 for x in L))


def _median_us(torch, fn, stream, reps=20, warm=3):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for i in range(reps):
        ev[i].record(stream)
        fn()
    ev[reps].record(stream)
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps))
    return t[reps // 2]


def extras(torch, np, pa, dev, up, dec, stream):
    """Rows beyond the step: the decode workload served as varlen rows
    (Lq = 1), alone and mixed with prompts in one launch; and a small-batch
    decode step replayed from a captured graph against eager calls."""
    from synth import PrefillSpec, make_case, make_prefill
    from paged_kv_cache_85_amd.graphs import DecodeGraph, bucket_size
    res = {}
    log("extras: decode rows and a mixed batch through pa_prefill_varlen")
    L = dec.context_lens.astype(int)
    prompts = (512, 512, 512, 512)
    mixes = {"decode_as_varlen": ((1,) * len(L), tuple(int(x) - 1 for x in L)),
             "mixed": ((1,) * len(L) + prompts, tuple(int(x) - 1 for x in L) + (0,) * 4)}
    spec0 = PrefillSpec("mixed-qwen3", dec.num_q_heads, dec.num_kv_heads, dec.head_dim, "bf16",
                        dec.block_size, q_len_range=(1, 1))
    for name, (ql, pl) in mixes.items():
        c = make_prefill(spec0, 95, q_lens=ql, prefix_lens=pl)
        kc, vc = up(c.k_cache), up(c.v_cache)
        pa.pa_store_kv(up(c.k_new), up(c.v_new), kc, vc, up(c.slot_mapping), stream=stream)
        q = up(c.q)
        out = torch.empty_like(q)
        bt, cq, ck = up(c.block_tables), up(c.cu_seqlens_q), up(c.cu_seqlens_k)
        us = _median_us(torch, lambda: pa.pa_prefill_varlen(
            out, q, kc, vc, bt, cq, ck, c.max_seqlen_q, c.max_seqlen_k, float(c.scale),
            stream=stream), stream)
        res[name] = {"launch_us": round(us, 2), "sequences": c.num_seqs,
                     "query_rows": c.total_q, "cached_tokens": int(c.k_lens.sum())}
        del kc, vc, q, out
    # the same prompts alone (the prefill half of the mixed launch)
    c = make_prefill(spec0, 96, q_lens=prompts, prefix_lens=(0,) * 4)
    kc, vc = up(c.k_cache), up(c.v_cache)
    q = up(c.q)
    out = torch.empty_like(q)
    bt, cq, ck = up(c.block_tables), up(c.cu_seqlens_q), up(c.cu_seqlens_k)
    res["prompts_alone_us"] = round(_median_us(torch, lambda: pa.pa_prefill_varlen(
        out, q, kc, vc, bt, cq, ck, c.max_seqlen_q, c.max_seqlen_k, float(c.scale),
        stream=stream), stream), 2)
    del kc, vc, q, out
    log("extras: store prologue (QK norm + rotary + store) on the varlen prefill tokens")
    from synth import make_prologue
    pc = make_prologue(4, 31)
    q, k, v = up(pc.q), up(pc.k), up(pc.v)
    kc, vc = up(pc.k_cache), up(pc.v_cache)
    qo = torch.empty_like(q)
    qw, kw, cs = up(pc.q_weight), up(pc.k_weight), up(pc.cos_sin)
    pos, sm = up(pc.positions), up(pc.slot_mapping)
    T, hq, d = pc.q.shape
    hkv = pc.k.shape[1]
    us = _median_us(torch, lambda: pa.pa_qk_norm_rope_store(qo, q, k, v, qw, kw, cs, pos, kc, vc,
                                                             sm, pc.eps, stream=stream), stream)
    moved = 2 * T * (hq + 2 * hkv) * d * 2 + 8 * T   # read and write q, k, v rows; positions, slots
    us_store = _median_us(torch, lambda: pa.pa_store_kv(k, v, kc, vc, sm, stream=stream), stream)
    res["store_prologue"] = {"tokens": T, "launch_us": round(us, 2),
                             "gbs": round(moved / us / 1e3, 1),
                             "frac_of_hbm_peak": round(moved / us / 1e3 / HBM_PEAK_GBS, 4),
                             "plain_store_us": round(us_store, 2)}
    del q, k, v, kc, vc, qo
    log("extras: graph-replayed decode steps (Qwen2.5-0.5B decode workload)")
    c = make_case(2)
    kc, vc = up(c.k_cache), up(c.v_cache)
    q, kn, vn = up(c.q), up(c.k_new), up(c.v_new)
    sl, cl, bt = up(c.slot_mapping), up(c.context_lens), up(c.block_tables)
    out = torch.empty_like(q)
    ws = torch.zeros(pa.pa_decode_workspace_bytes(c.num_seqs, c.num_q_heads, c.head_dim,
                                                  c.max_context_len), dtype=torch.uint8,
                     device=dev)

    def eager():
        pa.pa_store_kv(kn, vn, kc, vc, sl, stream=stream)
        pa.pa_decode(out, q, kc, vc, bt, cl, c.max_context_len, float(c.scale), workspace=ws,
                     stream=stream)

    g = DecodeGraph(kc, vc, c.num_q_heads, bucket_size(c.num_seqs), bt.shape[1],
                    c.max_context_len, float(c.scale))
    g(q, kn, vn, sl, cl, bt)   # inputs now sit in the graph's static buffers
    reps = 500

    def wall(fn):
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps * 1e6

    def wall_synced(fn):
        # one step at a time, the host waiting for each (a serving loop that
        # samples every token before it can launch the next step does this)
        for _ in range(20):
            fn()
            torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
            torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps * 1e6

    res["small_decode_step"] = {
        "workload": f"store + decode, {c.num_seqs} sequences, Qwen2.5-0.5B heads, block 16",
        "eager_us_per_step": round(wall(eager), 2),
        "graph_us_per_step": round(wall(g.graph.replay), 2),
        "eager_us_per_step_synced": round(wall_synced(eager), 2),
        "graph_us_per_step_synced": round(wall_synced(g.graph.replay), 2),
        "gpu_us_eager": round(_median_us(torch, eager, stream), 2)}
    res["block_manager"] = block_manager_rates(torch, np, pa, dec)
    return res


def small_decode_trace(torch, np, pa, dev, up, steps: int) -> None:
    """The small decode step (store + decode, Qwen2.5-0.5B decode workload,
    block 16) run `steps` times eagerly, then `steps` graph replays, each
    group after a synchronisation: under a kernel trace, the dispatch order
    separates the two groups, so kernel time and the gaps between kernels
    can be compared."""
    from synth import make_case
    from paged_kv_cache_85_amd.graphs import DecodeGraph, bucket_size
    c = make_case(2)
    kc, vc = up(c.k_cache), up(c.v_cache)
    q, kn, vn = up(c.q), up(c.k_new), up(c.v_new)
    sl, cl, bt = up(c.slot_mapping), up(c.context_lens), up(c.block_tables)
    out = torch.empty_like(q)
    ws = torch.zeros(pa.pa_decode_workspace_bytes(c.num_seqs, c.num_q_heads, c.head_dim,
                                                  c.max_context_len), dtype=torch.uint8,
                     device=dev)

    def eager():
        pa.pa_store_kv(kn, vn, kc, vc, sl)
        pa.pa_decode(out, q, kc, vc, bt, cl, c.max_context_len, float(c.scale), workspace=ws)

    g = DecodeGraph(kc, vc, c.num_q_heads, bucket_size(c.num_seqs), bt.shape[1],
                    c.max_context_len, float(c.scale))
    g(q, kn, vn, sl, cl, bt)
    for name, fn in (("eager", eager), ("graph", g.graph.replay)):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        log(f"small decode step, {name}: {steps} steps, "
            f"{(time.perf_counter() - t) / steps * 1e6:.2f} us per step (wall, pipelined)")


def block_manager_rates(torch, np, pa, dec):
    """Host cost of the block manager's per-step planning, into pinned host
    buffers: a decode step of the decode workload (one batched append + the
    tables and lengths), and a prefill step of the prefix-cache workload's
    shape (64 prompts behind one shared 1024-token prefix: allocate with
    prefix lookup, plan the packed rows, free)."""
    log("extras: host block manager planning rates")
    rng = np.random.default_rng(7)
    bs = dec.block_size
    L = dec.context_lens.astype(int)
    B = len(L)
    steps = 64
    width = int((L.max() + steps) // bs + 2)
    m = pa.BlockManager(int(sum(-(-(int(x) + steps) // bs) for x in L)) + 8, bs)
    for i, n in enumerate(L):
        m.allocate(i, rng.integers(0, 151936, int(n) - 1).astype(np.int32))
    ids = np.arange(B, dtype=np.int64)
    pin = {"block_tables": torch.zeros((B, width), dtype=torch.int32, pin_memory=True),
           "context_lens": torch.zeros(B, dtype=torch.int32, pin_memory=True)}
    toks = rng.integers(0, 151936, (steps, B)).astype(np.int32)
    t_dec = []
    for s in range(steps):
        t = time.perf_counter()
        _, n_ok = m.append_batch(ids, toks[s])
        m.plan_decode(ids, width, out=pin)
        t_dec.append(time.perf_counter() - t)
        assert n_ok == B
    prefix = rng.integers(0, 151936, 1024).astype(np.int32)
    pm = pa.BlockManager(64 * 6 + 8, bs)
    prompts = [np.concatenate([prefix, rng.integers(0, 151936, int(k)).astype(np.int32)])
               for k in rng.integers(64, 513, 64)]
    pid = np.arange(64, dtype=np.int64)
    rows = sum(len(p) for p in prompts)
    ppin = {"block_tables": torch.zeros((64, 8), dtype=torch.int32, pin_memory=True),
            "cu_seqlens_q": torch.zeros(65, dtype=torch.int32, pin_memory=True),
            "cu_seqlens_k": torch.zeros(65, dtype=torch.int32, pin_memory=True),
            "slot_mapping": torch.zeros(rows, dtype=torch.int32, pin_memory=True)}
    t_pre, cached = [], 0
    for r in range(21):
        t = time.perf_counter()
        cached = sum(pm.allocate(i, p) for i, p in enumerate(prompts))
        pm.plan_prefill(pid, 8, out=ppin)
        for i in range(64):
            pm.free(i)
        if r:                                      # the first pass fills the cache
            t_pre.append(time.perf_counter() - t)
    return {"decode_step": {"sequences": B, "block_size": bs,
                            "us_per_step": round(float(np.median(t_dec)) * 1e6, 1)},
            "prefill_step": {"sequences": 64, "prompt_tokens": rows, "cached_tokens": cached,
                             "us_per_step": round(float(np.median(t_pre)) * 1e6, 1)}}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the 512 MiB read that evicts L2 and the 256 MB MALL before "
                         "each step")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the mixed-batch and graph-replay measurements")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, run the known-size kernels that calibrate "
                         "the HBM byte counters: a 1 GiB elementwise copy, and the prefill "
                         "kernel on one-row sequences (each key/value tile read once), "
                         "three times each")
    ap.add_argument("--small-decode-trace", type=int, default=0, metavar="N",
                    help="only run the small decode step N times eagerly, then N graph "
                         "replays (for a kernel trace), and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode "
              "(each GPU would run its own share of heads or sequences)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_cache_85_amd as pa
    from synth import make_case

    if not os.path.exists(pa.LIB_PATH):
        from paged_kv_cache_85_amd import build
        build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(a)
        return t.to(dev)

    if args.small_decode_trace:
        small_decode_trace(torch, np, pa, dev, up, args.small_decode_trace)
        return 0

    log("generating inputs")
    dec = make_case(3)
    pre4 = make_case(4)
    pre5 = make_case(5)

    class Staged:
        pass

    def stage(case, kind):
        s = Staged()
        s.case = case
        s.kc, s.vc = up(case.k_cache), up(case.v_cache)
        s.k_new, s.v_new, s.slots = up(case.k_new), up(case.v_new), up(case.slot_mapping)
        s.q = up(case.q)
        s.out = torch.empty_like(s.q)
        s.bt = up(case.block_tables)
        if kind == "decode":
            s.cl = up(case.context_lens)
            n = pa.pa_decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.head_dim,
                                             case.max_context_len)
            s.ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=dev)
        else:
            s.cq, s.ck = up(case.cu_seqlens_q), up(case.cu_seqlens_k)
        return s

    log("uploading")
    D = stage(dec, "decode")
    P4 = stage(pre4, "prefill")
    P5 = stage(pre5, "prefill")
    stream = torch.cuda.current_stream()

    def store(s):
        pa.pa_store_kv(s.k_new, s.v_new, s.kc, s.vc, s.slots, stream=stream)

    def decode(s):
        c = s.case
        pa.pa_decode(s.out, s.q, s.kc, s.vc, s.bt, s.cl, c.max_context_len, float(c.scale),
                     workspace=s.ws, stream=stream)

    def prefill(s):
        c = s.case
        pa.pa_prefill_varlen(s.out, s.q, s.kc, s.vc, s.bt, s.cq, s.ck, c.max_seqlen_q,
                             c.max_seqlen_k, float(c.scale), stream=stream)

    # Evict L2 and the MALL before each step by reading a 512 MiB buffer, so
    # that no stage starts with its inputs cached by the previous step.  A read
    # leaves clean lines behind (a write would leave dirty ones, whose
    # write-back the next stage would pay).  Timed as a stage of its own and
    # excluded from every rate.
    flush_buf = None if args.no_flush else torch.ones(FLUSH_BYTES // 4, dtype=torch.float32,
                                                       device=dev)

    def flush():
        if flush_buf is not None:
            flush_buf.sum()

    stages = [("flush", flush),
              ("store_decode", lambda: store(D)), ("decode", lambda: decode(D)),
              ("store_prefill", lambda: store(P4)), ("prefill", lambda: prefill(P4)),
              ("store_prefix", lambda: store(P5)), ("prefix_prefill", lambda: prefill(P5))]

    def step(events=None):
        for i, (_, fn) in enumerate(stages):
            if events is not None:
                events[i].record(stream)
            fn()
        if events is not None:
            events[-1].record(stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    all_events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
                  for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(all_events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    dur = {name: [] for name, _ in stages}
    for ev in all_events:
        for i, (name, _) in enumerate(stages):
            dur[name].append(ev[i].elapsed_time(ev[i + 1]) * 1e-3)   # seconds
    avg = {k: float(np.mean(v)) for k, v in dur.items()}
    med = {k: float(np.median(v)) for k, v in dur.items()}

    dec_bytes = decode_bytes(dec)
    dec_gbs = dec_bytes / avg["decode"] / 1e9
    f4, f5 = prefill_flops(pre4), prefill_flops(pre5)
    t4, t5 = f4 / avg["prefill"] / 1e12, f5 / avg["prefix_prefill"] / 1e12
    dec_path_bytes = dec_bytes + store_bytes(dec.num_seqs, dec)
    dec_path_s = avg["decode"] + avg["store_decode"]

    traffic = measured_traffic("decode_qwen3_0.6b")
    traffic4 = measured_traffic("prefill_varlen_qwen3_0.6b")
    traffic5 = measured_traffic("prefill_prefix_qwen3_0.6b")
    result = {
        "metric": "paged-attn decode HBM GB/s & prefill TFLOP/s (% of peak), Qwen3-0.6B shapes",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, shuffled physical block IDs)",
        "config": {
            "workload": "Qwen3-0.6B attention shapes: decode 256 seqs L~U[100,2048] + "
                        "varlen prefill <=16384 tokens + 64-seq 1024-token prefix-cache prefill",
            "num_q_heads": 16, "num_kv_heads": 8, "head_dim": 128, "block_size": 256,
            "decode_seqs": dec.num_seqs, "decode_cached_tokens": int(dec.context_lens.sum()),
            "prefill_prompts": pre4.num_seqs, "prefill_tokens": pre4.total_q,
            "prefix_seqs": pre5.num_seqs, "prefix_new_tokens": pre5.total_q,
            "parallelism": "none (one GPU)",
        },
        "roofline": {
            "kernel": "pa_decode (partition + combine kernels)",
            "bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dec_bytes,
            "avg_launch_us": round(avg["decode"] * 1e6, 2),
            "median_launch_us": round(med["decode"] * 1e6, 2),
        },
        "roofline_prefill": {
            "varlen": {"bound": "mfma", "achieved": round(t4, 2), "peak": BF16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(t4 / BF16_PEAK_TFLOPS, 4),
                       "flops_per_launch": f4, "avg_launch_us": round(avg["prefill"] * 1e6, 2),
                       "algorithmic_bytes_per_launch": prefill_bytes(pre4),
                       "traffic": traffic4,
                       "hbm_frac": round(prefill_bytes(pre4) / avg["prefill"] / 1e9
                                         / HBM_PEAK_GBS, 4),
                       "hbm_frac_measured": None if traffic4 is None else
                       round(traffic4 / avg["prefill"] / 1e9 / HBM_PEAK_GBS, 4)},
            "prefix_cache": {"bound": "mfma", "achieved": round(t5, 2),
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(t5 / BF16_PEAK_TFLOPS, 4), "flops_per_launch": f5,
                             "avg_launch_us": round(avg["prefix_prefill"] * 1e6, 2),
                             "algorithmic_bytes_per_launch": prefill_bytes(pre5),
                             "traffic": traffic5},
            "median": {"varlen_tflops": round(f4 / med["prefill"] / 1e12, 2),
                       "prefix_cache_tflops": round(f5 / med["prefix_prefill"] / 1e12, 2),
                       "decode_gbs": round(dec_bytes / med["decode"] / 1e9, 2)},
        },
        "cache_flush": None if args.no_flush else
        f"{FLUSH_BYTES >> 20} MiB read before each step (own stage, excluded from rates)",
        "stages_us": {k: round(v * 1e6, 2) for k, v in avg.items()},
        "stages_median_us": {k: round(v * 1e6, 2) for k, v in med.items()},
        "decode_path_gbs": round(dec_path_bytes / dec_path_s / 1e9, 2),
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle")
        cpu = cpu_oracle_baseline(dec, pre4)
        result["cpu_baseline"] = cpu["decode"]
        result["cpu_baseline_prefill"] = cpu["prefill"]
        log("timing the fp64 CPU oracle on one thread")
        cpu1 = cpu_oracle_baseline(dec, pre4, threads=1)
        result["cpu_baseline_1thread"] = {"decode": cpu1["decode"], "prefill": cpu1["prefill"]}
    if not args.no_extras:
        del D, P4, P5
        result["next_rows"] = extras(torch, np, pa, dev, up, dec, stream)
    if args.copy_probe:
        copy_probe(torch, dev, pa, up, dec, stream)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
