"""Decode-step benchmark of page-selected sparse decode on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--configs all|none|a,b]

One step = one decode step of the whole hot path over one batch: refresh of
each request's tail-page metadata, page scores, selection, sparse split-KV
decode and merge (two launches: refresh+score, then select+decode+merge). R
independent input batches are drawn and the timed steps cycle through them,
so each step reads data that the previous steps evicted from the 256 MB
memory-side cache (the working set of one step is about 204 MB at the
b32/64k workload). The K timed steps are replays of one HIP graph holding
G steps, whole passes over the input sets in order, at least 16 (a decode
step sits in a model's captured forward once per layer, and the graph's
launch cost is shared the same way): K // G replays, plus K % G one-step
graphs, each replay between its own HIP events. `value` is the median
per-step time over those replays, `ms_per_step` the mean over the whole
timed region. Before
timing, one step is checked against the fp64 oracle on sampled (request, KV
head) units; no timing is printed if that check fails.

Printed: one JSON line with the headline workload's step time (us per
decode step), effective HBM bandwidth on algorithmic bytes, the score
kernel's roofline (the kernel that moves the most bytes), per-kernel times,
the in-house dense decode's step time and the speedup over it, the oracle
timed on the host's cores (all of them, and one) and, under "configs", the
same figures for every workload (each with its own parity gate). With the
default bf16 metadata the headline inputs are also run with 8-bit metadata
bounds (--meta-format fp8 makes that the timed step; "metadata_fp8") and
with top-delta selection ("topdelta_selection"); "topdelta_binds" times
top-delta selection on a workload where the threshold removes pages.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/decode-step + effective HBM GB/s (fraction of peak) at batch 32, 64k ctx"
PEAK_HBM_GBPS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")


HEADLINE = "b32_64k_needles_local4"
# every workload of the configuration list, in its order (the tiny workload is
# measured at budget 8 and, as "tiny_dense", at budget 64 = every page)
CONFIGS = ("tiny", "tiny_dense", "b8_16k_needles_sink_page", HEADLINE, "b16_32k_learned_sink",
           "b64_ragged_4k_128k_shared_pool")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--configs", default="all",
                    help="workloads measured besides the headline under 'configs': all, none, "
                         "or a comma-separated list of names")
    ap.add_argument("--config-steps", type=int, default=160,
                    help="timed steps of each workload under 'configs'")
    ap.add_argument("--sets", type=int, default=None,
                    help="independent input batches cycled (default: enough that one pass "
                         "over them touches 3x the 256 MB memory-side cache, 4 to 32)")
    ap.add_argument("--dense-steps", type=int, default=20)
    ap.add_argument("--parity-units", type=int, default=6)
    ap.add_argument("--cpu-units", type=int, default=0,
                    help="(request, KV head) units of one headline step the oracle is timed "
                         "on (0: all of them)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="wall time the headline oracle timing aims for (whole passes)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (0: the host cores this process may use, "
                         "at most 16)")
    ap.add_argument("--n-splits", type=int, default=None, help="override the sparse split count")
    ap.add_argument("--dense-splits", type=int, default=None,
                    help="override the dense split count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--meta-format", default="kv", choices=("kv", "fp8"),
                    help="page metadata: in the key dtype (kv) or 8-bit E4M3 bounds (fp8)")
    ap.add_argument("--meta-layout", default=None, choices=("physical", "logical"),
                    help="page metadata per physical page or per request in logical page "
                         "order (the score then reads no page table); default: each "
                         "workload's measured choice")
    ap.add_argument("--fp8-meta-layout", default="physical", choices=("physical", "logical"),
                    help="metadata layout of the 8-bit metadata line (physical measured "
                         "faster with 8-bit codes)")
    ap.add_argument("--no-fp8-line", action="store_true",
                    help="skip the 8-bit metadata measurement of a default run")
    ap.add_argument("--no-topdelta-line", action="store_true",
                    help="skip the top-delta selection measurements of a default run")
    ap.add_argument("--delta", type=float, default=5.0,
                    help="delta of the top-delta selection lines (natural-log units)")
    ap.add_argument("--only-kernel", default=None,
                    help="profiling aid: after setup, launch only this stage --steps times "
                         "(score | step | copy: a 1 GiB device-to-device copy)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# setup


MALL_BYTES = 256 << 20  # memory-side (Infinity) cache of the chip

# A step is timed inside a graph of at least this many steps, as a decode
# step sits in the captured forward of a model once per layer: the input sets
# are cycled in order (each set's bytes are evicted from the memory-side cache
# between two of its uses) and the graph's launch cost is shared by the steps
# as a forward's layers share it.
MIN_GRAPH_STEPS = 16


def default_sets(w, meta_format, acc):
    """Input sets to cycle so that the steps between two uses of one set
    touch at least three times the memory-side cache: every timed step then
    reads its bytes from HBM (4 to 32 sets; the smallest workloads are bound
    by launches, not bytes)."""
    if w.lengths is not None:
        lens = list(w.lengths)
    elif w.context is not None:
        lens = [w.context] * w.batch
    else:
        lens = [(w.ctx_range[0] + w.ctx_range[1]) // 2] * w.batch
    elem = 2 if w.kv_dtype == "bf16" else 4
    meta_elem = 1 if meta_format == "fp8" else elem
    touched = (acc.meta_bytes(lens, w.num_kv_heads, w.head_dim, meta_elem, w.page_size) +
               acc.selected_kv_bytes_uniform(lens, w.num_kv_heads, w.head_dim, elem,
                                             w.page_size, w.budget_pages))
    return int(min(32, max(4, math.ceil(3 * MALL_BYTES / max(touched, 1)))))


def layout_of(args, w):
    """The metadata layout a workload is run with: the command line's, else
    the workload's own (measured) choice."""
    return args.meta_layout or w.meta_layout


def make_set(w, seed, torch, wl, ps, meta_format="kv", inp=None, meta_layout="physical"):
    inp = wl.make_inputs(w, device="cuda", seed=seed) if inp is None else inp
    g = ps.Geometry.of(inp["q"], inp["k_pool"], inp["page_table"], meta_format, meta_layout)
    meta = ps.build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    step = ps.DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, w.n_splits, w.dense_splits,
                         inp["scale"])
    tail = torch.tensor([int(n) - 1 for n in inp["n_pages_host"]], device="cuda",
                        dtype=torch.int32)
    return {"inp": inp, "g": g, "meta": meta, "step": step, "tail": tail,
            "meta_format": meta_format}


def run_sparse_step(s):
    """One decode step after a token append: the last pages' metadata are
    refreshed, then score, select, sparse decode and merge."""
    inp, step = s["inp"], s["step"]
    return step.sparse(inp["q"], inp["k_pool"], inp["v_pool"], s["meta"], inp["page_table"],
                       inp["seq_lens"], inp["sink"], refresh_tail=True)


def run_dense_step(s):
    inp, step = s["inp"], s["step"]
    return step.dense(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                      inp["seq_lens"], inp["sink"])


def capture_steps(fn, sets, torch):
    """One graph of whole passes over the input sets, at least
    MIN_GRAPH_STEPS steps; returns (graph, steps in it)."""
    passes = -(-MIN_GRAPH_STEPS // len(sets))

    def body(_):
        for _ in range(passes):
            for s in sets:
                fn(s)
    return capture(body, None, torch), passes * len(sets)


def capture(fn, s, torch):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn(s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn(s)
    torch.cuda.synchronize()
    return graph


# ---------------------------------------------------------------------------
# oracle views (host copies of one (request, KV head) unit)


def unit_host(inp, b, g, wl, meta_format="kv"):
    w = inp["workload"]
    grp = w.group
    n = int(inp["n_pages_host"][b])
    phys = inp["page_table"][b, :n].long()
    import numpy as np
    sink = None if inp["sink"] is None else inp["sink"][g * grp:(g + 1) * grp].cpu().numpy()
    return {
        "q": inp["q"][b:b + 1, g * grp:(g + 1) * grp].cpu().numpy(),
        "k_pool": wl.kv_bits_numpy(inp["k_pool"][phys, g:g + 1]),
        "v_pool": wl.kv_bits_numpy(inp["v_pool"][phys, g:g + 1]),
        "kv_dtype": w.kv_dtype,
        "page_table": np.arange(n, dtype=np.int32)[None, :],
        "seq_lens": inp["seq_lens"][b:b + 1].cpu().numpy(),
        "page_size": w.page_size,
        "scale": inp["scale"],
        "sink": sink,
        "meta_format": "fp8_e4m3" if meta_format == "fp8" else None,
    }


def sample_units(w, k):
    units = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    if k >= len(units):
        return units
    stride = len(units) / k
    return [units[int(i * stride)] for i in range(k)]


def selection_diagnostics(s, w, sel_h, cnt_h, units, torch):
    """Diagnostics of what the selection keeps (not gates): needle recall over
    every (request, KV head) that has needle pages, and, on sampled units, the
    share of each query head's exact softmax mass (over every valid token of
    the request, no sink) that lies on the selected tokens. Plain torch ops
    on the device in fp32."""
    inp = s["inp"]
    ps_ = w.page_size
    rec = []
    for (b, g), pages in inp["needle_pages"].items():
        if pages:
            chosen = set(int(x) for x in sel_h[b, g, :int(cnt_h[b, g])])
            rec.append(sum(p in chosen for p in pages) / len(pages))
    masses = []
    for b, g in units:
        n_tok = int(inp["seq_lens_host"][b])
        n = -(-n_tok // ps_)
        phys = inp["page_table"][b, :n].long()
        keys = inp["k_pool"][phys, g].reshape(n * ps_, w.head_dim)[:n_tok].float()
        q = inp["q"][b, g * w.group:(g + 1) * w.group].float()
        x = (q @ keys.T.contiguous()) * inp["scale"]
        prob = torch.softmax(x, dim=1)
        kept = torch.zeros(n, dtype=torch.bool, device=x.device)
        kept[torch.as_tensor(sel_h[b, g, :int(cnt_h[b, g])], device=x.device).long()] = True
        on = kept.repeat_interleave(ps_)[:n_tok]
        masses += prob[:, on].sum(dim=1).tolist()
    out = {"kind": "diagnostic, not a gate", "mass_units": len(units)}
    if rec:
        out.update(needle_recall_mean=round(float(sum(rec) / len(rec)), 4),
                   needle_recall_min=round(float(min(rec)), 4))
    if masses:
        out.update(captured_mass_mean=round(float(sum(masses) / len(masses)), 4),
                   captured_mass_min=round(float(min(masses)), 4))
    return out


def parity_gate(s, w, units, wl):
    """Selection identical to the oracle outside the ambiguity band; output
    rel-L2 within the gate. Returns a summary dict; raises on failure."""
    import numpy as np

    import oracle as ref

    gate = 2e-3 if w.kv_dtype == "bf16" else 1e-5
    step, inp = s["step"], s["inp"]
    delta = step.delta  # top-delta selection when set
    sel = step.sel.cpu().numpy()
    cnt = step.sel_count.cpu().numpy()
    out = step.out.cpu().double().numpy()
    worst, n_amb, n_diff = 0.0, 0, 0
    for b, g in units:
        hu = unit_host(inp, b, g, wl, s["meta_format"])
        r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local, delta=delta)
        k = int(cnt[b, g])
        if delta is None:
            if k != min(w.budget_pages, r["n"]):
                raise AssertionError(f"parity: sel_count {k} at unit {(b, g)}")
            amb, _ = ref.ambiguous_pages(r["scores"], r["n"], w.budget_pages, w.n_sink,
                                         w.n_local, mag=r["mag"])
        else:  # threshold band: the device compares its fp32 scores
            n = r["n"]
            forced = sorted(set(range(min(w.n_sink, n))) | set(range(max(0, n - w.n_local), n)))
            kf = ref.gather_tokens(hu["k_pool"], hu["kv_dtype"], hu["page_table"],
                                   hu["seq_lens"], 0, 0, forced if w.budget_pages < n else [],
                                   hu["page_size"])
            mt = ref.pseudo_max(hu["q"][0].astype(np.float64), kf, hu["scale"])
            amb = ref.ambiguous_pages_topdelta(r["scores"], n, w.budget_pages, w.n_sink,
                                               w.n_local, hu["scale"], mt, delta,
                                               mag=r["mag"])
        got = set(int(x) for x in sel[b, g, :k])
        want = set(int(x) for x in r["sel"])
        if got - amb != want - amb:
            raise AssertionError(f"parity: selection differs outside the band at {(b, g)}")
        n_amb += len(amb)
        if got != want:
            n_diff += 1
            r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local,
                              sel_override=sel[b, g, :k])
        for i in range(w.group):
            o = out[b, g * w.group + i]
            e = float(np.linalg.norm(o - r["out"][i]) / np.linalg.norm(r["out"][i]))
            worst = max(worst, e)
    if not worst <= gate:
        raise AssertionError(f"parity: rel-L2 {worst} above {gate}")
    return {"units_checked": len(units), "max_rel_l2": worst, "gate": gate,
            "ambiguous_pages": n_amb, "units_differing_inside_band": n_diff}


# The oracle's step on the host. Every (request, KV head) unit of the timed
# sample is laid out once in one shared-memory block (queries, the
# precomputed metadata as on the device, the unit's K and V pages); worker
# processes started fresh (spawn) attach to it and run the oracle's stages
# 2-4 (scores, selection, attention) unit by unit.

_ORACLE = {}


def _oracle_attach(spec):
    """Worker initialiser: attach to the shared block (the parent, which
    shares its resource tracker with the workers, unlinks it)."""
    from multiprocessing import shared_memory

    _ORACLE.update(shm=shared_memory.SharedMemory(name=spec["name"]), spec=spec)


def _oracle_view(i):
    import numpy as np

    spec, buf = _ORACLE["spec"], _ORACLE["shm"].buf
    u = spec["units"][i]

    def arr(key):
        off, dtype, shape = u[key]
        return np.ndarray(shape, dtype=dtype, buffer=buf, offset=off)
    return u, arr


def _oracle_unit(i):
    """Stages 2-4 of the oracle for unit i: scores from the precomputed
    metadata, selection, softmax attention of every query head of the group
    over the kept pages (with the sink when there is one)."""
    import numpy as np

    import oracle as ref

    spec = _ORACLE["spec"]
    u, arr = _oracle_view(i)
    qg, kmax, kmin = arr("q"), arr("kmax"), arr("kmin")
    k_pool, v_pool = arr("k"), arr("v")
    n = kmax.shape[0]
    table = np.arange(n, dtype=np.int32)[None, :]
    lens = np.array([u["len"]], dtype=np.int64)
    _, sc = ref.unit_scores(qg, kmax, kmin)
    sel, _, _ = ref.select_pages(sc, n, spec["budget"], spec["n_sink"], spec["n_local"])
    keys = ref.gather_tokens(k_pool, spec["kv_dtype"], table, lens, 0, 0, sel, spec["page"])
    vals = ref.gather_tokens(v_pool, spec["kv_dtype"], table, lens, 0, 0, sel, spec["page"])
    sink = None if u["sink"] is None else u["sink"]
    for h in range(qg.shape[0]):
        ref.attend(qg[h], keys, vals, spec["scale"], None if sink is None else sink[h])
    return 0


def _oracle_pack(s, w, units, wl):
    """Lay out the units' oracle inputs in one new shared-memory block.
    Returns (SharedMemory, spec)."""
    import numpy as np
    from multiprocessing import shared_memory

    import oracle as ref

    inp = s["inp"]
    records, arrays, off = [], [], 0
    for b, g in units:
        hu = unit_host(inp, b, g, wl)
        kmax, kmin = ref.unit_page_meta(hu["k_pool"], hu["kv_dtype"], hu["page_table"],
                                        hu["seq_lens"], 0, 0, hu["page_size"])
        rec = {"len": int(hu["seq_lens"][0]),
               "sink": None if hu["sink"] is None else [float(x) for x in hu["sink"]]}
        for key, a in (("q", hu["q"][0].astype(np.float64)), ("kmax", kmax), ("kmin", kmin),
                       ("k", hu["k_pool"]), ("v", hu["v_pool"])):
            a = np.ascontiguousarray(a)
            rec[key] = (off, a.dtype.str, a.shape)
            arrays.append((off, a))
            off += (a.nbytes + 255) // 256 * 256
        records.append(rec)
    shm = shared_memory.SharedMemory(create=True, size=max(off, 1))
    for o, a in arrays:
        np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf, offset=o)[...] = a
    spec = {"name": shm.name, "units": records, "budget": w.budget_pages, "n_sink": w.n_sink,
            "n_local": w.n_local, "kv_dtype": w.kv_dtype, "page": w.page_size,
            "scale": inp["scale"]}
    return shm, spec


def oracle_workers(requested):
    """Worker processes for the oracle: the cores this process may run on,
    at most 16 (the host share of one GPU), or the number requested."""
    avail = len(os.sched_getaffinity(0))
    return max(1, min(requested, avail) if requested > 0 else min(avail, 16))


def cpu_baseline(s, w, units, wl, seconds, workers, single_core=True):
    """The fp64 oracle's decode step (scores, selection, attention; metadata
    given, as on the device) timed on the host: whole passes over the given
    units, on `workers` processes (one BLAS thread each), repeated until about
    `seconds` of wall time, scaled to the whole step when the units are a
    sample; with single_core, the same passes in this process, one thread."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    shm, spec = _oracle_pack(s, w, units, wl)
    total_units = w.batch * w.num_kv_heads
    scale = total_units / len(units)
    out = {"unit": "us/decode-step", "kind": "oracle"}
    try:
        ctx = mp.get_context("spawn")
        env_threads = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                      "MKL_NUM_THREADS")}
        for k in env_threads:  # one BLAS thread per worker (inherited by the spawned children)
            os.environ[k] = "1"
        try:
            with ctx.Pool(workers, initializer=_oracle_attach, initargs=(spec,)) as pool:
                pool.map(_oracle_unit, range(len(units)), chunksize=1)  # warm-up pass
                passes, total = 0, 0.0
                while passes == 0 or total < seconds:
                    t0 = time.perf_counter()
                    pool.map(_oracle_unit, range(len(units)), chunksize=1)
                    total += time.perf_counter() - t0
                    passes += 1
        finally:
            for k, v in env_threads.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        out["value"] = total / passes * scale * 1e6
        out["cores"] = workers
        what = (f"all {total_units} (request, KV head) units of one step" if scale == 1
                else f"{len(units)} of {total_units} (request, KV head) units of one step, "
                     f"scaled x{total_units}/{len(units)}")
        out["sample"] = (f"{what}; {passes} passes ({total:.1f} s wall) on {workers} worker "
                         f"processes, numpy fp64, one BLAS thread each; metadata precomputed "
                         f"as on the device")
        if single_core:
            _ORACLE.update(shm=shm, spec=spec)
            with threadpool_limits(limits=1):
                passes1, total1 = 0, 0.0
                while passes1 == 0 or total1 < seconds / 2:
                    t0 = time.perf_counter()
                    for i in range(len(units)):
                        _oracle_unit(i)
                    total1 += time.perf_counter() - t0
                    passes1 += 1
            _ORACLE.clear()
            out["single_core_value"] = total1 / passes1 * scale * 1e6
            out["single_core_sample"] = f"the same units, {passes1} passes ({total1:.1f} s) in one thread"
    finally:
        shm.close()
        shm.unlink()
    return out


# ---------------------------------------------------------------------------
# measured HBM traffic (committed rocprofv3 counter summary)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("ps_score.hip", "ps_device.h", "ps_meta.h"):
        with open(os.path.join(ROOT, "sparse_long_context_page_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """Bytes per score-kernel dispatch from the committed counter summary,
    or None when the summary is absent or was taken on other kernel source."""
    path = os.path.join(PROFILE_DIR, f"score_pages_{workload}.pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------


def timed_steps(multi, singles, r, steps, torch):
    """Time exactly `steps` decode steps: steps // r replays of the graph of
    r steps, then steps % r one-step graphs, each replay between its own HIP
    events on torch's current stream (the stream the graphs are launched on).
    Returns (ms from the first event to the last, sorted per-step us of the
    r-step replays, or of the one-step replays when there are none)."""
    n_multi = steps // r
    ev = []
    for i in range(n_multi + steps % r):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        (multi if i < n_multi else singles[(i - n_multi) % len(singles)]).replay()
        b.record()
        ev.append((a, b, r if i < n_multi else 1))
    torch.cuda.synchronize()
    total = ev[0][0].elapsed_time(ev[-1][1])
    sel = [e for e in ev if e[2] == r] if n_multi else ev
    return total, sorted(a.elapsed_time(b) * 1e3 / k for a, b, k in sel)


def pct(sorted_vals, p):
    return sorted_vals[min(len(sorted_vals) - 1, int(round(p * (len(sorted_vals) - 1))))]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the decode step has "
                                   "no cross-GPU work: every (request, KV head) is "
                                   "independent, so requests or KV heads shard over GPUs "
                                   "without communication",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as wl
    import sparse_long_context_page_amd as ps
    from sparse_long_context_page_amd import _lib
    from sparse_long_context_page_amd import accounting as acc

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    _lib.load()  # no fallback: fails loudly if the HIP library is missing
    w = wl.WORKLOADS[args.workload]
    if args.n_splits:
        w = w.replace(n_splits=args.n_splits)
    if args.dense_splits:
        w = w.replace(dense_splits=args.dense_splits)
    if args.sets is None:
        args.sets = default_sets(w, args.meta_format, acc)
    print(f"# setup {w.name}: {args.sets} input sets", file=sys.stderr, flush=True)
    sets = [make_set(w, w.seed + 17 * i, torch, wl, ps, args.meta_format,
                     meta_layout=layout_of(args, w))
            for i in range(args.sets)]
    torch.cuda.synchronize()

    # -- parity gate on set 0 (eager) --------------------------------------
    s0 = sets[0]
    path = s0["step"].path_for(s0["inp"]["seq_lens_host"])
    if path != "sparse":
        raise SystemExit(f"workload {w.name} takes the {path} path; nothing sparse to time")
    out_eager, _ = run_sparse_step(s0)
    out_eager = out_eager.clone()
    torch.cuda.synchronize()
    print("# parity gate", file=sys.stderr, flush=True)
    parity = parity_gate(s0, w, sample_units(w, args.parity_units), wl)

    if args.only_kernel:
        profile_only(args, sets, torch, ps)
        return

    # -- graph-captured step loop (the timed region) -----------------------
    # One graph holds G decode steps, whole passes over the input sets in
    # order (at least MIN_GRAPH_STEPS), as steps sit inside a captured model
    # forward; K steps are K // G replays of it plus K % G one-step graphs.
    # Every step is the whole hot path.
    graphs = [capture(run_sparse_step, s, torch) for s in sets]
    graphs[0].replay()
    torch.cuda.synchronize()
    if not torch.equal(s0["step"].out, out_eager):
        raise SystemExit("graph replay differs from the eager step")

    multi, r_graph = capture_steps(run_sparse_step, sets, torch)
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    multi.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gpu_ms, per_step = timed_steps(multi, graphs, r_graph, args.steps, torch)
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = gpu_ms / args.steps
    step_us = pct(per_step, 0.5)  # the median replay
    print(f"# timed {args.steps} steps: median {step_us:.2f} us/step, mean "
          f"{ms_per_step * 1e3:.2f}", file=sys.stderr, flush=True)

    # -- warm steps: as many steps per graph as the timed graph on ONE input
    # set, whose working set then stays in the memory-side cache ("warm",
    # reported as such)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def same_set(_):  # as many steps per graph as the timed graph, one input set
        for _ in sets:
            run_sparse_step(s0)
    warm_graph = capture(same_set, None, torch)
    for _ in range(3):
        warm_graph.replay()
    e0.record()
    for _ in range(max(args.steps // len(sets), 1)):
        warm_graph.replay()
    e1.record()
    torch.cuda.synchronize()
    warm_us = e0.elapsed_time(e1) / (max(args.steps // len(sets), 1) * len(sets)) * 1e3
    del warm_graph

    # -- the same steps, one graph per step ---------------------------------
    e0.record()
    for i in range(args.steps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    one_graph_us = e0.elapsed_time(e1) / args.steps * 1e3

    # -- the same steps launched eagerly (no graph), back to back -------------
    for i in range(args.warmup):
        run_sparse_step(sets[i % len(sets)])
    torch.cuda.synchronize()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record()
    for i in range(args.steps):
        run_sparse_step(sets[i % len(sets)])
    g1.record()
    torch.cuda.synchronize()
    eager_us = g0.elapsed_time(g1) / args.steps * 1e3

    # -- per-kernel times: each launch of the step repeated back to back over
    # the input sets, captured as one graph of n_k launches (so host launch
    # cost cannot starve the small kernels) and replayed between two HIP
    # events on torch's current stream ---------------------------------------
    n_k, n_rep = 40, max(args.steps // 40, 3)

    def time_launches(fn):
        def batch(_):
            for i in range(n_k):
                fn(sets[i % len(sets)])
        gk = capture(batch, None, torch)
        gk.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n_rep):
            gk.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (n_rep * n_k) * 1e3

    def k_refresh_score(s):
        inp, step = s["inp"], s["step"]
        ps.ps_refresh_score_pages(s["g"], inp["q"], inp["k_pool"], s["meta"], inp["page_table"],
                                  inp["seq_lens"], step.scores)

    def k_select_decode(s, merge=True):
        inp, step = s["inp"], s["step"]
        acc_t, ml_t = step.partials(step.n_splits)
        if step.n_splits == 1:  # the merge is in the same launch
            ps.ps_select_sparse_decode(s["g"], inp["q"], inp["k_pool"], inp["v_pool"],
                                       inp["page_table"], inp["seq_lens"], step.scores,
                                       step.budget, step.n_sink, step.n_local, step.scale, 1,
                                       step.sel, step.sel_count, None, None, inp["sink"],
                                       step.out, step.lse)
        elif merge and step.merge_in_launch:  # the last split of each unit merges
            ps.ps_select_sparse_decode(s["g"], inp["q"], inp["k_pool"], inp["v_pool"],
                                       inp["page_table"], inp["seq_lens"], step.scores,
                                       step.budget, step.n_sink, step.n_local, step.scale,
                                       step.n_splits, step.sel, step.sel_count, acc_t, ml_t,
                                       inp["sink"], step.out, step.lse,
                                       arrivals=step.arrivals)
        else:
            ps.ps_select_sparse_decode(s["g"], inp["q"], inp["k_pool"], inp["v_pool"],
                                       inp["page_table"], inp["seq_lens"], step.scores,
                                       step.budget, step.n_sink, step.n_local, step.scale,
                                       step.n_splits, step.sel, step.sel_count, acc_t, ml_t)

    def k_combine(s):
        inp, step = s["inp"], s["step"]
        acc_t, ml_t = step.partials(step.n_splits)
        ps.ps_combine(s["g"], acc_t, ml_t, step.n_splits, inp["sink"], step.out, step.lse)

    def k_tail_meta(s):
        inp, step = s["inp"], s["step"]
        step.refresh_tail_meta(inp["k_pool"], inp["page_table"], inp["seq_lens"], s["tail"],
                               s["meta"])

    def k_score(s):
        inp, step = s["inp"], s["step"]
        ps.ps_score_pages(s["g"], inp["q"], s["meta"], inp["page_table"], inp["seq_lens"],
                          step.scores)

    def k_select(s):
        inp, step = s["inp"], s["step"]
        ps.ps_select_topk(s["g"], step.scores, inp["seq_lens"], step.budget, step.n_sink,
                          step.n_local, step.sel, step.sel_count)

    def k_sparse_decode(s):
        inp, step = s["inp"], s["step"]
        acc_t, ml_t = step.partials(step.n_splits)
        ps.ps_sparse_decode(s["g"], inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                            inp["seq_lens"], step.sel, step.sel_count, step.budget, step.scale,
                            step.n_splits, acc_t, ml_t)

    fused = s0["step"].fused
    kern_us = {}
    kern_us["refresh_score"] = time_launches(k_refresh_score)  # the step's own launches
    if fused:
        kern_us["select_decode"] = time_launches(k_select_decode)
        if s0["step"].merge_in_launch and s0["step"].n_splits > 1:
            kern_us["select_decode_partials_only"] = time_launches(
                lambda s: k_select_decode(s, merge=False))
    kern_us["combine"] = time_launches(k_combine)
    # the unfused entry points, one stage each
    kern_us["tail_meta"] = time_launches(k_tail_meta)
    kern_us["score"] = time_launches(k_score)
    kern_us["select"] = time_launches(k_select)
    kern_us["sparse_decode"] = time_launches(k_sparse_decode)
    for s in sets:  # leave every set as one whole step leaves it
        run_sparse_step(s)
    torch.cuda.synchronize()

    # -- dense baseline ----------------------------------------------------
    dgraphs = [capture(run_dense_step, s, torch) for s in sets]
    for i in range(3):
        dgraphs[i % len(dgraphs)].replay()
    torch.cuda.synchronize()
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record()
    for i in range(args.dense_steps):
        dgraphs[i % len(dgraphs)].replay()
    d1.record()
    torch.cuda.synchronize()
    dense_us = d0.elapsed_time(d1) / args.dense_steps * 1e3

    # -- achievable bandwidth: a plain 2 GiB device-to-device copy --------------
    src = torch.empty(1 << 29, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 4 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    # achievable read stream: row sums of the same 2 GiB (reads only; torch's
    # reduction, about 6 TB/s on this chip)
    rows = src.view(4096, -1)
    for _ in range(2):
        rows.sum(dim=1)
    c0.record()
    for _ in range(5):
        rows.sum(dim=1)
    c1.record()
    torch.cuda.synchronize()
    read_gbps = src.numel() * 4 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst, rows

    # -- bytes ---------------------------------------------------------------
    inp0 = s0["inp"]
    lens = [int(x) for x in inp0["seq_lens_host"]]
    elem = 2 if w.kv_dtype == "bf16" else 4
    meta_elem = 1 if args.meta_format == "fp8" else elem
    meta_b = acc.meta_bytes(lens, w.num_kv_heads, w.head_dim, meta_elem, w.page_size)
    run_sparse_step(s0)
    torch.cuda.synchronize()
    sel_h = s0["step"].sel.cpu().numpy()
    lists = {(b, g): list(sel_h[b, g]) for b in range(w.batch) for g in range(w.num_kv_heads)}
    kv_b = acc.selected_kv_bytes(lens, lists, w.head_dim, elem, w.page_size)
    touched = meta_b + kv_b
    dense_b = acc.dense_kv_bytes(lens, w.num_kv_heads, w.head_dim, elem)
    eff_gbps = touched / (step_us * 1e-6) / 1e9
    # the dominant kernel: the step's score launch with the last-page
    # refresh: metadata of every page read, one fp32 score per page written,
    # and per (request, KV head) the last page's 16 key rows read and its
    # metadata written
    units = w.batch * w.num_kv_heads
    scores_b = sum(-(-n // w.page_size) for n in lens) * w.num_kv_heads * 4
    tail_b = units * (w.page_size * elem + 2 * meta_elem) * w.head_dim
    dom_key = "refresh_score"
    dom_b = meta_b + scores_b + tail_b
    score_gbps = dom_b / (kern_us[dom_key] * 1e-6) / 1e9
    dec_key = "select_decode" if fused else "sparse_decode"
    decode_gbps = kv_b / (kern_us[dec_key] * 1e-6) / 1e9

    traffic = measured_traffic(w.name + ("_fp8meta" if args.meta_format == "fp8" else "") +
                               ("_logicalmeta" if layout_of(args, w) == "logical" else ""))
    result = {
        "metric": METRIC,
        "value": round(step_us, 3),
        "unit": "us/decode-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "context": w.context if w.context else list(w.ctx_range),
                   "page_size": w.page_size, "budget_pages": w.budget_pages,
                   "n_sink_pages": w.n_sink, "n_local_pages": w.n_local, "needles": w.needles,
                   "kv_storage": w.kv_dtype, "metadata": args.meta_format,
                   "metadata_layout": layout_of(args, w),
                   "n_splits": w.n_splits, "input_sets": len(sets),
                   "path": path,
                   "graph_captured": f"{r_graph} steps ({r_graph // len(sets)} passes over "
                                     f"the {len(sets)} input sets) per graph"},
        "effective_hbm_gbps": round(eff_gbps, 1),
        "hbm_frac_of_peak": round(eff_gbps / PEAK_HBM_GBPS, 4),
        "touched_bytes": touched,
        "touched_bytes_split": {"metadata": meta_b, "selected_kv": kv_b},
        "kernels_us": {k: round(v, 3) for k, v in kern_us.items()},
        "step_launches": step_launches(s0["step"]),
        "selection_overhead_us": round(kern_us["select"], 3),
        "selection_in_decode_us": (round(kern_us.get("select_decode_partials_only",
                                                     kern_us["select_decode"])
                                         - kern_us["sparse_decode"], 3) if fused else None),
        "score_plus_select_us": round(kern_us["score"] + kern_us["select"], 3),
        "sparse_decode_gbps": round(decode_gbps, 1),
        "dense_us_per_step": round(dense_us, 3),
        "dense_bytes": dense_b,
        "dense_hbm_gbps": round(dense_b / (dense_us * 1e-6) / 1e9, 1),
        "speedup_vs_dense": round(dense_us / step_us, 3),
        "copy_gbps_read_plus_write": round(copy_gbps, 1),
        "read_stream_gbps": round(read_gbps, 1),
        "timed_wall_ms": round(wall_ms, 3),
        "mean_us_per_step": round(ms_per_step * 1e3, 3),
        "eager_us_per_step": round(eager_us, 3),
        "us_per_step_p10_p50_p90": [round(pct(per_step, 0.1), 3), round(pct(per_step, 0.5), 3),
                                    round(pct(per_step, 0.9), 3)],
        "timed_replays": len(per_step),
        "warm_same_set_us_per_step": round(warm_us, 3),
        "one_step_per_graph_us_per_step": round(one_graph_us, 3),
        "parity": parity,
        "selection": selection_diagnostics(
            s0, w, sel_h, s0["step"].sel_count.cpu().numpy(),
            sample_units(w, args.parity_units), torch),
        "roofline": {"kernel": "ps_refresh_score_pages",
                     "bound": "hbm",
                     "achieved": round(score_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(score_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom_b,
                     "avg_launch_us": round(kern_us[dom_key], 3),
                     "achievable_read_gbps": round(read_gbps, 1),
                     "frac_of_achievable_read": round(score_gbps / read_gbps, 4)},
    }
    if args.meta_format == "kv" and not args.no_fp8_line:
        print("# 8-bit metadata", file=sys.stderr, flush=True)
        result["metadata_fp8"] = fp8_line(args, w, sets, step_us, torch, wl, ps, acc)
    if args.meta_format == "kv" and not args.no_topdelta_line:
        print("# top-delta selection", file=sys.stderr, flush=True)
        result["topdelta_selection"] = topdelta_line(args, w, sets, step_us, torch, wl, ps)
    workers = oracle_workers(args.cpu_workers)
    if not args.no_cpu_baseline:
        print("# cpu baseline", file=sys.stderr, flush=True)
        n_units = w.batch * w.num_kv_heads
        result["cpu_baseline"] = cpu_baseline(
            s0, w, sample_units(w, args.cpu_units if args.cpu_units > 0 else n_units), wl,
            args.cpu_seconds, workers)
    headline_entry = {
        "us_per_step_median": result["value"],
        "us_per_step_p10_p50_p90": result["us_per_step_p10_p50_p90"],
        "effective_hbm_gbps": result["effective_hbm_gbps"],
        "hbm_frac_of_peak": result["hbm_frac_of_peak"], "touched_bytes": touched,
        "dense_us_per_step": result["dense_us_per_step"],
        "speedup_vs_dense": result["speedup_vs_dense"], "parity": parity,
        "n_splits": w.n_splits, "input_sets": len(sets), "path": path,
        "selection_in_decode_us": result["selection_in_decode_us"],
        "oracle_us_per_step": (result["cpu_baseline"]["value"]
                               if "cpu_baseline" in result else None),
        "oracle_cores": workers if "cpu_baseline" in result else None}
    # free the headline's input sets before the other workloads
    del sets, graphs, multi, dgraphs
    if "s0" in locals():
        del s0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    names = [n for n in CONFIGS if n != w.name] if args.configs == "all" else (
        [] if args.configs == "none" else [n for n in args.configs.split(",") if n])
    configs = {w.name: headline_entry}
    for name in names:
        print(f"# config {name}", file=sys.stderr, flush=True)
        configs[name] = config_line(args, wl.WORKLOADS[name], workers, torch, wl, ps, acc)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    result["configs"] = {n: configs[n] for n in CONFIGS if n in configs}
    for n in configs:
        if n not in result["configs"]:
            result["configs"][n] = configs[n]
    if args.meta_format == "kv" and not args.no_topdelta_line:
        print("# top-delta where the threshold binds", file=sys.stderr, flush=True)
        result["topdelta_binds"] = topdelta_binds_line(args, torch, wl, ps, acc)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    print(json.dumps(result), flush=True)


def dense_parity(s, w, units, wl):
    """The dense path (budget covering every page) against exact softmax
    attention of the oracle; returns a summary dict, raises on failure."""
    import numpy as np

    import oracle as ref

    gate = 2e-3 if w.kv_dtype == "bf16" else 1e-5
    out = s["step"].out.cpu().double().numpy()
    worst = 0.0
    for b, g in units:
        hu = unit_host(s["inp"], b, g, wl)
        for i in range(w.group):
            o, _ = ref.full_decode(hu, 0, i)
            e = float(np.linalg.norm(out[b, g * w.group + i] - o) / np.linalg.norm(o))
            worst = max(worst, e)
    if not worst <= gate:
        raise AssertionError(f"parity: dense rel-L2 {worst} above {gate}")
    return {"units_checked": len(units), "max_rel_l2": worst, "gate": gate,
            "oracle": "exact softmax attention over every valid token"}


def config_line(args, w, workers, torch, wl, ps, acc):
    """One workload under "configs": its parity gate (every unit of the small
    workloads, sampled units of the others), then its step timed as the
    headline's (one graph of one step per input set, each replay between its
    own events, median), the touched bytes and their rate, the dense decode
    and the speedup over it, and the oracle on the host's cores (sampled
    units, scaled to the step)."""
    import numpy as np

    r = default_sets(w, "kv", acc)
    sets = [make_set(w, w.seed + 17 * i, torch, wl, ps, meta_layout=layout_of(args, w))
            for i in range(r)]
    torch.cuda.synchronize()
    s0 = sets[0]
    path = s0["step"].path_for(s0["inp"]["seq_lens_host"])
    run = run_sparse_step if path == "sparse" else run_dense_step
    n_units = w.batch * w.num_kv_heads
    units = sample_units(w, n_units if n_units <= 16 else args.parity_units)
    run(s0)
    torch.cuda.synchronize()
    parity = (parity_gate(s0, w, units, wl) if path == "sparse"
              else dense_parity(s0, w, units, wl))
    graphs = [capture(run, s, torch) for s in sets]

    multi, r_graph = capture_steps(run, sets, torch)
    for i in range(args.warmup):
        graphs[i % r].replay()
    multi.replay()
    torch.cuda.synchronize()
    total_ms, per = timed_steps(multi, graphs, r_graph, args.config_steps, torch)
    step_us = pct(per, 0.5)

    lens = [int(x) for x in s0["inp"]["seq_lens_host"]]
    elem = 2 if w.kv_dtype == "bf16" else 4
    if path == "sparse":
        meta_b = acc.meta_bytes(lens, w.num_kv_heads, w.head_dim, elem, w.page_size)
        sel_h = s0["step"].sel.cpu().numpy()
        lists = {(b, g): list(sel_h[b, g]) for b in range(w.batch)
                 for g in range(w.num_kv_heads)}
        kv_b = acc.selected_kv_bytes(lens, lists, w.head_dim, elem, w.page_size)
    else:
        meta_b, kv_b = 0, acc.dense_kv_bytes(lens, w.num_kv_heads, w.head_dim, elem)
    touched = meta_b + kv_b
    gbps = touched / (step_us * 1e-6) / 1e9
    out = {"us_per_step_median": round(step_us, 3),
           "us_per_step_p10_p50_p90": [round(pct(per, 0.1), 3), round(pct(per, 0.5), 3),
                                       round(pct(per, 0.9), 3)],
           "mean_us_per_step": round(total_ms * 1e3 / args.config_steps, 3),
           "timed_steps": args.config_steps, "timed_replays": len(per),
           "touched_bytes": touched,
           "touched_bytes_split": {"metadata": meta_b, "kv": kv_b},
           "effective_hbm_gbps": round(gbps, 1),
           "hbm_frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
           "path": path, "n_splits": w.n_splits if path == "sparse" else w.dense_splits,
           "input_sets": r, "steps_per_graph": r_graph, "parity": parity,
           "config": {"batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                      "head_dim": w.head_dim,
                      "context": w.context if w.context else list(w.ctx_range),
                      "budget_pages": w.budget_pages, "n_sink_pages": w.n_sink,
                      "n_local_pages": w.n_local, "needles": w.needles,
                      "kv_storage": w.kv_dtype, "learned_sink": w.sink_logits,
                      "permuted_pool": w.permuted_pool,
                      "metadata_layout": layout_of(args, w)}}
    if w.kv_dtype == "bf16" or path == "sparse":
        out["launches"] = (step_launches(s0["step"]) if path == "sparse"
                           else ["ps_full_decode", "ps_combine"])
    if path == "sparse":  # the in-house dense decode on the same inputs
        dgraphs = [capture(run_dense_step, s, torch) for s in sets]
        for i in range(3):
            dgraphs[i % r].replay()
        torch.cuda.synchronize()
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        d0.record()
        for i in range(args.dense_steps):
            dgraphs[i % r].replay()
        d1.record()
        torch.cuda.synchronize()
        dense_us = d0.elapsed_time(d1) / args.dense_steps * 1e3
        out["dense_us_per_step"] = round(dense_us, 3)
        out["speedup_vs_dense"] = round(dense_us / step_us, 3)
        del dgraphs
    if not args.no_cpu_baseline:
        cb = cpu_baseline(s0, w, sample_units(w, min(n_units, 16)), wl, 3.0, workers,
                          single_core=False)
        out["oracle_us_per_step"] = round(cb["value"], 1)
        out["oracle_cores"] = cb["cores"]
        out["oracle_sample"] = cb["sample"]
    del sets, graphs, multi, s0
    return out


def topdelta_binds_line(args, torch, wl, ps, acc):
    """Top-delta selection on a workload where the threshold removes pages
    (one query head per KV head; a forced sink page whose keys follow the
    needle recipe, so the pseudo-max over the forced tokens is high): parity
    against the oracle's top-delta rule, the step timed as the headline's,
    the pages kept per unit against the budget, the bytes actually read, and
    the top-k step on the same inputs."""
    import numpy as np

    w = wl.TOPDELTA_BINDS
    r = default_sets(w, "kv", acc)
    base = [make_set(w, w.seed + 17 * i, torch, wl, ps, meta_layout=layout_of(args, w))
            for i in range(r)]
    sets = [dict(s, step=ps.DecodeStep(s["g"], w.budget_pages, w.n_sink, w.n_local, w.n_splits,
                                       w.dense_splits, s["inp"]["scale"], delta=args.delta))
            for s in base]
    run_sparse_step(sets[0])
    torch.cuda.synchronize()
    parity = parity_gate(sets[0], w, sample_units(w, args.parity_units), wl)
    kept = sets[0]["step"].sel_count.cpu().numpy()
    res = {}
    for kind, ss in (("topdelta", sets), ("topk", base)):
        graphs = [capture(run_sparse_step, s, torch) for s in ss]

        multi, r_graph = capture_steps(run_sparse_step, ss, torch)
        for i in range(args.warmup):
            graphs[i % r].replay()
        torch.cuda.synchronize()
        _, per = timed_steps(multi, graphs, r_graph, args.config_steps, torch)
        res[kind] = pct(per, 0.5)
        del graphs, multi
    for s in sets:  # leave every set as one whole top-delta step leaves it
        run_sparse_step(s)
    torch.cuda.synchronize()
    lens = [int(x) for x in sets[0]["inp"]["seq_lens_host"]]
    meta_b = acc.meta_bytes(lens, w.num_kv_heads, w.head_dim, 2, w.page_size)
    sel_h = sets[0]["step"].sel.cpu().numpy()
    lists = {(b, g): list(sel_h[b, g][:int(kept[b, g])]) for b in range(w.batch)
             for g in range(w.num_kv_heads)}
    kv_b = acc.selected_kv_bytes(lens, lists, w.head_dim, 2, w.page_size)
    out = {"workload": w.name, "delta": args.delta,
           "us_per_step_median": round(res["topdelta"], 3),
           "topk_us_per_step_median": round(res["topk"], 3),
           "kept_pages_per_unit": {"mean": round(float(np.mean(kept)), 2), "min": int(kept.min()),
                                   "max": int(kept.max()), "budget": w.budget_pages},
           "touched_bytes": meta_b + kv_b,
           "touched_bytes_split": {"metadata": meta_b, "selected_kv": kv_b},
           "effective_hbm_gbps": round((meta_b + kv_b) / (res["topdelta"] * 1e-6) / 1e9, 1),
           "launches": step_launches(sets[0]["step"]),
           "parity": dict(parity, oracle="top-delta rule")}
    del sets, base
    return out


def step_launches(step):
    """The launches of one sparse step (with the tail refresh) in order."""
    sel = "ps_select_topk" if step.delta is None else "ps_select_topdelta"
    if step.fused:
        fused = ("ps_select_sparse_decode" if step.delta is None
                 else "ps_select_topdelta_sparse_decode")
        merged = step.n_splits == 1 or step.merge_in_launch
        return ["ps_refresh_score_pages", fused] + ([] if merged else ["ps_combine"])
    return ["ps_refresh_score_pages", sel, "ps_sparse_decode", "ps_combine"]


def topdelta_line(args, w, sets, step_us_topk, torch, wl, ps):
    """The same inputs with top-delta selection (delta = args.delta): parity
    against the oracle's top-delta rule, the step timed as the main one
    (refresh+score, then the top-delta selection fused into the sparse
    decode, then the merge when there are several splits), the standalone
    selection launch on its own, and the pages kept per unit."""
    import numpy as np

    sets_d = []
    for s in sets:
        inp = s["inp"]
        step = ps.DecodeStep(s["g"], w.budget_pages, w.n_sink, w.n_local, w.n_splits,
                             w.dense_splits, inp["scale"], delta=args.delta)
        sets_d.append(dict(s, step=step))
    run_sparse_step(sets_d[0])
    torch.cuda.synchronize()
    parity = parity_gate(sets_d[0], w, sample_units(w, args.parity_units), wl)
    kept = sets_d[0]["step"].sel_count.cpu().numpy()

    multi, r_graph = capture_steps(run_sparse_step, sets_d, torch)
    for _ in range(3):
        multi.replay()
    torch.cuda.synchronize()
    reps = max(args.steps // r_graph, 1)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        multi.replay()
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) / (reps * r_graph) * 1e3

    n_k = 40

    def batch(_):
        for i in range(n_k):
            s = sets_d[i % len(sets_d)]
            inp, st = s["inp"], s["step"]
            ps.ps_select_topdelta(s["g"], inp["q"], inp["k_pool"], inp["page_table"],
                                  inp["seq_lens"], st.scores, st.budget, st.n_sink, st.n_local,
                                  st.scale, st.delta, st.sel, st.sel_count)
    gk = capture(batch, None, torch)
    gk.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        gk.replay()
    e1.record()
    torch.cuda.synchronize()
    sel_us = e0.elapsed_time(e1) / (reps * n_k) * 1e3
    for s in sets_d:  # leave the pools as whole steps leave them
        run_sparse_step(s)
    torch.cuda.synchronize()
    return {"delta": args.delta, "us_per_step": round(step_us, 3),
            "vs_topk_step": round(step_us / step_us_topk, 3),
            "select_topdelta_us": round(sel_us, 3),
            "kept_pages_per_unit": {"mean": round(float(np.mean(kept)), 2),
                                    "min": int(kept.min()), "max": int(kept.max())},
            "launches": step_launches(sets_d[0]["step"]),
            "parity": dict(parity, oracle="top-delta rule")}


def fp8_line(args, w, sets, step_us_kv, torch, wl, ps, acc):
    """The same inputs with 8-bit metadata bounds: parity against the oracle
    scoring the 8-bit bounds, then the step timed as the main one (one graph
    of one step per input set) and the refresh+score launch on its own."""
    sets8 = [make_set(w, None, torch, wl, ps, "fp8", inp=s["inp"],
                      meta_layout=args.fp8_meta_layout)
             for s in sets]
    run_sparse_step(sets8[0])
    torch.cuda.synchronize()
    parity = parity_gate(sets8[0], w, sample_units(w, args.parity_units), wl)

    multi, r_graph = capture_steps(run_sparse_step, sets8, torch)
    for _ in range(3):
        multi.replay()
    torch.cuda.synchronize()
    reps = max(args.steps // r_graph, 1)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        multi.replay()
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) / (reps * r_graph) * 1e3

    n_k = 40

    def batch(_):
        for i in range(n_k):
            s = sets8[i % len(sets8)]
            inp = s["inp"]
            ps.ps_refresh_score_pages(s["g"], inp["q"], inp["k_pool"], s["meta"],
                                      inp["page_table"], inp["seq_lens"], s["step"].scores)
    gk = capture(batch, None, torch)
    gk.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        gk.replay()
    e1.record()
    torch.cuda.synchronize()
    score_us = e0.elapsed_time(e1) / (reps * n_k) * 1e3
    for s in sets8:  # leave the pools as whole steps leave them
        run_sparse_step(s)
    torch.cuda.synchronize()

    lens = [int(x) for x in sets8[0]["inp"]["seq_lens_host"]]
    elem = 2 if w.kv_dtype == "bf16" else 4
    meta_b = acc.meta_bytes(lens, w.num_kv_heads, w.head_dim, 1, w.page_size)
    units = w.batch * w.num_kv_heads
    scores_b = sum(-(-n // w.page_size) for n in lens) * w.num_kv_heads * 4
    dom_b = meta_b + scores_b + units * (w.page_size * elem + 2) * w.head_dim
    sel_h = sets8[0]["step"].sel.cpu().numpy()
    lists = {(b, g): list(sel_h[b, g]) for b in range(w.batch) for g in range(w.num_kv_heads)}
    kv_b = acc.selected_kv_bytes(lens, lists, w.head_dim, elem, w.page_size)
    del sets8
    gbps = dom_b / (score_us * 1e-6) / 1e9
    return {"us_per_step": round(step_us, 3),
            "speedup_vs_kv_dtype_metadata": round(step_us_kv / step_us, 3),
            "touched_bytes": meta_b + kv_b,
            "effective_hbm_gbps": round((meta_b + kv_b) / (step_us * 1e-6) / 1e9, 1),
            "refresh_score_us": round(score_us, 3),
            "refresh_score_gbps": round(gbps, 1),
            "refresh_score_frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "refresh_score_algorithmic_bytes": dom_b,
            "metadata_layout": args.fp8_meta_layout,
            "parity": dict(parity, oracle="scores on the 8-bit bounds")}


def profile_only(args, sets, torch, ps):
    """Launch one stage repeatedly (for rocprofv3 counter runs)."""
    for i in range(args.steps):
        s = sets[i % len(sets)]
        inp, step, g = s["inp"], s["step"], s["g"]
        if args.only_kernel == "score":  # the step's score launch
            ps.ps_refresh_score_pages(g, inp["q"], inp["k_pool"], s["meta"], inp["page_table"],
                                      inp["seq_lens"], step.scores)
        elif args.only_kernel == "step":
            run_sparse_step(s)
        elif args.only_kernel == "copy":
            # calibration for the HBM byte counters: a plain 1 GiB device copy
            if i == 0:
                src = torch.empty(1 << 28, device="cuda", dtype=torch.float32)
                dst = torch.empty_like(src)
            dst.copy_(src)
        else:
            raise SystemExit(f"unknown stage {args.only_kernel}")
    torch.cuda.synchronize()
    print(json.dumps({"profile_only": args.only_kernel, "launches": args.steps}), flush=True)


if __name__ == "__main__":
    main()
