#!/usr/bin/env python3
"""Batch-1 decode benchmark of the 27B-shape hybrid W4 stack on one MI355X.

Workload (the full synthetic stack): 64 layers (48 Gated DeltaNet + 16 gated
attention, 3:1), W4A16 group-32 random weights (~14.2 GB), int8 lm_head with
vocab 248320, an 8192-token random prompt, then greedy decode.  The pages the
method comes from measure single-user decode speed of this model class in
tok/s and attribute it to weight streaming (page 5, bs178.com llamAmpere
article, "为什么它真能这么快" point 二); the metric here is decode tok/s plus
the fraction of the HBM roofline (algorithmic bytes per token / 8 TB/s).

Timed region: `--steps` greedy steps through aw4_decode_greedy (one captured
HIP graph per token, argmax fed back on the device), after `--warmup` steps,
with weights, prompt state and caches already resident in HBM.

Prints one JSON line.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


# HBM bytes per launch of the gate/up GEMV from the FETCH_SIZE / WRITE_SIZE
# counter runs recorded in profiles/hbm_traffic_8k_decode.md, valid only for
# the kernel source whose sha256 prefix is recorded with them.
GATEUP_TRAFFIC = {"k_gemv_sha256": "c5ad4ccaf7ce5010", "bytes": 100812527}


def gateup_traffic():
    import hashlib
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "attention_w4_amd", "csrc", "k_gemv.hip")
    try:
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    return GATEUP_TRAFFIC["bytes"] if h == GATEUP_TRAFFIC["k_gemv_sha256"] else None


def step_bytes(shape, pos):
    """Algorithmic HBM bytes of one decode step at position pos (the token
    attends to pos + 1 cached positions)."""
    from synth import workloads as W
    H, F = shape.hidden, shape.ffn
    w4 = lambda r, c: r * c // 2 + r * (c // 32) * 2
    b = 0
    for t in shape.pattern:
        b += w4(W.mixer_in_rows(shape, t), H) + w4(H, W.mixer_out_cols(shape, t))
        b += 2 * w4(F, H) + w4(H, F)
    if shape.vocab:
        b += shape.vocab * H + shape.vocab * (H // 32) * 2      # int8 head
        b += shape.vocab * 4                                    # logits
    ng = shape.pattern.count("G")
    na = shape.pattern.count("A")
    b += ng * shape.gdn_v_heads * shape.gdn_head_dim ** 2 * 4 * 2   # state read + write
    b += na * kv_bytes_per_pos(shape) * (pos + 1)               # cache read incl. the new entry
    return b


def kv_bytes_per_pos(shape):
    """cache bytes of one position of one attention layer, all kv heads: key
    codes, value codes and the two fp16 scales per 32 dims (format 1 stores 4-bit
    keys and values, formats 0 and 2 int8 keys and 3-bit values)"""
    d = shape.attn_head_dim
    codes = d // 2 + d // 2 if getattr(shape, "kv_format", 0) == 1 else d + d * 3 // 8
    return shape.attn_kv_heads * (codes + 2 * (d // 32) * 2)


def cpu_baseline(ctx, seed, long_ctx=0):
    """Oracle on a bounded sample: one GDN layer step and one attention layer
    step at `ctx` cached positions (synthetic state), and the int8 head over a
    1/8 slice of the vocabulary; scaled to one full token.  With long_ctx, also
    one attention layer step at long_ctx cached positions, scaled the same way
    (the GDN layers and the head do not depend on the context)."""
    import numpy as np
    import oracle
    import synth
    from synth import state as SS
    from synth import workloads as W
    full = W.FULL_27B
    g = W.with_(full, pattern="G", vocab=0, max_ctx=ctx + 8, draft_vocab=0)
    a = W.with_(full, pattern="A", vocab=full.vocab // 8, max_ctx=ctx + 8, draft_vocab=0)
    og = oracle.from_recipe(g, seed)
    oa = oracle.from_recipe(a, seed)
    SS.fill(og, g, ctx, seed)
    SS.fill(oa, a, ctx, seed)
    x = synth.normal(1, full.hidden, 1.0, seed, W.STREAM_HIDDEN)[0].astype(np.float64)

    def med(f, n=3):
        f()
        ts = []
        for _ in range(n):
            t0 = time.perf_counter()
            f()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    def step_g():
        og.set_pos(ctx)
        og.forward_layers(x)

    def step_a():
        oa.set_pos(ctx)
        oa.forward_layers(x)

    tg, ta = med(step_g), med(step_a)
    th = med(lambda: oa.head(x)) * 8
    ng, na = full.pattern.count("G"), full.pattern.count("A")
    per_token = ng * tg + na * ta + th
    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    out = {"value": round(1.0 / per_token, 4), "unit": "tok/s", "cores": min(cores, threads), "kind": "oracle",
           "sample": (f"fp64 C oracle: 1 GDN layer step ({tg:.3f} s) and 1 attention layer step ({ta:.3f} s) at "
                      f"{ctx} cached positions, int8 head over vocab/8 ({th / 8:.3f} s); median of 3; "
                      f"scaled to 48 + 16 layers + full head = {per_token:.2f} s/token")}
    if long_ctx:
        del oa
        al = W.with_(full, pattern="A", vocab=0, max_ctx=long_ctx + 8, draft_vocab=0)
        ol = oracle.from_recipe(al, seed)
        SS.fill(ol, al, long_ctx, seed)

        def step_l():
            ol.set_pos(long_ctx)
            ol.forward_layers(x)

        tl = med(step_l)
        per_long = ng * tg + na * tl + th
        out["ctx_" + ("262k" if long_ctx == 262144 else str(long_ctx))] = {
            "value": round(1.0 / per_long, 4), "unit": "tok/s",
            "sample": (f"1 attention layer step at {long_ctx} cached positions ({tl:.3f} s, median of 3) with the "
                       f"GDN layer and head times above; scaled to {per_long:.2f} s/token")}
    return out


def stream_probe(torch, A, sizes=((1 << 30, 20), (100_000_000 // 16 * 16, 100))):
    """Measured streaming-read bandwidth of the device: a plain read
    (aw4_time_stream_read: 512 workgroups over contiguous chunks, 16-byte
    non-temporal loads, eight 4 KB loads in flight per workgroup) of 1 GiB and
    of 100 MB, average over reps launches."""
    out = {}
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for nbytes, reps in sizes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        us = A.time_stream_read(buf, sink, stream, reps)
        out["read_1GiB" if nbytes == 1 << 30 else f"read_{nbytes // 1_000_000}MB"] = {
            "bytes": nbytes, "avg_us": round(us, 2), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del buf
    torch.cuda.empty_cache()
    return out


def long_leg(args, torch, A, W, SS, synth):
    """Greedy decode and draft verification at a long cached context.  The
    cache and the recurrent states are a seeded synthetic state (prefilling
    262K positions token by token would take about 20 minutes); drafts come
    from a synthetic draft distribution q (softmax of N(0, 1.43^2) logits,
    fixed per draft slot), so the acceptance rate is that of an unrelated
    draft model and says nothing about a trained one."""
    import numpy as np
    from synth.gpu_load import load_recipe
    ctx = args.long_ctx
    k = 3
    shape = W.with_(W.FULL_27B, max_ctx=ctx + 16 + args.long_steps + (k + 1) * (args.verify_passes + args.draft_passes) + 16)
    m = A.Model(shape)
    load_recipe(m, shape, args.seed)
    t0 = time.time()
    # the seeded state, generated a few layers at a time on host threads
    from concurrent.futures import ThreadPoolExecutor
    SS.fill(m, shape, ctx - 1, args.seed, kv=False)
    alayers = [l for l, t in enumerate(shape.pattern) if t == "A"]
    with ThreadPoolExecutor(4) as ex:
        for l, kv in zip(alayers, ex.map(lambda l: SS.kv_state(shape, l, ctx - 1, args.seed), alayers)):
            m.import_kv(l, *kv)
    m.set_pos(ctx - 1)
    m.sync()
    t_fill = time.time() - t0
    first = int(synth.tokens(1, shape.vocab, args.seed + 1)[0])
    warm = m.decode_greedy(first, 8)
    tok = int(warm[-1])
    pos0 = m.pos
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    toks = m.decode_greedy(tok, args.long_steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nbytes = sum(step_bytes(shape, p) for p in range(pos0, pos0 + args.long_steps))
    res = {"tok/s": round(args.long_steps / wall, 2), "ms_per_step": round(wall * 1e3 / args.long_steps, 4),
           "steps": args.long_steps, "ctx_start": int(pos0),
           "algorithmic_GB_per_step": round(nbytes / args.long_steps / 1e9, 4),
           "achieved_GB/s": round(nbytes / wall / 1e9, 1), "frac_of_8TB/s": round(nbytes / wall / 1e9 / HBM_PEAK_GBS, 4),
           "state": "seeded synthetic cache and recurrent states", "setup_fill_s": round(t_fill, 1)}
    if args.verify_passes:
        V = shape.vocab
        logits = synth.normal(k, V, W.DRAFT_LOGIT_STD, args.seed, W.STREAM_DRAFT).astype(np.float64)
        z = np.exp(logits - logits.max(axis=1, keepdims=True))
        q = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
        cq = np.cumsum(q.astype(np.float64), axis=1)
        qd = torch.from_numpy(q).cuda()
        du = synth.uniform(k * args.verify_passes, args.seed, W.STREAM_UNIFORM, i0=1 << 20).reshape(-1, k)
        uu = synth.uniform((k + 1) * args.verify_passes, args.seed, W.STREAM_UNIFORM, i0=1 << 22).reshape(-1, k + 1)
        t = int(toks[-1])
        emitted = accepted = 0
        m.verify_k([t] + [int(np.searchsorted(cq[j], du[0, j] * cq[j, -1], side="right")) for j in range(k)],
                   qd, uu[0], 1.0)   # warm-up pass (graph-free path, first-use costs)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for p in range(args.verify_passes):
            drafts = [min(V - 1, int(np.searchsorted(cq[j], du[p, j] * cq[j, -1], side="right"))) for j in range(k)]
            out = m.verify_k([t] + drafts, qd, uu[p], 1.0)
            emitted += len(out)
            accepted += len(out) - 1
            t = out[-1]
        wall = time.perf_counter() - t0
        res["verify"] = {"drafts_per_pass": k, "passes": args.verify_passes,
                         "passes/s": round(args.verify_passes / wall, 2),
                         "ms_per_pass": round(wall * 1e3 / args.verify_passes, 3),
                         "emitted_tok/s": round(emitted / wall, 2),
                         "accepted_per_pass": round(accepted / args.verify_passes, 3),
                         "temperature": 1.0, "draft_q": "softmax of N(0, 1.43^2) logits per slot (synthetic)"}
    if args.draft_passes:
        t_last = t if args.verify_passes else int(toks[-1])
        res["draft_head"] = draft_leg(args, torch, A, m, shape, synth, W, t_last)
    m.close()
    del m
    torch.cuda.empty_cache()
    return res


def draft_leg(args, torch, A, m, shape, synth, W, t):
    """Speculative decoding with the model's own draft head: per pass, three
    drafts from aw4_draft (temperature 1, q over the 65,536 mapped ids) then one
    aw4_verify_k pass with that q.  With random weights the draft head and the
    target are unrelated, so the acceptance rate says nothing about a trained
    draft head; the timings are what this leg measures.  Also times the draft
    head's mapped int8 projection against the full output head."""
    import numpy as np
    k, P = 3, args.draft_passes
    V = shape.vocab
    q = torch.empty(k, V, dtype=torch.float32, device="cuda")
    du = synth.uniform(k * (P + 1), args.seed, W.STREAM_UNIFORM, i0=1 << 24).reshape(-1, k)
    uu = synth.uniform((k + 1) * (P + 1), args.seed, W.STREAM_UNIFORM, i0=1 << 25).reshape(-1, k + 1)
    d = m.draft(t, k, 1.0, du[P], q=q)   # warm-up pass (t: the last emitted token)
    t = m.verify_k([t] + d, q, uu[P], 1.0)[-1]
    torch.cuda.synchronize()
    t_draft = t_verify = 0.0
    emitted = accepted = 0
    for p in range(P):
        t0 = time.perf_counter()
        d = m.draft(t, k, 1.0, du[p], q=q)
        t1 = time.perf_counter()
        out = m.verify_k([t] + d, q, uu[p], 1.0)
        t2 = time.perf_counter()
        t_draft += t1 - t0
        t_verify += t2 - t1
        emitted += len(out)
        accepted += len(out) - 1
        t = out[-1]
    wall = t_draft + t_verify
    reps = max(8, args.phase_reps // 4)
    us_map, b_map = m.time_phase(A.PHASE_DRAFT_HEAD, reps)
    us_full, b_full = m.time_phase(A.PHASE_HEAD, reps)
    return {"drafts_per_pass": k, "passes": P, "temperature": 1.0,
            "passes/s": round(P / wall, 2), "ms_per_pass": round(wall * 1e3 / P, 3),
            "draft_ms_per_call": round(t_draft * 1e3 / P, 3), "verify_ms_per_pass": round(t_verify * 1e3 / P, 3),
            "emitted_tok/s": round(emitted / wall, 2), "accepted_per_pass": round(accepted / P, 3),
            "draft_cache_entries": int(m.dpos),
            "mapped_head": {"ids": shape.draft_vocab, "avg_us": round(us_map, 2), "bytes": b_map,
                            "GB/s": round(b_map / (us_map * 1e-6) / 1e9, 1)},
            "full_head": {"ids": V, "avg_us": round(us_full, 2), "bytes": b_full,
                          "GB/s": round(b_full / (us_full * 1e-6) / 1e9, 1)},
            "mapped_over_full_MACs": round(shape.draft_vocab / V, 4),
            "mapped_over_full_time": round(us_map / us_full, 4),
            "weights": "random: acceptance is that of an untrained draft head"}


def window_leg(args, torch, A, W, SS, synth):
    """Greedy decode with the recent-window KV variant (the last W positions of
    every attention layer read at fp16, older ones from their codes), from a
    seeded synthetic state of ctx positions whose ring holds fp16 values, at
    each context of --window-ctx.  Algorithmic bytes per step: the plain step's
    bytes with the window's positions counted at 2 x 2 x dh bytes (fp16 key and
    value) instead of the 384 bytes of their codes and scales, per kv head and
    attention layer."""
    from concurrent.futures import ThreadPoolExecutor
    from synth.gpu_load import load_recipe
    out = {"window": args.window}
    for ctx in [int(c) for c in args.window_ctx.split(",") if c]:
        shape = W.with_(W.FULL_27B, max_ctx=ctx + args.window_steps + 32, draft_vocab=0, kv_window=args.window)
        m = A.Model(shape)
        load_recipe(m, shape, args.seed)
        t0 = time.time()
        SS.fill(m, shape, ctx - 1, args.seed, kv=False)
        alayers = [l for l, t in enumerate(shape.pattern) if t == "A"]
        with ThreadPoolExecutor(4) as ex:
            for l, kv in zip(alayers, ex.map(lambda l: SS.kv_state(shape, l, ctx - 1, args.seed), alayers)):
                m.import_kv(l, *kv)
                m.import_win(l, *SS.win_state(shape, l, args.seed))
        m.set_pos(ctx - 1)
        m.sync()
        t_fill = time.time() - t0
        first = int(synth.tokens(1, shape.vocab, args.seed + 2)[0])
        tok = int(m.decode_greedy(first, 8)[-1])
        pos0 = m.pos
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        m.decode_greedy(tok, args.window_steps)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        d, nkv, na = shape.attn_head_dim, shape.attn_kv_heads, shape.pattern.count("A")
        nbytes = sum(step_bytes(shape, p) + na * nkv * min(args.window, p + 1) * (4 * d - 384)
                     for p in range(pos0, pos0 + args.window_steps))
        out[f"ctx_{ctx}"] = {"tok/s": round(args.window_steps / wall, 2),
                             "ms_per_step": round(wall * 1e3 / args.window_steps, 4),
                             "steps": args.window_steps, "ctx_start": int(pos0),
                             "algorithmic_GB_per_step": round(nbytes / args.window_steps / 1e9, 4),
                             "frac_of_8TB/s": round(nbytes / wall / 1e9 / HBM_PEAK_GBS, 4),
                             "setup_fill_s": round(t_fill, 1)}
        m.close()
        del m
        torch.cuda.empty_cache()
    out["state"] = "seeded synthetic cache, recurrent states and fp16 ring"
    return out


def kvformat_leg(args, torch, A, W, SS, synth):
    """Greedy decode at a long context with the other cache codecs: format 1
    (q4_0, keys and values 4-bit, values not rotated) and format 2 (int8 keys,
    values rotated then coded with the Lloyd-Max codebook), each from a seeded
    synthetic state in its format.  Algorithmic bytes count the format's cache
    bytes per position."""
    from concurrent.futures import ThreadPoolExecutor
    from synth.gpu_load import load_recipe
    out = {}
    ctx = args.kvformat_ctx
    for fmt in (1, 2):
        shape = W.with_(W.FULL_27B, max_ctx=ctx + args.kvformat_steps + 32, draft_vocab=0, kv_format=fmt)
        m = A.Model(shape)
        load_recipe(m, shape, args.seed)
        t0 = time.time()
        SS.fill(m, shape, ctx - 1, args.seed, kv=False)
        alayers = [l for l, t in enumerate(shape.pattern) if t == "A"]
        with ThreadPoolExecutor(4) as ex:
            for l, kv in zip(alayers, ex.map(lambda l: SS.kv_state(shape, l, ctx - 1, args.seed), alayers)):
                m.import_kv(l, *kv)
        m.set_pos(ctx - 1)
        m.sync()
        t_fill = time.time() - t0
        tok = int(m.decode_greedy(int(synth.tokens(1, shape.vocab, args.seed + 3)[0]), 8)[-1])
        pos0 = m.pos
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        m.decode_greedy(tok, args.kvformat_steps)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        nbytes = sum(step_bytes(shape, p) for p in range(pos0, pos0 + args.kvformat_steps))
        out[f"format_{fmt}"] = {"codec": "q4_0: K and V 4-bit, V not rotated" if fmt == 1 else
                                "K int8, V rotated + 3-bit Lloyd-Max codebook",
                                "tok/s": round(args.kvformat_steps / wall, 2),
                                "ms_per_step": round(wall * 1e3 / args.kvformat_steps, 4),
                                "steps": args.kvformat_steps, "ctx_start": int(pos0),
                                "cache_bytes_per_position": kv_bytes_per_pos(shape) * len(alayers),
                                "algorithmic_GB_per_step": round(nbytes / args.kvformat_steps / 1e9, 4),
                                "frac_of_8TB/s": round(nbytes / wall / 1e9 / HBM_PEAK_GBS, 4),
                                "setup_fill_s": round(t_fill, 1)}
        m.close()
        del m
        torch.cuda.empty_cache()
    out["state"] = "seeded synthetic cache and recurrent states in each format"
    return out


def batch_leg(args, torch, m, shape, SS, synth):
    """Batch decode: B sequences (B = 1..4), each from its own seeded synthetic
    state of ctx positions, one greedy step each per aw4_decode_batch call;
    aggregate tok/s over the B sequences."""
    for b in range(4):
        m.select_sequence(b)
        SS.fill(m, shape, args.ctx, args.seed + b)
    m.select_sequence(0)
    first = [int(t) for t in synth.tokens(4, shape.vocab, args.seed, i0=1 << 20)]
    res = {}
    cur = list(first)
    for B in (1, 2, 3, 4):
        m.decode_batch(cur[:B])   # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.batch_steps):
            out = m.decode_batch(cur[:B])
            cur[:B] = out
        wall = time.perf_counter() - t0
        pos = args.ctx
        state = shape.pattern.count("G") * shape.gdn_v_heads * shape.gdn_head_dim ** 2 * 8
        kv = shape.pattern.count("A") * kv_bytes_per_pos(shape) * (pos + 1)
        weights = step_bytes(shape, 0) - state - shape.pattern.count("A") * kv_bytes_per_pos(shape)
        nbytes = weights + B * (state + kv)
        res[f"B{B}"] = {"tok/s": round(B * args.batch_steps / wall, 1),
                        "ms_per_step": round(wall * 1e3 / args.batch_steps, 3),
                        "algorithmic_GB_per_step": round(nbytes / 1e9, 3),
                        "frac_of_8TB/s": round(nbytes / (wall / args.batch_steps) / 1e9 / HBM_PEAK_GBS, 4)}
    res["note"] = (f"each sequence from its own seeded {args.ctx}-position synthetic state, "
                   f"{args.batch_steps} steps per batch size, weights read once per step")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--ctx", type=int, default=8192, help="prompt length before the timed steps")
    ap.add_argument("--prompt", choices=["decode", "synthetic"], default="decode",
                    help="decode: run the random prompt through the model; synthetic: import a seeded "
                         "cache/state of ctx positions")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--phase-reps", type=int, default=128)
    ap.add_argument("--long-ctx", type=int, default=262144,
                    help="second leg: cached positions of the long-context decode and verify runs (0: skip)")
    ap.add_argument("--long-steps", type=int, default=256, help="timed greedy steps at --long-ctx")
    ap.add_argument("--verify-passes", type=int, default=64, help="timed verify_k passes at --long-ctx (3 drafts)")
    ap.add_argument("--draft-passes", type=int, default=64,
                    help="timed draft (aw4_draft, 3 drafts) + verify passes at --long-ctx")
    ap.add_argument("--batch-steps", type=int, default=64, help="timed aw4_decode_batch steps per batch size 1..4 (0: skip)")
    ap.add_argument("--window", type=int, default=2048,
                    help="recent-window leg: positions kept at fp16 per attention layer (0: skip)")
    ap.add_argument("--window-ctx", default="8192,131072", help="contexts of the recent-window leg")
    ap.add_argument("--window-steps", type=int, default=128, help="timed greedy steps per window context")
    ap.add_argument("--kvformat-ctx", type=int, default=262144,
                    help="cached positions of the q4_0 and codebook cache legs (0: skip)")
    ap.add_argument("--kvformat-steps", type=int, default=128, help="timed greedy steps per cache format")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size kernel for counter runs)")
    args = ap.parse_args()
    if args.phase_reps < 1:
        ap.error("--phase-reps must be at least 1 (the roofline figure times the dominant kernel)")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the batch-1 decode path is built "
                                   "and measured on a single MI355X; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import attention_w4_amd as A
    import synth
    from synth import workloads as W
    from synth import state as SS
    from synth.gpu_load import load_recipe

    if args.calib_copy_mb:
        n = args.calib_copy_mb << 18   # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    shape = W.with_(W.FULL_27B, max_ctx=max(args.ctx + args.warmup + args.steps, args.ctx + 4 * args.batch_steps) + 8,
                    max_batch=4 if args.batch_steps else 1)
    t0 = time.time()
    m = A.Model(shape)
    load_recipe(m, shape, args.seed)
    t_load = time.time() - t0
    prompt = synth.tokens(args.ctx, shape.vocab, args.seed)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if args.prompt == "decode":
        m.prefill(prompt[:-1])
    else:
        SS.fill(m, shape, args.ctx - 1, args.seed)
    m.sync()
    t_prompt = time.perf_counter() - t0
    first = int(prompt[-1])
    warm = m.decode_greedy(first, args.warmup) if args.warmup else [first]
    tok = int(warm[-1])
    pos0 = m.pos

    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(m.stream)
    t0 = time.perf_counter()
    toks = m.decode_greedy(tok, args.steps)
    ev1.record(m.stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    gpu_ms = ev0.elapsed_time(ev1)
    tok_s = args.steps / wall
    ms_step = wall * 1e3 / args.steps
    total_bytes = sum(step_bytes(shape, p) for p in range(pos0, pos0 + args.steps))
    gbs = total_bytes / wall / 1e9

    # dominant kernel: the fused RMSNorm + gate/up W4 GEMV + SwiGLU (66% of the
    # weight bytes are FFN, gate/up alone 46% of the step)
    us, nbytes = m.time_phase(A.PHASE_FFN_GATE_UP, args.phase_reps)
    ach = nbytes / (us * 1e-6) / 1e9
    probe = stream_probe(torch, A)
    probe_gbs = probe["read_1GiB"]["GB/s"]
    others = {}
    for name, ph in (("ffn_down", A.PHASE_FFN_DOWN), ("mixer_in", A.PHASE_MIX_IN)):
        u, b = m.time_phase(ph, args.phase_reps)
        others[name] = {"avg_us": round(u, 2), "bytes": b, "GB/s": round(b / (u * 1e-6) / 1e9, 1)}
    # prefill: the prompt above through aw4_prefill (chunks of 1024 tokens),
    # and its dominant kernel, the gate/up W4 GEMM over one chunk, on MFMA
    prefill = None
    if args.prompt == "decode":
        pu, pf = m.time_phase(A.PHASE_PREFILL_GATE_UP, max(16, args.phase_reps // 2))
        prefill = {"tokens": args.ctx - 1, "s": round(t_prompt, 3), "tok/s": round((args.ctx - 1) / t_prompt, 1),
                   "chunk": 1024, "note": "also feeds the draft head one entry per prompt position",
                   "gemm_roofline": {"kernel": "k_gemm_w4 (FFN gate/up + SwiGLU), M 1024 tokens, N 34816, K 5120",
                                     "bound": "mfma", "achieved": round(pf / (pu * 1e-6) / 1e12, 1),
                                     "peak": 2500.0, "unit": "TFLOP/s",
                                     "frac": round(pf / (pu * 1e-6) / 1e12 / 2500.0, 4), "avg_launch_us": round(pu, 2),
                                     "flops_per_launch": pf}}

    out = {
        "metric": "batch-1 decode tok/s (27B-shape W4) + % of HBM roofline, 8K and 262K ctx",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "w4a16 (int4 codes x fp16 scales, fp16 activations, fp32 accumulate)",
        "data": "synthetic (seeded random weights, random prompt)",
        "config": {"workload": f"27B-shape hybrid stack, 64 layers (48 GDN + 16 gated attention), "
                               f"{args.ctx}-token random prompt then greedy decode, batch 1",
                   "ctx_start": int(pos0), "prompt": args.prompt, "global_batch": 1},
        "hbm": {"algorithmic_GB_per_step": round(total_bytes / args.steps / 1e9, 4),
                "achieved_GB/s": round(gbs, 1), "frac_of_8TB/s": round(gbs / HBM_PEAK_GBS, 4),
                "frac_of_measured_read": round(gbs / probe_gbs, 4), "gpu_event_ms": round(gpu_ms, 3),
                "measured_read_probe": probe},
        "roofline": {"kernel": "k_gemv_stream (RMSNorm + FFN gate/up W4 GEMV + SwiGLU), K=5120, 34816 rows",
                     "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "frac_of_measured_read": round(ach / probe_gbs, 4),
                     "traffic": gateup_traffic(),
                     "avg_launch_us": round(us, 3), "bytes_per_launch": nbytes, "other_kernels": others},
        "prefill": prefill,
        "setup_s": {"load": round(t_load, 1), "prompt": round(t_prompt, 1)},
        "first_tokens": [int(t) for t in toks[:8]],
    }
    if args.batch_steps:
        out["batch"] = batch_leg(args, torch, m, shape, SS, synth)
    if args.window:
        out["kv_window"] = window_leg(args, torch, A, W, SS, synth)
    m.close()
    del m
    torch.cuda.empty_cache()
    if args.long_ctx:
        out["ctx_262k" if args.long_ctx == 262144 else f"ctx_{args.long_ctx}"] = long_leg(args, torch, A, W, SS, synth)
    if args.kvformat_ctx:
        out["kv_formats"] = kvformat_leg(args, torch, A, W, SS, synth)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.ctx, args.seed, args.long_ctx)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
