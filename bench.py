#!/usr/bin/env python3
"""Packed segment-id masked attention, fwd+bwd, on one MI355X.

One step = the whole hot path over the 4 x 288-frame pack (episodes of
119/177/285/239 valid frames padded to 288 frames, 32 tokens per frame ->
36,864 tokens, 24 heads x 128, bf16): per-token seq ids from the valid frame
counts, the block mask, the forward, and the backward (row sums, dQ, dK/dV).
Inputs are synthetic (seeded, N(0,1)*0.5 bf16) and already resident in HBM.

Prints ONE JSON line on stdout.  value = useful TFLOP/s = 14 * d * P * H /
step time, where P counts only the allowed (same id, id >= 0) query-key pairs
per head (value_12dPH: the same time counted without the recompute).
Per-stage times (HIP events on the stream the library launches on) go to
stderr and into the JSON's "stages_ms" object.  After the timed steps the
other workloads are measured the same way (extras.configs: the 4 x 120-frame
pack, all 40 batches of the length-bucketed sweep, self and cross, the
64k mixed pack, and the 4 x 288 pack's segments permuted in 512-token pieces),
the block-mask builder alone (extras.mask_builder: GB/s of
its algorithmic bytes on the 4 x 288 and 64k packs and a 1,048,576-token case),
then the next rows (masked loss, unpadded pack, planner, AdaLN) and the fp64
CPU oracle on all heads of the pack (cpu_baseline).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "masked-attn fwd+bwd useful TFLOP/s, 4×288-frame pack; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
# algorithmic flops per allowed (query, key) pair per head, in units of head_dim
FLOPS_PER_PAIR = {"fwd": 4, "bwd_dq": 6, "bwd_dkdv": 8}


KERNEL_SOURCES = {  # the files a kernel's code comes from (hashed to validate traffic figures)
    "fwd": ["packed_variable_length_amd/csrc/attn_fwd.hip"],
    "bwd_dq": ["packed_variable_length_amd/csrc/attn_bwd.hip"],
    "bwd_dkdv": ["packed_variable_length_amd/csrc/attn_bwd.hip"],
    "adaln_fwd": ["packed_variable_length_amd/csrc/adaln.hip"],
    "adaln_bwd": ["packed_variable_length_amd/csrc/adaln.hip"],
    "masked_loss": ["packed_variable_length_amd/csrc/masked_loss.hip"],
}
COMMON_SOURCES = ["packed_variable_length_amd/csrc/pa_tile.h",
                  "packed_variable_length_amd/csrc/pa_common.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha256(stage):
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[stage] + COMMON_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(stage, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none for this kernel and workload or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}_hbm.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_sha256(stage):
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(spec, q, k, v, do, heads):
    """Time the fp64 CPU oracle on a bounded sample (a subset of heads)."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import seqids as osid
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity size
        threads = len(os.sched_getaffinity(0))
    ids = (spec.segment_ids if spec.segment_ids is not None else
           osid.seq_ids_from_valid_frames(spec.valid_frames, spec.frames_padded,
                                          spec.q_tokens_per_frame))
    t0 = time.perf_counter()
    oatt.forward_backward(q, k, v, do, ids, ids, spec.scale, heads=heads)
    dt = time.perf_counter() - t0
    pairs = oatt.useful_pairs(ids, ids)
    flops = 14.0 * spec.head_dim * pairs * len(heads)
    del np
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{spec.name}: fp64 fwd+bwd of heads {heads} of {spec.heads} "
                      f"(all {spec.nq} tokens), useful flops 14*d*P per head"}


PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published


def time_calls(fn, iters, warmup=3):
    """Average ms per call of fn() from HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def bench_masked_loss(pa, ids, channels=192, iters=50):
    """Frame-valid masked loss (fused value + gradient) on the pack's token ids:
    a latent regression output of `channels` bf16 values per token."""
    import torch
    n = ids.numel()
    g = torch.Generator(device=ids.device).manual_seed(7)
    pred = torch.randn((n, channels), generator=g, device=ids.device).to(torch.bfloat16)
    target = torch.randn((n, channels), generator=g, device=ids.device).to(torch.bfloat16)
    stats = torch.empty(4, dtype=torch.float32, device=ids.device)
    dpred = torch.empty_like(pred)
    ws = torch.empty(pa.masked_mse_workspace_bytes(n), dtype=torch.uint8, device=ids.device)
    ms = time_calls(lambda: pa.masked_mse_fwd_bwd(pred, target, ids, 1.0, stats, dpred, ws), iters)
    nv = int((ids >= 0).sum().item())
    # reads: ids twice (count, main pass), pred and target of valid rows; writes:
    # every gradient row (zeros on padding rows); partials are negligible
    nbytes = 2 * 4 * n + 2 * 2 * channels * nv + 2 * channels * n
    return {"entry": "masked_mse_fwd_bwd", "shape": f"{n} x {channels} bf16, {nv} valid rows",
            "traffic": measured_traffic("masked_loss", f"latent-{n}x{channels}"),
            "avg_call_ms": round(ms, 5), "algorithmic_bytes": nbytes,
            "achieved_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak_GBs": PEAK_HBM_GBS,
            "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "bound": "hbm"}


def bench_unpadded_pack(pa, iters=5):
    """Whole hot path (ids from lengths, mask, fwd, bwd) on the first 68,000-token
    unpadded pack the next-fit packer makes from the episode stream."""
    import numpy as np
    import torch

    import workloads as wl
    lengths = wl.episode_stream()
    pack_of, _ = pa.plan_token_packs(lengths, wl.UNPADDED_BUDGET)
    sel = lengths[pack_of == 0]
    s = wl.unpadded_pack(sel)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(11)
    mk = lambda: (0.5 * torch.randn((s.nq, s.heads, s.head_dim), generator=g,  # noqa: E731
                                    device=dev)).to(torch.bfloat16)
    Q, K, V = mk(), mk(), mk()
    DO = (2 * mk().float()).to(torch.bfloat16)
    L = torch.from_numpy(sel).to(dev)
    ids = torch.empty(s.nq, dtype=torch.int32, device=dev)
    O, dQ, dK, dV = (torch.empty_like(Q) for _ in range(4))
    lse = torch.empty((s.heads, s.nq), dtype=torch.float32, device=dev)
    ws = torch.empty(pa.attn_packed_bwd_workspace_bytes(torch.bfloat16, s.nq, s.nq, s.heads,
                                                        s.head_dim), dtype=torch.uint8,
                     device=dev)
    mstore = torch.empty(pa.build_block_mask_bytes(s.nq, s.nq, 128, 128), dtype=torch.uint8,
                         device=dev)

    def step():
        pa.seq_ids_from_lengths(L, s.nq, out=ids)
        mask = pa.build_block_mask(ids, ids, 128, 128, storage=mstore)
        pa.attn_packed_fwd(Q, K, V, ids, ids, mask, s.scale, out=O, lse=lse)
        pa.attn_packed_bwd(Q, K, V, O, DO, lse, ids, ids, mask, s.scale, workspace=ws,
                           grads=(dQ, dK, dV))
    ms = time_calls(step, iters, warmup=2)
    pairs = int((sel.astype(np.int64) ** 2).sum())
    useful = 14.0 * s.head_dim * pairs * s.heads
    tf = useful / (ms * 1e-3) / 1e12
    return {"workload": f"{len(sel)} episodes ({int(sel.sum())} tokens) back to back in a "
                        f"{s.nq}-token buffer, {s.heads} heads x {s.head_dim} bf16",
            "ms_per_step": round(ms, 4), "useful_TFLOPs": round(tf, 2),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "tokens_per_s": round(int(sel.sum()) / (ms * 1e-3), 1)}


def bench_adaln(pa, spec, ids, dim=3072, iters=20):
    """Fused AdaLN forward and backward on the pack's rows (dim features, one
    modulation row per episode), with the unfused torch chain timed beside it."""
    import torch
    n = spec.nq
    dev = ids.device
    g = torch.Generator(device=dev).manual_seed(5)
    x = torch.randn((n, dim), generator=g, device=dev).to(torch.bfloat16)
    dy = torch.randn((n, dim), generator=g, device=dev).to(torch.bfloat16)
    S = spec.n_episodes
    shift = 0.5 * torch.randn((S, dim), generator=g, device=dev)
    scale = 0.5 * torch.randn((S, dim), generator=g, device=dev)
    per = spec.frames_padded * spec.q_tokens_per_frame
    off = (torch.arange(S + 1, device=dev, dtype=torch.int32) * per)
    y, mean, rstd = pa.adaln_fwd(x, ids, off, shift, scale)
    dx, dsh, dsc = pa.adaln_bwd(x, dy, ids, off, scale, mean, rstd)
    ws = torch.empty(pa.adaln_bwd_workspace_bytes(n, dim, S), dtype=torch.uint8, device=dev)
    fwd_ms = time_calls(lambda: pa.adaln_fwd(x, ids, off, shift, scale, out=(y, mean, rstd)),
                        iters)
    bwd_ms = time_calls(lambda: pa.adaln_bwd(x, dy, ids, off, scale, mean, rstd, ws,
                                             out=(dx, dsh, dsc)), iters)
    nv = int((ids >= 0).sum().item())
    # algorithmic bytes: fwd reads valid x rows, writes every y row and the row
    # statistics; bwd reads valid x, dy rows and their statistics, writes every
    # dx row and the two modulation-gradient tables; ids read once per pass
    fwd_bytes = 2 * dim * nv + 2 * dim * n + 8 * n + 4 * n + 8 * S * dim
    bwd_bytes = 2 * 2 * dim * nv + 8 * nv + 2 * dim * n + 4 * n + 2 * 4 * S * dim + 4 * S * dim

    seg = (torch.arange(n, device=dev) // per).clamp_max(S - 1)
    valid = (ids >= 0).to(torch.bfloat16)[:, None]
    xr = x.detach().clone().requires_grad_(True)
    shr, scr = shift.clone().requires_grad_(True), scale.clone().requires_grad_(True)

    def unfused():
        xn = torch.nn.functional.layer_norm(xr, (dim,), eps=1e-6)
        out = (xn * (1 + scr[seg]) + shr[seg]).to(torch.bfloat16) * valid
        out.backward(dy)
    unfused_ms = time_calls(unfused, max(iters // 4, 3))
    fused_ms = fwd_ms + bwd_ms
    return {"shape": f"{n} x {dim} bf16, {S} segments, {nv} valid rows",
            "fwd_ms": round(fwd_ms, 4), "fwd_GBs": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9, 1),
            "fwd_frac": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bwd_ms": round(bwd_ms, 4), "bwd_GBs": round(bwd_bytes / (bwd_ms * 1e-3) / 1e9, 1),
            "bwd_frac": round(bwd_bytes / (bwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "fwd_bytes": fwd_bytes, "bwd_bytes": bwd_bytes, "bound": "hbm",
            "fwd_traffic": measured_traffic("adaln_fwd", f"adaln-{n}x{dim}"),
            "bwd_traffic": measured_traffic("adaln_bwd", f"adaln-{n}x{dim}"),
            "peak_GBs": PEAK_HBM_GBS,
            "torch_unfused_fwd_bwd_ms": round(unfused_ms, 4),
            "speedup_vs_unfused": round(unfused_ms / fused_ms, 2)}


def bench_planner(pa, heads=24, head_dim=128, iters=3):
    """Fit step time ~ a + b*B*S^p of the packed attention fwd+bwd (ids, mask,
    forward, backward) to a scan of packs of B equal episodes of S tokens, then
    plan the 160-episode stream with fixed batches of 4 and with the dual
    constraint, and compare the spread of the predicted step times."""
    import numpy as np
    import torch

    import workloads as wl
    dev = torch.device("cuda:0")
    budget = wl.UNPADDED_BUDGET
    g = torch.Generator(device=dev).manual_seed(13)
    big = (0.5 * torch.randn((4, budget, heads, head_dim), generator=g, device=dev)).to(
        torch.bfloat16)
    shapes = [(B, S) for S in (2048, 4096, 8192, 12288, 16384) for B in (1, 2, 4, 8)
              if B * S <= budget]
    Bs, Ss, ts = [], [], []
    for B, S in shapes:
        n = B * S
        Q, K, V, DO = (big[j, :n] for j in range(4))
        vf = torch.full((B,), S // 32, dtype=torch.int32, device=dev)

        def step():
            ids = pa.seq_ids_from_valid_frames(vf, S // 32, 32)
            mask = pa.build_block_mask(ids, ids, 128, 128)
            o, lse = pa.attn_packed_fwd(Q, K, V, ids, ids, mask)
            pa.attn_packed_bwd(Q, K, V, o, DO, lse, ids, ids, mask)
        Bs.append(B)
        Ss.append(S)
        ts.append(time_calls(step, iters, warmup=1))
    a, b, p = pa.fit_step_cost(Bs, Ss, ts)
    pred = [a + b * B * S ** p for B, S in zip(Bs, Ss)]
    fit_err = max(abs(x - y) / y for x, y in zip(pred, ts))
    # plan the episode stream: fixed batches of 4 vs the dual constraint with
    # M_mem = the token budget and M_comp = 4 episodes of the median padded length
    frames = (wl.episode_stream() // 32).tolist()
    med = float(np.median([-(-f // 8) * 8 * 32 for f in frames]))
    dual = (float(budget), 4.0 * med ** p, p, 32)

    def cost_cov(batches, fpad):
        c = np.array([a + b * len(bt) * (f * 32) ** p for bt, f in zip(batches, fpad)])
        per_ep = c.sum() / sum(len(bt) for bt in batches)
        return float(c.std() / c.mean()), len(batches), float(per_ep)
    fixed = pa.length_bucket_batches(frames, 0, 0, 200, 8, 4)
    dualb = pa.length_bucket_batches(frames, 0, 0, 200, 8, 0, dual=dual)
    cf, nf, ef = cost_cov(*fixed)
    cd, nd, ed = cost_cov(*dualb)
    return {"scan": [{"B": B, "S": S, "ms": round(t, 4)} for B, S, t in zip(Bs, Ss, ts)],
            "fit": {"a_ms": round(a, 5), "b_ms": b, "p": round(p, 4),
                    "max_rel_err": round(fit_err, 4)},
            "plan_160_episodes": {
                "fixed_batch_4": {"batches": nf, "cost_cov": round(cf, 4),
                                  "pred_ms_per_episode": round(ef, 4)},
                "dual_constraint": {"batches": nd, "cost_cov": round(cd, 4),
                                    "pred_ms_per_episode": round(ed, 4),
                                    "m_mem_tokens": budget, "m_comp": dual[1]}}}


def run_extras(pa, spec, ids, extras):
    """The measurements of the loss, unpadded-pack, planner and AdaLN rows."""
    extras["masked_loss"] = r = bench_masked_loss(pa, ids)
    log(f"[bench] masked_loss: {r['avg_call_ms'] * 1e3:.1f} us, {r['achieved_GBs']} GB/s "
        f"({100 * r['frac']:.1f}% of HBM peak)")
    extras["unpadded_pack"] = r = bench_unpadded_pack(pa)
    log(f"[bench] unpadded pack: {r['ms_per_step']:.3f} ms, {r['useful_TFLOPs']} TFLOP/s useful")
    extras["planner"] = r = bench_planner(pa)
    log(f"[bench] planner fit a={r['fit']['a_ms']} ms p={r['fit']['p']} "
        f"(max rel err {r['fit']['max_rel_err']}); cost CoV fixed "
        f"{r['plan_160_episodes']['fixed_batch_4']['cost_cov']} -> dual "
        f"{r['plan_160_episodes']['dual_constraint']['cost_cov']}")
    extras["adaln"] = r = bench_adaln(pa, spec, ids)
    log(f"[bench] adaln fwd {r['fwd_ms'] * 1e3:.1f} us {r['fwd_GBs']} GB/s, "
        f"bwd {r['bwd_ms'] * 1e3:.1f} us {r['bwd_GBs']} GB/s; "
        f"unfused torch fwd+bwd {r['torch_unfused_fwd_bwd_ms']:.3f} ms "
        f"({r['speedup_vs_unfused']}x)")


def _useful_pairs(q_ids, kv_ids):
    """Allowed (query, key) pairs per head: for every id e >= 0, n_q(e) * n_kv(e)
    (bench accounting of the useful work, from the ids the step built)."""
    import numpy as np
    qv, kv = q_ids[q_ids >= 0], kv_ids[kv_ids >= 0]
    if qv.size == 0 or kv.size == 0:
        return 0
    m = int(max(qv.max(), kv.max())) + 1
    return int((np.bincount(qv, minlength=m).astype(np.int64) *
                np.bincount(kv, minlength=m).astype(np.int64)).sum())


STAGES = ["seq_ids", "block_mask", "fwd", "bwd_dq", "bwd_dkdv"]  # bwd_dq includes the row terms


class PackStep:
    """One pass of the hot path over one pack: ids (from valid frames; given
    directly for a pack of segment ids), block mask, forward, backward
    preprocess, dQ, dK/dV.  Inputs are prefixes of caller buffers resident in HBM;
    every output buffer is allocated here once."""

    def __init__(self, pa, spec, Q, K, V, DO):
        import torch
        self.pa, self.spec = pa, spec
        dev = Q.device
        self.Q, self.K, self.V, self.DO = Q[:spec.nq], K[:spec.nkv], V[:spec.nkv], DO[:spec.nq]
        nq, nkv, H, d = spec.nq, spec.nkv, spec.heads, spec.head_dim
        if spec.segment_ids is not None:
            self.vf = None
            ids = torch.from_numpy(spec.segment_ids).to(dev)
            self.qids, self.kids = ids, ids
        else:
            self.vf = torch.from_numpy(spec.valid_frames).to(dev)
            self.qids = torch.empty(nq, dtype=torch.int32, device=dev)
            self.kids = (self.qids if not spec.cross else
                         torch.empty(nkv, dtype=torch.int32, device=dev))
        self.O, self.dQ = torch.empty_like(self.Q), torch.empty_like(self.Q)
        self.dK, self.dV = torch.empty_like(self.K), torch.empty_like(self.V)
        self.lse = torch.empty((H, nq), dtype=torch.float32, device=dev)
        self.ws = torch.empty(pa.attn_packed_bwd_workspace_bytes(torch.bfloat16, nq, nkv, H, d),
                              dtype=torch.uint8, device=dev)
        self.mstore = torch.empty(pa.build_block_mask_bytes(nq, nkv, 128, 128),
                                  dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.mask = None

    def ids(self):
        s = self.spec
        if self.vf is not None:
            self.pa.seq_ids_from_valid_frames(self.vf, s.frames_padded, s.q_tokens_per_frame,
                                              out=self.qids)
            if s.cross:
                self.pa.seq_ids_from_valid_frames(self.vf, s.frames_padded,
                                                  s.kv_tokens_per_frame, out=self.kids)

    def build_mask(self):
        self.mask = self.pa.build_block_mask(self.qids, self.kids, 128, 128, storage=self.mstore)
        return self.mask

    def __call__(self, ev=None):
        pa, s = self.pa, self.spec

        def mark(i):
            if ev is not None:
                ev[i].record(self.stream)
        mark(0)
        self.ids()
        mark(1)
        mask = self.build_mask()
        mark(2)
        pa.attn_packed_fwd(self.Q, self.K, self.V, self.qids, self.kids, mask, s.scale,
                           out=self.O, lse=self.lse)
        mark(3)
        pa.attn_packed_bwd_dq(self.Q, self.K, self.V, self.O, self.DO, self.lse, self.ws,
                              self.qids, self.kids, mask, s.scale, dq=self.dQ)
        mark(4)
        pa.attn_packed_bwd_dkdv(self.Q, self.K, self.V, self.DO, self.lse, self.ws, self.qids,
                                self.kids, mask, s.scale, dk=self.dK, dv=self.dV)
        mark(5)

    def pairs(self):
        import torch
        torch.cuda.synchronize()
        return _useful_pairs(self.qids.cpu().numpy(), self.kids.cpu().numpy())


def time_steps(step, iters):
    """(mean ms per step, mean ms per stage) from HIP events on the library's stream."""
    import numpy as np
    import torch
    ne = len(STAGES) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ne)] for _ in range(iters)]
    torch.cuda.synchronize()
    for i in range(iters):
        step(evs[i])
    torch.cuda.synchronize()
    stage = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
             for j, n in enumerate(STAGES)}
    total = float(np.mean([e[0].elapsed_time(e[ne - 1]) for e in evs]))
    return total, stage


def device_values(n_q, n_kv, heads, head_dim, seed, dev):
    """Timing-only inputs drawn on the device: q, k, v ~ N(0,1)*0.5, dO ~ N(0,1), bf16
    (the distribution of the seeded packs; the parity tests use the host draws)."""
    import torch
    g = torch.Generator(device=dev).manual_seed(seed)
    mk = lambda n, sd: (sd * torch.randn((n, heads, head_dim), generator=g,  # noqa: E731
                                         device=dev)).to(torch.bfloat16)
    return mk(n_q, 0.5), mk(n_kv, 0.5), mk(n_kv, 0.5), mk(n_q, 1.0)


def bench_pack_list(pa, specs, name, iters=5, warmup=1, seed=21):
    """fwd+bwd of every pack in `specs` (one after the other, like the batches of
    an epoch): summed time, summed useful flops, per-stage sums."""
    import torch
    dev = torch.device("cuda:0")
    H, d = specs[0].heads, specs[0].head_dim
    vals = device_values(max(s.nq for s in specs), max(s.nkv for s in specs), H, d, seed, dev)
    total_ms, stages, pairs, tokens_q = 0.0, {n: 0.0 for n in STAGES}, 0, 0
    for s in specs:
        step = PackStep(pa, s, *vals)
        for _ in range(warmup):
            step()
        ms, st = time_steps(step, iters)
        total_ms += ms
        for n in STAGES:
            stages[n] += st[n]
        pairs += step.pairs()
        tokens_q += s.nq
        del step
    useful = 14.0 * d * pairs * H
    tf = useful / (total_ms * 1e-3) / 1e12
    return {"workload": name, "packs": len(specs), "query_tokens": tokens_q,
            "valid_pairs_per_head": pairs, "useful_flops": useful, "ms": round(total_ms, 4),
            "useful_TFLOPs": round(tf, 2), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "useful_TFLOPs_12dPH": round(tf * 12 / 14, 2),
            "stages_ms": {n: round(v, 4) for n, v in stages.items()}}


def mask_builder_bytes(nq, nkv, nnz, bq=128, bkv=128):
    """Algorithmic HBM bytes of one block-mask build: the two id arrays read, the
    class matrix (one byte per tile pair), both CSR lists (nnz entries each), their
    row pointers and the two longest-first orders written."""
    tq, tk = -(-nq // bq), -(-nkv // bkv)
    return 4 * (nq + nkv) + tq * tk + 4 * 2 * nnz + 4 * (tq + tk + 2) + 4 * (tq + tk)


def bench_mask_builder(pa, name, q_ids, kv_ids, iters=20):
    """block_mask build alone: event-timed average and GB/s of its algorithmic bytes."""
    import torch
    nq, nkv = q_ids.numel(), kv_ids.numel()
    store = torch.empty(pa.build_block_mask_bytes(nq, nkv, 128, 128), dtype=torch.uint8,
                        device=q_ids.device)
    ms = time_calls(lambda: pa.build_block_mask(q_ids, kv_ids, 128, 128, storage=store), iters)
    mask = pa.build_block_mask(q_ids, kv_ids, 128, 128, storage=store)
    nnz = int(mask.csr()[0][-1].item())
    nbytes = mask_builder_bytes(nq, nkv, nnz)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": name, "tokens": nq, "tiles": mask.nq_tiles * mask.nkv_tiles,
            "nonempty_tiles": nnz, "avg_call_ms": round(ms, 5), "algorithmic_bytes": nbytes,
            "achieved_GBs": round(gbs, 1), "peak_GBs": PEAK_HBM_GBS,
            "frac": round(gbs / PEAK_HBM_GBS, 5), "bound": "hbm (launch-latency at these sizes)"}


def stress_ids(n=1 << 20, seg=4096):
    """Ids of the mask-builder stress case: n tokens in consecutive segments of seg."""
    import numpy as np
    return (np.arange(n, dtype=np.int64) // seg).astype(np.int32)


def run_configs(pa, configs, extras_out):
    """The other workloads, each as whole fwd+bwd passes (summed over the packs
    of the bucketed sweep), and the mask builder's GB/s."""
    import torch

    import workloads as wl
    dev = torch.device("cuda:0")
    out = {}
    for c in configs:
        if c == "2":
            out[c] = r = bench_pack_list(pa, [wl.config(2)], "equal-4x120")
        elif c == "4self":
            out[c] = r = bench_pack_list(pa, wl.bucketed_sweep(), "bucketed sweep, 40 batches")
        elif c == "4cross":
            out[c] = r = bench_pack_list(pa, wl.bucketed_sweep(cross=True),
                                         "bucketed sweep, cross (6 action -> 32 video tok/frame)")
        elif c == "5":
            out[c] = r = bench_pack_list(pa, [wl.config(5)], "long-64k (ids given)")
        elif c == "3":
            out[c] = r = bench_pack_list(pa, [wl.config(3)], "var-4x288 (values drawn on the "
                                         "device like the other configs)")
        elif c == "scatter":
            out[c] = r = bench_pack_list(pa, [wl.scattered_pack()],
                                         "var-4x288 in permuted 512-token pieces (ids given)")
        elif c == "mask":
            continue  # the block-mask builder alone, below
        else:
            raise SystemExit(f"unknown config {c}")
        log(f"[bench] config {c}: {r['ms']:.3f} ms, {r['useful_TFLOPs']} TFLOP/s useful "
            f"({100 * r['frac_of_bf16_peak']:.1f}% of bf16 peak)")
    extras_out["configs"] = out
    if "mask" not in configs:
        return
    mb = {}
    s3 = wl.config(3)
    vf = torch.from_numpy(s3.valid_frames).to(dev)
    ids3 = pa.seq_ids_from_valid_frames(vf, s3.frames_padded, s3.q_tokens_per_frame)
    mb["3"] = bench_mask_builder(pa, "var-4x288", ids3, ids3)
    ids5 = torch.from_numpy(wl.config(5).segment_ids).to(dev)
    mb["5"] = bench_mask_builder(pa, "long-64k", ids5, ids5)
    idss = torch.from_numpy(stress_ids()).to(dev)
    mb["stress"] = bench_mask_builder(pa, "1,048,576 tokens in 4,096-token segments", idss, idss)
    for k, r in mb.items():
        log(f"[bench] mask builder {k}: {r['avg_call_ms'] * 1e3:.1f} us, "
            f"{r['achieved_GBs']} GB/s of {r['algorithmic_bytes']} algorithmic bytes")
    extras_out["mask_builder"] = mb


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3,
                    help="workload of the timed steps (3 = the metric; 2 and 5 also run)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=str, default="all",
                    help="heads the oracle baseline computes ('all' or a list like 0,23)")
    ap.add_argument("--configs", type=str, default="2,3,4self,4cross,5,scatter,mask",
                    help="other workloads measured after the timed steps ('' for none; "
                         "'mask' = the block-mask builder alone)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the loss / unpadded-pack / planner / AdaLN measurements")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the packed path shards by whole packs, one per GPU, with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import packed_variable_length_amd as pa
    import workloads as wl

    spec = wl.config(args.config)
    assert spec.dtype == "bf16" and args.config in (2, 3, 5), "timed workload: 2, 3 or 5"
    log(f"[bench] workload {spec.name}: nq={spec.nq} heads={spec.heads} d={spec.head_dim}")
    q, k, v, do = wl.make_values(spec)
    dev = torch.device("cuda:0")
    T = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)  # noqa: E731
    step = PackStep(pa, spec, T(q), T(k), T(v), T(do))
    H, d, nq = spec.heads, spec.head_dim, spec.nq

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {n} bytes done")
        del src, dst
    pairs = step.pairs()
    useful = 14.0 * d * pairs * H

    # timed region: wall clock around exactly `steps` steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    # per-stage HIP events over a second pass of the same steps
    _, stage_ms = time_steps(step, args.steps)
    for n in STAGES:
        log(f"[bench] {n:10s} {stage_ms[n]:8.3f} ms")
    tflops = useful / wall / 1e12
    log(f"[bench] step {wall * 1e3:.3f} ms  useful {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak; "
        f"{tflops * 12 / 14:.1f} TFLOP/s counting 12*d*P*H, without the recompute)")

    kernels = {n: stage_ms[n] for n in FLOPS_PER_PAIR}
    dom = max(kernels, key=kernels.get)
    achieved = FLOPS_PER_PAIR[dom] * d * pairs * H / (kernels[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": {"fwd": "fwd_bf16_pair_kernel<128>",
                                            "bwd_dq": "dq_bf16_pair_kernel<128>",
                                            "bwd_dkdv": "dkdv_bf16_split_kernel<128>"}[dom],
                "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom, spec.name),
                "flops_per_launch": FLOPS_PER_PAIR[dom] * d * pairs * H,
                "avg_launch_ms": round(kernels[dom], 4),
                "source_sha256": source_sha256(dom)}
    per_kernel = {n: {"ms": round(kernels[n], 4),
                      "achieved_TFLOPs": round(FLOPS_PER_PAIR[n] * d * pairs * H
                                               / (kernels[n] * 1e-3) / 1e12, 2)}
                  for n in FLOPS_PER_PAIR}
    del step

    extras = {}
    cfgs = [c for c in args.configs.split(",") if c]
    if cfgs:
        run_configs(pa, cfgs, extras)
    if not args.no_extras:
        s3 = wl.config(3)
        ids3 = pa.seq_ids_from_valid_frames(torch.from_numpy(s3.valid_frames).to(dev),
                                            s3.frames_padded, s3.q_tokens_per_frame)
        run_extras(pa, s3, ids3, extras)

    cpu = None
    if not args.no_cpu_baseline:
        heads = (list(range(spec.heads)) if args.cpu_heads == "all"
                 else [int(x) for x in args.cpu_heads.split(",")])
        log(f"[bench] cpu baseline: oracle on heads {heads} ...")
        cpu = cpu_baseline(spec, q, k, v, do, heads)
        log(f"[bench] cpu baseline {cpu['value']:.4f} TFLOP/s in {cpu['seconds']} s")

    if spec.segment_ids is not None:
        wdesc = f"{spec.name}: {nq} tokens with given segment ids, {H} heads x {d}"
    else:
        wdesc = (f"{spec.name}: {spec.n_episodes} episodes of "
                 f"{'/'.join(str(int(x)) for x in spec.valid_frames)} valid frames padded to "
                 f"{spec.frames_padded}, 32 tokens/frame, {nq} tokens, {H} heads x {d}")
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*0.5 bf16; stands in for FurnitureBench episodes)",
        "config": {"workload": wdesc, "tokens": nq, "heads": H, "head_dim": d,
                   "valid_pairs_per_head": pairs, "useful_flops": useful,
                   "parallelism": "single GPU"},
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "value_12dPH": round(tflops * 12 / 14, 2),
        "stages_ms": {n: round(stage_ms[n], 4) for n in STAGES},
        "kernels": per_kernel,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
