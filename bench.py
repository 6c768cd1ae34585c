#!/usr/bin/env python3
"""Throughput of the causal GQA / paged-KV / MLA attention path on one MI355X.

One step is one pass of the whole hot path over seeded synthetic inputs that
are already resident in HBM, push then attend:
  1. push (kv_append) of this step's K/V row of the 64 decode sequences into
     their paged pool, at position seq_len - 1 (the same row every step);
  2. paged GQA decode, bf16: 64 sequences, lengths uniform on [512, 8192],
     H=32, Hkv=8, D=128, block size 16, shuffled block tables over a pool
     with 10% slack (attn_decode_paged: split-K partial + combine);
  3. the same decode with a layer's arms (attn_decode_paged_ext: window 4096,
     logit softcap 30, ALiBi slopes, sink logits);
  4. MLA step, bf16, 32 sequences x 4096 tokens, 128 heads, latent 512 + 64:
     absorb (mla_absorb_q), push of the latent row with k_rot rotated
     (mla_append_latent), latent attention (mla_decode_latent), value
     up-projection (mla_up_proj); then the latent attention over a paged
     copy of the latent (mla_decode_latent_paged, block size 16);
  5. chunked prefill on paged K/V, bf16: 8 sequences, 3584 cached + 512 new,
     H=32, Hkv=8, scale 0.05 (attn_prefill, paged);
  6. ragged chunked prefill on one paged pool, bf16: 16 sequences with chunks
     U[1, 1024] after U[0, 4096] cached tokens (attn_prefill_varlen);
  7. causal prefill, bf16: B=1, H=28, Hkv=4, D=128, 4096 tokens (attn_prefill).
The order lets the 1.16 GB decode streams evict the 256 MB Infinity Cache
before the workloads whose data would otherwise fit in it.

The headline value is the paged decode's algorithmic HBM bandwidth (each K/V
byte once, plus Q, O and the block-table entries read) over the duration of
its call, timed with HIP events on the launch stream; the causal prefill's
TFLOP/s (causal pairs only) is reported next to it, as is the roofline of
every call. The CPU baseline times the f64 oracle on a bounded sample.
Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense bf16 MFMA
METRIC = "paged GQA decode HBM GB/s (% peak); causal prefill TFLOP/s (% MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "decode": ["decode.hip", "common.hpp"],
    "prefill": ["prefill.hip", "common.hpp"],
    "mla": ["mla.hip", "common.hpp"],
    "append": ["append.hip", "common.hpp"],
    "mla_proj": ["mla_proj.hip", "common.hpp"],
}
WORKLOADS = ["append", "decode", "decode_arms", "mla_absorb", "mla_append", "mla", "mla_up",
             "mla_paged", "chunked", "varlen", "prefill"]


def source_digest(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "paged_kv_attention_causal_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kind):
    """HBM bytes per launch of one workload from committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, each scaled by its plain-copy calibration), or None
    when the kernel source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[workload]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_digest") != source_digest(kind):
        return None
    return t.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the f64 oracle on the host")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU work budget of the oracle sample")
    ap.add_argument("--only", choices=WORKLOADS + ["copy"], default=None,
                    help="time one workload only (for profiler runs; the decode arms and the "
                         "push share the decode inputs, the MLA pieces the MLA inputs); 'copy' "
                         "runs a plain 1 GiB device copy three times, the calibration for the "
                         "FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_attention_causal_amd as pk
    from paged_kv_attention_causal_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    pk.lib()  # fail loudly here if the HIP library is missing
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.only == "copy":
        x = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)   # exactly 1 GiB
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": x.numel() * 2, "launches": 3}))
        return

    def to(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(dev)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    want = (lambda *ks: args.only is None or args.only in ks)
    work = {}

    def add(name, fn, nbytes, flops, bound, kind, kernel):
        work[name] = dict(fn=fn, bytes=int(nbytes), flops=int(flops), bound=bound, kind=kind,
                          kernel=kernel)

    # ---- 1-3. push, paged decode, decode with arms
    d_case = None
    if want("append", "decode", "decode_arms"):
        d = inputs.paged_decode_case(args.seed)
        dq, dk, dv = to(d.q), to(d.k_pool), to(d.v_pool)
        dbt, dl = i32(d.block_table), i32(d.seq_lens)
        dmax = int(d.block_table.shape[1] * d.block_size)
        dws = torch.empty(pk.attn_decode_workspace_size(64, 32, 8, 128, dmax), dtype=torch.uint8,
                          device=dev)
        dout = torch.empty_like(dq)
        total = int(d.seq_lens.sum())
        blocks = int(((d.seq_lens + 15) // 16).sum())
        kv_bytes = total * 8 * 128 * 2 * 2
        q_o = 2 * dq.numel() * 2
        if want("append"):
            rng = np.random.default_rng(args.seed + 100)
            kn = to(inputs.to_storage(rng.standard_normal((64, 1, 8, 128), dtype=np.float32), "bf16"))
            vn = to(inputs.to_storage(rng.standard_normal((64, 1, 8, 128), dtype=np.float32), "bf16"))
            pos = i32(d.seq_lens - 1)      # this step's row: the last of each sequence
            add("append", lambda: pk.kv_append(kn, vn, dk, dv, pos, block_table=dbt),
                64 * 8 * 128 * 2 * 2 * 2 + 64 * 4 * 2, 0, "hbm", "append", "kv_append_kernel")
        if want("decode"):
            add("decode", lambda: pk.attn_decode_paged(dq, dk, dv, dbt, dl, max_seq_len=dmax,
                                                       attention_scale=d.scale, out=dout,
                                                       workspace=dws),
                kv_bytes + q_o + blocks * 4 + 64 * 4, 4 * 32 * 128 * total, "hbm", "decode",
                "decode_partial + decode_combine")
            d_case = d
        if want("decode_arms"):
            slopes, sinks = f32(inputs.alibi_slopes(32)), f32(inputs.sink_logits(args.seed, 32))
            eff = np.minimum(d.seq_lens, 4096)
            e_tot = int(eff.sum())
            add("decode_arms",
                lambda: pk.attn_decode_paged_ext(dq, dk, dv, dbt, dl, max_seq_len=dmax,
                                                 attention_scale=d.scale, window=4096,
                                                 softcap=30.0, alibi=slopes, sinks=sinks,
                                                 out=dout, workspace=dws),
                e_tot * 8 * 128 * 2 * 2 + q_o + int(((eff + 15) // 16).sum()) * 4 + 64 * 4 +
                2 * 32 * 4, 4 * 32 * 128 * e_tot, "hbm", "decode",
                "decode_partial<ext> + decode_combine<ext>")

    # ---- 4. MLA step
    if want("mla_absorb", "mla_append", "mla", "mla_up", "mla_paged"):
        m = inputs.mla_case(args.seed)
        mq, ml, mlens = to(m.q_abs), to(m.latent), i32(m.seq_lens)
        mout = torch.empty((32, 128, 512), dtype=torch.bfloat16, device=dev)
        mws = torch.empty(max(16, pk.mla_decode_workspace_size(32, 128, 512, 4096)),
                          dtype=torch.uint8, device=dev)
        lat_bytes = 32 * 4096 * 576 * 2
        if want("mla_absorb", "mla_up"):
            w = inputs.mla_proj_case(args.seed)
            wq, wkb, wvb = to(w.q), to(w.k_b), to(w.v_b)
            wup = torch.empty((32, 128, 128), dtype=torch.bfloat16, device=dev)
            proj_flops = 2 * 32 * 128 * 512 * 128
            if want("mla_absorb"):
                add("mla_absorb", lambda: pk.mla_absorb_q(wq, wkb, out=mq),
                    wkb.numel() * 2 + wq.numel() * 2 + mq.numel() * 2, proj_flops, "hbm",
                    "mla_proj", "mla_proj_kernel (absorb)")
        if want("mla_append"):
            a = inputs.mla_append_case(args.seed + 1, batch=1, held=[0])
            cn = to(np.repeat(a.c_new, 32, axis=0))
            kr = to(np.repeat(a.k_rot_new, 32, axis=0))
            mpos = i32(m.seq_lens - 1)
            add("mla_append", lambda: pk.mla_append_latent(cn, kr, ml, mpos, rope_theta=1e4),
                32 * 576 * 2 * 2 + 32 * 4, 0, "hbm", "append", "mla_append_kernel")
        if want("mla"):
            add("mla", lambda: pk.mla_decode_latent(mq, ml, mlens, kv_lora_rank=512,
                                                    max_seq_len=4096, attention_scale=m.scale,
                                                    out=mout, workspace=mws),
                lat_bytes + mq.numel() * 2 + mout.numel() * 2 + 32 * 4,
                32 * 128 * 4096 * (2 * 576 + 2 * 512), "hbm", "mla", "mla_kernel + mla_combine")
        if want("mla_up"):
            add("mla_up", lambda: pk.mla_up_proj(mout, wvb, out=wup),
                wvb.numel() * 2 + mout.numel() * 2 + wup.numel() * 2, proj_flops, "hbm",
                "mla_proj", "mla_proj_kernel (up-projection)")
        if want("mla_paged"):
            rng = np.random.default_rng(args.seed + 7)
            nblk = 32 * 4096 // 16
            perm = rng.permutation(nblk + nblk // 10)
            mbt = perm[:nblk].reshape(32, 256).astype(np.int32)
            pool = torch.empty((nblk + nblk // 10, 16, 576), dtype=torch.bfloat16, device=dev)
            pool[torch.from_numpy(mbt.reshape(-1)).long().to(dev)] = ml.reshape(nblk, 16, 576)
            mbt_d = i32(mbt)
            mpout = torch.empty_like(mout)
            add("mla_paged", lambda: pk.mla_decode_latent_paged(mq, pool, mbt_d, mlens,
                                                                kv_lora_rank=512, max_seq_len=4096,
                                                                attention_scale=m.scale, out=mpout,
                                                                workspace=mws),
                lat_bytes + mq.numel() * 2 + mout.numel() * 2 + 32 * 4 + nblk * 4,
                32 * 128 * 4096 * (2 * 576 + 2 * 512), "hbm", "mla",
                "mla_kernel<paged> + mla_combine")
        m.latent = m.q_abs = None

    # ---- 5. chunked prefill on paged K/V
    if want("chunked"):
        c = inputs.chunked_paged_prefill_case(args.seed)
        cq, ck, cv, cbt = to(c.q), to(c.k), to(c.v), i32(c.block_table)
        cout = torch.empty_like(cq)
        pairs = sum(c.position_offset + i + 1 for i in range(c.seq_q)) * c.batch
        add("chunked", lambda: pk.attn_prefill(cq, ck, cv, seq_kv=c.seq_kv,
                                               position_offset=c.position_offset,
                                               attention_scale=c.scale, block_table=cbt, out=cout),
            (c.batch * c.seq_kv * 8 * 128 * 2 * 2) + 2 * cq.numel() * 2, 4 * 128 * 32 * pairs,
            "mfma", "prefill", "prefill_kernel")
        c.q = c.k = c.v = None

    # ---- 6. ragged chunked prefill
    if want("varlen"):
        r = inputs.varlen_prefill_case(args.seed)
        rq, rk, rv, rbt = to(r.q), to(r.k), to(r.v), i32(r.block_table)
        rcu, rkv = i32(r.cu_q), i32(r.seq_kv)
        rout = torch.empty_like(rq)
        rmax = int(r.q_lens.max())
        pairs = sum(int(r.seq_kv[b] - r.q_lens[b]) * int(r.q_lens[b]) +
                    int(r.q_lens[b]) * (int(r.q_lens[b]) + 1) // 2 for b in range(r.batch))
        add("varlen", lambda: pk.attn_prefill_varlen(rq, rk, rv, rcu, rkv, max_seq_q=rmax,
                                                     attention_scale=r.scale, block_table=rbt,
                                                     out=rout),
            int(r.seq_kv.sum()) * 8 * 128 * 2 * 2 + 2 * rq.numel() * 2, 4 * 128 * 32 * pairs,
            "mfma", "prefill", "prefill_kernel<varlen>")
        r.q = r.k = r.v = None

    # ---- 7. causal prefill
    if want("prefill"):
        p = inputs.prefill_case(args.seed)
        pq, pk_, pv = to(p.q), to(p.k), to(p.v)
        pout = torch.empty_like(pq)
        add("prefill", lambda: pk.attn_prefill(pq, pk_, pv, seq_kv=p.seq_kv, position_offset=0,
                                               attention_scale=p.scale, out=pout),
            pq.numel() * 2 * 2 + pk_.numel() * 2 * 2, 4 * 128 * 28 * (4096 * 4097 // 2), "mfma",
            "prefill", "prefill_kernel")
        p.q = p.k = p.v = None

    order = [k for k in WORKLOADS if k in work]
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        for k in order:
            if events is not None:
                events[k][0].record(stream)
            work[k]["fn"]()
            if events is not None:
                events[k][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [{k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for k in order} for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    res = {}
    for k in order:
        ts = np.array([evs[s][k][0].elapsed_time(evs[s][k][1]) for s in range(args.steps)]) * 1e-3
        w = work[k]
        avg = float(ts.mean())
        res[k] = dict(us_avg=avg * 1e6, us_min=float(ts.min()) * 1e6,
                      us_median=float(np.median(ts)) * 1e6,
                      gbps=w["bytes"] / avg / 1e9, tflops=w["flops"] / avg / 1e12)

    def roofline(k):
        w, r = work[k], res[k]
        if w["bound"] == "hbm":
            ach, peak, unit = w["bytes"] / (r["us_avg"] * 1e-6) / 1e9, HBM_PEAK / 1e9, "GB/s"
        else:
            ach, peak, unit = w["flops"] / (r["us_avg"] * 1e-6) / 1e12, MFMA_BF16_PEAK / 1e12, "TFLOP/s"
        return {"bound": w["bound"], "achieved": round(ach, 2), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": measured_traffic(k, w["kind"]),
                "kernel": w["kernel"], "us_per_launch": round(r["us_avg"], 2),
                "algorithmic_bytes": w["bytes"], "algorithmic_flops": w["flops"]}

    line = {"metric": METRIC, "unit": "GB/s", "higher_is_better": True, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "paged GQA decode bf16 (64 seqs, seq_lens U[512,8192], H=32 Hkv=8 "
                                   "D=128, block 16) with its K/V push and an arms variant + MLA "
                                   "step bf16 (32x4096, H=128, 512+64: absorb, latent push, latent "
                                   "decode contiguous and paged, up-projection) + chunked paged "
                                   "prefill bf16 (8 x (3584+512), H=32 Hkv=8) + ragged paged "
                                   "prefill bf16 (16 seqs) + causal prefill bf16 (B=1 S=4096 H=28 "
                                   "Hkv=4 D=128)",
                       "seed": args.seed, "parallelism": "single GPU"}}
    if "decode" in res:
        line["value"] = round(res["decode"]["gbps"], 2)
        line["roofline"] = roofline("decode")
    elif order:
        k0 = order[0]
        line["value"] = round(res[k0]["gbps"] if work[k0]["bound"] == "hbm" else res[k0]["tflops"], 2)
        line["unit"] = "GB/s" if work[k0]["bound"] == "hbm" else "TFLOP/s"
        line["roofline"] = roofline(k0)
    if "prefill" in res:
        line["prefill_tflops"] = round(res["prefill"]["tflops"], 2)
        line["prefill_frac_mfma_peak"] = round(res["prefill"]["tflops"] * 1e12 / MFMA_BF16_PEAK, 4)
    line["rooflines"] = {k: roofline(k) for k in order}
    line["kernels"] = {k: {kk: round(vv, 3) for kk, vv in res[k].items()} for k in order}

    # ---- CPU baseline: the f64 oracle on a bounded sample of the paged decode
    if not args.no_cpu_baseline and d_case is not None:
        line["cpu_baseline"] = cpu_baseline(d_case, args.cpu_seconds, args.seed)
    print(json.dumps(line), flush=True)


def cpu_baseline(d, budget_s, seed):
    import numpy as np
    from oracle import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    t0 = time.perf_counter()
    done, toks = 0, 0
    while done < d.batch and time.perf_counter() - t0 < budget_s:
        O.decode_paged(d.q, d.k_pool, d.v_pool, d.block_table, d.block_size, d.seq_lens,
                       d.n_heads, d.n_kv_heads, d.scale, batch_indices=[done])
        toks += int(d.seq_lens[done])
        done += 1
    el = time.perf_counter() - t0
    nbytes = toks * 8 * 128 * 2 * 2 + done * 2 * 32 * 128 * 2
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"f64 oracle decode_paged on the first {done} of 64 sequences "
                      f"({toks} tokens) of the seed-{seed} paged decode draw, {el:.1f} s"}


if __name__ == "__main__":
    main()
