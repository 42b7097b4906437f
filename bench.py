#!/usr/bin/env python3
"""Benchmark of the grouped MoE backward GEMMs on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic
inputs already resident in HBM:

  dswiglu       gg_dglu,   dSwiGLU, L 8,  K 2048, N 1024, M 16384, dense B
  wgrad_moe     gg_wgrad,  hidden 4096, intermediate 2048, 64 experts,
                           65536 tokens (Zipf 1.2), A M-major, B N-major,
                           bf16 dense output, overwrite
  dgeglu        gg_dglu,   dGeGLU, L 32, K 4096, N 1536, M 32768,
                           discrete K-major B, dbias
  dsrelu_mxfp8  gg_dsrelu, MXFP8, L 16, K 7168, N 2048, M 65536, dense B

and, as single-op workloads outside the default step:

  dglu_mxfp8    gg_dglu_mx, MXFP8 dSwiGLU with amax, L 32, K 4096, N 1536,
                M 32768, discrete B (b_ptrs / sfb_ptrs)
  wgrad_mxfp8   gg_wgrad_mx, the wgrad_moe shape on MXFP8 K-major operands,
                bf16 dense output, overwrite
  dsrelu_mxfp8_fp8out, dglu_mxfp8_fp8out
                the two block-scaled dgrad workloads with FP8 (E4M3) D_row
                and D_col and their E8M0 scales instead of a bf16 D
  dsrelu_mxfp8_nmajor  the dsReLU workload with discrete N-major B
  wgrad_moe_kmajor  the wgrad workload with A K-major
  wgrad_moe_f32acc  the wgrad workload into discrete per-expert fp32
                outputs (int64 pointer array), accumulate mode: the
                variant whose roofline is HBM (old outputs read and
                written back), reported in GB/s against the HBM peak

value = algorithmic FLOPs of the step (2 sum_e M_e N_e K_e per GEMM) over the
measured wall time of K steps.  Every call is also bracketed by HIP events on
the stream it runs on, which gives each kernel's average duration; the kernel
with the largest share is reported against its roofline: MFMA, or HBM when
its algorithmic bytes at 8 TB/s take longer than its FLOPs at the MFMA
peak.  The CPU oracle is timed on a bounded sample of rows of the same
workloads (cpu_baseline).

After the step, every op is launched --reps times on its own, back to back
("warm") and with a 512 MiB read-modify-write before each launch that evicts
the 256 MB MALL ("cold"); the median, p10 and p90 of its HIP-event durations
go into its `kernels` entry, with the median engine clock (amdsmi GPU
metrics, mean over the XCDs) over a further 0.4 s of back-to-back
launches.  With the default workload the MoE wgrad's other modes
(A K-major; bf16 and fp32-discrete accumulate) are timed the same way
beside the step.  Inside the step every op reads and writes 0.2-4.7 GB
between two launches of the same op, more than the MALL holds, so the
step's own launches are cold as well.

`measured_peaks` holds this GPU's sustained dense MFMA rates (bf16 and
MXFP8 probe kernels with no memory traffic, and the engine clock under
them) and its device-to-device copy rate; every `kernels` entry gives its
fraction of the measured MFMA peak and of the roofline built from the
measured peaks, beside the published ones.  `cpu_baseline.per_core` is
the oracle on one thread over the small wgrad workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--reps R]
                  [--no-extras] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "fp8": 5000.0}        # MI355X dense MFMA, TFLOP/s
HBM_PEAK = 8000.0                              # GB/s
# The sources each kernel's code is compiled from (with the build flags of
# build.py): the HBM traffic recorded for a kernel is reported only while
# their hash is unchanged.
KERNEL_SOURCES = {
    "wgrad_kernel": ["gg_internal.hpp", "gg_tile.hpp", "gg_wgrad_epi.hpp", "gg_wgrad.hip"],
    "dglu_kernel": ["gg_internal.hpp", "gg_tile.hpp", "gg_fp8out.hpp", "gg_dglu_epi.hpp",
                    "gg_dglu.hip"],
    "dglu_mx_kernel": ["gg_internal.hpp", "gg_tile.hpp", "gg_mx.hpp", "gg_fp8out.hpp",
                       "gg_dglu_epi.hpp", "gg_dglu_mx.hpp", "gg_dglu_mx_inst.hip"],
    "dsrelu_kernel": ["gg_internal.hpp", "gg_tile.hpp", "gg_mx.hpp", "gg_fp8out.hpp",
                      "gg_dsrelu.hpp", "gg_dsrelu_inst.hip"],
    "wgrad_mx_kernel": ["gg_internal.hpp", "gg_tile.hpp", "gg_mx.hpp", "gg_wgrad_epi.hpp",
                        "gg_wgrad_mx.hip"],
}


def source_hash(kernel):
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "moe_grouped_gemm_offset_amd")
    for f in [os.path.join("csrc", x) for x in KERNEL_SOURCES[kernel]] + ["build.py"]:
        with open(os.path.join(pkg, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class Op:
    """One grouped-GEMM call of the step: inputs on the device and a run()."""

    def __init__(self, name, kernel, flops, dtype, run, alg_bytes, oracle_sample):
        self.name, self.kernel, self.flops, self.dtype = name, kernel, flops, dtype
        self.run, self.alg_bytes, self.oracle_sample = run, alg_bytes, oracle_sample


def _cpu(d):
    import torch
    out = {}
    for k, v in d.items():
        if isinstance(v, torch.Tensor):
            out[k] = v.cpu()
        elif isinstance(v, list) and v and isinstance(v[0], torch.Tensor):
            out[k] = [x.cpu() for x in v]
        else:
            out[k] = v
    return out


def make_dglu(name, dev):
    import numpy as np
    import torch
    from moe_grouped_gemm_offset_amd import binding as B, synth
    from oracle import oracle as orc
    w = synth.WORKLOADS[name]
    counts = synth.workload_counts(name)
    inp = synth.dglu_inputs(w["L"], w["K"], w["N"], counts, c_std=w["c_std"], seed=w["seed"],
                            device=dev, discrete=w["discrete"])
    M, N, K, L = inp["M"], inp["N"], inp["K"], inp["L"]
    act = B.GG_DSWIGLU if w["act"] == "dswiglu" else B.GG_DGEGLU
    bptrs = None
    if inp["b_dense"] is None:
        bptrs = torch.tensor([x.data_ptr() for x in inp["b_list"]], dtype=torch.int64, device=dev)
    d = torch.empty(M, 2 * N, dtype=torch.bfloat16, device=dev)
    dprob = torch.zeros(M, dtype=torch.float32, device=dev)
    dbias = torch.zeros(L, 2 * N, dtype=torch.bfloat16, device=dev) if w["dbias"] else None
    ws = torch.empty(B.gg_dglu_workspace_size(L, N, dbias is not None), dtype=torch.uint8, device=dev)

    def run():
        B.gg_dglu(inp["a"], inp["b_dense"], bptrs, B.GG_MAJOR_K, N, inp["c"], inp["padded_offsets"],
                  inp["alpha"], inp["beta"], inp["prob"], d, dprob, dbias, act=act, workspace=ws)

    vm = inp["valid_m"]
    alg = 2 * (M * K + L * N * K + 2 * M * 2 * N) + 8 * M + (L * 2 * N * 4 if dbias is not None else 0)

    def sample(nrows):
        cpu = _cpu(inp)
        rows = np.linspace(0, vm - 1, nrows).astype(np.int64)
        t0 = time.perf_counter()
        orc.dglu(synth.bits(cpu["a"]), M, K, [synth.bits(x) for x in cpu["b_list"]], 0, N,
                 synth.bits(cpu["c"]), orc.BF16, cpu["padded_offsets"].numpy(), cpu["alpha"].numpy(),
                 cpu["beta"].numpy(), cpu["prob"].numpy(), act=act, rows=rows)
        return time.perf_counter() - t0, 2.0 * nrows * N * K

    return Op(name, "dglu_kernel", synth.flops_dgrad(vm, N, K), "bf16", run, alg, sample)


def make_wgrad(dev, a_major="m", f32acc=False, bf16acc=False):
    import numpy as np
    import torch
    from moe_grouped_gemm_offset_amd import binding as B, synth
    from oracle import oracle as orc
    w = synth.WORKLOADS["wgrad_moe"]
    counts = synth.workload_counts("wgrad_moe")
    inp = synth.wgrad_inputs(w["hidden"], w["inter"], counts, a_major, w["b_major"], seed=w["seed"],
                             device=dev)
    E, h, i, T = len(counts), inp["hidden"], inp["inter"], inp["tokens_sum"]
    ws = torch.empty(B.gg_wgrad_workspace_size(E), dtype=torch.uint8, device=dev)
    am = B.GG_MAJOR_K if a_major == "k" else B.GG_MAJOR_M
    if f32acc:
        # discrete per-expert fp32 outputs, separate allocations, accumulated
        # into from seeded N(0,1) values
        init = synth.wgrad_initial(E, h, i, torch.float32, seed=1003, device=dev)
        outs = [init[e].clone() for e in range(E)]
        del init
        ptrs = torch.tensor([o.data_ptr() for o in outs], dtype=torch.int64, device=dev)

        def run():
            B.gg_wgrad(inp["a"], am, inp["b"], B.GG_MAJOR_N, inp["offsets"], T, h, i,
                       wgrad_ptrs=ptrs, wgrad_dtype=B.GG_F32, accumulate=True, workspace=ws)

        # operands once; old outputs read and written back on the non-empty
        # experts (empty ones are left untouched)
        alg = 2 * (h * T + T * i) + 2 * 4 * int(np.sum(counts > 0)) * h * i
        run.keep = outs
    elif bf16acc:
        # the bf16 dense output accumulated into (from seeded N(0,1) values)
        out = synth.wgrad_initial(E, h, i, torch.bfloat16, seed=1003, device=dev)

        def run():
            B.gg_wgrad(inp["a"], am, inp["b"], B.GG_MAJOR_N, inp["offsets"], T, h, i,
                       wgrad_dense=out, accumulate=True, workspace=ws)

        alg = 2 * (h * T + T * i) + 2 * 2 * int(np.sum(counts > 0)) * h * i
    else:
        out = torch.empty(E, h, i, dtype=torch.bfloat16, device=dev)

        def run():
            B.gg_wgrad(inp["a"], am, inp["b"], B.GG_MAJOR_N, inp["offsets"], T, h, i,
                       wgrad_dense=out, workspace=ws)

        alg = 2 * (h * T + T * i) + 2 * E * h * i

    def sample(nrows):
        cpu = _cpu(inp)
        rows = np.linspace(0, h - 1, nrows).astype(np.int32)
        t0 = time.perf_counter()
        orc.wgrad(synth.bits(cpu["a"]), 0 if a_major == "k" else 1, synth.bits(cpu["b"]), 1,
                  cpu["offsets"].numpy(), h, i, T, out_dtype=orc.BF16, hrows=rows)
        return time.perf_counter() - t0, 2.0 * nrows * i * T

    return Op("wgrad_moe", "wgrad_kernel", synth.flops_wgrad(h, i, counts), "bf16", run, alg, sample)


def make_wgrad_mx(dev):
    import numpy as np
    import torch
    from moe_grouped_gemm_offset_amd import binding as B, synth
    from oracle import oracle as orc
    w = synth.WORKLOADS["wgrad_mxfp8"]
    counts = synth.workload_counts("wgrad_mxfp8")
    inp = synth.wgrad_mx_inputs(w["hidden"], w["inter"], counts, seed=w["seed"], device=dev)
    E, h, i, T = len(counts), inp["hidden"], inp["inter"], inp["tokens_sum"]
    out = torch.empty(E, h, i, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(B.gg_wgrad_workspace_size(E), dtype=torch.uint8, device=dev)
    a8, b8 = inp["a"].view(torch.uint8), inp["b"].view(torch.uint8)

    def run():
        B.gg_wgrad_mx(a8, inp["sfa"], b8, inp["sfb"], inp["offsets"], T, h, i, wgrad_dense=out,
                      workspace=ws)

    # codes and scales once, bf16 output written once
    alg = (h + i) * T + (h + i) * T // 32 + 2 * E * h * i

    def sample(nrows):
        cpu = _cpu(inp)
        rows = np.linspace(0, h - 1, nrows).astype(np.int32)
        t0 = time.perf_counter()
        orc.wgrad_mx(synth.bits(cpu["a"]), synth.bits(cpu["sfa"]), synth.bits(cpu["b"]),
                     synth.bits(cpu["sfb"]), cpu["offsets"].numpy(), h, i, T, out_dtype=orc.BF16,
                     hrows=rows)
        return time.perf_counter() - t0, 2.0 * nrows * i * T

    return Op("wgrad_mxfp8", "wgrad_mx_kernel", synth.flops_wgrad(h, i, counts), "fp8", run, alg,
              sample)


def make_dsrelu(dev, fp8out=False, nmajor=False):
    """The dsReLU workload; nmajor: B as discrete per-expert (K, N) N-major
    codes (the same values, transposed), scales unchanged."""
    import numpy as np
    import torch
    from moe_grouped_gemm_offset_amd import binding as B, synth
    from oracle import oracle as orc
    w = synth.WORKLOADS["dsrelu_mxfp8"]
    counts = synth.workload_counts("dsrelu_mxfp8")
    inp = synth.dsrelu_inputs(w["L"], w["K"], w["N"], counts, seed=w["seed"], device=dev,
                              discrete=nmajor)
    M, N, K, L = inp["M"], inp["N"], inp["K"], inp["L"]
    d = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    q = None
    if fp8out:
        d, q = _fp8_outputs(M, N, dev)
    dprob = torch.zeros(M, dtype=torch.float32, device=dev)
    amax = torch.zeros(L, dtype=torch.float32, device=dev)
    ws = torch.empty(B.gg_dsrelu_workspace_size(L), dtype=torch.uint8, device=dev)
    a8 = inp["a"].view(torch.uint8)
    if nmajor:
        bl = [x.view(torch.uint8).t().contiguous() for x in inp["b_list"]]
        bp = torch.tensor([x.data_ptr() for x in bl], dtype=torch.int64, device=dev)
        sp = torch.tensor([x.data_ptr() for x in inp["sfb_list"]], dtype=torch.int64, device=dev)

        def run():
            B.gg_dsrelu(a8, inp["sfa"], None, None, bp, sp, N, inp["c"], inp["padded_offsets"],
                        inp["alpha"], inp["prob"], d, dprob, amax, fp8_out=q, workspace=ws,
                        b_major=B.GG_MAJOR_N)
        run.keep = bl
    else:
        b8 = inp["b_dense"].view(torch.uint8)

        def run():
            B.gg_dsrelu(a8, inp["sfa"], b8, inp["sfb_dense"], None, None, N, inp["c"],
                        inp["padded_offsets"], inp["alpha"], inp["prob"], d, dprob, amax, fp8_out=q,
                        workspace=ws)

    vm = inp["valid_m"]
    d_bytes = M * N * 2 if not fp8out else 2 * M * N + 2 * M * N // 32
    alg = M * K + L * N * K + (M + L * N) * K // 32 + M * N * 2 + d_bytes + 8 * M

    def sample(nrows):
        cpu = _cpu(inp)
        rows = np.linspace(0, vm - 1, nrows).astype(np.int64)
        t0 = time.perf_counter()
        orc.dsrelu(synth.bits(cpu["a"]), synth.bits(cpu["sfa"]), M, K,
                   [synth.bits(x) for x in cpu["b_list"]], [synth.bits(x) for x in cpu["sfb_list"]],
                   N, synth.bits(cpu["c"]), orc.BF16, cpu["padded_offsets"].numpy(),
                   cpu["alpha"].numpy(), cpu["prob"].numpy(), rows=rows)
        return time.perf_counter() - t0, 2.0 * nrows * N * K

    name = "dsrelu_mxfp8" + ("_fp8out" if fp8out else "") + ("_nmajor" if nmajor else "")
    return Op(name, "dsrelu_kernel", synth.flops_dgrad(vm, N, K), "fp8", run, alg, sample)


def _fp8_outputs(M, W, dev):
    """E4M3 D_row with the rest of the FP8 output (D_col, both scale arrays,
    norm_const 1)."""
    import torch
    P = (M + 31) // 32
    d = torch.empty(M, W, dtype=torch.float8_e4m3fn, device=dev)
    q = dict(d_col=torch.empty(M, W, dtype=torch.uint8, device=dev),
             sfd_row=torch.empty(M, W // 32, dtype=torch.uint8, device=dev),
             sfd_col=torch.empty(W, P, dtype=torch.uint8, device=dev),
             norm_const=torch.ones(1, dtype=torch.float32, device=dev))
    return d, q


def make_dglu_mx(dev, fp8out=False):
    import numpy as np
    import torch
    from moe_grouped_gemm_offset_amd import binding as B, synth
    from oracle import oracle as orc
    w = synth.WORKLOADS["dglu_mxfp8"]
    counts = synth.workload_counts("dglu_mxfp8")
    inp = synth.dglu_mx_inputs(w["L"], w["K"], w["N"], counts, c_std=w["c_std"], seed=w["seed"],
                               device=dev, discrete=w["discrete"])
    M, N, K, L = inp["M"], inp["N"], inp["K"], inp["L"]
    d = torch.empty(M, 2 * N, dtype=torch.bfloat16, device=dev)
    q = None
    if fp8out:
        d, q = _fp8_outputs(M, 2 * N, dev)
    dprob = torch.zeros(M, dtype=torch.float32, device=dev)
    amax = torch.zeros(L, 2, dtype=torch.float32, device=dev)
    ws = torch.empty(B.gg_dglu_workspace_size(L, N, 0), dtype=torch.uint8, device=dev)
    a8 = inp["a"].view(torch.uint8)
    bp = torch.tensor([x.data_ptr() for x in inp["b_list"]], dtype=torch.int64, device=dev)
    sp = torch.tensor([x.data_ptr() for x in inp["sfb_list"]], dtype=torch.int64, device=dev)

    def run():
        B.gg_dglu_mx(a8, inp["sfa"], None, None, bp, sp, N, inp["c"], inp["padded_offsets"],
                     inp["alpha"], inp["beta"], inp["prob"], d, dprob, amax=amax, fp8_out=q,
                     workspace=ws)

    vm = inp["valid_m"]
    # A, B and their scales once, C read (bf16, 2N wide), D written (bf16;
    # or E4M3 D_row and D_col with their scales), prob read, dprob written
    d_bytes = M * 2 * N * 2 if not fp8out else 2 * M * 2 * N + 2 * M * 2 * N // 32
    alg = M * K + L * N * K + (M + L * N) * K // 32 + M * 2 * N * 2 + d_bytes + 8 * M

    def sample(nrows):
        cpu = _cpu(inp)
        rows = np.linspace(0, vm - 1, nrows).astype(np.int64)
        t0 = time.perf_counter()
        orc.dglu_mx(synth.bits(cpu["a"]), synth.bits(cpu["sfa"]), M, K,
                    [synth.bits(x) for x in cpu["b_list"]], [synth.bits(x) for x in cpu["sfb_list"]],
                    N, synth.bits(cpu["c"]), orc.BF16, cpu["padded_offsets"].numpy(),
                    cpu["alpha"].numpy(), cpu["beta"].numpy(), cpu["prob"].numpy(), rows=rows)
        return time.perf_counter() - t0, 2.0 * nrows * N * K

    return Op("dglu_mxfp8_fp8out" if fp8out else "dglu_mxfp8", "dglu_mx_kernel",
              synth.flops_dgrad(vm, N, K), "fp8", run, alg, sample)


WORKLOAD_OPS = {
    "moe_backward": ["dswiglu", "wgrad_moe", "dgeglu", "dsrelu_mxfp8"],
    "dswiglu": ["dswiglu"],
    "wgrad_moe": ["wgrad_moe"],
    "wgrad_moe_kmajor": ["wgrad_moe_kmajor"],
    "wgrad_moe_f32acc": ["wgrad_moe_f32acc"],
    "wgrad_moe_bf16acc": ["wgrad_moe_bf16acc"],
    "dgeglu": ["dgeglu"],
    "dsrelu_mxfp8": ["dsrelu_mxfp8"],
    "dglu_mxfp8": ["dglu_mxfp8"],
    "wgrad_mxfp8": ["wgrad_mxfp8"],
    "dsrelu_mxfp8_fp8out": ["dsrelu_mxfp8_fp8out"],
    "dglu_mxfp8_fp8out": ["dglu_mxfp8_fp8out"],
    "dsrelu_mxfp8_nmajor": ["dsrelu_mxfp8_nmajor"],
}


def build_op(name, dev):
    if name in ("dswiglu", "dgeglu"):
        return make_dglu(name, dev)
    if name == "wgrad_moe":
        return make_wgrad(dev, "m")
    if name == "wgrad_moe_kmajor":
        op = make_wgrad(dev, "k")
        op.name = name
        return op
    if name == "wgrad_moe_f32acc":
        op = make_wgrad(dev, "m", f32acc=True)
        op.name = name
        return op
    if name == "wgrad_moe_bf16acc":
        op = make_wgrad(dev, "m", bf16acc=True)
        op.name = name
        return op
    if name == "dglu_mxfp8":
        return make_dglu_mx(dev)
    if name == "wgrad_mxfp8":
        return make_wgrad_mx(dev)
    if name == "dglu_mxfp8_fp8out":
        return make_dglu_mx(dev, fp8out=True)
    if name == "dsrelu_mxfp8_fp8out":
        return make_dsrelu(dev, fp8out=True)
    if name == "dsrelu_mxfp8_nmajor":
        return make_dsrelu(dev, nmajor=True)
    return make_dsrelu(dev)


# The kernel each single-op workload runs.
KERNEL_OF = {"dswiglu": "dglu_kernel", "dgeglu": "dglu_kernel", "wgrad_moe": "wgrad_kernel",
             "wgrad_moe_kmajor": "wgrad_kernel", "wgrad_moe_f32acc": "wgrad_kernel",
             "wgrad_moe_bf16acc": "wgrad_kernel", "dsrelu_mxfp8": "dsrelu_kernel",
             "dglu_mxfp8": "dglu_mx_kernel", "wgrad_mxfp8": "wgrad_mx_kernel",
             "dsrelu_mxfp8_fp8out": "dsrelu_kernel", "dglu_mxfp8_fp8out": "dglu_mx_kernel",
             "dsrelu_mxfp8_nmajor": "dsrelu_kernel"}

# Ops timed beside a workload's step (per-op statistics only; not part of the
# step or its value): the MoE wgrad's other output modes and A major.
EXTRA_OPS = {"moe_backward": ["wgrad_moe_kmajor", "wgrad_moe_bf16acc", "wgrad_moe_f32acc"]}

FLUSH_BYTES = 512 << 20       # > the 256 MB MALL: a read-modify-write of it evicts the cache


class ClockSampler:
    """Samples the GPU's current engine clock (amdsmi GPU metrics, MHz) in a
    background thread while ops run; None where the metrics are unavailable."""

    def __init__(self):
        self.h = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            if hs:
                self.amdsmi, self.h = amdsmi, hs[0]
                if self._read() is None:
                    self.h = None
        except Exception:
            self.h = None

    def _read(self):
        try:
            m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.h)
        except Exception:
            return None
        # per-XCD engine clocks (MHz), averaged; else the single value
        for key in ("current_gfxclks", "current_gfxclk", "average_gfxclk_frequency"):
            v = m.get(key)
            if isinstance(v, (list, tuple)):
                v = [x for x in v if isinstance(x, (int, float)) and 0 < x < 10000]
                v = sum(v) / len(v) if v else None
            if isinstance(v, (int, float)) and 0 < v < 10000:
                return float(v)
        return None

    def __enter__(self):
        import threading
        self.samples, self.stop, self.t0 = [], threading.Event(), time.perf_counter()
        if self.h is not None:
            def loop():
                while not self.stop.is_set():
                    v = self._read()
                    if v is not None:
                        self.samples.append((time.perf_counter(), v))
                    self.stop.wait(0.005)
            self.t = threading.Thread(target=loop, daemon=True)
            self.t.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        if self.h is not None:
            self.t.join()

    def median(self, skip_s=0.0):
        """Median of the samples taken at least skip_s after sampling began
        (the metrics refresh about every 100 ms, so a value read right after
        a change of load still describes the previous one)."""
        v = sorted(x for t, x in self.samples if t >= self.t0 + skip_s)
        return v[len(v) // 2] if v else None


CLOCK_RUN_S, CLOCK_SKIP_S = 0.4, 0.15


def per_op_stats(ops, reps, dev, clock):
    """Median, p10 and p90 of each op's per-launch HIP-event durations over
    `reps` launches, warm (back to back) and cold (a read-modify-write of
    FLUSH_BYTES before each launch, outside its events, evicts the MALL);
    and the median engine clock over a separate CLOCK_RUN_S of back-to-back
    launches (samples from its first CLOCK_SKIP_S dropped)."""
    import torch
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    out = {}
    for op in ops:
        for _ in range(3):
            op.run()
        torch.cuda.synchronize()
        st = {}
        for mode in ("warm", "cold"):
            evs = []
            with clock:
                for _ in range(reps):
                    if mode == "cold":
                        flush.add_(1.0)
                    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    s.record()
                    op.run()
                    e.record()
                    evs.append((s, e))
                torch.cuda.synchronize()
            t = sorted(s.elapsed_time(e) for s, e in evs)
            q = lambda f: round(t[min(len(t) - 1, int(f * (len(t) - 1) + 0.5))], 4)
            st[mode] = {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9)}
        clk = None
        if clock.h is not None:
            n = max(1, int(CLOCK_RUN_S / (st["warm"]["p50"] * 1e-3)))
            with clock:
                for _ in range(n):
                    op.run()
                torch.cuda.synchronize()
            clk = clock.median(CLOCK_SKIP_S)
        st["clock_mhz"] = None if clk is None else round(clk)
        out[op.name] = st
    del flush
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(ops, budget_s):
    """Oracle throughput on a bounded row sample of each op, extrapolated to
    the step: total FLOPs over the sum of the projected per-op times."""
    from oracle import oracle as orc
    threads = orc.num_threads()
    per = budget_s / len(ops)
    proj, parts = 0.0, []
    for op in ops:
        t, f = op.oracle_sample(threads)                # calibration: one row per thread
        rate = f / max(t, 1e-9)
        n = max(threads, int(threads * max(1.0, per / max(t, 1e-9))))
        t, f = op.oracle_sample(n)
        rate = f / t
        proj += op.flops / rate
        parts.append(f"{op.name}: {n} rows, {t:.1f} s, {rate / 1e9:.2f} GFLOP/s")
    total = sum(op.flops for op in ops)
    return {"value": total / proj / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "per_core": per_core_rate(),
            "sample": "; ".join(parts) + " (rows spread over every group, extrapolated by FLOPs)"}


def per_core_rate():
    """The oracle on one thread over the whole small wgrad workload (hidden
    256, intermediate 256, counts [256, 0, 512, 256]): one core's rate."""
    from oracle import oracle as orc
    from moe_grouped_gemm_offset_amd import synth
    w = synth.WORKLOADS["wgrad_small"]
    inp = synth.wgrad_inputs(w["hidden"], w["inter"], w["counts"], a_major=w["a_major"],
                             b_major=w["b_major"], seed=w["seed"])
    threads = orc.num_threads()
    orc.set_threads(1)
    try:
        t0 = time.perf_counter()
        orc.wgrad(synth.bits(inp["a"]), 0 if inp["a_major"] == "k" else 1, synth.bits(inp["b"]),
                  0 if inp["b_major"] == "k" else 1, inp["offsets"].numpy(), inp["hidden"],
                  inp["inter"], inp["tokens_sum"])
        t = time.perf_counter() - t0
    finally:
        orc.set_threads(threads)
    flops = 2.0 * w["hidden"] * w["inter"] * int(inp["tokens_sum"])
    return {"workload": "wgrad_small", "threads": 1, "s": round(t, 3),
            "gflop_s": round(flops / t / 1e9, 3)}


COPY_BYTES = 1 << 30          # calibration copy: 1 GiB read + 1 GiB written
PEAK_LIB = os.path.join(ROOT, "moe_grouped_gemm_offset_amd", "libgg_peak.so")


def measured_peaks(dev, clock):
    """This GPU's sustained rates, measured here: dense MFMA from the probe
    kernels of libgg_peak.so (four independent MFMAs per wave per round,
    register operands, no memory traffic; 1024 workgroups of 8 waves), with
    the engine clock during them; and HBM from a device-to-device copy of
    COPY_BYTES (read plus written bytes).  Each rate is the best of 20 MFMA
    runs (about 18 ms each) or 5 copies."""
    import ctypes
    import torch
    if not os.path.exists(PEAK_LIB):
        return None
    L = ctypes.CDLL(PEAK_LIB)
    L.gg_peak_mfma.restype = ctypes.c_double
    L.gg_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_void_p]
    out = torch.zeros(1024, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    res = {}
    for kind, name, iters in ((0, "mfma_bf16", 32768), (1, "mfma_fp8", 16384)):
        if L.gg_peak_mfma(kind, 1024, iters, ctypes.c_void_p(out.data_ptr()), stream) <= 0:
            return None
        torch.cuda.synchronize()
        evs = []
        with clock:
            for _ in range(20):
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                f = L.gg_peak_mfma(kind, 1024, iters, ctypes.c_void_p(out.data_ptr()), stream)
                e.record()
                evs.append((s, e))
            torch.cuda.synchronize()
        ms = min(s.elapsed_time(e) for s, e in evs)
        clk = clock.median(CLOCK_SKIP_S) if clock.h is not None else None
        res[name] = {"tflops": round(f / (ms * 1e-3) / 1e12, 1),
                     "clock_mhz": None if clk is None else round(clk)}
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        dst.copy_(src)
        e.record()
        ts.append((s, e))
    torch.cuda.synchronize()
    ms = min(s.elapsed_time(e) for s, e in ts)
    res["hbm_copy_gb_s"] = round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1)
    del src, dst
    return res


def calibrate_copy(dev, reps=3):
    """A plain device-to-device copy of COPY_BYTES, so that rocprofv3's
    FETCH_SIZE / WRITE_SIZE can be scaled by what they read for known bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def summarize_pmc(fetch_csv, write_csv, workload_kernels, out_path):
    """Per-launch HBM traffic of our kernels from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each counter is scaled
    by COPY_BYTES over what it reads for the calibration copy."""
    import csv
    import collections

    def per_kernel(path, counter):
        vals = collections.defaultdict(list)
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            vals[row["Kernel_Name"]].append(float(row["Counter_Value"]) * 1024.0)
        return vals

    out = {}
    if os.path.exists(out_path):
        with open(out_path) as f:
            out = {k: v for k, v in json.load(f).items() if not k.startswith("_")}
    scales = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        # the calibration copy is a same-dtype device copy, which the runtime
        # runs as its copyBuffer kernel; it is the largest such dispatch
        copies = [max(v) for k, v in vals.items() if "copyBuffer" in k]
        measured = max(copies) if copies else None
        scale = COPY_BYTES / measured if measured else None
        scales[counter] = {"copy_measured_bytes": measured, "scale": scale}
        for name, (kernel, workload) in workload_kernels.items():
            hits = [v for k, v in vals.items() if kernel in k]
            if not hits or scale is None:
                continue
            samples = [x for v in hits for x in v]
            key = f"{kernel}:{workload}"
            if counter == "FETCH_SIZE" or key not in out:
                out[key] = {"source_hash": source_hash(kernel)}
            out[key][counter.lower() + "_bytes"] = sum(samples) / len(samples) * scale
            out[key][counter.lower() + "_scale"] = scale
    for ent in out.values():
        if "fetch_size_bytes" in ent and "write_size_bytes" in ent:
            ent["bytes_per_launch"] = ent["fetch_size_bytes"] + ent["write_size_bytes"]
    out["_scale"] = scales
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    return out


# rocprofv3 counter passes behind the utilisation summaries (each within one
# pass's hardware limits: at most 8 SQ, 4 TCP, 2 TA, 2 TD, 2 GRBM counters).
COUNTER_GROUPS = {
    "sq": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_LDS",
           "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_ANY", "SQ_BUSY_CYCLES",
           "GRBM_GUI_ACTIVE"],
    "mem": ["TCP_TCR_TCP_STALL_CYCLES", "TCP_PENDING_STALL_CYCLES", "TCP_TCP_TA_DATA_STALL_CYCLES",
            "TCP_READ_TAGCONFLICT_STALL_CYCLES", "TD_TD_BUSY", "TD_TC_STALL", "TA_TA_BUSY",
            "TA_DATA_STALLED_BY_TC_CYCLES", "GRBM_GUI_ACTIVE"],
    "l2": ["TCC_HIT_sum", "TCC_MISS_sum", "GRBM_GUI_ACTIVE", "GRBM_COUNT"],
}
N_XCD, N_CU, N_SIMD = 8, 256, 1024


def counter_command(workload, group, kernel):
    return (f"cd /tmp && TMPDIR=/tmp timeout -s KILL 120 rocprofv3 --pmc {' '.join(COUNTER_GROUPS[group])} "
            f"--kernel-include-regex {kernel} -d $R/gpurun_out/pmc/{workload}_{group} -o out "
            f"--output-format csv -- python3 $R/bench.py --workload {workload} --steps 3 --warmup 1 "
            f"--reps 0 --no-extras --no-cpu-baseline")


def summarize_counters(workload, kernel, root, out_path):
    """Per-dispatch averages of the COUNTER_GROUPS passes of one workload
    (root/<workload>_<group>/out_counter_collection.csv) and the
    utilisations derived from them, written as a markdown summary."""
    import csv
    import collections
    vals, durs = collections.defaultdict(list), collections.defaultdict(dict)
    for group in COUNTER_GROUPS:
        path = os.path.join(root, f"{workload}_{group}", "out_counter_collection.csv")
        for r in csv.DictReader(open(path)):
            if kernel not in r["Kernel_Name"]:
                continue
            vals[(group, r["Counter_Name"])].append(float(r["Counter_Value"]))
            durs[group][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    out = {}
    for group in COUNTER_GROUPS:
        d = list(durs[group].values())
        t_us = sum(d) / len(d)
        cyc = avg[(group, "GRBM_GUI_ACTIVE")] / N_XCD          # engine cycles per XCD
        out[group] = {"dispatches": len(d), "us": t_us, "ghz": cyc / (t_us * 1e3), "cyc": cyc}
    sq, mem, l2 = (out[g]["cyc"] for g in ("sq", "mem", "l2"))
    derived = [
        ("engine clock during the kernel (GRBM_GUI_ACTIVE / 8 XCDs / duration)",
         f"{out['sq']['ghz']:.2f} GHz ({out['mem']['ghz']:.2f}, {out['l2']['ghz']:.2f} in the other passes)"),
        ("MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles)",
         f"{avg[('sq', 'SQ_VALU_MFMA_BUSY_CYCLES')] / (N_SIMD * sq):.3f}"),
        ("MFMA busy x clock / 2.4 GHz (share of the published peak the pipe delivered)",
         f"{avg[('sq', 'SQ_VALU_MFMA_BUSY_CYCLES')] / (N_SIMD * sq) * out['sq']['ghz'] / 2.4:.3f}"),
        ("LDS busy: SQ_LDS_IDX_ACTIVE / (256 CUs x cycles)", f"{avg[('sq', 'SQ_LDS_IDX_ACTIVE')] / (N_CU * sq):.3f}"),
        ("LDS bank conflicts: SQ_LDS_BANK_CONFLICT / (256 CUs x cycles)",
         f"{avg[('sq', 'SQ_LDS_BANK_CONFLICT')] / (N_CU * sq):.3f}"),
        ("TD busy: TD_TD_BUSY / (256 x cycles)", f"{avg[('mem', 'TD_TD_BUSY')] / (N_CU * mem):.3f}"),
        ("TD stalled on the TC: TD_TC_STALL / (256 x cycles)", f"{avg[('mem', 'TD_TC_STALL')] / (N_CU * mem):.3f}"),
        ("TCP waiting for L2 data: TCP_PENDING_STALL_CYCLES / (256 x cycles)",
         f"{avg[('mem', 'TCP_PENDING_STALL_CYCLES')] / (N_CU * mem):.3f}"),
        ("TCP stalled by the TCR (L1 -> L2 requests): TCP_TCR_TCP_STALL_CYCLES / (256 x cycles)",
         f"{avg[('mem', 'TCP_TCR_TCP_STALL_CYCLES')] / (N_CU * mem):.3f}"),
        ("TA busy: TA_TA_BUSY / (256 x cycles)", f"{avg[('mem', 'TA_TA_BUSY')] / (N_CU * mem):.3f}"),
        ("L2 hit rate: TCC_HIT / (TCC_HIT + TCC_MISS)",
         f"{avg[('l2', 'TCC_HIT_sum')] / (avg[('l2', 'TCC_HIT_sum')] + avg[('l2', 'TCC_MISS_sum')]):.3f}"),
    ]
    lines = [f"# {kernel} on the {workload} workload — rocprofv3 counters", "",
             "Three counter passes, each in its own run (from the repository root `$R` on the GPU box):", ""]
    lines += ["    " + counter_command(workload, g, kernel) for g in COUNTER_GROUPS]
    lines += ["", f"Summarised by `python3 bench.py --workload {workload} --summarize-counters "
              f"$R/gpurun_out/pmc`.", "",
              "| pass | dispatches | average duration µs (under counter collection) | clock GHz |",
              "|---|---|---|---|"]
    lines += [f"| {g} | {o['dispatches']} | {o['us']:.1f} | {o['ghz']:.2f} |" for g, o in out.items()]
    lines += ["", "| derived (per-dispatch averages) | value |", "|---|---|"]
    lines += [f"| {a} | {b} |" for a, b in derived]
    lines += ["", "| counter (pass) | per-dispatch average |", "|---|---|"]
    lines += [f"| {c} ({g}) | {v:.6g} |" for (g, c), v in sorted(avg.items())]
    lines += ["", f"Kernel source hash at measurement: `{source_hash(kernel)}`.", ""]
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    return derived


def bound_of(op):
    """The roofline that bounds an op: "hbm" when its algorithmic bytes at
    the HBM peak take longer than its FLOPs at the MFMA peak, else "mfma"."""
    t_hbm = op.alg_bytes / (HBM_PEAK * 1e9)
    t_mfma = op.flops / (PEAK[op.dtype] * 1e12)
    return "hbm" if t_hbm > t_mfma else "mfma"


def traffic_for(kernel, workload):
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(f"{kernel}:{workload}")
    if not ent or ent.get("source_hash") != source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="moe_backward", choices=sorted(WORKLOAD_OPS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reps", type=int, default=50,
                    help="per-op launches for the warm / cold medians (0: skip that phase)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the ops timed beside the step (other wgrad modes)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="with a single-op --workload: summarise the counter passes of "
                         "COUNTER_GROUPS found under DIR into profiles/, and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="with a single-op --workload: record its per-launch HBM traffic from "
                         "two rocprofv3 --pmc runs in profiles/hbm_traffic.json, and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        names = WORKLOAD_OPS[args.workload]
        if len(names) != 1:
            sys.exit("--summarize-counters needs a single-op --workload")
        kernel = KERNEL_OF[names[0]]
        path = os.path.join(ROOT, "profiles", f"counters-{kernel}-{names[0]}.md")
        for a, b in summarize_counters(names[0], kernel, args.summarize_counters, path):
            print(f"{a}: {b}")
        return
    if args.summarize_pmc:
        names = WORKLOAD_OPS[args.workload]
        if len(names) != 1:
            sys.exit("--summarize-pmc needs a single-op --workload")
        kernel = KERNEL_OF[names[0]]
        path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
        res = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1],
                            {names[0]: (kernel, names[0])}, path)
        print(json.dumps(res, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from moe_grouped_gemm_offset_amd import binding as B
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    B.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] building inputs for {args.workload}", file=sys.stderr, flush=True)
    ops = [build_op(n, dev) for n in WORKLOAD_OPS[args.workload]]
    torch.cuda.synchronize()
    if args.calibrate_copy:
        calibrate_copy(dev)

    for _ in range(args.warmup):
        for op in ops:
            op.run()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    ev = {op.name: [] for op in ops}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for op in ops:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            op.run()
            e.record()
            ev[op.name].append((s, e))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)

    def entry(op, ms):
        """An op's figures at a per-launch duration of ms."""
        tf = op.flops / (ms * 1e-3) / 1e12
        k = {"kernel": op.kernel, "ms": round(ms, 4), "gflop": round(op.flops / 1e9, 2),
             "tflops": round(tf, 1), "peak_frac": round(tf / PEAK[op.dtype], 4),
             "dtype": op.dtype, "alg_gb_s": round(op.alg_bytes / (ms * 1e-3) / 1e9, 1)}
        tr = traffic_for(op.kernel, op.name)
        k["hbm_gb_per_launch"] = None if tr is None else round(tr / 1e9, 3)
        k["bound"] = bound_of(op)
        # the roofline time (the larger of the MFMA-peak and HBM-peak times)
        # over the measured time
        t_roof = max(op.flops / (PEAK[op.dtype] * 1e12), op.alg_bytes / (HBM_PEAK * 1e9))
        k["roofline_frac"] = round(t_roof / (ms * 1e-3), 4)
        return k

    kernels = {}
    for op in ops:
        times = sorted(s.elapsed_time(e) for s, e in ev[op.name])
        pct = lambda q: times[min(len(times) - 1, int(q * (len(times) - 1) + 0.5))]
        # the timed region's mean duration (the step's own launches)
        kernels[op.name] = entry(op, sum(times) / len(times))
        kernels[op.name]["in_step"] = True
        kernels[op.name]["step_ms_p10_p50_p90"] = [round(pct(0.1), 4), round(pct(0.5), 4),
                                                   round(pct(0.9), 4)]

    # every op again on its own: warm and cold (MALL evicted) medians over
    # --reps launches, with the engine clock; plus the ops timed beside the
    # step, whose figures come from their warm median
    extras = [] if args.no_extras else [build_op(n, dev) for n in EXTRA_OPS.get(args.workload, [])]
    if args.reps > 0:
        print(f"[bench] per-op medians over {args.reps} launches ({len(ops) + len(extras)} ops)",
              file=sys.stderr, flush=True)
        stats = per_op_stats(ops + extras, args.reps, dev, ClockSampler())
        for op in ops + extras:
            if op in extras:
                kernels[op.name] = entry(op, stats[op.name]["warm"]["p50"])
                kernels[op.name]["in_step"] = False
            kernels[op.name]["warm"] = stats[op.name]["warm"]
            kernels[op.name]["cold"] = stats[op.name]["cold"]
            kernels[op.name]["clock_mhz"] = stats[op.name]["clock_mhz"]
    # the chip's measured peaks, and each op against them
    mpk = None if args.reps <= 0 else measured_peaks(dev, ClockSampler())
    if mpk:
        for op in ops + extras:
            k = kernels[op.name]
            mf = mpk["mfma_bf16" if op.dtype == "bf16" else "mfma_fp8"]["tflops"]
            k["measured_peak_frac"] = round(k["tflops"] / mf, 4)
            t_roof = max(op.flops / (mf * 1e12), op.alg_bytes / (mpk["hbm_copy_gb_s"] * 1e9))
            k["measured_roofline_frac"] = round(t_roof / (k["ms"] * 1e-3), 4)
    total_flops = sum(op.flops for op in ops)
    value = total_flops / (ms_step * 1e-3) / 1e12
    dom = max(ops, key=lambda o: kernels[o.name]["ms"])
    kd = kernels[dom.name]
    src = source_hash(dom.kernel)
    if bound_of(dom) == "hbm":
        achieved, peak, unit = dom.alg_bytes / (kd["ms"] * 1e-3) / 1e9, HBM_PEAK, "GB/s"
    else:
        achieved, peak, unit = dom.flops / (kd["ms"] * 1e-3) / 1e12, PEAK[dom.dtype], "TFLOP/s"
    roofline = {"bound": bound_of(dom), "achieved": round(achieved, 1), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": traffic_for(dom.kernel, dom.name), "kernel": dom.kernel,
                "workload": dom.name, "source_hash": src}
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a row sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(ops, args.cpu_budget)
    dtypes = sorted({op.dtype for op in ops})
    line = {
        "metric": "grouped-GEMM TFLOP/s and % of MI355X bf16/fp8 MFMA peak, 1 GPU",
        "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "+".join("bf16" if d == "bf16" else "mxfp8" for d in dtypes),
        "data": "synthetic",
        "config": {"workload": args.workload, "ops": [op.name for op in ops],
                   "gflop_per_step": round(total_flops / 1e9, 1), "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "measured_peaks": mpk,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
