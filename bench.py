#!/usr/bin/env python3
"""Throughput of the R2L selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: one R2LM denoising step = 7 hooked reverse scans (every 4th
of 28 decoder layers), each over a batch of 64 generation blocks of 32 tokens
at D = 2048, N = 16, bf16 inputs with fp32 state, res = x and s ~ U(0, 0.1).
Inputs are seeded synthetic tensors (``synth``), resident in HBM before the
timed region; the buffer sets rotate over more than 1 GB so that every step
reads HBM rather than the 256 MB Infinity Cache.

One JSON line on stdout: ``value`` is token·channels per second of whole
steps; ``roofline`` rates the dominant entry point's launches (one call's
kernels; average duration from HIP events on the launch stream over the timed
region) against the roofline that binds it; ``cpu_baseline`` is the fp64
oracle timed on the host, and ``parity_vs_oracle`` compares the timed calls'
GPU results with the oracle's on that sample.
Other workloads (``--workload``) are the prefill reverse scan (8 x 4096 x 4096),
the ragged serving step (reverse scan + block commit over 256 blocks of
U{16..64} tokens at D = 4096), the ragged prefix-state prefill, and the fp32
block-restricted and tiny cases.
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

HBM_PEAK_GBS = 8000.0
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz: one fp32 VALU instruction per lane per clock
VALU_PEAK_TLANEOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# VALU issue slots one v_exp_f32 / v_log_f32 takes on gfx950 in code that mixes
# it with fp32 FMAs as the scan does (one exp per four FMAs): the issue-rate
# micro-benchmark `bench.py --alu-rates` (csrc/alu_rates.hip), summarised with
# its command in profiles/alu_rates__v_exp_f32_issue_rate.md
TRANS_SLOTS = 1.75


def alu_ops_per_tc(readout: bool, res: bool) -> float:
    """Algorithmic VALU lane-ops per token·channel (N = 16), trans ops weighted.

    per state n : exp(Delta*A) [trans] + Delta*A + B*(Delta*x) + state fma (+ readout fma)
    per channel : softplus (2 trans + 4 ops) + Delta*x (+ Dskip fma) (+ gate fma)
    """
    per_n = TRANS_SLOTS + (4 if readout else 3)
    per_tc = 2 * TRANS_SLOTS + 4 + 1 + (1 if readout else 0) + (1 if res else 0)
    return 16 * per_n + per_tc


def scan_bytes(tok, D, es, readout=True, res_separate=False, h_in=False, h_out=False, batch=0,
               state_rw=False):
    """Algorithmic HBM bytes: every input read once, every output written once."""
    N = 16
    b = tok * D * es * 2 + tok * N * es          # x, dt, Bm
    b += 4 * D * N                               # A
    if readout:
        b += tok * N * es + tok * D * es + 4 * D  # Cm, out, Dskip
        if res_separate:
            b += tok * D * es
    if h_in:
        b += 4 * batch * D * N
    if h_out:
        b += 4 * batch * D * N
    if state_rw:
        b += 8 * batch * D * N
    return b


KERNEL_SOURCES = ("scan_device.h", "scan_geometry.h", "scan_internal.h", "scan_segment.h",
                  "scan_kernels.hip", "bidir_kernels.hip", "bwd_kernels.hip")


def kernel_sha() -> str:
    """Hash of the device code (every kernel source and the headers they include)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "reverse_mamba_selective_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM traffic per call from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "segment_scan__%s__traffic.json" % workload)
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("bytes_per_launch")


class Parity:
    """Error of the GPU results of the timed calls against the oracle's values
    on the CPU-baseline sample: max|err| / max|ref| against the tolerance and,
    for bf16 outputs, the worst element measured in (one bf16 ulp of the
    oracle's value + the fp32 bound 1e-5 * max|ref|), which must stay <= 1."""

    def __init__(self, what, dtype, tol):
        self.what, self.dtype, self.tol = what, dtype, tol
        self.err = self.ref = self.worst = 0.0
        self.n = 0

    def add(self, got, ref, slack=0.0):
        """slack: an absolute allowance added to the fp32 bound of the bf16
        element check (the sidecar's bf16 intermediates)."""
        import numpy as np
        ref = np.asarray(ref, dtype=np.float64)
        got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
        if ref.size == 0:
            return
        d = np.abs(got - ref)
        scale = float(np.max(np.abs(ref)))
        self.err = max(self.err, float(np.max(d)))
        self.ref = max(self.ref, scale)
        self.n += ref.size
        if self.dtype == "bf16":
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
            self.worst = max(self.worst, float(np.max(d / (ulp + max(1e-5 * scale, slack)))))

    def result(self):
        rel = self.err / max(self.ref, 1e-30)
        r = {"what": self.what, "elements": self.n, "max_err_over_max_ref": rel,
             "tol": self.tol}
        ok = rel <= self.tol
        if self.dtype == "bf16":
            r["worst_vs_ulp_bound"] = self.worst
            ok = ok and self.worst <= 1.0
        r["pass"] = bool(ok)
        return r


def host_cpu():
    """Model string and CPU count of the host the oracle runs on."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "cpus_available": avail}


def copy_bandwidth_gbs(torch, nbytes=1 << 30, reps=5):
    """Device-to-device copy rate of HBM (bytes read + bytes written per second)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def percentiles(v):
    import numpy as np
    p10, p50, p90 = np.percentile(np.asarray(v, dtype=np.float64), [10, 50, 90])
    return {"p10": float(p10), "median": float(p50), "p90": float(p90)}


# ---------------------------------------------------------------------------
class Workload:
    name = ""
    config: dict = {}
    dtype = "bf16"

    def setup(self, torch, r2l):
        raise NotImplementedError

    step_calls: list = []   # per rotating set: the entry-point calls of one step
    measure: list = []      # per timed entry point: label, calls, bytes, alu, tc per launch
    step_entries: list = [0]  # index into measure of each call of a step
    launches_per_step = 1
    graph_ok = True           # the step may be captured in a hipGraph
    isolate_entries = False   # time each entry point in a loop of its own (see main)

    def step(self, i, stream):
        for c in self.step_calls[i % len(self.step_calls)]:
            c.launch(stream)

    def cpu_baseline(self, budget_s, nthreads=0, parity=None):
        """Oracle token·channels/s on a bounded sample of the workload; with a
        Parity object, also compares the GPU results of the timed calls."""
        raise NotImplementedError


def _dev(torch, a, dtype):
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).to("cuda")


def _rotation(set_bytes, floor=1 << 30):
    return max(1, math.ceil(floor / max(set_bytes, 1)))


class Denoise(Workload):
    """7 hooked reverse scans of one denoising step, 64 x 32 x 2048, bf16."""
    name = "denoise_step_bf16_b64_blk32_D2048_N16_7hooks"
    HOOKS, B, L, D = 7, 64, 32, 2048
    reverse = True
    entry = "r2l_scan"

    def setup(self, torch, r2l):
        import synth
        self.torch = torch
        self.gates = synth.denoise_gates()
        self.inputs = [synth.denoise_hook_inputs(h) for h in range(self.HOOKS)]
        tok = self.B * self.L
        self.tc_per_launch = tok * self.D
        self.tc_per_step = self.tc_per_launch * self.HOOKS
        self.bytes_per_launch = scan_bytes(tok, self.D, 2, readout=True)
        self.alu_per_launch = self.tc_per_launch * alu_ops_per_tc(True, True)
        self.launches_per_step = self.HOOKS
        base = []
        for h, inp in enumerate(self.inputs):
            g = {k: _dev(torch, getattr(inp, k), "bf16").view(self.B, self.L, -1)
                 for k in ("x", "dt", "Bm", "Cm")}
            g["A"] = torch.from_numpy(inp.A).cuda()
            g["Dskip"] = torch.from_numpy(inp.Dskip).cuda()
            base.append(g)
        set_bytes = self.bytes_per_launch * self.HOOKS
        self.R = _rotation(set_bytes)
        self.step_calls = []
        self.outs0 = []
        self._bound_inputs = {}
        for r in range(self.R):
            row = []
            for h, g in enumerate(base):
                x = g["x"].clone()
                out = torch.empty_like(x)
                if r == 0:
                    self.outs0.append(out)
                ins = {"dt": g["dt"].clone(), "Bm": g["Bm"].clone(), "Cm": g["Cm"].clone(),
                       "A": g["A"], "Dskip": g["Dskip"]}
                self._bound_inputs.setdefault(r, {})[h] = dict(ins, x=x)
                row.append(r2l.bind(self.entry, x=x, res=x, s=float(self.gates[h]), out=out,
                                    **ins))
            self.step_calls.append(row)
        self.step_entries = [0] * self.HOOKS
        self.measure = [dict(label="%s (one hook)" % self.entry,
                             calls=[c for row in self.step_calls for c in row],
                             bytes=self.bytes_per_launch, alu=self.alu_per_launch,
                             tc=self.tc_per_launch)]
        self.config = {"workload": self.name, "batch": self.B, "block_tokens": self.L,
                       "D": self.D, "N": 16, "hooks_per_step": self.HOOKS,
                       "in_dtype": "bf16", "state_dtype": "fp32", "res": "x",
                       "rotating_sets": self.R, "rotating_bytes": set_bytes * self.R,
                       "parallelism": "single_gpu"}

    def cpu_baseline(self, budget_s, nthreads=0, parity=None):
        import oracle
        tc, secs, reps, hooks = 0, 0.0, 0, 0
        while secs < budget_s and reps < 200:
            for h, inp in enumerate(self.inputs):
                t = {}
                r = oracle.selective_scan(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip,
                                          reverse=self.reverse, res=inp.x,
                                          s=float(self.gates[h]), seq_offsets=inp.offsets,
                                          timing=t, want_y=False, want_out=True,
                                          nthreads=nthreads)
                if parity is not None and reps == 0:
                    parity.add(self.outs0[h].float().cpu().numpy().reshape(r["out"].shape),
                               r["out"])
                secs += t["seconds"]
                tc += inp.x.size
                hooks += 1
                if nthreads == 1 and secs >= budget_s:
                    break
            reps += 1
        return {"value": tc / secs, "unit": "tokens*channels/s",
                "cores": nthreads or oracle.max_threads(), "kind": "oracle",
                "sample": "%d hooks of the 7-hook step (%d token-channels), %.1f s of oracle "
                          "time" % (hooks, tc, secs)}

    parity_spec = ("out", "bf16", 2e-2,
                   "out = x + s*y of all 7 hooks (first buffer set) vs the oracle's")


def bwd_alu_ops_per_tc() -> float:
    """Algorithmic VALU lane-ops per token·channel of the backward (N = 16,
    trans ops weighted), without recomputation: the forward states (84.5), per
    state the adjoint (g += dy*C; dy*h and its sum over channels; the dDelta
    term B*x + A*(abar*h_prev) and its fma; dA += g*Delta*(abar*h_prev); dx's
    g*B; g*Delta*x and its sum over channels; g *= abar: 13), per channel dy,
    dDskip, dx (2) and sigmoid (2 trans + 2), and ds (1: ds is the contraction
    of the unscaled dCm and dDskip with Cm and Dskip, so the readout y is not
    needed)."""
    return alu_ops_per_tc(False, False) + 16 * 13 + 1 + 1 + 2 + (2 * TRANS_SLOTS + 2) + 1


class DenoiseBackward(Denoise):
    """The backward of the 7 hooked reverse scans of one denoising step (training
    the R2L stream): r2l_scan_backward with res = x, all gradients."""
    name = "denoise_backward_bf16_b64_blk32_D2048_N16_7hooks"

    def setup(self, torch, r2l):
        import synth
        super().setup(torch, r2l)
        tok = self.B * self.L
        # bytes: x, dt, dout in; dx, ddt out (bf16); Bm, Cm in (bf16); dBm, dCm out (fp32);
        # A in, dA out, Dskip in, dDskip out, ds
        self.bytes_per_launch = (tok * self.D * 2 * 5 + tok * 16 * (2 * 2 + 4 * 2) +
                                 self.D * 16 * 4 * 2 + self.D * 4 * 2 + 4)
        self.alu_per_launch = self.tc_per_launch * bwd_alu_ops_per_tc()
        self.bwd_calls, self.bwd_grads, self._douts = [], [], []
        for r, row in enumerate(self.step_calls):
            brow = []
            self._douts.append([])
            for h in range(len(row)):
                x = self._bound_inputs[r][h]["x"]
                g = torch.Generator(device="cuda")
                g.manual_seed(5000 + 7 * r + h)
                dout = torch.randn(x.shape, generator=g, device="cuda").to(x.dtype)
                self._douts[r].append(dout)
                inp_args = self._bound_inputs[r][h]
                bc = r2l.bind_backward(x, inp_args["dt"], inp_args["Bm"], inp_args["Cm"],
                                       inp_args["A"], inp_args["Dskip"], dout=dout, res=x,
                                       s=float(self.gates[h]))
                brow.append(bc)
                if r == 0:
                    self.bwd_grads.append((h, dout, bc.grads))
            self.bwd_calls.append(brow)
        self.step_calls = self.bwd_calls
        self.measure = [dict(label="r2l_scan_backward (one hook)",
                             calls=[c for row in self.bwd_calls for c in row],
                             bytes=self.bytes_per_launch, alu=self.alu_per_launch,
                             tc=self.tc_per_launch)]
        self.config = dict(self.config, workload=self.name, op="r2l_scan_backward",
                           grads=list(r2l.GRADS))

    def cpu_baseline(self, budget_s, nthreads=0, parity=None):
        import oracle
        tc, secs, hooks = 0, 0.0, 0
        while secs < budget_s and hooks < 7 * 20:
            h, dout, grads = self.bwd_grads[hooks % len(self.bwd_grads)]
            inp = self.inputs[h]
            t = {}
            ref = oracle.selective_scan_backward(
                inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, reverse=True,
                dout=dout.float().cpu().numpy().reshape(inp.x.shape), res_kind="x",
                s=float(self.gates[h]), seq_offsets=inp.offsets, timing=t, nthreads=nthreads)
            if parity is not None and hooks < len(self.bwd_grads):
                parity.add(grads["dA"].cpu().numpy(), ref["dA"])
                parity.add(grads["dBm"].cpu().numpy().reshape(ref["dBm"].shape), ref["dBm"])
            secs += t["seconds"]
            tc += inp.x.size
            hooks += 1
        return {"value": tc / secs, "unit": "tokens*channels/s",
                "cores": nthreads or oracle.max_threads(), "kind": "oracle",
                "sample": "%d hook backwards (%d token-channels), %.1f s of oracle time"
                          % (hooks, tc, secs)}

    parity_spec = ("dA, dBm", "f32", 1e-4,
                   "dA and dBm of all 7 hooks (first buffer set) vs the oracle's fp64 backward")


class DenoiseTrain(DenoiseBackward):
    """Training the R2L stream over one denoising step: per hook, the forward
    that saves the backward's state checkpoints (r2l_scan_save, out = x + s*y)
    and the backward from them (r2l_scan_backward_saved, all gradients); 7
    hooks of 64 x 32 x 2048, bf16. The unsaved pair (r2l_scan, then
    r2l_scan_backward, whose state pass rescans the forward) is the
    "denoise" and "denoise_bwd" workloads."""
    name = "denoise_train_bf16_b64_blk32_D2048_N16_7hooks"
    # an event between every call of this step costs ~2.6 us per call (the
    # eager step with them against the graph-replayed step without them), so
    # each entry point is timed again in a loop of its own calls
    isolate_entries = True

    def setup(self, torch, r2l):
        super().setup(torch, r2l)
        tok = self.B * self.L
        # checkpoint rows written (and read back): one per started group of 8
        # visited tokens of each sequence (the buffer also holds one unused
        # row per sequence and one more, which are not traffic)
        ck_bytes = self.B * ((self.L + 7) // 8) * self.D * 16 * 4
        fwd_bytes = scan_bytes(tok, self.D, 2, readout=True) + ck_bytes
        bwd_bytes = self.bytes_per_launch + ck_bytes
        fwd_alu = self.tc_per_launch * alu_ops_per_tc(True, True)
        # the backward's algorithmic work without the forward states, which the
        # saving forward computed already
        bwd_alu = self.tc_per_launch * (bwd_alu_ops_per_tc() - alu_ops_per_tc(False, False))
        self.step_calls, self.train_grads = [], []
        save_calls, bwd_calls = [], []
        for r in range(self.R):
            row = []
            for h in range(self.HOOKS):
                ins = self._bound_inputs[r][h]
                x = ins["x"]
                sc = r2l.bind("r2l_scan_save", x=x, res=x, s=float(self.gates[h]),
                              out=self.outs0[h] if r == 0 else torch.empty_like(x),
                              **{k: v for k, v in ins.items() if k != "x"})
                bc = r2l.bind_backward(x, ins["dt"], ins["Bm"], ins["Cm"], ins["A"],
                                       ins["Dskip"], dout=self._douts[r][h], res=x,
                                       s=float(self.gates[h]), ckpt=sc.ckpt)
                row += [sc, bc]
                save_calls.append(sc)
                bwd_calls.append(bc)
                if r == 0:
                    self.train_grads.append((h, self._douts[r][h], bc.grads))
            self.step_calls.append(row)
        self.bwd_calls = None
        self.bwd_grads = self.train_grads
        self.step_entries = [0, 1] * self.HOOKS
        self.launches_per_step = 2 * self.HOOKS
        self.measure = [dict(label="r2l_scan_save (one hook)", calls=save_calls,
                             bytes=fwd_bytes, alu=fwd_alu, tc=self.tc_per_launch),
                        dict(label="r2l_scan_backward_saved (one hook)", calls=bwd_calls,
                             bytes=bwd_bytes, alu=bwd_alu, tc=self.tc_per_launch)]
        self.config = dict(self.config, workload=self.name,
                           op="r2l_scan_save + r2l_scan_backward_saved",
                           checkpoint_bytes_per_hook=ck_bytes)

    def cpu_baseline(self, budget_s, nthreads=0, parity=None):
        import oracle
        if parity is not None:   # the saving forward's outputs of the first buffer set
            fwd = Parity("out", "bf16", 2e-2)
            for h, inp in enumerate(self.inputs):
                r = oracle.selective_scan(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip,
                                          reverse=True, res=inp.x, s=float(self.gates[h]),
                                          seq_offsets=inp.offsets, want_y=False,
                                          want_out=True, nthreads=nthreads)
                fwd.add(self.outs0[h].float().cpu().numpy().reshape(r["out"].shape), r["out"])
            self.parity_extra = dict(fwd.result(), sample="out = x + s*y of all 7 hooks "
                                     "(first buffer set) vs the oracle's")
        return super().cpu_baseline(budget_s, nthreads, parity)

    parity_spec = ("dA, dBm", "f32", 1e-4,
                   "dA and dBm of the backward from the saved checkpoints, all 7 hooks (first "
                   "buffer set) vs the oracle's fp64 backward; the forward's out in 'forward'")


class DenoiseL2R(Denoise):
    """The L2R-Mamba ablation of the same step: 7 hooked forward scans with readout and
    gated residual (prefix_scan_state with Cm, res and out), 64 x 32 x 2048, bf16."""
    name = "l2r_ablation_step_bf16_b64_blk32_D2048_N16_7hooks"
    reverse = False
    entry = "prefix_scan_state"


def sleep_cycles_per_ms(torch):
    """Calibrate torch.cuda._sleep (a spinning kernel) in cycles per millisecond."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    a.record()
    torch.cuda._sleep(2_000_000)
    b.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(a.elapsed_time(b), 1e-3)


def device_inputs(torch, key, lengths, D, dtype):
    """Seeded inputs drawn on the GPU (same distributions as synth) for the large
    workloads: x ~ N(0,1), dt ~ N(-2, 0.5), Bm, Cm ~ N(0,1), A = -(n+1), Dskip ~ N(0,1)."""
    import numpy as np
    tok = int(np.sum(lengths))
    g = torch.Generator(device="cuda")
    g.manual_seed(int(key))
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.randn((tok, D), generator=g, device="cuda").to(td)
    dt = (torch.randn((tok, D), generator=g, device="cuda") * 0.5 - 2.0).to(td)
    Bm = torch.randn((tok, 16), generator=g, device="cuda").to(td)
    Cm = torch.randn((tok, 16), generator=g, device="cuda").to(td)
    A = -(torch.arange(16, device="cuda", dtype=torch.float32) + 1).repeat(D, 1).contiguous()
    Dskip = torch.randn((D,), generator=g, device="cuda")
    return {"x": x, "dt": dt, "Bm": Bm, "Cm": Cm, "A": A, "Dskip": Dskip}


def oracle_sample_rate(torch, g, offsets, seqs, budget_s, reverse=True, readout=True,
                       nthreads=0, parity=None, got=None):
    """Oracle token·channels/s over the listed sequences (copied back from the GPU).
    With `parity`, the GPU result `got` (token-major y, or [batch, D, N] states
    when not `readout`) of each sampled sequence is compared with the oracle's."""
    import numpy as np
    import oracle
    tc, secs = 0, 0.0
    for b in seqs:
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        x = g["x"][r0:r1].float().cpu().numpy()
        dt = g["dt"][r0:r1].float().cpu().numpy()
        Bm = g["Bm"][r0:r1].float().cpu().numpy()
        Cm = g["Cm"][r0:r1].float().cpu().numpy() if readout else None
        t = {}
        r = oracle.selective_scan(x, dt, Bm, Cm, g["A"].cpu().numpy(), g["Dskip"].cpu().numpy(),
                                  reverse=reverse, seq_offsets=np.array([0, r1 - r0]),
                                  want_y=readout, want_h_out=not readout, timing=t,
                                  nthreads=nthreads)
        if parity is not None:
            if readout:
                parity.add(got[r0:r1].float().cpu().numpy(), r["y"])
            else:
                parity.add(got[b].cpu().numpy(), r["h_out"][0])
        secs += t["seconds"]
        tc += x.size
        if secs >= budget_s:
            break
    return tc / secs, tc, secs


class Prefill(Workload):
    """Full reverse scan, 8 x 4096 x 4096, bf16, out = y."""
    name = "prefill_r2l_bf16_b8_L4096_D4096_N16"
    B, L, D = 8, 4096, 4096

    def setup(self, torch, r2l):
        import numpy as np
        self.torch = torch
        self.g = device_inputs(torch, 103, [self.L] * self.B, self.D, "bf16")
        tok = self.B * self.L
        self.offsets = np.arange(self.B + 1) * self.L
        self.tc_per_launch = tok * self.D
        self.tc_per_step = self.tc_per_launch
        self.bytes_per_launch = scan_bytes(tok, self.D, 2, readout=True)
        self.alu_per_launch = self.tc_per_launch * alu_ops_per_tc(True, False)
        self.launches_per_step = 1
        g = self.g
        view = lambda t: t.view(self.B, self.L, -1)
        self.R = _rotation(self.bytes_per_launch)
        self.calls = []
        for r in range(self.R):
            src = g if r == 0 else {k: v.clone() for k, v in g.items()}
            out = torch.empty_like(view(src["x"]))
            if r == 0:
                self.out0 = out.view(tok, self.D)
            self.calls.append(r2l.bind("r2l_scan", x=view(src["x"]), dt=view(src["dt"]),
                                       Bm=view(src["Bm"]), Cm=view(src["Cm"]), A=g["A"],
                                       Dskip=g["Dskip"], out=out))
        self.step_calls = [[c] for c in self.calls]
        self.measure = [dict(label="r2l_scan", calls=self.calls, bytes=self.bytes_per_launch,
                             alu=self.alu_per_launch, tc=self.tc_per_launch)]
        self.config = {"workload": self.name, "batch": self.B, "seqlen": self.L, "D": self.D,
                       "N": 16, "in_dtype": "bf16", "state_dtype": "fp32", "res": None,
                       "rotating_sets": self.R, "parallelism": "single_gpu",
                       "plan": self.calls[0].plan()}

    def cpu_baseline(self, budget_s, nthreads=0, parity=None):
        import oracle
        rate, tc, secs = oracle_sample_rate(self.torch, self.g, self.offsets, range(self.B),
                                            budget_s, nthreads=nthreads, parity=parity,
                                            got=self.out0)
        return {"value": rate, "unit": "tokens*channels/s",
                "cores": nthreads or oracle.max_threads(), "kind": "oracle",
                "sample": "%d of the %d sequences (%d token-channels), %.1f s"
                % (tc // (self.L * self.D), self.B, tc, secs)}

    parity_spec = ("y", "bf16", 2e-2, "y of the sampled sequences (first buffer set)")


class PrefillBackward(Prefill):
    """The backward of the prefill-shape reverse scan (8 x 4096 x 4096, bf16, out = y):
    the training shape of the R2L stream at the expanded width, all gradients."""
    name = "prefill_backward_bf16_b8_L4096_D4096_N16"

    def setup(self, torch, r2l):
        import numpy as np
        super().setup(torch, r2l)
        tok, N = self.B * self.L, 16
        g = self.g
        view = lambda t: t.view(self.B, self.L, -1)   # noqa: E731
        gen = torch.Generator(device="cuda")
        gen.manual_seed(7103)
        self.dout = torch.randn((tok, self.D), generator=gen, device="cuda").to(torch.bfloat16)
        # x, dt, dout in and dx, ddt out (bf16); Bm, Cm in (bf16) and dBm, dCm out (fp32);
        # A, Dskip in and dA, dDskip out
        self.bytes_per_launch = (tok * self.D * 2 * 5 + tok * N * (2 * 2 + 4 * 2) +
                                 self.D * N * 4 * 2 + self.D * 4 * 2)
        self.alu_per_launch = self.tc_per_launch * bwd_alu_ops_per_tc()
        self.R = 1   # 1.3 GB of inputs and outputs per call: HBM-resident, not cache-resident
        self.bcall = r2l.bind_backward(view(g["x"]), view(g["dt"]), view(g["Bm"]), view(g["Cm"]),
                                       g["A"], g["Dskip"], dout=view(self.dout))
        self.calls = [self.bcall]
        self.step_calls = [[self.bcall]]
        self.measure = [dict(label="r2l_scan_backward", calls=self.calls,
                             bytes=self.bytes_per_launch, alu=self.alu_per_launch,
                             tc=self.tc_per_launch)]
        self.config = {"workload": self.name, "batch": self.B, "seqlen": self.L, "D": self.D,
                       "N": 16, "in_dtype": "bf16", "state_dtype": "fp32", "res": None,
                       "op": "r2l_scan_backward", "grads": ["dx", "ddt", "dBm", "dCm", "dA",
                                                            "dDskip", "dh_in"],
                       "parallelism": "single_gpu"}

    def cpu_baseline(self, budget_s, nthreads=0, parity=None):
        import numpy as np
        import oracle
        torch = self.torch
        L, D = self.L, self.D
        tc, secs, n = 0, 0.0, 0
        grads = self.bcall.grads
        for b in range(self.B):     # whole sequences, until the budget is spent
            if secs >= budget_s:
                break
            rows = slice(b * L, (b + 1) * L)
            host = lambda t: t[rows].float().cpu().numpy()   # noqa: E731
            t = {}
            ref = oracle.selective_scan_backward(
                host(self.g["x"]), host(self.g["dt"]), host(self.g["Bm"]), host(self.g["Cm"]),
                self.g["A"].cpu().numpy(), self.g["Dskip"].cpu().numpy(), reverse=True,
                dout=host(self.dout), batch=1, seqlen=L, timing=t, nthreads=nthreads)
            if parity is not None:
                parity.add(grads["dx"].reshape(-1, D)[rows].float().cpu().numpy(), ref["dx"])
                parity.add(grads["ddt"].reshape(-1, D)[rows].float().cpu().numpy(), ref["ddt"])
            secs += t["seconds"]
            tc += L * D
            n += 1
        return {"value": tc / secs, "unit": "tokens*channels/s",
                "cores": nthreads or oracle.max_threads(), "kind": "oracle",
                "sample": "%d of the %d sequences (%d token-channels), %.1f s of oracle time"
                          % (n, self.B, tc, secs)}

    parity_spec = ("dx, ddt", "bf16", 2e-2,
                   "dx and ddt of the sampled sequences vs the oracle's fp64 backward")


class PrefillTrain(PrefillBackward):
    """Training the R2L stream at the prefill shape (8 x 4096 x 4096, bf16, out =
    y): the forward that saves the backward's checkpoints (r2l_scan_save) and the
    backward from them (r2l_scan_backward_saved), all gradients. The unsaved
    pair is the "prefill" and "prefill_bwd" workloads."""
    name = "prefill_train_bf16_b8_L4096_D4096_N16"
    isolate_entries = True

    def setup(self, torch, r2l):
        super().setup(torch, r2l)
        g = self.g
        tok, N = self.B * self.L, 16
        view = lambda t: t.view(self.B, self.L, -1)   # noqa: E731
        # checkpoint rows written and read back: one per started group of 8
        ck_bytes = self.B * ((self.L + 7) // 8) * self.D * N * 4
        self.out_save = torch.empty_like(view(g["x"]))
        sc = r2l.bind("r2l_scan_save", x=view(g["x"]), dt=view(g["dt"]), Bm=view(g["Bm"]),
                      Cm=view(g["Cm"]), A=g["A"], Dskip=g["Dskip"], out=self.out_save)
        self.bcall = r2l.bind_backward(view(g["x"]), view(g["dt"]), view(g["Bm"]), view(g["Cm"]),
                                       g["A"], g["Dskip"], dout=view(self.dout), ckpt=sc.ckpt)
        self.step_calls = [[sc, self.bcall]]
        self.step_entries = [0, 1]
        self.launches_per_step = 2
        fwd_alu = self.tc_per_launch * alu_ops_per_tc(True, False)
        bwd_alu = self.tc_per_launch * (bwd_alu_ops_per_tc() - alu_ops_per_tc(False, False))
        self.measure = [dict(label="r2l_scan_save", calls=[sc],
                             bytes=scan_bytes(tok, self.D, 2, readout=True) + ck_bytes,
                             alu=fwd_alu, tc=self.tc_per_launch),
                        dict(label="r2l_scan_backward_saved", calls=[self.bcall],
                             bytes=self.bytes_per_launch + ck_bytes, alu=bwd_alu,
                             tc=self.tc_per_launch)]
        self.config = dict(self.config, workload=self.name,
                           op="r2l_scan_save + r2l_scan_backward_saved",
                           checkpoint_bytes=ck_bytes)

    parity_spec = ("dx, ddt", "bf16", 2e-2,
                   "dx and ddt of the backward from the saved checkpoints, sampled sequences, "
                   "vs the oracle's fp64 backward")


class RaggedServing(Workload):
    """256 ragged blocks of U{16..64} tokens at D = 4096, bf16: the reverse scan over
    the active blocks and block_commit_state over the committed blocks."""
    name = "ragged_serving_bf16_b256_blk16to64_D4096_N16"
    D = 4096

    def setup(self, torch, r2l):
        import numpy as np
        import synth
        self.torch = torch
        lens = synth.ragged_block_lengths()
        self.offsets = synth.offsets(lens)
        tok = int(self.offsets[-1])
        self.g = device_inputs(torch, 104, lens, self.D, "bf16")
        self.gc = device_inputs(torch, 1104, lens, self.D, "bf16")
        cu = torch.from_numpy(self.offsets.astype(np.int32)).cuda()
        B = len(lens)
        self.tc_per_launch = tok * self.D
        self.tc_per_step = 2 * tok * self.D
        self.bytes_per_launch = scan_bytes(tok, self.D, 2, readout=True)
        self.commit_bytes = scan_bytes(tok, self.D, 2, readout=False, batch=B, state_rw=True)
        self.alu_per_launch = self.tc_per_launch * alu_ops_per_tc(True, False)
        self.launches_per_step = 1
        self.R = _rotation(self.bytes_per_launch + self.commit_bytes)
        self.calls = []
        for r in range(self.R):
            g = self.g if r == 0 else {k: v.clone() for k, v in self.g.items()}
            gc = self.gc if r == 0 else {k: v.clone() for k, v in self.gc.items()}
            out = torch.empty_like(g["x"])
            if r == 0:
                self.out0 = out
            state = torch.randn((B, self.D, 16), device="cuda")
            scan = r2l.bind("r2l_scan", x=g["x"], dt=g["dt"], Bm=g["Bm"], Cm=g["Cm"], A=g["A"],
                            Dskip=g["Dskip"], out=out, cu_seqlens=cu, max_seqlen=int(lens.max()))
            commit = r2l.bind("block_commit_state", state=state, x=gc["x"], dt=gc["dt"],
                              Bm=gc["Bm"], A=gc["A"], cu_seqlens=cu, max_seqlen=int(lens.max()))
            self.calls.append((scan, commit))
        self.step_calls = [list(sc) for sc in self.calls]
        self.step_entries = [0, 1]
        self.measure = [
            dict(label="r2l_scan (ragged blocks)", calls=[sc[0] for sc in self.calls],
                 bytes=self.bytes_per_launch, alu=self.alu_per_launch, tc=self.tc_per_launch),
            dict(label="block_commit_state (ragged blocks)", calls=[sc[1] for sc in self.calls],
                 bytes=self.commit_bytes, alu=self.tc_per_launch * alu_ops_per_tc(False, False),
                 tc=self.tc_per_launch)]
        self.config = {"workload": self.name, "batch": B, "tokens": tok, "D": self.D, "N": 16,
                       "block_len": "U{16..64}", "in_dtype": "bf16", "state_dtype": "fp32",
                       "ops": ["r2l_scan (out = y)", "block_commit_state (in place)"],
                       "rotating_sets": self.R, "parallelism": "single_gpu"}

    def cpu_baseline(self, budget_s, nthreads=0, parity=None):
        import oracle
        rate, tc, secs = oracle_sample_rate(self.torch, self.g, self.offsets,
                                            range(len(self.offsets) - 1), budget_s,
                                            nthreads=nthreads, parity=parity, got=self.out0)
        return {"value": rate, "unit": "tokens*channels/s",
                "cores": nthreads or oracle.max_threads(), "kind": "oracle",
                "sample": "reverse scan of the first sequences (%d token-channels), %.1f s"
                % (tc, secs)}

    parity_spec = ("y", "bf16", 2e-2,
                   "y of the reverse scan over the sampled blocks (first buffer set)")


class RaggedPrefix(Workload):
    """prefix_scan_state over 256 ragged prefixes of U{256..8192} tokens at D = 4096."""
    name = "ragged_prefix_state_bf16_b256_P256to8192_D4096_N16"
    D = 4096

    def setup(self, torch, r2l):
        import numpy as np
        import synth
        self.torch = torch
        lens = synth.ragged_prefix_lengths()
        self.offsets = synth.offsets(lens)
        tok = int(self.offsets[-1])
        B = len(lens)
        self.g = device_inputs(torch, 2104, lens, self.D, "bf16")
        cu = torch.from_numpy(self.offsets.astype(np.int32)).cuda()
        self.tc_per_launch = tok * self.D
        self.tc_per_step = self.tc_per_launch
        self.bytes_per_launch = scan_bytes(tok, self.D, 2, readout=False, batch=B, h_out=True)
        self.alu_per_launch = self.tc_per_launch * alu_ops_per_tc(False, False)
        self.launches_per_step = 1
        self.R = 1  # 17.8 GB per launch: far beyond every cache
        h = torch.empty((B, self.D, 16), device="cuda")
        self.h = h
        g = self.g
        self.calls = [r2l.bind("prefix_scan_state", x=g["x"], dt=g["dt"], Bm=g["Bm"], A=g["A"],
                               h_out=h, cu_seqlens=cu, max_seqlen=int(lens.max()))]
        self.step_calls = [self.calls]
        self.measure = [dict(label="prefix_scan_state (ragged prefill)", calls=self.calls,
                             bytes=self.bytes_per_launch, alu=self.alu_per_launch,
                             tc=self.tc_per_launch)]
        self.config = {"workload": self.name, "batch": B, "tokens": tok, "D": self.D, "N": 16,
                       "prefix_len": "U{256..8192}", "in_dtype": "bf16", "state_dtype": "fp32",
                       "parallelism": "single_gpu",
                       "plan": self.calls[0].plan()}

    def cpu_baseline(self, budget_s, nthreads=0, parity=None):
        import oracle
        rate, tc, secs = oracle_sample_rate(self.torch, self.g, self.offsets,
                                            range(len(self.offsets) - 1), budget_s,
                                            reverse=False, readout=False, nthreads=nthreads,
                                            parity=parity, got=self.h)
        return {"value": rate, "unit": "tokens*channels/s",
                "cores": nthreads or oracle.max_threads(), "kind": "oracle",
                "sample": "prefix states of the first prefixes (%d token-channels), %.1f s"
                % (tc, secs)}

    parity_spec = ("h_out", "f32", 1e-5, "final state of the sampled prefixes")


class DenoiseBidir(Denoise):
    """The full-window bidirectional variant of the same step: 7 hooked bidir_scan
    calls over the denoising window (forward scan + reverse scan of x, each
    direction with its own dt, Bm, Cm, A, Dskip, readouts added, gated residual
    in place), 64 x 32 x 2048, bf16."""
    name = "bidir_window_step_bf16_b64_L32_D2048_N16_7hooks"
    entry = "bidir_scan"

    def setup(self, torch, r2l):
        import synth
        self.torch = torch
        self.gates = synth.bidir_gates()
        self.inputs = [synth.bidir_inputs(h) for h in range(self.HOOKS)]
        self.revs = [synth.bidir_reverse(h) for h in range(self.HOOKS)]
        tok = self.B * self.L
        N = 16
        self.tc_per_launch = tok * self.D
        self.tc_per_step = self.tc_per_launch * self.HOOKS
        # x, out; dt of each direction (bf16); Bm, Cm of each direction; A, Dskip of each
        self.bytes_per_launch = (tok * self.D * 2 * 4 + tok * N * 2 * 4 +
                                 2 * (self.D * N * 4 + self.D * 4))
        # the reverse readout, then the forward readout with the residual and the sum
        self.alu_per_launch = self.tc_per_launch * (alu_ops_per_tc(True, False) +
                                                    alu_ops_per_tc(True, True) + 1)
        self.launches_per_step = self.HOOKS
        set_bytes = self.bytes_per_launch * self.HOOKS
        self.R = _rotation(set_bytes)
        self.step_calls, self.outs0 = [], []
        shape = lambda t: t.view(self.B, self.L, -1)   # noqa: E731
        for r in range(self.R):
            row = []
            for h, (inp, rv) in enumerate(zip(self.inputs, self.revs)):
                x = shape(_dev(torch, inp.x, "bf16"))
                ins = {k: shape(_dev(torch, getattr(inp, k), "bf16")) for k in ("dt", "Bm", "Cm")}
                ins["A"] = torch.from_numpy(inp.A).cuda()
                ins["Dskip"] = torch.from_numpy(inp.Dskip).cuda()
                rev = {k: shape(_dev(torch, rv[k], "bf16")) for k in ("dt", "Bm", "Cm")}
                rev["A"] = torch.from_numpy(rv["A"]).cuda()
                rev["Dskip"] = torch.from_numpy(rv["Dskip"]).cuda()
                out = torch.empty_like(x)
                if r == 0:
                    self.outs0.append(out)
                row.append(r2l.bind("bidir_scan", x=x, res=x, s=float(self.gates[h]), out=out,
                                    rev=rev, **ins))
            self.step_calls.append(row)
        self.step_entries = [0] * self.HOOKS
        self.measure = [dict(label="bidir_scan (one hook)",
                             calls=[c for row in self.step_calls for c in row],
                             bytes=self.bytes_per_launch, alu=self.alu_per_launch,
                             tc=self.tc_per_launch)]
        self.config = {"workload": self.name, "batch": self.B, "window_tokens": self.L,
                       "D": self.D, "N": 16, "hooks_per_step": self.HOOKS,
                       "in_dtype": "bf16", "state_dtype": "fp32", "res": "x",
                       "reverse_parameters": "separate", "op": "bidir_scan",
                       "rotating_sets": self.R, "rotating_bytes": set_bytes * self.R,
                       "parallelism": "single_gpu"}

    def cpu_baseline(self, budget_s, nthreads=0, parity=None):
        import oracle
        tc, secs, reps, hooks = 0, 0.0, 0, 0
        while secs < budget_s and reps < 200:
            for h, (inp, rv) in enumerate(zip(self.inputs, self.revs)):
                t = {}
                r = oracle.bidir_scan(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, rev=rv,
                                      res=inp.x, s=float(self.gates[h]), seq_offsets=inp.offsets,
                                      timing=t, nthreads=nthreads)
                if parity is not None and reps == 0:
                    parity.add(self.outs0[h].float().cpu().numpy().reshape(r["out"].shape),
                               r["out"])
                secs += t["seconds"]
                tc += inp.x.size
                hooks += 1
                if nthreads == 1 and secs >= budget_s:
                    break
            reps += 1
        return {"value": tc / secs, "unit": "tokens*channels/s",
                "cores": nthreads or oracle.max_threads(), "kind": "oracle",
                "sample": "%d bidirectional hooks of the 7-hook step (%d token-channels), "
                          "%.1f s of oracle time" % (hooks, tc, secs)}

    parity_spec = ("out", "bf16", 2e-2,
                   "out = x + s*(y_forward + y_reverse) of all 7 hooks (first buffer set) vs "
                   "the oracle's")


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


class DenoiseSidecar(Denoise):
    """The denoising step with the whole sidecar block per hook (r2l_sidecar_forward):
    in-projection, conv + SiLU, x/dt projections, the gated R2L scan, out-projection
    with the s-gated residual, 7 hooks over 64 x 32 tokens at d_model 2048,
    d_inner 4096, bf16."""
    name = "sidecar_step_bf16_b64_blk32_dm2048_di4096_N16_7hooks"
    DM, DI, R = 2048, 4096, 128
    # library GEMMs may record memsets (split-K scratch) that graph replays do
    # not repeat reliably here: eager launches only
    graph_ok = False

    def setup(self, torch, r2l):
        import synth
        self.torch = torch
        self.hooks = [synth.sidecar_hook(h) for h in range(self.HOOKS)]
        tok = self.B * self.L
        N = 16
        self.tc_per_launch = tok * self.DI          # token-channels of the scan inside
        self.tc_per_step = self.tc_per_launch * self.HOOKS
        dm, di, R = self.DM, self.DI, self.R
        self.gemm_flops = 2 * tok * (dm * 2 * di + di * (R + 2 * N) + R * di + di * dm)
        # bytes: hidden in, out; the four weights; conv, dt bias, A, Dskip
        self.bytes_per_launch = (tok * dm * 2 * 2 + 2 * (2 * di * dm + (R + 2 * N) * di +
                                                         di * R + dm * di) +
                                 4 * (di * 4 + di + di * N + di + di))
        self.alu_per_launch = self.tc_per_launch * alu_ops_per_tc(True, False)
        self.launches_per_step = self.HOOKS
        set_bytes = self.bytes_per_launch * self.HOOKS
        self.R = _rotation(set_bytes)
        self.step_calls, self.outs0 = [], []
        weights = []
        for hid, w, s in self.hooks:
            weights.append({k: (torch.from_numpy(v).cuda() if k in
                                ("conv_w", "conv_b", "dt_bias", "A", "Dskip")
                                else _dev(torch, v, "bf16")) for k, v in w.items()})
        ws = None
        for r in range(self.R):
            row = []
            for h, (hid, w, s) in enumerate(self.hooks):
                x = _dev(torch, hid, "bf16").view(self.B, self.L, -1)
                out = torch.empty_like(x)
                if r == 0:
                    self.outs0.append(out)
                call = r2l.bind_sidecar(x, weights[h], s=s, out=out, workspace=ws)
                ws = call.workspace          # one workspace serves every call (stream-ordered)
                if r == 0 and h == 0:
                    call.tune()              # time the GEMM candidates once (shared shapes)
                row.append(call)
            self.step_calls.append(row)
        self.step_entries = [0] * self.HOOKS
        self.measure = [dict(label="r2l_sidecar_forward (one hook)",
                             calls=[c for row in self.step_calls for c in row],
                             bytes=self.bytes_per_launch, alu=self.alu_per_launch,
                             tc=self.tc_per_launch, flops=self.gemm_flops)]
        self.config = {"workload": self.name, "batch": self.B, "block_tokens": self.L,
                       "d_model": dm, "d_inner": di, "N": 16, "dt_rank": R, "d_conv": 4,
                       "hooks_per_step": self.HOOKS, "in_dtype": "bf16", "state_dtype": "fp32",
                       "op": "r2l_sidecar_forward", "rotating_sets": self.R,
                       "rotating_bytes": set_bytes * self.R, "parallelism": "single_gpu",
                       "weights": "random init (synthetic)"}

    def cpu_baseline(self, budget_s, nthreads=0, parity=None):
        import numpy as np
        import oracle
        tc, secs, hooks = 0, 0.0, 0
        while secs < budget_s and hooks < 7 * 5:
            h = hooks % self.HOOKS
            hid, w, s = self.hooks[h]
            t = {}
            r = oracle.sidecar_forward(hid, w["W_in"], w["conv_w"], w["conv_b"], w["W_x"],
                                       w["W_dt"], w["dt_bias"], w["A"], w["Dskip"], w["W_out"],
                                       s=s, batch=self.B, seqlen=self.L, store="bf16",
                                       nthreads=nthreads, timing=t)
            if parity is not None and hooks < self.HOOKS:
                # bar of the sidecar's GPU tests: one bf16 ulp + 2e-2 * max|s * o|
                parity.add(self.outs0[h].float().cpu().numpy().reshape(r["out"].shape), r["out"],
                           slack=2e-2 * float(np.max(np.abs(s * r["o"]))))
            secs += t["seconds"]
            tc += self.tc_per_launch
            hooks += 1
        return {"value": tc / secs, "unit": "tokens*channels/s",
                "cores": nthreads or oracle.max_threads(), "kind": "oracle",
                "sample": "%d sidecar hooks (%d scan token-channels), %.1f s of oracle time "
                          "(numpy fp64 projections on the host's BLAS threads, C scan)"
                          % (hooks, tc, secs)}

    parity_spec = ("out", "bf16", 2e-2,
                   "out = hidden + s * sidecar(hidden) of all 7 hooks (first buffer set) vs the "
                   "oracle's (intermediates rounded to bf16 where the GPU stores them); element "
                   "bound: one bf16 ulp + 2e-2 * max|s * o|, as in the sidecar's GPU tests")


class _Call:
    """A unit of a step that bench.py's timing loop launches: ``fn(stream)``."""

    def __init__(self, fn):
        self.fn = fn

    def launch(self, stream):
        self.fn(stream)


class StubBackbone:
    """A causal decoder stub shaped like Qwen3-1.7B (pre-norm RMSNorm, grouped-query
    attention, SiLU-gated MLP; random weights, no rotary embedding) with a KV
    cache, in plain torch on any device and dtype. ``forward(h, at, hooks)``
    runs every layer on h [B, T, dm] in place for the tokens at cache positions
    [at, at + T): their keys and values go to the cache and each query attends
    causally over the cache up to its own position; after layer l, hooks[l](h)
    (if given) updates h in place — the R2L sidecar hooks. Only timing and the
    hooks' inputs depend on this stub."""

    def __init__(self, torch, *, layers, dm, hq, hkv, hd, ff, batch, max_tokens, device, dtype,
                 seed):
        self.torch = torch
        self.layers, self.DM, self.HQ, self.HKV, self.HD, self.FF = layers, dm, hq, hkv, hd, ff
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)

        def w(i, o):
            return (torch.randn((i, o), generator=gen, device=device, dtype=torch.float32)
                    / math.sqrt(i)).to(dtype)

        nq, nkv = hq * hd, hkv * hd
        self.W = [{"ln1": torch.ones(dm, dtype=dtype, device=device),
                   "ln2": torch.ones(dm, dtype=dtype, device=device),
                   "qkv": w(dm, nq + 2 * nkv), "o": w(nq, dm),
                   "gate": w(dm, ff), "up": w(dm, ff), "down": w(ff, dm)}
                  for _ in range(layers)]
        self.Kt = [torch.zeros((batch, hkv, hd, max_tokens), dtype=dtype, device=device)
                   for _ in range(layers)]
        self.V = [torch.zeros((batch, hkv, max_tokens, hd), dtype=dtype, device=device)
                  for _ in range(layers)]

    def cache_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.Kt + self.V)

    def layer(self, l, h, at, q_chunk=None):
        """Layer l on h [B, T, DM] in place, the tokens at cache positions
        [at, at + T); queries in chunks of q_chunk tokens (memory only)."""
        torch = self.torch
        import torch.nn.functional as F
        W = self.W[l]
        B, T, _ = h.shape
        g = self.HQ // self.HKV
        acc = torch.promote_types(h.dtype, torch.float32)      # the norms' accumulation type
        a = h.to(acc)
        a = (a * torch.rsqrt(a.pow(2).mean(-1, keepdim=True) + 1e-6)).to(h.dtype) * W["ln1"]
        qkv = torch.matmul(a, W["qkv"])                       # [B, T, (HQ + 2 HKV) HD]
        q = qkv[..., :self.HQ * self.HD].reshape(B, T, self.HKV, g, self.HD)
        k = qkv[..., self.HQ * self.HD:(self.HQ + self.HKV) * self.HD].reshape(B, T, self.HKV, self.HD)
        v = qkv[..., (self.HQ + self.HKV) * self.HD:].reshape(B, T, self.HKV, self.HD)
        Kt, V = self.Kt[l], self.V[l]                          # [B, HKV, HD, S], [B, HKV, S, HD]
        Kt[:, :, :, at:at + T] = k.permute(0, 2, 3, 1)
        V[:, :, at:at + T, :] = v.permute(0, 2, 1, 3)
        # queries grouped per key-value head, scaled: [B, HKV, T * g, HD] (token-major)
        qg = (q.permute(0, 2, 1, 3, 4).reshape(B, self.HKV, T * g, self.HD) *
              (self.HD ** -0.5)).contiguous()
        out = torch.empty((B, self.HKV, T * g, self.HD), dtype=h.dtype, device=h.device)
        step = T if q_chunk is None else q_chunk
        for c0 in range(0, T, step):
            c1 = min(T, c0 + step)
            end = at + c1                                      # keys visible to the chunk
            sc = torch.matmul(qg[:, :, c0 * g:c1 * g].contiguous(),
                              Kt[:, :, :, :end].contiguous())
            # only the chunk's own keys can lie in a query's future
            pos = torch.arange(c0, c1, device=h.device).repeat_interleave(g)
            keys = torch.arange(c0, c1, device=h.device)
            sc[..., at + c0:end].masked_fill_(keys[None, :] > pos[:, None], float("-inf"))
            pr = torch.softmax(sc, dim=-1)                     # fp32 inside for bf16
            out[:, :, c0 * g:c1 * g] = torch.matmul(pr, V[:, :, :end].contiguous())
        o = out.reshape(B, self.HKV, T, g, self.HD).permute(0, 2, 1, 3, 4).reshape(B, T, -1)
        h += torch.matmul(o, W["o"])
        m = h.to(acc)
        m = (m * torch.rsqrt(m.pow(2).mean(-1, keepdim=True) + 1e-6)).to(h.dtype) * W["ln2"]
        h += torch.matmul(F.silu(torch.matmul(m, W["gate"])) * torch.matmul(m, W["up"]), W["down"])

    def forward(self, h, at, hooks=None, q_chunk=None, mark=None):
        """Every layer on h in place (cache positions [at, at + T)), hooks[l](h)
        after layer l; mark(kind, l), if given, is called before each layer
        ("layer") and hook ("hook") and once at the end ("end", None)."""
        for l in range(self.layers):
            if mark:
                mark("layer", l)
            self.layer(l, h, at, q_chunk)
            if hooks and l in hooks:
                if mark:
                    mark("hook", l)
                hooks[l](h)
        if mark:
            mark("end", None)
        return h


class ServingStep(Workload):
    """A denoising step of the serving harness: a stub causal backbone shaped like
    Qwen3-1.7B (28 decoder layers, hidden 2048, 16 query / 8 key-value heads of
    128, MLP 6144; random weights, no rotary embedding) over a generation block of
    32 tokens for a batch of 8 whose 4096-token prompts were prefilled into a KV
    cache, with the sidecar block (r2l_sidecar_forward, d_inner 4096) hooked after
    every 4th layer. Prefill runs once in setup with the hooks active over each
    prompt (the R2L sidecar over the 4096 prompt tokens at every hooked layer), so
    the KV cache of the later layers holds keys and values of post-hook hidden
    states, and the post-hook hidden states of every hooked layer are kept as
    well; it is timed with an event before every layer and hook (prefill split
    between hooks and backbone). The timed step is the block's pass through all
    28 layers and 7 hooks, with an event before every layer group and hook, so
    that the hooks' share of the step is measured in place. The backbone is plain
    torch (matmuls on contiguous operands, softmax accumulating in fp32), its
    layers between two hooks replayed as one hipGraph; only the hooks are this
    library."""
    name = "serving_step_bf16_b8_P4096_blk32_qwen3-1.7b-stub_28L_7hooks"
    B, P, L = 8, 4096, 32
    DM, HQ, HKV, HD, FF, LAYERS, EVERY = 2048, 16, 8, 128, 6144, 28, 4
    DI, R = 4096, 128
    graph_ok = False

    def setup(self, torch, r2l):
        import synth
        self.torch = torch
        dev = "cuda"
        bf = torch.bfloat16
        self.bb = StubBackbone(torch, layers=self.LAYERS, dm=self.DM, hq=self.HQ, hkv=self.HKV,
                               hd=self.HD, ff=self.FF, batch=self.B, max_tokens=self.P + self.L,
                               device=dev, dtype=bf, seed=707)
        gen = torch.Generator(device=dev)
        gen.manual_seed(708)
        # the sidecar hooks (random init), one per hooked layer
        self.hook_layers = [l for l in range(self.LAYERS) if (l + 1) % self.EVERY == 0]
        self.hooks = []
        for j, l in enumerate(self.hook_layers):
            wt = synth.sidecar_weights(SERVING_KEY * 100 + j, self.DM, self.DI, self.R,
                                       dtype="bf16")
            wd = {k: (torch.from_numpy(v).cuda() if k in ("conv_w", "conv_b", "dt_bias", "A",
                                                          "Dskip") else _dev(torch, v, "bf16"))
                  for k, v in wt.items()}
            self.hooks.append((wt, wd, float(synth.gates(SERVING_KEY, 7, 0.0, 0.1)[j])))
        # Prefill: the prompts through every layer with the hooks active over them
        # (the R2L sidecar over each whole prompt), keys / values into the cache;
        # the post-hook hidden states of every hooked layer are kept. An event
        # before every layer and hook splits its time.
        prompt = torch.randn((self.B, self.P, self.DM), generator=gen, device=dev).to(bf)
        pws = None
        pre_hooks = {}
        for j, l in enumerate(self.hook_layers):
            wt, wd, s = self.hooks[j]
            c = r2l.bind_sidecar(prompt, wd, s=s, out=prompt, workspace=pws)
            pws = c.workspace
            pre_hooks[l] = c
        self.hook_states = {}

        def hook_at(l):
            def run(h):
                pre_hooks[l].launch(torch.cuda.current_stream().cuda_stream)
                self.hook_states[l] = h.clone()
            return run

        marks = []

        def mark(kind, l):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            marks.append((kind, e))

        for _ in range(2):   # the first pass warms up; the second is timed and kept
            for t in self.bb.Kt + self.bb.V:
                t.zero_()
            x = prompt.clone()
            marks.clear()
            torch.cuda.synchronize()
            self.bb.forward(x, 0, hooks={l: hook_at(l) for l in self.hook_layers}, q_chunk=512,
                            mark=mark)
            torch.cuda.synchronize()
        spans = [(marks[i][0], marks[i][1].elapsed_time(marks[i + 1][1]))
                 for i in range(len(marks) - 1)]
        self.prefill_ms = marks[0][1].elapsed_time(marks[-1][1])
        self.prefill_hooks_ms = sum(t for k, t in spans if k == "hook")
        self.prefill_backbone_ms = sum(t for k, t in spans if k == "layer")
        self.prefill_hook_in = None
        del x, prompt, pws, pre_hooks
        self.cache_gb = (self.bb.cache_bytes() + sum(t.numel() * t.element_size()
                                                     for t in self.hook_states.values())) / 1e9
        # rotating generation blocks (noisy-token embeddings stand-ins)
        self.R_sets = 4
        self.blocks = [torch.randn((self.B, self.L, self.DM), generator=gen, device=dev).to(bf)
                       for _ in range(self.R_sets)]
        self.h = torch.empty_like(self.blocks[0])
        ws = None
        self.bound = []
        for j in range(len(self.hook_layers)):
            wt, wd, s = self.hooks[j]
            c = r2l.bind_sidecar(self.h, wd, s=s, out=self.h, workspace=ws)
            ws = c.workspace
            if j == 0:
                c.tune()      # time the GEMM candidates once (every hook has these shapes)
            self.bound.append(c)
        self.R = self.R_sets
        # The stub's layers between two hooks replay as one hipGraph each (the
        # host would otherwise pace the ~25 small torch kernels of every layer);
        # the hooks launch eagerly in between. Only timing depends on the stub.
        starts = [0] + [l + 1 for l in self.hook_layers[:-1]]
        segs = [list(range(a, l + 1)) for a, l in zip(starts, self.hook_layers)]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):            # warm-up before capture
            self.h.copy_(self.blocks[0])
            for seg in segs:
                for l in seg:
                    self.bb.layer(l, self.h, self.P)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()

        def capture(fn):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            return g

        def run_seg(seg, r=None):
            if r is not None:
                self.h.copy_(self.blocks[r])
            for l in seg:
                self.bb.layer(l, self.h, self.P)

        first = [capture(lambda r=r: run_seg(segs[0], r)) for r in range(self.R_sets)]
        rest = [capture(lambda seg=seg: run_seg(seg)) for seg in segs[1:]]
        torch.cuda.synchronize()
        self._graphs = first + rest
        self.step_calls, entries = [], []
        for r in range(self.R_sets):
            row, ent = [], []
            for j in range(len(segs)):
                g = first[r] if j == 0 else rest[j - 1]
                row.append(_Call(lambda st, g=g: g.replay()))
                ent.append(1)
                row.append(self.bound[j])
                ent.append(0)
            self.step_calls.append(row)
            entries = ent
        self.step_entries = entries
        tok = self.B * self.L
        self.tc_per_launch = tok * self.DI
        self.tc_per_step = self.tc_per_launch * len(self.hook_layers)
        N, dm, di, R = 16, self.DM, self.DI, self.R
        flops = 2 * tok * (dm * 2 * di + di * (R + 2 * N) + R * di + di * dm)
        wbytes = 2 * (2 * di * dm + (R + 2 * N) * di + di * R + dm * di) + 4 * di * (4 + 3 + N)
        self.measure = [dict(label="r2l_sidecar_forward (one hook, in the step)",
                             calls=[c for row in self.step_calls for c in row if c in self.bound],
                             bytes=tok * dm * 2 * 2 + wbytes,
                             alu=self.tc_per_launch * alu_ops_per_tc(True, False),
                             tc=self.tc_per_launch, flops=flops),
                        dict(label="backbone: 4 stub layers between hooks (one hipGraph replay)",
                             calls=[], bytes=0, alu=0, tc=0)]
        # one hook's input and output inside a step, for parity against the oracle
        self.h.copy_(self.blocks[0])
        for l in range(self.LAYERS):
            self.bb.layer(l, self.h, self.P)
            if l == self.hook_layers[0]:
                self.hook_in = self.h.clone()
                self.bound[0].launch(torch.cuda.current_stream().cuda_stream)
                self.hook_out = self.h.clone()
                break
        torch.cuda.synchronize()
        self.config = {"workload": self.name, "batch": self.B, "prompt_tokens": self.P,
                       "block_tokens": self.L, "backbone": "stub: 28 layers, hidden 2048, 16/8 "
                       "heads x 128, MLP 6144, random init, no rotary", "hooks_per_step": 7,
                       "hook": "r2l_sidecar_forward (d_inner 4096, N 16, dt_rank 128, K 4)",
                       "in_dtype": "bf16", "prefill_ms": round(self.prefill_ms, 3),
                       "prefill_split_ms": {"hooks (7 x R2L sidecar over 8 x 4096 prompt "
                                            "tokens)": round(self.prefill_hooks_ms, 3),
                                            "backbone (28 stub layers)":
                                                round(self.prefill_backbone_ms, 3)},
                       "prefill_hook_share": round(self.prefill_hooks_ms / self.prefill_ms, 4),
                       "prefill_cache_gb": round(self.cache_gb, 3),
                       "prefill_cache": "K/V of all 28 layers over prompt + block slots (from "
                                        "post-hook hidden states after the first hook) and the "
                                        "post-hook hidden states of the 7 hooked layers",
                       "parallelism": "single_gpu", "weights": "random init (synthetic)"}

    def cpu_baseline(self, budget_s, nthreads=0, parity=None):
        import numpy as np
        import oracle
        hid = self.hook_in.float().cpu().numpy().reshape(-1, self.DM)
        wt, _, s = self.hooks[0]
        tc, secs, n = 0, 0.0, 0
        while secs < budget_s and n < 50:
            t = {}
            r = oracle.sidecar_forward(hid, wt["W_in"], wt["conv_w"], wt["conv_b"], wt["W_x"],
                                       wt["W_dt"], wt["dt_bias"], wt["A"], wt["Dskip"],
                                       wt["W_out"], s=s, batch=self.B, seqlen=self.L,
                                       store="bf16", nthreads=nthreads, timing=t)
            if parity is not None and n == 0:
                parity.add(self.hook_out.float().cpu().numpy().reshape(r["out"].shape), r["out"],
                           slack=2e-2 * float(np.max(np.abs(s * r["o"]))))
            secs += t["seconds"]
            tc += self.tc_per_launch
            n += 1
        return {"value": tc / secs, "unit": "tokens*channels/s",
                "cores": nthreads or oracle.max_threads(), "kind": "oracle",
                "sample": "%d runs of the first hook's sidecar block on its input inside a "
                          "step (%d scan token-channels), %.1f s of oracle time" % (n, tc, secs)}

    parity_spec = ("out", "bf16", 2e-2,
                   "the first hook's output inside a denoising step vs the oracle's sidecar "
                   "block on the same input; element bound one bf16 ulp + 2e-2 * max|s * o|")


SERVING_KEY = 107

WORKLOADS = {"denoise": Denoise, "prefill": Prefill, "ragged": RaggedServing,
             "prefix": RaggedPrefix, "l2r": DenoiseL2R, "denoise_bwd": DenoiseBackward,
             "bidir": DenoiseBidir, "sidecar": DenoiseSidecar, "serving": ServingStep,
             "prefill_bwd": PrefillBackward, "denoise_train": DenoiseTrain,
             "prefill_train": PrefillTrain}


def build_info() -> dict:
    """git commit and ROCm release of the build (where the tree has no .git,
    as on a machine the tree was copied to, the file the build wrote is
    read), torch's HIP version."""
    info = {"git_sha": None, "git_dirty": None, "git_sha_from": None, "rocm": None}
    try:
        import subprocess
        info["git_sha"] = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"],
                                         capture_output=True, text=True,
                                         check=True).stdout.strip()
        info["git_dirty"] = bool(subprocess.run(
            ["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
            capture_output=True, text=True, check=True).stdout.strip())
        info["git_sha_from"] = "git"
    except Exception:
        p = os.path.join(ROOT, "reverse_mamba_selective_amd", "BUILD_INFO.json")
        if os.path.exists(p):
            b = json.load(open(p))
            info.update(git_sha=b.get("git_sha"), git_dirty=b.get("git_dirty"),
                        git_sha_from="the library's build")
    try:
        info["rocm"] = open(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), ".info",
                                         "version")).read().strip()
    except OSError:
        pass
    try:
        import torch
        info["torch"] = torch.__version__
        info["torch_hip"] = torch.version.hip
    except Exception:
        pass
    return info


def alu_rates(blocks_per_cu=(1, 2, 4, 8), iters=4000, reps=5):
    """Issue rates of the vector ALU on this device (csrc/alu_rates.hip). Each
    kind runs 16 independent dependency chains per lane at 1, 2, 4 and 8 waves
    per SIMD (blocks of 4 waves, 1..8 blocks per CU, all resident at once).
    Thread 0 of every block reads the shader clock counter and the constant
    wall clock around its loop, which gives the shader clock the device ran at
    and the SIMD cycles per wave64 instruction (the block's loop cycles over
    the wave instructions its SIMD issued in that time). Slots are FMA issue
    slots: a transcendental's cycles over an FMA's, alone (kinds 1 and 3) and
    beside four FMAs (kind 2: its cycles minus those of the 65 other VALU
    instructions of the iteration, per exp)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "reverse_mamba_selective_amd", "libr2l_alu_rates.so"))
    lib.r2l_alu_rate_launch.restype = ctypes.c_int
    lib.r2l_alu_rate_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.r2l_alu_wall_clock_khz.restype = ctypes.c_int
    khz = ctypes.c_int(0)
    assert lib.r2l_alu_wall_clock_khz(ctypes.byref(khz)) == 0 and khz.value > 0
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream().cuda_stream
    # wave instructions per iteration: (label, all VALU incl. transcendental, transcendental)
    kinds = {0: ("v_fma_f32", 16, 0), 1: ("v_exp_f32", 16, 16),
             2: ("v_exp_f32 + 4 v_fma_f32", 81, 16), 3: ("v_log_f32", 16, 16)}
    nb = max(blocks_per_cu) * cus
    out = torch.empty(nb * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(nb * 4, dtype=torch.int64, device="cuda")
    res = {"cus": cus, "iters": iters, "threads_per_block": 256,
           "wall_clock_khz": khz.value,
           "loop_body_per_iteration": {"0": "16 v_fma_f32", "1": "16 v_exp_f32",
                                       "2": "16 v_exp_f32, 64 v_fma_f32, 1 v_mov_b32",
                                       "3": "16 v_log_f32"},
           "per_waves_per_simd": {}}
    for bpc in blocks_per_cu:
        blocks = bpc * cus
        row = {"ms": {}, "clock_ghz": {}, "cycles_per_wave_instr": {}}
        cyc = {}
        for k, (label, nv, nt) in kinds.items():
            for _ in range(2):
                assert lib.r2l_alu_rate_launch(k, blocks, iters, out.data_ptr(), clk.data_ptr(),
                                               stream) == 0
            times, cycles, ghz = [], [], []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                assert lib.r2l_alu_rate_launch(k, blocks, iters, out.data_ptr(), clk.data_ptr(),
                                               stream) == 0
                b.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b))
                c = clk[:blocks * 4].view(blocks, 4).cpu().double()
                dc, dw = c[:, 1] - c[:, 0], c[:, 3] - c[:, 2]
                cycles.append(float(dc.median()))
                ghz.append(float((dc / (dw / (khz.value * 1e3))).median()) / 1e9)
            med = lambda v: sorted(v)[len(v) // 2]   # noqa: E731
            # bpc waves share each SIMD for the whole loop
            cyc[k] = med(cycles) / (bpc * iters * nv)
            row["ms"][label] = round(med(times), 4)
            row["clock_ghz"][label] = round(med(ghz), 3)
            row["cycles_per_wave_instr"][label] = round(cyc[k], 3)
        fma = cyc[0]
        row["exp_slots_alone"] = round(cyc[1] / fma, 3)
        row["log_slots_alone"] = round(cyc[3] / fma, 3)
        row["exp_slots_beside_4_fma"] = round((cyc[2] * 81 - 65 * fma) / 16 / fma, 3)
        row["fma_tlane_ops_at_measured_clock"] = round(
            cus * 4 * 64 / fma * row["clock_ghz"]["v_fma_f32"] * 1e9 / 1e12, 3)
        res["per_waves_per_simd"][str(bpc)] = row
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="denoise", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time budget of the CPU baseline (0: skip it)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--queue-ahead", action="store_true",
                    help="queue the timed launches behind a spinning kernel and time them with "
                         "GPU events only (for kernel-trace profiles: no host gaps between "
                         "dispatches); implies --no-graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch copies of MIB MiB (reference for HBM byte counters)")
    ap.add_argument("--alu-rates", action="store_true",
                    help="only run the vector-ALU issue-rate micro-benchmark (FMA, exp, log)")
    args = ap.parse_args()
    if args.alu_rates:
        print(json.dumps(dict(alu_rates(), build=build_info())))
        return
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the scan is independent per (sequence, channel), "
              "so more GPUs only split the batch; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import reverse_mamba_selective_amd as r2l

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X", file=sys.stderr)
        sys.exit(1)
    wl = WORKLOADS[args.workload]()
    wl.setup(torch, r2l)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream().cuda_stream
    wl.launches_per_step = len(wl.step_calls[0])

    # (1) eager: every step launched from the host loop. HIP events on the
    # launch stream bracket the timed region; with more than one entry point
    # per step, an event also precedes every call, so that each entry point's
    # average duration comes from the timed region itself.
    entries = wl.step_entries
    per_call = len(wl.measure) > 1
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev_start, ev_end = ev(), ev()
    call_ev = [ev() for _ in range(args.steps * len(entries))] if per_call else []
    for i in range(args.warmup):
        wl.step(i, stream)
    torch.cuda.synchronize()
    if args.queue_ahead:
        # hold the stream with a spinning kernel long enough for the host to
        # queue every timed launch first (3x the warm-up's enqueue rate + 50 ms)
        h0 = time.perf_counter()
        wl.step(0, stream)
        enqueue_ms = (time.perf_counter() - h0) * 1e3
        torch.cuda.synchronize()
        torch.cuda._sleep(int(sleep_cycles_per_ms(torch) * (3 * enqueue_ms * args.steps + 50)))
    t0 = time.perf_counter()
    ev_start.record()
    for i in range(args.steps):
        for j, c in enumerate(wl.step_calls[i % len(wl.step_calls)]):
            if per_call:
                call_ev[i * len(entries) + j].record()
            c.launch(stream)
    ev_end.record()
    torch.cuda.synchronize()
    eager_s = (time.perf_counter() - t0) / args.steps
    region_ms = ev_start.elapsed_time(ev_end)
    timed = []
    step_split = None
    if per_call:
        marks = call_ev + [ev_end]
        dur = [marks[k].elapsed_time(marks[k + 1]) for k in range(len(call_ev))]
        for e, m in enumerate(wl.measure):
            mine = [d for k, d in enumerate(dur) if entries[k % len(entries)] == e]
            timed.append(dict(m, ms=sum(mine) / len(mine), reps=len(mine), src=m))
        n = len(entries)
        step_ms = [sum(dur[i * n:(i + 1) * n]) for i in range(args.steps)]
        spread_how = "per-step sums of the per-call events of the timed region"
        if wl.isolate_entries and not args.queue_ahead:
            # each entry point's calls again, back to back in a loop of their own
            # between two events (no event between the calls)
            for t in timed:
                calls = t["calls"]
                reps = args.steps * sum(1 for e in entries if wl.measure[e] is t["src"])
                for c in calls:
                    c.launch(stream)
                a0, a1 = ev(), ev()
                torch.cuda.synchronize()
                a0.record()
                for k in range(reps):
                    calls[k % len(calls)].launch(stream)
                a1.record()
                torch.cuda.synchronize()
                t["ms_per_call_events"] = t["ms"]
                t["ms"], t["reps"] = a0.elapsed_time(a1) / reps, reps
        step_split = {t["label"]: round(t["ms"] * sum(1 for e in entries if e == k), 4)
                      for k, t in enumerate(timed)}
    elif args.queue_ahead:
        launches = args.steps * len(entries)
        timed.append(dict(wl.measure[0], ms=region_ms / launches, reps=launches))
        step_ms = [region_ms / args.steps]
        spread_how = "not measured (queued-ahead run)"
    else:
        launches = args.steps * len(entries)
        timed.append(dict(wl.measure[0], ms=region_ms / launches, reps=launches))
        # spread: a second, instrumented pass with one event per step
        marks = [ev() for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        marks[0].record()
        for i in range(args.steps):
            wl.step(i, stream)
            marks[i + 1].record()
        torch.cuda.synchronize()
        step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
        spread_how = "a second pass of the same steps with one event after each step"
    step_spread = {k: round(v * 1e3, 3) for k, v in percentiles(step_ms).items()}

    # (2) the step captured once per rotating set in a hipGraph and replayed
    graph_s = None
    if not (args.no_graph or args.queue_ahead) and wl.launches_per_step > 1 and wl.graph_ok:
        graphs = []
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for r in range(wl.R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    wl.step(r, s.cuda_stream)
                graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % wl.R].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % wl.R].replay()
        torch.cuda.synchronize()
        graph_s = (time.perf_counter() - t0) / args.steps

    copy_gbs = copy_bandwidth_gbs(torch)

    step_s = min(eager_s, graph_s) if graph_s else eager_s
    if args.queue_ahead:   # the host clock also ran over the spin: GPU time only
        step_s = region_ms * 1e-3 / args.steps
    value = wl.tc_per_step / step_s

    def rooflines(m):
        kern_s = m["ms"] * 1e-3
        hbm_gbs = m["bytes"] / kern_s / 1e9
        alu_t = m["alu"] / kern_s / 1e12
        hbm = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": load_traffic(wl.name)}
        alu = {"bound": "alu", "achieved": round(alu_t, 3), "peak": round(VALU_PEAK_TLANEOPS, 3),
               "unit": "Tlane-op/s", "frac": round(alu_t / VALU_PEAK_TLANEOPS, 4),
               "traffic": hbm["traffic"]}
        if m.get("flops"):
            tf = m["flops"] / kern_s / 1e12
            mf = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                  "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                  "traffic": hbm["traffic"],
                  "note": "the whole call (GEMMs, conv, scan) against the bf16 matrix peak"}
            return mf, alu
        return (alu, hbm) if alu["frac"] >= hbm["frac"] else (hbm, alu)

    kernels = []
    for m in timed:
        bind_, other_ = rooflines(m)
        kernels.append({"entry": m["label"], "avg_launch_us": round(m["ms"] * 1e3, 3),
                        "launches_timed": m["reps"],
                        "timed_how": ("its calls back to back in a loop of their own, two events"
                                      if "ms_per_call_events" in m else
                                      "events of the timed region"),
                        "avg_launch_us_per_call_events": (
                            round(m["ms_per_call_events"] * 1e3, 3)
                            if "ms_per_call_events" in m else None),
                        "bytes_per_launch": m["bytes"],
                        "tc_per_launch": m["tc"], "tc_per_s": m["tc"] / (m["ms"] * 1e-3),
                        "roofline": bind_, "roofline_other": other_})
    binding, other = kernels[0]["roofline"], kernels[0]["roofline_other"]
    hbm_gbs = round(timed[0]["bytes"] / (timed[0]["ms"] * 1e-3) / 1e9, 1)

    cpu = parity = None
    if args.cpu_seconds > 0:
        what, pdtype, tol, sample = wl.parity_spec
        par = Parity(what, pdtype, tol)
        cpu = wl.cpu_baseline(args.cpu_seconds, parity=par)
        parity = dict(par.result(), sample=sample)
        extra = getattr(wl, "parity_extra", None)
        if extra:
            parity["forward"] = extra
            parity["pass"] = parity["pass"] and extra["pass"]
        single = wl.cpu_baseline(args.cpu_seconds / 4, nthreads=1)
        cpu.update(single_thread_value=single["value"], single_thread_sample=single["sample"],
                   **host_cpu())

    line = {
        "metric": "R2L selective-scan tokens*channels/s and HBM GB/s (% of peak), 1xMI355X",
        "value": value,
        "unit": "tokens*channels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",   # arithmetic type (storage type: config.in_dtype)
        "data": "synthetic (seeded)",
        "config": wl.config,
        "roofline": binding,
        "roofline_other": other,
        "hbm_gbs": hbm_gbs,
        "hbm_frac_of_8TBs": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "copy_gbs_measured": round(copy_gbs, 1),
        "hbm_frac_of_copy": round(hbm_gbs / copy_gbs, 4),
        "kernels": kernels,
        "alu_model": {"lane_ops_per_tc_readout_res": alu_ops_per_tc(True, True),
                      "lane_ops_per_tc_state_only": alu_ops_per_tc(False, False),
                      "trans_slots": TRANS_SLOTS},
        "source_sha": kernel_sha(),
        "build": build_info(),
        "timing": ("queued ahead of a spinning kernel, GPU events" if args.queue_ahead
                   else "host clock around the steps (synchronised); GPU events per entry point"),
        "ms_per_step_eager": eager_s * 1e3,
        "ms_per_step_eager_gpu_events": region_ms / args.steps,
        "step_us_spread": dict(step_spread, how=spread_how),
        "ms_per_step_graph": graph_s * 1e3 if graph_s else None,
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "step_split_ms": step_split,
        "step_share": ({k: round(v / sum(step_split.values()), 4) for k, v in step_split.items()}
                       if step_split else None),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
