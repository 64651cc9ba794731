#!/usr/bin/env python3
"""Throughput of the QLoRA NF4 linear (forward + backward) on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input,
issued as the layer calls a caller makes: qlora_linear_fwd then
qlora_linear_bwd (the step time and `value`). At large token counts they run
  forward   T = X A^T (+ bf16 hi/lo split)            rowdot
            F = expanded W' with [B | B] appended      row expansion
            Y = [X | sT] F^T, one bf16 rounding         bf16 MFMA GEMM
  backward  U = dY B (+ split)                          rowdot
            G = expanded W'^T with [A ; A] appended    transposing expansion
            dX = [dY | sU] G^T                          bf16 MFMA GEMM
            dA = s U^T X, dB = s dY^T T                 split-M MFMA + ordered reduce
(medium M: fused dequant GEMMs; M <= 16: dequant GEMV). A second timed
region issues the same kernels as the exported building-block calls, each
bracketed by HIP events on the launch stream, for the per-piece breakdown and
the dominant kernel's roofline. Inputs are resident in HBM when the timed
regions start; the weight is encoded once before them. Also reported: the
10th/50th/90th percentile step (one event per step boundary), the forward and
backward passes each timed as a region of their own, and what this box
sustains (a matrix-core loop without memory traffic, a 1 GiB streaming read)
beside the published peaks, the adapter merge (round(W' + s B A) into a bf16
copy) of each weight, timed alone against the HBM roofline, and the same step
over bf16 base weights (the bf16-base LoRA layer calls in place of the QLoRA
ones) with QLoRA's slowdown over it, and the AdamW
step over all adapter parameters with the moments in device memory and in
pinned host memory ("paged"), and the offline encode (quantize + double
quantization) and the bf16 dequant of each weight shape, each timed alone,
the storage-format ablations (NF4 or a uniform INT4 grid, with or without
double quantization) on the first weight: bits per weight, reconstruction
error and the layer step with each, and the step with LoRA dropout (0.05)
on every linear beside the plain step timed the same way.

Default workload: the 65B-class stack, 80 layers of seven linears (q, k, v,
o 8192x8192; gate, up 8192->22016; down 22016->8192), M = 4096 tokens, LoRA
r = 64, alpha = 16, forward then backward through all of them -- the largest
workload that fits one GPU (33.4 GB packed). --config selects the others
(1: 1024^2 at M = 16; 2: the 7B-class attention projection 4096^2 at
M = 4096; 3: 7B MLP block chained through SiLU; 4: 70B-class decode GEMVs).

The side measurements (evented breakdown, step distribution, bf16-base,
dropout and fp16 regions) run at most as many steps as fit in about five
seconds of GPU time, so a long workload stays within a few minutes; the
step time and `value` always come from exactly --steps timed steps.

Parity: the outputs of the first linear right after the timed steps are
snapshotted and compared with the CPU oracle on the same inputs; the line
carries `parity_ok`, and the process exits with status 3 when any relative
error is above 2e-3. Prints one JSON line.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from bit_nf4_quantized_02_amd import synth  # noqa: E402

METRIC = "QLoRA linear fwd+bwd TFLOP/s and packed-weight GB/s vs roofline, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed steps (default 50; 5 for config 5)")
    p.add_argument("--warmup", type=int, default=None, help="warm-up steps (default 10; 1 for config 5)")
    p.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5],
                   help="workload (default 5: the 65B-class stack, the largest that fits one GPU)")
    p.add_argument("--path", choices=["auto", "fused", "expanded"], default="auto",
                   help="large-M kernels: the library's choice (auto) or one forced, for comparison")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-side", action="store_true",
                   help="only the step regions (for counter and trace runs): no step distribution, attainable-peak "
                        "probes, merge, AdamW, encode, format, dropout, fp16 or bf16-base regions")
    p.add_argument("--layers", type=int, default=None,
                   help="layers of the 65B-class stack (default 80, the whole stack; fewer only for per-dispatch "
                        "counter runs, which measure one launch of each shape; the line then names the count)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle CPU time")
    p.add_argument("--json", default=None, help="also write the JSON line to this file")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB 3 times (the known-size kernel that "
                        "scales FETCH_SIZE / WRITE_SIZE counter readings) and exit")
    a = p.parse_args()
    if a.steps is None:
        a.steps = 5 if a.config == 5 else 50
    if a.warmup is None:
        a.warmup = 1 if a.config == 5 else 10
    return a


def copy_calibration(mib: int):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings per
    dispatch, divided by the bytes it must move, give the factor that turns
    those counters into bytes for the other kernels of the same run."""
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "dispatches": 3}), flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- one linear

class Pool:
    """Device buffers shared by linears that run one after another on one
    stream: workspaces, expansions, and outputs nothing reads after the next
    call. One buffer per (role, shape, dtype)."""

    def __init__(self):
        self.bufs = {}

    def __call__(self, role, shape, dtype):
        key = (role, tuple(shape), dtype)
        if key not in self.bufs:
            self.bufs[key] = torch.empty(shape, dtype=dtype, device="cuda")
        return self.bufs[key]


def _own(role, shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


class LinearPlan:
    """Device tensors and prebuilt C-ABI calls of one QLoRA linear. With a
    pool, the buffers no later call reads (workspaces, expansions, TS / U /
    US, Y unless given, dX) come from it; T, dA, dB stay the linear's own."""

    def __init__(self, q, li: synth.LinearInputs, backward: bool = True, X=None, dY=None, force_path=None,
                 pool=None, Y=None):
        dev = "cuda"
        m = li.meta
        self.n, self.k, self.r, self.s = m["n"], m["k"], m["r"], li.scale
        self.m = m["m"] if m["m"] is not None else X.shape[0]
        self.li = li
        M, N, K, r = self.m, self.n, self.k, self.r
        buf = _own if pool is None else pool
        self.W = q.quantize_nf4(li.W.to(dev))
        self.X = li.X.to(dev) if X is None else X
        self.dY = li.dY.to(dev) if dY is None else dY
        self.A = li.A.to(dev).contiguous()
        self.B = li.B.to(dev).contiguous()
        xc = q.lowrank_split_cols(r)
        self.T = torch.empty((M, r), dtype=torch.float32, device=dev)
        self.TS = buf("TS", (M, xc), torch.bfloat16)
        self.Y = buf("Y", (M, N), torch.bfloat16) if Y is None else Y
        self.U = buf("U", (M, r), torch.float32)
        self.US = buf("US", (M, xc), torch.bfloat16)
        self.dX = buf("dX", (M, K), torch.bfloat16)
        self.dA = torch.empty((r, K), dtype=torch.float32, device=dev)
        self.dB = torch.empty((N, r), dtype=torch.float32, device=dev)
        lib = q.raw()
        pw = max(lib.qlora_lowrank_project_workspace_bytes(M, K, r), lib.qlora_lowrank_project_workspace_bytes(M, N, r))
        gw = max(lib.qlora_lowrank_grad_workspace_bytes(M, K, r), lib.qlora_lowrank_grad_workspace_bytes(M, N, r))
        bw = max(lib.qlora_bf16_gemm_workspace_bytes(M, K, r, N), lib.qlora_bf16_gemm_workspace_bytes(M, N, r, K))
        vw = lib.qlora_nf4_gemv_workspace_bytes(K)
        dw = lib.qlora_nf4_gemv_dx_workspace_bytes(N, K)
        self.ws = buf("ws", (max(pw, gw, bw, vw, dw, 256),), torch.uint8)
        st = q._stream()
        P = q._ptr
        self.wst = self.W.struct()
        wref = q.ctypes.byref(self.wst)
        ws, wsn = P(self.ws), self.ws.numel()
        self.fwd, self.bwd = [], []
        # the kernels qlora_linear_fwd / _bwd choose at this size (or a forced
        # large-M variant, for comparing the two)
        self.path_fwd = q.linear_path(M, N, K, r, False)
        self.path_bwd = q.linear_path(M, N, K, r, True)
        if force_path is not None and self.path_fwd != q.PATH_GEMV:
            self.path_fwd = force_path
            self.path_bwd = force_path if (force_path != q.PATH_EXPANDED or N % 8 == 0) else q.PATH_FUSED
        if self.path_fwd == q.PATH_EXPANDED:
            self.Fw = buf("Fw", (q.nf4_expand_bytes(N, K, r, False) // 2,), torch.bfloat16)
        if backward and self.path_bwd == q.PATH_EXPANDED:
            # dX operand: contraction-major (as the layer call builds it) when
            # N % 64 == 0, else transposed
            self.dx_mode = 2 if N % 64 == 0 else 1
            self.Fx = buf("Fx", (q.nf4_expand_bytes(N, K, r, self.dx_mode) // 2,), torch.bfloat16)
        if self.path_fwd == q.PATH_GEMV:
            self.fwd.append(("lowrank_project_T", 2 * M * K * r,
                             q.Call("qlora_lowrank_project", P(self.X), M, K, P(self.A), 0, r, self.s, P(self.T), None,
                                    ws, wsn, st)))
            self.fwd.append(("nf4_gemv_fwd", 2 * M * N * K + 2 * M * N * r,
                             q.Call("qlora_nf4_gemv_fwd", wref, P(self.X), M, P(self.T), P(self.B), r, self.s,
                                    P(self.Y), ws, wsn, st, keep=(self.wst,))))
        else:
            self.fwd.append(("lowrank_project_T", 2 * M * K * r,
                             q.Call("qlora_lowrank_project", P(self.X), M, K, P(self.A), 0, r, self.s, P(self.T),
                                    P(self.TS), ws, wsn, st)))
            if self.path_fwd == q.PATH_FUSED:
                self.fwd.append(("nf4_gemm_fwd", 2 * M * N * K + 2 * M * N * r,
                                 q.Call("qlora_nf4_gemm_fwd", wref, P(self.X), M, P(self.TS), P(self.B), r, P(self.Y),
                                        st, keep=(self.wst,))))
            else:
                self.fwd.append(("nf4_expand_fwd", 0,
                                 q.Call("qlora_nf4_expand", wref, P(self.B), r, 0, P(self.Fw), self.Fw.numel() * 2, st,
                                        keep=(self.wst,))))
                self.fwd.append(("bf16_gemm_fwd", 2 * M * N * K + 2 * M * N * r,
                                 q.Call("qlora_bf16_gemm", P(self.X), M, K, P(self.TS), r, P(self.Fw), N, P(self.Y),
                                        ws, wsn, st)))
        if backward:
            gdx = self.path_bwd == q.PATH_GEMV
            self.bwd.append(("lowrank_project_U", 2 * M * N * r,
                             q.Call("qlora_lowrank_project", P(self.dY), M, N, P(self.B), 1, r, self.s, P(self.U),
                                    None if gdx else P(self.US), ws, wsn, st)))
            if gdx:
                self.bwd.append(("nf4_gemv_dx", 2 * M * N * K + 2 * M * K * r,
                                 q.Call("qlora_nf4_gemv_dx", wref, P(self.dY), M, P(self.U), P(self.A), r, self.s,
                                        P(self.dX), ws, wsn, st, keep=(self.wst,))))
            elif self.path_bwd == q.PATH_FUSED:
                self.bwd.append(("nf4_gemm_dx", 2 * M * N * K + 2 * M * K * r,
                                 q.Call("qlora_nf4_gemm_dx", wref, P(self.dY), M, P(self.US), P(self.A), r,
                                        P(self.dX), st, keep=(self.wst,))))
            else:
                self.bwd.append(("nf4_expand_dx", 0,
                                 q.Call("qlora_nf4_expand", wref, P(self.A), r, self.dx_mode, P(self.Fx),
                                        self.Fx.numel() * 2, st, keep=(self.wst,))))
                self.bwd.append(("bf16_gemm_dx", 2 * M * N * K + 2 * M * K * r,
                                 q.Call("qlora_bf16_gemm_nn" if self.dx_mode == 2 else "qlora_bf16_gemm", P(self.dY),
                                        M, N, P(self.US), r, P(self.Fx), K, P(self.dX), ws, wsn, st)))
            self.bwd.append(("lowrank_grad_dA", 2 * M * K * r,
                             q.Call("qlora_lowrank_grad", P(self.X), M, K, P(self.U), r, self.s, P(self.dA), 0, 0, ws,
                                    wsn, st)))
            self.bwd.append(("lowrank_grad_dB", 2 * M * N * r,
                             q.Call("qlora_lowrank_grad", P(self.dY), M, N, P(self.T), r, self.s, P(self.dB), 1, 0, ws,
                                    wsn, st)))

        # the layer calls themselves (what a caller runs: same kernels, launched
        # back to back inside one C call per pass)
        fw = lib.qlora_linear_workspace_bytes(M, N, K, r, 0)
        bw = lib.qlora_linear_workspace_bytes(M, N, K, r, 1) if backward else 0
        self.lws = buf("lws", (max(fw, bw, 256),), torch.uint8)
        lw, lwn = P(self.lws), self.lws.numel()
        self.api_fwd = q.Call("qlora_linear_fwd", wref, P(self.X), M, P(self.A), P(self.B), r, self.s, P(self.Y),
                              P(self.T), lw, lwn, st, keep=(self.wst,))
        self.api_bwd = None
        if backward:
            self.api_bwd = q.Call("qlora_linear_bwd", wref, P(self.X), P(self.T), P(self.dY), M, P(self.A),
                                  P(self.B), r, self.s, P(self.dX), P(self.dA), P(self.dB), 0, lw, lwn, st,
                                  keep=(self.wst,))

    @property
    def packed_bytes(self):
        return self.W.nbytes()

    def snapshot(self):
        """Copies of this linear's outputs (Y, and dX, dA, dB with a backward)
        as they stand: later regions that reuse the buffers cannot change
        what the parity check sees."""
        out = {"Y": self.Y.clone()}
        if self.api_bwd is not None:
            out.update(dX=self.dX.clone(), dA=self.dA.clone(), dB=self.dB.clone())
        torch.cuda.synchronize()
        return out


# ----------------------------------------------------------------------------- workloads

class Workload:
    def __init__(self, cid: int, q, force_path=None, layers=None):
        self.cid = cid
        self.c = synth.CONFIGS[cid]
        if layers is not None and layers != self.c.layers:
            if cid != 5 or not 1 <= layers <= self.c.layers:
                raise SystemExit(f"--layers applies to config 5 only, 1..{self.c.layers}")
            self.c = dataclasses.replace(self.c, layers=layers,
                                         title=self.c.title.replace(f"{self.c.layers} layers", f"{layers} layers"))
        self.tag = {1: "proj_1024_m16", 2: "attn_proj_4096_m4096", 3: "mlp_7b_m2048", 4: "decode_70b",
                    5: "stack_65b_m4096"}[cid]
        c = self.c
        self.pieces = []      # (name, flops, call): the building blocks, for the per-piece breakdown
        self.api = []         # the layer calls of one step, in order
        self.n_fwd = 0        # how many of them (from the start) form the forward pass
        self.plans = []
        self.passes_bytes = 0  # packed-weight bytes streamed per step
        if cid in (1, 2):
            lin = c.linears[0]
            li = synth.linear_inputs(cid, 0, 0, lin.n, lin.k, c.m[0], c.r, c.scale, sigma=c.sigma)
            p = LinearPlan(q, li, force_path=force_path)
            self.plans.append(p)
            self.pieces = p.fwd + p.bwd
            self.api = [p.api_fwd, p.api_bwd]
            self.n_fwd = 1
            self.passes_bytes = 2 * p.packed_bytes
            self.desc = dict(workload=c.title, M=c.m[0], N=lin.n, K=lin.k, r=c.r, alpha=c.alpha, passes="fwd+bwd")
        elif cid == 3:
            M = c.m[0]
            gate, up, down = c.linears
            X = synth.normal_bf16((M, gate.k), 1.0, cid, 0, synth.T_X).cuda()
            lg = synth.linear_inputs(cid, 0, 0, gate.n, gate.k, M, c.r, c.scale, sigma=c.sigma,
                                     outlier_frac=c.outlier_frac)
            lu = synth.linear_inputs(cid, 0, 1, up.n, up.k, M, c.r, c.scale, sigma=c.sigma, outlier_frac=c.outlier_frac)
            ld = synth.linear_inputs(cid, 0, 2, down.n, down.k, M, c.r, c.scale, sigma=c.sigma,
                                     outlier_frac=c.outlier_frac)
            H = torch.empty((M, gate.n), dtype=torch.bfloat16, device="cuda")
            dG = torch.empty_like(H)
            dU = torch.empty_like(H)
            pd = LinearPlan(q, ld, X=H, force_path=force_path)
            pg = LinearPlan(q, lg, X=X, dY=dG, force_path=force_path)
            pu = LinearPlan(q, lu, X=X, dY=dU, force_path=force_path)
            cnt = M * gate.n
            st = q._stream()
            P = q._ptr
            silu_f = q.Call("qlora_silu_mul_fwd", P(pg.Y), P(pu.Y), P(H), cnt, st)
            silu_b = q.Call("qlora_silu_mul_bwd", P(pg.Y), P(pu.Y), P(pd.dX), P(dG), P(dU), cnt, st)
            ren = lambda pl, tag: [(f"{tag}.{nme}", f, cl) for nme, f, cl in pl]  # noqa: E731
            self.pieces = (ren(pg.fwd, "gate") + ren(pu.fwd, "up") + [("silu_mul_fwd", 0, silu_f)] + ren(pd.fwd, "down")
                           + ren(pd.bwd, "down") + [("silu_mul_bwd", 0, silu_b)] + ren(pu.bwd, "up")
                           + ren(pg.bwd, "gate"))
            self.plans = [pg, pu, pd]
            self.api = [pg.api_fwd, pu.api_fwd, silu_f, pd.api_fwd, pd.api_bwd, silu_b, pu.api_bwd, pg.api_bwd]
            self.n_fwd = 4
            self.passes_bytes = 2 * sum(p.packed_bytes for p in self.plans)
            self.desc = dict(workload=c.title, M=M, r=c.r, alpha=c.alpha, passes="fwd+bwd, chained through SiLU")
        elif cid == 4:
            for li_i, lin in enumerate(c.linears):
                for M in c.m:
                    li = synth.linear_inputs(cid, 0, li_i, lin.n, lin.k, M, c.r, c.scale, sigma=c.sigma)
                    p = LinearPlan(q, li, backward=False)
                    self.plans.append(p)
                    self.api.append(p.api_fwd)
                    self.pieces += [(f"{lin.name}.M{M}.{nme}", f, cl) for nme, f, cl in p.fwd]
                    self.passes_bytes += p.packed_bytes
            self.n_fwd = len(self.api)
            self.desc = dict(workload=c.title, M=list(c.m), r=c.r, alpha=c.alpha, passes="fwd")
        elif cid == 5:
            self._stack(q, force_path)
        self.flops = sum(f for _, f, _ in self.pieces)

    def _stack(self, q, force_path):
        """The 65B-class stack: forward through the seven linears of every
        layer in order (q, k, v, o; gate, up; SiLU(gate) * up; down), then the
        backward in reverse. No attention or normalisation math: every
        attention linear and gate / up read one synthetic X, every
        8192-wide output gradient is one synthetic dY, and within a layer the
        MLP is chained through SiLU (gate and up outputs and H are the
        layer's own, as a training step keeps them for its backward). Layer 0
        draws its weights on the host (the tensors the full-size parity test
        uses) and owns all its buffers; the other layers draw W, A, B on the
        device and share one pool of workspaces and transient outputs."""
        c = self.c
        M = c.m[0]
        names = [lin.name for lin in c.linears]
        gi, ui, di = names.index("gate"), names.index("up"), names.index("down")
        width, ff = c.linears[0].k, c.linears[gi].n
        bf = torch.bfloat16
        X = synth.normal_bf16((M, width), 1.0, self.cid, 0, synth.T_X).cuda()
        dY = synth.normal_bf16((M, width), 1.0, self.cid, 0, synth.T_DY).cuda()
        pool = Pool()
        st, P = q._stream(), q._ptr
        ren = lambda pl, tag: [(f"{tag}.{nme}", f, cl) for nme, f, cl in pl]  # noqa: E731
        fwd_api, fwd_pc, bwd_layers = [], [], []
        for layer in range(c.layers):
            G = torch.empty((M, ff), dtype=bf, device="cuda")
            Uo = torch.empty((M, ff), dtype=bf, device="cuda")
            H = torch.empty((M, ff), dtype=bf, device="cuda")
            dG, dU = pool("dG", (M, ff), bf), pool("dU", (M, ff), bf)
            per = {}
            for li_i, lin in enumerate(c.linears):
                if layer == 0:
                    li = synth.linear_inputs(self.cid, 0, li_i, lin.n, lin.k, M, c.r, c.scale, sigma=c.sigma)
                else:
                    li = synth.device_linear_inputs(self.cid, layer, li_i, lin.n, lin.k, c.r, c.scale, sigma=c.sigma)
                pl = LinearPlan(q, li, X=H if li_i == di else X,
                                dY=dG if li_i == gi else dU if li_i == ui else dY,
                                force_path=force_path, pool=None if layer == 0 else pool,
                                Y=G if li_i == gi else Uo if li_i == ui else None)
                if layer > 0:
                    li.W = None  # the step reads only the encoding
                per[lin.name] = pl
                self.plans.append(pl)
            pg, pu, pd = per["gate"], per["up"], per["down"]
            attn = [per[n_] for n_ in names if n_ not in ("gate", "up", "down")]
            silu_f = q.Call("qlora_silu_mul_fwd", P(pg.Y), P(pu.Y), P(H), M * ff, st)
            silu_b = q.Call("qlora_silu_mul_bwd", P(pg.Y), P(pu.Y), P(pd.dX), P(dG), P(dU), M * ff, st)
            fwd_api += [pl.api_fwd for pl in attn] + [pg.api_fwd, pu.api_fwd, silu_f, pd.api_fwd]
            for pl in attn:
                fwd_pc += ren(pl.fwd, names[pl.li.meta["linear"]])
            fwd_pc += ren(pg.fwd, "gate") + ren(pu.fwd, "up") + [("silu_mul_fwd", 0, silu_f)] + ren(pd.fwd, "down")
            bapi = [pd.api_bwd, silu_b, pu.api_bwd, pg.api_bwd] + [pl.api_bwd for pl in reversed(attn)]
            bpc = ren(pd.bwd, "down") + [("silu_mul_bwd", 0, silu_b)] + ren(pu.bwd, "up") + ren(pg.bwd, "gate")
            for pl in reversed(attn):
                bpc += ren(pl.bwd, names[pl.li.meta["linear"]])
            bwd_layers.append((bapi, bpc))
        self.api = fwd_api + [cl for bapi, _ in reversed(bwd_layers) for cl in bapi]
        self.pieces = fwd_pc + [pc for _, bpc in reversed(bwd_layers) for pc in bpc]
        self.n_fwd = len(fwd_api)
        self.passes_bytes = 2 * sum(p.packed_bytes for p in self.plans)
        self.desc = dict(workload=c.title, M=M, layers=c.layers, r=c.r, alpha=c.alpha,
                         packed_GB=round(sum(p.packed_bytes for p in self.plans) / 1e9, 2),
                         passes=f"fwd through all {c.layers} layers, then bwd in reverse; MLP chained through SiLU "
                                "within a layer; one synthetic X and dY shared by the layers")

    def dominant_kernels(self):
        return [nme for nme, _, _ in self.pieces if "gemm" in nme or "gemv" in nme]


AUX_REGION_MS = 5000.0  # GPU time allotted to each side region


def time_steps(wl: Workload, steps: int, warmup: int):
    """Two timed regions over the same workload.

    A (the step time and `value`): K steps of the layer calls exactly as a
      caller issues them; nothing else on the stream, synchronize before and
      after; one event pair brackets the whole region.
    B (breakdown and roofline): K steps of the same kernels issued as the
      building-block calls, each bracketed by HIP events on the launch stream.
      Every event adds a few microseconds of idle time at its boundary, so the
      pieces of B sum to more than A's step; each piece's own duration is
      what the breakdown and the dominant-kernel roofline use.
    """
    for w_ in range(warmup):
        for cl in wl.api:
            cl()
        if w_ == 0:
            for _, _, cl in wl.pieces:
                cl()
    torch.cuda.synchronize()
    # region A
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        for cl in wl.api:
            cl()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev_step = e0.elapsed_time(e1) / steps
    # the timed step's own outputs of the first linear, for the parity check
    snap = wl.plans[0].snapshot()
    aux = max(2, min(steps, int(AUX_REGION_MS / (wall * 1e3))))
    steps = aux
    # region B
    calls = [cl for _, _, cl in wl.pieces]
    npc = len(calls)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(npc + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        ev = evs[s]
        ev[0].record()
        for i, cl in enumerate(calls):
            cl()
            ev[i + 1].record()
    torch.cuda.synchronize()
    per = np.zeros(npc)
    for s in range(steps):
        for i in range(npc):
            per[i] += evs[s][i].elapsed_time(evs[s][i + 1])
    per_ms = per / steps
    pieces_step = float(np.mean([evs[s][0].elapsed_time(evs[s][-1]) for s in range(steps)]))
    return wall * 1e3, ev_step, per_ms, pieces_step, snap, aux


def region_ms(calls, steps: int) -> float:
    """Mean time of `calls` issued back to back `steps` times, one event pair
    around the whole region."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        for cl in calls:
            cl()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def step_distribution(wl: Workload, steps: int):
    """Per-step times of the layer calls with one event at each step boundary
    (the only addition to region A), and the forward and backward passes each
    timed as a region of their own (a backward reuses the forward's saved T,
    which stays valid). Returns (p10, p50, p90 in us, fwd us, bwd us or None)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for s_ in range(steps):
        for cl in wl.api:
            cl()
        evs[s_ + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]) * 1e3
    p10, p50, p90 = (float(np.percentile(per, q_)) for q_ in (10, 50, 90))
    fwd = region_ms(wl.api[:wl.n_fwd], steps) * 1e3
    bwd = region_ms(wl.api[wl.n_fwd:], steps) * 1e3 if wl.n_fwd < len(wl.api) else None
    return p10, p50, p90, fwd, bwd


def lora_bf16_base(wl: Workload, q, steps: int):
    """The same step over bf16 base weights, the LoRA layer the pages compare
    QLoRA with: every QLoRA layer call replaced by the bf16-base layer call
    (qlora_lora_linear_fwd / _bwd) on the same activations, adapters and
    output buffers, everything else (SiLU) as is, timed as one region like the
    step, beside the QLoRA step timed the same way. The base weight is the
    linear's dequantized weight (2 B per weight); the 65B stack holds a few
    distinct bf16 copies per shape instead of 130 GB (each linear of a layer
    its own, alternating between even and odd layers), so no call re-reads a
    weight the last-level cache kept from the call before. Only for token
    counts that run matrix-core GEMMs (M >= 17). Returns (ms per bf16-base
    step, ms per QLoRA step) or None."""
    if any(p.m <= 16 for p in wl.plans):
        return None
    P, st = q._ptr, q._stream()
    hold, swap = [], {}
    copies = {}
    nws = max(max(q.lora_linear_workspace_bytes(p.m, p.n, p.k, p.r, False),
                  q.lora_linear_workspace_bytes(p.m, p.n, p.k, p.r, True) if p.api_bwd is not None else 0)
              for p in wl.plans)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda")
    per_layer = len(wl.c.linears)
    for i, p in enumerate(wl.plans):
        if wl.cid == 5:
            layer, li = divmod(i, per_layer)
            key = (p.n, p.k, li, layer % 2)
            if key not in copies:
                copies[key] = q.dequant(p.W) if i < per_layer else \
                    (torch.randn((p.n, p.k), device="cuda") * 0.02).to(torch.bfloat16)
            Wb = copies[key]
        else:
            Wb = q.dequant(p.W)
            hold.append(Wb)
        swap[id(p.api_fwd)] = q.Call("qlora_lora_linear_fwd", P(Wb), p.n, p.k, P(p.X), p.m, P(p.A), P(p.B), p.r, p.s,
                                     P(p.Y), P(p.T), P(ws), ws.numel(), st)
        if p.api_bwd is not None:
            swap[id(p.api_bwd)] = q.Call("qlora_lora_linear_bwd", P(Wb), p.n, p.k, P(p.X), P(p.T), P(p.dY), p.m,
                                         P(p.A), P(p.B), p.r, p.s, P(p.dX), P(p.dA), P(p.dB), 0, P(ws), ws.numel(),
                                         st)
    calls = [swap.get(id(cl), cl) for cl in wl.api]
    for cl in calls:
        cl()
    out = (region_ms(calls, steps), region_ms(wl.api, steps))
    del hold, copies, ws
    return out


def merge_rows(wl: Workload, q, reps: int = 20):
    """The adapter merge (fold s B A into a dequantized bf16 copy) of every
    weight of the workload, timed alone: one event pair around `reps`
    launches per weight. Bytes per launch: the packed weight (0.5159 B per
    weight) read once, the bf16 copy (2 B per weight) written once."""
    rows = {}
    for p in wl.plans:
        if p.r == 0 or f"{p.n}x{p.k}" in rows:
            continue
        out = torch.empty((p.n, p.k), dtype=torch.bfloat16, device="cuda")
        fn = q.Call("qlora_adapter_merge", q.ctypes.byref(p.wst), q._ptr(p.A), q._ptr(p.B), p.r, p.s, q._ptr(out), 0,
                    q._stream(), keep=(p.wst,))
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps * 1e-3
        nbytes = p.packed_bytes + 2 * p.n * p.k
        rows[f"{p.n}x{p.k}"] = dict(us=round(t * 1e6, 2), bytes=nbytes, GBps=round(nbytes / t / 1e9, 1))
        del out
    return rows


def _region_us(fn, reps: int) -> float:
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def encode_rows(wl: Workload, q, reps: int = 10):
    """The offline encode (qlora_quantize_nf4: 4-bit codes, block absmax,
    double quantization of the absmax) and qlora_dequant (the bf16 weight a
    caller can materialize) of each distinct weight shape, each timed alone
    on the weight's bf16 values in HBM. Bytes per launch: quantize reads 2 B
    per weight and writes the packed form, dequant the reverse."""
    rows = {}
    for p in wl.plans:
        key = f"{p.n}x{p.k}"
        if key in rows or p.li.W is None:
            continue
        W = p.li.W.to("cuda")
        w = q.NF4Weight.empty(p.n, p.k)
        wsn = max(q.quantize_workspace_bytes(p.n, p.k), 256)
        ws = torch.empty(wsn, dtype=torch.uint8, device="cuda")
        out = torch.empty((p.n, p.k), dtype=torch.bfloat16, device="cuda")
        st = w.struct()
        fq = q.Call("qlora_quantize_nf4", q._ptr(W), q.DT_BF16, q.ctypes.byref(st), q._ptr(ws), wsn, q._stream(),
                    keep=(st,))
        fd = q.Call("qlora_dequant", q.ctypes.byref(st), q._ptr(out), q._stream(), keep=(st,))
        nbytes = 2 * p.n * p.k + p.packed_bytes
        tq, td = _region_us(fq, reps), _region_us(fd, reps)
        rows[key] = dict(quantize_us=round(tq, 2), quantize_GBps=round(nbytes / tq / 1e3, 1),
                         dequant_us=round(td, 2), dequant_GBps=round(nbytes / td / 1e3, 1), bytes=nbytes,
                         dequant_frac=round(nbytes / td / 1e3 / PEAK_HBM_GBPS, 4))
        del W, w, ws, out
    return rows


def variant_rows(wl: Workload, q, reps: int = 10):
    """The ablations of the storage format on the workload's first weight:
    NF4 or the uniform INT4 grid, with double quantization or without it
    (one fp32 or one bf16 scale per block). For
    each: bits per weight, the relative Frobenius error of its dequantized
    bf16 weight against the bf16 weight it encodes, and the layer calls of
    one step (forward, and backward where the workload has one) timed as a
    region with that encoding, on the same activations and adapter. The
    ablation calls write outputs of their own (Y, T, dX, dA, dB), so the
    linear's buffers keep the plain step's results."""
    p = wl.plans[0]
    if p.li.W is None:
        return {}
    W = p.li.W.to("cuda")
    Wf = W.double()
    st = q._stream()
    P = q._ptr
    Y, T, dX = torch.empty_like(p.Y), torch.empty_like(p.T), torch.empty_like(p.dX)
    dA, dB = torch.empty_like(p.dA), torch.empty_like(p.dB)
    forms = (("dq", True, torch.float32), ("no_dq", False, torch.float32), ("no_dq_bf16_scale", False, torch.bfloat16))
    rows = []
    for grid in ("nf4", "uniform"):
        cb = torch.tensor(q.build_nf4_codebook() if grid == "nf4" else q.build_uniform4_codebook(),
                          dtype=torch.float32, device="cuda")
        for tag, dq, sd in forms:
            w = q.quantize_nf4(W, codebook=cb, double_quant=dq, scale_dtype=sd)
            err = float(torch.linalg.norm(q.dequant(w).double() - Wf) / torch.linalg.norm(Wf))
            wst = w.struct()
            wref = q.ctypes.byref(wst)
            lw, lwn = P(p.lws), p.lws.numel()
            calls = [q.Call("qlora_linear_fwd", wref, P(p.X), p.m, P(p.A), P(p.B), p.r, p.s, P(Y), P(T), lw,
                            lwn, st, keep=(wst,))]
            if p.api_bwd is not None:
                calls.append(q.Call("qlora_linear_bwd", wref, P(p.X), P(T), P(p.dY), p.m, P(p.A), P(p.B), p.r,
                                    p.s, P(dX), P(dA), P(dB), 0, lw, lwn, st, keep=(wst,)))
            rows.append((f"{grid}_{tag}", w, err, calls))
    # the forms timed round-robin, three rounds, each form's best round: the
    # first form timed alone once read ~10% slow (clock and cache state after
    # the encodes), which is the order, not the format
    best = {name: float("inf") for name, *_ in rows}
    for _ in range(3):
        for name, w, err, calls in rows:
            best[name] = min(best[name], _region_us(lambda: [cl() for cl in calls], reps))
    out = {}
    for name, w, err, calls in rows:
        out[name] = dict(bits_per_weight=round(8.0 * w.nbytes() / (w.n * w.k), 4), weight_relerr=round(err, 5),
                         step_us=round(best[name], 2))
    del rows
    return out


def dropout_step(wl: Workload, q, steps: int):
    """The step with LoRA dropout (p = 0.05, a seeded keep mask per linear):
    every layer call replaced by its dropout form, everything else (SiLU)
    as is, timed as one region like the step itself. Returns (ms per step,
    ms per plain step timed the same way) or None where the workload has no
    backward."""
    if any(p.api_bwd is None for p in wl.plans) or wl.cid == 5:
        return None
    P = q._ptr
    st = q._stream()
    keep = 1.0 / (1.0 - 0.05)
    swap = {}
    hold = []
    for i, p in enumerate(wl.plans):
        mask = synth.dropout_mask(p.m, p.k, 0.05, wl.cid, i, synth.T_MASK).cuda()
        hold.append(mask)
        ws = p.lws
        wref = q.ctypes.byref(p.wst)
        swap[id(p.api_fwd)] = q.Call("qlora_linear_fwd_dropout", wref, P(p.X), p.m, P(p.A), P(p.B), p.r, p.s,
                                     P(mask), keep, P(p.Y), P(p.T), P(ws), ws.numel(), st, keep=(p.wst,))
        swap[id(p.api_bwd)] = q.Call("qlora_linear_bwd_dropout", wref, P(p.X), P(p.T), P(p.dY), p.m, P(p.A),
                                     P(p.B), p.r, p.s, P(mask), keep, P(p.dX), P(p.dA), P(p.dB), 0, P(ws),
                                     ws.numel(), st, keep=(p.wst,))
    calls = [swap.get(id(cl), cl) for cl in wl.api]
    for cl in calls:
        cl()
    out = (region_ms(calls, steps), region_ms(wl.api, steps))
    del hold
    return out


def f16_step(wl: Workload, q, steps: int):
    """The step in fp16 compute: every layer call replaced by its fp16 form
    over fp16 copies of X, A, B and dY (same shapes, same values rounded to
    fp16), SiLU calls as they are (same bytes), timed as one region like the
    step itself. Returns (ms per step, ms per plain step timed the same way)
    or None for the 65B stack."""
    if wl.cid == 5:
        return None
    P = q._ptr
    st = q._stream()
    swap = {}
    hold = []
    for p in wl.plans:
        X, A, B = p.X.half(), p.A.half(), p.B.half()
        Y = torch.empty(p.Y.shape, dtype=torch.float16, device="cuda")
        nws = q.linear_workspace_bytes(p.m, p.n, p.k, p.r, False, torch.float16)
        if p.api_bwd is not None:
            nws = max(nws, q.linear_workspace_bytes(p.m, p.n, p.k, p.r, True, torch.float16))
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
        wref = q.ctypes.byref(p.wst)
        swap[id(p.api_fwd)] = q.Call("qlora_linear_fwd_f16", wref, P(X), p.m, P(A), P(B), p.r, p.s, P(Y), P(p.T),
                                     P(ws), ws.numel(), st, keep=(p.wst,))
        hold += [X, A, B, Y, ws]
        if p.api_bwd is not None:
            dY = p.dY.half()
            dX = torch.empty(p.dX.shape, dtype=torch.float16, device="cuda")
            swap[id(p.api_bwd)] = q.Call("qlora_linear_bwd_f16", wref, P(X), P(p.T), P(dY), p.m, P(A), P(B), p.r,
                                         p.s, P(dX), P(p.dA), P(p.dB), 0, P(ws), ws.numel(), st, keep=(p.wst,))
            hold += [dY, dX]
    calls = [swap.get(id(cl), cl) for cl in wl.api]
    for cl in calls:
        cl()
    out = (region_ms(calls, steps), region_ms(wl.api, steps))
    del hold
    return out


def adamw_rows(wl: Workload, q, reps: int = 20):
    """The AdamW step over every adapter parameter of the workload (A and B
    of each linear, fp32 masters, the step's dA / dB as gradients, bf16 copy
    written), with the moments in device memory and in pinned host memory,
    each timed alone. Bytes per parameter: gradient 4, master 4 + 4, moments
    2 x (4 + 4), bf16 copy 2 = 30."""
    plans = [p for p in wl.plans if p.r and p.bwd]
    if not plans:
        return {}
    n = sum(p.dA.numel() + p.dB.numel() for p in plans)
    grad = torch.cat([torch.cat([p.dA.reshape(-1), p.dB.reshape(-1)]) for p in plans])
    theta = torch.cat([torch.cat([p.A.float().reshape(-1), p.B.float().reshape(-1)]) for p in plans])
    t16 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    rows = {}
    reps = reps if n < (1 << 27) else 5
    for where in ("device", "pinned_host"):
        if where == "device":
            m = torch.zeros(n, dtype=torch.float32, device="cuda")
            v = torch.zeros(n, dtype=torch.float32, device="cuda")
        else:
            m = torch.zeros(n, dtype=torch.float32).pin_memory()
            v = torch.zeros(n, dtype=torch.float32).pin_memory()
        th = theta.clone()
        fn = q.Call("qlora_adamw_step", q._ptr(th), q._ptr(t16), q._ptr(grad), q.ctypes.c_void_p(m.data_ptr()),
                    q.ctypes.c_void_p(v.data_ptr()), n, 1, 2e-4, 0.9, 0.999, 1e-8, 0.0, q._stream())
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps * 1e-3
        rows[where] = dict(params=n, us=round(t * 1e6, 2), GBps=round(30 * n / t / 1e9, 1))
    rows["device"]["frac"] = round(rows["device"]["GBps"] / PEAK_HBM_GBPS, 4)
    return rows


def attainable(q):
    """What this machine sustains: a matrix-core loop with no memory traffic
    (bf16 MFMA TFLOP/s) and one streaming read of a 1 GiB buffer (GB/s)."""
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    out = {}
    for nme, fn in (("mfma_bf16_tflops", lambda: q.calib_mfma(cus, 2048, sink)),
                    ("hbm_read_gbps", lambda: q.calib_stream_read(buf, sink))):
        work = fn()  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 5 * 1e-3
        out[nme] = round(work / t / (1e12 if nme.startswith("mfma") else 1e9), 1)
    del buf
    return out


def gemm_traffic(tag: str, launches):
    """Measured HBM bytes per launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled), averaged over the named launches of
    the workload; used only while every entry exists and its kernel's source
    file still matches the one the counters came from (sha256 recorded
    beside each entry)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        vals = []
        for nme in launches:
            ent = data["kernels"].get(f"{tag}.{nme}")
            if ent is None:
                return None
            src = os.path.join(ROOT, "bit_nf4_quantized_02_amd", "csrc", ent["source"])
            if hashlib.sha256(open(src, "rb").read()).hexdigest() != ent["source_sha256"]:
                return None
            vals.append(float(ent["bytes_per_launch"]))
        return round(sum(vals) / len(vals), 0)
    except Exception:
        return None


# ----------------------------------------------------------------------------- CPU oracle leg

PARITY_TOL = 2e-3  # relative Frobenius error against the fp64 oracle (Y, dX, dA, dB)


def cpu_baseline(wl: Workload, target_s: float, snap: dict):
    """The oracle as it stands, timed on this host's cores on a bounded sample
    of the same workload: whole steps of the first linear (all M tokens),
    repeated until about target_s seconds; the weight's oracle encoding is
    made once beforehand, timed on its own and not counted in the steps. The
    parts of a step (scale decode + bf16 expansion, forward, backward) are
    timed separately as well."""
    from oracle import linear as olin
    from oracle import nf4 as onf4
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"]
                      or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    p = wl.plans[0]
    li = p.li
    t0 = time.perf_counter()
    ow = onf4.NF4Weight(li.W.float().numpy())
    t_encode = time.perf_counter() - t0
    # the inputs this linear actually consumed on the GPU (for chained
    # workloads X or dY come from the previous GPU step)
    X, A, B, dY = (t.float().cpu().numpy().astype(np.float64) for t in (p.X, li.A, li.B, p.dY))
    backward = len(p.bwd) > 0
    flops = sum(f for _, f, _ in p.fwd + p.bwd)
    n, spent = 0, 0.0
    parts = np.zeros(3)
    out = None
    while (spent < target_s and n < 200) or n == 0:
        t0 = time.perf_counter()
        cp = onf4.decode_scales(ow.code8, ow.s2, ow.mean)
        Wd = onf4.dequant(ow.codes, cp, ow.levels)
        t1 = time.perf_counter()
        Y, T = olin.linear_fwd(X, Wd, A, B, li.scale)
        t2 = time.perf_counter()
        if backward:
            dX, dA, dB, _ = olin.linear_bwd(X, Wd, A, B, li.scale, dY, T)
            out = (Y, dX, dA, dB)
        else:
            out = (Y,)
        t3 = time.perf_counter()
        parts += (t1 - t0, t2 - t1, t3 - t2)
        spent += t3 - t0
        n += 1
    # parity of the timed step's GPU outputs (snapshotted right after it)
    # against this sample
    errs = {nme: olin.relerr(snap[nme].float().cpu().numpy(), o) for nme, o in zip(["Y", "dX", "dA", "dB"], out)}
    return dict(value=flops * n / spent / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{n} whole fwd{'+bwd' if backward else ''} step(s) of linear '{wl.c.linears[0].name}' "
                       f"(M={p.m}, N={p.n}, K={p.k}, r={p.r}): numpy fp64 products, bf16 expansion of the "
                       f"encoded weight each step; {spent:.1f} s total",
                seconds=spent, parity_relerr=errs, parity_tol=PARITY_TOL,
                parity_ok=bool(all(e <= PARITY_TOL for e in errs.values())),
                parts_s={"encode_once": round(t_encode, 3), "dequant": round(float(parts[0]) / n, 4),
                         "fwd": round(float(parts[1]) / n, 4), "bwd": round(float(parts[2]) / n, 4)})


# ----------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (the layer shards by data "
                                   "parallelism, one replica per GPU); --gpus must be 1"}), flush=True)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)
        return
    from bit_nf4_quantized_02_amd import qlora as q
    log(f"bench: building workload config {args.config}")
    force = {"auto": None, "fused": q.PATH_FUSED, "expanded": q.PATH_EXPANDED}[args.path]
    wl = Workload(args.config, q, force_path=force, layers=args.layers)
    names_of = {q.PATH_GEMV: "gemv", q.PATH_FUSED: "fused", q.PATH_EXPANDED: "expanded"}
    wl.desc["kernels"] = sorted({f"fwd:{names_of[p.path_fwd]}" for p in wl.plans}
                                | {f"bwd:{names_of[p.path_bwd]}" for p in wl.plans if p.bwd})
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps after {args.warmup} warmup")
    ms_wall, ms_ev, per_ms, ms_pieces, snap, aux = time_steps(wl, args.steps, args.warmup)
    if args.no_side:
        p10 = p50 = p90 = fwd_us = bwd_us = float("nan")
        att = {"mfma_bf16_tflops": float("nan"), "hbm_read_gbps": float("nan")}
        merges, lora_ms, adamw, encode, variants, drop, f16 = {}, None, {}, {}, {}, None, None
    else:
        log(f"bench: side regions with {aux} steps each")
        p10, p50, p90, fwd_us, bwd_us = step_distribution(wl, aux)
        att = attainable(q)
        merges = merge_rows(wl, q) if args.config in (1, 2, 3, 5) else {}
        lora_ms = lora_bf16_base(wl, q, aux)
        adamw = adamw_rows(wl, q)
        encode = encode_rows(wl, q)
        variants = variant_rows(wl, q)
        drop = dropout_step(wl, q, aux)
        f16 = f16_step(wl, q, aux)
    for row in merges.values():
        row["frac"] = round(row["GBps"] / PEAK_HBM_GBPS, 4)
        row["frac_of_attainable"] = round(row["GBps"] / att["hbm_read_gbps"], 4)
    names = [nme for nme, _, _ in wl.pieces]
    flops = [f for _, f, _ in wl.pieces]
    value = wl.flops / (ms_wall * 1e-3) / 1e12
    gbps = wl.passes_bytes / (ms_wall * 1e-3) / 1e9
    # mean per launch of each named piece (a name repeats only in the 65B
    # stack, once per layer)
    agg = {}
    for nme, t in zip(names, per_ms):
        a = agg.setdefault(nme, [0.0, 0])
        a[0] += t
        a[1] += 1
    avg_ms = {nme: a[0] / a[1] for nme, a in agg.items()}
    breakdown = {nme: round(t * 1e3, 2) for nme, t in avg_ms.items()}

    # dominant kernel: the matrix kernel (GEMM or GEMV) with the largest
    # time per step, taken together with every launch of the same kernel at
    # the same algorithmic size (within 1%: the 65B stack's six 22016-wide
    # GEMMs per layer are one such group, 480 launches), so the average
    # launch duration is the one a kernel trace reports for it
    tot = {}
    for nme, f, t in zip(names, flops, per_ms):
        if "gemm" in nme or "gemv" in nme:
            tot[nme] = tot.get(nme, 0.0) + t
    dom = max(tot, key=tot.get)
    i = names.index(dom)
    dom_base = dom.split(".")[-1]
    kind = "gemv" if "gemv" in dom_base else "gemm"
    group = [j for j, nme in enumerate(names)
             if kind in nme.split(".")[-1] and abs(flops[j] - flops[i]) <= 0.01 * flops[i]]
    grp_ms = float(sum(per_ms[j] for j in group))
    dom_ms = grp_ms / len(group)
    plan_of = {}
    for pl in wl.plans:
        for _, _, c in pl.fwd + pl.bwd:
            plan_of[id(c)] = pl
    pl = plan_of[id(wl.pieces[i][2])]
    if pl.m <= 16:
        # few tokens: the packed weight streamed from HBM bounds the kernel
        nbytes = sum(plan_of[id(wl.pieces[j][2])].packed_bytes for j in group)
        achieved = nbytes / (grp_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBPS, 4), attainable=att["hbm_read_gbps"],
                    frac_of_attainable=round(achieved / att["hbm_read_gbps"], 4))
    else:
        achieved = sum(flops[j] for j in group) / (grp_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4), attainable=att["mfma_bf16_tflops"],
                    frac_of_attainable=round(achieved / att["mfma_bf16_tflops"], 4))
    roof["kernel"] = dom_base
    roof["launches"] = sorted({names[j] for j in group})
    roof["launches_per_step"] = len(group)
    roof["avg_launch_us"] = round(dom_ms * 1e3, 2)
    roof["traffic"] = gemm_traffic(wl.tag, roof["launches"])

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,sigma) weights, N(0,1) activations; no dataset)",
        "config": wl.desc,
        "packed_weight_GBps": round(gbps, 1),
        "ms_per_step_events": round(ms_ev, 4),
        "ms_per_step_evented_pieces": round(ms_pieces, 4),
        "step_us_p10_p50_p90": [round(p10, 1), round(p50, 1), round(p90, 1)],
        "fwd_us": round(fwd_us, 1),
        "bwd_us": None if bwd_us is None else round(bwd_us, 1),
        "attainable": att,
        "adapter_merge_bf16": merges,
        "adamw_step": adamw,
        "encode": encode,
        "format_variants": variants,
        "lora_dropout": None if drop is None else {
            "p": 0.05, "ms_per_step": round(drop[0], 4), "tflops": round(wl.flops / (drop[0] * 1e-3) / 1e12, 2),
            "plain_ms_per_step_same_region": round(drop[1], 4), "overhead": round(drop[0] / drop[1], 3)},
        "fp16_compute": None if f16 is None else {
            "ms_per_step": round(f16[0], 4), "tflops": round(wl.flops / (f16[0] * 1e-3) / 1e12, 2),
            "bf16_ms_per_step_same_region": round(f16[1], 4), "ratio": round(f16[0] / f16[1], 3)},
        "lora_bf16_base": None if lora_ms is None else {
            "ms_per_step": round(lora_ms[0], 4),
            "tflops": round(wl.flops / (lora_ms[0] * 1e-3) / 1e12, 2),
            "qlora_same_calls_ms_per_step": round(lora_ms[1], 4),
            "qlora_slowdown": round(lora_ms[1] / lora_ms[0], 3)},
        "flops_per_step": wl.flops,
        "breakdown_us": breakdown,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, snap)
        res["parity_ok"] = res["cpu_baseline"]["parity_ok"]
    line = json.dumps(res)
    print(line, flush=True)
    if args.json:
        with open(args.json, "w") as f:
            f.write(line + "\n")
    if res.get("parity_ok") is False:
        log(f"bench: PARITY FAILED (relative error above {PARITY_TOL}): {res['cpu_baseline']['parity_relerr']}")
        sys.exit(3)


if __name__ == "__main__":
    main()
