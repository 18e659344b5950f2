"""Benchmark of the W4A16 skinny GEMM / top-8 MoE hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  A step is one pass of the path over one batch of
synthetic, seeded inputs: one qgemm call for the GEMM workloads, one router
call plus one grouped-MoE call for the MoE workload.  The weights are
resident in HBM before timing starts and rotate over enough distinct device
copies (>= 2 GiB in total) that neither the 256 MB Infinity Cache nor L2 can
serve them, so every step streams its weights from HBM.

W eager warmup steps run first; then K steps are captured into one HIP graph
(the launches themselves, nothing else), the graph is replayed once untimed,
and the timed region is exactly one replay of the K steps, bracketed by
synchronizations and timed both with HIP events on the launch stream and with
the host clock.

value        = algorithmic weight bytes per step * K / host wall time of the K steps
roofline     = algorithmic bytes of the dominant launch / its mean duration (the
               event-timed replay / K) against the 8 TB/s HBM peak; traffic =
               the counted HBM bytes per launch from the committed counter summary
               (profiles/traffic.json) when it was taken on the current kernel
               sources, else null
               stream_ceiling = q4_stream_read of the same number of bytes (16-byte
               non-temporal loads and nothing else, rotated like the weights, the
               fastest of a few launch shapes): the measured floor for those bytes
cpu_baseline = the float64 CPU oracle on a bounded sample of the same workload, on
               this host's cores
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "weight-stream HBM GB/s (% of ~8 TB/s) for W4A16 GEMM M=1/16 & top-8 MoE"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense f16 matrix-core peak
DEFAULT_WORKLOAD = "nvfp4_verify_m16_k4096_n8192"
ROTATE_BYTES = 2 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--hot", action="store_true", help="no weight rotation (cache-resident weights)")
    ap.add_argument("--copy-kernel", type=int, default=0,
                    help="instead of the path, time a device copy of this many MiB (counter calibration)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph replay")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the stream-read ceiling measurement")
    return ap.parse_args()


def threads_used():
    try:
        from threadpoolctl import threadpool_info
        n = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        n = 1
    return int(n)


def sources_sha256(kind):
    """Hash of the kernel sources a workload runs (traffic figures are tied to it)."""
    import hashlib
    csrc = os.path.join(ROOT, "moe_w4a16_skinny_amd", "csrc")
    names = ["q4mi_tiles.h", "q4mi_internal.h"] + {"moe": ["q4mi_moe.hip"],
                                                    "moe_block": ["q4mi_moe.hip", "q4mi_block.hip"],
                                                    "quant": ["q4mi_quant.hip"],
                                                    "prefill": ["q4mi_prefill.hip"],
                                                    "affine_bits": ["q4mi_affineb.hip"]}.get(kind, ["q4mi_gemm.hip"])
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_for(workload, kind):
    """Counted HBM bytes per launch (fetch + write) if taken on the current sources, else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha256") != sources_sha256(kind):
        return None
    return int(rec["fetch_bytes"]) + int(rec["write_bytes"])


# ------------------------------------------------------------------ workloads

def torch_f32():
    import torch
    return torch.float32


class GemmWork:
    def __init__(self, name, spec, hot):
        import numpy as np
        import torch

        import moe_w4a16_skinny_amd as q4
        import synth
        self.name, self.spec = name, spec
        self.q4 = q4
        M, K, N = spec["M"], spec["K"], spec["N"]
        self.M, self.K, self.N = M, K, N
        t0 = time.time()
        if spec["kind"] == "nvfp4":
            inp = synth.nvfp4_gemm(spec["seed"], M, K, N)
            packed = q4.q4_nvfp4_repack(inp.codes, inp.scales)
            self.a = torch.from_numpy(inp.a).cuda()
            self.g = float(inp.g)
            self.alg_bytes = N * K // 2 + N * K // 16 + 4
            self.dtype = "f16"
            self.flops = 2 * M * N * K  # the prefill rows (M > 16) make the product matrix-core bound
        elif spec["kind"] == "affine_bits":
            bits = spec["bits"]
            q, sc, bi = synth.affine_weights_bits(spec["seed"], N, K, bits)
            a = synth.act_bf16_bits(spec["seed"] + 1, M, K)
            inp = synth.AffineGemmInputs(q, sc, bi, a)
            packed = q4.q4_affine_bits_repack(q, sc, bi, bits)
            self.a = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
            self.alg_bytes = N * K * bits // 8 + 2 * N * (K // 64) * 2
            self.dtype = "bf16"
        else:
            inp = synth.affine_gemm(spec["seed"], M, K, N)
            packed = q4.q4_affine4_repack(inp.codes, inp.scale, inp.bias)
            self.a = torch.from_numpy(inp.a.view(np.int16)).cuda().view(torch.bfloat16)
            self.alg_bytes = N * K // 2 + 2 * N * (K // 64) * 2
            self.dtype = "bf16"
        self.inp = inp
        log(f"[bench] {name}: inputs generated and packed in {time.time() - t0:.1f}s")
        nb = packed.size
        self.copies = 1 if hot else max(2, -(-ROTATE_BYTES // nb))
        self.stride = -(-nb // 256) * 256
        base = torch.from_numpy(packed).cuda()
        self.wbuf = torch.empty(self.copies * self.stride, dtype=torch.uint8, device="cuda")
        for i in range(self.copies):
            self.wbuf[i * self.stride:i * self.stride + nb].copy_(base)
        del base
        self.sample = spec.get("sample")  # fused sampling: softcap, temperature; tokens only
        out_kind = spec.get("out", "f32")
        out_dt = {"f32": torch.float32, "f16": torch.float16, "none": torch.float32}[out_kind]
        self.out = torch.empty((M, N), dtype=out_dt, device="cuda") if out_kind != "none" else None
        self.want_argmax = bool(spec.get("argmax")) or bool(self.sample)
        self.amax = torch.empty(16, dtype=torch.int32, device="cuda")
        if spec["kind"] == "nvfp4":
            self.wsb = q4.raw().qgemm_nvfp4_workspace_bytes(M, K, N, int(self.want_argmax))
        elif spec["kind"] == "affine_bits":
            self.wsb = 0
        else:
            self.wsb = q4.raw().qgemm_affine4_workspace_bytes(M, K, N)
        self.ws = q4.workspace(max(self.wsb, 256))
        self.i = 0
        self.kind = "prefill" if M > 16 else "gemm"  # more than 16 rows run the prefill kernel
        self.kernel_names = ["qgemm_prefill_kernel" if M > 16 else "qgemm_kernel"]
        if spec["kind"] == "affine_bits":
            self.kind = "affine_bits"
            self.kernel_names = ["qgemm_affineb_kernel"]

    def step(self):
        import ctypes as C
        q4 = self.q4
        lib = q4.raw()
        w = C.c_void_p(self.wbuf.data_ptr() + (self.i % self.copies) * self.stride)
        self.i += 1
        s = q4._stream()
        if self.sample:  # one offset per step, so that every step draws fresh noise
            rc = lib.qgemm_nvfp4_sample(w, self.g, C.c_void_p(self.a.data_ptr()), self.M, self.K, self.N,
                                        float(self.sample["softcap"]), float(self.sample["temperature"]),
                                        0x5EED, self.i, None, q4._dtype_code(torch_f32()),
                                        C.c_void_p(self.amax.data_ptr()), C.c_void_p(self.ws.data_ptr()),
                                        self.ws.numel(), s)
        elif self.spec["kind"] == "nvfp4":
            rc = lib.qgemm_nvfp4(w, self.g, C.c_void_p(self.a.data_ptr()), self.M, self.K, self.N,
                                 C.c_void_p(self.out.data_ptr()), q4._dtype_code(self.out.dtype),
                                 C.c_void_p(self.amax.data_ptr()) if self.want_argmax else None,
                                 C.c_void_p(self.ws.data_ptr()), self.ws.numel(), s)
        elif self.spec["kind"] == "affine_bits":
            rc = lib.qgemm_affine_bits(w, C.c_void_p(self.a.data_ptr()), self.M, self.K, self.N, self.spec["bits"],
                                       C.c_void_p(self.out.data_ptr()), q4._dtype_code(self.out.dtype), s)
        else:
            rc = lib.qgemm_affine4(w, C.c_void_p(self.a.data_ptr()), self.M, self.K, self.N,
                                   C.c_void_p(self.out.data_ptr()), q4._dtype_code(self.out.dtype),
                                   C.c_void_p(self.ws.data_ptr()), self.ws.numel(), s)
        if rc != 0:
            q4._check(rc)

    def config(self):
        c = {"workload": self.name, "M": self.M, "K": self.K, "N": self.N,
             "weights": self.spec["kind"], "out": self.spec.get("out", "f32"),
             "fused_argmax": self.want_argmax, "weight_copies_rotated": self.copies}
        if self.sample:
            c["fused_sampling"] = dict(self.sample, noise="Philox4x32-10 Gumbel-max, offset = step")
        return c

    def cpu_oracle_sample(self, seconds):
        """Time the oracle on row blocks of the same weights for about `seconds`."""
        import oracle
        inp = self.inp
        N = self.N
        rows = min(N, 2048)
        done = 0
        t0 = time.perf_counter()
        while True:
            r0 = (done * rows) % N
            r1 = min(N, r0 + rows)
            if self.spec["kind"] == "nvfp4":
                oracle.nvfp4_gemm_ref(inp.codes[r0:r1], inp.scales[r0:r1], inp.g, inp.a, want_bound=False)
            elif self.spec["kind"] == "affine_bits":
                oracle.affine_bits_gemm_ref(inp.codes[r0:r1], inp.scale[r0:r1], inp.bias[r0:r1], inp.a,
                                            self.spec["bits"], want_bound=False)
            else:
                oracle.affine_gemm_ref(inp.codes[r0:r1], inp.scale[r0:r1], inp.bias[r0:r1], inp.a,
                                       want_bound=False)
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        bytes_done = done * rows * self.alg_bytes / N
        return bytes_done / el / 1e9, f"{done} oracle GEMMs of {rows} weight rows (M={self.M}, K={self.K}) " \
                                      f"in {el:.1f}s"


class MoeWork:
    """One step = moe_route_grouped_qgemm (the router, then the grouped layer;
    the top-k taken inside the gate/up launch) on the 128 + 1 expert layer."""

    def __init__(self, name, spec, hot):
        import numpy as np
        import torch

        import moe_w4a16_skinny_amd as q4
        import synth
        self.name, self.spec, self.q4 = name, spec, q4
        t0 = time.time()
        moe = synth.moe_layer(spec["seed"], T=spec["T"], D=spec["D"], E=spec["E"], F=spec["F"], k=spec["k"],
                              has_shared=spec["has_shared"])
        self.moe = moe
        mw = q4.moe_pack_experts(moe.gate, moe.up, moe.down, moe.E, moe.has_shared)
        log(f"[bench] {name}: layer generated and packed in {time.time() - t0:.1f}s")
        self.x = torch.from_numpy(moe.x).cuda()
        self.wr = torch.from_numpy(moe.w_router).cuda()
        layer_bytes = mw.gate.numel() + mw.up.numel() + mw.down.numel()
        self.copies = 1 if hot else max(2, -(-ROTATE_BYTES // layer_bytes))
        self.layers = [mw]
        for _ in range(self.copies - 1):
            self.layers.append(q4.MoeWeights(mw.E, mw.has_shared, mw.D, mw.F, mw.gate.clone(), mw.up.clone(),
                                              mw.down.clone(), mw.g_gate, mw.g_up, mw.g_down))
        self.out = torch.empty((moe.T, moe.D), dtype=torch.float32, device="cuda")
        self.i = 0
        # algorithmic bytes: router matrix + every expert that receives a token + the shared one
        _, idx, _ = q4.moe_route_topk(self.x, self.wr, moe.k, want_logits=False)
        torch.cuda.synchronize()
        self.active = len(set(idx.cpu().numpy().ravel().tolist()))
        per_matrix = moe.F * moe.D // 2 + moe.F * moe.D // 16 + 4
        self.alg_bytes = moe.D * moe.E * 4 + (self.active + int(moe.has_shared)) * 3 * per_matrix
        self.kind = "moe"
        self.kernel_names = ["moe step: route_kernel + moe_gate_up_kernel + moe_down_kernel + moe_combine_kernel"]
        self.dtype = "f16"
        import ctypes as C
        self.descs = [m.desc() for m in self.layers]
        self.idx = torch.empty((moe.T, moe.k), dtype=torch.int32, device="cuda")
        self.w = torch.empty((moe.T, moe.k), dtype=torch.float32, device="cuda")
        self.wsb = q4.raw().moe_route_grouped_workspace_bytes(C.byref(self.descs[0]), moe.T, moe.k)
        self.ws = q4.workspace(self.wsb)

    def step(self):
        import ctypes as C
        q4 = self.q4
        d = self.descs[self.i % self.copies]
        self.i += 1
        m = self.moe
        rc = q4.raw().moe_route_grouped_qgemm(C.byref(d), C.c_void_p(self.x.data_ptr()), C.c_void_p(self.wr.data_ptr()),
                                              m.T, m.k, 0, None, C.c_void_p(self.idx.data_ptr()),
                                              C.c_void_p(self.w.data_ptr()), C.c_void_p(self.out.data_ptr()),
                                              q4.Q4_F32, C.c_void_p(self.ws.data_ptr()), self.ws.numel(),
                                              q4._stream())
        if rc != 0:
            q4._check(rc)

    def config(self):
        m = self.moe
        return {"workload": self.name, "T": m.T, "D": m.D, "E": m.E, "shared_experts": int(m.has_shared),
                "F": m.F, "top_k": m.k, "active_experts": self.active, "weights": "nvfp4",
                "weight_copies_rotated": self.copies}

    def cpu_oracle_sample(self, seconds):
        import oracle
        m = self.moe
        t0 = time.perf_counter()
        _, idx, w = oracle.route_topk(m.x, m.w_router, m.k)
        oracle.moe_ref_grouped(m, idx, w)
        el = time.perf_counter() - t0
        return self.alg_bytes / el / 1e9, f"1 full oracle layer (router + {self.active}+1 experts, T={m.T}) in {el:.1f}s"


class MoeBlockWork:
    """One step = moe_block_forward: input norms, router (matmul, then the
    block's score norm and top-k), the experts and the dense branch (one
    gate/up and one down launch), combine: 5 launches on the residual."""

    def __init__(self, name, spec, hot):
        import numpy as np
        import torch

        import moe_w4a16_skinny_amd as q4
        import synth
        self.name, self.spec, self.q4 = name, spec, q4
        t0 = time.time()
        blk = synth.moe_block(spec["seed"], T=spec["T"], D=spec["D"], E=spec["E"], F=spec["F"],
                              F_dense=spec["F_dense"], k=spec["k"])
        self.blk = blk
        bw = q4.moe_block_pack(blk)
        log(f"[bench] {name}: block generated and packed in {time.time() - t0:.1f}s")
        self.res0 = torch.from_numpy(blk.residual).cuda()
        self.res = self.res0.clone()
        ex, de = bw.experts, bw.dense
        layer_bytes = sum(t.numel() for t in (ex.gate, ex.up, ex.down, de.gate, de.up, de.down))
        self.copies = 1 if hot else max(2, -(-ROTATE_BYTES // layer_bytes))
        self.blocks = [bw]
        for _ in range(self.copies - 1):
            e2 = q4.MoeWeights(ex.E, False, ex.D, ex.F, ex.gate.clone(), ex.up.clone(), ex.down.clone(), ex.g_gate,
                               ex.g_up, ex.g_down)
            d2 = q4.MoeWeights(1, False, de.D, de.F, de.gate.clone(), de.up.clone(), de.down.clone(), de.g_gate,
                               de.g_up, de.g_down)
            self.blocks.append(q4.MoeBlockWeights(e2, d2, bw.w_router, bw.router_scale, bw.down_scale, bw.norms,
                                                  bw.eps))
        self.i = 0
        # algorithmic bytes: router matrix, dense branch, every expert that receives a token (the device's
        # routing of the initial residual), residual in and out
        _, idx, _ = q4.moe_block_forward(bw, self.res0.clone(), blk.k, want_routing=True)
        self.active = len(set(idx.cpu().numpy().ravel().tolist()))
        D, F, Fd, T = blk.D, spec["F"], spec["F_dense"], blk.T
        per = lambda f: 2 * (f * D // 2 + f * D // 16 + 4) + (D * f // 2 + D * f // 16 + 4)
        self.alg_bytes = D * blk.E * 4 + per(Fd) + self.active * per(F) + 2 * T * D * 4
        self.kind = "moe_block"
        self.kernel_names = ["block step: block_norm_in + route (with the block's scores) + 2 x (moe_gate_up + "
                             "moe_down) + block_combine"]
        self.dtype = "f16"

    def step(self):
        bw = self.blocks[self.i % self.copies]
        self.i += 1
        # the residual is updated in place, step after step, like successive layers
        self.q4.moe_block_forward(bw, self.res, self.blk.k)

    def config(self):
        b = self.blk
        return {"workload": self.name, "T": b.T, "D": b.D, "E": b.E, "F": self.spec["F"],
                "F_dense": self.spec["F_dense"], "top_k": b.k, "active_experts": self.active, "weights": "nvfp4",
                "weight_copies_rotated": self.copies}

    def cpu_oracle_sample(self, seconds):
        import oracle
        t0 = time.perf_counter()
        oracle.moe_block_ref(self.blk, self.blk.residual)
        el = time.perf_counter() - t0
        return self.alg_bytes / el / 1e9, f"1 full oracle block (T={self.blk.T}) in {el:.1f}s"


class QuantWork:
    """One step = q4_nvfp4_quantize of an fp32 [N][K] matrix with the global
    scale taken from its amax: a pass for the amax, a pass that quantizes and
    writes the packed layout."""

    def __init__(self, name, spec, hot):
        import torch

        import moe_w4a16_skinny_amd as q4
        import synth
        self.name, self.spec, self.q4 = name, spec, q4
        N, K = spec["N"], spec["K"]
        self.N, self.K = N, K
        t0 = time.time()
        w = synth.normal_f32(spec["seed"], synth.TAG_WEIGHT, N, K, spec["std"])
        self.w_host = w
        self.w = torch.from_numpy(w).cuda()  # N * K * 4 bytes >= 2 GiB at the tied-embedding size: no rotation
        log(f"[bench] {name}: matrix generated in {time.time() - t0:.1f}s")
        self.nb = q4.q4_nvfp4_packed_bytes(N, K)
        self.packed = torch.empty((self.nb,), dtype=torch.uint8, device="cuda")
        self.g = torch.empty((1,), dtype=torch.float32, device="cuda")
        self.wsb = q4.raw().q4_nvfp4_quantize_workspace_bytes()
        self.ws = q4.workspace(self.wsb)
        # algorithmic bytes: the amax pass reads w; the quantizing pass reads w
        # again and writes codes (K/2 per row) and scales (K/16 per row)
        self.alg_bytes = 2 * N * K * 4 + N * K // 2 + N * K // 16 + 4
        self.kind = "quant"
        self.kernel_names = ["quantize step: quant_zero_kernel + quant_amax_kernel + quant_pack_kernel"]
        self.dtype = "f32"
        self.copies = 1

    def step(self):
        import ctypes as C
        q4 = self.q4
        rc = q4.raw().q4_nvfp4_quantize(C.c_void_p(self.w.data_ptr()), self.N, self.K, 0.0,
                                        C.c_void_p(self.packed.data_ptr()), self.nb, C.c_void_p(self.g.data_ptr()),
                                        C.c_void_p(self.ws.data_ptr()), self.ws.numel(), q4._stream())
        if rc != 0:
            q4._check(rc)

    def config(self):
        return {"workload": self.name, "N": self.N, "K": self.K, "input": "fp32, N(0, 0.02)",
                "global_scale": "amax / (448 * 6), computed on the device", "output": "packed NVFP4"}

    def cpu_oracle_sample(self, seconds):
        """The oracle quantizer on 1024-row blocks (each taking its own amax) for about `seconds`."""
        import oracle
        rows = min(self.N, 1024)
        done = 0
        t0 = time.perf_counter()
        while True:
            r0 = (done * rows) % self.N
            oracle.nvfp4_quantize_f32(self.w_host[r0:r0 + rows])
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        bytes_done = done * rows * self.alg_bytes / self.N
        return bytes_done / el / 1e9, f"{done} oracle quantizations of {rows} rows (K={self.K}) in {el:.1f}s"


class CopyWork:
    """A plain device copy of known size, for scaling the HBM byte counters."""

    def __init__(self, mib):
        import torch
        self.nbytes = mib << 20
        self.src = torch.ones(self.nbytes // 4, dtype=torch.float32, device="cuda")
        self.dst = torch.empty_like(self.src)
        self.alg_bytes = 2 * self.nbytes
        self.kernel_names = ["copy"]
        self.dtype = "f32"

    def step(self):
        self.dst.copy_(self.src)

    def config(self):
        return {"workload": f"device_copy_{self.nbytes >> 20}MiB"}


def stream_ceiling(nbytes, steps):
    """The stream-read ceiling for `nbytes`: q4_stream_read over rotated copies
    (>= 2 GiB in total, as for the weights), each launch shape timed as a HIP
    graph of `steps` launches; the fastest shape is the ceiling."""
    import ctypes as C

    import torch

    import moe_w4a16_skinny_amd as q4
    lib = q4.raw()
    n = -(-nbytes // 16) * 16
    stride = -(-n // 4096) * 4096
    copies = max(2, -(-ROTATE_BYTES // stride))
    buf = torch.zeros(copies * stride, dtype=torch.uint8, device="cuda")
    out = torch.empty(65536, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = None
    n16 = n // 16
    shapes = [(mode, grid, depth) for mode in (0, 1) for depth in (2, 4, 8) for grid in (256, 512, 1024, 2048)]
    # and the grids in which every lane issues exactly one or two batches
    shapes += [(0, max(1, min(65536, -(-n16 // (256 * depth * nb)))), depth) for depth in (2, 4, 8) for nb in (1, 2)]
    # one batch per lane, 512-thread workgroups (the GEMMs' shape), where a
    # workgroup's chunk is at most 32 loads per lane
    shapes += [(2, grid, 0) for grid in (256, 512, 768, 1024) if -(-n16 // grid) <= 512 * 32]
    for mode, grid, depth in shapes:
        def step(i):
            rc = lib.q4_stream_read(C.c_void_p(buf.data_ptr() + (i % copies) * stride), n, grid, mode, depth,
                                    C.c_void_p(out.data_ptr()), q4._stream())
            if rc != 0:
                q4._check(rc)
        for i in range(3):
            step(i)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        if best is None or us < best["mean_launch_us"]:
            best = {"bytes": n, "mean_launch_us": round(us, 3), "GB/s": round(n / us / 1e3, 1),
                    "frac_of_peak": round(n / us / 1e3 / HBM_PEAK_GBS, 4), "grid": grid, "depth": depth,
                    "mode": ["grid-stride", "chunk per workgroup", "one batch per lane"][mode],
                    "kernel": "stream_read_kernel (q4_stream_read)"}
        del g
    del buf
    return best


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); multi-GPU sharding of this path "
              "is described in the design notes and not launched here.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import synth

    if args.copy_kernel:
        work = CopyWork(args.copy_kernel)
        name = work.config()["workload"]
    else:
        name = args.workload
        spec = synth.WORKLOADS[name]
        if spec["kind"] == "moe":
            work = MoeWork(name, spec, args.hot)
        elif spec["kind"] == "moe_block":
            work = MoeBlockWork(name, spec, args.hot)
        elif spec["kind"] == "quant":
            work = QuantWork(name, spec, args.hot)
        else:
            work = GemmWork(name, spec, args.hot)

    for _ in range(args.warmup):
        work.step()
    torch.cuda.synchronize()

    K = args.steps
    stream = torch.cuda.current_stream()
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(K):
                work.step()
        graph.replay()  # untimed: the first replay uploads the graph
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(K):
            work.step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_launch = e0.elapsed_time(e1) * 1e-3 / K  # seconds per step on the launch stream

    # dispatch interval of a trivial kernel launched the same way (stream-ordered, back to back)
    tiny = torch.zeros(1, device="cuda")
    for _ in range(20):
        tiny.add_(1.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(200):
        tiny.add_(1.0)
    e1.record(stream)
    torch.cuda.synchronize()
    launch_interval = e0.elapsed_time(e1) * 1e-3 / 200

    value = work.alg_bytes * K / wall / 1e9
    achieved = work.alg_bytes / mean_launch / 1e9
    flops = getattr(work, "flops", 0)
    mfma_bound = flops / MFMA_F16_PEAK_TFLOPS / 1e12 > work.alg_bytes / HBM_PEAK_GBS / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": work.dtype,
        "data": "synthetic (seeded; NVFP4 / affine 4-bit weights drawn and encoded by the workload recipe)",
        "config": work.config(),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(flops / mean_launch / 1e12, 2) if mfma_bound else round(achieved, 2),
            "peak": MFMA_F16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round((flops / mean_launch / 1e12 / MFMA_F16_PEAK_TFLOPS) if mfma_bound
                          else achieved / HBM_PEAK_GBS, 4),
            "traffic": (traffic_for(name, getattr(work, "kind", "gemm")) if not args.copy_kernel else None),
            "kernel": work.kernel_names[0],
            "alg_bytes_per_launch": work.alg_bytes,
            "flops_per_launch": flops,
            "mean_launch_us": round(mean_launch * 1e6, 3),
            "timing": "HIP graph of the K steps" if graph is not None else "eager launches",
            "empty_kernel_interval_us": round(launch_interval * 1e6, 3),
        },
    }
    if not args.copy_kernel and not args.no_ceiling and rec["roofline"]["bound"] == "hbm":
        ceil = stream_ceiling(work.alg_bytes, min(K, 100))
        rec["roofline"]["stream_ceiling"] = ceil
        rec["roofline"]["frac_of_ceiling"] = round(achieved / ceil["GB/s"], 4)
    if not args.no_cpu_baseline and not args.copy_kernel:
        gbs, sample = work.cpu_oracle_sample(args.cpu_seconds)
        rec["cpu_baseline"] = {"value": round(gbs, 4), "unit": "GB/s", "cores": threads_used(),
                               "kind": "oracle", "sample": sample}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
