"""Benchmark of the dual-mode INT4 linear layer and verify step on one MI355X.

Default workload (one "step" = one self-speculative round over the four
projections of one Qwen2.5-7B-shaped decoder layer at batch 8, gamma 4):
    4 draft passes:  per projection quant_act (M=8) + W4A4 GEMM (M=8)
    1 verify pass:   per projection W4A16 GEMM (M = 8 * (4+1) = 40)
    acceptance:      verify (speculative sampling) on B=8, gamma=4 logits over
                     the Qwen2.5 vocabulary (152064)
Projections (K -> N): QKV 3584->4608, O 3584->3584, gate|up 3584->37888,
down 18944->3584, all reading one shared packed INT4 buffer (g=128, fp16
scales) per pass.  Each pass reads its own copy of the packed weights (5
copies, 601 MB) so no pass is served from the 256 MB Infinity Cache.  The
step is captured once in a HIP graph and replayed; inputs are resident in HBM.

value = whole-step algorithmic HBM bytes / step time (GB/s).
roofline = the dominant kernel (W4A4 on gate|up at M=8, four launches per
step): algorithmic bytes per launch / its mean duration (HIP events around
graph replays of exactly those launches), against 8 TB/s.
cpu_baseline = the CPU oracle on a bounded sample of the same step.

Other workloads (--workload): prefill (M=2048 W4A4 vs W4A16 on the 7B
shapes), llama (Llama-3-8B lm_head GEMV at M=1 and the verify step at B=32,
V=128256).  Only the default prints the contract line's metric on the
configuration it is quoted on; the others print their own lines.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0

QWEN7B = [("qkv", 4608, 3584), ("o", 3584, 3584), ("gate_up", 37888, 3584),
          ("down", 3584, 18944)]
QWEN_VOCAB = 152064


def wbytes(N, K):
    """packed INT4 codes + fp16 group scales"""
    return N * K // 2 + N * (K // 128) * 2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
class Decode:
    """Qwen2.5-7B decode layer round: B=8, gamma=4."""

    name = "qwen2.5-7b-layer-selfspec-round"

    def __init__(self, torch, q, B=8, gamma=4, V=QWEN_VOCAB, copies=5, seed=1):
        import synth
        self.torch, self.q = torch, q
        self.B, self.gamma, self.V = B, gamma, V
        dev = "cuda:0"
        rng = synth.make_rng(1, 0)
        self.proj = []
        for name, N, K in QWEN7B:
            W = synth.weights(rng, N, K)
            Wd = torch.from_numpy(W).to(dev)
            del W
            Wq, Ws = q.pack_w4(Wd)
            del Wd
            cps = [(Wq, Ws)] + [(Wq.clone(), Ws.clone()) for _ in range(copies - 1)]
            X = synth.activations(rng, B * (gamma + 1), K, n_outliers=synth.outlier_count(K))
            Xd = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(dev)
            M4, M16 = B, B * (gamma + 1)
            self.proj.append(dict(
                name=name, N=N, K=K, copies=cps, X16=Xd, X4=Xd[:M4].contiguous(),
                Xq=torch.empty((M4, K // 2), dtype=torch.uint8, device=dev),
                Xs=torch.empty((M4,), dtype=torch.float32, device=dev),
                Y4=torch.empty((M4, N), dtype=torch.float32, device=dev),
                Y16=torch.empty((M16, N), dtype=torch.float32, device=dev),
                ws4=torch.zeros(max(1, q.workspace_bytes(1, M4, N, K)), dtype=torch.uint8, device=dev),
                ws16=torch.zeros(max(1, q.workspace_bytes(2, M16, N, K)), dtype=torch.uint8, device=dev),
            ))
        tgt, drf = synth.verify_logits(rng, B, gamma, V)
        d = synth.gumbel_drafts(rng, drf)
        vin = dict(tgt=torch.from_numpy(tgt).to(dev), drf=torch.from_numpy(drf).to(dev),
                   d=torch.from_numpy(d).to(dev),
                   ua=torch.from_numpy(synth.uniforms(rng, (B, gamma))).to(dev),
                   us=torch.from_numpy(synth.uniforms(rng, (B,))).to(dev))
        # distinct copies of the verify logits, one per step graph and more
        # than 512 MB in all, so no step finds them in the 256 MB Infinity
        # Cache (the weights of a step are 601 MB of distinct copies already)
        vb = (tgt.nbytes + drf.nbytes)
        self.vcopies = max(2, -(-(512 << 20) // vb) + 1)
        self.vins = [vin] + [dict(vin, tgt=vin["tgt"].clone(), drf=vin["drf"].clone())
                             for _ in range(self.vcopies - 1)]
        self.vin = vin
        self.host_inputs = dict(tgt=tgt, drf=drf, d=d)
        self.n_acc = torch.empty((B,), dtype=torch.int32, device=dev)
        self.out_tok = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
        self.wsv = torch.empty(q.workspace_bytes(3, B, gamma, V), dtype=torch.uint8, device=dev)
        self.dominant = "w4a4_gate_up_M8"

    # algorithmic HBM bytes --------------------------------------------------
    def bytes_w4a4(self, p):
        M, N, K = self.B, p["N"], p["K"]
        return wbytes(N, K) + M * K // 2 + M * 4 + M * N * 4

    def bytes_quant(self, p):
        M, K = self.B, p["K"]
        return M * K * 2 + M * K // 2 + M * 4

    def bytes_w4a16(self, p):
        M, N, K = self.B * (self.gamma + 1), p["N"], p["K"]
        return wbytes(N, K) + M * K * 2 + M * N * 4

    def bytes_verify(self):
        B, g, V = self.B, self.gamma, self.V
        # one pass over target and draft logits + the residual row pair
        return (B * (g + 1) * V + B * g * V) * 4 + B * 2 * V * 4

    def step_bytes(self):
        tot = 0
        for p in self.proj:
            tot += self.gamma * (self.bytes_quant(p) + self.bytes_w4a4(p)) + self.bytes_w4a16(p)
        return tot + self.bytes_verify()

    def step_ops(self):
        tot = 0
        for p in self.proj:
            tot += 2 * self.gamma * self.B * p["N"] * p["K"]
            tot += 2 * self.B * (self.gamma + 1) * p["N"] * p["K"]
        return tot

    # launches ---------------------------------------------------------------
    def draft_pass(self, d):
        q = self.q
        for p in self.proj:
            Wq, Ws = p["copies"][d]
            q.quant_act(p["X4"], p["Xq"], p["Xs"])
            q.gemm_w4a4(p["Xq"], p["Xs"], Wq, Ws, Y=p["Y4"], ws=p["ws4"])

    def verify_pass(self, c=0):
        q = self.q
        for p in self.proj:
            Wq, Ws = p["copies"][self.gamma]
            q.gemm_w4a16(p["X16"], Wq, Ws, Y=p["Y16"], ws=p["ws16"])
        v = self.vins[c]
        q.verify(q.VERIFY_SAMPLE, v["tgt"], v["d"], v["drf"], v["ua"], v["us"],
                 n_accept=self.n_acc, out_tok=self.out_tok, ws=self.wsv)

    def step(self, c=0):
        """one self-speculative round; c picks the verify logits copy"""
        for d in range(self.gamma):
            self.draft_pass(d)
        self.verify_pass(c)

    def dominant_launches(self):
        """the dominant kernel's launches of one step, same buffers"""
        q = self.q
        p = [x for x in self.proj if x["name"] == "gate_up"][0]
        for d in range(self.gamma):
            Wq, Ws = p["copies"][d]
            q.gemm_w4a4(p["Xq"], p["Xs"], Wq, Ws, Y=p["Y4"], ws=p["ws4"])
        return self.gamma, self.bytes_w4a4(p)

    # CPU oracle on a bounded sample ------------------------------------------
    def cpu_baseline(self, frac_rows=1.0):
        import oracle
        import synth
        rng = synth.make_rng(1, 7)
        work = []
        bytes_sample = 0
        for name, N, K in QWEN7B:
            n = max(16, int(round(N * frac_rows)))
            W = synth.weights(rng, n, K)
            Wq, Ws = oracle.pack_w4(W)
            X = synth.activations(rng, self.B * (self.gamma + 1), K,
                                  n_outliers=synth.outlier_count(K))
            work.append((Wq, Ws, X))
            p = dict(N=n, K=K)
            bytes_sample += self.gamma * (self.bytes_quant(p) + self.bytes_w4a4(p)) + self.bytes_w4a16(p)
        bytes_sample += self.bytes_verify()
        h = self.host_inputs
        ua = np.asarray(self.vin["ua"].cpu())
        us = np.asarray(self.vin["us"].cpu())
        # whole rounds, repeated until at least 10 s of CPU work (at most 6)
        t0 = time.perf_counter()
        rounds = 0
        while rounds < 6 and (rounds == 0 or time.perf_counter() - t0 < 10.0):
            for Wq, Ws, X in work:
                for _ in range(self.gamma):
                    Xq, Xs = oracle.quant_act(X[:self.B])
                    oracle.gemm_w4a4(Xq, Xs, Wq, Ws)
                oracle.gemm_w4a16(X, Wq, Ws)
            oracle.verify_sample(h["tgt"], h["drf"], h["d"], ua, us)
            rounds += 1
        dt = time.perf_counter() - t0
        bytes_sample *= rounds
        return dict(value=bytes_sample / dt / 1e9, unit="GB/s", cores=_blas_threads(),
                    kind="oracle",
                    sample=(f"{rounds} whole round(s) (4 draft passes, 1 verify pass, the verify "
                            f"step) on freshly drawn weights of the same shapes; {dt:.1f} s"
                            if frac_rows >= 1 else
                            f"{rounds} round(s) on {frac_rows:g} of every projection's output "
                            f"rows (all K, all M) plus the full verify step; {dt:.1f} s"))


def measure_prefill(torch, q, wl, reps=5):
    """Prefill-shaped GEMMs (M = 2048 tokens) on the same packed buffers:
    W4A4 (int8 MFMA) vs W4A16 (bf16 MFMA), per projection; kernel time from
    HIP events around graph replays of 3 launches each.  Also the W4A4 layer
    with a bf16 output (what a chained prefill hands the next op: half the
    output bytes)."""
    import synth
    rng = synth.make_rng(2, 0)
    M = 2048
    out = {}
    tot4 = tot4b = tot16 = ops_all = 0.0
    for p in wl.proj:
        N, K = p["N"], p["K"]
        X = synth.activations(rng, M, K)
        Xd = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        Xq, Xs = q.quant_act(Xd)
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        Yb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        Wq, Ws = p["copies"][0]
        t4 = _graph_time(torch, lambda: q.gemm_w4a4(Xq, Xs, Wq, Ws, Y=Y), reps)
        t4b = _graph_time(torch, lambda: q.gemm_w4a4_bf16(Xq, Xs, Wq, Ws, Y=Yb), reps)
        t16 = _graph_time(torch, lambda: q.gemm_w4a16(Xd, Wq, Ws, Y=Y), reps)
        tq = _graph_time(torch, lambda: q.quant_act(Xd, Xq, Xs), reps)
        ops = 2.0 * M * N * K
        out[p["name"]] = {"w4a4_us": round(t4, 2), "w4a4_tops": round(ops / t4 / 1e6, 1),
                          "w4a4_frac_int8": round(ops / t4 / 1e6 / INT8_PEAK_TOPS, 4),
                          "w4a4_bf16out_us": round(t4b, 2),
                          "w4a4_bf16out_frac_int8": round(ops / t4b / 1e6 / INT8_PEAK_TOPS, 4),
                          "w4a16_us": round(t16, 2), "w4a16_tflops": round(ops / t16 / 1e6, 1),
                          "w4a16_frac_bf16": round(ops / t16 / 1e6 / BF16_PEAK_TFLOPS, 4),
                          "quant_act_us": round(tq, 2), "w4a16_over_w4a4": round(t16 / t4, 3)}
        tot4 += t4
        tot4b += t4b
        tot16 += t16
        ops_all += ops
        del Xd, Xq, Xs, Y, Yb
    out["all"] = {"w4a4_tops": round(ops_all / tot4 / 1e6, 1),
                  "w4a4_frac_int8": round(ops_all / tot4 / 1e6 / INT8_PEAK_TOPS, 4),
                  "w4a4_bf16out_tops": round(ops_all / tot4b / 1e6, 1),
                  "w4a4_bf16out_frac_int8": round(ops_all / tot4b / 1e6 / INT8_PEAK_TOPS, 4),
                  "w4a16_tflops": round(ops_all / tot16 / 1e6, 1),
                  "w4a16_frac_bf16": round(ops_all / tot16 / 1e6 / BF16_PEAK_TFLOPS, 4)}
    return out


def measure_batch_sweep(torch, q, wl, reps=10, Ms=(8, 16, 32, 64, 128, 256, 512)):
    """Batched serving: one pass over the four Qwen2.5-7B projections at M
    tokens in each mode -- draft (quant_act + W4A4) and verify (W4A16) --
    with each replay reading a different weight copy (HBM).  Where the
    ratio w4a16/w4a4 passes 1 the drafter's lower precision pays for itself."""
    import synth
    rng = synth.make_rng(1, 4)
    out = {}
    for M in Ms:
        t4 = t16 = 0.0
        for p in wl.proj:
            N, K = p["N"], p["K"]
            X = torch.from_numpy(synth.activations(rng, M, K, n_outliers=synth.outlier_count(K))
                                 .view(np.int16)).view(torch.bfloat16).to("cuda:0")
            Xq = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda:0")
            Xs = torch.empty((M,), dtype=torch.float32, device="cuda:0")
            Y = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
            ws = torch.zeros(max(1, q.workspace_bytes(1, M, N, K), q.workspace_bytes(2, M, N, K)),
                             dtype=torch.uint8, device="cuda:0")
            cps = p["copies"]

            def f4():
                for Wq, Ws in cps:
                    q.quant_act(X, Xq, Xs)
                    q.gemm_w4a4(Xq, Xs, Wq, Ws, Y=Y, ws=ws)

            def f16():
                for Wq, Ws in cps:
                    q.gemm_w4a16(X, Wq, Ws, Y=Y, ws=ws)
            t4 += _graph_time(torch, f4, reps, launches=1) / len(cps)
            t16 += _graph_time(torch, f16, reps, launches=1) / len(cps)
            del X, Xq, Xs, Y, ws
        ops = sum(2.0 * M * p["N"] * p["K"] for p in wl.proj)
        out[f"M{M}"] = {"draft_w4a4_us": round(t4, 1), "verify_w4a16_us": round(t16, 1),
                        "w4a16_over_w4a4": round(t16 / t4, 3),
                        "draft_tops": round(ops / t4 / 1e6, 1), "verify_tflops": round(ops / t16 / 1e6, 1)}
    return out


def measure_rotation(torch, q, wl, reps=20):
    """Per-group Hadamard rotation ahead of the quantizers at the decode batch
    (M = 8 draft rows, M = 40 verify rows): kernel times of the rotated
    quantizer against the plain one and of the verifier's bf16 rotation, and
    the drafter layer's relative error against the exact product with and
    without the rotation (Qwen2.5-7B QKV shape, x20 outlier channels,
    512 sampled output columns computed exactly on the host)."""
    import synth
    rng = synth.make_rng(1, 5)
    out = {"times_us": {}}
    warm = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda:0")
    _graph_time(torch, lambda: q.quant_act(warm), reps)   # first graph of the process: not timed
    for p in wl.proj:
        K = p["K"]
        X8 = torch.from_numpy(synth.activations(rng, 8, K, n_outliers=synth.outlier_count(K))
                              .view(np.int16)).view(torch.bfloat16).to("cuda:0")
        X40 = torch.from_numpy(synth.activations(rng, 40, K, n_outliers=synth.outlier_count(K))
                               .view(np.int16)).view(torch.bfloat16).to("cuda:0")
        Xq = torch.empty((8, K // 2), dtype=torch.uint8, device="cuda:0")
        Xs = torch.empty((8,), dtype=torch.float32, device="cuda:0")
        Xr = torch.empty_like(X40)
        tq = _graph_time(torch, lambda: q.quant_act(X8, Xq, Xs), reps)
        tr = _graph_time(torch, lambda: q.quant_act_rot(X8, Xq, Xs), reps)
        tx = _graph_time(torch, lambda: q.rotate_x(X40, Xr), reps)
        out["times_us"][p["name"]] = {"quant_act_M8": round(tq, 2), "quant_act_rot_M8": round(tr, 2),
                                      "rotate_x_M40": round(tx, 2)}
    N, K, ncols = 4608, 3584, 512
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, 8, K, n_outliers=synth.outlier_count(K))
    cols = np.sort(rng.choice(N, size=ncols, replace=False))
    x = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = x @ W[cols].astype(np.float64).T
    Wd = torch.from_numpy(W).to("cuda:0")
    Xd = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    Wq, Ws = q.pack_w4(Wd)
    Y = q.gemm_w4a4(*q.quant_act(Xd), Wq, Ws, N=N)
    Wrq, Wrs = q.pack_w4(q.rotate_w(Wd))
    Yr = q.gemm_w4a4(*q.quant_act_rot(Xd), Wrq, Wrs, N=N)
    Y16 = q.gemm_w4a16(Xd, Wq, Ws, N=N)
    Y16r = q.gemm_w4a16(q.rotate_x(Xd), Wrq, Wrs, N=N)
    torch.cuda.synchronize()

    def rel(t):
        return round(float(np.linalg.norm(t.cpu().numpy()[:, cols] - y) / np.linalg.norm(y)), 4)
    out["rel_error_vs_exact_qkv_M8"] = {"w4a4": rel(Y), "w4a4_rotated": rel(Yr),
                                         "w4a16": rel(Y16), "w4a16_rotated": rel(Y16r)}
    return out


def measure_w4a8_tier(torch, q, wl, reps=10):
    """The W4A8 middle tier on the shared buffer at the draft batch (M = 8):
    per projection the time of quantizer + GEMM against W4A4 and W4A16, all
    three in the AUTO family (each replay reads another weight copy), and on
    the QKV shape with x20 outlier
    channels each layer's relative error against the exact product
    (512 sampled output columns computed exactly on the host)."""
    import synth
    rng = synth.make_rng(1, 6)
    out = {"times_us": {}}
    for p in wl.proj:
        N, K = p["N"], p["K"]
        X8 = p["X16"][:8].contiguous()
        Y = torch.empty((8, N), dtype=torch.float32, device="cuda:0")
        ws = torch.zeros(max(1, q.workspace_bytes(1, 8, N, K), q.workspace_bytes(2, 8, N, K),
                             q.workspace_bytes(4, 8, N, K)), dtype=torch.uint8, device="cuda:0")
        q4 = (torch.empty((8, K // 2), dtype=torch.uint8, device="cuda:0"),
              torch.empty((8,), dtype=torch.float32, device="cuda:0"))
        q8 = (torch.empty((8, K), dtype=torch.int8, device="cuda:0"),
              torch.empty((8,), dtype=torch.float32, device="cuda:0"))
        cps = p["copies"]

        def f4():
            for Wq, Ws in cps:
                q.gemm_w4a4(*q.quant_act(X8, *q4), Wq, Ws, Y=Y, ws=ws)

        def f8():
            for Wq, Ws in cps:
                q.gemm_w4a8(*q.quant_act8(X8, *q8), Wq, Ws, Y=Y, ws=ws)

        def f16():
            for Wq, Ws in cps:
                q.gemm_w4a16(X8, Wq, Ws, Y=Y, ws=ws)
        t = [_graph_time(torch, f, reps, launches=1) / len(cps) for f in (f4, f8, f16)]
        out["times_us"][p["name"]] = {"w4a4": round(t[0], 2), "w4a8": round(t[1], 2),
                                      "w4a16": round(t[2], 2)}
    N, K, ncols = 4608, 3584, 512
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, 8, K, n_outliers=synth.outlier_count(K))
    cols = np.sort(rng.choice(N, size=ncols, replace=False))
    x = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = x @ W[cols].astype(np.float64).T
    Wq, Ws = q.pack_w4(torch.from_numpy(W).to("cuda:0"))
    Xd = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    Ys = {"w4a4": q.gemm_w4a4(*q.quant_act(Xd), Wq, Ws, N=N),
          "w4a8": q.gemm_w4a8(*q.quant_act8(Xd), Wq, Ws, N=N),
          "w4a16": q.gemm_w4a16(Xd, Wq, Ws, N=N)}
    torch.cuda.synchronize()
    out["rel_error_vs_exact_qkv_M8"] = {
        k: round(float(np.linalg.norm(v.cpu().numpy()[:, cols] - y) / np.linalg.norm(y)), 4)
        for k, v in Ys.items()}
    out["note"] = ("draft-side times include the quantizer; W4A8 reads the same packed INT4 buffer "
                   "(no extra weight copy)")
    return out


def measure_decode_gemv(torch, q, wl, reps=10):
    """W4A16 at the decode-verify shapes of batch 1 (M = 1 * (4+1) = 5) on
    gate|up and down, and the Llama-3-8B lm_head (4096 -> 128256) at M = 1.
    Each replay rotates through distinct weight copies, more than 512 MB for
    every shape (the lm_head's two copies are 541 MB), so no launch finds its
    weights in the 256 MB Infinity Cache, and a replay holds enough launches
    (16 or more) that its own start-up cost is not charged to them."""
    import synth
    rng = synth.make_rng(1, 3)
    out = {}
    for p in wl.proj:
        if p["name"] not in ("gate_up", "down"):
            continue
        N, K = p["N"], p["K"]
        X = p["X16"][:5].contiguous()
        Y = torch.empty((5, N), dtype=torch.float32, device="cuda:0")
        ws = torch.zeros(max(1, q.workspace_bytes(2, 5, N, K)), dtype=torch.uint8, device="cuda:0")
        cps = list(p["copies"])
        while len(cps) < 16 or len(cps) * wbytes(N, K) <= (512 << 20):
            cps.append((cps[0][0].clone(), cps[0][1].clone()))

        def fn():
            for Wq, Ws in cps:
                q.gemm_w4a16(X, Wq, Ws, Y=Y, ws=ws)
        us = _graph_time(torch, fn, reps, launches=1) / len(cps)
        b = wbytes(N, K) + 5 * K * 2 + 5 * N * 4
        out[f"{p['name']}_M5"] = {"us": round(us, 2), "GBps": round(b / us / 1e3, 1),
                                  "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBPS, 4),
                                  "weight_copies": len(cps)}
        del cps
    N, K = 128256, 4096
    cps = []
    for _ in range(2):
        W = torch.empty((N, K), dtype=torch.float32, device="cuda:0").normal_(0.0, 0.02)
        cps.append(q.pack_w4(W))
        del W
    X = torch.from_numpy(synth.activations(rng, 1, K).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    Y = torch.empty((1, N), dtype=torch.float32, device="cuda:0")
    ws = torch.zeros(max(1, q.workspace_bytes(2, 1, N, K)), dtype=torch.uint8, device="cuda:0")

    def fh():
        for Wq, Ws in cps:
            q.gemm_w4a16(X, Wq, Ws, Y=Y, ws=ws)
    us = _graph_time(torch, fh, reps, launches=8) / len(cps)
    b = wbytes(N, K) + K * 2 + N * 4
    out["lm_head_M1"] = {"us": round(us, 2), "GBps": round(b / us / 1e3, 1),
                         "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBPS, 4)}
    del cps
    return out


def measure_llama_verify_batch(torch, q, reps=5):
    """Llama-3-8B-shaped layers in W4A16 at the verify batch of 32 sequences:
    M = 32 (gamma + 1) = 160 and 288 (gamma 4 / 8), AUTO family, each replay
    reading another weight copy (> 512 MB per shape); TFLOPS and the
    fraction of the dense bf16 MFMA peak."""
    shapes = [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 28672, 4096),
              ("down", 4096, 14336), ("lm_head", 128256, 4096)]
    out = {}
    tot = {160: [0.0, 0.0], 288: [0.0, 0.0]}
    for name, N, K in shapes:
        W = torch.empty((N, K), dtype=torch.float32, device="cuda:0").normal_(0.0, 0.02)
        Wq, Ws = q.pack_w4(W)
        del W
        nc = max(2, -(-600_000_000 // wbytes(N, K)))
        cps = [(Wq, Ws)] + [(Wq.clone(), Ws.clone()) for _ in range(nc - 1)]
        X = torch.randn((288, K), device="cuda:0").to(torch.bfloat16)
        Y = torch.empty((288, N), dtype=torch.float32, device="cuda:0")
        ws = torch.zeros(max(1, q.workspace_bytes(2, 288, N, K)), dtype=torch.uint8, device="cuda:0")
        r = {}
        for M in (160, 288):
            Xm = X[:M].contiguous()
            Ym = Y[:M]

            def fn():
                for Wc, Sc in cps:
                    q.gemm_w4a16(Xm, Wc, Sc, Y=Ym, ws=ws)
            us = _graph_time(torch, fn, reps, launches=1) / len(cps)
            tf = 2.0 * M * N * K / us / 1e6
            r[f"M{M}"] = {"us": round(us, 2), "tflops": round(tf, 1),
                          "frac_bf16": round(tf / BF16_PEAK_TFLOPS, 4)}
            tot[M][0] += 2.0 * M * N * K
            tot[M][1] += us
        out[name] = r
        del cps, Wq, Ws
        torch.cuda.empty_cache()
    for M, (fl, us) in tot.items():
        out[f"all_M{M}"] = {"tflops": round(fl / us / 1e6, 1),
                            "frac_bf16": round(fl / us / 1e6 / BF16_PEAK_TFLOPS, 4)}
    return out


def measure_verify_llama(torch, q, reps=10):
    """verify at batch 32, V = 128256 (Llama-3 vocabulary), gamma 4 and 8,
    greedy and speculative sampling; bytes = one pass over the logits read
    plus, for sampling, the residual row pair per sequence."""
    import synth
    rng = synth.make_rng(3, 0)
    B, V = 32, 128256
    out = {}
    for gamma in (4, 8):
        tgt, drf = synth.verify_logits(rng, B, gamma, V)
        d = synth.gumbel_drafts(rng, drf)
        t = lambda a: torch.from_numpy(a).to("cuda:0")  # noqa: E731
        T, D, Dt = t(tgt), t(drf), t(d)
        ua, us_ = t(synth.uniforms(rng, (B, gamma))), t(synth.uniforms(rng, (B,)))
        n_acc = torch.empty((B,), dtype=torch.int32, device="cuda:0")
        o = torch.empty((B, gamma + 1), dtype=torch.int32, device="cuda:0")
        ws = torch.empty(q.workspace_bytes(3, B, gamma, V), dtype=torch.uint8, device="cuda:0")
        bg = B * (gamma + 1) * V * 4
        bs = bg + B * gamma * V * 4 + B * 2 * V * 4
        # distinct logits copies read in turn, more than 512 MB per pass over
        # them, so no call is served from the Infinity Cache
        ncp = max(2, -(-(512 << 20) // (bg + B * gamma * V * 4)) + 1)
        cps = [(T, D)] + [(T.clone(), D.clone()) for _ in range(ncp - 1)]

        def fg():
            for Tc, _ in cps:
                q.verify(q.VERIFY_GREEDY, Tc, Dt, n_accept=n_acc, out_tok=o, ws=ws)

        def fs():
            for Tc, Dc in cps:
                q.verify(q.VERIFY_SAMPLE, Tc, Dt, Dc, ua, us_, n_accept=n_acc, out_tok=o, ws=ws)
        tg = _graph_time(torch, fg, reps, launches=1) / ncp
        ts = _graph_time(torch, fs, reps, launches=1) / ncp
        out[f"gamma{gamma}"] = {"greedy_us": round(tg, 2), "greedy_GBps": round(bg / tg / 1e3, 1),
                                "greedy_frac_hbm": round(bg / tg / 1e3 / HBM_PEAK_GBPS, 4),
                                "sample_us": round(ts, 2), "sample_GBps": round(bs / ts / 1e3, 1),
                                "sample_frac_hbm": round(bs / ts / 1e3 / HBM_PEAK_GBPS, 4),
                                "logits_copies": ncp}
        del T, D, Dt, cps
    return out


def measure_e2e(torch, B=16, P=128, n_gen=256, gamma=4):
    """The end-to-end loop: random-init 8-layer d=2048 decoder (16 q / 4 kv
    heads of 128, SwiGLU 5632, vocabulary 32000) on one shared INT4 buffer,
    batch 16, 128-token random prompts, 256 generated tokens; greedy
    self-speculation (W4A4 drafts, gamma 4, W4A16 verify) against pure W4A16
    greedy decoding of the same model, and the same loop with the W4A8 tier
    drafting."""
    import synth
    from quantization_self_speculation_amd.e2e import Decoder
    cfg = synth.E2E_MODEL
    rng = synth.make_rng(4, 0)
    w = synth.model_weights(rng, cfg)
    prompts = synth.prompts(rng, B, P, cfg.vocab)
    dec = Decoder(cfg, w, B, P, n_gen, gamma)
    dec8 = Decoder(cfg, w, B, P, n_gen, gamma, draft_mode="w4a8")
    del w
    dec.run(prompts, speculative=True, max_rounds=2)      # warm-up (graph capture, caches)
    pure = dec.run(prompts, speculative=False)
    spec = dec.run(prompts, speculative=True)
    dec8.run(prompts, speculative=True, max_rounds=2)
    spec8 = dec8.run(prompts, speculative=True)
    del dec8
    toks = B * n_gen
    alpha = spec["accepted"] / max(1, gamma * spec["active_rows"])
    alpha8 = spec8["accepted"] / max(1, gamma * spec8["active_rows"])
    return {
        "model": "random-init 8L d2048 16q/4kv x128 ffn5632 V32000, shared int4 g128",
        "batch": B, "prompt": P, "generated": n_gen, "gamma": gamma,
        "greedy_equal": bool(np.array_equal(spec["tokens"], pure["tokens"])),
        "acceptance_rate": round(alpha, 4),
        "tokens_per_round": round((spec["accepted"] + spec["active_rows"]) /
                                  max(1, spec["active_rows"]), 3),
        "rounds": spec["rounds"],
        "selfspec_tok_s": round(toks / spec["decode_s"], 1),
        "selfspec_tok_s_incl_prefill": round(toks / (spec["decode_s"] + spec["prefill_s"]), 1),
        "pure_w4a16_tok_s": round(toks / pure["decode_s"], 1),
        "pure_w4a16_tok_s_incl_prefill": round(toks / (pure["decode_s"] + pure["prefill_s"]), 1),
        "speedup_vs_pure": round(pure["decode_s"] / spec["decode_s"], 3),
        "prefill_ms": round(spec["prefill_s"] * 1e3, 3),
        "pure_ms_per_step": round(pure["decode_s"] * 1e3 / max(1, pure["rounds"]), 4),
        "selfspec_ms_per_round": round(spec["decode_s"] * 1e3 / max(1, spec["rounds"]), 4),
        # the W4A8 tier as the drafter of the same loop (same weights, same verify)
        "w4a8_drafter": {
            "greedy_equal": bool(np.array_equal(spec8["tokens"], pure["tokens"])),
            "acceptance_rate": round(alpha8, 4),
            "tokens_per_round": round((spec8["accepted"] + spec8["active_rows"]) /
                                      max(1, spec8["active_rows"]), 3),
            "rounds": spec8["rounds"],
            "selfspec_tok_s": round(toks / spec8["decode_s"], 1),
            "speedup_vs_pure": round(pure["decode_s"] / spec8["decode_s"], 3),
            "selfspec_ms_per_round": round(spec8["decode_s"] * 1e3 / max(1, spec8["rounds"]), 4),
        },
    }


def measure_ceilings(torch, q, sizes):
    """What this GPU sustains, with the library's probe kernels (qspec_probe.h):
    the pure-read rate for each byte count in `sizes` (every byte read once,
    distinct copies read in turn, more than 512 MB per pass, in a graph the
    way the hot path runs; the best of a few launch shapes), the rates of
    independent int8 and bf16 MFMA chains, and the cost of an empty launch.
    The hot path's fractions are quoted against these next to the published
    peaks."""
    pb = q.binding  # the probes are diagnostics, not package API
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    sinkf = torch.zeros(256, dtype=torch.float32, device="cuda:0")
    out = {"hbm_read_GBps": {}}
    for name, nbytes in sizes.items():
        n = int(nbytes) // 16 * 16
        ncp = max(2, -(-(512 << 20) // n) + 1)
        cps = [torch.ones(n, dtype=torch.uint8, device="cuda:0") for _ in range(ncp)]
        best = 0.0
        for blocks, unr in ((256, 8), (512, 4), (2048, 8), (2048, 16)):
            def f():
                for c in cps:
                    pb.probe_read(c, blocks, unr, sink)
            us = _graph_time(torch, f, 5, launches=1) / ncp
            best = max(best, n / us / 1e3)
        out["hbm_read_GBps"][name] = round(best, 1)
        del cps
    for kind, key, opm in ((0, "mfma_int8_TOPS", 32768), (1, "mfma_bf16_TFLOPS", 16384)):
        blocks, iters = 2048, 400
        us = _graph_time(torch, lambda: pb.probe_mfma(kind, blocks, iters, sinkf), 3, launches=1)
        out[key] = round(blocks * 4 * iters * 8 * opm / us / 1e6, 1)

    def empties():
        for _ in range(100):
            pb.probe_empty()
    out["empty_launch_us"] = round(_graph_time(torch, empties, 5, launches=1) / 100, 3)
    torch.cuda.empty_cache()
    return out


def _graph_time(torch, fn, reps, launches=3):
    """mean microseconds of fn() over graph replays (launches per replay)"""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * launches)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:
        return 1


# ---------------------------------------------------------------------------
def timed_graph(torch, fn, reps):
    """capture fn() in a HIP graph; time `reps` replays with HIP events on the
    capture stream (torch's current stream during replay)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                       # warm allocations outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def run(args):
    import torch
    import quantization_self_speculation_amd as q
    q.lib()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    log("setting up workload", args.workload)
    wl = Decode(torch, q)
    torch.cuda.synchronize()

    # one graph per verify-logits copy, replayed in turn
    g_steps = [timed_graph(torch, lambda c=c: wl.step(c), 1) for c in range(wl.vcopies)]
    box = {}

    def dom():
        box["n"], box["bytes"] = wl.dominant_launches()
    g_dom = timed_graph(torch, dom, 1)

    for i in range(args.warmup):
        g_steps[i % len(g_steps)].replay()
        g_dom.replay()
    torch.cuda.synchronize()

    # timed region: K steps, bracketed by synchronize on both sides
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        g_steps[i % len(g_steps)].replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps

    # the dominant kernel's launches alone (same buffers, same copies)
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record()
    for _ in range(args.steps):
        g_dom.replay()
    d1.record()
    torch.cuda.synchronize()
    us_dom = d0.elapsed_time(d1) * 1e3 / (args.steps * box["n"])
    achieved = box["bytes"] / (us_dom * 1e-6) / 1e9

    step_bytes = wl.step_bytes()
    value = step_bytes / (ms_step * 1e-3) / 1e9
    traffic = read_traffic()
    log("ceilings: pure reads, MFMA loops, empty launch")
    ceil = measure_ceilings(torch, q, {
        "w4a4_gate_up_M8": box["bytes"],
        "gate_up_M5": wbytes(37888, 3584) + 5 * 3584 * 2 + 5 * 37888 * 4,
        "down_M5": wbytes(3584, 18944) + 5 * 18944 * 2 + 5 * 3584 * 4,
        "lm_head_M1": wbytes(128256, 4096) + 4096 * 2 + 128256 * 4})
    read_ceil = ceil["hbm_read_GBps"]["w4a4_gate_up_M8"]

    line = {
        "metric": "W4A4/W4A16 layer TOPS & HBM GB/s vs roofline; self-spec accepted tokens/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int4-w/int8-mfma+bf16-mfma,fp32-acc",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) bf16 activations with 0.1% x20 "
                "outlier channels, N(0,3) rho=0.9 logits)",
        "config": {"workload": wl.name, "batch": wl.B, "gamma": wl.gamma,
                   "draft_M": wl.B, "verify_M": wl.B * (wl.gamma + 1), "vocab": wl.V,
                   "projections": {n: [k, nn] for n, nn, k in QWEN7B},
                   "weight_copies": 5, "step_bytes": step_bytes,
                   "step_tops": round(wl.step_ops() / (ms_step * 1e-3) / 1e12, 2)},
        "roofline": {"bound": "hbm", "kernel": wl.dominant, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "us_per_launch": round(us_dom, 3), "bytes_per_launch": box["bytes"],
                     "measured_ceiling": read_ceil,
                     "frac_of_measured": round(achieved / read_ceil, 4)},
        "ceilings_measured": ceil,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_extra:
        log("decode GEMV points")
        line["decode_gemv_w4a16"] = measure_decode_gemv(torch, q, wl)
        for k, v in line["decode_gemv_w4a16"].items():
            c = ceil["hbm_read_GBps"][k]
            v["read_ceiling_GBps"] = c
            v["frac_of_measured"] = round(v["GBps"] / c, 4)
            v["traffic"] = read_traffic("w4a16_" + k)
        log("prefill-shaped GEMMs")
        line["prefill_m2048"] = measure_prefill(torch, q, wl)
        al = line["prefill_m2048"]["all"]
        al["w4a4_frac_of_measured_int8"] = round(al["w4a4_tops"] / ceil["mfma_int8_TOPS"], 4)
        al["w4a4_bf16out_frac_of_measured_int8"] = round(al["w4a4_bf16out_tops"] / ceil["mfma_int8_TOPS"], 4)
        al["w4a16_frac_of_measured_bf16"] = round(al["w4a16_tflops"] / ceil["mfma_bf16_TFLOPS"], 4)
        log("batched serving sweep")
        line["batch_sweep_layer"] = measure_batch_sweep(torch, q, wl)
        log("rotation ahead of the quantizers")
        line["rotation"] = measure_rotation(torch, q, wl)
        log("W4A8 middle tier")
        line["w4a8_tier"] = measure_w4a8_tier(torch, q, wl)
        log("Llama-3-8B layers at the verify batch (M = 160, 288)")
        line["llama8b_w4a16_verify_batch"] = measure_llama_verify_batch(torch, q)
        log("verify at batch 32, V=128256")
        line["verify_b32_v128256"] = measure_verify_llama(torch, q)
        log("end-to-end self-speculative loop")
        line["e2e_selfspec"] = measure_e2e(torch)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        line["cpu_baseline"] = wl.cpu_baseline()
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# HBM traffic of a GEMM from rocprofv3 counters.
#   1) rocprofv3 --pmc FETCH_SIZE -d <dir> -o fetch --output-format csv -- python bench.py --counters T
#   2) the same with WRITE_SIZE (a separate run: one counter block per pass)
#   3) python bench.py --traffic <fetch counter csv> <write counter csv> --counters T
# --counters T runs a plain 1 GiB fp32 copy (calibration: 1 GiB read + 1 GiB
# written) and 20 launches of target T (the dominant kernel by default, or
# one of the W4A16 decode points); --traffic scales T's mean FETCH/WRITE KiB
# per dispatch by the copy's measured/known ratio and writes
# profiles/traffic_<T>.json, stamped with the hash of the GEMM source so a
# later kernel change voids it.
COPY_ELEMS = 1 << 28
COUNTER_TARGETS = ("w4a4_gate_up_M8", "w4a16_gate_up_M5", "w4a16_down_M5", "w4a16_lm_head_M1")
GEMM_KERNEL_TAGS = ("skinny_kernel", "stream_kernel", "gemv_kernel", "prefill_kernel")


def traffic_file(target):
    return os.path.join(ROOT, "profiles", f"traffic_{target}.json")


def run_only(which):
    import torch
    import quantization_self_speculation_amd as q
    q.lib()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if which == "verify":
        res = measure_verify_llama(torch, q)
    elif which in ("batch", "rotation", "w4a8"):
        wl = Decode(torch, q)
        torch.cuda.synchronize()
        res = {"batch": measure_batch_sweep, "rotation": measure_rotation,
               "w4a8": measure_w4a8_tier}[which](torch, q, wl)
    elif which == "llama":
        res = measure_llama_verify_batch(torch, q)
    elif which == "e2e":
        res = measure_e2e(torch)
    else:
        wl = Decode(torch, q)
        torch.cuda.synchronize()
        res = (measure_prefill if which == "prefill" else measure_decode_gemv)(torch, q, wl)
    print(json.dumps({which: res}), flush=True)


def _gemm_source_hash():
    import hashlib
    src = os.path.join(ROOT, "quantization_self_speculation_amd", "csrc", "gemm.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def _counter_workload(torch, q, target):
    """-> (launch(), algorithmic bytes of one launch) for a counter target"""
    wl = Decode(torch, q)
    if target == "w4a4_gate_up_M8":
        p = [x for x in wl.proj if x["name"] == "gate_up"][0]
        q.quant_act(p["X4"], p["Xq"], p["Xs"])
        cps = p["copies"][:4]

        def f():
            for Wq, Ws in cps:
                q.gemm_w4a4(p["Xq"], p["Xs"], Wq, Ws, Y=p["Y4"], ws=p["ws4"])
        return f, 4, wl.bytes_w4a4(p)
    if target in ("w4a16_gate_up_M5", "w4a16_down_M5"):
        p = [x for x in wl.proj if x["name"] == target.split("_", 1)[1].rsplit("_", 1)[0]][0]
        N, K = p["N"], p["K"]
        X = p["X16"][:5].contiguous()
        Y = torch.empty((5, N), dtype=torch.float32, device="cuda:0")
        ws = torch.zeros(max(1, q.workspace_bytes(2, 5, N, K)), dtype=torch.uint8, device="cuda:0")
        cps = p["copies"]

        def f():
            for Wq, Ws in cps:
                q.gemm_w4a16(X, Wq, Ws, Y=Y, ws=ws)
        return f, len(cps), wbytes(N, K) + 5 * K * 2 + 5 * N * 4
    import synth
    del wl
    N, K = 128256, 4096
    cps = []
    for _ in range(2):
        W = torch.empty((N, K), dtype=torch.float32, device="cuda:0").normal_(0.0, 0.02)
        cps.append(q.pack_w4(W))
        del W
    X = torch.from_numpy(synth.activations(synth.make_rng(1, 3), 1, K).view(np.int16)).view(
        torch.bfloat16).to("cuda:0")
    Y = torch.empty((1, N), dtype=torch.float32, device="cuda:0")
    ws = torch.zeros(max(1, q.workspace_bytes(2, 1, N, K)), dtype=torch.uint8, device="cuda:0")

    def f():
        for Wq, Ws in cps:
            q.gemm_w4a16(X, Wq, Ws, Y=Y, ws=ws)
    return f, 2, wbytes(N, K) + K * 2 + N * 4


def run_counters(target):
    import torch
    import quantization_self_speculation_amd as q
    q.lib()
    torch.cuda.set_device(0)
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    f, per_call, _ = _counter_workload(torch, q, target)
    calls = -(-20 // per_call)
    for _ in range(calls):
        f()
    torch.cuda.synchronize()
    log(f"counters workload done: 3 copies of 1 GiB, {calls * per_call} launches of {target}")


def _counter_means(path, counter):
    import csv
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    # the calibration is the 1 GiB device-to-device copy: the largest copy
    # dispatch (weight copies are smaller; torch's fill and random-number
    # kernels are not copies -- the one that fills the lm_head weights writes
    # 2 GB)
    copy = [v for (k, _), v in per.items() if "copybuffer" in k.lower()]
    dom = [v for (k, _), v in per.items() if any(t in k for t in GEMM_KERNEL_TAGS)]
    if not copy or not dom:
        raise SystemExit(f"{path}: no copy ({len(copy)}) or GEMM ({len(dom)}) dispatches for {counter}")
    return max(copy), sum(dom) / len(dom), len(dom)


def write_traffic(fetch_csv, write_csv, target):
    import torch  # noqa: F401  (the algorithmic bytes come from the workload's shapes)
    known_kib = COPY_ELEMS * 4 / 1024.0
    cf, df, nf = _counter_means(fetch_csv, "FETCH_SIZE")
    cw, dw, nw = _counter_means(write_csv, "WRITE_SIZE")
    sf, sw = known_kib / cf, known_kib / cw
    alg = {"w4a4_gate_up_M8": wbytes(37888, 3584) + 8 * 3584 // 2 + 8 * 4 + 8 * 37888 * 4,
           "w4a16_gate_up_M5": wbytes(37888, 3584) + 5 * 3584 * 2 + 5 * 37888 * 4,
           "w4a16_down_M5": wbytes(3584, 18944) + 5 * 18944 * 2 + 5 * 3584 * 4,
           "w4a16_lm_head_M1": wbytes(128256, 4096) + 4096 * 2 + 128256 * 4}[target]
    moved = int(round((df * sf + dw * sw) * 1024))
    rec = {"kernel": target, "gemm_source_sha256_16": _gemm_source_hash(),
           "fetch_kib_per_dispatch": round(df, 1), "write_kib_per_dispatch": round(dw, 1),
           "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
           "fetch_scale": round(sf, 5), "write_scale": round(sw, 5),
           "dispatches": [nf, nw],
           "bytes_per_launch": moved, "algorithmic_bytes": alg,
           "traffic_over_algorithmic": round(moved / alg, 4)}
    with open(traffic_file(target), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def read_traffic(target="w4a4_gate_up_M8"):
    """the stored traffic figure, or None when absent or taken on another
    version of the GEMM source"""
    try:
        rec = json.load(open(traffic_file(target)))
    except Exception:
        return None
    if rec.get("gemm_source_sha256_16") != _gemm_source_hash():
        return None
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the decode-GEMV, prefill and verify side measurements")
    ap.add_argument("--only", choices=["decode_gemv", "prefill", "verify", "e2e", "batch", "rotation", "w4a8", "llama"],
                    help="run one side measurement alone and print its JSON (for profiling)")
    ap.add_argument("--counters", nargs="?", const=COUNTER_TARGETS[0], choices=COUNTER_TARGETS,
                    help="run only the copy calibration and 20 launches of one GEMM (the dominant "
                         "kernel by default; for rocprofv3 --pmc)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 counter CSVs of --counters [T] into the stored "
                         "traffic figure of T")
    args = ap.parse_args()
    if args.traffic:
        write_traffic(*args.traffic, target=args.counters or COUNTER_TARGETS[0])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.counters:
        run_counters(args.counters)
        return
    if args.only:
        run_only(args.only)
        return
    run(args)


if __name__ == "__main__":
    main()
