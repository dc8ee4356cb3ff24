"""Greedy self-speculative decoding on one GPU, every step in libqspec.so.

Per round (one HIP graph, no host work inside): gamma draft forwards with the
W4A4 linear layers (one row per sequence, each at its own position), one
verify forward with the W4A16 layers over [last, d_0 .. d_{gamma-1}] that
overwrites those KV rows, the greedy verify kernel, and the device-side
commit.  The host reads one counter per round (sequences still running).
Both modes read the same packed INT4 weights and write the same KV cache
("QSpec: Speculative Decoding with Complementary Quantization Schemes",
Abstract (arXiv)); the verify step accepts the matching prefix and rewrites
the first mismatch (the agihunt.info review of SpecQuant, method paragraph).
The drafter may instead run the W4A8 tier (8-bit activation codes on the
same INT4 weights: a middle precision over one base, "SpecQuant", Abstract
(arXiv)), with the same verify step.

The W4A16 layers of decode and verify forwards use one kernel family
(`GEMM_SKINNY`), whose per-row result does not depend on the row count (the
gate|up layer with its SwiGLU in the epilogue, on rows packed in pair
order), and
every other kernel computes rows independently: a verify forward therefore
reproduces bit for bit what pure W4A16 decoding computes, and greedy
self-speculation emits exactly the pure greedy tokens.  The drafter's layers
need no such invariance (greedy verification fixes the tokens, and the
verify forward overwrites the drafter's KV rows), so they take the fastest
family for their shape (`GEMM_AUTO`).

This module is orchestration: buffers (torch allocations), graph capture and
the host loop.  The model is described by any object with the fields
vocab, d, n_layers, n_heads, n_kv, head_dim, ffn, eps, rope_base.
"""

import numpy as np
import torch

from . import binding as b

DRAFT, VERIFY, DRAFT8 = "w4a4", "w4a16", "w4a8"


def _unpair_cols(Y):
    """[M, 2F] columns in pair order (see binding.pair_rows) -> gate columns
    then up columns (a copy)."""
    M, N = Y.shape
    return Y.reshape(M, N // 16, 2, 8).transpose(1, 2).reshape(M, N).clone()


def _view(buf, *shape):
    n = 1
    for s in shape:
        n *= s
    return buf[:n].view(*shape)


class Decoder:
    """Packed weights, KV cache and work buffers of one decoder for a batch of
    B sequences with P-token prompts, up to `max_gen` generated tokens, draft
    length `gamma`."""

    def __init__(self, cfg, weights, B, P, max_gen, gamma, device="cuda:0",
                 variant=b.GEMM_SKINNY, draft_mode=DRAFT, draft_variant=b.GEMM_AUTO):
        if cfg.head_dim != 128:
            raise ValueError("head_dim must be 128")
        self.cfg, self.B, self.P, self.max_gen, self.gamma = cfg, B, P, max_gen, gamma
        self.dev = torch.device(device)
        self.variant = variant
        self.draft_variant = draft_variant
        # the drafter's layers: W4A4 (the method); W4A8 (the middle tier of
        # several precisions over one base, on the same INT4 weights);
        # W4A16 turns the drafter into the verifier itself, which must then
        # accept every draft (a check of the loop's bookkeeping)
        if draft_mode not in (DRAFT, DRAFT8, VERIFY):
            raise ValueError("draft_mode must be 'w4a4', 'w4a8' or 'w4a16'")
        self.draft_mode = draft_mode
        dev = self.dev

        def packed(W):
            Wd = torch.as_tensor(np.ascontiguousarray(W)).to(dev)
            Wq, Ws = b.pack_w4(Wd)
            del Wd
            return (Wq, Ws, int(W.shape[0]), int(W.shape[1]))

        emb = np.ascontiguousarray(weights["emb"]).view(np.int16)
        self.emb = torch.from_numpy(emb).to(dev).view(torch.bfloat16)
        # gate|up rows in pair order (8 gate rows, then their 8 up rows, per
        # 16-row block): the W4A16 layer can then finish with the SwiGLU in
        # its epilogue (qspec_gemm_w4a16_swiglu); the drafters' outputs go
        # through the pair-order silu_mul
        if cfg.ffn % 8 != 0:
            raise ValueError("ffn must be a multiple of 8")
        self.layers = [{k: packed(b.pair_rows(L[k]) if k == "gu" else L[k])
                        for k in ("qkv", "o", "gu", "down")}
                       for L in weights["layers"]]
        self.lm = packed(weights["lm"])

        # a frozen sequence keeps being drafted and verified at positions up to
        # len - 1 + gamma with len <= P + max_gen + gamma
        self.cap = P + max_gen + 2 * gamma + 1
        kvshape = (B, cfg.n_kv, self.cap, cfg.head_dim)
        self.kc = [torch.zeros(kvshape, dtype=torch.bfloat16, device=dev) for _ in self.layers]
        self.vc = [torch.zeros(kvshape, dtype=torch.bfloat16, device=dev) for _ in self.layers]

        Mmax = max(B * P, B * (gamma + 1))
        d, F = cfg.d, cfg.ffn
        qd = cfg.n_heads * cfg.head_dim
        qkv_rows = qd + 2 * cfg.n_kv * cfg.head_dim
        Kmax = max(d, qd, F)
        f32, bf, i32 = torch.float32, torch.bfloat16, torch.int32
        self.x = torch.empty(Mmax * d, dtype=f32, device=dev)
        self.h = torch.empty(Mmax * Kmax, dtype=bf, device=dev)
        self.qkv = torch.empty(Mmax * qkv_rows, dtype=f32, device=dev)
        self.q = torch.empty(Mmax * qd, dtype=f32, device=dev)
        self.att = torch.empty(Mmax * qd, dtype=bf, device=dev)
        self.o = torch.empty(Mmax * d, dtype=f32, device=dev)
        self.gu = torch.empty(Mmax * 2 * F, dtype=f32, device=dev)
        self.a = torch.empty(Mmax * F, dtype=bf, device=dev)
        self.dn = torch.empty(Mmax * d, dtype=f32, device=dev)
        Mlog = max(B, B * (gamma + 1))
        self.logits = torch.empty(Mlog * cfg.vocab, dtype=f32, device=dev)
        self.Xq = torch.empty(Mmax * Kmax // 2, dtype=torch.uint8, device=dev)
        self.Xs = torch.empty(Mmax, dtype=f32, device=dev)
        # 8-bit codes of a W4A8 forward (draft forwards have B rows)
        self.Xq8 = torch.empty(B * Kmax, dtype=torch.int8, device=dev)
        ws = 1
        for M in (B, B * (gamma + 1), B * P):
            for W in [t for L in self.layers for t in L.values()] + [self.lm]:
                _, _, N, K = W
                ws = max(ws, b.workspace_bytes(b.OP_GEMM_W4A16, M, N, K),
                         b.workspace_bytes(b.OP_GEMM_W4A4, M, N, K),
                         b.workspace_bytes(b.OP_GEMM_W4A8, M, N, K))
        self.ws = torch.zeros(ws, dtype=torch.uint8, device=dev)   # zero before first use
        self.wsv = torch.empty(max(1, b.workspace_bytes(b.OP_VERIFY, B, max(gamma, 1), cfg.vocab)),
                               dtype=torch.uint8, device=dev)
        # row descriptors and round state
        self.seq = torch.empty(Mmax, dtype=i32, device=dev)
        self.pos = torch.empty(Mmax, dtype=i32, device=dev)
        self.tok = torch.empty(Mmax, dtype=i32, device=dev)
        self.len = torch.empty(B, dtype=i32, device=dev)
        self.vtok = torch.zeros(B * (gamma + 1), dtype=i32, device=dev)
        self.drafts = torch.zeros(B * max(gamma, 1), dtype=i32, device=dev)
        self.n_acc = torch.zeros(B, dtype=i32, device=dev)
        self.out_tok = torch.zeros(B * (gamma + 1), dtype=i32, device=dev)
        self.first = torch.zeros(B, dtype=i32, device=dev)
        self.gen = torch.zeros((B, max_gen + gamma + 1), dtype=i32, device=dev)
        self.n_gen = torch.zeros(B, dtype=i32, device=dev)
        self.stats = torch.zeros(3, dtype=torch.int64, device=dev)

    # ------------------------------------------------------------ one forward
    def _codes(self, M, K):
        return _view(self.Xq, M, K // 2), _view(self.Xs, M)

    def _linear(self, mode, X, W, Y, variant, coded=False):
        """coded: the producer of X already wrote its 4-bit codes into the
        code buffers (draft mode)."""
        Wq, Ws, N, K = W
        M = X.shape[0]
        if mode == DRAFT:
            Xq, Xs = self._codes(M, K)
            if not coded:
                b.quant_act(X, Xq, Xs)
            b.gemm_w4a4(Xq, Xs, Wq, Ws, variant=variant, Y=Y, ws=self.ws, N=N)
        elif mode == DRAFT8:
            Xq8, Xs = _view(self.Xq8, M, K), _view(self.Xs, M)
            if not coded:
                b.quant_act8(X, Xq8, Xs)
            b.gemm_w4a8(Xq8, Xs, Wq, Ws, variant=variant, Y=Y, ws=self.ws, N=N)
        else:
            b.gemm_w4a16(X, Wq, Ws, variant=variant, Y=Y, ws=self.ws, N=N)

    def _gu_family(self, mode, M, variant):
        """The family of the fused gate|up + SwiGLU launch for this forward,
        or None where the layer runs unfused: the verifier's SKINNY family
        (a row's bits the same at every M) and the drafters' STREAM family."""
        N, K = 2 * self.cfg.ffn, self.cfg.d
        if mode == VERIFY:
            return b.GEMM_SKINNY if variant == b.GEMM_SKINNY else None
        op = b.OP_GEMM_W4A4 if mode == DRAFT else b.OP_GEMM_W4A8
        fam = b.gemm_family(op, M, N, K, variant)
        return fam if fam == b.GEMM_STREAM else None

    def forward(self, mode, M, variant, last_of=None, trace=None):
        """rows 0..M-1 described by self.seq/pos/tok; logits of every row (or,
        with last_of=P, of rows P-1, 2P-1, ...) land in self.logits.  With a
        list `trace`, copies of every linear layer's input and output are
        appended as (layer, name, input, output) for op-by-op checks."""
        cfg = self.cfg
        d, F = cfg.d, cfg.ffn
        qd = cfg.n_heads * cfg.head_dim
        qkv_rows = qd + 2 * cfg.n_kv * cfg.head_dim
        # B rows are one row per sequence (spec_prepare's phase 0, or a
        # one-token prefill): RoPE and attention then share one launch
        one_per_seq = M == self.B

        def lin(li, name, X, W, Y, coded=False):
            self._linear(mode, X, W, Y, variant, coded)
            if trace is not None:
                # gate|up outputs back in gate-then-up column order
                trace.append((li, name, X.clone(), _unpair_cols(Y) if name == "gu" else Y.clone()))

        # in draft modes the RMSNorm kernel also writes the drafter's 4-bit
        # (W4A4) or 8-bit (W4A8) codes of its bf16 output (one launch, not two)
        draft = mode in (DRAFT, DRAFT8)

        def norm(x_, add_, h_):
            if mode == DRAFT:
                b.add_rmsnorm_quant(x_, add_, h_, *self._codes(h_.shape[0], d), cfg.eps)
            elif mode == DRAFT8:
                rows = h_.shape[0]
                b.add_rmsnorm_quant8(x_, add_, h_, _view(self.Xq8, rows, d), _view(self.Xs, rows),
                                     cfg.eps)
            else:
                b.add_rmsnorm(x_, add_, h_, cfg.eps)

        x = _view(self.x, M, d)
        b.embed(self.emb, self.tok[:M], x)
        add = None
        for li, L in enumerate(self.layers):
            h = _view(self.h, M, d)
            norm(x, add, h)
            qkv = _view(self.qkv, M, qkv_rows)
            lin(li, "qkv", h, L["qkv"], qkv, coded=draft)
            q = _view(self.q, M, qd)
            att = _view(self.att, M, qd)
            if one_per_seq:
                # decode and draft forwards: one launch, the same bits
                b.rope_attention(qkv, self.seq, self.pos, q, self.kc[li], self.vc[li], att,
                                 cfg.n_heads, cfg.n_kv, cfg.rope_base)
            else:
                b.rope_kv(qkv, self.seq, self.pos, q, self.kc[li], self.vc[li], cfg.n_heads,
                          cfg.n_kv, cfg.rope_base)
                b.attention(q, self.kc[li], self.vc[li], self.seq, self.pos, att, cfg.n_heads,
                            cfg.n_kv)
            o = _view(self.o, M, d)
            lin(li, "o", att, L["o"], o)
            norm(x, o, h)
            gu = _view(self.gu, M, 2 * F)
            a = _view(self.a, M, F)
            fam = self._gu_family(mode, M, variant)
            if fam is not None:
                # one launch: the gate|up layer and its SwiGLU
                Wq, Ws, N, K = L["gu"]
                if mode == VERIFY:
                    b.gemm_w4a16_swiglu(h, Wq, Ws, A=a, ws=self.ws, N=N)
                elif mode == DRAFT:
                    b.gemm_w4a4_swiglu(*self._codes(M, K), Wq, Ws, A=a, N=N)
                else:  # the codes of h, written by the RMSNorm above
                    Xq8, Xs = _view(self.Xq8, M, K), _view(self.Xs, M)
                    b.gemm_w4a8_swiglu(Xq8, Xs, Wq, Ws, A=a, N=N)
                if trace is not None:
                    trace.append((li, "gu_swiglu", h.clone(), a.clone()))
            else:
                lin(li, "gu", h, L["gu"], gu, coded=draft)
                b.silu_mul_pairs(gu, a)
            dn = _view(self.dn, M, d)
            lin(li, "down", a, L["down"], dn)
            add = dn
        if last_of is None:
            rows, xs, adds = M, x, add
        else:
            rows = M // last_of
            xs, adds = x[last_of - 1::last_of], add[last_of - 1::last_of]
        hf = _view(self.h, rows, d)
        norm(xs, adds, hf)
        logits = _view(self.logits, rows, cfg.vocab)
        lin(len(self.layers), "lm", hf, self.lm, logits, coded=draft)
        return logits

    # ------------------------------------------------------------ phases
    def reset(self):
        for t in self.kc + self.vc:
            t.zero_()
        self.stats.zero_()
        self.n_gen.zero_()
        self.gen.zero_()
        self.vtok.zero_()

    def prefill(self, prompts):
        """W4A16 over all prompt rows; the first generated token of every
        sequence is committed (gen, len = P + 1, vtok[:, 0])."""
        B, P = self.B, self.P
        pr = torch.as_tensor(np.ascontiguousarray(prompts, dtype=np.int32)).to(self.dev)
        self.tok[:B * P].copy_(pr.view(-1))
        self.seq[:B * P].copy_(torch.arange(B, device=self.dev, dtype=torch.int32)
                               .repeat_interleave(P))
        self.pos[:B * P].copy_(torch.arange(P, device=self.dev, dtype=torch.int32).repeat(B))
        logits = self.forward(VERIFY, B * P, b.GEMM_AUTO, last_of=P)
        b.argmax(logits, self.first)
        self.len.fill_(P)
        b.spec_commit(B, 0, None, self.first, self.len, self.vtok, self.gamma + 1, self.gen,
                      self.n_gen, self.max_gen, self.stats)

    def _round(self):
        B, g = self.B, self.gamma
        V = self.cfg.vocab
        for j in range(g):
            b.spec_prepare(0, B, g, j, self.len, self.vtok, None, self.seq, self.pos, self.tok)
            # a W4A16 drafter stays in the verifier's family (its drafts must
            # be exactly the verifier's tokens); the W4A4 drafter takes its own
            dv = self.variant if self.draft_mode == VERIFY else self.draft_variant
            logits = self.forward(self.draft_mode, B, dv)
            b.argmax(logits, self.vtok[j + 1:], out_stride=g + 1)
        b.spec_prepare(1, B, g, 0, self.len, self.vtok, self.drafts, self.seq, self.pos, self.tok)
        logits = self.forward(VERIFY, B * (g + 1), self.variant)
        b.verify(b.VERIFY_GREEDY, logits.view(B, g + 1, V), self.drafts.view(B, g),
                 n_accept=self.n_acc, out_tok=self.out_tok.view(B, g + 1), ws=self.wsv)
        b.spec_commit(B, g, self.n_acc, self.out_tok, self.len, self.vtok, g + 1, self.gen,
                      self.n_gen, self.max_gen, self.stats)

    def _step(self):
        """one pure W4A16 greedy decode step (gamma plays no part)"""
        B = self.B
        b.spec_prepare(0, B, 0, 0, self.len, self.vtok, None, self.seq, self.pos, self.tok)
        logits = self.forward(VERIFY, B, self.variant)
        b.argmax(logits, self.out_tok)
        b.spec_commit(B, 0, None, self.out_tok, self.len, self.vtok, 1, self.gen, self.n_gen,
                      self.max_gen, self.stats)

    def _capture(self, fn):
        s = torch.cuda.Stream(device=self.dev)
        s.wait_stream(torch.cuda.current_stream(self.dev))
        torch.cuda.synchronize(self.dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
        torch.cuda.synchronize(self.dev)
        return g

    # ------------------------------------------------------------ loops
    def run(self, prompts, speculative, use_graph=True, max_rounds=None, record=None):
        """Prefill then decode greedily until every sequence has max_gen
        tokens.  Returns dict(tokens [B, max_gen] int32 numpy, rounds,
        accepted, drafted_rows, prefill_s, decode_s).  With a list `record`
        (speculative only; it reads device state after every round, so the
        timings then include those reads), every round appends dict(n_gen [B]
        = tokens generated before the round, active [B] bool = n_gen <
        max_gen, drafts [B, gamma], n_accept [B])."""
        if speculative and self.gamma < 1:
            raise ValueError("speculative decoding needs gamma >= 1")
        self.reset()
        fn = self._round if speculative else self._step
        graph = self._capture(fn) if use_graph else None
        torch.cuda.synchronize(self.dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e2 = torch.cuda.Event(enable_timing=True)
        e0.record()
        self.prefill(prompts)
        if not speculative:
            # the pure step keeps each sequence's last token at vtok[b] (row
            # stride 1); the prefill commit wrote it with the round's stride
            self.vtok[:self.B].copy_(self.first)
        # the round statistics count decode rounds only (the prefill commit
        # counts its rows as active)
        self.stats[:2].zero_()
        e1.record()
        rounds = 0
        if speculative:
            limit = self.max_gen if max_rounds is None else max_rounds
            B, g = self.B, self.gamma
            while rounds < limit:
                if record is not None:
                    n_gen0 = self.n_gen.cpu().numpy()
                graph.replay() if graph is not None else fn()
                rounds += 1
                if record is not None:
                    record.append(dict(n_gen=n_gen0, active=n_gen0 < self.max_gen,
                                       drafts=self.vtok.view(B, g + 1)[:, 1:].cpu().numpy(),
                                       n_accept=self.n_acc.cpu().numpy()))
                if int(self.stats[2].item()) == 0:
                    break
        else:
            for _ in range(self.max_gen - 1):
                graph.replay() if graph is not None else fn()
                rounds += 1
        e2.record()
        torch.cuda.synchronize(self.dev)
        st = self.stats.cpu().numpy()
        return dict(tokens=self.gen[:, :self.max_gen].cpu().numpy(), rounds=rounds,
                    accepted=int(st[0]), active_rows=int(st[1]),
                    prefill_s=e0.elapsed_time(e1) / 1e3, decode_s=e1.elapsed_time(e2) / 1e3)
