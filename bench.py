#!/usr/bin/env python3
"""Decode-step benchmark of the C-ABI library on one MI355X.

One step = one decode step of every sequence in the batch: for each loop t
in order and each layer, one decode call (latent scan + exact window +
combine), then each layer's latent writes (Eq. 2 of the Hybrid Latent
Attention summary).  Inputs are synthetic and resident in HBM before timing.

Prints ONE JSON line: decode tokens/s, the step's algorithmic HBM bytes per
second and its fraction of 8 TB/s, the dominant kernel's roofline figures
(timed live with HIP events around its launches), and the fp64 oracle timed
on the host cores on a bounded sample.
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode tokens/s and achieved HBM GB/s (% roofline), Ouro-1.4B shape, 4k ctx"
METRIC_PARALLEL = "parallel-pass positions/s and attention MFMA TFLOP/s (% roofline), Ouro-1.4B shape"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="workload number (3 = HLA, batch 128, 4k)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--entry", choices=["auto", "hla", "absorbed", "reconstruct", "full", "parallel"],
                    default="auto",
                    help="decode entry point (auto: hla for HLA workloads, reconstruct for LLA ones; "
                         "full: the uncompressed per-loop cache at the workload's attention shape; "
                         "parallel: the second pass over whole sequences, batch 8 x 2048 positions "
                         "unless --batch / --context say otherwise)")
    ap.add_argument("--context", type=int, default=0, help="override the context / sequence length (0 = default)")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch (0 = workload's)")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = workload's)")
    ap.add_argument("--fused", action="store_true",
                    help="absorbed / HLA reads as one fused launch per call (LLA_FLAG_FUSED)")
    ap.add_argument("--latent-fp8", action="store_true",
                    help="store latents as OCP e4m3 codes with per-token scales (absorbed / HLA entries)")
    ap.add_argument("--writes", choices=["auto", "serial", "overlapped"], default="auto",
                    help="serial: the step's latent writes after all its decode calls, on one stream; "
                         "overlapped: each layer's writes on a second stream once its last-loop decode call is "
                         "issued; auto: overlapped for the HLA entry (workload 3: 19.00 -> 18.94 ms per step with "
                         "the GPU idle before each run), serial for the LLA entries (workload 2's writes slowed its "
                         "scans)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every kernel eagerly instead of replaying the step as one HIP graph")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run one device-to-device copy of BYTES (HBM counter calibration)")
    return ap.parse_args()


class Hip:
    """Raw HIP events (the library's kernels run on torch's current stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventSynchronize(b) == 0
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)


# --------------------------------------------------------------------------- HLA
ENTRY_CODE = {"reconstruct": 0, "absorbed": 1, "hla": 2}


def fp8_store_fill(desc, n_pages, seed, std):
    """A synthetic fp8 latent store on the device: codes uniform over the
    finite e4m3 codes (0x7F and 0xFF, the NaNs, moved one code down) and
    per-token scales std * 4/448 * U[0.5, 1.5) (a part's max |x| near 4 std
    maps to the top code) in the 128 scale bytes that end each 16-token tile."""
    import torch
    from compressed_cross_loop_amd import binding as B
    R = desc.r_k + desc.r_v
    tb = 16 * R + 128
    g = torch.Generator(device="cuda")
    g.manual_seed(int(seed))
    raw = torch.empty(B.store_bytes(desc, n_pages), dtype=torch.uint8, device="cuda").random_(0, 256, generator=g)
    raw.sub_(((raw & 0x7F) == 0x7F).to(torch.uint8))
    scales = raw.view(-1, tb)[:, 16 * R:].view(torch.float32)
    scales.uniform_(0.5, 1.5, generator=g).mul_(std * 4.0 / 448.0)
    return raw


class DecodeStep:
    """Every buffer of one decode step (all layers, all loops), on the GPU."""

    def __init__(self, w, splits=0, seed=0, entry="auto", fp8=False, flags=0, overlap_writes=True):
        import torch
        from compressed_cross_loop_amd import binding as B
        from synth import gen
        self.torch, self.B, self.w = torch, B, w
        dev = "cuda"
        dt = gen.TORCH_DTYPE[w.dtype]
        L, T, H, dh, Bt, P, W = w.layers, w.loops, w.heads, w.head_dim, w.batch, w.page_size, w.window
        self.i = w.context - 1
        ppseq = -(-w.context // P)
        self.sets = []
        for k, s in enumerate(w.sets):
            desc = B.set_desc(n_heads=H, head_dim=dh, groups=s.groups, r_k=s.r_k, r_v=s.r_v,
                              loop_first=s.loop_first, loop_last=s.loop_last, page_size=P,
                              rope_baked=w.rope_baked, rope_base=w.rope_base,
                              dtype=B.LLA_BF16 if w.dtype == "bf16" else B.LLA_F32, latent_fp8=int(fp8))
            g = gen.rng(seed, 77, k)
            bt = torch.from_numpy(gen.block_table(g, Bt, ppseq)[0]).to(dev)
            n_pages = Bt * ppseq
            row = s.groups * P * (s.r_k + s.r_v)
            std = float(np.sqrt(s.n_loops))  # latents of |L_s| unit-variance loops
            traj = None
            if w.inputs == "trajectory":
                traj = [self.trajectory_layer(w, s, desc, bt, n_pages, seed * 1000 + 10 * l + k) for l in range(L)]
                pages = [t["pages"] for t in traj]
                enc = [t["enc"] for t in traj]
                x = [t["cur"][:, None].contiguous() for t in traj]
            else:
                if fp8:
                    pages = [fp8_store_fill(desc, n_pages, seed * 1000 + 10 * l + k, std) for l in range(L)]
                else:
                    pages = [gen.device_normal((n_pages, row), w.dtype, seed * 1000 + 10 * l + k, std)
                             for l in range(L)]
                enc = [gen.device_normal((s.n_loops, s.groups, s.r_k + s.r_v, s.d_in), w.dtype,
                                         seed * 1000 + 500 + 10 * l + k, 1.0 / np.sqrt(s.d_in)) for l in range(L)]
                x = [gen.device_normal((Bt, 1, s.n_loops, s.groups, s.d_in), w.dtype,
                                       seed * 1000 + 700 + 10 * l + k) for l in range(L)]
            self.sets.append(dict(spec=s, desc=desc, bt=bt, pages=pages, enc=enc, x=x, traj=traj,
                                  stores=[B.store(pg, bt) for pg in pages]))
        self.pos = torch.full((Bt,), self.i, dtype=torch.int32, device=dev)
        self.wpos = torch.full((Bt, 1), self.i, dtype=torch.int32, device=dev)
        ws = max(B.lla_decode_workspace_bytes(st["desc"], Bt, self.i, W, splits) for st in self.sets)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        wws = max(B.lla_write_workspace_bytes(st["desc"], Bt, 1, st["spec"].d_in) for st in self.sets)
        self.wws = torch.empty(max(wws, 256), dtype=torch.uint8, device=dev)
        self.fp8 = fp8
        self.flags = flags
        # The token's latents are written into the store at position i, and the
        # step's decode calls read latent tokens below i - W only (the token
        # itself is in the exact window), so no call of the step reads them:
        # each layer's writes may run beside the remaining decode calls, from
        # the point where a model would have that layer's last-loop state.
        self.overlap_writes = overlap_writes
        self.side = torch.cuda.Stream() if overlap_writes else None
        self.layer_done = [torch.cuda.Event() for _ in range(L)] if overlap_writes else None
        self.calls = []   # (loop, set index, desc, store, args)
        self.outs = []
        for t in range(1, T + 1):
            k = w.set_for_loop(t)
            s = w.sets[k]
            for l in range(L):
                sd = seed * 100000 + 1000 * t + 10 * l
                q = gen.device_normal((Bt, H, dh), w.dtype, sd + 1)
                traj = self.sets[k]["traj"]
                if traj is not None:
                    # the current token's own loop-t key and value; the loop's
                    # fitted decoders (B_t^T = U^V_t)
                    cur = traj[l]["cur"][:, t - s.loop_first]
                    kc, vc = cur[..., :dh].contiguous(), cur[..., dh:].contiguous()
                    A_np, Bv_np = traj[l]["codec"].decoders(t - s.loop_first + 1)
                    A = gen.as_stored(A_np, w.dtype).to(dev)
                    Bm = gen.as_stored(Bv_np.transpose(0, 2, 1), w.dtype).to(dev)
                    ex_std = 1.0
                else:
                    ex_std = float(np.sqrt(s.n_loops))
                    kc = gen.device_normal((Bt, H, dh), w.dtype, sd + 2, ex_std)
                    vc = gen.device_normal((Bt, H, dh), w.dtype, sd + 3, ex_std)
                    A = gen.device_normal((H, dh, s.r_k), w.dtype, sd + 6, 1.0 / np.sqrt(s.r_k))
                    Bm = gen.device_normal((H, dh, s.r_v), w.dtype, sd + 7, 1.0 / np.sqrt(s.r_v))   # B_t^T
                rk = gen.device_normal((Bt, W + 1, H, dh), w.dtype, sd + 4, ex_std)
                rv = gen.device_normal((Bt, W + 1, H, dh), w.dtype, sd + 5, ex_std)
                out = torch.empty((Bt, H, dh), dtype=dt, device=dev)
                bufs = (q, kc, vc, rk, rv, A, Bm, out)
                args = B.decode_args(loop=t, window=W, pos=self.pos, q=q, k_cur=kc, v_cur=vc, ring_k=rk,
                                     ring_v=rv, A=A, B=Bm, out=out, workspace=self.ws,
                                     max_pos_hint=self.i, splits=splits, flags=flags)
                self.calls.append((t, k, l, self.sets[k]["desc"], self.sets[k]["stores"][l], args, bufs))
        if entry == "auto":
            entry = "hla" if w.family == "hla" else "reconstruct"
        self.entry_name = entry
        self.entry = {"hla": B.hla_decode_windowed, "absorbed": B.lla_decode_absorbed,
                      "reconstruct": B.lla_decode_reconstruct}[entry]
        torch.cuda.synchronize()

    def trajectory_layer(self, w, s, desc, bt, n_pages, seed):
        """One layer's store built from per-head loop trajectories (rank 8 +
        0.05 noise), with decoders fit to a calibration sample: the writer
        fills tokens 0..i-1 in one bulk call.  Returns the pages, the encoders,
        the codec and the current token's trajectory cur [B, T, H, 2 d_h]."""
        torch, B = self.torch, self.B
        from synth import gen
        i, Bt = self.i, w.batch
        codec = gen.trajectory_codec(seed, heads=w.heads, head_dim=w.head_dim, loops=s.n_loops, rank=8,
                                     r=s.r_k, noise=0.05)
        x = gen.trajectory_tokens(codec, batch=Bt, n_tok=i + 1, seed=seed + 1, dtype=w.dtype)
        enc = gen.as_stored(codec.encoders(), w.dtype).cuda()
        pages = torch.empty((n_pages, s.groups * w.page_size * (s.r_k + s.r_v)), dtype=x.dtype, device="cuda")
        if i > 0:
            xw = x[:, :i].contiguous()
            wpos = torch.arange(i, dtype=torch.int32, device="cuda").repeat(Bt, 1).contiguous()
            ws = torch.empty(max(B.lla_write_workspace_bytes(desc, Bt, i, s.d_in), 4), dtype=torch.uint8,
                             device="cuda")
            B.lla_write_latents(desc, B.store(pages, bt), pos=wpos, x=xw, enc=enc, workspace=ws)
            torch.cuda.synchronize()
            del xw, wpos, ws
        return dict(pages=pages, enc=enc, codec=codec, cur=x[:, i].contiguous())

    def write_layer(self, l, stream=None):
        for st in self.sets:
            self.B.lla_write_latents(st["desc"], st["stores"][l], pos=self.wpos, x=st["x"][l],
                                     enc=st["enc"][l], workspace=self.wws, stream=stream)

    def step(self):
        import torch
        T = self.w.loops
        if not self.overlap_writes:
            for (t, k, l, desc, st, args, _) in self.calls:
                self.entry(desc, st, self.w.batch, args)
            for l in range(self.w.layers):
                self.write_layer(l)
            return
        main = torch.cuda.current_stream()
        for (t, k, l, desc, st, args, _) in self.calls:
            self.entry(desc, st, self.w.batch, args)
            if t == T:
                # layer l's last loop is issued: its writes go on the side stream
                self.layer_done[l].record(main)
                self.side.wait_event(self.layer_done[l])
                self.write_layer(l, stream=self.side)
        main.wait_stream(self.side)

    def step_bytes(self):
        """Algorithmic HBM bytes of one step (what the method itself must move)."""
        w = self.w
        e = 2 if w.dtype == "bf16" else 4
        H, dh, Bt, W = w.heads, w.head_dim, w.batch, w.window
        n_lat = max(0, self.i - W)
        n_win = min(W, self.i)
        total = 0
        per_call = {}
        # one token's latent of one group: r_k + r_v elements, or as fp8 codes
        # one byte each plus the two fp32 scales
        row = (lambda s: s.r_k + s.r_v + 8) if self.fp8 else (lambda s: (s.r_k + s.r_v) * e)
        for (t, k, l, *_rest) in self.calls:
            s = w.sets[k]
            lat = Bt * n_lat * s.groups * row(s)
            win = Bt * n_win * H * dh * 2 * e
            act = Bt * H * dh * e * (4 + 2)          # q, k_cur, v_cur, out + ring slot write (K, V)
            maps = H * dh * (s.r_k + s.r_v) * e
            # bytes the scan kernel itself must read: latents (+ the exact window,
            # fused into the scan on the matrix-core path) (+ the decoders when
            # keys and values are rebuilt)
            scan = lat + (win if self.entry_name != "reconstruct" else maps)
            flop = 2 * Bt * n_lat * s.groups * (s.r_k + s.r_v) * (H // s.groups) * \
                (dh if self.entry_name == "reconstruct" else 1) * (1 if self.entry_name == "reconstruct" else 2)
            per_call[k] = (scan, lat + win + act + maps, flop)
            total += lat + win + act + maps
        for s in w.sets:
            total += w.layers * (Bt * s.n_loops * s.groups * s.d_in * e
                                 + s.n_loops * s.groups * (s.r_k + s.r_v) * s.d_in * e
                                 + Bt * s.groups * row(s))
        return total, per_call


class ParallelStep:
    """One step of the parallel (second) pass over whole sequences, every
    layer: the latent writes of every token (both sets), then one parallel
    attention call per (layer, loop) in loop order.  Every layer and loop has
    its own store, maps and q / k / v."""

    def __init__(self, w, seed=0):
        import torch
        from compressed_cross_loop_amd import binding as B
        from synth import gen
        self.torch, self.B, self.w = torch, B, w
        dev = "cuda"
        L, T, H, dh, Bt, P, W, n = w.layers, w.loops, w.heads, w.head_dim, w.batch, w.page_size, w.window, w.context
        pps = -(-n // P)
        self.sets = []
        for k, s in enumerate(w.sets):
            desc = B.set_desc(n_heads=H, head_dim=dh, groups=s.groups, r_k=s.r_k, r_v=s.r_v,
                              loop_first=s.loop_first, loop_last=s.loop_last, page_size=P,
                              rope_baked=w.rope_baked, rope_base=w.rope_base, dtype=B.LLA_BF16)
            bt = torch.from_numpy(gen.block_table(gen.rng(seed, 79, k), Bt, pps)[0]).to(dev)
            row = s.groups * P * (s.r_k + s.r_v)
            pages = [gen.device_normal((Bt * pps, row), "bf16", seed * 1000 + 10 * l + k) for l in range(L)]
            enc = [gen.device_normal((s.n_loops, s.groups, s.r_k + s.r_v, s.d_in), "bf16",
                                     seed * 1000 + 500 + 10 * l + k, 1.0 / np.sqrt(s.d_in)) for l in range(L)]
            x = [gen.device_normal((Bt, n, s.n_loops, s.groups, s.d_in), "bf16", seed * 1000 + 700 + 10 * l + k)
                 for l in range(L)]
            self.sets.append(dict(spec=s, desc=desc, enc=enc, x=x, stores=[B.store(pg, bt) for pg in pages]))
        self.wpos = torch.arange(n, dtype=torch.int32, device=dev).repeat(Bt, 1).contiguous()
        self.n_tok = torch.full((Bt,), n, dtype=torch.int32, device=dev)
        ws = max(B.lla_parallel_workspace_bytes(st["desc"], Bt, n) for st in self.sets)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        wws = max(B.lla_write_workspace_bytes(st["desc"], Bt, n, st["spec"].d_in) for st in self.sets)
        self.wws = torch.empty(max(wws, 256), dtype=torch.uint8, device=dev)
        self.out = torch.empty((Bt, n, H, dh), dtype=torch.bfloat16, device=dev)
        self.calls = []
        for t in range(1, T + 1):
            k = w.set_for_loop(t)
            s = w.sets[k]
            for l in range(L):
                sd = seed * 100000 + 1000 * t + 10 * l
                q = gen.device_normal((Bt, n, H, dh), "bf16", sd + 1)
                kk = gen.device_normal((Bt, n, H, dh), "bf16", sd + 2, float(np.sqrt(s.n_loops)))
                vv = gen.device_normal((Bt, n, H, dh), "bf16", sd + 3, float(np.sqrt(s.n_loops)))
                A = gen.device_normal((H, dh, s.r_k), "bf16", sd + 6, 1.0 / np.sqrt(s.r_k))
                Bm = gen.device_normal((H, dh, s.r_v), "bf16", sd + 7, 1.0 / np.sqrt(s.r_v))   # B_t^T
                args = B.parallel_args(loop=t, window=W, n_tok=self.n_tok, q=q, k=kk, v=vv, A=A, B=Bm,
                                       out=self.out, workspace=self.ws)
                self.calls.append((t, k, l, self.sets[k]["desc"], self.sets[k]["stores"][l], args, None))
        self.entry_name = "parallel"
        self.entry = B.hla_attention_parallel
        torch.cuda.synchronize()

    def step(self):
        B = self.B
        for l in range(self.w.layers):
            for st in self.sets:
                B.lla_write_latents(st["desc"], st["stores"][l], pos=self.wpos, x=st["x"][l], enc=st["enc"][l],
                                    workspace=self.wws)
        for (t, k, l, desc, st, args, _) in self.calls:
            self.entry(desc, st, self.w.batch, args)

    def attn_flop(self):
        """Algorithmic FLOPs of one attention kernel launch: causal attention in
        head space, 4 d_h per (position, key) pair, n (n+1) / 2 pairs per
        sequence and head."""
        w = self.w
        return 4 * w.head_dim * w.batch * w.heads * w.context * (w.context + 1) // 2

    def step_bytes(self):
        """(step FLOPs, per-call {set: (attention FLOPs, _, _)}): the step's
        matrix work -- writer GEMMs, key/value rebuild GEMMs, attention."""
        w = self.w
        tok = w.batch * w.context
        total = 0
        per_call = {}
        for k, s in enumerate(w.sets):
            writer = 2 * tok * s.n_loops * s.groups * (s.r_k + s.r_v) * s.d_in
            rebuild = 2 * tok * (s.r_k + s.r_v) * w.heads * w.head_dim
            total += w.layers * writer + w.layers * s.n_loops * (rebuild + self.attn_flop())
            per_call[k] = (self.attn_flop(), None, self.attn_flop())
        return total, per_call


class FullStep:
    """Every buffer of one decode step of the uncompressed model: one exact
    paged K/V cache per (layer, loop), the same attention shape and context as
    the workload.  The decode call appends the current token itself."""

    def __init__(self, w, splits=0, seed=0):
        import torch
        from compressed_cross_loop_amd import binding as B
        from synth import gen
        self.torch, self.B, self.w = torch, B, w
        dev = "cuda"
        dt = gen.TORCH_DTYPE[w.dtype]
        L, T, H, dh, Bt, P = w.layers, w.loops, w.heads, w.head_dim, w.batch, w.page_size
        self.i = w.context - 1
        ppseq = -(-w.context // P)
        self.desc = B.kv_desc(n_heads=H, head_dim=dh, page_size=P, rope_base=w.rope_base,
                              dtype=B.LLA_BF16 if w.dtype == "bf16" else B.LLA_F32)
        n_pages = Bt * ppseq
        need = L * T * 2 * n_pages * P * H * dh * (2 if w.dtype == "bf16" else 4)
        free = torch.cuda.mem_get_info()[0]
        if need > 0.97 * free:
            raise MemoryError(f"the exact per-loop cache of {L} layers x {T} loops at batch {Bt}, context "
                              f"{w.context} needs {need / 2**30:.1f} GiB; {free / 2**30:.1f} GiB of HBM is free")
        bt = torch.from_numpy(gen.block_table(gen.rng(seed, 78), Bt, ppseq)[0]).to(dev)
        self.pos = torch.full((Bt,), self.i, dtype=torch.int32, device=dev)
        self.ws = torch.empty(B.lla_full_decode_workspace_bytes(self.desc, Bt, self.i, splits), dtype=torch.uint8,
                              device=dev)
        self.calls = []
        for t in range(1, T + 1):
            for l in range(L):
                sd = seed * 100000 + 1000 * t + 10 * l
                kp = gen.device_normal((n_pages, P, H, dh), w.dtype, sd + 4)
                vp = gen.device_normal((n_pages, P, H, dh), w.dtype, sd + 5)
                q = gen.device_normal((Bt, H, dh), w.dtype, sd + 1)
                kc = gen.device_normal((Bt, H, dh), w.dtype, sd + 2)
                vc = gen.device_normal((Bt, H, dh), w.dtype, sd + 3)
                out = torch.empty((Bt, H, dh), dtype=dt, device=dev)
                args = B.full_decode_args(pos=self.pos, q=q, k_cur=kc, v_cur=vc, out=out, workspace=self.ws,
                                          max_pos_hint=self.i, splits=splits)
                self.calls.append((t, 0, l, self.desc, B.kv_cache(kp, vp, bt), args, (kp, vp, q, kc, vc, out)))
        self.entry_name = "full"
        self.entry = B.lla_decode_full_cache
        torch.cuda.synchronize()

    def step(self):
        for (t, k, l, desc, cache, args, _) in self.calls:
            self.entry(desc, cache, self.w.batch, args)

    def step_bytes(self):
        """Algorithmic HBM bytes: every call reads the cached K and V of tokens
        0..i-1 and moves q, k_cur, v_cur, out and the appended K/V row."""
        w = self.w
        e = 2 if w.dtype == "bf16" else 4
        kv = w.batch * self.i * w.heads * w.head_dim * 2 * e
        act = w.batch * w.heads * w.head_dim * e * 6
        flop = 2 * 2 * w.batch * self.i * w.heads * w.head_dim
        return len(self.calls) * (kv + act), {0: (kv, kv + act, flop)}


def cpu_baseline_full(w, budget_s, seed=0):
    """The fp64 oracle's full_cache_decode on whole sequences at the same
    shape, on the host cores, scaled to decode tokens/s of the full step."""
    import threadpoolctl
    import oracle as O
    from synth import gen
    H, dh, P = w.heads, w.head_dim, w.page_size
    i = w.context - 1
    g = gen.rng(seed, 992)
    nps = -(-w.context // P)
    kp = g.standard_normal((nps, P, H, dh)).astype(np.float32).astype(np.float64)
    vp = g.standard_normal((nps, P, H, dh)).astype(np.float32).astype(np.float64)
    bt = np.arange(nps)[None]
    q, kc, vc = (g.standard_normal((1, H, dh)) for _ in range(3))
    n, t0 = 0, time.perf_counter()
    while True:
        O.full_cache_decode(kp, vp, bt, [i], q, kc, vc, page_size=P, rope_base=w.rope_base)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    t_call = (time.perf_counter() - t0) / n
    info = threadpoolctl.threadpool_info()
    blas_threads = max([d.get("num_threads", 1) for d in info] or [1])
    return {
        "value": 1.0 / (w.layers * w.loops * t_call), "unit": "tokens/s", "cores": int(blas_threads),
        "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": (f"oracle full_cache_decode (fp64 numpy) on {n} whole sequences ({t_call * 1e3:.1f} ms/seq/call) "
                   f"in {time.perf_counter() - t0:.1f} s, scaled to {w.layers} layers x {w.loops} loops per token"),
    }


def cpu_baseline_parallel(w, budget_s, seed=0):
    """The fp64 oracle's parallel_attention, timed on the host cores on
    evenly spaced positions of one sequence per set (a position's cost grows
    with its index, so their mean is the mean over the sequence), scaled to
    tokens/s of the full step (attention only: B n positions per step over
    L T calls)."""
    import threadpoolctl
    import oracle as O
    from synth import gen
    H, dh, W, n = w.heads, w.head_dim, w.window, w.context
    g = gen.rng(seed, 992)
    t_row = []
    n_rows = 0
    t0 = time.perf_counter()
    for s in w.sets:
        sK = [g.standard_normal((n, s.groups, s.r_k))]
        sV = [g.standard_normal((n, s.groups, s.r_v))]
        q, k, v = (g.standard_normal((1, n, H, dh)) for _ in range(3))
        A = g.standard_normal((H, dh, s.r_k)) / np.sqrt(s.r_k)
        Bv = g.standard_normal((H, s.r_v, dh)) / np.sqrt(s.r_v)
        rows, ts = 0, time.perf_counter()
        for step in range(256):
            i = int((step + 0.5) * n / 256)
            O.parallel_attention(sK, sV, [n], q, k, v, A, Bv, window=W, rope_base=w.rope_base, rows=[(0, i)])
            rows += 1
            if time.perf_counter() - ts >= budget_s / len(w.sets):
                break
        t_row.append((time.perf_counter() - ts) / rows)
        n_rows += rows
    t_call = [w.batch * n * t for t in t_row]                   # one (layer, loop) call
    t_step = sum(w.layers * w.sets[k].n_loops * t_call[k] for k in range(len(w.sets)))
    info = threadpoolctl.threadpool_info()
    return {
        "value": w.batch * n / t_step, "unit": "tokens/s", "cores": int(max([d.get("num_threads", 1) for d in info] or [1])),
        "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": (f"oracle parallel_attention (fp64 numpy) on {n_rows} evenly spaced positions (all heads) of one "
                   f"{n}-position sequence per set in {time.perf_counter() - t0:.1f} s "
                   f"({', '.join(f'{t * 1e3:.1f} ms/position set{k}' for k, t in enumerate(t_row))}), scaled to "
                   f"{w.batch} x {n} positions x {w.layers} layers x {w.loops} loops (attention only)"),
    }


def cpu_baseline(w, budget_s, seed=0, entry="hla", fp8=False):
    """The fp64 oracle timed on the host cores on whole sequences of the same
    workload, scaled to decode tokens/s of the full step: the textbook form
    (rebuild every latent token's key and value, then attend) is the reported
    value, the absorbed form (Eqs. 3-4 as written) a second figure beside it;
    each gets half the time budget.  With fp8 latents the oracle gathers and
    dequantizes the codes (gather_latents_fp8) before the same decodes."""
    first = cpu_baseline_form(w, budget_s / 2, seed, "textbook", fp8)
    second = cpu_baseline_form(w, budget_s / 2, seed, "absorbed", fp8)
    first["absorbed_form"] = {k: second[k] for k in ("value", "unit", "sample")}
    return first


def cpu_baseline_form(w, budget_s, seed, form, fp8):
    """One oracle form (textbook_decode or absorbed_decode), timed as above."""
    import threadpoolctl
    import oracle as O
    from synth import gen
    H, dh, W, P = w.heads, w.head_dim, w.window, w.page_size
    i = w.context - 1
    n_lat = max(0, i - W)
    g = gen.rng(seed, 991)
    per_set = []
    for s in w.sets:
        nps = -(-w.context // P)
        if fp8:
            R = s.r_k + s.r_v
            pages = g.integers(0, 256, size=(nps * s.groups * (P // 16), 16 * R + 128), dtype=np.uint8)
            pages[(pages & 0x7F) == 0x7F] -= 1
            sc = (g.uniform(0.5, 1.5, size=(pages.shape[0], 32)) * np.sqrt(s.n_loops) * 4 / 448).astype(np.float32)
            pages[:, 16 * R:] = sc.view(np.uint8)
        else:
            pages = (g.standard_normal((nps, s.groups * P * (s.r_k + s.r_v))) * np.sqrt(s.n_loops)) \
                .astype(np.float32).astype(np.float64)
        bt = np.arange(nps, dtype=np.int64)[None]
        q = g.standard_normal((1, H, dh))
        kc = g.standard_normal((1, H, dh))
        vc = g.standard_normal((1, H, dh))
        rk = g.standard_normal((1, W + 1, H, dh))
        rv = g.standard_normal((1, W + 1, H, dh))
        A = g.standard_normal((H, dh, s.r_k)) / np.sqrt(s.r_k)
        Bv = g.standard_normal((H, s.r_v, dh)) / np.sqrt(s.r_v)
        per_set.append((s, pages, bt, q, kc, vc, rk, rv, A, Bv))

    def one_sequence(k):
        s, pages, bt, q, kc, vc, rk, rv, A, Bv = per_set[k]
        gather = O.gather_latents_fp8 if fp8 else O.gather_latents
        sK, sV = gather(pages, bt, 0, n_lat, groups=s.groups, page_size=P, r_k=s.r_k, r_v=s.r_v)
        fn = O.textbook_decode if form == "textbook" else O.absorbed_decode
        fn([sK], [sV], [i], q, kc, vc, rk, rv, A, Bv, window=W, rope_base=w.rope_base)

    t_set = []
    n_done = 0
    t_start = time.perf_counter()
    per_share = budget_s / len(w.sets)
    for k in range(len(w.sets)):
        n, t0 = 0, time.perf_counter()
        while True:
            one_sequence(k)
            n += 1
            if time.perf_counter() - t0 >= per_share:
                break
        t_set.append((time.perf_counter() - t0) / n)
        n_done += n
    wall = time.perf_counter() - t_start
    # one step of one sequence: every (layer, loop) call
    t_seq_step = sum(w.layers * w.sets[k].n_loops * t_set[k] for k in range(len(w.sets)))
    info = threadpoolctl.threadpool_info()
    blas_threads = max([d.get("num_threads", 1) for d in info] or [1])
    return {
        "value": 1.0 / t_seq_step, "unit": "tokens/s", "cores": int(blas_threads),
        "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": (f"oracle {'gather_latents_fp8 + ' if fp8 else ''}"
                   f"{form}_decode (fp64 numpy) "
                   f"on {n_done} whole sequences "
                   f"({', '.join(f'{t * 1e3:.1f} ms/seq/call set{k}' for k, t in enumerate(t_set))}) "
                   f"in {wall:.1f} s, scaled to {w.layers} layers x {w.loops} loops per token"),
    }


def calibrate_copy(nbytes):
    """One plain copy of known size, so that profiler HBM byte counters can be
    scaled (a copy reads and writes nbytes each)."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes}))


def stream_copy_gbs(nbytes=1 << 31, reps=10):
    """HBM bandwidth a plain device copy reaches on this GPU (read + write
    bytes per second): the practical streaming ceiling beside the 8 TB/s peak."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del x, y
    torch.cuda.empty_cache()
    return 2 * nbytes / dt / 1e9


def source_sha(name):
    import hashlib
    path = os.path.join(ROOT, "compressed_cross_loop_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(workload_name, kernel):
    """HBM bytes per launch of the scan kernel family from the profiler counters
    kept in profiles/traffic.json, or None when there are none for this
    workload or they were taken on other source."""
    tp = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(tp):
        return None
    rec = json.load(open(tp)).get("kernels", {}).get(kernel)
    if not rec or rec.get("source_sha") != source_sha(rec["source"]):
        return None
    return rec.get("workloads", {}).get(workload_name)


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU per process; --gpus must be 1"}))
        sys.exit(2)
    if a.calibrate_copy:
        calibrate_copy(a.calibrate_copy)
        return
    import torch
    from synth import configs
    w = configs.get(a.workload)
    hip = Hip()
    if a.layers:
        w = w.with_(layers=a.layers)
    if a.entry == "parallel":
        if w.family != "hla" or w.dtype != "bf16":
            print(json.dumps({"error": "the parallel pass runs on the HLA bf16 workloads"}))
            sys.exit(2)
        w = w.with_(batch=a.batch or 8, context=a.context or 2048)
        w = w.with_(name=f"hla-parallel-ouro1.4b-b{w.batch}-n{w.context}")
        st = ParallelStep(w)
    else:
        if a.batch:
            w = w.with_(batch=a.batch, name=f"{w.name}@b{a.batch}")
        if a.context:
            w = w.with_(context=a.context, name=f"{w.name}@ctx{a.context}")
        if a.entry == "full":
            w = w.with_(name=f"full-cache-L{w.layers}xT{w.loops}-h{w.heads}x{w.head_dim}-b{w.batch}-ctx{w.context}")
            try:
                st = FullStep(w, splits=a.splits)
            except MemoryError as err:
                print(json.dumps({"error": str(err), "config": {"workload": w.name}}))
                sys.exit(3)
        else:
            if a.latent_fp8:
                if a.entry == "reconstruct" or (a.entry == "auto" and w.family != "hla") or w.dtype != "bf16":
                    print(json.dumps({"error": "fp8 latents serve the absorbed / HLA reads of bf16 workloads"}))
                    sys.exit(2)
                w = w.with_(name=f"{w.name}-fp8")
            if a.fused:
                w = w.with_(name=f"{w.name}-fused")
            hla_entry = a.entry == "hla" or (a.entry == "auto" and w.family == "hla")
            overlap = a.writes == "overlapped" or (a.writes == "auto" and hla_entry)
            st = DecodeStep(w, splits=a.splits, entry=a.entry, fp8=a.latent_fp8,
                            flags=2 if a.fused else 0, overlap_writes=overlap)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(max(1, a.warmup)):
        st.step()
    torch.cuda.synchronize()
    run_step = st.step
    if not a.no_graph:
        # the whole step (every decode call and latent write) as one HIP graph:
        # the library allocates, clears and synchronises nothing, so its
        # launches capture as they are
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            st.step()
        torch.cuda.synchronize()
        run_step = graph.replay
        for _ in range(max(1, a.warmup)):
            run_step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(a.steps):
        run_step()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(e0, e1) / a.steps
    step_bytes, per_call = st.step_bytes()

    # dominant kernel: the scan of the set serving the most loops, timed live
    main_k = 0 if st.entry_name == "full" else max(per_call, key=lambda k: per_call[k][0] * w.sets[k].n_loops)
    evs = []
    rsteps = max(2, min(a.steps, 5))
    for _ in range(rsteps):
        for (t, k, l, desc, stc, args, _) in st.calls:
            ev_field = "attn_events" if st.entry_name == "parallel" else "scan_events"
            if k == main_k:
                pair = (ctypes.c_void_p * 2)(hip.event().value, hip.event().value)
                setattr(args, ev_field, ctypes.addressof(pair))
                evs.append(pair)
            st.entry(desc, stc, w.batch, args)
            setattr(args, ev_field, None)
    torch.cuda.synchronize()
    scan_ms = float(np.mean([hip.elapsed_ms(ctypes.c_void_p(p[0]), ctypes.c_void_p(p[1])) for p in evs]))
    scan_bytes, _, scan_flop = per_call[main_k]
    if st.entry_name == "full":
        kname, loops_served = "k_full_scan", (1, w.loops)
    elif st.entry_name == "parallel":
        s_main = w.sets[main_k]
        kname, loops_served = "k_par_attn", (s_main.loop_first, s_main.loop_last)
    else:
        s_main = w.sets[main_k]
        loops_served = (s_main.loop_first, s_main.loop_last)
        scan_bytes += w.batch * w.heads * s_main.r_k * (2 if w.dtype == "bf16" else 4) \
            if st.entry_name != "reconstruct" else 0
        main_desc = next(c[3] for c in st.calls if c[1] == main_k)
        kname = st.B.lla_decode_scan_kernel(main_desc, ENTRY_CODE[st.entry_name], getattr(st, "flags", 0))
    reconstruct_mfma_bound = st.entry_name == "reconstruct" and scan_flop / scan_bytes > 312
    if reconstruct_mfma_bound or st.entry_name == "parallel":
        roof = {"bound": "mfma", "achieved": scan_flop / (scan_ms * 1e-3) / 1e12, "peak": 2500.0,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": scan_bytes / (scan_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name, kname) if st.entry_name != "parallel" else None
    roof.update({"kernel": f"{kname} (" + ("every (layer, loop) call" if st.entry_name == "full" else
                                         f"set serving loops {loops_served[0]}..{loops_served[1]}") + ")",
                 "avg_launch_ms": scan_ms, "bytes_per_launch": scan_bytes, "flop_per_launch": scan_flop})

    parallel = st.entry_name == "parallel"
    gbs = step_bytes / (ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC_PARALLEL if parallel else METRIC,
        "value": w.batch * (w.context if parallel else 1) / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "entry": st.entry_name, "inputs": w.inputs, "layers": w.layers,
                   "loops": w.loops,
                   "batch": w.batch, "context": w.context, "window": w.window, "heads": w.heads,
                   "head_dim": w.head_dim,
                   "sets": ("exact K/V per loop" if st.entry_name == "full" else
                            [dict(loops=[s.loop_first, s.loop_last], groups=s.groups, r_k=s.r_k, r_v=s.r_v)
                             for s in w.sets]),
                   "splits": a.splits or "auto", "launch": "eager" if a.no_graph else "hip_graph",
                   "writes": ("overlapped" if getattr(st, "overlap_writes", False) else "serial"),
                   "latents": "e4m3+scale" if getattr(st, "fp8", False) else w.dtype},
        "stream_copy_gbs": stream_copy_gbs(),
        "roofline": roof,
    }
    if parallel:
        # step_bytes holds the step's matrix FLOPs here (writer, rebuild, attention)
        rec.update({"step_flop": step_bytes, "step_tflops": step_bytes / (ms * 1e-3) / 1e12})
    else:
        rec.update({"step_bytes": step_bytes, "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS})
    if not a.no_cpu_baseline:
        if st.entry_name == "full":
            rec["cpu_baseline"] = cpu_baseline_full(w, a.cpu_seconds)
        elif parallel:
            rec["cpu_baseline"] = cpu_baseline_parallel(w, a.cpu_seconds)
        else:
            rec["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds, entry=st.entry_name, fp8=getattr(st, "fp8", False))
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
