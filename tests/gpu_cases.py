"""Shared machinery of the GPU parity tests: seeded inputs for both sides, a call through
the C ABI, and the oracle's answer for any request.  The HIP side gets its tree metadata
from the library's own builder; the oracle side from ``oracle.meta``; the two agree
bit-exactly (checked separately)."""
import numpy as np

import tree_attention_draft_amd as tv
from oracle import attn as oattn
from oracle import meta as ometa
from oracle import rope as orope
from tree_attention_draft_amd import workloads

TOL = {"bf16": 2e-2, "f32": 1e-5}


def say(*a):
    print("[case]", *a, flush=True)


class Case:
    """One batch: prefix lengths, per-request trees (rank paths or explicit parent arrays),
    head shape, dtype, layout."""

    def __init__(self, name, prefix_lens, trees=None, parents=None, Hq=32, Hkv=8, D=128,
                 dtype="bf16", seed=1000, k_scale=False, page_size=0, page_seed=3000):
        self.name = name
        self.L = np.asarray(prefix_lens, np.int32)
        self.B = len(self.L)
        self.Hq, self.Hkv, self.D, self.dtype = Hq, Hkv, D, dtype
        if parents is not None:
            self.parent_gpu = [list(p) for p in parents]
            self.parent_oracle = [list(p) for p in parents]
        else:
            per_request = bool(trees) and isinstance(trees[0], list)
            if not per_request:
                trees = [list(trees or [])] * self.B
            self.parent_gpu = [tv.tree_meta_build(t, 0)["parent"].tolist() for t in trees]
            self.parent_oracle = [ometa.build_from_paths(t, 0)["parent"] for t in trees]
        self.N = len(self.parent_gpu[0])
        assert all(len(p) == self.N for p in self.parent_gpu)
        self.page_size = page_size
        self.sm_scale = None  # the oracle's default (1/sqrt(D)) unless a run sets one
        self.rope_theta = 0.0  # fused rotary embedding of the last run (0: none)
        say(name, f"B={self.B} N={self.N} Hq={Hq} Hkv={Hkv} D={D} {dtype} "
            f"L=[{self.L.min() if self.B else 0},{self.L.max() if self.B else 0}] "
            f"paged={page_size} seed={seed}")
        self.host = workloads.build_batch(seed, self.L, self.N, Hq, Hkv, D, dtype,
                                          k_scale=k_scale, page_size=page_size,
                                          page_seed=page_seed)
        self._dev = None

    # ------------------------------------------------------------------ device ------
    def device(self):
        import torch
        if self._dev is None:
            def up(a):
                if a.dtype == np.uint16:
                    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
                return torch.from_numpy(a).cuda()
            d = {"q": up(self.host["q"]), "k": up(self.host["k"]), "v": up(self.host["v"]),
                 "prefix_len": torch.from_numpy(self.L).cuda(),
                 "parent": torch.tensor(np.array(self.parent_gpu, np.int32)).cuda()}
            if self.page_size:
                d["page_table"] = torch.from_numpy(self.host["page_table"]).cuda()
            self._dev = d
        return self._dev

    def run(self, **kw):
        """Call tree_verify_attn; returns (out, lse) as float64 numpy arrays."""
        import torch
        d = self.device()
        kw.setdefault("max_prefix_len", int(self.L.max()) if self.B else 0)
        if self.page_size:
            kw.setdefault("page_table", d["page_table"])
            kw.setdefault("page_size", self.page_size)
        parent = kw.pop("parent", d["parent"])
        if kw.get("sm_scale"):
            self.sm_scale = float(kw["sm_scale"])
        self.rope_theta = float(kw.get("rope_theta", 0.0))
        say(self.name, "tree_verify_attn", {k: v for k, v in kw.items()
                                            if k in ("num_splits", "path", "max_prefix_len",
                                                     "rope_theta")})
        out, lse = tv.tree_verify_attn(d["q"], d["k"], d["v"], parent, d["prefix_len"], **kw)
        torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)

    # ------------------------------------------------------------------ oracle ------
    def _decode(self, a):
        if self.dtype == "bf16":
            return oattn.bf16_bits_to_f64(a)
        return np.asarray(a, np.float64)

    def request_inputs(self, b):
        L = int(self.L[b])
        T = L + self.N
        q = self._decode(self.host["q"][b])
        if self.page_size:
            kb = oattn.gather_paged(self.host["k"], self.host["page_table"][b], self.page_size, T)
            vb = oattn.gather_paged(self.host["v"], self.host["page_table"][b], self.page_size, T)
        else:
            kb = self.host["k"][b, :T]
            vb = self.host["v"][b, :T]
        return q, self._decode(kb), self._decode(vb)

    def oracle(self, b):
        q, k, v = self.request_inputs(b)
        if self.rope_theta > 0:
            return orope.tree_attention_request_rope(q, k, v, self.parent_oracle[b],
                                                     int(self.L[b]), self.rope_theta,
                                                     sm_scale=self.sm_scale)
        return oattn.tree_attention_request(q, k, v, self.parent_oracle[b], int(self.L[b]),
                                            sm_scale=self.sm_scale)

    def check(self, out, lse, requests=None, tol=None):
        """Max-abs error of the given outputs vs the oracle over ``requests`` (all by
        default); asserts it is within the dtype's tolerance and returns it."""
        tol = TOL[self.dtype] if tol is None else tol
        reqs = range(self.B) if requests is None else requests
        worst = 0.0
        for b in reqs:
            o_ref, l_ref = self.oracle(b)
            assert np.isfinite(out[b]).all() and np.isfinite(lse[b]).all(), (self.name, b)
            eo = float(np.abs(out[b] - o_ref).max())
            el = float(np.abs(lse[b] - l_ref).max())
            worst = max(worst, eo, el)
            assert eo <= tol and el <= tol, (self.name, b, eo, el)
        say(self.name, f"max_abs_err={worst:.3e} over requests {list(reqs)[:8]}")
        return worst


class StreamedPagedCase(Case):
    """A paged batch too large to hold on the host (long context at large batch): every
    request's K and V are drawn with ``workloads.request_tensors`` (the same per-request
    streams ``workloads.build_batch`` uses, so values match a host-built batch of the same
    seeds) and copied into a NaN-filled device pool page by page, one request at a time.
    The oracle regenerates a sampled request's tensors on the host from the same seed."""

    def __init__(self, name, prefix_lens, trees, Hq=32, Hkv=8, D=128, seed=1000,
                 page_size=16, page_seed=3000):
        import concurrent.futures
        import os
        import torch
        self.name = name
        self.L = np.asarray(prefix_lens, np.int32)
        self.B = len(self.L)
        self.Hq, self.Hkv, self.D, self.dtype = Hq, Hkv, D, "bf16"
        self.parent_gpu = [tv.tree_meta_build(t, 0)["parent"].tolist() for t in trees]
        self.parent_oracle = [ometa.build_from_paths(t, 0)["parent"] for t in trees]
        self.N = len(self.parent_gpu[0])
        self.page_size = page_size
        self.sm_scale = None
        self.rope_theta = 0.0
        self.seed = seed
        S = int(self.L.max()) + self.N
        prng = np.random.Generator(np.random.PCG64(page_seed))
        table, n_pages = workloads.page_table(prng, self.B, S, page_size)
        say(name, f"B={self.B} N={self.N} streamed paged pool {n_pages} pages "
            f"({2 * n_pages * page_size * Hkv * D * 2 / 1e9:.1f} GB K+V) seed={seed}")
        nan = torch.tensor(workloads.BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16)
        kpool = torch.full((n_pages, page_size, Hkv, D), float(nan.float()),
                           dtype=torch.bfloat16, device="cuda")
        vpool = torch.full_like(kpool, float(nan.float()))
        q = np.empty((self.B, self.N, Hq, D), np.uint16)

        def draw(b):
            Lb = int(self.L[b])
            qb, kb, vb = workloads.request_tensors(seed, b, self.N, Lb, Hq, Hkv, D)
            T = Lb + self.N
            npg = -(-T // page_size)
            blocks = []
            for x in (kb, vb):
                pad = np.full((npg * page_size, Hkv, D), workloads.BF16_NAN_BITS, np.uint16)
                pad[:T] = workloads.encode(x, "bf16")
                blocks.append(pad.reshape(npg, page_size, Hkv, D))
            return b, workloads.encode(qb, "bf16"), blocks, npg

        def upload(result):
            b, qb, (kblk, vblk), npg = result
            q[b] = qb
            idx = torch.from_numpy(table[b, :npg].astype(np.int64)).cuda()
            for pool, blk in ((kpool, kblk), (vpool, vblk)):
                src = torch.from_numpy(blk.view(np.int16)).view(torch.bfloat16).cuda()
                pool.index_copy_(0, idx, src)
            if b % 16 == 15:
                say(name, f"uploaded {b + 1}/{self.B} requests")

        # at most 2 x workers requests are held on the host at any time
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            pending = []
            for b in range(self.B):
                pending.append(ex.submit(draw, b))
                if len(pending) >= 2 * workers:
                    upload(pending.pop(0).result())
            for f in pending:
                upload(f.result())
        torch.cuda.synchronize()
        self.host = {"q": q, "page_table": table}
        self._dev = {"q": torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda(),
                     "k": kpool, "v": vpool,
                     "prefix_len": torch.from_numpy(self.L).cuda(),
                     "parent": torch.tensor(np.array(self.parent_gpu, np.int32)).cuda(),
                     "page_table": torch.from_numpy(table).cuda()}

    def request_inputs(self, b):
        Lb = int(self.L[b])
        qb, kb, vb = workloads.request_tensors(self.seed, b, self.N, Lb, self.Hq, self.Hkv,
                                               self.D)
        dec = oattn.bf16_bits_to_f64
        return (dec(workloads.encode(qb, "bf16")), dec(workloads.encode(kb, "bf16")),
                dec(workloads.encode(vb, "bf16")))

    def release(self):
        self._dev = None
        import torch
        torch.cuda.empty_cache()
