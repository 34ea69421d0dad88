"""Shared helpers of the GPU parity tests.

A layer on the GPU is checked against the oracle in two halves that meet at h, the one
intermediate with several correct values (an fp32 evaluation may put an h value on the
other side of an e4m3 rounding boundary than the exact value):

1. routing tables bit-exact, gates within the fp32 bound, x codes and scales bit-exact,
   the GPU's weight codes and scales equal to the oracle quantiser's;
2. every GPU h code and scale of the checked rows inside the analytic window of
   ``windows.py`` (derived from the oracle's exact GEMM1 and its sum of |x w|, never
   from the device);
3. the oracle's GEMM2 + b2 evaluated in float64 on the GPU's own h codes and scales
   ("oracle(GPU h)"): the GPU's y within the fp32-accumulation + fp16-storage bound, and
   the GPU's out within the literal tolerance max(2e-2 RMS(oracle out), one bf16 ulp)
   of sum_j g_j y_j, and within the analytic combine bound;
4. the GPU's out against the plain oracle (its own h): relative Frobenius <= 5e-3.
"""
from __future__ import annotations

import sys
from collections import OrderedDict
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import sparse_moe_ffn_gemm_amd as moe
from oracle import moe_ref as R
from synth import LayerShape, expert_weights, make_inputs
import windows as W
from layouts import untile_fp4, untile_scales

REL_FRO_TOL = 5e-3
MAX_ELT_TOL = 2e-2
GATE_TOL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


class GpuLayer:
    """Device tensors of one layer; expert weights quantised by the library (``fmt``
    "block": 128x128 block scales, "mxfp8": MXFP8, "mxfp4": MXFP4 weights)."""

    def __init__(self, shape: LayerShape, inputs=None, device="cuda", fmt="block"):
        self.shape = shape
        self.fmt = fmt
        self.li = inputs if inputs is not None else make_inputs(shape)
        li = self.li
        self.x = bf16_dev(li.x, device)
        b13 = bf16_dev(li.b13, device) if shape.expert_bias else None
        b2 = bf16_dev(li.b2, device) if shape.expert_bias else None
        self.layer = moe.MoELayer.from_expert_weights(
            torch.from_numpy(li.router_w), torch.from_numpy(li.router_b), shape.top_k, b13, b2,
            lambda e: expert_weights(shape, "w13", e, device),
            lambda e: expert_weights(shape, "w2", e, device), device=device, fmt=fmt)
        torch.cuda.synchronize()

    def run(self, fused=False):
        """The layer on the GPU (``fused``: moe_forward_fused, whose bounded waits must all
        have completed) -> (out, routing tables)."""
        s = self.shape
        routing = moe.new_routing(s.T, s.E, s.top_k)
        say(f"forward{' fused' if fused else ''} [{self.fmt}] {s.name}: T={s.T} H={s.H} E={s.E} "
            f"k={s.top_k} I={s.I}")
        out = self.layer(self.x, routing=routing, fused=fused)
        torch.cuda.synchronize()
        if fused:
            assert moe.fused_status(self.layer.workspace(s.T), s.T, s.H, s.E, s.top_k, s.I) == 0
        return out, routing

    def ws_view(self, region: str, dtype, shape) -> torch.Tensor:
        s = self.shape
        r = moe.workspace_layout(s.T, s.H, s.E, s.top_k, s.I)
        off = getattr(r, region)
        nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        return self.layer.workspace(s.T)[off:off + nbytes].view(dtype).view(*shape)


# The host work of a check (dequantised weights, products, windows) is per expert and
# independent: it runs on CHECK_THREADS threads with single-threaded BLAS (numpy releases
# the GIL), and nothing of it reads the device.
CHECK_THREADS = 16


def par_map(fn, items):
    """[fn(i) for i in items] on the check threads, in order."""
    items = list(items)
    if len(items) <= 1:
        return [fn(i) for i in items]
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=CHECK_THREADS) as ex:
        return list(ex.map(fn, items))


def quantize_by_rows(quant, w: np.ndarray, rows: int = 128):
    """The oracle's weight quantiser applied to 128-row slices of w (every format's scale
    blocks lie within one slice, so the result is the whole-matrix one; the slices keep the
    oracle's per-element temporaries in cache)."""
    parts = [quant(w[i:i + rows]) for i in range(0, w.shape[0], rows)]
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _base(shape):
    from synth.cases import _base_shape
    return _base_shape(shape)


class OracleExperts:
    """Lazily quantised experts for the oracle (from the generator's fp32 weights, by the
    oracle's own quantiser), in the block-scaled, the MXFP8 or the MXFP4-weight format.
    ``OracleExperts.of`` shares them between the checks of layers drawn from the same
    weights (a decode layer and the prefill layer whose draw it reuses, the multi-kernel
    and the one-kernel forward)."""

    _shared: "OrderedDict" = OrderedDict()
    KEEP = 4   # weight draws x formats kept

    @classmethod
    def of(cls, shape: LayerShape, li, fmt="block"):
        key = (_base(shape), fmt)
        ox = cls._shared.pop(key, None)
        if ox is None:
            ox = cls(shape, li, fmt)
        cls._shared[key] = ox
        while len(cls._shared) > cls.KEEP:
            cls._shared.popitem(last=False)
        return ox

    def __init__(self, shape: LayerShape, li, fmt="block"):
        self.shape, self.li = shape, li
        self.fmt = fmt
        self.cache = {}
        self.dev = "cuda" if _base(shape).weights_on_device else "cpu"

    def prepare(self, experts, threads=16):
        todo = [int(e) for e in experts if int(e) not in self.cache]
        quant = {"block": R.quantize_blocks, "mxfp8": R.quantize_mx,
                 "mxfp4": R.quantize_mxfp4}[self.fmt]

        def q(item):
            e, (w13, w2) = item
            c13, s13 = quantize_by_rows(quant, w13)
            c2, s2 = quantize_by_rows(quant, w2)
            return e, (c13, s13, c2, s2)

        # draw on the device serially (a few experts at a time), quantise on the host in parallel
        for i in range(0, len(todo), 32):
            host = {e: (expert_weights(self.shape, "w13", e, self.dev).cpu().numpy(),
                        expert_weights(self.shape, "w2", e, self.dev).cpu().numpy())
                    for e in todo[i:i + 32]}
            with ThreadPoolExecutor(max_workers=threads) as ex:
                for e, v in ex.map(q, host.items()):
                    self.cache[e] = v
            say(f"  oracle quantised {min(i + 32, len(todo))}/{len(todo)} experts ({self.fmt})")

    def view(self, idx):
        cache = self.cache

        class _V:
            def __getitem__(self, e):
                return cache[int(e)][idx]
        return _V()

    def dequant_w(self, codes, scales):
        deq = {"block": R.dequantize_blocks, "mxfp8": R.dequantize_mx,
               "mxfp4": R.dequantize_mxfp4}[self.fmt]
        return deq(codes, scales)


def bf16_ulp(ref: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(int) - 7)


def gate_tolerance(ref_logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Per-token gate tolerance: 1e-6 plus the fp32 floor of the selected logits.

    The device evaluates logits in fp32 (two-level sum over H) and the softmax in fp32, so
    each selected logit carries a few fp32 ulps of its own magnitude; the softmax over the
    selected logits moves a gate by at most half the largest logit error.  Allowing 8 ulps
    per logit: tol_t = 1e-6 + 0.5 * 8 * ulp32(max_j |l_tj|)."""
    sel = np.take_along_axis(ref_logits, ids.astype(np.int64), axis=1)
    mx = np.abs(sel).max(axis=1)
    ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(mx, 2.0 ** -126))).astype(int) - 23)
    return GATE_TOL + 4.0 * ulp


def routing_exact(gpu: dict, ref: dict, what=""):
    ids = gpu["topk_ids"].cpu().numpy()
    assert np.array_equal(ids, ref["ids"]), f"{what}: ids differ at {np.argwhere(ids != ref['ids'])[:5]}"
    assert np.array_equal(gpu["expert_counts"].cpu().numpy(), ref["counts"]), what
    assert np.array_equal(gpu["expert_offsets"].cpu().numpy(), ref["offsets"]), what
    assert np.array_equal(gpu["perm"].cpu().numpy(), ref["perm"]), what
    assert np.array_equal(gpu["inv_perm"].cpu().numpy(), ref["inv"]), what
    g = gpu["topk_gates"].cpu().numpy().astype(np.float64)
    err = np.abs(g - ref["gates"]).max(axis=1)
    tol = gate_tolerance(ref["logits"], ref["ids"])
    say(f"  routing {what}: exact; max |gate err| = {err.max():.2e} (tolerance {tol.min():.1e}.."
        f"{tol.max():.1e})")
    assert np.all(err <= tol), np.argwhere(err > tol)[:5]


_E4M3_POS = np.sort(R.e4m3_decode(np.arange(0x7F)))


def _codes_between(lo, hi):
    """Number of e4m3 values in [lo, hi] (decoded bounds), zero counted once."""
    n_hi = np.searchsorted(_E4M3_POS, np.abs(hi), side="right")
    n_lo = np.searchsorted(_E4M3_POS, np.abs(lo), side="right")
    same = np.sign(lo) * np.sign(hi) >= 0
    return np.where(same, np.abs(n_hi - n_lo) + 1, n_hi + n_lo - 1)


class LayerCheck:
    """The checks of the module docstring for one forward of ``g`` (``out``, ``routing``)."""

    def __init__(self, g: GpuLayer, out: torch.Tensor, routing: dict):
        self.g, self.shape, self.fmt = g, g.shape, g.fmt
        s, li = self.shape, g.li
        self.T, self.H, self.E, self.k, self.I = s.T, s.H, s.E, s.top_k, s.I
        self.rows = s.T * s.top_k
        self.ox = OracleExperts.of(s, li, g.fmt)
        self.y_cache = {}
        self.q_act, self.dq_act, _ = R._quantizer(g.fmt)
        self.out_bits = bits_host(out)
        # routing (all tokens)
        self.logits = R.router_logits(li.x, li.router_w, li.router_b)
        self.ids, self.gates = R.topk_softmax(self.logits, s.top_k)
        self.counts, self.offsets, self.perm, self.inv = R.permute(self.ids, s.E)
        routing_exact(routing, dict(ids=self.ids, gates=self.gates, counts=self.counts,
                                    offsets=self.offsets, perm=self.perm, inv=self.inv,
                                    logits=self.logits), s.name)
        self.gates_dev = routing["topk_gates"].cpu().numpy()
        # x codes and scales, bit-exact (all tokens)
        x32 = R.bf16_to_f64(li.x).astype(np.float32)
        xq, sx = self.q_act(x32)
        gxq = g.ws_view("xq", torch.uint8, (s.T, s.H)).cpu().numpy()
        assert np.array_equal(gxq, xq), "x codes"
        if g.fmt == "block":
            gsx = g.ws_view("sx", torch.float32, (s.T, -(-s.H // 128))).cpu().numpy()
            assert np.array_equal(gsx.view(np.uint32), sx.view(np.uint32)), "x scales"
        else:
            gsx = g.ws_view("sx", torch.uint8, (s.T, moe.mx_row(s.H))).cpu().numpy()
            assert np.array_equal(gsx[:, :s.H // 32], sx) and np.all(gsx[:, s.H // 32:] == 127), "x scales"
        self.xd = self.dq_act(xq, sx)
        self.tok = self.perm // s.top_k
        self.weights_checked = set()
        self.rms = None

    # ---- device data ----
    def _rows(self, region, dtype, width, p):
        v = self.g.ws_view(region, dtype, (self.rows, width))
        return v[torch.as_tensor(np.asarray(p, np.int64), device=v.device)].cpu().numpy()

    def gpu_h(self, p):
        """(codes [n, I], scales: fp32 [n, ceil(I/128)] or E8M0 [n, I/32]) of dispatch rows p."""
        I = self.I
        hq = self._rows("h", torch.uint8, I, p)
        if self.fmt == "block":
            return hq, self._rows("sh", torch.float32, -(-I // 128), p)
        hs = self._rows("sh", torch.uint8, moe.mx_row(I), p)
        assert np.all(hs[:, I // 32:] == 127), "h scale pads"
        return hq, hs[:, :I // 32]

    def gpu_y(self, p):
        return self._rows("y", torch.float16, self.H, p).astype(np.float64)

    def h_dequant(self, hq, hs):
        if self.fmt == "block":
            return R.dequantize_blocks(hq, hs, rows=1)
        return R.dequantize_mx(hq, hs)

    def check_weights(self, e):
        """The GPU's codes and scales of expert e equal the oracle quantiser's."""
        if e in self.weights_checked:
            return
        L, (c13, s13, c2, s2) = self.g.layer, self.ox.cache[e]
        H, I = self.H, self.I
        if self.fmt == "block":
            got = (L.w13[e].cpu().numpy(), L.w13_scales[e].cpu().numpy(), L.w2[e].cpu().numpy(),
                   L.w2_scales[e].cpu().numpy())
            for a, b in zip(got, (c13, s13, c2, s2)):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"expert {e} weights"
        else:
            def sc(t, N, K):
                rows = untile_scales(t[e:e + 1].cpu().numpy(), N, K)[0]
                assert np.all(rows[:, K // 32:] == 127)
                return rows[:, :K // 32]
            if self.fmt == "mxfp4":
                w13 = untile_fp4(L.w13[e:e + 1].cpu().numpy(), 2 * I, H)[0][0]
                w2 = untile_fp4(L.w2[e:e + 1].cpu().numpy(), H, I)[0][0]
            else:
                w13, w2 = L.w13[e].cpu().numpy(), L.w2[e].cpu().numpy()
            assert np.array_equal(w13, c13) and np.array_equal(w2, c2), f"expert {e} codes"
            assert np.array_equal(sc(L.w13_scales, 2 * I, H), s13), f"expert {e} w13 scales"
            assert np.array_equal(sc(L.w2_scales, H, I), s2), f"expert {e} w2 scales"
        self.weights_checked.add(e)

    # ---- the two halves ----
    # Each check reads what it needs from the device first (serially), then does its host
    # arithmetic per expert on the check threads; the per-expert reports are printed and the
    # assertions made afterwards, in expert order.
    def _h_host(self, e, hq, hs):
        """(ok, report) of GPU h codes hq and scales hs of expert e's rows against the window
        (host arithmetic only; ``self.rows_of[e]`` names the rows)."""
        p, what = self.rows_of[e]
        c13, s13, _, _ = self.ox.cache[e]
        W13 = self.ox.dequant_w(c13, s13)
        C, C_abs, C_gmax = W.product_sums(self.xd[self.tok[p]], W13)
        C += R.bf16_to_f64(self.g.li.b13[e])
        del W13
        h, dh = W.swiglu_window(C, C_abs, self.H, self.I, C_gmax)
        del C, C_abs, C_gmax
        if self.fmt == "block":
            sok, cok, diag = W.block_h_check(h, dh, hq, hs)
        else:
            sok, cok, diag = W.mx_h_check(h, dh, hq, hs)
        oq, osc = self.q_act(h.astype(np.float32))
        nd = int((hq != oq).sum())
        width = np.mean(_codes_between(diag["lo"], diag["hi"]))
        rep = [f"  h {what}expert {e} ({len(p)} rows): scales outside the window {int((~sok).sum())} "
               f"of {sok.size}, codes outside {int((~cok).sum())} of {cok.size}; codes unlike the "
               f"oracle's own {nd} ({nd / max(hq.size, 1):.1e}); admissible codes per element "
               f"{width:.2f} on average"]
        ok = bool(sok.all() and cok.all())
        if not ok:
            for rr, cc in np.argwhere(~cok)[:5]:
                rep.append(f"    row {rr} col {cc}: gpu code {hq[rr, cc]:#04x} oracle {oq[rr, cc]:#04x} "
                           f"h={h[rr, cc]:.6g} dh={dh[rr, cc]:.3g}")
        return ok, rep

    def _y_host(self, e, hq, hs):
        """oracle(GPU h): (y_ref, bound) for expert e's rows with GPU h codes hq, scales hs."""
        _, _, c2, s2 = self.ox.cache[e]
        W2 = self.ox.dequant_w(c2, s2)
        y, y_abs, y_gmax = W.product_sums(self.h_dequant(hq, hs), W2)
        y += R.bf16_to_f64(self.g.li.b2[e])
        dy = W.y_bound(y, y_abs, self.I, y_gmax)
        return y, dy

    def _prepare(self, rows_of):
        """Quantised experts, their weights checked, and the GPU h of their rows."""
        self.rows_of = rows_of
        experts = list(rows_of)
        self.ox.prepare(experts)
        for e in experts:
            self.check_weights(e)
        return {e: self.gpu_h(rows_of[e][0]) for e in experts}

    def check_experts(self, experts=None):
        """h window and y bound on every dispatch row of the experts (all active ones by default)."""
        experts = [e for e in (range(self.E) if experts is None else experts) if self.counts[e] > 0]
        rows_of = {int(e): (np.arange(self.offsets[e], self.offsets[e + 1]), "") for e in experts}
        gh = self._prepare(rows_of)
        gy = {e: self.gpu_y(rows_of[e][0]) for e in rows_of}

        def work(e):
            ok, rep = self._h_host(e, *gh[e])
            y, dy = self._y_host(e, *gh[e])
            assert np.abs(y).max() < W.F16_MAX
            ratio = np.abs(gy[e] - y) / dy
            bad = int((ratio > 1).sum())
            rep.append(f"  y expert {e} ({len(rows_of[e][0])} rows): max |err| / bound {ratio.max():.3f}, "
                       f"outside {bad} of {ratio.size}")
            return ok and bad == 0, rep, (y, dy)

        res = par_map(work, list(rows_of))
        for e, (ok, rep, yd) in zip(rows_of, res):
            for line in rep:
                say(line)
            self.y_cache[(e, np.asarray(rows_of[e][0], np.int64).tobytes())] = yd
        for e, (ok, rep, _) in zip(rows_of, res):
            assert ok, f"expert {e}"

    def plain_oracle_out(self, toks):
        """The plain oracle's out of the tokens: its forward's per-token steps (routing over
        all tokens, x quantisation of the tokens, each expert's FFN on its rows, the
        gate-weighted sum), with the experts' FFNs (``oracle.expert_ffn``) on the check
        threads.  Equal to ``oracle.forward(..., token_subset=toks)["out"]`` bit for bit
        (``tests/test_oracle_layer.py`` pins that on the CPU)."""
        return oracle_forward_out(self.g.li, self.k, self.I, self.ox, toks, self.fmt)

    def check_tokens(self, toks=None, h_window=True):
        """out of the tokens: oracle(GPU h) at the literal bound and the combine bound; the
        plain oracle at rel. Frobenius <= 5e-3.  With h_window the tokens' h rows are
        checked against the window too."""
        T, k, H = self.T, self.k, self.H
        toks = np.arange(T) if toks is None else np.asarray(toks)
        flat = (toks[:, None] * k + np.arange(k)[None, :]).reshape(-1)
        p_all = self.inv[flat]
        e_all = self.ids[toks].reshape(-1)
        what = "of the sampled tokens, " if toks.size < T else ""
        sel_of = {int(e): np.nonzero(e_all == e)[0] for e in np.unique(e_all)}
        gh = self._prepare({e: (p_all[sel], what) for e, sel in sel_of.items()})

        def work(e):
            p = self.rows_of[e][0]
            ok, rep = self._h_host(e, *gh[e]) if h_window else (True, [])
            yd = self.y_cache.get((e, np.asarray(p, np.int64).tobytes()))
            if yd is None:
                yd = self._y_host(e, *gh[e])
            assert np.abs(yd[0]).max() < W.F16_MAX
            return ok, rep, yd

        res = par_map(work, list(sel_of))
        yr = np.zeros((toks.size * k, H))
        dy = np.zeros((toks.size * k, H))
        for e, (ok, rep, (y, d)) in zip(sel_of, res):
            for line in rep:
                say(line)
            yr[sel_of[e]], dy[sel_of[e]] = y, d
        for e, (ok, _, _) in zip(sel_of, res):
            assert ok, f"expert {e}"
        yr = yr.reshape(toks.size, k, H)
        dy = dy.reshape(toks.size, k, H)
        out2 = np.einsum("tk,tkh->th", self.gates[toks], yr)
        got = R.bf16_to_f64(self.out_bits[toks])
        # the plain oracle (its own h) on the same tokens
        ref_out = self.plain_oracle_out(toks)
        rms = np.sqrt(np.mean(ref_out ** 2))
        d2 = np.abs(got - out2)
        lit = np.maximum(MAX_ELT_TOL * rms, bf16_ulp(out2))
        cb = W.combine_bound(self.gates[toks], self.gates_dev[toks], yr, dy, out2)
        rel2 = np.linalg.norm(got - out2) / np.linalg.norm(out2)
        rel = np.linalg.norm(got - ref_out) / np.linalg.norm(ref_out)
        lit_plain = np.abs(got - ref_out).max() / rms
        say(f"  out ({toks.size} tokens): vs oracle(GPU h) max/RMS {d2.max() / rms:.3e}, over the literal "
            f"bound {int((d2 > lit).sum())}, over the combine bound {int((d2 > cb).sum())}, rel_fro "
            f"{rel2:.3e}; vs plain oracle rel_fro {rel:.3e} (max/RMS {lit_plain:.3e}) of {d2.size}")
        assert not (d2 > lit).any()
        assert not (d2 > cb).any()
        assert rel2 <= REL_FRO_TOL and rel <= REL_FRO_TOL
        return dict(rel_fro=rel, max_over_rms=d2.max() / rms, rel_fro_gpu_h=rel2)


def oracle_forward_out(li, top_k, I, ox, toks, fmt):
    """``oracle.forward(...)["out"]`` of the tokens ``toks``, its per-expert FFNs on the check
    threads (``ox``: an OracleExperts holding every expert the tokens use)."""
    q_act, dq_act, _ = R._quantizer(fmt)
    logits = R.router_logits(li.x, li.router_w, li.router_b)
    ids, gates = R.topk_softmax(logits, top_k)
    x32 = R.bf16_to_f64(li.x).astype(np.float32)
    toks = np.asarray(toks)
    xq, sx = q_act(x32[toks])
    xd = dq_act(xq, sx)
    H = li.x.shape[1]
    experts = [int(e) for e in np.unique(ids[toks])]
    ox.prepare(experts)

    def ffn(e):
        rows_t, rows_j = np.nonzero(ids[toks] == e)
        c13, s13, c2, s2 = ox.cache[e]
        ye = R.expert_ffn(xd[rows_t], c13, s13, li.b13[e], c2, s2, li.b2[e], I, fmt)[0]
        return rows_t, rows_j, ye

    y = np.zeros((toks.size, top_k, H))
    for rows_t, rows_j, ye in par_map(ffn, experts):
        y[rows_t, rows_j] = ye
    return np.einsum("tk,tkh->th", gates[toks], y)


def pick_experts(counts, bm=256, extra=16):
    """Experts whose every row the prefill checks cover: one whose single M-tile holds rows
    past 256 (256 < rows <= 256 + extra: the full tile's extra rows; MXFP4 splits it), one with a full 256-row tile and a narrow overflow tile
    (256 + extra < rows <= 320), if any, the hottest, and the least busy active one."""
    act = np.nonzero(counts > 0)[0]
    pick = [int(act[np.argmax(counts[act])]), int(act[np.argmin(counts[act])])]
    for lo, hi in ((bm + extra, bm + 64), (bm, bm + extra)):
        over = np.nonzero((counts > lo) & (counts <= hi))[0]
        if over.size:
            pick.insert(0, int(over[0]))
    return list(dict.fromkeys(pick))


def check_all_rows(shape, fmt="block", fused=False):
    """Every routed row's h and y and every token's out (small and decode-sized layers);
    ``fused``: the layer through the one-kernel decode path."""
    g = GpuLayer(shape, fmt=fmt)
    out, routing = g.run(fused=fused)
    chk = LayerCheck(g, out, routing)
    chk.check_experts()
    chk.check_tokens(h_window=False)


def check_prefill(shape, fmt, n_sample, seed):
    """A full-size layer: whole experts (pick_experts) and sampled tokens, the last included."""
    g = GpuLayer(shape, fmt=fmt)
    out, routing = g.run()
    chk = LayerCheck(g, out, routing)
    experts = pick_experts(chk.counts)
    say(f"  whole experts {experts} with {[int(chk.counts[e]) for e in experts]} rows")
    chk.check_experts(experts)
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(shape.T, size=n_sample, replace=False))
    toks[-1] = shape.T - 1                                   # the last token (ragged tiles)
    chk.check_tokens(toks)
