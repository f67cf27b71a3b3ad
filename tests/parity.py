"""Helpers for the GPU parity tests: run the CPU oracle and the HIP path on the
same seeded inputs and compare them.

Bar (stated once here, used by every GPU test):
  * bit-exact: labels, row offsets, W4/W8 bytes, FP32 scale bits, INT8
    activation codes, FP32 activation-scale bits, INT32 tile products;
  * outputs (FP32 epilogue vs the FP64 oracle):
      (i)  normwise   max|Y - y| <= 1e-4 * max|y|
      (ii) componentwise |Y - y| <= 1e-4 * (sum_j |s_x s_W P_j| + |bias_n|) + 1e-30
    An FP32 evaluation of eq. 19 with C tile terms and the bias errs by at
    most about (C + 3) * 2^-24 * (sum_j |term_j| + |bias_n|), far inside (ii)
    for C <= 200.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import mixed_precision_int_amd as aq
from oracle import aq_oracle as O

REL_TOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def packed_to_host(pw: aq.PackedWeights) -> dict:
    p = pw.plan
    torch.cuda.synchronize()
    return dict(
        labels=pw.labels[:p.labels_bytes].cpu().numpy(),
        row_off4=pw.row_off4[:p.offs_bytes].cpu().numpy().view(np.int32),
        row_off8=pw.row_off8[:p.offs_bytes].cpu().numpy().view(np.int32),
        w4=pw.w4[:p.w4_bytes].cpu().numpy(),
        w8=pw.w8[:p.w8_bytes].cpu().numpy(),
        s4=pw.s4[:p.s4_bytes].cpu().numpy().view(np.float32),
        s8=pw.s8[:p.s8_bytes].cpu().numpy().view(np.float32),
    )


def assert_packed_equal(gpu: dict, ref: dict, name=""):
    for k in ("labels", "row_off4", "row_off8", "w4", "w8"):
        g, r = np.asarray(gpu[k]), np.asarray(ref[k])
        assert g.shape == r.shape, (name, k, g.shape, r.shape)
        bad = np.flatnonzero(g.view(np.uint8) != r.astype(g.dtype).view(np.uint8)) if g.size else []
        assert len(bad) == 0, f"{name}: {k} differs at {len(bad)} bytes, first {bad[:8]}"
    for k in ("s4", "s8"):
        g, r = gpu[k].view(np.uint32), ref[k].astype(np.float32).view(np.uint32)
        assert g.shape == r.shape and np.array_equal(g, r), f"{name}: {k} bits differ"


def assert_output_close(Y: np.ndarray, y: np.ndarray, contrib: np.ndarray, name=""):
    Y = np.asarray(Y, dtype=np.float64)
    assert Y.shape == y.shape, (name, Y.shape, y.shape)
    assert np.all(np.isfinite(Y)), f"{name}: non-finite output"
    d = np.abs(Y - y)
    ymax = float(np.max(np.abs(y))) if y.size else 0.0
    normwise = float(d.max() / ymax) if ymax > 0 else float(d.max())
    comp_ok = d <= REL_TOL * contrib + 1e-30
    say(f"  {name}: normwise err {normwise:.3e}, componentwise worst ratio "
        f"{float(np.max(d / (contrib + 1e-30))) if y.size else 0:.3e}")
    assert normwise <= REL_TOL, f"{name}: normwise error {normwise:.3e} > {REL_TOL}"
    assert comp_ok.all(), f"{name}: componentwise gate fails at {np.argwhere(~comp_ok)[:5].tolist()}"


class Case:
    """One linear problem run through both sides."""

    def __init__(self, W, zmap, X, bN=64, bK=128, bias=None, name="case"):
        self.W = np.ascontiguousarray(W, dtype=np.float32)
        self.zmap = np.asarray(zmap)
        self.X = np.ascontiguousarray(X, dtype=np.float32)
        self.bN, self.bK = bN, bK
        self.bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        self.name = name
        self._ref = None

    # ---- oracle side
    def ref(self, rows=None):
        if self._ref is None:
            codes, sW = O.quant_weights(self.W, self.zmap, self.bN, self.bK)
            pk = O.pack(codes, sW, self.zmap, self.bN, self.bK)
            qx, sx = O.quant_act(self.X)
            self._ref = dict(codes=codes, sW=sW, pk=pk, qx=qx, sx=sx)
        r = self._ref
        if rows is not None and "P_rows" not in r:
            P = O.tile_partials(r["qx"][rows], r["codes"], self.bK)
            r["P_rows"] = P
            r["y_rows"] = O.linear_from_partials(P, r["sx"][rows], r["sW"], self.bias)
            r["c_rows"] = O.abs_contrib(P, r["sx"][rows], r["sW"])
            if self.bias is not None:
                r["c_rows"] = r["c_rows"] + np.abs(self.bias.astype(np.float64))[None, :]
            r["rows"] = rows
        return r

    # ---- HIP side
    def gpu_pack(self):
        labels = aq.aq_labels_from_map(self.zmap.astype(np.uint8))
        self.pw = aq.aq_pack_weights(to_dev(self.W), labels, self.bN, self.bK)
        return self.pw

    def gpu_quant(self):
        self.qx_d, self.sx_d = aq.aq_quant_act(to_dev(self.X))
        return self.qx_d, self.sx_d

    def check_all(self, rows=None, phases=("decode", "prefill"), splits=(0,)):
        """Pack, quantize, partials and outputs against the oracle."""
        say(f"[{self.name}] N={self.W.shape[0]} K={self.W.shape[1]} M={self.X.shape[0]} "
            f"tile={self.bN}x{self.bK} T8={int(np.sum(self.zmap == 8))}/{self.zmap.size}")
        M = self.X.shape[0]
        rows = np.arange(M) if rows is None else np.asarray(rows)
        ref = self.ref(rows)
        pw = self.gpu_pack()
        assert_packed_equal(packed_to_host(pw), ref["pk"], self.name)
        qx_d, sx_d = self.gpu_quant()
        torch.cuda.synchronize()
        assert np.array_equal(qx_d.cpu().numpy().astype(np.int64), ref["qx"]), f"{self.name}: qx differs"
        assert np.array_equal(sx_d.cpu().numpy().view(np.uint32),
                              ref["sx"].astype(np.float32).view(np.uint32)), f"{self.name}: sx bits differ"
        rows_d = torch.from_numpy(rows).cuda()
        qx_rows = qx_d.index_select(0, rows_d).contiguous()
        sx_rows = sx_d.index_select(0, rows_d).contiguous()
        bias_d = None if self.bias is None else to_dev(self.bias)
        out = {}
        for ph in phases:
            phase = aq.AQ_PHASE_DECODE if ph == "decode" else aq.AQ_PHASE_PREFILL
            P = aq.aq_linear_tile_partials(pw, qx_rows, phase)
            torch.cuda.synchronize()
            Pg = P.cpu().numpy().astype(np.int64)
            bad = np.argwhere(Pg != ref["P_rows"])
            assert bad.size == 0, f"{self.name}/{ph}: {len(bad)} partials differ, first {bad[:4].tolist()}"
            if ph == "decode":
                Wv = 16  # waves per decode workgroup
                ok = {0, Wv, Wv // 2, Wv // 4}
                for s in sorted({s for s in splits if s in ok} | {0}):
                    Y = aq.aq_linear_decode(pw, qx_rows, sx_rows, bias_d, split=s)
                    torch.cuda.synchronize()
                    assert_output_close(Y.cpu().numpy(), ref["y_rows"], ref["c_rows"],
                                        f"{self.name}/decode/split{s}")
                    out[f"decode{s}"] = Y
            else:
                Y = aq.aq_linear_prefill(pw, qx_rows, sx_rows, bias_d)
                torch.cuda.synchronize()
                assert_output_close(Y.cpu().numpy(), ref["y_rows"], ref["c_rows"], f"{self.name}/prefill")
                out["prefill"] = Y
        return out
