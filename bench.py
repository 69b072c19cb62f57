#!/usr/bin/env python3
"""Throughput of the WKV-4 forward hot path on one MI355X.

One step = one ``wkv4_forward`` call (the whole operator: every kernel it launches) over
the B=8, T=1024, C=768 float32 workload (169m-style width), synthetic seeded inputs
already resident in HBM.  Prints ONE JSON line on stdout; diagnostics go to stderr.

Input/output buffer sets are rotated so that the 256 MB last-level cache (MALL) cannot
serve a repeated call: R = ceil(2 * 256 MB / footprint) sets.

The line also carries ``stream_ceiling`` (the same bytes moved by a plain elementwise
kernel, y = k + v, over the same rotated buffers), ``copy_probe_GBps`` (a 1 GiB device copy)
and ``workloads``: the WKV forward, backward and checkpointed training step at B=8 T=4096
C=2560, the real scan and fused minGRU at B=64 T=4096 C=256 and the LRU complex scan at B=1
T=262144 C=1024, a few launches each (``--no-workloads`` skips them).

``--all`` also measures the other rows (WKV-4 forward, backward and gated backward at B=8
T=4096 C=2560; the real scan, minGRU, minLSTM, the per-channel decay and their adjoints at
B=64 T=4096 C=256; the LRU complex scan, the normalised LRU and their adjoints at B=1
T=262144 C=1024; the RWKV token shift and its backward at B=8 T=1024 C=768 with 3 mixes),
logs each on stderr and, with ``--all-out PATH``, writes them to PATH (they are parity
workloads, not the headline line).
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "WKV elements/s + achieved HBM GB/s (% peak), B=8 T=1024 C=768 fp32"
PEAK_HBM_GBPS = 8000.0          # MI355X published HBM3E bandwidth
MALL_BYTES = 256 * 1024 * 1024  # MI355X Infinity Cache
# Algorithmic bytes per element: inputs read once, outputs written once.
BYTES_PER_ELEM = {"wkv4_forward": 12, "wkv4_backward": 20, "scan_real": 12, "scan_complex": 16,
                  "scan_real_backward": 20,      # read a, x, gx; write ga, gb
                  "scan_complex_backward": 24,   # read x, gx; write gu (complex64)
                  "scan_mingru": 12,             # read kz, h; write x
                  "scan_minlstm": 16,            # read kf, ki, h; write x
                  "scan_real_decay": 8,          # read u; write x
                  "scan_complex_normalized": 16, # read u; write x (complex64)
                  "token_shift": 16,             # read x; write 3 mixes
                  "token_shift_backward": 20,    # read x, 3 gradients; write gx
                  "wkv4_backward_gated": 28,     # read k, v, r, gy; write gk, gv, gr
                  "wkv4_forward_gated": 16,      # read k, v, r; write sigma(r) wkv
                  "scan_mingru_backward": 24,    # read kz, h, x, gx; write gkz, gh
                  "scan_minlstm_backward": 32,   # read kf, ki, h, x, gx; write gkf, gki, gh
                  "scan_real_decay_backward": 12,  # read x, gx; write gu
                  "scan_complex_normalized_backward": 32,  # read u, x, gx; write gu (complex64)
                  "wkv4_train_step": 32,         # forward (12) then backward (20), separate passes
                  "wkv4_train_step_ckpt": 32,    # the same step, the backward from the forward's sums
                  "wkv4_train_step_gated": 44,   # gated forward (16) then gated backward (28)
                  "wkv4_train_step_gated_ckpt": 44,
                  "wkv4_train_step_state": 32,   # forward then backward of a piece with a carried state
                  "wkv4_train_step_state_ckpt": 32}
SHIFT_M = 3  # token-shift mixes timed: the r, k, v inputs of the time mix

# The rows of --all after the headline, in order: (workload id, row, timed steps, time steps of
# the oracle baseline's sample).
ALL_ROWS = (
    (3, "wkv4_forward", 20, 512), (3, "wkv4_backward", 20, 256),
    (4, "scan_real", 20, 512), (5, "scan_complex", 10, 16384),
    (4, "scan_real_backward", 20, 512),
    (5, "scan_complex_backward", 10, 16384),
    (4, "scan_mingru", 20, 512), (4, "scan_minlstm", 20, 512),
    (4, "scan_real_decay", 20, 512), (5, "scan_complex_normalized", 10, 16384),
    (2, "token_shift", 50, None), (2, "token_shift_backward", 50, None),
    (3, "wkv4_forward_gated", 20, 512), (3, "wkv4_backward_gated", 20, 256),
    (4, "scan_mingru_backward", 20, 512), (4, "scan_minlstm_backward", 20, 512),
    (4, "scan_real_decay_backward", 20, 512),
    (5, "scan_complex_normalized_backward", 10, 16384),
    (3, "wkv4_train_step", 10, 256), (3, "wkv4_train_step_ckpt", 10, 256),
    (3, "wkv4_train_step_gated", 10, 256),
    (3, "wkv4_train_step_gated_ckpt", 10, 256),
    (3, "wkv4_train_step_state", 10, 256),
    (3, "wkv4_train_step_state_ckpt", 10, 256))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources each entry point's kernels are built from (the launch plan lives in api.hip).
_SCAN_SOURCES = ("api.hip", "chunk_scan.hip", "chunk_scan.hpp", "scan_kernel.hpp", "scan_ops.hpp", "lookback.hpp",
                 "part_reduce.hpp",
                 "device_common.hpp", "wkv_math.hpp")
KERNEL_SOURCES = {
    "wkv4_forward": _SCAN_SOURCES,
    "wkv4_forward_gated": _SCAN_SOURCES,
    "scan_real": _SCAN_SOURCES,
    "scan_complex": _SCAN_SOURCES,
    "scan_real_backward": _SCAN_SOURCES,
    "scan_complex_backward": _SCAN_SOURCES,
    "scan_mingru": _SCAN_SOURCES + ("scan_kernel.hpp", "scan_variants.hip"),
    "scan_minlstm": _SCAN_SOURCES + ("scan_kernel.hpp", "scan_variants.hip"),
    "scan_real_decay": _SCAN_SOURCES + ("scan_kernel.hpp", "scan_variants.hip"),
    "scan_complex_normalized": _SCAN_SOURCES + ("scan_kernel.hpp", "scan_variants.hip"),
    "token_shift": ("api.hip", "token_shift.hip", "token_shift.hpp", "device_common.hpp"),
    "token_shift_backward": ("api.hip", "token_shift.hip", "token_shift.hpp", "device_common.hpp"),
    "wkv4_backward": ("api.hip", "wkv_backward.hip", "wkv_backward.hpp", "lookback.hpp", "device_common.hpp",
                      "wkv_math.hpp", "wkv_sums.hpp"),
    "wkv4_backward_gated": ("api.hip", "wkv_backward.hip", "wkv_backward.hpp", "lookback.hpp",
                            "device_common.hpp", "wkv_math.hpp", "wkv_sums.hpp"),
}
KERNEL_SOURCES["wkv4_train_step"] = tuple(sorted(set(_SCAN_SOURCES + KERNEL_SOURCES["wkv4_backward"])))
KERNEL_SOURCES["wkv4_train_step_gated"] = KERNEL_SOURCES["wkv4_train_step"]
KERNEL_SOURCES["wkv4_train_step_gated_ckpt"] = tuple(sorted(set(
    _SCAN_SOURCES + KERNEL_SOURCES["wkv4_backward"] + ("wkv_ckpt.hip", "wkv_sums.hpp"))))
KERNEL_SOURCES["wkv4_train_step_state"] = KERNEL_SOURCES["wkv4_train_step"]
KERNEL_SOURCES["wkv4_train_step_state_ckpt"] = KERNEL_SOURCES["wkv4_train_step_gated_ckpt"]
KERNEL_SOURCES["wkv4_train_step_ckpt"] = tuple(sorted(set(
    _SCAN_SOURCES + KERNEL_SOURCES["wkv4_backward"] + ("wkv_ckpt.hip", "wkv_sums.hpp"))))
for _k in ("scan_mingru_backward", "scan_minlstm_backward", "scan_real_decay_backward",
           "scan_complex_normalized_backward"):
    KERNEL_SOURCES[_k] = _SCAN_SOURCES + ("scan_variants.hip",)
VARIANT_BWD = ("scan_mingru_backward", "scan_minlstm_backward", "scan_real_decay_backward")


def kernel_source_digest(kind: str = "wkv4_forward") -> str:
    """Digest of the HIP sources of one entry point: counter figures taken from an older
    build of those kernels do not apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_recurrence_rnn_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[kind]):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def counter_traffic(kind: str, B: int, T: int, C: int):
    """HBM bytes per step of row `kind` at (B, T, C) from the committed rocprofv3 counter
    record (profiles/counters.json), if it was taken on the current kernel sources; None
    otherwise."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)["rows"].get("%s@%dx%dx%d" % (kind, B, T, C))
    except (OSError, ValueError, KeyError, AttributeError):
        return None
    if not rec or rec.get("source_digest") != kernel_source_digest(kind):
        return None
    return rec.get("hbm_bytes_per_step")


class Row:
    """Pre-marshalled launches of one entry point over R rotated buffer sets."""

    def __init__(self, lib, kind, B, T, C, host, rotations):
        import torch

        self.kind, self.B, self.T, self.C = kind, B, T, C
        self.elements = B * T * C
        dev = torch.device("cuda")
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.keep = []
        self.calls = []
        to = lambda x: torch.from_numpy(x).to(dev)  # noqa: E731
        if kind == "wkv4_forward":
            w, u = to(host["w"]), to(host["u"])
            nws = int(lib.wkv4_forward_workspace_size(B, T, C))
            for _ in range(rotations):
                k, v = to(host["k"]), to(host["v"])
                y = torch.empty_like(k)
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += [k, v, y, ws]
                self.calls.append((lib.wkv4_forward, (B, T, C, w.data_ptr(), u.data_ptr(), k.data_ptr(),
                                   v.data_ptr(), y.data_ptr(), ws.data_ptr(), nws, stream)))
            self.keep += [w, u]
        elif kind == "wkv4_backward":
            w, u = to(host["w"]), to(host["u"])
            nws = int(lib.wkv4_backward_workspace_size(B, T, C))
            for _ in range(rotations):
                k, v, gy = to(host["k"]), to(host["v"]), to(host["gy"])
                gk, gv = torch.empty_like(k), torch.empty_like(k)
                gw = torch.empty(C, dtype=torch.float32, device=dev)
                gu = torch.empty(C, dtype=torch.float32, device=dev)
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += [k, v, gy, gk, gv, gw, gu, ws]
                self.calls.append((lib.wkv4_backward, (B, T, C, w.data_ptr(), u.data_ptr(), k.data_ptr(),
                                   v.data_ptr(), gy.data_ptr(), gw.data_ptr(), gu.data_ptr(),
                                   gk.data_ptr(), gv.data_ptr(), ws.data_ptr(), nws, stream)))
            self.keep += [w, u]
        elif kind.startswith("wkv4_train_step") and "_state" not in kind:
            # One training step of the WKV layer: the forward, then the backward of its output
            # (with the sigma(r) gate of the time mix for the gated rows).
            w, u = to(host["w"]), to(host["u"])
            ck = kind.endswith("_ckpt")
            gated = "_gated" in kind
            nfw = int(lib.wkv4_forward_ckpt_workspace_size(B, T, C) if ck else lib.wkv4_forward_workspace_size(B, T, C))
            nbw = int(lib.wkv4_backward_ckpt_workspace_size(B, T, C) if ck else
                      lib.wkv4_backward_workspace_size(B, T, C))
            nck = int(lib.wkv4_checkpoint_size(B, T, C)) if ck else 0
            fws = torch.empty(max(nfw, 1), dtype=torch.uint8, device=dev)
            bws = torch.empty(max(nbw, 1), dtype=torch.uint8, device=dev)
            gw = torch.empty(C, dtype=torch.float32, device=dev)
            gu = torch.empty(C, dtype=torch.float32, device=dev)
            self.keep += [w, u, fws, bws, gw, gu]
            for _ in range(rotations):
                k, v, gy = to(host["k"]), to(host["v"]), to(host["gy"])
                y, gk, gv = torch.empty_like(k), torch.empty_like(k), torch.empty_like(k)
                cbuf = torch.empty(max(nck, 1), dtype=torch.uint8, device=dev)
                self.keep += [k, v, gy, y, gk, gv, cbuf]
                p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
                r = to(host["r"]) if gated else None
                gr = torch.empty_like(k) if gated else None
                self.keep += [r, gr]
                if ck:
                    fa = (lib.wkv4_forward_ckpt, (B, T, C, p(w), p(u), p(k), p(v), p(r), p(y), p(cbuf), nck, p(fws),
                                                  nfw, stream))
                    ba = (lib.wkv4_backward_ckpt, (B, T, C, p(w), p(u), p(k), p(v), p(r), p(gy), p(cbuf), nck, p(gw),
                                                   p(gu), p(gk), p(gv), p(gr), p(bws), nbw, stream))
                elif gated:
                    fa = (lib.wkv4_forward_ex, (B, T, C, p(w), p(u), p(k), p(v), p(r), None, p(y), None, p(fws), nfw,
                                                stream))
                    ba = (lib.wkv4_backward_ex, (B, T, C, p(w), p(u), p(k), p(v), p(r), None, None, p(gy), None, p(gw),
                                                 p(gu), p(gk), p(gv), p(gr), None, p(bws), nbw, stream))
                else:
                    fa = (lib.wkv4_forward, (B, T, C, p(w), p(u), p(k), p(v), p(y), p(fws), nfw, stream))
                    ba = (lib.wkv4_backward, (B, T, C, p(w), p(u), p(k), p(v), p(gy), p(gw), p(gu), p(gk), p(gv),
                                              p(bws), nbw, stream))

                def both(fa=fa, ba=ba):
                    st = fa[0](*fa[1])
                    return st if st else ba[0](*ba[1])
                self.calls.append((both, ()))
        elif kind.startswith("wkv4_train_step_state"):
            # One training step of a piece of a longer sequence: the forward from a carried
            # state (writing the state after the piece), then the backward with the gradient
            # of that final state (plain: wkv4_forward_ex / wkv4_backward_ex; checkpointed:
            # wkv4_forward_ckpt_ex / wkv4_backward_ckpt_ex).
            w, u = to(host["w"]), to(host["u"])
            ck = kind.endswith("_ckpt")
            nfw = int(lib.wkv4_forward_ckpt_workspace_size(B, T, C) if ck else lib.wkv4_forward_workspace_size(B, T, C))
            nbw = int(lib.wkv4_backward_ckpt_workspace_size(B, T, C) if ck else
                      lib.wkv4_backward_workspace_size(B, T, C))
            nck = int(lib.wkv4_checkpoint_size(B, T, C)) if ck else 0
            fws = torch.empty(max(nfw, 1), dtype=torch.uint8, device=dev)
            bws = torch.empty(max(nbw, 1), dtype=torch.uint8, device=dev)
            gw = torch.empty(C, dtype=torch.float32, device=dev)
            gu = torch.empty(C, dtype=torch.float32, device=dev)
            s_in, gs_out = to(host["s_in"]), to(host["gs_out"])
            s_out = torch.empty_like(s_in)
            gs_in = torch.empty_like(gs_out)
            self.keep += [w, u, fws, bws, gw, gu, s_in, gs_out, s_out, gs_in]
            p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
            for _ in range(rotations):
                k, v, gy = to(host["k"]), to(host["v"]), to(host["gy"])
                y, gk, gv = torch.empty_like(k), torch.empty_like(k), torch.empty_like(k)
                cbuf = torch.empty(max(nck, 1), dtype=torch.uint8, device=dev)
                self.keep += [k, v, gy, y, gk, gv, cbuf]
                if ck:
                    fa = (lib.wkv4_forward_ckpt_ex, (B, T, C, p(w), p(u), p(k), p(v), None, p(s_in), p(y), p(s_out),
                                                     p(cbuf), nck, p(fws), nfw, stream))
                    ba = (lib.wkv4_backward_ckpt_ex, (B, T, C, p(w), p(u), p(k), p(v), None, p(s_in), p(s_out), p(gy),
                                                      p(gs_out), p(cbuf), nck, p(gw), p(gu), p(gk), p(gv), None,
                                                      p(gs_in), p(bws), nbw, stream))
                else:
                    fa = (lib.wkv4_forward_ex, (B, T, C, p(w), p(u), p(k), p(v), None, p(s_in), p(y), p(s_out),
                                                p(fws), nfw, stream))
                    ba = (lib.wkv4_backward_ex, (B, T, C, p(w), p(u), p(k), p(v), None, p(s_in), p(s_out), p(gy),
                                                 p(gs_out), p(gw), p(gu), p(gk), p(gv), None, p(gs_in), p(bws), nbw,
                                                 stream))

                def both(fa=fa, ba=ba):
                    st = fa[0](*fa[1])
                    return st if st else ba[0](*ba[1])
                self.calls.append((both, ()))
        elif kind == "wkv4_forward_gated":
            w, u = to(host["w"]), to(host["u"])
            nws = int(lib.wkv4_forward_workspace_size(B, T, C))
            for _ in range(rotations):
                k, v, r = to(host["k"]), to(host["v"]), to(host["r"])
                y = torch.empty_like(k)
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += [k, v, r, y, ws]
                self.calls.append((lib.wkv4_forward_ex, (B, T, C, w.data_ptr(), u.data_ptr(), k.data_ptr(),
                                   v.data_ptr(), r.data_ptr(), None, y.data_ptr(), None, ws.data_ptr(), nws,
                                   stream)))
            self.keep += [w, u]
        elif kind == "wkv4_backward_gated":
            w, u = to(host["w"]), to(host["u"])
            nws = int(lib.wkv4_backward_workspace_size(B, T, C))
            gw = torch.empty(C, dtype=torch.float32, device=dev)
            gu = torch.empty(C, dtype=torch.float32, device=dev)
            for _ in range(rotations):
                k, v, r, gy = to(host["k"]), to(host["v"]), to(host["r"]), to(host["gy"])
                gk, gv, gr = torch.empty_like(k), torch.empty_like(k), torch.empty_like(k)
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += [k, v, r, gy, gk, gv, gr, ws]
                self.calls.append((lib.wkv4_backward_ex, (B, T, C, w.data_ptr(), u.data_ptr(), k.data_ptr(),
                                   v.data_ptr(), r.data_ptr(), None, None, gy.data_ptr(), None, gw.data_ptr(),
                                   gu.data_ptr(), gk.data_ptr(), gv.data_ptr(), gr.data_ptr(), None,
                                   ws.data_ptr(), nws, stream)))
            self.keep += [w, u, gw, gu]
        elif kind in VARIANT_BWD:
            names = {"scan_mingru_backward": ("kz", "h"), "scan_minlstm_backward": ("kf", "ki", "h"),
                     "scan_real_decay_backward": ()}[kind]
            n_out = {"scan_mingru_backward": 2, "scan_minlstm_backward": 3, "scan_real_decay_backward": 1}[kind]
            fn = getattr(lib, "linrec_" + kind)
            nws = int(lib.linrec_scan_backward_workspace_size(B, T, C, 0))
            lam = to(host["lam"]) if kind == "scan_real_decay_backward" else None
            glam = torch.empty(C, dtype=torch.float32, device=dev)
            for _ in range(rotations):
                ins = [to(host[n]) for n in names]
                x, gx = to(host["x"]), to(host["gx"])
                outs = [torch.empty_like(x) for _ in range(n_out)]
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += ins + [x, gx, ws] + outs
                if lam is not None:
                    ptrs = [lam.data_ptr(), None, x.data_ptr(), gx.data_ptr(), glam.data_ptr(), outs[0].data_ptr()]
                else:
                    ptrs = [t.data_ptr() for t in ins] + [None, x.data_ptr(), gx.data_ptr()] + [o.data_ptr() for o in outs]
                self.calls.append((fn, (B, T, C, *ptrs, None, ws.data_ptr(), nws, stream)))
            self.keep += [glam] + ([lam] if lam is not None else [])
        elif kind == "scan_complex_normalized_backward":
            lam = to(host["lam"])
            nws = int(lib.linrec_scan_backward_workspace_size(B, T, C, 1))
            glam = torch.empty(C, dtype=torch.complex64, device=dev)
            for _ in range(rotations):
                u, x, gx = to(host["u"]), to(host["x"]), to(host["gx"])
                gu = torch.empty_like(x)
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += [u, x, gx, gu, ws]
                self.calls.append((lib.linrec_scan_complex_normalized_backward,
                                   (B, T, C, lam.data_ptr(), u.data_ptr(), None, x.data_ptr(), gx.data_ptr(),
                                    glam.data_ptr(), gu.data_ptr(), None, ws.data_ptr(), nws, stream)))
            self.keep += [lam, glam]
        elif kind == "scan_real":
            nws = int(lib.linrec_scan_workspace_size(B, T, C, 0))
            for _ in range(rotations):
                a, b = to(host["a"]), to(host["b"])
                x = torch.empty_like(a)
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += [a, b, x, ws]
                self.calls.append((lib.linrec_scan_real, (B, T, C, a.data_ptr(), b.data_ptr(), None,
                                   x.data_ptr(), ws.data_ptr(), nws, stream)))
        elif kind == "scan_complex":
            lam = to(host["lam"])
            nws = int(lib.linrec_scan_workspace_size(B, T, C, 1))
            for _ in range(rotations):
                u = to(host["u"])
                x = torch.empty_like(u)
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += [u, x, ws]
                self.calls.append((lib.linrec_scan_complex, (B, T, C, lam.data_ptr(), u.data_ptr(), None,
                                   x.data_ptr(), ws.data_ptr(), nws, stream)))
            self.keep.append(lam)
        elif kind == "scan_real_backward":
            nws = int(lib.linrec_scan_backward_workspace_size(B, T, C, 0))
            for _ in range(rotations):
                a, x, gx = to(host["a"]), to(host["x"]), to(host["gx"])
                ga, gb = torch.empty_like(a), torch.empty_like(a)
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += [a, x, gx, ga, gb, ws]
                self.calls.append((lib.linrec_scan_real_backward, (B, T, C, a.data_ptr(), None, x.data_ptr(),
                                   gx.data_ptr(), ga.data_ptr(), gb.data_ptr(), None, ws.data_ptr(), nws,
                                   stream)))
        elif kind == "scan_complex_backward":
            lam = to(host["lam"])
            nws = int(lib.linrec_scan_backward_workspace_size(B, T, C, 1))
            glam = torch.empty(C, dtype=torch.complex64, device=dev)
            for _ in range(rotations):
                x, gx = to(host["x"]), to(host["gx"])
                gu = torch.empty_like(x)
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += [x, gx, gu, ws]
                self.calls.append((lib.linrec_scan_complex_backward, (B, T, C, lam.data_ptr(), None, x.data_ptr(),
                                   gx.data_ptr(), glam.data_ptr(), gu.data_ptr(), None, ws.data_ptr(), nws,
                                   stream)))
            self.keep += [lam, glam]
        elif kind in ("scan_mingru", "scan_minlstm", "scan_real_decay"):
            names = {"scan_mingru": ("kz", "h"), "scan_minlstm": ("kf", "ki", "h"), "scan_real_decay": ("h",)}[kind]
            fn = getattr(lib, "linrec_" + kind)
            nws = int(lib.linrec_scan_workspace_size(B, T, C, 0))
            lam = to(host["lam"]) if kind == "scan_real_decay" else None
            for _ in range(rotations):
                ins = [to(host[n]) for n in names]
                x = torch.empty_like(ins[0])
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += ins + [x, ws]
                ptrs = ([lam.data_ptr()] if lam is not None else []) + [t.data_ptr() for t in ins]
                self.calls.append((fn, (B, T, C, *ptrs, None, x.data_ptr(), ws.data_ptr(), nws, stream)))
            if lam is not None:
                self.keep.append(lam)
        elif kind == "scan_complex_normalized":
            lam = to(host["lam"])
            nws = int(lib.linrec_scan_workspace_size(B, T, C, 1))
            for _ in range(rotations):
                u = to(host["u"])
                x = torch.empty_like(u)
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += [u, x, ws]
                self.calls.append((lib.linrec_scan_complex_normalized, (B, T, C, lam.data_ptr(), u.data_ptr(), None,
                                   x.data_ptr(), ws.data_ptr(), nws, stream)))
            self.keep.append(lam)
        elif kind == "token_shift":
            M = host["mu"].shape[0]
            mu = to(host["mu"])
            for _ in range(rotations):
                x = to(host["x"])
                out = torch.empty((M, B, T, C), dtype=torch.float32, device=dev)
                self.keep += [x, out]
                self.calls.append((lib.rwkv_token_shift, (B, T, C, M, x.data_ptr(), None, mu.data_ptr(),
                                   out.data_ptr(), stream)))
            self.keep.append(mu)
        elif kind == "token_shift_backward":
            M = host["mu"].shape[0]
            mu = to(host["mu"])
            nws = int(lib.rwkv_token_shift_backward_workspace_size(B, T, C, M))
            gmu = torch.empty((M, C), dtype=torch.float32, device=dev)
            for _ in range(rotations):
                x, g = to(host["x"]), to(host["g"])
                gx = torch.empty_like(x)
                ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
                self.keep += [x, g, gx, ws]
                self.calls.append((lib.rwkv_token_shift_backward, (B, T, C, M, x.data_ptr(), None, mu.data_ptr(),
                                   g.data_ptr(), gx.data_ptr(), gmu.data_ptr(), None, ws.data_ptr(), nws,
                                   stream)))
            self.keep += [mu, gmu]
        else:
            raise KeyError(kind)

    def launch(self, i):
        fn, args = self.calls[i % len(self.calls)]
        st = fn(*args)
        if st != 0:
            raise RuntimeError("%s returned status %d" % (self.kind, st))

    def run(self, steps, warmup, min_warm_s=0.0):
        """Times `steps` launches after `warmup` untimed ones; with ``min_warm_s``, the warm-up
        goes on (in batches of `warmup`) until that much wall time has passed, so that the GPU
        has left its idle clocks (a backward at B8 T4096 C2560 runs ~10% slower for its first
        ~50 launches after an idle second).  Returns (wall seconds, event seconds)."""
        import torch

        t_w = time.perf_counter()
        i = 0
        while True:
            for _ in range(warmup):
                self.launch(i)
                i += 1
            if warmup <= 0 or min_warm_s <= 0.0:
                break
            torch.cuda.synchronize()
            if time.perf_counter() - t_w >= min_warm_s:
                break
        warmup = i
        stream = torch.cuda.current_stream()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            self.launch(warmup + i)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, ev0.elapsed_time(ev1) / 1e3


def rotations_for(footprint_bytes: int) -> int:
    return max(1, math.ceil(2 * MALL_BYTES / footprint_bytes))


def roofline(kind, elements, launch_s, traffic):
    algo = BYTES_PER_ELEM[kind] * elements
    achieved = algo / launch_s / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
            "algorithmic_bytes": algo}


def _state_step(host):
    """The oracle's training step of a piece with a carried state."""
    import oracle

    _, s_out = oracle.wkv4_forward_ex(host["w"], host["u"], host["k"], host["v"], s_in=host["s_in"])
    return oracle.wkv4_backward_ex(host["w"], host["u"], host["k"], host["v"], host["gy"], s_in=host["s_in"],
                                   s_out=s_out.astype("float32"), gs_out=host["gs_out"])


def cpu_baseline(kind, host, budget_s):
    """The fp64 oracle, as it stands, on the host cores: median seconds per call."""
    import oracle

    fn = {"wkv4_forward": lambda: oracle.wkv4_forward(host["w"], host["u"], host["k"], host["v"]),
          "wkv4_backward": lambda: oracle.wkv4_backward(host["w"], host["u"], host["k"], host["v"],
                                                        host["gy"]),
          "wkv4_train_step": lambda: (oracle.wkv4_forward(host["w"], host["u"], host["k"], host["v"]),
                                      oracle.wkv4_backward(host["w"], host["u"], host["k"], host["v"], host["gy"])),
          "wkv4_train_step_ckpt": lambda: (oracle.wkv4_forward(host["w"], host["u"], host["k"], host["v"]),
                                           oracle.wkv4_backward(host["w"], host["u"], host["k"], host["v"],
                                                                host["gy"])),
          "wkv4_train_step_gated": lambda: (
              oracle.wkv4_forward_ex(host["w"], host["u"], host["k"], host["v"], r=host["r"]),
              oracle.wkv4_backward_gated(host["w"], host["u"], host["k"], host["v"], host["r"], host["gy"])),
          "wkv4_train_step_gated_ckpt": lambda: (
              oracle.wkv4_forward_ex(host["w"], host["u"], host["k"], host["v"], r=host["r"]),
              oracle.wkv4_backward_gated(host["w"], host["u"], host["k"], host["v"], host["r"], host["gy"])),
          "wkv4_train_step_state": lambda: _state_step(host),
          "wkv4_train_step_state_ckpt": lambda: _state_step(host),
          "scan_real": lambda: oracle.scan_real(host["a"], host["b"]),
          "scan_complex": lambda: oracle.scan_complex(host["lam"], host["u"]),
          "scan_real_backward": lambda: oracle.scan_real_backward(host["a"], host["x"], host["gx"]),
          "scan_complex_backward": lambda: oracle.scan_complex_backward(host["lam"], host["x"], host["gx"]),
          "scan_mingru": lambda: oracle.scan_mingru(host["kz"], host["h"]),
          "scan_minlstm": lambda: oracle.scan_minlstm(host["kf"], host["ki"], host["h"]),
          "scan_real_decay": lambda: oracle.scan_real_decay(host["lam"], host["h"]),
          "scan_complex_normalized": lambda: oracle.scan_complex_normalized(host["lam"], host["u"]),
          "token_shift": lambda: oracle.token_shift(host["x"], host["mu"]),
          "token_shift_backward": lambda: oracle.token_shift_backward(host["x"], host["mu"], host["g"],
                                                                      want_gx_prev=False),
          "wkv4_forward_gated": lambda: oracle.wkv4_forward_ex(host["w"], host["u"], host["k"], host["v"],
                                                               r=host["r"]),
          "wkv4_backward_gated": lambda: oracle.wkv4_backward_gated(host["w"], host["u"], host["k"], host["v"],
                                                                    host["r"], host["gy"]),
          "scan_mingru_backward": lambda: oracle.scan_mingru_backward(host["kz"], host["h"], host["x"], host["gx"]),
          "scan_minlstm_backward": lambda: oracle.scan_minlstm_backward(host["kf"], host["ki"], host["h"], host["x"],
                                                                        host["gx"]),
          "scan_real_decay_backward": lambda: oracle.scan_real_decay_backward(host["lam"], host["x"], host["gx"]),
          "scan_complex_normalized_backward": lambda: oracle.scan_complex_normalized_backward(
              host["lam"], host["u"], host["x"], host["gx"])}[kind]
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= budget_s or len(times) >= 5000:
            break
    return statistics.median(times), len(times), oracle.num_threads()


def copy_probe():
    """Device-to-device copy of 1 GiB: attainable-bandwidth sanity figure (read + write)."""
    import torch

    n = 1 << 28
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    reps = 20
    for _ in range(reps):
        b.copy_(a)
    ev1.record()
    torch.cuda.synchronize()
    s = ev0.elapsed_time(ev1) / 1e3 / reps
    del a, b
    return round(2 * 4 * n / s / 1e9, 1)


def host_info():
    """The host the CPU baseline ran on: logical CPUs, the threads the process may use, the
    OpenMP setting and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"os_cpu_count": os.cpu_count(), "usable_cpus": usable,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "cpu_model": model}


def stream_ceiling(B, T, C, rotations, steps, warmup):
    """The same bytes as one wkv4_forward call moved by a plain elementwise kernel:
    y = k + v (torch.add) over the same rotated buffer sets, 8 B read and 4 B written per
    element, timed with HIP events on the launch stream like the forward.  It is the
    attainable streaming rate for this footprint and access pattern on the box."""
    import torch

    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    sets = []
    for _ in range(rotations):
        k = torch.randn((B, T, C), device=dev, generator=g)
        v = torch.randn((B, T, C), device=dev, generator=g)
        sets.append((k, v, torch.empty_like(k)))
    for i in range(warmup):
        k, v, y = sets[i % rotations]
        torch.add(k, v, out=y)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(steps):
        k, v, y = sets[(warmup + i) % rotations]
        torch.add(k, v, out=y)
    ev1.record(stream)
    torch.cuda.synchronize()
    s = ev0.elapsed_time(ev1) / 1e3 / steps
    del sets
    torch.cuda.empty_cache()
    gbps = 12 * B * T * C / s / 1e9
    return {"what": "torch.add(k, v, out=y), fp32 (B=%d, T=%d, C=%d), %d rotated buffer sets" % (B, T, C, rotations),
            "us_per_launch": round(s * 1e6, 3), "GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4)}


def summary(res):
    """The figures of one measured row for the headline line's per-workload block."""
    rf = res["roofline"]
    return {"kind": res["kind"], "workload": res["workload"], "B": res["B"], "T": res["T"], "C": res["C"],
            "steps": res["steps"], "us_per_launch": round(res["event_ms_per_step"] * 1e3, 2),
            "elements_per_s": res["elements_per_s"], "GBps": rf["achieved"], "frac": rf["frac"],
            "traffic": rf["traffic"], "algorithmic_bytes": rf["algorithmic_bytes"]}


def make_host(wid, kind, shape=None):
    """The seeded host inputs of one row: workload ``wid``'s generator at ``shape``."""
    from linear_recurrence_rnn_amd import workloads

    wl = workloads.WORKLOADS[wid]
    B, T, C = shape or (wl.B, wl.T, wl.C)
    if kind.startswith("token_shift"):
        host = workloads.make_token_shift(B, T, C, SHIFT_M, wl.seed, with_grad=kind.endswith("_backward"))
    elif kind in ("scan_mingru", "scan_minlstm", "scan_real_decay") or kind in VARIANT_BWD:
        host = workloads.make_gated(B, T, C, wl.seed, with_grad=kind in VARIANT_BWD)
        host["lam"] = (0.5 + 0.5 * np.abs(host["lam"])).astype(np.float32)
        if kind in VARIANT_BWD:
            host["x"] = host["h"]  # stand-in of the forward output's distribution (timing only)
    else:
        host = workloads.make_inputs(wid, shape=(B, T, C))
    if kind in ("wkv4_backward_gated", "wkv4_forward_gated") or kind.startswith("wkv4_train_step_gated"):
        host["r"] = host["v"]  # stand-in receptance ~ N(0,1) (timing only)
    if kind.startswith("wkv4_train_step_state"):
        # A carried state (a, b, p) and the gradient of the final state, seeded (timing only).
        rng = np.random.default_rng(wl.seed + 17)
        host["s_in"] = np.stack([rng.standard_normal((B, C)), rng.uniform(0.2, 3.0, (B, C)),
                                 rng.uniform(-5.0, 20.0, (B, C))], axis=-1).astype(np.float32)
        host["gs_out"] = rng.standard_normal((B, C, 2)).astype(np.float32)
    if kind.endswith("_backward") and kind.startswith("scan_") and kind not in VARIANT_BWD:
        host.update(workloads.make_scan_adjoint_inputs(wid, host))
    return host


def measure(lib, wid, kind, steps, warmup, cpu_budget, shape=None, cpu_slice=None, host=None, min_warm_s=0.0):
    from linear_recurrence_rnn_amd import workloads

    wl = workloads.WORKLOADS[wid]
    B, T, C = shape or (wl.B, wl.T, wl.C)
    if host is None:
        host = make_host(wid, kind, (B, T, C))
    elements = B * T * C
    label = wl.label
    variant_labels = {"scan_mingru": "minGRU from gate logits", "scan_minlstm": "minLSTM from gate logits",
                      "scan_real_decay": "real scan with one decay per channel",
                      "scan_complex_normalized": "LRU with normalised input"}
    base_kind = kind[:-len("_backward")] if kind.endswith("_backward") else kind
    if base_kind in variant_labels:
        label = variant_labels[base_kind] + (", backward" if kind.endswith("_backward") else "") + \
            " fp32 B=%d T=%d C=%d" % (B, T, C)
    if kind == "wkv4_backward_gated":
        label = "WKV-4 backward through the sigma(r) gate fp32 B=%d T=%d C=%d" % (B, T, C)
    if kind == "wkv4_forward_gated":
        label = "WKV-4 forward with the sigma(r) gate fp32 B=%d T=%d C=%d" % (B, T, C)
    if kind.startswith("wkv4_train_step"):
        label = "WKV-4 training step (%sforward, then backward%s%s) fp32 B=%d T=%d C=%d" % (
            "sigma(r)-gated " if "_gated" in kind else "",
            " from the forward's kept sums" if kind.endswith("_ckpt") else "",
            ", a piece with a carried state" if "_state" in kind else "", B, T, C)
    if kind.startswith("token_shift"):
        label = "RWKV token shift%s, %d mixes, fp32 B=%d T=%d C=%d" % (
            " backward" if kind.endswith("_backward") else "", SHIFT_M, B, T, C)
    footprint = BYTES_PER_ELEM[kind] * elements
    R = rotations_for(footprint)
    log("[bench] %s %s: B=%d T=%d C=%d, %d buffer set(s) of %.1f MB" % (
        kind, label, B, T, C, R, footprint / 1e6))
    row = Row(lib, kind, B, T, C, host, R)
    wall, ev_s = row.run(steps, warmup, min_warm_s)
    per_step = wall / steps
    per_launch = ev_s / steps
    out = {
        "kind": kind, "workload": label, "B": B, "T": T, "C": C, "rotations": R, "steps": steps,
        "ms_per_step": round(per_step * 1e3, 5), "event_ms_per_step": round(per_launch * 1e3, 5),
        "elements_per_s": elements / per_step,
        "roofline": roofline(kind, elements, per_launch, counter_traffic(kind, B, T, C)),
    }
    del row
    import torch
    torch.cuda.empty_cache()
    if cpu_budget > 0:
        sample = host
        desc = "full workload"
        if cpu_slice is not None:
            Ts = cpu_slice
            per_step = lambda k, v: hasattr(v, "ndim") and k not in ("s_in", "gs_out")  # noqa: E731
            sample = {k: (v[:, :Ts] if per_step(k, v) and v.ndim == 3 else
                          (v[:, :, :Ts] if per_step(k, v) and v.ndim == 4 else v)) for k, v in host.items()}
            desc = "first %d of %d time steps, all batch rows and channels" % (Ts, T)
        if kind in ("scan_real_backward", "scan_complex_backward"):
            # The adjoint's forward input: the oracle's own forward scan of the sample.
            import oracle
            sample = dict(sample)
            sample["x"] = (oracle.scan_real(sample["a"], sample["b"]).astype("float32") if "a" in sample
                           else oracle.scan_complex(sample["lam"], sample["u"]).astype("complex64"))
        med, reps, cores = cpu_baseline(kind, sample, cpu_budget)
        n_el = B * (cpu_slice or T) * C
        out["cpu_baseline"] = {"value": n_el / med, "unit": "elements/s", "cores": cores, "kind": "oracle",
                               "sample": "%s (%d elements), median of %d run(s)" % (desc, n_el, reps),
                               "host": host_info()}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="the headline's warm-up goes on (in batches of --warmup) for at least this long")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the oracle CPU baseline (0 skips it)")
    ap.add_argument("--no-copy-probe", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads' figures in the headline line")
    ap.add_argument("--all", action="store_true", help="also measure the other workloads")
    ap.add_argument("--all-out", default=None, help="write the --all rows to this JSON file")
    ap.add_argument("--only", default=None,
                    help="KIND@WORKLOAD[,...]: time only these rows (e.g. wkv4_backward@3), one JSON "
                         "line each, no headline line (for profiler runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        log("bench.py measures one GPU only: every box here has a single MI355X and this path "
            "has no multi-GPU mode (--gpus %d requested)." % args.gpus)
        sys.exit(2)

    import torch

    from linear_recurrence_rnn_amd import binding

    if not torch.cuda.is_available():
        log("bench.py needs a ROCm GPU")
        sys.exit(1)
    lib = binding.load()
    if args.only:
        for item in args.only.split(","):
            kind, wid = item.split("@")
            if kind not in BYTES_PER_ELEM:
                log("unknown row %r; rows: %s" % (kind, ", ".join(sorted(BYTES_PER_ELEM))))
                sys.exit(2)
            print(json.dumps(measure(lib, int(wid), kind, args.steps, args.warmup, 0)), flush=True)
        return
    res = measure(lib, 2, "wkv4_forward", args.steps, args.warmup, args.cpu_seconds, min_warm_s=args.warm_seconds)
    line = {
        "metric": METRIC,
        "value": res["elements_per_s"],
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded: k,v~N(0,1), u~N(0,0.5), w=exp(U(-3,1)))",
        "config": {"workload": "wkv4_forward B=8 T=1024 C=768 (169m-style width)", "B": 8, "T": 1024,
                   "C": 768, "buffer_sets": res["rotations"]},
        "hbm_GBps": res["roofline"]["achieved"],
        "pct_peak_hbm": round(100 * res["roofline"]["frac"], 2),
        "roofline": res["roofline"],
    }
    if "cpu_baseline" in res:
        line["cpu_baseline"] = res["cpu_baseline"]
    if not args.no_copy_probe:
        line["stream_ceiling"] = stream_ceiling(8, 1024, 768, res["rotations"], args.steps, args.warmup)
        # the headline's HIP-event time per launch against the ceiling's, both timed the same way
        line["stream_ceiling"]["headline_vs_ceiling"] = round(
            line["stream_ceiling"]["us_per_launch"] / (res["event_ms_per_step"] * 1e3), 4)
        line["copy_probe_GBps"] = copy_probe()
    if not args.no_workloads:
        # The other workloads, measured in the same run with a few launches each: the WKV
        # forward, backward and checkpointed training step at B=8 T=4096 C=2560, the real
        # scan and fused minGRU at B=64 T=4096 C=256 (the minGRU page's batch 64 x seq 4096)
        # and the LRU complex scan at B=1 T=262144 C=1024.
        # At least 10 warm-up launches and 0.1 s each (the GPU ramps its clocks after idling).
        extras = []
        h3 = make_host(3, "wkv4_backward")
        for kind in ("wkv4_forward", "wkv4_backward", "wkv4_train_step_ckpt"):
            extras.append(summary(measure(lib, 3, kind, 20, 10, 0, host=h3, min_warm_s=0.1)))
            log("[bench] " + json.dumps(extras[-1]))
        del h3
        for wid, kind, steps in ((4, "scan_real", 20), (4, "scan_mingru", 20), (5, "scan_complex", 10)):
            extras.append(summary(measure(lib, wid, kind, steps, 10, 0, min_warm_s=0.1)))
            log("[bench] " + json.dumps(extras[-1]))
        line["workloads"] = extras
    print(json.dumps(line), flush=True)

    if args.all:
        rows = [res]
        for wid, kind, steps, cpu_slice in ALL_ROWS:
            rows.append(measure(lib, wid, kind, steps, 10, min(args.cpu_seconds, 3.0), cpu_slice=cpu_slice,
                                min_warm_s=0.1))
            log("[bench] " + json.dumps(rows[-1]))
        if args.all_out:
            os.makedirs(os.path.dirname(os.path.abspath(args.all_out)), exist_ok=True)
            with open(args.all_out, "w") as f:
                json.dump(rows, f, indent=1)


if __name__ == "__main__":
    main()
