"""The full 70B-shaped linear stack resident on one GPU, with many delta sets.

"BitDelta: Serving 14 Zen Models from One GPU Cluster": [MF] gives the memory
arithmetic (a 70B bf16 base of 140 GB plus ~8.75 GB of packed signs per
variant, 14 variants) and [SA] the layout (one HBM-resident W_base read by
every entry of the delta cache).  On one MI355X (288 GB) the whole stack is
resident: 80 layers x {q, k, v, o, gate, up, down} = 68.45 G base weights
(136.9 GB) plus 14 x (8.556 GB of signs + 26.9 MB of alpha) = 257.1 GB.

This module only holds and drives the tensors: allocation, the per-matrix
compress of a variant (streamed: the caller supplies one fp32 W_ft at a time),
and passes of the fused linear through every matrix for one variant.  Every
call goes through the C ABI on the caller's stream; nothing allocates after
construction and reserve().  Filling the base weights and inputs is the
caller's job.
"""
from __future__ import annotations

import ctypes

from . import BD_ALPHA_MATRIX, BD_ALPHA_ROW, BD_F32, BD_BF16, check, lib

# (name, d_out, d_in) of one layer of the 70B-class model
LAYER_SHAPES = (("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
                ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672))


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


class LinearStack:
    """Base weights of n_layers layers and n_variants packed delta sets."""

    def __init__(self, n_layers: int = 80, n_variants: int = 14, shapes=LAYER_SHAPES, device=None,
                 per_matrix_alpha: bool = False):
        import torch

        self.torch = torch
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.n_layers = n_layers
        self.n_variants = n_variants
        self.shapes = tuple(shapes)
        self.mode = BD_ALPHA_MATRIX if per_matrix_alpha else BD_ALPHA_ROW
        self.base = {}
        self.signs = {}
        self.alpha = {}
        for l in range(n_layers):
            for name, d_out, d_in in self.shapes:
                self.base[l, name] = torch.empty((d_out, d_in), dtype=torch.bfloat16, device=self.device)
        for v in range(n_variants):
            for l in range(n_layers):
                for name, d_out, d_in in self.shapes:
                    self.signs[v, l, name] = torch.empty((d_out, d_in // 8), dtype=torch.uint8, device=self.device)
                    self.alpha[v, l, name] = torch.empty((1 if per_matrix_alpha else d_out,), dtype=torch.float32,
                                                         device=self.device)
        max_rows = max(d_out for _, d_out, _ in self.shapes)
        self._ws = torch.empty((lib.bitdelta_compress_workspace(max_rows, 8, BD_ALPHA_MATRIX),), dtype=torch.uint8,
                               device=self.device)
        self._lin_ws = torch.empty((1,), dtype=torch.uint8, device=self.device)

    def reserve(self, m: int) -> None:
        """Size the linear workspace (split partial sums) for inputs of up to m
        rows and for every decode width (1..16 rows)."""
        need = max(lib.bitdelta_linear_workspace(mm, d_out, d_in) for mm in (m, *range(1, 17))
                   for _, d_out, d_in in self.shapes)
        if need > self._lin_ws.numel():
            self._lin_ws = self.torch.empty((need,), dtype=self.torch.uint8, device=self.device)

    # ------------------------------------------------------------ bookkeeping
    def matrices(self):
        for l in range(self.n_layers):
            for name, d_out, d_in in self.shapes:
                yield l, name, d_out, d_in

    def params(self) -> int:
        return self.n_layers * sum(d_out * d_in for _, d_out, d_in in self.shapes)

    def resident_bytes(self) -> int:
        per_variant = sum(t.numel() * t.element_size() for (v, *_), t in self.signs.items() if v == 0) + \
            sum(t.numel() * t.element_size() for (v, *_), t in self.alpha.items() if v == 0)
        return self.params() * 2 + self.n_variants * per_variant

    def _stream(self, stream):
        s = stream if stream is not None else self.torch.cuda.current_stream(self.device)
        return ctypes.c_void_p(s.cuda_stream)

    # ------------------------------------------------------------------ calls
    def compress_into(self, v: int, l: int, name: str, w_ft, stream=None) -> None:
        """Compress one matrix of variant v from its fine-tuned weights w_ft
        (fp32 or bf16 [d_out, d_in] on the device) into the stack's signs/alpha."""
        torch = self.torch
        wb = self.base[l, name]
        d_out, d_in = wb.shape
        if tuple(w_ft.shape) != (d_out, d_in) or not w_ft.is_contiguous():
            raise ValueError("w_ft must be a contiguous tensor of the matrix's shape")
        ft = BD_F32 if w_ft.dtype == torch.float32 else BD_BF16
        nws = lib.bitdelta_compress_workspace(d_out, d_in, self.mode)
        check(lib.bitdelta_compress(_p(wb), _p(w_ft), ft, d_out, d_in, self.mode, _p(self.signs[v, l, name]),
                                    _p(self.alpha[v, l, name]), _p(self._ws) if nws else None, nws,
                                    self._stream(stream)))

    def compress_variant(self, v: int, make_w_ft, stream=None, on_matrix=None) -> None:
        """Compress every matrix of variant v.  make_w_ft(l, name, base) returns
        that matrix's fine-tuned weights; only one is alive at a time.
        on_matrix(l, name) runs after each compress is enqueued (timing hooks)."""
        for l, name, _, _ in self.matrices():
            w_ft = make_w_ft(l, name, self.base[l, name])
            self.compress_into(v, l, name, w_ft, stream)
            if on_matrix is not None:
                on_matrix(l, name)
            del w_ft

    def linear(self, v: int, l: int, name: str, x, y, stream=None) -> None:
        """y = x (W_base + alpha_v sign(Delta_v))^T for one matrix; x [m, d_in], y [m, d_out]."""
        wb = self.base[l, name]
        d_out, d_in = wb.shape
        m = x.shape[0]
        nws = lib.bitdelta_linear_workspace(m, d_out, d_in)
        if nws > self._lin_ws.numel():
            raise ValueError(f"call reserve({m}) before a linear with m={m}")
        check(lib.bitdelta_linear(_p(x), m, _p(wb), _p(self.signs[v, l, name]), _p(self.alpha[v, l, name]),
                                  self.mode, d_out, d_in, _p(y), _p(self._lin_ws), nws, self._stream(stream)))

    def forward(self, v: int, xs, ys, stream=None) -> None:
        """One pass through every linear of every layer for variant v.  Each
        linear reads its own input: xs[name] [m, d_in] and writes ys[name]
        [m, d_out] (the stack has no norms or activations, so inputs are not
        chained; see the design notes)."""
        for l, name, _, _ in self.matrices():
            self.linear(v, l, name, xs[name], ys[name], stream)

    def flops(self, m: int) -> float:
        return 2.0 * m * self.params()

    def linear_bytes(self, m: int) -> int:
        """Algorithmic bytes of one forward pass: W_base + signs + alpha + x + y per matrix."""
        total = 0
        for _, name, d_out, d_in in self.matrices():
            a = 4 if self.mode == BD_ALPHA_MATRIX else 4 * d_out
            total += d_out * d_in * 2 + d_out * d_in // 8 + a + 2 * m * d_in + 2 * m * d_out
        return total
