"""One INT8 W8A8 linear layer in quantized training, as a sequence of C-ABI calls.

State (mini_trainer guide: INT8 direction with a float magnitude per output
row, no float master weight; OneTrainer PR #1681: the weight lives in the
rotated basis): qw [N,K] int8, sw [N] fp32, optional float bias, and the
saved INT8 input (qx, sx) of the last forward.  Buffers for up to
``max_tokens`` rows are allocated once, so the steps allocate nothing.

Step order of one training step:
  forward   qlin_quantize_rows(x, rotate)          -> qx, sx   (saved)
            qlin_product_ws(FWD: qx, sx, qw, sw, bias)          -> y
  backward  qlin_quantize_grad(dY, sw, sx)         -> qg1, sg1 (rows of dY*sw),
                                                      qg2, sg2 (columns of dY*sx), db
            qlin_product_ws(DX: qg1, sg1, qw, rotate back)      -> dx
            qlin_product_ws(DW: qg2, sg2, qx)                   -> dw
  update    qlin_sgd_requant(qw, sw, dw, lr, seed, step, bias, db)

The products go through the workspace entry point (the same kernels as
qlin_fwd / qlin_bwd_dx / qlin_bwd_dw): its workspace, zero-filled once and
shared by the three calls, lets each product split the tiles of its last
partial round along the contraction, and takes contractions past the int32
bound.
"""
import torch

from . import _native as nat


class LinearW8A8Training:
    def __init__(self, weight, bias=None, had_block=128, max_tokens=0, weight_norm=False):
        """weight: [N, K] float GPU tensor in the original basis (rotated here).

        weight_norm: row weight normalization (the guide's INT8 direction with a
        floating magnitude per output row, trained as its own parameter): the
        represented weight is g q / ||q||, the direction s q (s in self.s),
        and the products take the column scale sw = g / ||q||.  It starts as
        the absmax weight.  Updates go through wn_sgd_step."""
        self.timer = None    # optional callable(label) invoked after each call
        N, K = weight.shape
        self.N, self.K, self.had = N, K, int(had_block)
        dev = weight.device
        w = weight.to(torch.float32).contiguous()
        self.qw, self.sw = nat.qlin_quantize_rows(w, had_block=self.had)
        if bool((self.sw == 0).any()):
            raise ValueError("weight has an all-zero row (zero direction)")
        self.weight_norm = bool(weight_norm)
        if self.weight_norm:
            self.s = self.sw
            self.g, self.sw = nat.qlin_wn_init(self.qw, self.s)
        self.bias = None if bias is None else bias.to(torch.float32).contiguous().clone()
        self.max_tokens = 0
        self.dw = torch.empty((N, K), dtype=torch.float32, device=dev)
        self.db = None if bias is None else torch.empty(N, dtype=torch.float32, device=dev)
        self._ws = torch.zeros(0, dtype=torch.uint8, device=dev)
        self._ws_for = set()
        self._alloc(max_tokens, dev)

    def _workspace(self, M):
        """The shared product workspace, grown (zero-filled) to what the three
        products need at M tokens."""
        if M not in self._ws_for:
            need = max(nat.qlin_product_ws_bytes(op, M, self.N, self.K)
                       for op in (nat.QLIN_OP_FWD, nat.QLIN_OP_DX, nat.QLIN_OP_DW))
            if need > self._ws.numel():
                self._ws = torch.zeros(need, dtype=torch.uint8, device=self._ws.device)
            self._ws_for.add(M)
        return self._ws

    def _alloc(self, M, dev):
        if M <= self.max_tokens:
            return
        N, K = self.N, self.K
        self.max_tokens = M
        self._qx = torch.empty((M, K), dtype=torch.int8, device=dev)
        self._sx = torch.empty(M, dtype=torch.float32, device=dev)
        self._y = torch.empty((M, N), dtype=torch.float32, device=dev)
        self._qg1 = torch.empty((M, N), dtype=torch.int8, device=dev)
        self._sg1 = torch.empty(M, dtype=torch.float32, device=dev)
        self._qg2 = torch.empty((M, N), dtype=torch.int8, device=dev)
        self._sg2 = torch.empty(N, dtype=torch.float32, device=dev)
        self._dx = torch.empty((M, K), dtype=torch.float32, device=dev)

    def forward(self, x):
        M = x.shape[0]
        self._alloc(M, x.device)
        self.M = M
        self.qx, self.sx = nat.qlin_quantize_rows(x, had_block=self.had, q=self._qx[:M],
                                                  s=self._sx[:M])
        self._tick("quantize_x")
        y = nat.qlin_product_ws(nat.QLIN_OP_FWD, self.qx, self.sx, self.qw, M, self.N, self.K,
                                scol=self.sw, bias=self.bias, out=self._y[:M],
                                workspace=self._workspace(M))
        self._tick("fwd")
        return y

    def backward(self, dy):
        """Returns dx in the original basis; keeps dw (and db) for the update."""
        M = self.M
        qg1, sg1, qg2, sg2, _ = nat.qlin_quantize_grad(
            dy, self.sw, self.sx, q1=self._qg1[:M], s1=self._sg1[:M], q2=self._qg2[:M],
            s2=self._sg2, col_sum=self.db)
        self._tick("quantize_dy")
        ws = self._workspace(M)
        dx = nat.qlin_product_ws(nat.QLIN_OP_DX, qg1, sg1, self.qw, M, self.N, self.K,
                                 had_block=self.had, out=self._dx[:M], workspace=ws)
        self._tick("bwd_dx")
        nat.qlin_product_ws(nat.QLIN_OP_DW, qg2, sg2, self.qx, M, self.N, self.K, out=self.dw,
                            workspace=ws)
        self._tick("bwd_dw")
        return dx

    def sgd_step(self, lr, seed, step):
        if self.weight_norm:
            return self.wn_sgd_step(lr, seed, step)
        nat.qlin_sgd_requant(self.qw, self.sw, self.dw, lr, seed, step, bias=self.bias, db=self.db)
        self._tick("sgd_requant")

    def wn_sgd_step(self, lr, seed, step):
        """SGD on the magnitude g and the direction s q of a weight-normalized
        layer, with the direction's stochastic requant; refreshes sw."""
        if not self.weight_norm:
            raise ValueError("the layer was not built with weight_norm=True")
        nat.qlin_wn_sgd_requant(self.qw, self.s, self.g, self.sw, self.dw, lr, seed, step,
                                bias=self.bias, db=self.db)
        self._tick("wn_sgd_requant")

    def adamw_step(self, lr, seed, step, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0):
        """AdamW update + stochastic requant (step >= 1).  The fp32 moments (and
        the bias moments) are allocated, zeroed, on the first call."""
        if self.weight_norm:
            raise ValueError("AdamW is built for the absmax weight only")
        if getattr(self, "_m", None) is None:
            self._m = torch.zeros_like(self.dw)
            self._v = torch.zeros_like(self.dw)
            if self.bias is not None:
                self._bm = torch.zeros_like(self.bias)
                self._bv = torch.zeros_like(self.bias)
        has_b = self.bias is not None
        nat.qlin_adamw_requant(self.qw, self.sw, self.dw, self._m, self._v, lr, betas[0],
                               betas[1], eps, weight_decay, seed, step,
                               bias=self.bias, db=self.db if has_b else None,
                               bias_m=self._bm if has_b else None,
                               bias_v=self._bv if has_b else None)
        self._tick("adamw_requant")

    def unquantized_weight(self):
        """The represented weight fl(s_w * Q_w) (with weight normalization
        sw = g / ||q||), rotated back to the original basis (a new [N, K] fp32
        tensor)."""
        return nat.qlin_dequantize_weight(self.qw, self.sw, had_block=self.had)

    def _tick(self, label):
        if self.timer is not None:
            self.timer(label)
