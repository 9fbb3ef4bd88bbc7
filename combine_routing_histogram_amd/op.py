"""EpDispatchCombineConfig / EpDispatchCombineOp: the MORI-EP method surface
(MORI "Communication APIs" page, MORI-EP section, methods table) on top of the
C ABI.  PyTorch provides device memory and the current HIP stream; every step
of dispatch and combine runs in the HIP kernels behind libepdc.so.

Receive buffers are allocated once per op at capacity (max_tokens * topk rows)
-- the analogue of MORI's pre-registered buffers -- and dispatch/combine
return views of them without synchronizing the host.  Rows
[rank_off[r], rank_off[r+1]) of every received tensor belong to virtual rank r;
only the first sum(recv_count) rows are written by a dispatch.
"""
from __future__ import annotations

import dataclasses
import enum
from typing import Optional, Tuple

import torch

from . import binding as B

QUANT = {"none": B.EPDC_QUANT_NONE, "fp8_e4m3_b128": B.EPDC_QUANT_FP8_E4M3_B128,
         "mxfp4_b32": B.EPDC_QUANT_MXFP4_B32}


class EpDispatchCombineKernelType(enum.IntEnum):
    """The kernel types of the MORI-EP section ("Communication APIs" page,
    kernel types table), kept with their values so that code written against
    that enum imports unchanged.  On one GPU the destination ranks are
    segments of one HBM buffer, which is the intra-node case; the others move
    data across nodes or through SDMA queues and are not built here."""
    IntraNode = 0
    InterNode = 1
    InterNodeV1 = 2
    InterNodeV1LL = 3
    AsyncLL = 4


@dataclasses.dataclass
class EpDispatchCombineConfig:
    max_tokens: int
    hidden: int
    topk: int
    num_experts: int
    num_ranks: int
    quant: str = "none"            # "none", "fp8_e4m3_b128", "mxfp4_b32"
    raw_row_bytes: int = 0         # > 0: dispatch carries opaque byte rows
    scale_row_bytes: int = 0       # bytes of a carried per-token scale row
    kernel_type: int = EpDispatchCombineKernelType.IntraNode

    def __post_init__(self):
        kt = EpDispatchCombineKernelType(self.kernel_type)   # ValueError for unknown values
        if kt != EpDispatchCombineKernelType.IntraNode:
            raise ValueError(f"kernel_type {kt.name} moves rows between nodes or through SDMA "
                             "queues; on one GPU only IntraNode (rank segments of one HBM "
                             "buffer) exists")
        if self.quant not in QUANT:
            raise ValueError(f"quant must be one of {sorted(QUANT)}")

    def to_c(self) -> B.epdc_config:
        kind = B.EPDC_IN_RAW if self.raw_row_bytes > 0 else B.EPDC_IN_BF16
        return B.make_config(self.max_tokens, self.hidden, self.topk, self.num_experts,
                             self.num_ranks, kind, QUANT[self.quant], self.raw_row_bytes,
                             self.scale_row_bytes)


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _raw_stream(device_index: int) -> int:
    """The current stream of the device as a raw handle."""
    return torch._C._cuda_getCurrentRawStream(device_index)


if not hasattr(torch._C, "_cuda_getCurrentRawStream"):  # older torch
    def _raw_stream(device_index: int) -> int:  # noqa: F811
        return torch.cuda.current_stream(device_index).cuda_stream


class EpDispatchCombineOp:
    def __init__(self, config: EpDispatchCombineConfig, device: Optional[torch.device] = None):
        self.config = config
        self.device = torch.device(device) if device is not None else torch.device(
            "cuda", torch.cuda.current_device())
        c = config.to_c()
        self._c = c
        ws_bytes = B.epdc_workspace_bytes(c)
        self.payload_row_bytes, self.scale_row_bytes = B.epdc_row_bytes(c)
        n_cap = config.max_tokens * config.topk
        self.n_cap = n_cap
        dev = self.device
        with torch.cuda.device(dev):
            self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            self._out = torch.empty((n_cap, self.payload_row_bytes), dtype=torch.uint8, device=dev)
            self._out_weights = torch.empty((n_cap, config.topk), dtype=torch.float32, device=dev)
            self._out_indices = torch.empty((n_cap, config.topk), dtype=torch.int32, device=dev)
            self._out_scales = (torch.empty((n_cap, self.scale_row_bytes), dtype=torch.uint8,
                                            device=dev) if self.scale_row_bytes else None)
            self._recv_count = torch.empty(config.num_ranks, dtype=torch.int32, device=dev)
            self._combined = torch.empty((config.max_tokens, config.hidden), dtype=torch.bfloat16,
                                         device=dev)
            self._combined_weights = torch.empty((config.max_tokens, config.topk),
                                                 dtype=torch.float32, device=dev)
            self._combine_in = None
            self._op = B.epdc_create(c, self.workspace.data_ptr(), ws_bytes)
        self._tokens = 0
        self._scales_dtype = None
        self._dev_index = self.device.index if self.device.index is not None else \
            torch.cuda.current_device()
        L = B.lib()
        self._f_dispatch, self._f_combine = L.epdc_dispatch, L.epdc_combine
        self._views = {}
        self._payload_v = self._payload_view(self._out)
        self._combined_cut = (-1, None)   # (T, (output view, weights view))
        self._side_stream = None
        self._sent_dispatch = None
        self._sent_combine = None
        self.u_cap = config.max_tokens * min(config.topk, config.num_ranks)
        self._last_dedup = False
        self._staging = None
        self._units = None          # unit-row buffers, allocated on first use
        self._unit_carried = (False, False)

    def __del__(self):
        op = getattr(self, "_op", None)
        if op:
            try:
                B.epdc_destroy(op)
            except Exception:
                pass
            self._op = None

    # ---- helpers -------------------------------------------------------------------
    # Host cost matters for small batches (a 128-token step is ~16 us of GPU
    # time): the stream is read as a raw handle, library functions and buffer
    # views are looked up once, and the argument checks use cheap accessors.
    def _stream(self) -> int:
        return _raw_stream(self._dev_index)

    def _need(self, t: torch.Tensor, name: str, dtype=None, shape=None):
        if t.get_device() != self._dev_index:
            raise ValueError(f"{name} is on {t.device}, op is on {self.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if shape is not None and t.shape != shape:
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")

    def _ws_view(self, ptr: int, count: int) -> torch.Tensor:
        off = ptr - self.workspace.data_ptr()
        return self.workspace[off:off + 4 * count].view(torch.int32)

    def _side(self) -> torch.cuda.Stream:
        # default priority: the send phases run here while the caller's stream computes
        if self._side_stream is None:
            self._side_stream = torch.cuda.Stream(device=self.device)
        return self._side_stream

    def _check_payload(self, input, weights, scales, T: int) -> None:
        cfg = self.config
        if cfg.raw_row_bytes:
            self._need(input, "input")
            if input.numel() * input.element_size() != T * cfg.raw_row_bytes:
                raise ValueError("input must hold raw_row_bytes per token")
        else:
            self._need(input, "input", torch.bfloat16, (T, cfg.hidden))
        if weights is not None:
            self._need(weights, "weights", torch.float32, (T, cfg.topk))
        if scales is not None:
            self._need(scales, "scales")
            if scales.numel() * scales.element_size() != T * cfg.scale_row_bytes:
                raise ValueError("scales must hold scale_row_bytes per token")
            self._scales_dtype = scales.dtype

    def _dispatch_ptrs(self, input, weights, scales):
        quant = self.config.quant != "none"
        return (_ptr(input), _ptr(weights), _ptr(scales), _ptr(self._out),
                _ptr(self._out_weights) if weights is not None else 0,
                _ptr(self._out_scales) if (scales is not None or quant) else 0)

    def _dispatch_views(self, weights, scales):
        return (self.received_payload(),
                self._out_weights if weights is not None else None,
                self.received_scales(scales is not None),
                self._out_indices, self._recv_count)

    # ---- methods table ---------------------------------------------------------------
    def dispatch(self, input: torch.Tensor, weights: Optional[torch.Tensor],
                 scales: Optional[torch.Tensor], indices: torch.Tensor):
        """Route tokens to expert slots.

        Returns (output, weights, scales, indices, recv_count) as views of the
        op's capacity-sized receive buffers (scales is None when there are
        none).  output is bf16 [N_cap, H] for bf16 input, float8_e4m3fn
        [N_cap, H] for FP8, uint8 [N_cap, H/2] (packed E2M1) for MXFP4, or
        uint8 [N_cap, raw_row_bytes] for raw rows.
        """
        T = indices.shape[0]
        self._need(indices, "indices", torch.int32, (T, self.config.topk))
        self._check_payload(input, weights, scales, T)
        i, w, s, o, ow, os_ = self._dispatch_ptrs(input, weights, scales)
        st = self._f_dispatch(self._op, _raw_stream(self._dev_index), T, i or None, w or None,
                              s or None, indices.data_ptr(), o, ow or None, os_ or None,
                              self._out_indices.data_ptr(), self._recv_count.data_ptr())
        if st:
            B._check(st)
        self._tokens = T
        self._last_dedup = False
        return self._dispatch_views(weights, scales)

    def dispatch_replay(self, input: torch.Tensor, weights: Optional[torch.Tensor] = None,
                        scales: Optional[torch.Tensor] = None):
        """Dispatch a new payload for the same tokens with the routing of the
        last dispatch (no histogram, scan or ranking).  Returns the views of
        dispatch(); indices and recv_count keep the recorded dispatch's values."""
        T = self._tokens
        units = self._last_dedup
        views = (lambda: self._unit_views(weights is not None, scales is not None)) if units \
            else (lambda: self._dispatch_views(weights, scales))
        if T == 0:
            # nothing to move; the library still refuses a replay with no dispatch recorded
            B.epdc_dispatch_replay(self._op, self._stream(), 0, 0, 0, 0, 0, 0)
            return views()
        self._check_payload(input, weights, scales, T)
        if units:  # a rank-deduplicated dispatch replays into the unit rows
            ub = self._unit_buffers()
            quant = self.config.quant != "none"
            i, w, s = _ptr(input), _ptr(weights), _ptr(scales)
            o = _ptr(ub["out"])
            ow = _ptr(ub["weights"]) if weights is not None else 0
            os_ = _ptr(ub["scales"]) if (scales is not None or quant) else 0
        else:
            i, w, s, o, ow, os_ = self._dispatch_ptrs(input, weights, scales)
        B.epdc_dispatch_replay(self._op, self._stream(), i, w, s, o, ow, os_)
        return views()

    def dispatch_send(self, input: torch.Tensor, weights: Optional[torch.Tensor],
                      scales: Optional[torch.Tensor], indices: torch.Tensor) -> None:
        """First phase of a split dispatch: enqueue the whole dispatch on the
        op's side stream (after the work already on the caller's stream) and
        return at once, so the caller's stream can compute meanwhile."""
        T = int(indices.shape[0])
        self._need(indices, "indices", torch.int32, (T, self.config.topk))
        self._check_payload(input, weights, scales, T)
        side = self._side()
        side.wait_stream(torch.cuda.current_stream(self.device))
        for t in (input, weights, scales, indices):
            if t is not None:
                t.record_stream(side)
        i, w, s, o, ow, os_ = self._dispatch_ptrs(input, weights, scales)
        B.epdc_dispatch_send(self._op, side.cuda_stream, T, i, w, s, _ptr(indices), o, ow, os_,
                             _ptr(self._out_indices), _ptr(self._recv_count))
        self._tokens = T
        self._last_dedup = False
        self._sent_dispatch = (weights is not None, scales is not None)

    def dispatch_recv(self):
        """Second phase: the caller's stream waits for the sent dispatch;
        returns what dispatch() returns."""
        if self._sent_dispatch is None:
            raise B.EpdcError(B.EPDC_ERR_BAD_STATE, "dispatch_recv without a dispatch_send")
        B.epdc_dispatch_recv(self._op, self._stream())
        has_w, has_s = self._sent_dispatch
        self._sent_dispatch = None
        return (self.received_payload(), self._out_weights if has_w else None,
                self.received_scales(has_s), self._out_indices, self._recv_count)

    def _payload_view(self, buf: torch.Tensor) -> torch.Tensor:
        cfg = self.config
        if cfg.raw_row_bytes:
            return buf
        if cfg.quant == "none":
            return self._view(buf, torch.bfloat16)
        if cfg.quant == "fp8_e4m3_b128":
            return self._view(buf, torch.float8_e4m3fn)
        return buf

    def _view(self, buf: torch.Tensor, dtype) -> torch.Tensor:
        """buf viewed as dtype; the op's buffers live as long as the op, so
        the views are made once."""
        key = (id(buf), dtype)
        v = self._views.get(key)
        if v is None:
            v = self._views[key] = buf.view(dtype)
        return v

    def _scales_view(self, buf: Optional[torch.Tensor], carried: bool) -> Optional[torch.Tensor]:
        cfg = self.config
        if cfg.quant == "fp8_e4m3_b128":
            return self._view(buf, torch.float32)
        if cfg.quant == "mxfp4_b32":
            return buf
        if not carried or buf is None:
            return None
        return self._view(buf, self._scales_dtype or torch.uint8)

    def received_payload(self) -> torch.Tensor:
        return self._payload_v

    def _combined_views(self, T: int):
        if self._combined_cut[0] != T:  # the views of the last token count are kept
            self._combined_cut = (T, (self._combined[:T], self._combined_weights[:T]))
        return self._combined_cut[1]

    def received_scales(self, carried: bool = True) -> Optional[torch.Tensor]:
        return self._scales_view(self._out_scales, carried)

    def combine(self, input: torch.Tensor, weights: Optional[torch.Tensor] = None,
                indices: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
        """Weighted gather of the expert outputs back to token order.

        input: bf16 [n, H] in the received layout with n >= T*K of the last
        dispatch (e.g. the dispatch output itself); weights: fp32 [n, K] in
        the received layout or None.  Returns (output bf16 [T, H], weights fp32 [T, K]).
        """
        self._check_combine(input, weights)
        st = self._f_combine(self._op, _raw_stream(self._dev_index), input.data_ptr(),
                             None if weights is None else weights.data_ptr(),
                             None if indices is None else indices.data_ptr(),
                             self._combined.data_ptr(), self._combined_weights.data_ptr())
        if st:
            B._check(st)
        return self._combined_views(self._tokens)

    def combine_scatter(self, input: torch.Tensor, weights: Optional[torch.Tensor] = None,
                        indices: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
        """Scatter combine: every received row pushes its weighted fp32 product
        to a per-(token, k) staging row, then each token adds its K staging
        rows in k order; same arguments and (bit-identical) result as combine().
        The fp32 staging rows (max_tokens*topk x hidden) are allocated on
        first use and kept."""
        self._check_combine(input, weights)
        if self._staging is None:
            self._staging = torch.empty((self.n_cap, self.config.hidden), dtype=torch.float32,
                                        device=self.device)
        B.epdc_combine_scatter(self._op, self._stream(), _ptr(input), _ptr(weights),
                               _ptr(indices), _ptr(self._staging), _ptr(self._combined),
                               _ptr(self._combined_weights))
        T = self._tokens
        return self._combined[:T], self._combined_weights[:T]

    def combine_send(self, input: torch.Tensor, weights: Optional[torch.Tensor] = None,
                     indices: Optional[torch.Tensor] = None) -> None:
        """First phase of a split combine, on the op's side stream (see dispatch_send)."""
        self._check_combine(input, weights)
        side = self._side()
        side.wait_stream(torch.cuda.current_stream(self.device))
        for t in (input, weights, indices):
            if t is not None:
                t.record_stream(side)
        B.epdc_combine_send(self._op, side.cuda_stream, _ptr(input), _ptr(weights), _ptr(indices),
                            _ptr(self._combined), _ptr(self._combined_weights))
        self._sent_combine = True

    def combine_recv(self) -> Tuple[torch.Tensor, torch.Tensor]:
        """Second phase: the caller's stream waits for the sent combine;
        returns what combine() returns."""
        if not self._sent_combine:
            raise B.EpdcError(B.EPDC_ERR_BAD_STATE, "combine_recv without a combine_send")
        B.epdc_combine_recv(self._op, self._stream())
        self._sent_combine = None
        T = self._tokens
        return self._combined[:T], self._combined_weights[:T]

    def _check_combine(self, input, weights) -> None:
        cfg = self.config
        self._need(input, "input", torch.bfloat16)
        if input.dim() != 2 or input.shape[1] != cfg.hidden:
            raise ValueError("combine input must be [rows, hidden] bf16")
        rows = self._tokens * cfg.topk          # received rows are a prefix of these
        if input.shape[0] < rows:
            raise ValueError(f"combine input needs at least {rows} rows")
        if weights is not None:
            self._need(weights, "weights", torch.float32)
            if weights.dim() != 2 or weights.shape[0] < rows or weights.shape[1] != cfg.topk:
                raise ValueError(f"combine weights must be [>= {rows}, topk] fp32")

    # ---- rank-deduplicated dispatch and the standard-MoE conversion -------------------
    def _unit_buffers(self) -> dict:
        if self._units is None:
            cfg, dev = self.config, self.device
            u = self.u_cap
            with torch.cuda.device(dev):
                self._units = {
                    "out": torch.empty((u, self.payload_row_bytes), dtype=torch.uint8, device=dev),
                    "weights": torch.empty((u, cfg.topk), dtype=torch.float32, device=dev),
                    "indices": torch.empty((u, cfg.topk), dtype=torch.int32, device=dev),
                    "scales": (torch.empty((u, self.scale_row_bytes), dtype=torch.uint8,
                                           device=dev) if self.scale_row_bytes else None),
                    "recv": torch.empty(cfg.num_ranks, dtype=torch.int32, device=dev),
                    "partial": torch.empty((u, cfg.hidden), dtype=torch.bfloat16, device=dev),
                }
        return self._units

    def received_unit_payload(self) -> torch.Tensor:
        """The unit rows of the last rank-deduplicated dispatch ([U_cap, ...])."""
        return self._payload_view(self._unit_buffers()["out"])

    def received_unit_scales(self, carried: bool = True) -> Optional[torch.Tensor]:
        return self._scales_view(self._unit_buffers()["scales"], carried)

    def _unit_views(self, has_w: bool, has_s: bool):
        ub = self._unit_buffers()
        return (self._payload_view(ub["out"]), ub["weights"] if has_w else None,
                self._scales_view(ub["scales"], has_s), ub["indices"], ub["recv"])

    def dispatch_dedup(self, input: torch.Tensor, weights: Optional[torch.Tensor],
                       scales: Optional[torch.Tensor], indices: torch.Tensor):
        """Dispatch with one received row per (token, destination rank).

        Returns (output, weights, scales, indices, recv_count) like dispatch()
        but over unit rows: views of [U_cap, ...] buffers, U_cap = max_tokens *
        min(topk, num_ranks); rank r owns rows [unit_off[r], unit_off[r+1])
        (get_unit_routing) and recv_count[r] of them."""
        T = int(indices.shape[0])
        self._need(indices, "indices", torch.int32, (T, self.config.topk))
        self._check_payload(input, weights, scales, T)
        ub = self._unit_buffers()
        quant = self.config.quant != "none"
        B.epdc_dispatch_dedup(self._op, self._stream(), T, _ptr(input), _ptr(weights),
                              _ptr(scales), _ptr(indices), _ptr(ub["out"]),
                              _ptr(ub["weights"]) if weights is not None else 0,
                              _ptr(ub["scales"]) if (scales is not None or quant) else 0,
                              _ptr(ub["indices"]), _ptr(ub["recv"]))
        self._tokens = T
        self._last_dedup = True
        self._unit_carried = (weights is not None, scales is not None)
        return self._unit_views(*self._unit_carried)

    def get_unit_routing(self):
        """(unit_off [R+1], unit_of [T*K], unit_src [U_cap]) of the last
        rank-deduplicated dispatch (only the first unit_off[R] of unit_src
        are meaningful)."""
        a, b, c = B.epdc_get_unit_routing(self._op)
        cfg = self.config
        return (self._ws_view(a, cfg.num_ranks + 1), self._ws_view(b, self._tokens * cfg.topk),
                self._ws_view(c, self.u_cap))

    def units_to_experts(self, input: Optional[torch.Tensor] = None,
                         weights: Optional[torch.Tensor] = None,
                         scales: Optional[torch.Tensor] = None,
                         indices: Optional[torch.Tensor] = None):
        """Standard-MoE conversion: expand unit rows (by default the op's own,
        with whatever the last dispatch_dedup carried) into the expert-layout
        rows dispatch() would have written; returns dispatch()'s views."""
        if input is None:
            has_w, has_s = self._unit_carried
            ub = self._unit_buffers()
            input, indices = ub["out"], ub["indices"]
            weights = ub["weights"] if has_w else None
            scales = ub["scales"] if (has_s or self.config.quant != "none") else None
        self._check_unit_rows(input, weights, scales, indices)
        B.epdc_units_to_experts(self._op, self._stream(), _ptr(input), _ptr(weights),
                                _ptr(scales), _ptr(indices), _ptr(self._out),
                                _ptr(self._out_weights) if weights is not None else 0,
                                _ptr(self._out_scales) if scales is not None else 0,
                                _ptr(self._out_indices) if indices is not None else 0)
        return (self.received_payload(), self._out_weights if weights is not None else None,
                self.received_scales(scales is not None), self._out_indices, None)

    def _check_unit_rows(self, input, weights, scales, indices) -> None:
        """The conversion reads up to T * min(K, R) unit rows of each given
        array (T of the last dispatch): check rows, row widths and dtypes on
        the host so that no undersized tensor reaches the kernel."""
        cfg = self.config
        rows = self._tokens * min(cfg.topk, cfg.num_ranks)
        for t, name, row_bytes, dtype in ((input, "input", self.payload_row_bytes, None),
                                          (weights, "weights", 4 * cfg.topk, torch.float32),
                                          (scales, "scales", self.scale_row_bytes, None),
                                          (indices, "indices", 4 * cfg.topk, torch.int32)):
            if t is None:
                continue
            self._need(t, name, dtype)
            if t.dim() < 1 or t.shape[0] < rows:
                raise ValueError(f"{name} needs at least {rows} unit rows, got "
                                 f"{tuple(t.shape)}")
            if t.shape[0] and (t.numel() // t.shape[0]) * t.element_size() != row_bytes:
                raise ValueError(f"{name} rows must be {row_bytes} bytes, got "
                                 f"{(t.numel() // t.shape[0]) * t.element_size()}")

    def experts_to_units(self, input: torch.Tensor,
                         weights: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Weighted sum of each unit's expert rows (bf16 [>= T*K, H] in the
        expert layout, fp32 weights [>= T*K, K] or None) into bf16 unit rows
        [U_cap, H] (an op-owned buffer)."""
        self._check_combine(input, weights)
        part = self._unit_buffers()["partial"]
        B.epdc_experts_to_units(self._op, self._stream(), _ptr(input), _ptr(weights), _ptr(part))
        return part

    def combine_units(self, input: Optional[torch.Tensor] = None,
                      weights: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
        """Sum each token's unit rows (by default the last experts_to_units
        result); weights: the unit rows' fp32 [U_cap, K] weights to hand back
        per token, or None.  Returns (output bf16 [T, H], weights fp32 [T, K])."""
        cfg = self.config
        ub = self._unit_buffers()
        if input is None:
            input = ub["partial"]
        self._need(input, "input", torch.bfloat16)
        if input.dim() != 2 or input.shape[1] != cfg.hidden or input.shape[0] < self.u_cap:
            raise ValueError(f"unit rows must be bf16 [>= {self.u_cap}, {cfg.hidden}]")
        if weights is not None:
            self._need(weights, "weights", torch.float32)
            if weights.dim() != 2 or weights.shape[0] < self.u_cap or weights.shape[1] != cfg.topk:
                raise ValueError(f"unit weights must be fp32 [>= {self.u_cap}, {cfg.topk}]")
        B.epdc_combine_units(self._op, self._stream(), _ptr(input), _ptr(weights),
                             _ptr(self._combined), _ptr(self._combined_weights))
        T = self._tokens
        return self._combined[:T], self._combined_weights[:T]

    def reset(self) -> None:
        B.epdc_reset(self._op)
        self._tokens = 0
        self._last_dedup = False
        self._sent_dispatch = self._sent_combine = None

    def get_dispatch_src_token_pos(self) -> torch.Tensor:
        """Per received row, the pair index t*K + k it came from (the first
        sum(recv_count) entries are meaningful)."""
        ptr, n = B.epdc_get_dispatch_src_token_pos(self._op)
        return self._ws_view(ptr, n)

    def get_routing(self):
        """(expert_off [E+1], rank_off [R+1], slot_of [T*K]) of the last dispatch."""
        a, b, c = B.epdc_get_routing(self._op)
        cfg = self.config
        return (self._ws_view(a, cfg.num_experts + 1), self._ws_view(b, cfg.num_ranks + 1),
                self._ws_view(c, self._tokens * cfg.topk))

    def get_offsets(self):
        """(expert_off [E+1], rank_off [R+1]) of the last dispatch."""
        a, b = B.epdc_get_offsets(self._op)
        cfg = self.config
        return self._ws_view(a, cfg.num_experts + 1), self._ws_view(b, cfg.num_ranks + 1)

    def set_debug(self, check_indices: bool = True) -> None:
        """With check_indices, combine checks a given `indices` against the
        recorded routing and raises bit 4 of the device error flag on a mismatch."""
        B.epdc_set_debug(self._op, B.EPDC_DEBUG_CHECK_INDICES if check_indices else 0)

    def set_combine_hint(self, recent_input: bool) -> None:
        """Say whether combine's input rows were written just before it (the
        expert output, or the dispatch output itself); only how the combine
        launches and stores depends on it (epdc_set_combine_hint), never its
        result."""
        B.epdc_set_combine_hint(self._op, B.EPDC_COMBINE_INPUT_RECENT if recent_input
                                else B.EPDC_COMBINE_INPUT_COLD)

    def get_registered_combine_input_buffer(self, dtype=torch.bfloat16) -> torch.Tensor:
        """A capacity-sized [N_cap, H] buffer owned by the op, for expert outputs."""
        if dtype != torch.bfloat16:
            raise ValueError("combine input is bf16")
        if self._combine_in is None:
            self._combine_in = torch.empty((self.n_cap, self.config.hidden), dtype=torch.bfloat16,
                                           device=self.device)
        return self._combine_in

    def device_error(self) -> int:
        """Synchronize and return/clear the sticky bad-expert-id flag."""
        return B.epdc_get_device_error(self._op, self._stream())

    # ---- timing ------------------------------------------------------------------------
    def profile_begin(self, max_launches: int) -> None:
        B.epdc_profile_begin(self._op, max_launches)

    def profile_end(self):
        """{kernel name: (total ms, launches)} for the launches since profile_begin."""
        ms, n = B.epdc_profile_end(self._op)
        return {B.epdc_kernel_name(k): (ms[k], n[k]) for k in range(B.EPDC_NUM_KERNELS) if n[k]}
