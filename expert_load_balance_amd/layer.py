"""Buffers and call sequence for one MoE layer forward on the GPU.

Plumbing only: torch allocates the device buffers once per shape (static
shapes: nothing here depends on the routing), and ``forward`` calls the C
entry points in the layer's order on one stream. No arithmetic happens in
Python.
"""
from __future__ import annotations

import torch

from . import (MOE_BF16, Shape, moe_combine, moe_count_plan, moe_gemm_down, moe_gemm_gateup,
               moe_gemm_schedule, moe_grouped_gemm_slots, moe_grouped_gemm_train, moe_permute,
               moe_plan, moe_plan_layout, moe_prefetch_replicas, moe_route, moe_workspace_bytes)

STAGES = ("route", "count_plan", "permute", "gemm_schedule", "gemm_gateup", "gemm_down",
          "shared", "combine")


def alloc(shape, dtype, device):
    """torch.empty that never hands out a null pointer (empty shapes keep a
    one-element allocation behind a zero-length view)."""
    n = 1
    for d in shape:
        n *= d
    return torch.empty(max(n, 1), dtype=dtype, device=device)[:n].view(shape)


class MoeLayerBuffers:
    """Every buffer of one layer call, sized by the shape alone.

    shared_F: width of an always-on shared expert (None: no shared expert).
    """

    def __init__(self, shape: Shape, device="cuda", shared_F: int | None = None):
        self.shape = shape
        T, H, E, k, R = shape.T, shape.H, shape.E, shape.k, shape.R
        N = T * k
        act = torch.bfloat16 if shape.dtype == MOE_BF16 else torch.float32
        i32 = torch.int32
        self.ids = alloc((T, k), i32, device)
        self.w = alloc((T, k), torch.float32, device)
        self.err = torch.zeros(1, dtype=i32, device=device)
        self.counts = alloc((E,), i32, device)
        self.offsets = alloc((E + 1,), i32, device)
        self.eidx = alloc((N,), i32, device)
        self.rank_load = alloc((R,), i32, device)
        self.plan = alloc((moe_plan_layout(shape)["total"],), i32, device)
        self.buf = alloc((N, H), act, device)
        self.dest_row = alloc((T, k), i32, device)
        self.row_src = alloc((N,), i32, device)
        self.y = alloc((N, H), act, device)
        self.out = alloc((T, H), act, device)
        self.ws = torch.empty(max(moe_workspace_bytes(shape), 256), dtype=torch.uint8, device=device)
        self.shared_shape = None
        if shared_F is not None:
            # one expert, one rank, k = 1: the plan is a single piece of T rows
            self.shared_shape = Shape(T, H, 1, 1, shared_F, 1, 0, shape.dtype)
            self.shared_counts = torch.full((1,), T, dtype=i32, device=device)
            self.shared_plan = alloc((moe_plan_layout(self.shared_shape)["total"],), i32, device)
            self.shared_ws = torch.empty(max(moe_workspace_bytes(self.shared_shape), 256),
                                         dtype=torch.uint8, device=device)
            self.shared_y = alloc((T, H), act, device)
            moe_plan(self.shared_shape, self.shared_counts, self.shared_plan)

    def forward(self, logits, bias, x, w_gate, w_up, w_down, shared_w=None, stream=None,
                marks=None, pool=None, gu=None):
        """Route -> count + plan (one launch up to 16384 assignments) -> permute ->
        grouped GEMM -> (shared) -> combine.

        marks: optional dict stage -> (start_event, end_event) recorded around
        each stage on the stream ("gemm" spans the routed grouped GEMM's three
        calls: schedule, gate/up, down). pool: a device buffer of
        moe_pool_bytes(shape) bytes; with it the planned replicas are
        prefetched into their slots after the plan and the grouped GEMM runs
        by plan segment, reading them (stages "prefetch" and "gemm_slots").
        gu: a bf16 [N, 2F] buffer; with it the grouped GEMM also keeps g | u
        for the backward (stage "gemm_train"). Returns self.out."""
        s = self.shape
        st = stream if stream is not None else torch.cuda.current_stream()

        def mark(name, i):
            if marks is not None and name in marks:
                marks[name][i].record(st)

        self.err.zero_()
        mark("route", 0)
        moe_route(s, logits, bias, self.ids, self.w, self.err, st)
        mark("route", 1)
        mark("count_plan", 0)
        moe_count_plan(s, self.ids, self.counts, self.offsets, self.eidx, self.rank_load, self.err,
                       self.ws, self.plan, st)
        mark("count_plan", 1)
        if pool is not None:
            mark("prefetch", 0)
            moe_prefetch_replicas(s, self.plan, w_gate, w_up, w_down, pool, st)
            mark("prefetch", 1)
        mark("permute", 0)
        moe_permute(s, x, self.ids, self.eidx, self.plan, self.buf, self.dest_row, self.row_src, st)
        mark("permute", 1)
        if gu is not None:
            mark("gemm_train", 0)
            moe_grouped_gemm_train(s, self.buf, self.plan, w_gate, w_up, w_down, self.y, gu,
                                   self.ws, st)
            mark("gemm_train", 1)
        elif pool is not None:
            mark("gemm_slots", 0)
            moe_grouped_gemm_slots(s, self.buf, self.plan, w_gate, w_up, w_down, pool, self.y,
                                   self.ws, st)
            mark("gemm_slots", 1)
        else:
            mark("gemm", 0)
            mark("gemm_schedule", 0)
            moe_gemm_schedule(s, self.plan, self.ws, st)
            mark("gemm_schedule", 1)
            mark("gemm_gateup", 0)
            moe_gemm_gateup(s, self.buf, self.plan, w_gate, w_up, self.ws, st)
            mark("gemm_gateup", 1)
            mark("gemm_down", 0)
            moe_gemm_down(s, self.plan, w_down, self.y, self.ws, st)
            mark("gemm_down", 1)
            mark("gemm", 1)
        shared_y = None
        if self.shared_shape is not None and shared_w is not None:
            mark("shared", 0)
            sg, su, sd = shared_w
            moe_gemm_schedule(self.shared_shape, self.shared_plan, self.shared_ws, st)
            moe_gemm_gateup(self.shared_shape, x, self.shared_plan, sg, su, self.shared_ws, st)
            moe_gemm_down(self.shared_shape, self.shared_plan, sd, self.shared_y, self.shared_ws, st)
            mark("shared", 1)
            shared_y = self.shared_y
        mark("combine", 0)
        moe_combine(s, self.y, self.dest_row, self.w, shared_y, self.out, st)
        mark("combine", 1)
        return self.out
