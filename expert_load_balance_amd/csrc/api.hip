// api.hip -- the extern "C" entry points of libmoe.so: validate on the host,
// then launch on the caller's stream. Nothing here allocates device memory.
// Operation semantics and their sources are documented in include/moe.h.
#include <math.h>
#include <string.h>

#include "common.h"

namespace {

moe_status_t check(const moe_shape_t* s)
{
    if (!s) return MOE_EINVAL;
    if (s->T < 0 || s->E < 1 || s->E > 256 || s->k < 1 || s->k > s->E || s->k > 64) return MOE_EINVAL;
    if (s->R < 1 || s->R > 64 || s->E % s->R != 0 || s->S < 0) return MOE_EINVAL;
    if (s->H < 1 || s->F < 1) return MOE_EINVAL;
    const int64_t N = (int64_t)s->T * s->k;
    if (N >= (int64_t(1) << 31)) return MOE_EINVAL;
    const int64_t wide = s->H > s->F ? s->H : s->F;
    if (N * wide >= (int64_t(1) << 40)) return MOE_EINVAL;
    if (s->dtype == MOE_BF16) {
        if (s->H % 64 || s->F % 64) return MOE_EUNSUPPORTED;
        // the GEMM addresses rows of the buffer, of one expert's weights and
        // of one 256-row tile of h with 32-bit byte offsets, all below the
        // out-of-range offset its padding rows take
        const int64_t lim = (int64_t(1) << 32) - 128;
        if (N * s->H * 2 >= lim || (int64_t)s->F * s->H * 2 >= lim || (int64_t)512 * s->F >= lim)
            return MOE_EUNSUPPORTED;
    } else if (s->dtype == MOE_F32) {
        if (s->H % 4 || s->F % 4) return MOE_EUNSUPPORTED;
    } else {
        return MOE_EINVAL;
    }
    return MOE_OK;
}

inline moe_status_t dev(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EDEVICE; }

// A pointer to a zero-length array may be NULL; any other NULL is an error.
inline bool bad(const void* p, int64_t n) { return p == nullptr && n > 0; }

inline hipStream_t as_stream(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* moe_status_str(moe_status_t status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or dtype";
    case MOE_EDEVICE: return "HIP runtime error";
    case MOE_EDATA: return "device error word set (non-finite logits or bad expert ids)";
    }
    return "unknown status";
}

moe_status_t moe_check_shape(const moe_shape_t* shape) { return check(shape); }

moe_status_t moe_plan_layout(const moe_shape_t* shape, moe_plan_layout_t* out)
{
    const moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    if (!out) return MOE_EINVAL;
    const moe::PlanLayout L = moe::plan_layout(shape->E, shape->R);
    out->quota = L.quota;
    out->win_off = L.win_off;
    out->seg_num = L.seg_num;
    out->seg_expert = L.seg_expert;
    out->seg_row = L.seg_row;
    out->seg_cnt = L.seg_cnt;
    out->slots_needed = L.slots_needed;
    out->slot_expert = L.slot_expert;
    out->donor = L.donor;
    out->piece_num = L.piece_num;
    out->piece_rank = L.piece_rank;
    out->piece_row = L.piece_row;
    out->piece_cnt = L.piece_cnt;
    out->total = L.total;
    return MOE_OK;
}

size_t moe_plan_bytes(const moe_shape_t* shape)
{
    if (check(shape) != MOE_OK) return 0;
    return (size_t)moe::plan_layout(shape->E, shape->R).total * sizeof(int32_t);
}

moe_status_t moe_plan_bind(const moe_shape_t* shape, void* block, moe_plan_t* out)
{
    const moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    if (!block || !out) return MOE_EINVAL;
    const moe::PlanLayout L = moe::plan_layout(shape->E, shape->R);
    int32_t* b = static_cast<int32_t*>(block);
    out->quota = b + L.quota;
    out->win_off = b + L.win_off;
    out->seg_expert = b + L.seg_expert;
    out->seg_row = b + L.seg_row;
    out->seg_cnt = b + L.seg_cnt;
    out->seg_num = b + L.seg_num;
    out->slot_expert = b + L.slot_expert;
    out->slots_needed = b + L.slots_needed;
    out->piece_rank = b + L.piece_rank;
    out->piece_row = b + L.piece_row;
    out->piece_cnt = b + L.piece_cnt;
    out->piece_num = b + L.piece_num;
    out->donor = b + L.donor;
    return MOE_OK;
}

size_t moe_workspace_bytes(const moe_shape_t* shape)
{
    if (check(shape) != MOE_OK) return 0;
    return moe::ws_layout(*shape).total;
}

moe_status_t moe_route(const moe_shape_t* shape, const float* d_logits, const float* d_bias,
                       int32_t* d_ids, float* d_w, int32_t* d_err, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t T = shape->T, N = T * shape->k;
    if (bad(d_logits, T) || bad(d_ids, N) || bad(d_w, N) || !d_err) return MOE_EINVAL;
    return dev(moe_launch_route(*shape, d_logits, d_bias, d_ids, d_w, d_err, as_stream(stream)));
}

moe_status_t moe_count(const moe_shape_t* shape, const int32_t* d_ids, int32_t* d_counts,
                       int32_t* d_offsets, int32_t* d_eidx, int32_t* d_rank_load, int32_t* d_err,
                       void* d_ws, size_t ws_bytes, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t N = (int64_t)shape->T * shape->k;
    if (bad(d_ids, N) || !d_counts || !d_offsets || bad(d_eidx, N) || !d_rank_load || !d_err ||
        !d_ws)
        return MOE_EINVAL;
    if (ws_bytes < moe::ws_layout(*shape).total) return MOE_EINVAL;
    return dev(moe_launch_count(*shape, d_ids, d_counts, d_offsets, d_eidx, d_rank_load, d_err,
                                static_cast<char*>(d_ws), as_stream(stream)));
}

moe_status_t moe_count_noalloc(const moe_shape_t* shape, const int32_t* d_ids, int32_t* d_counts,
                               int32_t* d_offsets, int32_t* d_eidx, int32_t* d_rank_load,
                               int32_t* d_err, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t N = (int64_t)shape->T * shape->k;
    if (bad(d_ids, N) || !d_counts || !d_offsets || bad(d_eidx, N) || !d_rank_load || !d_err)
        return MOE_EINVAL;
    if (2 * moe::count_table_bytes(N, shape->E) > moe::kCountScratchBytes) return MOE_EINVAL;
    return dev(moe_launch_count_noalloc(*shape, d_ids, d_counts, d_offsets, d_eidx, d_rank_load,
                                        d_err, as_stream(stream)));
}

moe_status_t moe_plan(const moe_shape_t* shape, const int32_t* d_counts, int32_t* d_plan,
                      moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    if (!d_counts || !d_plan) return MOE_EINVAL;
    return dev(moe_launch_plan(*shape, d_counts, d_plan, as_stream(stream)));
}

moe_status_t moe_count_plan(const moe_shape_t* shape, const int32_t* d_ids, int32_t* d_counts,
                            int32_t* d_offsets, int32_t* d_eidx, int32_t* d_rank_load,
                            int32_t* d_err, void* d_ws, size_t ws_bytes, int32_t* d_plan,
                            moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t N = (int64_t)shape->T * shape->k;
    if (bad(d_ids, N) || !d_counts || !d_offsets || bad(d_eidx, N) || !d_rank_load || !d_err ||
        !d_ws || !d_plan)
        return MOE_EINVAL;
    if (ws_bytes < moe::ws_layout(*shape).total) return MOE_EINVAL;
    return dev(moe_launch_count_plan(*shape, d_ids, d_counts, d_offsets, d_eidx, d_rank_load, d_err,
                                     static_cast<char*>(d_ws), d_plan, as_stream(stream)));
}

moe_status_t moe_permute(const moe_shape_t* shape, const void* d_x, const int32_t* d_ids,
                         const int32_t* d_eidx, const int32_t* d_plan, void* d_buf,
                         int32_t* d_dest_row, int32_t* d_row_src, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t T = shape->T, N = T * shape->k;
    if (bad(d_x, T) || bad(d_ids, N) || bad(d_eidx, N) || !d_plan || bad(d_buf, N) ||
        bad(d_dest_row, N) || bad(d_row_src, N))
        return MOE_EINVAL;
    return dev(moe_launch_permute(*shape, d_x, d_ids, d_eidx, d_plan, d_buf, d_dest_row,
                                  d_row_src, as_stream(stream)));
}

moe_status_t moe_gemm_schedule(const moe_shape_t* shape, const int32_t* d_plan, void* d_ws,
                               size_t ws_bytes, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    if (!d_plan || !d_ws) return MOE_EINVAL;
    if (ws_bytes < moe::ws_layout(*shape).total) return MOE_EINVAL;
    return dev(moe_launch_gemm_schedule(*shape, d_plan, static_cast<char*>(d_ws), as_stream(stream),
                                        moe::expert_groups(*shape)));
}

moe_status_t moe_gemm_gateup(const moe_shape_t* shape, const void* d_a, const int32_t* d_plan,
                             const void* d_w_gate, const void* d_w_up, void* d_ws,
                             size_t ws_bytes, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t N = (int64_t)shape->T * shape->k;
    if (bad(d_a, N) || !d_plan || !d_w_gate || !d_w_up || !d_ws) return MOE_EINVAL;
    if (ws_bytes < moe::ws_layout(*shape).total) return MOE_EINVAL;
    return dev(moe_launch_gemm_gateup(*shape, d_a, d_plan, d_w_gate, d_w_up,
                                      static_cast<char*>(d_ws), as_stream(stream),
                                      moe::expert_groups(*shape)));
}

moe_status_t moe_gemm_down(const moe_shape_t* shape, const int32_t* d_plan, const void* d_w_down,
                           void* d_y, void* d_ws, size_t ws_bytes, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t N = (int64_t)shape->T * shape->k;
    if (!d_plan || !d_w_down || bad(d_y, N) || !d_ws) return MOE_EINVAL;
    if (ws_bytes < moe::ws_layout(*shape).total) return MOE_EINVAL;
    return dev(moe_launch_gemm_down(*shape, d_plan, d_w_down, d_y, static_cast<char*>(d_ws),
                                    as_stream(stream), moe::expert_groups(*shape)));
}

moe_status_t moe_grouped_gemm(const moe_shape_t* shape, const void* d_a, const int32_t* d_plan,
                              const void* d_w_gate, const void* d_w_up, const void* d_w_down,
                              void* d_y, void* d_ws, size_t ws_bytes, moe_stream_t stream)
{
    moe_status_t st = moe_gemm_schedule(shape, d_plan, d_ws, ws_bytes, stream);
    if (st == MOE_OK)
        st = moe_gemm_gateup(shape, d_a, d_plan, d_w_gate, d_w_up, d_ws, ws_bytes, stream);
    if (st != MOE_OK) return st;
    return moe_gemm_down(shape, d_plan, d_w_down, d_y, d_ws, ws_bytes, stream);
}

size_t moe_pool_bytes(const moe_shape_t* shape)
{
    if (check(shape) != MOE_OK) return 0;
    return moe::pool_bytes(*shape);
}

moe_status_t moe_prefetch_replicas(const moe_shape_t* shape, const int32_t* d_plan,
                                   const void* d_w_gate, const void* d_w_up, const void* d_w_down,
                                   void* d_pool, size_t pool_bytes, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const size_t need = moe::pool_bytes(*shape);
    if (!d_plan || !d_w_gate || !d_w_up || !d_w_down || (need > 0 && !d_pool) ||
        pool_bytes < need)
        return MOE_EINVAL;
    return dev(moe_launch_prefetch(*shape, d_plan, d_w_gate, d_w_up, d_w_down, d_pool,
                                   as_stream(stream)));
}

moe_status_t moe_grouped_gemm_slots(const moe_shape_t* shape, const void* d_a,
                                    const int32_t* d_plan, const void* d_w_gate,
                                    const void* d_w_up, const void* d_w_down, const void* d_pool,
                                    size_t pool_bytes, void* d_y, void* d_ws, size_t ws_bytes,
                                    moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t N = (int64_t)shape->T * shape->k;
    const size_t need = moe::pool_bytes(*shape);
    if (bad(d_a, N) || !d_plan || !d_w_gate || !d_w_up || !d_w_down || bad(d_y, N) || !d_ws ||
        (need > 0 && !d_pool) || pool_bytes < need)
        return MOE_EINVAL;
    const moe::WsLayout W = moe::ws_layout(*shape);
    if (ws_bytes < W.total) return MOE_EINVAL;
    char* ws = static_cast<char*>(d_ws);
    hipStream_t hs = as_stream(stream);
    uint64_t* wtab = reinterpret_cast<uint64_t*>(ws + W.wtab);
    const moe::GemmGroups g{2 * shape->E, true, wtab};
    hipError_t e = moe_launch_slot_table(*shape, d_plan, d_w_gate, d_w_up, d_w_down, d_pool, wtab, hs);
    if (e == hipSuccess) e = moe_launch_gemm_schedule(*shape, d_plan, ws, hs, g);
    if (e == hipSuccess) e = moe_launch_gemm_gateup(*shape, d_a, d_plan, d_w_gate, d_w_up, ws, hs, g);
    if (e == hipSuccess) e = moe_launch_gemm_down(*shape, d_plan, d_w_down, d_y, ws, hs, g);
    return dev(e);
}

moe_status_t moe_grouped_gemm_train(const moe_shape_t* shape, const void* d_a,
                                    const int32_t* d_plan, const void* d_w_gate,
                                    const void* d_w_up, const void* d_w_down, void* d_y,
                                    void* d_gu, void* d_ws, size_t ws_bytes, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t N = (int64_t)shape->T * shape->k;
    if (bad(d_a, N) || !d_plan || !d_w_gate || !d_w_up || !d_w_down || bad(d_y, N) ||
        (shape->dtype == MOE_BF16 && bad(d_gu, N)) || !d_ws)
        return MOE_EINVAL;
    if (ws_bytes < moe::ws_layout(*shape).total) return MOE_EINVAL;
    char* ws = static_cast<char*>(d_ws);
    hipStream_t hs = as_stream(stream);
    const moe::GemmGroups g = moe::expert_groups(*shape);
    hipError_t e = moe_launch_gemm_schedule(*shape, d_plan, ws, hs, g);
    if (e == hipSuccess)
        e = moe_launch_gemm_gateup(*shape, d_a, d_plan, d_w_gate, d_w_up, ws, hs, g,
                                   shape->dtype == MOE_BF16 ? d_gu : nullptr);
    if (e == hipSuccess) e = moe_launch_gemm_down(*shape, d_plan, d_w_down, d_y, ws, hs, g);
    return dev(e);
}

moe_status_t moe_combine(const moe_shape_t* shape, const void* d_y, const int32_t* d_dest_row,
                         const float* d_w, const void* d_shared_y, void* d_out,
                         moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t T = shape->T, N = T * shape->k;
    if (bad(d_y, N) || bad(d_dest_row, N) || bad(d_w, N) || bad(d_out, T)) return MOE_EINVAL;
    return dev(moe_launch_combine(*shape, d_y, d_dest_row, d_w, d_shared_y, d_out,
                                  as_stream(stream)));
}

size_t moe_backward_workspace_bytes(const moe_shape_t* shape)
{
    if (check(shape) != MOE_OK) return 0;
    return moe::bwd_ws_layout(*shape).total;
}

moe_status_t moe_combine_backward(const moe_shape_t* shape, const void* d_dout, const void* d_y,
                                  const int32_t* d_dest_row, const float* d_w, void* d_dy,
                                  float* d_dw, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t T = shape->T, N = T * shape->k;
    if (bad(d_dout, T) || bad(d_y, N) || bad(d_dest_row, N) || bad(d_w, N) || bad(d_dy, N) ||
        bad(d_dw, N))
        return MOE_EINVAL;
    return dev(moe_launch_combine_backward(*shape, d_dout, d_y, d_dest_row, d_w, d_dy, d_dw,
                                           as_stream(stream)));
}

moe_status_t moe_ffn_backward(const moe_shape_t* shape, const void* d_buf, const int32_t* d_plan,
                              const void* d_w_gate, const void* d_w_up, const void* d_w_down,
                              const void* d_gu, const void* d_dy, void* d_dbuf, float* d_dw_gate,
                              float* d_dw_up, float* d_dw_down, void* d_ws, size_t ws_bytes,
                              moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t N = (int64_t)shape->T * shape->k;
    if (bad(d_buf, N) || !d_plan || !d_w_gate || !d_w_up || !d_w_down || bad(d_dy, N) ||
        bad(d_dbuf, N) || !d_dw_gate || !d_dw_up || !d_dw_down || !d_ws)
        return MOE_EINVAL;
    if (ws_bytes < moe::bwd_ws_layout(*shape).total) return MOE_EINVAL;
    // fp32 always recomputes (the saved g | u are a bf16 training forward's)
    const void* gu = shape->dtype == MOE_BF16 ? d_gu : nullptr;
    return dev(moe_launch_ffn_backward(*shape, d_buf, d_plan, d_w_gate, d_w_up, d_w_down, gu, d_dy,
                                       d_dbuf, d_dw_gate, d_dw_up, d_dw_down,
                                       static_cast<char*>(d_ws), as_stream(stream)));
}

size_t moe_replica_grad_bytes(const moe_shape_t* shape)
{
    if (check(shape) != MOE_OK) return 0;
    return moe::replica_grad_bytes(*shape);
}

moe_status_t moe_ffn_backward_replicas(const moe_shape_t* shape, const void* d_buf,
                                       const int32_t* d_plan, const void* d_w_gate,
                                       const void* d_w_up, const void* d_w_down, const void* d_gu,
                                       const void* d_dy, void* d_dbuf, float* d_dw_gate,
                                       float* d_dw_up, float* d_dw_down, float* d_rgrad,
                                       size_t rgrad_bytes, void* d_ws, size_t ws_bytes,
                                       moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    if (shape->dtype != MOE_BF16) return MOE_EUNSUPPORTED;
    const int64_t N = (int64_t)shape->T * shape->k;
    if (bad(d_buf, N) || !d_plan || !d_w_gate || !d_w_up || !d_w_down || bad(d_dy, N) ||
        bad(d_dbuf, N) || !d_dw_gate || !d_dw_up || !d_dw_down || !d_rgrad || !d_ws)
        return MOE_EINVAL;
    if (rgrad_bytes < moe::replica_grad_bytes(*shape)) return MOE_EINVAL;
    if (ws_bytes < moe::bwd_ws_layout(*shape).total) return MOE_EINVAL;
    return dev(moe_launch_ffn_backward(*shape, d_buf, d_plan, d_w_gate, d_w_up, d_w_down, d_gu,
                                       d_dy, d_dbuf, d_dw_gate, d_dw_up, d_dw_down,
                                       static_cast<char*>(d_ws), as_stream(stream), d_rgrad));
}

moe_status_t moe_permute_backward(const moe_shape_t* shape, const void* d_dbuf,
                                  const int32_t* d_dest_row, void* d_dx, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t T = shape->T, N = T * shape->k;
    if (bad(d_dbuf, N) || bad(d_dest_row, N) || bad(d_dx, T)) return MOE_EINVAL;
    return dev(moe_launch_combine_rows(*shape, N, d_dbuf, d_dest_row, nullptr, nullptr, d_dx,
                                       as_stream(stream)));
}

moe_status_t moe_route_backward(const moe_shape_t* shape, const int32_t* d_ids, const float* d_w,
                                const float* d_dw, float* d_dlogits, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t T = shape->T, N = T * shape->k;
    if (bad(d_ids, N) || bad(d_w, N) || bad(d_dw, N) || bad(d_dlogits, T)) return MOE_EINVAL;
    return dev(moe_launch_route_backward(*shape, d_ids, d_w, d_dw, d_dlogits, as_stream(stream)));
}

size_t moe_router_workspace_bytes(const moe_shape_t* shape)
{
    if (check(shape) != MOE_OK) return 0;
    return moe::router_ws_bytes(*shape);
}

moe_status_t moe_router(const moe_shape_t* shape, const void* d_x, const void* d_w_router,
                        const float* d_bias, float* d_logits, int32_t* d_ids, float* d_w,
                        int32_t* d_err, void* d_ws, size_t ws_bytes, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    const int64_t T = shape->T, N = T * shape->k;
    if (bad(d_x, T) || !d_w_router || bad(d_logits, T) || bad(d_ids, N) || bad(d_w, N) || !d_err)
        return MOE_EINVAL;
    // W_r rows are addressed with 32-bit byte offsets
    if (shape->dtype == MOE_BF16 && (int64_t)shape->E * shape->H * 2 >= (int64_t(1) << 32))
        return MOE_EUNSUPPORTED;
    const moe::RouterSplit sp = moe::router_split(*shape);
    const size_t need = moe::router_ws_bytes(*shape);
    if (need > 0 && (!d_ws || ws_bytes < need)) return MOE_EINVAL;
    hipStream_t hs = as_stream(stream);
    if (sp.parts > 1) {
        float* planes = static_cast<float*>(d_ws);
        hipError_t e = moe_launch_router_logits(*shape, d_x, d_w_router, planes, hs);
        if (e != hipSuccess) return MOE_EDEVICE;
        return dev(moe_launch_route(*shape, planes, d_bias, d_ids, d_w, d_err, hs, sp.parts,
                                    T * shape->E, d_logits));
    }
    hipError_t e = moe_launch_router_logits(*shape, d_x, d_w_router, d_logits, hs);
    if (e != hipSuccess) return MOE_EDEVICE;
    return dev(moe_launch_route(*shape, d_logits, d_bias, d_ids, d_w, d_err, hs));
}

moe_status_t moe_bias_update(const moe_shape_t* shape, const int32_t* d_counts, float* d_bias,
                             float gamma, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    if (!d_counts || !d_bias || !(gamma >= 0.0f) || !isfinite(gamma)) return MOE_EINVAL;
    return dev(moe_launch_bias_update(*shape, d_counts, gamma, d_bias, as_stream(stream)));
}

int32_t moe_capacity_rows(const moe_shape_t* shape, double capacity_factor)
{
    if (check(shape) != MOE_OK) return -1;
    if (!(capacity_factor > 0.0) || !isfinite(capacity_factor)) return -1;
    const int64_t N = (int64_t)shape->T * shape->k;
    // the page's formula in the page's order: N / E * factor (as in moe_stats)
    const double capd = ceil((double)N / (double)shape->E * capacity_factor);
    if (!(capd * shape->E < 2147483647.0)) return -1;
    return (int32_t)capd;
}

namespace {
// cap >= 1 and the [E][cap] buffer addressable like an N-row one
inline bool bad_cap(const moe_shape_t* s, int32_t cap)
{
    return cap < 1 || (int64_t)cap * s->E >= (int64_t(1) << 31);
}
}  // namespace

moe_status_t moe_capacity_dispatch(const moe_shape_t* shape, int32_t cap, const int32_t* d_counts,
                                   const void* d_x, const int32_t* d_ids, const int32_t* d_eidx,
                                   void* d_buf, int32_t* d_dest_row, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    if (bad_cap(shape, cap)) return MOE_EINVAL;
    const int64_t T = shape->T, N = T * shape->k;
    if (!d_counts || bad(d_x, T) || bad(d_ids, N) || bad(d_eidx, N) || !d_buf ||
        bad(d_dest_row, N))
        return MOE_EINVAL;
    return dev(moe_launch_capacity_dispatch(*shape, cap, d_counts, d_x, d_ids, d_eidx, d_buf,
                                            d_dest_row, as_stream(stream)));
}

moe_status_t moe_capacity_plan(const moe_shape_t* shape, int32_t cap, int32_t* d_plan,
                               moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    if (bad_cap(shape, cap) || !d_plan) return MOE_EINVAL;
    return dev(moe_launch_capacity_plan(*shape, cap, d_plan, as_stream(stream)));
}

moe_status_t moe_capacity_combine(const moe_shape_t* shape, int32_t cap, const void* d_y,
                                  const int32_t* d_dest_row, const float* d_w,
                                  const void* d_shared_y, void* d_out, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    if (bad_cap(shape, cap)) return MOE_EINVAL;
    const int64_t T = shape->T, N = T * shape->k;
    if (!d_y || bad(d_dest_row, N) || bad(d_w, N) || bad(d_out, T)) return MOE_EINVAL;
    return dev(moe_launch_combine_rows(*shape, (int64_t)cap * shape->E, d_y, d_dest_row, d_w,
                                       d_shared_y, d_out, as_stream(stream)));
}

moe_status_t moe_repack(const moe_shape_t* shape, const int32_t* d_counts, int32_t* d_mapping,
                        moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    if (!d_counts || !d_mapping) return MOE_EINVAL;
    return dev(moe_launch_repack(*shape, d_counts, d_mapping, as_stream(stream)));
}

moe_status_t moe_stats(const moe_shape_t* shape, const int32_t* d_counts, const int32_t* d_ids,
                       const int32_t* d_plan, const int32_t* d_dest_row,
                       const int32_t* d_mapping, const int32_t* d_origin, const int32_t* d_err,
                       double capacity_factor, void* d_ws, size_t ws_bytes, moe_stats_t* h_out,
                       int32_t* h_rank_loads, moe_stream_t stream)
{
    moe_status_t st = check(shape);
    if (st != MOE_OK) return st;
    if (!d_counts || bad(d_ids, (int64_t)shape->T * shape->k) || !d_plan || !d_ws || !h_out)
        return MOE_EINVAL;
    if (!(capacity_factor > 0.0) || !isfinite(capacity_factor)) return MOE_EINVAL;
    const moe::WsLayout W = moe::ws_layout(*shape);
    if (ws_bytes < W.total) return MOE_EINVAL;
    const int E = shape->E, R = shape->R;
    const int64_t N = (int64_t)shape->T * shape->k;
    // capacity from the page's formula in the page's order: N / E * factor
    const double capd = ceil((double)N / (double)E * capacity_factor);
    if (!(capd < 2147483647.0)) return MOE_EINVAL;
    const int32_t cap = (int32_t)capd;
    int64_t* d_out = reinterpret_cast<int64_t*>(static_cast<char*>(d_ws) + W.stats);
    hipStream_t hs = as_stream(stream);
    hipError_t e = moe_launch_stats(*shape, d_counts, d_ids, d_plan, d_dest_row, d_mapping,
                                    d_origin, d_err, cap, d_out, hs);
    if (e != hipSuccess) return MOE_EDEVICE;
    int64_t h[moe::kStScalars + 3 * 64];
    const size_t nb = sizeof(int64_t) * moe::stats_slots(R);
    e = hipMemcpyAsync(h, d_out, nb, hipMemcpyDeviceToHost, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e != hipSuccess) return MOE_EDEVICE;

    auto maxvio = [](int64_t mx, int M, int64_t total) {
        return total <= 0 ? 0.0 : (double)(mx * (int64_t)M - total) / (double)total;
    };
    auto bal = [](int64_t mx, int M, int64_t total) {
        return mx <= 0 ? 1.0 : (double)total / (double)(mx * (int64_t)M);
    };
    memset(h_out, 0, sizeof(*h_out));
    h_out->N = h[moe::kStN];
    h_out->E = E;
    h_out->R = R;
    h_out->max_count = (int32_t)h[moe::kStMax];
    h_out->min_count = (int32_t)h[moe::kStMin];
    h_out->active_experts = (int32_t)h[moe::kStActive];
    h_out->maxvio_expert = maxvio(h[moe::kStMax], E, h[moe::kStN]);
    h_out->balancedness_expert = bal(h[moe::kStMax], E, h[moe::kStN]);
    int64_t hm = 0, mm = 0, pm = 0, pmin = -1;
    for (int r = 0; r < R; ++r) {
        const int64_t hv = h[moe::kStScalars + r], mv = h[moe::kStScalars + R + r],
                      pv = h[moe::kStScalars + 2 * R + r];
        hm = hv > hm ? hv : hm;
        mm = mv > mm ? mv : mm;
        pm = pv > pm ? pv : pm;
        pmin = (pmin < 0 || pv < pmin) ? pv : pmin;
        if (h_rank_loads) {
            h_rank_loads[r] = (int32_t)hv;
            h_rank_loads[R + r] = (int32_t)mv;
            h_rank_loads[2 * R + r] = (int32_t)pv;
        }
    }
    h_out->home_max = (int32_t)hm;
    h_out->maxvio_rank_home = maxvio(hm, R, h_out->N);
    h_out->balancedness_rank_home = bal(hm, R, h_out->N);
    if (d_mapping) {
        h_out->mapped_max = (int32_t)mm;
        h_out->maxvio_rank_mapped = maxvio(mm, R, h_out->N);
        h_out->balancedness_rank_mapped = bal(mm, R, h_out->N);
    }
    h_out->planned_max = (int32_t)pm;
    h_out->planned_min = (int32_t)(pmin < 0 ? 0 : pmin);
    h_out->maxvio_rank_planned = maxvio(pm, R, h_out->N);
    h_out->balancedness_rank_planned = bal(pm, R, h_out->N);
    h_out->capacity = cap;
    h_out->processed = h[moe::kStProcessed];
    h_out->overflow = h[moe::kStOverflow];
    h_out->padding = h[moe::kStPadding];
    h_out->remote_home = h[moe::kStRemoteHome];
    h_out->remote_mapped = h[moe::kStRemoteMapped];
    h_out->remote_planned = h[moe::kStRemotePlanned];
    h_out->replica_pieces = (int32_t)h[moe::kStReplicas];
    h_out->max_slots_needed = (int32_t)h[moe::kStMaxSlots];
    h_out->ranks_over_slots = (int32_t)h[moe::kStOverSlots];
    h_out->nonlocal_rows = h[moe::kStNonlocal];
    h_out->err = (int32_t)h[moe::kStErr];
    return h_out->err ? MOE_EDATA : MOE_OK;
}

}  // extern "C"
