// decoder.cpp -- the decode loop's per-step host work in one call (C ABI in include/pkv.h).
//
// Per step: reserve every sequence's next slot in the block manager, write the
// step's metadata (positions | copy pairs | block tables) into a pinned buffer,
// and enqueue on the caller's stream the copy of that buffer to the device
// followed by the step -- one step-graph replay, or the eager calls.  Two
// metadata sets alternate: the host only waits for the step that last used the
// set (two steps back), so it prepares step k+1 while the GPU runs step k (the
// "Injecting Adrenaline into LLM Serving" review, section 3.2.1, metadata
// prepared ahead of the step; section 3.2.2, graphs against launch overhead).
//
// Where the copy runs is chosen per step from the K/V bytes the step reads.  On
// MI355X with ROCm a dependency across streams (event recorded on a copy
// stream, waited for on the compute stream) costs ~17 us per step, while the
// copy itself, in order on the compute stream, costs ~4 us for a few KB and
// ~10 us for the ~100 KB tables of a long-context batch.  A short step (below
// kSideStreamBytes) copies in order; a long step copies on a side stream,
// where the copy and the dependency overlap the previous step's kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>

#include "pkv.h"
#include "pkv_host.h"

using pkv::fail;

namespace {
constexpr double kSideStreamBytes = 512.0 * 1024 * 1024;   // K/V bytes a step reads
}

struct pkv_decoder {
    pkv_decoder_desc d{};
    pkv_block_manager* bm = nullptr;
    int32_t meta_len = 0;                      // ints per metadata set
    int32_t* host[2] = {nullptr, nullptr};     // pinned
    int32_t* dev[2] = {nullptr, nullptr};
    hipStream_t side = nullptr;
    hipEvent_t staged[2] = {nullptr, nullptr};
    hipEvent_t done[2] = {nullptr, nullptr};
    double kv_bytes_per_token = 0;
    pkv_step_graphs* graphs[2] = {nullptr, nullptr};
    int32_t* bcaps = nullptr;                  // copies of the capacity lists
    int32_t* ccaps = nullptr;
    uint64_t steps = 0;

    ~pkv_decoder() {
        for (int s = 0; s < 2; ++s) {
            if (done[s]) (void)hipEventSynchronize(done[s]);
            pkv_step_graphs_destroy(graphs[s]);
            if (staged[s]) (void)hipEventDestroy(staged[s]);
            if (done[s]) (void)hipEventDestroy(done[s]);
            if (dev[s]) (void)hipFree(dev[s]);
            if (host[s]) (void)hipHostFree(host[s]);
        }
        if (side) (void)hipStreamDestroy(side);
        pkv_bm_destroy(bm);
        delete[] bcaps;
        delete[] ccaps;
    }
};

namespace {

// Device views of metadata set s.
struct MetaView {
    int32_t* positions;
    int32_t* cow_src;
    int32_t* cow_dst;
    int32_t* tables;
};

MetaView view(int32_t* base, int32_t max_batch) {
    return {base, base + max_batch, base + 2 * (int64_t)max_batch, base + 3 * (int64_t)max_batch};
}

bool increasing(const int32_t* v, int32_t n) {
    for (int32_t i = 0; i < n; ++i)
        if (v[i] <= 0 || (i && v[i] <= v[i - 1])) return false;
    return true;
}

}  // namespace

extern "C" {

pkv_decoder* pkv_decoder_create(const pkv_decoder_desc* desc) {
    if (!desc) {
        fail(PKV_ERR_NULL, "desc is NULL");
        return nullptr;
    }
    const pkv_decoder_desc& d = *desc;
    if (d.max_batch <= 0 || d.bt_stride <= 0 || d.block_size <= 0 || d.n_blocks <= 0) {
        fail(PKV_ERR_INVALID_ARG, "max_batch, bt_stride, block_size and n_blocks must be positive");
        return nullptr;
    }
    if ((int64_t)d.max_batch * (3 + (int64_t)d.bt_stride) > (1 << 28)) {
        fail(PKV_ERR_INVALID_ARG, "max_batch * bt_stride is too large");
        return nullptr;
    }
    const int32_t max_ctx = d.bt_stride * d.block_size;
    if (d.n_batch_caps > 0) {
        if (!d.batch_caps || !d.ctx_caps || d.n_ctx_caps <= 0 || !increasing(d.batch_caps, d.n_batch_caps) ||
            !increasing(d.ctx_caps, d.n_ctx_caps) || d.batch_caps[d.n_batch_caps - 1] != d.max_batch ||
            d.ctx_caps[d.n_ctx_caps - 1] != max_ctx) {
            fail(PKV_ERR_INVALID_ARG, "capacity lists must increase and end at max_batch = %d and "
                 "bt_stride * block_size = %d", d.max_batch, max_ctx);
            return nullptr;
        }
    }
    if (!d.k_scale != !d.v_scale || !d.k_mx_scale != !d.v_mx_scale || (d.k_scale && d.k_mx_scale)) {
        fail(PKV_ERR_INVALID_ARG, "set k_scale and v_scale (FP8 pools) or k_mx_scale and v_mx_scale (MXFP4 pools), "
             "both of a pair or neither");
        return nullptr;
    }
    if (d.partition_size > 0) {
        const size_t need = pkv_decode_workspace_bytes(d.max_batch, d.H_q, d.D, max_ctx, d.partition_size);
        if (need && (!d.workspace || d.workspace_bytes < need)) {
            fail(PKV_ERR_WORKSPACE, "the decoder needs %zu bytes of workspace, got %zu", need, d.workspace_bytes);
            return nullptr;
        }
    }
    pkv_decoder* dec = new (std::nothrow) pkv_decoder();
    if (!dec) {
        fail(PKV_ERR_INVALID_ARG, "out of host memory");
        return nullptr;
    }
    dec->d = d;
    dec->d.batch_caps = dec->d.ctx_caps = nullptr;
    dec->bm = pkv_bm_create(d.n_blocks, d.block_size, d.shuffle_seed);
    if (!dec->bm) {
        delete dec;
        return nullptr;
    }
    dec->meta_len = d.max_batch * (3 + d.bt_stride);
    const size_t bytes = (size_t)dec->meta_len * sizeof(int32_t);
    const int eb = d.dtype == PKV_F32 ? 4 : 2;
    dec->kv_bytes_per_token = d.k_scale      ? 2.0 * d.H_kv * (d.D + 4)
                              : d.k_mx_scale ? 2.0 * d.H_kv * (d.D / 2 + d.D / 32)
                                             : 2.0 * d.H_kv * d.D * eb;
    hipError_t e = hipStreamCreateWithFlags(&dec->side, hipStreamNonBlocking);
    for (int s = 0; s < 2 && e == hipSuccess; ++s) {
        e = hipHostMalloc(reinterpret_cast<void**>(&dec->host[s]), bytes, hipHostMallocDefault);
        if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&dec->dev[s]), bytes);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&dec->staged[s], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&dec->done[s], hipEventDisableTiming);
        if (e == hipSuccess) {
            std::fill(dec->host[s], dec->host[s] + dec->meta_len, -1);
            e = hipMemcpy(dec->dev[s], dec->host[s], bytes, hipMemcpyHostToDevice);
        }
        if (e == hipSuccess) e = hipEventRecord(dec->done[s], nullptr);
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        fail(PKV_ERR_HIP, "decoder set-up: %s", hipGetErrorString(e));
        delete dec;
        return nullptr;
    }
    if (d.n_batch_caps > 0) {
        dec->bcaps = new (std::nothrow) int32_t[d.n_batch_caps];
        dec->ccaps = new (std::nothrow) int32_t[d.n_ctx_caps];
        if (!dec->bcaps || !dec->ccaps) {
            fail(PKV_ERR_INVALID_ARG, "out of host memory");
            delete dec;
            return nullptr;
        }
        std::copy(d.batch_caps, d.batch_caps + d.n_batch_caps, dec->bcaps);
        std::copy(d.ctx_caps, d.ctx_caps + d.n_ctx_caps, dec->ccaps);
        dec->d.batch_caps = dec->bcaps;
        dec->d.ctx_caps = dec->ccaps;
        for (int s = 0; s < 2; ++s) {
            const MetaView m = view(dec->dev[s], d.max_batch);
            pkv_step_desc g{};
            g.dtype = d.dtype;
            g.H_q = d.H_q;
            g.H_kv = d.H_kv;
            g.D = d.D;
            g.block_size = d.block_size;
            g.n_blocks = d.n_blocks;
            g.scale = d.scale;
            g.partition_size = d.partition_size;
            g.out = d.out;
            g.q = d.q;
            g.q_row_stride = d.q_row_stride;
            g.k_new = d.k_new;
            g.v_new = d.v_new;
            g.new_row_stride = d.new_row_stride;
            g.k_pool = d.k_pool;
            g.v_pool = d.v_pool;
            g.block_tables = m.tables;
            g.bt_stride = d.bt_stride;
            g.positions = m.positions;
            g.cow_src = m.cow_src;
            g.cow_dst = m.cow_dst;
            g.workspace = d.workspace;
            g.workspace_bytes = d.workspace_bytes;
            g.k_scale = d.k_scale;
            g.v_scale = d.v_scale;
            g.k_mx_scale = d.k_mx_scale;
            g.v_mx_scale = d.v_mx_scale;
            dec->graphs[s] = pkv_step_graphs_create(&g, dec->bcaps, d.n_batch_caps, dec->ccaps, d.n_ctx_caps);
            if (!dec->graphs[s]) {
                delete dec;   // pkv_last_error() holds the reason
                return nullptr;
            }
        }
    }
    pkv::clear_error();
    return dec;
}

void pkv_decoder_destroy(pkv_decoder* dec) { delete dec; }

pkv_block_manager* pkv_decoder_block_manager(pkv_decoder* dec) { return dec ? dec->bm : nullptr; }

int pkv_decoder_step(pkv_decoder* dec, const int64_t* seq_ids, int32_t B, void* stream, int32_t* n_copies) {
    if (n_copies) *n_copies = 0;
    if (!dec) return fail(PKV_ERR_NULL, "decoder is NULL");
    const pkv_decoder_desc& d = dec->d;
    if (B < 0 || B > d.max_batch) return fail(PKV_ERR_INVALID_ARG, "B = %d outside [0, %d]", B, d.max_batch);
    if (B == 0) {
        pkv::clear_error();
        return PKV_OK;
    }
    if (!seq_ids) return fail(PKV_ERR_NULL, "seq_ids is NULL");
    const int s = (int)(dec->steps & 1);
    hipError_t e = hipEventSynchronize(dec->done[s]);      // the step that last used set s is over
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "waiting for step: %s", hipGetErrorString(e));

    const MetaView h = view(dec->host[s], d.max_batch);
    int32_t nc = 0;
    int st = pkv_bm_append_batch(dec->bm, seq_ids, B, h.tables, d.bt_stride, h.positions, h.cow_src, h.cow_dst, &nc);
    if (st) return st;
    // rows the chosen bucket runs beyond B are padding; unused copy pairs are skipped
    int32_t Bc = B;
    if (dec->graphs[s]) Bc = *std::lower_bound(dec->bcaps, dec->bcaps + d.n_batch_caps, B);
    std::fill(h.positions + B, h.positions + Bc, -1);
    std::fill(h.cow_src + nc, h.cow_src + Bc, -1);
    std::fill(h.cow_dst + nc, h.cow_dst + Bc, -1);
    int32_t max_len = 0;
    int64_t history = 0;
    for (int32_t b = 0; b < B; ++b) {
        max_len = std::max(max_len, h.positions[b] + 1);
        history += h.positions[b];
    }

    // positions | copy pairs (all max_batch slots) | the first Bc table rows
    const size_t bytes = ((size_t)3 * d.max_batch + (size_t)Bc * d.bt_stride) * sizeof(int32_t);
    hipStream_t cs = reinterpret_cast<hipStream_t>(stream);
    if ((double)history * dec->kv_bytes_per_token >= kSideStreamBytes) {
        e = hipStreamWaitEvent(dec->side, dec->done[s], 0);
        if (e == hipSuccess) e = hipMemcpyAsync(dec->dev[s], dec->host[s], bytes, hipMemcpyHostToDevice, dec->side);
        if (e == hipSuccess) e = hipEventRecord(dec->staged[s], dec->side);
        if (e == hipSuccess) e = hipStreamWaitEvent(cs, dec->staged[s], 0);
    } else {
        e = hipMemcpyAsync(dec->dev[s], dec->host[s], bytes, hipMemcpyHostToDevice, cs);
    }
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "staging metadata: %s", hipGetErrorString(e));
    ++dec->steps;

    const MetaView m = view(dec->dev[s], d.max_batch);
    if (dec->graphs[s]) {
        st = pkv_step_graphs_launch(dec->graphs[s], B, max_len, nc, stream);
    } else if (d.k_mx_scale) {
        uint8_t* kp = static_cast<uint8_t*>(d.k_pool);
        uint8_t* vp = static_cast<uint8_t*>(d.v_pool);
        st = nc ? pkv_copy_blocks_mxfp4(kp, vp, d.k_mx_scale, d.v_mx_scale, m.cow_src, m.cow_dst, nc, d.H_kv, d.D,
                                        d.block_size, d.n_blocks, stream)
                : PKV_OK;
        if (st == PKV_OK)
            st = pkv_append_decode_attention_mxfp4(d.dtype, d.out, d.q, d.q_row_stride, d.k_new, d.v_new,
                                                   d.new_row_stride, kp, vp, d.k_mx_scale, d.v_mx_scale, m.tables,
                                                   d.bt_stride, m.positions, B, d.H_q, d.H_kv, d.D, d.block_size,
                                                   d.n_blocks, max_len, d.scale, d.partition_size, d.workspace,
                                                   d.workspace_bytes, stream);
    } else if (d.k_scale) {
        uint8_t* kp = static_cast<uint8_t*>(d.k_pool);
        uint8_t* vp = static_cast<uint8_t*>(d.v_pool);
        st = nc ? pkv_copy_blocks_fp8(kp, vp, d.k_scale, d.v_scale, m.cow_src, m.cow_dst, nc, d.H_kv, d.D,
                                      d.block_size, d.n_blocks, stream)
                : PKV_OK;
        if (st == PKV_OK)
            st = pkv_append_decode_attention_fp8(d.dtype, d.out, d.q, d.q_row_stride, d.k_new, d.v_new,
                                                 d.new_row_stride, kp, vp, d.k_scale, d.v_scale, m.tables,
                                                 d.bt_stride, m.positions, B, d.H_q, d.H_kv, d.D, d.block_size,
                                                 d.n_blocks, max_len, d.scale, d.partition_size, d.workspace,
                                                 d.workspace_bytes, stream);
    } else {
        st = nc ? pkv_copy_blocks(d.dtype, d.k_pool, d.v_pool, m.cow_src, m.cow_dst, nc, d.H_kv, d.D, d.block_size,
                                  d.n_blocks, stream)
                : PKV_OK;
        if (st == PKV_OK)
            st = pkv_append_decode_attention(d.dtype, d.out, d.q, d.q_row_stride, d.k_new, d.v_new,
                                             d.new_row_stride, d.k_pool, d.v_pool, m.tables, d.bt_stride,
                                             m.positions, B, d.H_q, d.H_kv, d.D, d.block_size, d.n_blocks, max_len,
                                             d.scale, d.partition_size, d.workspace, d.workspace_bytes, stream);
    }
    e = hipEventRecord(dec->done[s], cs);
    if (st) return st;
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "recording step: %s", hipGetErrorString(e));
    if (n_copies) *n_copies = nc;
    pkv::clear_error();
    return PKV_OK;
}

}  // extern "C"
