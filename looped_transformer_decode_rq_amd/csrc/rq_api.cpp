// C ABI of librq: argument validation, pool geometry, workspace carving and
// kernel launches. Nothing here allocates, frees or synchronizes.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "rq_internal.h"

namespace rq {

static bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

rq_status make_geom(const rq_layout *lay, Geom *g) {
    if (!lay || !g) return RQ_ERR_NULL;
    const int H = lay->num_heads, D = lay->head_dim, G = lay->group_size, L = lay->num_loops;
    if (H < 1 || L < 1 || L > RQ_MAX_LOOPS || lay->num_blocks < 1) return RQ_ERR_SHAPE;
    if (G < 1 || D < 1 || D % G != 0) return RQ_ERR_SHAPE;
    if (lay->block_size != 16) return RQ_ERR_UNSUPPORTED;
    if (D != 64 && D != 96 && D != 128) return RQ_ERR_UNSUPPORTED;
    bool g_ok = false;
    if (D == 128) g_ok = (G == 32 || G == 64 || G == 128);
    if (D == 96) g_ok = (G == 96);
    if (D == 64) g_ok = (G == 16 || G == 32 || G == 64);
    if (!g_ok) return RQ_ERR_UNSUPPORTED;
    if (lay->meta_dtype != RQ_DTYPE_F16 && lay->meta_dtype != RQ_DTYPE_F32) return RQ_ERR_UNSUPPORTED;
    if (lay->kv_dtype != RQ_DTYPE_BF16 && lay->kv_dtype != RQ_DTYPE_F32) return RQ_ERR_UNSUPPORTED;
    if (lay->mode != RQ_MODE_RESIDUAL && lay->mode != RQ_MODE_DIRECT) return RQ_ERR_UNSUPPORTED;
    g->direct = lay->mode == RQ_MODE_DIRECT;
    g->H = H; g->D = D; g->G = G; g->L = L; g->bs = 16; g->nblk = lay->num_blocks;
    g->meta = lay->meta_dtype; g->kvdt = lay->kv_dtype;
    g->msz = lay->meta_dtype == RQ_DTYPE_F16 ? 2 : 4;
    g->meta_bytes = g->bs * (D / G) * 2 * g->msz;
    int64_t off = 0;
    for (int l = 0; l < RQ_MAX_LOOPS; ++l) {
        g->bits[l] = 0; g->code_bytes[l] = 0; g->rec[l] = 0; g->loop_off[l] = 0;
    }
    for (int l = 0; l < L; ++l) {
        const int b = (l == L - 1 && !g->direct) ? 4 : (int)lay->loop_bits[l];
        if (b != 2 && b != 4) return RQ_ERR_UNSUPPORTED;
        g->bits[l] = b;
        g->code_bytes[l] = g->bs * D * b / 8;
        const int alpha = (l < L - 1 && !g->direct) ? g->bs * g->msz : 0;
        g->rec[l] = (int)round_up((size_t)(g->code_bytes[l] + g->meta_bytes + alpha), 16);
        g->loop_off[l] = off;
        off += 2 * (int64_t)g->rec[l];
    }
    g->loop_off[L] = off;
    g->slab = off;
    return RQ_OK;
}

// Compute units of the current device (queried once per device; 256 if the
// query fails).
static int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

int auto_split_pages(int units, int max_blocks, bool per_split) {
    // A split-K launch runs in rounds of resident workgroups (about three per
    // CU for these kernels); the last round is partly empty. Enough
    // workgroups for ~8 rounds (per-loop packed calls: four splits per
    // workgroup, merged into one partial) or ~14 rounds of one-split units
    // (one partial per split: the multi-loop kernel, whose workgroup reads a
    // page once for all its loops, and the bf16 baseline) keep that tail
    // small without shrinking the splits to where per-split setup and the
    // partials' merge dominate. The pages are then spread evenly over the
    // splits of a row, and the split rounded up to a multiple of 8 pages:
    // measured on MI355X at 16 sequences x 32768 tokens x 16 heads, such
    // splits run all three split kernels faster than their neighbours (the
    // per-loop residual call ~2% at 24 pages against 22, 23 or 25).
    const int waves = per_split ? 1 : kSplitWaves;
    const int64_t target = (int64_t)(per_split ? 14 : 8) * 3 * device_cus();
    const int64_t wg_per_unit = std::max<int64_t>(1, (target + units - 1) / std::max(units, 1));
    int64_t sp = ((int64_t)max_blocks + waves * wg_per_unit - 1) / (waves * wg_per_unit);
    sp = std::min<int64_t>(kMaxSplitPages, std::max<int64_t>(kMinAutoSplitPages, sp));
    const int64_t nwg = ((int64_t)max_blocks + waves * sp - 1) / (waves * sp);
    sp = ((int64_t)max_blocks + waves * nwg - 1) / (waves * nwg);
    sp = std::min<int64_t>(kMaxSplitPages, (sp + 7) / 8 * 8);
    return (int)std::max<int64_t>(1, sp);
}

static int nsplit_of(int max_blocks, int sp) { return (max_blocks + sp - 1) / sp; }

int partials_per_row(int n, int max_blocks, int sp) {
    const int ns = nsplit_of(max_blocks, sp);
    return n >= 2 ? ns : (ns + kSplitWaves - 1) / kSplitWaves;
}

// Several loop calls in one request share a multi-loop kernel (one split per
// workgroup); direct-mode calls are decoded one kernel per loop.
static bool multi_mode(const Geom &g, int n_loops) { return n_loops >= 2 && !g.direct; }

static size_t decode_ws(const Geom &g, int n, int B, int max_blocks, int sp) {
    const size_t qp = round_up((size_t)n * B * g.H * qpack_bytes(g.D), 256);
    const size_t parts =
        (size_t)n * B * g.H * partials_per_row(n, max_blocks, sp) * partial_floats(g.D) * sizeof(float);
    return qp + parts;
}

// Chunked prefill: each workgroup carries 64 queries over a long run of pages
// (compute-heavy), so the launch aims for about two rounds of workgroups at
// two per CU; a split is any number of pages.
static int chunk_split_pages(int B, int H, int C, int max_blocks) {
    const int64_t units = (int64_t)B * H * ((C + 63) / 64);
    const int64_t target = 4LL * device_cus();
    int64_t ns = std::max<int64_t>(1, std::min<int64_t>(max_blocks, (target + units - 1) / std::max<int64_t>(units, 1)));
    ns = std::max<int64_t>(ns, (max_blocks + kMaxChunkSplit - 1) / kMaxChunkSplit);
    return (int)((max_blocks + ns - 1) / ns);
}

static size_t chunk_ws(const Geom &g, int B, int C, int max_blocks, int sp) {
    const int64_t rows = (int64_t)B * C * g.H;
    return round_up((size_t)rows * chunk_qrec_bytes(g.D), 256) +
           (size_t)rows * nsplit_of(max_blocks, sp) * partial_floats(g.D) * sizeof(float);
}

// Scratch of the allocation-free decode entry point: a file-scope device
// array (one copy per GPU, held until the process ends). Host code never uses
// the array's name as an address: the device address is looked up once per
// device with hipGetSymbolAddress and kept.
__device__ __align__(256) uint8_t scratch[RQ_NOALLOC_SCRATCH_BYTES];

static void *scratch_address(hipError_t *err) {
    static std::mutex mu;
    static void *addr[64];
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= 64) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

static size_t bf16_ws(int H, int D, int B, int max_blocks, int sp) {
    return (size_t)B * H * nsplit_of(max_blocks, sp) * (2 + D) * sizeof(float);
}

}  // namespace rq

using namespace rq;

extern "C" {

const char *rq_status_string(rq_status s) {
    switch (s) {
        case RQ_OK: return "ok";
        case RQ_ERR_NULL: return "null pointer argument";
        case RQ_ERR_SHAPE: return "inconsistent or out-of-range sizes";
        case RQ_ERR_UNSUPPORTED: return "unsupported configuration";
        case RQ_ERR_WORKSPACE: return "workspace too small";
        case RQ_ERR_HIP: return "HIP runtime or launch failure";
        case RQ_ERR_SCRATCH: return "request needs more scratch than the allocation-free entry point holds";
        default: return "unknown status";
    }
}

rq_status rq_layout_check(const rq_layout *layout) {
    Geom g;
    return make_geom(layout, &g);
}

size_t rq_pool_bytes(const rq_layout *layout) {
    Geom g;
    if (make_geom(layout, &g) != RQ_OK) return 0;
    return (size_t)g.nblk * g.H * g.slab;
}

size_t rq_record_bytes(const rq_layout *layout, int32_t loop) {
    Geom g;
    if (make_geom(layout, &g) != RQ_OK || loop < 0 || loop >= g.L) return 0;
    return (size_t)g.rec[loop];
}

int64_t rq_record_offset(const rq_layout *layout, int32_t block, int32_t head, int32_t loop, int32_t kv) {
    Geom g;
    if (make_geom(layout, &g) != RQ_OK) return -1;
    if (block < 0 || block >= g.nblk || head < 0 || head >= g.H || loop < 0 || loop >= g.L || kv < 0 || kv > 1)
        return -1;
    return ((int64_t)block * g.H + head) * g.slab + g.loop_off[loop] + (int64_t)kv * g.rec[loop];
}

size_t rq_encode_workspace_bytes(const rq_layout *layout, int32_t num_tokens) {
    Geom g;
    if (num_tokens < 0 || make_geom(layout, &g) != RQ_OK) return SIZE_MAX;
    return 0;
}

rq_status rq_encode_pack(const rq_layout *layout, void *pool, const void *kv_new, const float *rot,
                         const int64_t *slot_mapping, int32_t num_tokens, void *stream) {
    Geom g;
    rq_status st = make_geom(layout, &g);
    if (st != RQ_OK) return st;
    if (num_tokens < 0) return RQ_ERR_SHAPE;
    if (num_tokens == 0) return RQ_OK;
    if (!pool || !kv_new || !slot_mapping || (g.L > 1 && !g.direct && !rot)) return RQ_ERR_NULL;
    if (!aligned(pool, 16)) return RQ_ERR_SHAPE;
    if (num_tokens > (1 << 30) / 16) return RQ_ERR_SHAPE;
    EncodeCall c;
    c.g = &g; c.pool = (uint8_t *)pool; c.kv_new = kv_new; c.rot = rot; c.slots = slot_mapping;
    c.T = num_tokens; c.stream = (hipStream_t)stream;
    return launch_encode(c) == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

size_t rq_decode_workspace_bytes(const rq_layout *layout, int32_t n_loops, int32_t batch,
                                 int32_t max_blocks_per_seq, int32_t split_pages) {
    Geom g;
    if (make_geom(layout, &g) != RQ_OK || n_loops < 1 || batch < 0 || max_blocks_per_seq < 1 || split_pages < 0 ||
        split_pages > kMaxSplitPages)
        return 0;
    const int sp = split_pages > 0 ? split_pages : auto_split_pages(batch * g.H, max_blocks_per_seq, multi_mode(g, n_loops));
    return decode_ws(g, n_loops, batch, max_blocks_per_seq, sp);
}

int32_t rq_decode_auto_split_pages(const rq_layout *layout, int32_t n_loops, int32_t batch,
                                   int32_t max_blocks_per_seq) {
    Geom g;
    if (make_geom(layout, &g) != RQ_OK || n_loops < 1 || batch < 1 || max_blocks_per_seq < 1) return 0;
    return auto_split_pages(batch * g.H, max_blocks_per_seq, multi_mode(g, n_loops));
}

int32_t rq_bf16_auto_split_pages(int32_t num_heads, int32_t batch, int32_t max_blocks_per_seq) {
    if (num_heads < 1 || batch < 1 || max_blocks_per_seq < 1) return 0;
    return auto_split_pages(batch * num_heads, max_blocks_per_seq, true);
}

static rq_status decode_impl(const rq_layout *layout, const void *pool, const int32_t *loops, int32_t n_loops,
                             const void *q, const float *rot, const int32_t *block_table, const int32_t *seq_lens,
                             int32_t batch, int32_t max_blocks_per_seq, const void *tail_k, const void *tail_v,
                             float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                             const rq_decode_opts *opts, void *stream, void *enc_pool, const void *kv_new,
                             const int64_t *slot_mapping, int32_t num_tokens, bool stream_probe = false) {
    Geom g;
    rq_status st = make_geom(layout, &g);
    if (st != RQ_OK) return st;
    if (num_tokens < 0 || num_tokens > (1 << 30) / 16) return RQ_ERR_SHAPE;
    if (num_tokens > 0 && (!kv_new || !slot_mapping || !enc_pool || (g.L > 1 && !g.direct && !rot)))
        return RQ_ERR_NULL;
    if (!loops) return RQ_ERR_NULL;
    if (n_loops < 1 || n_loops > RQ_MAX_LOOPS || batch < 0 || batch > 65535 || max_blocks_per_seq < 1)
        return RQ_ERR_SHAPE;
    bool any_res = false;
    for (int i = 0; i < n_loops; ++i) {
        if (loops[i] < 0 || loops[i] >= g.L) return RQ_ERR_SHAPE;
        any_res = any_res || (loops[i] != g.L - 1 && !g.direct);
    }
    if (!isfinite(softmax_scale)) return RQ_ERR_SHAPE;
    if ((tail_k == nullptr) != (tail_v == nullptr)) return RQ_ERR_NULL;
    const int sp_req = opts ? opts->split_pages : 0;
    if (sp_req < 0) return RQ_ERR_SHAPE;
    if (sp_req > kMaxSplitPages) return RQ_ERR_UNSUPPORTED;
    if (batch == 0) return RQ_OK;
    if (!pool || !block_table || !seq_lens) return RQ_ERR_NULL;
    if (!stream_probe && (!q || !out || (any_res && !rot))) return RQ_ERR_NULL;
    if (!aligned(pool, 16)) return RQ_ERR_SHAPE;
    if ((int64_t)max_blocks_per_seq * 16 > (int64_t)1 << 30) return RQ_ERR_SHAPE;
    const int sp = sp_req > 0 ? sp_req : auto_split_pages(batch * g.H, max_blocks_per_seq, multi_mode(g, n_loops));
    const size_t need = decode_ws(g, n_loops, batch, max_blocks_per_seq, sp);
    if (!workspace) return RQ_ERR_NULL;
    if (workspace_bytes < need) return RQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return RQ_ERR_SHAPE;

    DecodeCall c;
    c.g = &g; c.pool = (const uint8_t *)pool; c.n = n_loops;
    for (int i = 0; i < RQ_MAX_LOOPS; ++i) c.loops[i] = i < n_loops ? loops[i] : 0;
    c.q = q; c.rot = rot; c.block_table = block_table; c.seq_lens = seq_lens;
    c.B = batch; c.max_blocks = max_blocks_per_seq; c.tail_k = tail_k; c.tail_v = tail_v;
    c.softmax_scale = softmax_scale; c.out = out;
    c.qpack = (uint8_t *)workspace;
    c.partials = (float *)((uint8_t *)workspace + round_up((size_t)n_loops * batch * g.H * qpack_bytes(g.D), 256));
    c.split_pages = sp; c.nsplit = nsplit_of(max_blocks_per_seq, sp);
    // direct mode decodes loop calls one kernel each (nothing shared between loops)
    c.nparts = g.direct ? partials_per_row(1, max_blocks_per_seq, sp) : partials_per_row(n_loops, max_blocks_per_seq, sp);
    c.ev_begin = opts ? (hipEvent_t)opts->event_main_begin : nullptr;
    c.ev_end = opts ? (hipEvent_t)opts->event_main_end : nullptr;
    c.stream = (hipStream_t)stream;
    c.enc_pool = (uint8_t *)enc_pool; c.enc_kv = kv_new; c.enc_slots = slot_mapping; c.enc_T = num_tokens;
    c.stream_probe = stream_probe;
    if (stream_probe) c.partials = (float *)workspace;   // the checksums, at the start of the workspace
    return launch_decode(c) == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

rq_status rq_decode_attention_ex(const rq_layout *layout, const void *pool, const int32_t *loops,
                                 int32_t n_loops, const void *q, const float *rot,
                                 const int32_t *block_table, const int32_t *seq_lens, int32_t batch,
                                 int32_t max_blocks_per_seq, const void *tail_k, const void *tail_v,
                                 float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                                 const rq_decode_opts *opts, void *stream) {
    return decode_impl(layout, pool, loops, n_loops, q, rot, block_table, seq_lens, batch, max_blocks_per_seq,
                       tail_k, tail_v, softmax_scale, out, workspace, workspace_bytes, opts, stream, nullptr,
                       nullptr, nullptr, 0);
}

rq_status rq_decode_attention_noalloc(const rq_layout *layout, const void *pool, const int32_t *loops,
                                      int32_t n_loops, const void *q, const float *rot,
                                      const int32_t *block_table, const int32_t *seq_lens, int32_t batch,
                                      int32_t max_blocks_per_seq, const void *tail_k, const void *tail_v,
                                      float softmax_scale, float *out, const rq_decode_opts *opts, void *stream) {
    hipError_t err = hipSuccess;
    void *ws = scratch_address(&err);
    if (!ws) return RQ_ERR_HIP;
    const rq_status st = decode_impl(layout, pool, loops, n_loops, q, rot, block_table, seq_lens, batch,
                                     max_blocks_per_seq, tail_k, tail_v, softmax_scale, out, ws,
                                     RQ_NOALLOC_SCRATCH_BYTES, opts, stream, nullptr, nullptr, nullptr, 0);
    return st == RQ_ERR_WORKSPACE ? RQ_ERR_SCRATCH : st;
}

rq_status rq_decode_stream_probe(const rq_layout *layout, const void *pool, int32_t loop, const int32_t *block_table,
                                 const int32_t *seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                                 void *workspace, size_t workspace_bytes, const rq_decode_opts *opts, void *stream) {
    Geom g;
    const rq_status st = make_geom(layout, &g);
    if (st != RQ_OK) return st;
    if (loop < 0 || loop >= g.L) return RQ_ERR_SHAPE;
    const int32_t loops[1] = {loop};
    return decode_impl(layout, pool, loops, 1, nullptr, nullptr, block_table, seq_lens, batch, max_blocks_per_seq,
                       nullptr, nullptr, 1.0f, nullptr, workspace, workspace_bytes, opts, stream, nullptr, nullptr,
                       nullptr, 0, true);
}

rq_status rq_decode_attention_encode(const rq_layout *layout, void *pool, const int32_t *loops, int32_t n_loops,
                                     const void *q, const float *rot, const int32_t *block_table,
                                     const int32_t *seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                                     const void *tail_k, const void *tail_v, float softmax_scale, float *out,
                                     void *workspace, size_t workspace_bytes, const void *kv_new,
                                     const int64_t *slot_mapping, int32_t num_tokens, const rq_decode_opts *opts,
                                     void *stream) {
    return decode_impl(layout, pool, loops, n_loops, q, rot, block_table, seq_lens, batch, max_blocks_per_seq,
                       tail_k, tail_v, softmax_scale, out, workspace, workspace_bytes, opts, stream, pool, kv_new,
                       slot_mapping, num_tokens);
}

rq_status rq_decode_attention(const rq_layout *layout, const void *pool, const int32_t *loops, int32_t n_loops,
                              const void *q, const float *rot, const int32_t *block_table,
                              const int32_t *seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                              const void *tail_k, const void *tail_v, float softmax_scale, float *out,
                              void *workspace, size_t workspace_bytes, void *stream) {
    return rq_decode_attention_ex(layout, pool, loops, n_loops, q, rot, block_table, seq_lens, batch,
                                  max_blocks_per_seq, tail_k, tail_v, softmax_scale, out, workspace,
                                  workspace_bytes, nullptr, stream);
}

// Layouts the chunked-prefill kernels support (RQ_OK) or the reason.
static rq_status chunk_supported(const Geom &g) {
    if (g.direct || g.G != g.D || g.kvdt != RQ_DTYPE_BF16) return RQ_ERR_UNSUPPORTED;
    return RQ_OK;
}

size_t rq_chunk_workspace_bytes(const rq_layout *layout, int32_t chunk, int32_t batch, int32_t max_blocks_per_seq,
                                int32_t split_pages) {
    Geom g;
    if (make_geom(layout, &g) != RQ_OK || chunk_supported(g) != RQ_OK || chunk < 1 || chunk > kMaxChunk ||
        batch < 0 || max_blocks_per_seq < 1 || split_pages < 0)
        return 0;
    const int sp = split_pages > 0 ? split_pages : chunk_split_pages(batch, g.H, chunk, max_blocks_per_seq);
    return chunk_ws(g, batch, chunk, max_blocks_per_seq, sp);
}

rq_status rq_chunk_attention(const rq_layout *layout, const void *pool, int32_t loop, int32_t chunk, const void *q,
                             const float *rot, const int32_t *block_table, const int32_t *seq_lens, int32_t batch,
                             int32_t max_blocks_per_seq, const void *chunk_k, const void *chunk_v,
                             float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                             const rq_decode_opts *opts, void *stream) {
    Geom g;
    rq_status st = make_geom(layout, &g);
    if (st != RQ_OK) return st;
    st = chunk_supported(g);
    if (st != RQ_OK) return st;
    if (loop < 0 || loop >= g.L || chunk < 1 || batch < 0 || batch > 65535 || max_blocks_per_seq < 1)
        return RQ_ERR_SHAPE;
    if (chunk > kMaxChunk) return RQ_ERR_UNSUPPORTED;
    if (!isfinite(softmax_scale)) return RQ_ERR_SHAPE;
    if ((chunk_k == nullptr) != (chunk_v == nullptr)) return RQ_ERR_NULL;
    const int sp_req = opts ? opts->split_pages : 0;
    if (sp_req < 0) return RQ_ERR_SHAPE;
    if (sp_req > kMaxChunkSplit) return RQ_ERR_UNSUPPORTED;
    if (batch == 0) return RQ_OK;
    if (!pool || !q || !block_table || !seq_lens || !out || (loop != g.L - 1 && !rot)) return RQ_ERR_NULL;
    if (!aligned(pool, 16) || !aligned(q, 16) || (chunk_k && (!aligned(chunk_k, 16) || !aligned(chunk_v, 16))))
        return RQ_ERR_SHAPE;
    if ((int64_t)max_blocks_per_seq * 16 > (int64_t)1 << 30) return RQ_ERR_SHAPE;
    const int sp = sp_req > 0 ? sp_req : chunk_split_pages(batch, g.H, chunk, max_blocks_per_seq);
    // launch grids: splits, sequences x 64-query groups, 16-row tiles and
    // sequences x 16-query tiles each within 65535
    if (nsplit_of(max_blocks_per_seq, sp) > 65535 || (int64_t)batch * ((chunk + 63) / 64) > 65535 ||
        ((int64_t)batch * chunk + 15) / 16 > 65535 || (int64_t)batch * ((chunk + 15) / 16) > 65535)
        return RQ_ERR_UNSUPPORTED;
    if (!workspace) return RQ_ERR_NULL;
    if (workspace_bytes < chunk_ws(g, batch, chunk, max_blocks_per_seq, sp)) return RQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return RQ_ERR_SHAPE;
    ChunkCall c;
    c.g = &g; c.pool = (const uint8_t *)pool; c.loop = loop; c.B = batch; c.C = chunk;
    c.max_blocks = max_blocks_per_seq; c.q = q; c.rot = rot; c.block_table = block_table; c.seq_lens = seq_lens;
    c.chunk_k = chunk_k; c.chunk_v = chunk_v; c.softmax_scale = softmax_scale; c.out = out;
    c.qrec = (uint8_t *)workspace;
    c.partials = (float *)((uint8_t *)workspace + round_up((size_t)batch * chunk * g.H * chunk_qrec_bytes(g.D), 256));
    c.split_pages = sp; c.nsplit = nsplit_of(max_blocks_per_seq, sp);
    c.ev_begin = opts ? (hipEvent_t)opts->event_main_begin : nullptr;
    c.ev_end = opts ? (hipEvent_t)opts->event_main_end : nullptr;
    c.stream = (hipStream_t)stream;
    return launch_chunk(c) == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

size_t rq_bf16_workspace_bytes(int32_t num_heads, int32_t head_dim, int32_t batch, int32_t max_blocks_per_seq,
                               int32_t split_pages) {
    if (num_heads < 1 || batch < 0 || max_blocks_per_seq < 1 || split_pages < 0) return 0;
    if (head_dim != 64 && head_dim != 96 && head_dim != 128) return 0;
    const int sp = split_pages > 0 ? split_pages : auto_split_pages(batch * num_heads, max_blocks_per_seq, true);
    return bf16_ws(num_heads, head_dim, batch, max_blocks_per_seq, sp);
}

rq_status rq_bf16_decode_attention_ex(int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      const void *k_cache, const void *v_cache, const void *q,
                                      const int32_t *block_table, const int32_t *seq_lens, int32_t batch,
                                      int32_t max_blocks_per_seq, const void *tail_k, const void *tail_v,
                                      float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                                      const rq_decode_opts *opts, void *stream) {
    if (num_heads < 1 || num_blocks < 1 || batch < 0 || batch > 65535 || max_blocks_per_seq < 1) return RQ_ERR_SHAPE;
    if (block_size != 16) return RQ_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 96 && head_dim != 128) return RQ_ERR_UNSUPPORTED;
    if (!isfinite(softmax_scale)) return RQ_ERR_SHAPE;
    if ((tail_k == nullptr) != (tail_v == nullptr)) return RQ_ERR_NULL;
    const int sp_req = opts ? opts->split_pages : 0;
    if (sp_req < 0) return RQ_ERR_SHAPE;
    if (batch == 0) return RQ_OK;
    if (!k_cache || !v_cache || !q || !block_table || !seq_lens || !out) return RQ_ERR_NULL;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(q, 16)) return RQ_ERR_SHAPE;
    if ((int64_t)max_blocks_per_seq * 16 > (int64_t)1 << 30) return RQ_ERR_SHAPE;
    const int sp = sp_req > 0 ? sp_req : auto_split_pages(batch * num_heads, max_blocks_per_seq, true);
    if (!workspace) return RQ_ERR_NULL;
    if (workspace_bytes < bf16_ws(num_heads, head_dim, batch, max_blocks_per_seq, sp)) return RQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return RQ_ERR_SHAPE;
    Bf16Call c;
    c.H = num_heads; c.D = head_dim; c.nblk = num_blocks;
    c.kc = (const uint16_t *)k_cache; c.vc = (const uint16_t *)v_cache; c.q = (const uint16_t *)q;
    c.block_table = block_table; c.seq_lens = seq_lens; c.B = batch; c.max_blocks = max_blocks_per_seq;
    c.tail_k = (const uint16_t *)tail_k; c.tail_v = (const uint16_t *)tail_v;
    c.softmax_scale = softmax_scale; c.out = out; c.partials = (float *)workspace;
    c.split_pages = sp; c.nsplit = nsplit_of(max_blocks_per_seq, sp);
    c.ev_begin = opts ? (hipEvent_t)opts->event_main_begin : nullptr;
    c.ev_end = opts ? (hipEvent_t)opts->event_main_end : nullptr;
    c.stream = (hipStream_t)stream;
    return launch_bf16_decode(c) == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

rq_status rq_bf16_decode_attention(int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   const void *k_cache, const void *v_cache, const void *q,
                                   const int32_t *block_table, const int32_t *seq_lens, int32_t batch,
                                   int32_t max_blocks_per_seq, const void *tail_k, const void *tail_v,
                                   float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    return rq_bf16_decode_attention_ex(num_heads, head_dim, block_size, num_blocks, k_cache, v_cache, q,
                                       block_table, seq_lens, batch, max_blocks_per_seq, tail_k, tail_v,
                                       softmax_scale, out, workspace, workspace_bytes, nullptr, stream);
}

rq_status rq_bf16_write(int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                        void *k_cache, void *v_cache, const void *kv_new, const int64_t *slot_mapping,
                        int32_t num_tokens, void *stream) {
    if (num_heads < 1 || num_blocks < 1 || num_tokens < 0) return RQ_ERR_SHAPE;
    if (block_size != 16) return RQ_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 96 && head_dim != 128) return RQ_ERR_UNSUPPORTED;
    if (num_tokens == 0) return RQ_OK;
    if (!k_cache || !v_cache || !kv_new || !slot_mapping) return RQ_ERR_NULL;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(kv_new, 16)) return RQ_ERR_SHAPE;
    return launch_bf16_write(num_heads, head_dim, num_blocks, (uint16_t *)k_cache, (uint16_t *)v_cache,
                             (const uint16_t *)kv_new, slot_mapping, num_tokens, (hipStream_t)stream) == hipSuccess
               ? RQ_OK
               : RQ_ERR_HIP;
}

}  // extern "C"
