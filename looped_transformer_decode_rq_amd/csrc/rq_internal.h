// Internal declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq.h"

namespace rq {

// Derived geometry of one layer's packed pool (see the format in rq.h).
struct Geom {
    int H, D, G, L, bs, nblk, meta, kvdt, msz;
    bool direct;                    // RQ_MODE_DIRECT: every loop on its own, no alpha
    int bits[RQ_MAX_LOOPS];
    int code_bytes[RQ_MAX_LOOPS];   // per record
    int rec[RQ_MAX_LOOPS];          // record bytes (16-aligned)
    int64_t loop_off[RQ_MAX_LOOPS + 1];
    int meta_bytes;                 // per record: bs * (D/G) * 2 * msz
    int64_t slab;                   // bytes per (block, head)
};

// Fills g from a layout; returns RQ_OK or the validation failure.
rq_status make_geom(const rq_layout *layout, Geom *g);

// Lanes per token used by the split-K kernels for a head dim.
inline int lanes_per_token(int D) { return D == 96 ? 2 : 4; }

// Per-(loop call, sequence, head) query record written by the query prep kernel:
// a 64-byte header (per lane slice: the fixed-point scale and the sum of the
// fixed-point values, for q and q'), then the 4-bit limbs of q (kQueryLimbs
// per channel: 24-bit fixed point) and of q' = R_K q (kRotLimbs: 20-bit).
constexpr int kQueryLimbs = 6;
constexpr int kRotLimbs = 5;
__host__ __device__ constexpr int qpack_bytes(int D) { return 64 + (kQueryLimbs + kRotLimbs) * D / 2; }
__host__ __device__ constexpr int partial_floats(int D) { return 2 + 2 * D; }
// Per-(query row, head) record of the chunked-prefill query prep: the sums
// of round(q 2^e) and of round(q' 2^e), 2^-e twice (floats), then the three
// base-256 digits of the fixed point q and of q' = R_K q, (D/4 + 15)/16 steps
// of 4 lane slots x 16 bytes each
__host__ __device__ constexpr int chunk_qrec_bytes(int D) { return 16 + 2 * 3 * 64 * ((D / 4 + 15) / 16); }

// Pages per split chosen when the caller passes 0: sized so that a launch
// has several rounds of resident workgroups (units = sequences x heads;
// per_split = one partial per split: multi-loop calls and the bf16 baseline).
int auto_split_pages(int units, int max_blocks, bool per_split);

constexpr int kSplitWaves = 4;     // waves (splits) per split-K workgroup
constexpr int kMaxSplitPages = 64; // pages per split: one block-table entry per lane
constexpr int kMinAutoSplitPages = 16;  // smallest split the automatic choice aims for
constexpr int kMaxMultiLoops = 8;  // loop calls (waves) per multi-loop workgroup

// Partials per (loop call, sequence, head) row: one per split workgroup of 4
// waves for a single loop call, one per split when several loops are decoded
// together (the multi-loop kernel).
int partials_per_row(int n_loops, int max_blocks, int split_pages);

// ------------------------------------------------------------------ launchers
struct DecodeCall {
    const Geom *g;
    const uint8_t *pool;
    int n;                        // loop calls in this request
    int loops[RQ_MAX_LOOPS];
    const void *q;
    const float *rot;
    const int32_t *block_table;
    const int32_t *seq_lens;
    int B, max_blocks;
    const void *tail_k, *tail_v;
    float softmax_scale;
    float *out;
    uint8_t *qpack;               // workspace: [n][B][H][qpack_bytes]
    float *partials;              // workspace: [n][B][H][nparts][partial_floats]
    int split_pages, nsplit, nparts;   // pages per split, splits, partials per row
    hipEvent_t ev_begin, ev_end;
    hipStream_t stream;
    // optional encode of the current tokens in the same launches (enc_T = 0: none)
    uint8_t *enc_pool;
    const void *enc_kv;
    const int64_t *enc_slots;
    int enc_T;
    // run the per-loop split kernel's streaming reference instead of the call
    // (one loop call; its per-workgroup checksums go to `partials`)
    bool stream_probe = false;
};

hipError_t launch_decode(const DecodeCall &c);

// Chunked prefill over the packed cache: C queries per sequence of one loop.
struct ChunkCall {
    const Geom *g;
    const uint8_t *pool;
    int loop, B, C, max_blocks;
    const void *q;                // [B][C][H][D] bf16
    const float *rot;
    const int32_t *block_table, *seq_lens;
    const void *chunk_k, *chunk_v;    // [B][C][H][D] bf16 or NULL
    float softmax_scale;
    float *out;                   // [B][C][H][D]
    uint8_t *qrec;                // workspace: [B*C][H][chunk_qrec_bytes]
    float *partials;              // workspace: [B*C][H][nsplit][partial_floats]
    int split_pages, nsplit;
    hipEvent_t ev_begin, ev_end;
    hipStream_t stream;
};

constexpr int kMaxChunk = 256;    // queries per sequence in one chunked call
constexpr int kMaxChunkSplit = 1024;   // pages per split of a chunked call

hipError_t launch_chunk(const ChunkCall &c);

struct EncodeCall {
    const Geom *g;
    uint8_t *pool;
    const void *kv_new;
    const float *rot;
    const int64_t *slots;
    int T;
    hipStream_t stream;
};

hipError_t launch_encode(const EncodeCall &c);

// One pass of the rotation fit over device-resident calibration rows (float64):
// y = R d per row, its group quantization, the squared error and M = sum yhat d^T.
constexpr int kFitBlocks = 64;     // workgroups of a pass (one partial M each)
struct FitPass {
    const float *x;                // [n][D] device
    int64_t n;
    int D, bits, G, meta;
    const double *r;               // [D][D] device
    double *mpart, *epart;         // workspace: [kFitBlocks][D][D], [kFitBlocks]
    double *m, *err;               // workspace: [D][D], [1]
    hipStream_t stream;
};
hipError_t launch_fit_pass(const FitPass &p);

struct Bf16Call {
    int H, D, nblk;
    const uint16_t *kc, *vc;
    const uint16_t *q;
    const int32_t *block_table, *seq_lens;
    int B, max_blocks;
    const uint16_t *tail_k, *tail_v;
    float softmax_scale;
    float *out;
    float *partials;              // [B][H][nsplit][2 + D]
    int split_pages, nsplit;
    hipEvent_t ev_begin, ev_end;
    hipStream_t stream;
};

hipError_t launch_bf16_decode(const Bf16Call &c);
hipError_t launch_bf16_write(int H, int D, int nblk, uint16_t *kc, uint16_t *vc,
                             const uint16_t *kv_new, const int64_t *slots, int T,
                             hipStream_t stream);

}  // namespace rq
