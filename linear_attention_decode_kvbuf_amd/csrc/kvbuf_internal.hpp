// Internal interface between the C-ABI layer (abi.cpp) and the kernel
// launchers (*.hip).  Not installed; the public interface is include/kvbuf.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvbuf.h"

namespace kvbuf {

// What one launch does to each (request, head) tile.
enum Mode : int32_t {
    MODE_DECODE = 0,       // append one token, output, advance (maybe fold)
    MODE_VERIFY = 1,       // append n drafts, n outputs, no advance
    MODE_DIRECT = 2,       // decode from the buffer alone (no state, no fold)
    MODE_FLUSH = 3,        // fold requests whose buffer holds >= m tokens
    MODE_COMMIT = 4,       // advance by accepted[b], fold when eager and full
    MODE_MATERIALIZE = 5,  // write the effective state elsewhere; change nothing
    MODE_RECURRENT = 6     // m = 0: read, update and write the state every token
};

// Kernel arguments, passed by value.  Pointers are device pointers.
struct TileParams {
    int32_t batch;  // B; workgroup w serves request w % B, head w / B
    int32_t H, block_size, blocks_per_req, m, num_blocks, num_slots;
    int32_t n;      // tokens appended per request by this call (decode 1, verify n)
    int32_t mode;   // Mode
    int32_t fuse;   // eager policy: fold inside decode / commit
    int32_t fold_chunk;  // tokens staged in LDS per fold round (0: this launch never folds)
    float scale;
    float* state;
    void* key;
    void* value;
    float* gate;
    const int32_t* slot;  // [B]
    int32_t* table;       // [B][blocks_per_req]: the requests' rows, written by head 0's workgroup
    int32_t* occ;         // [B]: the requests' occupancies, likewise
    int32_t* tmeta;       // [B][H][1 + blocks_per_req]: per-tile occupancy and row, read and advanced
    int32_t* err;
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    void* out;            // fp32, or bf16 when out_bf16 (store_out)
    int out_bf16;
    const int32_t* accepted;
    float* states_out;
    const int32_t* parent;  // tree drafts: [B][n] parent of each draft (-1 = the buffer), else null
    const int32_t* leaf;    // tree commit: [B] accepted leaf (-1 = none), else null
    int sparse;             // flush after a decode launch: fold only the full tiles of each group
};

// Launchers: each picks the template instance for (rule, d, io dtype) and
// enqueues one grid of B * H workgroups.  Return hipSuccess or the launch error.
// launch_chunk serves decode and verify; one-token calls with table rows of
// at most 64 positions (decode and one-draft verify of the linear, gated and
// per-channel rules) go to the split-role kernel (launch_decode), the rest to
// the general chunk kernel.  Exception: launches of at most kFewTiles tiles
// at d = 128, bf16, whose m the chunk kernel folds itself (decode_eligible).
hipError_t launch_chunk(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s);
hipError_t launch_decode(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s);
constexpr int64_t kFewTiles = 4096;
bool decode_eligible(int rule, int d, int io, int n, int cap, int m, int64_t tiles);
int decode_fold_limit(int rule, int d, int io);
hipError_t launch_fold(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s);
// Per-channel rule: decode over rows of more than 64 positions, verify of
// 1-8 drafts (chain or tree; parent != null).
hipError_t launch_channel(const TileParams& p, int d, int io, int batch, hipStream_t s);
// Per-request metadata into the per-tile copies (requests [count], or all
// B when null), and the comparison of the two.
hipError_t launch_admit(const TileParams& p, const int32_t* requests, int count, hipStream_t s);
hipError_t launch_check(const TileParams& p, hipStream_t s);
// Buffer-only decode (kvbuf_direct), every rule: one wave per tile.
hipError_t launch_direct(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s);
// Largest m that a decode launch of n tokens over `tiles` tiles folds itself
// (eager policy).
int chunk_fold_limit(int rule, int d, int io, int n, int cap, int m, int64_t tiles);
hipError_t launch_recurrent(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s);
// Verification with temporary states (m = 0) and its commit, temp
// [n][B][H][d][d] fp32.
hipError_t launch_verify_recurrent(const TileParams& p, int rule, int d, int io, float* temp, hipStream_t s);
hipError_t launch_commit_recurrent(const TileParams& p, int d, const float* temp, hipStream_t s);

// Head dims with compiled kernels (d_k == d_v).
inline bool supported_dim(int d) { return d == 16 || d == 64 || d == 128; }

constexpr int kMaxDrafts = 8;
constexpr int kFoldChunk = 32;  // most tokens staged in LDS per fold round
constexpr int kRawFoldChunk = 32;  // ... when staged as stored (bf16 rows take half the LDS)
constexpr int kMaxTableRow = 64;
// Most buffer positions per request (block_size * blocks_per_req): the
// per-position LDS tables of the chunk and fold kernels (pool rows, gates,
// scores of up to eight queries) are sized by it, and the parity tests cover
// buffers up to this length.
constexpr int kMaxCapacity = 512;

}  // namespace kvbuf
