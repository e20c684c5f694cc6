// Internal interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;     // workgroup size
constexpr int kRows = 8;                  // K/V rows each lane group loads per step

// Rows processed by one workgroup per step (the natural LeanTile size):
// a row of d halves is d/8 lanes of 16 bytes, so a wave holds 512/d rows per
// load and the workgroup 2048/d; each lane group takes kRows of them.
constexpr int chunk_rows(int d) { return (2048 / d) * kRows; }
// Single-head ranges of at least this many steps (of chunk_rows(d) rows) read
// K in 16-row blocks, shorter ones by whole rows.
constexpr int kBlockMinSteps = 8;

// Stride in floats of one partial record (Obar[d], m, l), padded to 16 bytes.
constexpr int part_stride(int d) { return d + 4; }

// Where a lean workgroup finds its segments: in tables built and uploaded by
// the host (kSrcTables), or -- for up to kInlineB requests -- derived by the
// workgroup itself with the host scheduler's partition and unit walk, from
// per-request prefix sums carried in the kernel arguments (kSrcArgs, up to
// 2^32 - 1 tokens in all) or from context lengths it reads from device memory
// (kSrcDevice: nothing about the lengths passes through the host, so a
// captured launch stays valid while they change).
constexpr int kInlineB = 256;
// Most requests whose lengths the lean kernels read from device memory.
constexpr int kMaxDeviceB = 1024;
constexpr int kSrcTables = 0, kSrcArgs = 1, kSrcDevice = 2;

// Device error word bits.
constexpr uint32_t kErrTimeout = 1u;     // a wait gave up
constexpr uint32_t kErrLengths = 2u;     // device context lengths out of range

// Control block of a lean exchange (partials and flags), 256 bytes of
// uint32 words, each on its own 64-byte line:
//   err    sticky error bits, cleared only by the host (la_sync_check)
//   epoch  epoch of the last launch that completed on this exchange
//   exit   workgroups of the current launch that have finished (zero between
//          launches: the last one out resets it)
//   abort  epoch of a launch in which a wait gave up
// A launch's epoch is the completed epoch plus one (never 0). Peers raise
// their flag to the launch's epoch and hosts wait for exactly that value, so
// a flag left from an earlier launch -- a late peer whose host gave up --
// never counts, and a give-up makes the other waits of the same launch give
// up at once without touching later launches. Flags need no lowering.
constexpr int kCtlErr = 0, kCtlEpoch = 16, kCtlExit = 32, kCtlAbort = 48;
// After those words: how many workgroups of the running lean launch each CU
// holds, one word per CU slot (XCC_ID & 15) * 256 + HW_ID bits 15:8 (CU, SH
// and SE ids). Every workgroup adds one at entry and takes it back at exit,
// so the words are zero between launches.
constexpr int kCtlCu = 64, kCuSlots = 4096;
constexpr int kCtlWords = kCtlCu + kCuSlots;

struct SchedArgs {
    const int4* seg;           // tables: [nseg] (u, t0, t1, host | finishing << 1)
    const int32_t* cta_seg;    // tables: [G+1]
    const int32_t* cta_begin;  // tables: [G+1]
    const int32_t* last_cta;   // tables: [B*U]
    const int32_t* ctx;        // tables: [B] n_b
    const int64_t* tok_off;    // tables: [B] sum_{b'<b} n_b'
    const int32_t* dlens;      // device: [B] n_b
    int src;                   // kSrcTables, kSrcArgs or kSrcDevice
    int B;                     // requests
    int U;                     // schedule units per request
    int G;                     // workgroups launched
    int L;                     // device: tile tokens
    int n_min, n_max;          // device: valid n_b range (new tokens per request, cache rows per head)
    int32_t tp[kInlineB + 1];  // inline: tiles of the requests before b (exclusive prefix)
    uint32_t tok[kInlineB + 1];// inline: tokens of the requests before b
};

struct LeanArgs {
    const uint16_t* q;         // [B*H, d]
    const uint16_t* k;         // packed rows [H * sum n_b, d]
    const uint16_t* v;
    float* out;                // [B*H, d]
    float* m_out;              // optional [B*H]
    float* l_out;              // optional [B*H]
    SchedArgs sched;
    float* part;               // [G * part_stride(d)]
    uint32_t* flags;           // [G]: epoch of the launch whose record each holds
    uint32_t* ctl;             // control block (kCtl* words)
    int32_t* tile_owner;       // optional [I]
    uint64_t* ts;              // optional [G*4]: start, end, XCC_ID/HW_ID, host wait
    int H;
    int L;                     // tile tokens
    int kv_stride;             // 0: K/V packed per request; else rows per head of a [B, H, kv_stride, d] cache
    float sl2e;                // scale * log2(e)
    uint64_t wait_ticks;       // 100 MHz clock ticks before a wait gives up
    int cu_fair;               // ceil(grid / CUs): a CU holding more of the launch's workgroups is crowded
    int rotate;                // 1: long ranges start at a per-workgroup step (uniform contexts)
};

struct SplitArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    float* out;                // per-head kernel: output; split kernel: unused
    float* m_out;
    float* l_out;
    const int32_t* ctx;
    const int64_t* tok_off;
    float* part;               // split kernel: [B*H*splits * part_stride(d)]
    uint64_t* ts;              // optional [blocks*4]: start, end, XCC_ID/HW_ID, 0
    int H;
    int L;
    int kv_stride;             // as in LeanArgs
    int splits;
    float sl2e;
};

struct CombineArgs {
    const float* part;
    float* out;
    float* m_out;
    float* l_out;
    int splits;
};

// Grouped-query heads and several new tokens per request: the g = H / Hk
// query heads sharing a K/V head, times the Nq new tokens, are that K/V head's
// g * Nq query columns. The schedule unit is (request, K/V head, block of up
// to 16 columns); a unit produces 16 partial records (one per column) of
// part_stride(d) floats.
struct GqaArgs {
    const uint16_t* q;         // [B*Nq*H, d]
    const uint16_t* k;         // packed rows [Hk * sum n_b, d]
    const uint16_t* v;
    float* out;                // [B*Nq*H, d]
    float* m_out;              // optional [B*Nq*H]
    float* l_out;              // optional [B*Nq*H]
    const int32_t* ctx;        // [B] (fixed split, per unit, pull)
    const int64_t* tok_off;    // [B]
    SchedArgs sched;           // lean (units instead of heads)
    float* part;               // lean: [G*16]; split: [units*splits*16] records
    uint32_t part_bytes;       // size of the lean exchange buffer (bounds its accesses)
    uint32_t* flags;           // lean: [G], as in LeanArgs
    uint32_t* ctl;             // lean: control block (kCtl* words)
    int32_t* tile_owner;
    uint64_t* ts;              // optional [blocks*4], as in LeanArgs
    int H;                     // query heads per request
    int Hk;                    // K/V heads per request
    int g;                     // H / Hk
    int Nq;                    // new tokens per request
    int cols;                  // query columns per K/V head: g * Nq
    int QB;                    // column blocks of 16 per K/V head: ceil(cols / 16)
    int L;
    int kv_stride;             // 0: K/V packed per request; else rows per K/V head ([B, Hk, kv_stride, d])
    int splits;
    float sl2e;
    uint64_t wait_ticks;
    // dynamic pull (as in PullArgs; part then holds [2 * nchunks * 2 * 16] records)
    const int32_t* head_start;
    const int32_t* chunk_head;
    uint32_t* gcount;
    uint32_t* arrive;
    uint32_t* pull;
    int C;
    int I;
    int nchunks;
    int dynamic;
};

// Dynamic tile pull. The linearised tile sequence (as in the lean schedule)
// is cut into fixed chunks of C tiles; workgroups take chunks from an atomic
// counter (dynamic) or one chunk each (grid = nchunks). A head spanning
// several chunks leaves one partial record per chunk, at slot (chunk, side):
// side 0 if its piece starts the chunk, else 1. The head's chunks form groups
// of kMergeFanIn: the last piece of a group to arrive (group counter at the
// slot of the group's first chunk) folds the group and stores the group's
// record at that slot of the second level; the last group (per-head counter)
// folds the group records and writes the output. Nothing ever waits.
constexpr int kMergeFanIn = 16;
struct PullArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    float* out;
    float* m_out;
    float* l_out;
    const int32_t* ctx;        // [B]
    const int64_t* tok_off;    // [B]
    const int32_t* head_start; // [BU + 1]: first tile iteration of each head; [BU] = I
    const int32_t* chunk_head; // [nchunks]: head holding the chunk's first tile
    float* part;               // [2 levels * nchunks * 2 * part_stride(d)]
    uint32_t* gcount;          // [nchunks * 2] group counters, zero at launch and at exit
    uint32_t* arrive;          // [BU], zero at launch and at exit
    uint32_t* pull;            // [2]: next chunk, workgroups done; zero at launch and at exit
    int32_t* tile_owner;       // optional [I]
    uint64_t* ts;              // optional [grid*4]
    int H;
    int L;
    int kv_stride;             // as in LeanArgs
    int C;                     // tiles per chunk
    int I;                     // tile iterations
    int nchunks;
    int dynamic;               // 1: pull chunks from the counter; 0: chunk = blockIdx.x
    float sl2e;
    uint32_t* ctl;             // dynamic pull: the stream's lean control block (its per-CU counters)
    int cu_fair;               // > 0: as in LeanArgs
};

const void* lean_kernel_ptr(int dtype, int d, int src);
uint64_t stream_read_unit();   // bytes per workgroup per loop trip of stream_read_kernel
hipError_t launch_stream_read(const void* src, uint64_t chunk, int grid, uint32_t* sink,
                              hipStream_t s);
hipError_t launch_pull(int dtype, int d, const PullArgs& a, int grid, hipStream_t s);
const void* lean_gqa_kernel_ptr(int dtype, int d, int src);
hipError_t launch_lean_gqa(int dtype, int d, const GqaArgs& a, int grid, hipStream_t s,
                           bool cooperative);
hipError_t launch_split_gqa(int dtype, int d, const GqaArgs& a, int blocks, hipStream_t s);
hipError_t launch_combine_gqa(int d, const GqaArgs& a, int units, hipStream_t s);
hipError_t launch_per_head_gqa(int dtype, int d, const GqaArgs& a, int units, hipStream_t s);
hipError_t launch_pull_gqa(int dtype, int d, const GqaArgs& a, int grid, hipStream_t s);
hipError_t launch_lean(int dtype, int d, const LeanArgs& a, int grid, hipStream_t s,
                       bool cooperative);
hipError_t launch_split(int dtype, int d, const SplitArgs& a, int blocks, hipStream_t s);
hipError_t launch_combine(int d, const CombineArgs& a, int heads, hipStream_t s);
hipError_t launch_per_head(int dtype, int d, const SplitArgs& a, int heads, hipStream_t s);

}  // namespace la
