/*
 * la_decode.h -- exact decode-phase attention over a KV cache on MI355X
 * (gfx950), with the LeanAttention stream-K decomposition.
 *
 * The operation (xllm-io paper review of arXiv 2405.10480, §3.1 and §3.2;
 * LeanAttention talk summary, "Background"): for every request b and head h,
 * one query row q = q[b,h,:] attends over the n_b cached keys and values of
 * that request and head:
 *
 *     s_j = scale * (q . K_j)           j = 0 .. n_b - 1
 *     m   = max_j s_j
 *     l   = sum_j exp(s_j - m)
 *     out = sum_j exp(s_j - m) V_j / l
 *
 * No mask other than the length: the decode query sees the whole cache.
 *
 * How it is computed (same pages, §3.3-§3.5): the context of every head is cut
 * into LeanTiles of `tile_tokens` tokens; the tile iterations of all heads are
 * laid end to end and split into equal contiguous ranges over a persistent grid
 * of co-resident workgroups (each workgroup derives its own range from
 * per-request prefix sums passed with the launch, or reads tables a host-side
 * scheduler builds); each workgroup streams its tiles with an online softmax,
 * and partial
 * (m, l, Obar) results of heads that span several workgroups are merged inside
 * the same launch with the associative rescaling reduction
 *     f(x, y): m = max(m_x, m_y), l = e^{m_x-m} l_x + e^{m_y-m} l_y,
 *              Obar = e^{m_x-m} Obar_x + e^{m_y-m} Obar_y
 * by the workgroup that holds the head's first tile (its "host").
 *
 * Conventions for every entry point:
 *  - Device pointers: q, k_cache, v_cache, out and the optional outputs in
 *    la_opts. They must be 16-byte aligned. The caller owns them.
 *  - Host pointers: ctx_lens (B entries, each >= 1) and the la_schedule
 *    tables. ctx_lens is read before the call returns, so the caller may reuse
 *    it immediately. With la_opts.ctx_lens_device the lengths are a device
 *    array read by the kernel instead, and ctx_lens may be NULL.
 *  - Layouts: q is [B, H, d] (fp16 or bf16). K and V are packed per request:
 *    request b's block is [H, n_b, d] and starts at element
 *    H * d * sum_{b' < b} n_{b'}; for equal lengths this is [B, H, n, d]
 *    (the (batch, heads, seq_len, head_dim) layout of §7.4); la_opts.kv_stride
 *    selects a [B, H, S, d] cache with room for S >= n_b tokens per head
 *    instead. out is [B, H, d] fp32.
 *  - d must be 64 or 128. scale must be finite. One head's K (or V) block,
 *    n_b * d * 2 bytes, must not exceed 4 GiB (LA_EUNSUPPORTED otherwise).
 *  - Calls are asynchronous on `stream` (a hipStream_t; 0 is the null
 *    stream). Argument and launch errors are returned synchronously. A
 *    device-side wait that exceeds its bound sets an error word that
 *    la_sync_check() reports.
 *  - Nothing throws across this boundary. On failure la_last_error() returns a
 *    message for the calling thread.
 *  - Reproducibility: for a given kind, grid and tile size every sum and merge
 *    runs in a fixed order, so outputs are bitwise the same from call to call,
 *    with one exception. A single-head lean or pull workgroup whose CU holds
 *    more of its launch's workgroups than their fair share (other work taking
 *    CUs, or a CU-masked stream) reads K by whole rows, which adds each score's
 *    partial products in another order; outputs then stay within the usual
 *    tolerance, but their last bits depend on where the workgroups ran.
 *  - Workspaces (partials buffer, flags, schedule tables, pinned staging) are
 *    owned by the library, one per (device, stream), allocated on first use and
 *    freed by la_shutdown(). Calls on the same stream are ordered; calls from
 *    several host threads are serialised inside the library.
 *  - Types across the boundary are plain C: streams and events are passed as
 *    void* (a hipStream_t / hipEvent_t converts unchanged), and the dtype and
 *    kind travel as int holding an la_dtype / la_kind value, so that no HIP
 *    header and no enum size enters the ABI. The argument list of
 *    la_decode_bf16 / la_decode_f16 is exactly (q, k_cache, v_cache,
 *    ctx_lens, B, H, d, scale, out, stream); la_decode adds the dtype as a
 *    trailing argument, since a void* cannot carry the element type.
 */
#ifndef LA_DECODE_H
#define LA_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_EINVAL = 1,        /* bad argument: null pointer, size < 1, misaligned, ... */
    LA_EUNSUPPORTED = 2,  /* valid but not implemented: d not 64/128, too many tiles */
    LA_EHIP = 3,          /* a HIP runtime call failed */
    LA_ETIMEOUT = 4,      /* a device-side wait exceeded its bound (la_sync_check) */
    LA_ENOMEM = 5         /* workspace allocation failed */
} la_status;

typedef enum { LA_F16 = 0, LA_BF16 = 1 } la_dtype;

typedef enum {
    LA_KIND_LEAN = 0,         /* stream-K over a persistent grid, one launch */
    LA_KIND_FIXED_SPLIT = 1,  /* each head cut into num_splits pieces + a combine launch */
    LA_KIND_PER_HEAD = 2,     /* one workgroup per (request, head), whole context */
    LA_KIND_AUTO = 3,         /* one of the above, chosen from the shape (la_select) */
    LA_KIND_PULL = 4,         /* fixed chunks of the tile sequence pulled dynamically by a
                                 persistent grid */
    LA_KIND_CHUNKS = 5        /* the same chunks, one workgroup each (non-persistent) */
} la_kind;

/*
 * la_decode_bf16 / la_decode_f16: decode attention for bf16 or fp16 inputs,
 * lean schedule, default tile size and grid. Arguments as described above;
 * `stream` is a hipStream_t passed as void*.
 */
la_status la_decode_bf16(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* ctx_lens, int B, int H, int d, float scale,
                         float* out, void* stream);
la_status la_decode_f16(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* ctx_lens, int B, int H, int d, float scale,
                        float* out, void* stream);

/* Same as above with the input dtype as a trailing argument (la_dtype). */
la_status la_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* ctx_lens, int B, int H, int d, float scale,
                    float* out, void* stream, int dtype);

/*
 * Options for la_decode_ex. Zero-initialise (or call la_opts_init) and set
 * what you need.
 *   kind        la_kind. LA_KIND_AUTO resolves kind and (if grid is 0) the
 *               grid as la_select does, on the CUs the stream may use: on a
 *               stream created with a CU mask (hipExtStreamCreateWithCUMask)
 *               the grid rule counts the masked CUs, and a single-head lean
 *               pick becomes LA_KIND_PULL on one workgroup per CU of the
 *               device (grouped heads keep lean there: measured with 7/8 of
 *               the CUs, lean on their grid took 561 us on the grouped ragged
 *               batch where pull took 625, and pull 1264 us on 512k where
 *               lean on the device grid took 1574). It takes no tile_owner or
 *               cta_timestamps, since those depend on the kind
 *   tile_tokens LeanTile size in tokens; 0 = library default for d
 *   grid        lean: workgroups in the persistent grid; 0 = one per CU the
 *               stream may use (la_default_grid on a stream without a CU
 *               mask), except single heads on a stream with under 70% of the
 *               CUs, which keep la_default_grid (within what the stream's CUs
 *               hold): there two workgroups on a CU read faster than one
 *               per CU does. Every workgroup must be resident at once on those
 *               CUs, so a grid above la_max_grid scaled to the stream's
 *               share of the CUs (its mask's set bits over the device's
 *               CUs) -> LA_EINVAL
 *   num_splits  fixed split: pieces per head; 0 = smallest power of two with
 *               B*H*splits >= capacity, capped at 64
 *   cooperative lean: 1 = hipLaunchCooperativeKernel, which refuses a grid
 *               that cannot be co-resident; 0 = ordinary launch. Both cap the
 *               grid at la_max_grid, so every workgroup a host waits for can be
 *               resident; the cooperative form also guarantees it while other
 *               work shares the device, at the cost of a slower launch.
 *               Once lean calls have run on two or more streams of a device,
 *               the library also keeps the unfinished lean launches of all
 *               those streams within the co-resident capacity together (each
 *               counted as grid / capacity of its kernel on its stream's
 *               CUs; streams whose CU masks overlap only in part are not
 *               covered): a call whose grid
 *               does not fit beside the other streams' unfinished launches
 *               runs on the largest grid that does, or waits on the host for
 *               the oldest of them when none fits. Its outputs then follow the
 *               smaller grid's schedule (equal within tolerance, not bitwise).
 *               Graph replays and la_decode_noalloc calls are not counted.
 *   m_out, l_out     optional device [B*H] fp32: m (natural-log units, on
 *               scaled logits) and l of every head
 *   tile_owner  optional device int32 [I]: lean, pull and chunks kinds; entry
 *               i receives the workgroup that processed tile iteration i of
 *               the linearised schedule (for checking the schedule the kernel
 *               executed)
 *   cta_timestamps optional device uint64 [blocks*4], blocks = the grid of
 *               the call's first kernel (lean: min(grid, I), or the grid
 *               itself with ctx_lens_device; fixed split:
 *               B*H*num_splits, which must then be given; per head: B*H). Per
 *               workgroup: realtime clock (100 MHz) at entry and at exit, then
 *               XCC_ID << 32 | HW_ID of the CU it ran on, then -- kind lean,
 *               for a workgroup that hosts a split unit -- when its wait for
 *               the peers began and ended, in ticks after entry, as
 *               (end << 32) | begin; 0 for every other workgroup and kind
 *   ev_start, ev_stop optional hipEvent_t: recorded on `stream` right before
 *               the first and right after the last kernel of the call (the
 *               schedule table copy is outside this pair)
 *   kv_heads    grouped-query attention: K/V heads per request, dividing H
 *               (0 = H, plain multi-head attention). Query head h attends over
 *               K/V head h / (H / kv_heads); k_cache and v_cache are then
 *               packed as [kv_heads, n_b, d] per request while q and out keep
 *               H heads. Groups of more than 16 query heads stream their K/V
 *               head once per 16 query heads. With kv_heads < H the lean
 *               schedule's units (tables, tile_owner, grid) are
 *               (request, K/V head, block of 16 query heads).
 *   q_tokens    new tokens per request decoded together, as when a draft of
 *               several tokens is verified (0 or 1 = one token; at most 64).
 *               q is then [B, q_tokens, H, d] (token-major) and out
 *               [B, q_tokens, H, d] fp32, m_out/l_out [B*q_tokens*H]. The new
 *               tokens are the last q_tokens positions of each request's
 *               cache (their own K/V rows are already in it, so every
 *               ctx_lens[b] >= q_tokens, else LA_EINVAL), and token t attends
 *               causally to cache positions 0 .. ctx_lens[b] - q_tokens + t.
 *               A K/V head's query columns are then its H/kv_heads query
 *               heads times q_tokens, ordered (head, token); the schedule's
 *               units are (request, K/V head, block of 16 columns) whenever
 *               there is more than one column. The causal mask among the new
 *               tokens is a reading: the pages name combining the method with
 *               speculative decoding (xllm-io paper review, §7.4) and masked
 *               tokens as a case to qualify (siliconandsystems digest,
 *               "Exactness and numerical qualification") but fix no mask.
 *   chunk_tiles pull kinds: tiles per chunk; 0 = ceil(I / (8 G)), or
 *               ceil(I / (4 G)) for grouped units, with G the pull grid (or
 *               one workgroup per CU), and at least min(32, ceil(I / G)).
 *   host_tables lean kind: 1 = the host builds the schedule tables and copies
 *               them to the device on `stream` before the kernel; 0 = with up
 *               to 256 requests and 2^32-1 tokens in all, the per-request
 *               prefix sums of tiles and tokens travel in the kernel
 *               arguments and every workgroup derives its own segments with
 *               the same rules (no copy on the stream); with up to 1024
 *               requests only the lengths are copied and the launch derives
 *               the segments from them; else as 1. All give the same
 *               tile-to-workgroup map and the same output bits.
 *   kv_stride   K/V cache layout: 0 = packed per request (request b's block
 *               [Hk, n_b, d] at row Hk * sum_{b' < b} n_b'); > 0 = a cache of
 *               kv_stride rows per head, [B, Hk, kv_stride, d] (head h of
 *               request b starts at row (b * Hk + h) * kv_stride; only its
 *               first n_b rows are read, so a decode loop appends to it in
 *               place). Every n_b must be <= kv_stride (else LA_EINVAL).
 *   ctx_lens_device optional device int32 [B]: the context lengths, read by
 *               the kernel in the launch instead of from the host array
 *               (ctx_lens may then be NULL and is ignored). Nothing about the
 *               lengths passes through the host, so a launch captured into a
 *               HIP graph stays valid while a decode loop grows them on the
 *               device. Lean kind only (LA_KIND_AUTO means lean here), on a
 *               kv_stride cache (whose size
 *               bounds every read), up to 1024 requests, no tile_owner; the
 *               grid is `grid` (or the default) and workgroups beyond the tile
 *               iterations stay idle. Lengths outside [max(1, q_tokens),
 *               kv_stride] make the kernel compute nothing and la_sync_check
 *               return LA_EINVAL. Same tile map and output bits as the host
 *               lengths on the same grid. Each workgroup reads every length
 *               once at its start: writes to them must be ordered before the
 *               call (on its stream, or synchronised with it).
 *   shared_gpu  1 = the caller runs other work on the device at the same time
 *               (kernels of other streams that may hold CUs), the selector
 *               input "current GPU contention" of the siliconandsystems
 *               digest ("A useful control policy"). LA_KIND_AUTO (and
 *               la_select) then picks LA_KIND_PULL, on one workgroup per CU,
 *               wherever it would pick LA_KIND_LEAN: an equal static split
 *               waits for the workgroups that share a CU with other work,
 *               while chunks pulled from a counter follow the CUs that are
 *               free (the same digest, "The hardware-aware part"). Measured
 *               with 1/8 of the CUs taken, pull lost 3-10% against its own
 *               time on the whole device, lean on one workgroup per CU of
 *               the device 28-63%; alone on the device pull is 0-11% slower
 *               than lean. Per-head picks stay. Ignored with
 *               ctx_lens_device, where auto means lean. A stream confined to
 *               part of the CUs by a CU mask needs no flag: kind auto reads
 *               the mask (see kind). 0 = the launch has the device to itself
 *               (default).
 *
 * The pull kinds (siliconandsystems digest, "Exact softmax can be reduced in
 * pieces": workgroups pull the next piece of the global tile order instead of
 * holding a fixed split; "The hardware-aware part": persistent and
 * non-persistent scheduling). The tile sequence of the lean schedule is cut
 * into chunks of chunk_tiles tiles. LA_KIND_PULL: a persistent grid of `grid`
 * workgroups (0 = la_default_grid, at most 65536) takes chunks from an atomic
 * counter until none is left. LA_KIND_CHUNKS: one workgroup per chunk. A head
 * spread over several chunks leaves one partial record per chunk; its chunks
 * form groups of 16, the workgroup whose piece arrives last in a group folds
 * the group with f in chunk order, and the last group folds the groups in
 * order. The tree is fixed, so outputs are bitwise the same whichever
 * workgroup took which chunk. No workgroup ever waits for another (any grid
 * is safe, co-resident or not).
 * With kv_heads or q_tokens the chunks cut the grouped units' tiles, and the
 * grouped exchange (16 records per chunk side) must fit 2 GiB, else
 * LA_EUNSUPPORTED. tile_owner receives the workgroup that processed each
 * tile; cta_timestamps needs an explicit grid (pull: grid*4 entries) or
 * chunk_tiles (chunks: ceil(I / chunk_tiles)*4 entries).
 */
typedef struct la_opts {
    int dtype;
    int kind;
    int tile_tokens;
    int grid;
    int num_splits;
    int cooperative;
    float* m_out;
    float* l_out;
    int32_t* tile_owner;
    uint64_t* cta_timestamps;
    void* ev_start;
    void* ev_stop;
    int kv_heads;
    int q_tokens;
    int chunk_tiles;
    int host_tables;
    int kv_stride;
    const int32_t* ctx_lens_device;
    int shared_gpu;
} la_opts;

void la_opts_init(la_opts* opts);

/* Calls are asynchronous on `stream`. A stream that is being captured into a
 * HIP graph takes only the lean kind with its schedule derived in the launch
 * (ctx_lens_device, or host lengths within the in-launch limits and no
 * host_tables) as an ordinary launch (cooperative = 0), and only once an
 * earlier call on the stream has sized its
 * workspace for this grid and head dim: partials and flags live in a
 * per-stream workspace that growing would reallocate, and table uploads go
 * through staging buffers that later calls reuse. Anything else is refused
 * with LA_EUNSUPPORTED before anything is enqueued. A captured launch with
 * host lengths replays those lengths. The graph uses the capturing stream's
 * workspace, which that stream's later calls share: replay it on that stream
 * (or order it against the stream's other work). Once a launch has been
 * captured on a stream, a later call there that needs a larger workspace
 * allocates new buffers and keeps the old ones until la_shutdown, so the
 * graph stays valid; la_shutdown ends every captured graph's validity. */
la_status la_decode_ex(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* ctx_lens, int B, int H, int d, float scale,
                       float* out, void* stream, const la_opts* opts);

/*
 * la_decode_noalloc: la_decode_ex for callers that cannot allocate -- code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It calls no hipMalloc, hipFree or other allocating routine and
 * uses no per-stream workspace: the lean exchange (partial records, flags and
 * control words) lives in a fixed array of device memory, one per GPU, that
 * the library holds until the process ends: 8 MiB of partial records plus
 * 24832 bytes of flags, control words and per-CU workgroup counters.
 *
 * Arguments and options are those of la_decode_ex, restricted to:
 *   - kind LA_KIND_LEAN (LA_EINVAL otherwise);
 *   - a schedule derived in the launch: host lengths for at most 256 requests
 *     and 2^32 - 1 tokens in all with host_tables = 0, or ctx_lens_device
 *     (LA_EUNSUPPORTED otherwise);
 *   - a grid of at most 2048 workgroups whose partial records fit the 8 MiB:
 *     grid * (d + 4) * 4 bytes with one query column per K/V head, 16 times
 *     that with kv_heads < H or q_tokens > 1 -- at d = 128 that allows 992
 *     grouped workgroups (LA_EUNSUPPORTED otherwise);
 *   - while `stream` is being captured: cooperative = 0, and an earlier
 *     call of this entry point on the device (the first one sets up the
 *     array and is refused under capture).
 * Every rejection happens before anything is enqueued. For the same options
 * the outputs are bitwise those of la_decode_ex (same kernels, same schedule).
 *
 * The first call on a device (the current one) looks up the array's address
 * and enqueues one small kernel on `stream` that clears its control words
 * and flags; every later call enqueues only the attention kernel. All calls
 * on a GPU share that GPU's array, which keeps the last call's contents:
 * calls that overlap on one GPU -- on streams not ordered with each other,
 * graph replays included -- race and give undefined results, so order them.
 * A wait that gives up is reported, and the array's error word cleared, by
 * la_sync_check on any stream of the device.
 */
la_status la_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* ctx_lens, int B, int H, int d, float scale,
                            float* out, void* stream, const la_opts* opts);

/*
 * la_select_for: the kind and lean grid that LA_KIND_AUTO uses, for a device
 * with `cus` compute units whose lean kernel fits `coresident` workgroups at
 * once. Host only: reads nothing from a device. A shape-driven control policy
 * in the spirit of the siliconandsystems digest ("A useful control policy"),
 * built on the reductions of xllm-io paper review §4.3:
 *   grid  = 2*cus if B * units >= 2*cus (at least two heads per CU, whose
 *           switches a second workgroup per CU hides) and the heads average
 *           fewer than 128 tiles (sum over b of ceil(n_b / tile) < 128 * B),
 *           else cus; capped at coresident. units = H, or with kv_heads /
 *           q_tokens the grouped units (K/V head x block of 16 query columns).
 *   kind  = LA_KIND_PER_HEAD if the lean schedule on that grid splits no
 *           head (every workgroup holds whole heads) and, for grouped units,
 *           they average at least 4 tiles; also LA_KIND_PER_HEAD, with one query column per
 *           K/V head, when every head's K and V fit in 256 KiB
 *           (max n_b * 4 * d bytes) and B * H <= cus (a latency-bound launch
 *           that runs every head at once); else LA_KIND_LEAN.
 *           LA_KIND_FIXED_SPLIT is never chosen.
 * tile_tokens 0 = la_default_tile(d). Returns LA_EINVAL on bad arguments
 * (as la_decode_ex validates kv_heads, q_tokens, d), LA_EUNSUPPORTED if the
 * iteration count does not fit in int32.
 */
la_status la_select_for(const int32_t* ctx_lens, int B, int H, int d, int kv_heads, int q_tokens,
                        int tile_tokens, int cus, int coresident, int* kind, int* grid);

/* la_select: la_select_for on the current device, with d, dtype, kv_heads,
 * q_tokens and tile_tokens taken from `opts` (which may be null: defaults),
 * for a stream that may use every CU (LA_KIND_AUTO on a CU-masked stream
 * decides on that stream's CUs; see la_opts.kind).
 * With opts->shared_gpu set, a lean pick becomes LA_KIND_PULL on the default
 * pull grid (one workgroup per CU), as LA_KIND_AUTO does then. */
la_status la_select(const int32_t* ctx_lens, int B, int H, int d, const la_opts* opts, int* kind,
                    int* grid);

/*
 * la_schedule_dims: sizes of the stream-K tables for a batch, host only.
 * Outputs: *iters = I = H * sum_b ceil(n_b / tile_tokens); *grid_used =
 * min(grid, I); *max_rows = grid_used + B*H (an upper bound on segments).
 * Returns LA_EUNSUPPORTED if I does not fit in int32.
 */
la_status la_schedule_dims(const int32_t* ctx_lens, int B, int H, int tile_tokens, int grid,
                           int64_t* iters, int* grid_used, int* max_rows);

/*
 * la_schedule: the host-side stream-K scheduler (§3.4-§3.5), host only.
 * Iterations are ordered request, then head, then tile; CTA c gets
 * [c*q + min(c, r), (c+1)*q + min(c+1, r)) with q = I / G, r = I mod G.
 * Outputs (caller-allocated host arrays):
 *   cta_begin [G+1]   iteration bounds per CTA
 *   cta_seg   [G+1]   segment-row bounds per CTA
 *   seg       [max_rows * 6]  rows (cta, u = b*H + h, t0, t1, host, finishing)
 *   host_cta, last_cta [B*H]  CTA holding each head's first and last tile
 *   *n_seg            number of rows written
 * `grid` is the requested G; the tables use min(grid, I) (la_schedule_dims).
 */
la_status la_schedule(const int32_t* ctx_lens, int B, int H, int tile_tokens, int grid,
                      int32_t* cta_begin, int32_t* cta_seg, int32_t* seg, int max_rows,
                      int* n_seg, int32_t* host_cta, int32_t* last_cta);

/* Default LeanTile size (tokens) for head dim d; 0 if d is unsupported. */
int la_default_tile(int d);

/*
 * Co-resident workgroup capacity of the lean kernel for (d, dtype) on the
 * current device: occupancy per CU times the CU count. Returns <= 0 on error.
 * This is the bound on la_opts.grid for calls with one query column per K/V
 * head; calls with kv_heads < H or q_tokens > 1 run the grouped kernel, whose
 * bound is la_max_grid_grouped. On a CU-masked stream the bound is the
 * occupancy per CU times the stream's CUs.
 */
int la_max_grid(int d, int dtype);

/* The same for the grouped (MFMA) lean kernel. */
int la_max_grid_grouped(int d, int dtype);

/*
 * Grid the lean kind uses when la_opts.grid is 0: one workgroup per CU on the
 * current device (never more than la_max_grid). On a CU-masked stream the
 * call's default follows la_opts.grid's description. Returns <= 0 on error.
 */
int la_default_grid(int d, int dtype);

/*
 * Synchronises `stream` and reads the sticky device error word of its
 * workspace, and that of the device's la_decode_noalloc array. LA_EINVAL if lengths read on the device (ctx_lens_device) were
 * out of range, LA_ETIMEOUT if a device-side wait exceeded its bound, since
 * the last check (the word is then cleared); LA_EHIP if the stream reports an
 * error; LA_OK otherwise. An error affects only the launch that raised it:
 * later launches are computed normally whether or not this is called.
 */
la_status la_sync_check(void* stream);

/*
 * Bound, in microseconds, on one device-side wait of a host workgroup for a
 * peer's partial, for calls enqueued after this one (0 restores the default,
 * 2 s). A wait that runs out -- and every other wait of the same launch after
 * it -- gives up and raises the error word reported by la_sync_check(); the
 * output of that launch is then undefined. Later launches are not affected:
 * flags hold the epoch of the launch that raised them, so a late peer's flag
 * never satisfies a later launch's wait. Small bounds force this path in
 * tests.
 */
void la_set_wait_limit_us(uint32_t us);

/*
 * Measurement aid, not part of attention: reads the device buffer `src`
 * (16-byte aligned, `bytes` long) once on `stream` with the load pattern of
 * the attention kernels and nothing else, so that the achievable read
 * bandwidth of the device can be set next to the attention kernels' (the
 * peak of the data sheet is not reachable). Each of `grid` workgroups reads
 * one contiguous chunk as two halves side by side, like a K and a V cache:
 * the first half as 64 bytes of each of 16 rows of 256 bytes per wave
 * instruction, the second as contiguous 1 KiB per wave instruction, with 16
 * non-temporal 16-byte loads per lane in flight.
 * grid 0 = one workgroup per CU. Reads the largest multiple of 64 KiB per
 * workgroup that fits; that byte count is stored in *bytes_read. `sink` is a
 * device word that the kernel may write (it only keeps the loads from being
 * optimised away). LA_EINVAL for null or misaligned pointers, a grid outside
 * [1, 65535], or fewer than 64 KiB per workgroup. Asynchronous on `stream`.
 */
la_status la_stream_read(const void* src, size_t bytes, int grid, uint32_t* sink, void* stream,
                         size_t* bytes_read);

/* Message for the last failing call on this thread ("" if none). */
const char* la_last_error(void);

/* Frees every library-owned workspace after synchronising its stream. */
void la_shutdown(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_DECODE_H */
