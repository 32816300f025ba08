/*
 * ar.h -- C ABI of the MI355X (gfx950) per-GPU reduction kernels of a custom
 * all-reduce: one-shot, two-shot (reduce-scatter, flag barrier, all-gather)
 * and the LL / LL128 flag-packed protocols.
 *
 * Sources (page titles as printed):
 *  [CAR]  "0-custom-all-reduce" (obnotes, Inference/sglang/jit_kernel): the
 *         one-shot pull kernel, 实现 steps 1-6 -- a pointer table with one
 *         mapped buffer per GPU, 16-byte vectors, fp32 accumulation in GPU
 *         index order, one round-to-nearest cast, 16-byte alignment, the
 *         two-shot divisibility requirement, start/end synchronisation, and
 *         the rule that the output must not be a buffer others still read.
 *  [NCCL] "集合通信：NCCL 的算法、协议与推理框架的定制 all-reduce"
 *         (anrans.github.io, serving/comm/nccl): 算法 (one-shot, two-shot),
 *         协议 table (LL, LL128, Simple), 练习 3 (registered buffers).
 *  [MGPU] "多 GPU 与 NCCL" (anrans.github.io, cuda/tools/multi-gpu): 集合通信
 *         table, all-reduce = reduce-scatter + all-gather.
 *  [SMF]  "Sm-free Allreduce using sharp" (obnotes, Big-Feature): 0 前言 --
 *         moving the data with asynchronous copies instead of SM kernels.
 *
 * Conventions shared by every entry point
 *  - n emulated ranks, 2 <= n <= AR_MAX_RANKS ([CAR] supports up to 16 GPUs).
 *    Rank i's buffer is the i-th pointer of a pointer table; on one GPU the
 *    n "registered buffers" are n separate device allocations.  Pointer
 *    tables are host arrays; they are copied by value into the kernel
 *    arguments, so they may be freed as soon as the call returns.
 *  - Every data pointer is device memory of the current HIP device, 16-byte
 *    aligned ([CAR] step 1: 128-bit accesses).  All memory is caller-owned;
 *    the library never allocates on these paths.
 *  - numel counts elements per rank, at most 2^34 bytes (16 GiB) per rank
 *    (else AR_ERR_ARG); dtype is an ar_dtype.  Sums are taken in
 *    fp32, rank 0 first, starting from +0.0, and rounded once to the output
 *    type with round-to-nearest-even ([CAR] step 4).  Results are therefore
 *    identical bit for bit on every rank and on every call.
 *  - stream is a hipStream_t (NULL = the null stream).  Every call validates
 *    its arguments synchronously, then enqueues its kernels and returns.
 *    A call that returns an error enqueued nothing.
 *  - Written buffers (outputs, segments, wire buffers) must not overlap any
 *    other buffer of the same call (AR_ERR_ALIAS): [CAR] step 5 -- without a
 *    staging copy the output must be a fresh buffer, not one a peer reads.
 *  - Waits on flags are bounded by a wall-clock budget (ar_set_poll_timeout_ns).
 *    A wait that runs out does not hang: the kernel writes
 *    AR_ERR_TIMEOUT | phase << 8 | rank << 16 into status word 0 of the flag
 *    region (first error wins), the index of the tile or line it waited on
 *    into word 1, skips the work that depended on it, and exits normally.
 *    Read the status after synchronising the stream.
 *  - Reuse: a producer may overwrite a segment or wire buffer for step s+1
 *    only after every consumer has finished step s (the end synchronisation
 *    of [CAR] step 6).  On one GPU, stream order gives this.
 *  - Calls that share a flag region must be ordered, for example by issuing
 *    them on one stream; auto step ids in particular rely on each call seeing
 *    the epochs the previous one left.  Calls on one flag region that overlap
 *    in time race.
 */
#ifndef AR_H
#define AR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AR_MAX_RANKS 16
/* Flag slots per rank in the two-shot barrier region (see ar_flag_bytes). */
#define AR_SLOTS_PER_RANK 1024
/* Epoch copies per rank for auto step ids: one per wavefront of an auto-step
 * two-shot launch, whose grid is two 256-lane workgroups per CU (see
 * ar_flag_bytes). */
#define AR_EPOCH_COPIES 4096

typedef enum {
    AR_OK = 0,
    AR_ERR_ARG = 1,       /* null pointer, n out of range, numel 0, LL step 0, bad dtype/proto/ranks */
    AR_ERR_ALIGN = 2,     /* a data pointer is not 16-byte aligned */
    AR_ERR_DIVISIBLE = 3, /* two-shot: numel % n != 0 or a segment is not a whole number of 16-byte vectors */
    AR_ERR_ALIAS = 4,     /* a written buffer overlaps another buffer of the call */
    AR_ERR_TIMEOUT = 5,   /* asynchronous only: a flag wait ran out (status word of the flag region) */
    AR_ERR_HIP = 6,       /* a HIP runtime call failed (launch, device query, cooperative launch) */
    AR_ERR_SIZE = 7       /* ar_twoshot_noalloc: more than AR_NOALLOC_MAX_BYTES per rank */
} ar_status;

typedef enum { AR_F32 = 0, AR_BF16 = 1 } ar_dtype;
typedef enum { AR_PROTO_LL = 0, AR_PROTO_LL128 = 1 } ar_proto;

/* Phases reported in bits 8..15 of a timeout status word. */
#define AR_PHASE_TWOSHOT_AG 1
#define AR_PHASE_LL 2
#define AR_PHASE_LL128 3
#define AR_PHASE_RMSNORM 4

/* Bytes of the flag region used by the two-shot barrier and the LL status
 * word for up to n ranks: a 128-byte status line (word 0 status, word 1
 * detail), then AR_SLOTS_PER_RANK 32-bit arrival slots per rank, then
 * AR_EPOCH_COPIES groups of n 32-bit epoch copies (auto step ids; group w
 * belongs to wavefront w of an auto launch, word r of it to rank r): in all
 * 128 + n * (AR_SLOTS_PER_RANK + AR_EPOCH_COPIES) * 4 bytes.  Returns 0
 * if n is out of range. */
size_t ar_flag_bytes(int n);

/* Wire bytes for one rank's message of nbytes bytes ([NCCL] 协议 table):
 * LL    -- 8-byte lines, each 4 data bytes then a 32-bit flag: 8*ceil(nbytes/4);
 * LL128 -- 128-byte lines, each 120 data bytes then a 64-bit flag:
 *          128*ceil(nbytes/120).
 * The last line's data bytes past the message are zero.  Returns 0 on a bad
 * proto. */
size_t ar_ll_wire_bytes(int proto, size_t nbytes);

/* Budget for every device-side flag wait, in nanoseconds (default 1 s).
 * Process-wide; read at launch time.  0 restores the default. */
void ar_set_poll_timeout_ns(uint64_t ns);
uint64_t ar_get_poll_timeout_ns(void);

/* Short English name of a status code (static storage). */
const char* ar_status_string(int status);

/* One-shot all-reduce, one GPU's share ([CAR] 实现 steps 1-5; [NCCL] 算法,
 * one-shot): out[k] = round(sum over i = 0..n-1 of in[i][k]) for k < numel.
 *  in    : host array of n device pointers, each numel elements of dtype.
 *  out   : device buffer of numel elements; must not overlap any in[i].
 * Reads n*S bytes and writes S bytes (S = numel * element size).  Any numel
 * >= 1 is accepted; a partial last vector is handled element by element and
 * no byte past numel is read or written.
 * Errors: AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_ALIAS, AR_ERR_HIP. */
int ar_oneshot(const void* const* in, int n, void* out, size_t numel, int dtype, void* stream);

/* One-shot all-reduce fused with a residual add and RMSNorm.  [NCCL] names
 * such a fused kernel among the inference frameworks' paths (all-reduce +
 * RMSNorm, the FlashInfer kernel SGLang integrates) without defining it; this
 * library's reading, for rows x hidden elements stored row-major:
 *   h[i][k] = (ar_oneshot's fp32 fold of the ranks' element, rank order)
 *             + residual[i][k]                      (one more fp32 add)
 *   residual_out[i][k] = h rounded once to dtype
 *   out[i][k] = round(h * (1 / sqrt(sum over k of h^2 / hidden + eps))
 *                     * weight[k]), in fp32.
 *  in           : host array of n device pointers, rows * hidden elements each.
 *  residual     : rows * hidden elements; residual_out may be the same buffer
 *                 (updated in place) but may not otherwise overlap anything.
 *  weight       : hidden elements, the same for every row.
 *  out          : rows * hidden elements; may not overlap any other buffer.
 *  workspace    : NULL, or ar_rmsnorm_workspace_bytes() bytes, 16-byte
 *                 aligned and zeroed before its first use, owned by one call
 *                 site (calls sharing it must be ordered).  With it, few
 *                 heavy rows (rows * ceil(vectors per row / 64) <= 512 and
 *                 (n + 1) * hidden * element size >= 128 KiB: a decode
 *                 step's tokens) are split over a fixed grid of one-wavefront
 *                 workgroups that exchange their partial sums of squares
 *                 through it; its step ids advance by themselves, so the call
 *                 may be captured once into a graph.
 *                 A part that waits longer than the poll budget writes
 *                 AR_ERR_TIMEOUT | AR_PHASE_RMSNORM << 8 to its first word
 *                 (detail word: the row) and leaves that part of out unwritten.
 *  hidden * element size must be a multiple of 16 and at most 64 KiB
 *  (32768 bf16 / 16384 fp32 elements); eps >= 0 and finite.
 * residual_out matches the oracle bit for bit; out is fp32 arithmetic whose
 * sum of squares is taken in a tree, within one unit in the last place of
 * the correctly rounded value.  Reads (n + 1) * S + hidden * element size
 * bytes and writes 2 * S (S = rows * hidden * element size).
 * Errors: AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_DIVISIBLE, AR_ERR_ALIAS, AR_ERR_HIP. */
size_t ar_rmsnorm_workspace_bytes(void);
int ar_oneshot_rmsnorm(const void* const* in, int n, const void* residual, const void* weight, void* residual_out,
                       void* out, size_t rows, size_t hidden, float eps, int dtype, uint32_t* workspace,
                       void* stream);

/* The same op in two-shot form ([NCCL] 算法, two-shot; the fused op as read
 * for ar_oneshot_rmsnorm).  The reduce-scatter owns whole rows: rank r's
 * group is rows [r G, (r+1) G), G = rows / n, so the rank finishes the norm
 * of its rows alone.  Two forms, chosen by size (the same for every rank's
 * launch of a step):
 *  - heavy rows, few per rank (n + 1 streams of at least 128 KiB a row,
 *    G < 256): each row is cut into parts of 64 16-byte vectors, one
 *    wavefront each, that exchange their partial sums of squares through
 *    8-byte {value, step id} slots in the rank's segment; a part writes its
 *    results (its own outputs and the segment's copies), then, once those
 *    stores are complete, its done flag (the step id) in the segment; the
 *    all-gather copies a peer's part once its done flag holds the step;
 *  - otherwise a workgroup per row (the code of ar_oneshot_rmsnorm's
 *    workgroup-per-row path), each tile of rows published with an arrival
 *    slot in the flag region; the all-gather copies a tile once its slot
 *    holds the step.
 * Each form's results are identical to ar_oneshot_rmsnorm's on the same kind
 * of path.
 *  in           : n device pointers, rows * hidden elements each.
 *  residual     : n device pointers, rank r's copy of the residual stream
 *                 (rows * hidden elements); only ranks [r0, r1) are read.
 *  weight       : hidden elements.
 *  seg          : n device pointers, ar_rmsnorm_segment_bytes(n, rows,
 *                 hidden, dtype) bytes each, zeroed before their first use
 *                 (their slots and flags carry step ids, and they end with
 *                 the epoch words of auto ids); seg[r] for r in [r0, r1)
 *                 written, the peers' read when fused.
 *  residual_out, out : NULL (the reduce-scatter of ranks [r0, r1) alone),
 *                 or n device pointers of rows * hidden elements, entries in
 *                 [r0, r1) used, and then r1 = r0 + 1: one rank's share in
 *                 one launch (its own rows straight from the reduce-scatter,
 *                 the peers' through the all-gather).
 *  flags, step  : a flag region of ar_flag_bytes(n) and the step id, >= 1
 *                 and above every earlier call's on these segments and flags
 *                 (the peers' reduce-scatters of this step publish it); or 0
 *                 (auto): seg[r] ends with an epoch word per wavefront of
 *                 rank r's reduce-scatter and of its all-gather; each
 *                 wavefront uses its word + 1 as the id and stores that back
 *                 when it ends.  Every rank's launch of a step takes the same
 *                 id as long as each rank's rows are reduce-scattered once
 *                 per step (by its share or a reduce-scatter-only call) and
 *                 each share runs once per step, with the same rows, hidden
 *                 and dtype, so a call captured once into a HIP graph takes a
 *                 new id on every replay ([CAR] 实现: the graph path keeps
 *                 fixed registered addresses).  Zeroing the segments restarts
 *                 the epochs; do not mix explicit and auto ids between
 *                 zeroings, and zero them before 2^32 - 1 calls.  A step in
 *                 which some rank's rows were not reduce-scattered leaves
 *                 that rank's words a step behind: the shares' all-gathers
 *                 time out on it until the segments are zeroed (and the flag
 *                 region reset).
 * A wait that runs out writes AR_ERR_TIMEOUT | phase << 8 | rank << 16 to the
 * flag region's status word: AR_PHASE_TWOSHOT_AG with the peer (all-gather),
 * AR_PHASE_RMSNORM with the rank (a row's parts); detail: the row in the
 * rank's group.
 * rows must be a multiple of n, hidden as for ar_oneshot_rmsnorm.  One
 * rank's share reads S + S/n + (one row) + 2 (n-1) S/n bytes and writes
 * 2 S/n (own rows) + 2 S/n (segment) + 2 (n-1) S/n (S = rows * hidden *
 * element size), besides the slots and flags.
 * Errors: AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_DIVISIBLE, AR_ERR_ALIAS, AR_ERR_HIP. */
size_t ar_rmsnorm_segment_bytes(int n, size_t rows, size_t hidden, int dtype);
int ar_twoshot_rmsnorm(const void* const* in, int n, const void* const* residual, const void* weight,
                       void* const* seg, void* const* residual_out, void* const* out, size_t rows, size_t hidden,
                       float eps, int dtype, int r0, int r1, uint32_t* flags, uint32_t step, void* stream);

/* Reduce with a broadcast store: the kBroadcast store path of [CAR] step 5
 * -- each result written to every rank's output, not only the local one --
 * applied to one rank's share of the elements, which makes a two-shot whose
 * all-gather the producer pushes ([NCCL] 算法, two-shot), with no barrier
 * between the phases.  With V = floor(numel / (16 / element size)) whole
 * 16-byte vectors, emulated rank r owns vectors [floor(r*V/n),
 * floor((r+1)*V/n)) and rank n-1 also the partial last vector.  Every rank r
 * in [r0, r1) sums its vectors of all n inputs exactly as ar_oneshot and
 * stores the results at the same offsets of out[0..n).  [0, n) is the whole
 * all-reduce in one launch (every out[j] = ar_oneshot's result); [me, me+1)
 * is one GPU's share: reads S, writes S, S = numel * element size.
 *  in, out : n device pointers each, numel elements of dtype; outputs must
 *            not overlap each other or any input.
 * Any numel >= 1; bytes of out outside the owned range are not touched.
 * Errors: AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_ALIAS, AR_ERR_HIP. */
int ar_reduce_bcast(const void* const* in, int n, void* const* out, size_t numel, int dtype, int r0, int r1,
                    void* stream);

/* Push copy for the one-shot push of [CAR] 实现: sender i copies its message
 * src[i] (numel elements of dtype) into dst[i*ndst + j] for j < ndst -- its
 * slot in every rank's staging buffer -- after which each rank reduces its
 * own staging slots with ar_oneshot, reading only local memory.  With
 * ndst = 1 it is the staging copy of the non-graph path ([CAR] step 5: the
 * caller's tensor is copied into its registered buffer, the reduction reads
 * the registered buffers and may then write the caller's tensor in place).
 *  src : nsrc device pointers, 1 <= nsrc <= AR_MAX_RANKS;
 *  dst : nsrc * ndst device pointers, 1 <= ndst <= AR_MAX_RANKS, none
 *        overlapping another destination or a source.
 * A sender reads S and writes ndst * S.  Any numel >= 1.
 * Errors: AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_ALIAS, AR_ERR_HIP. */
int ar_push(const void* const* src, int nsrc, void* const* dst, int ndst, size_t numel, int dtype, void* stream);

/* Two-shot phase 1, reduce-scatter ([NCCL] 算法, two-shot; [MGPU] 集合通信),
 * optionally fused with the flag barrier and phase 2 in the same launch.
 * With m = numel / n, emulated rank r in [r0, r1) sums segment r of every
 * rank -- elements [r*m, (r+1)*m) -- into seg[r] (m elements, rounded once),
 * then publishes step in its arrival slots of the flag region.
 *  in    : n device pointers, numel elements each.
 *  seg   : n device pointers, m elements each (only seg[r0..r1) written;
 *          with out != NULL all n are read).
 *  r0,r1 : 0 <= r0 < r1 <= n.  [0, n) emulates every rank with groups of
 *          workgroups; [me, me+1) is one GPU's share.
 *  flags : flag region of ar_flag_bytes(n) bytes, zeroed once by
 *          ar_flag_barrier_reset before first use.
 *  step  : step id, 1..2^32-1, increasing from call to call; or 0 (auto):
 *          rank r's step id is its epoch, kept in the flag region (a copy
 *          per wavefront), plus one, and the launch advances the epoch.
 *          Auto launches use a fixed grid of two workgroups per CU
 *          (AR_ERR_HIP on a device with more than AR_EPOCH_COPIES / 8 CUs).  Auto steps let a call
 *          captured once into a HIP graph take a new id on every replay
 *          with nothing reset in between ([CAR] 实现: the graph path keeps
 *          fixed registered addresses).  Do not mix explicit and auto ids on
 *          one flag region between resets; reset before 2^32 - 1 calls.
 *  out   : NULL for reduce-scatter only.  Otherwise n device pointers
 *          (entries outside [r0, r1) ignored); the launch becomes one
 *          persistent grid (no larger than the device holds at once) that, after the reduce-scatter, waits
 *          for every rank's slot >= step and copies seg[0..n) into out[r]
 *          for r in [r0, r1) -- the same as calling ar_twoshot_ag next.
 *          Segments of ranks outside [r0, r1) must have been published
 *          already by earlier calls at this step or later.
 * Requires numel % n == 0 and m * element size % 16 == 0 ([CAR] step 2:
 * the two-shot kernel needs divisible sizes) -- else AR_ERR_DIVISIBLE.
 * Errors: AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_DIVISIBLE, AR_ERR_ALIAS,
 * AR_ERR_HIP; asynchronously AR_ERR_TIMEOUT (phase AR_PHASE_TWOSHOT_AG). */
int ar_twoshot_rs(const void* const* in, int n, void* const* seg, size_t numel, int dtype,
                  int r0, int r1, uint32_t* flags, uint32_t step, void* const* out, void* stream);

/* Two-shot phase 2, all-gather ([NCCL] 算法, two-shot; [MGPU] 集合通信):
 * for every rank r in [r0, r1), wait until each segment's arrival slots are
 * >= step, then copy seg[0], ..., seg[n-1] in order into out[r] (a bit copy,
 * no rounding).  Arguments as for ar_twoshot_rs; seg entries are read-only
 * here.  With step 0 (auto) it waits for each rank's current epoch, the id of
 * the auto reduce-scatter before it, and leaves the epoch as it is.
 * Errors as ar_twoshot_rs. */
int ar_twoshot_ag(const void* const* seg, int n, void* const* out, size_t numel, int dtype,
                  int r0, int r1, uint32_t* flags, uint32_t step, void* stream);

/* Two-shot phase 2 on the copy engines: the same result as ar_twoshot_ag,
 * with the compute units left to other work ([NCCL] 协议: communication run
 * as thread blocks competes with compute for the SMs; [SMF] 0 前言: move the
 * data with asynchronous copies instead).  One workgroup waits until every arrival slot of
 * every segment is >= step (for step 0, the largest current epoch of the
 * ranks in [r0, r1)); then, for every r in [r0, r1), n hipMemcpyAsync copies
 * of kind hipMemcpyDeviceToDeviceNoCU move seg[0..n) into out[r].  Captured
 * into a HIP graph, the runtime runs these copies on the copy engines; called
 * eagerly on one device it may run them as copy kernels instead.  On a
 * timeout the status is written as for ar_twoshot_ag, but the copies still
 * run: their output is then not valid.  Arguments and errors as
 * ar_twoshot_ag (AR_ERR_HIP also when the runtime refuses a copy).
 * A fallback for callers whose compute units must stay free, not a fast
 * path: the n copies of an output run one after another, measured on MI355X
 * (graph-replayed, n = 8) at 43 us per rank at 16 KiB and 223 us at 64 MiB
 * per rank, against 4.4 us and 37.7 us for the whole fused two-shot on the
 * compute units.  ar_select_algo never returns it. */
int ar_twoshot_ag_copy(const void* const* seg, int n, void* const* out, size_t numel, int dtype,
                       int r0, int r1, uint32_t* flags, uint32_t step, void* stream);

/* Sender side of LL / LL128 ([NCCL] 协议 table): pack count messages, each
 * numel elements of dtype taken as bytes, into their wire buffers
 * (ar_ll_wire_bytes(proto, numel * element size) bytes each).  Every line
 * carries step as its flag (32-bit for LL, 64-bit for LL128), after its data.
 * step 0 (auto): each line's flag becomes its previous flag + 1, so that
 * calls captured once into a HIP graph advance every line by one per replay
 * with no step id from the host ([CAR] step 5, graph path); the wire must
 * start zeroed and must not mix explicit and auto ids.
 * count >= 1 (1 = this GPU's own message; n = every emulated rank at once).
 * Errors: AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_ALIAS, AR_ERR_HIP. */
int ar_ll_pack(const void* const* src, void* const* wire, int count, size_t numel, int dtype,
               int proto, uint32_t step, void* stream);

/* Receiver side of LL ([NCCL] 协议 table): for every line of every rank's
 * wire buffer wait until its flag is >= step, take the 4 data bytes out,
 * and reduce the n messages exactly as ar_oneshot into out (numel elements).
 *  flags : flag region (only the status words are used).
 * Errors: AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_ALIAS, AR_ERR_HIP; asynchronously
 * AR_ERR_TIMEOUT (phase AR_PHASE_LL, rank and line of a missing line). */
int ar_ll_reduce_unpack(const void* const* wire, int n, void* out, size_t numel, int dtype,
                        uint32_t step, uint32_t* flags, void* stream);

/* Receiver side of LL128: as ar_ll_reduce_unpack with 128-byte lines holding
 * 120 data bytes and a 64-bit flag.  Phase AR_PHASE_LL128 on timeout.
 * Producers must be ordered before this call: the pack of every wire must
 * be complete when the call starts (earlier on the same stream, or behind
 * an event the stream waits for).  A line is accepted on its flag alone, and
 * the pages' LL128 premise -- a 128-byte line written and read whole
 * ([NCCL] 协议 table) -- does not hold here: a line is read as separate
 * 64-byte requests, so against a pack running at the same time the data
 * beside a flag of step s may still be that of step s-1.  For producers
 * that run at the same time use LL (a line's data and flag are one 8-byte
 * word, read whole) or the ordered LL128 of ar_twoshot_ll128. */
int ar_ll128_reduce_unpack(const void* const* wire, int n, void* out, size_t numel, int dtype,
                           uint32_t step, uint32_t* flags, void* stream);

/* One GPU's LL or LL128 step in one launch ([NCCL] 协议 table; the sender
 * and the receiver of the protocol run in the same kernel, as a rank both
 * sends its message and receives the others'):
 *  - pack rank me's message src (numel elements) into wire[me] with flag
 *    step, exactly as ar_ll_pack;
 *  - wait for every line of every other rank's wire[r] to carry a flag >=
 *    step and reduce the n messages into out exactly as ar_oneshot, rank
 *    me's term taken from src (wire[me] is written, not read back).
 *  Each wavefront writes its lines of wire[me] before it waits on any peer
 *  line, and after a timeout wire[me] still holds the whole packed message.
 *  With LL, peers' launches may run at the same time as this one: no rank's
 *  launch waits on a line that a peer's launch holds back behind a wait of
 *  its own, and a line's 4 data bytes and flag are one 8-byte word, read
 *  whole.  With LL128 the peers' packs must be complete before this call
 *  starts (stream-ordered), for the reason given at ar_ll128_reduce_unpack:
 *  a line's flag is read beside, not before, its data.
 *  wire  : n wire buffers of ar_ll_wire_bytes(proto, numel * elem) bytes, in
 *          rank order; wire[me] is rank me's own (written), the others are
 *          read.  Zeroed once before first use: a line counts as arrived
 *          when its flag is >= step.
 *  me    : 0 <= me < n.
 *  step  : 1..2^32-1, increasing from call to call; or 0 (auto): each line
 *          of wire[me] takes its previous flag + 1, and the peers' line at
 *          the same position must carry at least that -- every rank's call
 *          advances every one of its lines by one, so the ranks' auto calls
 *          stay in step (the same rule for ar_ll_pack with step 0).  After a
 *          timeout the ranks' wires may be a step apart: zero every wire (and
 *          reset the status words) before the next auto call.
 *  flags : flag region (only the status words are used).
 * out, src and wire[me] may not overlap one another or any wire buffer;
 * all pointers 16-byte aligned.  LL takes one line per lane up to 16 MiB
 * per rank and two above, as ar_ll_reduce_unpack does.
 * Errors: AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_ALIAS, AR_ERR_HIP; asynchronously
 * AR_ERR_TIMEOUT (phase AR_PHASE_LL or AR_PHASE_LL128, rank and line of a
 * missing line). */
int ar_ll_allreduce(const void* src, void* const* wire, int n, int me, void* out, size_t numel, int dtype,
                    int proto, uint32_t step, uint32_t* flags, void* stream);

/* Two-shot under the LL protocol ([NCCL] 算法, two-shot, with the 协议
 * table's LL lines): as ar_twoshot_rs, but each reduced segment is written
 * as an LL wire -- every 4 data bytes beside the step id in one 8-byte line,
 * ar_ll_wire_bytes(AR_PROTO_LL, m * element size) = 2 * m * element size
 * bytes -- and the all-gather reads the peers' lines and checks their flags
 * (>= step) itself, so there are no arrival slots and no wait between a
 * segment's stores and its flag.
 *  segw  : n LL segment wires (segw[r0..r1) written, all n read with out),
 *          zeroed once before first use: a line counts as arrived when its
 *          flag is >= step, so a wire must never hold a flag at or above a
 *          step that has not written it yet.
 *  step  : 1..2^32-1, increasing from call to call; or 0 (auto), with the
 *          epochs, fixed grid and rules of ar_twoshot_rs's auto ids: rank r's
 *          lines carry its epoch + 1 and the all-gather waits for that.
 *  out   : NULL for the reduce-scatter only; else the fused launch as in
 *          ar_twoshot_rs (one persistent grid, out[r] for r in [r0, r1)).
 *  flags : flag region of ar_flag_bytes(n) bytes (the status words; with
 *          auto ids also the epochs).
 * The result is bit for bit that of ar_twoshot_rs and ar_oneshot.  Sizes,
 * divisibility and errors as ar_twoshot_rs; asynchronously AR_ERR_TIMEOUT
 * (phase AR_PHASE_TWOSHOT_AG, segment and tile of a line that stayed
 * behind).  A line's 4 data bytes and its flag are one 8-byte word, written
 * and read whole, so a reader never sees a flag without its data: this
 * holds against producers that run at the same time (another workgroup of
 * the same launch, or another GPU). */
int ar_twoshot_ll(const void* const* in, int n, void* const* segw, size_t numel, int dtype, int r0, int r1,
                  uint32_t* flags, uint32_t step, void* const* out, void* stream);

/* Two-shot under the LL128 protocol ([NCCL] 算法, two-shot, with the 协议
 * table's LL128 lines): as ar_twoshot_ll, with each reduced segment written
 * as an LL128 wire -- 128-byte lines of 120 data bytes (zero past the
 * segment's end) and a 64-bit flag, ar_ll_wire_bytes(AR_PROTO_LL128,
 * m * element size) bytes per segment.  The pages' LL128 relies on a
 * 128-byte line being written and read whole; here a line is written by 8
 * lanes and read as separate 64-byte requests, so the protocol is kept by
 * ordering instead: the producer writes a line's 120 data bytes, waits until
 * they are complete, then writes its flag; the all-gather first polls the
 * flags of the lines it copies and loads their data only after every flag
 * is >= step.  The result is therefore correct also when the producers run
 * at the same time as the consumer (another workgroup of the same launch,
 * or another GPU), at the cost of a second dependent memory round trip per
 * line, as with the arrival slots of ar_twoshot_rs.
 *  segw  : n LL128 segment wires (segw[r0..r1) written, all n read with out),
 *          zeroed once before first use.
 *  step  : 1..2^32-1, increasing from call to call; or 0 (auto), with the
 *          epochs, fixed grid and rules of ar_twoshot_rs's auto ids.
 *  out   : NULL for the reduce-scatter only; else the fused launch: one
 *          wavefront per item when r1 - r0 == 1 with an explicit step (no
 *          wave of the launch waits on another), a persistent grid otherwise.
 * The result is bit for bit that of ar_twoshot_rs and ar_oneshot.  Sizes,
 * divisibility and errors as ar_twoshot_rs; asynchronously AR_ERR_TIMEOUT
 * (phase AR_PHASE_TWOSHOT_AG, segment and line of a line that stayed
 * behind). */
int ar_twoshot_ll128(const void* const* in, int n, void* const* segw, size_t numel, int dtype, int r0, int r1,
                     uint32_t* flags, uint32_t step, void* const* out, void* stream);

/* Algorithm selection from measured costs ([NCCL] 算法 and 协议: no
 * algorithm or protocol is best at every size, so the choice goes by message
 * size and rank count; [CAR] keeps such a per-rank-count threshold map).
 * The modelled time of algo for numel elements of dtype per rank over n ranks
 * is t_share + k * sync_us, where
 *  - t_share is the time of one GPU's share measured on MI355X with this
 *    library's kernels (cold HBM, graph-replayed; one-shot; one rank's fused
 *    two-shot; one rank's LL / LL128 send and receive in one launch
 *    (ar_ll_allreduce); one rank's push
 *    plus its one-shot over its staging slots; one rank's reduce-broadcast
 *    share; one rank's fused two-shot under LL and under LL128), tabulated for
 *    n = 2..16 over 16 KiB..64 MiB per rank, interpolated linearly in the
 *    size, flat below the grid and extended with the last slope above it;
 *  - k is the number of cross-GPU semaphore synchronisations per call, the
 *    alpha terms of the [NCCL] 算法 alpha-beta model (2 for the one-shot, 4
 *    for the two-shot; 协议 names the semaphore as alpha's main source),
 *    2 for the push and the reduce-broadcast (start and end, as the one-shot;
 *    the broadcast has no barrier between its phases), 2 for the two-shot
 *    under LL and under LL128 (their reduce-scatter still reads the peers'
 *    inputs, so start and end stay; the barrier between the phases travels
 *    in the lines), and 0
 *    for LL / LL128, whose flags travel with the data ([NCCL] 协议);
 *  - sync_us >= 0 is the cost of one such synchronisation on the caller's
 *    interconnect (0 when the ranks share one GPU).
 * ar_algo_cost_us returns that time in microseconds, or a negative value for
 * bad arguments or a two-shot the size cannot split into n whole 16-byte
 * segments.  ar_select_algo returns the ar_algo of least modelled time (the
 * lower value on a tie), or -AR_ERR_ARG for bad arguments. */
typedef enum {
    AR_ALGO_ONESHOT = 0, /* ar_oneshot */
    AR_ALGO_TWOSHOT = 1, /* ar_twoshot_rs with out (fused) */
    AR_ALGO_LL = 2,      /* ar_ll_allreduce, LL (or ar_ll_pack + ar_ll_reduce_unpack) */
    AR_ALGO_LL128 = 3,   /* ar_ll_allreduce, LL128 (or ar_ll_pack + ar_ll128_reduce_unpack) */
    AR_ALGO_PUSH = 4,    /* ar_push into the staging slots + ar_oneshot over them */
    AR_ALGO_BCAST = 5,   /* ar_reduce_bcast */
    AR_ALGO_TWOSHOT_LL = 6, /* ar_twoshot_ll with out (fused) */
    AR_ALGO_TWOSHOT_LL128 = 7 /* ar_twoshot_ll128 with out (fused) */
} ar_algo;
double ar_algo_cost_us(int algo, int n, size_t numel, int dtype, double sync_us);
int ar_select_algo(int n, size_t numel, int dtype, double sync_us);

/* Allocation-free two-shot, for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * same all-reduce as ar_twoshot_rs with out (fused, every rank [0, n) in one
 * launch), but the n segments and the arrival slots live in a device array
 * of the library (AR_NOALLOC_MAX_BYTES of segments plus the slots of 16
 * ranks), which every device that runs the call holds from its first call
 * until the process ends.  The caller passes only the inputs and outputs.
 *  in, out : n device pointers each, numel elements of dtype, 16-byte
 *            aligned; outputs must not overlap each other or any input.
 * Each call first clears the slots with a fill kernel on stream, then runs
 * the fused two-shot with step id 1, so no state carries over from one call
 * to the next (another n, an earlier timeout).  The first call on a device
 * looks up that device's copy of the array (hipGetSymbolAddress); it
 * allocates nothing, and no call does.  Calls share their device's array:
 * calls that overlap in time on one device race (issue them on one stream).
 * A wait that times out cannot be reported (the status words are in the
 * array); in one launch that holds every rank it would need another kernel
 * to keep the device's compute units for the whole wait budget.
 * Errors: AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_DIVISIBLE, AR_ERR_ALIAS,
 * AR_ERR_SIZE (numel * element size above AR_NOALLOC_MAX_BYTES), AR_ERR_HIP. */
#define AR_NOALLOC_MAX_BYTES (64u << 20)
int ar_twoshot_noalloc(const void* const* in, int n, void* const* out, size_t numel, int dtype, void* stream);

/* Zero the whole flag region of ar_flag_bytes(n) bytes (status words and
 * every arrival slot) with a fill kernel, so that steps may start again at
 * 1: at set-up, after a timeout, and before step ids would wrap.
 * Errors: AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_HIP. */
int ar_flag_barrier_reset(uint32_t* flags, int n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AR_H */
