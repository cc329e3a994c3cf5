/*
 * moe_ep.h -- C ABI of the MI355X (gfx950) expert-parallel dispatch/combine
 * library libmoe_ep.so.
 *
 * The path, for P logical expert-parallel ranks emulated in one GPU's HBM:
 *   moe_route_topk   router softmax + top-k + renormalised weights
 *   moe_dispatch     count, prefix sums, stable permute-and-pack of the hidden
 *                    rows plus a combine handle into all-to-all-v send
 *                    buffers, then the exchange into the receive buffers
 *   moe_expert_stub  a per-expert scalar stand-in for the grouped GEMM
 *   moe_combine      reverse exchange, then the routing-weighted top-k
 *                    reduction back into original token order
 *
 * Sources (web pages on expert-parallel all-to-all; cited by title and section):
 *  [EP]   "Expert Parallel: MoE Token 为什么要两次穿过 GPU 网络" (charlestar.github.io)
 *  [A2A]  "[Infra-10] All-to-All Optimization" (xutianle.me)
 *  [PPLX] "高效且便携的专家混合通信" (Perplexity's pplx-kernels article)
 *
 * Conventions for every call:
 *  - Shapes: P = num_ranks, T/P = tokens_per_rank (token t lives on rank
 *    s = t / (T/P), local index i = t mod (T/P)), E = num_experts (expert e is
 *    owned by rank e / (E/P)), k = top_k, H = hidden, N_a = T * k assignments.
 *  - Every data pointer is a DEVICE pointer into caller-owned memory on the
 *    current HIP device; ctx, shape, handle and status outputs are HOST
 *    pointers.  `stream` is a hipStream_t (NULL = default stream).
 *  - Alignment: row buffers (x, send_buf, recv_buf, gathered, expert_out,
 *    comb_buf, y) start on 16 bytes, since kernels move rows 16 bytes per
 *    lane; logits, topk_ids, topk_w and the scale arrays on 4 bytes.  Else
 *    MOE_ERR_INVALID_ARG.  torch and hipMalloc allocations, and whole-row
 *    slices of them, satisfy both.
 *  - Calls only enqueue work on `stream`: they never allocate device memory,
 *    never synchronise and never read device data on the host ([A2A] 3.5: a
 *    count read back to the CPU puts a hole before the exchange; [EP]
 *    "显存账不只有 expert 权重": buffers are preallocated at the maximum size).
 *  - Host-detectable errors are returned synchronously and nothing is
 *    enqueued; launch failures return MOE_ERR_HIP.  Expert ids outside
 *    [0, E) or repeated within a token are outside the contract.
 *  - Debug mode (environment MOE_EP_DEBUG=1 when the ctx is created): both
 *    dispatch calls first count such ids on the device, wait for the count
 *    (the one place the library synchronises) and return MOE_ERR_INVALID_ARG,
 *    with the count in moe_last_error(), before launching anything else.
 *  - T = 0 is a valid no-op.  No C++ exception crosses this ABI.
 *  - Threads: a ctx holds host state (the handle generation, the phase of the
 *    split calls, timing records), so calls on one ctx must not overlap.
 *    Different ctxs may be used from different threads at once.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,   /* null pointer, bad size or shape */
    MOE_ERR_UNSUPPORTED = -2,   /* shape outside the supported limits below */
    MOE_ERR_WORKSPACE = -3,     /* workspace smaller than moe_workspace_bytes() */
    MOE_ERR_STALE_HANDLE = -4,  /* handle not from the latest moe_dispatch of this ctx */
    MOE_ERR_HIP = -5,           /* a HIP runtime call or kernel launch failed */
    MOE_ERR_NO_MEMORY = -6      /* a host allocation inside the library failed */
} moe_status;

typedef enum {
    MOE_DTYPE_BF16 = 0,         /* rows of H bfloat16 values (2H bytes) */
    MOE_DTYPE_FP8_E4M3 = 1      /* rows of H OCP E4M3 codes + H/128 fp32 scales */
} moe_dtype;

/* Problem shape, with T = P * tokens_per_rank.  moe_ctx_create returns
 * MOE_ERR_INVALID_ARG for P < 1, tokens_per_rank < 0, E < 1, E % P != 0,
 * k < 1 or k > E, H < 8 or H % 8 != 0, or an unknown dispatch_dtype; and
 * MOE_ERR_UNSUPPORTED, outside the supported limits, for E > 1024,
 * E/P > 32767, k > 32, H > 65536, FP8 with H % 128 != 0, T * k >= 2^31,
 * T * k * (H/1024 + 1) >= 2^31 or (T * k + P) * (H/8 + 512) >= 2^32 (the grid
 * of a row kernel). */
typedef struct {
    int32_t num_ranks;
    int32_t tokens_per_rank;
    int32_t num_experts;
    int32_t top_k;
    int32_t hidden;
    int32_t dispatch_dtype;     /* moe_dtype */
} moe_shape;

/* The 16-byte record that travels with every dispatched row ([EP] "dispatch
 * payload": local expert id, source token index, top-k slot and routing
 * weight; [EP] "combine handle": source rank and token, top-k slot, weight;
 * [PPLX] dispatch-receive stores source rank, expert and token index for the
 * combine). */
typedef struct {
    int32_t src_rank;           /* s */
    int32_t src_token;          /* i, index local to rank s */
    int16_t slot;               /* j, top-k slot of the assignment */
    int16_t local_expert;       /* e mod (E/P) */
    float weight;               /* topk_w[t, j] */
} moe_meta;

/* Opaque host-side context: shape, workspace layout, handle generation.  It
 * owns no device memory. */
typedef struct moe_ctx moe_ctx;

/* What moe_dispatch returns for the combine and for the expert stage ([EP]
 * "Combine 不是简单把结果发回来": dispatch hands the combine a handle that
 * holds the buffer positions, source rank and token, top-k slot, per-expert
 * counts and the weight, and exposes each local expert's received count for
 * the grouped GEMM shape).  All arrays are device pointers into the caller's
 * workspace, valid until the next moe_dispatch on the same ctx. */
typedef struct {
    const int32_t* expert_counts;       /* [E]     N[e], rows received by expert e */
    const int32_t* expert_offsets;      /* [E+1]   first receive row of expert e */
    const int32_t* rank_recv_offsets;   /* [P+1]   first receive row of rank r */
    const int32_t* count_matrix;        /* [P][P]  C[s][r], rows sent from s to r */
    const int32_t* rank_expert_counts;  /* [P][E]  n[s][e] */
    const int32_t* send_offsets;        /* [P][E]  first send row of bucket (s -> e) */
    const int32_t* recv_offsets;        /* [P][E]  first receive row of bucket (s -> e) */
    const int32_t* send_pos;            /* [T][k]  send row of assignment (t, j) */
    const int32_t* recv_pos;            /* [T][k]  receive row of assignment (t, j) */
    const moe_meta* send_meta;          /* [N_a]   record of each send row */
    const moe_meta* recv_meta;          /* [N_a]   record of each receive row */
    const void* ctx;                    /* the ctx that issued it */
    uint64_t generation;                /* dispatch sequence number on that ctx */
} moe_handle;

/* Per-kernel timing record (moe_timing_end). */
typedef struct {
    const char* kernel;         /* static name of the kernel */
    int32_t launches;
    float total_ms;             /* sum of HIP-event durations of its launches */
} moe_kernel_time;

/* ---- context and sizes ---------------------------------------------------- */

/* Validates the shape and creates a context.  Returns MOE_ERR_INVALID_ARG or
 * MOE_ERR_UNSUPPORTED (and *out = NULL) for shapes outside the limits, and
 * MOE_ERR_NO_MEMORY if the context cannot be allocated. */
moe_status moe_ctx_create(const moe_shape* shape, moe_ctx** out);
void moe_ctx_destroy(moe_ctx* ctx);

/* Device workspace moe_dispatch needs (counts, offsets, positions, the send
 * and receive handle records).  0 for a NULL ctx. */
size_t moe_workspace_bytes(const moe_ctx* ctx);
/* Bytes of one dispatched row: 2H (bf16) or H (e4m3).  0 for a NULL ctx. */
size_t moe_dispatch_row_bytes(const moe_ctx* ctx);
/* fp32 scales per dispatched row: H/128 for e4m3, 0 for bf16. */
int32_t moe_scales_per_row(const moe_ctx* ctx);
/* N_a = T * k, the rows of every send, receive, expert-output and combine buffer. */
int64_t moe_num_assignments(const moe_ctx* ctx);

/* ---- the path ------------------------------------------------------------- */

/* Router ([PPLX] router paragraph: a small linear layer yields a probability
 * distribution over experts, the top-k experts are taken and their outputs
 * are averaged with the router's weights; [EP] "Dispatch 前为什么必须 count 和
 * permute": the router output is [num_tokens, top_k] expert ids and weights).
 *   logits   fp32 [T][E], row-major
 *   topk_ids int32 [T][k] out: slot j holds the expert with the j-th largest
 *            probability (softmax is strictly increasing, so: the j-th largest
 *            logit); equal logits are ordered by lower expert id
 *   topk_w   fp32 [T][k] out: p_e / sum of p over the k chosen experts, with
 *            p = softmax(logits row) (computed in double, rounded to fp32)
 * Error: MOE_ERR_INVALID_ARG on a NULL ctx or (T > 0) a NULL array. */
moe_status moe_route_topk(moe_ctx* ctx, const float* logits, int32_t* topk_ids, float* topk_w,
                          void* stream);

/* Dispatch ([EP] sections "Dispatch 前为什么必须 count 和 permute" and
 * "All-to-All-v 才接近真实通信形状"; [A2A] 3.5 count / prefix sum / scatter /
 * pack, 4.3 and 5.1 write the permutation straight into the communication
 * buffer, 5.2 destination-contiguous send layout bucketed by local expert;
 * [A2A] 1 all-to-all as a distributed transpose).
 *   x            bf16 [T][H] hidden states (uint16 bit patterns)
 *   topk_ids     int32 [T][k], topk_w fp32 [T][k] (from moe_route_topk or the caller)
 *   workspace    device scratch of >= moe_workspace_bytes() bytes, 256-byte aligned
 *   send_buf     [N_a][row] out: rank s owns rows [s*(T/P)*k, (s+1)*(T/P)*k),
 *                ordered by destination rank, then local expert, then token
 *   send_scales  fp32 [N_a][H/128] out (e4m3 only, else NULL): per token and
 *                128-channel block, scale = amax / 448 and code = e4m3(x / scale)
 *                (fp32 division, round to nearest even, saturating)
 *   recv_buf     [N_a][row] out: rank r's region is contiguous; inside it rows
 *                are grouped by expert, then source rank, then token
 *   recv_scales  fp32 [N_a][H/128] out (e4m3 only, else NULL)
 *   handle       host out: see moe_handle
 * Errors: MOE_ERR_INVALID_ARG (NULL pointer, scales given for bf16 or missing
 * for e4m3, misaligned workspace), MOE_ERR_WORKSPACE, MOE_ERR_HIP. */
moe_status moe_dispatch(moe_ctx* ctx, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                        void* workspace, size_t workspace_bytes,
                        void* send_buf, float* send_scales, void* recv_buf, float* recv_scales,
                        moe_handle* handle, void* stream);

/* Expert stub, standing in for the grouped GEMM that reads the
 * expert-contiguous receive rows ([A2A] 5.2: the receive layout is the expert
 * kernel's input; [EP] worked example: each rank runs its local experts on
 * what it received).  For receive row q of expert e:
 *   expert_out[q] = bf16( deq(recv[q]) * m_e ),  m_e = (E + e) / E in fp32,
 * deq = the bf16 value, or the fp32 product code * scale for e4m3 rows; each
 * product rounds to fp32 and the result rounds once to bf16 (nearest even).
 *   expert_out   bf16 [N_a][H] out, in receive order
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_STALE_HANDLE, MOE_ERR_HIP. */
moe_status moe_expert_stub(moe_ctx* ctx, const moe_handle* handle, const void* recv_buf,
                           const float* recv_scales, uint16_t* expert_out, void* stream);

/* Combine ([EP] "Combine 不是简单把结果发回来": outputs go back to their source
 * token by the handle, never in arrival order, and are summed with the router
 * weights; [PPLX] combine sends unquantised 16-bit activations back and the
 * receiver writes the weighted sum into a caller-allocated tensor).
 *   expert_out   bf16 [N_a][H] from the expert stage, in receive order
 *   topk_w       fp32 [T][k], the source side's routing weights
 *   comb_buf     bf16 [N_a][H] out: the reverse exchange; row t*k + j holds
 *                the output of assignment (t, j)
 *   y            bf16 [T][H] out: y[t] = bf16(acc), acc = fma(w[t][j],
 *                comb[t*k+j], acc) over j = 0..k-1 from acc = 0 in fp32
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_STALE_HANDLE, MOE_ERR_HIP. */
moe_status moe_combine(moe_ctx* ctx, const moe_handle* handle, const uint16_t* expert_out,
                       const float* topk_w, uint16_t* comb_buf, uint16_t* y, void* stream);

/* ---- dispatch without a caller workspace ----------------------------------- */

/* moe_dispatch for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels, outputs and handle as moe_dispatch, with the workspace taken
 * from a static array of 8 MiB that the library holds on each GPU it runs on
 * (allocated with the code object, kept until the process ends) instead of a
 * caller buffer.  The call allocates nothing: no hipMalloc or hipFree, no
 * events (per-kernel timing skips its kernels) and no host read-back (the
 * MOE_EP_DEBUG id check is not done here).  Nothing in that array has to be
 * cleared between calls: every dispatch writes each word before reading it.
 * The handle's arrays point into the current device's copy.  They stay valid
 * until the next dispatch of this ctx, or the next moe_dispatch_noalloc on the
 * same device by any ctx; moe_expert_stub and the combines then return
 * MOE_ERR_STALE_HANDLE.  Every call on one GPU shares that GPU's copy, so
 * calls that overlap in time on one GPU (other threads, or streams not ordered
 * after the previous handle's combine) race on it.
 *   Arguments as moe_dispatch without workspace / workspace_bytes.
 * Errors: MOE_ERR_WORKSPACE when moe_workspace_bytes(ctx) > 8 MiB (about
 * 150,000 assignments; the shape then needs moe_dispatch), MOE_ERR_INVALID_ARG,
 * MOE_ERR_HIP (also when the array's device address cannot be obtained). */
moe_status moe_dispatch_noalloc(moe_ctx* ctx, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                                void* send_buf, float* send_scales, void* recv_buf, float* recv_scales,
                                moe_handle* handle, void* stream);

/* ---- direct forms (pack straight into the receive rows, reduce straight from
 * the expert output) ------------------------------------------------------- */

/* Dispatch that writes every row, scale and handle record straight into its
 * receive row, with no send buffer and no separate exchange ([A2A] 4.3: the
 * preferred form permutes the input straight into the destination buffer;
 * [PPLX] further improvements: over a shared-memory link, buffers shared across
 * devices remove copies).  On one GPU this models each source rank writing into
 * its peers' receive regions.  Same counts, offsets, positions, receive rows,
 * scales and receive records as moe_dispatch; the handle's send_meta is NULL.
 * Arguments as moe_dispatch without send_buf / send_scales.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_WORKSPACE, MOE_ERR_HIP. */
moe_status moe_dispatch_direct(moe_ctx* ctx, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                               void* workspace, size_t workspace_bytes, void* recv_buf, float* recv_scales,
                               moe_handle* handle, void* stream);

/* Combine that reads each assignment's expert output through the handle
 * (row recv_pos[t][j]) and reduces it in place of the reverse exchange, with no
 * combine buffer ([A2A] 5.1: the combine fuses the inverse index, the weight
 * multiply and the reduction).  y is bit-identical to moe_combine's.  Accepts a
 * handle from either dispatch.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_STALE_HANDLE, MOE_ERR_HIP. */
moe_status moe_combine_direct(moe_ctx* ctx, const moe_handle* handle, const uint16_t* expert_out,
                              const float* topk_w, uint16_t* y, void* stream);

/* ---- the all-gather dispatcher --------------------------------------------- */

/* Dispatch by all-gather ([EP] "为什么不用 AllGather 收集所有 token": every rank
 * gathers all tokens and picks out the assignments of its own experts; no
 * variable-length point-to-point permutation, but every token reaches every
 * rank, so it pays only with few ranks, a large top-k or a tiny batch).  The
 * all-gather writes every token's dispatched row (FP8 codes and scales
 * computed once per token) into each rank's copy; each rank then picks its
 * receive rows from its own copy.  Receive rows, scales, records, counts,
 * offsets and positions equal moe_dispatch's; the handle's send_meta is NULL
 * and it serves moe_expert_stub, moe_combine and moe_combine_direct.
 *   gathered         [P*T][row] out: row r*T + t holds token t in rank r's copy
 *   gathered_scales  fp32 [P*T][H/128] out (e4m3 only, else NULL)
 * Other arguments as moe_dispatch.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_WORKSPACE, MOE_ERR_HIP; MOE_ERR_UNSUPPORTED
 * when P * T * (H/8 + 512) >= 2^32 (the gathered rows in one grid dimension). */
moe_status moe_dispatch_allgather(moe_ctx* ctx, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                                  void* workspace, size_t workspace_bytes, void* gathered, float* gathered_scales,
                                  void* recv_buf, float* recv_scales, moe_handle* handle, void* stream);

/* ---- split phases ([PPLX]: dispatch and combine each run as a send half and
 * a receive half, so that other work can run in between; [A2A] 7: overlap pays
 * only when there is independent work to hide the exchange behind) --------- */

/* moe_dispatch = moe_dispatch_send then moe_dispatch_recv; moe_combine =
 * moe_combine_send then moe_combine_recv.  The halves may be issued on
 * different streams; ordering them (an event recorded after one half and
 * waited on before the next) is the caller's job.  The host enforces the call
 * order per handle: the receive half of dispatch before the expert stage and
 * the combine, the send half of combine before its receive half (else
 * MOE_ERR_INVALID_ARG, reason in moe_last_error()).  Base form only.
 *   moe_dispatch_send  count, prefix sums, pack into send_buf (+ scales) and the
 *                      handle; arguments as moe_dispatch without the receive side
 *   moe_dispatch_recv  the exchange into recv_buf (+ scales) and the receive records
 *   moe_combine_send   the reverse exchange into comb_buf
 *   moe_combine_recv   the weighted reduction of comb_buf into y
 * Errors: as the corresponding whole calls. */
moe_status moe_dispatch_send(moe_ctx* ctx, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                             void* workspace, size_t workspace_bytes, void* send_buf, float* send_scales,
                             moe_handle* handle, void* stream);
moe_status moe_dispatch_recv(moe_ctx* ctx, const moe_handle* handle, const void* send_buf, const float* send_scales,
                             void* recv_buf, float* recv_scales, void* stream);
moe_status moe_combine_send(moe_ctx* ctx, const moe_handle* handle, const uint16_t* expert_out,
                            uint16_t* comb_buf, void* stream);
moe_status moe_combine_recv(moe_ctx* ctx, const moe_handle* handle, const uint16_t* comb_buf, const float* topk_w,
                            uint16_t* y, void* stream);

/* Events for ordering the split phases across two streams of one device: record
 * one on a stream after a half, wait for it on another stream before the next.
 * They are HIP events created without timing and without the system-scope fence:
 * the ordered work is on the same device, where each kernel's own release and
 * acquire make its stores visible, so a record-and-wait pair costs less than
 * with a default event.  A wait refers to the latest record enqueued before
 * it, so an event can be recorded again once its wait is enqueued.
 *   moe_event_create   a new event on the current device, in *event
 *   moe_event_destroy  destroys it (NULL: nothing)
 *   moe_event_record   records event on stream (NULL: the null stream)
 *   moe_stream_wait_event  work enqueued on stream after this call waits for the
 *                      event's latest record
 * MOE_ERR_INVALID_ARG for a NULL event (or out pointer), MOE_ERR_UNSUPPORTED
 * while the stream is capturing a graph, MOE_ERR_HIP if a HIP call fails. */
moe_status moe_event_create(void** event);
moe_status moe_event_destroy(void* event);
moe_status moe_event_record(void* event, void* stream);
moe_status moe_stream_wait_event(void* stream, void* event);

/* ---- measurement aids (not part of the path) ------------------------------- */

/* Ceilings of this GPU for the row kernels' access pattern ([A2A] 11.2: read a
 * kernel's bandwidth against what the hardware delivers, measured the same
 * way): 16-byte loads (and stores) with one unit per lane, consecutive lanes on
 * consecutive units.
 *   moe_probe_copy  dst[0, bytes) = src[0, bytes); policy 0: temporal loads and
 *                   write-back stores, 1: nontemporal loads and stores, 2:
 *                   temporal loads and write-through (device-scope) stores, as
 *                   the row kernels store rows that another XCD reads next
 *   moe_probe_read  reads src[0, bytes) and discards it, temporal or
 *                   (nontemporal != 0) nontemporal; sink is a device array of
 *                   256 uint32 that a lane writes only if its fold of a unit
 *                   equals 0xA5A5A5A5 (never, for a zero-filled source)
 *   moe_probe_gather  row r of dst (rows of row_bytes) = row perm[r] of src, for
 *                   r < rows, with the policies of moe_probe_copy; the
 *                   streaming exchange's pattern (nontemporal gathers of at
 *                   least 128 MiB in one-wave workgroups, as the library's
 *                   streaming row kernels), so that a chain of such
 *                   copies, each reading through a permutation what the one
 *                   before wrote, shows the cost of handing rows from one
 *                   kernel to the next in another order.  perm: device array
 *                   of `rows` int32; an entry outside [0, src_rows) is clamped
 *                   into it (src holds src_rows rows).  row_bytes a positive
 *                   multiple of 16, rows >= 0, src_rows > 0 (else
 *                   MOE_ERR_INVALID_ARG; MOE_ERR_UNSUPPORTED when
 *                   rows * (row_bytes / 16 + 512) reaches 2^32).
 * src, dst: device pointers on 16 bytes, bytes a multiple of 16 (else
 * MOE_ERR_INVALID_ARG, as for a policy outside 0..2; MOE_ERR_UNSUPPORTED
 * beyond 2^31 workgroups of 4 KiB).  Only enqueue on `stream`; MOE_ERR_HIP if
 * the launch fails. */
moe_status moe_probe_copy(const void* src, void* dst, size_t bytes, int32_t policy, void* stream);
moe_status moe_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t nontemporal, void* stream);
moe_status moe_probe_gather(const void* src, int32_t src_rows, void* dst, const int32_t* perm, int32_t rows,
                            int32_t row_bytes, int32_t policy, void* stream);

/* ---- diagnostics ---------------------------------------------------------- */

/* Static, human-readable text of a status code. */
const char* moe_status_string(moe_status status);
/* The reason for the status of this thread's latest library call: the HIP
 * error, the argument that failed its check, or the call that must come first.
 * Each call that returns a moe_status clears it on entry, so it is "" after
 * such a call succeeded.  The pointer stays valid until this thread's next call
 * that returns a moe_status. */
const char* moe_last_error(void);

/* Per-kernel timing: between moe_timing_begin and moe_timing_end every kernel
 * the ctx launches carries a start and a stop HIP event in its own dispatch
 * (hipExtLaunchKernelGGL), so a duration covers that kernel's execution and
 * not the gaps between launches.  moe_timing_end waits for the recorded
 * events, writes up to `max` records (one per kernel name, in first-launch
 * order) and returns how many kernels were seen in *count.  Kernel names:
 * route_topk, count, scan, pack, count_pack (the pack kernel counting by
 * itself, small problems), exchange, stub, reverse_exchange, reduce;
 * pack_direct, count_pack_direct, reduce_direct for the direct forms;
 * allgather, handles or count_handles, select for the all-gather dispatcher. */
moe_status moe_timing_begin(moe_ctx* ctx);
moe_status moe_timing_end(moe_ctx* ctx, moe_kernel_time* out, int32_t max, int32_t* count);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
