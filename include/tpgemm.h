/*
 * tpgemm.h -- C ABI of the MI355X (gfx950) staged tensor-parallel GEMM share.
 *
 * One GPU runs the rank-local share of a tensor-parallel GEMM as P ordered
 * stages. The peers' shards are ordinary device buffers in the same HBM;
 * each stage's input is delivered by an asynchronous device-to-device copy
 * (the library's copy kernel, the runtime's shader copy or the SDMA copy
 * engines, below) and gated by a cross-stream dependency (a stream memory
 * write and wait on a word of the library's; a HIP event in a recorded
 * graph), so the matrix cores start on
 * the local shard while the rest is delivered ("Distributed GEMM", Hassani
 * et al., SHI Labs, Dec 2024: Introduction and Background, Figures 3 and 4).
 * Which copy: by default the library's own copy kernel (non-temporal
 * loads, eight 16-byte vectors in flight per thread: seven 8 MiB slices in
 * 22.8 us with cold caches, against 40 us for the runtime's copies and
 * ~64 us on the SDMA copy engines). The all-gather's deliveries are on its
 * critical path; the reduce-scatter's hide behind the emitted blocks, and
 * there too the copy kernel measured fastest, although its workgroups take
 * CUs from those GEMMs where the pages' design uses copy engines (the bf16
 * RS share, 8192 x 8192 x 3584 in 8 blocks: 403-404 us, against 413 with the
 * shader copy and 423-430 on the copy engines; tiling B 403-405 / 415 /
 * 455-459). TPG_COPY_SDMA / TPG_COPY_SHADER / TPG_COPY_KERNEL override the
 * default (one at most).
 *
 * Conventions shared by every entry point
 *   - All pointers to tensor data are DEVICE pointers owned by the caller;
 *     pointer arrays (a_slices, incoming, src) are HOST arrays of device
 *     pointers, read during the call only. The library never frees or
 *     retains caller memory beyond the cached graphs described below.
 *   - Matrices are dense row-major with the leading dimension equal to the
 *     row length stated for each argument. bf16 is IEEE binary32's top half;
 *     e4m3 is OCP 8-bit E4M3FN (bias 7, max 448, no infinities).
 *   - Every call is asynchronous on `stream` (a hipStream_t, NULL = the
 *     legacy default stream): the call forks its internal streams from
 *     `stream` and joins them back before returning, so work enqueued later
 *     on `stream` sees the results. No call blocks the host on the GPU,
 *     with two exceptions: a call that fails after enqueuing work waits for
 *     the streams it used; and a call waits for older calls to finish when
 *     the device lags so far behind the host that calls in flight hold 7/8
 *     of the library's 65536 cross-stream dependency words (a dependency
 *     between the library's streams is a stream memory write and wait on
 *     one of them; a word is reused only once its last user has finished).
 *   - Inputs are never written (p04 statement, "Interface, layout, and
 *     parameters": inputs must not be mutated).
 *   - Arguments are validated before anything is enqueued; a failing call
 *     enqueues nothing and returns a non-zero status, with a message from
 *     tpg_last_error(). There is no fallback path.
 *   - Issue policy. Calls are issued eagerly by default. TPG_FORCE_GRAPH
 *     records the call into a hipGraph on first use and replays it after.
 *     On MI355X (ROCm 7) replay was measured no faster than eager issue for
 *     every workload here, and slower for calls that fan out over streams
 *     (us, eager vs graph: e4m3 AG share 104 vs 125, P = 2 bf16 AG 20 vs
 *     35, SwiGLU AG 250 vs 273; bf16 RS 477 vs 472). A staged AG or RS call
 *     of under 1 GFLOP that leaves the grouping to the library
 *     (groups = 0) is latency-bound and runs as if TPG_SERIAL_STAGES were
 *     set: the same stages in the same order on one stream, without
 *     cross-stream dependencies. An all-gather under 20 GFLOP with library
 *     grouping that meets the shape rules of TPG_IN_KERNEL_GATES, whose
 *     tiles and copy workgroups fit on the chip at once and whose stream is
 *     not being captured instead runs as one launch carrying its deliveries
 *     as extra workgroups, the delivered slices' tiles waiting inside the
 *     kernel for them (P = 2 bf16 share 256 x 256 x 512: 20.1 -> 11.4 us;
 *     1024^3 in 2 slices: 34 -> 17 us). TPG_NO_GRAPH, TPG_PROFILE and
 *     TPG_DEBUG_HOLD_DELIVERIES never replay a graph.
 *   - A caller may record a call into its own graph by capturing `stream`
 *     around it: the call then orders its internal streams with events,
 *     which join them to the capture, and never takes the latency-bound
 *     single-launch form (a replay would wait on a stale count). TPG_IN_KERNEL_GATES
 *     calls are refused under capture.
 *   - Graph cache: a recorded graph is keyed by (entry point, shapes,
 *     pointers, scalars, flags). A changed pointer makes a new graph, never
 *     a stale replay. Freeing a buffer a cached graph refers to is safe as
 *     long as that exact argument set is not called again;
 *     tpg_release_caches() drops all graphs. When the cache is full (512
 *     graphs) its graphs are retired: each is destroyed by a later call once
 *     an event recorded after its last replay has completed (polled, never
 *     waited on).
 *   - Calls on one device serialise on an internal lock; two calls whose
 *     workspaces overlap must not be in flight at once on different streams.
 */
#ifndef TPGEMM_H
#define TPGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TPG_OK = 0,
  TPG_ERR_INVALID = 1,      /* bad shape, rank, NULL pointer, aliasing, beta != 0 without C */
  TPG_ERR_UNSUPPORTED = 2,  /* valid request the library does not implement (dtype/layout/alignment) */
  TPG_ERR_WORKSPACE = 3,    /* workspace missing or smaller than *_workspace_size() */
  TPG_ERR_HIP = 4           /* a HIP runtime call failed; see tpg_last_error() */
} tpg_status;

typedef enum { TPG_BF16 = 0, TPG_E4M3 = 1 } tpg_dtype;

/* Layout of the B operand. NK: B is (N, K) row-major, as the distributed GEMM
 * op takes it ("Pytorch Op for blackwell distributed gemm", Note on Tensor
 * Layouts). KN: B is (K, N) row-major, the weight layout of the p04 FFN
 * (w1 [L, D, 2H], wout [L, H, D]) and of the torchtitan SwiGLU shards. */
typedef enum { TPG_B_NK = 0, TPG_B_KN = 1 } tpg_blayout;

typedef enum {
  TPG_EPI_ALPHA_BETA = 0,   /* D = alpha * acc + beta * C */
  TPG_EPI_SWIGLU = 1        /* acc has N = 2n columns [u | v]; D = silu(alpha u) * (alpha v) + beta * C, D is (M, n) */
} tpg_epilogue;

/* flags (bitwise or) */
enum {
  TPG_UNSTAGED = 1u,        /* single stage: deliver everything, then one GEMM (the non-overlapped baseline) */
  TPG_NO_COPY = 2u,         /* read peer buffers in place; no deliveries (compute-only timing) */
  TPG_NO_GRAPH = 4u,        /* enqueue eagerly even with TPG_FORCE_GRAPH */
  TPG_COPY_SDMA = 8u,       /* deliver with the SDMA copy engines (no CUs) */
  TPG_SERIAL_STAGES = 16u,  /* run all stage GEMMs on one compute stream (no inter-stage concurrency) */
  TPG_PROFILE = 32u,        /* eager only: time every GEMM launch with HIP events (tpg_profile_read) */
  TPG_FORCE_GRAPH = 64u,    /* record the call into a hipGraph once, replay it after */
  TPG_DEBUG_HOLD_DELIVERIES = 128u, /* testing: issue eagerly, with the deliveries queued behind a 20 ms
                                       host callback; every gated stage must still see its data */
  TPG_COPY_SHADER = 256u,   /* deliver with the runtime's shader copy (hipMemcpyAsync, uses CUs) */
  TPG_COPY_KERNEL = 512u,   /* deliver with the library's copy kernel (uses CUs); the default */
  TPG_DEBUG_NO_GATE = 1024u, /* testing, the negative control of the gate tests: staged rotating-A
                               all-gathers and reduce-scatters issue every stage run that reads
                               delivered data on an internal stream WITHOUT waiting for its
                               deliveries. With TPG_DEBUG_HOLD_DELIVERIES those runs read the
                               receive slots before the deliveries land, so the result is wrong
                               (never a fault: the slots are valid workspace memory). Issues
                               eagerly; rejected with TPG_UNSTAGED or TPG_SERIAL_STAGES
                               (TPG_ERR_INVALID) and by the other entry points
                               (TPG_ERR_UNSUPPORTED). With TPG_IN_KERNEL_GATES the launch's
                               tiles skip their counter waits instead. */
  TPG_IN_KERNEL_GATES = 2048u, /* staged rotating-A all-gather as ONE GEMM launch over all M rows:
                                 the tiles of each delivered slice wait inside the kernel, K-chunk
                                 by K-chunk, on counters that the library's copy kernel (running
                                 beside it on an internal stream) bumps as each chunk lands. No
                                 stage boundaries between launches. A call under 20 GFLOP whose
                                 tiles and copy workgroups fit on the chip at once (and without
                                 the two TPG_DEBUG_* delivery flags) carries the copy in the GEMM
                                 launch itself as extra workgroups, one counter for all of them:
                                 one stream and one launch.
                                 Needs P <= 8, M/P a multiple of 128, K * element bytes a
                                 multiple of 128 and the copy kernel
                                 (no other TPG_COPY_* flag); rejected with TPG_UNSTAGED,
                                 TPG_SERIAL_STAGES, TPG_ROTATE_B and by the other entry points
                                 (TPG_ERR_UNSUPPORTED); with TPG_NO_COPY the slices must be back to
                                 back in memory. The workspace grows by 256 bytes of
                                 counters. Always issued eagerly (TPG_FORCE_GRAPH is ignored):
                                 the GEMM depends on the copy kernel running concurrently, which
                                 the call arranges on its own streams; do not capture such a call
                                 into a graph. A tile that waits 2 s without its data gives up
                                 and writes NaN (never a hang). groups is ignored. */
  TPG_DEBUG_GATE_TIMEOUT = 4096u /* testing, the bounded wait of TPG_IN_KERNEL_GATES (required with
                                    it, else TPG_ERR_INVALID): every in-kernel wait asks for one
                                    arrival more than will ever come and gives up after 20 us, so
                                    every tile of a delivered slice writes NaN while the local
                                    slice's rows stay right, and every kernel still exits. */
};

/* ------------------------------------------------------------------------
 * All-gather staged GEMM.
 * D = alpha * A * B^T + beta * C with A (M, K) split into P row slices of
 * m = M/P rows; slice s is rank s's shard ("Pytorch Op for blackwell
 * distributed gemm", Usage: alpha * (A @ B_T) + beta * C; "Distributed GEMM",
 * Approach: schedule AllGather1D_TilingCD_RotatingA, C and D tiled by the same
 * rows). Stage t computes rows [s*m, (s+1)*m) of D from slice
 * s = (rank + t) mod P, the local slice first (Background, Figure 4).
 *
 *   M, N, K      M % P == 0. N = rows of B (NK) or columns of B (KN);
 *                with TPG_EPI_SWIGLU N is even and D has N/2 columns.
 *   P, rank      1 <= P <= 64, 0 <= rank < P.
 *   ab_dtype     TPG_BF16 (K % 8 == 0) or TPG_E4M3 (K % 16 == 0, NK only).
 *   b_layout     TPG_B_NK or TPG_B_KN (KN needs N % 8 == 0).
 *   a_slices     host array of P device pointers, each (m, K) row-major.
 *   b            (N, K) or (K, N) row-major.
 *   c            bf16 (M, Nout); never read when beta == 0 (may be NULL then).
 *   d            bf16 (M, Nout) output; must not overlap any input.
 *   workspace    device buffer of at least tpgemm_stage_ag_workspace_size()
 *                bytes (receive slots for the P-1 delivered slices; with
 *                TPG_UNSTAGED the whole gathered A). May be NULL if that size
 *                is 0. Contents are scratch.
 *   groups       how the P-1 remote stages are gated: they are cut, in ring
 *                order, into `groups` runs of consecutive stages; each run
 *                gets one completion dependency and one GEMM launch over its
 *                (contiguous) receive slots, and deliveries of slices that are
 *                adjacent in memory are merged into one copy. groups = P-1 is
 *                one gate per stage; 1 runs the local stage while everything
 *                else is delivered; 0 lets the library choose (one gate; a
 *                call under 20 GFLOP that meets the shape rules of
 *                TPG_IN_KERNEL_GATES, fits on the chip with its copy
 *                workgroups and is not being captured runs as one GEMM launch
 *                carrying its deliveries, the delivered slices' tiles waiting
 *                in-kernel for them; other calls under 1 GFLOP run on one
 *                stream). Values above P-1 are clamped. The
 *                result does not depend on it.
 *   schedule     TPG_ROTATE_A (the above) or TPG_ROTATE_B, the column dual
 *                (Approach: schedule AllGather1D_TilingCD_RotatingB; its
 *                layout is the plain reading stated here): A (M, K) is local,
 *                B arrives as P slices of n = N/P rows (NK: (n, K) each; KN:
 *                the (K, n) column block of B^T each), slice s from rank s,
 *                and stage t computes columns [s*n, (s+1)*n) of D (and reads
 *                those of C) from slice s = (rank + t) mod P, local first.
 *                TPG_ROTATE_B needs N % P == 0, n % 8 == 0 and
 *                TPG_EPI_ALPHA_BETA; a_slices[0] is then the whole A (the
 *                other entries are not read), b is not read, and b_slices
 *                holds the P slices. Receive slots then hold B slices (NK:
 *                back to back; KN: one (K, (P-1)*n) matrix).
 *   b_slices     TPG_ROTATE_B: host array of P device pointers; else unused.
 * All device pointers must be 16-byte aligned.
 * ---------------------------------------------------------------------- */
enum { TPG_ROTATE_A = 0, TPG_ROTATE_B = 1 };

typedef struct {
  int64_t M, N, K;
  int32_t P, rank;
  int32_t ab_dtype;
  int32_t b_layout;
  int32_t epilogue;
  const void* const* a_slices;
  const void* b;
  const void* c;
  void* d;
  float alpha, beta;
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;
  int32_t groups;
  int32_t schedule;
  const void* const* b_slices;
} tpg_ag_args;

size_t tpgemm_stage_ag_workspace_size(const tpg_ag_args* args);
tpg_status tpgemm_stage_ag(const tpg_ag_args* args, void* stream);

/* ------------------------------------------------------------------------
 * tpgemm_stage_ag without a workspace, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid hipMalloc). The same computation, kernels and results as
 * tpgemm_stage_ag (bit for bit); args->workspace and workspace_bytes are
 * ignored. The receive slots live in a static device array of 64 MiB
 * (67108864 bytes) that the library holds on every GPU it runs on until the
 * process ends. The first call on a device also creates the library's
 * internal streams and events and resolves that array's address; after
 * that, calls make no device allocation of any kind (no hipMalloc, no
 * graphs). Always issued eagerly.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: two calls in flight at once on one GPU (different streams, or
 * different host threads without stream ordering between them) race on it.
 * Calls on one stream are ordered and safe.
 * Errors: those of tpgemm_stage_ag; TPG_ERR_WORKSPACE when
 * tpgemm_stage_ag_workspace_size(args) exceeds 64 MiB (e.g. the e4m3
 * all-gather of 8192 x 8192 in P = 8 slices needs 56 MiB staged and 64 MiB
 * unstaged); TPG_ERR_UNSUPPORTED with TPG_FORCE_GRAPH or TPG_PROFILE.
 * ---------------------------------------------------------------------- */
tpg_status tpgemm_stage_ag_noalloc(const tpg_ag_args* args, void* stream);

/* ------------------------------------------------------------------------
 * Several column-parallel projections sharing one all-gathered input
 * ("Add dist GEMM attention and FFN backend", Structure: AllGatherLinearMulti
 * serves several linears that share one input with one all-gather;
 * AllGatherFusedQKVLinear is the three-way case with wq, wk and wv in their
 * stock layouts). For i < n_out:
 *   d[i] = alpha * A * b[i]^T,   A = the P row slices gathered in rank order,
 * staged exactly as tpgemm_stage_ag (stage t multiplies slice (rank + t) mod
 * P, local first, deliveries gated as there). The projections run as one
 * GEMM over the weights side by side, each output column block stored to
 * its own d[i]; weights that do not already sit back to back in memory are
 * copied side by side into the workspace first.
 *
 *   M, K         M % P == 0; K % 8 == 0 (bf16) or 16 (e4m3).
 *   n_out        1..4; n[i] % 8 == 0 (n[i] == 0 allowed: that output is
 *                untouched).
 *   a_slices     host array of P device pointers, (m, K) row-major each.
 *   b[i]         (n[i], K) row-major weights, ab_dtype.
 *   d[i]         bf16 (M, n[i]) row-major outputs; no overlaps with inputs
 *                or with each other.
 *   alpha        scale of every product (no C term, no bias).
 *   workspace    >= tpgemm_stage_ag_multi_workspace_size() bytes.
 *   flags, groups as for tpgemm_stage_ag (rotating A only).
 * Errors: as tpgemm_stage_ag, plus TPG_ERR_INVALID for n_out or an n[i].
 * ---------------------------------------------------------------------- */
enum { TPG_MAX_PROJ = 4 };

typedef struct {
  int64_t M, K;
  int32_t P, rank;
  int32_t ab_dtype;
  int32_t n_out;
  const void* const* a_slices;
  const void* b[TPG_MAX_PROJ];
  int64_t n[TPG_MAX_PROJ];
  void* d[TPG_MAX_PROJ];
  float alpha;
  uint32_t flags;
  int32_t groups;
  void* workspace;
  size_t workspace_bytes;
} tpg_agm_args;

size_t tpgemm_stage_ag_multi_workspace_size(const tpg_agm_args* args);
tpg_status tpgemm_stage_ag_multi(const tpg_agm_args* args, void* stream);

/* ------------------------------------------------------------------------
 * Reduce-scatter staged GEMM (the dual).
 * A (M, K) is this rank's K shard, so E = alpha * A * B^T is a partial sum
 * whose P row blocks of m = M/P belong to the P ranks ("Distributed GEMM",
 * Background, Figure 3: GEMM + Reduce Scatter; Approach: schedule
 * ReduceScatter1D_TilingA_RotatingC). Stage t computes block
 * (rank + 1 + t) mod P, own block last. Block b != rank of D receives the
 * emitted partial alpha * E_b; block rank receives
 * alpha * E_rank + sum_{j != rank} incoming[j], accumulated in fp32 and
 * rounded once to bf16. The incoming partials are delivered into the
 * workspace and gate the last stage only.
 *
 *   M, N, K      M % P == 0; K % 8 == 0 (bf16) or 16 (e4m3, NK only).
 *   a            (M, K) row-major.   b  (N, K) or (K, N) row-major.
 *   incoming     NULL, or a host array of P device pointers to bf16 (m, N)
 *                partials; entry [rank] and NULL entries are ignored.
 *   d            bf16 (M, N) output; must not overlap any input.
 *   workspace    >= tpgemm_stage_rs_workspace_size() bytes (receive slots).
 *   groups       the P-1 emitted blocks (stages 0..P-2) are computed by
 *                `groups` launches of consecutive blocks (0: library choice;
 *                clamped to [1, P-1]); the own block is always its own launch,
 *                gated on every delivery. The result does not depend on it.
 *   schedule     TPG_TILE_A (the above: row blocks) or TPG_TILE_B, the column
 *                dual (Approach: schedule ReduceScatter1D_TilingB_RotatingC;
 *                its layout is the plain reading stated here): the blocks
 *                are the P column blocks of n = N/P columns of E, block b
 *                owed to rank b, and the incoming partials are bf16 (M, n).
 *                TPG_TILE_B needs N % P == 0 and n % 8 == 0 (M % P is then
 *                not required).
 * ---------------------------------------------------------------------- */
enum { TPG_TILE_A = 0, TPG_TILE_B = 1 };

typedef struct {
  int64_t M, N, K;
  int32_t P, rank;
  int32_t ab_dtype;
  int32_t b_layout;
  const void* a;
  const void* b;
  const void* const* incoming;
  void* d;
  float alpha;
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;
  int32_t groups;
  int32_t schedule;
} tpg_rs_args;

size_t tpgemm_stage_rs_workspace_size(const tpg_rs_args* args);
tpg_status tpgemm_stage_rs(const tpg_rs_args* args, void* stream);

/* ------------------------------------------------------------------------
 * Weight gradient of the all-gather / reduce-scatter linears, staged over
 * the gathered token rows ("Add dist GEMM attention and FFN backend",
 * Structure: the backward of AllGatherLinear and LinearReduceScatter needs
 * the same two collectives; their data gradients are this library's RS and
 * AG calls with the weight read in the (K, N) layout, and their weight
 * gradients are this call):
 *   d (N, K) = alpha * sum_{i < M} G[i, n] * X[i, k]
 * with the M token rows split into P slices of m = M/P, one operand local
 * (all M rows) and the other arriving as the P slices (the all-gathered
 * operand: X = the gathered input for AllGatherLinear, G = the gathered
 * output gradient for LinearReduceScatter). Stage t contributes the rows of
 * slice (rank + t) mod P, local first, as in the all-gather form
 * ("Distributed GEMM", Background, Figures 3-4). The stages split the
 * contraction, so they add into one fp32 partial in the workspace and the
 * last launch rounds once to bf16.
 *
 *   M, N, K      M % P == 0, m % 64 == 0; N % 8 == 0; K % 8 == 0.
 *                M == 0 writes zeros to d.
 *   gathered     TPG_GATHER_X: local is G (M, N), slices are X's (m, K);
 *                TPG_GATHER_G: local is X (M, K), slices are G's (m, N).
 *   local        bf16 row-major, all M rows (never modified).
 *   slices       host array of P device pointers to bf16 row-major slices;
 *                slice s holds rows [s*m, (s+1)*m) of the gathered operand,
 *                [rank] is this rank's own (never modified).
 *   d            bf16 (N, K) row-major output; must not overlap any input.
 *   workspace    >= tpgemm_stage_wgrad_workspace_size() bytes: receive slots
 *                ((P-1) slices staged, P unstaged, none with TPG_NO_COPY)
 *                and, when the call makes more than one launch (staged,
 *                P > 1), the fp32 (N, K) partial.
 *   groups       >= 1: staged, the P-1 remote stages forming `groups` runs
 *                (clamped to P-1) after the local stage, each gated by its
 *                own deliveries. 0: library choice, which is one gathered
 *                launch (as TPG_UNSTAGED): measured on MI355X at the weight
 *                gradients of the e4m3 all-gather shape and of the SwiGLU
 *                block, it beats the staged chain (212 vs 233 us, 252 vs
 *                278 us, 162 vs 181 us), because every stage spans the whole
 *                output. The result depends on the choice only through
 *                fp32 rounding order.
 *   flags        as for tpgemm_stage_ag. TPG_UNSTAGED gathers all P slices
 *                in rank order first and makes one launch; with
 *                TPG_NO_COPY it needs the slices contiguous in rank order.
 * Errors: TPG_ERR_INVALID (P, rank, M % P, NULL pointers, overlaps, flags,
 * gathered), TPG_ERR_UNSUPPORTED (m % 64, N % 8, K % 8, alignment, sizes
 * past the kernel's 31-bit offsets), TPG_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
enum { TPG_GATHER_X = 0, TPG_GATHER_G = 1 };

typedef struct {
  int64_t M, N, K;
  int32_t P, rank;
  int32_t gathered;
  int32_t groups;
  const void* local;
  const void* const* slices;
  void* d;
  float alpha;
  uint32_t flags;
  void* workspace;
  size_t workspace_bytes;
} tpg_wg_args;

size_t tpgemm_stage_wgrad_workspace_size(const tpg_wg_args* args);
tpg_status tpgemm_stage_wgrad(const tpg_wg_args* args, void* stream);

/* ------------------------------------------------------------------------
 * Per-token-slot FFN, compute-only part of the p04 layer ("Computation and
 * communication example"; comp_only in "Interface, layout, and parameters").
 * For n < PB = P*B rows and slot l < L = T/P, with H the hidden width:
 *   z = x[n, l, :] @ w1[l] + b1[l];  u = z[:H], g = z[H:]
 *   h = LN(u; gx, bx) * silu(LN(g; gg, bg)),  LN with population variance
 *       and eps inside the square root
 *   y[n, l, :] = h @ wout[l] + bout[l]
 * All tensors bf16, row-major: x, y [PB, L, D]; w1 [L, D, 2H]; b1 [L, 2H];
 * wout [L, H, D]; bout [L, D]; gx, bx, gg, bg [H]. D % 8 == 0, H % 8 == 0.
 * Intermediates z (bf16) and h (bf16) live in the workspace
 * (>= ffn_slot_forward_workspace_size() bytes: two z buffers of PB x 2H,
 * one with TPG_SERIAL_STAGES, and the h of every slot, L x PB x H, so that
 * the second GEMM of all slots is one launch); accumulation and the
 * LayerNorm statistics are fp32.
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t PB, L, D, H;
  const void* x;
  const void* w1;
  const void* b1;
  const void* wout;
  const void* bout;
  const void* gx;
  const void* bx;
  const void* gg;
  const void* bg;
  float eps;
  void* y;
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;
} tpg_ffn_args;

size_t ffn_slot_forward_workspace_size(const tpg_ffn_args* args);
tpg_status ffn_slot_forward(const tpg_ffn_args* args, void* stream);

/* ------------------------------------------------------------------------
 * Backward of the per-token-slot FFN (p04 statement, "Interface, layout, and
 * parameters": autograd propagates through the layer to its input and every
 * parameter). With the forward's tensors and notation and the upstream
 * gradient dy = dL/dY [PB, L, D], for every slot l (a, b the two LayerNorm
 * outputs, s = silu(b)):
 *   dwout[l] = h^T dY_l;  dbout[l] = sum_n dY_l;  dh = dY_l wout[l]^T
 *   da = dh s;  db = dh a silu'(b);  dz = [LN_x^T(da) | LN_gate^T(db)]
 *   dw1[l] = X_l^T dz;  db1[l] = sum_n dz;  dx[:, l, :] = dz w1[l]^T
 *   dgx = sum over slots and rows of da * (u - mean u) / sqrt(var u + eps),
 *   dbx = sum of da; dgg, dbg likewise for the gate half
 * where LN^T is the LayerNorm input gradient. z and h are recomputed from x
 * (no activations are kept by the forward call). Products accumulate in fp32;
 * dh and dz are stored bf16 between the steps; column sums are fp32 in a
 * fixed block order (deterministic). Outputs are bf16 with the parameter
 * shapes: dx [PB, L, D], dw1 [L, D, 2H], db1 [L, 2H], dwout [L, H, D],
 * dbout [L, D], dgx, dbx, dgg, dbg [H].
 *   PB % 64 == 0 (the weight gradients contract over the PB rows), D % 8 == 0,
 *   H % 8 == 0, H <= 8192. Inputs are never modified; outputs must not
 *   overlap inputs or each other. workspace >=
 *   ffn_slot_backward_workspace_size() bytes. flags: TPG_PROFILE only
 *   (besides TPG_NO_GRAPH / TPG_FORCE_GRAPH).
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t PB, L, D, H;
  const void* x;
  const void* w1;
  const void* b1;
  const void* wout;
  const void* gx;
  const void* bx;
  const void* gg;
  const void* bg;
  float eps;
  const void* dy;
  void* dx;
  void* dw1;
  void* db1;
  void* dwout;
  void* dbout;
  void* dgx;
  void* dbx;
  void* dgg;
  void* dbg;
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;
} tpg_ffnb_args;

size_t ffn_slot_backward_workspace_size(const tpg_ffnb_args* args);
tpg_status ffn_slot_backward(const tpg_ffnb_args* args, void* stream);

/* ------------------------------------------------------------------------
 * All-to-All dispatch / combine as single-GPU layout permutes (p04 statement,
 * "Interface, layout, and parameters" and "Computation and communication
 * example"). With L = T/P (T % P == 0):
 *   dispatch_permute: dst[s*B + b, l, :] = src[s][b, rank*L + l, :]
 *     src: host array of P device pointers, each [B, T, D]; dst [P*B, L, D].
 *   combine_permute:  dst[b, s*L + l, :] = src[s][rank*B + b, l, :]
 *     src: host array of P device pointers, each [P*B, L, D]; dst [B, T, D].
 * elem_bytes is the element size (1, 2, 4 or 8); the copy is bit-exact.
 * dst must not overlap any source. 1 <= P <= 64.
 * ---------------------------------------------------------------------- */
tpg_status dispatch_permute(const void* const* src, void* dst, int32_t P, int32_t rank,
                            int64_t B, int64_t T, int64_t D, int32_t elem_bytes, void* stream);
tpg_status combine_permute(const void* const* src, void* dst, int32_t P, int32_t rank,
                           int64_t B, int64_t T, int64_t D, int32_t elem_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The stage delivery alone ("Distributed GEMM", Background, Figure 4: each
 * stage's input is copied in while the previous stage computes), as the
 * staged calls issue it: n slices of `bytes`, slice i from src[i] to
 * dst + i * dst_stride, on `stream`, with the copy kind the flags select
 * (TPG_COPY_KERNEL when none; only copy-kind flags are accepted). src is a
 * host array of n device pointers; dst must not overlap any source.
 * Bit-exact. Errors: TPG_ERR_INVALID (n outside [0, 64], NULL pointers,
 * dst_stride < bytes, overlap, flags).
 * ---------------------------------------------------------------------- */
tpg_status tpg_deliver(const void* const* src, int32_t n, size_t bytes, void* dst, size_t dst_stride,
                       uint32_t flags, void* stream);

/* ------------------------------------------------------------------------
 * Measurement aids, outside the staged GEMM: the rate the matrix cores
 * reach on this chip, against which the stage GEMMs' percent-of-peak figures
 * (the pages' measurement of GEMM efficiency as a fraction of the MMA peak)
 * can also be read.
 * tpg_device_info: compute units, peak engine clock and wall-clock counter
 *   rate (both kHz) of the current device; any pointer may be NULL.
 * tpg_mfma_probe: enqueues on `stream` `blocks` workgroups of 512 threads
 *   whose waves run `iters` iterations of four independent 32x32 MFMAs of
 *   `dtype` (TPG_BF16: 32x32x16, TPG_E4M3: 32x32x64) on register operands,
 *   with no memory traffic. *flop (if not NULL) receives the algorithmic
 *   flop count of the launch; the caller times it. `sink` is a device buffer
 *   of at least blocks * 8 * 16 bytes, 8-byte aligned: wave w writes
 *   sink[2w] = shader-clock ticks and sink[2w+1] = wall-clock ticks over its
 *   loop (their ratio times the wall-clock rate is the engine clock).
 *   Errors: TPG_ERR_UNSUPPORTED (dtype, alignment), TPG_ERR_INVALID (iters
 *   outside [1, 2^24], blocks outside [1, 65536]), TPG_ERR_WORKSPACE (sink
 *   too small or NULL).
 * ---------------------------------------------------------------------- */
tpg_status tpg_device_info(int32_t* cus, int32_t* clock_khz, int32_t* wall_clock_khz);
tpg_status tpg_mfma_probe(int32_t dtype, int32_t iters, int32_t blocks, uint64_t* sink, size_t sink_bytes,
                          double* flop, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics.
 * tpg_last_error: message of the last failing call on this host thread
 *   (empty string if none); valid until the next call on the thread.
 * tpg_release_caches: synchronises the device, then destroys cached graphs,
 *   internal streams and events. Later calls recreate them.
 * tpg_profile_read: after calls made with TPG_PROFILE (and a host sync),
 *   writes up to `cap` per-launch durations in milliseconds and their
 *   algorithmic work, oldest first, clears the record and returns how many
 *   were written. The work is the flop count of a GEMM launch, or the
 *   negative of the algorithmic HBM bytes of a row-kernel launch (the per-slot
 *   FFN's LayerNorm / SiLU pass: z read, h written).
 * ---------------------------------------------------------------------- */
const char* tpg_last_error(void);
void tpg_release_caches(void);
int32_t tpg_profile_read(float* ms, double* flop, int32_t cap);

#ifdef __cplusplus
}
#endif
#endif /* TPGEMM_H */
