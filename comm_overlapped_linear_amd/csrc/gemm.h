// Internal interface of the stage GEMM kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpg {

constexpr int kMaxAddList = 16;

// One GEMM launch: D = epilogue(alpha * A * B^T) over an (M, Ncols) block.
// A (M, K) with row stride lda elements; B (N, K) (nk) or (K, N) (kn) with
// row stride ldb. C / D / bias / addends are bf16 bit patterns.
constexpr int kMaxSeg = 4;
constexpr int kMaxCopySlices = 8;
constexpr int kMaxGateSlices = 8;
// Deadline of one in-kernel gate wait, in ticks of the 100 MHz wall clock
// (2 s; the low 32 bits of the clock are compared): a wave that has waited
// this long stops waiting, and its workgroup writes NaN for the whole tile
// instead of hanging.
constexpr unsigned kGateDeadline = 200000000u;

struct GemmParams {
  const void* a;
  const void* b;
  const uint16_t* c;
  uint16_t* d;
  const uint16_t* bias;        // [N out] or nullptr
  int64_t lda, ldb, ldc, ldd;  // in elements
  int M, N, K;                 // N = accumulator columns (2n for swiglu)
  float alpha, beta;
  // extra bf16 addends summed into rows [add_row0, add_row1) and columns
  // [add_col0, add_col1) of the output (the reduce-scatter incoming
  // partials), fp32 accumulate; addend element (r, c) of output (row, col)
  // is at (row - add_row0) * ld_add + (col - add_col0). Column bounds are
  // multiples of 8. Addends:
  //   add_list[0..n_add_list) and add_base + i * add_stride (i < n_add_strided)
  const uint16_t* add_list[kMaxAddList];
  int n_add_list;
  const uint16_t* add_base;
  int64_t add_stride;          // elements between strided addends
  int n_add_strided;
  int64_t ld_add;              // row stride of every addend (elements)
  int add_row0, add_row1;
  int add_col0, add_col1;
  int vec_ok;                  // 1 if ldc, ldd and ld_add are multiples of 8 (16-byte row vectors)
  // A run of stages that wraps past the last slice as one launch: with
  // wrap_row > 0 (a multiple of the tile height), the tiles at or past row
  // wrap_row write C's and D's rows wrap_back earlier, and with wrap_a also
  // read A's rows wrap_back earlier. (Direct-to-LDS kernel, row-major A.)
  int wrap_row;
  int wrap_back;
  int wrap_a;
  // The same along columns (a run of B column slices): with wrap_col > 0 (a
  // multiple of 256) the tiles at or past column wrap_col write C's and D's
  // columns wrap_back_col earlier; B is read unshifted. (Direct-to-LDS
  // kernel, alpha/beta epilogue, no addends.)
  int wrap_col;
  int wrap_back_col;
  // set by the launcher: a batched launch of 8k batches gives each XCD
  // whole batches (workgroup i, in dispatch order, takes batch i mod 8 of
  // its group of 8 and that batch's tiles in row-major order), so the tiles
  // an XCD runs at once share their A rows and B columns
  int batch_xcd;
  // batched launch (blockIdx.y = batch index): element strides between the
  // operands of consecutive batches (0 = shared); C and addends unbatched
  int batch;                   // >= 1
  int64_t a_bstride, b_bstride, d_bstride, bias_bstride;
  // CUs the tile choice may count on (0: the whole device). Stage launches
  // that run side by side each get their share, so that together they make
  // one wave of tiles instead of each sizing its tiles for the whole chip.
  int cu_budget;
  // Upper bound on the persistent grid (0: none): workgroups beyond it would
  // hold CUs that work beside this launch (shader-copy deliveries) needs.
  int grid_cap;
  // Contraction-major A (the weight gradient, launch_gemm_at): A is stored
  // (K, M) row-major with row stride lda, B is (K, N). Contraction rows wrap:
  // K-steps at contraction index >= a_kwrap (if > 0) read the A rows
  // kwrap_rows earlier, and likewise b_kwrap for B, so a run of stages in
  // ring order over one (tokens, .) tensor is one launch.
  int a_kwrap, b_kwrap;
  int64_t kwrap_rows;
  // fp32 chains between launches that split one contraction (weight
  // gradient only): acc_in (if set) is added before rounding, and acc_out (if
  // set) receives the fp32 result instead of bf16 d. Row stride ld_acc.
  const float* acc_in;
  float* acc_out;
  int64_t ld_acc;
  // Column-segmented output (several projections of one input): with
  // n_seg > 0, output columns [seg_col[i], seg_col[i+1]) go to seg_d[i] (row
  // stride seg_ld[i], column 0 = seg_col[i]) instead of d; seg_col[0] == 0,
  // boundaries multiples of 8. beta must be 0 and there is no bias.
  // Output store policy: 0 (default) non-temporal 16-byte stores (the
  // output is not read again by this call: measured 2-3% faster on MI355X);
  // 1 ordinary stores, for an intermediate the next kernel reads while it is
  // still in L2 / the Infinity Cache.
  int keep_out;
  int n_seg;
  int seg_col[kMaxSeg];
  uint16_t* seg_d[kMaxSeg];
  int64_t seg_ld[kMaxSeg];
  // Stage deliveries carried by this launch (a latency-bound staged call on
  // one stream): cp_blocks workgroups past the tile workgroups copy cp_n
  // slices of cp_nvec 16-byte vectors, slice i from cp_src[i] to cp_dst +
  // i * cp_dst_stride (16-byte aligned), and exit; 0 = none. Only the
  // direct-to-LDS kernel takes them (launch_gemm_carrying_copy).
  int cp_blocks;
  int cp_n;
  const uint8_t* cp_src[kMaxCopySlices];
  uint8_t* cp_dst;
  int64_t cp_dst_stride;
  int64_t cp_nvec;
  // Tile-rows per group of the direct-to-LDS kernel's tile order, set by its
  // launcher (callers leave 0: the kernel's own power-of-two rule).
  int tile_gm;
  // In-kernel stage gates: the staged all-gather as one launch over all M
  // rows. With a_slice_rows > 0 (a multiple of 128 dividing M), A is read
  // in slices of a_slice_rows rows (row stride lda) and a is not: slice
  // gate_local at a_local, and slice i != gate_local at a_slots + j * (its
  // bytes), j = (i - gate_local - 1) mod (M / a_slice_rows) its delivery
  // slot (slices arrive in ring order after the local one; gate_local = -1:
  // slice i at a_slots + i * (its bytes)). With gate != nullptr, a tile of
  // slice i != gate_local waits, before it issues the DMA of a K-step that
  // starts one of its chunks of gate_ksteps K-steps, until
  // gate[j * gate_nch + chunk] >= gate_need, and loads that slice
  // device-coherently (the copy kernel writes it from another stream while
  // this launch runs). gate_off = 1 skips the waits (negative control). Only
  // the direct-to-LDS kernel takes gates. When the launch also carries a copy
  // job (cp_blocks > 0) and gate != nullptr, each copy workgroup stores
  // system-scope and then adds 1 to gate[0]; with gate_nch = 0 and
  // gate_ksteps >= the K-steps, every tile of a delivered slice waits once,
  // before its first DMA, for gate[0] >= gate_need = cp_blocks.
  int a_slice_rows;
  const uint8_t* a_local;
  const uint8_t* a_slots;
  unsigned* gate;
  int gate_nch, gate_ksteps, gate_local, gate_off;
  unsigned gate_need;
  unsigned gate_deadline;   // ticks of the 100 MHz clock per wait; 0: kGateDeadline
  // Carried gates without a zeroing launch: with gate64 != nullptr the copy
  // workgroups come first (blockIdx.x < cp_blocks, ahead of the tiles), each
  // adds 1 to *gate64 once its stores have completed (one atomic add, no
  // compare-and-swap), and every tile of a delivered slice waits, before its
  // first DMA, for *gate64 == gate_want64: the word's count before this
  // launch (kept by the host, which knows every add to it) plus cp_blocks.
  // gate_nch and gate_ksteps are then 0 and the K-steps.
  unsigned long long* gate64;
  unsigned long long gate_want64;
};

// Raises a kernel's dynamic-LDS limit on the current device the first time
// it is launched there (the attribute may be per device); `done` holds one
// bit per device. Callers hold the library's lock.
inline hipError_t lds_limit_once(const void* kern, int bytes, uint64_t& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
  if (bit != 0 && (done & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done |= bit;
  return e;
}

enum GemmDtype { kBf16 = 0, kE4m3 = 1 };
enum GemmLayout { kNK = 0, kKN = 1 };
enum GemmEpi { kEpiAlphaBeta = 0, kEpiSwiglu = 1 };

// Compute units of the current device.
int device_cus();

// Output tiles the DMA launcher would make for this shape and CU budget.
int gemm_tiles(int M, int N, int dtype, int epi, int batch, int cu_budget);
// Output tiles of a gated launch (GemmParams a_slice_rows > 0).
int gated_tiles(int M, int N, int dtype, int epi, int copy_wgs);

// Picks a tile shape for (M, N) and launches on `s`. Host-side checks of the
// shapes and alignment are the caller's job (api.cpp validates every call).
hipError_t launch_gemm(const GemmParams& p, int dtype, int layout, int epi, hipStream_t s);
// Whether launch_gemm runs a wrapping launch (GemmParams wrap_row > 0) of
// these operands as one kernel (else as two launches, one per stretch).
bool wrap_in_one_launch(const GemmParams& p, int dtype, int layout);

// launch_gemm with the copy job of p (cp_n slices, see GemmParams) done by
// extra workgroups of the same launch when the direct-to-LDS kernel runs the
// GEMM; otherwise the copy runs as its own kernel right before the GEMM, in
// stream order. Either way the copy and the GEMM share no data.
hipError_t launch_gemm_carrying_copy(const GemmParams& p, int dtype, int layout, int epi, hipStream_t s);

// D (M, N) = alpha * A^T B with A (K, M) and B (K, N), both bf16 row-major
// (contraction over their rows), on the direct-to-LDS kernel; needs
// K % 64 == 0, M % 8 == 0 and N % 8 == 0 (checked by the caller).
hipError_t launch_gemm_at(const GemmParams& p, hipStream_t s);
bool gemm_at_supported(const GemmParams& p);

// Register-only MFMA rate probe: `blocks` workgroups of kProbeThreads, each
// wave running `iters` iterations of four independent MFMAs; sink holds two
// uint64 per wave (shader-clock ticks, wall-clock ticks over the loop).
constexpr int kProbeThreads = 512;
double probe_flop_per_iter(int dtype);    // per workgroup and iteration
hipError_t launch_mfma_probe(int dtype, int iters, int blocks, unsigned long long* sink, hipStream_t s);

// Row-wise LayerNorm(u) * silu(LayerNorm(g)) over z = [u | g] (each H wide).
hipError_t launch_ln_silu(const uint16_t* z, int64_t ldz, uint16_t* h, int64_t ldh, int rows, int H,
                          const uint16_t* gx, const uint16_t* bx, const uint16_t* gg,
                          const uint16_t* bg, float eps, hipStream_t s);

// FFN backward, row part: dz = [du | dg] from z = [u | g] and dh, plus fp32
// column partials (one block of rows per workgroup, nblk workgroups):
// part_gb [nblk][4][H] = (da xu, da, db xg, db), added to the buffer's
// contents when accumulate != 0; part_b1 [nblk][2H] = (du, dg).
hipError_t launch_ffn_bwd_rows(const uint16_t* z, int64_t ldz, const uint16_t* dh, int64_t lddh, uint16_t* dz,
                               int64_t lddz, int rows, int H, const uint16_t* gx, const uint16_t* bx,
                               const uint16_t* gg, const uint16_t* bg, float eps, float* part_gb, int accumulate,
                               float* part_b1, int nblk, hipStream_t s);
// out[c] = bf16(sum over nblk blocks of part[b * blk_stride + c]).
hipError_t launch_colsum_f32(const float* part, int nblk, int64_t blk_stride, int ncols, uint16_t* out,
                             hipStream_t s);
// part[b][c] = fp32 sum of src[row * ld + c] over the b-th block of rows.
hipError_t launch_colsum_bf16(const uint16_t* src, int rows, int cols, int64_t ld, float* part, int nblk,
                              hipStream_t s);

// Zeroes `bytes` (a multiple of 16) at p (16-byte aligned) with a kernel, so
// the fill may sit in a captured graph.
hipError_t launch_fill_zero16(void* p, size_t bytes, hipStream_t s);

// Stage deliveries K-chunk by K-chunk for in-kernel gates: n slices of rows
// x row_bytes (row-major, src row stride = dst row stride = row_bytes), slice
// i from src[i] to dst + i * rows * row_bytes, in nch chunks of chunk_bytes
// of every row (the last may be shorter); after a workgroup has stored its
// rows of chunk c of slice i it adds 1 to gate[i * nch + c], so that a
// chunk is complete when the count reaches wg_per_slice (the host takes
// chunk_deliver_wgs_per_slice(rows)). Stores are system-scope (visible at
// the device coherence point once complete). 16-byte alignment of
// everything.
struct ChunkDeliverParams {
  const uint8_t* src[kMaxGateSlices];
  uint8_t* dst;
  unsigned* gate;
  int64_t rows, row_bytes, chunk_bytes;
  int n, nch, wg_per_slice;
};
int chunk_deliver_wgs_per_slice(int64_t rows);
hipError_t launch_chunk_deliver(const ChunkDeliverParams& p, hipStream_t s);

// Stage deliveries (the library's own copy kernel): n slices of `bytes`,
// slice i from src[i] to dst + i * dst_stride. deliver_ok says whether the
// kernel takes the arguments (16-byte aligned pointers, sizes and stride,
// n <= kMaxDeliver); the caller uses a runtime copy otherwise.
constexpr int kMaxDeliver = 64;
struct DeliverParams {
  const uint8_t* src[kMaxDeliver];
  uint8_t* dst;
  int64_t dst_stride;
  int64_t nvec;            // 16-byte vectors per slice
};
bool deliver_ok(const void* const* src, int n, size_t bytes, const void* dst, size_t dst_stride);
hipError_t launch_deliver(const void* const* src, int n, size_t bytes, void* dst, size_t dst_stride, hipStream_t s);

// Static receive-slot scratch of the allocation-free all-gather entry point
// (scratch.hip): its device address on the current device, resolved with
// hipGetSymbolAddress on the first request per device (callers hold the
// library's lock).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
hipError_t static_scratch(void** ptr);
// Gate words of the carried in-kernel gates (scratch.hip): a static device
// array, zero when the library loads, one 64-bit counter per call slot,
// resolved like the scratch. Calls take slots round-robin; a counter only
// ever grows, and the host keeps each one's total, so a word never has to
// be cleared before a call.
constexpr int kGateWords = 1 << 20;
hipError_t gate_words(unsigned long long** ptr);
// Words of the cross-stream dependencies of eager calls (scratch.hip): a
// static device array, zero at load; each dependency takes a word
// round-robin and a value that grows on every reuse of the word (the host
// hands a word out again only once its previous users have completed).
constexpr int kSyncWords = 65536;
hipError_t sync_words(unsigned long long** ptr);

// Bit-exact run permute used by dispatch / combine.
struct PermuteParams {
  const uint8_t* src[64];
  uint8_t* dst;
  int64_t B;              // runs per source
  int64_t run_bytes;
  int64_t src_base, src_bstride;
  int64_t dst_sstride, dst_bstride;
};
hipError_t launch_permute(const PermuteParams& p, int P, hipStream_t s);

}  // namespace tpg
