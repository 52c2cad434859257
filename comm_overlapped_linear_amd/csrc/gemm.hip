// Stage GEMM kernels for gfx950 (CDNA4): bf16 and OCP fp8-e4m3 MFMA tiles.
//
// Computes one stage of the staged tensor-parallel GEMM, D = alpha * A * B^T
// + beta * C on an (M, N) block ("Pytorch Op for blackwell distributed gemm",
// Usage; "Distributed GEMM", Approach), with the epilogues of the per-slot FFN
// (bias, p04 statement "Computation and communication example"), of the
// SwiGLU pair (silu(x w1) * (x w3), torchtitan PR #4044, Structure) and of the
// reduce-scatter own block (sum of incoming partials).
//
// Design (gfx950):
//  * 256 threads = 4 wave64s in a 2 x 2 grid; block tiles 256x256, 256x128 or
//    128x128; each wave owns a (BM/2) x (BN/2) sub-tile of 32x32 MFMA blocks.
//  * One K-step moves 128 bytes of K per tile row (64 bf16 or 128 fp8).
//    Global -> register loads are 16-byte vectors; tiles live in LDS as
//    [row][128 B] with the 16-byte chunk index XOR-swizzled by the row so the
//    MFMA fragment reads (32 rows x 16 B per half-wave) spread over all banks.
//    Two LDS buffers: the next K-step's global loads are in flight while the
//    current one feeds the MFMAs; one barrier per K-step.
//  * B in (K, N) layout (the pages' weight layout) is transposed 8x8 in
//    registers on its way to LDS, so both layouts share the MFMA loop.
//  * The MFMA takes the B fragment as its first operand, so each lane ends up
//    holding 4 consecutive output columns of one row: 8-byte C loads and D
//    stores in the epilogue.
//  * bf16: v_mfma_f32_32x32x16_bf16 (8 bf16 per lane). fp8: the unscaled
//    v_mfma_f32_32x32x64_f8f6f4 with both formats E4M3 (32 bytes per lane).
//    Accumulation is fp32; D is rounded once to bf16 (nearest even).
#include "common.h"
#include <algorithm>
#include <atomic>

#include "gemm.h"

namespace tpg {

namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;   // K bytes per tile row per K-step

// 16-byte chunk swizzle inside an LDS row of ROWB bytes (128: 8 chunks,
// 64: 4 chunks). Any 16 consecutive rows read at one logical chunk hit 16
// distinct 16-byte bank groups of a 256-byte bank window.
template <int ROWB>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (ROWB == 128) return chunk ^ ((row >> 1) & 7);
  else return chunk ^ ((row >> 2) & 3);
}

struct OpBf16 {
  static constexpr int kElemBytes = 2;
  static constexpr int kSliceBytes = 32;   // k bytes per lane-half pair of one MFMA
  static constexpr int kSubSteps = 4;      // 32-byte k slices per 128-byte K-step
  static constexpr int kReadsPerFrag = 1;
  typedef bf16x8_t frag_t;
  template <int ROWB = kRowBytes>
  __device__ static frag_t load(const uint8_t* lds, int row, int kk, int half) {
    const int c = kk * 2 + half;
    uint4 v = *reinterpret_cast<const uint4*>(lds + row * ROWB + swz<ROWB>(row, c) * 16);
    return __builtin_bit_cast(frag_t, v);
  }
  __device__ static f32x16_t mma(frag_t x, frag_t y, f32x16_t acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc, 0, 0, 0);
  }
};

struct OpE4m3 {
  static constexpr int kElemBytes = 1;
  static constexpr int kSliceBytes = 64;
  static constexpr int kSubSteps = 2;      // 64-byte k slices per 128-byte K-step
  static constexpr int kReadsPerFrag = 2;
  typedef i32x8_t frag_t;
  template <int ROWB = kRowBytes>
  __device__ static frag_t load(const uint8_t* lds, int row, int kk, int half) {
    const int c = kk * 4 + half * 2;
    uint4 lo = *reinterpret_cast<const uint4*>(lds + row * ROWB + swz<ROWB>(row, c) * 16);
    uint4 hi = *reinterpret_cast<const uint4*>(lds + row * ROWB + swz<ROWB>(row, c + 1) * 16);
    i32x8_t f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
  }
  __device__ static f32x16_t mma(frag_t x, frag_t y, f32x16_t acc) {
    // format 0 = FP8 E4M3 for both operands; scale operands 0 select the
    // unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc, 0, 0, 0, 0, 0, 0);
  }
};

// Global column of B feeding LDS B-row i of tile tn (or -1 past the edge).
template <bool SWIGLU, int BN>
__device__ __forceinline__ int b_col(int tn, int i, int N) {
  if (!SWIGLU) {
    const int n = tn * BN + i;
    return n < N ? n : -1;
  }
  const int nh = N >> 1;
  const int half = i >= BN / 2;
  const int u = tn * (BN / 2) + (i - half * (BN / 2));
  return u < nh ? u + half * nh : -1;
}

// Operand pointers of batch z of a batched launch. (The parameter
// block itself stays in the kernel-argument segment: a private copy would be
// spilled to scratch because the epilogue indexes add_list dynamically.)
struct BatchPtrs {
  const uint8_t* a;
  const uint8_t* b;
  uint16_t* d;
  const uint16_t* bias;
};

template <int EB>
__device__ __forceinline__ BatchPtrs batch_ptrs(const GemmParams& p, int64_t z) {
  BatchPtrs q;
  q.a = static_cast<const uint8_t*>(p.a) + z * p.a_bstride * EB;
  q.b = static_cast<const uint8_t*>(p.b) + z * p.b_bstride * EB;
  q.d = p.d + z * p.d_bstride;
  q.bias = p.bias ? p.bias + z * p.bias_bstride : nullptr;
  return q;
}

// Adds beta * C, the bias and the addends to x[0..8) for output (row, col ..
// col + 7) and stores bf16. Full 16-byte vectors when the row stride allows.
__device__ __forceinline__ void add_row8(const uint16_t* src, int64_t off, bool vec, int n, float scale,
                                         float* x) {
  if (vec) {
    const uint4 c = *reinterpret_cast<const uint4*>(src + off);
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] += scale * bf16_to_f32(w[e] & 0xffff);
      x[2 * e + 1] += scale * bf16_to_f32(w[e] >> 16);
    }
  } else {
    for (int e = 0; e < n; ++e) x[e] += scale * bf16_to_f32(src[off + e]);
  }
}

// Destination of output vector (row, col .. col + 7): d, or with a
// column-segmented output the segment holding col (uniform selects; segment
// boundaries are multiples of 8, so a vector never straddles two).
__device__ __forceinline__ uint16_t* out_at(const GemmParams& p, const BatchPtrs& bp, int row, int col) {
  if (p.n_seg == 0) return bp.d + static_cast<int64_t>(row) * p.ldd + col;
  // the segment index, then its fields by a per-lane index into the
  // parameter block (memory loads, not SGPRs that would stay live over the
  // whole kernel)
  int t = 0;
#pragma unroll
  for (int i = 1; i < kMaxSeg; ++i) t += (i < p.n_seg && col >= p.seg_col[i]) ? 1 : 0;
  uint16_t* base = p.seg_d[t];
  const int64_t ld = p.seg_ld[t];
  const int c0 = p.seg_col[t];
  return base + static_cast<int64_t>(row) * ld + (col - c0);
}

template <bool F32IO>
__device__ __forceinline__ void epilogue_vec8(const GemmParams& p, const BatchPtrs& bp, int row, int col, int nout,
                                              float* x) {
  const int n = min(8, nout - col);
  const bool vec = p.vec_ok && n == 8;
  if constexpr (F32IO) {
    if (p.acc_in) {
      const float* src = p.acc_in + static_cast<int64_t>(row) * p.ld_acc + col;
      if (vec) {
        const float4 lo = *reinterpret_cast<const float4*>(src), hi = *reinterpret_cast<const float4*>(src + 4);
        x[0] += lo.x; x[1] += lo.y; x[2] += lo.z; x[3] += lo.w;
        x[4] += hi.x; x[5] += hi.y; x[6] += hi.z; x[7] += hi.w;
      } else {
        for (int e = 0; e < n; ++e) x[e] += src[e];
      }
    }
  }
  if (p.beta != 0.0f) add_row8(p.c, static_cast<int64_t>(row) * p.ldc + col, vec, n, p.beta, x);
  if (bp.bias) add_row8(bp.bias, col, n == 8, n, 1.0f, x);
  if (row >= p.add_row0 && row < p.add_row1 && col >= p.add_col0 && col < p.add_col1) {
    const int64_t off = static_cast<int64_t>(row - p.add_row0) * p.ld_add + (col - p.add_col0);
    for (int t = 0; t < p.n_add_list; ++t) add_row8(p.add_list[t], off, vec, n, 1.0f, x);
    for (int t = 0; t < p.n_add_strided; ++t) add_row8(p.add_base + t * p.add_stride, off, vec, n, 1.0f, x);
  }
  if constexpr (F32IO) {
    if (p.acc_out) {
      float* dst = p.acc_out + static_cast<int64_t>(row) * p.ld_acc + col;
      if (vec) {
        *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(x[4], x[5], x[6], x[7]);
      } else {
        for (int e = 0; e < n; ++e) dst[e] = x[e];
      }
      return;
    }
  }
  uint16_t* dst = out_at(p, bp, row, col);
  if (vec) {
    uint4 o;
    o.x = pack_bf16x2(x[0], x[1]);
    o.y = pack_bf16x2(x[2], x[3]);
    o.z = pack_bf16x2(x[4], x[5]);
    o.w = pack_bf16x2(x[6], x[7]);
    *reinterpret_cast<uint4*>(dst) = o;
  } else {
    for (int e = 0; e < n; ++e) dst[e] = f32_to_bf16(x[e]);
  }
}

__device__ __forceinline__ void add_vec8(const uint4 c, float scale, float* x) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] += scale * bf16_to_f32(w[e] & 0xffff);
    x[2 * e + 1] += scale * bf16_to_f32(w[e] >> 16);
  }
}

// The LDS sweep of one epilogue pass for a tile with no edge: every output
// vector exists and rows are 16-byte aligned, so for each input (C, bias,
// then each addend in order) the loads of all NV vectors of a thread are
// issued together before any is used. The arithmetic, and so the result, is
// that of epilogue_vec8; only the memory latency is overlapped.
template <int NV, bool F32IO>
__device__ __forceinline__ void sweep_interior(const GemmParams& p, const BatchPtrs& bp, const float* stage,
                                               int sld, int tid, int nt, int vec_per_row, int row0, int wtm,
                                               int tcol0) {
  float x[NV][8];
  int row[NV], col[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int v = tid + u * nt;
    const int sr = v / vec_per_row, sc = (v % vec_per_row) * 8;
    row[u] = row0 + (sr >> 5) * wtm + (sr & 31);
    col[u] = tcol0 + sc;
    const float4 lo = *reinterpret_cast<const float4*>(stage + sr * sld + sc);
    const float4 hi = *reinterpret_cast<const float4*>(stage + sr * sld + sc + 4);
    x[u][0] = lo.x; x[u][1] = lo.y; x[u][2] = lo.z; x[u][3] = lo.w;
    x[u][4] = hi.x; x[u][5] = hi.y; x[u][6] = hi.z; x[u][7] = hi.w;
  }
  if constexpr (F32IO) {
    if (p.acc_in) {
      float4 f[NV][2];
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const float* src = p.acc_in + int64_t(row[u]) * p.ld_acc + col[u];
        f[u][0] = *reinterpret_cast<const float4*>(src);
        f[u][1] = *reinterpret_cast<const float4*>(src + 4);
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        x[u][0] += f[u][0].x; x[u][1] += f[u][0].y; x[u][2] += f[u][0].z; x[u][3] += f[u][0].w;
        x[u][4] += f[u][1].x; x[u][5] += f[u][1].y; x[u][6] += f[u][1].z; x[u][7] += f[u][1].w;
      }
    }
  }
  uint4 c[NV];
  if (p.beta != 0.0f) {
#pragma unroll
    for (int u = 0; u < NV; ++u) c[u] = *reinterpret_cast<const uint4*>(p.c + int64_t(row[u]) * p.ldc + col[u]);
#pragma unroll
    for (int u = 0; u < NV; ++u) add_vec8(c[u], p.beta, x[u]);
  }
  if (bp.bias) {
#pragma unroll
    for (int u = 0; u < NV; ++u) c[u] = *reinterpret_cast<const uint4*>(bp.bias + col[u]);
#pragma unroll
    for (int u = 0; u < NV; ++u) add_vec8(c[u], 1.0f, x[u]);
  }
  const int nadd = p.n_add_list + p.n_add_strided;
  if (nadd > 0 && p.add_row1 > p.add_row0 && p.add_col1 > p.add_col0) {
    // vectors outside the addend rectangle take no addends; their (clamped,
    // valid) loads are discarded
    bool in[NV];
    int64_t off[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      in[u] = row[u] >= p.add_row0 && row[u] < p.add_row1 && col[u] >= p.add_col0 && col[u] < p.add_col1;
      const int ra = min(max(row[u] - p.add_row0, 0), max(p.add_row1 - p.add_row0 - 1, 0));
      const int ca = min(max(col[u] - p.add_col0, 0), max(p.add_col1 - p.add_col0 - 8, 0));
      off[u] = int64_t(ra) * p.ld_add + ca;
    }
    // each addend is read once: non-temporal, so it does not evict what the
    // launches running beside this one keep in L2 (bf16 reduce-scatter
    // workload 447 -> 438 us)
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    for (int t = 0; t < nadd; ++t) {
      const uint16_t* src = t < p.n_add_list ? p.add_list[t] : p.add_base + (t - p.n_add_list) * p.add_stride;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off[u]));
        c[u] = make_uint4(v.x, v.y, v.z, v.w);
      }
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (in[u]) add_vec8(c[u], 1.0f, x[u]);
    }
  }
  if constexpr (F32IO) {
    if (p.acc_out) {
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        float* dst = p.acc_out + int64_t(row[u]) * p.ld_acc + col[u];
        *reinterpret_cast<float4*>(dst) = make_float4(x[u][0], x[u][1], x[u][2], x[u][3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(x[u][4], x[u][5], x[u][6], x[u][7]);
      }
      return;
    }
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    uint4 o;
    o.x = pack_bf16x2(x[u][0], x[u][1]);
    o.y = pack_bf16x2(x[u][2], x[u][3]);
    o.z = pack_bf16x2(x[u][4], x[u][5]);
    o.w = pack_bf16x2(x[u][6], x[u][7]);
    uint4* dst = reinterpret_cast<uint4*>(out_at(p, bp, row[u], col[u]));
    if (p.keep_out) {
      *dst = o;
    } else {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 v = {o.x, o.y, o.z, o.w};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
    }
  }
}

// Epilogue shared by both kernels, staged through LDS in FM passes of WM x 32
// rows: (1) every wave writes alpha * acc (or silu(u) * v) of its rows
// wm*WTM + i*32 + [0, 32) as fp32 into a [WM*32][BNO + 4] LDS block; (2) all
// threads sweep that block in 8-column vectors: + beta * C, + bias, + addends,
// one bf16 rounding, 16-byte coalesced stores. The caller has synchronised
// the workgroup, so the LDS is free.
template <int BM, int BN, int WM, int WN, bool SWIGLU, bool F32IO = false>
__device__ __forceinline__ void store_tile(const GemmParams& p, const BatchPtrs& bp,
                                           const f32x16_t (&acc)[BM / WM / 32][BN / WN / 32], uint8_t* smem,
                                           int tm, int tn) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int m0 = tm * BM;
  constexpr int JN = SWIGLU ? FN / 2 : FN;     // output column blocks per wave
  constexpr int BNO = SWIGLU ? BN / 2 : BN;    // output columns per tile
  constexpr int WNO = BNO / WN;                // output columns per wave
  constexpr int SLD = BNO + 4;                 // padded LDS row (floats)
  float* stage = reinterpret_cast<float*>(smem);
  const int nout = SWIGLU ? (p.N >> 1) : p.N;
  const int tcol0 = tn * BNO;
  constexpr int VEC_PER_ROW = BNO / 8;
  constexpr int VEC_PASS = WM * 32 * VEC_PER_ROW;
  constexpr int NV = VEC_PASS / NT;            // 8-column vectors per thread and pass
  static_assert(NV * NT == VEC_PASS, "each thread sweeps the same number of vectors");
  const bool interior = p.vec_ok && m0 + BM <= p.M && tcol0 + BNO <= nout;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    float* wst = stage + (wm * 32 + l32) * SLD + wn * WNO + half * 4;
#pragma unroll
    for (int j = 0; j < JN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 o;
        float* ov = reinterpret_cast<float*>(&o);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x = p.alpha * acc[i][j][g * 4 + q];
          if constexpr (SWIGLU) {
            ov[q] = silu_f32(x) * (p.alpha * acc[i][j + FN / 2][g * 4 + q]);
          } else {
            ov[q] = x;
          }
        }
        *reinterpret_cast<float4*>(wst + j * 32 + g * 8) = o;
      }
    }
    __syncthreads();
    if (interior) {
      // at most four vectors in flight per thread (two with the fp32 chain,
      // whose inputs are twice as wide): register budget
      constexpr int GMAX = F32IO ? 2 : 4;
      constexpr int G = NV < GMAX ? NV : GMAX;
      static_assert(NV % G == 0, "vector groups");
#pragma unroll
      for (int g0 = 0; g0 < NV; g0 += G)
        sweep_interior<G, F32IO>(p, bp, stage, SLD, tid + g0 * NT, NT, VEC_PER_ROW, m0 + i * 32, WTM, tcol0);
    } else {
      for (int v = tid; v < VEC_PASS; v += NT) {
        const int sr = v / VEC_PER_ROW, sc = (v % VEC_PER_ROW) * 8;
        const int row = m0 + (sr >> 5) * WTM + i * 32 + (sr & 31);
        const int col = tcol0 + sc;
        if (row >= p.M || col >= nout) continue;
        float x[8];
        const float4 lo = *reinterpret_cast<const float4*>(stage + sr * SLD + sc);
        const float4 hi = *reinterpret_cast<const float4*>(stage + sr * SLD + sc + 4);
        x[0] = lo.x; x[1] = lo.y; x[2] = lo.z; x[3] = lo.w;
        x[4] = hi.x; x[5] = hi.y; x[6] = hi.z; x[7] = hi.w;
        epilogue_vec8<F32IO>(p, bp, row, col, nout, x);
      }
    }
    __syncthreads();
  }
}


template <typename Op, int BM, int BN, bool KN, bool SWIGLU>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const GemmParams p) {
  const BatchPtrs bp = batch_ptrs<Op::kElemBytes>(p, blockIdx.y);
  constexpr int WM = 2, WN = 2;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  constexpr int A_LD = BM * 8 / kThreads;            // 16-byte chunks per thread
  constexpr int B_LD_NK = BN * 8 / kThreads;
  constexpr int B_BLK_KN = (BN / 8) * 8;             // 8x8 blocks per K-step (kn, bf16)
  constexpr int B_LD_KN = (B_BLK_KN + kThreads - 1) / kThreads;
  static_assert(!SWIGLU || (FN % 2 == 0), "swiglu pairs wave column blocks");
  static_assert(2 * 32 * ((SWIGLU ? BN / 2 : BN) + 4) * 4 <= 2 * (BM + BN) * kRowBytes, "epilogue stage fits in LDS");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int ntm = (p.M + BM - 1) / BM;
  const int tm = blockIdx.x % ntm;
  const int tn = blockIdx.x / ntm;
  const int m0 = tm * BM;

  const uint8_t* A = bp.a;
  const uint8_t* Bp = bp.b;
  const int64_t lda_b = p.lda * Op::kElemBytes;
  const int64_t ldb_b = p.ldb * Op::kElemBytes;
  const int kbytes = p.K * Op::kElemBytes;
  const int nk = (kbytes + kRowBytes - 1) / kRowBytes;

  uint4 ra[A_LD];
  uint4 rb[KN ? B_LD_KN * 8 : B_LD_NK];

  auto load_global = [&](int kt) {
    const int k0b = kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int id = i * kThreads + tid;
      const int r = id >> 3, c = id & 7;
      const int grow = m0 + r, kb = k0b + c * 16;
      ra[i] = make_uint4(0, 0, 0, 0);
      if (grow < p.M && kb < kbytes) ra[i] = *reinterpret_cast<const uint4*>(A + grow * lda_b + kb);
    }
    if (!KN) {
#pragma unroll
      for (int i = 0; i < B_LD_NK; ++i) {
        const int id = i * kThreads + tid;
        const int r = id >> 3, c = id & 7;
        const int n = b_col<SWIGLU, BN>(tn, r, p.N);
        const int kb = k0b + c * 16;
        rb[i] = make_uint4(0, 0, 0, 0);
        if (n >= 0 && kb < kbytes) rb[i] = *reinterpret_cast<const uint4*>(Bp + n * ldb_b + kb);
      }
    } else {
      // 8x8 bf16 blocks: block = (kb8 = k/8 within the step, nb = n/8 within the tile)
#pragma unroll
      for (int i = 0; i < B_LD_KN; ++i) {
        const int blk = i * kThreads + tid;
        const int kb8 = blk & 7, nb = blk >> 3;
        const int n = (blk < B_BLK_KN) ? b_col<SWIGLU, BN>(tn, nb * 8, p.N) : -1;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int k = kt * (kRowBytes / 2) + kb8 * 8 + r;
          rb[i * 8 + r] = make_uint4(0, 0, 0, 0);
          if (n >= 0 && k < p.K)
            rb[i * 8 + r] = *reinterpret_cast<const uint4*>(Bp + (int64_t)k * ldb_b + n * 2);
        }
      }
    }
  };

  auto store_lds = [&](int buf) {
    uint8_t* la = smem + buf * (A_BYTES + B_BYTES);
    uint8_t* lb = la + A_BYTES;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int id = i * kThreads + tid;
      const int r = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(la + r * kRowBytes + swz<kRowBytes>(r, c) * 16) = ra[i];
    }
    if (!KN) {
#pragma unroll
      for (int i = 0; i < B_LD_NK; ++i) {
        const int id = i * kThreads + tid;
        const int r = id >> 3, c = id & 7;
        *reinterpret_cast<uint4*>(lb + r * kRowBytes + swz<kRowBytes>(r, c) * 16) = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_LD_KN; ++i) {
        const int blk = i * kThreads + tid;
        if (blk < B_BLK_KN) {
          const int kb8 = blk & 7, nb = blk >> 3;
          const uint32_t* w = reinterpret_cast<const uint32_t*>(&rb[i * 8]);  // w[r*4 + q]: (k=r, n=2q,2q+1)
#pragma unroll
          for (int c = 0; c < 8; ++c) {            // output row n = nb*8 + c holds k = kb8*8 .. +7
            const int q = c >> 1;
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t lo = w[(2 * j) * 4 + q], hi = w[(2 * j + 1) * 4 + q];
              o[j] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            const int r = nb * 8 + c;
            *reinterpret_cast<uint4*>(lb + r * kRowBytes + swz<kRowBytes>(r, kb8) * 16) =
                make_uint4(o[0], o[1], o[2], o[3]);
          }
        }
      }
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // LDS row (within the B tile) read by this lane for wave column block j
  auto b_row = [&](int j) {
    if constexpr (!SWIGLU) {
      return wn * WTN + j * 32 + l32;
    } else {
      const int hj = j % (FN / 2), part = j / (FN / 2);
      return part * (BN / 2) + wn * (WTN / 2) + hj * 32 + l32;
    }
  };

  if (nk > 0) {
    load_global(0);
    store_lds(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_global(kt + 1);
    const uint8_t* la = smem + cur * (A_BYTES + B_BYTES);
    const uint8_t* lb = la + A_BYTES;
#pragma unroll
    for (int kk = 0; kk < Op::kSubSteps; ++kk) {
      typename Op::frag_t fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = Op::load(la, wm * WTM + i * 32 + l32, kk, half);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = Op::load(lb, b_row(j), kk, half);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Op::mma(fb[j], fa[i], acc[i][j]);
    }
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  store_tile<BM, BN, 2, 2, SWIGLU>(p, bp, acc, smem, tm, tn);
}

// Workgroup -> output tile. Consecutive workgroup ids are dealt round-robin
// to the 8 XCDs, each with its own L2, so id b is first re-numbered to
// (b mod 8) * (nt / 8) + b / 8: each XCD then owns one contiguous run of the
// tile order. The tile order walks groups of GM tile-rows column by column,
// with GM chosen so that one XCD's run is a compact rectangle of tiles
// (about sqrt(run) rows): its A rows and B columns are shared in its L2.
// The launcher may fix GM instead (gm_fixed > 0; see group_rows).
__device__ __forceinline__ void tile_of_block(int vt, int nt, int ntm, int gm_fixed, int& tm, int& tn) {
  int bid = vt;
  if ((nt & 7) == 0) bid = (bid & 7) * (nt >> 3) + (bid >> 3);
  const int run = (nt & 7) == 0 ? (nt >> 3) : nt;
  int gm = gm_fixed;
  if (gm <= 0) {
    gm = 1;
    while ((gm * 2) * (gm * 2) <= run && gm * 2 <= ntm) gm *= 2;
  }
  const int ntn = nt / ntm;
  const int group = bid / (gm * ntn);
  const int first = group * gm;
  const int rows = min(gm, ntm - first);
  const int in_group = bid - group * gm * ntn;
  tm = first + in_group % rows;
  tn = in_group / rows;
}

// ---------------------------------------------------------------------------
// v2 mainloop: direct-to-LDS loads (gfx950 global_load_lds_dwordx4).
// Each 16-byte chunk goes from HBM straight into its LDS slot, with no
// staging registers, into a ring of STAGES tile buffers, so several K-steps
// of loads are in flight while the MFMAs consume the oldest one. A DMA
// instruction of one wave fills 1 KB of LDS, lane q at byte 16 q, i.e. eight
// 128-byte rows; the XOR swizzle is realised by which global chunk lane q
// fetches. The loads are issued from inline assembly so that the compiler
// does not order every LDS read after every outstanding DMA; the waits are
// explicit (vmcnt for this wave's DMA, then a barrier for everyone's).
// Requires K * element size to be a multiple of 128 bytes and B in (N, K).
// m0 carries the LDS destination; nothing else in these kernels uses m0 on
// gfx950 (LDS instructions do not read it), so clobbering it is safe here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Whether a DMA tile shape runs as persistent workgroups. The fp8 256 x 256
// tile and the contraction-major-A 256 x 256 tile do not: their registers
// leave no room for the tile loop (the loop would spill), so they keep one
// workgroup per tile.
template <typename Op, int BM, int BN, bool AT = false>
constexpr bool persistent_tiles() {
  return !((Op::kElemBytes == 1 || AT) && BM == 256 && BN == 256);
}

// 16 bytes per lane from base + voff (a uniform 64-bit base in SGPRs and a
// 32-bit per-lane offset) into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// The same load, device-coherent (sc0 sc1): it reads data another kernel has
// just written through to memory, not a stale line of this XCD's L2.
__device__ __forceinline__ void dma16_coherent(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 sc0 sc1" ::"s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}

// all LDS reads of this wave done, then workgroup barrier (no fence: the
// DMA loads still in flight must not be waited for here)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// (K, N)-layout B tiles: chunk swizzle of a k-row and the transposing
// fragment read (ds_read_b64_tr_b16, two per 8-k fragment). Each half-wave
// of a transposing read takes 4 consecutive k-rows (k mod 4 = 0..3) by 4
// consecutive 16-byte chunks (chunk mod 4 = 0..3), and every row starts on
// the same bank (rows of 256 or 512 bytes): XOR-ing the chunk with
// (k mod 4) * 4 puts those 16 chunks on 16 distinct chunk positions mod 16,
// i.e. all 64 banks once. (With (k mod 8) * 2 two of them shared each
// position: the (K, N) GEMM at the FFN's first-GEMM shape counted 6x the
// bank-conflict cycles of the (N, K) one.)
__device__ __forceinline__ int kn_swz(int kr) { return (kr & 3) << 2; }

template <int BN>
__device__ __forceinline__ bf16x8_t load_kn_frag(const uint8_t* lb, int kr, int n) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  constexpr int PITCH = BN * 2;
  auto addr = [&](int k) {
    const int c = (n >> 3) ^ kn_swz(k);
    return (__attribute__((address_space(3))) v4i16*)(lb + k * PITCH + c * 16 + (n & 7) * 2);
  };
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(addr(kr));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(addr(kr + 4));
  bf16x8_t f;
  const v4i16 both[2] = {lo, hi};
  f = __builtin_bit_cast(bf16x8_t, both);
  return f;
}

// Scheduling pattern for one sub-step: NM MFMAs with the NR LDS reads of the
// next sub-step spread over the first half of them, so the reads have at
// least NM/2 MFMAs of time to land before they are needed (one
// sched_group_barrier per group, constant counts).
template <int I, int NM, int NR>
struct Interleave {
  __device__ __forceinline__ static void run() {
    if constexpr (I < NM) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      constexpr int H = NM / 2 > 0 ? NM / 2 : 1;
      constexpr int reads = I < H ? ((I + 1) * NR) / H - (I * NR) / H : 0;
      if constexpr (reads > 0) __builtin_amdgcn_sched_group_barrier(0x100, reads, 0);
      Interleave<I + 1, NM, NR>::run();
    }
  }
};

// The copy job of a launch that carries stage deliveries (GemmParams cp_*):
// workgroup b of the p.cp_blocks copy workgroups strides over the vectors of
// every slice.
constexpr int kCopyUnroll = 4;

__device__ __forceinline__ void copy_job(const GemmParams& p, int b) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int64_t total = int64_t(p.cp_n) * p.cp_nvec;
  const int64_t step = int64_t(p.cp_blocks) * blockDim.x;
  const bool gated = p.gate != nullptr || p.gate64 != nullptr;
  // kCopyUnroll vectors in flight per thread: their loads are all issued
  // before the first store
  for (int64_t i0 = int64_t(b) * blockDim.x + threadIdx.x; i0 < total; i0 += kCopyUnroll * step) {
    u32x4 x[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + u * step;
      if (i < total) {
        const int sl = static_cast<int>(i / p.cp_nvec);
        x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.cp_src[sl]) + (i - sl * p.cp_nvec));
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + u * step;
      if (i < total) {
        const int sl = static_cast<int>(i / p.cp_nvec);
        u32x4* dst = reinterpret_cast<u32x4*>(p.cp_dst + sl * p.cp_dst_stride) + (i - sl * p.cp_nvec);
        if (gated)   // read by this launch's gated tiles: system-scope store
          asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(dst), "v"(x[u]) : "memory");
        else
          *dst = x[u];
      }
    }
  }
  if (gated) {
    // every store of this workgroup has completed (and is visible at the
    // device coherence point) before it counts itself done
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      if (p.gate64 != nullptr) {
        // one add per workgroup: the host knows the count every earlier
        // call left and waits for it plus this launch's copy workgroups (a
        // compare-and-swap loop here cost a round trip per retry)
        __hip_atomic_fetch_add(p.gate64, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        __hip_atomic_fetch_add(p.gate, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// GATE: A rows come from slices (GemmParams a_slice_rows, a_local,
// a_slots), and the tiles of delivered slices wait on their chunk counters
// before each chunk's DMA (GemmParams gate; the staged all-gather as one
// launch). The loop is otherwise the same, so the results are the same bits.
template <typename Op, int BM, int BN, int WM, int WN, int ROWB, int STAGES, bool KN, bool SWIGLU, bool AT,
          bool GATE = false>
__global__ __launch_bounds__(64 * WM * WN, WM * WN / 4) void gemm_dma_kernel(const GemmParams p) {
  // workgroups past the tile workgroups carry the launch's copy job, if any
  // (ahead of them with a carried gate counter: dispatched first, the copy can
  // never wait behind tiles that wait for it)
  const int tile_grid = static_cast<int>(gridDim.x) - p.cp_blocks;
  const bool copy_first = GATE && p.gate64 != nullptr;
  const int wg = copy_first ? static_cast<int>(blockIdx.x) - p.cp_blocks : static_cast<int>(blockIdx.x);
  if (wg < 0 || wg >= tile_grid) {
    copy_job(p, copy_first ? static_cast<int>(blockIdx.x) : wg - tile_grid);
    return;
  }
  constexpr int NW = WM * WN;                  // waves: 4 (one per SIMD) or 8 (two per SIMD)
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE = A_BYTES + B_BYTES;
  constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                // rows per DMA instruction (1 KB)
  constexpr int A_INSTR = BM / (NW * RPI), B_INSTR = BN / (NW * RPI), INSTR = A_INSTR + B_INSTR;
  static_assert(A_INSTR * NW * RPI == BM && B_INSTR * NW * RPI == BN, "DMA instructions cover the tile");
  static_assert(!SWIGLU || (FN % 2 == 0), "swiglu pairs wave column blocks");
  constexpr int KSUB = ROWB / Op::kSliceBytes; // MFMA k slices per K-step
  constexpr int UNR = (KSUB % 2 == 0) ? 1 : 2; // K-steps per loop trip: fragment set stays static
  static_assert(KSUB >= 1 && STAGES >= 2 && (STAGES - 1) * INSTR <= 63, "pipeline shape");
  static_assert(!KN || (Op::kElemBytes == 2 && ROWB == 128), "(K, N) B tiles: bf16, 64 k-rows per K-step");
  // (K, N) layout: the B tile sits in LDS as [64 k-rows][BN n] exactly as in
  // memory; 16-byte chunks of a k-row are XOR-swizzled by (k-row mod 4) * 4 so
  // the transposing fragment reads of four consecutive k-rows hit distinct
  // banks (kn_swz)
  constexpr int CPRB = BN * 2 / 16;            // chunks per k-row
  constexpr int RPIB = 64 / CPRB;              // k-rows per DMA instruction
  // Contraction-major A (AT): the A tile sits in LDS as [64 k-rows][BM m],
  // swizzled and read like a (K, N) B tile; 64 k-rows of BM columns take as
  // many DMA instructions as BM rows of 128 bytes.
  static_assert(!AT || (KN && !SWIGLU && Op::kElemBytes == 2 && ROWB == 128 && BM >= 128),
                "contraction-major A: bf16 weight-gradient tiles");
  constexpr int CPRA = BM * 2 / 16;
  constexpr int RPIA = 64 / CPRA;
  static_assert(WM * 32 * ((SWIGLU ? BN / 2 : BN) + 4) * 4 <= STAGES * STAGE, "epilogue stage fits in LDS");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // uniform per wave: each DMA destination below is then scalar arithmetic
  // (s_add, s_mov m0) instead of a VALU add read back with v_readfirstlane
  // (measured 1-3% on the stage-GEMM shapes)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int ntm = (p.M + BM - 1) / BM;
  const int ntn = SWIGLU ? ((p.N >> 1) + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  const int ntiles = ntm * ntn;
  // the batch and first tile of this workgroup: blockIdx (y, x), or whole
  // batches per XCD (consecutive workgroups in dispatch order go to
  // consecutive XCDs)
  int64_t bz = blockIdx.y;
  int wgt = wg;
  if (p.batch_xcd) {
    const int64_t linear = int64_t(blockIdx.y) * gridDim.x + blockIdx.x;
    bz = (linear / (8 * int64_t(ntiles))) * 8 + linear % 8;
    wgt = static_cast<int>((linear / 8) % ntiles);
  }
  const BatchPtrs bp = batch_ptrs<Op::kElemBytes>(p, bz);

  const uint8_t* A = bp.a;
  const uint8_t* Bp = bp.b;
  const int64_t lda_b = p.lda * Op::kElemBytes;
  const int64_t ldb_b = p.ldb * Op::kElemBytes;
  const int64_t b_step = KN ? 64 * ldb_b : ROWB;   // B bytes per K-step
  const int nk = (p.K * Op::kElemBytes) / ROWB;
  const uint32_t lds0 =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)smem));

  // Persistent workgroups: each walks tiles vt = blockIdx.x + i * gridDim.x
  // (a grid of at most one workgroup per CU), so the next tile's loads are
  // issued right behind this tile's output stores instead of waiting for a
  // new workgroup to be dispatched once every wave of this one has retired.
  // With a grid that is a multiple of 8, all tiles of a workgroup come from
  // its own XCD's run of the tile order.
  const int rsub = lane / CPR, pc = lane % CPR;
  static_assert(!GATE || !AT, "gated launches have row-major A");
  auto run_tile = [&](int vt) {
  int tm, tn;
  if (p.batch_xcd) {            // row-major within the batch: an XCD's round is whole tile-rows
    tm = vt / ntn;
    tn = vt % ntn;
  } else {
    tile_of_block(vt, ntiles, ntm, p.tile_gm, tm, tn);
  }
  const int m0 = tm * BM;
  // gated launches: the slice holding this tile's rows, and the counters of
  // its delivery slot (nullptr: no waits)
  const unsigned* gate_row = nullptr;
  const unsigned long long* gate_word = nullptr;   // the carried copy's counter
  bool timed_out = false;
  const uint8_t* a_base = A;
  int64_t a_row0 = m0;
  if constexpr (GATE) {
    // slice sl: the local one in place, the others in their delivery slots
    // (all scalar arithmetic: no table in the arguments to index)
    const int sl = m0 / p.a_slice_rows;
    const int nsl = p.M / p.a_slice_rows;
    int slot = sl - p.gate_local - 1;
    if (slot < 0) slot += nsl;
    const bool local = sl == p.gate_local;
    a_base = local ? p.a_local : p.a_slots + int64_t(slot) * p.a_slice_rows * lda_b;
    a_row0 = m0 - int64_t(sl) * p.a_slice_rows;
    if (p.gate != nullptr && !p.gate_off && !local) gate_row = p.gate + slot * p.gate_nch;
    if (p.gate64 != nullptr && !p.gate_off && !local) gate_word = p.gate64;
    // the wait's state lives in VGPRs: the mainloop needs every SGPR
    asm volatile("" : "+v"(gate_row), "+v"(gate_word));
  }
  // a tile past the wrap of a run that goes on past the last slice writes
  // (and reads C of) rows wrap_back earlier, and with wrap_a reads A there too
  int tm_out = tm;
  if constexpr (!GATE && !AT) {
    if (p.wrap_row > 0 && m0 >= p.wrap_row) {
      tm_out = tm - p.wrap_back / BM;
      if (p.wrap_a) a_row0 = m0 - p.wrap_back;
    }
  }
  // This lane's source chunk in each DMA instruction, as a 32-bit offset
  // from a uniform base (the tile's first A row; B itself), which the host
  // keeps below 2^31. Rows past the edge read a valid row instead (their
  // products only reach outputs never stored).
  const uint8_t* a_tile = a_base + a_row0 * lda_b;
  uint32_t aoff[A_INSTR];
  uint32_t boff[B_INSTR];
#pragma unroll
  for (int j = 0; j < A_INSTR; ++j) {
    if constexpr (!AT) {
      const int r = (j * NW + wave) * RPI + rsub;
      const int grow = min(m0 + r, p.M - 1);
      aoff[j] = static_cast<uint32_t>(int64_t(grow - m0) * lda_b + swz<ROWB>(r, pc) * 16);
    } else {
      const int kr = (j * NW + wave) * RPIA + lane / CPRA;
      const int c = (lane % CPRA) ^ kn_swz(kr);
      int mc = m0 + c * 8;
      if (mc >= p.M) mc = 0;
      aoff[j] = static_cast<uint32_t>(int64_t(kr) * lda_b + mc * 2);
    }
  }
#pragma unroll
  for (int j = 0; j < B_INSTR; ++j) {
    if constexpr (!KN) {
      const int r = (j * NW + wave) * RPI + rsub;
      int n = b_col<SWIGLU, BN>(tn, r, p.N);
      if (n < 0) n = 0;
      boff[j] = static_cast<uint32_t>(int64_t(n) * ldb_b + swz<ROWB>(r, pc) * 16);
    } else {
      const int kr = (j * NW + wave) * RPIB + lane / CPRB;
      const int c = (lane % CPRB) ^ kn_swz(kr);
      int n = b_col<SWIGLU, BN>(tn, c * 8, p.N);
      if (n < 0) n = 0;
      boff[j] = static_cast<uint32_t>(int64_t(kr) * ldb_b + n * 2);
    }
  }

  auto issue = [&](int kt, int buf) {
    const uint32_t sb = lds0 + buf * STAGE;
    const uint8_t* ab;
    if constexpr (AT) {
      int64_t k0 = int64_t(kt) * 64;
      if (p.a_kwrap > 0 && k0 >= p.a_kwrap) k0 -= p.kwrap_rows;
      ab = A + k0 * lda_b;
    } else {
      ab = a_tile + int64_t(kt) * ROWB;
    }
    const uint8_t* bb;
    if constexpr (KN) {
      int64_t k0 = int64_t(kt) * 64;
      if (p.b_kwrap > 0 && k0 >= p.b_kwrap) k0 -= p.kwrap_rows;
      bb = Bp + k0 * ldb_b;
    } else {
      bb = Bp + int64_t(kt) * b_step;
    }
    if constexpr (GATE) {
      if (gate_row != nullptr || gate_word != nullptr) {
        // a K-step that starts a chunk waits for that chunk to have landed
        // (bounded: past the deadline the wait gives up and the tile's
        // output becomes NaN)
        if (kt % p.gate_ksteps == 0) {
          unsigned deadline = p.gate_deadline != 0u ? p.gate_deadline : kGateDeadline;
          const unsigned t0 = static_cast<unsigned>(__builtin_amdgcn_s_memrealtime());
          if (gate_word != nullptr) {
            // the whole copy: the counter's total once every copy workgroup has added to it
            unsigned long long want = p.gate_want64;
            asm volatile("" : "+v"(want), "+v"(deadline));
            while (!timed_out && __hip_atomic_load(gate_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want) {
              if (static_cast<unsigned>(__builtin_amdgcn_s_memrealtime()) - t0 > deadline) timed_out = true;
              __builtin_amdgcn_s_sleep(2);
            }
          } else {
            const unsigned* g = gate_row + kt / p.gate_ksteps;
            unsigned need = p.gate_need;
            asm volatile("" : "+v"(g), "+v"(need), "+v"(deadline));
            while (!timed_out && __hip_atomic_load(g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
              if (static_cast<unsigned>(__builtin_amdgcn_s_memrealtime()) - t0 > deadline) timed_out = true;
              __builtin_amdgcn_s_sleep(2);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < A_INSTR; ++j)
          dma16_coherent(ab, aoff[j], __builtin_amdgcn_readfirstlane(sb + (j * NW + wave) * 1024));
      } else {
#pragma unroll
        for (int j = 0; j < A_INSTR; ++j)
          dma16(ab, aoff[j], __builtin_amdgcn_readfirstlane(sb + (j * NW + wave) * 1024));
      }
    } else {
#pragma unroll
    for (int j = 0; j < A_INSTR; ++j)
      dma16(ab, aoff[j], __builtin_amdgcn_readfirstlane(sb + (j * NW + wave) * 1024));
    }
#pragma unroll
    for (int j = 0; j < B_INSTR; ++j)
      dma16(bb, boff[j], __builtin_amdgcn_readfirstlane(sb + A_BYTES + (j * NW + wave) * 1024));
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto b_row = [&](int j) {
    if constexpr (!SWIGLU) {
      return wn * WTN + j * 32 + l32;
    } else {
      const int hj = j % (FN / 2), part = j / (FN / 2);
      return part * (BN / 2) + wn * (WTN / 2) + hj * 32 + l32;
    }
  };

  // Software pipeline. Fragments are double-buffered: the LDS reads of
  // sub-step g+1 are issued before the MFMAs of sub-step g. Before the last
  // sub-step of K-step kt the wave waits for its DMA of K-step kt+1, joins the
  // barrier (after which every wave has finished reading K-step kt's buffer)
  // and refills that buffer with K-step kt+STAGES.
  typename Op::frag_t fa[2][FM], fb[2][FN];
  auto load_frags = [&](int set, const uint8_t* la, int kk) {
    const uint8_t* lb = la + A_BYTES;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (!AT) {
        fa[set][i] = Op::template load<ROWB>(la, wm * WTM + i * 32 + l32, kk, half);
      } else {
        // the transposing read of the (K, N) B tile, over A's m columns
        const int g = lane >> 4, lq = lane & 15;
        const int kr = kk * 16 + 8 * (g >> 1) + (lq >> 2);
        fa[set][i] = load_kn_frag<BM>(la, kr, wm * WTM + i * 32 + 16 * (g & 1) + 4 * (lq & 3));
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (!KN) {
        fb[set][j] = Op::template load<ROWB>(lb, b_row(j), kk, half);
      } else {
        // lane l of 16-lane group g: k-rows kk*16 + 8*(g>>1) + (l'>>2) (+4),
        // columns col0(j) + 16*(g&1) + 4*(l'&3); the hardware transposes each
        // 16-lane group so lane l ends with 8 consecutive k of column col0 + l%32
        const int g = lane >> 4, lq = lane & 15;
        const int kr = kk * 16 + 8 * (g >> 1) + (lq >> 2);
        const int n = b_row(j) - l32 + 16 * (g & 1) + 4 * (lq & 3);
        fb[set][j] = load_kn_frag<BN>(lb, kr, n);
      }
    }
  };
  auto mma_all = [&](int set) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = Op::mma(fb[set][j], fa[set][i], acc[i][j]);
  };
  // interleave the MFMAs of one sub-step with the LDS reads of the next in
  // proportion, so no MFMA waits behind a long queue of younger reads
  constexpr int NMFMA = FM * FN;
  constexpr int NREAD = (FM + FN) * Op::kReadsPerFrag;

  // The loop body has no branches, so the scheduler sees each sub-step as one
  // region: every K-step issues exactly one DMA group (past the end of K it
  // re-reads the last K-step, an L2 hit, into a buffer nobody reads again),
  // which also makes every vmcnt wait a constant. nk >= 1 and nk % UNR == 0
  // (host-checked).
#pragma unroll
  for (int st = 0; st < STAGES; ++st) issue(min(st, nk - 1), st);
  wait_vmcnt<(STAGES - 1) * INSTR>();
  lds_barrier();
  load_frags(0, smem, 0);
  for (int kt = 0; kt < nk; kt += UNR) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int ks = kt + u;
      const uint8_t* la = smem + (ks % STAGES) * STAGE;
#pragma unroll
      for (int kk = 0; kk < KSUB; ++kk) {
        const int cur = (u * KSUB + kk) & 1;
        if (kk + 1 < KSUB) {
          load_frags(cur ^ 1, la, kk + 1);
        } else {
          wait_vmcnt<(STAGES - 2) * INSTR>();
          lds_barrier();
          issue(min(ks + STAGES, nk - 1), ks % STAGES);
          load_frags(cur ^ 1, smem + ((ks + 1) % STAGES) * STAGE, 0);
        }
        mma_all(cur);
        Interleave<0, NMFMA, NREAD>::run();
      }
    }
  }
  wait_vmcnt<0>();
  bool nan_out = false;
  if constexpr (GATE) {
    // a workgroup any of whose waves gave up waiting leaves NaN, never a
    // silent wrong value
    nan_out = __syncthreads_or(timed_out);
  } else {
    __syncthreads();
  }
  if constexpr (GATE) {
    if (nan_out) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_nanf("");
    }
  }
  int tn_out = tn;
  if constexpr (!GATE && !AT && !SWIGLU) {
    if (p.wrap_col > 0 && tn * BN >= p.wrap_col) tn_out = tn - p.wrap_back_col / BN;
  }
  store_tile<BM, BN, WM, WN, SWIGLU, AT>(p, bp, acc, smem, tm_out, tn_out);   // ends with a barrier: LDS free
  };
  if constexpr (persistent_tiles<Op, BM, BN, AT>()) {
    // (batched launches have one workgroup per tile: one trip, at wgt)
    for (int vt = wgt; vt < ntiles; vt += tile_grid) run_tile(vt);
  } else {
    run_tile(wgt);
  }
}

int cu_count();

// Group height for tile_of_block when a launch is one round of tiles (every
// tile has a workgroup at once, the tiles split evenly over the 8 XCDs): the
// height, among those that make each XCD's run of tiles one whole rectangle,
// with the fewest A rows plus B columns per XCD, i.e. the least L2 fill for
// the tiles that run together. 0 (the kernel's power-of-two rule) otherwise,
// or when no height gives whole rectangles. For 224 tiles of 128 x 256 over
// 56 x 4 (the 7168-row stage run of 1024 columns) the power-of-two rule
// groups 4 tile-rows, so most XCD runs straddle three groups and read 12 A
// tile-rows; 7 gives each XCD 7 tile-rows by all 4 columns.
int group_rows(int ntm, int ntn, int bm, int bn, int grid) {
  const int64_t nt = int64_t(ntm) * ntn;
  if (nt % 8 != 0 || nt > grid || nt > cu_count()) return 0;
  const int64_t run = nt / 8;
  int best = 0;
  int64_t best_cost = 0;
  for (int gm = 1; gm <= std::min(ntm, 64); ++gm) {
    if (ntm % gm != 0) continue;
    const int64_t group = int64_t(gm) * ntn;
    int64_t rows, cols;
    if (run % group == 0) {                          // each XCD: whole groups
      rows = run / ntn;
      cols = ntn;
    } else if (group % run == 0 && run % gm == 0) {  // each XCD: whole columns of one group
      rows = gm;
      cols = run / gm;
    } else {
      continue;
    }
    const int64_t cost = rows * bm + cols * bn;
    if (best == 0 || cost < best_cost) {
      best = gm;
      best_cost = cost;
    }
  }
  return best;
}

template <typename Op, int BM, int BN, int WM, int WN, int ROWB, int STAGES, bool KN, bool SWIGLU, bool AT = false,
          bool GATE = false>
hipError_t launch_dma_tile(const GemmParams& p_in, hipStream_t s) {
  constexpr int smem = STAGES * (BM + BN) * ROWB;
  constexpr int nt = 64 * WM * WN;
  auto kern = gemm_dma_kernel<Op, BM, BN, WM, WN, ROWB, STAGES, KN, SWIGLU, AT, GATE>;
  static uint64_t lds_set = 0;
  if (hipError_t e = lds_limit_once(reinterpret_cast<const void*>(kern), smem, lds_set); e != hipSuccess) return e;
  GemmParams p = p_in;
  const int nout_tiles = SWIGLU ? ((p.N / 2) + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  const int tiles = ((p.M + BM - 1) / BM) * nout_tiles;
  if (tiles == 0 || p.batch < 1) return hipSuccess;
  // at most one persistent workgroup per CU (all tiles when batched). The
  // CU budget shaped the tiles only: once launches beside this one finish,
  // their CUs are this launch's to use.
  int grid = (p.batch == 1 && persistent_tiles<Op, BM, BN, AT>()) ? std::min(tiles, cu_count()) : tiles;
  if (p.grid_cap >= 8 && p.batch == 1 && persistent_tiles<Op, BM, BN, AT>()) grid = std::min(grid, p.grid_cap & ~7);
  if (p.cp_blocks > 0 && p.batch != 1) return hipErrorInvalidValue;   // a copy job needs a single batch
  p.tile_gm = p.batch == 1 ? group_rows((p.M + BM - 1) / BM, nout_tiles, BM, BN, grid) : 0;
  p.batch_xcd = (p.batch > 1 && p.batch % 8 == 0 && p.cp_blocks == 0) ? 1 : 0;
  hipLaunchKernelGGL(kern, dim3(grid + p.cp_blocks, p.batch), dim3(nt), smem, s, p);
  return hipGetLastError();
}

template <typename Op, int BM, int BN, bool KN, bool SWIGLU>
hipError_t launch_tile(const GemmParams& p, hipStream_t s) {
  constexpr int smem = 2 * (BM + BN) * kRowBytes;
  auto kern = gemm_kernel<Op, BM, BN, KN, SWIGLU>;
  static uint64_t lds_set = 0;
  if (hipError_t e = lds_limit_once(reinterpret_cast<const void*>(kern), smem, lds_set); e != hipSuccess) return e;
  const int nout_tiles = SWIGLU ? ((p.N / 2) + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  const int grid = ((p.M + BM - 1) / BM) * nout_tiles;
  if (grid == 0 || p.batch < 1) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid, p.batch), dim3(kThreads), smem, s, p);
  return hipGetLastError();
}

// Number of compute units of the current device (cached per device; read
// also by calls that do not take the library's lock).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Tile choice by a small cost model: waves of workgroups over the CUs times
// the tile's work divided by its relative MFMA efficiency (measured on
// MI355X with 8-wave workgroups: a 128x256 tile runs at ~0.86 and a 128x128
// tile at ~0.73 of the 256x256 tile's per-CU rate). The v1 fallback uses the
// same index for 256x256, 256x128 and 128x128.
int pick_tile(int M, int N, int epi, int batch, int budget, double* cost_out = nullptr) {
  const int n = epi == kEpiSwiglu ? N / 2 : N;
  const int bn_div = epi == kEpiSwiglu ? 2 : 1;
  const int cus = budget > 0 ? std::min(budget, cu_count()) : cu_count();
  const int bm[3] = {256, 128, 128}, bn[3] = {256, 256, 128};
  // relative efficiency per tile shape, measured (the (K, N) second GEMM of
  // the per-slot FFN: 256 x 256 over 2.5 waves beats 128 x 256 over 5)
  const double eff[3] = {1.0, 0.75, 0.6};
  int best = 0;
  double best_cost = 0.0;
  for (int t = 0; t < 3; ++t) {
    const long tiles = long(batch) * ((M + bm[t] - 1) / bm[t]) * ((n + bn[t] / bn_div - 1) / (bn[t] / bn_div));
    const long waves = (tiles + cus - 1) / cus;
    const double cost = double(waves) * bm[t] * bn[t] / eff[t];
    if (t == 0 || cost < best_cost) {
      best = t;
      best_cost = cost;
    }
  }
  if (cost_out) *cost_out = best_cost;
  return best;
}

// Output columns [0, n1) of a launch that should run apart from the rest,
// or 0. A launch whose tiles end in a partial round (the per-slot FFN's
// batched second GEMM: 8 x 4096 x 1280, 640 tiles of 256 x 256 on 256 CUs,
// 2.5 rounds) runs as two launches in stream order: a column block that
// makes whole rounds of 256 x 256 tiles, then the other columns with the
// tile the cost model picks for them (there one round of 128 x 256). Taken
// when the cost model saves at least 5%; measured on MI355X at that shape
// (bf16, (K, N) weights, K = 7680): 604 us as one launch, 570 us split into
// 1024 + 256 columns. Plain launches on the whole chip only: no copy job,
// gates, addends, column segments or SwiGLU pairing.
int round_split_cols(const GemmParams& p, int epi) {
  if (epi != kEpiAlphaBeta || p.cu_budget != 0 || p.grid_cap != 0 || p.cp_blocks != 0 || p.a_slice_rows != 0 ||
      p.n_seg != 0 || p.n_add_list != 0 || p.n_add_strided != 0 || p.acc_in || p.acc_out || p.wrap_col != 0 ||
      p.M <= 0 ||
      p.N <= 256 || p.batch < 1)
    return 0;
  double whole = 0.0;
  pick_tile(p.M, p.N, epi, p.batch, 0, &whole);
  const int64_t per_col = int64_t(p.batch) * ((p.M + 255) / 256);    // 256 x 256 tiles per 256 columns
  const int cus = cu_count();
  int best_n1 = 0;
  double best = whole * 0.95;
  for (int c = 1; 256 * c < p.N; ++c) {
    if ((per_col * c) % cus != 0) continue;
    double rest = 0.0;
    pick_tile(p.M, p.N - 256 * c, epi, p.batch, 0, &rest);
    const double cost = double(per_col * c / cus) * 256 * 256 + rest;
    if (cost < best) {
      best = cost;
      best_n1 = 256 * c;
    }
  }
  return best_n1;
}

// Whether a launch runs on the direct-to-LDS kernel: 128-byte K-steps, and a
// tile's A rows and all of B addressable with 31-bit offsets.
bool dma_path(const GemmParams& p, int64_t eb, bool kn) {
  const bool offsets_fit = int64_t(256) * p.lda * eb < (int64_t(1) << 31) &&
                           (kn ? int64_t(64) * p.ldb * eb + int64_t(p.N) * 2
                               : int64_t(p.N) * p.ldb * eb) < (int64_t(1) << 31);
  return p.M > 0 && p.N > 0 && p.K > 0 && (p.K * eb) % 128 == 0 && offsets_fit;
}

template <typename Op, bool KN, bool SW>
hipError_t dispatch_tile(const GemmParams& p, hipStream_t s) {
  // direct-to-LDS mainloop: 128-byte K-steps (measured faster on gfx950 than
  // 64-byte K-steps with twice the ring depth: half the barriers per byte)
  const bool dma = dma_path(p, Op::kElemBytes, KN);
  const int epi = SW ? kEpiSwiglu : kEpiAlphaBeta;
  if (p.a_slice_rows > 0) {
    // the staged all-gather as one launch (gated): 128 x 256 tiles, whose
    // registers leave each SIMD room for a wave of the copy kernel, or
    // 128 x 128 for a small call
    if (!dma || p.batch != 1 || p.a_slice_rows % 128 != 0 || p.M % p.a_slice_rows != 0 ||
        p.M / p.a_slice_rows > kMaxGateSlices || p.gate_local < -1 ||
        p.gate_local >= p.M / p.a_slice_rows || !p.a_slots || (p.gate_local >= 0 && !p.a_local))
      return hipErrorInvalidValue;
    if (!gated_small_tile(p.M, p.N, Op::kElemBytes == 1 ? kE4m3 : kBf16, epi, p.cp_blocks))
      return launch_dma_tile<Op, 128, 256, 2, 4, 128, 3, KN, SW, false, true>(p, s);
    if constexpr (SW) return launch_dma_tile<Op, 128, 128, 4, 2, 128, 4, KN, SW, false, true>(p, s);
    else if constexpr (Op::kElemBytes == 2) return launch_dma_tile<Op, 128, 128, 2, 4, 128, 4, KN, SW, false, true>(p, s);
    else return hipErrorInvalidValue;   // not reached: gated_small_tile is false for it
  }
  if (dma) {
    switch (pick_tile(p.M, p.N, epi, p.batch, p.cu_budget)) {
      case 0: return launch_dma_tile<Op, 256, 256, 2, 4, 128, 2, KN, SW>(p, s);
      case 1: return launch_dma_tile<Op, 128, 256, 2, 4, 128, 3, KN, SW>(p, s);
      default:   // the SwiGLU epilogue pairs two column blocks per wave
        if constexpr (SW) return launch_dma_tile<Op, 128, 128, 4, 2, 128, 4, KN, SW>(p, s);
        else return launch_dma_tile<Op, 128, 128, 2, 4, 128, 4, KN, SW>(p, s);
    }
  }
  switch (pick_tile(p.M, p.N, epi, p.batch, p.cu_budget)) {
    case 0: return launch_tile<Op, 256, 256, KN, SW>(p, s);
    case 1: return launch_tile<Op, 256, 128, KN, SW>(p, s);
    default: return launch_tile<Op, 128, 128, KN, SW>(p, s);
  }
}

// Contraction-major A (the weight gradient): bf16, B in (K, N), the DMA
// kernel only. The same cost model picks the tile.
bool at_offsets_fit(const GemmParams& p) {
  return int64_t(64) * p.lda * 2 + int64_t(p.M) * 2 < (int64_t(1) << 31) &&
         int64_t(64) * p.ldb * 2 + int64_t(p.N) * 2 < (int64_t(1) << 31);
}

hipError_t dispatch_at(const GemmParams& p, hipStream_t s) {
  switch (pick_tile(p.M, p.N, kEpiAlphaBeta, p.batch, p.cu_budget)) {
    case 0: return launch_dma_tile<OpBf16, 256, 256, 2, 4, 128, 2, true, false, true>(p, s);
    case 1: return launch_dma_tile<OpBf16, 128, 256, 2, 4, 128, 3, true, false, true>(p, s);
    default: return launch_dma_tile<OpBf16, 128, 128, 2, 4, 128, 4, true, false, true>(p, s);
  }
}

// Register-only MFMA loop: the matrix cores' attainable rate at the clocks
// the chip holds under this load, with no memory traffic. Each wave keeps
// four independent accumulators in flight, so the MFMA pipe never waits on
// a result. Lane 0 of every wave records its shader-clock and wall-clock
// ticks over the loop (the wall clock runs at a fixed rate), from which the
// host derives the engine clock.
template <typename Op>
__global__ void __launch_bounds__(kProbeThreads) mfma_probe_kernel(unsigned long long* sink, int iters) {
  typedef typename Op::frag_t frag_t;
  struct Words { unsigned v[sizeof(frag_t) / 4]; };
  const int lane = threadIdx.x & 63;
  Words wx, wy;
  for (int i = 0; i < int(sizeof(frag_t) / 4); ++i) {
    // small nonzero operands (bf16 pairs near 2^-7, e4m3 bytes 0.5 .. 0.875)
    const unsigned w = Op::kElemBytes == 2 ? 0x3C003C00u + (lane & 15) * 0x00010001u
                                           : 0x30303030u + (lane & 7) * 0x01010101u;
    wx.v[i] = w;
    wy.v[i] = w ^ 0x00010001u;
  }
  const frag_t x = __builtin_bit_cast(frag_t, wx), y = __builtin_bit_cast(frag_t, wy);
  f32x16_t a0 = {}, a1 = {}, a2 = {}, a3 = {};
  const unsigned long long c0 = clock64(), r0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
    a0 = Op::mma(x, y, a0);
    a1 = Op::mma(y, x, a1);
    a2 = Op::mma(x, x, a2);
    a3 = Op::mma(y, y, a3);
  }
  const unsigned long long c1 = clock64(), r1 = wall_clock64();
  float acc = 0.0f;
  for (int e = 0; e < 16; ++e) acc += a0[e] + a1[e] + a2[e] + a3[e];
  const int wave = blockIdx.x * (kProbeThreads / 64) + threadIdx.x / 64;
  if (lane == 0) {
    sink[2 * wave] = c1 - c0;
    sink[2 * wave + 1] = r1 - r0;
  }
  if (acc == -1.0f) sink[2 * wave] = 0;   // keeps every accumulator live
}

}  // namespace

int device_cus() { return cu_count(); }

bool gemm_at_supported(const GemmParams& p) {
  return p.M > 0 && p.N > 0 && p.K > 0 && p.K % 64 == 0 && p.M % 8 == 0 && p.N % 8 == 0 && p.lda % 8 == 0 &&
         p.ldb % 8 == 0 && p.batch == 1 && at_offsets_fit(p);
}

hipError_t launch_gemm_at(const GemmParams& p, hipStream_t s) {
  if (!gemm_at_supported(p)) return hipErrorInvalidValue;
  return dispatch_at(p, s);
}

double probe_flop_per_iter(int dtype) {
  return double(kProbeThreads / 64) * 4 * (dtype == kE4m3 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16);
}

hipError_t launch_mfma_probe(int dtype, int iters, int blocks, unsigned long long* sink, hipStream_t s) {
  if (dtype == kE4m3)
    hipLaunchKernelGGL(mfma_probe_kernel<OpE4m3>, dim3(blocks), dim3(kProbeThreads), 0, s, sink, iters);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<OpBf16>, dim3(blocks), dim3(kProbeThreads), 0, s, sink, iters);
  return hipGetLastError();
}

// Tile of a gated launch: 128 x 256, or 128 x 128 when twice as many tiles
// still fit on the chip beside the copy workgroups the launch carries
// (copy_wgs; 0 with the copy on a stream of its own): twice the CUs, half
// the time per tile. The e4m3 alpha/beta 128 x 128 form is left out: with
// the gate's registers it needs a stack frame.
bool gated_small_tile(int M, int N, int dtype, int epi, int copy_wgs) {
  if (dtype == kE4m3 && epi != kEpiSwiglu) return false;
  const int ncols = epi == kEpiSwiglu ? (N / 2 + 127) / 128 : (N + 255) / 256;
  return int64_t((M + 127) / 128) * ncols * 2 + copy_wgs <= cu_count();
}

int gated_tiles(int M, int N, int dtype, int epi, int copy_wgs) {
  const bool small = gated_small_tile(M, N, dtype, epi, copy_wgs);
  const int bn = small ? 128 : 256;
  const int ncols = epi == kEpiSwiglu ? (N / 2 + bn / 2 - 1) / (bn / 2) : (N + bn - 1) / bn;
  return ((M + 127) / 128) * ncols;
}

int gemm_tiles(int M, int N, int dtype, int epi, int batch, int cu_budget) {
  const int t = pick_tile(M, N, epi, batch, cu_budget);
  const int bm = t == 0 ? 256 : 128, bn = t == 2 ? 128 : 256;
  const int n = epi == kEpiSwiglu ? N / 2 : N, bno = epi == kEpiSwiglu ? bn / 2 : bn;
  (void)dtype;
  return batch * ((M + bm - 1) / bm) * ((n + bno - 1) / bno);
}

hipError_t launch_gemm(const GemmParams& p, int dtype, int layout, int epi, hipStream_t s) {
  const bool kn = layout == kKN, sw = epi == kEpiSwiglu;
  const int64_t eb = dtype == kE4m3 ? 1 : 2;
  if (p.wrap_row > 0) {
    if (p.wrap_row >= p.M || p.wrap_row % 256 != 0 || p.wrap_back % 256 != 0 || p.wrap_back < p.wrap_row ||
        p.M % 256 != 0 || p.batch != 1 || p.a_slice_rows != 0 || p.add_row1 > p.add_row0)
      return hipErrorInvalidValue;
    if (!dma_path(p, eb, kn)) {
      // the register-staged kernel takes no wrap: the two stretches as two launches
      GemmParams head = p, tail = p;
      head.wrap_row = tail.wrap_row = 0;
      head.M = p.wrap_row;
      tail.M = p.M - p.wrap_row;
      const int64_t back = int64_t(p.wrap_row) - p.wrap_back;       // the tail's first output row, from d
      tail.a = static_cast<const char*>(p.a) + (p.wrap_a ? back : int64_t(p.wrap_row)) * p.lda * eb;
      tail.d = p.d + back * p.ldd;
      if (p.c) tail.c = p.c + back * p.ldc;
      if (hipError_t e = launch_gemm(head, dtype, layout, epi, s); e != hipSuccess) return e;
      return launch_gemm(tail, dtype, layout, epi, s);
    }
  }
  if (p.wrap_col > 0) {
    if (p.wrap_col >= p.N || p.wrap_col % 256 != 0 || p.wrap_back_col % 256 != 0 ||
        p.wrap_back_col < p.wrap_col || p.N % 256 != 0 || p.batch != 1 || p.a_slice_rows != 0 ||
        p.wrap_row != 0 || sw || p.n_add_list + p.n_add_strided != 0 || p.n_seg != 0)
      return hipErrorInvalidValue;
    if (!dma_path(p, eb, kn)) {
      // the register-staged kernel takes no wrap: the two stretches as two launches
      GemmParams head = p, tail = p;
      head.wrap_col = tail.wrap_col = 0;
      head.N = p.wrap_col;
      tail.N = p.N - p.wrap_col;
      const int64_t back = int64_t(p.wrap_col) - p.wrap_back_col;   // the tail's first output column, from d
      tail.b = static_cast<const char*>(p.b) + (kn ? int64_t(p.wrap_col) * eb : int64_t(p.wrap_col) * p.ldb * eb);
      tail.d = p.d + back;
      if (p.c) tail.c = p.c + back;
      if (p.bias) tail.bias = p.bias + back;
      if (hipError_t e = launch_gemm(head, dtype, layout, epi, s); e != hipSuccess) return e;
      return launch_gemm(tail, dtype, layout, epi, s);
    }
  }
  if (const int n1 = round_split_cols(p, epi); n1 > 0 && dma_path(p, eb, kn)) {
    GemmParams left = p, right = p;
    left.N = n1;
    right.N = p.N - n1;
    right.b = static_cast<const char*>(p.b) + (kn ? int64_t(n1) * eb : int64_t(n1) * p.ldb * eb);
    if (p.c) right.c = p.c + n1;
    right.d = p.d + n1;
    if (p.bias) right.bias = p.bias + n1;
    if (hipError_t e = launch_gemm(left, dtype, layout, epi, s); e != hipSuccess) return e;
    return launch_gemm(right, dtype, layout, epi, s);
  }
  if (dtype == kBf16) {
    if (kn) return sw ? dispatch_tile<OpBf16, true, true>(p, s) : dispatch_tile<OpBf16, true, false>(p, s);
    return sw ? dispatch_tile<OpBf16, false, true>(p, s) : dispatch_tile<OpBf16, false, false>(p, s);
  }
  if (kn) return hipErrorInvalidValue;     // fp8 is NK only (validated on the host)
  return sw ? dispatch_tile<OpE4m3, false, true>(p, s) : dispatch_tile<OpE4m3, false, false>(p, s);
}

bool wrap_in_one_launch(const GemmParams& p, int dtype, int layout) {
  return dma_path(p, dtype == kE4m3 ? 1 : 2, layout == kKN);
}

hipError_t launch_gemm_carrying_copy(const GemmParams& p, int dtype, int layout, int epi, hipStream_t s) {
  if (p.cp_blocks <= 0) return launch_gemm(p, dtype, layout, epi, s);
  if (p.cp_n < 1 || p.cp_n > kMaxCopySlices || p.batch != 1) return hipErrorInvalidValue;
  if (dma_path(p, dtype == kE4m3 ? 1 : 2, layout == kKN)) return launch_gemm(p, dtype, layout, epi, s);
  // the register-staged kernel takes no copy job: the copy goes first
  GemmParams q = p;
  q.cp_blocks = 0;
  const void* src[kMaxCopySlices];
  for (int i = 0; i < p.cp_n; ++i) src[i] = p.cp_src[i];
  hipError_t e = launch_deliver(src, p.cp_n, size_t(p.cp_nvec) * 16, p.cp_dst, size_t(p.cp_dst_stride), s);
  if (e != hipSuccess) return e;
  return launch_gemm(q, dtype, layout, epi, s);
}

}  // namespace tpg
