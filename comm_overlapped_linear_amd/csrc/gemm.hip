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
#include "gemm.h"

namespace tpg {

namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;   // K bytes per tile row per K-step

// 16-byte chunk swizzle inside a 128-byte LDS row.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

struct OpBf16 {
  static constexpr int kElemBytes = 2;
  static constexpr int kSubSteps = 4;   // 32-byte k slices per K-step
  typedef bf16x8_t frag_t;
  __device__ static frag_t load(const uint8_t* lds, int row, int kk, int half) {
    const int c = kk * 2 + half;
    uint4 v = *reinterpret_cast<const uint4*>(lds + row * kRowBytes + swz(row, c) * 16);
    return __builtin_bit_cast(frag_t, v);
  }
  __device__ static f32x16_t mma(frag_t x, frag_t y, f32x16_t acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc, 0, 0, 0);
  }
};

struct OpE4m3 {
  static constexpr int kElemBytes = 1;
  static constexpr int kSubSteps = 2;   // 64-byte k slices per K-step
  typedef i32x8_t frag_t;
  __device__ static frag_t load(const uint8_t* lds, int row, int kk, int half) {
    const int c = kk * 4 + half * 2;
    uint4 lo = *reinterpret_cast<const uint4*>(lds + row * kRowBytes + swz(row, c) * 16);
    uint4 hi = *reinterpret_cast<const uint4*>(lds + row * kRowBytes + swz(row, c + 1) * 16);
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

template <typename Op, int BM, int BN, bool KN, bool SWIGLU>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const GemmParams p) {
  constexpr int WM = 2, WN = 2;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  constexpr int A_LD = BM * 8 / kThreads;            // 16-byte chunks per thread
  constexpr int B_LD_NK = BN * 8 / kThreads;
  constexpr int B_BLK_KN = (BN / 8) * 8;             // 8x8 blocks per K-step (kn, bf16)
  constexpr int B_LD_KN = (B_BLK_KN + kThreads - 1) / kThreads;
  static_assert(!SWIGLU || (FN % 2 == 0), "swiglu pairs wave column blocks");

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

  const uint8_t* A = static_cast<const uint8_t*>(p.a);
  const uint8_t* Bp = static_cast<const uint8_t*>(p.b);
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
      *reinterpret_cast<uint4*>(la + r * kRowBytes + swz(r, c) * 16) = ra[i];
    }
    if (!KN) {
#pragma unroll
      for (int i = 0; i < B_LD_NK; ++i) {
        const int id = i * kThreads + tid;
        const int r = id >> 3, c = id & 7;
        *reinterpret_cast<uint4*>(lb + r * kRowBytes + swz(r, c) * 16) = rb[i];
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
            *reinterpret_cast<uint4*>(lb + r * kRowBytes + swz(r, kb8) * 16) =
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
    if (!SWIGLU) return wn * WTN + j * 32 + l32;
    const int hj = j % (FN / 2), part = j / (FN / 2);
    return part * (BN / 2) + wn * (WTN / 2) + hj * 32 + l32;
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

  // ---- epilogue: lane holds rows m0 + wm*WTM + i*32 + l32, 4 consecutive columns per reg group
  const int nout = SWIGLU ? (p.N >> 1) : p.N;
  constexpr int JN = SWIGLU ? FN / 2 : FN;
  const int ncol0 = SWIGLU ? tn * (BN / 2) + wn * (WTN / 2) : tn * BN + wn * WTN;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = m0 + wm * WTM + i * 32 + l32;
    if (row >= p.M) continue;
    const bool do_add = row >= p.add_row0 && row < p.add_row1;
#pragma unroll
    for (int j = 0; j < JN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = ncol0 + j * 32 + g * 8 + half * 4;
        if (col >= nout) continue;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x = p.alpha * acc[i][j][g * 4 + q];
          if (SWIGLU) {
            const float y = p.alpha * acc[i][j + JN][g * 4 + q];
            v[q] = silu_f32(x) * y;
          } else {
            v[q] = x;
          }
        }
        const bool full = p.vec_ok && (col + 3 < nout);
        auto add_src = [&](const uint16_t* src, int64_t ld, float scale) {
          if (full) {
            const uint2 cv = *reinterpret_cast<const uint2*>(src + row * ld + col);
            v[0] += scale * bf16_to_f32(cv.x & 0xffff);
            v[1] += scale * bf16_to_f32(cv.x >> 16);
            v[2] += scale * bf16_to_f32(cv.y & 0xffff);
            v[3] += scale * bf16_to_f32(cv.y >> 16);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (col + q < nout) v[q] += scale * bf16_to_f32(src[row * ld + col + q]);
          }
        };
        if (p.beta != 0.0f) add_src(p.c, p.ldc, p.beta);
        if (p.bias) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (col + q < nout) v[q] += bf16_to_f32(p.bias[col + q]);
        }
        if (do_add) {   // addends are (add_row1 - add_row0) x nout blocks
          const int64_t shift = static_cast<int64_t>(p.add_row0) * p.ld_add;
          for (int t = 0; t < p.n_add_list; ++t) add_src(p.add_list[t] - shift, p.ld_add, 1.0f);
          for (int t = 0; t < p.n_add_strided; ++t)
            add_src(p.add_base + t * p.add_stride - shift, p.ld_add, 1.0f);
        }
        uint16_t* dst = p.d + row * p.ldd + col;
        if (full) {
          uint2 o;
          o.x = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
          o.y = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
          *reinterpret_cast<uint2*>(dst) = o;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (col + q < nout) dst[q] = f32_to_bf16(v[q]);
        }
      }
    }
  }
}

template <typename Op, int BM, int BN, bool KN, bool SWIGLU>
hipError_t launch_tile(const GemmParams& p, hipStream_t s) {
  constexpr int smem = 2 * (BM + BN) * kRowBytes;
  auto kern = gemm_kernel<Op, BM, BN, KN, SWIGLU>;
  static bool attr_set = false;   // per process; the attribute is per function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nout_tiles = SWIGLU ? ((p.N / 2) + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  const int grid = ((p.M + BM - 1) / BM) * nout_tiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), smem, s, p);
  return hipGetLastError();
}

// Tile choice: the largest tile that still gives about one workgroup per CU.
int pick_tile(int M, int N, int epi) {
  const int n = epi == kEpiSwiglu ? N / 2 : N;
  const int bn_div = epi == kEpiSwiglu ? 2 : 1;
  auto tiles = [&](int bm, int bn) {
    return ((M + bm - 1) / bm) * ((n + bn / bn_div - 1) / (bn / bn_div));
  };
  if (tiles(256, 256) >= 240) return 0;
  if (tiles(256, 128) >= 240) return 1;
  return 2;
}

template <typename Op, bool KN, bool SW>
hipError_t dispatch_tile(const GemmParams& p, hipStream_t s) {
  switch (pick_tile(p.M, p.N, SW ? kEpiSwiglu : kEpiAlphaBeta)) {
    case 0: return launch_tile<Op, 256, 256, KN, SW>(p, s);
    case 1: return launch_tile<Op, 256, 128, KN, SW>(p, s);
    default: return launch_tile<Op, 128, 128, KN, SW>(p, s);
  }
}

}  // namespace

int gemm_grid_size(int M, int N, int epi) {
  const int t = pick_tile(M, N, epi);
  const int bm = t == 2 ? 128 : 256, bn = t == 0 ? 256 : 128;
  const int n = epi == kEpiSwiglu ? N / 2 : N;
  const int bno = epi == kEpiSwiglu ? bn / 2 : bn;
  return ((M + bm - 1) / bm) * ((n + bno - 1) / bno);
}

hipError_t launch_gemm(const GemmParams& p, int dtype, int layout, int epi, hipStream_t s) {
  const bool kn = layout == kKN, sw = epi == kEpiSwiglu;
  if (dtype == kBf16) {
    if (kn) return sw ? dispatch_tile<OpBf16, true, true>(p, s) : dispatch_tile<OpBf16, true, false>(p, s);
    return sw ? dispatch_tile<OpBf16, false, true>(p, s) : dispatch_tile<OpBf16, false, false>(p, s);
  }
  if (kn) return hipErrorInvalidValue;     // fp8 is NK only (validated on the host)
  return sw ? dispatch_tile<OpE4m3, false, true>(p, s) : dispatch_tile<OpE4m3, false, false>(p, s);
}

}  // namespace tpg
