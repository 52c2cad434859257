// Row kernels: the FFN's LayerNorm / SiLU gate and the All-to-All permutes.
//
// ln_silu: for each row of z = [u | g] (p04 statement, "Computation and
// communication example"), h = LN(u; gx, bx) * silu(LN(g; gg, bg)) with
// LN(v) = (v - mean) / sqrt(mean((v - mean)^2) + eps) * gamma + beta.
// One 256-thread workgroup per row; the row is read once from HBM into
// registers (16-byte loads), the mean and then the centred second moment are
// formed with wave64 butterfly reductions plus a 4-entry LDS exchange, and
// the gated product is written as bf16. HBM-bound: 6H bytes per row.
//
// permute: the dispatch / combine layout maps of the same statement ("Interface,
// layout, and parameters") are unions of contiguous runs (one per source rank
// and batch row, L*D elements long); each workgroup copies 16-byte chunks of
// one run, bit-exactly.
#include <algorithm>
#include <cstring>

#include "common.h"
#include "gemm.h"

namespace tpg {

namespace {

constexpr int kRowThreads = 256;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over the workgroup of two values at once.
__device__ __forceinline__ float2 block_sum2(float a, float b, float2* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = make_float2(a, b);
  __syncthreads();
  float2 s = red[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / 64; ++w) { s.x += red[w].x; s.y += red[w].y; }
  return s;
}

__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xffff);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// CH = 8-element chunks per thread per half (H <= 8 * 256 * CH).
template <int CH>
__global__ __launch_bounds__(kRowThreads) void ln_silu_kernel(
    const uint16_t* __restrict__ z, int64_t ldz, uint16_t* __restrict__ h, int64_t ldh, int H,
    const uint16_t* __restrict__ gx, const uint16_t* __restrict__ bx,
    const uint16_t* __restrict__ gg, const uint16_t* __restrict__ bg, float eps) {
  __shared__ float2 red[kRowThreads / 64];
  const int64_t row = blockIdx.x;
  const uint16_t* zu = z + row * ldz;
  const uint16_t* zg = zu + H;
  const int nchunk = H >> 3;
  float u[CH][8], g[CH][8];
  float su = 0.f, sg = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = c * kRowThreads + threadIdx.x;
    if (ch < nchunk) {
      // z is read once: non-temporal, so it does not evict what the GEMM
      // running beside this pass keeps in L2 (layer 2171 -> 2127 us)
      const u32x4 vu = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(zu + ch * 8));
      const u32x4 vg = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(zg + ch * 8));
      unpack8(make_uint4(vu.x, vu.y, vu.z, vu.w), u[c]);
      unpack8(make_uint4(vg.x, vg.y, vg.z, vg.w), g[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) { su += u[c][e]; sg += g[c][e]; }
    }
  }
  const float inv_h = 1.0f / static_cast<float>(H);
  float2 s = block_sum2(su, sg, red);
  const float mu = s.x * inv_h, mg = s.y * inv_h;
  float qu = 0.f, qg = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = c * kRowThreads + threadIdx.x;
    if (ch < nchunk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float du = u[c][e] - mu, dg = g[c][e] - mg;
        qu += du * du;
        qg += dg * dg;
      }
    }
  }
  s = block_sum2(qu, qg, red);
  const float ru = rsqrtf(s.x * inv_h + eps), rg = rsqrtf(s.y * inv_h + eps);
  uint16_t* hr = h + row * ldh;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = c * kRowThreads + threadIdx.x;
    if (ch < nchunk) {
      float a[8], b[8], cc[8], d[8];
      unpack8(*reinterpret_cast<const uint4*>(gx + ch * 8), a);
      unpack8(*reinterpret_cast<const uint4*>(bx + ch * 8), b);
      unpack8(*reinterpret_cast<const uint4*>(gg + ch * 8), cc);
      unpack8(*reinterpret_cast<const uint4*>(bg + ch * 8), d);
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float x0 = (u[c][e] - mu) * ru * a[e] + b[e];
        const float x1 = (u[c][e + 1] - mu) * ru * a[e + 1] + b[e + 1];
        const float y0 = (g[c][e] - mg) * rg * cc[e] + d[e];
        const float y1 = (g[c][e + 1] - mg) * rg * cc[e + 1] + d[e + 1];
        o[e / 2] = pack_bf16x2(x0 * silu_f32(y0), x1 * silu_f32(y1));
      }
      // h is read back only after every slot's pass: non-temporal too
      const u32x4 ov = {o[0], o[1], o[2], o[3]};
      __builtin_nontemporal_store(ov, reinterpret_cast<u32x4*>(hr + ch * 8));
    }
  }
}

// ---------------------------------------------------------------------------
// FFN backward, row part. For each row of z = [u | g] with upstream gradient
// dh (the gradient of h = LN_x(u) * silu(LN_gate(g))):
//   a = LN_x(u), b = LN_gate(g), s = silu(b), sg = logistic(b)
//   da = dh * s,  db = dh * a * sg * (1 + b (1 - sg))
//   du = (da gx - mean(da gx) - xu mean(da gx xu)) * ru   (xu = (u - mu) ru)
//   dg likewise;  dz = [du | dg] (bf16)
// and, summed over the workgroup's rows in fp32 registers, the column
// partials of the LayerNorm parameter gradients (da xu, da, db xg, db) and of
// the first bias gradient (du, dg). Workgroup w takes rows [w R, (w+1) R) and
// writes its partials to block w of two fp32 buffers; the gamma / beta
// partials are added to what the block already holds when `accumulate` is
// set (they sum over slots). Two workgroup reductions per row (the shifted
// first and second moments; the two backward means). HBM-bound: 10H bytes
// per row (z and dh in, dz out).
constexpr int kBwdThreads = 512;

// Sum over the workgroup of four values; `red` alternates between two buffers
// on consecutive calls, so one barrier suffices: a wave can only overwrite a
// buffer two reductions later, after every wave has passed the barrier of the
// reduction in between and so has finished reading it.
__device__ __forceinline__ float4 block_sum4(float a, float b, float c, float d, float4* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  c = wave_sum(c);
  d = wave_sum(d);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = make_float4(a, b, c, d);
  __syncthreads();
  float4 s = red[0];
#pragma unroll
  for (int w = 1; w < kBwdThreads / 64; ++w) {
    s.x += red[w].x;
    s.y += red[w].y;
    s.z += red[w].z;
    s.w += red[w].w;
  }
  return s;
}

__device__ __forceinline__ void store8_bf16(uint16_t* dst, const float* f) {
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
  *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ void put8(float* at, const float* v, int accumulate) {
  float4* dst = reinterpret_cast<float4*>(at);
  float4 lo = make_float4(v[0], v[1], v[2], v[3]);
  float4 hi = make_float4(v[4], v[5], v[6], v[7]);
  if (accumulate) {
    const float4 ol = dst[0], oh = dst[1];
    lo.x += ol.x; lo.y += ol.y; lo.z += ol.z; lo.w += ol.w;
    hi.x += oh.x; hi.y += oh.y; hi.z += oh.z; hi.w += oh.w;
  }
  dst[0] = lo;
  dst[1] = hi;
}

// One 16-byte load (a single dwordx4) of 8 bf16, or zeros when !on.
__device__ __forceinline__ uint4 load16_or_zero(const uint16_t* p, bool on) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v = {0u, 0u, 0u, 0u};
  if (on) v = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// CH = 8-column chunks per thread and half (H <= 8 * kBwdThreads * CH).
// Memory schedule: the four LayerNorm parameter vectors are read once, into
// registers (packed bf16), and every global read of a row (z, dh and the
// row's first elements, which shift the moment sums) is issued one row ahead,
// so the only wait per row is for loads issued a whole row earlier. The row statistics come
// from one reduction of sums shifted by the row's first element
// (sum (v - v0), sum (v - v0)^2), which keeps the variance free of
// cancellation for rows whose mean is large against their spread.
template <int CH>
__global__ __launch_bounds__(kBwdThreads) void ffn_bwd_rows_kernel(
    const uint16_t* __restrict__ z, int64_t ldz, const uint16_t* __restrict__ dh, int64_t lddh,
    uint16_t* __restrict__ dz, int64_t lddz, int rows, int rows_per_block, int H,
    const uint16_t* __restrict__ gx, const uint16_t* __restrict__ bx, const uint16_t* __restrict__ gg,
    const uint16_t* __restrict__ bg, float eps, float* __restrict__ part_gb, int accumulate,
    float* __restrict__ part_b1) {
  __shared__ float4 red[2][kBwdThreads / 64];
  // the gamma / beta partials [4][H] live in LDS (each thread owns its
  // columns, so there are no conflicts); the b1 partials in registers
  extern __shared__ __attribute__((aligned(16))) float lds_gb[];
  const int nchunk = H >> 3;
  const float inv_h = 1.0f / static_cast<float>(H);
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  uint4 q_gx[CH], q_bx[CH], q_gg[CH], q_bg[CH];   // this thread's parameter chunks
  float p_du[CH][8], p_dg[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = c * kBwdThreads + threadIdx.x;
    const bool on = ch < nchunk;
    q_gx[c] = load16_or_zero(gx + ch * 8, on);
    q_bx[c] = load16_or_zero(bx + ch * 8, on);
    q_gg[c] = load16_or_zero(gg + ch * 8, on);
    q_bg[c] = load16_or_zero(bg + ch * 8, on);
#pragma unroll
    for (int e = 0; e < 8; ++e) p_du[c][e] = p_dg[c][e] = 0.f;
    if (on)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        reinterpret_cast<float4*>(lds_gb + q * H + ch * 8)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
        reinterpret_cast<float4*>(lds_gb + q * H + ch * 8)[1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
  }
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(rows, r0 + rows_per_block);
  uint4 nu[CH], ng[CH], nd[CH];
  uint16_t nu0 = 0, ng0 = 0;
  auto fetch = [&](int row) {
    const bool live = row < r1;                // past the block's rows: nothing is read
    const uint16_t* zr = z + int64_t(live ? row : 0) * ldz;
    const uint16_t* dr = dh + int64_t(live ? row : 0) * lddh;
    nu0 = live ? zr[0] : uint16_t(0);
    ng0 = live ? zr[H] : uint16_t(0);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = c * kBwdThreads + threadIdx.x;
      const bool on = live && ch < nchunk;
      nu[c] = load16_or_zero(zr + ch * 8, on);
      ng[c] = load16_or_zero(zr + H + ch * 8, on);
      nd[c] = load16_or_zero(dr + ch * 8, on);
    }
  };
  fetch(r0);
  int k = 0;                                   // reduction buffer
  for (int row = r0; row < r1; ++row) {
    const float u0 = bf16_to_f32(nu0), g0 = bf16_to_f32(ng0);
    float u[CH][8], g[CH][8], d[CH][8], dg[CH][8];
    uint4 dq[CH];                              // this row's dh, packed
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      unpack8(nu[c], u[c]);
      unpack8(ng[c], g[c]);
      dq[c] = nd[c];
    }
    fetch(row + 1);                            // lands while this row is worked on
    float su = 0.f, sg = 0.f, qu = 0.f, qg = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const bool on = c * kBwdThreads + int(threadIdx.x) < nchunk;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a = on ? u[c][e] - u0 : 0.f, b = on ? g[c][e] - g0 : 0.f;
        su += a;
        sg += b;
        qu += a * a;
        qg += b * b;
      }
    }
    float4 s4 = block_sum4(su, sg, qu, qg, red[k]);
    k ^= 1;
    const float du0 = s4.x * inv_h, dg0 = s4.y * inv_h;   // mean - v0
    const float mu = u0 + du0, mg = g0 + dg0;
    const float ru = rsqrtf(fmaxf(s4.z * inv_h - du0 * du0, 0.f) + eps);
    const float rg = rsqrtf(fmaxf(s4.w * inv_h - dg0 * dg0, 0.f) + eps);
    float m0 = 0.f, m1 = 0.f, m2 = 0.f, m3 = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = c * kBwdThreads + threadIdx.x;
      const bool on = ch < nchunk;
      float ag[8], ab[8], cg[8], cb[8], dhv[8];
      unpack8(q_gx[c], ag);
      unpack8(q_bx[c], ab);
      unpack8(q_gg[c], cg);
      unpack8(q_bg[c], cb);
      unpack8(dq[c], dhv);
      float t_gx[8], t_bx[8], t_gg[8], t_bg[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xu = on ? (u[c][e] - mu) * ru : 0.f, xg = on ? (g[c][e] - mg) * rg : 0.f;
        const float a = xu * ag[e] + ab[e];
        const float b = xg * cg[e] + cb[e];
        const float sgm = sigmoid_f32(b);
        const float da = dhv[e] * (b * sgm);
        const float db = dhv[e] * a * sgm * (1.0f + b * (1.0f - sgm));
        t_gx[e] = da * xu;
        t_bx[e] = da;
        t_gg[e] = db * xg;
        t_bg[e] = db;
        const float dxu = da * ag[e], dxg = db * cg[e];
        m0 += dxu;
        m1 += dxu * xu;
        m2 += dxg;
        m3 += dxg * xg;
        u[c][e] = xu;          // u, g: the normalised rows
        g[c][e] = xg;
        d[c][e] = dxu;         // da * gx and db * gg, for the last phase
        dg[c][e] = dxg;
      }
      if (on) {
        float* lp = lds_gb + ch * 8;
        const float* t[4] = {t_gx, t_bx, t_gg, t_bg};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float4* v = reinterpret_cast<float4*>(lp + q * H);
          float4 lo = v[0], hi = v[1];
          lo.x += t[q][0]; lo.y += t[q][1]; lo.z += t[q][2]; lo.w += t[q][3];
          hi.x += t[q][4]; hi.y += t[q][5]; hi.z += t[q][6]; hi.w += t[q][7];
          v[0] = lo;
          v[1] = hi;
        }
      }
    }
    s4 = block_sum4(m0, m1, m2, m3, red[k]);
    k ^= 1;
    const float mdu = s4.x * inv_h, mdux = s4.y * inv_h, mdg = s4.z * inv_h, mdgx = s4.w * inv_h;
    uint16_t* dzr = dz + int64_t(row) * lddz;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = c * kBwdThreads + threadIdx.x;
      if (ch < nchunk) {
        float ou[8], og[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xu = u[c][e], xg = g[c][e];
          ou[e] = (d[c][e] - mdu - xu * mdux) * ru;
          og[e] = (dg[c][e] - mdg - xg * mdgx) * rg;
          p_du[c][e] += ou[e];
          p_dg[c][e] += og[e];
        }
        store8_bf16(dzr + ch * 8, ou);
        store8_bf16(dzr + H + ch * 8, og);
      }
    }
  }
  // partials of this block: gamma/beta [4][H] (accumulated over slots), b1 [2H]
  float* pgb = part_gb + int64_t(blockIdx.x) * 4 * H;
  float* pb1 = part_b1 + int64_t(blockIdx.x) * 2 * H;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = c * kBwdThreads + threadIdx.x;
    if (ch < nchunk) {
#pragma unroll
      for (int q = 0; q < 4; ++q) put8(pgb + q * H + ch * 8, lds_gb + q * H + ch * 8, accumulate);
      put8(pb1 + ch * 8, p_du[c], 0);
      put8(pb1 + H + ch * 8, p_dg[c], 0);
    }
  }
}

// Column sums of fp32 partials: out[c] = bf16(sum_b part[b * blk_stride + c]).
// A 256-thread workgroup takes 32 columns; its 8 row groups each sum a
// fixed, interleaved eighth of the blocks, and the 8 group sums are added in
// group order (deterministic).
constexpr int kSumCols = 32;

__global__ __launch_bounds__(256) void colsum_f32_kernel(const float* __restrict__ part, int nblk, int64_t blk_stride,
                                                          int ncols, uint16_t* __restrict__ out) {
  __shared__ float acc[256 / kSumCols][kSumCols];
  const int cl = threadIdx.x % kSumCols, grp = threadIdx.x / kSumCols;
  const int c = blockIdx.x * kSumCols + cl;
  float s = 0.f;
  if (c < ncols)
    for (int b = grp; b < nblk; b += 256 / kSumCols) s += part[int64_t(b) * blk_stride + c];
  acc[grp][cl] = s;
  __syncthreads();
  if (grp == 0 && c < ncols) {
    float t = acc[0][cl];
#pragma unroll
    for (int g = 1; g < 256 / kSumCols; ++g) t += acc[g][cl];
    out[c] = f32_to_bf16(t);
  }
}

// fp32 column partials of a bf16 matrix, one per block of rows:
// part[blk][c] = sum over rows [blk R, (blk+1) R) of src[row * ld + c].
__global__ __launch_bounds__(256) void colsum_bf16_kernel(const uint16_t* __restrict__ src, int rows, int cols,
                                                           int64_t ld, int rows_per_block, float* __restrict__ part) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  const int r0 = blockIdx.y * rows_per_block, r1 = min(rows, r0 + rows_per_block);
  float s = 0.f;
  for (int r = r0; r < r1; ++r) s += bf16_to_f32(src[int64_t(r) * ld + c]);
  part[int64_t(blockIdx.y) * cols + c] = s;
}

constexpr int kPermThreads = 256;
constexpr int kPermUnroll = 4;

__global__ __launch_bounds__(kPermThreads) void permute16_kernel(const PermuteParams p) {
  const int64_t run = blockIdx.x;          // run = s * B + b
  const int s = static_cast<int>(run / p.B);
  const int64_t b = run - s * p.B;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* src = reinterpret_cast<const u32x4*>(p.src[s] + p.src_base + b * p.src_bstride);
  u32x4* dst = reinterpret_cast<u32x4*>(p.dst + s * p.dst_sstride + b * p.dst_bstride);
  const int64_t nvec = p.run_bytes >> 4;
  const int64_t base = static_cast<int64_t>(blockIdx.y) * kPermThreads * kPermUnroll + threadIdx.x;
  u32x4 v[kPermUnroll];
#pragma unroll
  for (int u = 0; u < kPermUnroll; ++u) {
    const int64_t i = base + u * kPermThreads;
    if (i < nvec) v[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < kPermUnroll; ++u) {
    const int64_t i = base + u * kPermThreads;
    if (i < nvec) __builtin_nontemporal_store(v[u], dst + i);
  }
}

__global__ __launch_bounds__(kPermThreads) void permute1_kernel(const PermuteParams p) {
  const int64_t run = blockIdx.x;
  const int s = static_cast<int>(run / p.B);
  const int64_t b = run - s * p.B;
  const uint8_t* src = p.src[s] + p.src_base + b * p.src_bstride;
  uint8_t* dst = p.dst + s * p.dst_sstride + b * p.dst_bstride;
  for (int64_t i = static_cast<int64_t>(blockIdx.y) * kPermThreads + threadIdx.x; i < p.run_bytes;
       i += static_cast<int64_t>(gridDim.y) * kPermThreads)
    dst[i] = src[i];
}

// Stage deliveries: n slices of nvec 16-byte vectors, slice s from src[s] to
// dst + s * dst_stride. blockIdx.y picks the slice; the x blocks stride over
// it, eight vectors in flight per thread. The loads are non-temporal (the
// sources are read once); the stores are ordinary, so the receive slots stay
// in L2 and the Infinity Cache for the stage GEMM that reads them next.
// Measured on MI355X, 7 x 8 MiB with cold caches: 22.8 us (5.1 TB/s read +
// write), against 40 us for seven runtime copies and 34 us for the same
// kernel with ordinary loads.
constexpr int kDelThreads = 256;
constexpr int kDelUnroll = 8;

__global__ __launch_bounds__(kDelThreads) void deliver16_kernel(const DeliverParams p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* src = reinterpret_cast<const u32x4*>(p.src[blockIdx.y]);
  u32x4* dst = reinterpret_cast<u32x4*>(p.dst + int64_t(blockIdx.y) * p.dst_stride);
  const int64_t step = int64_t(gridDim.x) * kDelThreads * kDelUnroll;
  for (int64_t base = int64_t(blockIdx.x) * kDelThreads * kDelUnroll + threadIdx.x; base < p.nvec; base += step) {
    u32x4 v[kDelUnroll];
#pragma unroll
    for (int u = 0; u < kDelUnroll; ++u) {
      const int64_t i = base + u * kDelThreads;
      if (i < p.nvec) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kDelUnroll; ++u) {
      const int64_t i = base + u * kDelThreads;
      if (i < p.nvec) dst[i] = v[u];
    }
  }
}

// Deliveries for in-kernel gates: workgroup (r, i) copies rows
// [r * rows / R, (r + 1) * rows / R) of slice i, chunk by chunk along the
// row (chunk-major, so every slice's first chunk lands first, as the links
// of a real all-gather deliver all peers at once), eight 16-byte vectors in
// flight per thread. Stores are system-scope (sc0 sc1): each completes
// (vmcnt 0) only once it is visible at the device coherence point, so a
// workgroup on another XCD that reads with device-coherent loads sees it.
// Only after every store of the chunk has completed is the chunk's counter
// bumped, with a relaxed device-scope atomic: the stores need no release
// fence (whose L2 writeback cost ~57 us per call on the e4m3 workload), since
// they leave nothing behind in this XCD's L2. Vector stores and atomics only.
constexpr int kChunkThreads = 256;
constexpr int kChunkUnroll = 8;

__global__ __launch_bounds__(kChunkThreads) void chunk_deliver_kernel(const ChunkDeliverParams p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int i = blockIdx.y, r = blockIdx.x, R = p.wg_per_slice;
  const int64_t row0 = int64_t(r) * p.rows / R, row1 = int64_t(r + 1) * p.rows / R;
  const int64_t nrows = row1 - row0;
  const uint8_t* src = p.src[i];
  uint8_t* dst = p.dst + int64_t(i) * p.rows * p.row_bytes;
  for (int c = 0; c < p.nch; ++c) {
    const int64_t b0 = int64_t(c) * p.chunk_bytes;
    const int64_t cb = min(p.chunk_bytes, p.row_bytes - b0);
    const int64_t vpr = cb / 16;                 // vectors per row in this chunk
    const int64_t nvec = nrows * vpr;
    for (int64_t base = threadIdx.x; base < nvec; base += int64_t(kChunkThreads) * kChunkUnroll) {
      u32x4 v[kChunkUnroll];
#pragma unroll
      for (int u = 0; u < kChunkUnroll; ++u) {
        const int64_t k = base + int64_t(u) * kChunkThreads;
        if (k < nvec) {
          const int64_t off = (row0 + k / vpr) * p.row_bytes + b0 + (k % vpr) * 16;
          v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off));
        }
      }
#pragma unroll
      for (int u = 0; u < kChunkUnroll; ++u) {
        const int64_t k = base + int64_t(u) * kChunkThreads;
        if (k < nvec) {
          const int64_t off = (row0 + k / vpr) * p.row_bytes + b0 + (k % vpr) * 16;
          asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(dst + off), "v"(v[u]) : "memory");
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(p.gate + i * p.nch + c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Zero fill in 16-byte vector stores (used where a result is an empty sum).
__global__ __launch_bounds__(256) void fill_zero16_kernel(uint4* p, int64_t n16) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += int64_t(gridDim.x) * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_fill_zero16(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = int64_t(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n16 + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero16_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

int chunk_deliver_wgs_per_slice(int64_t rows) { return static_cast<int>(std::min<int64_t>(32, std::max<int64_t>(1, rows / 8))); }

hipError_t launch_chunk_deliver(const ChunkDeliverParams& p, hipStream_t s) {
  if (!p.dst || !p.gate || p.n < 1 || p.n > kMaxGateSlices || p.nch < 1 || p.rows < 1 || p.wg_per_slice < 1 ||
      p.row_bytes % 16 ||
      p.chunk_bytes % 16 || p.chunk_bytes < 16 || int64_t(p.nch) * p.chunk_bytes < p.row_bytes)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(chunk_deliver_kernel, dim3(p.wg_per_slice, p.n), dim3(kChunkThreads), 0, s, p);
  return hipGetLastError();
}

bool deliver_ok(const void* const* src, int n, size_t bytes, const void* dst, size_t dst_stride) {
  if (n < 1 || n > kMaxDeliver || bytes % 16 || dst_stride % 16 || dst_stride < bytes ||
      reinterpret_cast<uintptr_t>(dst) % 16)
    return false;
  for (int i = 0; i < n; ++i)
    if (!src[i] || reinterpret_cast<uintptr_t>(src[i]) % 16) return false;
  return true;
}

hipError_t launch_deliver(const void* const* src, int n, size_t bytes, void* dst, size_t dst_stride, hipStream_t s) {
  if (n == 0 || bytes == 0) return hipSuccess;
  if (!deliver_ok(src, n, bytes, dst, dst_stride)) return hipErrorInvalidValue;
  DeliverParams p;
  std::memset(&p, 0, sizeof(p));
  for (int i = 0; i < n; ++i) p.src[i] = static_cast<const uint8_t*>(src[i]);
  p.dst = static_cast<uint8_t*>(dst);
  p.dst_stride = static_cast<int64_t>(dst_stride);
  p.nvec = static_cast<int64_t>(bytes / 16);
  // about eight workgroups per CU over all slices (measured best), none idle
  const int64_t per_slice = (p.nvec + kDelThreads * kDelUnroll - 1) / (kDelThreads * kDelUnroll);
  const int64_t want = std::max<int64_t>(1, (int64_t(8) * device_cus() + n - 1) / n);
  const int64_t bx = std::min(per_slice, want);
  hipLaunchKernelGGL(deliver16_kernel, dim3(static_cast<unsigned>(bx), static_cast<unsigned>(n)), dim3(kDelThreads),
                     0, s, p);
  return hipGetLastError();
}

hipError_t launch_ln_silu(const uint16_t* z, int64_t ldz, uint16_t* h, int64_t ldh, int rows, int H,
                          const uint16_t* gx, const uint16_t* bx, const uint16_t* gg,
                          const uint16_t* bg, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int nchunk = H / 8;
  const int per = (nchunk + kRowThreads - 1) / kRowThreads;
  dim3 grid(rows), block(kRowThreads);
  if (per <= 1)
    hipLaunchKernelGGL(ln_silu_kernel<1>, grid, block, 0, s, z, ldz, h, ldh, H, gx, bx, gg, bg, eps);
  else if (per <= 2)
    hipLaunchKernelGGL(ln_silu_kernel<2>, grid, block, 0, s, z, ldz, h, ldh, H, gx, bx, gg, bg, eps);
  else if (per <= 4)
    hipLaunchKernelGGL(ln_silu_kernel<4>, grid, block, 0, s, z, ldz, h, ldh, H, gx, bx, gg, bg, eps);
  else if (per <= 8)
    hipLaunchKernelGGL(ln_silu_kernel<8>, grid, block, 0, s, z, ldz, h, ldh, H, gx, bx, gg, bg, eps);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_ffn_bwd_rows(const uint16_t* z, int64_t ldz, const uint16_t* dh, int64_t lddh, uint16_t* dz,
                               int64_t lddz, int rows, int H, const uint16_t* gx, const uint16_t* bx,
                               const uint16_t* gg, const uint16_t* bg, float eps, float* part_gb, int accumulate,
                               float* part_b1, int nblk, hipStream_t s) {
  if (rows == 0 || H == 0) return hipSuccess;
  if (nblk < 1 || H % 8) return hipErrorInvalidValue;
  const int per = (H / 8 + kBwdThreads - 1) / kBwdThreads;
  const int rpb = (rows + nblk - 1) / nblk;
  dim3 grid(nblk), block(kBwdThreads);
  const size_t lds = size_t(4) * H * sizeof(float);
  static uint64_t lds_set[2] = {0, 0};
  const void* kern = per <= 1 ? reinterpret_cast<const void*>(ffn_bwd_rows_kernel<1>)
                              : reinterpret_cast<const void*>(ffn_bwd_rows_kernel<2>);
  if (per <= 2) {
    if (hipError_t e = lds_limit_once(kern, 4 * 8192 * 4, lds_set[per - 1]); e != hipSuccess) return e;
  }
  if (per <= 1)
    hipLaunchKernelGGL(ffn_bwd_rows_kernel<1>, grid, block, lds, s, z, ldz, dh, lddh, dz, lddz, rows, rpb, H, gx, bx,
                       gg, bg, eps, part_gb, accumulate, part_b1);
  else if (per <= 2)      // H <= 8192 (more would spill at 512 threads)
    hipLaunchKernelGGL(ffn_bwd_rows_kernel<2>, grid, block, lds, s, z, ldz, dh, lddh, dz, lddz, rows, rpb, H, gx, bx,
                       gg, bg, eps, part_gb, accumulate, part_b1);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_colsum_f32(const float* part, int nblk, int64_t blk_stride, int ncols, uint16_t* out,
                             hipStream_t s) {
  if (ncols == 0) return hipSuccess;
  hipLaunchKernelGGL(colsum_f32_kernel, dim3((ncols + kSumCols - 1) / kSumCols), dim3(256), 0, s, part, nblk,
                     blk_stride, ncols, out);
  return hipGetLastError();
}

hipError_t launch_colsum_bf16(const uint16_t* src, int rows, int cols, int64_t ld, float* part, int nblk,
                              hipStream_t s) {
  if (cols == 0 || nblk < 1) return hipSuccess;
  const int rpb = (rows + nblk - 1) / nblk;
  hipLaunchKernelGGL(colsum_bf16_kernel, dim3((cols + 255) / 256, nblk), dim3(256), 0, s, src, rows, cols, ld, rpb,
                     part);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteParams& p, int P, hipStream_t s) {
  const int64_t runs = static_cast<int64_t>(P) * p.B;
  if (runs == 0 || p.run_bytes == 0) return hipSuccess;
  bool aligned = (p.run_bytes % 16 == 0) && (p.src_base % 16 == 0) && (p.src_bstride % 16 == 0) &&
                 (p.dst_sstride % 16 == 0) && (p.dst_bstride % 16 == 0) &&
                 (reinterpret_cast<uintptr_t>(p.dst) % 16 == 0);
  for (int i = 0; i < P; ++i) aligned = aligned && (reinterpret_cast<uintptr_t>(p.src[i]) % 16 == 0);
  if (aligned) {
    const int64_t nvec = p.run_bytes / 16;
    const int64_t gx = (nvec + kPermThreads * kPermUnroll - 1) / (kPermThreads * kPermUnroll);
    hipLaunchKernelGGL(permute16_kernel, dim3(static_cast<unsigned>(runs), static_cast<unsigned>(gx)),
                       dim3(kPermThreads), 0, s, p);
  } else {
    int64_t gx = (p.run_bytes + kPermThreads - 1) / kPermThreads;
    if (gx > 64) gx = 64;
    hipLaunchKernelGGL(permute1_kernel, dim3(static_cast<unsigned>(runs), static_cast<unsigned>(gx)),
                       dim3(kPermThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace tpg
