// MXFP8 matrix product on gfx950 scaled MFMA: out[M, N] = A[M, K] . B[N, K]^T.
//
// The consumer of the planes: a linear layer quantizes its bf16 activation on
// the fly and multiplies it by a pre-quantized weight (Megatron-Core
// quantization.utils page, mm_mxfp8); the AMD block-scaled matmul takes the
// plain rank-2 scale layout as its a_scales (Mojo
// DistributedAllGatherRMSNormQuantMXFP8 page, Limitations).  Both operands
// are rowwise planes: A = (qa [M, K], sa [M, K/32]) and B = (qb [N, K],
// sb [N, K/32]), i.e. both blocked along K.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, one E8M0 scale per 32 k):
// lane l holds row l % 32 of its operand; lane group h = l / 32 holds
// k = 16h .. 16h+15 in bytes 0-15 and k = 32+16h .. 32+16h+15 in bytes 16-31,
// and lane l supplies the scale of k block h of its row (block 0 is k 0..31,
// block 1 is k 32..63).  Output register r of lane l is row
// 8 (r / 4) + 4 h + r % 4, column l % 32.  This layout was established by a
// lane-layout probe of the instruction on the GPU; the parity tests check it
// end to end.
//
// Tiling: a workgroup computes a 128 x 128 tile with 4 waves of 64 x 64 (2 x 2
// MFMA tiles each).  K advances in tiles of 128 bytes staged through LDS: the
// next tile is loaded from HBM into registers while the current one feeds the
// MFMAs, then written to the other LDS buffer.  LDS rows are padded to 144
// bytes so that the 16-byte fragment reads of 8 consecutive rows fall on
// distinct banks.  Rows and columns past M or N read as zero and are not
// stored; K must be a multiple of 128.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kGT = 128;              // workgroup tile side (M and N)
constexpr int kGK = 128;              // K bytes per LDS tile
constexpr int kLdsStride = kGK + 16;  // padded LDS row
constexpr int kLdsTile = kGT * kLdsStride;

struct GemmParams {
  const uint8_t* qa;
  const uint8_t* sa;
  const uint8_t* qb;
  const uint8_t* sb;
  void* out;
  int64_t M, N, K;
  int32_t out_bf16;
  int32_t tiles_n;
};

__device__ __forceinline__ u32x4 ld_global(const uint8_t* base, int64_t rows, int64_t row,
                                           int64_t K, int64_t k) {
  return row < rows ? load16_cached(base + row * K + k) : u32x4{0, 0, 0, 0};
}

__global__ __launch_bounds__(kThreads) void mxfp8_gemm_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kLdsTile];   // [buffer][A, B]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)(blockIdx.x / p.tiles_n) * kGT;
  const int64_t n0 = (int64_t)(blockIdx.x % p.tiles_n) * kGT;
  const int64_t K = p.K, kblocks = K / kBlock;

  // global -> LDS: thread t moves 16-byte chunks t + 256 u (u < 4) of each
  // 128 x 128-byte tile: row (t >> 3) + 32 u, k offset 16 (t & 7)
  const int lrow = tid >> 3, lk = (tid & 7) * 16;
  u32x4 ra[4], rb[4];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ra[u] = ld_global(p.qa, p.M, m0 + lrow + 32 * u, K, k0 + lk);
      rb[u] = ld_global(p.qb, p.N, n0 + lrow + 32 * u, K, k0 + lk);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<u32x4*>(&lds[buf][0][(lrow + 32 * u) * kLdsStride + lk]) = ra[u];
      *reinterpret_cast<u32x4*>(&lds[buf][1][(lrow + 32 * u) * kLdsStride + lk]) = rb[u];
    }
  };

  // this lane's operand rows in each of the wave's two 32-row tiles
  const int h = lane >> 5;
  const int fr = lane & 31;
  int64_t arow[2], brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    arow[i] = m0 + wm * 64 + 32 * i + fr;
    brow[i] = n0 + wn * 64 + 32 * i + fr;
  }
  // scale bytes of this lane for k tile k0: index [tile i][64-k step s]
  auto scales = [&](const uint8_t* s, const int64_t* rows, int64_t nrows, int64_t k0,
                    uint32_t (&out)[2][2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int st = 0; st < 2; ++st)
        out[i][st] = rows[i] < nrows ? s[rows[i] * kblocks + k0 / kBlock + 2 * st + h] : 127u;
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  uint32_t sa_cur[2][2], sb_cur[2][2], sa_nxt[2][2], sb_nxt[2][2];
  fetch(0);
  scales(p.sa, arow, p.M, 0, sa_cur);
  scales(p.sb, brow, p.N, 0, sb_cur);
  stash(0);
  __syncthreads();

  const int64_t ktiles = K / kGK;
  for (int64_t kt = 0; kt < ktiles; ++kt) {
    const int buf = (int)(kt & 1);
    const bool more = kt + 1 < ktiles;
    if (more) {
      fetch((kt + 1) * kGK);
      scales(p.sa, arow, p.M, (kt + 1) * kGK, sa_nxt);
      scales(p.sb, brow, p.N, (kt + 1) * kGK, sb_nxt);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      v8i fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint8_t* la = &lds[buf][0][(wm * 64 + 32 * i + fr) * kLdsStride + 64 * st + 16 * h];
        const uint8_t* lb = &lds[buf][1][(wn * 64 + 32 * i + fr) * kLdsStride + 64 * st + 16 * h];
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(la);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(la + 32);
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(lb);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(lb + 32);
        fa[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        fb[i] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[i], fb[j], acc[i][j], 0, 0, 0, (int)sa_cur[i][st], 0, (int)sb_cur[j][st]);
    }
    if (more) {
      // the other buffer was last read in the previous iteration, which every
      // wave finished before that iteration's barrier
      stash(buf ^ 1);
      __syncthreads();          // the next tile is in LDS
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          sa_cur[i][st] = sa_nxt[i][st];
          sb_cur[i][st] = sb_nxt[i][st];
        }
    }
  }

  // store: register r of tile (i, j) is row 8 (r/4) + 4 h + r % 4, column fr
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + 32 * j + fr;
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
        if (row >= p.M) continue;
        if (p.out_bf16)
          reinterpret_cast<uint16_t*>(p.out)[row * p.N + col] = (uint16_t)f32_to_bf16(acc[i][j][r]);
        else
          __builtin_nontemporal_store(acc[i][j][r], reinterpret_cast<float*>(p.out) + row * p.N + col);
      }
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                       int64_t M, int64_t N, int64_t K, void* out, bool out_bf16, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmParams p;
  p.qa = qa; p.sa = sa; p.qb = qb; p.sb = sb; p.out = out;
  p.M = M; p.N = N; p.K = K;
  p.out_bf16 = out_bf16 ? 1 : 0;
  p.tiles_n = (int32_t)((N + kGT - 1) / kGT);
  const int64_t tiles = ((M + kGT - 1) / kGT) * p.tiles_n;
  hipLaunchKernelGGL(mxfp8_gemm_kernel, dim3((uint32_t)tiles), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mx
