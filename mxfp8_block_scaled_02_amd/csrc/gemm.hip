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
// block 1 is k 32..63) in the low byte of its scale register.  Output register
// r of lane l is row 8 (r / 4) + 4 h + r % 4, column l % 32.  This layout was
// established by a lane-layout probe of the instruction on the GPU; the parity
// tests check it end to end.
//
// Three kinds of tiling share that fragment layout:
//
// * ring tiles (M > 128, K >= 512, a weight wide enough to fill the CUs): a workgroup of
//   four waves (2 x 2) computes a 256 x 256, 128 x 256, 128 x 128 or 64 x 128
//   tile, one workgroup per CU.  K advances in stages of 64 bytes through a ring of four
//   LDS slots that the loads fill directly (global_load_lds_dwordx4, no
//   register staging): the loads of stage s + 4 go out while stage s
//   computes, and the fragments of stage s + 1 are read into a second
//   register set meanwhile, so a stage waits only for data requested three
//   stages earlier.  Scales travel the same way, 16 bytes (512 k) per row and
//   operand every eight stages; with K % 512 != 0 the last eight stages start
//   with repeats of the stage before, whose scale bytes are set to 0, so that
//   the group is a whole one.  Waits count the loads still allowed in
//   flight (s_waitcnt vmcnt(n)) instead of draining them all at each barrier.
//   Workgroups are mapped to tiles so that each XCD works on a compact block
//   of the output (its L2 holds the shared panels), and XCD pairs start K at
//   different quarters.  The tile size is the one whose rounds of tiles over
//   the 256 CUs take least time: large tiles move fewer bytes per MFMA, small
//   ones keep more CUs busy when M or N is small.
// * tile128: 128 x 128 tiles (four waves of 64 x 64) staged through registers
//   into padded LDS rows; it takes the problems with M > 128 and K < 512 that
//   the skinny kernel does not.
// * skinny (decode and small batches, M <= 128; or any M whose 32-, 64- or,
//   up to 512 rows, 128-row blocks times the 32-column strips of B fit one
//   workgroup per CU): 32 output columns of one row block per workgroup, K
//   split over its waves, B streamed once through LDS (see the section
//   below).
//
// Rows of A or B past M or N read a valid row (the last one) and their
// outputs are not stored.  K must be a multiple of 128, and the scale planes'
// rows are a caller-given pitch apart (a multiple of 4: the ring tiles' 16-byte
// scale loads into LDS need only 4-byte aligned addresses).  The
// order in which the 64-deep MFMA steps accumulate depends on the tiling and,
// for the ring tiles, on the tile's starting quarter; every order stays
// within the tolerance that the tests derive for the instruction.
#include <vector>

#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

struct GemmParams {
  const uint8_t* qa;
  const uint8_t* sa;
  const uint8_t* qb;
  const uint8_t* sb;
  void* out;
  int64_t M, N, K;
  int64_t sa_ld, sb_ld;       // bytes between scale rows of A and of B
  int64_t sa_gs, sb_gs;       // bytes between 16-block scale groups of a row
                              // (16 compact or padded, rows * 16 in the MFMA order)
  int64_t ldo;                // elements between output rows (>= N)
  int32_t out_bf16;
  int32_t tiles_m, tiles_n;
};

// A table of products for one grouped launch (the kernel argument segment
// holds at most 4 KiB).
constexpr int kGemmGroupMax = 32;
struct GemmGroupArgs {
  int32_t n;
  int32_t task_start[kGemmGroupMax + 1];
  GemmParams d[kGemmGroupMax];
};
static_assert(sizeof(GemmGroupArgs) <= 4096, "kernel arguments");

__device__ __forceinline__ v8i frag(const u32x4& lo, const u32x4& hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ v16f mfma(const v8i& a, const v8i& b, const v16f& c, uint32_t sa,
                                     uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, (int)sa, 0, (int)sb);
}

// store register r of an MFMA tile whose top-left output is (row0, col0)
__device__ __forceinline__ void store_tile(const GemmParams& p, const v16f& acc, int64_t row0,
                                           int64_t col, int h) {
  if (col >= p.N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t row = row0 + 8 * (r / 4) + 4 * h + (r % 4);
    if (row >= p.M) continue;
    if (p.out_bf16)
      reinterpret_cast<uint16_t*>(p.out)[row * p.ldo + col] = (uint16_t)f32_to_bf16(acc[r]);
    else
      __builtin_nontemporal_store(acc[r], reinterpret_cast<float*>(p.out) + row * p.ldo + col);
  }
}

// bf16 output of two 32 x 32 tiles side by side (columns col .. col + 63,
// rows row0 + 8 (r / 4) + 4 h + r % 4; the columns lie inside the output and
// N and the row pitch are even; ROWS_IN says every row lies inside too, else rows past M are
// skipped), written as whole 128-byte row segments.  Lane fr
// packs its values of the two tiles (columns fr and 32 + fr) into one dword;
// lane d then takes columns 2d and 2d + 1 from lanes 2d and 2d + 1 (mod 32,
// same half h), so 32 lanes store one row's 128 bytes.  Storing each lane's
// own column instead leaves half lines, which cost several times the bytes'
// HBM time; the nontemporal hint, as for float32 output, saves a little more.
template <bool ROWS_IN = true>
__device__ __forceinline__ void store_bf16_pair(const GemmParams& p, const v16f& lo, const v16f& hi,
                                                int64_t row0, int64_t col, int fr, int h) {
  const int src0 = 4 * (((2 * fr) & 31) + 32 * h), src1 = src0 + 4;
  const uint32_t sel = fr < 16 ? 0x05040100u : 0x07060302u;   // low or high halves
  uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + col + 2 * fr;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int ab = (int)pack_bf16x2(lo[r], hi[r]);
    const uint32_t x0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src0, ab);
    const uint32_t x1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src1, ab);
    const int64_t row = row0 + 8 * (r / 4) + 4 * h + (r % 4);
    if (ROWS_IN || row < p.M)
      __builtin_nontemporal_store(__builtin_amdgcn_perm(x1, x0, sel),
                                  reinterpret_cast<uint32_t*>(o + row * p.ldo));
  }
}

// ---- ring tiles (256 x 256, 128 x 256, 128 x 128, 64 x 128) ---------------

constexpr int kBT = 256;                // largest workgroup tile side
constexpr int kBK = 64;                 // K bytes per stage (one MFMA step)
constexpr int kStages = 4;              // LDS ring depth
constexpr int kOpBytes = kBT * kBK;     // one operand's stage in LDS at most (16 KiB)
constexpr int kGroup = 8;               // stages per scale group (512 k, 16 scale bytes a row)
constexpr int kScBytes = kBT * 16;      // one operand's scale group in LDS (4 KiB)
constexpr int kGroupM = 8;              // tile rows per group of the tile order
constexpr int kCUs = 256;               // one ring tile per CU at a time (LDS-limited)

// one LDS array per ring slot (A then B) and per scale buffer (A then B): the
// compiler tells in-flight LDS loads apart by the array they write, and only
// for a handful of arrays
__shared__ __attribute__((aligned(1024))) uint8_t s_slot0[2 * kOpBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_slot1[2 * kOpBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_slot2[2 * kOpBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_slot3[2 * kOpBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_scale0[2 * kScBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_scale1[2 * kScBytes];

typedef __attribute__((address_space(3))) void* lds_ptr;

template <int N> __device__ __forceinline__ uint8_t* slot_a() {
  return N == 0 ? s_slot0 : N == 1 ? s_slot1 : N == 2 ? s_slot2 : s_slot3;
}

// LDS placement of a 64-byte row: its 16-byte chunk c sits at chunk
// c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3, so that the 16-byte fragment
// reads of 32 consecutive rows hit distinct banks in 8- and 16-lane phases
__device__ __forceinline__ int row_swizzle(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// rows r0 .. r0+ROWS-1, k0 .. k0+63 of one operand into a ring slot: wave w's
// load u covers the 16 rows of group g = 4u + w, lane L the physical chunk
// L % 4 of row 16 g + L / 4 (1 KiB per load, written lane after lane)
template <int ROWS>
__device__ __forceinline__ void load_stage(const uint8_t* base, int64_t rows, int64_t r0, int64_t K,
                                           int64_t k0, uint8_t* lds, int wave, int lane) {
  const int lr = lane >> 2;
#pragma unroll
  for (int u = 0; u < ROWS / 64; ++u) {
    const int g = 4 * u + wave;
    const int c = (lane & 3) ^ row_swizzle(16 * g + lr);
    int64_t row = r0 + 16 * g + lr;
    row = row < rows ? row : rows - 1;
    __builtin_amdgcn_global_load_lds(base + row * K + k0 + 16 * c, (lds_ptr)(lds + 1024 * g), 16, 0, 0);
  }
}

// the 16 scale bytes of 512 k (k blocks kb0 .. kb0+15) of rows r0 .. r0+255,
// one row per lane: wave w loads rows 64 w .. 64 w + 63.  Rows are ld bytes
// apart and 16-block groups gs (in the MFMA order, 16 and rows * 16: the wave
// reads 1 KiB in one run).
__device__ __forceinline__ void load_scales(const uint8_t* s, int64_t rows, int64_t r0,
                                            int64_t ld, int64_t gs, int64_t kb0, uint8_t* lds,
                                            int wave, int lane) {
  int64_t row = r0 + 64 * wave + lane;
  row = row < rows ? row : rows - 1;
  __builtin_amdgcn_global_load_lds(s + row * ld + kb0 + (kb0 >> 4) * (gs - 16), (lds_ptr)(lds + 1024 * wave),
                                   16, 0, 0);
}

// Scale word w (the 4 blocks of 128 k) of a row starting at row_base, with
// 16-block groups gs bytes apart: a word never straddles a group.
__device__ __forceinline__ const uint8_t* scale_word(const uint8_t* row_base, int64_t w, int64_t gs) {
  return row_base + w * 4 + (w >> 2) * (gs - 16);
}

// s_waitcnt vmcnt(n) lgkmcnt(0) (expcnt left alone)
template <int N> __device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// this wave's loads up to the N most recent have landed and its LDS reads
// have returned; then the workgroup meets.  A plain workgroup barrier would
// also wait for every LDS load still in flight (its release fence covers
// them); the empty asm keeps the compiler from moving memory accesses across.
template <int N> __device__ __forceinline__ void ring_barrier() {
  wait_loads<N>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A ring tile of BM x BN outputs (BM in {64, 128, 256}, BN in {128, 256}):
// four waves in a 2 x 2 layout, each (BM/2) x (BN/2) = MI x NJ MFMA tiles of
// 32 x 32.  A ring slot holds A's BM rows then B's BN rows of one 64-deep
// stage.
template <int BM, int BN>
struct TileRing {
  static constexpr int MI = BM / 64, NJ = BN / 64;
  static constexpr int kLoads = BM / 64 + BN / 64;   // LDS loads of one stage per wave
  const GemmParams& p;
  int wave, lane, fr, h;
  int64_t m0, n0, K, stages;
  int64_t kstart;               // first stage of this tile (K order rotated per tile)
  int vstages;                  // stages run: K / 64 rounded up to whole groups of 8
  int dead;                     // stages of the last group past K (0 if K % 512 == 0)
  int swz;                      // row_swizzle of this lane's fragment rows
  int arow, brow;               // LDS byte offset of this lane's row in tile 0
  v16f acc[MI][NJ];
  v8i fa[2][MI], fb[2][NJ];     // fragments, double-buffered by stage parity
  u32x4 sca[2][MI], scb[2][NJ]; // scale groups, double-buffered by group parity

  __device__ TileRing(const GemmParams& pp, int64_t mm0, int64_t nn0, int w, int l, int64_t ks)
      : p(pp), wave(w), lane(l), m0(mm0), n0(nn0), kstart(ks) {
    fr = lane & 31;
    h = lane >> 5;
    K = p.K;
    stages = K / kBK;
    vstages = (int)((stages + kGroup - 1) / kGroup * kGroup);
    dead = vstages - (int)stages;
    swz = row_swizzle(fr);
    arow = ((wave >> 1) * (BM / 2) + fr) * kBK;
    brow = ((wave & 1) * (BN / 2) + fr) * kBK;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = v16f{};
  }

  template <int SLOT> __device__ __forceinline__ uint8_t* sa_slot() { return slot_a<SLOT>(); }
  template <int SLOT> __device__ __forceinline__ uint8_t* sb_slot() { return slot_a<SLOT>() + BM * kBK; }

  // loads of stage t into ring slot t % 4 (stages past the end reload the
  // last one, into a slot nobody reads again); a stage that opens a scale
  // group also brings that group's scales (each wave 64 rows of A and of B:
  // rows past the tile are loaded and never read).
  // With K % 512 != 0 the last group is run whole: its first `dead` stages
  // reload the last stage of the group before (and take scale bytes 0, see
  // read_scales), its others take the remaining K, and its scales are the
  // row's last 16 bytes, so that every stage keeps its position in a group.
  template <int SLOT, bool GROUP_START>
  __device__ __forceinline__ void issue(int64_t t) {
    int tt = (int)t < vstages ? (int)t : vstages - 1;
    tt += (int)kstart;
    if (tt >= vstages) tt -= vstages;
    const int kt = max(tt - dead, min(tt, (dead ? vstages - kGroup : vstages) - 1));
    load_stage<BM>(p.qa, p.M, m0, K, (int64_t)kt * kBK, sa_slot<SLOT>(), wave, lane);
    load_stage<BN>(p.qb, p.N, n0, K, (int64_t)kt * kBK, sb_slot<SLOT>(), wave, lane);
    if (GROUP_START) {
      const int64_t kb0 = min((tt / kGroup) * 16, (int)(K / kBlock) - 16);
      const int gpar = (int)((t / kGroup) & 1);
      uint8_t* sc = gpar ? s_scale1 : s_scale0;
      load_scales(p.sa, p.M, m0, p.sa_ld, p.sa_gs, kb0, sc, wave, lane);
      load_scales(p.sb, p.N, n0, p.sb_ld, p.sb_gs, kb0, sc + kScBytes, wave, lane);
    }
  }

  // fragment reads of ring slot SLOT into fragment buffer FB
  template <int SLOT, int FB>
  __device__ __forceinline__ void read_frags() {
    const uint8_t* la = sa_slot<SLOT>();
    const uint8_t* lb = sb_slot<SLOT>();
    const int o0 = 16 * (h ^ swz), o1 = 16 * ((h + 2) ^ swz);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const uint8_t* pa = la + arow + 32 * kBK * i;
      fa[FB][i] = frag(*reinterpret_cast<const u32x4*>(pa + o0), *reinterpret_cast<const u32x4*>(pa + o1));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint8_t* pb = lb + brow + 32 * kBK * j;
      fb[FB][j] = frag(*reinterpret_cast<const u32x4*>(pb + o0), *reinterpret_cast<const u32x4*>(pb + o1));
    }
  }

  // scale group GP into registers.  Words below zw (the dead stages of a
  // short last group, two stages a word) become 0: those stages' products,
  // scaled by 2^-254, round to zero, and a NaN among them is one that the
  // stage they repeat has already added.
  template <int GP>
  __device__ __forceinline__ void read_scales(int zw) {
    const uint8_t* la = GP ? s_scale1 : s_scale0;
    const uint8_t* lb = la + kScBytes;
#pragma unroll
    for (int i = 0; i < MI; ++i)
      sca[GP][i] = *reinterpret_cast<const u32x4*>(la + 16 * ((wave >> 1) * (BM / 2) + 32 * i + fr));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      scb[GP][j] = *reinterpret_cast<const u32x4*>(lb + 16 * ((wave & 1) * (BN / 2) + 32 * j + fr));
#pragma unroll
    for (int k = 0; k < 3; ++k) {
#pragma unroll
      for (int i = 0; i < MI; ++i) sca[GP][i][k] = k < zw ? 0u : sca[GP][i][k];
#pragma unroll
      for (int j = 0; j < NJ; ++j) scb[GP][j][k] = k < zw ? 0u : scb[GP][j][k];
    }
  }

  // the MI x NJ MFMAs of a stage at position POS of its scale group
  template <int FB, int GP, int POS>
  __device__ __forceinline__ void mma() {
    const int sh = 16 * (POS & 1) + 8 * h;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = mfma(fa[FB][i], fb[FB][j], acc[i][j], sca[GP][i][POS >> 1] >> sh,
                         scb[GP][j][POS >> 1] >> sh);
  }

  // one stage s = 8 q + POS (POS = s % 8, group parity GP = q % 2):
  // barrier, loads of stage s + 4, reads of stage s + 1, MFMAs of stage s
  template <int POS, int GP>
  __device__ __forceinline__ void step(int64_t s) {
    // loads issued after those of stage s + 1: stages s + 2 and s + 3, kLoads
    // LDS loads each plus two for a stage that opens a scale group
    constexpr int kAfter = 2 * kLoads + (((POS + 2) % kGroup) == 0 ? 2 : 0) + (((POS + 3) % kGroup) == 0 ? 2 : 0);
    ring_barrier<kAfter>();     // stage s+1 is in LDS; every read of stage s has returned
    issue<(POS + 4) % kStages, ((POS + 4) % kGroup) == 0>(s + 4);
    read_frags<(POS + 1) % kStages, (POS + 1) & 1>();
    if (POS == kGroup - 1) read_scales<GP ^ 1>((int)s + 1 == vstages - kGroup ? dead >> 1 : 0);
    mma<POS & 1, GP, POS>();
    // Order: the fragment reads of the next stage go between this stage's
    // MFMAs (they write the other fragment buffer), a few ahead so that the
    // last one returns four MFMAs before the stage ends, and the loads are
    // spread evenly.  Issuing every read before the first MFMA left the
    // matrix cores idle at the head of each stage (8192^3: 493 against
    // 466 us; 2048 x 7168 x 7168: 113 against 102 us).
    constexpr int kReads = 2 * (MI + NJ), kMfma = MI * NJ;
    constexpr int kFirst = kReads - kMfma + 4 < 0 ? 0 : (kReads - kMfma + 4 > kReads ? kReads : kReads - kMfma + 4);
    constexpr int kEvery = kLoads >= kMfma ? 1 : kMfma / kLoads;
#pragma unroll
    for (int n = 0; n < kFirst; ++n) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int n = 0; n < kMfma; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (kFirst + n < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (n % kEvery == 0 && n / kEvery < kLoads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  template <int GP>
  __device__ __forceinline__ void group(int64_t s) {
    step<0, GP>(s);
    step<1, GP>(s + 1);
    step<2, GP>(s + 2);
    step<3, GP>(s + 3);
    step<4, GP>(s + 4);
    step<5, GP>(s + 5);
    step<6, GP>(s + 6);
    step<7, GP>(s + 7);
  }

  __device__ __forceinline__ void run() {
    issue<0, true>(0);
    issue<1, false>(1);
    issue<2, false>(2);
    issue<3, false>(3);
    ring_barrier<3 * kLoads>(); // stage 0 and scale group 0 have landed
    read_frags<0, 0>();
    read_scales<0>(0);          // K >= 512: the first group is whole
    // stages come in groups of 8, two groups per trip so that the scale
    // buffers are named statically
    int64_t s = 0;
    for (; s + 2 * kGroup <= vstages; s += 2 * kGroup) {
      group<0>(s);
      group<1>(s + kGroup);
    }
    if (s < vstages) group<0>(s);
    wait_loads<0>();            // no load may land after the workgroup ends
  }
};

__device__ __forceinline__ const GemmParams& product_of(const GemmParams& p, int) { return p; }
__device__ __forceinline__ const GemmParams& product_of(const GemmGroupArgs& a, int i) { return a.d[i]; }

// Arg: GemmParams, one product; or GemmGroupArgs, a table of products whose
// tiles share one launch (each product's tiles in its own order).
template <int BM, int BN, class Arg = GemmParams>
__global__ __launch_bounds__(kThreads) void mxfp8_gemm_ring_kernel(const Arg pp) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroups go round-robin over the 8 XCDs: give XCD x the x-th contiguous
  // run of the tile order, then walk groups of kGroupM tile rows column by column
  // (a grouped launch: the order over the whole grid, then the task's product
  // by binary search over the prefix sum of tile counts)
  const uint32_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  int prod = 0;
  uint32_t v;
  if constexpr (!__is_same(Arg, GemmParams)) {
    const uint32_t T = gridDim.x, per = T / 8, rem = T % 8;
    v = xcd * per + (xcd < rem ? xcd : rem) + slot;
    prod = find_desc(pp.task_start, pp.n, (int32_t)v);
    v -= (uint32_t)pp.task_start[prod];
  }
  const GemmParams p = product_of(pp, prod);
  if constexpr (__is_same(Arg, GemmParams)) {
    const uint32_t T = (uint32_t)p.tiles_m * (uint32_t)p.tiles_n;
    const uint32_t per = T / 8, rem = T % 8;
    v = xcd * per + (xcd < rem ? xcd : rem) + slot;
  }
  const uint32_t gsize = (uint32_t)kGroupM * (uint32_t)p.tiles_n;
  const uint32_t grp = v / gsize, first_m = grp * kGroupM;
  const uint32_t gm = min((uint32_t)p.tiles_m - first_m, (uint32_t)kGroupM);
  const uint32_t idx = v - grp * gsize;
  const int64_t m0 = (int64_t)(first_m + idx % gm) * BM;
  const int64_t n0 = (int64_t)(idx / gm) * BN;

  // XCD pairs start K at different quarters (whole scale groups) so that
  // concurrent tiles on different XCDs do not stream the same K columns,
  // whose rows sit a power-of-two stride apart, at the same time
  const int64_t ngroups = p.K / (kBK * kGroup);
  // (not with K % 512 != 0: the short group has to come last)
  const int64_t ks = p.K % (kBK * kGroup) ? 0 : ((int64_t)((xcd / 2) % 4) * ngroups / 4) * kGroup;
  TileRing<BM, BN> t(p, m0, n0, wave, lane, ks);
  t.run();

  constexpr int MI = BM / 64, NJ = BN / 64;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, fr = lane & 31;
  const int64_t r0 = m0 + wm * (BM / 2), c0 = n0 + wn * (BN / 2) + fr;
  if (m0 + BM <= p.M && n0 + BN <= p.N && p.out_bf16 && ((p.N | p.ldo) & 1) == 0) {
    // a full tile with bf16 output: whole row segments
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jp = 0; jp < NJ / 2; ++jp)
        store_bf16_pair(p, t.acc[i][2 * jp], t.acc[i][2 * jp + 1], r0 + 32 * i, n0 + wn * (BN / 2) + 64 * jp,
                        fr, h);
  } else if (m0 + BM <= p.M && n0 + BN <= p.N) {
    // a full tile: no bounds to check
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t at = (r0 + 32 * i + 8 * (r / 4) + 4 * h + (r % 4)) * p.ldo + c0 + 32 * j;
          if (p.out_bf16)
            reinterpret_cast<uint16_t*>(p.out)[at] = (uint16_t)f32_to_bf16(t.acc[i][j][r]);
          else
            __builtin_nontemporal_store(t.acc[i][j][r], reinterpret_cast<float*>(p.out) + at);
        }
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) store_tile(p, t.acc[i][j], r0 + 32 * i, c0 + 32 * j, h);
  }
}

// ---- tile128 ---------------------------------------------------------------

constexpr int kGT = 128;              // workgroup tile side (M and N)
constexpr int kGK = 128;              // K bytes per LDS tile
constexpr int kLdsStride = kGK + 16;  // padded LDS row
constexpr int kLdsTile = kGT * kLdsStride;

// One 128-deep k tile of a workgroup in registers: thread t holds 16-byte
// chunks t + 256 u (u < 4) of the 128 x 128-byte A and B tiles (row
// (t >> 3) + 32 u, k offset 16 (t & 7)), and the scale word (4 bytes: the 4
// blocks of the k tile) of this lane's fragment row in each of the wave's two
// 32-row tiles of A and of B.
struct Tile128Regs {
  u32x4 a[4], b[4];
  uint32_t sa[2], sb[2];
};

// Two k tiles in flight: while one is in LDS and feeding the MFMAs, the next
// two are loading into the two register sets.  Rows past M or N read the last
// row (their outputs are not stored), so no load sits behind a condition and
// the compiler waits only for the register set it is about to store.
__global__ __launch_bounds__(kThreads) void mxfp8_gemm_tile128_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kLdsTile];   // [buffer][A, B]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)(blockIdx.x / p.tiles_n) * kGT;
  const int64_t n0 = (int64_t)(blockIdx.x % p.tiles_n) * kGT;
  const int64_t K = p.K;
  const int lrow = tid >> 3, lk = (tid & 7) * 16;
  const int h = lane >> 5;
  const int fr = lane & 31;

  const uint8_t* ga[4];
  const uint8_t* gb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ga[u] = p.qa + min(m0 + lrow + 32 * u, p.M - 1) * K + lk;
    gb[u] = p.qb + min(n0 + lrow + 32 * u, p.N - 1) * K + lk;
  }
  const uint8_t* gsa[2];
  const uint8_t* gsb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    gsa[i] = p.sa + min(m0 + wm * 64 + 32 * i + fr, p.M - 1) * p.sa_ld;
    gsb[i] = p.sb + min(n0 + wn * 64 + 32 * i + fr, p.N - 1) * p.sb_ld;
  }
  // k tile kt into c: the scale words first (their loop copies wait for them)
  auto fetch = [&](int64_t kt, Tile128Regs& c) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      c.sa[i] = *reinterpret_cast<const uint32_t*>(scale_word(gsa[i], kt, p.sa_gs));
      c.sb[i] = *reinterpret_cast<const uint32_t*>(scale_word(gsb[i], kt, p.sb_gs));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c.a[u] = load16_cached(ga[u] + kt * kGK);
      c.b[u] = load16_cached(gb[u] + kt * kGK);
    }
  };
  auto stash = [&](int buf, const Tile128Regs& c) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<u32x4*>(&lds[buf][0][(lrow + 32 * u) * kLdsStride + lk]) = c.a[u];
      *reinterpret_cast<u32x4*>(&lds[buf][1][(lrow + 32 * u) * kLdsStride + lk]) = c.b[u];
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
  auto compute = [&](int buf, const uint32_t (&sa)[2], const uint32_t (&sb)[2]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      v8i fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint8_t* la = &lds[buf][0][(wm * 64 + 32 * i + fr) * kLdsStride + 64 * st + 16 * h];
        const uint8_t* lb = &lds[buf][1][(wn * 64 + 32 * i + fr) * kLdsStride + 64 * st + 16 * h];
        fa[i] = frag(*reinterpret_cast<const u32x4*>(la), *reinterpret_cast<const u32x4*>(la + 32));
        fb[i] = frag(*reinterpret_cast<const u32x4*>(lb), *reinterpret_cast<const u32x4*>(lb + 32));
      }
      const int sh = 16 * st + 8 * h;    // the scale byte of this lane's 32-k block
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma(fa[i], fb[j], acc[i][j], sa[i] >> sh, sb[j] >> sh);
    }
  };

  const int64_t ktiles = K / kGK;
  Tile128Regs c0, c1;
  fetch(0, c0);
  fetch(min((int64_t)1, ktiles - 1), c1);
  stash(0, c0);
  uint32_t sa0[2] = {c0.sa[0], c0.sa[1]}, sb0[2] = {c0.sb[0], c0.sb[1]};
  __syncthreads();
  for (int64_t kt = 0; kt < ktiles; kt += 2) {
    // tile kt is in lds[0] (its scales in sa0/sb0), tile kt + 1 loading in c1
    fetch(min(kt + 2, ktiles - 1), c0);
    compute(0, sa0, sb0);
    stash(1, c1);
    const uint32_t sa1[2] = {c1.sa[0], c1.sa[1]}, sb1[2] = {c1.sb[0], c1.sb[1]};
    __syncthreads();
    // tile kt + 1 (past the end for an odd count: skipped) is in lds[1]
    fetch(min(kt + 3, ktiles - 1), c1);
    if (kt + 1 < ktiles) compute(1, sa1, sb1);
    stash(0, c0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sa0[i] = c0.sa[i];
      sb0[i] = c0.sb[i];
    }
    __syncthreads();
  }

  if (m0 + kGT <= p.M && n0 + kGT <= p.N && p.out_bf16 && ((p.N | p.ldo) & 1) == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) store_bf16_pair(p, acc[i][0], acc[i][1], m0 + wm * 64 + 32 * i, n0 + wn * 64, fr, h);
    return;
  }
  if (p.out_bf16 && ((p.N | p.ldo) & 1) == 0 && n0 + wn * 64 + 64 <= p.N) {
    // a partial tile whose wave columns lie inside N: rows past M skipped
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (m0 + wm * 64 + 32 * i < p.M)
        store_bf16_pair<false>(p, acc[i][0], acc[i][1], m0 + wm * 64 + 32 * i, n0 + wn * 64, fr, h);
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      store_tile(p, acc[i][j], m0 + wm * 64 + 32 * i, n0 + wn * 64 + 32 * j + fr, h);
}

// ---- skinny (M <= 128) ---------------------------------------------------------
//
// A few activation rows against a large weight (decode): the product is bound
// by streaming B once from HBM.  A workgroup owns 32 output columns and its
// four waves split K into contiguous ranges of 128-deep units.  For each unit
// a wave loads the 32 B rows and the A rows (MT 32-row tiles, M <= 32 MT)
// into registers with coalesced loads, two units ahead: every load covers
// 8 rows x 128 bytes (1 KiB).  It writes them into its own LDS region (the
// 16-byte chunk c of row r at chunk c ^ (r % 8) ^ ((r / 8) % 2)), reads the
// MFMA fragments back, and multiplies.  A rows past M are zero.  The four
// partial tiles meet in LDS and are summed in wave order.  Under a weight of
// few strips the rows are cut into blocks, one workgroup per block and
// strip, and the blocks of a strip run on one XCD so that its L2 serves them
// the strip (the launcher's notes give the rule and its measurements).
//
// Measured on 16 x 7168 x 7168 with the weight read from HBM (rotating
// copies): loading B straight into LDS (global_load_lds) and the A fragments
// one per lane and row, one unit in flight, took 15.7 us; this register path
// takes 12.7 us (13.3 us with paired scale-word loads instead of staged
// ones).  Reading B alone in the same pattern takes 8.9 us.

constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyRegion = 32 * 128;   // one operand tile of one unit in LDS (4 KiB)

__device__ __forceinline__ int skinny_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt lgkmcnt(0), vmcnt and expcnt left alone
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ void skinny_pin() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

// Scale words.  STAGED (a wave's K range of at most staged_units<MT>() units):
// the wave copies the words of its whole range into LDS once,
// with loads in which consecutive lanes read consecutive words of a row, and
// reads one word per row and unit from there.  Otherwise (PAIRED, K >= 256)
// every other unit one load per tile brings two units' words, one per row.
// A load of one word per row touches one cache line per row, 32 per load;
// on 16 x 7168 x 7168 one-word loads cost about 3.8 us of 14.2, paired loads
// about 2 us of 13.3.
// units a wave can stage (LDS: 32 for one or two A tiles, 16 for four), the
// words between staged rows (odd: no bank conflicts), the words of one tile
template <int MT> constexpr int staged_units() { return MT <= 2 ? 32 : 16; }
template <int MT> constexpr int staged_stride() { return staged_units<MT>() + 1; }
template <int MT> constexpr int staged_tile() { return 32 * staged_stride<MT>(); }
enum { kSkinnyStaged = 0, kSkinnyPaired = 1 };

// one unit in registers: lane l holds row 8 g + l / 8 of each 32-row tile,
// chunk l % 8.  PAIRED: the scale words of units ps and ps + 1 in fragment
// order (row l % 32), and `off` (0 or 1, the same for the wave) says which of
// them is this unit's.
template <int MT>
struct SkinnyUnit {
  u32x4 b[4];
  u32x4 a[MT][4];
  u32x2 sa[MT], sb;
  int64_t off;
};

template <int MT, int SC>
struct Skinny {
  const GemmParams& p;
  int lane, fr, h, lr, ch;
  int64_t n0, K, units;
  uint8_t* region;              // this wave's LDS: B tile, then the MT A tiles
  uint32_t* sreg;               // STAGED: this wave's scale words, B tile then the A tiles
  const uint8_t* psa[MT];
  const uint8_t* psb;

  __device__ Skinny(const GemmParams& pp, int w, int l, int64_t nn0, uint8_t* lds, uint32_t* slds)
      : p(pp), lane(l), fr(l & 31), h(l >> 5), lr(l >> 3), ch(l & 7), n0(nn0), K(pp.K),
        units(pp.K / 128), region(lds + w * (1 + MT) * kSkinnyRegion),
        sreg(slds + w * (1 + MT) * staged_tile<MT>()) {
#pragma unroll
    for (int t = 0; t < MT; ++t) psa[t] = p.sa + min((int64_t)(32 * t + fr), p.M - 1) * p.sa_ld;
    psb = p.sb + min(n0 + fr, p.N - 1) * p.sb_ld;
  }

  // STAGED: the scale words of units u0 .. u0 + U - 1 (U <= staged_units) of
  // the B tile and the A tiles into sreg, word k of row r at r * stride + k.
  // Lane l of load i takes entry e = l + 64 i of the row-major 32 x U block,
  // so a load reads whole runs of one row.  All loads go out before the first
  // LDS write.
  __device__ __forceinline__ void stage_scales(int64_t u0, int U) const {
    constexpr int kLoads = staged_units<MT>() * 32 / 64;
    const int n = 32 * U, iters = (n + 63) / 64;
    // e / U as (e * m) >> 16 with m = ceil(2^16 / U): exact for e < 2^16 / U
    const uint32_t m = (65536u + (uint32_t)U - 1u) / (uint32_t)U;
    uint32_t v[1 + MT][kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      if (i < iters) {                            // the same for the whole wave
        const int e = min(lane + 64 * i, n - 1);
        const int r = (int)(((uint32_t)e * m) >> 16), k = e - r * U;
        v[0][i] = *reinterpret_cast<const uint32_t*>(
            scale_word(p.sb + min(n0 + r, p.N - 1) * p.sb_ld, u0 + k, p.sb_gs));
#pragma unroll
        for (int t = 0; t < MT; ++t)
          v[1 + t][i] = *reinterpret_cast<const uint32_t*>(
              scale_word(p.sa + min((int64_t)(32 * t + r), p.M - 1) * p.sa_ld, u0 + k, p.sa_gs));
      }
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e = lane + 64 * i;
      if (i < iters && e < n) {
        const int r = (int)(((uint32_t)e * m) >> 16), k = e - r * U;
#pragma unroll
        for (int t = 0; t <= MT; ++t) sreg[t * staged_tile<MT>() + r * staged_stride<MT>() + k] = v[t][i];
      }
    }
  }

  // STAGED, both planes in the MFMA order (then K % 512 == 0): the 16-byte
  // pieces (4 words) of the groups that hold units u0 .. u0 + U - 1, one
  // piece a lane, consecutive lanes on consecutive rows of a group, so that a
  // load reads two runs of 512 bytes.  Words of a piece outside the range are
  // not written.  All loads go out before the first LDS write.
  __device__ __forceinline__ void stage_scales_grouped(int64_t u0, int U) const {
    constexpr int kIters = (staged_units<MT>() / 4 + 2 + 1) / 2;
    const int64_t g0 = u0 >> 2;
    const int ng = (int)(((u0 + U - 1) >> 2) - g0 + 1), iters = (ng + 1) / 2;
    const int r = lane & 31;
    u32x4 v[1 + MT][kIters];
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      if (i < iters) {                            // the same for the whole wave
        const int64_t g = g0 + min(2 * i + (lane >> 5), ng - 1);
        v[0][i] = *reinterpret_cast<const u32x4*>(p.sb + min(n0 + r, p.N - 1) * p.sb_ld + g * p.sb_gs);
#pragma unroll
        for (int t = 0; t < MT; ++t)
          v[1 + t][i] = *reinterpret_cast<const u32x4*>(
              p.sa + min((int64_t)(32 * t + r), p.M - 1) * p.sa_ld + g * p.sa_gs);
      }
    }
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int gi = 2 * i + (lane >> 5);
      if (i < iters && gi < ng) {
        const int k0 = (int)((g0 + gi) * 4 - u0);   // unit of word 0, relative to u0
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (k0 + j >= 0 && k0 + j < U) {
#pragma unroll
            for (int t = 0; t <= MT; ++t) sreg[t * staged_tile<MT>() + r * staged_stride<MT>() + k0 + j] = v[t][i][j];
          }
        }
      }
    }
  }

  // STAGED: the scale words of unit u0 + k in fragment order
  __device__ __forceinline__ void staged_words(int k, uint32_t (&sa)[MT], uint32_t& sb) const {
    sb = sreg[fr * staged_stride<MT>() + k];
#pragma unroll
    for (int t = 0; t < MT; ++t) sa[t] = sreg[(1 + t) * staged_tile<MT>() + fr * staged_stride<MT>() + k];
  }

  // Unit u into c.  PAIRED scale words go out first: the register copies the
  // loop makes of them wait for their loads, and loads complete in order,
  // so a wait for an early load leaves the later ones in flight.
  __device__ __forceinline__ void load(int64_t u, SkinnyUnit<MT>& c, bool scales) const {
    if (scales) {                                 // PAIRED only; K >= 256
      // both words inside the row.  A pair that is used starts at an even
      // unit (u, or units - 2 with units % 4 == 0 in the MFMA order), so it
      // never straddles a 16-block group; a pair loaded past a wave's range
      // may start at an odd unit, but never in the row's last group, so it
      // stays inside the plane.
      const int64_t ps = min(u, units - 2);
#pragma unroll
      for (int t = 0; t < MT; ++t) c.sa[t] = *reinterpret_cast<const u32x2_a4*>(scale_word(psa[t], ps, p.sa_gs));
      c.sb = *reinterpret_cast<const u32x2_a4*>(scale_word(psb, ps, p.sb_gs));
      c.off = u - ps;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t row = min(n0 + 8 * g + lr, p.N - 1);
      c.b[g] = load16(p.qb + row * K + u * 128 + 16 * ch);
    }
    // rows past M read row M - 1 (a cache hit) and are zeroed in stage(); a
    // select here would make the compiler wait for the load at once
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t row = min((int64_t)(32 * t + 8 * g + lr), p.M - 1);
        c.a[t][g] = load16_cached(p.qa + row * K + u * 128 + 16 * ch);
      }
    }
  }

  // the unit's tiles into this wave's LDS region, swizzled
  __device__ __forceinline__ void stage(const SkinnyUnit<MT>& c) const {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r = 8 * g + lr;
      const int at = r * 128 + 16 * (ch ^ skinny_swizzle(r));
      *reinterpret_cast<u32x4*>(region + at) = c.b[g];
#pragma unroll
      for (int t = 0; t < MT; ++t)
        *reinterpret_cast<u32x4*>(region + (1 + t) * kSkinnyRegion + at) =
            32 * t + r < p.M ? c.a[t][g] : u32x4{0, 0, 0, 0};
    }
  }

  // the unit in c through LDS and the MFMAs with scale words sa, sb (its B
  // fragments ANDed with keep); c is refilled with unit next
  __device__ __forceinline__ void step(SkinnyUnit<MT>& c, const uint32_t (&sa)[MT], uint32_t sb,
                                       int64_t next, bool scales, uint32_t keep, v16f (&acc)[MT]) const {
    stage(c);
    skinny_pin();
    load(next, c, scales);
    skinny_pin();
    wait_lds();                                  // the unit's LDS writes are done
    skinny_pin();
    compute(sa, sb, keep, acc);
  }

  __device__ __forceinline__ void compute(const uint32_t (&sa)[MT], uint32_t sb, uint32_t keep,
                                          v16f (&acc)[MT]) const {
    const uint8_t* row = region + fr * 128;
    const int f = skinny_swizzle(fr);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c0 = 16 * ((4 * j + h) ^ f), c1 = 16 * ((4 * j + h + 2) ^ f);
      const v8i fb = frag(*reinterpret_cast<const u32x4*>(row + c0) & keep,
                          *reinterpret_cast<const u32x4*>(row + c1) & keep);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint8_t* ra = row + (1 + t) * kSkinnyRegion;
        const v8i fa = frag(*reinterpret_cast<const u32x4*>(ra + c0), *reinterpret_cast<const u32x4*>(ra + c1));
        acc[t] = mfma(fa, fb, acc[t], sa[t] >> (16 * j + 8 * h), sb >> (16 * j + 8 * h));
      }
    }
  }
};

// Arg: GemmParams, one product; or GemmGroupArgs, a table of products (MoE
// experts, each with a few rows) in one launch, every one in row blocks.
template <int MT, int SC, bool RB = false, class Arg = GemmParams>
__global__ __launch_bounds__(kSkinnyWaves * 64) void mxfp8_gemm_skinny_kernel(const Arg pp) {
  // RB, row blocks (for weights too narrow to give every CU a column strip):
  // tasks R i .. R i + R - 1 (R = tiles_m) take rows 32 MT r .. of A for
  // column strip i.
  constexpr bool kGrouped = !__is_same(Arg, GemmParams);
  static_assert(!kGrouped || RB, "grouped products run in row blocks");
  uint32_t bid = blockIdx.x;
  GemmParams p;
  if constexpr (RB) {
    // workgroups go round-robin over the 8 XCDs: XCD x takes the x-th
    // contiguous run of tasks, so the row blocks of a strip share its L2 and
    // its B strip is fetched once (256 x 2048 x 7168: 22.7 -> 18.3 us, fetched
    // bytes 0.45 times; 512 x 1024 x 7168: 25.2 -> 17.8 us)
    const uint32_t T = gridDim.x, xcd = bid % 8, slot = bid / 8, per = T / 8, rem = T % 8;
    bid = xcd * per + (xcd < rem ? xcd : rem) + slot;
    if constexpr (kGrouped) {
      // the task's product: binary search over the prefix sum of task counts
      const int i = find_desc(pp.task_start, pp.n, (int32_t)bid);
      p = pp.d[i];
      bid -= (uint32_t)pp.task_start[i];
    } else {
      p = pp;
    }
    const uint32_t nrb = (uint32_t)p.tiles_m, rb = bid % nrb;
    bid /= nrb;
    const int64_t r0 = (int64_t)rb * 32 * MT;
    p.qa += r0 * p.K;
    p.sa += r0 * p.sa_ld;
    p.out = static_cast<uint8_t*>(p.out) + r0 * p.ldo * (p.out_bf16 ? 2 : 4);
    p.M = min(p.M - r0, (int64_t)(32 * MT));
  } else {
    p = pp;
  }
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kSkinnyWaves * (1 + MT) * kSkinnyRegion];
  __shared__ uint32_t slds[SC == kSkinnyStaged ? kSkinnyWaves * (1 + MT) * staged_tile<MT>() : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, h = lane >> 5;
  const int64_t n0 = (int64_t)bid * 32;
  const int64_t units = p.K / 128;
  constexpr bool kPaired = SC == kSkinnyPaired;
  // PAIRED: every wave's range starts at an even unit, so each pair of scale
  // words it uses (units u, u + 1 with u even) lies inside one 16-block group
  const auto split = [&](int w) -> int64_t {
    if (w == kSkinnyWaves) return units;
    return kPaired ? 2 * ((units / 2) * w / kSkinnyWaves) : units * w / kSkinnyWaves;
  };
  const int64_t u0 = split(wave), u1 = split(wave + 1);

  const Skinny<MT, SC> sk(p, wave, lane, n0, lds, slds);
  v16f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v16f{};
  if (u0 < u1) {
    // Two units in flight: while unit u goes through LDS and the MFMAs, the
    // loads of units u + 1 and u + 2 are outstanding.  The two register sets
    // alternate (c0 even units from u0, c1 odd); a load past the wave's range
    // reads its last unit again (a cache hit), so every iteration issues the
    // same loads and the compiler waits for exactly the set it is about to
    // use.  PAIRED: c0's scale load also brings c1's words.  STAGED: the
    // scale words are copied into LDS behind the first two units' loads.
    SkinnyUnit<MT> c0, c1;
    sk.load(u0, c0, kPaired);
    sk.load(min(u0 + 1, u1 - 1), c1, false);
    if constexpr (!kPaired) {
      if (p.sa_gs != 16 && p.sb_gs != 16)
        sk.stage_scales_grouped(u0, (int)(u1 - u0));
      else
        sk.stage_scales(u0, (int)(u1 - u0));
    }
    for (int64_t u = u0; u < u1; u += 2) {
      skinny_pin();
      uint32_t sa[MT], sb, sa1[MT], sb1;
      if constexpr (kPaired) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          sa[t] = c0.off ? c0.sa[t].y : c0.sa[t].x;
          sa1[t] = c0.sa[t].y;
        }
        sb = c0.off ? c0.sb.y : c0.sb.x;
        sb1 = c0.sb.y;
      } else {
        sk.staged_words((int)(u - u0), sa, sb);
        sk.staged_words((int)(min(u + 1, u1 - 1) - u0), sa1, sb1);
      }
      sk.step(c0, sa, sb, min(u + 2, u1 - 1), kPaired, ~0u, acc);
      // Unconditional, so that the compiler's wait counts are the same on
      // every path.  Past the range (an odd count) its B fragments are zero,
      // and its A fragments and scale words come from inside the product
      // (the wave's last unit, or the next unit's words), so it adds zeros,
      // or a NaN that the exact result already holds.
      skinny_pin();
      sk.step(c1, sa1, sb1, min(u + 3, u1 - 1), false, u + 1 < u1 ? ~0u : 0u, acc);
    }
    skinny_pin();
  }

  // the partial tiles reuse the LDS regions once every wave is done, one
  // 32-row A tile at a time
  float (*part)[32][32] = reinterpret_cast<float (*)[32][32]>(lds);
  static_assert(sizeof(float) * kSkinnyWaves * 32 * 32 <= sizeof(lds), "partials fit");
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wave][8 * (r / 4) + 4 * h + (r % 4)][fr] = acc[t][r];
    __syncthreads();
    for (int e = tid; e < 32 * 32; e += kSkinnyWaves * 64) {
      const int row = 32 * t + (e >> 5), col = e & 31;
      float sum = part[0][e >> 5][col];
#pragma unroll
      for (int w = 1; w < kSkinnyWaves; ++w) sum += part[w][e >> 5][col];
      if (row < p.M && n0 + col < p.N) {
        const int64_t at = row * p.ldo + n0 + col;
        if (p.out_bf16)
          reinterpret_cast<uint16_t*>(p.out)[at] = (uint16_t)f32_to_bf16(sum);
        else
          reinterpret_cast<float*>(p.out)[at] = sum;
      }
    }
  }
}

// staged scale words when every wave's range fits the staging area (K up to
// 16384 for one or two A tiles, 8192 for four), otherwise paired loads (which
// need K >= 256, true whenever staging does not fit)
// RB: the workgroups are column strips times the row blocks in p.tiles_m
template <int MT, bool RB = false>
void launch_skinny(const GemmParams& p, int64_t workgroups, hipStream_t s) {
  const int64_t units = p.K / 128, per_wave = (units + kSkinnyWaves - 1) / kSkinnyWaves;
  const bool staged = per_wave <= staged_units<MT>();
  if (staged)
    hipLaunchKernelGGL((mxfp8_gemm_skinny_kernel<MT, kSkinnyStaged, RB>), dim3((uint32_t)workgroups),
                       dim3(kSkinnyWaves * 64), 0, s, p);
  else
    hipLaunchKernelGGL((mxfp8_gemm_skinny_kernel<MT, kSkinnyPaired, RB>), dim3((uint32_t)workgroups),
                       dim3(kSkinnyWaves * 64), 0, s, p);
}

}  // namespace

namespace {

GemmParams make_params(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t M,
                       int64_t N, int64_t K, ScaleStride sa_stride, ScaleStride sb_stride, void* out,
                       int64_t out_ld, bool out_bf16) {
  GemmParams p;
  p.qa = qa; p.sa = sa; p.qb = qb; p.sb = sb; p.out = out;
  p.M = M; p.N = N; p.K = K;
  p.ldo = out_ld;
  p.sa_ld = sa_stride.row; p.sb_ld = sb_stride.row;
  p.sa_gs = sa_stride.grp; p.sb_gs = sb_stride.grp;
  p.out_bf16 = out_bf16 ? 1 : 0;
  p.tiles_m = p.tiles_n = 0;
  return p;
}

// Tasks one grouped launch carries at most (so that the prefix sums stay
// within 32 bits).
constexpr int64_t kMaxGroupTasks = (int64_t)1 << 30;

template <int MT, int SC>
hipError_t flush_group(GemmGroupArgs& g, int64_t& tasks, hipStream_t s) {
  if (g.n == 0) return hipSuccess;
  hipLaunchKernelGGL((mxfp8_gemm_skinny_kernel<MT, SC, true, GemmGroupArgs>), dim3((uint32_t)tasks),
                     dim3(kSkinnyWaves * 64), 0, s, g);
  g.n = 0;
  tasks = 0;
  return hipGetLastError();
}

// the ring tiles, in the order of the single-call cost model, and the time of
// one tile at full load in eighths of a 256 x 256 tile's
struct RingTile { int bm, bn; int64_t weight; };
constexpr RingTile kRingTiles[4] = {{256, 256, 8}, {128, 256, 5}, {128, 128, 3}, {64, 128, 2}};

template <int BM, int BN>
hipError_t flush_ring_group(GemmGroupArgs& g, int64_t& tasks, hipStream_t s) {
  if (g.n == 0) return hipSuccess;
  hipLaunchKernelGGL((mxfp8_gemm_ring_kernel<BM, BN, GemmGroupArgs>), dim3((uint32_t)tasks), dim3(kThreads), 0,
                     s, g);
  g.n = 0;
  tasks = 0;
  return hipGetLastError();
}

hipError_t flush_ring_table(int t, GemmGroupArgs& g, int64_t& tasks, hipStream_t s) {
  switch (t) {
    case 0: return flush_ring_group<256, 256>(g, tasks, s);
    case 1: return flush_ring_group<128, 256>(g, tasks, s);
    case 2: return flush_ring_group<128, 128>(g, tasks, s);
    default: return flush_ring_group<64, 128>(g, tasks, s);
  }
}

// table t: A tiles per workgroup 1, 2 or 4 (t / 2), staged or paired scale words (t % 2)
hipError_t flush_table(int t, GemmGroupArgs& g, int64_t& tasks, hipStream_t s) {
  switch (t) {
    case 0: return flush_group<1, kSkinnyStaged>(g, tasks, s);
    case 1: return flush_group<1, kSkinnyPaired>(g, tasks, s);
    case 2: return flush_group<2, kSkinnyStaged>(g, tasks, s);
    case 3: return flush_group<2, kSkinnyPaired>(g, tasks, s);
    case 4: return flush_group<4, kSkinnyStaged>(g, tasks, s);
    default: return flush_group<4, kSkinnyPaired>(g, tasks, s);
  }
}

}  // namespace

hipError_t launch_gemm_grouped(const GemmDesc* d, int n, bool out_bf16, hipStream_t s) {
  constexpr int kTables = 6, kRingTables = 4;
  // about 4 KiB a table: on the heap, not on the caller's stack
  std::vector<GemmGroupArgs> tables(kTables + kRingTables);
  GemmGroupArgs* g = tables.data();
  GemmGroupArgs* rg = g + kTables;
  int64_t tasks[kTables] = {}, rtasks[kRingTables] = {};
  for (GemmGroupArgs& t : tables) {
    t.n = 0;
    t.task_start[0] = 0;
  }
  for (int i = 0; i < n; ++i) {
    const GemmDesc& e = d[i];
    if (e.M == 0 || e.N == 0) continue;
    // Products of more than 32 rows take ring tiles when K allows (K >= 512):
    // with a grouped grid that large they beat the skinny kernel's tiles
    // (64 experts x [2048, 7168]: 33 tokens each 207 against 275 us, 64
    // tokens 212 against 315 us, 128 tokens 222 against 435 us).
    const bool ring = e.M > kGroupSkinnyRows && e.K >= kBK * kGroup;
    if (!ring && e.M > kGemmGroupRows) {
      // K below one scale group: the single call's tile128 route
      if (hipError_t r = launch_gemm(e.qa, e.sa, e.qb, e.sb, e.M, e.N, e.K, e.sa_stride, e.sb_stride, e.out,
                                     e.out_ld, out_bf16, s))
        return r;
      continue;
    }
    if (ring) {
      // the tile with the least time over all its tiles (the grouped grid is
      // large, so there are no rounds over the CUs to weigh)
      int best = 0;
      int64_t best_cost = 0;
      for (int c = 0; c < kRingTables; ++c) {
        const int64_t tiles = ((e.M + kRingTiles[c].bm - 1) / kRingTiles[c].bm) *
                              ((e.N + kRingTiles[c].bn - 1) / kRingTiles[c].bn);
        if (c == 0 || tiles * kRingTiles[c].weight < best_cost) {
          best = c;
          best_cost = tiles * kRingTiles[c].weight;
        }
      }
      GemmParams p = make_params(e.qa, e.sa, e.qb, e.sb, e.M, e.N, e.K, e.sa_stride, e.sb_stride, e.out,
                                 e.out_ld, out_bf16);
      p.tiles_m = (int32_t)((e.M + kRingTiles[best].bm - 1) / kRingTiles[best].bm);
      p.tiles_n = (int32_t)((e.N + kRingTiles[best].bn - 1) / kRingTiles[best].bn);
      const int64_t t = (int64_t)p.tiles_m * p.tiles_n;
      if (rg[best].n == kGemmGroupMax || rtasks[best] + t > kMaxGroupTasks) {
        if (hipError_t r = flush_ring_table(best, rg[best], rtasks[best], s)) return r;
      }
      rg[best].d[rg[best].n] = p;
      rtasks[best] += t;
      rg[best].task_start[++rg[best].n] = (int32_t)rtasks[best];
      continue;
    }
    GemmParams p = make_params(e.qa, e.sa, e.qb, e.sb, e.M, e.N, e.K, e.sa_stride, e.sb_stride, e.out, e.out_ld,
                               out_bf16);
    // one workgroup per strip with as many A tiles as the product has rows
    // (more than 32 only with K < 512): a grouped grid is large already, so
    // each strip of B is streamed once (with K = 7168, before ring tiles took
    // these products: 64 tokens each 354 -> 314 us against 32-row blocks,
    // 128 tokens 582 -> 435 us)
    const int mt = e.M <= 32 ? 1 : e.M <= 64 ? 2 : 4;
    p.tiles_m = (int32_t)((e.M + 32 * mt - 1) / (32 * mt));
    const int64_t t = p.tiles_m * ((e.N + 31) / 32);
    const int64_t per_wave = (e.K / 128 + kSkinnyWaves - 1) / kSkinnyWaves;
    const int limit = mt == 4 ? staged_units<4>() : staged_units<1>();
    const int k = (mt == 1 ? 0 : mt == 2 ? 2 : 4) + (per_wave <= limit ? 0 : 1);
    if (g[k].n == kGemmGroupMax || tasks[k] + t > kMaxGroupTasks) {
      if (hipError_t r = flush_table(k, g[k], tasks[k], s)) return r;
    }
    g[k].d[g[k].n] = p;
    tasks[k] += t;
    g[k].task_start[++g[k].n] = (int32_t)tasks[k];
  }
  for (int k = 0; k < kTables; ++k)
    if (hipError_t r = flush_table(k, g[k], tasks[k], s)) return r;
  for (int k = 0; k < kRingTables; ++k)
    if (hipError_t r = flush_ring_table(k, rg[k], rtasks[k], s)) return r;
  return hipSuccess;
}

hipError_t launch_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                       int64_t M, int64_t N, int64_t K, ScaleStride sa_stride, ScaleStride sb_stride,
                       void* out, int64_t out_ld, bool out_bf16, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmParams p = make_params(qa, sa, qb, sb, M, N, K, sa_stride, sb_stride, out, out_ld, out_bf16);
  const int64_t skinny = (N + 31) / 32;
  const int64_t r32 = (M + 31) / 32, r64 = (M + 63) / 64, r128 = (M + 127) / 128;
  // A weight of few column strips leaves CUs idle (each workgroup streams its
  // strip at a fixed rate, and the ring tiles of such a product are few): the
  // rows are then split into blocks of 32, else 64, else (M <= 512) 128 rows,
  // one workgroup per block and strip, while those still fit one per CU.
  // Measured with the weight read from HBM: 128 x 1024 x 4096 18.0 -> 10.8
  // us, 80 x 4096 x 14336 50.1 -> 35.2 us, 192 x 1024 x 7168 (ring tiles
  // before) 39.5 -> 16.9 us, 512 x 1024 x 7168 39.6 -> 24.5 us, 512 x 2048 x
  // 7168 40.5 -> 31.2 us.  128-row blocks past M = 512 measured 0.95 to 1.09
  // times the ring tiles and are not taken; splitting further than one
  // workgroup per CU loses (128 x 7168 x 7168 in 64-row halves 28.9 -> 39.4 us)
  if (M > 32 && r32 * skinny <= kCUs) {
    p.tiles_m = (int32_t)r32;
    launch_skinny<1, true>(p, r32 * skinny, s);
  } else if (M > 64 && r64 * skinny <= kCUs) {
    p.tiles_m = (int32_t)r64;
    launch_skinny<2, true>(p, r64 * skinny, s);
  } else if (M > 128 && M <= 512 && r128 * skinny <= kCUs) {
    p.tiles_m = (int32_t)r128;
    launch_skinny<4, true>(p, r128 * skinny, s);
  } else if (M <= 32) {
    launch_skinny<1>(p, skinny, s);
  } else if (M <= 128 && !(K >= kBK * kGroup && r64 * ((N + 127) / 128) * 16 >= 9 * (int64_t)kCUs)) {
    // two or four A tiles.  With the weight read from HBM they beat the ring
    // tiles while those are few (128 x 7168 x 7168: 29 us against 43 us; 64 x
    // 14336 x 7168: 40 against 46 us; 33 x 16384 x 4096: 25 against 29 us, at
    // 112, 112 and 128 tiles of 64 x 128).  From 144 such tiles on (9/16 of
    // the CUs) the ring tiles, chosen as below, win: 64 x 18432 x
    // 7168 55 -> 48 us, 128 x 12288 x 4096 37 -> 27 us, 64 x 28672 x 7168
    // 75 -> 52 us, 128 x 28672 x 7168 107 -> 59 us.  With up to 32 rows the
    // single A tile wins at any width (16 x 28672 x 7168: 42 against 48 us).
    if (M <= 64)
      launch_skinny<2>(p, skinny, s);
    else
      launch_skinny<4>(p, skinny, s);
  } else if (K >= kBK * kGroup) {
    // the ring tile with the least rounds of tiles over the CUs times the
    // time of one tile at full load, in eighths of a 256 x 256 tile's
    // (measured on 8192^3: 128 x 256 takes 5, 128 x 128 3 and 64 x 128 2)
    struct Choice { int bm, bn; int64_t weight; };
    constexpr Choice kChoices[4] = {{256, 256, 8}, {128, 256, 5}, {128, 128, 3}, {64, 128, 2}};
    int best = 0;
    int64_t best_cost = 0;
    for (int c = 0; c < 4; ++c) {
      const int64_t tiles = ((M + kChoices[c].bm - 1) / kChoices[c].bm) * ((N + kChoices[c].bn - 1) / kChoices[c].bn);
      const int64_t cost = kChoices[c].weight * ((tiles + kCUs - 1) / kCUs);
      if (c == 0 || cost < best_cost) { best = c; best_cost = cost; }
    }
    p.tiles_m = (int32_t)((M + kChoices[best].bm - 1) / kChoices[best].bm);
    p.tiles_n = (int32_t)((N + kChoices[best].bn - 1) / kChoices[best].bn);
    const dim3 grid((uint32_t)((int64_t)p.tiles_m * p.tiles_n));
    switch (best) {
      case 0: hipLaunchKernelGGL((mxfp8_gemm_ring_kernel<256, 256>), grid, dim3(kThreads), 0, s, p); break;
      case 1: hipLaunchKernelGGL((mxfp8_gemm_ring_kernel<128, 256>), grid, dim3(kThreads), 0, s, p); break;
      case 2: hipLaunchKernelGGL((mxfp8_gemm_ring_kernel<128, 128>), grid, dim3(kThreads), 0, s, p); break;
      default: hipLaunchKernelGGL((mxfp8_gemm_ring_kernel<64, 128>), grid, dim3(kThreads), 0, s, p); break;
    }
  } else {
    p.tiles_m = (int32_t)((M + kGT - 1) / kGT);
    p.tiles_n = (int32_t)((N + kGT - 1) / kGT);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    hipLaunchKernelGGL(mxfp8_gemm_tile128_kernel, dim3((uint32_t)tiles), dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace mx
